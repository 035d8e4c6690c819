"""GPU parity of the input-gradient backward against the backward oracle
(oracle/backward.py, pinned by finite differences), stage by stage: each
stage's oracle runs on the GPU's own inputs to that stage, as the forward's
parity protocol does.

  * the transposed packed weights equal the forward's blocks transposed, bit
    for bit;
  * gate backward: dY's 1x128 codes and scales bit-exact (dY = fl32(g * dh) on
    both sides); dlogit within the per-row bound;
  * GEMM(dY, W2^T) = dh_row and GEMM(dz, W13^T) = dx within the per-row bound
    of the oracle's FP64 product of the same codes (z comes from GEMM1's
    epilogue that keeps it, whose h codes must equal the forward's);
  * SwiGLU backward: every dz code within half an E4M3 step of the FP64 value
    (plus the FP32 arithmetic's slack), scales within tolerance;
  * du and de within the per-row bound.
The FP8 backward against the unquantised FP64 backward is reported (and only
loosely bounded): that is the quantisation error, not a parity target."""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_top_routing_02_amd as moe
import workloads
from helpers import TOL, dev, np_, rowinf_rel, say, u16
from oracle import backward as bw
from test_gpu_layer import pack_all, run_steps

pytestmark = pytest.mark.gpu


def _bf16_f64(t):
    return (u16(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_codes(q, sc, s_ref, x_ref, mag):
    """Every dequantised code within half an E4M3 step of the exact value plus
    1e-5 of the size of the value's terms (`mag`), for an expanded (per
    element) scale sc; the scales within tolerance of the reference ones."""
    assert np.all(np.abs(sc.astype(np.float64) / s_ref.astype(np.float64) - 1) <= TOL)
    table = oracle.e4m3_table()
    vals = np.unique(table[np.isfinite(table)])
    gaps = np.diff(vals)
    half = np.zeros(256)
    for c in range(256):
        if np.isfinite(table[c]):
            i = np.searchsorted(vals, table[c])
            half[c] = max(gaps[i - 1] if i > 0 else gaps[0], gaps[i] if i < gaps.size else gaps[-1]) / 2
    deq = table[q] * sc
    bound = half[q] * sc * (1 + 1e-6) + 1e-5 * mag + 1e-7 * sc
    bad = np.abs(deq - x_ref) > bound
    assert not bad.any(), f"{int(bad.sum())} codes further from the exact value than allowed"


def _check_dz_codes(q, s, x_ref, mag):
    """Codes and scales of a fused-quantised FP32 GPU value, against its exact
    FP64 value: the scale within tolerance of the oracle's quantiser applied
    to the FP32-rounded exact value, and every dequantised code within half an
    E4M3 step of the exact value plus the FP32 arithmetic's error, taken as
    1e-5 of `mag`, the size of the terms the value is made of (dz_gate's factor
    1 + z (1 - sigma(z)) cancels near z = -1.28, so the error is not relative
    to the result)."""
    q_ref, s_ref = oracle.quant_1x128(x_ref.astype(np.float32))
    assert np.all(np.abs(s.astype(np.float64) / s_ref.astype(np.float64) - 1) <= TOL)
    table = oracle.e4m3_table()
    vals = np.unique(table[np.isfinite(table)])
    gaps = np.diff(vals)
    half = np.zeros(256)
    for c in range(256):
        if np.isfinite(table[c]):
            i = np.searchsorted(vals, table[c])
            half[c] = max(gaps[i - 1] if i > 0 else gaps[0], gaps[i] if i < gaps.size else gaps[-1]) / 2
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    deq = table[q] * sc
    bound = half[q] * sc * (1 + 1e-6) + 1e-5 * mag + 1e-7 * sc
    bad = np.abs(deq - x_ref) > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} dz codes further from the exact value than allowed; first at "
                             f"{tuple(i)}: exact {x_ref[tuple(i)]:.6e}, decoded {deq[tuple(i)]:.6e}, "
                             f"bound {bound[tuple(i)]:.3e}, term size {mag[tuple(i)]:.3e}")
    return int((q != q_ref).sum())



def _check_block_starts(kb_start, go_h):
    """The device-built row-block starts equal the exclusive scan of
    ceil(rows_g / 128), integer for integer; returned on the host."""
    kb = np_(kb_start).astype(np.int64)
    nkb = (np.diff(np.asarray(go_h, np.int64)) + 127) // 128
    np.testing.assert_array_equal(kb, np.concatenate([[0], np.cumsum(nkb)]))
    return kb


CASES = [
    # (T, d, E, K, I): 32-row GEMM tiles; 128-row tiles; the decode layer's shapes
    (128, 512, 16, 4, 256),
    (2048, 512, 16, 4, 256),
    (256, 7168, 256, 8, 2048),
]


@pytest.mark.parametrize("T,d,E,K,I", CASES)
def test_backward_dgrad_staged(T, d, E, K, I):
    sh = workloads.custom_shape(T=T, d=d, E=E, K=K, I=I)
    G, R = E + 1, T * K + T
    say(f"backward T={T} d={d} E={E} K={K} I={I}: forward")
    u = workloads.activations(sh).to(dev())
    e, b = workloads.centroids(sh).to(dev()), workloads.bias(sh).to(dev())
    packed = pack_all(sh)
    f = run_steps(u, e, b, packed, sh)
    dh = workloads.normal((T, d), 1.0, workloads.seed_for("backward", "dh", T), device=dev())

    say("  transposed weights")
    packed_t = moe.moe_prepare_backward_weights(packed, G, d, I)
    w13q, w2q, w13s, w2s = moe.packed_views(packed, G, d, I)
    t13q, t2q, t13s, t2s = moe.packed_views(packed_t, G, d, I)
    t13q, t13s = t13q.view(G, d, 2 * I), t13s.view(G, d // 128, 2 * I // 128)
    t2q, t2s = t2q.view(G, I, d), t2s.view(G, I // 128, d // 128)
    torch.cuda.synchronize()
    assert torch.equal(t13q, w13q.transpose(1, 2)) and torch.equal(t2q, w2q.transpose(1, 2))
    assert torch.equal(t13s, w13s.transpose(1, 2)) and torch.equal(t2s, w2s.transpose(1, 2))

    say("  GPU backward")
    go = f["go"]
    dy_q, dy_s, dlogit, row_dlogit = moe.moe_gate_backward(dh, f["y"], f["gate"], f["slot_row"], f["s"],
                                                           f["idx"], shared_row0=T * K)
    dh_row = moe.grouped_gemm_fp8_blockscaled(dy_q, dy_s, go, R, t2q, t2s, epi=moe.MOE_EPI_STORE_F32)
    # z as a training forward keeps it (the quantising epilogue that also stores
    # z); its h codes are the forward's own
    hq_z, hs_z, z = moe.grouped_gemm_fp8_blockscaled(f["uq"], f["us"], go, R, w13q, w13s,
                                                     epi=moe.MOE_EPI_SWIGLU_QUANT_Z, a_row_index=f["row_token"])
    dz_q, dz_s = moe.moe_swiglu_backward(z, dh_row)
    dx = moe.grouped_gemm_fp8_blockscaled(dz_q, dz_s, go, R, t13q, t13s, epi=moe.MOE_EPI_STORE_F32)
    du, de = moe.moe_router_backward(dh, dx, f["slot_row"], dlogit, f["idx"], e, u, row_dlogit,
                                     f["row_token"], go, shared_row0=T * K)
    torch.cuda.synchronize()
    assert torch.equal(hq_z, f["hq"]) and torch.equal(hs_z.view(torch.int32), f["hs"].view(torch.int32))

    # ---- gate backward
    say("  oracle: gate backward")
    go_h, slot_h, idx_h = np_(go), np_(f["slot_row"]), np_(f["idx"])
    _, dy_ref, dl_ref = bw.gate_backward(np_(dh), np_(f["y"]), T * K, np_(f["gate"]), slot_h, np_(f["s"]), idx_h)
    qy_ref, sy_ref = oracle.quant_1x128(dy_ref.astype(np.float32))
    np.testing.assert_array_equal(np_(dy_q), qy_ref)
    np.testing.assert_array_equal(np_(dy_s).view(np.uint32), sy_ref.view(np.uint32))
    err = rowinf_rel(np_(dlogit), dl_ref)
    say(f"  dlogit per-row rel err {err:.3e}")
    assert err <= TOL
    rd = np_(row_dlogit)
    np.testing.assert_array_equal(rd[slot_h], np_(dlogit))

    # ---- the expert GEMMs and the SwiGLU backward, on sampled groups (all groups when small)
    cnt = np.diff(go_h)
    groups = list(range(G)) if R <= 4096 else sorted({0, int(np.argmax(cnt[:E])), E})
    say(f"  oracle: expert GEMMs and SwiGLU backward on {len(groups)} groups")
    dyq_h, dys_h = np_(dy_q), np_(dy_s)
    t2q_h, t2s_h, t13q_h, t13s_h = np_(t2q), np_(t2s), np_(t13q), np_(t13s)
    dh_row_h, z_h, dzq_h, dzs_h, dx_h = np_(dh_row), np_(z), np_(dz_q), np_(dz_s), np_(dx)
    flips = 0
    for g in groups:
        r0, r1 = int(go_h[g]), int(go_h[g + 1])
        if r1 == r0:
            continue
        ref = oracle.gemm_blockscaled(dyq_h[r0:r1], dys_h[r0:r1], t2q_h[g], t2s_h[g])
        assert rowinf_rel(dh_row_h[r0:r1], ref) <= TOL
        zz = z_h[r0:r1].reshape(r1 - r0, I // 128, 2, 128).astype(np.float64)
        zg_, zu_ = zz[:, :, 0].reshape(r1 - r0, I), zz[:, :, 1].reshape(r1 - r0, I)
        dhr = dh_row_h[r0:r1].astype(np.float64)
        dzg, dzu = bw.swiglu_backward(zg_, zu_, dhr)
        sg = 1 / (1 + np.exp(-zg_))
        mag_g = np.abs(dhr * zu_) * sg * (1 + np.abs(zg_) * (1 - sg))
        mag_u = np.abs(dhr * zg_) * sg

        def inter(a, b):   # back to z's layout: per 256 columns, 128 gate then 128 up
            return np.stack([a.reshape(r1 - r0, I // 128, 128), b.reshape(r1 - r0, I // 128, 128)],
                            axis=2).reshape(r1 - r0, 2 * I)
        flips += _check_dz_codes(dzq_h[r0:r1], dzs_h[r0:r1], inter(dzg, dzu), inter(mag_g, mag_u))
        ref = oracle.gemm_blockscaled(dzq_h[r0:r1], dzs_h[r0:r1], t13q_h[g], t13s_h[g])
        assert rowinf_rel(dx_h[r0:r1], ref) <= TOL
    say(f"  dz codes that differ from the oracle's rounding (midpoints): {flips}")

    # ---- du and de
    say("  oracle: du, de")
    u_h, e_h = _bf16_f64(u), _bf16_f64(e)
    du_r, de_ref = bw.router_backward(u_h, e_h, idx_h, np_(dlogit), E)
    du_ref = bw.assemble_du(np_(dh), dx_h, np_(f["row_token"])) + du_r
    err_u, err_e = rowinf_rel(np_(du), du_ref), rowinf_rel(np_(de), de_ref)
    say(f"  du per-row rel err {err_u:.3e}, de {err_e:.3e}")
    assert err_u <= TOL and err_e <= TOL

    # ---- weight gradients
    say("  GPU weight gradients")
    dw13, dw2, ops, kb_start = moe.moe_wgrad(dh, f["gate"], f["slot_row"], f["row_token"], z, dh_row, u, go,
                                             shared_row0=T * K)
    torch.cuda.synchronize()
    kb_start = _check_block_starts(kb_start, go_h)
    say(f"  oracle: weight gradients on {len(groups)} groups")
    rt = np_(f["row_token"])
    gate_h, dh_h = np_(f["gate"]), np_(dh)
    row_w = np.ones(R, np.float32)
    row_w[slot_h.reshape(-1)] = gate_h.reshape(-1)
    cs_h, cs_x = (I // 128 + 3) // 4 * 4, (d // 128 + 3) // 4 * 4
    o = {k: np_(v) for k, v in ops.items()}
    for g in groups:
        r0, r1 = int(go_h[g]), int(go_h[g + 1])
        n = int(kb_start[g + 1] - kb_start[g])
        kb0, kp = int(kb_start[g]), 128 * n
        if n == 0:
            assert not np_(dw2[g]).any() and not np_(dw13[g]).any()
            continue
        rows = np.arange(r0, r1)
        pad = kp - (r1 - r0)
        # dY^T, bit-exact: fl32(w_r * dh) rows, zero padding, 1x128 along the rows
        dyT = np.zeros((d, kp), np.float32)
        dyT[:, :r1 - r0] = (row_w[rows, None] * dh_h[rt[rows]]).astype(np.float32).T
        q_ref, s_ref = oracle.quant_1x128(dyT)
        aq = o["dyT_q"][d * 128 * kb0:d * 128 * kb0 + d * kp].reshape(d, kp)
        as_ = o["dyT_s"][d * kb0:d * kb0 + d * n].reshape(d, n)
        np.testing.assert_array_equal(aq, q_ref)
        np.testing.assert_array_equal(as_.view(np.uint32), s_ref.view(np.uint32))
        # u^T, bit-exact: 128x128 blocks
        xT = np.zeros((d, kp), np.float32)
        xT[:, :r1 - r0] = u_h[rt[rows]].astype(np.float32).T
        qx_ref, sx_ref = oracle.quant_128x128(xT)
        xq = o["xT_q"][d * 128 * kb0:d * 128 * kb0 + d * kp].reshape(d, kp)
        xs = o["xT_s"][cs_x * kb0:cs_x * kb0 + (d // 128) * n].reshape(d // 128, n)
        np.testing.assert_array_equal(xq, qx_ref)
        np.testing.assert_array_equal(xs.view(np.uint32), sx_ref.view(np.uint32))
        # h^T and dz^T: within half a step plus the FP32 slack
        zz = z_h[r0:r1].reshape(r1 - r0, I // 128, 2, 128).astype(np.float64)
        zg_, zu_ = zz[:, :, 0].reshape(r1 - r0, I), zz[:, :, 1].reshape(r1 - r0, I)
        sg = 1 / (1 + np.exp(-zg_))
        hT = np.zeros((I, kp))
        hT[:, :r1 - r0] = (zg_ * sg * zu_).T
        mag = np.zeros((I, kp))
        mag[:, :r1 - r0] = np.abs(zg_ * sg * zu_).T
        hq = o["hT_q"][I * 128 * kb0:I * 128 * kb0 + I * kp].reshape(I, kp)
        hs = o["hT_s"][cs_h * kb0:cs_h * kb0 + (I // 128) * n].reshape(I // 128, n)
        _, hs_ref = oracle.quant_128x128(hT.astype(np.float32))
        _check_codes(hq, np.repeat(np.repeat(hs.astype(np.float64), 128, 0), 128, 1),
                     np.repeat(np.repeat(hs_ref.astype(np.float64), 128, 0), 128, 1), hT, mag)
        dhr = dh_row_h[r0:r1].astype(np.float64)
        dzg, dzu = bw.swiglu_backward(zg_, zu_, dhr)
        mg = np.abs(dhr * zu_) * sg * (1 + np.abs(zg_) * (1 - sg))
        mu = np.abs(dhr * zg_) * sg

        def inter(a, b):
            return np.stack([a.reshape(-1, I // 128, 128), b.reshape(-1, I // 128, 128)], axis=2).reshape(-1, 2 * I)
        dzT = np.zeros((2 * I, kp))
        dzT[:, :r1 - r0] = inter(dzg, dzu).T
        magz = np.zeros((2 * I, kp))
        magz[:, :r1 - r0] = inter(mg, mu).T
        zq = o["dzT_q"][2 * I * 128 * kb0:2 * I * 128 * kb0 + 2 * I * kp].reshape(2 * I, kp)
        zs = o["dzT_s"][2 * I * kb0:2 * I * kb0 + 2 * I * n].reshape(2 * I, n)
        _, zs_ref = oracle.quant_1x128(dzT.astype(np.float32))
        _check_codes(zq, np.repeat(zs.astype(np.float64), 128, 1), np.repeat(zs_ref.astype(np.float64), 128, 1),
                     dzT, magz)
        # the GEMMs on those codes
        ref2 = oracle.gemm_blockscaled(aq, as_, hq, hs)
        ref13 = oracle.gemm_blockscaled(zq, zs, xq, xs)
        e2, e13 = rowinf_rel(np_(dw2[g]), ref2), rowinf_rel(np_(dw13[g]), ref13)
        assert e2 <= TOL and e13 <= TOL, (g, e2, e13)
    say("  weight gradients within the bound")

    # ---- reported: against the unquantised FP64 backward (small cases only)
    if d <= 512:
        w = [workloads.expert_weights(sh, g, device=dev()) for g in range(G)]     # as pack_all drew them
        W1 = np.stack([np_(x[0]) for x in w]).astype(np.float64)
        W3 = np.stack([np_(x[1]) for x in w]).astype(np.float64)
        W2 = np.stack([np_(x[2]) for x in w]).astype(np.float64)
        rt = np_(f["row_token"])
        grp = np.searchsorted(go_h, np.arange(R), side="right") - 1
        x = u_h[rt]
        zg = np.einsum("rid,rd->ri", W1[grp], x)
        zu = np.einsum("rid,rd->ri", W3[grp], x)
        y64 = np.einsum("rdi,ri->rd", W2[grp], zg / (1 + np.exp(-zg)) * zu)
        s64 = 1 / (1 + np.exp(-(u_h @ e_h.T)))
        sc = s64[np.arange(T)[:, None], idx_h]
        _, dy64, dl64 = bw.gate_backward(np_(dh), y64, T * K, sc / sc.sum(1, keepdims=True), slot_h, s64, idx_h)
        dx64 = np.zeros((R, d))
        for g in range(G):
            r0, r1 = int(go_h[g]), int(go_h[g + 1])
            if r1 > r0:
                dx64[r0:r1] = bw.expert_dgrad(dy64[r0:r1], zg[r0:r1], zu[r0:r1], W1[g], W3[g], W2[g])[3]
        du64 = bw.assemble_du(np_(dh), dx64, rt) + bw.router_backward(u_h, e_h, idx_h, dl64, E)[0]
        q_err = rowinf_rel(np_(du), du64)
        say(f"  FP8 backward vs unquantised FP64 backward: du per-row rel err {q_err:.3e}")
        assert q_err < 0.2
        w_err = 0.0
        for g in range(G):
            r0, r1 = int(go_h[g]), int(go_h[g + 1])
            if r1 == r0:
                continue
            dhr64 = dy64[r0:r1] @ W2[g]
            dW2, dW1, dW3 = bw.expert_wgrad(dy64[r0:r1], zg[r0:r1], zu[r0:r1], dhr64, x[r0:r1])
            got13 = np_(dw13[g]).reshape(I // 128, 2, 128, d)
            w_err = max(w_err, rowinf_rel(np_(dw2[g]), dW2), rowinf_rel(got13[:, 0].reshape(I, d), dW1),
                        rowinf_rel(got13[:, 1].reshape(I, d), dW3))
        say(f"  FP8 weight gradients vs unquantised FP64: per-row rel err {w_err:.3e}")
        assert w_err < 0.5


@pytest.mark.gpu
def test_wgrad_groups_of_uneven_depth_and_empty_groups():
    """The weight-gradient GEMMs run K-grouped: each expert's inner dimension is
    its own padded row count.  Routing built by hand so that two experts get no
    rows, two get 260 rows (three 128-blocks, a ragged last one) and two get 40;
    the shared block has 300 rows.  dW2 has N = I = 128, half a 256-column tile.
    Every expert's dW2 and dW13 must match the oracle's FP64 product of the
    operand codes (the operands themselves are pinned by the staged test), and
    the empty experts must get exact zeros."""
    T, K, E, d, I = 300, 2, 6, 256, 128
    G = E + 1
    gen = torch.Generator().manual_seed(11)
    idx = np.zeros((T, K), np.int64)
    idx[:260] = (0, 2)
    idx[260:] = (3, 5)
    pairs = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K))
    R = T * K + T
    row_token = np.zeros(R, np.int32)
    slot_row = np.zeros((T, K), np.int32)
    for r, (g, t, k) in enumerate(pairs):
        row_token[r], slot_row[t, k] = t, r
    row_token[T * K:] = np.arange(T)
    counts = np.bincount(idx.reshape(-1), minlength=E).tolist() + [T]
    go_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    assert counts[1] == 0 and counts[4] == 0 and counts[0] == 260
    dh = torch.randn(T, d, generator=gen).to(dev())
    gate = torch.rand(T, K, generator=gen).add_(0.1).to(dev())
    z = torch.randn(R, 2 * I, generator=gen).to(dev())
    dh_row = torch.randn(R, I, generator=gen).mul_(0.5).to(dev())
    u = torch.randn(T, d, generator=gen).to(torch.bfloat16).to(dev())
    go = torch.from_numpy(go_h).to(dev())
    say(f"wgrad K-grouped: T={T} K={K} E={E} d={d} I={I}, rows per group {counts}")
    dw13, dw2, ops, kb_start = moe.moe_wgrad(dh, gate, torch.from_numpy(slot_row).to(dev()),
                                             torch.from_numpy(row_token).to(dev()), z, dh_row, u, go,
                                             shared_row0=T * K)
    torch.cuda.synchronize()
    kb_start = _check_block_starts(kb_start, go_h)
    o = {k: np_(v) for k, v in ops.items()}
    cs_h, cs_x = (I // 128 + 3) // 4 * 4, (d // 128 + 3) // 4 * 4
    for g in range(G):
        n = int(kb_start[g + 1] - kb_start[g])
        kb0, kp = int(kb_start[g]), 128 * n
        if n == 0:
            assert not np_(dw2[g]).any() and not np_(dw13[g]).any(), g
            continue
        aq = o["dyT_q"][d * 128 * kb0:d * 128 * kb0 + d * kp].reshape(d, kp)
        as_ = o["dyT_s"][d * kb0:d * kb0 + d * n].reshape(d, n)
        hq = o["hT_q"][I * 128 * kb0:I * 128 * kb0 + I * kp].reshape(I, kp)
        hs = o["hT_s"][cs_h * kb0:cs_h * kb0 + (I // 128) * n].reshape(I // 128, n)
        zq = o["dzT_q"][2 * I * 128 * kb0:2 * I * 128 * kb0 + 2 * I * kp].reshape(2 * I, kp)
        zs = o["dzT_s"][2 * I * kb0:2 * I * kb0 + 2 * I * n].reshape(2 * I, n)
        xq = o["xT_q"][d * 128 * kb0:d * 128 * kb0 + d * kp].reshape(d, kp)
        xs = o["xT_s"][cs_x * kb0:cs_x * kb0 + (d // 128) * n].reshape(d // 128, n)
        e2 = rowinf_rel(np_(dw2[g]), oracle.gemm_blockscaled(aq, as_, hq, hs))
        e13 = rowinf_rel(np_(dw13[g]), oracle.gemm_blockscaled(zq, zs, xq, xs))
        say(f"  group {g}: {n} K-blocks, dW2 {e2:.2e}, dW13 {e13:.2e}")
        assert e2 <= TOL and e13 <= TOL, (g, e2, e13)


@pytest.mark.parametrize("T", [128, 2048])
def test_backward_graph_capture_replays(T):
    """The whole backward step (gate backward, the two dgrad GEMMs, SwiGLU
    backward, du and de, then the weight gradients with their device-built
    row-block starts) captured in a HIP graph: it reads nothing back to the
    host.  Replayed three times, with eager backward work on other inputs in
    between; every replay's du, de, dW13 and dW2 equal the eager result bit
    for bit.  T = 128 runs the 32-row GEMM tiles, T = 2048 the 128-row ones."""
    d, E, K, I = 512, 16, 4, 256
    sh = workloads.custom_shape(T=T, d=d, E=E, K=K, I=I)
    G, R = E + 1, T * K + T
    say(f"backward graph capture T={T}")
    u = workloads.activations(sh).to(dev())
    e, b = workloads.centroids(sh).to(dev()), workloads.bias(sh).to(dev())
    packed = pack_all(sh)
    f = run_steps(u, e, b, packed, sh)
    packed_t = moe.moe_prepare_backward_weights(packed, G, d, I)
    w13q, w2q, w13s, w2s = moe.packed_views(packed, G, d, I)
    t13q, t2q, t13s, t2s = moe.packed_views(packed_t, G, d, I)
    t13q, t13s = t13q.view(G, d, 2 * I), t13s.view(G, d // 128, 2 * I // 128)
    t2q, t2s = t2q.view(G, I, d), t2s.view(G, I // 128, d // 128)
    go = f["go"]
    _, _, z = moe.grouped_gemm_fp8_blockscaled(f["uq"], f["us"], go, R, w13q, w13s,
                                               epi=moe.MOE_EPI_SWIGLU_QUANT_Z, a_row_index=f["row_token"])
    ws = torch.empty(moe.moe_gemm_workspace_bytes(G, R, max(2 * I, d), max(2 * I, d)), dtype=torch.uint8,
                     device=dev())

    def step(dh):
        dy_q, dy_s, dlogit, row_dlogit = moe.moe_gate_backward(dh, f["y"], f["gate"], f["slot_row"], f["s"],
                                                               f["idx"], shared_row0=T * K)
        dh_row = moe.grouped_gemm_fp8_blockscaled(dy_q, dy_s, go, R, t2q, t2s, epi=moe.MOE_EPI_STORE_F32, ws=ws)
        dz_q, dz_s = moe.moe_swiglu_backward(z, dh_row)
        dx = moe.grouped_gemm_fp8_blockscaled(dz_q, dz_s, go, R, t13q, t13s, epi=moe.MOE_EPI_STORE_F32, ws=ws)
        du, de = moe.moe_router_backward(dh, dx, f["slot_row"], dlogit, f["idx"], e, u, row_dlogit,
                                         f["row_token"], go, shared_row0=T * K)
        dw13, dw2, _, _ = moe.moe_wgrad(dh, f["gate"], f["slot_row"], f["row_token"], z, dh_row, u, go,
                                        shared_row0=T * K)
        return du, de, dw13, dw2

    dh = workloads.normal((T, d), 1.0, workloads.seed_for("backward", "dh", T), device=dev())
    dh2 = torch.flip(dh, dims=[0]).contiguous()
    ref = [x.clone() for x in step(dh)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(dh)                                   # warm the allocator on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(dh)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("du", "de", "dw13", "dw2"), outs, ref):
            assert torch.equal(x.view(torch.int32), r.view(torch.int32)), (rep, name)
        other = step(dh2)                          # eager work between replays
        torch.cuda.synchronize()
        assert other[0].shape == ref[0].shape
