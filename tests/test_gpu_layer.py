"""GPU parity of the whole DeepSeekMoE layer forward against the CPU oracle.

nlp-lineage summary, "The notation": h'_t = u_t + sum_shared FFN_i(u_t) +
sum_routed g_(i,t) FFN_i(u_t).

Every stage of the GPU path is compared with the oracle run independently on
the same inputs:
  * bit-exact: router indices and gates, dispatch arrays, 1x128 codes and
    scales of u, the packed 128x128 weight codes and scales;
  * GEMM1's SwiGLU output h (FP32) within 2e-3 per-row relative error of the
    oracle's FP64 h on the same quantised operands;
  * the 1x128 codes of h: equal to the oracle's, except adjacent codes where
    the oracle's exact value sits on a rounding midpoint (the FP32 vs FP64
    accumulation decides which side; both roundings are correct);
  * Y (GEMM2) and h' within 2e-3 per-row relative error, after widening the
    bound by the exact effect of those midpoint flips (computed from the
    oracle's own dequantised W2).
The composite moe_layer_forward must equal the step-by-step calls bit for bit.
Small workload: every token.  Decode and prefill workloads (full size, the
configuration the benchmark times): every token for routing/dispatch/quant;
the FFN stages on rows of every non-empty group and on every row of the 64
largest-|u|_inf tokens (plus the first and last), whose outputs are checked.
"""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_top_routing_02_amd as moe
import workloads
from helpers import TOL, dev, np_, rowinf_rel, say, u16
from test_gpu_quant_gemm import check_codes_close

pytestmark = pytest.mark.gpu


def pack_all(sh):
    """Quantise every expert's FP32 masters (drawn on the GPU) into one packed buffer."""
    G = sh.E + 1
    packed = torch.empty(moe.moe_packed_weight_bytes(G, sh.d, sh.I), dtype=torch.uint8, device=dev())
    for g in range(G):
        w1, w3, w2 = workloads.expert_weights(sh, g, device=dev())
        moe.moe_prepare_expert_weights(w1, w3, w2, g, G, packed)
    torch.cuda.synchronize()
    return packed


def host_weights(sh, g):
    w1, w3, w2 = workloads.expert_weights(sh, g, device=dev())
    return w1.cpu().numpy(), w3.cpu().numpy(), w2.cpu().numpy()


def run_steps(u, e, b, packed, sh):
    """The layer through the individual C-ABI calls, keeping every intermediate."""
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    G = E + 1
    w13q, w2q, w13s, w2s = moe.packed_views(packed, G, d, I)
    idx, gate, s = moe.moe_router_topk(u, e, b, K)
    count, go, row_token, slot_row = moe.moe_dispatch(idx, E, True)
    uq, us = moe.fp8_quant_1x128(u)
    R = T * K + T
    h = moe.grouped_gemm_fp8_blockscaled(uq, us, go, R, w13q, w13s, epi=moe.MOE_EPI_SWIGLU_F32,
                                         a_row_index=row_token)
    hq, hs = moe.grouped_gemm_fp8_blockscaled(uq, us, go, R, w13q, w13s, epi=moe.MOE_EPI_SWIGLU_QUANT,
                                              a_row_index=row_token)
    y = moe.grouped_gemm_fp8_blockscaled(hq, hs, go, R, w2q, w2s, epi=moe.MOE_EPI_STORE_F32)
    out = moe.moe_combine(u, y, gate, slot_row, shared_row0=T * K)
    torch.cuda.synchronize()
    return dict(idx=idx, gate=gate, s=s, count=count, go=go, row_token=row_token, slot_row=slot_row,
                uq=uq, us=us, h=h, hq=hq, hs=hs, y=y, out=out)


def deq_block(q, s):
    t = oracle.e4m3_table()
    return t[q] * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)


def flip_allowance(hq_gpu, hq_ref, hs_ref, q2, s2):
    """Per-element bound of how much Y may move because of midpoint flips in
    h's codes: |deq(hq_gpu) - deq(hq_ref)| @ |W2|^T, computed for the rows
    that have a flip (W2 dequantised from its codes only then)."""
    table = oracle.e4m3_table()
    out = np.zeros((hq_gpu.shape[0], q2.shape[0]))
    rows = np.nonzero((hq_gpu != hq_ref).any(axis=1))[0]
    if rows.size == 0:
        return out
    dv = np.abs(table[hq_gpu[rows]] - table[hq_ref[rows]]) * np.repeat(hs_ref[rows].astype(np.float64), 128, 1)
    out[rows] = dv @ np.abs(deq_block(q2, s2)).T
    return out


def check_y(y_gpu, y_ref, allow):
    excess = np.maximum(np.abs(y_gpu - y_ref) - allow * (1 + 1e-6), 0).max(axis=1)
    den = np.abs(y_ref).max(axis=1)
    return float((excess / np.where(den == 0, 1, den)).max())


def _check_packed_expert(sh, g, w13q, w2q, w13s, w2s):
    """The packed 128x128 codes and scales of expert g equal the oracle's
    quantiser on the expert's FP32 masters (gate/up blocks interleaved)."""
    I = sh.I
    w1, w3, w2 = host_weights(sh, g)
    q1, s1 = oracle.quant_128x128(w1)
    q3, s3 = oracle.quant_128x128(w3)
    q2, s2 = oracle.quant_128x128(w2)
    for j in range(I // 128):
        np.testing.assert_array_equal(w13q[256 * j:256 * j + 128], q1[128 * j:128 * j + 128])
        np.testing.assert_array_equal(w13q[256 * j + 128:256 * j + 256], q3[128 * j:128 * j + 128])
        np.testing.assert_array_equal(w13s[2 * j], s1[j])
        np.testing.assert_array_equal(w13s[2 * j + 1], s3[j])
    np.testing.assert_array_equal(w2q, q2)
    np.testing.assert_array_equal(w2s, s2)


def check_layer(sh, u, e, b, packed, g_out, token_sample=None, group_rows=None, quant_check=None):
    """Staged parity of the layer (bit-exact routing, dispatch and quant(u) on
    every token; h, h codes, Y and h' on the checked rows and tokens).

    token_sample: the tokens whose output h' is checked (all of their K + 1
    GEMM rows are checked); None = every token.  group_rows: extra GEMM rows
    to check, as {group: [rows]} (at least one row of every non-empty
    group).  quant_check: the experts whose packed weight codes and
    scales are checked bit-exact against the oracle's quantiser of their FP32
    masters; None = every expert.  The oracle's GEMMs take the packed codes as
    operands (checked experts: the oracle's own codes, equal to them)."""
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    u_h, e_h, b_h = u16(u), u16(e), np_(b)
    # ---- bit-exact stages, every token
    say("  oracle router / dispatch / quant(u)")
    idx_r, gate_r, s_r = oracle.router_topk(u_h, e_h, b_h, K)
    np.testing.assert_array_equal(np_(g_out["idx"]), idx_r)
    np.testing.assert_array_equal(np_(g_out["gate"]).view(np.uint32), gate_r.view(np.uint32))
    cnt_r, go_r, rt_r, sr_r = oracle.dispatch(idx_r, E, True)
    np.testing.assert_array_equal(np_(g_out["count"]), cnt_r)
    np.testing.assert_array_equal(np_(g_out["go"]), go_r)
    np.testing.assert_array_equal(np_(g_out["row_token"]), rt_r)
    np.testing.assert_array_equal(np_(g_out["slot_row"]), sr_r)
    uf = (u_h.astype(np.uint32) << 16).view(np.float32)
    uq_r, us_r = oracle.quant_1x128(uf)
    np.testing.assert_array_equal(np_(g_out["uq"]), uq_r)
    np.testing.assert_array_equal(np_(g_out["us"]).view(np.uint32), us_r.view(np.uint32))

    # ---- which rows get the FFN checks
    tokens = np.arange(T) if token_sample is None else np.asarray(token_sample)
    want = {}
    for t in tokens:
        for k in range(K):
            want.setdefault(int(idx_r[t, k]), set()).add(int(sr_r[t, k]))
        want.setdefault(E, set()).add(T * K + int(t))       # the shared row
    for g, rows in (group_rows or {}).items():
        want.setdefault(int(g), set()).update(int(r) for r in rows)
    w13q_d, w2q_d, w13s_d, w2s_d = moe.packed_views(packed, E + 1, d, I)
    gate_cols = np.concatenate([np.arange(256 * j, 256 * j + 128) for j in range(I // 128)])

    def rows_of(name, rows):   # copy only the rows the oracle checks
        return np_(g_out[name][torch.from_numpy(np.asarray(rows, np.int64)).to(dev())])
    y_ref_rows, allow_rows = {}, {}
    worst = dict(h=0.0, y=0.0, flips=0, rows=0, groups=0, quant_checked=0)
    for g in sorted(want):
        rows = np.array(sorted(want[g]), dtype=np.int64)
        assert np.all((rows >= go_r[g]) & (rows < go_r[g + 1])), g
        w13q, w2q, w13s, w2s = (np_(v[g]) for v in (w13q_d, w2q_d, w13s_d, w2s_d))
        if quant_check is None or g in quant_check:
            say(f"  expert {g}: packed weights vs the oracle's quantiser")
            _check_packed_expert(sh, g, w13q, w2q, w13s, w2s)
            worst["quant_checked"] += 1
        z_r = oracle.gemm_blockscaled(uq_r, us_r, w13q, w13s, a_rows=rt_r[rows])
        h_r = oracle.swiglu(z_r[:, gate_cols], z_r[:, gate_cols + 128])
        h_g, hq_g, hs_g, y_g = (rows_of(k, rows) for k in ("h", "hq", "hs", "y"))
        worst["h"] = max(worst["h"], rowinf_rel(h_g, h_r))
        hq_r, hs_r = oracle.quant_1x128(h_r.astype(np.float32))
        worst["flips"] += check_codes_close(hq_g, hs_g, hq_r, hs_r, h_r, h_g)
        y_r = oracle.gemm_blockscaled(hq_r, hs_r, w2q, w2s)
        allow = flip_allowance(hq_g, hq_r, hs_r, w2q, w2s)
        worst["y"] = max(worst["y"], check_y(y_g, y_r, allow))
        worst["rows"] += rows.size
        worst["groups"] += 1
        for i, r in enumerate(rows):
            y_ref_rows[int(r)] = y_r[i]
            allow_rows[int(r)] = allow[i]
    say(f"  {worst['rows']} rows of {worst['groups']} groups: h err {worst['h']:.3e}  y err {worst['y']:.3e}  "
        f"h-code midpoint flips {worst['flips']}")
    assert worst["h"] <= TOL and worst["y"] <= TOL
    # ---- h' for the checked tokens
    ref = np.empty((len(tokens), d))
    allow_t = np.zeros((len(tokens), d))
    for i, t in enumerate(tokens):
        v = uf[t].astype(np.float64) + y_ref_rows[T * K + int(t)]
        a = allow_rows[T * K + int(t)].copy()
        for k in range(K):
            r = int(sr_r[t, k])
            v = v + float(gate_r[t, k]) * y_ref_rows[r]
            a += float(gate_r[t, k]) * allow_rows[r]
        ref[i] = v
        allow_t[i] = a
    err = check_y(rows_of("out", tokens), ref, allow_t)
    say(f"  h' err {err:.3e} over {len(tokens)} tokens")
    assert err <= TOL
    worst["out"] = err
    return worst


def test_layer_tiny_every_token():
    sh = workloads.SHAPES["tiny"]
    say("layer tiny")
    u, e, b = (x.to(dev()) for x in (workloads.activations(sh), workloads.centroids(sh), workloads.bias(sh)))
    packed = pack_all(sh)
    g_out = run_steps(u, e, b, packed, sh)
    comp = moe.moe_layer_forward(u, e, b, packed, sh.K, sh.I)
    comp2 = moe.moe_layer_forward(u, e, b, packed, sh.K, sh.I)
    torch.cuda.synchronize()
    assert torch.equal(comp.view(torch.int32), g_out["out"].view(torch.int32))
    assert torch.equal(comp.view(torch.int32), comp2.view(torch.int32))
    check_layer(sh, u, e, b, packed, g_out)


def test_layer_tiny_quantisation_error_report():
    """Reported, not gated tighter than a sanity bound: the FP8 layer vs the
    FP64 layer with no quantisation at all."""
    sh = workloads.SHAPES["tiny"]
    u, e, b = workloads.activations(sh), workloads.centroids(sh), workloads.bias(sh)
    packed = pack_all(sh)
    out = moe.moe_layer_forward(u.to(dev()), e.to(dev()), b.to(dev()), packed, sh.K, sh.I)
    torch.cuda.synchronize()
    W = {g: host_weights(sh, g) for g in range(sh.E + 1)}
    f = oracle.layer_forward_unquantised(u16(u), u16(e), b.numpy(), sh.K, lambda g: W[g])
    uf = (u16(u).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ffn_gpu, ffn_ref = np_(out) - uf, f["out"] - uf
    fro = np.linalg.norm(ffn_gpu - ffn_ref) / np.linalg.norm(ffn_ref)
    say(f"tiny layer FP8 quantisation error (FFN part, Frobenius): {fro:.4f}")
    assert fro < 0.1


def _sample_tokens(u_h, T, n_big=64):
    """The first and last token and the n_big tokens with the largest
    |u|_inf (the 0.1% x100 outliers sit there)."""
    uf = np.abs((u_h.astype(np.uint32) << 16).view(np.float32)).max(axis=1)
    big = np.argsort(-uf, kind="stable")[:n_big]
    return sorted({0, T - 1} | set(int(t) for t in big))


def _group_rows(go, rng):
    """At least one GEMM row of every non-empty group: its last row (the
    group's ragged last tile), its first row and one seeded row between."""
    out = {}
    for g in range(go.size - 1):
        r0, r1 = int(go[g]), int(go[g + 1])
        if r1 > r0:
            out[g] = {r0, r1 - 1, int(rng.integers(r0, r1))}
    return out


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_layer_full_size_sampled(name):
    """The decode and prefill layers at full size, in the launch configuration
    the benchmark times: routing, dispatch and quant(u) bit-exact on every
    token; GEMM1/SwiGLU/requant and GEMM2 checked on the first, last and a
    seeded row of every non-empty group (all 257) and on every row of the 64
    largest-|u|_inf tokens plus the first and last token, whose outputs h' are
    checked too.  The packed weights of the shared expert, the busiest and the
    least-loaded routed expert and two seeded others are checked bit-exact
    against the oracle's quantiser of their FP32 masters; every other
    expert's GEMMs take the GPU's packed codes as the oracle's operands (a
    stage boundary of the staged protocol)."""
    sh = workloads.SHAPES[name]
    say(f"layer {name}: inputs")
    u_c = workloads.activations(sh)
    u, e, b = u_c.to(dev()), workloads.centroids(sh).to(dev()), workloads.bias(sh).to(dev())
    packed = pack_all(sh)
    say(f"layer {name}: GPU steps")
    g_out = run_steps(u, e, b, packed, sh)
    comp = moe.moe_layer_forward(u, e, b, packed, sh.K, sh.I)
    torch.cuda.synchronize()
    assert torch.equal(comp.view(torch.int32), g_out["out"].view(torch.int32))
    cnt = np_(g_out["count"])
    say(f"  load max/mean {cnt.max() / cnt.mean():.3f}")
    if name == "prefill":
        assert 3.5 < cnt.max() / cnt.mean() < 4.5
    rng = np.random.default_rng(17)
    tokens = _sample_tokens(u16(u_c), sh.T)
    used = np.nonzero(cnt)[0]
    quant_check = {sh.E, int(cnt.argmax()), int(used[np.argmin(cnt[used])])} | \
        set(int(x) for x in rng.choice(used, 2, replace=False))
    worst = check_layer(sh, u, e, b, packed, g_out, token_sample=tokens,
                        group_rows=_group_rows(np_(g_out["go"]), rng), quant_check=quant_check)
    assert worst["groups"] == int((cnt > 0).sum()) + 1      # every non-empty group, and the shared one
    assert worst["quant_checked"] == len(quant_check)


@pytest.mark.parametrize("T", [128, 2048])
def test_layer_graph_capture_replays(T):
    """moe_layer_forward captured in a HIP graph (it allocates nothing, reads
    nothing back to the host and records no memset) and replayed three times,
    with eager layer calls on other inputs in between: every replay equals the
    eager result bit for bit.  T = 128 runs the 32-row GEMM tiles, T = 2048
    (about 600 rows per group) the 128-row tiles."""
    sh = workloads.custom_shape(T=T, d=512, E=16, K=4, I=256)
    say(f"layer graph capture T={T}")
    u = workloads.activations(sh).to(dev())
    e, b = workloads.centroids(sh).to(dev()), workloads.bias(sh).to(dev())
    packed = pack_all(sh)
    ws = torch.empty(moe.load_library().moe_layer_workspace_bytes(T, sh.d, sh.E, sh.K, sh.I),
                     dtype=torch.uint8, device=dev())
    out = torch.empty(T, sh.d, device=dev())
    ref = moe.moe_layer_forward(u, e, b, packed, sh.K, sh.I).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layer_forward(u, e, b, packed, sh.K, sh.I, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_layer_forward(u, e, b, packed, sh.K, sh.I, out=out, ws=ws)
    torch.cuda.synchronize()
    u2 = torch.flip(u, dims=[0]).contiguous()
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep
        other = moe.moe_layer_forward(u2, e, b, packed, sh.K, sh.I)      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other[0].view(torch.int32), ref[T - 1].view(torch.int32))
