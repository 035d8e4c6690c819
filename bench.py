"""Benchmark of the DeepSeekMoE layer forward on one MI355X.

One step = one pass of the whole layer over one batch held in HBM:
router (sigmoid affinity + biased top-K + gates) -> dispatch (histogram, scan,
permutation) -> 1x128 FP8 quantisation of u -> grouped GEMM1 with SwiGLU and
1x128 re-quantisation -> grouped GEMM2 -> combine (u + shared + gated routed)
-> bias update (into the next step's bias).  Expert weights are quantised to
128x128-block E4M3 once, before timing (an offline step).

Default workload: the prefill-shaped layer, T=16384 tokens, d=7168, 256 routed
experts top-8 + 1 shared, SwiGLU inter=2048, router bias calibrated for a
Zipf(1.1)-like expert load (max/mean ~4), u ~ N(0,1) with 0.1% outliers x100.
Other workloads (--workload): decode (T=256), rdc (router + dispatch + permute
+ combine with identity experts, T=8192), dense (block-scaled FP8 GEMM,
M=8192, N=7168, K=4096), tiny.

Prints one JSON line: tokens/s for the whole step, the roofline of the
dominant kernel (its average duration from HIP events on the launch stream
over the timed steps), and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sigmoid_top_routing_02_amd as moe  # noqa: E402
import workloads  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
MAX_SCLK_MHZ = 2400.0         # the shader clock the published peaks assume
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(name):
    with open(os.path.join(ROOT, "sigmoid_top_routing_02_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel_key, src):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel calibration), or None if the kernel
    source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(src):
        return None
    return rec.get("bytes_per_launch")


class Events:
    def __init__(self):
        self.pairs = {}

    def mark(self, name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        return ev

    def add(self, name, a, b):
        self.pairs.setdefault(name, []).append((a, b))

    def avg_ms(self, name):
        p = self.pairs.get(name, [])
        return float(np.mean([a.elapsed_time(b) for a, b in p])) if p else float("nan")


# ----------------------------------------------------------------------------- layer workloads
def pack_weights(sh):
    G = sh.E + 1
    packed = torch.empty(moe.moe_packed_weight_bytes(G, sh.d, sh.I), dtype=torch.uint8, device="cuda")
    for g in range(G):
        w1, w3, w2 = workloads.expert_weights(sh, g, device="cuda")
        moe.moe_prepare_expert_weights(w1, w3, w2, g, G, packed)
        del w1, w3, w2
    torch.cuda.synchronize()
    return packed


def layer_setup(sh):
    u = workloads.activations(sh).cuda()
    e = workloads.centroids(sh).cuda()
    b = workloads.bias(sh).cuda()
    packed = pack_weights(sh)
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    R = T * K + T
    dev = u.device
    st = dict(
        u=u, e=e, b=b, b_next=torch.empty_like(b), packed=packed,
        views=moe.packed_views(packed, E + 1, d, I),
        scores=torch.empty(T, E, dtype=torch.float32, device=dev),
        idx=torch.empty(T, K, dtype=torch.int32, device=dev),
        gate=torch.empty(T, K, dtype=torch.float32, device=dev),
        uq=torch.empty(T, d, dtype=torch.uint8, device=dev),
        us=torch.empty(T, d // 128, dtype=torch.float32, device=dev),
        hq=torch.empty(R, I, dtype=torch.uint8, device=dev),
        hs=torch.empty(R, I // 128, dtype=torch.float32, device=dev),
        y=torch.empty(R, d, dtype=torch.float32, device=dev),
        out=torch.empty(T, d, dtype=torch.float32, device=dev),
        dws=torch.empty(max(moe.moe_dispatch_workspace_bytes(T, E), 256), dtype=torch.uint8, device=dev),
        gws=torch.empty(max(moe.moe_gemm_workspace_bytes(E + 1, R, max(2 * I, d), max(I, d)), 256), dtype=torch.uint8, device=dev),
        # the shared expert's FFN as launches of its own (two-stream step):
        # one group of T rows, its own GEMM workspace, a second stream
        go_shared=torch.tensor([0, T], dtype=torch.int32, device=dev),
        gws_shared=torch.empty(max(moe.moe_gemm_workspace_bytes(1, T, max(2 * I, d), max(I, d)), 256), dtype=torch.uint8, device=dev),
        stream_b=torch.cuda.Stream(),
        ev_start=torch.cuda.Event(), ev_quant=torch.cuda.Event(), ev_shared=torch.cuda.Event(),
    )
    return st


def layer_step(sh, st, ev=None):
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    R = T * K + T
    w13q, w2q, w13s, w2s = st["views"]
    m = [ev.mark("start")] if ev else None
    moe.moe_router_topk(st["u"], st["e"], st["b"], K, st["scores"], st["idx"], st["gate"])
    if ev: m.append(ev.mark("router"))
    count, go, row_token, slot_row = moe.moe_dispatch(st["idx"], E, True, ws=st["dws"])
    if ev: m.append(ev.mark("dispatch"))
    moe.fp8_quant_1x128(st["u"], st["uq"], st["us"])
    if ev: m.append(ev.mark("quant"))
    moe.grouped_gemm_fp8_blockscaled(st["uq"], st["us"], go, R, w13q, w13s, epi=moe.MOE_EPI_SWIGLU_QUANT,
                                     a_row_index=row_token, out_q=st["hq"], out_scale=st["hs"], ws=st["gws"])
    if ev: m.append(ev.mark("gemm1"))
    moe.grouped_gemm_fp8_blockscaled(st["hq"], st["hs"], go, R, w2q, w2s, epi=moe.MOE_EPI_STORE_F32,
                                     out=st["y"], ws=st["gws"])
    if ev: m.append(ev.mark("gemm2"))
    moe.moe_combine(st["u"], st["y"], st["gate"], slot_row, shared_row0=T * K, out=st["out"])
    if ev: m.append(ev.mark("combine"))
    st["b_next"].copy_(st["b"])
    moe.moe_bias_update(st["b_next"], count, T * K, sh.gamma)
    if ev:
        m.append(ev.mark("bias"))
        names = ["router", "dispatch", "quant", "gemm1", "gemm2", "combine", "bias_update"]
        for i, n in enumerate(names):
            ev.add(n, m[i], m[i + 1])
    st["count"] = count


def layer_step_two_streams(sh, st):
    """The same layer step with the shared expert's FFN on a second stream.
    The shared expert's rows (GEMM rows T*K .. T*K+T-1) need no routing, so
    quant(u) goes first and the shared expert's GEMM1 and GEMM2 (one group of
    T rows, through offset views of the same h and Y buffers) run on stream B
    beside the router, dispatch and the routed experts' GEMMs (E groups, the
    first T*K rows) on the main stream; the combine waits for both.  Every
    output row is computed by the same tile arithmetic as in layer_step, so h'
    is bit-identical (checked by a GPU test); the gain is the two GEMM chains
    filling each other's partial last rounds of tiles.  The bias restore copy
    of the benchmark runs on stream B too.  The views start at GEMM row T*K,
    and the library takes 16-byte aligned buffers only: T*K*(I/128) must be a
    multiple of 4 (the h scales' rows; see shared_views_aligned)."""
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    TK = T * K
    w13q, w2q, w13s, w2s = st["views"]
    A, B = torch.cuda.current_stream(), st["stream_b"]
    moe.fp8_quant_1x128(st["u"], st["uq"], st["us"])
    st["ev_quant"].record(A)
    B.wait_event(st["ev_quant"])
    with torch.cuda.stream(B):
        st["b_next"].copy_(st["b"])
        moe.grouped_gemm_fp8_blockscaled(st["uq"], st["us"], st["go_shared"], T, w13q[E:], w13s[E:],
                                         epi=moe.MOE_EPI_SWIGLU_QUANT, out_q=st["hq"][TK:],
                                         out_scale=st["hs"][TK:], ws=st["gws_shared"])
        moe.grouped_gemm_fp8_blockscaled(st["hq"][TK:], st["hs"][TK:], st["go_shared"], T, w2q[E:], w2s[E:],
                                         epi=moe.MOE_EPI_STORE_F32, out=st["y"][TK:], ws=st["gws_shared"])
        st["ev_shared"].record(B)
    moe.moe_router_topk(st["u"], st["e"], st["b"], K, st["scores"], st["idx"], st["gate"])
    count, go, row_token, slot_row = moe.moe_dispatch(st["idx"], E, True, ws=st["dws"])
    moe.grouped_gemm_fp8_blockscaled(st["uq"], st["us"], go[:E + 1], TK, w13q[:E], w13s[:E],
                                     epi=moe.MOE_EPI_SWIGLU_QUANT, a_row_index=row_token[:TK],
                                     out_q=st["hq"][:TK], out_scale=st["hs"][:TK], ws=st["gws"])
    moe.grouped_gemm_fp8_blockscaled(st["hq"][:TK], st["hs"][:TK], go[:E + 1], TK, w2q[:E], w2s[:E],
                                     epi=moe.MOE_EPI_STORE_F32, out=st["y"][:TK], ws=st["gws"])
    A.wait_event(st["ev_shared"])
    moe.moe_combine(st["u"], st["y"], st["gate"], slot_row, shared_row0=TK, out=st["out"])
    moe.moe_bias_update(st["b_next"], count, TK, sh.gamma)
    st["count"] = count


def layer_step_gemm_events(sh, st, gev, quant_beside_router=False):
    """layer_step with HIP events around the two GEMM launches only (the
    roofline's live kernel times; events between every launch cost the
    decode step about 2%).  quant_beside_router: quant(u), which needs no
    routing, and the bias restore copy run on a second stream beside the
    router and dispatch (the matrix-core router and the bandwidth-bound quant
    share the chip; 9.455 -> 9.409 ms at prefill on one box), and GEMM1 waits
    for them; every launch the events bracket stays on the main stream."""
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    R = T * K + T
    w13q, w2q, w13s, w2s = st["views"]
    if quant_beside_router:
        A, B = torch.cuda.current_stream(), st["stream_b"]
        st["ev_start"].record(A)           # the previous step no longer reads uq, us or b_next
        B.wait_event(st["ev_start"])
        with torch.cuda.stream(B):
            moe.fp8_quant_1x128(st["u"], st["uq"], st["us"])
            st["b_next"].copy_(st["b"])
            st["ev_quant"].record(B)
    moe.moe_router_topk(st["u"], st["e"], st["b"], K, st["scores"], st["idx"], st["gate"])
    count, go, row_token, slot_row = moe.moe_dispatch(st["idx"], E, True, ws=st["dws"])
    if quant_beside_router:
        A.wait_event(st["ev_quant"])
    else:
        moe.fp8_quant_1x128(st["u"], st["uq"], st["us"])
    m = [gev.mark("gemm1")]
    moe.grouped_gemm_fp8_blockscaled(st["uq"], st["us"], go, R, w13q, w13s, epi=moe.MOE_EPI_SWIGLU_QUANT,
                                     a_row_index=row_token, out_q=st["hq"], out_scale=st["hs"], ws=st["gws"])
    m.append(gev.mark("gemm2"))
    moe.grouped_gemm_fp8_blockscaled(st["hq"], st["hs"], go, R, w2q, w2s, epi=moe.MOE_EPI_STORE_F32,
                                     out=st["y"], ws=st["gws"])
    m.append(gev.mark("end"))
    gev.add("gemm1", m[0], m[1])
    gev.add("gemm2", m[1], m[2])
    moe.moe_combine(st["u"], st["y"], st["gate"], slot_row, shared_row0=T * K, out=st["out"])
    if not quant_beside_router:
        st["b_next"].copy_(st["b"])
    moe.moe_bias_update(st["b_next"], count, T * K, sh.gamma)
    st["count"] = count


ONE_STREAM = False     # --one-stream: time the one-stream step at every size


def shared_views_aligned(sh):
    """The two-stream step's views of h codes, h scales and Y start at row
    T*K; each must start on a 16-byte boundary (d and I are multiples of 128,
    so only the h scales, I/128 floats per row, can miss it)."""
    return (sh.T * sh.K * (sh.I // 128)) % 4 == 0


def two_stream_step(sh):
    """Decode-shaped layers (T < 4096 at the model's width d >= 4096, weight
    streaming) time the two-stream step; at prefill the shared expert's GEMMs
    are a large share of the GEMM work and one stream keeps the GEMM pair's
    kernel times well defined, and a small layer (the tiny one: d = 512) is
    launch-bound, where the extra launches and cross-stream waits cost more
    than they hide (0.19 against 0.11 ms per step).  --one-stream times the
    one-stream step everywhere (counter profiles of whole-GEMM launches)."""
    return sh.T < 4096 and sh.d >= 4096 and shared_views_aligned(sh) and not ONE_STREAM


def layer_flops(sh):
    R = sh.T * (sh.K + 1)
    g1 = 2.0 * R * (2 * sh.I) * sh.d
    g2 = 2.0 * R * sh.d * sh.I
    return g1, g2


def gemm1_bytes(sh, count):
    """Algorithmic HBM bytes of GEMM1: every expert's W13 codes + scales that
    at least one row uses, the gathered A rows (codes + scales, once per
    row), and the h codes + scales written."""
    used = int((count > 0).sum()) + 1
    w = used * (2 * sh.I * sh.d + (2 * sh.I // 128) * (sh.d // 128) * 4)
    R = sh.T * (sh.K + 1)
    a = sh.T * (sh.d + sh.d // 128 * 4)
    h = R * (sh.I + sh.I // 128 * 4)
    return w + a + h


def layer_bytes(sh, count):
    """Algorithmic HBM bytes of one layer step as this path moves them: the
    W13 and W2 codes + scales of every expert with at least one row (and the
    shared one), u read once and the centroids, quantised u written and read,
    h codes + scales written and read, Y (FP32) written and read, h' written,
    and the routing arrays (scores, idx, gates, dispatch)."""
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    R = T * (K + 1)
    used = int((count > 0).sum()) + 1
    parts = {
        "weights": used * (3 * I * d + (2 * I // 128 + I // 128) * (d // 128) * 4),
        "u_centroids": T * d * 2 + E * d * 2,
        "u_quant": 2 * T * (d + d // 128 * 4),
        "h": 2 * R * (I + I // 128 * 4),
        "y": 2 * R * d * 4,
        "out": T * d * 4,
        "routing": T * E * 4 * 2 + T * K * 8 * 2 + R * 4 * 2 + T * K * 4 * 2,
    }
    parts["total"] = sum(parts.values())
    return parts


# ----------------------------------------------------------------------------- CPU baseline
def _oracle_layer_sample(sh, st, nt, groups, max_rows, budget_s, wq):
    """One timed oracle pass: router + dispatch + quant(u) on the first nt
    tokens, the FFN (GEMM1 + SwiGLU + h quant + GEMM2) of up to max_rows rows
    of each expert in `groups` (weights quantised beforehand, untimed), then
    combine + bias update.  Returns (per-token seconds, rows, seconds)."""
    import oracle
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    u_h = st["u"][:nt].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    e_h = st["e"].view(torch.int16).cpu().numpy().view(np.uint16)
    b_h = st["b"].cpu().numpy()
    t0 = time.perf_counter()
    idx, gate, s = oracle.router_topk(u_h, e_h, b_h, K)
    count, go, rt, sr = oracle.dispatch(idx, E, True)
    uf = (u_h.astype(np.uint32) << 16).view(np.float32)
    uq, us = oracle.quant_1x128(uf)
    t_route = time.perf_counter() - t0
    rows_done, t_ffn = 0, 0.0
    yfull = np.zeros((nt * (K + 1), d))
    for g in groups:
        r0, r1 = int(go[g]), int(go[g + 1])
        rows = np.arange(r0, min(r1, r0 + max_rows))
        if rows.size == 0:
            continue
        (q1, s1), (q3, s3), (q2, s2) = wq[g]
        t1 = time.perf_counter()
        zg = oracle.gemm_blockscaled(uq, us, q1, s1, a_rows=rt[rows])
        zu = oracle.gemm_blockscaled(uq, us, q3, s3, a_rows=rt[rows])
        h = oracle.swiglu(zg, zu).astype(np.float32)
        hq, hs = oracle.quant_1x128(h)
        yfull[rows] = oracle.gemm_blockscaled(hq, hs, q2, s2)
        t_ffn += time.perf_counter() - t1
        rows_done += rows.size
        if t_route + t_ffn > budget_s:
            break
    t2 = time.perf_counter()
    oracle.combine(u_h, yfull, nt * K, gate, sr)
    oracle.bias_update(b_h, count, nt * K, sh.gamma)
    t_comb = time.perf_counter() - t2
    whole = rows_done == nt * (K + 1)
    per_token = (t_route + t_ffn + t_comb) / nt if whole else \
        (t_route + t_comb) / nt + (K + 1) * t_ffn / rows_done
    return per_token, rows_done, t_route + t_ffn + t_comb, whole, [int(g) for g in groups]


def cpu_baseline_layer(sh, st, budget_s=15.0):
    """The oracle (untuned) timed on the host cores: on the tiny layer the
    whole layer over every token (with all threads, then on one thread); on
    the large layers a bounded sample -- router, dispatch, quant and combine
    on up to 4096 tokens, the FFNs of the shared expert and the 7 busiest
    experts' first 256 rows -- scaled to tokens/s (labelled extrapolated)."""
    import oracle
    oracle.lib()
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    whole_layer = T * (K + 1) <= 4096
    nt = T if whole_layer else min(T, 4096)
    if whole_layer:
        groups = list(range(E + 1))
    else:
        idx = st["idx"][:nt].cpu().numpy()
        busiest = np.argsort(-np.bincount(idx.reshape(-1), minlength=E), kind="stable")[:7]
        groups = [E] + [int(g) for g in busiest]
    wq = {}
    for g in groups:
        w1, w3, w2 = (w.cpu().numpy() for w in workloads.expert_weights(sh, g, device="cuda"))
        wq[g] = (oracle.quant_128x128(w1), oracle.quant_128x128(w3), oracle.quant_128x128(w2))
    threads = oracle.max_threads()
    max_rows = nt * (K + 1) if whole_layer else 256
    per_token, rows, secs, whole, groups = _oracle_layer_sample(sh, st, nt, groups, max_rows, budget_s, wq)
    res = {
        "value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "cpu_model": cpu_model(), "extrapolated": not whole,
        "sample": (f"the whole layer on all {nt} tokens ({secs:.1f}s)" if whole else
                   f"router+dispatch+quant+combine+bias on the first {nt} tokens; FFN on {rows} rows of experts "
                   f"{groups}; per-token cost = slice cost/{nt} + {K + 1} x per-row FFN cost ({secs:.1f}s)"),
    }
    if whole_layer:
        oracle.set_threads(1)
        try:
            pt1, _, secs1, _, _ = _oracle_layer_sample(sh, st, nt, groups, max_rows, budget_s, wq)
        finally:
            oracle.set_threads(threads)
        res["single_thread"] = {"value": round(1.0 / pt1, 2), "unit": "tokens/s", "cores": 1,
                                "sample": f"the whole layer on all {nt} tokens ({secs1:.1f}s)"}
    return res


# ----------------------------------------------------------------------------- runners
def layer_quant_error(sh, st, n_tok=4):
    """Quantisation error of the FP8 layer, reported beside the parity tests: the
    last step's output on sampled tokens (first, last and seeded others) against
    the same layer evaluated in FP64 with the unquantised FP32 master weights,
    the same bf16 input and the same routing (idx, gates): per-row inf-norm
    relative error, max over the tokens.  Plain torch on the GPU in FP64."""
    T, E = sh.T, sh.E
    toks = sorted({0, T - 1} | set(np.random.default_rng(5).integers(0, T, n_tok - 2).tolist()))
    u = st["u"][toks].double()
    idx = st["idx"][toks].cpu().numpy()
    gate = st["gate"][toks].double()
    ref = u.clone()
    for ex in sorted(set(idx.ravel().tolist()) | {E}):
        w1, w3, w2 = (w.double() for w in workloads.expert_weights(sh, ex, device="cuda"))
        for i in range(len(toks)):
            if ex == E:
                wgt = 1.0
            else:
                hit = np.nonzero(idx[i] == ex)[0]
                if hit.size == 0:
                    continue
                wgt = gate[i, int(hit[0])]
            z1, z3 = w1 @ u[i], w3 @ u[i]
            ref[i] += wgt * (w2 @ (z1 * torch.sigmoid(z1) * z3))
        del w1, w3, w2
    got = st["out"][toks].double()
    rel = float(((got - ref).abs().amax(dim=1) / ref.abs().amax(dim=1)).max())
    return {"tokens": len(toks), "norm": "per-row inf-norm relative, max over tokens",
            "vs_unquantised_fp64": round(rel, 6)}


def run_layer_backward(sh, steps, warmup):
    """The backward of the layer after one forward step whose GEMM1 kept z:
    gate backward (dY quantised), GEMM(dY, W2^T), SwiGLU backward (dz
    quantised), GEMM(dz, W13^T), du and the centroid gradient, then the expert
    weight gradients (transposed operands, one GEMM launch per expert and
    weight; the expert sizes are read back to the host for those launches).  One step = that chain for the whole batch
    with dL/dh' ~ N(0,1); the transposed weights are prepared once, untimed
    (like the forward's weight quantisation)."""
    log(f"[bench] setup {sh.name} backward: T={sh.T} d={sh.d} E={sh.E} K={sh.K} I={sh.I}")
    st = layer_setup(sh)
    layer_step(sh, st)
    T, d, E, K, I = sh.T, sh.d, sh.E, sh.K, sh.I
    G, R = E + 1, T * K + T
    count, go, row_token, slot_row = moe.moe_dispatch(st["idx"], E, True, ws=st["dws"])
    packed_t = moe.moe_prepare_backward_weights(st["packed"], G, d, I)
    w13q, w2q, w13s, w2s = st["views"]
    t13q, t2q, t13s, t2s = moe.packed_views(packed_t, G, d, I)
    t13q, t13s = t13q.view(G, d, 2 * I), t13s.view(G, d // 128, 2 * I // 128)
    t2q, t2s = t2q.view(G, I, d), t2s.view(G, I // 128, d // 128)
    dh = workloads.normal((T, d), 1.0, workloads.seed_for("backward", "dh", T), device="cuda")
    dev = dh.device
    # a training forward keeps GEMM1's output z for the SwiGLU backward: the
    # quantising epilogue that also stores z; its cost over the inference
    # epilogue is reported beside the backward
    z = torch.empty(R, 2 * I, device=dev)
    ev0 = Events()
    for kind in ("inference", "training"):
        for rep in range(3 + steps):
            a0 = ev0.mark("s")
            if kind == "inference":
                moe.grouped_gemm_fp8_blockscaled(st["uq"], st["us"], go, R, w13q, w13s, epi=moe.MOE_EPI_SWIGLU_QUANT,
                                                 a_row_index=row_token, out_q=st["hq"], out_scale=st["hs"],
                                                 ws=st["gws"])
            else:
                moe.grouped_gemm_fp8_blockscaled(st["uq"], st["us"], go, R, w13q, w13s,
                                                 epi=moe.MOE_EPI_SWIGLU_QUANT_Z, a_row_index=row_token,
                                                 out=z, out_q=st["hq"], out_scale=st["hs"], ws=st["gws"])
            if rep >= 3:
                ev0.add(kind, a0, ev0.mark("e"))
    torch.cuda.synchronize()
    fwd_gemm1 = {"inference_epilogue_ms": round(ev0.avg_ms("inference"), 4),
                 "training_epilogue_ms": round(ev0.avg_ms("training"), 4)}
    nk = max(2 * I, d)
    b = dict(dh_row=torch.empty(R, I, device=dev), z=z, dx=torch.empty(R, d, device=dev),
             ws=torch.empty(max(moe.moe_gemm_workspace_bytes(G, R, nk, nk), 256), dtype=torch.uint8, device=dev))

    def step(ev=None):
        m = [ev.mark("start")] if ev else None
        dy_q, dy_s, dlogit, row_dlogit = moe.moe_gate_backward(dh, st["y"], st["gate"], slot_row, st["scores"],
                                                               st["idx"], shared_row0=T * K)
        if ev: m.append(ev.mark("gate_bwd"))
        moe.grouped_gemm_fp8_blockscaled(dy_q, dy_s, go, R, t2q, t2s, epi=moe.MOE_EPI_STORE_F32,
                                         out=b["dh_row"], ws=b["ws"])
        if ev: m.append(ev.mark("gemm2_dgrad"))
        dz_q, dz_s = moe.moe_swiglu_backward(b["z"], b["dh_row"])
        if ev: m.append(ev.mark("swiglu_bwd"))
        moe.grouped_gemm_fp8_blockscaled(dz_q, dz_s, go, R, t13q, t13s, epi=moe.MOE_EPI_STORE_F32,
                                         out=b["dx"], ws=b["ws"])
        if ev: m.append(ev.mark("gemm1_dgrad"))
        moe.moe_router_backward(dh, b["dx"], slot_row, dlogit, st["idx"], st["e"], st["u"], row_dlogit,
                                row_token, go, shared_row0=T * K)
        if ev: m.append(ev.mark("router_bwd"))
        moe.moe_wgrad(dh, st["gate"], slot_row, row_token, b["z"], b["dh_row"], st["u"], go, shared_row0=T * K)
        if ev:
            m.append(ev.mark("wgrad"))
            names = ["gate_bwd", "gemm2_dgrad", "swiglu_bwd", "gemm1_dgrad", "router_bwd", "wgrad"]
            for i, n in enumerate(names):
                ev.add(n, m[i], m[i + 1])

    for _ in range(warmup):
        step()
    ev = Events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(ev)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    stages = {n: round(ev.avg_ms(n), 4) for n in ev.pairs}
    f2 = 2.0 * R * d * I              # GEMM(dY, W2^T)
    f1 = 2.0 * R * d * 2 * I          # GEMM(dz, W13^T)
    tf = {"gemm2_dgrad": round(f2 / (ev.avg_ms("gemm2_dgrad") * 1e-3) / 1e12, 1),
          "gemm1_dgrad": round(f1 / (ev.avg_ms("gemm1_dgrad") * 1e-3) / 1e12, 1),
          "wgrad_incl_operands": round((f1 + f2) / (ev.avg_ms("wgrad") * 1e-3) / 1e12, 1)}
    k_ms = ev.avg_ms("gemm1_dgrad")
    if T >= 4096:
        ach = f1 / (k_ms * 1e-3) / 1e12
        roof = {"kernel": "grouped_gemm_fp8_blockscaled (GEMM(dz, W13^T))", "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None,
                "algorithmic_per_launch": f1, "avg_launch_ms": round(k_ms, 4)}
    else:
        used = int((count.cpu() > 0).sum()) + 1
        nbytes = used * (d * 2 * I + (d // 128) * (2 * I // 128) * 4) + R * (2 * I + 2 * I // 128 * 4) + R * d * 4
        ach = nbytes / (k_ms * 1e-3) / 1e9
        roof = {"kernel": "grouped_gemm_fp8_blockscaled (GEMM(dz, W13^T))", "bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                "algorithmic_per_launch": nbytes, "avg_launch_ms": round(k_ms, 4)}
    log(f"[bench] backward {ms:.3f} ms/step; stages {stages}")
    return {
        "metric": "MoE-layer backward (input and weight gradients) tokens/s (d=7168, 256E top-8, FP8)",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": f"moe_layer_{sh.name}_backward", "T": T, "d": d, "routed_experts": E, "top_k": K,
                   "shared_experts": 1, "inter": I, "parallelism": "single GPU"},
        "roofline": roof, "stages_ms": stages, "gemm_tflops": tf,
        "forward_gemm1_for_training": fwd_gemm1,
    }


def run_layer(sh, steps, warmup, with_cpu):
    log(f"[bench] setup {sh.name}: T={sh.T} d={sh.d} E={sh.E} K={sh.K} I={sh.I}")
    t = time.time()
    st = layer_setup(sh)
    log(f"[bench] inputs + packed weights ready in {time.time() - t:.1f}s")
    two = two_stream_step(sh)
    gev = Events()
    # the timed step: two streams at decode (no events), one stream with
    # events around the GEMM pair at prefill (the roofline's kernel times)
    beside = sh.T >= 4096 and not ONE_STREAM   # prefill: quant(u) beside the router
    timed = ((lambda: layer_step_two_streams(sh, st)) if two else
             (lambda: layer_step_gemm_events(sh, st, gev, quant_beside_router=beside)))
    for _ in range(warmup):
        timed()
    torch.cuda.synchronize()
    gev.pairs.clear()
    log("[bench] warmup done")
    clocks_before = gpu_clocks()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        timed()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clocks_after = gpu_clocks()
    ms = wall * 1e3 / steps
    count = st["count"].cpu().numpy()
    # stage times: a separate pass of the one-stream step with events between
    # every launch (they lengthen the step, so they stay out of the timed loop)
    ev = Events()
    for _ in range(min(steps, 10)):
        layer_step(sh, st, ev)
    torch.cuda.synchronize()
    stages = {n: round(ev.avg_ms(n), 4) for n in ev.pairs}
    g1, g2 = layer_flops(sh)
    g1_ms, g2_ms = (ev.avg_ms("gemm1"), ev.avg_ms("gemm2")) if two else (gev.avg_ms("gemm1"), gev.avg_ms("gemm2"))
    if sh.T >= 4096:
        # the grouped GEMM as the pair of launches one step makes (GEMM1 with
        # the SwiGLU + requant epilogue, GEMM2 with the FP32 store): their
        # flops over their summed time, each launch also reported on its own
        achieved = (g1 + g2) / ((g1_ms + g2_ms) * 1e-3) / 1e12
        t1 = traffic_for(f"gemm1_{sh.name}", "gemm.hip")
        t2 = traffic_for(f"gemm2_{sh.name}", "gemm.hip")
        roof = {"kernel": "grouped_gemm_fp8_blockscaled (GEMM1 + GEMM2, the two launches of a step)",
                "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                "traffic": (t1 + t2) / 2 if t1 is not None and t2 is not None else None,
                "algorithmic_per_launch": (g1 + g2) / 2, "avg_launch_ms": round((g1_ms + g2_ms) / 2, 4),
                "gemm1": {"achieved": round(g1 / (g1_ms * 1e-3) / 1e12, 2),
                          "frac": round(g1 / (g1_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                          "algorithmic_per_launch": g1, "avg_launch_ms": round(g1_ms, 4), "traffic": t1},
                "gemm2": {"achieved": round(g2 / (g2_ms * 1e-3) / 1e12, 2),
                          "frac": round(g2 / (g2_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                          "algorithmic_per_launch": g2, "avg_launch_ms": round(g2_ms, 4), "traffic": t2}}
    else:
        # weight streaming: the whole layer step against HBM, with GEMM1 (the
        # largest stream) on its own
        nbytes = layer_bytes(sh, count)
        achieved = nbytes["total"] / (ms * 1e-3) / 1e9
        b1 = gemm1_bytes(sh, count)
        a1 = b1 / (g1_ms * 1e-3) / 1e9
        roof = {"kernel": "the whole layer step (all kernels" +
                          ("; the shared expert's FFN on a second stream)" if two else ", one stream)"),
                "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "algorithmic_per_launch": nbytes["total"], "avg_launch_ms": round(ms, 4),
                "bytes": nbytes,
                "gemm1": {"achieved": round(a1, 1), "frac": round(a1 / PEAK_HBM_GBS, 4),
                          "algorithmic_per_launch": b1, "avg_launch_ms": round(g1_ms, 4),
                          "timing": "one-stream pass with events between launches, after the timed loop",
                          "traffic": traffic_for(f"gemm1_{sh.name}", "gemm.hip")}}
    log(f"[bench] {ms:.3f} ms/step; stages {stages}")
    clk = sustained_clock(timed)
    log(f"[bench] sustained shader clock under this step: {clk}")
    if roof["bound"] == "mfma":
        at_clock(roof, clk)
    qerr = layer_quant_error(sh, st)
    log(f"[bench] quantisation error vs the unquantised layer: {qerr}")
    res = {
        "metric": "MoE-layer tokens/s (d=7168, 256E top-8, FP8) + % of FP8 MFMA / HBM roofline",
        "value": round(sh.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": f"moe_layer_{sh.name}", "T": sh.T, "d": sh.d, "routed_experts": sh.E,
                   "top_k": sh.K, "shared_experts": sh.shared, "inter": sh.I,
                   "load_max_over_mean": round(float(count.max() / count.mean()), 3),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "timed_step": ("two streams (the shared expert's FFN beside the routing and the routed experts), "
                       "no events") if two else
                      ("quant(u) on a second stream beside the router; routing and the GEMMs on one stream, "
                       "events around the two GEMM launches only") if beside else
                      "one stream, events around the two GEMM launches only",
        "stages_ms": stages,
        "stages_note": "one-stream step with events between every launch, a separate pass after the timed loop",
        "gemm_tflops": {"gemm1": round(g1 / (ev.avg_ms("gemm1") * 1e-3) / 1e12, 1),
                        "gemm2": round(g2 / (ev.avg_ms("gemm2") * 1e-3) / 1e12, 1)},
        "gpu_clocks_mhz": {"before": clocks_before, "after": clocks_after, "sustained": clk},
    }
    if with_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline_layer(sh, st)
    res["quant_error"] = qerr
    res["copy_ceiling_gbs"] = copy_ceiling_gbs()
    return res


def run_rdc(steps, warmup, with_cpu):
    """Router + dispatch + permute + combine with identity experts (Y = the
    permuted bf16 rows, no shared expert) + bias update, T=8192, d=7168,
    256 experts top-8: the bandwidth-bound part of the layer."""
    sh = workloads.SHAPES["rdc"]
    T, d, E, K = sh.T, sh.d, sh.E, sh.K
    log(f"[bench] setup rdc: T={T} d={d} E={E} K={K}")
    u = workloads.activations(sh).cuda()
    e = workloads.centroids(sh).cuda()
    b = workloads.bias(sh).cuda()
    st = dict(scores=torch.empty(T, E, device="cuda"), idx=torch.empty(T, K, dtype=torch.int32, device="cuda"),
              gate=torch.empty(T, K, device="cuda"), xp=torch.empty(T * K, d, dtype=torch.bfloat16, device="cuda"),
              out=torch.empty(T, d, device="cuda"), b_next=torch.empty_like(b),
              dws=torch.empty(max(moe.moe_dispatch_workspace_bytes(T, E), 256), dtype=torch.uint8, device="cuda"))

    def step(ev=None):
        m = [ev.mark("s")] if ev else None
        moe.moe_router_topk(u, e, b, K, st["scores"], st["idx"], st["gate"])
        if ev: m.append(ev.mark("router"))
        count, go, row_token, slot_row = moe.moe_dispatch(st["idx"], E, False, ws=st["dws"])
        if ev: m.append(ev.mark("dispatch"))
        moe.moe_permute_rows(u, row_token, out=st["xp"])
        if ev: m.append(ev.mark("permute"))
        moe.moe_combine(u, st["xp"], st["gate"], slot_row, shared_row0=-1, out=st["out"])
        if ev: m.append(ev.mark("combine"))
        st["b_next"].copy_(b)
        moe.moe_bias_update(st["b_next"], count, T * K, sh.gamma)
        if ev:
            m.append(ev.mark("bias"))
            for i, n in enumerate(["router", "dispatch", "permute", "combine", "bias_update"]):
                ev.add(n, m[i], m[i + 1])

    for _ in range(warmup):
        step()
    ev = Events()
    clocks_before = gpu_clocks()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(ev)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    clocks_after = gpu_clocks()
    stages = {n: round(ev.avg_ms(n), 4) for n in ev.pairs}
    balance = balance_loss_timing(st, steps)
    grouped = grouped_router_timing(u, e, b, K, st, steps)
    # algorithmic bytes of the combine: K bf16 rows of X_perm + u read, FP32 h' written, gates and slots
    comb_bytes = T * K * d * 2 + T * d * 2 + T * d * 4 + T * K * 8
    comb_ms = ev.avg_ms("combine")
    ach = comb_bytes / (comb_ms * 1e-3) / 1e9
    perm_bytes = T * K * d * 2 * 2 + T * K * 4
    res = {
        "metric": "router+dispatch+combine tokens/s (d=7168, 256E top-8) + % of HBM roofline",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 router/combine", "data": "synthetic (seeded)",
        "config": {"workload": "router_dispatch_combine", "T": T, "d": d, "routed_experts": E, "top_k": K,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "moe_combine", "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("combine_rdc", "combine.hip"),
                     "algorithmic_per_launch": comb_bytes, "avg_launch_ms": round(comb_ms, 4)},
        "stages_ms": stages,
        "permute_gbs": round(perm_bytes / (ev.avg_ms("permute") * 1e-3) / 1e9, 1),
        "grouped_router": grouped,
        "seq_balance_loss": balance,
        "router_tflops": round(2.0 * T * E * d / (ev.avg_ms("router") * 1e-3) / 1e12, 2),
        "gpu_clocks_mhz": {"before": clocks_before, "after": clocks_after},
    }
    if with_cpu:
        import oracle
        oracle.lib()

        def rdc_pass(nt):
            u_h = u[:nt].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            e_h = e.view(torch.int16).cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            idx, gate, s = oracle.router_topk(u_h, e_h, b.cpu().numpy(), K)
            cnt, go, rt, sr = oracle.dispatch(idx, E, False)
            uf = (u_h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            y = uf[rt]
            oracle.combine(u_h, y, -1, gate, sr)
            oracle.bias_update(b.cpu().numpy(), cnt, nt * K, sh.gamma)
            return time.perf_counter() - t0
        threads = oracle.max_threads()
        nt = 2048
        dt = rdc_pass(nt)
        oracle.set_threads(1)
        try:
            nt1 = 256
            dt1 = rdc_pass(nt1)
        finally:
            oracle.set_threads(threads)
        res["cpu_baseline"] = {"value": round(nt / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "cpu_model": cpu_model(), "extrapolated": True,
                               "sample": f"the whole rdc pass on the first {nt} of {T} tokens ({dt:.1f}s); "
                                         f"per-token work is independent, so tokens/s carries over",
                               "single_thread": {"value": round(nt1 / dt1, 1), "unit": "tokens/s", "cores": 1,
                                                 "sample": f"the same pass on the first {nt1} tokens ({dt1:.1f}s)"}}
    res["copy_ceiling_gbs"] = copy_ceiling_gbs()
    return res


COPY_ROWS, COPY_D = 32768, 65536     # 32768 rows x 65536 bf16 = 4 GiB


def copy_calibration():
    """A plain copy kernel of known size: 4 GiB read, 4 GiB written.  The
    source is 16x the 256 MB Infinity Cache, so nearly all of it comes from
    HBM."""
    src = torch.ones(COPY_ROWS, COPY_D, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    ident = torch.arange(COPY_ROWS, dtype=torch.int32, device="cuda")
    for _ in range(2):
        moe.moe_permute_rows(src, ident, out=dst)
    torch.cuda.synchronize()
    del src, dst


def balance_loss_timing(st, steps, seq_len=4096, alpha=1e-4):
    """The sequence-wise balance loss over the batch's scores and choices
    (sequences of 4096 tokens): time, the bytes it reads per second, values."""
    T, E = st["scores"].shape
    K = st["idx"].shape[1]
    moe.moe_seq_balance_loss(st["scores"], st["idx"], seq_len, alpha)
    ev = Events()
    for _ in range(steps):
        a0 = ev.mark("s")
        loss = moe.moe_seq_balance_loss(st["scores"], st["idx"], seq_len, alpha)
        ev.add("loss", a0, ev.mark("e"))
    torch.cuda.synchronize()
    ms = ev.avg_ms("loss")
    return {"seq_len": seq_len, "alpha": alpha, "ms": round(ms, 4),
            "read_gbs": round((T * E * 4 + T * K * 4) / (ms * 1e-3) / 1e9, 1),
            "loss": [round(float(x), 8) for x in loss.cpu()]}


def grouped_router_timing(u, e, b, K, st, steps, n_groups=8, topk_groups=4):
    """The group-limited router (8 groups of 32 experts, at most 4 groups per
    token, as the pages' 4-node limit) beside the plain one on the same batch:
    both calls run the score kernel and a top-K kernel; the difference is the
    group stage.  Also checks that no token's experts span more than 4 groups."""
    E = e.shape[0]
    ev = Events()
    for grouped in (False, True):
        kw = dict(n_groups=n_groups, topk_groups=topk_groups) if grouped else {}
        moe.moe_router_topk(u, e, b, K, st["scores"], st["idx"], st["gate"], **kw)
        for _ in range(steps):
            a0 = ev.mark("s")
            moe.moe_router_topk(u, e, b, K, st["scores"], st["idx"], st["gate"], **kw)
            ev.add("grouped" if grouped else "plain", a0, ev.mark("e"))
    torch.cuda.synchronize()
    groups = (st["idx"] // (E // n_groups)).cpu().numpy()
    span = max(len(set(r.tolist())) for r in groups)
    return {"n_groups": n_groups, "topk_groups": topk_groups, "router_ms": round(ev.avg_ms("plain"), 4),
            "grouped_router_ms": round(ev.avg_ms("grouped"), 4), "max_groups_per_token": span}


def copy_ceiling_gbs(reps=10):
    """The practical HBM ceiling: a plain 1 GiB bf16 copy (the library's row
    copy with the identity permutation; the source is 4x the 256 MB Infinity
    Cache), read + written bytes over the median of `reps` timed copies."""
    rows, d = 1 << 16, 8192
    src = torch.ones(rows, d, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    ident = torch.arange(rows, dtype=torch.int32, device="cuda")
    moe.moe_permute_rows(src, ident, out=dst)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_permute_rows(src, ident, out=dst)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    return round(2.0 * rows * d * 2 / (float(np.median(ts)) * 1e-3) / 1e9, 1)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_clocks():
    """Current GPU clocks in MHz as rocm-smi reports them (shader clock sclk,
    memory clock mclk, ...), or the reason they could not be read.  Read in a
    child process; a failure never stops the benchmark.  Skipped with
    --no-clock (profiler runs, whose preloaded library would follow the
    child process into rocm-smi)."""
    import re
    import subprocess
    if CLOCK_SECONDS <= 0:
        return {"skipped": "--no-clock"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
    except Exception as exc:              # tool missing, no permission, unparsable output
        return {"error": type(exc).__name__}
    out = {}
    for card, vals in data.items():
        if not isinstance(vals, dict):
            continue
        for k, v in vals.items():
            m = re.search(r"\(?(\d+)\s*Mhz", str(v), re.I)
            if m:
                out[f"{card}:{k}"] = int(m.group(1))
    return out or {"error": "no clock values in rocm-smi output"}


CLOCK_SECONDS = 3.0            # 0: skip the sustained-clock reading (--no-clock, for profiler runs)


def sustained_clock(step_fn, seconds=None):
    """The shader clock the GPU holds under this workload: step_fn runs back
    to back for `seconds` (synchronising every few calls) while a thread reads
    rocm-smi's current sclk every 0.25 s; the median of the samples after the
    first second (the clock starts near its maximum and settles as power
    rises).  Run after the timed region, so it never disturbs the timing."""
    import threading
    seconds = CLOCK_SECONDS if seconds is None else seconds
    if seconds <= 0:
        return {"skipped": "--no-clock"}
    samples, done = [], threading.Event()

    def sample():
        t0 = time.perf_counter()
        while not done.is_set():
            c = gpu_clocks()
            v = next((val for key, val in c.items() if "sclk clock speed" in key), None)
            if v is not None:
                samples.append((time.perf_counter() - t0, v))
            done.wait(0.25)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step_fn()
        torch.cuda.synchronize()
    done.set()
    th.join(timeout=35)
    late = [v for t, v in samples if t >= 1.0] or [v for _, v in samples]
    if not late:
        return {"error": "rocm-smi gave no sclk"}
    return {"sclk_median_mhz": int(np.median(late)), "sclk_min_mhz": int(min(late)),
            "sclk_max_mhz": int(max(late)), "samples": len(late), "seconds": seconds}


def at_clock(roof, clk):
    """Adds the MFMA peak at the measured sustained shader clock (the
    published peak assumes the 2.4 GHz maximum) and the fraction of it."""
    mhz = clk.get("sclk_median_mhz") if isinstance(clk, dict) else None
    if mhz:
        peak = PEAK_FP8_TFLOPS * mhz / MAX_SCLK_MHZ
        roof["peak_at_sustained_sclk"] = round(peak, 1)
        roof["frac_at_sustained_sclk"] = round(roof["achieved"] / peak, 4)
    return roof


def run_dense(steps, warmup, K=4096):
    M, N = workloads.DENSE["M"], workloads.DENSE["N"]
    log(f"[bench] dense GEMM M={M} N={N} K={K}")
    a, b = workloads.dense_operands(M, N, K, device="cuda")
    aq, as_ = moe.fp8_quant_1x128(a)
    bq, bs = moe.fp8_quant_128x128(b)
    # rows checked after timing: first, last and six seeded others
    rows = sorted({0, M - 1} | set(np.random.default_rng(11).integers(0, M, 6).tolist()))
    a_rows = a[rows].double().cpu()
    b_host = b.cpu()
    del a, b
    go = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    out = torch.empty(M, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(moe.moe_gemm_workspace_bytes(1, M, N, K), 256), dtype=torch.uint8, device="cuda")
    bq3, bs3 = bq.view(1, N, K), bs.view(1, N // 128, K // 128)
    for _ in range(warmup):
        moe.grouped_gemm_fp8_blockscaled(aq, as_, go, M, bq3, bs3, out=out, ws=ws)
    ev = Events()
    clocks_before = gpu_clocks()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        a0 = ev.mark("s")
        moe.grouped_gemm_fp8_blockscaled(aq, as_, go, M, bq3, bs3, out=out, ws=ws)
        ev.add("gemm", a0, ev.mark("e"))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    clocks_after = gpu_clocks()
    flops = 2.0 * M * N * K
    g_ms = ev.avg_ms("gemm")
    ach = flops / (g_ms * 1e-3) / 1e12
    clk = sustained_clock(lambda: moe.grouped_gemm_fp8_blockscaled(aq, as_, go, M, bq3, bs3, out=out, ws=ws))
    log(f"[bench] sustained shader clock under this GEMM: {clk}")
    err = dense_errors(out, aq, as_, bq, bs, rows, a_rows, b_host)
    del b_host
    acc = accumulation_probe(aq, bq, K)
    return {
        "metric": "block-scaled FP8 GEMM TFLOP/s", "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic", "config": {"workload": "dense_blockscaled_gemm", "M": M, "N": N, "K": K},
        "roofline": at_clock({"kernel": "grouped_gemm_fp8_blockscaled (1 group)", "bound": "mfma",
                              "achieved": round(ach, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(ach / PEAK_FP8_TFLOPS, 4),
                              "traffic": traffic_for(f"dense_k{K}", "gemm.hip")}, clk),
        "error": err,
        "accumulation": acc,
        "gpu_clocks_mhz": {"before": clocks_before, "after": clocks_after, "sustained": clk},
    }


def accumulation_probe(aq, bq, K, n=256):
    """FP8 MFMA accumulation with unit scales on the first n rows of A and B:
    one FP32 accumulator carried through every slice's MFMA (chained) against
    a fresh MFMA per 128-wide slice plus FP32 adds (promoted, the GEMM's path),
    both against the FP64 sum of the decoded codes."""
    a, b = aq[:n].contiguous(), bq[:n].contiguous()
    cha = moe.moe_fp8_mfma_accumulation_probe(a, b, chained=True)
    pro = moe.moe_fp8_mfma_accumulation_probe(a, b, chained=False)
    torch.cuda.synchronize()
    tab = torch.tensor([oracle_free_e4m3(c) for c in range(256)], dtype=torch.float64)
    exact = (tab[a.cpu().long()] @ tab[b.cpu().long()].T).numpy()
    def rel(x):
        x = x.double().cpu().numpy()
        den = np.maximum(np.abs(exact).max(axis=1), 1e-300)
        return float((np.abs(x - exact).max(axis=1) / den).max())
    return {"rows": n, "cols": n, "K": K, "scales": "unit (codes as quantised)",
            "norm": "per-row inf-norm relative vs FP64, max over rows",
            "chained": rel(cha), "promoted_per_128": rel(pro)}


def oracle_free_e4m3(code):
    """Value of an OCP E4M3 code (bias 7, no infinities, S.1111.111 = NaN)."""
    sgn = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    return sgn * (m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))


def dense_errors(out, aq, as_, bq, bs, rows, a_rows, b_host):
    """Per-row infinity-norm relative error of sampled output rows against the
    FP64 product of the dequantised operands (the GEMM's own contract) and
    against the FP64 product of the unquantised operands (the quantisation
    error), computed with plain torch on the host."""
    def deq(q, sc, rep_rows):
        v = q.view(torch.float8_e4m3fn).cpu().double()
        s = sc.cpu().double().repeat_interleave(128, dim=1)
        if rep_rows:
            s = s.repeat_interleave(128, dim=0)
        return v * s[: v.shape[0], : v.shape[1]]
    da = deq(aq[rows], as_[rows], False)
    db = deq(bq, bs, True)
    got = out[rows].double().cpu()
    ref_q = da @ db.T
    ref_u = a_rows @ b_host.double().T
    rel = lambda x, r: float(((x - r).abs().amax(dim=1) / r.abs().amax(dim=1)).max())
    return {"rows": len(rows), "norm": "per-row inf-norm relative, max over rows",
            "vs_fp64_of_dequantised": round(rel(got, ref_q), 8),
            "vs_unquantised": round(rel(got, ref_u), 6)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for the dense GEMM, whose step is ~0.3 ms, "
                         "and for the decode and tiny layers, whose steps take ~1.2 ms and less)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 5; 200 for the decode and tiny layers: their "
                         "short steps would otherwise be timed while the shader clock still ramps up)")
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "tiny", "rdc", "dense", "dense16k",
                             "prefill_bwd", "decode_bwd", "tiny_bwd"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-copy", action="store_true",
                    help="first run a plain 4 GiB copy kernel (moe_permute_rows with the identity "
                         "permutation) so a counter profile can calibrate FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock readings (rocm-smi before and after the timed region, and the "
                         "~3 s sustained-clock reading after it): profiler runs")
    ap.add_argument("--one-stream", action="store_true",
                    help="layer workloads: time the one-stream step also where the two-stream step is "
                         "the default (decode, tiny), so every GEMM launch covers all rows")
    args = ap.parse_args()
    if args.one_stream:
        global ONE_STREAM
        ONE_STREAM = True
    if args.no_clock:
        global CLOCK_SECONDS
        CLOCK_SECONDS = 0.0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this layer forward is a single-GPU path "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    short_step = args.workload in ("decode", "tiny")
    if args.steps is None:
        args.steps = 200 if args.workload in ("dense", "dense16k") or short_step else 20
    if args.warmup is None:
        args.warmup = 200 if short_step else 5
    moe.load_library()
    if args.with_copy:
        copy_calibration()
    if args.workload == "rdc":
        res = run_rdc(args.steps, args.warmup, with_cpu=not args.no_cpu_baseline)
    elif args.workload.endswith("_bwd"):
        res = run_layer_backward(workloads.SHAPES[args.workload[:-4]], args.steps, args.warmup)
    elif args.workload in ("dense", "dense16k"):
        res = run_dense(args.steps, args.warmup, K=4096 if args.workload == "dense" else 16384)
    else:
        res = run_layer(workloads.SHAPES[args.workload], args.steps, args.warmup,
                        with_cpu=not args.no_cpu_baseline)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
