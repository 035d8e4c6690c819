"""Pins for the oracle's whole-layer composition (nlp-lineage summary, "The
notation": h'_t = u_t + sum_shared FFN_i(u_t) + sum_routed g_(i,t) FFN_i(u_t)).

Special case that reduces to a plain formula: when every expert (shared and
routed) holds the same weights and K = E, every routed gate set sums to 1, so
    h' = u + FFN(u) + (sum_k g_k) FFN(u) = u + 2 FFN(u).
The unquantised layer must match that with FFN computed by torch in FP64; the
quantised layer must match it with FFN computed by numpy/torch on the
dequantised operands (u per 1x128 tile, weights per 128x128 block, h per 1x128
tile).  A dropped shared term, a wrong gate or a transposed weight fails it.
"""
import numpy as np
import torch

import workloads


def _setup(T=8, d=256, E=4, I=128, K=4, seed=30):
    rng = np.random.default_rng(seed)
    u = (rng.standard_normal((T, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    e = ((rng.standard_normal((E, d)) * d ** -0.5).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    w1 = (rng.standard_normal((I, d)) * d ** -0.5).astype(np.float32)
    w3 = (rng.standard_normal((I, d)) * d ** -0.5).astype(np.float32)
    w2 = (rng.standard_normal((d, I)) * d ** -0.5).astype(np.float32)
    return u, e, b, (w1, w3, w2), K


def _ffn_torch(x, w1, w3, w2):
    x, w1, w3, w2 = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, w1, w3, w2))
    return (torch.nn.functional.silu(x @ w1.T) * (x @ w3.T) @ w2.T).numpy()


def test_unquantised_layer_identical_experts(oracle_mod):
    u, e, b, W, K = _setup()
    r = oracle_mod.layer_forward_unquantised(u, e, b, K, lambda g: W, shared=True)
    uf = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = uf + 2.0 * _ffn_torch(uf, *W)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-6, atol=1e-6)


def test_quantised_layer_identical_experts(oracle_mod):
    u, e, b, W, K = _setup()
    r = oracle_mod.layer_forward(u, e, b, K, lambda g: W, shared=True)
    table = oracle_mod.e4m3_table()
    uf = (u.astype(np.uint32) << 16).view(np.float32)
    uq, us = oracle_mod.quant_1x128(uf)
    ud = table[uq] * np.repeat(us.astype(np.float64), 128, 1)

    def deq_block(w):
        q, s = oracle_mod.quant_128x128(w)
        return table[q] * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)

    w1d, w3d, w2d = (deq_block(w) for w in W)
    h = (torch.nn.functional.silu(torch.from_numpy(ud @ w1d.T)) * torch.from_numpy(ud @ w3d.T)).numpy()
    hq, hs = oracle_mod.quant_1x128(h.astype(np.float32))
    hd = table[hq] * np.repeat(hs.astype(np.float64), 128, 1)
    ffn = hd @ w2d.T
    ref = uf.astype(np.float64) + 2.0 * ffn
    np.testing.assert_allclose(r["out"], ref, rtol=1e-6, atol=1e-6)


def test_quantised_vs_unquantised_tiny_workload(oracle_mod):
    """Quantisation error of the tiny workload, reported and loosely bounded.
    Every E4M3 rounding has a relative RMS error of roughly 2.5%; u, W1/W3, h
    and W2 are each rounded once and a dot product does not average relative
    errors away, so the FFN part of h' carries a few percent."""
    sh = workloads.SHAPES["tiny"]
    u = workloads.activations(sh).view(torch.int16).numpy().view(np.uint16)
    e = workloads.centroids(sh).view(torch.int16).numpy().view(np.uint16)
    b = workloads.bias(sh).numpy()
    W = {g: tuple(t.numpy() for t in workloads.expert_weights(sh, g)) for g in range(sh.E + 1)}
    q = oracle_mod.layer_forward(u, e, b, sh.K, lambda g: W[g])
    f = oracle_mod.layer_forward_unquantised(u, e, b, sh.K, lambda g: W[g])
    np.testing.assert_array_equal(q["idx"], f["idx"])
    uf = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ffn_q = q["out"] - uf
    ffn_f = f["out"] - uf
    fro = np.linalg.norm(ffn_q - ffn_f) / np.linalg.norm(ffn_f)
    rel_max = np.abs(ffn_q - ffn_f).max() / np.abs(ffn_f).max()
    print(f"tiny workload FP8 quantisation error of the FFN sum: frobenius {fro:.4f}, max {rel_max:.4f}")
    assert fro < 0.10 and rel_max < 0.20, (fro, rel_max)
    # structural facts: K distinct routed experts + 1 shared per token, no drop
    assert q["row_token"].shape[0] == sh.T * sh.K + sh.T
    assert q["count"].sum() == sh.T * sh.K
