"""Pins for the oracle's 1x128 / 128x128 quantisers, the block-scaled GEMM,
SwiGLU and the combine.

  * quantiser: the tile maximum encodes to +-448, the scale is amax/448,
    E4M3-exact tiles whose maximum is 448*2^-j round-trip exactly, the error
    bound of an E4M3 rounding holds after rescaling, an all-zero tile gets
    scale 1, one outlier only affects its own tile ("DeepSeek-V3 Technical
    Report" notes, FP8 paragraph), and codes equal torch's float8_e4m3fn
    conversion of x*inv;
  * GEMM: integer-valued operands give the exact int64 matmul; general
    operands equal numpy's FP64 matmul of the dequantised matrices; gathered
    rows equal the GEMM on the gathered matrix;
  * SwiGLU: torch's silu in FP64;
  * combine: zero expert outputs return u exactly; identity experts with gates
    summing to 1 return u + 2x (shared + routed).
"""
import numpy as np
import pytest
import torch


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_quant_1x128_properties(oracle_mod):
    rng = np.random.default_rng(20)
    rows, cols = 33, 512
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 6, (rows, 1)))).astype(np.float32)
    x[3, 7] = 100.0 * np.abs(x[3]).max()   # outlier
    x[5, 128:256] = 0.0           # all-zero tile
    q, sc = oracle_mod.quant_1x128(x)
    table = oracle_mod.e4m3_table()
    tiles = x.reshape(rows, cols // 128, 128)
    amax = np.abs(tiles).max(-1)
    nz = amax > 0
    np.testing.assert_array_equal(sc[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    assert sc[5, 1] == 1.0 and np.all(q[5, 128:256] == 0)
    # the element holding the tile maximum encodes to +-448
    qt = q.reshape(rows, cols // 128, 128)
    arg = np.abs(tiles).argmax(-1)
    top = np.take_along_axis(qt, arg[..., None], -1)[..., 0]
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # codes are torch's E4M3 rounding of x * fl32(448/amax)
    inv = np.where(nz, (np.float32(448) / np.where(nz, amax, 1)).astype(np.float32), np.float32(1))
    scaled = (tiles * inv[..., None]).astype(np.float32)
    np.testing.assert_array_equal(qt, _torch_e4m3(scaled))
    # dequantised error bound: half an E4M3 step, relative 2^-4 in the normal range
    deq = table[qt] * sc[..., None].astype(np.float64)
    err = np.abs(deq - tiles)
    bound = np.maximum(2.0 ** -4 * np.abs(tiles), 2.0 ** -10 * sc[..., None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the outlier's effect stays inside its tile: other tiles of row 3 keep small scales
    assert sc[3, 0] > 10 * np.median(sc[3, 1:])


def test_quant_exact_tiles_roundtrip(oracle_mod):
    """A tile of E4M3 values whose maximum is 448*2^-j is represented exactly."""
    rng = np.random.default_rng(21)
    table = oracle_mod.e4m3_table()
    finite = np.array([c for c in range(256) if np.isfinite(table[c])])
    codes = rng.choice(finite, (4, 384))
    vals = table[codes].astype(np.float32)
    vals[:, ::128] = 448.0
    for j, r in enumerate(vals):
        vals[j] = r * np.float32(2.0 ** -j)
    q, sc = oracle_mod.quant_1x128(vals)
    np.testing.assert_array_equal(oracle_mod.dequant_1x128(q, sc), vals.astype(np.float64))


def test_quant_128x128_properties(oracle_mod):
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[130, 5] = 3.0
    q, sc = oracle_mod.quant_128x128(w)
    blocks = w.reshape(2, 128, 3, 128).transpose(0, 2, 1, 3)
    amax = np.abs(blocks).max((-1, -2))
    np.testing.assert_array_equal(sc, (amax / np.float32(448)).astype(np.float32))
    inv = (np.float32(448) / amax).astype(np.float32)
    scaled = (blocks * inv[..., None, None]).astype(np.float32)
    qb = q.reshape(2, 128, 3, 128).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(qb, _torch_e4m3(scaled))
    assert q[130, 5] == 0x7E
    # the outlier inflates only block (1, 0)
    assert sc[1, 0] > 20 * sc[0, 0]


def test_quant_128x128_matches_1x128_on_constant_scale_rows(oracle_mod):
    """If every row of a 128x128 block shares the block maximum, the 128x128
    quantiser and the 1x128 quantiser give the same codes."""
    rng = np.random.default_rng(23)
    w = rng.uniform(-1, 1, (128, 256)).astype(np.float32)
    w[:, 0] = 2.0
    w[:, 128] = -2.0
    q1, s1 = oracle_mod.quant_1x128(w)
    q2, s2 = oracle_mod.quant_128x128(w)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1[0], s2[0])


# ------------------------------------------------------------------ GEMM
def _int_codes(rng, shape, table, maxabs=8):
    """E4M3 codes of small integers (exact in E4M3)."""
    v = rng.integers(-maxabs, maxabs + 1, shape).astype(np.float32)
    return _torch_e4m3(v), v


def test_gemm_integer_operands_exact(oracle_mod):
    rng = np.random.default_rng(24)
    table = oracle_mod.e4m3_table()
    M, N, K = 19, 256, 384
    qa, va = _int_codes(rng, (M, K), table)
    qb, vb = _int_codes(rng, (N, K), table)
    out = oracle_mod.gemm_blockscaled(qa, np.ones((M, K // 128), np.float32), qb,
                                      np.ones((N // 128, K // 128), np.float32))
    exact = va.astype(np.int64) @ vb.astype(np.int64).T
    np.testing.assert_array_equal(out, exact.astype(np.float64))


def test_gemm_matches_fp64_matmul_of_dequantised(oracle_mod):
    rng = np.random.default_rng(25)
    table = oracle_mod.e4m3_table()
    M, N, K = 23, 384, 640
    xa = rng.standard_normal((M, K)).astype(np.float32)
    xb = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    qa, sa = oracle_mod.quant_1x128(xa)
    qb, sb = oracle_mod.quant_128x128(xb)
    out = oracle_mod.gemm_blockscaled(qa, sa, qb, sb)
    da = table[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    db = table[qb] * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)
    ref = da @ db.T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # per-slice scales matter: swapping two slices' scales changes the result
    sa2 = sa.copy()
    sa2[:, [0, 1]] = sa2[:, [1, 0]]
    out2 = oracle_mod.gemm_blockscaled(qa, sa2, qb, sb)
    assert np.abs(out2 - out).max() > 1e-6


def test_gemm_gathered_rows(oracle_mod):
    rng = np.random.default_rng(26)
    M, N, K = 30, 128, 256
    qa, sa = oracle_mod.quant_1x128(rng.standard_normal((M, K)).astype(np.float32))
    qb, sb = oracle_mod.quant_128x128(rng.standard_normal((N, K)).astype(np.float32))
    rows = rng.integers(0, M, 50).astype(np.int32)
    a = oracle_mod.gemm_blockscaled(qa, sa, qb, sb, a_rows=rows)
    b = oracle_mod.gemm_blockscaled(qa[rows], sa[rows], qb, sb)
    np.testing.assert_array_equal(a, b)
    assert oracle_mod.gemm_blockscaled(qa, sa, qb, sb, a_rows=np.zeros(0, np.int32)).shape == (0, N)


def test_swiglu_matches_torch_silu(oracle_mod):
    rng = np.random.default_rng(27)
    zg = rng.standard_normal(10000) * 4
    zu = rng.standard_normal(10000)
    h = oracle_mod.swiglu(zg, zu)
    ref = (torch.nn.functional.silu(torch.from_numpy(zg)) * torch.from_numpy(zu)).numpy()
    np.testing.assert_allclose(h, ref, rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------ combine
def _u_bits(rng, T, d):
    return (rng.standard_normal((T, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_combine_zero_experts_returns_u(oracle_mod):
    rng = np.random.default_rng(28)
    T, d, K, E = 20, 256, 4, 8
    u = _u_bits(rng, T, d)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, row_token, slot_row = oracle_mod.dispatch(idx, E, True)
    gate = rng.uniform(0, 1, (T, K)).astype(np.float32)
    out = oracle_mod.combine(u, np.zeros((T * K + T, d)), T * K, gate, slot_row)
    uf = (u.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(out, uf.astype(np.float64))


def test_combine_identity_experts_conserve(oracle_mod):
    """With every expert the identity, h' = u + x_shared + sum_k g_k x = u + 2x
    (gates sum to 1); without the shared term, u + x."""
    rng = np.random.default_rng(29)
    T, d, K, E = 25, 128, 8, 32
    u = _u_bits(rng, T, d)
    x = rng.standard_normal((T, d))
    s = oracle_mod.sigmoid_spec_array(rng.standard_normal((T, E)).astype(np.float32))
    idx, gate = oracle_mod.topk_from_scores(s, np.zeros(E, np.float32), K)
    uf = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for shared in (True, False):
        _, _, row_token, slot_row = oracle_mod.dispatch(idx, E, shared)
        y = x[row_token]
        out = oracle_mod.combine(u, y, T * K if shared else -1, gate, slot_row)
        np.testing.assert_allclose(out, uf + (2.0 if shared else 1.0) * x, atol=1e-6)
