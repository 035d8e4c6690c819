"""GPU parity: E4M3 quantisers (bit-exact) and the block-scaled grouped FP8
GEMM with its three epilogues (FP32 outputs within the per-row relative
bound, integer-valued cases bit-exact, quantised SwiGLU output checked code by
code)."""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_top_routing_02_amd as moe
from helpers import TOL, dev, np_, rowinf_rel, say

pytestmark = pytest.mark.gpu


def _special_rows(cols):
    """Rows that exercise zero tiles, subnormal-range values, saturation and
    rounding midpoints."""
    rows = []
    rows.append(np.zeros(cols, np.float32))
    r = np.full(cols, 1e-30, np.float32)
    r[::7] = 3e-38
    rows.append(r)
    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    r = np.resize(np.concatenate([mids, -mids]), cols).astype(np.float32)
    r[0] = 448.0             # tile max 448 -> inv = 1: midpoints stay midpoints
    r[128::128] = 448.0
    rows.append(r)
    r = np.linspace(-1e4, 1e4, cols).astype(np.float32)
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("rows,cols", [(1, 128), (333, 512), (4096, 7168)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_1x128_bit_exact(rows, cols, dtype):
    say(f"quant 1x128 {rows}x{cols} {dtype}")
    g = torch.Generator().manual_seed(rows + cols)
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 3)
    if rows > 10:
        x[:4] = torch.from_numpy(_special_rows(cols))
        x[5, 17] = 1e4           # outlier
    x = x.to(dtype)
    q, sc = moe.fp8_quant_1x128(x.to(dev()))
    torch.cuda.synchronize()
    xf = x.float().numpy()
    q_ref, sc_ref = oracle.quant_1x128(xf)
    np.testing.assert_array_equal(np_(sc).view(np.uint32), sc_ref.view(np.uint32))
    np.testing.assert_array_equal(np_(q), q_ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_1x128_nan_and_inf(dtype):
    """Non-finite inputs through the E4M3 encoder: a NaN input keeps its sign
    (code 0x7F / 0xFF) and does not enter the tile maximum; a tile holding
    +-inf has amax = inf, so inv = 448/inf = 0 and scale = inf (the scale rule
    as written), and inf * 0 is a NaN generated inside the quantiser, whose
    sign IEEE leaves to the platform: there the codes must be NaN codes
    (low seven bits 0x7F), elsewhere they are bit-exact."""
    say(f"quant 1x128 nan/inf {dtype}")
    x = np.ones((4, 256), np.float32) * np.linspace(-3, 3, 256, dtype=np.float32)
    x[0, 3], x[0, 4], x[0, 200] = np.nan, -np.nan, np.nan      # NaNs of both signs
    x[1, 5], x[1, 6], x[1, 130] = np.inf, -np.inf, 1e30         # tiles with +-inf
    x[2, :] = 0.0
    x[2, 7] = -np.nan
    x[3, 129] = np.inf
    xt = torch.from_numpy(x).to(dtype)
    q, sc = moe.fp8_quant_1x128(xt.to(dev()))
    torch.cuda.synchronize()
    q_ref, sc_ref = oracle.quant_1x128(xt.float().numpy())
    np.testing.assert_array_equal(np_(sc).view(np.uint32), sc_ref.view(np.uint32))
    qg = np_(q)
    generated = np.zeros_like(qg, dtype=bool)          # inf * 0 inside a tile with amax = inf
    tile_inf = np.isinf(xt.float().numpy()).reshape(4, 2, 128).any(axis=2)
    generated |= (np.repeat(tile_inf, 128, axis=1) & np.isinf(xt.float().numpy()))
    np.testing.assert_array_equal(qg[~generated], q_ref[~generated])
    assert np.all((qg[generated] & 0x7F) == 0x7F) and np.all((q_ref[generated] & 0x7F) == 0x7F)


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 640), (2048, 7168)])
def test_quant_128x128_bit_exact(rows, cols):
    say(f"quant 128x128 {rows}x{cols}")
    g = torch.Generator().manual_seed(rows * 3 + cols)
    w = torch.randn(rows, cols, generator=g) * cols ** -0.5
    w[0, :128] = 0.0
    w[0:128, 0:128] = 0.0    # an all-zero block -> scale 1
    w[min(130, rows - 1), 300 % cols] = 5.0
    q, sc = moe.fp8_quant_128x128(w.to(dev()))
    torch.cuda.synchronize()
    q_ref, sc_ref = oracle.quant_128x128(w.numpy())
    np.testing.assert_array_equal(np_(sc).view(np.uint32), sc_ref.view(np.uint32))
    np.testing.assert_array_equal(np_(q), q_ref)


# ------------------------------------------------------------------ GEMM helpers
def _groups(sizes):
    go = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return go


def _int_operands(M, N, K, G, seed):
    """E4M3 codes of small integers; all scales 1 -> every result is an exact integer."""
    rng = np.random.default_rng(seed)
    va = rng.integers(-8, 9, (M, K)).astype(np.float32)
    vb = rng.integers(-8, 9, (G, N, K)).astype(np.float32)
    qa = oracle.e4m3_encode_array(va)
    qb = oracle.e4m3_encode_array(vb)
    return va, vb, qa, qb


# The library takes 128-row tiles when the groups average more than 64 rows
# and 32-row tiles otherwise; the cases below cover both.
@pytest.mark.parametrize("sizes,N,K", [
    ([600, 0, 900], 512, 384),         # large ragged groups incl. an empty one (128-row tiles)
    ([513], 384, 256),                 # N % 256 == 128, one row in the last tile (128)
    ([1024], 256, 128),                # a single K slice (128)
    ([768, 400], 256, 640),            # five slices: the three-stage remainder (128)
    ([128], 256, 128),                 # one tile (128-row tiles)
    ([1], 256, 256),                   # one row (32-row tiles)
    ([200, 0, 57, 128, 1], 512, 384),  # ragged groups incl. an empty one (128)
    ([300], 384, 256),                 # N % 256 == 128, masked half tile (128)
    ([5, 40, 0, 33, 9, 64], 512, 384), # ragged groups, 32-row tiles
    ([7, 31, 70], 384, 256),           # N % 256 == 128 with 32-row tiles
    ([5, 40, 0, 33, 9, 64], 512, 640), # 32-row tiles of five slices
    ([7, 31, 70], 384, 1024),          # N % 256 == 128, 32-row tiles of eight slices
])
def test_gemm_integer_exact(sizes, N, K):
    """Exact integer results pin the MFMA operand/accumulator layouts, the
    k-slice walk, the gather and the group map bit for bit."""
    G = len(sizes)
    go = _groups(sizes)
    M = int(go[-1])
    say(f"gemm integer sizes={sizes} N={N} K={K}")
    va, vb, qa, qb = _int_operands(M + 5, N, K, G, seed=M + N)
    rows = np.random.default_rng(1).permutation(M + 5)[:M].astype(np.int32)   # gather
    out = moe.grouped_gemm_fp8_blockscaled(
        torch.from_numpy(qa).to(dev()), torch.ones(M + 5, K // 128, device=dev()),
        torch.from_numpy(go).to(dev()), M, torch.from_numpy(qb).to(dev()),
        torch.ones(G, N // 128, K // 128, device=dev()), epi=moe.MOE_EPI_STORE_F32,
        a_row_index=torch.from_numpy(rows).to(dev()))
    torch.cuda.synchronize()
    ref = np.zeros((M, N))
    for gi in range(G):
        r0, r1 = go[gi], go[gi + 1]
        ref[r0:r1] = va[rows[r0:r1]].astype(np.int64) @ vb[gi].astype(np.int64).T
    np.testing.assert_array_equal(np_(out), ref.astype(np.float32))


@pytest.mark.parametrize("G", [4096, 4100])
def test_gemm_integer_exact_many_groups(G):
    """The tile map for many groups: up to 4096 groups the map, the tile list
    and the scale gather run as one launch that scans the groups in each list
    block; beyond, as three launches.  Two non-empty groups (one of them the
    last), every other group empty; B is only filled where it is read."""
    N, K = 256, 256
    sizes = np.zeros(G, np.int64)
    sizes[17], sizes[G - 1] = 200, 77
    go = _groups(sizes)
    M = int(go[-1])
    say(f"gemm integer G={G} M={M} N={N} K={K}")
    va, vb2, qa, qb2 = _int_operands(M, N, K, 2, seed=G)
    qb = torch.zeros(G, N, K, dtype=torch.uint8, device=dev())
    qb[17] = torch.from_numpy(qb2[0]).to(dev())
    qb[G - 1] = torch.from_numpy(qb2[1]).to(dev())
    out = moe.grouped_gemm_fp8_blockscaled(
        torch.from_numpy(qa).to(dev()), torch.ones(M, K // 128, device=dev()),
        torch.from_numpy(go).to(dev()), M, qb,
        torch.ones(G, N // 128, K // 128, device=dev()), epi=moe.MOE_EPI_STORE_F32)
    torch.cuda.synchronize()
    ref = np.zeros((M, N))
    ref[:200] = va[:200].astype(np.int64) @ vb2[0].astype(np.int64).T
    ref[200:] = va[200:].astype(np.int64) @ vb2[1].astype(np.int64).T
    np.testing.assert_array_equal(np_(out), ref.astype(np.float32))


def _scaled_operands(M, N, K, G, seed, outliers=True):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(M, K, generator=g)
    if outliers:
        pos = torch.randperm(M * K, generator=g)[: max(1, M * K // 1000)]
        a.view(-1)[pos] *= 100
    b = torch.randn(G, N, K, generator=g) * K ** -0.5
    qa, sa = oracle.quant_1x128(a.numpy())
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, N // 128, K // 128), np.float32)
    for gi in range(G):
        qb[gi], sb[gi] = oracle.quant_128x128(b[gi].numpy())
    return qa, sa, qb, sb


@pytest.mark.parametrize("sizes,N,K", [([129, 3, 0, 250], 256, 512), ([1000], 768, 1024),
                                       ([20, 3, 0, 45, 9], 256, 512)])
def test_gemm_store_f32_vs_oracle(sizes, N, K):
    G = len(sizes)
    go = _groups(sizes)
    M = int(go[-1])
    say(f"gemm store sizes={sizes} N={N} K={K}")
    qa, sa, qb, sb = _scaled_operands(M, N, K, G, seed=N + K)
    out = moe.grouped_gemm_fp8_blockscaled(
        torch.from_numpy(qa).to(dev()), torch.from_numpy(sa).to(dev()), torch.from_numpy(go).to(dev()),
        M, torch.from_numpy(qb).to(dev()), torch.from_numpy(sb).to(dev()), epi=moe.MOE_EPI_STORE_F32)
    torch.cuda.synchronize()
    ref = np.zeros((M, N))
    for gi in range(G):
        r0, r1 = go[gi], go[gi + 1]
        ref[r0:r1] = oracle.gemm_blockscaled(qa[r0:r1], sa[r0:r1], qb[gi], sb[gi])
    err = rowinf_rel(np_(out), ref)
    say(f"  per-row rel err {err:.3e}")
    assert err <= TOL


def _interleave(w1, w3):
    """Packed gate/up rows: 128-row blocks of W1 and W3 alternate."""
    I = w1.shape[0]
    out = np.empty((2 * I,) + w1.shape[1:], w1.dtype)
    for j in range(I // 128):
        out[256 * j:256 * j + 128] = w1[128 * j:128 * (j + 1)]
        out[256 * j + 128:256 * j + 256] = w3[128 * j:128 * (j + 1)]
    return out


@pytest.mark.parametrize("sizes,I,d", [([130, 0, 77, 256], 256, 512), ([64], 512, 256), ([700, 300], 256, 640),
                                       ([9, 0, 33, 12, 50], 256, 512)])
def test_gemm_swiglu_epilogues(sizes, I, d):
    """SwiGLU FP32 h against the oracle's FP64 h; the fused quantising
    epilogue equals SwiGLU_F32 followed by fp8_quant_1x128 bit for bit; its
    codes equal the oracle's quantiser on the oracle's h except where the
    FP32/FP64 difference straddles a rounding midpoint."""
    G = len(sizes)
    go = _groups(sizes)
    M = int(go[-1])
    say(f"gemm swiglu sizes={sizes} I={I} d={d}")
    g = torch.Generator().manual_seed(M + I)
    u = torch.randn(M + 3, d, generator=g)
    rows = torch.randperm(M + 3, generator=g)[:M].to(torch.int32)
    qa, sa = oracle.quant_1x128(u.numpy())
    qb = np.empty((G, 2 * I, d), np.uint8)
    sb = np.empty((G, 2 * I // 128, d // 128), np.float32)
    w1s, w3s = [], []
    for gi in range(G):
        w1 = (torch.randn(I, d, generator=g) * d ** -0.5).numpy()
        w3 = (torch.randn(I, d, generator=g) * d ** -0.5).numpy()
        q1, s1 = oracle.quant_128x128(w1)
        q3, s3 = oracle.quant_128x128(w3)
        qb[gi] = _interleave(q1, q3)
        sb[gi] = _interleave(s1.repeat(128, 0), s3.repeat(128, 0))[::128]
        w1s.append((q1, s1))
        w3s.append((q3, s3))
    args = (torch.from_numpy(qa).to(dev()), torch.from_numpy(sa).to(dev()), torch.from_numpy(go).to(dev()),
            M, torch.from_numpy(qb).to(dev()), torch.from_numpy(sb).to(dev()))
    rows_d = rows.to(dev())
    h = moe.grouped_gemm_fp8_blockscaled(*args, epi=moe.MOE_EPI_SWIGLU_F32, a_row_index=rows_d)
    hq, hs = moe.grouped_gemm_fp8_blockscaled(*args, epi=moe.MOE_EPI_SWIGLU_QUANT, a_row_index=rows_d)
    hq2, hs2 = moe.fp8_quant_1x128(h)
    torch.cuda.synchronize()
    # fused == unfused, bit for bit
    np.testing.assert_array_equal(np_(hq), np_(hq2))
    np.testing.assert_array_equal(np_(hs).view(np.uint32), np_(hs2).view(np.uint32))
    # h vs the oracle
    rows_np = rows.numpy()
    h_ref = np.zeros((M, I))
    for gi in range(G):
        r0, r1 = go[gi], go[gi + 1]
        if r1 == r0:
            continue
        zg = oracle.gemm_blockscaled(qa, sa, *w1s[gi], a_rows=rows_np[r0:r1])
        zu = oracle.gemm_blockscaled(qa, sa, *w3s[gi], a_rows=rows_np[r0:r1])
        h_ref[r0:r1] = oracle.swiglu(zg, zu)
    err = rowinf_rel(np_(h), h_ref)
    say(f"  h per-row rel err {err:.3e}")
    assert err <= TOL
    # codes vs the oracle's quantiser on its own h
    hq_ref, hs_ref = oracle.quant_1x128(h_ref.astype(np.float32))
    flips = check_codes_close(np_(hq), np_(hs), hq_ref, hs_ref, h_ref, np_(h))
    say(f"  h-code midpoint flips: {flips} of {hq_ref.size}")
    # the quantising epilogue that also keeps z: the same h codes bit for bit,
    # and z (gate and up columns interleaved as B's rows) against the oracle
    hq3, hs3, z = moe.grouped_gemm_fp8_blockscaled(*args, epi=moe.MOE_EPI_SWIGLU_QUANT_Z, a_row_index=rows_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_(hq3), np_(hq))
    np.testing.assert_array_equal(np_(hs3).view(np.uint32), np_(hs).view(np.uint32))
    z_ref = np.zeros((M, 2 * I))
    for gi in range(G):
        r0, r1 = go[gi], go[gi + 1]
        if r1 > r0:
            z_ref[r0:r1] = oracle.gemm_blockscaled(qa, sa, qb[gi], sb[gi], a_rows=rows_np[r0:r1])
    err = rowinf_rel(np_(z), z_ref)
    say(f"  z per-row rel err {err:.3e}")
    assert err <= TOL


def check_codes_close(q, s, q_ref, s_ref, x_ref, x_gpu):
    """E4M3 codes of an FP32 GPU result checked against the oracle's exact
    result x_ref.  The scales (amax/448 of each 1x128 tile) agree within the
    output tolerance, and every dequantised GPU value lies within half an E4M3
    step (at its code) of the GPU's own value plus the GPU-vs-oracle
    difference of that value: a code can only differ from the oracle's where
    the two (both within tolerance) values round differently.  The quantiser
    scales in FP32 (the value times the rounded 448/amax, dequantised by the
    rounded amax/448): three roundings of at most 2^-24 each, so the bound
    also holds 2^-22 |x|.  A wrong scale or a wrong code fails.  Returns how
    many codes differ from the oracle's."""
    s64, sr64 = s.astype(np.float64), s_ref.astype(np.float64)
    assert np.all(np.abs(s64 / sr64 - 1) <= TOL)
    table = oracle.e4m3_table()
    vals = np.unique(table[np.isfinite(table)])
    gaps = np.diff(vals)
    half = np.zeros(256)
    for c in range(256):
        if np.isfinite(table[c]):
            i = np.searchsorted(vals, table[c])
            lo = gaps[i - 1] if i > 0 else gaps[0]
            hi = gaps[i] if i < gaps.size else gaps[-1]
            half[c] = max(lo, hi) / 2
    sc = np.repeat(s64, 128, axis=1)
    deq = table[q] * sc
    xg = np.asarray(x_gpu, np.float64)
    xr = np.asarray(x_ref, np.float64)
    bound = half[q] * sc * (1 + 1e-6) + np.abs(xg - xr) * (1 + 1e-6) + 1e-7 * sc + 2.0 ** -22 * np.abs(xr)
    bad = np.abs(deq - xr) > bound
    assert not bad.any(), f"{int(bad.sum())} E4M3 codes further from the exact value than allowed"
    return int((table[q] != table[q_ref]).sum())


@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (32, 64, 1024), (64, 48, 4096)])
def test_mfma_accumulation_probe(M, N, K):
    """The accumulation probe (unit scales).  Integer operands: the promoted
    path (one MFMA per slice, FP32 adds) is exact; with a single slice the
    chained and promoted paths are the same computation, bit for bit.  Random
    E4M3 operands: the promoted path within the FP tolerance of the FP64 sum;
    the chained path's error is what the probe measures, so it is only
    reported (and bounded loosely, which still catches a wrong layout)."""
    say(f"accumulation probe M={M} N={N} K={K}")
    va, vb, qa, qb = _int_operands(M, N, K, 1, seed=K + M)
    a, b = torch.from_numpy(qa).to(dev()), torch.from_numpy(qb[0]).to(dev())
    pro = moe.moe_fp8_mfma_accumulation_probe(a, b, chained=False)
    cha = moe.moe_fp8_mfma_accumulation_probe(a, b, chained=True)
    torch.cuda.synchronize()
    ref = va.astype(np.int64) @ vb[0].astype(np.int64).T
    np.testing.assert_array_equal(np_(pro), ref.astype(np.float32))
    if K == 128:
        np.testing.assert_array_equal(np_(cha), np_(pro))
    rng = np.random.default_rng(K)
    qa2 = oracle.e4m3_encode_array(rng.standard_normal((M, K)).astype(np.float32) * 16)
    qb2 = oracle.e4m3_encode_array(rng.standard_normal((N, K)).astype(np.float32) * 16)
    tab = oracle.e4m3_table()
    exact = tab[qa2] @ tab[qb2].T
    a, b = torch.from_numpy(qa2).to(dev()), torch.from_numpy(qb2).to(dev())
    pro = moe.moe_fp8_mfma_accumulation_probe(a, b, chained=False)
    cha = moe.moe_fp8_mfma_accumulation_probe(a, b, chained=True)
    torch.cuda.synchronize()
    errp, errc = rowinf_rel(np_(pro), exact), rowinf_rel(np_(cha), exact)
    say(f"  per-row rel err: promoted {errp:.3e}, chained {errc:.3e}")
    assert errp <= TOL
    assert errc <= 0.1


@pytest.mark.parametrize("K", [4096, 16384])
def test_dense_full_size_sampled(K):
    """The dense block-scaled GEMM workload at full size (M = 8192, N = 7168;
    A and B ~ N(0,1) with 0.1% outliers x100), in the launch configuration the
    benchmark times (one group, FP32 store).  Sampled A rows: their 1x128
    codes and scales and every 128x128 code and scale of B bit-exact against
    the oracle's quantisers, then those rows of C (all 7168 columns) within
    the per-row bound of the oracle's FP64 product of the same operands."""
    import workloads
    M, N = workloads.DENSE["M"], workloads.DENSE["N"]
    say(f"dense full size M={M} N={N} K={K}")
    a, b = workloads.dense_operands(M, N, K, device=dev())
    aq, as_ = moe.fp8_quant_1x128(a)
    bq, bs = moe.fp8_quant_128x128(b)
    go = torch.tensor([0, M], dtype=torch.int32, device=dev())
    ws = torch.empty(moe.moe_gemm_workspace_bytes(1, M, N, K), dtype=torch.uint8, device=dev())
    out = moe.grouped_gemm_fp8_blockscaled(aq, as_, go, M, bq.view(1, N, K), bs.view(1, N // 128, K // 128),
                                           ws=ws)
    torch.cuda.synchronize()
    rows = sorted({0, M - 1} | set(np.random.default_rng(K).integers(0, M, 6).tolist()))
    a_rows = np_(a[rows])
    qa_ref, sa_ref = oracle.quant_1x128(a_rows)
    np.testing.assert_array_equal(np_(aq[rows]), qa_ref)
    np.testing.assert_array_equal(np_(as_[rows]).view(np.uint32), sa_ref.view(np.uint32))
    qb_ref, sb_ref = oracle.quant_128x128(np_(b))
    np.testing.assert_array_equal(np_(bq), qb_ref)
    np.testing.assert_array_equal(np_(bs).view(np.uint32), sb_ref.view(np.uint32))
    ref = oracle.gemm_blockscaled(qa_ref, sa_ref, qb_ref, sb_ref)
    err = rowinf_rel(np_(out[rows]), ref)
    say(f"  per-row rel err {err:.3e} over {len(rows)} rows")
    assert err <= TOL


# ------------------------------------------------------------------ persistent multi-tile path
def _pow2_operands(sizes, N, K, seed):
    """Integer E4M3 codes (|v| <= 8) with power-of-two scales: 1x128 A scales
    per row and slice and 128x128 B scales per group, block and slice.  Every
    per-slice product is an exact integer of magnitude at most 2^13.  With the
    scales in 2^-2 .. 2^2 when K <= 512 (at most 4 slices: partial sums below
    4 * 2^17 = 2^19) and in 2^-2 .. 2^0 otherwise (at most 128 slices: below
    128 * 2^13 = 2^20), every scaled partial sum is a multiple of 2^-4 below
    2^20, which FP32 holds exactly: the result must equal the oracle's FP64
    value bit for bit, and a wrong, stale or misplaced scale changes it."""
    assert K // 128 <= 128
    e_hi = 3 if K <= 512 else 1
    rng = np.random.default_rng(seed)
    G = len(sizes)
    M = int(np.sum(sizes))
    codes = oracle.e4m3_encode_array(np.arange(-8, 9, dtype=np.float32))   # codes of -8..8
    qa = codes[rng.integers(0, 17, (M, K))]
    qb = np.empty((G, N, K), np.uint8)
    for gi in range(G):                 # group by group: no G x N x K index array
        qb[gi] = codes[rng.integers(0, 17, (N, K))]
    sa = np.ldexp(1.0, rng.integers(-2, e_hi, (M, K // 128))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-2, e_hi, (G, N // 128, K // 128))).astype(np.float32)
    return qa, sa, qb, sb


def _zipf_sizes(n, total, rng):
    w = 1.0 / (np.arange(1, n + 1) + 3.0) ** 1.1
    s = np.floor(w / w.sum() * total).astype(np.int64)
    s = s[rng.permutation(n)]
    s[rng.integers(0, n, 2)] = 0                    # two empty groups
    return s


@pytest.mark.parametrize("kind", ["rows128_short_k", "rows128_k10", "rows128_k16", "rows128_long_k",
                                  "rows32", "rows32_long_k"])
def test_gemm_multi_tile_exact_pow2_scales(kind):
    """The persistent schedules over many more tiles than CUs (each block runs
    several tiles, so the tile-to-tile hand-over -- the next tile's DMAs
    overlapping this tile's epilogue, the per-tile B-scale table and gathered
    rows, the tile sequence of each XCD -- is exercised everywhere), with a
    gather and ragged, Zipf-sized groups, compared element by element with the
    oracle.  rows128_short_k: 26 groups, ~40k rows, 128-row tiles of 5 K
    slices (the kernel whose DMA ring runs on across tiles; its FP32 tiles
    carry part of their output into the next tile, and a 5-slice tile stores
    the pieces it had no phase for at its end); rows128_k10 and rows128_k16:
    the same with 10 and 16 slices (every carried piece stored in a phase of
    the next tile, then phases with nothing to carry; 16 is the expert
    down-projection's K = 2048); rows128_long_k: 18 K slices (the kernel that
    restarts its pipeline per tile); rows32: 1500 groups of 0..60 rows
    (32-row tiles of 3 slices); rows32_long_k: the same groups with 8 slices,
    through the SwiGLU epilogues too."""
    rows32 = kind.startswith("rows32")
    rng = np.random.default_rng(8 if rows32 else 7)
    N = 512
    K = {"rows128_short_k": 640, "rows128_k10": 1280, "rows128_k16": 2048, "rows128_long_k": 2304,
         "rows32": 384, "rows32_long_k": 1024}[kind]
    if not rows32:
        sizes = _zipf_sizes(26, 40_000, rng)
    else:
        sizes = rng.integers(0, 61, 1500)
    G = len(sizes)
    go = _groups(sizes)
    M = int(go[-1])
    bm = 32 if M <= 64 * G else 128
    n_tiles = int(np.sum((sizes + bm - 1) // bm)) * (N // 256)
    say(f"gemm multi-tile {kind}: G={G} M={M} N={N} K={K}, {bm}-row tiles, {n_tiles} tiles")
    assert (bm == 128) == (not rows32) and n_tiles > 2 * 256
    qa, sa, qb, sb = _pow2_operands(sizes, N, K, seed=M)
    extra = 37
    rows = rng.permutation(M + extra)[:M].astype(np.int32)           # gather from a larger A
    qa_full = np.zeros((M + extra, K), np.uint8)
    sa_full = np.ones((M + extra, K // 128), np.float32)
    qa_full[rows], sa_full[rows] = qa, sa
    args = (torch.from_numpy(qa_full).to(dev()), torch.from_numpy(sa_full).to(dev()),
            torch.from_numpy(go).to(dev()), M, torch.from_numpy(qb).to(dev()), torch.from_numpy(sb).to(dev()))
    rows_d = torch.from_numpy(rows).to(dev())
    out = moe.grouped_gemm_fp8_blockscaled(*args, epi=moe.MOE_EPI_STORE_F32, a_row_index=rows_d)
    torch.cuda.synchronize()
    say("  oracle")
    ref = np.zeros((M, N))
    for gi in range(G):
        r0, r1 = go[gi], go[gi + 1]
        if r1 > r0:
            ref[r0:r1] = oracle.gemm_blockscaled(qa_full, sa_full, qb[gi], sb[gi], a_rows=rows[r0:r1])
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref), "reference not exact in FP32"
    got = np_(out)
    bad = got != ref.astype(np.float32)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} elements differ; first at {np.argwhere(bad)[0]}"
    if kind == "rows32":
        return
    # the SwiGLU epilogue that keeps z: z exact, the fused h codes equal
    # SwiGLU_F32 followed by the quantiser, h within the bound of the oracle's
    # FP64 SwiGLU of the exact z, its codes per the midpoint rule
    say("  SwiGLU epilogues")
    hq, hs, z = moe.grouped_gemm_fp8_blockscaled(*args, epi=moe.MOE_EPI_SWIGLU_QUANT_Z, a_row_index=rows_d)
    h = moe.grouped_gemm_fp8_blockscaled(*args, epi=moe.MOE_EPI_SWIGLU_F32, a_row_index=rows_d)
    hq2, hs2 = moe.fp8_quant_1x128(h)
    torch.cuda.synchronize()
    zg = np_(z)
    bad = zg != ref.astype(np.float32)
    assert not bad.any(), f"z: {int(bad.sum())} elements differ; first at {np.argwhere(bad)[0]}"
    np.testing.assert_array_equal(np_(hq), np_(hq2))
    np.testing.assert_array_equal(np_(hs).view(np.uint32), np_(hs2).view(np.uint32))
    gate_cols = np.concatenate([np.arange(256 * j, 256 * j + 128) for j in range(N // 256)])
    h_ref = oracle.swiglu(ref[:, gate_cols], ref[:, gate_cols + 128])
    assert rowinf_rel(np_(h), h_ref) <= TOL
    hq_ref, hs_ref = oracle.quant_1x128(h_ref.astype(np.float32))
    flips = check_codes_close(np_(hq), np_(hs), hq_ref, hs_ref, h_ref, np_(h))
    say(f"  h-code midpoint flips: {flips} of {hq_ref.size}")


# ------------------------------------------------------------------ the E4M3 encoder, exhaustively
_E4M3_P = 0x43E00001          # the non-negative binary32 patterns +0.0 .. 448.0
_E4M3_NAN = (1 << 23) - 1     # NaN payloads of one sign


def _binary32_patterns(lo, hi):
    """Positions [lo, hi) of the enumeration: +0 .. 448, then -0 .. -448, then
    the positive NaNs, then the negative NaNs (uint32 bit patterns)."""
    p = np.arange(lo, hi, dtype=np.int64)
    out = np.empty(p.size, np.int64)
    P, NN = _E4M3_P, _E4M3_NAN
    m = p < P
    out[m] = p[m]
    m = (p >= P) & (p < 2 * P)
    out[m] = (p[m] - P) | 0x80000000
    m = (p >= 2 * P) & (p < 2 * P + NN)
    out[m] = 0x7F800001 + (p[m] - 2 * P)
    m = p >= 2 * P + NN
    out[m] = 0xFF800001 + (p[m] - 2 * P - NN)
    return out.astype(np.uint32)


def test_quant_1x128_every_encoder_input():
    """The quantiser's E4M3 step (gfx950's conversion instruction with the
    library's clamp and NaN-sign handling) against the oracle's encoder on
    every input the quantiser can give it.  Each 1x128 tile holds 448 and 127
    test values, so amax = 448, inv = 1, scale = 1 and each code is the
    encoding of the value itself: every binary32 pattern with |x| <= 448
    (both zeros, the subnormals, every midpoint) and every NaN of either sign,
    about 2.29e9 values in chunks.  Above 448 the encoder only ever sees a
    tile maximum times its rounded inverse, which can round to 448.00003:
    tiles with such maxima check the clamp."""
    total = 2 * _E4M3_P + 2 * _E4M3_NAN
    per_chunk = 127 * (1 << 21)
    checked = 0
    for c0 in range(0, total, per_chunk):
        c1 = min(total, c0 + per_chunk)
        n = c1 - c0
        say(f"E4M3 encoder inputs {c0}..{c1} of {total}")
        vals = _binary32_patterns(c0, c1).view(np.float32)
        tiles = (n + 126) // 127
        body = np.zeros(tiles * 127, np.float32)
        body[:n] = vals
        x = np.empty((tiles, 128), np.float32)
        x[:, 0] = 448.0
        x[:, 1:] = body.reshape(tiles, 127)
        del body
        q, sc = moe.fp8_quant_1x128(torch.from_numpy(x).to(dev()))
        torch.cuda.synchronize()
        assert np.all(np_(sc).view(np.uint32) == np.float32(1.0).view(np.uint32))
        qh = np_(q)
        del q, sc
        assert np.all(qh[:, 0] == 0x7E)
        got = qh[:, 1:].reshape(-1)[:n]
        ref = oracle.e4m3_encode_array(vals)
        bad = got != ref
        if bad.any():
            i = int(np.argmax(bad))
            raise AssertionError(f"{int(bad.sum())} codes differ; first input bits 0x{vals.view(np.uint32)[i]:08x}: "
                                 f"GPU 0x{got[i]:02x}, oracle 0x{ref[i]:02x}")
        checked += n
    assert checked == total
    # the clamp: maxima a with fl32(a * fl32(448 / a)) = 448.00003, in tiles
    # of +-a and values below a, against the oracle's quantiser
    a = (np.float32(1.0) + np.arange(200_000, dtype=np.float32) * np.float32(1e-5)).astype(np.float32)
    a = np.unique(a)
    a = a[(a * (np.float32(448.0) / a).astype(np.float32)).astype(np.float32) > np.float32(448.0)][:4096]
    rng = np.random.default_rng(3)
    x = (rng.uniform(-1, 1, (a.size, 128)).astype(np.float32) * a[:, None]).astype(np.float32)
    x[:, 0], x[:, 1] = a, -a
    say(f"E4M3 clamp tiles: {a.size}")
    q, sc = moe.fp8_quant_1x128(torch.from_numpy(x).to(dev()))
    torch.cuda.synchronize()
    q_ref, sc_ref = oracle.quant_1x128(x)
    np.testing.assert_array_equal(np_(sc).view(np.uint32), sc_ref.view(np.uint32))
    np.testing.assert_array_equal(np_(q), q_ref)
    assert np.all(q_ref[:, 0] == 0x7E) and np.all(q_ref[:, 1] == 0xFE)
