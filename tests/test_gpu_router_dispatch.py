"""GPU parity: router (affinity, biased top-K, gates), dispatch, permute,
bias update against the CPU oracle.  All of these are bit-exact: the router's
scores follow the same binary32 FMA chain and sigmoid on both sides, and the
dispatch is integer work."""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_top_routing_02_amd as moe
import workloads
from helpers import TOL, dev, np_, rowinf_rel, say, u16

pytestmark = pytest.mark.gpu


def _inputs(T, d, E, seed, std_e=None, ties=False):
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(T, d, generator=g).to(torch.bfloat16)
    e = (torch.randn(E, d, generator=g) * (std_e if std_e else d ** -0.5)).to(torch.bfloat16)
    if ties and E >= 4:
        e[3] = e[1]            # identical centroids -> identical scores -> index tie-break
    b = (torch.rand(E, generator=g) - 0.5) * 0.1
    if ties and E >= 4:
        b[3] = b[1]
    return u, e, b


ROUTER_CASES = [
    # (T, d, E, K)
    (128, 512, 16, 4),        # tiny workload shape
    (37, 256, 16, 4),         # ragged T
    (300, 1024, 256, 8),      # full expert count, ragged T
    (1000, 384, 40, 6),       # E not a multiple of 64
    (1, 128, 8, 8),           # one token, K = E
    (4096, 512, 256, 8),      # the matrix-core chains (T >= 4096), fewest tokens
    (16384, 256, 256, 8),     # the matrix-core chains, many blocks
    (8200, 128, 256, 8),      # the matrix-core chains with a ragged last token block
    (4100, 256, 200, 6),      # the matrix-core chains, E not a multiple of the 128-expert block
    (256, 7168, 256, 8),      # decode: blocks of 4 tokens x 64 experts, one logit per lane
    (50, 256, 200, 6),        # decode layout with idle lanes (E not a multiple of 64, T of 4)
    (3, 16512, 72, 4),        # decode layout, long rows, one token block
]


@pytest.mark.parametrize("T,d,E,K", ROUTER_CASES)
def test_router_bit_exact(T, d, E, K):
    say(f"router T={T} d={d} E={E} K={K}")
    u, e, b = _inputs(T, d, E, seed=T * 7 + E, ties=True)
    idx, gate, s = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), K)
    torch.cuda.synchronize()
    s_ref = oracle.router_scores(u16(u), u16(e))
    np.testing.assert_array_equal(np_(s).view(np.uint32), s_ref.view(np.uint32))
    idx_ref, gate_ref = oracle.topk_from_scores(s_ref, b.numpy(), K)
    np.testing.assert_array_equal(np_(idx), idx_ref)
    np.testing.assert_array_equal(np_(gate).view(np.uint32), gate_ref.view(np.uint32))


def test_router_mfma_certificate_fallback():
    """The matrix-core router reproduces the FMA chain only while every product
    and partial sum stays in FP32's normal range, which each block certifies
    from its inputs' exponents; a block outside recomputes on the VALU.  Single
    planted values push blocks outside: a 2^-100 token element (a product's
    last bit below 2^-126), a 2^126 token element (the overflow bound) and a
    2^-110 centroid element (every block of that expert block).  Scores,
    indices and gates must still equal the oracle bit for bit everywhere."""
    T, d, E, K = 4096, 256, 256, 8
    u, e, b = _inputs(T, d, E, seed=99)
    u[5, 17] = 2.0 ** -100
    u[130, 40] = 2.0 ** 126
    e[200, 3] = 2.0 ** -110
    say("router certificate fallback")
    idx, gate, s = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), K)
    torch.cuda.synchronize()
    s_ref = oracle.router_scores(u16(u), u16(e))
    np.testing.assert_array_equal(np_(s).view(np.uint32), s_ref.view(np.uint32))
    idx_ref, gate_ref = oracle.topk_from_scores(s_ref, b.numpy(), K)
    np.testing.assert_array_equal(np_(idx), idx_ref)
    np.testing.assert_array_equal(np_(gate).view(np.uint32), gate_ref.view(np.uint32))


GROUPED_CASES = [
    # (T, d, E, K, n_groups, topk_groups)
    (300, 512, 256, 8, 8, 4),      # the pages' shape: 8 groups of 32, at most 4 per token
    (1000, 256, 64, 6, 8, 3),      # groups of 8
    (37, 128, 16, 4, 4, 2),        # ragged T, groups of 4, with score ties
    (256, 7168, 256, 8, 8, 4),     # decode-layout scores
    (8200, 128, 256, 8, 64, 2),    # 64 groups of 4: K equals the kept experts
    (50, 256, 200, 6, 8, 3),       # groups of 25 straddle the lanes' expert slots
    (64, 128, 96, 5, 1, 1),        # one group: plain top-K
]


@pytest.mark.parametrize("T,d,E,K,ng,m", GROUPED_CASES)
def test_router_grouped_bit_exact(T, d, E, K, ng, m):
    say(f"grouped router T={T} d={d} E={E} K={K} groups={ng} keep={m}")
    u, e, b = _inputs(T, d, E, seed=T * 11 + E + ng, ties=True)
    idx, gate, s = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), K, n_groups=ng,
                                       topk_groups=m)
    torch.cuda.synchronize()
    s_ref = oracle.router_scores(u16(u), u16(e))
    np.testing.assert_array_equal(np_(s).view(np.uint32), s_ref.view(np.uint32))
    idx_ref, gate_ref = oracle.topk_grouped_from_scores(s_ref, b.numpy(), K, ng, m)
    np.testing.assert_array_equal(np_(idx), idx_ref)
    np.testing.assert_array_equal(np_(gate).view(np.uint32), gate_ref.view(np.uint32))
    assert max(len(set(r.tolist())) for r in np_(idx) // (E // ng)) <= m


def test_router_tiny_workload_and_determinism():
    sh = workloads.SHAPES["tiny"]
    u, e, b = workloads.activations(sh), workloads.centroids(sh), workloads.bias(sh)
    say("router tiny workload x2")
    r1 = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), sh.K)
    r2 = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), sh.K)
    torch.cuda.synchronize()
    idx_ref, gate_ref, s_ref = oracle.router_topk(u16(u), u16(e), b.numpy(), sh.K)
    for r in (r1, r2):
        np.testing.assert_array_equal(np_(r[0]), idx_ref)
        np.testing.assert_array_equal(np_(r[1]).view(np.uint32), gate_ref.view(np.uint32))


def test_router_rdc_workload_slice():
    """The router+dispatch+combine workload's shapes (d=7168, 256 experts,
    top-8) on its first 512 tokens (the oracle's cost is per token)."""
    sh = workloads.SHAPES["rdc"]
    u = workloads.activations(sh)[:512].contiguous()
    e, b = workloads.centroids(sh), workloads.bias(sh)
    say("router rdc slice 512 tokens")
    idx, gate, s = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), sh.K)
    torch.cuda.synchronize()
    idx_ref, gate_ref, s_ref = oracle.router_topk(u16(u), u16(e), b.numpy(), sh.K)
    np.testing.assert_array_equal(np_(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(np_(idx), idx_ref)
    np.testing.assert_array_equal(np_(gate).view(np.uint32), gate_ref.view(np.uint32))


def _rand_idx(T, E, K, seed, skew=False):
    rng = np.random.default_rng(seed)
    p = None
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


# T <= 1024 runs the one-block kernel, larger T the three-launch path
DISPATCH_CASES = [(1, 4, 2), (63, 16, 4), (64, 16, 4), (65, 16, 4), (1000, 256, 8), (4097, 256, 8),
                  (300, 8, 8), (2000, 200, 16), (1024, 256, 16), (1025, 256, 8)]


@pytest.mark.parametrize("T,E,K", DISPATCH_CASES)
@pytest.mark.parametrize("shared", [True, False])
def test_dispatch_bit_exact(T, E, K, shared):
    say(f"dispatch T={T} E={E} K={K} shared={shared}")
    idx = _rand_idx(T, E, K, seed=T + E, skew=(T % 2 == 0))
    count, go, row_token, slot_row = moe.moe_dispatch(torch.from_numpy(idx).to(dev()), E, shared)
    torch.cuda.synchronize()
    c_ref, go_ref, rt_ref, sr_ref = oracle.dispatch(idx, E, shared)
    np.testing.assert_array_equal(np_(count), c_ref)
    np.testing.assert_array_equal(np_(go), go_ref)
    np.testing.assert_array_equal(np_(row_token), rt_ref)
    np.testing.assert_array_equal(np_(slot_row), sr_ref)


def test_dispatch_all_tokens_one_expert():
    """Degenerate routing: every token picks the same K experts."""
    T, E, K = 777, 64, 4
    idx = np.tile(np.array([5, 0, 63, 7], np.int32), (T, 1))
    say("dispatch degenerate")
    count, go, row_token, slot_row = moe.moe_dispatch(torch.from_numpy(idx).to(dev()), E, True)
    torch.cuda.synchronize()
    c_ref, go_ref, rt_ref, sr_ref = oracle.dispatch(idx, E, True)
    np.testing.assert_array_equal(np_(count), c_ref)
    np.testing.assert_array_equal(np_(row_token), rt_ref)
    np.testing.assert_array_equal(np_(slot_row), sr_ref)


@pytest.mark.parametrize("T,E,K,shared", [(3000, 256, 8, True), (777, 40, 6, False), (64, 16, 16, True)])
def test_dispatch_status_word(T, E, K, shared):
    """The debug status word: 0 on every dispatch result, and each broken
    invariant (planted by editing the arrays with torch, never by a kernel)
    raises its own bit; out-of-range slots and tokens are reported, not
    followed."""
    say(f"dispatch status word T={T} E={E} K={K} shared={shared}")
    bits = moe.MOE_CHECK_BITS
    rng = np.random.default_rng(T + E)
    idx = torch.from_numpy(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)).to(dev())
    count, go, row_token, slot_row = moe.moe_dispatch(idx, E, shared)

    def word(c=count, g=go, rt=row_token, sr=slot_row, full=True):
        st = moe.moe_dispatch_check(c, g, T, K, *((idx, rt, sr) if full else (None, None, None)))
        torch.cuda.synchronize()
        return int(np_(st)[0]) & 0xFFFFFFFF

    assert word() == 0 and word(full=False) == 0
    c = count.clone(); c[3] += 1
    assert word(c=c) == bits["count_sum"] | bits["count_ne_offsets"]
    c = count.clone(); c[0] = -c[0] - 1
    assert word(c=c) & bits["negative_count"]
    g = go.clone(); g[1], g[2] = go[2].item() + 1, go[1].item()
    w = word(g=g, full=False)
    assert w & bits["offsets_not_monotone"] and w & bits["count_ne_offsets"]
    g = go.clone(); g[0] = 1
    assert word(g=g, full=False) & bits["first_offset"]
    g = go.clone(); g[E] += 1
    assert word(g=g, full=False) & bits["routed_total"]
    sr = slot_row.clone(); sr[5, 0] = -7
    assert word(sr=sr) == bits["slot_row"]
    sr = slot_row.clone(); sr[T - 1, K - 1] = T * (K + 1) + 1000        # past every row
    assert word(sr=sr) == bits["slot_row"]
    sr = slot_row.clone(); sr[2, 0], sr[2, 1] = slot_row[2, 1].item(), slot_row[2, 0].item()
    assert word(sr=sr) == bits["slot_row"]
    if shared:
        rt = row_token.clone(); rt[T * K + 2] = 0
        assert word(rt=rt) == bits["shared_rows"]
        g = go.clone(); g[E + 1] -= 1
        assert word(g=g, full=False) & bits["shared_group"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute_rows_and_unpermute(dtype):
    T, E, K, d = 333, 32, 4, 384
    idx = _rand_idx(T, E, K, seed=5)
    x = torch.randn(T, d).to(dtype)
    say(f"permute {dtype}")
    count, go, row_token, slot_row = moe.moe_dispatch(torch.from_numpy(idx).to(dev()), E, False)
    xp = moe.moe_permute_rows(x.to(dev()), row_token)
    torch.cuda.synchronize()
    _, _, rt_ref, sr_ref = oracle.dispatch(idx, E, False)
    np.testing.assert_array_equal(np_(xp.view(torch.int16) if dtype == torch.bfloat16 else xp),
                                  np_(x.view(torch.int16) if dtype == torch.bfloat16 else x)[rt_ref])
    back = xp[slot_row.long()]            # [T, K, d]: every slot returns the token's own row
    for k in range(K):
        assert torch.equal(back[:, k].cpu(), x)


def test_bias_update_bit_exact():
    E, T, K = 256, 8192, 8
    rng = np.random.default_rng(9)
    count = rng.multinomial(T * K, np.ones(E) / E).astype(np.int32)
    count[:4] = T * K // E          # exactly at the mean
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    say("bias update")
    bd = torch.from_numpy(b).to(dev())
    moe.moe_bias_update(bd, torch.from_numpy(count).to(dev()), T * K, 1e-3)
    torch.cuda.synchronize()
    ref = oracle.bias_update(b, count, T * K, 1e-3)
    np.testing.assert_array_equal(np_(bd).view(np.uint32), ref.view(np.uint32))
    np.testing.assert_array_equal(np_(bd)[:4], b[:4])


@pytest.mark.parametrize("T,d,E,K", [(300, 512, 16, 4), (1000, 7168, 256, 8)])
def test_combine_identity_experts_bf16(T, d, E, K):
    """The router-dispatch-combine path with identity experts: Y is the
    permuted bf16 input, no shared term; h' against the oracle's FP64 combine
    (per-row relative error <= 2e-3), and the conservation h' ~ 2u (sum g = 1)."""
    u, e, b = _inputs(T, d, E, seed=T + d)
    say(f"combine identity experts T={T} d={d} E={E} K={K}")
    idx, gate, _ = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), K)
    count, go, row_token, slot_row = moe.moe_dispatch(idx, E, False)
    xp = moe.moe_permute_rows(u.to(dev()), row_token)
    out = moe.moe_combine(u.to(dev()), xp, gate, slot_row, shared_row0=-1)
    torch.cuda.synchronize()
    y = (u16(xp).astype(np.uint32) << 16).view(np.float32)
    ref = oracle.combine(u16(u), y, -1, np_(gate), np_(slot_row))
    err = rowinf_rel(np_(out), ref)
    say(f"  per-row rel err {err:.3e}")
    assert err <= TOL
    uf = (u16(u).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert rowinf_rel(np_(out), 2 * uf) <= 1e-5


@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_permute_combine_past_grid_rows(ydt):
    """More token rows than the 65,535 grid rows of the permute and combine
    launches (the rows wrap round the grid), with a row that does not fill
    the last column block (d = 136: 17 words of bf16, 34 of FP32).  Permute is
    bit-exact; combine (with a shared row block) within the FP tolerance."""
    T, K, d, E = 70003, 2, 136, 8
    rng = np.random.default_rng(21)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    g = torch.Generator().manual_seed(22)
    u = torch.randn(T, d, generator=g).to(torch.bfloat16)
    say(f"permute + combine past the grid rows, Y {ydt}")
    count, go, row_token, slot_row = moe.moe_dispatch(torch.from_numpy(idx).to(dev()), E, True)
    xp = moe.moe_permute_rows(u.to(dev()), row_token)                     # R = T*K + T rows
    torch.cuda.synchronize()
    _, _, rt_ref, _ = oracle.dispatch(idx, E, True)
    np.testing.assert_array_equal(u16(xp), u16(u)[rt_ref])
    y = xp.to(ydt)
    gate = torch.rand(T, K, generator=g).to(dev())
    out = moe.moe_combine(u.to(dev()), y, gate, slot_row, shared_row0=T * K)
    torch.cuda.synchronize()
    yf = np_(y.float()).astype(np.float64)
    ref = oracle.combine(u16(u), yf, T * K, np_(gate), np_(slot_row))
    err = rowinf_rel(np_(out), ref)
    say(f"  per-row rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("T,E,K,L", [(8192, 256, 8, 4096), (300, 64, 6, 300), (257, 16, 4, 1), (1040, 200, 8, 80)])
def test_seq_balance_loss(T, E, K, L):
    """The sequence-wise balance loss on the router's own scores and choices
    against the oracle's FP64 value (relative 1e-5: FP32 sums over a sequence)."""
    d = 256
    u, e, b = _inputs(T, d, E, seed=T + E + L)
    say(f"balance loss T={T} E={E} K={K} seq_len={L}")
    idx, gate, s = moe.moe_router_topk(u.to(dev()), e.to(dev()), b.to(dev()), K)
    loss = moe.moe_seq_balance_loss(s, idx, L, 1e-4)
    torch.cuda.synchronize()
    ref = oracle.seq_balance_loss(np_(s), np_(idx), L, 1e-4)
    np.testing.assert_allclose(np_(loss), ref, rtol=1e-5)
    # deterministic: a second call gives the same bits
    again = moe.moe_seq_balance_loss(s, idx, L, 1e-4)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int32), loss.view(torch.int32))
