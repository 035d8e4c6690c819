"""Pins for the oracle's router (affinity, biased top-K, gates), dispatch and
bias update.

What pins them (none of it re-runs the oracle's own formula):
  * exact special cases: small-integer bf16 inputs make every logit an exact
    integer in any summation order, so the score must be sigmoid_spec of the
    integer numpy dot product;
  * brute force over all K-subsets (tiny E) and numpy's lexsort;
  * the page facts: exactly K distinct experts, gates sum to 1 over the chosen
    ones, the bias changes the choice but never the gate values
    ("DeepSeek-V3 Technical Report" notes, bias and MoE-routing paragraphs;
    nlp-lineage summary, "The notation");
  * numpy bincount / cumsum / stable argsort for the dispatch;
  * the sign table of the bias update.
"""
import itertools

import numpy as np
import pytest


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Exact float32 -> bf16 bits (inputs here are chosen bf16-representable)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


def _rand_bf16(rng, shape, std=1.0):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: still a valid bf16 sample


def test_router_scores_exact_integer_case(oracle_mod):
    rng = np.random.default_rng(10)
    T, d, E = 9, 256, 12
    u = rng.integers(-3, 4, (T, d)).astype(np.float32)
    e = rng.integers(-2, 3, (E, d)).astype(np.float32) / 64.0
    s = oracle_mod.router_scores(_bf16_bits(u), _bf16_bits(e))
    logits = (u.astype(np.int64) @ (e * 64).astype(np.int64).T).astype(np.float64) / 64.0
    expect = oracle_mod.sigmoid_spec_array(logits.astype(np.float32))
    np.testing.assert_array_equal(s, expect)
    # and within 4 ulps of the FP64 sigmoid of the exact logits
    ref = 1 / (1 + np.exp(-logits))
    assert np.max(np.abs(s - ref) / np.spacing(np.abs(ref).astype(np.float32))) <= 4


def test_router_scores_close_to_fp64(oracle_mod):
    rng = np.random.default_rng(11)
    T, d, E = 16, 512, 8
    u = _rand_bf16(rng, (T, d))
    e = _rand_bf16(rng, (E, d), d ** -0.5)
    s = oracle_mod.router_scores(u, e)
    uf = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ef = (e.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = 1 / (1 + np.exp(-(uf @ ef.T)))
    assert np.max(np.abs(s - ref)) < 1e-5


def _keys(s, b):
    return (s + b[None, :]).astype(np.float32)


def test_topk_brute_force_tiny(oracle_mod):
    """For E <= 8, the chosen set is the K-subset with the largest keys under
    the (key desc, index asc) order; slot order is that ranking."""
    rng = np.random.default_rng(12)
    for E, K in [(5, 2), (6, 3), (8, 4), (8, 8), (7, 1)]:
        T = 40
        s = rng.uniform(0, 1, (T, E)).astype(np.float32)
        s[:, 1] = s[:, 3]            # force exact ties
        b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
        b[3] = b[1]
        idx, gate = oracle_mod.topk_from_scores(s, b, K)
        key = _keys(s, b)
        for t in range(T):
            order = sorted(range(E), key=lambda i: (-float(key[t, i]), i))
            assert list(idx[t]) == order[:K]
            # brute force: best K-subset by sorted key tuples, then lowest indices
            best = max(itertools.combinations(range(E), K),
                       key=lambda c: (sorted((float(key[t, i]) for i in c), reverse=True),
                                      [-i for i in sorted(c)]))
            assert set(best) == set(idx[t])


def test_topk_lexsort_and_dominance(oracle_mod):
    rng = np.random.default_rng(13)
    T, E, K = 300, 64, 8
    s = rng.uniform(0, 1, (T, E)).astype(np.float32)
    s[:, 10:20] = s[:, 0:10]   # duplicated scores -> ties broken by index
    b = np.zeros(E, np.float32)
    idx, gate = oracle_mod.topk_from_scores(s, b, K)
    key = _keys(s, b)
    for t in range(T):
        order = np.lexsort((np.arange(E), -key[t].astype(np.float64)))
        np.testing.assert_array_equal(idx[t], order[:K])
        chosen = set(idx[t].tolist())
        kmin = min((float(key[t, i]), -i) for i in chosen)
        for j in range(E):
            if j not in chosen:
                assert (float(key[t, j]), -j) < kmin


def test_topk_exactly_k_distinct_and_gates_sum_to_one(oracle_mod):
    rng = np.random.default_rng(14)
    T, E, K = 500, 256, 8
    s = oracle_mod.sigmoid_spec_array(rng.standard_normal((T, E)).astype(np.float32))
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, gate = oracle_mod.topk_from_scores(s, b, K)
    for t in range(T):
        assert len(set(idx[t].tolist())) == K
    assert np.all((idx >= 0) & (idx < E))
    assert np.max(np.abs(gate.astype(np.float64).sum(1) - 1.0)) <= K * 2.0 ** -23
    # gates are the raw scores normalised over the chosen experts (no bias)
    raw = np.take_along_axis(s, idx, 1).astype(np.float64)
    np.testing.assert_allclose(gate, raw / raw.sum(1, keepdims=True), rtol=3e-7)


def test_bias_changes_choice_not_gates(oracle_mod):
    """Shifting the bias of the already-chosen experts up keeps the set and,
    per expert, the gate values; a large bias on an unchosen expert pulls it
    in, and its gate is its raw score over the new chosen sum."""
    rng = np.random.default_rng(15)
    T, E, K = 200, 32, 4
    s = oracle_mod.sigmoid_spec_array(rng.standard_normal((T, E)).astype(np.float32))
    b = np.zeros(E, np.float32)
    idx0, g0 = oracle_mod.topk_from_scores(s, b, K)
    # uniform shift of every bias by a power of two keeps every key order
    idx1, g1 = oracle_mod.topk_from_scores(s, b + np.float32(4.0), K)
    same_order = np.all(idx0 == idx1, axis=1)
    np.testing.assert_array_equal(g0[same_order], g1[same_order])
    for t in range(T):
        d0 = dict(zip(idx0[t].tolist(), g0[t].tolist()))
        d1 = dict(zip(idx1[t].tolist(), g1[t].tolist()))
        assert d0.keys() == d1.keys()
        for k in d0:
            assert abs(d0[k] - d1[k]) <= 2 * 2.0 ** -24
    # a huge bias forces expert 5 into every token's choice, first slot
    b2 = b.copy()
    b2[5] = 10.0
    idx2, g2 = oracle_mod.topk_from_scores(s, b2, K)
    assert np.all(idx2[:, 0] == 5)
    raw = np.take_along_axis(s, idx2, 1).astype(np.float64)
    np.testing.assert_allclose(g2, raw / raw.sum(1, keepdims=True), rtol=3e-7)


def test_topk_k_equals_e_ignores_bias_for_selection(oracle_mod):
    rng = np.random.default_rng(16)
    T, E = 50, 12
    s = rng.uniform(0, 1, (T, E)).astype(np.float32)
    for b in (np.zeros(E, np.float32), rng.uniform(-1, 1, E).astype(np.float32)):
        idx, gate = oracle_mod.topk_from_scores(s, b, E)
        assert all(sorted(r) == list(range(E)) for r in idx.tolist())


def test_topk_degenerate_all_zero_scores(oracle_mod):
    s = np.zeros((3, 6), np.float32)
    b = np.array([0, 0.1, 0, 0.2, 0, 0], np.float32)
    idx, gate = oracle_mod.topk_from_scores(s, b, 3)
    np.testing.assert_array_equal(idx[0], [3, 1, 0])
    assert np.all(gate == 0)


# ------------------------------------------------------------------ dispatch
def _random_idx(rng, T, E, K):
    return np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("shared", [True, False])
def test_dispatch_against_numpy(oracle_mod, shared):
    rng = np.random.default_rng(17)
    for T, E, K in [(1, 4, 2), (37, 16, 4), (300, 256, 8), (64, 8, 8)]:
        idx = _random_idx(rng, T, E, K)
        count, go, row_token, slot_row = oracle_mod.dispatch(idx, E, shared)
        np.testing.assert_array_equal(count, np.bincount(idx.ravel(), minlength=E))
        exp_go = np.concatenate([[0], np.cumsum(count)])
        if shared:
            exp_go = np.concatenate([exp_go, [T * K + T]])
        np.testing.assert_array_equal(go, exp_go)
        tok = np.repeat(np.arange(T), K)
        order = np.lexsort((tok, idx.ravel()))      # by expert, then token
        np.testing.assert_array_equal(row_token[:T * K], tok[order])
        if shared:
            np.testing.assert_array_equal(row_token[T * K:], np.arange(T))
        assert row_token.shape[0] == T * K + (T if shared else 0)
        # slot_row is the inverse permutation
        inv = np.empty(T * K, np.int64)
        inv[order] = np.arange(T * K)
        np.testing.assert_array_equal(slot_row.ravel(), inv)
        # conservation: every token appears K (+1 shared) times, no drop
        np.testing.assert_array_equal(np.bincount(row_token, minlength=T), np.full(T, K + (1 if shared else 0)))
        # each row lies in its expert's group
        for t in range(T):
            for k in range(K):
                r = slot_row[t, k]
                e = idx[t, k]
                assert go[e] <= r < go[e + 1] and row_token[r] == t


def test_permute_unpermute_identity(oracle_mod):
    rng = np.random.default_rng(18)
    T, E, K, d = 50, 16, 4, 8
    idx = _random_idx(rng, T, E, K)
    count, go, row_token, slot_row = oracle_mod.dispatch(idx, E, False)
    x = rng.standard_normal((T, d))
    xp = x[row_token]
    back = xp[slot_row]          # [T, K, d]
    for k in range(K):
        np.testing.assert_array_equal(back[:, k], x)


def test_dispatch_rejects_bad_index(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.dispatch(np.array([[0, 5]], np.int32), 4, True)


# ------------------------------------------------------------------ bias update
def test_bias_update_sign_table(oracle_mod):
    """Overloaded (above the batch mean) -> b - gamma, underloaded -> b + gamma,
    exactly at the mean -> unchanged; gamma = 0 leaves b unchanged."""
    E, TK = 4, 40            # mean load 10
    count = np.array([11, 9, 10, 0], np.int32)
    b = np.array([0.5, -0.25, 0.125, 0.0], np.float32)
    out = oracle_mod.bias_update(b, count, TK, 0.125)
    np.testing.assert_array_equal(out, np.array([0.375, -0.125, 0.125, 0.125], np.float32))
    np.testing.assert_array_equal(oracle_mod.bias_update(b, count, TK, 0.0), b)
    # FP32 rounding of the update
    out = oracle_mod.bias_update(np.array([0.01, 0.01, 0, 0], np.float32), count, TK, 1e-3)
    assert out[0] == np.float32(np.float32(0.01) - np.float32(1e-3))
    assert out[1] == np.float32(np.float32(0.01) + np.float32(1e-3))


def test_bias_update_feedback_balances_load(oracle_mod):
    """Repeating route -> count -> update on fixed scores drives the most
    loaded expert's load down (the page's stated purpose of the rule)."""
    rng = np.random.default_rng(19)
    T, E, K = 2000, 16, 2
    base = rng.standard_normal(E) * 0.5
    s = oracle_mod.sigmoid_spec_array((rng.standard_normal((T, E)) * 0.3 + base).astype(np.float32))
    b = np.zeros(E, np.float32)
    idx, _ = oracle_mod.topk_from_scores(s, b, K)
    c0 = np.bincount(idx.ravel(), minlength=E)
    for _ in range(200):
        idx, _ = oracle_mod.topk_from_scores(s, b, K)
        c = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
        b = oracle_mod.bias_update(b, c, T * K, 0.01)
    assert c.max() / c.mean() < 0.5 * c0.max() / c0.mean()


# ---------------------------------------------------------------- group-limited routing
# "DeepSeek-V3 Technical Report" notes, MoE-routing paragraph: each token is
# sent to at most 4 nodes.  The group rule (a group's score is its best key;
# the topk_groups best groups are kept) is this build's reading, so these pins
# fix the reading's consequences: its reductions to plain top-K, brute force
# over all group subsets, a worked example, and the "at most M groups" fact.

def test_grouped_topk_reduces_to_plain_topk(oracle_mod):
    rng = np.random.default_rng(30)
    T, E, K = 200, 64, 6
    s = rng.uniform(0, 1, (T, E)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx0, g0 = oracle_mod.topk_from_scores(s, b, K)
    for ng, m in [(1, 1), (8, 8), (64, 64), (16, 16)]:
        idx, g = oracle_mod.topk_grouped_from_scores(s, b, K, ng, m)
        np.testing.assert_array_equal(idx, idx0)
        np.testing.assert_array_equal(g.view(np.uint32), g0.view(np.uint32))


def test_grouped_topk_brute_force_over_group_subsets(oracle_mod):
    """The kept groups are the M-subset whose scores, sorted descending, are
    largest (ties to lower group indices); the experts are then the top K of
    that subset's experts (itself brute-forced over K-subsets)."""
    rng = np.random.default_rng(31)
    for E, ng, m, K in [(8, 4, 2, 3), (12, 4, 2, 4), (12, 6, 3, 2), (16, 8, 2, 4), (16, 4, 1, 4)]:
        gs = E // ng
        T = 30
        s = rng.uniform(0, 1, (T, E)).astype(np.float32)
        s[:, gs] = s[:, 0]              # equal best keys in groups 0 and 1 for some tokens
        b = np.zeros(E, np.float32)
        idx, gate = oracle_mod.topk_grouped_from_scores(s, b, K, ng, m)
        key = _keys(s, b)
        for t in range(T):
            score = [max(float(key[t, i]) for i in range(g * gs, (g + 1) * gs)) for g in range(ng)]
            kept = max(itertools.combinations(range(ng), m),
                       key=lambda c: (sorted((score[g] for g in c), reverse=True), [-g for g in sorted(c)]))
            cand = [i for g in kept for i in range(g * gs, (g + 1) * gs)]
            best = max(itertools.combinations(cand, K),
                       key=lambda c: (sorted((float(key[t, i]) for i in c), reverse=True),
                                      [-i for i in sorted(c)]))
            assert set(best) == set(idx[t].tolist())
            # slot order: key descending, index ascending
            assert list(idx[t]) == sorted(best, key=lambda i: (-float(key[t, i]), i))


def test_grouped_topk_worked_example(oracle_mod):
    """8 experts in 4 groups of 2, keep 2 groups, K = 3.  Keys by expert:
    0.9 0.1 | 0.8 0.7 | 0.85 0.2 | 0.3 0.3.  Group scores 0.9, 0.8, 0.85, 0.3:
    groups 0 and 2 are kept, so the experts are 0 (0.9), 4 (0.85), 5 (0.2),
    while plain top-3 would take 0, 4, 2."""
    s = np.array([[0.9, 0.1, 0.8, 0.7, 0.85, 0.2, 0.3, 0.3]], np.float32)
    b = np.zeros(8, np.float32)
    idx, gate = oracle_mod.topk_grouped_from_scores(s, b, 3, 4, 2)
    assert idx.tolist() == [[0, 4, 5]]
    assert oracle_mod.topk_from_scores(s, b, 3)[0].tolist() == [[0, 4, 2]]
    D = np.float32(np.float32(np.float32(0.9) + np.float32(0.85)) + np.float32(0.2))
    np.testing.assert_array_equal(gate[0], (s[0, [0, 4, 5]] / D).astype(np.float32))


def test_grouped_topk_at_most_m_groups_and_bias_invariant_gates(oracle_mod):
    rng = np.random.default_rng(32)
    T, E, K, ng, m = 400, 256, 8, 8, 4
    s = oracle_mod.sigmoid_spec_array(rng.standard_normal((T, E)).astype(np.float32))
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, gate = oracle_mod.topk_grouped_from_scores(s, b, K, ng, m)
    groups = idx // (E // ng)
    assert max(len(set(r.tolist())) for r in groups) <= m
    assert all(len(set(r.tolist())) == K for r in idx)
    assert np.max(np.abs(gate.astype(np.float64).sum(1) - 1.0)) <= K * 2.0 ** -23
    raw = np.take_along_axis(s, idx, 1).astype(np.float64)
    np.testing.assert_allclose(gate, raw / raw.sum(1, keepdims=True), rtol=3e-7)
    # raising the bias of a token's chosen experts keeps its choice and gates
    bump = np.zeros(E, np.float32)
    t0 = 0
    bump[idx[t0]] = 0.5
    idx2, gate2 = oracle_mod.topk_grouped_from_scores(s[t0:t0 + 1], b + bump, K, ng, m)
    assert set(idx2[0].tolist()) == set(idx[t0].tolist())
    np.testing.assert_array_equal(np.sort(gate2[0]), np.sort(gate[t0]))


# ---------------------------------------------------------------- sequence-wise balance loss
# The pages name the loss but give no formula; the reading (frequency times
# normalised score, per sequence) is pinned by its closed forms and invariances.

def test_seq_balance_loss_uniform_use_gives_alpha(oracle_mod):
    """Every expert chosen equally often and equal scores: f_i = 1, P_i = 1/E."""
    E, K, L = 16, 4, 32
    s = np.full((2 * L, E), 0.3, np.float32)
    idx = np.array([[(t * K + k) % E for k in range(K)] for t in range(2 * L)], np.int32)
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s, idx, L, 0.01), [0.01, 0.01], rtol=1e-14)


def test_seq_balance_loss_extreme_imbalance_gives_alpha_e_over_k(oracle_mod):
    """Every token on experts 0..K-1 with all of its score there: f_i = E/K
    and P_i = 1/K for those K experts, so the sum is E/K."""
    E, K, L = 32, 8, 50
    s = np.zeros((L, E), np.float32)
    s[:, :K] = 0.7
    idx = np.tile(np.arange(K, dtype=np.int32), (L, 1))
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s, idx, L, 1.0), [E / K], rtol=1e-14)


def test_seq_balance_loss_invariances(oracle_mod):
    """Scaling a token's scores, reordering tokens inside a sequence, or
    relabelling experts consistently leaves the loss unchanged; it is linear
    in alpha; sequences are independent."""
    rng = np.random.default_rng(40)
    E, K, L, n = 24, 3, 40, 3
    s = rng.uniform(0.01, 1, (n * L, E)).astype(np.float32)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(n * L)]).astype(np.int32)
    base = oracle_mod.seq_balance_loss(s, idx, L, 1.0)
    s2 = (s * np.float32(4.0)).astype(np.float32)          # exact power-of-two scaling
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s2, idx, L, 1.0), base, rtol=1e-13)
    perm = np.concatenate([q * L + rng.permutation(L) for q in range(n)])
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s[perm], idx[perm], L, 1.0), base, rtol=1e-13)
    relabel = rng.permutation(E)
    s3 = np.empty_like(s)
    s3[:, relabel] = s
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s3, relabel[idx].astype(np.int32), L, 1.0), base,
                               rtol=1e-13)
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s, idx, L, 0.25), base * 0.25, rtol=1e-15)
    np.testing.assert_allclose(oracle_mod.seq_balance_loss(s[L:2 * L], idx[L:2 * L], L, 1.0), base[1:2],
                               rtol=1e-15)
    # f_i <= E/K and the P_i sum to 1, so the sum is positive and at most E/K
    whole = oracle_mod.seq_balance_loss(s, idx, n * L, 1.0)[0]
    assert 0 < whole <= E / K
