"""Pins for the backward oracle (oracle/backward.py): central finite
differences of the layer's FP64 forward, written here straight from the
output equation (nlp-lineage summary, "The notation"; gates normalised over
the chosen experts, "DeepSeek-V3 Technical Report" notes), with the chosen
experts held fixed (the bias only selects them, so the selection is constant
under small changes).  The analytic gradients of L = <dh, h'> with respect to
u and the centroids e must match, as must dL/dg (the per-slot a) and the
gradient reaching each expert output."""
import numpy as np
import pytest

from oracle import backward as bw


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _setup(seed, T=4, d=6, E=5, K=2, I=3):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    e = rng.standard_normal((E, d)) * 0.5
    b = rng.uniform(-0.05, 0.05, E)
    W1 = rng.standard_normal((E + 1, I, d)) * 0.5
    W3 = rng.standard_normal((E + 1, I, d)) * 0.5
    W2 = rng.standard_normal((E + 1, d, I)) * 0.5
    s = 1.0 / (1.0 + np.exp(-(u @ e.T)))
    idx = np.argsort(-(s + b), axis=1, kind="stable")[:, :K]
    dh = rng.standard_normal((T, d))
    return u, e, W1, W3, W2, idx, dh


def _ffn(W1, W3, W2, g, x):
    return W2[g] @ (_silu(W1[g] @ x) * (W3[g] @ x))


def _loss(u, e, W1, W3, W2, idx, dh):
    """L = <dh, h'> with h'_t = u_t + FFN_shared(u_t) + sum_k g_k FFN_(i_k)(u_t)."""
    T, K = idx.shape
    E = e.shape[0]
    s = 1.0 / (1.0 + np.exp(-(u @ e.T)))
    L = 0.0
    for t in range(T):
        sc = s[t, idx[t]]
        g = sc / sc.sum()
        h = u[t] + _ffn(W1, W3, W2, E, u[t])
        for k in range(K):
            h = h + g[k] * _ffn(W1, W3, W2, idx[t, k], u[t])
        L += float(dh[t] @ h)
    return L


def _analytic(u, e, W1, W3, W2, idx, dh):
    """The oracle's backward, with rows laid out as the dispatch lays them
    (by expert, then token; the shared expert's T rows last)."""
    T, K = idx.shape
    E = e.shape[0]
    pairs = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K))
    R = T * K + T
    row_token = np.zeros(R, np.int64)
    row_group = np.zeros(R, np.int64)
    slot_row = np.zeros((T, K), np.int64)
    for r, (g, t, k) in enumerate(pairs):
        row_token[r], row_group[r], slot_row[t, k] = t, g, r
    row_token[T * K:] = np.arange(T)
    row_group[T * K:] = E
    s = 1.0 / (1.0 + np.exp(-(u @ e.T)))
    sc = s[np.arange(T)[:, None], idx]
    gate = sc / sc.sum(axis=1, keepdims=True)
    x = u[row_token]
    zg = np.einsum("rid,rd->ri", W1[row_group], x)
    zu = np.einsum("rid,rd->ri", W3[row_group], x)
    y = np.einsum("rdi,ri->rd", W2[row_group], _silu(zg) * zu)
    a, dy, dlogit = bw.gate_backward(dh, y, T * K, gate, slot_row, s, idx)
    dx = np.zeros_like(x)
    for g in range(E + 1):
        rows = np.nonzero(row_group == g)[0]
        if len(rows):
            dx[rows] = bw.expert_dgrad(dy[rows], zg[rows], zu[rows], W1[g], W3[g], W2[g])[3]
    du_r, de = bw.router_backward(u, e, idx, dlogit, E)
    du = bw.assemble_du(dh, dx, row_token) + du_r
    return dict(du=du, de=de, a=a, dy=dy, y=y, slot_row=slot_row)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_backward_matches_finite_differences(seed):
    u, e, W1, W3, W2, idx, dh = _setup(seed)
    an = _analytic(u, e, W1, W3, W2, idx, dh)
    eps = 1e-6
    du_fd = np.zeros_like(u)
    for t in range(u.shape[0]):
        for c in range(u.shape[1]):
            up, um = u.copy(), u.copy()
            up[t, c] += eps
            um[t, c] -= eps
            du_fd[t, c] = (_loss(up, e, W1, W3, W2, idx, dh) - _loss(um, e, W1, W3, W2, idx, dh)) / (2 * eps)
    de_fd = np.zeros_like(e)
    for i in range(e.shape[0]):
        for c in range(e.shape[1]):
            ep, em = e.copy(), e.copy()
            ep[i, c] += eps
            em[i, c] -= eps
            de_fd[i, c] = (_loss(u, ep, W1, W3, W2, idx, dh) - _loss(u, em, W1, W3, W2, idx, dh)) / (2 * eps)
    np.testing.assert_allclose(an["du"], du_fd, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(an["de"], de_fd, rtol=1e-6, atol=1e-7)


def test_gate_gradient_and_expert_output_gradient():
    """dL/dg_k = <dh, Y_k> and dL/dY_k = g_k dh, checked by moving one gate or
    one expert output in the forward's final sum."""
    u, e, W1, W3, W2, idx, dh = _setup(7)
    an = _analytic(u, e, W1, W3, W2, idx, dh)
    T, K = idx.shape
    y = an["y"]
    for t in range(T):
        for k in range(K):
            np.testing.assert_allclose(an["a"][t, k], dh[t] @ y[an["slot_row"][t, k]], rtol=1e-13)
    # dY of the shared rows is dh itself; of routed rows g * dh
    np.testing.assert_array_equal(an["dy"][T * K:], dh)
    s = 1.0 / (1.0 + np.exp(-(u @ e.T)))
    sc = s[np.arange(T)[:, None], idx]
    g = sc / sc.sum(axis=1, keepdims=True)
    for t in range(T):
        for k in range(K):
            np.testing.assert_allclose(an["dy"][an["slot_row"][t, k]], g[t, k] * dh[t], rtol=1e-15)


def test_gate_backward_zero_gradient_cases():
    """Uniform a (every chosen expert contributes the same to L): moving the
    scores only redistributes weight among equal terms, so dlogit = 0.  A
    token whose chosen scores sum to 0 gets dlogit 0."""
    T, K, d, E = 3, 4, 5, 8
    rng = np.random.default_rng(9)
    dh = rng.standard_normal((T, d))
    y = np.tile(rng.standard_normal((1, d)), (T * K, 1))       # every routed row the same
    slot_row = np.arange(T * K).reshape(T, K)
    idx = np.tile(np.arange(K), (T, 1))
    s = rng.uniform(0.1, 0.9, (T, E))
    gate = s[:, :K] / s[:, :K].sum(1, keepdims=True)
    _, _, dl = bw.gate_backward(dh, y, -1, gate, slot_row, s, idx)
    np.testing.assert_allclose(dl, 0.0, atol=1e-15)
    s0 = s.copy()
    s0[0, :K] = 0.0
    _, _, dl0 = bw.gate_backward(dh, rng.standard_normal((T * K, d)), -1, gate, slot_row, s0, idx)
    assert np.all(dl0[0] == 0.0)


@pytest.mark.parametrize("seed", [4, 5])
def test_weight_gradients_match_finite_differences(seed):
    """dL/dW1, dW3, dW2 of every expert (shared included) from the oracle's
    per-expert weight gradients over its rows, against central differences
    of the FP64 forward on a sample of weight entries."""
    u, e, W1, W3, W2, idx, dh = _setup(seed)
    T, K = idx.shape
    E = e.shape[0]
    an = _analytic(u, e, W1, W3, W2, idx, dh)
    pairs = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K))
    row_token = np.array([t for _, t, _ in pairs] + list(range(T)))
    row_group = np.array([g for g, _, _ in pairs] + [E] * T)
    x = u[row_token]
    zg = np.einsum("rid,rd->ri", W1[row_group], x)
    zu = np.einsum("rid,rd->ri", W3[row_group], x)
    grads = {}
    for g in range(E + 1):
        rows = np.nonzero(row_group == g)[0]
        dh_row = an["dy"][rows] @ W2[g]
        grads[g] = bw.expert_wgrad(an["dy"][rows], zg[rows], zu[rows], dh_row, x[rows])
    rng = np.random.default_rng(seed)
    eps = 1e-6
    for which, W in ((0, W2), (1, W1), (2, W3)):
        for _ in range(12):
            g = int(rng.integers(0, E + 1))
            i, j = (int(rng.integers(0, n)) for n in W.shape[1:])
            Wp, Wm = W.copy(), W.copy()
            Wp[g, i, j] += eps
            Wm[g, i, j] -= eps
            if which == 0:
                fd = (_loss(u, e, W1, W3, Wp, idx, dh) - _loss(u, e, W1, W3, Wm, idx, dh)) / (2 * eps)
            elif which == 1:
                fd = (_loss(u, e, Wp, W3, W2, idx, dh) - _loss(u, e, Wm, W3, W2, idx, dh)) / (2 * eps)
            else:
                fd = (_loss(u, e, W1, Wp, W2, idx, dh) - _loss(u, e, W1, Wm, W2, idx, dh)) / (2 * eps)
            np.testing.assert_allclose(grads[g][which][i, j], fd, rtol=1e-6, atol=1e-8)
