"""CPU oracle for the backward of the DeepSeekMoE layer (input and weight
gradients)
-- TEST INFRASTRUCTURE ONLY (the tests may import it; the HIP library never
does, and this module imports nothing from it).

Plain FP64 numpy, written from the layer's output equation (nlp-lineage
summary, "The notation"):
    h'_t = u_t + FFN_shared(u_t) + sum_k g_(k,t) FFN_(i_k)(u_t),
    g_(k,t) = s_(i_k,t) / D_t,  D_t = sum_k s_(i_k,t),  s_(i,t) = sigmoid(u_t . e_i)
("DeepSeek-V3 Technical Report" notes, MoE-routing paragraph: the two
formulas on the second line; bias paragraph: b only ranks the experts, so it
has no gradient and the chosen set is constant under small changes).  FFN(x) = W2 (SiLU(W1 x) * W3 x) is this build's reading
of the expert form.  Given dL/dh' = dh for a scalar loss L, the chain rule
gives, for token t and slot k:
    a_k      = <dh, Y_k>                          (dL/dg_k, Y_k the expert output)
    dL/ds_k  = (a_k - sum_j g_j a_j) / D          (through the normalisation)
    dlogit_k = dL/ds_k * s_k (1 - s_k)            (through the sigmoid)
    dY_k     = g_k dh,   dY_shared = dh           (into the expert outputs)
and per expert row, with z_g = W1 x, z_u = W3 x, h = SiLU(z_g) z_u:
    dh_row   = W2^T dY
    dz_u     = dh_row * SiLU(z_g)
    dz_g     = dh_row * z_u * sigma(z_g) (1 + z_g (1 - sigma(z_g)))
    dx       = W1^T dz_g + W3^T dz_u
and finally
    du_t = dh_t + sum over the token's rows of dx + sum_k dlogit_k e_(i_k)
    de_i = sum over the (t, k) that chose i of dlogit_k u_t
and, per expert, the weight gradients over its rows:
    dW2 = sum_r dY_r^T h_r,  dW1 = sum_r dz_g,r^T x_r,  dW3 = sum_r dz_u,r^T x_r.
Each function takes the operands it is given (dequantised FP8 ones for GPU
parity, unquantised ones for the finite-difference pins) and computes in FP64.
"""
from __future__ import annotations

import numpy as np


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def gate_backward(dh, y, shared_row0: int, gate, slot_row, s, idx):
    """a [T,K], dY [R,d] and dlogit [T,K] (FP64) for upstream gradient dh [T,d],
    expert outputs y [R,d] (rows as the dispatch lays them out), the gates and
    slot rows [T,K], the raw scores s [T,E] and the choices idx [T,K].  Rows of
    y not used by any slot or the shared block get a zero dY.  A token whose
    chosen scores sum to 0 gets dlogit 0."""
    dh = np.asarray(dh, np.float64)
    y = np.asarray(y, np.float64)
    g = np.asarray(gate, np.float64)
    slot_row = np.asarray(slot_row, np.int64)
    idx = np.asarray(idx, np.int64)
    T, K = g.shape
    a = np.einsum("tc,tkc->tk", dh, y[slot_row])
    sc = np.asarray(s, np.float64)[np.arange(T)[:, None], idx]
    D = sc.sum(axis=1)
    safe = np.where(D == 0, 1.0, D)
    ds = (a - (g * a).sum(axis=1, keepdims=True)) / safe[:, None]
    ds[D == 0] = 0.0
    dlogit = ds * sc * (1.0 - sc)
    dy = np.zeros_like(y)
    dy[slot_row] = g[:, :, None] * dh[:, None, :]
    if shared_row0 >= 0:
        dy[shared_row0:shared_row0 + T] = dh
    return a, dy, dlogit


def swiglu_backward(zg, zu, dh_row):
    """dz_gate, dz_up (FP64) of h = SiLU(z_gate) * z_up."""
    zg = np.asarray(zg, np.float64)
    zu = np.asarray(zu, np.float64)
    dh_row = np.asarray(dh_row, np.float64)
    sg = _sigmoid(zg)
    dzu = dh_row * zg * sg
    dzg = dh_row * zu * sg * (1.0 + zg * (1.0 - sg))
    return dzg, dzu


def expert_dgrad(dy_rows, zg, zu, w1, w3, w2):
    """Rows of one expert: dh_row = dY W2, then the SwiGLU backward, then
    dx = dz_g W1 + dz_u W3.  w1, w3 [I,d], w2 [d,I] (dequantised or masters)."""
    w1, w3, w2 = (np.asarray(w, np.float64) for w in (w1, w3, w2))
    dh_row = np.asarray(dy_rows, np.float64) @ w2
    dzg, dzu = swiglu_backward(zg, zu, dh_row)
    return dh_row, dzg, dzu, dzg @ w1 + dzu @ w3


def router_backward(u, e, idx, dlogit, E: int):
    """du_router [T,d] = sum_k dlogit_k e_(i_k); de [E,d] = sum over the (t,k)
    that chose i of dlogit_k u_t (FP64; u and e as values)."""
    u = np.asarray(u, np.float64)
    e = np.asarray(e, np.float64)
    idx = np.asarray(idx, np.int64)
    dlogit = np.asarray(dlogit, np.float64)
    du = np.einsum("tk,tkc->tc", dlogit, e[idx])
    de = np.zeros((E, u.shape[1]), np.float64)
    np.add.at(de, idx.reshape(-1), (dlogit[:, :, None] * u[:, None, :]).reshape(-1, u.shape[1]))
    return du, de


def assemble_du(dh, dx_rows, row_token):
    """du_t = dh_t + the sum of dx over the GEMM rows of token t (the router
    term is added by the caller)."""
    du = np.array(dh, np.float64, copy=True)
    np.add.at(du, np.asarray(row_token, np.int64), np.asarray(dx_rows, np.float64))
    return du


def expert_wgrad(dy_rows, zg, zu, dh_row, x_rows):
    """Weight gradients of one expert from its rows (FP64):
        dW2 [d,I] = sum_r dY_r^T h_r,  h = SiLU(z_g) z_u
        dW1 [I,d] = sum_r dz_g,r^T x_r,  dW3 [I,d] = sum_r dz_u,r^T x_r
    with dz from swiglu_backward(z_g, z_u, dh_row)."""
    zg = np.asarray(zg, np.float64)
    zu = np.asarray(zu, np.float64)
    h = zg * _sigmoid(zg) * zu
    dzg, dzu = swiglu_backward(zg, zu, dh_row)
    dy = np.asarray(dy_rows, np.float64)
    x = np.asarray(x_rows, np.float64)
    return dy.T @ h, dzg.T @ x, dzu.T @ x
