"""CPU oracle for the backward pass of the dropless MoE layer.

TEST INFRASTRUCTURE ONLY, like moe_oracle: only the tests, the smoke check and the
bench's CPU leg may use it; it shares no code with the HIP library.

The course notes "Dropless and grouped GEMM" (topic-01-dropless) name the backward of
the grouped layer as the next step after the forward: the gradients of the grouped
GEMMs are grouped GEMMs again (data gradients through the transposed weights, weight
gradients reducing over each expert's rows), and the permutation is replayed from the
saved sort indices rather than recomputed.  The pages print no formulas for it, so
this module is the chain rule of the forward definition (moe_oracle), step by step in
reverse order, in fp64:

  combine   out[t] = sum_j w[t,j] y[pos[t,j]] + s[t]
            -> dy[pos[t,j]] = w[t,j] dout[t];  dw[t,j] = <dout[t], y[pos[t,j]]>;
               ds[t] = dout[t]
  down      y[r] = act[r] W2[e]
            -> dact[r] = dy[r] W2[e]^T;  dW2[e] = sum_{r in e} act[r]^T dy[r]
  SwiGLU    act = silu(g) u,  g = xp W1[e],  u = xp W3[e]
            -> dg = dact u silu'(g),  du = dact silu(g),
               silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
  gate/up   -> dxp[r] = dg[r] W1[e]^T + du[r] W3[e]^T;
               dW1[e] = sum xp^T dg;  dW3[e] = sum xp^T du
  permute   -> dx[t] += sum_j dxp[pos[t,j]]
  shared    the same three steps for one expert over all tokens, output gradient ds
  router    w = softmax(logits)[idx] (optionally divided by its sum over the k slots):
            -> dlogits from dw through the softmax (and renormalisation) Jacobian,
               with the selection itself held fixed (it is piecewise constant);
               dW_g = x^T dlogits;  dbias = sum_t dlogits;  dx += dlogits W_g^T
Pins: tests/test_backward_oracle_pins.py (central finite differences of <dout, out>
on small inputs, and torch fp64 autograd of an independent per-token formulation).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from oracle import moe_oracle as O

F64 = np.float64


def sigmoid(z):
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu_grad(z):
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, F64)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def combine_backward(dout, y, pos, w, k: int):
    """(dy rows [n_rows, d] (zero on rows no slot uses), dw [T, k])."""
    dout = np.asarray(dout, F64)
    y = np.asarray(y, F64)
    w = np.asarray(w, F64)
    T = dout.shape[0]
    pos = np.asarray(pos).reshape(T, k)
    dy = np.zeros_like(y)
    dw = np.zeros((T, k), dtype=F64)
    for j in range(k):
        dy[pos[:, j]] = w[:, j:j + 1] * dout
        dw[:, j] = np.sum(dout * y[pos[:, j]], axis=1)
    return dy, dw


def swiglu_backward(rows, w1, w3, dact):
    """Recompute g, u from the rows and return (dg, du, act)."""
    r = np.asarray(rows, F64)
    g = r @ np.asarray(w1, F64)
    u = r @ np.asarray(w3, F64)
    dact = np.asarray(dact, F64)
    act = O.silu(g) * u
    return dact * u * silu_grad(g), dact * O.silu(g), act


def expert_backward(rows, w1, w3, w2, dy):
    """One expert (or the shared one) on its rows: (drows, dW1, dW3, dW2)."""
    r = np.asarray(rows, F64)
    dy = np.asarray(dy, F64)
    g = r @ np.asarray(w1, F64)
    u = r @ np.asarray(w3, F64)
    act = O.silu(g) * u
    dact = dy @ np.asarray(w2, F64).T
    dW2 = act.T @ dy
    dg, du, _ = swiglu_backward(r, w1, w3, dact)
    drows = dg @ np.asarray(w1, F64).T + du @ np.asarray(w3, F64).T
    return drows, r.T @ dg, r.T @ du, dW2


def grouped_backward(x_perm, counts, block_m, w1, w3, w2, dy):
    """The per-expert loop over the padded segments: (dx_perm, dW1, dW3, dW2); experts
    without rows get zero weight gradients."""
    P = O.padded_offsets(counts, block_m)
    w1 = np.asarray(w1, F64)
    w3 = np.asarray(w3, F64)
    w2 = np.asarray(w2, F64)
    dxp = np.zeros_like(np.asarray(x_perm, F64))
    dW1, dW3, dW2 = np.zeros_like(w1), np.zeros_like(w3), np.zeros_like(w2)
    for e, c in enumerate(np.asarray(counts, np.int64)):
        if c == 0:
            continue
        lo, hi = int(P[e]), int(P[e]) + int(c)
        dxp[lo:hi], dW1[e], dW3[e], dW2[e] = expert_backward(x_perm[lo:hi], w1[e], w3[e], w2[e],
                                                             dy[lo:hi])
    return dxp, dW1, dW3, dW2


def unpermute_sum(dx_perm, pos, T: int, k: int):
    """dx[t] = sum_j dx_perm[pos[t, j]], j ascending."""
    dxp = np.asarray(dx_perm, F64)
    pos = np.asarray(pos).reshape(T, k)
    dx = np.zeros((T, dxp.shape[1]), dtype=F64)
    for j in range(k):
        dx += dxp[pos[:, j]]
    return dx


def router_backward(logits, idx, dw, renormalize: bool):
    """dlogits [T, E] from the gradient of the routing weights, the selection fixed."""
    logits = np.asarray(logits, F64)
    idx = np.asarray(idx, np.int64)
    dw = np.asarray(dw, F64)
    T, E = logits.shape
    p = O.softmax(logits)
    ps = np.take_along_axis(p, idx, axis=1)             # p at the selected experts
    if renormalize:
        Z = ps.sum(axis=1, keepdims=True)
        w = ps / Z
        dps = (dw - np.sum(dw * w, axis=1, keepdims=True)) / Z
    else:
        dps = dw
    # dp[t, e] = sum over slots choosing e of dps; softmax: dl = p * (dp - <dp, p>)
    dp = np.zeros((T, E), dtype=F64)
    for j in range(idx.shape[1]):
        np.add.at(dp, (np.arange(T), idx[:, j]), dps[:, j])
    return p * (dp - np.sum(dp * p, axis=1, keepdims=True))


@dataclass
class LayerGrads:
    dx: np.ndarray
    dw1: np.ndarray
    dw3: np.ndarray
    dw2: np.ndarray
    dws1: Optional[np.ndarray]
    dws3: Optional[np.ndarray]
    dws2: Optional[np.ndarray]
    dtopk_w: np.ndarray
    dlogits: Optional[np.ndarray]
    dw_gate: Optional[np.ndarray]
    dbias: Optional[np.ndarray]
    # intermediates of the backward, for stage-wise checks
    dy: np.ndarray
    dact: np.ndarray
    dg: np.ndarray
    du: np.ndarray
    dx_perm: np.ndarray


def moe_layer_backward(fwd, x, w1, w3, w2, dout, *, k, block_m, w_gate=None, bias=None,
                       renormalize=False, ws1=None, ws3=None, ws2=None, routed=False):
    """Gradients of <dout, out> for the layer whose forward result is ``fwd``
    (moe_oracle.moe_layer's LayerResult on the same inputs).  ``routed``: the routes
    were given (no router, no router gradients)."""
    x = np.asarray(x, F64)
    T = x.shape[0]
    E = np.asarray(w1).shape[0]
    dout = np.asarray(dout, F64)
    dy, dw = combine_backward(dout, fwd.y, fwd.pos, fwd.topk_w, k)
    xp = O.permute(x, fwd.pos, k, len(fwd.row_src))
    P = fwd.padded_offsets
    dact = np.zeros((len(fwd.row_src), np.asarray(w1).shape[2]), dtype=F64)
    dg = np.zeros_like(dact)
    du = np.zeros_like(dact)
    for e, c in enumerate(np.asarray(fwd.counts, np.int64)):
        if c == 0:
            continue
        lo, hi = int(P[e]), int(P[e]) + int(c)
        dact[lo:hi] = dy[lo:hi] @ np.asarray(w2[e], F64).T
        dg[lo:hi], du[lo:hi], _ = swiglu_backward(xp[lo:hi], w1[e], w3[e], dact[lo:hi])
    dxp, dW1, dW3, dW2 = grouped_backward(xp, fwd.counts, block_m, w1, w3, w2, dy)
    dx = unpermute_sum(dxp, fwd.pos, T, k)
    dws1 = dws3 = dws2 = None
    if ws1 is not None:
        dxs, dws1, dws3, dws2 = expert_backward(x, ws1, ws3, ws2, dout)
        dx = dx + dxs
    dlogits = dw_gate = dbias = None
    if not routed:
        dlogits = router_backward(fwd.logits, fwd.topk_idx, dw, renormalize)
        dw_gate = x.T @ dlogits
        dbias = dlogits.sum(axis=0)
        dx = dx + dlogits @ np.asarray(w_gate, F64).T
    return LayerGrads(dx, dW1, dW3, dW2, dws1, dws3, dws2, dw, dlogits, dw_gate, dbias,
                      dy, dact, dg, du, dxp)
