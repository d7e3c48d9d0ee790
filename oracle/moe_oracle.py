"""CPU oracle for the forward pass of a dropless MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the tests, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

It is the plain, slow definition of what the layer computes, in fp64, written in
the order the pages give the steps.  Sources, cited by page title and section:

  [TL]  TileLang tutorial, chapter "MoE, MLA and sparse-attention operators"
        (tilelang-tutorial.huandu.me/16-operators-moe-mla): section 2.2 router and
        gating, 2.3 dispatch/permute, 2.4 grouped GEMM, 2.5 combine.
  [DG]  Course notes "Dropless and grouped GEMM" (topic-01-dropless): section 1
        (shared expert, received rows), 3 (pad every segment to a multiple of 128),
        4 (the per-step tensor table), 5 (offsets as a prefix sum, tile -> expert
        tables), 7 (the per-expert for-loop formulation), 10 (decode boundary cases),
        11 (the unpadded alternative: boundary tiles executed once per group).

Readings taken where the pages are silent or ambiguous (each one is also listed in
the design notes):
  * padding: ceil(c / bm) * bm per expert, so an empty expert gets no rows [DG §3,
    §10]; the "+1" form printed in [TL §2.3] is not used.
  * experts are chosen on fp32 logits (the precision the device computes them in),
    by k rounds of "take the largest remaining", ties to the lower expert id [TL §2.2];
    softmax over all E experts gives the weights; renormalisation is optional.
  * group-limited routing: experts form n_groups contiguous id ranges; a group's
    score is its largest logit; the topk_groups best groups stay eligible (ties to
    the lower group id) [TL §2.2; DG §4 step 4].
  * within an expert's segment rows keep ascending assignment order a = t*k + j (a
    stable sort by expert id) [TL §2.3 "source addresses come from the argsort"].
  * W1 is the gate and W3 the up projection: act = silu(x W1) * (x W3), y = act W2
    [TL §2.4 (c)].  The routing weight is applied in combine [TL §2.5].
  * combine sums the k slots in ascending j, then adds the shared expert [TL §2.5;
    DG §1].

Function pins (what fixes each function other than itself) live in
tests/test_oracle_pins.py.  Parity unpinned: none of the functions below; the
``waste_report`` numbers of [TL §2.3] (320 rows, 150 %, 3.31x) cannot be
reproduced because the simulation's input is not on the page, so only the report's
definition is pinned, not those values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Step 1 - router GEMM  [TL §2.2: logits = x[T,d] @ W_g[d,E], an M=T, N=E, K=d GEMM]
# ----------------------------------------------------------------------------
def router_logits(x, w_gate, bias=None):
    """fp64 logits[t, e] = sum_i x[t, i] * W_g[i, e] (+ bias[e]).

    The per-expert bias is part of the logit: it moves both the choice of experts
    and their softmax weights.
    """
    logits = np.asarray(x, F64) @ np.asarray(w_gate, F64)
    if bias is not None:
        logits = logits + np.asarray(bias, F64)[None, :]
    return logits


# ----------------------------------------------------------------------------
# Step 2 - group limit, top-k, softmax weights  [TL §2.2; DG §4 steps 3-4]
# ----------------------------------------------------------------------------
def eligible_experts(logits, n_groups: int, topk_groups: int):
    """Boolean [T, E] mask of experts a token may pick.

    No group limit (n_groups == 0): every expert.  Otherwise the E experts form
    n_groups contiguous blocks of E / n_groups ids; each block is scored by its
    largest logit and the topk_groups best blocks stay eligible, taken one at a time
    by "largest remaining score, lower group id on ties".
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if n_groups == 0:
        return np.ones((T, E), dtype=bool)
    gsize = E // n_groups
    gscore = logits.reshape(T, n_groups, gsize).max(axis=2).astype(F64)
    keep = np.zeros((T, n_groups), dtype=bool)
    rows = np.arange(T)
    for _ in range(topk_groups):
        g = np.argmax(np.where(keep, -np.inf, gscore), axis=1)  # first max = lower id
        keep[rows, g] = True
    return np.repeat(keep, gsize, axis=1)


def topk_by_repeated_max(logits, k: int, eligible=None):
    """[T, k] expert ids: k rounds of "largest remaining logit", ties to the lower id.

    This is the small-k selection of [TL §2.2] (take the maximum, remove it, repeat),
    so slot j holds the j-th largest eligible logit.  Comparisons are made on the
    values exactly as given (fp32 logits in every use here).
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    taken = np.zeros((T, E), dtype=bool)
    if eligible is None:
        eligible = np.ones((T, E), dtype=bool)
    rows = np.arange(T)
    idx = np.empty((T, k), dtype=np.int32)
    vals = logits.astype(F64)
    for j in range(k):
        cand = np.where(eligible & ~taken, vals, -np.inf)
        e = np.argmax(cand, axis=1)                 # numpy returns the first maximum
        idx[:, j] = e
        taken[rows, e] = True
    return idx


def softmax(logits):
    """Row softmax over all E experts in fp64 (maximum subtracted first)."""
    l = np.asarray(logits, F64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def gate_weights(logits, idx, renormalize: bool):
    """w[t, j] = softmax(logits)[t, idx[t, j]], optionally divided by sum_j w[t, j]."""
    p = softmax(logits)
    w = np.take_along_axis(p, np.asarray(idx, np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def route(x, w_gate, bias, k, n_groups=0, topk_groups=0, renormalize=False,
          decision_logits=None):
    """Router, top-k and weights.

    The expert choice is an integer decided by floating point, so it is taken in
    the precision the device keeps logits in (fp32).  ``decision_logits`` lets a
    test hand in the device's own fp32 logits, so both sides decide on identical
    numbers; otherwise the fp64 logits rounded to fp32 are used.
    """
    logits = router_logits(x, w_gate, bias)
    dec = (logits.astype(np.float32) if decision_logits is None
           else np.asarray(decision_logits, np.float32))
    elig = eligible_experts(dec, n_groups, topk_groups)
    idx = topk_by_repeated_max(dec, k, elig)
    w = gate_weights(dec, idx, renormalize)
    return logits, idx, w


# ----------------------------------------------------------------------------
# Step 3 - counts -> offsets -> padded offsets -> block metadata
# [TL §2.2 item 2 and §2.3 item 2; DG §3 padding table, §5 offsets, §10]
# ----------------------------------------------------------------------------
def expert_counts(idx, E: int):
    """c[e] = number of (token, slot) pairs routed to expert e."""
    flat = np.asarray(idx).ravel()
    c = np.zeros(E, dtype=np.int64)
    np.add.at(c, flat, 1)
    return c


def group_offsets(counts):
    """Exclusive prefix sum: off[e] is the first row of expert e, off[E] = T*k."""
    c = np.asarray(counts, np.int64)
    off = np.zeros(len(c) + 1, dtype=np.int64)
    off[1:] = np.cumsum(c)
    return off


def padded_offsets(counts, block_m: int):
    """P[e+1] = P[e] + ceil(c[e] / block_m) * block_m, P[0] = 0.

    Every segment is rounded up to the next multiple of block_m; an exact multiple
    gains nothing and an empty expert keeps zero rows [DG §3, §10].
    """
    c = np.asarray(counts, np.int64)
    seg = -(-c // block_m) * block_m
    P = np.zeros(len(c) + 1, dtype=np.int64)
    P[1:] = np.cumsum(seg)
    return P


def block_metadata(counts, block_m: int):
    """Rows of (expert, m_start, valid_m), one per block_m-row block, experts in
    ascending order; the table has sum_e ceil(c[e] / block_m) rows [TL §2.3 item 2,
    §2.4 (a)]."""
    P = padded_offsets(counts, block_m)
    out = []
    for e, c in enumerate(np.asarray(counts, np.int64)):
        nb = -(-int(c) // block_m)
        for i in range(nb):
            out.append((e, int(P[e]) + i * block_m, min(block_m, int(c) - i * block_m)))
    return np.asarray(out, dtype=np.int64).reshape(-1, 3)


def permutation(idx, E: int, block_m: int):
    """pos[a] = padded row of assignment a = t*k + j; row_src[row] = a (or -1 on pads).

    A stable sort of the assignments by expert id puts expert 0's assignments first,
    each segment in ascending a; segment e starts at the padded offset P[e].
    """
    flat = np.asarray(idx, np.int64).ravel()
    M = flat.size
    counts = expert_counts(flat, E)
    off = group_offsets(counts)
    P = padded_offsets(counts, block_m)
    order = np.argsort(flat, kind="stable")
    e_sorted = flat[order]
    pos = np.empty(M, dtype=np.int64)
    pos[order] = P[e_sorted] + (np.arange(M) - off[e_sorted])
    row_src = np.full(int(P[-1]), -1, dtype=np.int64)
    row_src[pos] = np.arange(M)
    return pos, row_src


# ----------------------------------------------------------------------------
# Step 3' - unpadded segments  [DG §11: a boundary tile executed once per group]
# ----------------------------------------------------------------------------
def unpadded_tile_table(counts, tile: int):
    """The executions of the unpadded layout, rows (expert, m_start, valid_m).

    [DG §11]: no segment is rounded up; expert e keeps rows [off[e], off[e+1]) of the
    M = sum(c) rows (off = group_offsets).  The row space is cut into tiles of ``tile``
    rows (the last one may be short), and a tile holding rows of several experts is
    executed once for each of them with that expert's weights, restricted to that
    expert's rows.  Executions are listed tile by tile and, inside a tile, by expert;
    m_start is the expert's first row in the tile, valid_m its number of rows there.
    """
    off = group_offsets(counts)
    M = int(off[-1])
    out = []
    for t0 in range(0, M, tile):
        t1 = min(t0 + tile, M)
        for e in range(len(off) - 1):
            lo, hi = max(t0, int(off[e])), min(t1, int(off[e + 1]))
            if hi > lo:
                out.append((e, lo, hi - lo))
    return np.asarray(out, dtype=np.int64).reshape(-1, 3)


def permutation_unpadded(idx, E: int):
    """pos / row_src of the unpadded layout: the stable sort of ``permutation`` with
    every segment at its real length (a padding multiple of 1), so row_src covers
    exactly the M assignments."""
    return permutation(idx, E, 1)


# ----------------------------------------------------------------------------
# Step 4 - permute  [TL §2.3: a data-dependent gather; DG §4 steps 5-6]
# ----------------------------------------------------------------------------
def permute(x, pos, k: int, n_rows: int):
    """x_perm[pos[t*k + j]] = x[t]; pad rows are zero (they are never used)."""
    x = np.asarray(x, F64)
    xp = np.zeros((n_rows, x.shape[1]), dtype=F64)
    a = np.arange(len(pos))
    xp[np.asarray(pos)] = x[a // k]
    return xp


# ----------------------------------------------------------------------------
# Step 5 - experts: SwiGLU gate/up, then down  [TL §2.4 (c); DG §4 steps 7-9, §7]
# ----------------------------------------------------------------------------
def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_act(rows, w1, w3):
    """act = silu(rows @ W1) * (rows @ W3)."""
    r = np.asarray(rows, F64)
    return silu(r @ np.asarray(w1, F64)) * (r @ np.asarray(w3, F64))


def expert_ffn(rows, w1, w3, w2):
    """y = (silu(rows @ W1) * (rows @ W3)) @ W2."""
    return swiglu_act(rows, w1, w3) @ np.asarray(w2, F64)


def grouped_ffn(x_perm, counts, block_m, w1, w3, w2):
    """The per-expert loop over contiguous padded segments [DG §7]: expert e's
    segment starts at P[e] and holds c[e] real rows; pad rows stay zero.

    Returns (act, y), both [P[E], ...] fp64.
    """
    P = padded_offsets(counts, block_m)
    n_rows = int(P[-1])
    d_e = np.asarray(w1).shape[2]
    d = np.asarray(w2).shape[2]
    act = np.zeros((n_rows, d_e), dtype=F64)
    y = np.zeros((n_rows, d), dtype=F64)
    for e, c in enumerate(np.asarray(counts, np.int64)):
        if c == 0:
            continue
        lo, hi = int(P[e]), int(P[e]) + int(c)
        act[lo:hi] = swiglu_act(x_perm[lo:hi], w1[e], w3[e])
        y[lo:hi] = act[lo:hi] @ np.asarray(w2[e], F64)
    return act, y


# ----------------------------------------------------------------------------
# Step 6 - shared expert and combine  [DG §1 shared expert; TL §2.5]
# ----------------------------------------------------------------------------
def shared_expert(x, ws1, ws3, ws2):
    """A dense SwiGLU MLP on the unpermuted input: every token goes through it."""
    return expert_ffn(x, ws1, ws3, ws2)


def combine(y, pos, w, k: int, shared=None):
    """out[t] = sum_{j = 0..k-1, ascending} w[t, j] * y[pos[t*k + j]] (+ shared[t])."""
    y = np.asarray(y, F64)
    w = np.asarray(w, F64)
    T = w.shape[0]
    pos = np.asarray(pos).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=F64)
    for j in range(k):
        out += w[:, j:j + 1] * y[pos[:, j]]
    if shared is not None:
        out += np.asarray(shared, F64)
    return out


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------
@dataclass
class LayerResult:
    logits: Optional[np.ndarray]
    topk_idx: np.ndarray
    topk_w: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    padded_offsets: np.ndarray
    block_meta: np.ndarray
    pos: np.ndarray
    row_src: np.ndarray
    act: Optional[np.ndarray]
    y: Optional[np.ndarray]
    shared: Optional[np.ndarray]
    out: np.ndarray


def moe_layer(x, w1, w3, w2, *, k, block_m, w_gate=None, bias=None, n_groups=0,
              topk_groups=0, renormalize=False, ws1=None, ws3=None, ws2=None,
              topk_idx=None, topk_w=None, decision_logits=None):
    """Router -> top-k -> counts/offsets -> permute -> grouped SwiGLU -> combine.

    With ``topk_idx``/``topk_w`` given the router is skipped (rows already routed,
    as on one rank of an expert-parallel group [DG §4 step 5]).
    """
    x = np.asarray(x)
    E = np.asarray(w1).shape[0]
    logits = None
    if topk_idx is None:
        logits, topk_idx, topk_w = route(x, w_gate, bias, k, n_groups, topk_groups,
                                         renormalize, decision_logits)
    topk_idx = np.asarray(topk_idx, np.int64)
    counts = expert_counts(topk_idx, E)
    off = group_offsets(counts)
    P = padded_offsets(counts, block_m)
    meta = block_metadata(counts, block_m)
    pos, row_src = permutation(topk_idx, E, block_m)
    xp = permute(x, pos, k, int(P[-1]))
    act, y = grouped_ffn(xp, counts, block_m, w1, w3, w2)
    s = shared_expert(x, ws1, ws3, ws2) if ws1 is not None else None
    out = combine(y, pos, topk_w, k, s)
    return LayerResult(logits, topk_idx.astype(np.int32), np.asarray(topk_w, F64), counts,
                       off, P, meta, pos, row_src, act, y, s, out)


def direct_layer(x, w1, w3, w2, topk_idx, topk_w, ws1=None, ws3=None, ws2=None):
    """Each token evaluated against the experts it chose, with no permutation:
    out[t] = sum_j w[t, j] * FFN_{idx[t, j]}(x[t]) (+ shared(x[t])), j ascending.
    Equal to ``moe_layer`` because permute/combine only move rows [TL §2.3]."""
    x = np.asarray(x, F64)
    T, k = np.asarray(topk_idx).shape
    out = np.zeros((T, np.asarray(w2).shape[2]), dtype=F64)
    for t in range(T):
        acc = np.zeros(out.shape[1], dtype=F64)
        for j in range(k):
            e = int(topk_idx[t, j])
            acc += float(topk_w[t, j]) * expert_ffn(x[t:t + 1], w1[e], w3[e], w2[e])[0]
        if ws1 is not None:
            acc += expert_ffn(x[t:t + 1], ws1, ws3, ws2)[0]
        out[t] = acc
    return out


# ----------------------------------------------------------------------------
# Padding-waste report of the skewed-routing simulation [TL §2.3 item 3]
# ----------------------------------------------------------------------------
def waste_report(counts, block_m: int):
    """Padded rows, waste as a fraction of real assignments, hottest expert / mean."""
    c = np.asarray(counts, np.int64)
    P = padded_offsets(c, block_m)
    real = int(c.sum())
    padded = int(P[-1])
    return {
        "assignments": real,
        "padded_rows": padded,
        "waste": (padded - real) / real if real else 0.0,
        "hottest_over_mean": float(c.max() / (real / len(c))) if real else 0.0,
    }
