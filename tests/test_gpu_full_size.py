"""Parity at the full workload sizes, through moe_layer_fwd (the launches the
benchmark times), against the oracle.

At these sizes the oracle cannot run the whole layer in seconds, so:
  * routing, counts, offsets, padded offsets, block table, pos and row_src are
    checked in full (cheap integer work and one small fp64 product for the logits);
    integers bit-exactly;
  * x_perm, act and y on sampled rows: the first and last rows of every expert
    segment plus a seeded random set, each recomputed by the oracle on its own;
  * the layer output on sampled tokens (first, last, seeded random), each from the
    oracle's per-token definition, at the layer tolerance;
  * pad rows and unwritten rows keep their sentinel, and every real row is finite.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import moe_oracle as O
from workloads.configs import get_config
from workloads.gen import make_inputs

from gpu_util import (TOL_LOGITS, TOL_OUT, TOL_STAGE, TOL_W_REL, LayerRun, assert_close, f64,
                      i64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
FULL = ["fusedmoe-8x2048", "ep-share-4x2048", "decode-256x2048", "zipf-skew-64x1408"]
N_ROWS = 48      # sampled permuted rows (plus segment ends)
N_TOK = 24       # sampled tokens (plus first and last)


@pytest.fixture(scope="module", params=FULL)
def full(request):
    cfg = get_config(request.param)
    print(f"[full-size] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_e={cfg.d_e}",
          flush=True)
    inp = make_inputs(cfg, DEV)
    run = LayerRun(cfg, inp)
    yield cfg, inp, run
    del run, inp
    torch.cuda.empty_cache()


def _routing(cfg, inp, run):
    """(topk_idx, topk_w) the layer used, checked against the oracle when it routed."""
    if run.routed:
        return i64(inp.topk_idx), f64(inp.topk_w)
    idx_dev, w_dev = (t.cpu().numpy() for t in run.topk())
    return idx_dev.astype(np.int64), w_dev.astype(np.float64)


def test_full_size_routing(full):
    cfg, inp, run = full
    if run.routed:
        pytest.skip("rows arrive already routed")
    x, wg = f64(inp.x), f64(inp.w_gate)
    bias = None if inp.bias is None else f64(inp.bias)
    ref_logits = O.router_logits(x, wg, bias)
    dev_logits = run.logits().cpu().numpy()
    assert_close(dev_logits, ref_logits, TOL_LOGITS[cfg.dtype], "logits")
    _, idx_ref, w_ref = O.route(x, wg, bias, cfg.k, cfg.n_groups, cfg.topk_groups,
                                cfg.renormalize, decision_logits=dev_logits)
    idx_dev, w_dev = _routing(cfg, inp, run)
    assert np.array_equal(idx_dev, idx_ref)
    assert np.all(np.abs(w_dev - w_ref) <= TOL_W_REL * np.abs(w_ref) + 1e-30)


def test_full_size_integer_stages(full):
    cfg, inp, run = full
    idx, _ = _routing(cfg, inp, run)
    got = run.ints()
    assert got["err_flag"] == 0
    c = O.expert_counts(idx, cfg.E)
    assert np.array_equal(got["counts"], c)
    assert np.array_equal(got["offsets"], O.group_offsets(c))
    P = O.padded_offsets(c, cfg.block_m)
    assert np.array_equal(got["padded_offsets"], P)
    meta = O.block_metadata(c, cfg.block_m)
    assert got["num_blocks"] == len(meta)
    assert np.array_equal(got["block_meta"], np.asarray(meta).reshape(-1, 3))
    pos, row_src = O.permutation(idx, cfg.E, cfg.block_m)
    assert np.array_equal(got["pos"], pos)
    n = int(P[-1])
    assert np.array_equal(got["row_src"][:n], row_src)
    assert np.all(got["row_src"][n:] == -1)
    assert got["num_blocks"] <= B.moe_max_blocks(run.shape)


def _sample_rows(cfg, c, P, rng):
    rows = set()
    for e in range(cfg.E):
        if c[e]:
            rows.update({int(P[e]), int(P[e] + c[e] - 1)})
    real = np.concatenate([np.arange(P[e], P[e] + c[e]) for e in range(cfg.E)]).astype(np.int64)
    rows.update(int(r) for r in rng.choice(real, size=min(N_ROWS, len(real)), replace=False))
    rows = np.array(sorted(rows), np.int64)
    expert = np.searchsorted(P, rows, side="right") - 1
    return rows, expert


def test_full_size_grouped_gemm_rows(full):
    """Sampled permuted rows: x_perm exact, act = silu(x W1) * (x W3) and y = act W2 per
    the oracle, each stage fed the device's own input row (stage tolerance)."""
    cfg, inp, run = full
    idx, _ = _routing(cfg, inp, run)
    c = O.expert_counts(idx, cfg.E)
    P = O.padded_offsets(c, cfg.block_m)
    pos, row_src = O.permutation(idx, cfg.E, cfg.block_m)
    rng = np.random.default_rng(cfg.seed + 7)
    rows, expert = _sample_rows(cfg, c, P, rng)
    rt = torch.from_numpy(rows).to(DEV)
    xp = f64(run.x_perm()[rt])
    act = f64(run.act()[rt])
    y = f64(run.y()[rt])
    x = inp.x
    xp_ref = f64(x[torch.from_numpy(row_src[rows] // cfg.k).to(DEV)])
    assert np.array_equal(xp, xp_ref)
    w_cache = {}

    def w(e):
        if e not in w_cache:
            w_cache[e] = (f64(inp.w1[e]), f64(inp.w3[e]), f64(inp.w2[e]))
        return w_cache[e]

    act_ref = np.stack([O.swiglu_act(xp[i:i + 1], *w(int(e))[:2])[0] for i, e in enumerate(expert)])
    y_ref = np.stack([act[i:i + 1] @ w(int(e))[2] for i, e in enumerate(expert)])[:, 0]
    assert_close(act, act_ref, TOL_STAGE[cfg.dtype], "act rows")
    assert_close(y, y_ref, TOL_STAGE[cfg.dtype], "y rows")


def test_full_size_sampled_tokens(full):
    cfg, inp, run = full
    idx, w = _routing(cfg, inp, run)
    rng = np.random.default_rng(cfg.seed + 11)
    toks = sorted({0, cfg.T - 1} | set(int(t) for t in rng.choice(cfg.T, size=min(N_TOK, cfg.T),
                                                                     replace=False)))
    tt = torch.tensor(toks, device=DEV)
    out = f64(run.out[tt])
    assert np.all(np.isfinite(f64(run.out)))
    x = f64(inp.x[tt])
    used = sorted(set(int(e) for t in toks for e in idx[t]))
    W = {e: (f64(inp.w1[e]), f64(inp.w3[e]), f64(inp.w2[e])) for e in used}
    sh = (f64(inp.ws1), f64(inp.ws3), f64(inp.ws2)) if cfg.d_e_shared else (None, None, None)
    ref = []
    for i, t in enumerate(toks):
        xr = x[i][None, :]
        acc = np.zeros(cfg.d)
        for j, e in enumerate(idx[t]):
            acc += float(w[t, j]) * O.expert_ffn(xr, *W[int(e)])[0]
        if sh[0] is not None:
            acc += O.shared_expert(xr, *sh)[0]
        ref.append(acc)
    ref = np.stack(ref)
    rel = assert_close(out, ref, TOL_OUT[cfg.dtype], "sampled tokens")
    print(f"[full-size] {cfg.name}: sampled out max|d|/max|ref| = {rel:.2e}")
