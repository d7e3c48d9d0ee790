"""Backward parity at full workload sizes, through moe_layer_bwd (the call the benchmark's
backward times), against the backward oracle's definitions on sampled outputs.

The oracle cannot run the whole backward at these sizes, so each sampled output is
recomputed from the device's own upstream values (the stage it comes out of is then the
only arithmetic compared), at the stage tolerances of test_gpu_backward:
  * rows of dy, dact, dg | du and dx_perm (first and last row of every expert segment
    plus a seeded random set): 5e-3 * max|ref| over the sample;
  * dtopk_w and dx on sampled tokens: dx is the sum of three stages, each stored in bf16
    (the shared expert's dx, the router's dx on top of it, the sum over the token's k
    rows), so each is checked against the device's own inputs to it;
  * sampled entries of dW2, dW1, dW3 (each a sum over the expert's rows, up to 21,733
    of them), every dbias entry and sampled dW_g entries: 1e-4 * max|ref| over the
    sample (fp32 sums of exact bf16 products).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import moe_backward_oracle as BW
from workloads.configs import get_config
from workloads.gen import make_inputs

from gpu_util import TOL_STAGE, LayerRun, assert_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
FULL = ["ep-share-4x2048", "fusedmoe-8x2048"]
N_ROWS = 24
N_TOK = 16
N_W = 48
TOL_W = 1e-4


@pytest.fixture(scope="module", params=FULL)
def full(request):
    cfg = get_config(request.param)
    print(f"[full-size bwd] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_e={cfg.d_e}",
          flush=True)
    inp = make_inputs(cfg, DEV)
    run = LayerRun(cfg, inp)
    s = run.shape
    g = torch.Generator(device=DEV)
    g.manual_seed(29)
    dout = torch.randn((cfg.T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    d, E, de, ds = cfg.d, cfg.E, cfg.d_e, cfg.d_e_shared
    f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=DEV)
    routed = run.routed
    gr = dict(dx=torch.empty((cfg.T, d), dtype=torch.bfloat16, device=DEV), dw1=f(E, d, de),
              dw3=f(E, d, de), dw2=f(E, de, d), dws1=f(d, ds) if ds else None,
              dws3=f(d, ds) if ds else None, dws2=f(ds, d) if ds else None,
              dw_gate=None if routed else f(d, E), dbias=None if routed else f(E),
              dtopk_w=f(cfg.T, cfg.k))
    bws = B.alloc_bwd_workspace(s)
    B.moe_layer_bwd(s, inp.x, None if routed else inp.w_gate, inp.w1, inp.w3, inp.w2, inp.ws1,
                    inp.ws3, inp.ws2, inp.topk_idx if routed else None,
                    inp.topk_w if routed else None, dout, run.ws, gr["dx"], gr["dw1"], gr["dw3"],
                    gr["dw2"], gr["dws1"], gr["dws3"], gr["dws2"], gr["dw_gate"], gr["dbias"],
                    gr["dtopk_w"], bws)
    torch.cuda.synchronize()
    yield cfg, inp, run, dout, gr, bws
    del run, inp, gr, bws
    torch.cuda.empty_cache()


def _bview(run, bws, name, dtype, shape):
    return B.bwd_ws_view(bws, run.shape, name, dtype, shape)


def _segments(run):
    ints = run.ints()
    return ints["counts"], ints["padded_offsets"], ints["pos"].reshape(run.cfg.T, run.cfg.k)


def _sample_rows(counts, P, rng):
    rows, experts = [], []
    for e, c in enumerate(counts):
        if c:
            rows += [int(P[e]), int(P[e] + c - 1)]
            experts += [e, e]
    live = np.concatenate([np.arange(P[e], P[e] + c) for e, c in enumerate(counts) if c])
    pick = rng.choice(live, size=N_ROWS, replace=False)
    for r in pick:
        e = int(np.searchsorted(P, r, side="right") - 1)
        rows.append(int(r))
        experts.append(e)
    return np.asarray(rows), np.asarray(experts)


def _routing(run, inp):
    if run.routed:
        return inp.topk_idx.cpu().numpy().astype(np.int64), f64(inp.topk_w)
    i, w = run.topk()
    return i.cpu().numpy().astype(np.int64), f64(w)


def test_full_size_bwd_rows(full):
    """dy, dact, dg | du and dx_perm rows, each from the device's upstream row."""
    cfg, inp, run, dout, gr, bws = full
    rows_n = B.moe_max_rows(run.shape)
    d, de = cfg.d, cfg.d_e
    counts, P, pos = _segments(run)
    rng = np.random.default_rng(3)
    rows, experts = _sample_rows(counts, P, rng)
    dr = torch.from_numpy(rows).to(DEV)
    take = lambda name, width: f64(_bview(run, bws, name, torch.bfloat16, (rows_n, width))[dr])
    dy, dact, dgu = take("dy", d), take("dact", de), take("dgu", 2 * de)
    xp, dxp = take("x_perm", d), take("dx_perm", d)
    y = f64(run.y()[dr])
    # dy row r = w[t, j] dout[t] for the slot (t, j) with pos = r
    row_src = run.ints()["row_src"][rows]
    idx, w = _routing(run, inp)
    t, j = row_src // cfg.k, row_src % cfg.k
    dout_h = f64(dout[torch.from_numpy(t).to(DEV)])
    assert_close(dy, w[t, j][:, None] * dout_h, TOL_STAGE["bf16"], "dy rows")
    assert np.array_equal(idx[t, j], experts)
    # x_perm row r = x[t]
    assert np.array_equal(xp, f64(inp.x[torch.from_numpy(t).to(DEV)]))
    dact_ref = np.zeros_like(dact)
    dg_ref, du_ref = np.zeros((len(rows), de)), np.zeros((len(rows), de))
    dxp_ref = np.zeros_like(dxp)
    for e in np.unique(experts):
        sel = experts == e
        w1, w3, w2 = f64(inp.w1[e]), f64(inp.w3[e]), f64(inp.w2[e])
        dact_ref[sel] = dy[sel] @ w2.T
        dg_ref[sel], du_ref[sel], _ = BW.swiglu_backward(xp[sel], w1, w3, dact[sel])
        dxp_ref[sel] = dgu[sel, :de] @ w1.T + dgu[sel, de:] @ w3.T
    assert_close(dact, dact_ref, TOL_STAGE["bf16"], "dact rows")
    assert_close(dgu[:, :de], dg_ref, TOL_STAGE["bf16"], "dg rows")
    assert_close(dgu[:, de:], du_ref, TOL_STAGE["bf16"], "du rows")
    assert_close(dxp, dxp_ref, TOL_STAGE["bf16"], "dx_perm rows")
    assert np.all(np.isfinite(y))


def test_full_size_bwd_tokens(full):
    """dtopk_w and dx on sampled tokens."""
    cfg, inp, run, dout, gr, bws = full
    rows_n = B.moe_max_rows(run.shape)
    d, ds = cfg.d, cfg.d_e_shared
    counts, P, pos = _segments(run)
    rng = np.random.default_rng(4)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, N_TOK, replace=False)]))
    dt = torch.from_numpy(toks).to(DEV)
    p = pos[toks]                                          # [n, k]
    y = f64(run.y()[torch.from_numpy(p.reshape(-1)).to(DEV)]).reshape(len(toks), cfg.k, d)
    dout_h = f64(dout[dt])
    dtw_ref = np.einsum("nd,nkd->nk", dout_h, y)
    assert_close(f64(gr["dtopk_w"][dt]), dtw_ref, TOL_W, "dtopk_w")
    dxp = f64(_bview(run, bws, "dx_perm", torch.bfloat16, (rows_n, d))[
        torch.from_numpy(p.reshape(-1)).to(DEV)]).reshape(len(toks), cfg.k, d)
    # each term of dx is stored in bf16 by its own stage: the shared expert's dx, the
    # router's dx on top of it, then the sum over the token's k rows; each is checked
    # against the device's own inputs to it
    extra = np.zeros((len(toks), d))
    if ds:
        sdgu = f64(_bview(run, bws, "shared_dgu", torch.bfloat16, (cfg.T, 2 * ds))[dt])
        sdx = f64(_bview(run, bws, "shared_dx", torch.bfloat16, (cfg.T, d))[dt])
        assert_close(sdx, sdgu[:, :ds] @ f64(inp.ws1).T + sdgu[:, ds:] @ f64(inp.ws3).T,
                     TOL_STAGE["bf16"], "shared dx tokens")
        extra = sdx
    if not run.routed:
        dl = f64(_bview(run, bws, "dlogits", torch.float32, (cfg.T, cfg.E))[dt])
        rdx = f64(_bview(run, bws, "router_dx", torch.bfloat16, (cfg.T, d))[dt])
        assert_close(rdx, extra + dl @ f64(inp.w_gate).T, TOL_STAGE["bf16"], "router dx tokens")
        extra = rdx
    assert_close(f64(gr["dx"][dt]), dxp.sum(axis=1) + extra, TOL_STAGE["bf16"], "dx tokens")


def test_full_size_bwd_weight_gradients(full):
    """Sampled entries of dW2, dW1, dW3 (sums over each expert's rows), dbias in full and
    sampled dW_g entries, from the device's upstream rows."""
    cfg, inp, run, dout, gr, bws = full
    rows_n = B.moe_max_rows(run.shape)
    d, de, E = cfg.d, cfg.d_e, cfg.E
    counts, P, _ = _segments(run)
    rng = np.random.default_rng(5)
    col = lambda t, c: t[:, c].double().cpu().numpy()
    dy = _bview(run, bws, "dy", torch.bfloat16, (rows_n, d))
    dgu = _bview(run, bws, "dgu", torch.bfloat16, (rows_n, 2 * de))
    xp = _bview(run, bws, "x_perm", torch.bfloat16, (rows_n, d))
    act = run.act()
    for name, X, D, C, nsplit, width_x, width_d in (
            ("dw2", act, dy, gr["dw2"], None, de, d),
            ("dw1", xp, dgu, gr["dw1"], 0, d, de),
            ("dw3", xp, dgu, gr["dw3"], de, d, de)):
        got, ref = [], []
        for _ in range(N_W):
            e = int(rng.integers(0, E))
            i, jj = int(rng.integers(0, width_x)), int(rng.integers(0, width_d))
            lo, hi = int(P[e]), int(P[e] + counts[e])
            jd = jj if nsplit is None else nsplit + jj
            ref.append(float(np.dot(col(X[lo:hi], i), col(D[lo:hi], jd))) if hi > lo else 0.0)
            got.append(float(C[e, i, jj].item()))
        assert_close(np.asarray(got), np.asarray(ref), TOL_W, name)
    if not run.routed:
        dl = _bview(run, bws, "dlogits", torch.float32, (cfg.T, E))
        assert_close(f64(gr["dbias"]), dl.double().sum(dim=0).cpu().numpy(), TOL_W, "dbias")
        got, ref = [], []
        for _ in range(N_W):
            c, e = int(rng.integers(0, d)), int(rng.integers(0, E))
            ref.append(float(np.dot(col(inp.x, c), col(dl, e))))
            got.append(float(gr["dw_gate"][c, e].item()))
        assert_close(np.asarray(got), np.asarray(ref), TOL_W, "dW_g")
