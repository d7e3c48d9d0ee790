"""Parity at the full workload sizes for the layer's variants, through the C ABI (the
launches the benchmark times), against the oracle:

  * fp8 (e4m3) weights with per-block scales ([DG] §12) at the decode shape (E = 256,
    K = 7168, the weight-streaming kernels) and at the fusedmoe shape (experts
    averaging >= 256 rows, the prefill kernels).  The weights are seeded fp8 codes and
    scales (workloads.make_fp8_weights), the layer's own inputs; the oracle evaluates
    the layer with the exactly dequantised weights (oracle/fp8_oracle.py);
  * unpadded segments ([DG] §11) at the 65,536-row expert-parallel share (515 table
    entries, boundary tiles executed once per expert).

As in test_gpu_full_size.py the oracle cannot run the whole layer in seconds at these
sizes, so:
  * routing (when the layer routes), counts, offsets, the block table, pos and row_src
    are checked in full, integers bit-exactly;
  * act and y on sampled rows and the output on sampled tokens, each recomputed by the
    oracle on its own, expert by expert;
  * every output element is finite.
Tolerances: an fp8-weight GEMM stage 1e-2 * max|ref| (the bf16 stage bound plus one
bf16 rounding of each dequantised weight, see test_gpu_fp8.py), a bf16 stage
5e-3 * max|ref|, the layer output 2e-2 * max|ref|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import fp8_oracle as F
from oracle import moe_oracle as O
from workloads import get_config, make_fp8_weights, make_inputs

from gpu_util import (TOL_LOGITS, TOL_OUT, TOL_STAGE, TOL_W_REL, LayerRun, assert_close, f64,
                      i64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_STAGE_FP8 = 1e-2
# sampled tokens per workload (plus the first and the last); decode's tokens each touch
# 8 of 256 experts, and every touched expert is dequantised on the host
N_TOK = {"decode-256x2048": 4, "fusedmoe-8x2048": 14}


def _ints(ws, s, cfg):
    v = lambda n, shape: B.ws_view(ws, s, n, torch.int32, shape)
    mb, rows, M = B.moe_max_blocks(s), B.moe_max_rows(s), cfg.T * cfg.k
    nb = int(v("num_blocks", (1,)).item())
    return dict(counts=i64(v("counts", (cfg.E,))), offsets=i64(v("offsets", (cfg.E + 1,))),
                padded_offsets=i64(v("padded_offsets", (cfg.E + 1,))), num_blocks=nb,
                block_meta=i64(v("block_meta", (mb, 3)))[:nb], pos=i64(v("pos", (M,))),
                row_src=i64(v("row_src", (rows,))), err_flag=int(v("err_flag", (1,)).item()))


def _check_offsets(cfg, got, idx, unpadded=False):
    """Counts, offsets, the block table and the permutation, bit-exact."""
    assert got["err_flag"] == 0
    c = O.expert_counts(idx, cfg.E)
    assert np.array_equal(got["counts"], c)
    assert np.array_equal(got["offsets"], O.group_offsets(c))
    if unpadded:
        assert np.array_equal(got["padded_offsets"], O.group_offsets(c))
        tab = np.asarray(O.unpadded_tile_table(c, cfg.block_m)).reshape(-1, 3)
        pos, row_src = O.permutation_unpadded(idx, cfg.E)
        n = cfg.T * cfg.k
    else:
        P = O.padded_offsets(c, cfg.block_m)
        assert np.array_equal(got["padded_offsets"], P)
        tab = np.asarray(O.block_metadata(c, cfg.block_m)).reshape(-1, 3)
        pos, row_src = O.permutation(idx, cfg.E, cfg.block_m)
        n = int(P[-1])
    assert got["num_blocks"] == len(tab)
    assert np.array_equal(got["block_meta"], tab)
    assert np.array_equal(got["pos"], pos)
    assert np.array_equal(got["row_src"][:n], row_src[:n])
    assert np.all(got["row_src"][n:] == -1)
    return c


def _sample_tokens(cfg, n, seed):
    rng = np.random.default_rng(seed)
    return sorted({0, cfg.T - 1} | set(int(t) for t in rng.choice(cfg.T, size=min(n, cfg.T),
                                                                     replace=False)))


def _check_tokens_and_rows(cfg, x, out, act, y, toks, idx, w, pos, expert_weights, shared,
                           tol_stage, what):
    """For every sampled token t: its k rows of act and y (rows pos[t, j]) at the stage
    tolerance (act from x[t], y from the device's own act row), and out[t] from the
    oracle's per-token definition (slots summed in ascending j, then the shared expert)
    at the layer tolerance.  expert_weights(e) gives expert e's fp64 (W1, W3, W2); the
    experts are visited one at a time, so only one expert's weights are held."""
    k = cfg.k
    tt = torch.tensor(toks, device=DEV)
    xs = f64(x[tt])
    got_out = f64(out[tt])
    rows = np.array([[pos[t * k + j] for j in range(k)] for t in toks], np.int64)
    assert np.all(rows >= 0)
    rt = torch.from_numpy(rows.reshape(-1)).to(DEV)
    got_act = f64(act[rt]).reshape(len(toks), k, -1)
    got_y = f64(y[rt]).reshape(len(toks), k, -1)
    ref_act = np.zeros_like(got_act)
    ref_y = np.zeros_like(got_y)
    ffn = {}
    by_expert = {}
    for i, t in enumerate(toks):
        for j in range(k):
            by_expert.setdefault(int(idx[t, j]), []).append((i, j))
    for e in sorted(by_expert):
        W1, W3, W2 = expert_weights(e)
        for i, j in by_expert[e]:
            xr = xs[i][None, :]
            ref_act[i, j] = O.swiglu_act(xr, W1, W3)[0]
            ref_y[i, j] = got_act[i, j][None, :] @ W2
            ffn[(i, j)] = O.expert_ffn(xr, W1, W3, W2)[0]
        del W1, W3, W2
    ref_out = np.zeros_like(got_out)
    for i, t in enumerate(toks):
        for j in range(k):
            ref_out[i] += float(w[t, j]) * ffn[(i, j)]
    if shared is not None:
        ref_out += O.shared_expert(xs, *shared)
    flat = lambda a: a.reshape(-1, a.shape[-1])
    assert_close(flat(got_act), flat(ref_act), tol_stage, f"{what}: act rows")
    assert_close(flat(got_y), flat(ref_y), tol_stage, f"{what}: y rows")
    rel = assert_close(got_out, ref_out, TOL_OUT["bf16"], f"{what}: sampled tokens")
    print(f"[full-size] {what}: sampled out max|d|/max|ref| = {rel:.2e}", flush=True)


# ----------------------------------------------------------------------------
# fp8 weights at full size
# ----------------------------------------------------------------------------
FP8_FULL = ["decode-256x2048", "fusedmoe-8x2048"]


@pytest.fixture(scope="module", params=FP8_FULL)
def fp8_full(request):
    cfg = get_config(request.param)
    print(f"[full-size fp8] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_e={cfg.d_e}",
          flush=True)
    inp = make_inputs(cfg, DEV, expert_weights=False)
    w = make_fp8_weights(cfg, DEV)
    s = B.shape_of_config(cfg)
    assert B.fp8_supported(s)
    ws = B.alloc_workspace(s, fp8=True)
    out = torch.full((cfg.T, cfg.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, w.q1, w.s1, w.q3, w.s3, w.q2, w.s2,
                        w.qs1, w.ss1, w.qs3, w.ss3, w.qs2, w.ss2, None, None, out, ws)
    torch.cuda.synchronize()
    yield cfg, inp, w, s, ws, out
    del ws, out, w, inp
    torch.cuda.empty_cache()


def _dequantised(q, sc):
    """fp64 weights of one fp8 matrix [K, N] with its scales [kb, nb] (device tensors)."""
    return F.dequantize(q.cpu().numpy()[None], sc.cpu().numpy()[None])[0]


def test_fp8_full_size_routing_and_offsets(fp8_full):
    cfg, inp, w, s, ws, out = fp8_full
    x, wg = f64(inp.x), f64(inp.w_gate)
    bias = None if inp.bias is None else f64(inp.bias)
    dev_logits = B.ws_view(ws, s, "logits", torch.float32, (cfg.T, cfg.E)).cpu().numpy()
    assert_close(dev_logits, O.router_logits(x, wg, bias), TOL_LOGITS["bf16"], "logits")
    _, idx_ref, w_ref = O.route(x, wg, bias, cfg.k, cfg.n_groups, cfg.topk_groups,
                                cfg.renormalize, decision_logits=dev_logits)
    idx = i64(B.ws_view(ws, s, "topk_idx", torch.int32, (cfg.T, cfg.k)))
    wd = f64(B.ws_view(ws, s, "topk_w", torch.float32, (cfg.T, cfg.k)))
    assert np.array_equal(idx, idx_ref)
    assert np.all(np.abs(wd - w_ref) <= TOL_W_REL * np.abs(w_ref) + 1e-30)
    _check_offsets(cfg, _ints(ws, s, cfg), idx)


def test_fp8_full_size_sampled_tokens(fp8_full):
    cfg, inp, w, s, ws, out = fp8_full
    assert torch.isfinite(out.float()).all()
    idx = i64(B.ws_view(ws, s, "topk_idx", torch.int32, (cfg.T, cfg.k)))
    tw = f64(B.ws_view(ws, s, "topk_w", torch.float32, (cfg.T, cfg.k)))
    pos = i64(B.ws_view(ws, s, "pos", torch.int32, (cfg.T * cfg.k,)))
    rows = B.moe_max_rows(s)
    act = B.ws_view(ws, s, "act", torch.bfloat16, (rows, cfg.d_e))
    y = B.ws_view(ws, s, "y", torch.bfloat16, (rows, cfg.d))
    toks = _sample_tokens(cfg, N_TOK[cfg.name], cfg.seed + 13)
    weights = lambda e: (_dequantised(w.q1[e], w.s1[e]), _dequantised(w.q3[e], w.s3[e]),
                         _dequantised(w.q2[e], w.s2[e]))
    shared = None
    if cfg.d_e_shared:
        shared = (_dequantised(w.qs1, w.ss1), _dequantised(w.qs3, w.ss3),
                  _dequantised(w.qs2, w.ss2))
    _check_tokens_and_rows(cfg, inp.x, out, act, y, toks, idx, tw, pos, weights, shared,
                           TOL_STAGE_FP8, f"{cfg.name} fp8")


def test_fp8_full_size_minimal_workspace_gives_the_same_output(fp8_full):
    """With a workspace of moe_workspace_bytes only, the fp8 layer dequantises in registers
    (the wide kernel where experts average >= 256 rows) instead of into the workspace: the
    same bf16 weights, tiles and order of the sums, so the output is bitwise the same.
    Where experts average at most 64 rows (decode) the full workspace also holds the
    streaming kernel's scratch, with which the last round of its grid is split along K:
    only the order of fp32 partial sums of those items differs, so the outputs agree to
    bf16 rounding."""
    cfg, inp, w, s, ws, out = fp8_full
    wsm = torch.empty(B.moe_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    out2 = torch.empty_like(out)
    B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, w.q1, w.s1, w.q3, w.s3, w.q2, w.s2,
                        w.qs1, w.ss1, w.qs3, w.ss3, w.qs2, w.ss2, None, None, out2, wsm)
    torch.cuda.synchronize()
    M = cfg.T * cfg.k
    if M <= 64 * min(cfg.E, M):
        a, b = out2.double(), out.double()
        assert torch.isfinite(a).all()
        assert (a - b).abs().max().item() <= 2 ** -6 * b.abs().max().item()
    else:
        assert torch.equal(out2.view(torch.int16), out.view(torch.int16))


# ----------------------------------------------------------------------------
# Unpadded segments at full size
# ----------------------------------------------------------------------------
@pytest.fixture(scope="module")
def unpadded_full():
    cfg = get_config("ep-share-4x2048")
    print(f"[full-size unpadded] {cfg.name}", flush=True)
    inp = make_inputs(cfg, DEV)
    run_u = LayerRun(cfg.scaled(name=cfg.name + "-unpadded", unpadded=True), inp)
    run_p = LayerRun(cfg, inp)
    yield cfg, inp, run_u, run_p
    del run_u, run_p, inp
    torch.cuda.empty_cache()


def test_unpadded_full_size_offsets(unpadded_full):
    cfg, inp, run_u, _ = unpadded_full
    got = run_u.ints()
    assert got["num_blocks"] == 515
    _check_offsets(run_u.cfg, got, i64(inp.topk_idx), unpadded=True)


def test_unpadded_full_size_equals_padded(unpadded_full):
    """Each row's arithmetic is the same in both layouts: the outputs are bitwise equal."""
    _, _, run_u, run_p = unpadded_full
    assert torch.equal(run_u.out.view(torch.int16), run_p.out.view(torch.int16))


def test_unpadded_full_size_sampled_tokens(unpadded_full):
    cfg, inp, run_u, _ = unpadded_full
    assert torch.isfinite(run_u.out.float()).all()
    toks = _sample_tokens(cfg, 14, cfg.seed + 17)
    pos = run_u.ints()["pos"]

    def weights(e):
        return f64(inp.w1[e]), f64(inp.w3[e]), f64(inp.w2[e])

    _check_tokens_and_rows(cfg, inp.x, run_u.out, run_u.act(), run_u.y(), toks, i64(inp.topk_idx),
                           f64(inp.topk_w), pos, weights, None, TOL_STAGE["bf16"],
                           f"{cfg.name} unpadded")
