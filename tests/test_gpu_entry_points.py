"""Each C-ABI entry point on its own, against the oracle, on the edge cases of the
method: empty experts, exact multiples of block_m, everything on one expert,
T*k < block_m, a single token, duplicate experts within a token, out-of-range ids,
exact logit ties, many chunks, and the dropless notes' worked example."""
import json
import os

import ctypes

import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import moe_oracle as O

from gpu_util import TOL_LOGITS, TOL_STAGE, TOL_W_REL, assert_close, f64, i64

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_offsets(idx, E, bm, dtype="fp32"):
    """moe_build_offsets on a [T, k] id array; returns numpy outputs."""
    idx = np.asarray(idx, np.int32)
    T, k = idx.shape
    s = B.make_shape(T=T, d=8, E=E, k=k, d_e=8, block_m=bm, dtype=dtype)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    M = T * k
    t = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.reshape(-1).copy()).to(DEV)
    counts, offs, pad, meta, nblk = t(E), t(E + 1), t(E + 1), t(mb * 3), t(1)
    pos, row_src, err = t(M), t(rows), t(1)
    ws = B.alloc_workspace(s)
    print(f"[offsets] T={T} k={k} E={E} bm={bm}", flush=True)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    torch.cuda.synchronize()
    nb = int(nblk.item())
    return dict(counts=i64(counts)[:E], offsets=i64(offs), padded=i64(pad), num_blocks=nb,
                meta=i64(meta)[:nb * 3].reshape(-1, 3), meta_tail=i64(meta)[nb * 3:],
                pos=i64(pos)[:M], row_src=i64(row_src)[:rows], err=int(err.item()))


def check_offsets(idx, E, bm, dtype="fp32"):
    g = run_offsets(idx, E, bm, dtype)
    idx = np.asarray(idx)
    c = O.expert_counts(idx, E)
    assert g["err"] == 0
    assert np.array_equal(g["counts"], c)
    assert np.array_equal(g["offsets"], O.group_offsets(c))
    assert np.array_equal(g["padded"], O.padded_offsets(c, bm))
    meta = O.block_metadata(c, bm)
    assert g["num_blocks"] == len(meta)
    assert np.array_equal(g["meta"], meta)
    assert np.all(g["meta_tail"] == -7), "entries past num_blocks must be left untouched"
    pos, row_src = O.permutation(idx, E, bm)
    assert np.array_equal(g["pos"], pos)
    assert np.array_equal(g["row_src"][:len(row_src)], row_src)
    assert np.all(g["row_src"][len(row_src):] == -1)
    return g


@pytest.mark.parametrize("name,idx,E,bm", [
    ("all-on-one-expert", np.full((300, 1), 5), 8, 128),
    ("exact-multiples", np.repeat(np.array([0] * 128 + [1] * 256 + [3] * 128), 1).reshape(-1, 1), 4, 128),
    ("empty-first-middle-last", np.array([[1, 2], [2, 1], [1, 1], [2, 2]] * 40), 4, 128),
    ("single-token", np.array([[3]]), 8, 128),
    ("single-token-all-experts", np.array([[3, 0, 2, 1]]), 4, 128),
    ("tk-below-block", np.array([[0, 1], [1, 0], [7, 7]]), 8, 128),
    ("block-1", np.random.default_rng(0).integers(0, 5, (97, 3)), 5, 1),
    ("block-7", np.random.default_rng(1).integers(0, 9, (97, 3)), 9, 7),
])
def test_offsets_edge_cases(name, idx, E, bm):
    check_offsets(idx, E, bm)


@pytest.mark.parametrize("T,k,E,bm", [(50, 8, 4, 128), (5000, 1, 16, 128), (64, 8, 1024, 128),
                                      (137500, 8, 64, 128), (4099, 6, 64, 32)])
def test_offsets_random_with_duplicates_and_many_chunks(T, k, E, bm):
    rng = np.random.default_rng(T + E)
    p = rng.dirichlet(np.full(E, 0.5))
    idx = rng.choice(E, size=(T, k), p=p)      # duplicates within a token allowed
    check_offsets(idx, E, bm, "bf16" if bm % 128 == 0 else "fp32")


def test_offsets_worked_example_on_device():
    """The dropless notes' per-card example, computed on the device: padded sizes
    21,760/15,104/18,048/10,880 (65,792 rows) and 514 blocks."""
    g = json.load(open(os.path.join(GOLDEN, "dropless_padding_worked_example.json")))
    rng = np.random.default_rng(2)
    ids = np.repeat(np.arange(4), g["counts"])
    rng.shuffle(ids)
    out = check_offsets(ids.reshape(8192, 8), 4, 128, "bf16")
    assert list(np.diff(out["padded"])) == g["padded_sizes"]
    assert list(out["offsets"]) == g["group_offsets"]
    assert out["num_blocks"] == g["blocks_total_derived"]


def test_offsets_out_of_range_ids_set_the_flag():
    idx = np.array([[0, 1], [9, 2], [-1, 1], [2, 2]])
    g = run_offsets(idx, 4, 128)
    assert g["err"] == 1
    flat = idx.reshape(-1)
    bad = (flat < 0) | (flat >= 4)
    assert np.all(g["pos"][bad] == -1)
    assert np.array_equal(g["counts"], O.expert_counts(flat[~bad], 4))
    # the valid assignments still form a correct stable permutation
    P = g["padded"]
    for e in range(4):
        rows = sorted(g["pos"][(flat == e)])
        assert rows == list(range(P[e], P[e] + int((flat == e).sum())))


# ---------------------------------------------------------------------------
# moe_route on its own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,E,k,ng,tg,renorm,dtype", [
    (200, 512, 8, 4, 0, 0, False, "bf16"),
    (64, 1024, 256, 8, 8, 4, False, "bf16"),
    (33, 520, 64, 6, 0, 0, True, "bf16"),
    (16, 256, 1024, 8, 16, 2, True, "bf16"),
    (50, 128, 8, 2, 0, 0, True, "fp32"),
    (100, 384, 4, 3, 0, 0, False, "bf16"),       # 8 lanes per token, 4 idle
    (130, 256, 16, 4, 4, 2, True, "bf16"),       # 16 lanes per token, group limit
    (77, 640, 20, 5, 0, 0, False, "bf16"),       # 32 lanes per token
    (4500, 256, 96, 6, 0, 0, False, "bf16"),     # many token blocks: all experts per block
    (4100, 264, 8, 2, 0, 0, True, "bf16"),       # many token blocks, K tail in a window
    # the fused router (one block per 16 / 32 / 64 tokens, whole K, selection in the
    # block): every tile configuration, token tails, E not a multiple of 16, group limits
    (4096, 512, 8, 2, 0, 0, False, "bf16"),
    (5000, 768, 32, 4, 0, 0, False, "bf16"),
    (4104, 1024, 64, 6, 0, 0, True, "bf16"),
    (8192, 1024, 64, 6, 0, 0, True, "bf16"),
    (9000, 384, 24, 3, 0, 0, False, "bf16"),
    (8200, 512, 16, 4, 4, 2, True, "bf16"),
    (16384, 256, 16, 4, 4, 2, True, "bf16"),
    (16390, 256, 40, 8, 8, 4, False, "bf16"),
    (16400, 384, 32, 5, 0, 0, True, "bf16"),
])
def test_route_standalone(T, d, E, k, ng, tg, renorm, dtype):
    g = torch.Generator(device=DEV)
    g.manual_seed(T * 31 + E)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    wg = (torch.randn((d, E), generator=g, device=DEV) / d ** 0.5).to(dt)
    bias = torch.randn(E, generator=g, device=DEV) * 0.3
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=8, block_m=128 if dtype == "bf16" else 1,
                     dtype=dtype, n_groups=ng, topk_groups=tg, renormalize=renorm)
    logits = torch.empty((T, E), device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), device=DEV)
    ws = B.alloc_workspace(s)
    B.moe_route(s, x, wg, bias, logits, idx, w, ws)
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    B.moe_route(s, x, wg, bias, None, idx2, w2, ws)          # logits not stored
    torch.cuda.synchronize()
    ref = O.router_logits(f64(x), f64(wg), f64(bias))
    assert_close(f64(logits), ref, TOL_LOGITS[dtype], "logits")
    dec = logits.cpu().numpy()
    ridx = O.topk_by_repeated_max(dec, k, O.eligible_experts(dec, ng, tg))
    assert np.array_equal(i64(idx), ridx)
    np.testing.assert_allclose(f64(w), O.gate_weights(dec, ridx, renorm), rtol=TOL_W_REL, atol=0)
    assert torch.equal(idx, idx2) and torch.equal(w, w2)


@pytest.mark.parametrize("T", [64, 4096])
def test_route_exact_ties_go_to_the_lower_id(T):
    """Duplicated router columns give bitwise-equal logits; the lower id must win (the
    split-K router with its selection kernel, and the fused router)."""
    d, E, k = 256, 16, 4
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    x = torch.randn((T, d), generator=g, device=DEV).to(torch.bfloat16)
    wg = (torch.randn((d, E), generator=g, device=DEV) / 16).to(torch.bfloat16)
    wg[:, 9] = wg[:, 2]
    wg[:, 13] = wg[:, 2]
    wg[:, 7] = wg[:, 11]
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=8, block_m=128)
    logits = torch.empty((T, E), device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), device=DEV)
    B.moe_route(s, x, wg, None, logits, idx, w, B.alloc_workspace(s))
    torch.cuda.synchronize()
    L = logits.cpu().numpy()
    assert np.array_equal(L[:, 9], L[:, 2]) and np.array_equal(L[:, 7], L[:, 11])
    assert np.array_equal(i64(idx), O.topk_by_repeated_max(L, k))
    # whenever both members of a tied pair are chosen, the lower id comes first
    for row in i64(idx):
        r = list(row)
        if 2 in r and 9 in r:
            assert r.index(2) < r.index(9)
        if 7 in r and 11 in r:
            assert r.index(7) < r.index(11)


# ---------------------------------------------------------------------------
# permute -> grouped GEMM x2 -> combine, each entry point called on its own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,E,k,d_e,bm,dtype,mode", [
    (200, 512, 8, 2, 256, 128, "bf16", "random"),
    (96, 264, 6, 3, 136, 128, "bf16", "one-row-per-block"),
    (512, 256, 4, 1, 128, 128, "bf16", "full-blocks"),
    (70, 64, 5, 2, 48, 16, "fp32", "random"),
    (40, 256, 4, 70, 128, 128, "bf16", "random"),      # k > 64: slots handed out in two rounds
    (3, 128, 2, 5, 64, 128, "bf16", "random"),         # k not a multiple of the slot batch
    (9, 8200, 3, 2, 64, 128, "bf16", "random"),        # row of 1025 vectors: partial chunks
    (1100, 256, 3, 1, 128, 128, "bf16", "random"),     # 256-row tiles, odd block counts
])
def test_stage_entry_points(T, d, E, k, d_e, bm, dtype, mode):
    rng = np.random.default_rng(T + d)
    if mode == "random":
        idx = rng.integers(0, E, size=(T, k))
    elif mode == "one-row-per-block":
        # each expert gets few rows: blocks with valid_m of 1..3
        idx = np.zeros((T, k), np.int64)
        idx[:] = rng.integers(0, E, size=(T, k))
        idx[:E, 0] = np.arange(E)
        idx[E:, :] = 0
    else:
        idx = np.repeat(np.arange(E), T // E)[rng.permutation(T)].reshape(T, k)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    sh = (torch.randn((T, d), generator=g, device=DEV)).to(dt)
    tw = torch.rand((T, k), generator=g, device=DEV)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=bm, dtype=dtype)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    M = T * k
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(M), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    x_perm = torch.empty((rows, d), dtype=dt, device=DEV)
    act = torch.empty((rows, d_e), dtype=dt, device=DEV)
    y = torch.empty((rows, d), dtype=dt, device=DEV)
    out = torch.empty((T, d), dtype=dt, device=DEV)
    out_ns = torch.empty((T, d), dtype=dt, device=DEV)
    B.moe_permute(s, x, pos, x_perm)
    B.moe_grouped_gemm(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, w1, w3, meta, nblk, mb, act)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act, w2, None, meta, nblk, mb, y)
    B.moe_combine(s, y, pos, tw, sh, out)
    B.moe_combine(s, y, pos, tw, None, out_ns)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_pos, ref_src = O.permutation(idx, E, bm)
    assert np.array_equal(i64(pos), ref_pos)
    c = O.expert_counts(idx, E)
    xh = f64(x)
    xp_ref = O.permute(xh, ref_pos, k, len(ref_src))
    valid = np.nonzero(ref_src >= 0)[0]
    assert np.array_equal(f64(x_perm)[valid], xp_ref[valid])
    act_ref, _ = O.grouped_ffn(xp_ref, c, bm, f64(w1), f64(w3), f64(w2))
    assert_close(f64(act)[valid], act_ref[valid], TOL_STAGE[dtype], "act")
    _, y_ref = O.grouped_ffn(np.zeros_like(xp_ref), c, bm, f64(w1), f64(w3), f64(w2))
    act_dev = f64(act)
    P = O.padded_offsets(c, bm)
    for e in range(E):
        lo, hi = P[e], P[e] + c[e]
        y_ref[lo:hi] = act_dev[lo:hi] @ f64(w2)[e]
    assert_close(f64(y)[valid], y_ref[valid], TOL_STAGE[dtype], "y")
    y_dev = f64(y)
    out_ref = O.combine(y_dev, ref_pos, f64(tw), k, f64(sh))
    assert_close(f64(out), out_ref, TOL_STAGE[dtype], "out")
    assert_close(f64(out_ns), O.combine(y_dev, ref_pos, f64(tw), k), TOL_STAGE[dtype], "out")


@pytest.mark.parametrize("T,d,d_e,dtype", [(300, 256, 136, "bf16"), (129, 512, 256, "bf16"),
                                           (1, 256, 128, "bf16"), (77, 96, 40, "fp32")])
def test_grouped_gemm_dense_mode_is_the_shared_expert(T, d, d_e, dtype):
    """Dense mode (no block table): all T rows through one expert, as the shared expert
    of the layer; rows past T are neither read nor written."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    bm = 128 if dtype == "bf16" else 32
    g = torch.Generator(device=DEV)
    g.manual_seed(T + d_e)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=1, k=1, d_e=d_e, block_m=bm, dtype=dtype)
    act = torch.full((T + 1, d_e), 7.0, dtype=dt, device=DEV)
    y = torch.full((T + 1, d), 7.0, dtype=dt, device=DEV)
    B.moe_grouped_gemm(s, B.MOE_OP_GATEUP_SWIGLU, x, w1, w3, None, None, 0, act)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act, w2, None, None, None, 0, y)
    torch.cuda.synchronize()
    assert_close(f64(act)[:T], O.swiglu_act(f64(x), f64(w1), f64(w3)), TOL_STAGE[dtype], "act")
    assert_close(f64(y)[:T], f64(act)[:T] @ f64(w2), TOL_STAGE[dtype], "y")
    assert bool((act[T] == 7.0).all()) and bool((y[T] == 7.0).all())


@pytest.mark.parametrize("T,d,E,k,d_e,d_es,dtype", [
    (200, 512, 8, 2, 256, 256, "bf16"),      # one launch for both halves
    (64, 256, 16, 4, 128, 128, "bf16"),      # decode-like: few rows per expert
    (150, 512, 4, 2, 256, 128, "bf16"),      # d_e_shared != d_e: two launches
    (90, 264, 6, 3, 136, 136, "bf16"),       # K % 32 != 0 for down: register-staged kernel
    (70, 64, 5, 2, 48, 32, "fp32"),
])
def test_grouped_gemm_shared_matches_separate_calls(T, d, E, k, d_e, d_es, dtype):
    """moe_grouped_gemm_shared = moe_grouped_gemm on the block table + its dense mode on
    the shared expert, bit for bit, and the shared half matches the oracle."""
    rng = np.random.default_rng(T + d_es)
    idx = rng.integers(0, E, size=(T, k))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    bm = 128 if dtype == "bf16" else 16
    g = torch.Generator(device=DEV)
    g.manual_seed(17 + T)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    ws1 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
    ws3 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
    ws2 = (torch.randn((d_es, d), generator=g, device=DEV) / d_es ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=bm, dtype=dtype, d_e_shared=d_es)
    s_sh = B.make_shape(T=T, d=d, E=1, k=1, d_e=d_es, block_m=bm, dtype=dtype)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    x_perm = torch.empty((rows, d), dtype=dt, device=DEV)
    B.moe_permute(s, x, pos, x_perm)
    e = lambda *sh: torch.empty(sh, dtype=dt, device=DEV)
    act, y, sact, sout = e(rows, d_e), e(rows, d), e(T, d_es), e(T, d)
    act2, y2, sact2, sout2 = e(rows, d_e), e(rows, d), e(T, d_es), e(T, d)
    B.moe_grouped_gemm_shared(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, w1, w3, meta, nblk, mb, act,
                              x, ws1, ws3, sact)
    B.moe_grouped_gemm_shared(s, B.MOE_OP_DOWN, act, w2, None, meta, nblk, mb, y,
                              sact, ws2, None, sout)
    B.moe_grouped_gemm(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, w1, w3, meta, nblk, mb, act2)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act2, w2, None, meta, nblk, mb, y2)
    B.moe_grouped_gemm(s_sh, B.MOE_OP_GATEUP_SWIGLU, x, ws1, ws3, None, None, 0, sact2)
    B.moe_grouped_gemm(s_sh, B.MOE_OP_DOWN, sact2, ws2, None, None, None, 0, sout2)
    torch.cuda.synchronize()
    valid = torch.from_numpy(np.nonzero(O.permutation(idx, E, bm)[1] >= 0)[0]).to(DEV)
    bits = torch.int16 if dtype == "bf16" else torch.int32
    for a, b in ((act[valid], act2[valid]), (y[valid], y2[valid]), (sact, sact2), (sout, sout2)):
        assert torch.equal(a.view(bits), b.view(bits))
    assert_close(f64(sact), O.swiglu_act(f64(x), f64(ws1), f64(ws3)), TOL_STAGE[dtype], "shared act")
    assert_close(f64(sout), f64(sact) @ f64(ws2), TOL_STAGE[dtype], "shared out")


@pytest.mark.parametrize("tile", ["128", "384"])
@pytest.mark.parametrize("T,d,E,k,d_e,d_es", [
    (200, 512, 8, 2, 256, 256),      # shared expert in the same launch
    (64, 256, 16, 4, 128, 128),      # decode-like: few rows per expert
    (150, 512, 4, 2, 256, 0),        # no shared expert
    (1100, 256, 3, 1, 200, 72),      # column tails; shared expert in launches of its own
    (900, 1024, 4, 8, 128, 0),       # duplicate experts within a token, many full groups
])
def test_grouped_gemm_gather_is_permute_then_gemm(tile, T, d, E, k, d_e, d_es, monkeypatch):
    """moe_grouped_gemm_gather = moe_permute then moe_grouped_gemm(_shared) gate/up, bit
    for bit, on both tile heights; it never writes past the valid rows."""
    monkeypatch.setenv("MOE_GG_TILE_ROWS", tile)
    rng = np.random.default_rng(T + d + k)
    idx = rng.integers(0, E, size=(T, k))
    dt = torch.bfloat16
    g = torch.Generator(device=DEV)
    g.manual_seed(5 + T)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16", d_e_shared=d_es)
    assert B.gather_supported(s)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    x_perm = torch.empty((rows, d), dtype=dt, device=DEV)
    B.moe_permute(s, x, pos, x_perm)
    act = torch.full((rows, d_e), 3.0, dtype=dt, device=DEV)
    act2 = torch.empty((rows, d_e), dtype=dt, device=DEV)
    if d_es:
        ws1 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
        ws3 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
        sact = torch.empty((T, d_es), dtype=dt, device=DEV)
        sact2 = torch.empty((T, d_es), dtype=dt, device=DEV)
        B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act, ws1, ws3, sact)
        B.moe_grouped_gemm_shared(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, w1, w3, meta, nblk, mb, act2,
                                  x, ws1, ws3, sact2)
    else:
        B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act)
        B.moe_grouped_gemm(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, w1, w3, meta, nblk, mb, act2)
    torch.cuda.synchronize()
    ref_pos, ref_src = O.permutation(idx, E, 128)
    valid = np.nonzero(ref_src >= 0)[0]
    dv = torch.from_numpy(valid).to(DEV)
    assert torch.equal(act[dv].view(torch.int16), act2[dv].view(torch.int16))
    pad_rows = torch.from_numpy(np.nonzero(ref_src < 0)[0]).to(DEV)
    assert bool((act[pad_rows] == 3.0).all())
    if d_es:
        assert torch.equal(sact.view(torch.int16), sact2.view(torch.int16))
    c = O.expert_counts(idx, E)
    xp_ref = O.permute(f64(x), ref_pos, k, len(ref_src))
    act_ref, _ = O.grouped_ffn(xp_ref, c, 128, f64(w1), f64(w3), np.zeros((E, d_e, d)))
    assert_close(f64(act)[valid], act_ref[valid], TOL_STAGE["bf16"], "act")


@pytest.mark.parametrize("cap", ["1", "3", "8", "24"])
def test_wide_tiles_with_a_capped_grid(cap, monkeypatch):
    """A persistent grid of 1, 3, 8 or 24 work groups: each walks more than 64 items of
    the 384-row kernel (its group list is rebuilt every 64 items); 8 and 24 (multiples
    of 8) take the XCD supertile order, 1 and 3 the plain one; gate/up (gathered) and
    down match the 128-row kernel bit for bit."""
    T, d, E, k, d_e = 900, 1024, 4, 8, 128
    rng = np.random.default_rng(3)
    idx = rng.integers(0, E, size=(T, k))
    dt = torch.bfloat16
    g = torch.Generator(device=DEV)
    g.manual_seed(23)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16")
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    e = lambda *sh: torch.empty(sh, dtype=dt, device=DEV)
    act, y, act2, y2 = e(rows, d_e), e(rows, d), e(rows, d_e), e(rows, d)
    monkeypatch.setenv("MOE_GG_TILE_ROWS", "384")
    monkeypatch.setenv("MOE_GG_GRID_CAP", cap)
    B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act, w2, None, meta, nblk, mb, y)
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_GG_TILE_ROWS", "128")
    monkeypatch.delenv("MOE_GG_GRID_CAP")
    B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act2)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act2, w2, None, meta, nblk, mb, y2)
    torch.cuda.synchronize()
    valid = torch.from_numpy(np.nonzero(O.permutation(idx, E, 128)[1] >= 0)[0]).to(DEV)
    # more than 64 down items per work group at cap 1 (the group list is rebuilt)
    groups = sum(-(-(-(-int(c) // 128)) // 3) for c in O.expert_counts(idx, E))
    assert cap != "1" or groups * (d // 256) > 64
    assert torch.equal(act[valid].view(torch.int16), act2[valid].view(torch.int16))
    assert torch.equal(y[valid].view(torch.int16), y2[valid].view(torch.int16))


@pytest.mark.parametrize("d,d_e,cap", [(32, 32, "8"), (64, 96, "8"), (96, 64, "24"),
                                       (160, 128, "8"), (224, 160, "0")])
def test_wide_tiles_short_k(d, d_e, cap, monkeypatch):
    """K of 1 to 7 slices (32 deep): the four-slot ring wraps within an item and
    between consecutive items of a work group, and the refill copies of the last slices
    re-copy the final slice.  The capped grids give each work group many items.  Gate/up
    (gathered) and down match the 128-row kernel bit for bit."""
    T, E, k = 4800, 3, 2          # ~25 blocks per expert: 9 groups each, one of 1 block
    rng = np.random.default_rng(d + d_e)
    idx = rng.integers(0, E, size=(T, k))
    dt = torch.bfloat16
    g = torch.Generator(device=DEV)
    g.manual_seed(d * 7 + d_e)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16")
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    e = lambda *sh: torch.full(sh, 3.0, dtype=dt, device=DEV)
    act, y, act2, y2 = e(rows, d_e), e(rows, d), e(rows, d_e), e(rows, d)
    print(f"[wide short K] d={d} d_e={d_e} cap={cap}", flush=True)
    monkeypatch.setenv("MOE_GG_TILE_ROWS", "384")
    if cap != "0":
        monkeypatch.setenv("MOE_GG_GRID_CAP", cap)
    B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act, w2, None, meta, nblk, mb, y)
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_GG_TILE_ROWS", "128")
    monkeypatch.delenv("MOE_GG_GRID_CAP", raising=False)
    B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act2)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act2, w2, None, meta, nblk, mb, y2)
    torch.cuda.synchronize()
    valid = torch.from_numpy(np.nonzero(O.permutation(idx, E, 128)[1] >= 0)[0]).to(DEV)
    assert torch.equal(act[valid].view(torch.int16), act2[valid].view(torch.int16))
    assert torch.equal(y[valid].view(torch.int16), y2[valid].view(torch.int16))
    c = O.expert_counts(idx, E)
    xp_ref = O.permute(f64(x), O.permutation(idx, E, 128)[0], k, rows)
    act_ref, _ = O.grouped_ffn(xp_ref, c, 128, f64(w1), f64(w3), np.zeros((E, d_e, d)))
    vn = valid.cpu().numpy()
    assert_close(f64(act)[vn], act_ref[vn], TOL_STAGE["bf16"], "act")


def _random_wide_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([32, 64, 96, 256, 544, 1024]))
        d_e = int(rng.choice([32, 96, 128, 200, 384]))
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(200, 3000))
        cap = str(rng.choice(["0", "0", "1", "5", "8", "37"]))
        cases.append((i, T, d, E, k, d_e, cap))
    return cases


@pytest.mark.parametrize("i,T,d,E,k,d_e,cap", _random_wide_cases())
def test_wide_tiles_random_shapes(i, T, d, E, k, d_e, cap, monkeypatch):
    """Seeded random shapes, routings and persistent-grid caps: the 384-row kernel
    (gathered gate/up, then down) matches the 128-row kernel bit for bit, whatever the
    group sizes, K, column tails, last-round split and item order."""
    rng = np.random.default_rng(1000 + i)
    # skewed routing, so that groups of one, two and three blocks all occur
    p = rng.dirichlet(np.full(E, 0.7))
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    dt = torch.bfloat16
    g = torch.Generator(device=DEV)
    g.manual_seed(77 + i)
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16")
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err,
                        B.alloc_workspace(s))
    e = lambda *sh: torch.full(sh, -5.0, dtype=dt, device=DEV)
    act, y, act2, y2 = e(rows, d_e), e(rows, d), e(rows, d_e), e(rows, d)
    print(f"[wide random {i}] T={T} d={d} E={E} k={k} d_e={d_e} cap={cap}", flush=True)
    monkeypatch.setenv("MOE_GG_TILE_ROWS", "384")
    if cap != "0":
        monkeypatch.setenv("MOE_GG_GRID_CAP", cap)
    B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act, w2, None, meta, nblk, mb, y)
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_GG_TILE_ROWS", "128")
    monkeypatch.delenv("MOE_GG_GRID_CAP", raising=False)
    B.moe_grouped_gemm_gather(s, x, row_src, w1, w3, meta, nblk, mb, act2)
    B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act2, w2, None, meta, nblk, mb, y2)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    src = O.permutation(idx, E, 128)[1]
    valid = torch.from_numpy(np.nonzero(src >= 0)[0]).to(DEV)
    assert torch.equal(act[valid].view(torch.int16), act2[valid].view(torch.int16))
    assert torch.equal(y[valid].view(torch.int16), y2[valid].view(torch.int16))
    # pad rows are never written
    padr = torch.from_numpy(np.nonzero(src < 0)[0]).to(DEV)
    if len(padr):
        assert torch.all(act[padr] == -5.0) and torch.all(y[padr] == -5.0)


def test_combine_skips_negative_positions():
    T, d, k = 8, 64, 2
    s = B.make_shape(T=T, d=d, E=4, k=k, d_e=64, block_m=128)
    y = torch.randn((B.moe_max_rows(s), d), device=DEV).to(torch.bfloat16)
    pos = torch.tensor([0, -1, 1, 2, -1, -1, 3, 4, 5, 6, 7, 8, 9, 10, -1, 11], dtype=torch.int32,
                       device=DEV)
    w = torch.rand((T, k), device=DEV)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    B.moe_combine(s, y, pos, w, None, out)
    torch.cuda.synchronize()
    yh, p, wh = f64(y), i64(pos).reshape(T, k), f64(w)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if p[t, j] >= 0:
                ref[t] += wh[t, j] * yh[p[t, j]]
    assert_close(f64(out), ref, TOL_STAGE["bf16"], "out")


@pytest.mark.parametrize("tile", ["128", "384"])
@pytest.mark.parametrize("op", ["gateup", "down"])
def test_negative_block_count_runs_no_routed_block(tile, op, monkeypatch):
    """A block count below zero in device memory (a caller's corrupt table) is read as
    zero: no routed row is written, and the shared expert's dense segment in the same
    launch is still computed, bitwise as with the real table."""
    monkeypatch.setenv("MOE_GG_TILE_ROWS", tile)
    T, d, E, k, d_e = 256, 256, 4, 2, 128
    rng = np.random.default_rng(41)
    idx = rng.integers(0, E, size=(T, k))
    dt = torch.bfloat16
    g = torch.Generator(device=DEV)
    g.manual_seed(41)
    rnd = lambda *sh: (torch.randn(sh, generator=g, device=DEV) / sh[-2] ** 0.5).to(dt)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16", d_e_shared=d_e)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err,
                        B.alloc_workspace(s))
    if op == "gateup":
        opc, K, N = B.MOE_OP_GATEUP_SWIGLU, d, d_e
        w0, w1 = rnd(E, d, d_e), rnd(E, d, d_e)
        s0, s1 = rnd(d, d_e), rnd(d, d_e)
    else:
        opc, K, N = B.MOE_OP_DOWN, d_e, d
        w0, w1, s0, s1 = rnd(E, d_e, d), None, rnd(d_e, d), None
    A = torch.randn((rows, K), generator=g, device=DEV).to(dt)
    A_sh = torch.randn((T, K), generator=g, device=DEV).to(dt)
    sentinel = torch.full((rows, N), -7.0, dtype=dt, device=DEV)
    C = sentinel.clone()
    C_sh, C_sh_ref = (torch.empty((T, N), dtype=dt, device=DEV) for _ in range(2))
    C_ref = torch.empty((rows, N), dtype=dt, device=DEV)
    B.moe_grouped_gemm_shared(s, opc, A, w0, w1, meta, nblk, mb, C_ref, A_sh, s0, s1, C_sh_ref)
    bad = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    B.moe_grouped_gemm_shared(s, opc, A, w0, w1, meta, bad, mb, C, A_sh, s0, s1, C_sh)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), sentinel.view(torch.int16))
    assert torch.equal(C_sh.view(torch.int16), C_sh_ref.view(torch.int16))
