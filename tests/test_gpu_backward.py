"""Backward pass on the GPU, through the C ABI, against the backward oracle.

Stage by stage, each entry point is fed the device's own upstream values (so that only
its own arithmetic is compared), then the whole moe_layer_bwd against the oracle's
chain rule on the fp64 inputs.  Tolerances:
  * a bf16 output of one stage (dy, dact, dg | du, dx_perm, the router's dx): one bf16
    rounding (<= 2^-9 relative) plus fp32 accumulation, within TOL_STAGE = 5e-3 * max|ref|;
  * fp32 outputs whose products are exact in fp32 (weight gradients: bf16 x bf16;
    dtopk_w: bf16 x bf16) and are summed in fp32 over at most a few thousand terms:
    the sum's rounding is ~sqrt(n) 2^-24 relative, far inside 1e-4 * max|ref|;
  * dlogits: fp32 softmax (as the forward's weights, <= 4e-6 relative) and a k-term
    chain: 1e-5 * max|ref|;
  * the layer's gradients: every intermediate is rounded to bf16 once per stage (the
    forward's act and y, then dy, dact, dg | du, dx_perm), the same kind of chain as the
    forward output, held to the same bound 2e-2 * max|ref|.
"""
import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import moe_backward_oracle as BW
from oracle import moe_oracle as O
from workloads import get_config, make_inputs

from gpu_util import TOL_OUT, TOL_STAGE, LayerRun, assert_close, f64, host_inputs, i64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_WGRAD = 1e-4
TOL_DLOGITS = 1e-5
TOL_GRAD = TOL_OUT["bf16"]


def _seg(run):
    c = run.cfg
    ints = run.ints()
    return ints["counts"], ints["padded_offsets"], ints["pos"].reshape(c.T, c.k)


def _dout(cfg, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn((cfg.T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)


STAGE_CASES = [
    # a shared expert with the routed inner size; ragged expert counts
    ("fusedmoe-8x2048", dict(name="fusedmoe-bwd-s", T=300, d=512, d_e=256, d_e_shared=256)),
    # 4 zero-row experts, renormalised weights, shared expert absent
    ("zipf-skew-64x1408", dict(name="zipf-bwd-s", T=400, d=256, d_e=160)),
    # inner sizes above one 512-column tile, ragged in 256-column tiles
    ("zipf-skew-64x1408", dict(name="zipf-bwd-wide-n", T=200, d=256, E=8, k=2, d_e=640,
                               n_dead=2)),
    # group-limited routing, few rows per expert, shared expert of another size
    ("decode-256x2048", dict(name="decode-bwd-s", T=24, d=512, E=64, d_e=128, d_e_shared=192)),
]


@pytest.mark.parametrize("name,scale", STAGE_CASES)
def test_backward_stages_against_oracle(name, scale):
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    run = LayerRun(cfg, inp)
    s = run.shape
    assert B.backward_supported(s)
    T, d, E, k, de, ds = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_e, cfg.d_e_shared
    rows, mb = B.moe_max_rows(s), B.moe_max_blocks(s)
    counts, P, pos = _seg(run)
    h = host_inputs(inp)
    bf = torch.bfloat16
    e = lambda *sh: torch.empty(sh, dtype=bf, device=DEV)
    f = lambda *sh: torch.full(sh, float("nan"), dtype=torch.float32, device=DEV)
    idx, tw = run.topk()
    meta = run.view("block_meta", torch.int32, (mb, 3))
    nblk = run.view("num_blocks", torch.int32, (1,))
    dcounts = run.view("counts", torch.int32, (E,))
    dpad = run.view("padded_offsets", torch.int32, (E + 1,))
    dpos = run.view("pos", torch.int32, (T * k,))
    row_src = run.view("row_src", torch.int32, (rows,))
    dout = _dout(cfg, 7)

    def rows_of(ex):
        return slice(int(P[ex]), int(P[ex] + counts[ex]))

    valid = np.concatenate([np.arange(P[ex], P[ex] + counts[ex]) for ex in range(E)]).astype(np.int64)

    # combine backward on the forward's y
    dy, dtw = e(rows, d), f(T, k)
    B.moe_combine_bwd(s, dout, run.y(), dpos, tw, dy, dtw)
    torch.cuda.synchronize()
    y_dev, dout_h, w_dev = f64(run.y()), f64(dout), f64(tw)
    dy_ref, dw_ref = BW.combine_backward(dout_h, y_dev, pos, w_dev, k)
    assert_close(f64(dy)[valid], dy_ref[valid], TOL_STAGE["bf16"], "dy")
    assert_close(f64(dtw), dw_ref, TOL_WGRAD, "dtopk_w")

    # down: data gradient and weight gradient on the device's dy
    dact, dw2 = e(rows, de), f(E, de, d)
    B.moe_grouped_gemm_dgrad(s, B.MOE_OP_DOWN, dy, inp.w2, None, meta, nblk, mb, dact)
    B.moe_grouped_gemm_wgrad(s, B.MOE_OP_DOWN, run.act(), dy, dcounts, dpad, dw2, None)
    torch.cuda.synchronize()
    dy_h, act_h = f64(dy), f64(run.act())
    dact_ref = np.zeros((rows, de))
    dw2_ref = np.zeros((E, de, d))
    for ex in range(E):
        r = rows_of(ex)
        dact_ref[r] = dy_h[r] @ h["w2"][ex].T
        dw2_ref[ex] = act_h[r].T @ dy_h[r]
    assert_close(f64(dact)[valid], dact_ref[valid], TOL_STAGE["bf16"], "dact")
    assert_close(f64(dw2), dw2_ref, TOL_WGRAD, "dW2")
    # the same weight gradient through the work queue (largest expert first): bitwise
    sched = torch.empty(B.moe_grouped_gemm_wgrad_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    dw2_q = torch.full_like(dw2, float("nan"))
    B.moe_grouped_gemm_wgrad(s, B.MOE_OP_DOWN, run.act(), dy, dcounts, dpad, dw2_q, None, sched)
    torch.cuda.synchronize()
    assert torch.equal(dw2.view(torch.int32), dw2_q.view(torch.int32))
    # the same data gradient on the forward kernels against weights transposed into a
    # workspace
    dact_t = e(rows, de)
    wt = torch.empty(B.moe_grouped_gemm_dgrad_workspace_bytes(s, B.MOE_OP_DOWN), dtype=torch.uint8,
                     device=DEV)
    B.moe_grouped_gemm_dgrad(s, B.MOE_OP_DOWN, dy, inp.w2, None, meta, nblk, mb, dact_t, wt)
    torch.cuda.synchronize()
    assert_close(f64(dact_t)[valid], dact_ref[valid], TOL_STAGE["bf16"], "dact (transposed)")
    for ex in np.nonzero(counts == 0)[0]:
        assert not torch.any(dw2[ex] != 0), f"expert {ex} has no rows: dW2 must be 0"

    # SwiGLU backward with the gate/up products recomputed: from x_perm, and gathered
    xp = run.x_perm()
    dgu, dgu_g = e(rows, 2 * de), e(rows, 2 * de)
    B.moe_swiglu_bwd(s, xp, None, inp.w1, inp.w3, dact, meta, nblk, mb, dgu)
    B.moe_swiglu_bwd(s, inp.x, row_src, inp.w1, inp.w3, dact, meta, nblk, mb, dgu_g)
    torch.cuda.synchronize()
    dv = torch.from_numpy(valid).to(DEV)
    assert torch.equal(dgu[dv].view(torch.int16), dgu_g[dv].view(torch.int16))
    xp_h, dact_h = f64(xp), f64(dact)
    dg_ref = np.zeros((rows, de))
    du_ref = np.zeros((rows, de))
    for ex in range(E):
        r = rows_of(ex)
        dg_ref[r], du_ref[r], _ = BW.swiglu_backward(xp_h[r], h["w1"][ex], h["w3"][ex], dact_h[r])
    assert_close(f64(dgu[:, :de])[valid], dg_ref[valid], TOL_STAGE["bf16"], "dg")
    assert_close(f64(dgu[:, de:])[valid], du_ref[valid], TOL_STAGE["bf16"], "du")

    # gate/up: data gradient and weight gradients on the device's dg | du
    dxp, dw1, dw3 = e(rows, d), f(E, d, de), f(E, d, de)
    B.moe_grouped_gemm_dgrad(s, B.MOE_OP_GATEUP_SWIGLU, dgu, inp.w1, inp.w3, meta, nblk, mb, dxp)
    B.moe_grouped_gemm_wgrad(s, B.MOE_OP_GATEUP_SWIGLU, xp, dgu, dcounts, dpad, dw1, dw3)
    dw1_q, dw3_q = torch.full_like(dw1, float("nan")), torch.full_like(dw3, float("nan"))
    B.moe_grouped_gemm_wgrad(s, B.MOE_OP_GATEUP_SWIGLU, xp, dgu, dcounts, dpad, dw1_q, dw3_q, sched)
    torch.cuda.synchronize()
    assert torch.equal(dw1.view(torch.int32), dw1_q.view(torch.int32))
    assert torch.equal(dw3.view(torch.int32), dw3_q.view(torch.int32))
    dgu_h = f64(dgu)
    dxp_ref = np.zeros((rows, d))
    dw1_ref, dw3_ref = np.zeros((E, d, de)), np.zeros((E, d, de))
    for ex in range(E):
        r = rows_of(ex)
        dxp_ref[r] = dgu_h[r, :de] @ h["w1"][ex].T + dgu_h[r, de:] @ h["w3"][ex].T
        dw1_ref[ex] = xp_h[r].T @ dgu_h[r, :de]
        dw3_ref[ex] = xp_h[r].T @ dgu_h[r, de:]
    assert_close(f64(dxp)[valid], dxp_ref[valid], TOL_STAGE["bf16"], "dx_perm")
    dxp_t = e(rows, d)
    wt = torch.empty(B.moe_grouped_gemm_dgrad_workspace_bytes(s, B.MOE_OP_GATEUP_SWIGLU),
                     dtype=torch.uint8, device=DEV)
    B.moe_grouped_gemm_dgrad(s, B.MOE_OP_GATEUP_SWIGLU, dgu, inp.w1, inp.w3, meta, nblk, mb, dxp_t,
                             wt)
    torch.cuda.synchronize()
    assert_close(f64(dxp_t)[valid], dxp_ref[valid], TOL_STAGE["bf16"], "dx_perm (transposed)")
    assert_close(f64(dw1), dw1_ref, TOL_WGRAD, "dW1")
    assert_close(f64(dw3), dw3_ref, TOL_WGRAD, "dW3")

    # permute backward: the combine with unit weights sums each token's k rows
    dx_sum = e(T, d)
    B.moe_combine(s, dxp, dpos, None, None, dx_sum)
    torch.cuda.synchronize()
    assert_close(f64(dx_sum), BW.unpermute_sum(f64(dxp), pos, T, k), TOL_STAGE["bf16"], "unpermute")

    # the shared expert: dense-mode dgrad / wgrad (E = 1, d_e = d_e_shared)
    if ds:
        s1 = B.make_shape(T=T, d=d, E=1, k=1, d_e=ds, block_m=cfg.block_m)
        sdact, sdgu, sdx = e(T, ds), e(T, 2 * ds), e(T, d)
        dws1, dws3, dws2 = f(d, ds), f(d, ds), f(ds, d)
        sact = run.view("shared_act", bf, (T, ds))
        B.moe_grouped_gemm_dgrad(s1, B.MOE_OP_DOWN, dout, inp.ws2, None, None, None, 0, sdact)
        B.moe_grouped_gemm_wgrad(s1, B.MOE_OP_DOWN, sact, dout, None, None, dws2, None)
        torch.cuda.synchronize()
        assert_close(f64(sdact), dout_h @ h["ws2"].T, TOL_STAGE["bf16"], "shared dact")
        assert_close(f64(dws2), f64(sact).T @ dout_h, TOL_WGRAD, "dWs2")
        # the shared set rides along in the routed launch (or its own when sizes differ)
        B.moe_swiglu_bwd(s, xp, None, inp.w1, inp.w3, dact, meta, nblk, mb, dgu, inp.x, inp.ws1,
                         inp.ws3, sdact, sdgu)
        B.moe_grouped_gemm_dgrad(s1, B.MOE_OP_GATEUP_SWIGLU, sdgu, inp.ws1, inp.ws3, None, None, 0,
                                 sdx)
        B.moe_grouped_gemm_wgrad(s1, B.MOE_OP_GATEUP_SWIGLU, inp.x, sdgu, None, None, dws1, dws3)
        torch.cuda.synchronize()
        assert torch.equal(dgu[dv].view(torch.int16), dgu_g[dv].view(torch.int16))
        sg, su, _ = BW.swiglu_backward(h["x"], h["ws1"], h["ws3"], f64(sdact))
        assert_close(f64(sdgu[:, :ds]), sg, TOL_STAGE["bf16"], "shared dg")
        assert_close(f64(sdgu[:, ds:]), su, TOL_STAGE["bf16"], "shared du")
        sdgu_h = f64(sdgu)
        assert_close(f64(sdx), sdgu_h[:, :ds] @ h["ws1"].T + sdgu_h[:, ds:] @ h["ws3"].T,
                     TOL_STAGE["bf16"], "shared dx")
        sdx_t = e(T, d)
        wt = torch.empty(B.moe_grouped_gemm_dgrad_workspace_bytes(s1, B.MOE_OP_GATEUP_SWIGLU),
                         dtype=torch.uint8, device=DEV)
        B.moe_grouped_gemm_dgrad(s1, B.MOE_OP_GATEUP_SWIGLU, sdgu, inp.ws1, inp.ws3, None, None, 0,
                                 sdx_t, wt)
        torch.cuda.synchronize()
        assert_close(f64(sdx_t), sdgu_h[:, :ds] @ h["ws1"].T + sdgu_h[:, ds:] @ h["ws3"].T,
                     TOL_STAGE["bf16"], "shared dx (transposed)")
        assert_close(f64(dws1), h["x"].T @ sdgu_h[:, :ds], TOL_WGRAD, "dWs1")
        assert_close(f64(dws3), h["x"].T @ sdgu_h[:, ds:], TOL_WGRAD, "dWs3")

    # router backward on the device's logits and dtopk_w
    dl, dwg, db, dxr = f(T, E), f(d, E), f(E), e(T, d)
    B.moe_router_bwd(s, inp.x, inp.w_gate, run.logits(), idx, dtw, dl, dwg, db, dx_sum, dxr)
    torch.cuda.synchronize()
    dl_ref = BW.router_backward(f64(run.logits()), i64(idx), f64(dtw), cfg.renormalize)
    assert_close(f64(dl), dl_ref, TOL_DLOGITS, "dlogits")
    dl_h = f64(dl)
    assert_close(f64(dwg), h["x"].T @ dl_h, TOL_WGRAD, "dW_g")
    assert_close(f64(db), dl_h.sum(axis=0), TOL_WGRAD, "dbias")
    assert_close(f64(dxr), f64(dx_sum) + dl_h @ h["w_gate"].T, TOL_STAGE["bf16"], "router dx")


def _layer_grads(cfg, inp, dout, tile=None):
    run = LayerRun(cfg, inp)
    s = run.shape
    T, d, E, de, ds = cfg.T, cfg.d, cfg.E, cfg.d_e, cfg.d_e_shared
    f = lambda *sh: torch.full(sh, float("nan"), dtype=torch.float32, device=DEV)
    g = dict(dx=torch.empty((T, d), dtype=torch.bfloat16, device=DEV), dw1=f(E, d, de),
             dw3=f(E, d, de), dw2=f(E, de, d), dtopk_w=f(T, cfg.k))
    g.update(dws1=f(d, ds) if ds else None, dws3=f(d, ds) if ds else None,
             dws2=f(ds, d) if ds else None)
    routed = run.routed
    g.update(dw_gate=None if routed else f(d, E), dbias=None if routed else f(E))
    ws = B.alloc_bwd_workspace(s)
    B.moe_layer_bwd(s, inp.x, None if routed else inp.w_gate, inp.w1, inp.w3, inp.w2, inp.ws1,
                    inp.ws3, inp.ws2, inp.topk_idx if routed else None,
                    inp.topk_w if routed else None, dout, run.ws, g["dx"], g["dw1"], g["dw3"],
                    g["dw2"], g["dws1"], g["dws3"], g["dws2"], g["dw_gate"], g["dbias"],
                    g["dtopk_w"], ws)
    torch.cuda.synchronize()
    return run, g


LAYER_CASES = [
    ("fusedmoe-8x2048", dict(name="fusedmoe-bwd-l", T=256, d=512, d_e=256, d_e_shared=256), None),
    ("fusedmoe-8x2048", dict(name="fusedmoe-bwd-384", T=600, d=256, d_e=128, d_e_shared=128), "384"),
    # 256-row blocks; a shared expert (d_e_shared 1088) with its own launches, N > 512
    ("fusedmoe-8x2048", dict(name="fusedmoe-bwd-bm256", T=200, d=256, d_e=192, d_e_shared=1088,
                             block_m=256), None),
    ("zipf-skew-64x1408", dict(name="zipf-bwd-l", T=300, d=256, d_e=160), None),
    # experts averaging >= 256 rows: data gradients on transposed weights, shared expert
    # of another size in launches of its own
    ("fusedmoe-8x2048", dict(name="fusedmoe-bwd-tw", T=640, d=256, d_e=192, d_e_shared=320), None),
    ("ep-share-4x2048", dict(name="ep-share-bwd-l", T=128, d=512, d_e=256,
                             fixed_counts=(400, 0, 333, 291)), None),
    ("decode-256x2048", dict(name="decode-bwd-l", T=16, d=512, E=64, d_e=128, d_e_shared=192), None),
]


@pytest.mark.parametrize("name,scale,tile", LAYER_CASES)
def test_layer_bwd_against_oracle(name, scale, tile, monkeypatch):
    if tile:
        monkeypatch.setenv("MOE_GG_TILE_ROWS", tile)
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    dout = _dout(cfg, 11)
    run, g = _layer_grads(cfg, inp, dout)
    h = host_inputs(inp)
    fwd = _oracle_forward(cfg, h, run, inp)
    ref = BW.moe_layer_backward(fwd, h["x"], h["w1"], h["w3"], h["w2"], f64(dout), k=cfg.k,
                                block_m=cfg.block_m, w_gate=h["w_gate"], bias=h["bias"],
                                renormalize=cfg.renormalize, ws1=h["ws1"], ws3=h["ws3"],
                                ws2=h["ws2"], routed=run.routed)
    rel = {}
    rel["dx"] = assert_close(f64(g["dx"]), ref.dx, TOL_GRAD, "dx")
    for n in ("dw1", "dw3", "dw2", "dws1", "dws3", "dws2", "dw_gate", "dbias"):
        if g[n] is not None:
            rel[n] = assert_close(f64(g[n]), getattr(ref, n), TOL_GRAD, n)
    rel["dtopk_w"] = assert_close(f64(g["dtopk_w"]), ref.dtopk_w, TOL_GRAD, "dtopk_w")
    empty = np.nonzero(np.asarray(fwd.counts) == 0)[0]
    for ex in empty:
        for n in ("dw1", "dw3", "dw2"):
            assert not torch.any(g[n][ex] != 0), f"{n}[{ex}] of an expert without rows"
    print(f"[bwd parity] {cfg.name}: " + " ".join(f"{n}={v:.1e}" for n, v in rel.items()))


def _oracle_forward(cfg, h, run, inp):
    kw = dict(k=cfg.k, block_m=cfg.block_m, ws1=h["ws1"], ws3=h["ws3"], ws2=h["ws2"])
    if run.routed:
        return O.moe_layer(h["x"], h["w1"], h["w3"], h["w2"], topk_idx=i64(inp.topk_idx),
                           topk_w=f64(inp.topk_w), **kw)
    fwd = O.moe_layer(h["x"], h["w1"], h["w3"], h["w2"], w_gate=h["w_gate"], bias=h["bias"],
                      n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                      renormalize=cfg.renormalize, decision_logits=run.logits().cpu().numpy(), **kw)
    return fwd


def test_layer_bwd_without_tokens_zeroes_the_weight_gradients():
    """T == 0: no rows reach any expert, so every weight gradient is zero (the buffers
    start as NaN).  Token buffers are one-row stand-ins that are never read."""
    cfg = get_config("fusedmoe-8x2048").scaled(name="fusedmoe-bwd-t0", T=4, d=256, d_e=128,
                                               d_e_shared=128)
    inp = make_inputs(cfg, device=DEV)
    s = B.make_shape(T=0, d=cfg.d, E=cfg.E, k=cfg.k, d_e=cfg.d_e, block_m=cfg.block_m,
                     d_e_shared=cfg.d_e_shared)
    d, E, de, ds = cfg.d, cfg.E, cfg.d_e, cfg.d_e_shared
    f = lambda *sh: torch.full(sh, float("nan"), dtype=torch.float32, device=DEV)
    g = dict(dw1=f(E, d, de), dw3=f(E, d, de), dw2=f(E, de, d), dws1=f(d, ds), dws3=f(d, ds),
             dws2=f(ds, d), dw_gate=f(d, E), dbias=f(E))
    stand_in = torch.zeros((1, d), dtype=torch.bfloat16, device=DEV)
    fwd_ws, ws = B.alloc_workspace(s), B.alloc_bwd_workspace(s)
    B.moe_layer_bwd(s, stand_in, inp.w_gate, inp.w1, inp.w3, inp.w2, inp.ws1, inp.ws3, inp.ws2,
                    None, None, stand_in, fwd_ws, stand_in.clone(), g["dw1"], g["dw3"], g["dw2"],
                    g["dws1"], g["dws3"], g["dws2"], g["dw_gate"], g["dbias"], None, ws)
    torch.cuda.synchronize()
    for n, v in g.items():
        assert torch.count_nonzero(v).item() == 0, n


@pytest.mark.parametrize("name,scale", [
    ("fusedmoe-8x2048", dict(name="fusedmoe-bwd-det", T=640, d=256, d_e=192, d_e_shared=320)),
    ("zipf-skew-64x1408", dict(name="zipf-bwd-det", T=300, d=256, d_e=160)),
])
def test_layer_bwd_is_deterministic(name, scale):
    """Two backward passes of the same layer produce bitwise-equal gradients: every sum
    (weight gradients over an expert's rows, the router's chunked weight gradient, dx
    over a token's k rows) runs in a fixed order, with no atomics."""
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    dout = _dout(cfg, 13)
    _, g1 = _layer_grads(cfg, inp, dout)
    _, g2 = _layer_grads(cfg, inp, dout)
    for n, a in g1.items():
        if a is None:
            continue
        v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(v), g2[n].view(v)), n


# Router backward off and on the 8-wide kernels: expert counts that are not multiples of
# 8, a partial group of experts, column tails, one and several token chunks.  Operands 4
# bytes past a 16-byte boundary (dlogits, W_g) send the work to the scalar loads.
ROUTER_BWD_SHAPES = [
    dict(T=700, d=192, E=6, k=2, renormalize=True),
    dict(T=520, d=288, E=12, k=3, renormalize=False),
    dict(T=1000, d=544, E=16, k=4, renormalize=True),
    dict(T=5, d=256, E=8, k=2, renormalize=False),
]


def _shifted(t):
    """A contiguous tensor equal to t that starts 4 bytes past a 16-byte boundary."""
    off = 4 // t.element_size()
    buf = torch.empty(t.numel() + 16, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.gpu
@pytest.mark.parametrize("sh", ROUTER_BWD_SHAPES, ids=lambda s: f"T{s['T']}-d{s['d']}-E{s['E']}")
def test_router_bwd_shapes_and_alignment(sh):
    T, d, E, k = sh["T"], sh["d"], sh["E"], sh["k"]
    print(f"router bwd T={T} d={d} E={E} k={k}", flush=True)
    g = torch.Generator().manual_seed(1000 * E + d)
    x = torch.randn(T, d, generator=g).to(torch.bfloat16)
    wg = (torch.randn(d, E, generator=g) / d ** 0.5).to(torch.bfloat16)
    logits = torch.randn(T, E, generator=g)
    idx = torch.topk(logits, k, dim=1).indices.to(torch.int32)
    dtw = torch.randn(T, k, generator=g)
    base = torch.randn(T, d, generator=g).to(torch.bfloat16)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=128, block_m=128, renormalize=sh["renormalize"])
    xd, wgd, ld, idd, dtd, bd = (t.to(DEV) for t in (x, wg, logits, idx, dtw, base))
    f = lambda *shp: torch.full(shp, float("nan"), dtype=torch.float32, device=DEV)
    outs = []
    for shift in (False, True):
        dl = _shifted(f(T, E)) if shift else f(T, E)
        wgs = _shifted(wgd) if shift else wgd
        dwg, db = f(d, E), f(E)
        dxr = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
        dx0 = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
        B.moe_router_bwd(s, xd, wgs, ld, idd, dtd, dl, dwg, db, bd, dxr)
        B.moe_router_bwd(s, xd, wgs, ld, idd, dtd, dl, dwg, None, None, dx0)
        torch.cuda.synchronize()
        outs.append((dl.clone(), dwg.clone(), db.clone(), dxr.clone(), dx0.clone()))
    dl_ref = BW.router_backward(logits.double().numpy(), idx.numpy(), dtw.double().numpy(),
                                sh["renormalize"])
    dl, dwg, db, dxr, dx0 = outs[0]
    assert_close(f64(dl), dl_ref, TOL_DLOGITS, "dlogits")
    dl_h = f64(dl)
    xh, wh = x.double().numpy(), wg.double().numpy()
    assert_close(f64(dwg), xh.T @ dl_h, TOL_WGRAD, "dW_g")
    assert_close(f64(db), dl_h.sum(axis=0), TOL_WGRAD, "dbias")
    assert_close(f64(dxr), base.double().numpy() + dl_h @ wh.T, TOL_STAGE["bf16"], "router dx")
    assert_close(f64(dx0), dl_h @ wh.T, TOL_STAGE["bf16"], "router dx, no base")
    # aligned and shifted operands take the same additions: equal bit for bit
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(_bits(a), _bits(b))
