"""Unpadded segments ([DG] §11) on the GPU, through the C ABI.

  * counts, offsets, the block table (one entry per tile and expert) and the
    permutation are integers: bit-exact against the oracle's unpadded_tile_table and
    permutation_unpadded;
  * every output row is computed by the same arithmetic as in the padded layout (the
    same A row, the same weights, the same order over K; the weight gradients reduce
    over the same rows in the same order), so the layer's forward output, its fp8
    variant and every gradient of its backward are bitwise equal to the padded layout's,
    and the forward also meets the oracle's output bound.
"""
import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import moe_oracle as O
from workloads import get_config, make_inputs

from gpu_util import TOL_OUT, LayerRun, assert_close, f64, host_inputs, oracle_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _offsets(s, idx):
    E, M = s.E, s.T * s.k
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(np.asarray(idx, np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(M), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    torch.cuda.synchronize()
    n = lambda t: t.cpu().numpy().astype(np.int64)
    return dict(counts=n(counts), offsets=n(offs), padded=n(pad), meta=n(meta).reshape(-1, 3),
                nblk=int(nblk.item()), pos=n(pos)[:M], row_src=n(row_src)[:rows], err=int(err.item()))


def _routes(kind, T, E, k, rng):
    if kind == "random":
        return rng.integers(0, E, size=(T, k))
    if kind == "one-expert":
        return np.full((T, k), E - 1)
    if kind == "empty-experts":
        return rng.choice([0, E - 1], size=(T, k))
    if kind == "tile-multiples":          # every segment a multiple of the tile height
        return np.repeat(np.arange(E), T * k // E)[rng.permutation(T * k)].reshape(T, k)
    raise ValueError(kind)


@pytest.mark.parametrize("kind,T,E,k,bm", [
    ("random", 300, 8, 2, 128), ("random", 1000, 64, 6, 128), ("random", 37, 5, 3, 16),
    ("one-expert", 200, 4, 2, 128), ("empty-experts", 500, 16, 4, 128),
    ("tile-multiples", 512, 4, 2, 128), ("random", 3000, 3, 1, 256), ("random", 5, 8, 3, 128),
])
def test_build_offsets_unpadded_bit_exact(kind, T, E, k, bm):
    rng = np.random.default_rng(T + E + k)
    idx = _routes(kind, T, E, k, rng)
    dt = "bf16" if bm % 128 == 0 else "fp32"
    s = B.make_shape(T=T, d=8, E=E, k=k, d_e=8, block_m=bm, dtype=dt, unpadded=True)
    assert B.moe_max_rows(s) == T * k
    got = _offsets(s, idx)
    counts = O.expert_counts(idx, E)
    off = O.group_offsets(counts)
    tab = O.unpadded_tile_table(counts, bm)
    pos, row_src = O.permutation_unpadded(idx, E)
    assert got["err"] == 0
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], off)
    assert np.array_equal(got["padded"], off)                 # no padding
    assert got["nblk"] == len(tab) <= B.moe_max_blocks(s)
    assert np.array_equal(got["meta"][:len(tab)], tab)
    assert np.array_equal(got["pos"], pos)
    assert np.array_equal(got["row_src"], row_src)


def test_build_offsets_unpadded_worked_example():
    """The pages' 65,536-row share: 515 entries (512 tiles, three boundaries inside tiles)
    against 514 padded blocks; tile 169 split 101 / 27 rows."""
    cfg = get_config("ep-share-4x2048")
    inp = make_inputs(cfg.scaled(name="ep-share-idx", d=8, d_e=8), device=DEV)
    s = B.make_shape(T=cfg.T, d=8, E=cfg.E, k=cfg.k, d_e=8, block_m=128, unpadded=True)
    got = _offsets(s, inp.topk_idx.cpu().numpy())
    assert list(got["counts"]) == [21733, 15004, 17982, 10817]
    assert got["nblk"] == 515
    at169 = [tuple(r) for r in got["meta"][:515] if r[1] // 128 == 169]
    assert at169 == [(0, 21632, 101), (1, 21733, 27)]


def _layer(cfg, inp, unpadded, fp8=False):
    c = cfg.scaled(name=cfg.name + ("-unpadded" if unpadded else "-padded"), unpadded=unpadded)
    s = B.shape_of_config(c)
    ws = B.alloc_workspace(s, fp8=fp8)
    out = torch.empty((c.T, c.d), dtype=inp.x.dtype, device=DEV)
    routed = inp.topk_idx is not None
    ri, rw = (inp.topk_idx, inp.topk_w) if routed else (None, None)
    if fp8:
        q = [B.quantize_fp8(w) for w in (inp.w1, inp.w3, inp.w2)]
        qs = ([B.quantize_fp8(w) for w in (inp.ws1, inp.ws3, inp.ws2)] if c.d_e_shared
              else [(None, None)] * 3)
        B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *q[0], *q[1], *q[2], *qs[0], *qs[1],
                            *qs[2], ri, rw, out, ws)
    else:
        B.moe_layer_fwd(s, inp.x, inp.w_gate, inp.bias, inp.w1, inp.w3, inp.w2, inp.ws1, inp.ws3,
                        inp.ws2, ri, rw, out, ws)
    torch.cuda.synchronize()
    return c, s, ws, out


LAYER_CASES = [
    ("fusedmoe-8x2048", dict(name="fm-u", T=300, d=512, d_e=256, d_e_shared=256), None),
    ("fusedmoe-8x2048", dict(name="fm-u384", T=900, d=256, d_e=128, d_e_shared=128), "384"),
    ("zipf-skew-64x1408", dict(name="zipf-u", T=400, d=256, d_e=160), None),
    ("ep-share-4x2048", dict(name="ep-u", T=256, d=512, d_e=256,
                             fixed_counts=(700, 0, 733, 615)), "384"),
    ("decode-256x2048", dict(name="dec-u", T=24, d=512, E=64, d_e=128, d_e_shared=192), None),
    ("tiny-fp32", dict(name="tiny-u"), None),
]


@pytest.mark.parametrize("name,scale,tile", LAYER_CASES)
def test_layer_unpadded_equals_padded(name, scale, tile, monkeypatch):
    if tile:
        monkeypatch.setenv("MOE_GG_TILE_ROWS", tile)
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    _, _, _, out_p = _layer(cfg, inp, False)
    cu, su, wsu, out_u = _layer(cfg, inp, True)
    v = torch.int16 if out_p.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out_p.view(v), out_u.view(v))
    # and the oracle bound, on the unpadded run's own routing
    run = LayerRun.__new__(LayerRun)
    run.cfg, run.shape, run.ws, run.routed, run.x = cu, su, wsu, inp.topk_idx is not None, inp.x
    ref = oracle_layer(cu, host_inputs(inp), run, inp)
    assert_close(f64(out_u), ref.out, TOL_OUT[cu.dtype], "out")


@pytest.mark.parametrize("T", [300, 600])
def test_layer_fp8_unpadded_equals_padded(T):
    """T = 300: the fp8 kernels; T = 600 (experts average 300 rows): the weights
    dequantised, then the bf16 kernels."""
    cfg = get_config("fusedmoe-8x2048").scaled(name=f"fm-u-fp8-{T}", T=T, d=512, d_e=256,
                                               d_e_shared=256)
    inp = make_inputs(cfg, device=DEV)
    _, _, _, out_p = _layer(cfg, inp, False, fp8=True)
    _, _, _, out_u = _layer(cfg, inp, True, fp8=True)
    assert torch.equal(out_p.view(torch.int16), out_u.view(torch.int16))


@pytest.mark.parametrize("name,scale", [
    ("fusedmoe-8x2048", dict(name="fm-u-bwd", T=300, d=512, d_e=256, d_e_shared=256)),
    ("zipf-skew-64x1408", dict(name="zipf-u-bwd", T=400, d=256, d_e=160)),
])
def test_layer_bwd_unpadded_equals_padded(name, scale):
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    dout = torch.randn((cfg.T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    res = []
    for unpadded in (False, True):
        c, s, ws, _ = _layer(cfg, inp, unpadded)
        d, E, de, ds = c.d, c.E, c.d_e, c.d_e_shared
        f = lambda *sh: torch.full(sh, float("nan"), dtype=torch.float32, device=DEV)
        gr = dict(dx=torch.empty((c.T, d), dtype=torch.bfloat16, device=DEV), dw1=f(E, d, de),
                  dw3=f(E, d, de), dw2=f(E, de, d), dws1=f(d, ds) if ds else None,
                  dws3=f(d, ds) if ds else None, dws2=f(ds, d) if ds else None, dwg=f(d, E),
                  db=f(E), dtw=f(c.T, c.k))
        bws = B.alloc_bwd_workspace(s)
        B.moe_layer_bwd(s, inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, inp.ws1, inp.ws3, inp.ws2,
                        None, None, dout, ws, gr["dx"], gr["dw1"], gr["dw3"], gr["dw2"], gr["dws1"],
                        gr["dws3"], gr["dws2"], gr["dwg"], gr["db"], gr["dtw"], bws)
        torch.cuda.synchronize()
        res.append(gr)
    for n, a in res[0].items():
        if a is None:
            continue
        b = res[1][n]
        v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(v), b.view(v)), n
