"""The debug build of the library (libmoe_debug.so, compiled with MOE_DEBUG).

On valid work none of the kernels' bounds checks fires - no MOE_DBG bit is set - and
every result is bit for bit the release library's.  Block tables, block counts and row
positions that a caller corrupts are skipped or clamped exactly as in the release build
(same outputs), and the debug build reports them."""
import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from workloads import get_config, make_inputs

from gpu_util import LayerRun

pytestmark = pytest.mark.gpu
DEV = "cuda"


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.fixture(autouse=True)
def clear_debug_word():
    with B.debug_library():
        B.moe_debug_flags(clear=True)
    yield


LAYER_CASES = [
    # wide 384-row tiles (512 rows per expert), then the 128-row kernel
    ("fusedmoe-8x2048", dict(name="dbg-wide", T=1024, d=512, d_e=256, d_e_shared=256), None),
    ("fusedmoe-8x2048", dict(name="dbg-128", T=1024, d=512, d_e=256, d_e_shared=256), "128"),
    ("fusedmoe-8x2048", dict(name="dbg-unpadded", T=700, d=256, d_e=128, unpadded=True), None),
    ("zipf-skew-64x1408", dict(name="dbg-zipf", T=512, d=256, d_e=128), None),
    ("decode-256x2048", dict(name="dbg-decode", T=64, d=512, d_e=256), None),
    ("tiny-fp32", dict(), None),
]


@pytest.mark.parametrize("name,scale,tile", LAYER_CASES)
def test_layer_forward_sets_no_debug_bit_and_matches_release(name, scale, tile, monkeypatch):
    if tile:
        monkeypatch.setenv("MOE_GG_TILE_ROWS", tile)
    cfg = get_config(name).scaled(**scale) if scale else get_config(name)
    torch.manual_seed(0)
    inp = make_inputs(cfg, device=DEV)
    print(f"[debug layer] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} tile={tile}", flush=True)
    rel = LayerRun(cfg, inp)
    with B.debug_library():
        dbg = LayerRun(cfg, inp)
        flags = B.moe_debug_flags()
    assert flags == 0, hex(flags)
    assert same_bits(rel.out, dbg.out)
    s = rel.shape
    M = cfg.T * cfg.k
    for n, dt, sh in (("topk_idx", torch.int32, (M,)), ("pos", torch.int32, (M,)),
                      ("block_meta", torch.int32, (3 * B.moe_max_blocks(s),))):
        a, b = rel.view(n, dt, sh), dbg.view(n, dt, sh)
        if n == "block_meta":
            nb = int(rel.view("num_blocks", torch.int32, (1,)).item())
            a, b = a[:3 * nb], b[:3 * nb]
        assert torch.equal(a, b), n


def test_fp8_layer_sets_no_debug_bit_and_matches_release():
    cfg = get_config("decode-256x2048").scaled(name="dbg-fp8", T=128, d=512, d_e=256)
    torch.manual_seed(1)
    inp = make_inputs(cfg, device=DEV)
    s = B.shape_of_config(cfg)
    qz = [B.quantize_fp8(w) for w in (inp.w1, inp.w3, inp.w2)]
    qs = [B.quantize_fp8(w) for w in (inp.ws1, inp.ws3, inp.ws2)] if cfg.d_e_shared else [(None, None)] * 3
    routed = inp.topk_idx is not None
    outs = []
    for debug in (False, True):
        out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
        ws = B.alloc_workspace(s, fp8=True)
        print(f"[debug fp8] debug={debug} T={cfg.T} d={cfg.d}", flush=True)
        if debug:
            with B.debug_library():
                B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *qz[0], *qz[1], *qz[2], *qs[0],
                                    *qs[1], *qs[2], inp.topk_idx if routed else None,
                                    inp.topk_w if routed else None, out, ws)
                assert B.moe_debug_flags() == 0
        else:
            B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *qz[0], *qz[1], *qz[2], *qs[0],
                                *qs[1], *qs[2], inp.topk_idx if routed else None,
                                inp.topk_w if routed else None, out, ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert same_bits(outs[0], outs[1])


def test_layer_backward_sets_no_debug_bit_and_matches_release():
    cfg = get_config("fusedmoe-8x2048").scaled(name="dbg-bwd", T=256, d=256, d_e=128, d_e_shared=128)
    torch.manual_seed(2)
    inp = make_inputs(cfg, device=DEV)
    dout = torch.randn((cfg.T, cfg.d), device=DEV).to(torch.bfloat16)
    T, d, E, de, ds = cfg.T, cfg.d, cfg.E, cfg.d_e, cfg.d_e_shared
    res = []
    for debug in (False, True):
        print(f"[debug bwd] debug={debug}", flush=True)
        ctx = B.debug_library() if debug else _null()
        with ctx:
            run = LayerRun(cfg, inp)
            s = run.shape
            f = lambda *sh: torch.zeros(sh, dtype=torch.float32, device=DEV)
            g = dict(dx=torch.empty((T, d), dtype=torch.bfloat16, device=DEV), dw1=f(E, d, de),
                     dw3=f(E, d, de), dw2=f(E, de, d), dws1=f(d, ds), dws3=f(d, ds), dws2=f(ds, d),
                     dw_gate=f(d, E), dbias=f(E), dtopk_w=f(T, cfg.k))
            ws = B.alloc_bwd_workspace(s)
            B.moe_layer_bwd(s, inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, inp.ws1, inp.ws3, inp.ws2,
                            None, None, dout, run.ws, g["dx"], g["dw1"], g["dw3"], g["dw2"],
                            g["dws1"], g["dws3"], g["dws2"], g["dw_gate"], g["dbias"], g["dtopk_w"], ws)
            torch.cuda.synchronize()
            if debug:
                assert B.moe_debug_flags() == 0
        res.append(g)
    for n in res[0]:
        assert same_bits(res[0][n], res[1][n]), n


class _null:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def _routed_table(T, d, E, k, d_e, seed):
    """A bf16 shape, its block table from moe_build_offsets and random operands."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, k))
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16")
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.full((max(n, 1),), -1, dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err,
                        B.alloc_workspace(s))
    torch.cuda.synchronize()
    return s, mb, rows, meta, nblk, pos


@pytest.mark.parametrize("tile", ["128", "384"])
@pytest.mark.parametrize("fault", ["expert", "count"])
def test_corrupt_block_table_is_skipped_alike_and_reported(tile, fault, monkeypatch):
    """An entry naming expert E, or a block count above max_blocks (the entries past the
    real count hold expert -1): both builds skip the same entries and write the same C;
    the debug build reports the table and the count."""
    monkeypatch.setenv("MOE_GG_TILE_ROWS", tile)
    T, d, E, k, d_e = 512, 256, 4, 2, 128
    s, mb, rows, meta, nblk, _ = _routed_table(T, d, E, k, d_e, 7)
    nb = int(nblk.item())
    assert nb < mb
    if fault == "expert":
        meta[3] = E                      # entry 1's expert
        want = B.MOE_DBG_BLOCK_TABLE
    else:
        nblk.fill_(mb + 3)               # entries nb .. mb-1 keep expert -1 from the fill
        want = B.MOE_DBG_BLOCK_COUNT | B.MOE_DBG_BLOCK_TABLE
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    A = torch.randn((rows, d), generator=g, device=DEV).to(torch.bfloat16)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(torch.bfloat16)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(torch.bfloat16)
    Cs = []
    for debug in (False, True):
        print(f"[debug table] tile={tile} fault={fault} debug={debug}", flush=True)
        C = torch.full((rows, d_e), -7.0, dtype=torch.bfloat16, device=DEV)
        ctx = B.debug_library() if debug else _null()
        with ctx:
            B.moe_grouped_gemm(s, B.MOE_OP_GATEUP_SWIGLU, A, w1, w3, meta, nblk, mb, C)
            torch.cuda.synchronize()
            if debug:
                assert B.moe_debug_flags() == want
        Cs.append(C)
    assert same_bits(Cs[0], Cs[1])
    if fault == "expert":   # entry 1's rows were skipped: still the fill value
        r0 = int(meta[4].item())
        assert torch.all(Cs[0][r0:r0 + 128] == -7.0)


def test_positions_out_of_range_are_skipped_alike_and_reported():
    T, d, E, k, d_e = 256, 256, 4, 2, 128
    s, mb, rows, meta, nblk, pos = _routed_table(T, d, E, k, d_e, 9)
    bad = pos.clone()
    bad[5] = rows          # one past the row buffers
    bad[17] = -5           # below the "dropped" marker
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    x = torch.randn((T, d), generator=g, device=DEV).to(torch.bfloat16)
    y = torch.randn((rows, d), generator=g, device=DEV).to(torch.bfloat16)
    w = torch.rand((T, k), generator=g, device=DEV)
    res = []
    for debug in (False, True):
        print(f"[debug positions] debug={debug}", flush=True)
        xp = torch.zeros((rows, d), dtype=torch.bfloat16, device=DEV)
        out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
        ctx = B.debug_library() if debug else _null()
        with ctx:
            B.moe_permute(s, x, bad, xp)
            B.moe_combine(s, y, bad, w, None, out)
            torch.cuda.synchronize()
            res.append((xp.clone(), out.clone()))
            if debug:
                assert B.moe_debug_flags() == B.MOE_DBG_POSITION
                # the valid positions alone set nothing
                B.moe_permute(s, x, pos, xp)
                B.moe_combine(s, y, pos, w, None, out)
                assert B.moe_debug_flags() == 0
    assert same_bits(res[0][0], res[1][0]) and same_bits(res[0][1], res[1][1])
