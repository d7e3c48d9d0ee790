"""The layer's forward and backward inside a HIP graph.

The library enqueues kernels only (no allocation, no memset, no host synchronisation),
so a whole moe_layer_fwd (router, offsets, grouped GEMMs, combine) and moe_layer_bwd can
be captured once and replayed.  Each replay must equal the eager call bitwise; replays
are separated by eager work on the same buffers (the inputs change between replays and
are restored), so a replay that reused stale state would be caught.
"""
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name,scale", [
    ("fusedmoe-8x2048", dict(name="graph-fm", T=600, d=512, d_e=256, d_e_shared=256)),
    ("decode-256x2048", dict(name="graph-decode", d=512, d_e=256, d_e_shared=256)),
    ("tiny-fp32", dict(name="graph-tiny")),
])
def test_layer_fwd_replays_in_a_graph(name, scale):
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    s = B.shape_of_config(cfg)
    ws = B.alloc_workspace(s)
    out = torch.empty((cfg.T, cfg.d), dtype=inp.x.dtype, device=DEV)
    routed = inp.topk_idx is not None
    ri, rw = (inp.topk_idx, inp.topk_w) if routed else (None, None)
    call = lambda: B.moe_layer_fwd(s, inp.x, inp.w_gate, inp.bias, inp.w1, inp.w3, inp.w2,
                                   inp.ws1, inp.ws3, inp.ws2, ri, rw, out, ws)
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    bits = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    x0 = inp.x.clone()
    for rep in range(3):
        out.zero_()
        ws.fill_(0xA5)                # the replay must rebuild every intermediate
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(bits), ref.view(bits)), f"replay {rep}"
        # eager work in between: another input, then the original restored
        inp.x.mul_(-1)
        call()
        torch.cuda.synchronize()
        inp.x.copy_(x0)


def test_layer_bwd_replays_in_a_graph():
    cfg = get_config("fusedmoe-8x2048").scaled(name="graph-bwd", T=640, d=256, d_e=192,
                                               d_e_shared=320)
    inp = make_inputs(cfg, device=DEV)
    s = B.shape_of_config(cfg)
    ws, bws = B.alloc_workspace(s), B.alloc_bwd_workspace(s)
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    dout = torch.randn((cfg.T, cfg.d), generator=gen, device=DEV).to(torch.bfloat16)
    d, E, de, ds = cfg.d, cfg.E, cfg.d_e, cfg.d_e_shared
    f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=DEV)
    gr = dict(dx=torch.empty((cfg.T, d), dtype=torch.bfloat16, device=DEV), dw1=f(E, d, de),
              dw3=f(E, d, de), dw2=f(E, de, d), dws1=f(d, ds), dws3=f(d, ds), dws2=f(ds, d),
              dwg=f(d, E), db=f(E), dtw=f(cfg.T, cfg.k))

    def call():
        B.moe_layer_fwd(s, inp.x, inp.w_gate, inp.bias, inp.w1, inp.w3, inp.w2, inp.ws1, inp.ws3,
                        inp.ws2, None, None, out, ws)
        B.moe_layer_bwd(s, inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, inp.ws1, inp.ws3, inp.ws2,
                        None, None, dout, ws, gr["dx"], gr["dw1"], gr["dw3"], gr["dw2"], gr["dws1"],
                        gr["dws3"], gr["dws2"], gr["dwg"], gr["db"], gr["dtw"], bws)

    call()
    torch.cuda.synchronize()
    ref = {n: v.clone() for n, v in gr.items()}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for v in gr.values():
            v.fill_(float("nan")) if v.dtype == torch.float32 else v.zero_()
        bws.fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        for n, v in gr.items():
            bits = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(v.view(bits), ref[n].view(bits)), f"replay {rep}: {n}"
        call()                        # eager work between replays
        torch.cuda.synchronize()
