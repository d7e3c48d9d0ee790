"""Helpers for the GPU parity tests: run the HIP path through the C ABI, fetch its
intermediates from the workspace, and compare with the CPU oracle.

Tolerances (floating point; integers are compared bit-exactly):
  * layer output: max|d| <= 2e-2 * max|ref| (bf16), 1e-5 * max|ref| (fp32), the
    stated acceptance bound;
  * a grouped-GEMM stage fed exactly the inputs the oracle gets: one bf16 rounding of
    the stored result (<= 2^-9 relative, so <= 2^-9 * max|ref|) plus fp32
    accumulation error, bounded by 5e-3 * max|ref|;
  * router logits: exact bf16 products accumulated in fp32 over d terms; the
    random-walk error is ~sqrt(d) * 2^-24 * sum|x w|, far below 1e-3 * max|ref|,
    while dropping even 8 of 7168 terms would exceed it;
  * routing weights: fp32 softmax (exp within 1 ulp, a log2(E)-level tree sum, one
    division) and renormalisation: <= 4e-6 relative per weight.
"""
from __future__ import annotations

import numpy as np
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import moe_oracle as O

TOL_OUT = {"bf16": 2e-2, "fp32": 1e-5}
TOL_STAGE = {"bf16": 5e-3, "fp32": 1e-5}
TOL_LOGITS = {"bf16": 1e-3, "fp32": 1e-5}
TOL_W_REL = 4e-6


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def i64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def max_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = float(np.abs(gpu - ref).max()) if ref.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return err, scale


def assert_close(gpu, ref, rel, what):
    err, scale = max_err(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert err <= rel * scale, f"{what}: max|d| = {err:.3e} > {rel:g} * max|ref| = {rel * scale:.3e}"
    return err / scale if scale else 0.0


class LayerRun:
    """One moe_layer_fwd call and typed views of every intermediate."""

    def __init__(self, cfg, inp, routed=None):
        self.cfg = cfg
        self.x = inp.x
        self.shape = B.shape_of_config(cfg)
        dev = inp.x.device
        self.ws = B.alloc_workspace(self.shape, dev)
        self.out = torch.empty((cfg.T, cfg.d), dtype=inp.x.dtype, device=dev)
        if routed is None:
            routed = inp.topk_idx is not None
        self.routed = routed
        B.moe_layer_fwd(self.shape, inp.x, inp.w_gate, inp.bias, inp.w1, inp.w3, inp.w2,
                        inp.ws1, inp.ws3, inp.ws2,
                        inp.topk_idx if routed else None, inp.topk_w if routed else None,
                        self.out, self.ws)
        torch.cuda.synchronize()
        self.layout = B.moe_workspace_layout(self.shape)

    def view(self, name, dtype, shape):
        return B.ws_view(self.ws, self.shape, name, dtype, shape)

    def ints(self):
        c, s = self.cfg, self.shape
        mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
        M = c.T * c.k
        nb = int(self.view("num_blocks", torch.int32, (1,)).item())
        return dict(
            counts=i64(self.view("counts", torch.int32, (c.E,))),
            offsets=i64(self.view("offsets", torch.int32, (c.E + 1,))),
            padded_offsets=i64(self.view("padded_offsets", torch.int32, (c.E + 1,))),
            num_blocks=nb,
            block_meta=i64(self.view("block_meta", torch.int32, (mb, 3)))[:nb],
            pos=i64(self.view("pos", torch.int32, (M,))),
            row_src=i64(self.view("row_src", torch.int32, (rows,))),
            err_flag=int(self.view("err_flag", torch.int32, (1,)).item()),
        )

    def dt(self):
        return torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32

    def logits(self):
        return self.view("logits", torch.float32, (self.cfg.T, self.cfg.E))

    def topk(self):
        c = self.cfg
        return (self.view("topk_idx", torch.int32, (c.T, c.k)),
                self.view("topk_w", torch.float32, (c.T, c.k)))

    def act(self):
        return self.view("act", self.dt(), (B.moe_max_rows(self.shape), self.cfg.d_e))

    def y(self):
        return self.view("y", self.dt(), (B.moe_max_rows(self.shape), self.cfg.d))

    def x_perm(self):
        """x permuted by the layer's own pos.  Where the layer fuses the permute into the
        gate/up loads (x_perm never written), the standalone moe_permute produces it."""
        rows = B.moe_max_rows(self.shape)
        if not B.gather_supported(self.shape):
            return self.view("x_perm", self.dt(), (rows, self.cfg.d))
        xp = torch.empty((rows, self.cfg.d), dtype=self.dt(), device=self.x.device)
        B.moe_permute(self.shape, self.x, self.view("pos", torch.int32, (self.cfg.T * self.cfg.k,)),
                      xp)
        torch.cuda.synchronize()
        return xp


def host_inputs(inp):
    """fp64 host copies of every floating input (exact for bf16 and fp32)."""
    g = lambda t: None if t is None else f64(t)
    return dict(x=g(inp.x), w_gate=g(inp.w_gate), bias=g(inp.bias), w1=g(inp.w1), w3=g(inp.w3),
                w2=g(inp.w2), ws1=g(inp.ws1), ws3=g(inp.ws3), ws2=g(inp.ws2))


def oracle_layer(cfg, h, run: LayerRun, inp):
    """The oracle layer on the same inputs.  Routing decisions are taken on the
    device's own fp32 logits (the selection is integer work decided by floating
    point, so both sides decide on identical numbers)."""
    kw = dict(k=cfg.k, block_m=cfg.block_m, ws1=h["ws1"], ws3=h["ws3"], ws2=h["ws2"])
    if run.routed:
        return O.moe_layer(h["x"], h["w1"], h["w3"], h["w2"], topk_idx=i64(inp.topk_idx),
                           topk_w=f64(inp.topk_w), **kw)
    return O.moe_layer(h["x"], h["w1"], h["w3"], h["w2"], w_gate=h["w_gate"], bias=h["bias"],
                       n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                       renormalize=cfg.renormalize,
                       decision_logits=run.logits().cpu().numpy(), **kw)


def check_routing_selection_margin(cfg, ref_logits64, gpu_idx, tol_abs):
    """The oracle's own choice (on its fp64 logits rounded to fp32) must equal the
    device's, except on tokens whose deciding logits are closer than the logits
    tolerance (there either choice is a correct result)."""
    dec = ref_logits64.astype(np.float32)
    own = O.topk_by_repeated_max(dec, cfg.k, O.eligible_experts(dec, cfg.n_groups, cfg.topk_groups))
    diff = np.nonzero(np.any(own != gpu_idx, axis=1))[0]
    for t in diff:
        srt = np.sort(ref_logits64[t])[::-1]
        gaps = np.abs(np.diff(srt))
        assert gaps.min() <= 2 * tol_abs, f"token {t}: routing differs with no near-tie"
    return len(diff)
