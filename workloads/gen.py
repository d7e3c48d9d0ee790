"""Seeded input generators.

Every tensor is drawn from one ``torch.Generator`` seeded with the config's seed,
in a fixed order, on the requested device.  The same seed on the same device type
gives byte-identical tensors; the CPU oracle always receives host copies of
whatever the device side used, so the two sides never need to agree on a random
stream.

Value distributions (the stated recipe of each workload):
  x ~ N(0, 1); W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/d_e) (i.e. N(0, 1/fan_in));
  W_g ~ N(0, 1/d), so router logits are ~N(0, 1); shared-expert weights likewise.
  Router bias recipes are described in ``workloads.configs.MoEConfig``.
  Fixed routing: the multiset of expert ids with the given counts is shuffled by a
  seeded permutation and laid out as [T, k]; slot weights are Dirichlet(1, ..., 1)
  per token, drawn as normalised Exp(1) variables.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import MoEConfig


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor                       # [T, d]
    w_gate: Optional[torch.Tensor]        # [d, E]      (None when routing is fixed)
    bias: Optional[torch.Tensor]          # [E] fp32    (None: no bias)
    w1: torch.Tensor                      # [E, d, d_e] gate projection
    w3: torch.Tensor                      # [E, d, d_e] up projection
    w2: torch.Tensor                      # [E, d_e, d] down projection
    ws1: Optional[torch.Tensor] = None    # [d, d_e_shared]
    ws3: Optional[torch.Tensor] = None    # [d, d_e_shared]
    ws2: Optional[torch.Tensor] = None    # [d_e_shared, d]
    topk_idx: Optional[torch.Tensor] = None   # [T, k] int32 (fixed routing only)
    topk_w: Optional[torch.Tensor] = None     # [T, k] fp32  (fixed routing only)


def _normal(g, shape, std, dtype, device, chunk_elems=1 << 26):
    """N(0, std^2) drawn in fp32 and rounded once to ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        v = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        flat[s:e].copy_(v)
    return out


def make_inputs(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> MoEInputs:
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed if seed is None else seed)
    dt = torch_dtype(cfg.dtype)
    T, d, E, k, de = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_e

    x = _normal(g, (T, d), 1.0, dt, device)

    w_gate = bias = topk_idx = topk_w = None
    if cfg.fixed_counts is None:
        w_gate = _normal(g, (d, E), 1.0 / math.sqrt(d), dt, device)
        if cfg.bias == "hot":
            hot = int(torch.randint(0, E, (1,), generator=g, device=device).item())
            bias = torch.zeros(E, dtype=torch.float32, device=device)
            bias[hot] = cfg.bias_value
        elif cfg.bias == "normal":
            bias = torch.randn(E, generator=g, device=device, dtype=torch.float32) * cfg.bias_value
        elif cfg.bias == "zipf":
            ranks = torch.randperm(E, generator=g, device=device).to(torch.float64) + 1.0
            b = -cfg.bias_value * torch.log(ranks)
            b[ranks > E - cfg.n_dead] = -30.0
            bias = b.to(torch.float32)
        elif cfg.bias != "none":
            raise ValueError(cfg.bias)
    else:
        counts = list(cfg.fixed_counts)
        if len(counts) != E or sum(counts) != T * k:
            raise ValueError("fixed_counts must have E entries summing to T*k")
        ids = torch.repeat_interleave(torch.arange(E, device=device, dtype=torch.int32),
                                      torch.tensor(counts, device=device))
        perm = torch.randperm(T * k, generator=g, device=device)
        topk_idx = ids[perm].view(T, k).contiguous()
        u = torch.rand((T, k), generator=g, device=device, dtype=torch.float64)
        ex = -torch.log1p(-u)                      # Exp(1)
        topk_w = (ex / ex.sum(dim=1, keepdim=True)).to(torch.float32).contiguous()

    w1 = torch.empty((E, d, de), dtype=dt, device=device)
    w3 = torch.empty((E, d, de), dtype=dt, device=device)
    w2 = torch.empty((E, de, d), dtype=dt, device=device)
    for e in range(E):
        w1[e].copy_(_normal(g, (d, de), 1.0 / math.sqrt(d), dt, device))
        w3[e].copy_(_normal(g, (d, de), 1.0 / math.sqrt(d), dt, device))
        w2[e].copy_(_normal(g, (de, d), 1.0 / math.sqrt(de), dt, device))

    ws1 = ws3 = ws2 = None
    if cfg.d_e_shared:
        ds = cfg.d_e_shared
        ws1 = _normal(g, (d, ds), 1.0 / math.sqrt(d), dt, device)
        ws3 = _normal(g, (d, ds), 1.0 / math.sqrt(d), dt, device)
        ws2 = _normal(g, (ds, d), 1.0 / math.sqrt(ds), dt, device)

    return MoEInputs(cfg, x, w_gate, bias, w1, w3, w2, ws1, ws3, ws2, topk_idx, topk_w)
