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


def make_inputs(cfg: MoEConfig, device="cpu", seed: Optional[int] = None,
                expert_weights: bool = True) -> MoEInputs:
    """Every input of the workload.  expert_weights=False leaves w1, w3, w2 (and the
    shared expert's) as None and draws everything else exactly as with them (the
    weights come last in the stream), for runs that take their weights elsewhere."""
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

    if not expert_weights:
        return MoEInputs(cfg, x, w_gate, bias, None, None, None, None, None, None, topk_idx,
                         topk_w)

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


@dataclass
class Fp8Weights:
    """fp8 (e4m3) expert weights as codes plus one fp32 scale per 128 x 128 block, the
    inputs of the fp8-weight layer: q* uint8 in the bf16 weights' [E, K, N] layout,
    s* fp32 [E, ceil(K/128), ceil(N/128)]; the shared expert's without the E axis."""
    q1: torch.Tensor
    s1: torch.Tensor
    q3: torch.Tensor
    s3: torch.Tensor
    q2: torch.Tensor
    s2: torch.Tensor
    qs1: Optional[torch.Tensor] = None
    ss1: Optional[torch.Tensor] = None
    qs3: Optional[torch.Tensor] = None
    ss3: Optional[torch.Tensor] = None
    qs2: Optional[torch.Tensor] = None
    ss2: Optional[torch.Tensor] = None


FP8_CODE_STD = 64.0


def _fp8_matrix(g, lead, K, N, device):
    """Seeded codes and scales of lead matrices [K, N] (lead == 0: one matrix without
    the leading axis).  Codes: the e4m3 value nearest to a N(0, 64^2) draw (torch's own
    conversion; |draw| > 448 is clipped first), so codes span the format's range like
    those of a quantised Gaussian matrix.  Scales: U(0.75, 1.25) / (64 sqrt(K)), so the
    weights code * scale are ~N(0, 1/K) within a factor 1.25, as the bf16 recipe."""
    n = max(lead, 1)
    kb, nb = -(-K // 128), -(-N // 128)
    q = torch.empty((n, K, N), dtype=torch.uint8, device=device)
    for i in range(n):
        v = torch.randn((K, N), generator=g, device=device, dtype=torch.float32)
        v.mul_(FP8_CODE_STD).clamp_(-448.0, 448.0)
        q[i].copy_(v.to(torch.float8_e4m3fn).view(torch.uint8))
    u = torch.rand((n, kb, nb), generator=g, device=device, dtype=torch.float32)
    sc = (0.75 + 0.5 * u) / (FP8_CODE_STD * math.sqrt(K))
    if lead == 0:
        return q[0], sc[0].contiguous()
    return q, sc


def make_fp8_weights(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> Fp8Weights:
    """fp8 expert weights for the workload's shapes, from their own seeded stream
    (seed + 500 by default), so they do not depend on whether make_inputs drew the
    bf16 weights."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed((cfg.seed if seed is None else seed) + 500)
    d, E, de = cfg.d, cfg.E, cfg.d_e
    q1, s1 = _fp8_matrix(g, E, d, de, device)
    q3, s3 = _fp8_matrix(g, E, d, de, device)
    q2, s2 = _fp8_matrix(g, E, de, d, device)
    w = Fp8Weights(q1, s1, q3, s3, q2, s2)
    if cfg.d_e_shared:
        ds = cfg.d_e_shared
        w.qs1, w.ss1 = _fp8_matrix(g, 0, d, ds, device)
        w.qs3, w.ss3 = _fp8_matrix(g, 0, d, ds, device)
        w.qs2, w.ss2 = _fp8_matrix(g, 0, ds, d, device)
    return w
