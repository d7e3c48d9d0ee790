"""The five MoE-layer workloads, each a seeded synthetic stand-in for a shape the
pages discuss.

Shapes come from:
  * the TileLang fusedmoe default shape (T=8192, d=7168, d_e=2048, E=8, k=4),
    "MoE operators" chapter of the TileLang tutorial, section 1.2;
  * the per-GPU expert-parallel share with received rows 21,733 / 15,004 /
    17,982 / 10,817 for 4 local experts, "Dropless and grouped GEMM" notes,
    section 1 (table of received rows) and section 3 (padding table);
  * DeepSeek-V3 decode: 256 routed experts in 8 groups with at most 4 groups per
    token, top-8, one shared expert, TileLang chapter section 2.2 and the
    dropless notes sections 1, 4 and 10;
  * the skewed-routing simulation (8 experts, 128 assignments, block_M=32),
    TileLang chapter section 2.3.
"""
from __future__ import annotations

from dataclasses import dataclass, replace, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                     # tokens
    d: int                     # hidden size
    E: int                     # routed experts
    k: int                     # experts per token
    d_e: int                   # expert inner size (SwiGLU)
    block_m: int               # padding multiple = grouped-GEMM row granularity
    dtype: str                 # "bf16" or "fp32" for x / weights / out
    d_e_shared: int = 0        # 0: no shared expert
    n_groups: int = 0          # 0: no group-limited routing
    topk_groups: int = 0
    renormalize: bool = False
    seed: int = 0
    # router logit bias recipe: "none", "hot" (one hot expert), "normal" (N(0, bias_std^2)),
    # "zipf" (bias_e = -s*ln(rank_e), with the n_dead lowest-ranked experts at -30)
    bias: str = "none"
    bias_value: float = 0.0    # "hot": the hot expert's bias; "normal": std; "zipf": s
    n_dead: int = 0
    # fixed routing (router bypassed): per-expert row counts; ids shuffled, weights Dirichlet(1)
    fixed_counts: Optional[Tuple[int, ...]] = None
    # row layout: padded segments (False) or unpadded segments with per-expert entries
    # for tiles that straddle an expert boundary (True)
    unpadded: bool = False
    description: str = ""

    @property
    def M(self) -> int:
        """Number of (token, slot) assignments."""
        return self.T * self.k

    def scaled(self, **kw) -> "MoEConfig":
        """A smaller variant with the same recipe (used by parity tests)."""
        if "fixed_counts" not in kw and self.fixed_counts is not None and "T" in kw:
            raise ValueError("fixed-count configs must give fixed_counts when T changes")
        return replace(self, name=kw.pop("name", self.name + "-scaled"), **kw)


C1 = MoEConfig(
    name="tiny-fp32", T=64, d=256, E=8, k=2, d_e=512, block_m=32, dtype="fp32",
    renormalize=True, seed=1000, bias="hot",
    # With logits ~N(0,1), an expert whose logit carries +1.5 lands in the top-2 of 8
    # for about 75% of tokens (a Gaussian order-statistics estimate), i.e. about 48 of
    # 128 assignments: 3x the mean of 16.
    bias_value=1.5,
    description="Tiny dropless MoE layer, fp32, T=64, k=2, E=8, d=256, d_e=512, block_M=32, "
                "one hot expert at ~3x the mean, renormalised top-2, no shared expert")

C2 = MoEConfig(
    name="fusedmoe-8x2048", T=8192, d=7168, E=8, k=4, d_e=2048, block_m=128, dtype="bf16",
    d_e_shared=2048, seed=1001, bias="normal", bias_value=0.5,
    description="T=8192, d=7168, E=8, k=4, d_e=2048 SwiGLU + 1 shared expert (d_e=2048), "
                "bf16 with fp32 accumulate, padding 128, softmax top-4")

C3 = MoEConfig(
    name="ep-share-4x2048", T=8192, d=7168, E=4, k=8, d_e=2048, block_m=128, dtype="bf16",
    seed=1002, fixed_counts=(21733, 15004, 17982, 10817),
    description="One GPU's expert-parallel share: 4 local experts with 21,733/15,004/17,982/"
                "10,817 rows (65,536 -> 65,792 padded), d=7168, d_e=2048, router bypassed")

C4 = MoEConfig(
    name="decode-256x2048", T=64, d=7168, E=256, k=8, d_e=2048, block_m=128, dtype="bf16",
    d_e_shared=2048, n_groups=8, topk_groups=4, seed=1003,
    description="Small-M decode: T=64, E=256 in 8 groups, top-4 groups then top-8, "
                "d=7168, d_e=2048 + 1 shared expert, weight-streaming")

C5 = MoEConfig(
    name="zipf-skew-64x1408", T=16384, d=2048, E=64, k=6, d_e=1408, block_m=128, dtype="bf16",
    renormalize=True, seed=1004, bias="zipf", bias_value=1.2, n_dead=4,
    description="Heavy skew: T=16384, E=64, k=6, d=2048, d_e=1408, Zipf(1.2) expert "
                "popularity with 4 zero-row experts, renormalised top-6")

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}
ORDERED = (C1, C2, C3, C4, C5)


def get_config(name_or_index) -> MoEConfig:
    if isinstance(name_or_index, int):
        return ORDERED[name_or_index]
    return CONFIGS[name_or_index]
