"""Algorithmic FLOP and byte counts for the MoE layer forward pass.

These are the figures the roofline fractions are computed from: real rows only
(no FLOPs on pad rows) and every tensor counted once.  The pages' own ledgers
(TileLang MoE chapter sections 1.2, 2.2, 2.3, 2.6; dropless notes section 4) are
reproduced by the ``pages_*`` helpers so that the tests can pin the formulas to
the printed numbers; the bench uses the minimal counts.
"""
from __future__ import annotations


def router_flops(T, d, E):
    """logits = x[T, d] @ W_g[d, E]: one multiply-add per (t, i, e)."""
    return 2 * T * d * E


def router_bytes(T, d, E, b, logit_bytes=4):
    """Read x and W_g once, write fp32 logits."""
    return (T * d + d * E) * b + T * E * logit_bytes


def expert_flops_per_row(d, d_e):
    """gate, up and down projections of one row: 3 GEMMs of 2*d*d_e each."""
    return 6 * d * d_e


def gateup_flops(rows, d, d_e):
    return 4 * rows * d * d_e


def down_flops(rows, d, d_e):
    return 2 * rows * d_e * d


def gateup_bytes(rows, active_experts, d, d_e, b, wb=None):
    """Read the permuted rows and W1, W3 of every expert with rows once; write act.
    wb: bytes per weight (default b)."""
    wb = b if wb is None else wb
    return (rows * d + rows * d_e) * b + 2 * active_experts * d * d_e * wb


def gateup_gather_bytes(T, rows, active_experts, d, d_e, b, wb=None):
    """Gate/up with the permute fused into its loads: read each token row of x once (the
    k gathered copies are re-reads of it), W1 and W3 of every expert with rows once;
    write act."""
    wb = b if wb is None else wb
    return (T * d + rows * d_e) * b + 2 * active_experts * d * d_e * wb


def shared_gateup_bytes(T, d, d_es, b, reads_x=True, wb=None):
    """The shared expert's gate/up: x (unless the routed half already reads it), Ws1,
    Ws3; write its act."""
    wb = b if wb is None else wb
    return ((T * d if reads_x else 0) + T * d_es) * b + 2 * d * d_es * wb


def shared_down_bytes(T, d, d_es, b, wb=None):
    wb = b if wb is None else wb
    return (T * d_es + T * d) * b + d_es * d * wb


def fp8_scale_bytes(matrices, K, N, block=128):
    """fp32 scales of `matrices` fp8 weight matrices [K, N], one per block x block."""
    return matrices * (-(-K // block)) * (-(-N // block)) * 4


def down_bytes(rows, active_experts, d, d_e, b, wb=None):
    """Read act and W2 of every expert with rows once; write y."""
    wb = b if wb is None else wb
    return (rows * d_e + rows * d) * b + active_experts * d_e * d * wb


def permute_bytes(T, k, d, b):
    """Read each token row once, write its k copies."""
    return T * d * b + T * k * d * b


def combine_bytes(T, k, d, b, shared=False):
    """Read the k expert rows of each token (and the shared-expert row), write out."""
    return T * k * d * b + T * d * b + (T * d * b if shared else 0)


# ---- the pages' own ledger formulas (used only to pin against printed numbers) ----
def pages_permute_bytes(T, k, d, b):
    """TileLang chapter section 2.3: read T*k rows and write T*k rows."""
    return 2 * T * k * d * b


def pages_permute_plus_combine_bytes(T, k, d, b):
    """TileLang chapter section 2.6 item 1."""
    return 4 * T * k * d * b


def pages_grouped_gemm_bytes(T, k, E, d, d_e, b):
    """The printed 2.11 GB for the fusedmoe default shape fits three passes of
    (all expert weights + the T*k permuted rows); the page gives no formula."""
    return 3 * (E * d * d_e + T * k * d) * b
