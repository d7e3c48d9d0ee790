"""The bench's FLOP/byte ledger against the figures the pages print."""
import json
import os

from dropless_grouped_gemm_amd import ledger as L

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ledger_figures.json")))


def test_fusedmoe_shape_figures():
    s = G["fusedmoe_shape"]
    T, d, de, E, k, b = s["T"], s["d"], s["d_e"], s["E"], s["k"], s["b"]
    rf = L.router_flops(T, d, E)
    assert round(rf / 1e9, 2) == G["router_gflop"]
    assert round(rf / L.router_bytes(T, d, E, b, logit_bytes=b), 1) == G["router_flop_per_byte"]
    assert L.pages_permute_bytes(T, k, d, b) / 2**20 == G["permute_mib"]
    assert round(L.expert_flops_per_row(d, de) * T * k / 1e12, 2) == G["grouped_gemm_tflop"]
    assert round(L.pages_grouped_gemm_bytes(T, k, E, d, de, b) / 1e9, 2) == G["grouped_gemm_gb_decimal"]
    assert L.pages_permute_plus_combine_bytes(T, k, d, b) / 2**30 == G["permute_plus_combine_gib"]
    # the minimal counts used by the bench are never above the pages' counts
    assert L.permute_bytes(T, k, d, b) <= L.pages_permute_bytes(T, k, d, b)
    assert L.gateup_flops(T * k, d, de) + L.down_flops(T * k, d, de) == L.expert_flops_per_row(d, de) * T * k


def test_per_card_figures():
    s = G["per_card_shape"]
    d, de, b = s["d"], s["d_e"], s["b"]
    assert round(L.expert_flops_per_row(d, de) / 1e6, 2) == G["mflop_per_row"]
    for rows, tf in G["tflop_by_rows"].items():
        assert round(L.expert_flops_per_row(d, de) * int(rows) / 1e12, 3) == tf
    for name, (r, c, gib) in G["gib_by_tensor"].items():
        assert round(r * c * b / 2**30, 2) == gib, name
