"""Host logic of the profile summaries: counter scaling by the copy probe, and the
benchmark's rule that a traffic figure taken from another kernel source is dropped."""
import csv
import json
import os

from dropless_grouped_gemm_amd import profsum as PS


def _counter_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, v in rows:
            w.writerow([name, counter, v])


def test_short_name_drops_parameters_keeps_templates():
    assert PS.short_name("void moe::k_gg_bf16_v2<0, false>(unsigned short const*, int)") == \
        "moe::k_gg_bf16_v2<0, false>"
    assert PS.short_name("void at::native::(anonymous namespace)::f<int>(int)") == \
        "at::native::{anon}::f<int>"
    assert PS.short_name("moe::k_select(float const*, int)") == "moe::k_select"


def test_traffic_scaled_by_probe_and_tied_to_source(tmp_path):
    probe = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(x)>(int)"
    kern = "void moe::k_gg_bf16_v2<0, false>(unsigned short const*)"
    # the probe reads 1 GiB but FETCH_SIZE shows half of it; writes are counted in full
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [(probe, 524288), (kern, 1000), (kern, 3000)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [(probe, 1048576), (kern, 10), (kern, 30)])
    text = PS.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "k_gg_bf16_v2<0, false>",
                              "gateup", "wl", "cmd")
    blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert blob["fetch_bytes"] == 2000 * 1024 * 2.0
    assert blob["write_bytes"] == 20 * 1024 * 1.0
    assert blob["bytes_per_launch"] == blob["fetch_bytes"] + blob["write_bytes"]
    p = tmp_path / "s.md"
    p.write_text(text)
    assert PS.read_traffic(str(p), "gateup", "wl") == blob["bytes_per_launch"]
    assert PS.read_traffic(str(p), "down", "wl") is None
    assert PS.read_traffic(str(p), "gateup", "other") is None
    p.write_text(text.replace(blob["source_sha256"], "0" * 64))
    assert PS.read_traffic(str(p), "gateup", "wl") is None
    assert PS.read_traffic(str(tmp_path / "missing.md"), "gateup", "wl") is None
