"""Host-side logic of bench.py (CPU only): the algorithmic byte counts behind the headline rate, the visible-slot
count, the reduction of rocprofv3 counter runs into HBM bytes per launch, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_diffusion_drafter_02_amd import synth  # noqa: E402


def test_headline_bytes_per_step():
    """Real dims, bf16 weights and ring, ring full at n_past 2048: every weight once, the 2047 ring slots that some
    block row can see (K and V, all layers and kv heads), the norm vectors, 16 embedding rows, the logits."""
    E, F, V, L, D, Hq, Hkv = 6656, 19968, 8192, 5, 128, 32, 8
    per_layer = (Hq * D + 2 * Hkv * D) * E + E * Hq * D + 2 * F * E + E * F
    weights = (L * per_layer + V * E) * 2
    ring = L * Hkv * 2047 * D * 2 * 2
    other = (L * (2 * E + 2 * D) + E) * 4 + 16 * E * 2 + 16 * V * 4 + 15 * 4
    b = bench.step_bytes(synth.REAL, "bf16", "bf16", [bench.visible_slots(2048, 2048, 16)])
    assert b["weights"] == weights == 4_777_836_544
    assert b["ring"] == ring == 41_922_560
    assert b["total"] == weights + ring + other == 4_820_794_428


def test_fp8_bytes_add_row_scales():
    b8 = bench.step_bytes(synth.REAL, "fp8", "bf16", [2047])
    b16 = bench.step_bytes(synth.REAL, "bf16", "bf16", [2047])
    E, F, V, L, D, Hq, Hkv = 6656, 19968, 8192, 5, 128, 32, 8
    rows = L * (Hq * D + 2 * Hkv * D + E + 2 * F + E) + V
    assert b8["weights"] == b16["weights"] // 2 + 4 * rows


@pytest.mark.parametrize("n_past,window", [(0, 64), (1, 64), (40, 64), (64, 64), (80, 64), (2048, 2048), (2300, 2048)])
def test_visible_slots_by_brute_force(n_past, window):
    held = range(max(0, n_past - window), n_past)  # positions the ring holds after injecting 0..n_past-1 in order
    seen = {p for p in held for i in range(16) if 0 <= n_past + i - p < window}
    assert bench.visible_slots(n_past, window, 16) == len(seen)


def _write_counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_reduction(tmp_path, monkeypatch):
    """Five 1 GiB copies that count half their bytes on FETCH_SIZE and all on WRITE_SIZE calibrate the factors
    (2 and 1); the gate/up dispatches' mean then scales to bytes. Small copies and other kernels are ignored."""
    gu = f"void {bench.GU_KERNEL}(GemvArgs)"
    cp = bench.COPY_KERNEL
    big = 1 << 20  # KiB in 1 GiB
    fetch = [(gu, "FETCH_SIZE", 1000.0), (gu, "FETCH_SIZE", 1200.0), ("other_kernel", "FETCH_SIZE", 5.0)]
    fetch += [(cp, "FETCH_SIZE", big / 2)] * 5 + [(cp, "FETCH_SIZE", 0.03)] * 7
    write = [(gu, "WRITE_SIZE", 10.0), (gu, "WRITE_SIZE", 30.0)] + [(cp, "WRITE_SIZE", float(big))] * 5
    _write_counter_csv(str(tmp_path / "f" / "sub"), fetch)
    _write_counter_csv(str(tmp_path / "w"), write)
    out_file = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS", str(out_file))
    out = bench.write_counters(str(tmp_path / "f"), str(tmp_path / "w"), 1024, ["cmd a", "cmd b"])
    assert out["calibration"]["fetch_factor"] == 2.0 and out["calibration"]["write_factor"] == 1.0
    assert out["hbm_bytes_per_launch"] == int((1100.0 * 2 + 20.0) * 1024)
    assert out["kernel_src_sha256_16"] == bench.kernel_src_hash()
    assert json.loads(out_file.read_text())["hbm_bytes_per_launch"] == out["hbm_bytes_per_launch"]
    # the stored figure is what bench reports while the kernel sources are unchanged
    assert bench.read_traffic(0) == out["hbm_bytes_per_launch"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_trace_summary_spans_and_non_gemm_share(tmp_path):
    """Three block steps of a synthetic kernel trace (embed, a projection, attention, combine, a projection;
    then a host-loop copy) after one setup kernel: spans run from each step's first kernel to the end of its
    last one, copies are not counted, and the non-GEMM share is attention + combine + embed over all."""
    path = tmp_path / "t"
    os.makedirs(path)
    rows, t = [("tile_weights_kernel(x)", 0, 50)], 100
    for _ in range(3):
        for name, d in (("embed_kernel(EmbedArgs)", 5), ("void gemv_kernel<1>(GemvArgs)", 20),
                        ("void attn_partial_kernel<128>(AttnArgs)", 10), ("attn_combine_kernel(CombArgs)", 5),
                        ("void gemv_kernel<2>(GemvArgs)", 60), ("__amd_rocclr_copyBuffer", 2)):
            rows.append((name, t, t + d))
            t += d + 1
    with open(path / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, a, b in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": a * 1000, "End_Timestamp": b * 1000})
    out = bench.summarize_trace(str(path), skip_steps=0)
    assert out["steps"] == 2  # the last step has no following step start and is dropped
    assert out["span_us_median"] == 5 + 1 + 20 + 1 + 10 + 1 + 5 + 1 + 60
    assert out["non_gemm_share"] == round(20 / 100, 4)
    assert out["kernels"]["gemv_kernel<2>"]["us_per_step"] == 60
