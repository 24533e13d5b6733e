"""Host-side checks of the rocprofv3 summary code (no GPU): the copy-kernel
calibration arithmetic, the machine-readable traffic lines and the
source-digest guard that bench.py relies on."""
import csv
import os

from efficient_transformer_attention_mean_amd import profiling


def _write_counters(path, counter, values):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, vals in values.items():
            for v in vals:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>(int)"
ADD = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>, x>(int)"
APPLY = "void nys::k_apply<nys::BF16, 64, 4, 33, true>(nys::BF16::T const*, int)"


def test_traffic_scaling_and_guard(tmp_path):
    # The fetch counter reports half the bytes of the 256 MiB copy, the write
    # counter all of them: a kernel reading 1000 reported KiB read 2000 KiB.
    _write_counters(tmp_path / "f", "FETCH_SIZE", {FILL: [15.0], ADD: [131072.0, 131072.0], APPLY: [1000.0, 1000.0]})
    _write_counters(tmp_path / "w", "WRITE_SIZE", {FILL: [262144.0], ADD: [262144.0], APPLY: [500.0]})
    text = profiling.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "cmd-f", "cmd-w", "t")
    assert "scale factors 2.0000 (fetch) and 1.0000 (write)" in text
    assert "traffic_bytes_per_launch apply 2.56e+06" in text  # (2000 + 500) KiB
    out = tmp_path / "traffic.txt"
    out.write_text(text)
    assert profiling.read_traffic(str(out), "apply") == 2000 * 1024 + 500 * 1024
    assert profiling.read_traffic(str(out), "landmark_bv") is None
    # A summary made from other kernel sources is ignored.
    out.write_text(text.replace(profiling.sources_digest(), "0" * 64))
    assert profiling.read_traffic(str(out), "apply") is None
    assert profiling.read_traffic(str(tmp_path / "missing.txt"), "apply") is None


def test_stats_summary_and_names(tmp_path):
    p = tmp_path / "run_kernel_stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                          "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": APPLY, "Calls": 4, "TotalDurationNs": 4000, "AverageNs": 1000, "Percentage": 80,
                    "MinNs": 900, "MaxNs": 1100, "StdDev": 1})
        w.writerow({"Name": "void nys::k_segment_mean<nys::BF16, 64>(int)", "Calls": 4, "TotalDurationNs": 1000,
                    "AverageNs": 250, "Percentage": 20, "MinNs": 200, "MaxNs": 300, "StdDev": 1})
    text = profiling.stats_summary(str(p), "the command", "title")
    lines = [ln for ln in text.splitlines() if ln.startswith("| k_")]
    assert lines[0].startswith("| k_apply<BF16, 64, 4, 33, true> | 4 | 1.00 | 0.90 | 1.10 | 80.0% |")
    assert lines[1].startswith("| k_segment_mean<BF16, 64> | 4 | 0.25 |")
    assert profiling.family(APPLY) == "apply"
    assert profiling.family("void nys::k_pinv_planes<64, 64>(float const*)") == "pinv_planes"
    anon = "void nys::(anonymous namespace)::k_bwd_key_mm<64>(unsigned short const*, float const*)"
    assert profiling.short_name(anon) == "k_bwd_key_mm<64>"
    assert profiling.family(anon) == "bwd_key_mm"


def test_stats_mean_lookup_and_guard(tmp_path):
    p = tmp_path / "run_kernel_stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                          "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": APPLY, "Calls": 2, "TotalDurationNs": 44000, "AverageNs": 22000, "Percentage": 100,
                    "MinNs": 21000, "MaxNs": 23000, "StdDev": 1})
    out = tmp_path / "kernels.txt"
    out.write_text(profiling.stats_summary(str(p), "cmd", "t"))
    assert profiling.read_kernel_mean_us(str(out), "apply") == 22.0
    assert profiling.read_kernel_mean_us(str(out), "landmark_pass") is None
    out.write_text(out.read_text().replace(profiling.sources_digest(), "f" * 64))
    assert profiling.read_kernel_mean_us(str(out), "apply") is None


def test_counters_summary_derived_figures(tmp_path):
    # Two passes: SQ counters in one, L2 counters in the other; the derived
    # figures combine them per kernel.
    _write_counters(tmp_path / "a", "SQ_BUSY_CU_CYCLES", {APPLY: [1000.0, 1000.0]})
    with open(tmp_path / "a" / "run_counter_collection.csv", "a", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerow({"Kernel_Name": APPLY, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 800.0})
        w.writerow({"Kernel_Name": APPLY, "Counter_Name": "SQ_LDS_BANK_CONFLICT", "Counter_Value": 150.0})
        w.writerow({"Kernel_Name": APPLY, "Counter_Name": "SQ_INSTS_LDS", "Counter_Value": 50.0})
    _write_counters(tmp_path / "b", "TCC_HIT_sum", {APPLY: [30.0]})
    with open(tmp_path / "b" / "run_counter_collection.csv", "a", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerow({"Kernel_Name": APPLY, "Counter_Name": "TCC_MISS_sum", "Counter_Value": 10.0})
        w.writerow({"Kernel_Name": FILL, "Counter_Name": "TCC_MISS_sum", "Counter_Value": 10.0})
    text = profiling.counters_summary([(str(tmp_path / "a"), "cmd a"), (str(tmp_path / "b"), "cmd b")], "t",
                                      kernels="k_apply")
    assert "    cmd a" in text and "    cmd b" in text
    assert "## k_apply<BF16, 64, 4, 33, true>" in text and "FillFunctor" not in text
    assert "| MFMA busy (% of SIMD cycles while CUs busy) | 20 |" in text  # 800 / (4 x 1000)
    assert "| L2 hit rate (%) | 75 |" in text
    assert "| LDS bank-conflict cycles per LDS instruction | 3 |" in text
    assert "| LDS bank-conflict cycles (% of CU busy cycles) | 15 |" in text
