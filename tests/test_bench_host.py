"""Host-side logic of bench.py (no GPU): work counts, rocprofv3 summaries,
the HBM traffic report and its calibration, and the one-GPU refusal."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pairs_by_loops(pos):
    doc = oracle.doc_ids(pos)
    n = len(pos)
    return sum(1 for i in range(n) for j in range(i + 1) if doc[i] == doc[j])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_useful_pairs_and_document_lengths(seed):
    pos = synth.random_positions(200, seed)
    assert bench.useful_pairs(pos) == _pairs_by_loops(pos)
    lengths = bench.doc_lengths_of(pos)
    assert lengths.sum() == 200
    assert len(lengths) == oracle.doc_ids(pos)[-1] + 1
    # a first token whose position id is not 0 still starts a document
    pos2 = np.array([3, 4, 0, 1], dtype=np.int32)
    assert bench.doc_lengths_of(pos2).tolist() == [2, 2]
    assert bench.useful_pairs(pos2) == 6


def test_million_share_counts():
    pos = synth.workload_positions("million")
    N = 1 << 20
    assert bench.useful_pairs(pos) == N * (N + 1) / 2 == 549756338176
    rd, wr = bench.relayout_bytes_per_step("million")
    # Q, K, V in and O out (bf16), then dO in and dQ, dK, dV out (fp32), 4 q / 1 KV heads of 128
    fwd = N * 128 * 2 * (4 + 1 + 1 + 4)
    bwd = N * 128 * (2 * 4 + 4 * 4 + 4 * 1 + 4 * 1)
    assert rd == wr == fwd + bwd == 6.5 * 2 ** 30
    assert bench.relayout_bytes_per_step("llama8b_1doc") == (0, 0)


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_summarize_rocprof_tables(tmp_path):
    d = tmp_path / "prof"
    _write_csv(str(d / "x" / "run_kernel_stats.csv"), [
        dict(Name="void ul::(anonymous namespace)::dkdv_kernel<128>(...)", Calls=1, TotalDurationNs=2.0e9,
             AverageNs=2.0e9, MinNs=2.0e9, MaxNs=2.0e9, Percentage=60.0),
        dict(Name="void at::native::elementwise_kernel<...>", Calls=3, TotalDurationNs=3.0e6, AverageNs=1.0e6,
             MinNs=1.0e6, MaxNs=1.0e6, Percentage=1.0)])
    rows = []
    for c, v in [("SQ_WAVE_CYCLES", 1000.0), ("SQ_WAIT_ANY", 250.0), ("SQ_INSTS_MFMA", 10.0),
                 ("SQ_INSTS_VALU", 37.0)]:
        rows.append(dict(Kernel_Name="dkdv_kernel<128>", Counter_Name=c, Counter_Value=v, Start_Timestamp=0,
                         End_Timestamp=2_000_000))
    _write_csv(str(d / "x" / "run_counter_collection.csv"), rows)
    text = bench.summarize_rocprof(str(d))
    assert "| dkdv_kernel | 1 | 2000.000 | 2000.000 | 2000.000 | 2000.000 | 60.00 |" in text
    assert "| torch:" in text  # input-generation kernels are listed, marked as torch's
    assert "| dkdv_kernel | 0.250 |" in text  # SQ_WAIT_ANY / SQ_WAVE_CYCLES
    assert "| dkdv_kernel | 3.70 |" in text  # SQ_INSTS_VALU / SQ_INSTS_MFMA


def test_traffic_report_calibrates_with_the_exchange_copy(tmp_path):
    rd, wr = bench.relayout_bytes_per_step("million")
    kib = 1024.0

    def counters(name, relayout_total, dkdv):
        rows = [dict(Kernel_Name="relayout_kernel", Counter_Name=name, Counter_Value=relayout_total / 8 / kib)
                for _ in range(8)]
        rows.append(dict(Kernel_Name="dkdv_kernel<128>", Counter_Name=name, Counter_Value=dkdv / kib))
        return rows

    fd, wd = tmp_path / "f", tmp_path / "w"
    # FETCH_SIZE reads twice the bytes a copy moves, WRITE_SIZE exactly them
    _write_csv(str(fd / "run_counter_collection.csv"), counters("FETCH_SIZE", 2 * rd, 2 * 5.0e12))
    _write_csv(str(wd / "run_counter_collection.csv"), counters("WRITE_SIZE", wr, 1.0e9))
    text = bench.traffic_report("million", str(fd), str(wd))
    assert "FETCH_SIZE x 0.500, WRITE_SIZE x 1.000" in text
    import json
    import re

    blob = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    rec = blob["kernels"]["dkdv_kernel"]
    assert rec["fetch_bytes"] == pytest.approx(5.0e12)
    assert rec["write_bytes"] == pytest.approx(1.0e9)
    assert rec["source_sha256"] == bench._source_sha("dkdv_kernel")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one-GPU" in r.stderr and r.stdout == ""


def _smi_metric_json(power, clocks):
    clock = {f"gfx_{i}": {"clk": {"value": c, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                          "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED"}
             for i, c in enumerate(clocks)}
    clock["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    clock["vclk_0"] = "N/A"
    return json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": power, "unit": "W"},
                                                         "gfx_voltage": "N/A"}, "clock": clock}]})


def test_power_clock_parsing():
    """Board power and the mean graphics clock over the XCDs from amd-smi's JSON; memory clocks are ignored."""
    p, c = bench.parse_smi_metric(_smi_metric_json(1309, [1834, 1763, 1833, 1720, 1873, 1776, 1882, 1798]))
    assert p == 1309.0 and c == pytest.approx(1809.875)
    p, c = bench.parse_smi_metric(_smi_metric_json("N/A", []))
    assert p is None and c is None
    listing = json.dumps([{"gpu": 0, "bdf": "0000:05:00.0"}, {"gpu": 3, "bdf": "0000:F5:00.0"}])
    assert bench.smi_index_of("0000:f5:00", listing) == 3
    assert bench.smi_index_of("0000:75:00", listing) is None


def test_power_sampler_without_a_device_reports_nothing():
    """No PCI address (no GPU here): no polling thread, every summary field None, zero samples."""
    class _NoCuda:
        class cuda:
            @staticmethod
            def get_device_properties(i):
                raise RuntimeError("no GPU")

    s = bench.PowerSampler(_NoCuda)
    with s:
        pass
    out = s.summary()
    assert out["samples"] == 0 and out["board_power_w"] is None and out["gfx_clock_mhz"] is None


def test_power_sampler_starts_no_process_under_rocprofv3(monkeypatch):
    """Inside a rocprofv3 run (ROCPROF_* in the environment) the sampler starts no amd-smi process at all,
    even with a device present: the profiler's preload would make amd-smi's `env` exec from a process that
    has initialised the GPU."""
    class _Props:
        pci_domain_id, pci_bus_id, pci_device_id = 0, 0x75, 0

    class _Cuda:
        class cuda:
            @staticmethod
            def get_device_properties(i):
                return _Props

    started = []
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: started.append(a) or (_ for _ in ()).throw(
        AssertionError("a process was started")))
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert bench.under_profiler()
    s = bench.PowerSampler(_Cuda)
    with s:
        pass
    assert started == [] and s.summary()["samples"] == 0
    assert not bench.under_profiler({"PATH": "/usr/bin", "HIP_VISIBLE_DEVICES": "0"})


def test_power_clock_context_scales_the_peak_by_the_clock():
    roof = {"bound": "mfma", "achieved": 1100.0}
    out = bench.power_clock_context({"samples": 3, "gfx_clock_mhz": 1800.0, "board_power_w": 1330.0}, roof)
    assert out["mfma_peak_at_clock_tflops"] == pytest.approx(1875.0)
    assert out["dominant_frac_at_clock"] == pytest.approx(1100.0 / 1875.0)
    out = bench.power_clock_context({"samples": 0, "gfx_clock_mhz": None, "board_power_w": None}, roof)
    assert out["mfma_peak_at_clock_tflops"] is None and out["dominant_frac_at_clock"] is None
    # one or two polls of a short timed region may see the board idle (163 MHz once gave a "fraction" of 6.5)
    out = bench.power_clock_context({"samples": 1, "gfx_clock_mhz": 163.0, "board_power_w": 255.0}, roof)
    assert out["mfma_peak_at_clock_tflops"] is None and out["dominant_frac_at_clock"] is None and out["note"]


def test_cpu_host_info_and_extrapolation():
    info = bench.cpu_host_info()
    assert info["affinity_cores"] >= 1
    assert set(info) == {"cpu_model", "affinity_cores", "blas"}
    # 2 s on 32768 tokens -> 2 * 32^2 s on 1M tokens, labelled as an extrapolation
    ex = bench.extrapolate_oracle(2.0, 32768, 1 << 20, 3.9407e15)
    assert ex["extrapolated"] is True
    assert ex["seconds"] == pytest.approx(2.0 * 1024)
    assert ex["value"] == pytest.approx(3.9407e15 / 2048.0 / 1e12)


def test_traffic_report_calibrates_with_the_plain_copy(tmp_path):
    kib, mib = 1024.0, 256
    known = mib * 2**20

    def counters(name, copy, dkdv):
        return [dict(Kernel_Name="void at::native::vectorized_elementwise_kernel<4, MulFunctor<float>>",
                     Counter_Name=name, Counter_Value=copy / kib),
                dict(Kernel_Name="dkdv_kernel<128>", Counter_Name=name, Counter_Value=dkdv / kib)]

    fd, wd = tmp_path / "f", tmp_path / "w"
    # FETCH_SIZE counts half of what the copy reads, WRITE_SIZE all of it
    _write_csv(str(fd / "run_counter_collection.csv"), counters("FETCH_SIZE", known / 2, 1.0e12))
    _write_csv(str(wd / "run_counter_collection.csv"), counters("WRITE_SIZE", known, 1.0e9))
    text = bench.traffic_report("million", str(fd), str(wd), cal_mib=mib)
    assert "plain copy of known size in the same run" in text and "FETCH_SIZE x 2.000, WRITE_SIZE x 1.000" in text
    import json
    import re

    rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))["kernels"]["dkdv_kernel"]
    assert rec["fetch_bytes"] == pytest.approx(2.0e12) and rec["write_bytes"] == pytest.approx(1.0e9)


def test_counter_report_request_sizes_and_mfma_counts(tmp_path):
    w = synth.WORKLOADS["million"]
    pos = synth.workload_positions("million")
    tiles = bench.attention_tile_counts(pos, 4, w["N"])
    # one document of 2^20 tokens: column blocks cb see key tiles 0..cb, key blocks kb see 65536 - 8 kb tiles
    ncb, nkb = (w["N"] * 4) // 256, w["N"] // 128
    assert tiles["fwd_dq"] == ncb * (ncb + 1) // 2
    assert tiles["dkdv"] == sum(65536 - 8 * kb for kb in range(nkb))
    rows = []

    def add(kern, c, v, n=1):
        for _ in range(n):
            rows.append(dict(Kernel_Name=kern, Counter_Name=c, Counter_Value=v / n))

    # relayout: 1000 x 128-byte and 10 x 32-byte reads, 500 x 64-byte writes
    add("relayout_kernel", "TCC_EA0_RDREQ_sum", 1010, 8)
    add("relayout_kernel", "TCC_EA0_RDREQ_32B_sum", 10, 8)
    add("relayout_kernel", "TCC_BUBBLE_sum", 1000, 8)
    add("relayout_kernel", "TCC_EA0_WRREQ_sum", 500, 8)
    add("relayout_kernel", "TCC_EA0_WRREQ_64B_sum", 500, 8)
    pred = tiles["dkdv"] * 256
    add("dkdv_kernel<128>", "SQ_INSTS_MFMA", pred, 32)
    add("dkdv_kernel<128>", "SQ_INSTS_VALU_MFMA_MOPS_BF16", pred * 64, 32)
    _write_csv(str(tmp_path / "a" / "run_counter_collection.csv"), rows)
    text = bench.counter_report("million", [str(tmp_path / "a")])
    assert f"| relayout_kernel | 8 | 1010 | 10 | 0 | 1000 | - | {(1000 * 128 + 320) / 2**30:.3f} |" in text
    assert f"| relayout_kernel | 8 | 500 | 500 | - | {500 * 64 / 2**30:.3f} |" in text
    line = [ln for ln in text.splitlines() if ln.startswith("| dkdv_kernel |")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "32" and cells[4] == "1.0000" and cells[7] == "1.0000"
