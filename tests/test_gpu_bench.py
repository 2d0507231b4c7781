"""bench.py end to end on MI355X, in a child process: one JSON line with the
fields its readers rely on, self-consistent, and a CPU baseline that agrees
with the GPU's first step."""
import json
import os
import subprocess
import sys

import pytest

import synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_consistent_json_line():
    print("case bench.py --steps 3 --warmup 1 --no-extras --cpu-seconds 1", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-extras", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    w = synth.WORKLOADS[synth.BENCH_WORKLOAD]

    assert d["unit"] == "Gparam/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["data"] == "synthetic" and d["dtype"] == "f32" and d["vs_baseline"] is None
    assert d["config"]["workload"] == w.name and d["config"]["params"] == w.numel
    assert d["config"]["replicas"] == w.replicas
    # value is the parameters updated per second over the timed region
    assert d["value"] == pytest.approx(w.numel / (d["ms_per_step"] / 1e3) / 1e9, rel=1e-9)

    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["algorithmic_bytes_per_launch"] == w.traffic_bytes == \
        (2 * w.replicas + 26) * w.numel
    assert rf["achieved"] == pytest.approx(
        w.traffic_bytes / (rf["mean_launch_ms"] / 1e3) / 1e9, rel=1e-9)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-12)
    assert 0.0 < rf["frac"] < 1.0
    assert rf["min_launch_ms"] <= rf["mean_launch_ms"] <= rf["max_launch_ms"]
    assert rf["traffic"] is None or rf["traffic"] > 0

    # the stream probe: the same bytes, measured on the same layer
    sp = d["stream_probe"]
    assert sp["gbs"] == pytest.approx(w.traffic_bytes / sp["ms"] / 1e6, rel=1e-9)
    assert rf["frac_of_stream_probe"] == pytest.approx(rf["achieved"] / sp["gbs"], rel=1e-9)
    assert 0.0 < sp["frac"] < 1.0

    # every workload, each with the update and the probe
    pw = d["per_workload"]
    assert set(pw) == set(synth.WORKLOADS)
    for name, e in pw.items():
        ww = synth.WORKLOADS[name]
        assert e["params"] == ww.numel and e["bytes_per_param"] == ww.bytes_per_param
        for k in ("update", "probe"):
            assert e[k]["gbs"] == pytest.approx(ww.traffic_bytes / e[k]["ms"] / 1e6, rel=1e-9)
            assert e[k]["gparams"] == pytest.approx(ww.numel / e[k]["ms"] / 1e6, rel=1e-9)
        if ww.with_flag:
            assert e["overflow_flag"] == 0
    assert "note" in pw["tiny"]

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert cb["unit"] == "Gparam/s" and cb["sample"]
    par = cb["parity_vs_gpu_first_step"]
    assert par["params"] > 0 and par["max_ulp"] <= 2 and par["bf16_mismatch"] == 0


def test_bench_extras_on_a_smaller_layer():
    """The extras (everything after the timed region) on the Qwen3-4B-shaped
    layer: present, and consistent with the byte model."""
    print("case bench.py --workload qwen3_4b_layer (extras)", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload",
                        "qwen3_4b_layer", "--steps", "3", "--warmup", "1", "--no-per-workload",
                        "--cpu-seconds", "1"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([x for x in r.stdout.splitlines() if x.strip()][-1])
    w = synth.WORKLOADS["qwen3_4b_layer"]
    x = d["extras"]
    for k in ("range_64MiB_chunks", "check_gradients", "check_then_gated_step",
              "fp16_compute_copy", "no_compute_copy", "host_us_per_call", "one_shard_of_g",
              "host_resident_state", "producer_overlap", "direction_split", "replica_sweep"):
        assert k in x, k
    assert set(x["replica_sweep"]) == {"1", "2", "4"}   # the 4B layer has R = 4
    for R, e in x["replica_sweep"].items():
        assert e["bytes_per_param"] == 2 * int(R) + 26
        for k in ("update", "probe"):
            assert e[k]["gbs"] == pytest.approx(e["bytes_per_param"] * w.numel / e[k]["ms"] / 1e6,
                                                rel=1e-9)
    ds = x["direction_split"]
    assert ds["read_bytes_per_param"] == 2 * w.replicas + 12
    assert ds["read_bytes_per_param"] + ds["write_bytes_per_param"] == w.bytes_per_param
    for k in ("reads_alone", "writes_alone", "at_once_two_streams"):
        assert ds[k]["ms"] > 0 and 0.0 < ds[k]["frac"] < 1.0, k
    assert ds["in_sequence"]["ms"] == pytest.approx(ds["reads_alone"]["ms"] +
                                                    ds["writes_alone"]["ms"], rel=1e-9)
    assert set(ds["alternating_phases"]) == {"1", "4", "16", "64"}
    rf = d["roofline"]
    assert rf["frac_of_mixed_reference"] == pytest.approx(
        rf["achieved"] / ds["at_once_two_streams"]["gbs"], rel=1e-9)
    for p in ("gemm", "host_link"):
        e = x["producer_overlap"][p]
        assert e["gradients_reproduced"] is True
        assert e["overlapped_ms"] > 0 and e["producer_ms"] > 0 and e["update_ms"] > 0
