"""The benchmark's host-side reporting: the overlap model it prints beside each measurement, the
per-workload statistics, and the refusal of more than one GPU (all on the CPU, no GPU call)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_overlap_model_of_a_link_bound_decode_step():
    # 8 sequences of 32768 past keys, bf16: 1 GiB of host reads at 50 GB/s is 21.47 ms; the
    # compute at the MFMA peak adds only one tile's worth
    past = np.full(8, 32768, dtype=np.int32)
    host = 8 * 8 * 32768 * 2 * 256
    m = bench._overlap_model(1, past, host, 4.7e9, 2500.0, 21.5, 50.0)
    assert m["n_tiles"] == 513
    assert m["expected_ms"] == pytest.approx(host / 50e9 * 1e3, rel=1e-6)
    assert m["measured_over_expected"] == pytest.approx(21.5 / m["expected_ms"])
    assert bench._overlap_model(1, past, host, 4.7e9, 2500.0, 21.5, None) is None


def test_overlap_model_of_a_compute_bound_step():
    # with no host bytes the model is the compute time plus one tile's (zero) transfer
    past = np.zeros(1, dtype=np.int32)
    m = bench._overlap_model(8192, past, 0, 2.5e12, 2500.0, 2.0, 50.0)
    assert m["n_tiles"] == 128
    assert m["expected_ms"] == pytest.approx(1.0)


def test_prefill_and_decode_statistics_of_the_8b_workloads():
    w = synth.workload("llama8b_prefill_T8192_on_L24576_bf16")
    past = np.asarray(w.past, dtype=np.int32)
    st = bench._prefill_stats(w, past, 5.0, 55.0)
    assert st["host_read_bytes"] == 24576 * 8 * 2 * 256            # every past row, K and V, once
    assert st["host_write_bytes"] == 8192 * 8 * 2 * 256            # the new rows
    assert st["tok_per_s"] == pytest.approx(8192 / 5e-3)
    assert 0 < st["mfma_frac"] < 1 and st["overlap_model"]["expected_ms"] < 5.0
    wd = synth.workload("llama8b_decode_b8_L32768_bf16")
    pd = np.asarray(wd.past, dtype=np.int32)
    sd = bench._decode_stats(wd, pd, 19.3, 55.8)
    assert sd["host_read_bytes"] == 1 << 30
    assert sd["host_read_GBps"] == pytest.approx((1 << 30) / 19.3e-3 / 1e9)
    assert sd["frac_of_measured_read_peak"] == pytest.approx(sd["host_read_GBps"] / 55.8)


def test_prefill_roofline_from_kernel_timing():
    """achieved = the step's algorithmic attention flops per launch over the launches' mean
    duration; the 70B-shaped step is 2 x 4 * 128 * 64 * (16384 * 49152 + 16384 * 16385 / 2) flops."""
    w = synth.workload("llama70b_prefill_T16384_on_L49152_b2_bf16")
    past = np.asarray(w.past, dtype=np.int32)
    kern = {"prefill_attention": {"ms_per_step": 60.0, "launches_per_step": 32.0, "avg_launch_ms": 1.875}}
    r = bench._prefill_roofline(w, past, kern, "no_such_profile")
    flops = 2 * 4 * 128 * 64 * (16384 * 49152 + 16384 * 16385 / 2)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["algorithmic_flops_per_launch"] == pytest.approx(flops / 32)
    assert r["achieved"] == pytest.approx(flops / 60e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0)
    assert r["traffic"] is None                              # no counter summary for this name
    assert bench._prefill_roofline(w, past, {"prefill_attention": None}, "x") is None


def test_decode_roofline_from_kernel_timing():
    w = synth.workload("llama8b_decode_b8_L32768_bf16")
    past = np.asarray(w.past, dtype=np.int32)
    kern = {"decode_attention": {"ms_per_step": 19.2, "launches_per_step": 1.0, "avg_launch_ms": 19.2}}
    r = bench._decode_roofline(w, past, kern, 56.0, "no_such_profile")
    assert r["bound"] == "host_link" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx((1 << 30) / 19.2e-3 / 1e9)
    assert r["frac_of_measured_read_peak"] == pytest.approx(r["achieved"] / 56.0)
    assert r["algorithmic_bytes_per_launch"] == (1 << 30) + 8 * 8 * 2 * 256


def test_counter_summary_is_gated_on_the_kernel_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "wl_counters.txt").write_text("# comment\nkernel_source_sha1: abc\nattn_fetch_plus_write_bytes_per_launch: 1.5e9\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_counter_summary("wl", "abc")["attn_fetch_plus_write_bytes_per_launch"] == "1.5e9"
    assert bench.read_counter_summary("wl", "def") is None
    assert bench.read_counter_summary("other", "abc") is None


def test_counters_summary_means_per_dispatch(tmp_path, capsys):
    f = tmp_path / "c.csv"
    f.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
                 "1,kA(int),FETCH_SIZE,10\n1,kA(int),FETCH_SIZE,20\n2,kA(int),FETCH_SIZE,30\n"
                 "3,kB,WRITE_SIZE,4\n")
    bench.counters_summary([str(f)])
    import json
    out = json.loads(capsys.readouterr().out)
    assert out["kA"]["dispatches"] == 2 and out["kA"]["FETCH_SIZE"] == pytest.approx(30.0)
    assert out["kB"]["WRITE_SIZE"] == pytest.approx(4.0)


def test_cpu_baseline_uses_the_threaded_c_oracle():
    import bench
    r = bench.cpu_baseline_prefill("tiny_f32_prefill128_decode1", n_tokens=8)
    assert r["kind"] == "oracle" and r["unit"] == "prefill tok/s per layer"
    assert r["cores"] == bench._oracle_threads() >= 1
    assert r["value"] > 0 and "C oracle" in r["sample"] and r["cpu_model"]
