"""Host-side checks of bench.py: the one-GPU contract, the algorithmic byte
counts the reported bandwidth divides by, and the folding of rocprofv3
counter runs into the committed traffic summary.  No GPU needed."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_closed_forms():
    # 4-bit: N K / 2 packed nibbles + G N fp16 scales + G N / 2 zero bytes + x + y.
    M, N, K, g = 1, 7168, 5120, 128
    G = K // g
    assert bench.alg_bytes(M, N, K, g) == N * K // 2 + G * N * 2 + G * N // 2 + M * K * 2 + M * N * 4
    # Bytes per weight: 0.5 + 2.5 / 128.
    big = bench.alg_bytes(0, 1 << 12, 1 << 12, 128)
    assert big / (1 << 24) == pytest.approx(0.5 + 2.5 / 128)
    # Ternary: 2 bits per weight + fp16 scales; MXFP4: 4 bits + one byte per 32.
    assert bench.w2t_bytes(0, 4096, 4096, 128) / (1 << 24) == pytest.approx(0.25 + 2 / 128)
    assert bench.mx_bytes(0, 4096, 4096) / (1 << 24) == pytest.approx(0.5 + 1 / 32)
    # The 64-layer sweep the headline divides by.
    layer = sum(bench.alg_bytes(1, N_, K_, 128) for (_, K_, N_) in bench.SHAPES)
    assert layer * 64 == pytest.approx(11.0e9, rel=0.01)


def test_kernel_key_normalises_profiler_and_variant_names():
    prof = "void (anonymous namespace)::w4_gemv_kernel<false, 4, 5, 3, false>(unsigned short const*, ...)"
    var = "w4_mfma16 f16 g128 kernel=w4_gemv_kernel<false, 4, 5, 3> tiles=2176"
    assert bench.kernel_key(prof) == bench.kernel_key(var) == "w4_gemv_kernel<false, 4, 5, 3>"
    assert bench.kernel_key("w4_gemv_kernel<true, 4, 5, 1, true>") == "w4_gemv_kernel<true, 4, 5, 1, true>"
    # Six arguments: MXFP4 mode and per-unit x staging.
    assert bench.kernel_key("void (anonymous namespace)::w4_gemv_kernel<false, 4, 17, 1, false, false>(int)") \
        == "w4_gemv_kernel<false, 4, 17, 1>"
    px = "w4_gemv_kernel<false, 4, 5, 3, false, true>"
    assert bench.kernel_key("void (anonymous namespace)::" + px + "(int)") == px
    assert bench.kernel_key("w4_mfma16 f16 g128 kernel=" + px + " tiles=2176") == px
    assert bench.kernel_key("w16_gemv_kernel<false, 1>") == "w16_gemv_kernel<false, 1>"
    assert bench.kernel_key("w16_mfma16 f16 kernel=w16_ksplit_kernel<false> tiles=448") == \
        "w16_ksplit_kernel<false>"
    assert bench.kernel_key("w16_dot f16 kernel=w16_dot_kernel<false, 1> tiles=320") == \
        "w16_dot_kernel<false, 1>"
    assert bench.kernel_key("__amd_rocclr_copyBuffer") is None
    # Trailing default template arguments (MX, PX, balanced plan = false)
    # are dropped; a set one keeps those before it.
    assert bench.kernel_key("w4_gemv_kernel<false, 4, 5, 3, false, true, false>") == \
        "w4_gemv_kernel<false, 4, 5, 3, false, true>"
    assert bench.kernel_key("w4_gemv_kernel<false, 4, 17, 1, false, false, false>") == "w4_gemv_kernel<false, 4, 17, 1>"
    bal = "w4_gemv_kernel<false, 4, 17, 1, false, false, true>"
    assert bench.kernel_key("void (anonymous namespace)::" + bal + "(int)") == bal


# gate_up's instantiation at M = 1: three tiles per workgroup, x staged unit by unit.
GATE_UP = "w4_gemv_kernel<false, 4, 5, 3, false, true>"


def test_committed_traffic_summary_is_consistent():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert {"fetch", "write"} <= set(t["calibration"])
    assert 1.9 < t["calibration"]["fetch"]["factor"] < 2.1      # FETCH_SIZE counts half
    assert 0.95 < t["calibration"]["write"]["factor"] < 1.05
    # Each instantiation of the sweep moves about its algorithmic bytes.
    alg = {GATE_UP: bench.alg_bytes(1, 34816, 5120, 128),
           "w4_gemv_kernel<false, 4, 17, 1, false, false, true>": bench.alg_bytes(1, 5120, 17408, 128)}
    for k, a in alg.items():
        ratio = t["kernels"][k]["bytes_per_dispatch"] / a
        assert 1.0 <= ratio < 1.03, (k, ratio)
    # The bench reports it only while the kernel source is the profiled one.
    got = bench.load_traffic(GATE_UP)
    if t["kernel_source_sha256_16"] == bench.kernel_source_hash():
        assert got == t["kernels"][GATE_UP]["bytes_per_dispatch"]
    else:
        assert got is None


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
        for i, (name, kib) in enumerate(rows):
            f.write(f'{i},"{name}",256,{counter},{kib}\n')


def test_ingest_pmc_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    # The 1 GiB copy counted as 512 MiB fetched -> factor 2; writes count true.
    gemv = "void (anonymous namespace)::w4_gemv_kernel<false, 4, 5, 3, false>(int)"
    copy = "__amd_rocclr_copyBuffer"
    f_csv, w_csv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f_csv, "FETCH_SIZE", [(copy, 512 * 1024), (gemv, 1000.0), (gemv, 1002.0)])
    _counter_csv(w_csv, "WRITE_SIZE", [(copy, 1024 * 1024), (gemv, 10.0), (gemv, 10.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.ingest_pmc(str(f_csv), str(w_csv), "test command")
    t = json.loads(out.read_text())
    k = t["kernels"]["w4_gemv_kernel<false, 4, 5, 3>"]
    assert k["dispatches"] == [2, 2]
    assert k["fetch_bytes_per_dispatch"] == round(1001.0 * 1024 * 2)
    assert k["write_bytes_per_dispatch"] == 10 * 1024
    assert k["bytes_per_dispatch"] == round(1001.0 * 1024 * 2 + 10 * 1024)
    assert t["command"] == "test command"


def test_headline_is_the_last_line_and_small(capsys, tmp_path):
    # A result shaped like a real run, with a large `extra` block: the last
    # stdout line is the compact headline, which parses and stays small; the
    # detail goes to a file.
    shape = {"us": 17.8, "GBps": 5206.6, "bytes": 92760064, "kernel": "k", "variant": "v" * 150}
    extra = {"pct_of_peak": 50.5, "bw_probe_GBps": 6331.0, "value_pct_of_probe": 63.8,
             "m1_per_shape": {n: dict(shape) for n in ("qkv", "o_proj", "gate_up", "down")},
             "m4_sweep": {"ms_per_token": 2.9, "pct_of_peak": 47.4,
                          "per_shape": {n: dict(shape) for n in ("qkv", "o_proj", "gate_up", "down")}},
             "skinny_sweep": [dict(shape, M=m) for m in range(200)]}
    result = {"metric": "m", "value": 4039.0, "unit": "GB/s", "n_gpus": 1, "steps": 20, "warmup": 3,
              "ms_per_step": 2.72, "dtype": "f16", "config": {"workload": "w"},
              "roofline": {"bound": "hbm", "achieved": 5206.6, "peak": 8000.0, "unit": "GB/s",
                           "frac": 0.6508, "traffic": 93053843},
              "cpu_baseline": {"value": 0.7, "unit": "GB/s", "cores": 16, "kind": "oracle",
                               "sample": "s"}}
    out = tmp_path / "sub" / "extra.json"
    bench.emit(result, extra, str(out))
    cap = capsys.readouterr()
    last = cap.out.strip().splitlines()[-1]
    assert len(last.encode()) <= bench.HEADLINE_MAX_BYTES
    head = json.loads(last)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "ms_per_step", "dtype", "config",
                "roofline", "cpu_baseline"):
        assert key in head
    assert "extra" not in head
    assert head["summary"]["m4_us"]["gate_up"] == 17.8
    assert json.loads(out.read_text())["skinny_sweep"][199]["M"] == 199
    assert len(cap.err) < 200
