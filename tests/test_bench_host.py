"""Host-side logic of bench.py, on the CPU: the algorithmic byte counts behind the roofline
figures, the guard that keeps a counter-based traffic figure to the kernel sources it was
measured on, the scaling of HBM counters by a plain copy of known size, and the one-GPU
limit of the command line."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench


def test_dense_bytes_decode_workload():
    # K=8192, N=28672, group 128: packed codes N*K/2 = 117,440,512 B, fp16 scale and zero
    # point 4*N*K/128 = 7,340,032 B, then per row K int8 codes, a 4-byte row scale and N fp32
    # outputs -- 124.90 / 125.76 / 126.75 MB for M = 1 / 8 / 16
    assert bench.dense_bytes(1, 28672, 8192) == 117_440_512 + 7_340_032 + 8192 + 4 + 4 * 28672
    mb = [round(bench.dense_bytes(m, 28672, 8192) / 1e6, 2) for m in (1, 8, 16)]
    assert mb == [124.90, 125.76, 126.75]


def test_dense_bytes_prefill_workload():
    # M=4096, K=N=8192: 203.4 MB, of which 134.2 MB is the fp32 output
    total = bench.dense_bytes(4096, 8192, 8192)
    assert round(total / 1e6, 1) == 203.4
    assert round(4 * 4096 * 8192 / 1e6, 1) == 134.2


def test_dense_bytes_group_sizes():
    # the scale/zp bytes halve with group 256 and double with group 64; nothing else changes
    base = bench.dense_bytes(8, 4096, 1024, group=128)
    assert bench.dense_bytes(8, 4096, 1024, group=64) - base == 4 * 4096 * 8
    assert base - bench.dense_bytes(8, 4096, 1024, group=256) == 4 * 4096 * 4


def test_quant_bytes():
    assert bench.quant_bytes(16, 8192) == 16 * 8192 * 4 + 16 * 8192 + 16 * 4


def _write_traffic(path, digest, value):
    with open(path, "w") as f:
        f.write("# HBM traffic of gemm_decode_kernel\n")
        f.write(f"kernel_sources_sha256: {digest}\n")
        f.write(f"traffic_bytes_per_launch: {value}\n")


def test_read_traffic_kept_only_for_the_measured_sources(tmp_path, monkeypatch):
    path = str(tmp_path / "traffic.txt")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.read_traffic() is None  # no summary
    _write_traffic(path, bench.kernel_digest(), 130006408)
    assert bench.read_traffic() == 130006408.0
    _write_traffic(path, "0" * 64, 130006408)
    assert bench.read_traffic() is None  # taken on other kernel sources


def test_committed_traffic_summary_matches_the_sources():
    # the committed summary is the one bench.py reports; it must describe the current kernels
    assert bench.read_traffic() is not None


def _write_counters(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, value) in enumerate(rows):
            f.write(f'{i},"{kernel}",{counter},{value}\n')


def test_summarize_traffic_scales_by_the_copy(tmp_path):
    # the copy of 512 MiB reads as 2x its size in FETCH_SIZE (factor 0.5) and as its size in
    # WRITE_SIZE (factor 1); the GEMM's raw KiB are scaled by those factors
    copy_kib = bench.COPY_BYTES / 1024.0
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    _write_counters(fetch, "FETCH_SIZE", [("void gemm_decode_kernel<4, 2>(...)", 250000.0),
                                          ("void gemm_decode_kernel<4, 2>(...)", 250002.0),
                                          ("__amd_rocclr_copyBuffer", 2 * copy_kib)])
    _write_counters(write, "WRITE_SIZE", [("void gemm_decode_kernel<4, 2>(...)", 1000.0),
                                          ("__amd_rocclr_copyBuffer", copy_kib)])
    text = bench.summarize_traffic(fetch, write, ["cmd"])
    kv = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith("#"))
    assert float(kv["fetch_scale"]) == pytest.approx(0.5)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(250001.0 * 1024 * 0.5 + 1000.0 * 1024, abs=1)
    alg = sum(bench.dense_bytes(m, bench.N_DEC, bench.K_DEC) for m in bench.M_DEC) / 3
    assert float(kv["algorithmic_bytes_per_launch"]) == pytest.approx(alg, abs=1)
    assert kv["kernel_sources_sha256"] == bench.kernel_digest()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("extra", [["--group", "64"], ["--path", "5"], []])
def test_tile_major_option_is_checked_before_any_gpu_work(extra):
    only = ["--only", "toy_moe"] if not extra else ["--only", "prefill"]
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), *only, "--tile-major", *extra],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--tile-major" in r.stderr
