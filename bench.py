"""Benchmark: the W4A8 decode layer (K=8192, N=28672, group 128, M = 1, 8 and 16
tokens) on one MI355X, plus the prefill and MoE workloads as secondary figures.

One step = per-token INT8 quantization of the activations followed by the W4A8
GEMM, for M = 1, 8 and 16 (three layer calls).  Inputs are resident in HBM before
the timed region.  The packed weights (124.9 MB with scale/zp) fit in the 256 MB
Infinity Cache, so the benchmark rotates through enough independent weight copies
that every call reads its weights from HBM.

Printed: one JSON line.  `value` = algorithmic bytes of a step / step time (GB/s).
`roofline` = the GEMM kernel's algorithmic bytes per launch / its average launch
duration (HIP events on the launch stream), against 8 TB/s.  `cpu_baseline` = the
CPU oracle timed on the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8 GEMM TOPS & weight GB/s (% of MI355X INT8/HBM peak), decode+prefill+MoE"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
K_DEC, N_DEC, M_DEC = 8192, 28672, (1, 8, 16)
GROUP = 128


def dense_bytes(M, N, K):
    """Algorithmic HBM bytes of one W4A8 GEMM launch: packed weights (K/2 per column),
    fp16 scale + zp (4 B per 128 weights), INT8 activations, fp32 row scales, fp32 output."""
    return N * K // 2 + 4 * N * (K // GROUP) + M * K + 4 * M + 4 * M * N


def quant_bytes(M, K):
    """Per-token quantizer: fp32 x read, INT8 codes and fp32 row scale written."""
    return 4 * M * K + M * K + 4 * M


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--copies", type=int, default=6, help="weight copies rotated to defeat the MALL")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the prefill / MoE figures")
    p.add_argument("--profile-copy", action="store_true",
                   help="also launch one plain 512 MiB device copy (calibrates HBM counters)")
    return p.parse_args()


class EventTimer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.torch.cuda.current_stream())
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.torch.cuda.current_stream())
        self.pairs.append((s, e))

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs]))


def decode_setup(torch, w4, synthetic, copies):
    dev = torch.device("cuda:0")
    W = torch.empty((N_DEC, K_DEC), dtype=torch.float32, device=dev)
    synthetic.fill_weights_device(W, 0, synthetic.TAG_W, 0, K_DEC, 0, "outliers")
    layers = [w4.pack_weights_device(W)]
    for _ in range(copies - 1):
        layers.append(tuple(t.clone() for t in layers[0]))
    del W
    x = torch.from_numpy(synthetic.activations_with_outlier_channels(0, 16, K_DEC)).to(dev)
    xs = {M: x[:M].contiguous() for M in M_DEC}
    torch.cuda.synchronize()
    return layers, xs


def run_decode(torch, w4, layers, xs, steps, warmup):
    calls = [0]
    gemm_timer = EventTimer(torch)

    def step(timed):
        for M in M_DEC:
            layer = layers[calls[0] % len(layers)]
            calls[0] += 1
            qa, sc = w4.quantize_act(xs[M])
            if timed:
                s = gemm_timer.start()
            w4.gemm(qa, sc, *layer)
            if timed:
                gemm_timer.stop(s)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    step_bytes = sum(dense_bytes(M, N_DEC, K_DEC) + quant_bytes(M, K_DEC) for M in M_DEC)
    gemm_bytes = float(np.mean([dense_bytes(M, N_DEC, K_DEC) for M in M_DEC]))
    gemm_ms = gemm_timer.mean_ms()
    per_m = {}
    for i, M in enumerate(M_DEC):
        ms = float(np.mean([s.elapsed_time(e) for s, e in gemm_timer.pairs[i::len(M_DEC)]]))
        per_m[str(M)] = {"gemm_us": round(ms * 1e3, 2),
                         "GB/s": round(dense_bytes(M, N_DEC, K_DEC) / (ms * 1e-3) / 1e9, 1),
                         "TOPS": round(2 * M * N_DEC * K_DEC / (ms * 1e-3) / 1e12, 3)}
    return ms_per_step, step_bytes, gemm_bytes, gemm_ms, per_m


def cpu_baseline(synthetic):
    """The oracle on the decode step (quantize + GEMM for M = 1, 8, 16), host threads."""
    import oracle
    orc = oracle.default()
    W = synthetic.fill_weights_host(0, synthetic.TAG_W, 0, K_DEC, 0, N_DEC, "outliers")
    q, s, z = orc.quantize_weights(W)   # offline weight conversion, not part of the step
    del W
    x = synthetic.activations_with_outlier_channels(0, 16, K_DEC)
    reps, t_total = 0, 0.0
    while t_total < 10.0 and reps < 20:
        t0 = time.perf_counter()
        for M in M_DEC:
            qa, sc = orc.quantize_act(x[:M])
            orc.gemm(qa, sc, q, s, z)
        t_total += time.perf_counter() - t0
        reps += 1
    step_bytes = sum(dense_bytes(M, N_DEC, K_DEC) + quant_bytes(M, K_DEC) for M in M_DEC)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(step_bytes * reps / t_total / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full decode step (M=1,8,16; K=8192; N=28672), {reps} repetitions, "
                      f"{t_total:.1f} s; weight quantization excluded (offline)"}


def secondary(torch, w4, synthetic):
    """Prefill (M=4096, K=N=8192) TOPS and MoE layer times; context figures."""
    dev = torch.device("cuda:0")
    out = {}
    # prefill
    M, N, K = 4096, 8192, 8192
    W = torch.empty((N, K), dtype=torch.float32, device=dev)
    synthetic.fill_weights_device(W, 0, synthetic.TAG_W, 0, K, 0, "offset")
    layer = w4.pack_weights_device(W)
    del W
    x = torch.from_numpy(synthetic.activations(0, M, K)).to(dev)
    qa, sc = w4.quantize_act(x)
    for _ in range(3):
        w4.gemm(qa, sc, *layer)
    t = EventTimer(torch)
    for _ in range(10):
        s = t.start()
        w4.gemm(qa, sc, *layer)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    tops = 2 * M * N * K / (ms * 1e-3) / 1e12
    out["prefill_M4096_K8192_N8192"] = {"gemm_us": round(ms * 1e3, 1), "TOPS": round(tops, 1),
                                        "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
    del layer, x, qa, sc
    torch.cuda.empty_cache()
    # MoE FFN layer, 384 experts + shared, top-8, H=7168, I=2048
    from tests.gpu_common import device_experts
    E, k, H, I = 384, 8, 7168, 2048
    gate_up = device_experts(0, synthetic.TAG_W, E + 1, 2 * I, H)
    down = device_experts(0, synthetic.TAG_W_DOWN, E + 1, H, I)
    for T in (64, 4096):
        x = torch.from_numpy(synthetic.activations(0, T, H)).to(dev)
        logits = torch.from_numpy(synthetic.router_logits_skewed(0, T, E)).to(dev)
        for _ in range(2):
            w4.moe_ffn(x, logits, k, gate_up, down)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 5
        for _ in range(reps):
            _, inter = w4.moe_ffn(x, logits, k, gate_up, down)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        counts = np.diff(inter["offsets"].cpu().numpy())
        touched = int((counts > 0).sum())
        wbytes = touched * (2 * I * H // 2 + 4 * 2 * I * H // GROUP + H * I // 2 + 4 * H * I // GROUP)
        ops = 2 * (T * k + T) * (2 * I * H + H * I)
        out[f"moe_ffn_T{T}"] = {"layer_us": round(ms * 1e3, 1), "experts_touched": touched,
                                "weight_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
                                "TOPS": round(ops / (ms * 1e-3) / 1e12, 2)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is described in DESIGN.md, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    import synthetic
    import w4a8_quantized_gemm_token_amd as w4

    w4.load()
    layers, xs = decode_setup(torch, w4, synthetic, args.copies)
    ms_per_step, step_bytes, gemm_bytes, gemm_ms, per_m = run_decode(torch, w4, layers, xs, args.steps, args.warmup)
    if args.profile_copy:
        a = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    del layers
    torch.cuda.empty_cache()
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "W4A8 decode linear: per-token INT8 quant + GEMM, K=8192, N=28672, group=128, "
                               "M=1,8,16 per step (0.1% x20 weight outliers, 4 x50 activation channels)",
                   "weight_copies_rotated": args.copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemm_stream_kernel (streaming W4A8 GEMM)",
                     "bytes_per_launch": gemm_bytes, "avg_launch_us": round(gemm_ms * 1e3, 2)},
        "decode_per_M": per_m,
    }
    if not args.no_secondary:
        result["secondary"] = secondary(torch, w4, synthetic)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synthetic)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
