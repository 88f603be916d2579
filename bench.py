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


def dense_bytes(M, N, K, group=GROUP):
    """Algorithmic HBM bytes of one W4A8 GEMM launch: packed weights (K/2 per column),
    fp16 scale + zp (4 B per group), INT8 activations, fp32 row scales, fp32 output."""
    return N * K // 2 + 4 * N * (K // group) + M * K + 4 * M + 4 * M * N


def quant_bytes(M, K):
    """Per-token quantizer: fp32 x read, INT8 codes and fp32 row scale written."""
    return 4 * M * K + M * K + 4 * M


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "gemm_decode_kernel.decode_K8192_N28672_M1-8-16.traffic.txt")
DECODE_KERNEL = "gemm_decode_kernel"
COPY_BYTES = 512 << 20
KERNEL_SOURCES = ("w4a8_quantized_gemm_token_amd/csrc/gemm_kernels.hip",
                  "w4a8_quantized_gemm_token_amd/csrc/w4a8_internal.hpp")


def kernel_digest():
    """sha256 over the GEMM kernel sources: a traffic figure taken from counters is only
    reported while the kernels it was measured on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per decode-GEMM launch from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_digest():
        return None
    return float(kv["traffic_bytes_per_launch"])


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_traffic(fetch_csv, write_csv, cmd):
    """Text summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch):
    the decode GEMM's per-launch figures, scaled by what the same counters read for one plain
    512 MiB device copy."""
    out = []
    vals = {}
    for label, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == label]
        gem = [float(r["Counter_Value"]) for r in rows if DECODE_KERNEL in r["Kernel_Name"]]
        cop = [(float(r["Counter_Value"]), r["Kernel_Name"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not gem or not cop:
            raise SystemExit(f"{path}: no {DECODE_KERNEL} or copy dispatch with {label}")
        copy_kib, copy_name = max(cop)
        factor = COPY_BYTES / (copy_kib * 1024.0)
        vals[label] = (float(np.mean(gem)), len(gem), copy_kib, copy_name, factor)
    f_kib, f_n, f_copy, copy_name, f_fac = vals["FETCH_SIZE"]
    w_kib, w_n, w_copy, _, w_fac = vals["WRITE_SIZE"]
    traffic = f_kib * 1024 * f_fac + w_kib * 1024 * w_fac
    alg = float(np.mean([dense_bytes(M, N_DEC, K_DEC) for M in M_DEC]))
    out.append(f"# HBM traffic of {DECODE_KERNEL}: decode W4A8 GEMM, K={K_DEC} N={N_DEC}, M=1,8,16 rotated")
    out.append("# commands (run from /tmp with TMPDIR=/tmp; <repo> = the repository root):")
    for c in cmd:
        out.append("#   " + c)
    out.append(f"# calibration kernel: {copy_name[:60]} copying {COPY_BYTES} bytes once")
    out.append(f"kernel_sources_sha256: {kernel_digest()}")
    out.append(f"gemm_dispatches: {f_n} (FETCH_SIZE run), {w_n} (WRITE_SIZE run)")
    out.append(f"fetch_kib_per_launch_raw: {f_kib:.1f}")
    out.append(f"write_kib_per_launch_raw: {w_kib:.1f}")
    out.append(f"copy_fetch_kib_raw: {f_copy:.1f}")
    out.append(f"copy_write_kib_raw: {w_copy:.1f}")
    out.append(f"fetch_scale: {f_fac:.4f}")
    out.append(f"write_scale: {w_fac:.4f}")
    out.append(f"fetch_bytes_per_launch: {f_kib * 1024 * f_fac:.0f}")
    out.append(f"write_bytes_per_launch: {w_kib * 1024 * w_fac:.0f}")
    out.append(f"traffic_bytes_per_launch: {traffic:.0f}")
    out.append(f"algorithmic_bytes_per_launch: {alg:.0f}")
    out.append(f"traffic_over_algorithmic: {traffic / alg:.4f}")
    return "\n".join(out)


def summarize_kernel_traffic(fetch_csv, write_csv, cmd, kernel):
    """Text summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) for every kernel whose
    name contains `kernel`: HBM bytes per dispatch (mean, min, max), each counter scaled by what it
    reads for one plain 512 MiB device copy in the same process."""
    out = [f"# HBM traffic per dispatch of kernels matching '{kernel}'",
           "# commands (run from /tmp with TMPDIR=/tmp; <repo> = the repository root):"]
    for c in cmd:
        out.append("#   " + c)
    scaled = {}
    for label, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == label]
        cop = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not cop:
            raise SystemExit(f"{path}: no copy dispatch with {label}")
        factor = COPY_BYTES / (max(cop) * 1024.0)
        out.append(f"{label.lower()}_scale: {factor:.4f}")
        for r in rows:
            if kernel in r["Kernel_Name"]:
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
                scaled.setdefault(name.strip(), {}).setdefault(label, []).append(
                    float(r["Counter_Value"]) * 1024.0 * factor)
    for name, d in sorted(scaled.items()):
        for label in ("FETCH_SIZE", "WRITE_SIZE"):
            v = d.get(label, [])
            if v:
                out.append(f"{name} {label.lower()}_bytes: mean {np.mean(v):.0f} min {np.min(v):.0f} "
                           f"max {np.max(v):.0f} ({len(v)} dispatches)")
    return "\n".join(out)


def summarize_stats(stats_csv, cmd, top=12):
    """Short text table of a rocprofv3 --kernel-trace --stats kernel summary."""
    rows = _counter_rows(stats_csv)
    out = ["# rocprofv3 kernel statistics", "# command (run from /tmp with TMPDIR=/tmp; <repo> = the repository root):"]
    for c in cmd:
        out.append("#   " + c)
    out.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
    for r in rows[:top]:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("at::native::", "")
        if name.startswith("void "):
            name = name[5:]
        short = name.split("(")[0][:70]
        out.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                   f"{float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>6.2f}  {short.strip()}")
    return "\n".join(out)


def summarize_counters(csvs, kernel, cmd):
    """Text summary of rocprofv3 --pmc runs (SQ_* / GRBM_* counters) for one kernel: the mean of
    each counter over that kernel's dispatches, then a few ratios derived from them."""
    vals, n = {}, {}
    for path in csvs:
        for r in _counter_rows(path):
            if kernel not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel} in {csvs}")
    avg = {k: float(np.mean(v)) for k, v in vals.items()}
    out = [f"# hardware counters of {kernel}, mean per dispatch",
           "# commands (run from /tmp with TMPDIR=/tmp; <repo> = the repository root):"]
    for c in cmd:
        out.append("#   " + c)
    out.append(f"kernel_sources_sha256: {kernel_digest()}")
    for k in sorted(avg):
        out.append(f"{k}: {avg[k]:.0f}   ({len(vals[k])} dispatches)")

    def ratio(name, a, b, scale=1.0):
        if a in avg and b in avg and avg[b] > 0:
            out.append(f"{name}: {scale * avg[a] / avg[b]:.3f}")

    out.append("# derived")
    ratio("valu_insts_per_mfma_inst", "SQ_INSTS_VALU", "SQ_INSTS_MFMA")
    ratio("lds_insts_per_mfma_inst", "SQ_INSTS_LDS", "SQ_INSTS_MFMA")
    ratio("wave_cycles_waiting_on_loads_frac", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")
    ratio("wave_cycles_waiting_any_frac", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
    ratio("coexec_over_mfma_busy", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES")
    ratio("valu_active_over_wave_cycles", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")
    return "\n".join(out)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=2000,
                   help="untimed steps after the fixed-duration warm-up")
    p.add_argument("--warmup-seconds", type=float, default=1.0,
                   help="untimed steps for at least this long first, whatever --warmup is (the GPU leaves "
                        "its idle clock state: a decode launch measured 28 us cold, 25.5 us warm)")
    p.add_argument("--copies", type=int, default=6, help="weight copies rotated to defeat the MALL")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the prefill / MoE figures")
    p.add_argument("--profile-copy", action="store_true",
                   help="also launch one plain 512 MiB device copy (calibrates HBM counters)")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="print the traffic summary of two rocprofv3 --pmc counter_collection.csv files; no GPU")
    p.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                   help="print a short table of a rocprofv3 kernel_stats.csv; no GPU")
    p.add_argument("--summarize-counters", nargs="+", metavar="COUNTER_CSV",
                   help="print the mean SQ/GRBM counters of --kernel over rocprofv3 --pmc runs; no GPU")
    p.add_argument("--kernel", default="gemm_tiled3_kernel", help="kernel named by --summarize-counters")
    p.add_argument("--summarize-kernel-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="print the HBM traffic per dispatch of the kernels matching --kernel; no GPU")
    p.add_argument("--cmd", action="append", default=[], help="command text recorded in a summary")
    p.add_argument("--only", choices=["prefill", "toy_moe", "moe_ffn"],
                   help="run one secondary workload alone and print its figures (for counter runs)")
    p.add_argument("--size", type=int, action="append",
                   help="batch B (toy_moe) or tokens T (moe_ffn) for --only; repeatable")
    p.add_argument("--group", type=int, default=GROUP, choices=(64, 128, 256),
                   help="group size of the weights for --only prefill")
    p.add_argument("--reps", type=int, default=10, help="timed launches for --only")
    p.add_argument("--path", type=int, action="append",
                   help="main loop of --only prefill (as w4a8_gemm_path; default: the one w4a8_gemm picks); "
                        "repeatable, each timed in turn")
    p.add_argument("--tile-major", action="store_true",
                   help="--only prefill on the tile-major weight array (w4a8_gemm_tm; group 128)")
    return p.parse_args()


def decode_setup(torch, w4, synthetic, copies):
    """`copies` copies of the decode layer in the standard layout and in the tile-major one
    (converted offline, outside any timed region), and the activations."""
    dev = torch.device("cuda:0")
    W = torch.empty((N_DEC, K_DEC), dtype=torch.float32, device=dev)
    synthetic.fill_weights_device(W, 0, synthetic.TAG_W, 0, K_DEC, 0, "outliers")
    layers = [w4.pack_weights_device(W)]
    for _ in range(copies - 1):
        layers.append(tuple(t.clone() for t in layers[0]))
    del W
    tms = [w4.weights_to_tm(*layer) for layer in layers]
    x = torch.from_numpy(synthetic.activations_with_outlier_channels(0, 16, K_DEC)).to(dev)
    xs = {M: x[:M].contiguous() for M in M_DEC}
    torch.cuda.synchronize()
    return layers, tms, xs


def run_decode(torch, w4, prep, n_layers, xs, steps, warmup, warmup_s=0.0):
    """Times `steps` decode steps, then the GEMM kernel alone.

    `prep(qa, sc, i, out)` prepares the GEMM over weight copy i.  Each launch is prepared once
    (pointers marshalled), so the host stays ahead of the GPU and kernels run back to back.
    HIP event records are themselves queue packets that cost a few microseconds each, so none
    sits between the kernels of a step; the GEMM's launch duration is taken from one event pair
    around max(`steps`, 200) back-to-back GEMM launches per M (rotating weight copies,
    activations from the step) on the same stream."""
    dev = torch.device("cuda:0")
    quant, gemms = {}, {}
    for M in M_DEC:
        qa = torch.empty((M, K_DEC), dtype=torch.int8, device=dev)
        sc = torch.empty((M,), dtype=torch.float32, device=dev)
        out = torch.empty((M, N_DEC), dtype=torch.float32, device=dev)
        quant[M] = w4.prepare_quantize_act(xs[M], qa, sc)
        gemms[M] = [prep(qa, sc, i, out) for i in range(n_layers)]
    stream = torch.cuda.current_stream()
    calls = 0

    def step():
        nonlocal calls
        for M in M_DEC:
            quant[M]()
            gemms[M][calls % n_layers]()
            calls += 1

    tw = time.perf_counter()
    while time.perf_counter() - tw < warmup_s:   # fixed-duration warm-up, then the counted one
        for _ in range(100):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    warmed_s = time.perf_counter() - tw
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    step_bytes = sum(dense_bytes(M, N_DEC, K_DEC) + quant_bytes(M, K_DEC) for M in M_DEC)

    per_m, launch_ms = {}, []
    for M in M_DEC:
        # a few milliseconds of the same launches first: after the host's synchronize above the
        # GPU idles briefly, and the first launches after an idle gap run at a lower clock (the
        # M timed first measured 1-3 us slower than the same M timed later); the GPU is also
        # still busy when the start event is reached
        for i in range(max(n_layers, 200)):
            gemms[M][i % n_layers]()
        # at least 200 launches between the events: an event record costs a few microseconds,
        # which over 20 launches would add about 1% to each
        n_timed = max(steps, 200)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for i in range(n_timed):
            gemms[M][i % n_layers]()
        e.record(stream)
        e.synchronize()
        ms = s.elapsed_time(e) / n_timed
        launch_ms.append(ms)
        per_m[str(M)] = {"gemm_us": round(ms * 1e3, 2),
                         "GB/s": round(dense_bytes(M, N_DEC, K_DEC) / (ms * 1e-3) / 1e9, 1),
                         "TOPS": round(2 * M * N_DEC * K_DEC / (ms * 1e-3) / 1e12, 3)}
    gemm_bytes = float(np.mean([dense_bytes(M, N_DEC, K_DEC) for M in M_DEC]))
    gemm_ms = float(np.mean(launch_ms))
    return ms_per_step, step_bytes, gemm_bytes, gemm_ms, per_m, warmed_s


def cpu_baseline(synthetic):
    """The oracle on the decode step (quantize + GEMM for M = 1, 8, 16), host threads."""
    import oracle
    orc = oracle.default()
    W = synthetic.fill_weights_host(0, synthetic.TAG_W, 0, K_DEC, 0, N_DEC, "outliers")
    q, s, z = orc.quantize_weights(W)   # offline weight conversion, not part of the step
    del W
    x = synthetic.activations_with_outlier_channels(0, 16, K_DEC)
    reps, t_total = 0, 0.0
    while t_total < 12.0 and reps < 200:
        t0 = time.perf_counter()
        for M in M_DEC:
            qa, sc = orc.quantize_act(x[:M])
            orc.gemm(qa, sc, q, s, z)
        t_total += time.perf_counter() - t0
        reps += 1
    step_bytes = sum(dense_bytes(M, N_DEC, K_DEC) + quant_bytes(M, K_DEC) for M in M_DEC)
    threads = orc.num_threads()
    return {"value": round(step_bytes * reps / t_total / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full decode step (M=1,8,16; K=8192; N=28672), {reps} repetitions, "
                      f"{t_total:.1f} s; weight quantization excluded (offline)"}


def cpu_prefill_context(synthetic, rows=32):
    """The oracle on a row sample of the prefill GEMM (the first `rows` of M=4096; all of K=N=8192),
    repeated for about 4 s; host threads.  Context for the GPU prefill figure, not a baseline of
    the headline workload."""
    import oracle
    orc = oracle.default()
    W = synthetic.fill_weights_host(0, synthetic.TAG_W, 0, 8192, 0, 8192, "offset")
    q, s, z = orc.quantize_weights(W)   # offline weight conversion, not timed
    del W
    x = synthetic.activations(0, rows, 8192)
    reps, t_total = 0, 0.0
    while t_total < 4.0 and reps < 100:
        t0 = time.perf_counter()
        qa, sc = orc.quantize_act(x)
        orc.gemm(qa, sc, q, s, z)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"TOPS": round(2.0 * rows * 8192 * 8192 * reps / t_total / 1e12, 4), "cores": orc.num_threads(),
            "kind": "oracle", "sample": f"rows 0..{rows - 1} of the M=4096 prefill GEMM (K=N=8192), {reps} "
                                       f"repetitions, {t_total:.1f} s; weight quantization excluded"}


def prefill(torch, w4, synthetic, reps=20, group=GROUP, paths=(0,), tile_major=False):
    """The prefill-shaped dense GEMM (M=4096, K=N=8192): quantize once, then `reps`
    back-to-back prepared launches timed with one event pair on the launch stream.
    Group sizes other than 128 are packed by the host packer (the device packer takes 128).
    tile_major: the same weights converted to the tile-major array, run by w4a8_gemm_tm."""
    dev = torch.device("cuda:0")
    M, N, K = 4096, 8192, 8192
    W = torch.empty((N, K), dtype=torch.float32, device=dev)
    synthetic.fill_weights_device(W, 0, synthetic.TAG_W, 0, K, 0, "offset")
    if group == GROUP:
        layer = w4.pack_weights_device(W)
    else:
        packed, scale, zp = w4.pack_weights(W.cpu().numpy(), group=group)
        layer = (torch.from_numpy(packed).to(dev), torch.from_numpy(scale.view(np.int16)).to(dev),
                 torch.from_numpy(zp.view(np.int16)).to(dev))
    del W
    x = torch.from_numpy(synthetic.activations(0, M, K)).to(dev)
    qa, sc = w4.quantize_act(x)
    out_buf = torch.empty((M, N), dtype=torch.float32, device=dev)
    res = {}
    if tile_major:
        layer = (w4.weights_to_tm(*layer),)
        paths = ("tm",)
    for path in paths:  # (0: the loop w4a8_gemm picks; others force one, for comparisons)
        if tile_major:
            launch = w4.prepare_gemm_tm(qa, sc, layer[0], out_buf)
        else:
            launch = w4.prepare_gemm(qa, sc, *layer, out_buf, group=group, path=path)
        _warm(torch, [launch])
        stream = torch.cuda.current_stream()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            launch()
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tops = 2 * M * N * K / (ms * 1e-3) / 1e12
        res[path] = {"gemm_us": round(ms * 1e3, 1), "TOPS": round(tops, 1),
                     "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
    del layer, x, qa, sc, out_buf
    torch.cuda.empty_cache()
    return res[paths[0]] if len(paths) == 1 else res


def quant_variants(torch, w4, synthetic):
    """Packer variants and per-channel smoothing on the decode workload (K=8192, 0.1% x20 weight outliers, 4 x50
    activation channels): the first 4096 output columns, factors from 48 calibration tokens
    (rows 16..63 of the activation draw), error of 16 other tokens against the fp64
    unquantized product, plain vs smoothed; and the quantizer's time with and without
    the per-channel factor (M=16)."""
    dev = torch.device("cuda:0")
    N, K, M = 4096, 8192, 16
    W = torch.empty((N, K), dtype=torch.float32, device=dev)
    synthetic.fill_weights_device(W, 0, synthetic.TAG_W, 0, K, 0, "outliers")
    x = torch.from_numpy(synthetic.activations_with_outlier_channels(0, 64, K)).to(dev)
    xe, xcal = x[:M].contiguous(), x[M:].contiguous()
    exact = xe.double() @ W.double().T
    aw = w4.channel_absmax(W).cpu().numpy()
    ax = w4.channel_absmax(xcal).cpu().numpy()

    def rel_err(qa, sc, packed, scale, zp):
        y = w4.gemm(qa, sc, packed, scale, zp).double()
        return float(torch.linalg.norm(y - exact) / torch.linalg.norm(exact))

    res = {"rel_err_plain": round(rel_err(*w4.quantize_act(xe), *w4.pack_weights_device(W)), 4)}
    # host packer variants on the same columns: symmetric codes, 99.9-percentile clipping
    Wh = W.cpu().numpy()
    for name, kw in (("rel_err_symmetric", {"symmetric": True}), ("rel_err_clip99.9", {"clip_percent": 99.9})):
        packed, scale, zp = w4.pack_weights(Wh, **kw)
        res[name] = round(rel_err(*w4.quantize_act(xe), torch.from_numpy(packed).to(dev),
                                  torch.from_numpy(scale.view(np.int16)).to(dev),
                                  torch.from_numpy(zp.view(np.int16)).to(dev)), 4)
    del Wh
    for alpha in (0.25, 0.5, 0.75):
        s, inv = w4.smooth_factors(ax, aw, alpha)
        s_d, inv_d = torch.from_numpy(s).to(dev), torch.from_numpy(inv).to(dev)
        res[f"rel_err_alpha{alpha}"] = round(rel_err(*w4.quantize_act_smooth(xe, inv_d),
                                                     *w4.pack_weights_device_smooth(W, s_d)), 4)
    qa = torch.empty((M, K), dtype=torch.int8, device=dev)
    sc = torch.empty((M,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for name, launch in (("quantize_us_plain", w4.prepare_quantize_act(xe, qa, sc)),
                         ("quantize_us_smoothed", w4.prepare_quantize_act_smooth(xe, inv_d, qa, sc))):
        for _ in range(50):
            launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(500):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = round(a.elapsed_time(b) / 500 * 1e3, 2)
    del W, exact
    torch.cuda.empty_cache()
    return res


def decode_group_sizes(torch, w4, synthetic, copies, reps=200):
    """The decode GEMM (K=8192, N=28672, M = 1, 8, 16, standard layout) at group 64 and 256:
    per M, one event pair around `reps` back-to-back prepared launches that rotate `copies`
    weight copies (device packer, outlier weights)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    x = torch.from_numpy(synthetic.activations_with_outlier_channels(0, 16, K_DEC)).to(dev)
    res = {}
    for group in (64, 256):
        W = torch.empty((N_DEC, K_DEC), dtype=torch.float32, device=dev)
        synthetic.fill_weights_device(W, 0, synthetic.TAG_W, 0, K_DEC, 0, "outliers")
        layers = [w4.pack_weights_device(W, group=group)]
        del W
        for _ in range(copies - 1):
            layers.append(tuple(t.clone() for t in layers[0]))
        per_m = {}
        for M in M_DEC:
            qa, sc = w4.quantize_act(x[:M].contiguous())
            o = torch.empty((M, N_DEC), dtype=torch.float32, device=dev)
            launches = [w4.prepare_gemm(qa, sc, *layers[i], o, group=group) for i in range(copies)]
            _warm(torch, launches)   # steady clock before the start event
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for i in range(reps):
                launches[i % copies]()
            e.record(stream)
            e.synchronize()
            ms = s.elapsed_time(e) / reps
            per_m[str(M)] = {"gemm_us": round(ms * 1e3, 2),
                             "GB/s": round(dense_bytes(M, N_DEC, K_DEC, group) / (ms * 1e-3) / 1e9, 1),
                             "TOPS": round(2 * M * N_DEC * K_DEC / (ms * 1e-3) / 1e12, 3)}
        res[f"decode_K8192_N28672_group{group}_per_M"] = per_m
        del layers
        torch.cuda.empty_cache()
    return res


def secondary(torch, w4, synthetic, copies):
    """torch's own streaming kernels on this machine, prefill (M=4096, K=N=8192) TOPS, decode at group 64 and
    256, MoE layer times and the smoothing figures; context."""
    out = {"torch_streaming_1GiB": torch_streaming(torch),
           **decode_group_sizes(torch, w4, synthetic, copies),
           "prefill_M4096_K8192_N8192": prefill(torch, w4, synthetic),
           "prefill_M4096_K8192_N8192_tile_major": prefill(torch, w4, synthetic, tile_major=True),
           "prefill_M4096_K8192_N8192_group64": prefill(torch, w4, synthetic, group=64),
           "prefill_M4096_K8192_N8192_group256": prefill(torch, w4, synthetic, group=256),
           "quant_variants_K8192_N4096_M16": quant_variants(torch, w4, synthetic)}

    out.update(toy_moe(torch, w4, synthetic, (1, 2, 4, 512)))
    out.update(moe_ffn_layer(torch, w4, synthetic, (64, 4096)))
    return out


def _device_experts(torch, w4, synthetic, seed, tag, E, N, K):
    dev = torch.device("cuda:0")
    return w4.pack_experts_device(
        E, N, K, lambda e, W: synthetic.fill_weights_device(W, seed, tag, e, K, 0, "plain"), dev)


def _warm(torch, fns, seconds=0.3):
    """Runs the launches for at least `seconds` (in batches, synchronized): the clock of a GPU that
    was idle or on lighter work takes longer than a few launches to settle."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fns[i % len(fns)]()
            i += 1
        torch.cuda.synchronize()


def _timed(torch, fns, reps):
    stream = torch.cuda.current_stream()
    _warm(torch, fns)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for i in range(reps):
        fns[i % len(fns)]()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def torch_streaming(torch, nbytes=1 << 30, reps=20):
    """A plain read (sum) and a copy of 1 GiB with torch's own kernels (larger than the 256 MB
    MALL): the HBM bandwidth an ordinary streaming kernel gets on this machine.  Context for the
    roofline fractions, which stay against the 8 TB/s datasheet peak."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    red = torch.empty((), dtype=torch.float32, device="cuda:0")
    read_ms = _timed(torch, [lambda: torch.sum(a, dim=0, out=red)], reps)
    copy_ms = _timed(torch, [lambda: b.copy_(a)], reps)
    del a, b, red
    torch.cuda.empty_cache()
    return {"read_GB/s": round(nbytes / (read_ms * 1e-3) / 1e9, 1),
            "copy_GB/s": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
            "kernels": "torch.sum over 1 GiB of fp32 (read bytes); torch copy_ of 1 GiB (read + write bytes)"}


def toy_moe(torch, w4, synthetic, batches, reps=60):
    """Toy MoE: 8 experts, top-1, K=4096, N=14336.  The grouped GEMM is timed alone over
    back-to-back prepared launches that rotate three copies of the 250 MB expert set (so no
    call finds its weights in the 256 MB Infinity Cache); the layer (route, quantize,
    grouped GEMM, combine) is timed the same way."""
    dev = torch.device("cuda:0")
    out = {}
    E8, K8, N8, copies = 8, 4096, 14336, 3
    sets = [_device_experts(torch, w4, synthetic, 0, synthetic.TAG_W, E8, N8, K8) for _ in range(copies)]
    ebytes = N8 * K8 // 2 + 4 * N8 * (K8 // GROUP)  # packed codes + fp16 scale and zero point
    for B in batches:
        x = torch.from_numpy(synthetic.activations(100 + B, B, K8)).to(dev)
        logits = torch.from_numpy(synthetic.router_logits_iid(100 + B, B, E8)).to(dev)
        i32, f32 = torch.int32, torch.float32
        routed = (torch.empty((B, 1), dtype=i32, device=dev), torch.empty((B, 1), dtype=f32, device=dev),
                  torch.empty((E8 + 1,), dtype=i32, device=dev), torch.empty((B,), dtype=i32, device=dev),
                  torch.empty((B,), dtype=i32, device=dev), torch.empty((B,), dtype=i32, device=dev))
        qa8 = torch.empty((B, K8), dtype=torch.int8, device=dev)
        sc8 = torch.empty((B,), dtype=f32, device=dev)
        y8 = torch.empty((B, N8), dtype=f32, device=dev)
        o8 = torch.empty((B, N8), dtype=f32, device=dev)
        route = w4.prepare_moe_route(logits, 1, routed)
        quant = w4.prepare_quantize_act(x, qa8, sc8)
        ggs = [w4.prepare_moe_grouped_gemm(qa8, sc8, routed[4], routed[2], *sets[c], B, y8) for c in range(copies)]
        comb = w4.prepare_moe_combine(y8, routed[5], routed[1], o8)
        route()
        quant()
        torch.cuda.synchronize()
        touched = int((np.diff(routed[2].cpu().numpy()) > 0).sum())
        gemm_ms = _timed(torch, ggs, reps)
        layers = [lambda c=c: (route(), quant(), ggs[c](), comb()) for c in range(copies)]
        layer_ms = _timed(torch, layers, reps)
        gbytes = touched * ebytes + B * (K8 + 4) + 4 * B * N8
        t_roof = max(gbytes / (HBM_PEAK_GBS * 1e9), 2.0 * B * N8 * K8 / (INT8_PEAK_TOPS * 1e12))
        out[f"toy_moe_B{B}"] = {"gemm_us": round(gemm_ms * 1e3, 2), "experts_touched": touched,
                                "GB/s": round(gbytes / (gemm_ms * 1e-3) / 1e9, 1),
                                "frac_roofline": round(t_roof / (gemm_ms * 1e-3), 4),
                                "layer_us": round(layer_ms * 1e3, 2)}
    del sets
    torch.cuda.empty_cache()
    return out


def moe_ffn_layer(torch, w4, synthetic, tokens, reps=5):
    """MoE FFN layer, 384 experts + shared, top-8, H=7168, I=2048, true-normal activations
    and skewed router logits; `reps` back-to-back layers after four untimed ones."""
    dev = torch.device("cuda:0")
    out = {}
    E, k, H, I = 384, 8, 7168, 2048
    gate_up = _device_experts(torch, w4, synthetic, 0, synthetic.TAG_W, E + 1, 2 * I, H)
    down = _device_experts(torch, w4, synthetic, 0, synthetic.TAG_W_DOWN, E + 1, H, I)
    for T in tokens:
        x = torch.from_numpy(synthetic.activations(0, T, H)).to(dev)
        logits = torch.from_numpy(synthetic.router_logits_skewed(0, T, E)).to(dev)
        total, _ = w4.moe_ffn_workspace(T, H, I, E, k)
        ws = torch.empty((total,), dtype=torch.uint8, device=dev)
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        for _ in range(4):
            _, inter = w4.moe_ffn(x, logits, k, gate_up, down, workspace=ws, out=y)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(torch.cuda.current_stream())
        for _ in range(reps):
            w4.moe_ffn(x, logits, k, gate_up, down, workspace=ws, out=y)
        e.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        counts = np.diff(inter["offsets"].cpu().numpy())
        touched = int((counts > 0).sum())
        wbytes = touched * (2 * I * H // 2 + 4 * 2 * I * H // GROUP + H * I // 2 + 4 * H * I // GROUP)
        ops = 2 * (T * k + T) * (2 * I * H + H * I)
        out[f"moe_ffn_T{T}"] = {"layer_us": round(ms * 1e3, 1), "experts_touched": touched,
                                "weight_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
                                "TOPS": round(ops / (ms * 1e-3) / 1e12, 2)}
        del ws, y, inter
        torch.cuda.empty_cache()
    return out


def profile_copy(torch):
    """One plain 512 MiB device copy: the known-size dispatch that calibrates the HBM counters."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    args = parse()
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.cmd))
        return
    if args.summarize_kernel_traffic:
        print(summarize_kernel_traffic(*args.summarize_kernel_traffic, args.cmd, args.kernel))
        return
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, args.cmd))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.kernel, args.cmd))
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sharding the layer over several GPUs is designed but not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.tile_major and (args.only != "prefill" or args.group != GROUP or args.path):
        print("bench.py: --tile-major goes with --only prefill at group 128 and takes no --path",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synthetic
    import w4a8_quantized_gemm_token_amd as w4

    w4.load()
    if args.only:
        if args.only == "prefill":
            key = "prefill_M4096_K8192_N8192_" + ("tile_major" if args.tile_major else f"group{args.group}")
            res = {key: prefill(torch, w4, synthetic, args.reps, args.group, tuple(args.path or (0,)),
                                tile_major=args.tile_major)}
        elif args.only == "toy_moe":
            res = toy_moe(torch, w4, synthetic, args.size or (1, 2, 4, 512), args.reps)
        else:
            res = moe_ffn_layer(torch, w4, synthetic, args.size or (64, 4096), args.reps)
        if args.profile_copy:
            profile_copy(torch)
        print(json.dumps(res), flush=True)
        return
    layers, tms, xs = decode_setup(torch, w4, synthetic, args.copies)
    ms_per_step, step_bytes, gemm_bytes, gemm_ms, per_m, warmed_s = run_decode(
        torch, w4, lambda qa, sc, i, out: w4.prepare_gemm_tm(qa, sc, tms[i], out), len(tms), xs, args.steps,
        args.warmup, args.warmup_seconds)
    std_per_m = None
    if not args.no_secondary:  # the same step over the standard layout, for comparison
        std_per_m = run_decode(torch, w4, lambda qa, sc, i, out: w4.prepare_gemm(qa, sc, *layers[i], out),
                               len(layers), xs, args.steps, 200)[4]
    if args.profile_copy:
        profile_copy(torch)
    del layers, tms
    torch.cuda.empty_cache()
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    traffic = read_traffic()
    achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(warmed_s, 2),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "W4A8 decode linear: per-token INT8 quant + GEMM, K=8192, N=28672, group=128, "
                               "M=1,8,16 per step (0.1% x20 weight outliers, 4 x50 activation channels)",
                   "weight_layout": "tile-major (offline reorder of the packed codes, scales and zero points)",
                   "weight_copies_rotated": args.copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "gemm_decode_kernel, tile-major weights (decode W4A8 GEMM, activations staged in LDS)",
                     "bytes_per_launch": gemm_bytes, "avg_launch_us": round(gemm_ms * 1e3, 2)},
        "decode_per_M": per_m,
    }
    if not args.no_secondary:
        result["secondary"] = {"decode_standard_layout_per_M": std_per_m,
                               **secondary(torch, w4, synthetic, args.copies)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synthetic)
        if "secondary" in result:
            result["secondary"]["cpu_oracle_prefill"] = cpu_prefill_context(synthetic)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
