"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no arithmetic of the quantization method.  It only draws the
fp32 tensors (weights, activations, router logits) that both sides consume.

Every value is a pure function of (seed, tensor tag, sub-stream, element index),
so any slice can be regenerated on its own and the GPU-side filler in
``gen_device.hip`` produces the same bytes:

  mix64(z)     SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
               pseudorandom number generators", OOPSLA 2014), all mod 2^64.
  key          mix64(mix64(seed * GOLDEN + tag) + sub * GOLDEN)
  bits(key,i)  mix64(key + (i + 1) * GOLDEN)
  normal       Irwin-Hall(4) stand-in for N(0,1), used for weights only: the four
               16-bit fields of bits() are summed, centred (integer in
               [-131070, 131070], exact in fp32) and multiplied by
               fp32(sqrt(3)/65536); variance 1 - 2^-32.  Its tails stop at
               +-2*sqrt(3) (about 3.46 sigma).
  weights      fp32(normal * fp32(std)), std = 0.02
  uniform24    bits >> 40, a 24-bit integer

Activations and router logits are true N(0,1) draws: numpy's PCG64 generator
seeded with the integer triple (seed, tag, sub) through SeedSequence, float64
standard_normal in row-major order, rounded once to fp32.  They are drawn on the
host and copied to the device, so both sides read the same bytes.  Their tails
matter: with the skewed router bias, cold experts are reached only through tail
draws, so a bounded stand-in would route to far fewer experts.  The weights'
stand-in changes neither the routing (logits are a separate draw) nor any byte
count (sizes are fixed by the shapes).

The recipes per workload (shapes, outliers, offsets, router bias) live in the
functions below.
"""
from __future__ import annotations

import math

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
IH4_UNIT = np.float32(math.sqrt(3.0) / 65536.0)
WEIGHT_STD = np.float32(0.02)
OUTLIER_P_BITS = np.uint64(int(round(0.001 * 2.0 ** 53)))  # P(outlier) = 0.001
OUTLIER_W_FACTOR = np.float32(20.0)
OUTLIER_X_FACTOR = np.float32(50.0)
MU_UNIT = np.float32(0.01 / 2.0 ** 23)

# tensor tags (one per kind of tensor, so the streams never overlap)
TAG_W = 1            # dense / expert weights
TAG_W_DOWN = 2       # MoE down-projection weights
TAG_X = 3            # activations
TAG_LOGIT = 4        # router logits
TAG_OUTLIER = 5      # weight outlier mask
TAG_CHANNEL = 6      # activation outlier channels
TAG_MU = 7           # per-column weight mean offset
TAG_GU = 8           # synthetic gate/up activations (stage tests)
TAG_Y = 9            # synthetic expert outputs (stage tests)
TAG_W_SHARED = 10    # shared expert gate/up
TAG_W_SHARED_DOWN = 11


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * _M1
        z = z ^ (z >> np.uint64(27))
        z = z * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def stream_key(seed: int, tag: int, sub: int = 0) -> int:
    with np.errstate(over="ignore"):
        a = np.array([seed], np.uint64) * GOLDEN + np.uint64(tag)
        b = mix64(a) + np.array([sub], np.uint64) * GOLDEN
        return int(mix64(b)[0])


def bits(key: int, idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + (idx + np.uint64(1)) * GOLDEN)


def normal(key: int, idx: np.ndarray) -> np.ndarray:
    b = bits(key, idx)
    m = np.uint64(0xFFFF)
    s = (b & m) + ((b >> np.uint64(16)) & m) + ((b >> np.uint64(32)) & m) + (b >> np.uint64(48))
    centred = s.astype(np.int64) - 131070
    return centred.astype(np.float32) * IH4_UNIT


def uniform24(key: int, idx: np.ndarray) -> np.ndarray:
    return (bits(key, idx) >> np.uint64(40)).astype(np.int64)


# ----------------------------------------------------------------------------- weights
def _row_indices(rows, N):
    return np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)


def weights(seed: int, tag: int, sub: int, N: int, K: int, rows=None) -> np.ndarray:
    """W[n][k] ~ 0.02 * N(0,1) (Irwin-Hall stand-in); rows selects a subset of n."""
    r = _row_indices(rows, N)
    idx = (r[:, None] * K + np.arange(K, dtype=np.int64)[None, :]).ravel()
    z = normal(stream_key(seed, tag, sub), idx)
    return (z * WEIGHT_STD).reshape(len(r), K)


def weights_with_outliers(seed: int, N: int, K: int, rows=None) -> np.ndarray:
    """Decode workload: each entry independently an outlier (x20) with probability 0.001."""
    r = _row_indices(rows, N)
    W = weights(seed, TAG_W, 0, N, K, rows=r)
    idx = (r[:, None] * K + np.arange(K, dtype=np.int64)[None, :]).ravel()
    mask = (bits(stream_key(seed, TAG_OUTLIER), idx) >> np.uint64(11)) < OUTLIER_P_BITS
    W = W.ravel()
    W[mask] = W[mask] * OUTLIER_W_FACTOR
    return W.reshape(len(r), K)


def column_means(seed: int, N: int, rows=None) -> np.ndarray:
    """Prefill workload: per-column mean offset mu_n ~ U(-0.01, 0.01)."""
    r = _row_indices(rows, N)
    u = uniform24(stream_key(seed, TAG_MU), r)
    return (u - (1 << 23)).astype(np.float32) * MU_UNIT


def weights_with_offset(seed: int, N: int, K: int, rows=None) -> np.ndarray:
    r = _row_indices(rows, N)
    W = weights(seed, TAG_W, 0, N, K, rows=r)
    return (column_means(seed, N, rows=r)[:, None] + W).astype(np.float32)


# ----------------------------------------------------------------------------- activations
def gauss(seed: int, tag: int, sub: int, shape) -> np.ndarray:
    """True N(0,1) draws: PCG64 seeded with SeedSequence([seed, tag, sub]), float64, rounded to fp32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag), int(sub)])))
    return g.standard_normal(shape).astype(np.float32)


def activations(seed: int, M: int, K: int, tag: int = TAG_X, sub: int = 0, rows=None) -> np.ndarray:
    """x[m][k] ~ N(0,1) (true normal, see gauss); rows selects a subset of m."""
    x = gauss(seed, tag, sub, (M, K))
    return x if rows is None else x[np.asarray(rows, dtype=np.int64)]


def outlier_channels(seed: int, K: int, count: int = 4) -> np.ndarray:
    """The first `count` distinct channels of a seeded sequence."""
    key = stream_key(seed, TAG_CHANNEL)
    out = []
    j = 0
    while len(out) < count:
        c = int(bits(key, np.array([j]))[0] % np.uint64(K))
        if c not in out:
            out.append(c)
        j += 1
    return np.array(out, dtype=np.int64)


def activations_with_outlier_channels(seed: int, M: int, K: int, rows=None) -> np.ndarray:
    """Decode workload: 4 fixed channels scaled x50 in every token."""
    x = activations(seed, M, K, rows=rows)
    ch = outlier_channels(seed, K)
    x[:, ch] = x[:, ch] * OUTLIER_X_FACTOR
    return x


# ----------------------------------------------------------------------------- router
def router_logits_iid(seed: int, T: int, E: int) -> np.ndarray:
    """Toy MoE: iid N(0,1) logits (true normal), so top-1 routing is uniform over experts."""
    return gauss(seed, TAG_LOGIT, 0, (T, E))


def zipf_bias(E: int, s: float = 1.1) -> np.ndarray:
    """Per-expert bias b_e = -s * ln(e + 1): selection odds fall like a Zipf law of rank e+1."""
    return np.array([-s * math.log(e + 1) for e in range(E)], dtype=np.float64).astype(np.float32)


def router_logits_skewed(seed: int, T: int, E: int) -> np.ndarray:
    z = router_logits_iid(seed, T, E)
    return (z + zipf_bias(E)[None, :]).astype(np.float32)


# ----------------------------------------------------------------------------- workloads
CONFIGS = {
    "c1_small": dict(M=4, K=256, N=128),
    "c2_decode": dict(M=(1, 8, 16), K=8192, N=28672),
    "c3_prefill": dict(M=4096, K=8192, N=8192),
    "c4_toy_moe": dict(E=8, topk=1, B=(1, 2, 4, 512), K=4096, N=14336),
    "c5_moe_ffn": dict(E=384, topk=8, H=7168, I=2048, T=(64, 4096), shared=1),
}
GROUP = 128


# ----------------------------------------------------------------------------- device filler
_DEV_LIB = None
_DEV_SRC = __import__("os").path.join(__import__("os").path.dirname(__file__), "gen_device.hip")
DEV_LIB_PATH = _DEV_SRC.replace("gen_device.hip", "libsynth.so")


def build_device(verbose: bool = False) -> str:
    """Compile the GPU filler (gfx950) in-tree."""
    import subprocess
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", _DEV_SRC, "-o", DEV_LIB_PATH]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for the synthetic filler:\n" + res.stderr)
    return DEV_LIB_PATH


def _dev_lib():
    global _DEV_LIB
    if _DEV_LIB is None:
        import ctypes
        lib = ctypes.CDLL(DEV_LIB_PATH)
        lib.synth_fill_weights.restype = ctypes.c_int
        lib.synth_fill_weights.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_void_p]
        _DEV_LIB = lib
    return _DEV_LIB


def fill_weights_device(out, seed: int, tag: int, sub: int, K: int, row0: int = 0, mode: str = "plain"):
    """Fill the device fp32 tensor out [rows][K] with rows [row0, row0+rows) of the same weights the
    numpy recipes give: mode 'plain' (weights), 'outliers' (weights_with_outliers, tag must be TAG_W,
    sub 0), 'offset' (weights_with_offset)."""
    import ctypes
    import torch
    rows = out.shape[0]
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.shape[1] == K
    m = {"plain": 0, "outliers": 1, "offset": 2}[mode]
    key = stream_key(seed, tag, sub)
    key_o = stream_key(seed, TAG_OUTLIER) if m == 1 else (stream_key(seed, TAG_MU) if m == 2 else 0)
    rc = _dev_lib().synth_fill_weights(ctypes.c_void_p(out.data_ptr()), key, key_o, row0, rows, K,
                                       float(IH4_UNIT), float(WEIGHT_STD), m, int(OUTLIER_P_BITS),
                                       float(OUTLIER_W_FACTOR), float(MU_UNIT),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synthetic filler launch failed ({rc})")
    return out


# ----------------------------------------------------------------------------- host filler (C)
_HOST_LIB = None
HOST_SRC = _DEV_SRC.replace("gen_device.hip", "gen_host.c")
HOST_LIB_PATH = _DEV_SRC.replace("gen_device.hip", "libsynth_host.so")


def build_host() -> str:
    import subprocess
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           HOST_SRC, "-o", HOST_LIB_PATH])
    return HOST_LIB_PATH


def _host_lib():
    global _HOST_LIB
    if _HOST_LIB is None:
        import ctypes
        import os
        if not os.path.exists(HOST_LIB_PATH):
            build_host()
        lib = ctypes.CDLL(HOST_LIB_PATH)
        lib.synth_fill_weights_host.restype = None
        lib.synth_fill_weights_host.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                                ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_float]
        _HOST_LIB = lib
    return _HOST_LIB


def fill_weights_host(seed: int, tag: int, sub: int, K: int, row0: int, rows: int, mode: str = "plain"):
    """Rows [row0, row0+rows) of a weight recipe, from the C filler (fast; same bytes as numpy)."""
    import ctypes
    m = {"plain": 0, "outliers": 1, "offset": 2}[mode]
    key = stream_key(seed, tag, sub)
    key_o = stream_key(seed, TAG_OUTLIER) if m == 1 else (stream_key(seed, TAG_MU) if m == 2 else 0)
    out = np.empty((rows, K), np.float32)
    _host_lib().synth_fill_weights_host(out.ctypes.data_as(ctypes.c_void_p), key, key_o, row0, rows, K,
                                        float(IH4_UNIT), float(WEIGHT_STD), m, int(OUTLIER_P_BITS),
                                        float(OUTLIER_W_FACTOR), float(MU_UNIT))
    return out


def weight_rows_host(seed: int, tag: int, sub: int, K: int, rows, mode: str = "plain"):
    """Arbitrary (sorted or not) rows of a weight recipe via the C filler."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), K), np.float32)
    for i, r in enumerate(rows):
        out[i] = fill_weights_host(seed, tag, sub, K, int(r), 1, mode)[0]
    return out
