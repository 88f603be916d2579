"""CPU oracle for the W4A8 linear layer (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it shares no code with the HIP library.

The arithmetic lives in ``w4a8_oracle.c`` (plain C, IEEE fp32 steps, double
reference epilogue); this module only marshals numpy arrays into it, plus the
toy-router closed form and its exhaustive enumeration, written in pure Python.

Page keys used in citations:
  [p1] "Kimi 2.7 MoE: from 4-bit storage to INT8 compute" (hotelren.com/news/5173946)
  [p2] "Kimi 2.7 MoE, 4-bit storage to INT8, dissected"   (pptc.cn/news/121597)
  [p3] "LLM quantization primer"                            (hotelren.com/news/5982361)
  [p4] "MoE deployment: active parameters are not the storage bill" (feinterview.poetries.top)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "w4a8_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True, source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no FP contraction, no fast-math."""
    if force or not os.path.exists(out):
        subprocess.check_call(["gcc", *CFLAGS, source, "-o", out, "-lm"])
    return out


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """numpy front end of one compiled copy of the C oracle (the default one, or a
    deliberately broken copy that the pin tests use to show that they catch mistakes)."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        lib = ctypes.CDLL(lib_path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f16_to_f32.restype = ctypes.c_float
        lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_quantize_weights.restype = ctypes.c_int
        lib.orc_quantize_weights.argtypes = [p, i64, i64, i64, p, p, p]
        lib.orc_dequantize_weights.restype = None
        lib.orc_dequantize_weights.argtypes = [p, p, p, i64, i64, i64, p]
        lib.orc_pack_nibbles.restype = ctypes.c_int
        lib.orc_pack_nibbles.argtypes = [p, i64, i64, p]
        lib.orc_quantize_weights_sym.restype = ctypes.c_int
        lib.orc_quantize_weights_sym.argtypes = [p, i64, i64, i64, p, p, p]
        lib.orc_percentile.restype = ctypes.c_double
        lib.orc_percentile.argtypes = [p, i64, ctypes.c_double]
        lib.orc_clip_rows.restype = None
        lib.orc_clip_rows.argtypes = [p, i64, i64, ctypes.c_double, p]
        lib.orc_channel_absmax.restype = None
        lib.orc_channel_absmax.argtypes = [p, i64, i64, p]
        lib.orc_smooth_factors.restype = None
        lib.orc_smooth_factors.argtypes = [p, p, i64, ctypes.c_double, p, p]
        lib.orc_smooth_weights.restype = None
        lib.orc_smooth_weights.argtypes = [p, i64, i64, p, p]
        lib.orc_quantize_act_smooth.restype = None
        lib.orc_quantize_act_smooth.argtypes = [p, i64, i64, i64, p, p, p]
        lib.orc_unpack_nibbles.restype = None
        lib.orc_unpack_nibbles.argtypes = [p, i64, i64, p]
        lib.orc_quantize_act.restype = None
        lib.orc_quantize_act.argtypes = [p, i64, i64, i64, p, p]
        lib.orc_group_isums.restype = None
        lib.orc_group_isums.argtypes = [p, p, p, i64, i64, i64, i64, p]
        lib.orc_gemm_at.restype = None
        lib.orc_gemm_at.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, p, i64, p, p]
        lib.orc_gemm.restype = None
        lib.orc_gemm.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, p]
        lib.orc_route_topk.restype = ctypes.c_int
        lib.orc_route_topk.argtypes = [p, i64, i32, i32, p, p]
        lib.orc_bucket.restype = ctypes.c_int
        lib.orc_bucket.argtypes = [p, i64, i32, p, p]
        lib.orc_silu_mul.restype = None
        lib.orc_silu_mul.argtypes = [p, i64, i64, p]
        lib.orc_combine.restype = None
        lib.orc_combine.argtypes = [p, p, p, p, i64, i32, i64, p]
        self.lib = lib

    # --------------------------------------------------------------------------- fp16
    def num_threads(self) -> int:
        """Host threads the oracle's parallel loops run on."""
        return int(self.lib.orc_num_threads())

    def f32_to_f16_bits(self, x) -> np.ndarray:
        """fp32 -> fp16 bit pattern, round to nearest even (binary16 definition)."""
        lib = self.lib
        x = np.asarray(x, dtype=np.float32).ravel()
        return np.array([lib.orc_f32_to_f16(float(v)) for v in x], dtype=np.uint16)


    def f16_bits_to_f32(self, h) -> np.ndarray:
        lib = self.lib
        h = np.asarray(h, dtype=np.uint16).ravel()
        return np.array([lib.orc_f16_to_f32(int(v)) for v in h], dtype=np.float32)


    # --------------------------------------------------------------------------- O1
    def quantize_weights(self, W: np.ndarray, group: int = 128):
        """[p2 §2.1-2.2] group-wise asymmetric 4-bit quantization of W[N][K].

        Returns (q[N][K] uint8 codes, scale[G][N] fp16 bits, zp[G][N] fp16 bits)."""
        lib = self.lib
        W = _c(W, np.float32)
        N, K = W.shape
        G = K // group
        q = np.empty((N, K), np.uint8)
        s = np.empty((G, N), np.uint16)
        z = np.empty((G, N), np.uint16)
        rc = lib.orc_quantize_weights(_ptr(W), N, K, group, _ptr(q), _ptr(s), _ptr(z))
        if rc != 0:
            raise ValueError("oracle: weights cannot be quantized (sizes, non-finite input or fp16 overflow)")
        return q, s, z


    def dequantize_weights(self, q, scale16, zp16, group: int = 128) -> np.ndarray:
        lib = self.lib
        q = _c(q, np.uint8)
        N, K = q.shape
        out = np.empty((N, K), np.float64)
        lib.orc_dequantize_weights(_ptr(q), _ptr(_c(scale16, np.uint16)), _ptr(_c(zp16, np.uint16)),
                                   N, K, group, _ptr(out))
        return out


    def pack_nibbles(self, q: np.ndarray) -> np.ndarray:
        """[p2 §2.2] two codes per byte, first code in the low nibble."""
        lib = self.lib
        q = _c(q, np.uint8)
        N, K = q.shape
        out = np.empty((N, K // 2), np.uint8)
        if lib.orc_pack_nibbles(_ptr(q), N, K, _ptr(out)) != 0:
            raise ValueError("oracle: codes out of range or odd K")
        return out


    def unpack_nibbles(self, packed: np.ndarray, K: int) -> np.ndarray:
        lib = self.lib
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        out = np.empty((N, K), np.uint8)
        lib.orc_unpack_nibbles(_ptr(packed), N, K, _ptr(out))
        return out


    # --------------------------------------------------------------------------- O2
    def quantize_act(self, x: np.ndarray):
        """[p1 §5.3, p3 §2.1] per-token symmetric INT8: returns (qa[M][K] int8, a_scale[M] fp32)."""
        lib = self.lib
        x = _c(x, np.float32)
        M, K = x.shape
        qa = np.empty((M, K), np.int8)
        sc = np.empty((M,), np.float32)
        lib.orc_quantize_act(_ptr(x), M, K, K, _ptr(qa), _ptr(sc))
        return qa, sc


    # --------------------------------------------------------------------------- O9/O10
    def quantize_weights_sym(self, W, group: int = 128):
        """[p3 §2.1] symmetric 4-bit: (codes q+8 uint8 [N][K], scale fp16 bits [G][N], zp fp16 bits = 8)."""
        W = _c(W, np.float32)
        N, K = W.shape
        q = np.empty((N, K), np.uint8)
        sc = np.empty((K // group, N), np.uint16)
        zp = np.empty((K // group, N), np.uint16)
        rc = self.lib.orc_quantize_weights_sym(_ptr(W), N, K, group, _ptr(q), _ptr(sc), _ptr(zp))
        if rc != 0:
            raise ValueError("orc_quantize_weights_sym rejected the input")
        return q, sc, zp

    def percentile(self, v, pct: float) -> float:
        """Linear-interpolation percentile of a float32 vector, in double."""
        v = _c(v, np.float32)
        return self.lib.orc_percentile(_ptr(v), v.shape[0], float(pct))

    def clip_rows(self, W, pct: float) -> np.ndarray:
        """[p2 §2.2, §5.1] each row clamped to its [100-pct, pct] percentiles (fp32)."""
        W = _c(W, np.float32)
        N, K = W.shape
        out = np.empty((N, K), np.float32)
        self.lib.orc_clip_rows(_ptr(W), N, K, float(pct), _ptr(out))
        return out

    # --------------------------------------------------------------------------- O8
    def channel_absmax(self, A: np.ndarray) -> np.ndarray:
        """max over rows of |A[r][k]| (fp32 [K])."""
        A = _c(A, np.float32)
        rows, K = A.shape
        out = np.empty((K,), np.float32)
        self.lib.orc_channel_absmax(_ptr(A), rows, K, _ptr(out))
        return out

    def smooth_factors(self, ax, aw, alpha: float = 0.5):
        """[p3 §3.4] per-channel smoothing factors s and 1/s (fp32 [K] each)."""
        ax = _c(ax, np.float32)
        aw = _c(aw, np.float32)
        K = ax.shape[0]
        s = np.empty((K,), np.float32)
        inv = np.empty((K,), np.float32)
        self.lib.orc_smooth_factors(_ptr(ax), _ptr(aw), K, float(alpha), _ptr(s), _ptr(inv))
        return s, inv

    def smooth_weights(self, W, s) -> np.ndarray:
        """W[n][k] * s[k] (fp32)."""
        W = _c(W, np.float32)
        N, K = W.shape
        out = np.empty((N, K), np.float32)
        self.lib.orc_smooth_weights(_ptr(W), N, K, _ptr(_c(s, np.float32)), _ptr(out))
        return out

    def quantize_act_smooth(self, x, inv_s):
        """Per-token INT8 of x[m][k] * inv_s[k]: (qa int8 [M][K], a_scale fp32 [M])."""
        x = _c(x, np.float32)
        M, K = x.shape
        qa = np.empty((M, K), np.int8)
        sc = np.empty((M,), np.float32)
        self.lib.orc_quantize_act_smooth(_ptr(x), M, K, K, _ptr(_c(inv_s, np.float32)), _ptr(qa), _ptr(sc))
        return qa, sc

    # --------------------------------------------------------------------------- O3/O4
    def group_isums(self, qa, q, zp16, group: int = 128) -> np.ndarray:
        """[p2 §3.2, §5.4] isum[g][m][n] with int32 accumulation."""
        lib = self.lib
        qa = _c(qa, np.int8)
        q = _c(q, np.uint8)
        M, K = qa.shape
        N = q.shape[0]
        out = np.empty((K // group, M, N), np.int32)
        lib.orc_group_isums(_ptr(qa), _ptr(q), _ptr(_c(zp16, np.uint16)), M, N, K, group, _ptr(out))
        return out


    def gemm(self, qa, a_scale, q, scale16, zp16, group: int = 128):
        """Full reference output (double) and the tolerance magnitude sum_g |terms|."""
        lib = self.lib
        qa = _c(qa, np.int8)
        q = _c(q, np.uint8)
        M, K = qa.shape
        N = q.shape[0]
        out = np.empty((M, N), np.float64)
        mag = np.empty((M, N), np.float64)
        lib.orc_gemm(_ptr(qa), _ptr(_c(a_scale, np.float32)), _ptr(q), _ptr(_c(scale16, np.uint16)),
                     _ptr(_c(zp16, np.uint16)), M, N, K, group, _ptr(out), _ptr(mag))
        return out, mag


    def gemm_at(self, qa, a_scale, q, scale16, zp16, ms, ns, group: int = 128):
        """Reference outputs at sampled (m, n) positions (double) and their magnitudes."""
        lib = self.lib
        qa = _c(qa, np.int8)
        q = _c(q, np.uint8)
        M, K = qa.shape
        N = q.shape[0]
        ms = _c(ms, np.int64)
        ns = _c(ns, np.int64)
        assert ms.shape == ns.shape
        assert (ms >= 0).all() and (ms < M).all() and (ns >= 0).all() and (ns < N).all()
        out = np.empty(ms.shape, np.float64)
        mag = np.empty(ms.shape, np.float64)
        lib.orc_gemm_at(_ptr(qa), _ptr(_c(a_scale, np.float32)), _ptr(q), _ptr(_c(scale16, np.uint16)),
                        _ptr(_c(zp16, np.uint16)), M, N, K, group, _ptr(ms), _ptr(ns), ms.size,
                        _ptr(out), _ptr(mag))
        return out, mag


    def tolerance(self, mag):
        """Pass bound for fp32 outputs: 1e-5 * sum_g |a_scale * w_scale * isum_g| + 1e-6."""
        return 1e-5 * np.asarray(mag) + 1e-6


    # --------------------------------------------------------------------------- O5
    def route_topk(self, logits: np.ndarray, k: int):
        """[p1 §5.2] top-k experts per token (ties -> lower id), softmax weights over the k."""
        lib = self.lib
        logits = _c(logits, np.float32)
        T, E = logits.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float32)
        if lib.orc_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w)) != 0:
            raise ValueError("oracle: bad routing sizes")
        return ids, w


    def bucket(self, ids: np.ndarray, E: int):
        """Per-expert offsets (E+1) and the stable expert-sorted list of pair indices."""
        lib = self.lib
        ids = _c(ids, np.int32).ravel()
        off = np.empty((E + 1,), np.int32)
        perm = np.empty(ids.shape, np.int32)
        if lib.orc_bucket(_ptr(ids), ids.size, E, _ptr(off), _ptr(perm)) != 0:
            raise ValueError("oracle: expert id out of range")
        return off, perm


    def silu_mul(self, gu: np.ndarray) -> np.ndarray:
        lib = self.lib
        gu = _c(gu, np.float32)
        P, twoI = gu.shape
        out = np.empty((P, twoI // 2), np.float64)
        lib.orc_silu_mul(_ptr(gu), P, twoI // 2, _ptr(out))
        return out


    def combine(self, y, slot_of_pair, w, y_shared=None) -> np.ndarray:
        lib = self.lib
        y = _c(y, np.float32)
        w = _c(w, np.float32)
        T, k = w.shape
        H = y.shape[1]
        sop = _c(slot_of_pair, np.int32)
        out = np.empty((T, H), np.float64)
        ys = _ptr(_c(y_shared, np.float32)) if y_shared is not None else None
        lib.orc_combine(_ptr(y), _ptr(sop), _ptr(w), ys, T, k, H, _ptr(out))
        return out


# --------------------------------------------------------------------------- toy router [p4]
def toy_router_expected_unique(experts: int, tokens: int) -> float:
    """[p4] closed form: each of E experts is missed by one uniform top-1 token with
    probability (E-1)/E, by all B tokens with ((E-1)/E)^B; E[unique] = E(1 - ((E-1)/E)^B)."""
    return experts * (1.0 - (1.0 - 1.0 / experts) ** tokens)


def toy_router_exhaustive(experts: int, tokens: int) -> float:
    """[p4] average number of distinct experts over all E^B equally likely top-1 routings,
    by brute force: routing r in [0, E^B) assigns token i the i-th base-E digit of r."""
    total = 0
    count = experts ** tokens
    for r in range(count):
        touched = 0
        for _ in range(tokens):
            touched |= 1 << (r % experts)
            r //= experts
        total += bin(touched).count("1")
    return total / count


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # module-level access to the default oracle's methods: oracle.quantize_act(...) etc.
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
