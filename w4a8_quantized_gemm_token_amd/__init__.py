"""Python binding of libw4a8.so, the MI355X (gfx950) W4A8 linear-layer library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels (or, for ``pack_weights``, its host packer).  torch provides device
memory and the current stream; nothing here computes any part of the method.
The C names and argument meanings are documented in ``include/w4a8.h``.

Loading fails loudly (ImportError at first use) when the library is missing or
no GPU is present for a device call -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

GROUP = 128
ABI_VERSION = 6          # W4A8_ABI_VERSION of the header this binding follows
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a8.so")

# names exported by include/w4a8.h (checked by the test suite against the header)
EXPORTS = (
    "w4a8_abi_version", "w4a8_status_str", "w4a8_last_error",
    "w4a8_pack_weights", "w4a8_pack_weights_ex", "w4a8_pack_weights_device", "w4a8_unpack_weights",
    "w4a8_quantize_act", "w4a8_gemm", "w4a8_gemm_debug_isums", "w4a8_gemm_path",
    "w4a8_tm_bytes", "w4a8_weights_to_tm", "w4a8_gemm_tm",
    "w4a8_channel_absmax", "w4a8_smooth_factors", "w4a8_pack_weights_device_smooth", "w4a8_quantize_act_smooth",
    "w4a8_moe_route", "w4a8_moe_grouped_gemm", "w4a8_moe_grouped_gemm_debug_isums", "w4a8_silu_mul_quantize",
    "w4a8_moe_combine",
    "w4a8_moe_ffn_workspace_size", "w4a8_moe_ffn_workspace_layout", "w4a8_moe_ffn",
    "w4a8_moe_ffn_noalloc_max_bytes", "w4a8_moe_ffn_noalloc",
)
# order of the parts of the MoE FFN workspace (enum w4a8_moe_ws_part)
WS_PARTS = ("ids", "w", "offsets", "perm", "row_index", "slot_of_pair", "qa", "a_scale", "gu", "qh",
            "h_scale", "y")

_lib = None


class W4A8Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libw4a8.so (built in-tree by build.py); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python w4a8_quantized_gemm_token_amd/build.py` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "w4a8_abi_version": (ctypes.c_int, []),
        "w4a8_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "w4a8_last_error": (ctypes.c_char_p, []),
        "w4a8_pack_weights": (ctypes.c_int, [p, i64, i64, i32, p, p, p]),
        "w4a8_pack_weights_ex": (ctypes.c_int, [p, i64, i64, i32, i32, ctypes.c_double, p, p, p]),
        "w4a8_pack_weights_device": (ctypes.c_int, [p, i64, i64, i32, p, p, p, p]),
        "w4a8_unpack_weights": (ctypes.c_int, [p, p, p, i64, i64, i32, p, p]),
        "w4a8_quantize_act": (ctypes.c_int, [p, i64, i64, i64, p, p, p]),
        "w4a8_gemm": (ctypes.c_int, [p, p, i64, i64, p, p, p, i64, i32, p, p]),
        "w4a8_gemm_debug_isums": (ctypes.c_int, [p, i64, i64, p, p, i64, i32, i32, p, p]),
        "w4a8_gemm_path": (ctypes.c_int, [p, p, i64, i64, p, p, p, i64, i32, i32, p, p]),
        "w4a8_channel_absmax": (ctypes.c_int, [p, i64, i64, i64, p, p]),
        "w4a8_smooth_factors": (ctypes.c_int, [p, p, i64, ctypes.c_double, p, p]),
        "w4a8_pack_weights_device_smooth": (ctypes.c_int, [p, i64, i64, i32, p, p, p, p, p]),
        "w4a8_quantize_act_smooth": (ctypes.c_int, [p, i64, i64, i64, p, p, p, p]),
        "w4a8_tm_bytes": (sz, [i64, i64]),
        "w4a8_weights_to_tm": (ctypes.c_int, [p, p, p, i64, i64, i32, p, p]),
        "w4a8_gemm_tm": (ctypes.c_int, [p, p, i64, i64, p, i64, i32, p, p]),
        "w4a8_moe_route": (ctypes.c_int, [p, i64, i32, i32, i32, p, p, p, p, p, p, p]),
        "w4a8_moe_grouped_gemm": (ctypes.c_int, [p, p, i64, p, p, i32, i64, p, p, p, i64, i32, i64, p, p]),
        "w4a8_moe_grouped_gemm_debug_isums": (ctypes.c_int, [p, i64, p, p, i32, i64, p, p, i64, i32, i64, p, p]),
        "w4a8_silu_mul_quantize": (ctypes.c_int, [p, i64, i64, p, p, p, p]),
        "w4a8_moe_combine": (ctypes.c_int, [p, p, p, p, i64, i32, i64, p, p]),
        "w4a8_moe_ffn_workspace_size": (sz, [i64, i64, i64, i32, i32]),
        "w4a8_moe_ffn_workspace_layout": (ctypes.c_int, [i64, i64, i64, i32, i32, p]),
        "w4a8_moe_ffn": (ctypes.c_int, [p, p, i64, i64, i64, i32, i32, p, p, p, p, p, p, p, p, sz, p]),
        "w4a8_moe_ffn_noalloc_max_bytes": (sz, []),
        "w4a8_moe_ffn_noalloc": (ctypes.c_int, [p, p, i64, i64, i64, i32, i32, p, p, p, p, p, p, p, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.w4a8_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.w4a8_abi_version()}, this binding needs {ABI_VERSION}: "
                          "rebuild it")
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        lib = load()
        raise W4A8Error(fn, status, lib.w4a8_last_error().decode(errors="replace"))


def _call(name: str, *args):
    _check(name, getattr(load(), name)(*args))


class Launch:
    """One library call with its arguments marshalled once (device pointers, sizes and the
    stream current at preparation time).  Calling it re-issues the call with no per-call
    Python work beyond the ctypes dispatch; the tensors it was prepared from must stay alive.
    Raises W4A8Error on a non-zero status."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.name = name
        self.fn = getattr(load(), name)
        self.args = args
        self.keep = keep

    def __call__(self):
        status = self.fn(*self.args)
        if status != 0:
            _check(self.name, status)


# ----------------------------------------------------------------- torch plumbing
def _torch():
    import torch
    return torch


def _dev_ptr(t):
    if t is None:
        return None
    torch = _torch()
    assert isinstance(t, torch.Tensor) and t.is_cuda, "device tensor expected"
    assert t.is_contiguous(), "contiguous tensor expected"
    return ctypes.c_void_p(t.data_ptr())


def _dev_rows_ptr(t):
    """Device pointer of a 2-D tensor whose rows may be strided (unit stride inside a row)."""
    torch = _torch()
    assert isinstance(t, torch.Tensor) and t.is_cuda and t.dim() == 2, "2-D device tensor expected"
    assert t.stride(1) == 1 or t.shape[1] <= 1 or t.shape[0] == 0, "rows must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _empty(shape, dtype, like):
    torch = _torch()
    return torch.empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------- packing
def pack_weights(W: np.ndarray, group: int = GROUP, symmetric: bool = False, clip_percent: float = 100.0):
    """Host packer: W float32 [N][K] (numpy) -> (packed u8 [N][K/2], scale u16 [G][N], zp u16 [G][N]).
    symmetric / clip_percent select the w4a8_pack_weights_ex variants (same stored format)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    G = K // group if group else 0
    packed = np.empty((N, K // 2), np.uint8)
    scale = np.empty((max(G, 1), N), np.uint16)
    zp = np.empty((max(G, 1), N), np.uint16)
    vp = ctypes.c_void_p
    if symmetric or clip_percent != 100.0:
        _call("w4a8_pack_weights_ex", W.ctypes.data_as(vp), N, K, group, 1 if symmetric else 0, float(clip_percent),
              packed.ctypes.data_as(vp), scale.ctypes.data_as(vp), zp.ctypes.data_as(vp))
    else:
        _call("w4a8_pack_weights", W.ctypes.data_as(vp), N, K, group, packed.ctypes.data_as(vp),
              scale.ctypes.data_as(vp), zp.ctypes.data_as(vp))
    return packed, scale, zp


def unpack_weights(packed: np.ndarray, scale: np.ndarray, zp: np.ndarray, group: int = GROUP):
    """Host: (codes u8 [N][K], dequantized float32 [N][K])."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N, K2 = packed.shape
    K = 2 * K2
    q = np.empty((N, K), np.uint8)
    w = np.empty((N, K), np.float32)
    vp = ctypes.c_void_p
    _call("w4a8_unpack_weights", packed.ctypes.data_as(vp),
          np.ascontiguousarray(scale, np.uint16).ctypes.data_as(vp),
          np.ascontiguousarray(zp, np.uint16).ctypes.data_as(vp), N, K, group,
          q.ctypes.data_as(vp), w.ctypes.data_as(vp))
    return q, w


def pack_weights_device(W, group: int = GROUP, out=None):
    """Device packer: W float32 [N][K] (device) -> (packed u8, scale i16-bits, zp i16-bits) device
    tensors.  `out` may pass preallocated (packed, scale, zp) views to fill."""
    torch = _torch()
    N, K = W.shape
    if out is None:
        out = (_empty((N, K // 2), torch.uint8, W), _empty((K // group, N), torch.int16, W),
               _empty((K // group, N), torch.int16, W))
    packed, scale, zp = out
    _call("w4a8_pack_weights_device", _dev_ptr(W), N, K, group, _dev_ptr(packed), _dev_ptr(scale),
          _dev_ptr(zp), _stream(W.device))
    return packed, scale, zp


# ----------------------------------------------------------------- layer
def quantize_act(x):
    """x float32 [M][K] (device) -> (qa int8 [M][K], a_scale float32 [M])."""
    torch = _torch()
    M, K = x.shape
    qa = _empty((M, K), torch.int8, x)
    sc = _empty((M,), torch.float32, x)
    _call("w4a8_quantize_act", _dev_rows_ptr(x), M, K, x.stride(0), _dev_ptr(qa), _dev_ptr(sc),
          _stream(x.device))
    return qa, sc


def gemm(qa, a_scale, packed, scale, zp, path: int = 0, out=None, group: int = GROUP):
    """out float32 [M][N] = W4A8 product of the quantized activations and packed weights."""
    torch = _torch()
    M, K = qa.shape
    N = packed.shape[0]
    if out is None:
        out = _empty((M, N), torch.float32, qa)
    _call("w4a8_gemm_path", _dev_ptr(qa), _dev_ptr(a_scale), M, K, _dev_ptr(packed), _dev_ptr(scale),
          _dev_ptr(zp), N, group, path, _dev_ptr(out), _stream(qa.device))
    return out


# ----------------------------------------------------------------- smoothing [p3 §3.4]
def channel_absmax(A):
    """A float32 [rows][K] (device, unit column stride) -> max over rows of |A| (float32 [K], device)."""
    torch = _torch()
    rows, K = A.shape
    out = _empty((K,), torch.float32, A)
    _call("w4a8_channel_absmax", _dev_rows_ptr(A), rows, K, A.stride(0) if rows else K, _dev_ptr(out),
          _stream(A.device))
    return out


def smooth_factors(ax: np.ndarray, aw: np.ndarray, alpha: float = 0.5):
    """Host: (s, inv_s) float32 [K] from the activation and weight channel maxima."""
    ax = np.ascontiguousarray(ax, np.float32)
    aw = np.ascontiguousarray(aw, np.float32)
    K = ax.shape[0]
    assert aw.shape == (K,)
    s = np.empty((K,), np.float32)
    inv = np.empty((K,), np.float32)
    vp = ctypes.c_void_p
    _call("w4a8_smooth_factors", ax.ctypes.data_as(vp), aw.ctypes.data_as(vp), K, float(alpha),
          s.ctypes.data_as(vp), inv.ctypes.data_as(vp))
    return s, inv


def pack_weights_device_smooth(W, s, group: int = GROUP):
    """Device packer of the smoothed weights W[n][k] * s[k] (W float32 [N][K], s float32 [K], device)."""
    torch = _torch()
    N, K = W.shape
    assert tuple(s.shape) == (K,) and s.is_contiguous()
    out = (_empty((N, K // 2), torch.uint8, W), _empty((K // group, N), torch.int16, W),
           _empty((K // group, N), torch.int16, W))
    _call("w4a8_pack_weights_device_smooth", _dev_ptr(W), N, K, group, _dev_ptr(s), _dev_ptr(out[0]),
          _dev_ptr(out[1]), _dev_ptr(out[2]), _stream(W.device))
    return out


def quantize_act_smooth(x, inv_s):
    """Per-token INT8 of x[m][k] * inv_s[k] (device): (qa int8 [M][K], a_scale float32 [M])."""
    torch = _torch()
    M, K = x.shape
    assert tuple(inv_s.shape) == (K,) and inv_s.is_contiguous()
    qa = _empty((M, K), torch.int8, x)
    sc = _empty((M,), torch.float32, x)
    _call("w4a8_quantize_act_smooth", _dev_rows_ptr(x), M, K, x.stride(0), _dev_ptr(inv_s), _dev_ptr(qa),
          _dev_ptr(sc), _stream(x.device))
    return qa, sc


def prepare_quantize_act_smooth(x, inv_s, qa, a_scale) -> Launch:
    """Prepared w4a8_quantize_act_smooth writing into preallocated qa and a_scale."""
    M, K = x.shape
    assert tuple(qa.shape) == (M, K) and tuple(a_scale.shape) == (M,) and tuple(inv_s.shape) == (K,)
    return Launch("w4a8_quantize_act_smooth", (_dev_rows_ptr(x), M, K, x.stride(0), _dev_ptr(inv_s), _dev_ptr(qa),
                                               _dev_ptr(a_scale), _stream(x.device)), (x, inv_s, qa, a_scale))


def prepare_quantize_act(x, qa, a_scale) -> Launch:
    """Prepared w4a8_quantize_act writing into preallocated qa int8 [M][K] and a_scale float32 [M]."""
    M, K = x.shape
    assert tuple(qa.shape) == (M, K) and tuple(a_scale.shape) == (M,)
    return Launch("w4a8_quantize_act", (_dev_rows_ptr(x), M, K, x.stride(0), _dev_ptr(qa), _dev_ptr(a_scale),
                                        _stream(x.device)), (x, qa, a_scale))


def prepare_gemm(qa, a_scale, packed, scale, zp, out, group: int = GROUP, path: int = 0) -> Launch:
    """Prepared w4a8_gemm (path 0) or w4a8_gemm_path writing into a preallocated out
    float32 [M][N]."""
    M, K = qa.shape
    N = packed.shape[0]
    assert tuple(out.shape) == (M, N)
    if path:
        return Launch("w4a8_gemm_path", (_dev_ptr(qa), _dev_ptr(a_scale), M, K, _dev_ptr(packed), _dev_ptr(scale),
                                         _dev_ptr(zp), N, group, path, _dev_ptr(out), _stream(qa.device)),
                      (qa, a_scale, packed, scale, zp, out))
    return Launch("w4a8_gemm", (_dev_ptr(qa), _dev_ptr(a_scale), M, K, _dev_ptr(packed), _dev_ptr(scale),
                                _dev_ptr(zp), N, group, _dev_ptr(out), _stream(qa.device)),
                  (qa, a_scale, packed, scale, zp, out))


def gemm_debug_isums(qa, packed, zp, path: int = 0, group: int = GROUP):
    """int32 [K/group][M][N] per-group integer sums (test aid)."""
    torch = _torch()
    M, K = qa.shape
    N = packed.shape[0]
    isums = _empty((K // group, M, N), torch.int32, qa)
    _call("w4a8_gemm_debug_isums", _dev_ptr(qa), M, K, _dev_ptr(packed), _dev_ptr(zp), N, group, path,
          _dev_ptr(isums), _stream(qa.device))
    return isums


def tm_bytes(N: int, K: int) -> int:
    """Bytes of the tile-major weight array for an N x K weight (0 if the shape has none)."""
    return int(load().w4a8_tm_bytes(N, K))


def weights_to_tm(packed, scale, zp, group: int = GROUP, out=None):
    """Tile-major copy (uint8 [N/16][K/256][2176]) of standard-layout device weights."""
    torch = _torch()
    N = packed.shape[0]
    K = 2 * packed.shape[1]
    if out is None:
        out = _empty((N // 16, K // 256, 2176), torch.uint8, packed)
    _call("w4a8_weights_to_tm", _dev_ptr(packed), _dev_ptr(scale), _dev_ptr(zp), N, K, group, _dev_ptr(out),
          _stream(packed.device))
    return out


def _tm_n(tm) -> int:
    return 16 * tm.shape[0]


def gemm_tm(qa, a_scale, tm, out=None, group: int = GROUP):
    """out float32 [M][N] from tile-major weights: the same bytes as gemm() for M <= 16 (decode
    loop) and as gemm(..., path=5) above (the 256x256 tiled loop)."""
    torch = _torch()
    M, K = qa.shape
    N = _tm_n(tm)
    if out is None:
        out = _empty((M, N), torch.float32, qa)
    _call("w4a8_gemm_tm", _dev_ptr(qa), _dev_ptr(a_scale), M, K, _dev_ptr(tm), N, group, _dev_ptr(out),
          _stream(qa.device))
    return out


def prepare_gemm_tm(qa, a_scale, tm, out, group: int = GROUP) -> Launch:
    """Prepared w4a8_gemm_tm writing into a preallocated out float32 [M][N]."""
    M, K = qa.shape
    N = _tm_n(tm)
    assert tuple(out.shape) == (M, N)
    return Launch("w4a8_gemm_tm", (_dev_ptr(qa), _dev_ptr(a_scale), M, K, _dev_ptr(tm), N, group, _dev_ptr(out),
                                   _stream(qa.device)), (qa, a_scale, tm, out))


def linear(x, packed, scale, zp, path: int = 0):
    """Quantize x per token and run the W4A8 product: float32 [M][N]."""
    qa, sc = quantize_act(x)
    return gemm(qa, sc, packed, scale, zp, path=path)


# ----------------------------------------------------------------- MoE
def moe_route(logits, topk: int, with_shared: bool = False):
    """-> (ids [T][k] i32, w [T][k] f32, offsets [E+1(+1)] i32, perm [T*k] i32,
    row_index [T*k(+T)] i32, slot_of_pair [T*k] i32).  with_shared appends a shared expert
    (index E) visited by every token; row_index is the activation row of each slot."""
    torch = _torch()
    T, E = logits.shape
    sh = 1 if with_shared else 0
    ids = _empty((T, topk), torch.int32, logits)
    w = _empty((T, topk), torch.float32, logits)
    off = _empty((E + 1 + sh,), torch.int32, logits)
    perm = _empty((T * topk,), torch.int32, logits)
    rows = _empty((T * topk + sh * T,), torch.int32, logits)
    sop = _empty((T * topk,), torch.int32, logits)
    _call("w4a8_moe_route", _dev_ptr(logits), T, E, topk, sh, _dev_ptr(ids), _dev_ptr(w), _dev_ptr(off),
          _dev_ptr(perm), _dev_ptr(rows), _dev_ptr(sop), _stream(logits.device))
    return ids, w, off, perm, rows, sop


def moe_grouped_gemm(qa, a_scale, row_index, offsets, packed, scale, zp, max_slots: int, out=None,
                     group: int = GROUP):
    """Expert-grouped product: out[s] = W4A8(qa[row_index[s]], expert of slot s).  packed [E][N][K/2]."""
    torch = _torch()
    R, K = qa.shape
    E, N = packed.shape[0], packed.shape[1]
    if out is None:
        out = _empty((max_slots, N), torch.float32, qa)
    _call("w4a8_moe_grouped_gemm", _dev_ptr(qa), _dev_ptr(a_scale), R, _dev_ptr(row_index), _dev_ptr(offsets),
          E, K, _dev_ptr(packed), _dev_ptr(scale), _dev_ptr(zp), N, group, max_slots, _dev_ptr(out),
          _stream(qa.device))
    return out


def moe_grouped_gemm_debug_isums(qa, row_index, offsets, packed, zp, max_slots: int, group: int = GROUP):
    """int32 [K/group][max_slots][N] per-group integer sums of every slot (test aid)."""
    torch = _torch()
    R, K = qa.shape
    E, N = packed.shape[0], packed.shape[1]
    isums = torch.zeros((K // group, max_slots, N), dtype=torch.int32, device=qa.device)
    _call("w4a8_moe_grouped_gemm_debug_isums", _dev_ptr(qa), R, _dev_ptr(row_index), _dev_ptr(offsets), E, K,
          _dev_ptr(packed), _dev_ptr(zp), N, group, max_slots, _dev_ptr(isums), _stream(qa.device))
    return isums


def pack_experts_device(E: int, N: int, K: int, fill, device, group: int = GROUP, out=None):
    """Stacked expert weights from the device packer: (packed u8 [E][N][K/2], scale, zp i16-bits
    [E][K/group][N]).  fill(e, W) writes expert e's fp32 weights into the device tensor W [N][K];
    one fp32 buffer is reused for all experts."""
    torch = _torch()
    G = K // group
    if out is None:
        out = (torch.empty((E, N, K // 2), dtype=torch.uint8, device=device),
               torch.empty((E, G, N), dtype=torch.int16, device=device),
               torch.empty((E, G, N), dtype=torch.int16, device=device))
    packed, scale, zp = out
    W = torch.empty((N, K), dtype=torch.float32, device=device)
    for e in range(E):
        fill(e, W)
        pack_weights_device(W, group=group, out=(packed[e], scale[e], zp[e]))
    del W
    return packed, scale, zp


def prepare_moe_route(logits, topk: int, outs) -> Launch:
    """Prepared w4a8_moe_route (no shared expert) into outs = (ids, w, offsets, perm, row_index,
    slot_of_pair), shaped as moe_route returns them."""
    T, E = logits.shape
    ids, w, off, perm, rows, sop = outs
    assert tuple(ids.shape) == (T, topk) and tuple(off.shape) == (E + 1,) and tuple(rows.shape) == (T * topk,)
    return Launch("w4a8_moe_route", (_dev_ptr(logits), T, E, topk, 0, _dev_ptr(ids), _dev_ptr(w), _dev_ptr(off),
                                     _dev_ptr(perm), _dev_ptr(rows), _dev_ptr(sop), _stream(logits.device)),
                  (logits,) + tuple(outs))


def prepare_moe_grouped_gemm(qa, a_scale, row_index, offsets, packed, scale, zp, max_slots: int, out,
                             group: int = GROUP) -> Launch:
    """Prepared w4a8_moe_grouped_gemm writing into a preallocated out float32 [max_slots][N]."""
    R, K = qa.shape
    E, N = packed.shape[0], packed.shape[1]
    assert tuple(out.shape) == (max_slots, N)
    return Launch("w4a8_moe_grouped_gemm", (_dev_ptr(qa), _dev_ptr(a_scale), R, _dev_ptr(row_index),
                                            _dev_ptr(offsets), E, K, _dev_ptr(packed), _dev_ptr(scale),
                                            _dev_ptr(zp), N, group, max_slots, _dev_ptr(out), _stream(qa.device)),
                  (qa, a_scale, row_index, offsets, packed, scale, zp, out))


def prepare_moe_combine(y, slot_of_pair, topk_w, out) -> Launch:
    """Prepared w4a8_moe_combine (no shared expert) into a preallocated out float32 [T][H]."""
    T, k = topk_w.shape
    H = y.shape[1]
    assert tuple(out.shape) == (T, H)
    return Launch("w4a8_moe_combine", (_dev_ptr(y), _dev_ptr(slot_of_pair), _dev_ptr(topk_w), None, T, k, H,
                                       _dev_ptr(out), _stream(y.device)), (y, slot_of_pair, topk_w, out))


def silu_mul_quantize(gu, want_h: bool = False):
    """gu float32 [P][2I] -> (qh int8 [P][I], h_scale float32 [P][, h float32 [P][I]])."""
    torch = _torch()
    P, twoI = gu.shape
    I = twoI // 2
    qh = _empty((P, I), torch.int8, gu)
    hs = _empty((P,), torch.float32, gu)
    h = _empty((P, I), torch.float32, gu) if want_h else None
    _call("w4a8_silu_mul_quantize", _dev_ptr(gu), P, I, _dev_ptr(qh), _dev_ptr(hs), _dev_ptr(h),
          _stream(gu.device))
    return (qh, hs, h) if want_h else (qh, hs)


def moe_combine(y, slot_of_pair, topk_w, y_shared=None, out=None):
    torch = _torch()
    T, k = topk_w.shape
    H = y.shape[1]
    if out is None:
        out = _empty((T, H), torch.float32, y)
    _call("w4a8_moe_combine", _dev_ptr(y), _dev_ptr(slot_of_pair), _dev_ptr(topk_w), _dev_ptr(y_shared), T, k, H,
          _dev_ptr(out), _stream(y.device))
    return out


def moe_ffn_workspace(T: int, H: int, I: int, E: int, topk: int):
    """(total bytes, {part name: (byte offset, byte size)}) of the MoE FFN workspace."""
    lib = load()
    offs = (ctypes.c_int64 * (len(WS_PARTS) + 1))()
    _check("w4a8_moe_ffn_workspace_layout", lib.w4a8_moe_ffn_workspace_layout(T, H, I, E, topk, offs))
    parts = {name: (offs[i], offs[i + 1] - offs[i]) for i, name in enumerate(WS_PARTS)}
    return offs[len(WS_PARTS)], parts


def moe_ffn(x, logits, topk: int, gate_up, down, workspace=None, out=None):
    """One MoE FFN layer in one library call (w4a8_moe_ffn): route (+ shared expert at index E)
    -> quantize x -> gate/up grouped GEMM -> silu*up + INT8 requant -> down grouped GEMM -> combine.

    gate_up = (packed [E+1][2I][H/2], scale, zp); down = (packed [E+1][H][I/2], scale, zp).
    Returns (out [T][H] float32, intermediates: views of the workspace)."""
    torch = _torch()
    T, H = x.shape
    E = logits.shape[1]
    I = gate_up[0].shape[1] // 2
    total, parts = moe_ffn_workspace(T, H, I, E, topk)
    if workspace is None:
        workspace = torch.empty((total,), dtype=torch.uint8, device=x.device)
    assert workspace.numel() >= total and workspace.data_ptr() % 256 == 0, "workspace too small or misaligned"
    if out is None:
        out = _empty((T, H), torch.float32, x)
    _call("w4a8_moe_ffn", _dev_ptr(x), _dev_ptr(logits), T, H, I, E, topk, _dev_ptr(gate_up[0]),
          _dev_ptr(gate_up[1]), _dev_ptr(gate_up[2]), _dev_ptr(down[0]), _dev_ptr(down[1]), _dev_ptr(down[2]),
          _dev_ptr(out), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(x.device))
    P, S = T * topk, T * topk + T
    shapes = {"ids": ((T, topk), torch.int32), "w": ((T, topk), torch.float32), "offsets": ((E + 2,), torch.int32),
              "perm": ((P,), torch.int32), "row_index": ((S,), torch.int32), "slot_of_pair": ((P,), torch.int32),
              "qa": ((T, H), torch.int8), "a_scale": ((T,), torch.float32), "gu": ((S, 2 * I), torch.float32),
              "qh": ((S, I), torch.int8), "h_scale": ((S,), torch.float32), "y": ((S, H), torch.float32)}
    inter = {}
    for name, (shape, dt) in shapes.items():
        o, _ = parts[name]
        n = int(np.prod(shape)) * torch.empty((), dtype=dt).element_size()
        inter[name] = workspace[o:o + n].view(dt).view(shape)
    return out, inter


def moe_ffn_noalloc(x, logits, topk: int, gate_up, down, out=None):
    """w4a8_moe_ffn_noalloc: the MoE FFN layer with its intermediates in the library's fixed
    per-GPU scratch (no allocation inside the call; sizes above the scratch are rejected)."""
    torch = _torch()
    T, H = x.shape
    E = logits.shape[1]
    I = gate_up[0].shape[1] // 2
    if out is None:
        out = _empty((T, H), torch.float32, x)
    _call("w4a8_moe_ffn_noalloc", _dev_ptr(x), _dev_ptr(logits), T, H, I, E, topk, _dev_ptr(gate_up[0]),
          _dev_ptr(gate_up[1]), _dev_ptr(gate_up[2]), _dev_ptr(down[0]), _dev_ptr(down[1]), _dev_ptr(down[2]),
          _dev_ptr(out), _stream(x.device))
    return out


def moe_ffn_noalloc_max_bytes() -> int:
    return int(load().w4a8_moe_ffn_noalloc_max_bytes())
