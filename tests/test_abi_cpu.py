"""The C-ABI library on the CPU: it loads, exports every function include/w4a8.h
declares, rejects bad arguments before any launch, and its host packer is
bit-identical to the oracle's quantization + packing."""
import ctypes
import os
import re

import numpy as np
import pytest

import synthetic
import w4a8_quantized_gemm_token_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

EINVAL, EUNSUPPORTED, EWORKSPACE = 1, 2, 4


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a8_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_header_function():
    lib = w4.load()
    names = header_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), f"{name} declared in w4a8.h but not exported"
    assert sorted(w4.EXPORTS) == names
    version = int(re.search(r"#define W4A8_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.w4a8_abi_version() == version == w4.ABI_VERSION
    assert lib.w4a8_status_str(2) == b"unsupported"


P = ctypes.c_void_p


def _fake(addr=4096):
    return ctypes.c_void_p(addr)


def test_validation_rejects_before_launch():
    lib = w4.load()
    f = _fake()
    # null pointers
    assert lib.w4a8_gemm(None, f, 4, 256, f, f, f, 128, 128, f, None) == EINVAL
    # group sizes other than 64, 128, 256: unsupported, never a silent fallback
    assert lib.w4a8_gemm(f, f, 4, 256, f, f, f, 128, 32, f, None) == EUNSUPPORTED
    assert b"group" in lib.w4a8_last_error()
    # 64 and 256 take the decode loop (path 1) only for M <= 16 and K % 256 == 0
    assert lib.w4a8_gemm_path(f, f, 17, 256, f, f, f, 128, 64, 1, f, None) == EUNSUPPORTED
    assert lib.w4a8_gemm_path(f, f, 4, 384, f, f, f, 128, 64, 1, f, None) == EUNSUPPORTED
    assert lib.w4a8_gemm_path(f, f, 4, 384, f, f, f, 128, 256, 2, f, None) == EINVAL   # K % 256
    assert lib.w4a8_gemm_path(f, f, 0, 512, f, f, f, 128, 256, 0, f, None) == 0        # M == 0: no launch
    assert lib.w4a8_pack_weights_device(f, 16, 256, 32, f, f, f, None) == EUNSUPPORTED
    assert lib.w4a8_pack_weights_device(_fake(4104), 16, 256, 256, f, f, f, None) == EINVAL  # 16-byte W
    assert lib.w4a8_pack_weights_device(f, 16, 384, 256, f, f, f, None) == EINVAL            # K % group
    # K not a multiple of 128
    assert lib.w4a8_gemm(f, f, 4, 200, f, f, f, 128, 128, f, None) == EINVAL
    # N not a multiple of 16
    assert lib.w4a8_gemm(f, f, 4, 256, f, f, f, 120, 128, f, None) == EINVAL
    # misaligned packed pointer
    assert lib.w4a8_gemm(f, f, 4, 256, _fake(4097), f, f, 128, 128, f, None) == EINVAL
    assert b"aligned" in lib.w4a8_last_error()
    # negative M
    assert lib.w4a8_gemm(f, f, -1, 256, f, f, f, 128, 128, f, None) == EINVAL
    # bad path
    assert lib.w4a8_gemm_path(f, f, 4, 256, f, f, f, 128, 128, 7, f, None) == EINVAL
    assert lib.w4a8_gemm_path(f, f, 4, 256, f, f, f, 128, 128, -1, f, None) == EINVAL
    # streaming path with too many rows
    assert lib.w4a8_gemm_path(f, f, 65, 256, f, f, f, 128, 128, 1, f, None) == EINVAL
    # M == 0 is a no-op that launches nothing
    assert lib.w4a8_gemm(f, f, 0, 256, f, f, f, 128, 128, f, None) == 0
    # quantize_act
    assert lib.w4a8_quantize_act(None, 4, 256, 256, f, f, None) == EINVAL
    assert lib.w4a8_quantize_act(f, 4, 256, 100, f, f, None) == EINVAL
    assert lib.w4a8_quantize_act(f, 4, 250, 256, f, f, None) == EINVAL
    assert lib.w4a8_quantize_act(f, 0, 256, 256, f, f, None) == 0
    # router
    assert lib.w4a8_moe_route(f, 4, 8, 9, 0, f, f, f, f, f, f, None) == EINVAL
    assert lib.w4a8_moe_route(f, 4, 2000, 8, 0, f, f, f, f, f, f, None) == EINVAL
    assert lib.w4a8_moe_route(f, 4, 8, 0, 0, f, f, f, f, f, f, None) == EINVAL
    assert lib.w4a8_moe_route(f, 4, 8, 2, 2, f, f, f, f, f, f, None) == EINVAL
    # grouped gemm
    assert lib.w4a8_moe_grouped_gemm(f, f, 4, None, None, 8, 256, f, f, f, 128, 128, 16, f, None) == EINVAL
    assert lib.w4a8_moe_grouped_gemm(f, f, 4, None, f, 0, 256, f, f, f, 128, 128, 16, f, None) == EINVAL
    assert lib.w4a8_moe_grouped_gemm(f, f, 4, None, f, 8, 256, f, f, f, 128, 32, 16, f, None) == EUNSUPPORTED
    assert lib.w4a8_moe_grouped_gemm(f, f, 4, None, f, 8, 384, f, f, f, 128, 256, 16, f, None) == EINVAL
    # silu + requant, combine
    assert lib.w4a8_silu_mul_quantize(f, 4, 100, f, f, None, None) == EINVAL
    assert lib.w4a8_moe_combine(f, f, f, None, 4, 1, 102, f, None) == EINVAL
    assert lib.w4a8_moe_combine(f, f, f, None, 4, 0, 128, f, None) == EINVAL
    # device packer sizes
    assert lib.w4a8_pack_weights_device(f, 128, 200, 128, f, f, f, None) == EINVAL
    # tile-major weights: size query, conversion and GEMM
    assert lib.w4a8_tm_bytes(28672, 8192) == 28672 * 8192 // 2 + 4 * 28672 * 64
    assert lib.w4a8_tm_bytes(24, 256) == 0 and lib.w4a8_tm_bytes(16, 384) == 0
    assert lib.w4a8_weights_to_tm(f, f, f, 128, 384, 128, f, None) == EINVAL
    assert lib.w4a8_weights_to_tm(f, f, f, 120, 256, 128, f, None) == EINVAL
    assert lib.w4a8_weights_to_tm(f, f, f, 128, 256, 64, f, None) == EUNSUPPORTED
    assert lib.w4a8_weights_to_tm(f, f, f, 128, 256, 128, _fake(4104), None) == EINVAL
    assert lib.w4a8_gemm_tm(f, f, 1 << 20, 4096, f, 128, 128, f, None) == EINVAL  # M*K = 2^32 (tiled loop)
    assert lib.w4a8_gemm_tm(f, f, 64, 8192, f, 1 << 20, 128, f, None) == EINVAL  # tile-major array >= 4 GiB
    assert b"4 GiB" in lib.w4a8_last_error()
    assert lib.w4a8_gemm_tm(f, f, 4, 384, f, 128, 128, f, None) == EINVAL
    assert lib.w4a8_gemm_tm(f, f, 16, 9216, f, 128, 128, f, None) == EINVAL  # staged rows past the LDS
    assert lib.w4a8_gemm_tm(f, f, 4, 256, f, 120, 128, f, None) == EINVAL
    assert lib.w4a8_gemm_tm(f, f, 4, 256, f, 128, 256, f, None) == EUNSUPPORTED
    assert lib.w4a8_gemm_tm(None, f, 4, 256, f, 128, 128, f, None) == EINVAL
    assert lib.w4a8_gemm_tm(f, f, 0, 256, f, 128, 128, f, None) == 0
    # smoothing entry points
    assert lib.w4a8_channel_absmax(f, 4, 256, 200, f, None) == EINVAL
    assert lib.w4a8_channel_absmax(None, 4, 256, 256, f, None) == EINVAL
    assert lib.w4a8_quantize_act_smooth(f, 4, 256, 256, None, f, f, None) == EINVAL
    assert lib.w4a8_quantize_act_smooth(f, 4, 200, 256, f, f, f, None) == EINVAL
    assert lib.w4a8_quantize_act_smooth(f, 0, 256, 256, f, f, f, None) == 0
    assert lib.w4a8_pack_weights_device_smooth(f, 16, 256, 128, _fake(4100), f, f, f, None) == EINVAL
    assert lib.w4a8_pack_weights_device_smooth(f, 16, 256, 32, f, f, f, f, None) == EUNSUPPORTED
    assert lib.w4a8_pack_weights_device_smooth(f, 16, 256, 256, _fake(4104), f, f, f, None) == EINVAL
    # MoE FFN layer: sizes, workspace alignment and size
    need = lib.w4a8_moe_ffn_workspace_size(64, 7168, 2048, 384, 8)
    assert need > 0
    assert lib.w4a8_moe_ffn_workspace_size(64, 7100, 2048, 384, 8) == 0
    args = (f, f, 64, 7168, 2048, 384, 8, f, f, f, f, f, f, f)
    assert lib.w4a8_moe_ffn(*args, f, need - 1, None) == EWORKSPACE
    assert lib.w4a8_moe_ffn(*args, _fake(4096 + 64), need, None) == EINVAL
    assert lib.w4a8_moe_ffn(f, f, 64, 7168, 2048, 384, 9, f, f, f, f, f, f, f, f, need, None) == EINVAL
    assert lib.w4a8_moe_ffn(f, f, 64, 7168, 2048, 1024, 8, f, f, f, f, f, f, f, f, need, None) == EINVAL


def test_grouped_isums_entry_rejects_before_launch():
    lib = w4.load()
    f = _fake()
    # (qa, R, row_index, offsets, E, K, packed, zp, N, group, max_slots, isums, stream)
    assert lib.w4a8_moe_grouped_gemm_debug_isums(f, 8, f, f, 4, 256, f, f, 128, 32, 8, f, None) == EUNSUPPORTED
    assert lib.w4a8_moe_grouped_gemm_debug_isums(f, 8, f, f, 4, 384, f, f, 128, 256, 8, f, None) == EINVAL
    assert lib.w4a8_moe_grouped_gemm_debug_isums(f, 8, f, None, 4, 256, f, f, 128, 128, 8, f, None) == EINVAL
    assert lib.w4a8_moe_grouped_gemm_debug_isums(f, 8, f, f, 0, 256, f, f, 128, 128, 8, f, None) == EINVAL
    assert lib.w4a8_moe_grouped_gemm_debug_isums(f, 8, f, f, 4, 256, f, f, 120, 128, 8, f, None) == EINVAL
    assert lib.w4a8_moe_grouped_gemm_debug_isums(f, 8, f, f, 4, 256, f, f, 128, 128, 0, f, None) == 0


def test_moe_ffn_noalloc_rejects_layers_above_its_scratch():
    """The entry point that allocates nothing refuses, on the host, a layer whose intermediates
    exceed its fixed scratch (64 MiB: at H=7168, I=2048, E=384, top-8, T above 155)."""
    lib = w4.load()
    f = _fake()
    assert lib.w4a8_moe_ffn_noalloc_max_bytes() == 64 << 20
    assert lib.w4a8_moe_ffn_workspace_size(155, 7168, 2048, 384, 8) <= 64 << 20
    assert lib.w4a8_moe_ffn_workspace_size(156, 7168, 2048, 384, 8) > 64 << 20
    assert lib.w4a8_moe_ffn_noalloc(f, f, 156, 7168, 2048, 384, 8, f, f, f, f, f, f, f, None) == EWORKSPACE
    assert b"scratch" in lib.w4a8_last_error()
    assert lib.w4a8_moe_ffn_noalloc(f, f, 64, 7100, 2048, 384, 8, f, f, f, f, f, f, f, None) == EINVAL


def test_moe_ffn_workspace_layout():
    """Parts in enum order, 256-byte aligned, each at least its tensor's size, total = size query."""
    T, H, I, E, k = 64, 7168, 2048, 384, 8
    total, parts = w4.moe_ffn_workspace(T, H, I, E, k)
    assert total == w4.load().w4a8_moe_ffn_workspace_size(T, H, I, E, k)
    P, S = T * k, T * k + T
    need = {"ids": 4 * P, "w": 4 * P, "offsets": 4 * (E + 2), "perm": 4 * P, "row_index": 4 * S,
            "slot_of_pair": 4 * P, "qa": T * H, "a_scale": 4 * T, "gu": 4 * S * 2 * I, "qh": S * I,
            "h_scale": 4 * S, "y": 4 * S * H}
    last_end = 0
    for name in w4.WS_PARTS:
        off, size = parts[name]
        assert off % 256 == 0 and off >= last_end and size >= need[name], name
        last_end = off + need[name]
    assert last_end <= total


def test_host_packer_rejects_bad_weights():
    W = np.zeros((2, 256), np.float32)
    W[1, 7] = np.nan
    with pytest.raises(w4.W4A8Error) as e:
        w4.pack_weights(W)
    assert e.value.status == EINVAL
    W[1, 7] = 1e7  # range / 15 exceeds the largest fp16
    with pytest.raises(w4.W4A8Error):
        w4.pack_weights(W)
    with pytest.raises(w4.W4A8Error) as e:
        w4.pack_weights(np.zeros((2, 256), np.float32), group=32)
    assert e.value.status == EUNSUPPORTED
    with pytest.raises(w4.W4A8Error) as e:
        w4.pack_weights(np.zeros((2, 384), np.float32), group=256)
    assert e.value.status == EINVAL


def _packer_matches_oracle(orc, W):
    q, s, z = orc.quantize_weights(W)
    p_ref = orc.pack_nibbles(q)
    packed, scale, zp = w4.pack_weights(W)
    assert np.array_equal(packed, p_ref)
    assert np.array_equal(scale, s)
    assert np.array_equal(zp, z)
    q2, w_hat = w4.unpack_weights(packed, scale, zp)
    assert np.array_equal(q2, q)
    assert np.allclose(w_hat, orc.dequantize_weights(q, s, z), rtol=0, atol=1e-7)


@pytest.mark.parametrize("case", ["c1", "c2_rows", "c3_rows", "c4_rows", "c5_rows", "edge"])
def test_host_packer_bit_exact_vs_oracle(orc, case):
    if case == "c1":
        W = synthetic.weights(0, synthetic.TAG_W, 0, 128, 256)
    elif case == "c2_rows":
        W = synthetic.weights_with_outliers(0, 28672, 8192, rows=np.arange(0, 28672, 449))
    elif case == "c3_rows":
        W = synthetic.weights_with_offset(0, 8192, 8192, rows=np.arange(0, 8192, 127))
    elif case == "c4_rows":
        W = synthetic.weights(0, synthetic.TAG_W, 3, 14336, 4096, rows=np.arange(0, 14336, 211))
    elif case == "c5_rows":
        W = synthetic.weights(0, synthetic.TAG_W_DOWN, 17, 7168, 2048, rows=np.arange(0, 7168, 97))
    else:
        rng = np.random.default_rng(9)
        W = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
        W[0] = 0.0                       # all-zero groups -> scale 1, zp 0
        W[1] = np.abs(W[1]) + 0.01       # one-signed groups
        W[2] = -np.abs(W[2]) - 0.01
        W[3] = (np.arange(512) % 16).astype(np.float32)   # integer lattice, exact ties at x.5 absent
        W[4, :128] = 1e-9                # scale underflows to an fp16 subnormal
        W[5, :128] = 3e-8                # fp16 subnormal scale
        W[6] = np.linspace(-1, 1, 512)
        W[7, ::2] = 0.5                  # ties in w / s
        W[8] = W[8] * 1000               # large range
    _packer_matches_oracle(orc, W)


def test_smooth_factors_bit_exact_vs_oracle_and_rejects(orc):
    """The host factor routine gives the oracle's fp32 factors bit for bit (both take
    the power in double, round once to fp32, and invert the stored fp32 factor)."""
    K = 8192
    x = synthetic.activations_with_outlier_channels(0, 64, K)
    W = synthetic.weights(7, synthetic.TAG_W, 0, 96, K)
    ax, aw = orc.channel_absmax(x[16:]), orc.channel_absmax(W)
    ax[:5] = 0.0
    aw[5:9] = 0.0
    for alpha in (0.0, 0.25, 0.5, 0.8, 1.0):
        s, inv = w4.smooth_factors(ax, aw, alpha)
        so, invo = orc.smooth_factors(ax, aw, alpha)
        assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), alpha
        assert np.array_equal(inv.view(np.uint32), invo.view(np.uint32)), alpha
    for bad_alpha in (-0.1, 1.5, float("nan")):
        with pytest.raises(w4.W4A8Error):
            w4.smooth_factors(ax, aw, bad_alpha)
    neg = ax.copy()
    neg[3] = -1.0
    with pytest.raises(w4.W4A8Error):
        w4.smooth_factors(neg, aw, 0.5)
    with pytest.raises(w4.W4A8Error):      # 1 / 1e-45 overflows fp32
        w4.smooth_factors(np.ones(4, np.float32), np.full(4, 1e-45, np.float32), 0.0)


@pytest.mark.parametrize("symmetric,clip", [(True, 100.0), (False, 99.9), (True, 99.9), (False, 90.0), (True, 50.0)])
@pytest.mark.parametrize("case", ["c2_rows", "c3_rows", "edge"])
def test_host_packer_variants_bit_exact_vs_oracle(orc, case, symmetric, clip):
    """Symmetric codes (q + 8, zp 8) and percentile clipping: the host packer's bytes equal
    the oracle's, on outlier rows, offset rows and hand-made edge rows (zero groups, ties,
    a constant row, a single spike)."""
    if case == "c2_rows":
        W = synthetic.weights_with_outliers(0, 28672, 8192, rows=np.arange(0, 28672, 997))
    elif case == "c3_rows":
        W = synthetic.weights_with_offset(0, 8192, 8192, rows=np.arange(0, 8192, 701))
    else:
        W = np.zeros((5, 512), np.float32)
        W[1] = 0.25
        W[2, :128] = np.arange(128) * 0.5 - 32.0
        W[3, 300] = 9.0
        W[4] = np.random.default_rng(5).standard_normal(512).astype(np.float32)
    src = orc.clip_rows(W, clip) if clip < 100.0 else W
    q, s, z = (orc.quantize_weights_sym if symmetric else orc.quantize_weights)(src)
    packed, scale, zp = w4.pack_weights(W, symmetric=symmetric, clip_percent=clip)
    assert np.array_equal(packed, orc.pack_nibbles(q))
    assert np.array_equal(scale, s) and np.array_equal(zp, z)
    if symmetric:
        assert np.all(zp == np.float16(8.0).view(np.uint16))


def test_host_packer_variant_rejects():
    W = np.zeros((2, 256), np.float32)
    for kw in ({"clip_percent": 49.0}, {"clip_percent": 100.5}, {"clip_percent": float("nan")}):
        with pytest.raises(w4.W4A8Error):
            w4.pack_weights(W, **kw)
    lib = w4.load()
    f = _fake()
    assert lib.w4a8_pack_weights_ex(f, 2, 256, 128, 2, 100.0, f, f, f) == EINVAL
    W[1, 3] = np.inf
    with pytest.raises(w4.W4A8Error):
        w4.pack_weights(W, symmetric=True, clip_percent=99.0)


@pytest.mark.parametrize("group", [64, 256])
@pytest.mark.parametrize("symmetric", [False, True])
def test_host_packer_group_sizes_bit_exact_vs_oracle(orc, group, symmetric):
    """Group sizes 64 and 256 ([p2 §4.3] weighs 64/128/256): bytes, scales and zero points
    equal the oracle's for the same group size; the unpacker inverts them."""
    W = synthetic.weights_with_offset(0, 8192, 1536, rows=np.arange(0, 8192, 331))
    W[3, :group] = 0.0
    q, s, z = (orc.quantize_weights_sym if symmetric else orc.quantize_weights)(W, group)
    packed, scale, zp = w4.pack_weights(W, group=group, symmetric=symmetric)
    assert scale.shape == (1536 // group, W.shape[0])
    assert np.array_equal(packed, orc.pack_nibbles(q))
    assert np.array_equal(scale, s) and np.array_equal(zp, z)
    q2, w_hat = w4.unpack_weights(packed, scale, zp, group=group)
    assert np.array_equal(q2, q)
    assert np.allclose(w_hat, orc.dequantize_weights(q, s, z, group), rtol=0, atol=1e-7)
