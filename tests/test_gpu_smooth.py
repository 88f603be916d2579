"""GPU parity of the offline transforms around the layer.

Per-channel smoothing ([p3 §3.4]): channel maxima, the smoothed weight packer and the
smoothed per-token quantizer are integer/byte work (bit-exact against the oracle), and the
layer over their outputs is the unchanged GEMM (oracle tolerance
1e-5 * sum_g |a_scale * w_scale * isum_g| + 1e-6).  The host packer variants (symmetric
codes, percentile clipping) are checked byte for byte on the CPU; here every GEMM loop runs
over their output against the oracle's product of the same codes.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import check_close, cuda, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_quantized_gemm_token_amd as w4
    w4.load()
    yield
    torch.cuda.synchronize()


def w4mod():
    import w4a8_quantized_gemm_token_amd as w4
    return w4


@pytest.mark.parametrize("rows,K,pad", [(0, 64, 0), (1, 100, 0), (48, 8192, 0), (37, 1000, 24), (2000, 320, 0)])
def test_channel_absmax_bit_exact(orc, rows, K, pad):
    w4 = w4mod()
    rng = np.random.default_rng(rows + K)
    A = (rng.standard_normal((rows, K + pad)) * np.exp(rng.uniform(-4, 4, K + pad))).astype(np.float32)
    A[:, ::7] *= -1
    dev = to_dev(A)[:, :K]
    got = to_host(w4.channel_absmax(dev))
    want = orc.channel_absmax(A[:, :K]) if rows else np.zeros(K, np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# K: single-pass row kernel (<= 8192 and <= 16384 floats), the two-pass kernel for longer
# rows, and a row stride that is not a multiple of 4 floats (scalar loads)
@pytest.mark.parametrize("M,K,ldx", [(1, 256, 256), (16, 8192, 8192), (5, 16384, 16384), (3, 20480, 20480),
                                     (7, 1024, 1030), (64, 7168, 7168)])
def test_quantize_act_smooth_bit_exact(orc, M, K, ldx):
    w4 = w4mod()
    x = synthetic.activations_with_outlier_channels(M + K, M, ldx)
    x[0, : K // 3] = 0.0
    if M > 2:
        x[2] = 0.0
    W = synthetic.weights(K, synthetic.TAG_W, 0, 64, K)
    _, inv = orc.smooth_factors(orc.channel_absmax(x[:, :K]), orc.channel_absmax(W), 0.5)
    qr, sr = orc.quantize_act_smooth(x[:, :K], inv)
    qa, sc = w4.quantize_act_smooth(to_dev(x)[:, :K], to_dev(inv))
    assert np.array_equal(to_host(qa), qr)
    assert np.array_equal(to_host(sc).view(np.uint32), sr.view(np.uint32))


@pytest.mark.parametrize("N,K", [(16, 128), (96, 1024), (336, 2048)])
def test_pack_weights_smooth_bit_exact(orc, N, K):
    w4 = w4mod()
    W = synthetic.weights(N, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(N, N)[:, None] * 2
    x = synthetic.activations_with_outlier_channels(N, 32, K)
    s, _ = orc.smooth_factors(orc.channel_absmax(x), orc.channel_absmax(W), 0.5)
    q, sw, zw = orc.quantize_weights(orc.smooth_weights(W, s))
    packed, scale, zp = w4.pack_weights_device_smooth(to_dev(W), to_dev(s))
    assert np.array_equal(to_host(packed), orc.pack_nibbles(q))
    assert np.array_equal(to_host(scale).view(np.uint16), sw)
    assert np.array_equal(to_host(zp).view(np.uint16), zw)


def test_smoothed_decode_layer_full_size(orc):
    """Decode layer K=8192, N=28672 (0.1% x20 weight outliers, 4 x50 activation channels):
    channel maxima of all weights, factors from 48 calibration tokens, smoothed pack on the
    device (sampled columns bit-exact), smoothed quantizer for 16 evaluation tokens
    (bit-exact), the tile-major decode GEMM over both (sampled outputs within tolerance), and
    a lower error against the unquantized product than the plain path on those samples."""
    w4 = w4mod()
    N, K, M = 28672, 8192, 16
    Wd = torch.empty((N, K), dtype=torch.float32, device=cuda())
    synthetic.fill_weights_device(Wd, 0, synthetic.TAG_W, 0, K, 0, "outliers")
    x = synthetic.activations_with_outlier_channels(0, 64, K)
    xe, xcal = x[:M], x[M:]
    aw = to_host(w4.channel_absmax(Wd))
    rng = np.random.default_rng(12)
    cols = np.unique(np.concatenate([[0, 15, 16, N - 1], rng.choice(N, 60, replace=False)]))
    Wcols = synthetic.weight_rows_host(0, synthetic.TAG_W, 0, K, cols, "outliers")
    assert np.array_equal(to_host(Wd[torch.as_tensor(cols, device=cuda())]), Wcols)
    # the full-matrix maximum by numpy's own reduction, over host slices of W
    want_aw = np.zeros(K, np.float32)
    for r0 in range(0, N, 4096):
        want_aw = np.maximum(want_aw, np.abs(to_host(Wd[r0:r0 + 4096])).max(0))
    assert np.array_equal(aw.view(np.uint32), want_aw.view(np.uint32))
    ax = to_host(w4.channel_absmax(to_dev(xcal)))
    s, inv = w4.smooth_factors(ax, aw, 0.5)
    so, invo = orc.smooth_factors(orc.channel_absmax(xcal), want_aw, 0.5)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
    packed, scale, zp = w4.pack_weights_device_smooth(Wd, to_dev(s))
    plain = w4.pack_weights_device(Wd)
    del Wd
    q, sw, zw = orc.quantize_weights(orc.smooth_weights(Wcols, so))
    ct = torch.as_tensor(cols, device=cuda())
    assert np.array_equal(to_host(packed[ct]), orc.pack_nibbles(q))
    assert np.array_equal(to_host(scale[:, ct]).view(np.uint16), sw)
    assert np.array_equal(to_host(zp[:, ct]).view(np.uint16), zw)
    qr, sr = orc.quantize_act_smooth(xe, invo)
    qa, sc = w4.quantize_act_smooth(to_dev(xe), to_dev(inv))
    assert np.array_equal(to_host(qa), qr) and np.array_equal(to_host(sc), sr)
    out = to_host(w4.gemm_tm(qa, sc, w4.weights_to_tm(packed, scale, zp)))
    ms, ns = np.meshgrid(np.arange(M), np.arange(len(cols)), indexing="ij")
    ref, mag = orc.gemm_at(qr, sr, q, sw, zw, ms.ravel(), ns.ravel())
    check_close(out[:, cols].ravel(), ref, mag, "smoothed decode layer")
    exact = xe.astype(np.float64) @ Wcols.astype(np.float64).T
    qa0, sc0 = w4.quantize_act(to_dev(xe))
    out0 = to_host(w4.gemm(qa0, sc0, *plain))
    err_s = np.linalg.norm(out[:, cols] - exact) / np.linalg.norm(exact)
    err_p = np.linalg.norm(out0[:, cols] - exact) / np.linalg.norm(exact)
    assert err_s < err_p, (err_s, err_p)


@pytest.mark.parametrize("symmetric,clip", [(True, 100.0), (False, 99.9), (True, 99.9)])
@pytest.mark.parametrize("M", [1, 16, 40, 300])
def test_gemm_over_packer_variants(orc, symmetric, clip, M):
    """Decode (M <= 16, standard and tile-major), streaming (M <= 64) and tiled loops over
    symmetric and clipped packs of outlier weights."""
    w4 = w4mod()
    N, K = 272, 2048
    W = synthetic.weights_with_outliers(0, 28672, K, rows=np.arange(N) * 97)
    x = synthetic.activations_with_outlier_channels(M, M, K)
    src = orc.clip_rows(W, clip) if clip < 100.0 else W
    q, sw, zw = (orc.quantize_weights_sym if symmetric else orc.quantize_weights)(src)
    qr, sr = orc.quantize_act(x)
    ref, mag = orc.gemm(qr, sr, q, sw, zw)
    packed, scale, zp = w4.pack_weights(W, symmetric=symmetric, clip_percent=clip)
    dp, ds, dz = to_dev(packed), to_dev(scale.view(np.int16)), to_dev(zp.view(np.int16))
    qa, sc = w4.quantize_act(to_dev(x))
    check_close(to_host(w4.gemm(qa, sc, dp, ds, dz)), ref, mag, f"variant sym={symmetric} clip={clip} M={M}")
    if M <= 16:
        out = to_host(w4.gemm_tm(qa, sc, w4.weights_to_tm(dp, ds, dz)))
        check_close(out, ref, mag, f"tile-major variant sym={symmetric} clip={clip} M={M}")
