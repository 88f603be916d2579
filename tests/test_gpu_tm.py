"""GPU parity of the tile-major weight path (w4a8_weights_to_tm, w4a8_gemm_tm).

The conversion must reproduce, byte for byte, the block order include/w4a8.h
defines, built here in plain numpy from the oracle's own codes, scales and zero
points.  The GEMM over tile-major weights must match the oracle within the fp32
bound (1e-5 * sum_g |a_scale * w_scale * isum_g| + 1e-6) and, since it runs the
same arithmetic in the same order as the decode loop over the standard layout,
give exactly the bytes w4a8_gemm gives.  Above 16 rows it runs the 256x256 tiled loop and must
give exactly the bytes of that loop over the standard layout (w4a8_gemm_path, path 5).
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import check_close, cuda, device_layer, oracle_columns, to_dev, to_host

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


def tm_expected(q: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Tile-major bytes written out from the definition, one block at a time, from the
    4-bit codes q[N][K] and the fp16 bits of the scales and zero points [G][N]."""
    N, K = q.shape
    G = K // 128
    out = np.zeros((N // 16, G // 2, 2176), np.uint8)
    for t in range(N // 16):
        for w in range(G // 2):
            blk = out[t, w]
            for h in range(2):
                g = 2 * w + h
                for lane in range(64):
                    col, quarter = 16 * t + (lane & 15), lane >> 4
                    codes = q[col, 128 * g + 32 * quarter:128 * g + 32 * quarter + 32].reshape(4, 8)
                    chunk = codes[:, :4] | (codes[:, 4:] << 4)
                    blk[1024 * h + 16 * lane:1024 * h + 16 * lane + 16] = chunk.reshape(16)
            zint = z.view(np.float16).astype(np.int64)      # zero points are integers 0..15
            for c in range(16):
                col = 16 * t + c
                area = blk[2048 + 8 * c:2048 + 8 * c + 8]
                area[0:4] = s[2 * w:2 * w + 2, col].astype(np.uint16).view(np.uint8)
                area[4] = (-zint[2 * w, col]) & 0xFF
                area[5] = (-zint[2 * w + 1, col]) & 0xFF
                area[6:8] = 0
    return out


@pytest.mark.parametrize("N,K", [(16, 256), (48, 512), (80, 1280)])
def test_weights_to_tm_bytes(orc, N, K):
    w4 = w4mod()
    W = synthetic.weights(N + K, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(N + K, N)[:, None] * 3
    q, s, z = orc.quantize_weights(W)
    packed = orc.pack_nibbles(q)
    tm = w4.weights_to_tm(to_dev(packed), to_dev(s.view(np.int16)), to_dev(z.view(np.int16)))
    assert tm.numel() == w4.tm_bytes(N, K) == N * K // 2 + 4 * N * (K // 128)
    assert np.array_equal(to_host(tm), tm_expected(q.astype(np.uint8), s, z))


# (M, N, K): ring depth 4 with two and four K parts per tile, depth 2 and 1, one K
# part (odd window count), rows staged in a loop, several tiles per workgroup with a
# ragged last workgroup, tiles per workgroup rounded up to whole rounds of the waves
TM_SHAPES = [
    (1, 16, 256),
    (4, 128, 256),
    (3, 48, 768),
    (16, 272, 1024),
    (8, 336, 2048),
    (5, 96, 4096),
    (16, 64, 8704),
    (2, 4112, 3072),
    (3, 20496, 8192),
    (2, 28640, 512),    # 1790 tiles: 8 tiles per workgroup (rounded up from 7), last workgroup 6
]


@pytest.mark.parametrize("M,N,K", TM_SHAPES)
def test_gemm_tm_matches_oracle_and_standard_layout(orc, M, N, K):
    w4 = w4mod()
    seed = 3 * M + N
    W = synthetic.weights(seed, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(seed, N)[:, None] * 3
    x = synthetic.activations(seed, M, K)
    q, s, z = orc.quantize_weights(W)
    qr, sr = orc.quantize_act(x)
    ref, mag = orc.gemm(qr, sr, q, s, z)
    packed, scale, zp = to_dev(orc.pack_nibbles(q)), to_dev(s.view(np.int16)), to_dev(z.view(np.int16))
    tm = w4.weights_to_tm(packed, scale, zp)
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm_tm(qa, sc, tm))
    check_close(out, ref, mag, f"tile-major M={M} N={N} K={K}")
    std = to_host(w4.gemm(qa, sc, packed, scale, zp))
    assert np.array_equal(out.view(np.uint32), std.view(np.uint32))


# (M, N, K) above 16 rows: the 256x256 tiled loop over tile-major weights; ragged row and column
# tiles (17, 257, 513 rows; 272, 528, 1040 columns), one window of two groups (K=256), an odd
# number of windows (K=768)
TM_TILED_SHAPES = [
    (17, 272, 1024),
    (64, 528, 768),
    (257, 256, 256),
    (260, 1040, 2048),
    (513, 528, 512),
]


@pytest.mark.parametrize("M,N,K", TM_TILED_SHAPES)
def test_gemm_tm_tiled_matches_oracle_and_path5(orc, M, N, K):
    w4 = w4mod()
    seed = 5 * M + N
    W = synthetic.weights(seed, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(seed, N)[:, None] * 3
    x = synthetic.activations(seed, M, K)
    q, s, z = orc.quantize_weights(W)
    qr, sr = orc.quantize_act(x)
    ref, mag = orc.gemm(qr, sr, q, s, z)
    packed, scale, zp = to_dev(orc.pack_nibbles(q)), to_dev(s.view(np.int16)), to_dev(z.view(np.int16))
    tm = w4.weights_to_tm(packed, scale, zp)
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm_tm(qa, sc, tm))
    check_close(out, ref, mag, f"tile-major tiled M={M} N={N} K={K}")
    std = to_host(w4.gemm(qa, sc, packed, scale, zp, path=5))
    assert np.array_equal(out.view(np.uint32), std.view(np.uint32))


@pytest.mark.parametrize("seed", [0, 1])
def test_gemm_tm_prefill_full_size_sampled(orc, seed):
    """Prefill layer M=4096, K=N=8192 (per-column mean offsets; seed 0 is the one the benchmark
    times) on tile-major weights, in the launch configuration the benchmark times: sampled outputs
    against the oracle, every output byte against the 256x256 loop over the standard layout."""
    w4 = w4mod()
    M, N, K = 4096, 8192, 8192
    packed, scale, zp = device_layer(seed, synthetic.TAG_W, 0, N, K, mode="offset")
    tm = w4.weights_to_tm(packed, scale, zp)
    rng = np.random.default_rng(17 + seed)
    cols = np.unique(np.concatenate([[0, 15, 16, 255, 256, N - 1], rng.choice(N, 40, replace=False)]))
    q, s, z = oracle_columns(orc, seed, synthetic.TAG_W, 0, K, cols, mode="offset")
    x = synthetic.activations(seed, M, K)
    qr, sr = orc.quantize_act(x)
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm_tm(qa, sc, tm))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 150, replace=False)]))
    ms, ns = np.meshgrid(rows, np.arange(len(cols)), indexing="ij")
    ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel())
    check_close(out[rows][:, cols].ravel(), ref, mag, "tile-major prefill")
    del tm
    std = to_host(w4.gemm(qa, sc, packed, scale, zp, path=5))
    assert np.array_equal(out.view(np.uint32), std.view(np.uint32))


def test_gemm_tm_zero_row_and_rejects():
    w4 = w4mod()
    M, N, K = 6, 64, 512
    W = synthetic.weights(4, synthetic.TAG_W, 0, N, K)
    x = synthetic.activations(4, M, K)
    x[2] = 0.0
    packed, scale, zp = (to_dev(a) for a in w4.pack_weights(W))
    tm = w4.weights_to_tm(packed, scale, zp)
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm_tm(qa, sc, tm))
    assert not out[2].any() and out[0].any()
    x[3] = 0.0  # the same in the tiled loop (M > 16)
    xt = np.concatenate([x, synthetic.activations(5, 14, K)])
    xt[17] = 0.0
    qa, sc = w4.quantize_act(to_dev(xt))
    out = to_host(w4.gemm_tm(qa, sc, tm))
    assert not out[17].any() and out[18].any()
    odd = torch.zeros((20, 384), dtype=torch.int8, device=cuda())  # K % 256 != 0
    with pytest.raises(w4.W4A8Error) as e:
        w4.gemm_tm(odd, torch.zeros(20, device=cuda()), tm)
    assert e.value.status == 1


def test_gemm_tm_full_size_sampled(orc):
    """Decode layer K=8192, N=28672 (0.1% x20 weight outliers, 4 x50 activation channels),
    M = 1, 8, 16, in the launch configuration the benchmark times."""
    w4 = w4mod()
    N, K = 28672, 8192
    packed, scale, zp = device_layer(0, synthetic.TAG_W, 0, N, K, mode="outliers")
    tm = w4.weights_to_tm(packed, scale, zp)
    rng = np.random.default_rng(11)
    cols = np.unique(np.concatenate([[0, 15, 16, N - 17, N - 1], rng.choice(N, 96, replace=False)]))
    q, s, z = oracle_columns(orc, 0, synthetic.TAG_W, 0, K, cols, mode="outliers")
    x = synthetic.activations_with_outlier_channels(0, 16, K)
    for M in (1, 8, 16):
        xm = x[:M]
        qr, sr = orc.quantize_act(xm)
        qa, sc = w4.quantize_act(to_dev(xm))
        out = to_host(w4.gemm_tm(qa, sc, tm))
        ms, ns = np.meshgrid(np.arange(M), np.arange(len(cols)), indexing="ij")
        ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel())
        check_close(out[:, cols].ravel(), ref, mag, f"tile-major decode M={M}")
        std = to_host(w4.gemm(qa, sc, packed, scale, zp))
        assert np.array_equal(out.view(np.uint32), std.view(np.uint32)), f"M={M}"
