"""GPU parity of group sizes 64 and 256 ([p2 §4.3] weighs 64, 128 and 256): the device
packer bit-exact; on the tiled loop (both workgroup tiles, odd and even 128-k stage
counts, ragged row and column tiles, the prefill shape sampled), the decode loop (every
K split and window ring depth it picks, the decode shape sampled) and the expert-grouped
loops (16-row chunks and tiles of 128 and 256 rows), per-group int32 sums bit-exact
against the oracle and outputs within the oracle tolerance
1e-5 * sum_g |a_scale * w_scale * isum_g| + 1e-6.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import check_close, device_layer, oracle_columns, to_dev, to_host

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


# (group, M, N, K): one stage pair, odd stage counts (64 only), ragged tiles, long K
SHAPES = [
    (64, 1, 64, 128),
    (64, 37, 144, 1152),
    (64, 200, 272, 2048),
    (64, 130, 80, 8192),
    (256, 1, 64, 256),
    (256, 37, 144, 1280),
    (256, 200, 272, 2048),
    (256, 300, 528, 8704),
]


@pytest.mark.parametrize("group,M,N,K", SHAPES)
@pytest.mark.parametrize("path", [3, 4])
def test_tiled_group_sizes(orc, group, M, N, K, path):
    w4 = w4mod()
    seed = group + M + N
    W = synthetic.weights(seed, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(seed, N)[:, None] * 3
    x = synthetic.activations(seed, M, K)
    x[M // 2] = 0.0
    q, s, z = orc.quantize_weights(W, group)
    qr, sr = orc.quantize_act(x)
    ref, mag = orc.gemm(qr, sr, q, s, z, group)
    packed, scale, zp = w4.pack_weights(W, group=group)
    assert np.array_equal(packed, orc.pack_nibbles(q))
    dp, ds, dz = to_dev(packed), to_dev(scale.view(np.int16)), to_dev(zp.view(np.int16))
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm(qa, sc, dp, ds, dz, path=path, group=group))
    check_close(out, ref, mag, f"group {group} path {path} M={M} N={N} K={K}")
    isums = to_host(w4.gemm_debug_isums(qa, dp, dz, path=path, group=group))
    assert np.array_equal(isums, orc.group_isums(qr, q, z, group))
    if path == 3:  # the default choice (path 0): the decode loop for M = 1 and K % 256 == 0
        out0 = to_host(w4.gemm(qa, sc, dp, ds, dz, group=group))
        check_close(out0, ref, mag, f"group {group} default path M={M}")


@pytest.mark.parametrize("group", [64, 256])
def test_tiled_group_sizes_prefill_sampled(orc, group):
    """Prefill shape M=4096, K=N=8192 (offset weights) in the launch configuration the
    benchmark times: sampled outputs against the oracle's one-by-one products."""
    w4 = w4mod()
    M, N, K = 4096, 8192, 8192
    rng = np.random.default_rng(group)
    cols = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.choice(N, 40, replace=False)]))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 40, replace=False)]))
    Wd = torch.empty((N, K), dtype=torch.float32, device="cuda:0")
    synthetic.fill_weights_device(Wd, 0, synthetic.TAG_W, 0, K, 0, "offset")
    packed, scale, zp = w4.pack_weights(to_host(Wd), group=group)
    Wc = to_host(Wd[torch.as_tensor(cols, device="cuda:0")])
    del Wd
    q, s, z = orc.quantize_weights(Wc, group)
    assert np.array_equal(packed[cols], orc.pack_nibbles(q))
    x = synthetic.activations(0, M, K)
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm(qa, sc, to_dev(packed), to_dev(scale.view(np.int16)), to_dev(zp.view(np.int16)),
                          group=group))
    qr, sr = orc.quantize_act(x[rows])
    assert np.array_equal(to_host(qa)[rows], qr)
    ms, ns = np.meshgrid(np.arange(len(rows)), np.arange(len(cols)), indexing="ij")
    ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel(), group)
    check_close(out[np.ix_(rows, cols)].ravel(), ref, mag, f"prefill group {group}")


def u16(t):
    return to_host(t).view(np.uint16)


def _edge_weights(K):
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((24, K)) * 0.02).astype(np.float32)
    W[0] = 0.0
    W[1] = np.abs(W[1]) + 0.01
    W[2] = -np.abs(W[2]) - 0.01
    W[3] = (np.arange(K) % 16).astype(np.float32)
    W[4, :64] = 1e-9                 # a tiny first 64-group (scale underflows in fp16)
    W[5, 64:128] = 0.0               # an all-zero second 64-group
    W[6] = np.linspace(-1, 1, K)
    W[7, ::2] = 0.5
    W[8] = W[8] * 1000
    W[9, 192:256] = 7.0              # one 64-group far off the rest of its 256-group
    return W


@pytest.mark.parametrize("group", [64, 256])
@pytest.mark.parametrize("case", ["edge", "plain", "outliers"])
def test_device_packer_group_sizes_bit_exact(orc, group, case):
    """The device packer at group 64 and 256: codes, scales and zero points equal the
    oracle's for the same group size."""
    w4 = w4mod()
    if case == "edge":
        W = _edge_weights(1024)
    elif case == "plain":
        W = synthetic.weights(group, synthetic.TAG_W, 0, 96, 1280)
    else:
        W = synthetic.fill_weights_host(0, synthetic.TAG_W, 0, 8192, 28000, 64, "outliers")
    packed, scale, zp = w4.pack_weights_device(to_dev(W), group=group)
    q, s, z = orc.quantize_weights(W, group)
    assert scale.shape == (W.shape[1] // group, W.shape[0])
    assert np.array_equal(to_host(packed), orc.pack_nibbles(q))
    assert np.array_equal(u16(scale), s)
    assert np.array_equal(u16(zp), z)


# (M, N, K): the decode loop's K parts (1, 2, 4), window ring depths (1, 2), one-load and
# batched row staging, rows staged in a loop, and more than four tiles per workgroup
DECODE_SHAPES = [
    (1, 64, 256),       # one window, K in one part
    (4, 128, 512),      # one window per K part, two parts
    (3, 48, 768),       # three windows, one part
    (16, 272, 1024),    # four K parts
    (5, 96, 1536),      # two parts of three windows
    (8, 336, 2048),     # four parts, two windows in flight
    (16, 64, 8704),     # rows staged in a loop; two parts of 17 windows
    (2, 16400, 1024),   # five tiles per workgroup: two K parts
]


@pytest.mark.parametrize("M,N,K", DECODE_SHAPES)
@pytest.mark.parametrize("group", [64, 256])
def test_decode_group_sizes(orc, group, M, N, K):
    w4 = w4mod()
    seed = group + M + K
    W = synthetic.weights(seed, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(seed, N)[:, None] * 3
    x = synthetic.activations(seed, M, K)
    if M > 2:
        x[M // 2] = 0.0
    q, s, z = orc.quantize_weights(W, group)
    qr, sr = orc.quantize_act(x)
    packed, scale, zp = w4.pack_weights(W, group=group)
    dp, ds, dz = to_dev(packed), to_dev(scale.view(np.int16)), to_dev(zp.view(np.int16))
    qa, sc = w4.quantize_act(to_dev(x))
    isums = to_host(w4.gemm_debug_isums(qa, dp, dz, path=1, group=group))
    assert np.array_equal(isums, orc.group_isums(qr, q, z, group))
    ref, mag = orc.gemm(qr, sr, q, s, z, group)
    for path in (1, 0):  # forced, and the default choice for M <= 16
        out = to_host(w4.gemm(qa, sc, dp, ds, dz, path=path, group=group))
        check_close(out, ref, mag, f"decode group {group} path {path} M={M} N={N} K={K}")


@pytest.mark.parametrize("group", [64, 256])
def test_decode_group_sizes_full_size_sampled(orc, group):
    """Decode layer K=8192, N=28672 (0.1% x20 weight outliers, 4 x50 activation channels) at
    group 64 and 256, M = 1 and 16, weights from the device packer -- the launch
    configuration the benchmark times; sampled columns against the oracle."""
    w4 = w4mod()
    N, K = 28672, 8192
    packed, scale, zp = device_layer(0, synthetic.TAG_W, 0, N, K, mode="outliers", group=group)
    rng = np.random.default_rng(group)
    cols = np.unique(np.concatenate([[0, 1, 15, 16, N - 1], rng.choice(N, 64, replace=False)]))
    q, s, z = oracle_columns(orc, 0, synthetic.TAG_W, 0, K, cols, mode="outliers", group=group)
    assert np.array_equal(to_host(packed[cols]), orc.pack_nibbles(q))
    assert np.array_equal(u16(scale)[:, cols], s) and np.array_equal(u16(zp)[:, cols], z)
    x = synthetic.activations_with_outlier_channels(0, 16, K)
    for M in (1, 16):
        xm = x[:M]
        qr, sr = orc.quantize_act(xm)
        qa, sc = w4.quantize_act(to_dev(xm))
        assert np.array_equal(to_host(qa), qr)
        out = to_host(w4.gemm(qa, sc, packed, scale, zp, group=group))
        ms, ns = np.meshgrid(np.arange(M), np.arange(len(cols)), indexing="ij")
        ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel(), group)
        check_close(out[:, cols].ravel(), ref, mag, f"decode group {group} M={M}")
        isums = to_host(w4.gemm_debug_isums(qa, packed, zp, group=group))
        assert np.array_equal(isums[:, :, cols], orc.group_isums(qr, q, z, group))


# (counts, N, K): 16-row chunks (up to 16 slots), 128-row tiles (17..128), 256-row tiles
# (above); K/128 = 6, not a multiple of 4, has no 16-row loop (every expert tiled)
GROUPED_GROUP_CASES = [
    ([16, 17, 3, 0, 64, 128, 129, 300], 544, 2048),
    ([1, 9, 40, 200], 160, 384 * 2),
    ([2, 5, 130], 160, 8704),
]


@pytest.mark.parametrize("counts,N,K", GROUPED_GROUP_CASES)
@pytest.mark.parametrize("group", [64, 256])
def test_grouped_gemm_group_sizes(orc, group, counts, N, K):
    """Expert-grouped GEMM at group 64 and 256: every slot's per-group int32 sums bit for bit
    (debug entry) and every output element within the oracle tolerance."""
    w4 = w4mod()
    if K % group:
        pytest.skip("K is not a multiple of the group size")
    E, S, R = len(counts), sum(counts), 301
    rng = np.random.default_rng(K + N + group)
    row_index = rng.integers(0, R, S).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synthetic.activations(K + group, R, K)
    qr, sr = orc.quantize_act(x)
    packed = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda:0")
    scale = torch.empty((E, K // group, N), dtype=torch.int16, device="cuda:0")
    zp = torch.empty((E, K // group, N), dtype=torch.int16, device="cuda:0")
    refs = []
    for e in range(E):
        W = synthetic.fill_weights_host(K + group, synthetic.TAG_W, e, K, 0, N, "offset" if e % 2 else "plain")
        q, s_, z = orc.quantize_weights(W, group)
        packed[e] = to_dev(orc.pack_nibbles(q))
        scale[e] = to_dev(s_.view(np.int16))
        zp[e] = to_dev(z.view(np.int16))
        refs.append((q, s_, z))
    qa, sc = w4.quantize_act(to_dev(x))
    assert np.array_equal(to_host(qa), qr)
    ri, off = to_dev(row_index), to_dev(offsets)
    isums = to_host(w4.moe_grouped_gemm_debug_isums(qa, ri, off, packed, zp, max_slots=S, group=group))
    out = to_host(w4.moe_grouped_gemm(qa, sc, ri, off, packed, scale, zp, max_slots=S, group=group))
    for e in range(E):
        s0, s1 = offsets[e], offsets[e + 1]
        if s0 == s1:
            continue
        q, s_, z = refs[e]
        rows = row_index[s0:s1]
        iref = orc.group_isums(qr[rows], q, z, group)
        bad = isums[:, s0:s1] != iref
        assert not bad.any(), f"group {group} expert {e} ({s1 - s0} slots): {int(bad.sum())} sums differ"
        ref, mag = orc.gemm(qr[rows], sr[rows], q, s_, z, group)
        check_close(out[s0:s1], ref, mag, f"group {group} expert {e} ({s1 - s0} slots)")
