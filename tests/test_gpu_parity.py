"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Integer stages (INT8 activation codes, packed weights, fp16 scale/zp bits, per-
group int32 sums, routing tables) must be bit-identical; fp32 outputs must lie
within 1e-5 * sum_g |a_scale * w_scale * isum_g| + 1e-6 of the oracle's double
result.  Small shapes are checked element by element; the full-size workloads
(decode K=8192 N=28672, prefill 4096x8192x8192, toy MoE, MoE FFN) are checked on
sampled output columns/rows that the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import check_close, cuda, device_experts, device_layer, oracle_columns, to_dev, to_host

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


def u16(t):
    return to_host(t).view(np.uint16)


# ------------------------------------------------------------------ generator
def test_device_filler_matches_numpy():
    for mode, sub, ref in [("plain", 5, lambda r: synthetic.weights(3, synthetic.TAG_W, 5, 300, 512, rows=r)),
                           ("outliers", 0, lambda r: synthetic.weights_with_outliers(3, 300, 512, rows=r)),
                           ("offset", 0, lambda r: synthetic.weights_with_offset(3, 300, 512, rows=r))]:
        W = torch.empty((40, 512), dtype=torch.float32, device=cuda())
        synthetic.fill_weights_device(W, 3, synthetic.TAG_W, sub, 512, 17, mode)
        assert np.array_equal(to_host(W).view(np.uint32), ref(np.arange(17, 57)).view(np.uint32)), mode


# ------------------------------------------------------------------ activation quantizer
def _act_cases():
    rng = np.random.default_rng(21)
    x_edge = rng.standard_normal((9, 512)).astype(np.float32)
    tiny = np.float32(2.0 ** -149)
    x_edge[1] = 0.0
    x_edge[2] = 0.0
    x_edge[2, :3] = np.array([-400, 150, 2], np.float32) * tiny
    x_edge[3] = 0.0
    x_edge[3, 5] = 60 * tiny
    x_edge[4, :6] = [127.0, 2.5, 3.5, -2.5, 0.5, -126.5]
    x_edge[4, 6:] = 0.25
    x_edge[5] *= 1e-30
    x_edge[6] *= 1e30
    return {
        "c1": synthetic.activations(0, 4, 256),
        "c2": synthetic.activations_with_outlier_channels(0, 16, 8192),
        "c3": synthetic.activations(0, 4096, 8192),
        "c5": synthetic.activations(0, 64, 7168),
        "edge": x_edge,
        "one_row": synthetic.activations(1, 1, 128),
    }


@pytest.mark.parametrize("case", ["c1", "c2", "c3", "c5", "edge", "one_row"])
def test_quantize_act_bit_exact(orc, case):
    w4 = w4mod()
    x = _act_cases()[case]
    qa, sc = w4.quantize_act(to_dev(x))
    qr, sr = orc.quantize_act(x)
    assert np.array_equal(to_host(sc).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(to_host(qa), qr)


@pytest.mark.parametrize("pad", [4, 1])
def test_quantize_act_strided_rows(orc, pad):
    """Row stride ldx > K: pad=4 keeps float4 alignment, pad=1 takes the scalar loader."""
    w4 = w4mod()
    M, K = 7, 384
    big = synthetic.activations(2, M, K + pad)
    xd = to_dev(big)[:, :K]
    qa, sc = w4.quantize_act(xd)
    qr, sr = orc.quantize_act(np.ascontiguousarray(big[:, :K]))
    assert np.array_equal(to_host(qa), qr) and np.array_equal(to_host(sc), sr)


# ------------------------------------------------------------------ device packer
def _pack_edge_weights():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
    W[0] = 0.0
    W[1] = np.abs(W[1]) + 0.01
    W[2] = -np.abs(W[2]) - 0.01
    W[3] = (np.arange(512) % 16).astype(np.float32)
    W[4, :128] = 1e-9
    W[5, :128] = 3e-8
    W[6] = np.linspace(-1, 1, 512)
    W[7, ::2] = 0.5
    W[8] = W[8] * 1000
    return W


@pytest.mark.parametrize("case", ["c1", "edge", "c3_slice", "c2_slice"])
def test_device_packer_bit_exact(orc, case):
    w4 = w4mod()
    if case == "c1":
        W = synthetic.weights(0, synthetic.TAG_W, 0, 128, 256)
    elif case == "edge":
        W = _pack_edge_weights()
    elif case == "c3_slice":
        W = synthetic.fill_weights_host(0, synthetic.TAG_W, 0, 8192, 4000, 96, "offset")
    else:
        W = synthetic.fill_weights_host(0, synthetic.TAG_W, 0, 8192, 28000, 64, "outliers")
    packed, scale, zp = w4.pack_weights_device(to_dev(W))
    q, s, z = orc.quantize_weights(W)
    assert np.array_equal(to_host(packed), orc.pack_nibbles(q))
    assert np.array_equal(u16(scale), s)
    assert np.array_equal(u16(zp), z)


# ------------------------------------------------------------------ dense GEMM, small shapes
ALL = (1, 2, 3, 4, 5)          # streaming; tiled with the default tile, 128x128, 256x128, 256x256
TILED = (2, 3, 4, 5)
SHAPES = [  # (M, N, K, paths)
    (4, 128, 256, ALL),         # the small config
    (1, 16, 128, ALL),
    (3, 48, 384, ALL),
    (16, 272, 1024, ALL),
    (8, 336, 2048, ALL),        # decode with four K parts per tile and two windows in flight
    (5, 96, 4096, (1,)),        # decode, rows staged eight loads per thread, the last batch partial
    (16, 64, 8704, (1,)),       # decode, rows too long for one staging batch (staged in a loop)
    (17, 64, 256, ALL),
    (33, 32, 512, ALL),
    (64, 16, 128, ALL),
    (65, 128, 256, TILED),
    (130, 144, 384, TILED),     # ragged M and an N tail inside a 128-wide tile
    (257, 400, 640, TILED),
    (300, 128, 1152, TILED),    # odd group count over several groups
]


def _small_layer(orc, M, N, K, seed):
    W = synthetic.weights(seed, synthetic.TAG_W, 0, N, K)
    W += synthetic.column_means(seed, N)[:, None] * 3
    x = synthetic.activations(seed, M, K)
    q, s, z = orc.quantize_weights(W)
    return W, x, q, s, z


@pytest.mark.parametrize("M,N,K,paths", SHAPES)
def test_gemm_isums_bit_exact(orc, M, N, K, paths):
    w4 = w4mod()
    W, x, q, s, z = _small_layer(orc, M, N, K, seed=M + N)
    qr, sr = orc.quantize_act(x)
    iref = orc.group_isums(qr, q, z)
    packed, scale, zp = (to_dev(a) for a in w4.pack_weights(W))
    qa = to_dev(qr)
    for path in paths:
        isums = w4.gemm_debug_isums(qa, packed, zp, path=path)
        assert np.array_equal(to_host(isums), iref), f"path {path}"


@pytest.mark.parametrize("M,N,K,paths", SHAPES)
def test_gemm_fp32_within_tolerance(orc, M, N, K, paths):
    w4 = w4mod()
    W, x, q, s, z = _small_layer(orc, M, N, K, seed=M * 7 + N)
    ref, mag = orc.gemm(*orc.quantize_act(x), q, s, z)
    packed, scale, zp = (to_dev(a) for a in w4.pack_weights(W))
    qa, sc = w4.quantize_act(to_dev(x))
    for path in paths:
        out = w4.gemm(qa, sc, packed, scale, zp, path=path)
        check_close(to_host(out), ref, mag, f"path {path}")


def test_gemm_zero_rows_and_default_path(orc):
    """An all-zero activation row gives scale 0 and an all-zero output row; path 0
    picks the streaming loop for M <= 64 and the tiled loop above."""
    w4 = w4mod()
    M, N, K = 80, 64, 256
    W, x, q, s, z = _small_layer(orc, M, N, K, seed=5)
    x[3] = 0.0
    packed, scale, zp = (to_dev(a) for a in w4.pack_weights(W))
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.gemm(qa, sc, packed, scale, zp))
    assert not out[3].any()
    ref, mag = orc.gemm(*orc.quantize_act(x), q, s, z)
    check_close(out, ref, mag)
    out16 = to_host(w4.gemm(qa[:16].contiguous(), sc[:16].contiguous(), packed, scale, zp))
    check_close(out16, ref[:16], mag[:16])


def test_gemm_deterministic():
    w4 = w4mod()
    M, N, K = 300, 256, 1024
    W = synthetic.weights(1, synthetic.TAG_W, 0, N, K)
    packed, scale, zp = (to_dev(a) for a in w4.pack_weights(W))
    qa, sc = w4.quantize_act(to_dev(synthetic.activations(1, M, K)))
    a = to_host(w4.gemm(qa, sc, packed, scale, zp))
    b = to_host(w4.gemm(qa, sc, packed, scale, zp))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ full-size dense workloads
def _sample_cols(N, count, seed):
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([[0, 1, 15, 16, N - 1], rng.choice(N, count, replace=False)]))
    return cols


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_full_size_sampled(orc, seed):
    """Decode layer K=8192, N=28672 (0.1% x20 weight outliers, 4 x50 activation channels),
    M = 1, 8, 16 -- the launch configuration the benchmark times (seed 0), and seeds 1, 2."""
    w4 = w4mod()
    N, K = 28672, 8192
    packed, scale, zp = device_layer(seed, synthetic.TAG_W, 0, N, K, mode="outliers")
    cols = _sample_cols(N, 96, 1 + 10 * seed)
    q, s, z = oracle_columns(orc, seed, synthetic.TAG_W, 0, K, cols, mode="outliers")
    assert np.array_equal(to_host(packed[cols]), orc.pack_nibbles(q))
    assert np.array_equal(u16(scale)[:, cols], s) and np.array_equal(u16(zp)[:, cols], z)
    x = synthetic.activations_with_outlier_channels(seed, 16, K)
    for M in (1, 8, 16):
        xm = x[:M]
        qr, sr = orc.quantize_act(xm)
        qa, sc = w4.quantize_act(to_dev(xm))
        assert np.array_equal(to_host(qa), qr)
        out = to_host(w4.gemm(qa, sc, packed, scale, zp))
        ms, ns = np.meshgrid(np.arange(M), np.arange(len(cols)), indexing="ij")
        ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel())
        check_close(out[:, cols].ravel(), ref, mag, f"decode M={M}")
        isums = to_host(w4.gemm_debug_isums(qa, packed, zp))
        assert np.array_equal(isums[:, :, cols], orc.group_isums(qr, q, z))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_full_size_sampled(orc, seed):
    """Prefill layer M=4096, K=8192, N=8192 with per-column mean offsets (seed 0 is the one the
    benchmark times)."""
    w4 = w4mod()
    M, N, K = 4096, 8192, 8192
    packed, scale, zp = device_layer(seed, synthetic.TAG_W, 0, N, K, mode="offset")
    cols = _sample_cols(N, 48, 2 + 10 * seed)
    q, s, z = oracle_columns(orc, seed, synthetic.TAG_W, 0, K, cols, mode="offset")
    assert np.array_equal(to_host(packed[cols]), orc.pack_nibbles(q))
    assert np.array_equal(u16(scale)[:, cols], s) and np.array_equal(u16(zp)[:, cols], z)
    assert (z != 0).any()
    x = synthetic.activations(seed, M, K)
    qr, sr = orc.quantize_act(x)
    qa, sc = w4.quantize_act(to_dev(x))
    assert np.array_equal(to_host(qa), qr)
    out = w4.gemm(qa, sc, packed, scale, zp)
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1],
                                     np.random.default_rng(3 + seed).choice(M, 200, replace=False)]))
    ms, ns = np.meshgrid(rows, np.arange(len(cols)), indexing="ij")
    ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel())
    got = to_host(out)[rows][:, cols].ravel()
    check_close(got, ref, mag, "prefill")
    isums = w4.gemm_debug_isums(qa[:256].contiguous(), packed, zp)
    assert np.array_equal(to_host(isums)[:, :, cols], orc.group_isums(qr[:256], q, z))


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("T,E,k,kind,seed", [(1, 8, 1, "iid", 7), (2, 8, 1, "iid", 7), (4, 8, 1, "iid", 7),
                                             (512, 8, 1, "iid", 7), (64, 384, 8, "skewed", 0),
                                             (4096, 384, 8, "skewed", 0), (64, 384, 8, "skewed", 1),
                                             (4096, 384, 8, "skewed", 1), (64, 384, 8, "skewed", 2),
                                             (4096, 384, 8, "skewed", 2), (3000, 1024, 8, "iid", 7),
                                             (0, 8, 1, "iid", 7)])
def test_route_bit_exact(orc, T, E, k, kind, seed):
    w4 = w4mod()
    logits = (synthetic.router_logits_iid(seed, T, E) if kind == "iid" else synthetic.router_logits_skewed(seed, T, E))
    ids, w, off, perm, rows, sop = (to_host(t) for t in w4.moe_route(to_dev(logits).reshape(T, E), k))
    ids_r, w_r = orc.route_topk(logits.reshape(T, E), k)
    off_r, perm_r = orc.bucket(ids_r, E)
    assert np.array_equal(ids, ids_r)
    assert np.allclose(w, w_r, rtol=2e-6, atol=1e-7)
    assert np.array_equal(off, off_r) and np.array_equal(perm, perm_r)
    inv = np.empty_like(perm_r)
    inv[perm_r] = np.arange(len(perm_r), dtype=np.int32)
    assert np.array_equal(sop, inv)
    assert np.array_equal(rows, perm_r // k)


@pytest.mark.parametrize("T,E,k,kind,shared", [(16, 384, 8, "skewed", True), (13, 1024, 8, "iid", False),
                                               (16, 40, 3, "iid", True), (5, 8, 2, "iid", False)])
def test_route_small_batch_one_launch(orc, T, E, k, kind, shared):
    """Batches of at most 16 tokens are routed and bucketed by one workgroup (one launch); the
    tables are the oracle's bit for bit, with the shared expert's slots appended when asked."""
    w4 = w4mod()
    logits = (synthetic.router_logits_iid(11, T, E) if kind == "iid" else synthetic.router_logits_skewed(1, T, E))
    ids, w, off, perm, rows, sop = (to_host(t) for t in w4.moe_route(to_dev(logits).reshape(T, E), k, shared))
    ids_r, w_r = orc.route_topk(logits.reshape(T, E), k)
    off_r, perm_r = orc.bucket(ids_r, E)
    assert np.array_equal(ids, ids_r)
    assert np.allclose(w, w_r, rtol=2e-6, atol=1e-7)
    assert np.array_equal(off[:E + 1], off_r) and np.array_equal(perm, perm_r)
    inv = np.empty_like(perm_r)
    inv[perm_r] = np.arange(len(perm_r), dtype=np.int32)
    assert np.array_equal(sop, inv)
    assert np.array_equal(rows[:T * k], perm_r // k)
    if shared:
        assert off[E + 1] == T * k + T
        assert np.array_equal(rows[T * k:], np.arange(T, dtype=np.int32))


def test_route_ties_go_to_lower_expert():
    w4 = w4mod()
    logits = np.zeros((3, 16), np.float32)
    logits[1, [3, 9, 12]] = 2.0
    ids, w, off, perm, rows, sop = (to_host(t) for t in w4.moe_route(to_dev(logits), 2))
    assert ids[0].tolist() == [0, 1] and ids[1].tolist() == [3, 9] and ids[2].tolist() == [0, 1]
    assert np.allclose(w, 0.5)


# ------------------------------------------------------------------ grouped GEMM
@pytest.mark.parametrize("K", [384, 1024, 8192, 8704])
def test_grouped_gemm_mixed_bucket_sizes(orc, K):
    """Experts with 0, 1, 17, 64, 65 and 200 slots: both loops (K=1024, 8192 and 8704
    take the decode-style loop for the small experts, the last with its staged rows
    near the LDS limit; K=384 the streaming one), an empty expert, ragged tails,
    gathered rows; every output element checked."""
    w4 = w4mod()
    counts = [0, 1, 17, 64, 65, 200]
    E, N = len(counts), 160
    R = 90
    rng = np.random.default_rng(4)
    S = sum(counts)
    row_index = rng.integers(0, R, S).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synthetic.activations(4, R, K)
    qr, sr = orc.quantize_act(x)
    packs, refs = [], []
    for e in range(E):
        W = synthetic.weights(4, synthetic.TAG_W, e, N, K)
        packs.append(w4.pack_weights(W))
        refs.append(orc.quantize_weights(W))
    packed = to_dev(np.stack([p[0] for p in packs]))
    scale = to_dev(np.stack([p[1] for p in packs]))
    zp = to_dev(np.stack([p[2] for p in packs]))
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.moe_grouped_gemm(qa, sc, to_dev(row_index), to_dev(offsets), packed, scale, zp, max_slots=S))
    for e in range(E):
        s0, s1 = offsets[e], offsets[e + 1]
        if s0 == s1:
            continue
        q, s, z = refs[e]
        ref, mag = orc.gemm(qr[row_index[s0:s1]], sr[row_index[s0:s1]], q, s, z)
        check_close(out[s0:s1], ref, mag, f"expert {e} ({s1 - s0} slots)")


@pytest.mark.parametrize("clamp", [0, 40])
def test_grouped_gemm_size_class_edges(orc, clamp):
    """Slot counts on both sides of every size class (16/17, 32/33, 64/65, 128/129),
    N = 544 (two full 256-column blocks and a partial one), K = 2048 (16 groups, four
    activation slices), so the loops cross units, chunks and experts inside one
    workgroup's range.  Slots whose row index is outside [0, R) are not written, and
    with `clamp` > 0 the slot count passed is smaller than the slots routed: slots at
    and past it are ignored and nothing is written beyond the output rows."""
    w4 = w4mod()
    counts = [16, 17, 3, 32, 33, 0, 64, 65, 1, 128, 129]
    E, N, K, R = len(counts), 544, 2048, 150
    rng = np.random.default_rng(7)
    S = sum(counts)
    row_index = rng.integers(0, R, S).astype(np.int32)
    bad = rng.choice(S, 6, replace=False)
    row_index[bad[:3]] = R + 5
    row_index[bad[3:]] = -1
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synthetic.activations(7, R, K)
    qr, sr = orc.quantize_act(x)
    packs, refs = [], []
    for e in range(E):
        W = synthetic.weights(7, synthetic.TAG_W, e, N, K)
        packs.append(w4.pack_weights(W))
        refs.append(orc.quantize_weights(W))
    packed = to_dev(np.stack([p[0] for p in packs]))
    scale = to_dev(np.stack([p[1] for p in packs]))
    zp = to_dev(np.stack([p[2] for p in packs]))
    qa, sc = w4.quantize_act(to_dev(x))
    max_slots = S - clamp
    import torch
    full = torch.full((S + 8, N), float("nan"), dtype=torch.float32, device=cuda())
    w4.moe_grouped_gemm(qa, sc, to_dev(row_index), to_dev(offsets), packed, scale, zp, max_slots=max_slots,
                        out=full[:max_slots])
    out = to_host(full)
    assert np.isnan(out[max_slots:]).all(), "rows past max_slots were written"
    valid = (row_index >= 0) & (row_index < R)
    for e in range(E):
        s0, s1 = min(offsets[e], max_slots), min(offsets[e + 1], max_slots)
        if s0 == s1:
            continue
        ok = np.nonzero(valid[s0:s1])[0] + s0
        assert np.isnan(out[s0:s1][~valid[s0:s1]]).all(), f"expert {e}: slots with an invalid row were written"
        q, s, z = refs[e]
        ref, mag = orc.gemm(qr[row_index[ok]], sr[row_index[ok]], q, s, z)
        check_close(out[ok], ref, mag, f"expert {e} ({offsets[e + 1] - offsets[e]} slots, max_slots {max_slots})")


def test_grouped_gemm_weight_streaming_loop(orc):
    """Experts with 17..128 slots and enough column blocks (N = 9216: 36 blocks of 256,
    396 units) that the weight-streaming loop runs rather than handing them to the
    decode loop; three whole column blocks (first, middle, last) checked per expert."""
    w4 = w4mod()
    counts = [17, 40, 64, 65, 100, 128, 20, 33]
    E, N, K, R = len(counts), 9216, 1024, 300
    rng = np.random.default_rng(11)
    S = sum(counts)
    row_index = rng.integers(0, R, S).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synthetic.activations(11, R, K)
    qr, sr = orc.quantize_act(x)
    cols = np.concatenate([np.arange(0, 256), np.arange(17 * 256, 18 * 256), np.arange(N - 256, N)])
    packs, refs = [], []
    for e in range(E):
        W = synthetic.weights(11, synthetic.TAG_W, e, N, K)
        packs.append(w4.pack_weights(W))
        q, s_, z = orc.quantize_weights(W[cols])
        refs.append((q, s_, z))
    packed = to_dev(np.stack([p[0] for p in packs]))
    scale = to_dev(np.stack([p[1] for p in packs]))
    zp = to_dev(np.stack([p[2] for p in packs]))
    qa, sc = w4.quantize_act(to_dev(x))
    out = to_host(w4.moe_grouped_gemm(qa, sc, to_dev(row_index), to_dev(offsets), packed, scale, zp, max_slots=S))
    for e in range(E):
        s0, s1 = offsets[e], offsets[e + 1]
        q, s_, z = refs[e]
        ref, mag = orc.gemm(qr[row_index[s0:s1]], sr[row_index[s0:s1]], q, s_, z)
        check_close(out[s0:s1][:, cols], ref, mag, f"expert {e} ({s1 - s0} slots)")


# Size classes of the expert loops: up to 16 slots (16-row chunks), 17-128 (one weight pass
# per 64 rows; handed to the 16-row loop when it has too few units for the machine), more than
# 128 (256-row tiles); and, when K/128 is not a multiple of 4, up to 64 slots streamed and the
# rest tiled (128-row tiles up to 128 slots).
GROUPED_ISUM_CASES = [  # (counts, N, K)
    ([16, 17, 3, 32, 33, 0, 64, 65, 1, 128, 129, 300], 2048, 2048),   # every class at the MoE down K
    ([5, 100, 20], 256, 2048),                  # a lone mid-size expert: the 16-row loop takes it
    ([1, 9, 40, 64, 65, 128, 200], 544, 384),   # K/128 = 3: streamed up to 64, tiled above
    ([7, 70, 150, 100, 40], 4096, 7168),        # the MoE gate/up shape
    ([2, 130], 160, 8704),                      # 16-row chunks with their rows near the LDS limit
]


@pytest.mark.parametrize("counts,N,K", GROUPED_ISUM_CASES)
def test_grouped_gemm_isums_bit_exact(orc, counts, N, K):
    """The per-group int32 sums of every slot of the expert-grouped GEMM, through the debug entry
    (the main loops each slot count selects), against the oracle's, bit for bit."""
    w4 = w4mod()
    E = len(counts)
    S = sum(counts)
    R = 311
    rng = np.random.default_rng(K + N)
    row_index = rng.integers(0, R, S).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qr, _ = orc.quantize_act(synthetic.activations(K + 3, R, K))
    packed = torch.empty((E, N, K // 2), dtype=torch.uint8, device=cuda())
    zp = torch.empty((E, K // 128, N), dtype=torch.int16, device=cuda())
    refs = []
    for e in range(E):
        W = synthetic.fill_weights_host(K, synthetic.TAG_W, e, K, 0, N, "offset" if e % 2 else "plain")
        q, s_, z = orc.quantize_weights(W)
        packed[e] = to_dev(orc.pack_nibbles(q))
        zp[e] = to_dev(z.view(np.int16))
        refs.append((q, z))
    isums = to_host(w4.moe_grouped_gemm_debug_isums(to_dev(qr), to_dev(row_index), to_dev(offsets), packed, zp,
                                                    max_slots=S))
    for e in range(E):
        s0, s1 = offsets[e], offsets[e + 1]
        if s0 == s1:
            continue
        q, z = refs[e]
        iref = orc.group_isums(qr[row_index[s0:s1]], q, z)
        bad = isums[:, s0:s1] != iref
        assert not bad.any(), f"expert {e} ({s1 - s0} slots): {int(bad.sum())} sums differ"


def test_grouped_gemm_256x256_loop(orc):
    """Enough slots and columns (2692 slots, N = 13440: 53 column tiles of 256, the last one
    half full) that the experts above 128 slots run on 256x256 tiles, small and mid-size experts
    beside them: per-group int32 sums bit-exact and fp32 outputs within tolerance for every slot
    on three sampled column ranges (the first tile, a middle one, the last one and a half)."""
    w4 = w4mod()
    counts = [3, 129, 700, 60, 1500, 300]
    E, N, K, R = len(counts), 13440, 1024, 311
    S = sum(counts)
    rng = np.random.default_rng(13)
    row_index = rng.integers(0, R, S).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synthetic.activations(13, R, K)
    qr, sr = orc.quantize_act(x)
    cols = np.concatenate([np.arange(0, 256), np.arange(6656, 6912), np.arange(N - 384, N)])
    packed, scale, zp = device_experts(13, synthetic.TAG_W, E, N, K)
    qa, sc = w4.quantize_act(to_dev(x))
    assert np.array_equal(to_host(qa), qr)
    ri, od, cd = to_dev(row_index), to_dev(offsets), to_dev(cols)
    isums = to_host(w4.moe_grouped_gemm_debug_isums(qa, ri, od, packed, zp, max_slots=S)[:, :, cd])
    out = to_host(w4.moe_grouped_gemm(qa, sc, ri, od, packed, scale, zp, max_slots=S)[:, cd])
    for e in range(E):
        s0, s1 = offsets[e], offsets[e + 1]
        q, s_, z = oracle_columns(orc, 13, synthetic.TAG_W, e, K, cols)
        rows = row_index[s0:s1]
        bad = isums[:, s0:s1] != orc.group_isums(qr[rows], q, z)
        assert not bad.any(), f"expert {e} ({s1 - s0} slots): {int(bad.sum())} sums differ"
        ref, mag = orc.gemm(qr[rows], sr[rows], q, s_, z)
        check_close(out[s0:s1], ref, mag, f"expert {e} ({s1 - s0} slots)")


def test_grouped_gemm_rows_past_32bit_offsets(orc):
    """R * K above 2^32 (1,052,672 activation rows of K = 4096, 4.3 GB): the loops that address
    rows with 32-bit offsets are not launched, and the streaming and 128-row tiled loops that
    take every slot class (5, 40, 100 and 200 slots) gather rows on both sides of the 4 GiB
    boundary; int32 sums bit-exact and fp32 outputs within tolerance for every slot."""
    w4 = w4mod()
    K, N = 4096, 256
    R = (1 << 20) + 4096
    assert R * K > (1 << 32)
    counts = [5, 40, 100, 200]
    E, S = len(counts), sum(counts)
    rng = np.random.default_rng(17)
    row_index = rng.integers((1 << 20) - 2048, R, S).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    gen = torch.Generator(device=cuda()).manual_seed(17)
    qa = torch.randint(-127, 128, (R, K), dtype=torch.int8, device=cuda(), generator=gen)
    sc = torch.rand((R,), dtype=torch.float32, device=cuda(), generator=gen) * 0.01 + 1e-3
    ri = to_dev(row_index)
    qrows, srows = to_host(qa[ri.long()]), to_host(sc[ri.long()])
    packed, scale, zp = device_experts(17, synthetic.TAG_W, E, N, K)
    od = to_dev(offsets)
    isums = to_host(w4.moe_grouped_gemm_debug_isums(qa, ri, od, packed, zp, max_slots=S))
    out = to_host(w4.moe_grouped_gemm(qa, sc, ri, od, packed, scale, zp, max_slots=S))
    del qa
    for e in range(E):
        s0, s1 = offsets[e], offsets[e + 1]
        q, s_, z = oracle_columns(orc, 17, synthetic.TAG_W, e, K, np.arange(N))
        bad = isums[:, s0:s1] != orc.group_isums(qrows[s0:s1], q, z)
        assert not bad.any(), f"expert {e} ({s1 - s0} slots): {int(bad.sum())} sums differ"
        ref, mag = orc.gemm(qrows[s0:s1], srows[s0:s1], q, s_, z)
        check_close(out[s0:s1], ref, mag, f"expert {e} ({s1 - s0} slots)")


@pytest.mark.parametrize("B,seed", [(1, 0), (2, 0), (4, 0), (512, 0), (512, 1), (512, 2)])
def test_toy_moe_full_size_sampled(orc, B, seed):
    """8 experts, top-1, K=4096, N=14336: route on the GPU, grouped GEMM, combine; the
    number of distinct experts is the oracle's, and B=512 touches all 8.  Seed 0 is the draw
    the benchmark times; seeds 1, 2 redraw weights, logits and activations at B=512."""
    w4 = w4mod()
    E, K, N = 8, 4096, 14336
    packed, scale, zp = device_experts(seed, synthetic.TAG_W, E, N, K)
    logits = synthetic.router_logits_iid(100 + B + 1000 * seed, B, E)
    x = synthetic.activations(100 + B + 1000 * seed, B, K)
    ids, w, off, perm, row_index, sop = w4.moe_route(to_dev(logits), 1)
    qa, sc = w4.quantize_act(to_dev(x))
    y = w4.moe_grouped_gemm(qa, sc, row_index, off, packed, scale, zp, max_slots=B)
    out = to_host(w4.moe_combine(y, sop, w))
    ids_r, w_r = orc.route_topk(logits, 1)
    off_r, _ = orc.bucket(ids_r, E)
    assert np.array_equal(to_host(ids), ids_r)
    touched = int((np.diff(off_r) > 0).sum())
    assert int((np.diff(to_host(off)) > 0).sum()) == touched
    if B == 1:
        assert touched == 1
    if B == 512:
        assert touched == 8
    qr, sr = orc.quantize_act(x)
    cols = _sample_cols(N, 40, B + seed)
    for e in np.unique(ids_r):
        q, s, z = oracle_columns(orc, seed, synthetic.TAG_W, int(e), K, cols)
        assert np.array_equal(to_host(packed[int(e)][cols]), orc.pack_nibbles(q))
        toks = np.nonzero(ids_r[:, 0] == e)[0]
        ms, ns = np.meshgrid(toks, np.arange(len(cols)), indexing="ij")
        ref, mag = orc.gemm_at(qr, sr, q, s, z, ms.ravel(), ns.ravel())
        check_close(out[toks][:, cols].ravel(), ref, mag, f"B={B} expert {e}")


# ------------------------------------------------------------------ SiLU*up + requant, combine
def _ambiguous(h, s):
    """Codes whose value h/s lies so close to a rounding boundary (x.5) or to the clamp
    that an fp32 ulp difference in h may decide them either way."""
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s[:, None] > 0, h / s[:, None].astype(np.float64), 0.0)
    frac = np.abs(np.abs(r) - np.floor(np.abs(r)) - 0.5)
    return frac < 1e-4 + 4e-6 * np.abs(r)


@pytest.mark.parametrize("P,I", [(37, 2048), (5, 3072), (3, 8192), (1, 16)])
def test_silu_mul_quantize(orc, P, I):
    w4 = w4mod()
    gu = synthetic.activations(31, P, 2 * I) * np.float32(3.0)
    qh, hs, h = (to_host(t) for t in w4.silu_mul_quantize(to_dev(gu), want_h=True))
    h_ref = orc.silu_mul(gu)
    assert np.allclose(h, h_ref, rtol=4e-6, atol=1e-30)
    gxu = np.abs(gu[:, :I].astype(np.float64) * gu[:, I:].astype(np.float64))
    assert (np.abs(h - h_ref) <= 1e-5 * gxu + 1e-7).all()
    # the codes and row scales: bit-exact against the per-token quantizer applied to the
    # kernel's own fp32 h
    q_o2, s_o2 = orc.quantize_act(h)
    assert np.array_equal(qh, q_o2)
    assert np.array_equal(hs.view(np.uint32), s_o2.view(np.uint32))
    # the per-token quantizer kernel over the same h bytes gives the same codes
    qx, sx = (to_host(t) for t in w4.quantize_act(to_dev(h)))
    assert np.array_equal(qx, qh) and np.array_equal(sx.view(np.uint32), hs.view(np.uint32))
    amax = np.abs(h_ref).max(1)
    assert np.allclose(hs, amax / 127.0, rtol=1e-5)
    # codes: the oracle's quantizer applied to the oracle's own h (rounded to fp32);
    # equal wherever the decision is not within fp32 noise of a tie
    q_ref, s_ref = orc.quantize_act(h_ref.astype(np.float32))
    amb = _ambiguous(h_ref, s_ref)
    diff = qh.astype(np.int32) - q_ref.astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert not (diff[~amb] != 0).any(), f"{int((diff[~amb] != 0).sum())} unambiguous codes differ"


@pytest.mark.parametrize("k", [8, 3, 1, 11])
def test_combine(orc, k):
    """Top-k of 1, 3, 8 and 11 rows per token, against the oracle, and bit for bit against
    a sequential fp32 fma chain in pick order."""
    w4 = w4mod()
    T, H = 33, 7168
    S = T * k + 5
    y = synthetic.activations(41, S, H)
    ys = synthetic.activations(42, T, H)
    rng = np.random.default_rng(5)
    sop = rng.permutation(S)[:T * k].astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    out = to_host(w4.moe_combine(to_dev(y), to_dev(sop.ravel()), to_dev(w), to_dev(ys)))
    ref = orc.combine(y, sop, w, ys)
    mag = np.abs(w).astype(np.float64) @ np.ones((k, 1)) * np.abs(y).max() + np.abs(ys)
    assert (np.abs(out - ref) <= 1e-6 * mag + 1e-7).all()
    out2 = to_host(w4.moe_combine(to_dev(y), to_dev(sop.ravel()), to_dev(w)))
    assert np.allclose(out2, orc.combine(y, sop, w), rtol=1e-5, atol=1e-6)
    # the same fmas in the same order as a plain sequential fp32 chain: identical bits.
    # fma emulated in x87 extended precision (the product of two fp32 is exact there; the
    # sum is rounded twice only in cases of probability ~2^-39 per step)
    ld = np.longdouble
    chain = np.zeros((T, H), np.float32)
    for j in range(k):
        chain = (w[:, j:j + 1].astype(ld) * y[sop[:, j]].astype(ld) + chain.astype(ld)).astype(np.float32)
    assert np.array_equal(out2, chain)
