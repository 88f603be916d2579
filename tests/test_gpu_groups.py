"""GPU parity of group sizes 64 and 256 ([p2 §4.3] weighs 64, 128 and 256) on the tiled
loop: per-group int32 sums bit-exact against the oracle, outputs within the oracle
tolerance 1e-5 * sum_g |a_scale * w_scale * isum_g| + 1e-6, both workgroup tiles, odd and
even 128-k stage counts, ragged row and column tiles, and the prefill shape sampled.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import check_close, to_dev, to_host

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
    if path == 3:  # the default choice (path 0) for this group size is the tiled loop too
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
