"""The seeded input generator: published SplitMix64 outputs, moments of the
N(0,1) stand-in, and the workload recipes' structure."""
import numpy as np

import synthetic


def test_splitmix64_reference_outputs():
    # SplitMix64 seeded with 0 (state advanced by the golden gamma before each output):
    # the first outputs of the published reference generator.
    got = synthetic.bits(0, np.arange(2))
    assert [hex(int(v)) for v in got] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4"]


def test_normal_standin_moments():
    z = synthetic.normal(synthetic.stream_key(0, synthetic.TAG_X), np.arange(1 << 20))
    assert z.dtype == np.float32
    assert abs(z.mean()) < 0.005 and abs(z.std() - 1.0) < 0.005
    assert np.abs(z).max() <= 2 * np.sqrt(3) + 1e-6


def test_activations_true_normal():
    # activations and router logits are true N(0,1) draws, tails included
    from scipy import stats
    x = synthetic.activations(0, 256, 4096)
    assert x.dtype == np.float32 and abs(x.mean()) < 0.005 and abs(x.std() - 1.0) < 0.005
    assert stats.kstest(x.ravel()[:200000].astype(np.float64), "norm").pvalue > 1e-3
    # P(|z| > 4) = 6.33e-5: about 66 of 2^20 draws, none under a +-3.46 sigma stand-in
    assert 30 < int((np.abs(x) > 4).sum()) < 110
    assert np.array_equal(synthetic.activations(0, 256, 4096, rows=[7, 200]), x[[7, 200]])
    assert not np.array_equal(synthetic.activations(1, 4, 64), synthetic.activations(0, 4, 64))


def test_moe_layer_routing_spread():
    # full MoE layer, 384 experts, top-8, Zipf(1.1) bias: with true-normal logits seed 0 reaches the
    # cold experts the configured skew implies (about 166 at T=4096 and about 53 at T=64 on average)
    for T, lo, hi in [(64, 42, 59), (4096, 155, 177)]:
        z = synthetic.router_logits_skewed(0, T, 384)
        ids = np.argsort(-z, axis=1, kind="stable")[:, :8]
        assert lo <= len(np.unique(ids)) <= hi, T


def test_weight_recipes():
    W = synthetic.weights(0, synthetic.TAG_W, 0, 64, 256)
    assert W.shape == (64, 256) and abs(W.std() - 0.02) < 0.001
    # any subset of rows regenerates identically
    assert np.array_equal(synthetic.weights(0, synthetic.TAG_W, 0, 64, 256, rows=[5, 63]), W[[5, 63]])
    Wo = synthetic.weights_with_outliers(0, 256, 4096)
    frac = (np.abs(Wo) > 0.02 * 2 * np.sqrt(3) + 1e-6).mean()
    assert 0.0002 < frac < 0.002
    mu = synthetic.column_means(0, 8192)
    assert mu.min() >= -0.01 and mu.max() < 0.01 and abs(mu.mean()) < 0.001
    x = synthetic.activations_with_outlier_channels(0, 4, 8192)
    ch = synthetic.outlier_channels(0, 8192)
    assert len(set(ch.tolist())) == 4 and np.abs(x[:, ch]).max() > 10


def test_router_recipes():
    z = synthetic.router_logits_skewed(0, 64, 384)
    b = synthetic.zipf_bias(384)
    assert b[0] == 0 and np.all(np.diff(b) < 0)
    assert z.shape == (64, 384) and z.dtype == np.float32


def test_host_filler_matches_numpy():
    # plain, outliers and offset recipes: the C filler gives the numpy bytes
    for mode, ref in [("plain", lambda r: synthetic.weights(3, synthetic.TAG_W, 5, 300, 512, rows=r)),
                      ("outliers", lambda r: synthetic.weights_with_outliers(3, 300, 512, rows=r)),
                      ("offset", lambda r: synthetic.weights_with_offset(3, 300, 512, rows=r))]:
        sub = 5 if mode == "plain" else 0
        got = synthetic.fill_weights_host(3, synthetic.TAG_W, sub, 512, 17, 40, mode)
        assert np.array_equal(got.view(np.uint32), ref(np.arange(17, 57)).view(np.uint32)), mode
    rows = [299, 3, 150]
    assert np.array_equal(synthetic.weight_rows_host(3, synthetic.TAG_W, 5, 512, rows),
                          synthetic.weights(3, synthetic.TAG_W, 5, 300, 512, rows=rows))
