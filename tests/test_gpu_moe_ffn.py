"""GPU parity of the whole MoE FFN layer (route -> quantize -> gate/up grouped GEMM
(+ shared expert) -> silu*up -> INT8 requant -> down grouped GEMM -> combine).

The oracle runs its own chain from the same seeded inputs: routing and the first
GEMM's integer stages must match exactly; the re-quantized hidden codes are decided
from each side's own fp32 h, so a code whose value lies within fp32 noise of a
rounding tie may differ by one.  The output tolerance is the product tolerance plus,
for each such ambiguous code, the largest change one code step can make.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import cuda, device_experts, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ambiguous(h, s):
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s[:, None] > 0, h / s[:, None].astype(np.float64), 0.0)
    frac = np.abs(np.abs(r) - np.floor(np.abs(r)) - 0.5)
    return frac < 1e-4 + 4e-6 * np.abs(r)


def oracle_token(orc, x_t, experts, weights, gate_up_q, down_q, I):
    """Oracle output row of one token: sum_j w_j * down_j(requant(silu*up(gate_up_j(x)))) + shared.
    experts: list of expert indices (the shared expert last, weight 1).  gate_up_q / down_q:
    callables e -> oracle (q, scale, zp) of that expert.  Returns (ref, tolerance)."""
    qa, sa = orc.quantize_act(x_t[None, :])
    ref = 0.0
    mag = 0.0
    allow = 0.0
    for e, wj in zip(experts, weights):
        q, s, z = gate_up_q(e)
        gu, _ = orc.gemm(qa, sa, q, s, z)
        h = orc.silu_mul(gu.astype(np.float32))
        qh, sh = orc.quantize_act(h.astype(np.float32))
        qd, sd, zd = down_q(e)
        y, ymag = orc.gemm(qh, sh, qd, sd, zd)
        ref = ref + np.float64(wj) * y[0]
        mag = mag + abs(np.float64(wj)) * ymag[0]
        amb = _ambiguous(h, sh)[0]
        if amb.any():
            ks = np.nonzero(amb)[0]
            sc = sd.view(np.float16).astype(np.float64)           # [G][H]
            step = 15.0 * sc[ks // 128].sum(0)                     # one code step at each k
            allow = allow + abs(np.float64(wj)) * np.float64(sh[0]) * step
    return ref, 1e-5 * mag + 1e-6 + allow


def _run_gpu_ffn(x, logits, topk, gate_up, down):
    import w4a8_quantized_gemm_token_amd as w4
    out, inter = w4.moe_ffn(to_dev(x), to_dev(logits), topk, gate_up, down)
    return to_host(out), inter


def test_moe_ffn_small_all_tokens(orc):
    """E=16 routed experts + 1 shared, top-4, H=512, I=256, T=40 skewed tokens."""
    E, k, H, I, T = 16, 4, 512, 256, 40
    gate_up = device_experts(3, synthetic.TAG_W, E + 1, 2 * I, H)
    down = device_experts(3, synthetic.TAG_W_DOWN, E + 1, H, I)
    x = synthetic.activations(3, T, H)
    logits = synthetic.router_logits_skewed(3, T, E)
    out, inter = _run_gpu_ffn(x, logits, k, gate_up, down)
    ids_r, w_r = orc.route_topk(logits, k)
    assert np.array_equal(to_host(inter["ids"]), ids_r)
    cache_gu, cache_d = {}, {}

    def gu_q(e):
        if e not in cache_gu:
            cache_gu[e] = orc.quantize_weights(synthetic.weights(3, synthetic.TAG_W, e, 2 * I, H))
        return cache_gu[e]

    def d_q(e):
        if e not in cache_d:
            cache_d[e] = orc.quantize_weights(synthetic.weights(3, synthetic.TAG_W_DOWN, e, H, I))
        return cache_d[e]

    off_r, perm_r = orc.bucket(ids_r, E)
    assert np.array_equal(to_host(inter["perm"]), perm_r)
    assert np.array_equal(to_host(inter["offsets"]), np.concatenate([off_r, [T * k + T]]))
    assert np.array_equal(to_host(inter["row_index"]), np.concatenate([perm_r // k, np.arange(T)]))
    # first GEMM integer stage: activation codes bit-exact
    qa_r, sa_r = orc.quantize_act(x)
    assert np.array_equal(to_host(inter["qa"]), qa_r)
    for t in range(T):
        experts = list(ids_r[t]) + [E]
        weights = list(w_r[t]) + [1.0]
        ref, tol = oracle_token(orc, x[t], experts, weights, gu_q, d_q, I)
        err = np.abs(out[t] - ref)
        assert (err <= tol).all(), f"token {t}: worst {err.max():.3e} vs tol {tol[err.argmax()]:.3e}"


@pytest.mark.parametrize("T", [64, 4096])
def test_moe_ffn_full_size_sampled_tokens(orc, T):
    """384 routed experts (Zipf-skewed router bias) + 1 shared, top-8, H=7168, I=2048:
    the routing tables are compared in full, the output on sampled tokens."""
    E, k, H, I = 384, 8, 7168, 2048
    gate_up = device_experts(0, synthetic.TAG_W, E + 1, 2 * I, H)
    down = device_experts(0, synthetic.TAG_W_DOWN, E + 1, H, I)
    x = synthetic.activations(0, T, H)
    logits = synthetic.router_logits_skewed(0, T, E)
    out, inter = _run_gpu_ffn(x, logits, k, gate_up, down)
    ids_r, w_r = orc.route_topk(logits, k)
    off_r, perm_r = orc.bucket(ids_r, E)
    assert np.array_equal(to_host(inter["ids"]), ids_r)
    assert np.array_equal(to_host(inter["perm"]), perm_r)
    assert np.array_equal(to_host(inter["offsets"])[:E + 1], off_r)
    counts = np.diff(off_r)
    print(f"T={T}: experts touched {int((counts > 0).sum())}, largest bucket {int(counts.max())}")

    def gu_q(e):
        return orc.quantize_weights(synthetic.fill_weights_host(0, synthetic.TAG_W, int(e), H, 0, 2 * I))

    def d_q(e):
        return orc.quantize_weights(synthetic.fill_weights_host(0, synthetic.TAG_W_DOWN, int(e), I, 0, H))

    toks = [0, T - 1] if T > 64 else [0, 31, T - 1]
    for t in toks:
        experts = list(ids_r[t]) + [E]
        weights = list(w_r[t]) + [1.0]
        ref, tol = oracle_token(orc, x[t], experts, weights, gu_q, d_q, I)
        err = np.abs(out[t] - ref)
        assert (err <= tol).all(), f"token {t}: worst {err.max():.3e} vs tol {tol[err.argmax()]:.3e}"
