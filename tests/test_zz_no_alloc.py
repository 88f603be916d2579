"""The MoE FFN entry point that allocates nothing (w4a8_moe_ffn_noalloc, intermediates in
the library's fixed per-GPU scratch) against w4a8_moe_ffn with a caller workspace: the
same kernels on the same inputs, so the outputs must be identical bytes.  Two calls in a
row, the second on a smaller layer, so the second runs over scratch the first has left
filled; then a layer too large for the scratch is rejected before anything runs."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests.gpu_common import device_experts, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_matches_workspace_entry_point():
    import w4a8_quantized_gemm_token_amd as w4
    E, k, H, I = 16, 4, 512, 256
    gate_up = device_experts(5, synthetic.TAG_W, E + 1, 2 * I, H)
    down = device_experts(5, synthetic.TAG_W_DOWN, E + 1, H, I)
    for T in (48, 13):   # second call smaller: it reads nothing the first one left behind
        x = to_dev(synthetic.activations(20 + T, T, H))
        logits = to_dev(synthetic.router_logits_skewed(20 + T, T, E))
        ref, _ = w4.moe_ffn(x, logits, k, gate_up, down)
        got = w4.moe_ffn_noalloc(x, logits, k, gate_up, down)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(got).view(np.uint32), to_host(ref).view(np.uint32)), f"T={T}"
        assert np.isfinite(to_host(got)).all()


def test_noalloc_rejects_layers_above_the_scratch():
    import w4a8_quantized_gemm_token_amd as w4
    E, k, H, I = 384, 8, 7168, 2048
    limit = w4.moe_ffn_noalloc_max_bytes()
    assert limit == 64 << 20
    assert w4.load().w4a8_moe_ffn_workspace_size(155, H, I, E, k) <= limit
    assert w4.load().w4a8_moe_ffn_workspace_size(156, H, I, E, k) > limit
    x = torch.zeros((156, H), dtype=torch.float32, device="cuda:0")
    logits = torch.zeros((156, E), dtype=torch.float32, device="cuda:0")
    s16 = torch.zeros((16,), dtype=torch.int16, device="cuda:0")
    gu = (torch.zeros((E + 1, 2 * I, 16), dtype=torch.uint8, device="cuda:0"), s16, s16)
    dn = (torch.zeros((E + 1, H, 16), dtype=torch.uint8, device="cuda:0"), s16, s16)
    with pytest.raises(w4.W4A8Error) as ei:
        w4.moe_ffn_noalloc(x, logits, k, gu, dn)
    assert ei.value.status == 4   # W4A8_EWORKSPACE: rejected before anything is launched
