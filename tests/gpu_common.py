"""Shared helpers of the GPU parity tests: device-side layer construction from the
seeded generator, and oracle-side reconstruction of sampled weight columns.

The oracle side never reads a value produced by the HIP library: its inputs come
from the seeded generator on the host (numpy or the C filler, which are pinned to
each other), and it quantizes them itself."""
from __future__ import annotations

import numpy as np

import synthetic


def cuda():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(cuda())


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def device_layer(seed, tag, sub, N, K, mode="plain", group=128):
    """Packed weights of one [N][K] layer built on the device: the GPU filler writes
    the fp32 weights, the library's device packer quantizes them (groups of `group`)."""
    import torch
    import w4a8_quantized_gemm_token_amd as w4
    W = torch.empty((N, K), dtype=torch.float32, device=cuda())
    synthetic.fill_weights_device(W, seed, tag, sub, K, 0, mode)
    packed, scale, zp = w4.pack_weights_device(W, group=group)
    del W
    return packed, scale, zp


def device_experts(seed, tag, E, N, K, sub0=0, out=None, group=128):
    """Stacked expert weights [E][N][K/2], [E][K/group][N] x2, expert e drawn from sub-stream sub0 + e."""
    import w4a8_quantized_gemm_token_amd as w4
    return w4.pack_experts_device(
        E, N, K, lambda e, W: synthetic.fill_weights_device(W, seed, tag, sub0 + e, K, 0, "plain"), cuda(),
        group=group, out=out)


def oracle_columns(orc, seed, tag, sub, K, cols, mode="plain", group=128):
    """Oracle quantization of the weight rows (= output columns) `cols` of a layer."""
    W = synthetic.weight_rows_host(seed, tag, sub, K, cols, mode)
    return orc.quantize_weights(W, group)


def check_close(out, ref, mag, what=""):
    tol = 1e-5 * mag + 1e-6
    err = np.abs(out.astype(np.float64) - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"worst err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}, "
                           f"tol there {tol.ravel()[err.argmax()]:.3e}")
    return float((err / tol).max())
