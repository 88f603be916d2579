"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError when the
oracle disagrees with something the pages print, a closed form, a brute-force
enumeration or an independent library route (numpy / scipy).  The same pins run
against deliberately broken copies of the oracle (tests/test_oracle_mutants.py)
to show that a plausible mistake anywhere in it is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(x):
    return np.float32(np.float16(np.float32(x)))


# ------------------------------------------------------------------ fp16 conversion
def pin_f16_matches_numpy(orc):
    """fp32 -> fp16 (RNE) and fp16 -> fp32 agree with numpy's binary16 conversion."""
    rng = np.random.default_rng(1)
    vals = [0.0, -0.0, 1.0, 1.1, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 6.1e-5, 1.0 + 2.0 ** -11,
            1.0 + 3 * 2.0 ** -11, 2048.5, 0.0666666]
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 3000))
    vals = np.concatenate([np.array(vals), mags, -mags]).astype(np.float32)
    got = orc.f32_to_f16_bits(vals)
    exp = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp), f"fp16 RNE mismatch at {vals[got != exp][:5]}"
    allbits = np.arange(0, 1 << 16, 37, dtype=np.uint32).astype(np.uint16)
    allbits = allbits[(allbits & 0x7C00) != 0x7C00]
    back = orc.f16_bits_to_f32(allbits)
    assert np.array_equal(back, allbits.view(np.float16).astype(np.float32))


# ------------------------------------------------------------------ O1 weight quantization
def pin_p1_range_0_to_15(orc):
    """[p1 §2.1] a range of 0..15 gives scale 1 and the codes are the integers themselves."""
    g = _golden("p1_4bit_ranges.json")["cases"][0]
    w = (np.arange(128) % 16).astype(np.float32)[None, :]
    q, s, z = orc.quantize_weights(w)
    assert s[0, 0] == np.float16(g["scale"]).view(np.uint16)
    assert z[0, 0] == 0
    assert np.array_equal(q[0], w[0].astype(np.uint8))


def pin_round_half_even(orc):
    """Ties round to even (the workload statement's round-half-even), in both quantizers:
    a 0..15 weight group has scale 1, so 2.5 -> 2 and 3.5 -> 4; an activation row with
    max|x| = 127 has scale 1, so 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0."""
    w = (np.arange(128) % 16).astype(np.float32)[None, :]
    w[0, 20], w[0, 21], w[0, 22] = 2.5, 3.5, 12.5
    q, s, z = orc.quantize_weights(w)
    assert s[0, 0] == 0x3C00 and z[0, 0] == 0
    assert list(q[0, 20:23]) == [2, 4, 12]
    qa, sc = orc.quantize_act(np.array([[127.0, 2.5, 3.5, -2.5, 0.5, -126.5]], np.float32))
    assert sc[0] == 1.0 and list(qa[0]) == [127, 2, 4, -2, 0, -126]


def pin_p1_range_0_to_16_5(orc):
    """[p1 §2.1] a range of 0..16.5 gives scale about 1.1 (1.099609375 after fp16 rounding)."""
    g = _golden("p1_4bit_ranges.json")["cases"][1]
    w = np.linspace(0.0, 16.5, 128).astype(np.float32)[None, :]
    q, s, z = orc.quantize_weights(w)
    scale = np.uint16(s[0, 0]).view(np.float16)
    assert abs(float(scale) - g["scale_approx"]) < 0.001
    assert s[0, 0] == np.float16(np.float32(16.5) / np.float32(15.0)).view(np.uint16)
    assert z[0, 0] == 0 and q[0, 0] == 0 and q[0, -1] == 15


def _lattice_weights():
    """W[n][g*128 + i] = (i % 16 - zp0[n][g]) * step[n][g]: every group is an exact
    16-point lattice, so scale = step, zp = zp0 and q = i % 16 by the formulas."""
    N, G = 3, 2
    steps = np.array([[0.25, 2.0 ** -7], [0.5, 0.125], [2.0 ** -9, 1.5]], np.float32)   # [N][G]
    zps = np.array([[3, 12], [0, 7], [15, 5]], np.int64)
    W = np.empty((N, G * 128), np.float32)
    for n in range(N):
        for g in range(G):
            i = np.arange(128)
            W[n, g * 128:(g + 1) * 128] = ((i % 16) - zps[n, g]) * steps[n, g]
    return W, steps, zps


def pin_lattice_groups(orc):
    """Closed form on exact lattices: pins the [G][N] layout of scale/zp and the codes."""
    W, steps, zps = _lattice_weights()
    q, s, z = orc.quantize_weights(W)
    assert s.shape == (2, 3)
    assert np.array_equal(s, steps.T.astype(np.float16).view(np.uint16))
    assert np.array_equal(z, zps.T.astype(np.float16).view(np.uint16))
    assert np.array_equal(q, np.tile(np.arange(128) % 16, (3, 2)).astype(np.uint8))
    deq = orc.dequantize_weights(q, s, z)
    assert np.array_equal(deq, W.astype(np.float64))


def pin_weight_quant_invariants(orc):
    """0 <= q, zp <= 15; |q - zp| <= 15; unclamped entries lie within s/2 (plus fp32
    rounding of w/s) of their reconstruction; the grid spans [min(0,w), max(0,w)];
    clamping is rare (only where fp16 rounding shrinks the scale)."""
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    W[:8] += 0.05          # one-signed groups: the range must still contain 0
    W[8:16] -= 0.05
    W[16, :128] = 0.0      # all-zero group
    q, s, z = orc.quantize_weights(W)
    sc = s.view(np.float16).astype(np.float64)
    zp = z.view(np.float16).astype(np.float64)
    assert q.max() <= 15 and zp.min() >= 0 and zp.max() <= 15
    G = W.shape[1] // 128
    clamped = 0
    for n in range(W.shape[0]):
        for g in range(G):
            w = W[n, g * 128:(g + 1) * 128].astype(np.float64)
            qq = q[n, g * 128:(g + 1) * 128].astype(np.float64)
            sv, zv = sc[g, n], zp[g, n]
            if not w.any():
                assert sv == 1.0 and zv == 0 and not qq.any()
                continue
            lo, hi = min(0.0, w.min()), max(0.0, w.max())
            assert abs(sv - (hi - lo) / 15) <= (hi - lo) / 15 * 2.0 ** -10
            assert abs(zv - (-lo / sv)) <= 0.5 + 1e-6
            err = np.abs(w - (qq - zv) * sv)
            edge = (qq == 0) | (qq == 15)
            assert (err[~edge] <= sv * (0.5 + 2.0 ** -19)).all()
            bad = err > sv * (0.5 + 2.0 ** -19)
            clamped += int(bad.sum())
            assert (0 - zv) * sv <= lo + sv * 0.5 + 1e-12 and (15 - zv) * sv >= hi - sv * 0.51
    assert clamped <= 8, clamped


def pin_p2_overhead(orc):
    """[p2 §2.3] fp16 scale + fp16 zp per 128 weights = 0.03125 B/weight, ~3.8x vs fp16."""
    g = _golden("p2_storage_overhead.json")
    W = np.zeros((4, 256), np.float32)
    W[:, 0] = 1.0
    q, s, z = orc.quantize_weights(W)
    packed = orc.pack_nibbles(q)
    per_weight_overhead = (s.nbytes + z.nbytes) / W.size
    assert per_weight_overhead == g["overhead_bytes_per_weight"]
    ratio = 2.0 / ((packed.nbytes + s.nbytes + z.nbytes) / W.size)
    assert abs(ratio - g["compression_vs_fp16_approx"]) < 0.05


# ------------------------------------------------------------------ nibble packing
def pin_nibble_order_and_roundtrip(orc):
    """[p2 §2.2] first code in the low nibble, second in the high nibble; every byte
    round-trips through unpack/pack and every pair of codes through pack/unpack."""
    assert orc.pack_nibbles(np.array([[1, 2]], np.uint8))[0, 0] == 0x21
    a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    q = np.stack([a.ravel(), b.ravel()], 1).reshape(1, -1).astype(np.uint8)
    p = orc.pack_nibbles(q)
    assert np.array_equal(p[0], (a.ravel() | (b.ravel() << 4)).astype(np.uint8))
    assert np.array_equal(orc.unpack_nibbles(p, q.shape[1]), q)
    allbytes = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(orc.pack_nibbles(orc.unpack_nibbles(allbytes, 512)), allbytes)


# ------------------------------------------------------------------ O2 activation quantization
def pin_p3_worked_int8_example(orc):
    """[p3 §2.1] range 0.5: scale 0.5/127 ~ 0.00394, 0.2 -> 51 -> ~0.201 (<1% error);
    range 1.0: scale ~0.0079, 0.2 -> 25 or 26, error ~2%."""
    g = _golden("p3_int8_worked_example.json")
    qa, sc = orc.quantize_act(np.array([[g["range_a"], g["value"], -0.3]], np.float32))
    assert abs(sc[0] - g["scale_a_approx"]) < 5e-6
    assert qa[0, 1] == g["code_a"] and qa[0, 0] == 127
    deq = float(qa[0, 1]) * float(sc[0])
    assert abs(deq - g["dequant_a_approx"]) < 5e-4
    assert abs(deq - g["value"]) / g["value"] * 100 < g["dequant_a_error_pct_below"]
    qb, sb = orc.quantize_act(np.array([[-g["range_b"], g["value"]]], np.float32))
    assert abs(sb[0] - g["scale_b_approx"]) < 5e-5
    assert qb[0, 1] in g["code_b_options"] and qb[0, 0] == -127
    err_pct = abs(float(qb[0, 1]) * float(sb[0]) - g["value"]) / g["value"] * 100
    assert abs(err_pct - g["dequant_b_error_pct_approx"]) < 0.6


def pin_act_quant_invariants(orc):
    """|q| <= 127 (never -128), the absmax entry maps to +-127, every code is the
    nearest integer to x/s (within fp32 rounding), zero rows give scale 0 and code 0."""
    rng = np.random.default_rng(3)
    tiny = np.float32(2.0 ** -149)
    x = rng.standard_normal((11, 640)).astype(np.float32)
    x[1] *= 1e-30
    x[2] = 0.0
    x[3, 7] = -40.0
    x[4] = np.abs(x[4])
    x[5] = 0.0
    x[5, :3] = np.array([-400, 150, 2], np.float32) * tiny     # subnormal row: scale 3 * 2^-149
    x[6] = 0.0
    x[6, 0] = -tiny * 60                                       # max|x|/127 underflows to 0
    qa, sc = orc.quantize_act(x)
    assert qa.min() >= -127 and qa.max() <= 127
    assert sc[2] == 0 and not qa[2].any()
    assert sc[6] == 0 and not qa[6].any()
    assert sc[5] == 3 * tiny and list(qa[5, :3]) == [-127, 50, 1]   # -400/3 clamps to -127
    for m in range(x.shape[0]):
        if m in (2, 5, 6):
            continue
        amax = np.abs(x[m]).max()
        assert sc[m] == np.float32(amax) / np.float32(127.0)
        i = np.abs(x[m]).argmax()
        assert abs(int(qa[m, i])) == 127 and np.sign(qa[m, i]) == np.sign(x[m, i])
        ratio = x[m].astype(np.float64) / np.float64(sc[m])
        assert (np.abs(ratio - qa[m]) <= 0.5 + 1e-5).all()


# ------------------------------------------------------------------ O3/O4 product + epilogue
def _random_layer(rng, M, N, K):
    W = (rng.standard_normal((N, K)) * 0.02 + rng.uniform(-0.01, 0.01, (N, 1))).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    return W, x


def pin_group_sizes_64_256(orc):
    """[p2 §4.3] group sizes 64 and 256: the lattice closed form holds per group of that
    size ([K/group][N] layout), each group's int32 sum is the integer dot product over
    exactly its k range (brute force), and the dequantize-then-matmul route agrees."""
    rng = np.random.default_rng(34)
    for group in (64, 256):
        N, G = 3, 3
        steps = rng.choice(np.float32([0.25, 0.5, 2.0 ** -7, 0.125, 1.5]), (N, G))
        zps = rng.integers(0, 16, (N, G))
        i = np.arange(group)
        W = np.concatenate([((i % 16) - zps[:, g:g + 1]) * steps[:, g:g + 1] for g in range(G)], 1).astype(np.float32)
        q, s, z = orc.quantize_weights(W, group)
        assert s.shape == (G, N)
        assert np.array_equal(s, steps.T.astype(np.float16).view(np.uint16))
        assert np.array_equal(z, zps.T.astype(np.float16).view(np.uint16))
        assert np.array_equal(q, np.tile(i % 16, (N, G)).astype(np.uint8))
        M, K = 2, G * group
        qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
        isums = orc.group_isums(qa, q, z, group)
        zf = np.float16(z.view(np.float16)).astype(np.int64)
        for g in range(G):
            ks = slice(g * group, (g + 1) * group)
            want = qa[:, ks].astype(np.int64) @ (q[:, ks].astype(np.int64) - zf[g][:, None]).T
            assert np.array_equal(isums[g], want), group
        a_s = np.float32([0.01, 0.003])
        out, _ = orc.gemm(qa, a_s, q, s, z, group)
        deq = orc.dequantize_weights(q, s, z, group)
        ref = (qa.astype(np.float64) * a_s.astype(np.float64)[:, None]) @ deq.T
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def pin_integer_special_case(orc):
    """All scales 1, all zero points 0, a_scale 1: the layer is a plain integer matmul."""
    rng = np.random.default_rng(4)
    for M, N, K in [(1, 1, 128), (3, 17, 256), (2, 5, 384)]:
        qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
        q = rng.integers(0, 16, (N, K)).astype(np.uint8)
        G = K // 128
        ones = np.full((G, N), 0x3C00, np.uint16)
        zeros = np.zeros((G, N), np.uint16)
        exact = qa.astype(np.int64) @ q.astype(np.int64).T
        isums = orc.group_isums(qa, q, zeros)
        assert np.array_equal(isums.sum(0), exact)
        out, _ = orc.gemm(qa, np.ones(M, np.float32), q, ones, zeros)
        assert np.array_equal(out, exact.astype(np.float64))


def pin_dequantized_matmul_route(orc):
    """Independent route: dequantize both operands to double (s_m*qa, scale*(q-zp)) and
    multiply with numpy; it must agree with the per-group integer path to ~1e-12."""
    rng = np.random.default_rng(5)
    for M, N, K in [(1, 3, 128), (3, 17, 256), (2, 9, 512)]:
        W, x = _random_layer(rng, M, N, K)
        q, s, z = orc.quantize_weights(W)
        qa, sc = orc.quantize_act(x)
        G = K // 128
        sc_w = np.repeat(s.view(np.float16).astype(np.float64).T, 128, axis=1)   # [N][K]
        zp_w = np.repeat(z.view(np.float16).astype(np.float64).T, 128, axis=1)
        w_hat = (q.astype(np.float64) - zp_w) * sc_w
        x_hat = qa.astype(np.float64) * sc.astype(np.float64)[:, None]
        ref = x_hat @ w_hat.T
        out, mag = orc.gemm(qa, sc, q, s, z)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        at, mag_at = orc.gemm_at(qa, sc, q, s, z, ms.ravel(), ns.ravel())
        assert np.array_equal(at, out.ravel()) and np.array_equal(mag_at, mag.ravel())
        assert (mag >= np.abs(out) - 1e-12).all()
        # and the per-group int32 sums, group by group, against numpy's integer matmul
        isums = orc.group_isums(qa, q, z)
        for g in range(G):
            ks = slice(g * 128, (g + 1) * 128)
            exact = qa[:, ks].astype(np.int64) @ (q[:, ks].astype(np.int64) - zp_w[:, ks].astype(np.int64)).T
            assert np.array_equal(isums[g], exact)


def pin_int32_accumulator_range(orc):
    """[p2 §3.2, §5.4] the per-group sum needs int32: the extreme 128*127*15 = 243840
    (beyond int16) comes out exactly, with both signs."""
    qa = np.full((2, 128), 127, np.int8)
    qa[1] = -127
    q = np.full((1, 128), 15, np.uint8)
    isums = orc.group_isums(qa, q, np.zeros((1, 1), np.uint16))
    assert isums[0, 0, 0] == 243840 and isums[0, 1, 0] == -243840
    q0 = np.zeros((1, 128), np.uint8)
    isums = orc.group_isums(qa, q0, np.full((1, 1), np.float16(15).view(np.uint16), np.uint16))
    assert isums[0, 0, 0] == -243840


# ------------------------------------------------------------------ router and buckets
def pin_p4_toy_router(orc):
    """[p4] closed form 8*(1-(7/8)^B) equals exhaustive enumeration, and both print as
    the page's output for B = 1, 2, 4."""
    import oracle as orc_mod
    path = os.path.join(GOLDEN, "p4_toy_router_output.txt")
    lines = [ln.strip() for ln in open(path) if ln.startswith("toy")]
    for B, line in zip((1, 2, 4), lines):
        closed = orc_mod.toy_router_expected_unique(8, B)
        brute = orc_mod.toy_router_exhaustive(8, B)
        assert abs(closed - brute) < 1e-12
        assert f"toy batch={B}: {closed:.6f} unique experts" == line


def pin_topk_against_numpy(orc):
    """Top-k = numpy stable argsort of the negated logits (ties -> lower id), weights =
    scipy softmax over the selected logits."""
    rng = np.random.default_rng(6)
    for T, E, k in [(5, 8, 1), (7, 40, 8), (3, 384, 8)]:
        z = rng.standard_normal((T, E)).astype(np.float32)
        z[0, 3] = z[0, 5] = z[0].max() + 1     # an exact tie at the top
        ids, w = orc.route_topk(z, k)
        exp_ids = np.argsort(-z, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, exp_ids)
        sel = np.take_along_axis(z, exp_ids, 1).astype(np.float64)
        assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-6, atol=0)
    assert orc.route_topk(np.array([[0.0, 1.0, 1.0]], np.float32), 1)[0][0, 0] == 1


def pin_buckets_against_numpy(orc):
    """offsets = exclusive scan of np.bincount; perm = numpy stable argsort of the ids."""
    rng = np.random.default_rng(7)
    for P, E in [(1, 8), (37, 8), (512, 385)]:
        ids = rng.integers(0, E, P).astype(np.int32)
        off, perm = orc.bucket(ids, E)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(ids, minlength=E))]))
        assert np.array_equal(perm, np.argsort(ids, kind="stable"))


def pin_toy_router_monte_carlo(orc):
    """[p4] the oracle's top-1 routing of iid logits touches 8(1-(7/8)^B) experts on
    average (checked over many seeded draws; B = 512 touches all 8)."""
    import synthetic
    for B, draws in [(2, 4000), (4, 3000)]:
        logits = synthetic.router_logits_iid(11 + B, B * draws, 8)
        ids, _ = orc.route_topk(logits, 1)
        uniq = np.array([len(np.unique(ids[d * B:(d + 1) * B])) for d in range(draws)])
        expected = 8 * (1 - (7 / 8) ** B)
        sd = uniq.std() / math.sqrt(draws)
        assert abs(uniq.mean() - expected) < 5 * sd + 1e-9, (uniq.mean(), expected)
    logits = synthetic.router_logits_iid(5, 512, 8)
    ids, _ = orc.route_topk(logits, 1)
    off, _ = orc.bucket(ids, 8)
    assert (np.diff(off) > 0).sum() == 8


# ------------------------------------------------------------------ MoE pieces
def pin_silu_mul_and_combine(orc):
    """silu(g)*u against scipy's expit; the weighted combine against numpy."""
    rng = np.random.default_rng(8)
    gu = rng.standard_normal((5, 2 * 24)).astype(np.float32) * 4
    h = orc.silu_mul(gu)
    g, u = gu[:, :24].astype(np.float64), gu[:, 24:].astype(np.float64)
    assert np.allclose(h, g * scipy.special.expit(g) * u, rtol=1e-14, atol=1e-300)
    T, k, H = 4, 3, 10
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    sop = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    ys = rng.standard_normal((T, H)).astype(np.float32)
    out = orc.combine(y, sop, w, ys)
    ref = np.einsum("tk,tkh->th", w.astype(np.float64), y[sop].astype(np.float64)) + ys
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ packer variants
def pin_symmetric_weights_closed_forms(orc):
    """[p3 §2.1] b-bit symmetric: scale = max|w| / (2^(b-1) - 1) = max|w| / 7 for 4 bits,
    q = round(w / scale).  On an exact lattice j * step (j = -7..7, both ends present) the
    scale is step and the stored codes are j + 8 with zp 8; range [-1, 1] gives scale
    fp16(1/7) and 0.2 -> code 9; an all-zero group stores scale 1.0 and code 8."""
    rng = np.random.default_rng(31)
    N, K = 6, 512
    steps = np.array([2.0 ** -6, 0.375, 2.0 ** -10, 0.0625, 1.5, 2.0 ** -4], np.float32)
    j = rng.integers(-7, 8, (N, K))
    j[:, ::128] = 7
    j[:, 1::128] = -7
    W = (j * steps[:, None]).astype(np.float32)
    q, sc, zp = orc.quantize_weights_sym(W)
    assert np.array_equal(q.astype(np.int64), j + 8)
    assert np.array_equal(sc, np.tile(np.float16(steps).view(np.uint16), (K // 128, 1)))
    assert np.all(zp == np.float16(8.0).view(np.uint16))
    Wr = np.full((1, 128), 0.0, np.float32)
    Wr[0, 0], Wr[0, 1], Wr[0, 2] = -1.0, 1.0, 0.2
    q, sc, zp = orc.quantize_weights_sym(Wr)
    assert sc[0, 0] == np.float16(np.float32(1.0) / np.float32(7.0)).view(np.uint16)
    assert (q[0, 0], q[0, 1], q[0, 2], q[0, 3]) == (1, 15, 9, 8)
    q, sc, _ = orc.quantize_weights_sym(np.zeros((2, 128), np.float32))
    assert np.all(q == 8) and np.all(sc == 0x3C00)
    # reconstruction bound on random data: |w - (q - 8) * s| <= s / 2 (+ fp32 slack)
    W = rng.standard_normal((16, 1024)).astype(np.float32) * 0.02
    q, sc, _ = orc.quantize_weights_sym(W)
    s = np.repeat(np.float16(sc.view(np.float16)).astype(np.float64).T, 128, axis=1)
    err = np.abs(W - (q.astype(np.float64) - 8) * s)
    assert np.all(err <= s * (0.5 + 2.0 ** -19)) and q.min() >= 1 and q.max() <= 15


def pin_percentile_against_numpy(orc):
    """Linear-interpolation percentiles equal numpy's default method (computed in double);
    0 and 100 give the minimum and the maximum exactly."""
    rng = np.random.default_rng(32)
    for n in (1, 2, 7, 128, 1000, 8192):
        v = (rng.standard_normal(n) * np.exp(rng.uniform(-3, 3, n))).astype(np.float32)
        for pct in (0.0, 0.1, 12.5, 50.0, 99.9, 100.0):
            want = np.percentile(v.astype(np.float64), pct)
            # numpy forms the position as (n-1) * (pct/100), the oracle as (n-1) * pct / 100:
            # the two doubles differ by an ulp or so, which moves the result by ~1e-13 relative
            assert np.isclose(orc.percentile(v, pct), want, rtol=1e-12, atol=0), (n, pct)
        assert orc.percentile(v, 0.0) == v.min() and orc.percentile(v, 100.0) == v.max()


def pin_clip_rows(orc):
    """[p2 §2.2, §5.1] each row is clamped to its own [100-p, p] percentiles, rounded to
    fp32; p = 100 changes nothing; at 99.9 on a row with eight x20 outliers among 8192
    weights, only the tails move."""
    rng = np.random.default_rng(33)
    W = (rng.standard_normal((3, 8192)) * 0.02).astype(np.float32)
    W[0, rng.choice(8192, 8, replace=False)] *= 20
    assert np.array_equal(orc.clip_rows(W, 100.0), W)
    C = orc.clip_rows(W, 99.9)
    for n in range(3):
        lo = np.float32(np.percentile(W[n].astype(np.float64), 0.1))
        hi = np.float32(np.percentile(W[n].astype(np.float64), 99.9))
        assert np.array_equal(C[n], np.clip(W[n], lo, hi))
        assert (C[n] != W[n]).sum() <= 2 * 10
    assert np.abs(C[0]).max() < np.abs(W[0]).max() / 5


# ------------------------------------------------------------------ smoothing [p3 §3.4]
def pin_smoothing_factor_closed_forms(orc):
    """alpha = 0 gives s = 1/aw, alpha = 1 gives s = ax, alpha = 0.5 gives sqrt(ax/aw),
    which leaves both operands with the same channel maximum sqrt(ax*aw); a zero maximum on
    either side gives 1; inv_s is the fp32 rounding of 1/s for the stored fp32 s."""
    ax = np.array([4.0, 0.0, 9.0, 2.0, 1e-3, 50.0], np.float32)
    aw = np.array([1.0, 2.0, 0.25, 0.0, 3.0, 0.02], np.float32)
    live = (ax > 0) & (aw > 0)
    axd, awd = ax.astype(np.float64), aw.astype(np.float64)
    aws = np.where(live, awd, 1.0)
    for alpha, closed in ((0.0, 1.0 / aws), (1.0, axd), (0.5, np.sqrt(axd / aws))):
        s, inv = orc.smooth_factors(ax, aw, alpha)
        want = np.where(live, closed, 1.0)
        assert np.allclose(s, want, rtol=2.0 ** -23, atol=0), (alpha, s, want)
        assert np.array_equal(inv, (1.0 / s.astype(np.float64)).astype(np.float32))
    s, _ = orc.smooth_factors(ax, aw, 0.5)
    sd = s.astype(np.float64)
    assert np.allclose((axd / sd)[live], (awd * sd)[live], rtol=3e-7)
    assert np.allclose((axd / sd)[live], np.sqrt(axd * awd)[live], rtol=3e-7)
    rng = np.random.default_rng(21)
    ax = np.exp(rng.uniform(-8, 8, 4096)).astype(np.float32)
    aw = np.exp(rng.uniform(-8, 8, 4096)).astype(np.float32)
    s, inv = orc.smooth_factors(ax, aw, 0.37)
    want = ax.astype(np.float64) ** 0.37 / aw.astype(np.float64) ** 0.63
    assert np.allclose(s, want, rtol=2.0 ** -23, atol=0)
    assert np.array_equal(inv, (1.0 / s.astype(np.float64)).astype(np.float32))


def pin_smoothing_absmax_and_product(orc):
    """Channel maxima against numpy on a signed, non-square matrix; smoothing leaves the
    unquantized product unchanged up to the three fp32 roundings of each term."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((7, 300)).astype(np.float32) * np.exp(rng.uniform(-3, 3, 300)).astype(np.float32)
    x[:, 5] = -np.abs(x[:, 5]) * 40
    W = rng.standard_normal((11, 300)).astype(np.float32)
    W[:, 9] = 0.0
    ax, aw = orc.channel_absmax(x), orc.channel_absmax(W)
    assert np.array_equal(ax, np.abs(x).max(0)) and np.array_equal(aw, np.abs(W).max(0))
    s, inv = orc.smooth_factors(ax, aw, 0.5)
    assert s[9] == 1.0
    Ws = orc.smooth_weights(W, s)
    xd, Wd = x.astype(np.float64), W.astype(np.float64)
    xs = (xd * inv.astype(np.float64)).astype(np.float32)      # the product the quantizer sees
    ref = xd @ Wd.T
    got = xs.astype(np.float64) @ Ws.astype(np.float64).T
    bound = 4 * 2.0 ** -24 * (np.abs(xd) @ np.abs(Wd).T) + 1e-30
    assert np.all(np.abs(got - ref) <= bound)
    assert np.array_equal(Ws, (Wd * s.astype(np.float64)).astype(np.float32))


def pin_smoothing_quantizer_special_cases(orc):
    """inv_s = 1 is the plain per-token quantizer; alpha = 1 calibrated on the row itself
    divides each entry by its own magnitude, so every nonzero code is +-127 and the row
    scale is 1/127 (up to one ulp of the fp32 quotient x * (1/|x|))."""
    x = np.random.default_rng(23).standard_normal((5, 256)).astype(np.float32) * 3
    x[2, :7] = 0.0
    q0, s0 = orc.quantize_act(x)
    q1, s1 = orc.quantize_act_smooth(x, np.ones(256, np.float32))
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
    for r in range(5):
        ax = orc.channel_absmax(x[r:r + 1])
        s, inv = orc.smooth_factors(ax, np.ones(256, np.float32), 1.0)
        q, sc = orc.quantize_act_smooth(x[r:r + 1], inv)
        want = np.where(x[r] > 0, 127, np.where(x[r] < 0, -127, 0))
        assert np.array_equal(q[0], want), r
        assert abs(float(sc[0]) - 1.0 / 127.0) <= 2.0 ** -23 / 127.0, sc


PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
