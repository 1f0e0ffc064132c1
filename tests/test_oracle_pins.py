"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test names the passage (page title + section) or the
mathematical fact it checks.  Brute-force checks use exact rationals
(tests/exact.py) and share no code with the oracle.
"""
import json
import math
import os
from fractions import Fraction
from statistics import NormalDist

import numpy as np
import pytest
import torch

from tests.exact import frac, nearest_exact, rn32, round_half_even

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Codebook: 26. QLoRA and 4bit Quantization, Step 4 (printed table)
# --------------------------------------------------------------------------
def test_codebook_matches_printed_table(orc):
    g = _golden("ch26_step4_codebook.json")
    cb = orc.codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    np.testing.assert_array_equal(cb, np.array(g["codebook"], dtype=np.float32))


def test_codebook_shape_properties(orc):
    """Monotone, exact +0 at index 7, endpoints -1/+1 (Step 4 test asserts
    table[0] < 0 < table[-1])."""
    cb = orc.codebook()
    assert np.all(np.diff(cb) > 0)
    assert cb.view(np.uint32)[7] == 0  # +0.0, not -0.0
    assert cb[0] == -1.0 and cb[15] == 1.0
    assert cb[0] < 0 < cb[-1]


def test_codebook_vs_normal_quantiles(orc):
    """Step 2: q_i = Phi^-1((i - 0.5)/16), i = 1..16, normalised to [-1, 1].
    The printed table is called an approximation of these quantiles: every
    entry lies within 0.05 of the normalised quantile, with the same sign
    except the zero entry."""
    q = np.array([NormalDist().inv_cdf((i - 0.5) / 16) for i in range(1, 17)])
    qn = q / q[-1]
    cb = orc.codebook().astype(np.float64)
    assert np.max(np.abs(cb - qn)) <= 0.05
    for i in range(16):
        if i != 7:
            assert np.sign(cb[i]) == np.sign(qn[i])
    # denser near 0 than in the tails (Step 2: "denser near 0, sparser in the tails")
    gaps = np.diff(cb)
    assert gaps[6] < gaps[0] and gaps[8] < gaps[14]


# --------------------------------------------------------------------------
# Nearest codepoint: Step 2 worked example and exact brute force
# --------------------------------------------------------------------------
def test_worked_example_020_maps_to_0161(orc):
    g = _golden("ch26_step2_worked_example.json")
    cb = orc.codebook()
    i = orc.nearest_index(np.float32(g["normalised"]))
    assert cb[i] == np.float32(g["nearest_codepoint"])
    assert i == 9


def test_nearest_ties_go_low_and_neighbours(orc):
    """At every exact midpoint representable in fp32 the lower index wins; one
    ulp above, the upper index wins; one ulp below, the lower."""
    cb = orc.codebook()
    n_repr = 0
    for i in range(15):
        mid = (frac(cb[i]) + frac(cb[i + 1])) / 2
        m32 = np.float32(float(mid))
        if frac(m32) == mid:
            n_repr += 1
            assert orc.nearest_index(m32) == i
        up = np.nextafter(np.float32(float(mid)), np.float32(2))
        dn = np.nextafter(np.float32(float(mid)), np.float32(-2))
        if frac(up) > mid:
            assert orc.nearest_index(up) == i + 1
        if frac(dn) < mid:
            assert orc.nearest_index(dn) == i
    assert n_repr >= 1  # some midpoints are exact fp32 values, so ties occur


def test_nearest_matches_exact_rationals(orc):
    cb = orc.codebook()
    rng = np.random.default_rng(11)
    vs = np.concatenate([rng.uniform(-1, 1, 3000).astype(np.float32),
                         np.float32([-1, 1, 0, -0.0, 1e-30, -1e-30, 0.5, -0.5])])
    for v in vs:
        assert orc.nearest_index(v) == nearest_exact(frac(v), cb), v


# --------------------------------------------------------------------------
# Block quantisation (Lesson 09 sec. 9.2.1: normalise each block to [-1,1],
# nearest level, store 4-bit) and packing (22. ... Step 4: two per uint8)
# --------------------------------------------------------------------------
def _quantize_brute(w32: np.ndarray, block: int, cb):
    n = w32.size
    packed = bytearray((n + 1) // 2)
    absmax = []
    for b in range(0, n, block):
        blk = w32[b:b + block]
        a = max((abs(frac(v)) for v in blk), default=Fraction(0))
        absmax.append(np.float32(float(a)))
        for t, v in enumerate(blk):
            i = b + t
            idx = 7 if a == 0 else nearest_exact(frac(rn32(frac(v) / a)), cb)
            packed[i // 2] |= (idx << 4) if i % 2 == 0 else idx
    return np.frombuffer(bytes(packed), dtype=np.uint8), np.array(absmax, dtype=np.float32)


@pytest.mark.parametrize("n,block,dtype", [(64, 64, "f32"), (200, 64, "f32"), (129, 64, "bf16"),
                                           (77, 10, "f32"), (1, 64, "f32"), (64 * 5, 64, "bf16"),
                                           (128, 128, "f32"), (300, 128, "bf16"),
                                           (128 * 3 + 5, 128, "f32")])
def test_quantize_matches_exact_brute_force(orc, n, block, dtype):
    cb = orc.codebook()
    rng = np.random.default_rng(n * 7 + block)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if n > 8:
        w[3] = 0.0
        w[5] = -w[4]  # a +/- pair of equal magnitude
    if dtype == "bf16":
        w16 = orc.round_bf16(w)
        w = orc.bf16_to_f32(w16)
        packed, absmax = orc.quantize(w16, block)
    else:
        packed, absmax = orc.quantize(w, block)
    bp, ba = _quantize_brute(w, block, cb)
    np.testing.assert_array_equal(absmax, ba)
    np.testing.assert_array_equal(packed, bp)


def test_quantize_zero_block_codes_index_7(orc):
    w = np.zeros(128, dtype=np.float32)
    w[64:] = np.linspace(-0.3, 0.3, 64, dtype=np.float32)
    packed, absmax = orc.quantize(w, 64)
    assert absmax[0] == 0.0
    assert np.all(packed[:32] == 0x77)


def test_packing_fixture_ch26(orc):
    """Fixture indices [[0,1,2,3],[4,5,6,7],[8,9,10,11]] at scale 0.5 (Step 4
    tests).  Weights cb[idx]*0.5 normalise back to cb[idx] exactly, so the
    indices are recovered and packed two per byte, first element high."""
    g = _golden("ch26_step4_fixture.json")
    cb = orc.codebook()
    idx = np.array(g["indices"]).reshape(-1)
    w = (cb[idx] * np.float32(g["scale"])).astype(np.float32)
    packed, absmax = orc.quantize(w, 12)
    assert absmax.tolist() == [np.float32(0.5)]
    assert packed.tolist() == [0x01, 0x23, 0x45, 0x67, 0x89, 0xAB]
    np.testing.assert_array_equal(orc.unpack_indices(packed, 12), idx)


def test_odd_length_pads_low_nibble(orc):
    w = np.float32([0.1, -0.2, 0.3])
    packed, _ = orc.quantize(w, 64)
    assert packed.size == 2 and (packed[1] & 0x0F) == 0


def test_every_nonzero_block_hits_an_endpoint(orc):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(64 * 100) * 0.02).astype(np.float32)
    packed, _ = orc.quantize(w, 64)
    idx = orc.unpack_indices(packed, w.size).reshape(100, 64)
    assert np.all(np.any((idx == 0) | (idx == 15), axis=1))


# --------------------------------------------------------------------------
# Dequantisation (26. ... Step 4: table[idx] * scale)
# --------------------------------------------------------------------------
def test_dequant_fixture_ch26(orc):
    g = _golden("ch26_step4_fixture.json")
    cb_dec = [Fraction(str(c)) for c in _golden("ch26_step4_codebook.json")["codebook"]]
    idx = np.array(g["indices"]).reshape(-1)
    st = {"packed": np.uint8([0x01, 0x23, 0x45, 0x67, 0x89, 0xAB]), "n": 12, "block": 12,
          "block2": 256, "double_quant": False, "absmax": np.float32([g["scale"]])}
    w_hat = orc.dequantize(st)
    expect = [float(cb_dec[i] * Fraction(str(g["scale"]))) for i in idx]
    # [-0.5, -0.348, -0.2625, -0.1975, -0.142, -0.0925, -0.0455, 0, 0.04, 0.0805, 0.123, 0.169]
    np.testing.assert_allclose(w_hat, expect, rtol=2e-7, atol=0)


def test_dequant_error_bound_and_idempotence(orc):
    """Without double quantisation |w_hat - w| <= (largest half-gap) * absmax,
    the largest half-gap of the table being (1 - 0.696)/2 = 0.152.  Re-quantising
    the reconstruction gives back the same indices."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(64 * 512) * 0.02).astype(np.float32)
    st = orc.quantize_nf4(w, double_quant=False)
    w_hat = orc.dequantize(st)
    a = np.repeat(st["absmax"], 64)
    assert np.all(np.abs(w_hat - w) <= 0.152 * a * (1 + 1e-6))
    st2 = orc.quantize_nf4(w_hat, double_quant=False)
    np.testing.assert_array_equal(st2["packed"], st["packed"])


def test_nf4_beats_uniform_int4_on_normal_weights(orc):
    """gufacode ch.4 'NF4 principle' and 26. ... Step 2: on normal weights NF4
    loses less than uniform INT4 (16 evenly spaced levels on [-1,1], same
    block absmax).  Measured here: ratio about 0.84 clean and about 0.47 with
    0.1% outliers at 20 sigma (the pages' 1/3-1/2 is not reached on clean
    normals)."""
    gen = torch.Generator().manual_seed(7)
    w = (torch.randn(64 * 4096, generator=gen) * 0.02).numpy().astype(np.float32)

    def int4_mse(w):
        blk = w.reshape(-1, 64)
        a = np.abs(blk).max(axis=1, keepdims=True)
        levels = -1 + 2 * np.arange(16) / 15
        v = blk / a
        k = np.abs(v[..., None] - levels).argmin(-1)
        return float(np.mean((levels[k] * a - blk) ** 2))

    def nf4_mse(w):
        st = orc.quantize_nf4(w, double_quant=False)
        return float(np.mean((orc.dequantize(st).astype(np.float64) - w) ** 2))

    assert nf4_mse(w) / int4_mse(w) < 0.9
    wo = w.copy()
    pos = np.random.default_rng(1).choice(w.size, w.size // 1000, replace=False)
    wo[pos] = np.float32(0.4) * np.sign(np.random.default_rng(2).standard_normal(pos.size))
    assert nf4_mse(wo) / int4_mse(wo) < 0.6


# --------------------------------------------------------------------------
# Double quantisation (Lesson 09 sec. 9.2.2; gufacode ch.4: 4.5 -> ~4.127)
# --------------------------------------------------------------------------
def test_bits_per_param_arithmetic(orc):
    g = _golden("gc4_bits_per_param.json")
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(16384 * 4) * 0.02).astype(np.float32)
    st0 = orc.quantize_nf4(w, double_quant=False)
    st1 = orc.quantize_nf4(w, double_quant=True)
    assert orc.bits_per_param(st0) == g["bits_before_dq"]
    b1 = orc.bits_per_param(st1)
    assert b1 == 4 + 8 / 64 + 32 / (64 * 256) + 32 / w.size
    assert abs((4 + 8 / 64 + 32 / (64 * 256)) - g["bits_after_dq_approx"]) < 5e-4
    saved_gb = g["params_65b"] * (g["bits_before_dq"] - 4.126953125) / 8 / 1e9
    assert abs(saved_gb - g["saving_65b_gb_approx"]) < 0.1
    assert 1 - 4 / 16 == g["fp16_to_nf4_saving"]


def test_dq_mean_is_exact_mean(orc):
    rng = np.random.default_rng(13)
    a = np.abs(rng.standard_normal(10000) * 0.05).astype(np.float32)
    exact = sum((frac(v) for v in a), Fraction(0)) / a.size
    assert orc.dq_mean(a) == rn32(Fraction(float(exact)))  # fp64 then fp32, per the reading
    assert orc.dq_mean(a) == np.float32(np.mean(a.astype(np.float64)))


def test_dq_mean_exact_sum_decides_a_tie(orc):
    """Constants 2^60, 2^36, 2^7, 2^-100: the exact mean 2^58 + 2^34 + 2^5 +
    2^-102 lies just above the fp32 midpoint 2^58 + 2^34, so it rounds up to
    2^58 + 2^35; the exact sum rounded to fp64 (2^60 + 2^36 + 2^8, the
    2^-100 breaking the fp64 tie) keeps that.  A plain fp64 running sum drops
    2^7 at a tie and 2^-100, lands exactly on the fp32 midpoint and rounds
    down to 2^58: the pin fails an oracle that sums in fp64."""
    a = np.array([2.0 ** 60, 2.0 ** 36, 2.0 ** 7, 2.0 ** -100], dtype=np.float32)
    want = np.float32(2.0 ** 58 + 2.0 ** 35)
    assert orc.dq_mean(a) == want
    running = 0.0
    for v in a.tolist():
        running += v
    assert np.float32(running / a.size) != want
    exact = sum((frac(v) for v in a), Fraction(0)) / a.size
    assert rn32(exact) == want


def test_dq_mean_wide_range_matches_exact_rational(orc):
    """Constants spread over 2^-149 .. 2^120 (subnormals included): the mean
    is the exact sum rounded to fp64, divided by the count in fp64 and
    rounded to fp32."""
    rng = np.random.default_rng(31)
    e = rng.integers(-149, 120, 3000)
    a = (rng.uniform(1, 2, 3000) * np.exp2(e.astype(np.float64))).astype(np.float32)
    a[:5] = np.float32(2.0 ** -149) * np.arange(1, 6, dtype=np.float32)
    s = sum((frac(v) for v in a), Fraction(0))
    want = rn32(Fraction(float(Fraction(float(s)) / a.size)))
    assert orc.dq_mean(a) == want


def _dq_brute(absmax, mu, block2):
    q = []
    sig = []
    for c in range(0, absmax.size, block2):
        blk = absmax[c:c + block2]
        d = [rn32(frac(a) - frac(mu)) for a in blk]
        amax = max(abs(frac(v)) for v in d)
        s = rn32(amax / 127)
        sig.append(s)
        for v in d:
            if s == 0:
                q.append(0)
            else:
                t = round_half_even(frac(rn32(frac(v) / frac(s))))
                q.append(max(-127, min(127, t)))
    return np.array(q, dtype=np.int8), np.array(sig, dtype=np.float32)


@pytest.mark.parametrize("nb", [256, 1000, 5])
def test_dq_codes_match_exact_brute_force(orc, nb):
    rng = np.random.default_rng(nb)
    a = np.abs(rng.standard_normal(nb) * 0.04).astype(np.float32)
    a[0] = 0.4  # an outlier block constant
    mu = orc.dq_mean(a)
    q, s = orc.dq_codes(a, mu, 256)
    bq, bs = _dq_brute(a, mu, 256)
    np.testing.assert_array_equal(s, bs)
    np.testing.assert_array_equal(q, bq)


def test_dq_invariants(orc):
    rng = np.random.default_rng(21)
    w = (rng.standard_normal(64 * 256 * 6 + 64 * 17) * 0.02).astype(np.float32)
    st = orc.quantize_nf4(w, double_quant=True)
    q, s, mu, a = st["absmax_q"], st["absmax_scale"], st["absmax_mean"], st["absmax_raw"]
    assert s.size == math.ceil(a.size / 256)
    for c in range(s.size):
        blk = q[c * 256:(c + 1) * 256].astype(np.int32)
        assert np.max(np.abs(blk)) == 127  # the extreme constant of each block hits +/-127
    rec = (q.astype(np.float64) * np.repeat(s, 256)[:q.size].astype(np.float64) + float(mu))
    assert np.all(np.abs(rec - a) <= np.repeat(s, 256)[:q.size] * 0.5 * (1 + 1e-5) + 1e-9)
    # constant input: all constants equal -> sigma 0, codes 0, reconstruction = mean exactly
    wc = np.tile(np.float32([0.02] + [0.001] * 63), 300)
    stc = orc.quantize_nf4(wc, double_quant=True)
    assert np.all(stc["absmax_scale"] == 0) and np.all(stc["absmax_q"] == 0)
    np.testing.assert_array_equal(orc.dequantize(stc), orc.dequantize(orc.quantize_nf4(wc, False)))


def test_dq_dequant_uses_single_rounding_fma(orc):
    """The double-quantised scale is rebuilt as code*sigma + mu with one
    rounding; pinned against exact rationals."""
    rng = np.random.default_rng(4)
    w = (rng.standard_normal(64 * 300) * 0.02).astype(np.float32)
    st = orc.quantize_nf4(w, double_quant=True)
    w_hat = orc.dequantize(st)
    cb = orc.codebook()
    idx = orc.unpack_indices(st["packed"], w.size)
    for i in rng.integers(0, w.size, 400):
        b = i // 64
        a_rec = rn32(Fraction(int(st["absmax_q"][b])) * frac(st["absmax_scale"][b // 256])
                     + frac(st["absmax_mean"]))
        assert w_hat[i] == rn32(frac(cb[idx[i]]) * frac(a_rec))


def _rn_bf16_exact(f: Fraction) -> Fraction:
    """Exact round-to-nearest-even to 8 significant bits (bf16), normal range."""
    if f == 0:
        return Fraction(0)
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    return sign * round_half_even(a * Fraction(2) ** (7 - e)) * Fraction(2) ** (e - 7)


def test_round_bf16_is_rne(orc):
    vals = np.float32([1.0, 1.00390625, 1.005859375, 1.01171875, -2.5, 0.0, 3.0e-39, 65504.0, 0.161])
    got = orc.bf16_to_f32(orc.round_bf16(vals))
    for v, g in zip(vals, got):
        assert frac(g) == _rn_bf16_exact(frac(v)), v


def test_round_f16_hand_values(orc):
    """fp16 rounding (Gemma lesson 09, sec. 9.3 names fp16 as the other
    16-bit compute dtype): bit patterns worked out by hand from the binary16
    format (bias 15, 10 fraction bits, subnormal step 2^-24)."""
    cases = [
        (1.0, 0x3C00), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0 ** -11, 0x3C00),                 # tie between 1 and 1 + 2^-10: even
        (1.0 + 3 * 2.0 ** -11, 0x3C02),             # tie: up to the even 1 + 2^-9
        (1.0 + 2.0 ** -11 + 2.0 ** -20, 0x3C01),    # just past the tie
        (0.1, 0x2E66),                              # rint(0.1 * 2^14) = 1638 -> fraction 614
        (0.161, 0x3127),                            # rint(0.161 * 2^13) = 1319 -> fraction 295
        (65504.0, 0x7BFF),                          # largest finite
        (65519.99609375, 0x7BFF),                   # below the overflow tie
        (65520.0, 0x7C00),                          # tie with 2^16: to infinity
        (-1.0e6, 0xFC00),
        (2.0 ** -14, 0x0400),                       # smallest normal
        (2.0 ** -14 - 2.0 ** -25, 0x0400),          # subnormal tie 1023.5: up to the even 1024
        (2.0 ** -24, 0x0001),                       # smallest subnormal
        (2.0 ** -25, 0x0000),                       # tie with 0: even
        (1.5 * 2.0 ** -24, 0x0002),                 # tie 1.5: even 2
        (3.0e-39, 0x0000),                          # fp32 subnormal
    ]
    vals = np.float32([v for v, _ in cases])
    got = orc.round_f16(vals).view(np.uint16)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))


def _rn_f16_exact(v: Fraction) -> float:
    """Exact round-to-nearest-even of v to binary16: binade exponent e >= -14
    (the subnormals share the quantum 2^-24 of the lowest binade), 11
    significant bits; results past 65504 overflow to infinity."""
    a = abs(v)
    e = -14
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    r = round_half_even(a * Fraction(2) ** (10 - e)) * Fraction(2) ** (e - 10)
    out = math.inf if r > 65504 else float(r)
    return -out if v < 0 else out


def test_round_f16_matches_exact_rounding(orc):
    """Against exact rational rounding on a sweep over every binade of fp16
    (subnormals to overflow), the midpoints between neighbouring fp16 values
    and the fp32 values next to those midpoints."""
    rng = np.random.default_rng(17)
    mags = np.ldexp(rng.uniform(1, 2, 3000), rng.integers(-27, 17, 3000)).astype(np.float32)
    h = rng.integers(0, 0x7BFF, 500).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)  # exact: 12 significant bits
    vals = np.concatenate([mags, -mags[:500], mids, -mids[:100],
                           np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    got = orc.round_f16(vals).astype(np.float64)
    for v, g in zip(vals, got):
        want = _rn_f16_exact(frac(v))
        assert g == want and math.copysign(1, g) == math.copysign(1, want), (v, g, want)


# --------------------------------------------------------------------------
# The layer: 26. ... Step 3 (forward), Step 4 tests; 22. ... Step 1 (grads)
# --------------------------------------------------------------------------
def _fixture_exact():
    g = _golden("ch26_step4_fixture.json")
    cbd = [Fraction(str(c)) for c in _golden("ch26_step4_codebook.json")["codebook"]]
    W = [[cbd[i] * Fraction(str(g["scale"])) for i in row] for row in g["indices"]]
    A = [[Fraction(str(v)) for v in row] for row in g["A"]]
    B = [[Fraction(str(v)) for v in row] for row in g["B"]]
    x = [[Fraction(str(v)) for v in row] for row in g["x"]]
    s = Fraction(str(g["alpha"])) / g["r"]
    return g, W, A, B, x, s


def _fixture_arrays(orc, g):
    cb = orc.codebook()
    w_hat = (cb[np.array(g["indices"])] * np.float32(g["scale"])).astype(np.float32)
    return (w_hat, np.float32(g["A"]), np.float32(g["B"]), np.float32(g["x"]))


def test_forward_fixture_exact(orc):
    g, W, A, B, x, s = _fixture_exact()
    w_hat, A32, B32, x32 = _fixture_arrays(orc, g)
    y, u = orc.linear_fwd(x32, w_hat, A32, B32, g["alpha"], g["r"])
    N, K, r = len(W), len(W[0]), g["r"]
    for m in range(len(x)):
        uu = [sum(x[m][k] * A[j][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            ref = sum(x[m][k] * W[n][k] for k in range(K)) + s * sum(uu[j] * B[n][j] for j in range(r))
            assert abs(y[m, n] - float(ref)) <= 1e-6
    # derived values: [[-0.26815, -0.30535, -0.3868], [0.27095, 1.04135, 1.7974]]
    np.testing.assert_allclose(y, [[-0.26815, -0.30535, -0.3868], [0.27095, 1.04135, 1.7974]],
                               atol=1e-6)
    # the LoRA branch changes the output (Step 4 test_lora_branch_contract)
    y0, _ = orc.linear_fwd(x32, w_hat, A32, np.zeros_like(B32), g["alpha"], g["r"])
    assert np.max(np.abs(y - y0)) > 1e-3


def test_backward_fixture_dy_ones(orc):
    """The pages' backward is layer(x).sum().backward(): dy = 1."""
    g, W, A, B, x, s = _fixture_exact()
    w_hat, A32, B32, x32 = _fixture_arrays(orc, g)
    dy = np.ones((2, 3), dtype=np.float32)
    dx, dA, dB = orc.linear_bwd(x32, w_hat, A32, B32, dy, g["alpha"], g["r"])
    N, K, r, M = len(W), len(W[0]), g["r"], len(x)
    u = [[sum(x[m][k] * A[j][k] for k in range(K)) for j in range(r)] for m in range(M)]
    gg = [[s * sum(B[n][j] for n in range(N)) for j in range(r)] for m in range(M)]
    for n in range(N):
        for j in range(r):
            assert abs(dB[n, j] - float(s * sum(u[m][j] for m in range(M)))) <= 1e-6
    for j in range(r):
        for k in range(K):
            assert abs(dA[j, k] - float(sum(gg[m][j] * x[m][k] for m in range(M)))) <= 1e-6
    for m in range(M):
        for k in range(K):
            ref = sum(W[n][k] for n in range(N)) + sum(gg[m][j] * A[j][k] for j in range(r))
            assert abs(dx[m, k] - float(ref)) <= 1e-6
    np.testing.assert_allclose(dx[0], [1.478, 2.360, 3.175, 3.9715], atol=1e-6)
    np.testing.assert_allclose(dB, [[0.72, 2.32]] * 3, atol=1e-6)
    np.testing.assert_allclose(dA, [[1.68, 1.12, -1.12, 1.12], [2.16, 1.44, -1.44, 1.44]], atol=1e-6)
    assert np.all(dx[0] == dx[1])


def _rand_layer(seed, M, N, K, r):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    A = (rng.standard_normal((r, K)) * 0.1).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.1).astype(np.float32)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    return x, w, A, B, dy


def test_backward_matches_autograd(orc):
    """The hand-derived backward equals torch autograd (fp64, CPU) of the
    forward loss sum(y * dy)."""
    x, w, A, B, dy = _rand_layer(1, 5, 7, 6, 3)
    alpha, r = 6.0, 3
    dx, dA, dB = orc.linear_bwd(x, w, A, B, dy, alpha, r)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    At = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    Bt = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64)
    y = xt @ wt.T + (alpha / r) * (xt @ At.T) @ Bt.T
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-12)
    # the sampled-row form gives the same rows
    dx_s, dA_s, dB_s = orc.linear_bwd(x, w, A, B, dy, alpha, r, rows=[4, 0])
    np.testing.assert_array_equal(dx_s, dx[[4, 0]])
    np.testing.assert_array_equal(dA_s, dA)


def test_forward_special_cases(orc):
    x, w, A, B, dy = _rand_layer(2, 6, 9, 128, 4)
    # B = 0: the layer is the plain product x W^T (a textbook GEMM)
    y, _ = orc.linear_fwd(x, w, A, np.zeros_like(B), 8.0, 4)
    np.testing.assert_allclose(y, x.astype(np.float64) @ w.T.astype(np.float64), rtol=1e-12, atol=1e-12)
    # y - y_base is linear in alpha
    y1, _ = orc.linear_fwd(x, w, A, B, 1.0, 4)
    y3, _ = orc.linear_fwd(x, w, A, B, 3.0, 4)
    np.testing.assert_allclose(y3 - y, 3 * (y1 - y), rtol=1e-10, atol=1e-12)


def test_backward_special_cases(orc):
    x, w, A, B, dy = _rand_layer(3, 6, 9, 16, 4)
    _, dA, _ = orc.linear_bwd(x, w, A, np.zeros_like(B), dy, 8.0, 4)
    assert np.all(dA == 0)  # B = 0 -> no gradient reaches A
    _, _, dB = orc.linear_bwd(x, w, np.zeros_like(A), B, dy, 8.0, 4)
    assert np.all(dB == 0)  # A = 0 -> no gradient reaches B
    dx, _, _ = orc.linear_bwd(x, w, A, np.zeros_like(B), dy, 8.0, 4)
    np.testing.assert_allclose(dx, dy.astype(np.float64) @ w.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_forward_brute_force_exact_small(orc):
    x, w, A, B, dy = _rand_layer(4, 3, 4, 8, 2)
    alpha, r = 16.0, 2
    y, u = orc.linear_fwd(x, w, A, B, alpha, r)
    s = Fraction(16, 2)
    for m in range(3):
        uu = [sum(frac(x[m, k]) * frac(A[j, k]) for k in range(8)) for j in range(r)]
        for j in range(r):
            assert abs(u[m, j] - float(uu[j])) <= 1e-14
        for n in range(4):
            ref = sum(frac(x[m, k]) * frac(w[n, k]) for k in range(8)) + s * sum(
                uu[j] * frac(B[n, j]) for j in range(r))
            assert abs(y[m, n] - float(ref)) <= 1e-13


# ---------------------------------------------------------------------------
# AdamW on the LoRA factors ([gc4] "显存计算实战" / "分页优化器": AdamW with
# fp32 moments, 8 bytes per trainable parameter; [L9] 9.4: two states each)
# ---------------------------------------------------------------------------
def test_adamw_first_step_closed_form(orc):
    """At t = 1 the bias-corrected moments are exactly g and g^2, so the
    step is p (1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(11)
    p = rng.standard_normal(4096).astype(np.float32)
    g = (rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 2, 4096)).astype(np.float32)
    g[:8] = 0.0
    lr, wd, eps = 2e-4, 0.01, 1e-8
    p1, m1, v1, _ = orc.adamw_step(p, g, np.zeros_like(p), np.zeros_like(p), lr, eps=eps,
                                   weight_decay=wd, step=1)
    ref = p.astype(np.float64) * (1 - lr * wd) - lr * g / (np.abs(g.astype(np.float64)) + eps)
    np.testing.assert_allclose(p1, ref, rtol=2e-6, atol=1e-9)
    assert np.all(p1[:8] == np.float32(p[:8] * np.float32(1 - lr * wd)))  # g = 0: decay only
    np.testing.assert_allclose(m1, 0.1 * g.astype(np.float64), rtol=2e-7, atol=0)
    np.testing.assert_allclose(v1, 0.001 * g.astype(np.float64) ** 2, rtol=4e-7, atol=0)


def test_adamw_matches_torch_over_steps(orc):
    """Five steps against torch.optim.AdamW (CPU, fp32, single-tensor path),
    an independent implementation of the same definition.  Each step starts
    both from torch's current state, so only that step's roundings differ."""
    rng = np.random.default_rng(12)
    n = 1000
    p0 = rng.standard_normal(n).astype(np.float32)
    grads = [rng.standard_normal(n).astype(np.float32) * (0.1 ** k) for k in range(5)]
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                            foreach=False)
    for t, g in enumerate(grads, start=1):
        st = opt.state.get(tp, {})
        p = tp.detach().numpy().copy()
        m = st["exp_avg"].numpy().copy() if st else np.zeros(n, np.float32)
        v = st["exp_avg_sq"].numpy().copy() if st else np.zeros(n, np.float32)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p1, m1, v1, _ = orc.adamw_step(p, g, m, v, 2e-4, step=t)
        st = opt.state[tp]
        # torch forms m + (1 - b1)(g - m) (a lerp), the definition b1 m + (1 - b1) g:
        # equal in exact arithmetic, so they differ by the terms' roundings
        terms = 0.9 * np.abs(m.astype(np.float64)) + 0.1 * np.abs(g.astype(np.float64))
        assert np.all(np.abs(m1 - st["exp_avg"].numpy()) <= 3e-7 * terms)
        np.testing.assert_allclose(v1, st["exp_avg_sq"].numpy(), rtol=4e-7, atol=0)
        np.testing.assert_allclose(p1, tp.detach().numpy(), rtol=3e-7, atol=0)


def test_adamw_special_cases(orc):
    rng = np.random.default_rng(13)
    p = rng.standard_normal(257).astype(np.float32)
    g = rng.standard_normal(257).astype(np.float32)
    m = rng.standard_normal(257).astype(np.float32)
    v = np.abs(rng.standard_normal(257)).astype(np.float32)
    # lr = 0: parameters unchanged, moments still advance
    p1, m1, v1, _ = orc.adamw_step(p, g, m, v, 0.0, step=3)
    assert np.array_equal(p1, p)
    assert not np.array_equal(m1, m) and not np.array_equal(v1, v)
    # zero moments and zero gradient: only the decoupled weight decay acts
    z = np.zeros_like(p)
    p2, m2, v2, _ = orc.adamw_step(p, z, z, z, 1e-3, weight_decay=0.1, step=7)
    assert np.array_equal(p2, p * np.float32(1 - 1e-3 * 0.1))
    assert np.all(m2 == 0) and np.all(v2 == 0)
    # the bf16 copy is the RNE of the new parameters
    p3, _, _, pb = orc.adamw_step(p, g, m, v, 2e-4, step=2, want_bf16=True)
    assert np.array_equal(pb, orc.round_bf16(p3))
    with pytest.raises(ValueError):
        orc.adamw_step(p, g, m, v, 2e-4, step=0)


# ---------------------------------------------------------------------------
# LoRA dropout: counter-based mask (Philox4x32-10) and the layer with it
# ---------------------------------------------------------------------------
def test_philox_known_answer_vectors(orc):
    """The oracle's Philox4x32-10 reproduces the generator's published
    known-answer vectors (tests/golden/philox4x32_10_kat.json)."""
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        out = orc.philox4x32_10([int(h, 16) for h in v["ctr"]], [int(h, 16) for h in v["key"]])
        assert [f"{w:08x}" for w in out] == v["out"]


def test_dropout_mask_layout_and_threshold(orc):
    """keep[m, k] is word (mK + k) % 4 of Philox at counter (mK + k) / 4 with
    the seed as key, compared with floor(p 2^32)."""
    M, K, p, seed = 3, 40, 0.3, 0x0123456789ABCDEF
    keep = orc.dropout_keep(M, K, p, seed)
    thr, scale = orc.dropout_params(p)
    assert thr == math.floor(0.3 * 2 ** 32) and scale == np.float32(1 / 0.7)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for e in (0, 1, 5, 39, 40, 77, M * K - 1):
        w = orc.philox4x32_10([e // 4, 0, 0, 0], key)[e % 4]
        assert keep.reshape(-1)[e] == (1 if w >= thr else 0)
    assert orc.dropout_keep(M, K, 0.0, seed).all()  # p = 0 keeps everything


@pytest.mark.parametrize("p", [0.05, 0.5])
def test_dropout_mask_statistics(orc, p):
    """Keep fraction within 6 sigma of 1 - p; neighbouring elements (same and
    different Philox words) uncorrelated; another seed gives another mask."""
    M, K = 256, 4096
    keep = orc.dropout_keep(M, K, p, 7).astype(np.float64)
    n = keep.size
    assert abs(keep.mean() - (1 - p)) <= 6 * math.sqrt(p * (1 - p) / n)
    flat = keep.reshape(-1) - keep.mean()
    for lag in (1, 4, K):
        corr = (flat[:-lag] * flat[lag:]).mean() / flat.var()
        assert abs(corr) < 6 / math.sqrt(n)
    other = orc.dropout_keep(M, K, p, 8)
    assert (other != keep).mean() > 0.5 * 2 * p * (1 - p)


def test_dropout_layer_matches_autograd(orc):
    """With dropout multipliers d on the bypass input, the oracle's forward
    equals y = x W^T + s ((d .* x) A^T) B^T and its backward equals torch
    autograd (fp64, CPU) of sum(y * dy): a missing mask in dA or dx, or a
    mask on the base path, fails here."""
    M, N, K, r, alpha = 5, 7, 12, 3, 6.0
    x, w, A, B, dy = _rand_layer(3, M, N, K, r)
    d = orc.dropout_mult(M, K, 0.4, 99)
    assert 0 < (d == 0).sum() < d.size
    y, u = orc.linear_fwd(x, w, A, B, alpha, r, drop=d)
    dx, dA, dB = orc.linear_bwd(x, w, A, B, dy, alpha, r, drop=d)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    At = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    Bt = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64)
    dt = torch.tensor(d)
    ut = (dt * xt) @ At.T
    yt = xt @ wt.T + (alpha / r) * ut @ Bt.T
    np.testing.assert_allclose(u, ut.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    (yt * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-12)
    # all-ones multipliers are the layer without dropout, bit for bit
    ones = np.ones((M, K))
    np.testing.assert_array_equal(orc.linear_fwd(x, w, A, B, alpha, r, drop=ones)[0],
                                  orc.linear_fwd(x, w, A, B, alpha, r)[0])
