"""Pins of the oracle's code-book and second-level-scale variants (the 4-bit
float and 4-bit integer baselines the pages rank NF4 against, and the
full-range and mean-centred scale codes) to facts outside the oracle:
the bit layout of E2M1, closed forms, exact rational brute force, exact sums
and a large-sample closed form of a uniform quantizer's error."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

V = O.variants


def brute_code(n, levels):
    fr = Fraction(float(n))
    best_k, best_d = None, None
    for k, q in enumerate(levels):
        d = abs(fr - Fraction(float(q)))
        if best_d is None or d < best_d:       # strict: ties and repeats keep the smaller code
            best_k, best_d = k, d
    return best_k


def test_e2m1_from_its_bit_layout():
    """E2M1: 2 exponent bits (bias 1), 1 mantissa bit, exponent 0 subnormal.
    Magnitudes: the subnormal step is half the smallest normal, each of the
    three binades holds two equally spaced values, the largest is 1.5 * 4."""
    v = V.e2m1_values()
    mags = np.unique(np.abs(v))
    assert mags.size == 8 and mags[0] == 0.0
    smallest_normal = 2.0 ** (1 - 1)
    assert mags[1] == smallest_normal / 2                     # subnormal 0.1b x 2^0
    for e in range(3):
        lo = smallest_normal * 2 ** e
        b = mags[(mags >= lo) & (mags < 2 * lo)]
        assert np.array_equal(b, [lo, 1.5 * lo])
    assert mags[-1] == 6.0
    assert np.array_equal(v[8:], -v[:8])                       # sign bit
    lv = V.fp4_levels()
    assert np.allclose(np.sort(np.unique(v)) / 6.0, lv[:15], rtol=2 ** -24, atol=0)
    assert lv[15] == lv[14] == 1.0 and lv[7] == 0.0


def test_int4_levels_closed_form():
    lv = V.int4_levels().astype(np.float64)
    assert np.array_equal(np.rint(lv[:15] * 7), np.arange(-7, 8))
    assert np.all(np.abs(lv[:15] * 7 - np.arange(-7, 8)) <= 8 * 2.0 ** -24)
    assert lv[15] == lv[14] == 1.0 and lv[7] == 0.0


@pytest.mark.parametrize("book", ["fp4", "int4", "nf4"])
def test_nearest_code_bruteforce(book):
    lv = V.codebook_levels(book)
    mids = (lv[:-1].astype(np.float64) + lv[1:]) / 2
    vals = []
    for m in mids:
        x = np.float32(m)
        for _ in range(2):
            x = np.nextafter(x, np.float32(-2))
        for _ in range(5):
            vals.append(x)
            x = np.nextafter(x, np.float32(2))
    vals += list(np.random.default_rng(4).uniform(-1, 1, 300).astype(np.float32))
    vals += [np.float32(1), np.float32(-1), np.float32(0), np.float32(-0.0)]
    vals = np.array([v for v in vals if -1 <= v <= 1], np.float32)
    got = V.nearest_code(vals, lv)
    ref = [brute_code(v, lv) for v in vals]
    assert np.array_equal(got, ref)
    assert 15 not in got or book == "nf4"


def test_nf4_through_the_generic_encoder_is_the_contract():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    W[3, :64] = 0
    c, a = V.q4_quantize(W, O.nf4_levels())
    c0, a0 = O.nf4_quantize(W)
    assert np.array_equal(c, c0) and np.array_equal(a, a0)
    c2, c1, _ = V.double_quant(a, "groupmax")
    s = V.scales("groupmax", None, c2, c1)
    assert np.array_equal(V.q4_dequantize(c, s, O.nf4_levels(), 8, 256), O.nf4_dequantize(c, c2, c1, 8, 256))


def _e4m3_all():
    vals = []
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        vals.append((c, -v if s else v))
    return vals


def test_signed_e4m3_encoder_bruteforce():
    allv = _e4m3_all()
    pos = sorted(set(v for _, v in allv if v >= 0))
    rng = np.random.default_rng(12)
    ts = list(rng.uniform(-463.9, 463.9, 300)) + list(rng.uniform(-1, 1, 200)) + [0.0, 448.0, -448.0, 463.0]
    ts += [float((pos[i] + pos[i + 1]) / 2) * s for i in range(len(pos) - 1) for s in (1, -1)]   # exact ties
    got = V.e4m3fn_encode_signed(np.array(ts))
    for t, c in zip(ts, got):
        ft = Fraction(t)
        best = min(allv, key=lambda cv: (abs(cv[1] - ft), cv[0] & 1, cv[0]))   # nearest, ties to even code
        if best[1] == 0:
            assert (c & 0x7F) == 0, t                           # +-0: either sign
        else:
            assert c == best[0], (t, c, best)


def test_tree_sum_exact_and_bounded():
    ints = np.arange(1, 257, dtype=np.float32) * np.float32(3)   # every partial sum an integer < 2^24
    assert V.tree_sum_f32(ints) == np.float32(3 * 256 * 257 // 2)
    assert V.tree_sum_f32(ints[:100]) == np.float32(3 * 100 * 101 // 2)
    x = np.abs(np.random.default_rng(1).standard_normal(256)).astype(np.float32)
    exact = math.fsum(float(v) for v in x)
    assert abs(float(V.tree_sum_f32(x)) - exact) <= 8 * 2.0 ** -24 * exact


def _absmax_like(n, seed):
    """Block absmax values of N(0, 0.02) weights: the max of 64 |normal|."""
    w = np.random.default_rng(seed).standard_normal((n, 64)) * 0.02
    return np.max(np.abs(w), axis=1).astype(np.float32)


def test_fullrange_scales():
    a = _absmax_like(700, 2)
    a[256:512] = 0                                               # one all-zero group
    c2, c1, _ = V.double_quant(a, "fullrange")
    s = V.scales("fullrange", None, c2, c1)
    assert c1[1] == 0 and np.all(s[256:512] == 0)
    for g in (0, 2):
        seg = slice(g * 256, min((g + 1) * 256, a.size))
        m = np.max(a[seg])
        assert c1[g] == np.float32(m) / np.float32(448)
        assert c2[seg][np.argmax(a[seg])] == 0x7E                # the group max takes the top code (448)
        assert np.all(np.abs(s[seg] - a[seg]) <= 2.0 ** -4 * a[seg] + 2.0 ** -20 * m)


def test_mean_centred_scales():
    a = _absmax_like(600, 3)
    c2, c1, mu = V.double_quant(a, "mean")
    s = V.scales("mean", None, c2, c1, mu)
    for g in range(3):
        seg = slice(g * 256, min((g + 1) * 256, a.size))
        exact = math.fsum(float(v) for v in a[seg]) / (seg.stop - seg.start)
        assert abs(float(mu[g]) - exact) <= 16 * 2.0 ** -24 * exact
        d = a[seg].astype(np.float64) - float(mu[g])
        assert np.all(np.abs(s[seg] - a[seg]) <= 2.0 ** -4 * np.max(np.abs(d)) + 2.0 ** -20 * float(mu[g]))
    # an exact case: differences -16, -8, 8, 16 from the mean 16 code as -448, -224,
    # 224, 448 and come back exactly
    b = np.array([0, 8, 24, 32] * 64, np.float32)
    c2, c1, mu = V.double_quant(b, "mean")
    assert mu[0] == 16 and c1[0] == np.float32(16) / np.float32(448)
    assert np.array_equal(c2[:4], [0xFE, 0xF6, 0x76, 0x7E])
    assert np.array_equal(V.scales("mean", None, c2, c1, mu)[:4], [0, 8, 24, 32])


def test_int4_uniform_error_closed_form():
    """Uniform weights in [-1, 1]: an absmax int4 quantizer has step 1/7 (times a
    block max close to 1), so MSE -> step^2 / 12 and the normalised MSE ->
    (1/588) / (1/3); the code histogram's entropy -> 13/14 log2 14 + 1/14 log2 28
    (13 interior bins of width 1/7 and two end bins of width 1/14)."""
    rng = np.random.default_rng(6)
    W = rng.uniform(-1, 1, (512, 1024)).astype(np.float32)
    codes, absmax = V.q4_quantize(W, V.int4_levels())
    Wd = V.q4_dequantize(codes, absmax, V.int4_levels(), 512, 1024)
    st = V.error_stats(W, Wd, codes)
    amax = float(np.mean(absmax.astype(np.float64) ** 2))       # E[a^2] rescales the step
    assert abs(st["nmse"] - amax * (1 / 588) / (1 / 3)) <= 0.03 * (1 / 588) / (1 / 3)
    h = 13 / 14 * math.log2(14) + 1 / 14 * math.log2(28)
    assert abs(st["code_entropy_bits"] - h) <= 0.02


def test_nf4_beats_fp4_beats_int4_on_normal_blocks():
    """The ranking the pages report (by perplexity) holds for the plain
    quantization error of N(0, 1) blocks, with NF4's codes the most evenly used."""
    W = np.random.default_rng(7).standard_normal((256, 1024)).astype(np.float32)
    res = {}
    for b in V.CODEBOOKS:
        lv = V.codebook_levels(b)
        c, a = V.q4_quantize(W, lv)
        res[b] = V.error_stats(W, V.q4_dequantize(c, a, lv, 256, 1024), c)
    assert res["nf4"]["nmse"] < res["fp4"]["nmse"] < res["int4"]["nmse"]
    assert res["nf4"]["code_entropy_bits"] > max(res["fp4"]["code_entropy_bits"], res["int4"]["code_entropy_bits"])
