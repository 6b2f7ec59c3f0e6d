"""CPU oracle for the 4-bit code-book and second-level-scale variants that the
pages compare NF4 with (TEST INFRASTRUCTURE ONLY, like the rest of this
package: only the tests, the smoke check and the benchmark's CPU-baseline and
study legs may import it).

Sources: the nlp-lineage milestone page on QLoRA, section "What it showed"
(NF4 with double quantization against a standard 4-bit float and 4-bit
integers, ranked by perplexity) and section "The idea" (NF4 bullet: equal
shares of a normal distribution; double-quantisation bullet: scales to 8
bits); the inferensys glossary entry "QLoRA" (NF4 against standard 4-bit
integers; scales to 8-bit floats).

Readings (the pages name the baselines but do not define them):
  * 4-bit float: OCP E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa
    bit, exponent 0 subnormal) -- magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 --
    scaled by absmax / 6, so the block's absmax maps to the largest value.
    Its 16 bit patterns hold 15 distinct values (+0 and -0).
  * 4-bit integer: symmetric absmax integers round(7 w / absmax) in -7..7,
    i.e. levels k / 7; 15 distinct values.
  * Both are held as 16-entry ascending tables so that the NF4 encoder and
    dequantizer run them unchanged: the 15 distinct values take codes 0..14
    (zero is code 7, as in NF4) and code 15 repeats +1, so the nearest-level
    rule (ties to the smaller code) never produces it.
  * Second-level variants: "full range" scales the group by max / 448 so the
    scale codes use the whole E4M3FN range instead of [0, 1]; "mean-centred"
    subtracts the group mean first and codes the signed differences over the
    full range: mu = fl32(tree sum / count) with the fp32 tree sum over the
    zero-padded group of 256 (pairs i, i + h for h = 128, 64, ..., 1),
    d = fl32(a - mu), c1 = fl32(max |d| / 448), c2 = signed E4M3FN code of
    fl32(d / c1), and s' = fl32(mu + fl32(dec(c2) c1)).
"""
from __future__ import annotations

import numpy as np

from .qlora_oracle import (BLOCK, GROUP, bf16_bits, e4m3fn_decode, fp32, nf4_levels,
                           unpack_codes)

CODEBOOKS = ("nf4", "fp4", "int4")
SCALE_MODES = ("absmax", "groupmax", "fullrange", "mean")   # fp32 per block, then the three DQ variants


def e2m1_values() -> np.ndarray:
    """All 16 OCP E2M1 bit patterns decoded (float64, in code order)."""
    out = []
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        v = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        out.append(-v if s else v)
    return np.array(out, dtype=np.float64)


def _table(distinct) -> np.ndarray:
    v = np.array(sorted(set(float(x) for x in distinct)), dtype=np.float64)
    assert v.size == 15 and v[0] == -1.0 and v[-1] == 1.0 and v[7] == 0.0
    return fp32(np.concatenate([v, [1.0]]))


def fp4_levels() -> np.ndarray:
    """E2M1 values / 6 as a 16-entry ascending fp32 table (code 15 repeats +1)."""
    return _table(e2m1_values() / 6.0)


def int4_levels() -> np.ndarray:
    """k / 7 for k = -7..7 as a 16-entry ascending fp32 table (code 15 repeats +1)."""
    return _table(np.arange(-7, 8) / 7.0)


def codebook_levels(name: str) -> np.ndarray:
    return {"nf4": nf4_levels, "fp4": fp4_levels, "int4": int4_levels}[name]()


def nearest_code(n, levels) -> np.ndarray:
    """Nearest level of each float32 n; ties (and repeated levels) -> smaller code:
    the number of midpoints (exact in float64) strictly below n."""
    q = np.asarray(levels, np.float32).astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2.0
    n = np.asarray(n, dtype=np.float32).astype(np.float64)
    return np.searchsorted(mids, n, side="left").astype(np.uint8)


def q4_quantize(W, levels):
    """Blockwise absmax quantization of W [rows, cols] to a 16-entry table:
    n = fl32(w / absmax) (0 for an all-zero block), code = nearest level.
    Returns packed codes [rows, cols // 2] (even element low nibble), absmax fp32."""
    W = np.asarray(W, dtype=np.float32)
    rows, cols = W.shape
    if cols % BLOCK or not np.all(np.isfinite(W)):
        raise ValueError("cols must be a multiple of 64 and weights finite")
    blocks = W.reshape(-1, BLOCK)
    absmax = np.max(np.abs(blocks), axis=1)
    safe = np.where(absmax == 0, np.float32(1), absmax)
    n = np.where(absmax[:, None] == 0, np.float32(0), blocks / safe[:, None])
    codes = nearest_code(n, levels).reshape(-1)
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8).reshape(rows, cols // 2), absmax.astype(np.float32)


# ----------------------------------------------------------------------------
# second-level scale variants
# ----------------------------------------------------------------------------

_E4M3_POS = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))        # codes 0..126 (0 .. 448), ascending


def e4m3fn_encode_signed(t) -> np.ndarray:
    """Nearest E4M3FN byte (sign bit + magnitude code) of finite t with |t| < 464
    (magnitudes past 448 are nearest to 448); ties to the even code."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    if np.any(~np.isfinite(t)) or np.any(a >= 464.0):
        raise ValueError("e4m3fn_encode_signed expects |t| < 464")
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, _E4M3_POS.size - 1)
    lo = np.clip(hi - 1, 0, _E4M3_POS.size - 1)
    d_lo, d_hi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    mag = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (mag | np.where(np.signbit(t) & (mag != 0), 0x80, 0)).astype(np.uint8)


def _groups(absmax):
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    ng = (a.size + GROUP - 1) // GROUP
    return a, ng


def double_quant_fullrange(absmax):
    """c1 = fl32(group max / 448); c2 = E4M3FN(fl32(a / c1)) (0 when c1 == 0)."""
    a, ng = _groups(absmax)
    c1 = np.zeros(ng, np.float32)
    c2 = np.zeros(a.size, np.uint8)
    for g in range(ng):
        seg = a[g * GROUP:(g + 1) * GROUP]
        c = np.float32(np.max(seg)) / np.float32(448.0)            # IEEE fp32 division
        c1[g] = c
        t = np.zeros_like(seg) if c == 0 else seg / c
        c2[g * GROUP:(g + 1) * GROUP] = e4m3fn_encode_signed(t)
    return c2, c1


def tree_sum_f32(seg) -> np.float32:
    """fp32 sum of a group zero-padded to 256 by halving: x[i] += x[i + h], h = 128 .. 1."""
    x = np.zeros(GROUP, np.float32)
    x[:len(seg)] = seg
    h = GROUP // 2
    while h >= 1:
        x[:h] = x[:h] + x[h:2 * h]                                  # fp32 adds
        h //= 2
    return x[0]


def double_quant_mean(absmax):
    """Mean-centred variant: returns c2 (signed E4M3FN), c1 and mu per group."""
    a, ng = _groups(absmax)
    c1 = np.zeros(ng, np.float32)
    mu = np.zeros(ng, np.float32)
    c2 = np.zeros(a.size, np.uint8)
    for g in range(ng):
        seg = a[g * GROUP:(g + 1) * GROUP]
        m = tree_sum_f32(seg) / np.float32(len(seg))                # IEEE fp32 division
        d = seg - m                                                 # fp32 subtraction
        c = np.float32(np.max(np.abs(d))) / np.float32(448.0)
        mu[g], c1[g] = m, c
        t = np.zeros_like(d) if c == 0 else d / c
        c2[g * GROUP:(g + 1) * GROUP] = e4m3fn_encode_signed(t)
    return c2, c1, mu


def double_quant(absmax, mode: str):
    """(c2, c1, mu) of a second-level mode; mu is None except for "mean"."""
    if mode == "groupmax":
        from .qlora_oracle import nf4_double_quant
        c2, c1 = nf4_double_quant(absmax)
        return c2, c1, None
    if mode == "fullrange":
        c2, c1 = double_quant_fullrange(absmax)
        return c2, c1, None
    if mode == "mean":
        return double_quant_mean(absmax)
    raise ValueError(mode)


def scales(mode: str, absmax=None, c2=None, c1=None, mu=None) -> np.ndarray:
    """Per-block fp32 scale used by the dequantizer:
    absmax: a; groupmax / fullrange: fl32(dec(c2) c1); mean: fl32(mu + fl32(dec(c2) c1))."""
    if mode == "absmax":
        return np.asarray(absmax, np.float32).reshape(-1)
    c2 = np.asarray(c2, np.uint8).reshape(-1)
    g = np.arange(c2.size) // GROUP
    p = fp32(e4m3fn_decode(c2) * np.asarray(c1, np.float32)[g].astype(np.float64))
    if mode == "mean":
        return fp32(np.asarray(mu, np.float32)[g].astype(np.float64) + p.astype(np.float64))
    return p


def q4_dequantize(codes, block_scale, levels, rows: int, cols: int) -> np.ndarray:
    """W' = bf16(fl32(q[code] * s_b)) as bf16 bits [rows, cols]."""
    c = unpack_codes(np.asarray(codes, np.uint8).reshape(rows, cols // 2)).reshape(-1, BLOCK)
    q = np.asarray(levels, np.float32).astype(np.float64)
    s = np.asarray(block_scale, np.float32).astype(np.float64)
    return bf16_bits(fp32(q[c] * s[:, None])).reshape(rows, cols)


def error_stats(W, Wd_bits, codes) -> dict:
    """Quantization error of one weight matrix: normalised MSE sum (W' - W)^2 / sum W^2,
    and the entropy (bits) of the code histogram."""
    from .qlora_oracle import bf16_value
    W = np.asarray(W, np.float64)
    e = bf16_value(Wd_bits) - W
    c = unpack_codes(np.asarray(codes, np.uint8)).reshape(-1)
    p = np.bincount(c, minlength=16) / c.size
    p = p[p > 0]
    return {"nmse": float(np.sum(e * e) / np.sum(W * W)), "code_entropy_bits": float(-np.sum(p * np.log2(p)))}
