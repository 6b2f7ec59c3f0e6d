"""Plain CPU oracle for the QLoRA hot path: NF4 encoding, double quantization,
double dequantization and the LoRA-augmented linear layer with its backward.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the GPU library is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does, and this
module imports nothing from the product.

Everything is NumPy on the CPU.  Floating point is float64 except where the
method itself fixes a narrower format, and every such rounding point is a
visible call (``fp32``, ``bf16_round``, ``e4m3fn_encode``).

Sources (web pages on QLoRA; cited by page and section):
  [lineage]   nlp-lineage milestone page on QLoRA (2023), section "The idea":
              the NF4 bullet, the double-quantisation bullet and the
              "notation" paragraph that states the layer formula.
  [tecyfy]    tecyfy.com concept page "What is QLoRA ...", section
              "The 3 tricks".
  [examadda]  tech.examadda.org "QLoRA (Quantized LoRA)", sections
              "The Core Idea", "The Three Innovations", "Practical Notes".
  [inferensys] inferensys.com glossary entry "QLoRA", the paragraphs on NF4,
              double quantization, the frozen base and the dequant kernel.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):
  * NF4 levels: the pages only say that the 16 values split a normal
    distribution into equal-probability shares and include an exact zero
    ([lineage] NF4 bullet); the level formula itself is not on the pages.
    Reading: quantiles evenly spaced in probability on each side of zero,
    8 positive levels (including +1) and 7 negative (including -1), with the
    outermost probability offset delta = 1 - (1/32 + 1/30)/2, normalised so
    the extreme levels are exactly -1 and +1; evaluated in float64 and
    rounded once to float32.  Code order ascending (code 7 is zero).
  * Blocks of 64 run along the flat row-major weight [N, K] (so along K).
  * Normalisation is a correctly rounded float32 division w / absmax; an
    all-zero block normalises to 0.
  * Nearest level: exact comparison with the midpoints of adjacent levels;
    an exact tie goes to the smaller code.
  * Packing: two codes per byte, the even element in the low nibble.
  * Second level ("8-bit floats", [inferensys] double-quantization paragraph;
    "to 8 bits", [lineage]): scales grouped by 256, c1 = group max in fp32,
    c2 = OCP FP8 E4M3FN code of fl32(scale / c1) rounded to nearest-even.
  * Dequant: s' = fl32(dec(c2) * c1); W' = bf16(fl32(q[c] * s')).
  * Layer: Y = bf16(X W'^T + s (T L2)) with T = bf16(X L1); backward
    G = bf16(s dY L2^T), dX = bf16(dY W' + G L1^T), dL1 = fp32(X^T G),
    dL2 = fp32(s T^T dY); the frozen base gets no gradient ([lineage]
    notation paragraph; [examadda] "The Flow").
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

BLOCK = 64          # weights per first-level block ([lineage] double-quantisation bullet)
GROUP = 256         # first-level scales per second-level group (reading: 8/64 + 32/(64*256) ~ 0.127 bit)


# ----------------------------------------------------------------------------
# Rounding helpers (the only places where precision is narrowed)
# ----------------------------------------------------------------------------

def fp32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round finite values (float32 or float64) to the nearest bfloat16,
    ties to even, returned as float64 holding the bf16 value.

    bfloat16 has 8 significant bits and the float32 exponent range, so the
    rounding quantum of x is 2**(e - 8) for x = m * 2**e with m in [0.5, 1),
    never finer than the subnormal quantum 2**-133.  Dividing by a power of
    two is exact, so np.rint (ties to even) does the rounding exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q_exp = np.maximum(e.astype(np.int64) - 8, -133)
    scale = np.ldexp(1.0, q_exp)
    r = np.rint(x / scale) * scale
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return r


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit pattern (uint16) of bf16_round(x)."""
    r = bf16_round(x).astype(np.float32)           # exact: r has <= 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# NF4 codebook  ([lineage] NF4 bullet; [tecyfy] "The 3 tricks"; [inferensys] NF4 paragraph)
# ----------------------------------------------------------------------------

def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in float64, ascending.

    Each side of zero takes quantiles of N(0, 1) at probabilities evenly
    spaced from 1/2 out to delta (8 points on the positive side, 7 on the
    negative), scaled by 1 / Phi^-1(delta) so the outermost levels are +-1;
    zero is added exactly.
    """
    inv = NormalDist().inv_cdf
    delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    top = inv(delta)
    positive = [inv(delta - j * (delta - 0.5) / 8.0) / top for j in range(8)]
    negative = [-inv(delta - j * (delta - 0.5) / 7.0) / top for j in range(7)]
    return np.array(sorted(negative + [0.0] + positive), dtype=np.float64)


def nf4_levels() -> np.ndarray:
    """The NF4 levels rounded once to float32 (code k -> levels[k])."""
    return fp32(nf4_levels_f64())


def nf4_midpoints(levels=None) -> np.ndarray:
    """Midpoints between adjacent float32 levels, exact in float64."""
    q = (nf4_levels() if levels is None else np.asarray(levels, np.float32)).astype(np.float64)
    return (q[:-1] + q[1:]) / 2.0


def nf4_nearest_code(n) -> np.ndarray:
    """Index of the level nearest to each float32 value n; ties -> smaller index.

    The code is the number of midpoints strictly below n: a value equal to a
    midpoint is not past it, so it keeps the smaller index.
    """
    n = np.asarray(n, dtype=np.float32).astype(np.float64)
    return np.searchsorted(nf4_midpoints(), n, side="left").astype(np.uint8)


# ----------------------------------------------------------------------------
# OCP FP8 E4M3FN codec (the 8-bit float of the second quantization level)
# ----------------------------------------------------------------------------

def e4m3fn_decode(codes) -> np.ndarray:
    """float64 value of E4M3FN bytes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2**-6); 0x7F/0xFF are NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


_E4M3_POS_VALUES = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))   # codes 0..126, ascending


def e4m3fn_encode(t) -> np.ndarray:
    """E4M3FN byte nearest to each finite t in [0, 448]; ties to the code with an
    even mantissa (even code).  Values and candidates are exact in float64."""
    t = np.asarray(t, dtype=np.float64)
    if np.any(~np.isfinite(t)) or np.any(t < 0) or np.any(t > 448.0):
        raise ValueError("e4m3fn_encode expects finite values in [0, 448]")
    vals = _E4M3_POS_VALUES
    hi = np.clip(np.searchsorted(vals, t, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = t - vals[lo]
    d_hi = vals[hi] - t
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.uint8)


# ----------------------------------------------------------------------------
# First level: blockwise absmax NF4  ([lineage] NF4 and double-quantisation bullets)
# ----------------------------------------------------------------------------

def nf4_quantize(W) -> tuple[np.ndarray, np.ndarray]:
    """Quantize a weight matrix [rows, cols] (float32 values; bf16 inputs are
    passed as their exact float32 values) to packed NF4 codes and fp32 absmax.

    Returns codes uint8 [rows, cols // 2] and absmax float32 [rows * cols // 64].
    """
    W = np.asarray(W, dtype=np.float32)
    rows, cols = W.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 64")
    if not np.all(np.isfinite(W)):
        raise ValueError("weights must be finite")
    blocks = W.reshape(-1, BLOCK)                                  # flat row-major blocks of 64
    absmax = np.max(np.abs(blocks), axis=1)                        # exact in fp32
    safe = np.where(absmax == 0, np.float32(1), absmax)
    n = np.where(absmax[:, None] == 0, np.float32(0), blocks / safe[:, None])   # IEEE fp32 division
    codes = nf4_nearest_code(n).reshape(-1)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)  # even element in the low nibble
    return packed.reshape(rows, cols // 2), absmax.astype(np.float32)


def unpack_codes(packed) -> np.ndarray:
    """Split packed bytes back into per-element codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------
# Second level: double quantization of the absmax scales
# ([lineage] double-quantisation bullet; [inferensys] double-quantization paragraph;
#  [tecyfy] "The 3 tricks"; [examadda] "The Three Innovations")
# ----------------------------------------------------------------------------

def nf4_double_quant(absmax) -> tuple[np.ndarray, np.ndarray]:
    """Quantize fp32 block scales to E4M3FN codes c2 (one per block) with one
    fp32 scale c1 per group of 256 blocks (the last group may be partial)."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    ng = (nb + GROUP - 1) // GROUP
    c1 = np.zeros(ng, dtype=np.float32)
    c2 = np.zeros(nb, dtype=np.uint8)
    for g in range(ng):
        seg = a[g * GROUP:(g + 1) * GROUP]
        m = np.max(seg)
        c1[g] = m
        if m == 0:
            t = np.zeros_like(seg)
        else:
            t = seg / m                                            # IEEE fp32 division
        c2[g * GROUP:(g + 1) * GROUP] = e4m3fn_encode(t)
    return c2, c1


def block_scales(c2, c1) -> np.ndarray:
    """Reconstructed first-level scales s'_b = fl32(dec(c2_b) * c1_g), float32."""
    c2 = np.asarray(c2, dtype=np.uint8).reshape(-1)
    c1 = np.asarray(c1, dtype=np.float32).reshape(-1)
    g = np.arange(c2.size) // GROUP
    return fp32(e4m3fn_decode(c2) * c1[g].astype(np.float64))     # product exact in float64


def dequantize_blocks(block_codes, c2_b, c1_b) -> np.ndarray:
    """Dequantize a set of blocks: block_codes [nb, 64] unpacked codes, with each
    block's own c2 byte and c1 group scale.  Returns bf16 bits [nb, 64]:
    s'_b = fl32(dec(c2_b) * c1_b); W'_e = bf16(fl32(q[code_e] * s'_b))."""
    q = nf4_levels().astype(np.float64)
    d = e4m3fn_decode(np.asarray(c2_b, dtype=np.uint8).reshape(-1))
    s = fp32(d * np.asarray(c1_b, dtype=np.float32).reshape(-1).astype(np.float64)).astype(np.float64)
    w = fp32(q[np.asarray(block_codes)] * s[:, None])                # exact product, one fp32 rounding
    return bf16_bits(w)


def nf4_dequantize(codes, c2, c1, rows: int, cols: int) -> np.ndarray:
    """doubleDequant(c1, c2, W_NF4) as bf16 bit patterns [rows, cols]."""
    c = unpack_codes(np.asarray(codes, dtype=np.uint8).reshape(rows, cols // 2)).reshape(-1, BLOCK)
    c2 = np.asarray(c2, dtype=np.uint8).reshape(-1)
    c1 = np.asarray(c1, dtype=np.float32).reshape(-1)
    return dequantize_blocks(c, c2, c1[np.arange(c2.size) // GROUP]).reshape(rows, cols)


# ----------------------------------------------------------------------------
# The layer  ([lineage] notation paragraph: Y = X doubleDequant(c1, c2, W_NF4) + X L1 L2;
#             [examadda] "Practical Notes": bf16 compute)
# ----------------------------------------------------------------------------

def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_value(a)
    return a.astype(np.float64)


def qlora_forward(X, Wq, L1, L2, lora_scale: float = 1.0, rnd=bf16_bits):
    """Forward of one quantized LoRA linear.

    X [M, K] bf16 bits, Wq = dequantized weight [N, K] bf16 bits (stored out x in),
    L1 [K, r] and L2 [r, N] bf16 bits.  Returns (Y [M, N], T [M, r]) as rnd(...)
    of the float64 results: T = rnd(X L1); Y = rnd(X Wq^T + s (T L2)).
    """
    Xf, Wf, L1f, L2f = _f64(X), _f64(Wq), _f64(L1), _f64(L2)
    T = rnd(Xf @ L1f)
    Y = rnd(Xf @ Wf.T + lora_scale * (_f64(T) @ L2f))
    return Y, T


def qlora_backward(X, dY, Wq, L1, L2, lora_scale: float = 1.0, T=None, rnd=bf16_bits, compute_dx=True):
    """Backward of the quantized LoRA linear; the frozen base gets no gradient.

    Returns (dX [M, K], dL1 [K, r] fp32, dL2 [r, N] fp32, G [M, r], T [M, r]) with
      G = rnd(s dY L2^T), dX = rnd(dY Wq + G L1^T),
      dL1 = fp32(X^T G), dL2 = fp32(s T^T dY), T = rnd(X L1) when not given.
    With compute_dx=False, dX is None and Wq is not used (as when the caller
    passes no dX buffer).  Columns of dX/dL1 can be restricted by passing the
    matching columns of X, Wq and rows of L1 together with the full T.
    """
    Xf, dYf, L1f, L2f = _f64(X), _f64(dY), _f64(L1), _f64(L2)
    if T is None:
        T = rnd(Xf @ L1f)
    G = rnd(lora_scale * (dYf @ L2f.T))
    Gf = _f64(G)
    dX = rnd(dYf @ _f64(Wq) + Gf @ L1f.T) if compute_dx else None
    dL1 = fp32(Xf.T @ Gf)
    dL2 = fp32(lora_scale * (_f64(T).T @ dYf))
    return dX, dL1, dL2, G, T


def qlora_merge(codes, c2, c1, rows: int, cols: int, L1, L2, lora_scale: float = 1.0) -> np.ndarray:
    """Adapter merged into a bf16 copy of the base, for export after training:
    W_m = bf16(W' + s (L1 L2)^T), [rows = N, cols = K] bf16 bits.

    [examadda] "Practical Notes": merging an adapter into the 4-bit base is
    lossy, so the base is dequantised first.  The layer's output with the
    merged weight is X W_m^T = X W'^T + s X L1 L2 up to the one bf16 rounding of
    W_m ([lineage] notation paragraph).  W' is exact (nf4_dequantize), the
    low-rank term is float64, and the sum is rounded once."""
    Wd = bf16_value(nf4_dequantize(codes, c2, c1, rows, cols)).astype(np.float64)
    low = _f64(L1) @ _f64(L2)                       # [K, N]
    return bf16_bits(Wd + lora_scale * low.T)


def bits_per_weight(rows: int, cols: int) -> float:
    """Storage of the quantized base in bits per weight, from the buffer sizes
    that nf4_quantize / nf4_double_quant produce."""
    e = rows * cols
    nb = e // BLOCK
    ng = (nb + GROUP - 1) // GROUP
    codes_bytes = e // 2
    c2_bytes = nb
    c1_bytes = 4 * ng
    return 8.0 * (codes_bytes + c2_bytes + c1_bytes) / e
