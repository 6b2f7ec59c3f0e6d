"""Pins of the CPU oracle to facts that do not come from the oracle itself:
the pages' stated figures (tests/golden), closed forms, library routines used as
independent references (torch CPU casts, an independent inverse normal CDF),
exact rational brute force on tiny inputs, and finite differences.

Mutation checks at the end plant plausible mistakes in a copy of the oracle's
steps (on the CPU) and confirm that a pin catches each of them.
"""
import math
import os
from fractions import Fraction
from statistics import NormalDist

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split(";")[0].strip()
            if not line or line.startswith("#"):
                continue
            k, v = [s.strip() for s in line.split("=")]
            vals[k] = float(v)
    return vals


# --------------------------------------------------------------------------
# independent helpers (test-local; share nothing with the oracle's arithmetic)
# --------------------------------------------------------------------------

def inv_norm_bisect(p):
    """Phi^-1(p) by bisection on the complementary error function."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 0:
            break
    return 0.5 * (lo + hi)


def f32_of_fraction(fr):
    """Exactly rounded (ties-to-even) float32 of a rational."""
    x = np.float32(float(fr))
    best = None
    for c in (np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def brute_code_exact(n, levels):
    fr = Fraction(float(n))
    best_k, best_d = None, None
    for k, q in enumerate(levels):
        d = abs(fr - Fraction(float(q)))
        if best_d is None or d < best_d:        # strict: ties keep the smaller index
            best_k, best_d = k, d
    return best_k


def torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x32, np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# codebook
# --------------------------------------------------------------------------

def test_codebook_structure():
    q = O.nf4_levels()
    g = golden("accounting.txt")
    assert q.dtype == np.float32 and q.size == int(g["levels"])
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    assert q[0] == -1.0 and q[15] == 1.0 and q[7] == 0.0
    assert np.sum(q < 0) == 7 and np.sum(q > 0) == 8


def test_codebook_equal_probability_steps():
    """Each side's levels sit at N(0,1) quantiles evenly spaced in probability."""
    nd = NormalDist()
    qf = O.nf4_levels_f64()
    delta = 1.0 - 0.5 * (1 / 32 + 1 / 30)
    top = nd.inv_cdf(delta)
    pos = [nd.cdf(v * top) for v in qf[7:]]         # 0, q8..q15
    neg = [nd.cdf(-v * top) for v in qf[:8][::-1]]  # 0, -q6..-q0
    assert np.allclose(np.diff(pos), (delta - 0.5) / 8, atol=1e-12, rtol=0)
    assert np.allclose(np.diff(neg), (delta - 0.5) / 7, atol=1e-12, rtol=0)


def test_codebook_independent_inverse_cdf():
    """Levels from a bisection inverse CDF agree bitwise after fp32 rounding."""
    delta = 1.0 - 0.5 * (1 / 32 + 1 / 30)
    top = inv_norm_bisect(delta)
    pos = [inv_norm_bisect(delta - j * (delta - 0.5) / 8) / top for j in range(8)]
    neg = [-inv_norm_bisect(delta - j * (delta - 0.5) / 7) / top for j in range(7)]
    ref = np.array(sorted(neg + [0.0] + pos), dtype=np.float64).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), O.nf4_levels().view(np.uint32))
    from scipy.special import ndtri
    top = ndtri(delta)
    pos = [ndtri(delta - j * (delta - 0.5) / 8) / top for j in range(8)]
    neg = [-ndtri(delta - j * (delta - 0.5) / 7) / top for j in range(7)]
    ref2 = np.array(sorted(neg + [0.0] + pos), dtype=np.float64).astype(np.float32)
    assert np.array_equal(ref2.view(np.uint32), O.nf4_levels().view(np.uint32))


# --------------------------------------------------------------------------
# nearest-level rule and the encoder
# --------------------------------------------------------------------------

def _probe_values():
    q = O.nf4_levels()
    mids = O.nf4_midpoints()
    vals = []
    for v in list(q) + [np.float32(m) for m in mids]:
        x = np.float32(v)
        for _ in range(3):
            x = np.nextafter(x, np.float32(-np.inf))
        for _ in range(7):
            vals.append(x)
            x = np.nextafter(x, np.float32(np.inf))
    # midpoints that are not fp32-representable: both neighbours
    for m in mids:
        lo = np.float32(m)
        if float(lo) > m:
            lo = np.nextafter(lo, np.float32(-np.inf))
        vals += [lo, np.nextafter(lo, np.float32(np.inf))]
    rng = np.random.default_rng(5)
    vals += list(rng.uniform(-1, 1, 400).astype(np.float32))
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(1e-30), np.float32(-1e-30)]
    return np.array([v for v in vals if -1 <= v <= 1], dtype=np.float32)


def test_nearest_code_bruteforce():
    q = O.nf4_levels()
    vals = _probe_values()
    got = O.nf4_nearest_code(vals)
    ref = np.array([brute_code_exact(v, q) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_exact_ties_go_to_smaller_code():
    q = O.nf4_levels().astype(np.float64)
    ties = 0
    for k in range(15):
        m = (q[k] + q[k + 1]) / 2
        if float(np.float32(m)) == m:
            ties += 1
            assert O.nf4_nearest_code(np.float32(m)) == k
    assert ties >= 1


def test_quantize_bruteforce_tiny():
    """Codes and absmax of small matrices against exact rational arithmetic."""
    rng = np.random.default_rng(11)
    q = O.nf4_levels()
    W = (rng.standard_normal((3, 128)) * 0.02).astype(np.float32)
    W[1, 64:128] = 0.0                                   # all-zero block
    W[2, 5] = -4 * np.abs(W[2, :64]).max()               # negative absmax
    codes, absmax = O.nf4_quantize(W)
    blocks = W.reshape(-1, 64)
    for b in range(blocks.shape[0]):
        a = max(abs(Fraction(float(x))) for x in blocks[b])
        assert Fraction(float(absmax[b])) == a
        for j in range(64):
            w = blocks[b, j]
            n = np.float32(0) if a == 0 else f32_of_fraction(Fraction(float(w)) / a)
            code = brute_code_exact(n, q)
            e = b * 64 + j
            byte = codes.reshape(-1)[e // 2]
            got = (byte >> 4) if (e % 2) else (byte & 0xF)
            assert got == code, (b, j)


def test_division_adversarial_near_midpoints():
    """w placed +-1 ulp around midpoint * a: the fp32 division decides the code."""
    rng = np.random.default_rng(3)
    q = O.nf4_levels()
    mids = O.nf4_midpoints()
    for a in rng.uniform(0.005, 0.3, 12).astype(np.float32):
        row = np.zeros(64, np.float32)
        row[0] = a
        vals = []
        for m in mids:
            x = np.float32(m * float(a))
            for d in (-2, -1, 0, 1, 2):
                y = x
                for _ in range(abs(d)):
                    y = np.nextafter(y, np.float32(np.inf if d > 0 else -np.inf))
                vals.append(y)
        vals = [v for v in vals if abs(v) <= a][:63]
        row[1:1 + len(vals)] = vals
        codes, absmax = O.nf4_quantize(row[None, :])
        c = O.unpack_codes(codes).reshape(-1)
        for j in range(64):
            n = f32_of_fraction(Fraction(float(row[j])) / Fraction(float(a)))
            assert c[j] == brute_code_exact(n, q)


def test_roundtrip_codebook_values():
    """A block made of q_k * 2^e with absmax 2^e encodes to exactly k, and with a
    single-block group the scale and dequantized values come back exactly."""
    q = O.nf4_levels()
    for e in (-7, -3, 0, 2):
        row = np.array([q[i % 16] * 2.0 ** e for i in range(64)], dtype=np.float32)
        codes, absmax = O.nf4_quantize(row[None, :])
        assert absmax[0] == np.float32(2.0 ** e)
        assert np.array_equal(O.unpack_codes(codes).reshape(-1), np.arange(64) % 16)
        c2, c1 = O.nf4_double_quant(absmax)
        assert c2[0] == 0x38 and c1[0] == absmax[0]
        wq = O.nf4_dequantize(codes, c2, c1, 1, 64)
        assert np.array_equal(wq.reshape(-1), torch_bf16_bits(row))


def test_packing_low_nibble_first():
    q = O.nf4_levels()
    row = np.array([q[(3 * i) % 16] for i in range(64)], dtype=np.float32)
    codes, _ = O.nf4_quantize(row[None, :])
    assert codes[0, 0] == (0 | (3 << 4))
    assert codes[0, 1] == (6 | (9 << 4))


# --------------------------------------------------------------------------
# E4M3FN codec and double quantization
# --------------------------------------------------------------------------

def test_e4m3fn_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert O.e4m3fn_decode(np.uint8(0x38)) == 1.0
    assert O.e4m3fn_decode(np.uint8(0x7E)) == 448.0
    assert O.e4m3fn_decode(np.uint8(0x01)) == 2.0 ** -9


def test_e4m3fn_encode_matches_torch_cast():
    """RNE encoding of fp32 t in [0, 1]: a strided sweep of every fp32 bit
    pattern plus +-4 ulps around every value and midpoint of the format."""
    one = np.float32(1.0).view(np.uint32)
    sweep = np.arange(0, int(one) + 1, 4099, dtype=np.uint32).view(np.float32)
    vals = O.e4m3fn_decode(np.arange(0x39, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    near = []
    for v in np.concatenate([vals, mids]):
        x = np.float32(v)
        for d in range(-4, 5):
            y = x.view(np.uint32).astype(np.int64) + d
            if 0 <= y <= int(one):
                near.append(np.uint32(y))
    t = np.concatenate([sweep, np.array(near, np.uint32).view(np.float32)])
    ref = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3fn_encode(t)
    assert np.array_equal(got, ref)


def test_double_quant_invariants():
    rng = np.random.default_rng(2)
    a = np.abs(rng.standard_normal(256 * 3 + 17)).astype(np.float32) * 0.05
    a[600] = 0.0
    c2, c1 = O.nf4_double_quant(a)
    assert c1.size == 4 and c2.size == a.size
    for g in range(4):
        seg = a[g * 256:(g + 1) * 256]
        assert c1[g] == seg.max()
        assert c2[g * 256 + int(np.argmax(seg))] == 0x38
    s = O.block_scales(c2, c1).astype(np.float64)
    ratio = a / np.repeat(c1, 256)[:a.size]
    ok = ratio >= 2.0 ** -6
    assert np.all(np.abs(s[ok] - a[ok]) / a[ok] <= 2.0 ** -4)
    order = np.argsort(a[:256], kind="stable")
    assert np.all(np.diff(c2[:256][order].astype(int)) >= 0)
    z, zc1 = O.nf4_double_quant(np.zeros(300, np.float32))
    assert np.all(z == 0) and np.all(zc1 == 0)


def test_dequant_matches_library_products():
    """W' = bf16(fl32(q[c] * s')) with the products and roundings done by torch."""
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    codes, absmax = O.nf4_quantize(W)
    c2, c1 = O.nf4_double_quant(absmax)
    got = O.nf4_dequantize(codes, c2, c1, 4, 256)
    c = torch.from_numpy(O.unpack_codes(codes).reshape(-1).astype(np.int64))
    q = torch.from_numpy(O.nf4_levels())
    d = torch.from_numpy(c2).view(torch.float8_e4m3fn).to(torch.float32)
    s = d * torch.from_numpy(c1).repeat_interleave(256)[:d.numel()]
    w = q[c] * s.repeat_interleave(64)
    ref = w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(4, 256)
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(20000).astype(np.float32)
    u = x.view(np.uint32).copy()
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000                    # exact ties
    x = u.view(np.float32)
    assert np.array_equal(O.bf16_bits(x), torch_bf16_bits(x))
    tiny = np.array([1e-39, -3e-40, 2.0 ** -133, 3 * 2.0 ** -134], np.float32)
    assert np.array_equal(O.bf16_bits(tiny), torch_bf16_bits(tiny))


def test_bf16_rounding_from_float64_exact():
    """Single rounding from float64: compare with exact rational rounding."""
    rng = np.random.default_rng(8)
    xs = rng.standard_normal(300) * 10.0 ** rng.integers(-5, 5, 300)
    for x in xs:
        fr = Fraction(float(x))
        r = float(O.bf16_round(np.float64(x)))
        m, e = math.frexp(abs(x))
        quantum = Fraction(2) ** (e - 8)
        k = fr / quantum
        fl = math.floor(k)
        rem = k - fl
        n = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1) else 0)
        assert Fraction(r) == n * quantum


# --------------------------------------------------------------------------
# storage accounting against the pages' figures
# --------------------------------------------------------------------------

def test_accounting_matches_pages():
    g = golden("accounting.txt")
    bpw = O.bits_per_weight(8192, 8192)
    assert bpw == 4 + 8 / 64 + 32 / (64 * 256)
    overhead = bpw - 4
    assert g["first_level_scale_bits"] / g["first_level_block"] == g["overhead_before_dq_bits"]
    assert abs(overhead - g["overhead_after_dq_bits"]) < 5e-4
    saving = g["overhead_before_dq_bits"] - overhead
    assert abs(saving - g["dq_saving_bits"]) < 5e-3
    assert abs(saving * g["model_params_65b"] / 8 / 1e9 - g["dq_saving_gb_65b"]) < 0.1
    assert 16 / 4 == g["compression_16_to_4"]
    codes, absmax = O.nf4_quantize(np.zeros((4, 16384), np.float32))
    c2, c1 = O.nf4_double_quant(absmax)
    e = 4 * 16384
    assert 8 * (codes.nbytes + c2.nbytes + c1.nbytes) / e == O.bits_per_weight(4, 16384)


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

def _layer(M=6, K=128, N=64, r=4, seed=0, wstd=0.02, l2std=0.5):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * wstd).astype(np.float32)
    codes, absmax = O.nf4_quantize(W)
    c2, c1 = O.nf4_double_quant(absmax)
    Wq = O.nf4_dequantize(codes, c2, c1, N, K)
    b = lambda a: O.bf16_bits(a)
    X = b(rng.standard_normal((M, K)))
    L1 = b(rng.standard_normal((K, r)) / K)
    L2 = b(rng.standard_normal((r, N)) * l2std)
    dY = b(rng.standard_normal((M, N)))
    return X, Wq, L1, L2, dY


def test_forward_and_backward_vs_torch_autograd():
    ident = lambda a: np.asarray(a, np.float64)
    X, Wq, L1, L2, dY = _layer()
    s = 0.75
    Y, T = O.qlora_forward(X, Wq, L1, L2, s, rnd=ident)
    dX, dL1, dL2, G, _ = O.qlora_backward(X, dY, Wq, L1, L2, s, rnd=ident)
    tX = torch.tensor(O.bf16_value(X), requires_grad=True)
    tW = torch.tensor(O.bf16_value(Wq))
    tL1 = torch.tensor(O.bf16_value(L1), requires_grad=True)
    tL2 = torch.tensor(O.bf16_value(L2), requires_grad=True)
    out = tX @ tW.T + s * (tX @ tL1) @ tL2
    assert np.allclose(Y, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    out.backward(torch.tensor(O.bf16_value(dY)))
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dL1, tL1.grad.numpy(), rtol=1e-6, atol=1e-9)
    assert np.allclose(dL2, tL2.grad.numpy(), rtol=1e-6, atol=1e-9)


def test_backward_vs_finite_differences():
    ident = lambda a: np.asarray(a, np.float64)
    X, Wq, L1, L2, dY = _layer(M=3, K=64, N=8, r=2, seed=1)
    Xf, L1f, L2f = O.bf16_value(X), O.bf16_value(L1), O.bf16_value(L2)
    dYf = O.bf16_value(dY)
    s = 1.3

    def loss(Xv, L1v, L2v):
        Y, _ = O.qlora_forward(Xv, Wq, L1v, L2v, s, rnd=ident)
        return float(np.sum(Y * dYf))

    dX, dL1, dL2, _, _ = O.qlora_backward(X, dY, Wq, L1, L2, s, rnd=ident)
    h = 1e-6
    for (arr, grad, idxs) in ((Xf, dX, [(0, 0), (2, 63), (1, 17)]),
                              (L1f, dL1, [(0, 0), (63, 1), (5, 1)]),
                              (L2f, dL2, [(0, 0), (1, 7), (1, 3)])):
        for ij in idxs:
            p = arr.copy(); p[ij] += h
            m = arr.copy(); m[ij] -= h
            args_p = [Xf, L1f, L2f]; args_m = [Xf, L1f, L2f]
            k = [id(Xf), id(L1f), id(L2f)].index(id(arr))
            args_p[k] = p; args_m[k] = m
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - float(grad[ij])) <= 1e-6 * max(1.0, abs(fd)), (k, ij)


def test_special_cases_reduce_to_library_gemm():
    X, Wq, L1, L2, dY = _layer(M=5, K=64, N=32, r=4, seed=2)
    zero_l2 = np.zeros_like(L2)
    Y, _ = O.qlora_forward(X, Wq, L1, zero_l2, 1.0)
    ref = torch.tensor(O.bf16_value(X)) @ torch.tensor(O.bf16_value(Wq)).T
    assert np.array_equal(Y, ref.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    # identity input exposes W'^T plus the LoRA term row by row
    K = 64
    I = O.bf16_bits(np.eye(K))
    Yi, Ti = O.qlora_forward(I, Wq, L1, L2, 1.0)
    exp = O.bf16_bits(O.bf16_value(Wq).T + O.bf16_value(Ti) @ O.bf16_value(L2))
    assert np.array_equal(Yi, exp)
    assert np.array_equal(Ti, L1)
    # zero upstream gradient gives exactly zero gradients
    dX, dL1, dL2, G, _ = O.qlora_backward(X, np.zeros_like(dY), Wq, L1, L2, 1.0)
    assert not np.any(O.bf16_value(dX)) and not np.any(dL1) and not np.any(dL2) and not np.any(O.bf16_value(G))


def _quantized(N, K, seed, wstd=0.02):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * wstd).astype(np.float32)
    codes, absmax = O.nf4_quantize(W)
    c2, c1 = O.nf4_double_quant(absmax)
    return codes, c2, c1


def test_merge_zero_adapter_is_the_dequantized_base():
    """qlora_merge with L2 = 0 is exactly W' (the sum adds +0 before one
    rounding of an already-bf16 value)."""
    N, K, r = 48, 128, 4
    codes, c2, c1 = _quantized(N, K, 31)
    rng = np.random.default_rng(32)
    L1 = O.bf16_bits(rng.standard_normal((K, r)))
    Wm = O.qlora_merge(codes, c2, c1, N, K, L1, np.zeros((r, N), np.uint16), 0.75)
    assert np.array_equal(Wm, O.nf4_dequantize(codes, c2, c1, N, K))


def test_merge_zero_base_is_the_library_product():
    """An all-zero weight quantizes to W' = 0, so the merge is bf16(s L2^T L1^T),
    here from torch's float64 matmul."""
    N, K, r, s = 40, 192, 8, 1.5
    codes, absmax = O.nf4_quantize(np.zeros((N, K), np.float32))
    c2, c1 = O.nf4_double_quant(absmax)
    rng = np.random.default_rng(33)
    L1 = O.bf16_bits(rng.standard_normal((K, r)))
    L2 = O.bf16_bits(rng.standard_normal((r, N)))
    Wm = O.qlora_merge(codes, c2, c1, N, K, L1, L2, s)
    ref = s * (torch.tensor(O.bf16_value(L2)).T @ torch.tensor(O.bf16_value(L1)).T)
    assert np.array_equal(Wm, ref.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def _merge_identity_err(Wm_bits, codes, c2, c1, N, K, L1, L2, s, X):
    Wq = O.nf4_dequantize(codes, c2, c1, N, K)
    Xf = O.bf16_value(X)
    exact = Xf @ O.bf16_value(Wq).T + s * (Xf @ O.bf16_value(L1)) @ O.bf16_value(L2)
    merged = Xf @ O.bf16_value(Wm_bits).T
    return np.linalg.norm(merged - exact) / np.linalg.norm(exact)


def test_merge_layer_identity():
    """The layer with the merged weight, X W_m^T, reproduces X W'^T + s X L1 L2
    up to the one bf16 rounding of W_m (relative error about 2^-9); the adapter
    applied untransposed (square case) is caught."""
    N = K = 128
    r, s = 8, 1.0
    codes, c2, c1 = _quantized(N, K, 34)
    rng = np.random.default_rng(35)
    L1 = O.bf16_bits(rng.standard_normal((K, r)) * 0.05)
    L2 = O.bf16_bits(rng.standard_normal((r, N)) * 0.05)
    X = O.bf16_bits(rng.standard_normal((16, K)))
    Wm = O.qlora_merge(codes, c2, c1, N, K, L1, L2, s)
    assert _merge_identity_err(Wm, codes, c2, c1, N, K, L1, L2, s, X) < 2.0 ** -8
    Wq = O.bf16_value(O.nf4_dequantize(codes, c2, c1, N, K))
    wrong = O.bf16_bits(Wq + s * (O.bf16_value(L1) @ O.bf16_value(L2)))      # (L1 L2) not transposed
    assert _merge_identity_err(wrong, codes, c2, c1, N, K, L1, L2, s, X) > 1e-2


def test_rounding_points():
    """T, Y, G and dX are bf16-rounded once; dL1/dL2 are fp32."""
    X, Wq, L1, L2, dY = _layer(seed=7)
    Y, T = O.qlora_forward(X, Wq, L1, L2, 1.0)
    assert Y.dtype == np.uint16 and T.dtype == np.uint16
    dX, dL1, dL2, G, T2 = O.qlora_backward(X, dY, Wq, L1, L2, 1.0)
    assert dX.dtype == np.uint16 and G.dtype == np.uint16
    assert dL1.dtype == np.float32 and dL2.dtype == np.float32
    assert np.array_equal(T, T2)


# --------------------------------------------------------------------------
# mutation checks: plausible mistakes planted in copies of oracle steps
# --------------------------------------------------------------------------

def test_mutation_tie_to_larger_code_is_caught():
    q = O.nf4_levels()
    mids = O.nf4_midpoints()
    wrong = lambda n: np.searchsorted(mids, np.asarray(n, np.float64), side="right").astype(np.uint8)
    vals = _probe_values()
    ref = np.array([brute_code_exact(v, q) for v in vals], dtype=np.uint8)
    assert not np.array_equal(wrong(vals), ref)


def test_mutation_swapped_nibbles_is_caught():
    q = O.nf4_levels()
    row = np.array([q[(3 * i) % 16] for i in range(64)], dtype=np.float32)
    c = O.nf4_nearest_code(row / np.abs(row).max())
    swapped = (c[1::2] | (c[0::2] << 4)).astype(np.uint8)
    assert swapped[0] != (0 | (3 << 4))


def test_mutation_dropped_lora_term_in_dx_is_caught():
    ident = lambda a: np.asarray(a, np.float64)
    X, Wq, L1, L2, dY = _layer(l2std=2.0)
    tX = torch.tensor(O.bf16_value(X), requires_grad=True)
    out = tX @ torch.tensor(O.bf16_value(Wq)).T + (tX @ torch.tensor(O.bf16_value(L1))) @ torch.tensor(O.bf16_value(L2))
    out.backward(torch.tensor(O.bf16_value(dY)))
    wrong_dx = O.bf16_value(dY) @ O.bf16_value(Wq)          # the G L1^T term dropped
    assert not np.allclose(wrong_dx, tX.grad.numpy(), rtol=1e-6, atol=1e-9)


def test_mutation_wrong_delta_is_caught():
    nd = NormalDist()
    delta = 1.0 - 1 / 32                                     # one-sided offset instead of the average
    top = nd.inv_cdf(delta)
    pos = [nd.inv_cdf(delta - j * (delta - 0.5) / 8) / top for j in range(8)]
    neg = [-nd.inv_cdf(delta - j * (delta - 0.5) / 7) / top for j in range(7)]
    wrong = np.array(sorted(neg + [0.0] + pos)).astype(np.float32)
    d = 1.0 - 0.5 * (1 / 32 + 1 / 30)
    t2 = inv_norm_bisect(d)
    ref = np.array(sorted([-inv_norm_bisect(d - j * (d - 0.5) / 7) / t2 for j in range(7)] + [0.0] +
                          [inv_norm_bisect(d - j * (d - 0.5) / 8) / t2 for j in range(8)])).astype(np.float32)
    assert not np.array_equal(wrong, ref)


def test_requantizing_the_dequantized_base_keeps_its_codes():
    """Re-quantizing W' (a merge with a zero adapter) reproduces the NF4 codes:
    W'/absmax(W') lands within bf16 rounding of the original level, far from
    any midpoint; a lossy re-quantization therefore loses only what the adapter
    added.  A wrong level order, nibble order or scale in the chain fails it."""
    N, K = 64, 256
    codes, c2, c1 = _quantized(N, K, 41)
    Wd = O.bf16_value(O.nf4_dequantize(codes, c2, c1, N, K)).astype(np.float32)
    codes2, absmax2 = O.nf4_quantize(Wd)
    assert np.array_equal(codes2, codes)
    # and the block scales come back to within the bf16 rounding of s'
    sprime = O.e4m3fn_decode(c2).astype(np.float64) * np.repeat(np.asarray(c1, np.float64), 256)[: c2.size]
    assert np.allclose(absmax2, sprime, rtol=2.0 ** -8, atol=0)
