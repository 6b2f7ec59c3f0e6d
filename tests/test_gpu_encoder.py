"""GPU parity of the encoder, double quantization and dequantizer: every code,
scale and dequantized weight must equal the CPU oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pool
import workloads as WL
from gpu_util import assert_bitexact, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_encode(W_cpu):
    import bit_quantized_lora_blockwise_amd as q
    Wd = W_cpu.to(DEV)
    codes, absmax = q.nf4_quantize(Wd)
    c2, c1 = q.nf4_double_quant(absmax)
    deq = q.nf4_dequantize(codes, c2, c1, *Wd.shape)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), absmax.cpu().numpy(), c2.cpu().numpy(), c1.cpu().numpy(), bits(deq)


def check_encode(W_cpu, name):
    print(f"[encoder] {name} shape={tuple(W_cpu.shape)} dtype={W_cpu.dtype}", flush=True)
    rows, cols = W_cpu.shape
    g_codes, g_absmax, g_c2, g_c1, g_deq = gpu_encode(W_cpu)
    Wn = W_cpu.float().numpy()
    r_codes, r_absmax = O.nf4_quantize(Wn)
    r_c2, r_c1 = O.nf4_double_quant(r_absmax)
    r_deq = O.nf4_dequantize(r_codes, r_c2, r_c1, rows, cols)
    assert_bitexact(g_absmax.view(np.uint32), r_absmax.view(np.uint32), f"{name} absmax")
    assert_bitexact(g_codes, r_codes, f"{name} codes")
    assert_bitexact(g_c2, r_c2, f"{name} c2")
    assert_bitexact(g_c1.view(np.uint32), r_c1.view(np.uint32), f"{name} c1")
    assert_bitexact(g_deq, r_deq, f"{name} dequant")


def test_encoder_config1_fp32():
    check_encode(WL.config1()["W"], "512x512 fp32 N(0,0.02)")


def test_encoder_llama7b_up_outliers_bf16():
    check_encode(WL.weight_with_outliers(11008, 4096, 0.02, 0.001, 10.0, 10), "11008x4096 bf16 outliers")


def test_encoder_llama65b_student_t():
    check_encode(WL.config5_weight(0, "q", "t5"), "8192x8192 bf16 0.02*t5")


def _edge_matrix():
    rng = np.random.default_rng(21)
    q = O.nf4_levels()
    mids = O.nf4_midpoints()
    rows = []
    rows.append(np.zeros(256, np.float32))                                        # all-zero blocks
    for e in (-9, -1, 3):                                                         # codebook values x 2^e
        rows.append(np.array([q[i % 16] * 2.0 ** e for i in range(256)], np.float32))
    r = np.zeros(256, np.float32)                                                 # adversarial near midpoints
    for blk in range(4):
        a = np.float32(rng.uniform(0.01, 0.2))
        vals = [a]
        for m in mids:
            x = np.float32(m * float(a))
            vals += [np.nextafter(x, np.float32(-1)), x, np.nextafter(x, np.float32(1))]
        vals = [v for v in vals if abs(v) <= a][:64]
        r[blk * 64:blk * 64 + len(vals)] = vals
    rows.append(r)
    rows.append((rng.standard_normal(256) * 1e-40).astype(np.float32))          # subnormal weights
    neg0 = np.full(256, -0.0, np.float32)
    neg0[::7] = rng.standard_normal(37).astype(np.float32) * 0.01
    rows.append(neg0)                                                             # signed zeros
    rows.append((rng.standard_normal(256) * 3e4).astype(np.float32))             # large magnitudes
    rows.append(np.where(rng.random(256) < 0.5, 1.0, -1.0).astype(np.float32))   # +-absmax only
    # absmax at the ends of the normal range (16 / absmax overflows below 2^-124,
    # and its reciprocal is subnormal above 2^126): codebook values x 2^e
    for e in (-126, -125, -124, -123, 125, 126, 127):
        rows.append(np.array([np.float32(q[(5 * i) % 16]) * np.float32(2.0 ** e) for i in range(256)], np.float32))
    return np.stack(rows)


def test_encoder_edge_cases_fp32():
    check_encode(torch.from_numpy(_edge_matrix()), "edge cases fp32")


def test_encoder_edge_cases_bf16():
    W = torch.from_numpy(_edge_matrix()).to(torch.bfloat16)
    check_encode(W, "edge cases bf16")


@pytest.mark.parametrize("rows,cols", [(1, 64), (3, 320), (5, 64 * 51), (257, 64)])
def test_encoder_ragged_groups(rows, cols):
    W = WL.normal((rows, cols), 0.02, rows * 1000 + cols, torch.float32)
    check_encode(W, f"{rows}x{cols}")


def test_encoder_deterministic():
    import bit_quantized_lora_blockwise_amd as q
    W = WL.weight_gaussian(2048, 4096, 0.02, 77).to(DEV)
    a = q.nf4_quantize(W)
    b = q.nf4_quantize(W)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_double_quant_sweep():
    """Every 97th fp32 value in [0, 1] as a scale in groups whose max is 1.0: the
    E4M3FN code of each equals the oracle's."""
    import bit_quantized_lora_blockwise_amd as q
    one = int(np.float32(1.0).view(np.uint32))
    t = np.arange(0, one + 1, 97, dtype=np.uint32).view(np.float32)
    per = 255
    ng = (t.size + per - 1) // per
    a = np.zeros(ng * 256, np.float32)
    a.reshape(ng, 256)[:, 0] = 1.0
    body = a.reshape(ng, 256)[:, 1:].reshape(-1)
    body[:t.size] = t
    a.reshape(ng, 256)[:, 1:] = body.reshape(ng, 255)
    print(f"[double-quant sweep] {t.size} values in {ng} groups", flush=True)
    ad = torch.from_numpy(a).to(DEV)
    c2, c1 = q.nf4_double_quant(ad)
    torch.cuda.synchronize()
    r_c2, r_c1 = O.nf4_double_quant(a)
    assert_bitexact(c2.cpu().numpy(), r_c2, "c2 sweep")
    assert_bitexact(c1.cpu().numpy().view(np.uint32), r_c1.view(np.uint32), "c1 sweep")


def _blocks_with_absmax(vals, a):
    """Rows of 64 weights: a first, then 63 of `vals` (|v| <= a), zero padded."""
    per = 63
    nb = (vals.size + per - 1) // per
    W = np.zeros((nb, 64), np.float32)
    W[:, 0] = a
    body = np.zeros(nb * per, np.float32)
    body[:vals.size] = vals
    W[:, 1:] = body.reshape(nb, per)
    return W


def test_nearest_code_sweep():
    """Codes of weights w with block absmax a = 1 (so n = w exactly), for every
    fp32 within 2^16 ulp of each code midpoint and of each multiple of 1/16 in
    [-1, 1], and every 997th fp32 of [-1, 1]; then the same neighbourhoods of
    the midpoints scaled by a non-power-of-two absmax.  Every code must equal
    the oracle's nearest-level rule."""
    one = int(np.float32(1.0).view(np.uint32))
    pts = [float(m) for m in O.nf4_midpoints()] + [k / 16.0 for k in range(-16, 17)]
    chunks = []
    for p in pts:
        c = int(np.float32(abs(p)).view(np.uint32))
        lo, hi = max(c - 65536, 0), min(c + 65536, one)
        v = np.arange(lo, hi + 1, dtype=np.uint32).view(np.float32)
        chunks.append(v if p >= 0 else -v)
    stride = np.arange(0, one + 1, 997, dtype=np.uint32).view(np.float32)
    chunks += [stride, -stride]
    vals = np.concatenate(chunks)
    W1 = _blocks_with_absmax(vals, np.float32(1.0))
    a = np.float32(0.0371)
    near = []
    for m in O.nf4_midpoints():
        x = np.float32(float(m) * float(a))
        c = int(np.abs(x).view(np.uint32))
        v = np.arange(c - 64, c + 65, dtype=np.uint32).view(np.float32)
        near.append(v if x >= 0 else -v)
    near = np.concatenate(near)
    near = near[np.abs(near) <= a]
    Wa = _blocks_with_absmax(near, a)
    W = np.concatenate([W1, Wa])
    print(f"[nearest sweep] {vals.size + near.size} weights in {W.shape[0]} blocks", flush=True)
    import bit_quantized_lora_blockwise_amd as q
    codes, absmax = q.nf4_quantize(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    r_codes, r_absmax = O.nf4_quantize(W)
    assert_bitexact(absmax.cpu().numpy().view(np.uint32), r_absmax.view(np.uint32), "sweep absmax")
    assert_bitexact(codes.cpu().numpy(), r_codes, "sweep codes")


def _bit_range_chunks(total, chunk):
    for lo in range(0, total, chunk):
        yield lo, min(total, lo + chunk)


def test_nearest_code_exhaustive():
    """Every fp32 n in [-1, 1] (2 x 1,065,353,217 values): blocks of 64 whose
    first element is 1.0 (absmax 1, so n = w exactly) and 63 consecutive fp32
    bit patterns; the code of each must be the oracle's nearest-level rule.  The
    inputs are built on the GPU from the bit patterns; the expected codes come
    from the oracle on the CPU, one chunk per thread."""
    from concurrent.futures import ThreadPoolExecutor
    import bit_quantized_lora_blockwise_amd as q
    one = int(np.float32(1.0).view(np.uint32))
    total = one + 1                                                   # bit patterns 0 .. one
    per, nblk = 63, 1 << 20
    chunk = per * nblk

    def expect(lo, hi, sign):
        v = np.arange(lo, hi, dtype=np.uint32) | np.uint32(sign)
        return O.nf4_nearest_code(v.view(np.float32))

    def check(got, lo, hi, sign):
        exp = expect(lo, hi, sign)
        assert got.size == exp.size == hi - lo
        bad = np.flatnonzero(got != exp)
        return (lo, sign, bad.size, bad[:4], got[bad[:4]], exp[bad[:4]], exp.size)

    results = []
    with ThreadPoolExecutor(max_workers=8) as pool:
        futs = []
        for sign in (0, 0x80000000):
            for lo, hi in _bit_range_chunks(total, chunk):
                n = hi - lo
                nb = (n + per - 1) // per
                bits = torch.arange(lo, lo + nb * per, dtype=torch.int64, device=DEV)
                bits = torch.where(bits < hi, bits, torch.zeros_like(bits))
                vals = bits.to(torch.int32).view(torch.float32).view(nb, per)
                if sign:
                    vals = -vals                                      # sets the sign bit, -0.0 included
                W = torch.cat([torch.ones((nb, 1), dtype=torch.float32, device=DEV), vals], dim=1)
                codes, _ = q.nf4_quantize(W)
                c = codes.view(nb, 32)
                el = torch.stack([c & 15, c >> 4], dim=2).view(nb, 64)[:, 1:].reshape(-1)[:n]
                got = el.cpu().numpy()
                futs.append(pool.submit(check, got, lo, hi, sign))
                print(f"[nearest exhaustive] sign {sign:#x} bits {lo}..{hi} on the GPU", flush=True)
                if len(futs) >= 8:
                    results.append(futs.pop(0).result())
        results += [f.result() for f in futs]
    assert sum(r[6] for r in results) == 2 * total                  # every value of both halves checked
    bad = [r for r in results if r[2]]
    assert not bad, f"code mismatches (lo, sign, count, first, got, expected): {bad[:3]}"


def test_nearest_code_all_bf16():
    """Every bf16 n in [-1, 1] through the bf16-input encoder (blocks with absmax
    1.0), and the same values scaled by the bf16 absmax 0.0371 rounded to bf16,
    against the oracle (which takes the exact fp32 values of the bf16 inputs)."""
    import bit_quantized_lora_blockwise_amd as q
    one16 = 0x3F80
    pos = (np.arange(0, one16 + 1, dtype=np.uint32) << 16).view(np.float32)
    vals = np.concatenate([pos, -pos])
    W1 = _blocks_with_absmax(vals, np.float32(1.0))
    a = torch.tensor([0.0371]).to(torch.bfloat16).float().numpy()[0]
    scaled = torch.from_numpy(vals * a).to(torch.bfloat16).float().numpy()
    scaled = scaled[np.abs(scaled) <= a]
    Wa = _blocks_with_absmax(scaled, a)
    W = torch.from_numpy(np.concatenate([W1, Wa])).to(torch.bfloat16)
    Wf = W.float().numpy()
    codes, absmax = q.nf4_quantize(W.to(DEV))
    torch.cuda.synchronize()
    r_codes, r_absmax = O.nf4_quantize(Wf)
    assert_bitexact(absmax.cpu().numpy().view(np.uint32), r_absmax.view(np.uint32), "bf16 sweep absmax")
    assert_bitexact(codes.cpu().numpy(), r_codes, "bf16 sweep codes")


def test_e4m3fn_scale_exhaustive():
    """Every fp32 t in [0, 1] (1,065,353,218 values) as a block scale in groups of
    256 whose first scale is 1.0 (c1 = 1, so t = a exactly): each E4M3FN code must
    be the oracle's round-to-nearest-even encoding."""
    from concurrent.futures import ThreadPoolExecutor
    import bit_quantized_lora_blockwise_amd as q
    one = int(np.float32(1.0).view(np.uint32))
    total = one + 1
    per, ngrp = 255, 1 << 18
    chunk = per * ngrp

    def check(got, lo, hi):
        exp = O.e4m3fn_encode(np.arange(lo, hi, dtype=np.uint32).view(np.float32))
        assert got.size == exp.size == hi - lo
        bad = np.flatnonzero(got != exp)
        return (lo, bad.size, bad[:4], got[bad[:4]], exp[bad[:4]], exp.size)

    results = []
    with ThreadPoolExecutor(max_workers=8) as pool:
        futs = []
        for lo, hi in _bit_range_chunks(total, chunk):
            n = hi - lo
            ng = (n + per - 1) // per
            bits = torch.arange(lo, lo + ng * per, dtype=torch.int64, device=DEV)
            bits = torch.where(bits < hi, bits, torch.zeros_like(bits))
            vals = bits.to(torch.int32).view(torch.float32).view(ng, per)
            a = torch.cat([torch.ones((ng, 1), dtype=torch.float32, device=DEV), vals], dim=1).reshape(-1)
            c2, c1 = q.nf4_double_quant(a)
            got = c2.view(ng, 256)[:, 1:].reshape(-1)[:n].cpu().numpy()
            assert torch.all(c1 == 1.0)
            futs.append(pool.submit(check, got, lo, hi))
            print(f"[e4m3fn exhaustive] bits {lo}..{hi} on the GPU", flush=True)
            if len(futs) >= 8:
                results.append(futs.pop(0).result())
        results += [f.result() for f in futs]
    assert sum(r[5] for r in results) == total                       # every value checked
    bad = [r for r in results if r[1]]
    assert not bad, f"E4M3FN mismatches (lo, count, first, got, expected): {bad[:3]}"


@pytest.mark.parametrize("rows,cols,dtype", [(512, 512, "fp32"), (11008, 4096, "bf16"), (3, 320, "fp32"),
                                             (257, 64, "bf16"), (5, 64 * 51, "bf16")])
def test_fused_quantize_and_double_quant(rows, cols, dtype):
    """nf4_quantize_dq equals nf4_quantize followed by nf4_double_quant, bit for
    bit (and so the oracle), including partial last groups."""
    import bit_quantized_lora_blockwise_amd as q
    W = WL.normal((rows, cols), 0.02, rows * 31 + cols, torch.float32)
    W[0, :64] = 0.0                                           # an all-zero block
    if dtype == "bf16":
        W = W.to(torch.bfloat16)
    Wd = W.to(DEV)
    print(f"[fused encode] {rows}x{cols} {dtype}", flush=True)
    codes, c2, c1, absmax = q.nf4_quantize_dq(Wd, absmax=True)
    codes_s, absmax_s = q.nf4_quantize(Wd)
    c2_s, c1_s = q.nf4_double_quant(absmax_s)
    codes_n, c2_n, c1_n, _ = q.nf4_quantize_dq(Wd)            # without absmax
    torch.cuda.synchronize()
    assert torch.equal(codes, codes_s) and torch.equal(codes_n, codes_s)
    assert torch.equal(absmax.view(torch.int32), absmax_s.view(torch.int32))
    assert torch.equal(c2, c2_s) and torch.equal(c2_n, c2_s)
    assert torch.equal(c1.view(torch.int32), c1_s.view(torch.int32)) and torch.equal(c1_n.view(torch.int32),
                                                                                       c1_s.view(torch.int32))
    rc, ra, rc2, rc1, _ = oracle_pool.quantize(W.float().numpy(), dequant=False)
    assert_bitexact(codes.cpu().numpy().reshape(-1), rc.reshape(-1), "fused codes")
    assert_bitexact(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32), "fused absmax")
    assert_bitexact(c2.cpu().numpy(), rc2, "fused c2")
    assert_bitexact(c1.cpu().numpy().view(np.uint32), rc1.view(np.uint32), "fused c1")


@pytest.mark.parametrize("variant", ["gauss", "t5"])
@pytest.mark.parametrize("layer", [0, 1, 40, 79])
def test_fused_encoder_llama65b_layers(layer, variant):
    """The encoding workload of 80 LLaMA-65B blocks, sampled at layers 0, 1, 40
    and 79 of both weight distributions: the three distinct matrix shapes of a
    layer (q 8192 x 8192, gate 22016 x 8192, down 8192 x 22016), drawn on the
    GPU with the layer's seeds, go through the one-pass encoder; codes, c2 and
    c1 equal the oracle's bit for bit over the whole matrix, and so does the
    dequantized weight of the q matrix."""
    import bit_quantized_lora_blockwise_amd as q
    for name in ("q", "gate", "down"):
        W = WL.config5_weight(layer, name, variant, device=DEV)
        print(f"[fused encode 65B] layer {layer} {variant} {name} {tuple(W.shape)}", flush=True)
        codes, c2, c1, _ = q.nf4_quantize_dq(W)
        deq = q.nf4_dequantize(codes, c2, c1, *W.shape) if name == "q" else None
        torch.cuda.synchronize()
        rc, _, rc2, rc1, rq = oracle_pool.quantize(bits(W), dequant=deq is not None)
        tag = f"layer {layer} {variant} {name}"
        assert_bitexact(codes.cpu().numpy().reshape(-1), rc.reshape(-1), f"{tag} codes")
        assert_bitexact(c2.cpu().numpy(), rc2, f"{tag} c2")
        assert_bitexact(c1.cpu().numpy().view(np.uint32), rc1.view(np.uint32), f"{tag} c1")
        if deq is not None:
            assert_bitexact(bits(deq), rq, f"{tag} dequant")
        del W, codes, c2, c1, deq


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_encoder_edge_cases(dtype):
    """The one-pass encoder with double quantization on the edge-case matrix
    (zero blocks, codebook values x 2^e up to both ends of the normal range,
    midpoint neighbours, subnormals, signed zeros, large magnitudes): codes, c2
    and c1 equal the oracle's bit for bit."""
    import bit_quantized_lora_blockwise_amd as q
    W = torch.from_numpy(_edge_matrix())
    if dtype == "bf16":
        W = W.to(torch.bfloat16)
    codes, c2, c1, _ = q.nf4_quantize_dq(W.to(DEV))
    torch.cuda.synchronize()
    rc, ra = O.nf4_quantize(W.float().numpy())
    rc2, rc1 = O.nf4_double_quant(ra)
    assert_bitexact(codes.cpu().numpy(), rc, f"fused edge codes {dtype}")
    assert_bitexact(c2.cpu().numpy(), rc2, f"fused edge c2 {dtype}")
    assert_bitexact(c1.cpu().numpy().view(np.uint32), rc1.view(np.uint32), f"fused edge c1 {dtype}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_encoders_with_non_finite_weights(dtype):
    """Non-finite weights leave their own block's codes and their group's scales
    unspecified, but both encoders still complete, and every block without one
    (and every group of 256 blocks without one) keeps the oracle's codes,
    absmax, c2 and c1 bit for bit.  The NaN and infinite quotients reach the
    bucket lookup, whose address stays inside the table for them."""
    import bit_quantized_lora_blockwise_amd as q
    rows, cols = 64, 4096                                           # 4096 blocks, 16 groups
    W = WL.normal((rows, cols), 0.02, 77, torch.float32)
    flat = W.view(-1)
    bad_blocks = {}
    nan_neg = float(np.array([0xFFC00000], np.uint32).view(np.float32)[0])
    for blk, vals in ((3 * 256 + 5, [float("nan")]), (3 * 256 + 6, [float("inf")]),
                      (9 * 256 + 0, [float("-inf"), float("inf")]), (9 * 256 + 255, [nan_neg]),
                      (12 * 256 + 17, [float("nan")] * 64)):
        for i, v in enumerate(vals):
            flat[blk * 64 + (i * 13) % 64] = v
        bad_blocks[blk] = True
    if dtype == "bf16":
        W = W.to(torch.bfloat16)
    Wd = W.to(DEV)
    print(f"[encoder non-finite] {rows}x{cols} {dtype}", flush=True)
    codes, c2, c1, absmax = q.nf4_quantize_dq(Wd, absmax=True)
    codes_s, absmax_s = q.nf4_quantize(Wd)
    c2_s, c1_s = q.nf4_double_quant(absmax_s)
    torch.cuda.synchronize()
    Wf = W.float().numpy().copy().reshape(-1, 64)
    Wf[list(bad_blocks)] = 0.0                                     # the oracle sees finite blocks only
    rc, ra = O.nf4_quantize(Wf.reshape(rows, cols))
    rc2, rc1 = O.nf4_double_quant(ra)
    good = np.ones(rows * cols // 64, bool)
    good[list(bad_blocks)] = False
    good_groups = np.ones(16, bool)
    good_groups[[b // 256 for b in bad_blocks]] = False
    in_good_group = np.repeat(good_groups, 256)
    for tag, cd, am, s2, s1 in (("fused", codes, absmax, c2, c1), ("two calls", codes_s, absmax_s, c2_s, c1_s)):
        g_codes = cd.cpu().numpy().reshape(-1, 32)
        assert_bitexact(g_codes[good], rc.reshape(-1, 32)[good], f"{tag} codes of finite blocks")
        assert_bitexact(am.cpu().numpy().view(np.uint32)[good], ra.view(np.uint32)[good], f"{tag} absmax")
        assert_bitexact(s2.cpu().numpy()[in_good_group], rc2[in_good_group], f"{tag} c2 of finite groups")
        assert_bitexact(s1.cpu().numpy().view(np.uint32)[good_groups], rc1.view(np.uint32)[good_groups],
                        f"{tag} c1 of finite groups")


def test_encoders_beyond_2_gib():
    """A 16400 x 262144 bf16 weight (8.6 GB; its codes 2.15 GB): both encoders
    address the weights, codes, scale codes and group scales past 2^31 bytes.
    Each row holds 16 whole groups of 256 blocks, so a row's codes, c2 and c1
    depend on that row alone; the rows holding byte 2^31 of the weights and of
    the codes, and the first and last rows, are compared with the oracle."""
    import bit_quantized_lora_blockwise_amd as q
    rows, cols = 16400, 262144
    g = torch.Generator(device=DEV)
    g.manual_seed(2024)
    W = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, rows, 1024):                   # drawn in slabs to bound the fp32 temporary
        r1 = min(rows, r0 + 1024)
        W[r0:r1] = (torch.randn((r1 - r0, cols), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    print(f"[encoder 2 GiB+] {rows}x{cols} bf16", flush=True)
    codes, c2, c1, _ = q.nf4_quantize_dq(W)
    codes_s, absmax_s = q.nf4_quantize(W)
    torch.cuda.synchronize()
    gpr = cols // (64 * 256)                           # groups per row
    for row in sorted({0, (1 << 30) // cols, (1 << 32) // cols, rows - 1}):
        Wr = W[row:row + 1].float().cpu().numpy()
        rc, ra = O.nf4_quantize(Wr)
        rc2, rc1 = O.nf4_double_quant(ra)
        nb = cols // 64
        tag = f"row {row}"
        assert_bitexact(codes[row].cpu().numpy().reshape(1, -1), rc, f"{tag} fused codes")
        assert_bitexact(c2[row * nb:(row + 1) * nb].cpu().numpy(), rc2, f"{tag} fused c2")
        assert_bitexact(c1[row * gpr:(row + 1) * gpr].cpu().numpy().view(np.uint32), rc1.view(np.uint32),
                        f"{tag} fused c1")
        assert_bitexact(codes_s[row].cpu().numpy().reshape(1, -1), rc, f"{tag} codes")
        assert_bitexact(absmax_s[row * nb:(row + 1) * nb].cpu().numpy().view(np.uint32), ra.view(np.uint32),
                        f"{tag} absmax")
    del W, codes, c2, c1, codes_s, absmax_s
    torch.cuda.empty_cache()
