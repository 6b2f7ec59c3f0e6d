"""GPU parity of the adapter merge W_m = bf16(W' + s (L1 L2)^T) (examadda
page, "Practical Notes") against the CPU oracle.

Both sides quantize the same seeded weight independently (the codes and
scales are compared bit for bit first).  Tolerance per element: the kernel
sums the rank-r product in fp32 and adds it to W' in fp32 before its one
rounding, so an element may differ from the fp64 oracle by one bf16 ulp (at a
near-tie) plus the fp32 error 2^-18 (|W'| + |s| sum_c |L1[k][c] L2[c][n]|);
besides that, the relative L2 error is at most 2e-3.  Small and ragged shapes
are checked in full, the LLaMA-7B projections on row slabs whose scale
groups (256 blocks of 64) lie wholly inside them."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import assert_bitexact, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def qlib():
    import bit_quantized_lora_blockwise_amd as q
    return q


def check_merge(got, ref, Wd_bits, L1, L2, s, name):
    g, r = O.bf16_value(got), O.bf16_value(ref)
    Wd = O.bf16_value(Wd_bits)
    absprod = (np.abs(O.bf16_value(L1)) @ np.abs(O.bf16_value(L2))).T
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 7), 0.0)
    bound = ulp + 2.0 ** -18 * (np.abs(Wd) + abs(s) * absprod)
    err = np.abs(g - r)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    bad = np.argwhere(err > bound)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    diff = int(np.count_nonzero(got != ref))
    print(f"[merge] {name}: {diff} of {got.size} elements differ, rel_l2={rel:.3e}", flush=True)
    assert bad.size == 0, f"{name}: {len(bad)} beyond bound, first {bad[:3].tolist()}"
    assert rel <= 2e-3, f"{name}: rel_l2 {rel:.3e}"


def quantize_both(W_cpu):
    q = qlib()
    codes, absmax = q.nf4_quantize(W_cpu.to(DEV))
    c2, c1 = q.nf4_double_quant(absmax)
    rc, ra = O.nf4_quantize(W_cpu.float().numpy())
    rc2, rc1 = O.nf4_double_quant(ra)
    assert_bitexact(codes.cpu().numpy().reshape(-1), rc.reshape(-1), "codes")
    assert_bitexact(c2.cpu().numpy(), rc2, "c2")
    assert_bitexact(c1.cpu().numpy().view(np.uint32), np.asarray(rc1, np.float32).view(np.uint32), "c1")
    return (codes, c2, c1), (rc, rc2, rc1)


SHAPES = [  # N, K, r, s, l2_std
    (48, 128, 8, 1.0, 0.3), (33, 320, 5, 2.0, 0.3), (200, 576, 64, 0.5, 1.0), (1, 64, 1, 1.0, 1.0),
    (65, 256, 17, -0.75, 0.5), (130, 512, 33, 4.0, 0.05), (64, 1024, 24, 1.0, 0.3), (7, 192, 64, 2.0, 0.3),
    (300, 64, 16, 1.0, 0.3),
]


@pytest.mark.parametrize("N,K,r,s,l2_std", SHAPES)
def test_merge_shapes(N, K, r, s, l2_std):
    q = qlib()
    seed = 50000 + N * 131 + K * 7 + r
    W = WL.weight_gaussian(N, K, 0.02, seed)
    L1, L2 = WL.lora_pair(K, N, r, seed + 1, seed + 2, l2_std)
    gq, rq = quantize_both(W)
    got = bits(q.qlora_merge(*gq, N, K, L1.to(DEV), L2.to(DEV), s))
    ref = O.qlora_merge(*rq, N, K, bits(L1), bits(L2), s)
    check_merge(got, ref, O.nf4_dequantize(*rq, N, K), bits(L1), bits(L2), s, f"N={N} K={K} r={r} s={s}")


def test_merge_zero_adapter_and_zero_base():
    q = qlib()
    N, K, r = 96, 384, 16
    W = WL.weight_gaussian(N, K, 0.02, 777)
    L1, L2 = WL.lora_pair(K, N, r, 778, 779, 0.3)
    gq, rq = quantize_both(W)
    zero_l2 = torch.zeros((r, N), dtype=torch.bfloat16, device=DEV)
    got = q.qlora_merge(*gq, N, K, L1.to(DEV), zero_l2, 1.5)
    deq = q.nf4_dequantize(*gq, N, K)
    torch.cuda.synchronize()
    assert torch.equal(got.float(), deq.float())                      # equal in value
    assert np.array_equal(O.bf16_value(bits(got)), O.bf16_value(O.nf4_dequantize(*rq, N, K)))
    # all-zero weight: W' = 0 and the merge is the rounded adapter product alone
    Z = torch.zeros((N, K), dtype=torch.bfloat16)
    zq, zr = quantize_both(Z)
    got = bits(q.qlora_merge(*zq, N, K, L1.to(DEV), L2.to(DEV), 1.5))
    ref = O.qlora_merge(*zr, N, K, bits(L1), bits(L2), 1.5)
    check_merge(got, ref, np.zeros((N, K), np.uint16), bits(L1), bits(L2), 1.5, "zero base")


def test_merge_in_stream_order_with_layer_output():
    """The merged weight times X equals the layer's bf16 output up to the
    layer's own rounding of T = X L1: Y_merged = X W_m^T vs qlora_linear_fwd."""
    q = qlib()
    N, K, M, r, s = 256, 512, 64, 16, 2.0
    inp = WL.layer_inputs(N, K, M, r, 4242, l2_std=0.3)
    gq, _ = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    Wm = q.qlora_merge(*gq, N, K, L1, L2, s)
    Y, _ = q.qlora_linear_fwd(X, *gq, N, L1, L2, s, T_out=True)
    Ym = X.float() @ Wm.float().t()
    torch.cuda.synchronize()
    rel = (Ym - Y.float()).norm() / Y.float().norm()
    print(f"[merge] merged-weight product vs layer: rel_l2={rel.item():.3e}", flush=True)
    assert rel.item() < 1e-2


def _slab(codes, c2, c1, K, n0, R):
    """Codes and scales of rows n0 .. n0 + R (scale groups wholly inside)."""
    assert (n0 * K) % (64 * 256) == 0 and (R * K) % (64 * 256) == 0
    b0, nb = n0 * K // 64, R * K // 64
    return codes[n0:n0 + R], c2[b0:b0 + nb], c1[b0 // 256:(b0 + nb) // 256]


@pytest.mark.parametrize("which", ["up", "down"])
def test_merge_llama7b_slabs(which):
    """LLaMA-7B up (11008 x 4096) or down (4096 x 11008) projection, r = 64,
    0.1% outliers: merged on the GPU in full, checked on three 64-row slabs
    quantized and merged by the oracle on their own."""
    q = qlib()
    N, K = WL.LLAMA7B_UP if which == "up" else WL.LLAMA7B_DOWN
    r, s = 64, 2.0
    seed = 60 if which == "up" else 70
    W = WL.weight_with_outliers(N, K, 0.02, 0.001, 10.0, seed)
    L1, L2 = WL.lora_pair(K, N, r, seed + 1, seed + 2, 0.3)
    codes, absmax = q.nf4_quantize(W.to(DEV))
    c2, c1 = q.nf4_double_quant(absmax)
    print(f"[merge] {which} N={N} K={K} r={r}", flush=True)
    got = bits(q.qlora_merge(codes, c2, c1, N, K, L1.to(DEV), L2.to(DEV), s))
    L1b, L2b = bits(L1), bits(L2)
    for n0 in (0, (N // 2) // 64 * 64, N - 64):
        R = 64
        rc, ra = O.nf4_quantize(W[n0:n0 + R].float().numpy())
        rc2, rc1 = O.nf4_double_quant(ra)
        gc, gc2, gc1 = _slab(codes.cpu().numpy(), c2.cpu().numpy(), c1.cpu().numpy(), K, n0, R)
        assert_bitexact(gc.reshape(-1), rc.reshape(-1), f"codes slab {n0}")
        assert_bitexact(gc2, rc2, f"c2 slab {n0}")
        ref = O.qlora_merge(rc, rc2, rc1, R, K, L1b, L2b[:, n0:n0 + R], s)
        check_merge(got[n0:n0 + R], ref, O.nf4_dequantize(rc, rc2, rc1, R, K), L1b, L2b[:, n0:n0 + R], s,
                    f"{which} rows {n0}..{n0 + R}")


def _requant_stats(Wd, Wm, Wr):
    """rel. error of the re-quantized merged weight Wr against Wm, and the share
    of the adapter's update Wm - W' that survives: <Wr - W', D> / <D, D>."""
    D = Wm - Wd
    return {"rel_err": float(np.linalg.norm(Wr - Wm) / np.linalg.norm(Wm)),
            "retained": float(np.sum((Wr - Wd) * D) / np.sum(D * D))}


@pytest.mark.parametrize("l2_std", [0.003, 0.03, 0.3])
def test_requantize_merged_weight(l2_std):
    """The optional re-quantization of the merged weight to NF4 + double quant
    (the existing encoder entry points applied to W_m): codes and scales equal
    the oracle's wherever the merged inputs agree bit for bit, and the lossy
    error statistics agree with the oracle's to 1%."""
    q = qlib()
    N, K, r, s = 256, 1024, 16, 2.0
    W = WL.weight_gaussian(N, K, 0.02, 8100)
    L1, L2 = WL.lora_pair(K, N, r, 8101, 8102, l2_std)
    gq, rq = quantize_both(W)
    Wm = q.qlora_merge(*gq, N, K, L1.to(DEV), L2.to(DEV), s)
    codes2, absmax2 = q.nf4_quantize(Wm)
    c22, c12 = q.nf4_double_quant(absmax2)
    Wr = q.nf4_dequantize(codes2, c22, c12, N, K)
    gWm, gWr = bits(Wm), bits(Wr)
    gWd = bits(q.nf4_dequantize(*gq, N, K))

    rWm = O.qlora_merge(*rq, N, K, bits(L1), bits(L2), s)
    rcodes2, rabs2 = O.nf4_quantize(O.bf16_value(rWm).astype(np.float32))
    rc22, rc12 = O.nf4_double_quant(rabs2)
    rWr = O.nf4_dequantize(rcodes2, rc22, rc12, N, K)
    rWd = O.nf4_dequantize(*rq, N, K)

    same_block = np.all((gWm == rWm).reshape(-1, 64), axis=1)
    print(f"[requant] l2_std={l2_std}: {np.count_nonzero(~same_block)} of {same_block.size} blocks "
          f"hold a merged element that differs", flush=True)
    gc = codes2.cpu().numpy().reshape(-1, 32)
    assert np.array_equal(gc[same_block], rcodes2.reshape(-1, 32)[same_block])
    same_group = np.array([np.all(same_block[g * 256:(g + 1) * 256]) for g in range(c12.numel())])
    gc2 = c22.cpu().numpy()
    for g in np.nonzero(same_group)[0]:
        assert np.array_equal(gc2[g * 256:(g + 1) * 256], rc22[g * 256:(g + 1) * 256]), g
    assert np.array_equal(c12.cpu().numpy()[same_group].view(np.uint32),
                          np.asarray(rc12, np.float32)[same_group].view(np.uint32))

    gs = _requant_stats(*(O.bf16_value(x) for x in (gWd, gWm, gWr)))
    rs = _requant_stats(*(O.bf16_value(x) for x in (rWd, rWm, rWr)))
    print(f"[requant] l2_std={l2_std}: gpu {gs} oracle {rs}", flush=True)
    for k in gs:
        assert abs(gs[k] - rs[k]) <= 1e-2 * max(abs(rs[k]), 1e-3), k
