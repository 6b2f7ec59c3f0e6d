"""GPU parity of the code-book and scale-code variants (4-bit float and 4-bit
integer tables in the blockwise encoder and dequantizer; full-range and
mean-centred second-level codes) against the CPU oracle: every code, scale
and dequantized weight bit for bit, so the quantization-error study computed
from the GPU's outputs is the oracle's."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import assert_bitexact, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
V = O.variants
BOOKS = ("nf4", "fp4", "int4")


def qlib():
    import bit_quantized_lora_blockwise_amd as q
    return q


def _midpoint_rows(levels, seed):
    """Blocks whose weights sit at and around midpoint * absmax of a table."""
    rng = np.random.default_rng(seed)
    lv = np.asarray(levels, np.float32).astype(np.float64)
    mids = np.unique((lv[:-1] + lv[1:]) / 2)
    rows = np.zeros((4, 256), np.float32)
    for r in range(4):
        for blk in range(4):
            a = np.float32(rng.uniform(0.01, 0.3)) if (r, blk) != (0, 0) else np.float32(1.0)
            vals = [a]
            for m in mids:
                x = np.float32(m * float(a))
                vals += [np.nextafter(x, np.float32(-2)), x, np.nextafter(x, np.float32(2))]
            vals = [v for v in vals if abs(v) <= a][:64]
            rows[r, blk * 64:blk * 64 + len(vals)] = vals
    return rows


def _inputs():
    rng = np.random.default_rng(31)
    out = {
        "normal fp32": rng.standard_normal((512, 1024)).astype(np.float32),
        "t5 bf16": torch.from_numpy(rng.standard_t(5, (256, 1024)).astype(np.float32)).to(torch.bfloat16),
        "edge fp32": np.concatenate([np.zeros((1, 256), np.float32),
                                     (rng.standard_normal((1, 256)) * 1e-40).astype(np.float32),
                                     (rng.standard_normal((1, 256)) * 3e4).astype(np.float32),
                                     np.where(rng.random((1, 256)) < 0.5, 1.0, -1.0).astype(np.float32)]),
        "ragged 5x3264": WL.normal((5, 64 * 51), 0.02, 5051, torch.float32),
    }
    return out


@pytest.mark.parametrize("book", BOOKS)
def test_q4_encode_and_dequant_bitexact(book):
    q = qlib()
    lv = V.codebook_levels(book)
    cases = dict(_inputs())
    cases["midpoints"] = np.concatenate([_midpoint_rows(V.codebook_levels(b), 7 + i) for i, b in enumerate(BOOKS)])
    for name, W in cases.items():
        Wt = W if isinstance(W, torch.Tensor) else torch.from_numpy(W)
        rows, cols = Wt.shape
        print(f"[q4] {book} {name} {rows}x{cols} {Wt.dtype}", flush=True)
        codes, absmax = q.q4_quantize(Wt.to(DEV), book)
        rc, ra = V.q4_quantize(Wt.float().numpy(), lv)
        assert_bitexact(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32), f"{book} {name} absmax")
        assert_bitexact(codes.cpu().numpy(), rc, f"{book} {name} codes")
        if book != "nf4":
            assert not np.any(O.unpack_codes(rc) == 15)       # code 15 repeats +1 and is never chosen
        else:                                   # the generic encoder agrees with the bucketed one
            c0, a0 = q.nf4_quantize(Wt.to(DEV))
            assert torch.equal(c0, codes)
        for sc in ("absmax", "groupmax", "fullrange", "mean"):
            if sc == "absmax":
                c2 = c1 = mu = None
                rs = V.scales("absmax", ra)
            else:
                c2, c1, mu = q.q4_double_quant(absmax, sc)
                rc2, rc1, rmu = V.double_quant(ra, sc)
                assert_bitexact(c2.cpu().numpy(), rc2, f"{book} {name} {sc} c2")
                assert_bitexact(c1.cpu().numpy().view(np.uint32), rc1.view(np.uint32), f"{book} {name} {sc} c1")
                if sc == "mean":
                    assert_bitexact(mu.cpu().numpy().view(np.uint32), rmu.view(np.uint32), f"{book} {name} mu")
                rs = V.scales(sc, None, rc2, rc1, rmu)
            Wd = q.q4_dequantize(codes, rows, cols, book, sc, absmax=absmax if sc == "absmax" else None,
                                 c2=c2, c1=c1, mu=mu)
            torch.cuda.synchronize()
            assert_bitexact(bits(Wd), V.q4_dequantize(rc, rs, lv, rows, cols), f"{book} {name} {sc} dequant")


def test_q4_nf4_groupmax_is_the_contract_dequantizer():
    q = qlib()
    W = WL.weight_gaussian(384, 512, 0.02, 4242).to(DEV)
    codes, absmax = q.nf4_quantize(W)
    c2, c1 = q.nf4_double_quant(absmax)
    c2b, c1b, _ = q.q4_double_quant(absmax, "groupmax")
    a = q.nf4_dequantize(codes, c2, c1, 384, 512)
    b = q.q4_dequantize(codes, 384, 512, "nf4", "groupmax", c2=c2b, c1=c1b)
    torch.cuda.synchronize()
    assert torch.equal(c2, c2b) and torch.equal(c1.view(torch.int32), c1b.view(torch.int32))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _absmax_cases():
    rng = np.random.default_rng(44)
    w = rng.standard_normal((3000, 64)) * 0.02
    real = np.max(np.abs(w), axis=1).astype(np.float32)
    spread = (10.0 ** rng.uniform(-6, 2, 700)).astype(np.float32)             # eight decades in a group
    equal = np.full(300, 0.125, np.float32)                                   # max |d| = 0 for the mean
    zeros = np.zeros(256, np.float32)
    tiny = (rng.random(600) * 1e-38).astype(np.float32)                        # subnormal scales
    ints = np.tile(np.array([0, 8, 24, 32], np.float32), 64)                  # exact reconstruction case
    return {"real": real, "spread": spread, "equal": equal, "zeros+ints": np.concatenate([zeros, ints]),
            "tiny": tiny, "one": real[:1], "257": real[:257]}


@pytest.mark.parametrize("sc", ["groupmax", "fullrange", "mean"])
def test_second_level_variants_bitexact(sc):
    q = qlib()
    for name, a in _absmax_cases().items():
        print(f"[dq] {sc} {name} n={a.size}", flush=True)
        c2, c1, mu = q.q4_double_quant(torch.from_numpy(a).to(DEV), sc)
        torch.cuda.synchronize()
        rc2, rc1, rmu = V.double_quant(a, sc)
        assert_bitexact(c2.cpu().numpy(), rc2, f"{sc} {name} c2")
        assert_bitexact(c1.cpu().numpy().view(np.uint32), rc1.view(np.uint32), f"{sc} {name} c1")
        if sc == "mean":
            assert_bitexact(mu.cpu().numpy().view(np.uint32), rmu.view(np.uint32), f"{sc} {name} mu")


def test_quantization_error_study_matches_oracle():
    """The study's numbers from the GPU's outputs equal the oracle's (same bits),
    and the ranking NF4 < 4-bit float < 4-bit integer holds for N(0, 1) and t5
    blocks under every scale code."""
    q = qlib()
    rng = np.random.default_rng(77)
    mats = {"normal": rng.standard_normal((256, 1024)).astype(np.float32),
            "t5": rng.standard_t(5, (256, 1024)).astype(np.float32)}
    for dist, W in mats.items():
        res = {}
        for book in BOOKS:
            lv = V.codebook_levels(book)
            codes, absmax = q.q4_quantize(torch.from_numpy(W).to(DEV), book)
            rc, ra = V.q4_quantize(W, lv)
            for sc in ("absmax", "groupmax", "fullrange", "mean"):
                if sc == "absmax":
                    Wd = q.q4_dequantize(codes, 256, 1024, book, sc, absmax=absmax)
                    rs = V.scales(sc, ra)
                else:
                    c2, c1, mu = q.q4_double_quant(absmax, sc)
                    Wd = q.q4_dequantize(codes, 256, 1024, book, sc, c2=c2, c1=c1, mu=mu)
                    rs = V.scales(sc, None, *V.double_quant(ra, sc))
                torch.cuda.synchronize()
                g = V.error_stats(W, bits(Wd), codes.cpu().numpy())
                r = V.error_stats(W, V.q4_dequantize(rc, rs, lv, 256, 1024), rc)
                assert g == r, (dist, book, sc, g, r)
                res[(book, sc)] = g
        for sc in ("absmax", "groupmax", "fullrange", "mean"):
            print(f"[study] {dist} {sc}: " + ", ".join(f"{b} {res[(b, sc)]['nmse']:.5f}" for b in BOOKS), flush=True)
            assert res[("nf4", sc)]["nmse"] < res[("fp4", sc)]["nmse"] < res[("int4", sc)]["nmse"]
