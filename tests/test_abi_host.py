"""Host-only checks of the C ABI: the libraries load, export every entry point
declared in include/qlora.h and include/qlprobe.h, carry the NF4 table the
oracle derives, and reject bad arguments with the documented status before
touching the GPU; the Python binding rejects wrongly sized tensors before
calling the library.  Nothing here launches a kernel (every call below fails
validation first)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")
PROBE_HEADER = os.path.join(ROOT, "include", "qlprobe.h")

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "bit_quantized_lora_blockwise_amd", "libqlora.so")),
    reason="libqlora.so not built (run __graft_entry__.build())")


def _lib():
    import bit_quantized_lora_blockwise_amd as q
    return q, q.lib()


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    q, L = _lib()
    names = header_functions()
    assert {"nf4_quantize", "nf4_double_quant", "qlora_linear_fwd", "qlora_linear_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q.EXPORTS)


def test_probe_library_exports_every_declared_symbol():
    """The measurement helpers live in their own library and nowhere in the
    layer library."""
    import bit_quantized_lora_blockwise_amd.probe as P
    _, L = _lib()
    names = header_functions(PROBE_HEADER)
    assert set(names) == set(P.EXPORTS) == {"ql_read_probe", "ql_empty_probe"}
    PL = P.lib()
    for n in names:
        assert hasattr(PL, n), n
    for n in names:
        assert not hasattr(L, n), n
    assert not set(names) & set(header_functions())


def test_nf4_table_matches_oracle_bitwise():
    q, _ = _lib()
    lv = np.array(q.qlora_nf4_levels(), dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), O.nf4_levels().view(np.uint32))


P = ctypes.c_void_p
A = P(4096)        # a non-null, 16-byte aligned stand-in pointer (never dereferenced)
MIS = P(4104)      # 8-byte aligned only


def test_quantize_validation():
    _, L = _lib()
    assert L.nf4_quantize(None, 0, 4, 64, A, A, None) == -1
    assert L.nf4_quantize(A, 7, 4, 64, A, A, None) == -3
    assert L.nf4_quantize(A, 0, 4, 65, A, A, None) == -2
    assert L.nf4_quantize(A, 0, 0, 64, A, A, None) == -2
    assert L.nf4_quantize(A, 1, -1, 64, A, A, None) == -2
    assert L.nf4_quantize(MIS, 1, 4, 64, A, A, None) == -4
    assert L.nf4_double_quant(A, 0, A, A, None) == -2
    assert L.nf4_double_quant(A, 10, None, A, None) == -1
    assert L.nf4_double_quant(A, 10, A, MIS, None) == -4
    assert L.nf4_dequantize(A, A, A, 2, 96, A, None) == -2
    assert L.nf4_dequantize(A, A, None, 2, 64, A, None) == -1


def test_linear_validation_and_workspace():
    _, L = _lib()
    M, K, N, r = 32, 512, 512, 8
    ws = L.qlora_linear_fwd_workspace(M, K, N, r)
    assert ws > 0 and ws % 256 == 0
    assert L.qlora_linear_fwd_workspace(M, 100, N, r) == 0
    assert L.qlora_linear_bwd_workspace(M, K, N, 65) == 0
    assert L.qlora_linear_bwd_workspace(M, K, N, r) >= 2 * M * r * 2
    fwd = lambda X=A, M=M, K=K, N=N, r=r, ws_p=A, ws_b=ws, T=None: L.qlora_linear_fwd(
        X, M, K, N, A, A, A, A, A, r, 1.0, A, T, ws_p, ws_b, None)
    assert fwd(X=None) == -1
    assert fwd(K=100) == -2
    assert fwd(r=0) == -2
    assert fwd(r=65) == -2
    assert fwd(M=0) == -2
    assert fwd(X=MIS) == -4
    assert fwd(T=MIS) == -4
    assert fwd(ws_p=None) == -5
    assert fwd(ws_b=ws - 1) == -5
    wsb = L.qlora_linear_bwd_workspace(M, K, N, r)
    bwd = lambda dL1=A, ws_b=wsb, dX=None, N=N: L.qlora_linear_bwd(
        A, A, M, K, N, A, A, A, A, A, r, 1.0, None, dX, dL1, A, A, ws_b, None)
    assert bwd(dL1=None) == -1
    assert bwd(N=-3) == -2
    assert bwd(dX=MIS) == -4
    assert bwd(ws_b=wsb - 256) == -5


def test_status_strings():
    q, _ = _lib()
    for s in range(0, -8, -1):
        assert isinstance(q.ql_status_string(s), str) and q.ql_status_string(s)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import bit_quantized_lora_blockwise_amd._lib as B
    monkeypatch.setattr(B, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_stage_entry_validation():
    _, L = _lib()
    assert L.qlora_lora_down_workspace(64, 100, 8) == 0
    ws = L.qlora_lora_down_workspace(64, 128, 8)
    assert ws > 0
    assert L.qlora_lora_down(A, 64, 128, A, 8, None, A, ws, None) == -1
    assert L.qlora_lora_down(A, 64, 128, A, 8, A, A, ws - 1, None) == -5
    assert L.qlora_linear_fwd_t(A, 64, 128, 32, A, A, A, A, A, 0, 1.0, A, None) == -2
    assert L.qlora_linear_fwd_t(A, 64, 128, 32, A, A, A, MIS, A, 8, 1.0, A, None) == -4
    assert L.qlora_lora_grad_in_workspace(64, 0, 8) == 0
    wg = L.qlora_lora_grad_in_workspace(64, 33, 8)
    assert L.qlora_lora_grad_in(A, 64, 33, A, 8, 1.0, A, None, wg, None) == -5
    assert L.qlora_linear_dx(A, 64, 96, 32, A, A, A, A, A, 8, A, None) == -2
    assert L.qlora_linear_dx(A, 64, 128, 32, A, A, A, A, None, 8, A, None) == -1


def test_merge_validation():
    _, L = _lib()
    mrg = lambda codes=A, N=48, K=128, L1=A, r=8, out=A: L.qlora_merge(codes, A, A, N, K, L1, A, r, 1.0, out, None)
    assert mrg(codes=None) == -1
    assert mrg(out=None) == -1
    assert mrg(K=96) == -2
    assert mrg(N=0) == -2
    assert mrg(r=0) == -2
    assert mrg(r=65) == -2
    assert mrg(N=1 << 32) == -2
    assert mrg(N=1 << 26, K=1 << 11) == -2   # N K above 2^36
    assert mrg(L1=MIS) == -4
    assert mrg(out=MIS) == -4


def test_q4_levels_match_oracle_bitwise():
    q, _ = _lib()
    for name in ("nf4", "fp4", "int4"):
        lv = np.array(q.q4_levels(name), dtype=np.float32)
        assert np.array_equal(lv.view(np.uint32), O.variants.codebook_levels(name).view(np.uint32)), name


def test_q4_validation():
    _, L = _lib()
    assert L.q4_quantize(A, 0, 4, 64, 3, A, A, None) == -3
    assert L.q4_quantize(A, 0, 4, 64, -1, A, A, None) == -3
    assert L.q4_quantize(A, 0, 4, 96, 1, A, A, None) == -2
    assert L.q4_quantize(A, 0, 4, 64, 1, None, A, None) == -1
    assert L.q4_quantize(MIS, 1, 4, 64, 2, A, A, None) == -4
    assert L.q4_double_quant(A, 10, 4, A, A, A, None) == -3
    assert L.q4_double_quant(A, 10, 3, A, A, A, None) == -3       # absmax scales have no second level
    assert L.q4_double_quant(A, 10, 2, A, A, None, None) == -1    # mean-centred needs mu
    assert L.q4_double_quant(A, 0, 1, A, A, None, None) == -2
    assert L.q4_double_quant(A, 10, 2, A, A, MIS, None) == -4
    deq = lambda cb=0, sc=0, am=None, c2=A, c1=A, mu=None, cols=64: L.q4_dequantize(
        A, 4, cols, cb, sc, am, c2, c1, mu, A, None)
    assert deq(cb=5) == -3
    assert deq(sc=4) == -3
    assert deq(sc=3) == -1                                          # absmax missing
    assert deq(sc=2) == -1                                          # mu missing
    assert deq(c2=None) == -1
    assert deq(cols=100) == -2
    assert deq(sc=3, am=MIS) == -4
    buf = (ctypes.c_float * 16)()
    assert L.q4_levels(3, ctypes.cast(buf, ctypes.c_void_p)) == -3
    assert L.q4_levels(1, None) == -1


def test_group_and_adamw_validation():
    _, L = _lib()
    M, K, N, r = 64, 512, 256, 8
    assert L.qlora_group_fwd_workspace(M, K, N, 3, r) > 0
    assert L.qlora_group_fwd_workspace(M, K, 200, 3, r) == 0        # segments must be multiples of 256
    assert L.qlora_group_fwd_workspace(M, K, 200, 1, r) > 0         # a single segment is the plain layer
    assert L.qlora_group_fwd_workspace(16, K, N, 3, r) > 0          # decode size: X fits the decode kernel's LDS
    assert L.qlora_group_fwd_workspace(16, 2048, N, 3, r) == 0      # decode size with X above 32 KB
    assert L.qlora_group_fwd_workspace(4, K, N, 3, 6) == 0          # decode size needs r % 4 == 0
    assert L.qlora_group_bwd_workspace(16, K, N, 3, r) == 0         # the stacked backward needs M > 16
    assert L.qlora_group_fwd_workspace(M, K, N, 0, r) == 0
    assert L.qlora_group_fwd_workspace(M, K, N, 17, r) == 0
    assert L.qlora_group_bwd_workspace(M, K, N, 3, 65) == 0
    ws = L.qlora_group_fwd_workspace(M, K, N, 3, r)
    fwd = lambda X=A, G=3, ws_b=ws, Y=A: L.qlora_group_fwd(X, M, K, N, G, A, A, A, A, A, r, 1.0, Y, None, A, ws_b,
                                                           None)
    assert fwd(X=None) == -1
    assert fwd(G=0) == -2
    assert fwd(Y=MIS) == -4
    assert fwd(ws_b=ws - 1) == -5
    wb = L.qlora_group_bwd_workspace(M, K, N, 3, r)
    assert wb >= ws
    bwd = lambda dL2=A, ws_b=wb: L.qlora_group_bwd(A, A, M, K, N, 3, A, A, A, A, A, r, 1.0, None, None, A, dL2,
                                                   A, ws_b, None)
    assert bwd(dL2=None) == -1
    assert bwd(ws_b=wb - 256) == -5
    ad = lambda p=A, n=100, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=1, pb=None: L.qlora_adamw_step(
        p, A, A, A, pb, n, lr, b1, b2, eps, wd, step, None)
    assert ad(p=None) == -1
    assert ad(n=0) == -2
    assert ad(step=0) == -2
    assert ad(lr=-1.0) == -7
    assert ad(b1=1.0) == -7
    assert ad(b2=-0.1) == -7
    assert ad(eps=0.0) == -7
    assert ad(wd=-0.5) == -7
    assert ad(lr=float("nan")) == -7
    assert ad(p=MIS) == -4
    assert ad(pb=MIS) == -4


def test_fused_quantize_validation():
    _, L = _lib()
    assert L.nf4_quantize_dq(None, 0, 4, 64, A, A, A, A, None) == -1
    assert L.nf4_quantize_dq(A, 0, 4, 64, A, None, None, A, None) == -1
    assert L.nf4_quantize_dq(A, 5, 4, 64, A, None, A, A, None) == -3
    assert L.nf4_quantize_dq(A, 1, 4, 96, A, None, A, A, None) == -2
    assert L.nf4_quantize_dq(A, 1, 4, 64, A, MIS, A, A, None) == -4


def test_read_probe_validation():
    """The probes reject null pointers, sizes that are not a positive multiple
    of 16, unsupported load counts, bad grids and misaligned pointers before
    touching the GPU."""
    import bit_quantized_lora_blockwise_amd.probe as P
    L = P.lib()
    assert L.ql_read_probe(None, 64, 4, A, None) == -1
    assert L.ql_read_probe(A, 64, 4, None, None) == -1
    assert L.ql_read_probe(A, 0, 4, A, None) == -2
    assert L.ql_read_probe(A, 40, 4, A, None) == -2
    assert L.ql_read_probe(A, 64, 3, A, None) == -2
    assert L.ql_read_probe(A, 64, 32, A, None) == -2
    assert L.ql_read_probe(MIS, 64, 4, A, None) == -4
    assert L.ql_empty_probe(0, 256, None) == -2
    assert L.ql_empty_probe(4, 0, None) == -2
    assert L.ql_empty_probe(4, 1025, None) == -2


# ---- the binding's size checks (CPU tensors: every check below fires before
#      the device check, so nothing reaches the library)

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_binding_rejects_wrong_sized_outputs():
    import torch
    q, _ = _lib()
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    W = _t((4, 128), bf)
    with pytest.raises(ValueError, match="codes must hold 256"):
        q.nf4_quantize(W, codes=_t((255,), u8), absmax=_t((8,), f32))
    with pytest.raises(ValueError, match="absmax must hold 8"):
        q.nf4_quantize(W, codes=_t((4, 64), u8), absmax=_t((7,), f32))
    with pytest.raises(ValueError, match="c1 must hold 1"):
        q.nf4_quantize_dq(W, codes=_t((256,), u8), c2=_t((8,), u8), c1=_t((2,), f32))
    with pytest.raises(ValueError, match="c2 must hold 9"):
        q.nf4_double_quant(_t((9,), f32), c2=_t((8,), u8))
    codes, c2, c1 = _t((64, 64), u8), _t((128,), u8), _t((1,), f32)      # W [64, 128]
    with pytest.raises(ValueError, match="out must hold 8192"):
        q.nf4_dequantize(codes, c2, c1, 64, 128, out=_t((64, 127), bf))
    X, L1, L2 = _t((5, 128), bf), _t((128, 8), bf), _t((8, 64), bf)
    with pytest.raises(ValueError, match="Y must hold 320"):
        q.qlora_linear_fwd(X, codes, c2, c1, 64, L1, L2, Y=_t((5, 63), bf))
    with pytest.raises(ValueError, match="T_out must hold 40"):
        q.qlora_linear_fwd(X, codes, c2, c1, 64, L1, L2, Y=_t((5, 64), bf), T_out=_t((5, 7), bf))
    dY = _t((5, 64), bf)
    with pytest.raises(ValueError, match="dX must hold 640"):
        q.qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, dX=_t((5, 64), bf))
    with pytest.raises(ValueError, match="dL1 must hold 1024"):
        q.qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, dX=None, dL1=_t((128, 7), f32))
    with pytest.raises(ValueError, match="dL2 must hold 512"):
        q.qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, dX=None, dL1=_t((128, 8), f32), dL2=_t((8, 65), f32))
    with pytest.raises(ValueError, match="Y must hold 320"):
        q.qlora_linear_fwd_t(X, codes, c2, c1, 64, _t((5, 8), bf), L2, Y=_t((320 + 1,), bf))
    with pytest.raises(ValueError, match="dX must hold 640"):
        q.qlora_linear_dx(dY, codes, c2, c1, 128, _t((5, 8), bf), L1, dX=_t((5, 127), bf))
    with pytest.raises(ValueError, match="G must hold 40"):
        q.qlora_lora_grad_in(dY, L2, G=_t((5, 9), bf))
    with pytest.raises(ValueError, match="T must hold 40"):
        q.qlora_lora_down(X, L1, T=_t((4, 8), bf))
    with pytest.raises(ValueError, match="out must hold 8192"):
        q.qlora_merge(codes, c2, c1, 64, 128, L1, L2, out=_t((64, 64), bf))
    with pytest.raises(ValueError, match="workspace must hold at least"):
        q.qlora_linear_fwd(X, codes, c2, c1, 64, L1, L2, Y=_t((5, 64), bf), workspace=_t((16,), u8))


def test_binding_rejects_wrong_sized_inputs():
    import torch
    q, _ = _lib()
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    codes, c2, c1 = _t((64, 64), u8), _t((128,), u8), _t((1,), f32)      # W [64, 128]
    X, L1, L2 = _t((5, 128), bf), _t((128, 8), bf), _t((8, 64), bf)
    with pytest.raises(ValueError, match="codes must hold 4096"):
        q.qlora_linear_fwd(X, _t((64, 63), u8), c2, c1, 64, L1, L2)
    with pytest.raises(ValueError, match="c2 must hold 128"):
        q.qlora_linear_fwd(X, codes, _t((127,), u8), c1, 64, L1, L2)
    with pytest.raises(ValueError, match="c1 must hold 1"):
        q.qlora_linear_fwd(X, codes, c2, _t((0,), f32), 64, L1, L2)
    with pytest.raises(ValueError, match="L1 must have 128 rows"):
        q.qlora_linear_fwd(X, codes, c2, c1, 64, _t((64, 8), bf), L2)
    with pytest.raises(ValueError, match=r"L2 must have shape \(8, 64\)"):
        q.qlora_linear_fwd(X, codes, c2, c1, 64, L1, _t((8, 65), bf))
    with pytest.raises(ValueError, match="dY must have 5 rows"):
        q.qlora_linear_bwd(X, _t((4, 64), bf), codes, c2, c1, L1, L2)
    with pytest.raises(ValueError, match="T must hold 40"):
        q.qlora_linear_bwd(X, _t((5, 64), bf), codes, c2, c1, L1, L2, T=_t((5, 4), bf))
    with pytest.raises(ValueError, match="multiple of 64"):
        q.nf4_dequantize(codes, c2, c1, 64, 100)
    with pytest.raises(ValueError, match="grad must hold 10"):
        q.qlora_adamw_step(_t((10,), f32), _t((10,), f32), _t((10,), f32), _t((9,), f32), 1, 1e-3)
    with pytest.raises(ValueError, match=r"L2 must have shape \(3, 8, 256\)"):
        q.qlora_group_fwd(X, _t((768, 64), u8), _t((1536,), u8), _t((6,), f32), 256, 3, _t((3, 128, 8), bf),
                          _t((3, 8, 255), bf))
    # a correctly sized CPU tensor passes the size checks and is refused as not on the GPU
    with pytest.raises(ValueError, match="on the GPU"):
        q.qlora_linear_fwd(X, codes, c2, c1, 64, L1, L2)


def test_layer_calls_reject_matrices_of_2_gib():
    """The layer's kernels address X/dX, Y/dY and the packed codes with 32-bit
    offsets: a shape that makes any of them 2^31 bytes or more is refused on the
    host (the size queries return 0, the calls QL_ERR_SHAPE), one size below is
    accepted."""
    _, L = _lib()
    r = 16
    for M, K, N in [(262144, 4096, 256),        # X: 2 M K = 2^31 bytes
                    (262144, 256, 4096),        # Y / dY: 2 M N = 2^31 bytes
                    (64, 4096, 1 << 20)]:       # codes: N K / 2 = 2^31 bytes
        assert L.qlora_linear_fwd_workspace(M, K, N, r) == 0
        assert L.qlora_linear_bwd_workspace(M, K, N, r) == 0
        assert L.qlora_linear_fwd(A, M, K, N, A, A, A, A, A, r, 1.0, A, None, A, 1 << 40, None) == -2
        assert L.qlora_linear_bwd(A, A, M, K, N, A, A, A, A, A, r, 1.0, None, None, A, A, A, 1 << 40, None) == -2
        assert L.qlora_linear_fwd_t(A, M, K, N, A, A, A, A, A, r, 1.0, A, None) == -2
        assert L.qlora_linear_dx(A, M, K, N, A, A, A, A, A, r, A, None) == -2
    assert L.qlora_linear_fwd_workspace(262143, 4096, 256, r) > 0
    assert L.qlora_linear_fwd_workspace(64, 4096, (1 << 20) - 64, r) > 0
    assert L.qlora_lora_down_workspace(262144, 4096, r) == 0
    assert L.qlora_lora_grad_in_workspace(262144, 4096, r) == 0


def test_noalloc_forward_validation():
    """The forward that allocates nothing refuses sizes whose scratch exceeds its
    static array, and bad arguments, on the host (before any HIP call)."""
    q, L = _lib()
    M, K, N, r = 32768, 16384, 256, 64
    assert L.qlora_linear_fwd_workspace(M, K, N, r) > q.NOALLOC_SCRATCH_BYTES
    assert L.qlora_linear_fwd_noalloc(A, M, K, N, A, A, A, A, A, r, 1.0, A, None, None) == -5
    assert L.qlora_linear_fwd_noalloc(None, 64, 512, 256, A, A, A, A, A, 8, 1.0, A, None, None) == -1
    assert L.qlora_linear_fwd_noalloc(A, 64, 500, 256, A, A, A, A, A, 8, 1.0, A, None, None) == -2
    assert L.qlora_linear_fwd_noalloc(A, 64, 512, 256, A, A, A, A, A, 65, 1.0, A, None, None) == -2
    assert L.qlora_linear_fwd_noalloc(A, 64, 512, 256, A, A, A, A, A, 8, 1.0, MIS, None, None) == -4
    assert L.qlora_linear_fwd_noalloc(A, 64, 512, 256, A, A, A, A, A, 8, 1.0, A, MIS, None) == -4


def test_bf16_base_layer_validation():
    _, L = _lib()
    M, K, N, r = 64, 512, 256, 8
    ws = L.qlora_linear_fwd_workspace(M, K, N, r)
    fwd = lambda X=A, W=A, K=K, r=r, Y=A, ws_b=ws: L.lora_linear_fwd(X, M, K, N, W, A, A, r, 1.0, Y, None, A, ws_b,
                                                                     None)
    assert fwd(W=None) == -1
    assert fwd(K=500) == -2
    assert fwd(r=0) == -2
    assert fwd(Y=MIS) == -4
    assert fwd(ws_b=ws - 1) == -5
    wb = L.qlora_linear_bwd_workspace(M, K, N, r)
    bwd = lambda W=A, dL2=A, ws_b=wb: L.lora_linear_bwd(A, A, M, K, N, W, A, A, r, 1.0, None, None, A, dL2, A, ws_b,
                                                        None)
    assert bwd(W=None) == -1
    assert bwd(dL2=MIS) == -4
    assert bwd(ws_b=wb - 256) == -5
    assert L.lora_linear_fwd_t(A, M, K, N, None, A, A, r, 1.0, A, None) == -1
    assert L.lora_linear_fwd_t(A, M, K, N, A, A, A, 65, 1.0, A, None) == -2
    assert L.lora_linear_dx(A, M, K, N, A, A, MIS, r, A, None) == -4
    assert L.lora_linear_dx(A, M, K, 1 << 31, A, A, A, r, A, None) == -2     # W beyond 2^31 bytes
