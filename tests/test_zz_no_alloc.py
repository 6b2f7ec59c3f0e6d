"""The forward entry point that allocates nothing (qlora_linear_fwd_noalloc,
its scratch in the library's per-GPU static array) against qlora_linear_fwd
with a caller-supplied workspace: called through the C ABI twice in a row, the
second time with a smaller input, and compared bit for bit (the same kernels
run on the same inputs); then against the CPU oracle.  Sizes beyond the
array are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import assert_close, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _q():
    import bit_quantized_lora_blockwise_amd as q
    return q


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _layer(M, K, N, r, seed):
    q = _q()
    inp = WL.layer_inputs(N, K, M, r, seed_base=seed, l2_std=0.3)
    codes, c2, c1, _ = q.nf4_quantize_dq(inp["W"].to(DEV))
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    return inp, (codes, c2, c1), X, L1, L2


def _noalloc_call(X, codes, c2, c1, N, L1, L2, r, s, Y, T):
    L = _q().lib()
    M, K = X.shape
    st = L.qlora_linear_fwd_noalloc(_ptr(X), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r,
                                    float(s), _ptr(Y), _ptr(T), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _q().ql_status_string(st)


def _with_workspace(X, packed, N, L1, L2, s):
    q = _q()
    return q.qlora_linear_fwd(X, *packed, N, L1, L2, s, T_out=True)


@pytest.mark.parametrize("shapes", [((320, 1024, 768, 64), (5, 1024, 640, 16)),
                                    ((16, 4096, 2048, 64), (3, 512, 300, 8)),
                                    ((2048, 4096, 1024, 64), (40, 2048, 512, 24))])
def test_noalloc_matches_workspace_call_twice(shapes):
    s = 0.75
    for i, (M, K, N, r) in enumerate(shapes):
        print(f"[noalloc] call {i}: M={M} K={K} N={N} r={r}", flush=True)
        inp, packed, X, L1, L2 = _layer(M, K, N, r, 600 + 7 * i + M)
        Y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
        T = torch.full((M, r), 3.0, dtype=torch.bfloat16, device=DEV)
        _noalloc_call(X, *packed, N, L1, L2, r, s, Y, T)
        Yw, Tw = _with_workspace(X, packed, N, L1, L2, s)
        # the same call without T_out keeps T in the scratch array too
        Y2 = torch.empty_like(Y)
        _noalloc_call(X, *packed, N, L1, L2, r, s, Y2, None)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Yw.view(torch.int16)), (i, "Y")
        assert torch.equal(T.view(torch.int16), Tw.view(torch.int16)), (i, "T")
        assert torch.equal(Y2.view(torch.int16), Yw.view(torch.int16)), (i, "Y without T_out")
        rc, ra = O.nf4_quantize(inp["W"].float().numpy())
        rc2, rc1 = O.nf4_double_quant(ra)
        Wq = O.nf4_dequantize(rc, rc2, rc1, N, K)
        rY, rT = O.qlora_forward(bits(inp["X"]), Wq, bits(inp["L1"]), bits(inp["L2"]), s)
        assert_close(bits(T), rT, f"noalloc call {i} T")
        assert_close(bits(Y), rY, f"noalloc call {i} Y")


def test_noalloc_binding_and_limit():
    q = _q()
    inp, packed, X, L1, L2 = _layer(24, 512, 256, 8, 4711)
    Y, T = q.qlora_linear_fwd_noalloc(X, *packed, 256, L1, L2, 1.0, T_out=True)
    Yw, Tw = _with_workspace(X, packed, 256, L1, L2, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yw) and torch.equal(T, Tw)
    # a forward whose scratch exceeds the static array is refused on the host
    M, K, N, r = 32768, 16384, 256, 64
    assert q.qlora_linear_fwd_workspace(M, K, N, r) > q.NOALLOC_SCRATCH_BYTES
    L = q.lib()
    A = ctypes.c_void_p(4096)
    assert L.qlora_linear_fwd_noalloc(A, M, K, N, A, A, A, A, A, r, 1.0, A, None, None) == -5
