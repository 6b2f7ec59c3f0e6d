"""ctypes binding of libqlora.so: argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/qlora.h for the contract).  Tensors are torch tensors on the GPU; the
binding checks dtype/contiguity/device, allocates missing outputs with torch,
passes raw pointers and the current HIP stream, and raises QloraError on a
non-zero status.  All computation happens in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora.so")
_lib = None

QL_F32, QL_BF16 = 0, 1
CODEBOOKS = {"nf4": 0, "fp4": 1, "int4": 2}
SCALE_CODES = {"groupmax": 0, "fullrange": 1, "mean": 2, "absmax": 3}
STATUS = {0: "QL_OK", -1: "QL_ERR_NULL", -2: "QL_ERR_SHAPE", -3: "QL_ERR_DTYPE", -4: "QL_ERR_ALIGN",
          -5: "QL_ERR_WORKSPACE", -6: "QL_ERR_HIP", -7: "QL_ERR_VALUE"}
EXPORTS = ("nf4_quantize", "nf4_quantize_dq", "nf4_double_quant", "nf4_dequantize", "qlora_linear_fwd_workspace",
           "qlora_linear_fwd", "qlora_linear_bwd_workspace", "qlora_linear_bwd", "qlora_nf4_levels",
           "ql_status_string", "qlora_lora_down_workspace", "qlora_lora_down", "qlora_linear_fwd_t",
           "qlora_lora_grad_in_workspace", "qlora_lora_grad_in", "qlora_linear_dx", "qlora_merge",
           "q4_quantize", "q4_double_quant", "q4_dequantize", "q4_levels",
           "qlora_group_fwd_workspace", "qlora_group_fwd", "qlora_group_bwd_workspace", "qlora_group_bwd",
           "qlora_adamw_step", "ql_read_probe")


class QloraError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({lib().ql_status_string(status).decode()})")


def lib():
    """The loaded library; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_lora_blockwise_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        sig = {
            "nf4_quantize": ([P, I32, I64, I64, P, P, P], I32),
            "nf4_double_quant": ([P, I64, P, P, P], I32),
            "nf4_dequantize": ([P, P, P, I64, I64, P, P], I32),
            "nf4_quantize_dq": ([P, I32, I64, I64, P, P, P, P, P], I32),
            "qlora_linear_fwd_workspace": ([I64, I64, I64, I32], SZ),
            "qlora_linear_fwd": ([P, I64, I64, I64, P, P, P, P, P, I32, F32, P, P, P, SZ, P], I32),
            "qlora_linear_bwd_workspace": ([I64, I64, I64, I32], SZ),
            "qlora_linear_bwd": ([P, P, I64, I64, I64, P, P, P, P, P, I32, F32, P, P, P, P, P, SZ, P], I32),
            "qlora_nf4_levels": ([P], I32),
            "ql_status_string": ([I32], ctypes.c_char_p),
            "qlora_lora_down_workspace": ([I64, I64, I32], SZ),
            "qlora_lora_down": ([P, I64, I64, P, I32, P, P, SZ, P], I32),
            "qlora_linear_fwd_t": ([P, I64, I64, I64, P, P, P, P, P, I32, F32, P, P], I32),
            "qlora_lora_grad_in_workspace": ([I64, I64, I32], SZ),
            "qlora_lora_grad_in": ([P, I64, I64, P, I32, F32, P, P, SZ, P], I32),
            "qlora_linear_dx": ([P, I64, I64, I64, P, P, P, P, P, I32, P, P], I32),
            "qlora_merge": ([P, P, P, I64, I64, P, P, I32, F32, P, P], I32),
            "q4_quantize": ([P, I32, I64, I64, I32, P, P, P], I32),
            "q4_double_quant": ([P, I64, I32, P, P, P, P], I32),
            "q4_dequantize": ([P, I64, I64, I32, I32, P, P, P, P, P, P], I32),
            "q4_levels": ([I32, P], I32),
            "qlora_group_fwd_workspace": ([I64, I64, I64, I32, I32], SZ),
            "qlora_group_fwd": ([P, I64, I64, I64, I32, P, P, P, P, P, I32, F32, P, P, P, SZ, P], I32),
            "qlora_group_bwd_workspace": ([I64, I64, I64, I32, I32], SZ),
            "qlora_group_bwd": ([P, P, I64, I64, I64, I32, P, P, P, P, P, I32, F32, P, P, P, P, P, SZ, P], I32),
            "qlora_adamw_step": ([P, P, P, P, P, I64, F32, F32, F32, F32, F32, I64, P], I32),
            "ql_read_probe": ([P, I64, P, P], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t


def _check(fn, status):
    if status != 0:
        raise QloraError(fn, status)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def nf4_quantize(W, codes=None, absmax=None, stream=None):
    """Packed NF4 codes [rows, cols/2] (uint8) and fp32 absmax [rows*cols/64] of W [rows, cols]."""
    if W.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W must be float32 or bfloat16")
    _need(W, "W", W.dtype, 2)
    rows, cols = W.shape
    codes = _empty((rows, cols // 2), torch.uint8, W) if codes is None else _need(codes, "codes", torch.uint8)
    absmax = _empty((rows * cols // 64,), torch.float32, W) if absmax is None else _need(absmax, "absmax",
                                                                                        torch.float32)
    _check("nf4_quantize", lib().nf4_quantize(_ptr(W), QL_BF16 if W.dtype == torch.bfloat16 else QL_F32, rows, cols,
                                              _ptr(codes), _ptr(absmax), _stream(stream)))
    return codes, absmax


def nf4_quantize_dq(W, codes=None, c2=None, c1=None, absmax=None, stream=None):
    """Codes, c2 and c1 of W [rows, cols] in one pass (absmax written too when given a buffer or True)."""
    if W.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W must be float32 or bfloat16")
    _need(W, "W", W.dtype, 2)
    rows, cols = W.shape
    nb = rows * cols // 64
    codes = _empty((rows, cols // 2), torch.uint8, W) if codes is None else _need(codes, "codes", torch.uint8)
    c2 = _empty((nb,), torch.uint8, W) if c2 is None else _need(c2, "c2", torch.uint8)
    c1 = _empty(((nb + 255) // 256,), torch.float32, W) if c1 is None else _need(c1, "c1", torch.float32)
    if absmax is True:
        absmax = _empty((nb,), torch.float32, W)
    elif absmax is not None:
        _need(absmax, "absmax", torch.float32)
    _check("nf4_quantize_dq", lib().nf4_quantize_dq(_ptr(W), QL_BF16 if W.dtype == torch.bfloat16 else QL_F32, rows,
                                                    cols, _ptr(codes), _ptr(absmax), _ptr(c2), _ptr(c1),
                                                    _stream(stream)))
    return codes, c2, c1, absmax


def nf4_double_quant(absmax, c2=None, c1=None, stream=None):
    """E4M3FN codes c2 [n_blocks] (uint8) and fp32 group scales c1 [ceil(n_blocks/256)]."""
    _need(absmax, "absmax", torch.float32)
    nb = absmax.numel()
    c2 = _empty((nb,), torch.uint8, absmax) if c2 is None else _need(c2, "c2", torch.uint8)
    c1 = _empty(((nb + 255) // 256,), torch.float32, absmax) if c1 is None else _need(c1, "c1", torch.float32)
    _check("nf4_double_quant", lib().nf4_double_quant(_ptr(absmax), nb, _ptr(c2), _ptr(c1), _stream(stream)))
    return c2, c1


def read_probe(data, sink, stream=None):
    """One streaming read of the bytes of `data` (a measurement helper: the
    read-bandwidth ceiling for the decode forward); `sink` is an int32 [1]."""
    _need(sink, "sink", torch.int32)
    if not isinstance(data, torch.Tensor) or data.device.type != "cuda" or not data.is_contiguous():
        raise ValueError("data must be a contiguous GPU tensor")
    _check("ql_read_probe", lib().ql_read_probe(_ptr(data), data.numel() * data.element_size(), _ptr(sink),
                                                _stream(stream)))


def nf4_dequantize(codes, c2, c1, rows, cols, out=None, stream=None):
    """Bit-exact bf16 doubleDequant(c1, c2, W_NF4) [rows, cols]."""
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    out = _empty((rows, cols), torch.bfloat16, codes) if out is None else _need(out, "out", torch.bfloat16)
    _check("nf4_dequantize", lib().nf4_dequantize(_ptr(codes), _ptr(c2), _ptr(c1), rows, cols, _ptr(out),
                                                  _stream(stream)))
    return out


def _codebook(name):
    if name not in CODEBOOKS:
        raise ValueError(f"unknown code book {name!r} (one of {sorted(CODEBOOKS)})")
    return CODEBOOKS[name]


def _scale_code(name):
    if name not in SCALE_CODES:
        raise ValueError(f"unknown scale code {name!r} (one of {sorted(SCALE_CODES)})")
    return SCALE_CODES[name]


def q4_quantize(W, codebook="nf4", codes=None, absmax=None, stream=None):
    """Packed 4-bit codes [rows, cols/2] and fp32 absmax [rows*cols/64] with the given code book."""
    if W.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W must be float32 or bfloat16")
    _need(W, "W", W.dtype, 2)
    rows, cols = W.shape
    codes = _empty((rows, cols // 2), torch.uint8, W) if codes is None else _need(codes, "codes", torch.uint8)
    absmax = _empty((rows * cols // 64,), torch.float32, W) if absmax is None else _need(absmax, "absmax",
                                                                                        torch.float32)
    _check("q4_quantize", lib().q4_quantize(_ptr(W), QL_BF16 if W.dtype == torch.bfloat16 else QL_F32, rows, cols,
                                            _codebook(codebook), _ptr(codes), _ptr(absmax), _stream(stream)))
    return codes, absmax


def q4_double_quant(absmax, scale_code="groupmax", stream=None):
    """(c2 [n_blocks] uint8, c1 [groups] fp32, mu [groups] fp32 or None) for a scale code."""
    _need(absmax, "absmax", torch.float32)
    sc = _scale_code(scale_code)
    if sc == SCALE_CODES["absmax"]:
        raise ValueError("absmax scales need no second level")
    nb = absmax.numel()
    ng = (nb + 255) // 256
    c2 = _empty((nb,), torch.uint8, absmax)
    c1 = _empty((ng,), torch.float32, absmax)
    mu = _empty((ng,), torch.float32, absmax) if scale_code == "mean" else None
    _check("q4_double_quant", lib().q4_double_quant(_ptr(absmax), nb, sc, _ptr(c2), _ptr(c1),
                                                    _ptr(mu) if mu is not None else None, _stream(stream)))
    return c2, c1, mu


def q4_dequantize(codes, rows, cols, codebook="nf4", scale_code="groupmax", absmax=None, c2=None, c1=None, mu=None,
                  out=None, stream=None):
    """bf16 W' [rows, cols] from codes and the block scales of `scale_code`."""
    _need(codes, "codes", torch.uint8)
    for t, n, d in ((absmax, "absmax", torch.float32), (c2, "c2", torch.uint8), (c1, "c1", torch.float32),
                    (mu, "mu", torch.float32)):
        if t is not None:
            _need(t, n, d)
    out = _empty((rows, cols), torch.bfloat16, codes) if out is None else _need(out, "out", torch.bfloat16)
    p = lambda t: _ptr(t) if t is not None else None
    _check("q4_dequantize", lib().q4_dequantize(_ptr(codes), rows, cols, _codebook(codebook), _scale_code(scale_code),
                                                p(absmax), p(c2), p(c1), p(mu), _ptr(out), _stream(stream)))
    return out


def q4_levels(codebook="nf4"):
    """The 16 fp32 levels of a code book compiled into the library (host call)."""
    buf = (ctypes.c_float * 16)()
    _check("q4_levels", lib().q4_levels(_codebook(codebook), ctypes.cast(buf, ctypes.c_void_p)))
    return list(buf)


def qlora_merge(codes, c2, c1, N, K, L1, L2, lora_scale=1.0, out=None, stream=None):
    """Merged bf16 weight W' + lora_scale (L1 L2)^T [N, K], rounded once."""
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    _need(L1, "L1", torch.bfloat16); _need(L2, "L2", torch.bfloat16)
    r = L1.shape[1]
    if tuple(L1.shape) != (K, r) or tuple(L2.shape) != (r, N):
        raise ValueError(f"qlora_merge: L1 {tuple(L1.shape)} / L2 {tuple(L2.shape)} do not match N={N}, K={K}")
    out = _empty((N, K), torch.bfloat16, codes) if out is None else _need(out, "out", torch.bfloat16)
    _check("qlora_merge", lib().qlora_merge(_ptr(codes), _ptr(c2), _ptr(c1), N, K, _ptr(L1), _ptr(L2), r,
                                            float(lora_scale), _ptr(out), _stream(stream)))
    return out


def qlora_linear_fwd_workspace(M, K, N, r):
    return int(lib().qlora_linear_fwd_workspace(M, K, N, r))


def qlora_linear_bwd_workspace(M, K, N, r):
    return int(lib().qlora_linear_bwd_workspace(M, K, N, r))


def _workspace(nbytes, like, workspace):
    if workspace is not None:
        return _need(workspace, "workspace", torch.uint8)
    return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=like.device)


def qlora_linear_fwd(X, codes, c2, c1, N, L1, L2, lora_scale=1.0, Y=None, T_out=None, workspace=None,
                     stream=None):
    """Y = bf16(X W'^T + s T L2), T = bf16(X L1).  Returns (Y, T_out or None).

    T_out: None (not returned), True (allocated here) or a bf16 [M, r] tensor."""
    _need(X, "X", torch.bfloat16, 2); _need(L1, "L1", torch.bfloat16, 2); _need(L2, "L2", torch.bfloat16, 2)
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    M, K = X.shape
    r = L1.shape[1]
    Y = _empty((M, N), torch.bfloat16, X) if Y is None else _need(Y, "Y", torch.bfloat16)
    if T_out is True:
        T_out = _empty((M, r), torch.bfloat16, X)
    elif T_out is not None:
        _need(T_out, "T_out", torch.bfloat16)
    ws = _workspace(qlora_linear_fwd_workspace(M, K, N, r), X, workspace)
    _check("qlora_linear_fwd", lib().qlora_linear_fwd(
        _ptr(X), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(Y), _ptr(T_out), _ptr(ws), ws.numel(), _stream(stream)))
    return Y, T_out


def qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, lora_scale=1.0, T=None, dX=True, dL1=None, dL2=None,
                     workspace=None, stream=None):
    """(dX or None, dL1 fp32 [K, r], dL2 fp32 [r, N]); the frozen base gets no gradient.

    dX: True (allocated here), False/None (skipped) or a bf16 [M, K] tensor."""
    _need(X, "X", torch.bfloat16, 2); _need(dY, "dY", torch.bfloat16, 2)
    _need(L1, "L1", torch.bfloat16, 2); _need(L2, "L2", torch.bfloat16, 2)
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    M, K = X.shape
    N = dY.shape[1]
    r = L1.shape[1]
    if T is not None:
        _need(T, "T", torch.bfloat16)
    if dX is True:
        dX = _empty((M, K), torch.bfloat16, X)
    elif dX is False:
        dX = None
    elif dX is not None:
        _need(dX, "dX", torch.bfloat16)
    dL1 = _empty((K, r), torch.float32, X) if dL1 is None else _need(dL1, "dL1", torch.float32)
    dL2 = _empty((r, N), torch.float32, X) if dL2 is None else _need(dL2, "dL2", torch.float32)
    ws = _workspace(qlora_linear_bwd_workspace(M, K, N, r), X, workspace)
    _check("qlora_linear_bwd", lib().qlora_linear_bwd(
        _ptr(X), _ptr(dY), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream(stream)))
    return dX, dL1, dL2


def qlora_group_fwd(X, codes, c2, c1, N, G, L1, L2, lora_scale=1.0, Y=None, T_out=None, workspace=None,
                    stream=None):
    """G stacked linears sharing X (W [G N, K] quantized as one; L1 [G, K, r], L2 [G, r, N]):
    Y [M, G N] = [Y_0 | ... | Y_{G-1}].  Returns (Y, T_out [G, M, r] or None)."""
    _need(X, "X", torch.bfloat16, 2); _need(L1, "L1", torch.bfloat16, 3); _need(L2, "L2", torch.bfloat16, 3)
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    M, K = X.shape
    r = L1.shape[2]
    if tuple(L1.shape) != (G, K, r) or tuple(L2.shape) != (G, r, N):
        raise ValueError(f"qlora_group_fwd: L1 {tuple(L1.shape)} / L2 {tuple(L2.shape)} vs G={G}, K={K}, N={N}")
    Y = _empty((M, G * N), torch.bfloat16, X) if Y is None else _need(Y, "Y", torch.bfloat16)
    if T_out is True:
        T_out = _empty((G, M, r), torch.bfloat16, X)
    elif T_out is not None:
        _need(T_out, "T_out", torch.bfloat16)
    ws = _workspace(int(lib().qlora_group_fwd_workspace(M, K, N, G, r)), X, workspace)
    _check("qlora_group_fwd", lib().qlora_group_fwd(
        _ptr(X), M, K, N, G, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(Y), _ptr(T_out), _ptr(ws), ws.numel(), _stream(stream)))
    return Y, T_out


def qlora_group_bwd(X, dY, codes, c2, c1, G, L1, L2, lora_scale=1.0, T=None, dX=True, dL1=None, dL2=None,
                    workspace=None, stream=None):
    """(dX or None, dL1 [G, K, r], dL2 [G, r, N]) of G stacked linears; dX sums the segments, rounded once."""
    _need(X, "X", torch.bfloat16, 2); _need(dY, "dY", torch.bfloat16, 2)
    _need(L1, "L1", torch.bfloat16, 3); _need(L2, "L2", torch.bfloat16, 3)
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    M, K = X.shape
    N = dY.shape[1] // G
    r = L1.shape[2]
    if T is not None:
        _need(T, "T", torch.bfloat16)
    if dX is True:
        dX = _empty((M, K), torch.bfloat16, X)
    elif dX is False:
        dX = None
    elif dX is not None:
        _need(dX, "dX", torch.bfloat16)
    dL1 = _empty((G, K, r), torch.float32, X) if dL1 is None else _need(dL1, "dL1", torch.float32)
    dL2 = _empty((G, r, N), torch.float32, X) if dL2 is None else _need(dL2, "dL2", torch.float32)
    ws = _workspace(int(lib().qlora_group_bwd_workspace(M, K, N, G, r)), X, workspace)
    _check("qlora_group_bwd", lib().qlora_group_bwd(
        _ptr(X), _ptr(dY), M, K, N, G, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream(stream)))
    return dX, dL1, dL2


def qlora_adamw_step(param, exp_avg, exp_avg_sq, grad, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.0, param_bf16=None, stream=None):
    """One AdamW step over flat fp32 tensors (in place); param_bf16 (optional) gets bf16(param)."""
    for t, n in ((param, "param"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        _need(t, n, torch.float32)
    n = param.numel()
    if any(t.numel() != n for t in (exp_avg, exp_avg_sq, grad)):
        raise ValueError("qlora_adamw_step: all state tensors must have the parameter's size")
    if param_bf16 is not None:
        _need(param_bf16, "param_bf16", torch.bfloat16)
        if param_bf16.numel() != n:
            raise ValueError("qlora_adamw_step: param_bf16 must have the parameter's size")
    _check("qlora_adamw_step", lib().qlora_adamw_step(
        _ptr(param), _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(grad), _ptr(param_bf16), n, float(lr), float(beta1),
        float(beta2), float(eps), float(weight_decay), int(step), _stream(stream)))


def qlora_nf4_levels():
    """The 16 fp32 NF4 levels compiled into the library (host call, no GPU)."""
    buf = (ctypes.c_float * 16)()
    _check("qlora_nf4_levels", lib().qlora_nf4_levels(ctypes.cast(buf, ctypes.c_void_p)))
    return [float(v) for v in buf]


def ql_status_string(status):
    return lib().ql_status_string(int(status)).decode()


# --- stage entry points -------------------------------------------------------

def qlora_lora_down(X, L1, T=None, workspace=None, stream=None):
    """T = bf16(X L1) [M, r]."""
    _need(X, "X", torch.bfloat16, 2); _need(L1, "L1", torch.bfloat16, 2)
    M, K = X.shape
    r = L1.shape[1]
    T = _empty((M, r), torch.bfloat16, X) if T is None else _need(T, "T", torch.bfloat16)
    ws = _workspace(int(lib().qlora_lora_down_workspace(M, K, r)), X, workspace)
    _check("qlora_lora_down", lib().qlora_lora_down(_ptr(X), M, K, _ptr(L1), r, _ptr(T), _ptr(ws), ws.numel(),
                                                    _stream(stream)))
    return T


def qlora_linear_fwd_t(X, codes, c2, c1, N, T, L2, lora_scale=1.0, Y=None, stream=None):
    """Y = bf16(X W'^T + s T L2) given T (one kernel)."""
    _need(X, "X", torch.bfloat16, 2); _need(T, "T", torch.bfloat16, 2); _need(L2, "L2", torch.bfloat16, 2)
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    M, K = X.shape
    r = T.shape[1]
    Y = _empty((M, N), torch.bfloat16, X) if Y is None else _need(Y, "Y", torch.bfloat16)
    _check("qlora_linear_fwd_t", lib().qlora_linear_fwd_t(
        _ptr(X), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(T), _ptr(L2), r, float(lora_scale), _ptr(Y),
        _stream(stream)))
    return Y


def qlora_lora_grad_in(dY, L2, lora_scale=1.0, G=None, workspace=None, stream=None):
    """G = bf16(s dY L2^T) [M, r]."""
    _need(dY, "dY", torch.bfloat16, 2); _need(L2, "L2", torch.bfloat16, 2)
    M, N = dY.shape
    r = L2.shape[0]
    G = _empty((M, r), torch.bfloat16, dY) if G is None else _need(G, "G", torch.bfloat16)
    ws = _workspace(int(lib().qlora_lora_grad_in_workspace(M, N, r)), dY, workspace)
    _check("qlora_lora_grad_in", lib().qlora_lora_grad_in(_ptr(dY), M, N, _ptr(L2), r, float(lora_scale), _ptr(G),
                                                          _ptr(ws), ws.numel(), _stream(stream)))
    return G


def qlora_linear_dx(dY, codes, c2, c1, K, G, L1, dX=None, stream=None):
    """dX = bf16(dY W' + G L1^T) given G (one kernel)."""
    _need(dY, "dY", torch.bfloat16, 2); _need(G, "G", torch.bfloat16, 2); _need(L1, "L1", torch.bfloat16, 2)
    _need(codes, "codes", torch.uint8); _need(c2, "c2", torch.uint8); _need(c1, "c1", torch.float32)
    M, N = dY.shape
    r = G.shape[1]
    dX = _empty((M, K), torch.bfloat16, dY) if dX is None else _need(dX, "dX", torch.bfloat16)
    _check("qlora_linear_dx", lib().qlora_linear_dx(
        _ptr(dY), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(G), _ptr(L1), r, _ptr(dX), _stream(stream)))
    return dX
