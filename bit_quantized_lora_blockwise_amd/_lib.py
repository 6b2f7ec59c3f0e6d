"""ctypes binding of libqlora.so: argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/qlora.h for the contract).  Tensors are torch tensors on the GPU; the
binding checks dtype, shape or element count, contiguity and device of every
tensor (inputs and caller-supplied outputs), allocates missing outputs with torch,
passes raw pointers and the current HIP stream, and raises QloraError on a
non-zero status.  All computation happens in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

# QLORA_LIBRARY selects another build of the same library (the host-sanitized
# one that the sanitizer test runs the ABI checks against); default: in-tree.
_LIB_PATH = os.environ.get("QLORA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora.so")
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
           "qlora_adamw_step", "qlora_linear_fwd_noalloc",
           "lora_linear_fwd", "lora_linear_bwd", "lora_linear_fwd_t", "lora_linear_dx")


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
            "qlora_linear_fwd_noalloc": ([P, I64, I64, I64, P, P, P, P, P, I32, F32, P, P, P], I32),
            "lora_linear_fwd": ([P, I64, I64, I64, P, P, P, I32, F32, P, P, P, SZ, P], I32),
            "lora_linear_bwd": ([P, P, I64, I64, I64, P, P, P, I32, F32, P, P, P, P, P, SZ, P], I32),
            "lora_linear_fwd_t": ([P, I64, I64, I64, P, P, P, I32, F32, P, P], I32),
            "lora_linear_dx": ([P, I64, I64, I64, P, P, P, I32, P, P], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _ptr(t):
    """Device address of a tensor argument (None -> NULL).  Every tensor reaches
    the library through here, after all size checks: this is the device check."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"every tensor argument must be on the GPU (got a {t.device} tensor of shape "
                         f"{tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, ndim=None, shape=None, numel=None):
    """Check a tensor argument: type, dtype, rank, shape or element count and
    contiguity (the device is checked when its pointer is taken, after every
    size check of the call)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _packed(codes, c2, c1, rows, cols):
    """The packed base of a [rows, cols] weight: codes rows*cols/2 bytes, c2 one
    byte per block of 64, c1 one fp32 per group of 256 blocks."""
    if rows <= 0 or cols <= 0 or cols % 64:
        raise ValueError(f"weight shape [{rows}, {cols}]: sizes must be > 0 and cols a multiple of 64")
    nb = rows * cols // 64
    _need(codes, "codes", torch.uint8, numel=rows * cols // 2)
    _need(c2, "c2", torch.uint8, numel=nb)
    _need(c1, "c1", torch.float32, numel=(nb + 255) // 256)


def _out(t, name, dtype, shape, like):
    """An output: allocated here when None, else checked to have exactly the
    element count of `shape` (any contiguous layout of that many elements)."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    n = 1
    for d in shape:
        n *= d
    return _need(t, name, dtype, numel=n)


def _check(fn, status):
    if status != 0:
        raise QloraError(fn, status)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _wdtype(W):
    if not isinstance(W, torch.Tensor) or W.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W must be a float32 or bfloat16 torch.Tensor")
    return QL_BF16 if W.dtype == torch.bfloat16 else QL_F32


def nf4_quantize(W, codes=None, absmax=None, stream=None):
    """Packed NF4 codes [rows, cols/2] (uint8) and fp32 absmax [rows*cols/64] of W [rows, cols]."""
    dt = _wdtype(W)
    _need(W, "W", W.dtype, ndim=2)
    rows, cols = W.shape
    codes = _out(codes, "codes", torch.uint8, (rows, cols // 2), W)
    absmax = _out(absmax, "absmax", torch.float32, (rows * cols // 64,), W)
    _check("nf4_quantize", lib().nf4_quantize(_ptr(W), dt, rows, cols, _ptr(codes), _ptr(absmax), _stream(stream)))
    return codes, absmax


def nf4_quantize_dq(W, codes=None, c2=None, c1=None, absmax=None, stream=None):
    """Codes, c2 and c1 of W [rows, cols] in one pass (absmax written too when given a buffer or True)."""
    dt = _wdtype(W)
    _need(W, "W", W.dtype, ndim=2)
    rows, cols = W.shape
    nb = rows * cols // 64
    codes = _out(codes, "codes", torch.uint8, (rows, cols // 2), W)
    c2 = _out(c2, "c2", torch.uint8, (nb,), W)
    c1 = _out(c1, "c1", torch.float32, ((nb + 255) // 256,), W)
    if absmax is True:
        absmax = _empty((nb,), torch.float32, W)
    elif absmax is not None:
        _out(absmax, "absmax", torch.float32, (nb,), W)
    _check("nf4_quantize_dq", lib().nf4_quantize_dq(_ptr(W), dt, rows, cols, _ptr(codes), _ptr(absmax), _ptr(c2),
                                                    _ptr(c1), _stream(stream)))
    return codes, c2, c1, absmax


def nf4_double_quant(absmax, c2=None, c1=None, stream=None):
    """E4M3FN codes c2 [n_blocks] (uint8) and fp32 group scales c1 [ceil(n_blocks/256)]."""
    _need(absmax, "absmax", torch.float32)
    nb = absmax.numel()
    c2 = _out(c2, "c2", torch.uint8, (nb,), absmax)
    c1 = _out(c1, "c1", torch.float32, ((nb + 255) // 256,), absmax)
    _check("nf4_double_quant", lib().nf4_double_quant(_ptr(absmax), nb, _ptr(c2), _ptr(c1), _stream(stream)))
    return c2, c1


def nf4_dequantize(codes, c2, c1, rows, cols, out=None, stream=None):
    """Bit-exact bf16 doubleDequant(c1, c2, W_NF4) [rows, cols]."""
    _packed(codes, c2, c1, rows, cols)
    out = _out(out, "out", torch.bfloat16, (rows, cols), codes)
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
    dt = _wdtype(W)
    _need(W, "W", W.dtype, ndim=2)
    rows, cols = W.shape
    codes = _out(codes, "codes", torch.uint8, (rows, cols // 2), W)
    absmax = _out(absmax, "absmax", torch.float32, (rows * cols // 64,), W)
    _check("q4_quantize", lib().q4_quantize(_ptr(W), dt, rows, cols, _codebook(codebook), _ptr(codes), _ptr(absmax),
                                            _stream(stream)))
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
    if rows <= 0 or cols <= 0 or cols % 64:
        raise ValueError(f"weight shape [{rows}, {cols}]: sizes must be > 0 and cols a multiple of 64")
    nb = rows * cols // 64
    ng = (nb + 255) // 256
    _need(codes, "codes", torch.uint8, numel=rows * cols // 2)
    for t, n, d, cnt in ((absmax, "absmax", torch.float32, nb), (c2, "c2", torch.uint8, nb),
                         (c1, "c1", torch.float32, ng), (mu, "mu", torch.float32, ng)):
        if t is not None:
            _need(t, n, d, numel=cnt)
    out = _out(out, "out", torch.bfloat16, (rows, cols), codes)
    p = lambda t: _ptr(t) if t is not None else None
    _check("q4_dequantize", lib().q4_dequantize(_ptr(codes), rows, cols, _codebook(codebook), _scale_code(scale_code),
                                                p(absmax), p(c2), p(c1), p(mu), _ptr(out), _stream(stream)))
    return out


def q4_levels(codebook="nf4"):
    """The 16 fp32 levels of a code book compiled into the library (host call)."""
    buf = (ctypes.c_float * 16)()
    _check("q4_levels", lib().q4_levels(_codebook(codebook), ctypes.cast(buf, ctypes.c_void_p)))
    return list(buf)


def _rank(L1, K):
    """Rank r of the adapter from L1 [K, r]."""
    _need(L1, "L1", torch.bfloat16, ndim=2)
    if L1.shape[0] != K:
        raise ValueError(f"L1 must have {K} rows, got {tuple(L1.shape)}")
    return L1.shape[1]


def qlora_merge(codes, c2, c1, N, K, L1, L2, lora_scale=1.0, out=None, stream=None):
    """Merged bf16 weight W' + lora_scale (L1 L2)^T [N, K], rounded once."""
    _packed(codes, c2, c1, N, K)
    r = _rank(L1, K)
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    out = _out(out, "out", torch.bfloat16, (N, K), codes)
    _check("qlora_merge", lib().qlora_merge(_ptr(codes), _ptr(c2), _ptr(c1), N, K, _ptr(L1), _ptr(L2), r,
                                            float(lora_scale), _ptr(out), _stream(stream)))
    return out


def qlora_linear_fwd_workspace(M, K, N, r):
    return int(lib().qlora_linear_fwd_workspace(M, K, N, r))


def qlora_linear_bwd_workspace(M, K, N, r):
    return int(lib().qlora_linear_bwd_workspace(M, K, N, r))


def _workspace(nbytes, like, workspace):
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace must hold at least {nbytes} bytes, got {workspace.numel()}")
        return workspace
    return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=like.device)


def _opt_out(t, name, dtype, shape, like):
    """Optional output: True -> allocated here, None/False -> absent, else checked."""
    if t is True:
        return _empty(shape, dtype, like)
    if t is None or t is False:
        return None
    return _out(t, name, dtype, shape, like)


def qlora_linear_fwd(X, codes, c2, c1, N, L1, L2, lora_scale=1.0, Y=None, T_out=None, workspace=None,
                     stream=None):
    """Y = bf16(X W'^T + s T L2), T = bf16(X L1).  Returns (Y, T_out or None).

    T_out: None (not returned), True (allocated here) or a bf16 [M, r] tensor."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _packed(codes, c2, c1, N, K)
    r = _rank(L1, K)
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    Y = _out(Y, "Y", torch.bfloat16, (M, N), X)
    T_out = _opt_out(T_out, "T_out", torch.bfloat16, (M, r), X)
    ws = _workspace(qlora_linear_fwd_workspace(M, K, N, r), X, workspace)
    _check("qlora_linear_fwd", lib().qlora_linear_fwd(
        _ptr(X), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(Y), _ptr(T_out), _ptr(ws), ws.numel(), _stream(stream)))
    return Y, T_out


NOALLOC_SCRATCH_BYTES = 16777216      # QL_NOALLOC_SCRATCH_BYTES of include/qlora.h


def qlora_linear_fwd_noalloc(X, codes, c2, c1, N, L1, L2, lora_scale=1.0, Y=None, T_out=None, stream=None):
    """qlora_linear_fwd with its scratch in the library's per-GPU static array
    (for callers that cannot allocate; calls that overlap on one GPU race).
    Returns (Y, T_out or None); Y and T_out must be supplied to allocate nothing."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _packed(codes, c2, c1, N, K)
    r = _rank(L1, K)
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    Y = _out(Y, "Y", torch.bfloat16, (M, N), X)
    T_out = _opt_out(T_out, "T_out", torch.bfloat16, (M, r), X)
    _check("qlora_linear_fwd_noalloc", lib().qlora_linear_fwd_noalloc(
        _ptr(X), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(Y), _ptr(T_out), _stream(stream)))
    return Y, T_out


def qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, lora_scale=1.0, T=None, dX=True, dL1=None, dL2=None,
                     workspace=None, stream=None):
    """(dX or None, dL1 fp32 [K, r], dL2 fp32 [r, N]); the frozen base gets no gradient.

    dX: True (allocated here), False/None (skipped) or a bf16 [M, K] tensor."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _need(dY, "dY", torch.bfloat16, ndim=2)
    if dY.shape[0] != M:
        raise ValueError(f"dY must have {M} rows, got {tuple(dY.shape)}")
    N = dY.shape[1]
    _packed(codes, c2, c1, N, K)
    r = _rank(L1, K)
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    if T is not None:
        _need(T, "T", torch.bfloat16, numel=M * r)
    dX = _opt_out(dX, "dX", torch.bfloat16, (M, K), X)
    dL1 = _out(dL1, "dL1", torch.float32, (K, r), X)
    dL2 = _out(dL2, "dL2", torch.float32, (r, N), X)
    ws = _workspace(qlora_linear_bwd_workspace(M, K, N, r), X, workspace)
    _check("qlora_linear_bwd", lib().qlora_linear_bwd(
        _ptr(X), _ptr(dY), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream(stream)))
    return dX, dL1, dL2


def _group_adapters(L1, L2, G, K, N):
    _need(L1, "L1", torch.bfloat16, ndim=3)
    if L1.shape[0] != G or L1.shape[1] != K:
        raise ValueError(f"L1 must have shape ({G}, {K}, r), got {tuple(L1.shape)}")
    r = L1.shape[2]
    _need(L2, "L2", torch.bfloat16, shape=(G, r, N))
    return r


def qlora_group_fwd(X, codes, c2, c1, N, G, L1, L2, lora_scale=1.0, Y=None, T_out=None, workspace=None,
                    stream=None):
    """G stacked linears sharing X (W [G N, K] quantized as one; L1 [G, K, r], L2 [G, r, N]):
    Y [M, G N] = [Y_0 | ... | Y_{G-1}].  Returns (Y, T_out [G, M, r] or None)."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _packed(codes, c2, c1, G * N, K)
    r = _group_adapters(L1, L2, G, K, N)
    Y = _out(Y, "Y", torch.bfloat16, (M, G * N), X)
    T_out = _opt_out(T_out, "T_out", torch.bfloat16, (G, M, r), X)
    ws = _workspace(int(lib().qlora_group_fwd_workspace(M, K, N, G, r)), X, workspace)
    _check("qlora_group_fwd", lib().qlora_group_fwd(
        _ptr(X), M, K, N, G, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(Y), _ptr(T_out), _ptr(ws), ws.numel(), _stream(stream)))
    return Y, T_out


def qlora_group_bwd(X, dY, codes, c2, c1, G, L1, L2, lora_scale=1.0, T=None, dX=True, dL1=None, dL2=None,
                    workspace=None, stream=None):
    """(dX or None, dL1 [G, K, r], dL2 [G, r, N]) of G stacked linears; dX sums the segments, rounded once."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _need(dY, "dY", torch.bfloat16, ndim=2)
    if dY.shape[0] != M or dY.shape[1] % G:
        raise ValueError(f"dY must have {M} rows and a multiple of G={G} columns, got {tuple(dY.shape)}")
    N = dY.shape[1] // G
    _packed(codes, c2, c1, G * N, K)
    r = _group_adapters(L1, L2, G, K, N)
    if T is not None:
        _need(T, "T", torch.bfloat16, numel=G * M * r)
    dX = _opt_out(dX, "dX", torch.bfloat16, (M, K), X)
    dL1 = _out(dL1, "dL1", torch.float32, (G, K, r), X)
    dL2 = _out(dL2, "dL2", torch.float32, (G, r, N), X)
    ws = _workspace(int(lib().qlora_group_bwd_workspace(M, K, N, G, r)), X, workspace)
    _check("qlora_group_bwd", lib().qlora_group_bwd(
        _ptr(X), _ptr(dY), M, K, N, G, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(L1), _ptr(L2), r, float(lora_scale),
        _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream(stream)))
    return dX, dL1, dL2


def qlora_adamw_step(param, exp_avg, exp_avg_sq, grad, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.0, param_bf16=None, stream=None):
    """One AdamW step over flat fp32 tensors (in place); param_bf16 (optional) gets bf16(param)."""
    _need(param, "param", torch.float32)
    n = param.numel()
    for t, name in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        _need(t, name, torch.float32, numel=n)
    if param_bf16 is not None:
        _need(param_bf16, "param_bf16", torch.bfloat16, numel=n)
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
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    r = _rank(L1, K)
    T = _out(T, "T", torch.bfloat16, (M, r), X)
    ws = _workspace(int(lib().qlora_lora_down_workspace(M, K, r)), X, workspace)
    _check("qlora_lora_down", lib().qlora_lora_down(_ptr(X), M, K, _ptr(L1), r, _ptr(T), _ptr(ws), ws.numel(),
                                                    _stream(stream)))
    return T


def qlora_linear_fwd_t(X, codes, c2, c1, N, T, L2, lora_scale=1.0, Y=None, stream=None):
    """Y = bf16(X W'^T + s T L2) given T (one kernel)."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _packed(codes, c2, c1, N, K)
    _need(T, "T", torch.bfloat16, ndim=2)
    if T.shape[0] != M:
        raise ValueError(f"T must have {M} rows, got {tuple(T.shape)}")
    r = T.shape[1]
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    Y = _out(Y, "Y", torch.bfloat16, (M, N), X)
    _check("qlora_linear_fwd_t", lib().qlora_linear_fwd_t(
        _ptr(X), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(T), _ptr(L2), r, float(lora_scale), _ptr(Y),
        _stream(stream)))
    return Y


def qlora_lora_grad_in(dY, L2, lora_scale=1.0, G=None, workspace=None, stream=None):
    """G = bf16(s dY L2^T) [M, r]."""
    _need(dY, "dY", torch.bfloat16, ndim=2)
    M, N = dY.shape
    _need(L2, "L2", torch.bfloat16, ndim=2)
    if L2.shape[1] != N:
        raise ValueError(f"L2 must have {N} columns, got {tuple(L2.shape)}")
    r = L2.shape[0]
    G = _out(G, "G", torch.bfloat16, (M, r), dY)
    ws = _workspace(int(lib().qlora_lora_grad_in_workspace(M, N, r)), dY, workspace)
    _check("qlora_lora_grad_in", lib().qlora_lora_grad_in(_ptr(dY), M, N, _ptr(L2), r, float(lora_scale), _ptr(G),
                                                          _ptr(ws), ws.numel(), _stream(stream)))
    return G


def qlora_linear_dx(dY, codes, c2, c1, K, G, L1, dX=None, stream=None):
    """dX = bf16(dY W' + G L1^T) given G (one kernel)."""
    _need(dY, "dY", torch.bfloat16, ndim=2)
    M, N = dY.shape
    _packed(codes, c2, c1, N, K)
    _need(G, "G", torch.bfloat16, ndim=2)
    if G.shape[0] != M:
        raise ValueError(f"G must have {M} rows, got {tuple(G.shape)}")
    r = G.shape[1]
    _need(L1, "L1", torch.bfloat16, shape=(K, r))
    dX = _out(dX, "dX", torch.bfloat16, (M, K), dY)
    _check("qlora_linear_dx", lib().qlora_linear_dx(
        _ptr(dY), M, K, N, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(G), _ptr(L1), r, _ptr(dX), _stream(stream)))
    return dX


# --- LoRA over a bf16 base (same GEMM kernels, bf16 weight) --------------------

def _bf16_weight(W, N, K):
    return _need(W, "W", torch.bfloat16, shape=(N, K))


def lora_linear_fwd(X, W, L1, L2, lora_scale=1.0, Y=None, T_out=None, workspace=None, stream=None):
    """Y = bf16(X W^T + s T L2), T = bf16(X L1) with a bf16 base W [N, K]."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _need(W, "W", torch.bfloat16, ndim=2)
    N = W.shape[0]
    _bf16_weight(W, N, K)
    r = _rank(L1, K)
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    Y = _out(Y, "Y", torch.bfloat16, (M, N), X)
    T_out = _opt_out(T_out, "T_out", torch.bfloat16, (M, r), X)
    ws = _workspace(qlora_linear_fwd_workspace(M, K, N, r), X, workspace)
    _check("lora_linear_fwd", lib().lora_linear_fwd(
        _ptr(X), M, K, N, _ptr(W), _ptr(L1), _ptr(L2), r, float(lora_scale), _ptr(Y), _ptr(T_out), _ptr(ws),
        ws.numel(), _stream(stream)))
    return Y, T_out


def lora_linear_bwd(X, dY, W, L1, L2, lora_scale=1.0, T=None, dX=True, dL1=None, dL2=None, workspace=None,
                    stream=None):
    """(dX or None, dL1 fp32 [K, r], dL2 fp32 [r, N]) with a bf16 base W [N, K] (no gradient for W)."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _need(dY, "dY", torch.bfloat16, ndim=2)
    if dY.shape[0] != M:
        raise ValueError(f"dY must have {M} rows, got {tuple(dY.shape)}")
    N = dY.shape[1]
    _bf16_weight(W, N, K)
    r = _rank(L1, K)
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    if T is not None:
        _need(T, "T", torch.bfloat16, numel=M * r)
    dX = _opt_out(dX, "dX", torch.bfloat16, (M, K), X)
    dL1 = _out(dL1, "dL1", torch.float32, (K, r), X)
    dL2 = _out(dL2, "dL2", torch.float32, (r, N), X)
    ws = _workspace(qlora_linear_bwd_workspace(M, K, N, r), X, workspace)
    _check("lora_linear_bwd", lib().lora_linear_bwd(
        _ptr(X), _ptr(dY), M, K, N, _ptr(W), _ptr(L1), _ptr(L2), r, float(lora_scale), _ptr(T), _ptr(dX),
        _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream(stream)))
    return dX, dL1, dL2


def lora_linear_fwd_t(X, W, T, L2, lora_scale=1.0, Y=None, stream=None):
    """Y = bf16(X W^T + s T L2) given T, bf16 base W [N, K] (one kernel)."""
    _need(X, "X", torch.bfloat16, ndim=2)
    M, K = X.shape
    _need(W, "W", torch.bfloat16, ndim=2)
    N = W.shape[0]
    _bf16_weight(W, N, K)
    _need(T, "T", torch.bfloat16, ndim=2)
    if T.shape[0] != M:
        raise ValueError(f"T must have {M} rows, got {tuple(T.shape)}")
    r = T.shape[1]
    _need(L2, "L2", torch.bfloat16, shape=(r, N))
    Y = _out(Y, "Y", torch.bfloat16, (M, N), X)
    _check("lora_linear_fwd_t", lib().lora_linear_fwd_t(
        _ptr(X), M, K, N, _ptr(W), _ptr(T), _ptr(L2), r, float(lora_scale), _ptr(Y), _stream(stream)))
    return Y


def lora_linear_dx(dY, W, G, L1, dX=None, stream=None):
    """dX = bf16(dY W + G L1^T) given G, bf16 base W [N, K] (one kernel)."""
    _need(dY, "dY", torch.bfloat16, ndim=2)
    M, N = dY.shape
    _need(W, "W", torch.bfloat16, ndim=2)
    K = W.shape[1]
    _bf16_weight(W, N, K)
    _need(G, "G", torch.bfloat16, ndim=2)
    if G.shape[0] != M:
        raise ValueError(f"G must have {M} rows, got {tuple(G.shape)}")
    r = G.shape[1]
    _need(L1, "L1", torch.bfloat16, shape=(K, r))
    dX = _out(dX, "dX", torch.bfloat16, (M, K), dY)
    _check("lora_linear_dx", lib().lora_linear_dx(
        _ptr(dY), M, K, N, _ptr(W), _ptr(G), _ptr(L1), r, _ptr(dX), _stream(stream)))
    return dX
