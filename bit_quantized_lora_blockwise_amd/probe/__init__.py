"""ctypes binding of libqlprobe.so (include/qlprobe.h): measurement helpers
that the benchmark puts next to the layer's kernels -- a plain streaming read
of a byte range and an empty grid.  Not part of the method or of libqlora.so."""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "libqlprobe.so")
_lib = None
EXPORTS = ("ql_read_probe", "ql_empty_probe")


def lib():
    """The loaded probe library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_lora_blockwise_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.ql_read_probe.argtypes, L.ql_read_probe.restype = [P, I64, I32, P, P], I32
        L.ql_empty_probe.argtypes, L.ql_empty_probe.restype = [I64, I32, P], I32
        _lib = L
    return _lib


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def read_probe(data, sink, loads=4, stream=None):
    """One streaming read of the bytes of `data` (contiguous GPU tensor); `sink`
    is an int32 [1] GPU tensor; `loads` 16-byte loads in flight per thread."""
    if not isinstance(data, torch.Tensor) or data.device.type != "cuda" or not data.is_contiguous():
        raise ValueError("data must be a contiguous GPU tensor")
    if not isinstance(sink, torch.Tensor) or sink.dtype != torch.int32 or sink.device.type != "cuda":
        raise ValueError("sink must be an int32 GPU tensor")
    st = lib().ql_read_probe(ctypes.c_void_p(data.data_ptr()), data.numel() * data.element_size(), int(loads),
                             ctypes.c_void_p(sink.data_ptr()), _stream(stream))
    if st != 0:
        raise RuntimeError(f"ql_read_probe: status {st}")


def empty_probe(groups, threads=256, stream=None):
    """Launch an empty grid of `groups` work groups of `threads` threads."""
    st = lib().ql_empty_probe(int(groups), int(threads), _stream(stream))
    if st != 0:
        raise RuntimeError(f"ql_empty_probe: status {st}")
