"""ctypes binding over libbitlinear_probes.so (include/bitlinear_probes.h).

Two measurement kernels, apart from the forward path: a streaming read of
device memory and a loop of int8 matrix-core operations.  They measure the
GPU's achievable ceilings, against which the decode (memory-bound) and
prefill (matrix-core-bound) kernels are reported.  Raises ImportError if the
library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitlinear_probes.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_gemm_bitlinear_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
_lib.blprobe_stream_read.restype = ctypes.c_int
_lib.blprobe_stream_read.argtypes = [_vp, _i64, _vp, _vp]
_lib.blprobe_lut_decode_acc.restype = ctypes.c_int
_lib.blprobe_lut_decode_acc.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp]
_lib.blprobe_mfma_i8.restype = ctypes.c_int
_lib.blprobe_mfma_i8.argtypes = [_i64, _i32, _i32, _vp, _vp]

OPS_PER_ROUND_PER_WG = 65536 * 8 * 4  # eight 32x32x32 int8 operations per wave, four waves
SINK_WORDS = 256  # BLPROBE_SINK_WORDS


def lib() -> ctypes.CDLL:
    return _lib


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """XOR of every 32-bit word of `buf` into the SINK_WORDS int32s of `sink`
    (zeroed by the caller; their XOR is the buffer's)."""
    assert buf.is_cuda and buf.is_contiguous() and sink.dtype == torch.int32
    assert sink.numel() >= SINK_WORDS
    st = _lib.blprobe_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                  ctypes.c_void_p(sink.data_ptr()), _stream(buf.device))
    if st != 0:
        raise RuntimeError(f"blprobe_stream_read failed ({st})")


def lut_decode_acc(q: torch.Tensor, tiled: torch.Tensor, out: torch.Tensor | None = None):
    """The lookup-table contraction of one token row: q int8 [K], weights in
    the tiled layout [N/16, 4K] -> int32 [N]."""
    assert q.is_cuda and q.dtype == torch.int8 and q.dim() == 1 and q.is_contiguous()
    assert tiled.is_cuda and tiled.dtype == torch.uint8 and tiled.dim() == 2 and tiled.is_contiguous()
    k = q.numel()
    assert tiled.shape[1] == 4 * k
    n = 16 * tiled.shape[0]
    if out is None:
        out = torch.empty(max(n, 4), dtype=torch.int32, device=q.device)[:n]
    assert out.is_cuda and out.dtype == torch.int32 and out.numel() == n
    st = _lib.blprobe_lut_decode_acc(ctypes.c_void_p(q.data_ptr()), k, ctypes.c_void_p(tiled.data_ptr()),
                                     n, ctypes.c_void_p(out.data_ptr()), _stream(q.device))
    if st != 0:
        raise RuntimeError(f"blprobe_lut_decode_acc failed ({st})")
    return out


def mfma_i8(workgroups: int, iters: int, pattern: int, sink: torch.Tensor) -> int:
    """Runs the matrix-core loop; returns its int8 operation count."""
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= workgroups * 256
    st = _lib.blprobe_mfma_i8(workgroups, iters, pattern, ctypes.c_void_p(sink.data_ptr()),
                              _stream(sink.device))
    if st != 0:
        raise RuntimeError(f"blprobe_mfma_i8 failed ({st})")
    return OPS_PER_ROUND_PER_WG * iters * workgroups
