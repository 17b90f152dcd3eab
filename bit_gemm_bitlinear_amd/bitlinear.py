"""ctypes binding over libbitlinear.so (C ABI in include/bitlinear.h).

Argument marshalling only: every step of the BitLinear forward pass runs in
the library's HIP kernels.  PyTorch provides device memory and the current
HIP stream.  Importing this module loads the library and raises ImportError
if it has not been built (``python -m bit_gemm_bitlinear_amd.build``); there
is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitlinear.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m bit_gemm_bitlinear_amd.build` "
        "(hipcc for gfx950); the BitLinear kernels have no fallback")

_lib = ctypes.CDLL(LIB_PATH)

_i64, _i32, _sz, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p


class Projection(ctypes.Structure):
    """bl_projection: one projection of a grouped forward call."""
    _fields_ = [("x", _vp), ("packed", _vp), ("w_scale", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("layout", _i32), ("reserved", _i32)]


LAYOUT_ROWS = 0   # BL_LAYOUT_ROWS: packed uint8 [N, K/4]
LAYOUT_TILED = 1  # BL_LAYOUT_TILED: uint8 [N/16, 4*K], one row per block of 16 weight rows


_SIGS = {
    "bitlinear_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bitlinear_abi_version": (ctypes.c_int, []),
    "bitlinear_pack_workspace_bytes": (_sz, [_i64, _i64]),
    "bitlinear_pack_weights": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_unpack_weights": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "bitlinear_tile_weights": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "bitlinear_untile_weights": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "bitlinear_act_quant": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "bitlinear_forward_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bitlinear_forward": (ctypes.c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_forward_tiled": (ctypes.c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz,
                                               _vp]),
    "bitlinear_forward_grouped_workspace_bytes": (_sz, [_i32, ctypes.POINTER(Projection), _i64]),
    "bitlinear_forward_grouped": (ctypes.c_int, [_i32, ctypes.POINTER(Projection), _i64, _vp,
                                                 _sz, _vp]),
    "bitlinear_forward_acc": (ctypes.c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_forward_acc_tiled": (ctypes.c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz,
                                                   _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

STATUS = {0: "BL_OK", 1: "BL_EINVAL", 2: "BL_ESHAPE", 3: "BL_EALIGN", 4: "BL_EWORKSPACE",
          5: "BL_EHIP"}


class BitLinearError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = _lib.bitlinear_status_string(status).decode()
        super().__init__(f"{STATUS.get(status, status)}: {msg}")


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise BitLinearError(status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _require(t: torch.Tensor, dtype, ndim, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------

def pack_weights(w: torch.Tensor):
    """Latent fp32 weights [N, K] -> (packed uint8 [N, K/4], w_scale fp32 [1])."""
    _require(w, torch.float32, 2, "w")
    n, k = w.shape
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    w_scale = torch.empty(4, dtype=torch.float32, device=w.device)[:1]
    ws = _workspace(_lib.bitlinear_pack_workspace_bytes(n, k), w.device, None)
    _check(_lib.bitlinear_pack_weights(_ptr(w), n, k, _ptr(packed), _ptr(w_scale), _ptr(ws),
                                       ws.numel(), _stream(w)))
    return packed, w_scale


def unpack_weights(packed: torch.Tensor) -> torch.Tensor:
    """Packed [N, K/4] -> int8 [N, K] values c - 1."""
    _require(packed, torch.uint8, 2, "packed")
    n, kb = packed.shape
    u = torch.empty((n, 4 * kb), dtype=torch.int8, device=packed.device)
    _check(_lib.bitlinear_unpack_weights(_ptr(packed), n, 4 * kb, _ptr(u), _stream(packed)))
    return u


def tile_weights(packed: torch.Tensor) -> torch.Tensor:
    """Row-major packed [N, K/4] -> the 16-row tiled layout, as uint8
    [N/16, 4*K] (one row per block of 16 weight rows).  N % 16 == 0 and
    K % 256 == 0."""
    _require(packed, torch.uint8, 2, "packed")
    n, kb = packed.shape
    if n % 16:
        raise ValueError("the tiled layout needs N % 16 == 0")
    tiled = torch.empty((n // 16, 16 * kb), dtype=torch.uint8, device=packed.device)
    _check(_lib.bitlinear_tile_weights(_ptr(packed), n, 4 * kb, _ptr(tiled), _stream(packed)))
    return tiled


def untile_weights(tiled: torch.Tensor) -> torch.Tensor:
    """The inverse of tile_weights: [N/16, 4*K] -> row-major [N, K/4]."""
    _require(tiled, torch.uint8, 2, "tiled")
    nb, kb16 = tiled.shape
    if kb16 % 1024:
        raise ValueError("a tiled weight row holds 16 rows of K/4 bytes, K % 256 == 0")
    n, k = 16 * nb, kb16 // 4
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=tiled.device)
    _check(_lib.bitlinear_untile_weights(_ptr(tiled), n, k, _ptr(packed), _stream(tiled)))
    return packed


def weight_layout(w: torch.Tensor, k: int):
    """(N, layout) of a weight tensor used against K input features: [N, K/4]
    is row-major, [N/16, 4*K] the tiled layout."""
    if w.shape[1] * 4 == k:
        return w.shape[0], LAYOUT_ROWS
    if w.shape[1] == 4 * k and k % 256 == 0:
        return 16 * w.shape[0], LAYOUT_TILED
    raise ValueError("packed weights do not match K")


def act_quant(x: torch.Tensor):
    """bf16 activations [M, K] -> (int8 codes [M, K], fp32 scales [M])."""
    _require(x, torch.bfloat16, 2, "x")
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    s = torch.empty(max(m, 4), dtype=torch.float32, device=x.device)[:m]
    _check(_lib.bitlinear_act_quant(_ptr(x), m, k, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def forward_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(_lib.bitlinear_forward_workspace_bytes(m, n, k))


def forward(x: torch.Tensor, packed: torch.Tensor, w_scale: torch.Tensor,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """y = BitLinear(x) as bf16 [M, N]; `packed` in either layout."""
    _require(x, torch.bfloat16, 2, "x")
    _require(packed, torch.uint8, 2, "packed")
    m, k = x.shape
    n, layout = weight_layout(packed, k)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    ws = _workspace(forward_workspace_bytes(m, n, k), x.device, workspace)
    fn = _lib.bitlinear_forward_tiled if layout == LAYOUT_TILED else _lib.bitlinear_forward
    _check(fn(m, n, k, _ptr(x), _ptr(packed), _ptr(w_scale), _ptr(out),
              _ptr(ws), ws.numel() * ws.element_size(), _stream(x)))
    return out


def _projections(xs, packeds, w_scales, outs):
    arr = (Projection * len(xs))()
    for i, (x, p, s, y) in enumerate(zip(xs, packeds, w_scales, outs)):
        n, layout = weight_layout(p, x.shape[1])
        arr[i] = Projection(x.data_ptr(), p.data_ptr(), s.data_ptr(), y.data_ptr(),
                            n, x.shape[1], layout, 0)
    return arr


def forward_grouped_workspace_bytes(m: int, shapes: Sequence[tuple]) -> int:
    arr = (Projection * len(shapes))()
    for i, (n, k) in enumerate(shapes):
        arr[i] = Projection(0, 0, 0, 0, n, k)
    return int(_lib.bitlinear_forward_grouped_workspace_bytes(len(shapes), arr, m))


class GroupedCall:
    """A prepared grouped forward: descriptors and workspace built once, so
    repeated calls only enqueue the two kernels."""

    def __init__(self, xs, packeds, w_scales, outs=None, workspace=None):
        m = xs[0].shape[0]
        for x, p in zip(xs, packeds):
            _require(x, torch.bfloat16, 2, "x")
            _require(p, torch.uint8, 2, "packed")
            if x.shape[0] != m:
                raise ValueError("inconsistent token counts in grouped call")
            weight_layout(p, x.shape[1])
        if outs is None:
            outs = [torch.empty((m, weight_layout(p, x.shape[1])[0]), dtype=torch.bfloat16,
                                device=x.device) for x, p in zip(xs, packeds)]
        self.m = m
        self.outs = outs
        self._keep = (list(xs), list(packeds), list(w_scales), outs)
        self._arr = _projections(xs, packeds, w_scales, outs)
        need = int(_lib.bitlinear_forward_grouped_workspace_bytes(len(xs), self._arr, m))
        self.workspace = _workspace(need, xs[0].device, workspace)
        self._dev = xs[0]

    def __call__(self, stream=None):
        s = ctypes.c_void_p(stream) if stream is not None else _stream(self._dev)
        _check(_lib.bitlinear_forward_grouped(len(self._arr), self._arr, self.m,
                                              _ptr(self.workspace),
                                              self.workspace.numel(), s))
        return self.outs


def forward_grouped(xs, packeds, w_scales, outs=None, workspace=None):
    """Independent BitLinear forwards with one token count, one pass."""
    return GroupedCall(xs, packeds, w_scales, outs, workspace)()


def forward_acc(q: torch.Tensor, packed: torch.Tensor, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None):
    """Exact int32 accumulators q . u^T for caller-supplied int8 codes;
    `packed` in either layout."""
    _require(q, torch.int8, 2, "q")
    _require(packed, torch.uint8, 2, "packed")
    m, k = q.shape
    n, layout = weight_layout(packed, k)
    if out is None:
        out = torch.empty((m, n), dtype=torch.int32, device=q.device)
    ws = _workspace(forward_workspace_bytes(m, n, k), q.device, workspace)
    fn = _lib.bitlinear_forward_acc_tiled if layout == LAYOUT_TILED else _lib.bitlinear_forward_acc
    _check(fn(m, n, k, _ptr(q), _ptr(packed), _ptr(out), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(q)))
    return out


class BitLinear:
    """Inference-time BitLinear layer (no bias): packs fp32 latent weights
    once, then runs the forward pass on bf16 activations.  The weights are
    kept in the tiled layout when the shape allows it (N % 16 == 0,
    K % 256 == 0) unless tiled=False; `packed` holds them in that layout."""

    def __init__(self, weight: torch.Tensor, tiled: bool = True):
        self.out_features, self.in_features = weight.shape
        self.packed, self.w_scale = pack_weights(weight.contiguous())
        if tiled and self.out_features % 16 == 0 and self.in_features % 256 == 0:
            self.packed = tile_weights(self.packed)

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        y = forward(x.reshape(-1, self.in_features).contiguous(), self.packed, self.w_scale)
        return y.reshape(*lead, self.out_features)
