"""The entry point that allocates nothing, bitlinear_forward_grouped_noalloc,
called through the C ABI: its outputs must equal those of
bitlinear_forward_grouped (the same kernels with a caller workspace) bit for
bit, on two calls in a row, the second with a smaller input that reuses the
scratch memory the first one left dirty.  The second layer splits K across
workgroups, so it depends on the library clearing its partial sums and
arrival counters in that memory.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from bit_gemm_bitlinear_amd import workloads as wls

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def make_layer(bl, seed, m, shapes):
    """Per projection: x (device bf16), weights (packed, tiled when asked),
    w_scale, two output buffers, and the oracle's output."""
    out = []
    for i, (n, k, tiled) in enumerate(shapes):
        x, w = wls.random_case(seed + i, m, n, k, scale=2.0)
        packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
        if tiled:
            packed = bl.tile_weights(packed)
        y_ref = oracle.forward(x, *oracle.pack_weights(w))
        out.append(dict(x=dev_bf16(x), p=packed, s=ws, n=n, k=k, tiled=tiled, ref=y_ref,
                        y0=torch.full((m, n), 7.0, dtype=torch.bfloat16, device=DEV),
                        y1=torch.full((m, n), -3.0, dtype=torch.bfloat16, device=DEV)))
    return out


def descriptors(bl, layer, which):
    arr = (bl.Projection * len(layer))()
    for i, e in enumerate(layer):
        arr[i] = bl.Projection(e["x"].data_ptr(), e["p"].data_ptr(), e["s"].data_ptr(),
                               e[which].data_ptr(), e["n"], e["k"],
                               bl.LAYOUT_TILED if e["tiled"] else bl.LAYOUT_ROWS, 0)
    return arr


def run_both(bl, m, layer):
    lib = bl.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref_arr = descriptors(bl, layer, "y0")
    need = lib.bitlinear_forward_grouped_workspace_bytes(len(layer), ref_arr, m)
    assert 0 < need <= lib_scratch_bytes()
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    assert lib.bitlinear_forward_grouped(len(layer), ref_arr, m, ctypes.c_void_p(ws.data_ptr()),
                                         need, stream) == 0
    arr = descriptors(bl, layer, "y1")
    assert lib.bitlinear_forward_grouped_noalloc(len(layer), arr, m, stream) == 0
    torch.cuda.synchronize()
    for e in layer:
        got, want = host_bits(e["y1"]), host_bits(e["y0"])
        assert np.array_equal(got, want), f"no-alloc differs from the workspace call ({e['n']}x{e['k']})"
        assert np.array_equal(want, e["ref"]), f"workspace call differs from the oracle ({e['n']}x{e['k']})"


def lib_scratch_bytes():
    return 64 << 20  # BL_NOALLOC_SCRATCH_BYTES


def test_noalloc_matches_workspace_call_twice_then_smaller():
    from bit_gemm_bitlinear_amd import bitlinear as bl

    # first call: the matrix-core path, a prefill-sized layer (codes fill the
    # start of the scratch array)
    big = make_layer(bl, 500, 300, [(512, 9216, True), (384, 2048, False), (640, 4096, True)])
    run_both(bl, 300, big)
    # second and third calls, smaller: decode at M = 16 with K split across
    # workgroups (partial sums and arrival counters in the scratch array,
    # which now holds the first call's codes)
    small = make_layer(bl, 600, 16, [(640, 9216, False), (256, 2048, True)])
    run_both(bl, 16, small)
    for e in small:
        e["y1"].fill_(5.0)
    run_both(bl, 16, small)


def test_noalloc_rejects_oversized_call_before_launch():
    from bit_gemm_bitlinear_amd import bitlinear as bl

    lib = bl.lib()
    arr = (bl.Projection * 1)()
    arr[0] = bl.Projection(0x10000, 0x20000, 0x30000, 0x40000, 4096, 16384, 0, 0)
    need = lib.bitlinear_forward_grouped_workspace_bytes(1, arr, 4096)
    assert need > lib_scratch_bytes()
    # fake (never dereferenced) pointers: the size check rejects the call on
    # the host, so nothing is launched
    assert lib.bitlinear_forward_grouped_noalloc(1, arr, 4096, None) == 4
