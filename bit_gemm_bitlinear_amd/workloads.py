"""Seeded synthetic workloads for the BitLinear forward pass.

This module only draws inputs: it holds none of the method's arithmetic
(no quantization, packing, contraction or dequantization), so the CPU oracle
and the HIP path can both be fed from it without sharing any code.

The shapes stand in for the decoder layers the pages name (Falcon-E 1B/3B,
BitNet b1.58 2B/3B/8B-class models); no checkpoint is used.  Every tensor is
drawn from ``numpy.random.default_rng`` seeded with
``[20261203, workload_id, projection_index, role, ...]``:

* latent weights: fp32 ``standard_normal * 0.02`` (role 0);
* activations: fp32 draws rounded to bf16 by torch's round-to-nearest-even
  conversion (role 1, seeded also by the row count M and a variant number).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED = 20261203


@dataclass(frozen=True)
class Projection:
    name: str
    n: int  # output features (rows of the weight matrix)
    k: int  # input features


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    ms: tuple  # token counts this workload is run at
    projections: tuple
    act: str = "normal"  # "normal", "outlier_channels" or "student_t"
    zero_weight_frac: float = 0.0
    zero_rows: dict = field(default_factory=dict)  # M -> rows forced to zero
    description: str = ""

    @property
    def packed_bytes(self) -> int:
        return sum(p.n * p.k // 4 for p in self.projections)

    def ops(self, m: int) -> int:
        return sum(2 * m * p.n * p.k for p in self.projections)


def _layer(d, ffn, kv=None):
    kv = d if kv is None else kv
    return (
        Projection("q", d, d),
        Projection("k", kv, d),
        Projection("v", kv, d),
        Projection("o", d, d),
        Projection("gate", ffn, d),
        Projection("up", ffn, d),
        Projection("down", d, ffn),
    )


WORKLOADS = {
    w.name: w
    for w in (
        Workload(
            0, "single_2048_m8", (8,), (Projection("proj", 2048, 2048),),
            description="one BitLinear, M=8, 2048x2048, N(0,1) activations",
        ),
        Workload(
            1, "decode_1b_m1", (1,), _layer(2048, 8192),
            description="decode GEMV M=1 over the 7 projections of a d=2048, "
                        "ffn=8192 decoder layer",
        ),
        Workload(
            2, "decode_3b", (1, 4, 16), _layer(3072, 9216),
            act="outlier_channels",
            description="small-batch decode M in {1,4,16} over a d=3072, "
                        "ffn=9216 layer; 1% of input channels scaled x20",
        ),
        Workload(
            3, "prefill_2b_m2048", (2048,),
            (Projection("gate", 6912, 2560), Projection("up", 6912, 2560),
             Projection("down", 2560, 6912)),
            description="prefill M=2048 over the FFN of a d=2560, ffn=6912 layer",
        ),
        Workload(
            4, "layer_8b", (1, 512), _layer(4096, 14336, kv=1024),
            act="student_t", zero_weight_frac=0.30,
            zero_rows={512: (0, 1, 255, 511)},
            description="d=4096, ffn=14336, GQA k/v 1024 layer at M=1 and "
                        "M=512; Student-t(3) activations with all-zero rows; "
                        "30% of latent weights exactly zero",
        ),
    )
}

# The attention projections of the 2B-class layer (d=2560) are also timed
# as a side measurement of the prefill path.
PREFILL_2B_ATTN = (
    Projection("q", 2560, 2560), Projection("k", 2560, 2560),
    Projection("v", 2560, 2560), Projection("o", 2560, 2560),
)


def _rng(*key):
    return np.random.default_rng([SEED, *key])


def to_bf16_bits(xf: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(xf, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def weights(wl: Workload, pi: int) -> np.ndarray:
    """Latent fp32 weights [N, K] of projection ``pi``."""
    p = wl.projections[pi]
    rng = _rng(wl.wid, pi, 0)
    w = rng.standard_normal((p.n, p.k), dtype=np.float32) * np.float32(0.02)
    if wl.zero_weight_frac:
        w[rng.random((p.n, p.k)) < wl.zero_weight_frac] = 0.0
    return w


def activations(wl: Workload, pi: int, m: int, variant: int = 0) -> np.ndarray:
    """bf16 bit patterns [M, K] feeding projection ``pi``.

    ``variant`` 1 of the Student-t workload at M=1 is an all-zero row."""
    p = wl.projections[pi]
    rng = _rng(wl.wid, pi, 1, m, variant)
    if wl.act == "student_t":
        xf = rng.standard_t(3, size=(m, p.k)).astype(np.float32)
    else:
        xf = rng.standard_normal((m, p.k), dtype=np.float32)
    if wl.act == "outlier_channels":
        cols = rng.choice(p.k, p.k // 100, replace=False)
        xf[:, cols] *= np.float32(20.0)
    for r in wl.zero_rows.get(m, ()):
        xf[r, :] = 0.0
    if wl.act == "student_t" and m == 1 and variant == 1:
        xf[:] = 0.0
    return to_bf16_bits(xf)


def variants(wl: Workload, m: int):
    """Activation variants a workload is run with at a given M."""
    if wl.act == "student_t" and m == 1:
        return (0, 1)
    return (0,)


def random_case(seed: int, m: int, n: int, k: int, scale: float = 1.0,
                wscale: float = 0.02):
    """A small seeded (x bf16 bits, w fp32) case for parity sweeps."""
    rng = _rng(999, seed, m, n, k)
    xf = rng.standard_normal((m, k), dtype=np.float32) * np.float32(scale)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(wscale)
    return to_bf16_bits(xf), w
