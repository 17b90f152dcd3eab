"""CPU oracle for the BitNet b1.58 BitLinear forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library and imports nothing from the product package.

What is computed, and where the pages define it
-----------------------------------------------
Sources (the text of three renderings of one blog post, plus a news page):

* [FE-ar] "A series of powerful, universal and fine-tunable 1.58-bit language
  models" -- Arabic rendering of the Falcon-Edge blog on n77n.net, section
  "Falcon-Edge, a series of universal models": the functions
  ``activation_norm_quant``, ``BitLinear.post_quant_process``,
  ``BitLinear.forward`` and ``_weight_quant``.
* [FE-ko] "Introducing Falcon-Edge: powerful, universal, fine-tunable 1.58-bit
  language models" -- Korean rendering on molayo1419.me, same code fragments
  (truncated) and the prose around them.
* [GN] "BitNet: an inference framework for 1-bit LLMs" -- GeekNews
  (news.hada.io), section "Hacker News comments": the remark that the
  weights are really stored in 2 bits, which can hold four values
  (-1, 0, 1, 2).

Steps (every function below cites the one it follows):

1. activation quantization (``act_quant``): per token (last dim) absmax,
   scale = 127 / max(amax, 1e-5), q = clamp(round(x * scale), -128, 127);
   [FE-ar] ``activation_norm_quant``.
2. weight quantization (``weight_scale`` and ``ternarize``): per tensor
   absmean, scale = 1 / max(mean|w|, 1e-5), u = clamp(round(w * scale), -1, 1);
   [FE-ar] ``_weight_quant``.
3. 2-bit storage of u (``pack`` / ``unpack``); the pages only say the
   weights are kept packed (``unpack_weights`` in ``BitLinear.forward``) in
   2 bits ([GN]); the layout is this project's reading (below).
4. the contraction acc = q . u^T (``contract``), exact in integers;
   [FE-ar] the ``F.linear`` call in ``BitLinear.forward``.
5. dequantization y = acc / (input_scale * weight_scale) (``dequant``);
   [FE-ar] ``post_quant_process``, rounded to bfloat16 ("half precision" in
   the [FE-ko] prose under ``activation_norm_quant``).
6. the optional bias, added to the dequantized output (``add_bf16`` in
   ``forward``); [FE-ar] the last lines of ``BitLinear.forward``.  A residual
   tensor, which the layer around BitLinear adds, goes in the same way after
   it (a reading: the pages' code stops at the bias).
7. the "universal" bf16 export u / scale (``export_bf16``); [FE-ar] the
   ``state_dict`` loop after ``_weight_quant``.

Readings where the pages leave a step open (each is also listed in the
design notes of the repository):

R1  All quantization arithmetic is IEEE fp32 with round-to-nearest-even:
    bf16 inputs widen exactly to fp32; the scale is one correctly rounded
    fp32 division; x * scale is one fp32 multiply.
R2  mean|w| is the exact real sum of |w| divided by the element count,
    correctly rounded once to fp32 (so it does not depend on summation
    order).
R3  The constant 1e-5 is fp32(1e-5); the clamp applies to amax / mean
    before the division.
R4  ``round`` is round-half-to-even (torch ``round`` semantics).
R5  2-bit code c = u + 1 in {0, 1, 2}; byte ``packed[n, k // 4]`` holds
    c[n, k] at bits 2*(k % 4) .. 2*(k % 4) + 1 (least significant first);
    rows are contiguous, K/4 bytes per row.  Code 3 is never produced; on
    input it decodes as c - 1 = +2 (the fourth value named in [GN]).
R6  The contraction is exact integer arithmetic (int32 result), not a
    bf16/fp32 GEMM.
R7  Dequantization divides fp32(acc) by the fp32 product
    fp32(input_scale * weight_scale) (one correctly rounded division),
    then rounds to bfloat16 with round-to-nearest-even.
R12 The bias and the residual are bf16 tensors, added to the bf16 output one
    at a time as a bf16 tensor add does: both operands widened to fp32, one
    fp32 add, the sum rounded to bf16 (round-to-nearest-even); bias first,
    then residual.  The fp32 add of two bf16 values is exact whenever the
    result can differ from one of them after the bf16 rounding, so this is
    the exact sum rounded once to bf16.
R13 The export computes u / scale as one correctly rounded fp32 division
    and rounds the quotient to bf16 (the checkpoint the [FE-ar] text calls
    the bfloat16 variant).
R11 (a storage choice of this project, not a reading of the pages) The
    optional tiled layout (``tile`` / ``untile``) permutes the R5 bytes
    inside each block of 16 rows (N % 16 == 0, K % 256 == 0); it changes
    no result.

Parity status: every function here is pinned by tests that do not call it
to compute their expectation (hand derivations, exact rational arithmetic,
brute force, library routines, invariants).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

F32_1EM5 = np.float32(1e-5)  # R3: fp32(1e-5) = 9.99999974737875e-06


# --------------------------------------------------------------------------
# bfloat16 storage (uint16 bit patterns)
# --------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly: bf16 is the top half
    of an fp32 word."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, round-to-nearest-even (R7).

    The 16 low bits are dropped after adding 0x7FFF plus the lowest kept
    bit, which rounds half-way cases to the even neighbour.  NaN stays a
    quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = np.isnan(x)
    rounded = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), rounded)
    return rounded.astype(np.uint16)


# --------------------------------------------------------------------------
# Step 1: activation quantization
# --------------------------------------------------------------------------

def act_quant(x_bf16: np.ndarray):
    """Per-token absmax int8 quantization of bf16 activations [M, K].

    [FE-ar] ``activation_norm_quant``: scale = 127 / max_k |x| clamped at
    1e-5; q = round(x * scale) clamped to [-128, 127].  Readings R1, R3, R4.
    Returns (q int8 [M, K], scale fp32 [M])."""
    xf = bf16_to_f32(x_bf16)
    if not np.all(np.isfinite(xf)):
        raise ValueError("activations must be finite")
    amax = np.abs(xf).max(axis=-1)
    scale = np.float32(127.0) / np.maximum(amax, F32_1EM5)
    t = xf * scale[..., None]
    q = np.clip(np.rint(t), -128, 127).astype(np.int8)
    return q, scale.astype(np.float32)


# --------------------------------------------------------------------------
# Step 2: weight quantization
# --------------------------------------------------------------------------

def _round_to_f32(value: Fraction) -> np.float32:
    """Round a non-negative rational to the nearest fp32, ties to even,
    including the subnormal range (quantum 2**-149).  Values at or above the
    fp32 overflow threshold are not expected here (a mean of finite fp32
    magnitudes is below the largest finite one)."""
    if value < 0:
        raise ValueError("negative value")
    if value == 0:
        return np.float32(0.0)
    num, den = value.numerator, value.denominator
    # exponent e with 2**e <= value < 2**(e+1)
    e = num.bit_length() - den.bit_length()
    if Fraction(2) ** e > value:
        e -= 1
    elif Fraction(2) ** (e + 1) <= value:
        e += 1
    quantum_exp = max(e, -126) - 23
    quantum = Fraction(2) ** quantum_exp
    mant = round(value / quantum)  # Fraction.__round__ rounds half to even
    return np.float32(float(mant) * 2.0 ** quantum_exp)


def absmean_exact(w: np.ndarray) -> np.float32:
    """mean(|w|) of an fp32 tensor, correctly rounded to fp32 (reading R2).

    Each |w| is m * 2**(max(E, 1) - 150) with E the biased exponent and m the
    24-bit significand (implicit bit set when E > 0).  The significands are
    summed per exponent in int64 (at most 2**24 per element, so exact for
    fewer than 2**39 elements), the per-exponent sums are combined as one
    Python integer in units of 2**-149, and the quotient by the element
    count is rounded once."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.size == 0:
        raise ValueError("empty weight tensor")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    bits = w.reshape(-1).view(np.uint32) & np.uint32(0x7FFFFFFF)
    expo = (bits >> np.uint32(23)).astype(np.int64)
    mant = (bits & np.uint32(0x7FFFFF)).astype(np.int64) | ((expo > 0).astype(np.int64) << 23)
    total = 0  # exact sum of |w| in units of 2**-149
    for e in np.unique(expo):
        bucket = int(mant[expo == e].sum())
        total += bucket << (max(int(e), 1) - 1)
    return _round_to_f32(Fraction(total, w.size) / Fraction(2) ** 149)


def weight_scale(w: np.ndarray) -> np.float32:
    """Per-tensor weight scale 1 / max(mean|w|, 1e-5) in fp32.

    [FE-ar] ``_weight_quant``, first line; readings R1, R2, R3."""
    mean = absmean_exact(w)
    return np.float32(np.float32(1.0) / np.maximum(mean, F32_1EM5))


def ternarize(w: np.ndarray, w_scale: np.float32) -> np.ndarray:
    """u = clamp(round(w * scale), -1, 1) as int8.

    [FE-ar] ``_weight_quant``, second line; readings R1, R4."""
    w = np.asarray(w, dtype=np.float32)
    t = w * np.float32(w_scale)
    return np.clip(np.rint(t), -1, 1).astype(np.int8)


def weight_quant(w: np.ndarray):
    """Both lines of [FE-ar] ``_weight_quant``: returns (u int8, scale fp32)."""
    s = weight_scale(w)
    return ternarize(w, s), s


# --------------------------------------------------------------------------
# Step 3: 2-bit storage
# --------------------------------------------------------------------------

def pack(u: np.ndarray) -> np.ndarray:
    """Pack ternary codes [N, K] (K % 4 == 0) into [N, K/4] bytes, reading R5.

    Weight k of a row lands in byte k // 4 at bit 2*(k % 4) as c = u + 1."""
    u = np.asarray(u)
    n, k = u.shape
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    if np.any((u < -1) | (u > 1)):
        raise ValueError("codes must be ternary")
    c = (u.astype(np.int16) + 1).astype(np.uint8).reshape(n, k // 4, 4)
    out = np.zeros((n, k // 4), dtype=np.uint8)
    for j in range(4):
        out |= (c[:, :, j] << np.uint8(2 * j)).astype(np.uint8)
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack`` (the pages' ``unpack_weights``): [N, K/4] bytes ->
    [N, K] int8 values c - 1 in {-1, 0, 1, 2}; code 3 gives 2 (reading R5)."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, kb = packed.shape
    out = np.empty((n, kb, 4), dtype=np.int8)
    for j in range(4):
        out[:, :, j] = ((packed >> np.uint8(2 * j)) & np.uint8(3)).astype(np.int8) - 1
    return out.reshape(n, kb * 4)


def _tiled_position(row: int, o: int, rowbytes: int) -> int:
    """R11: where the 16 R5 bytes at byte o (a multiple of 16) of weight row
    `row` start in the tiled layout.  Rows 16b..16b+15 keep their block of
    16 * rowbytes bytes; it is cut along K into 1 KB tiles (64 bytes of each of
    the 16 rows), and inside a tile the 16-byte piece g = (o // 16) % 4 of row
    r = row % 16 comes at 256 * g + 16 * r."""
    block, r = divmod(row, 16)
    tile_no, g = divmod(o // 16, 4)
    return block * 16 * rowbytes + 1024 * tile_no + 256 * g + 16 * r


def tile(packed: np.ndarray) -> np.ndarray:
    """R5 bytes [N, K/4] -> the tiled layout (R11), as [N/16, 4K] bytes."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, rowbytes = packed.shape
    if n % 16 or rowbytes % 64:
        raise ValueError("the tiled layout needs N % 16 == 0 and K % 256 == 0")
    out = np.empty(n * rowbytes, dtype=np.uint8)
    for row in range(n):
        for o in range(0, rowbytes, 16):
            at = _tiled_position(row, o, rowbytes)
            out[at:at + 16] = packed[row, o:o + 16]
    return out.reshape(n // 16, 16 * rowbytes)


def untile(tiled: np.ndarray) -> np.ndarray:
    """The inverse of ``tile``: [N/16, 4K] bytes -> R5 bytes [N, K/4]."""
    tiled = np.asarray(tiled, dtype=np.uint8)
    nb, width = tiled.shape
    n, rowbytes = 16 * nb, width // 16
    if width % 1024:
        raise ValueError("the tiled layout needs K % 256 == 0")
    flat = tiled.reshape(-1)
    out = np.empty((n, rowbytes), dtype=np.uint8)
    for row in range(n):
        for o in range(0, rowbytes, 16):
            at = _tiled_position(row, o, rowbytes)
            out[row, o:o + 16] = flat[at:at + 16]
    return out


# --------------------------------------------------------------------------
# Step 4: contraction
# --------------------------------------------------------------------------

def contract(q: np.ndarray, u: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * u[n, k], exact, as int32 (reading R6).

    The products and every partial sum are integers of magnitude at most
    256 * K, so a float64 matrix product is exact while 256 * K < 2**53; the
    result is checked to be integral and to fit int32."""
    q = np.asarray(q)
    u = np.asarray(u)
    if q.shape[-1] != u.shape[-1]:
        raise ValueError("K mismatch")
    kdim = q.shape[-1]
    if 256 * kdim >= 2 ** 53:
        raise ValueError("K too large for an exact float64 product")
    acc = q.astype(np.float64) @ u.astype(np.float64).T
    acc_i = acc.astype(np.int64)
    assert np.array_equal(acc_i.astype(np.float64), acc)
    if np.any(np.abs(acc_i) >= 2 ** 31):
        raise OverflowError("accumulator exceeds int32")
    return acc_i.astype(np.int32)


def contract_loops(q: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The same sum written as plain Python integer loops (tiny shapes)."""
    m_, k_ = q.shape
    n_ = u.shape[0]
    out = np.zeros((m_, n_), dtype=np.int64)
    for m in range(m_):
        for n in range(n_):
            s = 0
            for k in range(k_):
                s += int(q[m, k]) * int(u[n, k])
            out[m, n] = s
    return out.astype(np.int32)


# --------------------------------------------------------------------------
# Step 5: dequantization
# --------------------------------------------------------------------------

def dequant(acc: np.ndarray, x_scale: np.ndarray, w_scale: np.float32) -> np.ndarray:
    """y = acc / (input_scale * weight_scale) in fp32, rounded to bf16.

    [FE-ar] ``BitLinear.post_quant_process`` (reading R7).  The page passes
    the two scales in the opposite order to the declared parameters; their
    fp32 product is the same either way."""
    acc = np.asarray(acc, dtype=np.int32)
    d = np.asarray(x_scale, dtype=np.float32) * np.float32(w_scale)
    yf = acc.astype(np.float32) / d[..., None]
    return f32_to_bf16(yf)


# --------------------------------------------------------------------------
# The whole forward pass
# --------------------------------------------------------------------------

def pack_weights(w: np.ndarray):
    """Offline weight preparation: (packed [N, K/4] uint8, w_scale fp32)."""
    u, s = weight_quant(w)
    return pack(u), s


def forward_acc(q: np.ndarray, packed: np.ndarray) -> np.ndarray:
    """int32 accumulators of given int8 codes against packed weights."""
    return contract(q, unpack(packed))


def add_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """a + b for bf16 tensors (broadcasting): both widened to fp32, one fp32
    add, the sum rounded to bf16 (reading R12).  [FE-ar] the
    ``y += self.bias`` line of ``BitLinear.forward``."""
    s = bf16_to_f32(a_bits) + bf16_to_f32(b_bits)
    return f32_to_bf16(s.astype(np.float32))


def forward(x_bf16: np.ndarray, packed: np.ndarray, w_scale: np.float32,
            bias: np.ndarray | None = None, residual: np.ndarray | None = None) -> np.ndarray:
    """[FE-ar] ``BitLinear.forward``: unpack the stored weights, quantize the
    activations, contract, dequantize, then add the bias (bf16 [N]) if one
    is given; then the residual (bf16 [M, N]) if one is given (R12).
    Returns bf16 bits."""
    u = unpack(packed)
    q, s = act_quant(x_bf16)
    acc = contract(q, u)
    y = dequant(acc, s, w_scale)
    if bias is not None:
        y = add_bf16(y, np.asarray(bias, np.uint16)[None, :])
    if residual is not None:
        y = add_bf16(y, residual)
    return y


# --------------------------------------------------------------------------
# Step 7: the "universal" bf16 export
# --------------------------------------------------------------------------

def export_bf16(packed: np.ndarray, w_scale: np.float32) -> np.ndarray:
    """Dense bf16 weights u / scale from the packed codes: [N, K/4] bytes ->
    [N, K] bf16 bits.  [FE-ar] the ``state_dict`` loop that follows
    ``_weight_quant`` (``param_value / param_scale``); reading R13."""
    u = unpack(packed).astype(np.float32)
    return f32_to_bf16((u / np.float32(w_scale)).astype(np.float32))
