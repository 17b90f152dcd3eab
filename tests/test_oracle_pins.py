"""Pins for the CPU oracle, computed without calling the oracle's own arithmetic.

Every expectation here comes from something other than the oracle: a hand
derivation from the formulas on the pages (the Falcon-Edge blog's
``activation_norm_quant``, ``_weight_quant`` and ``post_quant_process``),
exact rational arithmetic with a brute-force nearest-fp32 search, plain
integer loops, library routines (torch's bf16 cast, numpy's int64 einsum),
closed forms and invariants.  Each test is chosen so that a plausible slip in
the oracle (a dropped clamp, floor instead of round-half-even, mean instead of
max, a transposed operand, a swapped bit order, an order-dependent sum) fails.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bit_gemm_bitlinear_amd import workloads as wls

F1EM5 = np.float32(1e-5)


# ---------------------------------------------------------------- helpers

def nearest_f32(fr: Fraction) -> np.float32:
    """Brute force: the fp32 nearest to ``fr``, ties to the even bit pattern."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]

    def key(v):
        return (abs(Fraction(float(v)) - fr), int(np.array(v, dtype=np.float32).view(np.uint32)) & 1)

    return np.float32(min(cands, key=key))


def half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl + (fl & 1)


def torch_bf16_bits(xf):
    t = torch.from_numpy(np.ascontiguousarray(xf, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def ref_act_row(xbits_row):
    """One row of activation quantization from exact rationals."""
    xs = [Fraction(float(v)) for v in oracle.bf16_to_f32(xbits_row)]
    # bf16 -> fp32 widening itself is pinned against torch elsewhere
    amax = max(abs(v) for v in xs)
    denom = max(amax, Fraction(float(F1EM5)))
    s = nearest_f32(Fraction(127) / denom)
    q = []
    for v in xs:
        t = nearest_f32(v * Fraction(float(s)))
        q.append(max(-128, min(127, half_even(Fraction(float(t))))))
    return q, s


# ---------------------------------------------------------------- bf16 I/O

def test_bf16_widen_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite patterns only
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_to_f32(bits).view(np.uint32), ref.view(np.uint32))


def test_bf16_round_matches_torch_including_ties():
    rng = np.random.default_rng(2)
    hi = rng.integers(0, 2 ** 16, size=30000, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) < 0xFE]  # stay clear of the overflow boundary
    lo = rng.integers(0, 2 ** 16, size=hi.size, dtype=np.uint32)
    lo[: hi.size // 3] = 0x8000  # exact ties
    lo[hi.size // 3: hi.size // 2] = 0x7FFF
    xf = ((hi << 16) | lo).astype(np.uint32).view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16(xf), torch_bf16_bits(xf))


def test_bf16_round_hand_cases():
    # 1 + 2^-8 sits half-way between bf16 1.0 and 1 + 2^-7: even -> 1.0 (0x3F80)
    # 1 + 3*2^-8 sits half-way between 1 + 2^-7 and 1 + 2^-6: even -> 0x3F82
    xf = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert oracle.f32_to_bf16(xf).tolist() == [0x3F80, 0x3F82, 0xBF80]


# ---------------------------------------------------------------- activation quantization

def _bits(vals):
    return torch_bf16_bits(np.array(vals, dtype=np.float32))


def test_act_quant_hand_examples():
    # amax = 1 -> s = 127; x*s = [127, -63.5, 31.75, 0]; -63.5 is a tie -> -64
    q, s = oracle.act_quant(_bits([[1.0, -0.5, 0.25, 0.0]]))
    assert s.tolist() == [127.0] and q.tolist() == [[127, -64, 32, 0]]
    # amax = 2 -> s = 63.5; x*s = [127, 63.5, -63.5, 31.75] -> ties to even 64 / -64
    q, s = oracle.act_quant(_bits([[2.0, 1.0, -1.0, 0.5]]))
    assert s.tolist() == [63.5] and q.tolist() == [[127, 64, -64, 32]]
    # all-zero row: amax clamps to fp32(1e-5); 127 / 9.99999974737875e-06 =
    # 12700000.32..., whose nearest fp32 (spacing 1.0 there) is 12700000
    q, s = oracle.act_quant(_bits([[0.0, 0.0, 0.0, 0.0]]))
    assert s.tolist() == [12700000.0] and q.tolist() == [[0, 0, 0, 0]]


def test_act_quant_sub_threshold_row():
    # 0 < amax < 1e-5: the clamp binds, so max|q| stays below 127.
    x = _bits([[9.98e-7, -3.0e-7, 0.0, 0.0]])
    xs = oracle.bf16_to_f32(x)[0]
    q, s = oracle.act_quant(x)
    assert s[0] == np.float32(12700000.0)
    expect = [half_even(Fraction(float(nearest_f32(Fraction(float(v)) * 12700000)))) for v in xs]
    assert q[0].tolist() == expect == [13, -4, 0, 0]


@pytest.mark.parametrize("seed", range(6))
def test_act_quant_matches_exact_rationals(seed):
    rng = np.random.default_rng(100 + seed)
    m, k = 3, 37
    scale = [1.0, 1e-3, 1e3, 3e-6, 40.0, 1.0][seed]
    xf = rng.standard_normal((m, k)).astype(np.float32) * np.float32(scale)
    if seed == 5:
        xf[1] = 0.0
        xf[2, :5] = [1.5, -1.5, 0.5, 2.5, -2.5]
    x = torch_bf16_bits(xf)
    q, s = oracle.act_quant(x)
    for r in range(m):
        q_ref, s_ref = ref_act_row(x[r])
        assert s[r] == s_ref
        assert q[r].tolist() == q_ref


def test_act_quant_invariants_on_workload_rows():
    wl = wls.WORKLOADS["layer_8b"]
    x = wls.activations(wl, 6, 512)  # Student-t rows, K = 14336, with zero rows
    q, s = oracle.act_quant(x)
    xf = oracle.bf16_to_f32(x)
    amax = np.abs(xf).max(axis=1)
    live = amax >= F1EM5
    assert live.sum() == 512 - 4
    assert np.all(np.abs(q[live]).max(axis=1) == 127)
    assert np.all(q >= -127)
    # the absmax element itself maps to +-127
    arg = np.abs(xf).argmax(axis=1)
    assert np.all(np.abs(q[live, arg[live]]) == 127)
    # sign agreement and in-row monotonicity
    assert np.all((q == 0) | (np.sign(q) == np.sign(xf)))
    for r in (2, 100, 300):
        order = np.argsort(xf[r], kind="stable")
        assert np.all(np.diff(q[r, order].astype(np.int32)) >= 0)
    # rounding error at most half a code (plus one fp32 rounding of the product)
    t = xf.astype(np.float64) * s[:, None].astype(np.float64)
    assert np.all(np.abs(q - t) <= 0.5 + np.abs(t) * 2.0 ** -23)
    # zero rows -> zero codes and the clamped scale
    for r in (0, 1, 255, 511):
        assert not q[r].any() and s[r] == np.float32(12700000.0)


def test_act_quant_outlier_channels_use_row_absmax():
    wl = wls.WORKLOADS["decode_3b"]
    x = wls.activations(wl, 0, 4)
    xf = oracle.bf16_to_f32(x)
    q, s = oracle.act_quant(x)
    for r in range(4):
        q_ref, s_ref = ref_act_row(x[r])
        assert s[r] == s_ref and q[r].tolist() == q_ref
    # most ordinary channels shrink to small codes because an x20 channel sets amax
    assert np.median(np.abs(q)) < 10


# ---------------------------------------------------------------- weight quantization

def exact_mean_f32(w):
    tot = sum((abs(Fraction(float(v))) for v in w.reshape(-1)), Fraction(0))
    return nearest_f32(tot / w.size)


@pytest.mark.parametrize("seed", range(8))
def test_absmean_matches_fraction_sum(seed):
    rng = np.random.default_rng(200 + seed)
    n = [1, 2, 7, 64, 333, 1000, 513, 97][seed]
    w = (rng.standard_normal(n) * [0.02, 1.0, 1e-30, 3e4, 0.02, 1e-3, 1.0, 5e-39][seed]).astype(np.float32)
    if seed == 6:
        w[::3] = np.float32(1.401298464324817e-45)  # smallest subnormal
        w[1::7] = np.float32(3e38)
    assert oracle.absmean_exact(w) == exact_mean_f32(w)


def test_absmean_matches_float64_mean_on_large_tensor():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((1024, 1024), dtype=np.float32) * np.float32(0.02)
    m64 = np.abs(w.astype(np.float64)).mean()
    ref = np.float32(m64)
    # the float64 sum of 2^20 terms is within ~1e-10 relative of exact; only a
    # value within that distance of an fp32 half-way point could differ
    up = np.nextafter(ref, np.float32(np.inf))
    dn = np.nextafter(ref, np.float32(-np.inf))
    mid_gap = min(abs(m64 - (float(ref) + float(up)) / 2), abs(m64 - (float(ref) + float(dn)) / 2))
    assert mid_gap > 1e-9 * m64
    assert oracle.absmean_exact(w) == ref


def test_absmean_order_and_power_of_two_invariance():
    rng = np.random.default_rng(4)
    w = rng.standard_normal(200003).astype(np.float32) * np.float32(0.02)
    base = oracle.absmean_exact(w)
    for k in range(3):
        assert oracle.absmean_exact(rng.permutation(w)) == base
    for e in (-7, 5):
        assert oracle.absmean_exact(w * np.float32(2.0 ** e)) == base * np.float32(2.0 ** e)
    assert oracle.absmean_exact(np.full(1000, 0.3, np.float32)) == np.float32(0.3)


def test_weight_scale_and_ties():
    # mean(|w|) = (0.5 + 1.5 + 1 + 1) / 4 = 1 -> scale 1; w*1 = [0.5, -1.5, 1, 1]
    # round-half-even gives [0, -2, 1, 1]; the clamp makes -2 -> -1
    u, s = oracle.weight_quant(np.array([[0.5, -1.5, 1.0, 1.0]], np.float32))
    assert s == np.float32(1.0) and u.tolist() == [[0, -1, 1, 1]]
    # all zero: mean 0 clamps to fp32(1e-5); 1 / 9.99999974737875e-06 rounds to 100000
    u, s = oracle.weight_quant(np.zeros((2, 4), np.float32))
    assert s == np.float32(100000.0) and not u.any()


@pytest.mark.parametrize("seed", range(4))
def test_ternarize_matches_exact_rationals(seed):
    rng = np.random.default_rng(300 + seed)
    w = rng.standard_normal((5, 24)).astype(np.float32) * np.float32([0.02, 1.0, 7.0, 1e-7][seed])
    u, s = oracle.weight_quant(w)
    mc = max(exact_mean_f32(w), F1EM5)
    s_ref = nearest_f32(Fraction(1) / Fraction(float(mc)))
    assert s == s_ref
    for (i, j), v in np.ndenumerate(w):
        t = nearest_f32(Fraction(float(v)) * Fraction(float(s_ref)))
        assert u[i, j] == max(-1, min(1, half_even(Fraction(float(t)))))


def test_ternary_codes_and_zero_fraction_on_workload():
    wl = wls.WORKLOADS["layer_8b"]
    w = wls.weights(wl, 1)  # k projection, 1024 x 4096, 30% exact zeros
    u, s = oracle.weight_quant(w)
    assert set(np.unique(u).tolist()) <= {-1, 0, 1}
    assert np.all(u[w == 0] == 0)
    # for N(0, 0.02) with 30% zeros, |w| * scale = |w| / mean; the share of
    # nonzero codes is P(|w| > mean/2) among the nonzero draws
    frac_nz = np.count_nonzero(u) / u.size
    assert 0.45 < frac_nz < 0.6


# ---------------------------------------------------------------- 2-bit storage

def test_pack_hand_byte():
    # u = [0, -1, 1, 1] -> c = u + 1 = [1, 0, 2, 2] -> 1 + 0*4 + 2*16 + 2*64 = 0xA1
    assert oracle.pack(np.array([[0, -1, 1, 1]], np.int8)).tolist() == [[0xA1]]


def test_pack_is_base4_number_of_codes():
    import itertools

    tuples = np.array(list(itertools.product([-1, 0, 1], repeat=4)), np.int8)  # 81 x 4
    b = oracle.pack(tuples.reshape(1, -1))[0]
    expect = [sum((int(t[j]) + 1) * 4 ** j for j in range(4)) for t in tuples]
    assert b.tolist() == expect
    assert len(set(expect)) == 81
    assert all(((v >> (2 * j)) & 3) != 3 for v in expect for j in range(4))


def test_unpack_roundtrip_and_code3():
    rng = np.random.default_rng(5)
    u = rng.integers(-1, 2, size=(7, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack(oracle.pack(u)), u)
    allb = np.arange(256, dtype=np.uint8).reshape(1, -1)
    un = oracle.unpack(allb)
    for v in range(256):
        assert un[0, 4 * v: 4 * v + 4].tolist() == [((v >> (2 * j)) & 3) - 1 for j in range(4)]
    valid = np.array([v for v in range(256) if all(((v >> (2 * j)) & 3) != 3 for j in range(4))], np.uint8)
    assert np.array_equal(oracle.pack(oracle.unpack(valid.reshape(1, -1))), valid.reshape(1, -1))


# ---------------------------------------------------------------- tiled layout

def test_tile_matches_transpose_formulation():
    """The tiled layout as one numpy reshape/transpose of the row-major bytes:
    [block, row r, tile t, chunk g, byte j] -> [block, t, g, r, j]."""
    rng = np.random.default_rng(11)
    for n, k in [(16, 256), (32, 512), (48, 1024)]:
        packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.uint8)
        expect = packed.reshape(n // 16, 16, k // 256, 4, 16).transpose(0, 2, 3, 1, 4)
        got = oracle.tile(packed)
        assert got.shape == (n // 16, 4 * k)
        assert np.array_equal(got.reshape(-1), expect.reshape(-1))


def test_tile_hand_positions_and_inverse():
    """Single marked bytes land where the layout's rule puts them, block by
    block, and untile restores the rows."""
    n, k = 32, 512
    rb = k // 4
    for row, o in [(0, 0), (0, 16), (1, 0), (15, 63), (5, 64), (16, 0), (31, 127), (17, 80)]:
        packed = np.zeros((n, rb), np.uint8)
        packed[row, o] = 0xA5
        flat = oracle.tile(packed).reshape(-1)
        assert int(np.count_nonzero(flat)) == 1
        # worked by hand: block row // 16 starts at (row // 16) * 16 * rb; within
        # it tile o // 64 starts at 1024 * (o // 64); chunk (o % 64) // 16 of the
        # tile's 64-byte row piece at 256 * ((o % 64) // 16); row row % 16 at
        # 16 * (row % 16); byte o % 16 inside the chunk
        at = (row // 16) * 16 * rb + 1024 * (o // 64) + 256 * ((o % 64) // 16) + 16 * (row % 16) + o % 16
        assert flat[at] == 0xA5
    rng = np.random.default_rng(12)
    packed = rng.integers(0, 256, size=(n, rb), dtype=np.uint8)
    tiled = oracle.tile(packed)
    assert np.array_equal(oracle.untile(tiled), packed)
    # every block of 16 rows keeps its bytes in place (a permutation inside it)
    flat = tiled.reshape(-1)
    for b in range(n // 16):
        blk = slice(b * 16 * rb, (b + 1) * 16 * rb)
        assert np.array_equal(np.sort(flat[blk]), np.sort(packed[16 * b:16 * b + 16].reshape(-1)))
    with pytest.raises(ValueError):
        oracle.tile(np.zeros((8, 64), np.uint8))
    with pytest.raises(ValueError):
        oracle.tile(np.zeros((16, 32), np.uint8))


def test_tile_first_tile_is_the_16x16x64_operand_order():
    """Lane 16 g + r of a 64-lane read of the first 1 KB gets row r, bytes
    16 g .. 16 g + 15: the rows of the matrix-core operand, by brute force."""
    packed = np.random.default_rng(13).integers(0, 256, size=(16, 64), dtype=np.uint8)
    flat = oracle.tile(packed).reshape(-1)
    for lane in range(64):
        g, r = divmod(lane, 16)
        assert flat[16 * lane:16 * lane + 16].tolist() == packed[r, 16 * g:16 * g + 16].tolist()


# ---------------------------------------------------------------- contraction

@pytest.mark.parametrize("shape", [(1, 1, 4), (3, 5, 8), (4, 7, 33), (2, 9, 64)])
def test_contract_matches_loops_and_int64_einsum(shape):
    m, n, k = shape
    rng = np.random.default_rng(sum(shape))
    q = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    u = rng.integers(-1, 3, size=(n, k)).astype(np.int8)  # includes +2 (code 3)
    acc = oracle.contract(q, u)
    loops = oracle.contract_loops(q, u)
    ein = np.einsum("mk,nk->mn", q.astype(np.int64), u.astype(np.int64))
    assert np.array_equal(acc, loops) and np.array_equal(acc, ein)


def test_contract_closed_forms():
    rng = np.random.default_rng(6)
    q = rng.integers(-127, 128, size=(5, 96)).astype(np.int8)
    ones = np.ones((3, 96), np.int8)
    assert np.array_equal(oracle.contract(q, ones), np.repeat(q.astype(np.int64).sum(1, keepdims=True), 3, 1))
    assert np.array_equal(oracle.contract(q, -ones), -oracle.contract(q, ones))
    eye = np.eye(96, dtype=np.int8)[:10]
    assert np.array_equal(oracle.contract(q, eye), q[:, :10].astype(np.int32))
    perm = rng.permutation(96)
    u = rng.integers(-1, 2, size=(4, 96)).astype(np.int8)
    assert np.array_equal(oracle.contract(q[:, perm], u[:, perm]), oracle.contract(q, u))
    # not symmetric in its operands' roles: a transposed result would differ
    assert oracle.contract(q, u).shape == (5, 4)


# ---------------------------------------------------------------- dequantization

def test_dequant_hand_example():
    # acc = 96 (q = [127, -64, 32, 0] against u = [0, -1, 1, 1]), s = 127,
    # w_scale = 1: 96 / 127 = 0.755905...; bf16 spacing in [0.5, 1) is 2^-8 and
    # 0.755905 / 2^-8 = 193.51 -> 194 * 2^-8 = 0.7578125 = 0x3F42
    acc = oracle.contract(np.array([[127, -64, 32, 0]], np.int8), np.array([[0, -1, 1, 1]], np.int8))
    assert acc.tolist() == [[96]]
    y = oracle.dequant(acc, np.array([127.0], np.float32), np.float32(1.0))
    assert y.tolist() == [[0x3F42]]


@pytest.mark.parametrize("seed", range(3))
def test_dequant_matches_exact_rationals(seed):
    rng = np.random.default_rng(400 + seed)
    acc = rng.integers(-300000, 300000, size=(4, 50)).astype(np.int32)
    acc[0, :3] = [0, 1, -1]
    s = (rng.random(4) * 1000 + 0.01).astype(np.float32)
    ws = np.float32(rng.random() * 90 + 1)
    y = oracle.dequant(acc, s, ws)
    for (i, j), a in np.ndenumerate(acc):
        d = nearest_f32(Fraction(float(s[i])) * Fraction(float(ws)))
        yf = nearest_f32(Fraction(int(a)) / Fraction(float(d)))
        assert y[i, j] == torch_bf16_bits(np.array([yf], np.float32))[0]


# ---------------------------------------------------------------- whole forward

def test_forward_tiny_brute_force():
    x, w = wls.random_case(7, 3, 5, 12)
    # independent pipeline: exact-rational quantizers, integer loops, exact dequant
    mean = exact_mean_f32(w)
    ws = nearest_f32(Fraction(1) / Fraction(float(max(mean, F1EM5))))
    u = [[max(-1, min(1, half_even(Fraction(float(nearest_f32(Fraction(float(v)) * Fraction(float(ws)))))))) for v in row] for row in w]
    packed, ws_o = oracle.pack_weights(w)
    assert ws_o == ws
    y = oracle.forward(x, packed, ws_o)
    for m in range(3):
        q, s = ref_act_row(x[m])
        for n in range(5):
            a = sum(q[k] * u[n][k] for k in range(12))
            d = nearest_f32(Fraction(float(s)) * Fraction(float(ws)))
            yf = nearest_f32(Fraction(a) / Fraction(float(d)))
            assert y[m, n] == torch_bf16_bits(np.array([yf], np.float32))[0]


def test_forward_close_to_dequantized_float_product():
    # The pages' approximation x ~ x_quant / x_scale: y must be near
    # x @ (u / w_scale)^T, within half a code per term plus bf16 rounding.
    wl = wls.WORKLOADS["single_2048_m8"]
    w = wls.weights(wl, 0)[:256]
    x = wls.activations(wl, 0, 8)
    packed, ws = oracle.pack_weights(w)
    y = oracle.bf16_to_f32(oracle.forward(x, packed, ws)).astype(np.float64)
    u = oracle.unpack(packed).astype(np.float64)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    _, s = oracle.act_quant(x)
    approx = xf @ u.T / float(ws)
    bound = (np.abs(u).sum(1)[None, :] * 0.5 / (s[:, None].astype(np.float64) * float(ws))
             + np.abs(approx) * 2.0 ** -8 + 1e-30)
    assert np.all(np.abs(y - approx) <= bound)


def test_dequant_divides_rather_than_multiplying_by_reciprocal():
    # post_quant_process divides by the scale product.  Search (with plain
    # numpy fp32 ops, only to pick inputs) for accumulators where a division
    # and a multiply by the rounded reciprocal land on different bf16 values,
    # then check those against exact rational division.
    s = np.array([127.0], np.float32)
    ws = np.float32(0.9876543)
    d = s[0] * ws
    acc = np.arange(1, 2 ** 21, dtype=np.int32)
    a = acc.astype(np.float32)
    q1, q2 = a / d, a * (np.float32(1) / d)
    pick = acc[torch_bf16_bits(q1) != torch_bf16_bits(q2)][:8]
    assert pick.size >= 4
    y = oracle.dequant(pick.reshape(1, -1), s, ws)
    dd = nearest_f32(Fraction(127) * Fraction(float(ws)))
    for j, v in enumerate(pick):
        yf = nearest_f32(Fraction(int(v)) / Fraction(float(dd)))
        assert y[0, j] == torch_bf16_bits(np.array([yf], np.float32))[0]


# ---------------------------------------------------------------- bias and residual (R12)

def nearest_bf16_bits(fr: Fraction) -> int:
    """Brute force: the bf16 bit pattern nearest to the rational ``fr``, ties
    to the even pattern (no fp32 step in between)."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)  # bf16 spacing: 8 significant bits
    lo = (a / q).numerator // (a / q).denominator
    cands = [lo, lo + 1]

    def bits(mant):
        v = float(mant * q)
        return int(torch_bf16_bits(np.array([v], np.float32))[0])  # exact: 8-bit mantissa

    best = min(cands, key=lambda c: (abs(c * q - a), bits(c) & 1))
    return sign | bits(best)


def test_add_bf16_hand_cases():
    # 0.7578125 + 0.5 = 1.2578125 = 1 + 2^-2 + 2^-7, exactly a bf16 (0x3FA1)
    assert oracle.add_bf16(np.array([0x3F42], np.uint16), np.array([0x3F00], np.uint16)).tolist() == [0x3FA1]
    # 1 + 2^-8 lies half way between 1 (0x3F80) and 1 + 2^-7: ties to even -> 1
    assert oracle.add_bf16(np.array([0x3F80], np.uint16), np.array([0x3B80], np.uint16)).tolist() == [0x3F80]
    # (1 + 2^-7) + 2^-8: half way between 0x3F81 and 0x3F82 -> the even 0x3F82
    assert oracle.add_bf16(np.array([0x3F81], np.uint16), np.array([0x3B80], np.uint16)).tolist() == [0x3F82]
    # x + (-x) is +0 under round-to-nearest
    assert oracle.add_bf16(np.array([0x3F80], np.uint16), np.array([0xBF80], np.uint16)).tolist() == [0x0000]


def test_add_bf16_is_the_exact_sum_rounded_once():
    rng = np.random.default_rng(77)
    a = rng.integers(0, 0x10000, size=3000).astype(np.uint16)
    b = rng.integers(0, 0x10000, size=3000).astype(np.uint16)
    # close exponents (sums that cancel or carry) as well as distant ones
    b[:1000] = (a[:1000] ^ 0x8000) + rng.integers(-3, 4, size=1000).astype(np.uint16)
    fa, fb = oracle.bf16_to_f32(a), oracle.bf16_to_f32(b)
    ok = np.isfinite(fa) & np.isfinite(fb) & (np.abs(fa) < 1e38) & (np.abs(fb) < 1e38)
    ok &= (np.abs(fa) > 1e-37) | (fa == 0)
    ok &= (np.abs(fb) > 1e-37) | (fb == 0)
    got = oracle.add_bf16(a[ok], b[ok])
    for x, y, g in zip(fa[ok], fb[ok], got):
        want = nearest_bf16_bits(Fraction(float(x)) + Fraction(float(y)))
        if want == 0x8000:
            want = 0  # an exact zero sum is +0
        assert int(g) == want, (x, y)


def test_add_bf16_matches_torch_bf16_add():
    rng = np.random.default_rng(78)
    a = torch_bf16_bits(rng.standard_normal(5000).astype(np.float32) * 3)
    b = torch_bf16_bits(rng.standard_normal(5000).astype(np.float32))
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    want = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.add_bf16(a, b), want)


def test_forward_bias_and_residual_hand_example():
    # the worked example (y = 96/127 -> 0x3F42), then bias 0.5 -> 1.2578125
    # (0x3FA1), then residual -1.25 -> 2^-7 (0x3C00); the bias broadcasts
    # over token rows and is added before the residual
    x = torch_bf16_bits(np.array([[1.0, -0.5, 0.25, 0.0], [1.0, -0.5, 0.25, 0.0]], np.float32))
    w = np.array([[0.5, -1.5, 1.0, 1.0]], np.float32)
    packed, ws = oracle.pack_weights(w)
    assert oracle.forward(x, packed, ws).tolist() == [[0x3F42], [0x3F42]]
    bias = np.array([0x3F00], np.uint16)
    assert oracle.forward(x, packed, ws, bias=bias).tolist() == [[0x3FA1], [0x3FA1]]
    res = torch_bf16_bits(np.array([[-1.25], [0.0]], np.float32))
    assert oracle.forward(x, packed, ws, bias=bias, residual=res).tolist() == [[0x3C00], [0x3FA1]]
    # residual alone
    assert oracle.forward(x, packed, ws, residual=res).tolist() == [
        [int(torch_bf16_bits(np.array([0.7578125 - 1.25], np.float32))[0])], [0x3F42]]


def test_forward_adds_bias_before_residual():
    # x = [1, 2^-7, 0, 0] -> scale 127, q = [127, 1, 0, 0]; w = 1 everywhere ->
    # w_scale 1, u = 1; acc = 128 and 128/127 = 1.00787 rounds to the bf16
    # 1 + 2^-7 (0x3F81).  Bias 2^-8 then residual -2^-8: 1 + 2^-7 + 2^-8 is a
    # tie that goes to the even 1 + 2^-6 (0x3F82), and 1 + 2^-6 - 2^-8 is a
    # tie that stays at 0x3F82.  The other order would give 1 (0x3F80).
    x = torch_bf16_bits(np.array([[1.0, 2.0 ** -7, 0.0, 0.0]], np.float32))
    packed, ws = oracle.pack_weights(np.ones((1, 4), np.float32))
    assert oracle.forward(x, packed, ws).tolist() == [[0x3F81]]
    y = oracle.forward(x, packed, ws, bias=np.array([0x3B80], np.uint16),
                       residual=np.array([[0xBB80]], np.uint16))
    assert y.tolist() == [[0x3F82]]


# ---------------------------------------------------------------- bf16 export (R13)

def test_export_hand_example_and_torch_division():
    # w = [0.5, -1.5, 1, 1] -> w_scale 1, u = [0, -1, 1, 1] -> bf16 [0, -1, 1, 1]
    packed, ws = oracle.pack_weights(np.array([[0.5, -1.5, 1.0, 1.0]], np.float32))
    assert oracle.export_bf16(packed, ws).tolist() == [[0x0000, 0xBF80, 0x3F80, 0x3F80]]
    # scale 3: 1/3 in fp32 is 0x3EAAAAAB, which rounds up to the bf16 0x3EAB;
    # code 3 (value +2) exports as 2/3
    packed = np.array([[0b11100100]], np.uint8)  # codes 0, 1, 2, 3 -> u = -1, 0, 1, 2
    assert oracle.export_bf16(packed, np.float32(3.0)).tolist() == [[0xBEAB, 0x0000, 0x3EAB, 0x3F2B]]
    # against torch's fp32 division and bf16 cast on a workload tensor
    wl = wls.WORKLOADS["layer_8b"]
    w = wls.weights(wl, 1)[:64]
    packed, ws = oracle.pack_weights(w)
    u = torch.from_numpy(oracle.unpack(packed).astype(np.float32))
    want = (u / torch.tensor(ws, dtype=torch.float32)).to(torch.bfloat16)
    assert np.array_equal(oracle.export_bf16(packed, ws), want.view(torch.int16).numpy().view(np.uint16))
