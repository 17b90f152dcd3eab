"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer results (packed weights, int8 codes, int32 accumulators) must be
bit-exact; scales bit-exact; bf16 outputs within 1 ulp (and, since both sides
run the same fp32 operations, expected bit-exact -- the count of differing
outputs is asserted to be zero too).  Inputs come from the seeded workload
generator, shared by both sides.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from bit_gemm_bitlinear_amd import workloads as wls

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def bl():
    from bit_gemm_bitlinear_amd import bitlinear

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return bitlinear


# ------------------------------------------------------------------ helpers

def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_distance(a, b):
    def ordered(v):
        v = v.astype(np.int32)
        return np.where(v & 0x8000, -(v & 0x7FFF), v & 0x7FFF)

    return np.abs(ordered(a) - ordered(b))


def assert_bf16_close(got, want, what=""):
    d = ulp_distance(got, want)
    assert d.max(initial=0) <= 1, f"{what}: max ulp distance {d.max()}"
    assert int((d != 0).sum()) == 0, f"{what}: {(d != 0).sum()} outputs differ by 1 ulp"


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# ------------------------------------------------------------------ activation quantization

ACT_SHAPES = [(1, 4), (3, 12), (5, 36), (2, 64), (16, 2048), (7, 516), (33, 14336), (300, 260)]


@pytest.mark.parametrize("m,k", ACT_SHAPES)
def test_act_quant_parity(bl, m, k):
    x, _ = wls.random_case(11, m, 1, k, scale=3.0)
    xb = x.copy()
    if m > 2:
        xb[1] = 0  # all-zero row: clamped scale
        tiny = wls.to_bf16_bits(np.full(k, 3e-7, np.float32) * np.sign(np.arange(k) - k / 2))
        xb[2] = tiny  # sub-threshold row
    q, s = bl.act_quant(dev_bf16(xb))
    q_ref, s_ref = oracle.act_quant(xb)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits(s_ref))


def test_act_quant_ties_round_to_even(bl):
    # amax = 2 -> scale 63.5: +-1 map to +-63.5 (ties), 0.5 to 31.75
    row = wls.to_bf16_bits(np.array([[2.0, 1.0, -1.0, 0.5, 3.0 / 127 * 2, -1.5, 0, 0]], np.float32))
    q, s = bl.act_quant(dev_bf16(row))
    q_ref, s_ref = oracle.act_quant(row)
    assert q.cpu().numpy().tolist() == q_ref.tolist()
    assert q_ref[0, :3].tolist() == [127, 64, -64]


# ------------------------------------------------------------------ weight preparation

def special_weights():
    rng = np.random.default_rng(5)
    out = {
        "zeros": np.zeros((4, 16), np.float32),
        "ties": np.array([[0.5, -1.5, 1.0, 1.0] * 4] * 2, np.float32),
        "subnormal": np.full((3, 8), 1.401298464324817e-45, np.float32) * rng.integers(1, 9, (3, 8)).astype(np.float32),
        "huge": (rng.standard_normal((5, 12)) * 1e37).astype(np.float32),
        "mixed": np.concatenate([rng.standard_normal((2, 64)).astype(np.float32) * 1e-3,
                                 np.full((1, 64), 7.0, np.float32)]),
    }
    w = rng.standard_normal((64, 256)).astype(np.float32) * 0.02
    w[rng.random(w.shape) < 0.3] = 0
    out["sparse30"] = w
    return out


@pytest.mark.parametrize("n,k", [(1, 4), (3, 8), (16, 64), (33, 260), (100, 516), (2048, 2048),
                                 (1, 2 ** 16)])
def test_pack_parity_random(bl, n, k):
    _, w = wls.random_case(21, 1, n, k)
    check_pack(bl, w)


@pytest.mark.parametrize("name", sorted(special_weights()))
def test_pack_parity_special(bl, name):
    check_pack(bl, special_weights()[name])


def check_pack(bl, w):
    packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
    p_ref, ws_ref = oracle.pack_weights(w)
    assert f32_bits(ws.cpu().numpy()[0]) == f32_bits(ws_ref)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    u = bl.unpack_weights(packed).cpu().numpy()
    assert np.array_equal(u, oracle.unpack(p_ref))


def test_pack_order_independent(bl):
    rng = np.random.default_rng(9)
    w = rng.standard_normal((512, 1024)).astype(np.float32) * 0.02
    _, s1 = bl.pack_weights(torch.from_numpy(w).to(DEV))
    perm = rng.permutation(w.size)
    _, s2 = bl.pack_weights(torch.from_numpy(w.reshape(-1)[perm].reshape(w.shape).copy()).to(DEV))
    assert f32_bits(s1.cpu().numpy()) == f32_bits(s2.cpu().numpy())


def test_unpack_code3(bl):
    allb = np.tile(np.arange(256, dtype=np.uint8), (3, 1))
    u = bl.unpack_weights(torch.from_numpy(allb).to(DEV)).cpu().numpy()
    assert np.array_equal(u, oracle.unpack(allb))


# ------------------------------------------------------------------ contraction (int32)

ACC_SHAPES = [
    # decode path (M <= 16)
    (1, 16, 64), (1, 1, 4), (2, 17, 12), (3, 33, 68), (4, 100, 260), (5, 48, 516),
    (8, 300, 1024), (15, 129, 2048 + 64), (16, 64, 256), (16, 3072, 9216), (1, 200, 16384 + 4),
    (4, 40, 14336 * 2), (16, 20, 8192 + 16),
    # long rows: a workgroup streams all of K (several ring rounds, codes read from memory)
    (16, 300, 12288), (8, 100, 65536), (2, 48, 49152 + 64),
    # K split across workgroups with the staged codes close to the LDS code
    # budget (13 rows x 15 slabs per workgroup, 11 x 17, 5 x 40)
    (13, 77, 30720), (11, 50, 20480 + 64), (5, 33, 40960),
    # prefill path (M > 16)
    (17, 16, 64), (33, 130, 260), (128, 128, 256), (200, 257, 516), (300, 64, 12), (129, 40, 2048),
    (100, 257, 1088), (260, 520, 2112),  # K % 128 == 64: a last half-deep slab; ragged N and M
    # more tiles than one round of workgroups on 256 CUs: the last tile column
    # runs as narrow tiles (ragged, and with output rows not 16-byte aligned)
    (2048, 8400, 256), (2048, 8401, 256),
    # few tiles with long K: K split across workgroups (8 and 5 parts), the
    # parts added by the finishing pass (rows of partial sums not 16-byte
    # aligned; a half-deep last slab; ragged M)
    (256, 301, 16384), (200, 300, 8256),
]


@pytest.mark.parametrize("m,n,k", ACC_SHAPES)
def test_forward_acc_parity(bl, m, n, k):
    rng = np.random.default_rng(m * 1000003 + n * 1009 + k)
    q = rng.integers(-128, 128, size=(m, k), dtype=np.int16).astype(np.int8)
    packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.int16).astype(np.uint8)  # incl. code 3
    acc = bl.forward_acc(torch.from_numpy(q).to(DEV), torch.from_numpy(packed).to(DEV))
    ref = oracle.forward_acc(q, packed)
    assert np.array_equal(acc.cpu().numpy(), ref)


# ------------------------------------------------------------------ tiled weight layout

@pytest.mark.parametrize("n,k", [(16, 256), (32, 1024), (48, 14336), (160, 2560), (2048, 2048)])
def test_tile_parity(bl, n, k):
    rng = np.random.default_rng(n * 7 + k)
    packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.int16).astype(np.uint8)
    dp = torch.from_numpy(packed).to(DEV)
    tiled = bl.tile_weights(dp)
    assert tiled.shape == (n // 16, 4 * k)
    assert np.array_equal(tiled.cpu().numpy(), oracle.tile(packed))
    assert torch.equal(bl.untile_weights(tiled), dp)


TILED_ACC_SHAPES = [
    # decode: one row tile, split shape, ring shape, rows over several waves,
    # K split across waves and across workgroups
    (1, 16, 256), (1, 2048, 2048), (3, 32, 1024), (16, 64, 256), (4, 272, 4096),
    (16, 3072, 9216), (8, 112, 65536), (13, 80, 30720), (5, 48, 40960),
    # prefill: one tile, ragged M, K split across workgroups, a narrow tail
    (17, 16, 256), (128, 128, 256), (129, 48, 2048), (200, 304, 16384), (2048, 8448, 256),
]


@pytest.mark.parametrize("m,n,k", TILED_ACC_SHAPES)
def test_forward_acc_tiled_parity(bl, m, n, k):
    rng = np.random.default_rng(m * 1000003 + n * 1009 + k + 1)
    q = rng.integers(-128, 128, size=(m, k), dtype=np.int16).astype(np.int8)
    packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.int16).astype(np.uint8)  # incl. code 3
    tiled = torch.from_numpy(oracle.tile(packed)).to(DEV)
    acc = bl.forward_acc(torch.from_numpy(q).to(DEV), tiled)
    assert np.array_equal(acc.cpu().numpy(), oracle.forward_acc(q, packed))


@pytest.mark.parametrize("m,n,k", [(1, 2048, 2048), (4, 96, 4096), (16, 304, 9216), (64, 208, 512),
                                   (256, 384, 2560)])
def test_forward_tiled_parity(bl, m, n, k):
    x, w = wls.random_case(37, m, n, k, scale=2.0)
    if m > 4:
        x[m // 2] = 0
    p_ref, ws_ref = oracle.pack_weights(w)
    packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
    y = bl.forward(dev_bf16(x), bl.tile_weights(packed), ws)
    assert_bf16_close(host_bits(y), oracle.forward(x, p_ref, ws_ref), f"tiled {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 3, 16, 40, 300])
def test_grouped_mixed_layouts(bl, m):
    """Tiled and row-major projections in one launch, with a ragged
    row-major one that makes the launch use the narrow-load variants (the
    tiled projections then take their weights through those kernels)."""
    shapes = [(64, 256, True), (33, 260, False), (96, 1024, True), (40, 1024, False)]
    xs, ps, ss, refs = [], [], [], []
    for i, (n, k, tiled) in enumerate(shapes):
        x, w = wls.random_case(90 + 5 * m + i, m, n, k)
        p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
        xs.append(dev_bf16(x))
        ps.append(bl.tile_weights(p) if tiled else p)
        ss.append(s)
        refs.append(oracle.forward(x, *oracle.pack_weights(w)))
    for use in (slice(0, 4), slice(2, 4)):  # with and without the ragged projection
        ys = bl.forward_grouped(xs[use], ps[use], ss[use])
        for (n, k, t), y, r in zip(shapes[use], ys, refs[use]):
            assert_bf16_close(host_bits(y), r, f"mixed {m}x{n}x{k} tiled={t}")


@pytest.mark.parametrize("n,k,tiled", [(96, 512, True), (96, 512, False), (40, 260, True)])
def test_bitlinear_layer_class(bl, n, k, tiled):
    """The BitLinear layer class: packs once (tiled when the shape allows and
    asked for), takes activations of any leading shape."""
    x, w = wls.random_case(77, 6, n, k)
    layer = bl.BitLinear(torch.from_numpy(w).to(DEV), tiled=tiled)
    uses_tiles = tiled and n % 16 == 0 and k % 256 == 0
    assert tuple(layer.packed.shape) == ((n // 16, 4 * k) if uses_tiles else (n, k // 4))
    y = layer(dev_bf16(x).reshape(2, 3, k))
    assert tuple(y.shape) == (2, 3, n)
    y_ref = oracle.forward(x, *oracle.pack_weights(w))
    assert_bf16_close(host_bits(y.reshape(6, n).contiguous()), y_ref, "BitLinear class")


# ------------------------------------------------------------------ forward (bf16)

FWD_SHAPES = [(1, 16, 64), (1, 2048, 2048), (3, 50, 36), (8, 2048, 2048), (16, 96, 4096),
              (16, 300, 9216), (17, 64, 256), (64, 200, 516), (256, 384, 2560), (40, 1000, 68),
              (72, 250, 1088),
              # activation quantization of the prefill path: a half group (K % 16 == 8),
              # the 16-group-per-lane variant, and rows too long for it
              (48, 96, 1048), (20, 64, 14336), (18, 32, 16400),
              # decode with K split across workgroups near the LDS code budget
              (13, 64, 30720),
              # prefill with K split across workgroups (ragged output rows)
              (300, 201, 16448), (130, 256, 12288)]


@pytest.mark.parametrize("m,n,k", FWD_SHAPES)
def test_forward_parity(bl, m, n, k):
    x, w = wls.random_case(31, m, n, k, scale=2.0)
    if m > 4:
        x[m // 2] = 0
    p_ref, ws_ref = oracle.pack_weights(w)
    y_ref = oracle.forward(x, p_ref, ws_ref)
    packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
    y = bl.forward(dev_bf16(x), packed, ws)
    assert_bf16_close(host_bits(y), y_ref, f"forward {m}x{n}x{k}")


def test_forward_deterministic_and_grouped_equals_single(bl):
    xs, ps, ss, refs = [], [], [], []
    for i, (n, k) in enumerate([(64, 256), (100, 1024), (33, 9216)]):
        x, w = wls.random_case(40 + i, 4, n, k)
        p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
        xs.append(dev_bf16(x))
        ps.append(p)
        ss.append(s)
        refs.append(oracle.forward(x, *oracle.pack_weights(w)))
    ys = bl.forward_grouped(xs, ps, ss)
    ys2 = bl.forward_grouped(xs, ps, ss)
    for y, y2, x, p, s, r in zip(ys, ys2, xs, ps, ss, refs):
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        assert torch.equal(y.view(torch.int16), bl.forward(x, p, s).view(torch.int16))
        assert_bf16_close(host_bits(y), r)


@pytest.mark.parametrize("m", [1, 3, 16])
def test_grouped_ragged_layer(bl, m):
    """A layer whose row counts are not multiples of the workgroup's rows and
    whose K ranges differ: the layer-level plan (one workgroup per CU, rows
    and K split over the waves, 1-4 row tiles per wave) must cover every
    output exactly once."""
    shapes = [(1000, 2048), (3001, 3072), (70, 4352), (4100, 1024), (17, 8192), (2500, 2560)]
    xs, ps, ss, refs = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        x, w = wls.random_case(60 + 7 * m + i, m, n, k)
        p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
        xs.append(dev_bf16(x))
        ps.append(p)
        ss.append(s)
        refs.append(oracle.forward(x, *oracle.pack_weights(w)))
    ys = bl.forward_grouped(xs, ps, ss)
    for (n, k), y, r in zip(shapes, ys, refs):
        assert_bf16_close(host_bits(y), r, f"grouped ragged {m}x{n}x{k}")


def test_golden_cases(bl):
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small_cases.json")
    for c in json.load(open(path))["cases"]:
        x, w = wls.random_case(c["seed"], c["M"], c["N"], c["K"], scale=c["scale"])
        packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
        assert packed.cpu().numpy().tobytes().hex() == c["packed_hex"]
        assert int(f32_bits(ws.cpu().numpy()[0])) == c["w_scale_bits"]
        y = bl.forward(dev_bf16(x), packed, ws)
        assert host_bits(y).tolist() == c["y_bits"]
        acc = bl.forward_acc(torch.tensor(c["q"], dtype=torch.int8, device=DEV), packed)
        assert acc.cpu().numpy().tolist() == c["acc"]


# Grouped prefill launches with more tiles than one round of workgroups
# (2 per CU on 256 CUs), shaped so that the launch plan runs the last tile
# columns of the last projection as narrow tiles: 4 of 12 columns (narrow
# part 953 columns, ragged), 1 of 2 (44 columns), and the whole projection
# (200 columns, 25 row tiles).
NARROW_LAYERS = [
    (2000, [(7000, 2048), (3001, 1088)]),
    (3000, [(5000, 2048), (300, 1024)]),
    (3200, [(5000, 2048), (200, 1024)]),
]


@pytest.mark.parametrize("m,shapes", NARROW_LAYERS)
def test_grouped_prefill_narrow_tail(bl, m, shapes):
    xs, ps, ss, refs = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        x, w = wls.random_case(90 + m + i, m, n, k)
        p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
        xs.append(dev_bf16(x))
        ps.append(p)
        ss.append(s)
        refs.append(oracle.forward(x, *oracle.pack_weights(w)))
    ys = bl.forward_grouped(xs, ps, ss)
    for (n, k), y, r in zip(shapes, ys, refs):
        assert_bf16_close(host_bits(y), r, f"grouped prefill {m}x{n}x{k}")


# ------------------------------------------------------------------ full-size workloads

def workload_cases():
    out = []
    for wl in wls.WORKLOADS.values():
        for m in wl.ms:
            for v in wls.variants(wl, m):
                out.append(pytest.param(wl.name, m, v, id=f"{wl.name}-m{m}-v{v}"))
    return out


_PACK_CACHE = {}


def packed_workload(bl, wl):
    """GPU-packed weights of every projection, checked bit-exact against the
    oracle the first time a workload is used, and their tiled layout (two
    sampled blocks of 16 rows checked against the oracle's tiling)."""
    if wl.name not in _PACK_CACHE:
        _PACK_CACHE.clear()
        entries = []
        for pi in range(len(wl.projections)):
            w = wls.weights(wl, pi)
            p_ref, s_ref = oracle.pack_weights(w)
            p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
            assert f32_bits(s.cpu().numpy()[0]) == f32_bits(s_ref), wl.projections[pi].name
            assert torch.equal(p.cpu(), torch.from_numpy(p_ref)), wl.projections[pi].name
            t = bl.tile_weights(p)
            nb = p_ref.shape[0] // 16
            for b in (0, nb // 2 + 1, nb - 1):
                assert np.array_equal(t[b].cpu().numpy(),
                                      oracle.tile(p_ref[16 * b:16 * b + 16]).reshape(-1))
            entries.append((p, s, p_ref, s_ref, t))
            del w
        _PACK_CACHE[wl.name] = entries
    return _PACK_CACHE[wl.name]


@pytest.mark.parametrize("name,m,variant", workload_cases())
def test_workload_parity(bl, name, m, variant):
    """Every projection of the workload, full size, in one grouped call
    (the launch configuration the benchmark times, whose weights are tiled),
    with the weights in both layouts."""
    wl = wls.WORKLOADS[name]
    entries = packed_workload(bl, wl)
    xs = [wls.activations(wl, pi, m, variant) for pi in range(len(wl.projections))]
    dxs = [dev_bf16(x) for x in xs]
    scales = [e[1] for e in entries]
    ys = bl.forward_grouped(dxs, [e[0] for e in entries], scales)
    yts = bl.forward_grouped(dxs, [e[4] for e in entries], scales)
    for pi, (x, y, yt, e) in enumerate(zip(xs, ys, yts, entries)):
        y_ref = oracle.forward(x, e[2], e[3])
        assert_bf16_close(host_bits(y), y_ref, f"{name} {wl.projections[pi].name} M={m}")
        assert_bf16_close(host_bits(yt), y_ref, f"{name} {wl.projections[pi].name} M={m} tiled")
