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


def test_concurrent_calls_from_threads(bl):
    """Calls from several host threads at once, each on its own stream with
    its own workspace (ctypes releases the interpreter lock during each
    call, so the library's host code runs concurrently): decode layers with
    fused and with staged codes and a GEMM layer, repeated; every result
    equals the oracle's."""
    import threading

    cases = []
    for t, (m, shapes) in enumerate([(1, [(256, 2048), (64, 4096)]),
                                     (8, [(128, 1024), (96, 3072)]),
                                     (48, [(256, 1024), (64, 2048)])]):
        xs, ps, ss, refs = [], [], [], []
        for i, (n, k) in enumerate(shapes):
            x, w = wls.random_case(500 + 10 * t + i, m, n, k)
            p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
            xs.append(dev_bf16(x))
            ps.append(bl.tile_weights(p))
            ss.append(s)
            refs.append(oracle.forward(x, *oracle.pack_weights(w)))
        cases.append((xs, ps, ss, refs))
    torch.cuda.synchronize()
    errors = []

    def worker(xs, ps, ss, refs):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                call = bl.GroupedCall(xs, ps, ss)
                outs = []
                for _ in range(30):
                    ys = call()
                    outs.append([y.clone() for y in ys])
            stream.synchronize()
            for ys in outs:
                for y, r in zip(ys, refs):
                    if not np.array_equal(host_bits(y), r):
                        errors.append("a result differs from the oracle")
                        return
        except Exception as e:  # reported in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=c) for c in cases for _ in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:3]


@pytest.mark.parametrize("m,shapes", [
    (1, [(256, 2048), (64, 4096)]),     # decode, fused quantization
    (16, [(128, 3072), (96, 9216)]),    # decode, staged codes, K split across workgroups
    (48, [(256, 1024), (64, 8192)]),    # GEMM with 64-row tiles and a K-part sum
])
def test_graph_replay_matches_oracle(bl, m, shapes):
    """A grouped forward captured in a HIP graph and replayed three times,
    with new inputs copied in eagerly and a synchronization between the
    replays: every replay's outputs equal the oracle's for that replay's
    inputs (the split-K partial sums and counters that must start at zero
    are cleared by a kernel of the call, not by a memset node)."""
    ws = []
    for i, (n, k) in enumerate(shapes):
        _, w = wls.random_case(700 + i, 1, n, k)
        ws.append(w)
    packs = [bl.pack_weights(torch.from_numpy(w).to(DEV)) for w in ws]
    refs_w = [oracle.pack_weights(w) for w in ws]
    xs = [torch.zeros((m, k), dtype=torch.bfloat16, device=DEV) for _, k in shapes]
    call = bl.GroupedCall(xs, [p for p, _ in packs], [s for _, s in packs])
    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        new = [wls.random_case(710 + 10 * rep + i, m, n, k)[0] for i, (n, k) in enumerate(shapes)]
        for x, b in zip(xs, new):
            x.copy_(dev_bf16(b))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (n, k), y, b, (p_ref, s_ref) in zip(shapes, call.outs, new, refs_w):
            assert_bf16_close(host_bits(y), oracle.forward(b, p_ref, s_ref),
                              f"graph replay {rep}, {m}x{n}x{k}")


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


def check_inspection(name, x, y, ins, p_ref, s_ref, y_ref):
    """The forward path's own intermediates against the oracle: int8 codes,
    scales and code sums bit for bit (the blog's activation_norm_quant), the
    int32 accumulators bit for bit (the F.linear contraction), and the bf16
    output."""
    q_ref, xs_ref = oracle.act_quant(x)
    q = ins["q"].cpu().numpy()
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, f"{name}: {len(bad)} codes differ, first at {bad[0].tolist()}"
    assert np.array_equal(f32_bits(ins["x_scale"].cpu().numpy()), f32_bits(xs_ref)), f"{name}: scales"
    assert np.array_equal(ins["qsum"].cpu().numpy(), q_ref.astype(np.int64).sum(axis=1)), f"{name}: sums"
    acc_ref = oracle.contract(q_ref, oracle.unpack(p_ref))
    assert np.array_equal(ins["acc"].cpu().numpy(), acc_ref), f"{name}: accumulators"
    assert_bf16_close(host_bits(y), y_ref, f"{name} (inspect call)")


@pytest.mark.parametrize("name,m,variant", workload_cases())
def test_workload_parity(bl, name, m, variant):
    """Every projection of the workload, full size, in one grouped call
    (the launch configuration the benchmark times, whose weights are tiled),
    with the weights in both layouts.  The inspection call runs the same
    kernels and also returns the codes, scales, code sums and int32
    accumulators the forward path computed; each is compared element by
    element with the oracle."""
    wl = wls.WORKLOADS[name]
    entries = packed_workload(bl, wl)
    xs = [wls.activations(wl, pi, m, variant) for pi in range(len(wl.projections))]
    dxs = [dev_bf16(x) for x in xs]
    scales = [e[1] for e in entries]
    ys = bl.forward_grouped(dxs, [e[0] for e in entries], scales)
    yts = bl.forward_grouped(dxs, [e[4] for e in entries], scales)
    yis, inss, status = bl.forward_grouped_inspect(dxs, [e[4] for e in entries], scales)
    yri, insr, status_r = bl.forward_grouped_inspect(dxs, [e[0] for e in entries], scales)
    assert int(status.item()) == 0 and int(status_r.item()) == 0
    for pi, (x, y, yt, e) in enumerate(zip(xs, ys, yts, entries)):
        what = f"{name} {wl.projections[pi].name} M={m}"
        y_ref = oracle.forward(x, e[2], e[3])
        assert_bf16_close(host_bits(y), y_ref, what)
        assert_bf16_close(host_bits(yt), y_ref, f"{what} tiled")
        assert torch.equal(yis[pi].view(torch.int16), yt.view(torch.int16)), f"{what}: inspect call"
        check_inspection(f"{what} tiled", x, yis[pi], inss[pi], e[2], e[3], y_ref)
        check_inspection(f"{what} rows", x, yri[pi], insr[pi], e[2], e[3], y_ref)


def workload_shapes():
    """(workload, M, projection index) for every projection shape of every
    workload at its own token counts."""
    out = []
    for wl in wls.WORKLOADS.values():
        for m in wl.ms:
            for pi, p in enumerate(wl.projections):
                out.append(pytest.param(wl.name, m, pi, id=f"{wl.name}-m{m}-{p.name}"))
    return out


@pytest.mark.parametrize("name,m,pi", workload_shapes())
def test_forward_acc_with_oracle_codes(bl, name, m, pi):
    """The contraction alone at every workload shape: the oracle's own codes
    of the workload's activations against the GPU-packed, tiled weights; every
    int32 accumulator bit-equal to the oracle's."""
    wl = wls.WORKLOADS[name]
    entries = packed_workload(bl, wl)
    x = wls.activations(wl, pi, m, wls.variants(wl, m)[-1])
    q_ref, _ = oracle.act_quant(x)
    _, _, p_ref, _, tiled = entries[pi]
    acc = bl.forward_acc(torch.from_numpy(q_ref).to(DEV), tiled)
    assert np.array_equal(acc.cpu().numpy(), oracle.contract(q_ref, oracle.unpack(p_ref)))


def tie_rows(m, k, seed):
    """Rows whose codes are decided by round-half-to-even: absmax 127/64 (so
    the scale is exactly 64) and values (2j+1)/128, which scale to j + 0.5."""
    rng = np.random.default_rng(seed)
    j = rng.integers(-63, 63, size=(m, k))
    xf = ((2 * j + 1) / 128.0).astype(np.float32)
    xf[np.arange(m), rng.integers(0, k, size=m)] = np.float32(127 / 64) * np.where(
        rng.random(m) < 0.5, 1, -1).astype(np.float32)
    return wls.to_bf16_bits(xf)


# fused decode quantizer (M <= 4); decode rows staged by the activation kernel
# (M = 8, 16); GEMM rows, a workgroup per row (M = 40) and one, two or four
# waves per row (1100 or 1030 rows); the general row path (K % 8 != 0; K past
# the register batch)
@pytest.mark.parametrize("m,k", [(1, 2048), (4, 2048), (8, 2048), (16, 4096), (40, 1024),
                                 (1100, 2560), (1100, 6912), (1030, 14336), (24, 1036),
                                 (20, 16400)])
def test_forward_path_ties_round_to_even(bl, m, k):
    """Ties through the forward path's own quantizers: every code, scale and
    code sum equals the oracle's round-half-to-even result."""
    x = tie_rows(m, k, 100 + m)
    q_ref, s_ref = oracle.act_quant(x)
    assert np.all(s_ref == np.float32(64.0))
    frac = bf16_bits_to_f32(x) * np.float32(64.0)
    ties = np.abs(frac - np.floor(frac)) == 0.5
    assert ties.mean() > 0.9 and np.all(q_ref[ties] % 2 == 0)
    _, w = wls.random_case(7, 1, 64, k)
    p_ref, ws_ref = oracle.pack_weights(w)
    packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
    weights = bl.tile_weights(packed) if k % 256 == 0 else packed
    ys, inss, status = bl.forward_grouped_inspect([dev_bf16(x)], [weights], [ws])
    assert int(status.item()) == 0
    check_inspection(f"ties M={m} K={k}", x, ys[0], inss[0], p_ref, ws_ref,
                     oracle.forward(x, p_ref, ws_ref))


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_decode_wait_giveup_is_reported(bl):
    """The decode kernel's waits between its waves are bounded.  Forced to
    give up at once (wait_polls < 0, host-side), the split-shape launch must
    report it in the status word and poison its outputs (NaN / INT32_MIN)
    instead of returning numbers.  A following default call is exact again."""
    wl = wls.WORKLOADS["decode_1b_m1"]
    entries = packed_workload(bl, wl)
    xs = [dev_bf16(wls.activations(wl, pi, 1)) for pi in range(len(wl.projections))]
    packs, scales = [e[4] for e in entries], [e[1] for e in entries]
    ys, inss, status = bl.forward_grouped_inspect(xs, packs, scales, wait_polls=-1)
    assert int(status.item()) == 1
    for y, ins in zip(ys, inss):
        assert torch.all(y.view(torch.int16) == 0x7FC0), "outputs not poisoned"
        assert torch.all(ins["acc"] == -2 ** 31)
    ys2, _, status2 = bl.forward_grouped_inspect(xs, packs, scales)
    assert int(status2.item()) == 0
    for pi, y in enumerate(ys2):
        x = wls.activations(wl, pi, 1)
        assert_bf16_close(host_bits(y), oracle.forward(x, entries[pi][2], entries[pi][3]))


def test_binding_rejects_bad_outputs_and_scales(bl):
    """The binding checks caller-supplied outputs, scales and workspaces
    before the library sees them (wrong shape, dtype or device)."""
    x = torch.zeros((2, 256), dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros((32, 64), dtype=torch.uint8, device=DEV)
    ws = torch.ones(1, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        bl.forward(x, packed, ws, out=torch.empty((2, 31), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(TypeError):
        bl.forward(x, packed, ws, out=torch.empty((2, 32), dtype=torch.float32, device=DEV))
    with pytest.raises(TypeError):
        bl.forward(x, packed, torch.ones(1, dtype=torch.float32))  # host scale
    with pytest.raises(TypeError):
        bl.forward(x, packed, torch.ones(0, dtype=torch.float32, device=DEV))
    with pytest.raises(TypeError):
        bl.forward(x, packed, ws, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        bl.forward_acc(torch.zeros((2, 256), dtype=torch.int8, device=DEV), packed,
                       out=torch.empty((2, 32, 1), dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        bl.GroupedCall([x], [packed], [ws], outs=[torch.empty((3, 32), dtype=torch.bfloat16,
                                                              device=DEV)])
    # a workspace of 4-byte elements is counted in bytes
    need = bl.forward_grouped_workspace_bytes(2, [(32, 256)])
    wsp = torch.empty((need + 3) // 4, dtype=torch.int32, device=DEV)
    y = bl.GroupedCall([x], [packed], [ws], workspace=wsp)()
    torch.cuda.synchronize()
    assert y[0].shape == (2, 32)


# ------------------------------------------------------------------ bias and residual

def rand_bf16(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return wls.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


# decode: fused quantization (M <= 4), staged codes (M = 8), K split across
# workgroups (M = 16, K = 9216); prefill: one tile, K split across
# workgroups (the finishing pass), ragged N; rows not 16-byte aligned
# (K % 64 != 0: the register-staged prefill kernel and narrow decode loads)
def test_rows_kernel_multi_wave_rows(bl):
    """The GEMM's activation kernel with one, two and four waves per row (up
    to 256, 512 and 1024 groups of 16 codes) in one launch of four jobs, with
    rows that end in half a group (K % 16 == 8) and the padding rows of the
    128-row tiles (M = 300): codes, scales, code sums, accumulators and
    outputs against the oracle."""
    m = 300
    shapes = [(64, 1032), (64, 4104), (48, 8200), (32, 16384)]
    xs, ps, ss, refs = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        x, w = wls.random_case(300 + i, m, n, k)
        p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
        xs.append(x)
        ps.append(p)
        ss.append(s)
        refs.append(oracle.pack_weights(w))
    ys, inss, status = bl.forward_grouped_inspect([dev_bf16(x) for x in xs], ps, ss)
    assert int(status.item()) == 0
    for (n, k), x, y, ins, (p_ref, ws_ref) in zip(shapes, xs, ys, inss, refs):
        check_inspection(f"rows kernel {m}x{n}x{k}", x, y, ins, p_ref, ws_ref,
                         oracle.forward(x, p_ref, ws_ref))


BIAS_SHAPES = [(1, 2048, 2048), (4, 96, 4096), (8, 300, 1024), (16, 640, 9216), (40, 200, 1024),
               (256, 301, 16384), (300, 264, 2560), (3, 100, 1036), (70, 136, 1036)]


@pytest.mark.parametrize("m,n,k", BIAS_SHAPES)
def test_forward_bias_residual_parity(bl, m, n, k):
    """BitLinear.forward's bias line (and a residual add after it) in the
    epilogue: (bf16(y) + bias) + residual, each add rounded to bf16, exactly
    as the oracle computes it; also with the residual in place (it is y)."""
    x, w = wls.random_case(50, m, n, k, scale=2.0)
    bias = rand_bf16(51 + m, (n,), 0.5)
    res = rand_bf16(52 + m, (m, n))
    p_ref, ws_ref = oracle.pack_weights(w)
    packed, ws = bl.pack_weights(torch.from_numpy(w).to(DEV))
    dx, db, dr = dev_bf16(x), dev_bf16(bias), dev_bf16(res)
    y = bl.forward(dx, packed, ws, bias=db)
    assert_bf16_close(host_bits(y), oracle.forward(x, p_ref, ws_ref, bias=bias), f"bias {m}x{n}x{k}")
    y = bl.forward(dx, packed, ws, residual=dr)
    assert_bf16_close(host_bits(y), oracle.forward(x, p_ref, ws_ref, residual=res), f"res {m}x{n}x{k}")
    want = oracle.forward(x, p_ref, ws_ref, bias=bias, residual=res)
    y = bl.forward(dx, packed, ws, bias=db, residual=dr)
    assert_bf16_close(host_bits(y), want, f"bias+res {m}x{n}x{k}")
    inplace = dr.clone()  # y += BitLinear(x): the residual buffer is the output
    bl.forward(dx, packed, ws, bias=db, residual=inplace, out=inplace)
    assert_bf16_close(host_bits(inplace), want, f"in place {m}x{n}x{k}")
    if n % 16 == 0 and k % 256 == 0:
        y = bl.forward(dx, bl.tile_weights(packed), ws, bias=db, residual=dr)
        assert_bf16_close(host_bits(y), want, f"tiled bias+res {m}x{n}x{k}")


@pytest.mark.parametrize("name,m", [("decode_1b_m1", 1), ("decode_3b", 16),
                                    ("prefill_2b_m2048", 2048), ("layer_8b", 4),
                                    ("decode_3b", 4)])
def test_grouped_bias_residual_workload(bl, name, m):
    """Bias and residual on every projection of a workload in one grouped
    call (the decode kernel's split and ring shapes with staged and fused
    codes, the 4-row split instance with the larger code budget, the GEMM
    with its narrow tail)."""
    wl = wls.WORKLOADS[name]
    entries = packed_workload(bl, wl)
    xs = [wls.activations(wl, pi, m) for pi in range(len(wl.projections))]
    biases = [rand_bf16(60 + pi, (p.n,), 0.25) for pi, p in enumerate(wl.projections)]
    ress = [rand_bf16(70 + pi, (m, p.n)) for pi, p in enumerate(wl.projections)]
    call = bl.GroupedCall([dev_bf16(x) for x in xs], [e[4] for e in entries], [e[1] for e in entries],
                          biases=[dev_bf16(b) for b in biases], residuals=[dev_bf16(r) for r in ress])
    ys = call()
    for pi, (x, y, e) in enumerate(zip(xs, ys, entries)):
        want = oracle.forward(x, e[2], e[3], bias=biases[pi], residual=ress[pi])
        assert_bf16_close(host_bits(y), want, f"{name} {wl.projections[pi].name} bias+res")


def test_grouped_narrow_tail_bias(bl):
    """A grouped GEMM launch whose last projection runs partly as narrow
    tiles: the bias and residual of those columns are offset with them."""
    m, shapes = NARROW_LAYERS[0]
    xs, ps, ss, bs, rs, refs = [], [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        x, w = wls.random_case(190 + i, m, n, k)
        p, s = bl.pack_weights(torch.from_numpy(w).to(DEV))
        b, r = rand_bf16(200 + i, (n,)), rand_bf16(210 + i, (m, n))
        xs.append(dev_bf16(x))
        ps.append(p)
        ss.append(s)
        bs.append(dev_bf16(b))
        rs.append(dev_bf16(r))
        refs.append(oracle.forward(x, *oracle.pack_weights(w), bias=b, residual=r))
    ys = bl.GroupedCall(xs, ps, ss, biases=bs, residuals=rs)()
    for (n, k), y, ref in zip(shapes, ys, refs):
        assert_bf16_close(host_bits(y), ref, f"narrow tail {m}x{n}x{k} bias+res")


# ------------------------------------------------------------------ bf16 export

@pytest.mark.parametrize("n,k", [(1, 4), (16, 256), (33, 260), (64, 1088), (2048, 2048), (48, 14336)])
def test_export_bf16_parity(bl, n, k):
    """u / w_scale as bf16 from the packed codes (code 3 included), both
    layouts, against the oracle's export."""
    rng = np.random.default_rng(n + 3 * k)
    packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.int16).astype(np.uint8)
    s = np.float32(rng.random() * 50 + 0.5)
    ds = torch.tensor([s], dtype=torch.float32, device=DEV)
    out = bl.export_bf16(torch.from_numpy(packed).to(DEV), ds)
    want = oracle.export_bf16(packed, s)
    assert np.array_equal(host_bits(out), want)
    if n % 16 == 0 and k % 256 == 0:
        out_t = bl.export_bf16(torch.from_numpy(oracle.tile(packed)).to(DEV), ds, k=k)
        assert np.array_equal(host_bits(out_t), want)


def test_export_bf16_of_a_workload_projection(bl):
    """The export of GPU-packed workload weights equals the oracle's export of
    the oracle's packing."""
    wl = wls.WORKLOADS["layer_8b"]
    entries = packed_workload(bl, wl)
    p, s, p_ref, s_ref, t = entries[1]
    out = bl.export_bf16(t, s, k=wl.projections[1].k)
    assert np.array_equal(host_bits(out), oracle.export_bf16(p_ref, s_ref))


# ------------------------------------------------------------------ on-the-fly ternarization

@pytest.mark.parametrize("m,n,k", [(1, 2048, 2048), (4, 100, 260), (16, 640, 9216), (40, 200, 1024),
                                   (300, 257, 2560)])
def test_forward_latent_parity(bl, m, n, k):
    """The forward pass on latent fp32 weights (exact absmean, then
    ternarization and packing, then the forward) equals the oracle's
    pack-then-forward, scale included."""
    x, w = wls.random_case(80, m, n, k, scale=2.0)
    w[np.random.default_rng(81).random(w.shape) < 0.3] = 0
    y, ws = bl.forward_latent(dev_bf16(x), torch.from_numpy(w).to(DEV))
    p_ref, ws_ref = oracle.pack_weights(w)
    assert f32_bits(ws.cpu().numpy()[0]) == f32_bits(ws_ref)
    assert_bf16_close(host_bits(y), oracle.forward(x, p_ref, ws_ref), f"latent {m}x{n}x{k}")


# ------------------------------------------------------------------ mid-M (16 < M < 256)

MID_ACC_SHAPES = [
    # 32-row tiles (17..32 tokens), 64-row tiles (33..64), 128-row tiles
    # (65..); every launch with few tiles runs them all narrow; K split across
    # workgroups where one projection's K dominates; ragged N, K % 128 == 64
    (17, 16, 256), (32, 300, 1024), (33, 130, 2112), (48, 257, 4096), (64, 200, 16384),
    (65, 136, 2048), (100, 257, 1088), (128, 640, 4096), (20, 4096, 14336),
]


@pytest.mark.parametrize("m,n,k", MID_ACC_SHAPES)
def test_mid_m_forward_acc_parity(bl, m, n, k):
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    q = rng.integers(-128, 128, size=(m, k), dtype=np.int16).astype(np.int8)
    packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.int16).astype(np.uint8)  # incl. code 3
    ref = oracle.forward_acc(q, packed)
    acc = bl.forward_acc(torch.from_numpy(q).to(DEV), torch.from_numpy(packed).to(DEV))
    assert np.array_equal(acc.cpu().numpy(), ref)
    if n % 16 == 0 and k % 256 == 0:
        acc = bl.forward_acc(torch.from_numpy(q).to(DEV), torch.from_numpy(oracle.tile(packed)).to(DEV))
        assert np.array_equal(acc.cpu().numpy(), ref)


@pytest.mark.parametrize("m", [2, 3, 4, 5, 8, 16])
def test_layer_8b_few_rows_parity(bl, m):
    """The 8B-class layer at 2-16 token rows.  Up to 4 rows take the
    layer-level split plan with every projection quantized inside the
    kernel, the down projection's 4 x 14336 codes included (the split
    shape's larger code budget): one launch.  From 5 rows the codes are
    staged by the activation kernel (two launches), and the per-projection
    plans take the larger chunk target, so waves stream 28-32 chunks in
    four ring rounds (K split across workgroups for the down projection).
    Codes, scales, code sums, accumulators and outputs against the oracle."""
    wl = wls.WORKLOADS["layer_8b"]
    entries = packed_workload(bl, wl)
    shapes = [(p.n, p.k) for p in wl.projections]
    assert bl.forward_grouped_launches(m, shapes) == (1 if m <= 4 else 2)
    xs = [wls.activations(wl, pi, m) for pi in range(len(wl.projections))]
    dxs = [dev_bf16(x) for x in xs]
    ys, inss, status = bl.forward_grouped_inspect(dxs, [e[4] for e in entries], [e[1] for e in entries])
    assert int(status.item()) == 0
    plain = bl.forward_grouped(dxs, [e[4] for e in entries], [e[1] for e in entries])
    for pi, (x, y, yp, ins, e) in enumerate(zip(xs, ys, plain, inss, entries)):
        check_inspection(f"layer_8b {wl.projections[pi].name} M={m}", x, y, ins, e[2], e[3],
                         oracle.forward(x, e[2], e[3]))
        assert torch.equal(yp.view(torch.int16), y.view(torch.int16)), "plain call differs"


@pytest.mark.parametrize("name,m", [(n, m) for n in ("decode_3b", "layer_8b")
                                    for m in (17, 32, 64, 100, 128)])
def test_mid_m_workload_parity(bl, name, m):
    """The 3B- and 8B-class layers at mid-range token counts, one grouped
    call on tiled weights, with the forward path's codes, scales, code sums
    and accumulators compared element by element with the oracle."""
    wl = wls.WORKLOADS[name]
    entries = packed_workload(bl, wl)
    xs = [wls.activations(wl, pi, m) for pi in range(len(wl.projections))]
    ys, inss, status = bl.forward_grouped_inspect([dev_bf16(x) for x in xs],
                                                  [e[4] for e in entries], [e[1] for e in entries])
    assert int(status.item()) == 0
    for pi, (x, y, ins, e) in enumerate(zip(xs, ys, inss, entries)):
        check_inspection(f"{name} {wl.projections[pi].name} M={m}", x, y, ins, e[2], e[3],
                         oracle.forward(x, e[2], e[3]))
