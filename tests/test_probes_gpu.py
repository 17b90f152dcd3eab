"""GPU checks of the measurement kernels (include/bitlinear_probes.h): their
results are pinned, so the ceilings bench.py reports come from kernels that
really read every byte and really run the matrix-core loop."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def probes():
    from bit_gemm_bitlinear_amd import probes

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return probes


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 20, (3 << 20) + 16])
def test_stream_read_xor(probes, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros(probes.SINK_WORDS, dtype=torch.int32, device=DEV)
    probes.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))


def test_mfma_loop_constant_operands(probes):
    # every operand byte 1: each of the 128 accumulators of a thread gains
    # 32 per round, so a thread's sum is 4096 * iters
    wgs, iters = 300, 37
    sink = torch.full((wgs * 256,), -1, dtype=torch.int32, device=DEV)
    ops = probes.mfma_i8(wgs, iters, 0, sink)
    torch.cuda.synchronize()
    assert ops == 65536 * 8 * 4 * iters * wgs
    assert torch.all(sink == 4096 * iters)


def test_mfma_loop_random_operands_deterministic(probes):
    wgs, iters = 64, 5
    s1 = torch.zeros(wgs * 256, dtype=torch.int32, device=DEV)
    s2 = torch.ones(wgs * 256, dtype=torch.int32, device=DEV)
    probes.mfma_i8(wgs, iters, 1, s1)
    probes.mfma_i8(wgs, iters, 1, s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert int((s1 != 0).sum()) > wgs * 250  # data-dependent sums, not a constant


@pytest.mark.parametrize("n,k", [(16, 256), (2048, 2048), (8192, 4096), (1024, 8192), (48, 768)])
def test_lut_decode_matches_oracle(n, k):
    """The lookup-table contraction (the alternative the decode kernel is
    measured against) gives the oracle's exact accumulators, code 3 and
    q = -128 included."""
    import oracle
    from bit_gemm_bitlinear_amd import probes

    rng = np.random.default_rng(n + k)
    q = rng.integers(-128, 128, size=k, dtype=np.int16).astype(np.int8)
    packed = rng.integers(0, 256, size=(n, k // 4), dtype=np.int16).astype(np.uint8)
    acc = probes.lut_decode_acc(torch.from_numpy(q).cuda(), torch.from_numpy(oracle.tile(packed)).cuda())
    assert np.array_equal(acc.cpu().numpy(), oracle.forward_acc(q[None, :], packed)[0])
