"""The measurement probes of libmp_probe.so (include/mp_probe.h) on the GPU. The rates that
bench.py reports beside the datasheet peaks come from these kernels, so the tests check that they
move and compute what they claim: the copy reproduces its source, the write leaves its documented
pattern, the read's per-block XOR matches the host's, and the matrix-core probe's clock counters
advance at a plausible shader clock for both MFMA forms and both operand kinds."""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

NBYTES = 64 << 20                 # 4096 rounds of 16 KiB (256 threads x 4 vectors of 16 bytes)
ROUND_VECS = 1024


def _src():
    g = torch.Generator(device="cuda").manual_seed(5)
    return torch.randint(-2**31, 2**31 - 1, (NBYTES // 4,), dtype=torch.int32, device="cuda", generator=g)


@pytest.mark.parametrize("blocks", [0, 1000])      # one block per 16 KiB; a grid-stride loop over 4096 rounds
@pytest.mark.parametrize("nontemporal", [False, True])
def test_hbm_probe_copy_write_read(blocks, nontemporal):
    require_gpu()
    from mixed_precision_neural_amd import probe
    src = _src()
    dst = torch.zeros_like(src)
    probe.hbm(probe.COPY, src, dst, NBYTES, blocks, nontemporal)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)

    dst.zero_()
    probe.hbm(probe.WRITE, None, dst, NBYTES, blocks, nontemporal)
    v = dst.cpu().numpy().view(np.uint32).reshape(-1, 4)
    i = np.arange(v.shape[0], dtype=np.int64)
    base = i // ROUND_VECS * ROUND_VECS                # lane t writes vectors base + t + 256 u
    assert np.array_equal(v[:, 0], base.astype(np.uint32))
    assert np.array_equal(v[:, 1], ((i - base) % 256).astype(np.uint32))
    assert (v[:, 2] == 0x3C003C00).all() and (v[:, 3] == 0x3C003C00).all()

    rounds = NBYTES // (16 * ROUND_VECS)
    nblk = rounds if blocks == 0 else blocks
    out = torch.zeros(4096, dtype=torch.int32, device="cuda")
    probe.hbm(probe.READ, src, out, NBYTES, blocks, nontemporal)
    torch.cuda.synchronize()
    words = src.cpu().numpy().view(np.uint32).reshape(rounds, -1)
    per_round = np.bitwise_xor.reduce(words, axis=1)
    want = np.zeros(nblk, np.uint32)
    for k in range(rounds):                            # block b reads rounds b, b + nblk, ...
        want[k % nblk] ^= per_round[k]
    assert np.array_equal(out.cpu().numpy().view(np.uint32)[:nblk], want)


@pytest.mark.parametrize("shape", ["16x16x32", "32x32x16"])
@pytest.mark.parametrize("operands", ["constant", "random"])
def test_mfma_probe_counters_and_clock(shape, operands):
    require_gpu()
    from mixed_precision_neural_amd import probe
    sh = probe.MFMA_16X16X32 if shape == "16x16x32" else probe.MFMA_32X32X16
    op = probe.CONSTANT if operands == "constant" else probe.RANDOM
    blocks = 64
    out = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    khz = probe.mfma_clock(blocks, 2000, out, op, sh)
    torch.cuda.synchronize()
    t = out.cpu().numpy().reshape(blocks, 4).astype(np.float64)
    assert khz > 0
    assert (t[:, 1] > t[:, 0]).all() and (t[:, 3] > t[:, 2]).all()    # both counters advanced
    mhz = (t[:, 1] - t[:, 0]) / (t[:, 3] - t[:, 2]) * khz / 1000.0
    assert 300.0 < float(np.median(mhz)) < 3000.0
