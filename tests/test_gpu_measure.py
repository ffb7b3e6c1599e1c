"""The measurement probes of include/bitlinear_measure.h do the work they
claim: the streaming read touches every byte once (its per-workgroup XOR
checksums fold to the XOR of the whole buffer), and every workgroup of the
matrix-core loop performs iters x 8 MFMAs on the given operands (its checksum
equals the sum of all products, computed here on the host)."""
import numpy as np
import pytest

from gpu_helpers import bl, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20, (64 << 20) + 1040])
def test_stream_read_reads_every_byte(nbytes):
    torch = torch_cuda()
    L = bl()
    say(f"stream read {nbytes} bytes")
    host = np.random.default_rng(nbytes).integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = to_dev(host.view(np.int32))
    sink = torch.zeros(L.bitlinear_measure_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    L.bitlinear_measure_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    words = sink.cpu().numpy().view(np.uint32)   # unwritten words stay 0
    assert np.bitwise_xor.reduce(words) == np.bitwise_xor.reduce(host)


def mfma_checksum(xq: np.ndarray, packed: np.ndarray, iters: int) -> int:
    """Sum of every element of every MFMA result one wavefront accumulates.
    Lane l = 32 g + i supplies row i (A) or column i (B) with 16 bytes whose
    k positions depend only on (g, byte); so the sum over all 32 x 32 outputs
    of one MFMA is sum over (g, byte) of colsum_A * rowsum_B."""
    total = 0
    for j in range(8):
        a = xq[(j * 64) * 16:(j * 64 + 64) * 16].astype(np.int64).reshape(64, 16)
        w = packed[(j * 64) * 4:(j * 64 + 64) * 4].view(np.uint32).astype(np.int64)   # one word per lane
        # column 4 f + byte: byte `byte` of register f of the lane's B fragment
        b = np.stack([(w >> (2 * f + 8 * byte)) & 3 for f in range(4) for byte in range(4)], axis=1)
        for g in range(2):
            total += int((a[32 * g:32 * g + 32].sum(axis=0) * b[32 * g:32 * g + 32].sum(axis=0)).sum())
    return total * iters * 4   # four wavefronts per workgroup


def test_mfma_loop_performs_the_claimed_products():
    torch = torch_cuda()
    L = bl()
    rng = np.random.default_rng(7)
    xq = rng.integers(-127, 128, 8192, dtype=np.int8)
    packed = rng.integers(0, 256, 2048, dtype=np.uint8)   # any bytes: fields 0..3 all multiply
    sink = torch.zeros(L.bitlinear_measure_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    for iters in (1, 3):
        say(f"mfma loop iters={iters}")
        L.bitlinear_measure_mfma_i8(to_dev(xq), to_dev(packed), iters, sink)
        torch.cuda.synchronize()
        blocks = int(L.bitlinear_measure_mfma_ops(iters) / (4 * iters * 8 * 65536))
        got = sink.cpu().numpy()[:blocks].astype(np.int64) & 0xFFFFFFFF
        want = mfma_checksum(xq, packed, iters) & 0xFFFFFFFF
        assert blocks >= 2 and np.all(got == want), (got[:4], want)
