"""The two measurement references the bench divides by (needs an MI355X).

* pkv_stream_read_probe must read every 16-byte piece of the buffer exactly once.  Its fold picks
  two of the four words of each piece, which two depending on where the piece falls in a
  thread's four-load group; the test recomputes the same fold on the host from the documented
  traversal (grid of 2 x CU count workgroups of 256 threads, grid-stride loop unrolled by four,
  remainder loop on words x and w) and compares it with the device's, on a buffer whose length
  leaves a partial group at the end.  A piece skipped or read twice changes the fold.
* pkv_mfma_peak_probe must run its full and remainder loops, report the documented flop count and
  never write its sink.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_170_amd as m
    return m


def _host_fold(words: np.ndarray, stride: int) -> int:
    """XOR fold of the stream-read probe over uint32 `words` (4 per 16-byte piece)."""
    pieces = words.reshape(-1, 4)
    n16 = pieces.shape[0]
    i = np.arange(n16, dtype=np.int64)
    t = i % stride
    q = i // stride
    m = q // 4
    # Piece i is in a full group of four iff the group's last piece, t + (4m + 3) * stride, exists.
    full = t + (4 * m + 3) * stride < n16
    odd = (q % 4) % 2 == 1
    use_yz = full & odd
    picked = np.where(use_yz[:, None], pieces[:, [1, 2]], pieces[:, [0, 3]])
    return int(np.bitwise_xor.reduce(picked.ravel()))


@pytest.mark.parametrize("extra", [0, 1, 777])
def test_stream_read_probe_reads_every_piece_once(pkv, extra):
    dev = torch.device("cuda:0")
    stride = 2 * int(pkv._lib.pkv_device_cu_count()) * 256
    n16 = 5 * 4 * stride + extra  # five full rounds of four-load groups, then a partial group
    rng = np.random.default_rng(3 + extra)
    words = rng.integers(0, 2 ** 32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    _say(f"stream_read_probe: {n16} pieces, stride {stride}")
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    pkv.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32)[0])
    assert got == _host_fold(words, stride)


@pytest.mark.parametrize("iters", [16, 37, 3])
def test_mfma_peak_probe_runs_and_counts(pkv, iters):
    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    _say(f"mfma_peak_probe: iters {iters}")
    flop = pkv.mfma_peak_probe(iters, sink)
    torch.cuda.synchronize()
    assert flop == int(pkv._lib.pkv_device_cu_count()) * 8 * iters * 4 * 32768
    assert float(sink.item()) == 0.0
    with pytest.raises(Exception):
        pkv.mfma_peak_probe(0, sink)
