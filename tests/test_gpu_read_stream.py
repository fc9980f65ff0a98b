"""da_read_stream (the HBM read-bandwidth measurement aid): every 16-byte
unit is read exactly once, chunk g covering units [g*per, (g+1)*per) with
per = floor(n16 / n_groups) and the last chunk taking the rest -- checked by
the XOR of each chunk's 32-bit words, computed here with NumPy."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def expected(words: np.ndarray, n_groups: int) -> np.ndarray:
    n16 = words.size // 4
    per = n16 // n_groups
    out = np.zeros(n_groups, dtype=np.uint32)
    for g in range(n_groups):
        lo = 4 * g * per
        hi = words.size if g == n_groups - 1 else 4 * (g + 1) * per
        out[g] = np.bitwise_xor.reduce(words[lo:hi]) if hi > lo else 0
    return out


@pytest.mark.parametrize("n16,n_groups", [
    (65539, 7),        # ragged: the last chunk takes the remainder
    (65536, 1),        # one workgroup streams everything
    (100, 100),        # one unit per workgroup
    (1000, 3),         # chunks shorter than one unrolled trip (4 x 64 units)
    (1 << 20, 4096),   # the benchmark's grouping
])
def test_read_stream_xor_per_chunk(da, n16, n_groups):
    import torch
    rng = np.random.default_rng([7, n16, n_groups])
    words = rng.integers(0, 2 ** 32, size=4 * n16, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = da.da_read_stream(buf, n_groups=n_groups)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected(words, n_groups))
