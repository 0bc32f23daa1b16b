"""The measurement probes through the C ABI: the copy moves every byte, and the
read probe launches the grid it states (one sink word per wave, the xor of what
that wave read)."""
import numpy as np
import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 4 * 255, 4 * 256 * 5 + 4, 4 * 256 * 4096 * 2 + 12])
def test_copy_probe_moves_every_byte(n_words):
    torch, dg = require_gpu()
    src = torch.arange(n_words, dtype=torch.int32, device="cuda")
    dst = torch.full_like(src, -1)
    dg.dg_probe_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


@pytest.mark.parametrize("n_words", [4, 4 * 300, 4 * 256 * 4096 + 8, 4 * 256 * 4096 * 3])
def test_read_probe_grid_and_sink(n_words):
    torch, dg = require_gpu()
    n16 = n_words // 4
    blocks = min(4096, -(-n16 // 256))
    sink = torch.full((dg.PROBE_READ_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    zeros = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    dg.dg_probe_read(zeros, sink)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert np.all(s[:4 * blocks] == 0) and np.all(s[4 * blocks:] == -1)
    # one nonzero word: only the wave that read it reports it
    ones = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    k = n_words - 1
    ones[k] = 0x1234567
    dg.dg_probe_read(ones, sink)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    thread = (k // 4) % (blocks * 256)
    owner = thread // 64
    assert s[owner] == 0x1234567
    assert np.count_nonzero(s[:4 * blocks]) == 1
