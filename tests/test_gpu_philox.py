"""Device Philox4x32-10 and the canvas initialisation against the oracle: bit for bit."""
import numpy as np
import pytest

from gpu_util import log, require_gpu
from oracle import philox

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,c1,c2,c3", [(0, 0, 0, 0), (5, 17, 3, 0), (2**64 - 1, 2**32 - 1, 12345, 6),
                                           (0x0123456789ABCDEF, 255, 47, 1)])
def test_philox_bit_exact(seed, c1, c2, c3):
    torch, dg = require_gpu()
    n_ctr = 1 << 18                      # 2^20 output words
    log(f"philox seed={seed} c=({c1},{c2},{c3})")
    out = torch.empty(4 * n_ctr, dtype=torch.int32, device="cuda")
    dg.dg_philox_fill(out, seed, c1, c2, c3)
    got = out.cpu().numpy().view(np.uint32).reshape(n_ctr, 4)
    k0, k1 = philox.seed_key(seed)
    ref = np.stack(philox.philox4x32_10(np.arange(n_ctr, dtype=np.uint64), c1, c2, c3, k0, k1), axis=1)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("n,vocab,gstep", [(256, 262144, 0), (256, 4096, 77), (1, 2, 3), (100, 1001, 9)])
def test_canvas_init_matches_oracle(n, vocab, gstep):
    torch, dg = require_gpu()
    from oracle import sampler as S
    ctrl = dg.make_ctrl(seed=123, gstep=gstep, s_in_block=7)
    ids = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    mask = torch.ones(n, dtype=torch.uint8, device="cuda")
    dg.dg_canvas_init(ids, mask, ctrl, vocab)
    ref_ids, ref_mask, ref_ctrl = S.init_canvas(S.Ctrl(seed=123, gstep=gstep, s_in_block=7), n, vocab)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    assert mask.sum().item() == 0
    c = dg.read_ctrl(ctrl)
    assert c["s_in_block"] == 0 and c["gstep"] == gstep
