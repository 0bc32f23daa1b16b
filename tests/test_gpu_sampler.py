"""The diffusion sampler on the GPU against the oracle: decisions bit for bit outside the
1e-4 bands, confidences, and z = softmax(l)·E within relative L2 1e-4."""
from dataclasses import replace

import numpy as np
import pytest

import e2m3
import p_records as PR
import workloads
from gpu_util import check_step, check_z, log, require_gpu, to_dev
from oracle import sampler as S

pytestmark = pytest.mark.gpu


class GpuSampler:
    def __init__(self, torch, dg, emb, ids, mask, ctrl):
        self.torch, self.dg = torch, dg
        e32 = to_dev(emb)
        self.emb = dg.dg_embedding_pack(e32)
        del e32
        n = len(ids)
        self.ids = to_dev(np.asarray(ids, np.int32))
        self.mask = to_dev(np.asarray(mask, np.uint8))
        self.z = torch.empty((n, emb.shape[1]), dtype=torch.float32, device="cuda")
        self.kappa = torch.empty(n, dtype=torch.float32, device="cuda")
        self.nu = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ctrl = dg.make_ctrl(seed=ctrl.seed, gstep=ctrl.gstep, s_in_block=ctrl.s_in_block,
                                 s_max=ctrl.s_max, flags=ctrl.flags, tau=ctrl.tau,
                                 t_start=ctrl.t_start, t_end=ctrl.t_end)

    def step(self, logits):
        tl = logits if hasattr(logits, "data_ptr") else to_dev(logits)
        self.dg.dg_sampler_step(tl, self.emb, self.ids, self.mask, self.z, self.kappa, self.nu, self.ctrl)
        self.torch.cuda.synchronize()
        return (self.ids.cpu().numpy(), self.mask.cpu().numpy(), self.kappa.cpu().numpy(),
                self.z.cpu().numpy(), int(self.nu.item()))

    def set_state(self, ids, mask):
        self.ids.copy_(self.torch.from_numpy(np.asarray(ids, np.int32)))
        self.mask.copy_(self.torch.from_numpy(np.asarray(mask, np.uint8)))


def run_steps(workload, n_steps, z_every=True):
    torch, dg = require_gpu()
    c = workloads.CONFIGS[workload]
    emb = workloads.embedding(workload)
    ids, mask = workloads.initial_canvas(workload)
    ctrl = S.Ctrl(seed=workload, tau=c["tau"], s_max=48, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    e64 = emb.astype(np.float64)
    exempt = 0
    for step in range(n_steps):
        log(f"sampler workload {workload} step {step}")
        logits = workloads.step_logits(workload, step)
        ref = S.sampler_step(logits, e64, ids, mask, ctrl, z_rows="all" if z_every else None)
        gids, gmask, gk, gz, gnu = g.step(logits)
        exempt += check_step(ids, mask, gids, gmask, gk, ref, c["tau"])
        if z_every:
            check_z(gz, ref["z"])
        assert gnu == ref["n_uncommitted"] or exempt
        ctrl = ref["ctrl"]
        assert dg.read_ctrl(g.ctrl)["gstep"] == ctrl.gstep
        ids, mask = ref["ids"], ref["committed"]
        if exempt:
            g.set_state(ids, mask)
    return exempt


def test_workload1_eight_steps():
    assert run_steps(1, 8) == 0


def test_workload2_eight_steps():
    assert run_steps(2, 8) == 0


def test_workload3_full_vocab():
    """262144 x 3072 at full size: every decision, and z on all 256 rows."""
    torch, dg = require_gpu()
    log("sampler workload 3: generating inputs")
    emb = workloads.embedding(3)
    logits = workloads.step_logits(3, 0)
    ids, mask = workloads.initial_canvas(3)
    ctrl = S.Ctrl(seed=3, tau=0.9, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    log("sampler workload 3: gpu step")
    gids, gmask, gk, gz, gnu = g.step(logits)
    log("sampler workload 3: oracle (z for all 256 rows)")
    ref = S.sampler_step(logits, emb, ids, mask, ctrl, z_rows="all")
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.9) == 0
    worst, total = check_z(gz, ref["z"])
    log(f"workload 3: z relative L2 worst row {worst:.3e}, whole tensor {total:.3e}")
    assert gnu == ref["n_uncommitted"]
    log(f"workload 3: {int(gmask.sum())} committed of 256")


@pytest.mark.parametrize("n,vocab,d", [(256, 4097, 260), (100, 1001, 64), (1, 2, 4), (256, 33, 3),
                                       (17, 12345, 513)])
def test_ragged_shapes(n, vocab, d):
    torch, dg = require_gpu()
    log(f"sampler ragged n={n} V={vocab} d={d}")
    rng = np.random.default_rng(n * 7 + vocab)
    logits = (rng.standard_normal((n, vocab)) * 3).astype(np.float32)
    logits[::3, 0] += 12.0
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    ids = rng.integers(0, vocab, n).astype(np.int32)
    mask = (rng.random(n) < 0.2).astype(np.uint8)
    ctrl = S.Ctrl(seed=11, gstep=4, tau=0.9, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    gids, gmask, gk, gz, gnu = g.step(logits)
    ref = S.sampler_step(logits, emb, ids, mask, ctrl)
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.9) == 0
    check_z(gz, ref["z"])


@pytest.mark.parametrize("n_kb", [2, 4, 5, 6, 7])
def test_short_splits(n_kb):
    """One vocabulary split of n_kb 16-id k-blocks (the last one ragged): the
    contraction's prologue, whole pairs and a lone last k-block at the counts
    where they meet."""
    torch, dg = require_gpu()
    n, vocab, d = 64, 16 * n_kb - 3, 40
    log(f"sampler short split n_kb={n_kb} V={vocab}")
    rng = np.random.default_rng(n_kb)
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::4, vocab - 1] += 9.0
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    emb[vocab - 1] += 1.0                      # the ragged block's row stands out in z
    ids = rng.integers(0, vocab, n).astype(np.int32)
    mask = (rng.random(n) < 0.2).astype(np.uint8)
    ctrl = S.Ctrl(seed=5, gstep=2, tau=0.9, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    gids, gmask, gk, gz, gnu = g.step(logits)
    ref = S.sampler_step(logits, emb, ids, mask, ctrl)
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.9) == 0
    check_z(gz, ref["z"])


@pytest.mark.parametrize("spread", [6, 30])
def test_rows_of_very_different_size(spread):
    """Table rows scaled by 2^u, u uniform in [-spread, 0], some rows zero, and
    one large row among small ones in every k-block: each row is held at its
    own scale (the row shifts), so z meets the bound where one block-wide
    scale would lose the small rows' corrections."""
    torch, dg = require_gpu()
    n, vocab, d = 96, 4099, 200
    log(f"sampler row sizes spread={spread}")
    rng = np.random.default_rng(spread)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    emb *= np.exp2(rng.uniform(-spread, 0, vocab))[:, None].astype(np.float32)
    emb[::16] *= np.float32(2.0 ** spread)
    emb[5::23] = 0.0
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::5, 17] += 8.0
    ids = rng.integers(0, vocab, n).astype(np.int32)
    mask = (rng.random(n) < 0.2).astype(np.uint8)
    ctrl = S.Ctrl(seed=3, gstep=1, tau=0.9, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    gids, gmask, gk, gz, gnu = g.step(logits)
    ref = S.sampler_step(logits, emb, ids, mask, ctrl)
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.9) == 0
    worst, total = check_z(gz, ref["z"])
    log(f"row sizes spread={spread}: z relative L2 worst row {worst:.3e}")


@pytest.mark.parametrize("scale", [300.0, 1e-5, 0.02, 1e-25])
def test_table_scales(scale):
    """The packed table's exponent shift at both ends: z of tables with entries
    of order 300, 1e-5 and 1e-25 meets the bound like the 0.02 table (the shift
    c is chosen from max|E| when the table is packed; below 2^-72 it is capped
    and the row shifts take over)."""
    torch, dg = require_gpu()
    n, vocab, d = 64, 20000, 96
    rng = np.random.default_rng(int(scale * 1e6) % 997 + (7 if scale < 1e-20 else 0))
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::4, 123] += 10.0
    emb = (rng.standard_normal((vocab, d)) * scale).astype(np.float32)
    ctrl = S.Ctrl(seed=5, tau=0.9, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, np.zeros(n), np.zeros(n), ctrl)
    gids, gmask, gk, gz, _ = g.step(logits)
    ref = S.sampler_step(logits, emb, np.zeros(n), np.zeros(n), ctrl, z_rows="all")
    assert check_step(np.zeros(n), np.zeros(n), gids, gmask, gk, ref, 0.9) == 0
    worst, total = check_z(gz, ref["z"])
    log(f"table scale {scale}: z relative L2 worst row {worst:.3e}, whole tensor {total:.3e}")


def test_vocab_past_65536_blocks():
    """A vocabulary of more than 65536 16-id blocks (1048600 ids): the packing
    grid takes the blocks on its x dimension, and the step meets the oracle."""
    torch, dg = require_gpu()
    n, vocab, d = 4, 1048600, 8
    rng = np.random.default_rng(65537)
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[1, vocab - 1] += 20.0               # the winner in the last block
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    emb[vocab - 16:] += 1.0                    # the last block's rows stand out in z
    ctrl = S.Ctrl(seed=9, tau=0.5, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, np.zeros(n), np.zeros(n), ctrl)
    gids, gmask, gk, gz, _ = g.step(logits)
    ref = S.sampler_step(logits, emb, np.zeros(n), np.zeros(n), ctrl, z_rows="all")
    assert check_step(np.zeros(n), np.zeros(n), gids, gmask, gk, ref, 0.5) == 0
    assert gids[1] == vocab - 1 and gmask[1] == 1
    check_z(gz, ref["z"])


def test_identity_embedding_and_probability_sum():
    """E = I gives z = p; an all-ones column of E gives sum(p) = 1 (through the ABI)."""
    torch, dg = require_gpu()
    from scipy import special
    rng = np.random.default_rng(2)
    vocab = 64
    logits = (rng.standard_normal((32, vocab)) * 4).astype(np.float32)
    emb = np.eye(vocab, dtype=np.float32)
    g = GpuSampler(torch, dg, emb, np.zeros(32), np.zeros(32), S.Ctrl(tau=2.0))
    _, _, _, z, _ = g.step(logits)
    p = special.softmax(logits.astype(np.float64), axis=1)
    check_z(z, p)
    emb2 = (rng.standard_normal((vocab, 8)) * 0.02).astype(np.float32)
    emb2[:, 5] = 1.0
    g = GpuSampler(torch, dg, emb2, np.zeros(32), np.zeros(32), S.Ctrl(tau=2.0))
    _, _, _, z, _ = g.step(logits)
    np.testing.assert_allclose(z[:, 5], 1.0, atol=2e-5)


def test_ties_nan_and_inf_rows():
    torch, dg = require_gpu()
    vocab, n = 5000, 8
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((n, vocab)).astype(np.float32)
    logits[0, [40, 4000]] = 50.0            # tie: smallest id wins
    logits[1, 7] = np.nan
    logits[2, :] = -np.inf
    logits[3, 99] = np.inf
    logits[4, :] = 0.0                       # uniform: never commits
    logits[5, 4999] = 60.0                   # spike at the last id
    emb = (rng.standard_normal((vocab, 16)) * 0.02).astype(np.float32)
    ctrl = S.Ctrl(seed=1, tau=0.4, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, np.zeros(n), np.zeros(n), ctrl)
    gids, gmask, gk, gz, gnu = g.step(logits)
    ref = S.sampler_step(logits, emb, np.zeros(n), np.zeros(n), ctrl)
    assert check_step(np.zeros(n), np.zeros(n), gids, gmask, gk, ref, 0.4) == 0
    assert gids[0] == 40 and gmask[0] == 1
    assert gids[5] == 4999 and gmask[5] == 1
    assert np.all(np.isnan(gk[1:4])) and np.all(np.isnan(gz[1:4]))
    assert gmask[4] == 0
    ok = [0, 4, 5, 6, 7]
    check_z(gz[ok], ref["z"][ok])


def test_commit_only_and_last_step():
    torch, dg = require_gpu()
    rng = np.random.default_rng(5)
    n, vocab = 64, 3000
    logits = rng.standard_normal((n, vocab)).astype(np.float32)
    logits[:10, 3] += 40
    ids = rng.integers(0, vocab, n).astype(np.int32)
    mask = np.zeros(n, np.uint8); mask[5:15] = 1
    emb = (rng.standard_normal((vocab, 8)) * 0.02).astype(np.float32)
    ctrl = S.Ctrl(seed=2, gstep=3, tau=0.9, flags=S.COMMIT_ONLY | S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    gids, gmask, gk, gz, _ = g.step(logits)
    ref = S.sampler_step(logits, emb, ids, mask, ctrl)
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.9, commit_only=True) == 0
    assert set(np.nonzero(gids != ids)[0]) == set(range(5))
    # the last step of the budget commits every open defined row
    ctrl2 = S.Ctrl(seed=2, gstep=9, s_in_block=47, s_max=48, tau=0.99, flags=S.AUTO_ADVANCE)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl2)
    gids, gmask, gk, gz, gnu = g.step(logits)
    ref = S.sampler_step(logits, emb, ids, mask, ctrl2)
    assert gnu == 0 and gmask.sum() == n
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.99) == 0


@pytest.mark.parametrize("sched", [False, True])
def test_gumbel_and_temperature(sched):
    torch, dg = require_gpu()
    rng = np.random.default_rng(6)
    n, vocab = 256, 8192
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::2, 100] += 16.0
    emb = (rng.standard_normal((vocab, 64)) * 0.02).astype(np.float32)
    flags = S.GUMBEL | S.AUTO_ADVANCE | (S.T_SCHEDULE if sched else 0)
    ctrl = S.Ctrl(seed=99, gstep=12, s_in_block=20, s_max=48, tau=0.5, flags=flags,
                  t_start=0.8 if sched else 0.7, t_end=0.4)
    ids = rng.integers(0, vocab, n).astype(np.int32)
    mask = np.zeros(n, np.uint8)
    g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
    gids, gmask, gk, gz, _ = g.step(logits)
    ref = S.sampler_step(logits, emb, ids, mask, ctrl)
    assert check_step(ids, mask, gids, gmask, gk, ref, 0.5) == 0
    check_z(gz, ref["z"])
    assert 10 < gmask.sum() < n


def test_deterministic_and_resume():
    """Same inputs give bit-identical outputs; a step replayed from saved state matches."""
    torch, dg = require_gpu()
    emb = workloads.embedding(2)
    ids, mask = workloads.initial_canvas(2)
    ctrl = S.Ctrl(seed=2, tau=0.9, flags=S.AUTO_ADVANCE)
    outs = []
    for _ in range(2):
        g = GpuSampler(torch, dg, emb, ids, mask, ctrl)
        r0 = g.step(workloads.step_logits(2, 0))
        saved = (r0[0].copy(), r0[1].copy(), dg.read_ctrl(g.ctrl))
        r1 = g.step(workloads.step_logits(2, 1))
        outs.append((r0, r1))
    for a, b in zip(outs[0], outs[1]):
        for x, y in zip(a[:4], b[:4]):
            np.testing.assert_array_equal(x, y)
    # resume: a fresh sampler started from the state saved after step 0
    c = saved[2]
    g = GpuSampler(torch, dg, emb, saved[0], saved[1],
                   S.Ctrl(seed=c["seed"], gstep=c["gstep"], s_in_block=c["s_in_block"], s_max=c["s_max"],
                          flags=c["flags"], tau=c["tau"], t_start=c["t_start"], t_end=c["t_end"]))
    r1b = g.step(workloads.step_logits(2, 1))
    for x, y in zip(outs[0][1][:4], r1b[:4]):
        np.testing.assert_array_equal(x, y)


def _row_shifts(emb, c):
    """d_k = min(max(8 - c - e_k, 0), 40) with max|E_k| in [2^(e_k - 1), 2^e_k); 40 for zero rows."""
    m = np.abs(emb).max(axis=1).astype(np.float64)
    e = np.frexp(m)[1]
    return np.where(m > 0, np.clip(8 - c - e, 0, 40), 40).astype(np.int64)


@pytest.mark.parametrize("vocab,d,scale,spread", [(37, 260, 0.02, 0), (4096, 512, 0.02, 0), (16, 1, 0.02, 0),
                                                  (300, 64, 700.0, 0), (64, 8, 3e-6, 0), (48, 300, 0.5, 0),
                                                  (1000, 96, 0.02, 12), (77, 130, 1e-3, 50)])
def test_embedding_pack_layout(vocab, d, scale, spread):
    """The packed table: c such that max|E| 2^c lies in [2^7, 2^8), and for
    each id a shift d_k so that row k's Q = E_k 2^(c + d_k) reaches that range
    too (at most 40); for each pair of 16-id k-blocks and 256-column tile a
    24 KB block holding the fp16 Q16 of k-block 2j (256 columns x 16 ids),
    those of k-block 2j + 1, then per column 16 bytes for k-block 2j and 16 for
    2j + 1: the e2m3 codes of (Q - Q16) 2^11 (12 bytes, code i at bit 6i) under
    the scale 2^eB of the k-block and 64-column group, the byte 127 + eB and
    three zeros; after the blocks, the shift bytes (one per id of the whole
    k-block pairs, 256-byte aligned), 1024 floats of pack workspace and the
    record (2^-(14+c), c).  Every byte is compared with numpy's fp16 rounding
    and the e2m3 model.  spread > 0 scales the rows by 2^u, u uniform in
    [-spread, 0] (rows far apart in size, some zero)."""
    torch, dg = require_gpu()
    rng = np.random.default_rng(vocab + d)
    emb = (rng.standard_normal((vocab, d)) * scale).astype(np.float32)
    if spread:
        emb *= np.exp2(np.round(rng.uniform(-spread, 0, vocab)))[:, None].astype(np.float32)
        emb[::7] = 0.0
    packed = dg.dg_embedding_pack(to_dev(emb)).cpu().numpy()
    n_pairs, n_tiles = -(-vocab // 32), -(-d // 256)
    image = n_pairs * n_tiles * 24576
    n_sh = -(-n_pairs * 32 // 256) * 256
    assert packed.size == image + n_sh + 4096 + 256 == dg.dg_embedding_packed_bytes(vocab, d)
    tail = image + n_sh + 4096
    zscale = packed[tail:tail + 4].view(np.float32)[0]
    c = int(packed[tail + 4:tail + 8].view(np.int32)[0])
    top = float(np.abs(emb).max()) * 2.0 ** c
    assert 128.0 <= top < 256.0, (c, top)
    assert zscale == np.float32(2.0 ** -(14 + c))
    full = np.zeros((n_pairs * 32, n_tiles * 256), np.float32)
    full[:vocab, :d] = emb
    shifts = np.full(n_sh, 40, np.int64)
    shifts[:vocab] = _row_shifts(emb, c)
    np.testing.assert_array_equal(packed[image:image + n_sh], shifts)
    q = full * np.exp2(c + shifts[:n_pairs * 32])[:, None].astype(np.float32)    # [id, column], exact
    q16 = q.astype(np.float16)
    qe = ((q - q16.astype(np.float32)) * np.float32(2048.0)).astype(np.float64)
    nb, ng = n_pairs * 2, n_tiles * 4
    m = np.maximum(np.abs(qe), np.abs(q16.astype(np.float64))).reshape(nb, 16, ng, 64).max(axis=(1, 3))
    eb = e2m3.scale_exp(m, -126)                                      # [kb, group]
    codes = e2m3.encode(qe.reshape(nb, 16, ng, 64) / np.exp2(eb)[:, None, :, None])
    chunk = np.zeros((nb, ng, 64, 16), np.uint8)                      # [kb, group, column, byte]
    chunk[..., :12] = e2m3.pack16(codes.transpose(0, 2, 3, 1))
    chunk[..., 12] = np.broadcast_to((127 + eb)[:, :, None], (nb, ng, 64))
    # reference blocks [pair, tile, 24576]
    q16_kb = q16.reshape(n_pairs, 2, 16, n_tiles, 256).transpose(0, 3, 1, 4, 2)     # [pair, tile, kb&1, col, id]
    res_kb = chunk.reshape(n_pairs, 2, n_tiles, 256, 16).transpose(0, 2, 3, 1, 4)   # [pair, tile, col, kb&1, byte]
    blocks = packed[:image].reshape(n_pairs, n_tiles, 24576)
    np.testing.assert_array_equal(blocks[:, :, :16384].copy().view(np.float16).reshape(q16_kb.shape), q16_kb)
    np.testing.assert_array_equal(blocks[:, :, 16384:].reshape(res_kb.shape), res_kb)


def _sampler_plan(n, vocab, d):
    """The sampler's split plan (k-blocks of 16 ids; splits of an even number of
    k-blocks, at least 16 and at most 1024 each, about 256 workgroups for the
    contraction) and the byte offset of the p images in its workspace, after
    the per-(row, split) statistics records of 32 bytes."""
    n_mt, n_kb, n_tiles = -(-n // 256), -(-vocab // 16), -(-d // 256)
    splits = max(256 // (n_tiles * n_mt), 1)
    splits = min(splits, -(-n_kb // 16))
    splits = max(splits, -(-n_kb // 1024), 1)
    kbps = -(-n_kb // splits)
    kbps += kbps & 1
    n_splits = -(-n_kb // kbps)
    return n_kb, kbps, n_splits, -(-(n * n_splits * 32) // 256) * 256


@pytest.mark.parametrize("n,vocab,d", [(64, 4099, 200), (256, 20000, 64)])
def test_p_image_records(n, vocab, d):
    """The statistics pass's p records, read back from the workspace, against
    their definition (tests/p_records.py): for row i and k-block k (split s),
    P' = p 2^(14 - d_id) with p = exp2((l - m_s) log2 e) and d_id the table's
    row shifts.  P'16 matches fp16 of the reference to one fp16 ulp (the
    device's exp2 is not correctly rounded); the codes of P'16 match the e2m3
    model exactly; es is the rule applied to the record's own values; the codes
    of r are within half a code step of the reference residual
    (tests/test_p_records_check.py shows the check rejecting planted mistakes)."""
    torch, dg = require_gpu()
    log(f"p records n={n} V={vocab} d={d}")
    rng = np.random.default_rng(n + vocab)
    emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
    emb *= np.exp2(np.round(rng.uniform(-12, 0, vocab)))[:, None].astype(np.float32)
    emb[3::29] = 0.0
    logits = (rng.standard_normal((n, vocab)) * 2).astype(np.float32)
    logits[::3, 11] += 9.0
    packed = dg.dg_embedding_pack(to_dev(emb))
    ws = torch.empty(dg.dg_sampler_workspace_bytes(n, vocab, d), dtype=torch.uint8, device="cuda")
    ids = to_dev(rng.integers(0, vocab, n).astype(np.int32))
    mask = to_dev(np.zeros(n, np.uint8))
    z = torch.empty((n, d), dtype=torch.float32, device="cuda")
    kappa = torch.empty(n, dtype=torch.float32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    ctrl = dg.make_ctrl(seed=1, tau=0.9, flags=0)
    dg.dg_sampler_step(to_dev(logits), packed, ids, mask, z, kappa, nu, ctrl, workspace=ws)
    torch.cuda.synchronize()
    pk, wsb = packed.cpu().numpy(), ws.cpu().numpy()
    n_kb, kbps, n_splits, off = _sampler_plan(n, vocab, d)
    image = -(-vocab // 32) * -(-d // 256) * 24576
    shifts = pk[image:image + n_kb * 16].astype(np.int64)
    rec = wsb[off:off + n_kb * 256 * 64].reshape(n_kb, 256, 64)[:, :n]        # [kb, row, byte]; one row tile
    # reference P' per (row, id): fp64 exp2, rounded to float32
    lf = np.full((n, n_kb * 16), -np.inf, np.float32)
    lf[:, :vocab] = logits
    m_s = np.repeat(np.stack([lf[:, s * kbps * 16:(s + 1) * kbps * 16].max(axis=1) for s in range(n_splits)], 1),
                    kbps * 16, axis=1)[:, :n_kb * 16]                                   # split maxima per id
    log2e = np.float32(1.4426950408889634)
    p = np.exp2(lf.astype(np.float64) * float(log2e) - m_s.astype(np.float64) * float(log2e))
    pref = np.ldexp(p, (14 - shifts)[None, :]).astype(np.float32).reshape(n, n_kb, 16).transpose(1, 0, 2)
    PR.check_records(rec, pref)


@pytest.mark.parametrize("n,vocab,d", [(256, 262144, 3072), (256, 4097, 260), (17, 12345, 516), (1, 2, 4)])
def test_float32_table_matches_the_packed_image(n, vocab, d):
    """dg_sampler_step_f32 (bf16x3 on the float32 table) and dg_sampler_step
    (fp16 + fp8 on the packed table) take every decision from the same
    statistics: ids, mask, confidences, counts and the control block agree bit
    for bit; both z meet the oracle, and each other within the same bound."""
    torch, dg = require_gpu()
    log(f"sampler float32 table n={n} V={vocab} d={d}")
    if vocab == 262144:
        emb = workloads.embedding(3)
        logits = workloads.step_logits(3, 0)
        rows = np.array([0, 5, 77, 128, 255])
    else:
        rng = np.random.default_rng(vocab + d)
        logits = (rng.standard_normal((n, vocab)) * 3).astype(np.float32)
        logits[::3, vocab // 2] += 12.0
        emb = (rng.standard_normal((vocab, d)) * 0.02).astype(np.float32)
        rows = None
    ids = (np.arange(n) * 7919 % vocab).astype(np.int32)
    mask = (np.arange(n) % 5 == 0).astype(np.uint8)
    ctrl = S.Ctrl(seed=21, gstep=3, tau=0.9, flags=S.AUTO_ADVANCE)
    tl, te = to_dev(logits), to_dev(emb)
    outs = []
    for f32 in (False, True):
        t_ids, t_mask = to_dev(ids), to_dev(mask)
        z = torch.empty((n, d), dtype=torch.float32, device="cuda")
        kappa = torch.empty(n, dtype=torch.float32, device="cuda")
        nu = torch.zeros(1, dtype=torch.int32, device="cuda")
        c = dg.make_ctrl(seed=ctrl.seed, gstep=ctrl.gstep, tau=ctrl.tau, flags=ctrl.flags)
        if f32:
            dg.dg_sampler_step_f32(tl, te, t_ids, t_mask, z, kappa, nu, c)
        else:
            dg.dg_sampler_step(tl, dg.dg_embedding_pack(te), t_ids, t_mask, z, kappa, nu, c)
        torch.cuda.synchronize()
        outs.append([x.cpu().numpy() for x in (t_ids, t_mask, z, kappa, nu, c)])
    for a, b, name in zip(outs[0], outs[1], ("ids", "mask", "z", "kappa", "n_uncommitted", "ctrl")):
        if name != "z":
            np.testing.assert_array_equal(a, b, err_msg=f"float32 table differs from the packed image: {name}")
    check_z(outs[1][2], outs[0][2])
    ref = S.sampler_step(logits, emb, ids, mask, ctrl, z_rows="all" if rows is None else rows)
    for out in outs:
        gids, gmask, gz, gk = out[0], out[1], out[2], out[3]
        assert check_step(ids, mask, gids, gmask, gk, ref, 0.9) == 0
        check_z(gz if rows is None else gz[rows], ref["z"])
