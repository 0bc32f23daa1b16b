"""Pins for the oracle's Philox4x32-10 and the draws derived from it (CPU only)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers / hipcc not available")
    exe = str(tmp_path_factory.mktemp("rr") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-I/opt/rocm/include", os.path.join(HERE, "rocrand_philox_ref.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(1234)
    n = 4096
    c = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    c[:, 1] &= np.uint64(2**30 - 1)          # the rocRAND offset argument is 64-bit
    k = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    c[:8] = 0                                # include the all-zero counter, several keys
    k[:4] = 0
    lines = "\n".join(" ".join(f"{int(v):x}" for v in (*c[i], *k[i])) for i in range(n))
    out = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(x, 16) for x in ln.split()] for ln in out.strip().splitlines()], dtype=np.uint64)
    got = np.stack(philox.philox4x32_10(c[:, 0], c[:, 1], c[:, 2], c[:, 3], k[:, 0], k[:, 1]), axis=1)
    assert ref.shape == (n, 4)
    np.testing.assert_array_equal(got.astype(np.uint64), ref)


def test_uniform_is_exact_and_open():
    h = np.array([0, 1, 511, 512, 2**32 - 1, 2**31], dtype=np.uint32)
    u = philox.uniform_f32(h)
    assert u.dtype == np.float32
    assert np.all(u > 0) and np.all(u < 1)
    scaled = u.astype(np.float64) * 2.0 ** 24
    assert np.all(scaled == np.round(scaled)) and np.all(scaled.astype(np.int64) % 2 == 1)
    assert u[0] == np.float32(2.0 ** -24) and u[4] == np.float32(1 - 2.0 ** -24)


def test_range_id_uniform_chi2():
    vocab = 1000
    ids = philox.renoise_ids(seed=77, gstep=3, positions=np.arange(400_000), vocab=vocab)
    assert ids.min() >= 0 and ids.max() < vocab
    counts = np.bincount(ids, minlength=vocab)
    chi2, p = stats.chisquare(counts)
    assert p > 1e-4


def test_range_id_bounds_exact():
    h = np.array([0, 2**32 - 1], dtype=np.uint32)
    for vocab in (1, 2, 3, 262144, 2**31 + 7):
        ids = philox.range_id(h, vocab)
        assert ids[0] == 0 and ids[1] == vocab - 1


def test_gumbel_distribution():
    g = philox.gumbel_row(seed=9, gstep=0, position=0, vocab=400_000).astype(np.float64)
    # closed forms: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    assert abs(g.mean() - np.euler_gamma) < 0.01
    assert abs(g.var() - np.pi ** 2 / 6) < 0.03
    ks = stats.kstest(g, stats.gumbel_r.cdf)
    assert ks.pvalue > 1e-4


def test_gumbel_max_frequencies_match_softmax():
    # argmax(l + g) over fresh noise is a draw from softmax(l)
    logits = np.array([0.0, 1.0, -0.5, 2.0])
    p = np.exp(logits - logits.max()); p /= p.sum()
    draws = []
    for pos in range(20000):
        g = philox.gumbel_row(seed=5, gstep=1, position=pos, vocab=4).astype(np.float64)
        draws.append(int(np.argmax(logits + g)))
    counts = np.bincount(draws, minlength=4)
    chi2, pval = stats.chisquare(counts, p * len(draws))
    assert pval > 1e-4


def test_streams_and_steps_differ():
    a = philox.renoise_ids(1, 0, np.arange(256), 2**31)
    b = philox.init_ids(1, 0, np.arange(256), 2**31)
    c = philox.renoise_ids(1, 1, np.arange(256), 2**31)
    d = philox.renoise_ids(2, 0, np.arange(256), 2**31)
    for x, y in ((a, b), (a, c), (a, d)):
        assert np.mean(x == y) < 0.01


def test_gumbel_word_addressing():
    # id j uses word j & 3 of counter j >> 2: ids 4m..4m+3 share one Philox call
    k0, k1 = philox.seed_key(11)
    words = philox.philox4x32_10(5, 7, 2, philox.STREAM_GUMBEL, k0, k1)
    g = philox.gumbel_row(11, 2, 7, 24)
    np.testing.assert_array_equal(g[20:24], philox.gumbel_f32(np.array([int(w) for w in words], dtype=np.uint32)))


# ---- the C helper (oracle/philox_c.c) must draw exactly what the numpy oracle draws ----

def _native_or_skip():
    from oracle import native
    if native.lib() is None:
        pytest.skip("no C compiler for the oracle's C helper")
    return native


def test_native_philox_bit_exact():
    native = _native_or_skip()
    rng = np.random.default_rng(11)
    ctr = rng.integers(0, 2 ** 32, size=(4096, 4), dtype=np.uint64).astype(np.uint32)
    ctr[:4] = [[0, 0, 0, 0], [2 ** 32 - 1] * 4, [1, 2, 3, 4], [0, 7, 0, 6]]
    k0, k1 = 0xDEADBEEF, 0x01234567
    got = native.philox(ctr, k0, k1)
    ref = np.stack(philox.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], k0, k1), axis=1)
    assert np.array_equal(got, ref)


def test_native_gumbel_scores_match_numpy():
    """Same Philox words; float32 logs may differ by an ulp between libm and numpy."""
    native = _native_or_skip()
    vocab = 262144
    rng = np.random.default_rng(12)
    logits = (rng.standard_normal((3, vocab)) * 3).astype(np.float32)
    rows = np.array([0, 5, 255])
    seed, gstep, inv_t = (1 << 40) + 77, 9, np.float32(1.25)
    got = native.gumbel_scores(logits, inv_t, seed, gstep, rows)
    for r, pos in enumerate(rows):
        g = philox.gumbel_row(seed, gstep, int(pos), vocab)
        ref = (logits[r] * inv_t).astype(np.float32) + g
        # g = -log(t): an ulp of t (relative 2^-23) moves g by up to 2^-23 in
        # absolute terms, plus an ulp of g and one from rounding the sum
        tol = 2 * np.spacing(np.abs(g)) + 2.0 ** -22 + np.spacing(np.abs(ref))
        assert np.all(np.abs(got[r] - ref) <= tol)
        assert int(np.argmax(got[r])) == int(np.argmax(ref))


def test_native_synth_noise_bit_exact():
    native = _native_or_skip()
    from oracle import synth
    import workloads
    table = workloads.synth_table()
    vocab, rows = 5003, np.array([0, 3, 200])
    got = native.synth_noise(table, len(rows), vocab, 5, 17, rows)
    jj = np.arange(vocab, dtype=np.uint64)
    for r, pos in enumerate(rows):
        h = philox.word(5, philox.STREAM_SYN_NOISE, 17, int(pos), c0=jj >> np.uint64(2),
                        w=(jj & np.uint64(3)).astype(np.int64))
        assert np.array_equal(got[r], table[(h >> np.uint32(16)).astype(np.int64)])
