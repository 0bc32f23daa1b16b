"""Philox4x32-10 and the draws derived from it (oracle side; test infrastructure only).

The pages fix no generator: the decode loop only needs the canvas to start
"uniformly random" and non-accepted tokens to be "renoised uniformly at random"
(explainer "DiffusionGemma: Google's open diffusion LLM", section "A diffusion
language model refines 256 tokens in 12 steps", quoting report sections 3.1-3.3),
plus seeded Gumbel noise for sampled candidates.  The reading taken here is a
counter-based generator keyed by the seed and addressed by (id, position, step,
stream), so that any draw can be recomputed anywhere without carried state.

Philox4x32-10 is written from its published definition (J. K. Salmon, M. A.
Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11, section 3.2): a 4x32-bit counter block, a 2x32-bit key, ten rounds; each
round multiplies counter words 0 and 2 by two fixed 32-bit multipliers, keeps
the high and low halves of the 64-bit products, and rebuilds the block as
(hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key grows by two Weyl constants
between rounds.

Derived draws (shared definition with the GPU side, implemented independently):
  counter = (c0, position, gstep, stream), key = (seed mod 2^32, seed >> 32)
  GUMBEL   stream 0: c0 = id >> 2, output word id & 3
  RENOISE  stream 1: c0 = 0, word 0
  INIT     stream 2: c0 = 0, word 0
  SYN_*    streams 4, 5, 6: see oracle.synth
  u  = (2 * (h >> 9) + 1) * 2^-24      (exact in float32, strictly inside (0, 1))
  g  = -log(-log(u))                   (float32 arithmetic, the GPU's precision)
  id = (h * V) >> 32                   (Lemire's multiply-shift range reduction)

Pins: tests/test_oracle_philox.py compares philox4x32_10 with rocRAND's
host-callable Philox4x32-10 engine (an independent implementation) and checks
the uniform, Gumbel and range draws against their closed-form distributions.
"""
import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
MUL0 = np.uint64(0xD2511F53)
MUL1 = np.uint64(0xCD9E8D57)
WEYL0 = np.uint64(0x9E3779B9)
WEYL1 = np.uint64(0xBB67AE85)

STREAM_GUMBEL = 0
STREAM_RENOISE = 1
STREAM_INIT = 2
STREAM_SYN_CHOOSE = 4
STREAM_SYN_TARGET = 5
STREAM_SYN_NOISE = 6


def _u64(x):
    return np.asarray(x, dtype=np.uint64) & MASK32


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four 32-bit output words (uint32 arrays) for counter (c0..c3), key (k0, k1).

    Arguments broadcast against each other.  Products of two 32-bit values are
    formed exactly in uint64.
    """
    c0, c1, c2, c3 = _u64(c0), _u64(c1), _u64(c2), _u64(c3)
    k0, k1 = _u64(k0), _u64(k1)
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    k0 = k0.copy()
    k1 = k1.copy()
    for rnd in range(10):
        p0 = MUL0 * c0
        p1 = MUL1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
        if rnd < 9:
            k0 = (k0 + WEYL0) & MASK32
            k1 = (k1 + WEYL1) & MASK32
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def seed_key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def word(seed, stream, gstep, position, c0=0, w=0):
    """One 32-bit draw: output word ``w`` of counter (c0, position, gstep, stream)."""
    k0, k1 = seed_key(seed)
    out = philox4x32_10(c0, position, gstep, stream, k0, k1)
    w = np.asarray(w)
    stacked = np.stack(np.broadcast_arrays(*out), axis=0)
    if w.ndim == 0:
        return stacked[int(w)]
    idx = np.broadcast_to(w, stacked.shape[1:])
    return np.take_along_axis(stacked, idx[None].astype(np.int64), axis=0)[0]


def uniform_f32(h):
    """u = (2*(h>>9)+1) * 2^-24 as float32; exact, in (0, 1)."""
    h = np.asarray(h, dtype=np.uint32)
    odd = (h >> np.uint32(9)).astype(np.uint64) * np.uint64(2) + np.uint64(1)
    return (odd.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_f32(h):
    """g = -log(-log(u)) evaluated in float32, u from uniform_f32."""
    u = uniform_f32(h)
    t = -np.log(u)            # float32 in, float32 out
    return (-np.log(t)).astype(np.float32)


def range_id(h, vocab):
    """Lemire multiply-shift: floor(h * V / 2^32), an id in [0, V)."""
    h = np.asarray(h, dtype=np.uint64)
    return ((h * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


def gumbel_row(seed, gstep, position, vocab):
    """Gumbel noise g[0..V) for one canvas position at one step (float32)."""
    ids = np.arange(vocab, dtype=np.uint64)
    h = word(seed, STREAM_GUMBEL, gstep, position, c0=ids >> np.uint64(2),
             w=(ids & np.uint64(3)).astype(np.int64))
    return gumbel_f32(h)


def renoise_ids(seed, gstep, positions, vocab):
    h = word(seed, STREAM_RENOISE, gstep, np.asarray(positions, dtype=np.uint64))
    return range_id(h, vocab)


def init_ids(seed, gstep, positions, vocab):
    h = word(seed, STREAM_INIT, gstep, np.asarray(positions, dtype=np.uint64))
    return range_id(h, vocab)
