/*
 * Plain C helpers for the CPU oracle (test infrastructure only): the same
 * Philox4x32-10 draws as oracle/philox.py, evaluated row by row so that full
 * 262k-vocabulary decode runs finish in seconds.  Written from the published
 * definition (Salmon et al., SC'11); pinned in the tests against the numpy
 * oracle, which is itself pinned against rocRAND's engine.  Compile with
 * -ffp-contract=off: the Gumbel score is one float32 multiply then one float32
 * add, like the numpy oracle.
 */
#include <math.h>
#include <stdint.h>

static void philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1,
                   uint32_t out[4]) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    if (r < 9) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void dg_oracle_philox(const uint32_t* ctr, int64_t n, uint32_t k0, uint32_t k1, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i)
    philox(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], k0, k1, out + 4 * i);
}

static float gumbel(uint32_t h) {
  const float u = (float)(((uint64_t)(h >> 9) << 1) | 1u) * 5.9604644775390625e-08f;
  const float t = -logf(u);
  return -logf(t);
}

/* scores[r, j] = logits[r, j] * inv_t + g(seed, gstep, positions[r], j), float32 */
void dg_oracle_gumbel_scores(const float* logits, int64_t n_rows, int64_t vocab, float inv_t,
                             uint64_t seed, uint32_t gstep, const int64_t* positions,
                             float* scores) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    const float* l = logits + r * vocab;
    float* s = scores + r * vocab;
    for (int64_t c = 0; 4 * c < vocab; ++c) {
      uint32_t h[4];
      philox((uint32_t)c, (uint32_t)positions[r], gstep, 0u, k0, k1, h);
      for (int w = 0; w < 4 && 4 * c + w < vocab; ++w) {
        const int64_t j = 4 * c + w;
        const float a = l[j] * inv_t;
        s[j] = a + gumbel(h[w]);
      }
    }
  }
}

/* noise[r, j] = table[h >> 16], h = word (j & 3) of counter (j >> 2, positions[r], gstep, 6) */
void dg_oracle_synth_noise(const float* table, int64_t n_rows, int64_t vocab, uint64_t seed,
                           uint32_t gstep, const int64_t* positions, float* out) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    float* o = out + r * vocab;
    for (int64_t c = 0; 4 * c < vocab; ++c) {
      uint32_t h[4];
      philox((uint32_t)c, (uint32_t)positions[r], gstep, 6u, k0, k1, h);
      for (int w = 0; w < 4 && 4 * c + w < vocab; ++w) o[4 * c + w] = table[h[w] >> 16];
    }
  }
}
