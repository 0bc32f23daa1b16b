// Diffusion sampler for one canvas step on gfx950 (DiffusionGemma Technical
// Report part 4/6, section 6 "Sampling": full-precision softmax over the
// vocabulary for every canvas position plus the self-conditioning embedding
// product; explainer "DiffusionGemma: Google's open diffusion LLM", sections
// quoting report 3.1-3.3, and AlphaSignal "How text diffusion actually works":
// confident positions are locked in, the others re-noised uniformly).
//
// Four kernels, serialised on one stream:
//   samp_stats     one pass over the logits: per (row, vocab chunk) the max, the
//                  sums of exp(l - m) at T = 1 and at T, the greedy argmax and the
//                  Gumbel-perturbed argmax.  HBM-bound.
//   samp_gemm      z_partial[split] = sum_j exp(l_j - m) E_j over a vocab split:
//                  a 256 x 256 tile per workgroup, bf16x3 split precision on
//                  v_mfma_f32_32x32x16_bf16 (p = p_hi + p_lo, E = E_hi + E_lo,
//                  p_hi E_hi + p_hi E_lo + p_lo E_hi accumulated in fp32), the
//                  exponentials computed while staging the tile into LDS.
//   samp_combine   per row: merge the chunk statistics, pick the candidate,
//                  confidence, commit / re-noise, and z = sum(z_partial) / S.
//   samp_finalize  count open positions; advance the step counters.
#include "dg_common.hpp"
#include "dg_internal.hpp"

namespace dg {

struct StatsPartial {
  float m;           // max logit of the chunk (-inf if none)
  float s1;          // sum exp(l - m)
  float st;          // sum exp((l - m) / T)
  uint32_t best_id;  // smallest id attaining m
  float gscore;      // best Gumbel-perturbed score
  uint32_t gid;      // its id
  uint32_t bad;      // NaN or +inf seen
  uint32_t pad;
};

constexpr int kStatsThreads = 256;
constexpr int kStatsChunk = 16384;

__device__ __forceinline__ float rescale_factor(float m_old, float m_new, float c) {
  return (m_old == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_old - m_new) * c);
}

// Merge (m, s1, st) pairs taken relative to their own maxima.
__device__ __forceinline__ void merge_sums(float& m, float& s1, float& st, float om, float os1,
                                           float ost, float c_t) {
  const float mn = fmaxf(m, om);
  if (mn == -INFINITY) return;
  s1 = s1 * rescale_factor(m, mn, kLog2e) + os1 * rescale_factor(om, mn, kLog2e);
  st = st * rescale_factor(m, mn, c_t) + ost * rescale_factor(om, mn, c_t);
  m = mn;
}

template <bool kAligned>
__global__ __launch_bounds__(kStatsThreads) void samp_stats(const float* __restrict__ logits,
                                                            const dg_ctrl* __restrict__ ctrl,
                                                            StatsPartial* __restrict__ part,
                                                            int vocab, int chunk_len) {
  const int row = blockIdx.y;
  const int chunk = blockIdx.x;
  const dg_ctrl cb = *ctrl;
  const float temp = temperature(cb);
  const float inv_t = 1.0f / temp;
  const bool tempered = inv_t != 1.0f;
  const bool gumbel = (cb.flags & DG_GUMBEL) != 0;
  const float c_t = kLog2e * inv_t;
  const uint32_t k0 = seed_lo(cb.seed), k1 = seed_hi(cb.seed);
  const float* x = logits + (size_t)row * (size_t)vocab;
  const int j0 = chunk * chunk_len;
  const int j1 = min(vocab, j0 + chunk_len);

  float m = -INFINITY, s1 = 0.f, st = 0.f;
  uint32_t bid = 0xFFFFFFFFu;
  float gbest = -INFINITY;
  uint32_t gid = 0xFFFFFFFFu;
  uint32_t bad = 0;

  for (int j = j0 + 4 * (int)threadIdx.x; j < j1; j += 4 * kStatsThreads) {
    float v[4];
    if (kAligned && j + 3 < j1) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(x + j);
      v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (j + e < j1) ? x[j + e] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) bad |= (v[e] != v[e]) | (v[e] == INFINITY);
    const float lmax = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    if (lmax > m) {
      const uint32_t li = (v[0] == lmax) ? j : (v[1] == lmax) ? j + 1 : (v[2] == lmax) ? j + 2 : j + 3;
      s1 *= rescale_factor(m, lmax, kLog2e);
      st *= rescale_factor(m, lmax, c_t);
      m = lmax;
      bid = li;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dlt = v[e] - m;
      s1 += __builtin_amdgcn_exp2f(fmaxf(dlt * kLog2e, -200.f));
      if (tempered) st += __builtin_amdgcn_exp2f(fmaxf(dlt * c_t, -200.f));
    }
    if (gumbel) {
      const Philox4 h = philox4x32_10((uint32_t)j >> 2, (uint32_t)row, cb.gstep, kStreamGumbel, k0, k1);
      const uint32_t hw[4] = {h.w0, h.w1, h.w2, h.w3};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sc = v[e] * inv_t + gumbel_from_bits(hw[e]);
        if (sc > gbest) { gbest = sc; gid = (uint32_t)(j + e); }
      }
    }
  }
  if (!tempered) st = s1;

  // wavefront reduction
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o), os1 = __shfl_xor(s1, o), ost = __shfl_xor(st, o);
    const uint32_t obid = __shfl_xor(bid, o);
    const float mm = m;
    merge_sums(m, s1, st, om, os1, ost, c_t);
    if (better(om, obid, mm, bid)) bid = obid;
    const float og = __shfl_xor(gbest, o);
    const uint32_t ogid = __shfl_xor(gid, o);
    if (better(og, ogid, gbest, gid)) { gbest = og; gid = ogid; }
    bad |= __shfl_xor(bad, o);
  }
  __shared__ StatsPartial red[kStatsThreads / kWave];
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = StatsPartial{m, s1, st, bid, gbest, gid, bad, 0};
  __syncthreads();
  if (threadIdx.x == 0) {
    StatsPartial r = red[0];
    for (int i = 1; i < kStatsThreads / kWave; ++i) {
      const StatsPartial o = red[i];
      const float mm = r.m;
      merge_sums(r.m, r.s1, r.st, o.m, o.s1, o.st, c_t);
      if (better(o.m, o.best_id, mm, r.best_id)) r.best_id = o.best_id;
      if (better(o.gscore, o.gid, r.gscore, r.gid)) { r.gscore = o.gscore; r.gid = o.gid; }
      r.bad |= o.bad;
    }
    part[(size_t)row * gridDim.x + chunk] = r;
  }
}

// ---------------------------------------------------------------------------
// z_partial = exp(l - m) · E over one vocabulary split, bf16x3 on MFMA.
// ---------------------------------------------------------------------------
constexpr int kGM = 256;        // canvas rows per tile
constexpr int kGN = 256;        // embedding columns per tile
constexpr int kGK = 32;         // vocabulary entries per k step
constexpr int kGThreads = 256;  // 4 waves (one per SIMD): 2 (rows) x 2 (columns), 128 x 128 each
constexpr int kArrBytes = kGM * kGK * 2;        // 16 KB per bf16 array
constexpr int kStageBytes = 4 * kArrBytes;      // A_hi, A_lo, B_hi, B_lo

// LDS rows are 64 bytes (32 bf16 = four 16-byte chunks); the chunk index is
// xor-swizzled with row bits so a wavefront's 16-byte reads of one chunk
// column spread over all banks.
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * 64 + ((chunk ^ (((row >> 1) ^ (row >> 2)) & 3)) << 4);
}

// One k step's global data held by a thread between its load and its LDS store.
struct GemmRegs {
  f32x4 a[8];     // logits: rows (t>>3) + 32q, k = 4*(t&7) .. +3
  float b[32];    // E: column t, all 32 k
};

// Per-lane addressing fixed for the whole k loop: 32-bit byte offsets from
// uniform (scalar) bases; rows/columns past the end read a valid address and
// are masked when the tile is staged.
struct GemmLanes {
  uint32_t a_off0;    // byte offset of (row t>>3, k 4*(t&7)) from the logits base
  uint32_t a_step;    // bytes between rows r and r + 32
  uint32_t b_off;     // byte offset of column col0 + t from an E row base
  uint32_t row_ok;    // bit q: row (t>>3) + 32q < n_rows
  bool col_ok;
};

__device__ __forceinline__ GemmLanes gemm_lanes(int n_rows, int vocab, int d, int col0) {
  GemmLanes g;
  const int t = threadIdx.x;
  g.row_ok = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) g.row_ok |= ((t >> 3) + 32 * q < n_rows) ? (1u << q) : 0u;
  g.a_off0 = ((uint32_t)(t >> 3) * (uint32_t)vocab + 4u * (uint32_t)(t & 7)) * 4u;
  g.a_step = 32u * (uint32_t)vocab * 4u;
  const int col = col0 + t;
  g.col_ok = col < d;
  g.b_off = (uint32_t)(g.col_ok ? col : d - 1) * 4u;
  return g;
}

__device__ __forceinline__ uint32_t a_offset(const GemmLanes& g, int q) {
  return ((g.row_ok >> q) & 1u) ? g.a_off0 + (uint32_t)q * g.a_step : 0u;
}

// Interior k step: every k index is in range, no per-element checks.
__device__ __forceinline__ void gemm_load_full(GemmRegs& r, const GemmLanes& g,
                                               const float* __restrict__ logits,
                                               const float* __restrict__ emb, int d, int kbase) {
  const char* abase = reinterpret_cast<const char*>(logits + kbase);
#pragma unroll
  for (int q = 0; q < 8; ++q) r.a[q] = *reinterpret_cast<const f32x4*>(abase + a_offset(g, q));
  const char* bbase = reinterpret_cast<const char*>(emb + (size_t)kbase * (size_t)d);
  const size_t row_bytes = (size_t)d * 4u;
#pragma unroll
  for (int e = 0; e < 32; ++e) r.b[e] = *reinterpret_cast<const float*>(bbase + e * row_bytes + g.b_off);
}

// Last (ragged) k step, or an unaligned vocabulary: element-wise with k checks.
template <bool kAligned>
__device__ __forceinline__ void gemm_load_tail(GemmRegs& r, const GemmLanes& g,
                                               const float* __restrict__ logits,
                                               const float* __restrict__ emb, int d, int kbase,
                                               int kend) {
  const int t = threadIdx.x;
  const int kk = kbase + 4 * (t & 7);
  const char* abase = reinterpret_cast<const char*>(logits + kbase);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float* src = reinterpret_cast<const float*>(abase + a_offset(g, q));
    if (kAligned && kk + 3 < kend) {
      r.a[q] = *reinterpret_cast<const f32x4*>(src);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) r.a[q][e] = (kk + e < kend) ? src[e] : -INFINITY;
    }
  }
  const char* bbase = reinterpret_cast<const char*>(emb);
#pragma unroll
  for (int e = 0; e < 32; ++e)
    r.b[e] = (kbase + e < kend)
                 ? *reinterpret_cast<const float*>(bbase + (size_t)(kbase + e) * d * 4u + g.b_off)
                 : 0.0f;
}

// exp, split and store one k step's tiles into an LDS stage.
__device__ __forceinline__ void gemm_store(const GemmRegs& r, const GemmLanes& g, uint8_t* stage,
                                           const float* rm) {
  const int t = threadIdx.x;
  uint8_t* a_hi = stage;
  uint8_t* a_lo = stage + kArrBytes;
  uint8_t* b_hi = stage + 2 * kArrBytes;
  uint8_t* b_lo = stage + 3 * kArrBytes;
  const int kk = 4 * (t & 7);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = (t >> 3) + 32 * q;
    const bool ok = (g.row_ok >> q) & 1u;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = r.a[q][e];
      p[e] = (!ok || x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((x - rm[q]) * kLog2e);
    }
    uint32_t h0, l0, h1, l1;
    split2(p[0], p[1], h0, l0);
    split2(p[2], p[3], h1, l1);
    const int off = swz_off(row, kk >> 3) + ((kk & 4) << 1);
    *reinterpret_cast<u32x2*>(a_hi + off) = (u32x2){h0, h1};
    *reinterpret_cast<u32x2*>(a_lo + off) = (u32x2){l0, l1};
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = g.col_ok ? r.b[8 * c + 2 * e] : 0.f;
      const float x1 = g.col_ok ? r.b[8 * c + 2 * e + 1] : 0.f;
      split2(x0, x1, h[e], l[e]);
    }
    const int off = swz_off(t, c);
    *reinterpret_cast<u32x4*>(b_hi + off) = (u32x4){h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u32x4*>(b_lo + off) = (u32x4){l[0], l[1], l[2], l[3]};
  }
}

// acc[mb][nb] += A_tile(rows 128*wm + 32*mb ..) x B_tile(cols 128*wn + 32*nb ..), bf16x3.
__device__ __forceinline__ void gemm_mma(const uint8_t* stage, f32x16 (&acc)[4][4], int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const uint8_t* a_hi = stage;
  const uint8_t* a_lo = stage + kArrBytes;
  const uint8_t* b_hi = stage + 2 * kArrBytes;
  const uint8_t* b_lo = stage + 3 * kArrBytes;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = 2 * ks + (lane >> 5);
    bf16x8 ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int oa = swz_off(128 * wm + 32 * i + (lane & 31), chunk);
      ah[i] = *reinterpret_cast<const bf16x8*>(a_hi + oa);
      al[i] = *reinterpret_cast<const bf16x8*>(a_lo + oa);
      const int ob = swz_off(128 * wn + 32 * i + (lane & 31), chunk);
      bh[i] = *reinterpret_cast<const bf16x8*>(b_hi + ob);
      bl[i] = *reinterpret_cast<const bf16x8*>(b_lo + ob);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl[nb], acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  }
}

template <bool kAligned>
__global__ __launch_bounds__(kGThreads, 1) void samp_gemm(const float* __restrict__ logits,
                                                          const float* __restrict__ emb,
                                                          const StatsPartial* __restrict__ part,
                                                          float* __restrict__ zp, int n_rows,
                                                          int vocab, int d, int n_chunks,
                                                          int n_tiles, int ks_per_split) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  __shared__ float rowmax[kGM];

  // Workgroups are dealt round-robin to the 8 XCDs; renumber them so the
  // d-tiles of one vocabulary split sit on the same XCD and share its L2 copy
  // of the logits slice.
  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int lin = xcd * per + min(xcd, rem) + slot;
  const int tile = lin % n_tiles;
  const int split = lin / n_tiles;
  const int col0 = tile * kGN;
  const int kbegin = split * ks_per_split * kGK;
  const int kend = min(vocab, kbegin + ks_per_split * kGK);
  const int nsteps = (kend - kbegin + kGK - 1) / kGK;

  const int t = threadIdx.x;
  {
    float m = -INFINITY;
    if (t < n_rows)
      for (int c = 0; c < n_chunks; ++c) m = fmaxf(m, part[(size_t)t * n_chunks + c].m);
    rowmax[t] = m;
  }
  __syncthreads();
  float rm[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) rm[q] = rowmax[(t >> 3) + 32 * q];

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  const GemmLanes g = gemm_lanes(n_rows, vocab, d, col0);
  // Interior steps [0, nfull) run software-pipelined with two register sets:
  // step k is loaded into set k&1 and staged into LDS buffer k&1; iteration s
  // runs the MFMAs of step s, then stages step s+1 and issues the loads of step
  // s+3, so every global load has a full iteration of MFMAs to land.
  const int nfull = kAligned ? (kend - kbegin) / kGK : 0;
  GemmRegs ra, rb;
  if (nfull > 0) {
    gemm_load_full(ra, g, logits, emb, d, kbegin);
    if (nfull > 1) gemm_load_full(rb, g, logits, emb, d, kbegin + kGK);
    gemm_store(ra, g, smem, rm);
    if (nfull > 2) gemm_load_full(ra, g, logits, emb, d, kbegin + 2 * kGK);
  }
  __syncthreads();
  int s = 0;
  for (; s + 4 < nfull; s += 2) {
    gemm_mma(smem, acc, wm, wn);
    gemm_store(rb, g, smem + kStageBytes, rm);
    gemm_load_full(rb, g, logits, emb, d, kbegin + (s + 3) * kGK);
    __syncthreads();
    gemm_mma(smem + kStageBytes, acc, wm, wn);
    gemm_store(ra, g, smem, rm);
    gemm_load_full(ra, g, logits, emb, d, kbegin + (s + 4) * kGK);
    __syncthreads();
  }
  for (; s < nfull; ++s) {
    const bool odd = s & 1;
    gemm_mma(smem + (odd ? kStageBytes : 0), acc, wm, wn);
    if (s + 1 < nfull) gemm_store(odd ? ra : rb, g, smem + (odd ? 0 : kStageBytes), rm);
    if (s + 3 < nfull) gemm_load_full(odd ? ra : rb, g, logits, emb, d, kbegin + (s + 3) * kGK);
    __syncthreads();
  }
  GemmRegs& regs = ra;
  // The ragged last step (or every step of an unaligned vocabulary): checked
  // loads, not pipelined.
  for (int s = nfull; s < nsteps; ++s) {
    gemm_load_tail<kAligned>(regs, g, logits, emb, d, kbegin + s * kGK, kend);
    gemm_store(regs, g, smem, rm);
    __syncthreads();
    gemm_mma(smem, acc, wm, wn);
    __syncthreads();
  }

  // epilogue: lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 block, column lane%32
  const int lane = t & 63;
  float* out = zp + (size_t)split * (size_t)n_rows * (size_t)d;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = col0 + 128 * wn + 32 * nb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 128 * wm + 32 * mb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < n_rows && col < d) out[(size_t)row * d + col] = acc[mb][nb][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per row: statistics merge, candidate, confidence, commit / re-noise, z.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void samp_combine(const float* __restrict__ logits,
                                                    const StatsPartial* __restrict__ part,
                                                    int n_chunks, const float* __restrict__ zp,
                                                    int n_splits, const dg_ctrl* __restrict__ ctrl,
                                                    int32_t* __restrict__ ids,
                                                    uint8_t* __restrict__ committed,
                                                    float* __restrict__ z, float* __restrict__ conf,
                                                    int n_rows, int vocab, int d) {
  const int row = blockIdx.x;
  __shared__ float s_inv_s1;
  __shared__ uint32_t s_bad;
  if (threadIdx.x == 0) {
    const dg_ctrl cb = *ctrl;
    const float temp = temperature(cb);
    const float inv_t = 1.0f / temp;
    const float c_t = kLog2e * inv_t;
    StatsPartial r = part[(size_t)row * n_chunks];
    for (int c = 1; c < n_chunks; ++c) {
      const StatsPartial o = part[(size_t)row * n_chunks + c];
      const float mm = r.m;
      merge_sums(r.m, r.s1, r.st, o.m, o.s1, o.st, c_t);
      if (better(o.m, o.best_id, mm, r.best_id)) r.best_id = o.best_id;
      if (better(o.gscore, o.gid, r.gscore, r.gid)) { r.gscore = o.gscore; r.gid = o.gid; }
      r.bad |= o.bad;
    }
    const bool bad = r.bad || !(r.m > -INFINITY);
    const bool gumbel = (cb.flags & DG_GUMBEL) != 0;
    uint32_t cand = gumbel ? r.gid : r.best_id;
    if (cand >= (uint32_t)vocab) cand = 0;
    float kappa;
    if (bad) {
      kappa = __builtin_nanf("");
    } else {
      const float lc = logits[(size_t)row * vocab + cand];
      kappa = exp2f((lc - r.m) * c_t) / r.st;
    }
    if (conf) conf[row] = kappa;
    if (!committed[row]) {
      const bool last = cb.s_in_block + 1u >= cb.s_max;
      if (!bad && (kappa >= cb.tau || last)) {
        ids[row] = (int32_t)cand;
        committed[row] = 1;
      } else if (!(cb.flags & DG_COMMIT_ONLY)) {
        const Philox4 h = philox4x32_10(0u, (uint32_t)row, cb.gstep, kStreamRenoise,
                                        seed_lo(cb.seed), seed_hi(cb.seed));
        ids[row] = (int32_t)range_draw(h.w0, (uint32_t)vocab);
      }
    }
    s_inv_s1 = 1.0f / r.s1;
    s_bad = bad;
  }
  __syncthreads();
  const float inv = s_inv_s1;
  const bool bad = s_bad != 0;
  const size_t stride = (size_t)n_rows * (size_t)d;
  for (int col = threadIdx.x; col < d; col += blockDim.x) {
    const float* src = zp + (size_t)row * d + col;
    float acc = 0.f;
    for (int s = 0; s < n_splits; ++s) acc += src[s * stride];
    z[(size_t)row * d + col] = bad ? __builtin_nanf("") : acc * inv;
  }
}

__global__ __launch_bounds__(256) void samp_finalize(const uint8_t* __restrict__ committed,
                                                     uint32_t* __restrict__ n_unc,
                                                     dg_ctrl* __restrict__ ctrl, int n_rows) {
  const int t = threadIdx.x;
  const int open = (t < n_rows && !committed[t]) ? 1 : 0;
  const int count = __syncthreads_count(open);
  if (t == 0) {
    n_unc[0] = (uint32_t)count;
    if (ctrl->flags & DG_AUTO_ADVANCE) {
      ctrl->gstep += 1u;
      ctrl->s_in_block += 1u;
    }
  }
}

// ---------------------------------------------------------------------------
SamplerPlan sampler_plan(int n, int vocab, int d) {
  SamplerPlan p{};
  p.n = n; p.vocab = vocab; p.d = d;
  p.chunk_len = kStatsChunk;
  p.n_chunks = (vocab + kStatsChunk - 1) / kStatsChunk;
  p.n_tiles = (d + kGN - 1) / kGN;
  const int ksteps = (vocab + kGK - 1) / kGK;
  int splits = 256 / p.n_tiles;
  if (splits < 1) splits = 1;
  const int by_len = (ksteps + 7) / 8;
  if (splits > by_len) splits = by_len;
  if (splits < 1) splits = 1;
  p.ks_per_split = (ksteps + splits - 1) / splits;
  p.n_splits = (ksteps + p.ks_per_split - 1) / p.ks_per_split;
  p.off_stats = 0;
  p.off_zp = align_up((size_t)n * p.n_chunks * sizeof(StatsPartial), 256);
  p.total = p.off_zp + align_up((size_t)p.n_splits * n * d * sizeof(float), 256);
  return p;
}

hipError_t launch_sampler(const SamplerPlan& p, const float* logits, const float* emb,
                          int32_t* ids, uint8_t* committed, float* z, float* conf,
                          uint32_t* n_unc, dg_ctrl* ctrl, void* ws, hipStream_t s) {
  StatsPartial* part = reinterpret_cast<StatsPartial*>(static_cast<uint8_t*>(ws) + p.off_stats);
  float* zp = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.off_zp);
  const bool aligned = (p.vocab % 4) == 0;

  prof_begin("samp_stats", s);
  if (aligned)
    samp_stats<true><<<dim3(p.n_chunks, p.n), kStatsThreads, 0, s>>>(logits, ctrl, part, p.vocab, p.chunk_len);
  else
    samp_stats<false><<<dim3(p.n_chunks, p.n), kStatsThreads, 0, s>>>(logits, ctrl, part, p.vocab, p.chunk_len);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  prof_begin("samp_gemm", s);
  const int nwg = p.n_tiles * p.n_splits;
  if (aligned)
    samp_gemm<true><<<nwg, kGThreads, 0, s>>>(logits, emb, part, zp, p.n, p.vocab, p.d, p.n_chunks,
                                              p.n_tiles, p.ks_per_split);
  else
    samp_gemm<false><<<nwg, kGThreads, 0, s>>>(logits, emb, part, zp, p.n, p.vocab, p.d, p.n_chunks,
                                               p.n_tiles, p.ks_per_split);
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  prof_begin("samp_combine", s);
  samp_combine<<<p.n, 256, 0, s>>>(logits, part, p.n_chunks, zp, p.n_splits, ctrl, ids, committed,
                                   z, conf, p.n, p.vocab, p.d);
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  prof_begin("samp_finalize", s);
  samp_finalize<<<1, 256, 0, s>>>(committed, n_unc, ctrl, p.n);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace dg
