// Diffusion sampler for one canvas step on gfx950 (DiffusionGemma Technical
// Report part 4/6, section 6 "Sampling": full-precision softmax over the
// vocabulary for every canvas position plus the self-conditioning embedding
// product; explainer "DiffusionGemma: Google's open diffusion LLM", sections
// quoting report 3.1-3.3, and AlphaSignal "How text diffusion actually works":
// confident positions are locked in, the others re-noised uniformly).
//
// The vocabulary is cut into splits (a few hundred k-blocks of 16 ids each);
// every (row, split) pair keeps its own maximum m_s, so no pass needs the
// global row maximum before the contraction.
//
//   samp_stats     per (split, row), from one read of the logits held in
//                  registers: the max, the greedy argmax and the Gumbel-perturbed
//                  argmax, then the sums of exp(l - m_s) at T = 1 and at T, and
//                  the weights p = exp(l - m_s) written as split-precision
//                  "images": per k-block of 16 ids, 256 row slots of 64 bytes.
//   samp_gemm      z_s = sum_j p_j E_j over one split for a 256 x 256 tile, both
//                  operands streamed through LDS, fp32 accumulation.  On the
//                  packed table (dg_embedding_pack) each product is one fp16
//                  term plus two fp6 corrections (below); on the plain float32
//                  table E is split into bf16 hi / lo while it streams and the
//                  product is bf16x3 (p_hi E_hi + p_hi E_lo + p_lo E_hi).
//   samp_combine   per row: merge the split statistics (log-sum-exp), the
//                  candidate, its confidence, commit / re-noise, and
//                  z = sum_s 2^((m_s - m) log2 e) z_s / S.
//   samp_finalize  count open positions; advance the step counters.
//
// fp16 + fp6 split precision.  The table holds each row at its own scale:
// Q_k = E_k 2^(c + d_k), where c puts max|E| 2^c in [2^7, 2^8) and the row
// shift d_k (0-40) brings row k's own maximum there as well; the weights carry
// the inverse shift, P'_k = p_k 2^(14 - d_k), so P'_k Q_k = 2^(14 + c) p_k E_k.
// With P'16 = fp16(P'), Q16 = fp16(Q), the contraction sums
//     P'16 Q16  +  P'16 (Q - Q16)  +  (P' - P'16) Q16
// = P'Q - (P' - P'16)(Q - Q16), the first term on fp16 matrix cores (exact
// products, fp32 sums), the two corrections (2^-11 of a term) on fp6 ones:
// e2m3 codes (three mantissa bits, 7.5 at most) under power-of-two block
// scales, one per row and 16-id k-block on the p side (the codes of P'16 and of
// fp16((P' - P'16) 2^11)) and one per 16-id k-block and 64-column group on
// the table side (the codes of (Q - Q16) 2^11 and of Q16).  A code keeps
// relative error <= 2^-4 unless it is far below its block's largest value;
// the row shifts keep the table's rows level, so that a block's small values
// belong to small terms.  The table stores Q16, the codes of (Q - Q16) 2^11 and
// their scale (3 bytes per element) and one shift byte per id; the codes of
// Q16 are formed in the contraction.  One v_mfma_f32_32x32x16_f16 per 16 ids
// and one v_mfma_scale_f32_32x32x64_f8f6f4 (fp6 x fp6, per-lane scales) per
// 32 ids (the corrections of two k-blocks side by side in K).  The combine
// multiplies by 2^-(14 + c), which dg_embedding_pack stores after the table.
#include "dg_common.hpp"
#include "dg_internal.hpp"

namespace dg {

struct StatsPartial {
  float m;           // max logit of the (row, split) range (-inf if none)
  float s1;          // sum exp(l - m)
  float st;          // sum exp((l - m) / T)
  uint32_t best_id;  // smallest id attaining m
  float gscore;      // best Gumbel-perturbed score
  uint32_t gid;      // its id
  uint32_t bad;      // NaN or +inf seen
  float sy;          // sum 2^y * y with y = (l - m) log2(e) / T (entropy of p_T)
};

// Per-row results the entropy-bounded mode hands from the combine to the
// selection kernel (workspace arrays), plus the caller's entropy output.
struct EbRows {
  bool on;
  float* ent;        // [n] entropy of p_T (nats), NaN for undefined rows
  int32_t* cand;     // [n] candidate id
  int32_t* argmax;   // [n] greedy argmax id
  float* ent_out;    // caller's [n] entropy output or null
};

constexpr int kKB = 16;            // vocabulary ids per k-block
constexpr int kImgRow = 64;        // bytes per row slot of a k-block image (16 ids)
constexpr int kGM = 256;           // canvas row slots per image / rows per contraction tile
constexpr int kGN = 256;           // embedding columns per contraction tile
constexpr int kPImg = kGM * kImgRow;   // 16 KB: the p image of one k-block
constexpr int kGThreads = 512;     // 8 waves (two per SIMD): 2 x 4, 128 x 64 each
constexpr int kArr = kGM * kImgRow;    // 16 KB: one operand of one LDS stage
constexpr int kStage = 2 * kArr;       // p tile + E tile
constexpr int kStatsThreads = 256;

// Record layouts of one 64-byte slot (16 ids of one row of p, or one column of E
// in LDS):
//   bf16x3:    bf16 hi of ids 0-15 | bf16 lo of ids 0-15
//   fp16 + fp6 (p side):  fp16 P'16 of ids 0-15 | 32 e2m3 codes (24 bytes) |
//              scale byte | 7 zero bytes (p_record)
//   fp16 + fp6 (E side, in LDS):  fp16 Q16 of ids 0-15 | the residual chunks
//              of this k-block and of the next (even k-blocks only), each 12
//              bytes of e2m3 codes, a scale byte and 3 zero bytes
constexpr int kPExp = 14;              // P = p 2^14 (before the row shift)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, (f16x2){(_Float16)a, (_Float16)b});
}

// e2m3 code (sign in bit 5, two exponent bits of bias 1, three mantissa bits)
// of v, |v| <= 7.5, rounded to the nearest value with ties to the even code.
// Below 1 the values are spaced 1/8 apart, so the code is rint(8 |v|) (8 is the
// code of 1.0); from 1 up the float's mantissa is rounded to three bits and
// its exponent rebiased from 127 to 1.  NaN gives 31.
__device__ __forceinline__ uint32_t e2m3_code(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ab = b & 0x7fffffffu;
  const float a = __uint_as_float(ab);
  const uint32_t nrm = min(((ab + 0x7ffffu + ((ab >> 20) & 1u)) >> 20) - 1008u, 31u);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 8.0f);
  return (a < 1.0f ? sub : nrm) | ((b >> 26) & 32u);
}

// The smallest e >= lo with m <= 7.5 2^e (m >= 0): for m = 1.f 2^E that is
// E - 2, plus one when 1.f > 1.875.
__device__ __forceinline__ int e2m3_scale_exp(float m, int lo) {
  const uint32_t b = __float_as_uint(m);
  return max((int)(b >> 23) - 129 + (int)((b & 0x7fffffu) > 0x700000u), lo);
}

// The correction half of a p record from the 16 weights P' of one row and
// k-block (P' = p 2^(14 - d), d the id's row shift in the table): fp16 P'16
// (eight dwords, id order), then 32 e2m3 codes (six dwords): P'16 of ids
// 0-15 and r = fp16((P' - P'16) 2^11) of ids 0-15, both divided by 2^es, the
// smallest power of two (at least 2^-116) that brings the largest of the 32
// fp16 values to 7.5 or below (the conversion rounds to nearest, ties to the
// even code); then the E8M0 byte 116 + es (so the matrix core multiplies the
// codes by 2^(es - 11)) and a zero dword.
__device__ __forceinline__ void p_record(const float (&x)[16], u32x4 (&rec)[4]) {
  // w: P'16 of ids 0-15 (dwords 0-7), then r of ids 0-15 (dwords 8-15)
  u32x16 w;
  float mx = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w[k] = pack_f16x2(x[2 * k], x[2 * k + 1]);
    const f16x2 hh = __builtin_bit_cast(f16x2, (uint32_t)w[k]);
    // (P' - P'16) 2^11, exact: both products are exact and so is their sum
    const float r0 = __builtin_fmaf((float)hh[0], -2048.0f, x[2 * k] * 2048.0f);
    const float r1 = __builtin_fmaf((float)hh[1], -2048.0f, x[2 * k + 1] * 2048.0f);
    w[8 + k] = pack_f16x2(r0, r1);
    mx = fmaxf(mx, fmaxf(fmaxf(x[2 * k], x[2 * k + 1]), fmaxf(fabsf(r0), fabsf(r1))));
  }
  // the largest of the 32 fp16 values: fp16 rounding is monotonic, so it is
  // the fp16 rounding of the largest float
  const int es = e2m3_scale_exp((float)(_Float16)mx, -116);
  const u32x6 c = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(__builtin_bit_cast(f16x32, w),
                                                              __uint_as_float((uint32_t)(127 + es) << 23));
  rec[0] = (u32x4){w[0], w[1], w[2], w[3]};
  rec[1] = (u32x4){w[4], w[5], w[6], w[7]};
  rec[2] = (u32x4){c[0], c[1], c[2], c[3]};
  rec[3] = (u32x4){c[4], c[5], (uint32_t)(116 + es), 0u};
}

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

// sy moves with the reference: y' = y + (m_a - m) c_t, so sy' = f (sy + st (m_a - m) c_t).
__device__ __forceinline__ float shift_sy(float sy, float st, float m_a, float m, float c_t) {
  if (m_a == -INFINITY) return 0.0f;
  return rescale_factor(m_a, m, c_t) * (sy + st * ((m_a - m) * c_t));
}

__device__ __forceinline__ void merge_partial(StatsPartial& r, const StatsPartial& o, float c_t) {
  const float mm = r.m;
  const float mn = fmaxf(r.m, o.m);
  if (mn != -INFINITY) r.sy = shift_sy(r.sy, r.st, r.m, mn, c_t) + shift_sy(o.sy, o.st, o.m, mn, c_t);
  merge_sums(r.m, r.s1, r.st, o.m, o.s1, o.st, c_t);
  if (better(o.m, o.best_id, mm, r.best_id)) r.best_id = o.best_id;
  if (better(o.gscore, o.gid, r.gscore, r.gid)) { r.gscore = o.gscore; r.gid = o.gid; }
  r.bad |= o.bad;
}

// 4 logits from id j on (ids >= vocab read as -inf); with 16-byte aligned rows
// (kAligned: vocab % 4 == 0) a group is wholly inside or outside the row.
template <bool kAligned>
__device__ __forceinline__ f32x4 load4(const float* __restrict__ x, int j, int vocab) {
  if (kAligned) {
    // non-temporal: the logits are read once and should not displace
    // lines that other workgroups will read again
    if (j < vocab) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + j));
    return (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (j + e < vocab) ? x[j + e] : -INFINITY;
  return v;
}

constexpr int kStatsRows = 2;                            // canvas rows per workgroup
constexpr int kStatsWavesPerRow = 4;
constexpr int kStatsLanes = 64 * kStatsWavesPerRow;      // lanes sharing one row
constexpr int kStatsIters = 4;                           // rounds of kStatsLanes k-blocks
constexpr int kStatsChunks = 4 * kStatsIters;            // 4-id groups held per lane
constexpr int kMaxKbPerSplit = kStatsLanes * kStatsIters;
constexpr int kStatsThreadsWG = 64 * kStatsRows * kStatsWavesPerRow;

// grid (n_splits, ceil(n_rows / 2)), two rows per workgroup, 4 waves per row (two rows
// fill whole 128-byte lines of the p image; two workgroups share a CU, so
// some load while others store).
// Round i covers k-blocks kb0 + 256 i .. kb0 + 256 i + 255 of the split.  In
// it, lane L holds the 4-id groups c = 4 i .. 4 i + 3, group c starting at id
// 16 kb0 + 4 (256 c + L): every load instruction of the row reads 1 KB of
// consecutive logits, and lanes 4k .. 4k + 3 hold one k-block.  The logits
// are read from HBM once and kept in registers: the split maximum is reduced
// first, then the same registers give exp(l - m_s), the sums and the p
// image records (kF16: fp16 + fp6 from p_record, else bf16 hi / lo).  Each
// round's image slots are staged in LDS and leave as 1 KB per store
// instruction (8 k-blocks' 128-byte lines of the image; staging through LDS
// measured faster than storing from the registers, and whole lines measured
// faster than one row's 64-byte halves).  For the fp6 records a lane needs a
// whole k-block: each lane writes its weights P' (already carrying the row
// shifts, which the split holds in LDS) into the slot of their k-block, and
// lane 4k + q then reads k-block 64 q + k' (k' = L / 4) back whole and
// replaces it with its record.  The four writers of a slot are the lanes of
// one quad, in the same wave, so no barrier separates the two.  Four waves
// per SIMD are kept (128 registers: two values spill, stored at the start and
// reloaded at the end).
//
// The staging holds one round's slots as [row][k-block][64 B], the 16-byte
// chunk position xor-swizzled with bits 6-7 of the k-block (the quad place of
// the lane that takes it), so that a wave's 16-byte accesses to the same chunk
// of 64 k-blocks spread over all banks.
__device__ __forceinline__ int stage_off(int r, int kb_local, int chunk) {
  return (r * kStatsLanes + kb_local) * kImgRow + 16 * (chunk ^ ((kb_local >> 6) & 3));
}

template <bool kAligned, bool kF16>
__global__ __launch_bounds__(kStatsThreadsWG) __attribute__((amdgpu_waves_per_eu(4)))
void samp_stats(const float* __restrict__ logits, const dg_ctrl* __restrict__ ctrl,
                StatsPartial* __restrict__ part, uint8_t* __restrict__ pimg,
                const uint8_t* __restrict__ shifts, int n_rows, int n_canvas, int vocab, int kb_per_split,
                int n_kb, bool want_h) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStatsLanes * kStatsRows * kImgRow];
  // kF16: the row shifts of the split's k-blocks (16 bytes each)
  __shared__ __attribute__((aligned(16))) uint8_t shl[kF16 ? kMaxKbPerSplit * kKB : 16];
  __shared__ StatsPartial red[kStatsRows][kStatsWavesPerRow];
  const int split = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int r = wave / kStatsWavesPerRow;                  // row within the workgroup
  const int L = (wave % kStatsWavesPerRow) * 64 + lane;    // lane within the row
  const int row0 = blockIdx.y * kStatsRows;
  const int row = row0 + r;
  const bool row_ok = row < n_rows;
  // rows of canvas c are c * n_canvas .. ; each canvas has its own control block
  const dg_ctrl cb = ctrl[row_ok ? row / n_canvas : 0];
  const uint32_t pos = (uint32_t)(row % n_canvas);   // position within the canvas
  const int mt = row0 / kGM;                         // 256-row image tile of this row
  const float temp = temperature(cb);
  const float inv_t = 1.0f / temp;
  const bool tempered = inv_t != 1.0f;
  const bool gumbel = (cb.flags & DG_GUMBEL) != 0;
  const float c_t = kLog2e * inv_t;
  const uint32_t k0 = seed_lo(cb.seed), k1 = seed_hi(cb.seed);
  const float* x = logits + (size_t)(row_ok ? row : 0) * (size_t)vocab;
  const int kb0 = split * kb_per_split;
  const int kb1 = min(n_kb, kb0 + kb_per_split);
  const int id_end = min(vocab, kb1 * kKB);          // first id past this split

  if constexpr (kF16) {
    // the split's shift bytes into LDS by direct loads, 1 KB per instruction
    // (bytes past the split read as zero); they land before the barrier that
    // follows the logits' first pass
    const __amdgpu_buffer_rsrc_t rs = rsrc(shifts + (size_t)kb0 * kKB, (uint32_t)(kb1 - kb0) * kKB);
#pragma unroll
    for (int k = 0; k < kMaxKbPerSplit * kKB / 1024 / (kStatsThreadsWG / 64); ++k) {
      const int piece = wave + (kStatsThreadsWG / 64) * k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(shl + 1024 * piece), 16, 1024 * piece + 16 * lane, 0,
                                               0, 0);
    }
  }
  // group c: first id, and whether it lies in the split
  auto gid0 = [&](int c) { return kb0 * kKB + 4 * (kStatsLanes * c + L); };
  f32x4 v[kStatsChunks];
#pragma unroll
  for (int c = 0; c < kStatsChunks; ++c) {
    const int j = gid0(c);
    if (row_ok && j < id_end) v[c] = load4<kAligned>(x, j, id_end);
    else v[c] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }

  // max, argmax, Gumbel argmax, undefined values
  float m = -INFINITY;
  uint32_t bid = 0xFFFFFFFFu;
  float gbest = -INFINITY;
  uint32_t gid = 0xFFFFFFFFu;
  uint32_t bad = 0;
#pragma unroll
  for (int c = 0; c < kStatsChunks; ++c) {
    const int j = gid0(c);
    if (!(row_ok && j < id_end)) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bad |= (v[c][e] != v[c][e]) | (v[c][e] == INFINITY);
      if (v[c][e] > m) { m = v[c][e]; bid = (uint32_t)(j + e); }
    }
    if (gumbel) {
      const Philox4 h = philox4x32_10((uint32_t)(j >> 2), pos, cb.gstep, kStreamGumbel, k0, k1);
      const uint32_t hw[4] = {h.w0, h.w1, h.w2, h.w3};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sc = v[c][e] * inv_t + gumbel_from_bits(hw[e]);
        if (sc > gbest) { gbest = sc; gid = (uint32_t)(j + e); }
      }
    }
  }
  wave_argmax(m, bid);
  wave_argmax(gbest, gid);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o);
  const int qw = wave % kStatsWavesPerRow;
  if (lane == 0) red[r][qw] = StatsPartial{m, 0.f, 0.f, bid, gbest, gid, bad, 0.f};
  if constexpr (kF16) wait_vmcnt<0>();   // this wave's shift loads have landed in LDS
  __syncthreads();
  {
    StatsPartial acc = red[r][0];
#pragma unroll
    for (int w = 1; w < kStatsWavesPerRow; ++w) {
      const StatsPartial o = red[r][w];
      if (better(o.m, o.best_id, acc.m, acc.best_id)) { acc.m = o.m; acc.best_id = o.best_id; }
      if (better(o.gscore, o.gid, acc.gscore, acc.gid)) { acc.gscore = o.gscore; acc.gid = o.gid; }
      acc.bad |= o.bad;
    }
    m = acc.m; bid = acc.best_id; gbest = acc.gscore; gid = acc.gid; bad = acc.bad;
  }

  // exp(l - m_s), its sums, the p image records, round by round
  const float mc = (m == -INFINITY) ? 0.0f : -m * kLog2e;
  float s1 = 0.f, st = 0.f, sy = 0.f;
#pragma unroll
  for (int i = 0; i < kStatsIters; ++i) {
    const int base = kb0 + kStatsLanes * i;
    if (base >= kb1) break;   // uniform over the workgroup
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * i + q;
      float pp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[c][e], kLog2e, mc));
        s1 += pp[e];
        if (tempered || want_h) {
          const float y = fmaxf((v[c][e] - m) * c_t, -200.f);   // log2 of the tempered weight
          const float et = tempered ? __builtin_amdgcn_exp2f(y) : pp[e];
          st += et;
          if (want_h) sy += et * y;
        }
      }
      // k-block 64 q + L / 4 of the round, ids 4 (L % 4) .. 4 (L % 4) + 3 of it
      const int kbq = kStatsLanes / 4 * q + L / 4;
      if constexpr (kF16) {
        // P' = p 2^(14 - d) per id, in the slot (chunk L % 4) of the lane that
        // takes this k-block
        const uint32_t d4 =
            *reinterpret_cast<const uint32_t*>(shl + (size_t)(kStatsLanes * i + kbq) * kKB + 4 * (L % 4));
        f32x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = __builtin_ldexpf(pp[e], kPExp - (int)((d4 >> (8 * e)) & 0xffu));
        *reinterpret_cast<f32x4*>(stage + stage_off(r, kbq, L % 4)) = w4;
      } else {
        uint32_t hi[2], lo[2];
        split2(pp[0], pp[1], hi[0], lo[0]);
        split2(pp[2], pp[3], hi[1], lo[1]);
        *reinterpret_cast<uint2*>(stage + stage_off(r, kbq, (L % 4) >> 1) + 8 * (L & 1)) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2*>(stage + stage_off(r, kbq, 2 + ((L % 4) >> 1)) + 8 * (L & 1)) =
            make_uint2(lo[0], lo[1]);
      }
    }
    if constexpr (kF16) {
      // this lane's k-block of the round, 64 (L % 4) + L / 4: its 16 weights
      // P' (the quad's lanes wrote them into its slot in this wave, so no
      // barrier is needed); the record then replaces them in the same slot
      const int kbo = kStatsLanes / 4 * (L % 4) + L / 4;
      float x[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(stage + stage_off(r, kbo, k));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * k + e] = w4[e];
      }
      u32x4 rec[4];
      p_record(x, rec);
#pragma unroll
      for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(stage + stage_off(r, kbo, k)) = rec[k];
    }
    __syncthreads();
    // write-out: the row slots of k-block kbl are contiguous; thread T moves
    // 16-byte pieces T, T + kStatsThreadsWG, ... of the round's staging
    constexpr int kPieces = kStatsLanes * kStatsRows * kImgRow / 16;
#pragma unroll
    for (int k = 0; k < kPieces / kStatsThreadsWG; ++k) {
      const int c = t + kStatsThreadsWG * k;
      const int kbl = c / (kStatsRows * kImgRow / 16);
      const int off = c % (kStatsRows * kImgRow / 16);          // 16-byte piece of the k-block's slots
      const int kb = base + kbl;
      if (kb < kb1 && row0 + off / (kImgRow / 16) < n_rows) {
        const u32x4 w =
            *reinterpret_cast<const u32x4*>(stage + stage_off(off / (kImgRow / 16), kbl, off % (kImgRow / 16)));
        // non-temporal: the images stream out rather than stay dirty in this
        // XCD's L2 (the contraction reads them from other XCDs); measured
        // ~5 us onto this kernel and ~15 us off the contraction that follows
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(pimg + ((size_t)mt * n_kb + kb) * kPImg +
                                                                  (size_t)(row0 % kGM) * kImgRow + off * 16));
      }
    }
    __syncthreads();
  }
  if (!tempered && !want_h) st = s1;
  s1 = wave_sum(s1);
  st = wave_sum(st);
  sy = wave_sum(sy);
  if (lane == 0) { red[r][qw].s1 = s1; red[r][qw].st = st; red[r][qw].sy = sy; }
  __syncthreads();
  if (qw == 0 && lane == 0 && row_ok) {
    float a1 = 0.f, at = 0.f, ay = 0.f;
#pragma unroll
    for (int w = 0; w < kStatsWavesPerRow; ++w) { a1 += red[r][w].s1; at += red[r][w].st; ay += red[r][w].sy; }
    part[(size_t)row * gridDim.x + split] = StatsPartial{m, a1, at, bid, gbest, gid, bad, ay};
  }
}

// ---------------------------------------------------------------------------
// E packing: Q_k = E_k 2^(c + d_k) as fp16 Q16 plus the e2m3 codes of
// (Q - Q16) 2^11.  Columns are padded to whole 256-column tiles and ids to
// whole pairs of 16-id k-blocks (zeros).  For each k-block pair j and column
// tile t, one 24 KB block at ((j n_tiles + t) 24 KB): the Q16 records of
// k-block 2j (256 columns x 32 B: ids 0-7, ids 8-15), those of k-block 2j + 1,
// then 256 columns x 32 B of residual chunks (16 B for k-block 2j, 16 for
// 2j + 1: 12 bytes of codes, code i at bit 6i, under the scale 2^eB of the
// k-block and 64-column group, then the byte 127 + eB and three zeros).  After
// the blocks: the row shifts d_k (one byte per id of the padded vocabulary,
// 256-byte aligned), kAmaxParts partial maxima of |E| (working space of the
// pack) and the PackTail record.
// ---------------------------------------------------------------------------
constexpr int kEBlock = 24576;          // bytes per (k-block pair, column tile)
constexpr int kEHalf = 8192;            // Q16 records of one k-block and tile
constexpr int kEResid = 16384;          // offset of the residual bytes in a block
constexpr int kAmaxParts = 1024;
struct PackTail {
  float zscale;    // 2^-(14 + c): undoes P = p 2^14 and Q = E 2^c in the combine
  int32_t c;       // the table's exponent shift
};
constexpr size_t kPackTailBytes = 256;

__device__ __forceinline__ float block_max256(float m, float* red) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Partial maxima of |E| over a grid-stride sweep (NaN entries are skipped;
// they reach z through the records all the same).
__global__ __launch_bounds__(256) void emb_amax_kernel(const float* __restrict__ emb, size_t n,
                                                       float* __restrict__ part) {
  __shared__ float red[4];
  const size_t stride = (size_t)gridDim.x * 256;
  float m = 0.0f;
  if ((reinterpret_cast<uintptr_t>(emb) & 15) == 0) {
    const f32x4* e4 = reinterpret_cast<const f32x4*>(emb);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n / 4; i += stride) {
      const f32x4 v = e4[i];
      m = fmaxf(fmaxf(m, fmaxf(fabsf(v[0]), fabsf(v[1]))), fmaxf(fabsf(v[2]), fabsf(v[3])));
    }
    for (size_t i = n / 4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
      m = fmaxf(m, fabsf(emb[i]));
  } else {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) m = fmaxf(m, fabsf(emb[i]));
  }
  m = block_max256(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// c = 8 - e for max|E| in [2^(e-1), 2^e), so max|Q| lies in [2^7, 2^8); capped
// at 80 so that the combine's weight 2^-(14 + c) / S (S <= 2^31) stays a normal
// float (tables with max|E| below 2^-72 keep fewer fp16 bits).  A zero or
// non-finite maximum leaves the table unscaled.
__global__ __launch_bounds__(256) void emb_scale_kernel(const float* __restrict__ part,
                                                        PackTail* __restrict__ tail) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < kAmaxParts; i += 256) m = fmaxf(m, part[i]);
  m = block_max256(m, red);
  if (threadIdx.x == 0) {
    int c = 0;
    if (m > 0.0f && m <= 3.4028234663852886e38f) {
      int e;
      (void)frexpf(m, &e);
      c = min(8 - e, 80);
    }
    tail->c = c;
    tail->zscale = ldexpf(1.0f, -(14 + c));
  }
}

// grid (2 n_pairs, n_tiles): one thread per column and k-block (k-blocks on x,
// which takes the large count).
// Row shifts: d_k = min(max(8 - c - e_k, 0), 40) for max|E_k| in
// [2^(e_k - 1), 2^e_k), so that max|E_k| 2^(c + d_k) lies in [2^7, 2^8) unless
// capped.  Rows without a positive finite maximum (zero rows) and ids past
// vocab take the largest shift, 40: their weights P' = P 2^-40 then never set
// a k-block's correction scale.  One wave per id.
__global__ __launch_bounds__(256) void emb_shift_kernel(const float* __restrict__ emb, int vocab, int d,
                                                        int n_ids, const PackTail* __restrict__ tail,
                                                        uint8_t* __restrict__ shifts) {
  const int id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (id >= n_ids) return;   // uniform over the wave
  float m = 0.0f;
  if (id < vocab) {
    const float* row = emb + (size_t)id * d;
    if ((d & 3) == 0 && (reinterpret_cast<uintptr_t>(emb) & 15) == 0) {
      const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
      for (int j = lane; j < d / 4; j += 64) {
        const f32x4 v = r4[j];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
      }
    } else {
      for (int j = lane; j < d; j += 64) m = fmaxf(m, fabsf(row[j]));
    }
  }
  m = wave_max(m);
  if (lane == 0) {
    int sh = 40;
    if (m > 0.0f && m <= 3.4028234663852886e38f) {
      int e;
      (void)frexpf(m, &e);
      sh = min(max(8 - tail->c - e, 0), 40);
    }
    shifts[id] = (uint8_t)sh;
  }
}

__global__ __launch_bounds__(256) void emb_pack_kernel(const float* __restrict__ emb,
                                                       uint8_t* __restrict__ out, int vocab, int d,
                                                       int n_tiles, const PackTail* __restrict__ tail,
                                                       const uint8_t* __restrict__ shifts) {
  const int cl = threadIdx.x;                 // column within the tile
  const int tile = blockIdx.y;
  const int col = tile * 256 + cl;
  const int kb = blockIdx.x;
  const int c = tail->c;
  uint32_t h16[8];
  float qe[16];
  float mx = 0.0f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    float x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k = kb * kKB + 2 * g + e;
      x[e] = (k < vocab && col < d) ? ldexpf(emb[(size_t)k * d + col], c + (int)shifts[k]) : 0.0f;
    }
    h16[g] = pack_f16x2(x[0], x[1]);
    const f16x2 h = __builtin_bit_cast(f16x2, h16[g]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      qe[2 * g + e] = (x[e] - (float)h[e]) * 2048.0f;
      mx = fmaxf(mx, fmaxf(fabsf(qe[2 * g + e]), fabsf((float)h[e])));
    }
  }
  // one scale per k-block and 64-column group (the group one wave holds)
  const int eb = e2m3_scale_exp(wave_max(mx), -126);
  const float inv = __uint_as_float((uint32_t)(127 - eb) << 23);
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = e2m3_code(qe[i] * inv);
    const int bit = 6 * i;
    w[bit / 32] |= c << (bit % 32);
    if (bit % 32 > 26) w[bit / 32 + 1] |= c >> (32 - bit % 32);
  }
  uint8_t* blk = out + ((size_t)(kb >> 1) * n_tiles + tile) * kEBlock;
  uint8_t* q = blk + (kb & 1) * kEHalf + cl * 32;
  *reinterpret_cast<u32x4*>(q) = (u32x4){h16[0], h16[1], h16[2], h16[3]};
  *reinterpret_cast<u32x4*>(q + 16) = (u32x4){h16[4], h16[5], h16[6], h16[7]};
  *reinterpret_cast<u32x4*>(blk + kEResid + cl * 32 + (kb & 1) * 16) = (u32x4){w[0], w[1], w[2], (uint32_t)(127 + eb)};
}

// ---------------------------------------------------------------------------
// z_s = p · E over one split on MFMA (fp16 + fp6 on the packed table, bf16x3
// on the float32 table).  A four-stage LDS pipeline fed
// by direct global-to-LDS loads: no staging registers and no LDS store
// instructions; the fragments of the next step are read while the MFMAs of
// the current one run.
// ---------------------------------------------------------------------------

// LDS rows are 64 bytes (four 16-byte chunks: ids 0-7 and 8-15 of the fp16 or
// bf16-hi values, then the two correction chunks); the chunk index is
// xor-swizzled with row bits so a wavefront's 16-byte reads of one chunk
// column spread over all banks.
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * 64 + ((chunk ^ (((row >> 1) ^ (row >> 2)) & 3)) << 4);
}

constexpr int kStages = 4;            // LDS stages of 32 KB (float32-table path)
constexpr int kDist = kStages - 1;     // DMA runs this many steps ahead (float32-table path)
constexpr int kDmaPerStep = 4;         // LDS DMA instructions per wave per k step (float32-table path)

// DMA one k step into an LDS stage: 16-byte buffer loads that write LDS
// directly (lane i of an instruction lands at destination + 16 i); lane i
// fetches the global chunk that belongs at its swizzled slot.
//   float32-table path (gemm_dma): wave w moves rows 32w..32w+31 of the p
//     image, and id rows 2w and 2w + 1 of the k-block from the plain float32
//     table [V, d], 1 KB each (the tile's 256 columns), into LDS rows of 1 KB;
//     lane i fetches the 16-byte chunk i ^ f(row) so id rows r and r + 8 sit
//     128 bytes apart in the banks.  Ids past the vocabulary and columns past
//     d read as zero (buffer range checks; d is a multiple of 4).
//   packed-table path (gemm_dma16): waves 0-3 alone move the step, wave w
//     the p rows and E columns 64w..64w+63.  The table's (k-block pair,
//     tile) blocks give each LDS column row its Q16 chunks and, for an even
//     k-block, the residual bytes of the pair; an odd k-block's residual
//     lanes point past the block's range, so they load zeros and move no
//     memory.
struct EOperand {
  const uint8_t* base;  // packed table, or float32 E
  int d;                // row length of float32 E (elements)
  int vocab;
  int n_tiles;          // column tiles of the packed table
};

__device__ __forceinline__ int e32_chunk(int row, int lane) { return lane ^ (row & 8); }

__device__ __forceinline__ void gemm_dma(uint8_t* stage, const uint8_t* __restrict__ pimg, const EOperand& eo,
                                         int kb, int col0, const uint32_t (&voff)[2], const uint32_t (&poff)[2],
                                         int wave) {
  const __amdgpu_buffer_rsrc_t ra = rsrc(pimg + (size_t)kb * kPImg, kPImg);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint8_t* dst = stage + (32 * wave + 16 * j) * kImgRow;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)dst, 16, poff[j], 0, 0, 0);
    const int row = 2 * wave + j;                       // id row of the k-block
    const int id = kb * kKB + row;
    const uint32_t valid = (id < eo.vocab && col0 < eo.d) ? (uint32_t)(eo.d - col0) * 4u : 0u;
    const __amdgpu_buffer_rsrc_t rb =
        rsrc(eo.base + ((size_t)min(id, eo.vocab - 1) * eo.d + col0) * 4, valid < 1024u ? valid : 1024u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(dst + kArr), 16, voff[j], 0, 0, 0);
  }
}

// kOdd: the step is an odd one of its split, whose k-block is odd (splits
// start at even k-blocks).  Past a split's last k-block the clamped block may
// have the other parity; such stages are never read.  Waves 4-7 return at once.
constexpr int kDma16 = 8;              // LDS DMA instructions per step of each of waves 0-3
template <bool kOdd>
__device__ __forceinline__ void gemm_dma16(uint8_t* stage, const uint8_t* __restrict__ pimg, const EOperand& eo,
                                           int kb, int col0, const uint32_t (&voff)[2][4],
                                           const uint32_t (&poff)[4], int wave) {
  if (wave >= 4) return;
  const __amdgpu_buffer_rsrc_t ra = rsrc(pimg + (size_t)kb * kPImg, kPImg);
  const __amdgpu_buffer_rsrc_t rb = rsrc(eo.base + ((size_t)(kb >> 1) * eo.n_tiles + col0 / kGN) * kEBlock, kEBlock);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint8_t* dst = stage + (64 * wave + 16 * j) * kImgRow;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)dst, 16, poff[j], 0, 0, 0);
    // E with the non-temporal policy (the nt bit of the cache-policy
    // argument): each line of the table is used once, while the p images
    // stay in L2 for the split's other column tiles
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(dst + kArr), 16, voff[kOdd ? 1 : 0][j], 0, 0, 2);
  }
}

struct Frags {
  bf16x8 ah[4], al[4], bh[2], bl[2];
};

__device__ __forceinline__ void gemm_frags(Frags& f, const uint8_t* stage, int wm, int wn, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = 128 * wm + 32 * i + (lane & 31);
    f.ah[i] = *reinterpret_cast<const bf16x8*>(stage + swz_off(ra, h));
    f.al[i] = *reinterpret_cast<const bf16x8*>(stage + swz_off(ra, 2 + h));
  }
  // The lane's two column fragments are the adjacent columns 64 wn + 2 c and
  // + 1 (c = lane % 32; the epilogue maps them back), so one 8-byte read per
  // id row serves both.  Ids 8h .. 8h + 7 come from their float32 rows and are
  // split into bf16 hi / lo pairs.
  const int cb = 64 * wn + 2 * (lane & 31);
  float x0[8], x1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = 8 * h + e;
    const f32x2 v = *reinterpret_cast<const f32x2*>(stage + kArr + row * 1024 + (e32_chunk(row, cb >> 2) << 4) +
                                                    (cb & 3) * 4);
    x0[e] = v[0];
    x1[e] = v[1];
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(x0[2 * e], x0[2 * e + 1], hi[e], lo[e]);
  f.bh[0] = __builtin_bit_cast(bf16x8, (u32x4){hi[0], hi[1], hi[2], hi[3]});
  f.bl[0] = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(x1[2 * e], x1[2 * e + 1], hi[e], lo[e]);
  f.bh[1] = __builtin_bit_cast(bf16x8, (u32x4){hi[0], hi[1], hi[2], hi[3]});
  f.bl[1] = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], lo[2], lo[3]});
}

// acc[mb][nb] += A(rows 128*wm + 32*mb ..) x B(cols 64*wn + 32*nb ..) for one 16-id k step.
__device__ __forceinline__ void gemm_mma(const Frags& f, f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[mb], f.bh[nb], acc[mb][nb], 0, 0, 0);
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[mb], f.bl[nb], acc[mb][nb], 0, 0, 0);
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.al[mb], f.bh[nb], acc[mb][nb], 0, 0, 0);
    }
}

// fp16 + fp6 operands.  The fp16 fragments of one k step are the first two
// chunks of the slots (ids 8h .. 8h + 7 for lane half h, as in the bf16 case).
// The fp6 corrections of k-blocks s and s + 1 (s even) feed one 32 x 32 x 64
// MFMA per output block: lane half h supplies the 32 codes of k-block s + h
// (six dwords) and their scale, which the MFMA applies to exactly those 32
// products; A and B pair code for code: A = [codes of P'16 | codes of r]
// (record dwords 8-13 of the p slot, scale dword 14, in k-block s + h's
// stage), B = [codes of (Q - Q16) 2^11 | codes of Q16] (the residual chunk
// 2 + h in stage s with its scale byte, and Q16 of k-block s + h converted
// under that scale).
struct Frags16 {
  f16x8 a[4], b[2];
};

__device__ __forceinline__ void gemm_frags16(Frags16& f, const uint8_t* stage, int wm, int wn, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<const f16x8*>(stage + swz_off(128 * wm + 32 * i + (lane & 31), h));
#pragma unroll
  for (int i = 0; i < 2; ++i)
    f.b[i] = *reinterpret_cast<const f16x8*>(stage + kArr + swz_off(64 * wn + 32 * i + (lane & 31), h));
}

// A codes and scale byte of row blocks kMb0 and kMb0 + 1, from this lane's
// stage (k-block s + h): the record's dwords 8-13 (e2m3 codes) and 14 (scale)
template <int kMb0>
__device__ __forceinline__ void gemm_reads6a(i32x8 (&a)[2], int (&sa)[2], const uint8_t* stage_h, int wm, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ra = 128 * wm + 32 * (kMb0 + i) + (lane & 31);
    const u32x4 c2 = *reinterpret_cast<const u32x4*>(stage_h + swz_off(ra, 2));
    const u32x4 c3 = *reinterpret_cast<const u32x4*>(stage_h + swz_off(ra, 3));
    a[i] = (i32x8){(int)c2[0], (int)c2[1], (int)c2[2], (int)c2[3], (int)c3[0], (int)c3[1], 0, 0};
    sa[i] = (int)c3[2];
  }
}

// B: the residual codes and scale of k-block s + h (chunk 2 + h of stage s)
__device__ __forceinline__ void gemm_reads6b(i32x8 (&b)[2], int& sb, const uint8_t* stage_s, int wn, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rb = 64 * wn + 32 * i + (lane & 31);
    const u32x4 qe = *reinterpret_cast<const u32x4*>(stage_s + kArr + swz_off(rb, 2 + h));
    // dwords 3-5 are written by gemm_convert6b; both column blocks lie in one
    // 64-column group and carry the same scale byte
#pragma unroll
    for (int e = 0; e < 3; ++e) b[i][e] = (int)qe[e];
    if (i == 0) sb = (int)qe[3];
  }
}

// The 16 Q16 values of k-block s + h for both column blocks (ids 0-7 in q0,
// 8-15 in q1), from the fp16 B fragments instead of LDS: lane half 0 holds
// chunk 0 (ids 0-7) of steps s (cur) and s + 1 (nxt), half 1 chunk 1 (ids
// 8-15); one swap between the halves (v_permlane32_swap: the upper half of
// its first operand trades places with the lower half of its second) leaves
// every lane both chunks of its own k-block.
struct Raw6 {
  u32x4 q0[2], q1[2];
};

__device__ __forceinline__ void gemm_q16_exchange(Raw6& r, const Frags16& cur, const Frags16& nxt) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 c4 = __builtin_bit_cast(u32x4, cur.b[i]);
    const u32x4 n4 = __builtin_bit_cast(u32x4, nxt.b[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto sw = __builtin_amdgcn_permlane32_swap(c4[e], n4[e], false, false);
      r.q0[i][e] = sw[0];
      r.q1[i][e] = sw[1];
    }
  }
}

// B's second half, the codes of Q16 of both column blocks, in one conversion
// under the group's scale (e2m3 of Q16 / 2^eB, nearest, ties to the even
// code).  kLone: k-block s is the split's last and has no partner, so lane
// half 1 contributes zero.
template <bool kLone>
__device__ __forceinline__ void gemm_convert6b(i32x8 (&b)[2], int sb, const Raw6& r, int lane) {
  const u32x16 w = (u32x16){r.q0[0][0], r.q0[0][1], r.q0[0][2], r.q0[0][3], r.q1[0][0], r.q1[0][1],
                            r.q1[0][2], r.q1[0][3], r.q0[1][0], r.q0[1][1], r.q0[1][2], r.q0[1][3],
                            r.q1[1][0], r.q1[1][1], r.q1[1][2], r.q1[1][3]};
  const u32x6 c = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(__builtin_bit_cast(f16x32, w),
                                                              __uint_as_float((uint32_t)sb << 23));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 3; ++e) b[i][3 + e] = (int)c[3 * i + e];
    if (kLone && lane >= 32) b[i] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void gemm_mma16(const Frags16& f, f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[mb], f.b[nb], acc[mb][nb], 0, 0, 0);
}

// fp6 MFMAs of row blocks kMb0, kMb0 + 1: e2m3 x e2m3 (format selectors 2;
// six dwords of each operand are read), per-lane E8M0 scales from the records
template <int kMb0>
__device__ __forceinline__ void gemm_mma6(const i32x8 (&a)[2], const int (&sa)[2], const i32x8 (&b)[2], int sb,
                                          f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      acc[kMb0 + i][nb] =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[nb], acc[kMb0 + i][nb], 2, 2, 0, sa[i], 0, sb);
}

// The packed-table pipeline keeps five LDS stages and synchronises once per
// pair of steps.  Waves 0-3 move every step (gemm_dma16), one step in each step
// of a pair: at the even step s, after the barrier, step s + 3 (into the stage
// of s - 2), and at the odd step s + 1 step s + 4 (into the stage of s - 1);
// both stages were last read before that barrier.  The even step waits until
// all but the newest step have landed (so s and s + 1 are in LDS) and then
// passes the barrier; a step is read only during its own pair, so its stage
// stays intact while the pair reads it.  The fp6 work of a pair (s, s + 1)
// spreads over both steps:
//   even s:  read the fp16 fragments of step s; fp6 MFMAs of the previous
//            pair's row blocks 2-3 (zeros before the first pair); read this
//            pair's B, the fp16 fragments of step s + 1 and the A codes of
//            row blocks 0-1; fp16 MFMAs of step s; convert B's Q16 half.
//   odd s+1: read the A codes of row blocks 2-3; fp16 MFMAs of step s + 1;
//            fp6 MFMAs of row blocks 0-1.
// Each step issues 12 MFMAs (8 fp16, 4 fp6).  Why waves 0-3 carry all the
// DMA: the hardware gives the older of two waves on a SIMD the matrix core
// first, so waves 0-3 (dispatched first) run ahead of waves 4-7 and reach the
// barrier early; their DMA instructions, which can stall on the CU's memory
// queue, sit where there is that slack, and waves 4-7 issue none.  The two
// groups run the same loop (gemm_loop16) with and without the DMA.
constexpr int kStages16 = 5;
__device__ __forceinline__ uint8_t* stage16(uint8_t* smem, int k) { return smem + (k % kStages16) * kStage; }

struct Ops6 {
  i32x8 a01[2], a23[2], b[2];
  int sa01[2], sa23[2], sb;
};

template <bool kLone, bool kDma>
__device__ __forceinline__ void gemm_even16(int s, uint8_t* smem, Frags16& cur, Frags16& nxt, Ops6& o,
                                            f32x16 (&acc)[4][2], const uint8_t* __restrict__ pimg,
                                            const EOperand& eo, int kb0, int kb_last, int col0,
                                            const uint32_t (&voff)[2][4], const uint32_t (&poff)[4], int wave,
                                            int wm, int wn, int lane) {
  // the MFMAs touch no memory: keep the scheduler from moving them across the
  // workgroup barrier into another iteration
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt_lgkm0<kDma16>();
  raw_barrier();
  __builtin_amdgcn_sched_barrier(0);
  gemm_frags16(cur, stage16(smem, s), wm, wn, lane);
  if constexpr (kDma)
    gemm_dma16<true>(stage16(smem, s + 3), pimg, eo, min(kb0 + s + 3, kb_last), col0, voff, poff, wave);
  gemm_mma6<2>(o.a23, o.sa23, o.b, o.sb, acc);
  // the previous pair's B is consumed before this pair's is read over it
  __builtin_amdgcn_sched_barrier(0);
  // reads in the order they are needed: B's residual codes, the next step's
  // fp16 fragments (first MFMAs of the odd step; with this step's they also
  // give B's Q16 values), the A codes of row blocks 0-1 (last MFMAs of the odd
  // step)
  const int h = lane >> 5;
  gemm_reads6b(o.b, o.sb, stage16(smem, s), wn, lane);
  gemm_frags16(nxt, stage16(smem, s + 1), wm, wn, lane);
  gemm_reads6a<0>(o.a01, o.sa01, stage16(smem, s + h), wm, lane);
  Raw6 raw;
  gemm_q16_exchange(raw, cur, nxt);
  gemm_mma16(cur, acc);
  __builtin_amdgcn_sched_barrier(0);
  gemm_convert6b<kLone>(o.b, o.sb, raw, lane);
}

template <bool kDma>
__device__ __forceinline__ void gemm_odd16(int s1, uint8_t* smem, Frags16& cur, Ops6& o, f32x16 (&acc)[4][2],
                                           const uint8_t* __restrict__ pimg, const EOperand& eo, int kb0,
                                           int kb_last, int col0, const uint32_t (&voff)[2][4],
                                           const uint32_t (&poff)[4], int wave, int wm, int lane) {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kDma)
    gemm_dma16<false>(stage16(smem, s1 + 3), pimg, eo, min(kb0 + s1 + 3, kb_last), col0, voff, poff, wave);
  __builtin_amdgcn_sched_barrier(0);
  // reads first (consumed after the next barrier), then the fp16 MFMAs on
  // fragments read in the even step, then the fp6 ones on the A codes read
  // last there
  gemm_reads6a<2>(o.a23, o.sa23, stage16(smem, s1 - 1 + (lane >> 5)), wm, lane);
  gemm_mma16(cur, acc);
  __builtin_amdgcn_sched_barrier(0);
  gemm_mma6<0>(o.a01, o.sa01, o.b, o.sb, acc);
}

// The whole k loop of one wave.  kDma: waves 0-3, which send the steps.
template <bool kDma>
__device__ __forceinline__ void gemm_loop16(uint8_t* smem, f32x16 (&acc)[4][2], const uint8_t* __restrict__ pimg,
                                            const EOperand& eo, int kb0, int kb_last, int nsteps, int col0,
                                            const uint32_t (&voff)[2][4], const uint32_t (&poff)[4], int wave,
                                            int wm, int wn, int lane) {
  Frags16 ga, gb;
  Ops6 o;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o.a01[i] = o.a23[i] = o.b[i] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
    o.sa01[i] = o.sa23[i] = 127;
  }
  o.sb = 127;
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    gemm_even16<false, kDma>(s, smem, ga, gb, o, acc, pimg, eo, kb0, kb_last, col0, voff, poff, wave, wm, wn, lane);
    gemm_odd16<kDma>(s + 1, smem, gb, o, acc, pimg, eo, kb0, kb_last, col0, voff, poff, wave, wm, lane);
  }
  if (s < nsteps) {
    // the split's last k-block has no partner: its corrections go alone.  Its
    // stage and the next (the clamped repeat) are in LDS by the barrier.
    gemm_even16<true, kDma>(s, smem, ga, gb, o, acc, pimg, eo, kb0, kb_last, col0, voff, poff, wave, wm, wn, lane);
    gemm_reads6a<2>(o.a23, o.sa23, stage16(smem, s + (lane >> 5)), wm, lane);
    gemm_mma6<0>(o.a01, o.sa01, o.b, o.sb, acc);
  }
  gemm_mma6<2>(o.a23, o.sa23, o.b, o.sb, acc);
}

// Iteration s of the pipeline: step s+1 has landed in LDS (waited before the
// barrier), step s+kDist is sent to the stage step s-1 used (kDma), the MFMAs
// consume the fragments of step s (read during iteration s-1) while the
// fragments of step s+1 are read (kFrags).  kAhead = number of DMA steps
// issued beyond s+1 at the wait.  Every variant is straight-line code, so the
// compiler's wait-count tracking stays exact across the unrolled iterations.
template <int kAhead, bool kDma, bool kFrags>
__device__ __forceinline__ void gemm_iter(int s, uint8_t* smem, Frags& cur, Frags& nxt,
                                          f32x16 (&acc)[4][2], const uint8_t* __restrict__ pimg,
                                          const EOperand& eo, int kb0, int kb_last, int col0,
                                          const uint32_t (&voff)[2], const uint32_t (&poff)[2],
                                          int wave, int wm, int wn, int lane) {
  // the fragments of step s were read an iteration ago: drain them here, before
  // this iteration's reads are queued behind them
  wait_vmcnt_lgkm0<kDmaPerStep * kAhead>();
  raw_barrier();
  // past the split's last k-block the DMA repeats that block into a stage that
  // is never read again, so every iteration runs the same code
  if (kDma)
    gemm_dma(smem + ((s + kDist) % kStages) * kStage, pimg, eo, min(kb0 + s + kDist, kb_last), col0, voff, poff,
             wave);
  if (kFrags) gemm_frags(nxt, smem + ((s + 1) % kStages) * kStage, wm, wn, lane);
  gemm_mma(cur, acc);
  // issue order: the next step's fragment reads first, then the MFMAs with the
  // LDS DMA instructions spread between them, so a DMA that has to wait for
  // queue space never holds back more than a few MFMAs
  if (kFrags) __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    if (kDma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

template <bool kF32E>
__global__ __launch_bounds__(kGThreads, 1) void samp_gemm(const uint8_t* __restrict__ pimg,
                                                          const uint8_t* __restrict__ eimg,
                                                          float* __restrict__ zp, int n_rows, int d,
                                                          int n_tiles, int n_mt,
                                                          int kb_per_split, int n_kb, int vocab) {
  const EOperand eo{eimg, d, vocab, n_tiles};
  __shared__ __attribute__((aligned(16))) uint8_t smem[(kF32E ? kStages : kStages16) * kStage];

  // Workgroups are dealt round-robin to the 8 XCDs; renumber them so the
  // d-tiles of one vocabulary split sit on the same XCD and share its L2 copy
  // of the p images, and (with several 256-row tiles, i.e. a batch of
  // canvases) the row tiles of one (split, d-tile) run side by side and share
  // its E tiles.
  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int lin = xcd * per + min(xcd, rem) + slot;
  const int mt = lin % n_mt;
  const int tile = (lin / n_mt) % n_tiles;
  const int split = lin / (n_mt * n_tiles);
  pimg += (size_t)mt * n_kb * kPImg;
  const int col0 = tile * kGN;
  const int kb0 = split * kb_per_split;
  const int nsteps = min(n_kb, kb0 + kb_per_split) - kb0;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  // Lane offsets of the 16-byte chunk that belongs at this lane's swizzled LDS
  // slot (p images and packed E tiles are both [row or column][64 B] per
  // k-block in LDS).  Past the split's last k-block the DMA repeats that block
  // into stages that are never read, so every iteration runs the same code.
  const int kb_last = kb0 + nsteps - 1;
  if constexpr (kF32E) {
    uint32_t voff[2], poff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 32 * wave + 16 * j + (lane >> 2);
      const int chunk = (lane & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
      poff[j] = (uint32_t)(row * kImgRow + chunk * 16);
      // id row 2 wave + j, lane's slot holds 16-byte chunk e32_chunk
      voff[j] = (uint32_t)(e32_chunk(2 * wave + j, lane) * 16);
    }
    // prologue: steps 0..kDist-1 in flight (clamped to the last k-block), step
    // 0 landed, its fragments read
    gemm_dma(smem, pimg, eo, min(kb0, kb_last), col0, voff, poff, wave);
    gemm_dma(smem + kStage, pimg, eo, min(kb0 + 1, kb_last), col0, voff, poff, wave);
    gemm_dma(smem + 2 * kStage, pimg, eo, min(kb0 + 2, kb_last), col0, voff, poff, wave);
    static_assert(kDist == 3, "the prologue sends three steps");
    wait_vmcnt<(kDist - 1) * kDmaPerStep>();
    raw_barrier();
    // every iteration sends a DMA step and reads the next step's fragments
    // (the last ones read data that is never used)
    Frags fa, fb;
    gemm_frags(fa, smem, wm, wn, lane);
#define DG_ITER(S, C, N) \
  gemm_iter<1, true, true>(S, smem, C, N, acc, pimg, eo, kb0, kb_last, col0, voff, poff, wave, wm, wn, lane)
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
      DG_ITER(s, fa, fb);
      DG_ITER(s + 1, fb, fa);
    }
    if (s < nsteps) DG_ITER(s, fa, fb);
#undef DG_ITER
  } else {
    // waves 0-3 move whole steps: rows / columns 64 (wave % 4) + 16 j + lane / 4;
    // voff[parity of the k-block][instruction].  A column row takes the Q16
    // chunks of k-block 2j' or 2j' + 1, or the pair's residual chunks (even
    // k-blocks only; odd ones load zeros).
    uint32_t voff[2][4], poff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 64 * (wave & 3) + 16 * j + (lane >> 2);
      const int chunk = (lane & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
      poff[j] = (uint32_t)(row * kImgRow + chunk * 16);
      const uint32_t q16 = (uint32_t)(row * 32 + (chunk & 1) * 16);
      voff[0][j] = chunk < 2 ? q16 : (uint32_t)(kEResid + row * 32 + (chunk - 2) * 16);
      voff[1][j] = chunk < 2 ? (uint32_t)kEHalf + q16 : (1u << 30);
    }
    // prologue: steps 0-2 in flight, 0 and 1 landed
    gemm_dma16<false>(smem, pimg, eo, min(kb0, kb_last), col0, voff, poff, wave);
    gemm_dma16<true>(smem + kStage, pimg, eo, min(kb0 + 1, kb_last), col0, voff, poff, wave);
    gemm_dma16<false>(smem + 2 * kStage, pimg, eo, min(kb0 + 2, kb_last), col0, voff, poff, wave);
    wait_vmcnt<kDma16>();
    raw_barrier();
    if (wave < 4)
      gemm_loop16<true>(smem, acc, pimg, eo, kb0, kb_last, nsteps, col0, voff, poff, wave, wm, wn, lane);
    else
      gemm_loop16<false>(smem, acc, pimg, eo, kb0, kb_last, nsteps, col0, voff, poff, wave, wm, wn, lane);
  }
  wait_vmcnt<0>();

  // epilogue: lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 block, column lane%32
  float* out = zp + (size_t)split * (size_t)n_rows * (size_t)d;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // float32 E: fragment nb holds the columns of parity nb (see gemm_frags)
      const int col = kF32E ? col0 + 64 * wn + 2 * (lane & 31) + nb : col0 + 64 * wn + 32 * nb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = kGM * mt + 128 * wm + 32 * mb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        // non-temporal: the partials leave as they are written instead of
        // in one write-back at the kernel's end
        if (row < n_rows && col < d) __builtin_nontemporal_store(acc[mb][nb][v], out + (size_t)row * d + col);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per row: statistics merge, candidate, confidence, commit / re-noise, z.
// grid (ceil(d / 1024), n_rows); each thread owns 4 columns of z.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void samp_combine(const float* __restrict__ logits,
                                                    const StatsPartial* __restrict__ part,
                                                    int n_splits, const float* __restrict__ zp,
                                                    const dg_ctrl* __restrict__ ctrl,
                                                    int32_t* __restrict__ ids,
                                                    uint8_t* __restrict__ committed,
                                                    float* __restrict__ z, float* __restrict__ conf,
                                                    int n_rows, int n_canvas, int vocab, int d,
                                                    EbRows eb, const PackTail* __restrict__ tail) {
  const int row = blockIdx.y;
  __shared__ float s_w[kMaxSamplerSplits];
  __shared__ uint32_t s_bad;
  const dg_ctrl cb = ctrl[row / n_canvas];
  const float temp = temperature(cb);
  const float inv_t = 1.0f / temp;
  const float c_t = kLog2e * inv_t;
  const StatsPartial* pr = part + (size_t)row * n_splits;
  if (threadIdx.x < kWave) {
    // wave 0 merges the split statistics; lane s takes splits s, s+64, ...
    StatsPartial r{-INFINITY, 0.f, 0.f, 0xFFFFFFFFu, -INFINITY, 0xFFFFFFFFu, 0u, 0.f};
    for (int sp = threadIdx.x; sp < n_splits; sp += kWave) merge_partial(r, pr[sp], c_t);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      StatsPartial q;
      q.m = __shfl_xor(r.m, o); q.s1 = __shfl_xor(r.s1, o); q.st = __shfl_xor(r.st, o);
      q.best_id = __shfl_xor(r.best_id, o); q.gscore = __shfl_xor(r.gscore, o);
      q.gid = __shfl_xor(r.gid, o); q.bad = __shfl_xor(r.bad, o); q.sy = __shfl_xor(r.sy, o);
      merge_partial(r, q, c_t);
    }
    const bool bad = r.bad || !(r.m > -INFINITY);
    // z_s of the fp16 + fp6 contraction is in units of 2^(14 + c)
    const float inv_s1 = (1.0f / r.s1) * (tail ? tail->zscale : 1.0f);
    for (int sp = threadIdx.x; sp < n_splits; sp += kWave)
      s_w[sp] = rescale_factor(pr[sp].m, r.m, kLog2e) * inv_s1;
    if (threadIdx.x == 0) {
      s_bad = bad;
      if (blockIdx.x == 0) {
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
        if (eb.on) {
          // entropy of p_T in nats: ln S_T - (sum e^x x) / S_T, x = (l - m) / T
          const float h = bad ? __builtin_nanf("") : logf(r.st) - r.sy * kLn2 / r.st;
          eb.ent[row] = h;
          if (eb.ent_out) eb.ent_out[row] = h;
          eb.cand[row] = (int32_t)cand;
          eb.argmax[row] = (bad || r.best_id >= (uint32_t)vocab) ? 0 : (int32_t)r.best_id;
        } else if (!committed[row]) {
          const bool last = cb.s_in_block + 1u >= cb.s_max;
          if (!bad && (kappa >= cb.tau || last)) {
            ids[row] = (int32_t)cand;
            committed[row] = 1;
          } else if (!(cb.flags & DG_COMMIT_ONLY)) {
            const Philox4 h = philox4x32_10(0u, (uint32_t)(row % n_canvas), cb.gstep, kStreamRenoise,
                                            seed_lo(cb.seed), seed_hi(cb.seed));
            ids[row] = (int32_t)range_draw(h.w0, (uint32_t)vocab);
          }
        }
      }
    }
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  const int col = blockIdx.x * 1024 + 4 * threadIdx.x;
  if (col >= d) return;
  const size_t stride = (size_t)n_rows * (size_t)d;
  const float* src = zp + (size_t)row * d + col;
  float* dst = z + (size_t)row * d + col;
  if ((d & 3) == 0) {
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < n_splits; ++sp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + sp * stride);
      const float wsp = s_w[sp];
      acc[0] += wsp * v[0]; acc[1] += wsp * v[1]; acc[2] += wsp * v[2]; acc[3] += wsp * v[3];
    }
    if (bad) acc = (f32x4){__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    *reinterpret_cast<f32x4*>(dst) = acc;
  } else {
    for (int e = 0; e < 4 && col + e < d; ++e) {
      float acc = 0.f;
      for (int sp = 0; sp < n_splits; ++sp) acc += s_w[sp] * src[sp * stride + e];
      dst[e] = bad ? __builtin_nanf("") : acc;
    }
  }
}

__global__ __launch_bounds__(256) void samp_finalize(const uint8_t* __restrict__ committed,
                                                     uint32_t* __restrict__ n_unc,
                                                     dg_ctrl* __restrict__ ctrl, int n_canvas) {
  // workgroup b handles canvas b
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int open = (t < n_canvas && !committed[(size_t)b * n_canvas + t]) ? 1 : 0;
  const int count = __syncthreads_count(open);
  if (t == 0) {
    n_unc[b] = (uint32_t)count;
    if (ctrl[b].flags & DG_AUTO_ADVANCE) {
      ctrl[b].gstep += 1u;
      ctrl[b].s_in_block += 1u;
    }
  }
}

// ---------------------------------------------------------------------------
// Entropy-bounded acceptance over the canvas (explainer "DiffusionGemma:
// Google's open diffusion LLM", section "A diffusion language model refines
// 256 tokens in 12 steps"; Table 2): sort the rows by (entropy, position),
// accept while the running sum of entropies stays within the budget (the
// first always), re-noise every other position, and test adaptive stopping
// (mean entropy below the threshold and the greedy ids unchanged since the
// previous step).  One workgroup of 256 threads: ranks by counting, fp64
// prefix sums.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void samp_eb_select(EbRows eb, int32_t* __restrict__ ids,
                                                      uint8_t* __restrict__ accepted,
                                                      int32_t* __restrict__ prev_argmax,
                                                      dg_eb_status* __restrict__ status,
                                                      dg_ctrl* __restrict__ ctrl, float budget,
                                                      float stop_entropy, int n_rows, int vocab) {
  __shared__ float key[256];
  __shared__ int idx[256];   // position at each rank
  __shared__ double csum[256];
  __shared__ uint8_t acc[256];
  const int t = threadIdx.x;
  // workgroup b handles canvas b (rows b * n_rows ..)
  {
    const size_t o = (size_t)blockIdx.x * n_rows;
    eb.ent += o; eb.cand += o; eb.argmax += o;
    ids += o; accepted += o; prev_argmax += o;
    status += blockIdx.x; ctrl += blockIdx.x;
  }
  const dg_ctrl cb = *ctrl;
  const float h = (t < n_rows) ? eb.ent[t] : __builtin_nanf("");
  const bool defined = t < n_rows && !(h != h);
  key[t] = defined ? h : INFINITY;
  acc[t] = 0;
  __syncthreads();
  // rank of (key, position) among all 256 entries: the number of entries that
  // sort before it (undefined rows, key +inf, sort last by position); the
  // sorted order is then written by scattering each entry to its rank
  const float mine = key[t];
  int rank = 0;
#pragma unroll 8
  for (int j = 0; j < 256; ++j) {
    const float kj = key[j];
    rank += (kj < mine) || (kj == mine && j < t);
  }
  __syncthreads();
  key[rank] = mine;
  idx[rank] = t;
  __syncthreads();
  // inclusive prefix sums of the sorted entropies (fp64, Hillis-Steele)
  const int n_def = __syncthreads_count(defined);
  double c = (t < n_def) ? (double)key[t] : 0.0;
  csum[t] = c;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const double add = (t >= o) ? csum[t - o] : 0.0;
    __syncthreads();
    c += add;
    csum[t] = c;
    __syncthreads();
  }
  const bool last = cb.s_in_block + 1u >= cb.s_max;
  if (t < n_def && (t == 0 || last || c <= (double)budget)) acc[idx[t]] = 1;
  // mean entropy over the defined rows (fixed-order reduction: the last prefix sum)
  const double total = csum[255];
  __syncthreads();
  const bool stable = __syncthreads_and(t >= n_rows || eb.argmax[t] == prev_argmax[t]) != 0;
  const float mean_h = (n_def > 0) ? (float)(total / (double)n_def) : __builtin_nanf("");
  const bool stop = n_def > 0 && mean_h < stop_entropy && stable;
  const int n_acc = __syncthreads_count(t < n_rows && acc[t]);
  if (t < n_rows) {
    int32_t id;
    if (stop) {
      id = eb.argmax[t];
    } else if (acc[t]) {
      id = eb.cand[t];
    } else {
      const Philox4 hh = philox4x32_10(0u, (uint32_t)t, cb.gstep, kStreamRenoise, seed_lo(cb.seed),
                                       seed_hi(cb.seed));
      id = (int32_t)range_draw(hh.w0, (uint32_t)vocab);
    }
    ids[t] = id;
    accepted[t] = acc[t];
    prev_argmax[t] = eb.argmax[t];
  }
  if (t == 0) {
    status->n_accepted = (uint32_t)n_acc;
    status->stop = stop ? 1u : 0u;
    status->mean_entropy = mean_h;
    status->n_defined = (uint32_t)n_def;
    if (cb.flags & DG_AUTO_ADVANCE) {
      ctrl->gstep += 1u;
      ctrl->s_in_block += 1u;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k truncated sampler.  The pages expect truncating the sampling step to
// the top k tokens to raise throughput at larger batches (explainer
// "DiffusionGemma: Google's open diffusion LLM", section "Throughput flips at
// about 32 concurrent users").  Per row the kept set S is the k largest
// logits, ties to the smaller id; the step is then the full one on logits
// with everything outside S at -inf, so the contraction shrinks to k rows of
// E per canvas row.
//   topk_slice   per (4096-id sub-slice, row), one wavefront each: a floor
//                that every member of the sub-slice's top k reaches, the keys
//                at or above it compacted into LDS, and a radix select over
//                those order-preserving keys (then by id among equal keys);
//                NaN / +inf flags.  topk_slice_rest redoes the rare
//                sub-slices where too many keys reach the floor.
//   topk_row     per row: the top k of the sub-slices' candidates (floor,
//                compaction, workgroup-wide select), then one split's
//                statistics record (max, argmax, Gumbel argmax within S, sums
//                at T = 1 and T, entropy term) and the weights exp(l - m) of S.
//   topk_z       z_0 = sum over S of exp(l - m) E[id] from the fp32 table.
//   samp_combine, samp_finalize / samp_eb_select as in the full sampler, with
//                one split.
// ---------------------------------------------------------------------------
constexpr int kTkThreads = 256;
constexpr int kTkRowPer = 64;                          // candidates per thread in the row pass

struct TopkItem {
  float v;       // logit (slice candidates) or weight exp(l - m) (row list)
  int32_t id;
};

// Larger float, larger key (NaN above +inf).
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct TkShared {
  uint32_t hist[256];
  uint32_t wsum[kTkThreads / kWave];
  uint32_t res[3];
};

// Inclusive prefix sum over the workgroup (one value per thread).
__device__ __forceinline__ uint32_t wg_scan(uint32_t x, TkShared& sh) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wsum[w] = x;
  __syncthreads();
  for (int i = 0; i < w; ++i) x += sh.wsum[i];
  __syncthreads();
  return x;
}

// The kk-th largest key (1-based) among the workgroup's active elements, by
// four 8-bit histogram passes from the top byte.  Returns tau, the number of
// active keys above it (gt) and equal to it (eq).  Needs kk <= number active.
template <int E, typename KeyF, typename ActF>
__device__ void wg_select(KeyF keyf, ActF act, uint32_t kk, TkShared& sh, uint32_t& tau, uint32_t& gt,
                          uint32_t& eq) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  gt = 0;
  eq = 0;
  // passes stay a loop: unrolled, the element loops inside would multiply the code size
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    sh.hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = keyf(e);
      if (act(e) && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t takes bin 255 - t, so its inclusive scan counts the keys in bins >= 255 - t
    const uint32_t h = sh.hist[255 - t];
    const uint32_t incl = wg_scan(h, sh);
    if (incl - h < kk && incl >= kk) {   // exactly one thread
      sh.res[0] = 255u - (uint32_t)t;
      sh.res[1] = incl - h;
      sh.res[2] = h;
    }
    __syncthreads();
    prefix |= sh.res[0] << shift;
    pmask |= 0xFFu << shift;
    kk -= sh.res[1];
    gt += sh.res[1];
    eq = sh.res[2];
    __syncthreads();
  }
  tau = prefix;
}

// Cut of the k largest active elements, ties to the smaller id: element e is
// kept iff key > tau, or key == tau and ~id >= tau2.
struct TopkCut {
  uint32_t tau, tau2;
};

template <int E, typename KeyF, typename IdF, typename ActF>
__device__ TopkCut wg_topk_cut(KeyF keyf, IdF idf, ActF act, uint32_t k, TkShared& sh) {
  TopkCut c{0u, 0u};
  uint32_t gt, eq;
  wg_select<E>(keyf, act, k, sh, c.tau, gt, eq);
  const uint32_t need = k - gt;   // equal keys to keep, 1 .. eq (uniform)
  if (need < eq) {
    uint32_t g2, e2;
    const uint32_t tau = c.tau;
    wg_select<E>([&](int e) { return ~idf(e); }, [&](int e) { return act(e) && keyf(e) == tau; }, need, sh,
                 c.tau2, g2, e2);
  }
  return c;
}

// A lower bound for the k largest keys (k <= the workgroup size): the k-th
// largest of the per-thread maxima.  At least k elements reach it, so the
// k-th largest key overall does too, and every element of the top k (ties
// included) has key >= the bound; only those need to enter the select.
template <int E, typename KeyF, typename ActF>
__device__ uint32_t wg_topk_floor(KeyF keyf, ActF act, uint32_t k, TkShared& sh) {
  uint32_t tmax = 0u;
  bool any = false;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (act(e)) { tmax = max(tmax, keyf(e)); any = true; }
  uint32_t n_any = wg_scan(any ? 1u : 0u, sh);
  // the last thread's inclusive count is the number of threads holding an element
  if (threadIdx.x == kTkThreads - 1) sh.res[0] = n_any;
  __syncthreads();
  n_any = sh.res[0];
  __syncthreads();
  if (n_any < k) return 0u;   // fewer holders than k: no cut
  uint32_t f, g, e;
  wg_select<1>([&](int) { return tmax; }, [&](int) { return any; }, k, sh, f, g, e);
  return f;
}

// ---- wave-level select (no workgroup barriers): one wavefront, 64 lanes,
// E elements per lane, a private 256-bin LDS histogram.  LDS instructions of
// one wave execute in order, so clearing, counting and reading the histogram
// need no barrier.

// Inclusive prefix sum over the wave.
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

template <int E, typename KeyF, typename ActF>
__device__ void wave_select(KeyF keyf, ActF act, uint32_t kk, uint32_t* hist, uint32_t& tau, uint32_t& gt,
                            uint32_t& eq) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  gt = 0;
  eq = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    *reinterpret_cast<u32x4*>(hist + 4 * lane) = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = keyf(e);
      if (act(e) && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    // lane L reads bins 255 - 4L .. 252 - 4L (descending), so the running sums
    // count the keys in higher bins
    const u32x4 hv = *reinterpret_cast<const u32x4*>(hist + 252 - 4 * lane);
    const uint32_t h[4] = {hv[3], hv[2], hv[1], hv[0]};
    const uint32_t tot = h[0] + h[1] + h[2] + h[3];
    uint32_t run = wave_scan(tot) - tot;
    uint32_t b = 0, above = 0, cnt = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!found && run < kk && run + h[j] >= kk) {
        found = true;
        b = 255u - 4u * (uint32_t)lane - (uint32_t)j;
        above = run;
        cnt = h[j];
      }
      run += h[j];
    }
    const uint64_t who = __builtin_amdgcn_ballot_w64(found);
    const int src = who ? (int)__builtin_ctzll(who) : 0;   // exactly one lane holds the bin
    b = __shfl(b, src);
    above = __shfl(above, src);
    cnt = __shfl(cnt, src);
    prefix |= b << shift;
    pmask |= 0xFFu << shift;
    kk -= above;
    gt += above;
    eq = cnt;
  }
  tau = prefix;
}

template <int E, typename KeyF, typename IdF, typename ActF>
__device__ TopkCut wave_topk_cut(KeyF keyf, IdF idf, ActF act, uint32_t k, uint32_t* hist) {
  TopkCut c{0u, 0u};
  uint32_t gt, eq;
  wave_select<E>(keyf, act, k, hist, c.tau, gt, eq);
  const uint32_t need = k - gt;   // equal keys to keep, 1 .. eq (uniform)
  if (need < eq) {
    uint32_t g2, e2;
    const uint32_t tau = c.tau;
    wave_select<E>([&](int e) { return ~idf(e); }, [&](int e) { return act(e) && keyf(e) == tau; }, need, hist,
                   c.tau2, g2, e2);
  }
  return c;
}

// Per-lane R largest keys (sorted, descending) of E keys.
template <int R, int E, typename KeyF>
__device__ __forceinline__ void lane_top(KeyF keyf, uint32_t (&top)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) top[r] = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t x = keyf(e);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t hi = max(top[r], x);
      x = min(top[r], x);
      top[r] = hi;
    }
  }
}

// Top k (k <= 256) of 4096-id sub-slices: grid (ceil(n_sub / 4), n_rows), one
// sub-slice per wavefront.  Lane L holds the 4-id groups c = 0..15 starting at
// id base + 4 (64 c + L) (each load instruction reads 1 KB of consecutive
// logits).  The floor: the k-th largest of the lanes' top-R lists (R = k / 64
// rounded up) is reached by at least k elements, so every member of the top k
// reaches it and only those enter the radix select.
constexpr int kTkWaveIds = 4096;
constexpr int kTkWaveChunks = kTkWaveIds / (4 * kWave);   // 16

// Per-wave LDS: the radix histogram and the compacted candidates.
constexpr int kTkCap = 1024;   // candidates above the floor kept in LDS (fast path)
struct TkWave {
  uint32_t hist[256];
  uint32_t ckey[kTkCap];
  uint32_t cid[kTkCap];
};

// Marker left in a sub-slice's first candidate when more than kTkCap keys reach
// the floor (many equal or near-equal logits); topk_slice_rest redoes those.
constexpr int32_t kTkOverflow = -2;

template <bool kAligned>
__device__ __forceinline__ void topk_load_keys(const float* __restrict__ x, int vocab, int base,
                                               uint32_t (&key)[4 * kTkWaveChunks], int& bad) {
  const int lane = threadIdx.x & 63;
  bad = 0;
#pragma unroll
  for (int c = 0; c < kTkWaveChunks; ++c) {
    const f32x4 v = load4<kAligned>(x, base + 4 * (kWave * c + lane), vocab);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bad |= (v[e] != v[e]) | (v[e] == INFINITY);
      key[4 * c + e] = order_key(v[e]);
    }
  }
}

template <int R>
__device__ __forceinline__ uint32_t topk_floor(const uint32_t (&key)[4 * kTkWaveChunks], int k, uint32_t* hist) {
  uint32_t top[R];
  lane_top<R, 4 * kTkWaveChunks>([&](int e) { return key[e]; }, top);
  uint32_t fl, g0, e0;
  wave_select<R>([&](int r) { return top[r]; }, [](int) { return true; }, (uint32_t)k, hist, fl, g0, e0);
  return fl;
}

// Fast path: the keys above the floor (lanes in order, each lane's in id
// order) go to LDS and the exact select runs on those alone.
template <bool kAligned, int R>
__device__ __forceinline__ void topk_wave_fast(const float* __restrict__ x, TopkItem* __restrict__ out,
                                               uint8_t* __restrict__ badp, int vocab, int base, int k,
                                               TkWave& L) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4 * kTkWaveChunks];
  int bad;
  topk_load_keys<kAligned>(x, vocab, base, key, bad);
  const bool any_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if (lane == 0) *badp = any_bad ? 1 : 0;
  auto idf = [&](int e) { return (uint32_t)(base + 4 * (kWave * (e >> 2) + lane) + (e & 3)); };
  const uint32_t fl = topk_floor<R>(key, k, L.hist);
  uint32_t n_act = 0;
#pragma unroll
  for (int e = 0; e < 4 * kTkWaveChunks; ++e) n_act += key[e] >= fl ? 1u : 0u;
  const uint32_t act_incl = wave_scan(n_act);
  const uint32_t total = __shfl(act_incl, 63);
  if (total > (uint32_t)kTkCap) {
    if (lane == 0) out[0] = TopkItem{0.f, kTkOverflow};
    return;
  }
  uint32_t off = act_incl - n_act;
#pragma unroll
  for (int e = 0; e < 4 * kTkWaveChunks; ++e)
    if (key[e] >= fl) { L.ckey[off] = key[e]; L.cid[off] = idf(e); ++off; }
  constexpr int kPer = kTkCap / kWave;
  uint32_t ck[kPer], ci[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t i = (uint32_t)(lane + kWave * j);
    ck[j] = i < total ? L.ckey[i] : 0u;
    ci[j] = i < total ? L.cid[i] : 0xFFFFFFFFu;
  }
  auto cact = [&](int j) { return (uint32_t)(lane + kWave * j) < total; };
  const TopkCut cut = wave_topk_cut<kPer>([&](int j) { return ck[j]; }, [&](int j) { return ci[j]; }, cact,
                                          (uint32_t)k, L.hist);
  auto kept = [&](int j) { return cact(j) && (ck[j] > cut.tau || (ck[j] == cut.tau && ~ci[j] >= cut.tau2)); };
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) cnt += kept(j) ? 1u : 0u;
  uint32_t o = wave_scan(cnt) - cnt;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (kept(j) && o < (uint32_t)k) out[o++] = TopkItem{key_value(ck[j]), (int32_t)ci[j]};
}

// Overflowed sub-slices: the select over all 4096 register-held keys.
template <bool kAligned, int R>
__device__ __forceinline__ void topk_wave_full(const float* __restrict__ x, TopkItem* __restrict__ out, int vocab,
                                               int base, int k, TkWave& L) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4 * kTkWaveChunks];
  int bad;
  topk_load_keys<kAligned>(x, vocab, base, key, bad);
  auto keyf = [&](int e) { return key[e]; };
  auto idf = [&](int e) { return (uint32_t)(base + 4 * (kWave * (e >> 2) + lane) + (e & 3)); };
  const uint32_t fl = topk_floor<R>(key, k, L.hist);
  auto act = [&](int e) { return key[e] >= fl; };
  const TopkCut cut = wave_topk_cut<4 * kTkWaveChunks>(keyf, idf, act, (uint32_t)k, L.hist);
  auto kept = [&](int e) { return key[e] > cut.tau || (key[e] == cut.tau && ~idf(e) >= cut.tau2); };
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < 4 * kTkWaveChunks; ++e) cnt += kept(e) ? 1u : 0u;
  uint32_t o = wave_scan(cnt) - cnt;
#pragma unroll
  for (int e = 0; e < 4 * kTkWaveChunks; ++e)
    if (kept(e) && o < (uint32_t)k) out[o++] = TopkItem{key_value(key[e]), (int32_t)idf(e)};
}

// R = k / 64 rounded up: the length of the per-lane lists behind the floor.
// grid (ceil(n_sub / 4), n_rows), one 4096-id sub-slice per wavefront.
template <bool kAligned, int R>
__global__ __launch_bounds__(kTkThreads) void topk_slice(const float* __restrict__ logits,
                                                         TopkItem* __restrict__ cand,
                                                         uint8_t* __restrict__ badf, int vocab, int n_sub,
                                                         int k) {
  __shared__ __attribute__((aligned(16))) TkWave lds_w[kTkThreads / kWave];
  const int w = threadIdx.x >> 6;
  const int sub = blockIdx.x * (kTkThreads / kWave) + w;
  const int row = blockIdx.y;
  if (sub >= n_sub) return;   // whole wavefront; no workgroup barrier follows
  topk_wave_fast<kAligned, R>(logits + (size_t)row * (size_t)vocab, cand + ((size_t)row * n_sub + sub) * k,
                              badf + (size_t)row * n_sub + sub, vocab, sub * kTkWaveIds, k, lds_w[w]);
}

// Same grid; only the sub-slices marked kTkOverflow do any work.
template <bool kAligned, int R>
__global__ __launch_bounds__(kTkThreads) void topk_slice_rest(const float* __restrict__ logits,
                                                              TopkItem* __restrict__ cand, int vocab, int n_sub,
                                                              int k) {
  __shared__ __attribute__((aligned(16))) TkWave lds_w[kTkThreads / kWave];
  const int w = threadIdx.x >> 6;
  const int sub = blockIdx.x * (kTkThreads / kWave) + w;
  const int row = blockIdx.y;
  if (sub >= n_sub) return;
  TopkItem* out = cand + ((size_t)row * n_sub + sub) * k;
  if (out[0].id != kTkOverflow) return;   // uniform over the wavefront
  topk_wave_full<kAligned, R>(logits + (size_t)row * (size_t)vocab, out, vocab, sub * kTkWaveIds, k, lds_w[w]);
}

template <bool kAligned, int R>
static void launch_topk_slice_r(const TopkPlan& p, const float* logits, TopkItem* cand, uint8_t* badf,
                                hipStream_t s) {
  const dim3 grid((p.n_slices + 3) / 4, p.n);
  topk_slice<kAligned, R><<<grid, kTkThreads, 0, s>>>(logits, cand, badf, p.vocab, p.n_slices, p.k);
  topk_slice_rest<kAligned, R><<<grid, kTkThreads, 0, s>>>(logits, cand, p.vocab, p.n_slices, p.k);
}

template <bool kAligned>
static void launch_topk_slice(const TopkPlan& p, const float* logits, TopkItem* cand, uint8_t* badf,
                              hipStream_t s) {
  if (p.k <= 64) launch_topk_slice_r<kAligned, 1>(p, logits, cand, badf, s);
  else if (p.k <= 128) launch_topk_slice_r<kAligned, 2>(p, logits, cand, badf, s);
  else if (p.k <= 192) launch_topk_slice_r<kAligned, 3>(p, logits, cand, badf, s);
  else launch_topk_slice_r<kAligned, 4>(p, logits, cand, badf, s);
}

constexpr int kTkRowCap = 2048;   // candidates above the floor compacted into LDS (fast path)

__global__ __launch_bounds__(kTkThreads) void topk_row(const TopkItem* __restrict__ cand,
                                                       const uint8_t* __restrict__ badf,
                                                       const dg_ctrl* __restrict__ ctrl,
                                                       StatsPartial* __restrict__ part,
                                                       TopkItem* __restrict__ list, int n_slices, int k,
                                                       int n_canvas, bool want_h) {
  __shared__ TkShared sh;
  __shared__ StatsPartial red[kTkThreads / kWave];
  __shared__ uint32_t ckey[kTkRowCap], cid[kTkRowCap];
  __shared__ uint32_t sel_key[256], sel_id[256];
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int count = n_slices * k;
  const TopkItem* src = cand + (size_t)row * count;
  uint32_t key[kTkRowPer], idv[kTkRowPer];
#pragma unroll
  for (int e = 0; e < kTkRowPer; ++e) {
    const int i = t + kTkThreads * e;
    if (i < count) {
      const TopkItem it = src[i];
      key[e] = order_key(it.v);
      idv[e] = (uint32_t)it.id;
    } else {
      key[e] = 0u;
      idv[e] = 0xFFFFFFFFu;
    }
  }
  auto held = [&](int e) { return t + kTkThreads * e < count; };
  auto keyf = [&](int e) { return key[e]; };
  auto idf = [&](int e) { return idv[e]; };
  const uint32_t floor_key = wg_topk_floor<kTkRowPer>(keyf, held, (uint32_t)k, sh);
  uint32_t n_act = 0;
#pragma unroll
  for (int e = 0; e < kTkRowPer; ++e) n_act += (held(e) && key[e] >= floor_key) ? 1u : 0u;
  const uint32_t act_incl = wg_scan(n_act, sh);
  if (t == kTkThreads - 1) sh.res[0] = act_incl;
  __syncthreads();
  const uint32_t total = sh.res[0];
  __syncthreads();
  // the k kept items, in a fixed order, into sel_key / sel_id
  if (total <= (uint32_t)kTkRowCap) {
    uint32_t off = act_incl - n_act;
#pragma unroll
    for (int e = 0; e < kTkRowPer; ++e)
      if (held(e) && key[e] >= floor_key) { ckey[off] = key[e]; cid[off] = idv[e]; ++off; }
    __syncthreads();
    constexpr int kPer = kTkRowCap / kTkThreads;   // 8
    uint32_t ck[kPer], ci[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)(t + kTkThreads * j);
      ck[j] = i < total ? ckey[i] : 0u;
      ci[j] = i < total ? cid[i] : 0xFFFFFFFFu;
    }
    auto cact = [&](int j) { return (uint32_t)(t + kTkThreads * j) < total; };
    const TopkCut cut = wg_topk_cut<kPer>([&](int j) { return ck[j]; }, [&](int j) { return ci[j]; }, cact,
                                          (uint32_t)k, sh);
    auto kept = [&](int j) { return cact(j) && (ck[j] > cut.tau || (ck[j] == cut.tau && ~ci[j] >= cut.tau2)); };
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) cnt += kept(j) ? 1u : 0u;
    uint32_t o = wg_scan(cnt, sh) - cnt;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (kept(j) && o < (uint32_t)k) { sel_key[o] = ck[j]; sel_id[o] = ci[j]; ++o; }
  } else {
    auto act = [&](int e) { return held(e) && key[e] >= floor_key; };
    const TopkCut cut = wg_topk_cut<kTkRowPer>(keyf, idf, act, (uint32_t)k, sh);
    auto kept = [&](int e) {
      return act(e) && (key[e] > cut.tau || (key[e] == cut.tau && ~idv[e] >= cut.tau2));
    };
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < kTkRowPer; ++e) cnt += kept(e) ? 1u : 0u;
    uint32_t o = wg_scan(cnt, sh) - cnt;
#pragma unroll
    for (int e = 0; e < kTkRowPer; ++e)
      if (kept(e) && o < (uint32_t)k) { sel_key[o] = key[e]; sel_id[o] = idv[e]; ++o; }
  }
  __syncthreads();

  // statistics over S, one kept item per thread (t < k)
  const dg_ctrl cb = ctrl[row / n_canvas];
  const uint32_t pos = (uint32_t)(row % n_canvas);
  const float temp = temperature(cb);
  const float inv_t = 1.0f / temp;
  const bool tempered = inv_t != 1.0f;
  const bool gumbel = (cb.flags & DG_GUMBEL) != 0;
  const float c_t = kLog2e * inv_t;
  const uint32_t k0 = seed_lo(cb.seed), k1 = seed_hi(cb.seed);
  const bool mine = t < k;
  const float v = mine ? key_value(sel_key[t]) : -INFINITY;
  const uint32_t id = mine ? sel_id[t] : 0xFFFFFFFFu;

  float m = v, gbest = -INFINITY;
  uint32_t bid = id, gid = 0xFFFFFFFFu;
  if (gumbel && mine) {
    const Philox4 h = philox4x32_10(id >> 2, pos, cb.gstep, kStreamGumbel, k0, k1);
    const uint32_t word = (id & 3u) == 0 ? h.w0 : (id & 3u) == 1 ? h.w1 : (id & 3u) == 2 ? h.w2 : h.w3;
    gbest = v * inv_t + gumbel_from_bits(word);
    gid = id;
  }
  wave_argmax(m, bid);
  wave_argmax(gbest, gid);
  if (lane == 0) red[w] = StatsPartial{m, 0.f, 0.f, bid, gbest, gid, 0u, 0.f};
  uint32_t bad = 0;
  for (int i = t; i < n_slices; i += kTkThreads) bad |= badf[(size_t)row * n_slices + i];
  bad = __syncthreads_or((int)bad) ? 1u : 0u;
  {
    StatsPartial acc = red[0];
#pragma unroll
    for (int o = 1; o < kTkThreads / kWave; ++o) {
      const StatsPartial q = red[o];
      if (better(q.m, q.best_id, acc.m, acc.best_id)) { acc.m = q.m; acc.best_id = q.best_id; }
      if (better(q.gscore, q.gid, acc.gscore, acc.gid)) { acc.gscore = q.gscore; acc.gid = q.gid; }
    }
    m = acc.m; bid = acc.best_id; gbest = acc.gscore; gid = acc.gid;
  }

  // weights exp(l - m) over S, their sums, and the row's list
  const float mc = (m == -INFINITY) ? 0.0f : -m * kLog2e;
  float s1 = 0.f, st = 0.f, sy = 0.f;
  if (mine) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(v, kLog2e, mc));
    s1 = p;
    if (tempered || want_h) {
      const float y = fmaxf((v - m) * c_t, -200.f);
      const float et = tempered ? __builtin_amdgcn_exp2f(y) : p;
      st = et;
      if (want_h) sy = et * y;
    } else {
      st = p;
    }
    list[(size_t)row * k + t] = TopkItem{p, (int32_t)id};
  }
  s1 = wave_sum(s1);
  st = wave_sum(st);
  sy = wave_sum(sy);
  __syncthreads();   // red is reused
  if (lane == 0) { red[w].s1 = s1; red[w].st = st; red[w].sy = sy; }
  __syncthreads();
  if (t == 0) {
    float a1 = 0.f, at = 0.f, ay = 0.f;
#pragma unroll
    for (int o = 0; o < kTkThreads / kWave; ++o) { a1 += red[o].s1; at += red[o].st; ay += red[o].sy; }
    part[row] = StatsPartial{m, a1, at, bid, gbest, gid, bad, ay};
  }
}

// z_0[row] = sum over the row's list of weight * E[id]; grid (ceil(d / 1024), n_rows),
// each thread 4 columns.  Ids past the vocabulary count with weight 0.
__global__ __launch_bounds__(256) void topk_z(const TopkItem* __restrict__ list, const float* __restrict__ emb,
                                              float* __restrict__ zp, int k, int vocab, int d) {
  const int row = blockIdx.y;
  const int col = blockIdx.x * 1024 + 4 * threadIdx.x;
  if (col >= d) return;
  const TopkItem* L = list + (size_t)row * k;
  float* dst = zp + (size_t)row * d + col;
  if ((d & 3) == 0) {
    // branch-free, so the loads of several ids are in flight together; ids past
    // the vocabulary (the fill of short rows) read row 0 with weight 0
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int i = 0; i < k; ++i) {
      const TopkItem it = L[i];
      const bool ok = it.id < vocab;
      const float wgt = ok ? it.v : 0.f;
      const f32x4 v = *reinterpret_cast<const f32x4*>(emb + (size_t)(ok ? it.id : 0) * d + col);
      acc[0] += wgt * v[0]; acc[1] += wgt * v[1]; acc[2] += wgt * v[2]; acc[3] += wgt * v[3];
    }
    *reinterpret_cast<f32x4*>(dst) = acc;
  } else {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < k; ++i) {
      const TopkItem it = L[i];
      if (it.id >= vocab) continue;
      const float* e = emb + (size_t)it.id * d + col;
      for (int q = 0; q < 4 && col + q < d; ++q) acc[q] += it.v * e[q];
    }
    for (int q = 0; q < 4 && col + q < d; ++q) dst[q] = acc[q];
  }
}

// ---------------------------------------------------------------------------
static size_t embedding_image_bytes(int vocab, int d) {
  const size_t n_pairs = ((size_t)(vocab + kKB - 1) / kKB + 1) / 2;
  const size_t n_tiles = (size_t)(d + kGN - 1) / kGN;
  return n_pairs * n_tiles * kEBlock;
}

// one row-shift byte per id of the padded vocabulary (whole k-block pairs), 256-byte aligned
static size_t shift_bytes(int vocab) {
  const size_t n_pairs = ((size_t)(vocab + kKB - 1) / kKB + 1) / 2;
  return align_up(n_pairs * 2 * kKB, 256);
}

size_t embedding_packed_bytes(int vocab, int d) {
  return embedding_image_bytes(vocab, d) + shift_bytes(vocab) + kAmaxParts * sizeof(float) + kPackTailBytes;
}

static const uint8_t* pack_shifts(const void* packed, int vocab, int d) {
  return static_cast<const uint8_t*>(packed) + embedding_image_bytes(vocab, d);
}

static const PackTail* pack_tail(const void* packed, int vocab, int d) {
  return reinterpret_cast<const PackTail*>(pack_shifts(packed, vocab, d) + shift_bytes(vocab) +
                                           kAmaxParts * sizeof(float));
}

hipError_t launch_embedding_pack(const float* emb, void* packed, int vocab, int d, hipStream_t s) {
  const int n_pairs = ((vocab + kKB - 1) / kKB + 1) / 2;
  const int n_tiles = (d + kGN - 1) / kGN;
  uint8_t* base = static_cast<uint8_t*>(packed);
  uint8_t* shifts = base + embedding_image_bytes(vocab, d);
  float* part = reinterpret_cast<float*>(shifts + shift_bytes(vocab));
  PackTail* tail = const_cast<PackTail*>(pack_tail(packed, vocab, d));
  prof_begin("emb_pack", s);
  emb_amax_kernel<<<kAmaxParts, 256, 0, s>>>(emb, (size_t)vocab * (size_t)d, part);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    emb_scale_kernel<<<1, 256, 0, s>>>(part, tail);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    const int n_ids = (int)shift_bytes(vocab);
    emb_shift_kernel<<<n_ids / 4, 256, 0, s>>>(emb, vocab, d, n_ids, tail, shifts);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    emb_pack_kernel<<<dim3(2 * n_pairs, n_tiles), 256, 0, s>>>(emb, base, vocab, d, n_tiles, tail, shifts);
    e = hipGetLastError();
  }
  prof_end(s);
  return e;
}

SamplerPlan sampler_plan(int n_canvas, int batch, int vocab, int d) {
  SamplerPlan p{};
  const int n = n_canvas * batch;
  p.n = n; p.n_canvas = n_canvas; p.batch = batch; p.vocab = vocab; p.d = d;
  p.n_mt = (n + kGM - 1) / kGM;
  p.n_kb = (vocab + kKB - 1) / kKB;
  p.n_tiles = (d + kGN - 1) / kGN;
  p.col_pad = p.n_tiles * kGN;
  int splits = 256 / (p.n_tiles * p.n_mt);
  if (splits < 1) splits = 1;
  const int by_len = (p.n_kb + 15) / 16;     // at least 16 k-blocks per split
  if (splits > by_len) splits = by_len;
  // the statistics pass holds a split's logits of one row in 256 lanes x 4 k-blocks
  const int by_regs = (p.n_kb + kMaxKbPerSplit - 1) / kMaxKbPerSplit;
  if (splits < by_regs) splits = by_regs;
  if (splits < 1) splits = 1;
  p.kb_per_split = (p.n_kb + splits - 1) / splits;
  // an even count: the contraction takes k-blocks in pairs from an even start
  p.kb_per_split += p.kb_per_split & 1;
  p.n_splits = (p.n_kb + p.kb_per_split - 1) / p.kb_per_split;
  p.off_stats = 0;
  p.off_pimg = align_up((size_t)n * p.n_splits * sizeof(StatsPartial), 256);
  p.off_zp = p.off_pimg + align_up((size_t)p.n_mt * p.n_kb * kPImg, 256);
  p.off_eb = p.off_zp + align_up((size_t)p.n_splits * n * d * sizeof(float), 256);
  p.total = p.off_eb + 3 * align_up((size_t)n * 4, 256);
  return p;
}

hipError_t launch_sampler(const SamplerPlan& p, const float* logits, const void* emb_packed,
                          int32_t* ids, uint8_t* committed, float* z, float* conf,
                          uint32_t* n_unc, dg_ctrl* ctrl, void* ws, hipStream_t s,
                          const EbCall& eb) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t eb_arr = align_up((size_t)p.n * 4, 256);
  EbRows rows{eb.on, reinterpret_cast<float*>(base + p.off_eb),
              reinterpret_cast<int32_t*>(base + p.off_eb + eb_arr),
              reinterpret_cast<int32_t*>(base + p.off_eb + 2 * eb_arr), eb.entropy_out};
  StatsPartial* part = reinterpret_cast<StatsPartial*>(base + p.off_stats);
  uint8_t* pimg = base + p.off_pimg;
  float* zp = reinterpret_cast<float*>(base + p.off_zp);
  const bool aligned = (p.vocab % 4) == 0;

  const uint8_t* shifts = eb.emb_f32 ? nullptr : pack_shifts(emb_packed, p.vocab, p.d);
  prof_begin("samp_stats", s);
  const dim3 sgrid(p.n_splits, (p.n + kStatsRows - 1) / kStatsRows);
#define DG_STATS(A, F)                                                                                  \
  samp_stats<A, F><<<sgrid, kStatsThreadsWG, 0, s>>>(logits, ctrl, part, pimg, shifts, p.n, p.n_canvas, \
                                                     p.vocab, p.kb_per_split, p.n_kb, eb.on)
  if (eb.emb_f32) {
    if (aligned) DG_STATS(true, false);
    else DG_STATS(false, false);
  } else {
    if (aligned) DG_STATS(true, true);
    else DG_STATS(false, true);
  }
#undef DG_STATS
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  prof_begin("samp_gemm", s);
  if (eb.emb_f32)
    samp_gemm<true><<<p.n_mt * p.n_tiles * p.n_splits, kGThreads, 0, s>>>(
        pimg, static_cast<const uint8_t*>(emb_packed), zp, p.n, p.d, p.n_tiles, p.n_mt,
        p.kb_per_split, p.n_kb, p.vocab);
  else
    samp_gemm<false><<<p.n_mt * p.n_tiles * p.n_splits, kGThreads, 0, s>>>(
        pimg, static_cast<const uint8_t*>(emb_packed), zp, p.n, p.d, p.n_tiles, p.n_mt,
        p.kb_per_split, p.n_kb, p.vocab);
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  prof_begin("samp_combine", s);
  samp_combine<<<dim3((p.d + 1023) / 1024, p.n), 256, 0, s>>>(
      logits, part, p.n_splits, zp, ctrl, ids, committed, z, conf, p.n, p.n_canvas, p.vocab, p.d, rows,
      eb.emb_f32 ? nullptr : pack_tail(emb_packed, p.vocab, p.d));
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (eb.on) {
    prof_begin("samp_eb_select", s);
    samp_eb_select<<<p.batch, 256, 0, s>>>(rows, ids, committed, eb.argmax, eb.status, ctrl, eb.budget,
                                           eb.stop_entropy, p.n_canvas, p.vocab);
    prof_end(s);
    return hipGetLastError();
  }
  prof_begin("samp_finalize", s);
  samp_finalize<<<p.batch, 256, 0, s>>>(committed, n_unc, ctrl, p.n_canvas);
  prof_end(s);
  return hipGetLastError();
}

TopkPlan topk_plan(int n_canvas, int batch, int vocab, int d, int k) {
  TopkPlan p{};
  p.n = n_canvas * batch; p.n_canvas = n_canvas; p.batch = batch; p.vocab = vocab; p.d = d; p.k = k;
  p.n_slices = (vocab + kTkWaveIds - 1) / kTkWaveIds;
  p.max_candidates = kTkThreads * kTkRowPer;
  p.off_part = 0;
  p.off_cand = align_up((size_t)p.n * sizeof(StatsPartial), 256);
  p.off_bad = p.off_cand + align_up((size_t)p.n * p.n_slices * k * sizeof(TopkItem), 256);
  p.off_list = p.off_bad + align_up((size_t)p.n * p.n_slices, 256);
  p.off_zp = p.off_list + align_up((size_t)p.n * k * sizeof(TopkItem), 256);
  p.off_eb = p.off_zp + align_up((size_t)p.n * d * sizeof(float), 256);
  p.total = p.off_eb + 3 * align_up((size_t)p.n * 4, 256);
  return p;
}

hipError_t launch_sampler_topk(const TopkPlan& p, const float* logits, const float* emb, int32_t* ids,
                               uint8_t* committed, float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl,
                               void* ws, hipStream_t s, const EbCall& eb) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t eb_arr = align_up((size_t)p.n * 4, 256);
  EbRows rows{eb.on, reinterpret_cast<float*>(base + p.off_eb),
              reinterpret_cast<int32_t*>(base + p.off_eb + eb_arr),
              reinterpret_cast<int32_t*>(base + p.off_eb + 2 * eb_arr), eb.entropy_out};
  StatsPartial* part = reinterpret_cast<StatsPartial*>(base + p.off_part);
  TopkItem* cand = reinterpret_cast<TopkItem*>(base + p.off_cand);
  uint8_t* badf = base + p.off_bad;
  TopkItem* list = reinterpret_cast<TopkItem*>(base + p.off_list);
  float* zp = reinterpret_cast<float*>(base + p.off_zp);

  prof_begin("topk_slice", s);
  if (p.vocab % 4 == 0)
    launch_topk_slice<true>(p, logits, cand, badf, s);
  else
    launch_topk_slice<false>(p, logits, cand, badf, s);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin("topk_row", s);
  topk_row<<<p.n, kTkThreads, 0, s>>>(cand, badf, ctrl, part, list, p.n_slices, p.k, p.n_canvas, eb.on);
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin("topk_z", s);
  topk_z<<<dim3((p.d + 1023) / 1024, p.n), 256, 0, s>>>(list, emb, zp, p.k, p.vocab, p.d);
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin("samp_combine", s);
  samp_combine<<<dim3((p.d + 1023) / 1024, p.n), 256, 0, s>>>(logits, part, 1, zp, ctrl, ids, committed, z, conf,
                                                              p.n, p.n_canvas, p.vocab, p.d, rows, nullptr);
  prof_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (eb.on) {
    prof_begin("samp_eb_select", s);
    samp_eb_select<<<p.batch, 256, 0, s>>>(rows, ids, committed, eb.argmax, eb.status, ctrl, eb.budget,
                                           eb.stop_entropy, p.n_canvas, p.vocab);
    prof_end(s);
    return hipGetLastError();
  }
  prof_begin("samp_finalize", s);
  samp_finalize<<<p.batch, 256, 0, s>>>(committed, n_unc, ctrl, p.n_canvas);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace dg
