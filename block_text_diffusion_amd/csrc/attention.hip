// Bidirectional canvas attention on gfx950 (DiffusionGemma Technical Report
// part 4/6, section 6 "Attention" and section 9.1: every canvas position attends
// to the committed KV-cache history and to all canvas positions, no mask).
//
// Work split.  The key sequence [prefix ; canvas] is cut into 64-key blocks
// that never straddle the prefix/canvas boundary; a workgroup takes one KV
// head, 128 packed query rows (canvas position x query head of the group, so
// the heads sharing a KV head share every K/V block) and a run of consecutive
// blocks (a chunk).  Chunks are merged by a log-sum-exp combine kernel; the
// partial outputs travel as fp16 scaled by the row's largest magnitude.
//
// Inside a workgroup.  Eight wavefronts: wave w owns query rows 32(w%4)..+31
// and keys 32(w/4)..+31 of every block, with its own running max and sum; the
// two key halves are merged through LDS at the end.  K and V blocks go to a
// double-buffered LDS stage through registers (each block's loads are issued
// two blocks ahead of its use), both kept as [key][d] rows with xor-swizzled
// 16-byte chunks.  Scores are formed
// transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16 (a lane holds 16 keys
// of one query, so the row softmax needs one cross-lane exchange) and feed
// O^T = V^T P^T straight from the score registers; the V^T operand comes from
// ds_read_b64_tr_b16, which transposes 16-bit elements across 16 lanes, so V
// needs no transposition pass.  Online softmax in fp32, base 2.
//
// FP8 (E4M3) inputs: K stays FP8 in LDS and the scores run on the FP8 matrix
// cores (v_mfma_f32_32x32x64_f8f6f4, four times the depth of a bf16 step at
// twice the rate); V is converted exactly to bf16 when staged and P.V stays on
// bf16 (P rounded to bf16, as for bf16 inputs).
#include <type_traits>

#include "dg_common.hpp"
#include "dg_internal.hpp"

namespace dg {

constexpr int kAWaves = 8;
constexpr int kAThreads = 64 * kAWaves;
constexpr int kARows = 128;   // packed query rows per workgroup
constexpr int kAKeys = 64;    // keys per block

template <int D>
struct AGeom {
  static constexpr int kRowBytes = D * 2;                       // one bf16 key row
  static constexpr int kCpr = D / 8;                            // 16-byte chunks per row
  static constexpr int kBlockBytes = kAKeys * kRowBytes;
  static constexpr int kStageBytes = 2 * kBlockBytes;           // K then V
  static_assert(kCpr * kAKeys % kAThreads == 0, "block does not split evenly over the threads");
};

// LDS stage of one block: K (bf16 rows, or raw FP8 rows of D bytes when the
// scores run on the FP8 matrix cores), then V (bf16 rows).
template <int D, bool kF8>
struct AStage {
  static constexpr int kKRowBytes = kF8 ? D : 2 * D;
  static constexpr int kKBytes = kAKeys * kKRowBytes;
  static constexpr int kVOffset = kKBytes;
  static constexpr int kBytes = kKBytes + AGeom<D>::kBlockBytes;
};

// FP8 K rows (D bytes): 16-byte chunk c of key k sits at slot c ^ f(k).  A
// 16-lane pass of a score-fragment read takes one chunk column over 16
// consecutive keys; with rows of 128 (64) bytes, key bits 0 (0-1) pick the half
// (quarter) of a 256-byte line and f supplies the other bits, so the 16 pieces
// land on 16 different slots.
template <int D>
__device__ __forceinline__ int k8_slot(int key, int c) {
  if constexpr (D == 128) return c ^ ((key >> 1) & 7);
  else return c ^ ((key >> 2) & 3);
}

// K rows: chunk c of key k sits at slot c ^ f(k); a wave's 16-byte reads of one
// chunk column over 32 consecutive keys spread over all banks.
template <int D>
__device__ __forceinline__ int k_slot(int key, int c) {
  if constexpr (D == 128) return c ^ (key & 15);
  else return c ^ ((key ^ (key >> 3)) & 7);
}
// V rows: a 16-lane group of a transposing read takes four consecutive keys
// (k & 3 = 0..3) in two adjacent chunks, and the two groups of a half-wave take
// the same keys in the next two chunks.  For D = 128 the map sends the sixteen
// 16-byte pieces of a half-wave to sixteen different slots (distinct modulo 8
// within each group), so the reads are free of bank conflicts whether the LDS
// serves 16 or 32 lanes of 8-byte reads per cycle.
template <int D>
__device__ __forceinline__ int v_slot(int key, int c) {
  if constexpr (D == 128) return c ^ ((4 * (key & 3)) ^ (2 * ((key ^ (key >> 1)) & 1)));
  else return c ^ (((key & 3) << 1) | ((key >> 2) & 1));
}

// Eight consecutive elements as eight bf16 (packed in 4 u32).
__device__ __forceinline__ u32x4 load8(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return (u32x4){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                 pack_bf16x2(b[2], b[3])};
}

// Eight OCP FP8 E4M3 values (8 bytes in two u32) as eight bf16: every E4M3
// value is exactly a bf16 value, so the conversion is exact.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  return (u32x4){pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                 pack_bf16x2(d[0], d[1])};
}
__device__ __forceinline__ u32x4 load8(const uint8_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return fp8x8_to_bf16(w[0], w[1]);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
}

// One block of K and V (one KV head, keys kb0.. of one segment) in flight in
// registers: each thread carries kPer 8-element chunks of K and of V, as bf16
// (16 bytes) or, with kF8, as the raw FP8 bytes (8 bytes, converted to bf16
// when stored to LDS, so the loads stay in flight across the block's math).
// Keys past the segment end are clamped to its last key (finite data, masked
// later).
template <int D, bool kF8>
struct KvRegs {
  static constexpr int kPer = AGeom<D>::kCpr * kAKeys / kAThreads;
  using Raw = std::conditional_t<kF8, u32x2, u32x4>;
  Raw k[kPer], v[kPer];
};

template <int D, bool kF8>
__device__ __forceinline__ void kv_fetch(KvRegs<D, kF8>& r, __amdgpu_buffer_rsrc_t rk,
                                         __amdgpu_buffer_rsrc_t rv, int kb0, int seg_len,
                                         int hkv, int kvh, int t) {
  using G = AGeom<D>;
  constexpr uint32_t kElemBytes = kF8 ? 1u : 2u;
#pragma unroll
  for (int i = 0; i < KvRegs<D, kF8>::kPer; ++i) {
    const int idx = t + kAThreads * i;
    const int key = min(kb0 + idx / G::kCpr, seg_len - 1);
    const uint32_t off = ((uint32_t)(key * hkv + kvh) * D + (uint32_t)(idx % G::kCpr) * 8u) * kElemBytes;
    if constexpr (kF8) {
      r.k[i] = __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, 0);
      r.v[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0);
    } else {
      r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  }
}

template <int D, bool kF8>
__device__ __forceinline__ void kv_store(const KvRegs<D, kF8>& r, uint8_t* stage, int t) {
  using G = AGeom<D>;
  using S = AStage<D, kF8>;
#pragma unroll
  for (int i = 0; i < KvRegs<D, kF8>::kPer; ++i) {
    const int idx = t + kAThreads * i;
    const int key = idx / G::kCpr, c = idx % G::kCpr;   // c: 8-element chunk of the row
    u32x4 vw;
    if constexpr (kF8) {
      // K stays FP8 for the FP8 matrix cores: 8 bytes into half of a 16-byte slot
      *reinterpret_cast<u32x2*>(stage + key * S::kKRowBytes + (k8_slot<D>(key, c >> 1) << 4) + 8 * (c & 1)) =
          r.k[i];
      vw = fp8x8_to_bf16(r.v[i][0], r.v[i][1]);
    } else {
      *reinterpret_cast<u32x4*>(stage + key * G::kRowBytes + (k_slot<D>(key, c) << 4)) = r.k[i];
      vw = r.v[i];
    }
    *reinterpret_cast<u32x4*>(stage + S::kVOffset + key * G::kRowBytes + (v_slot<D>(key, c) << 4)) = vw;
  }
}

// TQ: query element type (bf16 bits, float, or FP8 bytes); kF8: K/V are FP8
// bytes (otherwise bf16).  out_scale multiplies the normalised output (the V
// scale of FP8 inputs, 1 otherwise).  kBatch: more than one sequence; without
// it the sequence index is the constant 0, so a single sequence pays nothing
// for the per-sequence lookups.
template <int D, typename TQ, bool kF8, bool kBatch>
__global__ __launch_bounds__(kAThreads) void attn_partial(
    const TQ* __restrict__ q, const void* __restrict__ kp, const void* __restrict__ vp,
    const void* __restrict__ kc, const void* __restrict__ vc, float* __restrict__ out,
    _Float16* __restrict__ opart, float* __restrict__ ml, const AttnSeqs seqs, int n, int hq, int hkv,
    int blocks_per_chunk, int n_chunks, float scale_log2e, float out_scale) {
  using G = AGeom<D>;
  using S = AStage<D, kF8>;
  constexpr int KS = D / 16;   // 16-wide k steps over the head dimension (bf16 scores)
  constexpr int KS8 = D / 64;  // 64-wide k steps (FP8 scores)
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  // two stages, and the key-half merge of the epilogue (64 KB at D = 128)
  constexpr int kLdsBytes = 2 * G::kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  static_assert(2 * S::kBytes <= kLdsBytes, "stages exceed the LDS array");
  static_assert(4 * 4 * DB * 64 * 16 <= kLdsBytes, "key-half merge exceeds the LDS array");
  __shared__ float lds_ml[4][64][2];

  // Workgroups are dealt round-robin to the 8 XCDs; renumber them so that the
  // chunks of one (query tile, KV head) pair run on one XCD, which shares that
  // head's K/V blocks in its L2 (measured ~4% faster than chunk-major order).
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  const int bid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int xcd = bid & 7, xslot = bid >> 3;
  const int lin = xcd * (nwg >> 3) + min(xcd, nwg & 7) + xslot;
  const int chunk = lin % gridDim.x;
  const int qtile = (lin / gridDim.x) % gridDim.y;
  const int zi = lin / (gridDim.x * gridDim.y);   // sequence-major, then KV head
  const int seq = kBatch ? zi / hkv : 0;
  const int kvh = kBatch ? zi - seq * hkv : zi;
  const int n_prefix = seqs.n_prefix[seq];
  const bool causal = (seqs.causal >> seq) & 1u;
  const int blocks_prefix = (n_prefix + kAKeys - 1) / kAKeys;
  const int blocks_total = blocks_prefix + (n + kAKeys - 1) / kAKeys;
  const size_t rows_all = (size_t)seqs.batch * n * hq;   // output rows of the launch
  const int group = hq / hkv;
  const int rows = n * group;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wr = wave & 3;      // query row group
  const int wh = wave >> 2;     // key half of every block
  const int half = lane >> 5;

  const int gb0 = chunk * blocks_per_chunk;
  // a chunk past the end of a shorter sequence's keys is empty: it writes
  // m = -inf, l = 0 and a zero partial, which the merge weights by 0
  const int nb = max(0, min(blocks_total, gb0 + blocks_per_chunk) - gb0);

  constexpr size_t kEl = kF8 ? 1 : 2;
  const size_t pre_off = (size_t)seq * seqs.prefix_stride * hkv * D * kEl;
  const size_t can_off = (size_t)seq * n * hkv * D * kEl;
  const uint32_t pre_bytes = (uint32_t)((size_t)n_prefix * hkv * D * kEl);
  const uint32_t can_bytes = (uint32_t)((size_t)n * hkv * D * kEl);
  const __amdgpu_buffer_rsrc_t rkp = rsrc(static_cast<const uint8_t*>(kp) + pre_off, pre_bytes);
  const __amdgpu_buffer_rsrc_t rvp = rsrc(static_cast<const uint8_t*>(vp) + pre_off, pre_bytes);
  const __amdgpu_buffer_rsrc_t rkc = rsrc(static_cast<const uint8_t*>(kc) + can_off, can_bytes);
  const __amdgpu_buffer_rsrc_t rvc = rsrc(static_cast<const uint8_t*>(vc) + can_off, can_bytes);

  KvRegs<D, kF8> ra;
  auto fetch = [&](KvRegs<D, kF8>& r, int b) {
    const int gb = gb0 + b;
    if (gb < blocks_prefix)
      kv_fetch<D, kF8>(r, rkp, rvp, gb * kAKeys, n_prefix, hkv, kvh, t);
    else
      kv_fetch<D, kF8>(r, rkc, rvc, (gb - blocks_prefix) * kAKeys, n, hkv, kvh, t);
  };
  if (nb > 0) fetch(ra, 0);

  // this lane's query row (a column of S^T)
  const int r = qtile * kARows + wr * 32 + (lane & 31);
  const bool r_ok = r < rows;
  const int qn = r_ok ? r / group : 0;
  const int qh = kvh * group + (r_ok ? r % group : 0);
  // bf16 scores: lane half h holds elements 16 ks + 8 h .. +7 of its query row
  // in k step ks.  FP8 scores: 32 bytes, elements 64 ks + 32 h .. +31 (the FP8
  // matrix-core operands pair the same register bytes of the K and Q lanes, so
  // the K fragments below take the same elements of their key rows).
  bf16x8 qf[KS];
  i32x8 qf8[KS8];
  const size_t qrow = (((size_t)seq * n + qn) * hq + qh) * D;
  if constexpr (kF8) {
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      u32x4 lo = (u32x4){0u, 0u, 0u, 0u}, hi = lo;
      if (r_ok) {
        lo = *reinterpret_cast<const u32x4*>(q + qrow + 64 * ks + 32 * half);
        hi = *reinterpret_cast<const u32x4*>(q + qrow + 64 * ks + 32 * half + 16);
      }
      qf8[ks] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = (u32x4){0u, 0u, 0u, 0u};
      if (r_ok) w = load8(q + qrow + 16 * ks + 8 * half);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane LDS offsets that do not change from block to block
  const int kkey = 32 * wh + (lane & 31);             // K fragment row
  const int g16 = lane >> 4, r16 = lane & 15;          // transposing-read group / lane in group
  const int vkey0 = 32 * wh + 4 * (g16 >> 1) + (r16 >> 2);
  const int vbyte = 8 * (r16 & 1);

  if (nb > 0) kv_store<D, kF8>(ra, lds, t);
  // blocks 1 and 2 in flight before the loop: every block's loads are issued
  // two blocks ahead of their use
  KvRegs<D, kF8> rb;
  if (nb > 1) fetch(rb, 1);
  if (nb > 2) fetch(ra, 2);
  __syncthreads();

  // ---- one block in three phases: scores (matrix cores), online softmax
  // (vector ALU), O^T update (matrix cores) ----
  // scores of block b from its LDS stage: this wave's 32 keys of the block,
  // masked past the segment end (and after the row under the causal flag)
  auto scores = [&](int b, const uint8_t* ks_lds, float (&s)[16]) {
    const int gb = gb0 + b;
    const int seg_left = (gb < blocks_prefix) ? n_prefix - gb * kAKeys
                                              : n - (gb - blocks_prefix) * kAKeys;
    // S^T = K Q^T: two accumulators, even / odd k steps
    f32x16 sa, sb;
#pragma unroll
    for (int v = 0; v < 16; ++v) { sa[v] = 0.f; sb[v] = 0.f; }
    if constexpr (kF8) {
      // E4M3 x E4M3 on the FP8 matrix cores (products exact in fp32); format
      // selectors 0 = E4M3 for both operands, no block scales
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const int c0 = 4 * ks + 2 * half;   // 16-byte chunks c0, c0 + 1 of the key row
        const u32x4 lo = *reinterpret_cast<const u32x4*>(ks_lds + kkey * S::kKRowBytes + (k8_slot<D>(kkey, c0) << 4));
        const u32x4 hi =
            *reinterpret_cast<const u32x4*>(ks_lds + kkey * S::kKRowBytes + (k8_slot<D>(kkey, c0 + 1) << 4));
        const i32x8 kf = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        if (ks & 1)
          sb = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf8[ks], sb, 0, 0, 0, 0, 0, 0);
        else
          sa = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf8[ks], sa, 0, 0, 0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ks += 2) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(
            ks_lds + kkey * G::kRowBytes + (k_slot<D>(kkey, 2 * ks + half) << 4));
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(
            ks_lds + kkey * G::kRowBytes + (k_slot<D>(kkey, 2 * ks + 2 + half) << 4));
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[ks + 1], sb, 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = sa[v] + sb[v];
    // lane holds keys 32wh + 8(v/4) + 4half + v%4 of query r; with the causal
    // flag canvas key c is visible to canvas row qn only when c <= qn
    const bool canvas_blk = gb >= blocks_prefix;
    if (seg_left < kAKeys || (causal && canvas_blk)) {
      const int lim = (causal && canvas_blk) ? min(seg_left, qn - (gb - blocks_prefix) * kAKeys + 1)
                                             : seg_left;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 32 * wh + 8 * (v >> 2) + 4 * half + (v & 3);
        if (key >= lim) s[v] = -INFINITY;
      }
    }
  };

  // online softmax of one block's scores (raw score units; exp2 folds in the
  // scale): updates the running max / sum, rescales O when the reference
  // moves, and returns P as bf16 operands
  auto softmax = [&](const float (&s)[16], bf16x8 (&pf)[2]) {
    float mloc = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mloc = fmaxf(mloc, s[v]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // The exponent reference m_run moves only when a lane's block max exceeds
    // it by more than 8 (base 2): p then stays below 2^8, and the rescale of O
    // and l (exact, the shift cancels in O / l) runs a few times per chunk
    // instead of at almost every block.
    if (__builtin_amdgcn_ballot_w64((mloc - m_run) * scale_log2e > 8.0f)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2e);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : -m_run * scale_log2e;
    float lsum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float p[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * tt + v], scale_log2e, mc));
        lsum += p[v];
      }
      const u32x4 w = (u32x4){pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                              pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      pf[tt] = __builtin_bit_cast(bf16x8, w);
    }
    lsum += __shfl_xor(lsum, 32);
    l_run += lsum;
  };

  // O^T += V^T P^T from a block's LDS stage: 16-key steps; lane half h
  // supplies keys 16tt+4h+{0..3}, 16tt+8+4h+{0..3}
  auto pv = [&](const uint8_t* st, const bf16x8 (&pf)[2]) {
    const uint8_t* vs_lds = st + S::kVOffset;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d0 = 32 * db + 16 * (g16 & 1) + 4 * (r16 & 3);
        const int ka = vkey0 + 16 * tt, kb = ka + 8;
        const s16x4 lo = lds_read_tr16(vs_lds + ka * G::kRowBytes + (v_slot<D>(ka, d0 >> 3) << 4) + vbyte);
        const s16x4 hi = lds_read_tr16(vs_lds + kb * G::kRowBytes + (v_slot<D>(kb, d0 >> 3) << 4) + vbyte);
        const u32x2 lw = __builtin_bit_cast(u32x2, lo);
        const u32x2 hw = __builtin_bit_cast(u32x2, hi);
        const bf16x8 vfr = __builtin_bit_cast(bf16x8, (u32x4){lw[0], lw[1], hw[0], hw[1]});
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr, pf[tt], acc_o[db], 0, 0, 0);
      }
    }
  };

  // Two LDS stages; two register sets.  Iteration b multiplies block b,
  // stores block b + 1 (loaded during the two previous iterations) into the
  // other stage, and sends the loads of block b + 3 into the freed registers.
  // rn holds block b + 1: rb for even b, ra for odd b.
  auto iter = [&](int b, KvRegs<D, kF8>& rn) {
    const uint8_t* st = lds + (b & 1) * S::kBytes;
    float s[16];
    bf16x8 pf[2];
    scores(b, st, s);
    softmax(s, pf);
    pv(st, pf);
    if (b + 1 < nb) kv_store<D, kF8>(rn, lds + ((b + 1) & 1) * S::kBytes, t);
    if (b + 3 < nb) fetch(rn, b + 3);
    __syncthreads();
  };
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    iter(b, rb);
    iter(b + 1, ra);
  }
  if (b < nb) iter(b, rb);

  // ---- merge the two key halves: waves 4-7 hand (m, l, O) to waves 0-3 ----
  f32x4* xo = reinterpret_cast<f32x4*>(lds);   // [row group][16 DB-chunks][64 lanes]
  if (wh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        xo[(wr * 4 * DB + 4 * db + g) * 64 + lane] =
            (f32x4){acc_o[db][4 * g], acc_o[db][4 * g + 1], acc_o[db][4 * g + 2], acc_o[db][4 * g + 3]};
    lds_ml[wr][lane][0] = m_run;
    lds_ml[wr][lane][1] = l_run;
  }
  __syncthreads();
  const size_t orow = ((size_t)seq * n + qn) * hq + qh;
  float rmax = 0.f;
  if (wh == 0) {
    const float m2 = lds_ml[wr][lane][0];
    const float l2 = lds_ml[wr][lane][1];
    const float m = fmaxf(m_run, m2);
    const float a1 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m) * scale_log2e);
    const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m2 - m) * scale_log2e);
    l_run = l_run * a1 + l2 * a2;
    m_run = m;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o2 = xo[(wr * 4 * DB + 4 * db + g) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc_o[db][4 * g + e] * a1 + o2[e] * a2;
          acc_o[db][4 * g + e] = v;
          rmax = fmaxf(rmax, fabsf(v));
        }
      }
    if (n_chunks == 1) {
      // one chunk: the normalized output, straight from the registers
      if (r_ok) {
        const float inv = out_scale / l_run;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dd = 32 * db + 8 * g + 4 * half;
            *reinterpret_cast<f32x4*>(out + orow * D + dd) =
                (f32x4){acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv,
                        acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv};
          }
      }
      return;
    }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));   // the row's other half of d
  }
  if (n_chunks == 1) return;
  __syncthreads();   // every xo slot has been read

  // ---- partial output: fp16 values O / s with s = max_d |O| of the row, plus
  // (m, l, s) per row.  The tile is staged row-major in LDS and written out as
  // contiguous rows. ----
  constexpr int kTileRow = D * 2 + 16;   // padded fp16 row
  uint8_t* tile = lds;
  if (wh == 0) {
    const float inv_s = (rmax > 0.f) ? 1.0f / rmax : 0.f;
    const int i = wr * 32 + (lane & 31);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * half;
        const f16x4 hv = (f16x4){(_Float16)(acc_o[db][4 * g] * inv_s), (_Float16)(acc_o[db][4 * g + 1] * inv_s),
                                 (_Float16)(acc_o[db][4 * g + 2] * inv_s), (_Float16)(acc_o[db][4 * g + 3] * inv_s)};
        *reinterpret_cast<f16x4*>(tile + i * kTileRow + dd * 2) = hv;
      }
    if (half == 0 && r_ok)
      *reinterpret_cast<f32x4*>(ml + ((size_t)chunk * rows_all + orow) * 4) =
          (f32x4){m_run * scale_log2e, l_run, rmax, 0.f};
  }
  __syncthreads();
  constexpr int kCpr16 = D * 2 / 16;                 // 16-byte pieces per fp16 row
  _Float16* base = reinterpret_cast<_Float16*>(opart) + (size_t)chunk * rows_all * D;
#pragma unroll
  for (int k = 0; k < (kARows * kCpr16 + kAThreads - 1) / kAThreads; ++k) {
    const int idx = t + kAThreads * k;
    const int i = idx / kCpr16, c = idx % kCpr16;
    const int rr = qtile * kARows + i;
    if (i >= kARows || rr >= rows) continue;
    const size_t row_o = ((size_t)seq * n + rr / group) * hq + kvh * group + rr % group;
    // non-temporal: the partials leave as they are written instead of in one
    // cache flush at the end of the kernel (measured ~1 us off this kernel,
    // ~0.4 us onto the combine that reads them)
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tile + i * kTileRow + 16 * c),
                                reinterpret_cast<u32x4*>(base + row_o * D + 8 * c));
  }
}

// Merge key chunks: O = sum_c 2^(m_c - M) s_c h_c / sum_c 2^(m_c - M) l_c, with
// m in base-2 units and h_c the fp16 partial scaled by 1 / s_c.  D/4 lanes per
// output row, four dims each; a running merge, so no separate max pass, and
// the loads of different chunks do not depend on each other.
constexpr int kCThreads = 256;

template <int D>
__global__ __launch_bounds__(kCThreads) void attn_combine(const _Float16* __restrict__ opart,
                                                          const float* __restrict__ ml,
                                                          float* __restrict__ out,
                                                          int n_rows_total, int n_chunks, float out_scale) {
  constexpr int kLanesPerRow = D / 4;
  const int row = blockIdx.x * (kCThreads / kLanesPerRow) + threadIdx.x / kLanesPerRow;
  const int d4 = (threadIdx.x % kLanesPerRow) * 4;
  if (row >= n_rows_total) return;
  float m = -INFINITY, l = 0.f;
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int c = 0; c < n_chunks; ++c) {
    const size_t idx = (size_t)c * n_rows_total + row;
    const f32x4 rec = *reinterpret_cast<const f32x4*>(ml + idx * 4);
    const f16x4 h = *reinterpret_cast<const f16x4*>(opart + idx * D + d4);
    // a chunk whose keys were all masked for this row (causal) has m = -inf, l = 0
    // and weight 0
    const float mn = fmaxf(m, rec[0]);
    const float a = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float bw = (rec[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(rec[0] - mn);
    const float sw = bw * rec[2];
    acc = acc * a + (f32x4){(float)h[0] * sw, (float)h[1] * sw, (float)h[2] * sw, (float)h[3] * sw};
    l = l * a + rec[1] * bw;
    m = mn;
  }
  *reinterpret_cast<f32x4*>(out + (size_t)row * D + d4) = acc * (out_scale / l);
}

// fp32 K/V are rounded to bf16 once per call (the MFMA operand type).
__global__ __launch_bounds__(256) void attn_to_bf16(const float* __restrict__ src,
                                                    uint16_t* __restrict__ dst, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) *reinterpret_cast<u32x4*>(dst + 8 * i) = load8(src + 8 * i);
}

AttnPlan attn_plan(int n, int n_prefix, int hq, int hkv, int d, int batch) {
  AttnPlan p{};
  p.batch = batch;
  p.n = n; p.n_prefix = n_prefix; p.hq = hq; p.hkv = hkv; p.d = d;
  p.group = hq / hkv;
  p.rows = n * p.group;
  p.n_qtiles = (p.rows + kARows - 1) / kARows;
  p.blocks_prefix = (n_prefix + kAKeys - 1) / kAKeys;
  p.blocks_total = p.blocks_prefix + (n + kAKeys - 1) / kAKeys;
  // about one workgroup per CU: enough chunks to fill 256 CUs, no more (every
  // extra chunk adds a partial output to write and merge)
  const int base = hkv * p.n_qtiles * batch;
  int want = 256 / base;
  if (want > p.blocks_total) want = p.blocks_total;
  if (want < 1) want = 1;
  p.blocks_per_chunk = (p.blocks_total + want - 1) / want;
  p.n_chunks = (p.blocks_total + p.blocks_per_chunk - 1) / p.blocks_per_chunk;
  // workspace: [bf16 copies of fp32 K/V][fp16 partial O][(m, l, s, -) per row]
  const size_t kv_elems = (size_t)batch * (n_prefix + n) * hkv * d;
  p.off_kv16 = 0;
  p.kv16_bytes = align_up(2 * kv_elems * sizeof(uint16_t), 256);
  p.off_opart = p.kv16_bytes;
  if (p.n_chunks > 1) {
    p.off_ml = p.off_opart + align_up((size_t)p.n_chunks * batch * n * hq * d * sizeof(uint16_t), 256);
    p.total = p.off_ml + align_up((size_t)p.n_chunks * batch * n * hq * 4 * sizeof(float), 256);
  } else {
    p.off_ml = p.off_opart;
    p.total = p.off_opart;
  }
  return p;
}

template <int D, typename TQ, bool kF8>
static hipError_t launch_attn_t(const AttnPlan& p, const AttnSeqs& sq, const void* q, const void* kp,
                                const void* vp, const void* kc, const void* vc, float* out, float scale,
                                float out_scale, void* ws, hipStream_t s) {
  _Float16* opart = reinterpret_cast<_Float16*>(static_cast<uint8_t*>(ws) + p.off_opart);
  float* ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.off_ml);
  const float sl2 = scale * kLog2e;
  prof_begin("attn_partial", s);
  const dim3 grid(p.n_chunks, p.n_qtiles, p.hkv * sq.batch);
  if (sq.batch > 1)
    attn_partial<D, TQ, kF8, true><<<grid, kAThreads, 0, s>>>(static_cast<const TQ*>(q), kp, vp, kc, vc, out,
                                                              opart, ml, sq, p.n, p.hq, p.hkv,
                                                              p.blocks_per_chunk, p.n_chunks, sl2, out_scale);
  else
    attn_partial<D, TQ, kF8, false><<<grid, kAThreads, 0, s>>>(static_cast<const TQ*>(q), kp, vp, kc, vc, out,
                                                               opart, ml, sq, p.n, p.hq, p.hkv,
                                                               p.blocks_per_chunk, p.n_chunks, sl2, out_scale);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_chunks == 1) return e;
  const int rows_per_wg = kCThreads / (D / 4);
  prof_begin("attn_combine", s);
  const int rows_all = sq.batch * p.n * p.hq;
  attn_combine<D><<<(rows_all + rows_per_wg - 1) / rows_per_wg, kCThreads, 0, s>>>(
      opart, ml, out, rows_all, p.n_chunks, out_scale);
  prof_end(s);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_d(const AttnPlan& p, const AttnSeqs& sq, int dtype, const void* q, const void* kp,
                                const void* vp, const void* kc, const void* vc, float* out, float scale,
                                float out_scale, void* ws, hipStream_t s) {
  if (dtype == DG_FP8_E4M3)
    return launch_attn_t<D, uint8_t, true>(p, sq, q, kp, vp, kc, vc, out, scale, out_scale, ws, s);
  if (dtype == DG_BF16)
    return launch_attn_t<D, uint16_t, false>(p, sq, q, kp, vp, kc, vc, out, scale, out_scale, ws, s);
  return launch_attn_t<D, float, false>(p, sq, q, kp, vp, kc, vc, out, scale, out_scale, ws, s);
}

hipError_t launch_attention_batched(const AttnPlan& p, const AttnSeqs& sq, const void* q, const void* kp,
                                    const void* vp, const void* kc, const void* vc, float* out, int dtype,
                                    float scale, void* ws, hipStream_t s, float out_scale) {
  if (dtype == DG_F32) {
    // fp32 K/V: round to bf16 into the workspace first (the whole batched
    // buffers, prefix padding included)
    uint16_t* base = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + p.off_kv16);
    const size_t pre = (size_t)sq.batch * sq.prefix_stride * p.hkv * p.d;
    const size_t can = (size_t)sq.batch * p.n * p.hkv * p.d;
    uint16_t* kp_w = base;
    uint16_t* vp_w = kp_w + pre;
    uint16_t* kc_w = vp_w + pre;
    uint16_t* vc_w = kc_w + can;
    const struct { const void* src; uint16_t* dst; size_t n; } jobs[4] = {
        {kp, kp_w, pre}, {vp, vp_w, pre}, {kc, kc_w, can}, {vc, vc_w, can}};
    for (const auto& j : jobs) {
      if (j.n == 0) continue;
      const size_t n8 = j.n / 8;
      attn_to_bf16<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(static_cast<const float*>(j.src), j.dst, n8);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    kp = kp_w; vp = vp_w; kc = kc_w; vc = vc_w;
  }
  if (p.d == 128) return launch_attn_d<128>(p, sq, dtype, q, kp, vp, kc, vc, out, scale, out_scale, ws, s);
  return launch_attn_d<64>(p, sq, dtype, q, kp, vp, kc, vc, out, scale, out_scale, ws, s);
}

hipError_t launch_attention(const AttnPlan& p, const void* q, const void* kp, const void* vp,
                            const void* kc, const void* vc, float* out, int dtype, float scale,
                            void* ws, hipStream_t s, bool causal, float out_scale) {
  AttnSeqs sq{};
  sq.n_prefix[0] = p.n_prefix;
  sq.causal = causal ? 1u : 0u;
  sq.prefix_stride = p.n_prefix;
  sq.batch = 1;
  return launch_attention_batched(p, sq, q, kp, vp, kc, vc, out, dtype, scale, ws, s, out_scale);
}

}  // namespace dg
