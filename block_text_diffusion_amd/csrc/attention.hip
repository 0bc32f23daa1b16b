// Bidirectional canvas attention on gfx950 (DiffusionGemma Technical Report
// part 4/6, section 6 "Attention" and section 9.1: every canvas position attends
// to the committed KV-cache history and to all canvas positions, no mask).
//
// Layout per workgroup: one KV head, 128 packed query rows (canvas position x
// query head of the group, so the heads sharing a KV head share each K/V tile),
// one chunk of the key sequence [prefix ; canvas].  Four wavefronts each own 32
// query rows.  Scores are formed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16, so a lane holds 16 keys of one query and the
// row-wise softmax needs a single cross-lane exchange; the probabilities then
// feed O^T = V^T P^T straight from the score registers.  K is staged in LDS as
// [key][d], V transposed as [d][key]; both xor-swizzled.  Online softmax in
// fp32 (base 2).  Key chunks are merged by a log-sum-exp combine kernel.
#include "dg_common.hpp"
#include "dg_internal.hpp"

namespace dg {

constexpr int kAThreads = 256;
constexpr int kARows = 128;   // packed query rows per workgroup
constexpr int kAKeys = 64;    // keys per LDS block

template <int D>
__device__ __forceinline__ int k_swz(int key, int chunk) {
  // rows of D*2 bytes, 16-byte chunks
  if constexpr (D == 128) return key * (D * 2) + ((chunk ^ (key & 15)) << 4);
  else return key * (D * 2) + ((chunk ^ ((key ^ (key >> 3)) & 7)) << 4);
}

// V^T rows are 64 keys = 128 bytes = sixteen 8-byte units of 4 keys.
__device__ __forceinline__ int v_swz(int d, int unit) {
  return d * 128 + ((unit ^ ((d ^ (d >> 4)) & 15)) << 3);
}

// Load 8 consecutive elements as 8 bf16 (packed in 4 u32).
__device__ __forceinline__ u32x4 load8(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return (u32x4){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                 pack_bf16x2(b[2], b[3])};
}

template <int D, typename T>
__global__ __launch_bounds__(kAThreads) void attn_partial(
    const T* __restrict__ q, const T* __restrict__ kp, const T* __restrict__ vp,
    const T* __restrict__ kc, const T* __restrict__ vc, float* __restrict__ out,
    float* __restrict__ opart, float* __restrict__ ml, int n, int n_prefix, int hq, int hkv,
    int chunk_len, int n_chunks, float scale_log2e) {
  constexpr int KS = D / 16;   // 16-wide k steps over the head dimension
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint8_t ks_lds[kAKeys * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[D * kAKeys * 2];

  const int chunk = blockIdx.x;
  const int qtile = blockIdx.y;
  const int kvh = blockIdx.z;
  const int group = hq / hkv;
  const int rows = n * group;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int half = lane >> 5;

  // this lane's query row (a column of S^T)
  const int r = qtile * kARows + wave * 32 + (lane & 31);
  const bool r_ok = r < rows;
  const int qn = r_ok ? r / group : 0;
  const int qh = kvh * group + (r_ok ? r % group : 0);

  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 w = (u32x4){0u, 0u, 0u, 0u};
    if (r_ok) w = load8(q + ((size_t)qn * hq + qh) * D + 16 * ks + 8 * half);
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }

  const int total = n_prefix + n;
  const int k0 = chunk * chunk_len;
  const int k1 = min(total, k0 + chunk_len);

  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kb0 = k0; kb0 < k1; kb0 += kAKeys) {
    // ---- stage K [key][d] ----
#pragma unroll
    for (int i = 0; i < (kAKeys * D / 8) / kAThreads; ++i) {
      const int idx = t + kAThreads * i;
      const int key = idx / (D / 8);
      const int ch = idx % (D / 8);
      const int j = kb0 + key;
      u32x4 w = (u32x4){0u, 0u, 0u, 0u};
      if (j < k1) {
        const T* src = (j < n_prefix) ? kp + ((size_t)j * hkv + kvh) * D
                                      : kc + ((size_t)(j - n_prefix) * hkv + kvh) * D;
        w = load8(src + ch * 8);
      }
      *reinterpret_cast<u32x4*>(ks_lds + k_swz<D>(key, ch)) = w;
    }
    // ---- stage V^T [d][key]: each task moves 4 keys x 8 dims ----
    constexpr int VTASKS = (kAKeys / 4) * (D / 8);
    if (t < VTASKS) {
      const int kq = t / (D / 8);   // key quad
      const int dg = t % (D / 8);   // 8-dim group
      u32x4 rw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kb0 + 4 * kq + i;
        rw[i] = (u32x4){0u, 0u, 0u, 0u};
        if (j < k1) {
          const T* src = (j < n_prefix) ? vp + ((size_t)j * hkv + kvh) * D
                                        : vc + ((size_t)(j - n_prefix) * hkv + kvh) * D;
          rw[i] = load8(src + dg * 8);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // dims 2k (low halves) and 2k+1 (high halves) of word k
        const uint32_t e0a = (rw[0][k] & 0xFFFFu) | (rw[1][k] << 16);
        const uint32_t e0b = (rw[2][k] & 0xFFFFu) | (rw[3][k] << 16);
        const uint32_t e1a = (rw[0][k] >> 16) | (rw[1][k] & 0xFFFF0000u);
        const uint32_t e1b = (rw[2][k] >> 16) | (rw[3][k] & 0xFFFF0000u);
        const int d0 = dg * 8 + 2 * k;
        *reinterpret_cast<u32x2*>(vt_lds + v_swz(d0, kq)) = (u32x2){e0a, e0b};
        *reinterpret_cast<u32x2*>(vt_lds + v_swz(d0 + 1, kq)) = (u32x2){e1a, e1b};
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
      const int key = 32 * kb + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks_lds + k_swz<D>(key, 2 * ks + half));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // ---- online softmax over this block's 64 keys (base 2) ----
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb0 + 32 * kb + 8 * (v >> 2) + 4 * half + (v & 3);
        const float x = (key < k1) ? s[kb][v] * scale_log2e : -INFINITY;
        s[kb][v] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = __builtin_amdgcn_exp2f(s[kb][v] - m_new);
        lsum += p[v];
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 w = (u32x4){pack_bf16x2(p[8 * hh + 0], p[8 * hh + 1]),
                                pack_bf16x2(p[8 * hh + 2], p[8 * hh + 3]),
                                pack_bf16x2(p[8 * hh + 4], p[8 * hh + 5]),
                                pack_bf16x2(p[8 * hh + 6], p[8 * hh + 7])};
        pf[2 * kb + hh] = __builtin_bit_cast(bf16x8, w);
      }
    }
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;

    // ---- O^T += V^T P^T: 16-key steps; lane half h supplies keys 16t+4h+{0..3}, 16t+8+4h+{0..3} ----
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dd = 32 * db + (lane & 31);
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vt_lds + v_swz(dd, 4 * tt + half));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vt_lds + v_swz(dd, 4 * tt + 2 + half));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[tt], acc_o[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!r_ok) return;
  // lane holds O^T rows d = 32*db + 8*(v/4) + 4*half + v%4 for query r
  const size_t orow = (size_t)qn * hq + qh;
  if (n_chunks == 1) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * half;
        *reinterpret_cast<f32x4*>(out + orow * D + dd) =
            (f32x4){acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv, acc_o[db][4 * g + 2] * inv,
                    acc_o[db][4 * g + 3] * inv};
      }
  } else {
    float* dst = opart + ((size_t)chunk * n * hq + orow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * half;
        *reinterpret_cast<f32x4*>(dst + dd) =
            (f32x4){acc_o[db][4 * g], acc_o[db][4 * g + 1], acc_o[db][4 * g + 2], acc_o[db][4 * g + 3]};
      }
    if (half == 0) {
      float* mp = ml + ((size_t)chunk * n * hq + orow) * 2;
      mp[0] = m_run;
      mp[1] = l_run;
    }
  }
}

// Merge key chunks: O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
template <int D>
__global__ __launch_bounds__(D) void attn_combine(const float* __restrict__ opart,
                                                  const float* __restrict__ ml,
                                                  float* __restrict__ out, int n_rows_total,
                                                  int n_chunks) {
  const int row = blockIdx.x;
  const int d = threadIdx.x;
  float mx = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) mx = fmaxf(mx, ml[((size_t)c * n_rows_total + row) * 2]);
  float lsum = 0.f, acc = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const size_t idx = (size_t)c * n_rows_total + row;
    const float w = __builtin_amdgcn_exp2f(ml[idx * 2] - mx);
    lsum += w * ml[idx * 2 + 1];
    acc += w * opart[idx * D + d];
  }
  out[(size_t)row * D + d] = acc / lsum;
}

AttnPlan attn_plan(int n, int n_prefix, int hq, int hkv, int d) {
  AttnPlan p{};
  p.n = n; p.n_prefix = n_prefix; p.hq = hq; p.hkv = hkv; p.d = d;
  p.group = hq / hkv;
  p.rows = n * p.group;
  p.n_qtiles = (p.rows + kARows - 1) / kARows;
  const int total = n_prefix + n;
  const int blocks = (total + kAKeys - 1) / kAKeys;
  const int base = hkv * p.n_qtiles;
  int want = (512 + base - 1) / base;
  if (want > blocks) want = blocks;
  if (want < 1) want = 1;
  const int blocks_per_chunk = (blocks + want - 1) / want;
  p.chunk_len = blocks_per_chunk * kAKeys;
  p.n_chunks = (total + p.chunk_len - 1) / p.chunk_len;
  p.off_opart = 0;
  if (p.n_chunks > 1) {
    p.off_ml = align_up((size_t)p.n_chunks * n * hq * d * sizeof(float), 256);
    p.total = p.off_ml + align_up((size_t)p.n_chunks * n * hq * 2 * sizeof(float), 256);
  } else {
    p.off_ml = 0;
    p.total = 0;
  }
  return p;
}

template <int D, typename T>
static hipError_t launch_attn_t(const AttnPlan& p, const void* q, const void* kp, const void* vp,
                                const void* kc, const void* vc, float* out, float scale,
                                void* ws, hipStream_t s) {
  float* opart = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.off_opart);
  float* ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.off_ml);
  const float sl2 = scale * kLog2e;
  prof_begin("attn_partial", s);
  attn_partial<D, T><<<dim3(p.n_chunks, p.n_qtiles, p.hkv), kAThreads, 0, s>>>(
      static_cast<const T*>(q), static_cast<const T*>(kp), static_cast<const T*>(vp),
      static_cast<const T*>(kc), static_cast<const T*>(vc), out, opart, ml, p.n, p.n_prefix, p.hq,
      p.hkv, p.chunk_len, p.n_chunks, sl2);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_chunks == 1) return e;
  prof_begin("attn_combine", s);
  attn_combine<D><<<p.n * p.hq, D, 0, s>>>(opart, ml, out, p.n * p.hq, p.n_chunks);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnPlan& p, const void* q, const void* kp, const void* vp,
                            const void* kc, const void* vc, float* out, bool bf16_in,
                            float scale, void* ws, hipStream_t s) {
  if (p.d == 128)
    return bf16_in ? launch_attn_t<128, uint16_t>(p, q, kp, vp, kc, vc, out, scale, ws, s)
                   : launch_attn_t<128, float>(p, q, kp, vp, kc, vc, out, scale, ws, s);
  return bf16_in ? launch_attn_t<64, uint16_t>(p, q, kp, vp, kc, vc, out, scale, ws, s)
                 : launch_attn_t<64, float>(p, q, kp, vp, kc, vc, out, scale, ws, s);
}

}  // namespace dg
