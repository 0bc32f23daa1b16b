// Block-loop helpers on gfx950: canvas initialisation (a canvas starts as
// uniformly random tokens: explainer "DiffusionGemma: Google's open diffusion
// LLM", sections quoting report 3.1-3.3), the synthetic logit generator that
// stands in for the model in the decode-run workload, and a raw Philox dump.
#include "dg_common.hpp"
#include "dg_internal.hpp"

namespace dg {

__global__ __launch_bounds__(256) void canvas_init_kernel(int32_t* __restrict__ ids,
                                                          uint8_t* __restrict__ committed,
                                                          dg_ctrl* __restrict__ ctrl, int n,
                                                          int vocab) {
  const int i = threadIdx.x;
  const uint64_t seed = ctrl->seed;
  const uint32_t gstep = ctrl->gstep;
  if (i < n) {
    const Philox4 h = philox4x32_10(0u, (uint32_t)i, gstep, kStreamInit, seed_lo(seed), seed_hi(seed));
    ids[i] = (int32_t)range_draw(h.w0, (uint32_t)vocab);
    committed[i] = 0;
  }
  __syncthreads();
  if (i == 0) ctrl->s_in_block = 0u;
}

constexpr int kSynThreads = 256;
constexpr int kSynGroups = 8;          // 4-id groups per thread (one Philox call each)
constexpr float kSpike = 30.0f;
constexpr uint32_t kChoosePerStep = 20u;

// grid (ceil(V / (4 kSynGroups kSynThreads)), n); each thread produces kSynGroups
// groups of ids 4m..4m+3 (m strided by the workgroup size), one Philox call per
// group.  The row's spike target is drawn once per workgroup.
template <bool kAligned>
__global__ __launch_bounds__(kSynThreads) void synth_logits_kernel(
    float* __restrict__ logits, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ committed, const dg_ctrl* __restrict__ ctrl,
    const float* __restrict__ table, int n, int vocab) {
  const int row = blockIdx.y;
  const int t = threadIdx.x;
  const uint64_t seed = ctrl->seed;
  const uint32_t gstep = ctrl->gstep;
  const uint32_t k0 = seed_lo(seed), k1 = seed_hi(seed);
  const int open = (t < n && !committed[t]) ? 1 : 0;
  const uint32_t n_open = (uint32_t)__syncthreads_count(open);

  // the row's spike target, drawn once per workgroup
  __shared__ int s_target;
  if (t == 0) {
    int target = -1;
    if (committed[row]) {
      target = ids[row];
    } else {
      const Philox4 hc = philox4x32_10(0u, (uint32_t)row, gstep, kStreamSynChoose, k0, k1);
      if (range_draw(hc.w0, n_open) < kChoosePerStep) {
        const Philox4 ht = philox4x32_10(0u, (uint32_t)row, gstep, kStreamSynTarget, k0, k1);
        target = (int)range_draw(ht.w0, (uint32_t)vocab);
      }
    }
    s_target = target;
  }
  __syncthreads();
  const int target = s_target;
#pragma unroll 2
  for (int g = 0; g < kSynGroups; ++g) {
    const int j = 4 * ((blockIdx.x * kSynGroups + g) * kSynThreads + t);
    if (j >= vocab) return;
    const Philox4 h = philox4x32_10((uint32_t)j >> 2, (uint32_t)row, gstep, kStreamSynNoise, k0, k1);
    float v[4] = {table[h.w0 >> 16], table[h.w1 >> 16], table[h.w2 >> 16], table[h.w3 >> 16]};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e == target) v[e] = v[e] + kSpike;
    float* dst = logits + (size_t)row * vocab + j;
    if (kAligned && j + 3 < vocab) {
      *reinterpret_cast<f32x4*>(dst) = (f32x4){v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < vocab) dst[e] = v[e];
    }
  }
}

__global__ __launch_bounds__(256) void philox_fill_kernel(uint32_t* __restrict__ out, size_t n_ctr,
                                                          uint64_t seed, uint32_t c1, uint32_t c2,
                                                          uint32_t c3) {
  const size_t m = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= n_ctr) return;
  const Philox4 h = philox4x32_10((uint32_t)m, c1, c2, c3, seed_lo(seed), seed_hi(seed));
  *reinterpret_cast<u32x4*>(out + 4 * m) = (u32x4){h.w0, h.w1, h.w2, h.w3};
}

// ---- peak probes (measurement only) ----
// Matrix cores: every wave keeps four independent accumulator chains of
// v_mfma_f32_32x32x16_bf16 on register operands (a chain on one accumulator
// cannot issue back to back), so the loop runs at the rate the matrix cores
// sustain at the clock the chip holds under this load.
constexpr int kProbeWaves = 4;
__global__ __launch_bounds__(64 * kProbeWaves) void probe_mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + 0.0078125f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.5f - 0.0078125f * (float)((lane * 3 + e) & 7));
  }
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int v = 0; v < 16; ++v) { c0[v] = 0.f; c1[v] = 0.f; c2[v] = 0.f; c3[v] = 0.f; }
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc += c0[v] + c1[v] + c2[v] + c3[v];
  // every lane's sum is written: the loop's results are live
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// HBM: a plain copy, 16 bytes per lane per iteration, grid-stride.
__global__ __launch_bounds__(256) void probe_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                         size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// HBM: a plain read, 16 bytes per lane per load, four loads in flight per
// lane, grid-stride.  Each wave writes the xor of everything it read, so no
// load is dead.
constexpr int kProbeReadBlocks = 4096;
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = (u32x4){0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > kProbeReadBlocks) blocks = kProbeReadBlocks;
  probe_read_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(float* sink, int n_wg, int iters, hipStream_t s) {
  probe_mfma_kernel<<<n_wg, 64 * kProbeWaves, 0, s>>>(sink, iters);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  probe_copy_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

hipError_t launch_canvas_init(int32_t* ids, uint8_t* committed, dg_ctrl* ctrl, int n, int vocab,
                              hipStream_t s) {
  prof_begin("canvas_init", s);
  canvas_init_kernel<<<1, 256, 0, s>>>(ids, committed, ctrl, n, vocab);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_synth_logits(float* logits, const int32_t* ids, const uint8_t* committed,
                               const dg_ctrl* ctrl, const float* table, int table_size, int n,
                               int vocab, hipStream_t s) {
  (void)table_size;
  const dim3 grid((vocab + 4 * kSynGroups * kSynThreads - 1) / (4 * kSynGroups * kSynThreads), n);
  prof_begin("synth_logits", s);
  if (vocab % 4 == 0)
    synth_logits_kernel<true><<<grid, kSynThreads, 0, s>>>(logits, ids, committed, ctrl, table, n, vocab);
  else
    synth_logits_kernel<false><<<grid, kSynThreads, 0, s>>>(logits, ids, committed, ctrl, table, n, vocab);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_philox_fill(uint32_t* out, size_t n_words, uint64_t seed, uint32_t c1,
                              uint32_t c2, uint32_t c3, hipStream_t s) {
  const size_t n_ctr = n_words / 4;
  if (n_ctr == 0) return hipSuccess;
  const size_t blocks = (n_ctr + 255) / 256;
  philox_fill_kernel<<<(unsigned)blocks, 256, 0, s>>>(out, n_ctr, seed, c1, c2, c3);
  return hipGetLastError();
}

}  // namespace dg
