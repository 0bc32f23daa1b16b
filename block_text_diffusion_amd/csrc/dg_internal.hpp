// Host-side plans and launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dg.h"

namespace dg {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-kernel event bracketing for benchmarks (no-op unless enabled and not capturing).
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

// ---- sampler ----
struct SamplerPlan {
  int n;             // rows over the whole batch (n_canvas * batch)
  int n_canvas;      // rows per canvas
  int batch;         // canvases, each with its own control block
  int n_mt;          // 256-row image / contraction tiles
  int vocab, d;
  int n_kb;          // 16-id k-blocks of the vocabulary
  int n_tiles;       // 256-column tiles of d
  int col_pad;       // d rounded up to whole tiles
  int kb_per_split;  // k-blocks per vocabulary split
  int n_splits;      // vocabulary splits (own maxima, own partial z)
  size_t off_stats, off_pimg, off_zp, off_eb, total;
};
// Extra arguments of the entropy-bounded mode (on == false: threshold sampler).
struct EbCall {
  bool on;
  float budget, stop_entropy;
  float* entropy_out;       // [n] or null
  int32_t* argmax;          // [n] in/out
  dg_eb_status* status;
  bool emb_f32 = false;     // E is the plain float32 table [V, d] (not the packed image)
};
SamplerPlan sampler_plan(int n_canvas, int batch, int vocab, int d);
// The combine kernel keeps one merge weight per vocabulary split in LDS; a plan
// with more splits (a vocabulary above 4194304 ids) is refused on the host.
constexpr int kMaxSamplerSplits = 256;
constexpr int kMaxSamplerRows = 65535;   // rows over a batch: the y extent of the per-row launch grids
size_t embedding_packed_bytes(int vocab, int d);
hipError_t launch_embedding_pack(const float* emb, void* packed, int vocab, int d, hipStream_t s);
hipError_t launch_sampler(const SamplerPlan& p, const float* logits, const void* emb_packed,
                          int32_t* ids, uint8_t* committed, float* z, float* conf,
                          uint32_t* n_unc, dg_ctrl* ctrl, void* ws, hipStream_t s,
                          const EbCall& eb = EbCall{false, 0.f, 0.f, nullptr, nullptr, nullptr});

// ---- top-k truncated sampler ----
struct TopkPlan {
  int n, n_canvas, batch, vocab, d;
  int k;               // kept logits per row
  int n_slices;        // 4096-id sub-slices of the vocabulary (one wavefront each)
  int max_candidates;  // slice candidates one row pass can hold (n_slices * k must not exceed it)
  size_t off_part, off_cand, off_bad, off_list, off_zp, off_eb, total;
};
TopkPlan topk_plan(int n_canvas, int batch, int vocab, int d, int k);
hipError_t launch_sampler_topk(const TopkPlan& p, const float* logits, const float* emb, int32_t* ids,
                               uint8_t* committed, float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl,
                               void* ws, hipStream_t s, const EbCall& eb);

// ---- attention ----
struct AttnPlan {
  int n, n_prefix, hq, hkv, d, group, batch;
  int rows;          // n * group packed query rows per KV head
  int n_qtiles;      // 128-row query tiles per KV head
  int blocks_prefix;     // 64-key blocks of the prefix
  int blocks_total;      // prefix blocks then canvas blocks
  int blocks_per_chunk;  // blocks per key chunk
  int n_chunks;          // key chunks (partial outputs merged by the combine)
  size_t off_kv16, kv16_bytes;  // bf16 copies of fp32 K/V
  size_t off_opart, off_ml, total;
};
// n_prefix is the prefix row stride of a batch (the longest prefix); the
// partial outputs are sized for batch sequences.
AttnPlan attn_plan(int n, int n_prefix, int hq, int hkv, int d, int batch = 1);
// Per-sequence parameters of one launch over a batch of sequences: sequence s
// owns rows [s n, (s + 1) n) of Q, O and the canvas K/V, and prefix rows
// [s stride, s stride + n_prefix[s]) of the prefix K/V.  Passed by value in
// the kernel arguments.
constexpr int kMaxAttnSeqs = 64;
struct AttnSeqs {
  int n_prefix[kMaxAttnSeqs];
  uint64_t causal;     // bit s: sequence s sees canvas keys 0..i only
  int prefix_stride;   // prefix rows between consecutive sequences
  int batch;
};
// dtype: DG_F32 (K/V rounded to bf16 into the workspace first), DG_BF16, or
// DG_FP8_E4M3 (Q/K/V bytes converted exactly to bf16 while staged).
// out_scale multiplies the normalised output.
hipError_t launch_attention(const AttnPlan& p, const void* q, const void* kp, const void* vp,
                            const void* kc, const void* vc, float* out, int dtype,
                            float scale, void* ws, hipStream_t s, bool causal = false,
                            float out_scale = 1.0f);
// The same over sq.batch sequences (p planned with n_prefix = sq.prefix_stride
// and batch = sq.batch).
hipError_t launch_attention_batched(const AttnPlan& p, const AttnSeqs& sq, const void* q, const void* kp,
                                    const void* vp, const void* kc, const void* vc, float* out, int dtype,
                                    float scale, void* ws, hipStream_t s, float out_scale = 1.0f);

// ---- block loop helpers ----
hipError_t launch_canvas_init(int32_t* ids, uint8_t* committed, dg_ctrl* ctrl, int n, int vocab,
                              hipStream_t s);
hipError_t launch_synth_logits(float* logits, const int32_t* ids, const uint8_t* committed,
                               const dg_ctrl* ctrl, const float* table, int table_size, int n,
                               int vocab, hipStream_t s);
hipError_t launch_probe_mfma(float* sink, int n_wg, int iters, hipStream_t s);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_philox_fill(uint32_t* out, size_t n_words, uint64_t seed, uint32_t c1,
                              uint32_t c2, uint32_t c3, hipStream_t s);

}  // namespace dg
