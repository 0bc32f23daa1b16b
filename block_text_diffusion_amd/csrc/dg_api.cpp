// C ABI of the canvas-denoising library: host validation, workspace carving,
// launch sequencing, step-graph capture, per-kernel event profiling.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dg.h"
#include "dg_internal.hpp"

// Workspace of dg_canvas_attention_noalloc, for callers that cannot allocate
// device memory: a file-scope device array of fixed size.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never
// passes the array's name to a kernel or a copy (in host code it is only a
// host-side stand-in); it uses the device address looked up per device with
// hipGetSymbolAddress.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;
thread_local bool g_capturing = false;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DG_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- profiling ----
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_event_pool;
const char* g_prof_pending = nullptr;
hipEvent_t g_prof_pending_start = nullptr;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---- argument checks ----
int check_attention(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                    const float* out, int n, int np, int hq, int hkv, int d, int dtype) {
  if (!q || !kc || !vc || !out) return fail(DG_EINVAL, "attention: null q/k_canvas/v_canvas/out");
  if (np < 0) return fail(DG_EINVAL, "attention: n_prefix < 0");
  if (np > 0 && (!kp || !vp)) return fail(DG_EINVAL, "attention: null prefix with n_prefix > 0");
  if (n < 1) return fail(DG_EINVAL, "attention: n_canvas < 1");
  if (n > 256) return fail(DG_EUNSUPPORTED, "attention: n_canvas > 256");
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return fail(DG_EINVAL, "attention: hq %% hkv != 0 or < 1");
  if (d != 64 && d != 128) return fail(DG_EUNSUPPORTED, "attention: head_dim must be 64 or 128");
  if (dtype != DG_F32 && dtype != DG_BF16 && dtype != DG_FP8_E4M3) return fail(DG_EUNSUPPORTED, "attention: dtype");
  // K/V blocks are fetched with 32-bit buffer offsets
  const uint64_t elem = dtype == DG_FP8_E4M3 ? 1ull : 2ull;
  if ((uint64_t)np * (uint64_t)hkv * (uint64_t)d * elem >= (1ull << 31))
    return fail(DG_EUNSUPPORTED, "attention: prefix K/V must be below 2 GiB per tensor");
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(out) ||
      (np > 0 && (!aligned16(kp) || !aligned16(vp))))
    return fail(DG_EINVAL, "attention: pointers must be 16-byte aligned");
  return DG_OK;
}

int check_sampler(const float* logits, const void* emb, const int32_t* ids, const uint8_t* committed,
                  const float* z, const uint32_t* n_unc, const dg_ctrl* ctrl, int n, int vocab, int d,
                  int batch = 1) {
  if (!logits || !emb || !ids || !committed || !z || !n_unc || !ctrl)
    return fail(DG_EINVAL, "sampler: null pointer argument");
  if (n < 1) return fail(DG_EINVAL, "sampler: n_canvas < 1");
  if (n > 256) return fail(DG_EUNSUPPORTED, "sampler: n_canvas > 256");
  if (batch < 1) return fail(DG_EINVAL, "sampler: batch < 1");
  if (batch > 4096) return fail(DG_EUNSUPPORTED, "sampler: batch > 4096");
  if (vocab < 2) return fail(DG_EINVAL, "sampler: vocab < 2");
  if (d < 1) return fail(DG_EINVAL, "sampler: d_model < 1");
  if (dg::embedding_packed_bytes(vocab, d) >= (1ull << 40)) return fail(DG_EINVAL, "sampler: E too large");
  // the logits are addressed with 32-bit byte offsets
  if ((uint64_t)n * (uint64_t)batch * (uint64_t)vocab * 4ull >= (1ull << 32))
    return fail(DG_EUNSUPPORTED, "sampler: n_canvas * batch * vocab * 4 must be below 2^32");
  // rows are a launch-grid dimension of the per-row kernels
  if ((int64_t)n * batch > dg::kMaxSamplerRows)
    return fail(DG_EUNSUPPORTED, "sampler: n_canvas * batch above %d rows", dg::kMaxSamplerRows);
  if (!aligned16(logits) || !aligned16(emb) || !aligned16(z))
    return fail(DG_EINVAL, "sampler: logits/emb_packed/selfcond must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(ctrl) & 7u) != 0) return fail(DG_EINVAL, "sampler: ctrl misaligned");
  return DG_OK;
}

// The plan's vocabulary splits must fit the combine kernel's per-split weights.
int check_sampler_plan(const dg::SamplerPlan& p, const char* who) {
  if (p.n_splits > dg::kMaxSamplerSplits)
    return fail(DG_EUNSUPPORTED, "%s: vocab %d needs %d vocabulary splits, more than %d (vocab above 4194304)", who,
                p.vocab, p.n_splits, dg::kMaxSamplerSplits);
  return DG_OK;
}

// The device address of the current device's scratch array, looked up on the
// first call on that device, with that device current, and kept per device.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int check_topk(int k, const dg::TopkPlan& p, void* ws, size_t ws_bytes, const char* who) {
  if (k < 1) return fail(DG_EINVAL, "%s: top_k < 1", who);
  if (k > 256) return fail(DG_EUNSUPPORTED, "%s: top_k > 256", who);
  if ((int64_t)p.n_slices * k > p.max_candidates)
    return fail(DG_EUNSUPPORTED, "%s: slices * top_k = %lld candidates exceed %d (top_k too large for vocab)", who,
                (long long)p.n_slices * k, p.max_candidates);
  if (!ws || ws_bytes < p.total) return fail(DG_EWORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, p.total);
  if (!aligned16(ws)) return fail(DG_EINVAL, "%s: workspace misaligned", who);
  return DG_OK;
}

}  // namespace

namespace dg {

void prof_begin(const char* name, hipStream_t s) {
  if (!g_prof_on || g_capturing) return;
  hipEvent_t e = take_event();
  if (!e) return;
  // best effort: a pair whose record failed is skipped by dg_profile_read
  (void)hipEventRecord(e, s);
  g_prof_pending = name;
  g_prof_pending_start = e;
}

void prof_end(hipStream_t s) {
  if (!g_prof_on || g_capturing || !g_prof_pending) return;
  hipEvent_t e = take_event();
  if (!e) return;
  (void)hipEventRecord(e, s);
  g_prof_recs.push_back(ProfRec{g_prof_pending, g_prof_pending_start, e});
  g_prof_pending = nullptr;
  g_prof_pending_start = nullptr;
}

}  // namespace dg

extern "C" {

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_EINVAL: return "invalid argument";
    case DG_EUNSUPPORTED: return "unsupported configuration";
    case DG_EWORKSPACE: return "workspace too small";
    case DG_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dg_last_error(void) { return g_last_error.c_str(); }

size_t dg_attention_workspace_bytes(int n, int np, int hq, int hkv, int d) {
  if (n < 1 || n > 256 || np < 0 || hq < 1 || hkv < 1 || hq % hkv || (d != 64 && d != 128)) return 0;
  const size_t t = dg::attn_plan(n, np, hq, hkv, d).total;
  return t == 0 ? 256 : t;
}

size_t dg_attention_batched_workspace_bytes(int batch, int n, int stride, int hq, int hkv, int d) {
  if (batch < 1 || batch > dg::kMaxAttnSeqs) return 0;
  if (n < 1 || n > 256 || stride < 0 || hq < 1 || hkv < 1 || hq % hkv || (d != 64 && d != 128)) return 0;
  const size_t t = dg::attn_plan(n, stride, hq, hkv, d, batch).total;
  return t == 0 ? 256 : t;
}

size_t dg_sampler_workspace_bytes(int n, int vocab, int d) {
  return dg_sampler_workspace_bytes_batched(n, 1, vocab, d);
}

size_t dg_sampler_workspace_bytes_batched(int n, int batch, int vocab, int d) {
  if (n < 1 || n > 256 || batch < 1 || batch > 4096 || vocab < 2 || d < 1) return 0;
  if ((int64_t)n * batch > dg::kMaxSamplerRows) return 0;
  const dg::SamplerPlan p = dg::sampler_plan(n, batch, vocab, d);
  return p.n_splits > dg::kMaxSamplerSplits ? 0 : p.total;
}

size_t dg_denoise_workspace_bytes(int n, int np, int hq, int hkv, int d, int vocab, int dm) {
  const size_t a = dg_attention_workspace_bytes(n, np, hq, hkv, d);
  const size_t b = dg_sampler_workspace_bytes(n, vocab, dm);
  if (!a || !b) return 0;
  return a > b ? a : b;  // the two passes run one after the other and share it
}

int dg_canvas_attention(const void* q, const void* kp, const void* vp, const void* kc,
                        const void* vc, float* out, int n, int np, int hq, int hkv, int d,
                        int dtype, float scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  return dg_canvas_attention_ex(q, kp, vp, kc, vc, out, n, np, hq, hkv, d, dtype, scale, 0u, ws,
                                ws_bytes, stream);
}

int dg_canvas_attention_ex(const void* q, const void* kp, const void* vp, const void* kc,
                           const void* vc, float* out, int n, int np, int hq, int hkv, int d,
                           int dtype, float scale, uint32_t attn_flags, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (attn_flags & ~(uint32_t)DG_ATTN_CAUSAL) return fail(DG_EINVAL, "attention: unknown flag bits");
  if (dtype == DG_FP8_E4M3) return fail(DG_EINVAL, "attention: FP8 inputs take dg_canvas_attention_fp8 (scales)");
  int st = check_attention(q, kp, vp, kc, vc, out, n, np, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  const dg::AttnPlan p = dg::attn_plan(n, np, hq, hkv, d);
  if (p.total > 0 && (!ws || ws_bytes < p.total))
    return fail(DG_EWORKSPACE, "attention: workspace %zu < %zu bytes", ws_bytes, p.total);
  if (p.total > 0 && !aligned16(ws)) return fail(DG_EINVAL, "attention: workspace misaligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  hipError_t e = dg::launch_attention(p, q, kp, vp, kc, vc, out, dtype, scale, ws, stream,
                                      (attn_flags & DG_ATTN_CAUSAL) != 0);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return DG_OK;
}

size_t dg_static_scratch_bytes(void) { return kStaticScratchBytes; }

int dg_canvas_attention_noalloc(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                                float* out, int n, int np, int hq, int hkv, int d, int dtype, float scale,
                                uint32_t attn_flags, hipStream_t stream) {
  if (attn_flags & ~(uint32_t)DG_ATTN_CAUSAL) return fail(DG_EINVAL, "attention_noalloc: unknown flag bits");
  if (dtype == DG_FP8_E4M3)
    return fail(DG_EINVAL, "attention_noalloc: FP8 inputs take dg_canvas_attention_fp8 (scales)");
  int st = check_attention(q, kp, vp, kc, vc, out, n, np, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  const dg::AttnPlan p = dg::attn_plan(n, np, hq, hkv, d);
  if (p.total > kStaticScratchBytes)
    return fail(DG_EUNSUPPORTED, "attention_noalloc: these sizes need %zu workspace bytes, more than the %zu-byte "
                "static scratch (use dg_canvas_attention with a workspace)", p.total, kStaticScratchBytes);
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "attention_noalloc: scratch address");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  e = dg::launch_attention(p, q, kp, vp, kc, vc, out, dtype, scale, ws, stream, (attn_flags & DG_ATTN_CAUSAL) != 0);
  if (e != hipSuccess) return hip_fail(e, "attention_noalloc launch");
  return DG_OK;
}

int dg_canvas_attention_batched(const void* q, const void* kp, const void* vp, const void* kc,
                                const void* vc, float* out, const int32_t* n_prefix, const uint8_t* causal,
                                int batch, int n, int stride, int hq, int hkv, int d, int dtype, float scale,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  if (batch < 1) return fail(DG_EINVAL, "attention_batched: batch < 1");
  if (batch > dg::kMaxAttnSeqs) return fail(DG_EUNSUPPORTED, "attention_batched: batch > %d", dg::kMaxAttnSeqs);
  if (!n_prefix) return fail(DG_EINVAL, "attention_batched: null n_prefix");
  if (stride < 0) return fail(DG_EINVAL, "attention_batched: prefix_stride < 0");
  if (dtype == DG_FP8_E4M3) return fail(DG_EUNSUPPORTED, "attention_batched: FP8 inputs are not batched");
  int st = check_attention(q, kp, vp, kc, vc, out, n, stride, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  if ((int64_t)hkv * batch > 65535) return fail(DG_EUNSUPPORTED, "attention_batched: hkv * batch > 65535");
  dg::AttnSeqs sq{};
  for (int s = 0; s < batch; ++s) {
    if (n_prefix[s] < 0 || n_prefix[s] > stride)
      return fail(DG_EINVAL, "attention_batched: n_prefix[%d] = %d outside [0, prefix_stride = %d]", s,
                  n_prefix[s], stride);
    if (causal && causal[s] > 1) return fail(DG_EINVAL, "attention_batched: causal[%d] must be 0 or 1", s);
    sq.n_prefix[s] = n_prefix[s];
    if (causal && causal[s]) sq.causal |= 1ull << s;
  }
  sq.prefix_stride = stride;
  sq.batch = batch;
  const dg::AttnPlan p = dg::attn_plan(n, stride, hq, hkv, d, batch);
  if (p.total > 0 && (!ws || ws_bytes < p.total))
    return fail(DG_EWORKSPACE, "attention_batched: workspace %zu < %zu bytes", ws_bytes, p.total);
  if (p.total > 0 && !aligned16(ws)) return fail(DG_EINVAL, "attention_batched: workspace misaligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  hipError_t e = dg::launch_attention_batched(p, sq, q, kp, vp, kc, vc, out, dtype, scale, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "attention_batched launch");
  return DG_OK;
}

int dg_canvas_attention_fp8(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                            float* out, int n, int np, int hq, int hkv, int d, float scale, float q_scale,
                            float k_scale, float v_scale, uint32_t attn_flags, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (attn_flags & ~(uint32_t)DG_ATTN_CAUSAL) return fail(DG_EINVAL, "attention_fp8: unknown flag bits");
  int st = check_attention(q, kp, vp, kc, vc, out, n, np, hq, hkv, d, DG_FP8_E4M3);
  if (st != DG_OK) return st;
  if (!(q_scale > 0.f) || !std::isfinite(q_scale) || !(k_scale > 0.f) || !std::isfinite(k_scale) ||
      !(v_scale > 0.f) || !std::isfinite(v_scale))
    return fail(DG_EINVAL, "attention_fp8: q_scale, k_scale and v_scale must be finite and > 0");
  const dg::AttnPlan p = dg::attn_plan(n, np, hq, hkv, d);
  if (p.total > 0 && (!ws || ws_bytes < p.total))
    return fail(DG_EWORKSPACE, "attention_fp8: workspace %zu < %zu bytes", ws_bytes, p.total);
  if (p.total > 0 && !aligned16(ws)) return fail(DG_EINVAL, "attention_fp8: workspace misaligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  // the tensor scales fold into the score scale and the output
  hipError_t e = dg::launch_attention(p, q, kp, vp, kc, vc, out, DG_FP8_E4M3, scale * q_scale * k_scale, ws,
                                      stream, (attn_flags & DG_ATTN_CAUSAL) != 0, v_scale);
  if (e != hipSuccess) return hip_fail(e, "attention_fp8 launch");
  return DG_OK;
}

int dg_sampler_step(const float* logits, const void* emb, int32_t* ids, uint8_t* committed,
                    float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n, int vocab, int d,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return dg_sampler_step_batched(logits, emb, ids, committed, z, conf, n_unc, ctrl, n, 1, vocab, d, ws,
                                 ws_bytes, stream);
}

int dg_sampler_step_batched(const float* logits, const void* emb, int32_t* ids, uint8_t* committed,
                            float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n, int batch,
                            int vocab, int d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, d, batch);
  if (st != DG_OK) return st;
  const dg::SamplerPlan p = dg::sampler_plan(n, batch, vocab, d);
  st = check_sampler_plan(p, "sampler");
  if (st != DG_OK) return st;
  if (!ws || ws_bytes < p.total)
    return fail(DG_EWORKSPACE, "sampler: workspace %zu < %zu bytes", ws_bytes, p.total);
  if (!aligned16(ws)) return fail(DG_EINVAL, "sampler: workspace misaligned");
  hipError_t e = dg::launch_sampler(p, logits, emb, ids, committed, z, conf, n_unc, ctrl, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "sampler launch");
  return DG_OK;
}

int dg_sampler_step_f32(const float* logits, const float* emb, int32_t* ids, uint8_t* committed, float* z,
                        float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n, int vocab, int d, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, d, 1);
  if (st != DG_OK) return st;
  if (d % 4 != 0) return fail(DG_EUNSUPPORTED, "sampler_f32: d_model must be a multiple of 4 for the float32 table");
  const dg::SamplerPlan p = dg::sampler_plan(n, 1, vocab, d);
  st = check_sampler_plan(p, "sampler_f32");
  if (st != DG_OK) return st;
  if (!ws || ws_bytes < p.total)
    return fail(DG_EWORKSPACE, "sampler_f32: workspace %zu < %zu bytes", ws_bytes, p.total);
  if (!aligned16(ws)) return fail(DG_EINVAL, "sampler_f32: workspace misaligned");
  dg::EbCall call{false, 0.f, 0.f, nullptr, nullptr, nullptr};
  call.emb_f32 = true;
  hipError_t e = dg::launch_sampler(p, logits, emb, ids, committed, z, conf, n_unc, ctrl, ws, stream, call);
  if (e != hipSuccess) return hip_fail(e, "sampler_f32 launch");
  return DG_OK;
}

int dg_sampler_step_eb(const float* logits, const void* emb, int32_t* ids, uint8_t* accepted,
                       float* z, float* entropy, int32_t* argmax, dg_eb_status* status,
                       dg_ctrl* ctrl, float budget, float stop_entropy, int n, int vocab, int d,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return dg_sampler_step_eb_batched(logits, emb, ids, accepted, z, entropy, argmax, status, ctrl, budget,
                                    stop_entropy, n, 1, vocab, d, ws, ws_bytes, stream);
}

int dg_sampler_step_eb_batched(const float* logits, const void* emb, int32_t* ids, uint8_t* accepted,
                               float* z, float* entropy, int32_t* argmax, dg_eb_status* status,
                               dg_ctrl* ctrl, float budget, float stop_entropy, int n, int batch,
                               int vocab, int d, void* ws, size_t ws_bytes, hipStream_t stream) {
  // n_uncommitted is not used in this mode; pass a non-null stand-in to the shared check
  int st = check_sampler(logits, emb, ids, accepted, z, reinterpret_cast<const uint32_t*>(status),
                         ctrl, n, vocab, d, batch);
  if (st != DG_OK) return st;
  if (!argmax || !status) return fail(DG_EINVAL, "sampler_eb: null argmax or status");
  if (!(budget >= 0.f) || !std::isfinite(budget)) return fail(DG_EINVAL, "sampler_eb: budget must be finite and >= 0");
  if (!(stop_entropy >= 0.f) || !std::isfinite(stop_entropy))
    return fail(DG_EINVAL, "sampler_eb: stop_entropy must be finite and >= 0");
  const dg::SamplerPlan p = dg::sampler_plan(n, batch, vocab, d);
  st = check_sampler_plan(p, "sampler_eb");
  if (st != DG_OK) return st;
  if (!ws || ws_bytes < p.total)
    return fail(DG_EWORKSPACE, "sampler_eb: workspace %zu < %zu bytes", ws_bytes, p.total);
  if (!aligned16(ws)) return fail(DG_EINVAL, "sampler_eb: workspace misaligned");
  const dg::EbCall eb{true, budget, stop_entropy, entropy, argmax, status};
  hipError_t e = dg::launch_sampler(p, logits, emb, ids, accepted, z, nullptr, nullptr, ctrl, ws, stream, eb);
  if (e != hipSuccess) return hip_fail(e, "sampler_eb launch");
  return DG_OK;
}

size_t dg_sampler_workspace_bytes_topk(int n, int batch, int vocab, int d, int k) {
  if (n < 1 || n > 256 || batch < 1 || batch > 4096 || vocab < 2 || d < 1 || k < 1 || k > 256) return 0;
  if ((int64_t)n * batch > dg::kMaxSamplerRows) return 0;
  return dg::topk_plan(n, batch, vocab, d, k).total;
}

int dg_sampler_step_topk(const float* logits, const float* emb, int32_t* ids, uint8_t* committed, float* z,
                         float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n, int batch, int vocab, int d,
                         int k, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, d, batch);
  if (st != DG_OK) return st;
  if (k < 1 || k > 256) return fail(k < 1 ? DG_EINVAL : DG_EUNSUPPORTED, "sampler_topk: top_k must be in [1, 256]");
  const dg::TopkPlan p = dg::topk_plan(n, batch, vocab, d, k);
  st = check_topk(k, p, ws, ws_bytes, "sampler_topk");
  if (st != DG_OK) return st;
  hipError_t e = dg::launch_sampler_topk(p, logits, emb, ids, committed, z, conf, n_unc, ctrl, ws, stream,
                                         dg::EbCall{false, 0.f, 0.f, nullptr, nullptr, nullptr});
  if (e != hipSuccess) return hip_fail(e, "sampler_topk launch");
  return DG_OK;
}

int dg_sampler_step_eb_topk(const float* logits, const float* emb, int32_t* ids, uint8_t* accepted, float* z,
                            float* entropy, int32_t* argmax, dg_eb_status* status, dg_ctrl* ctrl, float budget,
                            float stop_entropy, int n, int batch, int vocab, int d, int k, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  int st = check_sampler(logits, emb, ids, accepted, z, reinterpret_cast<const uint32_t*>(status), ctrl, n,
                         vocab, d, batch);
  if (st != DG_OK) return st;
  if (!argmax || !status) return fail(DG_EINVAL, "sampler_eb_topk: null argmax or status");
  if (!(budget >= 0.f) || !std::isfinite(budget))
    return fail(DG_EINVAL, "sampler_eb_topk: budget must be finite and >= 0");
  if (!(stop_entropy >= 0.f) || !std::isfinite(stop_entropy))
    return fail(DG_EINVAL, "sampler_eb_topk: stop_entropy must be finite and >= 0");
  if (k < 1 || k > 256)
    return fail(k < 1 ? DG_EINVAL : DG_EUNSUPPORTED, "sampler_eb_topk: top_k must be in [1, 256]");
  const dg::TopkPlan p = dg::topk_plan(n, batch, vocab, d, k);
  st = check_topk(k, p, ws, ws_bytes, "sampler_eb_topk");
  if (st != DG_OK) return st;
  const dg::EbCall eb{true, budget, stop_entropy, entropy, argmax, status};
  hipError_t e = dg::launch_sampler_topk(p, logits, emb, ids, accepted, z, nullptr, nullptr, ctrl, ws, stream, eb);
  if (e != hipSuccess) return hip_fail(e, "sampler_eb_topk launch");
  return DG_OK;
}

int dg_denoise_step(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                    float* attn_out, int np, int hq, int hkv, int d, int dtype, float scale,
                    const float* logits, const void* emb, int32_t* ids, uint8_t* committed,
                    float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n, int vocab, int dm,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dtype == DG_FP8_E4M3) return fail(DG_EUNSUPPORTED, "denoise: FP8 attention inputs take dg_canvas_attention_fp8");
  int st = check_attention(q, kp, vp, kc, vc, attn_out, n, np, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, dm);
  if (st != DG_OK) return st;
  st = check_sampler_plan(dg::sampler_plan(n, 1, vocab, dm), "denoise");
  if (st != DG_OK) return st;
  const size_t need = dg_denoise_workspace_bytes(n, np, hq, hkv, d, vocab, dm);
  if (!ws || ws_bytes < need) return fail(DG_EWORKSPACE, "denoise: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(ws)) return fail(DG_EINVAL, "denoise: workspace misaligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  const dg::AttnPlan ap = dg::attn_plan(n, np, hq, hkv, d);
  hipError_t e = dg::launch_attention(ap, q, kp, vp, kc, vc, attn_out, dtype, scale, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "denoise attention launch");
  const dg::SamplerPlan sp = dg::sampler_plan(n, 1, vocab, dm);
  e = dg::launch_sampler(sp, logits, emb, ids, committed, z, conf, n_unc, ctrl, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "denoise sampler launch");
  return DG_OK;
}

int dg_denoise_step_fp8(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                        float* attn_out, int np, int hq, int hkv, int d, float scale, float q_scale, float k_scale,
                        float v_scale, const float* logits, const void* emb, int32_t* ids, uint8_t* committed,
                        float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n, int vocab, int dm, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int st = check_attention(q, kp, vp, kc, vc, attn_out, n, np, hq, hkv, d, DG_FP8_E4M3);
  if (st != DG_OK) return st;
  if (!(q_scale > 0.f) || !std::isfinite(q_scale) || !(k_scale > 0.f) || !std::isfinite(k_scale) ||
      !(v_scale > 0.f) || !std::isfinite(v_scale))
    return fail(DG_EINVAL, "denoise_fp8: q_scale, k_scale and v_scale must be finite and > 0");
  st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, dm);
  if (st != DG_OK) return st;
  st = check_sampler_plan(dg::sampler_plan(n, 1, vocab, dm), "denoise_fp8");
  if (st != DG_OK) return st;
  const size_t need = dg_denoise_workspace_bytes(n, np, hq, hkv, d, vocab, dm);
  if (!ws || ws_bytes < need) return fail(DG_EWORKSPACE, "denoise_fp8: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(ws)) return fail(DG_EINVAL, "denoise_fp8: workspace misaligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  const dg::AttnPlan ap = dg::attn_plan(n, np, hq, hkv, d);
  hipError_t e = dg::launch_attention(ap, q, kp, vp, kc, vc, attn_out, DG_FP8_E4M3, scale * q_scale * k_scale, ws,
                                      stream, false, v_scale);
  if (e != hipSuccess) return hip_fail(e, "denoise_fp8 attention launch");
  const dg::SamplerPlan sp = dg::sampler_plan(n, 1, vocab, dm);
  e = dg::launch_sampler(sp, logits, emb, ids, committed, z, conf, n_unc, ctrl, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "denoise_fp8 sampler launch");
  return DG_OK;
}

int dg_denoise_step_eb(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                       float* attn_out, int np, int hq, int hkv, int d, int dtype, float scale,
                       const float* logits, const void* emb, int32_t* ids, uint8_t* accepted, float* z,
                       float* entropy, int32_t* argmax, dg_eb_status* status, dg_ctrl* ctrl, float budget,
                       float stop_entropy, int n, int vocab, int dm, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  if (dtype == DG_FP8_E4M3) return fail(DG_EUNSUPPORTED, "denoise_eb: FP8 attention inputs take dg_canvas_attention_fp8");
  int st = check_attention(q, kp, vp, kc, vc, attn_out, n, np, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  st = check_sampler(logits, emb, ids, accepted, z, reinterpret_cast<const uint32_t*>(status), ctrl, n, vocab, dm);
  if (st != DG_OK) return st;
  if (!argmax || !status) return fail(DG_EINVAL, "denoise_eb: null argmax or status");
  st = check_sampler_plan(dg::sampler_plan(n, 1, vocab, dm), "denoise_eb");
  if (st != DG_OK) return st;
  if (!(budget >= 0.f) || !std::isfinite(budget)) return fail(DG_EINVAL, "denoise_eb: budget must be finite and >= 0");
  if (!(stop_entropy >= 0.f) || !std::isfinite(stop_entropy))
    return fail(DG_EINVAL, "denoise_eb: stop_entropy must be finite and >= 0");
  const size_t need = dg_denoise_workspace_bytes(n, np, hq, hkv, d, vocab, dm);
  if (!ws || ws_bytes < need) return fail(DG_EWORKSPACE, "denoise_eb: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(ws)) return fail(DG_EINVAL, "denoise_eb: workspace misaligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)d);
  const dg::AttnPlan ap = dg::attn_plan(n, np, hq, hkv, d);
  hipError_t e = dg::launch_attention(ap, q, kp, vp, kc, vc, attn_out, dtype, scale, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "denoise_eb attention launch");
  const dg::SamplerPlan sp = dg::sampler_plan(n, 1, vocab, dm);
  const dg::EbCall eb{true, budget, stop_entropy, entropy, argmax, status};
  e = dg::launch_sampler(sp, logits, emb, ids, accepted, z, nullptr, nullptr, ctrl, ws, stream, eb);
  if (e != hipSuccess) return hip_fail(e, "denoise_eb sampler launch");
  return DG_OK;
}

struct dg_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

}  // extern "C"

namespace {
// Capture whatever `record` launches on a private stream into one graph.
template <typename F>
int capture_step(F record, dg_step_graph** out) {
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "graph: stream create");
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return hip_fail(e, "graph: begin capture");
  }
  g_capturing = true;
  const int st = record(cs);
  g_capturing = false;
  hipGraph_t graph = nullptr;
  hipError_t e2 = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (st != DG_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e2 != hipSuccess) return hip_fail(e2, "graph: end capture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return hip_fail(e, "graph: instantiate");
  }
  *out = new dg_step_graph{graph, exec};
  return DG_OK;
}
}  // namespace

extern "C" {

int dg_step_graph_create(const void* q, const void* kp, const void* vp, const void* kc,
                         const void* vc, float* attn_out, int np, int hq, int hkv, int d, int dtype,
                         float scale, const float* logits, const void* emb, int32_t* ids,
                         uint8_t* committed, float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl,
                         int n, int vocab, int dm, void* ws, size_t ws_bytes, dg_step_graph** out) {
  if (!out) return fail(DG_EINVAL, "graph: null output handle");
  *out = nullptr;
  int st = check_attention(q, kp, vp, kc, vc, attn_out, n, np, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, dm);
  if (st != DG_OK) return st;
  st = check_sampler_plan(dg::sampler_plan(n, 1, vocab, dm), "graph");
  if (st != DG_OK) return st;
  return capture_step([&](hipStream_t cs) {
    return dg_denoise_step(q, kp, vp, kc, vc, attn_out, np, hq, hkv, d, dtype, scale, logits, emb, ids,
                           committed, z, conf, n_unc, ctrl, n, vocab, dm, ws, ws_bytes, cs);
  }, out);
}

int dg_step_graph_create_fp8(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                             float* attn_out, int np, int hq, int hkv, int d, float scale, float q_scale,
                             float k_scale, float v_scale, const float* logits, const void* emb, int32_t* ids,
                             uint8_t* committed, float* z, float* conf, uint32_t* n_unc, dg_ctrl* ctrl, int n,
                             int vocab, int dm, void* ws, size_t ws_bytes, dg_step_graph** out) {
  if (!out) return fail(DG_EINVAL, "graph: null output handle");
  *out = nullptr;
  int st = check_attention(q, kp, vp, kc, vc, attn_out, n, np, hq, hkv, d, DG_FP8_E4M3);
  if (st != DG_OK) return st;
  st = check_sampler(logits, emb, ids, committed, z, n_unc, ctrl, n, vocab, dm);
  if (st != DG_OK) return st;
  st = check_sampler_plan(dg::sampler_plan(n, 1, vocab, dm), "graph_fp8");
  if (st != DG_OK) return st;
  return capture_step([&](hipStream_t cs) {
    return dg_denoise_step_fp8(q, kp, vp, kc, vc, attn_out, np, hq, hkv, d, scale, q_scale, k_scale, v_scale, logits,
                               emb, ids, committed, z, conf, n_unc, ctrl, n, vocab, dm, ws, ws_bytes, cs);
  }, out);
}

int dg_step_graph_create_eb(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                            float* attn_out, int np, int hq, int hkv, int d, int dtype, float scale,
                            const float* logits, const void* emb, int32_t* ids, uint8_t* accepted, float* z,
                            float* entropy, int32_t* argmax, dg_eb_status* status, dg_ctrl* ctrl, float budget,
                            float stop_entropy, int n, int vocab, int dm, void* ws, size_t ws_bytes,
                            dg_step_graph** out) {
  if (!out) return fail(DG_EINVAL, "graph: null output handle");
  *out = nullptr;
  int st = check_attention(q, kp, vp, kc, vc, attn_out, n, np, hq, hkv, d, dtype);
  if (st != DG_OK) return st;
  st = check_sampler(logits, emb, ids, accepted, z, reinterpret_cast<const uint32_t*>(status), ctrl, n, vocab, dm);
  if (st != DG_OK) return st;
  st = check_sampler_plan(dg::sampler_plan(n, 1, vocab, dm), "graph_eb");
  if (st != DG_OK) return st;
  return capture_step([&](hipStream_t cs) {
    return dg_denoise_step_eb(q, kp, vp, kc, vc, attn_out, np, hq, hkv, d, dtype, scale, logits, emb, ids,
                              accepted, z, entropy, argmax, status, ctrl, budget, stop_entropy, n, vocab, dm,
                              ws, ws_bytes, cs);
  }, out);
}

int dg_step_graph_launch(dg_step_graph* g, hipStream_t stream) {
  if (!g) return fail(DG_EINVAL, "graph: null handle");
  hipError_t e = hipGraphLaunch(g->exec, stream);
  if (e != hipSuccess) return hip_fail(e, "graph launch");
  return DG_OK;
}

void dg_step_graph_destroy(dg_step_graph* g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

size_t dg_embedding_packed_bytes(int vocab, int d) {
  if (vocab < 2 || d < 1) return 0;
  return dg::embedding_packed_bytes(vocab, d);
}

int dg_embedding_pack(const float* emb, void* packed, int vocab, int d, hipStream_t stream) {
  if (!emb || !packed) return fail(DG_EINVAL, "embedding_pack: null pointer");
  if (vocab < 2 || d < 1) return fail(DG_EINVAL, "embedding_pack: bad sizes");
  if (dg::embedding_packed_bytes(vocab, d) >= (1ull << 40)) return fail(DG_EINVAL, "embedding_pack: E too large");
  if (!aligned16(packed)) return fail(DG_EINVAL, "embedding_pack: output misaligned");
  hipError_t e = dg::launch_embedding_pack(emb, packed, vocab, d, stream);
  if (e != hipSuccess) return hip_fail(e, "embedding_pack launch");
  return DG_OK;
}

int dg_canvas_init(int32_t* ids, uint8_t* committed, dg_ctrl* ctrl, int n, int vocab,
                   hipStream_t stream) {
  if (!ids || !committed || !ctrl) return fail(DG_EINVAL, "canvas_init: null pointer");
  if (n < 1) return fail(DG_EINVAL, "canvas_init: n_canvas < 1");
  if (n > 256) return fail(DG_EUNSUPPORTED, "canvas_init: n_canvas > 256");
  if (vocab < 2) return fail(DG_EINVAL, "canvas_init: vocab < 2");
  hipError_t e = dg::launch_canvas_init(ids, committed, ctrl, n, vocab, stream);
  if (e != hipSuccess) return hip_fail(e, "canvas_init launch");
  return DG_OK;
}

int dg_kv_append(void* kp, void* vp, const void* kc, const void* vc, int np, int capacity, int n, int hkv,
                 int d, int dtype, hipStream_t stream) {
  if (!kp || !vp || !kc || !vc) return fail(DG_EINVAL, "kv_append: null pointer");
  if (np < 0 || n < 1 || hkv < 1 || d < 1) return fail(DG_EINVAL, "kv_append: bad sizes");
  if ((int64_t)np + n > (int64_t)capacity)
    return fail(DG_EINVAL, "kv_append: n_prefix %d + n_canvas %d exceeds the prefix capacity of %d rows", np, n,
                capacity);
  if (dtype != DG_F32 && dtype != DG_BF16) return fail(DG_EUNSUPPORTED, "kv_append: dtype");
  const size_t es = dtype == DG_BF16 ? 2 : 4;
  const size_t row = (size_t)hkv * d * es;
  const size_t off = (size_t)np * row;
  const size_t bytes = (size_t)n * row;
  hipError_t e = hipMemcpyAsync(static_cast<uint8_t*>(kp) + off, kc, bytes, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(static_cast<uint8_t*>(vp) + off, vc, bytes, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "kv_append copy");
  return DG_OK;
}

int dg_synth_logits(float* logits, const int32_t* ids, const uint8_t* committed, const dg_ctrl* ctrl,
                    const float* table, int table_size, int n, int vocab, hipStream_t stream) {
  if (!logits || !ids || !committed || !ctrl || !table) return fail(DG_EINVAL, "synth: null pointer");
  if (table_size != 65536) return fail(DG_EINVAL, "synth: table_size must be 65536");
  if (n < 1) return fail(DG_EINVAL, "synth: n_canvas < 1");
  if (n > 256) return fail(DG_EUNSUPPORTED, "synth: n_canvas > 256");
  if (vocab < 2) return fail(DG_EINVAL, "synth: vocab < 2");
  if (!aligned16(logits)) return fail(DG_EINVAL, "synth: logits misaligned");
  hipError_t e = dg::launch_synth_logits(logits, ids, committed, ctrl, table, table_size, n, vocab, stream);
  if (e != hipSuccess) return hip_fail(e, "synth launch");
  return DG_OK;
}

int dg_philox_fill(uint32_t* out, size_t n_words, uint64_t seed, uint32_t c1, uint32_t c2,
                   uint32_t c3, hipStream_t stream) {
  if (!out) return fail(DG_EINVAL, "philox_fill: null pointer");
  if (n_words % 4 != 0) return fail(DG_EINVAL, "philox_fill: n_words must be a multiple of 4");
  if (n_words / 4 > 0xFFFFFFFFull) return fail(DG_EINVAL, "philox_fill: too many counters");
  if (!aligned16(out)) return fail(DG_EINVAL, "philox_fill: output misaligned");
  hipError_t e = dg::launch_philox_fill(out, n_words, seed, c1, c2, c3, stream);
  if (e != hipSuccess) return hip_fail(e, "philox_fill launch");
  return DG_OK;
}

int dg_probe_mfma_bf16(float* sink, int n_workgroups, int iters, hipStream_t stream) {
  if (!sink) return fail(DG_EINVAL, "probe_mfma: null sink");
  if (n_workgroups < 1 || n_workgroups > 65535 || iters < 1)
    return fail(DG_EINVAL, "probe_mfma: n_workgroups must be in [1, 65535] and iters >= 1");
  hipError_t e = dg::launch_probe_mfma(sink, n_workgroups, iters, stream);
  if (e != hipSuccess) return hip_fail(e, "probe_mfma launch");
  return DG_OK;
}

int dg_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!dst || !src) return fail(DG_EINVAL, "probe_copy: null pointer");
  if (bytes % 16 != 0) return fail(DG_EINVAL, "probe_copy: bytes must be a multiple of 16");
  if (!aligned16(dst) || !aligned16(src)) return fail(DG_EINVAL, "probe_copy: pointers must be 16-byte aligned");
  hipError_t e = dg::launch_probe_copy(dst, src, bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "probe_copy launch");
  return DG_OK;
}

int dg_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return fail(DG_EINVAL, "probe_read: null pointer");
  if (bytes % 16 != 0) return fail(DG_EINVAL, "probe_read: bytes must be a multiple of 16");
  if (!aligned16(src)) return fail(DG_EINVAL, "probe_read: src must be 16-byte aligned");
  hipError_t e = dg::launch_probe_read(src, bytes, sink, stream);
  if (e != hipSuccess) return hip_fail(e, "probe_read launch");
  return DG_OK;
}

int dg_profile_enable(int on) {
  g_prof_on = on != 0;
  return DG_OK;
}

int dg_profile_read(const char** names, double* total_ms, int* counts, int max) {
  std::vector<const char*> keys;
  std::vector<double> sums;
  std::vector<int> cnt;
  for (const ProfRec& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess) continue;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) continue;
    size_t k = 0;
    while (k < keys.size() && std::strcmp(keys[k], r.name) != 0) ++k;
    if (k == keys.size()) {
      keys.push_back(r.name);
      sums.push_back(0.0);
      cnt.push_back(0);
    }
    sums[k] += ms;
    cnt[k] += 1;
  }
  for (const ProfRec& r : g_prof_recs) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  int w = 0;
  for (size_t k = 0; k < keys.size() && w < max; ++k, ++w) {
    if (names) names[w] = keys[k];
    if (total_ms) total_ms[w] = sums[k];
    if (counts) counts[w] = cnt[k];
  }
  return w;
}

}  // extern "C"
