/*
 * dg.h - C ABI of the MI355X (gfx950) canvas-denoising kernels for block text
 * diffusion.
 *
 * One denoising step makes two passes over a canvas of up to 256 token slots:
 *   1. bidirectional canvas attention over the committed KV prefix plus every
 *      canvas position (DiffusionGemma Technical Report part 4/6, section 6,
 *      "Attention"; section 9.1);
 *   2. the diffusion sampler: a full-vocabulary softmax per canvas position, the
 *      self-conditioning product softmax(logits)·E, and confidence commit with
 *      uniform re-noise of the other positions (Technical Report section 6,
 *      "Sampling"; explainer "DiffusionGemma: Google's open diffusion LLM",
 *      sections quoting report 3.1-3.3; AlphaSignal page "How text diffusion
 *      actually works").
 * The whole step can be captured into one HIP graph so the host never
 * synchronises between the passes (Technical Report section 6, "Eliminating
 * CPU-GPU synchronization").
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise.  Tensors are dense,
 *     row-major, and 16-byte aligned.  The caller owns every buffer, including
 *     the workspace; the library never allocates, frees or synchronises inside
 *     dg_canvas_attention / dg_sampler_step / dg_denoise_step.
 *   - Work is enqueued asynchronously on `stream`; results are ready when the
 *     stream reaches that point.  Calls are capture-safe and deterministic
 *     (fixed reduction order, no floating-point atomics).
 *   - Arguments are validated on the host before any HIP call; on a validation
 *     error nothing is launched and a negative dg_status is returned.
 *     dg_last_error() gives a thread-local detail string.  A HIP launch error
 *     maps to DG_EHIP.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_OK = 0,
  DG_EINVAL = -1,        /* null / misaligned pointer, bad size */
  DG_EUNSUPPORTED = -2,  /* valid but not supported (head_dim, dtype, n_canvas > 256) */
  DG_EWORKSPACE = -3,    /* workspace smaller than the *_workspace_bytes query */
  DG_EHIP = -4           /* a HIP runtime call or launch failed */
} dg_status;

typedef enum dg_dtype { DG_F32 = 0, DG_BF16 = 1, DG_FP8_E4M3 = 2 } dg_dtype;

/* dg_ctrl.flags */
enum {
  DG_GUMBEL = 1u,       /* candidate = argmax(l/T + Gumbel noise); else greedy argmax */
  DG_COMMIT_ONLY = 2u,  /* commit confident positions, do not re-noise the others */
  DG_AUTO_ADVANCE = 4u, /* the step ends with gstep += 1, s_in_block += 1 on the device */
  DG_T_SCHEDULE = 8u    /* T = t_start + (t_end - t_start) * s_in_block / (s_max - 1) */
};

/*
 * Sampler control block.  It lives in DEVICE memory so a captured step graph can
 * be replayed: every kernel reads it, and (with DG_AUTO_ADVANCE) the last kernel
 * of a sampler step advances the step counters.  Table 2 of the explainer
 * ("Sampler settings that decide DiffusionGemma latency") gives the recommended
 * 48-step budget and the 0.8 -> 0.4 linear temperature schedule.
 *   seed        key of the counter-based generator (Philox4x32-10)
 *   gstep       global step index, part of every random draw's counter
 *   s_in_block  step index within the current canvas (temperature schedule, cap)
 *   s_max       step budget of a canvas; on step s_in_block + 1 >= s_max every
 *               remaining defined position commits its candidate
 *   tau         commit threshold on the candidate's probability at temperature T
 */
typedef struct dg_ctrl {
  uint64_t seed;
  uint32_t gstep;
  uint32_t s_in_block;
  uint32_t s_max;
  uint32_t flags;
  float tau;
  float t_start;
  float t_end;
  uint32_t reserved;
} dg_ctrl;

/* ------------------------------------------------------------------------ */
/* Canvas attention                                                          */
/* ------------------------------------------------------------------------ */

/* Workspace bytes dg_canvas_attention needs for these sizes (0 if invalid). */
size_t dg_attention_workspace_bytes(int n_canvas, int n_prefix, int hq, int hkv, int head_dim);

/*
 * Bidirectional canvas attention (Technical Report section 6 "Attention"):
 *   O[i,h] = sum_j softmax_j(scale * q[i,h] . k_j) v_j
 * over keys j = prefix rows 0..n_prefix-1 then canvas rows 0..n_canvas-1 of KV
 * head h / (hq / hkv); no mask.
 *   q          [n_canvas, hq, head_dim]     dtype
 *   k_prefix   [n_prefix, hkv, head_dim]    dtype (NULL allowed iff n_prefix == 0)
 *   v_prefix   [n_prefix, hkv, head_dim]    dtype (NULL allowed iff n_prefix == 0)
 *   k_canvas   [n_canvas, hkv, head_dim]    dtype
 *   v_canvas   [n_canvas, hkv, head_dim]    dtype
 *   out        [n_canvas, hq, head_dim]     float32 (written)
 *   n_canvas in [1, 256]; n_prefix >= 0; hq % hkv == 0; head_dim in {64, 128}.
 *   dtype DG_BF16 or DG_F32 (float32 inputs are rounded to bf16 when staged;
 *   products and the softmax accumulate in float32).  FP8 inputs take
 *   dg_canvas_attention_fp8 (DG_FP8_E4M3 here returns DG_EINVAL).
 *   scale <= 0 selects 1/sqrt(head_dim).
 */
int dg_canvas_attention(const void* q, const void* k_prefix, const void* v_prefix,
                        const void* k_canvas, const void* v_canvas, float* out,
                        int n_canvas, int n_prefix, int hq, int hkv, int head_dim,
                        int dtype, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Canvas attention with options (attn_flags, 0 = dg_canvas_attention).
 *   DG_ATTN_CAUSAL   canvas row i attends to every prefix key and to canvas
 *                    keys 0..i only: the KV-update pass, in which a finished
 *                    canvas is written into the cache as causal history
 *                    (explainer "DiffusionGemma: Google's open diffusion LLM",
 *                    section "Block-autoregressive generation, one canvas
 *                    after another": a causal encoder reads the history).
 * Other arguments, workspace and errors as dg_canvas_attention; unknown flag
 * bits return DG_EINVAL.
 */
enum { DG_ATTN_CAUSAL = 1u };
int dg_canvas_attention_ex(const void* q, const void* k_prefix, const void* v_prefix,
                           const void* k_canvas, const void* v_canvas, float* out,
                           int n_canvas, int n_prefix, int hq, int hkv, int head_dim,
                           int dtype, float scale, uint32_t attn_flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dg_canvas_attention_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of dg_static_scratch_bytes() bytes (64 MiB) inside the library; each GPU
 * holds its own copy from the first call on it until the process ends.  Inputs,
 * output, flags, results and errors as dg_canvas_attention_ex; sizes whose
 * workspace (dg_attention_workspace_bytes) exceeds the static scratch return
 * DG_EUNSUPPORTED before any HIP call.  The call allocates nothing.  Every
 * call on one GPU shares that GPU's scratch: calls that overlap in time on one
 * GPU (several streams or threads) race and must be serialised by the caller.
 */
size_t dg_static_scratch_bytes(void);
int dg_canvas_attention_noalloc(const void* q, const void* k_prefix, const void* v_prefix,
                                const void* k_canvas, const void* v_canvas, float* out,
                                int n_canvas, int n_prefix, int hq, int hkv, int head_dim,
                                int dtype, float scale, uint32_t attn_flags, hipStream_t stream);

/*
 * A batch of sequences in one launch, each with its own prefix length and its
 * own causal flag, so denoising passes and KV-update passes can share a batch
 * (Technical Report part 4/6, paragraph "Eliminating CPU-GPU synchronization":
 * both kinds of forward pass, with different attention masks, can occur in one
 * batch; explainer "DiffusionGemma: Google's open diffusion LLM", section
 * "Reference implementations in Transformers and vLLM": a per-sequence causal
 * flag).  Sequence s computes exactly what dg_canvas_attention_ex computes for
 * its own inputs:
 *   q          [batch, n_canvas, hq, head_dim]          dtype
 *   k_prefix   [batch, prefix_stride, hkv, head_dim]    dtype; sequence s uses
 *   v_prefix   rows 0..n_prefix[s]-1 of its slab and never reads the rest
 *              (NULL allowed iff prefix_stride == 0)
 *   k_canvas   [batch, n_canvas, hkv, head_dim]         dtype
 *   v_canvas   [batch, n_canvas, hkv, head_dim]         dtype
 *   out        [batch, n_canvas, hq, head_dim]          float32 (written)
 *   n_prefix   host array [batch], each in [0, prefix_stride]; read during the
 *              call only
 *   causal     host array [batch] of 0/1 (DG_ATTN_CAUSAL semantics for a 1),
 *              or NULL for all bidirectional; read during the call only
 *   batch in [1, 64]; dtype DG_BF16 or DG_F32 (DG_FP8_E4M3 returns
 *   DG_EUNSUPPORTED); the other sizes and scale as dg_canvas_attention.
 * Workspace: dg_attention_batched_workspace_bytes (0 if the sizes are
 * invalid).  Errors: DG_EINVAL for a null pointer, a misaligned pointer, an
 * n_prefix entry outside [0, prefix_stride] or a causal entry other than 0/1,
 * DG_EUNSUPPORTED for batch > 64 or hkv * batch > 65535, DG_EWORKSPACE if the
 * workspace is too small; nothing is launched on an error.
 */
size_t dg_attention_batched_workspace_bytes(int batch, int n_canvas, int prefix_stride, int hq, int hkv,
                                            int head_dim);
int dg_canvas_attention_batched(const void* q, const void* k_prefix, const void* v_prefix,
                                const void* k_canvas, const void* v_canvas, float* out,
                                const int32_t* n_prefix, const uint8_t* causal, int batch,
                                int n_canvas, int prefix_stride, int hq, int hkv, int head_dim,
                                int dtype, float scale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * FP8 canvas attention: the pages' timings are taken in FP8 (explainer
 * "DiffusionGemma: Google's open diffusion LLM", section "Throughput flips at
 * about 32 concurrent users", Figure 12 caption).  q, k_prefix, v_prefix,
 * k_canvas and v_canvas are OCP FP8 E4M3 bytes (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN) in the layouts of
 * dg_canvas_attention; the real values are q_scale * q, k_scale * k and
 * v_scale * v.  The scores q.k run on the FP8 matrix cores
 * (v_mfma_f32_32x32x64_f8f6f4: E4M3 products are exact in float32, summed in
 * float32); V is converted exactly to bf16 when staged and P.V runs on bf16
 * (P rounded to bf16, float32 softmax and accumulation).  The K/V bytes read
 * are half those of bf16.  The scales must be finite and > 0.  attn_flags, scale,
 * workspace (dg_attention_workspace_bytes) and errors as dg_canvas_attention_ex.
 */
int dg_canvas_attention_fp8(const void* q, const void* k_prefix, const void* v_prefix,
                            const void* k_canvas, const void* v_canvas, float* out,
                            int n_canvas, int n_prefix, int hq, int hkv, int head_dim,
                            float scale, float q_scale, float k_scale, float v_scale,
                            uint32_t attn_flags, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Diffusion sampler                                                         */
/* ------------------------------------------------------------------------ */

/* Workspace bytes dg_sampler_step needs for these sizes (0 if invalid). */
size_t dg_sampler_workspace_bytes(int n_canvas, int vocab, int d_model);

/*
 * The embedding table E in the layout the sampler streams.  The contraction
 * z = softmax(logits)·E runs on fp16 and fp6 matrix cores in split precision.
 * Each row k is held at its own scale, Q_k = E_k·2^(c + d_k): c brings
 * max|E|·2^c into [2^7, 2^8) and the row shift d_k (0-40) brings row k's own
 * maximum there too (zero rows take 40).  Each element is held as
 * Q16 = fp16(Q) plus an e2m3 (fp6) code of (Q - Q16)·2^11 under a power-of-two
 * scale shared by 16 ids and 64 columns (3 bytes per element; the contraction
 * forms the codes of Q16 itself), so E is converted once, when the weights are
 * loaded, rather than on every step:
 *   emb        [vocab, d_model] float32 (input)
 *   packed     dg_embedding_packed_bytes(vocab, d_model) bytes (output).  Ids
 *              are grouped in blocks of 16 and the blocks in pairs (ids past
 *              vocab are zero); columns in tiles of 256 (d_model rounded up,
 *              zero padded).  For pair j and tile t, a 24576-byte block at
 *              (j·n_tiles + t)·24576: the 256 columns' fp16 Q16 of the pair's
 *              first 16 ids (32 bytes per column, id order), the same for the
 *              second 16 ids, then per column 16 bytes for the first block and
 *              16 for the second: 12 bytes of e2m3 codes (code i at bits
 *              6i..6i+5, little-endian), the scale byte 127 + eB (the codes are
 *              of (Q - Q16)·2^11 / 2^eB, eB the smallest exponent, at least
 *              -126, with the block's and 64-column group's largest |Q - Q16|·2^11
 *              and |Q16| at most 7.5·2^eB; nearest, ties to the even code) and
 *              three zero bytes.  After the blocks: the row shifts d_k, one
 *              byte per id of the whole block pairs (ids past vocab: 40),
 *              padded to a multiple of 256 bytes; 4096 bytes the pack uses as
 *              working space; a 256-byte record: float 2^-(14 + c), int32 c.
 * E is expected finite: a non-finite entry makes z undefined (c = 0 then; a
 * zero table also gives c = 0).  c is at most 80; below max|E| = 2^-72 the
 * row shifts carry the rest, which keeps full precision down to about 2^-90
 * (further down the shifted weights leave fp16's normal range).  Rows more
 * than 2^40 below the largest keep fewer bits.  The caller owns both buffers.
 * Asynchronous on `stream`.
 */
size_t dg_embedding_packed_bytes(int vocab, int d_model);
int dg_embedding_pack(const float* emb, void* packed, int vocab, int d_model, hipStream_t stream);

/*
 * One sampler step over the canvas (Technical Report section 6 "Sampling").
 *   logits          [n_canvas, vocab]   float32
 *   emb_packed      the embedding table E [vocab, d_model] as written by
 *                   dg_embedding_pack
 *   canvas_ids      [n_canvas]          int32, in/out
 *   committed       [n_canvas]          uint8 0/1, in/out (a committed position is
 *                                       never changed again)
 *   selfcond        [n_canvas, d_model] float32 out: z = softmax(logits) · E for
 *                                       every row (temperature 1)
 *   confidence      [n_canvas]          float32 out, may be NULL: probability at
 *                                       temperature T of the row's candidate
 *   n_uncommitted   [1]                 uint32 out: positions still open after the step
 *   ctrl            device dg_ctrl, in (and advanced with DG_AUTO_ADVANCE)
 * For each open position: commit the candidate if confidence >= tau (or on the
 * last step of the budget), else, unless DG_COMMIT_ONLY, replace its id with a
 * uniform draw over [0, vocab).  A row holding a NaN or +inf, or no finite
 * logit, gets confidence NaN and z NaN and is never committed.
 *   n_canvas in [1, 256]; vocab >= 2 with n_canvas * vocab * 4 < 2^32; d_model >= 1.
 */
int dg_sampler_step(const float* logits, const void* emb_packed, int32_t* canvas_ids,
                    uint8_t* committed, float* selfcond, float* confidence,
                    uint32_t* n_uncommitted, dg_ctrl* ctrl,
                    int n_canvas, int vocab, int d_model,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dg_sampler_step on the plain float32 embedding table instead of the packed
 * image:
 *   emb             [vocab, d_model] float32, row-major, 16-byte aligned
 * The contraction splits each element of E into a bf16 pair (E_hi = bf16(E),
 * E_lo = bf16(E - E_hi)) while it streams and sums p_hi E_hi + p_hi E_lo +
 * p_lo E_hi.  Ids, commit mask, confidence, counts and ctrl equal
 * dg_sampler_step's bit for bit (they come from the same statistics pass); z
 * meets the same bound by another rounding.  d_model must be a multiple of 4
 * (DG_EUNSUPPORTED otherwise).  Other arguments, workspace
 * (dg_sampler_workspace_bytes) and errors as dg_sampler_step.
 */
int dg_sampler_step_f32(const float* logits, const float* emb, int32_t* canvas_ids,
                        uint8_t* committed, float* selfcond, float* confidence,
                        uint32_t* n_uncommitted, dg_ctrl* ctrl,
                        int n_canvas, int vocab, int d_model,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Entropy-bounded sampler step: the pages' default sampler (explainer
 * "DiffusionGemma: Google's open diffusion LLM", section "A diffusion language
 * model refines 256 tokens in 12 steps" and Table 2 "Sampler settings that
 * decide DiffusionGemma latency").
 *   logits, emb_packed, canvas_ids, selfcond, ctrl, sizes: as dg_sampler_step
 *   accepted        [n_canvas] uint8 out: 1 where this step accepted the candidate
 *   entropy         [n_canvas] float32 out, may be NULL: entropy (nats) of the
 *                   temperature-T distribution, NaN for undefined rows
 *   argmax          [n_canvas] int32 in/out: in, the previous step's greedy argmax
 *                   ids (any value that cannot match, e.g. -1, before the first
 *                   step of a canvas); out, this step's
 *   status          device dg_eb_status out
 *   budget          entropy budget (0.1 in Table 2), stop_entropy the adaptive
 *                   stopping threshold on the mean entropy (0.005)
 * The defined rows are ranked by (entropy, position); rank k is accepted when
 * the running sum of the first k + 1 entropies is <= budget, and rank 0 always.
 * Accepted positions take their candidate (greedy, or Gumbel with DG_GUMBEL);
 * every other position gets a uniform re-noise draw, whatever it held before
 * (tokens of the open canvas stay editable).  On the last step of the budget
 * every defined row is accepted.  When the mean entropy of the defined rows is
 * below stop_entropy and the greedy ids equal the incoming argmax, status.stop
 * is set and canvas_ids become the greedy ids.  DG_COMMIT_ONLY is ignored.
 */
typedef struct dg_eb_status {
  uint32_t n_accepted;   /* positions accepted this step */
  uint32_t stop;         /* 1: adaptive stopping fired, the canvas is final */
  float mean_entropy;    /* mean entropy of the defined rows (NaN if none) */
  uint32_t n_defined;    /* rows with a defined distribution */
} dg_eb_status;

int dg_sampler_step_eb(const float* logits, const void* emb_packed, int32_t* canvas_ids,
                       uint8_t* accepted, float* selfcond, float* entropy, int32_t* argmax,
                       dg_eb_status* status, dg_ctrl* ctrl, float budget, float stop_entropy,
                       int n_canvas, int vocab, int d_model,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * A batch of canvases in one sampler pass: `batch` independent canvases of
 * n_canvas positions each (independent requests), whose logits, ids, masks,
 * selfcond and confidence rows are stacked canvas after canvas
 * ([batch * n_canvas, ...]).  Each canvas has its own control block
 * (ctrl[batch], device) and open-position count (n_uncommitted[batch]); its
 * random draws use its own seed and step and the position within the canvas,
 * so canvas b's results are exactly those of dg_sampler_step on canvas b
 * alone.  The batch shares one pass over the embedding table, which raises
 * the contraction's arithmetic intensity by `batch`.
 *   batch in [1, 4096]; n_canvas * batch * vocab * 4 < 2^32; n_canvas * batch <= 65535
 *   (DG_EUNSUPPORTED otherwise).
 */
size_t dg_sampler_workspace_bytes_batched(int n_canvas, int batch, int vocab, int d_model);
int dg_sampler_step_batched(const float* logits, const void* emb_packed, int32_t* canvas_ids,
                            uint8_t* committed, float* selfcond, float* confidence,
                            uint32_t* n_uncommitted, dg_ctrl* ctrl,
                            int n_canvas, int batch, int vocab, int d_model,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
/* Entropy-bounded step over a batch (status[batch], argmax rows stacked). */
int dg_sampler_step_eb_batched(const float* logits, const void* emb_packed, int32_t* canvas_ids,
                               uint8_t* accepted, float* selfcond, float* entropy, int32_t* argmax,
                               dg_eb_status* status, dg_ctrl* ctrl, float budget, float stop_entropy,
                               int n_canvas, int batch, int vocab, int d_model,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Top-k truncated sampler steps (approximate sampler).  The pages expect
 * truncating the sampling step to the top k tokens to raise throughput at
 * larger batches with negligible effect on quality (explainer "DiffusionGemma:
 * Google's open diffusion LLM", section "Throughput flips at about 32
 * concurrent users").  Per row the kept set S holds the top_k largest logits,
 * ties going to the smaller id; every other logit counts as -inf, and the step
 * is then exactly dg_sampler_step_batched (threshold commit) or
 * dg_sampler_step_eb_batched (entropy-bounded) on those truncated logits:
 * softmax, z, candidate (greedy, or Gumbel within S), confidence and entropy
 * are those of the truncated row.  Rows holding a NaN or +inf, or no finite
 * logit, stay undefined.  Since z only needs the rows of E in S, these calls
 * take the plain fp32 table:
 *   emb             [vocab, d_model] float32, row-major (not the packed image)
 *   top_k           in [1, 256]; top_k >= vocab keeps every id (untruncated)
 *   other arguments as in the batched calls above.
 * Limits: n_canvas in [1, 256], batch in [1, 4096], n_canvas * batch <= 65535,
 * n_canvas * batch * vocab * 4 < 2^32, and ceil(vocab / 4096) * top_k <= 16384.
 */
size_t dg_sampler_workspace_bytes_topk(int n_canvas, int batch, int vocab, int d_model, int top_k);
int dg_sampler_step_topk(const float* logits, const float* emb, int32_t* canvas_ids,
                         uint8_t* committed, float* selfcond, float* confidence,
                         uint32_t* n_uncommitted, dg_ctrl* ctrl,
                         int n_canvas, int batch, int vocab, int d_model, int top_k,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);
int dg_sampler_step_eb_topk(const float* logits, const float* emb, int32_t* canvas_ids,
                            uint8_t* accepted, float* selfcond, float* entropy, int32_t* argmax,
                            dg_eb_status* status, dg_ctrl* ctrl, float budget, float stop_entropy,
                            int n_canvas, int batch, int vocab, int d_model, int top_k,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Whole denoising step and its graph                                        */
/* ------------------------------------------------------------------------ */

size_t dg_denoise_workspace_bytes(int n_canvas, int n_prefix, int hq, int hkv, int head_dim,
                                  int vocab, int d_model);

/*
 * Attention then sampler, serialised on one stream, one shared workspace
 * (arguments as in the two calls above).
 */
int dg_denoise_step(const void* q, const void* k_prefix, const void* v_prefix,
                    const void* k_canvas, const void* v_canvas, float* attn_out,
                    int n_prefix, int hq, int hkv, int head_dim, int dtype, float scale,
                    const float* logits, const void* emb_packed, int32_t* canvas_ids,
                    uint8_t* committed, float* selfcond, float* confidence,
                    uint32_t* n_uncommitted, dg_ctrl* ctrl,
                    int n_canvas, int vocab, int d_model,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same step with the entropy-bounded sampler (the pages' default):
 * attention, then dg_sampler_step_eb, on one stream with one workspace
 * (dg_denoise_workspace_bytes).  Sampler arguments as dg_sampler_step_eb.
 */
int dg_denoise_step_eb(const void* q, const void* k_prefix, const void* v_prefix,
                       const void* k_canvas, const void* v_canvas, float* attn_out,
                       int n_prefix, int hq, int hkv, int head_dim, int dtype, float scale,
                       const float* logits, const void* emb_packed, int32_t* canvas_ids,
                       uint8_t* accepted, float* selfcond, float* entropy, int32_t* argmax,
                       dg_eb_status* status, dg_ctrl* ctrl, float budget, float stop_entropy,
                       int n_canvas, int vocab, int d_model,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The step with FP8 attention inputs: dg_canvas_attention_fp8 (E4M3 Q/K/V with
 * per-tensor scales, the scores on the FP8 matrix cores) then dg_sampler_step,
 * on one stream with one workspace (dg_denoise_workspace_bytes).  The pages'
 * timings are taken in FP8 (explainer "DiffusionGemma: Google's open diffusion
 * LLM", section "Throughput flips at about 32 concurrent users", Figure 12
 * caption).  Attention arguments as dg_canvas_attention_fp8 (bidirectional),
 * sampler arguments as dg_sampler_step; the scales must be finite and > 0.
 */
int dg_denoise_step_fp8(const void* q, const void* k_prefix, const void* v_prefix,
                        const void* k_canvas, const void* v_canvas, float* attn_out,
                        int n_prefix, int hq, int hkv, int head_dim, float scale,
                        float q_scale, float k_scale, float v_scale,
                        const float* logits, const void* emb_packed, int32_t* canvas_ids,
                        uint8_t* committed, float* selfcond, float* confidence,
                        uint32_t* n_uncommitted, dg_ctrl* ctrl,
                        int n_canvas, int vocab, int d_model,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

typedef struct dg_step_graph dg_step_graph;

/*
 * Capture dg_denoise_step (same arguments) into an instantiated HIP graph.  The
 * handle is written to *graph.  Replays re-read ctrl from device memory, so one
 * graph serves every step of a canvas whose n_prefix is fixed.  Creation
 * allocates host-side graph objects and is not for the hot path.
 */
int dg_step_graph_create(const void* q, const void* k_prefix, const void* v_prefix,
                         const void* k_canvas, const void* v_canvas, float* attn_out,
                         int n_prefix, int hq, int hkv, int head_dim, int dtype, float scale,
                         const float* logits, const void* emb_packed, int32_t* canvas_ids,
                         uint8_t* committed, float* selfcond, float* confidence,
                         uint32_t* n_uncommitted, dg_ctrl* ctrl,
                         int n_canvas, int vocab, int d_model,
                         void* workspace, size_t workspace_bytes, dg_step_graph** graph);
/* Capture dg_denoise_step_eb (same arguments) into a graph, as above. */
int dg_step_graph_create_eb(const void* q, const void* k_prefix, const void* v_prefix,
                            const void* k_canvas, const void* v_canvas, float* attn_out,
                            int n_prefix, int hq, int hkv, int head_dim, int dtype, float scale,
                            const float* logits, const void* emb_packed, int32_t* canvas_ids,
                            uint8_t* accepted, float* selfcond, float* entropy, int32_t* argmax,
                            dg_eb_status* status, dg_ctrl* ctrl, float budget, float stop_entropy,
                            int n_canvas, int vocab, int d_model,
                            void* workspace, size_t workspace_bytes, dg_step_graph** graph);
/* Capture dg_denoise_step_fp8 (same arguments) into a graph, as above. */
int dg_step_graph_create_fp8(const void* q, const void* k_prefix, const void* v_prefix,
                             const void* k_canvas, const void* v_canvas, float* attn_out,
                             int n_prefix, int hq, int hkv, int head_dim, float scale,
                             float q_scale, float k_scale, float v_scale,
                             const float* logits, const void* emb_packed, int32_t* canvas_ids,
                             uint8_t* committed, float* selfcond, float* confidence,
                             uint32_t* n_uncommitted, dg_ctrl* ctrl,
                             int n_canvas, int vocab, int d_model,
                             void* workspace, size_t workspace_bytes, dg_step_graph** graph);
int dg_step_graph_launch(dg_step_graph* graph, hipStream_t stream);
void dg_step_graph_destroy(dg_step_graph* graph);

/* ------------------------------------------------------------------------ */
/* Block loop helpers                                                        */
/* ------------------------------------------------------------------------ */

/*
 * Start a canvas: canvas_ids[i] = uniform draw from the INIT stream at
 * (seed, gstep, i), committed[i] = 0, ctrl->s_in_block = 0 (explainer section
 * quoting report 3.1-3.3: a canvas starts from uniformly random tokens).
 */
int dg_canvas_init(int32_t* canvas_ids, uint8_t* committed, dg_ctrl* ctrl,
                   int n_canvas, int vocab, hipStream_t stream);

/*
 * Append a finished canvas's K/V rows to the prefix cache (explainer section
 * "Block-autoregressive generation, one canvas after another"): copies
 * k_canvas/v_canvas [n_canvas, hkv, head_dim] to rows n_prefix.. of
 * k_prefix/v_prefix [prefix_capacity, hkv, head_dim] (device, caller-owned).
 * dtype DG_BF16 or DG_F32.  Returns DG_EINVAL when n_prefix + n_canvas exceeds
 * prefix_capacity (nothing is copied), DG_EUNSUPPORTED for another dtype.
 * Asynchronous on `stream` (two device-to-device copies).
 */
int dg_kv_append(void* k_prefix, void* v_prefix, const void* k_canvas, const void* v_canvas,
                 int n_prefix, int prefix_capacity, int n_canvas, int hkv, int head_dim, int dtype,
                 hipStream_t stream);

/*
 * Synthetic logits for the decode-run workload (a stand-in for the model, used
 * by tests and benchmarks): noise l[i,j] = table[h >> 16] with h the Philox
 * word (j & 3) of counter (j >> 2, i, gstep, 6); an open row i is "chosen" when
 * (h_choose * n_open) >> 32 < 20 (counter (0, i, gstep, 4)) and gets +30 at id
 * (h_target * vocab) >> 32 (counter (0, i, gstep, 5)); a committed row gets +30
 * at its own id.  table has table_size = 65536 float32 entries.
 */
int dg_synth_logits(float* logits, const int32_t* canvas_ids, const uint8_t* committed,
                    const dg_ctrl* ctrl, const float* table, int table_size,
                    int n_canvas, int vocab, hipStream_t stream);

/*
 * Diagnostic: out[4m + w] = output word w of Philox4x32-10 at counter
 * (m, c1, c2, c3) with key (seed mod 2^32, seed >> 32), m in [0, n_words / 4).
 * n_words must be a multiple of 4.
 */
int dg_philox_fill(uint32_t* out, size_t n_words, uint64_t seed, uint32_t c1, uint32_t c2,
                   uint32_t c3, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Peak probes (measurement only)                                            */
/* ------------------------------------------------------------------------ */

/*
 * The matrix-core rate the chip sustains: n_workgroups workgroups of 4 waves,
 * each wave running `iters` iterations of four independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands, i.e.
 * n_workgroups * 4 * iters * 4 * 32768 flops.  sink: device float32 buffer of
 * n_workgroups * 256 entries (written, values meaningless).  n_workgroups in
 * [1, 65535], iters >= 1.  Asynchronous on `stream`.
 */
int dg_probe_mfma_bf16(float* sink, int n_workgroups, int iters, hipStream_t stream);

/*
 * The HBM rate of a plain copy: `bytes` (a multiple of 16) from src to dst,
 * both device pointers, 16-byte aligned, not overlapping; 16 bytes per lane
 * per load and store.  Asynchronous on `stream`.
 */
int dg_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/*
 * The HBM rate of a plain read: `bytes` (a multiple of 16) from src (device,
 * 16-byte aligned), 16 bytes per lane per load, grid-stride over at most 4096
 * workgroups of 256 lanes.  sink: device uint32 buffer of 16384 entries (one
 * per wave; written, values meaningless).  Asynchronous on `stream`.
 */
int dg_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Profiling and errors                                                      */
/* ------------------------------------------------------------------------ */

/*
 * With profiling on, eager (non-captured) calls record a HIP event pair around
 * each kernel they launch.  dg_profile_read waits for the recorded events and
 * returns, per kernel name, the summed milliseconds and launch count, then
 * clears the records.  Returns the number of kernel names written (<= max).
 * Host pointers.  Not thread-safe; for benchmarks.
 */
int dg_profile_enable(int on);
int dg_profile_read(const char** names, double* total_ms, int* counts, int max);

const char* dg_status_string(int status);
const char* dg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
