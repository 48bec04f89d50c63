/*
 * spec_verify.h -- C ABI of the block-draft verify pass on MI355X (gfx950).
 *
 * What the library computes (HunyuanOCR-1.5 / DFlash write-up, inference
 * loop, steps 3-5; "The Inference Stack Behind OCRia", speculative decoding
 * section):
 *
 *   A drafter proposes a block; the target model checks the whole block in
 *   ONE forward pass and keeps the longest prefix whose tokens equal the
 *   target's own greedy choices, cutting at the first left-to-right
 *   mismatch.  The pass also yields one more token from the target itself:
 *   the correction after a rejected draft, or the bonus after a fully
 *   accepted block ("LLM 推理加速" article, section 3.2, describes both).
 *
 * A block is 16 token ids per sequence: t[0] is the pending token (the last
 * token emitted, not yet in the KV cache) and t[1..15] are drafts.  Row j sits
 * at position p = kv_len[b] + j and sees cache keys 0 .. p (the committed
 * prefix plus the block rows up to itself).  g[j] = argmax of the lm_head at
 * row j (lowest id on ties).  The accepted length is
 *     tau = min{ j in [1,16) : t[j] != g[j-1] }, or 16 if there is none,
 * and bonus = g[tau-1].  tau counts block rows kept (pending included), so
 * the caller emits t[1..tau-1] followed by bonus, and commits tau KV rows.
 *
 * Model (pre-norm GQA decoder, no biases): h = E[t];
 *   per layer: x = RMSNorm(h); q,k,v = x Wqkv^T; RoPE(q,k) (rotate-half,
 *   inv_freq_i = theta^(-2i/D)); o = softmax(q k^T / sqrt(D)) v under the
 *   block-causal mask, query head h reading KV head h / (Hq/Hkv);
 *   h += o Wo^T; x = RMSNorm(h); h += (SiLU(x Wg^T) * (x Wu^T)) Wd^T;
 *   final x = RMSNorm(h); logits = x E^T (or x Wlm^T for an untied head).
 *
 * Numerics of this implementation: FP8 / MXFP4 weights decoded exactly to
 * FP16 and multiplied with FP16 activations (q, softmax weights, attention
 * output, SwiGLU output, and each RMSNorm's input h * g, whose normalisation
 * 1/sqrt(mean(h^2) + eps) the next projection applies to its fp32 outputs);
 * the KV cache is BF16, converted to FP16 inside attention (exact for
 * |v| < 65520 apart from FP16's subnormal range; larger values are not
 * supported); the lm_head multiplies its BF16 table with h * g of the final
 * RMSNorm rounded to BF16 and normalises its fp32 logits; fp32 accumulation,
 * residual stream, softmax statistics and logits.  A q, k, v or normed-input
 * value beyond FP16's range sets SPEC_DERR_RANGE.  With act_fmt =
 * SPEC_ACT_MXFP8 the inputs of the QKV, gate/up and down projections are
 * MXFP8 instead (see spec_act_fmt) and those products run on the scaled FP8
 * matrix cores.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).
 *   - The caller owns all device memory it passes in (weights, KV caches,
 *     kv_len, tokens, outputs).  The library owns only what it allocates in
 *     spec_verify_init (its workspace and its packed copy of the weights)
 *     and frees in spec_verify_destroy.
 *   - Work is enqueued on the given stream and returns without waiting;
 *     nothing is copied device->host except in spec_get_device_error.
 *   - Return values: SPEC_OK (0) or a negative spec_status; spec_last_error()
 *     describes the latest failure of the calling thread (for SPEC_E_HIP:
 *     which launch or runtime call failed, with the HIP error).  Argument
 *     errors are detected on the host before anything is enqueued.
 *     Conditions only the device can see (a token id >= vocab, a cache that
 *     would overflow) set bits in a sticky device error word; affected rows
 *     skip their writes, so no access ever leaves its buffer.
 *   - One context per stream; calls on one context must not overlap.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_BLOCK 16

typedef enum {
  SPEC_OK = 0,
  SPEC_E_ARG = -1,         /* NULL pointer, batch out of range, bad count   */
  SPEC_E_SHAPE = -2,       /* model/cache shape the kernels do not support  */
  SPEC_E_UNSUPPORTED = -3, /* weight format not supported for that matrix   */
  SPEC_E_HIP = -4,         /* a HIP runtime call failed                     */
  SPEC_E_NOMEM = -5        /* workspace allocation failed                   */
} spec_status;

/* Weight formats ("The Inference Stack Behind OCRia", quantization section:
 * FP8 halves the bytes per weight; per-layer mixes of precisions). */
typedef enum {
  SPEC_WFMT_FP8_E4M3_ROW = 1, /* uint8 OCP e4m3fn codes [rows][cols] + fp32
                                 scale per row: w = e4m3(code) * scale[row] */
  SPEC_WFMT_MXFP4 = 2,        /* uint8 [rows][cols/2] e2m1 nibbles, low nibble
                                 = even column, + uint8 e8m0 [rows][cols/32]:
                                 w = e2m1 * 2^(e8m0 - 127)                    */
  SPEC_WFMT_BF16 = 3          /* uint16 bf16 bit patterns [rows][cols]       */
} spec_wfmt;

/* Activation format of the QKV, gate/up and down projections' inputs (the
 * two RMSNorm outputs of a layer and the SwiGLU output).  "The Inference
 * Stack Behind OCRia" (kernel section) fuses the FP8 quantisation of these
 * activations into the kernels that produce them; the same is done here.
 * MXFP8 follows the OCP microscaling format: each 32 consecutive values along
 * the reduction axis share X = floor(log2(max |v|)) - 8 (clamped to
 * [-127, 127], -127 for an all-zero block), stored as the e8m0 byte X + 127,
 * and each value is the e4m3 code nearest to v * 2^-X (ties to even,
 * saturating at 448), all taken on the fp32 value.  The attention output that
 * feeds the O projection stays FP16. */
typedef enum {
  SPEC_ACT_FP16 = 0,  /* FP16 activations (the default) */
  SPEC_ACT_MXFP8 = 1  /* MXFP8 activations, FP8 / MXFP4 weights taken raw by
                         the scaled matrix-core instruction */
} spec_act_fmt;

/* Device error bits (sticky until read by spec_get_device_error). */
#define SPEC_DERR_TOKEN 1    /* a token id outside [0, vocab): row uses id 0  */
#define SPEC_DERR_CAPACITY 2 /* kv_len + 16 > max_ctx: the sequence's block
                                K/V writes are skipped                        */
#define SPEC_DERR_COMMIT 4   /* a commit count outside [0,16] or past max_ctx:
                                that sequence's kv_len is left unchanged      */
#define SPEC_DERR_LENGTH 8   /* spec_prefill: a prompt length outside [1, T]:
                                that sequence is not advanced                 */
#define SPEC_DERR_PAGE 16    /* paged cache: a page index the pass needs lies
                                outside [0, num_pages)                        */
#define SPEC_DERR_RANGE 32   /* a q, k, v or RMSNorm-input value beyond FP16's
                                range (|v| > 65504): results are not valid   */

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
  float rms_eps;     /* e.g. 1e-6 */
  float rope_theta;  /* e.g. 1e4  */
  int32_t attn_wfmt; /* format of w_qkv and w_o: SPEC_WFMT_FP8_E4M3_ROW       */
  int32_t mlp_wfmt;  /* format of w_gate_up and w_down: FP8_E4M3_ROW | MXFP4 */
  int32_t tied_lm_head; /* 1: logits use the embedding table */
  int32_t act_fmt;   /* spec_act_fmt */
} spec_model_desc;

/* Weight memory layout: row-major, outputs by inputs, as a checkpoint
 * stores them.  FP8_E4M3_ROW: uint8 codes [rows][cols] + fp32 scale [rows];
 * MXFP4: uint8 [rows][cols/2] (low nibble = even column) + uint8 e8m0
 * [rows][cols/32]; BF16: uint16 [rows][cols].  Rows are a multiple of 32 and
 * columns a multiple of 64.  spec_verify_init repacks every weight matrix
 * (and the lm_head table) into a library-owned copy in the order the kernels
 * stream it, so the library holds a second copy of the weights: for the
 * 0.5B-class model (24 layers, hidden 896, intermediate 4864, FP8) 0.36 GB of
 * layers plus 0.27 GB of BF16 lm_head; for the 8B-class model 7.0 GB plus
 * 1.05 GB.  The caller's weights may be freed after init; the embedding
 * table (read by row) and the norm gains may not. */

/* One decoder layer (all device pointers, caller-owned, row-major).
 *   w_qkv  [(Hq+2Hkv)*D][H], rows = q heads, then k heads, then v heads
 *   w_o    [H][Hq*D]
 *   w_gate_up [2I][H], rows = gate (I rows) then up (I rows)
 *   w_down [H][I]
 * s_* : fp32 [rows] for FP8_E4M3_ROW; e8m0 [rows][cols/32] for MXFP4.
 * attn_norm, mlp_norm: fp32 RMSNorm gains [H]. */
typedef struct {
  const void *w_qkv, *s_qkv;
  const void *w_o, *s_o;
  const void *w_gate_up, *s_gate_up;
  const void *w_down, *s_down;
  const float *attn_norm, *mlp_norm;
} spec_layer_weights;

typedef struct {
  const spec_layer_weights *layers; /* (host) array of n_layers; copied at init */
  const uint16_t *embed;            /* bf16 [V][H]                              */
  const uint16_t *lm_head;          /* bf16 [V][H]; NULL when tied              */
  const float *final_norm;          /* fp32 [H]                                */
} spec_weights;

/* KV cache, BF16, for K and for V.  kv_len[b] = committed length of
 * sequence b (int32, device).  A verify writes the block's K/V to positions
 * kv_len[b] .. kv_len[b]+15 without changing kv_len; positions >= kv_len are
 * otherwise unspecified.
 *
 * Contiguous layout (page_table NULL): [n_layers][max_batch][Hkv][max_ctx][D].
 *
 * Paged layout (page_table not NULL; "The Inference Stack Behind OCRia",
 * KV-cache section): a pool [n_layers][num_pages][Hkv][page_size][D];
 * position p of sequence b lives in page page_table[b][p / page_size] at row
 * p % page_size.  page_table is int32 [max_batch][max_ctx / page_size] on the
 * device, owned and filled by the caller (the pages a pass touches,
 * positions 0 .. kv_len[b]+15, must be valid; an index outside
 * [0, num_pages) sets SPEC_DERR_PAGE and that page is neither read nor
 * written).  page_size is a multiple of 64 and divides max_ctx, the
 * per-sequence capacity.  Commit and rollback remain length changes. */
typedef struct {
  uint16_t *k_cache, *v_cache;
  int32_t *kv_len;
  int32_t max_batch, max_ctx;
  const int32_t *page_table; /* NULL: contiguous layout */
  int32_t page_size, num_pages;
} spec_kv;

typedef struct spec_ctx spec_ctx;

/* Set up a verify context for one target model and its KV cache.  The
 * target's weights arrive as a checkpoint holds them: FP8 (or MXFP4) linear
 * layers with their scales and a BF16 embedding / lm_head ("The Inference
 * Stack Behind OCRia", quantization section: the weights that are streamed
 * on every decode step ship as FP8, mixed with other precisions per layer).
 * Validates the model and cache description, copies the pointer tables,
 * repacks the weights into library-owned memory (see the weight layout
 * above), and allocates the library workspace (activations for max_batch*16
 * rows, split attention partials, argmax partials, a RoPE cos/sin table for
 * positions < max_ctx, the device error word).  Supported: head_dim 64 or
 * 128, hidden and intermediate multiples of 64 with hidden <= 4096, vocab a
 * multiple of 64, Hq % Hkv == 0 with Hq / Hkv <= 8.  Errors: SPEC_E_ARG
 * (NULL or misaligned pointer), SPEC_E_SHAPE, SPEC_E_UNSUPPORTED (weight or
 * activation format), SPEC_E_NOMEM, SPEC_E_HIP.  Synchronous (allocations,
 * the repack and one table upload on `stream`).  *out is set only on
 * success. */
int spec_verify_init(const spec_model_desc *model /*host*/, const spec_weights *w /*host*/,
                     const spec_kv *kv /*host*/, hipStream_t stream, spec_ctx **out /*host*/);

/* One verify pass for sequences 0 .. batch-1.
 *   tokens     int32 [batch][16], row 0 = pending token
 *   accept_len int32 [batch] out: tau in [1,16]
 *   bonus      int32 [batch] out: g[tau-1]
 *   argmax     int32 [batch][16] out, or NULL: g for every row
 * Writes the block's K/V to cache slots kv_len[b]+j; never changes kv_len.
 * Asynchronous on `stream`.  SPEC_E_ARG for batch outside [1, max_batch]
 * or NULL tokens/accept_len/bonus. */
int spec_verify_block(spec_ctx *ctx, int32_t batch, const int32_t *tokens, int32_t *accept_len,
                      int32_t *bonus, int32_t *argmax, hipStream_t stream);

/* Lanes (a performance setting of the context; default 1).  With n > 1,
 * spec_verify_block cuts the batch into n contiguous ranges of sequences
 * (as equal as possible; fewer lanes when batch < n) and runs the complete
 * pass of each range on its own internal HIP stream, forked from and joined
 * back to the caller's stream with events: the call stays ordered on
 * `stream`, and a graph capture of the call records the lanes as parallel
 * branches, so the kernels of one lane fill the GPU while another waits.
 * Each range is computed exactly as a pass over that range alone would be
 * (the split-K and attention key splits follow the range's size), so
 * results are deterministic for a given lane count and agree with one lane
 * to rounding.  The first call with n > 1 allocates the per-lane split
 * buffers for SPEC_MAX_LANES lanes and creates the streams (synchronous);
 * later calls only set n.  SPEC_E_ARG for n outside [1, SPEC_MAX_LANES]. */
#define SPEC_MAX_LANES 4
int spec_verify_set_lanes(spec_ctx *ctx, int32_t lanes);

/* Commit the accepted rows ("HunyuanOCR-1.5 / DFlash" write-up, inference
 * loop, steps 4-5: keep the accepted prefix and continue from the bonus;
 * "The Inference Stack Behind OCRia", verification section: a rejected
 * suffix is dropped by moving a pointer back, not by copying state):
 * kv_len[b] += n_commit[b] for b < batch, or += the tau of the last verify
 * when n_commit is NULL (int32 [batch], device).  The K/V rows are already in
 * place, so this is a length bump and rejected rows are rolled back by not
 * counting them.  Counts must lie in [0, 16] and keep kv_len <= max_ctx,
 * else that sequence is left unchanged and SPEC_DERR_COMMIT is set.
 * SPEC_E_ARG for a NULL context or batch outside [1, max_batch].
 * Asynchronous. */
int spec_commit_kv(spec_ctx *ctx, int32_t batch, const int32_t *n_commit, hipStream_t stream);

/* Chunked prefill through the verify pass ("HunyuanOCR-1.5 / DFlash"
 * write-up, inference loop, step 1: the target processes the prompt before
 * the first draft).  For b < batch the prompt prompt[b][0 .. lengths[b])
 * (int32 [batch][T], row-major, device; lengths int32 [batch], device, each
 * in [1, T]) is appended to the cache at kv_len[b], 16 rows per pass:
 * chunk c runs rows 16c .. 16c+15 (token 0 past the prompt's end) and
 * commits the real ones.  On completion kv_len[b] += lengths[b];
 * pending[b] (int32, device) = the greedy next token after the prompt (the
 * argmax at its last row), which is row 0 of the first verify block; and,
 * when anchor_hidden is not NULL (BF16 [batch][hidden], 16-byte aligned,
 * device), the final normed hidden state of the prompt's last row.  Every
 * pass writes 16 K/V slots, so kv_len[b] + 16 * ceil(T/16) <= max_ctx is
 * needed (else SPEC_DERR_CAPACITY, as for a verify).  Lengths outside
 * [1, T] set SPEC_DERR_LENGTH and leave that sequence unchanged.  Runs
 * ceil(T/16) verify passes; asynchronous, no host synchronisation. */
int spec_prefill(spec_ctx *ctx, int32_t batch, const int32_t *prompt, int32_t T, const int32_t *lengths,
                 int32_t *pending, uint16_t *anchor_hidden, hipStream_t stream);

/* After spec_verify_block (or spec_prefill): out[b] (BF16 [batch][hidden],
 * 16-byte aligned, device) = the final normed hidden state of block row
 * tau_b - 1 of the last pass, i.e. the position whose argmax produced the
 * bonus (the pending token of the next block) -- the target feature a block
 * drafter is conditioned on ("HunyuanOCR-1.5 / DFlash" write-up, section 一:
 * the draft model reads the target's hidden states).  Must run before the
 * next pass overwrites them.  Asynchronous. */
int spec_export_hidden(spec_ctx *ctx, int32_t batch, uint16_t *out, hipStream_t stream);

/* Free the workspace.  The caller's buffers are untouched.  NULL is a no-op. */
int spec_verify_destroy(spec_ctx *ctx);

/* Read and clear the sticky device error word (a mask of SPEC_DERR_*).
 * Synchronises `stream`. */
int spec_get_device_error(spec_ctx *ctx, int32_t *code /*host*/, hipStream_t stream);

/* Static description of a spec_status value. */
const char *spec_status_str(int status);

/* The latest failure reported by a call on this thread: the call, the step
 * or runtime function that failed and, for SPEC_E_HIP, the HIP error name and
 * code; "" when no call has failed.  Valid until the thread's next failing
 * call. */
const char *spec_last_error(void);

/* Test hook: when hidden/logits are non-NULL, later verify passes also write
 * the final normed hidden state (fp32 [batch*16][H], the BF16 values fed to
 * the lm_head) and the logits (fp32 [batch*16][V]).  NULL disables. */
int spec_debug_set_dump(spec_ctx *ctx, float *hidden, float *logits);

/* Test hook: one weight-streaming linear on its own,
 *   y[m][n] = sum_k x[m][k] * w(n, k)     (fp32 out, [M][N])
 * x: FP16 bits [M][K] for FP8 / MXFP4 weights, BF16 bits for BF16 weights;
 * w row-major in format `wfmt` with scales as in spec_layer_weights (scales
 * NULL for BF16).  K and N multiples of 64.  Allocates a packed copy of w;
 * synchronous. */
int spec_debug_linear(int32_t M, int32_t N, int32_t K, const uint16_t *x, const void *w,
                      const void *scales, int32_t wfmt, float *y, hipStream_t stream);

/* Test hook: the MXFP8 encoding (spec_act_fmt) of fp32 rows x [M][K], K a
 * multiple of 32: e4m3 codes [M][K] and e8m0 bytes [M][K/32].  x and codes
 * 16-byte aligned.  Synchronous. */
int spec_debug_quant_mx8(int32_t M, int32_t K, const float *x, uint8_t *codes, uint8_t *scales,
                         hipStream_t stream);

/* Test hook: the pass's RMSNorm step on its own: x = h / sqrt(mean(h^2) +
 * eps) * gain over rows of h fp32 [M][H] (H <= 4096, a multiple of 32), gain
 * fp32 [H]; x written as FP16 bits [M][H] (act_fmt SPEC_ACT_FP16, xs unused)
 * or as MXFP8 codes [M][H] + e8m0 [M][H/32] (SPEC_ACT_MXFP8).  h, gain and x
 * 16-byte aligned.  Synchronous. */
int spec_debug_rmsnorm(int32_t M, int32_t H, const float *h, const float *gain, float eps, int32_t act_fmt,
                       void *x, uint8_t *xs, hipStream_t stream);

/* Test hook: the gate/up projection with its SiLU-and-multiply epilogue on
 * its own: a = SiLU(x Wg^T) * (x Wu^T), w = [gate rows; up rows] [2I][H]
 * row-major in FP8_E4M3_ROW or MXFP4 with scales as in spec_layer_weights
 * (a packed copy is allocated).  Input x: FP16
 * bits [M][H] (x_scales NULL) or MXFP8 codes [M][H] + e8m0 [M][H/32].  Output
 * a: FP16 bits [M][I] (out_fmt SPEC_ACT_FP16, a_scales unused) or MXFP8 codes
 * [M][I] + e8m0 [M][I/32] (SPEC_ACT_MXFP8).  H, I multiples of 64.
 * Synchronous. */
int spec_debug_swiglu(int32_t M, int32_t H, int32_t I, const void *x, const uint8_t *x_scales, const void *w,
                      const void *scales, int32_t wfmt, int32_t out_fmt, void *a, uint8_t *a_scales,
                      hipStream_t stream);

/* Test hook: spec_debug_linear with MXFP8 activations (codes [M][K], e8m0
 * [M][K/32]) and row-major FP8_E4M3_ROW or MXFP4 weights (BF16 weights are
 * rejected with SPEC_E_UNSUPPORTED).  Synchronous. */

/* Test hook: one residual projection with the next RMSNorm folded in, as the
 * pass runs its O and down projections:
 *   h_out = h_in + x W^T                      (fp32 [M][N])
 *   xg    = h_out * gain                      (FP16 bits [M][N], or BF16 bits
 *                                              with xg_bf16 = 1)
 *   ssp[m][j] = sum of h_out[m][n]^2 over n in [32j, 32j+32), j < N/32
 *                                             (fp32 [M][ld], ld = N/32
 *                                              rounded up to a multiple of 4;
 *                                              the last entries untouched)
 * x FP16 bits [M][K]; w row-major FP8_E4M3_ROW or MXFP4 [N][K] with scales;
 * gain fp32 [N]; N, K multiples of 64; all 16-byte aligned.  Synchronous. */
int spec_debug_residual(int32_t M, int32_t N, int32_t K, const uint16_t *x, const void *w, const void *scales,
                        int32_t wfmt, const float *h_in, const float *gain, int32_t xg_bf16, float *h_out,
                        uint16_t *xg, float *ssp, hipStream_t stream);
int spec_debug_linear_mx8(int32_t M, int32_t N, int32_t K, const uint8_t *x_codes, const uint8_t *x_scales,
                          const void *w, const void *scales, int32_t wfmt, float *y, hipStream_t stream);

/* Test hook: block-causal GQA attention on its own for sequences 0..batch-1:
 * q FP16 [batch*16][Hq*D] (already rotated), BF16 K/V caches of ONE layer
 * ([max_batch][Hkv][max_ctx][D], block rows already stored at kv_len+j),
 * o FP16 [batch*16][Hq*D].  split_len = keys per split (multiple of 64), or
 * 0 for the library's choice; a split length that gives more than 64 splits
 * of max_ctx is rejected (SPEC_E_ARG).  Synchronous. */
int spec_debug_attention(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                         int32_t max_batch, int32_t max_ctx, const uint16_t *q,
                         const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *kv_len,
                         uint16_t *o, int32_t split_len, hipStream_t stream);

/* spec_debug_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as spec_debug_attention, but the
 * split partials and the split plan live in a library-owned static device
 * buffer of SPEC_ATTN_SCRATCH_BYTES, which every GPU the library runs on holds
 * until the process ends; nothing is allocated or freed, and the call is
 * asynchronous (no host synchronisation; the caller orders or synchronises
 * `stream`).  A launch whose partials would exceed the buffer is rejected with
 * SPEC_E_ARG (e.g. 1 sequence x 8 KV heads of head_dim 128 and 8 query heads
 * each fits; see spec_last_error for the reason of a rejection).  Every call on
 * a GPU shares that GPU's buffer, so calls that overlap on one GPU (other
 * streams, other threads) race; the buffer keeps the last call's contents. */
#define SPEC_ATTN_SCRATCH_BYTES (32u << 20)
int spec_debug_attention_noalloc(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                 int32_t max_batch, int32_t max_ctx, const uint16_t *q, const uint16_t *k_cache,
                                 const uint16_t *v_cache, const int32_t *kv_len, uint16_t *o, int32_t split_len,
                                 hipStream_t stream);

/* Kernel classes for spec_debug_time_kernel.  SPEC_K_ATTENTION is the split
 * attention kernel alone; SPEC_K_ATTN_MERGE the kernel that merges its splits. */
typedef enum {
  SPEC_K_NONE = 0, SPEC_K_EMBED = 1, SPEC_K_RMSNORM = 2, SPEC_K_QKV = 3, SPEC_K_ATTENTION = 4,
  SPEC_K_OPROJ = 5, SPEC_K_GATE_UP = 6, SPEC_K_DOWN = 7, SPEC_K_LM_HEAD = 8, SPEC_K_ACCEPT = 9,
  SPEC_K_COMMIT = 10, SPEC_K_ATTN_MERGE = 11
} spec_kernel_kind;

/* Test/measurement hook: while `kind` is set, every launch of that kernel
 * class by later verify/commit calls is bracketed by a pair of HIP events on
 * the caller's stream (at most 8192 launches are recorded).  Eager use only:
 * not under graph capture.  SPEC_K_NONE stops recording. */
int spec_debug_time_kernel(spec_ctx *ctx, int32_t kind);

/* Measurement hook: while a kernel class is timed, issue each of its launches
 * `repeat` times back to back inside one event pair (1 <= repeat <= 64;
 * default 1), so the events' own overhead is shared by `repeat` launches.  The
 * repeated kernels only recompute the same outputs from the same inputs; the
 * RMSNorm and commit classes, which update state in place, are never
 * repeated. */
int spec_debug_set_repeat(spec_ctx *ctx, int32_t repeat);

/* Synchronises the recorded events, returns the summed duration (ms) and the
 * number of recorded launches (repeats included), and clears the record. */
int spec_debug_kernel_time(spec_ctx *ctx, float *total_ms /*host*/, int32_t *launches /*host*/);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
