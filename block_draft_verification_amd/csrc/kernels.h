// Internal launchers shared by the kernel sources and the C-ABI host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ---- weight-streaming linear: y = x W^T, W rows in wfmt ----
// x is FP16 [M][K] for FP8 / MXFP4 weights and BF16 [M][K] for BF16 weights,
// or MXFP8 (FP8 / MXFP4 weights only): e4m3 codes [M][K] in x and the e8m0
// exponent of each 32 consecutive k in xs [M][K/32].
struct ActIn {
  const void *x;
  const uint8_t *xs;  // NULL: FP16 / BF16 activations
};
// Weights are tile-major (the layout spec_pack_weights writes): 32-row x
// 64-column tiles, tile (rt, kt) at index rt * (cols / 64) + kt, so one row
// tile's k steps follow each other in memory.  Inside a tile, lane l = 32h + c
// (c = row in the tile, h = 0, 1) owns 16-byte chunks, chunk j of lane l at
// byte (j * 64 + l) * 16, in the order the GEMM's loads consume them; every
// wave-wide load is one contiguous kilobyte.
//   FP8   (2048 B): chunk j of lane l = row c, columns 16h + 32j .. +15
//   BF16  (4096 B): chunk j (0..3)   = row c, columns 32h + 8j .. +7
//   MXFP4 (1024 B): chunk 0          = row c, columns 32h .. 32h+31 (nibble
//                   pairs, low nibble = even column); its e8m0 scales form a
//                   64-byte tile, byte l = block h of row c
// FP8 per-row scales stay fp32 [rows].
struct LinearW {
  const void *w;   // tile-major codes / bf16 values
  const void *s;   // fp32 per-row scales (FP8), tile-major e8m0 (MXFP4), NULL (BF16)
  int wfmt;
};
__host__ __device__ constexpr int tile_bytes(int wfmt) { return wfmt == 3 ? 4096 : wfmt == 2 ? 1024 : 2048; }

// Row order of a packed matrix: packed row p holds logical row map(p).
//   kRowsPlain:  p
//   kRowsRope:   groups of D rows (one head); packed row 32t + i of a head is
//                dimension 16t + i (i < 16) or D/2 + 16t + (i - 16): a tile
//                holds 16 rotate-half RoPE pairs (d, d + D/2) as rows (i, i+16)
//   kRowsSwiglu: [gate; up] with I rows each; packed row 32t + i is gate row
//                16t + i (i < 16) or up row 16t + (i - 16)
enum RowMap { kRowsPlain = 0, kRowsRope = 1, kRowsSwiglu = 2 };
__host__ __device__ inline int packed_row_source(int map, int p, int param /* D or I */) {
  if (map == kRowsRope) {
    const int head = p / param, r = p % param, t = r >> 5, i = r & 31;
    return head * param + (i < 16 ? 16 * t + i : param / 2 + 16 * t + (i - 16));
  }
  if (map == kRowsSwiglu) {
    const int t = p >> 5, i = p & 31;
    return i < 16 ? 16 * t + i : param + 16 * t + (i - 16);
  }
  return p;
}
// Row-major -> tile-major in the row order of `map` (MXFP4 scales too, and
// FP8 per-row scales permuted into s_out); rows % 32 == 0, cols % 64 == 0
hipError_t launch_pack_weights(int wfmt, int rows, int cols, const void *w, const void *s, void *w_out, void *s_out,
                               int map, int map_param, hipStream_t st);

// Tiling of one launch (see gemm.hip): MT 32-row activation tiles per
// workgroup, NG waves along N by KS along K, nb x mb output tiles, K split
// across workgroups into nsplit pieces of spl steps.
struct GemmPlan {
  int MT, NG, KS, nb, mb, spl, nsplit, grid_x;
  bool fix = false;   // the nsplit splits are reduced inside the launch
  bool krot = false;  // the M blocks start their k loops at staggered steps
};
// Workspace of the GEMMs whose K splits are reduced inside the launch: each
// split writes an fp32 partial tile, the last split of a tile to finish adds
// them in split order and runs the epilogue.  The counters are zero between
// launches (zeroed once when allocated; each tile's last split resets its
// own), so one workspace serves the launches of one stream in turn.
struct SplitWs {
  float *part;
  int *cnt;
  size_t part_floats;
  int cnt_n;
};
// the workspace a decoder GEMM at M rows needs (0, 0: it does not split)
void split_ws_need(int kind, int M, int tiles, int ksteps, size_t *floats, int *counters);
GemmPlan gemm_plan(int M, int units, int ksteps, int MT, bool allow_split, int ng = 4);  // ng waves along N
// the decoder GEMMs, whose workgroup shapes are chosen per GEMM and row count
enum GemmKind { kGemmQkv = 0, kGemmOproj = 1, kGemmGateUp = 2, kGemmDown = 3 };
// the plan of a decoder GEMM with 16-bit activations over `tiles` 32-row weight tiles
// (ws non-NULL: K may be split, reduced inside the launch, within ws's sizes)
GemmPlan decoder_plan(int kind, int M, int tiles, int ksteps, const SplitWs *ws = nullptr);
// splits the MXFP8 mode's residual projection [M][K] x [N][K]^T uses (partials to reduce)
int residual_nsplit(int M, int N, int K);

// The input rows of a GEMM given as h * g (an RMSNorm's gain folded in, its
// normalisation left to the GEMM): ssp [M][ld] holds partial sums of h^2
// (entries past the real ones zero); the GEMM scales its outputs of row m by
// 1 / sqrt(sum_j ssp[m][j] / H + eps).  ssp NULL: the rows are used as given.
struct NormRows {
  const float *ssp;
  int ld, H;
  float eps;
};
// floats per row of the partial-sum buffer: one per 32 columns, padded to 4
inline int ssp_ld(int H) { return ((H / 32 + 3) / 4) * 4; }

// What a residual projection writes: h_out = h_in + y (fp32 [M][N]); xg =
// h_out * gain (FP16, or BF16 when xg_bf16), the input of the GEMM after the
// next RMSNorm; ssp[m][n / 32] = sum of h_out^2 over each 32 columns.
struct ResidualOut {
  const float *h_in;
  float *h_out;
  const float *gain;
  uint16_t *xg;
  int xg_bf16;
  float *ssp;
  int ssp_ld;
  int32_t *err;
};
// kind: kGemmOproj or kGemmDown (the workgroup shape)
hipError_t launch_residual(int kind, ActIn x, int M, int N, int K, LinearW w, const ResidualOut &o,
                           const SplitWs *ws, hipStream_t st);

// y fp32 [M][N] (test hook)
hipError_t launch_linear_f32(ActIn x, int M, int N, int K, LinearW w, float *y, hipStream_t st);

// QKV projection + RoPE; q -> q_out FP16 [M][Hq*D]; k, v -> BF16 caches at slot kv_len[b] + j.
// Where cache position `pos` of (sequence b, KV head h) lives, as a row index
// into one layer's K or V array (rows of D elements): contiguous
// [max_batch][Hkv][max_ctx], or paged [num_pages][Hkv][page_size] through
// pages[b][pos / page_size].  ok = false for a page index outside the pool
// (the row returned is then clamped into it).
struct KvLayout {
  const int32_t *pages;  // NULL: contiguous
  int page_size, max_pages, num_pages;
  __device__ __forceinline__ size_t row(int b, int h, int Hkv, int max_ctx, int pos, bool &ok) const {
    if (!pages) {
      ok = true;
      return ((size_t)b * Hkv + h) * max_ctx + pos;
    }
    int pg = pages[(size_t)b * max_pages + pos / page_size];
    ok = pg >= 0 && pg < num_pages;
    pg = pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : pg);
    return ((size_t)pg * Hkv + h) * page_size + pos % page_size;
  }
};

struct QkvOut {
  uint16_t *q_out;
  uint16_t *k_cache, *v_cache;  // layer base (contiguous or page pool)
  const int32_t *kv_len;
  const float2 *rope;           // [max_ctx][D/2] (cos, sin)
  int Hq, Hkv, D, max_ctx;
  KvLayout kvl;
  int32_t *err;                 // SPEC_DERR_RANGE: a q, k or v value beyond FP16's range
};
// q (FP16) and k, v (BF16 cache) from x; w packed with kRowsRope
hipError_t launch_qkv(ActIn x, int M, int H, LinearW w, QkvOut o, NormRows nr, const SplitWs *ws, hipStream_t st);

// a[m][n] = SiLU(x Wg^T) * (x Wu^T), W = [gate; up] with I rows each, packed
// with kRowsSwiglu: FP16 (a_scales NULL) or MXFP8 codes in a and e8m0
// [M][I/32] in a_scales
hipError_t launch_swiglu(ActIn x, int M, int H, int I, LinearW w, void *a, uint8_t *a_scales, NormRows nr,
                         const SplitWs *ws, hipStream_t st);

// part[z][m][n] = split z of (x W^T)[m][n] (fp32); residual_nsplit() splits.
// The following launch_norm adds them to h (the MXFP8-activation mode).
hipError_t launch_residual_partial(ActIn x, int M, int N, int K, LinearW w, float *part, hipStream_t st);

// lm_head (BF16 x, BF16 table) + argmax partials, one per (row, workgroup):
// part[m][p] over vocab slices of 4 * 32 * kLmNT rows
struct ArgmaxPart { float v; int32_t i; };
#ifndef GEMM_LM_NT
#define GEMM_LM_NT 1
#endif
constexpr int kLmNT = GEMM_LM_NT;  // 32-row vocab tiles per wave (one: two waves per SIMD fit)
hipError_t launch_lm_argmax(const uint16_t *x, int M, int V, int H, const uint16_t *table, ArgmaxPart *part,
                            float *logits_dump, NormRows nr, hipStream_t st);
inline int lm_parts(int V) { return (V / (32 * kLmNT) + 3) / 4; }

// ---- attention ----
// Split plan of one pass (attn_plan.h): plan[0] = {t, splits}, plan[1 + b] =
// {first slot of sequence b, splits per KV head of b, kv_len[b]}.
struct AttnPlanArgs {
  int4 *plan;   // [1 + batch]
  int batch, Hkv, max_ctx;
  int grid;     // workgroups of the attention launch (>= batch * Hkv)
  int nteam;    // key-tile teams per workgroup: t is a multiple of it
  int fixed_t;  // > 0: every split has fixed_t tiles; 0: the plan chooses
};
struct AttnArgs {
  const uint16_t *q;                 // FP16 [M][Hq*D]
  const uint16_t *k_cache, *v_cache; // BF16, layer base (contiguous or page pool)
  KvLayout kvl;
  const int4 *plan;                  // the pass's split plan
  uint16_t *o;                       // FP16 [M][Hq*D]
  uint16_t *part_o;                  // FP16 [grid][G*16][D]: o / l of each split (slot)
  float2 *part_ml;                   // [grid][G*16]: (m, l) of each split
  int batch, Hq, Hkv, max_ctx, grid;
};
// split attention (partials) followed by the merge kernel (writes o)
hipError_t launch_attention(const AttnArgs &a, int D, hipStream_t st);  // splits, then merge
hipError_t launch_attention_splits(const AttnArgs &a, int D, hipStream_t st);
hipError_t launch_attention_merge(const AttnArgs &a, int D, hipStream_t st);
// compute units of the current device
int attention_device_cus();
// workgroups (= partial slots) of the attention launch on a device with `cus`
// compute units: split_len > 0 fixes the split length (keys, a multiple of
// 64), 0 lets the plan choose.  A context fixes `cus` when it sizes its
// buffers, so its launches never outgrow them.
int attention_grid(int batch, int Hq, int Hkv, int max_ctx, int D, int split_len, int cus);
// the plan's arguments for a launch of attention_grid(...) workgroups
AttnPlanArgs attention_plan_args(int4 *plan, int batch, int Hq, int Hkv, int max_ctx, int D, int split_len, int cus);
// the plan on its own (one wave); the pass computes it inside launch_embed
hipError_t launch_attention_plan(const int32_t *kv_len, const AttnPlanArgs &p, hipStream_t st);

// ---- small kernels ----
// h = E[t] (table: the row-major BF16 embedding [V][H]); with xg non-NULL
// also xg = h * gain (FP16) and the partial sums of h^2 per 32 columns into
// ssp [M][ld] (the first RMSNorm, folded into the QKV step); with plan.plan
// non-NULL, the attention split plan of the pass.
hipError_t launch_embed(const int32_t *tokens, int M, int H, int V, const uint16_t *table, float *h,
                        const float *gain, uint16_t *xg, float *ssp, int ld, const int32_t *kv_len, int max_ctx,
                        KvLayout kvl, int32_t *err, const AttnPlanArgs &plan, hipStream_t st);
// The final normed hidden state of the rows the lm_head read, from its input
// xg = h * g (BF16 [M][H]) and the partial sums ssp: x = xg / sqrt(sum/H +
// eps).  rows: every row (row_of NULL, n rows) or row b*16 + row_of[b] - 1 for
// b < n (row_of = the accepted lengths; b is skipped when row_of[b] is outside
// [1, 16]).  Written as fp32 [n][H] (out_f32) or BF16 [n][H] (out_bf16).
hipError_t launch_final_hidden(const uint16_t *xg, const float *ssp, int ld, int H, float eps, int n,
                               const int32_t *row_of, float *out_f32, uint16_t *out_bf16, hipStream_t st);
// h_out = h + part[0] + ... + part[nsplit-1] (in that order; nsplit may be 0;
// h_out may be NULL, and is never h, so a launch can be repeated), then
// x = RMSNorm(h_out) * gain, written as FP16 (out_bf16 = 0) or BF16 (out_bf16 = 1)
hipError_t launch_norm(const float *h, float *h_out, const float *part, int nsplit, const float *gain, int M, int H,
                       float eps, uint16_t *x, int out_bf16, float *dump, hipStream_t st);
// h_out = h + part[0] + ... + part[nsplit-1] (in that order; h_out is never
// h), xg = h_out * gain (FP16, or BF16 with xg_bf16) and ssp[m][j] = sum of
// h_out^2 over columns 32j .. 32j+31 (entries past H/32 up to ld zeroed): the
// residual step after a split-K projection, with the next RMSNorm left to the
// GEMM that reads xg (NormRows).
hipError_t launch_fold(const float *h, float *h_out, const float *part, int nsplit, const float *gain, int M, int H,
                       uint16_t *xg, int xg_bf16, float *ssp, int ld, int32_t *err, hipStream_t st);
// the same as launch_norm, x written as MXFP8: e4m3 codes [M][H] in x8, e8m0 [M][H/32] in xs
// (dump, when non-NULL, gets the decoded values code * 2^(e - 127))
hipError_t launch_norm_mx8(const float *h, float *h_out, const float *part, int nsplit, const float *gain, int M,
                           int H, float eps, uint8_t *x8, uint8_t *xs, float *dump, hipStream_t st);
// MXFP8 encoding of fp32 rows x [M][K] (K a multiple of 32), the one the
// normalisation and SwiGLU steps apply
hipError_t launch_quant_mx8(const float *x, int M, int K, uint8_t *codes, uint8_t *scales, hipStream_t st);
hipError_t launch_accept(const ArgmaxPart *part, int nparts, int M, const int32_t *tokens, int batch,
                         int32_t *accept_len, int32_t *bonus, int32_t *argmax, int32_t *last_tau,
                         hipStream_t st);
hipError_t launch_commit(int batch, const int32_t *n_commit, const int32_t *last_tau, int32_t *kv_len,
                         int max_ctx, int32_t *err, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t st);
hipError_t launch_prefill_gather(const int32_t *prompt, int T, const int32_t *lens, int chunk, int batch,
                                 int32_t *tokens, int32_t *err, hipStream_t st);
// (the prompt's last row's final hidden state is written by
// launch_final_hidden with row_of = last_tau once the finish step has set it)
// sel[b] = the row count r of the chunk that holds prompt b's last token (the
// anchor row is r - 1), 0 for the other sequences
hipError_t launch_prefill_finish(const int32_t *lens, int T, int chunk, int batch, const int32_t *argmax,
                                 int32_t *n_commit, int32_t *pending, int32_t *last_tau, int32_t *sel,
                                 hipStream_t st);
