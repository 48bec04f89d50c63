// Host side of the C ABI declared in include/spec_verify.h.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "common.h"
#include "kernels.h"

// One decoder layer's weights as the kernels read them (library-owned packed
// copies; norm gains are the caller's).
struct PackedLayer {
  LinearW qkv, o, gate_up, down;
  const float *attn_norm, *mlp_norm;
};

struct spec_ctx {
  spec_model_desc m;
  std::vector<PackedLayer> layers;
  const uint16_t *embed;     // the caller's row-major BF16 table (gathered by row)
  const uint16_t *lm_table;  // packed BF16 lm_head (library-owned)
  const float *final_norm;
  spec_kv kv;
  int Mmax, part_units;  // part_units: (sequence, kv head, split) slots for attention partials
  int attn_cus;          // compute units the attention launches are sized for (fixed at init)
  int ld;                // floats per row of the partial sums of squares
  void *wbuf = nullptr;  // packed weights (one allocation)
  // workspace (one allocation)
  void *ws = nullptr;
  float *h, *h2;  // residual stream, ping-ponged so that every launch can be repeated
  uint16_t *x, *q, *ao, *act;    // x: a GEMM's 16-bit input (h * g, or the normed rows)
  float *ssp;                    // partial sums of squares of h [Mmax][ld]
  uint8_t *x8, *xs8, *a8, *as8;  // MXFP8 activations: normed x [Mmax][H] (+ e8m0 [Mmax][H/32]), SwiGLU [Mmax][I]
  uint16_t *part_o;  // attention split outputs, FP16
  float2 *part_ml;
  int32_t *last_tau, *err;
  ArgmaxPart *amax;
  float2 *rope;
  float *rpart;  // split-K partials of the MXFP8 mode's O and down projections [nsplit][Mmax][H]
  // prefill scratch: chunk tokens [Mmax], argmax [Mmax], commit counts, tau, bonus, anchor rows [max_batch]
  int32_t *pf_tokens, *pf_argmax, *pf_ncommit, *pf_acc, *pf_bonus, *pf_sel;
  float *dump_hidden, *dump_logits;
  // Lanes: the batch is cut into contiguous sequence ranges, each run as a
  // complete pass on its own stream (lane 0 on the caller's).  Row-indexed
  // buffers are shared (a lane touches only its own rows); the split partials
  // of attention and of the residual projections are per lane.
  int lanes = 1;
  struct LaneBufs {
    uint16_t *part_o;
    float *rpart;
    float2 *part_ml;
    int4 *plan;  // attention split plan of the lane's pass
    SplitWs fx;  // the GEMMs' K splits reduced inside their launches
  };
  LaneBufs lane_buf[SPEC_MAX_LANES] = {};
  void *lane_ws = nullptr;                      // lanes 1.. (one allocation)
  size_t lane_bytes[6] = {0, 0, 0, 0, 0, 0};    // part_o, part_ml, rpart, plan, split partials, counters of one lane
  hipStream_t lane_st[SPEC_MAX_LANES] = {};     // [0] unused (the caller's stream)
  hipEvent_t lane_ev[SPEC_MAX_LANES] = {};      // [0] fork, [i] join of lane i
  // launch timing of one kernel class (measurement hook)
  int prof_kind = SPEC_K_NONE;
  int prof_repeat = 1;         // back-to-back launches per timed launch (idempotent classes)
  std::vector<hipEvent_t> ev;  // pairs
  size_t ev_used = 0, ev_launches = 0;
};

static const size_t kMaxTimedLaunches = 8192;

// 1: the down projection (K = intermediate, the long one) splits K across
// workgroups and a small step adds the partials (launch_fold); 0 (the
// default) runs it as one residual launch like the O projection, its K split
// between the waves of each workgroup instead: measured over whole passes at
// 512 rows, one launch is faster than the split launch plus the fold.
#ifndef SPEC_DOWN_SPLIT
#define SPEC_DOWN_SPLIT 0
#endif
static constexpr bool kDownSplit = SPEC_DOWN_SPLIT != 0;

// The latest failure of a call on this thread (spec_last_error).
static thread_local char g_last_error[320] = "";

static int fail(int rc, const char *call, const char *what, hipError_t e = hipSuccess) {
  if (e != hipSuccess)
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s failed: %s (%d)", call, what, hipGetErrorName(e), (int)e);
  else
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s", call, what);
  return rc;
}

thread_local LaunchTimer g_launch_timer;

// Times one launch of a kernel class while that class is being timed.  With
// a repeat count of 1 the launch itself records a pair of events at its
// dispatch boundaries (launch_k), so the recorded time is the kernel's
// execution alone, as a kernel trace measures it.  With repeat r > 1 the call
// site issues the launch r times back to back between one pair of events on
// the stream (`reps` = r); commit, which updates its own input in place, is
// never repeated.
struct Timed {
  spec_ctx *c;
  hipStream_t st;
  bool on, ext;
  int reps;
  Timed(spec_ctx *c_, int kind, hipStream_t s) : c(c_), st(s), on(false), ext(false), reps(1) {
    if (c->prof_kind != kind || c->ev_used + 2 > c->ev.size()) return;
    if (kind != SPEC_K_COMMIT) reps = c->prof_repeat;
    ext = reps == 1;
    if (ext) {
      g_launch_timer = LaunchTimer{c->ev[c->ev_used], c->ev[c->ev_used + 1], false};
      on = true;
    } else {
      on = hipEventRecord(c->ev[c->ev_used], st) == hipSuccess;
    }
  }
  ~Timed() {
    if (!on) return;
    if (ext) {
      const bool used = g_launch_timer.used;
      g_launch_timer = LaunchTimer{};
      if (!used) return;  // the class launched nothing here
      c->ev_used += 2;
      c->ev_launches += 1;
    } else if (hipEventRecord(c->ev[c->ev_used + 1], st) == hipSuccess) {
      c->ev_used += 2;
      c->ev_launches += reps;
    }
  }
};

// A failed HIP call or launch: SPEC_E_HIP, with the expression and the HIP
// error kept for spec_last_error().
#define CK(expr)                                                   \
  do {                                                             \
    const hipError_t ck_e_ = (expr);                               \
    if (ck_e_ != hipSuccess) return fail(SPEC_E_HIP, __func__, #expr, ck_e_); \
  } while (0)

static bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

static KvLayout kv_layout(const spec_kv &kv) {
  if (!kv.page_table) return KvLayout{nullptr, 0, 0, 0};
  return KvLayout{kv.page_table, kv.page_size, kv.max_ctx / kv.page_size, kv.num_pages};
}

static int check_model(const spec_model_desc *m) {
  if (m->n_layers < 1 || m->hidden < 64 || m->n_q_heads < 1 || m->n_kv_heads < 1 || m->intermediate < 64 ||
      m->vocab < 64 || !(m->rms_eps > 0.f) || !(m->rope_theta > 0.f))
    return SPEC_E_SHAPE;
  if (m->head_dim != 64 && m->head_dim != 128) return SPEC_E_SHAPE;
  if (m->hidden % 64 || m->intermediate % 64 || m->vocab % 64) return SPEC_E_SHAPE;
  if (m->hidden > 4096) return SPEC_E_SHAPE;  // RMSNorm steps and partial sums are sized for rows up to 4096
  if (m->n_q_heads % m->n_kv_heads || m->n_q_heads / m->n_kv_heads > 8) return SPEC_E_SHAPE;
  if ((m->n_q_heads * m->head_dim) % 64) return SPEC_E_SHAPE;
  if (m->attn_wfmt != SPEC_WFMT_FP8_E4M3_ROW) return SPEC_E_UNSUPPORTED;
  if (m->mlp_wfmt != SPEC_WFMT_FP8_E4M3_ROW && m->mlp_wfmt != SPEC_WFMT_MXFP4) return SPEC_E_UNSUPPORTED;
  if (m->act_fmt != SPEC_ACT_FP16 && m->act_fmt != SPEC_ACT_MXFP8) return SPEC_E_UNSUPPORTED;
  return SPEC_OK;
}

// Bytes of a packed copy of a [rows][cols] matrix in format wfmt and of its
// scales (fp32 per row for FP8, e8m0 per 32 columns for MXFP4), each rounded
// up to 256 bytes.
static size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
static size_t code_bytes(int wfmt, int rows, int cols) {
  return round256(wfmt == SPEC_WFMT_BF16 ? (size_t)rows * cols * 2
                  : wfmt == SPEC_WFMT_MXFP4 ? (size_t)rows * cols / 2 : (size_t)rows * cols);
}
static size_t scale_bytes(int wfmt, int rows, int cols) {
  return round256(wfmt == SPEC_WFMT_BF16 ? 0 : wfmt == SPEC_WFMT_MXFP4 ? (size_t)rows * cols / 32 : (size_t)rows * 4);
}
static size_t packed_bytes(int wfmt, int rows, int cols) {
  return code_bytes(wfmt, rows, cols) + scale_bytes(wfmt, rows, cols);
}

// Packs one matrix at *cursor (advanced past it) and returns its LinearW.
static hipError_t pack_one(int wfmt, int rows, int cols, const void *w, const void *s, int map, int mp, char *&cursor,
                           LinearW &out, hipStream_t st) {
  void *wp = cursor;
  void *sp = wfmt == SPEC_WFMT_BF16 ? nullptr : cursor + code_bytes(wfmt, rows, cols);
  cursor += packed_bytes(wfmt, rows, cols);
  out = LinearW{wp, sp, wfmt};
  return launch_pack_weights(wfmt, rows, cols, w, s, wp, sp, map, mp, st);
}

extern "C" {

const char *spec_status_str(int s) {
  switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_E_ARG: return "invalid argument";
    case SPEC_E_SHAPE: return "unsupported model or cache shape";
    case SPEC_E_UNSUPPORTED: return "unsupported weight format";
    case SPEC_E_HIP: return "HIP runtime error";
    case SPEC_E_NOMEM: return "workspace allocation failed";
  }
  return "unknown status";
}

const char *spec_last_error(void) { return g_last_error; }

int spec_verify_init(const spec_model_desc *m, const spec_weights *w, const spec_kv *kv, hipStream_t st,
                     spec_ctx **out) {
  static const char *fn = "spec_verify_init";
  if (!m || !w || !kv || !out || !w->layers || !w->embed || !w->final_norm) return fail(SPEC_E_ARG, fn, "NULL argument");
  int rc = check_model(m);
  if (rc) return fail(rc, fn, "unsupported model description");
  if (!kv->k_cache || !kv->v_cache || !kv->kv_len || kv->max_batch < 1 || kv->max_ctx < 16)
    return fail(SPEC_E_ARG, fn, "bad KV cache description");
  if (kv->page_table && (kv->page_size < 64 || kv->page_size % 64 || kv->max_ctx % kv->page_size ||
                         kv->num_pages < 1))
    return fail(SPEC_E_ARG, fn, "bad page table description");
  if (!m->tied_lm_head && !w->lm_head) return fail(SPEC_E_ARG, fn, "untied model without lm_head");
  if (!aligned16(kv->k_cache) || !aligned16(kv->v_cache) || !aligned16(w->embed) ||
      !aligned16(w->final_norm) || (w->lm_head && !aligned16(w->lm_head)))
    return fail(SPEC_E_ARG, fn, "a cache or table pointer is not 16-byte aligned");
  for (int l = 0; l < m->n_layers; ++l) {
    const spec_layer_weights &L = w->layers[l];
    const void *ps[] = {L.w_qkv, L.s_qkv, L.w_o, L.s_o, L.w_gate_up, L.s_gate_up, L.w_down, L.s_down,
                        L.attn_norm, L.mlp_norm};
    for (const void *p : ps)
      if (!p || !aligned16(p)) return fail(SPEC_E_ARG, fn, "a layer weight pointer is NULL or not 16-byte aligned");
  }

  spec_ctx *c = new (std::nothrow) spec_ctx();
  if (!c) return fail(SPEC_E_NOMEM, fn, "host allocation");
  c->m = *m;
  c->embed = w->embed;
  c->final_norm = w->final_norm;
  c->kv = *kv;
  const int H = m->hidden, D = m->head_dim, Hq = m->n_q_heads, Hkv = m->n_kv_heads;
  const int G = Hq / Hkv, I = m->intermediate, V = m->vocab, mf = m->mlp_wfmt;
  const int QR = (Hq + 2 * Hkv) * D;
  c->Mmax = kv->max_batch * 16;
  c->ld = ssp_ld(H);

  // library-owned packed weights: QKV rows in RoPE-pair order, gate/up rows
  // interleaved in 16-row groups, O and down in plain order, the lm_head table
  const size_t per_layer = packed_bytes(SPEC_WFMT_FP8_E4M3_ROW, QR, H) + packed_bytes(SPEC_WFMT_FP8_E4M3_ROW, H, Hq * D) +
                           packed_bytes(mf, 2 * I, H) + packed_bytes(mf, H, I);
  const size_t wtotal = per_layer * m->n_layers + packed_bytes(SPEC_WFMT_BF16, V, H);
  if (hipMalloc(&c->wbuf, wtotal) != hipSuccess) {
    delete c;
    return fail(SPEC_E_NOMEM, fn, "packed weight allocation");
  }
  {
    char *cur = (char *)c->wbuf;
    c->layers.resize(m->n_layers);
    hipError_t e = hipSuccess;
    for (int l = 0; l < m->n_layers && e == hipSuccess; ++l) {
      const spec_layer_weights &L = w->layers[l];
      PackedLayer &P = c->layers[l];
      P.attn_norm = L.attn_norm;
      P.mlp_norm = L.mlp_norm;
      if (e == hipSuccess) e = pack_one(SPEC_WFMT_FP8_E4M3_ROW, QR, H, L.w_qkv, L.s_qkv, kRowsRope, D, cur, P.qkv, st);
      if (e == hipSuccess) e = pack_one(SPEC_WFMT_FP8_E4M3_ROW, H, Hq * D, L.w_o, L.s_o, kRowsPlain, 0, cur, P.o, st);
      if (e == hipSuccess) e = pack_one(mf, 2 * I, H, L.w_gate_up, L.s_gate_up, kRowsSwiglu, I, cur, P.gate_up, st);
      if (e == hipSuccess) e = pack_one(mf, H, I, L.w_down, L.s_down, kRowsPlain, 0, cur, P.down, st);
    }
    LinearW lm{};
    if (e == hipSuccess)
      e = pack_one(SPEC_WFMT_BF16, V, H, m->tied_lm_head ? w->embed : w->lm_head, nullptr, kRowsPlain, 0, cur, lm, st);
    c->lm_table = (const uint16_t *)lm.w;
    if (e != hipSuccess) {
      (void)hipFree(c->wbuf);
      delete c;
      return fail(SPEC_E_HIP, fn, "weight repack", e);
    }
  }

  int units = 0;
  c->attn_cus = attention_device_cus();
  for (int b = 1; b <= kv->max_batch; ++b)
    units = std::max(units, attention_grid(b, Hq, Hkv, kv->max_ctx, D, 0, c->attn_cus));
  c->part_units = units;
  size_t rfloats = 0;
  for (int b = 1; b <= kv->max_batch; ++b) {
    const int M = b * 16;
    int s = kDownSplit ? residual_nsplit(M, H, I) : 0;
    if (m->act_fmt == SPEC_ACT_MXFP8) s = std::max(residual_nsplit(M, H, Hq * D), residual_nsplit(M, H, I));
    rfloats = std::max(rfloats, (size_t)s * M * H);
  }

  // the in-launch split partials and counters of the decoder GEMMs, for every
  // row count a lane may run
  size_t fx_floats = 0;
  int fx_cnt = 0;
  for (int M = 16; M <= c->Mmax; M += 16) {
    const int shape[4][2] = {{(Hq + 2 * Hkv) * D / 32, H / 64}, {H / 32, Hq * D / 64}, {2 * I / 32, H / 64},
                             {H / 32, I / 64}};  // tiles, k steps of kGemmQkv .. kGemmDown
    for (int k = 0; k < 4; ++k) {
      size_t f;
      int n;
      split_ws_need(k, M, shape[k][0], shape[k][1], &f, &n);
      fx_floats = std::max(fx_floats, f);
      fx_cnt = std::max(fx_cnt, n);
    }
  }

  const size_t Mm = c->Mmax;
  size_t sizes[] = {2 * Mm * H * 4,                  // h, h2
                    Mm * H * 2,                      // x
                    Mm * Hq * D * 2,                 // q
                    Mm * Hq * D * 2,                 // ao
                    Mm * I * 2,                      // act
                    (size_t)units * G * 16 * D * 2,  // part_o
                    (size_t)units * G * 16 * 8,      // part_ml
                    (2 * Mm + 4 * (size_t)kv->max_batch) * 4,  // prefill scratch
                    (size_t)kv->max_batch * 4,       // last_tau
                    4,                               // err
                    (size_t)lm_parts(V) * Mm * 8,    // amax
                    (size_t)kv->max_ctx * (D / 2) * 8,  // rope
                    rfloats * 4 + 4,                 // residual split-K partials (MXFP8 mode)
                    m->act_fmt == SPEC_ACT_MXFP8 ? Mm * H + Mm * (H / 32) : 16,   // x8, xs8
                    m->act_fmt == SPEC_ACT_MXFP8 ? Mm * I + Mm * (I / 32) : 16,   // a8, as8
                    (1 + (size_t)kv->max_batch) * 16,  // attention split plan
                    Mm * c->ld * 4,                  // ssp
                    fx_floats * 4 + 16,              // in-launch split partials
                    (size_t)fx_cnt * 4 + 16};        // their counters
  const int NS = sizeof(sizes) / sizeof(sizes[0]);
  size_t off[NS], total = 0;
  for (int i = 0; i < NS; ++i) {
    off[i] = total;
    total += round256(sizes[i]);
  }
  if (hipMalloc(&c->ws, total) != hipSuccess) {
    (void)hipFree(c->wbuf);
    delete c;
    return fail(SPEC_E_NOMEM, fn, "workspace allocation");
  }
  char *base = (char *)c->ws;
  c->h = (float *)(base + off[0]);
  c->h2 = c->h + Mm * H;
  c->x = (uint16_t *)(base + off[1]);
  c->q = (uint16_t *)(base + off[2]);
  c->ao = (uint16_t *)(base + off[3]);
  c->act = (uint16_t *)(base + off[4]);
  c->part_o = (uint16_t *)(base + off[5]);
  c->part_ml = (float2 *)(base + off[6]);
  c->pf_tokens = (int32_t *)(base + off[7]);
  c->pf_argmax = c->pf_tokens + Mm;
  c->pf_ncommit = c->pf_argmax + Mm;
  c->pf_acc = c->pf_ncommit + kv->max_batch;
  c->pf_bonus = c->pf_acc + kv->max_batch;
  c->pf_sel = c->pf_bonus + kv->max_batch;
  c->last_tau = (int32_t *)(base + off[8]);
  c->err = (int32_t *)(base + off[9]);
  c->amax = (ArgmaxPart *)(base + off[10]);
  c->rope = (float2 *)(base + off[11]);
  c->rpart = (float *)(base + off[12]);
  c->x8 = (uint8_t *)(base + off[13]);
  c->xs8 = c->x8 + Mm * H;
  c->a8 = (uint8_t *)(base + off[14]);
  c->as8 = c->a8 + Mm * I;
  c->ssp = (float *)(base + off[16]);
  c->dump_hidden = c->dump_logits = nullptr;
  c->lane_buf[0] = spec_ctx::LaneBufs{c->part_o, c->rpart, c->part_ml, (int4 *)(base + off[15]),
                                      SplitWs{(float *)(base + off[17]), (int *)(base + off[18]), fx_floats, fx_cnt}};
  c->lane_bytes[0] = sizes[5];
  c->lane_bytes[1] = sizes[6];
  c->lane_bytes[2] = sizes[12];
  c->lane_bytes[3] = sizes[15];
  c->lane_bytes[4] = sizes[17];
  c->lane_bytes[5] = sizes[18];
  if (hipMemset(base + off[18], 0, sizes[18]) != hipSuccess) {  // the counters start at zero
    (void)hipFree(c->ws);
    (void)hipFree(c->wbuf);
    delete c;
    return fail(SPEC_E_HIP, fn, "split counter clear");
  }

  // RoPE table: angle = p * theta^(-2i/D), in double, stored as fp32 (cos, sin)
  std::vector<float2> rope((size_t)kv->max_ctx * (D / 2));
  for (int p = 0; p < kv->max_ctx; ++p)
    for (int i = 0; i < D / 2; ++i) {
      const double ang = (double)p * pow((double)m->rope_theta, -2.0 * i / D);
      rope[(size_t)p * (D / 2) + i] = make_float2((float)cos(ang), (float)sin(ang));
    }
  hipError_t e = hipMemcpyAsync(c->rope, rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = launch_fill_i32(c->last_tau, kv->max_batch, 0, st);
  if (e == hipSuccess) e = launch_fill_i32(c->err, 1, 0, st);
  if (e == hipSuccess) e = launch_fill_i32((int32_t *)c->ssp, (int)(Mm * c->ld), 0, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(c->ws);
    (void)hipFree(c->wbuf);
    delete c;
    return fail(SPEC_E_HIP, fn, "table upload", e);
  }
  *out = c;
  return SPEC_OK;
}

}  // extern "C"

// One complete pass for sequences b0 .. b0+batch-1 on stream st, with lane
// `lane`'s split buffers: every sequence-indexed pointer is offset to b0 and
// every row-indexed one to row 16*b0, so the kernels see sequences 0..batch-1.
//
// FP16 activations (the default): every RMSNorm is folded into its
// neighbours.  The step that updates the residual stream (embed, each O
// projection, and the fold step after each down projection's K splits)
// writes h, the next RMSNorm's input h * g and the per-32-column sums of h^2;
// the GEMM that follows (QKV, gate/up, lm_head) normalises its outputs by
// 1/sqrt(mean(h^2) + eps).  Seven launches per layer.
// MXFP8 activations: the RMSNorm steps quantise their output, so they stay
// kernels of their own, and the residual projections split K into partials
// that the next RMSNorm adds (eight launches per layer).
static int run_pass(spec_ctx *c, int lane, int b0, int batch, const int32_t *tokens, int32_t *accept_len,
                    int32_t *bonus, int32_t *argmax, hipStream_t st) {
  const spec_model_desc &m = c->m;
  const int M = batch * 16, H = m.hidden, D = m.head_dim, Hq = m.n_q_heads, Hkv = m.n_kv_heads;
  const int I = m.intermediate, V = m.vocab, max_ctx = c->kv.max_ctx, ld = c->ld;
  KvLayout kvl = kv_layout(c->kv);
  const size_t lstride = (kvl.pages ? (size_t)c->kv.num_pages * kvl.page_size : (size_t)c->kv.max_batch * max_ctx) *
                         Hkv * D;
  // sequence offset b0: contiguous caches move their base, paged ones their page-table rows
  size_t seq0 = 0;
  if (kvl.pages) kvl.pages += (size_t)b0 * kvl.max_pages;
  else seq0 = (size_t)b0 * Hkv * max_ctx * D;
  const size_t r0 = (size_t)b0 * 16;
  const int32_t *kv_len = c->kv.kv_len + b0;
  float *h = c->h + r0 * H, *h2 = c->h2 + r0 * H, *rpart = c->lane_buf[lane].rpart;
  uint16_t *x = c->x + r0 * H, *q = c->q + r0 * Hq * D, *ao = c->ao + r0 * Hq * D, *act = c->act + r0 * I;
  float *ssp = c->ssp + r0 * ld;
  uint8_t *x8 = c->x8 + r0 * H, *xs8 = c->xs8 + r0 * (H / 32), *a8 = c->a8 + r0 * I, *as8 = c->as8 + r0 * (I / 32);
  ArgmaxPart *amax = c->amax + r0 * lm_parts(V);
  float *dump_hidden = c->dump_hidden ? c->dump_hidden + r0 * H : nullptr;
  float *dump_logits = c->dump_logits ? c->dump_logits + r0 * V : nullptr;
  int32_t *last_tau = c->last_tau + b0;
  const bool mx = m.act_fmt == SPEC_ACT_MXFP8;
  const NormRows nr = mx ? NormRows{} : NormRows{ssp, ld, H, m.rms_eps};
  const SplitWs *fx = &c->lane_buf[lane].fx;

  const AttnPlanArgs plan = attention_plan_args(c->lane_buf[lane].plan, batch, Hq, Hkv, max_ctx, D, 0, c->attn_cus);
  AttnArgs aa{};
  aa.q = q;
  aa.plan = plan.plan;
  aa.grid = plan.grid;
  aa.o = ao;
  aa.part_o = c->lane_buf[lane].part_o;
  aa.part_ml = c->lane_buf[lane].part_ml;
  aa.batch = batch;
  aa.Hq = Hq;
  aa.Hkv = Hkv;
  aa.max_ctx = max_ctx;
  aa.kvl = kvl;

  {
    Timed t(c, SPEC_K_EMBED, st);
    for (int r = 0; r < t.reps; ++r)
      CK(launch_embed(tokens, M, H, V, c->embed, h, mx ? nullptr : c->layers[0].attn_norm, mx ? nullptr : x,
                      ssp, ld, kv_len, max_ctx, kvl, c->err, plan, st));
  }
  const int ns_o = mx ? residual_nsplit(M, H, Hq * D) : 0, ns_d = mx || kDownSplit ? residual_nsplit(M, H, I) : 0;
  const ActIn xin = mx ? ActIn{x8, xs8} : ActIn{x, nullptr};
  const ActIn ain = mx ? ActIn{a8, as8} : ActIn{act, nullptr};
  // MXFP8 mode: each RMSNorm step reads the residual stream from one buffer
  // and writes the updated stream to the other (h, h2 alternate), so it can be
  // repeated.
  auto norm = [&](int nsplit, const float *gain) {
    const hipError_t e = launch_norm_mx8(h, h2, rpart, nsplit, gain, M, H, m.rms_eps, x8, xs8, nullptr, st);
    std::swap(h, h2);
    return e;
  };
  auto timed_norm = [&](int nsplit, const float *gain) -> int {
    Timed t(c, SPEC_K_RMSNORM, st);
    for (int r = 0; r + 1 < t.reps; ++r) {  // repeats recompute the same output from the same input
      CK(norm(nsplit, gain));
      std::swap(h, h2);
    }
    CK(norm(nsplit, gain));
    return SPEC_OK;
  };
  int pending = 0;  // MXFP8 mode: splits of the last residual projection not yet added to h
  for (int l = 0; l < m.n_layers; ++l) {
    const PackedLayer &L = c->layers[l];
    uint16_t *kc = c->kv.k_cache + l * lstride + seq0, *vc = c->kv.v_cache + l * lstride + seq0;
    if (mx) {
      const int rc = timed_norm(pending, L.attn_norm);
      if (rc) return rc;
    }
    QkvOut qo{q, kc, vc, kv_len, c->rope, Hq, Hkv, D, max_ctx, kvl, c->err};
    {
      Timed t(c, SPEC_K_QKV, st);
      for (int r = 0; r < t.reps; ++r) CK(launch_qkv(xin, M, H, L.qkv, qo, nr, fx, st));
    }
    aa.k_cache = kc;
    aa.v_cache = vc;
    {
      Timed t(c, SPEC_K_ATTENTION, st);
      for (int r = 0; r < t.reps; ++r) CK(launch_attention_splits(aa, D, st));
    }
    {
      Timed t(c, SPEC_K_ATTN_MERGE, st);
      for (int r = 0; r < t.reps; ++r) CK(launch_attention_merge(aa, D, st));
    }
    {
      Timed t(c, SPEC_K_OPROJ, st);
      for (int r = 0; r < t.reps; ++r) {
        if (mx) CK(launch_residual_partial(ActIn{ao, nullptr}, M, H, Hq * D, L.o, rpart, st));
        else CK(launch_residual(kGemmOproj, ActIn{ao, nullptr}, M, H, Hq * D, L.o,
                                ResidualOut{h, h2, L.mlp_norm, x, 0, ssp, ld, c->err}, fx, st));
      }
    }
    if (mx) {
      const int rc = timed_norm(ns_o, L.mlp_norm);
      if (rc) return rc;
    }
    {
      Timed t(c, SPEC_K_GATE_UP, st);
      for (int r = 0; r < t.reps; ++r)
        CK(launch_swiglu(xin, M, H, I, L.gate_up, mx ? (void *)a8 : act, mx ? as8 : nullptr, nr, fx, st));
    }
    const bool last = l + 1 == m.n_layers;
    const float *next_gain = last ? c->final_norm : c->layers[l + 1].attn_norm;
    {
      Timed t(c, SPEC_K_DOWN, st);
      for (int r = 0; r < t.reps; ++r) {
        if (mx || kDownSplit) CK(launch_residual_partial(ain, M, H, I, L.down, rpart, st));
        else CK(launch_residual(kGemmDown, ain, M, H, I, L.down,
                                ResidualOut{h2, h, next_gain, x, last ? 1 : 0, ssp, ld, c->err}, fx, st));
      }
    }
    if (!mx && kDownSplit) {  // the down projection's K splits added to h, the next RMSNorm's input prepared
      Timed t(c, SPEC_K_RMSNORM, st);
      for (int r = 0; r < t.reps; ++r)
        CK(launch_fold(h2, h, rpart, ns_d, next_gain, M, H, x, last ? 1 : 0, ssp, ld, c->err, st));
    }
    pending = ns_d;
  }
  if (mx) {
    Timed t(c, SPEC_K_RMSNORM, st);
    for (int r = 0; r < t.reps; ++r)
      CK(launch_norm(h, nullptr, rpart, pending, c->final_norm, M, H, m.rms_eps, x, 1, dump_hidden, st));
  }
  {
    Timed t(c, SPEC_K_LM_HEAD, st);
    // the argmax does not need the final RMSNorm's (positive, per-row) scale;
    // only dumped logits are normalised
    for (int r = 0; r < t.reps; ++r)
      CK(launch_lm_argmax(x, M, V, H, c->lm_table, amax, dump_logits, dump_logits ? nr : NormRows{}, st));
  }
  if (dump_hidden && !mx) CK(launch_final_hidden(x, ssp, ld, H, m.rms_eps, M, nullptr, dump_hidden, nullptr, st));
  {
    Timed t(c, SPEC_K_ACCEPT, st);
    for (int r = 0; r < t.reps; ++r)
      CK(launch_accept(amax, lm_parts(V), M, tokens, batch, accept_len, bonus, argmax, last_tau, st));
  }
  return SPEC_OK;
}

extern "C" {

int spec_verify_block(spec_ctx *c, int32_t batch, const int32_t *tokens, int32_t *accept_len, int32_t *bonus,
                      int32_t *argmax, hipStream_t st) {
  static const char *fn = "spec_verify_block";
  if (!c || !tokens || !accept_len || !bonus) return fail(SPEC_E_ARG, fn, "NULL argument");
  if (batch < 1 || batch > c->kv.max_batch) return fail(SPEC_E_ARG, fn, "batch outside [1, max_batch]");
  // a timed kernel class is measured on one stream
  const int nl = c->prof_kind != SPEC_K_NONE ? 1 : std::min<int>(c->lanes, batch);
  if (nl == 1) return run_pass(c, 0, 0, batch, tokens, accept_len, bonus, argmax, st);
  // fork: lanes 1.. wait for the caller's stream; join: the caller waits for
  // every forked lane, also when a lane's pass fails part-way (so the
  // caller's stream stays ordered after all work already queued, and a
  // capture sees every branch joined)
  CK(hipEventRecord(c->lane_ev[0], st));
  int forked = 1;
  for (; forked < nl; ++forked)
    if (hipStreamWaitEvent(c->lane_st[forked], c->lane_ev[0], 0) != hipSuccess) break;
  int rc = forked == nl ? SPEC_OK : fail(SPEC_E_HIP, fn, "hipStreamWaitEvent (fork)");
  for (int i = 0; i < forked && rc == SPEC_OK; ++i) {
    const int b0 = batch * i / nl, b1 = batch * (i + 1) / nl;
    rc = run_pass(c, i, b0, b1 - b0, tokens + 16 * b0, accept_len + b0, bonus + b0,
                  argmax ? argmax + 16 * b0 : nullptr, i ? c->lane_st[i] : st);
  }
  for (int i = 1; i < forked; ++i) {
    const hipError_t e1 = hipEventRecord(c->lane_ev[i], c->lane_st[i]);
    const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(st, c->lane_ev[i], 0) : e1;
    if (e2 != hipSuccess && rc == SPEC_OK) rc = fail(SPEC_E_HIP, fn, "lane join", e2);
  }
  return rc;
}

int spec_verify_set_lanes(spec_ctx *c, int32_t lanes) {
  static const char *fn = "spec_verify_set_lanes";
  if (!c || lanes < 1 || lanes > SPEC_MAX_LANES) return fail(SPEC_E_ARG, fn, "lanes outside [1, SPEC_MAX_LANES]");
  if (lanes > 1 && !c->lane_ws) {
    size_t per = 0;
    for (size_t b : c->lane_bytes) per += round256(b);
    void *ws = nullptr;
    if (hipMalloc(&ws, per * (SPEC_MAX_LANES - 1)) != hipSuccess) return fail(SPEC_E_NOMEM, fn, "lane buffers");
    c->lane_ws = ws;
    char *p = (char *)ws;
    for (int i = 1; i < SPEC_MAX_LANES; ++i) {
      spec_ctx::LaneBufs &lb = c->lane_buf[i];
      lb.part_o = (uint16_t *)p;
      p += round256(c->lane_bytes[0]);
      lb.part_ml = (float2 *)p;
      p += round256(c->lane_bytes[1]);
      lb.rpart = (float *)p;
      p += round256(c->lane_bytes[2]);
      lb.plan = (int4 *)p;
      p += round256(c->lane_bytes[3]);
      lb.fx = c->lane_buf[0].fx;
      lb.fx.part = (float *)p;
      p += round256(c->lane_bytes[4]);
      lb.fx.cnt = (int *)p;
      p += round256(c->lane_bytes[5]);
    }
    CK(hipMemset(ws, 0, per * (SPEC_MAX_LANES - 1)));  // the split counters start at zero
    for (int i = 1; i < SPEC_MAX_LANES; ++i) CK(hipStreamCreateWithFlags(&c->lane_st[i], hipStreamNonBlocking));
    for (hipEvent_t &e : c->lane_ev) CK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  c->lanes = lanes;
  return SPEC_OK;
}

int spec_prefill(spec_ctx *c, int32_t batch, const int32_t *prompt, int32_t T, const int32_t *lengths,
                 int32_t *pending, uint16_t *anchor_hidden, hipStream_t st) {
  static const char *fn = "spec_prefill";
  if (!c || !prompt || !lengths || !pending) return fail(SPEC_E_ARG, fn, "NULL argument");
  if (batch < 1 || batch > c->kv.max_batch || T < 1) return fail(SPEC_E_ARG, fn, "batch or T out of range");
  if (anchor_hidden && !aligned16(anchor_hidden)) return fail(SPEC_E_ARG, fn, "anchor_hidden not 16-byte aligned");
  const int H = c->m.hidden;
  const bool mx = c->m.act_fmt == SPEC_ACT_MXFP8;
  for (int ch = 0; ch * 16 < T; ++ch) {
    CK(launch_prefill_gather(prompt, T, lengths, ch, batch, c->pf_tokens, c->err, st));
    const int rc = spec_verify_block(c, batch, c->pf_tokens, c->pf_acc, c->pf_bonus, c->pf_argmax, st);
    if (rc != SPEC_OK) return rc;
    CK(launch_prefill_finish(lengths, T, ch, batch, c->pf_argmax, c->pf_ncommit, pending, c->last_tau, c->pf_sel,
                             st));
    if (anchor_hidden)  // the final hidden state of each prompt's last row, for prompts that end in this chunk
      CK(launch_final_hidden(c->x, mx ? nullptr : c->ssp, c->ld, H, c->m.rms_eps, batch, c->pf_sel, nullptr,
                             anchor_hidden, st));
    CK(launch_commit(batch, c->pf_ncommit, c->last_tau, c->kv.kv_len, c->kv.max_ctx, c->err, st));
  }
  return SPEC_OK;
}

int spec_export_hidden(spec_ctx *c, int32_t batch, uint16_t *out, hipStream_t st) {
  static const char *fn = "spec_export_hidden";
  if (!c || !out || !aligned16(out)) return fail(SPEC_E_ARG, fn, "NULL or misaligned argument");
  if (batch < 1 || batch > c->kv.max_batch) return fail(SPEC_E_ARG, fn, "batch outside [1, max_batch]");
  const bool mx = c->m.act_fmt == SPEC_ACT_MXFP8;
  CK(launch_final_hidden(c->x, mx ? nullptr : c->ssp, c->ld, c->m.hidden, c->m.rms_eps, batch, c->last_tau, nullptr,
                         out, st));
  return SPEC_OK;
}

int spec_commit_kv(spec_ctx *c, int32_t batch, const int32_t *n_commit, hipStream_t st) {
  static const char *fn = "spec_commit_kv";
  if (!c) return fail(SPEC_E_ARG, fn, "NULL context");
  if (batch < 1 || batch > c->kv.max_batch) return fail(SPEC_E_ARG, fn, "batch outside [1, max_batch]");
  {
    Timed t(c, SPEC_K_COMMIT, st);
    CK(launch_commit(batch, n_commit, c->last_tau, c->kv.kv_len, c->kv.max_ctx, c->err, st));
  }
  return SPEC_OK;
}

int spec_verify_destroy(spec_ctx *c) {
  if (!c) return SPEC_OK;
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->lane_ev)
    if (e) (void)hipEventDestroy(e);
  for (hipStream_t s : c->lane_st)
    if (s) (void)hipStreamDestroy(s);
  if (c->lane_ws) (void)hipFree(c->lane_ws);
  const hipError_t e1 = hipFree(c->wbuf);
  const hipError_t e = hipFree(c->ws);
  delete c;
  return e == hipSuccess && e1 == hipSuccess ? SPEC_OK
                                              : fail(SPEC_E_HIP, "spec_verify_destroy", "hipFree", e != hipSuccess ? e : e1);
}

int spec_get_device_error(spec_ctx *c, int32_t *code, hipStream_t st) {
  if (!c || !code) return fail(SPEC_E_ARG, "spec_get_device_error", "NULL argument");
  int32_t v = 0;
  CK(hipMemcpyAsync(&v, c->err, 4, hipMemcpyDeviceToHost, st));
  CK(hipStreamSynchronize(st));
  CK(launch_fill_i32(c->err, 1, 0, st));
  CK(hipStreamSynchronize(st));
  *code = v;
  return SPEC_OK;
}

int spec_debug_set_repeat(spec_ctx *c, int32_t repeat) {
  if (!c || repeat < 1 || repeat > 64) return fail(SPEC_E_ARG, "spec_debug_set_repeat", "repeat outside [1, 64]");
  c->prof_repeat = repeat;
  return SPEC_OK;
}

int spec_debug_time_kernel(spec_ctx *c, int32_t kind) {
  if (!c || kind < SPEC_K_NONE || kind > SPEC_K_ATTN_MERGE) return fail(SPEC_E_ARG, "spec_debug_time_kernel", "kind");
  if (kind != SPEC_K_NONE && c->ev.empty()) {
    c->ev.resize(2 * kMaxTimedLaunches);
    for (hipEvent_t &e : c->ev) CK(hipEventCreate(&e));
  }
  c->prof_kind = kind;
  return SPEC_OK;
}

int spec_debug_kernel_time(spec_ctx *c, float *total_ms, int32_t *launches) {
  if (!c || !total_ms || !launches) return fail(SPEC_E_ARG, "spec_debug_kernel_time", "NULL argument");
  float sum = 0.f;
  for (size_t i = 0; i + 1 < c->ev_used; i += 2) {
    float ms = 0.f;
    CK(hipEventSynchronize(c->ev[i + 1]));
    CK(hipEventElapsedTime(&ms, c->ev[i], c->ev[i + 1]));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int32_t)c->ev_launches;
  c->ev_used = c->ev_launches = 0;
  return SPEC_OK;
}

int spec_debug_set_dump(spec_ctx *c, float *hidden, float *logits) {
  if (!c) return fail(SPEC_E_ARG, "spec_debug_set_dump", "NULL context");
  if ((hidden && !aligned16(hidden)) || (logits && !aligned16(logits)))
    return fail(SPEC_E_ARG, "spec_debug_set_dump", "buffers not 16-byte aligned");
  c->dump_hidden = hidden;
  c->dump_logits = logits;
  return SPEC_OK;
}

}  // extern "C"

// A test hook's packed copy of a row-major matrix (freed with the object).
struct TempPacked {
  void *buf = nullptr;
  LinearW w{};
  hipError_t make(int wfmt, int rows, int cols, const void *src, const void *s, int map, int mp, hipStream_t st) {
    const hipError_t e = hipMalloc(&buf, packed_bytes(wfmt, rows, cols));
    if (e != hipSuccess) return e;
    char *cur = (char *)buf;
    return pack_one(wfmt, rows, cols, src, s, map, mp, cur, w, st);
  }
  ~TempPacked() {
    if (buf) (void)hipFree(buf);
  }
};

extern "C" {

int spec_debug_linear(int32_t M, int32_t N, int32_t K, const uint16_t *x, const void *w, const void *scales,
                      int32_t wfmt, float *y, hipStream_t st) {
  static const char *fn = "spec_debug_linear";
  if (M < 1 || N < 64 || K < 64 || N % 64 || K % 64 || !x || !w || !y) return fail(SPEC_E_ARG, fn, "shape or NULL");
  if (wfmt != SPEC_WFMT_BF16 && !scales) return fail(SPEC_E_ARG, fn, "scales missing");
  if (wfmt != SPEC_WFMT_BF16 && wfmt != SPEC_WFMT_FP8_E4M3_ROW && wfmt != SPEC_WFMT_MXFP4)
    return fail(SPEC_E_UNSUPPORTED, fn, "weight format");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (wfmt == SPEC_WFMT_FP8_E4M3_ROW && !aligned16(scales)))
    return fail(SPEC_E_ARG, fn, "alignment");
  TempPacked p;
  CK(p.make(wfmt, N, K, w, scales, kRowsPlain, 0, st));
  CK(launch_linear_f32(ActIn{x, nullptr}, M, N, K, p.w, y, st));
  CK(hipStreamSynchronize(st));
  return SPEC_OK;
}

// the in-launch split workspace of one decoder GEMM (freed at scope exit), so
// that the debug hooks run the launch shapes the pass runs
struct TempSplit {
  void *buf = nullptr;
  SplitWs ws{};
  hipError_t make(int kind, int M, int tiles, int ksteps) {
    size_t f = 0;
    int n = 0;
    split_ws_need(kind, M, tiles, ksteps, &f, &n);
    if (!f) return hipSuccess;
    const size_t pb = round256(f * 4);
    hipError_t e = hipMalloc(&buf, pb + (size_t)n * 4);
    if (e == hipSuccess) e = hipMemset((char *)buf + pb, 0, (size_t)n * 4);
    ws = SplitWs{(float *)buf, (int *)((char *)buf + pb), f, n};
    return e;
  }
  const SplitWs *get() const { return buf ? &ws : nullptr; }
  ~TempSplit() {
    if (buf) (void)hipFree(buf);
  }
};

int spec_debug_residual(int32_t M, int32_t N, int32_t K, const uint16_t *x, const void *w, const void *scales,
                        int32_t wfmt, const float *h_in, const float *gain, int32_t xg_bf16, float *h_out,
                        uint16_t *xg, float *ssp, hipStream_t st) {
  static const char *fn = "spec_debug_residual";
  if (M < 1 || N < 64 || K < 64 || N % 64 || K % 64 || N > 4096 || !x || !w || !scales || !h_in || !gain || !h_out ||
      !xg || !ssp)
    return fail(SPEC_E_ARG, fn, "shape or NULL");
  if (wfmt != SPEC_WFMT_FP8_E4M3_ROW && wfmt != SPEC_WFMT_MXFP4) return fail(SPEC_E_UNSUPPORTED, fn, "weight format");
  if (!aligned16(x) || !aligned16(w) || !aligned16(h_in) || !aligned16(gain) || !aligned16(h_out) || !aligned16(xg) ||
      !aligned16(ssp) || (wfmt == SPEC_WFMT_FP8_E4M3_ROW && !aligned16(scales)) || h_in == h_out)
    return fail(SPEC_E_ARG, fn, "alignment or aliasing");
  TempPacked p;
  CK(p.make(wfmt, N, K, w, scales, kRowsPlain, 0, st));
  const int kind = K > 1024 ? kGemmDown : kGemmOproj;
  TempSplit fx;
  CK(fx.make(kind, M, N / 32, K / 64));
  CK(launch_residual(kind, ActIn{x, nullptr}, M, N, K, p.w,
                     ResidualOut{h_in, h_out, gain, xg, xg_bf16 ? 1 : 0, ssp, ssp_ld(N), nullptr}, fx.get(), st));
  CK(hipStreamSynchronize(st));
  return SPEC_OK;
}

int spec_debug_quant_mx8(int32_t M, int32_t K, const float *x, uint8_t *codes, uint8_t *scales, hipStream_t st) {
  static const char *fn = "spec_debug_quant_mx8";
  if (M < 1 || K < 32 || K % 32 || !x || !codes || !scales) return fail(SPEC_E_ARG, fn, "shape or NULL");
  if (!aligned16(x) || !aligned16(codes)) return fail(SPEC_E_ARG, fn, "alignment");
  CK(launch_quant_mx8(x, M, K, codes, scales, st));
  CK(hipStreamSynchronize(st));
  return SPEC_OK;
}

int spec_debug_rmsnorm(int32_t M, int32_t H, const float *h, const float *gain, float eps, int32_t act_fmt, void *x,
                       uint8_t *xs, hipStream_t st) {
  static const char *fn = "spec_debug_rmsnorm";
  if (M < 1 || H < 32 || H > 4096 || H % 32 || !h || !gain || !x || !(eps > 0.f)) return fail(SPEC_E_ARG, fn, "shape");
  if (!aligned16(h) || !aligned16(gain) || !aligned16(x)) return fail(SPEC_E_ARG, fn, "alignment");
  if (act_fmt == SPEC_ACT_FP16) {
    CK(launch_norm(h, nullptr, nullptr, 0, gain, M, H, eps, (uint16_t *)x, 0, nullptr, st));
  } else if (act_fmt == SPEC_ACT_MXFP8) {
    if (!xs) return fail(SPEC_E_ARG, fn, "xs missing");
    CK(launch_norm_mx8(h, nullptr, nullptr, 0, gain, M, H, eps, (uint8_t *)x, xs, nullptr, st));
  } else {
    return fail(SPEC_E_UNSUPPORTED, fn, "activation format");
  }
  CK(hipStreamSynchronize(st));
  return SPEC_OK;
}

int spec_debug_swiglu(int32_t M, int32_t H, int32_t I, const void *x, const uint8_t *x_scales, const void *w,
                      const void *scales, int32_t wfmt, int32_t out_fmt, void *a, uint8_t *a_scales, hipStream_t st) {
  static const char *fn = "spec_debug_swiglu";
  if (M < 1 || H < 64 || I < 64 || H % 64 || I % 64 || !x || !w || !scales || !a) return fail(SPEC_E_ARG, fn, "shape");
  if (wfmt != SPEC_WFMT_FP8_E4M3_ROW && wfmt != SPEC_WFMT_MXFP4) return fail(SPEC_E_UNSUPPORTED, fn, "weight format");
  if (out_fmt != SPEC_ACT_FP16 && out_fmt != SPEC_ACT_MXFP8) return fail(SPEC_E_UNSUPPORTED, fn, "output format");
  if (out_fmt == SPEC_ACT_MXFP8 && !a_scales) return fail(SPEC_E_ARG, fn, "a_scales missing");
  if (!aligned16(x) || !aligned16(w) || !aligned16(a) || (wfmt == SPEC_WFMT_FP8_E4M3_ROW && !aligned16(scales)))
    return fail(SPEC_E_ARG, fn, "alignment");
  TempPacked p;
  CK(p.make(wfmt, 2 * I, H, w, scales, kRowsSwiglu, I, st));
  TempSplit fx;
  CK(fx.make(kGemmGateUp, M, 2 * I / 32, H / 64));
  CK(launch_swiglu(ActIn{x, x_scales}, M, H, I, p.w, a, out_fmt == SPEC_ACT_MXFP8 ? a_scales : nullptr, NormRows{},
                   fx.get(), st));
  CK(hipStreamSynchronize(st));
  return SPEC_OK;
}

int spec_debug_linear_mx8(int32_t M, int32_t N, int32_t K, const uint8_t *x_codes, const uint8_t *x_scales,
                          const void *w, const void *scales, int32_t wfmt, float *y, hipStream_t st) {
  static const char *fn = "spec_debug_linear_mx8";
  if (M < 1 || N < 64 || K < 64 || N % 64 || K % 64 || !x_codes || !x_scales || !w || !scales || !y)
    return fail(SPEC_E_ARG, fn, "shape or NULL");
  if (wfmt != SPEC_WFMT_FP8_E4M3_ROW && wfmt != SPEC_WFMT_MXFP4) return fail(SPEC_E_UNSUPPORTED, fn, "weight format");
  if (!aligned16(x_codes) || !aligned16(w) || !aligned16(y) || (wfmt == SPEC_WFMT_FP8_E4M3_ROW && !aligned16(scales)))
    return fail(SPEC_E_ARG, fn, "alignment");
  TempPacked p;
  CK(p.make(wfmt, N, K, w, scales, kRowsPlain, 0, st));
  CK(launch_linear_f32(ActIn{x_codes, x_scales}, M, N, K, p.w, y, st));
  CK(hipStreamSynchronize(st));
  return SPEC_OK;
}

int spec_debug_attention(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_batch, int32_t max_ctx,
                         const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                         const int32_t *kv_len, uint16_t *o, int32_t split_len, hipStream_t st) {
  static const char *fn = "spec_debug_attention";
  if (!q || !k_cache || !v_cache || !kv_len || !o) return fail(SPEC_E_ARG, fn, "NULL argument");
  if (batch < 1 || batch > max_batch || Hkv < 1 || Hq % Hkv || Hq / Hkv > 8 || max_ctx < 16)
    return fail(SPEC_E_ARG, fn, "shape");
  if (D != 64 && D != 128) return fail(SPEC_E_SHAPE, fn, "head_dim");
  if (split_len < 0 || split_len % 64) return fail(SPEC_E_ARG, fn, "split_len");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o)) return fail(SPEC_E_ARG, fn, "alignment");
  // the merge step holds at most 64 splits per sequence
  if (split_len && (max_ctx + split_len - 1) / split_len > 64) return fail(SPEC_E_ARG, fn, "more than 64 splits");
  AttnPlanArgs p = attention_plan_args(nullptr, batch, Hq, Hkv, max_ctx, D, split_len, attention_device_cus());
  AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.o = o;
  a.batch = batch;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_ctx = max_ctx;
  a.grid = p.grid;
  const size_t units = (size_t)p.grid, R = (size_t)(Hq / Hkv) * 16;
  void *buf = nullptr;
  if (hipMalloc(&buf, units * R * D * 2 + units * R * 8 + (1 + (size_t)batch) * 16) != hipSuccess)
    return fail(SPEC_E_NOMEM, fn, "partials");
  a.part_o = (uint16_t *)buf;
  a.part_ml = (float2 *)((char *)buf + units * R * D * 2);
  p.plan = (int4 *)((char *)buf + units * R * D * 2 + units * R * 8);
  a.plan = p.plan;
  hipError_t e = launch_attention_plan(kv_len, p, st);
  if (e == hipSuccess) e = launch_attention(a, D, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  (void)hipFree(buf);
  return e == hipSuccess ? SPEC_OK : fail(SPEC_E_HIP, fn, "attention launch", e);
}

}  // extern "C"

// ---- block-causal attention without allocation ----
// For callers that cannot allocate device memory: the split partials and the
// split plan live in this static device buffer.  Host code never names it
// directly (its name is a host-side stand-in); each device's address of it is
// looked up once, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[SPEC_ATTN_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64] = {};

static int scratch_ptr(const char *fn, void **out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPEC_E_HIP, fn, "hipGetDevice", e);
  if (dev < 0 || dev >= 64) return fail(SPEC_E_ARG, fn, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || !p) return fail(SPEC_E_HIP, fn, "hipGetSymbolAddress(scratch)", es);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

extern "C" int spec_debug_attention_noalloc(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_batch,
                                            int32_t max_ctx, const uint16_t *q, const uint16_t *k_cache,
                                            const uint16_t *v_cache, const int32_t *kv_len, uint16_t *o,
                                            int32_t split_len, hipStream_t st) {
  static const char *fn = "spec_debug_attention_noalloc";
  if (!q || !k_cache || !v_cache || !kv_len || !o) return fail(SPEC_E_ARG, fn, "NULL argument");
  if (batch < 1 || batch > max_batch || Hkv < 1 || Hq % Hkv || Hq / Hkv > 8 || max_ctx < 16)
    return fail(SPEC_E_ARG, fn, "shape");
  if (D != 64 && D != 128) return fail(SPEC_E_SHAPE, fn, "head_dim");
  if (split_len < 0 || split_len % 64) return fail(SPEC_E_ARG, fn, "split_len");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o)) return fail(SPEC_E_ARG, fn, "alignment");
  if (split_len && (max_ctx + split_len - 1) / split_len > 64) return fail(SPEC_E_ARG, fn, "more than 64 splits");
  AttnPlanArgs p = attention_plan_args(nullptr, batch, Hq, Hkv, max_ctx, D, split_len, attention_device_cus());
  const size_t units = (size_t)p.grid, R = (size_t)(Hq / Hkv) * 16;
  const size_t o_bytes = round256(units * R * D * 2), ml_bytes = round256(units * R * 8);
  const size_t plan_bytes = round256((1 + (size_t)batch) * 16);
  if (o_bytes + ml_bytes + plan_bytes > SPEC_ATTN_SCRATCH_BYTES)
    return fail(SPEC_E_ARG, fn, "split partials exceed SPEC_ATTN_SCRATCH_BYTES");
  void *buf = nullptr;
  const int rc = scratch_ptr(fn, &buf);
  if (rc != SPEC_OK) return rc;
  AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.o = o;
  a.batch = batch;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_ctx = max_ctx;
  a.grid = p.grid;
  a.part_o = (uint16_t *)buf;
  a.part_ml = (float2 *)((char *)buf + o_bytes);
  p.plan = (int4 *)((char *)buf + o_bytes + ml_bytes);
  a.plan = p.plan;
  CK(launch_attention_plan(kv_len, p, st));  // writes the whole plan: nothing in the buffer needs clearing
  CK(launch_attention(a, D, st));
  return SPEC_OK;
}
