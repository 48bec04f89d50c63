// Internal launchers shared by the kernel sources and the C-ABI host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ---- weight-streaming linear: y = x W^T, x bf16 [M][K], W rows in wfmt ----
struct LinearW {
  const void *w;   // codes / bf16 rows
  const void *s;   // fp32 per-row scales (FP8), e8m0 [rows][K/32] (MXFP4), NULL (BF16)
  int wfmt;
};

// y fp32 [M][N] (test hook)
hipError_t launch_linear_f32(const uint16_t *x, int M, int N, int K, LinearW w, float *y, hipStream_t st);

// QKV projection + RoPE; q -> q_out bf16 [M][Hq*D]; k, v -> caches at slot kv_len[b] + j.
struct QkvOut {
  uint16_t *q_out;
  uint16_t *k_cache, *v_cache;  // layer base, [max_batch][Hkv][max_ctx][D]
  const int32_t *kv_len;
  const float2 *rope;           // [max_ctx][D/2] (cos, sin)
  int Hq, Hkv, max_ctx;
};
hipError_t launch_qkv(const uint16_t *x, int M, int H, int D, LinearW w, QkvOut o, hipStream_t st);

// a[m][n] = bf16(SiLU(x Wg^T) * (x Wu^T)), W = [gate; up] with I rows each
hipError_t launch_swiglu(const uint16_t *x, int M, int H, int I, LinearW w, uint16_t *a, hipStream_t st);

// h[m][n] += (x W^T)[m][n], h fp32 [M][N]
hipError_t launch_residual(const uint16_t *x, int M, int N, int K, LinearW w, float *h, hipStream_t st);

// lm_head + per-wave argmax partials: part[p][m] over vocab slices of 64
struct ArgmaxPart { float v; int32_t i; };
hipError_t launch_lm_argmax(const uint16_t *x, int M, int V, int H, const uint16_t *table,
                            ArgmaxPart *part, float *logits_dump, hipStream_t st);
inline int lm_parts(int V) { return V / 64; }

// ---- attention ----
struct AttnArgs {
  const uint16_t *q;                 // [M][Hq*D]
  const uint16_t *k_cache, *v_cache; // layer base
  const int32_t *kv_len;
  uint16_t *o;                       // [M][Hq*D]
  float *part_o;                     // [B][Hkv][nsplit][G*16][D]
  float2 *part_ml;                   // [B][Hkv][nsplit][G*16]
  int32_t *counters;                 // [B][Hkv], zero between launches
  int batch, Hq, Hkv, max_ctx, split_len, nsplit;
};
hipError_t launch_attention(const AttnArgs &a, int D, hipStream_t st);
int attention_split_len(int batch, int Hkv, int max_ctx);

// ---- small kernels ----
hipError_t launch_embed(const int32_t *tokens, int M, int H, int V, const uint16_t *table, float *h,
                        const int32_t *kv_len, int max_ctx, int32_t *err, hipStream_t st);
hipError_t launch_rmsnorm(const float *h, const float *gain, int M, int H, float eps, uint16_t *x,
                          float *dump, hipStream_t st);
hipError_t launch_accept(const ArgmaxPart *part, int nparts, int M, const int32_t *tokens, int batch,
                         int32_t *accept_len, int32_t *bonus, int32_t *argmax, int32_t *last_tau,
                         hipStream_t st);
hipError_t launch_commit(int batch, const int32_t *n_commit, const int32_t *last_tau, int32_t *kv_len,
                         int max_ctx, int32_t *err, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t st);
