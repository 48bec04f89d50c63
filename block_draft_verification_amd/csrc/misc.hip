// Embedding gather, RMSNorm, argmax reduction + prefix accept, KV commit,
// weight packing, the final hidden state.
#include "attn_plan.h"
#include "common.h"
#include "kernels.h"

__device__ __forceinline__ void store_bf16x4_misc(uint16_t *p, f32x4_t v) {
  *reinterpret_cast<u32x2_t *>(p) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// h[m][:] = E[t[m]][:] (BF16 -> fp32, the row-major table).  With xg set,
// also the first RMSNorm's input for the QKV step: xg = h * gain (FP16) and
// the sum of h^2 over each 32 columns into ssp[m][.] (the row's remaining
// entries zeroed).  Also checks that every sequence's block fits its cache
// (kv_len + 16 <= max_ctx); the QKV step skips the K/V writes of a sequence
// that does not.  One wave of the launch also computes the attention split
// plan of the pass (attn_plan.h), which depends only on kv_len: every
// attention launch of the pass then reads it.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ tokens, int H, int V,
                                                    const uint16_t *__restrict__ table, float *__restrict__ h,
                                                    const float *__restrict__ gain, uint16_t *__restrict__ xg,
                                                    float *__restrict__ ssp, int ld,
                                                    const int32_t *__restrict__ kv_len, int max_ctx, KvLayout kvl,
                                                    int32_t *err, AttnPlanArgs plan) {
  const int m = blockIdx.x;
  // the last workgroup's last wave also writes the pass's attention split plan
  if (plan.plan && m == (int)gridDim.x - 1 && threadIdx.x >= blockDim.x - 64)
    attn_plan_wave(kv_len, plan, threadIdx.x & 63);
  int t = tokens[m];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) set_error(err, SPEC_DERR_TOKEN);
    t = 0;
  }
  if ((m & 15) == 0 && threadIdx.x == 0) {
    const int n = kv_len[m >> 4];
    if (n < 0 || n + 16 > max_ctx) {
      set_error(err, SPEC_DERR_CAPACITY);
    } else if (kvl.pages) {  // every page the pass reads or writes: positions 0 .. n+15
      for (int p = 0; p < n + 16; p += kvl.page_size) {
        const int pg = kvl.pages[(size_t)(m >> 4) * kvl.max_pages + p / kvl.page_size];
        if (pg < 0 || pg >= kvl.num_pages) set_error(err, SPEC_DERR_PAGE);
      }
    }
  }
  // 8 columns (one 16-byte chunk of the row) per thread; the 4 threads of a
  // 32-column group are consecutive lanes and run every iteration together
  const uint16_t *src = table + (size_t)t * H;
  for (int k0 = 8 * threadIdx.x; k0 - 8 * (int)threadIdx.x < H; k0 += 8 * blockDim.x) {
    const bool in = k0 < H;
    const u32x4_t v = in ? *reinterpret_cast<const u32x4_t *>(src + k0) : u32x4_t{0u, 0u, 0u, 0u};
    const f32x4_t a = f32x4_t{bf16_to_f32(v.x & 0xffff), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffff),
                              bf16_to_f32(v.y >> 16)};
    const f32x4_t b = f32x4_t{bf16_to_f32(v.z & 0xffff), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xffff),
                              bf16_to_f32(v.w >> 16)};
    float ss = ((a[0] * a[0] + a[1] * a[1]) + (a[2] * a[2] + a[3] * a[3])) +
               ((b[0] * b[0] + b[1] * b[1]) + (b[2] * b[2] + b[3] * b[3]));
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (!in) continue;
    float *o = h + (size_t)m * H + k0;
    *reinterpret_cast<f32x4_t *>(o) = a;
    *reinterpret_cast<f32x4_t *>(o + 4) = b;
    if (xg) {
      const f32x4_t g0 = *reinterpret_cast<const f32x4_t *>(gain + k0), g1 = *reinterpret_cast<const f32x4_t *>(gain + k0 + 4);
      const f32x4_t x0 = a * g0, x1 = b * g1;
      *reinterpret_cast<u32x4_t *>(xg + (size_t)m * H + k0) =
          u32x4_t{pack_f16x2(x0[0], x0[1]), pack_f16x2(x0[2], x0[3]), pack_f16x2(x1[0], x1[1]), pack_f16x2(x1[2], x1[3])};
      const float mx = fmaxf(fmaxf(fmaxf(fabsf(x0[0]), fabsf(x0[1])), fmaxf(fabsf(x0[2]), fabsf(x0[3]))),
                             fmaxf(fmaxf(fabsf(x1[0]), fabsf(x1[1])), fmaxf(fabsf(x1[2]), fabsf(x1[3]))));
      if (!(mx <= 65504.f)) set_error(err, SPEC_DERR_RANGE);
      if ((k0 & 31) == 0) ssp[(size_t)m * ld + k0 / 32] = ss;
    }
  }
  if (xg && (int)threadIdx.x < ld - H / 32) ssp[(size_t)m * ld + H / 32 + threadIdx.x] = 0.f;
}

// Row-major -> tile-major weights (the layout kernels.h describes) in the row
// order of `map`: thread i writes destination chunk i (16 bytes) from one
// contiguous 16-byte run of its source row; MXFP4 scale tiles are written one
// byte per thread, FP8 row scales one float per thread.
template <int FMT>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ src, int rows, int cols,
                                                   uint8_t *__restrict__ dst, size_t nchunks, int map, int mp) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  constexpr int CPT = FMT == SPEC_WFMT_BF16 ? 256 : FMT == SPEC_WFMT_MXFP4 ? 64 : 128;  // chunks per tile
  const int ktiles = cols / 64;
  const size_t tile = i / CPT;
  const int q = (int)(i % CPT), j = q >> 6, l = q & 63, c = l & 31, hh = l >> 5;
  const int row = packed_row_source(map, (int)(tile / ktiles) * 32 + c, mp), kt = (int)(tile % ktiles);
  size_t off;  // byte offset of the chunk's first byte in the row-major source
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) off = (size_t)row * cols + kt * 64 + 16 * hh + 32 * j;
  else if constexpr (FMT == SPEC_WFMT_BF16) off = ((size_t)row * cols + kt * 64 + 32 * hh + 8 * j) * 2;
  else off = (size_t)row * (cols / 2) + (kt * 64 + 32 * hh) / 2;
  *reinterpret_cast<u32x4_t *>(dst + i * 16) = *reinterpret_cast<const u32x4_t *>(src + off);
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t *__restrict__ src, int rows, int cols,
                                                          uint8_t *__restrict__ dst, size_t n, int map, int mp) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int ktiles = cols / 64;
  const size_t tile = i / 64;
  const int l = (int)(i % 64), c = l & 31, hh = l >> 5;
  const int row = packed_row_source(map, (int)(tile / ktiles) * 32 + c, mp), kt = (int)(tile % ktiles);
  dst[i] = src[(size_t)row * (cols / 32) + 2 * kt + hh];
}

__global__ __launch_bounds__(256) void permute_rows_f32_kernel(const float *__restrict__ src, int rows,
                                                               float *__restrict__ dst, int map, int mp) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < rows) dst[p] = src[packed_row_source(map, p, mp)];
}

// Final normed hidden state from the lm_head's input: x = xg * r with r =
// 1 / sqrt(sum / H + eps) over the row's partial sums, added in the order the
// lm_head kernel adds them (lane chunks j = q + 8i summed per q, then over q),
// so x is the hidden state whose logits it took.
__global__ __launch_bounds__(256) void final_hidden_kernel(const uint16_t *__restrict__ xg,
                                                           const float *__restrict__ ssp, int ld, int H, float eps,
                                                           const int32_t *__restrict__ row_of, float *out_f32,
                                                           uint16_t *out_bf16) {
  __shared__ float rsh;
  const int b = blockIdx.x;
  int row = b;
  if (row_of) {
    const int r = row_of[b];
    if (r < 1 || r > 16) return;  // whole workgroup
    row = 16 * b + r - 1;
  }
  if (threadIdx.x == 0) {
    const int nch = ld / 4;
    float ss = 0.f;
    for (int q = 0; q < 8; ++q) {  // the lm_head's four-wave workgroup: 8 lane groups
      float ps = 0.f;
      for (int j = q; j < nch; j += 8) {
        const float *p = ssp + (size_t)row * ld + 4 * j;
        ps += (p[0] + p[1]) + (p[2] + p[3]);
      }
      ss += ps;
    }
    rsh = 1.0f / sqrtf(ss / (float)H + eps);
  }
  __syncthreads();
  const float r = rsh;
  for (int k = 4 * threadIdx.x; k < H; k += 4 * blockDim.x) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t *>(xg + (size_t)row * H + k);
    const f32x4_t x = f32x4_t{bf16_to_f32(v.x & 0xffff), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffff),
                              bf16_to_f32(v.y >> 16)} * r;
    if (out_f32) *reinterpret_cast<f32x4_t *>(out_f32 + (size_t)b * H + k) = x;
    if (out_bf16) store_bf16x4_misc(out_bf16 + (size_t)b * H + k, x);
  }
}

// h_out = h + part[0] + ... + part[ns-1] (split-K partials of the projection
// that just ran, added in split order; h_out may be NULL), then
// x = h_out / sqrt(mean(h_out^2) + eps) * gain
// rounded to FP16 (decoder layers) or BF16 (lm_head input).  One 256-thread
// workgroup per row; thread i owns the 4-column chunks c = 4i + 1024j (j < 4,
// so H <= 4096), and every load a thread needs -- its h and gain chunks, then
// the partials four splits at a time -- is issued before any of them is used,
// so a row costs one memory round trip and one block reduction.
// OUT: 0 FP16, 1 BF16, 2 MXFP8 (x = e4m3 codes, xs = e8m0 of each 32 columns;
// the 8 threads holding one 32-column block share its exponent by shuffles).
enum { kOutF16 = 0, kOutBF16 = 1, kOutMX8 = 2 };
template <int OUT>
__global__ __launch_bounds__(256) void norm_kernel(const float *__restrict__ h, float *__restrict__ h_out,
                                                   const float *__restrict__ part, int ns,
                                                   const float *__restrict__ gain, int M, int H, float eps,
                                                   void *__restrict__ x, uint8_t *__restrict__ xs,
                                                   float *__restrict__ dump) {
  pin_args(h, h_out, part, ns, gain, M, H, eps, x, xs, dump);
  constexpr int MAXC = 4;
  __shared__ float red[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float *hr = h + (size_t)m * H;
  float *ho = h_out ? h_out + (size_t)m * H : nullptr;
  const float *pr = part + (size_t)m * H;
  const size_t pstride = (size_t)M * H;
  f32x4_t t[MAXC], gv[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = 4 * tid + 1024 * i;
    if (c < H) {
      t[i] = *reinterpret_cast<const f32x4_t *>(hr + c);
      gv[i] = *reinterpret_cast<const f32x4_t *>(gain + c);
    }
  }
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    f32x4_t p[4][MAXC];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = 4 * tid + 1024 * i;
        if (c < H) p[q][i] = *reinterpret_cast<const f32x4_t *>(pr + (s + q) * pstride + c);
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < MAXC; ++i)
        if (4 * tid + 1024 * i < H) t[i] += p[q][i];
  }
  for (; s < ns; ++s) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = 4 * tid + 1024 * i;
      if (c < H) t[i] += *reinterpret_cast<const f32x4_t *>(pr + s * pstride + c);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = 4 * tid + 1024 * i;
    if (c < H) {
      if (ho) *reinterpret_cast<f32x4_t *>(ho + c) = t[i];
      ss += t[i][0] * t[i][0] + t[i][1] * t[i][1] + t[i][2] * t[i][2] + t[i][3] * t[i][3];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = 4 * tid + 1024 * i;
    if (c >= H) break;
    if constexpr (OUT == kOutMX8) {
      const f32x4_t y = f32x4_t{t[i][0] * rs * gv[i][0], t[i][1] * rs * gv[i][1], t[i][2] * rs * gv[i][2],
                                t[i][3] * rs * gv[i][3]};
      uint32_t e8;
      const uint32_t codes = mx8_quant4(y, e8);  // the block's 8 threads are all active (H % 32 == 0)
      *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(x) + (size_t)m * H + c) = codes;
      if ((tid & 7) == 0) xs[(size_t)m * (H / 32) + c / 32] = (uint8_t)e8;
      if (dump) {
        const float sc = __builtin_ldexpf(1.f, (int)e8 - 127);
        const u32x2_t hv = fp8x4_to_f16x4(codes);
        *reinterpret_cast<f32x4_t *>(dump + (size_t)m * H + c) =
            f32x4_t{f16_to_f32(hv.x & 0xffff), f16_to_f32(hv.x >> 16), f16_to_f32(hv.y & 0xffff),
                    f16_to_f32(hv.y >> 16)} * sc;
      }
      continue;
    }
    uint32_t lo, hi;
    if constexpr (OUT == kOutBF16) {
      lo = pack_bf16x2(t[i][0] * rs * gv[i][0], t[i][1] * rs * gv[i][1]);
      hi = pack_bf16x2(t[i][2] * rs * gv[i][2], t[i][3] * rs * gv[i][3]);
    } else {
      lo = pack_f16x2(t[i][0] * rs * gv[i][0], t[i][1] * rs * gv[i][1]);
      hi = pack_f16x2(t[i][2] * rs * gv[i][2], t[i][3] * rs * gv[i][3]);
    }
    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(x) + (size_t)m * H + c) = u32x2_t{lo, hi};
    if (dump) {
      f32x4_t o;
      if constexpr (OUT == kOutBF16)
        o = f32x4_t{bf16_to_f32(lo & 0xffff), bf16_to_f32(lo >> 16), bf16_to_f32(hi & 0xffff), bf16_to_f32(hi >> 16)};
      else
        o = f32x4_t{f16_to_f32(lo & 0xffff), f16_to_f32(lo >> 16), f16_to_f32(hi & 0xffff), f16_to_f32(hi >> 16)};
      *reinterpret_cast<f32x4_t *>(dump + (size_t)m * H + c) = o;
    }
  }
}

// The split-K partials of a residual projection added to the residual
// stream with the next RMSNorm's input prepared for its GEMM:
// h_out = h + part[0] + ... + part[ns-1] (in that order), xg = h_out * gain
// (FP16, or BF16 before the lm_head) and ssp[m][j] = sum of h_out^2 over
// columns 32j .. 32j+31 (the row's remaining entries zeroed); the
// normalisation itself is applied by the GEMM that reads xg.  One 256-thread
// workgroup per row as in norm_kernel; the 8 threads of a 32-column group
// are consecutive lanes.  An FP16 xg beyond the format's range sets
// SPEC_DERR_RANGE.
template <bool BF16>
__global__ __launch_bounds__(256) void fold_kernel(const float *__restrict__ h, float *__restrict__ h_out,
                                                   const float *__restrict__ part, int ns,
                                                   const float *__restrict__ gain, int M, int H,
                                                   uint16_t *__restrict__ xg, float *__restrict__ ssp, int ld,
                                                   int32_t *err) {
  pin_args(h, h_out, part, ns, gain, M, H, xg, ssp, ld, err);
  constexpr int MAXC = 4;
  const int m = blockIdx.x, tid = threadIdx.x;
  const float *hr = h + (size_t)m * H;
  const float *pr = part + (size_t)m * H;
  const size_t pstride = (size_t)M * H;
  f32x4_t t[MAXC], gv[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = 4 * tid + 1024 * i;
    t[i] = c < H ? *reinterpret_cast<const f32x4_t *>(hr + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    gv[i] = c < H ? *reinterpret_cast<const f32x4_t *>(gain + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  int s = 0;
  for (; s + 4 <= ns; s += 4) {  // four splits' loads issued together
    f32x4_t p[4][MAXC];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = 4 * tid + 1024 * i;
        p[q][i] = c < H ? *reinterpret_cast<const f32x4_t *>(pr + (s + q) * pstride + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < MAXC; ++i) t[i] += p[q][i];
  }
  for (; s < ns; ++s) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = 4 * tid + 1024 * i;
      if (c < H) t[i] += *reinterpret_cast<const f32x4_t *>(pr + s * pstride + c);
    }
  }
  bool range_ok = true;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = 4 * tid + 1024 * i;
    float ss = (t[i][0] * t[i][0] + t[i][1] * t[i][1]) + (t[i][2] * t[i][2] + t[i][3] * t[i][3]);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    if (c >= H) continue;
    *reinterpret_cast<f32x4_t *>(h_out + (size_t)m * H + c) = t[i];
    const f32x4_t x = t[i] * gv[i];
    uint32_t lo, hi;
    if constexpr (BF16) {
      lo = pack_bf16x2(x[0], x[1]);
      hi = pack_bf16x2(x[2], x[3]);
    } else {
      lo = pack_f16x2(x[0], x[1]);
      hi = pack_f16x2(x[2], x[3]);
      range_ok &= fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))) <= 65504.f;
    }
    *reinterpret_cast<u32x2_t *>(xg + (size_t)m * H + c) = u32x2_t{lo, hi};
    if ((c & 31) == 0) ssp[(size_t)m * ld + c / 32] = ss;
  }
  if (!range_ok) set_error(err, SPEC_DERR_RANGE);
  if (tid < ld - H / 32) ssp[(size_t)m * ld + H / 32 + tid] = 0.f;
}

// One workgroup of 16 waves per sequence, wave j = block row b*16+j:
// g[j] = argmax over the vocab partials of the row (lowest id on ties; lanes
// read the partials with independent loads, then a shuffle tree), then
// tau = first j >= 1 with t[j] != g[j-1] (16 if none) and bonus = g[tau-1]
// (HunyuanOCR-1.5 / DFlash write-up, inference loop, step 4).
__global__ __launch_bounds__(1024) void accept_kernel(const ArgmaxPart *__restrict__ part, int nparts, int M,
                                                      const int32_t *__restrict__ tokens, int32_t *accept_len,
                                                      int32_t *bonus, int32_t *argmax, int32_t *last_tau) {
  __shared__ int32_t gsh[16];
  const int b = blockIdx.x, j = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const ArgmaxPart *pr = part + (size_t)(b * 16 + j) * nparts;
  float bv = -INFINITY;
  int32_t bi = 0x7fffffff;
  int p = lane;
  for (; p + 192 < nparts; p += 256) {
    const ArgmaxPart q0 = pr[p], q1 = pr[p + 64], q2 = pr[p + 128], q3 = pr[p + 192];
    if (better(q0.v, q0.i, bv, bi)) bv = q0.v, bi = q0.i;
    if (better(q1.v, q1.i, bv, bi)) bv = q1.v, bi = q1.i;
    if (better(q2.v, q2.i, bv, bi)) bv = q2.v, bi = q2.i;
    if (better(q3.v, q3.i, bv, bi)) bv = q3.v, bi = q3.i;
  }
  for (; p < nparts; p += 64) {
    const ArgmaxPart q = pr[p];
    if (better(q.v, q.i, bv, bi)) bv = q.v, bi = q.i;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int32_t oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) bv = ov, bi = oi;
  }
  if (lane == 0) gsh[j] = bi == 0x7fffffff ? 0 : bi;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tau = 16;
    for (int k = 1; k < 16; ++k)
      if (tokens[b * 16 + k] != gsh[k - 1]) {
        tau = k;
        break;
      }
    accept_len[b] = tau;
    bonus[b] = gsh[tau - 1];
    last_tau[b] = tau;
  }
  if (argmax && threadIdx.x < 16) argmax[b * 16 + threadIdx.x] = gsh[threadIdx.x];
}

// kv_len[b] += n (n = n_commit[b], or the last verify's tau).  The block's
// K/V already sit in slots kv_len .. kv_len+15, so committing is a length
// bump and rejected rows are dropped by not counting them ("The Inference
// Stack Behind OCRia", verification section: rollback moves a pointer).
__global__ void commit_kernel(int batch, const int32_t *__restrict__ n_commit,
                              const int32_t *__restrict__ last_tau, int32_t *kv_len, int max_ctx,
                              int32_t *err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int n = n_commit ? n_commit[b] : last_tau[b];
  const int cur = kv_len[b];
  if (n < 0 || n > 16 || cur + n > max_ctx) {
    set_error(err, SPEC_DERR_COMMIT);
    return;
  }
  kv_len[b] = cur + n;
}

// Prefill through the verify pass: chunk c of every prompt goes through the
// pass as a 16-row block (rows past the prompt's end carry token 0), then all
// of the chunk's real rows are committed ("HunyuanOCR-1.5 / DFlash" write-up,
// inference loop, step 1: the target prefills the prompt before drafting).
__global__ void prefill_gather_kernel(const int32_t *__restrict__ prompt, int T, const int32_t *__restrict__ lens,
                                      int chunk, int32_t *tokens, int32_t *err) {
  const int b = blockIdx.x, j = threadIdx.x;
  const int len = lens[b];
  const bool ok = len >= 1 && len <= T;
  if (!ok && j == 0 && chunk == 0) set_error(err, SPEC_DERR_LENGTH);
  const int p = 16 * chunk + j;
  tokens[b * 16 + j] = ok && p < len ? prompt[(size_t)b * T + p] : 0;
}

// After chunk c: commit min(max(len - 16c, 0), 16) rows.  The chunk that holds
// a prompt's last token (r = len - 16c rows of it) also yields the pending token
// (the argmax at row r-1: the greedy next token after the prompt); sel[b] = r
// for it (0 otherwise) selects that row's final hidden state, the feature a
// block drafter is conditioned on.  last_tau = r, so the anchor row is
// last_tau - 1 as after a verify pass.
__global__ void prefill_finish_kernel(const int32_t *__restrict__ lens, int T, int chunk,
                                      const int32_t *__restrict__ argmax, int32_t *n_commit, int32_t *pending,
                                      int32_t *last_tau, int32_t *sel) {
  const int b = blockIdx.x;
  const int len = lens[b];
  const int rem = (len >= 1 && len <= T) ? len - 16 * chunk : 0;
  n_commit[b] = min(max(rem, 0), 16);
  const bool last = rem >= 1 && rem <= 16;
  sel[b] = last ? rem : 0;
  if (last) {
    pending[b] = argmax[b * 16 + rem - 1];
    last_tau[b] = rem;
  }
}

__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_embed(const int32_t *tokens, int M, int H, int V, const uint16_t *table, float *h,
                        const float *gain, uint16_t *xg, float *ssp, int ld, const int32_t *kv_len, int max_ctx,
                        KvLayout kvl, int32_t *err, const AttnPlanArgs &plan, hipStream_t st) {
  if (H % 32 || (xg && ld - H / 32 > 256)) return hipErrorInvalidValue;
  launch_k(embed_kernel, dim3(M), dim3(256), 0, st, tokens, H, V, table, h, gain, xg, ssp, ld, kv_len,
                     max_ctx, kvl, err, plan);
  return hipGetLastError();
}

hipError_t launch_final_hidden(const uint16_t *xg, const float *ssp, int ld, int H, float eps, int n,
                               const int32_t *row_of, float *out_f32, uint16_t *out_bf16, hipStream_t st) {
  if (H % 4 || n < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(final_hidden_kernel, dim3(n), dim3(256), 0, st, xg, ssp, ld, H, eps, row_of, out_f32, out_bf16);
  return hipGetLastError();
}

hipError_t launch_pack_weights(int wfmt, int rows, int cols, const void *w, const void *s, void *w_out, void *s_out,
                               int map, int mp, hipStream_t st) {
  if (rows % 32 || cols % 64 || rows < 32 || cols < 64) return hipErrorInvalidValue;
  if ((map == kRowsRope && (mp < 32 || mp % 32 || rows % mp)) || (map == kRowsSwiglu && (mp % 16 || rows != 2 * mp)))
    return hipErrorInvalidValue;
  const size_t tiles = (size_t)(rows / 32) * (cols / 64);
  const size_t chunks = tiles * (tile_bytes(wfmt) / 16);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  const uint8_t *src = static_cast<const uint8_t *>(w);
  uint8_t *dst = static_cast<uint8_t *>(w_out);
  if (wfmt == SPEC_WFMT_FP8_E4M3_ROW) {
    hipLaunchKernelGGL(pack_kernel<SPEC_WFMT_FP8_E4M3_ROW>, grid, dim3(256), 0, st, src, rows, cols, dst, chunks, map,
                       mp);
    if (s && s_out) {
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(permute_rows_f32_kernel, dim3((rows + 255) / 256), dim3(256), 0, st,
                         static_cast<const float *>(s), rows, static_cast<float *>(s_out), map, mp);
    }
  } else if (wfmt == SPEC_WFMT_BF16) {
    hipLaunchKernelGGL(pack_kernel<SPEC_WFMT_BF16>, grid, dim3(256), 0, st, src, rows, cols, dst, chunks, map, mp);
  } else if (wfmt == SPEC_WFMT_MXFP4) {
    hipLaunchKernelGGL(pack_kernel<SPEC_WFMT_MXFP4>, grid, dim3(256), 0, st, src, rows, cols, dst, chunks, map, mp);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const size_t n = tiles * 64;
    hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint8_t *>(s), rows, cols, static_cast<uint8_t *>(s_out), n, map, mp);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_norm(const float *h, float *h_out, const float *part, int nsplit, const float *gain, int M, int H,
                       float eps, uint16_t *x, int out_bf16, float *dump, hipStream_t st) {
  if (H > 4096 || H % 4 || h == h_out) return hipErrorInvalidValue;
  if (out_bf16)
    launch_k(norm_kernel<kOutBF16>, dim3(M), dim3(256), 0, st, h, h_out, part, nsplit, gain, M, H, eps,
                       (void *)x, (uint8_t *)nullptr, dump);
  else
    launch_k(norm_kernel<kOutF16>, dim3(M), dim3(256), 0, st, h, h_out, part, nsplit, gain, M, H, eps,
                       (void *)x, (uint8_t *)nullptr, dump);
  return hipGetLastError();
}

hipError_t launch_fold(const float *h, float *h_out, const float *part, int nsplit, const float *gain, int M, int H,
                       uint16_t *xg, int xg_bf16, float *ssp, int ld, int32_t *err, hipStream_t st) {
  if (H > 4096 || H % 32 || h == h_out || ld - H / 32 > 256) return hipErrorInvalidValue;
  if (xg_bf16)
    launch_k(fold_kernel<true>, dim3(M), dim3(256), 0, st, h, h_out, part, nsplit, gain, M, H, xg, ssp, ld,
                       err);
  else
    launch_k(fold_kernel<false>, dim3(M), dim3(256), 0, st, h, h_out, part, nsplit, gain, M, H, xg, ssp, ld,
                       err);
  return hipGetLastError();
}

hipError_t launch_norm_mx8(const float *h, float *h_out, const float *part, int nsplit, const float *gain, int M,
                           int H, float eps, uint8_t *x8, uint8_t *xs, float *dump, hipStream_t st) {
  if (H > 4096 || H % 32 || h == h_out) return hipErrorInvalidValue;
  launch_k(norm_kernel<kOutMX8>, dim3(M), dim3(256), 0, st, h, h_out, part, nsplit, gain, M, H, eps,
                     (void *)x8, xs, dump);
  return hipGetLastError();
}

// MXFP8 encoding of fp32 rows: thread i of the grid takes 4 consecutive
// values, 8 threads one 32-value block (n = M*K/4 threads, K % 32 == 0).
__global__ __launch_bounds__(256) void quant_mx8_kernel(const float *__restrict__ x, size_t n, uint8_t *codes,
                                                        uint8_t *scales) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const f32x4_t v = i < n ? *reinterpret_cast<const f32x4_t *>(x + 4 * i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t e8;
  const uint32_t q = mx8_quant4(v, e8);  // all lanes take part in the block shuffles
  if (i < n) {
    *reinterpret_cast<uint32_t *>(codes + 4 * i) = q;
    if ((i & 7) == 0) scales[i / 8] = (uint8_t)e8;
  }
}

hipError_t launch_quant_mx8(const float *x, int M, int K, uint8_t *codes, uint8_t *scales, hipStream_t st) {
  if (K % 32) return hipErrorInvalidValue;
  const size_t n = (size_t)M * K / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_mx8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n, codes, scales);
  return hipGetLastError();
}

hipError_t launch_accept(const ArgmaxPart *part, int nparts, int M, const int32_t *tokens, int batch,
                         int32_t *accept_len, int32_t *bonus, int32_t *argmax, int32_t *last_tau,
                         hipStream_t st) {
  launch_k(accept_kernel, dim3(batch), dim3(1024), 0, st, part, nparts, M, tokens, accept_len,
                     bonus, argmax, last_tau);
  return hipGetLastError();
}

hipError_t launch_commit(int batch, const int32_t *n_commit, const int32_t *last_tau, int32_t *kv_len,
                         int max_ctx, int32_t *err, hipStream_t st) {
  launch_k(commit_kernel, dim3((batch + 255) / 256), dim3(256), 0, st, batch, n_commit, last_tau,
                     kv_len, max_ctx, err);
  return hipGetLastError();
}

hipError_t launch_prefill_gather(const int32_t *prompt, int T, const int32_t *lens, int chunk, int batch,
                                 int32_t *tokens, int32_t *err, hipStream_t st) {
  hipLaunchKernelGGL(prefill_gather_kernel, dim3(batch), dim3(16), 0, st, prompt, T, lens, chunk, tokens, err);
  return hipGetLastError();
}

hipError_t launch_prefill_finish(const int32_t *lens, int T, int chunk, int batch, const int32_t *argmax,
                                 int32_t *n_commit, int32_t *pending, int32_t *last_tau, int32_t *sel,
                                 hipStream_t st) {
  hipLaunchKernelGGL(prefill_finish_kernel, dim3(batch), dim3(1), 0, st, lens, T, chunk, argmax, n_commit, pending,
                     last_tau, sel);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t st) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}
