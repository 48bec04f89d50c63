// Weight-streaming small-M linear layers with fused epilogues (gfx950).
//
// y[m][n] = sum_k x[m][k] * w(n, k) with x BF16 [M][K] (M = batch*16 block
// rows) and the weight rows decoded in registers from FP8-e4m3 (per-row fp32
// scale applied in the epilogue), MXFP4 (e2m1 codes times an e8m0 power of two
// per 32 inputs, applied while decoding) or BF16.  Decoding is exact, so the
// products are the BF16 MFMA of the BF16 activations with the exact weight
// values, accumulated in fp32.  "The Inference Stack Behind OCRia"
// (quantization section) is the reason the weights move as FP8/FP4: decode is
// memory bound, so fewer bytes per weight is the lever.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16): the weight tile is the A operand
// (16 output rows), the activation tile the B operand (16 block rows), so a
// lane (r = lane%16, g = lane/16) ends with outputs n = 4g..4g+3 of token r.
// Each lane reads 16 consecutive k of one weight row per 64-wide k step
// (one 16-byte load for FP8) and the matching 16 activations; the first and
// second half of those feed two MFMAs, which keeps the A/B k pairing equal.
//
// A workgroup is 4 waves; wave w owns one "unit" of NT 16-row weight tiles
// and loops over all of K, for MT 16-row activation tiles.  Epilogues decide
// which weight rows a unit reads and what happens to the fp32 tile.
#include "common.h"
#include "kernels.h"

template <int FMT> struct WRaw;
template <> struct WRaw<SPEC_WFMT_FP8_E4M3_ROW> { u32x4_t c; };
template <> struct WRaw<SPEC_WFMT_BF16> { u32x4_t lo, hi; };
template <> struct WRaw<SPEC_WFMT_MXFP4> { u32x2_t c; uint32_t e; };

template <int FMT>
__device__ __forceinline__ void load_w(WRaw<FMT> &r, const uint8_t *__restrict__ w,
                                       const uint8_t *__restrict__ s, int row, int K, int k) {
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
    r.c = *reinterpret_cast<const u32x4_t *>(w + (size_t)row * K + k);
  } else if constexpr (FMT == SPEC_WFMT_BF16) {
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint16_t *>(w) +
                                                         (size_t)row * K + k);
    r.lo = p[0];
    r.hi = p[1];
  } else {
    r.c = *reinterpret_cast<const u32x2_t *>(w + (size_t)row * (K / 2) + k / 2);
    r.e = s[(size_t)row * (K / 32) + k / 32];
  }
}

template <int FMT>
__device__ __forceinline__ void cvt_w(const WRaw<FMT> &r, u32x4_t &op0, u32x4_t &op1) {
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
    u32x2_t a = fp8x4_to_bf16x4(r.c.x), b = fp8x4_to_bf16x4(r.c.y);
    u32x2_t c = fp8x4_to_bf16x4(r.c.z), d = fp8x4_to_bf16x4(r.c.w);
    op0 = u32x4_t{a.x, a.y, b.x, b.y};
    op1 = u32x4_t{c.x, c.y, d.x, d.y};
  } else if constexpr (FMT == SPEC_WFMT_BF16) {
    op0 = r.lo;
    op1 = r.hi;
  } else {
    const float sc = __uint_as_float(r.e << 23);  // 2^(e-127); e = 0 only on all-zero blocks
    op0 = fp4x8_to_bf16x8(r.c.x, sc);
    op1 = fp4x8_to_bf16x8(r.c.y, sc);
  }
}

template <int FMT, int NT, int MT, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                   const uint8_t *__restrict__ w,
                                                   const uint8_t *__restrict__ s, Epi epi) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= epi.units) return;  // wave-uniform
  const int m0 = blockIdx.y * (16 * MT);

  int wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wrow[t] = epi.row(unit, t) + r;
  const uint16_t *xp[MT];
  bool mok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + 16 * mt + r;
    mok[mt] = m < M;
    xp[mt] = x + (size_t)(mok[mt] ? m : 0) * K + 16 * g;
  }

  f32x4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  WRaw<FMT> wc[NT];
  u32x4_t ac[MT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_w<FMT>(wc[t], w, s, wrow[t], K, 16 * g);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ac[mt][0] = reinterpret_cast<const u32x4_t *>(xp[mt])[0];
    ac[mt][1] = reinterpret_cast<const u32x4_t *>(xp[mt])[1];
  }

  for (int k0 = 0; k0 < K; k0 += 64) {
    const bool more = k0 + 64 < K;
    WRaw<FMT> wn[NT];
    u32x4_t an[MT][2];
    if (more) {
#pragma unroll
      for (int t = 0; t < NT; ++t) load_w<FMT>(wn[t], w, s, wrow[t], K, k0 + 64 + 16 * g);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        an[mt][0] = reinterpret_cast<const u32x4_t *>(xp[mt] + k0 + 64)[0];
        an[mt][1] = reinterpret_cast<const u32x4_t *>(xp[mt] + k0 + 64)[1];
      }
    }
    u32x4_t w0[NT], w1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) cvt_w<FMT>(wc[t], w0[t], w1[t]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4_t z = u32x4_t{0, 0, 0, 0};
      const u32x4_t a0 = mok[mt] ? ac[mt][0] : z, a1 = mok[mt] ? ac[mt][1] : z;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t][mt] = mfma16x16x32(w0[t], a0, acc[t][mt]);
        acc[t][mt] = mfma16x16x32(w1[t], a1, acc[t][mt]);
      }
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < NT; ++t) wc[t] = wn[t];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ac[mt][0] = an[mt][0];
        ac[mt][1] = an[mt][1];
      }
    }
  }
  epi.template store<NT, MT>(unit, m0, M, r, g, acc);
}

__device__ __forceinline__ void store_bf16x4(uint16_t *p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t *>(p) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

__device__ __forceinline__ f32x4_t row_scale4(const float *s, int n) {
  if (!s) return f32x4_t{1.f, 1.f, 1.f, 1.f};
  return *reinterpret_cast<const f32x4_t *>(s + n);
}

// ---------------------------------------------------------------- epilogues

template <int NTc>
struct EpiF32 {  // y = acc * scale, fp32 out
  int units, N;
  float *y;
  const float *scale;
  __device__ int row(int unit, int t) const { return unit * 16 * NTc + 16 * t; }
  template <int NT, int MT>
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT]) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + r, n = row(unit, t) + 4 * g;
        if (m < M) *reinterpret_cast<f32x4_t *>(y + (size_t)m * N + n) = acc[t][mt] * row_scale4(scale, n);
      }
  }
};

template <int NTc>
struct EpiResidual {  // h += acc * scale
  int units, N;
  float *h;
  const float *scale;
  __device__ int row(int unit, int t) const { return unit * 16 * NTc + 16 * t; }
  template <int NT, int MT>
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT]) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + r, n = row(unit, t) + 4 * g;
        if (m < M) {
          f32x4_t *p = reinterpret_cast<f32x4_t *>(h + (size_t)m * N + n);
          *p = *p + acc[t][mt] * row_scale4(scale, n);
        }
      }
  }
};

// One unit = one head of D = 16*NT rows: q heads, then k heads, then v heads.
// Rotate-half RoPE pairs d and d + D/2, which are tiles t and t + NT/2 in the
// same lane and register slot.
template <int NTc>
struct EpiQkv {
  int units;
  const float *scale;
  QkvOut o;
  __device__ int row(int unit, int t) const { return unit * 16 * NTc + 16 * t; }
  template <int NT, int MT>
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT]) const {
    constexpr int D = 16 * NT, HALF = D / 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + r;
      if (m >= M) continue;
      const int b = m >> 4, j = m & 15;
      const int n0 = o.kv_len[b];
      const int pos = n0 + j;
      const bool fits = n0 >= 0 && n0 + 16 <= o.max_ctx;
      if (unit < o.Hq + o.Hkv) {
        if (!fits) continue;  // flagged by the embed step
        uint16_t *dst;
        if (unit < o.Hq)
          dst = o.q_out + (size_t)m * (o.Hq * D) + unit * D;
        else
          dst = o.k_cache + (((size_t)b * o.Hkv + (unit - o.Hq)) * o.max_ctx + pos) * D;
#pragma unroll
        for (int t = 0; t < NT / 2; ++t) {
          const int d = 16 * t + 4 * g;
          const f32x4_t y1 = acc[t][mt] * row_scale4(scale, row(unit, t) + 4 * g);
          const f32x4_t y2 = acc[t + NT / 2][mt] * row_scale4(scale, row(unit, t + NT / 2) + 4 * g);
          float o1[4], o2[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float2 cs = o.rope[(size_t)pos * HALF + d + i];
            o1[i] = y1[i] * cs.x - y2[i] * cs.y;
            o2[i] = y2[i] * cs.x + y1[i] * cs.y;
          }
          store_bf16x4(dst + d, o1[0], o1[1], o1[2], o1[3]);
          store_bf16x4(dst + d + HALF, o2[0], o2[1], o2[2], o2[3]);
        }
      } else {
        if (!fits) continue;
        uint16_t *dst = o.v_cache + (((size_t)b * o.Hkv + (unit - o.Hq - o.Hkv)) * o.max_ctx + pos) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const f32x4_t y = acc[t][mt] * row_scale4(scale, row(unit, t) + 4 * g);
          store_bf16x4(dst + 16 * t + 4 * g, y[0], y[1], y[2], y[3]);
        }
      }
    }
  }
};

// Tiles [0, NT/2) read gate rows, tiles [NT/2, NT) the matching up rows.
template <int NTc>
struct EpiSwiglu {
  int units, I;
  const float *scale;  // per-row FP8 scales [2I], NULL when decoded with the scale
  uint16_t *a;
  __device__ int row(int unit, int t) const {
    return t < NTc / 2 ? unit * 8 * NTc + 16 * t : I + unit * 8 * NTc + 16 * (t - NTc / 2);
  }
  template <int NT, int MT>
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT]) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + r;
      if (m >= M) continue;
#pragma unroll
      for (int t = 0; t < NT / 2; ++t) {
        const int n = unit * 8 * NT + 16 * t + 4 * g;
        const f32x4_t gv = acc[t][mt] * row_scale4(scale, n);
        const f32x4_t uv = acc[t + NT / 2][mt] * row_scale4(scale ? scale + I : nullptr, n);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = gv[i] / (1.f + __expf(-gv[i])) * uv[i];
        store_bf16x4(a + (size_t)m * I + n, v[0], v[1], v[2], v[3]);
      }
    }
  }
};

// lm_head tile -> per (unit, row) argmax partial, lowest index on ties.
template <int NTc>
struct EpiArgmax {
  int units, V;
  ArgmaxPart *part;  // [units][M]
  float *logits;     // optional [M][V]
  __device__ int row(int unit, int t) const { return unit * 16 * NTc + 16 * t; }
  template <int NT, int MT>
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT]) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + r;
      float bv = -INFINITY;
      int32_t bi = 0x7fffffff;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = row(unit, t) + 4 * g + i;
          if (better(acc[t][mt][i], n, bv, bi)) {
            bv = acc[t][mt][i];
            bi = n;
          }
        }
#pragma unroll
      for (int off = 16; off < 64; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int32_t oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (m < M) {
        if (g == 0) part[(size_t)unit * M + m] = ArgmaxPart{bv, bi};
        if (logits) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4_t *>(logits + (size_t)m * V + row(unit, t) + 4 * g) = acc[t][mt];
        }
      }
    }
  }
};

// ---------------------------------------------------------------- launchers

template <int FMT, int NT, int MT, class Epi>
static hipError_t go(const uint16_t *x, int M, int K, const LinearW &w, const Epi &epi, hipStream_t st) {
  dim3 grid((epi.units + 3) / 4, (M + 16 * MT - 1) / (16 * MT));
  hipLaunchKernelGGL((gemm_kernel<FMT, NT, MT, Epi>), grid, dim3(256), 0, st, x, M, K,
                     reinterpret_cast<const uint8_t *>(w.w), reinterpret_cast<const uint8_t *>(w.s), epi);
  return hipGetLastError();
}

template <int FMT, int NT, class Epi>
static hipError_t go_m(const uint16_t *x, int M, int K, const LinearW &w, const Epi &epi, hipStream_t st) {
  if (M <= 16) return go<FMT, NT, 1>(x, M, K, w, epi, st);
  if (M <= 32 || NT > 4) return go<FMT, NT, 2>(x, M, K, w, epi, st);
  return go<FMT, NT, 4>(x, M, K, w, epi, st);
}

template <int NT, class Epi>
static hipError_t go_fmt(const uint16_t *x, int M, int K, const LinearW &w, const Epi &epi, hipStream_t st) {
  switch (w.wfmt) {
    case SPEC_WFMT_FP8_E4M3_ROW: return go_m<SPEC_WFMT_FP8_E4M3_ROW, NT>(x, M, K, w, epi, st);
    case SPEC_WFMT_MXFP4: return go_m<SPEC_WFMT_MXFP4, NT>(x, M, K, w, epi, st);
    case SPEC_WFMT_BF16: return go_m<SPEC_WFMT_BF16, NT>(x, M, K, w, epi, st);
  }
  return hipErrorInvalidValue;
}

static const float *fp8_scale(const LinearW &w) {
  return w.wfmt == SPEC_WFMT_FP8_E4M3_ROW ? reinterpret_cast<const float *>(w.s) : nullptr;
}

hipError_t launch_linear_f32(const uint16_t *x, int M, int N, int K, LinearW w, float *y, hipStream_t st) {
  EpiF32<1> e{N / 16, N, y, fp8_scale(w)};
  return go_fmt<1>(x, M, K, w, e, st);
}

hipError_t launch_residual(const uint16_t *x, int M, int N, int K, LinearW w, float *h, hipStream_t st) {
  EpiResidual<1> e{N / 16, N, h, fp8_scale(w)};
  return go_fmt<1>(x, M, K, w, e, st);
}

hipError_t launch_swiglu(const uint16_t *x, int M, int H, int I, LinearW w, uint16_t *a, hipStream_t st) {
  EpiSwiglu<4> e{I / 32, I, fp8_scale(w), a};
  return go_fmt<4>(x, M, H, w, e, st);
}

hipError_t launch_qkv(const uint16_t *x, int M, int H, int D, LinearW w, QkvOut o, hipStream_t st) {
  if (w.wfmt != SPEC_WFMT_FP8_E4M3_ROW) return hipErrorInvalidValue;
  const float *s = reinterpret_cast<const float *>(w.s);
  if (D == 64) {
    EpiQkv<4> e{o.Hq + 2 * o.Hkv, s, o};
    return go_m<SPEC_WFMT_FP8_E4M3_ROW, 4>(x, M, H, w, e, st);
  }
  if (D == 128) {
    EpiQkv<8> e{o.Hq + 2 * o.Hkv, s, o};
    return go_m<SPEC_WFMT_FP8_E4M3_ROW, 8>(x, M, H, w, e, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_lm_argmax(const uint16_t *x, int M, int V, int H, const uint16_t *table,
                            ArgmaxPart *part, float *logits_dump, hipStream_t st) {
  EpiArgmax<4> e{V / 64, V, part, logits_dump};
  LinearW w{table, nullptr, SPEC_WFMT_BF16};
  return go_m<SPEC_WFMT_BF16, 4>(x, M, H, w, e, st);
}
