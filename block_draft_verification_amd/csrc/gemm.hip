// Weight-streaming linear layers for the verify pass, with fused epilogues
// (gfx950, wave64).
//
// y[m][n] = sum_k x[m][k] * w(n, k), x [M][K] (M = batch*16 block rows).
// Weight rows are decoded in registers, exactly, from FP8-e4m3 (per-row fp32
// scale applied to the fp32 accumulator), MXFP4 (e2m1 times the e8m0 power of
// two of each 32 inputs) or BF16.  "The Inference Stack Behind OCRia"
// (quantization section) is why weights move as FP8/FP4: a decode step is
// bound by the bytes it moves.  Activations are FP16 for the decoder layers
// (FP8 and FP4 decode exactly to FP16, and FP16 keeps the rounding of the
// normed activations small enough for a 24-32 layer stack) and BF16 for the
// lm_head (whose BF16 table is then used as is).  fp32 accumulation.
//
// MFMA mapping (v_mfma_f32_16x16x32_{f16,bf16}): the weight tile is the A
// operand (16 output rows), the activation tile the B operand (16 block
// rows); lane (r, g) = (lane%16, lane/16) ends with outputs n = 4g..4g+3 of
// row r, so every epilogue (scale, RoPE pair, gate/up pair, residual,
// argmax) runs on registers.  Per 64-wide k step a lane reads 16 consecutive
// k of one weight row (one 16-byte load for FP8) and the matching 16
// activations; halves feed two MFMAs so A and B always pair the same k.
//
// Work split: a workgroup = 4 waves side by side along N (wave = one "unit"
// of NT 16-row weight tiles) sharing one activation tile of 16*MT rows,
// which is staged through LDS (double buffered, one barrier per k step)
// while each wave streams its own weight rows straight into registers one k
// step ahead.  Workgroups that share weight rows (all M blocks of one N
// block) are placed on one XCD so its L2 serves the re-reads.  Shapes with
// too few output tiles to fill 256 CUs split K over gridDim.z: each split
// writes fp32 partials and the last workgroup of a tile (integer atomic
// counter) adds them in split order and runs the epilogue, so results do not
// depend on timing.
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

// 16 weights -> two 8-element MFMA operands in the activation type
template <bool F16, int FMT>
__device__ __forceinline__ void cvt_w(const WRaw<FMT> &r, u32x4_t &op0, u32x4_t &op1) {
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
    u32x2_t a, b, c, d;
    if constexpr (F16) {
      a = fp8x4_to_f16x4(r.c.x), b = fp8x4_to_f16x4(r.c.y), c = fp8x4_to_f16x4(r.c.z), d = fp8x4_to_f16x4(r.c.w);
    } else {
      a = fp8x4_to_bf16x4(r.c.x), b = fp8x4_to_bf16x4(r.c.y), c = fp8x4_to_bf16x4(r.c.z), d = fp8x4_to_bf16x4(r.c.w);
    }
    op0 = u32x4_t{a.x, a.y, b.x, b.y};
    op1 = u32x4_t{c.x, c.y, d.x, d.y};
  } else if constexpr (FMT == SPEC_WFMT_BF16) {
    static_assert(!F16, "BF16 weights pair with BF16 activations");
    op0 = r.lo;
    op1 = r.hi;
  } else {
    const float sc = __uint_as_float(r.e << 23);  // 2^(e-127); e = 0 only on all-zero blocks
    if constexpr (F16) {
      op0 = fp4x8_to_f16x8(r.c.x, sc);
      op1 = fp4x8_to_f16x8(r.c.y, sc);
    } else {
      op0 = fp4x8_to_bf16x8(r.c.x, sc);
      op1 = fp4x8_to_bf16x8(r.c.y, sc);
    }
  }
}

template <bool F16>
__device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (F16) return mfma16x16x32_f16(a, b, c);
  else return mfma16x16x32(a, b, c);
}

struct GemmArgs {
  const uint16_t *x;  // activations [M][K] (fp16 or bf16 bits)
  int M, K;
  const uint8_t *w, *s;
  int nb, mb;         // N blocks (4 units each), M blocks
  int spl;            // k steps (of 64) per split; gridDim.z splits
  float *part;        // split partials
  int32_t *counters;  // per output tile, zero between launches
};

// Linear workgroup id -> (N block, M block): the M blocks of one N block are
// consecutive workgroups of one XCD (XCD = id % 8).
__device__ __forceinline__ bool tile_of(int L, int nb, int mb, int &n, int &m) {
  const int xcd = L & 7, k = L >> 3;
  n = xcd + 8 * (k / mb);
  m = k % mb;
  return n < nb;
}

template <bool F16, int FMT, int NT, int MT, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs ga, Epi epi) {
  constexpr int ROWS = 16 * MT;
  constexpr int AP = 64 + 8;              // LDS row pitch in 16-bit elements (144 B)
  constexpr int ACH = ROWS * 8;           // 16-byte chunks per activation tile
  constexpr int APT = (ACH + 255) / 256;  // chunks per thread
  __shared__ __align__(16) uint16_t As[2][ROWS * AP];
  __shared__ int s_last;

  int nblk, mblk;
  if (!tile_of(blockIdx.x, ga.nb, ga.mb, nblk, mblk)) return;  // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, g = lane >> 4;
  const int unit = nblk * 4 + wave;
  const bool active = unit < epi.units;  // wave-uniform
  const int m0 = mblk * ROWS;
  const int M = ga.M, K = ga.K, ksteps = K / 64;
  const int z = blockIdx.z, nsplit = gridDim.z;
  const int ks0 = z * ga.spl, ks1 = min(ks0 + ga.spl, ksteps);

  u32x4_t areg[APT];
  auto load_a = [&](int ks) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8, m = m0 + row;
      if (c < ACH)
        areg[i] = m < M ? *reinterpret_cast<const u32x4_t *>(ga.x + (size_t)m * K + ks * 64 + col)
                        : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      if (c < ACH) *reinterpret_cast<u32x4_t *>(&As[buf][row * AP + col]) = areg[i];
    }
  };

  int wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wrow[t] = epi.row(active ? unit : 0, t) + r;
  f32x4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  WRaw<FMT> wc[NT];
  if (active) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_w<FMT>(wc[t], ga.w, ga.s, wrow[t], K, ks0 * 64 + 16 * g);
  }
  load_a(ks0);
  store_a(0);
  __syncthreads();

  for (int ks = ks0; ks < ks1; ++ks) {
    const int buf = (ks - ks0) & 1;
    const bool more = ks + 1 < ks1;
    WRaw<FMT> wn[NT];
    if (more) {
      load_a(ks + 1);
      if (active) {
#pragma unroll
        for (int t = 0; t < NT; ++t) load_w<FMT>(wn[t], ga.w, ga.s, wrow[t], K, (ks + 1) * 64 + 16 * g);
      }
    }
    if (active) {
      u32x4_t w0[NT], w1[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) cvt_w<F16, FMT>(wc[t], w0[t], w1[t]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t *ap = &As[buf][(16 * mt + r) * AP + 16 * g];
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(ap);
        const u32x4_t a1 = *reinterpret_cast<const u32x4_t *>(ap + 8);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[t][mt] = mma<F16>(w0[t], a0, acc[t][mt]);
          acc[t][mt] = mma<F16>(w1[t], a1, acc[t][mt]);
        }
      }
    }
    if (more) {
      store_a(buf ^ 1);
#pragma unroll
      for (int t = 0; t < NT; ++t) wc[t] = wn[t];
    }
    __syncthreads();
  }

  if (nsplit == 1) {
    if (active) epi.template store<NT, MT>(unit, m0, M, r, g, acc);
    return;
  }
  // split K: partials in the accumulator layout, then the last arriver reduces
  constexpr int PER_WAVE = NT * MT * 256;
  const int tile = nblk * ga.mb + mblk, ntiles = ga.nb * ga.mb;
  if (active) {
    float *pw = ga.part + ((size_t)(z * ntiles + tile) * 4 + wave) * PER_WAVE;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4_t *>(pw + (t * MT + mt) * 256 + lane * 4) = acc[t][mt];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&ga.counters[tile], 1) == nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (active) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int zz = 0; zz < nsplit; ++zz) {
      const float *pz = ga.part + ((size_t)(zz * ntiles + tile) * 4 + wave) * PER_WAVE;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] += __builtin_nontemporal_load(
              reinterpret_cast<const f32x4_t *>(pz + (t * MT + mt) * 256 + lane * 4));
    }
    epi.template store<NT, MT>(unit, m0, M, r, g, acc);
  }
  if (tid == 0) ga.counters[tile] = 0;
}

__device__ __forceinline__ void store_f16x4(uint16_t *p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t *>(p) = u32x2_t{pack_f16x2(a, b), pack_f16x2(c, d)};
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
// same lane and register slot.  q goes out as FP16, k and v into the BF16 cache.
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
      if (n0 < 0 || n0 + 16 > o.max_ctx) continue;  // flagged by the embed step
      if (unit < o.Hq + o.Hkv) {
        const bool isq = unit < o.Hq;
        uint16_t *dst = isq ? o.q_out + (size_t)m * (o.Hq * D) + unit * D
                            : o.k_cache + (((size_t)b * o.Hkv + (unit - o.Hq)) * o.max_ctx + pos) * D;
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
          if (isq) {
            store_f16x4(dst + d, o1[0], o1[1], o1[2], o1[3]);
            store_f16x4(dst + d + HALF, o2[0], o2[1], o2[2], o2[3]);
          } else {
            store_bf16x4(dst + d, o1[0], o1[1], o1[2], o1[3]);
            store_bf16x4(dst + d + HALF, o2[0], o2[1], o2[2], o2[3]);
          }
        }
      } else {
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

// Tiles [0, NT/2) read gate rows, tiles [NT/2, NT) the matching up rows;
// a = SiLU(gate) * up goes out as FP16.
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
        store_f16x4(a + (size_t)m * I + n, v[0], v[1], v[2], v[3]);
      }
    }
  }
};

// lm_head tile -> per (row, unit) argmax partial, lowest index on ties.
template <int NTc>
struct EpiArgmax {
  int units, V;
  ArgmaxPart *part;  // [M][units]
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
        if (g == 0) part[(size_t)m * units + unit] = ArgmaxPart{bv, bi};
        if (logits) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4_t *>(logits + (size_t)m * V + row(unit, t) + 4 * g) = acc[t][mt];
        }
      }
    }
  }
};

// ---------------------------------------------------------------- planning

GemmPlan gemm_plan(int M, int units, int ksteps, int NT, int maxMT) {
  GemmPlan p;
  p.MT = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  if (p.MT > maxMT) p.MT = maxMT;
  p.nb = (units + 3) / 4;
  p.mb = (M + 16 * p.MT - 1) / (16 * p.MT);
  const int tiles = p.nb * p.mb;
  // split K until about 512 workgroups, keeping >= 4 k steps per split
  int s = (512 + tiles - 1) / tiles;
  if (s > ksteps / 4) s = ksteps / 4;
  if (s < 1) s = 1;
  p.spl = (ksteps + s - 1) / s;
  p.nsplit = (ksteps + p.spl - 1) / p.spl;  // every split non-empty
  p.part_floats = p.nsplit > 1 ? (size_t)p.nsplit * tiles * 4 * NT * p.MT * 256 : 0;
  p.grid_x = 8 * ((p.nb + 7) / 8) * p.mb;
  return p;
}

// ---------------------------------------------------------------- launchers

template <bool F16, int FMT, int NT, int MT, class Epi>
static hipError_t go(const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<F16, FMT, NT, MT, Epi>), dim3(p.grid_x, 1, p.nsplit), dim3(256), 0, st, ga,
                     epi);
  return hipGetLastError();
}

template <bool F16, int FMT, int NT, class Epi>
static hipError_t go_m(const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  switch (p.MT) {
    case 1: return go<F16, FMT, NT, 1>(p, ga, epi, st);
    case 2: return go<F16, FMT, NT, 2>(p, ga, epi, st);
    case 4: return go<F16, FMT, NT, 4>(p, ga, epi, st);
    default:
      if constexpr (NT <= 4) return go<F16, FMT, NT, 8>(p, ga, epi, st);
      else return go<F16, FMT, NT, 4>(p, ga, epi, st);
  }
}

template <int NT, class Epi>
static hipError_t run(const uint16_t *x, int M, int K, const LinearW &w, Epi epi, const GemmWork &wk,
                      hipStream_t st) {
  const GemmPlan p = gemm_plan(M, epi.units, K / 64, NT, NT > 4 ? 4 : 8);
  if (p.part_floats > wk.part_floats) return hipErrorInvalidValue;
  GemmArgs ga{x, M, K, reinterpret_cast<const uint8_t *>(w.w), reinterpret_cast<const uint8_t *>(w.s),
              p.nb, p.mb, p.spl, wk.part, wk.counters};
  switch (w.wfmt) {
    case SPEC_WFMT_FP8_E4M3_ROW: return go_m<true, SPEC_WFMT_FP8_E4M3_ROW, NT>(p, ga, epi, st);
    case SPEC_WFMT_MXFP4: return go_m<true, SPEC_WFMT_MXFP4, NT>(p, ga, epi, st);
    case SPEC_WFMT_BF16: return go_m<false, SPEC_WFMT_BF16, NT>(p, ga, epi, st);
  }
  return hipErrorInvalidValue;
}

static const float *fp8_scale(const LinearW &w) {
  return w.wfmt == SPEC_WFMT_FP8_E4M3_ROW ? reinterpret_cast<const float *>(w.s) : nullptr;
}

hipError_t launch_linear_f32(const uint16_t *x, int M, int N, int K, LinearW w, float *y, const GemmWork &wk,
                             hipStream_t st) {
  return run<1>(x, M, K, w, EpiF32<1>{N / 16, N, y, fp8_scale(w)}, wk, st);
}

hipError_t launch_residual(const uint16_t *x, int M, int N, int K, LinearW w, float *h, const GemmWork &wk,
                           hipStream_t st) {
  if (M <= 32) return run<1>(x, M, K, w, EpiResidual<1>{N / 16, N, h, fp8_scale(w)}, wk, st);
  return run<4>(x, M, K, w, EpiResidual<4>{N / 64, N, h, fp8_scale(w)}, wk, st);
}

hipError_t launch_swiglu(const uint16_t *x, int M, int H, int I, LinearW w, uint16_t *a, const GemmWork &wk,
                         hipStream_t st) {
  if (M <= 32) return run<2>(x, M, H, w, EpiSwiglu<2>{I / 16, I, fp8_scale(w), a}, wk, st);
  return run<4>(x, M, H, w, EpiSwiglu<4>{I / 32, I, fp8_scale(w), a}, wk, st);
}

hipError_t launch_qkv(const uint16_t *x, int M, int H, int D, LinearW w, QkvOut o, const GemmWork &wk,
                      hipStream_t st) {
  if (w.wfmt != SPEC_WFMT_FP8_E4M3_ROW) return hipErrorInvalidValue;
  const float *s = reinterpret_cast<const float *>(w.s);
  if (D == 64) return run<4>(x, M, H, w, EpiQkv<4>{o.Hq + 2 * o.Hkv, s, o}, wk, st);
  if (D == 128) return run<8>(x, M, H, w, EpiQkv<8>{o.Hq + 2 * o.Hkv, s, o}, wk, st);
  return hipErrorInvalidValue;
}

hipError_t launch_lm_argmax(const uint16_t *x, int M, int V, int H, const uint16_t *table, ArgmaxPart *part,
                            float *logits_dump, const GemmWork &wk, hipStream_t st) {
  return run<4>(x, M, H, LinearW{table, nullptr, SPEC_WFMT_BF16}, EpiArgmax<4>{V / 64, V, part, logits_dump},
                wk, st);
}

// Partial-buffer floats and counters the launches above may need for M rows.
size_t gemm_part_floats(int M, int H, int I, int V, int Hq, int Hkv, int D, size_t *counters) {
  struct S { int units, ksteps, NT; } shapes[] = {
      {M <= 32 ? H / 16 : H / 64, (Hq * D) / 64, M <= 32 ? 1 : 4},  // O-proj
      {M <= 32 ? H / 16 : H / 64, I / 64, M <= 32 ? 1 : 4},          // down
      {M <= 32 ? I / 16 : I / 32, H / 64, M <= 32 ? 2 : 4},          // gate/up
      {Hq + 2 * Hkv, H / 64, D / 16},                                // QKV
      {V / 64, H / 64, 4},                                            // lm_head
  };
  size_t mx = 0, cnt = 0;
  for (const S &s : shapes) {
    const GemmPlan p = gemm_plan(M, s.units, s.ksteps, s.NT, s.NT > 4 ? 4 : 8);
    if (p.part_floats > mx) mx = p.part_floats;
    if ((size_t)p.nb * p.mb > cnt) cnt = (size_t)p.nb * p.mb;
  }
  *counters = cnt;
  return mx;
}
