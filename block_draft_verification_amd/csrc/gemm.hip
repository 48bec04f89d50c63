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

// An empty asm that reads the registers: placed after the final wait, it
// keeps the last (discarded) prefetch's destination registers allocated until
// the load has landed, so the compiler cannot reuse them while it is in flight.
__device__ __forceinline__ void hold(const WRaw<SPEC_WFMT_FP8_E4M3_ROW> &r) { asm volatile("" ::"v"(r.c)); }
__device__ __forceinline__ void hold(const WRaw<SPEC_WFMT_BF16> &r) { asm volatile("" ::"v"(r.lo), "v"(r.hi)); }
__device__ __forceinline__ void hold(const WRaw<SPEC_WFMT_MXFP4> &r) { asm volatile("" ::"v"(r.c), "v"(r.e)); }

// Weight loads are issued as plain vector loads the compiler does not track:
// its wait analysis cannot count the LDS-DMA activation loads issued after
// them and would otherwise wait for every outstanding load before each use.
// The kernel waits for them explicitly (vmcnt) before touching the registers.
__device__ __forceinline__ u32x4_t vload16(const void *p) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ u32x2_t vload8(const void *p) {
  u32x2_t v;
  asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t vload1(const void *p) {
  uint32_t v;
  asm volatile("global_load_ubyte %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

template <int FMT>
__device__ __forceinline__ void load_w(WRaw<FMT> &r, const uint8_t *__restrict__ w,
                                       const uint8_t *__restrict__ s, int row, int K, int k) {
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
    r.c = vload16(w + (size_t)row * K + k);
  } else if constexpr (FMT == SPEC_WFMT_BF16) {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(w) + (size_t)row * K + k;
    r.lo = vload16(p);
    r.hi = vload16(p + 8);
  } else {
    r.c = vload8(w + (size_t)row * (K / 2) + k / 2);
    r.e = vload1(s + (size_t)row * (K / 32) + k / 32);
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
};

// Linear workgroup id -> (N block, M block): the M blocks of one N block are
// consecutive workgroups of one XCD (XCD = id % 8).
__device__ __forceinline__ bool tile_of(int L, int nb, int mb, int &n, int &m) {
  const int xcd = L & 7, k = L >> 3;
  n = xcd + 8 * (k / mb);
  m = k % mb;
  return n < nb;
}

// VMEM loads issued by one wave for one k step: activation rows straight to
// LDS (16-byte lanes), then the weight rows of its NT tiles into registers.
template <int FMT> constexpr int w_loads() { return FMT == SPEC_WFMT_FP8_E4M3_ROW ? 1 : 2; }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at "no wait").
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds + 16 * i.  Kept out of the kernel templates (the host pass drops a
// template kernel that names this builtin directly).
__device__ __forceinline__ void lds_load16(const void *g, void *l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

// Waves per SIMD the register budget is sized for: 2 where the accumulators
// of a wave fit half the register file, else 1.
template <int FMT, int NT, int MT> struct GemmOcc {
  static constexpr int value = (NT * MT <= 32 && NT <= 4 && FMT != 3) ? 2 : 1;
};

template <bool F16, int FMT, int NT, int MT, class Epi>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GemmOcc<FMT, NT, MT>::value, 8))) void
gemm_kernel(GemmArgs ga, Epi epi) {
  constexpr int ROWS = 16 * MT;
  constexpr int AJ = MT >= 2 ? MT / 2 : 1;  // 1 KB wave-loads per wave per stage
  constexpr int SE = 4 * AJ * 512;          // 16-bit elements per stage (MT = 1: half is padding)
  constexpr int NS = 3;                     // stages in flight
  // activation tile: 16-byte chunk c of row r stored at chunk slot r*8 + (c ^ (r & 7))
  __shared__ __align__(16) uint16_t As[NS * SE];

  int nblk, mblk;
  if (!tile_of(blockIdx.x, ga.nb, ga.mb, nblk, mblk)) return;  // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = nblk * 4 + wave;
  const bool active = unit < epi.units;  // wave-uniform; inactive waves compute on row 0 and store nothing
  const int m0 = mblk * ROWS;
  const int M = ga.M, K = ga.K, ksteps = K / 64;
  const int ks0 = blockIdx.z * ga.spl, nsteps = min(ks0 + ga.spl, ksteps) - ks0;

  // every wave issues AJ activation wave-loads and NT weight loads per step,
  // so the vmcnt waits below are the same compile-time count for all waves
  const uint16_t *agp[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i) {
    const int P = (wave + 4 * i) * 64 + lane, row = P >> 3, c = (P & 7) ^ (row & 7);
    const int m = (row < ROWS && m0 + row < M) ? m0 + row : 0;  // padding / rows past M read row 0
    agp[i] = ga.x + (size_t)m * K + ks0 * 64 + c * 8;
  }
  int wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wrow[t] = epi.row(active ? unit : 0, t) + r;

  f32x4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage, const WRaw<FMT>(&wr)[NT]) {
    __builtin_amdgcn_sched_barrier(0);  // keep the three unrolled steps from interleaving (register pressure)
    u32x4_t w0[NT], w1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) cvt_w<F16, FMT>(wr[t], w0[t], w1[t]);
    const uint16_t *base = As + stage * SE;
    auto read_a = [&](int mt, u32x4_t &a0, u32x4_t &a1) {
      const int row = 16 * mt + r;
      a0 = *reinterpret_cast<const u32x4_t *>(base + (row * 8 + ((2 * g) ^ (row & 7))) * 8);
      a1 = *reinterpret_cast<const u32x4_t *>(base + (row * 8 + ((2 * g + 1) ^ (row & 7))) * 8);
    };
    // activation fragments of tile mt+1 are read while tile mt's MFMAs run
    u32x4_t a0[2], a1[2];
    read_a(0, a0[0], a1[0]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt + 1 < MT) read_a(mt + 1, a0[(mt + 1) & 1], a1[(mt + 1) & 1]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t][mt] = mma<F16>(w0[t], a0[mt & 1], acc[t][mt]);
        acc[t][mt] = mma<F16>(w1[t], a1[mt & 1], acc[t][mt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Per k step s: activations for step s+2 go straight to LDS stage (s+2)%3,
  // weights for step s+1 into the "next" registers, then step s is computed.
  auto issue_a_to = [&](int step, int stage) {
#pragma unroll
    for (int i = 0; i < AJ; ++i) lds_load16(agp[i] + step * 64, As + stage * SE + (wave + 4 * i) * 512);
  };
  auto issue_a = [&](int step) { issue_a_to(step, step % NS); };
  auto issue_w = [&](WRaw<FMT>(&wr)[NT], int step) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_w<FMT>(wr[t], ga.w, ga.s, wrow[t], K, (ks0 + step) * 64 + 16 * g);
  };
  // VMEM order per step: [W(s+1)] then [A(s+2)].  Loads complete in issue
  // order, so waiting for the weight registers (at the copy below) never waits
  // for the younger activation loads, which stay two steps ahead.
  // Two weight register sets alternate (the loop is unrolled by two) so no
  // register copy of a load destination is ever needed: a copy would be
  // placed before the wait that covers the load.  Tail steps re-load the last
  // step into a stage nobody reads.  Issue order per step: [W(s+1)] [A(s+2)].
  // At the top of step s the outstanding loads are, oldest first, A(s), W(s),
  // A(s+1): waiting until at most AJ remain leaves only A(s+1) in flight.
  WRaw<FMT> wa[NT], wb[NT];
  issue_w(wa, 0);
  issue_a(0);
  issue_a(min(1, nsteps - 1));
  for (int s = 0; s < nsteps; s += 2) {
    WAIT_VMCNT(AJ);
    lds_barrier();  // stage s visible to all waves; stage (s+2)%3 = (s-1)%3 free again
    __builtin_amdgcn_sched_barrier(0);
    issue_w(wb, min(s + 1, nsteps - 1));
    issue_a_to(min(s + 2, nsteps - 1), (s + 2) % NS);
    __builtin_amdgcn_sched_barrier(0);
    compute(s % NS, wa);
    WAIT_VMCNT(AJ);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_w(wa, min(s + 2, nsteps - 1));
    issue_a_to(min(s + 3, nsteps - 1), (s + 3) % NS);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nsteps) compute((s + 1) % NS, wb);
  }
  WAIT_VMCNT(0);  // nothing may still be landing in LDS or registers past this point
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    hold(wa[t]);
    hold(wb[t]);
  }
  if (active) epi.template store<NT, MT>(unit, m0, M, r, g, acc, blockIdx.z);
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
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT], int z) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + r, n = row(unit, t) + 4 * g;
        if (m < M) *reinterpret_cast<f32x4_t *>(y + (size_t)m * N + n) = acc[t][mt] * row_scale4(scale, n);
      }
  }
};

// Split-K partial of a residual projection: P[z][m][n] = acc * scale.  The
// next RMSNorm adds the partials of every split to h in split order.
template <int NTc>
struct EpiPartial {
  int units, N;
  float *part;  // [nsplit][M][N]
  const float *scale;
  __device__ int row(int unit, int t) const { return unit * 16 * NTc + 16 * t; }
  template <int NT, int MT>
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT], int z) const {
    float *pz = part + (size_t)z * M * N;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + r, n = row(unit, t) + 4 * g;
        if (m < M) *reinterpret_cast<f32x4_t *>(pz + (size_t)m * N + n) = acc[t][mt] * row_scale4(scale, n);
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
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT], int z) const {
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
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT], int z) const {
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
  __device__ void store(int unit, int m0, int M, int r, int g, const f32x4_t (&acc)[NT][MT], int z) const {
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

GemmPlan gemm_plan(int M, int units, int ksteps, int MT, bool allow_split) {
  GemmPlan p;
  p.MT = MT;
  p.nb = (units + 3) / 4;
  p.mb = (M + 16 * MT - 1) / (16 * MT);
  const int tiles = p.nb * p.mb;
  // split K (residual projections only) until about 256 workgroups, >= 4 k steps per split
  int s = allow_split ? (256 + tiles - 1) / tiles : 1;
  if (s > ksteps / 4) s = ksteps / 4;
  if (s < 1) s = 1;
  p.spl = (ksteps + s - 1) / s;
  p.nsplit = (ksteps + p.spl - 1) / p.spl;  // every split non-empty
  p.grid_x = 8 * ((p.nb + 7) / 8) * p.mb;
  return p;
}

// activation rows per workgroup: enough workgroups first, then wide tiles
static int pick_mt(int M, int units, int maxMT) {
  int mt = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  if (mt > maxMT) mt = maxMT;
  while (mt > 2 && ((units + 3) / 4) * ((M + 16 * mt - 1) / (16 * mt)) < 128) mt /= 2;
  return mt;
}

int residual_nsplit(int M, int N, int K) {
  const int units = M <= 32 ? N / 16 : N / 64;
  return gemm_plan(M, units, K / 64, pick_mt(M, units, 8), true).nsplit;
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

// FMTS: bit (1 << format) set for each weight format a call site may pass;
// only those kernels are instantiated.
constexpr unsigned kFp8 = 1u << SPEC_WFMT_FP8_E4M3_ROW, kMx4 = 1u << SPEC_WFMT_MXFP4, kBf16 = 1u << SPEC_WFMT_BF16;

template <int NT, unsigned FMTS, class Epi>
static hipError_t run(const uint16_t *x, int M, int K, const LinearW &w, Epi epi, bool allow_split,
                      hipStream_t st) {
  const GemmPlan p = gemm_plan(M, epi.units, K / 64, pick_mt(M, epi.units, NT > 4 ? 4 : 8), allow_split);
  GemmArgs ga{x, M, K, reinterpret_cast<const uint8_t *>(w.w), reinterpret_cast<const uint8_t *>(w.s),
              p.nb, p.mb, p.spl};
  if constexpr ((FMTS & kFp8) != 0)
    if (w.wfmt == SPEC_WFMT_FP8_E4M3_ROW) return go_m<true, SPEC_WFMT_FP8_E4M3_ROW, NT>(p, ga, epi, st);
  if constexpr ((FMTS & kMx4) != 0)
    if (w.wfmt == SPEC_WFMT_MXFP4) return go_m<true, SPEC_WFMT_MXFP4, NT>(p, ga, epi, st);
  if constexpr ((FMTS & kBf16) != 0)
    if (w.wfmt == SPEC_WFMT_BF16) return go_m<false, SPEC_WFMT_BF16, NT>(p, ga, epi, st);
  return hipErrorInvalidValue;
}

static const float *fp8_scale(const LinearW &w) {
  return w.wfmt == SPEC_WFMT_FP8_E4M3_ROW ? reinterpret_cast<const float *>(w.s) : nullptr;
}

hipError_t launch_linear_f32(const uint16_t *x, int M, int N, int K, LinearW w, float *y, hipStream_t st) {
  return run<1, kFp8 | kMx4 | kBf16>(x, M, K, w, EpiF32<1>{N / 16, N, y, fp8_scale(w)}, false, st);
}

hipError_t launch_residual_partial(const uint16_t *x, int M, int N, int K, LinearW w, float *part, hipStream_t st) {
  if (M <= 32) return run<1, kFp8 | kMx4>(x, M, K, w, EpiPartial<1>{N / 16, N, part, fp8_scale(w)}, true, st);
  return run<4, kFp8 | kMx4>(x, M, K, w, EpiPartial<4>{N / 64, N, part, fp8_scale(w)}, true, st);
}

hipError_t launch_swiglu(const uint16_t *x, int M, int H, int I, LinearW w, uint16_t *a, hipStream_t st) {
  if (M <= 32) return run<2, kFp8 | kMx4>(x, M, H, w, EpiSwiglu<2>{I / 16, I, fp8_scale(w), a}, false, st);
  return run<4, kFp8 | kMx4>(x, M, H, w, EpiSwiglu<4>{I / 32, I, fp8_scale(w), a}, false, st);
}

hipError_t launch_qkv(const uint16_t *x, int M, int H, int D, LinearW w, QkvOut o, hipStream_t st) {
  if (w.wfmt != SPEC_WFMT_FP8_E4M3_ROW) return hipErrorInvalidValue;
  const float *s = reinterpret_cast<const float *>(w.s);
  if (D == 64) return run<4, kFp8>(x, M, H, w, EpiQkv<4>{o.Hq + 2 * o.Hkv, s, o}, false, st);
  if (D == 128) return run<8, kFp8>(x, M, H, w, EpiQkv<8>{o.Hq + 2 * o.Hkv, s, o}, false, st);
  return hipErrorInvalidValue;
}

hipError_t launch_lm_argmax(const uint16_t *x, int M, int V, int H, const uint16_t *table, ArgmaxPart *part,
                            float *logits_dump, hipStream_t st) {
  return run<4, kBf16>(x, M, H, LinearW{table, nullptr, SPEC_WFMT_BF16}, EpiArgmax<4>{V / 64, V, part, logits_dump},
                false, st);
}
