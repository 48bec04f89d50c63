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
// MFMA mapping (v_mfma_f32_32x32x16_{f16,bf16}, which on gfx950 issues at
// twice the rate of the 16x16x32 shape): the weight tile is the A operand (32
// output rows), the activation tile the B operand (32 block rows).  Per
// 64-wide k step lane (c, h) = (lane%32, lane/32) holds 32 k of one weight
// row: for FP8, k 16h..16h+15 and 32+16h..+15 (two 16-byte loads); for BF16
// and MXFP4 (whose scale block is exactly those k), 32h..32h+31.  It uses its
// 8-element slice i as the k operand of the step's i-th MFMA, and the
// activation side reads the same k slices (act_chunk), so A and B always pair
// the same k and the sum over k is complete.  The weights are tile-major
// (kernels.h): each wave-wide weight load is one contiguous kilobyte.
// Lane (c, h) ends with the outputs of block row c for the tile rows
// 8q + 4h + (0..3), q = 0..3, so rows r and r + 16 of a tile sit in the same
// lane: the library's packing puts the two rows an epilogue must combine
// (a RoPE pair, a gate row and its up row) at exactly those positions.
//
// Work split: a workgroup = NWV waves, NG side by side along N (a wave = a
// "unit" of NT 32-row weight tiles) times KS along K, sharing one activation
// tile of 32*MT rows.  A pipeline stage holds KS consecutive 64-wide k steps
// of the activation tile; the waves of k group g compute step g of each
// stage, and the groups' accumulators are added in group order at the end.
// The activation tile goes straight from global memory to LDS (one barrier
// per stage); each wave streams its own weight rows into registers.  Both run
// a few stages ahead of the MFMAs.  Workgroups that share weight rows (all M
// blocks of one N block) are placed on one XCD so its L2 serves the re-reads.
//
// Inputs that are an RMSNorm's product h * g (gain folded in, normalisation
// left out) come with per-row partial sums of squares of h: the kernel adds
// them up, in a fixed order, into r = 1 / sqrt(mean(h^2) + eps) and scales
// its outputs by r.  The residual projections produce exactly that: the new
// residual stream, h * g of the next RMSNorm, and the partial sums.
#include "common.h"
#include "kernels.h"

// Stages loaded ahead of the one computed, by activation tile height (32*MT
// rows): 3 for 32-row tiles, 2 for taller ones (measured over whole passes).
#ifndef GEMM_DEPTH_MT1
#define GEMM_DEPTH_MT1 3
#endif
#ifndef GEMM_DEPTH_MT2
#define GEMM_DEPTH_MT2 2
#endif
#ifndef GEMM_DEPTH_MT4
#define GEMM_DEPTH_MT4 2
#endif
#ifndef GEMM_LM_MAXMT
#define GEMM_LM_MAXMT 4
#endif
#ifndef GEMM_SPLIT_TARGET
#define GEMM_SPLIT_TARGET 256  // split-K workgroup target of the MXFP8 mode's residual projections
#endif
#ifndef GEMM_WG_TARGET
#define GEMM_WG_TARGET 200  // workgroups a decoder GEMM launch aims for (the chip has 256 compute units)
#endif

// Raw weight bytes of one 32-row tile for one lane and one k step.
template <int FMT> struct WRaw;
template <> struct WRaw<SPEC_WFMT_FP8_E4M3_ROW> { u32x4_t c[2]; };  // 32 codes
template <> struct WRaw<SPEC_WFMT_BF16> { u32x4_t c[4]; };          // 32 bf16
template <> struct WRaw<SPEC_WFMT_MXFP4> { u32x4_t c; uint32_t e; };  // 32 nibbles + e8m0

// VMEM instructions per tile and step
template <int FMT> constexpr int w_loads() { return FMT == SPEC_WFMT_BF16 ? 4 : 2; }
// registers of one tile's raw weights for one step
template <int FMT> constexpr int w_regs() { return FMT == SPEC_WFMT_BF16 ? 16 : FMT == SPEC_WFMT_MXFP4 ? 5 : 8; }

// Pipeline depth in stages: `depth` when given, else the tile height's depth
// (two when a stage holds several k steps), capped so that the register ring
// (depth + 1 sets of weights and activation exponents) stays within 112 VGPRs.
template <int FMT, int NT, int MT, bool A8, int KS, int DEPTH>
constexpr int gemm_depth() {
  const int want = DEPTH > 0 ? DEPTH : KS > 1 ? 2 : MT == 1 ? GEMM_DEPTH_MT1 : MT == 2 ? GEMM_DEPTH_MT2 : GEMM_DEPTH_MT4;
  const int cap = 112 / (NT * w_regs<FMT>() + (A8 ? MT : 0)) - 1;
  const int d = want < cap ? want : cap;
  return d < 2 ? 2 : d;
}

// Weight loads are issued as plain vector loads the compiler does not track:
// its wait analysis cannot count the LDS-DMA activation loads issued after
// them and would otherwise wait for every outstanding load before each use.
// The kernel waits for them explicitly (vmcnt) before touching the registers.
__device__ __forceinline__ u32x4_t vload16(const void *p) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t vload1(const void *p) {
  uint32_t v;
  asm volatile("global_load_ubyte %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// An empty asm that reads the registers: placed after the final wait, it
// keeps the last (discarded) prefetch's destination registers allocated until
// the load has landed, so the compiler cannot reuse them while it is in flight.
__device__ __forceinline__ void hold(const WRaw<SPEC_WFMT_FP8_E4M3_ROW> &r) {
  asm volatile("" ::"v"(r.c[0]), "v"(r.c[1]));
}
__device__ __forceinline__ void hold(const WRaw<SPEC_WFMT_BF16> &r) {
  asm volatile("" ::"v"(r.c[0]), "v"(r.c[1]), "v"(r.c[2]), "v"(r.c[3]));
}
__device__ __forceinline__ void hold(const WRaw<SPEC_WFMT_MXFP4> &r) { asm volatile("" ::"v"(r.c), "v"(r.e)); }

// One lane's raw weights of one tile for k step `ks`, from the tile-major
// layout: wl = the lane's chunk 0 of the tile row's first k step, sl = its
// scale byte (MXFP4).  FP8 lanes get k 16h..16h+15 and 32+16h..+15 of the
// step (the scaled FP8 instruction's operand order), BF16 and MXFP4 lanes the
// 32 consecutive k 32h..32h+31.
template <int FMT>
__device__ __forceinline__ void load_w(WRaw<FMT> &r, const uint8_t *wl, const uint8_t *sl, int ks) {
  const uint8_t *p = wl + (size_t)ks * tile_bytes(FMT);
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
    r.c[0] = vload16(p);
    r.c[1] = vload16(p + 1024);
  } else if constexpr (FMT == SPEC_WFMT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = vload16(p + 1024 * i);
  } else {
    r.c = vload16(p);
    r.e = vload1(sl + (size_t)ks * 64);
  }
}

// Activation chunk (8 k, 16 bytes) that pairs with the lane's weight slice i
// on the 32x32x16 MFMA: FP8 slices are k 16h + 8i (i < 2) and 32 + 16h +
// 8(i - 2); BF16 and MXFP4 slices are k 32h + 8i.
template <int FMT>
__device__ __forceinline__ int act_chunk(int i, int h) {
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) return (i < 2 ? 0 : 4) + 2 * h + (i & 1);
  else return 4 * h + i;
}

// 32 weights -> four 8-element MFMA operands in the activation type
template <bool F16, int FMT>
__device__ __forceinline__ void cvt_w(const WRaw<FMT> &r, u32x4_t (&op)[4]) {
  if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = r.c[i >> 1][(i & 1) * 2], hi = r.c[i >> 1][(i & 1) * 2 + 1];
      u32x2_t a, b;
      if constexpr (F16) {
        a = fp8x4_to_f16x4(lo), b = fp8x4_to_f16x4(hi);
      } else {
        a = fp8x4_to_bf16x4(lo), b = fp8x4_to_bf16x4(hi);
      }
      op[i] = u32x4_t{a.x, a.y, b.x, b.y};
    }
  } else if constexpr (FMT == SPEC_WFMT_BF16) {
    static_assert(!F16, "BF16 weights pair with BF16 activations");
#pragma unroll
    for (int i = 0; i < 4; ++i) op[i] = r.c[i];
  } else {
    const float sc = __uint_as_float(r.e << 23);  // 2^(e-127); e = 0 only on all-zero blocks
#pragma unroll
    for (int i = 0; i < 4; ++i) op[i] = F16 ? fp4x8_to_f16x8(r.c[i], sc) : fp4x8_to_bf16x8(r.c[i], sc);
  }
}

template <bool F16>
__device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (F16) return mfma32x32x16_f16(a, b, c);
  else return mfma32x32x16(a, b, c);
}

struct GemmArgs {
  const void *x;      // activations [M][K]: fp16 or bf16 bits, or e4m3 codes (A8)
  const uint8_t *xs;  // A8: e8m0 scale of each 32 activations [M][K/32]
  int M, K;
  const uint8_t *w, *s;
  int nb, mb;         // N blocks (NG units each), M blocks
  int per_xcd;        // tiles per XCD (gridDim.x = 8 * per_xcd)
  int spl;            // k steps (of 64) per split; gridDim.z splits
  NormRows nr;        // per-row normalisation of the input rows (nr.ssp NULL: none)
  float *fx_part;     // splits reduced inside the launch (fx_cnt non-NULL): fp32 partial tiles
  int *fx_cnt;        // arrival counter per tile, zero between launches
  int krot;           // nonzero: M block m starts its k loop at step m * nsteps / mb and wraps round
};

// Linear workgroup id -> (N block, M block).  Workgroup L runs on XCD L % 8;
// the nb*mb tiles, in N-major order, are cut into 8 contiguous ranges of
// per_xcd tiles, one per XCD, so the M blocks that share an N block's weight
// rows sit on one XCD (one L2) as far as possible and every XCD gets work even
// when there are fewer than 8 N blocks.
__device__ __forceinline__ bool tile_of(int L, int nb, int mb, int per_xcd, int &n, int &m) {
  const int t = (L & 7) * per_xcd + (L >> 3);
  n = t / mb;
  m = t % mb;
  return t < nb * mb;
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at "no wait").
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds + 16 * i.  Kept out of the kernel templates (the host pass drops a
// template kernel that names this builtin directly).
__device__ __forceinline__ void lds_load16(const void *g, void *l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

// Activation tile in LDS: 16-byte chunk c of row r sits at chunk slot
// r*8 + (c ^ swz(r)).  A fragment read has the 16 lanes of one LDS phase on 16
// consecutive rows at one logical chunk; swz sends them to 16 distinct 16-byte
// bank groups of a 256-byte window (and rows r..r+7 to distinct groups of a
// 128-byte window), so the reads are free of bank conflicts.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// FP8 activation tile (A8): 64-byte rows of four 16-byte chunks, chunk c of
// row r at slot r*4 + (c ^ swz8(r)); the 16 lanes of a read phase (rows r..r+15,
// one logical chunk) land on 16 distinct bank groups of a 256-byte window.
__device__ __forceinline__ int swz8(int row) { return (row >> 2) & 3; }

// Waves per SIMD the register budget is sized for: two while a wave holds at
// most four 32x32 accumulator tiles (BF16 weights included: the lm_head's one
// vocab tile per wave and 128 rows run two waves per SIMD).
template <int FMT, int NT, int MT> struct GemmOcc {
  static constexpr int value = NT * MT <= 4 ? 2 : 1;
};

// Lane (c, h) of wave w reads the partial sums of squares of block row
// m0 + 32mt + c in 16-byte chunks j = 2w + h + 2*NWV*i, i < NRL (a kernel
// parameter: 0 when the input rows are not h * g, 1 for rows up to 1024
// wide with four waves, 4 for rows up to 4096).
inline int norm_loads(const NormRows &nr, int nwv) {
  if (!nr.ssp) return 0;
  const int nl = (nr.ld / 4 + 2 * nwv - 1) / (2 * nwv);
  return nl <= 1 ? 1 : nl <= 4 ? 4 : -1;
}

// A8: activations are MXFP8 (e4m3 codes + e8m0 per 32) and the MFMA is the
// scaled 32x32x64 FP8/FP4 one: one MFMA per tile pair and k step, FP8 weights
// enter raw (their per-row scale stays in the epilogue) and MXFP4 weights with
// their own e8m0 scales.
// Compile-time shape of one gemm_kernel instantiation, shared with the host
// (which sizes the launch's LDS from it).
template <int FMT, int NT, int MT, class Epi, bool A8, int NWV, int KS, int DEPTH>
struct GemmCfg {
  static constexpr int NG = NWV / KS;              // waves side by side along N
  static constexpr int ROWS = 32 * MT;             // activation rows per workgroup
  static constexpr int SUB = ROWS * 64;            // 16-bit elements of one k step's activation tile
  // LDS-DMA instructions per wave per stage: KS * ROWS * 8 (16-bit) or ROWS * 4 (FP8) chunks of 16 bytes
  static constexpr int AJ = A8 ? (MT + 1) / 2 : 4 * MT * KS / NWV;
  static constexpr int SE = A8 ? AJ * 2048 : SUB * KS;  // 16-bit elements per stage
  static constexpr int DIST = gemm_depth<FMT, NT, MT, A8, KS, DEPTH>();  // stages loaded ahead of the one computed
  static constexpr int NS = DIST + 1;              // LDS stages = weight register sets
  // staged epilogue: per wave a [32][LD] fp32 tile of block rows x output columns
  static constexpr int COLS = Epi::template cols<NT>(), LD = COLS + 4;
  static constexpr int STAGE_BYTES = Epi::kStaged ? NG * 32 * LD * 4 : 0;
  // after the main loop: the k groups' accumulators, then the lanes' partial
  // sums of squares of the input rows
  static constexpr int RED_BYTES = (KS - 1) * NG * NT * MT * 4096;
  static constexpr int RSUM_BYTES = MT * 2 * NWV * 32 * 4;
  static constexpr int A_BYTES = NS * SE * 2 > STAGE_BYTES ? NS * SE * 2 : STAGE_BYTES;
  static constexpr int LDS_BYTES = A_BYTES > RED_BYTES + RSUM_BYTES ? A_BYTES : RED_BYTES + RSUM_BYTES;
};

template <bool F16, int FMT, int NT, int MT, class Epi, bool A8, int NWV, int KS, int DEPTH, int NRL>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(GemmOcc<FMT, NT, MT>::value, 8))) void
gemm_kernel(GemmArgs ga, Epi epi) {
  static_assert(!A8 || FMT != SPEC_WFMT_BF16, "A8 takes FP8 or MXFP4 weights");
  static_assert(NWV % KS == 0 && (!A8 || KS == 1), "k groups divide the waves; A8 runs one k group");
  using C = GemmCfg<FMT, NT, MT, Epi, A8, NWV, KS, DEPTH>;
  constexpr int NG = C::NG, ROWS = C::ROWS, SUB = C::SUB, AJ = C::AJ, SE = C::SE, DIST = C::DIST, NS = C::NS;
  constexpr int COLS = C::COLS, LD = C::LD;
  static_assert(A8 || (AJ >= 1 && (4 * MT * KS) % NWV == 0), "a stage's activation chunks fill whole waves");
  extern __shared__ __align__(16) uint16_t gemm_lds[];  // C::LDS_BYTES
  uint16_t *const As = gemm_lds;

  pin_args(ga, epi);
  int nblk, mblk;
  if (!tile_of(blockIdx.x, ga.nb, ga.mb, ga.per_xcd, nblk, mblk)) return;  // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = wave % NG, kg = wave / NG;
  const int unit = nblk * NG + ng;
  const bool active = unit < epi.units;  // wave-uniform; inactive waves compute on unit 0 and store nothing
  const int m0 = mblk * ROWS;
  const int M = ga.M, K = ga.K, ksteps = K / 64;
  const int ks0 = blockIdx.z * ga.spl, nsteps = min(ks0 + ga.spl, ksteps) - ks0;
  const int nstage = (nsteps + KS - 1) / KS;  // stages of KS k steps
  // k order: steps krot .. nsteps-1, then 0 .. krot-1 (krot = 0: in order)
  const int krot = ga.krot ? (mblk * nsteps) / ga.mb : 0;
  auto rk = [&](int x) { const int y = x + krot; return y < nsteps ? y : y - nsteps; };

  // Every wave issues AJ activation loads and NT*w_loads (+ MT scale loads for
  // A8) weight loads per stage, so the vmcnt waits below are one compile-time
  // count for all waves.  agp: byte address of the lane's 16-byte chunk at k
  // step 0; agk: the k step of the stage it carries (wave-uniform).
  const uint8_t *agp[AJ];
  int agk[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i) {
    const int P = (wave + NWV * i) * 64 + lane;
    int row, ch;
    if constexpr (A8) {
      row = P >> 2;
      ch = (P & 3) ^ swz8(row);
      agk[i] = 0;
    } else {
      const int p = P % (ROWS * 8);
      row = p >> 3;
      ch = (p & 7) ^ swz(row);
      agk[i] = P / (ROWS * 8);
    }
    const int m = row < ROWS && m0 + row < M ? m0 + row : 0;  // rows past M (or padding) read row 0, never stored
    agp[i] = reinterpret_cast<const uint8_t *>(ga.x) + ((size_t)m * K + ks0 * 64) * (A8 ? 1 : 2) + ch * 16;
  }
  const uint8_t *asp[A8 ? MT : 1];  // A8: e8m0 of block h of block row 32*mt + c at k step 0
  if constexpr (A8) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 32 * mt + c < M ? m0 + 32 * mt + c : 0;
      asp[mt] = ga.xs + (size_t)m * (K / 32) + ks0 * 2 + h;
    }
  }
  const uint8_t *wl[NT], *sl[NT];  // the lane's chunk 0 / scale byte at k step 0 of each tile
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const size_t tile0 = (size_t)(epi.row(active ? unit : 0, t) >> 5) * ksteps + ks0;
    wl[t] = ga.w + tile0 * tile_bytes(FMT) + lane * 16;
    sl[t] = FMT == SPEC_WFMT_MXFP4 ? ga.s + tile0 * 64 + lane : nullptr;
  }

  f32x16_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][mt][v] = 0.f;

  // Partial sums of squares of the input rows (when the input is h * g),
  // loaded like the epilogue inputs below and added up after the main loop.
  constexpr bool norm = NRL > 0;
  constexpr int NRA = NRL > 0 ? NRL : 1;
  f32x4_t nrr[MT][NRA];
  const int nch = ga.nr.ld / 4;  // 16-byte chunks per row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(m0 + 32 * mt + c, M - 1);
#pragma unroll
    for (int i = 0; i < NRA; ++i) {
      const int j = 2 * wave + h + 2 * NWV * i;
      nrr[mt][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (norm && j < nch) nrr[mt][i] = *reinterpret_cast<const f32x4_t *>(ga.nr.ssp + (size_t)m * ga.nr.ld + 4 * j);
    }
  }

  // Epilogue inputs (per-row weight scales, cache lengths, the residual rows a
  // residual projection adds to) are loaded here, before the main loop, and
  // used only after its final wait: the epilogue then starts without a
  // dependent memory round trip.
  typename Epi::template Pre<NT, MT> pre;
  if (kg == 0) epi.template prefetch<NT, MT>(active ? unit : 0, m0, M, lane, pre);

  auto compute_a8 = [&](int stage, const WRaw<FMT>(&wr)[NT], const uint32_t(&sc)[A8 ? MT : 1]) {
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *base = reinterpret_cast<const uint8_t *>(As) + stage * SE * 2;
    i32x8_t wv[NT];
    int sa[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (FMT == SPEC_WFMT_FP8_E4M3_ROW) {
        const WRaw<SPEC_WFMT_FP8_E4M3_ROW> &r = reinterpret_cast<const WRaw<SPEC_WFMT_FP8_E4M3_ROW> &>(wr[t]);
        wv[t] = i32x8_t{(int)r.c[0].x, (int)r.c[0].y, (int)r.c[0].z, (int)r.c[0].w,
                        (int)r.c[1].x, (int)r.c[1].y, (int)r.c[1].z, (int)r.c[1].w};
        sa[t] = 127;  // 2^0: the per-row fp32 scale is applied in the epilogue
      } else {
        const WRaw<SPEC_WFMT_MXFP4> &r = reinterpret_cast<const WRaw<SPEC_WFMT_MXFP4> &>(wr[t]);
        wv[t] = i32x8_t{(int)r.c.x, (int)r.c.y, (int)r.c.z, (int)r.c.w, 0, 0, 0, 0};
        sa[t] = (int)r.e;
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = 32 * mt + c, sw = swz8(row);
      const u32x4_t b0 = *reinterpret_cast<const u32x4_t *>(base + row * 64 + ((h) ^ sw) * 16);
      const u32x4_t b1 = *reinterpret_cast<const u32x4_t *>(base + row * 64 + ((2 + h) ^ sw) * 16);
      const i32x8_t bv = i32x8_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][mt] = mfma_mx<FMT == SPEC_WFMT_MXFP4 ? 4 : 0>(wv[t], bv, acc[t][mt], sa[t], (int)sc[mt]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the next step's wait and barrier behind these MFMAs
  };
  auto compute = [&](int stage, const WRaw<FMT>(&wr)[NT]) {
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t wop[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) cvt_w<F16, FMT>(wr[t], wop[t]);
    const uint16_t *base = As + stage * SE + kg * SUB;  // this k group's step of the stage
    // slice i of block row 32*mt + c: logical chunk 4h + i
    auto read_a = [&](int i, u32x4_t (&af)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = 32 * mt + c;
        af[mt] = *reinterpret_cast<const u32x4_t *>(base + (row * 8 + (act_chunk<FMT>(i, h) ^ swz(row))) * 8);
      }
    };
    // the fragments of slice i+1 are read while slice i's MFMAs run
    u32x4_t af[2][MT];
    read_a(0, af[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i + 1 < 4) read_a(i + 1, af[(i + 1) & 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][mt] = mma<F16>(wop[t][i], af[i & 1][mt], acc[t][mt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto issue_a = [&](int st, int stage) {
#pragma unroll
    for (int i = 0; i < AJ; ++i)
      lds_load16(agp[i] + rk(min(st * KS + agk[i], nsteps - 1)) * (A8 ? 64 : 128),
                 As + stage * SE + (wave + NWV * i) * 512);
  };
  auto issue_w = [&](WRaw<FMT>(&wr)[NT], uint32_t(&sc)[A8 ? MT : 1], int st) {
    const int step = rk(min(st * KS + kg, nsteps - 1));
#pragma unroll
    for (int t = 0; t < NT; ++t) load_w<FMT>(wr[t], wl[t], sl[t], step);
    if constexpr (A8) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sc[mt] = vload1(asp[mt] + step * 2);
    }
  };
  // Software pipeline, DIST stages deep.  At stage s the wave issues stage
  // s+DIST (weights into register set (s+DIST)%NS, then activations straight
  // to LDS stage (s+DIST)%NS) and computes its k step of stage s from set /
  // stage s%NS.  The loop is unrolled NS times so every register set has a
  // fixed name: a register copy of a load destination would be placed before
  // the wait that covers it.  Stages past the end re-load the last k step
  // into a set / stage nobody reads.  Loads complete in issue order, so
  // "stage s landed" is "at most the loads of stages s+1 .. s+DIST-1
  // outstanding".
  constexpr int PER_STEP = NT * w_loads<FMT>() + (A8 ? MT : 0) + AJ;
  static_assert(DIST * PER_STEP < 64, "vmcnt holds 6 bits");
  WRaw<FMT> wr[NS][NT];
  uint32_t scr[NS][A8 ? MT : 1];
#pragma unroll
  for (int i = 0; i < DIST; ++i) {
    issue_w(wr[i], scr[i], min(i, nstage - 1));
    issue_a(min(i, nstage - 1), i);
  }
  for (int s0 = 0; s0 < nstage; s0 += NS) {
#pragma unroll
    for (int ph = 0; ph < NS; ++ph) {
      const int s = s0 + ph;
      WAIT_VMCNT((DIST - 1) * PER_STEP);
      lds_barrier();  // stage s visible to all waves; every wave is done with stage s-1
      __builtin_amdgcn_sched_barrier(0);
      issue_w(wr[(ph + DIST) % NS], scr[(ph + DIST) % NS], min(s + DIST, nstage - 1));
      issue_a(min(s + DIST, nstage - 1), (ph + DIST) % NS);
      __builtin_amdgcn_sched_barrier(0);
      if (s * KS + kg < nsteps) {  // stages past the last (or a k group past the last step) only keep the counts uniform
        if constexpr (A8) compute_a8(ph, wr[ph], scr[ph]);
        else compute(ph, wr[ph]);
      }
    }
  }
  WAIT_VMCNT(0);  // nothing may still be landing in LDS or registers past this point
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
#pragma unroll
    for (int t = 0; t < NT; ++t) hold(wr[i][t]);
    if constexpr (A8) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) asm volatile("" ::"v"(scr[i][mt]));
    }
  }
  // After the main loop the stage memory holds the k groups' accumulators
  // (groups 1.. hand theirs to group 0, which adds them in group order, so
  // the result does not depend on timing) and each lane's partial sum of
  // squares of its input row (each lane's chunks summed in order).
  float rs[MT];
  if (KS > 1 || norm) {
    float *red = reinterpret_cast<float *>(As);
    float *rsum = red + C::RED_BYTES / 4;  // [MT][2 NWV][32]
    lds_barrier();  // every wave is done reading the activation stages
    if (KS > 1 && kg > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            red[((((kg - 1) * NG + ng) * NT + t) * MT + mt) * 1024 + v * 64 + lane] = acc[t][mt][v];
    }
    if (norm) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < NRA; ++i) ps += (nrr[mt][i][0] + nrr[mt][i][1]) + (nrr[mt][i][2] + nrr[mt][i][3]);
        rsum[(mt * 2 * NWV + 2 * wave + h) * 32 + c] = ps;
      }
    }
    lds_barrier();
    if (KS > 1 && kg == 0) {
#pragma unroll
      for (int g = 1; g < KS; ++g)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[t][mt][v] += red[((((g - 1) * NG + ng) * NT + t) * MT + mt) * 1024 + v * 64 + lane];
    }
    // per-row normalisation of the input: r = 1 / sqrt(sum / H + eps), the
    // lanes' sums added in a fixed order
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      rs[mt] = 1.f;
      if (norm) {
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < 2 * NWV; ++q) ss += rsum[(mt * 2 * NWV + q) * 32 + c];
        rs[mt] = 1.0f / sqrtf(ss / (float)ga.nr.H + ga.nr.eps);
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) rs[mt] = 1.f;
  }
  // Splits reduced inside the launch: every split's k group 0 writes its
  // partial tile (fp32, accumulator v of all 64 lanes contiguous) with
  // device-coherent stores, waits until they have completed, and counts its
  // arrival on the tile's counter; the last split to arrive (whichever it
  // is) reads the others' partials with device-coherent loads, adds all of
  // them in split order, sets the counter back to zero and runs the
  // epilogue; the others are done.  Only the partials and the counter cross
  // workgroups, each access coherent at device scope on its own, so no
  // fence (which would write back or invalidate the whole L2 of an XCD) is
  // needed.
  const bool fix = ga.fx_cnt != nullptr && gridDim.z > 1;
  if (fix) {
    const int S = gridDim.z, z = blockIdx.z, blk = mblk * ga.nb + nblk;
    auto tile_part = [&](int zz, int t, int mt) {
      return ga.fx_part + ((((size_t)blk * S + zz) * NG + ng) * (NT * MT) + t * MT + mt) * 1024 + lane;
    };
    if (kg == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          float *q = tile_part(z, t, mt);
#pragma unroll
          for (int v = 0; v < 16; ++v) __hip_atomic_store(q + 64 * v, acc[t][mt][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    WAIT_VMCNT(0);    // this wave's partials have reached the device's coherence point
    __syncthreads();  // every wave's (also: no wave still reads the reduction scratch below)
    volatile int *flag = reinterpret_cast<volatile int *>(As);
    if (tid == 0) *flag = __hip_atomic_fetch_add(ga.fx_cnt + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    const bool last = *flag != 0;
    if (!last) return;  // whole workgroup
    if (tid == 0) __hip_atomic_store(ga.fx_cnt + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (kg == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x16_t tot = acc[t][mt];
          for (int z0 = 0; z0 < S; z0 += 4) {
            float b[4][16];  // four splits' partials in flight at once (past the last: the last again)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float *q = tile_part(min(z0 + u, S - 1), t, mt);
#pragma unroll
              for (int v = 0; v < 16; ++v) b[u][v] = __hip_atomic_load(q + 64 * v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int zz = z0 + u;
              if (zz >= S) break;
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const float x = zz == z ? acc[t][mt][v] : b[u][v];
                tot[v] = zz == 0 ? x : tot[v] + x;
              }
            }
          }
          acc[t][mt] = tot;
        }
    }
  }
  const bool emit_ok = active && kg == 0;
  if constexpr (Epi::kStaged) {
    // Each wave of k group 0 writes its finished outputs (scaled, RoPE /
    // SwiGLU applied) as fp32 into its own LDS tile, then reads it back along
    // rows so that every global store covers consecutive columns of one row.
    // The tile is wave private and a wave's LDS operations run in order, so
    // only the barrier that retires the activation stages is needed.
    constexpr int LPR = COLS / 4, RPP = 64 / LPR;  // lanes per row, rows per pass
    static_assert(COLS % 4 == 0 && 64 % LPR == 0 && LPR <= 64, "staged tile shape");
    lds_barrier();  // every wave is done reading the activation stages (or the k groups' sums)
    float *st = reinterpret_cast<float *>(As) + ng * 32 * LD;
    if (emit_ok) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (m0 + 32 * mt >= M) break;
        epi.template emit<NT, MT>(unit, mt, c, h, acc, rs[mt], pre, st, LD);
#pragma unroll
        for (int r0 = 0; r0 < 32; r0 += RPP) {
          const int row = r0 + lane / LPR, col = 4 * (lane % LPR), m = m0 + 32 * mt + row;
          const f32x4_t v = *reinterpret_cast<const f32x4_t *>(st + row * LD + col);
          epi.template put<NT, MT>(unit, m, M, col, v, fix ? 0 : (int)blockIdx.z, mt, r0 / RPP, pre);
        }
      }
    }
  } else {
    epi.template store<NT, MT, NWV>(active ? unit : 0, nblk, emit_ok, wave, m0, M, c, h, acc, rs, As);
  }
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

// Outputs of lane (c, h) for tile rows 8q + 4h + (0..3) of a tile.
__device__ __forceinline__ f32x4_t quad(const f32x16_t &a, int q) {
  return f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
}

// Per-row scales of tile rows row(unit, t) + 8q + 4h + (0..3), the rows lane
// (., h) holds for tile t (1 without per-row scales), for up to two tiles per
// wave.
template <int NT>
struct ScalePre {
  f32x4_t s[NT][4];
};
template <int NT, class E>
__device__ __forceinline__ void prefetch_scales(const E &e, const float *scale, int unit, int h, ScalePre<NT> &p) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) p.s[t][q] = row_scale4(scale, e.row(unit, t) + 8 * q + 4 * h);
}

// ---------------------------------------------------------------- epilogues
// Each epilogue maps (unit, tile t) to the first of the tile's 32 packed
// weight rows (row()).  Lane (c, h) holds block row m0 + 32*mt + c and tile
// rows 8q + 4h + (0..3).  Staged epilogues emit() a wave's finished values
// for one 32-row block into the LDS tile st[block row][output column] (cols()
// columns), and put() stores 4 consecutive output columns of one row (pass p
// of the wave's row passes over block mt; m may be >= M: store nothing).
// prefetch() loads, before the main loop, what the epilogue will need into a
// Pre; r is the block row's normalisation (1 when the input is not h * g).

template <int NTc>
struct EpiF32 {  // y = acc * scale, fp32 out
  static constexpr bool kStaged = true;
  static constexpr bool kNormInput = false;
  static constexpr int kNT = NTc;
  int units, N;
  float *y;
  const float *scale;
  __device__ int row(int unit, int t) const { return unit * 32 * NTc + 32 * t; }
  template <int NT> static constexpr int cols() { return 32 * NT; }
  template <int NT, int MT> using Pre = ScalePre<NT>;
  template <int NT, int MT>
  __device__ void prefetch(int unit, int m0, int M, int lane, Pre<NT, MT> &p) const {
    prefetch_scales<NT>(*this, scale, unit, lane >> 5, p);
  }
  template <int NT, int MT>
  __device__ void emit(int unit, int mt, int c, int h, const f32x16_t (&acc)[NT][MT], float r, const Pre<NT, MT> &p,
                       float *st, int ld) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t *>(st + c * ld + 32 * t + 8 * q + 4 * h) = quad(acc[t][mt], q) * (p.s[t][q] * r);
  }
  template <int NT, int MT>
  __device__ void put(int unit, int m, int M, int col, f32x4_t v, int z, int mt, int pass, const Pre<NT, MT> &p) const {
    if (m < M) *reinterpret_cast<f32x4_t *>(y + (size_t)m * N + row(unit, 0) + col) = v;
  }
};

// Split-K partial of a residual projection: P[z][m][n] = acc * scale.  The
// next RMSNorm adds the partials of every split to h in split order (the
// MXFP8-activation mode, whose RMSNorm steps quantise their output).
template <int NTc>
struct EpiPartial {
  static constexpr bool kStaged = true;
  static constexpr bool kNormInput = false;
  static constexpr int kNT = NTc;
  int units, N, M;
  float *part;  // [nsplit][M][N]
  const float *scale;
  __device__ int row(int unit, int t) const { return unit * 32 * NTc + 32 * t; }
  template <int NT> static constexpr int cols() { return 32 * NT; }
  template <int NT, int MT> using Pre = ScalePre<NT>;
  template <int NT, int MT>
  __device__ void prefetch(int unit, int m0, int Mr, int lane, Pre<NT, MT> &p) const {
    prefetch_scales<NT>(*this, scale, unit, lane >> 5, p);
  }
  template <int NT, int MT>
  __device__ void emit(int unit, int mt, int c, int h, const f32x16_t (&acc)[NT][MT], float r, const Pre<NT, MT> &p,
                       float *st, int ld) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t *>(st + c * ld + 32 * t + 8 * q + 4 * h) = quad(acc[t][mt], q) * p.s[t][q];
  }
  template <int NT, int MT>
  __device__ void put(int unit, int m, int Mr, int col, f32x4_t v, int z, int mt, int pass, const Pre<NT, MT> &p) const {
    if (m < Mr) *reinterpret_cast<f32x4_t *>(part + ((size_t)z * M + m) * N + row(unit, 0) + col) = v;
  }
};

// Residual projection with the next RMSNorm folded in: h_out = h_in + acc *
// scale (fp32), xg = h_out * g of the RMSNorm that reads h_out (FP16, or BF16
// for the lm_head's input), and the sum of h_out^2 over each 32-column tile
// into ssp[m][n / 32] (the normalisation itself is applied by the consumer).
// An FP16 xg beyond the format's range sets SPEC_DERR_RANGE.
template <int NTc>
struct EpiResidual {
  static constexpr bool kStaged = true;
  static constexpr bool kNormInput = false;
  static constexpr int kNT = NTc;
  int units, N;
  const float *scale;
  ResidualOut o;
  __device__ int row(int unit, int t) const { return unit * 32 * NTc + 32 * t; }
  template <int NT> static constexpr int cols() { return 32 * NT; }
  static constexpr int kPasses = 32 / (64 / (8 * NTc));  // row passes of a 32-row block (LPR = 8 NT lanes per row)
  template <int NT, int MT>
  struct Pre {
    f32x4_t s[NT][4];
    f32x4_t hin[MT][kPasses];  // h_in at the lane's put() positions
    f32x4_t g;                 // the gain of the lane's 4 columns
  };
  template <int NT, int MT>
  __device__ void prefetch(int unit, int m0, int M, int lane, Pre<NT, MT> &p) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) p.s[t][q] = row_scale4(scale, row(unit, t) + 8 * q + 4 * (lane >> 5));
    constexpr int LPR = 8 * NT, RPP = 64 / LPR;
    const int n = row(unit, 0) + 4 * (lane % LPR);
    p.g = *reinterpret_cast<const f32x4_t *>(o.gain + n);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const int m = min(m0 + 32 * mt + ps * RPP + lane / LPR, M - 1);
        p.hin[mt][ps] = *reinterpret_cast<const f32x4_t *>(o.h_in + (size_t)m * N + n);
      }
  }
  template <int NT, int MT>
  __device__ void emit(int unit, int mt, int c, int h, const f32x16_t (&acc)[NT][MT], float r, const Pre<NT, MT> &p,
                       float *st, int ld) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t *>(st + c * ld + 32 * t + 8 * q + 4 * h) = quad(acc[t][mt], q) * p.s[t][q];
  }
  template <int NT, int MT>
  __device__ void put(int unit, int m, int M, int col, f32x4_t v, int z, int mt, int pass, const Pre<NT, MT> &p) const {
    const int n = row(unit, 0) + col;
    const f32x4_t hv = p.hin[mt][pass] + v;
    const f32x4_t xg = hv * p.g;
    // sum of squares over the 32-column tile: its 8 lanes are consecutive
    float ss = (hv[0] * hv[0] + hv[1] * hv[1]) + (hv[2] * hv[2] + hv[3] * hv[3]);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    if (m >= M) return;
    *reinterpret_cast<f32x4_t *>(o.h_out + (size_t)m * N + n) = hv;
    if (o.xg_bf16) {
      store_bf16x4(o.xg + (size_t)m * N + n, xg[0], xg[1], xg[2], xg[3]);
    } else {
      store_f16x4(o.xg + (size_t)m * N + n, xg[0], xg[1], xg[2], xg[3]);
      const float mx = fmaxf(fmaxf(fabsf(xg[0]), fabsf(xg[1])), fmaxf(fabsf(xg[2]), fabsf(xg[3])));
      if (!(mx <= 65504.f)) set_error(o.err, SPEC_DERR_RANGE);
    }
    if ((col & 31) == 0) o.ssp[(size_t)m * o.ssp_ld + n / 32] = ss;
  }
};

// QKV projection: a unit is NT tiles of the packed QKV rows.  Each head's D
// rows are packed so that tile tp of the head holds dimensions 16tp .. 16tp+15
// in tile rows 0..15 and D/2 + 16tp .. +15 in rows 16..31: the rotate-half
// RoPE pair (d, d + D/2) is then tile rows (r, r + 16), held by the same lane.
// Heads: q heads, then k heads, then v heads.  q goes out as FP16, k and v
// into the BF16 cache at slot kv_len[b] + j of block row m = 16b + j.
template <int NTc>
struct EpiQkv {
  static constexpr bool kStaged = true;
  static constexpr bool kNormInput = true;
  static constexpr int kNT = NTc;
  int units;  // units of NTc tiles
  const float *scale;  // packed per-row scales
  QkvOut o;
  __device__ int row(int unit, int t) const { return unit * 32 * NTc + 32 * t; }
  template <int NT> static constexpr int cols() { return 32 * NT; }
  __device__ bool slot_ok(int n0) const { return n0 >= 0 && n0 + 16 <= o.max_ctx; }  // else flagged by embed
  template <int NT, int MT>
  struct Pre {
    f32x4_t s[NT][4];
    int kvl[2 * MT];  // cache length of each of the block's sequences
  };
  template <int NT, int MT>
  __device__ void prefetch(int unit, int m0, int M, int lane, Pre<NT, MT> &p) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) p.s[t][q] = row_scale4(scale, row(unit, t) + 8 * q + 4 * (lane >> 5));
    // through the constant address space: scalar loads, which the vector
    // loads in flight need not wait for (kv_len does not change during the
    // kernel, and the scalar cache is invalidated at each launch)
    const __attribute__((address_space(4))) int32_t *kl = (const __attribute__((address_space(4))) int32_t *)o.kv_len;
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      const int b = (m0 >> 4) + i;
      p.kvl[i] = b < (M >> 4) ? kl[b] : 0;
    }
  }
  template <int NT, int MT>
  __device__ void emit(int unit, int mt, int c, int h, const f32x16_t (&acc)[NT][MT], float r, const Pre<NT, MT> &p,
                       float *st, int ld) const {
    const int D = o.D, TPH = D / 32;
    const int n0 = (c >> 4) ? p.kvl[2 * mt + 1] : p.kvl[2 * mt], pos = n0 + (c & 15);  // selects: no indexed registers
    const int half = D / 2;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int T = unit * NTc + t, head = T / TPH, tp = T % TPH;
      if (head < o.Hq + o.Hkv && slot_ok(n0)) {  // q and k heads are rotated
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int d = 16 * tp + 8 * q + 4 * h;  // < D/2; its pair is d + D/2
          const f32x4_t y1 = quad(acc[t][mt], q) * (p.s[t][q] * r);
          const f32x4_t y2 = quad(acc[t][mt], q + 2) * (p.s[t][q + 2] * r);
          const f32x4_t cs01 = *reinterpret_cast<const f32x4_t *>(o.rope + (size_t)pos * half + d);
          const f32x4_t cs23 = *reinterpret_cast<const f32x4_t *>(o.rope + (size_t)pos * half + d + 2);
          const float cs[4] = {cs01[0], cs01[2], cs23[0], cs23[2]}, sn[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
          f32x4_t o1, o2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o1[i] = y1[i] * cs[i] - y2[i] * sn[i];
            o2[i] = y2[i] * cs[i] + y1[i] * sn[i];
          }
          *reinterpret_cast<f32x4_t *>(st + c * ld + 32 * t + 8 * q + 4 * h) = o1;
          *reinterpret_cast<f32x4_t *>(st + c * ld + 32 * t + 8 * (q + 2) + 4 * h) = o2;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4_t *>(st + c * ld + 32 * t + 8 * q + 4 * h) = quad(acc[t][mt], q) * (p.s[t][q] * r);
      }
    }
  }
  template <int NT, int MT>
  __device__ void put(int unit, int m, int M, int col, f32x4_t v, int z, int mt, int pass, const Pre<NT, MT> &p) const {
    if (m >= M) return;
    const int D = o.D, TPH = D / 32;
    const int b = m >> 4, n0 = ((m & 31) >> 4) ? p.kvl[2 * mt + 1] : p.kvl[2 * mt];
    if (!slot_ok(n0)) return;
    const int T = unit * NTc + col / 32, head = T / TPH, tp = T % TPH, rr = col % 32;
    const int d = rr < 16 ? 16 * tp + rr : D / 2 + 16 * tp + (rr - 16);
    const float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    if (!(mx <= 65504.f)) set_error(o.err, SPEC_DERR_RANGE);  // attention reads q, k, v as FP16
    if (head < o.Hq) {
      store_f16x4(o.q_out + (size_t)m * (o.Hq * D) + head * D + d, v[0], v[1], v[2], v[3]);
    } else {
      const int pos = n0 + (m & 15);
      const bool isk = head < o.Hq + o.Hkv;
      const int kvh = isk ? head - o.Hq : head - o.Hq - o.Hkv;
      uint16_t *cache = isk ? o.k_cache : o.v_cache;
      bool ok;
      const size_t rrow = o.kvl.row(b, kvh, o.Hkv, o.max_ctx, pos, ok);
      if (ok) store_bf16x4(cache + rrow * D + d, v[0], v[1], v[2], v[3]);
    }
  }
};

// Gate/up projection with SiLU(gate) * up: tile T of the packed rows holds
// gate rows 16T .. 16T+15 in tile rows 0..15 and the matching up rows in rows
// 16..31, so each lane holds its gate values and their up partners.  A unit
// of NT tiles yields 16*NT outputs per row; a = SiLU(gate) * up goes out as
// FP16, or (MX8, NT = 2) as MXFP8: e4m3 codes [M][I] plus the e8m0 exponent of
// each 32 outputs [M][I/32], one block per unit and row, held by 8
// consecutive lanes of the staged store.
template <int NTc, bool MX8 = false>
struct EpiSwiglu {
  static constexpr bool kStaged = true;
  static constexpr bool kNormInput = true;
  static constexpr int kNT = NTc;
  static_assert(!MX8 || NTc == 2, "an MXFP8 block is the 32 outputs of one row of a unit");
  int units, I;
  const float *scale;  // packed per-row FP8 scales [2I], NULL when decoded with the scale
  void *a;             // FP16 bits or e4m3 codes
  uint8_t *as;         // MX8: e8m0 [M][I/32]
  __device__ int row(int unit, int t) const { return unit * 32 * NTc + 32 * t; }
  template <int NT> static constexpr int cols() { return 16 * NT; }
  template <int NT, int MT> using Pre = ScalePre<NT>;
  template <int NT, int MT>
  __device__ void prefetch(int unit, int m0, int M, int lane, Pre<NT, MT> &p) const {
    prefetch_scales<NT>(*this, scale, unit, lane >> 5, p);
  }
  template <int NT, int MT>
  __device__ void emit(int unit, int mt, int c, int h, const f32x16_t (&acc)[NT][MT], float r, const Pre<NT, MT> &p,
                       float *st, int ld) const {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4_t gv = quad(acc[t][mt], q) * (p.s[t][q] * r);
        const f32x4_t uv = quad(acc[t][mt], q + 2) * (p.s[t][q + 2] * r);
        f32x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = gv[i] * __builtin_amdgcn_rcpf(1.f + __expf(-gv[i])) * uv[i];  // SiLU(g) * u
        *reinterpret_cast<f32x4_t *>(st + c * ld + 16 * t + 8 * q + 4 * h) = v;
      }
  }
  template <int NT, int MT>
  __device__ void put(int unit, int m, int M, int col, f32x4_t v, int z, int mt, int pass, const Pre<NT, MT> &p) const {
    const int n = unit * 16 * NTc + col;
    if constexpr (MX8) {
      uint32_t e8;
      const uint32_t codes = mx8_quant4(v, e8);  // lanes col/4 = 0..7 of this row share the block
      if (m >= M) return;
      *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(a) + (size_t)m * I + n) = codes;
      if ((col & 31) == 0) as[(size_t)m * (I / 32) + n / 32] = (uint8_t)e8;
    } else {
      if (m < M) store_f16x4(static_cast<uint16_t *>(a) + (size_t)m * I + n, v[0], v[1], v[2], v[3]);
    }
  }
};

// lm_head tile -> one argmax partial per (row, workgroup), lowest index on
// ties: each wave reduces its 32*NT vocab rows in registers, the workgroup's
// waves meet in LDS, and wave 0 folds them in wave order (increasing vocab
// index).  Called by every wave of the workgroup (inactive ones contribute
// nothing), after the main loop.  The input rows are h * g of the final
// RMSNorm; its normalisation r > 0 scales a whole row of logits and so
// cannot move the row's argmax: the argmax is taken on the unscaled sums,
// and r is applied only to the logits a test dump asks for (the launch then
// passes the partial sums of squares).
template <int NTc>
struct EpiArgmax {
  static constexpr bool kStaged = false;
  static constexpr bool kNormInput = true;
  static constexpr int kNT = NTc;
  template <int NT> static constexpr int cols() { return 4; }
  template <int NT, int MT>
  struct Pre {};
  int units, V, nparts;
  ArgmaxPart *part;  // [M][nparts], nparts = workgroups along the vocab
  float *logits;     // optional [M][V]
  __device__ int row(int unit, int t) const { return unit * 32 * NTc + 32 * t; }
  template <int NT, int MT>
  __device__ void prefetch(int unit, int m0, int M, int lane, Pre<NT, MT> &p) const {}
  template <int NT, int MT, int NWV>
  __device__ void store(int unit, int nblk, bool active, int wave, int m0, int M, int c, int h,
                        const f32x16_t (&acc)[NT][MT], const float (&rs)[MT], void *lds) const {
    ArgmaxPart *red = static_cast<ArgmaxPart *>(lds);  // [NWV waves][32 * MT rows]
    lds_barrier();  // every wave is done reading the activation stages
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 32 * mt + c;
      // a lane visits its candidates in increasing vocab index, so a strict
      // ">" keeps the lowest index among equal maxima; selects, not branches
      float bv = -INFINITY;
      int32_t bi = 0x7fffffff;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int n = row(unit, t) + 8 * (v >> 2) + 4 * h + (v & 3);
          const float lv = acc[t][mt][v];
          const bool gt = lv > bv;
          bv = gt ? lv : bv;
          bi = gt ? n : bi;
        }
      const float ov = __shfl_xor(bv, 32);  // the other half holds the other rows of the same block row
      const int32_t oi = __shfl_xor(bi, 32);
      const bool take = better(ov, oi, bv, bi);
      bv = active && take ? ov : (active ? bv : -INFINITY);
      bi = active && take ? oi : (active ? bi : 0x7fffffff);
      if (h == 0) red[wave * 32 * MT + 32 * mt + c] = ArgmaxPart{bv, bi};
      if (active && m < M && logits) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4_t *>(logits + (size_t)m * V + row(unit, t) + 8 * q + 4 * h) = quad(acc[t][mt], q) * rs[mt];
      }
    }
    lds_barrier();
    if (wave != 0) return;
    const int lane = 32 * h + c;
#pragma unroll
    for (int r = lane; r < 32 * MT; r += 64) {
      ArgmaxPart b = red[r];
#pragma unroll
      for (int w = 1; w < NWV; ++w) {
        const ArgmaxPart o = red[w * 32 * MT + r];
        if (better(o.v, o.i, b.v, b.i)) b = o;
      }
      if (m0 + r < M) part[(size_t)(m0 + r) * nparts + nblk] = b;
    }
  }
};

// ---------------------------------------------------------------- planning

GemmPlan gemm_plan(int M, int units, int ksteps, int MT, bool allow_split, int ng) {
  GemmPlan p;
  p.MT = MT;
  p.NG = ng;
  p.KS = 1;
  p.nb = (units + ng - 1) / ng;
  p.mb = (M + 32 * MT - 1) / (32 * MT);
  const int tiles = p.nb * p.mb;
  // split K (the MXFP8 mode's residual projections only) until about
  // GEMM_SPLIT_TARGET workgroups, >= 4 k steps per split
  int s = allow_split ? (GEMM_SPLIT_TARGET + tiles - 1) / tiles : 1;
  if (s > ksteps / 4) s = ksteps / 4;
  if (s < 1) s = 1;
  p.spl = (ksteps + s - 1) / s;
  p.nsplit = (ksteps + p.spl - 1) / p.spl;  // every split non-empty
  p.grid_x = 8 * ((tiles + 7) / 8);
  return p;
}

// 32-row activation tiles per workgroup: wide tiles unless that leaves fewer
// than 256 workgroups (the MXFP8 mode and the lm_head)
static int pick_mt(int M, int units, int maxMT) {
  int mt = M <= 32 ? 1 : M <= 64 ? 2 : 4;
  if (mt > maxMT) mt = maxMT;
  while (mt > 1 && ((units + 3) / 4) * ((M + 32 * mt - 1) / (32 * mt)) < 256) mt /= 2;
  return mt;
}

// Workgroup shapes of the decoder GEMMs with 16-bit activations: NWV waves,
// NG of them side by side along N by KS along K, NT 32-row weight tiles per
// wave, a 32*MT-row activation tile, DEPTH stages in flight.  Short-K
// launches at these row counts are bound by how many memory round trips they
// wait for, so the shapes keep most of a K of 896 in flight; the one
// MFMA-heavy launch (gate/up at hundreds of rows) takes two tiles per wave,
// so that each activation fragment read from LDS feeds two MFMAs.
struct Shape {
  int nwv, ng, ks, mt, nt, depth;
};
enum ShapeId { kS412, kS222, kS411, kS221, kS141, kS241w8, kS812w8, kS181w8, kS4112, kNumShapes };
#ifndef GEMM_DEPTH_S221
#define GEMM_DEPTH_S221 3
#endif
#ifndef GEMM_DEPTH_S241W8
#define GEMM_DEPTH_S241W8 3
#endif
#ifndef GEMM_DEPTH_S812W8
#define GEMM_DEPTH_S812W8 2
#endif
static constexpr Shape kShapes[kNumShapes] = {
    {4, 4, 1, 2, 1, 4},                  // 128 weight rows x 64 activation rows
    {4, 2, 2, 2, 1, 3},                  // 64 x 64, two k groups
    {4, 4, 1, 1, 1, 6},                  // 128 x 32
    {4, 2, 2, 1, 1, GEMM_DEPTH_S221},    // 64 x 32, two k groups
    {4, 1, 4, 1, 1, 3},                  // 32 x 32, four k groups
    {8, 2, 4, 1, 1, GEMM_DEPTH_S241W8},  // 64 x 32, four k groups
    {8, 8, 1, 2, 2, GEMM_DEPTH_S812W8},  // 512 x 64, two tiles per wave
    {8, 1, 8, 1, 1, 2},                  // 32 x 32, eight k groups
    {4, 4, 1, 1, 2, 3},                  // 256 x 32, two tiles per wave
};

// Shape per GEMM and row count (the thresholds and choices measured over
// whole passes of the 0.5B model at 16, 256 and 512 rows and of the 8B model
// at 128 rows).  Gate/up: from 512 rows the 8-wave 512 x 64 tiles (152
// workgroups at 512 rows); from 256, 256 x 32 tiles with two per wave (304
// workgroups at 256 rows, where the wide tiles leave 180 CUs idle: 16.3 ->
// 12.4 us); below, 128 x 64.
#ifndef GEMM_SMALL_M
#define GEMM_SMALL_M 64
#endif
#ifndef GEMM_WIDE_M
#define GEMM_WIDE_M 512
#endif
#ifndef GEMM_MID_M
#define GEMM_MID_M 256
#endif
#ifndef GEMM_SHAPE_QKV
#define GEMM_SHAPE_QKV kS221
#endif
#ifndef GEMM_SHAPE_OPROJ
#define GEMM_SHAPE_OPROJ kS221
#endif
#ifndef GEMM_SHAPE_GATE_UP
#define GEMM_SHAPE_GATE_UP kS812w8
#endif
#ifndef GEMM_SHAPE_GATE_UP_MID
#define GEMM_SHAPE_GATE_UP_MID kS4112
#endif
#ifndef GEMM_SHAPE_GATE_UP_NARROW
#define GEMM_SHAPE_GATE_UP_NARROW kS412
#endif
#ifndef GEMM_SHAPE_DOWN
#define GEMM_SHAPE_DOWN kS241w8
#endif
#ifndef GEMM_SHAPE_SMALL
#define GEMM_SHAPE_SMALL kS141
#endif
#ifndef GEMM_SHAPE_DOWN_SMALL
#define GEMM_SHAPE_DOWN_SMALL kS181w8
#endif
static int decoder_shape(int kind, int M) {
  if (M <= GEMM_SMALL_M) return kind == kGemmDown ? GEMM_SHAPE_DOWN_SMALL : GEMM_SHAPE_SMALL;
  switch (kind) {
    case kGemmQkv: return GEMM_SHAPE_QKV;
    case kGemmOproj: return GEMM_SHAPE_OPROJ;
    case kGemmGateUp:
      return M >= GEMM_WIDE_M ? GEMM_SHAPE_GATE_UP : M >= GEMM_MID_M ? GEMM_SHAPE_GATE_UP_MID : GEMM_SHAPE_GATE_UP_NARROW;
    default: return GEMM_SHAPE_DOWN;
  }
}

// Split K, reduced inside the launch, for the GEMMs in GEMM_FIX_KINDS (bit
// per GemmKind) whose tiles give fewer than GEMM_FIX_TARGET workgroups: up to
// that many, at most 8 splits, each k group of a split at least
// GEMM_FIX_MIN_STEPS k steps, and only while the partials fit the workspace.
// Measured over whole passes of the 0.5B model: the down projection at 16
// rows (28 workgroups, 76 k steps) runs 12.1 -> 9.5 us with 4 splits; at
// 512 rows splitting any of the four GEMMs makes it slower (the partials'
// round trip and the arrival sit on every workgroup's path), so only down,
// and only launches that leave most CUs idle, split.
#ifndef GEMM_FIX_KINDS
#define GEMM_FIX_KINDS (1 << kGemmDown)
#endif
#ifndef GEMM_FIX_TARGET
#define GEMM_FIX_TARGET 128
#endif
#ifndef GEMM_FIX_MIN_STEPS
#define GEMM_FIX_MIN_STEPS 2
#endif
// The GEMMs whose M blocks walk K from staggered starting steps (bit 1 << kind),
// from GEMM_KROT_MIN_M rows: the M blocks that share a weight tile, on one
// XCD, then read different k steps of it at any one time instead of the same
// lines together.  Measured over whole passes, alternated on one box: down at
// 512 rows of the 0.5B model 16.6 -> 15.4 us per launch (K = 4864, 16 M
// blocks per tile), at 256 rows (MXFP4) unchanged, at 128 rows of the 8B
// model (K = 14336, 4 M blocks) 36 -> 42 us; QKV, O, gate/up and the lm_head
// at 512 rows ran slower staggered.
#ifndef GEMM_KROT_KINDS
#define GEMM_KROT_KINDS (1 << kGemmDown)
#endif
#ifndef GEMM_KROT_MIN_M
#define GEMM_KROT_MIN_M 512
#endif
GemmPlan decoder_plan(int kind, int M, int tiles, int ksteps, const SplitWs *ws) {
  const Shape &s = kShapes[decoder_shape(kind, M)];
  GemmPlan p = gemm_plan(M, tiles / s.nt, ksteps, s.mt, false, s.ng);
  p.KS = s.ks;
  p.krot = ((GEMM_KROT_KINDS >> kind) & 1) && M >= GEMM_KROT_MIN_M;
  if (!ws || !ws->cnt || !((GEMM_FIX_KINDS >> kind) & 1)) return p;
  const int wgs = p.nb * p.mb;
  int S = (GEMM_FIX_TARGET + wgs - 1) / wgs;
  S = std::min(S, std::min(8, ksteps / (s.ks * GEMM_FIX_MIN_STEPS)));
  const size_t tile_floats = (size_t)s.ng * s.nt * s.mt * 1024;
  while (S > 1 && (size_t)S * wgs * tile_floats > ws->part_floats) --S;
  if (S <= 1 || wgs > ws->cnt_n) return p;
  p.spl = (ksteps + S - 1) / S;
  p.nsplit = (ksteps + p.spl - 1) / p.spl;  // every split non-empty
  p.fix = p.nsplit > 1;
  return p;
}

// ---------------------------------------------------------------- launchers

template <bool F16, int FMT, int NT, int MT, bool A8, class Epi, int NWV, int KS, int DEPTH, int NRL>
static hipError_t go_n(const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  constexpr int lds = GemmCfg<FMT, NT, MT, Epi, A8, NWV, KS, DEPTH>::LDS_BYTES;
  static_assert(lds <= 160 * 1024, "LDS of one workgroup");
  static const hipError_t attr =  // once per instantiation: allow more than 64 KB of LDS
      hipFuncSetAttribute((const void *)gemm_kernel<F16, FMT, NT, MT, Epi, A8, NWV, KS, DEPTH, NRL>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  launch_k((gemm_kernel<F16, FMT, NT, MT, Epi, A8, NWV, KS, DEPTH, NRL>), dim3(p.grid_x, 1, p.nsplit),
                     dim3(64 * NWV), lds, st, ga, epi);
  return hipGetLastError();
}

// the instantiation for the number of partial-sum loads the input rows need
// (only epilogues that scale by the input's normalisation take them)
template <bool F16, int FMT, int NT, int MT, bool A8, class Epi, int NWV = 4, int KS = 1, int DEPTH = 0>
static hipError_t go(const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  const int nrl = norm_loads(ga.nr, NWV);
  if (nrl == 0) return go_n<F16, FMT, NT, MT, A8, Epi, NWV, KS, DEPTH, 0>(p, ga, epi, st);
  if constexpr (Epi::kNormInput) {
    if (nrl == 1) return go_n<F16, FMT, NT, MT, A8, Epi, NWV, KS, DEPTH, 1>(p, ga, epi, st);
    if (nrl == 4) return go_n<F16, FMT, NT, MT, A8, Epi, NWV, KS, DEPTH, 4>(p, ga, epi, st);
  }
  return hipErrorInvalidValue;
}

template <bool F16, int FMT, int NT, bool A8, class Epi>
static hipError_t go_m(const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  switch (p.MT) {
    case 1: return go<F16, FMT, NT, 1, A8>(p, ga, epi, st);
    case 2: return go<F16, FMT, NT, 2, A8>(p, ga, epi, st);
    default:
      if constexpr (NT <= 2) return go<F16, FMT, NT, 4, A8>(p, ga, epi, st);
      else return go<F16, FMT, NT, 2, A8>(p, ga, epi, st);
  }
}

// one decoder shape, FP16 activations (shapes whose tiles per wave differ
// from the epilogue's are not instantiated)
template <int FMT, class Epi, int ID>
static hipError_t go_shape(const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  constexpr Shape s = kShapes[ID];
  if constexpr (s.nt == Epi::kNT)
    return go<true, FMT, s.nt, s.mt, false, Epi, s.nwv, s.ks, s.depth>(p, ga, epi, st);
  return hipErrorInvalidValue;
}
template <int FMT, class Epi>
static hipError_t go_decoder(int id, const GemmPlan &p, const GemmArgs &ga, const Epi &epi, hipStream_t st) {
  switch (id) {
    case kS412: return go_shape<FMT, Epi, kS412>(p, ga, epi, st);
    case kS222: return go_shape<FMT, Epi, kS222>(p, ga, epi, st);
    case kS411: return go_shape<FMT, Epi, kS411>(p, ga, epi, st);
    case kS221: return go_shape<FMT, Epi, kS221>(p, ga, epi, st);
    case kS141: return go_shape<FMT, Epi, kS141>(p, ga, epi, st);
    case kS241w8: return go_shape<FMT, Epi, kS241w8>(p, ga, epi, st);
    case kS812w8: return go_shape<FMT, Epi, kS812w8>(p, ga, epi, st);
    case kS181w8: return go_shape<FMT, Epi, kS181w8>(p, ga, epi, st);
    case kS4112: return go_shape<FMT, Epi, kS4112>(p, ga, epi, st);
  }
  return hipErrorInvalidValue;
}

// FMTS: bit (1 << format) set for each weight format a call site may pass;
// only those kernels are instantiated.
constexpr unsigned kFp8 = 1u << SPEC_WFMT_FP8_E4M3_ROW, kMx4 = 1u << SPEC_WFMT_MXFP4, kBf16 = 1u << SPEC_WFMT_BF16;

static GemmArgs gemm_args(ActIn x, int M, int K, const LinearW &w, const GemmPlan &p, NormRows nr,
                          const SplitWs *ws = nullptr) {
  const bool fix = p.fix && ws;
  return GemmArgs{x.x, x.xs, M, K, reinterpret_cast<const uint8_t *>(w.w), reinterpret_cast<const uint8_t *>(w.s),
                  p.nb, p.mb, p.grid_x / 8, p.spl, nr, fix ? ws->part : nullptr, fix ? ws->cnt : nullptr, p.krot ? 1 : 0};
}

// x.xs == NULL: FP16 (BF16 for BF16 weights) activations on the 32x32x16 MFMA;
// else MXFP8 activations on the scaled 32x32x64 MFMA (FP8 / MXFP4 weights).
// Four waves side by side along N, one k group.
template <int NT, unsigned FMTS, class Epi, int MAXMT = (NT > 2 ? 2 : 4)>
static hipError_t run(ActIn x, int M, int K, const LinearW &w, Epi epi, bool allow_split, NormRows nr,
                      hipStream_t st) {
  const GemmPlan p = gemm_plan(M, epi.units, K / 64, pick_mt(M, epi.units, MAXMT), allow_split, 4);
  const GemmArgs ga = gemm_args(x, M, K, w, p, nr);
  const bool a8 = x.xs != nullptr;
  if constexpr ((FMTS & kFp8) != 0)
    if (w.wfmt == SPEC_WFMT_FP8_E4M3_ROW)
      return a8 ? go_m<true, SPEC_WFMT_FP8_E4M3_ROW, NT, true>(p, ga, epi, st)
                : go_m<true, SPEC_WFMT_FP8_E4M3_ROW, NT, false>(p, ga, epi, st);
  if constexpr ((FMTS & kMx4) != 0)
    if (w.wfmt == SPEC_WFMT_MXFP4)
      return a8 ? go_m<true, SPEC_WFMT_MXFP4, NT, true>(p, ga, epi, st)
                : go_m<true, SPEC_WFMT_MXFP4, NT, false>(p, ga, epi, st);
  if constexpr ((FMTS & kBf16) != 0)
    if (w.wfmt == SPEC_WFMT_BF16 && !a8) return go_m<false, SPEC_WFMT_BF16, NT, false>(p, ga, epi, st);
  return hipErrorInvalidValue;
}

// FP16 activations, the workgroup shape decoder_shape() picks for the GEMM
template <unsigned FMTS, class Epi>
static hipError_t run_decoder(int kind, ActIn x, int M, int K, const LinearW &w, Epi epi, NormRows nr,
                              const SplitWs *ws, hipStream_t st) {
  if (x.xs) return hipErrorInvalidValue;
  const int id = decoder_shape(kind, M);
  if (kShapes[id].nt != Epi::kNT) return hipErrorInvalidValue;
  const GemmPlan p = decoder_plan(kind, M, epi.units * Epi::kNT, K / 64, ws);
  const GemmArgs ga = gemm_args(x, M, K, w, p, nr, ws);
  if constexpr ((FMTS & kFp8) != 0)
    if (w.wfmt == SPEC_WFMT_FP8_E4M3_ROW) return go_decoder<SPEC_WFMT_FP8_E4M3_ROW>(id, p, ga, epi, st);
  if constexpr ((FMTS & kMx4) != 0)
    if (w.wfmt == SPEC_WFMT_MXFP4) return go_decoder<SPEC_WFMT_MXFP4>(id, p, ga, epi, st);
  return hipErrorInvalidValue;
}

static const float *fp8_scale(const LinearW &w) {
  return w.wfmt == SPEC_WFMT_FP8_E4M3_ROW ? reinterpret_cast<const float *>(w.s) : nullptr;
}

hipError_t launch_linear_f32(ActIn x, int M, int N, int K, LinearW w, float *y, hipStream_t st) {
  return run<1, kFp8 | kMx4 | kBf16>(x, M, K, w, EpiF32<1>{N / 32, N, y, fp8_scale(w)}, false, NormRows{}, st);
}

hipError_t launch_residual_partial(ActIn x, int M, int N, int K, LinearW w, float *part, hipStream_t st) {
  return run<2, kFp8 | kMx4>(x, M, K, w, EpiPartial<2>{N / 64, N, M, part, fp8_scale(w)}, true, NormRows{}, st);
}

int residual_nsplit(int M, int N, int K) {
  const int units = N / 64;
  return gemm_plan(M, units, K / 64, pick_mt(M, units, 4), true, 4).nsplit;
}

hipError_t launch_residual(int kind, ActIn x, int M, int N, int K, LinearW w, const ResidualOut &o,
                           const SplitWs *ws, hipStream_t st) {
  return run_decoder<kFp8 | kMx4>(kind, x, M, K, w, EpiResidual<1>{N / 32, N, fp8_scale(w), o}, NormRows{}, ws, st);
}

hipError_t launch_swiglu(ActIn x, int M, int H, int I, LinearW w, void *a, uint8_t *a_scales, NormRows nr,
                         const SplitWs *ws, hipStream_t st) {
  if (a_scales)  // MXFP8 output: a unit of two tiles gives one 32-wide block per row
    return run<2, kFp8 | kMx4>(x, M, H, w, EpiSwiglu<2, true>{I / 32, I, fp8_scale(w), a, a_scales}, false, nr, st);
  if (kShapes[decoder_shape(kGemmGateUp, M)].nt == 2)
    return run_decoder<kFp8 | kMx4>(kGemmGateUp, x, M, H, w, EpiSwiglu<2>{I / 32, I, fp8_scale(w), a, nullptr}, nr,
                                    ws, st);
  return run_decoder<kFp8 | kMx4>(kGemmGateUp, x, M, H, w, EpiSwiglu<1>{I / 16, I, fp8_scale(w), a, nullptr}, nr,
                                  ws, st);
}

hipError_t launch_qkv(ActIn x, int M, int H, LinearW w, QkvOut o, NormRows nr, const SplitWs *ws, hipStream_t st) {
  if (w.wfmt != SPEC_WFMT_FP8_E4M3_ROW || (o.D != 64 && o.D != 128)) return hipErrorInvalidValue;
  const float *s = reinterpret_cast<const float *>(w.s);
  const int tiles = (o.Hq + 2 * o.Hkv) * o.D / 32;
  if (x.xs) return run<1, kFp8>(x, M, H, w, EpiQkv<1>{tiles, s, o}, false, nr, st);
  return run_decoder<kFp8>(kGemmQkv, x, M, H, w, EpiQkv<1>{tiles, s, o}, nr, ws, st);
}

void split_ws_need(int kind, int M, int tiles, int ksteps, size_t *floats, int *counters) {
  SplitWs any{nullptr, reinterpret_cast<int *>(1), ~(size_t)0, 1 << 30};  // sizes only, never dereferenced
  const GemmPlan p = decoder_plan(kind, M, tiles, ksteps, &any);
  const Shape &s = kShapes[decoder_shape(kind, M)];
  *floats = p.fix ? (size_t)p.nsplit * p.nb * p.mb * s.ng * s.nt * s.mt * 1024 : 0;
  *counters = p.fix ? p.nb * p.mb : 0;
}

hipError_t launch_lm_argmax(const uint16_t *x, int M, int V, int H, const uint16_t *table, ArgmaxPart *part,
                            float *logits_dump, NormRows nr, hipStream_t st) {
  return run<kLmNT, kBf16, EpiArgmax<kLmNT>, GEMM_LM_MAXMT>(
      ActIn{x, nullptr}, M, H, LinearW{table, nullptr, SPEC_WFMT_BF16},
      EpiArgmax<kLmNT>{V / (32 * kLmNT), V, lm_parts(V), part, logits_dump}, false, nr, st);
}
