// Block-causal GQA attention of the 16 block rows over the KV cache (gfx950).
//
// Row j of sequence b sits at position n_b + j and sees keys 0 .. n_b + j:
// the committed prefix plus the block rows up to itself, which the QKV step
// has already stored at slots n_b .. n_b+15 (HunyuanOCR-1.5 / DFlash write-up,
// inference loop, step 3: the whole block is verified in one forward).
// Query head h reads KV head h / G, so the G*16 query rows of one KV head
// share every K/V tile: the pass is bound by reading the cache once.
//
// Work unit = (key split, kv head, sequence): one workgroup of ceil(G/2)
// waves; wave w owns the 32 query rows of heads 2w, 2w+1 (rows of a head past
// G are padding and never stored).  The split's keys are walked in tiles of
// 64: the next tile's K/V is loaded into registers while the current one is
// computed, converted from the BF16 cache to FP16 and stored in LDS (K
// row-major, V transposed with swizzled columns; two LDS buffers, one barrier
// per tile).
//
// MFMA v_mfma_f32_32x32x16_f16.  Scores are computed transposed, S^T = K Q^T,
// 32 keys x 32 queries per block: lane (c, h) supplies key c (A) and query c
// (B) at the d slice (D/2)h + 8i of MFMA i (the same permutation of d on both
// sides), and ends with query c's scores for keys 8q + 4h + (0..3).  Softmax
// statistics therefore need one xor-32 shuffle, and the FP16 probabilities
// are already the B operand of O^T = V^T P^T, whose 16-key slices use the
// keys 16s + 4h + (0..3) and 16s + 8 + 4h + (0..3) of lane half h.  Online
// softmax in fp32, base 2, with a lazily moved reference: the reference only
// follows the running maximum when a tile exceeds it by more than 2^8, so
// most tiles skip the rescale of the accumulators.  Rows that have seen no
// visible key yet use 0 as their reference, so exp2(-inf) = 0 and nothing
// becomes NaN.
//
// Splits write unnormalised partials (m, l, o); a second kernel merges them
// in split order per (query head, sequence), so the result does not depend on
// timing and no workgroup waits on another (a device-wide fence inside the
// kernel would flush the XCD's L2).
#include "common.h"
#include "kernels.h"

#define KT 64  // keys per LDS tile
#define RESCALE 8.f  // log2 headroom of the lazily moved softmax reference
#ifndef ATTN_TEAMS
#define ATTN_TEAMS 2  // wave groups per workgroup splitting a split's key tiles
#endif
#ifndef ATTN_NR
#define ATTN_NR 2  // K/V tiles in flight in registers
#endif

// V^T tile in LDS: key k of row d sits at column k ^ vsw(d).  The XOR moves
// whole 4-key groups (so key pairs and the 4-key pieces the MFMA reads stay
// contiguous) and makes the transposing stores free of bank conflicts (the
// operand reads stay at the 2-way minimum of 8-byte accesses).
__device__ __forceinline__ int vsw(int d) { return 4 * ((d ^ (d >> 2)) & 15); }

// LDS of one team: two K tiles and two V^T tiles (16-bit elements)
template <int D>
constexpr int attn_team_halfs() { return 2 * KT * (D + 8) + 2 * D * KT; }

template <int D, int NW, int NTEAM, int NR = ATTN_NR>  // NW = waves per team = ceil(G/2)
__global__ __launch_bounds__(64 * NW * NTEAM) void attn_kernel(AttnArgs a, float scale_log2) {
  constexpr int DS = D / 16;           // S MFMAs per 32-key block (k = 16 each)
  constexpr int DT = D / 32;           // 32-wide d tiles of O^T
  constexpr int KP = D + 8;            // K row pitch (16-bit elements): rows land on distinct bank groups
  constexpr int VP = KT;               // V^T row pitch (16-bit elements); columns swizzled by vsw()
  constexpr int KCH = KT * D / 8;      // K: 16-byte chunks (one key, 8 d) per tile
  constexpr int VCH = KT * D / 8;      // V: chunks of (2 keys, 4 d)
  extern __shared__ __align__(16) uint16_t attn_lds[];  // NTEAM x attn_team_halfs<D>()

  const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int n = a.kv_len[b];
  const int L = min(max(n, 0) + 16, a.max_ctx);
  const int nsplit = (L + a.split_len - 1) / a.split_len;
  if (sp >= nsplit) return;  // whole workgroup
  const int key_lo = sp * a.split_len, key_hi = min(key_lo + a.split_len, L);

  constexpr int T = 64 * NW;  // threads per team
  // Teams: NTEAM groups of NW waves walk alternate key tiles of the split
  // (tile i of the split goes to team i % NTEAM), each with its own LDS tiles,
  // and combine their softmax states through LDS at the end, so the split
  // still leaves one partial.  tid, lane and wave below are team-local.
  const int team = threadIdx.x / T, tid = threadIdx.x % T, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int wave = tid >> 6;
  uint16_t *const Ks = attn_lds + team * attn_team_halfs<D>();  // [2][KT * KP]
  uint16_t *const Vt = Ks + 2 * KT * KP;                         // [2][D * VP]
  const size_t unit = (size_t)b * a.Hkv + kvh;

  // this wave's queries: lane (c, h) -> head 2*wave + c/16 of the group, block row c%16
  const int hg = 2 * wave + (c >> 4), j = c & 15;
  const bool qvalid = hg < G;
  u32x4_t qf[DS];
  {
    const uint16_t *qp = a.q + (size_t)(b * 16 + j) * (a.Hq * D) + (kvh * G + (qvalid ? hg : 0)) * D + (D / 2) * h;
#pragma unroll
    for (int i = 0; i < DS; ++i)
      qf[i] = qvalid ? *reinterpret_cast<const u32x4_t *>(qp + 8 * i) : u32x4_t{0, 0, 0, 0};
  }
  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  // Tile loads are unconditional (key indices clamped to the split's last key,
  // whose finite values are masked out) so the wave never branches around them.
  // A tile's 64 keys share one cache page (pages hold a multiple of 64 rows), so
  // one row lookup per tile serves both layouts; tb = 64-aligned start of the
  // tile that holds the (clamped) keys.
  constexpr int KPT = (KCH + T - 1) / T, VPT = (VCH + T - 1) / T;  // chunks per thread (last one partial for NW = 3)
  struct TileRegs {
    u32x4_t k[KPT];
    u32x2_t v[VPT][2];
  };
  auto load_tile = [&](TileRegs &tr, int kt0) {
    const int tb = min(kt0, (key_hi - 1) & ~(KT - 1));
    bool ok;
    const size_t trow = a.kvl.row(b, kvh, a.Hkv, a.max_ctx, tb, ok);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ch = min(tid + T * i, KCH - 1), kk = ch / (D / 8), d0 = (ch % (D / 8)) * 8,
                key = min(kt0 + kk, key_hi - 1);
      tr.k[i] = *reinterpret_cast<const u32x4_t *>(a.k_cache + (trow + key - tb) * D + d0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int ch = min(tid + T * i, VCH - 1), kk = 2 * (ch / (D / 4)), d0 = (ch % (D / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = min(kt0 + kk + e, key_hi - 1);
        tr.v[i][e] = *reinterpret_cast<const u32x2_t *>(a.v_cache + (trow + key - tb) * D + d0);
      }
    }
  };
  auto store_tile = [&](const TileRegs &tr, int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ch = tid + T * i, kk = ch / (D / 8), d0 = (ch % (D / 8)) * 8;
      if (KCH % T != 0 && ch >= KCH) break;  // NW = 3: the last round is partial
      const u32x4_t v = tr.k[i];
      *reinterpret_cast<u32x4_t *>(Ks + buf * KT * KP + kk * KP + d0) =
          u32x4_t{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int ch = tid + T * i, kk = 2 * (ch / (D / 4)), d0 = (ch % (D / 4)) * 4;
      if (VCH % T != 0 && ch >= VCH) break;
      const uint32_t a0 = bf16x2_to_f16x2(tr.v[i][0].x), a1 = bf16x2_to_f16x2(tr.v[i][0].y);
      const uint32_t b0 = bf16x2_to_f16x2(tr.v[i][1].x), b1 = bf16x2_to_f16x2(tr.v[i][1].y);
      // (key kk, key kk+1) pairs for d0 .. d0+3
      uint16_t *vt = Vt + buf * D * VP;
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 0) * VP + (kk ^ vsw(d0 + 0))]) = (a0 & 0xffff) | (b0 << 16);
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 1) * VP + (kk ^ vsw(d0 + 1))]) = (a0 >> 16) | (b0 & 0xffff0000u);
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 2) * VP + (kk ^ vsw(d0 + 2))]) = (a1 & 0xffff) | (b1 << 16);
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 3) * VP + (kk ^ vsw(d0 + 3))]) = (a1 >> 16) | (b1 & 0xffff0000u);
    }
  };

  auto compute = [&](int kt0, int buf) {
    const uint16_t *ks = Ks + buf * KT * KP;
    const uint16_t *vt = Vt + buf * D * VP;
    // S^T for the tile's two 32-key blocks
    f32x16_t st[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[blk][v] = 0.f;
      const uint16_t *krow = ks + (32 * blk + c) * KP + (D / 2) * h;
#pragma unroll
      for (int i = 0; i < DS; ++i)
        st[blk] = mfma32x32x16_f16(*reinterpret_cast<const u32x4_t *>(krow + 8 * i), qf[i], st[blk]);
    }
    if (!(kt0 + KT <= n && kt0 + KT <= key_hi)) {  // the tile reaches past the committed prefix: mask
      const int last_visible = min(n + j, key_hi - 1);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt0 + 32 * blk + 8 * (v >> 2) + 4 * h + (v & 3);
          st[blk][v] = key <= last_visible ? st[blk][v] : -INFINITY;
        }
    }
    // tile maximum of the raw scores (a tree, not a 32-deep chain), both lane halves
    float t[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] = fmaxf(st[0][v], st[1][v]);
#pragma unroll
    for (int w = 8; w > 0; w >>= 1)
#pragma unroll
      for (int v = 0; v < w; ++v) t[v] = fmaxf(t[v], t[v + w]);
    const float tm = halves_max(t[0]) * scale_log2;
    // Lazy rescaling: the reference maximum mrow only moves when a tile's
    // maximum exceeds it by more than 2^RESCALE, so the probabilities stay
    // <= 2^RESCALE (exact in FP16's range) and the accumulators are rescaled
    // only on those rare tiles (a wave-uniform branch).
    const bool need = tm > mrow + RESCALE;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mnew = need ? tm : mrow;
      const float alpha = need ? __builtin_amdgcn_exp2f(mrow - mnew) : 1.f;  // mrow = -inf gives 0
      lrow *= alpha;
      mrow = mnew;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    const float mref = mrow == -INFINITY ? 0.f : mrow;  // a row with no visible key yet: every p is 0
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 16; ++v) st[blk][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[blk][v], scale_log2, -mref));
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] = st[0][v] + st[1][v];
#pragma unroll
    for (int w = 8; w > 0; w >>= 1)
#pragma unroll
      for (int v = 0; v < w; ++v) t[v] += t[v + w];
    lrow += halves_sum(t[0]);
    // O^T += V^T P^T over 4 slices of 16 keys
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int blk = sl >> 1, q0 = 2 * (sl & 1);
      const u32x4_t pb = u32x4_t{pack_f16x2(st[blk][4 * q0 + 0], st[blk][4 * q0 + 1]),
                                 pack_f16x2(st[blk][4 * q0 + 2], st[blk][4 * q0 + 3]),
                                 pack_f16x2(st[blk][4 * q0 + 4], st[blk][4 * q0 + 5]),
                                 pack_f16x2(st[blk][4 * q0 + 6], st[blk][4 * q0 + 7])};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + c, sw = vsw(d);
        const uint16_t *vrow = vt + d * VP;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow + ((16 * sl + 4 * h) ^ sw));
        const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + ((16 * sl + 8 + 4 * h) ^ sw));
        oacc[dt] = mfma32x32x16_f16(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb, oacc[dt]);
      }
    }
  };

  // Tile t is computed from LDS buffer t&1 while tiles t+1 .. t+NR are in
  // flight in NR register sets (the loop is unrolled by NR so every set has a
  // fixed name).  The barrier at each step makes tile t visible and frees
  // buffer (t+1)&1.  Loads and stores past the split end are unconditional
  // (clamped keys into a buffer nobody reads) so the body does not branch.
  auto tile_key = [&](int ti) { return key_lo + (ti * NTEAM + team) * KT; };  // the team's ti-th tile
  const int ntiles = (key_hi - key_lo + KT - 1) / KT, nteam = (ntiles + NTEAM - 1) / NTEAM;  // same for every team
  TileRegs rr[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) load_tile(rr[i], tile_key(i));
  store_tile(rr[0], 0);
  load_tile(rr[0], tile_key(NR));
  for (int ti0 = 0; ti0 < nteam; ti0 += NR) {
#pragma unroll
    for (int ph = 0; ph < NR; ++ph) {
      const int ti = ti0 + ph, par = ti & 1, t0 = tile_key(ti);
      lds_barrier();
      store_tile(rr[(ph + 1) % NR], par ^ 1);
      load_tile(rr[(ph + 1) % NR], tile_key(ti + NR + 1));
      if (t0 < key_hi) compute(t0, par);
    }
  }
  if constexpr (NTEAM > 1) {
    // teams 1.. leave (m, l, o) in their own LDS (lane-contiguous, same lane
    // layout as team 0's registers); team 0 folds them in team order
    constexpr int NV = DT * 16 + 2;
    static_assert(NV * NW * 64 * 4 <= attn_team_halfs<D>() * 2, "team state fits the team's LDS");
    lds_barrier();  // every team is done with its tiles
    float *mine = reinterpret_cast<float *>(Ks) + wave * NV * 64 + lane;
    if (team > 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[(dt * 16 + v) * 64] = oacc[dt][v];
      mine[DT * 16 * 64] = mrow;
      mine[(DT * 16 + 1) * 64] = lrow;
    }
    lds_barrier();
    if (team > 0) return;
#pragma unroll
    for (int tm = 1; tm < NTEAM; ++tm) {
      const float *o = reinterpret_cast<const float *>(attn_lds + tm * attn_team_halfs<D>()) + wave * NV * 64 + lane;
      const float m1 = o[DT * 16 * 64], l1 = o[(DT * 16 + 1) * 64];
      const float mx = fmaxf(mrow, m1);
      if (mx == -INFINITY) continue;  // neither team saw a visible key of this row
      const float a0 = __builtin_amdgcn_exp2f(mrow - mx), a1 = __builtin_amdgcn_exp2f(m1 - mx);  // -inf gives 0
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] = oacc[dt][v] * a0 + o[(dt * 16 + v) * 64] * a1;
      lrow = lrow * a0 + l1 * a1;
      mrow = mx;
    }
  }

  // partials: group row R = head*16 + j = 32*wave + c; lane (c, h) holds d = 32dt + 8q + 4h + (0..3)
  if (qvalid) {
    const int R = G * 16, row = 32 * wave + c;
    float *po = a.part_o + ((unit * a.nsplit + sp) * R + row) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t *>(po + 32 * dt + 8 * q + 4 * h) =
            f32x4_t{oacc[dt][4 * q], oacc[dt][4 * q + 1], oacc[dt][4 * q + 2], oacc[dt][4 * q + 3]};
    if (h == 0) a.part_ml[(unit * a.nsplit + sp) * R + row] = make_float2(mrow, lrow);
  }
}

// o[b*16+j][hq*D + d] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the
// splits of sequence b, in split order.  One workgroup per (query head, seq):
// the split statistics are loaded in parallel into LDS, each row's weights
// w_s = 2^(m_s - M) / den are formed once, then every thread sums its 4
// columns over the splits with independent loads.  A split that saw no key of
// a row has m_s = -inf and weight 0 (its partial is 0, never NaN).
#define MAX_SPLITS 64
#ifndef ATTN_WG_TARGET
#define ATTN_WG_TARGET 256
#endif

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  __shared__ float2 sML[MAX_SPLITS][16];
  __shared__ float sW[MAX_SPLITS][16];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = a.Hq / a.Hkv, kvh = hq / G, tq = hq % G, R = G * 16;
  const int n = a.kv_len[b];
  const int L = min(max(n, 0) + 16, a.max_ctx);
  const int nsplit = (L + a.split_len - 1) / a.split_len;
  const size_t unit = (size_t)b * a.Hkv + kvh;
  const float *po0 = a.part_o + (unit * a.nsplit) * R * D;
  const float2 *pml0 = a.part_ml + (unit * a.nsplit) * R;
  for (int i = tid; i < nsplit * 16; i += 256) sML[i >> 4][i & 15] = pml0[(i >> 4) * R + tq * 16 + (i & 15)];
  __syncthreads();
  if (tid < 16) {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, sML[s][tid].x);
    float den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float2 ml = sML[s][tid];
      const float e = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
      sW[s][tid] = e;
      den += e * ml.y;
    }
    const float inv = 1.f / den;
    for (int s = 0; s < nsplit; ++s) sW[s][tid] *= inv;
  }
  __syncthreads();
  for (int idx = tid; idx < 16 * D / 4; idx += 256) {
    const int j = idx / (D / 4), d = (idx % (D / 4)) * 4, row = tq * 16 + j;
    const float *p = po0 + (size_t)row * D + d;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) acc += sW[s][j] * *reinterpret_cast<const f32x4_t *>(p + (size_t)s * R * D);
    *reinterpret_cast<u32x2_t *>(a.o + (size_t)(b * 16 + j) * (a.Hq * D) + hq * D + d) =
        u32x2_t{pack_f16x2(acc[0], acc[1]), pack_f16x2(acc[2], acc[3])};
  }
}

// teams per workgroup: two for head_dim 64; one for 128, whose per-wave state
// would not fit the registers of a second team without spilling
static int attn_teams(int D) { return D == 64 ? ATTN_TEAMS : 1; }

int attention_split_len(int batch, int Hkv, int max_ctx, int D) {
  // Aim for about ATTN_WG_TARGET workgroups (with full contexts) across the
  // batch when two teams share a split, 768 with one; measured on the
  // 32-sequence 0.5B workload, fewer and longer splits win once a workgroup
  // holds two teams.  Splits are whole 64-key tiles and a sequence has at
  // most MAX_SPLITS of them.
  const long target = attn_teams(D) > 1 ? ATTN_WG_TARGET : 768;
  long sl = ((long)batch * Hkv * max_ctx + target - 1) / target;
  const long min_sl = (max_ctx + MAX_SPLITS - 1) / MAX_SPLITS;
  if (sl < min_sl) sl = min_sl;
  sl = ((sl + KT - 1) / KT) * KT;
  if (sl < KT) sl = KT;
  return (int)sl;
}

template <int D, int NW, int NTEAM>
static hipError_t go_attn(const AttnArgs &a, dim3 grid, float sc, hipStream_t st) {
  const int lds = NTEAM * attn_team_halfs<D>() * 2;
  static const hipError_t attr =  // once per instantiation: allow more than 64 KB of LDS
      hipFuncSetAttribute((const void *)attn_kernel<D, NW, NTEAM>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_kernel<D, NW, NTEAM>), grid, dim3(64 * NW * NTEAM), lds, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_attention_splits(const AttnArgs &a, int D, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  if (G < 1 || G > 8) return hipErrorInvalidValue;
  const int nw = (G + 1) / 2;
  const dim3 grid(a.nsplit, a.Hkv, a.batch);
  if (D == 64) {
    const float sc = (float)(1.4426950408889634 / 8.0);
    switch (nw) {
      case 1: return go_attn<64, 1, ATTN_TEAMS>(a, grid, sc, st);
      case 2: return go_attn<64, 2, ATTN_TEAMS>(a, grid, sc, st);
      case 3: return go_attn<64, 3, ATTN_TEAMS>(a, grid, sc, st);
      default: return go_attn<64, 4, ATTN_TEAMS>(a, grid, sc, st);
    }
  } else if (D == 128) {
    const float sc = (float)(1.4426950408889634 / 11.313708498984761);
    switch (nw) {
      case 1: return go_attn<128, 1, 1>(a, grid, sc, st);
      case 2: return go_attn<128, 2, 1>(a, grid, sc, st);
      case 3: return go_attn<128, 3, 1>(a, grid, sc, st);
      default: return go_attn<128, 4, 1>(a, grid, sc, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_merge(const AttnArgs &a, int D, hipStream_t st) {
  if (D == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(a.Hq, a.batch), dim3(256), 0, st, a);
  else if (D == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(a.Hq, a.batch), dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int D, hipStream_t st) {
  const hipError_t e = launch_attention_splits(a, D, st);
  return e != hipSuccess ? e : launch_attention_merge(a, D, st);
}
