// Block-causal GQA attention of the 16 block rows over the KV cache (gfx950).
//
// Row j of sequence b sits at position n_b + j and sees keys 0 .. n_b + j:
// the committed prefix plus the block rows up to itself, which the QKV step
// has already stored at slots n_b .. n_b+15 (HunyuanOCR-1.5 / DFlash write-up,
// inference loop, step 3: the whole block is verified in one forward).
// Query head h reads KV head h / G, so the G*16 query rows of one KV head
// share every K/V tile: the pass is bound by reading the cache once.
//
// Work unit = (key split, kv head, sequence), taken from the pass's split
// plan (attn_plan.h: equal splits sized from the actual cache lengths so that
// one resident round of workgroups covers every key); one team of ceil(G/2)
// waves per key tile; wave w owns the 32 query rows of heads 2w, 2w+1 (rows
// of a head past G are padding and never stored).  The split's keys are
// walked in tiles of 64: the next tile's K/V is loaded into registers while
// the current one is computed, converted from the BF16 cache to FP16 and
// stored in LDS (K row-major, V transposed with swizzled columns; two LDS
// buffers, one barrier per tile).
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
#include "attn_plan.h"
#include "common.h"
#include "kernels.h"

// Work-item and workgroup ids as intrinsics: this file is built without IEEE
// mode, and the device library's id functions, built with it, are then not
// inlined (each kernel would call them, and the workgroup id would come back
// in a vector register).
__device__ __forceinline__ int wg_x() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int wg_y() { return __builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int wi_x() { return __builtin_amdgcn_workitem_id_x(); }

#define KT 64  // keys per LDS tile
#define RESCALE 8.f  // log2 headroom of the lazily moved softmax reference
#ifndef ATTN_TEAMS
#define ATTN_TEAMS 2  // wave groups per workgroup splitting a split's key tiles
#endif
#ifndef ATTN_NR
#define ATTN_NR 2  // K/V tiles in flight in registers (head_dim 64)
#endif
#ifndef ATTN_NR128
#define ATTN_NR128 2  // the same for head_dim 128 with two or more waves per team
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

  // Workgroup w takes slot w of the pass's split plan: find its sequence b
  // (entries hold increasing first slots), KV head and split.
  pin_args(a, scale_log2);
  const int w = wg_x(), ln = wi_x() & 63;
  // the header and the first 64 sequences' entries go out together and are
  // waited for once (the compiler would otherwise order three round trips:
  // header, then the entries' first slots, then the rest)
  const int4 hdr = a.plan[0];
  int4 e = a.plan[1 + min(ln, a.batch - 1)];
  asm volatile("" ::"v"(hdr.x), "v"(hdr.y), "v"(e.x), "v"(e.y), "v"(e.z));
  if (w >= hdr.y) return;  // whole workgroup: past the plan's splits
  int b = 0, first = 0, nsp = 1, n = 0;
  {
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      if (b0 > 0) e = a.plan[1 + min(b0 + ln, a.batch - 1)];
      const int k = __popcll(__builtin_amdgcn_ballot_w64(b0 + ln < a.batch && e.x <= w));
      if (k > 0) {
        b = b0 + k - 1;
        first = __builtin_amdgcn_readlane(e.x, k - 1);
        nsp = __builtin_amdgcn_readlane(e.y, k - 1);
        n = __builtin_amdgcn_readlane(e.z, k - 1);
      }
      if (k < 64) break;
    }
  }
  const int kvh = (w - first) / nsp, sp = (w - first) - kvh * nsp;
  const int G = a.Hq / a.Hkv;
  const int L = min(max(n, 0) + 16, a.max_ctx), split_len = hdr.x * KT;
  const int key_lo = sp * split_len, key_hi = min(key_lo + split_len, L);

  constexpr int T = 64 * NW;  // threads per team
  // Teams: NTEAM groups of NW waves walk alternate key tiles of the split
  // (tile i of the split goes to team i % NTEAM), each with its own LDS tiles,
  // and combine their softmax states through LDS at the end, so the split
  // still leaves one partial.  tid, lane and wave below are team-local.
  const int team = __builtin_amdgcn_readfirstlane(wi_x() / T);
  const int tid = wi_x() % T, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t *const Ks = attn_lds + team * attn_team_halfs<D>();  // [2][KT * KP]
  uint16_t *const Vt = Ks + 2 * KT * KP;                         // [2][D * VP]

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
  // tile that holds the (clamped) keys.  A thread's chunks sit at fixed byte
  // offsets inside a tile (rows of 2D bytes), so a whole tile is loaded from
  // one scalar base with no per-load address arithmetic; only a tile that
  // reaches past the split clamps its rows.
  constexpr int KPT = (KCH + T - 1) / T, VPT = (VCH + T - 1) / T;  // chunks per thread (last one partial for NW = 3)
  struct TileRegs {
    u32x4_t k[KPT];
    u32x2_t v[VPT][2];
  };
  int kk_k[KPT], kk_v[VPT];            // tile row of each chunk (V: the first of its two keys)
  uint32_t dk[KPT], dv[VPT];           // byte offset of its d slice inside a row
  uint32_t ok[KPT], ov[VPT][2];        // byte offset of the chunk inside a whole tile
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int ch = min(tid + T * i, KCH - 1);
    kk_k[i] = ch / (D / 8);
    dk[i] = (ch % (D / 8)) * 16;
    ok[i] = kk_k[i] * 2 * D + dk[i];
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int ch = min(tid + T * i, VCH - 1);
    kk_v[i] = 2 * (ch / (D / 4));
    dv[i] = (ch % (D / 4)) * 8;
#pragma unroll
    for (int e = 0; e < 2; ++e) ov[i][e] = (kk_v[i] + e) * 2 * D + dv[i];
  }
  // scalar tile base + a 32-bit per-lane offset: the loads take the
  // SGPR-base form, with no 64-bit address arithmetic per load
  auto load_tile = [&](TileRegs &tr, int kt0) {
    const int tb = min(kt0, (key_hi - 1) & ~(KT - 1));
    bool okp;
    const size_t trow = a.kvl.row(b, kvh, a.Hkv, a.max_ctx, tb, okp);
    const char *kb = reinterpret_cast<const char *>(a.k_cache + trow * D);
    const char *vb = reinterpret_cast<const char *>(a.v_cache + trow * D);
    const int off = kt0 - tb, lim = key_hi - 1 - tb;  // row of key kt0 + kk is min(kk + off, lim)
    if (off == 0 && lim >= KT - 1) {  // the whole tile lies inside the split
#pragma unroll
      for (int i = 0; i < KPT; ++i) tr.k[i] = *reinterpret_cast<const u32x4_t *>(kb + ok[i]);
#pragma unroll
      for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) tr.v[i][e] = *reinterpret_cast<const u32x2_t *>(vb + ov[i][e]);
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        tr.k[i] = *reinterpret_cast<const u32x4_t *>(kb + (uint32_t)(min(kk_k[i] + off, lim) * 2 * D + dk[i]));
#pragma unroll
      for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          tr.v[i][e] =
              *reinterpret_cast<const u32x2_t *>(vb + (uint32_t)(min(kk_v[i] + e + off, lim) * 2 * D + dv[i]));
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
      // (key kk, key kk+1) pairs of column d0 + e, converted straight into
      // their FP16 pair: the low bf16 of a dword is column d0 + 2i, the high
      // one d0 + 2i + 1
      const u32x2_t x = tr.v[i][0], y = tr.v[i][1];
      uint16_t *vt = Vt + buf * D * VP;
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 0) * VP + (kk ^ vsw(d0 + 0))]) =
          pack_f16x2(__uint_as_float(x.x << 16), __uint_as_float(y.x << 16));
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 1) * VP + (kk ^ vsw(d0 + 1))]) =
          pack_f16x2(__uint_as_float(x.x & 0xffff0000u), __uint_as_float(y.x & 0xffff0000u));
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 2) * VP + (kk ^ vsw(d0 + 2))]) =
          pack_f16x2(__uint_as_float(x.y << 16), __uint_as_float(y.y << 16));
      *reinterpret_cast<uint32_t *>(&vt[(d0 + 3) * VP + (kk ^ vsw(d0 + 3))]) =
          pack_f16x2(__uint_as_float(x.y & 0xffff0000u), __uint_as_float(y.y & 0xffff0000u));
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
    // tile maximum of the raw scores (a tree, not a 32-deep chain), both lane
    // halves.  The file is built without NaN semantics and with the IEEE mode
    // bit off, so fmaxf is one v_max (or a third of a v_max3) per value
    // instead of first quieting every MFMA result.
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
    // row sum (a tree), then the FP16 probabilities, already in the B operand
    // layout of the 4 key slices
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] = st[0][v] + st[1][v];
#pragma unroll
    for (int w = 8; w > 0; w >>= 1)
#pragma unroll
      for (int v = 0; v < w; ++v) t[v] += t[v + w];
    lrow += halves_sum(t[0]);
    u32x4_t pb[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int blk = sl >> 1, q0 = 2 * (sl & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[sl][i] = pack_f16x2(st[blk][4 * q0 + 2 * i], st[blk][4 * q0 + 2 * i + 1]);
    }
    // O^T += V^T P^T over 4 slices of 16 keys
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + c, sw = vsw(d);
        const uint16_t *vrow = vt + d * VP;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow + ((16 * sl + 4 * h) ^ sw));
        const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + ((16 * sl + 8 + 4 * h) ^ sw));
        oacc[dt] = mfma32x32x16_f16(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb[sl], oacc[dt]);
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
      if (ti >= nteam) break;  // every team runs the same nteam steps
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

  // partials: group row R = head*16 + j = 32*wave + c; lane (c, h) holds d =
  // 32dt + 8q + 4h + (0..3).  The split's output is stored normalised, o / l
  // in FP16 (a convex combination of V rows, so within V's FP16 range), with
  // (m, l) in fp32: half the bytes of fp32 o, whose stores and re-reads by the
  // merge cost more than the rounding (2^-12 relative) that the merge then
  // averages.  A row that saw no key of this split stores 0 and l = 0.
  if (qvalid) {
    const int R = G * 16, row = 32 * wave + c;
    uint16_t *po = a.part_o + ((size_t)w * R + row) * D;
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2_t *>(po + 32 * dt + 8 * q + 4 * h) =
            u32x2_t{pack_f16x2(oacc[dt][4 * q] * inv, oacc[dt][4 * q + 1] * inv),
                    pack_f16x2(oacc[dt][4 * q + 2] * inv, oacc[dt][4 * q + 3] * inv)};
    if (h == 0) a.part_ml[(size_t)w * R + row] = make_float2(mrow, lrow);
  }
}

// o[b*16+j][hq*D + d] = sum_s 2^(m_s - M) l_s (o_s / l_s) / sum_s 2^(m_s - M) l_s
// over the splits of sequence b, in split order (o_s / l_s as stored, FP16).  One workgroup per (query head, seq);
// each thread owns 4 columns of one row and walks the splits in chunks of 8,
// issuing a chunk's (m, l) and o loads together (one memory round trip per
// chunk; every split of the batch-32 workload fits one chunk), and keeps a
// running maximum, rescaling its sums when a chunk raises it.  A split that
// saw no key of a row has m_s = -inf and weight 0 (its partial is 0).
#define MERGE_CHUNK 8

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  pin_args(a);
  const int hq = wg_x(), b = wg_y(), tid = wi_x();
  const int G = a.Hq / a.Hkv, kvh = hq / G, tq = hq % G, R = G * 16;
  // the plan entry is uniform: a scalar load (the plan does not change during
  // the kernel, and the scalar cache is invalidated at each launch), one
  // shorter round trip before the partials' loads
  const __attribute__((address_space(4))) int32_t *e = (const __attribute__((address_space(4))) int32_t *)(a.plan + 1 + b);
  const int nsplit = e[1];
  const size_t slot0 = (size_t)e[0] + (size_t)kvh * nsplit;  // the unit's splits, in key order
  const uint16_t *po0 = a.part_o + slot0 * R * D;
  const float2 *pml0 = a.part_ml + slot0 * R;
#pragma unroll
  for (int idx = tid; idx < 16 * D / 4; idx += 256) {
    const int j = idx / (D / 4), d = (idx % (D / 4)) * 4, row = tq * 16 + j;
    const uint16_t *p = po0 + (size_t)row * D + d;
    float mx = -INFINITY, den = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += MERGE_CHUNK) {
      float2 ml[MERGE_CHUNK];
      f32x4_t o[MERGE_CHUNK];
#pragma unroll
      for (int k = 0; k < MERGE_CHUNK; ++k) {
        const bool in = s0 + k < nsplit;
        ml[k] = in ? pml0[(size_t)(s0 + k) * R + row] : make_float2(-INFINITY, 0.f);
        const u32x2_t ob = in ? *reinterpret_cast<const u32x2_t *>(p + (size_t)(s0 + k) * R * D) : u32x2_t{0u, 0u};
        o[k] = f32x4_t{f16_to_f32(ob.x & 0xffff), f16_to_f32(ob.x >> 16), f16_to_f32(ob.y & 0xffff),
                       f16_to_f32(ob.y >> 16)};
      }
      float cm = mx;
#pragma unroll
      for (int k = 0; k < MERGE_CHUNK; ++k) cm = fmaxf(cm, ml[k].x);
      if (cm == -INFINITY) continue;  // no split so far saw a key of this row
      const float sc = mx == -INFINITY ? 0.f : exp2f(mx - cm);
      acc *= sc;
      den *= sc;
#pragma unroll
      for (int k = 0; k < MERGE_CHUNK; ++k) {
        const float w = ml[k].x == -INFINITY ? 0.f : exp2f(ml[k].x - cm) * ml[k].y;
        acc += w * o[k];
        den += w;
      }
      mx = cm;
    }
    const float inv = 1.f / den;
    *reinterpret_cast<u32x2_t *>(a.o + (size_t)(b * 16 + j) * (a.Hq * D) + hq * D + d) =
        u32x2_t{pack_f16x2(acc[0] * inv, acc[1] * inv), pack_f16x2(acc[2] * inv, acc[3] * inv)};
  }
}

// teams per workgroup: two for head_dim 64; one for 128, whose per-wave state
// would not fit the registers of a second team without spilling
static int attn_teams(int D) { return D == 64 ? ATTN_TEAMS : 1; }

// compute units of the current device (cached per device)
int attention_device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    cached[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cached[dev];
}

// Workgroups of one attention instantiation that fit on a CU at once
// (registers, LDS including the dynamic part, waves), from the runtime's
// occupancy query; once per instantiation.
template <int D, int NW, int NTEAM, int NR = ATTN_NR>
static int attn_resident_of() {
  static const int n = [] {
    const int lds = NTEAM * attn_team_halfs<D>() * 2;
    const void *f = (const void *)attn_kernel<D, NW, NTEAM, NR>;
    int r = 0;
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, f, 64 * NW * NTEAM, lds) != hipSuccess || r < 1)
      r = 1;
    return r;
  }();
  return n;
}

// the instantiation launch_attention_splits runs for (D, G)
static int attn_resident(int D, int G) {
  const int nw = (G + 1) / 2;
  if (D == 64) {
    switch (nw) {
      case 1: return attn_resident_of<64, 1, ATTN_TEAMS>();
      case 2: return attn_resident_of<64, 2, ATTN_TEAMS>();
      case 3: return attn_resident_of<64, 3, ATTN_TEAMS>();
      default: return attn_resident_of<64, 4, ATTN_TEAMS>();
    }
  }
  switch (nw) {
    case 1: return attn_resident_of<128, 1, 1, 1>();
    case 2: return attn_resident_of<128, 2, 1, ATTN_NR128>();
    case 3: return attn_resident_of<128, 3, 1, ATTN_NR128>();
    default: return attn_resident_of<128, 4, 1, ATTN_NR128>();
  }
}

int attention_grid(int batch, int Hq, int Hkv, int max_ctx, int D, int split_len, int cus) {
  const int units = batch * Hkv;
  if (split_len > 0) {  // at most ceil(ceil(max_ctx / 64) / t) splits per unit
    const int t = split_len / KT, tiles = (max_ctx + KT - 1) / KT;
    return units * ((tiles + t - 1) / t);
  }
  // One resident round of workgroups; every unit needs at least one.
  const int resident = (cus > 0 ? cus : 256) * attn_resident(D, Hq / Hkv);
  return units > resident ? units : resident;
}

AttnPlanArgs attention_plan_args(int4 *plan, int batch, int Hq, int Hkv, int max_ctx, int D, int split_len, int cus) {
  return AttnPlanArgs{plan, batch, Hkv, max_ctx, attention_grid(batch, Hq, Hkv, max_ctx, D, split_len, cus), attn_teams(D),
                      split_len > 0 ? split_len / KT : 0};
}

__global__ __launch_bounds__(64) void attn_plan_kernel(const int32_t *__restrict__ kv_len, AttnPlanArgs p) {
  attn_plan_wave(kv_len, p, wi_x());
}

hipError_t launch_attention_plan(const int32_t *kv_len, const AttnPlanArgs &p, hipStream_t st) {
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(64), 0, st, kv_len, p);
  return hipGetLastError();
}

template <int D, int NW, int NTEAM, int NR = ATTN_NR>
static hipError_t go_attn(const AttnArgs &a, dim3 grid, float sc, hipStream_t st) {
  const int lds = NTEAM * attn_team_halfs<D>() * 2;
  static const hipError_t attr =  // once per instantiation: allow more than 64 KB of LDS
      hipFuncSetAttribute((const void *)attn_kernel<D, NW, NTEAM, NR>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  launch_k((attn_kernel<D, NW, NTEAM, NR>), grid, dim3(64 * NW * NTEAM), lds, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_attention_splits(const AttnArgs &a, int D, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  if (G < 1 || G > 8) return hipErrorInvalidValue;
  const int nw = (G + 1) / 2;
  const dim3 grid(a.grid);
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
      // one wave holds a whole 64 x 128 K and V tile per register set: one set
      // in flight, as two would spill
      case 1: return go_attn<128, 1, 1, 1>(a, grid, sc, st);
      case 2: return go_attn<128, 2, 1, ATTN_NR128>(a, grid, sc, st);
      case 3: return go_attn<128, 3, 1, ATTN_NR128>(a, grid, sc, st);
      default: return go_attn<128, 4, 1, ATTN_NR128>(a, grid, sc, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_merge(const AttnArgs &a, int D, hipStream_t st) {
  if (D == 64)
    launch_k(attn_merge_kernel<64>, dim3(a.Hq, a.batch), dim3(256), 0, st, a);
  else if (D == 128)
    launch_k(attn_merge_kernel<128>, dim3(a.Hq, a.batch), dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int D, hipStream_t st) {
  const hipError_t e = launch_attention_splits(a, D, st);
  return e != hipSuccess ? e : launch_attention_merge(a, D, st);
}
