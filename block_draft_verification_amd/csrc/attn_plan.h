// Split plan of the block-causal attention of one pass (device code, one wave).
//
// The attention kernel's workgroups each take one key split of one (sequence,
// KV head) unit, and every split has the same length of t 64-key tiles; a
// unit with T tiles has ceil(T / t) splits.  The plan picks the smallest t,
// a multiple of the teams per workgroup, whose splits fit in the launch's
// `grid` workgroups (one resident round on the chip), so that the longest
// split, which bounds the kernel's time, is as short as the cache lengths of
// this pass allow.  It depends on kv_len, which lives on the device, so it is
// computed there, once per pass, and written to a small table:
//   plan[0]     = {t, total splits, 0, 0}
//   plan[1 + b] = {first slot of unit (b, 0), splits per unit of b, kv_len[b], 0}
// Unit (b, h) owns slots first + h * splits .. + splits - 1; slot = workgroup
// index of the attention launch = index of its partial (m, l, o).
#pragma once
#include "common.h"
#include "kernels.h"

#define ATTN_MAX_SPLITS 64  // splits per unit: bounds the merge step's work per row

__device__ __forceinline__ int plan_wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int plan_wave_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int plan_ceil_div(int a, int b) { return (a + b - 1) / b; }

// 64-key tiles a sequence's block rows read: keys 0 .. n+15, clamped to the cache
__device__ __forceinline__ int attn_seq_tiles(int n, int max_ctx) {
  const int L = min(max(n, 0) + 16, max_ctx);
  return (L + 63) >> 6;
}

// Called by all 64 lanes of one wave.
__device__ inline void attn_plan_wave(const int32_t *__restrict__ kv_len, const AttnPlanArgs &p, int lane) {
  auto tiles = [&](int b) { return b < p.batch ? attn_seq_tiles(kv_len[b], p.max_ctx) : 0; };
  int tsum = 0, tmax = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int T = tiles(b0 + lane);
    tsum += T;
    tmax = max(tmax, T);
  }
  tsum = plan_wave_sum(tsum);
  tmax = plan_wave_max(tmax);
  int t = p.fixed_t;
  if (t <= 0) {
    // workgroups needed with splits of t tiles
    auto count = [&](int tt) {
      int n = 0;
      for (int b0 = 0; b0 < p.batch; b0 += 64) n += plan_ceil_div(tiles(b0 + lane), tt);
      return p.Hkv * plan_wave_sum(n);
    };
    // search over s = tiles per team: t = s * nteam.  At s >= tmax / nteam
    // every unit has one split, Hkv * batch <= grid workgroups, so hi fits;
    // lo respects the merge step's split limit and the total-work bound.
    const int nt = p.nteam;
    int lo = max(plan_ceil_div(plan_ceil_div(p.Hkv * tsum, p.grid), nt),
                 plan_ceil_div(plan_ceil_div(tmax, ATTN_MAX_SPLITS), nt));
    int hi = max(lo, plan_ceil_div(tmax, nt));
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (count(mid * nt) <= p.grid) hi = mid;
      else lo = mid + 1;
    }
    t = lo * nt;
  }
  int carry = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int b = b0 + lane, nsp = plan_ceil_div(tiles(b), t), u = p.Hkv * nsp;
    int incl = u;  // inclusive scan of the units' slots over the chunk
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      incl += lane >= o ? y : 0;
    }
    if (b < p.batch) p.plan[1 + b] = make_int4(carry + incl - u, nsp, kv_len[b], 0);
    carry += __shfl(incl, 63);
  }
  if (lane == 0) p.plan[0] = make_int4(t, carry, 0, 0);
}
