// Block-causal GQA attention of the 16 block rows over the KV cache (gfx950).
//
// Row j of sequence b sits at position n_b + j and sees keys 0 .. n_b + j:
// the committed prefix plus the block rows up to itself, which the QKV step
// has already stored at slots n_b .. n_b+15 (HunyuanOCR-1.5 / DFlash write-up,
// inference loop, step 3: the whole block is verified in one forward).
// Query head h reads KV head h / G, so the G*16 query rows of one KV head
// share every K/V tile: the pass is bound by reading the cache once.
//
// Work unit = (split, kv head, sequence): one workgroup of 4 waves walks its
// split's keys in tiles of 64.  Each tile is loaded into registers two tiles
// ahead, converted from the BF16 cache to FP16 and stored in LDS (K
// row-major, V transposed).  A wave owns 16-row query tiles (one query head
// each, rows j = 0..15).  Scores are computed transposed, S^T = K Q^T, with
// the MFMA A operand taken from K in LDS and the B operand = Q^T (FP16) held
// in registers; in that layout a lane (r, g) holds 16 keys of query r, so
// softmax statistics need only xor-16/32 shuffles, and the FP16
// probabilities are already the B operand of O^T = V^T P^T.  Online softmax
// in fp32, base 2.
//
// Splits write unnormalised partials (m, l, o); a second kernel merges them
// in split order per (query head, sequence), so the result does not depend on
// timing and no workgroup waits on another (a device-wide fence inside the
// kernel would flush the XCD's L2).
#include "common.h"
#include "kernels.h"

#define KT 64  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a, float scale_log2) {
  constexpr int DT = D / 16;   // 16-wide d tiles
  constexpr int DK = D / 32;   // k32 steps over d
  constexpr int KP = D + 8;    // K row pitch (16-bit elements)
  constexpr int VP = KT + 4;   // V^T row pitch (16-bit elements), 8-byte aligned rows
  constexpr int KCH = KT * D / 8;        // K: 16-byte chunks (one key, 8 d) per tile
  constexpr int VCH = (KT / 2) * D / 4;  // V: chunks of (2 keys, 4 d)
  constexpr int KPT = KCH / 256, VPT = VCH / 256;
  __shared__ __align__(16) uint16_t Ks[KT * KP];
  __shared__ __align__(16) uint16_t Vt[D * VP];

  const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int n = a.kv_len[b];
  const int L = min(max(n, 0) + 16, a.max_ctx);
  const int nsplit = (L + a.split_len - 1) / a.split_len;
  if (sp >= nsplit) return;  // whole workgroup
  const int key_lo = sp * a.split_len, key_hi = min(key_lo + a.split_len, L);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, g = lane >> 4;
  const size_t cache_base = ((size_t)b * a.Hkv + kvh) * a.max_ctx;
  const size_t unit = (size_t)b * a.Hkv + kvh;
  const int qstride = a.Hq * D;

  // this wave's query tiles: wave, wave+4 (G <= 8)
  const int nqt = (G - wave + 3) / 4;
  u32x4_t qf[2][DK];
  f32x4_t oacc[2][DT];
  float mrow[2], lrow[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    mrow[u] = -INFINITY;
    lrow[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[u][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (u < nqt) {
      const int hq = kvh * G + wave + 4 * u;
      const uint16_t *qp = a.q + (size_t)(b * 16 + r) * qstride + hq * D + 8 * g;
#pragma unroll
      for (int kd = 0; kd < DK; ++kd) qf[u][kd] = *reinterpret_cast<const u32x4_t *>(qp + 32 * kd);
    }
  }

  struct TileRegs {
    u32x4_t k[KPT];
    u32x2_t v[VPT][2];
  };
  TileRegs ra, rb;
  // Loads are unconditional (indices clamped to the split's last key) so the
  // wave does not branch around them.
  auto load_tile = [&](TileRegs &tr, int kt0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i, kk = c / (D / 8), d0 = (c % (D / 8)) * 8, key = min(kt0 + kk, key_hi - 1);
      tr.k[i] = *reinterpret_cast<const u32x4_t *>(a.k_cache + (cache_base + key) * D + d0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + 256 * i, kk = 2 * (c / (D / 4)), d0 = (c % (D / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // keys past the split end repeat its last key: their scores are masked to -inf, so
        // p = 0 and the (finite) values never reach the output
        const int key = min(kt0 + kk + e, key_hi - 1);
        tr.v[i][e] = *reinterpret_cast<const u32x2_t *>(a.v_cache + (cache_base + key) * D + d0);
      }
    }
  };
  auto store_tile = [&](const TileRegs &tr) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i, kk = c / (D / 8), d0 = (c % (D / 8)) * 8;
      const u32x4_t v = tr.k[i];
      *reinterpret_cast<u32x4_t *>(&Ks[kk * KP + d0]) =
          u32x4_t{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + 256 * i, kk = 2 * (c / (D / 4)), d0 = (c % (D / 4)) * 4;
      const uint32_t a0 = bf16x2_to_f16x2(tr.v[i][0].x), a1 = bf16x2_to_f16x2(tr.v[i][0].y);
      const uint32_t b0 = bf16x2_to_f16x2(tr.v[i][1].x), b1 = bf16x2_to_f16x2(tr.v[i][1].y);
      // (key kk, key kk+1) pairs for d0 .. d0+3
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 0) * VP + kk]) = (a0 & 0xffff) | (b0 << 16);
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 1) * VP + kk]) = (a0 >> 16) | (b0 & 0xffff0000u);
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 2) * VP + kk]) = (a1 & 0xffff) | (b1 << 16);
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 3) * VP + kk]) = (a1 >> 16) | (b1 & 0xffff0000u);
    }
  };

  auto compute = [&](int kt0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u >= nqt) break;  // wave-uniform
      // S^T tiles: 4 subtiles of 16 keys; lane holds keys kt0 + 16ks + 4g + i for query r
      f32x4_t st[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        st[ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < DK; ++kd) {
          const u32x4_t kf = *reinterpret_cast<const u32x4_t *>(&Ks[(16 * ks + r) * KP + 32 * kd + 8 * g]);
          st[ks] = mfma16x16x32_f16(kf, qf[u][kd], st[ks]);
        }
      }
      const int last_visible = n + r;  // row j = r
      float tmax = -INFINITY;
      if (kt0 + KT <= n && kt0 + KT <= key_hi) {  // whole tile in the committed prefix: nothing to mask
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st[ks][i] *= scale_log2;
            tmax = fmaxf(tmax, st[ks][i]);
          }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt0 + 16 * ks + 4 * g + i;
            const float v = (key <= last_visible && key < key_hi) ? st[ks][i] * scale_log2 : -INFINITY;
            st[ks][i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrow[u], tmax);
      float alpha, psum = 0.f;
      u32x4_t pb[2];
      if (mnew == -INFINITY) {  // nothing visible yet for this row
        alpha = 1.f;
        pb[0] = pb[1] = u32x4_t{0, 0, 0, 0};
      } else {
        alpha = __builtin_amdgcn_exp2f(mrow[u] - mnew);
        float p[4][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[ks][i] = __builtin_amdgcn_exp2f(st[ks][i] - mnew);
            psum += p[ks][i];
          }
        // B operand for keys 32c + {4g+i} (slots 0-3) and 32c + 16 + {4g+i} (slots 4-7)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          pb[c] = u32x4_t{pack_f16x2(p[2 * c][0], p[2 * c][1]), pack_f16x2(p[2 * c][2], p[2 * c][3]),
                          pack_f16x2(p[2 * c + 1][0], p[2 * c + 1][1]),
                          pack_f16x2(p[2 * c + 1][2], p[2 * c + 1][3])};
      }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      mrow[u] = mnew;
      lrow[u] = lrow[u] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[u][dt] = oacc[u][dt] * alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t *vrow = &Vt[(16 * dt + r) * VP + 32 * c + 4 * g];
          const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + 16);
          oacc[u][dt] = mfma16x16x32_f16(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb[c], oacc[u][dt]);
        }
    }
  };

  load_tile(ra, key_lo);
  if (key_lo + KT < key_hi) load_tile(rb, key_lo + KT);
  // barriers only order LDS traffic (lds_barrier): a __syncthreads() here would
  // also wait for the prefetched tile and serialise the pipeline
  for (int kt0 = key_lo; kt0 < key_hi; kt0 += 2 * KT) {
    lds_barrier();  // previous tile consumed
    store_tile(ra);
    lds_barrier();
    if (kt0 + 2 * KT < key_hi) load_tile(ra, kt0 + 2 * KT);  // two tiles in flight during the math
    compute(kt0);
    if (kt0 + KT >= key_hi) break;
    lds_barrier();
    store_tile(rb);
    lds_barrier();
    if (kt0 + 3 * KT < key_hi) load_tile(rb, kt0 + 3 * KT);
    compute(kt0 + KT);
  }

  // partials: row R = tile*16 + j, o[d] with d = 16dt + 4g + i held by lane (r = j, g)
  const int R = G * 16;
  float *po = a.part_o + ((unit * a.nsplit + sp) * R) * D;
  float2 *pml = a.part_ml + (unit * a.nsplit + sp) * R;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u >= nqt) break;
    const int row = (wave + 4 * u) * 16 + r;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t *>(po + (size_t)row * D + 16 * dt + 4 * g) = oacc[u][dt];
    if (g == 0) pml[row] = make_float2(mrow[u], lrow[u]);
  }
}

// o[b*16+j][hq*D + d] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the
// splits of sequence b, in split order.  One workgroup per (query head, seq):
// the split statistics are loaded in parallel into LDS, each row's weights
// w_s = 2^(m_s - M) / den are formed once, then every thread sums its 4
// columns over the splits with independent loads.  A split that saw no key of
// a row has m_s = -inf and weight 0 (its partial is 0, never NaN).
#define MAX_SPLITS 64

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

int attention_split_len(int batch, int Hkv, int max_ctx) {
  // aim for about 768 workgroups across the batch; splits are whole 64-key
  // tiles and a sequence has at most MAX_SPLITS of them
  const long target = 768;
  long sl = ((long)batch * Hkv * max_ctx + target - 1) / target;
  const long min_sl = (max_ctx + MAX_SPLITS - 1) / MAX_SPLITS;
  if (sl < min_sl) sl = min_sl;
  sl = ((sl + KT - 1) / KT) * KT;
  if (sl < KT) sl = KT;
  return (int)sl;
}

hipError_t launch_attention_splits(const AttnArgs &a, int D, hipStream_t st) {
  dim3 grid(a.nsplit, a.Hkv, a.batch);
  if (D == 64)
    hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(256), 0, st, a, (float)(1.4426950408889634 / 8.0));
  else if (D == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, dim3(256), 0, st, a,
                       (float)(1.4426950408889634 / 11.313708498984761));
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
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
