// Embedding gather, RMSNorm, argmax reduction + prefix accept, KV commit.
#include "common.h"
#include "kernels.h"

// h[m][:] = E[t[m]][:] (BF16 -> fp32).  Also checks that every sequence's
// block fits its cache (kv_len + 16 <= max_ctx); the QKV step skips the K/V
// writes of a sequence that does not.
__global__ void embed_kernel(const int32_t *__restrict__ tokens, int H, int V,
                             const uint16_t *__restrict__ table, float *__restrict__ h,
                             const int32_t *__restrict__ kv_len, int max_ctx, int32_t *err) {
  const int m = blockIdx.x;
  int t = tokens[m];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) set_error(err, SPEC_DERR_TOKEN);
    t = 0;
  }
  if ((m & 15) == 0 && threadIdx.x == 0) {
    const int n = kv_len[m >> 4];
    if (n < 0 || n + 16 > max_ctx) set_error(err, SPEC_DERR_CAPACITY);
  }
  const uint16_t *row = table + (size_t)t * H;
  for (int c = threadIdx.x; c < H; c += blockDim.x) h[(size_t)m * H + c] = bf16_to_f32(row[c]);
}

// h += part[0] + ... + part[ns-1] (split-K partials of the projection that
// just ran, added in split order), then x = h / sqrt(mean(h^2) + eps) * gain
// rounded to FP16 (decoder layers) or BF16 (lm_head input).  One wave per row.
template <bool BF16>
__global__ void norm_kernel(float *__restrict__ h, const float *__restrict__ part, int ns,
                            const float *__restrict__ gain, int M, int H, float eps, uint16_t *__restrict__ x,
                            float *__restrict__ dump) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  float *hr = h + (size_t)m * H;
  float ss = 0.f;
  const int nc = (H + 255) / 256;
  for (int i = 0; i < nc; ++i) {
    const int c = lane * 4 + 256 * i;
    f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (c < H) {
      t = *reinterpret_cast<const f32x4_t *>(hr + c);
      for (int s = 0; s < ns; ++s) t += *reinterpret_cast<const f32x4_t *>(part + ((size_t)s * M + m) * H + c);
      if (ns) *reinterpret_cast<f32x4_t *>(hr + c) = t;
    }
    ss += t[0] * t[0] + t[1] * t[1] + t[2] * t[2] + t[3] * t[3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float rs = 1.0f / sqrtf(ss / (float)H + eps);
  for (int i = 0; i < nc; ++i) {
    const int c = lane * 4 + 256 * i;
    if (c >= H) continue;
    const f32x4_t t = *reinterpret_cast<const f32x4_t *>(hr + c);  // written above by this lane
    const f32x4_t gv = *reinterpret_cast<const f32x4_t *>(gain + c);
    uint32_t lo, hi;
    if constexpr (BF16) {
      lo = pack_bf16x2(t[0] * rs * gv[0], t[1] * rs * gv[1]);
      hi = pack_bf16x2(t[2] * rs * gv[2], t[3] * rs * gv[3]);
    } else {
      lo = pack_f16x2(t[0] * rs * gv[0], t[1] * rs * gv[1]);
      hi = pack_f16x2(t[2] * rs * gv[2], t[3] * rs * gv[3]);
    }
    *reinterpret_cast<u32x2_t *>(x + (size_t)m * H + c) = u32x2_t{lo, hi};
    if (dump) {
      f32x4_t o;
      if constexpr (BF16)
        o = f32x4_t{bf16_to_f32(lo & 0xffff), bf16_to_f32(lo >> 16), bf16_to_f32(hi & 0xffff), bf16_to_f32(hi >> 16)};
      else
        o = f32x4_t{f16_to_f32(lo & 0xffff), f16_to_f32(lo >> 16), f16_to_f32(hi & 0xffff), f16_to_f32(hi >> 16)};
      *reinterpret_cast<f32x4_t *>(dump + (size_t)m * H + c) = o;
    }
  }
}

// One workgroup per sequence: g[j] = argmax over the vocab partials of row
// b*16+j (lowest id on ties), then tau = first j >= 1 with t[j] != g[j-1]
// (16 if none) and bonus = g[tau-1] (HunyuanOCR-1.5 / DFlash write-up,
// inference loop, step 4).
__global__ void accept_kernel(const ArgmaxPart *__restrict__ part, int nparts, int M,
                              const int32_t *__restrict__ tokens, int32_t *accept_len, int32_t *bonus,
                              int32_t *argmax, int32_t *last_tau) {
  __shared__ float sv[256];
  __shared__ int32_t si[256];
  __shared__ int32_t gsh[16];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int j = 0; j < 16; ++j) {
    const int m = b * 16 + j;
    float bv = -INFINITY;
    int32_t bi = 0x7fffffff;
    for (int p = tid; p < nparts; p += 256) {
      const ArgmaxPart q = part[(size_t)m * nparts + p];
      if (better(q.v, q.i, bv, bi)) {
        bv = q.v;
        bi = q.i;
      }
    }
    sv[tid] = bv;
    si[tid] = bi;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s && better(sv[tid + s], si[tid + s], sv[tid], si[tid])) {
        sv[tid] = sv[tid + s];
        si[tid] = si[tid + s];
      }
      __syncthreads();
    }
    if (tid == 0) gsh[j] = si[0] == 0x7fffffff ? 0 : si[0];
    __syncthreads();
  }
  if (tid == 0) {
    int tau = 16;
    for (int j = 1; j < 16; ++j)
      if (tokens[b * 16 + j] != gsh[j - 1]) {
        tau = j;
        break;
      }
    accept_len[b] = tau;
    bonus[b] = gsh[tau - 1];
    last_tau[b] = tau;
  }
  if (argmax && tid < 16) argmax[b * 16 + tid] = gsh[tid];
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

__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_embed(const int32_t *tokens, int M, int H, int V, const uint16_t *table, float *h,
                        const int32_t *kv_len, int max_ctx, int32_t *err, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(256), 0, st, tokens, H, V, table, h, kv_len, max_ctx, err);
  return hipGetLastError();
}

hipError_t launch_norm(float *h, const float *part, int nsplit, const float *gain, int M, int H, float eps,
                       uint16_t *x, int out_bf16, float *dump, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL(norm_kernel<true>, dim3((M + 3) / 4), dim3(256), 0, st, h, part, nsplit, gain, M, H, eps, x,
                       dump);
  else
    hipLaunchKernelGGL(norm_kernel<false>, dim3((M + 3) / 4), dim3(256), 0, st, h, part, nsplit, gain, M, H, eps,
                       x, dump);
  return hipGetLastError();
}

hipError_t launch_accept(const ArgmaxPart *part, int nparts, int M, const int32_t *tokens, int batch,
                         int32_t *accept_len, int32_t *bonus, int32_t *argmax, int32_t *last_tau,
                         hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(256), 0, st, part, nparts, M, tokens, accept_len,
                     bonus, argmax, last_tau);
  return hipGetLastError();
}

hipError_t launch_commit(int batch, const int32_t *n_commit, const int32_t *last_tau, int32_t *kv_len,
                         int max_ctx, int32_t *err, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3((batch + 255) / 256), dim3(256), 0, st, batch, n_commit, last_tau,
                     kv_len, max_ctx, err);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t st) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}
