// CLS-aware training objectives on the router pre-activations (BlockFFN
// write-up, lsdiaocha.cn, §3): the activation-locality loss and the
// chunk-sparsification loss, with their gradient with respect to z.
//
// With the sharp sigmoid p = sigmoid(alpha z) as the soft activation pattern:
//   L_AL = 1 / ((T - 1) E) sum_{t < T-1} sum_i BCE(p_{t,i}, [z_{t+1,i} > 0])
//          (the pattern sequence shifted left by one token is the target)
//   L_CS = 1 / (C E) sum_c sum_i (1 - prod_{t in c} (1 - p_{t,i}))
//          (the probability that expert i fires for some token of chunk c)
//   dz   = w_al dL_AL/dz + w_cs dL_CS/dz
//
// One block per chunk, one thread per expert: the chunk's p values sit in
// LDS, every thread forms its expert's product and the leave-one-out
// products of its gradient, and the block's two loss sums go to a partial
// that a one-block kernel adds in chunk order (deterministic; no atomics).
#include "bffn_internal.h"

namespace bffn {
namespace {

constexpr int kClsThreads = 128;  // one per expert (E <= 128)

__device__ __forceinline__ float softplusf(float s) { return s > 0.f ? s + log1pf(__expf(-s)) : log1pf(__expf(s)); }

__device__ __forceinline__ float block_sum128(float v, float* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = kClsThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kClsThreads) void cls_chunk_kernel(const float* __restrict__ z, int64_t T, int E, int L,
                                                                float alpha, float w_al, float w_cs, float n_al,
                                                                float n_cs, float* __restrict__ partial,
                                                                float* __restrict__ dz) {
  __shared__ float p_lds[32][kClsThreads];
  __shared__ float red[kClsThreads];
  const int i = threadIdx.x;
  const int64_t c = blockIdx.x, t0 = c * L;
  const bool v = i < E;
  float q = 1.f, al = 0.f;
  for (int u = 0; u < L; ++u) {
    const float zi = v ? z[(t0 + u) * E + i] : 0.f;
    const float s = alpha * zi;
    const float p = 1.f / (1.f + __expf(-s));
    p_lds[u][i] = p;
    q *= 1.f - p;
    if (v && t0 + u + 1 < T) {
      const float y = z[(t0 + u + 1) * E + i] > 0.f ? 1.f : 0.f;
      al += softplusf(s) - y * s;
    }
  }
  if (dz && v) {
    for (int u = 0; u < L; ++u) {
      const float p = p_lds[u][i];
      float others = 1.f;
      for (int w = 0; w < L; ++w)
        if (w != u) others *= 1.f - p_lds[w][i];
      float g = w_cs * alpha * p * (1.f - p) * others / n_cs;
      if (t0 + u + 1 < T) {
        const float y = z[(t0 + u + 1) * E + i] > 0.f ? 1.f : 0.f;
        g += w_al * alpha * (p - y) / n_al;
      }
      dz[(t0 + u) * E + i] = g;
    }
  }
  const float al_sum = block_sum128(v ? al : 0.f, red);
  const float cs_sum = block_sum128(v ? 1.f - q : 0.f, red);
  if (i == 0) {
    partial[2 * c] = al_sum;
    partial[2 * c + 1] = cs_sum;
  }
}

// losses[0] = sum of the locality partials / n_al, losses[1] = chunk partials / n_cs
__global__ __launch_bounds__(kBlock) void cls_reduce_kernel(const float* __restrict__ partial, int64_t C, float n_al,
                                                            float n_cs, float* __restrict__ losses) {
  __shared__ float ra[kBlock], rc[kBlock];
  const int tid = threadIdx.x;
  float a = 0.f, b = 0.f;
  for (int64_t c = tid; c < C; c += kBlock) {
    a += partial[2 * c];
    b += partial[2 * c + 1];
  }
  ra[tid] = a;
  rc[tid] = b;
  __syncthreads();
  for (int off = kBlock / 2; off > 0; off >>= 1) {
    if (tid < off) {
      ra[tid] += ra[tid + off];
      rc[tid] += rc[tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    losses[0] = n_al > 0.f ? ra[0] / n_al : 0.f;
    losses[1] = n_cs > 0.f ? rc[0] / n_cs : 0.f;
  }
}

}  // namespace

size_t cls_losses_workspace_bytes(int64_t T, int L) { return (size_t)(T / L) * 2 * sizeof(float) + 256; }

hipError_t launch_cls_losses(int E, const float* z, int64_t T, int L, float alpha, float w_al, float w_cs,
                             void* workspace, float* losses, float* dz, hipStream_t s) {
  const int64_t C = T / L;
  const float n_al = (float)((double)(T - 1) * E), n_cs = (float)((double)C * E);
  float* partial = static_cast<float*>(workspace);
  if (C > 0)
    cls_chunk_kernel<<<dim3((unsigned)C), dim3(kClsThreads), 0, s>>>(z, T, E, L, alpha, w_al, w_cs,
                                                                     n_al > 0.f ? n_al : 1.f, n_cs, partial, dz);
  cls_reduce_kernel<<<dim3(1), dim3(kBlock), 0, s>>>(partial, C, T > 1 ? n_al : 0.f, C > 0 ? n_cs : 0.f, losses);
  return hipGetLastError();
}

}  // namespace bffn
