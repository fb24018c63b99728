// The router's epilogue, shared by every kernel that forms pre-activations:
// ReLU, then RMSNorm over the E outputs (or a baseline gate function), and
// the activation pattern (BlockFFN write-up, lsdiaocha.cn, §2 core design: a
// ReLU router followed by RMSNorm, which separates the activation pattern
// from its strength).
#pragma once

#include "bffn_internal.h"

namespace bffn {
namespace {

// Wave arg-max over the experts not yet taken: larger z wins, the lower index
// among equal z.  Every lane gets the winner's index.
__device__ __forceinline__ int wave_argmax(float c0, float c1, int lane) {
  float bz = c0;
  int bi = lane;
  if (c1 > bz) {
    bz = c1;
    bi = lane + 64;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float oz = __shfl_xor(bz, off, kWave);
    const int oi = __shfl_xor(bi, off, kWave);
    if (oz > bz || (oz == bz && oi < bi)) {
      bz = oz;
      bi = oi;
    }
  }
  return bi;
}

// Partial sums zp[part][e][n] (n < L) in LDS -> gates, masks, optional z.
// Wave w of the block's nw waves handles tokens n = w, w + nw, ...; lane l
// handles experts l, l + 64.
// kind selects the gate function: the BlockFFN router (ReLU, then RMSNorm
// over the E outputs) or one of the baseline routers (top-k of a softmax;
// ReLU divided by its sum).
// mask_lds (or nullptr): the tokens' mask words are also written there, token n at mask_lds[n * W].
template <int KIND>
__device__ void router_epilogue(const float* zp, int nparts, int E, int L, int64_t t0,
                                const float* __restrict__ b, const float* __restrict__ s, float eps, int top_k,
                                float* __restrict__ gates, uint64_t* __restrict__ masks,
                                float* __restrict__ preact, uint64_t* mask_lds = nullptr) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int W = (E + 63) >> 6;
  const bool v0 = lane < E, v1 = lane + 64 < E;
  const float b0 = (v0 && b) ? b[lane] : 0.f, b1 = (v1 && b) ? b[lane + 64] : 0.f;
  const float s0 = (v0 && s) ? s[lane] : 1.f, s1 = (v1 && s) ? s[lane + 64] : 1.f;
  for (int n = w; n < L; n += nw) {
    float z0 = 0.f, z1 = 0.f;
    for (int p = 0; p < nparts; ++p) {
      if (v0) z0 += zp[(p * E + lane) * L + n];
      if (v1) z1 += zp[(p * E + lane + 64) * L + n];
    }
    z0 += b0;
    z1 += b1;
    bool on0 = v0 && z0 > 0.f, on1 = v1 && z1 > 0.f;
    const float a0 = on0 ? z0 : 0.f, a1 = on1 ? z1 : 0.f;
    float g0, g1;
    if (KIND == BLOCKFFN_ROUTER_TOPK_SOFTMAX) {
      const float ninf = -__builtin_huge_valf();
      float c0 = v0 ? z0 : ninf, c1 = v1 ? z1 : ninf;
      float zmax = c0 > c1 ? c0 : c1;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(zmax, off, kWave);
        zmax = o > zmax ? o : zmax;
      }
      const float e0 = v0 ? __expf(z0 - zmax) : 0.f, e1 = v1 ? __expf(z1 - zmax) : 0.f;
      const float inv = 1.0f / wave_sum(e0 + e1);
      on0 = on1 = false;
      for (int r = 0; r < top_k; ++r) {
        const int win = wave_argmax(c0, c1, lane);
        if (win == lane) {
          on0 = true;
          c0 = ninf;
        }
        if (win == lane + 64) {
          on1 = true;
          c1 = ninf;
        }
      }
      g0 = on0 ? e0 * inv : 0.f;
      g1 = on1 ? e1 * inv : 0.f;
    } else if (KIND == BLOCKFFN_ROUTER_RELU_SUM) {
      const float sum = wave_sum(a0 + a1);
      const float inv = sum > 0.f ? 1.0f / sum : 0.f;
      g0 = a0 * inv;
      g1 = a1 * inv;
    } else {
      // mean over all E outputs, inactive ones included
      const float ms = wave_sum(a0 * a0 + a1 * a1) / (float)E;
      const float inv = 1.0f / sqrtf(ms + eps);
      g0 = s0 * a0 * inv;
      g1 = s1 * a1 * inv;
    }
    const int64_t t = t0 + n;
    if (v0) gates[t * E + lane] = g0;
    if (v1) gates[t * E + lane + 64] = g1;
    if (preact) {
      if (v0) preact[t * E + lane] = z0;
      if (v1) preact[t * E + lane + 64] = z1;
    }
    const uint64_t m0 = __ballot(on0);
    const uint64_t m1 = __ballot(on1);
    if (lane == 0) {
      masks[t * W] = m0;
      if (W > 1) masks[t * W + 1] = m1;
      if (mask_lds) {
        mask_lds[n * W] = m0;
        if (W > 1) mask_lds[n * W + 1] = m1;
      }
    }
  }
}

}  // namespace
}  // namespace bffn
