// Streaming MFMA contraction shared by the router and the chunk-path expert
// kernels: weights (operand A, 16 rows per stripe, 4 stripes per wave) stream
// from HBM straight into VGPRs in the v_mfma_f32_16x16x32_bf16 operand layout
// while the small token operand B (16 columns per tile) is reused per step.
//
// Operand layout (checked on gfx950): lane l supplies row l % 16 of A and
// column l % 16 of B, with elements 8 (l / 16) .. +7 of the 32-wide k block,
// and receives rows 4 (l / 16) + r (r < 4) of column l % 16 of D.  A 128-
// element step is four MFMAs; MFMA q takes elements [32 q + 8 g, +8) of lane
// group g, so one load instruction reads 64 contiguous bytes of each of 16
// rows and two consecutive instructions complete each 128-byte line.
#pragma once

#include "bffn_internal.h"

namespace bffn {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int NT>
struct Step {
  u32x4 a[4][4];   // [stripe][q]
  u32x4 b[NT][4];  // [token tile][q]
};

__device__ __forceinline__ int kofs(int g, int q) { return q * 32 + g * 8; }

// a_row[s]: this lane's row of stripe s; b_row[tl]: this lane's token row of
// tile tl.  Lanes of tokens past the chunk read a valid row of the chunk
// instead (MFMA output columns are independent and those columns are never
// stored), which keeps pipelined loops free of branches.
template <int NT>
__device__ __forceinline__ void load_step(Step<NT>& st, const uint16_t* const (&a_row)[4],
                                          const uint16_t* const (&b_row)[NT], int k0, int g) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q) st.a[s][q] = *reinterpret_cast<const u32x4*>(a_row[s] + k0 + kofs(g, q));
#pragma unroll
  for (int tl = 0; tl < NT; ++tl)
#pragma unroll
    for (int q = 0; q < 4; ++q) st.b[tl][q] = *reinterpret_cast<const u32x4*>(b_row[tl] + k0 + kofs(g, q));
}

// Keeps the compiler's scheduler from moving instructions across this point,
// so a step's loads stay issued ahead of the previous step's MFMAs (left
// alone, it sinks them and waits for every load before each MFMA).
__device__ __forceinline__ void fence_schedule() { __builtin_amdgcn_sched_barrier(0); }

template <int NT>
__device__ __forceinline__ void mfma_step(f32x4 (&acc)[4][NT], const Step<NT>& st) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tl = 0; tl < NT; ++tl)
        acc[s][tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.a[s][q]), as_bf16x8(st.b[tl][q]),
                                                             acc[s][tl], 0, 0, 0);
}

template <int NT>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[4][NT]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) acc[s][tl] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc += A[:, k_base : k_base + 128 nsteps] . B over `nsteps` 128-element
// steps, two-deep software pipeline with the tail peeled.
template <int NT>
__device__ __forceinline__ void stream_contract(f32x4 (&acc)[4][NT], const uint16_t* const (&a_row)[4],
                                                const uint16_t* const (&b_row)[NT], int k_base, int nsteps,
                                                int g) {
  Step<NT> s0, s1;
  load_step<NT>(s0, a_row, b_row, k_base, g);
  int k = 0;
  for (; k + 2 < nsteps; k += 2) {
    load_step<NT>(s1, a_row, b_row, k_base + ((k + 1) << 7), g);
    fence_schedule();
    mfma_step<NT>(acc, s0);
    fence_schedule();
    load_step<NT>(s0, a_row, b_row, k_base + ((k + 2) << 7), g);
    fence_schedule();
    mfma_step<NT>(acc, s1);
    fence_schedule();
  }
  if (k + 1 < nsteps) {
    load_step<NT>(s1, a_row, b_row, k_base + ((k + 1) << 7), g);
    mfma_step<NT>(acc, s0);
    mfma_step<NT>(acc, s1);
  } else {
    mfma_step<NT>(acc, s0);
  }
}

}  // namespace bffn
