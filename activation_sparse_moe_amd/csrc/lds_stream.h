// Weight streaming through a wave-private LDS ring, for the chunk-path expert
// kernels.
//
// Each wave owns kRingBufs buffers.  A buffer holds one 64-element k-step of
// a 64-row weight block (64 rows x 128 B) followed by 16 NT token rows of the
// small operand.  Rows are filled by global_load_lds_dwordx4: one instruction
// moves 64 lanes x 16 B to LDS at base + 16 lane, and the 8 lanes of a row
// read one whole 128-byte line, so every request is a full line and the
// weights can be loaded with the non-temporal policy (streamed once, never
// reused).  The 16-byte chunk a lane fetches is XOR-swizzled by row so that
// the MFMA operand reads (16 rows, one chunk each) spread over the LDS banks.
// Two steps are always in flight ahead of the one being multiplied, so the
// wait before a step is a constant vmcnt.
//
// Work items are shared out in two levels: each block gets a statically
// balanced share of the items (a contiguous range, or its turns in its XCD's
// range), and the block's waves take items from that share through an LDS
// counter (an LDS atomic waits on lgkmcnt, not on vmcnt, so taking work never
// drains the weight stream).
//
// Operand layout (v_mfma_f32_16x16x32_bf16, checked on gfx950): lane l
// supplies row l % 16 of A and column l % 16 of B with k elements
// 8 (l / 16) .. +7 of the 32-wide block, and receives rows 4 (l / 16) + r
// (r < 4) of column l % 16 of D.
#pragma once

#include "bffn_internal.h"

namespace bffn {

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

constexpr int kRingBufs = 3;
constexpr int kStepK = 64;           // k elements per step
constexpr int kRowBytes = 128;       // bytes of one row per step
constexpr int kABytes = 64 * kRowBytes;
constexpr unsigned kPolicyStream = 2;  // non-temporal
constexpr unsigned kPolicyReuse = 0;

// One buffer: A rows, then B rows, then (GATES) 64 fp32 per-token values.
template <int NT, bool GATES>
struct RingGeom {
  static constexpr int kBInstr = 2 * NT;  // 16 NT token rows, 8 per instruction
  static constexpr int kGateOff = kABytes + kBInstr * 1024;
  static constexpr int kBufBytes = kGateOff + (GATES ? 256 : 0);
  static constexpr int kLoadsPerStep = 8 + kBInstr + (GATES ? 1 : 0);
  static constexpr int kWaitAhead = (kRingBufs - 1) * kLoadsPerStep;  // loads of the steps in flight
};

__device__ __forceinline__ int ring_swz(int row) { return (row >> 1) & 7; }

// Element offset, within a row's 64-element step, of the chunk this lane
// fetches for row `row` (lane slot lane % 8 holds chunk slot ^ swizzle).
__device__ __forceinline__ int dma_chunk_elems(int row, int lane) { return ((lane & 7) ^ ring_swz(row)) * 8; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
  __builtin_amdgcn_sched_barrier(0);
}

// Block barrier for data that DMA has already delivered to LDS: no fence,
// so the DMA of later steps stays in flight (__syncthreads would drain it).
__device__ __forceinline__ void block_barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One DMA instruction: this lane's 16 bytes from src to LDS dst + 16 lane.
template <unsigned POLICY>
__device__ __forceinline__ void dma16(const uint16_t* src, uint8_t* dst_instr_base) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)dst_instr_base, 16, 0, POLICY);
}

// One DMA instruction of 4 bytes per lane (LDS dst + 4 lane).
__device__ __forceinline__ void dma4(const float* src, uint8_t* dst_instr_base) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)dst_instr_base, 4, 0, kPolicyReuse);
}

__device__ __forceinline__ bf16x8 ring_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Reads of one buffer: A row R (0..63), B row n (0..16 NT - 1), k chunk c.
__device__ __forceinline__ u32x4 ring_read_a(const uint8_t* buf, int R, int c) {
  return *reinterpret_cast<const u32x4*>(buf + R * kRowBytes + ((c ^ ring_swz(R)) << 4));
}
__device__ __forceinline__ u32x4 ring_read_b(const uint8_t* buf, int n, int c) {
  return *reinterpret_cast<const u32x4*>(buf + kABytes + n * kRowBytes + ((c ^ ring_swz(n)) << 4));
}

// acc[s][tl] += A rows 16 s + m  x  B rows 16 tl + m over this buffer's 64 k.
template <int NT>
__device__ __forceinline__ void ring_mfma(f32x4 (&acc)[4][NT], const uint8_t* buf, int m, int g) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    u32x4 a[4], b[NT];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = ring_read_a(buf, 16 * s + m, 4 * q + g);
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) b[tl] = ring_read_b(buf, 16 * tl + m, 4 * q + g);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tl = 0; tl < NT; ++tl)
        acc[s][tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring_bf16x8(a[s]), ring_bf16x8(b[tl]), acc[s][tl], 0,
                                                             0, 0);
  }
}

// Next item of the block's share for this wave: LDS counter k, broadcast,
// item lo + stride k.  The counter sits outside every ring buffer, so the
// atomic cannot race with the weight DMA; it is written as assembly (with its
// own lgkmcnt wait, so the result register is complete when the block ends)
// because the compiler cannot prove that and would otherwise drain every
// in-flight DMA first.
__device__ __forceinline__ int64_t take_item(unsigned* counter, int64_t lo, int64_t stride, int lane) {
  unsigned v = 0;
  if (lane == 0) {
    const unsigned addr = (unsigned)(uintptr_t)(lvoid_t*)counter;
    const unsigned one = 1u;
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr), "v"(one));
  }
  return lo + stride * (int64_t)__builtin_amdgcn_readfirstlane(__shfl(v, 0, kWave));
}

template <int NT>
__device__ __forceinline__ void ring_zero(f32x4 (&acc)[4][NT]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) acc[s][tl] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace bffn
