// Internal declarations shared by the gfx950 kernels of libblockffn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "blockffn.h"

namespace bffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // four waves
constexpr int kXcds = 8;     // MI355X: 8 accelerator complex dies, each with its own L2

// Kernel-side view of the layers a call's units cycle through: unit u uses
// layer u % n_layers.  The named pointers are layer 0's.  Either the layers
// lie evenly spaced in memory (layer l's tensors at ptr + l * stride bytes;
// the host finds this out, and a single layer has stride 0), or listed == 1
// and layer l's pointers are tab[tensor][l], at most kMaxListedLayers of
// them.  The table is a kernel argument: a lookup is one scalar load from
// the kernel-argument segment.
constexpr int kMaxListedLayers = 32;
enum LayerTensor { kTWRouter = 0, kTBRouter = 1, kTScale = 2, kTWIn = 3, kTWOut = 4, kLayerTensors = 5 };

struct LayerArgs {
  const void* w_router;
  const float* b_router;
  const float* rms_scale;
  const void* w_in;
  const void* w_out;
  int64_t stride;
  int32_t n_layers;
  int32_t listed;
  int32_t d, E, de;
  float eps;
  const void* tab[kLayerTensors][kMaxListedLayers];
};

// Tensor K of the layer that unit `unit` uses; p0 is layer 0's pointer.
template <int K, typename P>
__device__ __forceinline__ P layer_ptr(const LayerArgs& la, P p0, int64_t unit) {
  if (la.n_layers == 1) return p0;
  const int64_t l = unit % la.n_layers;
  if (la.listed) return reinterpret_cast<P>(la.tab[K][l]);
  if (p0 == nullptr) return p0;
  return reinterpret_cast<P>(reinterpret_cast<const char*>(p0) + la.stride * l);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 through gfx950's packed conversion (v_cvt_pk_bf16_f32):
// round to nearest even, denormals kept, NaN stays NaN.  One instruction
// per pair instead of a rounding sequence per value, which matters in MFMA
// epilogues.  pack2_bf16 puts `lo` in bits 0-15.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack2_bf16(f, 0.f) & 0xffffu; }

// Swish with beta = 1 (SiLU): u * logistic(u).
__device__ __forceinline__ float swish(float u) { return u / (1.0f + __expf(-u)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// 64-bit activation-mask helpers.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Number of set bits of v in lane positions below this lane.
__device__ __forceinline__ int rank_below(uint64_t v) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(v >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)v, 0u));
}

__device__ __forceinline__ uint64_t valid_bits(int E, int word) {
  const int nb = E - 64 * word;
  if (nb >= 64) return ~0ull;
  if (nb <= 0) return 0ull;
  return (1ull << nb) - 1ull;
}

// Lane l gets lane l - 1's value (lane 0 its own).
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v) {
  const uint32_t lo = __shfl_up((uint32_t)v, 1, kWave), hi = __shfl_up((uint32_t)(v >> 32), 1, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += shfl_xor_u64(v, off);
  return v;
}

// Blocks of one launch are handed to the 8 XCDs round-robin.  Renumber them
// so that each XCD works through one contiguous range of logical blocks:
// blocks of the same unit then share that XCD's L2 for their common operand.
// The grid is padded to a multiple of 8; returns -1 for padding blocks.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t bid, int64_t n_logical) {
  const int64_t per = (n_logical + kXcds - 1) / kXcds;
  const int64_t logical = (bid % kXcds) * per + bid / kXcds;
  return logical < n_logical ? logical : -1;
}
inline int64_t xcd_grid(int64_t n_logical) { return ((n_logical + kXcds - 1) / kXcds) * kXcds; }

// Caller-provided events recorded around the forward's kernels (may be empty).
struct StageEvents {
  hipEvent_t* ev = nullptr;
  int n = 0;
  void record(int k, hipStream_t s) const {
    if (ev != nullptr && k < n) (void)hipEventRecord(ev[k], s);
  }
};

// ---- launchers (host side, enqueue only; arguments already validated) ----
hipError_t launch_route(const LayerArgs& la, const void* x, int64_t n_tokens, int chunk_len, int dtype, int kind,
                        int top_k, float* gates, uint64_t* masks, float* preact, hipStream_t s);
hipError_t launch_chunk_union(int E, const uint64_t* masks, int64_t n_tokens, int chunk_len,
                              uint64_t* chunk_masks, int32_t* count, int32_t* list, hipStream_t s);
hipError_t launch_stats(int E, const uint64_t* masks, int64_t n_tokens, int chunk_len,
                        blockffn_stats* out, hipStream_t s);
hipError_t launch_forward_gemv(const LayerArgs& la, const void* x, int64_t n_tokens, int chunk_len,
                               int dtype, const float* gates, const int32_t* count, const int32_t* list,
                               bool dense, float* hbuf, float* y, const StageEvents& se, hipStream_t s);
// The chunk path split for a few units: up items cut into ks k-ranges, down
// items into sp ranges of the union's slots, with fp32 partial tiles in
// up_part / down_part.  ks == 0: no split.
struct ChunkSplit {
  int ks = 0, sp = 0;
  float* up_part = nullptr;
  float* down_part = nullptr;
};
constexpr int64_t kChunkSplitMaxUnits = 16;  // AUTO splits launches of at most this many units
bool chunk_split_factors(int d, int de, int64_t units, bool force, int* ks, int* sp);
size_t chunk_split_part_bytes(int d, int de, int E, int64_t units, int chunk_len, int ks, int sp,
                              size_t* down_offset);
hipError_t launch_forward_mfma(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, int chunk_len,
                               const float* gates, const int32_t* count, const int32_t* list, bool dense,
                               uint16_t* hbuf, int64_t* plan, const ChunkSplit& sp, float* y, const StageEvents& se,
                               hipStream_t s);

hipError_t launch_forward_grouped(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, const float* gates,
                                  void* workspace, float* y, const StageEvents& se, hipStream_t s);
size_t grouped_workspace_bytes(int64_t n_tokens, int E, int d, int de);
bool grouped_supported(int d, int de, int dtype);

hipError_t launch_backward(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, const float* preact,
                           const float* dy, const float* dz_extra, void* workspace, float* dx, float* d_w_router, float* d_b_router,
                           float* d_rms_scale, float* d_w_in, float* d_w_out, const StageEvents& se, hipStream_t s);
size_t backward_workspace_bytes(int64_t n_tokens, int E, int d, int de);
hipError_t launch_cls_losses(int E, const float* z, int64_t T, int L, float alpha, float w_al, float w_cs,
                             void* workspace, float* losses, float* dz, hipStream_t s);
size_t cls_losses_workspace_bytes(int64_t n_tokens, int chunk_len);

// One layer step (router, union, statistics, forward) of a short call in
// three launches (layer_step.hip): bf16, E a multiple of 16, d and d_e
// multiples of 128 with d <= 4096, at most kStepMaxUnits units and
// kStepMaxTokens tokens.  Its workspace: the router's partial
// pre-activations (fp32), then Swish(W_in x) (bf16).
constexpr int64_t kStepMaxTokens = 64;
constexpr int64_t kStepMaxUnits = 16;
bool layer_step_fused(int d, int E, int de, int dtype, int64_t n_tokens, int chunk_len);
size_t layer_step_zpart_bytes(int d, int E, int64_t n_tokens);
size_t layer_step_hs_bytes(int E, int de, int64_t n_tokens);
hipError_t launch_layer_step(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, int chunk_len, float* gates,
                             uint64_t* masks, float* preact, uint64_t* chunk_masks, int32_t* count, int32_t* list,
                             blockffn_stats* stats, float* zpart, uint16_t* hs, float* y, hipStream_t s);
// The step's up and down kernels as the forward of at most kStepMaxUnits units with a given union
// (workspace: layer_step_hs_bytes).
bool forward_few_supported(int d, int de, int dtype, int64_t units, int chunk_len);
hipError_t launch_forward_few(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, int chunk_len,
                              const float* gates, const int32_t* count, const int32_t* list, uint16_t* hs, float* y,
                              const StageEvents& se, hipStream_t s);

// Resident blocks of `kernel` on the current device (CUs x blocks per CU at
// `block` threads, no dynamic LDS).  Queried once per (device, kernel) and
// cached, so persistent launches cost no runtime query after the first.
hipError_t resident_blocks(const void* kernel, int block, int64_t* blocks);

bool route_uses_mfma(int d, int E, int chunk_len, int dtype);
bool forward_mfma_supported(int d, int de, int dtype);
size_t forward_mfma_plan_bytes(int64_t units);

}  // namespace bffn
