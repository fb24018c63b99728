// Router: z = W_r x + b, a = ReLU(z), g = s * a / sqrt(mean_E(a^2) + eps),
// activation pattern bit i = [z_i > 0].
// (BlockFFN write-up, lsdiaocha.cn, §2 core design: a ReLU router followed by
// RMSNorm, which separates the activation pattern from its strength; BlockFFN
// abstract, arXiv 2507.08771: a router integrating ReLU and RMSNorm.)
//
// One workgroup per unit (a chunk of L tokens, or one token when L == 1),
// or per 16-token tile when all units share one layer, computes the tokens'
// E pre-activations into LDS, then a fused epilogue applies ReLU + RMSNorm
// and builds the 64-bit activation words with wave64 ballots.  Three
// producers of the pre-activations:
//   * route_ring_kernel (bf16, every unit through one layer, any L): one
//     block per 16-token tile; each wave streams its quarter of d through a
//     private 3-slot DMA ring of whole 128-byte lines (lds_stream.h), and
//     the four partial sums are added in a fixed order in the epilogue.
//   * route_mfma_kernel (bf16, L >= 8, one unit per block through the unit's
//     own layer copy): the router is a genuine E x d x tokens contraction;
//     each wave streams a quarter of d for every expert row through
//     v_mfma_f32_16x16x32_bf16 (pipelined as in mfma_stream.h), partial sums
//     added in a fixed order.
//   * route_valu_kernel (fp32, or L < 8 with a layer copy per unit): a
//     bandwidth-bound GEMV; lane groups stride over d with 16-byte loads and
//     reduce with cross-lane shuffles.
#include "lds_stream.h"
#include "mfma_stream.h"
#include "router_epilogue.h"

namespace bffn {
namespace {

template <typename T>
__device__ __forceinline__ float dot16(const T* a, const T* b);

template <>
__device__ __forceinline__ float dot16<float>(const float* a, const float* b) {
  const f32x4 va = *reinterpret_cast<const f32x4*>(a);
  const f32x4 vb = *reinterpret_cast<const f32x4*>(b);
  return va.x * vb.x + va.y * vb.y + va.z * vb.z + va.w * vb.w;
}

template <>
__device__ __forceinline__ float dot16<uint16_t>(const uint16_t* a, const uint16_t* b) {
  const u32x4 va = *reinterpret_cast<const u32x4*>(a);
  const u32x4 vb = *reinterpret_cast<const u32x4*>(b);
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) acc += bf16_lo(va[q]) * bf16_lo(vb[q]) + bf16_hi(va[q]) * bf16_hi(vb[q]);
  return acc;
}

// lpr lanes per router row (a power of two dividing 64); each lane covers nv
// 16-byte vectors of the row.
template <typename T, int KIND>
__global__ __launch_bounds__(kBlock) void route_valu_kernel(LayerArgs la, const T* __restrict__ x, int L,
                                                            int lpr, int nv, int top_k,
                                                            float* __restrict__ gates,
                                                            uint64_t* __restrict__ masks,
                                                            float* __restrict__ preact) {
  extern __shared__ float zp[];  // [E][L]
  const int64_t unit = blockIdx.x;
  const T* wr = layer_ptr<kTWRouter>(la, static_cast<const T*>(la.w_router), unit);
  const float* b = layer_ptr<kTBRouter>(la, la.b_router, unit);
  const float* s = layer_ptr<kTScale>(la, la.rms_scale, unit);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = la.d, E = la.E;
  constexpr int VEC = 16 / sizeof(T);
  const int rpp = 64 / lpr, lg = lane / lpr, li = lane % lpr;
  const int64_t t0 = unit * L;
  for (int r0 = w * rpp; r0 < E; r0 += 4 * rpp) {
    const int r = r0 + lg;
    const bool rv = r < E;
    for (int n = 0; n < L; ++n) {
      float acc = 0.f;
      if (rv) {
        const T* wrow = wr + (int64_t)r * d;
        const T* xrow = x + (t0 + n) * d;
        for (int mm = 0; mm < nv; ++mm) {
          const int k = (li + mm * lpr) * VEC;
          acc += dot16<T>(wrow + k, xrow + k);
        }
      }
      for (int off = lpr >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
      if (rv && li == 0) zp[r * L + n] = acc;
    }
  }
  __syncthreads();
  router_epilogue<KIND>(zp, 1, E, L, t0, b, s, la.eps, top_k, gates, masks, preact);
}

// MFMA router.  Wave w owns d-range [w d/4, (w+1) d/4) for every expert row,
// in blocks of four 16-row stripes, streamed with the two-deep pipeline of
// mfma_stream.h; the last block's missing stripes repeat a valid stripe and
// are not stored.  The four per-wave partial sums meet in LDS and are added
// in a fixed order by the epilogue (deterministic).
//
// A block takes tokens [t0, t0 + tb); the launch gives it one unit (tb = L,
// the unit's own layer copy).  (A router shared by every token goes to
// route_ring_kernel.)  Blocks start at different stripe groups, which spreads
// simultaneous reads of a router they share.
// With one token tile the registers are capped for two waves per SIMD (two
// blocks per CU): 30.8 us instead of 33.9 us for 512 chunk-8 units.
template <int NT, int KIND>
__global__ __launch_bounds__(kBlock, NT == 1 ? 2 : 1) void route_mfma_kernel(LayerArgs la,
                                                                             const uint16_t* __restrict__ x,
                                                            int64_t T, int L, int tb, int top_k,
                                                            float* __restrict__ gates,
                                                            uint64_t* __restrict__ masks,
                                                            float* __restrict__ preact) {
  extern __shared__ float zp[];  // [4][E][Lb]
  const int64_t t0 = (int64_t)blockIdx.x * tb;
  const int Lb = T - t0 < tb ? (int)(T - t0) : tb;  // tokens of this block
  const int64_t unit = t0 / L;
  const uint16_t* wr = layer_ptr<kTWRouter>(la, static_cast<const uint16_t*>(la.w_router), unit);
  const float* b = layer_ptr<kTBRouter>(la, la.b_router, unit);
  const float* s = layer_ptr<kTScale>(la, la.rms_scale, unit);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int d = la.d, E = la.E;
  const int kw = d >> 2;
  const int nstripes = E >> 4;
  const int ngroups = (nstripes + 3) >> 2;
  const uint16_t* b_row[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) b_row[tl] = x + (t0 + (m + 16 * tl) % Lb) * d;
  for (int q = 0; q < ngroups; ++q) {
    const int sb = (int)((q + blockIdx.x) % ngroups) * 4;
    const uint16_t* a_row[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int stripe = sb + st < nstripes ? sb + st : nstripes - 1;
      a_row[st] = wr + (int64_t)(stripe * 16 + m) * d;
    }
    f32x4 acc[4][NT];
    zero_acc<NT>(acc);
    stream_contract<NT>(acc, a_row, b_row, w * kw, kw >> 7, g);
    // D layout: lane (m, g) holds rows 4 g + r, column m of each 16 x 16 tile.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (sb + st >= nstripes) continue;
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const int n = m + 16 * tl;
        if (n >= Lb) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) zp[(w * E + (sb + st) * 16 + 4 * g + r) * Lb + n] = acc[st][tl][r];
      }
    }
  }
  __syncthreads();
  router_epilogue<KIND>(zp, 4, E, Lb, t0, b, s, la.eps, top_k, gates, masks, preact);
}

// Router shared by every token (one layer), one 16-token tile per block, by
// DMA.  Streaming the router into registers in the MFMA layout makes every
// load instruction touch 16 rows at 64 bytes each (half lines); there the
// vector-memory pipeline of the CU, not L2, set the pace (measured: the
// texture addresser busy 57% of the time at ~56 cycles per load, L2 hits at
// ~260 cycles).  Here each wave streams its quarter of d through a private
// ring of the chunk path's geometry (lds_stream.h): a step is 64 router rows
// (one group of four stripes) and the tile's 16 token rows, 128 bytes each,
// so every DMA instruction reads 8 whole lines.  Groups follow one another
// (rotated per block, as in route_mfma_kernel); the partial sums of each
// group go to LDS and the common epilogue adds them in a fixed order.
constexpr int kRouteRingMaxE = 128;

template <int KIND>
__global__ __launch_bounds__(kBlock) void route_ring_kernel(LayerArgs la, const uint16_t* __restrict__ x, int64_t T,
                                                           int top_k, float* __restrict__ gates,
                                                           uint64_t* __restrict__ masks,
                                                           float* __restrict__ preact) {
  using G = RingGeom<1, false>;
  constexpr int kRings = (kBlock / kWave) * kRingBufs * G::kBufBytes;
  // one LDS object: the four waves' rings, then the partial sums [4][E][Lb]
  __shared__ __attribute__((aligned(16))) uint8_t lds[kRings + 4 * kRouteRingMaxE * 16 * 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int d = la.d, E = la.E;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int Lb = T - t0 < 16 ? (int)(T - t0) : 16;
  uint8_t* bufs = lds + w * (kRingBufs * G::kBufBytes);
  float* zp = reinterpret_cast<float*>(lds + kRings);
  const uint16_t* wr = static_cast<const uint16_t*>(la.w_router);
  const int kw = d >> 2;  // this wave's range of d
  const int S = kw / kStepK;
  const int nstripes = E >> 4, ngroups = (nstripes + 3) >> 2;
  const int total = ngroups * S;
  auto group_base = [&](int q) { return (int)((q + blockIdx.x) % ngroups) * 4; };
  // step t: group t / S, k step t % S (past the end: the last step again)
  auto issue = [&](int slot, int t) {
    const int tc = t < total ? t : total - 1;
    const int sb = group_base(tc / S);
    const int k0 = w * kw + (tc % S) * kStepK;
    uint8_t* buf = bufs + slot * G::kBufBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int R = 8 * j + (lane >> 3);
      const int st = sb + (R >> 4) < nstripes ? sb + (R >> 4) : nstripes - 1;  // missing stripes repeat one
      dma16<kPolicyReuse>(wr + (int64_t)(st * 16 + (R & 15)) * d + k0 + dma_chunk_elems(R, lane), buf + j * 1024);
    }
#pragma unroll
    for (int j = 0; j < G::kBInstr; ++j) {
      const int n = 8 * j + (lane >> 3);  // tokens past the tile repeat one
      dma16<kPolicyReuse>(x + (t0 + n % Lb) * d + k0 + dma_chunk_elems(n, lane), buf + kABytes + j * 1024);
    }
  };

  issue(0, 0);
  issue(1, 1);
  f32x4 acc[4][1];
  ring_zero<1>(acc);
  for (int t = 0; t < total; ++t) {
    issue((t + kRingBufs - 1) % kRingBufs, t + kRingBufs - 1);
    wait_vmcnt<G::kWaitAhead>();
    ring_mfma<1>(acc, bufs + (t % kRingBufs) * G::kBufBytes, m, g);
    __builtin_amdgcn_sched_barrier(0);
    if ((t + 1) % S == 0) {  // (uniform) group done: lane (m, g) holds rows 4 g + r of token m
      const int sb = group_base(t / S);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (sb + st >= nstripes || m >= Lb) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) zp[(w * E + (sb + st) * 16 + 4 * g + r) * Lb + m] = acc[st][0][r];
      }
      ring_zero<1>(acc);
    }
  }
  wait_vmcnt<0>();  // the repeats land before the LDS is read or given up
  __syncthreads();
  router_epilogue<KIND>(zp, 4, E, Lb, t0, la.b_router, la.rms_scale, la.eps, top_k, gates, masks, preact);
}

}  // namespace

bool route_uses_mfma(int d, int E, int chunk_len, int dtype) {
  return dtype == BLOCKFFN_BF16 && chunk_len >= 8 && E % 16 == 0 && d % 512 == 0;
}

template <int KIND>
hipError_t launch_route_kind(const LayerArgs& la, const void* x, int64_t units, int L, int dtype, int top_k,
                             float* gates, uint64_t* masks, float* preact, hipStream_t s) {
  const int64_t T = units * L;
  const bool shared = la.n_layers == 1 && route_uses_mfma(la.d, la.E, 16, dtype);
  if (shared && la.E <= kRouteRingMaxE) {  // (E never exceeds it: the layer check caps E at 128)
    route_ring_kernel<KIND><<<dim3((unsigned)((T + 15) / 16)), dim3(kBlock), 0, s>>>(
        la, static_cast<const uint16_t*>(x), T, top_k, gates, masks, preact);
  } else if (route_uses_mfma(la.d, la.E, L, dtype)) {
    // one unit per block, through the unit's own layer copy
    const int tb = L;
    const int64_t blocks = (T + tb - 1) / tb;
    const size_t lds = sizeof(float) * 4 * la.E * tb;
    if (tb <= 16)
      route_mfma_kernel<1, KIND><<<dim3((unsigned)blocks), dim3(kBlock), lds, s>>>(
          la, static_cast<const uint16_t*>(x), T, L, tb, top_k, gates, masks, preact);
    else
      route_mfma_kernel<2, KIND><<<dim3((unsigned)blocks), dim3(kBlock), lds, s>>>(
          la, static_cast<const uint16_t*>(x), T, L, tb, top_k, gates, masks, preact);
  } else {
    const size_t lds = sizeof(float) * la.E * L;
    const int vec = dtype == BLOCKFFN_F32 ? 4 : 8;
    const int nvec = la.d / vec;
    int lpr = 64;
    while (nvec % lpr) lpr >>= 1;
    const int nv = nvec / lpr;
    if (dtype == BLOCKFFN_F32)
      route_valu_kernel<float, KIND><<<dim3((unsigned)units), dim3(kBlock), lds, s>>>(
          la, static_cast<const float*>(x), L, lpr, nv, top_k, gates, masks, preact);
    else
      route_valu_kernel<uint16_t, KIND><<<dim3((unsigned)units), dim3(kBlock), lds, s>>>(
          la, static_cast<const uint16_t*>(x), L, lpr, nv, top_k, gates, masks, preact);
  }
  return hipGetLastError();
}

hipError_t launch_route(const LayerArgs& la, const void* x, int64_t n_tokens, int chunk_len, int dtype, int kind,
                        int top_k, float* gates, uint64_t* masks, float* preact, hipStream_t s) {
  const int64_t units = n_tokens / chunk_len;
  if (units == 0) return hipSuccess;
  switch (kind) {
    case BLOCKFFN_ROUTER_TOPK_SOFTMAX:
      return launch_route_kind<BLOCKFFN_ROUTER_TOPK_SOFTMAX>(la, x, units, chunk_len, dtype, top_k, gates, masks,
                                                             preact, s);
    case BLOCKFFN_ROUTER_RELU_SUM:
      return launch_route_kind<BLOCKFFN_ROUTER_RELU_SUM>(la, x, units, chunk_len, dtype, top_k, gates, masks, preact,
                                                         s);
    default:
      return launch_route_kind<BLOCKFFN_ROUTER_BLOCKFFN>(la, x, units, chunk_len, dtype, top_k, gates, masks, preact,
                                                         s);
  }
}

}  // namespace bffn
