// Expert streaming on the matrix cores: the chunk path (bf16, L >= 8).
// (BlockFFN write-up, lsdiaocha.cn, §4 acceleration kernel: multiply only by
// the experts in the union of the chunk's activations, batching the chunk's
// tokens, then mask the irrelevant activations; §7: an outer loop over the
// active experts with a batched product inside.)
//
// Up:   H'[unit][slot] (L x d_e) = g[:, i] * Swish(X_chunk W_in[i]^T), stored bf16
// Down: Y_chunk (L x d) = sum over the union's slots, in list order, of
//       H'[unit][slot] W_out[i]^T, accumulated in fp32 registers
//
// Both are tall-skinny products (L <= 32 tokens against 128..4096 weight
// rows), so weights are the streamed MFMA operand A (16 rows per stripe, four
// stripes per wave) and tokens the small operand B (16 columns per tile,
// padded past L).  Every weight element is used by exactly one lane, so A goes
// from HBM straight into registers with no LDS round trip, two steps in
// flight (mfma_stream.h).
#include "mfma_stream.h"

namespace bffn {
namespace {

// One up-projection item: 64 rows (block rb) of the expert in `slot` of
// chunk `unit`, over all of d, for every token of the chunk.
template <int NT>
__device__ __forceinline__ void up_item(const LayerArgs& la, const uint16_t* __restrict__ x, int L,
                                        const float* __restrict__ gates, int64_t unit, int slot, int rb, int i,
                                        uint16_t* __restrict__ hbuf) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int d = la.d, de = la.de, E = la.E;
  const uint16_t* wi = layer_ptr(static_cast<const uint16_t*>(la.w_in), la.stride, unit, la.n_layers);
  const uint16_t* a_row[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) a_row[s] = wi + ((int64_t)i * de + rb * 64 + s * 16 + m) * d;
  const int64_t t0 = unit * L;
  const uint16_t* b_row[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) b_row[tl] = x + (t0 + (m + 16 * tl) % L) * d;
  f32x4 acc[4][NT];
  zero_acc<NT>(acc);
  stream_contract<NT>(acc, a_row, b_row, 0, d >> 7, g);

  // D layout: lane (m, g) holds rows 4 g + r (r < 4), column m of each tile.
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int n = m + 16 * tl;
    if (n >= L) continue;
    const float gv = gates[(t0 + n) * E + i];
    uint16_t* hrow = hbuf + ((unit * E + slot) * L + n) * (int64_t)de + rb * 64 + 4 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 v = acc[s][tl];
      const uint32_t lo = f32_to_bf16(gv * swish(v[0])) | (f32_to_bf16(gv * swish(v[1])) << 16);
      const uint32_t hi = f32_to_bf16(gv * swish(v[2])) | (f32_to_bf16(gv * swish(v[3])) << 16);
      *reinterpret_cast<u32x2*>(hrow + s * 16) = u32x2{lo, hi};
    }
  }
}

// Exclusive prefix over chunks of the up-projection item counts
// (union size x row blocks, or E x row blocks in dense mode):
// prefix[u] = items of chunks < u, prefix[n_units] = total.  One block.
__global__ __launch_bounds__(1024) void plan_items_kernel(const int32_t* __restrict__ count, int64_t n_units,
                                                          int dense_E, int per_slot, int64_t* __restrict__ prefix) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n_units + 1023) / 1024;
  const int64_t b = tid * per, e = b + per < n_units ? b + per : n_units;
  int64_t sum = 0;
  for (int64_t u = b; u < e; ++u) sum += dense_E ? dense_E : count[u];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int64_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = part[tid] - sum;
  for (int64_t u = b; u < e; ++u) {
    prefix[u] = run * per_slot;
    run += dense_E ? dense_E : count[u];
  }
  if (tid == 1023) prefix[n_units] = part[1023] * per_slot;
}

// Persistent up-projection: a fixed grid sized to the resident capacity; wave
// gw takes items gw, gw + W, gw + 2W, ... of the chunk-major item list, so
// every wave streams weights and no block is spent on inactive slots.
template <int NT, bool DENSE>
__global__ __launch_bounds__(kBlock) void up_mfma_kernel(LayerArgs la, const uint16_t* __restrict__ x,
                                                         int64_t n_units, int L, const float* __restrict__ gates,
                                                         const int32_t* __restrict__ list,
                                                         const int64_t* __restrict__ prefix,
                                                         uint16_t* __restrict__ hbuf) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int rbs = la.de >> 6;
  const int64_t total = prefix[n_units];
  for (int64_t item = (int64_t)blockIdx.x * 4 + w; item < total; item += nwaves) {
    int64_t lo = 0, hi = n_units - 1;  // last chunk whose prefix <= item
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int64_t unit = lo;
    const int r = (int)(item - prefix[unit]);
    const int slot = r / rbs, rb = r % rbs;
    const int i = DENSE ? slot : list[unit * la.E + slot];
    up_item<NT>(la, x, L, gates, unit, slot, rb, i, hbuf);
  }
}

template <int NT, bool DENSE>
__global__ __launch_bounds__(kBlock) void down_mfma_kernel(LayerArgs la, int64_t n_units, int L,
                                                           const int32_t* __restrict__ count,
                                                           const int32_t* __restrict__ list,
                                                           int64_t blocks_per_unit,
                                                           const uint16_t* __restrict__ hbuf,
                                                           float* __restrict__ y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int64_t lb = xcd_logical_block(blockIdx.x, n_units * blocks_per_unit);
  if (lb < 0) return;
  const int64_t unit = lb / blocks_per_unit;
  const int wave_in_unit = (int)(lb % blocks_per_unit) * 4 + w;
  const int d = la.d, de = la.de, E = la.E;
  const int kb = wave_in_unit * 64;
  if (kb >= d) return;
  const int n_active = DENSE ? E : count[unit];
  const uint16_t* wo = layer_ptr(static_cast<const uint16_t*>(la.w_out), la.stride, unit, la.n_layers);
  const int64_t t0 = unit * L;
  const int spe = de >> 7;  // 128-element steps per expert
  const int n_steps = n_active * spe;

  f32x4 acc[4][NT];
  zero_acc<NT>(acc);

  // Step p covers slot p / spe, elements [128 (p % spe), +128) of that expert.
  auto load = [&](Step<NT>& st, int p) {
    const int slot = p / spe, j0 = (p % spe) * 128;
    const int i = DENSE ? slot : list[unit * E + slot];
    const uint16_t* a_row[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a_row[s] = wo + ((int64_t)i * d + kb + s * 16 + m) * de;
    const uint16_t* b_row[NT];
#pragma unroll
    for (int tl = 0; tl < NT; ++tl)
      b_row[tl] = hbuf + ((unit * E + slot) * L + (m + 16 * tl) % L) * (int64_t)de;
    load_step<NT>(st, a_row, b_row, j0, g);
  };

  // Two-deep software pipeline over the union's steps, tail peeled.
  Step<NT> s0, s1;
  if (n_steps > 0) {
    load(s0, 0);
    int p = 0;
    for (; p + 2 < n_steps; p += 2) {
      load(s1, p + 1);
      fence_schedule();
      mfma_step<NT>(acc, s0);
      fence_schedule();
      load(s0, p + 2);
      fence_schedule();
      mfma_step<NT>(acc, s1);
      fence_schedule();
    }
    if (p + 1 < n_steps) {
      load(s1, p + 1);
      mfma_step<NT>(acc, s0);
      mfma_step<NT>(acc, s1);
    } else {
      mfma_step<NT>(acc, s0);
    }
  }

#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int n = m + 16 * tl;
    if (n >= L) continue;
    float* yrow = y + (t0 + n) * d + kb + 4 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) *reinterpret_cast<f32x4*>(yrow + s * 16) = acc[s][tl];
  }
}

template <int NT, bool DENSE>
hipError_t launch_nt(const LayerArgs& la, const uint16_t* x, int64_t units, int L, const float* gates,
                     const int32_t* count, const int32_t* list, uint16_t* hbuf, int64_t* plan, float* y,
                     const StageEvents& se, hipStream_t s) {
  const int rbs = la.de >> 6;
  plan_items_kernel<<<dim3(1), dim3(1024), 0, s>>>(count, units, DENSE ? la.E : 0, rbs, plan);
  se.record(0, s);
  {
    // resident capacity: blocks per CU at this kernel's register use, times CUs
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, up_mfma_kernel<NT, DENSE>, kBlock, 0);
    if (e != hipSuccess) return e;
    const int64_t max_items = units * la.E * rbs;
    int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    const int64_t need = (max_items + 3) / 4;
    if (grid > need) grid = need;
    up_mfma_kernel<NT, DENSE><<<dim3((unsigned)grid), dim3(kBlock), 0, s>>>(la, x, units, L, gates, list, plan,
                                                                             hbuf);
  }
  se.record(1, s);
  {
    const int waves = la.d >> 6;
    const int64_t bpu = (waves + 3) / 4;
    const int64_t nlog = units * bpu;
    down_mfma_kernel<NT, DENSE><<<dim3((unsigned)xcd_grid(nlog)), dim3(kBlock), 0, s>>>(la, units, L, count, list,
                                                                                         bpu, hbuf, y);
  }
  se.record(2, s);
  return hipGetLastError();
}

}  // namespace

bool forward_mfma_supported(int d, int de, int dtype) {
  return dtype == BLOCKFFN_BF16 && d % 128 == 0 && de % 128 == 0;
}

hipError_t launch_forward_mfma(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, int chunk_len,
                               const float* gates, const int32_t* count, const int32_t* list, bool dense,
                               uint16_t* hbuf, int64_t* plan, float* y, const StageEvents& se, hipStream_t s) {
  const int64_t units = n_tokens / chunk_len;
  if (units == 0) return hipSuccess;
  if (dense) {
    if (chunk_len <= 16) return launch_nt<1, true>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, se, s);
    return launch_nt<2, true>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, se, s);
  }
  if (chunk_len <= 16) return launch_nt<1, false>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, se, s);
  return launch_nt<2, false>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, se, s);
}

}  // namespace bffn
