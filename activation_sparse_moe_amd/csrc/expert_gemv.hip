// Expert streaming on the vector ALUs: the path for single tokens, short
// chunks and fp32 layers, where each streamed weight meets at most a few
// tokens and the work is a bandwidth-bound GEMV.
// (BlockFFN write-up, lsdiaocha.cn, §2: non-gated Swish expert MLPs; §4: run
// only the union's experts and mask the irrelevant token-expert activations
// with the gates; §6: the single-token sparse kernel.)
//
// Up:   h'[unit][slot][n][j] = g[t_n][i] * Swish(W_in[i][j][:] . x[t_n])  (fp32)
// Down: y[t_n][k] = sum over slots s < count, in list order, of
//                   W_out[i_s][k][:] . h'[unit][s][n][:]
// Each down wave owns whole output rows and walks the chunk's list itself, so
// outputs need no atomics and no partial buffers.
#include "bffn_internal.h"

namespace bffn {
namespace {

template <typename T>
struct Vec16;  // 16 bytes of weights, widened against fp32 or same-type operands

template <>
struct Vec16<float> {
  static constexpr int kElems = 4;
  __device__ static float dot_same(const float* a, const float* b) {
    const f32x4 va = *reinterpret_cast<const f32x4*>(a);
    const f32x4 vb = *reinterpret_cast<const f32x4*>(b);
    return va.x * vb.x + va.y * vb.y + va.z * vb.z + va.w * vb.w;
  }
  __device__ static float dot_f32(const float* a, const float* h) { return dot_same(a, h); }
};

template <>
struct Vec16<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static float dot_same(const uint16_t* a, const uint16_t* b) {
    const u32x4 va = *reinterpret_cast<const u32x4*>(a);
    const u32x4 vb = *reinterpret_cast<const u32x4*>(b);
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc += bf16_lo(va[q]) * bf16_lo(vb[q]) + bf16_hi(va[q]) * bf16_hi(vb[q]);
    return acc;
  }
  __device__ static float dot_f32(const uint16_t* a, const float* h) {
    const u32x4 va = *reinterpret_cast<const u32x4*>(a);
    const f32x4 h0 = *reinterpret_cast<const f32x4*>(h);
    const f32x4 h1 = *reinterpret_cast<const f32x4*>(h + 4);
    return bf16_lo(va[0]) * h0.x + bf16_hi(va[0]) * h0.y + bf16_lo(va[1]) * h0.z + bf16_hi(va[1]) * h0.w +
           bf16_lo(va[2]) * h1.x + bf16_hi(va[2]) * h1.y + bf16_lo(va[3]) * h1.z + bf16_hi(va[3]) * h1.w;
  }
};

// Rows are split over lane groups of `lpr` lanes (a power of two); a group
// covers its row with `nv` 16-byte vectors per lane.  Four rows per group are
// in flight per iteration, against up to kTokGroup tokens of the unit.
constexpr int kTokGroup = 4;

template <typename T, bool DENSE>
__global__ __launch_bounds__(kBlock) void up_valu_kernel(LayerArgs la, const T* __restrict__ x, int64_t n_units,
                                                         int L, const float* __restrict__ gates,
                                                         const int32_t* __restrict__ count,
                                                         const int32_t* __restrict__ list,
                                                         int rows_per_wave, int lpr, int nv,
                                                         int64_t blocks_per_unit, float* __restrict__ hbuf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t lb = xcd_logical_block(blockIdx.x, n_units * blocks_per_unit);
  if (lb < 0) return;
  const int64_t unit = lb / blocks_per_unit;
  const int wave_in_unit = (int)(lb % blocks_per_unit) * 4 + w;
  const int de = la.de, d = la.d, E = la.E;
  const int rbs = de / rows_per_wave;
  const int slot = wave_in_unit / rbs, rb = wave_in_unit % rbs;
  const int n_active = DENSE ? E : count[unit];
  if (slot >= n_active) return;
  const int i = DENSE ? slot : list[unit * E + slot];
  const T* wi = layer_ptr<kTWIn>(la, static_cast<const T*>(la.w_in), unit) + (int64_t)i * de * d;
  constexpr int VEC = Vec16<T>::kElems;
  const int rpp = 64 / lpr, lg = lane / lpr, li = lane % lpr;
  const int64_t t0 = unit * L;
  const int r_end = (rb + 1) * rows_per_wave;
  // tokens kTokGroup at a time: each weight vector is loaded once per group
  // and meets every token of it (the per-(row, token) sums keep their order)
  for (int n0 = 0; n0 < L; n0 += kTokGroup) {
    for (int r0 = rb * rows_per_wave; r0 < r_end; r0 += 4 * rpp) {
      float acc[4][kTokGroup] = {};
      for (int mm = 0; mm < nv; ++mm) {
        const int k = (li + mm * lpr) * VEC;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = r0 + q * rpp + lg;
          if (r >= r_end) continue;
          const T* wrow = wi + (int64_t)r * d + k;
#pragma unroll
          for (int j = 0; j < kTokGroup; ++j)
            if (n0 + j < L) acc[q][j] += Vec16<T>::dot_same(wrow, x + (t0 + n0 + j) * d + k);
        }
      }
#pragma unroll
      for (int j = 0; j < kTokGroup; ++j) {
        if (n0 + j >= L) break;
        const float gate = gates[(t0 + n0 + j) * E + i];
        float* hrow = hbuf + ((unit * E + slot) * L + n0 + j) * (int64_t)de;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          for (int off = lpr >> 1; off > 0; off >>= 1) acc[q][j] += __shfl_xor(acc[q][j], off, kWave);
        if (li == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = r0 + q * rpp + lg;
            if (r < r_end) hrow[r] = gate * swish(acc[q][j]);
          }
        }
      }
    }
  }
}

template <typename T, bool DENSE>
__global__ __launch_bounds__(kBlock) void down_valu_kernel(LayerArgs la, int64_t n_units, int L,
                                                           const int32_t* __restrict__ count,
                                                           const int32_t* __restrict__ list,
                                                           int rows_per_wave, int lpr, int nv,
                                                           int64_t blocks_per_unit, const float* __restrict__ hbuf,
                                                           float* __restrict__ y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t lb = xcd_logical_block(blockIdx.x, n_units * blocks_per_unit);
  if (lb < 0) return;
  const int64_t unit = lb / blocks_per_unit;
  const int wave_in_unit = (int)(lb % blocks_per_unit) * 4 + w;
  const int de = la.de, d = la.d, E = la.E;
  const int k0 = wave_in_unit * rows_per_wave;
  if (k0 >= d) return;
  const int k_end = min(d, k0 + rows_per_wave);
  const int n_active = DENSE ? E : count[unit];
  const T* wo_base = layer_ptr<kTWOut>(la, static_cast<const T*>(la.w_out), unit);
  constexpr int VEC = Vec16<T>::kElems;
  const int rpp = 64 / lpr, lg = lane / lpr, li = lane % lpr;
  const int64_t t0 = unit * L;
  for (int n0 = 0; n0 < L; n0 += kTokGroup) {
    for (int r0 = k0; r0 < k_end; r0 += 4 * rpp) {
      float acc[4][kTokGroup] = {};
      for (int s = 0; s < n_active; ++s) {
        const int i = DENSE ? s : list[unit * E + s];
        const T* wo = wo_base + (int64_t)i * d * de;
        const float* hbase = hbuf + ((unit * E + s) * L + n0) * (int64_t)de;
        for (int mm = 0; mm < nv; ++mm) {
          const int j0 = (li + mm * lpr) * VEC;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = r0 + q * rpp + lg;
            if (r >= k_end) continue;
            const T* wrow = wo + (int64_t)r * de + j0;
#pragma unroll
            for (int j = 0; j < kTokGroup; ++j)
              if (n0 + j < L) acc[q][j] += Vec16<T>::dot_f32(wrow, hbase + (int64_t)j * de + j0);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kTokGroup; ++j) {
        if (n0 + j >= L) break;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          for (int off = lpr >> 1; off > 0; off >>= 1) acc[q][j] += __shfl_xor(acc[q][j], off, kWave);
        if (li == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = r0 + q * rpp + lg;
            if (r < k_end) y[(t0 + n0 + j) * d + r] = acc[q][j];
          }
        }
      }
    }
  }
}

void lane_split(int len, int vec, int* lpr, int* nv) {
  const int nvec = len / vec;
  int l = 64;
  while (nvec % l) l >>= 1;
  *lpr = l;
  *nv = nvec / l;
}

template <typename T, bool DENSE>
hipError_t launch_gemv_typed(const LayerArgs& la, const T* x, int64_t units, int L, const float* gates,
                             const int32_t* count, const int32_t* list, float* hbuf, float* y,
                             const StageEvents& se, hipStream_t s) {
  constexpr int VEC = Vec16<T>::kElems;
  se.record(0, s);
  // up: one wave per (slot, 16 rows of W_in[i]); E slots reserved per unit
  {
    const int rows = 16;
    const int waves = la.E * (la.de / rows);
    const int64_t bpu = (waves + 3) / 4;
    int lpr, nv;
    lane_split(la.d, VEC, &lpr, &nv);
    const int64_t nlog = units * bpu;
    up_valu_kernel<T, DENSE><<<dim3((unsigned)xcd_grid(nlog)), dim3(kBlock), 0, s>>>(
        la, x, units, L, gates, count, list, rows, lpr, nv, bpu, hbuf);
  }
  se.record(1, s);
  // down: one wave per 64 output rows
  {
    const int rows = 64;
    const int waves = (la.d + rows - 1) / rows;
    const int64_t bpu = (waves + 3) / 4;
    int lpr, nv;
    lane_split(la.de, VEC, &lpr, &nv);
    const int64_t nlog = units * bpu;
    down_valu_kernel<T, DENSE><<<dim3((unsigned)xcd_grid(nlog)), dim3(kBlock), 0, s>>>(
        la, units, L, count, list, rows, lpr, nv, bpu, hbuf, y);
  }
  se.record(2, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_gemv(const LayerArgs& la, const void* x, int64_t n_tokens, int chunk_len, int dtype,
                               const float* gates, const int32_t* count, const int32_t* list, bool dense,
                               float* hbuf, float* y, const StageEvents& se, hipStream_t s) {
  const int64_t units = n_tokens / chunk_len;
  if (units == 0) return hipSuccess;
  const float* xf = static_cast<const float*>(x);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (dtype == BLOCKFFN_F32)
    return dense ? launch_gemv_typed<float, true>(la, xf, units, chunk_len, gates, count, list, hbuf, y, se, s)
                 : launch_gemv_typed<float, false>(la, xf, units, chunk_len, gates, count, list, hbuf, y, se, s);
  return dense ? launch_gemv_typed<uint16_t, true>(la, xb, units, chunk_len, gates, count, list, hbuf, y, se, s)
               : launch_gemv_typed<uint16_t, false>(la, xb, units, chunk_len, gates, count, list, hbuf, y, se, s);
}

}  // namespace bffn
