// Grouped-by-expert batch path (prefill-like batches through one layer).
//
// When many chunks go through the same layer, streaming each chunk's union
// (the chunk path) would re-read the layer once per chunk.  Here every
// (token, expert) pair with a non-zero gate is grouped by expert and each
// expert's weights are read once for all of its tokens, in LDS-tiled MFMA
// GEMMs (the outer loop over active experts with a batched product inside,
// BlockFFN write-up §7, taken to the whole batch):
//
//   plan:    per-expert pair counts, pair offsets and tile offsets (one block)
//   fill:    per expert, its tokens in ascending order, their gates, and
//            pair_idx[t][i] for the combine (one block per expert)
//   up:      H'[p] = g_p * Swish(x[t_p] W_in[i]^T), bf16, grouped GEMM with
//            gathered token rows
//   down:    Part[p] = H'[p] W_out[i]^T, bf16 per-pair partial rows
//   combine: y[t] = sum over the token's experts in ascending order of
//            Part[pair_idx[t][i]], fp32 (no atomics; deterministic)
//
// The GEMM tile is 64 tokens x 128 outputs x 64 k on 256 threads (2 x 2
// waves of 32 x 64, v_mfma_f32_16x16x32_bf16); global rows are loaded as
// whole 128-byte lines and written to LDS with an XOR swizzle of the 16-byte
// chunk index so the MFMA operand reads spread over the banks.
#include "bffn_internal.h"

namespace bffn {
namespace {

constexpr int GBM = 64, GBN = 128, GBK = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte chunk position inside a 128-byte LDS row.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// ---- plan: counts, pair offsets, tile offsets ----
__global__ __launch_bounds__(1024) void group_plan_kernel(const float* __restrict__ gates, int64_t T, int E,
                                                          int n_tiles_up, int n_tiles_down,
                                                          int64_t* __restrict__ pair_off,
                                                          int64_t* __restrict__ tile_up,
                                                          int64_t* __restrict__ tile_down) {
  __shared__ unsigned int cnt[128];
  const int tid = threadIdx.x;
  for (int i = tid; i < 128; i += 1024) cnt[i] = 0;
  __syncthreads();
  for (int64_t idx = tid; idx < T * E; idx += 1024)
    if (gates[idx] > 0.f) atomicAdd(&cnt[idx % E], 1u);
  __syncthreads();
  if (tid == 0) {
    int64_t p = 0, tu = 0, td = 0;
    for (int i = 0; i < E; ++i) {
      pair_off[i] = p;
      tile_up[i] = tu;
      tile_down[i] = td;
      const int64_t mt = (cnt[i] + GBM - 1) / GBM;
      p += cnt[i];
      tu += mt * n_tiles_up;
      td += mt * n_tiles_down;
    }
    pair_off[E] = p;
    tile_up[E] = tu;
    tile_down[E] = td;
  }
}

// ---- fill: one block per expert, tokens in ascending order ----
__global__ __launch_bounds__(kBlock) void group_fill_kernel(const float* __restrict__ gates, int64_t T, int E,
                                                            const int64_t* __restrict__ pair_off,
                                                            int32_t* __restrict__ pair_tok,
                                                            float* __restrict__ pair_gate,
                                                            int32_t* __restrict__ pair_idx) {
  __shared__ int wave_cnt[4];
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t base = pair_off[i];
  for (int64_t t0 = 0; t0 < T; t0 += kBlock) {
    const int64_t t = t0 + threadIdx.x;
    const float gv = t < T ? gates[t * E + i] : 0.f;
    const bool on = gv > 0.f;
    const uint64_t bal = __ballot(on);
    if (lane == 0) wave_cnt[w] = __popcll(bal);
    __syncthreads();
    int before = 0;
    for (int ww = 0; ww < w; ++ww) before += wave_cnt[ww];
    const int total = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    if (on) {
      const int64_t p = base + before +
                        (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      pair_tok[p] = (int32_t)t;
      pair_gate[p] = gv;
      pair_idx[t * E + i] = (int32_t)p;
    }
    base += total;
    __syncthreads();
  }
}

// ---- grouped GEMM: C[p][n] = sum_k A[row(p)][k] B_i[n][k] over each expert's pairs ----
struct GemmArgs {
  const uint16_t* a;          // up: x [T][K]; down: hidden [P][K]
  const int32_t* a_tok;       // up: token of each pair; down: nullptr (row = pair)
  const uint16_t* b;          // [E][N][K] weights
  const int64_t* pair_off;    // [E + 1]
  const int64_t* tile_off;    // [E + 1]
  const float* pair_gate;     // up epilogue gates; nullptr for down
  uint16_t* out;              // [P][N] bf16
  int K, N, E;
};

template <bool UP>
__global__ __launch_bounds__(kBlock) void grouped_gemm_kernel(GemmArgs ga) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][GBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][GBN * 128];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m = lane & 15, g = lane >> 4;
  const int K = ga.K, N = ga.N, E = ga.E;
  const int n_ntiles = N / GBN;
  const int64_t total = ga.tile_off[E];
  // XCD-aware persistent striding: each XCD walks one contiguous range of
  // tiles, so the tiles sharing an expert's weight block share an L2.
  const int64_t nb = gridDim.x;
  const int64_t per_xcd_blocks = nb / kXcds;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int64_t local = blockIdx.x / kXcds;
  const int64_t span = (total + kXcds - 1) / kXcds;
  const int64_t t_begin = xcd * span, t_end = t_begin + span < total ? t_begin + span : total;

  for (int64_t tt = t_begin + local; tt < t_end; tt += per_xcd_blocks) {
    int lo = 0, hi = E - 1;  // last expert whose tile offset <= tt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ga.tile_off[mid] <= tt) lo = mid; else hi = mid - 1;
    }
    const int i = lo;
    const int64_t p0 = ga.pair_off[i];
    const int n_i = (int)(ga.pair_off[i + 1] - p0);
    const int m_tiles = (n_i + GBM - 1) / GBM;
    const int64_t local_t = tt - ga.tile_off[i];
    const int nt = (int)(local_t / m_tiles), mt = (int)(local_t % m_tiles);
    const int m0 = mt * GBM, n0 = nt * GBN;
    (void)n_ntiles;

    // global source rows of this thread's load slots
    const uint16_t* a_src[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = (tid + j * kBlock) >> 3;
      const int pr = m0 + r < n_i ? m0 + r : n_i - 1;  // rows past the group repeat a valid row
      const int64_t row = UP ? (int64_t)ga.a_tok[p0 + pr] : p0 + pr;
      a_src[j] = ga.a + row * K + ((tid + j * kBlock) & 7) * 8;
    }
    const uint16_t* b_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid + j * kBlock) >> 3;
      b_src[j] = ga.b + ((int64_t)i * N + n0 + r) * K + ((tid + j * kBlock) & 7) * 8;
    }
    u32x4 ra[2], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) ra[j] = *reinterpret_cast<const u32x4*>(a_src[j] + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) rb[j] = *reinterpret_cast<const u32x4*>(b_src[j] + k0);
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = tid + j * kBlock, r = c >> 3;
        *reinterpret_cast<u32x4*>(&lds_a[buf][r * 128 + swz(r, c & 7) * 16]) = ra[j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = tid + j * kBlock, r = c >> 3;
        *reinterpret_cast<u32x4*>(&lds_b[buf][r * 128 + swz(r, c & 7) * 16]) = rb[j];
      }
    };

    f32x4 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ksteps = K / GBK;
    gload(0);
    swrite(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < ksteps) gload((ks + 1) * GBK);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 av[2], bv[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int r = wm * 32 + a * 16 + m;
          av[a] = *reinterpret_cast<const u32x4*>(&lds_a[cur][r * 128 + swz(r, kk * 4 + g) * 16]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = wn * 64 + b * 16 + m;
          bv[b] = *reinterpret_cast<const u32x4*>(&lds_b[cur][r * 128 + swz(r, kk * 4 + g) * 16]);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[a]), as_bf16x8(bv[b]), acc[a][b], 0, 0, 0);
      }
      if (ks + 1 < ksteps) swrite(cur ^ 1);
      __syncthreads();
    }

    // D layout: lane (m, g) holds rows 4 g + r of column m of each 16 x 16 tile
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 32 + a * 16 + 4 * g + r;
        if (row >= n_i) continue;
        const int64_t p = p0 + row;
        const float gv = UP ? ga.pair_gate[p] : 1.f;
        uint16_t* orow = ga.out + p * N + n0 + wn * 64 + m;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float v = UP ? gv * swish(acc[a][b][r]) : acc[a][b][r];
          orow[b * 16] = (uint16_t)f32_to_bf16(v);
        }
      }
    }
  }
}

// ---- combine: y[t] = sum over active experts (ascending) of Part[pair_idx[t][i]] ----
__global__ __launch_bounds__(kBlock) void combine_kernel(const float* __restrict__ gates,
                                                         const int32_t* __restrict__ pair_idx,
                                                         const uint16_t* __restrict__ part, int64_t T, int E, int d,
                                                         float* __restrict__ y) {
  __shared__ int32_t plist[128];
  __shared__ int nlist;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const bool on0 = tid < E && gates[t * E + tid] > 0.f;
    const bool on1 = tid + 64 < E && gates[t * E + tid + 64] > 0.f;
    const uint64_t b0 = __ballot(on0), b1 = __ballot(on1);
    const int n0 = __popcll(b0);
    const int r0 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b0, 0u));
    const int r1 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b1, 0u));
    if (on0) plist[r0] = pair_idx[t * E + tid];
    if (on1) plist[n0 + r1] = pair_idx[t * E + tid + 64];
    if (tid == 0) nlist = n0 + __popcll(b1);
  }
  __syncthreads();
  const int n = nlist;
  for (int c0 = tid * 8; c0 < d; c0 += kBlock * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(part + (int64_t)plist[s] * d + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_lo(v[q]);
        acc[2 * q + 1] += bf16_hi(v[q]);
      }
    }
    f32x4* yo = reinterpret_cast<f32x4*>(y + t * d + c0);
    yo[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    yo[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

size_t r256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

bool grouped_supported(int d, int de, int dtype) {
  return dtype == BLOCKFFN_BF16 && d % GBN == 0 && de % GBN == 0;
}

// Workspace: offsets, pair arrays (capacity T*E pairs), pair_idx, hidden and partial rows.
size_t grouped_workspace_bytes(int64_t T, int E, int d, int de) {
  const size_t P = (size_t)T * E;
  return 3 * r256(sizeof(int64_t) * (E + 1)) + r256(4 * P) + r256(4 * P) + r256(4 * P) + r256(2 * P * de) +
         r256(2 * P * d);
}

hipError_t launch_forward_grouped(const LayerArgs& la, const uint16_t* x, int64_t T, const float* gates,
                                  void* workspace, float* y, const StageEvents& se, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int E = la.E, d = la.d, de = la.de;
  const size_t P = (size_t)T * E;
  char* ws = static_cast<char*>(workspace);
  auto take = [&](size_t bytes) {
    char* p = ws;
    ws += r256(bytes);
    return p;
  };
  int64_t* pair_off = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (E + 1)));
  int64_t* tile_up = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (E + 1)));
  int64_t* tile_down = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (E + 1)));
  int32_t* pair_tok = reinterpret_cast<int32_t*>(take(4 * P));
  float* pair_gate = reinterpret_cast<float*>(take(4 * P));
  int32_t* pair_idx = reinterpret_cast<int32_t*>(take(4 * P));
  uint16_t* hid = reinterpret_cast<uint16_t*>(take(2 * P * de));
  uint16_t* part = reinterpret_cast<uint16_t*>(take(2 * P * d));

  group_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(gates, T, E, de / GBN, d / GBN, pair_off, tile_up, tile_down);
  group_fill_kernel<<<dim3(E), dim3(kBlock), 0, s>>>(gates, T, E, pair_off, pair_tok, pair_gate, pair_idx);
  int dev = 0, cus = 0, per_cu_up = 0, per_cu_dn = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_up, grouped_gemm_kernel<true>, kBlock, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_dn, grouped_gemm_kernel<false>, kBlock, 0);
  if (e != hipSuccess) return e;
  // the persistent grids are a multiple of the XCD count, so every XCD gets the same number of blocks
  const int64_t grid_up = (int64_t)cus * (per_cu_up > 0 ? per_cu_up : 1) / kXcds * kXcds;
  const int64_t grid_dn = (int64_t)cus * (per_cu_dn > 0 ? per_cu_dn : 1) / kXcds * kXcds;

  se.record(0, s);
  GemmArgs up{x, pair_tok, static_cast<const uint16_t*>(la.w_in), pair_off, tile_up, pair_gate, hid, d, de, E};
  grouped_gemm_kernel<true><<<dim3((unsigned)(grid_up > 0 ? grid_up : kXcds)), dim3(kBlock), 0, s>>>(up);
  se.record(1, s);
  GemmArgs dn{hid, nullptr, static_cast<const uint16_t*>(la.w_out), pair_off, tile_down, nullptr, part, de, d, E};
  grouped_gemm_kernel<false><<<dim3((unsigned)(grid_dn > 0 ? grid_dn : kXcds)), dim3(kBlock), 0, s>>>(dn);
  se.record(2, s);
  combine_kernel<<<dim3((unsigned)T), dim3(kBlock), 0, s>>>(gates, pair_idx, part, T, E, d, y);
  se.record(3, s);
  return hipGetLastError();
}

}  // namespace bffn
