// Layer backward over one batch through one layer, grouped by expert.
//
// The chain rule through the forward (BlockFFN write-up, lsdiaocha.cn, §2:
// the ReLU + RMSNorm router is differentiable end to end; non-gated Swish
// experts), for a scalar loss with dL/dy = dy.  Per token t with
// r = (ms + eps)^(-1/2), a = ReLU(z), g = s a r, and every active pair (z > 0):
//
//   u = W_in[i] x,  h = Swish(u),  q = W_out[i]^T dy,  dg_i = q . h
//   du = g_i q Swish'(u),  Swish'(u) = sig (1 + u (1 - sig))
//   dW_out[i] += dy (g_i h)^T,  dW_in[i] += du x^T,  dx += W_in[i]^T du
//   ds_i += dg_i a_i r,  dr = sum_i dg_i s_i a_i,  dms = -dr r^3 / 2
//   dz_i = dg_i s_i r + dms 2 a_i / E,  db += dz,  dW_r += dz x^T,  dx += W_r^T dz
//
// Active pairs are grouped by expert (the forward's pair planning, on
// z > 0), and the per-expert products run as LDS-tiled MFMA GEMMs:
//
//   prep:    g and r per token (as the router computes them), dy -> bf16
//            (the products that contract over a weight's row index, dY W_out
//            and dU W_in, read the weight as it lies, by LDS transpose loads)
//   pair:    U = X_p W_in[i]^T and Q = dY_p W_out[i] in one pass over k = d;
//            epilogue: dU = g Q Swish'(U), HG = g Swish(U) (bf16), and the
//            partial dg = sum over the tile's hidden units of Q Swish(U)
//   router:  dz, ds terms per token; then db, ds by sums over tokens
//   weights: dW_out[i] = dY_p^T HG_p (computed as HG_p^T dY_p, stored
//            transposed), dW_in[i] = dU_p^T X_p and dW_r = dZ^T X (over token
//            ranges, then summed in order), each a sum over pairs (tokens) in
//            fp32 by a grouped GEMM that contracts over pairs (pair-major rows
//            in LDS, MFMA operands by transpose loads)
//   dx:      Part = dU W_in[i] + dz_i W_r[i] per pair (the forward's down
//            GEMM, reading W_in k-major, its products starting from the
//            router term), then per token the sum over its active experts,
//            ascending; with an extra router gradient, the inactive experts'
//            dz_i W_r[i] first, as one product, and the sum added onto it
//
// No atomics: every output element has one writer and a fixed summation
// order, so the result is bit-reproducible.
#include "grouped_kernels.h"

namespace bffn {
namespace {

constexpr int TBM = 128, TBN = 256, TBK = 32;  // transposing GEMM tile (TBK pairs per step)
constexpr int kRouterPad = 128;               // dZ rows padded to 128 experts (bf16)
constexpr int kRouterSplits = 16;             // dW_r: token range split for parallelism

// ---- prep: gates and 1/RMS as the router computes them; dy -> bf16 ----
// One block per token: wave 0 does the router quantities, all threads convert dy.
__global__ __launch_bounds__(kBlock) void bwd_prep_kernel(const float* __restrict__ z,
                                                          const float* __restrict__ rms_scale, float eps, int64_t T,
                                                          int E, int d, const float* __restrict__ dy,
                                                          float* __restrict__ g_out, float* __restrict__ r_out,
                                                          uint16_t* __restrict__ dyb, int64_t* __restrict__ all_off) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const bool v0 = lane < E, v1 = lane + 64 < E;
    const float z0 = v0 ? z[t * E + lane] : 0.f, z1 = v1 ? z[t * E + lane + 64] : 0.f;
    const float a0 = z0 > 0.f ? z0 : 0.f, a1 = z1 > 0.f ? z1 : 0.f;
    const float ms = wave_sum(a0 * a0 + a1 * a1) / (float)E;
    const float inv = 1.0f / sqrtf(ms + eps);
    const float s0 = (v0 && rms_scale) ? rms_scale[lane] : 1.f, s1 = (v1 && rms_scale) ? rms_scale[lane + 64] : 1.f;
    if (v0) g_out[t * E + lane] = s0 * a0 * inv;
    if (v1) g_out[t * E + lane + 64] = s1 * a1 * inv;
    if (lane == 0) r_out[t] = inv;
  }
  if (t == 0 && tid >= 64 && tid <= 64 + kRouterSplits)  // token range of each dW_r split
    all_off[tid - 64] = T * (tid - 64) / kRouterSplits;
  for (int c = tid * 8; c < d; c += kBlock * 8) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(dy + t * d + c);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(dy + t * d + c + 4);
    u32x4 o;
    o[0] = pack2_bf16(v0[0], v0[1]);
    o[1] = pack2_bf16(v0[2], v0[3]);
    o[2] = pack2_bf16(v1[0], v1[1]);
    o[3] = pack2_bf16(v1[2], v1[3]);
    *reinterpret_cast<u32x4*>(dyb + t * d + c) = o;
  }
}

// ---- pair: U and Q for a kPairRows (96)-pair x 128-hidden tile, fused epilogue ----
// A 64-wide k step stages 96 gathered x rows, 96 gathered dy rows and 128
// W_in rows (128 bytes each, chunk-swizzled), and 64 k-major W_out rows of the
// tile's 128 hidden units (256 bytes each), read back by transpose loads.  One
// LDS buffer (56 KiB) lets two blocks share a CU, with the registers capped for
// two waves per SIMD (a few spill; one block per CU without spills measured
// 30% slower); the registers hold the next step while this one is multiplied.
constexpr int kPairRows = 96;                     // pairs per tile: each wave 48 (three 16-pair groups)
constexpr int kPairStage = kPairRows * 8 / kBlock;  // 16-byte x (and dy) chunks per thread and step
struct PairArgs {
  const uint16_t* x;        // [T][d]
  const uint16_t* dy;       // [T][d] bf16
  const int32_t* pair_tok;
  const float* pair_gate;   // g of each pair
  const uint16_t* w_in;     // [E][de][d]
  const uint16_t* w_out;    // [E][d][de]
  const int64_t* pair_off;  // [E + 1]
  const int64_t* tile_off;  // [E + 1]
  uint16_t* du;             // [P][de] bf16
  uint16_t* hg;             // [P][de] bf16
  float* dgp;               // [P][de / 128]
  int d, de, E;
};

__global__ __launch_bounds__(kBlock, 2) void bwd_pair_kernel(PairArgs pa) {
  static_assert(kPairStage * kBlock == kPairRows * 8 && kPairRows % 32 == 0, "pair tile staging");
  __shared__ __attribute__((aligned(16))) uint8_t lds_x[kPairRows * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_y[kPairRows * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_wi[GBN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_wo[GBK * GBN * 2];  // k-major: 64 rows of 128 hidden units
  __shared__ float dg_part[2][kPairRows];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m = lane & 15, g = lane >> 4;
  const int K = pa.d, N = pa.de, E = pa.E;
  const int n_nt = N / GBN;
  const int64_t total = pa.tile_off[E];
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
      if (pa.tile_off[mid] <= tt) lo = mid; else hi = mid - 1;
    }
    const int i = lo;
    const int64_t p0 = pa.pair_off[i];
    const int n_i = (int)(pa.pair_off[i + 1] - p0);
    const int m_tiles = (n_i + kPairRows - 1) / kPairRows;
    const int64_t local_t = tt - pa.tile_off[i];
    const int nt = (int)(local_t / m_tiles), mt = (int)(local_t % m_tiles);
    const int m0 = mt * kPairRows, n0 = nt * GBN;

    const uint16_t* x_src[kPairStage];
    const uint16_t* y_src[kPairStage];
#pragma unroll
    for (int j = 0; j < kPairStage; ++j) {
      const int r = (tid + j * kBlock) >> 3;
      const int pr = m0 + r < n_i ? m0 + r : n_i - 1;  // rows past the group repeat a valid row
      const int64_t tok = pa.pair_tok[p0 + pr];
      x_src[j] = pa.x + tok * K + ((tid + j * kBlock) & 7) * 8;
      y_src[j] = pa.dy + tok * K + ((tid + j * kBlock) & 7) * 8;
    }
    const uint16_t* wi_src[4];
    const uint16_t* wo_src[4];  // W_out[i] rows k (d) of the tile's 128 hidden units: 16 chunks per row
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + j * kBlock;
      wi_src[j] = pa.w_in + ((int64_t)i * N + n0 + (c >> 3)) * K + (c & 7) * 8;
      wo_src[j] = pa.w_out + ((int64_t)i * K + (c >> 4)) * N + n0 + (c & 15) * 8;
    }
    u32x4 rx[kPairStage], ry[kPairStage], rwi[4], rwo[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < kPairStage; ++j) {
        rx[j] = *reinterpret_cast<const u32x4*>(x_src[j] + k0);
        ry[j] = *reinterpret_cast<const u32x4*>(y_src[j] + k0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rwi[j] = *reinterpret_cast<const u32x4*>(wi_src[j] + k0);
        rwo[j] = *reinterpret_cast<const u32x4*>(wo_src[j] + (int64_t)k0 * N);
      }
    };
    auto swrite = [&]() {
#pragma unroll
      for (int j = 0; j < kPairStage; ++j) {
        const int c = tid + j * kBlock;
        *reinterpret_cast<u32x4*>(&lds_x[lds_off<128>(c >> 3, c & 7)]) = rx[j];
        *reinterpret_cast<u32x4*>(&lds_y[lds_off<128>(c >> 3, c & 7)]) = ry[j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = tid + j * kBlock;
        *reinterpret_cast<u32x4*>(&lds_wi[lds_off<128>(c >> 3, c & 7)]) = rwi[j];
        *reinterpret_cast<u32x4*>(&lds_wo[tg_off(c >> 4, c & 15)]) = rwo[j];
      }
    };

    constexpr int PA = kPairRows / 32;  // 16-pair groups per wave
    f32x4 au[4][PA], aq[4][PA];       // [hidden stripe b][pair group a]
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int a = 0; a < PA; ++a) au[b][a] = aq[b][a] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ksteps = K / GBK;
    // one LDS buffer (two blocks fit on a CU): the registers hold step ks + 1
    // while step ks is multiplied; a fence-free barrier after the products
    // frees the buffer without waiting for those loads
    gload(0);
    for (int ks = 0; ks < ksteps; ++ks) {
      swrite();
      __syncthreads();
      if (ks + 1 < ksteps) gload((ks + 1) * GBK);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 vx[PA], vy[PA], vwi[4], vwo[4];
        tg_operands(lds_wo + kk * 32 * 256, wn * 64, lane, vwo);
#pragma unroll
        for (int a = 0; a < PA; ++a) {
          const int off = lds_off<128>(wm * (16 * PA) + a * 16 + m, kk * 4 + g);
          vx[a] = *reinterpret_cast<const u32x4*>(&lds_x[off]);
          vy[a] = *reinterpret_cast<const u32x4*>(&lds_y[off]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int off = lds_off<128>(wn * 64 + b * 16 + m, kk * 4 + g);
          vwi[b] = *reinterpret_cast<const u32x4*>(&lds_wi[off]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int a = 0; a < PA; ++a) {
            au[b][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vwi[b]), as_bf16x8(vx[a]), au[b][a], 0, 0, 0);
            aq[b][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vwo[b]), as_bf16x8(vy[a]), aq[b][a], 0, 0, 0);
          }
      }
      block_barrier_no_fence();
    }

    // lane (m, g): pair wm*16 PA + a*16 + m, hidden units n0 + wn*64 + b*16 + 4g .. +3
#pragma unroll
    for (int a = 0; a < PA; ++a) {
      const int row = m0 + wm * (16 * PA) + a * 16 + m;
      const bool valid = row < n_i;
      const float gv = valid ? pa.pair_gate[p0 + row] : 0.f;
      float dgl = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float du4[4], hg4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float u = au[b][a][r], q = aq[b][a][r];
          const float sig = 1.0f / (1.0f + __expf(-u));
          const float h = u * sig;
          dgl += q * h;
          du4[r] = gv * q * sig * (1.0f + u * (1.0f - sig));
          hg4[r] = gv * h;
        }
        if (valid) {
          const int64_t o = (p0 + row) * N + n0 + wn * 64 + b * 16 + 4 * g;
          *reinterpret_cast<u32x2*>(pa.du + o) = pack4_bf16(du4[0], du4[1], du4[2], du4[3]);
          *reinterpret_cast<u32x2*>(pa.hg + o) = pack4_bf16(hg4[0], hg4[1], hg4[2], hg4[3]);
        }
      }
      // the four lane groups g hold the same pair: sum them, then the two wn waves via LDS
      dgl += __shfl_xor(dgl, 16, kWave);
      dgl += __shfl_xor(dgl, 32, kWave);
      if (g == 0) dg_part[wn][wm * (16 * PA) + a * 16 + m] = dgl;
    }
    __syncthreads();
    if (tid < kPairRows && m0 + tid < n_i) pa.dgp[(p0 + m0 + tid) * n_nt + nt] = dg_part[0][tid] + dg_part[1][tid];
    // (dg_part is next written after this tile's k loop, which has barriers)
  }
}

// ---- router backward per token: dz (fp32 and bf16, and per pair for the dx rows), ds terms;
// with an extra router gradient also the inactive experts' dz (bf16, active ones 0) ----
// Wave w of a block handles token 4 blockIdx + w; lane l experts l and l + 64.
__global__ __launch_bounds__(kBlock) void bwd_router_kernel(const float* __restrict__ z,
                                                            const float* __restrict__ rms_scale,
                                                            const float* __restrict__ r_tok,
                                                            const int32_t* __restrict__ pair_idx,
                                                            const float* __restrict__ dgp, int n_nt, int64_t T, int E,
                                                            const float* __restrict__ dz_extra,
                                                            float* __restrict__ dz, uint16_t* __restrict__ dzb,
                                                            float* __restrict__ dsc, float* __restrict__ pair_dz,
                                                            uint16_t* __restrict__ dz_off) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float r = r_tok[t];
  float dgv[2], av[2], sv[2];
  bool on[2];
  int64_t pv[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    const bool v = i < E;
    const float zi = v ? z[t * E + i] : 0.f;
    on[h] = zi > 0.f;
    av[h] = on[h] ? zi : 0.f;
    sv[h] = (v && rms_scale) ? rms_scale[i] : 1.f;
    float dg = 0.f;
    if (on[h]) {
      const int64_t p = pair_idx[t * E + i];
      pv[h] = p;
      for (int q = 0; q < n_nt; ++q) dg += dgp[p * n_nt + q];
    }
    dgv[h] = dg;
  }
  const float dr = wave_sum(dgv[0] * sv[0] * av[0] + dgv[1] * sv[1] * av[1]);
  const float dms = -0.5f * dr * r * r * r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    const float da = dgv[h] * sv[h] * r + dms * 2.f * av[h] / (float)E;
    float dzi = on[h] ? da : 0.f;
    if (dz_extra && i < E) dzi += dz_extra[t * E + i];  // every (token, expert), active or not
    if (i < E) {
      dz[t * E + i] = dzi;
      dsc[t * E + i] = dgv[h] * av[h] * r;
    }
    if (on[h]) pair_dz[pv[h]] = dzi;
    dzb[t * kRouterPad + i] = (uint16_t)f32_to_bf16(i < E ? dzi : 0.f);
    if (dz_off) dz_off[t * kRouterPad + i] = (uint16_t)f32_to_bf16(i < E && !on[h] ? dzi : 0.f);
  }
}

// ---- db[i] = sum_t dz[t][i], ds[i] = sum_t dsc[t][i]: one block per expert ----
__global__ __launch_bounds__(kBlock) void bwd_reduce_kernel(const float* __restrict__ dz, const float* __restrict__ dsc,
                                                            int64_t T, int E, float* __restrict__ db,
                                                            float* __restrict__ ds) {
  __shared__ float sb[kBlock], ss[kBlock];
  const int i = blockIdx.x, tid = threadIdx.x;
  float b = 0.f, s = 0.f;
  for (int64_t t = tid; t < T; t += kBlock) {
    b += dz[t * E + i];
    s += dsc[t * E + i];
  }
  sb[tid] = b;
  ss[tid] = s;
  __syncthreads();
  for (int off = kBlock / 2; off > 0; off >>= 1) {
    if (tid < off) {
      sb[tid] += sb[tid + off];
      ss[tid] += ss[tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    db[i] = sb[0];
    ds[i] = ss[0];
  }
}

// ---- dW_r = sum of the split partials, in split order ----
__global__ __launch_bounds__(kBlock) void bwd_router_sum_kernel(const float* __restrict__ part, int64_t n,
                                                                float* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (k >= n) return;
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kRouterSplits; ++q) s += part[q * n + k];
  out[k] = s;
}

// ---- transposing grouped GEMM: C_g[m][n] = sum over pairs p of group g of A[p0 + p][m] B[rb(p)][n] ----
struct TGemmArgs {
  const uint16_t* a;        // pair rows of M (or more) bf16 elements, row stride lda: pair p is row p0 + p
  int64_t lda;
  const uint16_t* b;        // rows of N (or more) bf16 elements, row stride ldb
  int64_t ldb;
  const int32_t* b_rows;    // B row of pair p (nullptr: row p0 + p)
  const int64_t* grp_off;   // [G + 1] pair ranges (p0 = grp_off[g])
  float* c;                 // group g at c + g * c_stride: C[m][n] at m * ldc + n, or at n * ldc + m (c_nm)
  int64_t ldc, c_stride;
  int G, M, M_valid, N;     // M a multiple of TBM, N of 128
  bool c_nm;
};

// A tile is 128 rows of A's side by 256 columns of B's side, the gathered
// operand, so that every gathered B row piece (512 bytes) serves 128 rows and
// every A piece 256 columns.  The kernel is bound by the cache lines a CU keeps
// in flight: this tile requests 0.75 of the lines per product that a 128 x
// 128 tile does.
//
// The operands lie in memory pair-major (a pair's elements of m, or of n, are
// one row piece), and the contraction runs over pairs.  A step of TBK = 32
// pairs reaches LDS untouched, by DMA (global_load_lds, 16 bytes per lane; the
// gathered rows too, every lane with its own row), into a block-shared ring of
// kTgRing slots, kTgDepth steps ahead of the one being multiplied.  A slot
// holds the step's 32 A rows, then B's two 128-column halves as 32 rows each,
// all rows of 256 bytes; LDS row r holds pair r of the step.  Each wave moves
// the rows of 8 pairs.  The MFMA operands (8 consecutive pairs of one m or n
// per lane) are read with transpose loads (tg_operands).
//
// The B row indices come by DMA too, each wave its own 8 per step into its
// own index ring, issued kTgDepth steps before the rows that use them; the
// in-order vmcnt wait for a step's rows therefore also covers the indices of
// the step kTgDepth later, and every wait is a constant.  Pairs past the group
// read a row of zeros; a tile whose second column half lies past N loads the
// first half again there and stores only the first.
constexpr int kTgDepth = 2;
constexpr int kTgRing = kTgDepth + 1;
constexpr int kTgIdxSlots = 4;                        // > kTgDepth: indices in flight + the one being read
constexpr int kTgHalfBytes = TBK * 256;               // 32 rows of 128 bf16
constexpr int kTgSlotBytes = 3 * kTgHalfBytes;        // A rows, B columns 0..127, B columns 128..255
constexpr int kTgDmaPerWave = 6;                      // per step: 8 pairs x (1 A + 2 B) row pieces of 256 bytes
constexpr int kTgLoadsPerStep = kTgDmaPerWave + 1;    // + the index DMA

__device__ __attribute__((aligned(256))) const uint16_t kTgZeroRow[128] = {};

// 76 KiB of LDS and at most 256 registers: two blocks (waves per SIMD) per CU.
__global__ __launch_bounds__(kBlock, 2) void tgemm_kernel(TGemmArgs ta) {
  static_assert(TBM == 128 && TBN == 256 && TBK == 32, "tile geometry");
  static_assert((kBlock / kWave) * 8 == TBK && kTgDmaPerWave * 1024 == 8 * 3 * 256 && kTgIdxSlots > kTgDepth,
                "ring geometry");
  // one LDS object, the step ring then each wave's index ring (with the
  // index ring a separate object, the compiler waits for every DMA in flight
  // before reading it)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTgRing * kTgSlotBytes + (kBlock / kWave) * kTgIdxSlots * 256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;  // compute: rows wm*64 .. +63 against B's column half wn
  const int m16 = lane & 15, g = lane >> 4;
  uint8_t* my_idx = lds + kTgRing * kTgSlotBytes + w * kTgIdxSlots * 256;
  const int mtn = ta.M / TBM, ntn = (ta.N + TBN - 1) / TBN;
  const int64_t total = (int64_t)ta.G * mtn * ntn;
  const int64_t nb = gridDim.x;
  const int64_t per_xcd_blocks = nb / kXcds;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int64_t local = blockIdx.x / kXcds;
  const int64_t span = (total + kXcds - 1) / kXcds;
  const int64_t t_begin = xcd * span, t_end = t_begin + span < total ? t_begin + span : total;

  for (int64_t tt = t_begin + local; tt < t_end; tt += per_xcd_blocks) {
    const int grp = (int)(tt / (mtn * ntn));
    const int rem = (int)(tt % (mtn * ntn));
    const int m0 = (rem / ntn) * TBM, n0 = (rem % ntn) * TBN;
    const int64_t p0 = ta.grp_off[grp];
    const int64_t n_p = ta.grp_off[grp + 1] - p0;
    const int ksteps = (int)((n_p + TBK - 1) / TBK);
    const bool hi_ok = n0 + 128 < ta.N;  // the tile's second column half exists

    // index DMA of a step: lane l fetches the B row of pair 8 w + ((l >> 1) & 3) + 4 (l & 1), so that
    // the two pairs of lane group g (8 w + g, 8 w + 4 + g) are words 2 g and 2 g + 1 (an operand
    // without a row array fetches a valid dummy word)
    auto issue_idx = [&](int step) {
      const int st = step < ksteps ? step : ksteps - 1;
      int64_t p = (int64_t)st * TBK + 8 * w + ((lane >> 1) & 3) + 4 * (lane & 1);
      p = p < n_p ? p : n_p - 1;
      const int32_t* s = ta.b_rows ? ta.b_rows + p0 + p : reinterpret_cast<const int32_t*>(ta.grp_off);
      dma4(reinterpret_cast<const float*>(s), my_idx + (step % kTgIdxSlots) * 256);
    };
    // row DMA of a step: instruction q of each part moves LDS rows 8 w + 4 q .. +3 (pairs 8 w + 4 q + g)
    auto issue_rows = [&](int step) {
      const int st = step < ksteps ? step : ksteps - 1;
      uint8_t* dst = lds + (step % kTgRing) * kTgSlotBytes + (8 * w) * 256;
      const u32x2 rid = *reinterpret_cast<const u32x2*>(my_idx + (step % kTgIdxSlots) * 256 + 8 * g);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = 8 * w + 4 * q + g;
        const int64_t p = (int64_t)st * TBK + r;
        const int gc = (lane & 15) ^ tg_swz(r);
        const bool in = p < n_p;
        dma16<kPolicyReuse>(in ? ta.a + (p0 + p) * ta.lda + m0 + gc * 8 : kTgZeroRow + gc * 8, dst + q * 1024);
        const int64_t row = ta.b_rows ? (int64_t)(int32_t)rid[q] : p0 + p;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = n0 + (h && hi_ok ? 128 : 0) + gc * 8;
          dma16<kPolicyReuse>(in ? ta.b + row * ta.ldb + col : kTgZeroRow + gc * 8,
                              dst + (1 + h) * kTgHalfBytes + q * 1024);
        }
      }
    };

    f32x4 acc[4][8];  // [A stripe sa][B stripe sb]
#pragma unroll
    for (int sa = 0; sa < 4; ++sa)
#pragma unroll
      for (int sb = 0; sb < 8; ++sb) acc[sa][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ksteps > 0) {  // (uniform)
      // indices of the first kTgDepth steps, then kTgDepth steps issued as
      // the loop issues them: indices kTgDepth steps ahead of their rows
#pragma unroll
      for (int s = 0; s < kTgDepth; ++s) issue_idx(s);
      wait_vmcnt<0>();
#pragma unroll
      for (int s = 0; s < kTgDepth; ++s) {
        issue_idx(s + kTgDepth);
        issue_rows(s);
      }
    }
    for (int s = 0; s < ksteps; ++s) {
      wait_vmcnt<kTgLoadsPerStep * (kTgDepth - 1)>();  // this wave's rows of step s (and older indices)
      block_barrier_no_fence();                        // ... everyone's; step s - 1's slot is free
      issue_idx(s + 2 * kTgDepth);
      issue_rows(s + kTgDepth);
      const uint8_t* buf = lds + (s % kTgRing) * kTgSlotBytes;
      u32x4 av[4], bv0[4], bv1[4];
      tg_operands(buf, wm * 64, lane, av);
      tg_operands(buf + (1 + wn) * kTgHalfBytes, 0, lane, bv0);
      tg_operands(buf + (1 + wn) * kTgHalfBytes, 64, lane, bv1);
#pragma unroll
      for (int sa = 0; sa < 4; ++sa)
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          acc[sa][sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[sa]), as_bf16x8(bv0[sb]), acc[sa][sb], 0,
                                                                0, 0);
          acc[sa][4 + sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[sa]), as_bf16x8(bv1[sb]),
                                                                    acc[sa][4 + sb], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the tile's last DMAs (repeats) land and every wave is done with both
    // rings before the next tile refills them
    wait_vmcnt<0>();
    __syncthreads();
    // D: lane (m16, g) holds rows 4 g + r of column m16 of each 16 x 16 tile
    if (wn == 1 && !hi_ok) continue;  // (uniform per wave; no barrier follows before the next tile's)
    float* cg = ta.c + (int64_t)grp * ta.c_stride;
    const int nb0 = n0 + wn * 128;
    if (ta.c_nm) {  // C[m][n] at n * ldc + m: a lane's four rows are one 16-byte store
#pragma unroll
      for (int sa = 0; sa < 4; ++sa) {
        const int mm = m0 + wm * 64 + sa * 16 + 4 * g;
        if (mm >= ta.M_valid) continue;
#pragma unroll
        for (int sb = 0; sb < 8; ++sb)
          *reinterpret_cast<f32x4*>(cg + (int64_t)(nb0 + sb * 16 + m16) * ta.ldc + mm) = acc[sa][sb];
      }
    } else {
#pragma unroll
      for (int sa = 0; sa < 4; ++sa)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mm = m0 + wm * 64 + sa * 16 + 4 * g + r;
          if (mm >= ta.M_valid) continue;
#pragma unroll
          for (int sb = 0; sb < 8; ++sb) cg[(int64_t)mm * ta.ldc + nb0 + sb * 16 + m16] = acc[sa][sb][r];
        }
    }
  }
}

// ---- dx[t][n] = sum over the inactive experts i of dz[t][i] W_r[i][n] (an extra router gradient
// reaches every expert; the active ones are in their pair rows) ----
// Block: 128 columns x 64 tokens.  The block's slice of W_r (every expert's 128 columns) sits in
// LDS as k-major rows and reaches the MFMA as operand A (16 columns) through transpose loads; the
// tokens' inactive dz rows (bf16, padded to kRouterPad with zeros) are operand B.  Wave w takes
// tokens 16 w .. +15 of the block's 64.
__global__ __launch_bounds__(kBlock) void bwd_router_dx_kernel(const uint16_t* __restrict__ w_r, int E,
                                                               const uint16_t* __restrict__ dz_off, int64_t T,
                                                               int d, float* __restrict__ dx) {
  constexpr int kSteps = kRouterPad / 32;
  __shared__ __attribute__((aligned(16))) uint8_t rows[kRouterPad * 256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 128;
  const int64_t t0 = (int64_t)blockIdx.y * 64 + 16 * w;
  const int64_t tb = t0 + m < T ? t0 + m : T - 1;  // (a repeated token's column is not stored)
  const int ksteps = (E + 31) / 32;
  u32x4 b[kSteps];
#pragma unroll
  for (int kk = 0; kk < kSteps; ++kk)
    b[kk] = *reinterpret_cast<const u32x4*>(dz_off + tb * kRouterPad + 32 * kk + 8 * g);
  // row i of the slice: W_r[i][n0 .. n0 + 127] (rows past E: zeros), 16-byte chunk q % 16 of row q / 16
#pragma unroll
  for (int j = 0; j < kRouterPad * 16 / kBlock; ++j) {
    const int q = tid + j * kBlock, r = q >> 4, c = q & 15;
    const u32x4 v = r < E ? *reinterpret_cast<const u32x4*>(w_r + (int64_t)r * d + n0 + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(rows + tg_off(r, c)) = v;
  }
  __syncthreads();
  f32x4 acc[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < ksteps; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 a[4];
      tg_operands<4>(rows + kk * 32 * 256, 64 * h, lane, a);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[4 * h + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[j]), as_bf16x8(b[kk]), acc[4 * h + j],
                                                                 0, 0, 0);
    }
  // lane (m, g): columns n0 + 16 s + 4 g .. +3 of token t0 + m
  if (t0 + m >= T) return;
#pragma unroll
  for (int s = 0; s < 8; ++s) *reinterpret_cast<f32x4*>(dx + (t0 + m) * d + n0 + 16 * s + 4 * g) = acc[s];
}

// ---- dx[t] = sum over active i (ascending) of Part[pair_idx[t][i]] (each row already holds its
// dz[t][i] W_r[i]), added onto the inactive experts' router term in dx when `accumulate` ----
__global__ __launch_bounds__(1024) void bwd_combine_kernel(const float* __restrict__ z,
                                                           const int32_t* __restrict__ pair_idx,
                                                           const uint16_t* __restrict__ part, int E,
                                                           int d, bool accumulate, float* __restrict__ dx) {
  __shared__ int32_t plist[128];
  __shared__ int nlist;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // pre-activations and pair slots load together (a slot is used only where z > 0)
    const float z0 = tid < E ? z[t * E + tid] : 0.f, z1 = tid + 64 < E ? z[t * E + tid + 64] : 0.f;
    const int32_t q0 = tid < E ? pair_idx[t * E + tid] : 0, q1 = tid + 64 < E ? pair_idx[t * E + tid + 64] : 0;
    const bool on0 = z0 > 0.f, on1 = z1 > 0.f;
    const uint64_t b0 = __ballot(on0), b1 = __ballot(on1);
    const int n0 = __popcll(b0);
    const int r0 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b0, 0u));
    const int r1 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b1, 0u));
    if (on0) plist[r0] = q0;
    if (on1) plist[n0 + r1] = q1;
    if (tid == 0) nlist = n0 + __popcll(b1);
  }
  __syncthreads();
  const int n = nlist;
  for (int c0 = tid * 8; c0 < d; c0 += blockDim.x * 8) {
    f32x4* o = reinterpret_cast<f32x4*>(dx + t * d + c0);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (accumulate) {
      const f32x4 r0 = o[0], r1 = o[1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = r0[q];
        acc[4 + q] = r1[q];
      }
    }
    // kCombineInFlight partial rows in flight, added in ascending expert order
    for (int s = 0; s < n; s += kCombineInFlight) {
      u32x4 v[kCombineInFlight];
#pragma unroll
      for (int u = 0; u < kCombineInFlight; ++u)
        v[u] = s + u < n ? load_part(part + (int64_t)plist[s + u] * d + c0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kCombineInFlight; ++u)
        if (s + u < n)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += bf16_lo(v[u][q]);
            acc[2 * q + 1] += bf16_hi(v[u][q]);
          }
    }
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

struct BwdLayout {
  int32_t* blk;
  int64_t *pair_off, *tile_up, *all_off;
  int32_t *pair_tok, *pair_idx;
  float *pair_gate, *g_b, *r_b, *dgp, *dz, *dsc, *wr_part, *pair_dz;
  uint16_t *dyb, *du, *hg, *dzb, *dz_off, *part;
  size_t bytes;
};

BwdLayout bwd_layout(char* base, int64_t T, int E, int d, int de) {
  const size_t P = (size_t)T * E;
  const int rows = plan_rows(T);
  const size_t nblk = ((size_t)T + rows - 1) / rows;
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += r256(bytes);
    return p;
  };
  L.blk = reinterpret_cast<int32_t*>(take(4 * nblk * E));
  L.pair_off = reinterpret_cast<int64_t*>(take(8 * (size_t)(E + 1)));
  L.tile_up = reinterpret_cast<int64_t*>(take(8 * (size_t)(E + 1)));
  L.all_off = reinterpret_cast<int64_t*>(take(8 * (kRouterSplits + 1)));
  L.wr_part = reinterpret_cast<float*>(take(4 * (size_t)kRouterSplits * E * d));
  L.pair_tok = reinterpret_cast<int32_t*>(take(4 * P));
  L.pair_gate = reinterpret_cast<float*>(take(4 * P));
  L.pair_idx = reinterpret_cast<int32_t*>(take(4 * P));
  L.g_b = reinterpret_cast<float*>(take(4 * P));
  L.r_b = reinterpret_cast<float*>(take(4 * (size_t)T));
  L.dyb = reinterpret_cast<uint16_t*>(take(2 * (size_t)T * d));
  L.du = reinterpret_cast<uint16_t*>(take(2 * P * de));
  L.hg = reinterpret_cast<uint16_t*>(take(2 * P * de));
  L.dgp = reinterpret_cast<float*>(take(4 * P * (de / GBN)));
  L.dz = reinterpret_cast<float*>(take(4 * P));
  L.dsc = reinterpret_cast<float*>(take(4 * P));
  L.pair_dz = reinterpret_cast<float*>(take(4 * P));
  L.dzb = reinterpret_cast<uint16_t*>(take(2 * (size_t)T * kRouterPad));
  L.dz_off = reinterpret_cast<uint16_t*>(take(2 * (size_t)T * kRouterPad));
  L.part = reinterpret_cast<uint16_t*>(take(2 * P * d));
  L.bytes = off;
  return L;
}

}  // namespace

size_t backward_workspace_bytes(int64_t T, int E, int d, int de) { return bwd_layout(nullptr, T, E, d, de).bytes; }

hipError_t launch_backward(const LayerArgs& la, const uint16_t* x, int64_t T, const float* preact, const float* dy,
                           const float* dz_extra, void* workspace, float* dx, float* d_w_router, float* d_b_router, float* d_rms_scale,
                           float* d_w_in, float* d_w_out, const StageEvents& se, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int E = la.E, d = la.d, de = la.de;
  const BwdLayout L = bwd_layout(static_cast<char*>(workspace), T, E, d, de);
  const int rows = plan_rows(T);
  const int nblk = (int)((T + rows - 1) / rows);
  const uint16_t* w_r = static_cast<const uint16_t*>(la.w_router);
  const uint16_t* w_in = static_cast<const uint16_t*>(la.w_in);
  const uint16_t* w_out = static_cast<const uint16_t*>(la.w_out);

  se.record(0, s);
  bwd_prep_kernel<<<dim3((unsigned)T), dim3(kBlock), 0, s>>>(preact, la.rms_scale, la.eps, T, E, d, dy, L.g_b, L.r_b,
                                                             L.dyb, L.all_off);
  group_count_kernel<PairRule::kPositive><<<dim3((unsigned)nblk), dim3(kPlanThreads), 0, s>>>(preact, T, E, rows,
                                                                                              L.blk);
  group_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(L.blk, nblk, E, de / GBN, kPairRows, L.pair_off, L.tile_up);
  group_fill_kernel<PairRule::kPositive><<<dim3((unsigned)nblk), dim3(kPlanThreads), 0, s>>>(
      preact, L.g_b, T, E, rows, L.blk, L.pair_tok, L.pair_gate, L.pair_idx);

  const int64_t max_up_tiles = (int64_t)E * ((T + kPairRows - 1) / kPairRows) * (de / GBN);
  int64_t grid_pair = 0, grid_t = 0, grid_dn = 0;
  hipError_t e = persistent_grid(bwd_pair_kernel, max_up_tiles, &grid_pair);
  if (e == hipSuccess) e = persistent_grid(tgemm_kernel, (int64_t)E * (de / TBM) * ((d + TBN - 1) / TBN), &grid_t);
  if (e == hipSuccess)
    e = de == 128 ? persistent_grid(grouped_down_kernel<128, true>, down_blocks(E, d, de), &grid_dn)
                  : persistent_grid(grouped_down_kernel<256, true>, down_blocks(E, d, de), &grid_dn);
  if (e != hipSuccess) return e;

  se.record(1, s);
  PairArgs pa{x, L.dyb, L.pair_tok, L.pair_gate, w_in, w_out, L.pair_off, L.tile_up, L.du, L.hg, L.dgp, d, de, E};
  bwd_pair_kernel<<<dim3((unsigned)grid_pair), dim3(kBlock), 0, s>>>(pa);
  se.record(2, s);
  bwd_router_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(kBlock), 0, s>>>(
      preact, la.rms_scale, L.r_b, L.pair_idx, L.dgp, de / GBN, T, E, dz_extra, L.dz, L.dzb, L.dsc, L.pair_dz,
      dz_extra != nullptr ? L.dz_off : nullptr);
  bwd_reduce_kernel<<<dim3((unsigned)E), dim3(kBlock), 0, s>>>(L.dz, L.dsc, T, E, d_b_router, d_rms_scale);
  // dW_out[i][k][j] = sum_p HG[p][j] dY[t_p][k], stored transposed (the gathered dY rows on the wide side)
  TGemmArgs go{L.hg, de, L.dyb, d, L.pair_tok, L.pair_off, d_w_out, de, (int64_t)d * de, E, de, de, d, true};
  tgemm_kernel<<<dim3((unsigned)grid_t), dim3(kBlock), 0, s>>>(go);
  // dW_in[i][j][k] = sum_p dU[p][j] X[t_p][k]
  TGemmArgs gi{L.du, de, x, d, L.pair_tok, L.pair_off, d_w_in, d, (int64_t)de * d, E, de, de, d, false};
  tgemm_kernel<<<dim3((unsigned)grid_t), dim3(kBlock), 0, s>>>(gi);
  // dW_r[i][k] = sum_t dZ[t][i] X[t][k]: kRouterSplits token ranges as groups, then their sum
  TGemmArgs gr{L.dzb, kRouterPad, x, d, nullptr, L.all_off, L.wr_part, d, (int64_t)E * d, kRouterSplits,
               kRouterPad, E, d, false};
  tgemm_kernel<<<dim3((unsigned)grid_t), dim3(kBlock), 0, s>>>(gr);
  bwd_router_sum_kernel<<<dim3((unsigned)(((int64_t)E * d + kBlock - 1) / kBlock)), dim3(kBlock), 0, s>>>(
      L.wr_part, (int64_t)E * d, d_w_router);
  se.record(3, s);
  // dx: per-pair rows dU W_in[i] + dz W_r[i] (the forward's down GEMM, reading W_in k-major), then the
  // per-token sum
  DownArgs dn{L.du, w_in, L.pair_off, L.part, d, E, L.pair_dz, w_r};
  if (de == 128)
    grouped_down_kernel<128, true><<<dim3((unsigned)grid_dn), dim3(kBlock), 0, s>>>(dn);
  else
    grouped_down_kernel<256, true><<<dim3((unsigned)grid_dn), dim3(kBlock), 0, s>>>(dn);
  se.record(4, s);
  if (dz_extra != nullptr)  // the inactive experts' router term goes into dx first
    bwd_router_dx_kernel<<<dim3((unsigned)(d / 128), (unsigned)((T + 63) / 64)), dim3(kBlock), 0, s>>>(
        w_r, E, L.dz_off, T, d, dx);
  int cthreads = (d / 8 + 63) / 64 * 64;
  cthreads = cthreads < 64 ? 64 : (cthreads > 1024 ? 1024 : cthreads);
  bwd_combine_kernel<<<dim3((unsigned)T), dim3((unsigned)cthreads), 0, s>>>(preact, L.pair_idx, L.part, E, d,
                                                                           dz_extra != nullptr, dx);
  se.record(5, s);
  return hipGetLastError();
}

}  // namespace bffn
