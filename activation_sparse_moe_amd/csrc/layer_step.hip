// One layer step for a few chunks in three launches: router, union,
// statistics and the expert forward of a short call (the verify step of
// speculative decoding sends one chunk of draft tokens through each layer in
// turn: BlockFFN write-up, lsdiaocha.cn, §4 acceleration kernel and §6 real
// speed-up).
//
// Such a call moves little data (a 2048 x 64 layer's router is 256 KB, each
// expert 0.5 MB) and is bound by latency: by the dependent memory round trips
// and the launches, and by how many loads one CU keeps in flight (a single
// block streaming the router takes about 19 us).  So the work is spread over
// many blocks, every wave issues all the loads of its share before its first
// product, and no partial result crosses a block except through a kernel
// boundary (a counter-and-fence hand-off between blocks costs an L2
// write-back per block on this chip, more than the launch it saves):
//   1. route_split_kernel, blocks (chunk, d-range of 128): partial
//      pre-activations zpart[token][expert][range] (MFMA 16x16x32), each
//      pre-activation's partials contiguous.
//   2. step_up_kernel, blocks (chunk, expert, 16 hidden rows): each adds its
//      expert's partials for the chunk's tokens (the order of the router
//      epilogue, so it sees the same signs) and stops unless some token
//      activates the expert, i.e. unless the expert is in the chunk's union;
//      else its 8 waves split d and it stores Swish(W_in x), bf16.  One more
//      block per chunk completes the router: gates, patterns, the union and
//      its ascending list.  (Forming z inside these blocks instead, from the
//      router row and the tokens, saves the first launch but makes every
//      block, active or not, load the chunk's tokens: slower, 26.9 against
//      23.0 us for a chunk of 8.)
//   3. step_down_kernel, blocks (chunk, 16 output rows): its 8 waves split
//      the union's experts x d_e; each expert's product with Swish is
//      scaled by the token's gate in fp32 (0 where the token did not
//      activate the expert) and added, y = the sum, fp32.  One more block
//      computes the call's statistics.
// Every sum has a fixed order, so the results are reproducible.
//
// The last two kernels, with the up blocks taking their experts from a given
// union (count / list) instead, are also the forward of a few chunks whose
// union is already known (blockffn_forward's AUTO mode).
#include "bffn_internal.h"
#include "router_epilogue.h"

namespace bffn {
namespace {

constexpr int kRouteSplitK = 128;  // d elements of one router block
constexpr int kBatch = 16;         // MFMA steps whose loads are issued together
constexpr int kStepMaxL = 32;
constexpr int kStepWaves = 8;      // waves of an up or down block, which split its contraction
constexpr int kStepThreads = kStepWaves * kWave;
constexpr int kStepMaxD = kStepWaves * kBatch * 32;  // every up wave's share of d in one batch

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// acc[tl] += A[16 rows][k] B[k][16 tokens] over the MFMA steps [lo, hi) of 32
// k each (a_at(s): this lane's A row at step s; b_at(s, tl): its token row).
// Lane (m, g) passes its row's (and token's) k = 32 s + 8 g .. + 7, as the
// 16x16x32 product takes them.  All loads of a batch are issued before its
// first product.
template <int NT, typename APtr, typename BPtr>
__device__ __forceinline__ void mfma_range(f32x4 (&acc)[NT], int lo, int hi, APtr a_at, BPtr b_at) {
  for (int s0 = lo; s0 < hi; s0 += kBatch) {
    u32x4 a[kBatch], b[kBatch][NT];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < hi) {
        a[j] = ld16(a_at(s0 + j));
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) b[j][tl] = ld16(b_at(s0 + j, tl));
      }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < hi)
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) acc[tl] = mfma16(a[j], b[j][tl], acc[tl]);
  }
}

// The S contiguous partials of one pre-activation added in range order,
// every load of a batch issued first.  The up kernel's activity test and the
// router epilogue both take z from here, so they agree on every sign.
__device__ __forceinline__ float zpart_sum(const float* zp, int S) {
  float z = 0.f;
  if ((S & 3) == 0) {  // 16-byte loads (zp is 16-byte aligned when S is a multiple of 4)
    for (int s0 = 0; s0 < S; s0 += kBatch) {
      f32x4 v[kBatch / 4];
#pragma unroll
      for (int j = 0; j < kBatch / 4; ++j)
        v[j] = s0 + 4 * j < S ? *reinterpret_cast<const f32x4*>(zp + s0 + 4 * j) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kBatch / 4; ++j)
        if (s0 + 4 * j < S)
#pragma unroll
          for (int q = 0; q < 4; ++q) z = s0 + 4 * j + q == 0 ? v[j][q] : z + v[j][q];
    }
    return z;
  }
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = s0 + j < S ? zp[s0 + j] : 0.f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < S) z = s0 + j == 0 ? v[j] : z + v[j];
  }
  return z;
}

// Adds the block's kStepWaves partial tiles in wave order; wave 0 returns
// true with the sums in acc, the other waves false.
template <int NT>
__device__ __forceinline__ bool block_sum(f32x4 (&acc)[NT], f32x4 (*red)[NT][kWave], int w, int lane) {
  if (w > 0)
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) red[w - 1][tl][lane] = acc[tl];
  __syncthreads();
  if (w != 0) return false;
#pragma unroll
  for (int q = 0; q < kStepWaves - 1; ++q)
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) acc[tl] += red[q][tl][lane];
  return true;
}

// ---- 1. partial pre-activations zpart[t][e][s] over d-range s: block (chunk, s) ----
// Wave w takes expert stripes w, w + 4, ... (16 experts each); tokens past L
// repeat a valid token (their columns are not stored).
template <int NT>
__global__ __launch_bounds__(kBlock) void route_split_kernel(LayerArgs la, const uint16_t* __restrict__ x, int L,
                                                             int S, float* __restrict__ zpart) {
  const int64_t u = blockIdx.x / S;
  const int s = (int)(blockIdx.x % S);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int d = la.d, E = la.E;
  const uint16_t* wr = layer_ptr<kTWRouter>(la, static_cast<const uint16_t*>(la.w_router), u);
  const int k0 = s * kRouteSplitK + 8 * g;
  const uint16_t* brow[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) brow[tl] = x + (u * L + (m + 16 * tl) % L) * d + k0;
  for (int st = w; st < (E >> 4); st += kBlock / kWave) {
    const uint16_t* arow = wr + (int64_t)(st * 16 + m) * d + k0;
    f32x4 acc[NT];
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_range<NT>(
        acc, 0, kRouteSplitK / 32, [&](int j) { return arow + 32 * j; },
        [&](int j, int tl) { return brow[tl] + 32 * j; });
    // lane (m, g): experts st 16 + 4 g .. + 3 of token m + 16 tl
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      const int n = m + 16 * tl;
      if (n < L)
#pragma unroll
        for (int q = 0; q < 4; ++q) zpart[((u * L + n) * E + st * 16 + 4 * g + q) * S + s] = acc[tl][q];
    }
  }
}

// The rest of the router for one chunk (one block): gates, patterns, z, and
// the chunk's union and ascending list.
__device__ __forceinline__ void route_finish(const LayerArgs& la, int64_t u, int L, int S,
                                             const float* __restrict__ zpart, float* __restrict__ gates,
                                             uint64_t* __restrict__ masks, float* __restrict__ preact,
                                             uint64_t* __restrict__ chunk_masks, int32_t* __restrict__ count,
                                             int32_t* __restrict__ list, float* zl, uint64_t* ml, float* bs) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = la.E, W = (E + 63) >> 6;
  // bias and scale into LDS, their loads issued before the partials'
  const float* bias = layer_ptr<kTBRouter>(la, la.b_router, u);
  const float* scale = layer_ptr<kTScale>(la, la.rms_scale, u);
  float bv = 0.f, sv = 1.f;
  if (tid < E) {
    if (bias) bv = bias[tid];
    if (scale) sv = scale[tid];
  }
  for (int idx = tid; idx < E * L; idx += kStepThreads) {
    const int n = idx / E, e = idx % E;
    zl[e * L + n] = zpart_sum(zpart + ((u * L + n) * E + e) * S, S);
  }
  if (tid < E) {
    bs[tid] = bv;
    bs[128 + tid] = sv;
  }
  __syncthreads();
  router_epilogue<BLOCKFFN_ROUTER_BLOCKFFN>(zl, 1, E, L, u * L, bs, bs + 128, la.eps, 0, gates, masks, preact, ml);
  __syncthreads();
  if (w != 0) return;
  // the union: lane t < L holds token t's words, OR by xor shuffles, then each set bit at its rank
  uint64_t u0 = 0, u1 = 0;
  if (lane < L) {
    u0 = ml[lane * W];
    if (W > 1) u1 = ml[lane * W + 1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    u0 |= shfl_xor_u64(u0, off);
    u1 |= shfl_xor_u64(u1, off);
  }
  u0 &= valid_bits(E, 0);
  u1 &= valid_bits(E, 1);
  const int n0 = __popcll(u0), n = n0 + __popcll(u1);
  if (lane == 0) {
    chunk_masks[u * W] = u0;
    if (W > 1) chunk_masks[u * W + 1] = u1;
    count[u] = n;
  }
  int32_t* lc = list + u * E;
  if ((u0 >> lane) & 1ull) lc[rank_below(u0)] = lane;
  if ((u1 >> lane) & 1ull) lc[n0 + rank_below(u1)] = 64 + lane;
  for (int p = n + lane; p < E; p += 64) lc[p] = -1;
}

// ---- 2. up-projection: block (chunk, expert, 16 hidden rows); one more block per chunk: router epilogue ----
// hs[chunk][expert][token][d_e] = Swish(W_in[expert] x), bf16, for the experts in the chunk's union.
// With ZTEST false (a forward whose union is given) block (chunk, slot, 16 hidden rows) takes the slot's
// expert from count / list and there are no router blocks.
template <int NT, bool ZTEST>
__global__ __launch_bounds__(kStepThreads) void step_up_kernel(LayerArgs la, const uint16_t* __restrict__ x,
                                                               int64_t units, int L, int S,
                                                               const float* __restrict__ zpart,
                                                               uint16_t* __restrict__ hs, float* __restrict__ gates,
                                                               uint64_t* __restrict__ masks,
                                                               float* __restrict__ preact,
                                                               uint64_t* __restrict__ chunk_masks,
                                                               int32_t* __restrict__ count,
                                                               int32_t* __restrict__ list) {
  __shared__ f32x4 red[kStepWaves - 1][NT][kWave];
  __shared__ float zl[128 * kStepMaxL];
  __shared__ uint64_t ml[kStepMaxL * 2];
  __shared__ float bs[256];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int d = la.d, E = la.E, de = la.de, R = de >> 4;
  const int64_t b = blockIdx.x, nb = units * E * R;
  if (ZTEST && b >= nb) {
    route_finish(la, b - nb, L, S, zpart, gates, masks, preact, chunk_masks, count, list, zl, ml, bs);
    return;
  }
  const int64_t u = b / (E * R);
  const int rem = (int)(b % (E * R)), r16 = rem % R;
  int e;
  if constexpr (ZTEST) {
    // is expert e in the chunk's union?  z of token `lane` as the router epilogue forms it
    e = rem / R;
    bool on = false;
    if (lane < L) {
      const float* bias = layer_ptr<kTBRouter>(la, la.b_router, u);
      const float be = bias ? bias[e] : 0.f;  // (loaded before the partials)
      float z = 0.f;
      z += zpart_sum(zpart + ((u * L + lane) * E + e) * S, S);
      z += be;
      on = z > 0.f;
    }
    if (__ballot(on) == 0ull) return;  // (every wave computes the same: the whole block)
  } else {
    const int slot = rem / R;
    if (slot >= count[u]) return;  // (the whole block)
    e = list[u * E + slot];
  }
  const uint16_t* arow = layer_ptr<kTWIn>(la, static_cast<const uint16_t*>(la.w_in), u) +
                         ((int64_t)e * de + r16 * 16 + m) * d + 8 * g;
  const uint16_t* brow[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) brow[tl] = x + (u * L + (m + 16 * tl) % L) * d + 8 * g;
  const int KS = d >> 5;
  f32x4 acc[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_range<NT>(
      acc, w * KS / kStepWaves, (w + 1) * KS / kStepWaves, [&](int j) { return arow + 32 * j; },
      [&](int j, int tl) { return brow[tl] + 32 * j; });
  if (!block_sum<NT>(acc, red, w, lane)) return;
  // lane (m, g): hidden rows r16 16 + 4 g .. + 3 of token m + 16 tl
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int n = m + 16 * tl;
    if (n >= L) continue;
    const f32x4 v = acc[tl];
    *reinterpret_cast<u32x2*>(hs + ((u * E + e) * L + n) * (int64_t)de + r16 * 16 + 4 * g) =
        u32x2{pack2_bf16(swish(v[0]), swish(v[1])), pack2_bf16(swish(v[2]), swish(v[3]))};
  }
}

// Statistics of the call's T <= 64 tokens by one wave, lane t holding token t.
__device__ __forceinline__ void step_stats(const uint64_t* __restrict__ masks, const int32_t* __restrict__ count,
                                           int64_t T, int L, int E, blockffn_stats* __restrict__ out, unsigned* hist,
                                           int lane) {
  const int W = (E + 63) >> 6, hw = W - 1;
  const bool v = lane < T;
  const uint64_t x0 = v ? masks[lane * W] & valid_bits(E, 0) : 0ull;
  const uint64_t x1 = v ? masks[lane * W + hw] & valid_bits(E, 1) : 0ull;
  const int64_t units = T / L;
  const int cu = lane < units ? count[lane] : 0;  // the unions' sizes
  const uint64_t q0 = shfl_up_u64(x0), q1 = shfl_up_u64(x1);  // token t - 1 (lane 0: none)
  const bool vp = v && lane >= 1;
  const int nt = __popcll(x0) + __popcll(x1);
  const uint64_t pairs = wave_sum_u64(v ? nt : 0);
  const uint64_t rnum = wave_sum_u64(vp ? __popcll(x0 & q0) + __popcll(x1 & q1) : 0);
  const uint64_t rden = wave_sum_u64(vp ? __popcll(q0) + __popcll(q1) : 0);
  const uint64_t usum = wave_sum_u64((uint64_t)cu);
  // the histogram in LDS; this wave is its only user, so ordering its own LDS accesses suffices
  for (int k = lane; k <= 128; k += kWave) hist[k] = 0u;
  __threadfence_block();
  __builtin_amdgcn_wave_barrier();
  if (v) atomicAdd(&hist[nt], 1u);
  __threadfence_block();
  __builtin_amdgcn_wave_barrier();
  for (int k = lane; k <= 128; k += kWave) out->hist[k] = (int64_t)hist[k];
  if (lane == 0) {
    out->n_tokens = T;
    out->n_chunks = units;
    out->n_experts = E;
    out->chunk_len = L;
    out->active_pairs = (int64_t)pairs;
    out->reuse_num = (int64_t)rnum;
    out->reuse_den = (int64_t)rden;
    out->union_sum = (int64_t)usum;
  }
}

// ---- 3. down-projection: block (chunk, 16 output rows) over the union's experts x d_e; one more block: stats ----
template <int NT>
__global__ __launch_bounds__(kStepThreads) void step_down_kernel(LayerArgs la, int64_t units, int L,
                                                                 const float* __restrict__ gates,
                                                                 const int32_t* __restrict__ count,
                                                                 const int32_t* __restrict__ list,
                                                                 const uint16_t* __restrict__ hs,
                                                                 float* __restrict__ y,
                                                                 const uint64_t* __restrict__ masks,
                                                                 blockffn_stats* __restrict__ stats) {
  constexpr int DB = NT == 1 ? kBatch : kBatch / 2;  // steps whose loads are issued together
  __shared__ f32x4 red[kStepWaves - 1][NT][kWave];
  __shared__ unsigned hist[129];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int d = la.d, E = la.E, de = la.de;
  const int rbs = d >> 4;
  if ((int64_t)blockIdx.x == units * rbs) {
    if (stats != nullptr && w == 0) step_stats(masks, count, units * L, L, E, stats, hist, lane);
    return;
  }
  const int64_t u = blockIdx.x / rbs;
  const int rb = (int)(blockIdx.x % rbs);
  const int cnt = count[u];
  const int spe = de >> 5;  // MFMA steps per expert
  const int KS = cnt * spe;
  // lane l holds the experts of slots l and 64 + l
  const int32_t* lu = list + u * E;
  const int e0 = lane < cnt ? lu[lane] : 0, e1 = lane + 64 < cnt ? lu[lane + 64] : 0;
  const uint16_t* wo = layer_ptr<kTWOut>(la, static_cast<const uint16_t*>(la.w_out), u) +
                       ((int64_t)rb * 16 + m) * de + 8 * g;
  int tok[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) tok[tl] = (m + 16 * tl) % L;
  f32x4 acc[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lo = w * KS / kStepWaves, hi = (w + 1) * KS / kStepWaves;
  // pe: the current expert's product (over this wave's steps of it); at the
  // expert's last step here it is scaled by the token's gate and added to acc
  f32x4 pe[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) pe[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = lo; s0 < hi; s0 += DB) {
    u32x4 a[DB], h[DB][NT];
    float gv[DB][NT];
#pragma unroll
    for (int j = 0; j < DB; ++j)
      if (s0 + j < hi) {
        const int st = s0 + j, slot = st / spe, j0 = (st % spe) * 32;
        const int e = __builtin_amdgcn_readlane(slot < 64 ? e0 : e1, slot & 63);
        a[j] = ld16(wo + (int64_t)e * d * de + j0);
        const bool last = (st + 1) % spe == 0 || st + 1 == hi;
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) {
          h[j][tl] = ld16(hs + ((u * E + e) * L + tok[tl]) * (int64_t)de + j0 + 8 * g);
          gv[j][tl] = last ? gates[(u * L + tok[tl]) * E + e] : 0.f;
        }
      }
#pragma unroll
    for (int j = 0; j < DB; ++j)
      if (s0 + j < hi) {
        const int st = s0 + j;
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) pe[tl] = mfma16(a[j], h[j][tl], pe[tl]);
        if ((st + 1) % spe == 0 || st + 1 == hi)
#pragma unroll
          for (int tl = 0; tl < NT; ++tl) {
            acc[tl] += gv[j][tl] * pe[tl];
            pe[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
  }
  if (!block_sum<NT>(acc, red, w, lane)) return;
  // lane (m, g): output rows rb 16 + 4 g .. + 3 of token m + 16 tl
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int n = m + 16 * tl;
    if (n < L) *reinterpret_cast<f32x4*>(y + (u * L + n) * d + rb * 16 + 4 * g) = acc[tl];
  }
}

template <int NT>
hipError_t launch_few_nt(const LayerArgs& la, const uint16_t* x, int64_t T, int L, const float* gates,
                         const int32_t* count, const int32_t* list, uint16_t* hs, float* y, const StageEvents& se,
                         hipStream_t s) {
  const int64_t units = T / L;
  se.record(0, s);
  step_up_kernel<NT, false><<<dim3((unsigned)(units * la.E * (la.de >> 4))), dim3(kStepThreads), 0, s>>>(
      la, x, units, L, 0, nullptr, hs, nullptr, nullptr, nullptr, nullptr, const_cast<int32_t*>(count),
      const_cast<int32_t*>(list));
  se.record(1, s);
  const int64_t down_blocks = units * (la.d >> 4) + 1;
  step_down_kernel<NT><<<dim3((unsigned)down_blocks), dim3(kStepThreads), 0, s>>>(la, units, L, gates, count, list,
                                                                                  hs, y, nullptr, nullptr);
  se.record(2, s);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(const LayerArgs& la, const uint16_t* x, int64_t T, int L, float* gates, uint64_t* masks,
                     float* preact, uint64_t* chunk_masks, int32_t* count, int32_t* list, blockffn_stats* stats,
                     float* zpart, uint16_t* hs, float* y, hipStream_t s) {
  const int64_t units = T / L;
  const int S = la.d / kRouteSplitK;
  route_split_kernel<NT><<<dim3((unsigned)(units * S)), dim3(kBlock), 0, s>>>(la, x, L, S, zpart);
  const int64_t up_blocks = units * la.E * (la.de >> 4) + units;
  step_up_kernel<NT, true><<<dim3((unsigned)up_blocks), dim3(kStepThreads), 0, s>>>(
      la, x, units, L, S, zpart, hs, gates, masks, preact, chunk_masks, count, list);
  const int64_t down_blocks = units * (la.d >> 4) + 1;
  step_down_kernel<NT><<<dim3((unsigned)down_blocks), dim3(kStepThreads), 0, s>>>(la, units, L, gates, count, list,
                                                                                  hs, y, masks, stats);
  return hipGetLastError();
}

}  // namespace

bool layer_step_fused(int d, int E, int de, int dtype, int64_t n_tokens, int chunk_len) {
  const int64_t units = chunk_len > 0 ? n_tokens / chunk_len : 0;
  return forward_mfma_supported(d, de, dtype) && E % 16 == 0 && d <= kStepMaxD && units >= 1 &&
         units <= kStepMaxUnits && n_tokens <= kStepMaxTokens && chunk_len <= kStepMaxL;
}

bool forward_few_supported(int d, int de, int dtype, int64_t units, int chunk_len) {
  return forward_mfma_supported(d, de, dtype) && d <= kStepMaxD && units >= 1 && units <= kStepMaxUnits &&
         chunk_len <= kStepMaxL;
}

hipError_t launch_forward_few(const LayerArgs& la, const uint16_t* x, int64_t T, int L, const float* gates,
                              const int32_t* count, const int32_t* list, uint16_t* hs, float* y,
                              const StageEvents& se, hipStream_t s) {
  if (L <= 16) return launch_few_nt<1>(la, x, T, L, gates, count, list, hs, y, se, s);
  return launch_few_nt<2>(la, x, T, L, gates, count, list, hs, y, se, s);
}

size_t layer_step_zpart_bytes(int d, int E, int64_t n_tokens) {
  return (size_t)(d / kRouteSplitK) * n_tokens * E * sizeof(float);
}

size_t layer_step_hs_bytes(int E, int de, int64_t n_tokens) { return (size_t)n_tokens * E * de * sizeof(uint16_t); }

hipError_t launch_layer_step(const LayerArgs& la, const uint16_t* x, int64_t T, int L, float* gates, uint64_t* masks,
                             float* preact, uint64_t* chunk_masks, int32_t* count, int32_t* list, blockffn_stats* stats,
                             float* zpart, uint16_t* hs, float* y, hipStream_t s) {
  if (L <= 16)
    return launch_nt<1>(la, x, T, L, gates, masks, preact, chunk_masks, count, list, stats, zpart, hs, y, s);
  return launch_nt<2>(la, x, T, L, gates, masks, preact, chunk_masks, count, list, stats, zpart, hs, y, s);
}

}  // namespace bffn
