// Chunk union + compaction, and sparsity statistics.
//
// Union (BlockFFN write-up, lsdiaocha.cn, §4 acceleration kernel: the experts
// the chunk's tokens activate are united and only those run; BlockFFN
// abstract, arXiv 2507.08771: chunk-level sparsity is the share of
// parameters the union of consecutive tokens activates).  One wave per chunk:
// lane t < L loads token t's mask words, a 6-step xor-shuffle OR reduction
// gives every lane the union, and each lane places expert l (and l + 64) at
// its rank among the set bits with mbcnt, which yields the ascending list.
//
// Statistics (abstract and write-up §3: token- and chunk-level sparsity;
// write-up §5: consecutive-token expert reuse, experts-per-token histogram):
// one workgroup, integer counters only, so the result is exact and
// independent of scheduling.
#include "bffn_internal.h"

namespace bffn {
namespace {

__global__ __launch_bounds__(kBlock) void chunk_union_kernel(int E, const uint64_t* __restrict__ masks,
                                                             int64_t n_chunks, int L,
                                                             uint64_t* __restrict__ chunk_masks,
                                                             int32_t* __restrict__ count,
                                                             int32_t* __restrict__ list) {
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= n_chunks) return;
  const int W = (E + 63) >> 6;
  uint64_t u0 = 0, u1 = 0;
  if (lane < L) {
    const uint64_t* mt = masks + (c * L + lane) * W;
    u0 = mt[0];
    if (W > 1) u1 = mt[1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    u0 |= shfl_xor_u64(u0, off);
    u1 |= shfl_xor_u64(u1, off);
  }
  u0 &= valid_bits(E, 0);
  u1 &= valid_bits(E, 1);
  const int n0 = __popcll(u0);
  const int n = n0 + __popcll(u1);
  if (lane == 0) {
    chunk_masks[c * W] = u0;
    if (W > 1) chunk_masks[c * W + 1] = u1;
    count[c] = n;
  }
  int32_t* lc = list + c * E;
  if ((u0 >> lane) & 1ull) lc[rank_below(u0)] = lane;
  if ((u1 >> lane) & 1ull) lc[n0 + rank_below(u1)] = 64 + lane;
  for (int p = n + lane; p < E; p += 64) lc[p] = -1;
}

constexpr int kStatsMaxThreads = 1024;
constexpr int kStatsTokensPerRound = 4;  // tokens per thread and round, their loads issued together
constexpr int kStatsChunkBatch = 8;      // a chunk's token words loaded together

// One block of 64 to 1024 threads (sized to the tokens).  Every round issues
// all its loads before using any, so a thread waits for memory once per
// round instead of once per token.
__global__ __launch_bounds__(kStatsMaxThreads) void stats_kernel(int E, const uint64_t* __restrict__ masks,
                                                                 int64_t T, int L,
                                                                 blockffn_stats* __restrict__ out) {
  constexpr int kMaxWaves = kStatsMaxThreads / kWave;
  __shared__ unsigned long long hist[129];
  __shared__ unsigned long long part[kMaxWaves][4];
  const int nth = blockDim.x, waves = nth / kWave;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int W = (E + 63) >> 6;
  const int hw = W - 1;  // the high word; with one word it repeats word 0, which vb1 = 0 masks out
  const uint64_t vb0 = valid_bits(E, 0), vb1 = valid_bits(E, 1);
  for (int k = tid; k < 129; k += nth) hist[k] = 0;
  __syncthreads();
  unsigned long long pairs = 0, rnum = 0, rden = 0, usum = 0;
  for (int64_t t0 = tid; t0 < T; t0 += (int64_t)kStatsTokensPerRound * nth) {
    uint64_t a0[kStatsTokensPerRound], a1[kStatsTokensPerRound], p0[kStatsTokensPerRound],
        p1[kStatsTokensPerRound];
#pragma unroll
    for (int j = 0; j < kStatsTokensPerRound; ++j) {
      const int64_t t = t0 + (int64_t)j * nth;
      const bool v = t < T, vp = v && t >= 1;
      a0[j] = v ? masks[t * W] : 0ull;
      a1[j] = v ? masks[t * W + hw] : 0ull;
      p0[j] = vp ? masks[(t - 1) * W] : 0ull;  // no previous token for t = 0: no reuse terms
      p1[j] = vp ? masks[(t - 1) * W + hw] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kStatsTokensPerRound; ++j) {
      if (t0 + (int64_t)j * nth >= T) continue;
      const uint64_t x0 = a0[j] & vb0, x1 = a1[j] & vb1, q0 = p0[j] & vb0, q1 = p1[j] & vb1;
      const int n = __popcll(x0) + __popcll(x1);
      pairs += n;
      atomicAdd(&hist[n], 1ull);
      rnum += __popcll(x0 & q0) + __popcll(x1 & q1);
      rden += __popcll(q0) + __popcll(q1);
    }
  }
  const int64_t C = T / L;
  for (int64_t c = tid; c < C; c += nth) {
    uint64_t u0 = 0, u1 = 0;
    const uint64_t* mc = masks + c * L * W;
    for (int i0 = 0; i0 < L; i0 += kStatsChunkBatch) {
      uint64_t m0[kStatsChunkBatch], m1[kStatsChunkBatch];
#pragma unroll
      for (int j = 0; j < kStatsChunkBatch; ++j) {
        const bool v = i0 + j < L;
        m0[j] = v ? mc[(int64_t)(i0 + j) * W] : 0ull;
        m1[j] = v ? mc[(int64_t)(i0 + j) * W + hw] : 0ull;
      }
#pragma unroll
      for (int j = 0; j < kStatsChunkBatch; ++j) {
        u0 |= m0[j];
        u1 |= m1[j];
      }
    }
    usum += __popcll(u0 & vb0) + __popcll(u1 & vb1);
  }
  unsigned long long v[4] = {pairs, rnum, rden, usum};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)v[q], off, kWave);
      const uint32_t hi = __shfl_xor((uint32_t)(v[q] >> 32), off, kWave);
      v[q] += ((unsigned long long)hi << 32) | lo;
    }
    if (lane == 0) part[w][q] = v[q];
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long tot[4] = {0, 0, 0, 0};
    for (int ww = 0; ww < waves; ++ww)
      for (int q = 0; q < 4; ++q) tot[q] += part[ww][q];
    out->n_tokens = T;
    out->n_chunks = C;
    out->n_experts = E;
    out->chunk_len = L;
    out->active_pairs = (int64_t)tot[0];
    out->reuse_num = (int64_t)tot[1];
    out->reuse_den = (int64_t)tot[2];
    out->union_sum = (int64_t)tot[3];
  }
  for (int k = tid; k < 129; k += nth) out->hist[k] = (int64_t)hist[k];
}

}  // namespace

hipError_t launch_chunk_union(int E, const uint64_t* masks, int64_t n_tokens, int chunk_len,
                              uint64_t* chunk_masks, int32_t* count, int32_t* list, hipStream_t s) {
  const int64_t C = n_tokens / chunk_len;
  if (C == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((C + 3) / 4);
  chunk_union_kernel<<<dim3(blocks), dim3(kBlock), 0, s>>>(E, masks, C, chunk_len, chunk_masks, count, list);
  return hipGetLastError();
}

hipError_t launch_stats(int E, const uint64_t* masks, int64_t n_tokens, int chunk_len, blockffn_stats* out,
                        hipStream_t s) {
  // a thread per kStatsTokensPerRound tokens, whole waves, 64 to 1024 threads
  const int64_t waves = (n_tokens + kStatsTokensPerRound * kWave - 1) / (kStatsTokensPerRound * kWave);
  const int threads = waves >= kStatsMaxThreads / kWave ? kStatsMaxThreads : waves < 1 ? kWave : (int)waves * kWave;
  stats_kernel<<<dim3(1), dim3((unsigned)threads), 0, s>>>(E, masks, n_tokens, chunk_len, out);
  return hipGetLastError();
}

}  // namespace bffn
