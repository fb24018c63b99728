// Kernels of the grouped-by-expert paths (the batched forward and the layer
// backward): pair planning, the two LDS-tiled MFMA grouped GEMMs and the
// per-token combine.  Everything here has internal linkage; each launcher
// source includes it and instantiates what it uses.
//
// When many chunks go through the same layer, streaming each chunk's union
// (the chunk path) would re-read the layer once per chunk.  Here every
// (token, expert) pair with a non-zero gate is grouped by expert and each
// expert's weights are read once for all of its tokens, in LDS-tiled MFMA
// GEMMs (the outer loop over active experts with a batched product inside,
// BlockFFN write-up §7, taken to the whole batch):
//
//   count:   per block of tokens, each expert's pair count
//   scan:    per-expert pair offsets, up-tile offsets, and each token block's
//            first pair slot for every expert (one block)
//   fill:    per block of tokens, its pairs in ascending token order: token,
//            gate, and pair_idx[t][i] for the combine (the forward pairs
//            every non-zero gate; the backward every active pair)
//   up:      H'[p] = g_p * Swish(x[t_p] W_in[i]^T), bf16, grouped GEMM with
//            gathered token rows (192 pairs x 128 hidden x 64 k tiles), both
//            operands DMA'd into a block-shared LDS ring
//   down:    Part[p] = H'[p] W_out[i]^T, bf16 per-pair partial rows; each
//            wave keeps one 64-row slab of W_out[i] in registers and runs it
//            over all of expert i's pairs, read from block-shared LDS tiles
//   combine: y[t] = sum over the token's experts in ascending order of
//            Part[pair_idx[t][i]], fp32 (no atomics; deterministic)
//
// The up GEMM's MFMA tiles (v_mfma_f32_16x16x32_bf16) use 256 threads as
// 2 x 2 waves of 32 x 64.  LDS tiles hold 16-byte chunks XOR-swizzled by
// row, so that the 16 rows an MFMA operand read touches land in different
// banks (the up GEMM's DMA applies the swizzle on the source side; the down
// GEMM stages its hidden rows through registers).  Output tiles are staged
// in LDS and stored as whole 16-byte chunks of each row.
#pragma once

#include "bffn_internal.h"
#include "lds_stream.h"

namespace bffn {
namespace {

constexpr int GBM = 64, GBN = 128, GBK = 64;
constexpr int kPlanThreads = 128;     // one thread per expert (E <= 128)
constexpr int kPlanMaxBlocks = 512;   // token blocks of the count / fill kernels
constexpr int kPlanMinRows = 32;      // tokens per block at least (short scans)
constexpr int kPlanInFlight = 32;     // tokens whose gate loads a count / fill thread issues together

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Byte offset of 16-byte chunk `c` of row `r` in an LDS tile of ROW_BYTES-byte
// rows.  A 16-byte operand read serves 16 lanes (16 consecutive rows, one
// chunk each) per 256-byte pass over the banks, so the 16 rows must land on
// 16 different 16-byte bank groups: rows of 128 bytes alternate halves and
// XOR by (r >> 1) & 7; rows of 256 bytes or more XOR by r & 15.
template <int ROW_BYTES>
__device__ __forceinline__ int lds_off(int r, int c) {
  static_assert(ROW_BYTES == 128 || (ROW_BYTES >= 256 && ROW_BYTES % 256 == 0), "row size");
  const int f = ROW_BYTES == 128 ? ((r >> 1) & 7) : (r & 15);
  return r * ROW_BYTES + ((c ^ f) << 4);
}

int plan_rows(int64_t T) {
  const int64_t r = (T + kPlanMaxBlocks - 1) / kPlanMaxBlocks;
  return (int)(r < kPlanMinRows ? kPlanMinRows : r);
}

// Which (token, expert) entries form pairs: the forward takes every pair with
// a non-zero gate (an active pair whose gate is exactly 0 adds nothing; a
// negative RMS scale gives negative gates, which still count); the backward
// takes every active pair, z > 0, since its router gradient does not vanish
// with the gate.
enum class PairRule { kNonZero, kPositive };

template <PairRule R>
__device__ __forceinline__ bool pair_selected(float v) {
  return R == PairRule::kNonZero ? v != 0.f : v > 0.f;
}

// ---- count: pairs per (token block, expert) ----
template <PairRule R>
__global__ __launch_bounds__(kPlanThreads) void group_count_kernel(const float* __restrict__ sel, int64_t T, int E,
                                                                   int rows, int32_t* __restrict__ blk) {
  const int i = threadIdx.x;
  if (i >= E) return;
  const int64_t t0 = (int64_t)blockIdx.x * rows;
  const int64_t t1 = t0 + rows < T ? t0 + rows : T;
  int c = 0;
  for (int64_t t = t0; t < t1; t += kPlanInFlight) {  // (one round at the minimum block size)
    // (loads past t1 repeat token t1 - 1 and are not counted: no branch
    // around a load, so all of them are in flight together)
    float v[kPlanInFlight];
#pragma unroll
    for (int u = 0; u < kPlanInFlight; ++u) v[u] = sel[(t + u < t1 ? t + u : t1 - 1) * E + i];
#pragma unroll
    for (int u = 0; u < kPlanInFlight; ++u) c += t + u < t1 && pair_selected<R>(v[u]);
  }
  blk[(int64_t)blockIdx.x * E + i] = c;
}

// Exclusive prefix sum over the block's 1024 threads; returns the block total
// in *total.  `wsum` is LDS scratch of 16 entries.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* wsum, int64_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int q = 0; q < 16; ++q) {
    const int64_t ws = wsum[q];
    before += q < w ? ws : 0;
    all += ws;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// ---- scan: expert offsets, up-tile offsets (tiles of tile_rows pairs), per-block first slots (in place) ----
// Thread (part, i) owns expert i's counts of token blocks [b0, b1).
__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t* __restrict__ blk, int nblk, int E, int n_tiles_up,
                                                          int tile_rows, int64_t* __restrict__ pair_off,
                                                          int64_t* __restrict__ tile_up) {
  __shared__ int64_t part_sum[1024];
  __shared__ int64_t exp_off[128];
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x;
  const int nparts = 1024 / E;
  const int part = tid / E, i = tid % E;
  const bool act = part < nparts;
  const int b0 = act ? (int)((int64_t)nblk * part / nparts) : 0;
  const int b1 = act ? (int)((int64_t)nblk * (part + 1) / nparts) : 0;
  // (loads past b1 repeat block b1 - 1 and are not used: no branch around a
  // load, so each round's loads are in flight together)
  int64_t s = 0;
  for (int b = b0; b < b1; b += 8) {
    int c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = blk[(int64_t)(b + u < b1 ? b + u : b1 - 1) * E + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += b + u < b1 ? c[u] : 0;
  }
  part_sum[tid] = s;
  __syncthreads();
  // per-expert totals, then exclusive scans over experts of pairs and up tiles
  int64_t n = 0;
  if (tid < E)
    for (int q = 0; q < nparts; ++q) n += part_sum[q * E + tid];
  const int64_t tiles = (n + tile_rows - 1) / tile_rows * n_tiles_up;
  int64_t n_all = 0, t_all = 0;
  const int64_t p_ex = block_exclusive_scan(n, wsum, &n_all);
  const int64_t t_ex = block_exclusive_scan(tiles, wsum, &t_all);
  if (tid < E) {
    pair_off[tid] = p_ex;
    tile_up[tid] = t_ex;
    exp_off[tid] = p_ex;
  }
  if (tid == 0) {
    pair_off[E] = n_all;
    tile_up[E] = t_all;
  }
  __syncthreads();
  if (act) {
    int64_t off = exp_off[i];
    for (int q = 0; q < part; ++q) off += part_sum[q * E + i];
    for (int b = b0; b < b1; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blk[(int64_t)(b + u < b1 ? b + u : b1 - 1) * E + i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b + u < b1) {
          blk[(int64_t)(b + u) * E + i] = (int32_t)off;
          off += c[u];
        }
    }
  }
}

// ---- fill: each token block writes its pairs, tokens ascending per expert ----
// (sel decides the pairs, as in the count; val[t][i] is stored as the pair's gate)
template <PairRule R>
__global__ __launch_bounds__(kPlanThreads) void group_fill_kernel(const float* __restrict__ sel,
                                                                  const float* __restrict__ val, int64_t T, int E,
                                                                  int rows, const int32_t* __restrict__ blk_off,
                                                                  int32_t* __restrict__ pair_tok,
                                                                  float* __restrict__ pair_gate,
                                                                  int32_t* __restrict__ pair_idx) {
  const int i = threadIdx.x;
  if (i >= E) return;
  const int64_t t0 = (int64_t)blockIdx.x * rows;
  const int64_t t1 = t0 + rows < T ? t0 + rows : T;
  int32_t p = blk_off[(int64_t)blockIdx.x * E + i];
  for (int64_t t = t0; t < t1; t += kPlanInFlight) {  // a round of tokens' loads in flight, then in order
    float sv[kPlanInFlight], vv[kPlanInFlight];
#pragma unroll
    for (int u = 0; u < kPlanInFlight; ++u) {  // (as in the count: clamped, unconditional loads)
      const int64_t tt = t + u < t1 ? t + u : t1 - 1;
      sv[u] = sel[tt * E + i];
      vv[u] = val[tt * E + i];
    }
#pragma unroll
    for (int u = 0; u < kPlanInFlight; ++u) {
      if (t + u < t1 && pair_selected<R>(sv[u])) {
        pair_tok[p] = (int32_t)(t + u);
        pair_gate[p] = vv[u];
        pair_idx[(t + u) * E + i] = p;
        ++p;
      }
    }
  }
}

// The MFMAs take the weight rows as operand A and the pair rows as operand B,
// so D = W . X^T: lane (m, g) of a 16 x 16 tile holds outputs 4 g .. 4 g + 3
// of pair m, four consecutive row elements that it packs into 8 bytes.
__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  return u32x2{pack2_bf16(a, b), pack2_bf16(c, d)};
}

// ---- up: H'[p][n] = g_p Swish(sum_k x[tok(p)][k] W_in[i][n][k]) ----
struct UpArgs {
  const uint16_t* x;          // [T][K]
  const int32_t* pair_tok;    // token of each pair
  const float* pair_gate;     // gate of each pair
  const uint16_t* w;          // [E][N][K]
  const int64_t* pair_off;    // [E + 1]
  const int64_t* tile_off;    // [E + 1]
  uint16_t* hid;              // [P][N]
  int K, N, E;
};

// Tile: kUpRows (192) pairs x 128 hidden units over k in steps of 64; wave
// (wm, wn) computes pairs wm*96 .. +95 against hidden units wn*64 .. +63.  Both
// operands reach LDS by DMA (global_load_lds: 16 bytes per lane, each
// 128-byte row piece read whole; the gathered token rows too, every lane
// with its own row) into a block-shared ring of kUpRing buffers, with the
// three steps after the one being multiplied in flight.  A step's 40 DMA
// instructions are split over the four waves.  Each wave waits for its own
// share with a constant vmcnt, and one barrier per step tells every wave
// that the step has landed and that the buffer about to be refilled has
// been read by all of them.  The 16-byte chunks are swizzled on the source
// side (lane slot c of row r holds chunk c ^ ((r >> 1) & 7)), the layout the
// operand reads below expect.
//
// The kernel is bound by the cache lines a CU can have outstanding, so its
// time follows the lines the busiest CU requests: the weight rows are shared
// by a tile's pairs, while every pair brings its own token row.  At about 612
// pairs per expert, 192-pair tiles take 320 lines a step and at most two
// tiles per CU (640 per step of k); 128-pair tiles take 256 lines and up to
// three tiles (768), and 256-pair tiles 384 lines and up to two (768).
constexpr int kUpRing = 4;
constexpr int kUpAhead = kUpRing - 1;                               // steps in flight behind the one multiplied
constexpr int kUpRows = 192;                                        // pairs per up tile
constexpr int kUpWaveRows = kUpRows / 2;                            // pairs per wave
constexpr int kUpA = kUpWaveRows / 16;                              // 16-pair MFMA groups per wave
constexpr int kUpABytes = kUpRows * 128;                            // pair rows of 128 bytes
constexpr int kUpBufBytes = kUpABytes + GBN * 128;                  // + 128 weight rows: 40 KiB
constexpr int kUpDmaPerWave = (kUpRows + GBN) / 8 / (kBlock / kWave);  // 1 KiB instructions per wave and step

__global__ __launch_bounds__(kBlock) void grouped_up_kernel(UpArgs ua) {
  static_assert(GBK == kStepK && kUpDmaPerWave * (kBlock / kWave) * 8 == kUpRows + GBN, "ring geometry");
  static_assert(kUpRows % 32 == 0 && kUpRing * kUpBufBytes <= 160 * 1024, "tile and ring fit LDS");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kUpRing][kUpBufBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int m = lane & 15, g = lane >> 4;
  const int K = ua.K, N = ua.N, E = ua.E;
  const int64_t total = ua.tile_off[E];
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
      if (ua.tile_off[mid] <= tt) lo = mid; else hi = mid - 1;
    }
    const int i = lo;
    const int64_t p0 = ua.pair_off[i];
    const int n_i = (int)(ua.pair_off[i + 1] - p0);
    const int m_tiles = (n_i + kUpRows - 1) / kUpRows;
    const int64_t local_t = tt - ua.tile_off[i];
    const int nt = (int)(local_t / m_tiles), mt = (int)(local_t % m_tiles);
    const int m0 = mt * kUpRows, n0 = nt * GBN;

    // this wave's DMA instructions j = w kUpDmaPerWave + q of a step: j < 8
    // moves pair rows 8 j .. +7 (gathered token rows; rows past the group
    // repeat a valid row), j >= 8 weight rows 8 (j - 8) .. +7
    const uint16_t* src[kUpDmaPerWave];
    int dst[kUpDmaPerWave];
#pragma unroll
    for (int q = 0; q < kUpDmaPerWave; ++q) {
      const int j = w * kUpDmaPerWave + q;
      if (j < kUpRows / 8) {
        const int R = 8 * j + (lane >> 3);
        const int pr = m0 + R < n_i ? m0 + R : n_i - 1;
        src[q] = ua.x + (int64_t)ua.pair_tok[p0 + pr] * K + dma_chunk_elems(R, lane);
        dst[q] = j * 1024;
      } else {
        const int R = 8 * (j - kUpRows / 8) + (lane >> 3);
        src[q] = ua.w + ((int64_t)i * N + n0 + R) * K + dma_chunk_elems(R, lane);
        dst[q] = kUpABytes + (j - kUpRows / 8) * 1024;
      }
    }
    const int ksteps = K / GBK;
    auto issue = [&](int slot, int step) {  // steps past the last repeat it (constant vmcnt)
      const int st = step < ksteps ? step : ksteps - 1;
#pragma unroll
      for (int q = 0; q < kUpDmaPerWave; ++q) dma16<kPolicyReuse>(src[q] + st * GBK, &ring[slot][0] + dst[q]);
    };

    f32x4 acc[4][kUpA];  // [hidden stripe b][pair group a]
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int a = 0; a < kUpA; ++a) acc[b][a] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < kUpAhead; ++s) issue(s, s);
    for (int ks = 0; ks < ksteps; ++ks) {
      wait_vmcnt<(kUpAhead - 1) * kUpDmaPerWave>();  // this wave's share of step ks has landed
      block_barrier_no_fence();     // ... and everyone's; step ks - 1's buffer is free
      issue((ks + kUpAhead) % kUpRing, ks + kUpAhead);
      const uint8_t* buf = &ring[ks % kUpRing][0];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 av[kUpA], bv[4];
#pragma unroll
        for (int a = 0; a < kUpA; ++a)
          av[a] = *reinterpret_cast<const u32x4*>(buf + lds_off<128>(wm * kUpWaveRows + a * 16 + m, kk * 4 + g));
#pragma unroll
        for (int b = 0; b < 4; ++b)
          bv[b] = *reinterpret_cast<const u32x4*>(buf + kUpABytes + lds_off<128>(wn * 64 + b * 16 + m, kk * 4 + g));
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int a = 0; a < kUpA; ++a)
            acc[b][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bv[b]), as_bf16x8(av[a]), acc[b][a], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // lane (m, g): pair wm*64 + a*16 + m, hidden units n0 + wn*64 + b*16 + 4g .. +3
#pragma unroll
    for (int a = 0; a < kUpA; ++a) {
      const int row = m0 + wm * kUpWaveRows + a * 16 + m;
      if (row >= n_i) continue;
      const float gv = ua.pair_gate[p0 + row];
      uint16_t* orow = ua.hid + (p0 + row) * N + n0 + wn * 64 + 4 * g;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 v = acc[b][a];
        *reinterpret_cast<u32x2*>(orow + b * 16) =
            pack4_bf16(gv * swish(v[0]), gv * swish(v[1]), gv * swish(v[2]), gv * swish(v[3]));
      }
    }
    // the tile's last DMAs (repeats) land and every wave is done with the
    // ring before the next tile refills it
    wait_vmcnt<0>();
    __syncthreads();
  }
}

// ---- MFMA operands from k-major LDS rows by transpose loads ----
// LDS rows of 128 bf16 (256 bytes), row k holding element j of contraction
// index k.  An MFMA operand needs 8 consecutive k of one j per lane; the LDS
// transpose load ds_read_b64_tr_b16 delivers that: within each 16-lane group,
// lane L names 4 elements (8 bytes) and lane i receives element i % 4 of
// lanes 4 j + i / 4, j = 0..3 (checked on gfx950), so lanes naming row
// k0 + L / 4 at column c0 + 4 (L % 4) deliver rows k0 .. k0 + 3 of column
// c0 + i to lane i.
//
// 16-byte chunk position of chunk c in LDS row r (an XOR with an even value:
// the two chunks a 16-lane transpose read touches in a row stay adjacent, and
// the rows read together land on different bank groups).
__device__ __forceinline__ int tg_swz(int r) { return ((r & 3) | ((r >> 1) & 4)) << 1; }

// Byte offset of 16-byte chunk c of k-major row r.
__device__ __forceinline__ int tg_off(int r, int c) { return r * 256 + ((c ^ tg_swz(r)) << 4); }

typedef short tg_v4i16 __attribute__((ext_vector_type(4)));

// NS (4 or 2) MFMA operands of 16 columns c0 + 16 j .. +15, j < NS, over
// rows 0..31: 2 NS transpose reads.  They are written as one asm block that
// also waits for them (lgkmcnt), because the compiler's builtin for this load
// makes it wait for every LDS DMA in flight first (vmcnt 0), which would
// drain a DMA ring.
template <int NS>
__device__ __forceinline__ void tg_operands(const uint8_t* rows, int c0, int lane, u32x4 (&v)[NS]) {
  static_assert(NS == 4 || NS == 2, "stripes");
  const int L = lane & 15, k0 = 8 * (lane >> 4) + (L >> 2);
  unsigned a[2 * NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int c = c0 + 16 * j + 4 * (L & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      a[2 * j + h] = (unsigned)(uintptr_t)(lvoid_t*)(rows + tg_off(k0 + 4 * h, c >> 3) + (c & 7) * 2);
  }
  tg_v4i16 o[2 * NS];
  if constexpr (NS == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const u32x2 l2 = __builtin_bit_cast(u32x2, o[2 * j]), h2 = __builtin_bit_cast(u32x2, o[2 * j + 1]);
    v[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
}

// ---- down: Part[p][n] = sum_k H'[p][k] W_out[i][n][k], K = d_e in {128, 256} ----
struct DownArgs {
  const uint16_t* hid;        // [P][K]
  const uint16_t* w;          // [E][N][K], or [E][K][N] (KMAJOR)
  const int64_t* pair_off;    // [E + 1]
  uint16_t* part;             // [P][N]
  int N, E;
  // KMAJOR only (required there): each pair's row also gets pair_dz[p] * w_add[i] added before it is
  // rounded (the router's share of dx: dz times the expert's router row)
  const float* pair_dz;       // [P]
  const uint16_t* w_add;      // [E][N]
};

// Output columns of one wave in the down GEMM: its slab of W (SN rows x K)
// lives in 64 VGPRs per lane for the whole work item.
template <int K>
constexpr int down_slab() {
  return K == 128 ? 64 : 32;
}
constexpr int kDownPairs = 32;  // pairs per tile: two 16-pair MFMA groups
constexpr int kDownWaves = kBlock / kWave;

// Blocks that cover every down item once (the last group of an expert may
// be partial: N is a multiple of 128 only).
int64_t down_blocks(int E, int N, int K) {
  const int cols = kDownWaves * (K == 128 ? down_slab<128>() : down_slab<256>());
  return (int64_t)E * ((N + cols - 1) / cols);
}

// Byte offset of 16-byte chunk c of row r in a wave's staged output tile of
// RB-byte rows: the XOR spreads the 16 rows that one MFMA group writes over
// distinct bank groups (two rows per 256 bytes at RB = 128, four at RB = 64).
template <int RB>
__device__ __forceinline__ int stage_off(int r, int c) {
  static_assert(RB == 128 || RB == 64, "staged row size");
  const int f = RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
  return r * RB + ((c ^ f) << 4);
}

// A work item is (expert i, kDownWaves slabs of SN columns of W[i]); wave w
// takes slab w and holds it in the MFMA A-operand layout for all of expert
// i's pairs.  Each 32-pair tile of hidden rows is loaded once by the block
// with whole-row (coalesced) loads into a double-buffered LDS tile, the
// next tile's loads in flight during this tile's MFMAs; every wave reads the
// B operands from there.  Each wave writes its output through a private LDS
// stage as whole row segments (plain stores: the L2 acknowledges them sooner
// than non-temporal ones, and later waits include them).  Past the end of a
// group, hidden loads and output stores repeat the group's last pair (the
// same bytes again), so every path issues the same number of memory
// operations and the compiler's waits stay partial.
//
// KMAJOR: W[i] lies k-major ([K][N], the layout of W_in when the backward
// multiplies by it).  The block then loads its slabs (K rows of the item's
// kDownWaves SN columns) with whole-row loads, all in flight at once, and
// turns them into the A-operand layout 32 k rows at a time: written to the
// hidden-tile buffers as k-major 256-byte rows, read back by transpose loads.
// The staging registers live only while an item starts, so that variant is
// capped for three waves per SIMD, which it meets without spilling.  It also
// adds dz_p W_add[i] to each pair's row in fp32 before the row is rounded (the
// products start from it): the tile's 32 dz values travel with its hidden
// rows (loaded with them, staged in LDS beside them), and the item's slice of
// W_add[i] sits in LDS.
template <int K, bool KMAJOR = false>
__global__ __launch_bounds__(kBlock, KMAJOR ? 3 : 1) void grouped_down_kernel(DownArgs da) {
  constexpr int SN = down_slab<K>();
  constexpr int NB = SN / 16;                       // 16-column MFMA stripes
  constexpr int KK = K / 32;                        // 32-deep MFMA steps
  constexpr int RB = SN * 2;                        // bytes per staged output row
  constexpr int CPR = RB / 16;                      // 16-byte chunks per staged row
  constexpr int RPI = kWave / CPR;                  // staged rows per store instruction
  constexpr int HB = K * 2;                         // bytes per hidden row
  constexpr int HC = HB / 16;                       // 16-byte chunks per hidden row
  constexpr int HL = kDownPairs * HC / kBlock;      // hidden-tile loads per thread
  __shared__ __attribute__((aligned(16))) uint8_t htile[2][kDownPairs * HB];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kDownWaves][kDownPairs * RB];
  constexpr int kAddCols = KMAJOR ? SN * kDownWaves : 1;  // the item's columns of W_add[i]
  __shared__ __attribute__((aligned(16))) uint16_t wadd[kAddCols];
  __shared__ float hdz[2][KMAJOR ? kDownPairs : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int N = da.N, E = da.E;
  const int groups = (N + SN * kDownWaves - 1) / (SN * kDownWaves);
  const int64_t total = (int64_t)E * groups;
  // XCD-aware: XCD k walks one contiguous range of items (expert-major), so
  // the blocks reading an expert's hidden rows share an L2.
  const int64_t per_xcd_blocks = gridDim.x / kXcds;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int64_t local = blockIdx.x / kXcds;
  const int64_t span = (total + kXcds - 1) / kXcds;
  const int64_t it_begin = xcd * span, it_end = it_begin + span < total ? it_begin + span : total;
  uint8_t* st = stage[w];

  for (int64_t it = it_begin + local; it < it_end; it += per_xcd_blocks) {
    const int i = (int)(it / groups), grp = (int)(it % groups);
    const int n0 = (grp * kDownWaves + w) * SN;
    const bool has_slab = n0 < N;  // false only for waves past the end of a partial group
    const int64_t p0 = da.pair_off[i];
    const int n_i = (int)(da.pair_off[i + 1] - p0);
    if (n_i == 0) continue;  // (uniform over the block)
    const int tiles = (n_i + kDownPairs - 1) / kDownPairs;
    // The expert's blocks run at the same time; each starts at its own tile
    // (and wraps), so they do not all read the same hidden rows at once.
    const int rot = (int)((int64_t)grp * tiles / groups);
    auto phys = [&](int t) { return t + rot < tiles ? t + rot : t + rot - tiles; };
    // the slab: lane (m, g) holds row n0 + 16 b + m, elements 32 kk + 8 g .. +7
    u32x4 wa[NB][KK];
    if constexpr (!KMAJOR) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint16_t* src = da.w + ((int64_t)i * N + (has_slab ? n0 : 0) + 16 * b + m) * K + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) wa[b][kk] = *reinterpret_cast<const u32x4*>(src + 32 * kk);
      }
    } else {
      constexpr int COLS = SN * kDownWaves;       // the item's columns: 256 (K = 128) or 128 (K = 256)
      constexpr int CPK = COLS / 8;               // 16-byte chunks per k row
      constexpr int RL = 32 * CPK / kBlock;       // chunks per thread per 32 k rows
      static_assert(COLS % 128 == 0 && RL * kBlock == 32 * CPK && COLS / 128 * 32 * 256 <= 2 * kDownPairs * HB,
                    "k-major staging geometry");
      // thread chunk c = tid + j kBlock of each 32-row round: k row c / CPK,
      // columns 8 (c % CPK) .. +7 of the item (past N: column 0, unused)
      u32x4 raw[KK][RL];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int j = 0; j < RL; ++j) {
          const int c = tid + j * kBlock;
          const int col = grp * COLS + (c % CPK) * 8;
          raw[kk][j] = *reinterpret_cast<const u32x4*>(da.w + ((int64_t)i * K + 32 * kk + c / CPK) * N +
                                                       (col < N ? col : 0));
        }
      uint8_t* sbuf = &htile[0][0];  // COLS / 128 planes of 32 rows x 256 bytes
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int j = 0; j < RL; ++j) {
          const int c = tid + j * kBlock, cc = c % CPK;
          *reinterpret_cast<u32x4*>(sbuf + (cc >> 4) * (32 * 256) + tg_off(c / CPK, cc & 15)) = raw[kk][j];
        }
        __syncthreads();
        u32x4 v[NB];
        tg_operands(sbuf + ((w * SN) >> 7) * (32 * 256), (w * SN) & 127, lane, v);
#pragma unroll
        for (int b = 0; b < NB; ++b) wa[b][kk] = v[b];
        __syncthreads();
      }
    }
    // hidden tile pt: thread chunk c = tid + j kBlock is row c / HC, chunk c % HC
    // (KMAJOR: every lane also loads the dz of the tile's pair lane % 32, so all waves issue the same loads)
    u32x4 hr[HL];
    float hz = 0.f;
    auto hload = [&](int pt) {
#pragma unroll
      for (int j = 0; j < HL; ++j) {
        const int c = tid + j * kBlock, r = c / HC;
        const int pr = pt * kDownPairs + r < n_i ? pt * kDownPairs + r : n_i - 1;
        hr[j] = *reinterpret_cast<const u32x4*>(da.hid + (p0 + pr) * K + (c % HC) * 8);
      }
      if constexpr (KMAJOR) {
        const int r = lane & (kDownPairs - 1);
        hz = da.pair_dz[p0 + (pt * kDownPairs + r < n_i ? pt * kDownPairs + r : n_i - 1)];
      }
    };
    auto hwrite = [&](int buf) {
#pragma unroll
      for (int j = 0; j < HL; ++j) {
        const int c = tid + j * kBlock;
        *reinterpret_cast<u32x4*>(&htile[buf][lds_off<HB>(c / HC, c % HC)]) = hr[j];
      }
      if constexpr (KMAJOR)
        if (tid < kDownPairs) hdz[buf][tid] = hz;
    };
    auto tile = [&](int buf, int pt) {
      if (!has_slab) return;  // (such a wave still loads and meets the barriers)
      f32x4 acc[NB][2];
      if constexpr (KMAJOR) {
        // each product starts from dz_p W_add[i] at its four columns (lane (m, g): columns
        // 16 b + 4 g .. +3 of pair 16 a + m, as the MFMA leaves them)
        float z[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) z[a] = hdz[buf][16 * a + m];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const u32x2 wv = *reinterpret_cast<const u32x2*>(&wadd[w * SN + 16 * b + 4 * g]);
#pragma unroll
          for (int a = 0; a < 2; ++a)
            acc[b][a] = f32x4{z[a] * bf16_lo(wv[0]), z[a] * bf16_hi(wv[0]), z[a] * bf16_lo(wv[1]),
                              z[a] * bf16_hi(wv[1])};
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int a = 0; a < 2; ++a) acc[b][a] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 hb[2];  // lane (m, g): pair 16 a + m, elements 32 kk + 8 g .. +7
#pragma unroll
        for (int a = 0; a < 2; ++a)
          hb[a] = *reinterpret_cast<const u32x4*>(&htile[buf][lds_off<HB>(16 * a + m, 4 * kk + g)]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int a = 0; a < 2; ++a)
            acc[b][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[b][kk]), as_bf16x8(hb[a]), acc[b][a],
                                                               0, 0, 0);
      }
      // lane (m, g): outputs 16 b + 4 g .. +3 of the tile's pair 16 a + m
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int col = 16 * b + 4 * g;
          const f32x4 v = acc[b][a];
          *reinterpret_cast<u32x2*>(st + stage_off<RB>(16 * a + m, col >> 3) + (col & 7) * 2) =
              pack4_bf16(v[0], v[1], v[2], v[3]);
        }
      // A wave's LDS operations complete in issue order, so the reads below
      // see the writes above (and the next tile's writes follow these reads);
      // the empty asm keeps the compiler from moving LDS accesses across.
      asm volatile("" ::: "memory");
      const int last = n_i - 1 - pt * kDownPairs;  // the group's last row in this tile
#pragma unroll
      for (int q = 0; q < kDownPairs / RPI; ++q) {
        const int r = q * RPI + lane / CPR, c = lane % CPR;
        const int rr = r < last ? r : last;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + stage_off<RB>(rr, c));
        *reinterpret_cast<u32x4*>(da.part + (p0 + pt * kDownPairs + rr) * N + n0 + c * 8) = v;
      }
      asm volatile("" ::: "memory");
    };

    // htile[t & 1] holds tile t.  Tile t + 1's rows, loaded during tile
    // t - 1, go to the other buffer (last read by tile t - 1, before the
    // barrier) before tile t's MFMAs, and tile t + 2's loads are issued
    // ahead of tile t's stores: stores count in the same in-order counter as
    // loads, so a wait for those rows never waits for the latest stores.
    // Loads past the last tile repeat it.
    hload(phys(0));
    if constexpr (KMAJOR) {
      // the item's W_add[i] columns (past N: column 0, unused), loaded by every thread (the same
      // loads in every wave), stored by the first kAddCols / 8; published by the barrier below
      const int c8 = tid % (kAddCols / 8), col = grp * kAddCols + c8 * 8;
      const u32x4 wv = *reinterpret_cast<const u32x4*>(da.w_add + (int64_t)i * N + (col < N ? col : 0));
      hwrite(0);
      if (tid < kAddCols / 8) *reinterpret_cast<u32x4*>(&wadd[c8 * 8]) = wv;
    } else {
      hwrite(0);
    }
    hload(phys(tiles > 1 ? 1 : 0));
    __syncthreads();
    for (int t = 0; t < tiles; ++t) {
      if (t + 1 < tiles) hwrite((t + 1) & 1);  // (uniform over the block)
      hload(phys(t + 2 < tiles ? t + 2 : tiles - 1));
      tile(t & 1, phys(t));
      __syncthreads();
    }
  }
}

// Partial rows are read exactly once: non-temporal loads keep them from
// displacing anything in the caches (measured 1.3x faster than plain loads).
__device__ __forceinline__ u32x4 load_part(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---- combine: y[t] = sum over active experts (ascending) of Part[pair_idx[t][i]] ----
constexpr int kCombineInFlight = 8;  // partial-row loads per thread in flight

__global__ __launch_bounds__(1024) void combine_kernel(const float* __restrict__ gates,
                                                       const int32_t* __restrict__ pair_idx,
                                                       const uint16_t* __restrict__ part, int E, int d,
                                                       float* __restrict__ y) {
  __shared__ int32_t plist[128];
  __shared__ int nlist;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // gates and pair slots load together (a slot is used only where its gate is non-zero)
    const float g0 = tid < E ? gates[t * E + tid] : 0.f, g1 = tid + 64 < E ? gates[t * E + tid + 64] : 0.f;
    const int32_t q0 = tid < E ? pair_idx[t * E + tid] : 0, q1 = tid + 64 < E ? pair_idx[t * E + tid + 64] : 0;
    const bool on0 = g0 != 0.f, on1 = g1 != 0.f;
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
  auto add8 = [](float (&acc)[8], u32x4 v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_lo(v[q]);
      acc[2 * q + 1] += bf16_hi(v[q]);
    }
  };
  for (int c0 = tid * 8; c0 < d; c0 += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // eight partial rows in flight, added in ascending expert order
    for (int s = 0; s < n; s += kCombineInFlight) {
      u32x4 v[kCombineInFlight];
#pragma unroll
      for (int u = 0; u < kCombineInFlight; ++u)
        v[u] = s + u < n ? load_part(part + (int64_t)plist[s + u] * d + c0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kCombineInFlight; ++u)
        if (s + u < n) add8(acc, v[u]);
    }
    f32x4* yo = reinterpret_cast<f32x4*>(y + t * d + c0);
    yo[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    yo[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

size_t r256(size_t v) { return (v + 255) & ~size_t(255); }

// A persistent grid: the resident capacity, at most the work, and a multiple
// of the XCD count so that every XCD gets the same number of blocks.
template <typename F>
hipError_t persistent_grid(F kernel, int64_t n_items, int64_t* grid) {
  int64_t gsz = 0;
  const hipError_t e = resident_blocks(reinterpret_cast<const void*>(kernel), kBlock, &gsz);
  if (e != hipSuccess) return e;
  const int64_t need = xcd_grid(n_items > 0 ? n_items : 1);
  if (gsz > need) gsz = need;
  gsz = gsz / kXcds * kXcds;
  *grid = gsz > 0 ? gsz : kXcds;
  return hipSuccess;
}

}  // namespace
}  // namespace bffn
