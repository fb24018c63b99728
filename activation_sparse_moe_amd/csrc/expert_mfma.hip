// Expert streaming on the matrix cores: the chunk path (bf16, any chunk length;
// at L = 1 the idle token columns cost nothing, the kernels being bound by
// weight bytes).
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
// rows): weights are MFMA operand A (16 rows per stripe, four stripes = 64
// rows per work item) and tokens operand B (16 columns per tile, padded past
// L).  Every weight byte is used once, so weights stream from HBM with the
// non-temporal policy through a wave-private LDS ring (lds_stream.h): full
// 128-byte lines per load instruction, two 64-element steps in flight, the
// step stream continuing across work items.  Both kernels are persistent
// (one block per CU).  Each up block owns a contiguous equal share of the
// equal-sized up items; for the variable-length down items each XCD owns a
// range of equal step total, whose blocks take its items in turn (a chunk's
// hidden rows then stay in the XCD's L2).  A block's waves take its items
// through an LDS counter.  Items are decoded with scalar loads only, so
// nothing in the loop waits on a returning memory operation except the
// weight stream.
//
// The last eighth of the up items, and of each XCD's down items, is a pool
// that waves take through global counters once their static share is done,
// so whichever waves run ahead take the tail (chunk8: 1.1% off the step).
// A take waits for the wave's loads in flight (the counter's value is needed
// at once), so the pool is kept to the tail.  Down waves keep to their own
// XCD's pool: taking from other XCDs' pools (their chunks' hidden rows are
// in another L2) measured 7% slower.  Every item writes its own outputs, so
// the assignment of items to waves does not change any result.
//
// A few units cannot fill the GPU this way: one chunk of 8 tokens has about
// 38 up and 32 down items.  The SPLIT instantiations cut every up item into
// ks k-ranges and every down item into sp ranges of the union's slots; the
// items write fp32 partial tiles, and two small kernels add the partials in
// range order (then apply g * Swish, or store y).  The summation order
// differs from the unsplit kernels only in the last bits, and it is fixed
// for a given split, so results stay reproducible.
#include "lds_stream.h"

namespace bffn {
namespace {

// 64-bit wave shuffles, as two 32-bit halves.
__device__ __forceinline__ int64_t shfl_up64(int64_t v, int off) {
  const uint32_t lo = __shfl_up((uint32_t)v, off, kWave), hi = __shfl_up((uint32_t)((uint64_t)v >> 32), off, kWave);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)((uint64_t)v >> 32), off, kWave);
    v += (int64_t)(((uint64_t)hi << 32) | lo);
  }
  return v;
}

constexpr int kPlanMaxThreads = 1024;

// Exclusive prefix over chunks of the up-projection item counts
// (union size x row blocks, or E x row blocks in dense mode):
// prefix[u] = items of chunks < u, prefix[n_units] = total.  Then the down
// kernel's XCD ranges: the down items (chunk, 64 output rows) in chunk-major
// order start at step (U_u kbs + kb c_u) spe, with U_u the union sizes of
// the chunks before u; bounds[k] = the number of items starting before step
// k S / kXcds (S = all steps), the first item of XCD k's range.  One block of
// 64 to 1024 threads; each thread owns a run of consecutive chunks.  Scans
// and sums go through wave shuffles and one LDS exchange each, so the block
// meets at two barriers (this is on a single chunk's critical path).
__global__ __launch_bounds__(kPlanMaxThreads) void plan_items_kernel(const int32_t* __restrict__ count,
                                                                     int64_t n_units, int dense_E, int per_slot,
                                                                     int kbs, int spe,
                                                                     int64_t* __restrict__ prefix,
                                                                     int64_t* __restrict__ bounds) {
  constexpr int kMaxWaves = kPlanMaxThreads / kWave;
  __shared__ int64_t wave_tot[kMaxWaves];
  __shared__ int64_t wave_below[kXcds - 1][kMaxWaves];
  const int nth = blockDim.x, waves = nth / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int64_t per = (n_units + nth - 1) / nth;
  const int64_t b = tid * per, e = b + per < n_units ? b + per : n_units;
  int64_t sum = 0;
  for (int64_t u = b; u < e; ++u) sum += dense_E ? dense_E : count[u];
  // inclusive scan in the wave, then the totals of the waves before this one
  int64_t inc = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t v = shfl_up64(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane == kWave - 1) wave_tot[w] = inc;
  __syncthreads();
  int64_t first = inc - sum, total = 0;
  for (int j = 0; j < waves; ++j) {
    const int64_t t = wave_tot[j];
    if (j < w) first += t;
    total += t;
  }
  int64_t run = first;
  for (int64_t u = b; u < e; ++u) {
    prefix[u] = run * per_slot;
    run += dense_E ? dense_E : count[u];
  }
  if (tid == 0) prefix[n_units] = total * per_slot;
  // XCD ranges of the down items
  const int64_t S = total * kbs * spe;
  int64_t below[kXcds - 1];  // items of this thread's chunks starting before step k S / kXcds
#pragma unroll
  for (int k = 0; k < kXcds - 1; ++k) below[k] = 0;
  run = first;
  for (int64_t u = b; u < e; ++u) {
    const int64_t c = dense_E ? dense_E : count[u];
    const int64_t first_step = run * kbs * spe;  // step where chunk u's first item starts
#pragma unroll
    for (int k = 0; k < kXcds - 1; ++k) {
      const int64_t q = (int64_t)(k + 1) * S / kXcds - first_step;
      if (q <= 0) continue;
      if (c == 0) {
        below[k] += kbs;
      } else {
        const int64_t n = (q + c * spe - 1) / (c * spe);
        below[k] += n < kbs ? n : kbs;
      }
    }
    run += c;
  }
#pragma unroll
  for (int k = 0; k < kXcds - 1; ++k) {
    const int64_t v = wave_sum64(below[k]);
    if (lane == 0) wave_below[k][w] = v;
  }
  __syncthreads();
  if (tid < kXcds - 1) {
    int64_t v = 0;
    for (int j = 0; j < waves; ++j) v += wave_below[tid][j];
    bounds[tid + 1] = v;
  }
  if (tid == 0) {
    bounds[0] = 0;
    bounds[kXcds] = n_units * kbs;
  }
  // the pool counters after the bounds: [0] up items, [1 + k] XCD k's down items
  unsigned* pool = reinterpret_cast<unsigned*>(bounds + kXcds + 1);
  if (tid < 1 + kXcds) pool[tid] = 0;
}


constexpr int kPoolShift = 3;  // the pool is the last 1/8 of the items
constexpr int kUpShare = 4;    // blocks of one XCD that share an item range at two token tiles

// One ticket of a global work counter (agent scope), broadcast to the wave.
__device__ __forceinline__ int64_t take_global(unsigned* counter, int lane) {
  unsigned v = 0;
  if (lane == 0) v = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (int64_t)__builtin_amdgcn_readfirstlane(v);
}

struct UpItem {
  int64_t unit;
  int slot, rb, i, kp;
};

// ---- up-projection: H'[unit][slot] = g * Swish(X W_in[i]^T), items of 64 rows ----
template <int NT, bool DENSE, bool SPLIT>
__global__ __launch_bounds__(kBlock) void up_mfma_kernel(LayerArgs la, const uint16_t* __restrict__ x,
                                                         int64_t n_units, int L, const float* __restrict__ gates,
                                                         const int32_t* __restrict__ count,
                                                         const int32_t* __restrict__ list,
                                                         const int64_t* __restrict__ prefix,
                                                         uint16_t* __restrict__ hbuf, int ks,
                                                         float* __restrict__ part, unsigned* pool_ctr) {
  using G = RingGeom<NT, !SPLIT>;  // split items leave the gates to their epilogue
  // one LDS object: the four waves' rings, then the block's work counter
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kRingBufs * G::kBufBytes + 16];
  unsigned& taken = *reinterpret_cast<unsigned*>(lds + 4 * kRingBufs * G::kBufBytes);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int d = la.d, de = la.de, E = la.E, rbs = de >> 6;
  const int nsteps = d / kStepK / (SPLIT ? ks : 1);  // steps per item
  const int per_slot = SPLIT ? rbs * ks : rbs;       // items per union slot
  uint8_t* bufs = lds + w * kRingBufs * G::kBufBytes;
  // A split launch of at most kChunkSplitMaxUnits units gets no plan
  // (prefix == nullptr, which saves a launch on the single-chunk path): wave
  // 0 scans the chunks' item counts itself, lane u holding chunk u.
  __shared__ int64_t own_prefix[kChunkSplitMaxUnits + 1];
  if (SPLIT && prefix == nullptr) {  // (uniform)
    if (threadIdx.x < kWave) {
      const int u = threadIdx.x;
      int64_t c = u < n_units ? (int64_t)(DENSE ? E : count[u]) * per_slot : 0;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int64_t v = shfl_up64(c, off);
        if (u >= off) c += v;
      }
      if (u < n_units) own_prefix[u + 1] = c;
      if (u == 0) own_prefix[0] = 0;
    }
    __syncthreads();
    prefix = own_prefix;
  }
  // the block's items (all of equal size): a contiguous equal share.  With
  // two token tiles (a chunk's rows are 2 KiB x L, up to 256 KiB), kUpShare
  // blocks of one XCD take the union of their shares in turn, so that they
  // work on one chunk at a time and its token rows stay in that XCD's L2 (32
  // resident blocks each on its own chunk need 8 MB there).  (Giving all of
  // an XCD's blocks one range taken in turn keeps the rows in L2 too, but
  // then the XCD streams 32 neighbouring weight row blocks at once, in
  // 128-byte pieces 2 d bytes apart, and HBM efficiency drops more than the
  // re-read token rows cost: measured 5.45 against 6.49 TB/s at d = 4096.)
  const int64_t total = prefix[n_units];
  const int64_t pool_lo = SPLIT ? total : total - (total >> kPoolShift);
  constexpr int kShare = (NT == 2 && !SPLIT) ? kUpShare : 1;
  int64_t blk_lo, stride, item_end;
  if constexpr (kShare > 1) {  // the grid is a multiple of kXcds * kShare
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t lb = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;  // XCD-contiguous
    const int64_t grp = lb / kShare, groups = gridDim.x / kShare;
    blk_lo = grp * pool_lo / groups + lb % kShare;
    stride = kShare;
    item_end = (grp + 1) * pool_lo / groups;
  } else {
    blk_lo = (int64_t)blockIdx.x * pool_lo / gridDim.x;
    stride = 1;
    item_end = ((int64_t)blockIdx.x + 1) * pool_lo / gridDim.x;
  }
  bool in_pool = false;
  auto take = [&]() -> int64_t {  // an item index, or total when none is left
    if (!in_pool) {
      const int64_t it = take_item(&taken, blk_lo, stride, lane);
      if (it < item_end) return it;
      in_pool = true;
    }
    if constexpr (SPLIT) {
      return total;
    } else {
      const int64_t it = pool_lo + take_global(pool_ctr, lane);
      return it < total ? it : total;
    }
  };
  if (threadIdx.x == 0) taken = 0;
  __syncthreads();
  int64_t item = take();
  if (item >= total) return;

  auto decode = [&](int64_t it_idx) {
    int64_t lo = 0, hi = n_units - 1;  // last chunk whose prefix <= it_idx
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= it_idx) lo = mid; else hi = mid - 1;
    }
    UpItem it;
    it.unit = lo;
    const int r = (int)(it_idx - prefix[lo]);
    it.slot = r / per_slot;
    const int rem = r % per_slot;
    it.rb = SPLIT ? rem / ks : rem;
    it.kp = SPLIT ? rem % ks : 0;
    it.i = DENSE ? it.slot : list[lo * E + it.slot];
    return it;
  };
  // this lane's DMA sources for an item (step 0)
  const uint16_t* a_src[8];
  const uint16_t* b_src[G::kBInstr];
  const float* g_src;
  auto point = [&](const UpItem& it) {
    const uint16_t* wi = layer_ptr<kTWIn>(la, static_cast<const uint16_t*>(la.w_in), it.unit);
    const int k0 = it.kp * nsteps * kStepK;  // first k of the item's range
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int R = 8 * j + (lane >> 3);
      a_src[j] = wi + ((int64_t)it.i * de + it.rb * 64 + R) * d + k0 + dma_chunk_elems(R, lane);
    }
#pragma unroll
    for (int j = 0; j < G::kBInstr; ++j) {
      const int n = 8 * j + (lane >> 3);
      b_src[j] = x + (it.unit * L + n % L) * d + k0 + dma_chunk_elems(n, lane);
    }
    g_src = gates + (it.unit * L + lane % L) * E + it.i;
  };
  auto issue = [&](int slot, int k) {
    uint8_t* buf = bufs + slot * G::kBufBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16<kPolicyStream>(a_src[j] + k * kStepK, buf + j * 1024);
#pragma unroll
    for (int j = 0; j < G::kBInstr; ++j) dma16<kPolicyReuse>(b_src[j] + k * kStepK, buf + kABytes + j * 1024);
    if constexpr (!SPLIT) dma4(g_src, buf + G::kGateOff);
  };

  UpItem cmp = decode(item), nxt = cmp;
  point(cmp);
  int k_iss = 0, k_last = 0;
  bool iss_done = false, has_next = false;
  for (int b = 0; b < kRingBufs - 1; ++b) {  // nsteps >= kRingBufs - 1
    issue(b, k_iss);
    k_last = k_iss++;
  }
  f32x4 acc[4][NT];
  ring_zero<NT>(acc);
  int k_cmp = 0;
  for (int t = 0;; ++t) {
    // issue the step two ahead, or repeat a valid one past the end of the range
    if (!iss_done && k_iss == nsteps) {
      item = take();
      if (item < total) {
        nxt = decode(item);
        has_next = true;
        point(nxt);
        k_iss = 0;
      } else {
        iss_done = true;
      }
    }
    if (!iss_done) k_last = k_iss++;
    issue((t + kRingBufs - 1) % kRingBufs, k_last);
    wait_vmcnt<G::kWaitAhead>();
    const uint8_t* buf = bufs + (t % kRingBufs) * G::kBufBytes;
    ring_mfma<NT>(acc, buf, m, g);
    __builtin_amdgcn_sched_barrier(0);
    if (++k_cmp < nsteps) continue;
    if constexpr (SPLIT) {
      // item complete: its fp32 partial tile [token][64 rows]
      float* pb = part + ((((cmp.unit * E + cmp.slot) * rbs + cmp.rb) * (int64_t)ks + cmp.kp) * L) * 64;
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const int n = m + 16 * tl;
        if (n >= L) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s) *reinterpret_cast<f32x4*>(pb + n * 64 + 16 * s + 4 * g) = acc[s][tl];
      }
      if (!has_next) break;
      cmp = nxt;
      has_next = false;
      k_cmp = 0;
      ring_zero<NT>(acc);
      continue;
    }
    // item complete: g * Swish, bf16, to the hidden buffer (gates from this step's buffer)
    const float* gv_lds = reinterpret_cast<const float*>(buf + G::kGateOff);
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      const int n = m + 16 * tl;
      if (n >= L) continue;
      const float gv = gv_lds[n];
      uint16_t* hrow = hbuf + ((cmp.unit * E + cmp.slot) * L + n) * (int64_t)de + cmp.rb * 64 + 4 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f32x4 v = acc[s][tl];
        const uint32_t lo = pack2_bf16(gv * swish(v[0]), gv * swish(v[1]));
        const uint32_t hi = pack2_bf16(gv * swish(v[2]), gv * swish(v[3]));
        *reinterpret_cast<u32x2*>(hrow + s * 16) = u32x2{lo, hi};
      }
    }
    if (!has_next) break;
    cmp = nxt;
    has_next = false;
    k_cmp = 0;
    ring_zero<NT>(acc);
  }
  wait_vmcnt<0>();  // no LDS write may outlive the wave
}

// ---- up-projection at two token tiles, the block's four waves in lockstep ----
// At chunk lengths 17-32 a wave's ring slot (8 KiB of weights + 4 KiB of
// token rows) fills the LDS at three slots per wave, so each wave keeps two
// steps in flight.  Here the block takes groups of four consecutive items of
// one chunk, one per wave, which share the chunk's token rows: a slot holds
// the four waves' weight rows, the 32 token rows once, and the four waves'
// gates (37 KiB), and four slots keep three steps in flight per wave.  Each
// step a wave DMAs its 64 weight rows, 8 of the 32 token rows and its gates
// (10 instructions, so the wait is a constant), then meets the others at a
// barrier: past it every wave's loads for the step have landed and every
// wave has finished the step before, whose slot is refilled.  Items of a
// chunk are counted up to a multiple of four; a wave whose group position is
// past the chunk's items streams the group's first item (served from L2)
// and stores nothing.
constexpr int kLockBufs = 4;
constexpr int kLockA = 4 * kABytes;                // the four waves' weight rows
constexpr int kLockB = 32 * kRowBytes;             // the chunk's 32 token rows
constexpr int kLockGate = kLockA + kLockB;         // then 64 fp32 gates per wave
constexpr int kLockSlot = kLockGate + 4 * 256;
constexpr int kLockLoads = 8 + 1 + 1;              // DMA instructions per wave and step
constexpr int64_t kLockMaxUnits = 1024;            // group prefix kept in LDS
constexpr int kLockShare = 4;                      // blocks of one XCD that share a group range

__device__ __forceinline__ unsigned lds_addr(const uint8_t* p) { return (unsigned)(uintptr_t)(const lvoid_t*)p; }

// Six 16-byte LDS reads and their wait in one assembly block.  Written as C,
// the reads would be ordered after every LDS DMA in flight (the compiler
// cannot tell the ring's slots apart, and waits for vmcnt 0), which would
// drain the three steps this kernel keeps in flight; the slot read here was
// completed by the step's wait and barrier.
__device__ __forceinline__ void lds_read6(const unsigned (&ad)[6], u32x4 (&v)[6]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b128 %4, %10\n\t"
      "ds_read_b128 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5])
      : "memory");
}

// Two 4-byte LDS reads (the gates of a lane's two tokens) and their wait, for the same reason.
__device__ __forceinline__ void lds_read2f(unsigned a0, unsigned a1, float (&v)[2]) {
  asm volatile(
      "ds_read_b32 %0, %2\n\t"
      "ds_read_b32 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1])
      : "v"(a0), "v"(a1)
      : "memory");
}

__global__ __launch_bounds__(kBlock) void up_lock_kernel(LayerArgs la, const uint16_t* __restrict__ x,
                                                         int64_t n_units, int L, const float* __restrict__ gates,
                                                         const int32_t* __restrict__ count,
                                                         const int32_t* __restrict__ list,
                                                         uint16_t* __restrict__ hbuf, unsigned* pool_ctr) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLockBufs * kLockSlot];
  __shared__ int64_t gpre[kLockMaxUnits + 1];
  __shared__ int64_t wave_tot[kBlock / kWave];
  __shared__ unsigned pool_take;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
  const int d = la.d, de = la.de, E = la.E, rbs = de >> 6;
  const int nsteps = d / kStepK;
  // gpre[u] = groups of the chunks before u (a chunk's count x rbs items, rounded up to a multiple of 4)
  {
    const int64_t per = (n_units + kBlock - 1) / kBlock;
    const int64_t b = tid * per, e = b + per < n_units ? b + per : n_units;
    int64_t sum = 0;
    for (int64_t u = b; u < e; ++u) sum += ((int64_t)count[u] * rbs + 3) >> 2;
    int64_t inc = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int64_t v = shfl_up64(inc, off);
      if (lane >= off) inc += v;
    }
    if (lane == kWave - 1) wave_tot[w] = inc;
    __syncthreads();
    int64_t run = inc - sum, total = 0;
    for (int j = 0; j < kBlock / kWave; ++j) {
      if (j < w) run += wave_tot[j];
      total += wave_tot[j];
    }
    for (int64_t u = b; u < e; ++u) {
      gpre[u] = run;
      run += ((int64_t)count[u] * rbs + 3) >> 2;
    }
    if (tid == 0) gpre[n_units] = total;
    __syncthreads();
  }
  const int64_t total = gpre[n_units];
  // the block's groups: of the first 7/8, kLockShare blocks of one XCD take the union of their equal
  // shares in turn; then the block takes groups of the last 1/8 through the pool counter, one take per
  // block, broadcast through LDS (the take waits for wave 0's loads in flight, so it is kept to the tail)
  const int64_t pool_lo = total - (total >> kPoolShift);
  const int64_t per_xcd = gridDim.x / kXcds;  // the grid is a multiple of kXcds * kLockShare
  const int64_t lb = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int64_t grp = lb / kLockShare, groups = gridDim.x / kLockShare;
  const int64_t g_end = (grp + 1) * pool_lo / groups;
  int64_t g_static = grp * pool_lo / groups + lb % kLockShare;
  bool in_pool = false;
  auto next_group = [&]() -> int64_t {  // block-uniform: the next group, or -1
    if (!in_pool) {
      const int64_t gs = g_static;
      g_static += kLockShare;
      if (gs < g_end) return gs;
      in_pool = true;
    }
    if (threadIdx.x == 0) {
      pool_take = __hip_atomic_fetch_add(pool_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS write lands before the barrier (no fence there)
    }
    block_barrier_no_fence();
    const int64_t gp = pool_lo + (int64_t)__builtin_amdgcn_readfirstlane(pool_take);
    block_barrier_no_fence();  // every wave has read pool_take before a later take writes it
    return gp < total ? gp : -1;
  };
  const int64_t g_first = next_group();
  if (g_first < 0) return;  // (the whole block)

  struct LockItem {
    int64_t unit;
    int slot, rb, i;
    bool store;
  };
  auto decode = [&](int64_t gi) {
    int64_t lo = 0, hi = n_units - 1;  // last chunk whose group prefix <= gi
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (gpre[mid] <= gi) lo = mid; else hi = mid - 1;
    }
    LockItem it;
    it.unit = lo;
    const int first = (int)((gi - gpre[lo]) * 4);  // the group's first item in the chunk (always one of its items)
    int r = first + w;
    it.store = r < count[lo] * rbs;
    if (!it.store) r = first;
    it.slot = r / rbs;
    it.rb = r % rbs;
    it.i = list[lo * E + it.slot];
    return it;
  };
  const uint16_t* a_src[8];
  const uint16_t* b_src;
  const float* g_src;
  auto point = [&](const LockItem& it) {
    const uint16_t* wi = layer_ptr<kTWIn>(la, static_cast<const uint16_t*>(la.w_in), it.unit);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int R = 8 * j + (lane >> 3);
      a_src[j] = wi + ((int64_t)it.i * de + it.rb * 64 + R) * d + dma_chunk_elems(R, lane);
    }
    const int n = 8 * w + (lane >> 3);  // this wave's 8 of the 32 token rows
    b_src = x + (it.unit * L + n % L) * d + dma_chunk_elems(n, lane);
    g_src = gates + (it.unit * L + lane % L) * E + it.i;
  };
  auto issue = [&](int slot_i, int k) {
    uint8_t* buf = lds + slot_i * kLockSlot;
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16<kPolicyStream>(a_src[j] + k * kStepK, buf + w * kABytes + j * 1024);
    dma16<kPolicyReuse>(b_src + k * kStepK, buf + kLockA + w * 1024);
    dma4(g_src, buf + kLockGate + w * 256);
  };

  LockItem cmp = decode(g_first);
  point(cmp);
  int64_t g_pend = -1;  // the group the issue side has moved on to, not yet multiplied
  int k_iss = 0, k_last = 0;
  bool iss_done = false;
  for (int b = 0; b < kLockBufs - 1; ++b) {  // nsteps >= kLockBufs - 1 (d >= 192)
    issue(b, k_iss);
    k_last = k_iss++;
  }
  f32x4 acc[4][2];
  ring_zero<2>(acc);
  int k_cmp = 0;
  for (int t = 0;; ++t) {
    wait_vmcnt<(kLockBufs - 2) * kLockLoads>();  // this wave's loads of step t have landed
    block_barrier_no_fence();  // ... and every wave's; every wave is done with step t - 1
    // issue three steps ahead into step t - 1's slot, or repeat a valid one past the end
    if (!iss_done && k_iss == nsteps) {
      const int64_t gn = next_group();
      if (gn >= 0) {
        g_pend = gn;
        point(decode(gn));
        k_iss = 0;
      } else {
        iss_done = true;
      }
    }
    if (!iss_done) k_last = k_iss++;
    issue((t + kLockBufs - 1) % kLockBufs, k_last);
    // step t: this wave's 64 rows x the 32 shared token rows
    const uint8_t* buf = lds + (t % kLockBufs) * kLockSlot;
    const uint8_t* abuf = buf + w * kABytes;
    const uint8_t* bbuf = buf + kLockA;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      unsigned ad[6];  // LDS addresses: rows 16 s + m of A (s < 4), rows 16 tl + m of B
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int R = 16 * s + m;
        ad[s] = lds_addr(abuf + R * kRowBytes + (((4 * q + g) ^ ring_swz(R)) << 4));
      }
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        const int n = 16 * tl + m;
        ad[4 + tl] = lds_addr(bbuf + n * kRowBytes + (((4 * q + g) ^ ring_swz(n)) << 4));
      }
      u32x4 v[6];
      lds_read6(ad, v);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int tl = 0; tl < 2; ++tl)
          acc[s][tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring_bf16x8(v[s]), ring_bf16x8(v[4 + tl]), acc[s][tl],
                                                               0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (++k_cmp < nsteps) continue;
    // item complete: g * Swish, bf16, to the hidden buffer (gates from this step's slot)
    if (cmp.store) {
      const uint8_t* gv_lds = buf + kLockGate + w * 256;
      float gvs[2];
      lds_read2f(lds_addr(gv_lds + 4 * m), lds_addr(gv_lds + 4 * (m + 16)), gvs);
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        const int n = m + 16 * tl;
        if (n >= L) continue;
        const float gv = gvs[tl];
        uint16_t* hrow = hbuf + ((cmp.unit * E + cmp.slot) * L + n) * (int64_t)de + cmp.rb * 64 + 4 * g;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x4 v = acc[s][tl];
          const uint32_t lo = pack2_bf16(gv * swish(v[0]), gv * swish(v[1]));
          const uint32_t hi = pack2_bf16(gv * swish(v[2]), gv * swish(v[3]));
          *reinterpret_cast<u32x2*>(hrow + s * 16) = u32x2{lo, hi};
        }
      }
    }
    if (g_pend < 0) break;
    cmp = decode(g_pend);
    g_pend = -1;
    k_cmp = 0;
    ring_zero<2>(acc);
  }
  wait_vmcnt<0>();  // no LDS write may outlive the wave
}

// ---- down-projection: Y[unit][kb .. kb + 64) = sum over slots of H'[unit][slot] W_out[i]^T ----
// Items (chunk, 64 output rows) take count[chunk] * d_e / 64 steps; each XCD
// gets the items whose first step falls in its equal share of all steps.
template <int NT, bool DENSE, bool SPLIT>
__global__ __launch_bounds__(kBlock) void down_mfma_kernel(LayerArgs la, int64_t n_units, int L,
                                                           const int32_t* __restrict__ count,
                                                           const int32_t* __restrict__ list,
                                                           const int64_t* __restrict__ prefix,
                                                           const uint16_t* __restrict__ hbuf,
                                                           float* __restrict__ y, int sp,
                                                           float* __restrict__ part, unsigned* pool_ctr) {
  using G = RingGeom<NT, false>;
  // one LDS object: the four waves' rings, then the block's work counter
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kRingBufs * G::kBufBytes + 16];
  unsigned& taken = *reinterpret_cast<unsigned*>(lds + 4 * kRingBufs * G::kBufBytes);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int d = la.d, de = la.de, E = la.E;
  const int spe = de / kStepK;   // steps per expert
  const int kbs = d >> 6;        // 64-row blocks per chunk
  uint8_t* bufs = lds + w * kRingBufs * G::kBufBytes;

  auto nact = [&](int64_t u) { return (int64_t)(DENSE ? E : count[u]); };
  // the block's items: its turns in its XCD's range, the items whose first
  // step falls in an equal share of all steps (the last range also takes
  // items starting at the very end).  Split items (few units) are shared
  // out in contiguous ranges.
  const int64_t* bounds = prefix + n_units + 1;  // the XCD ranges, written by the plan kernel
  const int xcd = (int)(blockIdx.x % kXcds);
  int64_t blk_lo, stride, item_end;
  if constexpr (SPLIT) {
    const int64_t total = n_units * kbs * sp;
    blk_lo = (int64_t)blockIdx.x * total / gridDim.x;
    stride = 1;
    item_end = ((int64_t)blockIdx.x + 1) * total / gridDim.x;
  } else {  // the static part of the XCD's range, before its pool: block j of the XCD takes
            // the range's items j, j + (blocks per XCD), ..., so the XCD's waves work on
            // neighbouring items, whose chunks' hidden rows stay in its L2
    const int64_t lo = bounds[xcd], hi = bounds[xcd + 1];
    blk_lo = lo + (int64_t)blockIdx.x / kXcds;
    stride = gridDim.x / kXcds;  // the grid is a multiple of kXcds
    item_end = hi - ((hi - lo) >> kPoolShift);
  }
  bool in_pool = false;
  auto take = [&]() -> int64_t {  // an item index, or -1 when none is left
    if (!in_pool) {
      const int64_t it = take_item(&taken, blk_lo, stride, lane);
      if (it < item_end) return it;
      in_pool = true;
    }
    if constexpr (!SPLIT) {  // the XCD's pool: the rest of its range
      const int64_t hi = bounds[xcd + 1];
      const int64_t it = item_end + take_global(pool_ctr + 1 + xcd, lane);
      if (it < hi) return it;
    }
    return -1;
  };
  if (threadIdx.x == 0) taken = 0;
  __syncthreads();

  struct DownItem {
    int64_t unit, idx;
    int kb, nsteps, s0;
  };
  auto store_y = [&](const DownItem& it, const f32x4 (&acc)[4][NT]) {
    if constexpr (SPLIT) {  // the item's fp32 partial tile [token][64 rows]
      float* pb = part + it.idx * L * 64;
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const int n = m + 16 * tl;
        if (n >= L) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s) *reinterpret_cast<f32x4*>(pb + n * 64 + 16 * s + 4 * g) = acc[s][tl];
      }
      return;
    }
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      const int n = m + 16 * tl;
      if (n >= L) continue;
      float* yrow = y + (it.unit * L + n) * d + it.kb * 64 + 4 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<f32x4*>(yrow + s * 16) = acc[s][tl];
    }
  };
  // next item of the block's range with at least one step; chunks with an
  // empty union get y = 0 here
  auto next_item = [&](DownItem& it) -> bool {
    for (;;) {
      const int64_t item = take();
      if (item < 0) return false;
      it.idx = item;
      if constexpr (SPLIT) {  // (unit, kb, a range of the union's slots)
        it.unit = item / ((int64_t)kbs * sp);
        const int rem = (int)(item % ((int64_t)kbs * sp));
        it.kb = rem / sp;
        const int spi = rem % sp;
        const int S = (int)nact(it.unit), per = (S + sp - 1) / sp;
        const int s0 = spi * per < S ? spi * per : S;
        const int s1 = s0 + per < S ? s0 + per : S;
        it.s0 = s0;
        it.nsteps = (s1 - s0) * spe;
      } else {
        it.unit = item / kbs;
        it.kb = (int)(item % kbs);
        it.s0 = 0;
        it.nsteps = (int)nact(it.unit) * spe;
      }
      if (it.nsteps > 0) return true;
      f32x4 z[4][NT];
      ring_zero<NT>(z);
      store_y(it, z);
    }
    return false;
  };
  auto issue = [&](int slot_buf, const DownItem& it, int k) {
    const int sl = it.s0 + k / spe, j0 = (k % spe) * kStepK;
    const int i = DENSE ? sl : list[it.unit * E + sl];
    const uint16_t* wo = layer_ptr<kTWOut>(la, static_cast<const uint16_t*>(la.w_out), it.unit);
    const uint16_t* wbase = wo + ((int64_t)i * d + it.kb * 64) * de + j0;
    const uint16_t* hb = hbuf + ((it.unit * E + sl) * L) * (int64_t)de + j0;
    uint8_t* buf = bufs + slot_buf * G::kBufBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int R = 8 * j + (lane >> 3);
      dma16<kPolicyStream>(wbase + (int64_t)R * de + dma_chunk_elems(R, lane), buf + j * 1024);
    }
#pragma unroll
    for (int j = 0; j < G::kBInstr; ++j) {
      const int n = 8 * j + (lane >> 3);
      dma16<kPolicyReuse>(hb + (int64_t)(n % L) * de + dma_chunk_elems(n, lane), buf + kABytes + j * 1024);
    }
  };

  DownItem cmp;
  if (!next_item(cmp)) return;  // nothing issued
  DownItem iss = cmp, nxt = cmp, last_it = cmp;
  int k_iss = 0, k_last = 0;
  bool iss_done = false, has_next = false;
  auto advance_issue = [&]() {
    if (!iss_done && k_iss == iss.nsteps) {
      if (next_item(nxt)) {
        iss = nxt;
        has_next = true;
        k_iss = 0;
      } else {
        iss_done = true;
      }
    }
    if (!iss_done) {
      last_it = iss;
      k_last = k_iss++;
    }
  };
  for (int b = 0; b < kRingBufs - 1; ++b) {
    advance_issue();
    issue(b, last_it, k_last);
  }
  f32x4 acc[4][NT];
  ring_zero<NT>(acc);
  int k_cmp = 0;
  for (int t = 0;; ++t) {
    advance_issue();
    issue((t + kRingBufs - 1) % kRingBufs, last_it, k_last);
    wait_vmcnt<G::kWaitAhead>();
    ring_mfma<NT>(acc, bufs + (t % kRingBufs) * G::kBufBytes, m, g);
    __builtin_amdgcn_sched_barrier(0);
    if (++k_cmp < cmp.nsteps) continue;
    store_y(cmp, acc);
    if (!has_next) break;
    cmp = nxt;
    has_next = false;
    k_cmp = 0;
    ring_zero<NT>(acc);
  }
  wait_vmcnt<0>();  // no LDS write may outlive the wave
}

// ---- down-projection at two token tiles, the block's four waves in lockstep ----
// A group is (chunk, four consecutive 64-row output blocks), one block per
// wave; all four walk the chunk's union in the same order, so they share
// its hidden rows: a slot holds the four waves' W_out rows and the 32
// hidden rows once (36 KiB), and four slots keep three steps in flight (two
// with a slot per wave).  Each step a wave DMAs its 64 rows and
// a quarter of the hidden rows (9 instructions, so the wait is a constant)
// and meets the others at a fence-free barrier, as in up_lock_kernel.  XCD
// k takes the groups holding the plan's items [bounds[k], bounds[k + 1])
// (rounded up to whole groups); block j of the XCD takes its groups j,
// j + (blocks per XCD), ..., so the XCD works on neighbouring groups whose
// hidden rows stay in its L2, and the last eighth of the XCD's groups is a
// pool taken through the XCD's counter.  A chunk with an empty union gets
// y = 0 from the wave that takes its group.
constexpr int kDownLockA = 4 * kABytes;                  // the four waves' W_out rows
constexpr int kDownLockSlot = kDownLockA + 32 * kRowBytes;  // + the 32 hidden rows
constexpr int kDownLockLoads = 8 + 1;

__global__ __launch_bounds__(kBlock) void down_lock_kernel(LayerArgs la, int64_t n_units, int L,
                                                           const int32_t* __restrict__ count,
                                                           const int32_t* __restrict__ list,
                                                           const int64_t* __restrict__ prefix,
                                                           const uint16_t* __restrict__ hbuf,
                                                           float* __restrict__ y, unsigned* pool_ctr) {
  constexpr int NT = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLockBufs * kDownLockSlot];
  __shared__ unsigned pool_take;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int d = la.d, de = la.de, E = la.E;
  const int spe = de / kStepK;  // steps per expert
  const int gpc = (d >> 6) / 4;  // groups per chunk
  const int64_t* bounds = prefix + n_units + 1;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int64_t glo = (bounds[xcd] + 3) >> 2, ghi = (bounds[xcd + 1] + 3) >> 2;
  const int64_t gstat_end = ghi - ((ghi - glo) >> kPoolShift);
  const int64_t gstride = gridDim.x / kXcds;  // the grid is a multiple of kXcds
  int64_t g_static = glo + blockIdx.x / kXcds;
  bool in_pool = false;
  auto next_group = [&]() -> int64_t {  // block-uniform: the next group of this XCD, or -1
    if (!in_pool) {
      const int64_t gs = g_static;
      g_static += gstride;
      if (gs < gstat_end) return gs;
      in_pool = true;
    }
    if (threadIdx.x == 0) {
      pool_take = __hip_atomic_fetch_add(pool_ctr + 1 + xcd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS write lands before the barrier (no fence there)
    }
    block_barrier_no_fence();
    const int64_t gp = gstat_end + (int64_t)__builtin_amdgcn_readfirstlane(pool_take);
    block_barrier_no_fence();  // every wave has read pool_take before a later take writes it
    return gp < ghi ? gp : -1;
  };
  struct LockGroup {
    int64_t unit;
    int kb, nsteps;
  };
  auto decode = [&](int64_t gi) {
    LockGroup it;
    it.unit = gi / gpc;
    it.kb = (int)(gi % gpc) * 4 + w;
    it.nsteps = count[it.unit] * spe;
    return it;
  };
  auto store_y = [&](const LockGroup& it, const f32x4 (&acc)[4][NT]) {
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      const int n = m + 16 * tl;
      if (n >= L) continue;
      float* yrow = y + (it.unit * L + n) * d + it.kb * 64 + 4 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<f32x4*>(yrow + s * 16) = acc[s][tl];
    }
  };
  // the next group with at least one step; groups of chunks with an empty union get y = 0 here
  auto next_nonempty = [&](LockGroup& it) -> bool {
    for (;;) {
      const int64_t gi = next_group();
      if (gi < 0) return false;
      it = decode(gi);
      if (it.nsteps > 0) return true;
      f32x4 z[4][NT];
      ring_zero<NT>(z);
      store_y(it, z);
    }
  };
  auto issue = [&](int slot_i, const LockGroup& it, int k) {
    const int sl = k / spe, j0 = (k % spe) * kStepK;
    const int i = list[it.unit * E + sl];
    const uint16_t* wo = layer_ptr<kTWOut>(la, static_cast<const uint16_t*>(la.w_out), it.unit);
    const uint16_t* wbase = wo + ((int64_t)i * d + it.kb * 64) * de + j0;
    const uint16_t* hb = hbuf + ((it.unit * E + sl) * L) * (int64_t)de + j0;
    uint8_t* buf = lds + slot_i * kDownLockSlot;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int R = 8 * jj + (lane >> 3);
      dma16<kPolicyStream>(wbase + (int64_t)R * de + dma_chunk_elems(R, lane), buf + w * kABytes + jj * 1024);
    }
    const int n = 8 * w + (lane >> 3);  // this wave's 8 of the 32 hidden rows
    dma16<kPolicyReuse>(hb + (int64_t)(n % L) * de + dma_chunk_elems(n, lane), buf + kDownLockA + 8 * w * kRowBytes);
  };

  LockGroup cmp, iss;
  if (!next_nonempty(cmp)) return;  // (the whole block)
  iss = cmp;
  // groups the issue side has moved on to, not yet multiplied: three steps in flight and at least
  // two steps per group (d_e >= 128) make at most two
  LockGroup last_it = cmp, pend0 = cmp, pend1 = cmp;  // (named, not an array: kept in registers)
  int n_pend = 0;
  bool iss_done = false;
  int k_iss = 0, k_last = 0;
  auto advance_issue = [&]() {
    if (!iss_done && k_iss == iss.nsteps) {
      LockGroup nx;
      if (next_nonempty(nx)) {
        iss = nx;
        if (n_pend == 0)
          pend0 = nx;
        else
          pend1 = nx;
        ++n_pend;
        k_iss = 0;
      } else {
        iss_done = true;
      }
    }
    if (!iss_done) {
      last_it = iss;
      k_last = k_iss++;
    }
  };
  for (int b = 0; b < kLockBufs - 1; ++b) {
    advance_issue();
    issue(b, last_it, k_last);
  }
  f32x4 acc[4][NT];
  ring_zero<NT>(acc);
  int k_cmp = 0;
  for (int t = 0;; ++t) {
    wait_vmcnt<(kLockBufs - 2) * kDownLockLoads>();  // this wave's loads of step t have landed
    block_barrier_no_fence();  // ... and every wave's; every wave is done with step t - 1
    advance_issue();
    issue((t + kLockBufs - 1) % kLockBufs, last_it, k_last);
    const uint8_t* buf = lds + (t % kLockBufs) * kDownLockSlot;
    const uint8_t* abuf = buf + w * kABytes;
    const uint8_t* bbuf = buf + kDownLockA;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      unsigned ad[4 + NT];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int R = 16 * s + m;
        ad[s] = lds_addr(abuf + R * kRowBytes + (((4 * q + g) ^ ring_swz(R)) << 4));
      }
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const int n = 16 * tl + m;
        ad[4 + tl] = lds_addr(bbuf + n * kRowBytes + (((4 * q + g) ^ ring_swz(n)) << 4));
      }
      u32x4 v[4 + NT];
      lds_read6(ad, v);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int tl = 0; tl < NT; ++tl)
          acc[s][tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring_bf16x8(v[s]), ring_bf16x8(v[4 + tl]), acc[s][tl],
                                                               0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (++k_cmp < cmp.nsteps) continue;
    store_y(cmp, acc);
    if (n_pend == 0) break;
    cmp = pend0;
    pend0 = pend1;
    --n_pend;
    k_cmp = 0;
    ring_zero<NT>(acc);
  }
  wait_vmcnt<0>();  // no LDS write may outlive the wave
}

// h'[unit][slot][token][64 rb + r] = g * Swish(sum over k-ranges, in order, of
// the up items' partial tiles), bf16; one block per (unit, slot, row block).
__global__ __launch_bounds__(kBlock) void up_split_epilogue_kernel(const float* __restrict__ part,
                                                                   const float* __restrict__ gates,
                                                                   const int32_t* __restrict__ count,
                                                                   const int32_t* __restrict__ list, int L, int E,
                                                                   int de, int ks, uint16_t* __restrict__ hbuf) {
  const int rbs = de >> 6;
  const int64_t b = blockIdx.x;
  const int rb = (int)(b % rbs);
  const int slot = (int)((b / rbs) % E);
  const int64_t u = b / ((int64_t)rbs * E);
  if (slot >= count[u]) return;
  const int i = list[u * E + slot];
  const float* pb = part + (((u * E + slot) * rbs + rb) * (int64_t)ks) * L * 64;
  for (int idx = threadIdx.x; idx < L * 64; idx += kBlock) {
    const int n = idx >> 6, r = idx & 63;
    float v = pb[idx];
    for (int kp = 1; kp < ks; ++kp) v += pb[(int64_t)kp * L * 64 + idx];
    const float gv = gates[(u * L + n) * E + i];
    hbuf[((u * E + slot) * L + n) * (int64_t)de + rb * 64 + r] = (uint16_t)f32_to_bf16(gv * swish(v));
  }
}

// y[unit L + token][64 kb + r] = sum over slot ranges, in order, of the down
// items' partial tiles; one block per (unit, row block).
__global__ __launch_bounds__(kBlock) void down_split_combine_kernel(const float* __restrict__ part, int L, int d,
                                                                    int sp, float* __restrict__ y) {
  const int kbs = d >> 6;
  const int64_t b = blockIdx.x;
  const int kb = (int)(b % kbs);
  const int64_t u = b / kbs;
  const float* pb = part + b * sp * (int64_t)L * 64;
  for (int idx = threadIdx.x; idx < L * 64; idx += kBlock) {
    float v = pb[idx];
    for (int j = 1; j < sp; ++j) v += pb[(int64_t)j * L * 64 + idx];
    y[(u * L + (idx >> 6)) * (int64_t)d + kb * 64 + (idx & 63)] = v;
  }
}

template <int NT, bool DENSE, bool SPLIT>
hipError_t launch_nt(const LayerArgs& la, const uint16_t* x, int64_t units, int L, const float* gates,
                     const int32_t* count, const int32_t* list, uint16_t* hbuf, int64_t* plan, float* y,
                     const ChunkSplit& sp, const StageEvents& se, hipStream_t s) {
  const int rbs = la.de >> 6;
  const int ks = SPLIT ? sp.ks : 1;
  // A split launch of few units needs only the item prefix, which its up
  // kernel computes itself; every other launch gets the plan kernel (one
  // thread per chunk up to the block's maximum, whole waves).
  const bool own_prefix = SPLIT && units <= kChunkSplitMaxUnits;
  if (!own_prefix) {
    const int plan_threads =
        units < kPlanMaxThreads ? (int)((units + kWave - 1) / kWave * kWave) : kPlanMaxThreads;
    plan_items_kernel<<<dim3(1), dim3((unsigned)plan_threads), 0, s>>>(count, units, DENSE ? la.E : 0, rbs * ks,
                                                                       la.d >> 6, rbs, plan, plan + units + 1);
  }
  // persistent grids sized to the resident capacity (one block per CU at this LDS use)
  int64_t grid_up = 0, grid_dn = 0;
  hipError_t e =
      resident_blocks(reinterpret_cast<const void*>(&up_mfma_kernel<NT, DENSE, SPLIT>), kBlock, &grid_up);
  if (e == hipSuccess)
    e = resident_blocks(reinterpret_cast<const void*>(&down_mfma_kernel<NT, DENSE, SPLIT>), kBlock, &grid_dn);
  if (e != hipSuccess) return e;
  // the item shares assume the grid is a multiple of the XCD count
  const int64_t up_mult = (NT == 2 && !SPLIT) ? kXcds * kUpShare : kXcds;  // see the up kernel's item shares
  grid_up = grid_up / up_mult * up_mult > 0 ? grid_up / up_mult * up_mult : up_mult;
  grid_dn = grid_dn / kXcds * kXcds > 0 ? grid_dn / kXcds * kXcds : kXcds;
  // two token tiles: the lockstep up kernel (its group prefix lives in LDS; it needs three steps of d)
  const bool lock = NT == 2 && !DENSE && !SPLIT && units <= kLockMaxUnits && la.d / kStepK >= kLockBufs - 1;
  int64_t grid_lock = 0;
  if (lock) {
    e = resident_blocks(reinterpret_cast<const void*>(&up_lock_kernel), kBlock, &grid_lock);
    if (e != hipSuccess) return e;
    const int64_t mult = kXcds * kLockShare;  // see the kernel's group shares
    grid_lock = grid_lock / mult * mult > 0 ? grid_lock / mult * mult : mult;
  }
  // the lockstep down kernel at two token tiles: groups of four 64-row blocks of a chunk (d a multiple
  // of 256).  (At one token tile, where the shared hidden rows are a fifth of a step, it measured about
  // 1% slower than the per-wave kernel: 6.22 against 6.26 TB/s on chunk8, 6.56 against 6.67 on decode.)
  const bool down_lock = NT == 2 && !DENSE && !SPLIT && (la.d >> 6) % 4 == 0;
  int64_t grid_dn_lock = 0;
  if (down_lock) {
    e = resident_blocks(reinterpret_cast<const void*>(&down_lock_kernel), kBlock, &grid_dn_lock);
    if (e != hipSuccess) return e;
    grid_dn_lock = grid_dn_lock / kXcds * kXcds > 0 ? grid_dn_lock / kXcds * kXcds : kXcds;
  }
  se.record(0, s);
  // the pool counters follow the prefix and the XCD bounds in the plan
  unsigned* pool = reinterpret_cast<unsigned*>(plan + units + 1 + kXcds + 1);
  if (lock)
    up_lock_kernel<<<dim3((unsigned)grid_lock), dim3(kBlock), 0, s>>>(la, x, units, L, gates, count, list, hbuf,
                                                                      pool);
  else
    up_mfma_kernel<NT, DENSE, SPLIT><<<dim3((unsigned)grid_up), dim3(kBlock), 0, s>>>(
        la, x, units, L, gates, count, list, own_prefix ? nullptr : plan, hbuf, ks, sp.up_part, pool);
  if (SPLIT)
    up_split_epilogue_kernel<<<dim3((unsigned)(units * la.E * rbs)), dim3(kBlock), 0, s>>>(
        sp.up_part, gates, count, list, L, la.E, la.de, ks, hbuf);
  se.record(1, s);
  if (down_lock)
    down_lock_kernel<<<dim3((unsigned)grid_dn_lock), dim3(kBlock), 0, s>>>(la, units, L, count, list, plan, hbuf,
                                                                          y, pool);
  else
    down_mfma_kernel<NT, DENSE, SPLIT><<<dim3((unsigned)grid_dn), dim3(kBlock), 0, s>>>(
        la, units, L, count, list, plan, hbuf, y, SPLIT ? sp.sp : 1, sp.down_part, pool);
  if (SPLIT)
    down_split_combine_kernel<<<dim3((unsigned)(units * (la.d >> 6))), dim3(kBlock), 0, s>>>(sp.down_part, L, la.d,
                                                                                          sp.sp, y);
  se.record(2, s);
  return hipGetLastError();
}

}  // namespace

bool forward_mfma_supported(int d, int de, int dtype) {
  return dtype == BLOCKFFN_BF16 && d % 128 == 0 && de % 128 == 0;
}

size_t forward_mfma_plan_bytes(int64_t units) {
  return sizeof(int64_t) * (size_t)(units + 1 + kXcds + 1) + sizeof(unsigned) * (1 + kXcds);
}

bool chunk_split_factors(int d, int de, int64_t units, bool force, int* ks, int* sp) {
  (void)de;
  *ks = 1;
  *sp = 1;
  if (!force && (units < 1 || units > kChunkSplitMaxUnits)) return false;
  // k-ranges of at least 4 steps (the ring keeps two steps in flight), up to 8
  const int nsteps = d / kStepK;
  while (*ks < 8 && nsteps % (2 * *ks) == 0 && nsteps / (2 * *ks) >= 4) *ks *= 2;
  *sp = 8;
  return true;
}

size_t chunk_split_part_bytes(int d, int de, int E, int64_t units, int chunk_len, int ks, int sp,
                              size_t* down_offset) {
  const size_t up = (size_t)units * E * (de >> 6) * ks * chunk_len * 64 * sizeof(float);
  const size_t up_rounded = (up + 255) & ~size_t(255);
  const size_t down = (size_t)units * (d >> 6) * sp * chunk_len * 64 * sizeof(float);
  if (down_offset) *down_offset = up_rounded;
  return up_rounded + ((down + 255) & ~size_t(255));
}

hipError_t launch_forward_mfma(const LayerArgs& la, const uint16_t* x, int64_t n_tokens, int chunk_len,
                               const float* gates, const int32_t* count, const int32_t* list, bool dense,
                               uint16_t* hbuf, int64_t* plan, const ChunkSplit& sp, float* y,
                               const StageEvents& se, hipStream_t s) {
  const int64_t units = n_tokens / chunk_len;
  if (units == 0) return hipSuccess;
  if (dense) {
    if (chunk_len <= 16)
      return launch_nt<1, true, false>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, sp, se, s);
    return launch_nt<2, true, false>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, sp, se, s);
  }
  if (sp.ks > 0) {
    if (chunk_len <= 16)
      return launch_nt<1, false, true>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, sp, se, s);
    return launch_nt<2, false, true>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, sp, se, s);
  }
  if (chunk_len <= 16)
    return launch_nt<1, false, false>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, sp, se, s);
  return launch_nt<2, false, false>(la, x, units, chunk_len, gates, count, list, hbuf, plan, y, sp, se, s);
}

}  // namespace bffn
