// FFF tree layer: hard-routed walks through P perfect binary trees
// ("Dynamic sparsity in tree-structured feed-forward layers at scale",
// gist.science write-up, §2 methodology: architecture design and key
// mechanisms; §4: efficiency).
//
// Per token and tree the walk visits D + 1 heap-ordered nodes: at node n it
// forms c = w_node[n] . x + b[n], continues to the right child iff c > 0, and
// adds GELU(c) w_out[n] to the token's output (or c w_out[n], with GELU on
// the finished sum, in the post variant).  Dense mode visits every node.
//
// Each (token, tree) is a chain of dependent row fetches: the next node is
// known only once the current dot product is reduced.  A visited node
// streams its two rows (2 d elements) for about 4 d FLOP, so the layer is
// bound by HBM bandwidth, provided enough chains are in flight to cover the
// latency of each link.
//  * One block of four waves per token.  Wave w walks trees w, w + 4, ...,
//    kTreePar of them in lockstep, so a wave has 2 kTreePar rows in flight
//    per level, and a CU holds several blocks: thousands of independent
//    chains cover the memory latency.
//  * A row is spread over the wave in 16-byte pieces (piece j of lane l is
//    bytes 1024 j + 16 l), so every load instruction reads 1 KiB contiguous.
//    Node rows are read once per walk, with the non-temporal policy (10%
//    faster than cached loads at d = 2048, 64 trees of depth 6); a layer whose
//    node rows are interleaved (input row, then output row) costs one
//    contiguous read per visited node, a further 3%.
//    The token's x is held in registers in the same layout for the whole
//    walk, and so are the lane's output accumulators.
//  * The dot product is reduced by a butterfly and broadcast from lane 0, so
//    the turn is wave-uniform and the node index stays scalar.
//  * The waves' partial outputs are added in LDS in a fixed order (wave 0,
//    then 1, 2, 3), so the output is deterministic.
//  * Few tokens cannot fill the GPU one block each, and a lone token would
//    walk its trees a pair at a time.  A token's trees are then split into
//    G groups, one block each; the blocks write fp32 partial outputs to a
//    workspace and a second kernel adds the G partials in group order (and
//    applies the post-aggregation GELU).  G is chosen from the token count
//    alone, so a given call is reproducible.
#include "fff_probe_launch.h"

namespace bffn {
namespace {

constexpr int kFffWaves = 4;
constexpr int kTreePar = 2;  // trees a wave walks in lockstep

struct FffArgs {
  const uint8_t* w_node;
  const float* b_node;
  const uint8_t* w_out;
  int64_t stride;       // bytes between consecutive layers (0 with one layer)
  int64_t node_stride;  // bytes between consecutive nodes' rows
  int32_t n_layers;
  int32_t listed;       // 1: layer l's pointers are tab[*][l]
  int32_t P, D;
  int32_t post, dense;
  const uint8_t* x;
  float* y;
  int32_t* paths;
  float* preact;
  int32_t G;          // blocks per token
  int32_t per_group;  // trees per block
  float* partial;     // [T][G][d] when G > 1
  const void* tab[3][kMaxListedLayers];  // w_node, b_node, w_out of each listed layer
};

// exact GELU, c Phi(c)
__device__ __forceinline__ float gelu_erf(float c) { return 0.5f * c * (1.f + erff(c * 0.70710678118654752f)); }

template <bool BF16>
constexpr int piece_elems() {
  return BF16 ? 8 : 4;
}

// one 16-byte piece of a row, widened to fp32
template <bool BF16>
__device__ __forceinline__ void widen(const u32x4& v, float* f) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}

template <int NCH, bool BF16>
struct Walker {
  static constexpr int kEP = piece_elems<BF16>();
  static constexpr int kEL = NCH * kEP;  // elements of a row per lane
  static constexpr int64_t kRowBytes = int64_t(NCH) * 1024;

  const FffArgs& a;
  const uint8_t* wn;
  const uint8_t* wo;
  const float* bn;
  int64_t t, nodes;
  int lane;
  float xf[kEL];
  float acc[kEL];

  // Walk trees p, p + kFffWaves, ..., TP of them in lockstep.
  template <int TP>
  __device__ __forceinline__ void walk(int p) {
    int node[TP];
#pragma unroll
    for (int q = 0; q < TP; ++q) node[q] = 0;
    const int V = a.dense ? (int)nodes : a.D + 1;
    for (int l = 0; l < V; ++l) {
      u32x4 wv[TP][NCH], ov[TP][NCH];
      int64_t row[TP];
#pragma unroll
      for (int q = 0; q < TP; ++q) {
        row[q] = (int64_t)(p + kFffWaves * q) * nodes + (a.dense ? l : node[q]);
        const uint8_t* rn = wn + row[q] * a.node_stride + lane * 16;
        const uint8_t* ro = wo + row[q] * a.node_stride + lane * 16;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          wv[q][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rn + j * 1024));
          ov[q][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ro + j * 1024));
        }
      }
#pragma unroll
      for (int q = 0; q < TP; ++q) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          float f[kEP];
          widen<BF16>(wv[q][j], f);
#pragma unroll
          for (int i = 0; i < kEP; ++i) s = fmaf(f[i], xf[j * kEP + i], s);
        }
        s = wave_sum(s);
        float c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s)));
        if (bn) c += bn[row[q]];
        if (lane == 0) {
          const int64_t rec = (t * a.P + p + kFffWaves * q) * (a.D + 1) + l;
          if (a.paths) a.paths[rec] = node[q];
          if (a.preact) a.preact[rec] = c;
        }
        const float av = a.post ? c : gelu_erf(c);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          float f[kEP];
          widen<BF16>(ov[q][j], f);
#pragma unroll
          for (int i = 0; i < kEP; ++i) acc[j * kEP + i] = fmaf(av, f[i], acc[j * kEP + i]);
        }
        if (!a.dense) node[q] = 2 * node[q] + 1 + (c > 0.f ? 1 : 0);
      }
    }
  }
};

template <int NCH, bool BF16>
__global__ __launch_bounds__(kFffWaves * kWave) void fff_kernel(FffArgs a) {
  using W = Walker<NCH, BF16>;
  extern __shared__ __attribute__((aligned(16))) float part[];  // [kFffWaves - 1][d]
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = (int64_t)(blockIdx.x / (unsigned)a.G);
  const int g = (int)(blockIdx.x % (unsigned)a.G);
  const int64_t layer = a.n_layers > 1 ? t % a.n_layers : 0;
  const bool listed = a.listed && a.n_layers > 1;
  W wk{a,
       listed ? static_cast<const uint8_t*>(a.tab[0][layer]) : a.w_node + layer * a.stride,
       listed ? static_cast<const uint8_t*>(a.tab[2][layer]) : a.w_out + layer * a.stride,
       listed   ? static_cast<const float*>(a.tab[1][layer])
       : a.b_node ? reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.b_node) + layer * a.stride)
                  : nullptr,
       t,
       (int64_t(1) << (a.D + 1)) - 1,
       (int)(threadIdx.x & 63),
       {},
       {}};
  const uint8_t* xr = a.x + t * W::kRowBytes + wk.lane * 16;
#pragma unroll
  for (int j = 0; j < NCH; ++j) widen<BF16>(*reinterpret_cast<const u32x4*>(xr + j * 1024), wk.xf + j * W::kEP);
#pragma unroll
  for (int e = 0; e < W::kEL; ++e) wk.acc[e] = 0.f;

  const int p_lo = g * a.per_group;
  const int p_hi = p_lo + a.per_group < a.P ? p_lo + a.per_group : a.P;
  int p = p_lo + w;
  for (; p + kFffWaves * (kTreePar - 1) < p_hi; p += kFffWaves * kTreePar) wk.template walk<kTreePar>(p);
  for (; p < p_hi; p += kFffWaves) wk.template walk<1>(p);

  // fixed-order sum of the four waves' partial outputs
  const int d = NCH * 1024 / (BF16 ? 2 : 4);
  if (w > 0) {
    float* dst = part + (w - 1) * d;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < W::kEP; i += 4)
        *reinterpret_cast<f32x4*>(dst + (j * 64 + wk.lane) * W::kEP + i) =
            f32x4{wk.acc[j * W::kEP + i], wk.acc[j * W::kEP + i + 1], wk.acc[j * W::kEP + i + 2],
                  wk.acc[j * W::kEP + i + 3]};
  }
  __syncthreads();
  if (w == 0) {
    const bool whole = a.G == 1;  // else a partial output for the combine
    float* yr = whole ? a.y + t * d : a.partial + ((int64_t)t * a.G + g) * d;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < W::kEP; i += 4) {
        const int e = (j * 64 + wk.lane) * W::kEP + i;
        f32x4 v{wk.acc[j * W::kEP + i], wk.acc[j * W::kEP + i + 1], wk.acc[j * W::kEP + i + 2],
                wk.acc[j * W::kEP + i + 3]};
#pragma unroll
        for (int r = 0; r < kFffWaves - 1; ++r) v += *reinterpret_cast<const f32x4*>(part + r * d + e);
        if (whole && a.post) v = f32x4{gelu_erf(v[0]), gelu_erf(v[1]), gelu_erf(v[2]), gelu_erf(v[3])};
        *reinterpret_cast<f32x4*>(yr + e) = v;
      }
  }
}

// y[t] = sum over g = 0..G-1, in order, of partial[t][g] (then GELU in the
// post variant).  Block b covers 1024 elements of one token's row.
__global__ __launch_bounds__(kBlock) void fff_combine_kernel(const float* __restrict__ partial, int G, int d,
                                                             int chunks, int post, float* __restrict__ y) {
  const int64_t t = blockIdx.x / (unsigned)chunks;
  const int e = (int)(blockIdx.x % (unsigned)chunks) * 1024 + threadIdx.x * 4;
  if (e >= d) return;
  const float* src = partial + t * G * (int64_t)d + e;
  f32x4 v = *reinterpret_cast<const f32x4*>(src);
  for (int g = 1; g < G; ++g) v += *reinterpret_cast<const f32x4*>(src + (int64_t)g * d);
  if (post) v = f32x4{gelu_erf(v[0]), gelu_erf(v[1]), gelu_erf(v[2]), gelu_erf(v[3])};
  *reinterpret_cast<f32x4*>(y + t * d + e) = v;
}

template <int NCH, bool BF16>
hipError_t launch_nch(const FffArgs& a, int64_t n_tokens, hipStream_t s) {
  const int d = NCH * 1024 / (BF16 ? 2 : 4);
  const size_t lds = sizeof(float) * (kFffWaves - 1) * d;
  fff_kernel<NCH, BF16><<<dim3((unsigned)(n_tokens * a.G)), dim3(kFffWaves * kWave), lds, s>>>(a);
  if (a.G > 1) {
    const int chunks = (d + 1023) / 1024;
    fff_combine_kernel<<<dim3((unsigned)(n_tokens * chunks)), dim3(kBlock), 0, s>>>(a.partial, a.G, d, chunks,
                                                                                 a.post, a.y);
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const FffArgs& a, int nch, int64_t n_tokens, hipStream_t s) {
  switch (nch) {
    case 1: return launch_nch<1, BF16>(a, n_tokens, s);
    case 2: return launch_nch<2, BF16>(a, n_tokens, s);
    case 3: return launch_nch<3, BF16>(a, n_tokens, s);
    case 4: return launch_nch<4, BF16>(a, n_tokens, s);
    case 5: return launch_nch<5, BF16>(a, n_tokens, s);
    case 6: return launch_nch<6, BF16>(a, n_tokens, s);
    case 7: return launch_nch<7, BF16>(a, n_tokens, s);
    case 8: return launch_nch<8, BF16>(a, n_tokens, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int fff_max_split(int n_trees) { return (n_trees + kFffWaves - 1) / kFffWaves; }

int fff_split(int n_trees, int64_t n_tokens, int requested) {
  const int gmax = fff_max_split(n_trees);
  if (requested > 0) return requested < gmax ? requested : gmax;
  if (n_tokens <= 0 || n_tokens >= kFffTargetBlocks) return 1;
  const int64_t g = (kFffTargetBlocks + n_tokens - 1) / n_tokens;
  return (int)(g < gmax ? g : gmax);
}

size_t fff_workspace_bytes(int d, int n_trees, int64_t n_tokens, int requested) {
  const int G = fff_split(n_trees, n_tokens, requested);
  return G > 1 ? (size_t)n_tokens * G * d * sizeof(float) : 0;
}

bool fff_width_supported(int d, int dtype) {
  const int esz = dtype == BLOCKFFN_BF16 ? 2 : 4;
  return d > 0 && (d * esz) % 1024 == 0 && d * esz / 1024 <= kFffMaxPieces;
}

hipError_t launch_fff_forward(const blockffn_fff_layer& ly, const FffLayerSet& set, const void* x, int64_t n_tokens,
                              bool dense, int split, int32_t* paths, float* preact, void* workspace, float* y,
                              hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  FffArgs a;
  a.w_node = static_cast<const uint8_t*>(ly.w_node);
  a.b_node = ly.b_node;
  a.w_out = static_cast<const uint8_t*>(ly.w_out);
  a.stride = set.n_layers > 1 ? set.stride : 0;
  a.node_stride = ly.node_stride ? ly.node_stride : (int64_t)ly.d * (ly.dtype == BLOCKFFN_BF16 ? 2 : 4);
  a.n_layers = set.n_layers;
  a.listed = set.listed;
  for (int k = 0; k < 3; ++k)
    for (int l = 0; l < kMaxListedLayers; ++l) a.tab[k][l] = set.tab[k][l];
  a.P = ly.n_trees;
  a.D = ly.depth;
  a.post = ly.activation == BLOCKFFN_FFF_GELU_OUTPUT;
  a.dense = dense;
  a.x = static_cast<const uint8_t*>(x);
  a.y = y;
  a.paths = paths;
  a.preact = preact;
  a.G = fff_split(ly.n_trees, n_tokens, split);
  a.per_group = (ly.n_trees + a.G - 1) / a.G;
  a.partial = static_cast<float*>(workspace);
  const bool bf16 = ly.dtype == BLOCKFFN_BF16;
  const int nch = ly.d * (bf16 ? 2 : 4) / 1024;
  return bf16 ? launch_dtype<true>(a, nch, n_tokens, s) : launch_dtype<false>(a, nch, n_tokens, s);
}

}  // namespace bffn
