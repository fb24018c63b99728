// C ABI of libblockffn: host-side validation, mode selection and dispatch to
// the gfx950 kernels.  Validation never touches the HIP runtime, so a call
// that fails it enqueues nothing (and works on a machine without a GPU).
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include <map>
#include <mutex>
#include <utility>

#include "bffn_internal.h"
#include "fff_probe_launch.h"

#define BFFN_EXPORT extern "C" __attribute__((visibility("default")))

namespace bffn {

hipError_t resident_blocks(const void* kernel, int block, int64_t* blocks) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int64_t> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kernel});
    if (it != cache.end()) {
      *blocks = it->second;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
  std::lock_guard<std::mutex> lock(mu);
  cache[{dev, kernel}] = n;
  *blocks = n;
  return hipSuccess;
}

}  // namespace bffn

namespace {

thread_local char g_err[512];
thread_local bffn::StageEvents g_stage_events;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest number of units one call accepts: keeps every grid below 2^31 blocks.
constexpr int64_t kMaxUnits = int64_t(1) << 20;

int check_chunking(int64_t n_tokens, int32_t chunk_len) {
  if (chunk_len < 1 || chunk_len > 32) return fail(BLOCKFFN_ERR_CHUNK, "chunk_len %d outside [1, 32]", chunk_len);
  if (n_tokens < 0) return fail(BLOCKFFN_ERR_CHUNK, "n_tokens %lld is negative", (long long)n_tokens);
  if (n_tokens % chunk_len != 0)
    return fail(BLOCKFFN_ERR_CHUNK, "n_tokens %lld is not a multiple of chunk_len %d", (long long)n_tokens,
                chunk_len);
  if (n_tokens / chunk_len > kMaxUnits)
    return fail(BLOCKFFN_ERR_CHUNK, "%lld chunks exceed the per-call limit of %lld; split the call",
                (long long)(n_tokens / chunk_len), (long long)kMaxUnits);
  return BLOCKFFN_OK;
}

int check_experts(int32_t E) {
  if (E < 1 || E > 128) return fail(BLOCKFFN_ERR_SHAPE, "n_experts %d outside [1, 128]", E);
  return BLOCKFFN_OK;
}

int check_layer(const blockffn_layer* ly) {
  if (!ly) return fail(BLOCKFFN_ERR_NULL, "layer descriptor is NULL");
  if (ly->dtype != BLOCKFFN_F32 && ly->dtype != BLOCKFFN_BF16)
    return fail(BLOCKFFN_ERR_DTYPE, "unknown dtype %d", ly->dtype);
  if (int r = check_experts(ly->n_experts)) return r;
  if (ly->d < 64 || ly->d % 64 != 0 || ly->d > (1 << 16))
    return fail(BLOCKFFN_ERR_SHAPE, "d %d must be a positive multiple of 64 (at most 65536)", ly->d);
  if (ly->d_expert < 16 || ly->d_expert % 16 != 0 || ly->d_expert > 1024)
    return fail(BLOCKFFN_ERR_SHAPE, "d_expert %d must be a multiple of 16 in [16, 1024]", ly->d_expert);
  if (!std::isfinite(ly->rms_eps) || ly->rms_eps < 0.f)
    return fail(BLOCKFFN_ERR_SHAPE, "rms_eps must be finite and >= 0");
  if (ly->reserved != 0) return fail(BLOCKFFN_ERR_SHAPE, "reserved field must be 0");
  if (!ly->w_router || !ly->w_in || !ly->w_out)
    return fail(BLOCKFFN_ERR_NULL, "w_router, w_in and w_out must all be non-NULL");
  if (!aligned(ly->w_router, 16) || !aligned(ly->w_in, 16) || !aligned(ly->w_out, 16))
    return fail(BLOCKFFN_ERR_ALIGN, "weight pointers must be 16-byte aligned");
  if (!aligned(ly->b_router, 4) || !aligned(ly->rms_scale, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "b_router and rms_scale must be 4-byte aligned");
  return BLOCKFFN_OK;
}

// The pointers of descriptor l, in bffn::LayerTensor order.
void layer_ptrs(const blockffn_layer& ly, const void* p[bffn::kLayerTensors]) {
  p[bffn::kTWRouter] = ly.w_router;
  p[bffn::kTBRouter] = ly.b_router;
  p[bffn::kTScale] = ly.rms_scale;
  p[bffn::kTWIn] = ly.w_in;
  p[bffn::kTWOut] = ly.w_out;
}

// Reduces an array of per-unit layers to what the kernels index: the
// shortest period p (layers[l] == layers[l % p] for every l, p dividing n),
// then either an even spacing of that many layers (every pointer of layer
// l + 1 the same number of bytes past layer l's, NULL pointers NULL in
// every layer) or a table of at most kMaxListedLayers.  Host only.
template <int K, typename Desc, typename Ptrs>
int reduce_layers(const Desc* layers, int32_t n, Ptrs get_ptrs, int32_t* n_eff, int64_t* stride, bool* listed,
                  const void* tab[K][bffn::kMaxListedLayers]) {
  auto ptrs = [&](int l, const void* p[K]) { get_ptrs(layers[l], p); };
  auto same = [&](int a, int b) {
    const void *pa[K], *pb[K];
    ptrs(a, pa);
    ptrs(b, pb);
    for (int k = 0; k < K; ++k)
      if (pa[k] != pb[k]) return false;
    return true;
  };
  int32_t p = n;
  for (int32_t q = 1; q < n; ++q) {
    if (n % q != 0) continue;
    bool periodic = true;
    for (int32_t l = q; l < n && periodic; ++l) periodic = same(l, l % q);
    if (periodic) {
      p = q;
      break;
    }
  }
  *n_eff = p;
  *stride = 0;
  *listed = false;
  if (p == 1) return BLOCKFFN_OK;
  const void *p0[K], *p1[K];
  ptrs(0, p0);
  ptrs(1, p1);
  const int64_t s = (int64_t)(reinterpret_cast<uintptr_t>(p1[0]) - reinterpret_cast<uintptr_t>(p0[0]));
  bool even = true;
  for (int32_t l = 1; l < p && even; ++l) {
    const void* pl[K];
    ptrs(l, pl);
    for (int k = 0; k < K && even; ++k) {
      if ((p0[k] == nullptr) != (pl[k] == nullptr)) even = false;
      else if (p0[k] && (int64_t)(reinterpret_cast<uintptr_t>(pl[k]) - reinterpret_cast<uintptr_t>(p0[k])) != s * l)
        even = false;
    }
  }
  if (even) {
    *stride = s;
    return BLOCKFFN_OK;
  }
  if (p > bffn::kMaxListedLayers)
    return fail(BLOCKFFN_ERR_LAYERS,
                "%d distinct layers that are not evenly spaced in memory exceed the %d one call can list; "
                "split the call or place the layers at a fixed spacing", p, bffn::kMaxListedLayers);
  *listed = true;
  for (int32_t l = 0; l < p; ++l) {
    const void* pl[K];
    ptrs(l, pl);
    for (int k = 0; k < K; ++k) tab[k][l] = pl[k];
  }
  return BLOCKFFN_OK;
}

// Validates an array of n_layers descriptors (each one, and that they share
// one shape) and builds the kernels' view of it.  Host only: nothing is
// enqueued, so a failure leaves the stream untouched.
int layer_args(const blockffn_layer* layers, int32_t n_layers, bffn::LayerArgs* la) {
  if (!layers) return fail(BLOCKFFN_ERR_NULL, "layer descriptor array is NULL");
  if (n_layers < 1) return fail(BLOCKFFN_ERR_LAYERS, "n_layers %d < 1", n_layers);
  for (int32_t l = 0; l < n_layers; ++l) {
    const blockffn_layer& a = layers[0];
    const blockffn_layer& b = layers[l];
    if (int r = check_layer(&b)) return r;
    if (b.d != a.d || b.n_experts != a.n_experts || b.d_expert != a.d_expert || b.dtype != a.dtype ||
        b.rms_eps != a.rms_eps)
      return fail(BLOCKFFN_ERR_LAYERS, "layer %d differs from layer 0 in d, n_experts, d_expert, dtype or rms_eps", l);
  }
  const blockffn_layer* ly = &layers[0];
  *la = bffn::LayerArgs{};
  la->w_router = ly->w_router;
  la->b_router = ly->b_router;
  la->rms_scale = ly->rms_scale;
  la->w_in = ly->w_in;
  la->w_out = ly->w_out;
  la->d = ly->d;
  la->E = ly->n_experts;
  la->de = ly->d_expert;
  la->eps = ly->rms_eps;
  bool listed = false;
  int32_t n_eff = 1;
  if (int r = reduce_layers<bffn::kLayerTensors>(layers, n_layers, layer_ptrs, &n_eff, &la->stride, &listed,
                                                 la->tab))
    return r;
  la->n_layers = n_eff;
  la->listed = listed ? 1 : 0;
  return BLOCKFFN_OK;
}

enum class Path { kGemv, kMfma, kMfmaSplit, kFew, kGrouped };

// Resolves `mode` to a kernel family; returns a status code.
int resolve_mode(const blockffn_layer* ly, int64_t n_tokens, int32_t chunk_len, int32_t mode, Path* path,
                 bool* dense) {
  // The matrix-core path streams each chunk's union once for all its tokens;
  // at chunk_len 1 its idle token columns cost nothing (the kernels are bound
  // by weight bytes), so it is the default wherever the shapes allow it.  A
  // launch of a few units cuts each unit's work finer to fill the GPU: into
  // blocks of 16 rows whose waves split the contraction and add their parts
  // in LDS (kFew; without a step between blocks, so two kernels), or, for
  // shapes those kernels do not take, into k- and slot-ranges added by two
  // more kernels (kMfmaSplit).
  const bool mfma_ok = bffn::forward_mfma_supported(ly->d, ly->d_expert, ly->dtype);
  const bool auto_mfma = mfma_ok;
  int ks = 0, sp = 0;
  const bool few = bffn::chunk_split_factors(ly->d, ly->d_expert, n_tokens / chunk_len, false, &ks, &sp);
  *dense = false;
  switch (mode) {
    case BLOCKFFN_MODE_AUTO:
      if (!auto_mfma)
        *path = Path::kGemv;
      else if (!few)
        *path = Path::kMfma;
      else
        *path = bffn::forward_few_supported(ly->d, ly->d_expert, ly->dtype, n_tokens / chunk_len, chunk_len)
                    ? Path::kFew
                    : Path::kMfmaSplit;
      return BLOCKFFN_OK;
    case BLOCKFFN_MODE_CHUNK_SPLIT:
      if (!mfma_ok)
        return fail(BLOCKFFN_ERR_MODE, "CHUNK_SPLIT needs bf16 with d and d_expert multiples of 128");
      *path = Path::kMfmaSplit;
      return BLOCKFFN_OK;
    case BLOCKFFN_MODE_GEMV:
      *path = Path::kGemv;
      return BLOCKFFN_OK;
    case BLOCKFFN_MODE_CHUNK_MFMA:
      if (!mfma_ok)
        return fail(BLOCKFFN_ERR_MODE, "CHUNK_MFMA needs bf16 with d and d_expert multiples of 128");
      *path = Path::kMfma;
      return BLOCKFFN_OK;
    case BLOCKFFN_MODE_DENSE:
      *path = auto_mfma ? Path::kMfma : Path::kGemv;
      *dense = true;
      return BLOCKFFN_OK;
    case BLOCKFFN_MODE_GROUPED:
      if (!bffn::grouped_supported(ly->d, ly->d_expert, ly->dtype))
        return fail(BLOCKFFN_ERR_MODE, "GROUPED needs bf16, d a multiple of 128 and d_expert 128 or 256");
      *path = Path::kGrouped;
      return BLOCKFFN_OK;
    default:
      return fail(BLOCKFFN_ERR_MODE, "unknown mode %d", mode);
  }
}

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

size_t hbuf_bytes(const blockffn_layer* ly, int64_t n_tokens, Path path) {
  const size_t elem = path == Path::kMfma || path == Path::kMfmaSplit ? 2 : 4;
  return round256((size_t)n_tokens * (size_t)ly->n_experts * (size_t)ly->d_expert * elem);
}

// Work plan after the hidden buffer: one int64 per chunk plus a total, and
// two work counters.
size_t plan_bytes(int64_t n_tokens, int32_t chunk_len) {
  return round256(bffn::forward_mfma_plan_bytes(n_tokens / chunk_len));
}

// The split chunk path's partial tiles, after the plan.
size_t split_bytes(const blockffn_layer* ly, int64_t n_tokens, int32_t chunk_len, bffn::ChunkSplit* sp) {
  int ks = 0, s = 0;
  bffn::chunk_split_factors(ly->d, ly->d_expert, n_tokens / chunk_len, true, &ks, &s);
  if (sp) {
    sp->ks = ks;
    sp->sp = s;
  }
  return bffn::chunk_split_part_bytes(ly->d, ly->d_expert, ly->n_experts, n_tokens / chunk_len, chunk_len, ks, s,
                                      nullptr);
}

size_t workspace_bytes_for(const blockffn_layer* ly, int64_t n_tokens, int32_t chunk_len, Path path) {
  if (path == Path::kGrouped) return bffn::grouped_workspace_bytes(n_tokens, ly->n_experts, ly->d, ly->d_expert);
  if (path == Path::kFew) return round256(bffn::layer_step_hs_bytes(ly->n_experts, ly->d_expert, n_tokens));
  const size_t base = hbuf_bytes(ly, n_tokens, path) + plan_bytes(n_tokens, chunk_len);
  return path == Path::kMfmaSplit ? base + split_bytes(ly, n_tokens, chunk_len, nullptr) : base;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BLOCKFFN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return BLOCKFFN_OK;
}

}  // namespace

BFFN_EXPORT int blockffn_route(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                               int32_t chunk_len, float* gates, uint64_t* token_masks, float* preact,
                               hipStream_t stream) {
  bffn::LayerArgs la;
  if (int r = layer_args(layers, n_layers, &la)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  if (n_tokens == 0) return BLOCKFFN_OK;  // nothing is read or written; buffers may be NULL
  if (!x || !gates || !token_masks) return fail(BLOCKFFN_ERR_NULL, "x, gates and token_masks must be non-NULL");
  if (!aligned(x, 16) || !aligned(gates, 4) || !aligned(token_masks, 8) || !aligned(preact, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "x must be 16-byte, gates/preact 4-byte and token_masks 8-byte aligned");
  return hip_status(bffn::launch_route(la, x, n_tokens, chunk_len, layers->dtype, BLOCKFFN_ROUTER_BLOCKFFN, 0, gates,
                                       token_masks, preact, stream),
                    "router launch");
}

BFFN_EXPORT int blockffn_route_with(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                                    int32_t chunk_len, int32_t router, int32_t top_k, float* gates,
                                    uint64_t* token_masks, float* preact, hipStream_t stream) {
  bffn::LayerArgs la;
  if (int r = layer_args(layers, n_layers, &la)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  if (router != BLOCKFFN_ROUTER_BLOCKFFN && router != BLOCKFFN_ROUTER_TOPK_SOFTMAX && router != BLOCKFFN_ROUTER_RELU_SUM)
    return fail(BLOCKFFN_ERR_MODE, "unknown router %d", router);
  if (router == BLOCKFFN_ROUTER_TOPK_SOFTMAX && (top_k < 1 || top_k > layers->n_experts))
    return fail(BLOCKFFN_ERR_SHAPE, "top_k %d outside [1, n_experts %d]", top_k, layers->n_experts);
  if (n_tokens == 0) return BLOCKFFN_OK;
  if (!x || !gates || !token_masks) return fail(BLOCKFFN_ERR_NULL, "x, gates and token_masks must be non-NULL");
  if (!aligned(x, 16) || !aligned(gates, 4) || !aligned(token_masks, 8) || !aligned(preact, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "x must be 16-byte, gates/preact 4-byte and token_masks 8-byte aligned");
  return hip_status(bffn::launch_route(la, x, n_tokens, chunk_len, layers->dtype, router, top_k, gates, token_masks,
                                       preact, stream),
                    "router launch");
}

BFFN_EXPORT int blockffn_chunk_union(int32_t n_experts, const uint64_t* token_masks, int64_t n_tokens,
                                     int32_t chunk_len, uint64_t* chunk_masks, int32_t* active_count,
                                     int32_t* active_list, hipStream_t stream) {
  if (int r = check_experts(n_experts)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  if (n_tokens == 0) return BLOCKFFN_OK;
  if (!token_masks || !chunk_masks || !active_count || !active_list)
    return fail(BLOCKFFN_ERR_NULL, "token_masks, chunk_masks, active_count and active_list must be non-NULL");
  if (!aligned(token_masks, 8) || !aligned(chunk_masks, 8) || !aligned(active_count, 4) || !aligned(active_list, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "mask arrays must be 8-byte and count/list 4-byte aligned");
  return hip_status(bffn::launch_chunk_union(n_experts, token_masks, n_tokens, chunk_len, chunk_masks, active_count,
                                             active_list, stream),
                    "chunk-union launch");
}

BFFN_EXPORT size_t blockffn_workspace_size(const blockffn_layer* layer, int64_t n_tokens, int32_t chunk_len,
                                           int32_t mode) {
  if (check_layer(layer) != BLOCKFFN_OK || check_chunking(n_tokens, chunk_len) != BLOCKFFN_OK) return 0;
  Path path;
  bool dense;
  if (resolve_mode(layer, n_tokens, chunk_len, mode, &path, &dense) != BLOCKFFN_OK) return 0;
  return workspace_bytes_for(layer, n_tokens, chunk_len, path);
}

namespace {
hipError_t launch_forward_path(const bffn::LayerArgs& la, const blockffn_layer* layer, Path path, bool dense,
                               const void* x, int64_t n_tokens, int32_t chunk_len, const float* gates,
                               const int32_t* active_count, const int32_t* active_list, void* workspace, float* y,
                               hipStream_t stream);
}  // namespace

BFFN_EXPORT int blockffn_forward(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                                 int32_t chunk_len, const float* gates, const int32_t* active_count,
                                 const int32_t* active_list, int32_t mode, void* workspace, size_t workspace_bytes,
                                 float* y, hipStream_t stream) {
  bffn::LayerArgs la;
  if (int r = layer_args(layers, n_layers, &la)) return r;
  const blockffn_layer* layer = layers;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  Path path;
  bool dense;
  if (int r = resolve_mode(layer, n_tokens, chunk_len, mode, &path, &dense)) return r;
  if (path == Path::kGrouped && la.n_layers != 1)
    return fail(BLOCKFFN_ERR_LAYERS, "GROUPED runs one batch through one layer (%d distinct layers given)",
                la.n_layers);
  if (path == Path::kGrouped && n_tokens * layer->n_experts > INT32_MAX)
    return fail(BLOCKFFN_ERR_SHAPE, "GROUPED indexes pairs with 32 bits: n_tokens x n_experts must stay below 2^31");
  if (n_tokens == 0) return BLOCKFFN_OK;
  if (!x || !gates || !y) return fail(BLOCKFFN_ERR_NULL, "x, gates and y must be non-NULL");
  if (!dense && path != Path::kGrouped && (!active_count || !active_list))
    return fail(BLOCKFFN_ERR_NULL, "active_count and active_list must be non-NULL outside DENSE and GROUPED modes");
  if (!aligned(x, 16) || !aligned(gates, 4) || !aligned(y, 16) || !aligned(active_count, 4) ||
      !aligned(active_list, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "x and y must be 16-byte aligned, gates/count/list 4-byte aligned");
  const size_t need = workspace_bytes_for(layer, n_tokens, chunk_len, path);
  if (need > 0 && !workspace) return fail(BLOCKFFN_ERR_NULL, "workspace is NULL (need %zu bytes)", need);
  if (!aligned(workspace, 256)) return fail(BLOCKFFN_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(BLOCKFFN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return hip_status(launch_forward_path(la, layer, path, dense, x, n_tokens, chunk_len, gates, active_count,
                                        active_list, workspace, y, stream),
                    "forward launch");
}

namespace {

// Enqueues the forward on an already validated path and workspace.
hipError_t launch_forward_path(const bffn::LayerArgs& la, const blockffn_layer* layer, Path path, bool dense,
                               const void* x, int64_t n_tokens, int32_t chunk_len, const float* gates,
                               const int32_t* active_count, const int32_t* active_list, void* workspace, float* y,
                               hipStream_t stream) {
  hipError_t e;
  if (path == Path::kGrouped)
    e = bffn::launch_forward_grouped(la, static_cast<const uint16_t*>(x), n_tokens, gates, workspace, y,
                                     g_stage_events, stream);
  else if (path == Path::kFew)
    e = bffn::launch_forward_few(la, static_cast<const uint16_t*>(x), n_tokens, chunk_len, gates, active_count,
                                 active_list, static_cast<uint16_t*>(workspace), y, g_stage_events, stream);
  else if (path == Path::kMfma || path == Path::kMfmaSplit) {
    char* ws = static_cast<char*>(workspace);
    const size_t hb = hbuf_bytes(layer, n_tokens, path), pb = plan_bytes(n_tokens, chunk_len);
    bffn::ChunkSplit sp;
    if (path == Path::kMfmaSplit) {
      split_bytes(layer, n_tokens, chunk_len, &sp);
      size_t down_off = 0;
      bffn::chunk_split_part_bytes(layer->d, layer->d_expert, layer->n_experts, n_tokens / chunk_len, chunk_len,
                                   sp.ks, sp.sp, &down_off);
      sp.up_part = reinterpret_cast<float*>(ws + hb + pb);
      sp.down_part = reinterpret_cast<float*>(ws + hb + pb + down_off);
    }
    e = bffn::launch_forward_mfma(la, static_cast<const uint16_t*>(x), n_tokens, chunk_len, gates, active_count,
                                  active_list, dense, static_cast<uint16_t*>(workspace),
                                  reinterpret_cast<int64_t*>(ws + hb), sp, y, g_stage_events, stream);
  }
  else
    e = bffn::launch_forward_gemv(la, x, n_tokens, chunk_len, layer->dtype, gates, active_count, active_list, dense,
                                  static_cast<float*>(workspace), y, g_stage_events, stream);
  return e;
}

}  // namespace

// ---- blockffn_forward_noalloc: the forward with a static scratch array ----

namespace {

// Scratch of blockffn_forward_noalloc: one array per GPU, in the library's
// code object, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: kernels and copies get the
// device address from hipGetSymbolAddress (static_scratch_ptr), never the
// name.
constexpr size_t kStaticScratchBytes = size_t(BLOCKFFN_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  Returns a status code.
int static_scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (int r = hip_status(hipGetDevice(&dev), "hipGetDevice")) return r;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BLOCKFFN_ERR_HIP, "device %d is beyond the %d devices the static scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (int r = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return r;
    if (p == nullptr || !aligned(p, 256)) return fail(BLOCKFFN_ERR_HIP, "static scratch has no usable address");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return BLOCKFFN_OK;
}

}  // namespace

BFFN_EXPORT int blockffn_forward_noalloc(const blockffn_layer* layers, int32_t n_layers, const void* x,
                                         int64_t n_tokens, int32_t chunk_len, const float* gates,
                                         const int32_t* active_count, const int32_t* active_list, int32_t mode,
                                         float* y, hipStream_t stream) {
  // everything blockffn_forward checks that does not depend on the workspace, and the size it needs
  bffn::LayerArgs la;
  if (int r = layer_args(layers, n_layers, &la)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  Path path;
  bool dense;
  if (int r = resolve_mode(layers, n_tokens, chunk_len, mode, &path, &dense)) return r;
  const size_t need = workspace_bytes_for(layers, n_tokens, chunk_len, path);
  if (need > kStaticScratchBytes)
    return fail(BLOCKFFN_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch, beyond the %zu of the static array; split the call or use "
                "blockffn_forward with a workspace", need, kStaticScratchBytes);
  if (n_tokens == 0)  // validated as blockffn_forward would, and nothing to enqueue
    return blockffn_forward(layers, n_layers, x, n_tokens, chunk_len, gates, active_count, active_list, mode,
                            nullptr, 0, y, stream);
  void* ws = nullptr;
  if (int r = static_scratch_ptr(&ws)) return r;
  return blockffn_forward(layers, n_layers, x, n_tokens, chunk_len, gates, active_count, active_list, mode, ws,
                          kStaticScratchBytes, y, stream);
}

BFFN_EXPORT int blockffn_sparsity_stats(int32_t n_experts, const uint64_t* token_masks, int64_t n_tokens,
                                        int32_t chunk_len, blockffn_stats* stats_dev, hipStream_t stream) {
  if (int r = check_experts(n_experts)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  if (!token_masks || !stats_dev) return fail(BLOCKFFN_ERR_NULL, "token_masks and stats_dev must be non-NULL");
  if (!aligned(token_masks, 8) || !aligned(stats_dev, 8))
    return fail(BLOCKFFN_ERR_ALIGN, "token_masks and stats_dev must be 8-byte aligned");
  return hip_status(bffn::launch_stats(n_experts, token_masks, n_tokens, chunk_len, stats_dev, stream),
                    "stats launch");
}

// ---- blockffn_layer_forward: router, union, forward and statistics in one call ----

namespace {

// Workspace of the three-kernel step: the router's partial pre-activations [token][E][d/128] fp32, then
// Swish(W_in x) [chunk][expert][token][d_e] bf16.
size_t step_zpart_bytes(const blockffn_layer* ly, int64_t n_tokens) {
  return round256(bffn::layer_step_zpart_bytes(ly->d, ly->n_experts, n_tokens));
}

size_t step_workspace(const blockffn_layer* ly, int64_t n_tokens) {
  return step_zpart_bytes(ly, n_tokens) + round256(bffn::layer_step_hs_bytes(ly->n_experts, ly->d_expert, n_tokens));
}

bool step_fused(const blockffn_layer* ly, int64_t n_tokens, int32_t chunk_len) {
  return bffn::layer_step_fused(ly->d, ly->n_experts, ly->d_expert, ly->dtype, n_tokens, chunk_len);
}

}  // namespace

BFFN_EXPORT size_t blockffn_layer_forward_workspace_size(const blockffn_layer* layer, int64_t n_tokens,
                                                         int32_t chunk_len) {
  if (check_layer(layer) != BLOCKFFN_OK || check_chunking(n_tokens, chunk_len) != BLOCKFFN_OK) return 0;
  if (step_fused(layer, n_tokens, chunk_len)) return step_workspace(layer, n_tokens);
  Path path;
  bool dense;
  if (resolve_mode(layer, n_tokens, chunk_len, BLOCKFFN_MODE_AUTO, &path, &dense) != BLOCKFFN_OK) return 0;
  return workspace_bytes_for(layer, n_tokens, chunk_len, path);
}

BFFN_EXPORT int blockffn_layer_forward(const blockffn_layer* layers, int32_t n_layers, const void* x,
                                       int64_t n_tokens, int32_t chunk_len, float* gates, uint64_t* token_masks,
                                       float* preact, uint64_t* chunk_masks, int32_t* active_count,
                                       int32_t* active_list, blockffn_stats* stats_dev, void* workspace,
                                       size_t workspace_bytes, float* y, hipStream_t stream) {
  bffn::LayerArgs la;
  if (int r = layer_args(layers, n_layers, &la)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  if (n_tokens == 0) return BLOCKFFN_OK;  // nothing is read or written; buffers may be NULL
  if (!x || !gates || !token_masks || !chunk_masks || !active_count || !active_list || !y)
    return fail(BLOCKFFN_ERR_NULL, "x, gates, token_masks, chunk_masks, active_count, active_list and y must be "
                                   "non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(gates, 4) || !aligned(preact, 4) || !aligned(token_masks, 8) ||
      !aligned(chunk_masks, 8) || !aligned(active_count, 4) || !aligned(active_list, 4) || !aligned(stats_dev, 8))
    return fail(BLOCKFFN_ERR_ALIGN, "x and y must be 16-byte, masks and stats 8-byte, the rest 4-byte aligned");
  const blockffn_layer* layer = layers;
  const bool fused = step_fused(layer, n_tokens, chunk_len);
  Path path = Path::kMfmaSplit;
  bool dense = false;
  if (!fused)
    if (int r = resolve_mode(layer, n_tokens, chunk_len, BLOCKFFN_MODE_AUTO, &path, &dense)) return r;
  const size_t need = fused ? step_workspace(layer, n_tokens) : workspace_bytes_for(layer, n_tokens, chunk_len, path);
  if (need > 0 && !workspace) return fail(BLOCKFFN_ERR_NULL, "workspace is NULL (need %zu bytes)", need);
  if (!aligned(workspace, 256)) return fail(BLOCKFFN_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(BLOCKFFN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipError_t e;
  if (fused) {
    char* ws = static_cast<char*>(workspace);
    e = bffn::launch_layer_step(la, static_cast<const uint16_t*>(x), n_tokens, chunk_len, gates, token_masks, preact,
                                chunk_masks, active_count, active_list, stats_dev, reinterpret_cast<float*>(ws),
                                reinterpret_cast<uint16_t*>(ws + step_zpart_bytes(layer, n_tokens)), y, stream);
  } else {
    e = bffn::launch_route(la, x, n_tokens, chunk_len, layer->dtype, BLOCKFFN_ROUTER_BLOCKFFN, 0, gates, token_masks,
                           preact, stream);
    if (e == hipSuccess)
      e = bffn::launch_chunk_union(la.E, token_masks, n_tokens, chunk_len, chunk_masks, active_count, active_list,
                                   stream);
    if (e == hipSuccess)
      e = launch_forward_path(la, layer, path, dense, x, n_tokens, chunk_len, gates, active_count, active_list,
                              workspace, y, stream);
    if (e == hipSuccess && stats_dev)
      e = bffn::launch_stats(la.E, token_masks, n_tokens, chunk_len, stats_dev, stream);
  }
  return hip_status(e, "layer forward launch");
}

namespace {

int check_backward(const blockffn_layer* layer, int64_t n_tokens) {
  if (int r = check_layer(layer)) return r;
  if (n_tokens < 0) return fail(BLOCKFFN_ERR_SHAPE, "n_tokens %lld is negative", (long long)n_tokens);
  if (!bffn::grouped_supported(layer->d, layer->d_expert, layer->dtype))
    return fail(BLOCKFFN_ERR_MODE, "the backward needs bf16, d a multiple of 128 and d_expert 128 or 256");
  if (n_tokens * layer->n_experts > INT32_MAX)
    return fail(BLOCKFFN_ERR_SHAPE, "the backward indexes pairs with 32 bits: n_tokens x n_experts must stay below 2^31");
  return BLOCKFFN_OK;
}

}  // namespace

BFFN_EXPORT size_t blockffn_backward_workspace_size(const blockffn_layer* layer, int64_t n_tokens) {
  if (check_backward(layer, n_tokens) != BLOCKFFN_OK) return 0;
  return bffn::backward_workspace_bytes(n_tokens, layer->n_experts, layer->d, layer->d_expert);
}

BFFN_EXPORT int blockffn_backward(const blockffn_layer* layer, const void* x, int64_t n_tokens, const float* preact,
                                  const float* dy, const float* dz_extra, void* workspace, size_t workspace_bytes,
                                  float* dx, const blockffn_grads* grads, hipStream_t stream) {
  if (int r = check_backward(layer, n_tokens)) return r;
  if (n_tokens == 0) return BLOCKFFN_OK;
  if (!x || !preact || !dy || !dx || !grads) return fail(BLOCKFFN_ERR_NULL, "x, preact, dy, dx and grads must be non-NULL");
  if (!grads->d_w_router || !grads->d_b_router || !grads->d_rms_scale || !grads->d_w_in || !grads->d_w_out)
    return fail(BLOCKFFN_ERR_NULL, "every gradient pointer must be non-NULL");
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(preact, 4) || !aligned(dz_extra, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "x, dy and dx must be 16-byte aligned, preact and dz_extra 4-byte aligned");
  if (!aligned(grads->d_w_router, 16) || !aligned(grads->d_w_in, 16) || !aligned(grads->d_w_out, 16) ||
      !aligned(grads->d_b_router, 4) || !aligned(grads->d_rms_scale, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "weight gradients must be 16-byte aligned, d_b_router / d_rms_scale 4-byte");
  const size_t need = bffn::backward_workspace_bytes(n_tokens, layer->n_experts, layer->d, layer->d_expert);
  if (!workspace) return fail(BLOCKFFN_ERR_NULL, "workspace is NULL (need %zu bytes)", need);
  if (!aligned(workspace, 256)) return fail(BLOCKFFN_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(BLOCKFFN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  bffn::LayerArgs la;
  if (int r = layer_args(layer, 1, &la)) return r;
  return hip_status(bffn::launch_backward(la, static_cast<const uint16_t*>(x), n_tokens, preact, dy, dz_extra,
                                          workspace, dx,
                                          grads->d_w_router, grads->d_b_router, grads->d_rms_scale, grads->d_w_in,
                                          grads->d_w_out, g_stage_events, stream),
                    "backward launch");
}

BFFN_EXPORT size_t blockffn_cls_losses_workspace_size(int64_t n_tokens, int32_t chunk_len) {
  if (check_chunking(n_tokens, chunk_len) != BLOCKFFN_OK) return 0;
  return bffn::cls_losses_workspace_bytes(n_tokens, chunk_len);
}

BFFN_EXPORT int blockffn_cls_losses(int32_t n_experts, const float* preact, int64_t n_tokens, int32_t chunk_len,
                                    float alpha, float w_locality, float w_chunk, void* workspace,
                                    size_t workspace_bytes, float* losses, float* dz, hipStream_t stream) {
  if (int r = check_experts(n_experts)) return r;
  if (int r = check_chunking(n_tokens, chunk_len)) return r;
  if (!std::isfinite(alpha) || alpha <= 0.f) return fail(BLOCKFFN_ERR_SHAPE, "alpha must be finite and positive");
  if (!std::isfinite(w_locality) || !std::isfinite(w_chunk))
    return fail(BLOCKFFN_ERR_SHAPE, "loss weights must be finite");
  if (!losses || !workspace || (n_tokens > 0 && !preact))
    return fail(BLOCKFFN_ERR_NULL, "preact, workspace and losses must be non-NULL");
  if (!aligned(preact, 4) || !aligned(losses, 4) || !aligned(dz, 4) || !aligned(workspace, 256))
    return fail(BLOCKFFN_ERR_ALIGN, "preact, losses and dz must be 4-byte aligned, workspace 256-byte aligned");
  const size_t need = bffn::cls_losses_workspace_bytes(n_tokens, chunk_len);
  if (workspace_bytes < need)
    return fail(BLOCKFFN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return hip_status(bffn::launch_cls_losses(n_experts, preact, n_tokens, chunk_len, alpha, w_locality, w_chunk,
                                            workspace, losses, dz, stream),
                    "cls-losses launch");
}

namespace {

int check_fff_layer(const blockffn_fff_layer* layer) {
  if (!layer) return fail(BLOCKFFN_ERR_NULL, "layer descriptor is NULL");
  const blockffn_fff_layer& ly = *layer;
  if (ly.dtype != BLOCKFFN_F32 && ly.dtype != BLOCKFFN_BF16) return fail(BLOCKFFN_ERR_DTYPE, "unknown dtype %d", ly.dtype);
  if (!bffn::fff_width_supported(ly.d, ly.dtype))
    return fail(BLOCKFFN_ERR_SHAPE, "d %d: bf16 needs a multiple of 512 up to 4096, f32 a multiple of 256 up to 2048",
                ly.d);
  if (ly.n_trees < 1 || ly.n_trees > (1 << 16)) return fail(BLOCKFFN_ERR_SHAPE, "n_trees %d outside [1, 65536]", ly.n_trees);
  if (ly.depth < 0 || ly.depth > 15) return fail(BLOCKFFN_ERR_SHAPE, "depth %d outside [0, 15]", ly.depth);
  if (ly.activation != BLOCKFFN_FFF_GELU_NODES && ly.activation != BLOCKFFN_FFF_GELU_OUTPUT)
    return fail(BLOCKFFN_ERR_SHAPE, "unknown activation placement %d", ly.activation);
  const int64_t row_bytes = (int64_t)ly.d * (ly.dtype == BLOCKFFN_BF16 ? 2 : 4);
  if (ly.node_stride != 0 && (ly.node_stride < row_bytes || ly.node_stride % 16 != 0))
    return fail(BLOCKFFN_ERR_SHAPE, "node_stride %d must be 0 or a multiple of 16 of at least %lld", ly.node_stride,
                (long long)row_bytes);
  if (!ly.w_node || !ly.w_out) return fail(BLOCKFFN_ERR_NULL, "w_node and w_out must be non-NULL");
  if (!aligned(ly.w_node, 16) || !aligned(ly.w_out, 16))
    return fail(BLOCKFFN_ERR_ALIGN, "w_node and w_out must be 16-byte aligned");
  if (!aligned(ly.b_node, 4)) return fail(BLOCKFFN_ERR_ALIGN, "b_node must be 4-byte aligned");
  return BLOCKFFN_OK;
}

void fff_ptrs(const blockffn_fff_layer& ly, const void* p[3]) {
  p[0] = ly.w_node;
  p[1] = ly.b_node;
  p[2] = ly.w_out;
}

// Validates an array of FFF layer descriptors of one shape and reduces it
// as layer_args does.  Host only.
int fff_layer_set(const blockffn_fff_layer* layers, int32_t n_layers, bffn::FffLayerSet* set) {
  if (!layers) return fail(BLOCKFFN_ERR_NULL, "layer descriptor array is NULL");
  if (n_layers < 1) return fail(BLOCKFFN_ERR_LAYERS, "n_layers %d < 1", n_layers);
  for (int32_t l = 0; l < n_layers; ++l) {
    const blockffn_fff_layer& a = layers[0];
    const blockffn_fff_layer& b = layers[l];
    if (int r = check_fff_layer(&b)) return r;
    if (b.d != a.d || b.n_trees != a.n_trees || b.depth != a.depth || b.dtype != a.dtype ||
        b.activation != a.activation || b.node_stride != a.node_stride)
      return fail(BLOCKFFN_ERR_LAYERS,
                  "layer %d differs from layer 0 in d, n_trees, depth, dtype, activation or node_stride", l);
  }
  *set = bffn::FffLayerSet{};
  bool listed = false;
  int32_t n_eff = 1;
  if (int r = reduce_layers<3>(layers, n_layers, fff_ptrs, &n_eff, &set->stride, &listed, set->tab)) return r;
  set->n_layers = n_eff;
  set->listed = listed ? 1 : 0;
  return BLOCKFFN_OK;
}

int check_fff_split(const blockffn_fff_layer& ly, int64_t n_tokens, int32_t split) {
  if (n_tokens < 0 || n_tokens > INT32_MAX)
    return fail(BLOCKFFN_ERR_SHAPE, "n_tokens %lld outside [0, 2^31)", (long long)n_tokens);
  const int gmax = bffn::fff_max_split(ly.n_trees);
  if (split < 0 || split > gmax)
    return fail(BLOCKFFN_ERR_SHAPE, "split %d outside [0, %d] (0 = automatic)", split, gmax);
  if (n_tokens * bffn::fff_split(ly.n_trees, n_tokens, split) > INT32_MAX)
    return fail(BLOCKFFN_ERR_SHAPE, "n_tokens x blocks per token must stay below 2^31");
  return BLOCKFFN_OK;
}

}  // namespace

BFFN_EXPORT size_t blockffn_fff_workspace_size(const blockffn_fff_layer* layer, int64_t n_tokens, int32_t split) {
  if (check_fff_layer(layer) != BLOCKFFN_OK || check_fff_split(*layer, n_tokens, split) != BLOCKFFN_OK) return 0;
  return bffn::fff_workspace_bytes(layer->d, layer->n_trees, n_tokens, split);
}

BFFN_EXPORT int blockffn_fff_forward(const blockffn_fff_layer* layers, int32_t n_layers, const void* x,
                                     int64_t n_tokens, int32_t mode, int32_t split, int32_t* paths,
                                     float* node_preact, void* workspace, size_t workspace_bytes, float* y,
                                     hipStream_t stream) {
  bffn::FffLayerSet set;
  if (int r = fff_layer_set(layers, n_layers, &set)) return r;
  const blockffn_fff_layer& ly = *layers;
  if (mode != BLOCKFFN_FFF_SPARSE && mode != BLOCKFFN_FFF_DENSE) return fail(BLOCKFFN_ERR_MODE, "unknown mode %d", mode);
  if (mode == BLOCKFFN_FFF_DENSE && (paths || node_preact))
    return fail(BLOCKFFN_ERR_MODE, "paths and node_preact must be NULL in dense mode");
  if (int r = check_fff_split(ly, n_tokens, split)) return r;
  if (n_tokens > 0 && (!x || !y)) return fail(BLOCKFFN_ERR_NULL, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 16))
    return fail(BLOCKFFN_ERR_ALIGN, "x, y and workspace must be 16-byte aligned");
  if (!aligned(paths, 4) || !aligned(node_preact, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "paths and node_preact must be 4-byte aligned");
  const size_t need = bffn::fff_workspace_bytes(ly.d, ly.n_trees, n_tokens, split);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BLOCKFFN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace ? workspace_bytes : 0, need);
  return hip_status(bffn::launch_fff_forward(ly, set, x, n_tokens, mode == BLOCKFFN_FFF_DENSE, split, paths,
                                             node_preact, workspace, y, stream),
                    "fff forward launch");
}

BFFN_EXPORT int blockffn_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink,
                                    hipStream_t stream) {
  if (!sink || (bytes > 0 && !buf)) return fail(BLOCKFFN_ERR_NULL, "buf and sink must be non-NULL");
  if (!aligned(buf, 16) || bytes % 16 != 0 || !aligned(sink, 4))
    return fail(BLOCKFFN_ERR_ALIGN, "buf must be 16-byte aligned, bytes a multiple of 16, sink 4-byte aligned");
  if (blocks < 0) return fail(BLOCKFFN_ERR_SHAPE, "blocks %d < 0", blocks);
  if (bytes == 0) return BLOCKFFN_OK;
  return hip_status(bffn::launch_read_probe(buf, bytes, blocks, sink, stream), "read probe launch");
}

BFFN_EXPORT int blockffn_set_stage_events(hipEvent_t* events, int32_t n_events) {
  if (events != nullptr && n_events < 1) return fail(BLOCKFFN_ERR_SHAPE, "n_events %d < 1", n_events);
  g_stage_events.ev = events;
  g_stage_events.n = events != nullptr ? n_events : 0;
  return BLOCKFFN_OK;
}

BFFN_EXPORT const char* blockffn_status_string(int status) {
  switch (status) {
    case BLOCKFFN_OK: return "ok";
    case BLOCKFFN_ERR_NULL: return "a required pointer is NULL";
    case BLOCKFFN_ERR_SHAPE: return "unsupported or inconsistent shape";
    case BLOCKFFN_ERR_DTYPE: return "unknown dtype";
    case BLOCKFFN_ERR_CHUNK: return "bad chunk_len or n_tokens";
    case BLOCKFFN_ERR_WORKSPACE: return "workspace too small";
    case BLOCKFFN_ERR_MODE: return "unknown or unsupported mode";
    case BLOCKFFN_ERR_ALIGN: return "misaligned pointer or stride";
    case BLOCKFFN_ERR_LAYERS: return "bad layer count or stride";
    case BLOCKFFN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

BFFN_EXPORT const char* blockffn_last_error(void) { return g_err; }

BFFN_EXPORT int blockffn_version(void) { return BLOCKFFN_VERSION; }

#ifndef BLOCKFFN_BUILD_DIGEST
#define BLOCKFFN_BUILD_DIGEST "unknown"
#endif
BFFN_EXPORT const char* blockffn_build_digest(void) { return BLOCKFFN_BUILD_DIGEST; }
