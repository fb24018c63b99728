// Grouped-by-expert batch forward: the launcher (kernels in grouped_kernels.h).
//
// When many chunks go through the same layer, streaming each chunk's union
// (the chunk path) would re-read the layer once per chunk.  Here every
// (token, expert) pair with a non-zero gate is grouped by expert and each
// expert's weights are read once for all of its tokens (the outer loop over
// active experts with a batched product inside, BlockFFN write-up §7, taken
// to the whole batch).
#include "grouped_kernels.h"

namespace bffn {

bool grouped_supported(int d, int de, int dtype) {
  return dtype == BLOCKFFN_BF16 && d % GBN == 0 && (de == 128 || de == 256);
}

// Workspace: per-block slots, offsets, pair arrays (capacity T*E pairs),
// pair_idx, hidden and partial rows.
size_t grouped_workspace_bytes(int64_t T, int E, int d, int de) {
  const size_t P = (size_t)T * E;
  const size_t rows = (size_t)plan_rows(T);
  const size_t nblk = ((size_t)T + rows - 1) / rows;
  return r256(4 * nblk * E) + 2 * r256(sizeof(int64_t) * (E + 1)) + r256(4 * P) + r256(4 * P) + r256(4 * P) +
         r256(2 * P * de) + r256(2 * P * d);
}

hipError_t launch_forward_grouped(const LayerArgs& la, const uint16_t* x, int64_t T, const float* gates,
                                  void* workspace, float* y, const StageEvents& se, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int E = la.E, d = la.d, de = la.de;
  const size_t P = (size_t)T * E;
  const int rows = plan_rows(T);
  const int nblk = (int)((T + rows - 1) / rows);
  char* ws = static_cast<char*>(workspace);
  auto take = [&](size_t bytes) {
    char* p = ws;
    ws += r256(bytes);
    return p;
  };
  int32_t* blk = reinterpret_cast<int32_t*>(take(4 * (size_t)nblk * E));
  int64_t* pair_off = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (E + 1)));
  int64_t* tile_up = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (E + 1)));
  int32_t* pair_tok = reinterpret_cast<int32_t*>(take(4 * P));
  float* pair_gate = reinterpret_cast<float*>(take(4 * P));
  int32_t* pair_idx = reinterpret_cast<int32_t*>(take(4 * P));
  uint16_t* hid = reinterpret_cast<uint16_t*>(take(2 * P * de));
  uint16_t* part = reinterpret_cast<uint16_t*>(take(2 * P * d));

  group_count_kernel<PairRule::kNonZero><<<dim3((unsigned)nblk), dim3(kPlanThreads), 0, s>>>(gates, T, E, rows, blk);
  group_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(blk, nblk, E, de / GBN, kUpRows, pair_off, tile_up);
  group_fill_kernel<PairRule::kNonZero><<<dim3((unsigned)nblk), dim3(kPlanThreads), 0, s>>>(
      gates, gates, T, E, rows, blk, pair_tok, pair_gate, pair_idx);
  // upper bounds of the work (every pair active) cap the grids; the kernels
  // read the exact totals on the device
  const int64_t max_up_tiles = (int64_t)E * ((T + kUpRows - 1) / kUpRows) * (de / GBN);
  int64_t grid_up = 0, grid_dn = 0;
  hipError_t e = persistent_grid(grouped_up_kernel, max_up_tiles, &grid_up);
  if (e == hipSuccess)
    e = de == 128 ? persistent_grid(grouped_down_kernel<128>, down_blocks(E, d, de), &grid_dn)
                  : persistent_grid(grouped_down_kernel<256>, down_blocks(E, d, de), &grid_dn);
  if (e != hipSuccess) return e;

  se.record(0, s);
  UpArgs up{x, pair_tok, pair_gate, static_cast<const uint16_t*>(la.w_in), pair_off, tile_up, hid, d, de, E};
  grouped_up_kernel<<<dim3((unsigned)grid_up), dim3(kBlock), 0, s>>>(up);
  se.record(1, s);
  DownArgs dn{hid, static_cast<const uint16_t*>(la.w_out), pair_off, part, d, E, nullptr, nullptr};
  if (de == 128)
    grouped_down_kernel<128><<<dim3((unsigned)grid_dn), dim3(kBlock), 0, s>>>(dn);
  else
    grouped_down_kernel<256><<<dim3((unsigned)grid_dn), dim3(kBlock), 0, s>>>(dn);
  se.record(2, s);
  int cthreads = (d / 8 + 63) / 64 * 64;
  cthreads = cthreads < 64 ? 64 : (cthreads > 1024 ? 1024 : cthreads);
  combine_kernel<<<dim3((unsigned)T), dim3((unsigned)cthreads), 0, s>>>(gates, pair_idx, part, E, d, y);
  se.record(3, s);
  return hipGetLastError();
}

}  // namespace bffn
