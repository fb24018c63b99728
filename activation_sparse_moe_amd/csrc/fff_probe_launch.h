// Host-side declarations of the FFF tree layer's and the HBM read probe's
// launchers (arguments already validated by the C ABI).
#pragma once

#include "bffn_internal.h"

namespace bffn {

// FFF rows of d elements are 1..kFffMaxPieces pieces of 1 KiB per lane group.
constexpr int kFffMaxPieces = 8;
// Launches below this many blocks spread a token's trees over several blocks.
constexpr int64_t kFffTargetBlocks = 3072;
bool fff_width_supported(int d, int dtype);
int fff_max_split(int n_trees);
int fff_split(int n_trees, int64_t n_tokens, int requested);
size_t fff_workspace_bytes(int d, int n_trees, int64_t n_tokens, int requested);
// The FFF layers a call's tokens cycle through (token t uses layer
// t % n_layers), reduced by the C ABI as for BlockFFN layers: evenly spaced
// (layer l at ptr + l * stride) or, listed == 1, a table of each layer's
// pointers: tab[0] w_node, tab[1] b_node, tab[2] w_out.
struct FffLayerSet {
  int32_t n_layers = 1;
  int32_t listed = 0;
  int64_t stride = 0;
  const void* tab[3][kMaxListedLayers] = {};
};
hipError_t launch_fff_forward(const blockffn_fff_layer& ly, const FffLayerSet& set, const void* x, int64_t n_tokens,
                              bool dense, int split, int32_t* paths, float* preact, void* workspace, float* y,
                              hipStream_t s);

hipError_t launch_read_probe(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t s);

}  // namespace bffn
