/*
 * fff_oracle.c -- plain, slow CPU oracle of the fast feedforward (FFF) tree layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It includes no HIP header and shares no code, table
 * or helper with the GPU library.
 *
 * What it computes (source: "Dynamic sparsity in tree-structured feed-forward
 * layers at scale", write-up on gist.science, §2 methodology: architecture
 * design and key mechanisms; §4 results: efficiency):
 *
 *   The layer is P parallel perfect binary trees of depth D.  Tree p has
 *   N = 2^(D+1) - 1 nodes in heap order: the root is node 0 and node n has
 *   the children 2n + 1 (left) and 2n + 2 (right).  Node n of tree p holds an
 *   input row w_node[p][n][0..d), a bias b[p][n] and an output row
 *   w_out[p][n][0..d).
 *
 *   Hard routing: for a token x, in every tree, start at the root; at each
 *   level l = 0..D the current node n computes its pre-activation
 *       c = sum_k w_node[p][n][k] x_k + b[p][n]
 *   and the walk continues to the right child when c > 0, else to the left
 *   child.  A token therefore visits D + 1 of the N nodes of each tree.
 *
 *   Output (the visited nodes' activations, concatenated over the trees,
 *   through the final projection whose columns are the nodes' output rows):
 *       FFF      y = sum_p sum_l GELU(c_{p,l}) w_out[p][n_{p,l}]
 *       FFFpost  y = GELU( sum_p sum_l c_{p,l} w_out[p][n_{p,l}] )
 *   with GELU(c) = c Phi(c) = c (1 + erf(c / sqrt 2)) / 2.
 *
 *   Dense evaluation: the same sums over every node of every tree, i.e. the
 *   dense feed-forward block of width P N that the tree layer replaces.
 *
 * Every sum is accumulated in double, in the plain index order written
 * below (trees ascending, then levels or nodes ascending, then k), with no
 * blocking or reordering.  Inputs are read in their stored precision (IEEE
 * binary32, or bfloat16 = the upper 16 bits of a binary32) and widened here.
 * Pinned by CPU tests against hand-worked trees, closed forms, a library
 * matmul for the dense and depth-0 cases, and brute force over every leaf of
 * small trees; not "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FFF_F32 0
#define FFF_BF16 1
#define FFF_MAX_DEPTH 20

static double fff_widen(const void *base, int64_t idx, int dtype) {
  if (dtype == FFF_F32) return (double)((const float *)base)[idx];
  union {
    uint32_t u;
    float f;
  } v;
  v.u = (uint32_t)((const uint16_t *)base)[idx] << 16;
  return (double)v.f;
}

static double fff_gelu(double c) { return 0.5 * c * (1.0 + erf(c / sqrt(2.0))); }

/* pre-activation of node n of tree p for token t */
static double fff_node_preact(int d, int dtype, const void *x, int64_t t, const void *w_node, const float *b_node,
                              int64_t row) {
  double c = 0.0;
  for (int k = 0; k < d; ++k) c += fff_widen(w_node, row * d + k, dtype) * fff_widen(x, t * d + k, dtype);
  if (b_node) c += (double)b_node[row];
  return c;
}

/*
 * x[T][d], w_node[P][N][d], b_node[P][N] or NULL, w_out[P][N][d] (f32 or bf16
 * bits per dtype).  Outputs: y[T][d] (double); when walking (dense == 0)
 * optionally paths[T][P][D+1] (int32 node ids) and preact[T][P][D+1]; when
 * dense, paths must be NULL and preact, if given, is [T][P][N].
 * Returns 0, or -1 for invalid arguments.
 */
int oracle_fff_forward(int32_t d, int32_t P, int32_t D, int32_t dtype, int32_t post, int32_t dense, const void *x,
                       int64_t T, const void *w_node, const float *b_node, const void *w_out, int32_t *paths,
                       double *preact, double *y) {
  if (d < 1 || P < 1 || D < 0 || D > FFF_MAX_DEPTH || T < 0 || (dtype != FFF_F32 && dtype != FFF_BF16)) return -1;
  if (T > 0 && (!x || !w_node || !w_out || !y)) return -1;
  if (dense && paths) return -1;
  const int64_t N = ((int64_t)1 << (D + 1)) - 1;
  const int64_t V = dense ? N : (int64_t)D + 1; /* nodes visited per tree */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    double *yt = y + t * d;
    for (int k = 0; k < d; ++k) yt[k] = 0.0;
    for (int p = 0; p < P; ++p) {
      int64_t n = 0;
      for (int64_t l = 0; l < V; ++l) {
        if (dense) n = l;
        const int64_t row = (int64_t)p * N + n;
        const double c = fff_node_preact(d, dtype, x, t, w_node, b_node, row);
        const int64_t rec = (t * P + p) * V + l;
        if (paths) paths[rec] = (int32_t)n;
        if (preact) preact[rec] = c;
        const double a = post ? c : fff_gelu(c);
        for (int k = 0; k < d; ++k) yt[k] += a * fff_widen(w_out, row * d + k, dtype);
        if (!dense && l < D) n = 2 * n + 1 + (c > 0.0 ? 1 : 0);
      }
    }
    if (post)
      for (int k = 0; k < d; ++k) yt[k] = fff_gelu(yt[k]);
  }
  return 0;
}
