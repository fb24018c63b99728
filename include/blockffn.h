/*
 * blockffn.h -- C ABI of the BlockFFN layer forward on MI355X (gfx950).
 *
 * The layer (BlockFFN write-up, lsdiaocha.cn, §2 core design; abstract of
 * "BlockFFN: Towards End-Side Acceleration-Friendly Mixture-of-Experts with
 * Chunk-Level Activation Sparsity", arXiv 2507.08771):
 *
 *   router   z = W_r x + b;  a = ReLU(z);  g = s * a / sqrt(mean_E(a^2) + eps)
 *            expert i is active for the token iff z_i > 0
 *   experts  E_i(x) = W_out[i] Swish(W_in[i] x), a non-gated MLP d -> d_e -> d
 *   output   y = sum over the active experts of g_i E_i(x)
 *
 * and the chunk-level evaluation of write-up §4: for a chunk of L consecutive
 * tokens, the union of their active experts is found and only those experts
 * run, over every token of the chunk, each pair weighted by the token's own
 * gate (zero for the experts the token did not activate).
 *
 * One export per stage of that pipeline: blockffn_route (router),
 * blockffn_chunk_union (union + compacted expert list),
 * blockffn_forward (expert streaming, gate scaling and sum) and
 * blockffn_sparsity_stats (token- and chunk-level sparsity).
 *
 * General rules for every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the layer descriptors themselves (and blockffn_grads), which are host
 *     structs read during the call.  Buffers must stay valid until the
 *     queued work has completed; the library keeps no reference after the
 *     call returns.
 *   - No entry point allocates memory.  Scratch space for blockffn_forward is
 *     a caller-provided workspace of at least blockffn_workspace_size() bytes.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no
 *     entry point synchronises.  Apart from the optional per-thread stage
 *     timing events (blockffn_set_stage_events), calls carry no hidden state
 *     and may be made from several threads at once on different buffers.
 *   - Every entry point returns BLOCKFFN_OK (0) or a negative BLOCKFFN_ERR_*
 *     code.  Arguments are validated on the host before anything is
 *     enqueued: a call that fails validation enqueues nothing.
 *     blockffn_last_error() gives a message for the calling thread's last
 *     failure.  Nothing aborts and no C++ exception crosses the ABI.
 *   - Layout: every matrix is row-major in the [out][in] convention, so each
 *     expert's rows are contiguous: w_router[E][d], w_in[E][d_e][d],
 *     w_out[E][d][d_e], x[T][d], gates[T][E], y[T][d].
 *   - Chunks are the aligned, non-overlapping runs of chunk_len consecutive
 *     tokens; n_tokens must be a multiple of chunk_len.  Chunk c covers
 *     tokens [c*chunk_len, (c+1)*chunk_len).
 *   - Token masks: token t's activation pattern is W = ceil(E/64) 64-bit
 *     words at token_masks[t*W]; expert i is bit (i % 64) of word i / 64.
 *   - A call with n_tokens == 0 validates its other arguments and enqueues
 *     nothing; its token-sized buffers may then be NULL.
 *
 * Supported shapes: 1 <= E <= 128, d a multiple of 64, d_e a multiple of 16
 * (at most 1024), 1 <= chunk_len <= 32.  The MFMA forward additionally needs
 * bf16, d a multiple of 128 and d_e a multiple of 128.
 */
#ifndef BLOCKFFN_H_
#define BLOCKFFN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLOCKFFN_VERSION 2

/* Element type of x and of every weight matrix. */
#define BLOCKFFN_F32 0  /* IEEE binary32 */
#define BLOCKFFN_BF16 1 /* bfloat16: the upper 16 bits of a binary32 */

/* blockffn_forward modes. */
/* AUTO: where the matrix-core shapes hold (bf16, d and d_expert % 128 == 0), CHUNK_MFMA, except for at most 16
   units, which run as blocks of 16 rows whose waves split the contraction and add their parts in a fixed order
   (d <= 4096; y scales each expert's product with Swish(W_in x), bf16, by the gate in fp32), or else
   CHUNK_SPLIT; otherwise GEMV */
#define BLOCKFFN_MODE_AUTO 0
#define BLOCKFFN_MODE_GEMV 1       /* vector-ALU streaming of the active experts (any dtype) */
#define BLOCKFFN_MODE_CHUNK_MFMA 2 /* matrix-core tiles over each chunk's union (bf16) */
#define BLOCKFFN_MODE_GROUPED 3    /* token-expert pairs grouped by expert (bf16, d % 128 == 0, d_expert 128 or 256, one layer) */
#define BLOCKFFN_MODE_DENSE 4      /* every expert on every token (the comparison path) */
#define BLOCKFFN_MODE_CHUNK_SPLIT 5 /* CHUNK_MFMA with each unit's work cut finer (k ranges, union-slot ranges) and
                                       summed in fixed order: a few units (latency) fill the GPU (bf16) */

/* Status codes. */
#define BLOCKFFN_OK 0
#define BLOCKFFN_ERR_NULL (-1)      /* a required pointer is NULL */
#define BLOCKFFN_ERR_SHAPE (-2)     /* unsupported or inconsistent d / E / d_e */
#define BLOCKFFN_ERR_DTYPE (-3)     /* unknown dtype */
#define BLOCKFFN_ERR_CHUNK (-4)     /* chunk_len out of range or n_tokens % chunk_len != 0 */
#define BLOCKFFN_ERR_WORKSPACE (-5) /* workspace smaller than blockffn_workspace_size() */
#define BLOCKFFN_ERR_MODE (-6)      /* unknown mode, or a mode the layer's dtype/shape cannot use */
#define BLOCKFFN_ERR_ALIGN (-7)     /* a pointer is misaligned */
#define BLOCKFFN_ERR_LAYERS (-8)    /* n_layers < 1, layers of different shapes, or too many scattered layers */
#define BLOCKFFN_ERR_HIP (-9)       /* a HIP launch failed (see blockffn_last_error) */

/*
 * One BlockFFN layer (plain data; the library takes no ownership).
 *
 * Layer arrays.  blockffn_route, blockffn_route_with and blockffn_forward
 * take `layers`, a host array of n_layers >= 1 descriptors, and unit u
 * (chunk u of chunk_len tokens) uses layers[u % n_layers]: a call can send
 * consecutive chunks through different layers, as the verify step of
 * speculative decoding sends one chunk of candidate tokens through each
 * layer of the model in turn (BlockFFN write-up §4 acceleration kernel,
 * §6 real speed-up).  The descriptors must agree in d, n_experts, d_expert,
 * dtype and rms_eps (ERR_LAYERS otherwise); their tensors may live anywhere,
 * each layer in its own allocations.  The array is read during the call
 * only.  The library reduces it before launching: a repeating array counts
 * once per period (n copies of one descriptor are one layer); layers whose
 * every pointer lies a fixed number of bytes past the previous layer's (one
 * strided allocation; NULL pointers NULL in every layer) are indexed by
 * that spacing, in any number; otherwise at most 32 distinct layers are
 * passed to the kernels by address, and more return ERR_LAYERS.
 */
typedef struct blockffn_layer {
  int32_t d;          /* hidden size */
  int32_t n_experts;  /* E */
  int32_t d_expert;   /* d_e, hidden width of one expert MLP */
  int32_t dtype;      /* BLOCKFFN_F32 or BLOCKFFN_BF16, for x and every weight */
  float rms_eps;      /* RMSNorm epsilon, inside the square root (1e-6 typical) */
  int32_t reserved;   /* must be 0 */
  const void* w_router;     /* [E][d], dtype */
  const float* b_router;    /* [E] fp32 router bias, or NULL for none */
  const float* rms_scale;   /* [E] fp32 RMSNorm scale, or NULL for ones */
  const void* w_in;         /* [E][d_e][d], dtype */
  const void* w_out;        /* [E][d][d_e], dtype */
} blockffn_layer;

/* Sparsity statistics (BlockFFN abstract; write-up §3 and §5). */
typedef struct blockffn_stats {
  int64_t n_tokens, n_chunks, n_experts, chunk_len;
  int64_t active_pairs; /* sum over tokens of |M_t|; TLS = 1 - active_pairs / (T E) */
  int64_t union_sum;    /* sum over chunks of |U_c|; CLS = 1 - union_sum / (C E) */
  int64_t reuse_num;    /* sum over t >= 1 of |M_t and M_{t-1}| */
  int64_t reuse_den;    /* sum over t >= 1 of |M_{t-1}|; reuse = reuse_num / reuse_den */
  int64_t hist[129];    /* hist[k] = tokens with exactly k active experts, k <= E */
} blockffn_stats;

/*
 * Router: pre-activations, ReLU, RMSNorm over the E outputs, activation
 * pattern (write-up §2; abstract).
 *   layers       n_layers descriptors; chunk c uses layers[c % n_layers]
 *   x            [n_tokens][d] in the layer's dtype
 *   gates        [n_tokens][E] fp32 out: g = s * ReLU(z) / sqrt(mean_E(ReLU(z)^2) + eps),
 *                exactly 0 for inactive experts
 *   token_masks  [n_tokens][W] u64 out: bit i set iff z_i > 0
 *   preact       [n_tokens][E] fp32 out (z), or NULL
 *   chunk_len    maps tokens to chunks, and so to layers when n_layers > 1
 * z is accumulated in fp32.  Errors: NULL, SHAPE, DTYPE, CHUNK, ALIGN, LAYERS, HIP.
 */
int blockffn_route(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                   int32_t chunk_len, float* gates, uint64_t* token_masks, float* preact,
                   hipStream_t stream);

/* Router kinds of blockffn_route_with. */
#define BLOCKFFN_ROUTER_BLOCKFFN 0     /* ReLU, then RMSNorm over the E outputs (blockffn_route) */
#define BLOCKFFN_ROUTER_TOPK_SOFTMAX 1 /* softmax over E; the top_k largest z keep their probability */
#define BLOCKFFN_ROUTER_RELU_SUM 2     /* ReMoE: ReLU(z) divided by its sum over the E outputs */

/*
 * Router with a selectable gate function, for comparing routers on the same
 * layer (the MoE architecture blog, intelliparadigm.com: §2.1 gives the
 * Switch Transformer router, a softmax over x W_r with TOP-K selection;
 * §5.1 gives ReMoE, ReLU gates with the output divided by their sum).  The
 * union, forward and statistics calls take its gates and masks unchanged.
 *   router   BLOCKFFN_ROUTER_*; BLOCKFFN_ROUTER_BLOCKFFN is blockffn_route
 *   top_k    1 <= top_k <= E for BLOCKFFN_ROUTER_TOPK_SOFTMAX (ignored otherwise)
 * TOPK_SOFTMAX: z as in blockffn_route (bias included); the top_k largest z
 * are selected (the lower index first among equal z); g_i = softmax(z)_i
 * for those, 0 elsewhere; mask bit i set iff selected.
 * RELU_SUM: g_i = max(z_i, 0) / sum_j max(z_j, 0) (0 when none fires); mask
 * bit i set iff z_i > 0.  rms_scale and rms_eps apply to the BlockFFN router
 * only.  Other arguments, layout and ownership as blockffn_route.
 * Errors: as blockffn_route, plus MODE (unknown router) and SHAPE (top_k).
 */
int blockffn_route_with(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                        int32_t chunk_len, int32_t router, int32_t top_k, float* gates, uint64_t* token_masks,
                        float* preact, hipStream_t stream);

/*
 * Chunk union and compaction (write-up §4; abstract: the union of the
 * parameters several consecutive tokens activate).
 *   token_masks   [n_tokens][W] u64 in
 *   chunk_masks   [C][W] u64 out: OR of the chunk's token masks
 *   active_count  [C] i32 out: number of experts in the union
 *   active_list   [C][E] i32 out: the union's experts in ascending order,
 *                 entries [active_count[c], E) set to -1
 * Errors: NULL, SHAPE, CHUNK, ALIGN, HIP.
 */
int blockffn_chunk_union(int32_t n_experts, const uint64_t* token_masks, int64_t n_tokens,
                         int32_t chunk_len, uint64_t* chunk_masks, int32_t* active_count,
                         int32_t* active_list, hipStream_t stream);

/*
 * Expert evaluation over each chunk's union (write-up §4 acceleration
 * kernel: multiply only by the union's experts, batch the chunk's tokens,
 * mask the irrelevant activations with the gates; §7: outer loop over the
 * active experts).
 *   layers     n_layers descriptors; chunk c uses layers[c % n_layers]
 *   gates, active_count, active_list   as written by the two calls above
 *                                      (active_* are ignored, and may be NULL,
 *                                      in DENSE and GROUPED modes)
 *   y          [n_tokens][d] fp32 out, overwritten:
 *              y_t = sum over i in the chunk's union of g[t][i] E_i(x_t)
 *   workspace  device scratch of at least blockffn_workspace_size() bytes,
 *              256-byte aligned; its contents need no initialisation
 * GROUPED mode (one batch through one layer: every descriptor the same): every
 * (token, expert) pair with a non-zero gate (negative where the RMS scale
 * is negative) is grouped by expert, each expert's weights are read once
 * for all of its tokens in MFMA GEMMs, and each token's per-expert partial
 * rows are summed in ascending expert order.
 * It needs bf16, d a multiple of 128, d_expert 128 or 256 (MODE otherwise)
 * and n_tokens x n_experts below 2^31 (SHAPE otherwise).
 * Errors: NULL, SHAPE, DTYPE, CHUNK, WORKSPACE, MODE, ALIGN, LAYERS, HIP.
 */
int blockffn_forward(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                     int32_t chunk_len, const float* gates, const int32_t* active_count,
                     const int32_t* active_list, int32_t mode, void* workspace,
                     size_t workspace_bytes, float* y, hipStream_t stream);

/*
 * blockffn_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It takes no workspace: its scratch space is a static device
 * array of BLOCKFFN_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held
 * from the first call on that GPU until the process ends.  The call itself
 * allocates nothing.  Arguments, modes, results and errors are those of
 * blockffn_forward, plus:
 *   - WORKSPACE when blockffn_workspace_size() for these arguments exceeds
 *     BLOCKFFN_NOALLOC_SCRATCH_BYTES (split the call; at d_expert 128 and
 *     64 experts the chunk path fits about 2000 tokens per call);
 *   - HIP when the array's device address cannot be obtained.
 * Every call on one GPU uses that GPU's one array, which keeps the previous
 * call's contents (the kernels read nothing a call has not written itself).
 * Calls that overlap in time on one GPU (on different streams, or from
 * threads whose calls are not ordered on one stream) race on the array and
 * give wrong results; calls on one stream are ordered and safe.
 */
#define BLOCKFFN_NOALLOC_SCRATCH_BYTES (32u << 20)
int blockffn_forward_noalloc(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                             int32_t chunk_len, const float* gates, const int32_t* active_count,
                             const int32_t* active_list, int32_t mode, float* y, hipStream_t stream);

/*
 * Sparsity statistics of a mask stream (abstract: TLS and 8-token CLS;
 * write-up §5: consecutive-token expert reuse, experts-per-token histogram).
 *   stats_dev  one blockffn_stats in device memory, fully overwritten
 * Errors: NULL, SHAPE, CHUNK, ALIGN, HIP.
 */
int blockffn_sparsity_stats(int32_t n_experts, const uint64_t* token_masks, int64_t n_tokens,
                            int32_t chunk_len, blockffn_stats* stats_dev, hipStream_t stream);

/*
 * One layer step: blockffn_route, blockffn_chunk_union, blockffn_forward
 * (AUTO) and blockffn_sparsity_stats in a single call (write-up §4 and §6:
 * the chunk of draft tokens that speculative decoding verifies goes through
 * each layer in turn, so a step of one or a few chunks is latency bound and
 * every launch counts).
 *   layers, x, chunk_len     as blockffn_route
 *   gates, token_masks, preact (or NULL)            as blockffn_route
 *   chunk_masks, active_count, active_list          as blockffn_chunk_union
 *   stats_dev                as blockffn_sparsity_stats, or NULL
 *   y                        as blockffn_forward
 *   workspace                at least blockffn_layer_forward_workspace_size()
 *                            bytes, 256-byte aligned, contents need no
 *                            initialisation
 * For calls of at most 64 tokens and 16 chunks with bf16, E a multiple of 16,
 * d and d_expert multiples of 128 (d <= 4096) and chunk_len <= 32, the step
 * runs as three kernels: the router's product over d-ranges of 128; the
 * up-projection of every expert in a chunk's union (each block adds its
 * expert's partials and skips the expert unless a token activates it), with
 * one more block per chunk for the gates, patterns and union; and the
 * down-projection, with one more block for the statistics.  Each block's
 * waves split the contraction and add their parts in a fixed order, so
 * results are reproducible bit for bit; they differ from the separate calls'
 * in the last bits (another summation order), so a pattern bit whose z lies
 * within rounding of 0 may differ.  The down-projection there scales each
 * expert's product with Swish(W_in x) (bf16) by the token's gate in fp32
 * instead of rounding g * Swish to bf16 first.  The workspace then holds the
 * router's partial pre-activations (n_tokens x E x d/128 fp32) and
 * Swish(W_in x) (n_tokens x E x d_expert bf16).  Other calls run the four
 * separate calls.
 * Errors: NULL, SHAPE, DTYPE, CHUNK, WORKSPACE, MODE, ALIGN, LAYERS, HIP.
 */
int blockffn_layer_forward(const blockffn_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                           int32_t chunk_len, float* gates, uint64_t* token_masks, float* preact,
                           uint64_t* chunk_masks, int32_t* active_count, int32_t* active_list,
                           blockffn_stats* stats_dev, void* workspace, size_t workspace_bytes, float* y,
                           hipStream_t stream);
/* Workspace bytes of blockffn_layer_forward (0 for invalid arguments). */
size_t blockffn_layer_forward_workspace_size(const blockffn_layer* layer, int64_t n_tokens, int32_t chunk_len);

/* Gradient outputs of blockffn_backward: fp32, caller-owned device buffers,
 * fully overwritten. */
typedef struct blockffn_grads {
  float* d_w_router;  /* [E][d] */
  float* d_b_router;  /* [E] */
  float* d_rms_scale; /* [E] */
  float* d_w_in;      /* [E][d_e][d] */
  float* d_w_out;     /* [E][d][d_e] */
} blockffn_grads;

/*
 * Layer backward over one batch through one layer: the gradients of a scalar
 * loss L with respect to x and every parameter, given dy = dL/dy.  It is the
 * chain rule through the forward defined above (write-up §2: the ReLU +
 * RMSNorm router is differentiable end to end): for every active pair (z > 0)
 *   u = W_in[i] x, h = Swish(u), q = W_out[i]^T dy, dg_i = q . h,
 *   du = g_i q Swish'(u), dW_out[i] += dy (g_i h)^T, dW_in[i] += du x^T,
 *   dx += W_in[i]^T du;
 * and per token, with r = (ms + eps)^(-1/2) and a = ReLU(z),
 *   ds_i += dg_i a_i r, dms = -(sum_i dg_i s_i a_i) r^3 / 2,
 *   dz_i = [z_i > 0] (dg_i s_i r + dms 2 a_i / E), db += dz, dW_r += dz x^T,
 *   dx += W_r^T dz.
 * Inactive pairs contribute nothing.  Active pairs are grouped by expert and
 * every product runs on the matrix cores from bf16 operands (dy, the hidden
 * gradients and dz are rounded to bf16) with fp32 accumulation; no atomics,
 * so results are bit-reproducible.
 *   layer       one layer (bf16; d a multiple of 128; d_expert 128 or 256)
 *   x           [n_tokens][d] bf16, the forward's input
 *   preact      [n_tokens][E] fp32, z as written by blockffn_route
 *   dy          [n_tokens][d] fp32, 16-byte aligned
 *   dz_extra    [n_tokens][E] fp32 or NULL: a gradient with respect to z from
 *               other terms of the loss (blockffn_cls_losses), added to dz of
 *               every (token, expert), active or not, before db, dW_r, dx
 *   workspace   at least blockffn_backward_workspace_size() bytes, 256-byte
 *               aligned, no initialisation needed
 *   dx          [n_tokens][d] fp32 out, 16-byte aligned
 *   grads       the parameter gradients (all five pointers non-NULL)
 * n_tokens x n_experts must stay below 2^31.  n_tokens == 0 writes nothing.
 * Errors: NULL, SHAPE, DTYPE, WORKSPACE, MODE (unsupported shape or dtype),
 * ALIGN, HIP.
 */
int blockffn_backward(const blockffn_layer* layer, const void* x, int64_t n_tokens, const float* preact,
                      const float* dy, const float* dz_extra, void* workspace, size_t workspace_bytes, float* dx,
                      const blockffn_grads* grads, hipStream_t stream);

/* Workspace bytes blockffn_backward needs (0 on invalid input). */
size_t blockffn_backward_workspace_size(const blockffn_layer* layer, int64_t n_tokens);

/*
 * CLS-aware training objectives on the router pre-activations (write-up §3:
 * an activation-locality loss, a binary cross-entropy between neighbouring
 * tokens' activation patterns with a sharp sigmoid standing in for the
 * pattern; a chunk-sparsification loss, the probability that an expert fires
 * for at least one token of an L-token chunk).  With p = sigmoid(alpha z):
 *   losses[0] = L_AL = mean over t < T-1 and i of BCE(p[t][i], [z[t+1][i] > 0])
 *   losses[1] = L_CS = mean over chunks c and i of 1 - prod_{t in c} (1 - p[t][i])
 *   dz (if non-NULL) = w_locality dL_AL/dz + w_chunk dL_CS/dz, [n_tokens][E] fp32,
 *                      ready to pass to blockffn_backward as dz_extra
 *   preact      [n_tokens][E] fp32, z as written by blockffn_route
 *   losses      2 fp32 in device memory, overwritten
 *   workspace   blockffn_cls_losses_workspace_size() bytes, 256-byte aligned
 * The locality target takes no gradient.  Sums are fixed-order fp32
 * (deterministic).  Errors: NULL, SHAPE (E, alpha <= 0, weights), CHUNK,
 * WORKSPACE, ALIGN, HIP.
 */
int blockffn_cls_losses(int32_t n_experts, const float* preact, int64_t n_tokens, int32_t chunk_len, float alpha,
                        float w_locality, float w_chunk, void* workspace, size_t workspace_bytes, float* losses,
                        float* dz, hipStream_t stream);

/* Workspace bytes blockffn_cls_losses needs (0 on invalid input). */
size_t blockffn_cls_losses_workspace_size(int64_t n_tokens, int32_t chunk_len);

/*
 * ---- FFF tree layer (a second activation-sparse feed-forward block) ----
 *
 * Source: "Dynamic sparsity in tree-structured feed-forward layers at
 * scale", write-up on gist.science, §2 methodology (architecture design, key
 * mechanisms) and §4 (efficiency).  The layer is P parallel perfect binary
 * trees of depth D.  Tree p has N = 2^(D+1) - 1 nodes in heap order (root 0,
 * children of node n at 2n + 1 = left and 2n + 2 = right); node n holds an
 * input row w_node[p][n][0..d), a bias b_node[p][n] and an output row
 * w_out[p][n][0..d).  For a token x, every tree routes hard from the root:
 * at level l = 0..D the current node computes c = w_node[p][n] . x + b[p][n]
 * and the walk continues right iff c > 0, so D + 1 of the N nodes run.
 *   GELU_NODES  (FFF)      y = sum_p sum_l GELU(c_{p,l}) w_out[p][n_{p,l}]
 *   GELU_OUTPUT (FFFpost)  y = GELU(sum_p sum_l c_{p,l} w_out[p][n_{p,l}])
 * with the exact GELU(c) = c Phi(c).  Sums are fp32; the dot products are
 * reduced in a fixed order, so results are bit-reproducible.
 *
 * Node rows: node n of tree p has its input row at
 * (char*)w_node + (p N + n) * node_stride and its output row at
 * (char*)w_out + (p N + n) * node_stride.  node_stride = 0 means separate
 * dense arrays (d * element size).  A node's two rows may be interleaved in
 * one array, [P][N][2][d] with w_out = w_node + d * element size and
 * node_stride = 2 d * element size: a visited node is then one contiguous
 * read, which streams faster.
 *
 * blockffn_fff_forward takes a host array of n_layers descriptors and
 * token t uses layers[t % n_layers], with the rules of BlockFFN layer
 * arrays: the descriptors agree in everything but their three pointers,
 * and a repeating array counts once per period; evenly spaced layers are
 * taken in any number, at most 32 scattered ones (ERR_LAYERS otherwise).
 */
#define BLOCKFFN_FFF_GELU_NODES 0  /* GELU on every visited node's pre-activation */
#define BLOCKFFN_FFF_GELU_OUTPUT 1 /* visited nodes linear, GELU on the summed output */

#define BLOCKFFN_FFF_SPARSE 0 /* one root-to-leaf walk per tree */
#define BLOCKFFN_FFF_DENSE 1  /* every node of every tree: the dense block of width P N (the comparison path) */

typedef struct blockffn_fff_layer {
  int32_t d;            /* model width: bf16 a multiple of 512 up to 4096, f32 a multiple of 256 up to 2048 */
  int32_t n_trees;      /* P, 1 .. 65536 */
  int32_t depth;        /* D, 0 .. 15 */
  int32_t dtype;        /* BLOCKFFN_F32 or BLOCKFFN_BF16, for x, w_node and w_out */
  int32_t activation;   /* BLOCKFFN_FFF_GELU_NODES or BLOCKFFN_FFF_GELU_OUTPUT */
  int32_t node_stride;  /* bytes between consecutive nodes' rows: 0 (= d * element size) or a
                           multiple of 16 of at least d * element size */
  const void* w_node;   /* input rows, dtype, 16-byte aligned */
  const float* b_node;  /* [P][N] fp32, or NULL for no bias */
  const void* w_out;    /* output rows, dtype, 16-byte aligned */
} blockffn_fff_layer;

/*
 * FFF layer forward.
 *   x            [n_tokens][d] in the layer's dtype, 16-byte aligned
 *   mode         BLOCKFFN_FFF_SPARSE or BLOCKFFN_FFF_DENSE
 *   split        blocks per token: 0 lets the library choose from n_tokens
 *                (one block per token for large batches, a token's trees
 *                spread over several blocks for small ones); k >= 1 asks for
 *                k (at most ceil(P / 4)).  With more than one block per token
 *                each block sums its own trees and a second kernel adds the
 *                blocks' partial outputs in order, so results depend on the
 *                split in the last bits but are reproducible for a given one
 *   paths        [n_tokens][P][D+1] i32 out: the node visited at each level,
 *                or NULL (must be NULL in DENSE mode)
 *   node_preact  [n_tokens][P][D+1] fp32 out: c at each visited node, or
 *                NULL (must be NULL in DENSE mode)
 *   workspace    blockffn_fff_workspace_size() bytes, 16-byte aligned (NULL
 *                when that size is 0); no initialisation needed
 *   y            [n_tokens][d] fp32 out, overwritten, 16-byte aligned
 * n_tokens below 2^31, and n_tokens x blocks per token too; n_tokens == 0
 * enqueues nothing.
 * Errors: NULL, SHAPE, DTYPE, MODE, WORKSPACE, ALIGN, LAYERS, HIP.
 */
int blockffn_fff_forward(const blockffn_fff_layer* layers, int32_t n_layers, const void* x, int64_t n_tokens,
                         int32_t mode, int32_t split, int32_t* paths, float* node_preact, void* workspace,
                         size_t workspace_bytes, float* y, hipStream_t stream);

/* Workspace bytes blockffn_fff_forward needs for these arguments (0 when it
 * runs one block per token, or on invalid input). */
size_t blockffn_fff_workspace_size(const blockffn_fff_layer* layer, int64_t n_tokens, int32_t split);

/*
 * Stage timing (instrumentation for profilers and benchmarks).  While set,
 * every blockffn_forward or blockffn_backward call of the calling thread
 * records events[0] on its stream before its first timed kernel and events[k]
 * right after its k-th timed stage, for k < n_events.  The timed stages of
 * the forward are the expert up-projection and down-projection (GEMV,
 * CHUNK_MFMA and DENSE modes), plus the per-token combine in GROUPED mode.
 * Those of the backward are: the router quantities and pair planning, the
 * fused per-pair pass, the router and weight gradients, the per-pair input
 * gradient rows, and the per-token combine.  `events` are caller-created
 * hipEvents in caller memory that must stay valid while set; pass NULL to
 * stop.  Errors: SHAPE (n_events < 1 with non-NULL events).
 */
int blockffn_set_stage_events(hipEvent_t* events, int32_t n_events);

/*
 * HBM streaming-read ceiling probe (instrumentation for benchmarks): reads
 * `bytes` from `buf` once with 16-byte non-temporal loads, eight in flight
 * per thread, in a grid-stride sweep of `blocks` blocks of 256 threads
 * (0 = every block the device holds at once).  The time of the call is the
 * measured ceiling the layer kernels' bandwidth is compared with.
 *   buf    device memory, 16-byte aligned; bytes a multiple of 16
 *   sink   one u32 of device memory; written only if the XOR of all the data
 *          read equals a fixed constant, so that the loads stay live
 * Errors: NULL, ALIGN (buf or bytes), SHAPE (blocks < 0), HIP.
 */
int blockffn_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream);

/* Workspace bytes blockffn_forward needs for these arguments (0 on invalid input). */
size_t blockffn_workspace_size(const blockffn_layer* layer, int64_t n_tokens, int32_t chunk_len,
                               int32_t mode);

/* Static description of a status code. */
const char* blockffn_status_string(int status);

/* Message for the calling thread's most recent failed call ("" if none). */
const char* blockffn_last_error(void);

/* BLOCKFFN_VERSION of the built library. */
int blockffn_version(void);

/* Digest of the sources the library was built from (16 hex digits: a
 * sha256 prefix over every HIP source and header, by relative name and
 * contents, in name order), or "unknown" for a build that did not set it.
 * Lets a caller check that the library it loaded matches its sources. */
const char* blockffn_build_digest(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKFFN_H_ */
