/*
 * moe.h -- C ABI of libmoe.so: the forward pass of one expert-specialised MoE layer on an
 * AMD MI355X (gfx950) GPU, as five stages plus the whole chain.
 *
 * The stages follow the X-MoE review's training pipeline (web page "X-MoE:
 * 在HPC平台上实现新兴混合专家架构的可扩展训练", section 三 技术架构, 训练流程 steps 1-3, 5
 * and 6) with its padding-free token buffers ("PFT": token_ids / expert_ids / per-expert
 * counts, 模型组件 table; O(B*H) rows with no E*C capacity, PFT复杂度分析), and the
 * single-device share of the DMoE operator of the FlashDMoE blog (section 1.1: gate, send
 * tokens to experts, expert compute, weighted merge back).
 *
 * Conventions shared by every entry point
 *   - Pointers named x, wg, w1, ... are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory, never synchronises, and enqueues all work on
 *     `stream` (a hipStream_t; NULL = the default stream).  Calls are asynchronous and can
 *     be captured into a HIP graph (no memset nodes, no host reads of device data).
 *   - Row-major layouts, weights as nn.Linear ([out][in]):  x [T][H], wg [E][H],
 *     bias [E] (fp32), w1 and w3 [E][F][H] (SwiGLU gate and up), w2 [E][H][F] (down).
 *     N = T*k is the number of routed rows.
 *   - dt selects the storage type of x, wg, w1, w3, w2, xd, h, y and out: MOE_F32 (fp32) or
 *     MOE_BF16 (bf16).  Logits, routing weights and every accumulation are fp32.
 *   - Limits: T >= 0 (T == 0 is a successful no-op), 1 <= k <= MOE_K_MAX, k <= E,
 *     1 <= E <= MOE_E_MAX, H and F positive multiples of 64, N < 2^31.  Every device
 *     pointer must be 16-byte aligned.
 *   - The returned status covers host-side validation and launch errors only; a fault in
 *     a kernel surfaces at the caller's next synchronisation.  Invalid arguments are
 *     rejected before anything is enqueued.
 *   - Workspaces are caller-owned device buffers of at least moe_workspace_bytes() bytes.
 *     Their content between calls is scratch, except the error word described at
 *     moe_pft_build.  Concurrent calls must not share a workspace.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_K_MAX 64
#define MOE_E_MAX 1024

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_VALUE = 1,       /* a size or pointer argument is out of range / NULL */
    MOE_ERR_UNSUPPORTED = 2,         /* a shape outside the limits above */
    MOE_ERR_MISALIGNED = 3,          /* a device pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE_TOO_SMALL = 4, /* ws_bytes < moe_workspace_bytes(...) */
    MOE_ERR_LAUNCH = 5,              /* the HIP runtime refused a launch */
    MOE_ERR_SCRATCH_TOO_SMALL = 6    /* moe_layer_forward_noalloc: the call needs more than
                                        MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status_t;

/*
 * Routing function of the gate (FSMoE report, 第六部分: the routing functions a layer may
 * use include softmax and sigmoid).  Both select the k experts with the largest logits;
 * they differ in the weights (see moe_gate_topk).
 */
typedef enum {
    MOE_ROUTE_SOFTMAX = 0,
    MOE_ROUTE_SIGMOID = 1
} moe_routing_t;

/* Which call a workspace is for (argument of moe_workspace_bytes). */
typedef enum {
    MOE_WS_GATE = 0,
    MOE_WS_PFT = 1,
    MOE_WS_GEMM = 2,
    MOE_WS_LAYER = 3,
    MOE_WS_BACKWARD = 4
} moe_workspace_kind_t;

/* Bytes of workspace a call needs for these sizes (0 for unsupported arguments, including
 * H not a positive multiple of 64).  Sizes that do not matter to a call are ignored (e.g.
 * F for MOE_WS_PFT). */
size_t moe_workspace_bytes(int kind, int T, int H, int E, int F, int k, moe_dtype_t dt);

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(moe_status_t status);

/*
 * Top-k softmax gate (X-MoE review, 训练流程 step 2: gating produced straight in buffer
 * form, no dense dispatch mask; FSMoE report, 第三部分 item 1, Gating Function module).
 *   logit[t][e]        = sum_h x[t][h] * wg[e][h] + bias[e]          (fp32 accumulate)
 *   The selection is that of the exactly rounded logits fp32(exact sum + bias): a token
 *   whose k + 1 largest fp32-accumulated logits hold two neighbours within 2^-13
 *   (relative, at least absolute) of each other has the logits involved recomputed as
 *   double sums and rounded once, and is decided from those.
 *   top_experts[t][j]  = the j-th expert in the order (logit desc, expert id asc), j < k
 *   top_weights[t][j]  = MOE_ROUTE_SOFTMAX: softmax(logit[t])[pick j] renormalised over
 *                        the k picks = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *                      = MOE_ROUTE_SIGMOID: s_j / sum_{i<k} s_i,  s = 1 / (1 + exp(-l))
 *                        (the pages name sigmoid routing without a formula: this is the
 *                        plainest reading, renormalised like the softmax route)
 * bias may be NULL (no bias).  Outputs: top_experts [T][k] int32, top_weights [T][k] fp32.
 * ws: moe_workspace_bytes(MOE_WS_GATE, ...) bytes (depends on T, H, E and dt: it holds
 * fp32 partial logits over up to 8 splits of the hidden dimension, which the top-k step
 * adds in split order before the bias).  After the call completes, the int32 at byte 4 of
 * ws holds the number of tokens decided from recomputed exact logits.
 */
moe_status_t moe_gate_topk(moe_dtype_t dt, int T, int H, int E, int k, moe_routing_t routing,
                           const void *x, const void *wg, const float *bias,
                           int32_t *top_experts, float *top_weights, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * Padding-free token buffers (X-MoE review, 训练流程 step 1: flatten top_experts and sort
 * it into token_ids and expert_ids; 模型组件: token_ids, expert_ids and the per-expert
 * counts "num_ids").  With flat index i = t*k + j and e = top_experts[i]:
 *   counts[e]  = #{ i : top_experts[i] == e },  offsets = exclusive scan, offsets[E] = N
 *   position(i) = offsets[e] + #{ i' < i : top_experts[i'] == e }   (stable sort by expert)
 *   token_ids[position(i)] = t,  expert_ids[position(i)] = e,  dest_pos[t][j] = position(i)
 * Every one of the N rows is assigned exactly once: no capacity, no padding rows.
 * Outputs (device, int32): counts [E], offsets [E+1], token_ids [N], expert_ids [N],
 * dest_pos [T][k].
 * ws: moe_workspace_bytes(MOE_WS_PFT, ...) bytes.  After the call completes, the int32 at
 * byte 0 of ws holds the number of entries of top_experts outside [0, E); when it is
 * non-zero those entries get dest_pos -1 and the other outputs are incomplete.
 */
moe_status_t moe_pft_build(int T, int k, int E, const int32_t *top_experts, int32_t *counts,
                           int32_t *offsets, int32_t *token_ids, int32_t *expert_ids,
                           int32_t *dest_pos, void *ws, size_t ws_bytes, void *stream);

/*
 * Padding-free dispatch (X-MoE review, 训练流程 step 3; FlashDMoE blog, section 5: only the
 * routed tokens are moved, no zero-filled rows):  xd[dest_pos[t][j]] = x[t]  for all t, j.
 * A bit-exact row copy; x [T][H] -> xd [N][H].  dest_pos must be a permutation of [0, N)
 * as produced by moe_pft_build.
 */
moe_status_t moe_dispatch(moe_dtype_t dt, int T, int k, int H, const void *x,
                          const int32_t *dest_pos, void *xd, void *stream);

/*
 * Expert computation over the uneven per-expert segments (X-MoE review, 训练流程 step 5:
 * one GEMM per expert on its own rows; FlashDMoE blog, section 5: only local padding to
 * the tile shape, never to a capacity).  Rows p in [offsets[e], offsets[e+1]) use expert e:
 *   h[p][f] = silu(a) * g,   a = sum_c xd[p][c] * w1[e][f][c],  g = sum_c xd[p][c] * w3[e][f][c]
 *   y[p][c] = sum_f h[p][f] * w2[e][c][f],      silu(a) = a / (1 + exp(-a))
 * h is rounded once to the storage type and that rounded h feeds the second product.
 * xd [N][H], offsets [E+1] (device, as from moe_pft_build), h [N][F], y [N][H].
 * Experts with no rows cost nothing.  ws: moe_workspace_bytes(MOE_WS_GEMM, ...) bytes
 * (holds the device-built tile table; sized from N = T*k and E).
 * w2 and y both NULL: only h is computed (the gate/up product and its SwiGLU); exactly
 * one of them NULL is MOE_ERR_INVALID_VALUE.
 * token_ids not NULL: the dispatch is fused into the up product.  xd then points at the
 * token rows x [src_rows][H] and product row p reads x[token_ids[p]] (token_ids [N], as from
 * moe_pft_build; ids are clamped to [0, src_rows)), which gives the same h and y as
 * moe_dispatch followed by this call; src_rows < 1 is MOE_ERR_INVALID_VALUE.  token_ids
 * NULL: xd is [N][H] and src_rows is ignored.
 */
moe_status_t moe_grouped_gemm_swiglu(moe_dtype_t dt, int N, int E, int H, int F,
                                     const void *xd, const int32_t *token_ids, int src_rows,
                                     const int32_t *offsets, const void *w1, const void *w3,
                                     const void *w2, void *h, void *y, void *ws,
                                     size_t ws_bytes, void *stream);

/*
 * Padding-free weighted combine (X-MoE review, 训练流程 step 6; FlashDMoE blog, section 1.1:
 * expert results are merged back with the gate weights):
 *   out[t][c] = sum_{j=0}^{k-1} top_weights[t][j] * y[dest_pos[t][j]][c]
 * accumulated in fp32 in ascending j, rounded once to the storage type.  Deterministic
 * (token-major gather, no atomics).  y [N][H], dest_pos [T][k], top_weights [T][k] fp32,
 * out [T][H].
 */
moe_status_t moe_combine(moe_dtype_t dt, int T, int k, int H, const void *y,
                         const int32_t *dest_pos, const float *top_weights, void *out,
                         void *stream);

/* Caller-owned intermediates of moe_layer_forward (device pointers, sizes as above). */
typedef struct moe_layer_bufs {
    int32_t *top_experts; /* [T][k] */
    float *top_weights;   /* [T][k] */
    int32_t *counts;      /* [E]    */
    int32_t *offsets;     /* [E+1]  */
    int32_t *token_ids;   /* [N]    */
    int32_t *expert_ids;  /* [N]    */
    int32_t *dest_pos;    /* [T][k] */
    void *xd;             /* [N][H], or NULL (dispatch fused into the experts) */
    void *h;              /* [N][F] */
    void *y;              /* [N][H] */
    void *a;              /* [N][F] or NULL: a = xd.W1[e]^T, stored by the forward when a and g */
    void *g;              /* [N][F] or NULL: g = xd.W3[e]^T  are both set (for the backward)   */
} moe_layer_bufs;

/*
 * The whole layer forward: gate -> buffers -> dispatch -> experts -> combine, each stage
 * exactly as the entry point of the same name, enqueued back to back on `stream` with no
 * host synchronisation.  x [T][H] -> out [T][H]; intermediates land in *bufs (every
 * pointer required except xd).  bufs->xd NULL fuses the dispatch into the expert product
 * (rows gathered from x through token_ids as they are loaded, the next step the X-MoE
 * review's padding-free dispatch allows): xd is not written and the results are identical.
 * ws: moe_workspace_bytes(MOE_WS_LAYER, ...) bytes; after the call its byte-0 int32 is the
 * error word of moe_pft_build and its byte-4 int32 the gate's count of tokens decided from
 * exact logits (moe_gate_topk).
 */
moe_status_t moe_layer_forward(moe_dtype_t dt, int T, int H, int E, int F, int k,
                               moe_routing_t routing, const void *x, const void *wg,
                               const float *bias, const void *w1, const void *w3,
                               const void *w2, void *out,
                               const moe_layer_bufs *bufs, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * The layer forward for callers that cannot allocate device memory or hand over a
 * workspace: code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, stages and results as moe_layer_forward (the same
 * kernels, bit for bit), without ws / ws_bytes: the scratch lives in one static device
 * array of MOE_NOALLOC_SCRATCH_BYTES per GPU, created when the library's code is loaded on
 * that GPU and held until the process ends.  Its device address is looked up on the first
 * call on each device.  The call allocates nothing (no hipMalloc, no library allocation).
 *   - A call whose layer workspace, moe_workspace_bytes(MOE_WS_LAYER, ...), exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH_TOO_SMALL before enqueuing anything
 *     (32 MiB: every shape with T * E <= 2^22, e.g. 4096 tokens x 1024 experts, fits; the
 *     X-MoE Large layer, T = 4096, E = 256, H = 7168, top-8, needs 16.9 MB, mostly the
 *     gate's partial logits).
 *   - Every call on one GPU uses that GPU's one array, which keeps the last call's
 *     contents; each call writes every scratch byte it later reads, so nothing needs
 *     clearing between calls.  Calls that overlap in time on one GPU (several streams or
 *     threads) race on the array and must be serialised by the caller.
 *   - The scratch words moe_layer_forward reports at bytes 0 and 4 of its workspace are
 *     not reported here (the gate's own routing never has out-of-range ids).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

moe_status_t moe_layer_forward_noalloc(moe_dtype_t dt, int T, int H, int E, int F, int k,
                                       moe_routing_t routing, const void *x, const void *wg,
                                       const float *bias, const void *w1, const void *w3,
                                       const void *w2, void *out,
                                       const moe_layer_bufs *bufs, void *stream);

/*
 * The layer backward.  The pages present the layer as part of a training system (X-MoE
 * review, section 三, 训练流程: the forward pass is followed by the backward pass and the
 * weight update) but give no backward formulas; these are the derivatives of the forward
 * above for a loss L with dL/dout = dout, the expert picks held fixed:
 *   dy[p]      = top_weights[t][j] * dout[t],   dtop_weights[t][j] = <dout[t], y[p]>
 *   dh         = dy . W2[e],   da = dh * g * silu'(a),   dg = dh * silu(a)
 *                (a, g recomputed from the routed rows; silu'(a) = s (1 + a (1 - s)))
 *   dxd        = da . W1[e] + dg . W3[e]
 *   dW2[e]     = sum_p dy[p]^T h[p],  dW1[e] = sum_p da[p]^T xd[p],  dW3[e] = sum_p dg[p]^T xd[p]
 *   dl (picked logits) from dtop_weights through the routing weights: softmax over the picks,
 *                dl_j = w_j (dw_j - sum_i w_i dw_i); sigmoid, dl_j = (dw_j - sum_i w_i dw_i) / S
 *                * s_j (1 - s_j) with s = sigmoid(logit), S = sum of the picks' s
 *   dx[t]      = sum_j dxd[dest_pos[t][j]] + sum_j dl_tj Wg[e_tj]
 *   dWg[e]     = sum_t dl_te x[t],   dbias[e] = sum_t dl_te
 * (p = dest_pos[t][j], e = top_experts[t][j], h and y as the forward stored them).
 * Inputs: the forward's inputs and its intermediates in *fwd (top_experts, top_weights,
 * counts, offsets, token_ids, dest_pos, h and y required; xd may be NULL, the rows are
 * then gathered from x), and dout [T][H].  Outputs: dx [T][H], dwg [E][H], dw1 and dw3
 * [E][F][H], dw2 [E][H][F] in the storage type; dbias [E] fp32; dtop_weights [T][k] fp32
 * (may be NULL).  Experts without rows get zero weight gradients.  All accumulation is
 * fp32, each output is rounded once; results are deterministic (no atomics).
 * ws: moe_workspace_bytes(MOE_WS_BACKWARD, ...) bytes: row-sized intermediates, about
 * (3H + 5F)Tk + (H + E)(T + 63) elements plus small tables (2.1 GB at T=4096, H=7168,
 * E=256, F=2048, k=8, bf16); the weights and the row-major activations are read as stored,
 * never transposed into copies.  T == 0 is a no-op (nothing is written).
 */
moe_status_t moe_layer_backward(moe_dtype_t dt, int T, int H, int E, int F, int k,
                                moe_routing_t routing, const void *x, const void *wg,
                                const float *bias, const void *w1, const void *w3,
                                const void *w2, const moe_layer_bufs *fwd, const void *dout,
                                void *dx, void *dwg, float *dbias, void *dw1, void *dw3,
                                void *dw2, float *dtop_weights, void *ws, size_t ws_bytes,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
