// launch.h -- internal (C++) launchers behind the C ABI.  Each enqueues its kernels on the
// given stream and returns the runtime's launch status; arguments are validated by the
// caller (api.hip).  dt: 0 = fp32 storage, 1 = bf16 storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// The grouped GEMM's tile tables inside its workspace: built by the GEMM launch itself,
// or, in the layer, by the buffer build (which has the per-expert counts at hand).
// Experts with more than `small` rows get one `table` entry per btok-row token tile,
// (expert, index of its first entry, first row, rows); experts with 1..small rows one
// `stable` entry; count[0], count[1] = entries (table entries capped at cap).
struct TileTables {
    int* count;             // [0], [1]: entries; [kClaimUp, kClaimUp + kClaimWords): see below
    int4* table;
    int4* stable;
    int cap;
    int btok;
    int small;
};
TileTables gemm_tables(void* ws, long long N, int E, int F);
// Words of the table header after the entry counts: the per-XCD tile counters of the
// persistent expert grid, 8 for the up product from kClaimUp and 8 for the down product
// from kClaimDown, set to 0 by whichever kernel writes the tables.
constexpr int kClaimUp = 16, kClaimDown = 24, kClaimWords = 16;

// Gate logits x.Wg^T as gate_splits() fp32 partial sums over K splits, [split][T][E] in
// `partials` (no bias).  *zero_word (may be NULL) and zero_buf[0, zero_n) are set to 0 by
// the launch.
int gate_splits(int dt, int T, int H, int E);
hipError_t launch_gate_logits(int dt, int T, int H, int E, const void* x, const void* wg,
                              float* partials, int* zero_word, int* zero_buf, int zero_n,
                              hipStream_t s);
// Top-k selection and renormalised weights (routing 0 softmax, 1 sigmoid) from logits =
// (sum of the partials in split order) + bias; near-tie tokens are re-decided from exact
// logits recomputed from x and wg, and counted in *refined (may be NULL).  With hist (zeroed
// beforehand), hist[t / kPftSegTokens][e] counts the picks of e among tokens of that block.
hipError_t launch_topk(int dt, int T, int E, int k, int routing, int splits,
                       const float* partials, const float* bias, const void* x, const void* wg,
                       int H, int32_t* top_experts, float* top_weights, int* refined,
                       int* hist, hipStream_t s);

// Padding-free buffers.  Workspace: [0] error word, [1] free (the layer keeps the gate's
// count there), [64 ..) per-segment error counts, then the per-segment histograms.
constexpr int kPftSegTokens = 64;          // tokens per segment of the layer's buffer build
constexpr int kPftScanMax = 1 << 14;      // segments x experts of the two-launch builds
size_t pft_ws_bytes(long long N, int E);
size_t pft_layer_ws_bytes(int T, int k, int E);
hipError_t launch_pft(int T, int k, int E, const int32_t* top_experts, int32_t* counts,
                      int32_t* offsets, int32_t* token_ids, int32_t* expert_ids,
                      int32_t* dest_pos, void* ws, hipStream_t s);
// The layer's histogram (hist of the workspace's layout, filled by launch_topk) -> counts,
// offsets, the buffer arrays and the GEMM tile tables in one launch; false when the shape
// is beyond kPftScanMax (then use launch_topk without hist and launch_pft).
bool pft_layer_fast(int T, int E);
int* pft_layer_hist(void* ws, int T, int k);
hipError_t launch_pft_layer(int T, int k, int E, const int32_t* top_experts, int32_t* counts,
                            int32_t* offsets, int32_t* token_ids, int32_t* expert_ids,
                            int32_t* dest_pos, void* ws, const TileTables& tables,
                            hipStream_t s);

hipError_t launch_dispatch(int dt, int T, int k, int H, const void* x, const int32_t* dest_pos,
                           void* xd, hipStream_t s);
hipError_t launch_combine(int dt, int T, int k, int H, const void* y, const int32_t* dest_pos,
                          const float* top_weights, void* out, hipStream_t s);

size_t gemm_ws_bytes(long long N, int E);
// a, g (both or neither, [N][F] each): the up product's two halves are stored beside h.
// tables_ready: the workspace already holds the tile tables of these offsets.
hipError_t launch_grouped_gemm(int dt, int N, int E, int H, int F, const void* xd,
                               const int32_t* offsets, const void* w1, const void* w3,
                               const void* w2, void* h, void* y, void* ws, hipStream_t s,
                               void* a = nullptr, void* g = nullptr, bool tables_ready = false);
// The same product with the dispatch fused in: row p of the up product reads x[token_ids[p]]
// (x has T rows) instead of xd[p]; nothing is written for xd.
hipError_t launch_grouped_gemm_gather(int dt, int N, int E, int H, int F, const void* x, int T,
                                      const int32_t* token_ids, const int32_t* offsets,
                                      const void* w1, const void* w3, const void* w2, void* h,
                                      void* y, void* ws, hipStream_t s, void* a = nullptr,
                                      void* g = nullptr, bool tables_ready = false);

// ---- backward ----
// out[p][n] = sum_k act[p][k] * W_e[k][n] over the expert segments, with W_e's row k the
// row k of w_lo[e] below k_split and row k - k_split of w_hi[e] (nullable) from there on;
// rows w_ld elements apart, experts w_stride apart (k_split a multiple of 64, n_feat of 64).
// ws as for launch_grouped_gemm.
hipError_t launch_grouped_kmajor(int dt, int N, int E, int K, int n_feat, const void* act,
                                 const int32_t* offsets, const void* w_lo, const void* w_hi,
                                 int k_split, long long w_ld, long long w_stride, void* out,
                                 void* ws, hipStream_t s);
// a = act.W1[e]^T and g = act.W3[e]^T, [N][F] each (act rows through gather when not NULL).
hipError_t launch_grouped_pair(int dt, int N, int E, int H, int F, const void* act,
                               const int32_t* gather, int src_rows, const int32_t* offsets,
                               const void* w1, const void* w3, void* a, void* g, void* ws,
                               hipStream_t s);
// out[e][m][f] = sum over the rows k of expert e (offsets) of act[k][m] * w[k][f], act and w
// row-major with rows a_ld and w_ld elements apart (act may start at a column offset), for
// the experts listed in elist[0, *nlist) (E an upper bound of *nlist); M and n_feat
// multiples of 64; zero16: 16 zero bytes of device memory.
hipError_t launch_wgrad_rows(int dt, int E, int M, int n_feat, const void* act, long long a_ld,
                             const void* w, long long w_ld, const int32_t* offsets,
                             const int32_t* elist, const int32_t* nlist, const void* zero16,
                             void* out, hipStream_t s);
// out[e][m][f] = sum_{k in [kofs[e], kofs[e+1])} act[m][k] * w[f][k]; act [M][ktot],
// w [n_feat][ktot], kofs multiples of 64.  With elist (device, may be NULL) only the experts
// elist[0, *nlist) are computed, E being an upper bound of *nlist.
hipError_t launch_wgrad(int dt, int E, int M, int n_feat, int ktot, const void* act,
                        const void* w, const int32_t* kofs, const int32_t* elist,
                        const int32_t* nlist, void* out, hipStream_t s);

// The whole layer backward (backward.hip): forward intermediates in, gradients out.
struct BwdParams {
    int dt, T, H, E, F, k, routing;
    const void *x, *wg;
    const float* bias;
    const void *w1, *w3, *w2;
    const int32_t* top_experts;
    const float* top_weights;
    const int32_t *counts, *offsets, *token_ids, *dest_pos;
    const void *xd, *h, *y, *dout;      // xd may be NULL (rows gathered from x)
    const void *a, *g;                  // the forward's stored up-product halves, or NULL
    void *dx, *dwg;
    float* dbias;
    void *dw1, *dw3, *dw2;
    float* dtw;                         // may be NULL
    void* ws;
};
size_t backward_ws_bytes(int dt, int T, int H, int E, int F, int k);
hipError_t launch_layer_backward(const BwdParams& b, hipStream_t s);

}  // namespace moe
