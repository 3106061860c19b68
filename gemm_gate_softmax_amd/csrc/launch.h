// launch.h -- internal (C++) launchers behind the C ABI.  Each enqueues its kernels on the
// given stream and returns the runtime's launch status; arguments are validated by the
// caller (api.hip).  dt: 0 = fp32 storage, 1 = bf16 storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Gate logits x.Wg^T as gate_splits() fp32 partial sums over K splits, [split][T][E] in
// `partials` (no bias).
int gate_splits(int dt, int T, int H, int E);
hipError_t launch_gate_logits(int dt, int T, int H, int E, const void* x, const void* wg,
                              float* partials, hipStream_t s);
// Top-k selection and renormalised weights (routing 0 softmax, 1 sigmoid) from logits =
// (sum of the partials in split order) + bias.
hipError_t launch_topk(int T, int E, int k, int routing, int splits, const float* partials,
                       const float* bias, int32_t* top_experts, float* top_weights, hipStream_t s);

size_t pft_ws_bytes(long long N, int E);
hipError_t launch_pft(int T, int k, int E, const int32_t* top_experts, int32_t* counts,
                      int32_t* offsets, int32_t* token_ids, int32_t* expert_ids,
                      int32_t* dest_pos, void* ws, hipStream_t s);

hipError_t launch_dispatch(int dt, int T, int k, int H, const void* x, const int32_t* dest_pos,
                           void* xd, hipStream_t s);
hipError_t launch_combine(int dt, int T, int k, int H, const void* y, const int32_t* dest_pos,
                          const float* top_weights, void* out, hipStream_t s);

size_t gemm_ws_bytes(long long N, int E);
hipError_t launch_grouped_gemm(int dt, int N, int E, int H, int F, const void* xd,
                               const int32_t* offsets, const void* w1, const void* w3,
                               const void* w2, void* h, void* y, void* ws, hipStream_t s);
// The same product with the dispatch fused in: row p of the up product reads x[token_ids[p]]
// (x has T rows) instead of xd[p]; nothing is written for xd.
hipError_t launch_grouped_gemm_gather(int dt, int N, int E, int H, int F, const void* x, int T,
                                      const int32_t* token_ids, const int32_t* offsets,
                                      const void* w1, const void* w3, const void* w2, void* h,
                                      void* y, void* ws, hipStream_t s);

}  // namespace moe
