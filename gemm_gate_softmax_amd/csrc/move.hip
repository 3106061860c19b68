// move.hip -- the two row-streaming stages: padding-free dispatch (token rows into
// expert-contiguous buffer order) and the weighted combine back to token order.
//
// X-MoE review, section 三, 训练流程 steps 3 and 6 (dispatch and combine straight from the
// padding-free buffers); FlashDMoE blog, section 1.1 (results are merged back with the gate
// weights) and section 5 (only routed tokens are moved).  Both kernels are token-major:
// one workgroup per token reads or writes its row once with 16-byte vector accesses, so
// they run at HBM speed with no atomics and give the same bits on every run.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// xd[dest_pos[t][j]] = x[t] for every slot j: read the row once, write it k times.
// Rows whose dest_pos lies outside [0, N) (the -1 of an invalid routing entry) are skipped.
__global__ __launch_bounds__(kThreads) void dispatch_kernel(const uint4* __restrict__ x,
                                                            const int32_t* __restrict__ dest_pos,
                                                            uint4* __restrict__ xd, int k, int N,
                                                            int chunks) {
    const int t = blockIdx.x;
    const int32_t* dp = dest_pos + (size_t)t * k;
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
        const uint4 v = x[(size_t)t * chunks + c];
        for (int j = 0; j < k; ++j) {
            const int p = dp[j];
            if (p >= 0 && p < N) xd[(size_t)p * chunks + c] = v;
        }
    }
}

// out[t] = sum_j w[t][j] * y[dest_pos[t][j]], fp32 fused multiply-add in ascending j.
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint4* __restrict__ y,
                                                           const int32_t* __restrict__ dest_pos,
                                                           const float* __restrict__ w,
                                                           uint4* __restrict__ out, int k,
                                                           int N, int chunks) {
    constexpr int P = 16 / sizeof(T) == 8 ? 8 : 4;
    const int t = blockIdx.x;
    const int32_t* dp = dest_pos + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
        float acc[P];
#pragma unroll
        for (int i = 0; i < P; ++i) acc[i] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int p = dp[j];
            if (p < 0 || p >= N) continue;  // invalid slot contributes nothing
            float v[P];
            unpack16(y[(size_t)p * chunks + c], v, T{});
            const float wj = wt[j];
#pragma unroll
            for (int i = 0; i < P; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
        }
        out[(size_t)t * chunks + c] = pack16(acc, T{});
    }
}

}  // namespace

hipError_t launch_dispatch(int dt, int T, int k, int H, const void* x, const int32_t* dest_pos,
                           void* xd, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int chunks = H * (dt == 0 ? 4 : 2) / 16;
    hipLaunchKernelGGL(dispatch_kernel, dim3(T), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), dest_pos, static_cast<uint4*>(xd), k, T * k, chunks);
    return hipGetLastError();
}

hipError_t launch_combine(int dt, int T, int k, int H, const void* y, const int32_t* dest_pos,
                          const float* top_weights, void* out, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int chunks = H * (dt == 0 ? 4 : 2) / 16;
    if (dt == 0)
        hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(kThreads), 0, s,
                           static_cast<const uint4*>(y), dest_pos, top_weights,
                           static_cast<uint4*>(out), k, T * k, chunks);
    else
        hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(T), dim3(kThreads), 0, s,
                           static_cast<const uint4*>(y), dest_pos, top_weights,
                           static_cast<uint4*>(out), k, T * k, chunks);
    return hipGetLastError();
}

}  // namespace moe
