// move.hip -- the two row-streaming stages: padding-free dispatch (token rows into
// expert-contiguous buffer order) and the weighted combine back to token order.
//
// X-MoE review, section 三, 训练流程 steps 3 and 6 (dispatch and combine straight from the
// padding-free buffers); FlashDMoE blog, section 1.1 (results are merged back with the gate
// weights) and section 5 (only routed tokens are moved).  Both kernels are token-major:
// one workgroup per token reads or writes its row once with 16-byte vector accesses, so
// they run at HBM speed with no atomics and give the same bits on every run.  What the
// memory path allows a stream like theirs (one workgroup per CU, 16-byte accesses over a
// 1 GiB region, `bench.py --memory-ceilings`): loads 7.7-8.0 TB/s, stores 7.4 TB/s.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGroup = 8;          // expert rows per thread in flight in the combine
// Streamed buffers larger than the 256 MiB Infinity Cache are moved with non-temporal
// accesses (measured at X-MoE Large, xd / y of 470 MB: dispatch 105 -> 88 us, combine
// 107 -> 90 us); smaller ones stay cacheable, which measured faster for them.
constexpr size_t kStreamBytes = size_t(256) << 20;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ void store16(uint4* p, const uint4& v) {
    if constexpr (NT) {
        const u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    } else {
        *p = v;
    }
}

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
    if constexpr (NT) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(w.x, w.y, w.z, w.w);
    } else {
        return *p;
    }
}

// One workgroup per token, one thread per 16-byte chunk of the row (the block is sized to
// the row, up to 1024 threads).
inline int row_threads(int chunks) { return chunks >= 1024 ? 1024 : ((chunks + 63) / 64) * 64; }

// xd[dest_pos[t][j]] = x[t] for every slot j: read the row once, write it k times.  Rows
// whose dest_pos lies outside [0, N) (the -1 of an invalid routing entry) are skipped.
template <bool NT>
__global__ __launch_bounds__(1024) void dispatch_kernel(const uint4* __restrict__ x,
                                                        const int32_t* __restrict__ dest_pos,
                                                        uint4* __restrict__ xd, int k, int N,
                                                        int chunks) {
    const int t = blockIdx.x;
    const int32_t* dp = dest_pos + (size_t)t * k;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        const uint4 v = x[(size_t)t * chunks + c];
        for (int j = 0; j < k; ++j) {
            const int p = dp[j];
            if (p >= 0 && p < N) store16<NT>(xd + (size_t)p * chunks + c, v);
        }
    }
}

// out[t] = sum_j w[t][j] * y[dest_pos[t][j]], fp32 fused multiply-add in ascending j.  The
// expert rows are loaded kGroup at a time before their FMAs (an invalid slot loads row 0
// and is then not added), so a thread has kGroup loads in flight rather than one.
template <typename T, bool NT>
__global__ __launch_bounds__(1024) void combine_kernel(const uint4* __restrict__ y,
                                                       const int32_t* __restrict__ dest_pos,
                                                       const float* __restrict__ w,
                                                       uint4* __restrict__ out, int k, int N,
                                                       int chunks) {
    constexpr int P = 16 / sizeof(T) == 8 ? 8 : 4;
    const int t = blockIdx.x;
    const int32_t* dp = dest_pos + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        float acc[P];
#pragma unroll
        for (int i = 0; i < P; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kGroup) {
            uint4 raw[kGroup];
#pragma unroll
            for (int g = 0; g < kGroup; ++g) {
                const int j = j0 + g;
                const int p = j < k ? dp[j] : -1;
                const int row = (p >= 0 && p < N) ? p : 0;
                raw[g] = load16<NT>(y + (size_t)row * chunks + c);
            }
#pragma unroll
            for (int g = 0; g < kGroup; ++g) {
                const int j = j0 + g;
                const int p = j < k ? dp[j] : -1;
                if (p < 0 || p >= N) continue;      // invalid slot contributes nothing
                float v[P];
                unpack16(raw[g], v, T{});
                const float wj = wt[j];
#pragma unroll
                for (int i = 0; i < P; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
            }
        }
        out[(size_t)t * chunks + c] = pack16(acc, T{});
    }
}

template <typename T>
void combine_t(bool nt, int T_, int k, int chunks, const void* y, const int32_t* dest_pos,
               const float* w, void* out, hipStream_t s) {
    const dim3 grid(T_), block(row_threads(chunks));
    if (nt)
        hipLaunchKernelGGL((combine_kernel<T, true>), grid, block, 0, s, static_cast<const uint4*>(y),
                           dest_pos, w, static_cast<uint4*>(out), k, T_ * k, chunks);
    else
        hipLaunchKernelGGL((combine_kernel<T, false>), grid, block, 0, s, static_cast<const uint4*>(y),
                           dest_pos, w, static_cast<uint4*>(out), k, T_ * k, chunks);
}

}  // namespace

hipError_t launch_dispatch(int dt, int T, int k, int H, const void* x, const int32_t* dest_pos,
                           void* xd, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const size_t row_bytes = (size_t)H * (dt == 0 ? 4 : 2);
    const int chunks = (int)(row_bytes / 16);
    const bool nt = row_bytes * T * k > kStreamBytes;
    const dim3 grid(T), block(row_threads(chunks));
    if (nt)
        hipLaunchKernelGGL(dispatch_kernel<true>, grid, block, 0, s, static_cast<const uint4*>(x),
                           dest_pos, static_cast<uint4*>(xd), k, T * k, chunks);
    else
        hipLaunchKernelGGL(dispatch_kernel<false>, grid, block, 0, s, static_cast<const uint4*>(x),
                           dest_pos, static_cast<uint4*>(xd), k, T * k, chunks);
    return hipGetLastError();
}

hipError_t launch_combine(int dt, int T, int k, int H, const void* y, const int32_t* dest_pos,
                          const float* top_weights, void* out, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const size_t row_bytes = (size_t)H * (dt == 0 ? 4 : 2);
    const int chunks = (int)(row_bytes / 16);
    const bool nt = row_bytes * T * k > kStreamBytes;
    if (dt == 0) combine_t<float>(nt, T, k, chunks, y, dest_pos, top_weights, out, s);
    else combine_t<bf16_t>(nt, T, k, chunks, y, dest_pos, top_weights, out, s);
    return hipGetLastError();
}

}  // namespace moe
