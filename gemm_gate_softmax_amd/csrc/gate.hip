// gate.hip -- top-k selection and renormalised softmax weights, one wave64 per token.
//
// Gating as in the X-MoE review (section 三, 训练流程 step 2: the gate emits the routing in
// buffer form, no dense dispatch mask) with top-k routing (FSMoE report, 第六部分 lists the
// routing functions a layer may use, softmax and sigmoid among them).  Selection orders
// experts by (logit desc, expert id asc) for both, since both scores increase with the
// logit.  Softmax weights are softmax over all E logits renormalised over the k picks,
// which equals exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0) because the full denominator
// cancels; sigmoid weights are s_j / sum_{i<k} s_i with s = 1 / (1 + exp(-l)).
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

// Packed selection key: order-preserving logit in the high word, (0xffffffff - e) in the
// low word, so the largest key is the largest logit and, among equal logits, the lowest id.
__device__ __forceinline__ uint64_t make_key(float l, int e) {
    return (static_cast<uint64_t>(f32_order_key(l)) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t u = static_cast<uint32_t>(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// logit(t, e) = (partials[0][t][e] + partials[1][t][e] + ...) + bias[e], summed in split
// order so the result does not depend on scheduling.
template <int NPER, int ROUTE>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void topk_kernel(const float* __restrict__ partials,
                                                                      const float* __restrict__ bias,
                                                                      int T, int E, int k, int splits,
                                                                      int32_t* __restrict__ top_experts,
                                                                      float* __restrict__ top_weights) {
    const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const size_t stride = (size_t)T * E;
    const float* row = partials + (size_t)t * E;
    uint64_t key[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + kWave * i;
        if (e < E) {
            float l = row[e];
            for (int sp = 1; sp < splits; ++sp) l += row[sp * stride + e];
            if (bias) l += bias[e];
            key[i] = make_key(l, e);
        } else {
            key[i] = 0ull;
        }
    }
    uint64_t mine = 0;  // lane j keeps pick j
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NPER; ++i) best = key[i] > best ? key[i] : best;
        const uint64_t w = wave_max_u64(best);
        if (lane == j) mine = w;
        const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(w));
        if (lane == (e & 63)) {
#pragma unroll
            for (int i = 0; i < NPER; ++i)
                if (i == (e >> 6)) key[i] = 0ull;
        }
    }
    const float lj = key_logit(mine);
    const float l0 = __shfl(lj, 0, kWave);
    float ex = 0.0f;
    if (lane < k) ex = ROUTE == 0 ? expf(lj - l0) : 1.0f / (1.0f + expf(-lj));
    const float z = wave_sum_f32(ex);
    if (lane < k) {
        top_experts[(size_t)t * k + lane] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(mine));
        top_weights[(size_t)t * k + lane] = ex / z;
    }
}

template <int NPER>
hipError_t launch_topk_n(int T, int E, int k, int routing, int splits, const float* partials,
                         const float* bias, int32_t* te, float* tw, hipStream_t s) {
    const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    if (routing == 0)
        hipLaunchKernelGGL((topk_kernel<NPER, 0>), dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s,
                           partials, bias, T, E, k, splits, te, tw);
    else
        hipLaunchKernelGGL((topk_kernel<NPER, 1>), dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s,
                           partials, bias, T, E, k, splits, te, tw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(int T, int E, int k, int routing, int splits, const float* partials,
                       const float* bias, int32_t* te, float* tw, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (E <= 64) return launch_topk_n<1>(T, E, k, routing, splits, partials, bias, te, tw, s);
    if (E <= 128) return launch_topk_n<2>(T, E, k, routing, splits, partials, bias, te, tw, s);
    if (E <= 256) return launch_topk_n<4>(T, E, k, routing, splits, partials, bias, te, tw, s);
    if (E <= 512) return launch_topk_n<8>(T, E, k, routing, splits, partials, bias, te, tw, s);
    return launch_topk_n<16>(T, E, k, routing, splits, partials, bias, te, tw, s);
}

}  // namespace moe
