// gate.hip -- top-k selection and renormalised softmax weights, one wave64 per token.
//
// Gating as in the X-MoE review (section 三, 训练流程 step 2: the gate emits the routing in
// buffer form, no dense dispatch mask) with top-k routing (FSMoE report, 第六部分 lists the
// routing functions a layer may use, softmax and sigmoid among them).  Selection orders
// experts by (logit desc, expert id asc) for both, since both scores increase with the
// logit.  Softmax weights are softmax over all E logits renormalised over the k picks,
// which equals exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0) because the full denominator
// cancels; sigmoid weights are s_j / sum_{i<k} s_i with s = 1 / (1 + exp(-l)).
//
// The logits come from the MFMA GEMM as fp32 sums, which differ from the exact sums by
// accumulation rounding (a few 1e-6 at H = 7168).  The layer's logit is the exact sum
// rounded once to fp32, so near ties are re-decided: the logits involved are recomputed
// as double sums (exact products, double accumulation) and rounded once, and the picks
// and their order are those of these values.
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

// Share of the exact logits of token t for experts e1 and e2 held by one wave: the products
// over the 16-byte chunks [c_beg, c_end) of the rows summed in double (each product of two
// fp32 or bf16 values is exact in double).  Every lane returns the wave's sums (the
// butterfly adds commute).  Each lane issues the loads of kRefChunks chunks of the three
// rows before it uses any, so a pass costs about one memory latency.
constexpr int kRefChunks = 4;

template <typename T>
__device__ void exact_dots2(const T* __restrict__ x, const T* __restrict__ wg, int H, int t,
                            int e1, int e2, int c_beg, int c_end, int lane, double* d1,
                            double* d2) {
    constexpr int P = 16 / (int)sizeof(T);
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
    const uint4* w1 = reinterpret_cast<const uint4*>(wg + (size_t)e1 * H);
    const uint4* w2 = reinterpret_cast<const uint4*>(wg + (size_t)e2 * H);
    double s1 = 0.0, s2 = 0.0;
    for (int c0 = c_beg + lane; c0 < c_end; c0 += kRefChunks * kWave) {
        uint4 xa[kRefChunks], wa[kRefChunks], wb[kRefChunks];
#pragma unroll
        for (int u = 0; u < kRefChunks; ++u) {
            const int c = c0 + u * kWave;
            const bool in = c < c_end;
            xa[u] = in ? xr[c] : make_uint4(0, 0, 0, 0);
            wa[u] = in ? w1[c] : make_uint4(0, 0, 0, 0);
            wb[u] = in ? w2[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kRefChunks; ++u) {
            float a[P], b[P], d[P];
            unpack16(xa[u], a, T{});
            unpack16(wa[u], b, T{});
            unpack16(wb[u], d, T{});
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const double xv = static_cast<double>(a[i]);
                s1 = fma(xv, static_cast<double>(b[i]), s1);
                s2 = fma(xv, static_cast<double>(d[i]), s2);
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        s1 += __shfl_xor(s1, m, kWave);
        s2 += __shfl_xor(s2, m, kWave);
    }
    *d1 = s1;
    *d2 = s2;
}

// n rounds of wave max over the keys (consumed): lane j < n returns pick j; *last is the
// n-th pick on every lane.
template <int NPER>
__device__ __forceinline__ uint64_t select_top(uint64_t (&key)[NPER], int n, int lane,
                                               uint64_t* last) {
    uint64_t mine = 0, w = 0;
    for (int j = 0; j < n; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NPER; ++i) best = key[i] > best ? key[i] : best;
        w = wave_max_u64(best);
        if (lane == j) mine = w;
        const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(w));
        if (lane == (e & 63)) {
#pragma unroll
            for (int i = 0; i < NPER; ++i)
                if (i == (e >> 6)) key[i] = 0ull;
        }
    }
    *last = w;
    return mine;
}

// Relative gap below which two fp32-accumulated logits are re-decided from exact sums:
// 2^-13 (1.2e-4), about fifty times the largest difference between fp32-accumulated and
// double logits measured on these shapes (2.5e-6), so every other order is already the
// order of the exact values.
#ifndef MOE_TIE_REL
#define MOE_TIE_REL (1.0f / 8192.0f)
#endif
constexpr float kTieRel = MOE_TIE_REL;

// logit(t, e) = (partials[0][t][e] + partials[1][t][e] + ...) + bias[e], summed in split
// order so the result does not depend on scheduling.  Near ties are re-decided exactly:
// among a token's picks and the first expert left out, any two neighbours closer than
// kTieRel (relative, at least absolute) get their logits recomputed as exact sums, and
// when the last pick and the first one left out are that close, so does every expert
// left out within kTieRel of the last pick.  Every other pair is farther apart than twice
// the fp32 accumulation error, so the final order is that of the exactly rounded logits.
// The four waves of a block (one token each) share those dot products, a quarter of each
// row per wave, summed in wave order; such tokens are counted in *refined.
constexpr int kCandMax = 1024 + kWave;      // candidates of one token: at most E + 1
constexpr int kMaxSplits = 8;               // K splits of the gate logits (gate_splits)

template <typename T, int NPER, int ROUTE>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void topk_kernel(
    const float* __restrict__ partials, const float* __restrict__ bias, int T_, int E, int k,
    int splits, const T* __restrict__ x, const T* __restrict__ wg, int H,
    int32_t* __restrict__ top_experts, float* __restrict__ top_weights, int* refined,
    int* __restrict__ hist) {
    __shared__ int cand[kWavesPerBlock][kCandMax];
    __shared__ int ncand[kWavesPerBlock];
    __shared__ double part[kWavesPerBlock][2];
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * kWavesPerBlock + wv;
    const bool live = t < T_;                  // (no early exit: all waves meet the barriers)
    const int lane = threadIdx.x & 63;
    const size_t stride = (size_t)T_ * E;
    // every split's partial is loaded before any is added (one memory latency instead of
    // splits x NPER dependent ones), then they are added in split order
    uint64_t key[NPER], orig[NPER];
    float pv[NPER][kMaxSplits];
    const float* row = partials + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + kWave * i;
        const bool in = live && e < E;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            pv[i][sp] = in && sp < splits ? row[sp * stride + e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + kWave * i;
        if (live && e < E) {
            float l = pv[i][0];
#pragma unroll
            for (int sp = 1; sp < kMaxSplits; ++sp)
                if (sp < splits) l += pv[i][sp];
            if (bias) l += bias[e];
            key[i] = make_key(l, e);
        } else {
            key[i] = 0ull;
        }
        orig[i] = key[i];
    }
    // the picks and, when there is one, the first expert left out (the (k+1)-th)
    const bool more = k < E;
    uint64_t last = 0, mine = 0;
    if (live) mine = select_top(key, more ? k + 1 : k, lane, &last);
    // adjacent gaps among them: lane j < k compares pick j with the next one
    const float lj = key_logit(mine);
    const float lup = __shfl(lj, lane + 1 < kWave ? lane + 1 : lane, kWave);
    const float lnext = lane + 1 < k ? lup : key_logit(last);
    const bool close = live && (lane + 1 < k || (lane + 1 == k && more)) &&
                       (lj - lnext) <= kTieRel * fmaxf(1.0f, fabsf(lj));
    const uint64_t closes = __ballot(close);          // bit j: picks j and j + 1 are close
    // candidate list: when the last pick and the first one left out are close, every expert
    // left out within kTieRel of the last pick; then every pick in a close pair
    const uint64_t below = lanemask_lt();
    int nc = 0;
    if (closes != 0ull) {
        if ((closes >> (k - 1)) & 1ull) {
            const float lk = __shfl(lj, k - 1, kWave);
            const float floor_l = lk - kTieRel * fmaxf(1.0f, fabsf(lk));
#pragma unroll
            for (int i = 0; i < NPER; ++i) {
                const int e = lane + kWave * i;
                const bool c = e < E && orig[i] < last && key_logit(orig[i]) >= floor_l;
                const uint64_t m = __ballot(c);
                if (c) cand[wv][nc + __popcll(m & below)] = e;
                nc += __popcll(m);
            }
        }
        const int npick = more ? k + 1 : k;
        const uint64_t need = (closes | (closes << 1)) & (npick < 64 ? ((1ull << npick) - 1) : ~0ull);
        const int pe = static_cast<int>(0xffffffffu - static_cast<uint32_t>(mine));
        if ((need >> lane) & 1ull) cand[wv][nc + __popcll(need & below)] = pe;
        nc += __popcll(need);
        if (npick > 64 && ((closes >> 63) & 1ull)) {
            // the first expert left out of 64 picks sits beyond the lanes
            if (lane == 0) cand[wv][nc] = static_cast<int>(0xffffffffu - static_cast<uint32_t>(last));
            ++nc;
        }
    }
    if (lane == 0) ncand[wv] = nc;
    __syncthreads();
    if (ncand[0] + ncand[1] + ncand[2] + ncand[3] > 0) {
        constexpr int P = 16 / (int)sizeof(T);
        const int chunks = H / P, q = (chunks + kWavesPerBlock - 1) / kWavesPerBlock;
        const int c_beg = min(wv * q, chunks), c_end = min(c_beg + q, chunks);
        for (int w = 0; w < kWavesPerBlock; ++w) {
            const int nw = ncand[w];
            const int tw = blockIdx.x * kWavesPerBlock + w;
            for (int p = 0; p < nw; p += 2) {
                const int ea = cand[w][p], eb = p + 1 < nw ? cand[w][p + 1] : ea;
                double da, db;
                exact_dots2(x, wg, H, tw, ea, eb, c_beg, c_end, lane, &da, &db);
                if (lane == 0) {
                    part[wv][0] = da;
                    part[wv][1] = db;
                }
                __syncthreads();
                if (wv == w) {
                    double sa = 0.0, sb = 0.0;
#pragma unroll
                    for (int u = 0; u < kWavesPerBlock; ++u) {
                        sa += part[u][0];
                        sb += part[u][1];
                    }
                    if (bias) {
                        sa += static_cast<double>(bias[ea]);
                        sb += static_cast<double>(bias[eb]);
                    }
                    const float va = static_cast<float>(sa), vb = static_cast<float>(sb);
#pragma unroll
                    for (int i = 0; i < NPER; ++i) {
                        if (lane == (ea & 63) && i == (ea >> 6)) orig[i] = make_key(va, ea);
                        if (lane == (eb & 63) && i == (eb >> 6)) orig[i] = make_key(vb, eb);
                    }
                }
                __syncthreads();
            }
        }
    }
    if (!live) return;
    if (nc > 0) {
        if (lane == 0 && refined) atomicAdd(refined, 1);
#pragma unroll
        for (int i = 0; i < NPER; ++i) key[i] = orig[i];
        mine = select_top(key, k, lane, &last);
    }
    const float lp = key_logit(mine);
    const float l0 = __shfl(lp, 0, kWave);
    float ex = 0.0f;
    if (lane < k) ex = ROUTE == 0 ? expf(lp - l0) : 1.0f / (1.0f + expf(-lp));
    const float z = wave_sum_f32(ex);
    if (lane < k) {
        const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(mine));
        top_experts[(size_t)t * k + lane] = e;
        top_weights[(size_t)t * k + lane] = ex / z;
        // the buffer build's per-segment counts (integer adds: the totals do not depend on
        // the order the atomics land in)
        if (hist) atomicAdd(&hist[(size_t)(t / kPftSegTokens) * E + e], 1);
    }
}

template <typename T, int NPER>
hipError_t launch_topk_n(int T_, int E, int k, int routing, int splits, const float* partials,
                         const float* bias, const void* x, const void* wg, int H, int32_t* te,
                         float* tw, int* refined, int* hist, hipStream_t s) {
    const int blocks = (T_ + kWavesPerBlock - 1) / kWavesPerBlock;
    const T* xt = static_cast<const T*>(x);
    const T* wt = static_cast<const T*>(wg);
    if (routing == 0)
        hipLaunchKernelGGL((topk_kernel<T, NPER, 0>), dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s,
                           partials, bias, T_, E, k, splits, xt, wt, H, te, tw, refined, hist);
    else
        hipLaunchKernelGGL((topk_kernel<T, NPER, 1>), dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s,
                           partials, bias, T_, E, k, splits, xt, wt, H, te, tw, refined, hist);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_topk_t(int T_, int E, int k, int routing, int splits, const float* partials,
                         const float* bias, const void* x, const void* wg, int H, int32_t* te,
                         float* tw, int* refined, int* hist, hipStream_t s) {
#define MOE_TOPK(NPER) launch_topk_n<T, NPER>(T_, E, k, routing, splits, partials, bias, x, wg, H, te, tw, refined, hist, s)
    if (E <= 64) return MOE_TOPK(1);
    if (E <= 128) return MOE_TOPK(2);
    if (E <= 256) return MOE_TOPK(4);
    if (E <= 512) return MOE_TOPK(8);
    return MOE_TOPK(16);
#undef MOE_TOPK
}

}  // namespace

hipError_t launch_topk(int dt, int T, int E, int k, int routing, int splits, const float* partials,
                       const float* bias, const void* x, const void* wg, int H, int32_t* te,
                       float* tw, int* refined, int* hist, hipStream_t s) {
    if (T == 0) return hipSuccess;
    return dt == 0 ? launch_topk_t<float>(T, E, k, routing, splits, partials, bias, x, wg, H, te, tw, refined, hist, s)
                   : launch_topk_t<bf16_t>(T, E, k, routing, splits, partials, bias, x, wg, H, te, tw, refined, hist, s);
}

}  // namespace moe
