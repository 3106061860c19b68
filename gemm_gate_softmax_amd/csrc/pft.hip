// pft.hip -- padding-free token buffers: a stable counting sort of the flattened routing
// by expert, in three launches (segment histograms, scan, ranked scatter).
//
// X-MoE review, section 三: 训练流程 step 1 (flatten top_experts and sort it into token_ids
// and expert_ids) and 模型组件 (token_ids, expert_ids, per-expert counts).  The buffer has
// exactly N = T*k rows (PFT复杂度分析: O(B*H) instead of O(E*C*H)).
//
// The flat routing array (index i = t*k + j) is cut into segments of kSeg entries, one per
// wave.  Positions are offsets[e] + (entries of e in earlier segments) + (entries of e
// earlier in this segment); the last term comes from wave ballots on the bits of e, so
// the sort is stable without atomics and the result is the same on every run.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kSegChunks = 8;
constexpr int kSeg = kWave * kSegChunks;  // routing entries per wave
constexpr int kWavesPerBlock = 4;
constexpr int kEMax = 1024;

// Workspace: [0] error word, [64 ..) per-segment error counts, then hist[nseg][E].
struct PftWs {
    int* err;
    int* seg_err;
    int* hist;
};

__host__ __device__ inline long long pft_nseg(long long N) { return (N + kSeg - 1) / kSeg; }

__host__ __device__ inline PftWs carve(void* ws, long long N) {
    int* base = static_cast<int*>(ws);
    const long long nseg = pft_nseg(N);
    PftWs w;
    w.err = base;
    w.seg_err = base + 64;
    w.hist = base + 64 + ((nseg + 63) / 64) * 64;
    return w;
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void pft_hist_kernel(
    const int32_t* __restrict__ te, long long N, int E, int nseg, PftWs w) {
    __shared__ int hist[kWavesPerBlock][kEMax];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int seg = blockIdx.x * kWavesPerBlock + wv;
    for (int e = lane; e < E; e += kWave) hist[wv][e] = 0;
    __syncthreads();
    int bad = 0;
    if (seg < nseg) {
#pragma unroll 4
        for (int c = 0; c < kSegChunks; ++c) {
            const long long i = (long long)seg * kSeg + c * kWave + lane;
            if (i < N) {
                const int e = te[i];
                if (e >= 0 && e < E) atomicAdd(&hist[wv][e], 1);
                else ++bad;
            }
        }
    }
    __syncthreads();
    if (seg < nseg) {
        for (int e = lane; e < E; e += kWave) w.hist[(size_t)seg * E + e] = hist[wv][e];
        const int nbad = wave_sum_i32(bad);
        if (lane == 0) w.seg_err[seg] = nbad;
    }
}

// One workgroup: per-expert exclusive prefix over segments (the position of a segment's
// first entry of expert e within e's rows), counts and offsets.  Segment counts are read
// kBatch at a time before any is written back, so their latencies overlap.
__global__ __launch_bounds__(kEMax) void pft_scan_kernel(int E, int nseg, int32_t* counts,
                                                         int32_t* offsets, PftWs w) {
    constexpr int kBatch = 16;
    __shared__ int scan[2][kEMax];
    __shared__ int bad[kEMax];
    const int e = threadIdx.x;
    // out-of-range ids: a strided partial sum of the per-segment counts per thread, summed
    // over the block in the scan's steps below
    int my_bad = 0;
    for (int s = e; s < nseg; s += kEMax) my_bad += w.seg_err[s];
    int run = 0;
    if (e < E) {
        for (int s0 = 0; s0 < nseg; s0 += kBatch) {
            int v[kBatch];
            if (s0 + kBatch <= nseg) {           // a whole batch: the loads issue together
#pragma unroll
                for (int b = 0; b < kBatch; ++b) v[b] = w.hist[(size_t)(s0 + b) * E + e];
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    w.hist[(size_t)(s0 + b) * E + e] = run;
                    run += v[b];
                }
            } else {
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
                    v[b] = s0 + b < nseg ? w.hist[(size_t)(s0 + b) * E + e] : 0;
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    if (s0 + b < nseg) w.hist[(size_t)(s0 + b) * E + e] = run;
                    run += v[b];
                }
            }
        }
        counts[e] = run;
    }
    int cur = 0;
    scan[0][e] = run;
    bad[e] = my_bad;
    __syncthreads();
    for (int d = 1; d < kEMax; d <<= 1) {
        const int v = scan[cur][e] + (e >= d ? scan[cur][e - d] : 0);
        scan[cur ^ 1][e] = v;
        if ((e & (2 * d - 1)) == 0) bad[e] += bad[e + d];    // tree sum: bad[0] at the end
        cur ^= 1;
        __syncthreads();
    }
    const int incl = scan[cur][e];
    const int base = incl - run;
    if (e < E) {
        offsets[e] = base;
        if (e == E - 1) offsets[E] = incl;
    }
    if (e == 0) *w.err = bad[0];
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void pft_scatter_kernel(
    const int32_t* __restrict__ te, long long N, int k, int E, int nseg, int nbits, PftWs w,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ token_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ dest_pos) {
    __shared__ int next[kWavesPerBlock][kEMax];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int seg = blockIdx.x * kWavesPerBlock + wv;
    if (seg >= nseg) return;  // whole wave; the waves never meet at a block barrier
    for (int e = lane; e < E; e += kWave) next[wv][e] = offsets[e] + w.hist[(size_t)seg * E + e];
    wave_fence();
    const uint64_t below = lanemask_lt();
    for (int c = 0; c < kSegChunks; ++c) {
        const long long i = (long long)seg * kSeg + c * kWave + lane;
        const bool valid = i < N;
        const int e = valid ? te[i] : 0;
        const bool ok = valid && e >= 0 && e < E;
        uint64_t same = ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t set = ballot(bit);
            same &= bit ? set : ~set;
        }
        if (ok) {
            const int base = next[wv][e];
            const int pos = base + __popcll(same & below);
            token_ids[pos] = static_cast<int32_t>(i / k);
            expert_ids[pos] = e;
            dest_pos[i] = pos;
            if ((same >> lane) == 1ull) next[wv][e] = base + __popcll(same);  // last of its group
        } else if (valid) {
            dest_pos[i] = -1;
        }
        wave_fence();
    }
}

}  // namespace

size_t pft_ws_bytes(long long N, int E) {
    const long long nseg = pft_nseg(N);
    return (size_t)(64 + ((nseg + 63) / 64) * 64 + nseg * E) * sizeof(int);
}

hipError_t launch_pft(int T, int k, int E, const int32_t* te, int32_t* counts, int32_t* offsets,
                      int32_t* token_ids, int32_t* expert_ids, int32_t* dest_pos, void* ws,
                      hipStream_t s) {
    const long long N = (long long)T * k;
    const int nseg = static_cast<int>(pft_nseg(N));
    const PftWs w = carve(ws, N);
    const int blocks = (nseg + kWavesPerBlock - 1) / kWavesPerBlock;
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    if (nseg > 0) {
        hipLaunchKernelGGL(pft_hist_kernel, dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s, te, N,
                           E, nseg, w);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // The scan also runs for N == 0 so counts/offsets/error word are always written.
    hipLaunchKernelGGL(pft_scan_kernel, dim3(1), dim3(kEMax), 0, s, E, nseg, counts, offsets, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nseg == 0) return err;
    hipLaunchKernelGGL(pft_scatter_kernel, dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s, te, N,
                       k, E, nseg, nbits, w, offsets, token_ids, expert_ids, dest_pos);
    return hipGetLastError();
}

}  // namespace moe
