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

// ---- two-launch builds: segment counts, then one "place" launch ----
// When the segment-by-expert count matrix is small (nseg * E <= kPftScanMax), every block
// of the place kernel reads all of it and works out for itself what the scan kernel
// would have produced: each expert's total (counts), the exclusive scan over experts
// (offsets), and where each of its own segments' runs start within every expert.  That
// saves the scan launch; the matrix is at most 64 KiB, read whole into LDS.  Segments are
// seg_len consecutive routing entries (512 for moe_pft_build; 64 tokens x k in the layer,
// whose counts the top-k step adds up as it picks).
constexpr int kPlaceThreads = 256;
constexpr int kPlaceWaves = kPlaceThreads / kWave;   // each places a quarter of the segment
constexpr int kPlacePrefetch = 8;                   // routing chunks loaded ahead per wave

// In-place exclusive prefix sum of v[0, n) in LDS (n <= 4 * kPlaceThreads) by the whole
// block; returns the total.  The caller has synchronised after writing v.
__device__ int block_exclusive_scan(int* v, int n, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int loc[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = 4 * tid + i;
        loc[i] = idx < n ? v[idx] : 0;
        sum += loc[i];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    int run = incl - sum, total = 0;
#pragma unroll
    for (int i = 0; i < kPlaceWaves; ++i) {
        const int ws = wsum[i];
        if (i < w) run += ws;
        total += ws;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = 4 * tid + i;
        if (idx < n) v[idx] = run;
        run += loc[i];
    }
    __syncthreads();
    return total;
}

// Bitmask of the lanes holding the same valid expert id as this lane (0 for an invalid
// entry), from log2(E) ballots on the bits of the id.
__device__ __forceinline__ uint64_t same_expert(bool ok, int e, int nbits) {
    uint64_t same = ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t set = ballot(bit);
        same &= bit ? set : ~set;
    }
    return ok ? same : 0ull;
}

// One block per segment.  Each wave owns a quarter of the segment's entries: it first
// counts its quarter's entries per expert (into LDS), then, once every quarter is counted,
// places them after the segment's earlier quarters, chunk by chunk in entry order.
__global__ __launch_bounds__(kPlaceThreads) void pft_place_kernel(
    const int32_t* __restrict__ te, long long N, int k, int E, int nseg, int seg_len, int nbits,
    const int* __restrict__ hist, const int* __restrict__ seg_err, int* __restrict__ err,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ token_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ dest_pos, TileTables tt) {
    __shared__ __attribute__((aligned(16))) int hs[kPftScanMax];   // the whole [nseg][E] matrix
    __shared__ int qcnt[kPlaceWaves][kEMax];  // per quarter, then where its run of e starts
    __shared__ int cnt[kEMax], offs[kEMax], nm[kEMax], ns[kEMax], before[kEMax];
    __shared__ int wsum[kPlaceWaves];
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int seg = blockIdx.x;
    // this wave's quarter of the segment and its routing ids, loaded first
    const long long sbeg = (long long)seg * seg_len;
    const long long send = min(sbeg + seg_len, N);
    const int qlen = (seg_len + kPlaceWaves - 1) / kPlaceWaves;
    const long long q0 = min(sbeg + (long long)wv * qlen, send), q1 = min(q0 + qlen, send);
    const int nch = (int)((q1 - q0 + kWave - 1) / kWave);
    // 1. the count matrix into LDS (16-byte loads, all issued before any is used)
    {
        const int n = nseg * E;
        const int n4 = n >> 2;                 // E is not always a multiple of 4: tail below
        const int4* h4 = reinterpret_cast<const int4*>(hist);
        constexpr int kLd = kPftScanMax / 4 / kPlaceThreads;
        int4 v[kLd];
#pragma unroll
        for (int u = 0; u < kLd; ++u) {
            const int i = tid + u * kPlaceThreads;
            v[u] = i < n4 ? h4[i] : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kLd; ++u) {
            const int i = tid + u * kPlaceThreads;
            if (i < n4) reinterpret_cast<int4*>(hs)[i] = v[u];
        }
        for (int i = 4 * n4 + tid; i < n; i += kPlaceThreads) hs[i] = hist[i];
        for (int e = tid; e < E; e += kPlaceThreads)
#pragma unroll
            for (int w = 0; w < kPlaceWaves; ++w) qcnt[w][e] = 0;
    }
    __syncthreads();
    // 2. per expert: total count and the count in the segments before this one
    for (int e = tid; e < E; e += kPlaceThreads) {
        int run = 0, b = 0;
        for (int sg = 0; sg < nseg; ++sg) {
            if (sg == seg) b = run;
            run += hs[sg * E + e];
        }
        cnt[e] = run;
        offs[e] = run;
        before[e] = b;
    }
    // 3. this wave's quarter, counted per expert (the last lane of each group of equal ids
    // adds the group's size; every group of a chunk writes a different expert)
    const uint64_t below = lanemask_lt();
    for (int c = 0; c < nch; ++c) {
        const long long i = q0 + (long long)c * kWave + lane;
        const int e = i < q1 ? te[i] : -1;
        const bool ok = i < q1 && e >= 0 && e < E;
        const uint64_t same = same_expert(ok, e, nbits);
        if (ok && (same >> lane) == 1ull) qcnt[wv][e] += __popcll(same);
        wave_fence();
    }
    __syncthreads();
    // 4. offsets = exclusive scan of the counts over experts; each quarter's start per expert
    const int total = block_exclusive_scan(offs, E, wsum);
    for (int e = tid; e < E; e += kPlaceThreads) {
        int run = offs[e] + before[e];
#pragma unroll
        for (int w = 0; w < kPlaceWaves; ++w) {
            const int c = qcnt[w][e];
            qcnt[w][e] = run;
            run += c;
        }
    }
    if (blockIdx.x == 0) {
        // counts, offsets, the error word and the GEMM's tile tables
        int bad = 0;
        if (seg_err)
            for (int sg = tid; sg < nseg; sg += kPlaceThreads) bad += seg_err[sg];
        bad = wave_sum_i32(bad);
        for (int e = tid; e < E; e += kPlaceThreads) {
            counts[e] = cnt[e];
            offsets[e] = offs[e];
            const int c = cnt[e];
            nm[e] = tt.count && c > tt.small ? (c + tt.btok - 1) / tt.btok : 0;
            ns[e] = tt.count && c > 0 && c <= tt.small ? 1 : 0;
        }
        if (tid == 0) offsets[E] = total;
        if (lane == 0) wsum[wv] = bad;                 // (wsum is free: the scan has synced)
        __syncthreads();
        if (tid == 0) *err = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
        if (tt.count) {
            const int tot_m = block_exclusive_scan(nm, E, wsum);
            const int tot_s = block_exclusive_scan(ns, E, wsum);
            for (int e = tid; e < E; e += kPlaceThreads) {
                const int c = cnt[e], beg = offs[e], fm = nm[e];
                if (c > tt.small) {
                    const int n = (c + tt.btok - 1) / tt.btok;
                    for (int j = 0; j < n && fm + j < tt.cap; ++j)
                        tt.table[fm + j] = make_int4(e, fm, beg, c);
                } else if (c > 0) {
                    tt.stable[ns[e]] = make_int4(e, ns[e], beg, c);
                }
            }
            if (tid == 0) {
                tt.count[0] = min(tot_m, tt.cap);
                tt.count[1] = tot_s;
            }
            if (tid < kClaimWords) tt.count[kClaimUp + tid] = 0;   // persistent grid's counters
        }
    }
    __syncthreads();
    // 5. each wave places its quarter: rank among equal ids from the ballots, after the
    // quarter's earlier chunks
    int* next = qcnt[wv];
    for (int c0 = 0; c0 < nch; c0 += kPlacePrefetch) {
        int ev[kPlacePrefetch];
#pragma unroll
        for (int c = 0; c < kPlacePrefetch; ++c) {
            const long long i = q0 + (long long)(c0 + c) * kWave + lane;
            ev[c] = (c0 + c < nch && i < q1) ? te[i] : -1;
        }
#pragma unroll
        for (int c = 0; c < kPlacePrefetch; ++c) {
            if (c0 + c >= nch) break;
            const long long i = q0 + (long long)(c0 + c) * kWave + lane;
            const bool valid = i < q1;
            const int e = ev[c];
            const bool ok = valid && e >= 0 && e < E;
            const uint64_t same = same_expert(ok, e, nbits);
            if (ok) {
                const int base = next[e];
                const int pos = base + __popcll(same & below);
                token_ids[pos] = static_cast<int32_t>(i / k);
                expert_ids[pos] = e;
                dest_pos[i] = pos;
                if ((same >> lane) == 1ull) next[e] = base + __popcll(same);  // last of its group
            } else if (valid) {
                dest_pos[i] = -1;
            }
            wave_fence();
        }
    }
}

hipError_t launch_place(const int32_t* te, long long N, int k, int E, int nseg, int seg_len,
                        const int* hist, const int* seg_err, int* err, int32_t* counts,
                        int32_t* offsets, int32_t* token_ids, int32_t* expert_ids,
                        int32_t* dest_pos, const TileTables& tt, hipStream_t s) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const int blocks = nseg > 0 ? nseg : 1;
    hipLaunchKernelGGL(pft_place_kernel, dim3(blocks), dim3(kPlaceThreads), 0, s, te, N, k, E,
                       nseg, seg_len, nbits, hist, seg_err, err, counts, offsets, token_ids,
                       expert_ids, dest_pos, tt);
    return hipGetLastError();
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
    if ((long long)nseg * E <= kPftScanMax) {   // counts, offsets and placement in one launch
        const TileTables none{};
        return launch_place(te, N, k, E, nseg, kSeg, w.hist, w.seg_err, w.err, counts, offsets,
                            token_ids, expert_ids, dest_pos, none, s);
    }
    // The scan also runs for N == 0 so counts/offsets/error word are always written.
    hipLaunchKernelGGL(pft_scan_kernel, dim3(1), dim3(kEMax), 0, s, E, nseg, counts, offsets, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nseg == 0) return err;
    hipLaunchKernelGGL(pft_scatter_kernel, dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s, te, N,
                       k, E, nseg, nbits, w, offsets, token_ids, expert_ids, dest_pos);
    return hipGetLastError();
}

size_t pft_layer_ws_bytes(int T, int k, int E) {
    const long long N = (long long)T * k;
    const long long nseg512 = pft_nseg(N), nseg_tok = (T + kPftSegTokens - 1) / kPftSegTokens;
    const long long nseg = nseg512 > nseg_tok ? nseg512 : nseg_tok;
    return (size_t)(64 + ((nseg512 + 63) / 64) * 64 + nseg * E) * sizeof(int);
}

bool pft_layer_fast(int T, int E) {
    return (long long)((T + kPftSegTokens - 1) / kPftSegTokens) * E <= kPftScanMax;
}

int* pft_layer_hist(void* ws, int T, int k) { return carve(ws, (long long)T * k).hist; }

hipError_t launch_pft_layer(int T, int k, int E, const int32_t* te, int32_t* counts,
                            int32_t* offsets, int32_t* token_ids, int32_t* expert_ids,
                            int32_t* dest_pos, void* ws, const TileTables& tables,
                            hipStream_t s) {
    const long long N = (long long)T * k;
    const PftWs w = carve(ws, N);
    const int nseg = (T + kPftSegTokens - 1) / kPftSegTokens;
    return launch_place(te, N, k, E, nseg, kPftSegTokens * k, w.hist, nullptr, w.err, counts,
                        offsets, token_ids, expert_ids, dest_pos, tables, s);
}

}  // namespace moe
