// gemm.hip -- MFMA tile GEMM for gfx950 shared by the gate logits and the two expert
// products, with a device-built tile table over the ragged per-expert row segments.
//
// Expert computation follows the X-MoE review (section 三, 训练流程 step 5: one GEMM per
// expert over its uneven buffer segment) and the FlashDMoE blog (section 5: rows are only
// padded locally to the tile shape, never to an expert capacity): rows past a segment's
// end are computed from clamped addresses and never stored, and an expert with no rows
// contributes no tile, so its weights are never read.
//
// Every product here is "NT": both operands are rows contiguous in the shared dimension
// K (activations [rows][K], weights [features][K]).  One workgroup (4 waves) computes a
// tile of kBTok activation rows x kBFeat weight rows for NB weight operands at once (NB = 2
// fuses the SwiGLU gate and up products so the epilogue can form silu(a) * g in registers).
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

enum Epilogue { kEpiLogits = 0, kEpiSwiGLU = 1, kEpiStore = 2 };

// Tile shapes.  Expert products: 256 token rows x 128 features x 2 operands (gate/up with
// SwiGLU) or 256 x 256 x 1 (down); both use 512 LDS rows per stage (32 KiB) and a
// 5-stage ring, so 4 stages (128 KiB) are in flight while one is consumed.  The gate
// logits use small 64 x 64 tiles so a few thousand tokens still fill the chip.
#ifndef MOE_EXPERT_BTOK
#define MOE_EXPERT_BTOK 128
#define MOE_EXPERT_UP_BF 128
#define MOE_EXPERT_DOWN_BF 256
#define MOE_EXPERT_STAGES 3
#endif
constexpr int kExpertBTok = MOE_EXPERT_BTOK;
constexpr int kExpertUpBF = MOE_EXPERT_UP_BF;
constexpr int kExpertDownBF = MOE_EXPERT_DOWN_BF;
constexpr int kExpertStages = MOE_EXPERT_STAGES;
constexpr int kGroupTok = 4;      // token tiles per L2-sharing block (see gemm_nt_kernel)

template <typename T, int NB>
struct GemmParams {
    const T* act;           // activation rows [act_rows][K]
    int act_rows;           // rows addressable in act (loads are clamped below it)
    int K;                  // shared dimension, elements
    const T* w[NB];         // weight operands; expert e starts at w[b] + e * w_stride
    long long w_stride;     // elements per expert
    int n_feat;             // output features (weight rows per expert)
    int feat_tiles;         // ceil(n_feat / BF)
    const int4* table;      // per token tile: (expert, first tile of expert, row0, rows); null = dense
    const int* table_count; // number of token tiles in table
    int dense_rows;         // rows when table is null (single expert 0)
    void* out;              // [rows][n_feat]: fp32 logits or storage type
    const float* bias;      // logits epilogue only (nullable)
};

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// One 16-byte global -> LDS transfer per lane, no register round trip (gfx950).  The LDS
// destination of a wave's instruction is the 1 KiB block at byte address `lds_block`
// (wave-uniform, passed in M0), lane L landing at byte 16 L; the global source is per
// lane.  Issued from inline asm so that the compiler's wait insertion does not treat the
// transfer as a pending write of every LDS address (that would drain the whole ring before
// each LDS read); the ring's waits are explicit (wait_vm_and_barrier).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_block) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "{m0}"(lds_block)
                 : "memory");
}

// Wait until at most N of this wave's vector-memory operations are outstanding and (when
// LGKM) all of its LDS reads have returned, then meet the other waves.
template <int N, bool LGKM>
__device__ __forceinline__ void wait_vm_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // simm16: vmcnt[3:0] | expcnt[6:4] (7 = no wait) | lgkmcnt[11:8] (15 = no wait) | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((LGKM ? 0 : 15) << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
}

// Runtime number of stages still allowed in flight (0..M) -> compile-time wait.
template <int DMA, int M, bool LGKM>
__device__ __forceinline__ void wait_stages(int m) {
    if constexpr (M == 0) {
        wait_vm_and_barrier<0, LGKM>();
    } else {
        if (m >= M) wait_vm_and_barrier<M * DMA, LGKM>();
        else wait_stages<DMA, M - 1, LGKM>(m);
    }
}

// LDS layout: a stage holds BT activation rows then NB*BF weight rows, RB bytes each
// (RB = 128: whole cache lines, so every DMA instruction issues full-line L2 requests;
// half-line requests measured ~30% slower at the L2), unpadded.  The 16-byte chunk c of
// row r sits in slot c ^ (r & 7), which reads as fast as fully contiguous data for the
// 32x32 fragment pattern (lane l: row r0 + l % 32, chunk c0 + l / 32).
template <typename T, int NB, int EPI, int BT, int BF, int S>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(GemmParams<T, NB> p) {
    constexpr int kRowBytes = 128;                   // bytes of K per row and stage
    constexpr int kRowsPerDma = 1024 / kRowBytes;    // rows per 1 KiB DMA instruction
    constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
    constexpr int kRows = BT + NB * BF;              // LDS rows per stage
    constexpr int kStageBytes = kRows * kRowBytes;
    constexpr int kDma = kRows / (4 * kRowsPerDma);  // DMA instructions per wave per stage
    constexpr int TT = BT / 64, FT = BF / 64;        // 32x32 tiles per wave (tokens, features)
    constexpr int KS = kRowBytes / 32;               // k-steps (16-byte chunk pairs) per stage
    static_assert(kRows % (4 * kRowsPerDma) == 0 && BT % 64 == 0 && BF % 64 == 0, "tile shape");
    static_assert(BT % (4 * kRowsPerDma) == 0 && BF % (4 * kRowsPerDma) == 0, "operand blocks");
    static_assert(S >= 2 && (S - 2) * kDma < 64 && S * kStageBytes <= 160 * 1024, "ring");
    __shared__ __attribute__((aligned(1024))) char lds[S * kStageBytes];

    // ---- which tile: XCD-contiguous order over (expert, feature tile, token tile) ----
    const int ntt = p.table ? *p.table_count : (p.dense_rows + BT - 1) / BT;
    const int total = ntt * p.feat_tiles;
    const int chunk = (total + 7) >> 3;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= chunk) return;
    const int L = xcd * chunk + local;
    if (L >= total) return;
    int expert = 0, first = 0, seg0 = 0, segn = p.dense_rows;
    if (p.table) {
        const int4 te = p.table[L / p.feat_tiles];
        expert = te.x; first = te.y; seg0 = te.z; segn = te.w;
    }
    // Within an expert, tiles go in blocks of kGroupTok token tiles; inside a block the
    // feature tile varies slowest.  The 32 tiles an XCD runs at once then cover about
    // 4 token tiles x 8 feature tiles, so both operands are shared through that XCD's L2
    // (a single token-tile column would share the weights but re-read every activation
    // panel).  Experts with one token tile reduce to feature-tile order.
    const int n_e = (segn + BT - 1) / BT;
    const int q = L - p.feat_tiles * first;
    const int blk_tiles = kGroupTok * p.feat_tiles;
    const int blk = min(q / blk_tiles, (n_e - 1) / kGroupTok);
    const int width = min(kGroupTok, n_e - blk * kGroupTok);
    const int ql = q - blk * blk_tiles;
    const int ftile = ql / width;
    const int ttile = blk * kGroupTok + (ql - ftile * width);
    const int row0 = seg0 + ttile * BT;
    const int row_end = min(seg0 + segn, p.act_rows);
    const int f0 = ftile * BF;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const size_t row_bytes = (size_t)p.K * sizeof(T);

    // ---- DMA sources: wave w fills row blocks w + 4 i of every stage ----
    // Block b < BT/kRowsPerDma holds activation rows, the rest weight rows of operand
    // (4 kRowsPerDma i - BT) / BF: both compile-time once i is unrolled.
    constexpr int kBlkRows = 4 * kRowsPerDma;                         // rows per i step
    const char* src[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int rl = lane / kChunks;                                // row within the block
        const int r = (wave + 4 * i) * kRowsPerDma + rl;              // row within the stage
        const int c = (lane % kChunks) ^ (rl & 7);                    // chunk held by this slot
        if (i < BT / kBlkRows) {
            const int ar = min(row0 + r, p.act_rows - 1);
            src[i] = reinterpret_cast<const char*>(p.act) + (size_t)ar * row_bytes + c * 16;
        } else {
            const int b = (kBlkRows * i - BT) / BF;
            const int f = min(f0 + (r - BT) - b * BF, p.n_feat - 1);
            src[i] = reinterpret_cast<const char*>(p.w[b] + (size_t)expert * p.w_stride) +
                     (size_t)f * row_bytes + c * 16;
        }
    }
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char*)(lds)));
    auto issue = [&](int kt, int slot) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base + slot * kStageBytes + wave * 1024);
        const size_t off = (size_t)kt * kRowBytes;
#pragma unroll
        for (int i = 0; i < kDma; ++i) dma16(src[i] + off, base + i * 4096);   // 4 waves x 1 KiB
    };

    // ---- wave layout: 2 x 2 waves, each (BT/2) tokens x (BF/2) features per operand,
    // as TT x FT tiles of 32 x 32 (MFMA rows = features, MFMA columns = tokens) ----
    const int wt = wave & 1, wf = wave >> 1;
    const int l32 = lane & 31, lhalf = lane >> 5;
    const int swz = l32 & 7;                      // row & 7 for every fragment row
    f32x16_t acc[NB][FT][TT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FT; ++i)
#pragma unroll
            for (int j = 0; j < TT; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.0f;

    // ---- main loop: KS k-steps (16-byte chunk pairs) per stage, fragments double-
    // buffered in registers.  Each k-step first reads the next k-step's fragments, then
    // issues its MFMAs (scheduling barriers keep the compiler from interleaving the two),
    // so LDS latency hides behind a block of MFMAs.  The stage barrier sits before the
    // reads of stage kt+1: once every wave holds stage kt's last fragments, its slot is
    // refilled with stage kt+S while stage kt+1 (landed) starts to be read. ----
    uint4 fa0[TT], fw0[NB][FT], fa1[TT], fw1[NB][FT];
#define MOE_LOAD_FRAGS(STAGE, KSTEP, FA, FW)                                                  \
    do {                                                                                     \
        const char* st_ = (STAGE);                                                           \
        const int cs_ = ((2 * (KSTEP) + lhalf) ^ swz) * 16;                                  \
        _Pragma("unroll") for (int j = 0; j < TT; ++j) FA[j] =                               \
            *reinterpret_cast<const uint4*>(st_ + (wt * (BT / 2) + j * 32 + l32) * kRowBytes + cs_); \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                       \
            _Pragma("unroll") for (int i = 0; i < FT; ++i) FW[b][i] = *reinterpret_cast<const uint4*>( \
                st_ + (BT + b * BF + wf * (BF / 2) + i * 32 + l32) * kRowBytes + cs_);      \
    } while (0)
#define MOE_MFMAS(FA, FW)                                                                     \
    do {                                                                                     \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                       \
            _Pragma("unroll") for (int i = 0; i < FT; ++i)                                   \
                _Pragma("unroll") for (int j = 0; j < TT; ++j) Mfma<T>::mac(acc[b][i][j], FW[b][i], FA[j]); \
    } while (0)
    static_assert(KS % 2 == 0, "k-steps alternate between the two fragment buffers");

    const int nk = (int)(row_bytes / kRowBytes);
    for (int s = 0; s < S && s < nk; ++s) issue(s, s);
    wait_stages<kDma, S - 1, false>(min(S - 1, nk - 1));          // stage 0 landed
    MOE_LOAD_FRAGS(lds, 0, fa0, fw0);
    // The last stage is peeled off so every loop iteration has the same shape (otherwise
    // the compiler's wait insertion merges paths and drains the prefetched fragments).
    int slot = 0;
    for (int kt = 0; kt < nk - 1; ++kt) {
        const char* st = lds + slot * kStageBytes;
        const int next = slot == S - 1 ? 0 : slot + 1;
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            MOE_LOAD_FRAGS(st, ks + 1, fa1, fw1);
            __builtin_amdgcn_sched_barrier(0);
            MOE_MFMAS(fa0, fw0);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 2 < KS) {
                MOE_LOAD_FRAGS(st, ks + 2, fa0, fw0);
            } else {
                // this wave's reads of stage kt are complete; stage kt+1 landed everywhere
                wait_stages<kDma, (S >= 2 ? S - 2 : 0), true>(min(S - 2, nk - 2 - kt));
                if (kt + S < nk) issue(kt + S, slot);
                MOE_LOAD_FRAGS(lds + next * kStageBytes, 0, fa0, fw0);
            }
            __builtin_amdgcn_sched_barrier(0);
            MOE_MFMAS(fa1, fw1);
            __builtin_amdgcn_sched_barrier(0);
        }
        slot = next;
    }
    {
        const char* st = lds + slot * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            MOE_LOAD_FRAGS(st, ks + 1, fa1, fw1);
            MOE_MFMAS(fa0, fw0);
            if (ks + 2 < KS) MOE_LOAD_FRAGS(st, ks + 2, fa0, fw0);
            MOE_MFMAS(fa1, fw1);
        }
    }
#undef MOE_LOAD_FRAGS
#undef MOE_MFMAS

    // ---- epilogue: lane holds one token and, per 32-feature tile, 4 runs of 4 features ----
#pragma unroll
    for (int i = 0; i < FT; ++i) {
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            const int tok = row0 + wt * (BT / 2) + j * 32 + l32;
            if (tok >= row_end) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int feat = f0 + wf * (BF / 2) + i * 32 + 8 * g + 4 * lhalf;
                float a[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) a[v] = acc[0][i][j][4 * g + v];
                if constexpr (EPI == kEpiLogits) {
                    float* o = reinterpret_cast<float*>(p.out) + (size_t)tok * p.n_feat;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (feat + v < p.n_feat) o[feat + v] = a[v] + (p.bias ? p.bias[feat + v] : 0.0f);
                } else {
                    if (feat >= p.n_feat) continue;
                    float r[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        if constexpr (EPI == kEpiSwiGLU) r[v] = silu(a[v]) * acc[NB - 1][i][j][4 * g + v];
                        else r[v] = a[v];
                    }
                    if constexpr (sizeof(T) == 4) {
                        float* o = reinterpret_cast<float*>(p.out) + (size_t)tok * p.n_feat + feat;
                        *reinterpret_cast<float4*>(o) = make_float4(r[0], r[1], r[2], r[3]);
                    } else {
                        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (size_t)tok * p.n_feat + feat;
                        const uint32_t lo = f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
                        const uint32_t hi = f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
                        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
                    }
                }
            }
        }
    }
}

// Tile table: one entry per token tile, (expert, first token tile of that expert, first
// row, rows of the expert).  Single workgroup; E <= 1024.
// Segments are clipped to [0, rows) so malformed offsets can never address past the
// buffers, and no more than `capacity` entries are written.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* offsets, int E,
                                                          int rows, int btok, int capacity,
                                                          int4* table, int* count) {
    __shared__ int scan[2][1024];
    const int e = threadIdx.x;
    int beg = 0, cnt = 0, n = 0;
    if (e < E) {
        beg = min(max(offsets[e], 0), rows);
        cnt = max(min(offsets[e + 1], rows) - beg, 0);
        n = (cnt + btok - 1) / btok;
    }
    // inclusive Hillis-Steele scan of n over the block
    int cur = 0;
    scan[0][e] = n;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = scan[cur][e] + (e >= d ? scan[cur][e - d] : 0);
        scan[cur ^ 1][e] = v;
        cur ^= 1;
        __syncthreads();
    }
    const int incl = scan[cur][e];
    const int first = incl - n;
    for (int j = 0; j < n && first + j < capacity; ++j) table[first + j] = make_int4(e, first, beg, cnt);
    if (e == 1023) *count = min(incl, capacity);
}

template <typename T, int NB, int EPI, int BT, int BF, int S>
hipError_t launch_gemm(const GemmParams<T, NB>& p, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    grid = (grid + 7) & ~7;
    hipLaunchKernelGGL((gemm_nt_kernel<T, NB, EPI, BT, BF, S>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t gate_logits_t(int T_, int H, int E, const void* x, const void* wg, const float* bias,
                         float* logits, hipStream_t s) {
    constexpr int BT = 64, BF = 64, S = 4;
    GemmParams<T, 1> p{};
    p.act = static_cast<const T*>(x);
    p.act_rows = T_;
    p.K = H;
    p.w[0] = static_cast<const T*>(wg);
    p.w_stride = 0;
    p.n_feat = E;
    p.feat_tiles = (E + BF - 1) / BF;
    p.table = nullptr;
    p.table_count = nullptr;
    p.dense_rows = T_;
    p.out = logits;
    p.bias = bias;
    const int grid = ((T_ + BT - 1) / BT) * p.feat_tiles;
    return launch_gemm<T, 1, kEpiLogits, BT, BF, S>(p, grid, s);
}

template <typename T>
hipError_t grouped_t(int N, int E, int H, int F, const void* xd, const int32_t* offsets,
                     const void* w1, const void* w3, const void* w2, void* h, void* y, void* ws,
                     hipStream_t s) {
    constexpr int BT = kExpertBTok;
    int* count = static_cast<int*>(ws);
    int4* table = reinterpret_cast<int4*>(static_cast<char*>(ws) + 256);
    const int tok_tiles_max = (N + BT - 1) / BT + (E < N ? E : N);
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, offsets, E, N, BT,
                       tok_tiles_max, table, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    constexpr int UP_BF = kExpertUpBF, DN_BF = kExpertDownBF, STAGES = kExpertStages;
    GemmParams<T, 2> up{};
    up.act = static_cast<const T*>(xd);
    up.act_rows = N;
    up.K = H;
    up.w[0] = static_cast<const T*>(w1);
    up.w[1] = static_cast<const T*>(w3);
    up.w_stride = (long long)F * H;
    up.n_feat = F;
    up.feat_tiles = (F + UP_BF - 1) / UP_BF;
    up.table = table;
    up.table_count = count;
    up.out = h;
    err = launch_gemm<T, 2, kEpiSwiGLU, BT, UP_BF, STAGES>(up, tok_tiles_max * up.feat_tiles, s);
    if (err != hipSuccess) return err;

    GemmParams<T, 1> dn{};
    dn.act = static_cast<const T*>(h);
    dn.act_rows = N;
    dn.K = F;
    dn.w[0] = static_cast<const T*>(w2);
    dn.w_stride = (long long)H * F;
    dn.n_feat = H;
    dn.feat_tiles = (H + DN_BF - 1) / DN_BF;
    dn.table = table;
    dn.table_count = count;
    dn.out = y;
    return launch_gemm<T, 1, kEpiStore, BT, DN_BF, STAGES>(dn, tok_tiles_max * dn.feat_tiles, s);
}

}  // namespace

size_t gemm_ws_bytes(long long N, int E) {
    const long long tiles = (N + kExpertBTok - 1) / kExpertBTok + (E < N ? E : N);
    return 256 + (size_t)tiles * sizeof(int4);
}

hipError_t launch_gate_logits(int dt, int T, int H, int E, const void* x, const void* wg,
                              const float* bias, float* logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    return dt == 0 ? gate_logits_t<float>(T, H, E, x, wg, bias, logits, s)
                   : gate_logits_t<bf16_t>(T, H, E, x, wg, bias, logits, s);
}

hipError_t launch_grouped_gemm(int dt, int N, int E, int H, int F, const void* xd,
                               const int32_t* offsets, const void* w1, const void* w3,
                               const void* w2, void* h, void* y, void* ws, hipStream_t s) {
    if (N == 0) return hipSuccess;
    return dt == 0 ? grouped_t<float>(N, E, H, F, xd, offsets, w1, w3, w2, h, y, ws, s)
                   : grouped_t<bf16_t>(N, E, H, F, xd, offsets, w1, w3, w2, h, y, ws, s);
}

}  // namespace moe
