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
constexpr int kBTok = 128;        // activation rows per tile
constexpr int kBFeat = 128;       // weight rows (output features) per tile and operand
constexpr int kRowBytes = 128;    // bytes of K per row and stage (64 bf16 or 32 fp32)
constexpr int kStages = 3;        // LDS ring depth: two stages in flight while one is used

enum Epilogue { kEpiLogits = 0, kEpiSwiGLU = 1, kEpiStore = 2 };

template <typename T, int NB>
struct GemmParams {
    const T* act;           // activation rows [act_rows][K]
    int act_rows;           // rows addressable in act (loads are clamped below it)
    int K;                  // shared dimension, elements
    const T* w[NB];         // weight operands; expert e starts at w[b] + e * w_stride
    long long w_stride;     // elements per expert
    int n_feat;             // output features (weight rows per expert)
    int feat_tiles;         // ceil(n_feat / kBFeat)
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

// Wait until at most N of this wave's vector-memory operations are outstanding, then meet
// the other waves.  Written as one asm statement with a memory clobber so the compiler
// neither moves LDS accesses across it nor adds a full drain of the in-flight stages.
template <int N>
__device__ __forceinline__ void wait_vm_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // simm16: vmcnt[3:0] | expcnt[6:4] (7 = no wait) | lgkmcnt[11:8] (15 = no wait) | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
}

// LDS tile layout: each stage holds kBTok activation rows then NB*kBFeat weight rows, 128
// bytes each, unpadded.  The 16-byte chunk c of row r sits in slot c ^ swz(r) with
// swz(r) = (r & 7) ^ ((r >> 3) & 1): 16 lanes reading rows r0..r0+15 (r0 % 16 == 0) at
// one k-chunk then touch 16 distinct 16-byte bank groups of a 256-byte line, and any 8
// of them 8 distinct groups of a 128-byte line.
template <typename T, int NB, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(GemmParams<T, NB> p) {
    constexpr int kRows = kBTok + NB * kBFeat;       // LDS rows per stage
    constexpr int kStageBytes = kRows * kRowBytes;
    constexpr int kBlocks = kRows / 8;               // 1 KiB blocks per stage
    constexpr int kDma = kBlocks / 4;                // DMA instructions per wave per stage
    static_assert(kBlocks % 4 == 0 && kBTok % 32 == 0 && kBFeat % 32 == 0, "tile shape");
    __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];

    // ---- which tile: XCD-contiguous order over (expert, feature tile, token tile) ----
    const int ntt = p.table ? *p.table_count : (p.dense_rows + kBTok - 1) / kBTok;
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
    const int n_e = (segn + kBTok - 1) / kBTok;
    const int q = L - p.feat_tiles * first;
    const int ftile = q / n_e;
    const int row0 = seg0 + (q - ftile * n_e) * kBTok;
    const int row_end = min(seg0 + segn, p.act_rows);
    const int f0 = ftile * kBFeat;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const size_t row_bytes = (size_t)p.K * sizeof(T);

    // ---- DMA sources: wave w fills blocks w + 4 i of every stage (8 rows per block) ----
    // Block b < kBTok/8 holds activation rows, the rest weight rows of operand
    // (b*8 - kBTok) / kBFeat: both are compile-time once i is unrolled (w < 4).
    const char* src[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int r = (wave + 4 * i) * 8 + (lane >> 3);            // row within the stage
        const int c = (lane & 7) ^ (lane >> 3) ^ (wave & 1);        // chunk held by slot lane&7
        if (i < kBTok / 32) {
            const int ar = min(row0 + r, p.act_rows - 1);
            src[i] = reinterpret_cast<const char*>(p.act) + (size_t)ar * row_bytes + c * 16;
        } else {
            constexpr int kB0 = kBTok / 32;
            const int b = (i - kB0) / (kBFeat / 32);
            const int f = min(f0 + (r - kBTok) % kBFeat, p.n_feat - 1);
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
        for (int i = 0; i < kDma; ++i) dma16(src[i] + off, base + i * 4096);
    };

    // ---- wave layout: 2 x 2 waves, each 64 token rows x 64 features per operand ----
    const int wt = wave & 1, wf = wave >> 1;
    const int l16 = lane & 15, lgrp = lane >> 4;
    const int swz = (l16 & 7) ^ (l16 >> 3);
    f32x4_t acc[NB][4][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[b][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)(row_bytes / kRowBytes);
    issue(0, 0);
    if (nk > 1) issue(1, 1);
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt landed (only stage kt+1 may still be in flight) and every wave is done
        // reading the slot that stage kt+2 is about to overwrite
        if (kt + 1 < nk) wait_vm_and_barrier<kDma>();
        else wait_vm_and_barrier<0>();
        if (kt + 2 < nk) issue(kt + 2, slot == 0 ? 2 : slot - 1);
        const char* st = lds + slot * kStageBytes;
#pragma unroll
        for (int kg = 0; kg < kRowBytes / 64; ++kg) {
            const int cs = ((kg * 4 + lgrp) ^ swz) * 16;
            uint4 fa[4], fw[NB][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const uint4*>(st + (wt * 64 + i * 16 + l16) * kRowBytes + cs);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fw[b][i] = *reinterpret_cast<const uint4*>(
                        st + (kBTok + b * kBFeat + wf * 64 + i * 16 + l16) * kRowBytes + cs);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) Mfma<T>::mac(acc[b][i][j], fw[b][i], fa[j]);
        }
        slot = slot == kStages - 1 ? 0 : slot + 1;
    }

    // ---- epilogue: lane holds token (l16) x 4 consecutive features ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int feat = f0 + wf * 64 + i * 16 + lgrp * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tok = row0 + wt * 64 + j * 16 + l16;
            if (tok >= row_end) continue;
            const f32x4_t a = acc[0][i][j];
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
                    if constexpr (EPI == kEpiSwiGLU) r[v] = silu(a[v]) * acc[NB - 1][i][j][v];
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

template <typename T, int NB, int EPI>
hipError_t launch_gemm(const GemmParams<T, NB>& p, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    grid = (grid + 7) & ~7;
    hipLaunchKernelGGL((gemm_nt_kernel<T, NB, EPI>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t gate_logits_t(int T_, int H, int E, const void* x, const void* wg, const float* bias,
                         float* logits, hipStream_t s) {
    GemmParams<T, 1> p{};
    p.act = static_cast<const T*>(x);
    p.act_rows = T_;
    p.K = H;
    p.w[0] = static_cast<const T*>(wg);
    p.w_stride = 0;
    p.n_feat = E;
    p.feat_tiles = (E + kBFeat - 1) / kBFeat;
    p.table = nullptr;
    p.table_count = nullptr;
    p.dense_rows = T_;
    p.out = logits;
    p.bias = bias;
    const int grid = ((T_ + kBTok - 1) / kBTok) * p.feat_tiles;
    return launch_gemm<T, 1, kEpiLogits>(p, grid, s);
}

template <typename T>
hipError_t grouped_t(int N, int E, int H, int F, const void* xd, const int32_t* offsets,
                     const void* w1, const void* w3, const void* w2, void* h, void* y, void* ws,
                     hipStream_t s) {
    int* count = static_cast<int*>(ws);
    int4* table = reinterpret_cast<int4*>(static_cast<char*>(ws) + 256);
    const int tok_tiles_max = (N + kBTok - 1) / kBTok + (E < N ? E : N);
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, offsets, E, N, kBTok,
                       tok_tiles_max, table, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    GemmParams<T, 2> up{};
    up.act = static_cast<const T*>(xd);
    up.act_rows = N;
    up.K = H;
    up.w[0] = static_cast<const T*>(w1);
    up.w[1] = static_cast<const T*>(w3);
    up.w_stride = (long long)F * H;
    up.n_feat = F;
    up.feat_tiles = (F + kBFeat - 1) / kBFeat;
    up.table = table;
    up.table_count = count;
    up.out = h;
    err = launch_gemm<T, 2, kEpiSwiGLU>(up, tok_tiles_max * up.feat_tiles, s);
    if (err != hipSuccess) return err;

    GemmParams<T, 1> dn{};
    dn.act = static_cast<const T*>(h);
    dn.act_rows = N;
    dn.K = F;
    dn.w[0] = static_cast<const T*>(w2);
    dn.w_stride = (long long)H * F;
    dn.n_feat = H;
    dn.feat_tiles = (H + kBFeat - 1) / kBFeat;
    dn.table = table;
    dn.table_count = count;
    dn.out = y;
    return launch_gemm<T, 1, kEpiStore>(dn, tok_tiles_max * dn.feat_tiles, s);
}

}  // namespace

size_t gemm_ws_bytes(long long N, int E) {
    const long long tiles = (N + kBTok - 1) / kBTok + (E < N ? E : N);
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
