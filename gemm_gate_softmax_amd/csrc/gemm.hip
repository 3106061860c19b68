// gemm.hip -- MFMA tile GEMM for gfx950 shared by the gate logits and the two expert
// products, with a device-built tile table over the ragged per-expert row segments.
//
// Expert computation follows the X-MoE review (section 三, 训练流程 step 5: one GEMM per
// expert over its uneven buffer segment) and the FlashDMoE blog (section 5: rows are only
// padded locally to the tile shape, never to an expert capacity): rows past a segment's
// end are computed from clamped addresses and never stored, and an expert with no rows
// contributes no tile, so its weights are never read.
//
// The forward's products are "NT": both operands are rows contiguous in the shared
// dimension K (activations [rows][K], weights [features][K]).  The backward's products
// also take operands stored K-major (weights [K][features], activations [K][rows]) as they
// are, transposing them in the LDS fragment read.  NB = 2 fuses the SwiGLU gate and up
// products so the epilogue forms silu(a) * g in registers.
//
// An expert tile is 128 tokens x (128 x NB or 256) features, or 64 tokens for an expert
// with at most 64 rows (and for every expert of a problem too small to give each CU a
// usual tile).  A workgroup is 4 loader waves, which stage the operands through
// an LDS ring with direct-to-LDS transfers, and 4 compute waves in a 2 x 2 layout, which
// read the ring and issue the MFMAs.  An expert with a handful of rows still gets a whole
// tile (its MFMAs and activation transfers for empty token columns are skipped): its time
// goes to streaming the expert's weights, which measured no slower through this path than
// through registers.  The up product can
// gather its activation rows from the token rows through token_ids, which fuses the
// dispatch into it.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 512;   // 4 compute waves + 4 loader waves

// kEpiPair (NB = 2) stores both products, a to out and g to out2 (the backward needs them);
// kEpiSwiGLUPair stores h = silu(a) * g to out and also a to out2, g to out3 (a forward whose
// backward is to follow).
enum Epilogue { kEpiLogits = 0, kEpiSwiGLU = 1, kEpiStore = 2, kEpiPair = 3, kEpiSwiGLUPair = 4 };

// Tile shapes.  Expert products: 128 tokens; up product 128 features x 2 operands, down
// product 256 features; a 3-slot ring of 48 KiB k-slices (64 k per row, whole 128-byte
// lines).  The gate logits use small 64 x 64 tiles over K splits so a few thousand tokens
// still fill the chip.  The macros exist to build variants for measurement.
#ifndef MOE_SMALL_BTOK
#define MOE_SMALL_BTOK 64      // 0: no small tiles
#endif
#ifndef MOE_SMALL_STAGES
#define MOE_SMALL_STAGES 3
#endif
#ifndef MOE_EXPERT_BTOK
#define MOE_EXPERT_BTOK 128
#define MOE_EXPERT_UP_BF 128
#define MOE_EXPERT_DOWN_BF 256
#define MOE_EXPERT_STAGES 3
#define MOE_EXPERT_RB 128
#define MOE_GROUP_TOK 8
#endif
constexpr int kExpertBTok = MOE_EXPERT_BTOK;
constexpr int kExpertUpBF = MOE_EXPERT_UP_BF;
constexpr int kExpertDownBF = MOE_EXPERT_DOWN_BF;
constexpr int kExpertStages = MOE_EXPERT_STAGES;
constexpr int kExpertRowBytes = MOE_EXPERT_RB;
constexpr int kGroupTok = MOE_GROUP_TOK;   // token tiles per L2-sharing block (expert_gemm_kernel)
// The same when the activation rows are gathered from the token rows (the dispatch fused
// into the up product): x is T rows, which stay in the caches, so sharing a weight panel
// among more token tiles pays.  At X-MoE Large the fused layer measured 4.27 / 4.23 / 4.19 /
// 4.16 ms for blocks of 8 / 12 / 16 / 32, while the product reading xd slows from 2.87 to
// 3.09 ms at 32.
#ifndef MOE_GROUP_TOK_GATHER
#define MOE_GROUP_TOK_GATHER 32
#endif
constexpr int kGroupTokGather = MOE_GROUP_TOK_GATHER;
// The down product reads h (N x F, 134 MB at X-MoE Large, which the caches mostly hold
// after the up product wrote it): blocks of 32 measured 1.3% faster than 8 there.
#ifndef MOE_GROUP_TOK_DOWN
#define MOE_GROUP_TOK_DOWN 32
#endif
constexpr int kGroupTokDown = MOE_GROUP_TOK_DOWN;
// bf16 tiles: scheduling hints place one fragment read after each MFMA (compute_tile)
#ifndef MOE_INTERLEAVE_READS
#define MOE_INTERLEAVE_READS 1
#endif
constexpr bool kInterleave = MOE_INTERLEAVE_READS != 0;
// In a launch that also streams small experts' weights, a large tile starts its K loop at
// slice ((rb + w fb) mod P) * nk / P and wraps around (rb: its first row's 128-row block
// within the expert, fb: its first feature's block of the usual tile width, w: the expert's
// count of 128-row blocks capped at 32, so tiles of every height sum in the same order).
// There the large tiles start at staggered times as CUs free up from tiles of unequal
// length, one tile every nk / P slices or so per XCD; tiles go out in blocks of up to 32
// token tiles with the feature tile slowest, so a tile's neighbour in the token direction
// starts about nk / P slices later and its neighbour in the feature direction about w nk / P
// later, and with those offsets both read the same slices at about the same time, which
// lets them share operand slices in L2; without small tiles, tiles start and run together
// and the natural order shares best.  The start depends only on the tile and its expert's
// row count, so a gathered (fused-dispatch) product and one reading xd sum in the same
// order.  Measured (fused layer, on / off): X-MoE Large 4.19 / 4.25 ms, X-MoE Super 5.27 /
// 5.33 ms; X-MoE Medium (no small experts) 1.81 / 1.77 ms and dense products up to 30%
// slower with it, hence the condition.  P = 16 and 64 read more and ran slower at X-MoE
// Large; 0 switches it off.  A fixed feature step of 7 in place of w (tuned for blocks of 8
// token tiles): up product 2.544 / 2.527 ms and 2.546 / 2.527 ms (7 / w) at X-MoE Large,
// 0.564 / 0.559 ms at Small, 3.181 / 3.166 ms at Super.
#ifndef MOE_K_ROTATE
#define MOE_K_ROTATE 32
#endif
constexpr bool kRotate = MOE_K_ROTATE != 0;
constexpr int kRotPeriod = MOE_K_ROTATE > 0 ? MOE_K_ROTATE : 1;
// Products with one weight operand (the down product, the backward's dh and dxd) rotate
// only with MOE_K_ROTATE_DOWN=1: with the persistent tile loop the down product ran faster
// without it (fused layer at X-MoE Large, rotated / not: 4.005 / 3.970 ms and 4.011 / 3.973
// ms in two alternating rounds; X-MoE Small level).
#ifndef MOE_K_ROTATE_DOWN
#define MOE_K_ROTATE_DOWN 0
#endif
constexpr bool kRotateDown = MOE_K_ROTATE_DOWN != 0;
// Experts with at most kSmallBTok rows get one small tile: kSmallBTok tokens, the same
// features, a kSmallStages-slot ring.  Such a tile is mostly a weight stream; in its own
// list it can be spread evenly among the MFMA-heavy tiles of the large experts, and its
// MFMAs are shared by all four compute waves (a 128-token tile leaves two of them idle).
// Its weights, which no other tile reads, are loaded non-temporal so they do not displace
// the large tiles' shared operands from L2.  Measured on the X-MoE Large routing: grouped
// GEMM 4.58 -> 4.57 ms for the separate list, -> 4.40 ms with the non-temporal weights
// (same box); a fourth ring slot for the small tile (the LDS it frees allows one) changed
// nothing.
constexpr int kSmallBTok = MOE_SMALL_BTOK;
constexpr int kSmallStages = MOE_SMALL_STAGES;
// bf16 expert products (the forward's two, and the backward's recompute of a and g and its
// products with K-major weights, dh and dxd) run as a persistent tile loop, one workgroup
// per CU claiming tiles from per-XCD counters, so a tile's start-up (table lookups, the
// first slices' latency) overlaps the previous tile's epilogue (expert_gemm_kernel, PST).
// Measured, fused layer, one-tile-per-workgroup grid against the loop (same box,
// alternating): X-MoE Small 0.997 / 0.965 ms, Medium 1.743 / 1.714, Large 4.117 / 4.048;
// the top-2 fp32 layer, whose tiles are four times longer per k-slice, ran 2.243 / 2.282 ms
// with it, so fp32 keeps one tile per workgroup.  A static schedule (tile i, i + W, ... per
// workgroup) instead of the counters: X-MoE Large 4.180 ms.  The backward's dh and dxd on
// the loop: layer backward 14.90 -> 14.79 / 14.83 ms at X-MoE Large, 3.395 -> 3.373 ms at
// Small.  0 switches the loop off.
#ifndef MOE_PERSIST
#define MOE_PERSIST 1
#endif
constexpr bool kPersist = MOE_PERSIST != 0;

template <typename T, int NB>
struct GemmParams {
    const T* act;           // activation rows [act_rows][K], or [src_rows][K] when gathered
    int act_rows;           // rows of the product (loads are clamped below it)
    const int32_t* gather;  // nullable: product row r reads act row gather[r] (< src_rows)
    int src_rows;           // rows of act when gathered
    int K;                  // shared dimension, elements
    const T* w[NB];         // weight operands; expert e starts at w[b] + e * w_stride
    long long w_stride;     // elements per expert
    int n_feat;             // output features (weight rows per expert)
    int feat_tiles;         // compute tiles per token tile: ceil(n_feat / BF)
    const int4* table;      // token tiles: (expert, first entry of the expert, row0, rows)
    const int4* stable;     // small-tile experts: (expert, entry, row0, rows)
    const int* table_count; // [0] entries in table, [1] entries in stable
    int dense_rows;         // rows of the single expert of a dense product (gate)
    void* out;              // [rows][n_feat]: fp32 partial logits or storage type
    void* out2;             // kEpiPair: the second operand's product; kEpiSwiGLUPair: a
    void* out3;             // kEpiSwiGLUPair: g
    int k_slices;           // dense product: k-slices per K split
    int group_tok;          // expert product: token tiles per L2-sharing block (0: kGroupTok)
    long long w_ld;         // K-major weights: elements from one k row to the next
    int w_k2;               // K-major weights: first k-slice read from the second tensor
    long long w_k2_adj;     // bytes added to weight addresses from k-slice w_k2 on
    long long a_ld;         // K-major activations: elements from one k row to the next
    int k_rows;             // K-major operands: k rows of the tile's K range (rows past it
                            // are read from zero16)
    const void* zero16;     // 16 zero bytes
    int* zero_word;         // dense product: set to 0 by workgroup 0 (nullable)
    int* zero_buf;          // dense product: zero_buf[0, zero_n) set to 0 (nullable)
    int zero_n;
    int* claim;             // persistent expert grid: 8 per-XCD tile counters, 0 at launch
};

// Writes 4 consecutive fp32 partial logits of one token (per-element bounds: E need not be
// a multiple of 4; the top-k step adds the bias).
__device__ __forceinline__ void store_logits(float* out, int n_feat, int tok, int feat,
                                             const float (&r)[4]) {
    float* o = out + (size_t)tok * n_feat;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        if (feat + v < n_feat) o[feat + v] = r[v];
}

// Output element type of a product: fp32 for the gate's partial logits, else the storage type.
template <bool Logits, typename T>
struct PickOut {
    using type = T;
};
template <typename T>
struct PickOut<true, T> {
    using type = float;
};

#ifndef MOE_FAST_SILU
#define MOE_FAST_SILU 1
#endif
// silu(a) = a / (1 + e^-a).  The fast form multiplies by the hardware reciprocal (1 ulp)
// instead of an IEEE division (about ten instructions per output in every tile's
// epilogue); h is rounded to the storage type right after.
__device__ __forceinline__ float silu(float a) {
    if constexpr (MOE_FAST_SILU) return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
    else return a / (1.0f + __expf(-a));
}

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

// The same with the non-temporal hint, for data read exactly once.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds_block) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
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

// The same with a wave-uniform run-time count n in [LO, HI] (a compile-time wait per value).
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_and_barrier_rt(int n) {
    if constexpr (LO >= HI) {
        wait_vm_and_barrier<LO, false>();
    } else {
        if (n >= HI) wait_vm_and_barrier<HI, false>();
        else wait_vm_and_barrier_rt<LO, HI - 1>(n);
    }
}

// LDS layout: a stage holds BT activation rows then NB*BF weight rows, RB bytes each
// (RB = 128: whole cache lines; RB = 64: half lines, which halves a stage so the ring can
// be deeper), unpadded.  The 16-byte chunk c of row r sits in slot c ^ swz(r).  The LDS
// serves a 16-byte-per-lane read 16 lanes at a time from 64 four-byte banks, so the 16
// rows a fragment read touches at once (lane l: row r0 + l % 32, chunk c0 + l / 32) must
// land on 16 distinct 16-byte bank groups of a 256-byte window: rows r and r + 8 (128-byte
// rows) or r and r + 4 (64-byte rows) share the window position and differ in swz(r).
// Measured: 200 B/clk per CU, as fast as contiguous reads; c ^ (r & 7) reached 113.
template <int BT, int BF, int NB, int S, int RB>
struct CompTile {
    static_assert(RB == 64 || RB == 128, "row bytes");
    static constexpr int kRowBytes = RB;                    // bytes of K per row and stage
    static constexpr int kRows = BT + NB * BF;              // LDS rows per stage
    static constexpr int kStageBytes = kRows * kRowBytes;
    static constexpr int kLdsBytes = S * kStageBytes;
};

template <int RB>
__device__ __forceinline__ int chunk_swizzle(int r) {
    return RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

// K-major weights (the backward's dh = dy W2[e] and dxd = da W1[e] + dg W3[e] contract over
// the row index of the stored weights): a stage holds each k-slice as n-blocks of KPS = RB /
// sizeof(T) features, KPS k rows per n-block, each row the block's KPS features of one k
// (RB bytes, 16-byte chunks permuted by kmajor_swizzle).  The direct-to-LDS transfers stay
// whole-row copies; the transpose happens in the fragment read.
__device__ __forceinline__ int kmajor_swizzle(int k) { return ((k >> 1) & 1) << 2; }

typedef short moe_v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) int lds_int;

// This lane's weight fragment of a K-major region for features [mrow, mrow + 32) (mrow a
// multiple of 32) and k-step KSTEP: what the K-contiguous layout's 16-byte read gives, i.e.
// 8 consecutive k (bf16) or 4 (fp32, element e for the e-th MFMA) of feature mrow + l % 32.
// bf16 uses the gfx950 LDS transpose read: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes 4j + i / 4 (j = 0..3), so lane L of a group
// addresses features 4 (L % 4) .. +3 of k row L / 4, and lane i gets 4 consecutive k of one
// feature; two reads give the 8 k of the MFMA's operand.  fp32 reads its 4 k one by one.
template <typename T, int RB>
__device__ __forceinline__ uint4 kmajor_frag(const char* region, int mrow, int kstep, int lane) {
    constexpr int KPS = RB / (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
        const int g = lane >> 4, L = lane & 15;
        const int n = mrow + 16 * (g & 1) + 4 * (L & 3);
        const int nb = n / KPS, nn = n % KPS;
        const int k = 16 * kstep + 8 * (g >> 1) + (L >> 2);
        const char* a = region + (nb * KPS + k) * RB + (((nn >> 3) ^ kmajor_swizzle(k)) << 4) + (nn & 7) * 2;
        typedef __attribute__((address_space(3))) moe_v4s_t lds_v4s;
        const moe_v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(a));
        const moe_v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(a + 4 * RB));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        return make_uint4(l2.x, l2.y, h2.x, h2.y);
    } else {
        const int l32 = lane & 31, lhalf = lane >> 5;
        const int n = mrow + l32;
        const int nb = n / KPS, nn = n % KPS;
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 8 * kstep + 4 * lhalf + e;
            v[e] = *reinterpret_cast<const uint32_t*>(
                region + (nb * KPS + k) * RB + (((nn >> 2) ^ kmajor_swizzle(k)) << 4) + (nn & 3) * 4);
        }
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// One tile: activation rows [row0, row0 + BT) (stored below row_end) against weight rows
// [f0, f0 + BF) of each operand of `expert`, by a workgroup of 8 waves in two roles.
// Waves 4..7 only move data: each issues its share of every stage's direct-to-LDS
// transfers into an S-slot ring.  Waves 0..3 only read LDS and issue MFMAs.  A memory
// instruction waits at issue until the CU's address path (about 64 bytes per clock)
// accepts it, and a wave stalled there issues nothing else; with the roles split, the
// compute wave that shares a SIMD with a loader keeps its MFMAs going meanwhile.  One
// barrier per stage hands the slots over: before barrier kt every loader has seen stage kt
// land and every compute wave has finished reading stage kt-1, so after it stage kt is
// read while stage kt+S-1 is loaded into the slot stage kt-1 left.  WNT marks the weight
// transfers non-temporal: for a tile that is the only reader of its weights.  The tile
// visits k-slices rot, rot+1, ..., nk-1, 0, ..., rot-1 of its K range (rot < nk).  WKM:
// the weights are stored K-major (w[b][k][n], rows w_ld apart), see kmajor_frag; AKM: the
// activations too (act[k][m], rows a_ld apart; the tile's "rows" are then m).  K-major
// rows at or past k_rows read zeros.
//
// LDS_BYTES > 0: one of a run of tiles on the same workgroup (a persistent tile loop over
// an LDS array of LDS_BYTES).  The epilogue then stages its outputs in the last STG bytes
// of the array instead of the first, so the loaders can run ahead into the next tile's
// first stages while the compute waves still store this one: the stages whose slots lie
// below LDS_BYTES - STG are issued before barrier 0, the rest after it.  A loader lane with
// a non-null `note` claims the workgroup's next tile once its own transfers are done:
// it writes next_base + (*claim, incremented) to `note` (LDS) before the tile's last barrier.
template <typename T, int NB, int EPI, int BT, int BF, int S, int RB, bool FULL, bool WNT = false,
          bool WKM = false, bool AKM = false, int LDS_BYTES = 0, int STG = 0>
__device__ __forceinline__ void compute_tile(const GemmParams<T, NB>& p, char* lds, int expert,
                                             int row0, int row_end, int f0, int s0, int nk,
                                             int rot = 0, volatile lds_int* note = nullptr,
                                             int* claim = nullptr, int next_base = 0) {
    using Tile = CompTile<BT, BF, NB, S, RB>;
    constexpr int kRowBytes = Tile::kRowBytes;
    constexpr int kRowsPerDma = 1024 / kRowBytes;    // rows per 1 KiB DMA instruction
    constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
    constexpr int kRows = Tile::kRows;
    constexpr int kStageBytes = Tile::kStageBytes;
    constexpr int kDma = kRows / (4 * kRowsPerDma);  // DMA instructions per loader per stage
    constexpr int TT = BT / 64, FT = BF / 64;        // 32x32 tiles per compute wave
    constexpr int KS = kRowBytes / 32;               // k-steps (16-byte chunk pairs) per stage
    static_assert(kRows % (4 * kRowsPerDma) == 0 && BT % 64 == 0 && BF % 64 == 0, "tile shape");
    static_assert(BT % (4 * kRowsPerDma) == 0 && BF % (4 * kRowsPerDma) == 0, "operand blocks");
    static_assert(S >= 2 && (S - 2) * kDma < 64 && S * kStageBytes <= 160 * 1024, "ring");
    static_assert(KS % 2 == 0, "k-steps alternate between the two fragment buffers");
    constexpr bool kRun = LDS_BYTES > 0;
    // stages issued before barrier 0 (slots clear of the staging region when kRun)
    constexpr int kFree = kRun ? (LDS_BYTES - STG) / kStageBytes : S - 1;
    constexpr int PRE = kFree < S - 1 ? kFree : S - 1;
    static_assert(PRE >= 1 && (!kRun || (STG > 0 && STG <= LDS_BYTES && S * kStageBytes <= LDS_BYTES)),
                  "persistent layout");

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const size_t row_bytes = (size_t)p.K * sizeof(T);
    const size_t k_off = (size_t)s0 * kRowBytes;     // first k-slice of this tile's K range

    if (wave >= 4) {
        // ---- loader: wave 4 + w fills row blocks w + 4 i of every stage.  Block b <
        // BT/kRowsPerDma holds activation rows, the rest weight rows of operand
        // (4 kRowsPerDma i - BT) / BF: both compile-time once i is unrolled. ----
        const int lw = wave - 4;
        constexpr int kBlkRows = 4 * kRowsPerDma;                     // rows per i step
        constexpr int KPS = kRowBytes / (int)sizeof(T), kPer = 16 / (int)sizeof(T);
        const char* src[kDma];
        int krow[kDma];                                               // K-major: k row held
#pragma unroll
        for (int i = 0; i < kDma; ++i) {
            const int rl = lane / kChunks;                            // row within the block
            const int r = (lw + 4 * i) * kRowsPerDma + rl;            // row within the stage
            const int c = (lane % kChunks) ^ chunk_swizzle<RB>(r);    // chunk held by this slot
            krow[i] = 0;
            if (i < BT / kBlkRows && AKM) {
                // k row kr of n-block nb of the activations (n = m); this slot holds chunk cw
                const int nb = r / KPS, kr = r % KPS;
                const int cw = (lane % kChunks) ^ kmajor_swizzle(kr);
                const int m = min(row0 + nb * KPS + cw * kPer, p.act_rows - kPer);
                src[i] = reinterpret_cast<const char*>(p.act + ((size_t)s0 * KPS + kr) * p.a_ld + m);
                krow[i] = kr;
            } else if (i < BT / kBlkRows) {
                int ar = min(row0 + r, p.act_rows - 1);
                if (p.gather) ar = min(max(p.gather[ar], 0), p.src_rows - 1);   // fused dispatch
                src[i] = reinterpret_cast<const char*>(p.act) + (size_t)ar * row_bytes + k_off + c * 16;
            } else if constexpr (WKM) {
                // k row kr of n-block nb of operand b; this slot holds its chunk cw
                const int b = (kBlkRows * i - BT) / BF;
                const int rr = r - BT - b * BF, nb = rr / KPS, kr = rr % KPS;
                const int cw = (lane % kChunks) ^ kmajor_swizzle(kr);
                const int n = min(f0 + nb * KPS + cw * kPer, p.n_feat - kPer);
                src[i] = reinterpret_cast<const char*>(p.w[b] + (size_t)expert * p.w_stride +
                                                       ((size_t)s0 * KPS + kr) * p.w_ld + n);
                krow[i] = kr;
            } else {
                const int b = (kBlkRows * i - BT) / BF;
                const int f = min(f0 + (r - BT) - b * BF, p.n_feat - 1);
                src[i] = reinterpret_cast<const char*>(p.w[b] + (size_t)expert * p.w_stride) +
                         (size_t)f * row_bytes + k_off + c * 16;
            }
        }
        const uint32_t wbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                                   (__attribute__((address_space(3))) char*)(lds))) + lw * 1024;
        // all of stage KT into slot SLOT (4 loaders x 1 KiB per 4 KiB block).  Once every
        // stage has been issued, the remaining iterations issue nothing and wait for fewer
        // outstanding transfers (only a K range shorter than the ring issues clamped
        // copies of the last stage up front).  A tile that is not FULL transfers only the activation-row blocks holding a row
        // below row_end (the vector-memory path is limited by cache-line requests, and an
        // expert with a handful of rows would otherwise move mostly duplicate rows).  The
        // skipped rows' LDS holds stale data that only ever meets the MFMA columns of
        // tokens that are never stored.
        constexpr int kActDma = BT / kBlkRows;                         // activation blocks per loader
        const int nact = FULL || AKM ? kActDma
                                     : min(max((min(row_end - row0, BT) - lw * kRowsPerDma + kBlkRows - 1) /
                                                   kBlkRows, 0), kActDma);
        const int keff = kDma - (kActDma - nact);                     // transfers per slice
        // K-major weights advance by KPS rows per k-slice (and switch tensors at w_k2)
        const long long wslice = WKM ? (long long)KPS * p.w_ld * (long long)sizeof(T) : 0;
        const long long aslice = AKM ? (long long)KPS * p.a_ld * (long long)sizeof(T) : 0;
        const char* zero16 = static_cast<const char*>(p.zero16);
#define MOE_ISSUE(KT, SLOT)                                                                   \
        do {                                                                                 \
            const uint32_t b_ = __builtin_amdgcn_readfirstlane(wbase + (SLOT) * kStageBytes); \
            const int ks_ = (KT) + rot;                                                      \
            const int kk_ = ks_ >= nk ? ks_ - nk : ks_;                                      \
            const size_t o_ = (size_t)kk_ * kRowBytes;                                       \
            const long long ow_ = WKM ? kk_ * wslice + (kk_ >= p.w_k2 ? p.w_k2_adj : 0) : (long long)o_; \
            const long long oa_ = AKM ? kk_ * aslice : (long long)o_;                       \
            _Pragma("unroll") for (int i_ = 0; i_ < kDma; ++i_) {                            \
                const bool w_ = i_ >= kActDma;                                               \
                const char* a_ = src[i_] + (w_ ? ow_ : oa_);                                 \
                if ((w_ ? WKM : AKM) && kk_ * KPS + krow[i_] >= p.k_rows) a_ = zero16;       \
                if (w_ && WNT) dma16_nt(a_, b_ + i_ * 4096);                                 \
                else if (w_ || i_ < nact) dma16(a_, b_ + i_ * 4096);                         \
            }                                                                                \
        } while (0)
        if (nk == 1) {
            // a single k-slice (weight gradients of experts with at most 64 rows): no
            // clamped copies, nothing follows barrier 0
            MOE_ISSUE(0, 0);
            wait_vm_and_barrier<0, false>();
        } else {
            for (int s = 0; s < PRE; ++s) MOE_ISSUE(min(s, nk - 1), s);
            // barrier 0: stage 0 landed
            if constexpr (FULL) wait_vm_and_barrier<(PRE - 1) * kDma, false>();
            else wait_vm_and_barrier_rt<(PRE - 1) * (kDma - kActDma), (PRE - 1) * kDma>((PRE - 1) * keff);
            // the previous tile's staging is read by now: its slots can be filled
            for (int s = PRE; s < S - 1; ++s) MOE_ISSUE(min(s, nk - 1), s);
        }
        int refill = S - 1;
        for (int kt = 0; kt < nk - 1; ++kt) {
            // barrier kt+1: stage kt+1 landed
            if (kt + S - 1 < nk) {
                MOE_ISSUE(kt + S - 1, refill);                      // slot of stage kt-1
                if constexpr (FULL) wait_vm_and_barrier<(S - 2) * kDma, false>();
                else wait_vm_and_barrier_rt<(S - 2) * (kDma - kActDma), (S - 2) * kDma>((S - 2) * keff);
            } else if constexpr (S == 3) {
                wait_vm_and_barrier<0, false>();                     // nothing issued after kt+1
            } else {
                // the nk-2-kt (< S-2) stages after kt+1 may still be in flight
                wait_vm_and_barrier_rt<0, (S - 3) * kDma>((nk - 2 - kt) * (FULL ? kDma : keff));
            }
            refill = refill == S - 1 ? 0 : refill + 1;
        }
#undef MOE_ISSUE
        // (every transfer has landed: the last wait above was for none outstanding)
        if constexpr (kRun) {
            // the compute waves are still on the last stage: the claim's latency hides there
            if (note)
                *note = next_base + __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("" ::: "memory");                          // the write stays above
            __builtin_amdgcn_s_waitcnt(7 << 4);                      // vmcnt(0) lgkmcnt(0)
        } else {
            __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));       // vmcnt(0)
        }
        __builtin_amdgcn_s_barrier();                               // ring free: staging
        return;
    }

    // ---- compute: 2 x 2 waves, each (BT/2) tokens x (BF/2) features per operand, as
    // TT x FT tiles of 32 x 32 (MFMA rows = features, MFMA columns = tokens) ----
    const int wt = wave & 1, wf = wave >> 1;
    const int l32 = lane & 31, lhalf = lane >> 5;
    const int swz = chunk_swizzle<RB>(l32);       // fragment rows start at multiples of 32
    // A tile that is not FULL (an expert's last, or only, token tile) skips the MFMAs of
    // 32-token column tiles holding no row below row_end: for an expert with a handful of
    // rows most of the tile's MFMA work.
    const int jn = FULL ? TT : (min(max(row_end - (row0 + wt * (BT / 2)), 0), BT / 2) + 31) / 32;
    f32x16_t acc[NB][FT][TT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FT; ++i)
#pragma unroll
            for (int j = 0; j < TT; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.0f;

    // KS k-steps (16-byte chunk pairs) per stage, fragments double-buffered in registers.
    // Each k-step first reads the next k-step's fragments, then issues its MFMAs
    // (scheduling barriers keep the compiler from interleaving the two), so LDS latency
    // hides behind a block of MFMAs.  The stage barrier sits before the reads of stage
    // kt+1, once this wave's reads of stage kt have returned.
    uint4 fa0[TT], fw0[NB][FT], fa1[TT], fw1[NB][FT];
#define MOE_LOAD_FRAGS(STAGE, KSTEP, FA, FW)                                                  \
    do {                                                                                     \
        const char* st_ = (STAGE);                                                           \
        const int cs_ = ((2 * (KSTEP) + lhalf) ^ swz) * 16;                                  \
        _Pragma("unroll") for (int j = 0; j < TT; ++j) {                                     \
            if constexpr (AKM) FA[j] = kmajor_frag<T, RB>(st_, wt * (BT / 2) + j * 32, (KSTEP), lane); \
            else FA[j] = *reinterpret_cast<const uint4*>(                                    \
                st_ + (wt * (BT / 2) + j * 32 + l32) * kRowBytes + cs_);                     \
        }                                                                                    \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                       \
            _Pragma("unroll") for (int i = 0; i < FT; ++i) {                                 \
                if constexpr (WKM) FW[b][i] = kmajor_frag<T, RB>(st_ + (BT + b * BF) * kRowBytes, \
                                                               wf * (BF / 2) + i * 32, (KSTEP), lane); \
                else FW[b][i] = *reinterpret_cast<const uint4*>(                             \
                    st_ + (BT + b * BF + wf * (BF / 2) + i * 32 + l32) * kRowBytes + cs_);  \
            }                                                                                \
    } while (0)
    // Scheduling hint (bf16, one MFMA instruction per fragment pair): one fragment read after
    // each MFMA, so reads issue while the MFMA pipe is busy rather than as a block between
    // two MFMA runs.  (fp32 makes four MFMA instructions per pair; the hint cost it 1%.)
    constexpr int kMfmaPerStep = NB * FT * TT, kReadsPerStep = TT + NB * FT;
    constexpr bool kHint = kInterleave && sizeof(T) == 2;
#define MOE_INTERLEAVE()                                                                      \
    do {                                                                                     \
        if constexpr (kHint) {                                                               \
            _Pragma("unroll") for (int q_ = 0; q_ < kMfmaPerStep; ++q_) {                    \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           \
                if (q_ < kReadsPerStep) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   \
            }                                                                                \
            if constexpr (kReadsPerStep > kMfmaPerStep)                                      \
                __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerStep - kMfmaPerStep, 0); \
        }                                                                                    \
    } while (0)
#define MOE_MFMAS(FA, FW)                                                                     \
    do {                                                                                     \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                       \
            _Pragma("unroll") for (int i = 0; i < FT; ++i)                                   \
                _Pragma("unroll") for (int j = 0; j < TT; ++j)                               \
                    if (FULL || j < jn) Mfma<T>::mac(acc[b][i][j], FW[b][i], FA[j]);         \
    } while (0)
    __builtin_amdgcn_s_barrier();                                    // barrier 0
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
            if constexpr (!kHint) __builtin_amdgcn_sched_barrier(0);
            MOE_MFMAS(fa0, fw0);
            MOE_INTERLEAVE();
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 2 < KS) {
                MOE_LOAD_FRAGS(st, ks + 2, fa0, fw0);
                if constexpr (!kHint) __builtin_amdgcn_sched_barrier(0);
                MOE_MFMAS(fa1, fw1);
                MOE_INTERLEAVE();
            } else {
                __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (3 << 14));   // lgkmcnt(0)
                __builtin_amdgcn_s_barrier();                        // barrier kt+1
                MOE_LOAD_FRAGS(lds + next * kStageBytes, 0, fa0, fw0);
                if constexpr (!kHint) __builtin_amdgcn_sched_barrier(0);
                MOE_MFMAS(fa1, fw1);
                MOE_INTERLEAVE();
            }
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
#undef MOE_INTERLEAVE

    // ---- epilogue: lane holds one token and, per 32-feature tile, 4 runs of 4 features ----
    // Outputs go through LDS: each wave writes its (BT/2) x (BF/2) block into a region of
    // its own in the MFMA layout, then reads it back by rows so every store instruction
    // writes whole row segments (a direct store from the MFMA layout touches 32 rows per
    // instruction, 8 or 16 bytes each).  The barrier (the loaders' last, after their
    // transfers have landed) frees the ring for this.
    using OutT = typename PickOut<EPI == kEpiLogits, T>::type;   // fp32 partial logits
    constexpr int kRowOut = (BF / 2) * (int)sizeof(OutT);  // bytes of one token's block row
    constexpr int kPitch = kRowOut + 16;                   // +16: rows 16 apart share banks
    constexpr int kCpr = kRowOut / 16;                     // 16-byte chunks per row
    constexpr int kOutChunks = (BT / 2) * kCpr;
    static_assert(4 * (BT / 2) * kPitch <= (kRun ? STG : S * kStageBytes) && kOutChunks % 64 == 0,
                  "staging");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (3 << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (EPI == kEpiLogits && (p.n_feat & 3) != 0) {
        // rows of partial logits not 16-byte aligned: per-element stores (bounds per element)
#pragma unroll
        for (int i = 0; i < FT; ++i) {
#pragma unroll
            for (int j = 0; j < TT; ++j) {
                const int tok = row0 + wt * (BT / 2) + j * 32 + l32;
                if (tok >= row_end) continue;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float r[4] = {acc[0][i][j][4 * g], acc[0][i][j][4 * g + 1],
                                        acc[0][i][j][4 * g + 2], acc[0][i][j][4 * g + 3]};
                    store_logits(static_cast<float*>(p.out), p.n_feat, tok,
                                 f0 + wf * (BF / 2) + i * 32 + 8 * g + 4 * lhalf, r);
                }
            }
        }
        return;
    }
    char* stg = lds + (kRun ? LDS_BYTES - STG : 0) + wave * (BT / 2) * kPitch;
    const int tok0 = row0 + wt * (BT / 2), feat0 = f0 + wf * (BF / 2);
    constexpr int kOuts = EPI == kEpiPair ? 2 : (EPI == kEpiSwiGLUPair ? 3 : 1);
#pragma unroll
    for (int ob = 0; ob < kOuts; ++ob) {
        // (one wave's LDS operations run in order, so a pass's writes come after the
        // previous pass's reads of the same region)
#pragma unroll
        for (int i = 0; i < FT; ++i) {
#pragma unroll
            for (int j = 0; j < TT; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float r[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        if constexpr (EPI == kEpiSwiGLU || EPI == kEpiSwiGLUPair) {
                            if (ob == 0) r[v] = silu(acc[0][i][j][4 * g + v]) * acc[NB - 1][i][j][4 * g + v];
                            else r[v] = acc[ob - 1][i][j][4 * g + v];
                        } else {
                            r[v] = acc[ob][i][j][4 * g + v];
                        }
                    }
                    char* dst = stg + (j * 32 + l32) * kPitch + (i * 32 + 8 * g + 4 * lhalf) * (int)sizeof(OutT);
                    if constexpr (sizeof(OutT) == 4) {
                        *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
                    } else {
                        *reinterpret_cast<uint2*>(dst) =
                            make_uint2(f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16),
                                       f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16));
                    }
                }
            }
        }
        OutT* out = static_cast<OutT*>(ob == 0 ? p.out : (ob == 1 ? p.out2 : p.out3));
#pragma unroll
        for (int k = 0; k < kOutChunks / 64; ++k) {
            const int c = lane + 64 * k;
            const int r = c / kCpr, cc = c - r * kCpr;
            const int tok = tok0 + r, feat = feat0 + cc * (16 / (int)sizeof(OutT));
            const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kPitch + cc * 16);
            if (tok < row_end && feat < p.n_feat)            // n_feat is a multiple of 4 here
                *reinterpret_cast<uint4*>(out + (size_t)tok * p.n_feat + feat) = v;
        }
    }
    // (a run of tiles: this wave's staging reads have returned before the next tile's
    // barrier 0, after which the loaders may refill that region)
    if constexpr (kRun) __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (3 << 14));   // lgkmcnt(0)
}

// Dense product (the gate logits): one expert, rows [0, dense_rows), XCD-contiguous tiles.
template <typename T, int NB, int EPI, int BT, int BF, int S, int RB>
__global__ __launch_bounds__(kThreads, 1) void dense_gemm_kernel(GemmParams<T, NB> p) {
    __shared__ __attribute__((aligned(1024))) char lds[CompTile<BT, BF, NB, S, RB>::kLdsBytes];
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.zero_word) *p.zero_word = 0;
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < p.zero_n; i += gridDim.x * kThreads)
        p.zero_buf[i] = 0;
    // work item L = (split, token tile, feature tile), feature tile fastest so the
    // workgroups an XCD runs at once share their activation rows through its L2
    const int ntt = (p.dense_rows + BT - 1) / BT;
    const int nk_all = (int)((size_t)p.K * sizeof(T) / RB);
    const int splits = (nk_all + p.k_slices - 1) / p.k_slices;
    const int tiles = ntt * p.feat_tiles;
    const int total = tiles * splits;
    const int chunk = (total + 7) >> 3;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= chunk) return;
    const int L = xcd * chunk + local;
    if (L >= total) return;
    const int split = L / tiles, rem = L - split * tiles;
    const int ttile = rem / p.feat_tiles, ftile = rem - ttile * p.feat_tiles;
    const int s0 = split * p.k_slices, nk = min(p.k_slices, nk_all - s0);
    GemmParams<T, NB> q = p;
    q.out = static_cast<float*>(p.out) + (size_t)split * p.dense_rows * p.n_feat;
    const int row_end = min(p.dense_rows, p.act_rows);
    if (row_end - ttile * BT >= BT)
        compute_tile<T, NB, EPI, BT, BF, S, RB, true>(q, lds, 0, ttile * BT, row_end, ftile * BF, s0, nk);
    else
        compute_tile<T, NB, EPI, BT, BF, S, RB, false>(q, lds, 0, ttile * BT, row_end, ftile * BF, s0, nk);
}

// Grouped expert product.  Tiles come from two lists: experts with more than kSmallBTok
// rows (token tiles of BT rows) and experts with at most kSmallBTok rows (one small tile
// each).  XCD x (workgroups x, x + 8, ...) takes a contiguous share of each list and
// interleaves the two evenly in dispatch order, so the small tiles' weight streams overlap
// the large tiles' MFMA work throughout the launch.  Tiles of one large expert go in blocks
// of kGroupTok token tiles; inside a block the feature tile varies slowest, so the ~32
// tiles an XCD runs at once cover about 8 token tiles x 4 feature tiles and share both
// operands through its L2 (measured best among blocks of 2 to 32 on the X-MoE Large
// routing).
template <int BT, int BF, int NB, int S, int RB>
constexpr int expert_lds_bytes() {
    constexpr int a = CompTile<BT, BF, NB, S, RB>::kLdsBytes;
    constexpr int b = kSmallBTok > 0 ? CompTile<(kSmallBTok > 0 ? kSmallBTok : 64), BF, NB,
                                                kSmallStages, RB>::kLdsBytes : 0;
    return a > b ? a : b;
}

// Bytes of LDS a tile's epilogue stages through (4 compute waves x BT/2 token rows of BF/2
// outputs, padded), for the persistent tile loop, which keeps them clear of the next tile's
// first ring slots.
template <typename T, int BT, int BF>
constexpr int expert_stg_bytes() {
    return 4 * (BT / 2) * ((BF / 2) * (int)sizeof(T) + 16);
}

// Whether a tile run fits: the first ring slot of either tile size lies below the staging
// region, so a tile can start its transfers while the previous one stages its outputs
// (bf16 128 x (2 x 128) tiles stage 36 KiB and fill two slots ahead, 128 x 256 tiles stage
// 68 KiB and fill one; fp32 128 x 256 tiles stage 132 KiB and do not fit).
template <typename T, int NB, int BT, int BF, int S, int RB>
constexpr bool expert_run_fits() {
    constexpr int free_bytes = expert_lds_bytes<BT, BF, NB, S, RB>() - expert_stg_bytes<T, BT, BF>();
    constexpr int large = CompTile<BT, BF, NB, S, RB>::kStageBytes;
    constexpr int small = kSmallBTok > 0 ? CompTile<(kSmallBTok > 0 ? kSmallBTok : 64), BF, NB,
                                                    kSmallStages, RB>::kStageBytes : 0;
    return free_bytes >= large && free_bytes >= small;
}

// PST: a persistent grid of one workgroup per CU (8 x W workgroups, W per XCD) walking the
// same per-XCD tile order as the one-tile-per-workgroup grid.  Workgroup i of XCD x starts
// with the XCD's tile i; near the end of each tile one loader lane claims the workgroup's
// next tile, W + (the XCD's counter, incremented), and leaves it in LDS before the tile's
// last barrier, so tiles go to workgroups as they free up, as the hardware dispatcher would
// hand them out.  The loader waves start the next tile's transfers while the compute waves
// store the current one.  Both roles walk the same tile sequence and meet at the same
// barriers; no workgroup waits on another.
template <typename T, int NB, int EPI, int BT, int BF, int S, int RB, bool WKM = false,
          bool PST = false>
__global__ __launch_bounds__(kThreads, 1) void expert_gemm_kernel(GemmParams<T, NB> p) {
    constexpr int kLds = expert_lds_bytes<BT, BF, NB, S, RB>();
    __shared__ __attribute__((aligned(1024))) char lds[kLds];
    constexpr int kL = PST ? kLds : 0;
    constexpr int kStg = PST ? expert_stg_bytes<T, BT, BF>() : 0;
    const int tot_m = p.table_count[0] * p.feat_tiles;
    const int tot_s = p.table_count[1] * p.feat_tiles;
    const int chunk_m = (tot_m + 7) >> 3, chunk_s = (tot_s + 7) >> 3;
    const int xcd = blockIdx.x & 7;
    const int m_x = max(0, min(chunk_m, tot_m - xcd * chunk_m));
    const int s_x = max(0, min(chunk_s, tot_s - xcd * chunk_s));
    const int n_x = m_x + s_x;
    const int nk = (int)((size_t)p.K * sizeof(T) / RB);
    // the j-th tile of this XCD is large-list entry a0 when a1 > a0, else small entry j - a0
    const int w = PST ? (int)(gridDim.x >> 3) : 0;
    auto run = [&](int j, volatile lds_int* note) {
        const int a0 = (int)((long long)j * m_x / n_x), a1 = (int)((long long)(j + 1) * m_x / n_x);
        if (a1 > a0) {
            const int L = xcd * chunk_m + a0;
            const int4 te = p.table[L / p.feat_tiles];
            const int expert = te.x, first = te.y, seg0 = te.z, segn = te.w;
            const int n_e = (segn + BT - 1) / BT;
            const int q = L - p.feat_tiles * first;
            const int gtok = p.gather ? kGroupTokGather : (p.group_tok > 0 ? p.group_tok : kGroupTok);
            const int blk_tiles = gtok * p.feat_tiles;
            const int blk = min(q / blk_tiles, (n_e - 1) / gtok);
            const int width = min(gtok, n_e - blk * gtok);
            const int ql = q - blk * blk_tiles;
            const int ftile = ql / width;
            const int ttile = blk * gtok + (ql - ftile * width);
            const int row0 = seg0 + ttile * BT, row_end = min(seg0 + segn, p.act_rows);
            // keyed on the position (128-row block, feature block of the usual width) rather
            // than the tile index, so tiles of every height sum each output in the same order
            constexpr int kFeatUnit = NB == 2 ? kExpertUpBF : kExpertDownBF;
            const int rblk = ttile * BT / 128, fblk = ftile * BF / kFeatUnit;
            const bool rotate = kRotate && (NB == 2 || kRotateDown) && tot_s > 0;
            const int fstep = min((segn + 127) / 128, 32);
            const int rot = rotate ? ((rblk + fstep * fblk) % kRotPeriod) * nk / kRotPeriod : 0;
            if (row_end - row0 >= BT)
                compute_tile<T, NB, EPI, BT, BF, S, RB, true, false, WKM, false, kL, kStg>(
                    p, lds, expert, row0, row_end, ftile * BF, 0, nk, rot, note, p.claim + xcd, w);
            else
                compute_tile<T, NB, EPI, BT, BF, S, RB, false, false, WKM, false, kL, kStg>(
                    p, lds, expert, row0, row_end, ftile * BF, 0, nk, rot, note, p.claim + xcd, w);
        } else if constexpr (kSmallBTok > 0) {
            constexpr int SB = kSmallBTok > 0 ? kSmallBTok : 64;
            const int Ls = xcd * chunk_s + (j - a0);
            const int4 te = p.stable[Ls / p.feat_tiles];
            const int ftile = Ls - (Ls / p.feat_tiles) * p.feat_tiles;
            const int row0 = te.z, row_end = min(te.z + te.w, p.act_rows);
            if (row_end - row0 >= SB)
                compute_tile<T, NB, EPI, SB, BF, kSmallStages, RB, true, true, WKM, false, kL, kStg>(
                    p, lds, te.x, row0, row_end, ftile * BF, 0, nk, 0, note, p.claim + xcd, w);
            else
                compute_tile<T, NB, EPI, SB, BF, kSmallStages, RB, false, true, WKM, false, kL, kStg>(
                    p, lds, te.x, row0, row_end, ftile * BF, 0, nk, 0, note, p.claim + xcd, w);
        }
    };
    if constexpr (PST) {
        __shared__ int next_tile;
        volatile lds_int* next = (volatile lds_int*)&next_tile;
        const bool claimer = threadIdx.x == 4 * 64;          // lane 0 of the first loader wave
        int j = blockIdx.x >> 3;
        while (j < n_x) {
            run(j, claimer ? next : nullptr);
            asm volatile("" ::: "memory");                    // read after the tile's barriers
            j = *next;                                        // written before the last one
        }
    } else {
        const int j = blockIdx.x >> 3;
        if (j < n_x) run(j, nullptr);
    }
}

// Tile tables, built on the device from the offsets (no host read of the counts).  An
// expert with more than `small` rows gets one `table` entry per btok-row token tile,
// (expert, index of its first entry, first row, rows); an expert with 1..small rows gets
// one `stable` entry (expert, its index, first row, rows).  count[0], count[1] = entries.
// Segments are clipped to [0, rows) so malformed offsets can never address past the
// buffers, and no more than cap (table) or E (stable) entries are written.  The persistent
// grid's tile counters (count[kClaimUp ..]) are cleared.  Single
// workgroup; E <= 1024.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* offsets, int E, int rows,
                                                          int btok, int small, int cap,
                                                          int4* table, int4* stable, int* count) {
    __shared__ long long scan[2][1024];
    const int e = threadIdx.x;
    int beg = 0, cnt = 0, nm = 0, ns = 0;
    if (e < E) {
        beg = min(max(offsets[e], 0), rows);
        cnt = max(min(offsets[e + 1], rows) - beg, 0);
        if (cnt > small) nm = (cnt + btok - 1) / btok;
        else if (cnt > 0) ns = 1;
    }
    // inclusive Hillis-Steele scan of (nm, ns) packed in 64 bits
    int cur = 0;
    scan[0][e] = (long long)nm | ((long long)ns << 32);
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const long long v = scan[cur][e] + (e >= d ? scan[cur][e - d] : 0);
        scan[cur ^ 1][e] = v;
        cur ^= 1;
        __syncthreads();
    }
    const long long incl = scan[cur][e];
    const int first_m = (int)(incl & 0xffffffff) - nm;
    const int first_s = (int)(incl >> 32) - ns;
    for (int j = 0; j < nm && first_m + j < cap; ++j) table[first_m + j] = make_int4(e, first_m, beg, cnt);
    if (ns) stable[first_s] = make_int4(e, first_s, beg, cnt);
    if (e == 1023) {
        count[0] = min((int)(incl & 0xffffffff), cap);
        count[1] = (int)(incl >> 32);
    }
    if (e < kClaimWords) count[kClaimUp + e] = 0;
}

template <typename T, int NB, int EPI, int BT, int BF, int S, int RB>
hipError_t launch_dense(const GemmParams<T, NB>& p, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    grid = (grid + 7) & ~7;
    hipLaunchKernelGGL((dense_gemm_kernel<T, NB, EPI, BT, BF, S, RB>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// The grid covers the most (token tile, feature tile) items the two lists can hold
// together, max_items = tiles_cap x feature tiles: an expert adds at most one tile beyond
// its rows / BT, whichever list it is in.  XCD x runs ceil(m / 8) + ceil(s / 8) items of
// the m and s that exist, at most max_items / 8 + 2.  A persistent grid (bf16, see
// kPersist) has one workgroup per CU, or fewer when the upper bound is lower.
template <typename T, int NB, int EPI, int BT, int BF, int S, int RB, bool WKM = false>
hipError_t launch_expert(const GemmParams<T, NB>& p, int max_items, hipStream_t s) {
    int grid = 8 * ((max_items + 7) / 8 + 2);
    if (grid <= 0) return hipSuccess;
    if constexpr (kPersist && sizeof(T) == 2 && expert_run_fits<T, NB, BT, BF, S, RB>()) {
        if (p.claim == nullptr) return hipErrorInvalidValue;
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        grid = min(grid, 8 * max(cus / 8, 1));
        hipLaunchKernelGGL((expert_gemm_kernel<T, NB, EPI, BT, BF, S, RB, WKM, true>), dim3(grid),
                           dim3(kThreads), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((expert_gemm_kernel<T, NB, EPI, BT, BF, S, RB, WKM>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// Gate logits as K splits: (token tile, expert tile, K split) work items, each split's
// fp32 partial sums [T][E] written to its own slice of `partials`; the top-k kernel adds
// them in split order and adds the bias.  A tile covers 64 tokens and up to 256 experts,
// so x and Wg cross the L2 -> CU path few times (64 x 64 tiles moved 7.5x the operand
// bytes at X-MoE Large); splits (at most 8) bring the work items to about kGateItems.
#ifndef MOE_GATE_ITEMS
#define MOE_GATE_ITEMS 256
#endif
#ifndef MOE_GATE_BF_MAX
#define MOE_GATE_BF_MAX 256
#endif
#ifndef MOE_GATE_BT
#define MOE_GATE_BT 64
#endif
constexpr int kGateBT = MOE_GATE_BT, kGateRB = 128, kGateItems = MOE_GATE_ITEMS;

__host__ __device__ inline int gate_bf(int E) {
    return E <= 64 || MOE_GATE_BF_MAX == 64 ? 64 : (E <= 128 || MOE_GATE_BF_MAX == 128 ? 128 : 256);
}

__host__ __device__ inline int gate_k_slices(int dt, int T, int H, int E) {
    const int nk = H * (dt == 0 ? 4 : 2) / kGateRB;
    const int bf = gate_bf(E);
    const int tiles = ((T + kGateBT - 1) / kGateBT) * ((E + bf - 1) / bf);
    int splits = kGateItems / (tiles > 0 ? tiles : 1);
    splits = splits < 1 ? 1 : (splits > 8 ? 8 : splits);
    splits = splits > nk ? nk : splits;
    return (nk + splits - 1) / splits;              // k-slices per split
}

template <typename T, int BF, int S>
hipError_t gate_logits_bf(int dt, int T_, int H, int E, const void* x, const void* wg,
                          float* partials, int* zero_word, int* zero_buf, int zero_n,
                          hipStream_t s) {
    GemmParams<T, 1> p{};
    p.zero_word = zero_word;
    p.zero_buf = zero_buf;
    p.zero_n = zero_buf ? zero_n : 0;
    p.act = static_cast<const T*>(x);
    p.act_rows = T_;
    p.K = H;
    p.w[0] = static_cast<const T*>(wg);
    p.w_stride = 0;
    p.n_feat = E;
    p.feat_tiles = (E + BF - 1) / BF;
    p.dense_rows = T_;
    p.out = partials;
    p.k_slices = gate_k_slices(dt, T_, H, E);
    const int nk = H * (int)sizeof(T) / kGateRB;
    const int splits = (nk + p.k_slices - 1) / p.k_slices;
    const int grid = ((T_ + kGateBT - 1) / kGateBT) * p.feat_tiles * splits;
    return launch_dense<T, 1, kEpiLogits, kGateBT, BF, S, kGateRB>(p, grid, s);
}

template <typename T>
hipError_t gate_logits_t(int dt, int T_, int H, int E, const void* x, const void* wg,
                         float* partials, int* zero_word, int* zero_buf, int zero_n,
                         hipStream_t s) {
    switch (gate_bf(E)) {
        case 64: return gate_logits_bf<T, 64, 4>(dt, T_, H, E, x, wg, partials, zero_word, zero_buf, zero_n, s);
        case 128: return gate_logits_bf<T, 128, 4>(dt, T_, H, E, x, wg, partials, zero_word, zero_buf, zero_n, s);
        default: return gate_logits_bf<T, 256, 3>(dt, T_, H, E, x, wg, partials, zero_word, zero_buf, zero_n, s);
    }
}

__host__ __device__ inline long long tiles_cap(long long N, int E, int btok = kExpertBTok) {
    return (N + btok - 1) / btok + (E < N ? E : N);
}

// Small problems: when the usual tiles would not give every CU one (an upper bound on the
// up product's 128-token tiles, (ceil(N / 128) + min(E, N)) x ceil(F / 128), below the 256
// CUs), the forward's expert products use 64-token tiles with narrower feature tiles (up 64
// features per operand, down 128), so the few tiles there are spread over 4 to 8 times as
// many SIMDs.  A 128-token tile runs its MFMAs one after another on four SIMDs; with fp32
// (4096 flop per 64-cycle MFMA) a 128 x 256 x 256 tile alone takes about 30 us, which set
// the Tiny layer's time.  (A row-count threshold of 8192 also sent a dense 4096 x 7168 x
// 2048 up product to the small tiles: 335 us against 224 us on the usual ones.)
constexpr int kSmallProblemTiles = 256;
constexpr int kSmallProblemBTok = 64;

inline int fwd_btok(long long N, int E, int F) {
    const long long tiles = ((N + kExpertBTok - 1) / kExpertBTok + (E < N ? E : N)) *
                            ((F + kExpertUpBF - 1) / kExpertUpBF);
    return tiles < kSmallProblemTiles ? kSmallProblemBTok : kExpertBTok;
}

inline TileTables carve_tables(void* ws, long long N, int E, int btok = kExpertBTok) {
    TileTables t;
    char* w = static_cast<char*>(ws);
    t.count = reinterpret_cast<int*>(w);
    t.cap = (int)tiles_cap(N, E, btok);
    t.table = reinterpret_cast<int4*>(w + 256);
    t.stable = t.table + t.cap;
    t.btok = btok;
    t.small = kSmallBTok;
    return t;
}

hipError_t build_tables(const TileTables& tl, const int32_t* offsets, int E, int N, hipStream_t s) {
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, offsets, E, N, tl.btok,
                       tl.small, tl.cap, tl.table, tl.stable, tl.count);
    return hipGetLastError();
}

// The forward's two products on tiles of BT tokens (up: UP_BF features per operand, down:
// DN_BF features), over tables of BT-row token tiles.
template <typename T, int BT, int UP_BF, int DN_BF>
hipError_t grouped_tiles(int N, int E, int H, int F, const void* xd, const int32_t* gather,
                         int src_rows, const TileTables& tl, const void* w1, const void* w3,
                         const void* w2, void* h, void* y, void* a, void* g, hipStream_t s);

template <typename T>
hipError_t grouped_t(int N, int E, int H, int F, const void* xd, const int32_t* gather,
                     int src_rows, const int32_t* offsets, const void* w1, const void* w3,
                     const void* w2, void* h, void* y, void* a, void* g, void* ws,
                     bool tables_ready, hipStream_t s) {
    const TileTables tl = carve_tables(ws, N, E, fwd_btok(N, E, F));
    hipError_t err = tables_ready ? hipSuccess : build_tables(tl, offsets, E, N, s);
    if (err != hipSuccess) return err;
    if (tl.btok == kSmallProblemBTok)
        return grouped_tiles<T, kSmallProblemBTok, 64, 128>(N, E, H, F, xd, gather, src_rows, tl,
                                                            w1, w3, w2, h, y, a, g, s);
    return grouped_tiles<T, kExpertBTok, kExpertUpBF, kExpertDownBF>(N, E, H, F, xd, gather,
                                                                     src_rows, tl, w1, w3, w2,
                                                                     h, y, a, g, s);
}

template <typename T, int BT, int UP_BF, int DN_BF>
hipError_t grouped_tiles(int N, int E, int H, int F, const void* xd, const int32_t* gather,
                         int src_rows, const TileTables& tl, const void* w1, const void* w3,
                         const void* w2, void* h, void* y, void* a, void* g, hipStream_t s) {
    hipError_t err = hipSuccess;
    constexpr int STAGES = kExpertStages, RB = kExpertRowBytes;
    GemmParams<T, 2> up{};
    up.act = static_cast<const T*>(xd);
    up.act_rows = N;
    up.gather = gather;
    up.src_rows = src_rows;
    up.K = H;
    up.w[0] = static_cast<const T*>(w1);
    up.w[1] = static_cast<const T*>(w3);
    up.w_stride = (long long)F * H;
    up.n_feat = F;
    up.feat_tiles = (F + UP_BF - 1) / UP_BF;
    up.table = tl.table;
    up.stable = tl.stable;
    up.table_count = tl.count;
    up.claim = tl.count + kClaimUp;
    up.out = h;
    up.out2 = a;
    up.out3 = g;
    if (a != nullptr && g != nullptr)
        err = launch_expert<T, 2, kEpiSwiGLUPair, BT, UP_BF, STAGES, RB>(
            up, tl.cap * up.feat_tiles, s);
    else
        err = launch_expert<T, 2, kEpiSwiGLU, BT, UP_BF, STAGES, RB>(
            up, tl.cap * up.feat_tiles, s);
    if (err != hipSuccess || w2 == nullptr) return err;      // up product only

    GemmParams<T, 1> dn{};
    dn.act = static_cast<const T*>(h);
    dn.act_rows = N;
    dn.K = F;
    dn.w[0] = static_cast<const T*>(w2);
    dn.w_stride = (long long)H * F;
    dn.n_feat = H;
    dn.feat_tiles = (H + DN_BF - 1) / DN_BF;
    dn.table = tl.table;
    dn.stable = tl.stable;
    dn.table_count = tl.count;
    dn.claim = tl.count + kClaimDown;
    dn.group_tok = kGroupTokDown;
    dn.out = y;
    return launch_expert<T, 1, kEpiStore, BT, DN_BF, STAGES, RB>(
        dn, tl.cap * dn.feat_tiles, s);
}

// ---- backward products ----
// Grouped product over the expert segments with K-major weights: out[p][n] = sum_k act[p][k]
// * W_e[k][n] for the rows p of expert e, where row k of W_e is row k of w_lo[e] for k <
// k_split and row k - k_split of w_hi[e] from there on (w_ld elements per row, w_stride per
// expert).  The weights are read as stored: no transposed copies.  The forward's tile table
// and the 128 x 256 tile.
template <typename T>
hipError_t grouped_kmajor_t(int N, int E, int K, int n_feat, const void* act,
                            const int32_t* offsets, const void* w_lo, const void* w_hi,
                            int k_split, long long w_ld, long long w_stride, void* out, void* ws,
                            hipStream_t s) {
    constexpr int BT = kExpertBTok, BF = kExpertDownBF, STAGES = kExpertStages,
                  RB = kExpertRowBytes, KPS = RB / (int)sizeof(T);
    const TileTables tl = carve_tables(ws, N, E);
    hipError_t err = build_tables(tl, offsets, E, N, s);
    if (err != hipSuccess) return err;
    GemmParams<T, 1> q{};
    q.act = static_cast<const T*>(act);
    q.act_rows = N;
    q.K = K;
    q.w[0] = static_cast<const T*>(w_lo);
    q.w_stride = w_stride;
    q.w_ld = w_ld;
    q.k_rows = K;                // every row of the K range exists: nothing reads zero16
    q.w_k2 = 1 << 30;
    if (w_hi != nullptr) {
        // from k-slice w_k2 on, addresses computed from w_lo land in w_hi
        const long long wslice = (long long)KPS * w_ld * (long long)sizeof(T);
        q.w_k2 = k_split / KPS;
        q.w_k2_adj = (long long)(reinterpret_cast<uintptr_t>(w_hi) - reinterpret_cast<uintptr_t>(w_lo)) -
                     q.w_k2 * wslice;
    }
    q.n_feat = n_feat;
    q.feat_tiles = (n_feat + BF - 1) / BF;
    q.table = tl.table;
    q.stable = tl.stable;
    q.table_count = tl.count;
    q.claim = tl.count + kClaimUp;
    q.out = out;
    return launch_expert<T, 1, kEpiStore, BT, BF, STAGES, RB, true>(q, tl.cap * q.feat_tiles, s);
}

// The up product with both results stored: a = act.W1[e]^T, g = act.W3[e]^T (rows gathered
// through `gather` when it is not NULL, as in the forward).
template <typename T>
hipError_t grouped_pair_t(int N, int E, int H, int F, const void* act, const int32_t* gather,
                          int src_rows, const int32_t* offsets, const void* w1, const void* w3,
                          void* a, void* g, void* ws, hipStream_t s) {
    constexpr int BT = kExpertBTok, BF = kExpertUpBF, STAGES = kExpertStages,
                  RB = kExpertRowBytes;
    const TileTables tl = carve_tables(ws, N, E);
    hipError_t err = build_tables(tl, offsets, E, N, s);
    if (err != hipSuccess) return err;
    GemmParams<T, 2> q{};
    q.act = static_cast<const T*>(act);
    q.act_rows = N;
    q.gather = gather;
    q.src_rows = src_rows;
    q.K = H;
    q.w[0] = static_cast<const T*>(w1);
    q.w[1] = static_cast<const T*>(w3);
    q.w_stride = (long long)F * H;
    q.n_feat = F;
    q.feat_tiles = (F + BF - 1) / BF;
    q.table = tl.table;
    q.stable = tl.stable;
    q.table_count = tl.count;
    q.claim = tl.count + kClaimUp;
    q.out = a;
    q.out2 = g;
    return launch_expert<T, 2, kEpiPair, BT, BF, STAGES, RB>(q, tl.cap * q.feat_tiles, s);
}

// Weight gradients, out[e][m][f] = sum over expert e's rows k of act[k][m] * w[k][f], in two
// layouts.  KM: act [N][a_ld] and w [N][w_ld] as the forward and backward wrote them (row k
// of expert e in [kofs[e], kofs[e+1]), here the expert offsets), both read K-major; the
// last k-slice's rows past the expert's end read zeros.  Otherwise act [M][Ktot] and
// w [n_feat][Ktot] hold every expert's rows transposed into a column block starting at
// kofs[e] (a multiple of 64, zero padded to a multiple of 64).  Work item (expert, m tile,
// f tile) over every expert or over the experts listed in elist[0, *nlist); an expert with
// no rows gets a zero gradient.
template <typename T, int BT, int BF, int S, int RB, bool KM>
__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(GemmParams<T, 1> p,
                                                            const int32_t* kofs, int E, int M,
                                                            const int32_t* elist,
                                                            const int32_t* nlist) {
    __shared__ __attribute__((aligned(1024))) char lds[CompTile<BT, BF, 1, S, RB>::kLdsBytes];
    const int mtiles = (M + BT - 1) / BT;
    // Each XCD takes an equal contiguous share (per_x tiles) of every expert's tiles, expert
    // after expert, so the XCDs get equal work however unequal the experts' K ranges are
    // (contiguous chunks of the whole item list gave one XCD 1.9x the mean work on the
    // X-MoE Large routing), and the tiles an XCD runs at once share operand panels.
    const int per = mtiles * p.feat_tiles, per_x = (per + 7) / 8;
    const int xcd = blockIdx.x & 7;
    const long long local = blockIdx.x >> 3;
    if (local >= (long long)per_x * (elist ? *nlist : E)) return;
    const int i = (int)(local / per_x);
    const int rem = xcd * per_x + (int)(local - (long long)i * per_x);
    if (rem >= per) return;
    const int e = elist ? elist[i] : i;             // with a list, its i-th expert
    const int mt = rem / p.feat_tiles, ft = rem - mt * p.feat_tiles;
    GemmParams<T, 1> q = p;
    q.out = static_cast<T*>(p.out) + (size_t)e * M * p.n_feat;
    const int k0 = kofs[e], k1 = kofs[e + 1];
    constexpr int KPS = RB / (int)sizeof(T);
    const int nk = KM ? (k1 - k0 + KPS - 1) / KPS : (int)((size_t)(k1 - k0) * sizeof(T) / RB);
    const int row0 = mt * BT;
    if (nk <= 0) {                                  // whole workgroup: no barrier is pending
        constexpr int kPer = 16 / (int)sizeof(T);
        uint4* o = static_cast<uint4*>(q.out);
        const int fcs = BF / kPer, fc0 = ft * BF / kPer, fcn = p.n_feat / kPer;
        for (int i = threadIdx.x; i < BT * fcs; i += kThreads) {
            const int r = row0 + i / fcs, fc = fc0 + i % fcs;
            if (r < M && fc < fcn) o[(size_t)r * fcn + fc] = make_uint4(0, 0, 0, 0);
        }
        return;
    }
    if constexpr (KM) {
        q.act = p.act + (size_t)k0 * p.a_ld;
        q.w[0] = p.w[0] + (size_t)k0 * p.w_ld;
        q.k_rows = k1 - k0;
        if (row0 + BT <= M)
            compute_tile<T, 1, kEpiStore, BT, BF, S, RB, true, false, true, true>(q, lds, 0, row0, M, ft * BF, 0, nk);
        else
            compute_tile<T, 1, kEpiStore, BT, BF, S, RB, false, false, true, true>(q, lds, 0, row0, M, ft * BF, 0, nk);
    } else {
        const int s0 = (int)((size_t)k0 * sizeof(T) / RB);
        if (row0 + BT <= M)
            compute_tile<T, 1, kEpiStore, BT, BF, S, RB, true>(q, lds, 0, row0, M, ft * BF, s0, nk);
        else
            compute_tile<T, 1, kEpiStore, BT, BF, S, RB, false>(q, lds, 0, row0, M, ft * BF, s0, nk);
    }
}

template <typename T>
hipError_t wgrad_t(int E, int M, int n_feat, int ktot, const void* act, const void* w,
                   const int32_t* kofs, const int32_t* elist, const int32_t* nlist, void* out,
                   hipStream_t s) {
    constexpr int BT = kExpertBTok, BF = kExpertDownBF, STAGES = kExpertStages,
                  RB = kExpertRowBytes;
    GemmParams<T, 1> q{};
    q.act = static_cast<const T*>(act);
    q.act_rows = M;
    q.K = ktot;
    q.w[0] = static_cast<const T*>(w);
    q.w_stride = 0;
    q.n_feat = n_feat;
    q.feat_tiles = (n_feat + BF - 1) / BF;
    q.out = out;
    const long long per_x = ((long long)((M + BT - 1) / BT) * q.feat_tiles + 7) / 8;
    const long long grid = 8 * per_x * E;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((wgrad_kernel<T, BT, BF, STAGES, RB, false>), dim3((unsigned)grid), dim3(kThreads),
                       0, s, q, kofs, E, M, elist, nlist);
    return hipGetLastError();
}

template <typename T>
hipError_t wgrad_rows_t(int E, int M, int n_feat, const void* act, long long a_ld, const void* w,
                        long long w_ld, const int32_t* offsets, const int32_t* elist,
                        const int32_t* nlist, const void* zero16, void* out, hipStream_t s) {
    constexpr int BT = kExpertBTok, BF = kExpertDownBF, STAGES = kExpertStages,
                  RB = kExpertRowBytes;
    GemmParams<T, 1> q{};
    q.act = static_cast<const T*>(act);
    q.act_rows = M;
    q.a_ld = a_ld;
    q.w[0] = static_cast<const T*>(w);
    q.w_ld = w_ld;
    q.w_k2 = 1 << 30;
    q.zero16 = zero16;
    q.n_feat = n_feat;
    q.feat_tiles = (n_feat + BF - 1) / BF;
    q.out = out;
    const long long per_x = ((long long)((M + BT - 1) / BT) * q.feat_tiles + 7) / 8;
    const long long grid = 8 * per_x * E;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((wgrad_kernel<T, BT, BF, STAGES, RB, true>), dim3((unsigned)grid), dim3(kThreads),
                       0, s, q, offsets, E, M, elist, nlist);
    return hipGetLastError();
}

}  // namespace

size_t gemm_ws_bytes(long long N, int E) {
    return 256 + (size_t)(tiles_cap(N, E, kSmallProblemBTok) + E) * sizeof(int4);
}

TileTables gemm_tables(void* ws, long long N, int E, int F) {
    return carve_tables(ws, N, E, fwd_btok(N, E, F));
}

int gate_splits(int dt, int T, int H, int E) {
    const int nk = H * (dt == 0 ? 4 : 2) / kGateRB;
    const int per = gate_k_slices(dt, T, H, E);
    return (nk + per - 1) / per;
}

hipError_t launch_gate_logits(int dt, int T, int H, int E, const void* x, const void* wg,
                              float* partials, int* zero_word, int* zero_buf, int zero_n,
                              hipStream_t s) {
    if (T == 0) return hipSuccess;
    return dt == 0 ? gate_logits_t<float>(dt, T, H, E, x, wg, partials, zero_word, zero_buf, zero_n, s)
                   : gate_logits_t<bf16_t>(dt, T, H, E, x, wg, partials, zero_word, zero_buf, zero_n, s);
}

hipError_t launch_grouped_gemm(int dt, int N, int E, int H, int F, const void* xd,
                               const int32_t* offsets, const void* w1, const void* w3,
                               const void* w2, void* h, void* y, void* ws, hipStream_t s,
                               void* a, void* g, bool tables_ready) {
    if (N == 0) return hipSuccess;
    return dt == 0 ? grouped_t<float>(N, E, H, F, xd, nullptr, 0, offsets, w1, w3, w2, h, y, a, g, ws, tables_ready, s)
                   : grouped_t<bf16_t>(N, E, H, F, xd, nullptr, 0, offsets, w1, w3, w2, h, y, a, g, ws, tables_ready, s);
}

hipError_t launch_grouped_gemm_gather(int dt, int N, int E, int H, int F, const void* x, int T,
                                      const int32_t* token_ids, const int32_t* offsets,
                                      const void* w1, const void* w3, const void* w2, void* h,
                                      void* y, void* ws, hipStream_t s, void* a, void* g,
                                      bool tables_ready) {
    if (N == 0) return hipSuccess;
    return dt == 0 ? grouped_t<float>(N, E, H, F, x, token_ids, T, offsets, w1, w3, w2, h, y, a, g, ws, tables_ready, s)
                   : grouped_t<bf16_t>(N, E, H, F, x, token_ids, T, offsets, w1, w3, w2, h, y, a, g, ws, tables_ready, s);
}

hipError_t launch_grouped_kmajor(int dt, int N, int E, int K, int n_feat, const void* act,
                                 const int32_t* offsets, const void* w_lo, const void* w_hi,
                                 int k_split, long long w_ld, long long w_stride, void* out,
                                 void* ws, hipStream_t s) {
    if (N == 0) return hipSuccess;
    return dt == 0 ? grouped_kmajor_t<float>(N, E, K, n_feat, act, offsets, w_lo, w_hi, k_split, w_ld, w_stride, out, ws, s)
                   : grouped_kmajor_t<bf16_t>(N, E, K, n_feat, act, offsets, w_lo, w_hi, k_split, w_ld, w_stride, out, ws, s);
}

hipError_t launch_grouped_pair(int dt, int N, int E, int H, int F, const void* act,
                               const int32_t* gather, int src_rows, const int32_t* offsets,
                               const void* w1, const void* w3, void* a, void* g, void* ws,
                               hipStream_t s) {
    if (N == 0) return hipSuccess;
    return dt == 0 ? grouped_pair_t<float>(N, E, H, F, act, gather, src_rows, offsets, w1, w3, a, g, ws, s)
                   : grouped_pair_t<bf16_t>(N, E, H, F, act, gather, src_rows, offsets, w1, w3, a, g, ws, s);
}

hipError_t launch_wgrad_rows(int dt, int E, int M, int n_feat, const void* act, long long a_ld,
                             const void* w, long long w_ld, const int32_t* offsets,
                             const int32_t* elist, const int32_t* nlist, const void* zero16,
                             void* out, hipStream_t s) {
    return dt == 0 ? wgrad_rows_t<float>(E, M, n_feat, act, a_ld, w, w_ld, offsets, elist, nlist, zero16, out, s)
                   : wgrad_rows_t<bf16_t>(E, M, n_feat, act, a_ld, w, w_ld, offsets, elist, nlist, zero16, out, s);
}

hipError_t launch_wgrad(int dt, int E, int M, int n_feat, int ktot, const void* act,
                        const void* w, const int32_t* kofs, const int32_t* elist,
                        const int32_t* nlist, void* out, hipStream_t s) {
    return dt == 0 ? wgrad_t<float>(E, M, n_feat, ktot, act, w, kofs, elist, nlist, out, s)
                   : wgrad_t<bf16_t>(E, M, n_feat, ktot, act, w, kofs, elist, nlist, out, s);
}

}  // namespace moe
