// backward.hip -- the layer backward: gradients of the loss with dL/dout given, the expert
// picks held fixed (selection is piecewise constant in the logits).
//
// The pages present the layer as part of a training system (X-MoE review, section 三,
// 训练流程: the forward is followed by the backward and the weight update; FlashDMoE blog,
// section 10: training as future work) without backward formulas; the gradients here are
// the derivatives of the forward of this library:
//   combine:  dy[p] = w[t][j] dout[t],  dw[t][j] = <dout[t], y[p]>              (p = dest_pos[t][j])
//   experts:  dh = dy W2[e],  da = dh g silu'(a),  dg = dh silu(a),  dxd = da W1[e] + dg W3[e]
//             dW2[e] = dy_e^T h_e,  dW1[e] = da_e^T xd_e,  dW3[e] = dg_e^T xd_e
//   dispatch: dx[t] = sum_j dxd[p]
//   gate:     dl from dw through the routing weights of the picked logits (softmax over the
//             picks, or normalised sigmoids), dx[t] += sum_j dl_j Wg[e_j],
//             dWg = DL^T x, dbias = column sums of DL (DL [T][E] holds dl at the picks)
// Every product runs on the tile GEMM of gemm.hip, reading its operands as stored: dh and
// dxd take the weights K-major, and each expert's weight gradient is one GEMM over its own
// rows with both row-major operands read K-major (the transpose happens in the LDS
// fragment read; the last k-slice reads zeros past the expert's rows).  Only dWg reads x
// and the logit gradients transposed into a column block.  All accumulation is fp32;
// every gradient tensor is rounded once to its storage type (dbias, dw and dl stay fp32).
// Deterministic: no atomics.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTile = 64;   // transpose tile (elements per side)

inline int row_threads(int chunks) { return chunks >= 1024 ? 1024 : ((chunks + 63) / 64) * 64; }

template <typename T>
__device__ __forceinline__ T store_f(float v);
template <>
__device__ __forceinline__ float store_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t store_f<bf16_t>(float v) { return bf16_t{f32_to_bf16(v)}; }

// Sum of a per-thread value over the block, in a fixed order (wave butterflies, then the
// waves in order); the result is valid in thread 0.  `red` holds one float per wave.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum_f32(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float s = 0.0f;
    if (threadIdx.x == 0)
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
    __syncthreads();
    return s;
}

// ---- combine backward: one workgroup per token, one thread per 16-byte chunk ----
// dy[p] = w[t][j] * dout[t] (rounded once) and dw[t][j] = <dout[t], y[p]> (fp32, chunk order
// per thread, then the fixed block reduction).  Slots go 8 at a time.
template <typename T>
__global__ __launch_bounds__(1024) void combine_bwd_kernel(const uint4* __restrict__ dout,
                                                           const uint4* __restrict__ y,
                                                           const int32_t* __restrict__ dest_pos,
                                                           const float* __restrict__ tw,
                                                           uint4* __restrict__ dy,
                                                           float* __restrict__ dw, int k,
                                                           int N, int chunks) {
    constexpr int P = 16 / sizeof(T) == 8 ? 8 : 4;
    __shared__ float red[16][8];
    const int t = blockIdx.x;
    for (int j0 = 0; j0 < k; j0 += 8) {
        float part[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) part[g] = 0.0f;
        for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
            float d[P];
            unpack16(dout[(size_t)t * chunks + c], d, T{});
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const int j = j0 + g;
                if (j >= k) break;
                const int p = dest_pos[(size_t)t * k + j];
                if (p < 0 || p >= N) continue;          // an invalid routing entry
                float v[P], o[P];
                unpack16(y[(size_t)p * chunks + c], v, T{});
                const float w = tw[(size_t)t * k + j];
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    part[g] = fmaf(d[i], v[i], part[g]);
                    o[i] = w * d[i];
                }
                dy[(size_t)p * chunks + c] = pack16(o, T{});
            }
        }
        const int wv = threadIdx.x >> 6;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const float s = wave_sum_f32(part[g]);
            if ((threadIdx.x & 63) == 0) red[wv][g] = s;
        }
        __syncthreads();
        if (threadIdx.x < 8 && j0 + (int)threadIdx.x < k) {
            float s = 0.0f;
            for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i][threadIdx.x];
            dw[(size_t)t * k + j0 + threadIdx.x] = s;
        }
        __syncthreads();
    }
}

// ---- token gradient: dx[t] = sum_j dxd[dest_pos[t][j]] + sum_j dl[t][j] * Wg[e_tj] ----
template <typename T>
__global__ __launch_bounds__(1024) void token_grad_kernel(const uint4* __restrict__ dxd,
                                                          const int32_t* __restrict__ dest_pos,
                                                          const float* __restrict__ dl,
                                                          const int32_t* __restrict__ te,
                                                          const uint4* __restrict__ wg,
                                                          uint4* __restrict__ dx, int k,
                                                          int N, int chunks) {
    constexpr int P = 16 / sizeof(T) == 8 ? 8 : 4;
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        float acc[P];
#pragma unroll
        for (int i = 0; i < P; ++i) acc[i] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int p = dest_pos[(size_t)t * k + j];
            if (p < 0 || p >= N) continue;              // an invalid routing entry
            float v[P];
            unpack16(dxd[(size_t)p * chunks + c], v, T{});
#pragma unroll
            for (int i = 0; i < P; ++i) acc[i] += v[i];
        }
        for (int j = 0; j < k; ++j) {
            float v[P];
            unpack16(wg[(size_t)te[(size_t)t * k + j] * chunks + c], v, T{});
            const float d = dl[(size_t)t * k + j];
#pragma unroll
            for (int i = 0; i < P; ++i) acc[i] = fmaf(d, v[i], acc[i]);
        }
        dx[(size_t)t * chunks + c] = pack16(acc, T{});
    }
}

// ---- gate: logit gradients of the picks, one wave per token ----
// Picked logits are recomputed (x[t] . Wg[e] + bias, fp32, 16-byte chunks per lane), lane
// j < k holds pick j.
template <typename T>
__global__ __launch_bounds__(256) void gate_dl_kernel(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ wg,
                                                      const float* __restrict__ bias,
                                                      const int32_t* __restrict__ te,
                                                      const float* __restrict__ dw, int routing,
                                                      int T_, int chunks, int k,
                                                      float* __restrict__ dl) {
    constexpr int P = 16 / sizeof(T) == 8 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T_) return;                            // whole wave
    float mine = 0.0f;
    for (int j = 0; j < k; ++j) {
        const int e = te[(size_t)t * k + j];
        float s = 0.0f;
        for (int c = lane; c < chunks; c += 64) {
            float a[P], b[P];
            unpack16(x[(size_t)t * chunks + c], a, T{});
            unpack16(wg[(size_t)e * chunks + c], b, T{});
#pragma unroll
            for (int i = 0; i < P; ++i) s = fmaf(a[i], b[i], s);
        }
        s = wave_sum_f32(s);
        if (bias) s += bias[e];
        if (lane == j) mine = s;
    }
    const bool act = lane < k;
    float w, sg = 0.0f, S = 0.0f;
    if (routing == 0) {
        float m = act ? mine : -INFINITY;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float ex = act ? __expf(mine - m) : 0.0f;
        w = ex / wave_sum_f32(ex);
    } else {
        sg = act ? 1.0f / (1.0f + __expf(-mine)) : 0.0f;
        S = wave_sum_f32(sg);
        w = sg / S;
    }
    const float dwj = act ? dw[(size_t)t * k + lane] : 0.0f;
    const float wdw = wave_sum_f32(act ? w * dwj : 0.0f);
    if (act) {
        const float r = dwj - wdw;
        dl[(size_t)t * k + lane] = routing == 0 ? w * r : r / S * sg * (1.0f - sg);
    }
}

// DL^T [E][ld]: dl at (e_tj, t), zero elsewhere and in the padding columns t >= T.
template <typename T>
__global__ __launch_bounds__(256) void gate_dlt_kernel(const float* __restrict__ dl,
                                                       const int32_t* __restrict__ te, int T_,
                                                       int E, int k, int ld, T* __restrict__ dlt) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)E * ld) return;
    const int e = (int)(i / ld), t = (int)(i - (long long)e * ld);
    float v = 0.0f;
    if (t < T_)
        for (int j = 0; j < k; ++j)
            if (te[(size_t)t * k + j] == e) v = dl[(size_t)t * k + j];
    dlt[i] = store_f<T>(v);
}

// dbias[e] = sum of dl over expert e's buffer rows (ascending row order per thread, then the
// fixed block reduction); one workgroup per expert.
__global__ __launch_bounds__(256) void gate_dbias_kernel(const float* __restrict__ dl,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ token_ids,
                                                         const int32_t* __restrict__ dest_pos,
                                                         int k, float* __restrict__ dbias) {
    __shared__ float red[4];
    const int e = blockIdx.x;
    float s = 0.0f;
    for (int p = offsets[e] + threadIdx.x; p < offsets[e + 1]; p += 256) {
        const int t = token_ids[p];
        for (int j = 0; j < k; ++j)
            if (dest_pos[(size_t)t * k + j] == p) s += dl[(size_t)t * k + j];
    }
    s = block_sum(s, red);
    if (threadIdx.x == 0) dbias[e] = s;
}

// ---- SwiGLU backward, elementwise over 16-byte chunks: dag[p] = (da[0..F), dg[0..F)) ----
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint4* __restrict__ dh,
                                                         const uint4* __restrict__ a,
                                                         const uint4* __restrict__ g,
                                                         long long nchunks, int fchunks,
                                                         uint4* __restrict__ dag) {
    constexpr int P = 16 / sizeof(T) == 8 ? 8 : 4;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= nchunks) return;
    const long long p = i / fchunks;
    const int fc = (int)(i - p * fchunks);
    float av[P], gv[P], d[P], da[P], dg[P];
    unpack16(a[i], av, T{});
    unpack16(g[i], gv, T{});
    unpack16(dh[i], d, T{});
#pragma unroll
    for (int v = 0; v < P; ++v) {
        const float sg = 1.0f / (1.0f + __expf(-av[v]));
        da[v] = d[v] * gv[v] * sg * (1.0f + av[v] * (1.0f - sg));
        dg[v] = d[v] * av[v] * sg;
    }
    dag[p * 2 * fchunks + fc] = pack16(da, T{});
    dag[p * 2 * fchunks + fchunks + fc] = pack16(dg, T{});
}

// ---- transposes (64 x 64 tiles through LDS, 16-byte global accesses) ----
// Every transposed dimension here is a multiple of 64, so tiles are whole.  A thread reads
// 16-byte chunks of source rows into LDS (one 32-bit word per element, rows padded by one
// word), then gathers 16 bytes of a destination row from consecutive source rows.
template <typename T>
struct TileIO {
    static constexpr int kPer = 16 / (int)sizeof(T);   // elements per 16-byte chunk
    static constexpr int kChunks = kTile * kTile / kPer;
    __device__ static void put(uint32_t (*tile)[kTile + 1], int r, int c, const uint4& v) {
        float f[kPer];
        unpack16(v, f, T{});
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            tile[r][c + i] = sizeof(T) == 4 ? __float_as_uint(f[i]) : (__float_as_uint(f[i]) >> 16);
    }
    __device__ static uint4 get(uint32_t (*tile)[kTile + 1], int r, int c) {  // column c, rows r..
        float f[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            f[i] = sizeof(T) == 4 ? __uint_as_float(tile[r + i][c]) : __uint_as_float(tile[r + i][c] << 16);
        return pack16(f, T{});
    }
};

// Transpose into a zero-padded column block: out[c][q] = in[q][c] for q < R, 0 for R <= q
// < kmax.  C and kmax are multiples of 64.
template <typename T>
__global__ __launch_bounds__(256) void seg_transpose_kernel(const T* __restrict__ in, int C,
                                                            int R, int kmax, T* __restrict__ out) {
    using IO = TileIO<T>;
    constexpr int kPer = IO::kPer, kCpr = kTile / kPer;
    __shared__ uint32_t tile[kTile][kTile + 1];
    const int q0 = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
    for (int i = threadIdx.x; i < IO::kChunks; i += 256) {
        const int r = i / kCpr, cc = i - r * kCpr;
        const int q = q0 + r;
        const uint4 v = q < R ? *reinterpret_cast<const uint4*>(in + (size_t)q * C + c0 + cc * kPer)
                              : make_uint4(0, 0, 0, 0);
        IO::put(tile, r, cc * kPer, v);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < IO::kChunks; i += 256) {
        const int c = i / kCpr, rr = i - c * kCpr;
        *reinterpret_cast<uint4*>(out + (size_t)(c0 + c) * kmax + q0 + rr * kPer) =
            IO::get(tile, rr * kPer, c);
    }
}

// ---- weight gradients of small experts: outer products on the vector ALUs ----
// An expert with at most kOuterRows rows (most of them have one or two) makes a weight
// gradient that is almost all output: out[e][m][f] = sum_{i < r} a[p_i][aoff + m] *
// b[src(p_i)][f], p_i = offsets[e] + i, src = gather[p] or p, fp32 FMAs in ascending i, one
// rounding.  One workgroup per (expert, kOuterM output rows); each thread takes 16-byte
// chunks of f, so every store instruction writes whole row segments; the rows it reads are
// the untransposed ones.  The expert's source rows and its a values (the same for every
// thread) are staged in LDS once, and the b chunks of kOuterBatch rows are loaded before
// any of their FMAs, so a pass over f waits for about r / kOuterBatch memory latencies
// rather than r.  Experts without rows get zeros; larger experts are left to the tile GEMM.
constexpr int kOuterRows = 64;
constexpr int kOuterM = 16;
constexpr int kOuterBatch = 4;

template <typename T>
__global__ __launch_bounds__(256) void wgrad_outer_kernel(const T* __restrict__ a, int lda, int aoff,
                                                          const T* __restrict__ b, int ldb,
                                                          const int32_t* __restrict__ gather,
                                                          const int32_t* __restrict__ offsets,
                                                          int M, int Nf, T* __restrict__ out) {
    constexpr int P = 16 / (int)sizeof(T);
    constexpr int Q = kOuterM / P;                  // 16-byte chunks of a per row
    __shared__ int src_s[kOuterRows];
    __shared__ uint4 a_s[kOuterRows][Q];
    const int e = blockIdx.y, m0 = blockIdx.x * kOuterM;
    const int p0 = offsets[e], r = offsets[e + 1] - p0;
    if (r > kOuterRows) return;                     // whole workgroup
    for (int i = threadIdx.x; i < r; i += 256) src_s[i] = gather ? gather[p0 + i] : p0 + i;
    for (int j = threadIdx.x; j < r * Q; j += 256)
        a_s[j / Q][j % Q] = reinterpret_cast<const uint4*>(a + (size_t)(p0 + j / Q) * lda + aoff + m0)[j % Q];
    __syncthreads();
    T* o = out + ((size_t)e * M + m0) * Nf;
    const int nfc = Nf / P;
    for (int fc = threadIdx.x; fc < nfc; fc += 256) {
        float acc[kOuterM][P];
#pragma unroll
        for (int mm = 0; mm < kOuterM; ++mm)
#pragma unroll
            for (int v = 0; v < P; ++v) acc[mm][v] = 0.0f;
        for (int i0 = 0; i0 < r; i0 += kOuterBatch) {
            uint4 bq[kOuterBatch];
#pragma unroll
            for (int u = 0; u < kOuterBatch; ++u)
                if (i0 + u < r)
                    bq[u] = *reinterpret_cast<const uint4*>(b + (size_t)src_s[i0 + u] * ldb + (size_t)fc * P);
#pragma unroll
            for (int u = 0; u < kOuterBatch; ++u) {
                if (i0 + u >= r) break;
                float bv[P];
                unpack16(bq[u], bv, T{});
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    float av[P];
                    unpack16(a_s[i0 + u][q], av, T{});
#pragma unroll
                    for (int w = 0; w < P; ++w)
#pragma unroll
                        for (int v = 0; v < P; ++v) acc[q * P + w][v] = fmaf(av[w], bv[v], acc[q * P + w][v]);
                }
            }
        }
#pragma unroll
        for (int mm = 0; mm < kOuterM; ++mm)
            *reinterpret_cast<uint4*>(o + (size_t)mm * Nf + (size_t)fc * P) = pack16(acc[mm], T{});
    }
}

// list[0, *nlist) = the experts with more than `small` rows, ascending (one workgroup,
// E <= 1024).
__global__ __launch_bounds__(1024) void split_experts_kernel(const int32_t* __restrict__ counts,
                                                             int E, int small,
                                                             int32_t* __restrict__ list,
                                                             int32_t* __restrict__ nlist) {
    __shared__ int scan[2][1024];
    const int e = threadIdx.x;
    const int v = e < E && counts[e] > small ? 1 : 0;
    int cur = 0;
    scan[0][e] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int s_ = scan[cur][e] + (e >= d ? scan[cur][e - d] : 0);
        scan[cur ^ 1][e] = s_;
        cur ^= 1;
        __syncthreads();
    }
    if (v) list[scan[cur][e] - 1] = e;
    if (e == 1023) *nlist = scan[cur][e];
}

template <typename T>
hipError_t seg_transpose(const void* in, int C, int R, int kmax, void* out, hipStream_t s) {
    const dim3 grid((kmax + kTile - 1) / kTile, (C + kTile - 1) / kTile);
    hipLaunchKernelGGL(seg_transpose_kernel<T>, grid, dim3(256), 0, s, static_cast<const T*>(in),
                       C, R, kmax, static_cast<T*>(out));
    return hipGetLastError();
}

size_t align_up(size_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of the layer backward (every piece 256-byte aligned).
struct BwdWs {
    void *gemm, *dy, *dh, *a, *g, *dag, *dxd, *xd, *dlt, *xt;
    float *dw, *dl;
    int32_t *gofs, *elist, *nlist, *zero;
    int tpad;
    size_t bytes;
};

BwdWs carve_bwd(void* base, int dt, int T, int H, int E, int F, int k) {
    const size_t es = dt == 0 ? 4 : 2;
    const long long N = (long long)T * k;
    BwdWs w{};
    w.tpad = (T + kTile - 1) / kTile * kTile;
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t n) -> void* {
        void* r = p ? p + off : nullptr;
        off += align_up(n);
        return r;
    };
    w.gemm = take(gemm_ws_bytes(N, E));
    w.dy = take(es * N * H);
    w.dh = take(es * N * F);
    w.a = take(es * N * F);
    w.g = take(es * N * F);
    w.dag = take(es * N * 2 * F);
    w.dxd = take(es * N * H);
    w.xd = take(es * N * H);          // the dispatched rows, when the forward gathered them
    w.dlt = take(es * E * w.tpad);
    w.xt = take(es * H * w.tpad);
    w.dw = static_cast<float*>(take(4 * N));
    w.dl = static_cast<float*>(take(4 * N));
    w.gofs = static_cast<int32_t*>(take(8));
    w.zero = static_cast<int32_t*>(take(64));
    w.elist = static_cast<int32_t*>(take(4 * (size_t)E));
    w.nlist = static_cast<int32_t*>(take(4));
    w.bytes = off;
    return w;
}

// The gate gradient's one column block [0, tpad) and 64 zero bytes (what the weight
// gradients' last k-slice reads past an expert's rows).
__global__ void set_gofs_kernel(int32_t* gofs, int tpad, int32_t* zero) {
    if (threadIdx.x < 16) zero[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        gofs[0] = 0;
        gofs[1] = tpad;
    }
}

template <typename T>
hipError_t layer_backward_t(const BwdParams& b, hipStream_t s) {
    const int T_ = b.T, H = b.H, E = b.E, F = b.F, k = b.k, dt = b.dt;
    const int N = T_ * k;
    const BwdWs w = carve_bwd(b.ws, dt, T_, H, E, F, k);
    const int chunks_h = (int)((size_t)H * sizeof(T) / 16);
    hipError_t err;
#define MOE_CHECK(expr)                            \
    do {                                           \
        err = (expr);                              \
        if (err != hipSuccess) return err;         \
    } while (0)
    // combine backward: dy, dw (into the caller's dtw when given)
    float* dw = b.dtw ? b.dtw : w.dw;
    hipLaunchKernelGGL(combine_bwd_kernel<T>, dim3(T_), dim3(row_threads(chunks_h)), 0, s,
                       static_cast<const uint4*>(b.dout), static_cast<const uint4*>(b.y), b.dest_pos,
                       b.top_weights, static_cast<uint4*>(w.dy), dw, k, N, chunks_h);
    MOE_CHECK(hipGetLastError());
    // dh = dy . W2[e];  a, g recomputed;  dag = SwiGLU backward;  dxd = dag . [W1; W3].  The
    // weights are read as stored (W2[e] is [H][F], W1[e] and W3[e] are [F][H]: K-major here).
    MOE_CHECK(launch_grouped_kmajor(dt, N, E, H, F, w.dy, b.offsets, b.w2, nullptr, 0, F,
                                    (long long)H * F, w.dh, w.gemm, s));
    const void* act = b.xd ? b.xd : b.x;
    const int32_t* gather = b.xd ? nullptr : b.token_ids;
    // a and g: stored by the forward, or recomputed (the same tiles and summation order)
    const void* ag_a = b.a ? b.a : w.a;
    const void* ag_g = b.g ? b.g : w.g;
    if (!b.a)
        MOE_CHECK(launch_grouped_pair(dt, N, E, H, F, act, gather, T_, b.offsets, b.w1, b.w3, w.a,
                                      w.g, w.gemm, s));
    const int fchunks = (int)((size_t)F * sizeof(T) / 16);
    const long long nfc = (long long)N * fchunks;
    hipLaunchKernelGGL(swiglu_bwd_kernel<T>, dim3((unsigned)((nfc + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint4*>(w.dh), static_cast<const uint4*>(ag_a),
                       static_cast<const uint4*>(ag_g), nfc, fchunks, static_cast<uint4*>(w.dag));
    MOE_CHECK(hipGetLastError());
    MOE_CHECK(launch_grouped_kmajor(dt, N, E, 2 * F, H, w.dag, b.offsets, b.w1, b.w3, F, H,
                                    (long long)F * H, w.dxd, w.gemm, s));
    // the dispatched rows for the weight gradients (the forward gathered them from x)
    const void* xd_rows = b.xd;
    if (!b.xd) {
        MOE_CHECK(launch_dispatch(dt, T_, k, H, b.x, b.dest_pos, w.xd, s));
        xd_rows = w.xd;
    }
    hipLaunchKernelGGL(set_gofs_kernel, dim3(1), dim3(64), 0, s, w.gofs, w.tpad, w.zero);
    MOE_CHECK(hipGetLastError());
    // weight gradients: experts with at most kOuterRows rows (or none) as outer products,
    // the others on the tile GEMM over their rows
    hipLaunchKernelGGL(split_experts_kernel, dim3(1), dim3(1024), 0, s, b.counts, E, kOuterRows,
                       w.elist, w.nlist);
    MOE_CHECK(hipGetLastError());
    hipLaunchKernelGGL(wgrad_outer_kernel<T>, dim3(H / kOuterM, E), dim3(256), 0, s,
                       static_cast<const T*>(w.dy), H, 0, static_cast<const T*>(b.h), F, nullptr,
                       b.offsets, H, F, static_cast<T*>(b.dw2));
    MOE_CHECK(hipGetLastError());
    for (int half = 0; half < 2; ++half) {
        hipLaunchKernelGGL(wgrad_outer_kernel<T>, dim3(F / kOuterM, E), dim3(256), 0, s,
                           static_cast<const T*>(w.dag), 2 * F, half * F, static_cast<const T*>(act), H,
                           gather, b.offsets, F, H, static_cast<T*>(half ? b.dw3 : b.dw1));
        MOE_CHECK(hipGetLastError());
    }
    // the listed experts' gradients from the row-major buffers, read K-major
    const size_t es = sizeof(T);
    MOE_CHECK(launch_wgrad_rows(dt, E, H, F, w.dy, H, b.h, F, b.offsets, w.elist, w.nlist, w.zero,
                                b.dw2, s));
    MOE_CHECK(launch_wgrad_rows(dt, E, F, H, w.dag, 2 * F, xd_rows, H, b.offsets, w.elist, w.nlist,
                                w.zero, b.dw1, s));
    MOE_CHECK(launch_wgrad_rows(dt, E, F, H, static_cast<const char*>(w.dag) + es * F, 2 * F, xd_rows,
                                H, b.offsets, w.elist, w.nlist, w.zero, b.dw3, s));
    // gate: dl, then dx (dispatch backward + gate), dWg and dbias
    hipLaunchKernelGGL(gate_dl_kernel<T>, dim3((T_ + 3) / 4), dim3(256), 0, s,
                       static_cast<const uint4*>(b.x), static_cast<const uint4*>(b.wg), b.bias,
                       b.top_experts, dw, b.routing, T_, chunks_h, k, w.dl);
    MOE_CHECK(hipGetLastError());
    hipLaunchKernelGGL(token_grad_kernel<T>, dim3(T_), dim3(row_threads(chunks_h)), 0, s,
                       static_cast<const uint4*>(w.dxd), b.dest_pos, w.dl, b.top_experts,
                       static_cast<const uint4*>(b.wg), static_cast<uint4*>(b.dx), k, N, chunks_h);
    MOE_CHECK(hipGetLastError());
    const long long nd = (long long)E * w.tpad;
    hipLaunchKernelGGL(gate_dlt_kernel<T>, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, s, w.dl,
                       b.top_experts, T_, E, k, w.tpad, static_cast<T*>(w.dlt));
    MOE_CHECK(hipGetLastError());
    MOE_CHECK(seg_transpose<T>(b.x, H, T_, w.tpad, w.xt, s));
    MOE_CHECK(launch_wgrad(dt, 1, E, H, w.tpad, w.dlt, w.xt, w.gofs, nullptr, nullptr, b.dwg, s));
    hipLaunchKernelGGL(gate_dbias_kernel, dim3(E), dim3(256), 0, s, w.dl, b.offsets, b.token_ids,
                       b.dest_pos, k, b.dbias);
    MOE_CHECK(hipGetLastError());
#undef MOE_CHECK
    return hipSuccess;
}

}  // namespace

size_t backward_ws_bytes(int dt, int T, int H, int E, int F, int k) {
    return carve_bwd(nullptr, dt, T, H, E, F, k).bytes;
}

hipError_t launch_layer_backward(const BwdParams& b, hipStream_t s) {
    if (b.T == 0) return hipSuccess;
    return b.dt == 0 ? layer_backward_t<float>(b, s) : layer_backward_t<bf16_t>(b, s);
}

}  // namespace moe
