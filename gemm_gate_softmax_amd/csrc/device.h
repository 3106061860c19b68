// device.h -- gfx950 building blocks shared by the kernels of libmoe.so: storage types,
// bf16 conversion, 16-byte vector access, wave64 reductions and the two MFMA steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, nearest with ties to even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

// Storage-type traits: element size and the conversions used by epilogues.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    static constexpr int kPer16B = 4;
    __device__ static float load(const float* p, size_t i) { return p[i]; }
};
template <> struct Elem<bf16_t> {
    static constexpr int kBytes = 2;
    static constexpr int kPer16B = 8;
};

// Unpack a 16-byte chunk of storage elements to fp32 and back.
__device__ __forceinline__ void unpack16(const uint4& v, float (&o)[4], float) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const uint4& v, float (&o)[8], bf16_t) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack16(const float (&o)[4], float) {
    return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                      __float_as_uint(o[3]));
}
__device__ __forceinline__ uint4 pack16(const float (&o)[8], bf16_t) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(f32_to_bf16(o[2 * i])) |
               (static_cast<uint32_t>(f32_to_bf16(o[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- wave64 helpers --

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// One DPP lane move of a 64-bit value within each row of 16 lanes (CTRL: a dpp_ctrl code).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xf, 0xf, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xf, 0xf, false));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Maximum over the wave's 64 lanes, on every lane.  Within each row of 16 lanes the values
// meet through DPP lane moves (the lane 1 apart, 2 apart, then the mirrored lane in the half
// row and in the row), so every lane of a row holds the row's maximum; the four row maxima
// are read into scalar registers and combined.  No LDS round trip, unlike a shuffle.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o;
    o = dpp_u64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = o > v ? o : v;
    o = dpp_u64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v = o > v ? o : v;
    o = dpp_u64<0x141>(v);  // row_half_mirror
    v = o > v ? o : v;
    o = dpp_u64<0x140>(v);  // row_mirror
    v = o > v ? o : v;
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < kWave; r += 16) {
        const uint64_t x = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), r))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), r));
        m = x > m ? x : m;
    }
    return m;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Orders this lane's earlier LDS/global accesses before its later ones as seen by the
// other lanes of the same wave (cross-lane hand-off through LDS without a block barrier).
__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger integer).
// -0.0 is folded onto +0.0 first so the two compare equal, as IEEE comparison does.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------------ MFMA --
// 32x32 output tiles: on gfx950 the 32x32x16 bf16 instruction sustains about 2.1-2.2
// PFLOP/s chip-wide against about 1.3 for 16x16x32, so every product uses 32x32 tiles.
// One "k-step" consumes one 16-byte chunk per lane from each operand: lane l supplies
// row (l % 32) of the A side and column (l % 32) of the B side, and its chunk holds the
// k-slice of half l / 32 of the step.  The result tile gives lane l column (l % 32) and
// rows 8 j + 4 (l / 32) + v in register 4 j + v (j, v = 0..3).
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
    // one 32x32x16 instruction: the chunk is 8 consecutive k of this lane's half
    __device__ static __forceinline__ void mac(f32x16_t& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    // four 32x32x2 instructions: element e of the chunk is this lane's k for the e-th one
    __device__ static __forceinline__ void mac(f32x16_t& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

}  // namespace moe
