// probe.hip -- memory-path ceilings that the tile engine's roofline is read against.
//
// One workgroup per CU (grid 256) reads a region of R bytes round-robin with 16 bytes per
// lane, either the way the engine's loader waves do (direct-to-LDS transfers into a
// 3-slot ring of 48 KiB k-slices, at most two slices outstanding per wave) or as plain
// vector loads into registers; or writes it the same way with plain 16-byte stores.  A region of 1 MiB stays in every XCD's L2, 64 MiB fits the
// Infinity Cache, 1 GiB streams from HBM.  The rate per CU for 4 and 8 issuing waves and
// the chip's total show what bounds a kernel that moves its operands this way.
//
// Measurement only: built into libmoe_probe.so, which libmoe.so neither contains nor
// loads.  C ABI:
//   int moe_probe_stream(int kind, int waves, const void* buf, long long region_bytes,
//                        int grid, int iters, int* sink, void* stream)
//   kind 0: direct-to-LDS, 1: plain loads, 2: plain stores (buf is overwritten); waves 4 or
//   8; buf: device, 16-byte aligned,
//   region_bytes readable bytes, 48 KiB to 256 GiB; sink: device, grid * waves * 64 ints;
//   each workgroup reads iters x 48 KiB.  Returns 0, 1 for a bad argument, 2 when the
//   launch fails.  The launch goes to `stream` and is not waited for.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kSliceRows = 384;              // 48 KiB of 128-byte rows
constexpr int kSlice = kSliceRows * 128;

__device__ __forceinline__ void dma16(const void* src, uint32_t lds_block) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "{m0}"(lds_block)
                 : "memory");
}

// Each lane walks its rows of successive slices: the row of slice it + 1 is the row of
// slice it plus kSliceRows, wrapped once (rows >= kSliceRows), so an address costs one add
// and one compare as in the engine's loaders.
__device__ __forceinline__ int next_row(int row, int rows) {
    row += kSliceRows;
    return row >= rows ? row - rows : row;
}

// Wave w issues the 1 KiB blocks w, w + NW, ... of every slice (8 rows of 128 bytes each,
// chunks permuted within a row as the engine's LDS layout requires), keeping at most two
// slices outstanding; slot it % 3 of the ring receives slice it.
template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void lds_stream_kernel(const char* buf, int rows,
                                                                 int iters, int* sink) {
    __shared__ __attribute__((aligned(1024))) char lds[3 * kSlice];
    constexpr int kPer = kSliceRows / 8 / NW;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                              (__attribute__((address_space(3))) char*)(lds))) + w * 1024;
    const long long start = (long long)blockIdx.x * kSliceRows * 7;
    int row[kPer], chunk[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int r = (w + NW * i) * 8 + lane / 8;
        row[i] = (int)((start + r) % rows);
        chunk[i] = ((lane & 7) ^ ((r >> 1) & 7)) * 16;
    }
    for (int it = 0; it < iters; ++it) {
        const int slot = it % 3;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            dma16(buf + (size_t)row[i] * 128 + chunk[i],
                  __builtin_amdgcn_readfirstlane(base + slot * kSlice + (uint32_t)(i * NW * 1024)));
            row[i] = next_row(row[i], rows);
        }
        // vmcnt <= 2 kPer: simm16 = vmcnt[3:0] | expcnt 7 << 4 | lgkmcnt 15 << 8 | vmcnt[5:4] << 14
        constexpr int n = 2 * kPer;
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));      // vmcnt(0)
    __syncthreads();
    sink[blockIdx.x * NW * 64 + threadIdx.x] = lds[threadIdx.x];
}

// The same blocks read into registers (kPer loads in flight per wave), folded together.
template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void reg_stream_kernel(const uint4* buf, int rows,
                                                                int iters, int* sink) {
    constexpr int kPer = kSliceRows / 8 / NW;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long start = (long long)blockIdx.x * kSliceRows * 7;
    int row[kPer], chunk[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int r = (w * kPer + i) * 8 + lane / 8;
        row[i] = (int)((start + r) % rows);
        chunk[i] = (lane & 7) ^ ((r >> 1) & 7);
    }
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int it = 0; it < iters; ++it) {
        uint4 v[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            v[i] = buf[(size_t)row[i] * 8 + chunk[i]];
            row[i] = next_row(row[i], rows);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            acc.x ^= v[i].x;
            acc.y ^= v[i].y;
            acc.z ^= v[i].z;
            acc.w ^= v[i].w;
        }
    }
    sink[blockIdx.x * NW * 64 + threadIdx.x] = (int)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

// The same blocks written: every lane stores 16 bytes per block, kPer stores per slice.
template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void reg_store_kernel(uint4* buf, int rows, int iters,
                                                               int* sink) {
    constexpr int kPer = kSliceRows / 8 / NW;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long start = (long long)blockIdx.x * kSliceRows * 7;
    int row[kPer], chunk[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int r = (w * kPer + i) * 8 + lane / 8;
        row[i] = (int)((start + r) % rows);
        chunk[i] = (lane & 7) ^ ((r >> 1) & 7);
    }
    const uint4 v = make_uint4(blockIdx.x, threadIdx.x, 0, 1);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            buf[(size_t)row[i] * 8 + chunk[i]] = v;
            row[i] = next_row(row[i], rows);
        }
    }
    sink[blockIdx.x * NW * 64 + threadIdx.x] = row[0];
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int moe_probe_stream(
    int kind, int waves, const void* buf, long long region_bytes, int grid, int iters, int* sink,
    void* stream) {
    if ((kind < 0 || kind > 2) || (waves != 4 && waves != 8) || !buf || !sink ||
        (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || region_bytes < kSlice ||
        region_bytes / 128 > 0x7fffffffll || grid < 1 || grid > 4096 || iters < 1)
        return 1;
    const int rows = (int)(region_bytes / 128);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* b = static_cast<const char*>(buf);
    if (kind == 0) {
        if (waves == 4)
            hipLaunchKernelGGL(lds_stream_kernel<4>, dim3(grid), dim3(256), 0, s, b, rows, iters, sink);
        else
            hipLaunchKernelGGL(lds_stream_kernel<8>, dim3(grid), dim3(512), 0, s, b, rows, iters, sink);
    } else if (kind == 1) {
        const uint4* u = static_cast<const uint4*>(buf);
        if (waves == 4)
            hipLaunchKernelGGL(reg_stream_kernel<4>, dim3(grid), dim3(256), 0, s, u, rows, iters, sink);
        else
            hipLaunchKernelGGL(reg_stream_kernel<8>, dim3(grid), dim3(512), 0, s, u, rows, iters, sink);
    } else {
        uint4* u = static_cast<uint4*>(const_cast<void*>(buf));
        if (waves == 4)
            hipLaunchKernelGGL(reg_store_kernel<4>, dim3(grid), dim3(256), 0, s, u, rows, iters, sink);
        else
            hipLaunchKernelGGL(reg_store_kernel<8>, dim3(grid), dim3(512), 0, s, u, rows, iters, sink);
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
