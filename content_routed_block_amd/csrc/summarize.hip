// Block summary: the mean of each block of bs consecutive tokens (the first
// cumulant mu_c of the SSA routing score, SSA page "Algorithm and
// complexity").  HBM-bound streaming kernel: one wave per (head, block)
// (16-token blocks: k_summarize16, a lane per 8 dims of a block);
// lane l reads 16 bytes (8 dims) of token l/8 + 8i, so every load
// instruction covers 1 KB of consecutive memory, and a lane issues all of
// its loads before the first one is used.  Sums are kept in fp64 and
// rounded once to fp32, so the result is the fp32 rounding of the exact
// mean whenever the fp64 sum is exact (always, for bf16 data whose
// magnitudes span fewer than ~2^39).
#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

// Blocks of 16 tokens: a lane owns 8 dims of one block and sums its 16 rows
// itself (eight blocks per wave), so no cross-lane reduction is needed; a
// load instruction still reads whole 128-byte rows (eight lanes per row).
__global__ __launch_bounds__(256) void k_summarize16(const uint16_t* __restrict__ x,
                                                     float* __restrict__ xbar,
                                                     int64_t n_blocks) {
    const int lane = threadIdx.x & 63;
    const int64_t blk = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 8 + (lane >> 3);
    if (blk >= n_blocks) return;
    const int dg = lane & 7;  // dims 8*dg .. 8*dg+7
    // blocks are consecutive runs of 16 tokens, so block blk starts at row 16*blk
    const uint16_t* base = x + blk * 16 * kD + dg * 8;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)i * kD);
    double acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] += (double)f[d];
    }
    constexpr double inv = 1.0 / 16.0;
    f32x4 lo, hi;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        lo[d] = (float)(acc[d] * inv);
        hi[d] = (float)(acc[4 + d] * inv);
    }
    float* o = xbar + blk * kD + dg * 8;
    *reinterpret_cast<f32x4*>(o) = lo;
    *reinterpret_cast<f32x4*>(o + 4) = hi;
}

template <int BS>
__global__ __launch_bounds__(256) void k_summarize(const uint16_t* __restrict__ x,
                                                   float* __restrict__ xbar,
                                                   int64_t n_blocks, int N) {
    constexpr int LOADS = BS / 8;  // 16-byte loads per lane, all issued before any use
    const int lane = threadIdx.x & 63;
    const int64_t wblk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wblk >= n_blocks) return;
    const int nb = N / BS;
    const int64_t bh = wblk / nb;
    const int64_t c = wblk - bh * nb;
    const int dg = lane & 7;   // dims 8*dg .. 8*dg+7
    const int j0 = lane >> 3;  // tokens j0, j0+8, ...
    const uint16_t* base = x + (bh * N + c * BS + j0) * kD + dg * 8;
    u32x4 v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)i * 8 * kD);
    double acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] += (double)f[d];
    }
#pragma unroll
    for (int m = 8; m < 64; m <<= 1)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] += __shfl_xor(acc[d], m, kWave);
    if (j0 == 0) {
        constexpr double inv = 1.0 / (double)BS;  // a power of two: exact
        f32x4 lo, hi;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            lo[d] = (float)(acc[d] * inv);
            hi[d] = (float)(acc[4 + d] * inv);
        }
        float* o = xbar + wblk * kD + dg * 8;
        *reinterpret_cast<f32x4*>(o) = lo;
        *reinterpret_cast<f32x4*>(o + 4) = hi;
    }
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t value) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

hipError_t launch_summarize(const uint16_t* x, float* xbar, int BH, int N, int bs,
                            hipStream_t s) {
    const int64_t n_blocks = (int64_t)BH * (N / bs);
    const int64_t grid = (n_blocks + 3) / 4;
    switch (bs) {
        case 16:
            hipLaunchKernelGGL(k_summarize16, dim3((unsigned)((n_blocks + 31) / 32)), dim3(256), 0, s,
                               x, xbar, n_blocks);
            break;
        case 32: hipLaunchKernelGGL(k_summarize<32>, dim3((unsigned)grid), dim3(256), 0, s, x, xbar, n_blocks, N); break;
        case 64: hipLaunchKernelGGL(k_summarize<64>, dim3((unsigned)grid), dim3(256), 0, s, x, xbar, n_blocks, N); break;
        default: hipLaunchKernelGGL(k_summarize<128>, dim3((unsigned)grid), dim3(256), 0, s, x, xbar, n_blocks, N); break;
    }
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t grid = (n + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)grid), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

}  // namespace lsa
