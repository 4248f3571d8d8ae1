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

// With RouteOut (the layer's key summary feeding its own routing), the
// summary kernels also write the routing kernels' inputs: the bf16 hi/lo
// split of each block mean into rows of nb_pad per head (rows past nb
// zero), per chunk of 32 rows the largest norms |mean| and |lo| of its
// rows (route_split_store; kChunkMaxSlots partial maxima per chunk), and
// zeros into the router's counters.
struct RouteOut {
    uint16_t* khi;
    uint16_t* klo;
    float* ckn;    // chunk maxima, kChunkMaxStride floats apart
    float* clo;
    int nb_pad;
    uint32_t* counters;  // kRouteCounterWords words cleared by workgroup 0 (or NULL)
};

// Stores a workgroup's partial chunk maxima into `slot` of its chunk line
// (threads 0 .. kChunkMaxSlots - 1 of the workgroup; with fill, the other
// slots of the line are zeroed, for a workgroup that covers the whole
// chunk) and clears the router's counters from workgroup 0.
__device__ __forceinline__ void store_chunk_max(const RouteOut& ro, int64_t chunk, int slot,
                                                bool fill, float kmax, float lmax, int64_t wg) {
    const int t = threadIdx.x;
    if (t < kChunkMaxSlots && (fill || t == slot)) {
        const int64_t e = chunk * kChunkMaxStride + t;
        ro.ckn[e] = t == slot ? kmax : 0.f;
        ro.clo[e] = t == slot ? lmax : 0.f;
    }
    if (ro.counters && wg == 0 && t < kRouteCounterWords) ro.counters[t] = 0u;
}

// Blocks of 16 tokens: a lane owns 8 dims of one block and sums its 16 rows
// itself (eight blocks per wave), so no cross-lane reduction is needed; a
// load instruction still reads whole 128-byte rows (eight lanes per row).
// With PREP, rows run over heads x nb_pad, so a workgroup (32 rows) is one
// chunk and stores its maxima itself.  wg: this workgroup's index.
template <bool PREP>
__device__ __forceinline__ void summarize16(const uint16_t* __restrict__ x, float* __restrict__ xbar,
                                            int64_t n_blocks, int nb, const RouteOut& ro,
                                            int64_t wg) {
    __shared__ float s_n[2][4];
    const int lane = threadIdx.x & 63;
    const int64_t r = (wg * 4 + (threadIdx.x >> 6)) * 8 + (lane >> 3);
    const int dg = lane & 7;  // dims 8*dg .. 8*dg+7
    int64_t blk = r;          // the block summarised (PREP: row r of the padded layout)
    bool have = r < n_blocks;
    if (PREP) {
        const int64_t bh = r / ro.nb_pad;
        const int c = (int)(r - bh * ro.nb_pad);
        blk = bh * nb + c;
        have = bh * nb < n_blocks && c < nb;
        if (bh * nb < n_blocks && c >= nb) {  // padding row
            const int64_t o = r * kD + dg * 8;
            *reinterpret_cast<u32x4*>(ro.khi + o) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(ro.klo + o) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float kn = 0.f, ln = 0.f;
    if (have) {
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
        if (PREP) {
            const float f[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            route_split_store(f, ro.khi + r * kD + dg * 8, ro.klo + r * kD + dg * 8, kn, ln);
        }
    }
    if (!PREP) return;
    kn = wave_max_nonneg(kn);
    ln = wave_max_nonneg(ln);
    const int w = threadIdx.x >> 6;
    if (lane == 0) {
        s_n[0][w] = kn;
        s_n[1][w] = ln;
    }
    __syncthreads();
    const int64_t r0 = wg * 32;  // this workgroup's rows: one chunk
    if ((r0 / ro.nb_pad) * nb < n_blocks)
        store_chunk_max(ro, wg, 0, true,
                        fmaxf(fmaxf(s_n[0][0], s_n[0][1]), fmaxf(s_n[0][2], s_n[0][3])),
                        fmaxf(fmaxf(s_n[1][0], s_n[1][1]), fmaxf(s_n[1][2], s_n[1][3])), wg);
}

template <bool PREP>
__global__ __launch_bounds__(256) void k_summarize16(const uint16_t* __restrict__ x,
                                                     float* __restrict__ xbar,
                                                     int64_t n_blocks, int nb, RouteOut ro) {
    summarize16<PREP>(x, xbar, n_blocks, nb, ro, blockIdx.x);
}

// Image mode's two poolings in one launch: the first wg_k workgroups
// summarise the keys with the routing preparation, the rest pool the
// queries (both in blocks of 16 tokens).
__global__ __launch_bounds__(256) void k_summarize16_kq(const uint16_t* __restrict__ k,
                                                        float* __restrict__ kbar,
                                                        int64_t nk_blocks, RouteOut ro,
                                                        int64_t wg_k,
                                                        const uint16_t* __restrict__ q,
                                                        float* __restrict__ qbar,
                                                        int64_t nq_blocks, int nb) {
    if ((int64_t)blockIdx.x < wg_k)
        summarize16<true>(k, kbar, nk_blocks, nb, ro, blockIdx.x);
    else
        summarize16<false>(q, qbar, nq_blocks, nb, ro, blockIdx.x - wg_k);
}

// One wave per block.  With PREP, waves run over heads x nb_pad; a
// workgroup (four rows of one chunk) stores its norms' maxima into its own
// slot of the chunk's line (eight workgroups per chunk).
template <int BS, bool PREP>
__global__ __launch_bounds__(256) void k_summarize(const uint16_t* __restrict__ x,
                                                   float* __restrict__ xbar,
                                                   int64_t n_blocks, int N, RouteOut ro) {
    constexpr int LOADS = BS / 8;  // 16-byte loads per lane, all issued before any use
    __shared__ float s_n[2][4];
    const int lane = threadIdx.x & 63;
    const int64_t wblk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nb = N / BS;
    const int dg = lane & 7;   // dims 8*dg .. 8*dg+7
    const int j0 = lane >> 3;  // tokens j0, j0+8, ...
    int64_t bh = wblk / nb, c = wblk - bh * nb;
    bool have = wblk < n_blocks;
    if (PREP) {
        bh = wblk / ro.nb_pad;
        c = wblk - bh * ro.nb_pad;
        have = bh * nb < n_blocks && c < nb;
        if (bh * nb < n_blocks && c >= nb && j0 == 0) {  // padding row
            const int64_t o = wblk * kD + dg * 8;
            *reinterpret_cast<u32x4*>(ro.khi + o) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(ro.klo + o) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float kn = 0.f, ln = 0.f;
    if (have) {
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
            float* o = xbar + (bh * nb + c) * kD + dg * 8;
            *reinterpret_cast<f32x4*>(o) = lo;
            *reinterpret_cast<f32x4*>(o + 4) = hi;
            if (PREP) {
                const float f[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                const int64_t r = wblk * kD + dg * 8;
                route_split_store(f, ro.khi + r, ro.klo + r, kn, ln);
            }
        }
    }
    if (!PREP) return;
    const int w = threadIdx.x >> 6;
    if (lane == 0) {  // lanes 0..7 hold the row's norms
        s_n[0][w] = kn;
        s_n[1][w] = ln;
    }
    __syncthreads();
    const int64_t r0 = (int64_t)blockIdx.x * 4;  // this workgroup's rows, in one chunk
    static_assert(32 / 4 == kChunkMaxSlots, "a chunk spans one slot per workgroup");
    if ((r0 / ro.nb_pad) * nb < n_blocks)
        store_chunk_max(ro, r0 / 32, (int)(blockIdx.x % kChunkMaxSlots), false,
                        fmaxf(fmaxf(s_n[0][0], s_n[0][1]), fmaxf(s_n[0][2], s_n[0][3])),
                        fmaxf(fmaxf(s_n[1][0], s_n[1][1]), fmaxf(s_n[1][2], s_n[1][3])),
                        blockIdx.x);
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t value) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

template <bool PREP>
static hipError_t summarize(const uint16_t* x, float* xbar, int BH, int N, int bs, RouteOut ro,
                            hipStream_t s) {
    const int nb = N / bs;
    const int64_t n_blocks = (int64_t)BH * nb;
    const int64_t rows = PREP ? (int64_t)BH * ro.nb_pad : n_blocks;  // waves (16: lane groups)
    const int64_t grid = (rows + 3) / 4;
    switch (bs) {
        case 16:
            hipLaunchKernelGGL(k_summarize16<PREP>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0,
                               s, x, xbar, n_blocks, nb, ro);
            break;
        case 32: hipLaunchKernelGGL((k_summarize<32, PREP>), dim3((unsigned)grid), dim3(256), 0, s, x, xbar, n_blocks, N, ro); break;
        case 64: hipLaunchKernelGGL((k_summarize<64, PREP>), dim3((unsigned)grid), dim3(256), 0, s, x, xbar, n_blocks, N, ro); break;
        default: hipLaunchKernelGGL((k_summarize<128, PREP>), dim3((unsigned)grid), dim3(256), 0, s, x, xbar, n_blocks, N, ro); break;
    }
    return hipGetLastError();
}

hipError_t launch_summarize(const uint16_t* x, float* xbar, int BH, int N, int bs,
                            hipStream_t s) {
    return summarize<false>(x, xbar, BH, N, bs, RouteOut{}, s);
}

hipError_t launch_summarize_route(const uint16_t* x, float* xbar, int BH, int N, int bs,
                                  uint16_t* khi, uint16_t* klo, float* ckn, float* clo,
                                  int nb_pad, uint32_t* counters, hipStream_t s) {
    return summarize<true>(x, xbar, BH, N, bs, RouteOut{khi, klo, ckn, clo, nb_pad, counters}, s);
}

hipError_t launch_summarize_route_pool16(const uint16_t* k, float* kbar, int BHk, const uint16_t* q,
                                         float* qbar, int BHq, int N, uint16_t* khi, uint16_t* klo,
                                         float* ckn, float* clo, int nb_pad, uint32_t* counters,
                                         hipStream_t s) {
    const int nb = N / 16;
    const int64_t nk = (int64_t)BHk * nb, nq = (int64_t)BHq * nb;
    const int64_t wg_k = ((int64_t)BHk * nb_pad + 31) / 32;  // rows over heads x nb_pad
    const int64_t wg_q = (nq + 31) / 32;
    hipLaunchKernelGGL(k_summarize16_kq, dim3((unsigned)(wg_k + wg_q)), dim3(256), 0, s, k, kbar,
                       nk, RouteOut{khi, klo, ckn, clo, nb_pad, counters}, wg_k, q, qbar, nq, nb);
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
