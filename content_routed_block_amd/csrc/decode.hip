// Single-query decode against a key/value cache: the same content-routed
// selection and exact sparse softmax as the prefill path, for the query at
// position T-1 of a cache holding T tokens (SSA page, "Other measured
// evidence": decode steps against a growing cache at a fixed selection
// budget; selection rule as in lsa_route_topk, attention as in
// lsa_sparse_attend).
//
// A decode step is latency-bound and touches little data (per query head
// about top_k + window/bs blocks of K/V and the eligible block means), so it
// runs on the vector ALUs in fp32 with enough workgroups to spread the reads:
//   0. k_decode_summarize   the mean of the block that token T-1 completes
//                           (when T is a multiple of bs), kept in the caller's
//                           block-mean cache for later steps.
//   1. k_decode_route_chunk scores q . kbar_c for a chunk of 1024 eligible
//                           blocks per workgroup and keeps the chunk's top-k
//                           as 64-bit keys (score, then lower index).
//   2. k_decode_route_merge merges the chunk lists of a row into its top-k and
//                           writes the block ids in ascending order.
//   3. k_decode_attend      one workgroup per query head: exact softmax over
//                           the routed blocks and the block-aligned window,
//                           in passes of 1024 keys with an online softmax.
#include <math.h>

#include <algorithm>

#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

constexpr int DC_CHUNK = 1024;  // candidate blocks per routing workgroup
constexpr int DC_KEYS = 1024;   // keys per attention pass

struct DecodeArgs {
    const uint16_t* q;   // [B*Hq][64]
    const uint16_t* k;   // [B*Hkv][t_max][64]
    const uint16_t* v;   // [B*Hkv][t_max][64]
    float* kbar;         // [B*Hkv][t_max/bs][64]
    int32_t* idx;        // [B*Hq][top_k]
    float* out;          // [B*Hq][64]
    uint64_t* keys;      // [B*Hq][nchunk][kMaxTopK]
    int Hq, Hkv, T, t_max, bs, top_k, window, E, nchunk;
    float scale_log2;
};

__device__ __forceinline__ float block_max_f32(float x, float* s_red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    if (lane == 0) s_red[w] = x;
    __syncthreads();
    const float r = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_sum_f32(float x, float* s_red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    if (lane == 0) s_red[w] = x;
    __syncthreads();
    const float r = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    __syncthreads();
    return r;
}

// ------------------------------------------------------------ 0. block mean
// One wave per (b, KV head): the mean of block c (tokens [c*bs, c*bs + bs)),
// summed in fp64 and rounded once to fp32, as lsa_block_summarize does.
__global__ __launch_bounds__(64) void k_decode_summarize(DecodeArgs a, int c) {
    const int bg = blockIdx.x, lane = threadIdx.x;
    const int dg = lane & 7, j0 = lane >> 3;
    const uint16_t* base = a.k + ((int64_t)bg * a.t_max + (int64_t)c * a.bs) * kD + dg * 8;
    double acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.0;
    for (int j = j0; j < a.bs; j += 8) {
        float f[8];
        unpack8(*reinterpret_cast<const u32x4*>(base + (int64_t)j * kD), f);
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] += (double)f[d];
    }
#pragma unroll
    for (int m = 8; m < 64; m <<= 1)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] += __shfl_xor(acc[d], m, kWave);
    if (j0 == 0) {
        const double inv = 1.0 / (double)a.bs;  // a power of two: exact
        float* o = a.kbar + ((int64_t)bg * (a.t_max / a.bs) + c) * kD + dg * 8;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d] = (float)(acc[d] * inv);
    }
}

// ------------------------------------------------------------ top-k helpers
// The wave's keys are key[0..n) in every lane; returns, in every lane, the
// largest key below `below` over the wave (0 if none).
template <int n>
__device__ __forceinline__ uint64_t wave_max_below(const uint64_t (&key)[n], uint64_t below) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < n; ++i)
        if (key[i] < below && key[i] > best) best = key[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off, kWave);
        best = o > best ? o : best;
    }
    return best;
}

// ------------------------------------------------------------ 1. chunk top-k
// Workgroup (row, chunk): fp32 scores of the chunk's eligible blocks (the dot
// product accumulated over d in order).  Each wave extracts the top_k of its
// 256 candidates by rounds of "largest key below the previous one"; the first
// wave then does the same over the four wave lists.  The chunk list is
// written in descending order, ended by a zero key when shorter than top_k.
__global__ __launch_bounds__(256) void k_decode_route_chunk(DecodeArgs a) {
    __shared__ float s_q[kD];
    __shared__ uint64_t s_list[4][kMaxTopK];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = blockIdx.x / a.nchunk, ch = blockIdx.x - row * a.nchunk;
    const int h = row % a.Hq, b = row / a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    if (tid < kD) s_q[tid] = bf16_bits_to_f32(a.q[(int64_t)row * kD + tid]);
    __syncthreads();
    const int c0 = ch * DC_CHUNK + w * (DC_CHUNK / 4);
    const float* kb = a.kbar + (int64_t)bg * (a.t_max / a.bs) * kD;
    uint64_t key[DC_CHUNK / 256];
#pragma unroll
    for (int i = 0; i < DC_CHUNK / 256; ++i) {
        const int c = c0 + lane + 64 * i;
        key[i] = 0;
        if (c < a.E) {
            const f32x4* kr = reinterpret_cast<const f32x4*>(kb + (int64_t)c * kD);
            float s = 0.f;
#pragma unroll
            for (int d4 = 0; d4 < kD / 4; ++d4) {
                const f32x4 x = kr[d4];
                s = fmaf(s_q[4 * d4], x[0], s);
                s = fmaf(s_q[4 * d4 + 1], x[1], s);
                s = fmaf(s_q[4 * d4 + 2], x[2], s);
                s = fmaf(s_q[4 * d4 + 3], x[3], s);
            }
            key[i] = sel_key(s, (uint32_t)c);
        }
    }
    uint64_t prev = ~0ull;
    for (int j = 0; j < kMaxTopK; ++j) {
        const uint64_t best = j < a.top_k ? wave_max_below(key, prev) : 0;
        if (lane == 0) s_list[w][j] = best;
        prev = best;
    }
    __syncthreads();
    if (w == 0) {
        uint64_t k4[1];
        k4[0] = s_list[lane >> 4][lane & 15];
        uint64_t* out = a.keys + ((int64_t)row * a.nchunk + ch) * kMaxTopK;
        prev = ~0ull;
        for (int j = 0; j < a.top_k; ++j) {
            const uint64_t best = wave_max_below(k4, prev);
            if (lane == 0) out[j] = best;
            prev = best;
            if (best == 0) break;
        }
    }
}

// ------------------------------------------------------------ 2. merge
// One wave per row: lane c holds chunk list c (descending, zero-ended), the
// row's top_k comes from rounds of "largest key below the previous one", and
// lane j < m writes the j-th smallest chosen block id.
__global__ __launch_bounds__(256) void k_decode_route_merge(DecodeArgs a, int rows) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    uint64_t key[kMaxTopK];
    bool live = lane < a.nchunk;
    const uint64_t* in = a.keys + ((int64_t)row * a.nchunk + (live ? lane : 0)) * kMaxTopK;
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) {
        key[i] = (live && i < a.top_k) ? in[i] : 0;
        live = live && key[i] != 0;  // entries after the terminating zero are stale
    }
    int32_t sel[kMaxTopK];
    int m = 0;
    uint64_t prev = ~0ull;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        const uint64_t best = j < a.top_k ? wave_max_below(key, prev) : 0;
        sel[j] = best ? (int32_t)key_block(best) : 0x7FFFFFFF;
        m += best ? 1 : 0;
        prev = best ? best : prev;
    }
    // lane j < top_k: the j-th smallest of the m chosen ids (wave-uniform list)
    int32_t mine = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        int rank = 0;
#pragma unroll
        for (int i = 0; i < kMaxTopK; ++i) rank += sel[i] < sel[j] ? 1 : 0;
        if (j < m && rank == lane) mine = sel[j];
    }
    if (lane < a.top_k) a.idx[(int64_t)row * a.top_k + lane] = lane < m ? mine : -1;
}

// ------------------------------------------------------------ 3. attention
// One workgroup per query head.  The keys are the used routed blocks (an
// entry counts when it is eligible and above the previous used entry) and
// the window [bs*E, T-1], visited as one virtual list in passes of DC_KEYS:
// scores (fp32, in log2 units) into LDS, the pass maximum, probabilities,
// then P.V with thread (key group kg, dims 8dg..8dg+7) summing keys
// kg, kg+32, ... of the pass.
__global__ __launch_bounds__(256) void k_decode_attend(DecodeArgs a) {
    __shared__ float s_q[kD];
    __shared__ float s_p[DC_KEYS];
    __shared__ float s_red[4];
    __shared__ float s_acc[32][kD + 1];
    __shared__ int s_blk[kMaxTopK];
    __shared__ int s_nused;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int h = row % a.Hq, b = row / a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    const uint16_t* kbase = a.k + (int64_t)bg * a.t_max * kD;
    const uint16_t* vbase = a.v + (int64_t)bg * a.t_max * kD;
    if (tid < kD) s_q[tid] = bf16_bits_to_f32(a.q[(int64_t)row * kD + tid]) * a.scale_log2;
    if (tid == 0) {
        const int32_t* ir = a.idx + (int64_t)row * a.top_k;
        int n = 0, prev = -1;
        for (int s = 0; s < a.top_k; ++s) {
            const int c = ir[s];
            if (c > prev && c < a.E) {
                s_blk[n++] = c;
                prev = c;
            }
        }
        s_nused = n;
    }
    __syncthreads();
    const int n_routed = s_nused * a.bs;
    const int win0 = a.bs * a.E;
    const int total = n_routed + (a.T - win0);
    auto token_of = [&](int j) {
        return j < n_routed ? s_blk[j / a.bs] * a.bs + (j % a.bs) : win0 + (j - n_routed);
    };
    const int kg = tid >> 3, dg = tid & 7;  // P.V: key group, 8-dim group
    float o_acc[8];  // running output of dims 8dg.. (kept by threads with kg == 0)
#pragma unroll
    for (int d = 0; d < 8; ++d) o_acc[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    for (int p0 = 0; p0 < total; p0 += DC_KEYS) {
        const int np = min(DC_KEYS, total - p0);
        float mx = -INFINITY;
        for (int j = tid; j < np; j += 256) {
            const uint16_t* kr = kbase + (int64_t)token_of(p0 + j) * kD;
            float s = 0.f;
#pragma unroll
            for (int d8 = 0; d8 < kD / 8; ++d8) {
                float f[8];
                unpack8(*reinterpret_cast<const u32x4*>(kr + 8 * d8), f);
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(s_q[8 * d8 + e], f[e], s);
            }
            s_p[j] = s;
            mx = fmaxf(mx, s);
        }
        mx = block_max_f32(mx, s_red);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
        float sum = 0.f;
        for (int j = tid; j < np; j += 256) {
            const float pj = exp2f(s_p[j] - m_new);
            s_p[j] = pj;
            sum += pj;
        }
        sum = block_sum_f32(sum, s_red);  // its barrier also publishes s_p
        l_run = l_run * alpha + sum;
        m_run = m_new;
        float acc[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] = 0.f;
        for (int j = kg; j < np; j += 32) {
            const float pj = s_p[j];
            float f[8];
            unpack8(*reinterpret_cast<const u32x4*>(vbase + (int64_t)token_of(p0 + j) * kD + 8 * dg), f);
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[d] = fmaf(pj, f[d], acc[d]);
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) s_acc[kg][8 * dg + d] = acc[d];
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                float t = 0.f;
                for (int g2 = 0; g2 < 32; ++g2) t += s_acc[g2][8 * dg + d];
                o_acc[d] = o_acc[d] * alpha + t;
            }
        }
        __syncthreads();
    }
    if (kg == 0) {
        const float inv = 1.f / l_run;  // the window always holds key T-1
        float* o = a.out + (int64_t)row * kD + 8 * dg;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d] = o_acc[d] * inv;
    }
}

// ------------------------------------------------------------ host side
static int decode_chunks(const Geometry& g) {
    // sized for the longest sequence the parameters allow (g.N = T <= t_max)
    const int E = eligible_blocks(g.N - 1, g.bs, g.window);
    return std::max(1, (E + DC_CHUNK - 1) / DC_CHUNK);
}

size_t decode_workspace_bytes(const Geometry& g, int t_max) {
    Geometry gm = g;
    gm.N = t_max;
    const size_t rows = (size_t)g.B * g.Hq;
    return align_up(rows * decode_chunks(gm) * kMaxTopK * 8, 256) + align_up(rows * g.top_k * 4, 256);
}

hipError_t launch_decode(const Geometry& g, int t_max, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, float* kbar, float* out, int32_t* idx_out, void* ws,
                         hipStream_t s) {
    const int rows = g.B * g.Hq;
    DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.kbar = kbar;
    a.out = out;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.T = g.N;
    a.t_max = t_max;
    a.bs = g.bs;
    a.top_k = g.top_k;
    a.window = g.window;
    a.E = eligible_blocks(g.N - 1, g.bs, g.window);
    a.nchunk = std::max(1, (a.E + DC_CHUNK - 1) / DC_CHUNK);
    a.scale_log2 = g.scale * kLog2e;
    Geometry gm = g;
    gm.N = t_max;
    char* base = static_cast<char*>(ws);
    a.keys = reinterpret_cast<uint64_t*>(base);
    a.idx = idx_out ? idx_out
                    : reinterpret_cast<int32_t*>(
                          base + align_up((size_t)rows * decode_chunks(gm) * kMaxTopK * 8, 256));
    if (g.N % g.bs == 0)  // token T-1 completes block T/bs - 1
        hipLaunchKernelGGL(k_decode_summarize, dim3((unsigned)(g.B * g.Hkv)), dim3(64), 0, s, a,
                           g.N / g.bs - 1);
    hipLaunchKernelGGL(k_decode_route_chunk, dim3((unsigned)(rows * a.nchunk)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_decode_route_merge, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a,
                       rows);
    hipLaunchKernelGGL(k_decode_attend, dim3((unsigned)rows), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
