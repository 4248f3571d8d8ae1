// Single-query decode against a key/value cache: the same content-routed
// selection and exact sparse softmax as the prefill path, for the query at
// position T-1 of a cache holding T tokens (SSA page, "Other measured
// evidence": decode steps against a growing cache at a fixed selection
// budget; selection rule as in lsa_route_topk, attention as in
// lsa_sparse_attend).
//
// A decode step is latency-bound and touches little data (per query head
// about top_k + window/bs blocks of K/V and the eligible block means), so it
// runs on the vector ALUs in fp32, in two launches with enough workgroups to
// spread the reads:
//   1. k_decode_route   per (row, chunk of 256, 512 or 1024 eligible blocks,
//                       the smallest that keeps 16 chunks per row): scores
//                       q . kbar_c and keeps the chunk's top-k keys (score,
//                       then lower index).  Extra workgroups write the mean
//                       of the block that token T-1 completes (when T is a
//                       multiple of bs) into the caller's block-mean cache;
//                       no routing of this step reads that block, which
//                       lies in the window.
//   2. k_decode_attend  per (row, split of 256 keys): merges the row's chunk
//                       lists into its top-k, then an exact softmax over its
//                       share of the routed blocks and the block-aligned
//                       window; the last split of a row to finish (a device
//                       counter) combines the row's partial (max, mass,
//                       output) triples.
// Top-k sets are found by a radix select over the 64-bit keys with wave
// ballots: the threshold is built bit by bit from the count of keys at or
// above each candidate, so no shuffles or LDS round trips are needed; the
// block-id half of the keys is searched only when scores tie at the k-th
// place.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

// Scratch of the allocation-free decode entry point (lsa_decode_noalloc): a
// file-scope device array, so every GPU the library runs on holds its own
// copy from the moment the library's code is loaded there until the process
// ends.  Host code must not use its name as an address (in host code the name
// is a host-side stand-in); static_scratch() looks the device address up.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int DC_SPLIT = 256;   // keys per attention workgroup
constexpr int kMaxBlock = 128;  // largest key block (bs)
constexpr int DC_MAXCH = 64;    // chunk lists per row (E <= nb <= 65536)

// Candidate blocks per lane of a routing wave: the smallest chunk (256, 512
// or 1024 blocks) that covers the row in at most 16 chunks, so that the
// attention step merges at most 256 keys per row; past 16384 blocks, 1024
// (at most 64 chunks, as N/bs <= 65536).  Smaller chunks spread the block
// means over more workgroups; more chunks cost the merge more than they save.
static inline int decode_kpl(int E) { return E <= 16 * 256 ? 1 : (E <= 16 * 512 ? 2 : 4); }

struct DecodeArgs {
    const uint16_t* q;   // [B*Hq][64]
    const uint16_t* k;   // [B*Hkv][t_max][64]
    const uint16_t* v;   // [B*Hkv][t_max][64]
    float* kbar;         // [B*Hkv][t_max/bs][64]
    int32_t* idx;        // [B*Hq][top_k] or NULL
    float* out;          // [B*Hq][64]
    uint64_t* keys;      // [B*Hq][nchunk][KS] chunk key sets, zero-padded (KS: see below)
    uint32_t* counters;  // [B*Hq] finished splits per row
    float* part;         // [B*Hq][nsplit][2 + 64]: max, mass, output (log2 domain)
    int rows, Hq, Hkv, T, t_max, bs, top_k, window, E, nchunk, nsplit, summ_block;
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

// ------------------------------------------------------------ wave radix select
// A threshold th such that exactly min(k, #nonzero) of the wave's nonzero
// keys are >= th (0 when fewer than k are nonzero), built from the most
// significant bit down: a bit is set when at least k keys reach the
// candidate.  The score word (high 32 bits) goes first, on 32-bit compares;
// when exactly k keys reach the k-th largest score word no lower bit can
// change the selected set, so the search stops there (score ties at the
// threshold go on through the block-id word).  Keys are distinct, so the
// full search ends at the k-th largest key itself.
template <int n>
__device__ __forceinline__ int wave_count_ge_hi(const uint64_t (&key)[n], uint32_t cand) {
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < n; ++i)
        cnt += __popcll(__builtin_amdgcn_ballot_w64((uint32_t)(key[i] >> 32) >= cand));
    return cnt;
}

template <int n>
__device__ __forceinline__ uint64_t wave_kth_key(const uint64_t (&key)[n], int k) {
    uint32_t hi = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = hi | (1u << bit);
        if (wave_count_ge_hi(key, cand) >= k) hi = cand;
    }
    if (hi == 0) return 0;  // fewer than k nonzero keys: take them all
    uint64_t th = (uint64_t)hi << 32;
    if (wave_count_ge_hi(key, hi) == k) return th;
    for (int bit = 31; bit >= 0; --bit) {
        const uint64_t cand = th | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < n; ++i) cnt += __popcll(__builtin_amdgcn_ballot_w64(key[i] >= cand));
        if (cnt >= k) th = cand;
    }
    return th;
}

// Appends the wave's keys >= th (and nonzero) to list[0..), in lane order;
// returns their number (wave-uniform).
template <int n>
__device__ __forceinline__ int wave_compact(const uint64_t (&key)[n], uint64_t th, uint64_t* list) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int base = 0;
#pragma unroll
    for (int i = 0; i < n; ++i) {
        const bool sel = key[i] != 0 && key[i] >= th;
        const uint64_t m = __builtin_amdgcn_ballot_w64(sel);
        if (sel) list[base + __popcll(m & below)] = key[i];
        base += __popcll(m);
    }
    return base;
}

// ------------------------------------------------------------ 1. routing
// Workgroup (row, chunk): fp32 scores of the chunk's eligible blocks (the dot
// product accumulated over d in order); each wave selects its top_k, then the
// first wave selects the chunk's top_k among the four wave sets.  Workgroups
// past rows * nchunk update the block-mean cache instead (one per KV head);
// workgroup 0 also clears the rows' split counters for step 2.  KS: the
// length of a chunk key set (kMaxTopK, or kMaxTopKWide for top_k above it).
template <int KPL, int KS>
__global__ __launch_bounds__(256) void k_decode_route(DecodeArgs a) {
    __shared__ float s_q[kD];
    __shared__ uint64_t s_list[4 * KS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nroute = a.rows * a.nchunk;
    if ((int)blockIdx.x >= nroute) {
        // the mean of block summ_block (tokens [c*bs, c*bs + bs)), fp64 sum,
        // one fp32 rounding, as lsa_block_summarize
        if (w != 0) return;
        const int bg = blockIdx.x - nroute, c = a.summ_block;
        const int dg = lane & 7, j0 = lane >> 3;
        const uint16_t* base = a.k + ((int64_t)bg * a.t_max + (int64_t)c * a.bs) * kD + dg * 8;
        double acc[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] = 0.0;
        // all of this lane's rows requested before any is summed (bs / 8 <= 16)
        u32x4 raw[kMaxBlock / 8];
#pragma unroll
        for (int i = 0; i < kMaxBlock / 8; ++i) {
            const int j = j0 + 8 * i;
            raw[i] = j < a.bs ? *reinterpret_cast<const u32x4*>(base + (int64_t)j * kD)
                              : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kMaxBlock / 8; ++i) {
            if (j0 + 8 * i < a.bs) {
                float f[8];
                unpack8(raw[i], f);
#pragma unroll
                for (int d = 0; d < 8; ++d) acc[d] += (double)f[d];
            }
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
        return;
    }
    if (blockIdx.x == 0)
        for (int r = tid; r < a.rows; r += 256) a.counters[r] = 0u;
    const int row = blockIdx.x / a.nchunk, ch = blockIdx.x - row * a.nchunk;
    const int h = row % a.Hq, b = row / a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    if (tid < kD) s_q[tid] = bf16_bits_to_f32(a.q[(int64_t)row * kD + tid]);
    for (int i = tid; i < 4 * KS; i += 256) s_list[i] = 0;
    __syncthreads();
    const int c0 = ch * (256 * KPL) + w * (64 * KPL);
    const float* kb = a.kbar + (int64_t)bg * (a.t_max / a.bs) * kD;
    uint64_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
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
    wave_compact(key, wave_kth_key(key, a.top_k), s_list + w * KS);
    __syncthreads();
    if (w == 0) {
        constexpr int NW = 4 * KS / 64;  // the four wave sets, one or two keys per lane
        uint64_t k1[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) k1[i] = s_list[lane + 64 * i];
        const uint64_t th = wave_kth_key(k1, a.top_k);
        uint64_t* out = a.keys + ((int64_t)row * a.nchunk + ch) * KS;
        const int n = wave_compact(k1, th, out);
        if (lane >= n && lane < KS) out[lane] = 0;  // zero-pad the set
    }
}

// The top_k of a row's chunk sets (ntot keys, lane l holding keys l, l+64,
// ...), appended to list; returns their number.
template <int NPL>
__device__ __forceinline__ int merge_chunk_sets(const uint64_t* in, int ntot, int top_k,
                                                uint64_t* list) {
    const int lane = threadIdx.x & 63;
    uint64_t kk[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int j = lane + 64 * i;
        kk[i] = j < ntot ? in[j] : 0;
    }
    return wave_compact(kk, wave_kth_key(kk, top_k), list);
}

// ------------------------------------------------------------ 2. attention
// Workgroup (row, split): wave 0 merges the row's chunk sets into its top_k
// blocks (ascending).  The keys are the routed blocks, then the window
// [bs*E, T-1], as one virtual list; this split takes keys
// [256 split, 256 split + 256): fp32 scores in log2 units, the split's
// maximum and mass, and P.V with thread (key group kg, dims 8dg..8dg+7).
// The split's (max, mass, output) goes to the workspace; the row's last
// split to finish combines them.  KS: the chunk key set length, as in step 1.
template <int KS>
__global__ __launch_bounds__(256) void k_decode_attend(DecodeArgs a) {
    __shared__ float s_q[kD];
    __shared__ float s_p[DC_SPLIT];
    __shared__ float s_red[4];
    __shared__ float s_acc[32][kD + 1];
    __shared__ uint64_t s_sel[KS];
    __shared__ int s_blk[KS];
    __shared__ int s_nused, s_last;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = blockIdx.x / a.nsplit, sp = blockIdx.x - row * a.nsplit;
    const int h = row % a.Hq, b = row / a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    const uint16_t* kbase = a.k + (int64_t)bg * a.t_max * kD;
    const uint16_t* vbase = a.v + (int64_t)bg * a.t_max * kD;
    if (tid < kD) s_q[tid] = bf16_bits_to_f32(a.q[(int64_t)row * kD + tid]) * a.scale_log2;
    if (w == 0) {
        const uint64_t* in = a.keys + (int64_t)row * a.nchunk * KS;
        const int ntot = a.nchunk * KS;  // <= DC_MAXCH * KS
        int n;
        if (ntot <= 64) n = merge_chunk_sets<1>(in, ntot, a.top_k, s_sel);
        else if (ntot <= 128) n = merge_chunk_sets<2>(in, ntot, a.top_k, s_sel);
        else if (ntot <= 256) n = merge_chunk_sets<4>(in, ntot, a.top_k, s_sel);
        else if (ntot <= 512) n = merge_chunk_sets<8>(in, ntot, a.top_k, s_sel);
        else if (KS <= kMaxTopK || ntot <= 1024) n = merge_chunk_sets<16>(in, ntot, a.top_k, s_sel);
        else n = merge_chunk_sets<32>(in, ntot, a.top_k, s_sel);
        // ascending block ids: rank of each selected id among the n
        if (lane < n) {
            const int c = (int)key_block(s_sel[lane]);
            int rank = 0;
            for (int i = 0; i < n; ++i) rank += (int)key_block(s_sel[i]) < c ? 1 : 0;
            s_blk[rank] = c;
        }
        if (lane == 0) s_nused = n;
    }
    __syncthreads();
    const int nused = s_nused;
    if (sp == 0 && a.idx && tid < a.top_k)
        a.idx[(int64_t)row * a.top_k + tid] = tid < nused ? s_blk[tid] : -1;
    const int n_routed = nused * a.bs;
    const int win0 = a.bs * a.E;
    const int total = n_routed + (a.T - win0);
    const int p0 = sp * DC_SPLIT;
    const int np = max(0, min(DC_SPLIT, total - p0));
    auto token_of = [&](int j) {
        return j < n_routed ? s_blk[j / a.bs] * a.bs + (j % a.bs) : win0 + (j - n_routed);
    };
    float s = -INFINITY;
    // this thread's V pieces for the P.V step (keys kg, kg + 32, ..., dims
    // 8dg..8dg+7), requested together with the K row so that their latency
    // overlaps the scores and the softmax reductions
    const int kg = tid >> 3, dg = tid & 7;
    u32x4 vraw[DC_SPLIT / 32];
#pragma unroll
    for (int i = 0; i < DC_SPLIT / 32; ++i) {
        const int j = kg + 32 * i;
        vraw[i] = j < np ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)token_of(p0 + j) * kD + 8 * dg)
                         : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < np) {
        const uint16_t* kr = kbase + (int64_t)token_of(p0 + tid) * kD;
        u32x4 raw[kD / 8];
#pragma unroll
        for (int d8 = 0; d8 < kD / 8; ++d8) raw[d8] = *reinterpret_cast<const u32x4*>(kr + 8 * d8);
        s = 0.f;
#pragma unroll
        for (int d8 = 0; d8 < kD / 8; ++d8) {
            float f[8];
            unpack8(raw[d8], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(s_q[8 * d8 + e], f[e], s);
        }
    }
    const float mx = block_max_f32(s, s_red);
    const float pj = tid < np ? exp2f(s - mx) : 0.f;
    s_p[tid] = pj;
    const float l = block_sum_f32(pj, s_red);  // its barriers also publish s_p
    float acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.f;
#pragma unroll
    for (int i = 0; i < DC_SPLIT / 32; ++i) {
        const int j = kg + 32 * i;
        if (j < np) {
            float f[8];
            unpack8(vraw[i], f);
            const float pv = s_p[j];
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[d] = fmaf(pv, f[d], acc[d]);
        }
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) s_acc[kg][8 * dg + d] = acc[d];
    __syncthreads();
    float* part = a.part + ((int64_t)row * a.nsplit + sp) * (2 + kD);
    if (tid < kD) {
        float t = 0.f;
        for (int g2 = 0; g2 < 32; ++g2) t += s_acc[g2][tid];
        part[2 + tid] = t;
    }
    if (tid == 0) {
        part[0] = mx;
        part[1] = l;
    }
    // the last split of the row to finish combines the row's splits
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(a.counters + row, 1u) == (uint32_t)(a.nsplit - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (tid < kD) {
        // the splits in batches of eight, each batch's partials requested
        // before any is used; running maximum with rescaling between batches
        const float* pr = a.part + (int64_t)row * a.nsplit * (2 + kD);
        float M = -INFINITY, L = 0.f, O = 0.f;
        for (int i0 = 0; i0 < a.nsplit; i0 += 8) {
            float mi[8], li[8], oi[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u;
                const bool have = i < a.nsplit;
                mi[u] = have ? pr[i * (2 + kD)] : -INFINITY;
                li[u] = have ? pr[i * (2 + kD) + 1] : 0.f;
                oi[u] = have ? pr[i * (2 + kD) + 2 + tid] : 0.f;
            }
            float mb = M;
#pragma unroll
            for (int u = 0; u < 8; ++u) mb = fmaxf(mb, mi[u]);
            const float alpha = M == -INFINITY ? 0.f : exp2f(M - mb);
            L *= alpha;
            O *= alpha;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float f = mi[u] == -INFINITY ? 0.f : exp2f(mi[u] - mb);
                L = fmaf(li[u], f, L);
                O = fmaf(oi[u], f, O);
            }
            M = mb;
        }
        a.out[(int64_t)row * kD + tid] = O / L;  // the window always holds key T-1
    }
}

// ------------------------------------------------------------ host side
struct DecodeLayout {
    size_t keys, counters, part, total;
    int nchunk, nsplit;
};

// Chunk key set length for a selection of top_k blocks.
static inline int decode_ks(int top_k) { return top_k <= kMaxTopK ? kMaxTopK : kMaxTopKWide; }

static DecodeLayout decode_layout(const Geometry& g, int t_max) {
    DecodeLayout L{};
    // sized for the longest sequence the cache allows (T <= t_max)
    const int E = eligible_blocks(t_max - 1, g.bs, g.window);
    L.nchunk = std::max(1, (E + 256 * decode_kpl(E) - 1) / (256 * decode_kpl(E)));
    L.nchunk = std::max(L.nchunk, std::min(DC_MAXCH, (E + 255) / 256));  // any T <= t_max
    // keys per row: at most top_k routed blocks plus a window of < window + bs keys
    L.nsplit = (g.top_k * g.bs + g.window + g.bs + DC_SPLIT - 1) / DC_SPLIT;
    const size_t rows = (size_t)g.B * g.Hq;
    size_t off = 0;
    L.keys = off;     off += align_up(rows * L.nchunk * decode_ks(g.top_k) * 8, 256);
    L.counters = off; off += align_up(rows * 4, 256);
    L.part = off;     off += align_up(rows * L.nsplit * (2 + kD) * 4, 256);
    L.total = off;
    return L;
}

size_t decode_workspace_bytes(const Geometry& g, int t_max) { return decode_layout(g, t_max).total; }

hipError_t static_scratch(void** ptr) {
    // one lookup per device, with that device current; the address is kept
    // for every later call on the device
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

template <int KS>
static void launch_decode_steps(int kpl, dim3 rgrid, const DecodeArgs& a, hipStream_t s) {
    switch (kpl) {
        case 1: hipLaunchKernelGGL((k_decode_route<1, KS>), rgrid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_decode_route<2, KS>), rgrid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((k_decode_route<4, KS>), rgrid, dim3(256), 0, s, a); break;
    }
    hipLaunchKernelGGL(k_decode_attend<KS>, dim3((unsigned)(a.rows * a.nsplit)), dim3(256), 0, s,
                       a);
}

hipError_t launch_decode(const Geometry& g, int t_max, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, float* kbar, float* out, int32_t* idx_out, void* ws,
                         hipStream_t s) {
    const DecodeLayout L = decode_layout(g, t_max);
    char* base = static_cast<char*>(ws);
    DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.kbar = kbar;
    a.idx = idx_out;
    a.out = out;
    a.keys = reinterpret_cast<uint64_t*>(base + L.keys);
    a.counters = reinterpret_cast<uint32_t*>(base + L.counters);
    a.part = reinterpret_cast<float*>(base + L.part);
    a.rows = g.B * g.Hq;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.T = g.N;
    a.t_max = t_max;
    a.bs = g.bs;
    a.top_k = g.top_k;
    a.window = g.window;
    a.E = eligible_blocks(g.N - 1, g.bs, g.window);
    const int kpl = decode_kpl(a.E);
    a.nchunk = std::max(1, (a.E + 256 * kpl - 1) / (256 * kpl));
    if (a.nchunk > DC_MAXCH || a.nchunk > L.nchunk)
        return hipErrorInvalidValue;  // the merge holds 64 chunk sets
    // this step's keys: at most top_k routed blocks plus the window [bs*E, T-1]
    const int keys = std::min(a.E, g.top_k) * g.bs + (g.N - g.bs * a.E);
    a.nsplit = std::max(1, (keys + DC_SPLIT - 1) / DC_SPLIT);
    a.summ_block = g.N / g.bs - 1;  // token T-1 completes this block when bs divides T
    a.scale_log2 = g.scale * kLog2e;
    const int summ_wgs = g.N % g.bs == 0 ? g.B * g.Hkv : 0;
    const dim3 rgrid((unsigned)(a.rows * a.nchunk + summ_wgs));
    if (decode_ks(g.top_k) == kMaxTopK)
        launch_decode_steps<kMaxTopK>(kpl, rgrid, a, s);
    else
        launch_decode_steps<kMaxTopKWide>(kpl, rgrid, a, s);
    return hipGetLastError();
}

}  // namespace lsa
