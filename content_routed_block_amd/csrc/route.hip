// Routing: routing scores <q, mu_c> against the block means (SSA page,
// "Algorithm and complexity", the beta = 0 score) and per-query top-k with
// ties broken toward the lower block index.
//
// Causal rows consider only complete blocks before the block-aligned window
// (SSA page, "Mathematical status" / "Known limitations": causal only once
// cut at the query position; Subquadratic Sparse Attention page, "Why the
// layer is mathematically subquadratic": completed blocks exposed only when
// their last token precedes the cutoff).  Image-mode rows are pooled query
// blocks scored against every key block (LLSA page, "Minimum Usage").
//
// Design (gfx950).  A workgroup owns 128 query rows of one (b, h): four
// waves x 32 rows.  Candidate block means stream through LDS in chunks of
// 32, split into bf16 hi + bf16 lo parts.  Scores are 32x32x16 bf16 MFMA
// tiles S^T = Kbar_chunk . Q^T, so lane l holds query l%32 and 16
// candidates whose indices fall in one residue class mod 32 per register;
// lanes l and l^32 hold the two halves of the same query's chunk.
//   pass 1  hi-only scores a_c; every lane keeps the two largest values of
//           each of its residue classes (three for top_k above 16).  Their
//           k-th largest over the lane pair, th, is reached by at least k
//           candidates' a_c; delta bounds |a_c - b_c| against the
//           fp32-accurate score b_c, so at least k candidates have
//           b_c >= th - delta.
//   pass 2  one of two forms, chosen per launch by the row length:
//           full  hi+lo scores b_c (three MFMA products with fp32 queries,
//                 two otherwise); candidates with b_c >= th - delta join
//                 the query's survivor list in LDS (capacity RT_CAP = 29,
//                 RT_CAP_WIDE = 56 for top_k above 16);
//           lean  the hi-only a_c again (one product, half the staging and
//                 one barrier per chunk); candidates with a_c >= th - 2
//                 delta join the list, and each survivor's b_c = a_c +
//                 q . lo_c is then formed with bf16 dot products
//                 (v_dot2c_f32_bf16) over rows of the lo split read from
//                 L2, the lane pair splitting the 64 dims.
//           Either way every member of the exact top k survives.  The lean
//           form saves a third of the MFMA work per candidate but pays a
//           fixed, latency-bound rescoring per row, so it pays off only for
//           long rows (kRouteLeanMinCand candidates and more) of bf16
//           queries.
//   select  each lane of the pair ranks the survivors it found in a
//           16-entry (top_k above 16: 32-entry) sorted list of 64-bit keys
//           (score b_c, then lower index); the two lists are merged and the
//           chosen block ids written in ascending order.
// Queries whose survivor list overflows (ties on many blocks, adversarial
// inputs) are queued, and so is each workgroup holding one.  Up to FB_ROWS
// such rows are redone one by one by k_route_fallback.  With more, the
// queued workgroups rerun as k_route<.., EXACT = true>: the same scores,
// no threshold pass, and each lane keeps its 16 (32) best 64-bit keys, with
// no capacity to overflow.
//
// Consensus routing (one route per KV group, scored by the sum of the
// group's query heads' scores; SSA page, "Complete 10M transformer result")
// runs the same kernels over the group rows, with the group's summed query
// formed in fp32 by k_group_query and fed as a hi + lo bf16 pair like the
// pooled image-mode query.
#include <math.h>

#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

constexpr int RT_ROWS = 128;   // query rows per workgroup (4 waves x 32)
constexpr int RT_CH = 32;      // candidates per step
constexpr int RT_CAP = 29;     // survivor slots per query (five workgroups still fit a CU)
constexpr int RT_CAP_WIDE = 56;  // the same for top_k 17..32 (three workgroups per CU)
constexpr int RT_PITCH = 72;   // LDS row pitch of staged candidates (bf16), conflict-free
constexpr int FB_GRID = 1024;   // workgroups of the per-row exact pass (one row at a time)
constexpr int FB_ROWS = 16384;  // rows it takes; above this the queued tiles are redone whole
// the lean pass 2 is used when a row can have this many candidates
constexpr int kRouteLeanMinCand = 4096;

struct RouteArgs {
    const uint16_t* q;    // bf16 queries [B,Hq,N,64] (QF32 = false)
    const float* qbar;    // fp32 queries [B,Hq,P,64] (QF32 = true: pooled, or group sums)
    const float* kbar;    // [B,Hkv,nb,64]
    const uint16_t* khi;  // bf16 hi part of kbar [B*Hkv][nb_pad][64]
    const uint16_t* klo;  // bf16 lo part (kbar - hi) [B*Hkv][nb_pad][64]
    const float* ckn;     // per chunk of RT_CH blocks: max over its blocks of |kbar_c|, as
                          // kChunkMaxSlots partial maxima per chunk line [B*Hkv][ncb]
    const float* clo;     // the same for |lo_c| (lo = kbar - hi) [B*Hkv][ncb]
    int32_t* idx;         // [B,Hq,P,top_k] (Hq = routed heads: Hkv with consensus)
    uint32_t* ovf_count;  // queued overflow rows
    uint32_t* ovf_rows;   // [B*Hq*P]
    uint32_t* tile_count; // queued tiles (workgroups with an overflowing row)
    uint32_t* tile_queue; // [items]
    int Hq, Hkv, N, bs, nb, top_k, window;
    int P;       // rows per (b, h): N (causal) or nb (image)
    int tiles;   // ceil(P / RT_ROWS)
    int items;   // B * Hq * tiles
    int nb_pad;  // nb rounded up to a multiple of RT_CH
    int ncb;     // nb_pad / RT_CH
    int cshift;      // causal candidates are E(t) >> cshift (two-level routing: nodes of 16 blocks)
    int idx_stride;  // idx row stride (>= top_k)
    int tail_img;    // image-mode two-level routing: every row's tail node (-1: none)
};

// ------------------------------------------------------------ sorting networks
template <int N>
__device__ __forceinline__ void bitonic_sort_desc(float* v) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    const float a = v[i], b = v[j];
                    const float mx = fmaxf(a, b), mn = fminf(a, b);
                    if ((i & size) == 0) { v[i] = mx; v[j] = mn; }
                    else { v[i] = mn; v[j] = mx; }
                }
            }
}

template <int N>
__device__ __forceinline__ void bitonic_merge_desc(float* v) {
#pragma unroll
    for (int stride = N >> 1; stride > 0; stride >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int j = i ^ stride;
            if (j > i) {
                const float a = v[i], b = v[j];
                v[i] = fmaxf(a, b);
                v[j] = fminf(a, b);
            }
        }
}

template <int N>
__device__ __forceinline__ void bitonic_sort_asc_u32(uint32_t* v) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    const uint32_t a = v[i], b = v[j];
                    const uint32_t mx = a > b ? a : b, mn = a > b ? b : a;
                    if ((i & size) == 0) { v[i] = mn; v[j] = mx; }
                    else { v[i] = mx; v[j] = mn; }
                }
            }
}

// Sorts KM (16 or 32) 64-bit keys into descending order.
template <int KM>
__device__ __forceinline__ void bitonic_sort_desc_u64(uint64_t (&v)[KM]) {
#pragma unroll
    for (int size = 2; size <= KM; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < KM; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    const uint64_t a = v[i], b = v[j];
                    const bool desc = (i & size) == 0;
                    const bool swap = desc ? a < b : a > b;
                    v[i] = swap ? b : a;
                    v[j] = swap ? a : b;
                }
            }
}

// k-th largest (1 <= k <= 16) of the 64 values held as the per-class
// largest (m1) and second largest (m2) values of 16 classes in this lane and
// 16 more classes in lane ^ 32.  Both lanes of the pair return the same value.
__device__ __forceinline__ float kth_largest_top2_pair(float (&m1)[16], float (&m2)[16], int k) {
    bitonic_sort_desc<16>(m1);
    bitonic_sort_desc<16>(m2);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = fmaxf(m1[i], m2[15 - i]);  // top 16 of the 32, bitonic
    bitonic_merge_desc<16>(v);
    float w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float other = __shfl_xor(v[15 - i], 32, kWave);
        w[i] = fmaxf(v[i], other);  // top 16 of the pair's 64, bitonic
    }
    bitonic_merge_desc<16>(w);
    float r = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i == k - 1) r = w[i];
    return r;
}

// k-th largest (1 <= k <= 32) of the 96 values held as the three largest
// values (m1 >= m2 >= m3) of 16 classes in this lane and 16 more classes in
// lane ^ 32.  Both lanes of the pair return the same value.
__device__ __forceinline__ float kth_largest_top3_pair(float (&m1)[16], float (&m2)[16],
                                                       float (&m3)[16], int k) {
    bitonic_sort_desc<16>(m1);
    bitonic_sort_desc<16>(m2);
    bitonic_sort_desc<16>(m3);
    // top 32 of m1 and m2: m1 descending then m2 ascending is bitonic
    float v[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[i] = m1[i];
        v[16 + i] = m2[15 - i];
    }
    bitonic_merge_desc<32>(v);
    // top 32 of those and m3 (padded with -inf), bitonic, then sorted
#pragma unroll
    for (int i = 16; i < 32; ++i) v[i] = fmaxf(v[i], m3[31 - i]);
    bitonic_merge_desc<32>(v);
    // top 32 of the pair's two lists
    float w[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = fmaxf(v[i], __shfl_xor(v[31 - i], 32, kWave));
    bitonic_merge_desc<32>(w);
    float r = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        if (i == k - 1) r = w[i];
    return r;
}

// Bitonic merge of KM (16 or 32) 64-bit keys into descending order.
template <int KM>
__device__ __forceinline__ void bitonic_merge_desc_u64(uint64_t (&v)[KM]) {
#pragma unroll
    for (int stride = KM >> 1; stride > 0; stride >>= 1)
#pragma unroll
        for (int i = 0; i < KM; ++i) {
            const int j = i ^ stride;
            if (j > i) {
                const uint64_t a = v[i], b = v[j];
                const bool gt = a > b;
                v[i] = gt ? a : b;
                v[j] = gt ? b : a;
            }
        }
}

template <int KM>
__device__ __forceinline__ void insert_key(uint64_t (&L)[KM], uint64_t x) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        const uint64_t a = L[j];
        const bool gt = x > a;
        L[j] = gt ? x : a;
        x = gt ? a : x;
    }
}

// Writes one idx row (row stride `stride`) from a key list sorted by rank
// (m valid keys).
template <int KM>
__device__ __forceinline__ void write_selection(int32_t* out, const uint64_t (&L)[KM],
                                                int m, int top_k, int stride) {
    uint32_t cs[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) cs[j] = j < m ? key_block(L[j]) : 0xFFFFFFFFu;
    bitonic_sort_asc_u32<KM>(cs);
    if (((top_k | stride) & 3) == 0) {  // 16-byte stores (rows are 16-byte aligned)
        typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int j4 = 0; j4 < KM / 4; ++j4) {
            if (4 * j4 < top_k) {
                i32x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = 4 * j4 + r < m ? (int32_t)cs[4 * j4 + r] : -1;
                *reinterpret_cast<i32x4*>(out + 4 * j4) = v;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < top_k) out[j] = j < m ? (int32_t)cs[j] : -1;
    }
}

// Two-level routing's tail slot of causal row t: the partial node (fewer
// than kTreeFanout eligible blocks) that every row keeps after its beam, or
// -1 when the eligible blocks fill whole nodes.
__device__ __forceinline__ int tail_node(int t, int bs, int window) {
    const int E = eligible_blocks(t, bs, window);
    const int S = E >> kTreeFanoutLog2;
    return (S << kTreeFanoutLog2) < E ? S : -1;
}

// ------------------------------------------------------------ preparation
// One thread per (block row, 8 dims): bf16 hi/lo split of the block means
// (rows padded to a multiple of 32 with zeros), and per chunk of 32 rows
// (one workgroup) the largest norms |kbar_c| and |lo_c| of its valid rows,
// in slot 0 of the chunk's line (the other slots zeroed).
__global__ __launch_bounds__(256) void k_route_prep(const float* __restrict__ kbar,
                                                    uint16_t* __restrict__ khi,
                                                    uint16_t* __restrict__ klo,
                                                    float* __restrict__ ckn,
                                                    float* __restrict__ clo, int n_bg, int nb,
                                                    int nb_pad) {
    __shared__ float s_n[2][4];
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid >> 3;  // over n_bg * nb_pad rows: 32 per workgroup, one chunk
    const bool in = row < (int64_t)n_bg * nb_pad;
    const int bg = (int)(row / nb_pad), c = (int)(row - (int64_t)bg * nb_pad);
    const int d0 = (threadIdx.x & 7) * 8;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in && c < nb) {
        const float* src = kbar + ((int64_t)bg * nb + c) * kD + d0;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    }
    float kn = 0.f, ln = 0.f;
    if (in) route_split_store(f, khi + row * kD + d0, klo + row * kD + d0, kn, ln);
    kn = wave_max_nonneg(in ? kn : 0.f);  // padding rows hold zeros
    ln = wave_max_nonneg(in ? ln : 0.f);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_n[0][w] = kn;
        s_n[1][w] = ln;
    }
    __syncthreads();
    if (threadIdx.x < kChunkMaxSlots && (int64_t)blockIdx.x * 32 < (int64_t)n_bg * nb_pad) {
        const int64_t chunk = (int64_t)blockIdx.x;  // = bg * (nb_pad / 32) + c / 32
        const bool first = threadIdx.x == 0;
        ckn[chunk * kChunkMaxStride + threadIdx.x] =
            first ? fmaxf(fmaxf(s_n[0][0], s_n[0][1]), fmaxf(s_n[0][2], s_n[0][3])) : 0.f;
        clo[chunk * kChunkMaxStride + threadIdx.x] =
            first ? fmaxf(fmaxf(s_n[1][0], s_n[1][1]), fmaxf(s_n[1][2], s_n[1][3])) : 0.f;
    }
}

__device__ __forceinline__ int row_candidates(bool causal, int row, int P, int bs, int window,
                                              int nb, int cshift) {
    if (row >= P) return 0;
    return causal ? eligible_blocks(row, bs, window) >> cshift : nb;
}

// Staging of one chunk (32 candidate rows x 64 dims, bf16) through LDS:
// thread tid carries row tid/8, dims 8*(tid%8) .. +7 (16 bytes).
__device__ __forceinline__ u32x4 stage_load(const uint16_t* base, int cb, int tid) {
    return *reinterpret_cast<const u32x4*>(base + (int64_t)(cb + (tid >> 3)) * kD + (tid & 7) * 8);
}
__device__ __forceinline__ void stage_store(__bf16* buf, int tid, u32x4 v) {
    *reinterpret_cast<u32x4*>(buf + (tid >> 3) * RT_PITCH + (tid & 7) * 8) = v;
}
// A operands of one step: rows l%32, dims 8*half + 16*ks.
__device__ __forceinline__ void read_cands(const __bf16* buf, int l32, int half, bf16x8 (&A)[4]) {
    const __bf16* p = buf + l32 * RT_PITCH + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) A[ks] = *reinterpret_cast<const bf16x8*>(p + 16 * ks);
}

// acc + sum of the eight products a_i * b_i of two rows of 8 bf16, fp32
// accumulation (v_dot2c_f32_bf16, two products per step).  The pairs are
// taken with vector shuffles: a bit cast of one 32-bit element of a u32x4
// to bf16x2 inside an unrolled loop is compiled to element 0 every time.
__device__ __forceinline__ float dot8_bf16(bf16x8 a, bf16x8 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1),
                                          __builtin_shufflevector(b, b, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3),
                                          __builtin_shufflevector(b, b, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5),
                                          __builtin_shufflevector(b, b, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7),
                                          __builtin_shufflevector(b, b, 6, 7), acc, false);
    return acc;
}

// min(max(x, lo), hi) for lo <= hi in one instruction.
__device__ __forceinline__ int clamp_i32(int x, int lo, int hi) {
    int r;
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(lo), "v"(hi));
    return r;
}

// ------------------------------------------------------------ wave maxima
// Largest 32-bit value of the wave, in every lane: quad swaps, the half-row
// and row mirrors (DPP, folded into the max), then the 16- and 32-lane
// swaps, all in registers.
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t x) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
    return o > x ? o : x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max_dpp_u32<0xB1>(x);   // quad_perm(1,0,3,2): lane ^ 1
    x = max_dpp_u32<0x4E>(x);   // quad_perm(2,3,0,1): lane ^ 2
    x = max_dpp_u32<0x141>(x);  // row_half_mirror: the other quad of the 8
    x = max_dpp_u32<0x140>(x);  // row_mirror: the other 8 of the row
    // each swap leaves a lane its own value and its partner's, in some order
    const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = s16[0] > s16[1] ? s16[0] : s16[1];
    const auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return s32[0] > s32[1] ? s32[0] : s32[1];
}

// ------------------------------------------------------------ main kernel
// Each wave is independent (its own 32 rows and survivor lists); the
// workgroup only shares the staged candidate chunks.
// KM: the selection list length, kMaxTopK for top_k <= 16 or kMaxTopKWide
// for top_k 17..32.  The wide form keeps the three largest values per class
// in pass 1 (so that its threshold stays close to the k-th score) and
// RT_CAP_WIDE survivor slots per query, at three workgroups per CU.
template <bool CAUSAL, bool QF32, bool EXACT, bool LEAN, int KM = kMaxTopK>
__global__ __launch_bounds__(256, EXACT ? 2 : (KM > kMaxTopK ? 3 : (QF32 ? 4 : 5)))
void k_route(RouteArgs a) {
    static_assert(!(EXACT && LEAN), "the whole-tile exact pass scores b_c directly");
    static_assert(!(QF32 && LEAN), "fp32 queries take the full form");
    constexpr bool WIDE = KM > kMaxTopK;
    constexpr int CAP = WIDE ? RT_CAP_WIDE : RT_CAP;
    // candidate staging: pass 1 double-buffers the hi parts in s_stage[0..1];
    // pass 2 holds one chunk's hi part in s_stage[0] and lo part in
    // s_stage[1] (two barriers per chunk), which keeps the workgroup's LDS
    // small enough for five workgroups per CU (bf16 queries; the fp32-query
    // variant needs more registers and runs four)
    __shared__ __attribute__((aligned(16))) __bf16 s_stage[2][RT_CH * RT_PITCH];
    // survivor lists, slot-major ([slot][row]) so that the lanes of a wave
    // touch consecutive words
    // (scores: CAP*RT_ROWS floats, then the block ids as uint16)
    __shared__ __attribute__((aligned(16))) char s_list[CAP * RT_ROWS * 6];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int half = lane >> 5, l32 = lane & 31;
    // Items in workgroup order: workgroups are dealt round-robin to the 8
    // XCDs, so each XCD takes every 8th tile of every head, the same mix of
    // heavy and light tiles (a contiguous range per XCD left the busiest
    // XCD ~10% more candidates than the mean), and at any time all XCDs
    // work on the same heads, whose KV group's block means their L2s hold.
    // Tiles of a head run heavy (late positions, most candidates) first.
    int item;
    if constexpr (EXACT) {
        // the queued tiles, when more rows overflowed than the per-row pass takes
        if (__builtin_amdgcn_readfirstlane(*a.ovf_count) <= (uint32_t)FB_ROWS) return;
        if (blockIdx.x >= __builtin_amdgcn_readfirstlane(*a.tile_count)) return;
        item = (int)__builtin_amdgcn_readfirstlane(a.tile_queue[blockIdx.x]);
    } else {
        item = blockIdx.x;
        if (item >= a.items) return;
    }
    __shared__ uint32_t s_ovf;  // some row of the workgroup overflowed
    if (tid == 0) s_ovf = 0u;   // read after the passes' barriers
    const int bh = item / a.tiles;
    const int tile = a.tiles - 1 - (item - bh * a.tiles);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    const int P = a.P;
    const int r0 = tile * RT_ROWS + 32 * w;  // first row of this wave
    const uint16_t* khi = a.khi + (int64_t)bg * a.nb_pad * kD;
    const uint16_t* klo = a.klo + (int64_t)bg * a.nb_pad * kD;

    const int rq = r0 + l32;
    const int Erow = row_candidates(CAUSAL, rq, P, a.bs, a.window, a.nb, a.cshift);
    const int Emax =
        r0 < P ? row_candidates(CAUSAL, min(r0 + 31, P - 1), P, a.bs, a.window, a.nb, a.cshift) : 0;
    const int wg_last = min(tile * RT_ROWS + RT_ROWS, P) - 1;
    const int Ewg = row_candidates(CAUSAL, wg_last, P, a.bs, a.window, a.nb, a.cshift);  // loop bound
    const int Emin =
        (r0 + 31 < P) ? row_candidates(CAUSAL, r0, P, a.bs, a.window, a.nb, a.cshift) : 0;
    // the largest |kbar_c| and |lo_c| over the wave's candidates (chunk
    // maxima over c < Emax, rounded up to whole chunks); requested now,
    // reduced after pass 1
    uint32_t kn_bits = 0u, lo_bits = 0u;  // norms are >= 0: their bits order as integers
    if constexpr (!EXACT) {
        const int nc = (Emax + RT_CH - 1) / RT_CH;
        for (int i = lane; i < nc; i += 64) {
            // the chunk's partial maxima (kChunkMaxSlots = 8 of them)
            const int64_t e = ((int64_t)bg * a.ncb + i) * kChunkMaxStride;
            static_assert(kChunkMaxSlots == 8, "two 16-byte loads per chunk line");
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 kb = *reinterpret_cast<const u32x4*>(a.ckn + e + 4 * h);
                const u32x4 lb = *reinterpret_cast<const u32x4*>(a.clo + e + 4 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kn_bits = kb[j] > kn_bits ? kb[j] : kn_bits;
                    lo_bits = lb[j] > lo_bits ? lb[j] : lo_bits;
                }
            }
        }
    }

    // ---- the query as the B operand (B[d][t] = Q[t][d]): lane holds dims
    // 8*half + 16*ks .. +7 of row rq.
    bf16x8 Bq[4];
    bf16x8 Bql[4];  // fp32 queries: the lo part
    float qn, qln;
    {
        float s2 = 0.f, l2 = 0.f;
        if (rq < P) {
            if (!QF32) {
                const uint16_t* qp = a.q + ((int64_t)bh * a.N + rq) * kD + 8 * half;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
                    float f[8];
                    unpack8(raw, f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) s2 = fmaf(f[i], f[i], s2);
                    Bq[ks] = __builtin_bit_cast(bf16x8, raw);
                    Bql[ks] = bf16x8{};
                }
            } else {
                const float* qp = a.qbar + ((int64_t)bh * P + rq) * kD + 8 * half;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(qp + 16 * ks);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(qp + 16 * ks + 4);
                    const float f[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const __bf16 hi = (__bf16)f[i];
                        const __bf16 lo = (__bf16)(f[i] - (float)hi);
                        Bq[ks][i] = hi;
                        Bql[ks][i] = lo;
                        const float hf = (float)hi, lf = (float)lo;
                        s2 = fmaf(hf, hf, s2);
                        l2 = fmaf(lf, lf, l2);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Bq[ks] = bf16x8{};
                Bql[ks] = bf16x8{};
            }
        }
        s2 += __shfl_xor(s2, 32, kWave);
        l2 += __shfl_xor(l2, 32, kWave);
        qn = sqrtf(s2);
        qln = sqrtf(l2);
    }

    // ---- pass 1: hi-only scores, two (wide form: three) largest per
    // residue class.  Chunks below Efull are candidates of every row of the
    // wave (no mask).
    const int Efull = (Emin / RT_CH) * RT_CH;
    float m1[16], m2[16], m3[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        m1[r] = -INFINITY;
        m2[r] = -INFINITY;
        m3[r] = -INFINITY;
    }
    const int nch = (Ewg + RT_CH - 1) / RT_CH;  // chunks of the workgroup
    if constexpr (!EXACT) {  // the whole-tile exact pass keeps every candidate it needs
        // chunk j is staged in buffer j&1, one barrier per chunk; the global
        // loads run two chunks ahead in two register sets (the loop body is
        // written twice so that the sets swap roles without copies)
        u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = r0;
        if (nch > 0) {
            r0 = stage_load(khi, 0, tid);
            stage_store(s_stage[0], tid, r0);
        }
        if (nch > 1) r1 = stage_load(khi, RT_CH, tid);
        __syncthreads();
        auto body = [&](int j, u32x4& r_issue, const u32x4& r_store) {
            const int cb = j * RT_CH;
            if (j + 2 < nch) r_issue = stage_load(khi, cb + 2 * RT_CH, tid);
            if (cb < Emax) {
                bf16x8 A[4];
                read_cands(s_stage[j & 1], l32, half, A);
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma32(A[ks], Bq[ks], acc);
                if (cb >= Efull) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int c = cb + 8 * (r >> 2) + 4 * half + (r & 3);
                        acc[r] = c < Erow ? acc[r] : -INFINITY;
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // m1 >= m2 >= m3, so each new lower rank is a median
                    if constexpr (WIDE) m3[r] = __builtin_amdgcn_fmed3f(m2[r], m3[r], acc[r]);
                    m2[r] = __builtin_amdgcn_fmed3f(m1[r], m2[r], acc[r]);
                    m1[r] = fmaxf(m1[r], acc[r]);
                }
            }
            if (j + 1 < nch) stage_store(s_stage[(j + 1) & 1], tid, r_store);
            __syncthreads();
        };
        for (int j = 0; j < nch; j += 2) {
            body(j, r0, r1);
            if (j + 1 < nch) body(j + 1, r1, r0);
        }
    }

    // threshold: k-th largest class top-2 value minus delta (full: tested on
    // b_c) or twice delta (lean: tested on a_c), delta >= |a_c - b_c| =
    // |q_hi . k_lo + q_lo . k_hi| + rounding (Cauchy-Schwarz with the chunk
    // maxima of |kbar_c| and |lo_c|; the second term covers fp32
    // accumulation in the MFMA and the dot products)
    float theta = -INFINITY;
    if constexpr (!EXACT) {
        const float kn_max = __uint_as_float(wave_max_u32(kn_bits));
        const float lo_max = __uint_as_float(wave_max_u32(lo_bits));
        float th;
        if constexpr (WIDE) th = kth_largest_top3_pair(m1, m2, m3, a.top_k);
        else th = kth_largest_top2_pair(m1, m2, a.top_k);
        const float delta = 1.0625f * (qn * lo_max + qln * kn_max) + 6.2e-5f * (qn + qln) * kn_max;
        theta = th - (LEAN ? 2.f : 1.f) * delta;  // -inf stays -inf
    }

    // ---- pass 2: survivors to the row's LDS list.  The lane pair (l, l^32)
    // shares a row's list: half 0 fills it upward from slot 0, half 1
    // downward from slot CAP-1; slots are clamped to the list, so an
    // overflowing list stays in bounds (the row is then redone exactly).
    const int qrow = 32 * w + l32;  // row within the workgroup
    // whole-tile exact pass: each lane's KM best selection keys, descending
    uint64_t Lk[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) Lk[j] = 0;
    // list position kept as the byte offset of the score slot; the block
    // id of slot e sits at byte LIST_IDX + e/2
    constexpr int LIST_IDX = CAP * RT_ROWS * 4;
    const int step = half ? -RT_ROWS * 4 : RT_ROWS * 4;
    const int at_lo = qrow * 4, at_hi = ((CAP - 1) * RT_ROWS + qrow) * 4;
    int at = half ? at_hi : at_lo;
    // appends the chunk's scores at or above theta (masked to the row's
    // candidates in chunks past Efull); cl0 = first candidate of this lane
    auto append_survivors = [&](const f32x16& acc, int cb, int cl0) {
        if (cb < Efull) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (acc[r] >= theta) {
                    const int e = clamp_i32(at, at_lo, at_hi);
                    *reinterpret_cast<float*>(s_list + e) = acc[r];
                    *reinterpret_cast<uint16_t*>(s_list + LIST_IDX + (e >> 1)) =
                        (uint16_t)(cl0 + 8 * (r >> 2) + (r & 3));
                    at += step;
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = cl0 + 8 * (r >> 2) + (r & 3);
                if (acc[r] >= theta && c < Erow) {
                    const int e = clamp_i32(at, at_lo, at_hi);
                    *reinterpret_cast<float*>(s_list + e) = acc[r];
                    *reinterpret_cast<uint16_t*>(s_list + LIST_IDX + (e >> 1)) = (uint16_t)c;
                    at += step;
                }
            }
        }
    };
    if constexpr (EXACT || !LEAN) {
        // hi+lo scores b_c (one chunk's hi part in s_stage[0] and lo part in
        // s_stage[1], two barriers per chunk)
        u32x4 h0 = {0u, 0u, 0u, 0u}, l0 = h0, h1 = h0, l1 = h0;
        if (nch > 0) {
            h0 = stage_load(khi, 0, tid);
            l0 = stage_load(klo, 0, tid);
            stage_store(s_stage[0], tid, h0);
            stage_store(s_stage[1], tid, l0);
        }
        if (nch > 1) {
            h1 = stage_load(khi, RT_CH, tid);
            l1 = stage_load(klo, RT_CH, tid);
        }
        __syncthreads();
        auto body = [&](int j, u32x4& hi_issue, u32x4& lo_issue, const u32x4& hi_store,
                        const u32x4& lo_store) {
            const int cb = j * RT_CH;
            if (j + 2 < nch) {
                hi_issue = stage_load(khi, cb + 2 * RT_CH, tid);
                lo_issue = stage_load(klo, cb + 2 * RT_CH, tid);
            }
            if (cb < Emax) {
                bf16x8 ch[4], cl[4];
                read_cands(s_stage[0], l32, half, ch);
                read_cands(s_stage[1], l32, half, cl);
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    acc = mfma32(ch[ks], Bq[ks], acc);
                    acc = mfma32(cl[ks], Bq[ks], acc);
                    if (QF32) acc = mfma32(ch[ks], Bql[ks], acc);
                }
                const int cl0 = cb + 4 * half;
                if constexpr (EXACT) {
                    // 64-bit keys carry the tie-break (lower block) themselves
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int c = cl0 + 8 * (r >> 2) + (r & 3);
                        const uint64_t key = sel_key(acc[r], (uint32_t)c);
                        if (c < Erow && key > Lk[KM - 1]) insert_key(Lk, key);
                    }
                } else {
                    append_survivors(acc, cb, cl0);
                }
            }
            __syncthreads();  // every wave is done with chunk j
            if (j + 1 < nch) {
                stage_store(s_stage[0], tid, hi_store);
                stage_store(s_stage[1], tid, lo_store);
            }
            __syncthreads();
        };
        for (int j = 0; j < nch; j += 2) {
            body(j, h0, l0, h1, l1);
            if (j + 1 < nch) body(j + 1, h1, l1, h0, l0);
        }
    } else {
        // lean: hi-only scores a_c, staged and double-buffered as in pass 1
        u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = r0;
        if (nch > 0) {
            r0 = stage_load(khi, 0, tid);
            stage_store(s_stage[0], tid, r0);
        }
        if (nch > 1) r1 = stage_load(khi, RT_CH, tid);
        __syncthreads();
        auto body = [&](int j, u32x4& r_issue, const u32x4& r_store) {
            const int cb = j * RT_CH;
            if (j + 2 < nch) r_issue = stage_load(khi, cb + 2 * RT_CH, tid);
            if (cb < Emax) {
                bf16x8 A[4];
                read_cands(s_stage[j & 1], l32, half, A);
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma32(A[ks], Bq[ks], acc);
                append_survivors(acc, cb, cb + 4 * half);
            }
            if (j + 1 < nch) stage_store(s_stage[(j + 1) & 1], tid, r_store);
            __syncthreads();
        };
        for (int j = 0; j < nch; j += 2) {
            body(j, r0, r1);
            if (j + 1 < nch) body(j + 1, r1, r0);
        }
    }

    // ---- selection: each lane of the pair ranks the survivors it found,
    // then the pair merges its two sorted lists.
    const int64_t out_row = (int64_t)bh * P + rq;
    if constexpr (EXACT) {
        // the pair's lists hold disjoint candidates and merge in one
        // bitonic step
        uint64_t Mx[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            const uint64_t o = Lk[KM - 1 - j];
            const uint32_t olo = __shfl_xor((uint32_t)o, 32, kWave);
            const uint32_t ohi = __shfl_xor((uint32_t)(o >> 32), 32, kWave);
            const uint64_t other = ((uint64_t)ohi << 32) | olo;
            Mx[j] = Lk[j] > other ? Lk[j] : other;
        }
        bitonic_merge_desc_u64(Mx);
        if (rq < P && half == 0) {
            int m = 0;
#pragma unroll
            for (int j = 0; j < KM; ++j) m += (j < a.top_k && Mx[j] != 0ull) ? 1 : 0;
            write_selection(a.idx + out_row * a.idx_stride, Mx, m, a.top_k, a.idx_stride);
            if (a.idx_stride > a.top_k)
                a.idx[out_row * a.idx_stride + a.top_k] =
                    CAUSAL ? tail_node(rq, a.bs, a.window) : a.tail_img;
        }
        return;
    }
    const int n_mine = (half ? at_hi - at : at - at_lo) / (RT_ROWS * 4);
    const int n_pair = n_mine + __shfl_xor(n_mine, 32, kWave);
    // a workgroup with an overflowing row queues its tile once, for the
    // whole-tile exact pass that runs when many rows overflow
    if (rq < P && n_pair > CAP && half == 0) s_ovf = 1u;
    __syncthreads();
    if (tid == 0 && s_ovf != 0u) a.tile_queue[atomicAdd(a.tile_count, 1u)] = (uint32_t)item;
    if (rq >= P) return;
    if (n_pair > CAP) {
        if (half == 0) {
            const uint32_t slot = atomicAdd(a.ovf_count, 1u);
            a.ovf_rows[slot] = (uint32_t)out_row;
        }
        return;
    }
    // lean form (bf16 queries): exact scores of the survivors, b_c = a_c +
    // q . lo_c.  Step i takes half 0's i-th
    // entry (A) and half 1's i-th entry (B); each lane forms the correction
    // over its 32 dims for both, and the partner's half of its own entry
    // arrives by one cross-half swap.  Both lanes of a pair run the same
    // trip count.  The scattered row loads dominate a step; loading the
    // next step's rows ahead measured slower, as the extra registers cost a
    // workgroup per CU.
    if constexpr (LEAN) {
        const int n_oth = __shfl_xor(n_mine, 32, kWave);
        const int nA = half ? n_oth : n_mine, nB = half ? n_mine : n_oth;
        const int trips = nA > nB ? nA : nB;
        const int dim0 = 8 * half;
        // an empty entry reads block 0 (a valid row) and is discarded
        auto fetch = [&](int i, bf16x8 (&vA)[4], bf16x8 (&vB)[4]) {
            const int eA = at_lo + i * RT_ROWS * 4;
            const int eB = at_lo + (CAP - 1 - i) * RT_ROWS * 4;
            const int cA = i < nA ? *reinterpret_cast<const uint16_t*>(s_list + LIST_IDX + (eA >> 1)) : 0;
            const int cB = i < nB ? *reinterpret_cast<const uint16_t*>(s_list + LIST_IDX + (eB >> 1)) : 0;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                vA[ks] = load_bf16x8(klo + (int64_t)cA * kD + dim0 + 16 * ks);
                vB[ks] = load_bf16x8(klo + (int64_t)cB * kD + dim0 + 16 * ks);
            }
        };
        auto apply = [&](int i, const bf16x8 (&vA)[4], const bf16x8 (&vB)[4]) {
            float pA = 0.f, pB = 0.f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                pA = dot8_bf16(Bq[ks], vA[ks], pA);
                pB = dot8_bf16(Bq[ks], vB[ks], pB);
            }
            const float other = __shfl_xor(half ? pA : pB, 32, kWave);
            if (i < n_mine) {
                const int e = at_lo + (half ? CAP - 1 - i : i) * RT_ROWS * 4;
                float* sp = reinterpret_cast<float*>(s_list + e);
                *sp = *sp + ((half ? pB : pA) + other);
            }
        };
        bf16x8 xA[4], xB[4];
        for (int i = 0; i < trips; ++i) {
            fetch(i, xA, xB);
            apply(i, xA, xB);
        }
    }
    uint64_t L[KM];
    if (__builtin_amdgcn_ballot_w64(n_mine > KM) == 0) {
        // every lane found at most KM: read them all at once (slots past
        // n_mine hold stale values and become the zero key) and sort
#pragma unroll
        for (int i = 0; i < KM; ++i) {
            const int e = at_lo + (half ? CAP - 1 - i : i) * RT_ROWS * 4;
            const uint64_t key = sel_key(*reinterpret_cast<const float*>(s_list + e),
                                         *reinterpret_cast<const uint16_t*>(s_list + LIST_IDX + (e >> 1)));
            L[i] = i < n_mine ? key : 0;
        }
        bitonic_sort_desc_u64(L);
    } else {
#pragma unroll
        for (int j = 0; j < KM; ++j) L[j] = 0;
        for (int i = 0; i < n_mine; ++i) {
            const int e = at_lo + (half ? CAP - 1 - i : i) * RT_ROWS * 4;
            insert_key(L, sel_key(*reinterpret_cast<const float*>(s_list + e),
                                  *reinterpret_cast<const uint16_t*>(s_list + LIST_IDX + (e >> 1))));
        }
    }
    uint64_t M[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        const uint64_t o = L[KM - 1 - j];
        const uint32_t olo = __shfl_xor((uint32_t)o, 32, kWave);
        const uint32_t ohi = __shfl_xor((uint32_t)(o >> 32), 32, kWave);
        const uint64_t other = ((uint64_t)ohi << 32) | olo;
        M[j] = L[j] > other ? L[j] : other;  // top 16 of the pair, bitonic
    }
    bitonic_merge_desc_u64(M);
    if (half == 0) {
        const int m = n_pair < a.top_k ? n_pair : a.top_k;
        write_selection(a.idx + out_row * a.idx_stride, M, m, a.top_k, a.idx_stride);
        // two-level routing (rows of beam + 1 slots): the tail node, written
        // beside the row's other slots
        if (a.idx_stride > a.top_k)
            a.idx[out_row * a.idx_stride + a.top_k] =
                CAUSAL ? tail_node(rq, a.bs, a.window) : a.tail_img;
    }
}

// ------------------------------------------------------------ exact fallback
// The wave's KM largest keys, descending (0 past the last), from per-lane
// lists sorted descending; the lists are consumed.  Rank r takes the largest
// score word over the lanes' heads, then the largest id word among the heads
// with that score word; the lane holding it drops its head.  After rank r a
// list is read at most KM - 1 - r more times, so the drop shifts only that
// many entries.  Returns how many keys are valid.
template <int KM>
__device__ __forceinline__ int wave_top_keys(uint64_t (&L)[KM], uint64_t (&R)[KM], int top_k) {
    int m = 0;
#pragma unroll
    for (int r = 0; r < KM; ++r) {
        R[r] = 0;
        if (r < top_k && m == r) {
            const uint32_t hh = (uint32_t)(L[0] >> 32);
            const uint32_t hi = __builtin_amdgcn_readfirstlane(wave_max_u32(hh));
            if (hi != 0) {  // keys are unique and nonzero: exactly one lane holds the max
                const uint32_t lo = __builtin_amdgcn_readfirstlane(
                    wave_max_u32(hh == hi ? (uint32_t)L[0] : 0u));
                const uint64_t mx = ((uint64_t)hi << 32) | lo;
                R[r] = mx;
                m = r + 1;
                if (L[0] == mx) {
#pragma unroll
                    for (int j = 0; j + 1 < KM - r; ++j) L[j] = L[j + 1];
                }
            }
        }
    }
    return m;
}

// Queued rows are redone exactly, one workgroup per row, when there are at
// most FB_ROWS of them (more are redone by whole tiles, k_route<.., true>):
// fp32 scores of every candidate (fma chain over d = 0..63), each lane
// keeping the KM best keys of the candidates it scored in registers, then
// rank-by-rank wave maxima; wave 0 merges the four waves' lists through
// LDS.  Exact for any input, ties included.
// KM: the selection list length, as in k_route.
template <bool CAUSAL, bool QF32, int KM>
__global__ __launch_bounds__(256) void k_route_fallback(RouteArgs a) {
    __shared__ uint64_t s_top[4][KM];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t count = __builtin_amdgcn_readfirstlane(*a.ovf_count);
    if (count > (uint32_t)FB_ROWS) return;  // the whole-tile pass takes them
    for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
        const uint32_t rid = __builtin_amdgcn_readfirstlane(a.ovf_rows[i]);
        const int bh = (int)(rid / (uint32_t)a.P), row = (int)(rid % (uint32_t)a.P);
        const int h = bh % a.Hq, b = bh / a.Hq, g = h / (a.Hq / a.Hkv);
        const float* kb = a.kbar + (int64_t)(b * a.Hkv + g) * a.nb * kD;
        const int E = row_candidates(CAUSAL, row, a.P, a.bs, a.window, a.nb, a.cshift);
        // the query row is the same for every lane: scalar loads
        float qv[kD];
        if (QF32) {
            const __attribute__((address_space(4))) float* qp =
                (const __attribute__((address_space(4))) float*)(a.qbar + ((int64_t)bh * a.P + row) * kD);
#pragma unroll
            for (int d = 0; d < kD; ++d) qv[d] = qp[d];
        } else {
            const __attribute__((address_space(4))) uint32_t* qp =
                (const __attribute__((address_space(4))) uint32_t*)(a.q + ((int64_t)bh * a.N + row) * kD);
#pragma unroll
            for (int d2 = 0; d2 < kD / 2; ++d2) {
                const uint32_t u = qp[d2];
                qv[2 * d2] = __uint_as_float(u << 16);
                qv[2 * d2 + 1] = __uint_as_float(u & 0xFFFF0000u);
            }
        }
        uint64_t L[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) L[j] = 0;
        // one candidate per lane per trip (64 VGPRs of loads, four waves per SIMD)
        for (int c = threadIdx.x; c < E; c += 256) {
            const f32x4* kr = reinterpret_cast<const f32x4*>(kb + (int64_t)c * kD);
            f32x4 v[kD / 4];
#pragma unroll
            for (int d4 = 0; d4 < kD / 4; ++d4) v[d4] = kr[d4];
            float sc = 0.f;
#pragma unroll
            for (int d4 = 0; d4 < kD / 4; ++d4)
#pragma unroll
                for (int e = 0; e < 4; ++e) sc = fmaf(qv[4 * d4 + e], v[d4][e], sc);
            const uint64_t key = sel_key(sc, (uint32_t)c);
            if (key > L[KM - 1]) insert_key(L, key);
        }
        uint64_t R[KM];
        int m = wave_top_keys(L, R, a.top_k);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < KM; ++r) s_top[w][r] = R[r];
        }
        __syncthreads();
        if (w == 0) {
            // the four waves' sorted lists: lane l takes entries l % 16 + 16 j
            // of list l / 16 (descending, so a sorted list of KM / 16 keys)
#pragma unroll
            for (int j = 0; j < KM; ++j) L[j] = j < KM / 16 ? s_top[lane >> 4][(lane & 15) + 16 * j] : 0;
            m = wave_top_keys(L, R, a.top_k);
        }
        __syncthreads();
        if (w == 0 && lane == 0) {
            write_selection(a.idx + (int64_t)rid * a.idx_stride, R, m, a.top_k, a.idx_stride);
            if (a.idx_stride > a.top_k)
                a.idx[(int64_t)rid * a.idx_stride + a.top_k] =
                    CAUSAL ? tail_node(row, a.bs, a.window) : a.tail_img;
        }
    }
}

// ------------------------------------------------------------ second-cumulant routing
// Score r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q (SSA page, "Algorithm
// and complexity"), with Sigma_c the bs-normalised covariance of block c's
// keys.  Since q^T Sigma_c q is the variance over the block of the raw
// scores q . k_j, and <q, mu_c> their mean, the kernel computes the raw
// scores of every eligible key with bf16 MFMA (exact products, fp32 sums)
// and reduces each block to mean + (beta/2) * variance.
//
// A workgroup owns 128 query rows of one (b, h), four waves of 32 rows; the
// keys stream through LDS in chunks of 32 (double-buffered, loads two chunks
// ahead).  Tiles S^T = K_chunk . Q^T leave each lane 16 scores of its row,
// the lane pair (l, l^32) holding the chunk's 32.  Each lane accumulates the
// sum and the sum of squares of its scores over the block; at the block's
// end the pair adds its halves (one cross-half swap each) and forms
// variance = sum of squares / bs - mean^2.
//
// Selection: the two lanes of a pair take the even and the odd blocks
// respectively.  Each lane keeps its KM (16, or 32 for top_k above 16) best
// (score, block) pairs sorted by score.  A lane sees its blocks in ascending
// order, so a newcomer beats a kept entry exactly when its score is strictly
// larger (equal scores keep the lower, older block): the order (score desc,
// block asc) needs only float compares.  Blocks that beat the lane's last
// kept score are appended to a per-lane LDS queue and inserted in batches of
// CUM_Q offers, so that a wave runs the insertion about as often as its
// busiest lane needs it rather than whenever any lane does.  The pair's
// lists are merged once at the end.
// No survivor capacity, so no fallback.
constexpr int CUM_Q = 8;  // offers per lane between insertion batches

struct CumArgs {
    const uint16_t* q;  // [B,Hq,N,64] bf16
    const uint16_t* k;  // [B,Hkv,N,64] bf16
    int32_t* idx;       // [B,Hq,N,top_k]
    int Hq, Hkv, N, top_k, window, tiles, items;
    float half_beta;    // beta / 2
};

// v[l % 32] + v[l % 32 + 32] in every lane l (bitwise equal in both lanes).
__device__ __forceinline__ float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// KM: the per-lane list length (kMaxTopK; kMaxTopKWide for top_k 17..32,
// at half the occupancy).
template <int BS, int KM>
__global__ __launch_bounds__(256, KM > kMaxTopK ? 2 : 4) void k_route_cumulant(CumArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_k[2][RT_CH * RT_PITCH];
    __shared__ float s_qs[CUM_Q][256];  // queued scores, slot-major
    __shared__ int s_qc[CUM_Q][256];    // queued block ids
    constexpr int CPB = BS >= RT_CH ? BS / RT_CH : 1;  // chunks per block (BS >= 32)
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    // XCD-aware order as in k_route: the tiles of one head, and the heads of
    // one KV group, on one XCD, whose L2 then serves the group's keys.
    const int per_xcd = gridDim.x / 8;
    const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= a.items) return;
    const int bh = item / a.tiles;
    const int tile = a.tiles - 1 - (item - bh * a.tiles);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    const int N = a.N;
    const int r0 = tile * RT_ROWS + 32 * w;
    const int rq = r0 + l32;
    const int Erow = rq < N ? eligible_blocks(rq, BS, a.window) : 0;
    const int Emax = r0 < N ? eligible_blocks(min(r0 + 31, N - 1), BS, a.window) : 0;
    const int wg_last = min(tile * RT_ROWS + RT_ROWS, N) - 1;
    const int Ewg = eligible_blocks(wg_last, BS, a.window);
    const uint16_t* kb = a.k + (int64_t)bg * N * kD;
    const float hb = a.half_beta;
    constexpr float inv_bs = 1.f / (float)BS;

    bf16x8 Bq[4];
    if (rq < N) {
        const uint16_t* qp = a.q + ((int64_t)bh * N + rq) * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            Bq[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Bq[ks] = bf16x8{};
    }

    float Ls[KM];  // kept scores, descending
    int Lc[KM];    // their blocks
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        Ls[j] = -INFINITY;
        Lc[j] = 0;
    }
    int nq = 0;  // queued offers of this lane
    auto flush = [&]() {
        for (int i = 0; __builtin_amdgcn_ballot_w64(i < nq) != 0; ++i) {
            if (i < nq) {
                float x = s_qs[i][tid];
                int xc = s_qc[i][tid];
                if (x > Ls[KM - 1]) {
#pragma unroll
                    for (int j = 0; j < KM; ++j) {
                        const bool gt = x > Ls[j];
                        const float ts = Ls[j];
                        const int tc = Lc[j];
                        Ls[j] = gt ? x : ts;
                        Lc[j] = gt ? xc : tc;
                        x = gt ? ts : x;
                        xc = gt ? tc : xc;
                    }
                }
            }
        }
        nq = 0;
    };
    float s1 = 0.f, s2 = 0.f;  // this lane's sum and sum of squares over the block (BS >= 32)
    // chunks of 32 keys covering the eligible blocks; with BS = 16 an odd
    // block count ends half-way through the last chunk, whose other block
    // exists (it is at most the query's own block) and is masked by Erow
    const int nch = (Ewg * BS + RT_CH - 1) / RT_CH;
    const int wave_keys = Emax * BS;

    // Staging loads are issued unconditionally (the address clamped to the
    // last chunk), so the in-order load counter always has exactly one
    // younger load in flight when a staged chunk is stored, and the query
    // loads are complete before the loop: no wait drains the prefetch.
    const int last = (nch - 1) * RT_CH;  // used only when nch > 0 (workgroup-uniform)
    // block score from the pair's sums; queued by the lane of its parity when
    // it beats that lane's 16th kept score.  Every 2 * CUM_Q blocks (CUM_Q
    // offers per lane) the queues are inserted.
    auto offer = [&](float sum, float sq, int c) {
        const float m = pair_sum(sum) * inv_bs;
        const float var = pair_sum(sq) * inv_bs - m * m;
        const float score = fmaf(hb, var, m);
        if ((c & 1) == half && c < Erow && score > Ls[KM - 1]) {
            s_qs[nq][tid] = score;
            s_qc[nq][tid] = c;
            ++nq;
        }
        if ((c & (2 * CUM_Q - 1)) == 2 * CUM_Q - 1) flush();
    };
    auto body = [&](int j, u32x4& r_issue, const u32x4& r_store) {
        const int key0 = j * RT_CH;
        r_issue = stage_load(kb, min(key0 + 2 * RT_CH, last), tid);
        if (key0 < wave_keys) {
            bf16x8 A[4];
            read_cands(s_k[j & 1], l32, half, A);
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma32(A[ks], Bq[ks], acc);
            // register r holds key 8*(r/4) + 4*half + r%4 of the chunk
            if constexpr (BS == 16) {
                // keys 0-15 (block 2j) sit in registers 0-7, keys 16-31 in 8-15
                float a0 = 0.f, a1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    a0 += acc[r];
                    a1 += acc[r + 8];
                    q0 = fmaf(acc[r], acc[r], q0);
                    q1 = fmaf(acc[r + 8], acc[r + 8], q1);
                }
                offer(a0, q0, 2 * j);
                offer(a1, q1, 2 * j + 1);
            } else {
                const int jb = j % CPB;
                if (jb == 0) {
                    s1 = 0.f;
                    s2 = 0.f;
                }
                float t1 = 0.f, t2 = 0.f;  // two chains for the adder latency
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    s1 += acc[r];
                    t1 += acc[r + 1];
                    s2 = fmaf(acc[r], acc[r], s2);
                    t2 = fmaf(acc[r + 1], acc[r + 1], t2);
                }
                s1 += t1;
                s2 += t2;
                if (jb == CPB - 1) offer(s1, s2, j / CPB);
            }
        }
        stage_store(s_k[(j + 1) & 1], tid, r_store);
        __syncthreads();
    };
    if (nch > 0) {
        u32x4 r0v = stage_load(kb, 0, tid);
        u32x4 r1v = stage_load(kb, min(RT_CH, last), tid);
        __builtin_amdgcn_s_waitcnt(0);
        stage_store(s_k[0], tid, r0v);
        __syncthreads();
        for (int j = 0; j < nch; j += 2) {
            body(j, r0v, r1v);
            if (j + 1 < nch) body(j + 1, r1v, r0v);
        }
        flush();
    }

    // the pair's lists hold disjoint candidates (even and odd blocks); as
    // 64-bit keys (score, then lower block) they merge in one bitonic step
    uint64_t Mx[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        const int jj = KM - 1 - j;
        const uint64_t o = Ls[jj] == -INFINITY ? 0ull : sel_key(Ls[jj], (uint32_t)Lc[jj]);
        const uint64_t mine = Ls[j] == -INFINITY ? 0ull : sel_key(Ls[j], (uint32_t)Lc[j]);
        const uint32_t olo = __shfl_xor((uint32_t)o, 32, kWave);
        const uint32_t ohi = __shfl_xor((uint32_t)(o >> 32), 32, kWave);
        const uint64_t other = ((uint64_t)ohi << 32) | olo;
        Mx[j] = mine > other ? mine : other;
    }
    bitonic_merge_desc_u64(Mx);
    if (rq < N && half == 0) {
        const int m = Erow < a.top_k ? Erow : a.top_k;
        write_selection(a.idx + ((int64_t)bh * N + rq) * a.top_k, Mx, m, a.top_k, a.top_k);
    }
}

// ------------------------------------------------------------ group queries
// Consensus routing: out[b, g, p, :] = sum over the group's heads h of
// in[b, h, p, :], in fp32 (heads in ascending order).  One thread per 8
// dims of a row.  T = uint16_t (bf16 bits) or float.
template <typename T>
__global__ __launch_bounds__(256) void k_group_query(const T* __restrict__ in,
                                                     float* __restrict__ out, int Hq, int Hkv,
                                                     int P, int64_t n_threads) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_threads) return;
    const int rep = Hq / Hkv;
    const int64_t row = i >> 3;  // (b*Hkv + g)*P + p
    const int d0 = (int)(i & 7) * 8;
    const int64_t p = row % P, bg = row / P;
    const int64_t b = bg / Hkv, g = bg % Hkv;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int hh = 0; hh < rep; ++hh) {
        const T* src = in + ((b * Hq + g * rep + hh) * P + p) * kD + d0;
        float f[8];
        if constexpr (sizeof(T) == 2) {
            unpack8(*reinterpret_cast<const u32x4*>(src), f);
        } else {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
            f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
            f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += f[j];
    }
    float* dst = out + row * kD + d0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ------------------------------------------------------------ two-level routing, first level
// Node summaries: the mean of 16 consecutive block means (fp64 sum, one
// fp32 rounding), for the nn complete nodes of each group.  One thread per
// (node, 8 dims).
__global__ __launch_bounds__(256) void k_node_means(const float* __restrict__ kbar,
                                                    float* __restrict__ nu, int nb, int nn,
                                                    int64_t n_threads) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_threads) return;
    const int64_t gs = i >> 3;  // bg * nn + node
    const int d0 = (int)(i & 7) * 8;
    const int64_t bg = gs / nn, node = gs % nn;
    const float* src = kbar + (bg * nb + node * kTreeFanout) * kD + d0;
    double acc[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
    for (int c = 0; c < kTreeFanout; ++c) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + (int64_t)c * kD);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + (int64_t)c * kD + 4);
        acc[0] += x0[0]; acc[1] += x0[1]; acc[2] += x0[2]; acc[3] += x0[3];
        acc[4] += x1[0]; acc[5] += x1[1]; acc[6] += x1[2]; acc[7] += x1[3];
    }
    float* dst = nu + gs * kD + d0;
    *reinterpret_cast<f32x4*>(dst) =
        f32x4{(float)(acc[0] / kTreeFanout), (float)(acc[1] / kTreeFanout),
              (float)(acc[2] / kTreeFanout), (float)(acc[3] / kTreeFanout)};
    *reinterpret_cast<f32x4*>(dst + 4) =
        f32x4{(float)(acc[4] / kTreeFanout), (float)(acc[5] / kTreeFanout),
              (float)(acc[6] / kTreeFanout), (float)(acc[7] / kTreeFanout)};
}

// Slot `beam` of each row's slot list (causal rows: tail_node; image-mode
// rows: the same tail for every row), for launches where no row has a
// complete node and so no routing kernel runs to write it.
__global__ __launch_bounds__(256) void k_tree_tail(int32_t* __restrict__ slots, int beam,
                                                   int64_t rows, int N, int bs, int window,
                                                   int causal, int tail_img) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    slots[row * (beam + 1) + beam] = causal ? tail_node((int)(row % N), bs, window) : tail_img;
}

// ------------------------------------------------------------ host side
static int route_heads(const Geometry& g) { return g.consensus ? g.Hkv : g.Hq; }

// Rows per (b, routed head): positions, or query blocks in image mode (the
// first level of two-level routing keeps N and bs and routes over nodes, so
// its nb is not the row count).
static int route_P(const Geometry& g) { return g.causal ? g.N : g.N / g.bs; }

static size_t route_rows(const Geometry& g) {
    return (size_t)g.B * route_heads(g) * (size_t)route_P(g);
}

// Routing workgroups (tiles of RT_ROWS rows) over all (b, routed head).
static size_t route_items(const Geometry& g) {
    const size_t P = (size_t)route_P(g);
    return (size_t)g.B * route_heads(g) * ((P + RT_ROWS - 1) / RT_ROWS);
}

// The workspace starts with the words the router clears before each call:
// the two overflow counters (in the first 256 bytes) and the chunk maxima of
// the block-mean norms; one fill covers them.
struct RouteLayout {
    size_t cmax, ovf_rows, tiles, qbar, qsum, khi, klo, total;
    int nb_pad, ncb;
};

static RouteLayout route_layout(const Geometry& g) {
    RouteLayout L{};
    L.nb_pad = (g.nb + RT_CH - 1) / RT_CH * RT_CH;
    L.ncb = L.nb_pad / RT_CH;
    const size_t nbg = (size_t)g.B * g.Hkv;
    size_t off = kRouteCounterWords * 4;  // counters (queued rows, queued tiles)
    L.cmax = off;     off += align_up(2 * nbg * L.ncb * kChunkMaxStride * 4, 256);  // norms, then lo
    L.ovf_rows = off; off += align_up(route_rows(g) * 4, 256);
    L.tiles = off;    off += align_up(route_items(g) * 4, 256);
    L.qbar = off;     if (!g.causal) off += align_up((size_t)g.B * g.Hq * route_P(g) * kD * 4, 256);
    L.qsum = off;     if (g.consensus) off += align_up(route_rows(g) * kD * 4, 256);
    L.khi = off;      off += align_up(nbg * L.nb_pad * kD * 2, 256);
    L.klo = off;      off += align_up(nbg * L.nb_pad * kD * 2, 256);

    L.total = off;
    return L;
}

// Two-level routing: the first level is flat routing over the complete
// nodes (a geometry with nb = nodes and top_k = beam), followed by the node
// summaries, the slot lists, the block means' bf16 hi/lo split and the
// second level's own workspace.
struct TreeRouteLayout {
    RouteLayout L1;
    size_t lvl1, nu, qbar, slots, bhi, blo, bnorm, lvl2, total;
    int nn, nb_pad;
};

static Geometry tree_level1_geometry(const Geometry& g) {
    Geometry g1 = g;
    g1.nb = g.nb >> kTreeFanoutLog2;
    g1.top_k = g.beam;
    return g1;
}

static TreeRouteLayout tree_route_layout(const Geometry& g) {
    TreeRouteLayout T{};
    const size_t nbg = (size_t)g.B * g.Hkv;
    const size_t rows = (size_t)g.B * g.Hq * (g.causal ? (size_t)g.N : (size_t)g.nb);
    T.nn = g.nb >> kTreeFanoutLog2;
    T.nb_pad = (g.nb + RT_CH - 1) / RT_CH * RT_CH;
    size_t off = 0;
    T.lvl1 = off;
    if (T.nn > 0) {
        T.L1 = route_layout(tree_level1_geometry(g));
        off += align_up(T.L1.total, 256);
    }
    T.nu = off;    off += align_up(nbg * (T.nn > 0 ? T.nn : 1) * kD * 4, 256);
    T.qbar = off;  if (!g.causal) off += align_up(rows * kD * 4, 256);  // pooled queries
    T.slots = off; off += align_up(rows * (g.beam + 1) * 4, 256);
    T.bhi = off;   off += align_up(nbg * T.nb_pad * kD * 2, 256);
    T.blo = off;   off += align_up(nbg * T.nb_pad * kD * 2, 256);
    T.bnorm = off;  // chunk maxima of the block-mean norms (unused by the second level)
    off += align_up(2 * nbg * (T.nb_pad / RT_CH) * kChunkMaxStride * 4, 256);
    T.lvl2 = off;  off += tree_level2_bytes(g);
    T.total = off;
    return T;
}

size_t route_workspace_bytes(const Geometry& g) {
    return g.beam > 0 ? tree_route_layout(g).total : route_layout(g).total;
}

template <bool CAUSAL, bool QF32, int KM>
static void launch_route_kernels_km(const RouteArgs& a, dim3 grid, hipStream_t s,
                                    const hipEvent_t* ev) {
    // the longest row's candidate count picks the pass-2 form; fp32 queries
    // (group sums, pooled blocks) always take the full form: their delta
    // carries the q_lo term too, and the lean form's 2 * delta band
    // overflows the survivor lists
    const int cmax = CAUSAL ? (eligible_blocks(a.P - 1, a.bs, a.window) >> a.cshift) : a.nb;
    bool lean = false;
    if constexpr (!QF32) lean = cmax >= kRouteLeanMinCand;
    if constexpr (!QF32) {
        if (lean)
            hipLaunchKernelGGL((k_route<CAUSAL, false, false, true, KM>), grid, dim3(256), 0, s, a);
    }
    if (!lean) hipLaunchKernelGGL((k_route<CAUSAL, QF32, false, false, KM>), grid, dim3(256), 0, s, a);
    mark(ev, 2, s);
    // exactly one of the two exact passes does work, chosen on the device by
    // the number of overflowing rows
    hipLaunchKernelGGL((k_route_fallback<CAUSAL, QF32, KM>), dim3(FB_GRID), dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_route<CAUSAL, QF32, true, false, KM>), grid, dim3(256), 0, s, a);
}

template <bool CAUSAL, bool QF32>
static void launch_route_kernels(const RouteArgs& a, dim3 grid, hipStream_t s,
                                 const hipEvent_t* ev) {
    if (a.top_k <= kMaxTopK)
        launch_route_kernels_km<CAUSAL, QF32, kMaxTopK>(a, grid, s, ev);
    else
        launch_route_kernels_km<CAUSAL, QF32, kMaxTopKWide>(a, grid, s, ev);
}

// Flat routing of g's rows over g.nb summaries `summ` into idx (row stride
// idx_stride), candidates E >> cshift in causal mode; ws holds
// route_layout(g).
static hipError_t route_flat(const Geometry& g, const uint16_t* q, const float* summ,
                             int32_t* idx, int idx_stride, int cshift, void* ws, hipStream_t s,
                             const hipEvent_t* ev, const float* qbar_in = nullptr,
                             int tail_img = -1, bool prepared = false) {
    char* base = static_cast<char*>(ws);
    const RouteLayout L = route_layout(g);
    const int nbg = g.B * g.Hkv;
    RouteArgs a;
    a.ovf_count = reinterpret_cast<uint32_t*>(base);
    a.ovf_rows = reinterpret_cast<uint32_t*>(base + L.ovf_rows);
    a.tile_count = a.ovf_count + 1;  // the word after the row count
    a.tile_queue = reinterpret_cast<uint32_t*>(base + L.tiles);
    float* qbar = g.causal ? nullptr
                           : (qbar_in ? const_cast<float*>(qbar_in)
                                      : reinterpret_cast<float*>(base + L.qbar));
    float* qsum = g.consensus ? reinterpret_cast<float*>(base + L.qsum) : nullptr;
    uint16_t* khi = reinterpret_cast<uint16_t*>(base + L.khi);
    uint16_t* klo = reinterpret_cast<uint16_t*>(base + L.klo);
    float* ckn = reinterpret_cast<float*>(base + L.cmax);
    float* clo = ckn + (size_t)nbg * L.ncb * kChunkMaxStride;
    const int heads = route_heads(g);
    a.q = q;
    a.qbar = g.consensus ? qsum : qbar;
    a.kbar = summ;
    a.khi = khi;
    a.klo = klo;
    a.ckn = ckn;
    a.clo = clo;
    a.idx = idx;
    a.Hq = heads;  // rows of the router: (b, routed head, position)
    a.Hkv = g.Hkv;
    a.N = g.N;
    a.bs = g.bs;
    a.nb = g.nb;
    a.top_k = g.top_k;
    a.window = g.window;
    a.P = route_P(g);
    a.tiles = (a.P + RT_ROWS - 1) / RT_ROWS;
    a.items = g.B * heads * a.tiles;
    a.nb_pad = L.nb_pad;
    a.ncb = L.ncb;
    a.cshift = cshift;
    a.idx_stride = idx_stride;
    a.tail_img = tail_img;
    hipError_t e = hipSuccess;
    if (!prepared) {  // the counters (prepared: cleared by the caller, with the norm maxima)
        e = launch_fill_u32(a.ovf_count, kRouteCounterWords, 0u, s);
        if (e != hipSuccess) return e;
    }
    if (!g.causal && !qbar_in) {
        e = launch_summarize(q, qbar, g.B * g.Hq, g.N, g.bs, s);
        if (e != hipSuccess) return e;
    }
    if (g.consensus) {
        const int64_t n = (int64_t)route_rows(g) * 8;
        const dim3 gq((unsigned)((n + 255) / 256));
        if (g.causal)
            hipLaunchKernelGGL(k_group_query<uint16_t>, gq, dim3(256), 0, s, q, qsum, g.Hq, g.Hkv,
                               a.P, n);
        else
            hipLaunchKernelGGL(k_group_query<float>, gq, dim3(256), 0, s, qbar, qsum, g.Hq, g.Hkv,
                               a.P, n);
    }
    if (!prepared) {
        const int64_t prep_threads = (int64_t)nbg * L.nb_pad * 8;
        hipLaunchKernelGGL(k_route_prep, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256),
                           0, s, summ, khi, klo, ckn, clo, nbg, g.nb, L.nb_pad);
    }
    const dim3 grid((unsigned)(((int64_t)a.items + 7) / 8 * 8));  // a multiple of the XCD count
    if (g.causal && !g.consensus)
        launch_route_kernels<true, false>(a, grid, s, ev);
    else if (g.causal)
        launch_route_kernels<true, true>(a, grid, s, ev);
    else
        launch_route_kernels<false, true>(a, grid, s, ev);
    return hipGetLastError();
}

// Two-level routing (per query head; causal rows, or pooled query blocks in
// image mode).  Stage events: 2 after the first level and the tail slots, 3
// after the second level.
static hipError_t route_tree(const Geometry& g, const uint16_t* q, const float* kbar,
                             int32_t* idx, void* ws, hipStream_t s, const hipEvent_t* ev) {
    char* base = static_cast<char*>(ws);
    const TreeRouteLayout T = tree_route_layout(g);
    const int nbg = g.B * g.Hkv;
    const int P = g.causal ? g.N : g.nb;  // rows per (b, query head)
    const int64_t rows = (int64_t)g.B * g.Hq * P;
    const int stride = g.beam + 1;
    float* nu = reinterpret_cast<float*>(base + T.nu);
    int32_t* slots = reinterpret_cast<int32_t*>(base + T.slots);
    uint16_t* bhi = reinterpret_cast<uint16_t*>(base + T.bhi);
    uint16_t* blo = reinterpret_cast<uint16_t*>(base + T.blo);
    float* bn = reinterpret_cast<float*>(base + T.bnorm);
    // image mode: every row's candidates are all nb blocks, so its tail is
    // the same partial node for every row
    const int tail_img = (T.nn << kTreeFanoutLog2) < g.nb ? T.nn : -1;
    float* qbar = g.causal ? nullptr : reinterpret_cast<float*>(base + T.qbar);
    hipError_t e;
    if (!g.causal) {  // pooled queries, shared by both levels
        e = launch_summarize(q, qbar, g.B * g.Hq, g.N, g.bs, s);
        if (e != hipSuccess) return e;
    }
    if (T.nn > 0) {
        const int64_t n = (int64_t)nbg * T.nn * 8;
        hipLaunchKernelGGL(k_node_means, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kbar,
                           nu, g.nb, T.nn, n);
        e = route_flat(tree_level1_geometry(g), q, nu, slots, stride, kTreeFanoutLog2,
                       base + T.lvl1, s, nullptr, qbar, tail_img);
        // the routing kernels write each row's tail slot with its beam
    } else {
        e = launch_fill_u32(reinterpret_cast<uint32_t*>(slots), (size_t)rows * stride,
                            0xFFFFFFFFu, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_tree_tail, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                           slots, g.beam, rows, P, g.bs, g.window, g.causal, tail_img);
    }
    if (e != hipSuccess) return e;
    const int64_t prep_threads = (int64_t)nbg * T.nb_pad * 8;
    hipLaunchKernelGGL(k_route_prep, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, s,
                       kbar, bhi, blo, bn, bn + (size_t)nbg * (T.nb_pad / RT_CH) * kChunkMaxStride,
                       nbg, g.nb, T.nb_pad);
    mark(ev, 2, s);
    e = launch_tree_level2(g, q, qbar, bhi, blo, T.nb_pad, slots, idx, base + T.lvl2, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_summary_and_route_prep(const Geometry& g, const uint16_t* k, const uint16_t* q,
                                         float* kbar, void* ws, hipStream_t s) {
    const RouteLayout L = route_layout(g);
    char* base = static_cast<char*>(ws);
    const size_t nbg = (size_t)g.B * g.Hkv;
    float* ckn = reinterpret_cast<float*>(base + L.cmax);
    // the summary writes every chunk line and clears the counters itself
    uint32_t* counters = reinterpret_cast<uint32_t*>(base);
    uint16_t* khi = reinterpret_cast<uint16_t*>(base + L.khi);
    uint16_t* klo = reinterpret_cast<uint16_t*>(base + L.klo);
    float* clo = ckn + nbg * L.ncb * kChunkMaxStride;
    if (!g.causal)  // image mode: the query pooling joins the same launch
        return launch_summarize_route_pool16(k, kbar, g.B * g.Hkv, q,
                                             reinterpret_cast<float*>(base + L.qbar), g.B * g.Hq,
                                             g.N, khi, klo, ckn, clo, L.nb_pad, counters, s);
    return launch_summarize_route(k, kbar, g.B * g.Hkv, g.N, g.bs, khi, klo, ckn, clo, L.nb_pad,
                                  counters, s);
}

hipError_t launch_route_prepared(const Geometry& g, const uint16_t* q, const float* kbar,
                                 int32_t* idx, void* ws, hipStream_t s, const hipEvent_t* ev) {
    // image mode: the pooled queries were written by the key summary's launch
    const float* qbar = g.causal ? nullptr
                                 : reinterpret_cast<const float*>(static_cast<char*>(ws) +
                                                                  route_layout(g).qbar);
    hipError_t e = route_flat(g, q, kbar, idx, g.top_k, 0, ws, s, ev, qbar, -1, true);
    mark(ev, 3, s);
    return e;
}

hipError_t launch_route(const Geometry& g, const uint16_t* q, const float* kbar, int32_t* idx,
                        void* ws, hipStream_t s, const hipEvent_t* ev) {
    hipError_t e = g.beam > 0 ? route_tree(g, q, kbar, idx, ws, s, ev)
                              : route_flat(g, q, kbar, idx, g.top_k, 0, ws, s, ev);
    mark(ev, 3, s);
    return e;
}

template <int KM>
static void launch_cumulant(int bs, dim3 grid, const CumArgs& a, hipStream_t s) {
    switch (bs) {
        case 16: hipLaunchKernelGGL((k_route_cumulant<16, KM>), grid, dim3(256), 0, s, a); break;
        case 32: hipLaunchKernelGGL((k_route_cumulant<32, KM>), grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL((k_route_cumulant<64, KM>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((k_route_cumulant<128, KM>), grid, dim3(256), 0, s, a); break;
    }
}

hipError_t launch_route_cumulant(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                 int32_t* idx, hipStream_t s) {
    CumArgs a;
    a.q = q;
    a.k = k;
    a.idx = idx;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.N = g.N;
    a.top_k = g.top_k;
    a.window = g.window;
    a.tiles = (g.N + RT_ROWS - 1) / RT_ROWS;
    a.items = g.B * g.Hq * a.tiles;
    a.half_beta = 0.5f * g.beta;
    const dim3 grid((unsigned)(((int64_t)a.items + 7) / 8 * 8));  // a multiple of the XCD count
    if (g.top_k <= kMaxTopK)
        launch_cumulant<kMaxTopK>(g.bs, grid, a, s);
    else
        launch_cumulant<kMaxTopKWide>(g.bs, grid, a, s);
    return hipGetLastError();
}

}  // namespace lsa
