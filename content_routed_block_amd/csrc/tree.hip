// Second level of two-level routing (SSA page, "Algorithm and complexity":
// a hierarchical router with fixed block size and budget, the measured tree
// at fanout 16).  The first level (in the routing file) leaves, per causal
// row, a slot list: the beam of kept nodes (16 consecutive key blocks each,
// ascending, -1 padded) followed by the row's incomplete tail node, if any.
// Here every block of those nodes is scored and the row's top-k taken:
//   1. k_bucket<false> / k_bucket_scan / k_bucket<true> group the (row, slot)
//      pairs by node, as the attention groups them by block;
//   2. k_tree_score: one node's 16 block means (bf16 hi + lo) in LDS against
//      up to 64 gathered query rows, on 16x16x32 bf16 MFMA tiles: 16 scores
//      per pair (fp32 accuracy), written by pair position (contiguous);
//   3. k_tree_select: one lane per row merges each used slot's 16 scores,
//      as sorted 64-bit keys (score, then lower block), into the row's
//      running top-16 (top-32 when top_k exceeds 16) with a bitonic merge.
//      Blocks of the tail node past the row's candidates are left out.
// The node-major scoring gathers one 128-byte query row per pair instead of
// a node's 4 KB of block means per pair.
#include <math.h>

#include <algorithm>

#include "bucket.hpp"
#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

constexpr int TR_PITCH = 72;  // LDS pitch of the staged block means (bf16)

struct TreeScoreArgs {
    const uint16_t* q;         // [B,Hq,N,64] bf16 (causal rows)
    const float* qbar;         // [B*Hq*nb][64] fp32 pooled queries (image-mode rows)
    const uint16_t* bhi;       // block means, bf16 hi part [B*Hkv][nb_pad][64]
    const uint16_t* blo;       // bf16 lo part
    const uint32_t* pairs;     // pair ids in node order
    const uint32_t* offsets;   // [NB+1]
    const uint32_t* unit_off;  // [NB+1]
    float* scores;             // [npairs + 64][16] by pair position
    uint32_t dummy_pos;        // npairs: first of 64 rows written by lanes without a pair
    int nodes, NB, nb_pad, sp_log2;
};

// One resident wave of workgroups; each takes a contiguous range of 64-pair
// units, so a node's block means are staged once for all its units.  Wave w
// owns pairs 16w..16w+15 of a unit.  Tiles D = Kbar_node . Q^T: lane l holds
// pair l%16 and blocks 4(l/16)+r, i.e. 16 contiguous bytes of the pair's
// 64-byte score row.
template <bool QF32>
__global__ __launch_bounds__(256, 4) void k_tree_score(TreeScoreArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_h[kTreeFanout * TR_PITCH];
    __shared__ __attribute__((aligned(16))) __bf16 s_l[kTreeFanout * TR_PITCH];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t U = uniform_load(a.unit_off + a.NB);
    const uint32_t per = (U + gridDim.x - 1) / gridDim.x;
    const uint32_t u0 = blockIdx.x * per;
    const uint32_t u1 = min(U, u0 + per);
    if (u0 >= u1) return;
    UnitCursor cur;
    cur.seek(a.unit_off, a.NB, u0);
    const uint32_t my = 16 * w + (lane & 15);
    int loaded = -1;
    for (uint32_t u = u0; u < u1; ++u) {
        uint32_t p0, p1;
        cur.rows(a.unit_off, a.offsets, u, p0, p1);
        // every lane loads (a pair id, a query row), lanes past the unit's
        // end use pair 0 and store to a dummy row
        const bool valid = p0 + my < p1;
        const uint32_t pid = a.pairs[valid ? p0 + my : 0u];
        // the query as the B operand: dims 8(l/16) .. +7 and 32 + 8(l/16) .. +7;
        // an fp32 query is split into bf16 hi + lo parts
        bf16x8 b0, b1, b0l, b1l;
        if constexpr (QF32) {
            const float* qrow = a.qbar + (int64_t)(pid >> a.sp_log2) * kD + 8 * (lane >> 4);
#pragma unroll
            for (int hblk = 0; hblk < 2; ++hblk) {
                const f32x4 x0 = *reinterpret_cast<const f32x4*>(qrow + 32 * hblk);
                const f32x4 x1 = *reinterpret_cast<const f32x4*>(qrow + 32 * hblk + 4);
                const float f[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                bf16x8 hi, lo;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hi[i] = (__bf16)f[i];
                    lo[i] = (__bf16)(f[i] - (float)hi[i]);
                }
                if (hblk == 0) { b0 = hi; b0l = lo; } else { b1 = hi; b1l = lo; }
            }
        } else {
            const uint16_t* qrow = a.q + (int64_t)(pid >> a.sp_log2) * kD + 8 * (lane >> 4);
            b0 = load_bf16x8(qrow);
            b1 = load_bf16x8(qrow + 32);
        }
        if (cur.bucket != loaded) {
            __syncthreads();
            const int bg = cur.bucket / a.nodes, node = cur.bucket - bg * a.nodes;
            // 16 rows x 8 chunks of 16 bytes, hi then lo: one chunk per thread
            const int part = tid >> 7, r = (tid >> 3) & 15, ch = tid & 7;
            const uint16_t* src = (part ? a.blo : a.bhi) +
                                  ((int64_t)bg * a.nb_pad + node * kTreeFanout + r) * kD + 8 * ch;
            const u32x4 v = *reinterpret_cast<const u32x4*>(src);
            *reinterpret_cast<u32x4*>((part ? s_l : s_h) + r * TR_PITCH + 8 * ch) = v;
            __syncthreads();
            loaded = cur.bucket;
        }
        const int ar = lane & 15, ak = 8 * (lane >> 4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16(*reinterpret_cast<const bf16x8*>(s_h + ar * TR_PITCH + ak), b0, acc);
        acc = mfma16(*reinterpret_cast<const bf16x8*>(s_l + ar * TR_PITCH + ak), b0, acc);
        acc = mfma16(*reinterpret_cast<const bf16x8*>(s_h + ar * TR_PITCH + 32 + ak), b1, acc);
        acc = mfma16(*reinterpret_cast<const bf16x8*>(s_l + ar * TR_PITCH + 32 + ak), b1, acc);
        if constexpr (QF32) {  // q_lo . k_hi: with the two above, fp32-accurate
            acc = mfma16(*reinterpret_cast<const bf16x8*>(s_h + ar * TR_PITCH + ak), b0l, acc);
            acc = mfma16(*reinterpret_cast<const bf16x8*>(s_h + ar * TR_PITCH + 32 + ak), b1l, acc);
        }
        const uint32_t pos = valid ? p0 + my : a.dummy_pos + my;
        *reinterpret_cast<f32x4*>(a.scores + (int64_t)pos * kTreeFanout + 4 * (lane >> 4)) = acc;
    }
}

struct TreeSelectArgs {
    const int32_t* slots;  // [rows][beam + 1]
    const uint32_t* rev;   // [beam + 1][rows] pair positions, ~0 when the slot is unused
    const float* scores;   // [npairs][16] by position
    int32_t* idx;          // [rows][top_k]
    int64_t rows;
    int N, bs, window, top_k, beam;  // N: rows per (b, head) (image mode: query blocks)
    int causal, nb;                  // image mode: every row's candidates are all nb blocks
};

// Compare-exchange toward descending order.
__device__ __forceinline__ void cx_desc(uint64_t& a, uint64_t& b) {
    const bool gt = a > b;
    const uint64_t hi = gt ? a : b, lo = gt ? b : a;
    a = hi;
    b = lo;
}

// Bitonic sort of 16 keys into descending order.
__device__ __forceinline__ void sort16_desc(uint64_t (&v)[kTreeFanout]) {
#pragma unroll
    for (int size = 2; size <= kTreeFanout; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < kTreeFanout; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    if ((i & size) == 0) cx_desc(v[i], v[j]);
                    else cx_desc(v[j], v[i]);
                }
            }
}

// One lane per row.  Per used slot the 16 block scores become 64-bit keys
// (score, then lower block; 0 for blocks past the row's candidates), are
// sorted, and merged into the row's running top-KM (KM = 16, or 32 for
// top_k above 16) by one bitonic merge: branch-free, so the lanes of a wave
// never wait on each other's insertions.  The next slot's scores are loaded
// while the current one is merged.
template <int KM>
__global__ __launch_bounds__(256) void k_tree_select(TreeSelectArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= a.rows) return;
    const int t = (int)(row % a.N);
    const int E = a.causal ? eligible_blocks(t, a.bs, a.window) : a.nb;
    const int stride = a.beam + 1;
    uint64_t L[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) L[j] = 0;
    int ncand = 0;
    auto fetch = [&](int j, f32x4 (&sc)[4], int& c0) {
        const uint32_t pos = j < stride ? a.rev[(int64_t)j * a.rows + row] : 0xFFFFFFFFu;
        c0 = -1;
        if (pos != 0xFFFFFFFFu) {
            c0 = a.slots[row * stride + j] * kTreeFanout;
            const f32x4* sp = reinterpret_cast<const f32x4*>(a.scores + (int64_t)pos * kTreeFanout);
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) sc[i4] = sp[i4];
        }
    };
    f32x4 cur[4], nxt[4];
    int c_cur, c_nxt;
    fetch(0, cur, c_cur);
    for (int j = 0; j < stride; ++j) {
        fetch(j + 1, nxt, c_nxt);
        if (c_cur >= 0) {
            const int nvalid = min(kTreeFanout, E - c_cur);
            ncand += nvalid;
            uint64_t Nk[kTreeFanout];
#pragma unroll
            for (int i = 0; i < kTreeFanout; ++i)
                Nk[i] = i < nvalid ? sel_key(cur[i >> 2][i & 3], (uint32_t)(c_cur + i)) : 0ull;
            sort16_desc(Nk);
            // the new keys, zero-padded to KM, reversed against L: the
            // pairwise maxima are the top KM of the union, in bitonic order
#pragma unroll
            for (int i = 0; i < KM; ++i) {
                const int jn = KM - 1 - i;
                if (jn < kTreeFanout) L[i] = L[i] > Nk[jn] ? L[i] : Nk[jn];
            }
#pragma unroll
            for (int stride2 = KM >> 1; stride2 > 0; stride2 >>= 1)
#pragma unroll
                for (int i = 0; i < KM; ++i) {
                    const int jx = i ^ stride2;
                    if (jx > i) cx_desc(L[i], L[jx]);
                }
        }
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) cur[i4] = nxt[i4];
        c_cur = c_nxt;
    }
    // the chosen blocks in ascending order, -1 padded
    const int m = ncand < a.top_k ? ncand : a.top_k;
    uint32_t cs[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) cs[j] = j < m ? key_block(L[j]) : 0xFFFFFFFFu;
#pragma unroll
    for (int size = 2; size <= KM; size <<= 1)
#pragma unroll
        for (int stride2 = size >> 1; stride2 > 0; stride2 >>= 1)
#pragma unroll
            for (int i = 0; i < KM; ++i) {
                const int jx = i ^ stride2;
                if (jx > i) {
                    const uint32_t x = cs[i], y = cs[jx];
                    const uint32_t mx = x > y ? x : y, mn = x > y ? y : x;
                    if ((i & size) == 0) { cs[i] = mn; cs[jx] = mx; }
                    else { cs[i] = mx; cs[jx] = mn; }
                }
            }
    int32_t* out = a.idx + row * a.top_k;
#pragma unroll
    for (int j = 0; j < KM; ++j)
        if (j < a.top_k) out[j] = j < m ? (int32_t)cs[j] : -1;
}

// ------------------------------------------------------------ host side
struct TreeLayout {
    size_t counts, offsets, cursor, unit_off, pairs, rev, scores, total;
    int nodes, NB;
};

static TreeLayout tree_layout(const Geometry& g) {
    TreeLayout L{};
    L.nodes = (g.nb + kTreeFanout - 1) / kTreeFanout;
    L.NB = g.B * g.Hkv * L.nodes;
    const size_t rows = (size_t)g.B * g.Hq * (g.causal ? (size_t)g.N : (size_t)g.nb);
    const size_t slots = (size_t)g.beam + 1;
    size_t off = 0;
    L.counts = off;   off += align_up(((size_t)L.NB + 1) * 4, 256);
    L.offsets = off;  off += align_up(((size_t)L.NB + 1) * 4, 256);
    L.cursor = off;   off += align_up(((size_t)L.NB + 1) * 4, 256);
    L.unit_off = off; off += align_up(((size_t)L.NB + 1) * 4, 256);
    L.pairs = off;    off += align_up(rows * slots * 4, 256);
    L.rev = off;      off += align_up(rows * slots * 4, 256);
    L.scores = off;   off += align_up((rows * slots + 64) * kTreeFanout * 4, 256);
    L.total = off;
    return L;
}

size_t tree_level2_bytes(const Geometry& g) { return tree_layout(g).total; }

hipError_t launch_tree_level2(const Geometry& g, const uint16_t* q, const float* qbar,
                              const uint16_t* bhi, const uint16_t* blo, int nb_pad,
                              const int32_t* slots, int32_t* idx, void* ws, hipStream_t s) {
    const TreeLayout L = tree_layout(g);
    char* base = static_cast<char*>(ws);
    uint32_t* counts = reinterpret_cast<uint32_t*>(base + L.counts);
    uint32_t* offsets = reinterpret_cast<uint32_t*>(base + L.offsets);
    uint32_t* cursor = reinterpret_cast<uint32_t*>(base + L.cursor);
    uint32_t* unit_off = reinterpret_cast<uint32_t*>(base + L.unit_off);
    uint32_t* pairs = reinterpret_cast<uint32_t*>(base + L.pairs);
    uint32_t* rev = reinterpret_cast<uint32_t*>(base + L.rev);
    float* scores = reinterpret_cast<float*>(base + L.scores);
    const int nslots = g.beam + 1;
    const int sp_log2 = pair_stride_log2(nslots);
    const int P = g.causal ? g.N : g.nb;  // rows per (b, query head)
    const int64_t rows = (int64_t)g.B * g.Hq * P;
    const int nbg = g.B * g.Hkv;

    hipError_t e = launch_fill_u32(counts, (size_t)L.NB, 0u, s);
    if (e != hipSuccess) return e;
    const int rep = g.Hq / g.Hkv;
    int64_t tc = std::max<int64_t>(
        (4096 + rep - 1) / rep,
        (4 * (int64_t)L.nodes + (int64_t)rep * nslots - 1) / ((int64_t)rep * nslots));
    tc = std::min<int64_t>((tc + 63) / 64 * 64, P);
    BucketArgs ba{slots, counts, cursor, pairs, rev, rows, g.Hq, g.Hkv, P, g.bs, L.nodes, nslots,
                  g.window, (int)tc, sp_log2, 0, kTreeFanoutLog2};
    if (!g.causal) ba.fixed_cand = L.nodes;  // every query block may open every node
    const int nch = (int)((P + tc - 1) / tc);
    const dim3 bgrid((unsigned)(nbg * nch));
    const size_t lds = L.nodes <= BK_LDS_MAX ? (size_t)L.nodes * 4 : 0;
    launch_bucket<false>(bgrid, lds, s, ba);
    hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(1024), 0, s, counts, offsets, cursor, unit_off,
                       L.NB, 1);
    launch_bucket<true>(bgrid, lds, s, ba);

    TreeScoreArgs sa{q, qbar, bhi, blo, pairs, offsets, unit_off, scores,
                     (uint32_t)(rows * nslots), L.nodes, L.NB, nb_pad, sp_log2};
    if (g.causal) {
        static std::atomic<int> cache[kMaxDevices];
        const int grid = resident_grid(k_tree_score<false>, 256, cache);
        hipLaunchKernelGGL(k_tree_score<false>, dim3(grid), dim3(256), 0, s, sa);
    } else {
        static std::atomic<int> cache[kMaxDevices];
        const int grid = resident_grid(k_tree_score<true>, 256, cache);
        hipLaunchKernelGGL(k_tree_score<true>, dim3(grid), dim3(256), 0, s, sa);
    }

    TreeSelectArgs ta{slots, rev, scores, idx, rows, P, g.bs, g.window, g.top_k, g.beam,
                      g.causal, g.nb};
    const dim3 sgrid((unsigned)((rows + 255) / 256));
    if (g.top_k <= kMaxTopK)
        hipLaunchKernelGGL(k_tree_select<kMaxTopK>, sgrid, dim3(256), 0, s, ta);
    else
        hipLaunchKernelGGL(k_tree_select<kMaxTopKWide>, sgrid, dim3(256), 0, s, ta);
    return hipGetLastError();
}

}  // namespace lsa
