// Bucketing of (row, slot) pairs by the block (or node) each slot selected,
// shared by the block-major attention and the second level of two-level
// routing: count per bucket (LDS histogram per workgroup), exclusive scans of
// bucket sizes and of 64-row work units, and a scatter that writes pair ids
// in bucket order together with a slot-major table of each pair's position.
#pragma once

#include "lsa_common.hpp"

namespace lsa {

constexpr int UNIT_ROWS = 64;      // gathered rows per work unit of the block-major kernels
constexpr int BK_LDS_MAX = 16384;  // largest bucket count per group histogrammed in LDS

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// The top_k entries of one idx row (16-byte loads when the row length
// allows); entries past top_k are left as they are.  KM: the list length
// the caller holds (kMaxTopK, or kMaxTopKWide for top_k above it).
template <int KM = kMaxTopK>
__device__ __forceinline__ void load_idx_row(const int32_t* ir, int top_k, int (&c)[KM]) {
    if ((top_k & 3) == 0) {
#pragma unroll
        for (int s4 = 0; s4 < KM / 4; ++s4) {
            if (4 * s4 < top_k) {
                const i32x4 v = *reinterpret_cast<const i32x4*>(ir + 4 * s4);
                c[4 * s4] = v[0]; c[4 * s4 + 1] = v[1]; c[4 * s4 + 2] = v[2]; c[4 * s4 + 3] = v[3];
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < KM; ++s)
            if (s < top_k) c[s] = ir[s];
    }
}

// The same with the row's length fixed at compile time: KV 16-byte loads
// (top_k = 4 * KV), or, for KV = 0, the runtime-length form above.  Fixed
// lengths leave no guard between the loads of consecutive rows, so a
// thread's loads for several rows issue back to back.
template <int KV, int KM = kMaxTopK>
__device__ __forceinline__ void load_idx_row_kv(const int32_t* ir, int top_k, int (&c)[KM]) {
    static_assert(4 * KV <= KM, "row longer than the list");
    if constexpr (KV == 0) {
        load_idx_row<KM>(ir, top_k, c);
    } else {
#pragma unroll
        for (int s4 = 0; s4 < KV; ++s4) {
            const i32x4 v = *reinterpret_cast<const i32x4*>(ir + 4 * s4);
            c[4 * s4] = v[0]; c[4 * s4 + 1] = v[1]; c[4 * s4 + 2] = v[2]; c[4 * s4 + 3] = v[3];
        }
    }
}

// Used-slot mask of loaded idx entries: an entry counts when it is a
// candidate (< ncand) and larger than the previously used entry.
template <int KM = kMaxTopK>
__device__ __forceinline__ uint32_t used_mask(const int (&c)[KM], int top_k, int ncand) {
    uint32_t mask = 0;
    int prev = -1;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        if (s < top_k && c[s] > prev && c[s] < ncand) {
            mask |= 1u << s;
            prev = c[s];
        }
    }
    return mask;
}

// Used-slot mask of one idx row, loading it.
template <int KM = kMaxTopK>
__device__ __forceinline__ uint32_t row_used(const int32_t* ir, int top_k, int ncand,
                                             int (&c)[KM]) {
    load_idx_row<KM>(ir, top_k, c);
    return used_mask<KM>(c, top_k, ncand);
}


// ------------------------------------------------------------ bucketing
struct BucketArgs {
    const int32_t* idx;  // [B,Hq,N,top_k]; group_route: [B,Hkv,N,top_k]
    uint32_t* counts;    // [NB]
    uint32_t* cursor;    // [NB]
    uint32_t* pairs;     // [total pairs]
    uint32_t* rev;       // [top_k][rows], slot-major: position of pair (row, slot), ~0 if unused
    int64_t rows;        // B * Hq * N
    int Hq, Hkv, N, bs, nb, top_k, window, tchunk, sp_log2;
    int group_route;     // 1: one route per KV group, shared by its query heads
    // group_pairs (requires group_route): pairs are (group row, slot), one per
    // position and slot for all the group's query heads; rows (of rev and of
    // pair ids) are then the B * Hkv * N group rows, bg * N + t.
    int cshift;          // buckets group 2^cshift blocks: a row's candidate buckets are
                         // ceil(E(t) / 2^cshift) (0: buckets are blocks)
    // Position chunks (pc_log2 >= 0): buckets are (chunk, b * Hkv + g, block)
    // with chunk = t >> pc_log2, and pair ids are chunk-local: row (bh, t) is
    // local row bh * 2^pc_log2 + (t mod 2^pc_log2).  A workgroup's positions
    // must lie in one chunk (tchunk divides 2^pc_log2).  pc_log2 < 0: buckets
    // are (b * Hkv + g, block) and pair ids use the global row bh * N + t.
    int pc_log2 = -1;
    int nbg = 0;         // B * Hkv (with position chunks)
    int fixed_cand = 0;  // > 0: every row's candidate buckets (image-mode rows); else causal
    int group_pairs = 0;
    // with position chunks: buckets are (t >> bc_log2, b * Hkv + g, block),
    // bucket chunks no longer than the chunks (-1: bc_log2 = pc_log2)
    int bc_log2 = -1;
};

__device__ __forceinline__ int bucket_candidates(const BucketArgs& a, int t) {
    if (a.fixed_cand > 0) return a.fixed_cand;
    const int e = eligible_blocks(t, a.bs, a.window);
    return (e + (1 << a.cshift) - 1) >> a.cshift;
}

// Writes one row's entries of the slot-major position table, so that the
// lanes of a wave (consecutive rows) store consecutive words.
template <int KM = kMaxTopK>
__device__ __forceinline__ void write_rev_row(uint32_t* rev, int64_t rows, int64_t row,
                                              const uint32_t (&pos)[KM], int top_k) {
#pragma unroll
    for (int s = 0; s < KM; ++s)
        if (s < top_k) rev[s * rows + row] = pos[s];
}

// Threads per bucketing workgroup: a launch has only a few workgroups per CU
// (one per few thousand rows), so each brings many waves; the longer row
// lists (wide or runtime-length rows) hold more registers and take fewer.
template <int KV, int KM>
constexpr int bucket_threads() { return (KM > kMaxTopK || KV == 0) ? 512 : 1024; }

// Workgroup = (batch, KV head, chunk of tchunk positions) over all query
// heads of the group.  Histogram in LDS (when nb fits), then one global
// atomic per touched bucket: counts (SCATTER = false) or a reserved range
// of the pair list that pass B fills (SCATTER = true).
// KV: the idx row length in 16-byte vectors when top_k is a multiple of 4
// (top_k = 4 * KV), else 0.  KM: the row list length held per row
// (kMaxTopK, or kMaxTopKWide for top_k above it).
template <bool SCATTER, int KV, int KM>
__global__ __launch_bounds__((bucket_threads<KV, KM>())) void k_bucket(BucketArgs a) {
    constexpr int BT = bucket_threads<KV, KM>();
    extern __shared__ uint32_t s_h[];
    const int tid = threadIdx.x;
    const int nch = (a.N + a.tchunk - 1) / a.tchunk;
    const int bg = blockIdx.x / nch, ch = blockIdx.x - bg * nch;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int rep = a.Hq / a.Hkv;
    const int t0 = ch * a.tchunk, t1 = min(a.N, t0 + a.tchunk);
    const int span = t1 - t0;
    const bool lds = a.nb <= BK_LDS_MAX;
    const bool chunked = a.pc_log2 >= 0;
    const int bc_log2 = a.bc_log2 >= 0 ? a.bc_log2 : a.pc_log2;
    const int64_t bucket0 =
        chunked ? ((int64_t)(t0 >> bc_log2) * a.nbg + bg) * a.nb : (int64_t)bg * a.nb;
    // heads walked per position: the group's query heads, or one group row
    const int nh = a.group_pairs ? 1 : rep;
    // row (of rev) and idx row of head hh at position t
    auto row_of = [&](int hh, int t) -> int64_t {
        return a.group_pairs ? (int64_t)bg * a.N + t : ((int64_t)b * a.Hq + g * rep + hh) * a.N + t;
    };
    // pair-id row of head hh (group pairs: the group row) at position t
    auto pair_row = [&](int hh, int t, int64_t row) -> int64_t {
        if (!chunked) return row;
        const int64_t r = a.group_pairs ? (int64_t)bg : (int64_t)b * a.Hq + g * rep + hh;
        return (r << a.pc_log2) + (t & ((1 << a.pc_log2) - 1));
    };
    const int total = nh * span;
    if (!lds) {
        // block counts beyond the LDS histogram: global atomics per pair
        for (int i = tid; i < total; i += BT) {
            const int hh = i / span, t = t0 + (i - hh * span);
            const int64_t row = row_of(hh, t);
            const int64_t irow = a.group_route ? (int64_t)bg * a.N + t : row;
            int c[KM];
            uint32_t m = row_used<KM>(a.idx + irow * a.top_k, a.top_k, bucket_candidates(a, t), c);
            uint32_t posv[KM];
#pragma unroll
            for (int s = 0; s < KM; ++s) {
                posv[s] = 0xFFFFFFFFu;
                if (!((m >> s) & 1u)) continue;
                if (!SCATTER) {
                    atomicAdd(&a.counts[bucket0 + c[s]], 1u);
                } else {
                    const uint32_t pos = atomicAdd(&a.cursor[bucket0 + c[s]], 1u);
                    a.pairs[pos] = (uint32_t)((pair_row(hh, t, row) << a.sp_log2) | s);
                    posv[s] = pos;
                }
            }
            if (SCATTER) write_rev_row<KM>(a.rev, a.rows, row, posv, a.top_k);
        }
        return;
    }
    // The LDS passes walk BU rows per thread per step: every idx load of the
    // step is issued before the first mask needs one (a thread past the end
    // loads the chunk's last row and drops it).
    constexpr int BU = KM > kMaxTopK ? 2 : 4;
    struct Rows {
        int c[BU][KM];
        int t[BU], hh[BU];
    };
    auto load_rows = [&](int i0, Rows& r) {
#pragma unroll
        for (int u = 0; u < BU; ++u) {
            const int i = min(i0 + BT * u, total - 1);
            r.hh[u] = i / span;
            r.t[u] = t0 + (i - r.hh[u] * span);
            const int64_t irow = a.group_route ? (int64_t)bg * a.N + r.t[u] : row_of(r.hh[u], r.t[u]);
            load_idx_row_kv<KV, KM>(a.idx + irow * a.top_k, a.top_k, r.c[u]);
        }
    };
    for (int c = tid; c < a.nb; c += BT) s_h[c] = 0;
    __syncthreads();
    for (int i0 = tid; i0 < total; i0 += BT * BU) {
        Rows r;
        load_rows(i0, r);
#pragma unroll
        for (int u = 0; u < BU; ++u) {
            const uint32_t m = (i0 + BT * u < total)
                                   ? used_mask<KM>(r.c[u], a.top_k, bucket_candidates(a, r.t[u]))
                                   : 0u;
#pragma unroll
            for (int s = 0; s < KM; ++s)
                if ((m >> s) & 1u) atomicAdd(&s_h[r.c[u][s]], 1u);
        }
    }
    __syncthreads();
    for (int cc = tid; cc < a.nb; cc += BT) {
        const uint32_t n = s_h[cc];
        if (!SCATTER) {
            if (n) atomicAdd(&a.counts[bucket0 + cc], n);
        } else {
            s_h[cc] = n ? atomicAdd(&a.cursor[bucket0 + cc], n) : 0u;  // reserved base
        }
    }
    if (!SCATTER) return;
    __syncthreads();
    for (int i0 = tid; i0 < total; i0 += BT * BU) {
        Rows r;
        load_rows(i0, r);
#pragma unroll
        for (int u = 0; u < BU; ++u) {
            if (i0 + BT * u >= total) break;
            const uint32_t m = used_mask<KM>(r.c[u], a.top_k, bucket_candidates(a, r.t[u]));
            const int64_t row = row_of(r.hh[u], r.t[u]);
            // all LDS reservations first (their latencies overlap), then the stores
            uint32_t posv[KM];
#pragma unroll
            for (int s = 0; s < KM; ++s)
                posv[s] = ((m >> s) & 1u) ? atomicAdd(&s_h[r.c[u][s]], 1u) : 0xFFFFFFFFu;
            const int64_t prow = pair_row(r.hh[u], r.t[u], row);
#pragma unroll
            for (int s = 0; s < KM; ++s)
                if ((m >> s) & 1u) a.pairs[posv[s]] = (uint32_t)((prow << a.sp_log2) | s);
            write_rev_row<KM>(a.rev, a.rows, row, posv, a.top_k);
        }
    }
}

template <bool SCATTER, int KV, int KM>
static inline void launch_bucket_kv(dim3 grid, size_t lds, hipStream_t s, const BucketArgs& a) {
    hipLaunchKernelGGL((k_bucket<SCATTER, KV, KM>), grid, dim3(bucket_threads<KV, KM>()), lds, s, a);
}

// Launches k_bucket<SCATTER, KV, KM> with KV and KM picked from a.top_k.
template <bool SCATTER>
static inline void launch_bucket(dim3 grid, size_t lds, hipStream_t s, const BucketArgs& a) {
    constexpr int K = kMaxTopK, W = kMaxTopKWide;
    switch ((a.top_k & 3) == 0 ? a.top_k / 4 : 0) {
        case 1: launch_bucket_kv<SCATTER, 1, K>(grid, lds, s, a); break;
        case 2: launch_bucket_kv<SCATTER, 2, K>(grid, lds, s, a); break;
        case 3: launch_bucket_kv<SCATTER, 3, K>(grid, lds, s, a); break;
        case 4: launch_bucket_kv<SCATTER, 4, K>(grid, lds, s, a); break;
        case 5: launch_bucket_kv<SCATTER, 5, W>(grid, lds, s, a); break;
        case 6: launch_bucket_kv<SCATTER, 6, W>(grid, lds, s, a); break;
        case 7: launch_bucket_kv<SCATTER, 7, W>(grid, lds, s, a); break;
        case 8: launch_bucket_kv<SCATTER, 8, W>(grid, lds, s, a); break;
        default:
            if (a.top_k <= K)
                launch_bucket_kv<SCATTER, 0, K>(grid, lds, s, a);
            else
                launch_bucket_kv<SCATTER, 0, W>(grid, lds, s, a);
            break;
    }
}

// Exclusive scans of bucket sizes and of work units (ceil(count * expand /
// UNIT_ROWS): each pair stands for `expand` gathered rows); cursor starts at
// the bucket offsets.  Workgroup w scans segment w of the buckets (segments
// of a multiple of four buckets); its base is the sum over the buckets
// before the segment, which it reads itself (coalesced), so the workgroups
// need nothing from each other.  Any grid size is correct.
static __global__ __launch_bounds__(1024) void k_bucket_scan(const uint32_t* __restrict__ counts,
                                                      uint32_t* __restrict__ offsets,
                                                      uint32_t* __restrict__ cursor,
                                                      uint32_t* __restrict__ unit_off, int NB,
                                                      int expand) {
    __shared__ uint32_t s_p[1024], s_u[1024];
    const int tid = threadIdx.x;
    const int seg = ((NB + (int)gridDim.x - 1) / (int)gridDim.x + 3) & ~3;
    const int s0 = min(NB, (int)blockIdx.x * seg), s1 = min(NB, s0 + seg);
    // inclusive block scan of (s_p, s_u)
    auto block_scan = [&]() {
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele
            const uint32_t ap = tid >= off ? s_p[tid - off] : 0u;
            const uint32_t au = tid >= off ? s_u[tid - off] : 0u;
            __syncthreads();
            s_p[tid] += ap;
            s_u[tid] += au;
            __syncthreads();
        }
    };
    uint32_t base_p = 0, base_u = 0;
    if (s0 > 0) {
        uint32_t bp = 0, bu = 0;
        for (int i = tid; i < s0; i += 1024) {
            const uint32_t n = counts[i];
            bp += n;
            bu += (n * expand + UNIT_ROWS - 1) / UNIT_ROWS;
        }
        s_p[tid] = bp;
        s_u[tid] = bu;
        block_scan();
        base_p = s_p[1023];
        base_u = s_u[1023];
        __syncthreads();  // every thread has read the totals before s_p is reused
    }
    const int per = ((s1 - s0 + 1023) / 1024 + 3) & ~3;
    const int lo = min(s1, s0 + tid * per), hi = min(s1, lo + per);
    auto load4 = [&](int i) {
        if (i + 4 <= NB) return *reinterpret_cast<const u32x4*>(counts + i);
        u32x4 r = {0u, 0u, 0u, 0u};
        for (int j = 0; j < 4; ++j)
            if (i + j < NB) r[j] = counts[i + j];
        return r;
    };
    uint32_t sp = 0, su = 0;
#pragma unroll 4
    for (int i = lo; i < hi; i += 4) {
        const u32x4 n = load4(i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sp += n[j];
            su += (n[j] * expand + UNIT_ROWS - 1) / UNIT_ROWS;
        }
    }
    s_p[tid] = sp;
    s_u[tid] = su;
    block_scan();
    uint32_t rp = base_p + s_p[tid] - sp, ru = base_u + s_u[tid] - su;
#pragma unroll 4
    for (int i = lo; i < hi; i += 4) {
        const u32x4 n = load4(i);
        u32x4 o, u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[j] = rp;
            u[j] = ru;
            rp += n[j];
            ru += (n[j] * expand + UNIT_ROWS - 1) / UNIT_ROWS;
        }
        if (i + 4 <= NB) {
            *reinterpret_cast<u32x4*>(offsets + i) = o;
            *reinterpret_cast<u32x4*>(cursor + i) = o;
            *reinterpret_cast<u32x4*>(unit_off + i) = u;
        } else {
            for (int j = 0; j < 4 && i + j < NB; ++j) {
                offsets[i + j] = o[j];
                cursor[i + j] = o[j];
                unit_off[i + j] = u[j];
            }
        }
    }
    if (tid == 1023 && s1 == NB && (s0 < NB || blockIdx.x == 0)) {
        offsets[NB] = base_p + s_p[1023];
        unit_off[NB] = base_u + s_u[1023];
    }
}

// Wave-uniform read of a table that the kernel never writes, through the
// constant address space so that it becomes a scalar load: a vector load
// here would make the wave wait for all of its outstanding vector memory
// operations, prefetches included.
__device__ __forceinline__ uint32_t uniform_load(const uint32_t* p) {
    return *(const __attribute__((address_space(4))) uint32_t*)p;
}

// Work units (64 gathered rows of one bucket) are split into contiguous
// ranges per workgroup, so K/V of a bucket are staged once for all its units.
// Gathered rows are numbered expand * (pair position) + (0 .. expand - 1).
struct UnitCursor {
    int bucket;
    __device__ void seek(const uint32_t* unit_off, int NB, uint32_t u) {
        int lo = 0, hi = NB;  // last bucket b with unit_off[b] <= u
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (uniform_load(unit_off + mid) <= u) lo = mid; else hi = mid;
        }
        bucket = lo;
    }
    // Gathered rows [p0, p1) of unit u (u >= the unit of the previous call).
    __device__ void rows(const uint32_t* unit_off, const uint32_t* offsets, uint32_t u,
                         uint32_t& p0, uint32_t& p1, uint32_t expand = 1) {
        while (uniform_load(unit_off + bucket + 1) <= u) ++bucket;
        p0 = uniform_load(offsets + bucket) * expand +
             (u - uniform_load(unit_off + bucket)) * UNIT_ROWS;
        p1 = min(p0 + UNIT_ROWS, uniform_load(offsets + bucket + 1) * expand);
    }
};


}  // namespace lsa
