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

// Used-slot mask of one idx row: an entry counts when it is a candidate
// (< ncand) and larger than the previously used entry.  Read with 16-byte
// loads when the row length allows.
__device__ __forceinline__ uint32_t row_used(const int32_t* ir, int top_k, int ncand,
                                             int (&c)[kMaxTopK]) {
    if ((top_k & 3) == 0) {
#pragma unroll
        for (int s4 = 0; s4 < kMaxTopK / 4; ++s4) {
            if (4 * s4 < top_k) {
                const i32x4 v = *reinterpret_cast<const i32x4*>(ir + 4 * s4);
                c[4 * s4] = v[0]; c[4 * s4 + 1] = v[1]; c[4 * s4 + 2] = v[2]; c[4 * s4 + 3] = v[3];
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s)
            if (s < top_k) c[s] = ir[s];
    }
    uint32_t mask = 0;
    int prev = -1;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s < top_k && c[s] > prev && c[s] < ncand) {
            mask |= 1u << s;
            prev = c[s];
        }
    }
    return mask;
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
    int cshift;          // buckets group 2^cshift blocks: a row's candidate buckets are
                         // ceil(E(t) / 2^cshift) (0: buckets are blocks)
};

__device__ __forceinline__ int bucket_candidates(const BucketArgs& a, int t) {
    const int e = eligible_blocks(t, a.bs, a.window);
    return (e + (1 << a.cshift) - 1) >> a.cshift;
}

// Writes one row's entries of the slot-major position table, so that the
// lanes of a wave (consecutive rows) store consecutive words.
__device__ __forceinline__ void write_rev_row(uint32_t* rev, int64_t rows, int64_t row,
                                              const uint32_t (&pos)[kMaxTopK], int top_k) {
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        if (s < top_k) rev[s * rows + row] = pos[s];
}

// Workgroup = (batch, KV head, chunk of tchunk positions) over all query
// heads of the group.  Histogram in LDS (when nb fits), then one global
// atomic per touched bucket: counts (SCATTER = false) or a reserved range
// of the pair list that pass B fills (SCATTER = true).
template <bool SCATTER>
__global__ __launch_bounds__(256) void k_bucket(BucketArgs a) {
    extern __shared__ uint32_t s_h[];
    const int tid = threadIdx.x;
    const int nch = (a.N + a.tchunk - 1) / a.tchunk;
    const int bg = blockIdx.x / nch, ch = blockIdx.x - bg * nch;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int rep = a.Hq / a.Hkv;
    const int t0 = ch * a.tchunk, t1 = min(a.N, t0 + a.tchunk);
    const int span = t1 - t0;
    const bool lds = a.nb <= BK_LDS_MAX;
    const int64_t bucket0 = (int64_t)bg * a.nb;
    if (lds) {
        for (int c = tid; c < a.nb; c += 256) s_h[c] = 0;
        __syncthreads();
    }
    for (int i = tid; i < rep * span; i += 256) {
        const int hh = i / span, t = t0 + (i - hh * span);
        const int64_t row = ((int64_t)b * a.Hq + g * rep + hh) * a.N + t;
        const int64_t irow = a.group_route ? (int64_t)bg * a.N + t : row;
        int c[kMaxTopK];
        uint32_t m = row_used(a.idx + irow * a.top_k, a.top_k, bucket_candidates(a, t), c);
        uint32_t posv[kMaxTopK];
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s) {
            posv[s] = 0xFFFFFFFFu;
            if (!((m >> s) & 1u)) continue;
            if (lds) {
                atomicAdd(&s_h[c[s]], 1u);
            } else if (!SCATTER) {
                atomicAdd(&a.counts[bucket0 + c[s]], 1u);
            } else {
                const uint32_t pos = atomicAdd(&a.cursor[bucket0 + c[s]], 1u);
                a.pairs[pos] = (uint32_t)((row << a.sp_log2) | s);
                posv[s] = pos;
            }
        }
        if (SCATTER && !lds) write_rev_row(a.rev, a.rows, row, posv, a.top_k);
    }
    if (!lds) return;
    __syncthreads();
    for (int cc = tid; cc < a.nb; cc += 256) {
        const uint32_t n = s_h[cc];
        if (!SCATTER) {
            if (n) atomicAdd(&a.counts[bucket0 + cc], n);
        } else {
            s_h[cc] = n ? atomicAdd(&a.cursor[bucket0 + cc], n) : 0u;  // reserved base
        }
    }
    if (!SCATTER) return;
    __syncthreads();
    for (int i = tid; i < rep * span; i += 256) {
        const int hh = i / span, t = t0 + (i - hh * span);
        const int64_t row = ((int64_t)b * a.Hq + g * rep + hh) * a.N + t;
        const int64_t irow = a.group_route ? (int64_t)bg * a.N + t : row;
        int c[kMaxTopK];
        uint32_t m = row_used(a.idx + irow * a.top_k, a.top_k, bucket_candidates(a, t), c);
        // all LDS reservations first (their latencies overlap), then the stores
        uint32_t posv[kMaxTopK];
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s)
            posv[s] = ((m >> s) & 1u) ? atomicAdd(&s_h[c[s]], 1u) : 0xFFFFFFFFu;
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s)
            if ((m >> s) & 1u) a.pairs[posv[s]] = (uint32_t)((row << a.sp_log2) | s);
        write_rev_row(a.rev, a.rows, row, posv, a.top_k);
    }
}

// Single workgroup: exclusive scans of bucket sizes and of work units
// (ceil(count / UNIT_ROWS)); cursor starts at the bucket offsets.
static __global__ __launch_bounds__(1024) void k_bucket_scan(const uint32_t* __restrict__ counts,
                                                      uint32_t* __restrict__ offsets,
                                                      uint32_t* __restrict__ cursor,
                                                      uint32_t* __restrict__ unit_off, int NB) {
    __shared__ uint32_t s_p[1024], s_u[1024];
    const int tid = threadIdx.x;
    const int per = (NB + 1023) / 1024;
    const int lo = min(NB, tid * per), hi = min(NB, lo + per);
    uint32_t sp = 0, su = 0;
#pragma unroll 8
    for (int i = lo; i < hi; ++i) {
        const uint32_t n = counts[i];
        sp += n;
        su += (n + UNIT_ROWS - 1) / UNIT_ROWS;
    }
    s_p[tid] = sp;
    s_u[tid] = su;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
        const uint32_t ap = tid >= off ? s_p[tid - off] : 0u;
        const uint32_t au = tid >= off ? s_u[tid - off] : 0u;
        __syncthreads();
        s_p[tid] += ap;
        s_u[tid] += au;
        __syncthreads();
    }
    uint32_t rp = s_p[tid] - sp, ru = s_u[tid] - su;
#pragma unroll 8
    for (int i = lo; i < hi; ++i) {
        const uint32_t n = counts[i];
        offsets[i] = rp;
        cursor[i] = rp;
        unit_off[i] = ru;
        rp += n;
        ru += (n + UNIT_ROWS - 1) / UNIT_ROWS;
    }
    if (tid == 1023) {
        offsets[NB] = s_p[1023];
        unit_off[NB] = s_u[1023];
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
    // Rows [p0, p1) of unit u (u >= the unit of the previous call).
    __device__ void rows(const uint32_t* unit_off, const uint32_t* offsets, uint32_t u,
                         uint32_t& p0, uint32_t& p1) {
        while (uniform_load(unit_off + bucket + 1) <= u) ++bucket;
        p0 = uniform_load(offsets + bucket) + (u - uniform_load(unit_off + bucket)) * UNIT_ROWS;
        p1 = min(p0 + UNIT_ROWS, uniform_load(offsets + bucket + 1));
    }
};


}  // namespace lsa
