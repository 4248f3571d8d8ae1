// Exact softmax attention over the selected keys only (SSA page, opening
// paragraph; Subquadratic Sparse Attention page, "Architecture": selected
// attention alongside a causal sliding window).
//
// Causal mode runs key-block-major, because every query routes to its own
// blocks and a query-major gather would reuse nothing:
//   1. k_bucket<false>  counts, per (b, KV head, key block), the (row, slot)
//                       pairs that selected it (LDS histogram per workgroup).
//   2. k_bucket_scan    bucket offsets and the work units (64 rows each).
//   3. k_bucket<true>   scatters pair ids into bucket order.
//   4. k_block_partial  one K/V block in LDS against up to 64 gathered query
//                       rows: S = Q K^T and O = P V on bf16 MFMA; writes the
//                       normalised partial output (bf16) and its log-sum-exp.
//   5. k_window_merge   flash-style online softmax over the block-aligned
//                       window [bs*E(t), t] with a causal mask, then merges
//                       the row's routed partials with the append law of the
//                       SSA page ("Mathematical status": adding mass a to mass
//                       Z moves the read by a/(Z+a) times the displacement of
//                       the new value), and writes fp32 output.
// Image mode (k_image_attend): one wave per 16-token query block; its
// selected 16-key blocks are gathered straight into MFMA operands.
//
// MFMA orientation: S^T = K . Q^T on 16x16x32 tiles, so lane l holds query
// row l%16 and keys 16i + 4(l/16) + r.  Those probabilities are exactly the
// B operand of O^T = V^T . P^T when key slot j of lane l stands for key
// 32s + 4(l/16) + j (j < 4) or 32s + 16 + 4(l/16) + (j-4): no cross-lane
// movement.  V is staged transposed in LDS (4x4 register transposes).
// Softmax runs in the log2 domain: logits are scaled by scale*log2(e).
#include <math.h>

#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

constexpr int UNIT_ROWS = 64;   // gathered rows per work unit of the block-major kernel
constexpr int BK_TCHUNK = 2048; // query positions per bucketing workgroup
constexpr int BK_LDS_MAX = 16384;  // largest nb histogrammed in LDS
constexpr int KPITCH = 72;      // LDS pitch of K tiles [key][64 d] (bf16)
constexpr int PART_GRID = 2048; // workgroups of the persistent block-major kernel

// ------------------------------------------------------------ shared pieces
// Stages K rows [0, nkeys) of a tile into s_k[key][KPITCH] (16-byte chunks);
// rows >= valid are zero.
__device__ __forceinline__ void stage_k(__bf16* s_k, const uint16_t* src, int nkeys, int valid,
                                        int tid, int nthreads) {
    for (int ch = tid; ch < nkeys * 8; ch += nthreads) {
        const int key = ch >> 3, d0 = (ch & 7) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (key < valid) v = *reinterpret_cast<const u32x4*>(src + (int64_t)key * kD + d0);
        *reinterpret_cast<u32x4*>(s_k + key * KPITCH + d0) = v;
    }
}

// Stages V rows [0, nkeys) transposed into s_vt[d][vpitch] with 4x4
// register transposes; rows >= valid are zero.
__device__ __forceinline__ void stage_vt(__bf16* s_vt, int vpitch, const uint16_t* src,
                                         int nkeys, int valid, int tid, int nthreads) {
    const int kgroups = nkeys >> 2;
    for (int t = tid; t < kgroups * 16; t += nthreads) {
        const int kg = t % kgroups, dg = t / kgroups;
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kg * 4 + i;
            u32x2 v = {0u, 0u};
            if (key < valid) v = *reinterpret_cast<const u32x2*>(src + (int64_t)key * kD + dg * 4);
            lo[i] = v[0];  // d = 4dg, 4dg+1
            hi[i] = v[1];  // d = 4dg+2, 4dg+3
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t* w = (j < 2) ? lo : hi;
            const int sh = (j & 1) * 16;
            const uint32_t e0 = (w[0] >> sh) & 0xFFFFu, e1 = (w[1] >> sh) & 0xFFFFu;
            const uint32_t e2 = (w[2] >> sh) & 0xFFFFu, e3 = (w[3] >> sh) & 0xFFFFu;
            u32x2 packed = {e0 | (e1 << 16), e2 | (e3 << 16)};
            *reinterpret_cast<u32x2*>(s_vt + (dg * 4 + j) * vpitch + kg * 4) = packed;
        }
    }
}

// Q rows as the B operand of S^T = K Q^T: dims 8(l/16) + 32ks .. +7.
__device__ __forceinline__ void load_q_operand(const uint16_t* qrow, int lane, bool valid,
                                               bf16x8 (&Bq)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        if (valid)
            Bq[ks] = load_bf16x8(qrow + 8 * (lane >> 4) + 32 * ks);
        else
            Bq[ks] = bf16x8{};
    }
}

// S^T tile for keys [16i, 16i+16) of an LDS K tile.
__device__ __forceinline__ f32x4 score_tile(const __bf16* s_k, int i, int lane,
                                            const bf16x8 (&Bq)[2]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 A =
            *reinterpret_cast<const bf16x8*>(s_k + (16 * i + (lane & 15)) * KPITCH + 8 * (lane >> 4) + 32 * ks);
        acc = mfma16(A, Bq[ks], acc);
    }
    return acc;
}

// O^T += V^T P^T over KT 16-key tiles whose probabilities are p[i][r]
// (key 16i + 4(l/16) + r); V^T tile in LDS with pitch vpitch.
template <int KT>
__device__ __forceinline__ void pv_accumulate(const __bf16* s_vt, int vpitch, int lane,
                                              const float (&p)[KT][4], f32x4 (&o)[4]) {
    constexpr int KS = (KT + 1) / 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        bf16x8 Bp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Bp[j] = (__bf16)p[2 * s][j];
            Bp[4 + j] = (2 * s + 1 < KT) ? (__bf16)p[2 * s + 1][j] : (__bf16)0.f;
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const __bf16* vr = s_vt + (16 * mt + (lane & 15)) * vpitch + 32 * s + 4 * (lane >> 4);
            const u32x2 a0 = *reinterpret_cast<const u32x2*>(vr);
            u32x2 a1 = {0u, 0u};
            if (2 * s + 1 < KT) a1 = *reinterpret_cast<const u32x2*>(vr + 16);
            const u32x4 araw = {a0[0], a0[1], a1[0], a1[1]};
            o[mt] = mfma16(__builtin_bit_cast(bf16x8, araw), Bp, o[mt]);
        }
    }
}

// Slot of the n-th set bit of a mask (n < popcount(mask)).
__device__ __forceinline__ int nth_slot(uint32_t mask, int n) {
    for (int i = 0; i < n; ++i) mask &= mask - 1;
    return __builtin_ctz(mask);
}

// Row reductions across the 4 lanes that share row l%16.
__device__ __forceinline__ float row_max4(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, kWave));
    return fmaxf(v, __shfl_xor(v, 32, kWave));
}
__device__ __forceinline__ float row_sum4(float v) {
    v += __shfl_xor(v, 16, kWave);
    return v + __shfl_xor(v, 32, kWave);
}

// ------------------------------------------------------------ bucketing
struct BucketArgs {
    const int32_t* idx;  // [B,Hq,N,top_k]
    uint32_t* counts;    // [NB]
    uint32_t* cursor;    // [NB]
    uint32_t* pairs;     // [total pairs]
    int Hq, Hkv, N, bs, nb, top_k, window;
};

template <bool SCATTER>
__global__ __launch_bounds__(256) void k_bucket(BucketArgs a) {
    extern __shared__ uint32_t s_h[];
    const int tid = threadIdx.x;
    const int nch = (a.N + BK_TCHUNK - 1) / BK_TCHUNK;
    const int bg = blockIdx.x / nch, ch = blockIdx.x - bg * nch;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int rep = a.Hq / a.Hkv;
    const int t0 = ch * BK_TCHUNK, t1 = min(a.N, t0 + BK_TCHUNK);
    const int span = t1 - t0;
    const bool lds = a.nb <= BK_LDS_MAX;
    const int64_t bucket0 = (int64_t)bg * a.nb;
    if (lds) {
        for (int c = tid; c < a.nb; c += 256) s_h[c] = 0;
        __syncthreads();
    }
    // pass A: local histogram (or, without LDS, direct global work)
    for (int i = tid; i < rep * span; i += 256) {
        const int hh = i / span, t = t0 + (i - hh * span);
        const int64_t row = ((int64_t)b * a.Hq + g * rep + hh) * a.N + t;
        const int32_t* ir = a.idx + row * a.top_k;
        uint32_t m = used_slots(ir, a.top_k, eligible_blocks(t, a.bs, a.window));
        while (m) {
            const int s = __builtin_ctz(m);
            m &= m - 1;
            const int c = ir[s];
            if (lds) {
                atomicAdd(&s_h[c], 1u);
            } else if (!SCATTER) {
                atomicAdd(&a.counts[bucket0 + c], 1u);
            } else {
                const uint32_t pos = atomicAdd(&a.cursor[bucket0 + c], 1u);
                a.pairs[pos] = (uint32_t)(row * a.top_k + s);
            }
        }
    }
    if (!lds) return;
    __syncthreads();
    for (int c = tid; c < a.nb; c += 256) {
        const uint32_t n = s_h[c];
        if (!SCATTER) {
            if (n) atomicAdd(&a.counts[bucket0 + c], n);
        } else {
            s_h[c] = n ? atomicAdd(&a.cursor[bucket0 + c], n) : 0u;  // reserved base
        }
    }
    if (!SCATTER) return;
    __syncthreads();
    // pass B: place the pairs
    for (int i = tid; i < rep * span; i += 256) {
        const int hh = i / span, t = t0 + (i - hh * span);
        const int64_t row = ((int64_t)b * a.Hq + g * rep + hh) * a.N + t;
        const int32_t* ir = a.idx + row * a.top_k;
        uint32_t m = used_slots(ir, a.top_k, eligible_blocks(t, a.bs, a.window));
        while (m) {
            const int s = __builtin_ctz(m);
            m &= m - 1;
            const uint32_t pos = atomicAdd(&s_h[ir[s]], 1u);
            a.pairs[pos] = (uint32_t)(row * a.top_k + s);
        }
    }
}

// Single workgroup: exclusive scans of bucket sizes and of work units
// (ceil(count / UNIT_ROWS)); cursor starts at the bucket offsets.
__global__ __launch_bounds__(1024) void k_bucket_scan(const uint32_t* __restrict__ counts,
                                                      uint32_t* __restrict__ offsets,
                                                      uint32_t* __restrict__ cursor,
                                                      uint32_t* __restrict__ unit_off, int NB) {
    __shared__ uint32_t s_p[1024], s_u[1024];
    const int tid = threadIdx.x;
    const int per = (NB + 1023) / 1024;
    const int lo = min(NB, tid * per), hi = min(NB, lo + per);
    uint32_t sp = 0, su = 0;
    for (int i = lo; i < hi; ++i) {
        sp += counts[i];
        su += (counts[i] + UNIT_ROWS - 1) / UNIT_ROWS;
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
    for (int i = lo; i < hi; ++i) {
        offsets[i] = rp;
        cursor[i] = rp;
        unit_off[i] = ru;
        rp += counts[i];
        ru += (counts[i] + UNIT_ROWS - 1) / UNIT_ROWS;
    }
    if (tid == 1023) {
        offsets[NB] = s_p[1023];
        unit_off[NB] = s_u[1023];
    }
}

// ------------------------------------------------------------ block-major partials
struct PartArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint32_t* pairs;
    const uint32_t* offsets;   // [NB+1]
    const uint32_t* unit_off;  // [NB+1]
    uint16_t* part_o;          // bf16 bits [pairs][64]
    float* part_lse;           // [pairs], log2 domain
    int N, nb, top_k, NB;
    float scale_log2;
};

template <int BS>
__global__ __launch_bounds__(256, 2) void k_block_partial(PartArgs a) {
    constexpr int KT = BS / 16;
    constexpr int VP = BS + 8;
    __shared__ __attribute__((aligned(16))) __bf16 s_k[BS * KPITCH];
    __shared__ __attribute__((aligned(16))) __bf16 s_vt[kD * VP];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t U = a.unit_off[a.NB];
    const uint32_t per = (U + gridDim.x - 1) / gridDim.x;
    const uint32_t u0 = blockIdx.x * per;
    const uint32_t u1 = min(U, u0 + per);
    if (u0 >= u1) return;
    // bucket holding unit u0: last b with unit_off[b] <= u0
    int lo = 0, hi = a.NB;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.unit_off[mid] <= u0) lo = mid; else hi = mid;
    }
    int bucket = lo;
    int loaded = -1;
    for (uint32_t u = u0; u < u1; ++u) {
        while (a.unit_off[bucket + 1] <= u) ++bucket;
        const uint32_t p0 = a.offsets[bucket] + (u - a.unit_off[bucket]) * UNIT_ROWS;
        const uint32_t p1 = min(p0 + UNIT_ROWS, a.offsets[bucket + 1]);
        if (bucket != loaded) {
            __syncthreads();
            const int bg = bucket / a.nb, c = bucket - bg * a.nb;
            const int64_t kv0 = ((int64_t)bg * a.N + (int64_t)c * BS) * kD;
            stage_k(s_k, a.k + kv0, BS, BS, tid, 256);
            stage_vt(s_vt, VP, a.v + kv0, BS, BS, tid, 256);
            __syncthreads();
            loaded = bucket;
        }
        const uint32_t pi = p0 + 16 * w + (lane & 15);
        const bool valid = pi < p1;
        const uint32_t pid = valid ? a.pairs[pi] : 0u;
        const int64_t row = pid / (uint32_t)a.top_k;
        if (p0 + 16 * w >= p1) continue;  // whole wave idle (no barrier follows in this unit)
        bf16x8 Bq[2];
        load_q_operand(a.q + row * kD, lane, valid, Bq);
        float x[KT][4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            const f32x4 s = score_tile(s_k, i, lane, Bq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[i][r] = s[r] * a.scale_log2;
                mx = fmaxf(mx, x[i][r]);
            }
        }
        mx = row_max4(mx);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[i][r] = exp2f(x[i][r] - mx);
                sum += x[i][r];
            }
        sum = row_sum4(sum);
        f32x4 o[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        pv_accumulate<KT>(s_vt, VP, lane, x, o);
        if (valid) {
            const float inv = 1.f / sum;
            uint16_t* dst = a.part_o + (int64_t)pid * kD + 4 * (lane >> 4);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                bf16x4 ob;
#pragma unroll
                for (int r = 0; r < 4; ++r) ob[r] = (__bf16)(o[mt][r] * inv);
                *reinterpret_cast<bf16x4*>(dst + 16 * mt) = ob;
            }
            if (lane < 16) a.part_lse[pid] = mx + log2f(sum);
        }
    }
}

// ------------------------------------------------------------ window + merge
struct WinArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* idx;
    const uint16_t* part_o;
    const float* part_lse;
    float* out;
    int Hq, Hkv, N, bs, top_k, window, tiles;
    float scale_log2;
};

__global__ __launch_bounds__(256, 2) void k_window_merge(WinArgs a) {
    constexpr int VP = 64 + 8;
    __shared__ __attribute__((aligned(16))) __bf16 s_k[64 * KPITCH];
    __shared__ __attribute__((aligned(16))) __bf16 s_vt[kD * VP];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bh = blockIdx.x / a.tiles, tile = blockIdx.x - bh * a.tiles;
    const int h = bh % a.Hq, b = bh / a.Hq, g = h / (a.Hq / a.Hkv);
    const int t0 = tile * 64;
    const int t = t0 + 16 * w + (lane & 15);
    const bool valid = t < a.N;
    const int64_t row = (int64_t)bh * a.N + t;
    const int E = valid ? eligible_blocks(t, a.bs, a.window) : 0;
    const int lo_t = a.bs * E;  // first window key of this row
    const int key_lo = a.bs * eligible_blocks(t0, a.bs, a.window);
    const int key_hi = min(t0 + 63, a.N - 1);
    const int64_t kv0 = ((int64_t)b * a.Hkv + g) * a.N * kD;

    bf16x8 Bq[2];
    load_q_operand(a.q + row * kD, lane, valid, Bq);
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int kc = key_lo; kc <= key_hi; kc += 64) {
        const int nvalid = min(64, a.N - kc);
        __syncthreads();
        stage_k(s_k, a.k + kv0 + (int64_t)kc * kD, 64, nvalid, tid, 256);
        stage_vt(s_vt, VP, a.v + kv0 + (int64_t)kc * kD, 64, nvalid, tid, 256);
        __syncthreads();
        float x[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 s = score_tile(s_k, i, lane, Bq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kc + 16 * i + 4 * (lane >> 4) + r;
                const bool ok = valid && j >= lo_t && j <= t;
                x[i][r] = ok ? s[r] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, x[i][r]);
            }
        }
        mx = row_max4(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[i][r] = exp2f(x[i][r] - m_use);
                sum += x[i][r];
            }
        sum = row_sum4(sum);
        l_run = l_run * alpha + sum;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;
        m_run = m_new;
        pv_accumulate<4>(s_vt, VP, lane, x, o);
    }
    if (!valid) return;
    // merge the routed partials (each a normalised output with its log2 mass)
    const int32_t* ir = a.idx + row * a.top_k;
    uint32_t used = used_slots(ir, a.top_k, E);
    while (used) {
        const int s = __builtin_ctz(used);
        used &= used - 1;
        const int64_t pid = row * a.top_k + s;
        const float lse = a.part_lse[pid];
        const float m_new = fmaxf(m_run, lse);
        const float alpha = exp2f(m_run - m_new);
        const float beta = exp2f(lse - m_new);
        const uint16_t* src = a.part_o + pid * kD + 4 * (lane >> 4);
        l_run = l_run * alpha + beta;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const u32x2 raw = *reinterpret_cast<const u32x2*>(src + 16 * mt);
            const float v0 = __uint_as_float(raw[0] << 16), v1 = __uint_as_float(raw[0] & 0xFFFF0000u);
            const float v2 = __uint_as_float(raw[1] << 16), v3 = __uint_as_float(raw[1] & 0xFFFF0000u);
            o[mt][0] = o[mt][0] * alpha + beta * v0;
            o[mt][1] = o[mt][1] * alpha + beta * v1;
            o[mt][2] = o[mt][2] * alpha + beta * v2;
            o[mt][3] = o[mt][3] * alpha + beta * v3;
        }
        m_run = m_new;
    }
    const float inv = 1.f / l_run;
    float* dst = a.out + row * kD + 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt) = o[mt] * inv;
}

// ------------------------------------------------------------ image mode
struct ImgArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* idx;  // [B,Hq,nb,top_k]
    float* out;
    int Hq, Hkv, N, nb, top_k;
    int64_t n_qblocks;   // B*Hq*nb
    float scale_log2;
};

// One wave per 16-token query block (block size 16).  The selected blocks
// are processed four at a time (64 keys) with an online softmax; K feeds the
// MFMA straight from global memory, V is transposed through the wave's own
// LDS region.
__global__ __launch_bounds__(256, 2) void k_image_attend(ImgArgs a) {
    constexpr int VP = 64 + 8;
    __shared__ __attribute__((aligned(16))) __bf16 s_vt[4][kD * VP];
    __shared__ int s_n[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t qb = (int64_t)blockIdx.x * 4 + w;
    const bool active = qb < a.n_qblocks;
    const int64_t bh = active ? qb / a.nb : 0;
    const int i = active ? (int)(qb - bh * a.nb) : 0;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq), g = h / (a.Hq / a.Hkv);
    const int64_t kv0 = ((int64_t)b * a.Hkv + g) * a.N * kD;
    const int t = 16 * i + (lane & 15);
    const int64_t row = bh * a.N + t;

    // the used slots of this query block's idx row (wave-uniform)
    const int32_t* ir = a.idx + (active ? qb : 0) * a.top_k;
    const uint32_t used = active ? used_slots(ir, a.top_k, a.nb) : 0u;
    const int nused = __builtin_popcount(used);
    if (lane == 0) s_n[w] = nused;
    __syncthreads();
    const int nmax = max(max(s_n[0], s_n[1]), max(s_n[2], s_n[3]));

    bf16x8 Bq[2];
    load_q_operand(a.q + row * kD, lane, active, Bq);
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    __bf16* vt = s_vt[w];

    for (int c0 = 0; c0 < nmax; c0 += 4) {
        __syncthreads();
        // stage V^T of up to four blocks (16 keys each) into this wave's region
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const bool have = c0 + jb < nused;
            const int cblk = have ? ir[nth_slot(used, c0 + jb)] : 0;
            const uint16_t* src = a.v + kv0 + (int64_t)cblk * 16 * kD;
            // 16 keys x 64 dims = 64 4x4 tiles: one per lane
            const int kg = lane & 3, dg = lane >> 2;
            uint32_t lo4[4], hi4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u32x2 vv = {0u, 0u};
                if (have) vv = *reinterpret_cast<const u32x2*>(src + (int64_t)(kg * 4 + r) * kD + dg * 4);
                lo4[r] = vv[0];
                hi4[r] = vv[1];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t* wv = (j < 2) ? lo4 : hi4;
                const int sh = (j & 1) * 16;
                u32x2 packed = {((wv[0] >> sh) & 0xFFFFu) | (((wv[1] >> sh) & 0xFFFFu) << 16),
                                ((wv[2] >> sh) & 0xFFFFu) | (((wv[3] >> sh) & 0xFFFFu) << 16)};
                *reinterpret_cast<u32x2*>(vt + (dg * 4 + j) * VP + jb * 16 + kg * 4) = packed;
            }
        }
        __syncthreads();
        float x[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const bool have = c0 + jb < nused;
            const int cblk = have ? ir[nth_slot(used, c0 + jb)] : 0;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (have) {
                const uint16_t* kr = a.k + kv0 + ((int64_t)cblk * 16 + (lane & 15)) * kD + 8 * (lane >> 4);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) acc = mfma16(load_bf16x8(kr + 32 * ks), Bq[ks], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[jb][r] = have ? acc[r] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, x[jb][r]);
            }
        }
        mx = row_max4(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float sum = 0.f;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[jb][r] = exp2f(x[jb][r] - m_use);
                sum += x[jb][r];
            }
        sum = row_sum4(sum);
        l_run = l_run * alpha + sum;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;
        m_run = m_new;
        pv_accumulate<4>(vt, VP, lane, x, o);
    }
    if (!active) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* dst = a.out + row * kD + 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt) = o[mt] * inv;
}

// ------------------------------------------------------------ host side
struct AttendLayout {
    size_t counts, offsets, cursor, unit_off, pairs, part_o, part_lse, total;
};

static AttendLayout attend_layout(const Geometry& g) {
    AttendLayout L{};
    if (!g.causal) return L;
    const size_t NB = (size_t)g.B * g.Hkv * g.nb;
    const size_t npairs = (size_t)g.B * g.Hq * g.N * g.top_k;
    size_t off = 0;
    L.counts = off;   off += align_up(NB * 4, 256);
    L.offsets = off;  off += align_up((NB + 1) * 4, 256);
    L.cursor = off;   off += align_up(NB * 4, 256);
    L.unit_off = off; off += align_up((NB + 1) * 4, 256);
    L.pairs = off;    off += align_up(npairs * 4, 256);
    L.part_o = off;   off += align_up(npairs * kD * 2, 256);
    L.part_lse = off; off += align_up(npairs * 4, 256);
    L.total = off;
    return L;
}

size_t attend_workspace_bytes(const Geometry& g) { return attend_layout(g).total; }

template <int BS>
static void launch_partial(const PartArgs& pa, hipStream_t s) {
    hipLaunchKernelGGL(k_block_partial<BS>, dim3(PART_GRID), dim3(256), 0, s, pa);
}

hipError_t launch_attend(const Geometry& g, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* idx, float* out, void* ws,
                         hipStream_t s, const hipEvent_t* ev) {
    const float scale_log2 = g.scale * kLog2e;
    if (!g.causal) {
        ImgArgs a{q, k, v, idx, out, g.Hq, g.Hkv, g.N, g.nb, g.top_k,
                  (int64_t)g.B * g.Hq * g.nb, scale_log2};
        const unsigned grid = (unsigned)((a.n_qblocks + 3) / 4);
        for (int i = 4; i < 8; ++i) mark(ev, i, s);
        hipLaunchKernelGGL(k_image_attend, dim3(grid), dim3(256), 0, s, a);
        mark(ev, 8, s);
        return hipGetLastError();
    }
    const AttendLayout L = attend_layout(g);
    char* base = static_cast<char*>(ws);
    uint32_t* counts = reinterpret_cast<uint32_t*>(base + L.counts);
    uint32_t* offsets = reinterpret_cast<uint32_t*>(base + L.offsets);
    uint32_t* cursor = reinterpret_cast<uint32_t*>(base + L.cursor);
    uint32_t* unit_off = reinterpret_cast<uint32_t*>(base + L.unit_off);
    uint32_t* pairs = reinterpret_cast<uint32_t*>(base + L.pairs);
    uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
    float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
    const int NB = g.B * g.Hkv * g.nb;

    hipError_t e = launch_fill_u32(counts, (size_t)NB, 0u, s);
    if (e != hipSuccess) return e;
    BucketArgs ba{idx, counts, cursor, pairs, g.Hq, g.Hkv, g.N, g.bs, g.nb, g.top_k, g.window};
    const int nch = (g.N + BK_TCHUNK - 1) / BK_TCHUNK;
    const dim3 bgrid((unsigned)(g.B * g.Hkv * nch));
    const size_t lds = g.nb <= BK_LDS_MAX ? (size_t)g.nb * 4 : 0;
    hipLaunchKernelGGL(k_bucket<false>, bgrid, dim3(256), lds, s, ba);
    mark(ev, 4, s);
    hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(1024), 0, s, counts, offsets, cursor, unit_off,
                       NB);
    mark(ev, 5, s);
    hipLaunchKernelGGL(k_bucket<true>, bgrid, dim3(256), lds, s, ba);
    mark(ev, 6, s);

    PartArgs pa{q, k, v, pairs, offsets, unit_off, part_o, part_lse, g.N, g.nb, g.top_k, NB,
                scale_log2};
    switch (g.bs) {
        case 16: launch_partial<16>(pa, s); break;
        case 32: launch_partial<32>(pa, s); break;
        case 64: launch_partial<64>(pa, s); break;
        default: launch_partial<128>(pa, s); break;
    }
    mark(ev, 7, s);
    WinArgs wa{q, k, v, idx, part_o, part_lse, out, g.Hq, g.Hkv, g.N, g.bs, g.top_k, g.window,
               (g.N + 63) / 64, scale_log2};
    hipLaunchKernelGGL(k_window_merge, dim3((unsigned)(g.B * g.Hq * wa.tiles)), dim3(256), 0, s,
                       wa);
    mark(ev, 8, s);
    return hipGetLastError();
}

}  // namespace lsa
