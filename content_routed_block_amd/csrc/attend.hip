// Exact softmax attention over the selected keys only (SSA page, opening
// paragraph; Subquadratic Sparse Attention page, "Architecture": selected
// attention alongside a causal sliding window).
//
// Causal mode runs key-block-major, because every query routes to its own
// blocks and a query-major gather would reuse nothing:
//   0. k_transpose_v    V -> V^T in 64-key tiles, so every kernel stages V^T
//                       with plain 16-byte copies.
//   1. k_bucket<false>  counts, per (bucket chunk of query positions, b, KV
//                       head, key block), the (row, slot) pairs that selected
//                       it (LDS histogram per workgroup).
//   2. k_bucket_scan    bucket offsets and the work units (64 rows each).
//   3. k_bucket<true>   scatters pair ids into bucket order and records, per
//                       (row, slot), the pair's position in that order.
//   4. k_block_partial  one K/V block in LDS against up to 64 gathered query
//                       rows: S = Q K^T and O = P V on bf16 MFMA; writes the
//                       normalised partial output (bf16, by row and slot)
//                       and its log2 mass (by position, so those writes are
//                       contiguous).
//   5. k_window_merge   flash-style online softmax over the block-aligned
//                       window [bs*E(t), t] with a causal mask, then merges
//                       the row's routed partials with the append law of the
//                       SSA page ("Mathematical status": adding mass a to mass
//                       Z moves the read by a/(Z+a) times the displacement of
//                       the new value), and writes fp32 output.
// Image mode (k_image_attend): one wave per 16-token query block; its
// selected 16-key blocks are gathered straight into MFMA operands (K) or
// through LDS with transposing reads (V).
//
// MFMA orientation: S^T = K . Q^T on 16x16x32 tiles, so lane l holds query
// row l%16 and keys 16i + 4(l/16) + r.  Those probabilities are exactly the
// B operand of O^T = V^T . P^T when key slot j of lane l stands for key
// 32s + 4(l/16) + j (j < 4) or 32s + 16 + 4(l/16) + (j-4): no cross-lane
// movement.  Softmax runs in the log2 domain: exp2(s * scale*log2(e) - m)
// is one FMA and one exp per logit.
//
// Pair ids: pair (row, slot) is row * SP + slot with SP the power of two
// >= top_k, so the row is a shift away.
#include <math.h>

#include <algorithm>

#include "bucket.hpp"
#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

constexpr int KPITCH = 72;         // LDS pitch of K tiles [key][64 d] (bf16), 16-byte rows
constexpr int VT_TILE = 64;        // keys per V^T tile
constexpr int WVP = VT_TILE + 4;   // LDS pitch of 64-key V^T tiles: 2 mod 4 words
constexpr float RESCALE_SLACK = 8.f;  // log2 headroom before a running max is raised


// ------------------------------------------------------------ V transpose
// V [BG][N][64] -> V^T tiles [BG][ceil(N/TW)][64 d][TW keys]; keys >= N are
// zero.  The causal kernels take TW = 64 (image mode reads V rows itself and
// transposes them on their way out of LDS).  The same launch clears the
// bucket counts (nzero words at zero) for the bucketing that follows.
template <int TW>
__global__ __launch_bounds__(256) void k_transpose_v(const uint16_t* __restrict__ v,
                                                     uint16_t* __restrict__ vt, int N, int ntiles,
                                                     uint32_t* __restrict__ zero, size_t nzero) {
    __shared__ uint32_t s[VT_TILE][33];  // [key][d pair], odd pitch
    const int tid = threadIdx.x;
    for (size_t i = (size_t)blockIdx.x * 256 + tid; i < nzero; i += (size_t)gridDim.x * 256)
        zero[i] = 0u;
    const int bg = blockIdx.x / ntiles, tile = blockIdx.x - bg * ntiles;
    const int key0 = tile * VT_TILE;
    const int nvalid = min(VT_TILE, N - key0);
    const uint16_t* src = v + ((int64_t)bg * N + key0) * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ch = tid + 256 * i, key = ch >> 3, d0 = (ch & 7) * 8;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < nvalid) x = *reinterpret_cast<const u32x4*>(src + (int64_t)key * kD + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) s[key][d0 / 2 + j] = x[j];
    }
    __syncthreads();
    uint16_t* dst = vt + ((int64_t)bg * ntiles + tile) * (kD * VT_TILE);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ch = tid + 256 * i, d = ch >> 3, k0 = (ch & 7) * 8;
        uint16_t* out = dst + (k0 / TW) * (kD * TW) + d * TW + (k0 % TW);
        const int sh = 16 * (d & 1);
        u32x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = (s[k0 + 2 * j][d >> 1] >> sh) & 0xFFFFu;
            const uint32_t hi = (s[k0 + 2 * j + 1][d >> 1] >> sh) & 0xFFFFu;
            y[j] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(out) = y;
    }
}

// ------------------------------------------------------------ shared pieces
// 16 bytes into an LDS row that is only 8-byte aligned (V^T pitches).
__device__ __forceinline__ void lds_store_2x8(__bf16* dst, u32x4 v) {
    reinterpret_cast<u32x2*>(dst)[0] = u32x2{v[0], v[1]};
    reinterpret_cast<u32x2*>(dst)[1] = u32x2{v[2], v[3]};
}

// Copies 64 rows of 64 bf16 (128 B each) from a source with the given row
// stride into LDS rows of the given pitch; rows >= valid are zero.  K tiles
// (16-byte rows) use 16-byte LDS stores, V^T tiles 8-byte ones.
template <bool ROW16>
__device__ __forceinline__ void stage_rows(__bf16* dst, int pitch, const uint16_t* src,
                                           int64_t stride, int rows, int valid, int tid) {
    for (int ch = tid; ch < rows * 8; ch += 256) {
        const int r = ch >> 3, c0 = (ch & 7) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < valid) v = *reinterpret_cast<const u32x4*>(src + (int64_t)r * stride + c0);
        if (ROW16)
            *reinterpret_cast<u32x4*>(dst + r * pitch + c0) = v;
        else
            lds_store_2x8(dst + r * pitch + c0, v);
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

// Raw scores S^T for keys [16i, 16i+16) of an LDS K tile.
__device__ __forceinline__ f32x4 score_tile(const __bf16* s_k, int i, int lane,
                                            const bf16x8 (&Bq)[2]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(s_k + (16 * i + (lane & 15)) * KPITCH +
                                                          8 * (lane >> 4) + 32 * ks);
        acc = mfma16(A, Bq[ks], acc);
    }
    return acc;
}

// O^T += V^T P^T over KT 16-key tiles whose probabilities are p[i][r] (key
// 16i + 4(l/16) + r); V^T in LDS with pitch vpitch, keys from column koff.
template <int KT>
__device__ __forceinline__ void pv_accumulate(const __bf16* s_vt, int vpitch, int koff, int lane,
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
            const __bf16* vr =
                s_vt + (16 * mt + (lane & 15)) * vpitch + koff + 32 * s + 4 * (lane >> 4);
            const u32x2 a0 = *reinterpret_cast<const u32x2*>(vr);
            u32x2 a1 = {0u, 0u};
            if (2 * s + 1 < KT) a1 = *reinterpret_cast<const u32x2*>(vr + 16);
            const u32x4 araw = {a0[0], a0[1], a1[0], a1[1]};
            o[mt] = mfma16(__builtin_bit_cast(bf16x8, araw), Bp, o[mt]);
        }
    }
}

// 2^x with the bare hardware instruction (v_exp_f32).  Results below the
// smallest normal float come out as zero; a softmax weight that small is lost
// without effect on any sum it enters.  The libm exp2f wraps the same
// instruction in a denormal-range rescale (a compare, a select, an add and an
// ldexp per call).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Row reductions across the 4 lanes that share row l%16.
__device__ __forceinline__ float row_max4(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, kWave));
    return fmaxf(v, __shfl_xor(v, 32, kWave));
}
__device__ __forceinline__ float row_sum4(float v) {
    v += __shfl_xor(v, 16, kWave);
    return v + __shfl_xor(v, 32, kWave);
}

// Slot of the n-th set bit of a mask (n < popcount(mask)).
__device__ __forceinline__ int nth_slot(uint32_t mask, int n) {
    for (int i = 0; i < n; ++i) mask &= mask - 1;
    return __builtin_ctz(mask);
}

// c[i] for a runtime i < KM without dynamic register indexing.
template <int KM>
__device__ __forceinline__ int pick(const int (&c)[KM], int i) {
    int v = 0;
#pragma unroll
    for (int s = 0; s < KM; ++s) v = (s == i) ? c[s] : v;
    return v;
}

// ------------------------------------------------------------ block-major partials
struct PartArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* vt;        // V^T tiles [BG][ntiles][64 d][64 keys]
    const uint32_t* pairs;     // chunk-local pair ids, in bucket order
    const uint32_t* offsets;   // [NB+1]
    const uint32_t* unit_off;  // [NB+1]
    uint16_t* part_o;          // bf16 bits [crows * SP + 64][64] by chunk-local pair id,
                               // permuted (see k_block_partial)
    float* part_lse;           // [crows * top_k + 64] by pair position in the chunk, log2 domain
    uint32_t dummy_pid;        // crows * SP: first of 64 rows written by lanes without a pair
    uint32_t dummy_pos;        // crows * top_k: first of 64 log-mass slots for the same lanes
    int N, nb, NB, ntiles, sp_log2;
    int b0, b1;                // this launch's buckets [b0, b1): one position chunk
    int nbc;                   // buckets per bucket chunk (b1 - b0 is a multiple)
    int pc_log2, t_base;       // positions per chunk (log2); the chunk's first position
    float scale_log2;
    // 1, or the query heads per KV group when pairs are group pairs (one
    // route per group): gathered row e of the chunk is then head e % expand
    // of the group pair at position e / expand
    int expand;
};

// Per wave, pair ids run two units ahead and Q rows one unit ahead of the
// compute, hiding the dependent gather latency.  Partial rows are stored
// permuted: slot 16j + 4mt + r holds dim 16mt + 4j + r, so lane group j
// writes (and the merge reads) 32 contiguous bytes.
template <int BS>
__global__ __launch_bounds__(256, 2) void k_block_partial(PartArgs a) {
    constexpr int KT = BS / 16;
    constexpr int VC = BS > VT_TILE ? BS : VT_TILE;  // staged V^T columns
    constexpr int VP = VC + 4;                       // 2 mod 4 words: conflict-free 8-byte reads
    __shared__ __attribute__((aligned(16))) __bf16 s_k[BS * KPITCH];
    __shared__ __attribute__((aligned(16))) __bf16 s_vt[kD * VP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the position of this chunk's first pair
    const uint32_t pos_base = uniform_load(a.offsets + a.b0);
    uint32_t u1 = 0;  // end of this workgroup's units in the current bucket chunk
    UnitCursor cur, ahead;
    const uint32_t my = 16 * w + (lane & 15);  // this lane's row slot in a unit
    // Every vector memory operation below is issued unconditionally (lanes
    // without a row read the chunk's first pair, whose row lies in this
    // chunk, and write a dummy row), so the wait for a prefetched operand
    // never has to drain the stores issued after it.
    const uint32_t dummy = a.dummy_pid + my;
    const uint32_t dummy_pos = a.dummy_pos + my;
    const uint32_t pmask = (1u << a.pc_log2) - 1u;
    const uint32_t smask = (1u << a.sp_log2) - 1u;
    // the query pair id of this lane's gathered row of unit u
    auto fetch_pid = [&](uint32_t u, uint32_t& pid, bool& v) {
        uint32_t q0 = 0, q1 = 0;
        if (u < u1) ahead.rows(a.unit_off, a.offsets, u, q0, q1, (uint32_t)a.expand);
        const uint32_t e = q0 + my;
        v = e < q1;
        if (a.expand == 1) {
            pid = a.pairs[v ? e : pos_base];
        } else {
            // group pair (KV group bg, position, slot) -> the same position
            // and slot of query head bg * expand + h
            const uint32_t pos = e / (uint32_t)a.expand, h = e - pos * (uint32_t)a.expand;
            const uint32_t gp = a.pairs[v ? pos : pos_base];
            const uint32_t grow = gp >> a.sp_log2;
            const uint32_t qrow = (((grow >> a.pc_log2) * (uint32_t)a.expand + h) << a.pc_log2) |
                                  (grow & pmask);
            pid = (qrow << a.sp_log2) | (gp & smask);
        }
    };
    auto fetch_q = [&](uint32_t pid, bf16x8 (&B)[2]) {
        // chunk-local row -> (query head bh, position t) -> global row
        const uint32_t lrow = pid >> a.sp_log2;
        const int64_t grow = (int64_t)(lrow >> a.pc_log2) * a.N + a.t_base + (lrow & pmask);
        const uint16_t* qrow = a.q + grow * kD + 8 * (lane >> 4);
        B[0] = load_bf16x8(qrow);
        B[1] = load_bf16x8(qrow + 32);
    };

    int loaded = -1, koff = 0;
    // Bucket chunks (nbc buckets each: every key block of every (b, KV head)
    // for one span of query positions) run one after the other, each split
    // evenly over the workgroups: all of them gather the query rows of the
    // same positions at a time, so those rows stay cached between the
    // blocks that selected them.
    for (int sb0 = a.b0; sb0 < a.b1; sb0 += a.nbc) {
    const uint32_t ulo = uniform_load(a.unit_off + sb0);
    const uint32_t uhi = uniform_load(a.unit_off + sb0 + a.nbc);
    const uint32_t per = (uhi - ulo + gridDim.x - 1) / gridDim.x;
    const uint32_t u0 = ulo + blockIdx.x * per;
    u1 = min(uhi, u0 + per);
    if (u0 >= u1) continue;
    cur.seek(a.unit_off, a.NB, u0);
    ahead = cur;
    // prologue: pair ids of units u0 and u0+1, Q rows of unit u0
    bool v_cur, v_nxt;
    uint32_t pid_cur, pid_nxt;
    fetch_pid(u0, pid_cur, v_cur);
    fetch_pid(u0 + 1, pid_nxt, v_nxt);
    bf16x8 Bq[2];
    fetch_q(pid_cur, Bq);
    // drain the prologue loads, so that the loop's first wait (for the
    // carried pair id) does not fall back to draining everything each trip
    __builtin_amdgcn_s_waitcnt(0);

    for (uint32_t u = u0; u < u1; ++u) {
        uint32_t p0, p1;
        cur.rows(a.unit_off, a.offsets, u, p0, p1, (uint32_t)a.expand);
        // prefetch: pair ids of u+2, Q rows of u+1
        bool v_n2;
        uint32_t pid_n2;
        fetch_pid(u + 2, pid_n2, v_n2);
        bf16x8 Bq_nxt[2];
        fetch_q(pid_nxt, Bq_nxt);

        if (cur.bucket != loaded) {
            __syncthreads();
            // buckets of this chunk: [b0, b1) = (bucket chunk, b * Hkv + g,
            // key block), nbc = B * Hkv * nb buckets per bucket chunk
            const int rel = (cur.bucket - a.b0) % a.nbc;
            const int bg = rel / a.nb, c = rel - bg * a.nb;
            const int key0 = c * BS;
            stage_rows<true>(s_k, KPITCH, a.k + ((int64_t)bg * a.N + key0) * kD, kD, BS, BS, tid);
            // V^T columns [VC * (key0 / VC), +VC) from the 64-key tiles
            const int tile0 = (key0 / VC) * (VC / VT_TILE);
#pragma unroll
            for (int tt = 0; tt < VC / VT_TILE; ++tt)
                stage_rows<false>(s_vt + tt * VT_TILE, VP,
                                  a.vt + ((int64_t)bg * a.ntiles + tile0 + tt) * (kD * VT_TILE),
                                  VT_TILE, kD, kD, tid);
            koff = key0 % VC;
            __syncthreads();
            loaded = cur.bucket;
        }
        f32x4 sc[KT];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            sc[i] = score_tile(s_k, i, lane, Bq);
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[i][r]);
        }
        const float m2 = row_max4(mx) * a.scale_log2;
        float p[KT][4];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[i][r] = exp2_hw(fmaf(sc[i][r], a.scale_log2, -m2));
                sum += p[i][r];
            }
        sum = row_sum4(sum);
        f32x4 o[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        pv_accumulate<KT>(s_vt, VP, koff, lane, p, o);
        const float inv = 1.f / sum;
        const uint32_t pid_st = v_cur ? pid_cur : dummy;
        uint16_t* dst = a.part_o + (int64_t)pid_st * kD + 16 * (lane >> 4);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            bf16x8 ob;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ob[r] = (__bf16)(o[2 * h2][r] * inv);
                ob[4 + r] = (__bf16)(o[2 * h2 + 1][r] * inv);
            }
            *reinterpret_cast<bf16x8*>(dst + 8 * h2) = ob;
        }
        // by position: the wave's 16 rows are consecutive, so this store is
        // contiguous (the row's four lanes store the same value)
        a.part_lse[v_cur ? p0 + my - pos_base * (uint32_t)a.expand : dummy_pos] = m2 + log2f(sum);
        v_cur = v_nxt;
        pid_cur = pid_nxt;
        v_nxt = v_n2;
        pid_nxt = pid_n2;
        Bq[0] = Bq_nxt[0];
        Bq[1] = Bq_nxt[1];
    }
    }
}

// ------------------------------------------------------------ window + merge
struct WinArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* vt;
    const int32_t* idx;  // [B,Hq,N,top_k]; group_route: [B,Hkv,N,top_k]
    const uint16_t* part_o;   // the chunk's partial rows, by chunk-local pair id
    const float* part_lse;    // the chunk's log2 masses, by pair position in the chunk
    const uint32_t* rev;      // [top_k][rows]: global pair positions
    const uint32_t* offsets;  // [NB+1] bucket offsets (the chunk's first pair: offsets[b0])
    float* out;
    int64_t rows;             // rows of rev: query rows, or group rows with group pairs
    int Hq, Hkv, N, bs, top_k, window, tiles, items, ntiles, sp_log2;
    int b0, pc_log2, t_base;  // the chunk: first bucket, positions (log2), first position
    float scale_log2;
    int group_route;
    int expand;               // as in PartArgs: > 1 with group pairs
};

// One workgroup per (query head, 64 positions); wave w owns rows
// t0 + 16w .. +15 (lane l holds row l%16).  The window keys stream through
// double-buffered 64-key LDS tiles (64-aligned, so a V^T tile is one plain
// copy); the next tile is fetched into registers while the current one is
// used.  A row's running max is raised only when a chunk exceeds it by
// RESCALE_SLACK (log2 units), so most chunks skip rescaling the
// accumulator; masks are applied only on chunks that cross a row's window
// start or its causal end.  KM: the row's slot list length (kMaxTopK, or
// kMaxTopKWide for top_k above it, at lower occupancy).
template <int KM>
__global__ __launch_bounds__(256, KM > kMaxTopK ? 2 : 4) void k_window_merge(WinArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_k[2][64 * KPITCH];
    __shared__ __attribute__((aligned(16))) __bf16 s_vt[2][kD * WVP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
    // item = xcd * (grid / 8) + (blockIdx / 8) keeps consecutive items on one
    // XCD; items run head-fastest, so the query heads of a KV group that read
    // the same window tile share that XCD's L2.
    const int per_xcd = gridDim.x / 8;
    const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int rep = a.Hq / a.Hkv;
    if (item >= a.items) return;
    const int hh = item % rep;
    const int tile = (item / rep) % a.tiles;  // tiles of this chunk
    const int bg = item / (rep * a.tiles);
    const int b = bg / a.Hkv;
    const int h = (bg - b * a.Hkv) * rep + hh;
    const int bh = b * a.Hq + h;
    const int t0 = a.t_base + tile * 64;
    const int key_lo = a.bs * eligible_blocks(t0, a.bs, a.window);
    const int key_hi = min(t0 + 63, a.N - 1);
    const int lo_max = a.bs * eligible_blocks(key_hi, a.bs, a.window);  // largest row start
    const int kc0 = key_lo / VT_TILE * VT_TILE;
    const int64_t k0 = (int64_t)bg * a.N * kD;
    const int64_t vt0 = (int64_t)bg * a.ntiles * (kD * VT_TILE);
    const int t = t0 + 16 * w + (lane & 15);
    const bool valid = t < a.N;
    const int E = valid ? eligible_blocks(t, a.bs, a.window) : 0;
    const int lo_t = valid ? a.bs * E : a.N;
    const int64_t row = (int64_t)bh * a.N + t;
    // this head's gathered row of a pair: head hh with group pairs
    const uint32_t head_off = a.expand > 1 ? (uint32_t)hh : 0u;

    bf16x8 Bq[2];
    load_q_operand(a.q + row * kD, lane, valid, Bq);
    // the row's routed slots, read now so the loads overlap the window work
    int csel[KM];
    const int64_t irow = a.group_route ? (int64_t)bg * a.N + t : row;
    const uint32_t used = valid ? row_used<KM>(a.idx + irow * a.top_k, a.top_k, E, csel) : 0u;
    // the pair positions of the row's routed slots from the slot-major table
    // (rows are group rows with group pairs; the wave's 16 rows are
    // consecutive, so each load is contiguous), requested before the window
    // so that the merge's log-mass gathers can start as soon as it is done
    const int64_t rev_row = a.expand > 1 ? (int64_t)bg * a.N + t : row;
    uint32_t rs[KM];
#pragma unroll
    for (int sl = 0; sl < KM; ++sl)
        rs[sl] = (sl < a.top_k && ((used >> sl) & 1u)) ? a.rev[sl * a.rows + rev_row] : 0u;
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // staging: a K tile and a V^T tile, 512 chunks of 16 B each
    u32x4 kp[2], vp[2];
    auto fetch = [&](int kc) {
        const int nvalid = min(64, a.N - kc);
        const uint16_t* ks = a.k + k0 + (int64_t)kc * kD;
        const uint16_t* vs = a.vt + vt0 + (int64_t)(kc / VT_TILE) * (kD * VT_TILE);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = tid + 256 * i, r = ch >> 3, c0 = (ch & 7) * 8;
            kp[i] = r < nvalid ? *reinterpret_cast<const u32x4*>(ks + (int64_t)r * kD + c0)
                               : u32x4{0u, 0u, 0u, 0u};
            vp[i] = *reinterpret_cast<const u32x4*>(vs + r * VT_TILE + c0);
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = tid + 256 * i, r = ch >> 3, c0 = (ch & 7) * 8;
            *reinterpret_cast<u32x4*>(s_k[buf] + r * KPITCH + c0) = kp[i];
            lds_store_2x8(s_vt[buf] + r * WVP + c0, vp[i]);
        }
    };

    fetch(kc0);
    commit(0);
    __syncthreads();
    for (int kc = kc0, it = 0; kc <= key_hi; kc += 64, ++it) {
        const int buf = it & 1;
        const bool more = kc + 64 <= key_hi;
        if (more) fetch(kc + 64);
        const bool edge = kc < lo_max || kc + 63 > t0;
        f32x4 sc[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = score_tile(s_k[buf], i, lane, Bq);
            if (edge) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jk = kc + 16 * i + 4 * (lane >> 4) + r;
                    sc[i][r] = (jk >= lo_t && jk <= t) ? sc[i][r] : -INFINITY;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[i][r]);
        }
        const float mc = row_max4(mx) * a.scale_log2;
        const bool raise = mc > m_run + RESCALE_SLACK;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mc : m_run;
            const float alpha = (m_run == -INFINITY) ? 0.f : exp2_hw(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;
            m_run = m_new;
        }
        const float mu = (m_run == -INFINITY) ? 0.f : m_run;
        float p[4][4];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[i][r] = exp2_hw(fmaf(sc[i][r], a.scale_log2, -mu));
                sum += p[i][r];
            }
        l_run += row_sum4(sum);
        pv_accumulate<4>(s_vt[buf], WVP, 0, lane, p, o);
        if (more) commit(buf ^ 1);
        __syncthreads();
    }
    if (!valid) return;

    // merge the routed partials (normalised outputs with their log2 mass),
    // eight slots at a time so their loads are in flight together; a
    // partial row stores dim 16mt + 4j + r at slot 16j + 4mt + r
    const int64_t prow = (((int64_t)bh << a.pc_log2) + (t - a.t_base)) << a.sp_log2;
    const uint32_t pos_base = uniform_load(a.offsets + a.b0);
    // log2 masses: one 4-byte gather per used slot at its pair position
    // (group pairs: head hh's gathered row of the pair)
    float lse_all[KM];
    {
#pragma unroll
        for (int sl = 0; sl < KM; ++sl)
            lse_all[sl] = (sl < a.top_k && ((used >> sl) & 1u))
                              ? a.part_lse[(rs[sl] - pos_base) * (uint32_t)a.expand + head_off]
                              : -INFINITY;
    }
#pragma unroll
    for (int s0 = 0; s0 < KM; s0 += 8) {
        if (s0 >= a.top_k) break;
        u32x4 po[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int sl = s0 + i;
            const bool u = sl < a.top_k && ((used >> sl) & 1u);
            const uint16_t* src = a.part_o + (prow + sl) * kD + 16 * (lane >> 4);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                po[i][h2] = u ? *reinterpret_cast<const u32x4*>(src + 8 * h2) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int sl = s0 + i;
            if (!(sl < a.top_k && ((used >> sl) & 1u))) continue;
            const float lse = lse_all[sl];
            const float m_new = fmaxf(m_run, lse);
            const float alpha = exp2_hw(m_run - m_new);
            const float beta = exp2_hw(lse - m_new);
            l_run = l_run * alpha + beta;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint32_t w0 = po[i][mt >> 1][2 * (mt & 1)], w1 = po[i][mt >> 1][2 * (mt & 1) + 1];
                o[mt][0] = o[mt][0] * alpha + beta * __uint_as_float(w0 << 16);
                o[mt][1] = o[mt][1] * alpha + beta * __uint_as_float(w0 & 0xFFFF0000u);
                o[mt][2] = o[mt][2] * alpha + beta * __uint_as_float(w1 << 16);
                o[mt][3] = o[mt][3] * alpha + beta * __uint_as_float(w1 & 0xFFFF0000u);
            }
            m_run = m_new;
        }
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
    const uint16_t* v;   // [B,Hkv,N,64]: a 16-key block is 2 KB of contiguous rows
    const int32_t* idx;  // [B,Hq,nb,top_k]; group_route: [B,Hkv,nb,top_k]
    float* out;
    int Hq, Hkv, N, nb, top_k;
    int64_t n_qblocks;   // B*Hq*nb
    float scale_log2;
    int group_route;
};

// O^T += V^T P^T over four 16-key tiles (KT = 4) whose probabilities are
// p[i][r] (key 16i + 4(l/16) + r), with V in LDS as [key][dim] rows of pitch
// vpitch.  The A operand (V^T: a dim per lane, 8 keys) comes from
// ds_read_b64_tr_b16, which hands lane 4a + b of each 16-lane group element b
// of the 8-byte chunks addressed by lanes a, a + 4, a + 8 and a + 12 of the
// group: so lane s of the group addresses key row (base + s / 4) at dims
// 16 mt + 4 (s % 4), and lane m receives dim 16 mt + m of the four keys
// base .. base + 3.
__device__ __forceinline__ void pv_accumulate_rows(const __bf16* s_v, int vpitch, int lane,
                                                   const float (&p)[4][4], f32x4 (&o)[4]) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        bf16x8 Bp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Bp[j] = (__bf16)p[2 * ks][j];
            Bp[4 + j] = (__bf16)p[2 * ks + 1][j];
        }
        // key rows of this lane's address: 32 ks + 4 g + s / 4, and 16 more
        const __bf16* r0 = s_v + (32 * ks + 4 * g + (s >> 2)) * vpitch + 4 * (s & 3);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(r0 + 16 * mt));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(r0 + 16 * vpitch + 16 * mt));
            const s16x8 a8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[mt] = mfma16(__builtin_bit_cast(bf16x8, a8), Bp, o[mt]);
        }
    }
}

// One wave per 16-token query block (block size 16).  The selected blocks
// are processed four at a time (64 keys) with an online softmax; K feeds the
// MFMA straight from global memory, the blocks' V rows are copied into
// the wave's own LDS region.  KM: the slot list length, as in k_window_merge.
constexpr int IVP = kD + 8;  // LDS pitch of the image kernel's V rows (bf16): 16-byte rows
template <int KM>
__global__ __launch_bounds__(256, 2) void k_image_attend(ImgArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_v[4][64 * IVP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
    // item = xcd * (grid / 8) + blockIdx / 8 gives each XCD a contiguous run
    // of query blocks, i.e. whole heads, whose K and V its L2 then holds.
    const int per_xcd = gridDim.x / 8;
    const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int64_t qb = (int64_t)item * 4 + w;
    if (qb >= a.n_qblocks) return;  // the waves share no LDS and no barrier
    const int64_t bh = qb / a.nb;
    const int i = (int)(qb - bh * a.nb);
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq), g = h / (a.Hq / a.Hkv);
    const int64_t bg = (int64_t)b * a.Hkv + g;
    const int64_t k0 = bg * a.N * kD;
    const int t = 16 * i + (lane & 15);
    const int64_t row = bh * a.N + t;

    // the used slots of this query block's idx row (wave-uniform)
    const int64_t irow = a.group_route ? bg * a.nb + i : qb;
    int csel[KM];
    const uint32_t used = row_used<KM>(a.idx + irow * a.top_k, a.top_k, a.nb, csel);
    const int nused = __builtin_popcount(used);

    bf16x8 Bq[2];
    load_q_operand(a.q + row * kD, lane, true, Bq);
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    __bf16* sv = s_v[w];

    for (int c0 = 0; c0 < nused; c0 += 4) {
        // up to four 16-key blocks: their K rows (MFMA operands) and V rows
        // (lane l takes dims 16 (l % 4) .. +15 of key l / 4 of each block's
        // contiguous 2 KB, two 16-byte pieces) are all requested before any
        // is used, so the two gathers overlap
        int cblk[4];
        bf16x8 kop[4][2];
        u32x4 vpart[4][2];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const bool have = c0 + jb < nused;
            cblk[jb] = have ? pick<KM>(csel, nth_slot(used, c0 + jb)) : 0;
            const uint16_t* kr =
                a.k + k0 + ((int64_t)cblk[jb] * 16 + (lane & 15)) * kD + 8 * (lane >> 4);
            const uint16_t* src = a.v + k0 + ((int64_t)cblk[jb] * 16 + (lane >> 2)) * kD + 16 * (lane & 3);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) kop[jb][ks] = load_bf16x8(kr + 32 * ks);
#pragma unroll
            for (int part = 0; part < 2; ++part)
                vpart[jb][part] = *reinterpret_cast<const u32x4*>(src + 8 * part);
        }
        // the previous group's P.V reads of this wave's region are done
        // (LDS operations of one wave complete in order)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const bool have = c0 + jb < nused;
#pragma unroll
            for (int part = 0; part < 2; ++part)
                *reinterpret_cast<u32x4*>(sv + (jb * 16 + (lane >> 2)) * IVP + 16 * (lane & 3) + 8 * part) =
                    have ? vpart[jb][part] : u32x4{0u, 0u, 0u, 0u};
        }
        f32x4 sc[4];
        float mx = -INFINITY;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const bool have = c0 + jb < nused;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mfma16(kop[jb][ks], Bq[ks], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[jb][r] = have ? acc[r] : -INFINITY;
                mx = fmaxf(mx, sc[jb][r]);
            }
        }
        const float mc = row_max4(mx) * a.scale_log2;
        const float m_new = fmaxf(m_run, mc);
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2_hw(m_run - mu);
        float p[4][4];
        float sum = 0.f;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[jb][r] = exp2_hw(fmaf(sc[jb][r], a.scale_log2, -mu));
                sum += p[jb][r];
            }
        l_run = l_run * alpha + row_sum4(sum);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;
        m_run = m_new;
        __builtin_amdgcn_wave_barrier();  // the V stores above precede these reads
        pv_accumulate_rows(sv, IVP, lane, p, o);
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* dst = a.out + row * kD + 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt) = o[mt] * inv;
}

// ------------------------------------------------------------ host side
int pair_stride_log2(int top_k) {
    int l = 0;
    while ((1 << l) < top_k) ++l;
    return l;
}

// Causal attention runs over position chunks of 2^pc_log2 positions (all
// query heads of every batch).  A chunk's partial rows are written by the
// partial kernel and read back by the merge before the next chunk starts, so
// the partial storage is one chunk's worth.  Chunks cost time: each chunk
// splits every key block's bucket, so its staged K/V block serves fewer
// 64-row units, and adds two launches.  (Chunks small enough for their
// partials to stay in the 256 MB memory-side cache were measured slower,
// not faster.)  So a layer is one chunk unless its partials would exceed
// kChunkPartialBytes, and a chunk always gives each key block a few units.
constexpr int64_t kChunkPartialBytes = int64_t(32) << 30;  // partial rows per chunk
constexpr int64_t kMinPairsPerBucket = 192;                 // three 64-row units
// Within a chunk, buckets are ordered by bucket chunks of positions: the
// partial kernel's workgroups finish one bucket chunk's units before the
// next, so the query rows they gather are those of one span of positions
// at a time and stay cached between the blocks that selected them.  A
// bucket chunk is the shortest span whose buckets still hold about
// kBucketChunkPairs pairs each (its K/V blocks are staged once per ~14
// units), used only if its query rows fit in kBucketChunkQBytes.  At the
// 131072-token Qwen-0.5B shape that is 16384 positions (29 MB of query
// rows): partials 2.04 -> 1.91 ms; 8192 and 32768 positions measured 1.93
// and 1.94 ms.
constexpr int64_t kBucketChunkPairs = 896;
constexpr int64_t kBucketChunkQBytes = int64_t(64) << 20;

struct ChunkPlan {
    int pc_log2;   // positions per chunk (log2), >= 6
    int nchunk;    // ceil(N / 2^pc_log2)
    int bc_log2;   // positions per bucket chunk (log2), tc_log2 <= bc_log2 <= pc_log2
    int nbchunk;   // bucket chunks: ceil(N / 2^bc_log2)
    int tc_log2;   // positions per bucketing workgroup (log2), <= bc_log2
};

static ChunkPlan chunk_plan(const Geometry& g) {
    ChunkPlan c{};
    const int rep = g.Hq / g.Hkv;
    const int sp_log2 = pair_stride_log2(g.top_k);
    const int64_t row_bytes = (int64_t)g.B * g.Hq * ((int64_t)kD * 2) << sp_log2;  // per position
    int lmall = 6;
    while ((row_bytes << (lmall + 1)) <= kChunkPartialBytes) ++lmall;
    int locc = 6;
    while (((int64_t)rep * g.top_k << locc) < kMinPairsPerBucket * g.nb) ++locc;
    int ln = 6;
    while ((1 << ln) < g.N) ++ln;
    c.pc_log2 = std::min(std::max(lmall, locc), ln);
    if (g.chunk > 0) {  // the caller's choice (a power of two >= 64)
        int lc = 6;
        while ((1 << lc) < g.chunk) ++lc;
        c.pc_log2 = std::min(lc, ln);
    }
    c.nchunk = (int)(((int64_t)g.N + (1 << c.pc_log2) - 1) >> c.pc_log2);
    // bucketing workgroups: ~4096 rows over the group's query heads (one
    // group row per position with group routes), fewer when that would
    // leave under ~256 workgroups, but enough pairs to amortise the
    // per-bucket flush of the LDS histogram; a power of two within one chunk
    const int nbg = g.B * g.Hkv;
    const int hw = g.consensus ? 1 : rep;  // rows walked per position
    const int64_t flush_min =
        (4 * (int64_t)g.nb + (int64_t)hw * g.top_k - 1) / ((int64_t)hw * g.top_k);
    int64_t tc = std::min<int64_t>((4096 + hw - 1) / hw, (int64_t)nbg * g.N / 256);
    tc = std::max<int64_t>(tc, flush_min);
    int lt = 6;
    while (lt < c.pc_log2 && ((int64_t)1 << (lt + 1)) <= tc) ++lt;
    int lb = 6;
    while (lb < c.pc_log2 && ((int64_t)rep * g.top_k << lb) < kBucketChunkPairs * g.nb) ++lb;
    const int64_t q_bytes = (int64_t)g.B * g.Hq * (kD * 2) << lb;
    c.bc_log2 = q_bytes <= kBucketChunkQBytes ? lb : c.pc_log2;
    c.nbchunk = (int)(((int64_t)g.N + (1 << c.bc_log2) - 1) >> c.bc_log2);
    c.tc_log2 = std::min(lt, c.bc_log2);
    return c;
}

struct AttendLayout {
    size_t vt, counts, offsets, cursor, unit_off, pairs, rev, part_o, part_lse, total;
    ChunkPlan plan;
    int64_t NB;     // buckets: chunks x (b, KV head) x key blocks
    int64_t crows;  // rows of one chunk: B * Hq * 2^pc_log2
};

static AttendLayout attend_layout(const Geometry& g) {
    AttendLayout L{};
    const size_t nbg = (size_t)g.B * g.Hkv;
    const size_t ntiles = ((size_t)g.N + VT_TILE - 1) / VT_TILE;
    size_t off = 0;
    if (g.causal) {  // image mode reads V itself
        L.vt = off;       off += align_up(nbg * ntiles * kD * VT_TILE * 2, 256);
        L.plan = chunk_plan(g);
        L.NB = (int64_t)L.plan.nbchunk * nbg * g.nb;
        L.crows = (int64_t)g.B * g.Hq << L.plan.pc_log2;
        const size_t NB = (size_t)L.NB;
        const size_t rows = (size_t)g.B * g.Hq * g.N;
        const size_t npairs = rows * g.top_k;
        const size_t cslots = (size_t)L.crows << pair_stride_log2(g.top_k);
        L.counts = off;   off += align_up(NB * 4, 256);
        L.offsets = off;  off += align_up((NB + 1) * 4, 256);
        L.cursor = off;   off += align_up(NB * 4, 256);
        L.unit_off = off; off += align_up((NB + 1) * 4, 256);
        L.pairs = off;    off += align_up(npairs * 4, 256);
        L.rev = off;      off += align_up(npairs * 4, 256);
        L.part_o = off;   off += align_up((cslots + UNIT_ROWS) * kD * 2, 256);
        L.part_lse = off; off += align_up(((size_t)L.crows * g.top_k + UNIT_ROWS) * 4, 256);
    }
    L.total = off;
    return L;
}

size_t attend_workspace_bytes(const Geometry& g) { return attend_layout(g).total; }

template <int BS>
static void launch_partial(const PartArgs& pa, hipStream_t s) {
    // one resident wave of workgroups: CUs x workgroups per CU
    static std::atomic<int> cache[kMaxDevices];
    const int grid = resident_grid(k_block_partial<BS>, 256, cache);
    hipLaunchKernelGGL(k_block_partial<BS>, dim3(grid), dim3(256), 0, s, pa);
}

hipError_t launch_attend(const Geometry& g, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* idx, float* out, void* ws,
                         hipStream_t s, const hipEvent_t* ev) {
    const float scale_log2 = g.scale * kLog2e;
    const AttendLayout L = attend_layout(g);
    char* base = static_cast<char*>(ws);
    uint16_t* vt = reinterpret_cast<uint16_t*>(base + L.vt);
    const int ntiles = (g.N + VT_TILE - 1) / VT_TILE;
    const int nbg = g.B * g.Hkv;
    if (!g.causal) {
        ImgArgs a{q, k, v, idx, out, g.Hq, g.Hkv, g.N, g.nb, g.top_k,
                  (int64_t)g.B * g.Hq * g.nb, scale_log2, g.consensus};
        const unsigned grid = (unsigned)(((a.n_qblocks + 3) / 4 + 7) / 8 * 8);  // multiple of 8
        for (int i = 4; i < 8; ++i) mark(ev, i, s);
        if (g.top_k <= kMaxTopK)
            hipLaunchKernelGGL(k_image_attend<kMaxTopK>, dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(k_image_attend<kMaxTopKWide>, dim3(grid), dim3(256), 0, s, a);
        mark(ev, 8, s);
        return hipGetLastError();
    }
    uint32_t* counts = reinterpret_cast<uint32_t*>(base + L.counts);
    // the transpose also clears the bucket counts
    hipLaunchKernelGGL(k_transpose_v<VT_TILE>, dim3((unsigned)(nbg * ntiles)), dim3(256), 0, s, v,
                       vt, g.N, ntiles, counts, (size_t)L.NB);
    uint32_t* offsets = reinterpret_cast<uint32_t*>(base + L.offsets);
    uint32_t* cursor = reinterpret_cast<uint32_t*>(base + L.cursor);
    uint32_t* unit_off = reinterpret_cast<uint32_t*>(base + L.unit_off);
    uint32_t* pairs = reinterpret_cast<uint32_t*>(base + L.pairs);
    uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
    float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
    uint32_t* rev = reinterpret_cast<uint32_t*>(base + L.rev);
    const ChunkPlan& P = L.plan;
    const int NB = (int)L.NB;
    const int sp_log2 = pair_stride_log2(g.top_k);

    // one route per KV group: bucket (group row, slot) pairs, each gathered
    // once per query head of the group
    const int rep = g.Hq / g.Hkv;
    const int expand = g.consensus ? rep : 1;
    const int64_t rows = (int64_t)g.B * (g.consensus ? g.Hkv : g.Hq) * g.N;
    BucketArgs ba{idx, counts, cursor, pairs, rev, rows, g.Hq, g.Hkv, g.N, g.bs, g.nb, g.top_k, g.window,
                  1 << P.tc_log2, sp_log2, g.consensus, 0, P.pc_log2, nbg};
    ba.group_pairs = g.consensus;
    ba.bc_log2 = P.bc_log2;
    const int nch = (g.N + (1 << P.tc_log2) - 1) >> P.tc_log2;
    const dim3 bgrid((unsigned)(nbg * nch));
    const size_t lds = g.nb <= BK_LDS_MAX ? (size_t)g.nb * 4 : 0;
    launch_bucket<false>(bgrid, lds, s, ba);
    mark(ev, 4, s);
    // one scan workgroup per 4096 buckets (at most 16), each finding its base itself
    const unsigned scan_wg = (unsigned)std::min<int64_t>(16, std::max<int64_t>(1, L.NB / 4096));
    hipLaunchKernelGGL(k_bucket_scan, dim3(scan_wg), dim3(1024), 0, s, counts, offsets, cursor, unit_off,
                       NB, expand);
    mark(ev, 5, s);
    launch_bucket<true>(bgrid, lds, s, ba);
    mark(ev, 6, s);

    // stage events: with one chunk, 7 follows the partials and 8 the merge;
    // with several, 7 follows the last chunk's merge and stage 8 is empty
    const uint32_t cslots = (uint32_t)(L.crows << sp_log2);
    const uint32_t cpairs = (uint32_t)(L.crows * g.top_k);
    for (int c = 0; c < P.nchunk; ++c) {
        const int t_base = c << P.pc_log2;
        const int nbc = nbg * g.nb;  // buckets of one bucket chunk
        const int b0 = (c << (P.pc_log2 - P.bc_log2)) * nbc;
        const int b1 = std::min(NB, b0 + (nbc << (P.pc_log2 - P.bc_log2)));
        PartArgs pa{q, k, vt, pairs, offsets, unit_off, part_o, part_lse, cslots, cpairs, g.N,
                    g.nb, NB, ntiles, sp_log2, b0, b1, nbc, P.pc_log2, t_base, scale_log2,
                    expand};
        switch (g.bs) {
            case 16: launch_partial<16>(pa, s); break;
            case 32: launch_partial<32>(pa, s); break;
            case 64: launch_partial<64>(pa, s); break;
            default: launch_partial<128>(pa, s); break;
        }
        if (P.nchunk == 1) mark(ev, 7, s);
        const int span = std::min(1 << P.pc_log2, g.N - t_base);
        const int wtiles = (span + 63) / 64;
        WinArgs wa{q, k, vt, idx, part_o, part_lse, rev, offsets, out, rows, g.Hq, g.Hkv, g.N,
                   g.bs, g.top_k, g.window, wtiles, nbg * rep * wtiles, ntiles, sp_log2, b0,
                   P.pc_log2, t_base, scale_log2, g.consensus, expand};
        const int64_t wgrid = ((int64_t)wa.items + 7) / 8 * 8;  // multiple of the XCD count
        if (g.top_k <= kMaxTopK)
            hipLaunchKernelGGL(k_window_merge<kMaxTopK>, dim3((unsigned)wgrid), dim3(256), 0, s, wa);
        else
            hipLaunchKernelGGL(k_window_merge<kMaxTopKWide>, dim3((unsigned)wgrid), dim3(256), 0, s,
                               wa);
    }
    if (P.nchunk > 1) mark(ev, 7, s);
    mark(ev, 8, s);
    return hipGetLastError();
}

}  // namespace lsa
