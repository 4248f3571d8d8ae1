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
// Design (gfx950).  A workgroup owns 256 query rows of one (b, h): four
// waves x 64 rows.  Candidate block means stream through LDS in chunks of
// 32, split into bf16 hi + bf16 lo parts.  Scores are 32x32x16 bf16 MFMA
// tiles S^T = Kbar_chunk . Q^T, so lane l holds query l%32 (of each 32-row
// tile) and 16 candidates whose indices fall in one residue class mod 32
// per register.
//   pass 1  hi-only scores a_c; every lane keeps a running maximum per
//           register, i.e. the maximum over each residue class: 32 group
//           maxima per query.  The k-th largest group maximum, lowered by a
//           rigorous bound on |a_c - b_c|, is a threshold that at least k
//           of the pass-2 scores b_c reach.
//   pass 2  hi+lo scores b_c (fp32 accuracy); candidates at or above the
//           threshold are appended to the query's survivor list in LDS
//           (~20 per query on random data; capacity 32).
//   select  one lane per query inserts its survivors into a 16-entry sorted
//           list of 64-bit keys (score, then lower index), then sorts the
//           chosen block ids ascending.
// Queries whose survivor list overflows (ties, adversarial inputs) are
// queued and redone exactly by k_route_fallback.
#include <math.h>

#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace lsa {

constexpr int RT_ROWS = 256;   // query rows per workgroup
constexpr int RT_CH = 32;      // candidates per step
constexpr int RT_CAP = 32;     // survivor slots per query
constexpr int RT_PITCH = 72;   // padded LDS row pitch (bf16), conflict-free 16-byte reads
constexpr int FB_GRID = 256;   // workgroups of the exact fallback

struct RouteArgs {
    const uint16_t* q;    // causal: bf16 [B,Hq,N,64]
    const float* qbar;    // image: fp32 [B,Hq,nb,64]
    const float* kbar;    // [B,Hkv,nb,64]
    int32_t* idx;         // [B,Hq,P,top_k]
    uint32_t* ovf_count;  // queued overflow rows
    uint32_t* ovf_rows;   // [B*Hq*P]
    float* fb_scratch;    // [FB_GRID][nb]
    int Hq, Hkv, N, bs, nb, top_k, window;
    int P;      // rows per (b, h): N (causal) or nb (image)
    int tiles;  // ceil(P / RT_ROWS)
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

// k-th largest (1 <= k <= 16) of the 32 values held as 16 in this lane and 16
// in lane ^ 32.  Both lanes of the pair return the same value.
__device__ __forceinline__ float kth_largest_of_pair(float (&v)[16], int k) {
    bitonic_sort_desc<16>(v);
    float w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float other = __shfl_xor(v[15 - i], 32, kWave);
        w[i] = fmaxf(v[i], other);  // bitonic; holds the 16 largest of the union
    }
    bitonic_merge_desc<16>(w);
    float r = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i == k - 1) r = w[i];
    return r;
}

__device__ __forceinline__ void insert_key(uint64_t (&L)[kMaxTopK], uint64_t x) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        const uint64_t a = L[j];
        const bool gt = x > a;
        L[j] = gt ? x : a;
        x = gt ? a : x;
    }
}

// Writes one idx row from a key list sorted by rank (m valid keys).
__device__ __forceinline__ void write_selection(int32_t* out, const uint64_t (&L)[kMaxTopK],
                                                int m, int top_k) {
    uint32_t cs[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) cs[j] = j < m ? key_block(L[j]) : 0xFFFFFFFFu;
    bitonic_sort_asc_u32<kMaxTopK>(cs);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j < top_k) out[j] = j < m ? (int32_t)cs[j] : -1;
}

// ------------------------------------------------------------ staging
// Thread tid stages candidate row tid/8, dims 8*(tid%8) .. +7 of the chunk.
__device__ __forceinline__ void load_chunk(const float* kb, int cb, int nb, int tid,
                                           f32x4& p0, f32x4& p1) {
    const int c = cb + (tid >> 3);
    if (c < nb) {
        const float* src = kb + (int64_t)c * kD + (tid & 7) * 8;
        p0 = *reinterpret_cast<const f32x4*>(src);
        p1 = *reinterpret_cast<const f32x4*>(src + 4);
    } else {
        p0 = f32x4{0.f, 0.f, 0.f, 0.f};
        p1 = p0;
    }
}

// Splits the staged floats into bf16 hi/lo, stores them, and returns the
// squared norms of the full row (kn2) and of its lo part (lo2), reduced over
// the 8 threads that share the row.
__device__ __forceinline__ void store_chunk(__bf16* s_hi, __bf16* s_lo, int tid, f32x4 p0,
                                            f32x4 p1, float& kn2, float& lo2) {
    float f[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    bf16x8 hi, lo;
    kn2 = 0.f;
    lo2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (__bf16)f[i];
        const float r = f[i] - (float)hi[i];
        lo[i] = (__bf16)r;
        const float lf = (float)lo[i];
        kn2 = fmaf(f[i], f[i], kn2);
        lo2 = fmaf(lf, lf, lo2);
    }
    const int off = (tid >> 3) * RT_PITCH + (tid & 7) * 8;
    *reinterpret_cast<bf16x8*>(s_hi + off) = hi;
    *reinterpret_cast<bf16x8*>(s_lo + off) = lo;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        kn2 += __shfl_xor(kn2, m, kWave);
        lo2 += __shfl_xor(lo2, m, kWave);
    }
}

__device__ __forceinline__ int row_candidates(bool causal, int row, int P, int bs, int window,
                                              int nb) {
    if (row >= P) return 0;
    return causal ? eligible_blocks(row, bs, window) : nb;
}

// ------------------------------------------------------------ main kernel
template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void k_route(RouteArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_hi[RT_CH * RT_PITCH];
    __shared__ __attribute__((aligned(16))) __bf16 s_lo[RT_CH * RT_PITCH];
    __shared__ float s_score[RT_ROWS * RT_CAP];
    __shared__ uint16_t s_cidx[RT_ROWS * RT_CAP];
    __shared__ int s_cnt[RT_ROWS * 2];
    __shared__ float s_red[8];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.x / a.tiles;
    const int tile = a.tiles - 1 - (int)(blockIdx.x - bh * a.tiles);  // heavy tiles first
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = h / (a.Hq / a.Hkv);
    const int P = a.P;
    const int row0 = tile * RT_ROWS;
    const float* kb = a.kbar + (int64_t)(b * a.Hkv + g) * a.nb * kD;

    int rq[2], Erow[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        rq[tt] = row0 + 64 * w + 32 * tt + l32;
        Erow[tt] = row_candidates(CAUSAL, rq[tt], P, a.bs, a.window, a.nb);
    }
    const int last = min(row0 + RT_ROWS, P) - 1;
    const int Emax = row_candidates(CAUSAL, last, P, a.bs, a.window, a.nb);
    const int wfirst = row0 + 64 * w;
    const int Ewmin = (wfirst + 63 < P) ? row_candidates(CAUSAL, wfirst, P, a.bs, a.window, a.nb) : 0;

    // ---- queries as the B operand (B[d][t] = Q[t][d]): lane holds dims
    // 8*half + 16*ks .. +7 of row rq[tt].
    bf16x8 Bq[2][4];
    bf16x8 Bql[2][4];  // image mode: lo part of the pooled query
    float qn[2], qln[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        float s2 = 0.f, l2 = 0.f;
        if (rq[tt] < P) {
            if (CAUSAL) {
                const uint16_t* qp = a.q + ((int64_t)bh * a.N + rq[tt]) * kD + 8 * half;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
                    float f[8];
                    unpack8(raw, f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) s2 = fmaf(f[i], f[i], s2);
                    Bq[tt][ks] = __builtin_bit_cast(bf16x8, raw);
                    Bql[tt][ks] = bf16x8{};
                }
            } else {
                const float* qp = a.qbar + ((int64_t)bh * a.nb + rq[tt]) * kD + 8 * half;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(qp + 16 * ks);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(qp + 16 * ks + 4);
                    const float f[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const __bf16 hi = (__bf16)f[i];
                        const __bf16 lo = (__bf16)(f[i] - (float)hi);
                        Bq[tt][ks][i] = hi;
                        Bql[tt][ks][i] = lo;
                        const float hf = (float)hi, lf = (float)lo;
                        s2 = fmaf(hf, hf, s2);
                        l2 = fmaf(lf, lf, l2);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Bq[tt][ks] = bf16x8{};
                Bql[tt][ks] = bf16x8{};
            }
        }
        s2 += __shfl_xor(s2, 32, kWave);
        l2 += __shfl_xor(l2, 32, kWave);
        qn[tt] = sqrtf(s2);
        qln[tt] = sqrtf(l2);
    }

    // ---- pass 1: hi-only scores, group maxima, norms of the candidates
    float gm[2][16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) gm[tt][r] = -INFINITY;
    float kn2max = 0.f, lo2max = 0.f;
    f32x4 p0, p1;
    if (Emax > 0) load_chunk(kb, 0, a.nb, tid, p0, p1);
    for (int cb = 0; cb < Emax; cb += RT_CH) {
        __syncthreads();
        float kn2, lo2;
        store_chunk(s_hi, s_lo, tid, p0, p1, kn2, lo2);
        if (cb + (tid >> 3) < Emax) {
            kn2max = fmaxf(kn2max, kn2);
            lo2max = fmaxf(lo2max, lo2);
        }
        __syncthreads();
        if (cb + RT_CH < Emax) load_chunk(kb, cb + RT_CH, a.nb, tid, p0, p1);
        bf16x8 A[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            A[ks] = *reinterpret_cast<const bf16x8*>(s_hi + l32 * RT_PITCH + 8 * half + 16 * ks);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma32(A[ks], Bq[tt][ks], acc);
            if (cb + RT_CH <= Ewmin) {
#pragma unroll
                for (int r = 0; r < 16; ++r) gm[tt][r] = fmaxf(gm[tt][r], acc[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = cb + 8 * (r >> 2) + 4 * half + (r & 3);
                    gm[tt][r] = fmaxf(gm[tt][r], c < Erow[tt] ? acc[r] : -INFINITY);
                }
            }
        }
    }
    // workgroup maxima of the candidate norms
#pragma unroll
    for (int m = 8; m < 64; m <<= 1) {
        kn2max = fmaxf(kn2max, __shfl_xor(kn2max, m, kWave));
        lo2max = fmaxf(lo2max, __shfl_xor(lo2max, m, kWave));
    }
    if (lane == 0) {
        s_red[w] = kn2max;
        s_red[4 + w] = lo2max;
    }
    __syncthreads();
    const float kn_max = sqrtf(fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])));
    const float lo_max = sqrtf(fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7])));

    // threshold: k-th largest group maximum minus a bound on |a_c - b_c|:
    // |q_hi . k_lo| + |q_lo . k_hi| + fp32 accumulation error.
    float theta[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const float th = kth_largest_of_pair(gm[tt], a.top_k);
        const float delta = 1.0625f * (qn[tt] * lo_max + qln[tt] * kn_max) +
                            6.2e-5f * (qn[tt] + qln[tt]) * kn_max;
        theta[tt] = th - delta;  // -inf stays -inf
    }

    // ---- pass 2: hi+lo scores, survivors to LDS
    int n[2] = {0, 0};
    if (Emax > 0) load_chunk(kb, 0, a.nb, tid, p0, p1);
    for (int cb = 0; cb < Emax; cb += RT_CH) {
        __syncthreads();
        float kn2, lo2;
        store_chunk(s_hi, s_lo, tid, p0, p1, kn2, lo2);
        __syncthreads();
        if (cb + RT_CH < Emax) load_chunk(kb, cb + RT_CH, a.nb, tid, p0, p1);
        bf16x8 Ah[4], Al[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Ah[ks] = *reinterpret_cast<const bf16x8*>(s_hi + l32 * RT_PITCH + 8 * half + 16 * ks);
            Al[ks] = *reinterpret_cast<const bf16x8*>(s_lo + l32 * RT_PITCH + 8 * half + 16 * ks);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc = mfma32(Ah[ks], Bq[tt][ks], acc);
                acc = mfma32(Al[ks], Bq[tt][ks], acc);
                if (!CAUSAL) acc = mfma32(Ah[ks], Bql[tt][ks], acc);
            }
            const int qs = 64 * w + 32 * tt + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = cb + 8 * (r >> 2) + 4 * half + (r & 3);
                if (acc[r] >= theta[tt] && c < Erow[tt]) {
                    if (n[tt] < RT_CAP) {
                        const int pos = half ? (RT_CAP - 1 - n[tt]) : n[tt];
                        s_score[qs * RT_CAP + pos] = acc[r];
                        s_cidx[qs * RT_CAP + pos] = (uint16_t)c;
                    }
                    ++n[tt];
                }
            }
        }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) s_cnt[(64 * w + 32 * tt + l32) * 2 + half] = n[tt];
    __syncthreads();

    // ---- selection: lane -> query 64*w + lane
    const int qs = 64 * w + lane;
    const int row = row0 + qs;
    if (row < P) {
        const int n0 = s_cnt[qs * 2], n1 = s_cnt[qs * 2 + 1];
        const int nt = n0 + n1;
        if (nt > RT_CAP) {
            const uint32_t slot = atomicAdd(a.ovf_count, 1u);
            a.ovf_rows[slot] = (uint32_t)((int64_t)bh * P + row);
        } else {
            uint64_t L[kMaxTopK];
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) L[j] = 0;
            for (int i = 0; i < nt; ++i) {
                const int e = i < n0 ? i : (RT_CAP - 1 - (i - n0));
                insert_key(L, sel_key(s_score[qs * RT_CAP + e], s_cidx[qs * RT_CAP + e]));
            }
            const int m = nt < a.top_k ? nt : a.top_k;
            write_selection(a.idx + ((int64_t)bh * P + row) * a.top_k, L, m, a.top_k);
        }
    }
}

// ------------------------------------------------------------ exact fallback
// One workgroup per queued row: fp32 scores of every candidate into a
// private scratch row, then top_k rounds of "largest key below the previous
// one".  Slow but exact for any input (ties included).
template <bool CAUSAL>
__global__ __launch_bounds__(256) void k_route_fallback(RouteArgs a) {
    __shared__ float s_q[kD];
    __shared__ uint64_t s_red[4];
    __shared__ uint64_t s_keys[kMaxTopK];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t count = *a.ovf_count;
    float* sc = a.fb_scratch + (size_t)blockIdx.x * a.nb;
    for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
        const uint32_t rid = a.ovf_rows[i];
        const int bh = (int)(rid / (uint32_t)a.P), row = (int)(rid % (uint32_t)a.P);
        const int h = bh % a.Hq, b = bh / a.Hq, g = h / (a.Hq / a.Hkv);
        const float* kb = a.kbar + (int64_t)(b * a.Hkv + g) * a.nb * kD;
        const int E = row_candidates(CAUSAL, row, a.P, a.bs, a.window, a.nb);
        if (tid < kD) {
            s_q[tid] = CAUSAL ? bf16_bits_to_f32(a.q[((int64_t)bh * a.N + row) * kD + tid])
                              : a.qbar[((int64_t)bh * a.nb + row) * kD + tid];
        }
        __syncthreads();
        for (int c = tid; c < E; c += 256) {
            float s = 0.f;
            for (int d = 0; d < kD; ++d) s = fmaf(s_q[d], kb[(int64_t)c * kD + d], s);
            sc[c] = s;
        }
        __syncthreads();
        uint64_t prev = ~0ull;
        int m = 0;
        for (int j = 0; j < a.top_k; ++j) {
            uint64_t best = 0;
            for (int c = tid; c < E; c += 256) {
                const uint64_t key = sel_key(sc[c], (uint32_t)c);
                if (key < prev && key > best) best = key;
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const uint64_t o = __shfl_xor(best, off, kWave);
                best = o > best ? o : best;
            }
            if (lane == 0) s_red[w] = best;
            __syncthreads();
            best = s_red[0];
#pragma unroll
            for (int q = 1; q < 4; ++q) best = s_red[q] > best ? s_red[q] : best;
            __syncthreads();
            if (best == 0) break;
            if (tid == 0) s_keys[j] = best;
            prev = best;
            ++m;
        }
        __syncthreads();
        if (tid == 0) {
            uint64_t L[kMaxTopK];
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) L[j] = j < m ? s_keys[j] : 0;
            write_selection(a.idx + (int64_t)rid * a.top_k, L, m, a.top_k);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ host side
static size_t route_rows(const Geometry& g) {
    return (size_t)g.B * g.Hq * (g.causal ? (size_t)g.N : (size_t)g.nb);
}

size_t route_workspace_bytes(const Geometry& g) {
    size_t off = 256;                                          // overflow counter
    off += align_up(route_rows(g) * sizeof(uint32_t), 256);    // overflow rows
    off += align_up((size_t)FB_GRID * g.nb * sizeof(float), 256);
    if (!g.causal) off += align_up((size_t)g.B * g.Hq * g.nb * kD * sizeof(float), 256);
    return off;
}

hipError_t launch_route(const Geometry& g, const uint16_t* q, const float* kbar, int32_t* idx,
                        void* ws, hipStream_t s, const hipEvent_t* ev) {
    char* base = static_cast<char*>(ws);
    RouteArgs a;
    a.ovf_count = reinterpret_cast<uint32_t*>(base);
    size_t off = 256;
    a.ovf_rows = reinterpret_cast<uint32_t*>(base + off);
    off += align_up(route_rows(g) * sizeof(uint32_t), 256);
    a.fb_scratch = reinterpret_cast<float*>(base + off);
    off += align_up((size_t)FB_GRID * g.nb * sizeof(float), 256);
    float* qbar = nullptr;
    if (!g.causal) qbar = reinterpret_cast<float*>(base + off);
    a.q = q;
    a.qbar = qbar;
    a.kbar = kbar;
    a.idx = idx;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.N = g.N;
    a.bs = g.bs;
    a.nb = g.nb;
    a.top_k = g.top_k;
    a.window = g.window;
    a.P = g.causal ? g.N : g.nb;
    a.tiles = (a.P + RT_ROWS - 1) / RT_ROWS;
    hipError_t e = launch_fill_u32(a.ovf_count, 1, 0u, s);
    if (e != hipSuccess) return e;
    if (!g.causal) {
        e = launch_summarize(q, qbar, g.B * g.Hq, g.N, g.bs, s);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((int64_t)g.B * g.Hq * a.tiles));
    if (g.causal) {
        hipLaunchKernelGGL(k_route<true>, grid, dim3(256), 0, s, a);
        mark(ev, 2, s);
        hipLaunchKernelGGL(k_route_fallback<true>, dim3(FB_GRID), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(k_route<false>, grid, dim3(256), 0, s, a);
        mark(ev, 2, s);
        hipLaunchKernelGGL(k_route_fallback<false>, dim3(FB_GRID), dim3(256), 0, s, a);
    }
    mark(ev, 3, s);
    return hipGetLastError();
}

}  // namespace lsa
