// Internal launchers behind the liblsa C ABI (host side).  Every launcher
// assumes its arguments were validated by the ABI layer and enqueues work on
// `stream` without synchronising.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsa {

struct Geometry {
    int B, Hq, Hkv, N, D, bs, nb, top_k, window, causal;
    int consensus;  // 1: one route per KV group (idx heads = Hkv)
    float scale;    // resolved (> 0)
    float beta;     // second-cumulant weight (0: the block-mean score)
    int beam;       // two-level routing: nodes kept per row (0: flat routing)
};

// x [BH, N, 64] bf16 -> xbar [BH, N/bs, 64] fp32
hipError_t launch_summarize(const uint16_t* x, float* xbar, int BH, int N, int bs,
                            hipStream_t s);

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t s);

// Routing workspace (bytes) and launch.  qbar may be NULL in causal mode.
size_t route_workspace_bytes(const Geometry& g);
hipError_t launch_route(const Geometry& g, const uint16_t* q, const float* kbar,
                        int32_t* idx, void* ws, hipStream_t s,
                        const hipEvent_t* ev = nullptr);

// log2 of the pair-id stride: the smallest power of two >= top_k.
int pair_stride_log2(int top_k);

// Sparse attention workspace (bytes) and launch.
// Second level of two-level routing: scores every block of the nodes listed
// in slots [B*Hq*N][beam + 1] (kept nodes, then the tail node) and writes
// the top-k to idx.  bhi/blo: bf16 hi/lo block means [B*Hkv][nb_pad][64].
size_t tree_level2_bytes(const Geometry& g);
hipError_t launch_tree_level2(const Geometry& g, const uint16_t* q, const uint16_t* bhi,
                              const uint16_t* blo, int nb_pad, const int32_t* slots, int32_t* idx,
                              void* ws, hipStream_t s);

// Second-cumulant routing (beta != 0, causal, per query head): needs no
// workspace.
hipError_t launch_route_cumulant(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                 int32_t* idx, hipStream_t s);

size_t attend_workspace_bytes(const Geometry& g);
hipError_t launch_attend(const Geometry& g, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* idx, float* out, void* ws,
                         hipStream_t s, const hipEvent_t* ev = nullptr);

// Single-query decode against a cache of t_max tokens (g.N = tokens filled).
size_t decode_workspace_bytes(const Geometry& g, int t_max);
hipError_t launch_decode(const Geometry& g, int t_max, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, float* kbar, float* out, int32_t* idx_out, void* ws,
                         hipStream_t s);

// Records profiling event i (if any) on the stream.
inline void mark(const hipEvent_t* ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace lsa
