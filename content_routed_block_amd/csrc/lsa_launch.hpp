// Internal launchers behind the liblsa C ABI (host side).  Every launcher
// assumes its arguments were validated by the ABI layer and enqueues work on
// `stream` without synchronising.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace lsa {

struct Geometry {
    int B, Hq, Hkv, N, D, bs, nb, top_k, window, causal;
    int consensus;  // 1: one route per KV group (idx heads = Hkv)
    float scale;    // resolved (> 0)
    float beta;     // second-cumulant weight (0: the block-mean score)
    int beam;       // two-level routing: nodes kept per row (0: flat routing)
    int chunk;      // causal attention: positions per chunk (0: chosen from the geometry)
};

// x [BH, N, 64] bf16 -> xbar [BH, N/bs, 64] fp32
hipError_t launch_summarize(const uint16_t* x, float* xbar, int BH, int N, int bs,
                            hipStream_t s);

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t s);

// The key summary of a layer that routes on it: also writes the routing
// kernels' bf16 hi/lo block means [BH][nb_pad][64] and the chunk maxima of
// their norms (every slot of every chunk line), and clears the router's
// kRouteCounterWords counters (when counters is not NULL).
hipError_t launch_summarize_route(const uint16_t* x, float* xbar, int BH, int N, int bs,
                                  uint16_t* khi, uint16_t* klo, float* ckn, float* clo,
                                  int nb_pad, uint32_t* counters, hipStream_t s);
// The same for blocks of 16 tokens, with the pooling of q [BHq, N, 64] into
// qbar [BHq, N/16, 64] (fp32) in the same launch (image mode).
hipError_t launch_summarize_route_pool16(const uint16_t* k, float* kbar, int BHk, const uint16_t* q,
                                         float* qbar, int BHq, int N, uint16_t* khi, uint16_t* klo,
                                         float* ckn, float* clo, int nb_pad, uint32_t* counters,
                                         hipStream_t s);

// Routing workspace (bytes) and launch.  qbar may be NULL in causal mode.
size_t route_workspace_bytes(const Geometry& g);
hipError_t launch_route(const Geometry& g, const uint16_t* q, const float* kbar,
                        int32_t* idx, void* ws, hipStream_t s,
                        const hipEvent_t* ev = nullptr);
// A layer's key summary and the preparation of flat routing in one launch:
// summarises k into kbar, writes the router's inputs and clears its
// counters (in image mode the same launch pools q into the routing
// workspace); launch_route_prepared then routes.  Only for flat routing
// (beam = 0, beta = 0).
hipError_t launch_summary_and_route_prep(const Geometry& g, const uint16_t* k, const uint16_t* q,
                                         float* kbar, void* ws, hipStream_t s);
hipError_t launch_route_prepared(const Geometry& g, const uint16_t* q, const float* kbar,
                                 int32_t* idx, void* ws, hipStream_t s,
                                 const hipEvent_t* ev = nullptr);

// log2 of the pair-id stride: the smallest power of two >= top_k.
int pair_stride_log2(int top_k);

// Sparse attention workspace (bytes) and launch.
// Second level of two-level routing: scores every block of the nodes listed
// in slots [rows][beam + 1] (kept nodes, then the tail node) and writes the
// top-k to idx.  Rows are causal positions (B*Hq*N, queries q) or, in image
// mode, query blocks (B*Hq*nb, pooled fp32 queries qbar).  bhi/blo: bf16
// hi/lo block means [B*Hkv][nb_pad][64].
size_t tree_level2_bytes(const Geometry& g);
hipError_t launch_tree_level2(const Geometry& g, const uint16_t* q, const float* qbar,
                              const uint16_t* bhi, const uint16_t* blo, int nb_pad,
                              const int32_t* slots, int32_t* idx, void* ws, hipStream_t s);

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
// The library's static scratch array on the current device (see decode.hip):
// its size, and its device address (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_decode(const Geometry& g, int t_max, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, float* kbar, float* out, int32_t* idx_out, void* ws,
                         hipStream_t s);

// Records profiling event i (if any) on the stream.
inline void mark(const hipEvent_t* ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Grid of a persistent kernel: one resident wave of workgroups on the current
// device (CUs x workgroups per CU at `threads` threads and no dynamic LDS).
// Each kernel keeps one cached value per device; concurrent first calls from
// several host threads compute the same value, so plain atomic stores suffice.
constexpr int kMaxDevices = 64;
template <typename Kernel>
inline int resident_grid(Kernel kernel, int threads, std::atomic<int> (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>* slot = dev < kMaxDevices ? &cache[dev] : nullptr;
    int grid = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (grid > 0) return grid;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    grid = cus * per_cu;
    if (slot) slot->store(grid, std::memory_order_relaxed);
    return grid;
}

}  // namespace lsa
