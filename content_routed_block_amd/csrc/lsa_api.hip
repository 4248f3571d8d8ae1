// C ABI of liblsa (declared in include/lsa.h): argument validation,
// workspace layout and the launch sequence of each call.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "lsa.h"
#include "lsa_common.hpp"
#include "lsa_launch.hpp"

namespace {

using lsa::Geometry;

bool pow2_block(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// Validates the parameters; fills g on success.
lsa_status check_params(const lsa_params* p, Geometry* g) {
    if (!p) return LSA_ERR_NULL;
    if (p->batch < 1 || p->q_heads < 1 || p->kv_heads < 1 || p->seq_len < 1 || p->head_dim < 1 ||
        p->block < 1 || p->top_k < 1)
        return LSA_ERR_SHAPE;
    if (p->q_heads % p->kv_heads) return LSA_ERR_SHAPE;
    if (p->causal != 0 && p->causal != 1) return LSA_ERR_SHAPE;
    if (p->consensus != 0 && p->consensus != 1) return LSA_ERR_SHAPE;
    uint32_t beta_bits;
    memcpy(&beta_bits, &p->beta, 4);
    if ((beta_bits & 0x7FFFFFFFu) >= 0x7F800000u) return LSA_ERR_SHAPE;  // beta not finite
    if (p->seq_len % p->block) return LSA_ERR_SHAPE;
    if (p->causal) {
        if (p->window < p->block || p->window % p->block) return LSA_ERR_SHAPE;
    } else if (p->window != 0) {
        return LSA_ERR_SHAPE;
    }
    if (p->head_dim != 64) return LSA_ERR_UNSUPPORTED;
    if (!pow2_block(p->block)) return LSA_ERR_UNSUPPORTED;
    if (!p->causal && p->block != 16) return LSA_ERR_UNSUPPORTED;
    if (p->top_k > lsa::kMaxTopKWide) return LSA_ERR_UNSUPPORTED;
    if (p->beta != 0.f && (!p->causal || p->consensus)) return LSA_ERR_UNSUPPORTED;
    if (p->beam < 0) return LSA_ERR_SHAPE;
    if (p->chunk != 0 && (p->chunk < 64 || (p->chunk & (p->chunk - 1)))) return LSA_ERR_SHAPE;
    if (p->beam > 0 && (p->beam >= lsa::kMaxTopK || p->consensus || p->beta != 0.f))
        return LSA_ERR_UNSUPPORTED;
    const int64_t nb = p->seq_len / p->block;
    if (nb > 65536) return LSA_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)p->batch * p->q_heads * p->seq_len;
    if ((rows << lsa::pair_stride_log2(p->top_k)) + 64 >= ((int64_t)1 << 32))
        return LSA_ERR_UNSUPPORTED;  // 32-bit pair ids (+ 64 dummy rows)
    if (p->beam > 0 && (rows << lsa::pair_stride_log2(p->beam + 1)) + 64 >= ((int64_t)1 << 32))
        return LSA_ERR_UNSUPPORTED;  // the same for the two-level router's (row, node) pairs
    if ((int64_t)p->batch * p->q_heads * ((p->seq_len + 255) / 256) >= ((int64_t)1 << 31))
        return LSA_ERR_UNSUPPORTED;
    uint32_t scale_bits;
    memcpy(&scale_bits, &p->scale, 4);
    if ((scale_bits & 0x7FFFFFFFu) > 0x7F800000u) return LSA_ERR_SHAPE;  // NaN scale
    g->B = p->batch;
    g->Hq = p->q_heads;
    g->Hkv = p->kv_heads;
    g->N = p->seq_len;
    g->D = p->head_dim;
    g->bs = p->block;
    g->nb = (int)nb;
    g->top_k = p->top_k;
    g->window = p->window;
    g->causal = p->causal;
    g->consensus = p->consensus;
    g->beta = p->beta;
    g->beam = p->beam;
    g->chunk = p->chunk;
    g->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    return LSA_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

size_t route_idx_bytes(const Geometry& g) {
    return (size_t)g.B * (g.consensus ? g.Hkv : g.Hq) * (g.causal ? (size_t)g.N : (size_t)g.nb) *
           g.top_k * 4;
}

size_t forward_ws(const Geometry& g, bool with_idx) {
    size_t off = lsa::align_up((size_t)g.B * g.Hkv * g.nb * lsa::kD * 4, 256);  // kbar
    if (with_idx) off += lsa::align_up(route_idx_bytes(g), 256);
    const size_t r = lsa::route_workspace_bytes(g), at = lsa::attend_workspace_bytes(g);
    return off + (r > at ? r : at);
}

lsa_status from_hip(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_ERR_DEVICE; }

}  // namespace

extern "C" {

size_t lsa_workspace_bytes(const lsa_params* p, int32_t op) {
    Geometry g;
    if (check_params(p, &g) != LSA_OK) return (size_t)-1;
    switch (op) {
        case LSA_OP_SUMMARIZE: return 0;
        case LSA_OP_ROUTE: return lsa::route_workspace_bytes(g);
        case LSA_OP_ATTEND: return lsa::attend_workspace_bytes(g);
        case LSA_OP_FORWARD: return forward_ws(g, true);  // enough with or without idx_out
        case LSA_OP_DECODE:
            return g.causal && !g.consensus && g.beta == 0.f && !g.beam
                       ? lsa::decode_workspace_bytes(g, g.N)
                       : (size_t)-1;
        default: return (size_t)-1;
    }
}

lsa_status lsa_block_summarize(const lsa_params* p, const void* x, int32_t heads, float* xbar,
                               void* stream) {
    Geometry g;
    lsa_status st = check_params(p, &g);
    if (st != LSA_OK) return st;
    if (!x || !xbar) return LSA_ERR_NULL;
    if (heads < 1) return LSA_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(xbar, 16)) return LSA_ERR_ALIGN;
    return from_hip(lsa::launch_summarize(static_cast<const uint16_t*>(x), xbar, g.B * heads, g.N,
                                          g.bs, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_route_topk(const lsa_params* p, const void* q, const float* kbar, int32_t* idx,
                          void* workspace, size_t workspace_bytes, void* stream) {
    Geometry g;
    lsa_status st = check_params(p, &g);
    if (st != LSA_OK) return st;
    if (g.beta != 0.f) return LSA_ERR_UNSUPPORTED;  // the score needs the keys: lsa_route_cumulant
    if (!q || !kbar || !idx || !workspace) return LSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kbar, 16) || !aligned(idx, 16)) return LSA_ERR_ALIGN;
    if (!aligned(workspace, 256)) return LSA_ERR_ALIGN;
    if (workspace_bytes < lsa::route_workspace_bytes(g)) return LSA_ERR_WORKSPACE;
    return from_hip(lsa::launch_route(g, static_cast<const uint16_t*>(q), kbar, idx, workspace,
                                      static_cast<hipStream_t>(stream)));
}

lsa_status lsa_route_cumulant(const lsa_params* p, const void* q, const void* k, int32_t* idx,
                              void* stream) {
    Geometry g;
    lsa_status st = check_params(p, &g);
    if (st != LSA_OK) return st;
    if (!g.causal || g.consensus) return LSA_ERR_UNSUPPORTED;
    if (!q || !k || !idx) return LSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(idx, 16)) return LSA_ERR_ALIGN;
    return from_hip(lsa::launch_route_cumulant(g, static_cast<const uint16_t*>(q),
                                               static_cast<const uint16_t*>(k), idx,
                                               static_cast<hipStream_t>(stream)));
}

lsa_status lsa_sparse_attend(const lsa_params* p, const void* q, const void* k, const void* v,
                             const int32_t* idx, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
    Geometry g;
    lsa_status st = check_params(p, &g);
    if (st != LSA_OK) return st;
    if (!q || !k || !v || !idx || !out) return LSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 16) ||
        !aligned(out, 16))
        return LSA_ERR_ALIGN;
    const size_t need = lsa::attend_workspace_bytes(g);
    if (need) {
        if (!workspace) return LSA_ERR_NULL;
        if (!aligned(workspace, 256)) return LSA_ERR_ALIGN;
        if (workspace_bytes < need) return LSA_ERR_WORKSPACE;
    }
    return from_hip(lsa::launch_attend(g, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), idx, out, workspace,
                                       static_cast<hipStream_t>(stream)));
}

static lsa_status forward_impl(const lsa_params* p, const void* q, const void* k, const void* v,
                               float* out, int32_t* idx_out, void* workspace,
                               size_t workspace_bytes, void* stream, const hipEvent_t* ev) {
    Geometry g;
    lsa_status st = check_params(p, &g);
    if (st != LSA_OK) return st;
    if (!q || !k || !v || !out || !workspace) return LSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        (idx_out && !aligned(idx_out, 16)))
        return LSA_ERR_ALIGN;
    if (!aligned(workspace, 256)) return LSA_ERR_ALIGN;
    if (workspace_bytes < forward_ws(g, idx_out == nullptr)) return LSA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    float* kbar = reinterpret_cast<float*>(base);
    size_t off = lsa::align_up((size_t)g.B * g.Hkv * g.nb * lsa::kD * 4, 256);
    int32_t* idx = idx_out;
    if (!idx) {
        idx = reinterpret_cast<int32_t*>(base + off);
        off += lsa::align_up(route_idx_bytes(g), 256);
    }
    void* rest = base + off;
    lsa::mark(ev, 0, s);
    if (g.beta != 0.f) {  // second-cumulant score: routed from the keys themselves
        lsa::mark(ev, 1, s);
        st = from_hip(lsa::launch_route_cumulant(g, static_cast<const uint16_t*>(q),
                                                 static_cast<const uint16_t*>(k), idx, s));
        if (st != LSA_OK) return st;
        lsa::mark(ev, 2, s);
        lsa::mark(ev, 3, s);
    } else if (g.beam == 0) {
        // flat routing: the key summary also prepares the router's inputs
        st = from_hip(lsa::launch_summary_and_route_prep(g, static_cast<const uint16_t*>(k),
                                                         static_cast<const uint16_t*>(q), kbar,
                                                         rest, s));
        if (st != LSA_OK) return st;
        lsa::mark(ev, 1, s);
        st = from_hip(lsa::launch_route_prepared(g, static_cast<const uint16_t*>(q), kbar, idx,
                                                 rest, s, ev));
        if (st != LSA_OK) return st;
    } else {
        st = from_hip(lsa::launch_summarize(static_cast<const uint16_t*>(k), kbar, g.B * g.Hkv,
                                            g.N, g.bs, s));
        if (st != LSA_OK) return st;
        lsa::mark(ev, 1, s);
        st = from_hip(lsa::launch_route(g, static_cast<const uint16_t*>(q), kbar, idx, rest, s,
                                        ev));
        if (st != LSA_OK) return st;
    }
    return from_hip(lsa::launch_attend(g, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), idx, out, rest, s, ev));
}

lsa_status lsa_forward(const lsa_params* p, const void* q, const void* k, const void* v,
                       float* out, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
    return forward_impl(p, q, k, v, out, idx_out, workspace, workspace_bytes, stream, nullptr);
}

lsa_status lsa_forward_profiled(const lsa_params* p, const void* q, const void* k, const void* v,
                                float* out, int32_t* idx_out, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* events) {
    if (!events) return LSA_ERR_NULL;
    for (int i = 0; i < LSA_PROFILE_EVENTS; ++i)
        if (!events[i]) return LSA_ERR_NULL;
    return forward_impl(p, q, k, v, out, idx_out, workspace, workspace_bytes, stream,
                        reinterpret_cast<const hipEvent_t*>(events));
}

// Validation shared by the two decode entry points; fills g (g.N = T).
static lsa_status decode_check(const lsa_params* p, int32_t cache_len, const void* q,
                               const void* k_cache, const void* v_cache, const float* kbar_cache,
                               const float* out, const int32_t* idx_out, Geometry* g) {
    if (!p) return LSA_ERR_NULL;
    // the cache geometry is validated as a sequence of cache_len tokens
    lsa_params pc = *p;
    pc.seq_len = cache_len;
    lsa_status st = check_params(&pc, g);
    if (st != LSA_OK) return st;
    if (!p->causal) return LSA_ERR_SHAPE;
    if (p->consensus || p->beta != 0.f || p->beam) return LSA_ERR_UNSUPPORTED;
    if (p->seq_len < 1 || p->seq_len > cache_len) return LSA_ERR_SHAPE;
    if (!q || !k_cache || !v_cache || !kbar_cache || !out) return LSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(kbar_cache, 16) || !aligned(out, 16) || (idx_out && !aligned(idx_out, 16)))
        return LSA_ERR_ALIGN;
    return LSA_OK;
}

lsa_status lsa_decode(const lsa_params* p, int32_t cache_len, const void* q, const void* k_cache,
                      const void* v_cache, float* kbar_cache, float* out, int32_t* idx_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
    Geometry g;
    lsa_status st = decode_check(p, cache_len, q, k_cache, v_cache, kbar_cache, out, idx_out, &g);
    if (st != LSA_OK) return st;
    if (!workspace) return LSA_ERR_NULL;
    if (!aligned(workspace, 256)) return LSA_ERR_ALIGN;
    if (workspace_bytes < lsa::decode_workspace_bytes(g, cache_len)) return LSA_ERR_WORKSPACE;
    g.N = p->seq_len;
    return from_hip(lsa::launch_decode(g, cache_len, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k_cache),
                                       static_cast<const uint16_t*>(v_cache), kbar_cache, out,
                                       idx_out, workspace, static_cast<hipStream_t>(stream)));
}

lsa_status lsa_decode_noalloc(const lsa_params* p, int32_t cache_len, const void* q,
                              const void* k_cache, const void* v_cache, float* kbar_cache,
                              float* out, int32_t* idx_out, void* stream) {
    Geometry g;
    lsa_status st = decode_check(p, cache_len, q, k_cache, v_cache, kbar_cache, out, idx_out, &g);
    if (st != LSA_OK) return st;
    // the same workspace layout as lsa_decode, placed in the static array
    static_assert(lsa::kStaticScratchBytes == LSA_STATIC_SCRATCH_BYTES, "header and library");
    if (lsa::decode_workspace_bytes(g, cache_len) > lsa::kStaticScratchBytes)
        return LSA_ERR_SCRATCH;
    void* scratch = nullptr;
    if (lsa::static_scratch(&scratch) != hipSuccess) return LSA_ERR_DEVICE;
    g.N = p->seq_len;
    return from_hip(lsa::launch_decode(g, cache_len, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k_cache),
                                       static_cast<const uint16_t*>(v_cache), kbar_cache, out,
                                       idx_out, scratch, static_cast<hipStream_t>(stream)));
}

const char* lsa_status_str(lsa_status s) {
    switch (s) {
        case LSA_OK: return "ok";
        case LSA_ERR_NULL: return "a required pointer is NULL";
        case LSA_ERR_SHAPE: return "inconsistent sizes or parameters";
        case LSA_ERR_UNSUPPORTED: return "parameters outside what this build supports";
        case LSA_ERR_ALIGN: return "misaligned pointer";
        case LSA_ERR_WORKSPACE: return "workspace too small";
        case LSA_ERR_DEVICE: return "HIP launch failed";
        case LSA_ERR_SCRATCH: return "needs more scratch than the library's static array holds";
        default: return "unknown status";
    }
}

}  // extern "C"
