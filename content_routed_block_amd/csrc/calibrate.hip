// Access-pattern probe (include/lsa_calibration.h): 128-byte rows copied
// between two tables, the read side, the write side, both or neither taken
// from index lists.  Eight lanes move one row with 16-byte accesses, so a
// wave moves eight rows, as the partial kernel's gathers and stores do.
#include "lsa_calibration.h"
#include "lsa_common.hpp"

namespace {

__global__ __launch_bounds__(256) void k_access(const lsa::u32x4* __restrict__ src,
                                                lsa::u32x4* __restrict__ dst,
                                                const uint32_t* __restrict__ ridx,
                                                const uint32_t* __restrict__ widx,
                                                int64_t table_rows, int64_t n, int mode) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t i = t >> 3;
    const int part = (int)(t & 7);
    if (i >= n) return;
    const uint64_t r = (mode & 1) ? ridx[i] : (uint64_t)i;
    const uint64_t w = (mode & 2) ? widx[i] : (uint64_t)i;
    if (r >= (uint64_t)table_rows || w >= (uint64_t)table_rows) return;
    dst[w * 8 + part] = src[r * 8 + part];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" lsa_status lsa_calibrate_access(const void* src, void* dst, const uint32_t* ridx,
                                           const uint32_t* widx, int64_t table_rows, int64_t n,
                                           int32_t mode, void* stream) {
    if (mode < 0 || mode > 3 || n < 0 || table_rows < 0 || n >= ((int64_t)1 << 28))
        return LSA_ERR_SHAPE;
    if (!src || !dst || ((mode & 1) && !ridx) || ((mode & 2) && !widx)) return LSA_ERR_NULL;
    if (mode != 3 && n > table_rows) return LSA_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(dst)) return LSA_ERR_ALIGN;
    if (n == 0) return LSA_OK;
    const int64_t threads = n * 8;
    hipLaunchKernelGGL(k_access, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const lsa::u32x4*>(src),
                       static_cast<lsa::u32x4*>(dst), ridx, widx, table_rows, n, (int)mode);
    return hipGetLastError() == hipSuccess ? LSA_OK : LSA_ERR_DEVICE;
}
