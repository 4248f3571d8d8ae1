// Device-side helpers shared by the liblsa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;          // head dim supported by this build
constexpr int kMaxTopK = 16;    // selection list length of the tuned kernels (top_k <= 16)
constexpr int kMaxTopKWide = 32;  // the longest selection (top_k 17..32 take wider lists)
constexpr int kTreeFanout = 16;  // key blocks per node of two-level routing
constexpr int kTreeFanoutLog2 = 4;
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {  // 16-byte aligned
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// 8 bf16 (as raw bits in a u32x4) -> 8 floats
__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
}

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16: A lane l holds A[l%16][8(l/16)+v], B holds B[8(l/16)+v][l%16],
// D lane l reg r holds D[4(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x16 bf16: A lane l holds A[l%32][8(l/32)+v], B holds B[8(l/32)+v][l%32],
// D lane l reg r holds D[8(r/4)+4(l/32)+r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- ordering keys
// Monotone map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Selection key: higher score first, then lower block index.
__device__ __forceinline__ uint64_t sel_key(float score, uint32_t c) {
    return ((uint64_t)ordered_bits(score) << 32) | (uint64_t)(0xFFFFFFFFu - c);
}
__device__ __forceinline__ uint32_t key_block(uint64_t key) {
    return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

// ---------------------------------------------------------------- causal geometry
// Routed candidates of causal query position t: the complete blocks that end
// before the block-aligned window, c in [0, E(t)).
__host__ __device__ __forceinline__ int eligible_blocks(int t, int bs, int window) {
    int e = t / bs - window / bs + 1;
    return e > 0 ? e : 0;
}

// ---------------------------------------------------------------- routing preparation
// The routing kernels read block means as bf16 hi + lo parts (hi = bf16(x),
// lo = bf16(x - hi)) and bound their error with the largest norms |x| and
// |lo| over each chunk of 32 blocks.  One lane holds 8 dims of a row; the
// row's 8 lanes are consecutive.  Writes the row's hi and lo parts and
// returns its norms (the same in all 8 lanes).
constexpr int kChunkMaxStride = 32;  // floats between chunk maxima: one 128-byte line each
// Each chunk's maximum is stored as kChunkMaxSlots partial maxima (one per
// workgroup that summarises part of the chunk; unused slots zero), at the
// start of its line: every slot is written on every call, so no clearing
// pass and no atomics are needed, and readers take the largest.
constexpr int kChunkMaxSlots = 8;
// Words at the start of the routing workspace holding the router's counters
// (queued rows, queued tiles), cleared before each routing pass.
constexpr int kRouteCounterWords = 64;

__device__ __forceinline__ void route_split_store(const float (&f)[8], uint16_t* hi_dst,
                                                  uint16_t* lo_dst, float& kn, float& ln) {
    bf16x8 hi, lo;
    float k2 = 0.f, l2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (__bf16)f[i];
        lo[i] = (__bf16)(f[i] - (float)hi[i]);
        const float lf = (float)lo[i];
        k2 = fmaf(f[i], f[i], k2);
        l2 = fmaf(lf, lf, l2);
    }
    *reinterpret_cast<bf16x8*>(hi_dst) = hi;
    *reinterpret_cast<bf16x8*>(lo_dst) = lo;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        k2 += __shfl_xor(k2, m, 64);
        l2 += __shfl_xor(l2, m, 64);
    }
    kn = sqrtf(k2);
    ln = sqrtf(l2);
}

// Maximum over the wave of a non-negative float (its bits order as integers).
__device__ __forceinline__ float wave_max_nonneg(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}

}  // namespace lsa
