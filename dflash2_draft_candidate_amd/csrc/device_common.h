// Device helpers shared by the selector kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash2 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLn2 = 0.693147180559945309417232121458;

// ---- bf16 / fp32 element access ------------------------------------------------------------

// Two bf16 values packed in one 32-bit word (element 2w in the low half): exact widening.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerVec = 4;  // elements per 16-byte vector
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    // element i of vectors staged in LDS
    static __device__ __forceinline__ float lds_element(const u32x4 *v, int i) {
        return reinterpret_cast<const float *>(v)[i];
    }
    // a vector whose element 0 is x
    static __device__ __forceinline__ u32x4 single(float x) { return u32x4{__float_as_uint(x), 0u, 0u, 0u}; }
    static __device__ __forceinline__ void unpack(const u32x4 &v, float *x) {
        x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
    }
};
template <> struct Elem<uint16_t> {
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ float load(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ float lds_element(const u32x4 *v, int i) {
        return bf16_to_f32(reinterpret_cast<const uint16_t *>(v)[i]);
    }
    // x came from a bf16 value, so its upper half is exact
    static __device__ __forceinline__ u32x4 single(float x) { return u32x4{__float_as_uint(x) >> 16, 0u, 0u, 0u}; }
    static __device__ __forceinline__ void unpack(const u32x4 &v, float *x) {
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    }
};

// ---- candidate keys -----------------------------------------------------------------------
// The candidate order (higher logit first, equal logits by lower id, +0 == -0) as one unsigned
// 64-bit key: larger key = earlier candidate. High half: an order-preserving map of the logit's
// bits with -0 folded onto +0; low half: the id inverted. Key 0 never occurs for a finite logit
// and marks an empty slot.

__device__ __forceinline__ uint32_t value_key(float x) {
    uint32_t u = __float_as_uint(x);
    u = ((u << 1) == 0u) ? 0u : u;  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t vk) {
    return __uint_as_float((vk & 0x80000000u) ? (vk & 0x7FFFFFFFu) : ~vk);
}

__device__ __forceinline__ uint64_t cand_key(float x, int32_t id) {
    return ((uint64_t)value_key(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ int32_t key_id(uint64_t key) {
    return (int32_t)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ __forceinline__ float key_logit(uint64_t key) { return key_value((uint32_t)(key >> 32)); }

// ---- wave-wide sorting networks on 64-bit keys (one key per lane, lane 0 = largest) --------

__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t kmin(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Bitonic sort of the 64 lane keys into descending lane order.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key, int lane) {
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t other = __shfl_xor(key, stride, kWave);
            const bool desc = (lane & size) == 0;
            const bool lower = (lane & stride) == 0;
            key = (lower == desc) ? kmax(key, other) : kmin(key, other);
        }
    }
    return key;
}

// a and c are each sorted descending across the lanes; returns the 64 largest keys of both,
// sorted descending (bitonic merge).
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t a, uint64_t c, int lane) {
    const uint64_t c_rev = __shfl(c, kWave - 1 - lane, kWave);
    uint64_t m = kmax(a, c_rev);
#pragma unroll
    for (int stride = kWave / 2; stride > 0; stride >>= 1) {
        const uint64_t other = __shfl_xor(m, stride, kWave);
        m = ((lane & stride) == 0) ? kmax(m, other) : kmin(m, other);
    }
    return m;
}

// ---- cross-lane reductions (DPP: no LDS round trip) -----------------------------------------

constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

// Sum over each row of 16 lanes, in every lane of the row (rotations: each lane adds the same
// values in a different order; every partial is a sum of distinct lanes).
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRor8, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRor4, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppXor2, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppXor1, 0xF, 0xF, false));
    return v;
}

// Sum over the wave, wave-uniform: the four row sums (taken from the rows' first lanes) added in
// row order, so the result depends only on the lane values.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

// ---- logsumexp partial state ---------------------------------------------------------------
// (ref, sum) stands for log2-domain reference `ref` and sum = sum_i 2^(x_i*log2e - ref):
// logsumexp = (ref + log2(sum)) * ln 2. ref = -inf with sum = 0 is the empty state.

__device__ __forceinline__ void lse_combine(float &ref, float &sum, float oref, float osum) {
    const float r = fmaxf(ref, oref);
    if (r == -INFINITY) return;
    const float a = (ref == r) ? sum : sum * exp2f(ref - r);
    const float b = (oref == r) ? osum : osum * exp2f(oref - r);
    ref = r;
    sum = a + b;
}

__device__ __forceinline__ double lse_value(float ref, float sum) {
    return ((double)ref + log2((double)sum)) * kLn2;
}

}  // namespace dflash2
