// Device helpers shared by the selector kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash2 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

// ---- lane exchanges in the VALU (no LDS round trip) ------------------------------------------
// Lane l receives lane l ^ S. Within a row of 16 lanes: DPP quad permutations (S = 1, 2), the row
// rotations by 12 and 4 (row_ror:n reads lane (l - n) mod 16; S = 4 takes l + 4 or l - 4 by lane
// bit 2) and by 8 (S = 8). Across rows, gfx950's permlane swaps on two copies of the value:
// permlane16_swap(v, v) returns the even rows of v in both rows of each pair, then the odd rows;
// permlane32_swap(v, v) the low half of the wave in both halves, then the high half.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor12 = 0x12C;
constexpr int kDppRowMirror = 0x140;  // lane l reads lane 15 - l of its row

// (Every lane's source exists for these patterns, so the moves take no old value: with one,
// the compiler first clears the destination, an extra instruction per move.)
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "lane xor");
    if constexpr (S == 1)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, true);
    if constexpr (S == 2)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, true);
    if constexpr (S == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor12, 0xF, 0xF, true);
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor4, 0xF, 0xF, true);
        return (lane & 4) ? dn : up;
    }
    if constexpr (S == 8)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor8, 0xF, 0xF, true);
    if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    }
    if constexpr (S == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

template <int S>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int lane) {
    const uint32_t lo = xor_lane<S>((uint32_t)v, lane);
    const uint32_t hi = xor_lane<S>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Lane l receives lane 63 - l: the row mirror (l ^ 15 within a row), then l ^ 16 and l ^ 32.
__device__ __forceinline__ uint64_t reverse_lanes64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, kDppRowMirror, 0xF, 0xF, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kDppRowMirror, 0xF, 0xF, true);
    return xor_lane64<32>(xor_lane64<16>(((uint64_t)hi << 32) | lo, lane), lane);
}

// ---- wave-wide sorting networks on 64-bit keys (one key per lane, lane 0 = largest) --------

__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t kmin(uint64_t a, uint64_t b) { return a < b ? a : b; }

// One compare-exchange step with the partner l ^ S: the lower lane of the pair keeps the
// larger key when `desc`, the smaller otherwise (one compare decides which of the two it keeps;
// equal keys are the same either way).
template <int S>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t key, int lane, bool desc) {
    const uint64_t other = xor_lane64<S>(key, lane);
    const bool keep_max = ((lane & S) == 0) == desc;
    return ((key > other) == keep_max) ? key : other;
}

// Compare-exchange steps with the partners l ^ S, l ^ S/2, ..., l ^ 1 (one bitonic merge).
template <int S>
__device__ __forceinline__ uint64_t bitonic_merge_steps(uint64_t key, int lane, bool desc) {
    key = bitonic_step<S>(key, lane, desc);
    if constexpr (S > 1) key = bitonic_merge_steps<S / 2>(key, lane, desc);
    return key;
}

// Bitonic sort of the 64 lane keys into descending lane order.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key, int lane) {
    key = bitonic_merge_steps<1>(key, lane, (lane & 2) == 0);
    key = bitonic_merge_steps<2>(key, lane, (lane & 4) == 0);
    key = bitonic_merge_steps<4>(key, lane, (lane & 8) == 0);
    key = bitonic_merge_steps<8>(key, lane, (lane & 16) == 0);
    key = bitonic_merge_steps<16>(key, lane, (lane & 32) == 0);
    key = bitonic_merge_steps<32>(key, lane, true);
    return key;
}

// a and c are each sorted descending across the lanes; returns the 64 largest keys of both,
// sorted descending (bitonic merge).
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t a, uint64_t c, int lane) {
    const uint64_t m = kmax(a, reverse_lanes64(c, lane));
    return bitonic_merge_steps<32>(m, lane, true);
}

// ---- cross-lane reductions (DPP: no LDS round trip) -----------------------------------------

constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

// Sum over each row of 16 lanes, in every lane of the row (rotations: each lane adds the same
// values in a different order; every partial is a sum of distinct lanes).
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppRor8, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppRor4, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppXor2, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppXor1, 0xF, 0xF, true));
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
