// Row slices of the top-k passes: a unit is slice `slice` of row `row` of logits [R, V]; its
// whole 16-byte vectors and the elements of the row outside whole vectors (the ragged ends: the
// first slice takes the row's head, the last slice its tail).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash2 {

// Whole vectors of a unit and its ragged row ends (elements outside whole vectors: the first
// slice takes the head, the last slice the tail).
struct UnitRange {
    int64_t g0;      // first element of the row
    int64_t c0;      // first whole vector of the unit
    int nv;          // whole vectors of the unit
    int64_t h0, h1;  // ragged head [h0, h1)
    int64_t t0, t1;  // ragged tail [t0, t1)
};

// floor(n * s / S) for n < 2^31 and s <= S < 2^16, in 32-bit arithmetic (n = a S + b gives
// a s + floor(b s / S)); 64-bit divisions cost hundreds of scalar instructions.
__device__ __forceinline__ int64_t split_point(uint32_t n, uint32_t s, uint32_t S) {
    return (int64_t)(n / S) * s + (n % S) * s / S;
}

__device__ __forceinline__ UnitRange unit_range(int64_t unit, int V, int S, int EV) {
    UnitRange u;
    const uint32_t row = (uint32_t)unit / (uint32_t)S;  // units and slices fit in 31 bits
    const uint32_t slice = (uint32_t)unit - row * (uint32_t)S;
    u.g0 = (int64_t)row * V;
    const int64_t g1 = u.g0 + V;
    int64_t va = (u.g0 + EV - 1) / EV, vb = g1 / EV;
    if (va > vb) va = vb = 0;  // the row lies inside one vector: all of it is ragged
    const uint32_t nvec = (uint32_t)(vb - va);
    u.c0 = va + split_point(nvec, slice, (uint32_t)S);
    u.nv = (int)(va + split_point(nvec, slice + 1, (uint32_t)S) - u.c0);
    u.h0 = u.h1 = u.t0 = u.t1 = 0;
    if (slice == 0) {
        u.h0 = u.g0;
        u.h1 = nvec > 0 ? va * EV : g1;
    }
    if (slice == S - 1 && nvec > 0) {
        u.t0 = vb * EV;
        u.t1 = g1;
    }
    return u;
}

}  // namespace dflash2
