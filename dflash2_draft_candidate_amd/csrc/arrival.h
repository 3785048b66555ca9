// Arrival counters of one launch in workspace memory: a 64-bit word holds the launch's epoch
// above a count. Workgroups that each finish a part of a job (the slices of a row) count
// themselves in; the arrival that completes the count takes the job's last step. Nothing waits on
// another workgroup.
//
// Epochs grow from launch to launch (next_launch_epoch), so an atomic max of (epoch, 0) re-bases a
// counter left by an earlier launch and leaves one of this launch alone; a replay of a captured
// launch keeps its epoch, and the completing arrival clears the count for it. All accesses are
// device-scope atomics: the XCDs' L2 caches are not coherent with each other.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash2 {

// Re-base to (epoch, 0) unless the counter already holds this launch's epoch (not waited for).
__device__ __forceinline__ void arrival_rebase(uint64_t *ctr, uint32_t epoch) {
    __hip_atomic_fetch_max(ctr, (uint64_t)epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One arrival (a single lane calls it); true for the arrival that makes the count `target`. The
// caller's results must be complete in memory first (device-scope stores, then a wait for them).
// An arrival that still finds another launch's epoch (a counter holding a larger one, never set,
// or wrapped) re-bases it to (epoch, 0) unless another arrival has, then adds again: the adds
// made to stale values are dropped with them, and every arrival that made one repeats it.
__device__ __forceinline__ bool arrive(uint64_t *ctr, uint32_t epoch, uint32_t target) {
    uint64_t old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old >> 32) != epoch) {
        uint64_t cur = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while ((uint32_t)(cur >> 32) != epoch) {
            __hip_atomic_compare_exchange_strong(ctr, &cur, (uint64_t)epoch << 32, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // success or failure, cur now holds a value of this launch or a stale one changed
            // by another arrival
            if ((uint32_t)(cur >> 32) != epoch)
                cur = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return (uint32_t)old + 1u == target;
}

// After the completing arrival: (epoch, 0), so that a replay of the same launch starts from zero.
__device__ __forceinline__ void arrival_clear(uint64_t *ctr, uint32_t epoch) {
    __hip_atomic_store(ctr, (uint64_t)epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order this wave's earlier stores before a following arrival: wait until they have completed.
// (The signal fences keep the compiler from moving memory accesses across the wait; they emit
// nothing. A device-scope release fence would write back the whole L2 of the XCD.)
__device__ __forceinline__ void stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0), expcnt(0), lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace dflash2
