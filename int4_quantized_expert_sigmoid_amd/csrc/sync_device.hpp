// sync_device.hpp — hand-offs between workgroups of one launch.
//
// A producer workgroup writes its results with device-coherent stores
// (st_dev), waits until they have completed, and adds 1 to a counter with a
// relaxed device-scope atomic; a consumer polls the counter with coherent
// loads and then reads the results with coherent loads (ld_dev). Nothing is
// cached in a way another XCD could miss, so no device-wide release or
// acquire fence (an L2 writeback or invalidate) is needed. Every wait is
// bounded: past SPIN_LIMIT polls it sets a sticky error word and goes on, so
// a launch always finishes.
#pragma once
#include "device_common.hpp"

namespace coli {

constexpr unsigned SPIN_LIMIT = 1u << 21;

__device__ __forceinline__ unsigned ld_counter(const unsigned *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 waits (bounded) until *p >= target; then the workgroup goes on.
__device__ inline void wait_ge(const unsigned *p, unsigned target, unsigned *err)
{
    if (threadIdx.x == 0) {
        unsigned spins = 0;
        while (ld_counter(p) < target) {
            if (++spins > SPIN_LIMIT) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// Lanes 0..n-1 of wave 0 each wait (bounded) for their own counter p[lane]
// to reach target[lane]; then the workgroup goes on.
__device__ inline void wait_all_ge(const unsigned *p, const unsigned *target, int n, unsigned *err)
{
    if (threadIdx.x < (unsigned)n) {
        unsigned spins = 0;
        const unsigned tgt = target[threadIdx.x];
        while (ld_counter(p + threadIdx.x) < tgt) {
            if (++spins > SPIN_LIMIT) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// After this workgroup's coherent stores have completed, add 1 to *p.
// Returns the old value to thread 0 (other threads get 0).
__device__ inline unsigned signal_add(unsigned *p)
{
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    unsigned old = 0;
    if (threadIdx.x == 0) old = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return old;
}

} // namespace coli
