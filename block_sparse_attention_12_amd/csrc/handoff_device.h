// Hand-offs between workgroups of one launch without a cache-writeback fence.
//
// On this multi-die part each die's L2 is private, and a device-scope release
// fence writes back that L2 (measured: a per-workgroup fence serialised a
// 512-workgroup grid). Instead, data meant for another workgroup of the same
// launch is written with device-scope relaxed atomic stores, which write
// through to the device coherence point, and the writer waits for its own
// stores to complete before it signals; the reader uses device-scope relaxed
// atomic loads. Signals are 64-bit counter words in the caller's workspace,
// tagged with the call (tag << kTagShift | count): the tag is one more than
// an epoch word the previous call left, and each call stores its tag as the
// new epoch once no workgroup of it reads the epoch any more. A word carrying
// another tag (never written, or left by an interrupted call) counts as zero,
// so a workspace needs no clearing, and a captured graph replayed many times
// stays correct (the tag comes from device memory, not from a launch
// argument).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kTagShift = 20;                                // counter words: tag << 20 | count
constexpr uint64_t kTagMask = (1ull << (64 - kTagShift)) - 1;

__device__ __forceinline__ uint64_t load_dev(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until this thread's stores have completed (so they are visible at the
// device coherence point before a signal that follows).
__device__ __forceinline__ void wait_own_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The call's tag, from the epoch word the previous call left.
__device__ __forceinline__ uint64_t call_tag(const uint64_t *epoch) {
    return (load_dev(epoch) + 1) & kTagMask;
}

// Arrival at a tagged counter word: returns the number of arrivals of this
// call before this one. The word's last arrival of a call leaves it as (next
// tag, 0) (arm), so the next call's arrivals are one fetch-and-add each; a
// word carrying another tag is re-tagged by compare-and-swap (an arrival whose
// add landed on such a word counts itself again there).
__device__ __forceinline__ uint32_t arrive(uint64_t *w, uint64_t tag) {
    uint64_t old = __hip_atomic_fetch_add(w, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((old >> kTagShift) == tag) return (uint32_t)(old & ((1u << kTagShift) - 1));
    old = load_dev(w);
    for (;;) {
        const bool mine = (old >> kTagShift) == tag;
        const uint64_t next = mine ? old + 1 : ((tag << kTagShift) | 1u);
        if (__hip_atomic_compare_exchange_strong(w, &old, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return mine ? (uint32_t)(old & ((1u << kTagShift) - 1)) : 0u;
    }
}

// After the last arrival of this call: the word waits for the next call's tag.
__device__ __forceinline__ void arm(uint64_t *w, uint64_t tag) {
    store_dev(w, ((tag + 1) & kTagMask) << kTagShift);
}

}  // namespace sa
