// Count and position arithmetic of the token-level top-k chain (the radix
// select over 32-bit orderable keys and the ascending compaction into an
// index row of idx_cap slots). Host and device code: the kernels call these
// functions, and a host program drives them with inconsistent histograms and
// chunk counts to show that no slot outside [0, idx_cap) is ever addressed and
// no signed arithmetic overflows.
//
// Counts come from other workgroups (global histograms, per-chunk counts), so
// they are treated as untrusted: every difference and sum is formed in 64
// bits and clamped before it addresses the row.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

namespace sa {

// The bin of a 256-bin histogram (scanned from the top bin down) that holds
// the `remaining`-th largest counted key: above = keys in the bins above it,
// bcnt = its own count. If no bin qualifies (counts that do not add up), the
// result is digit 0, above 0 and bcnt = 0xffffffff, which can never equal a
// remaining count, so the search goes on to the next digit. Sequential
// statement; the device searches the same bins with a wave-wide prefix sum
// and picks the same bin (tok_bin_holds decides for both).
struct TokDigit {
    uint32_t digit, above, bcnt;
};

__host__ __device__ inline bool tok_bin_holds(uint64_t above, uint32_t count, int remaining) {
    return remaining > 0 && above < (uint64_t)remaining && above + count >= (uint64_t)remaining;
}

__host__ __device__ inline TokDigit tok_digit_seq(const uint32_t *hist, int remaining) {
    TokDigit d{0u, 0u, 0xffffffffu};
    uint64_t above = 0;
    for (int bin = 255; bin >= 0; --bin) {
        if (tok_bin_holds(above, hist[bin], remaining)) {
            d.digit = (uint32_t)bin;
            d.above = (uint32_t)above;
            d.bcnt = hist[bin];
            return d;
        }
        above += hist[bin];
    }
    return d;
}

// Keys still to take below the chosen digit: remaining - above, never below 0.
__host__ __device__ inline int tok_remaining_after(int remaining, uint32_t above) {
    const int64_t r = (int64_t)remaining - (int64_t)above;
    return r < 0 ? 0 : (int)r;
}

// Number of keys equal to the k-th key that are taken, as stored by the count
// kernel (an unsigned word): never negative.
__host__ __device__ inline int tok_take_eq(uint32_t stored) {
    return stored > 0x7fffffffu ? 0 : (int)stored;
}

// Entries of the row: surely taken + equal keys taken, within [0, idx_cap].
__host__ __device__ inline int tok_row_total(int64_t sure, int64_t eq, int take_eq, int idx_cap) {
    const int64_t t = sure + (eq < take_eq ? eq : (int64_t)take_eq);
    return t < 0 ? 0 : (t < idx_cap ? (int)t : idx_cap);
}

// Slot of a thread's first taken token: tokens of earlier chunks (sure ones and
// equal ones up to take_eq) plus those of earlier threads of the chunk.
__host__ __device__ inline int64_t tok_first_pos(int64_t sure_before, int64_t eq_before, int take_eq,
                                                  int scan) {
    const int64_t eq_taken = eq_before < 0 ? 0 : (eq_before < take_eq ? eq_before : (int64_t)take_eq);
    return sure_before + eq_taken + (int64_t)scan;
}

__host__ __device__ inline bool tok_slot_ok(int64_t pos, int idx_cap) {
    return pos >= 0 && pos < (int64_t)idx_cap;
}

}  // namespace sa
