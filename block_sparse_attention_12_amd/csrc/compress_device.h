// Compressed-key entries (Eq. 2 of the SparDA summary page, "Theoretical
// Foundation": mean pooling with kernel 32, stride 16), per lane of a 16-lane
// row group: entry j = (P_j + P_{j+1}) * 2^-5 rounded to the key dtype, P_m the
// fp32 sum of keys 16m .. 16m+15 in token order. Only additions and one exact
// scaling by a power of two: no operation here can be contracted, so every
// kernel that includes this computes the same bits.
#pragma once

#include "sa_device.h"

namespace sa {

template <typename T>
__device__ __forceinline__ void half_window_sum(const T *__restrict__ p, float (&acc)[8]) {
    Raw8<T> r[kCmpStride];
#pragma unroll
    for (int t = 0; t < kCmpStride; ++t) load_raw(p + (int64_t)t * kD, r[t]);
    unpack(r[0], acc);
#pragma unroll
    for (int t = 1; t < kCmpStride; ++t) {
        float x[8];
        unpack(r[t], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
    }
}

// Entries [j0, min(j0 + run, j_end)) of one unit's compressed keys for this
// lane's 8 channels: Ku / Kcu point at the unit's keys / entries, offset by the
// lane's channels. Consecutive entries share a half-window, carried in registers.
template <typename T, int RUN>
__device__ __forceinline__ void compress_run(const T *__restrict__ Ku, T *__restrict__ Kcu, int64_t j0,
                                             int64_t j_end) {
    float prev[8];
    half_window_sum(Ku + j0 * kCmpStride * kD, prev);
#pragma unroll
    for (int r = 0; r < RUN; ++r) {
        const int64_t j = j0 + r;
        if (j >= j_end) break;
        float next[8];
        half_window_sum(Ku + (j + 1) * kCmpStride * kD, next);
        float e[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) e[c] = (prev[c] + next[c]) * 0.03125f;
        store8(Kcu + j * kD, e);
#pragma unroll
        for (int c = 0; c < 8; ++c) prev[c] = next[c];
    }
}

// half_window_sum with few keys in flight (for rare paths inside kernels
// whose registers are needed elsewhere); same order, same bits.
template <typename T>
__device__ __forceinline__ void half_window_sum_lean(const T *__restrict__ p, float (&acc)[8]) {
    Raw8<T> r0;
    load_raw(p, r0);
    unpack(r0, acc);
#pragma unroll 3
    for (int t = 1; t < kCmpStride; ++t) {
        Raw8<T> r;
        load_raw(p + (int64_t)t * kD, r);
        float x[8];
        unpack(r, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
    }
}

// One entry j for this lane's 8 channels, rounded to the key dtype and
// returned in the raw register form a load of the stored entry would give.
__device__ __forceinline__ void compress_entry_raw(const bf16_t *__restrict__ Ku, int64_t j,
                                                   Raw8<bf16_t> &out) {
    float a[8], b[8], e[8];
    half_window_sum_lean(Ku + j * kCmpStride * kD, a);
    half_window_sum_lean(Ku + (j + 1) * kCmpStride * kD, b);
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] = (a[c] + b[c]) * 0.03125f;
    out.v.x = f32_to_bf16_bits(e[0]) | (f32_to_bf16_bits(e[1]) << 16);
    out.v.y = f32_to_bf16_bits(e[2]) | (f32_to_bf16_bits(e[3]) << 16);
    out.v.z = f32_to_bf16_bits(e[4]) | (f32_to_bf16_bits(e[5]) << 16);
    out.v.w = f32_to_bf16_bits(e[6]) | (f32_to_bf16_bits(e[7]) << 16);
}
__device__ __forceinline__ void compress_entry_raw(const float *__restrict__ Ku, int64_t j,
                                                   Raw8<float> &out) {
    float a[8], b[8];
    half_window_sum_lean(Ku + j * kCmpStride * kD, a);
    half_window_sum_lean(Ku + (j + 1) * kCmpStride * kD, b);
    out.a = make_float4((a[0] + b[0]) * 0.03125f, (a[1] + b[1]) * 0.03125f,
                        (a[2] + b[2]) * 0.03125f, (a[3] + b[3]) * 0.03125f);
    out.b = make_float4((a[4] + b[4]) * 0.03125f, (a[5] + b[5]) * 0.03125f,
                        (a[6] + b[6]) * 0.03125f, (a[7] + b[7]) * 0.03125f);
}

// Entry from its 32 keys staged in LDS (rows[t][l] = lane l's 8 channels of
// key 16j + t, bf16): the same sums in the same order as compress_entry_raw.
__device__ __forceinline__ void entry_from_rows(const uint4 (*rows)[16], int lane16,
                                                Raw8<bf16_t> &out) {
    float a[8], b[8], e[8];
    unpack(Raw8<bf16_t>{rows[0][lane16]}, a);
    unpack(Raw8<bf16_t>{rows[kCmpStride][lane16]}, b);
#pragma unroll 1
    for (int t = 1; t < kCmpStride; ++t) {     // not unrolled: few rows live at once
        float x[8], y[8];
        unpack(Raw8<bf16_t>{rows[t][lane16]}, x);
        unpack(Raw8<bf16_t>{rows[kCmpStride + t][lane16]}, y);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            a[c] = a[c] + x[c];
            b[c] = b[c] + y[c];
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] = (a[c] + b[c]) * 0.03125f;
    out.v.x = f32_to_bf16_bits(e[0]) | (f32_to_bf16_bits(e[1]) << 16);
    out.v.y = f32_to_bf16_bits(e[2]) | (f32_to_bf16_bits(e[3]) << 16);
    out.v.z = f32_to_bf16_bits(e[4]) | (f32_to_bf16_bits(e[5]) << 16);
    out.v.w = f32_to_bf16_bits(e[6]) | (f32_to_bf16_bits(e[7]) << 16);
}

__device__ __forceinline__ void store_raw(bf16_t *p, const Raw8<bf16_t> &r) {
    *reinterpret_cast<uint4 *>(p) = r.v;
}
__device__ __forceinline__ void store_raw(float *p, const Raw8<float> &r) {
    reinterpret_cast<float4 *>(p)[0] = r.a;
    reinterpret_cast<float4 *>(p)[1] = r.b;
}

}  // namespace sa
