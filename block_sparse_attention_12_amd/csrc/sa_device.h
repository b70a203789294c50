// Device-side helpers shared by the gfx950 kernels of libsparse_attn.
//
// Row layout used by every kernel: a row of d = 128 elements is read by 16
// consecutive lanes ("a row group"), each lane owning 8 consecutive channels
// (16 B of bf16 or 32 B of fp32). A 64-wide wavefront therefore covers 4 rows
// per load instruction, and dot products are finished by a reduction across
// the 16 lanes of a row group using DPP lane permutations (no LDS traffic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kD = 128;            // head dimension supported
constexpr int kRowLanes = 16;      // lanes per row
constexpr int kLaneElems = 8;      // channels per lane
constexpr int kBlock = 64;         // tokens per KV block
constexpr int kCmpKernel = 32;     // compression window
constexpr int kCmpStride = 16;     // compression stride

typedef uint16_t bf16_t;

__host__ __device__ __forceinline__ int64_t n_compressed(int64_t L) {
    return L < kCmpKernel ? 0 : (L - kCmpKernel) / kCmpStride + 1;
}
__host__ __device__ __forceinline__ int64_t n_blocks(int64_t L) {
    return (L + kBlock - 1) / kBlock;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---- 8-channel loads/stores of one lane's slice of a row -------------------

__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t *p, float (&x)[8]) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Raw (unconverted) register image of one lane's slice, so loads can be
// issued early and converted later.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { uint4 v; };
template <> struct Raw8<float> { float4 a, b; };

__device__ __forceinline__ void load_raw(const bf16_t *p, Raw8<bf16_t> &r) {
    r.v = *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void load_raw(const float *p, Raw8<float> &r) {
    r.a = reinterpret_cast<const float4 *>(p)[0];
    r.b = reinterpret_cast<const float4 *>(p)[1];
}
__device__ __forceinline__ void unpack(const Raw8<bf16_t> &r, float (&x)[8]) {
    x[0] = bf16_lo(r.v.x); x[1] = bf16_hi(r.v.x); x[2] = bf16_lo(r.v.y); x[3] = bf16_hi(r.v.y);
    x[4] = bf16_lo(r.v.z); x[5] = bf16_hi(r.v.z); x[6] = bf16_lo(r.v.w); x[7] = bf16_hi(r.v.w);
}
__device__ __forceinline__ void unpack(const Raw8<float> &r, float (&x)[8]) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(bf16_t *p, const float (&x)[8]) {
    uint4 v;
    v.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
    v.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
    v.z = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
    v.w = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
    *reinterpret_cast<uint4 *>(p) = v;
}

// ---- DPP lane permutations inside a 16-lane row ---------------------------

// DPP controls (GCN/CDNA encoding)
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each half row
constexpr int kDppRowRor4 = 0x124;       // rotate right by 4 within the row
constexpr int kDppRowRor8 = 0x128;       // rotate right by 8 within the row

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Partner selection for the four reduction steps over a row group. Step s
// pairs lanes that differ in bit (3 - s) of the lane's row position:
//   s = 0: mirror (i <-> 15-i), s = 1: half mirror (i <-> 7-i),
//   s = 2: xor 2, s = 3: xor 1.
template <int S>
__device__ __forceinline__ float partner(float v) {
    if constexpr (S == 0) return dpp<kDppRowMirror>(v);
    else if constexpr (S == 1) return dpp<kDppRowHalfMirror>(v);
    else if constexpr (S == 2) return dpp<kDppQuadXor2>(v);
    else return dpp<kDppQuadXor1>(v);
}

// Transposed sum over the 16 lanes of a row group of N partial values per
// lane (N a power of two). After the call v[0 .. max(N/16,1)) holds totals:
// for N >= 16 lane position i (= lane & 15) holds the totals of values
// [i*N/16, (i+1)*N/16); for N < 16 it holds value (i >> (4 - log2 N)).
// Each step halves the live values: the lane keeps the half selected by one
// bit of its position and receives the partner's copy of that half, so the
// whole reduction costs N-1 lane exchanges instead of 4N.
template <int S, int N, int LIVE>
__device__ __forceinline__ void transpose_reduce_step(float (&v)[N], int pos) {
    if constexpr (S < 4) {
        if constexpr (LIVE > 1) {
            constexpr int H = LIVE / 2;
            const bool upper = (pos >> (3 - S)) & 1;
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const float keep = upper ? v[k + H] : v[k];
                const float send = upper ? v[k] : v[k + H];
                v[k] = keep + partner<S>(send);
            }
            transpose_reduce_step<S + 1, N, H>(v, pos);
        } else {
            v[0] = v[0] + partner<S>(v[0]);
            transpose_reduce_step<S + 1, N, 1>(v, pos);
        }
    }
}

template <int N>
__device__ __forceinline__ void transpose_reduce16(float (&v)[N], int lane) {
    transpose_reduce_step<0, N, N>(v, lane & 15);
}

// ---- buffer loads: 32-bit offsets from an SGPR resource; reads at or past
// num_bytes return zeros (hardware range check), so tails need no branches.
typedef int sa_v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<bf16_t> &x) {
    const sa_v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    x.v = make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<float> &x) {
    const sa_v4i a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    const sa_v4i b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, 0);
    x.a = make_float4(__int_as_float(a.x), __int_as_float(a.y), __int_as_float(a.z), __int_as_float(a.w));
    x.b = make_float4(__int_as_float(b.x), __int_as_float(b.y), __int_as_float(b.z), __int_as_float(b.w));
}
// The same loads with the non-temporal (streaming) cache policy, for data a
// launch reads exactly once (gathered K/V rows, index keys, block statistics):
// it then does not displace cached data (measured: decode attention -4%,
// token index-key scan -9% time).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void load_raw_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<bf16_t> &x) {
    const sa_v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNT);
    x.v = make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ void load_raw_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<float> &x) {
    const sa_v4i a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNT);
    const sa_v4i b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, kCachePolicyNT);
    x.a = make_float4(__int_as_float(a.x), __int_as_float(a.y), __int_as_float(a.z), __int_as_float(a.w));
    x.b = make_float4(__int_as_float(b.x), __int_as_float(b.y), __int_as_float(b.z), __int_as_float(b.w));
}
// byte offset of a row, or an out-of-range offset (reads zeros) if it does not fit
__device__ __forceinline__ uint32_t row_offset(int64_t row, uint32_t row_bytes, uint32_t lane_off) {
    const int64_t o = row * (int64_t)row_bytes + lane_off;
    return (o < 0 || o > 0x7fffffffLL) ? 0xffffffffu : (uint32_t)o;
}

// bf16 pair dot product accumulated in fp32: a.lo*b.lo + a.hi*b.hi + c
// (v_dot2c_f32_bf16; bf16 products are exact in fp32).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Full-wave helpers (64 lanes)
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// A visible length clamped into [0, T_cap].
__device__ __forceinline__ int64_t clamp_len(int64_t L, int64_t T_cap) {
    return L < 0 ? 0 : (L > T_cap ? T_cap : L);
}

// e^x as 2^(x log2 e) on the hardware exp2 (v_exp_f32): a few ulp of
// relative error for the arguments here (x <= 0, softmax terms), against a
// longer libm-style sequence for expf.
__device__ __forceinline__ float hw_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896340736f);
}

// Merges a (max, sum of exp(x - max)) pair into another.
__device__ __forceinline__ void merge_ms(float &m, float &s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    s = s * expf(m - M) + s2 * expf(m2 - M);
    m = M;
}

// 32-bit key whose unsigned order is the order of the fp32 value (-0 and +0 tie).
__device__ __forceinline__ uint32_t orderable(float x) {
    if (x == 0.f) x = 0.f;                               // -0 and +0 tie
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- whole-wave scans on DPP (no LDS round trips) --------------------------
// Lane i takes lane i - n of its 16-lane row (row_shr:n), or lane 15 (31) of
// the previous row(s) (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows
// 2 and 3); a lane with no source, or in a row outside the row mask, keeps
// `ident`, the identity of the scan's operation.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t ident, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROW_MASK, 0xF, false);
}
// Inclusive scan over the 64 lanes with an associative operation `op` whose
// identity is `ident` (sum: 0, max: 0, min: ~0u): after six steps lane i
// holds op over lanes 0..i.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, uint32_t ident, Op op) {
    v = op(v, dpp_u32<kDppRowShr1>(ident, v));
    v = op(v, dpp_u32<kDppRowShr2>(ident, v));
    v = op(v, dpp_u32<kDppRowShr4>(ident, v));
    v = op(v, dpp_u32<kDppRowShr8>(ident, v));
    v = op(v, dpp_u32<kDppRowBcast15, 0xA>(ident, v));
    v = op(v, dpp_u32<kDppRowBcast31, 0xC>(ident, v));
    return v;
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    return wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// op over the whole wave, the same value on every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = wave_incl_scan(v, ~0u, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive prefix sum of one non-negative int per thread over the workgroup;
// also returns the total.
template <int NT>
__device__ __forceinline__ int wg_exclusive_scan(int x, int *s_wave, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int v = (int)wave_incl_sum((uint32_t)x);
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int sw = s_wave[w];
        if (w < wave) base += sw;
        total += sw;
    }
    __syncthreads();
    return base + v - x;
}

}  // namespace sa
