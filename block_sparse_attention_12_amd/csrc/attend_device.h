// Gathered sparse decode attention over one share of a (sequence, KV head)
// unit's selected blocks (Eq. 5 of the SparDA summary page, "Methodology":
// the attention query attends only to the keys and values of the selected
// blocks). Device code of the decode kernel (one share per workgroup).
//
// A workgroup of NW = 4 (the decode kernel) or 8 waves. Wave w owns rows 16 (w % 4) .. + 15 of
// every block it processes; the waves form NW / 4 wave sets that take the
// share's blocks in turn (set s: blocks s, s + NW/4, ...), so an 8-wave
// workgroup has twice the bytes in flight of a 4-wave one. Inside a wave, row
// group r = lane / 16 takes rows 16 (w % 4) + 4i + r (i = 0..3) and each lane
// owns 8 channels. A block costs each lane 4 K and 4 V loads of 16 B. Loads
// of a wave's next two blocks are in flight while a block is computed (three
// register buffers); block ids are uniform scalar loads, and the loads of an
// absent block use an out-of-range offset, so every wait in the loop is for
// data already in flight.
//
// The G query heads of the group (G = 1, 2, 4 or 8) are served from that
// single read (GQA packing). Logits for 4 rows x G heads are reduced across
// the 16 lanes of a row by the DPP transposed reduction: lane position p
// (lane & 15) ends with the logits of row p / 4 and, for G >= 4, of heads
// (p & 3) * G/4 .. + G/4 - 1; for G < 4 the 4G totals are replicated over
// 4/G lanes each (bf16 inputs use the packed bf16 dot product for q.k). The
// online softmax keeps a running max per head (wave-uniform) and per-lane
// partial sums, so no workgroup barrier is needed inside the block loop;
// probabilities reach the lanes holding the matching V rows through a
// wave-private LDS slot. Logits are in base-2 units (scaled by scale * log2 e)
// so each exponential is one exp2. At the end the waves' (max, sum, weighted
// values) meet in LDS.
//
// bf16 inputs (block and token lists) take attend_share_mfma instead: the
// same loads and block ring, with q.k and P.V on the matrix cores (4 + 8 MFMA
// per wave and block) and the softmax on one head's 4 logits per lane, about a
// fifth of the vector instructions of the path above. That path still serves
// fp32 inputs.
#pragma once

#include <math.h>

#include "handoff_device.h"
#include "sa_device.h"

namespace sa {

constexpr int kPartStride = kD + 4;          // acc[128], max, sum, 2 pad (16 B aligned rows)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// q for this lane's 8 channels of the group's G heads: packed bf16 pairs (bf16
// inputs, used with dot2) or fp32 values (fp32 inputs).
template <typename T, int G> struct QFrag;
template <int G> struct QFrag<bf16_t, G> { uint32_t w[G][4]; };
template <int G> struct QFrag<float, G> { float w[G][8]; };

template <int G>
__device__ __forceinline__ void load_q(const bf16_t *p, QFrag<bf16_t, G> &q) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p + (int64_t)g * kD);
        q.w[g][0] = v.x; q.w[g][1] = v.y; q.w[g][2] = v.z; q.w[g][3] = v.w;
    }
}
template <int G>
__device__ __forceinline__ void load_q(const float *p, QFrag<float, G> &q) {
#pragma unroll
    for (int g = 0; g < G; ++g) load8(p + (int64_t)g * kD, q.w[g]);
}
template <int G>
__device__ __forceinline__ float qk(const QFrag<bf16_t, G> &q, int g, const Raw8<bf16_t> &k) {
    float a = dot2_bf16(q.w[g][0], k.v.x, 0.f);
    a = dot2_bf16(q.w[g][1], k.v.y, a);
    a = dot2_bf16(q.w[g][2], k.v.z, a);
    return dot2_bf16(q.w[g][3], k.v.w, a);
}
template <int G>
__device__ __forceinline__ float qk(const QFrag<float, G> &q, int g, const Raw8<float> &k) {
    float x[8];
    unpack(k, x);
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a = fmaf(q.w[g][c], x[c], a);
    return a;
}

// bf16 block lists run both products on the matrix cores (attend_share_mfma).
typedef __attribute__((ext_vector_type(8))) __bf16 mf_bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short mf_s16x4_t;
typedef __attribute__((ext_vector_type(4))) float mf_f32x4_t;
typedef __attribute__((ext_vector_type(2))) float mf_f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 mf_bf16x2_t;

// q of the group as the B operand of S = K q^T on v_mfma_f32_16x16x32_bf16
// (four steps of 32 channels): lane l holds head l % 16 (zeros from G on),
// channels 32 s + 8 (l / 16) .. +7 of step s.
struct QMfma { uint4 w[4]; };
template <int G>
__device__ __forceinline__ void load_q_mfma(const bf16_t *group, int lane, QMfma &q) {
    const int h = lane & 15, c = 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        q.w[s] = h < G ? *reinterpret_cast<const uint4 *>(group + (int64_t)h * kD + 32 * s + c)
                       : make_uint4(0u, 0u, 0u, 0u);
}

// x combined with the lane 16 (32) apart, on v_permlane16_swap (32_swap):
// with both operands x, each lane's two results are x of the lane pair.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Where the reduced logits of a group of G heads live: NV logits per lane;
// for G < 4 each total sits on REP = 4/G lanes.
template <int G> struct HeadLayout {
    static constexpr int NV = G >= 4 ? G / 4 : 1;             // logits per lane
    static constexpr int REP = G >= 4 ? 1 : 4 / G;             // lanes per logit
    // head of a lane's e-th logit (p = lane & 15)
    __device__ static int head(int p, int e) { return G >= 4 ? (p & 3) * NV + e : (p / REP) % G; }
    // a lane (0..3) holding head g's logit, and its slot e
    __device__ static constexpr int lane_of(int g) { return G >= 4 ? g / NV : g * REP; }
    __device__ static constexpr int slot_of(int g) { return G >= 4 ? g % NV : 0; }
};

template <typename T>
struct BlockRegs {
    Raw8<T> k[4], v[4];
    int64_t t0;
    int ids[4];     // token lists: ids of this lane's 4 rows of the next tile this buffer loads
    int tmy;        // token lists: id of the row whose logit this lane holds (loaded tile);
                    // matrix-core share: visibility bits of the lane's 4 logits
    int idk;        // token lists, matrix-core share: id of the lane's K row of the next tile
};

// LDS of attend_share for G heads and NW waves.
template <int G, int NW> struct AttendSmem {
    static constexpr int NVAL = 4 * G;
    static constexpr int SP = NVAL > 16 ? NVAL : 16;
    __align__(16) float p[NW][4 * SP];
    float m[NW][G], l[NW][G];
    __align__(16) float acc[NW][G][kD];
};

// Where a share's result goes. Direct: O (and lse) of the G head rows.
// Partial: the (weighted values, max, sum) row of split `split` of each head
// row, part + (row * n_split + split) * kPartStride; COHERENT partial rows are
// written with device-scope stores (visible to other workgroups of the same
// launch once the writer has waited for them).
enum AttendMode { kAttendDirect = 0, kAttendPartial = 1, kAttendPartialCoherent = 2 };
struct AttendOut {
    float *part;
    int n_split, split;
    void *O;
    int out_bf16;
    float *lse;
};

// The waves' (max, sum, weighted values) in sm -> the share's result for the
// G head rows from row_base (O and LSE, or a partial row). Starts and ends
// with a workgroup barrier.
template <int G, int NW, int MODE>
__device__ __forceinline__ void merge_waves(AttendSmem<G, NW> &sm, int64_t row_base,
                                            const AttendOut &out) {
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x;
    __syncthreads();
    // thread -> (head g, channels 2c, 2c+1)
    for (int pair = tid; pair < G * (kD / 2); pair += NT) {
        const int g = pair / (kD / 2);
        const int c2 = (pair % (kD / 2)) * 2;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][g]);
        float lsum = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = sm.m[w][g];
            const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            lsum = fmaf(wt, sm.l[w][g], lsum);
            a0 = fmaf(wt, sm.acc[w][g][c2], a0);
            a1 = fmaf(wt, sm.acc[w][g][c2 + 1], a1);
        }
        const int64_t row = row_base + g;                    // query head row
        if constexpr (MODE != kAttendDirect) {
            float *dst = out.part + (row * out.n_split + out.split) * kPartStride;
            if constexpr (MODE == kAttendPartialCoherent) {
                store_dev(dst + c2, a0);
                store_dev(dst + c2 + 1, a1);
                if (c2 == 0) {
                    store_dev(dst + kD, M);
                    store_dev(dst + kD + 1, lsum);
                }
            } else {
                reinterpret_cast<float2 *>(dst)[c2 / 2] = make_float2(a0, a1);
                if (c2 == 0) {
                    dst[kD] = M;
                    dst[kD + 1] = lsum;
                }
            }
            continue;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if (out.out_bf16) {
            const uint32_t w = f32_to_bf16_bits(a0 * inv) | (f32_to_bf16_bits(a1 * inv) << 16);
            reinterpret_cast<uint32_t *>(out.O)[(row * kD + c2) / 2] = w;
        } else {
            reinterpret_cast<float2 *>(out.O)[(row * kD + c2) / 2] = make_float2(a0 * inv, a1 * inv);
        }
        if (out.lse && c2 == 0) out.lse[row] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
    }
    __syncthreads();                             // sm may be reused by the caller
}

// One share of a unit: items [e_lo, e_lo + nblk) of the list (ROWS = false:
// block ids, irow already at entry e_lo; ROWS = true: 64-entry tiles of token
// ids, irow at the list start, n entries). L is the unit's visible length,
// row_base the first query-head row of the group (b * Hq + kvh * G). Ends
// with a workgroup barrier; sm is free again afterwards.
template <typename T, int G, bool ROWS, int NW, int MODE>
__device__ __forceinline__ void attend_share(const QFrag<T, G> &q, const T *__restrict__ K,
                                             const T *__restrict__ V, int64_t T_cap, int unit,
                                             int64_t L, const int32_t *irow, int n, int e_lo,
                                             int nblk, float qscale, int64_t row_base,
                                             const AttendOut &out, AttendSmem<G, NW> &sm) {
    using HL = HeadLayout<G>;
    constexpr int NV = HL::NV;
    constexpr int NVAL = 4 * G;                  // logits per row group per block (4 rows x G heads)
    constexpr int NWS = NW / 4;                  // wave sets
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wq = wave & 3, wset = wave >> 2;
    const int lane16 = lane & 15, rgrp = lane >> 4;

    float acc[G][8];
    float m_my[NV], l_lane[NV];                  // this lane's heads: running max, partial sum
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        m_my[e] = -INFINITY;
        l_lane[e] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
    // per-unit K/V windows of L rows: rows at or past L read as zeros
    constexpr uint32_t kRowBytes = kD * sizeof(T);
    const uint32_t lane_off = lane16 * kLaneElems * sizeof(T);
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + (int64_t)unit * T_cap * kD, (uint32_t)(L * kRowBytes));
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + (int64_t)unit * T_cap * kD, (uint32_t)(L * kRowBytes));
    const int my_row = 16 * wq + 4 * (lane16 >> 2) + rgrp;     // row of the logits this lane holds
    const int row0 = 16 * wq + rgrp;                           // first row this lane loads
    const uint32_t row_lane_off = row0 * kRowBytes + lane_off;
    const int64_t nb = n_blocks(L);

    // item of this wave set's k-th iteration
    auto item_of = [&](int k) { return wset + k * NWS; };
    // The share's block ids, read once: lane i holds item i's id (a share never
    // has more than 64 items: every split takes at most 64 list entries), so
    // the loop takes ids with v_readlane and no load of an id waits, in order,
    // behind the K/V loads in flight. -1 (no rows) past the share or out of range.
    int id_lane = -1;
    if constexpr (!ROWS) {
        if (lane < nblk) {
            const int blk = irow[lane];
            id_lane = (blk >= 0 && blk < nb) ? blk : -1;
        }
    }
    auto block_id = [&](int it) -> int {
        return it < nblk ? __builtin_amdgcn_readlane(id_lane, it & 63) : -1;
    };
    // Issues the block's K/V loads unconditionally: id -1 maps every row to an
    // out-of-range offset, which reads zeros and moves no bytes, so the wait
    // counts stay exact.
    auto issue = [&](BlockRegs<T> &r, int blk) {
        r.t0 = (int64_t)blk * kBlock;
        const uint32_t base = blk < 0 ? 0xffffffffu : (uint32_t)blk * (kBlock * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = blk < 0 ? 0xffffffffu : base + row_lane_off + i * (4 * kRowBytes);
            load_raw_nt(rK, off, r.k[i]);
            load_raw_nt(rV, off, r.v[i]);
        }
    };
    // token lists: ids of this lane's rows (entries 64*tile + row0 + 4i) of
    // share tile it, or -1 past the share or the list
    auto load_ids = [&](int (&ids)[4], int it) {
        const int e0 = 64 * (e_lo + it) + row0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + 4 * i;
            ids[i] = (it < nblk && e < n) ? irow[e] : -1;
        }
    };
    // token lists: rows from the ids loaded for tile it (ids outside [0, L)
    // read zeros and are masked), then the ids of the wave set's tile three
    // iterations later
    auto issue_rows = [&](BlockRegs<T> &r, int it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = r.ids[i];
            const uint32_t off = (id >= 0 && id < L) ? (uint32_t)id * kRowBytes + lane_off : 0xffffffffu;
            load_raw_nt(rK, off, r.k[i]);
            load_raw_nt(rV, off, r.v[i]);
        }
        const int a = lane16 >> 2;                  // the logits this lane holds are of row i = a
        r.tmy = a == 0 ? r.ids[0] : (a == 1 ? r.ids[1] : (a == 2 ? r.ids[2] : r.ids[3]));
        load_ids(r.ids, it + 3 * NWS);
    };
    auto process = [&](const BlockRegs<T> &r) {
        float v[NVAL];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g) v[i * G + g] = qk<G>(q, g, r.k[i]);
        transpose_reduce16<NVAL>(v, lane);
        const int64_t my_t = ROWS ? (int64_t)r.tmy : r.t0 + my_row;
        const bool vis = my_t >= 0 && my_t < L;
        float p[NV], alpha_me[NV];
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            const float x = vis ? v[e] * qscale : -INFINITY;
            // block max per head over the wave (lanes sharing lane & 3 hold the same heads)
            float mx = fmaxf(x, dpp<kDppRowRor4>(x));
            mx = fmaxf(mx, dpp<kDppRowRor8>(mx));
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float m_new = fmaxf(m_my[e], mx);
            alpha_me[e] = (m_my[e] == -INFINITY) ? 0.f : exp2f(m_my[e] - m_new);
            m_my[e] = m_new;
            p[e] = (x == -INFINITY) ? 0.f : exp2f(x - m_new);
            l_lane[e] = l_lane[e] * alpha_me[e] + p[e];
        }
        // every head's rescale factor, broadcast from a lane that holds it
        float alpha[G];
#pragma unroll
        for (int g = 0; g < G; ++g)
            alpha[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, alpha_me[HL::slot_of(g)]),
                                                     HL::lane_of(g)));
        // probabilities of the row group's 4 rows x G heads, in value order
        if constexpr (G >= 4) {
#pragma unroll
            for (int e = 0; e < NV; ++e) sm.p[wave][lane * NV + e] = p[e];
        } else {
            sm.p[wave][lane] = p[0];
        }
        __builtin_amdgcn_wave_barrier();
        float pr[NVAL];
        if constexpr (G >= 4) {
            const float4 *src = reinterpret_cast<const float4 *>(&sm.p[wave][rgrp * NVAL]);
#pragma unroll
            for (int k = 0; k < NVAL / 4; ++k) {
                const float4 t = src[k];
                pr[4 * k] = t.x; pr[4 * k + 1] = t.y; pr[4 * k + 2] = t.z; pr[4 * k + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < NVAL; ++k) pr[k] = sm.p[wave][rgrp * 16 + k * HL::REP];
        }
        __builtin_amdgcn_wave_barrier();
        // rescale only when some head's running max moved (wave-uniform test)
        bool moved = false;
#pragma unroll
        for (int g = 0; g < G; ++g) moved = moved || alpha[g] != 1.f;
        if (moved) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[g][c] *= alpha[g];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v8[8];
            unpack(r.v[i], v8);                    // rows past L are zeros and have p = 0
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pg = pr[i * G + g];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(pg, v8[c], acc[g][c]);
            }
        }
    };

    // Three register buffers: the wave set's iterations k+1 and k+2 are in
    // flight while iteration k is computed. sched_barrier keeps the compiler
    // from sinking a prefetch below the compute it is meant to overlap.
    BlockRegs<T> bufA, bufB, bufC;
    auto start = [&](BlockRegs<T> &r, int k) {
        if constexpr (ROWS) issue_rows(r, item_of(k));
        else issue(r, block_id(item_of(k)));
    };
    if constexpr (ROWS) {
        load_ids(bufA.ids, item_of(0));
        load_ids(bufB.ids, item_of(1));
        load_ids(bufC.ids, item_of(2));
    }
    start(bufA, 0);
    start(bufB, 1);
#pragma unroll 1
    for (int k = 0; item_of(k) < nblk; k += 3) {
        start(bufC, k + 2);
        __builtin_amdgcn_sched_barrier(0);
        process(bufA);
        start(bufA, k + 3);
        __builtin_amdgcn_sched_barrier(0);
        if (item_of(k + 1) < nblk) process(bufB);
        start(bufB, k + 4);
        __builtin_amdgcn_sched_barrier(0);
        if (item_of(k + 2) < nblk) process(bufC);
    }

    // ---- merge inside the wave: l over the lanes of one head (lanes sharing
    // lane & 3; for G < 4 each of those classes covers every row once), acc
    // over row groups
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        float l = l_lane[e];
        l += dpp<kDppRowRor4>(l);
        l += dpp<kDppRowRor8>(l);
        l += shfl_xor(l, 16);
        l += shfl_xor(l, 32);
        l_lane[e] = l;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float a = acc[g][c];
            a += shfl_xor(a, 16);
            a += shfl_xor(a, 32);
            acc[g][c] = a;
        }
    if (rgrp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float4 *dst = reinterpret_cast<float4 *>(&sm.acc[wave][g][lane16 * 8]);
            dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
    }
    if (lane < 4) {
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            const int g = HL::head(lane, e);
            if (HL::lane_of(g) == lane) {       // one writer per head
                sm.m[wave][g] = m_my[e];
                sm.l[wave][g] = l_lane[e];
            }
        }
    }
    merge_waves<G, NW, MODE>(sm, row_base, out);
}

// One share of a unit's bf16 list on the matrix cores (same contract as
// attend_share). Wave w still owns rows 16 (w % 4) .. +15 of each block (ROWS:
// of each 64-entry tile of token ids); with g = lane / 16 and h = lane % 16:
//   S = K q^T, v_mfma_f32_16x16x32_bf16 x 4: the A operand's row h is key row
//     h / 4 + 4 (h % 4) of the wave's 16 (lane l loads channels 32 s + 8 g of
//     it in step s), so output element j of lane l is the logit of key
//     g + 4 j for head h: exactly the keys whose V rows the lane loads.
//   O^T += V^T P^T, v_mfma_f32_16x16x16_bf16 x 8: P^T is the B operand as it
//     comes out of the softmax (element j = key g + 4 j, head h, rounded to
//     bf16); tile t's A operand row h is channel 8 h + t, assembled with
//     v_perm from the lane's four V rows. Lane l accumulates head h,
//     channels 32 g + 8 j + t (element j of tile t).
// The softmax runs per lane on its head's 4 logits (max over the wave's 16
// keys by two lane swaps). The reference is raised only when a block's max
// exceeds it by more than kSlack (log2 units): after the first block almost
// never, so the accumulators are rarely touched by vector instructions; the
// probabilities stay below 2^kSlack (sums far inside the fp32 range). Heads
// G .. 15 carry zero queries and are discarded. exp2 is the hardware
// instruction (arguments <= kSlack; results below 2^-126 flush to zero).
// Token lists gather each row by its id (ids of a wave set's tile prefetched
// three tiles ahead with the buffer that uses them, as in attend_share); ids
// outside [0, L) read zeros and their logits are masked.
template <int G, bool ROWS, int NW, int MODE>
__device__ __forceinline__ void attend_share_mfma(const QMfma &q, const bf16_t *__restrict__ K,
                                                  const bf16_t *__restrict__ V, int64_t T_cap,
                                                  int unit, int64_t L, const int32_t *irow, int n,
                                                  int e_lo, int nblk, float qscale, int64_t row_base,
                                                  const AttendOut &out, AttendSmem<G, NW> &sm) {
    constexpr int NWS = NW / 4;                  // wave sets
    constexpr float kSlack = 32.f;
    constexpr uint32_t kRowBytes = kD * sizeof(bf16_t);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wq = wave & 3, wset = wave >> 2;
    const int h = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + (int64_t)unit * T_cap * kD, (uint32_t)(L * kRowBytes));
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + (int64_t)unit * T_cap * kD, (uint32_t)(L * kRowBytes));
    const int k_row = 16 * wq + (h >> 2) + 4 * (h & 3);           // the lane's K row of a block
    const uint32_t k_lane = k_row * kRowBytes + 16 * g;
    const uint32_t v_lane = (16 * wq + g) * kRowBytes + 16 * h;
    const int64_t nb = n_blocks(L);

    // block ids as in attend_share: lane i holds item i's id (-1: none)
    int id_lane = -1;
    if constexpr (!ROWS) {
        if (lane < nblk) {
            const int blk = irow[lane];
            id_lane = (blk >= 0 && blk < nb) ? blk : -1;
        }
    }
    auto item_of = [&](int k) { return wset + k * NWS; };
    auto block_id = [&](int it) -> int {
        return it < nblk ? __builtin_amdgcn_readlane(id_lane, it & 63) : -1;
    };
    // token lists: ids of share tile it (entry 64 (e_lo + it) + row) for the
    // lane's V rows g + 4j and its K row, -1 past the share or the list
    auto load_ids = [&](BlockRegs<bf16_t> &r, int it) {
        const int e0 = 64 * (e_lo + it) + 16 * wq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + g + 4 * j;
            r.ids[j] = (it < nblk && e < n) ? irow[e] : -1;
        }
        const int e = e0 + (k_row - 16 * wq);
        r.idk = (it < nblk && e < n) ? irow[e] : -1;
    };
    // token lists: rows of the ids loaded for tile it (ids outside [0, L) read
    // zeros, no bytes), their visibility bits, then the ids three tiles on
    auto issue_rows = [&](BlockRegs<bf16_t> &r, int it) {
        const bool kv = r.idk >= 0 && r.idk < L;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            load_raw_nt(rK, kv ? (uint32_t)r.idk * kRowBytes + 16 * g + 64 * i : 0xffffffffu, r.k[i]);
        int vis = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = r.ids[j] >= 0 && r.ids[j] < L;
            load_raw_nt(rV, ok ? (uint32_t)r.ids[j] * kRowBytes + 16 * h : 0xffffffffu, r.v[j]);
            vis |= ok ? 1 << j : 0;
        }
        r.tmy = vis;
        r.t0 = 0;
        load_ids(r, it + 3 * NWS);
    };
    // loads of an absent block (id -1) use an out-of-range offset: zeros, no bytes
    auto issue = [&](BlockRegs<bf16_t> &r, int blk) {
        r.t0 = (int64_t)blk * kBlock;
        const uint32_t base = blk < 0 ? 0xffffffffu : (uint32_t)blk * (kBlock * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            load_raw_nt(rK, blk < 0 ? 0xffffffffu : base + k_lane + 64 * i, r.k[i]);
            load_raw_nt(rV, blk < 0 ? 0xffffffffu : base + v_lane + i * (4 * kRowBytes), r.v[i]);
        }
    };

    float m_ref = -INFINITY, l_lane = 0.f;
    mf_f32x4_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = (mf_f32x4_t){0.f, 0.f, 0.f, 0.f};
    auto process = [&](const BlockRegs<bf16_t> &r) {
        if (r.t0 < 0) return;                    // absent block: nothing visible
        mf_f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8_t, r.k[st].v),
                                                      __builtin_bit_cast(mf_bf16x8_t, q.w[st]), s,
                                                      0, 0, 0);
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = s[j] * qscale;
        if constexpr (ROWS) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!((r.tmy >> j) & 1)) x[j] = -INFINITY;
        } else if (r.t0 + kBlock > L) {          // the visible length ends inside this block
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (r.t0 + 16 * wq + g + 4 * j >= L) x[j] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = max_xor32(max_xor16(mx));
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kSlack)) {     // wave-uniform
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_lane *= alpha;
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[t] *= alpha;
        }
        const float mref = m_ref == -INFINITY ? 0.f : m_ref;
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[j] - mref);
        l_lane += (p[0] + p[1]) + (p[2] + p[3]);
        const uint2 pw = make_uint2(
            __builtin_bit_cast(uint32_t, __builtin_convertvector((mf_f32x2_t){p[0], p[1]}, mf_bf16x2_t)),
            __builtin_bit_cast(uint32_t, __builtin_convertvector((mf_f32x2_t){p[2], p[3]}, mf_bf16x2_t)));
        const mf_s16x4_t pb = __builtin_bit_cast(mf_s16x4_t, pw);
        const uint32_t vw[4][4] = {{r.v[0].v.x, r.v[0].v.y, r.v[0].v.z, r.v[0].v.w},
                                   {r.v[1].v.x, r.v[1].v.y, r.v[1].v.z, r.v[1].v.w},
                                   {r.v[2].v.x, r.v[2].v.y, r.v[2].v.z, r.v[2].v.w},
                                   {r.v[3].v.x, r.v[3].v.y, r.v[3].v.z, r.v[3].v.w}};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            // channel 8 h + t of keys g, g + 4 (low word) and g + 8, g + 12
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
            const uint2 a = make_uint2(__builtin_amdgcn_perm(vw[1][t >> 1], vw[0][t >> 1], sel),
                                       __builtin_amdgcn_perm(vw[3][t >> 1], vw[2][t >> 1], sel));
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mf_s16x4_t, a), pb,
                                                              acc[t], 0, 0, 0);
        }
    };

    // three register buffers, as in attend_share
    BlockRegs<bf16_t> bufA, bufB, bufC;
    auto start = [&](BlockRegs<bf16_t> &r, int k) {
        if constexpr (ROWS) issue_rows(r, item_of(k));
        else issue(r, block_id(item_of(k)));
    };
    if constexpr (ROWS) {
        load_ids(bufA, item_of(0));
        load_ids(bufB, item_of(1));
        load_ids(bufC, item_of(2));
    }
    start(bufA, 0);
    start(bufB, 1);
#pragma unroll 1
    for (int k = 0; item_of(k) < nblk; k += 3) {
        start(bufC, k + 2);
        __builtin_amdgcn_sched_barrier(0);
        process(bufA);
        start(bufA, k + 3);
        __builtin_amdgcn_sched_barrier(0);
        if (item_of(k + 1) < nblk) process(bufB);
        start(bufB, k + 4);
        __builtin_amdgcn_sched_barrier(0);
        if (item_of(k + 2) < nblk) process(bufC);
    }

    // the wave's (reference, sum, weighted values) of heads 0 .. G-1
    l_lane = sum_xor32(sum_xor16(l_lane));
    if (h < G) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 *dst = reinterpret_cast<float4 *>(&sm.acc[wave][h][32 * g + 8 * j]);
            dst[0] = make_float4(acc[0][j], acc[1][j], acc[2][j], acc[3][j]);
            dst[1] = make_float4(acc[4][j], acc[5][j], acc[6][j], acc[7][j]);
        }
        if (g == 0) {
            sm.m[wave][h] = m_ref;
            sm.l[wave][h] = l_lane;
        }
    }
    merge_waves<G, NW, MODE>(sm, row_base, out);
}

}  // namespace sa
