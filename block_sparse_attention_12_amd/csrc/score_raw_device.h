// Raw-sum block scores (Eq. 4 of the SparDA summary page, "Methodology", in
// its raw form: the group-summed selector, or one Forecast vector per KV head,
// dotted with the compressed keys; a block's score is the max over its three
// inside entries) for one chunk of blocks of one (sequence, KV head) unit.
// Device code of the selection kernel, parameterised on the workgroup's row
// groups and the chunk size.
//
// A row group of 16 lanes reads 4 blocks x 3 inside entries per iteration
// (one 16 B load per lane per entry; the straddling entry 4b+3 feeds no block
// maximum and is not read), the next iteration's rows in flight while the
// current ones are reduced by the DPP transposed reduction; bf16 keys with a
// single selector use the packed bf16 dot product.
#pragma once

#include "compress_device.h"
#include "sa_device.h"

namespace sa {

constexpr int kRawChunkBlocks = 256;                // blocks per chunk
constexpr int kAppendColumn = 1;                    // the append as an extra column of workgroups
constexpr int kAppendInFirst = 2;                   // the append by each unit's chunk-0 workgroup
constexpr int kAppendElsewhere = 3;                 // another launch appends (scores only)

template <typename T>
struct RawIter {                         // one iteration: 4 blocks x 3 inside entries per row group
    Raw8<T> r[12];
};

// Raw-sum block scores of one chunk of CHUNK blocks of one unit, by
// a workgroup of NRG row groups (16 lanes each). APPEND (the decode step): the
// compressed entries completed between lens_prev and seq_lens are written by
// this launch itself, either by an extra column of workgroups
// (append_column) while the others score, or by each unit's chunk-0
// workgroup after its own blocks (app_mode kAppendInFirst), or by the next
// launch (kAppendElsewhere: this launch writes nothing to Kc). Scoring then
// reads only the entries that existed before (j < n_c(lens_prev)) from Kc and
// forms any newer entry it needs from K itself, with the same arithmetic, so
// it never depends on the concurrent writes.
template <typename T, bool APPEND, int NRG, int CHUNK = kRawChunkBlocks>
__device__ __forceinline__ void score_raw_chunk(
    const T *__restrict__ sel, int H_sel, int Gs, const T *__restrict__ Kc, int Hkv,
    int64_t nc_cap, int64_t T_cap, const int32_t *__restrict__ seq_lens, float *__restrict__ bscore,
    int64_t nb_cap, const T *__restrict__ K, T *__restrict__ Kc_w,
    const int32_t *__restrict__ lens_prev, int n_local, int app_mode, int chunk, int unit,
    bool append_column) {
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int64_t L = clamp_len(seq_lens[b], T_cap);
    const int64_t nc = n_compressed(L);
    const int lane = threadIdx.x & 63;
    const int lane16 = threadIdx.x & 15;
    const int group = threadIdx.x >> 4;                 // 0 .. NRG - 1
    constexpr uint32_t kRowBytes = kD * sizeof(T);
    constexpr int kStep = 4 * NRG;                      // blocks per iteration of the workgroup
    int64_t nc_old = nc;                                // entries readable from Kc
    if constexpr (APPEND) {
        int64_t Lp = lens_prev[b];
        Lp = Lp < 0 ? 0 : (Lp > L ? L : Lp);
        nc_old = n_compressed(Lp);
        if (append_column) {                            // the append column
            const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
            T *Kcu = Kc_w + (int64_t)unit * nc_cap * kD + lane16 * kLaneElems;
            for (int64_t j = nc_old + group; j < nc; j += NRG) {   // few keys in flight
                Raw8<T> r;
                compress_entry_raw(Ku, j, r);
                store_raw(Kcu + j * kD, r);
            }
            return;
        }
    }
    // rows at or past the readable entries read as zeros
    const __amdgpu_buffer_rsrc_t rKc = make_rsrc(Kc + (int64_t)unit * nc_cap * kD,
                                                (uint32_t)(nc_old * kRowBytes));
    const uint32_t lane_off = lane16 * kLaneElems * sizeof(T);
    const int64_t chunk0 = (int64_t)chunk * CHUNK;
    auto issue = [&](RawIter<T> &it, int64_t blk0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 3; ++e)
                load_raw(rKc, row_offset(4 * (blk0 + q) + e, kRowBytes, lane_off), it.r[q * 3 + e]);
    };
    // first rows go out before the selector is even loaded
    RawIter<T> bufA, bufB;
    issue(bufA, chunk0 + group * 4);

    // group-summed selector slice (sum in head order)
    float s[8];
    uint32_t s_bf[4];                       // the single selector as bf16 pairs (Gs == 1, bf16)
    {
        const T *sp = sel + ((int64_t)b * H_sel + (int64_t)kvh * Gs) * kD + lane16 * kLaneElems;
        Raw8<T> raw[8];
#pragma unroll
        for (int g = 0; g < 8; ++g)
            if (g < Gs) load_raw(sp + (int64_t)g * kD, raw[g]);
        unpack(raw[0], s);
#pragma unroll
        for (int g = 1; g < 8; ++g) {
            if (g < Gs) {
                float x[8];
                unpack(raw[g], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[e] = s[e] + x[e];
            }
        }
        if constexpr (sizeof(T) == 2) {
            const Raw8<bf16_t> &r0 = reinterpret_cast<const Raw8<bf16_t> &>(raw[0]);
            s_bf[0] = r0.v.x; s_bf[1] = r0.v.y; s_bf[2] = r0.v.z; s_bf[3] = r0.v.w;
        }
    }
    const bool use_dot2 = sizeof(T) == 2 && Gs == 1;
    float *bs = bscore + (int64_t)unit * nb_cap;

    auto process = [&](const RawIter<T> &it, int64_t blk0) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                float acc = 0.f;
                if constexpr (sizeof(T) == 2) {
                    if (use_dot2) {
                        const Raw8<bf16_t> &k8 = reinterpret_cast<const Raw8<bf16_t> &>(it.r[q * 3 + e]);
                        acc = dot2_bf16(s_bf[0], k8.v.x, acc);
                        acc = dot2_bf16(s_bf[1], k8.v.y, acc);
                        acc = dot2_bf16(s_bf[2], k8.v.z, acc);
                        acc = dot2_bf16(s_bf[3], k8.v.w, acc);
                    }
                }
                if (!use_dot2) {
                    float x[8];
                    unpack(it.r[q * 3 + e], x);
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc = fmaf(s[c], x[c], acc);
                }
                v[q * 4 + e] = acc;
            }
            v[q * 4 + 3] = 0.f;
        }
        transpose_reduce16<16>(v, lane);
        // lane position i holds block (i >> 2), inside entry (i & 3)
        const int q = lane16 >> 2, e = lane16 & 3;
        const int64_t blk = blk0 + q;
        const int64_t j = 4 * blk + e;
        float x = (e < 3 && j < nc) ? v[0] : -INFINITY;
        x = fmaxf(x, dpp<kDppQuadXor1>(x));
        x = fmaxf(x, dpp<kDppQuadXor2>(x));
        if (e == 0 && blk < nb_cap) bs[blk] = x;
    };

    // iterations of kStep blocks; the next iteration's rows are in flight while
    // the current ones are reduced (sched_barrier keeps the prefetch in place)
    constexpr int kIters = CHUNK / kStep;
    static_assert(CHUNK % kStep == 0, "chunk of whole iterations");
#pragma unroll
    for (int it = 0; it < kIters; it += 2) {
        const int64_t b0 = chunk0 + it * kStep + group * 4;
        if (it + 1 < kIters) issue(bufB, b0 + kStep);
        __builtin_amdgcn_sched_barrier(0);
        process(bufA, b0);
        if (it + 1 < kIters) {
            if (it + 2 < kIters) issue(bufA, b0 + 2 * kStep);
            __builtin_amdgcn_sched_barrier(0);
            process(bufB, b0 + kStep);
        }
    }
    if constexpr (APPEND) {
        // Blocks holding entries of this step's append were scored above with
        // those entries read as zeros. Each row group rescores its affected
        // candidate 4-block groups (rare: a single token's new window lies in
        // the local blocks) with the new entries formed from the keys (same
        // arithmetic as the append), through the same reduction, and
        // overwrites their scores. The scores of affected local blocks stay
        // provisional: the top-k never reads them, and this launch is used
        // without a block-score output. Runs after the main loop, so its
        // registers do not add to the loop's.
        // blocks with an inside entry in [nc_old, nc), below the local window
        // (local blocks are kept whatever their score; only top-k candidates
        // need exact scores)
        const int64_t b_lo = (nc_old + 1) / 4;                  // 4b + 2 >= nc_old
        int64_t b_hi = (nc - 1) / 4 + 1;                         // 4b <= nc - 1
        const int64_t cand_hi = n_blocks(L) - n_local;
        b_hi = b_hi < cand_hi ? b_hi : cand_hi;
        if (nc > nc_old && b_lo < b_hi) {
            const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
#pragma unroll 1
            for (int it = 0; it < kIters; ++it) {
                const int64_t b0 = chunk0 + it * kStep + group * 4;
                if (b0 + 3 < b_lo || b0 >= b_hi) continue;            // uniform per row group
                RawIter<T> fix;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 3; ++e) {
                        const int64_t j = 4 * (b0 + q) + e;
                        if (j >= nc_old && j < nc) compress_entry_raw(Ku, j, fix.r[q * 3 + e]);
                        else load_raw(rKc, row_offset(j, kRowBytes, lane_off), fix.r[q * 3 + e]);
                    }
                process(fix, b0);
            }
        }
    }
    // kAppendInFirst (chosen when the caller expects at most one new entry per
    // unit): after its own blocks, the unit's chunk-0 workgroup writes the new
    // entries. With bf16 keys and one new entry it loads the entry's 32 keys
    // (all in flight at once), stages them in LDS and one row group sums them
    // in token order. (Loads issued before the main loop, under a condition,
    // cost the loop its exact wait counts.) Otherwise (fp32 keys, or the
    // length grew by more than expected) it forms every new entry, one row
    // group per entry, so Kc never has gaps.
    if constexpr (APPEND) {
        const bool first = app_mode == kAppendInFirst && chunk == 0;      // uniform
        if (first && nc_old < nc && (sizeof(T) != 2 || nc_old + 1 < nc)) {
            const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
            T *Kcu = Kc_w + (int64_t)unit * nc_cap * kD + lane16 * kLaneElems;
            for (int64_t j = nc_old + group; j < nc; j += NRG) {
                Raw8<T> r;
                compress_entry_raw(Ku, j, r);
                store_raw(Kcu + j * kD, r);
            }
        } else if constexpr (sizeof(T) == 2) {
            if (first && nc_old < nc) {
                __shared__ uint4 s_rows[2 * kCmpStride][16];
                const T *Ka = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
                constexpr int kRows = 2 * kCmpStride / NRG;          // keys per row group
                Raw8<T> app_rows[kRows];
#pragma unroll
                for (int i = 0; i < kRows; ++i)
                    load_raw(Ka + (nc_old * kCmpStride + kRows * group + i) * kD, app_rows[i]);
#pragma unroll
                for (int i = 0; i < kRows; ++i) s_rows[kRows * group + i][lane16] = app_rows[i].v;
                __syncthreads();
                if (group == 0) {
                    Raw8<T> e;
                    entry_from_rows(s_rows, lane16, e);
                    store_raw(Kc_w + ((int64_t)unit * nc_cap + nc_old) * kD + lane16 * kLaneElems, e);
                }
            }
        }
    }
}

}  // namespace sa
