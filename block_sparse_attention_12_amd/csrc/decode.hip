// Gathered split-K sparse decode attention (Eq. 5 of the SparDA summary page,
// "Methodology": the attention query attends only to the keys and values of the
// selected blocks).
//
// Work unit: (sequence b, KV head kvh, split s). The unit's selected blocks
// idx[b, kvh, 0..cnt) are divided into n_split contiguous shares; each
// workgroup streams its share's K and V blocks (64 rows x 256 B each for bf16,
// contiguous in HBM) once and serves all G query heads of the group from that
// single read (GQA packing; G = 1, 2, 4 or 8, a template parameter).
//
// Mapping of a 256-thread workgroup: wave w owns rows 16w .. 16w+15 of every
// block; inside a wave, row group r = lane / 16 takes rows 16w + 4i + r
// (i = 0..3) and each lane owns 8 channels. A block costs each lane 4 K and
// 4 V loads of 16 B. Loads of the next two blocks are in flight while a block
// is computed (three register buffers); block ids are uniform scalar loads,
// and the loads of an absent block use an out-of-range offset, so every wait
// in the loop is for data already in flight.
//
// Logits for 4 rows x G heads are reduced across the 16 lanes of a row by the
// DPP transposed reduction: lane position p (lane & 15) ends with the logits
// of row p / 4 and, for G >= 4, of heads (p & 3) * G/4 .. + G/4 - 1 (G/4 of
// them per lane); for G < 4 the 4G totals are replicated over 4/G lanes each
// (bf16 inputs use the packed bf16 dot product for q.k). The online softmax
// keeps a running max per head (wave-uniform) and per-lane partial sums, so no
// workgroup barrier is needed inside the block loop; probabilities reach the
// lanes holding the matching V rows through a wave-private LDS slot. Logits
// are in base-2 units (scaled by scale * log2 e) so each exponential is one
// exp2.
//
// Split merge: every workgroup writes (max, sum, weighted values) for its G
// heads and combine_kernel, launched next on the same stream, merges the
// n_split partials with log-sum-exp weights. (Merging inside the last
// workgroup of a unit would need a device-scope release fence per workgroup,
// which on this multi-die part writes back L2 and serialises the grid.) With
// n_split = 1 the workgroup writes O directly.
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"
#include "topk_device.h"

namespace sa {

constexpr int kDecThreads = 256;
constexpr int kPartStride = kD + 4;          // acc[128], max, sum, 2 pad (16 B aligned rows)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// a split holds at most 64 blocks (one block id per lane)
int decode_min_split(int32_t idx_cap) { return (idx_cap + 63) / 64; }

int decode_auto_split(int B, int Hkv, int32_t idx_cap) {
    const int units = B * Hkv;
    // ~1 workgroup per CU: with streaming loads, fewer and longer workgroups
    // keep as many bytes in flight (3 blocks each) and pay the per-workgroup
    // start (and, in the decode step, the top-k prologue) less often (measured
    // against 512: 128K Forecast step +4%, 32K GQA +2%, no workload slower)
    const int target = 256;
    int s = (target + units - 1) / units;
    int max_s = idx_cap / 4 > 1 ? idx_cap / 4 : 1;       // at least ~4 blocks per split
    if (s > max_s) s = max_s;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return decode_min_split(idx_cap) > s ? decode_min_split(idx_cap) : s;
}

// workspace: the split partials [B * Hq][n_split][kPartStride] fp32
size_t decode_workspace_bytes(int B, int Hq, int32_t n_split) {
    if (n_split <= 1) return 0;
    return (size_t)B * Hq * n_split * kPartStride * sizeof(float);
}

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

// Where the reduced logits of a group of G heads live (see the file comment):
// NV logits per lane; for G < 4 each total sits on REP = 4/G lanes.
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
    int tmy;        // token lists: id of the row whose logit this lane holds (loaded tile)
};

// ROWS = false: idx lists 64-token blocks (contiguous rows). ROWS = true: idx
// lists single tokens (the token-level index); 64 consecutive list entries
// form a tile that is processed exactly like a block, except that each lane
// loads its 4 rows from the token ids of its entries. A lane's ids are
// prefetched three tiles ahead, together with the buffer that will use them,
// so waiting for them never waits for K/V loads that are still needed in
// flight.
// SG > 0: the workgroup first takes its own unit's top-k (topk_unit, with SG
// selector heads per group, SSOFT for the softmax-sum form) from the scoring
// kernels' output into LDS; every split of a unit computes the same set (the
// redundant work replaces a separate top-k launch on the critical path) and
// split 0 writes it out.
template <typename T, int G, bool DIRECT, bool ROWS, int SG = 0, bool SSOFT = false>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, int Hq, int Hkv,
    int64_t T_cap, const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int idx_cap, float qscale, int n_split,
    float *__restrict__ part, void *__restrict__ O, int out_bf16,
    float *__restrict__ lse, FusedSelect fs) {
    using HL = HeadLayout<G>;
    constexpr int NV = HL::NV;
    constexpr int NVAL = 4 * G;                  // logits per row group per block (4 rows x G heads)
    constexpr int SP = NVAL > 16 ? NVAL : 16;    // LDS floats per row group
    __shared__ __align__(16) float s_p[4][4 * SP];
    __shared__ float s_m[4][G], s_l[4][G];
    __shared__ __align__(16) float s_acc[4][G][kD];

    const int split = blockIdx.x, unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lane16 = lane & 15, rgrp = lane >> 4;
    int64_t L = seq_lens[b];
    L = L < 0 ? 0 : (L > T_cap ? T_cap : L);
    // the group's queries: loaded first, so the load overlaps the top-k below
    QFrag<T, G> q;
    load_q<G>(Q + ((int64_t)b * Hq + (int64_t)kvh * G) * kD + lane16 * kLaneElems, q);
    int n;
    const int32_t *idx_row;
    if constexpr (SG > 0) {
        __shared__ int32_t s_list[kFusedMaxCap];
        __shared__ int32_t s_cnt;
        topk_unit<SG, SSOFT, kDecThreads, kFusedMaxBlocks / kDecThreads>(
            unit, Hkv, T_cap, fs.nb_cap, seq_lens, fs.top_k, fs.n_init, fs.n_local, fs.logits,
            fs.nc_pad, fs.stats, fs.n_chunks, fs.bscore, nullptr, s_list, idx_cap, &s_cnt,
            fs.use_buckets);
        __syncthreads();
        if (split == 0) {
            for (int i = tid; i < idx_cap; i += kDecThreads)
                fs.idx_out[(int64_t)unit * idx_cap + i] = s_list[i];
            if (tid == 0) fs.cnt_out[unit] = s_cnt;
        }
        n = s_cnt;
        idx_row = s_list;
    } else {
        n = cnt[unit];
        idx_row = idx + (int64_t)unit * idx_cap;
    }
    n = n < 0 ? 0 : (n > idx_cap ? idx_cap : n);
    const int n_items = ROWS ? (n + 63) / 64 : n;      // blocks, or 64-entry tiles of tokens
    const int per = (n_items + n_split - 1) / n_split;
    const int e_lo = split * per < n_items ? split * per : n_items;
    const int nblk = (e_lo + per < n_items ? e_lo + per : n_items) - e_lo;

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
    const int32_t *irow = idx_row + (ROWS ? 0 : e_lo);
    const int my_row = 16 * wave + 4 * (lane16 >> 2) + rgrp;   // row of the logits this lane holds
    const int row0 = 16 * wave + rgrp;                          // first row this lane loads
    const uint32_t row_lane_off = row0 * kRowBytes + lane_off;
    const int64_t nb = n_blocks(L);

    // block id of iteration it (a uniform scalar load), or -1 (no rows) past
    // the share or out of range
    auto block_id = [&](int it) -> int {
        const int blk = it < nblk ? irow[it] : -1;
        return (blk >= 0 && blk < nb) ? blk : -1;
    };
    // Issues the block's K/V loads unconditionally: id -1 maps every row to an
    // out-of-range offset, which reads zeros and moves no bytes, so the wait
    // counts stay exact (one block in flight behind the current one).
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
    // split tile it, or -1 past the split or the list
    auto load_ids = [&](int (&ids)[4], int it) {
        const int e0 = 64 * (e_lo + it) + row0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + 4 * i;
            ids[i] = (it < nblk && e < n) ? irow[e] : -1;
        }
    };
    // token lists: rows from the ids loaded for tile it (ids outside [0, L)
    // read zeros and are masked), then the ids of tile it + 3
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
        load_ids(r.ids, it + 3);
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
            for (int e = 0; e < NV; ++e) s_p[wave][lane * NV + e] = p[e];
        } else {
            s_p[wave][lane] = p[0];
        }
        __builtin_amdgcn_wave_barrier();
        float pr[NVAL];
        if constexpr (G >= 4) {
            const float4 *src = reinterpret_cast<const float4 *>(&s_p[wave][rgrp * NVAL]);
#pragma unroll
            for (int k = 0; k < NVAL / 4; ++k) {
                const float4 t = src[k];
                pr[4 * k] = t.x; pr[4 * k + 1] = t.y; pr[4 * k + 2] = t.z; pr[4 * k + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < NVAL; ++k) pr[k] = s_p[wave][rgrp * 16 + k * HL::REP];
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

    // Three register buffers: blocks it+1 and it+2 are in flight while block it
    // is computed. sched_barrier keeps the compiler from sinking a prefetch
    // below the compute it is meant to overlap.
    BlockRegs<T> bufA, bufB, bufC;
    auto start = [&](BlockRegs<T> &r, int it) {
        if constexpr (ROWS) issue_rows(r, it);
        else issue(r, block_id(it));
    };
    if constexpr (ROWS) {
        load_ids(bufA.ids, 0);
        load_ids(bufB.ids, 1);
        load_ids(bufC.ids, 2);
    }
    start(bufA, 0);
    start(bufB, 1);
#pragma unroll 1
    for (int it = 0; it < nblk; it += 3) {
        start(bufC, it + 2);
        __builtin_amdgcn_sched_barrier(0);
        process(bufA);
        start(bufA, it + 3);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 1 < nblk) process(bufB);
        start(bufB, it + 4);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 2 < nblk) process(bufC);
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
            float4 *dst = reinterpret_cast<float4 *>(&s_acc[wave][g][lane16 * 8]);
            dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
    }
    if (lane < 4) {
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            const int g = HL::head(lane, e);
            if (HL::lane_of(g) == lane) {       // one writer per head
                s_m[wave][g] = m_my[e];
                s_l[wave][g] = l_lane[e];
            }
        }
    }
    __syncthreads();

    // ---- merge the four waves: thread -> (head g, channels 2c, 2c+1)
#pragma unroll
    for (int pair = tid; pair < G * (kD / 2); pair += kDecThreads) {
        const int g = pair / (kD / 2);
        const int c2 = (pair % (kD / 2)) * 2;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
        float lsum = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = s_m[w][g];
            const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            lsum = fmaf(wt, s_l[w][g], lsum);
            a0 = fmaf(wt, s_acc[w][g][c2], a0);
            a1 = fmaf(wt, s_acc[w][g][c2 + 1], a1);
        }
        const int64_t row = (int64_t)b * Hq + (int64_t)kvh * G + g;   // query head row
        if constexpr (!DIRECT) {
            float *dst = part + (row * n_split + split) * kPartStride;
            reinterpret_cast<float2 *>(dst)[c2 / 2] = make_float2(a0, a1);
            if (c2 == 0) {
                dst[kD] = M;
                dst[kD + 1] = lsum;
            }
            continue;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if (out_bf16) {
            const uint32_t w = f32_to_bf16_bits(a0 * inv) | (f32_to_bf16_bits(a1 * inv) << 16);
            reinterpret_cast<uint32_t *>(O)[(row * kD + c2) / 2] = w;
        } else {
            reinterpret_cast<float2 *>(O)[(row * kD + c2) / 2] = make_float2(a0 * inv, a1 * inv);
        }
        if (lse && c2 == 0) lse[row] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
    }
}

// Merges the n_split partials of query-head rows. A workgroup takes 4 rows
// (B * Hq rows in all): thread (row 4x + g, channels 2c, 2c+1) loads, for eight
// splits at a time, each split's (max, sum) pair (the same address on every
// lane of the wave, one cache line) and its own two weighted-value channels,
// all sixteen loads in flight at once, and merges them with log-sum-exp
// weights against the running maximum. Up to eight splits this is one memory
// round trip and no workgroup barrier.
__global__ __launch_bounds__(kDecThreads) void combine_kernel(
    const float *__restrict__ part, int n_split, int64_t n_rows, void *__restrict__ O,
    int out_bf16, float *__restrict__ lse) {
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * 4 + (tid >> 6);
    if (row >= n_rows) return;
    const int c2 = (tid & 63) * 2;
    const float *pg = part + row * n_split * kPartStride;
    float M = -INFINITY, lsum = 0.f, a0 = 0.f, a1 = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += 8) {
        float2 ml[8], a[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 + k < n_split) {
                const float *ps = pg + (int64_t)(s0 + k) * kPartStride;
                ml[k] = *reinterpret_cast<const float2 *>(ps + kD);
                a[k] = *reinterpret_cast<const float2 *>(ps + c2);
            } else {
                ml[k] = make_float2(-INFINITY, 0.f);
                a[k] = make_float2(0.f, 0.f);
            }
        }
        float Mc = M;
#pragma unroll
        for (int k = 0; k < 8; ++k) Mc = fmaxf(Mc, ml[k].x);
        if (Mc == -INFINITY) continue;                      // nothing seen yet
        const float w_old = (M == -INFINITY) ? 0.f : exp2f(M - Mc);
        lsum *= w_old;
        a0 *= w_old;
        a1 *= w_old;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float wt = (ml[k].x == -INFINITY) ? 0.f : exp2f(ml[k].x - Mc);
            lsum = fmaf(wt, ml[k].y, lsum);
            a0 = fmaf(wt, a[k].x, a0);
            a1 = fmaf(wt, a[k].y, a1);
        }
        M = Mc;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (out_bf16) {
        const uint32_t w = f32_to_bf16_bits(a0 * inv) | (f32_to_bf16_bits(a1 * inv) << 16);
        reinterpret_cast<uint32_t *>(O)[(row * kD + c2) / 2] = w;
    } else {
        reinterpret_cast<float2 *>(O)[(row * kD + c2) / 2] = make_float2(a0 * inv, a1 * inv);
    }
    if (lse && (tid & 63) == 0) lse[row] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
}

static void launch_combine(const float *part, int n_split, int B, int Hq, void *O, int out_bf16,
                           float *lse, hipStream_t stream) {
    const int64_t rows = (int64_t)B * Hq;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kDecThreads), 0,
                       stream, part, n_split, rows, O, out_bf16, lse);
}

template <typename T, int G, bool ROWS>
static void launch_decode_t(const void *Q, const void *K, const void *V, int B, int Hq, int Hkv,
                            int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                            const int32_t *cnt, int32_t idx_cap, float scale, void *O,
                            int out_bf16, float *lse, int32_t n_split, void *ws,
                            hipStream_t stream) {
    const dim3 grid((unsigned)n_split, (unsigned)(B * Hkv));
    const float qscale = scale * kLog2e;
    if (n_split == 1) {
        hipLaunchKernelGGL((decode_kernel<T, G, true, ROWS>), grid, dim3(kDecThreads), 0, stream,
                           (const T *)Q, (const T *)K, (const T *)V, Hq, Hkv, T_cap, seq_lens, idx,
                           cnt, idx_cap, qscale, 1, (float *)nullptr, O, out_bf16, lse, FusedSelect{});
    } else {
        hipLaunchKernelGGL((decode_kernel<T, G, false, ROWS>), grid, dim3(kDecThreads), 0, stream,
                           (const T *)Q, (const T *)K, (const T *)V, Hq, Hkv, T_cap, seq_lens, idx,
                           cnt, idx_cap, qscale, n_split, (float *)ws, O, out_bf16, lse, FusedSelect{});
        launch_combine((const float *)ws, n_split, B, Hq, O, out_bf16, lse, stream);
    }
}

// G = Hq / Hkv dispatch; other ratios are refused by the ABI before this
template <typename T, bool ROWS>
static int launch_decode_g(const void *Q, const void *K, const void *V, int B, int Hq, int Hkv,
                           int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                           const int32_t *cnt, int32_t idx_cap, float scale, void *O, int out_bf16,
                           float *lse, int32_t n_split, void *ws, hipStream_t stream) {
#define SA_DEC_ARGS (Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap, scale, O, out_bf16, \
                     lse, n_split, ws, stream)
    switch (Hq / Hkv) {
        case 1: launch_decode_t<T, 1, ROWS> SA_DEC_ARGS; break;
        case 2: launch_decode_t<T, 2, ROWS> SA_DEC_ARGS; break;
        case 4: launch_decode_t<T, 4, ROWS> SA_DEC_ARGS; break;
        case 8: launch_decode_t<T, 8, ROWS> SA_DEC_ARGS; break;
        default: return SA_ERR_UNSUPPORTED;
    }
#undef SA_DEC_ARGS
    return SA_OK;
}

template <bool ROWS>
static int launch_decode_any(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                             int Hkv, int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                             const int32_t *cnt, int32_t idx_cap, float scale, void *O,
                             int out_dtype, float *lse_out, int32_t n_split, void *workspace,
                             hipStream_t stream) {
    const int out_bf16 = out_dtype == SA_BF16 ? 1 : 0;
    const int st = dtype == SA_BF16
                       ? launch_decode_g<bf16_t, ROWS>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx,
                                                       cnt, idx_cap, scale, O, out_bf16, lse_out,
                                                       n_split, workspace, stream)
                       : launch_decode_g<float, ROWS>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx, cnt,
                                                      idx_cap, scale, O, out_bf16, lse_out, n_split,
                                                      workspace, stream);
    if (st) return st;
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

int launch_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq, int Hkv,
                  int64_t T_cap, const int32_t *seq_lens, const int32_t *idx, const int32_t *cnt,
                  int32_t idx_cap, float scale, void *O, int out_dtype, float *lse_out,
                  int32_t n_split, void *workspace, hipStream_t stream) {
    return launch_decode_any<false>(Q, K, V, dtype, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap,
                                    scale, O, out_dtype, lse_out, n_split, workspace, stream);
}

int launch_decode_rows(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                       int Hkv, int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                       const int32_t *cnt, int32_t idx_cap, float scale, void *O, int out_dtype,
                       float *lse_out, int32_t n_split, void *workspace, hipStream_t stream) {
    return launch_decode_any<true>(Q, K, V, dtype, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap,
                                   scale, O, out_dtype, lse_out, n_split, workspace, stream);
}

template <typename T, int G, int SG, bool SSOFT>
static void launch_decode_select_t(const void *Q, const void *K, const void *V, int B, int Hq,
                                   int Hkv, int64_t T_cap, const int32_t *seq_lens,
                                   int32_t idx_cap, float scale, void *O, int out_bf16, float *lse,
                                   int32_t n_split, void *ws, const FusedSelect &fs,
                                   hipStream_t stream) {
    const dim3 grid((unsigned)n_split, (unsigned)(B * Hkv));
    const float qscale = scale * kLog2e;
    if (n_split == 1) {
        hipLaunchKernelGGL((decode_kernel<T, G, true, false, SG, SSOFT>), grid, dim3(kDecThreads),
                           0, stream, (const T *)Q, (const T *)K, (const T *)V, Hq, Hkv, T_cap,
                           seq_lens, (const int32_t *)nullptr, (const int32_t *)nullptr, idx_cap,
                           qscale, 1, (float *)nullptr, O, out_bf16, lse, fs);
    } else {
        hipLaunchKernelGGL((decode_kernel<T, G, false, false, SG, SSOFT>), grid, dim3(kDecThreads),
                           0, stream, (const T *)Q, (const T *)K, (const T *)V, Hq, Hkv, T_cap,
                           seq_lens, (const int32_t *)nullptr, (const int32_t *)nullptr, idx_cap,
                           qscale, n_split, (float *)ws, O, out_bf16, lse, fs);
        launch_combine((const float *)ws, n_split, B, Hq, O, out_bf16, lse, stream);
    }
}

template <typename T, int SG, bool SSOFT>
static int launch_decode_select_g(const void *Q, const void *K, const void *V, int B, int Hq,
                                  int Hkv, int64_t T_cap, const int32_t *seq_lens, int32_t idx_cap,
                                  float scale, void *O, int out_bf16, float *lse, int32_t n_split,
                                  void *ws, const FusedSelect &fs, hipStream_t stream) {
#define SA_DS_ARGS (Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx_cap, scale, O, out_bf16, lse, n_split, \
                    ws, fs, stream)
    switch (Hq / Hkv) {
        case 1: launch_decode_select_t<T, 1, SG, SSOFT> SA_DS_ARGS; break;
        case 2: launch_decode_select_t<T, 2, SG, SSOFT> SA_DS_ARGS; break;
        case 4: launch_decode_select_t<T, 4, SG, SSOFT> SA_DS_ARGS; break;
        case 8: launch_decode_select_t<T, 8, SG, SSOFT> SA_DS_ARGS; break;
        default: return SA_ERR_UNSUPPORTED;
    }
#undef SA_DS_ARGS
    return SA_OK;
}

template <typename T>
static int launch_decode_select_sel(const void *Q, const void *K, const void *V, int B, int Hq,
                                    int Hkv, int64_t T_cap, const int32_t *seq_lens,
                                    int32_t idx_cap, float scale, void *O, int out_bf16,
                                    float *lse, int32_t n_split, void *ws, const FusedSelect &fs,
                                    int SGv, bool softmax, hipStream_t stream) {
#define SA_DSG(SGV, SM)                                                                           \
    launch_decode_select_g<T, SGV, SM>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx_cap, scale, O,   \
                                       out_bf16, lse, n_split, ws, fs, stream)
    if (!softmax) return SA_DSG(1, false);
    if (fs.epb != 4) return SA_ERR_UNSUPPORTED;
    if (SGv == 1) return SA_DSG(1, true);
    if (SGv == 2) return SA_DSG(2, true);
    if (SGv == 4) return SA_DSG(4, true);
#undef SA_DSG
    return SA_ERR_UNSUPPORTED;
}

int launch_decode_select(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                         int Hkv, int64_t T_cap, const int32_t *seq_lens, int32_t idx_cap,
                         float scale, void *O, int out_dtype, float *lse_out, int32_t n_split,
                         void *workspace, const FusedSelect &fs, int SGv, bool softmax,
                         hipStream_t stream) {
    const int out_bf16 = out_dtype == SA_BF16 ? 1 : 0;
    const int st = dtype == SA_BF16
                       ? launch_decode_select_sel<bf16_t>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens,
                                                          idx_cap, scale, O, out_bf16, lse_out,
                                                          n_split, workspace, fs, SGv, softmax, stream)
                       : launch_decode_select_sel<float>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens,
                                                         idx_cap, scale, O, out_bf16, lse_out,
                                                         n_split, workspace, fs, SGv, softmax, stream);
    if (st) return st;
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
