// Block top-k and union (Eq. 1 of the SparDA summary page, "Theoretical
// Foundation"; ties to the lower block index) for one (sequence, KV head) by
// one workgroup: from precomputed block scores (raw-sum mode) or from the
// entry logits and per-chunk softmax statistics (softmax-sum mode, Eq. 6
// form). Shared by the selection kernels and the decode kernel that selects
// its own blocks.
#pragma once

#include <float.h>
#include <math.h>

#include "sa_device.h"

namespace sa {

constexpr int kSoftmaxChunk = 512;                  // entries per scoring workgroup (softmax mode)
constexpr int kStatChunk = 256;                     // blocks per second-order scoring workgroup
constexpr int kBoundaryCap = 512;                   // boundary-bucket candidates ranked in LDS
constexpr int kBucketMinUnits = 1024;               // top-k grids this large take the bucket path

// Top-k + union of one (sequence, KV head) by one workgroup of NT threads:
// writes the ascending union (-1 padded to idx_cap) to row (global or LDS)
// and its count to *cnt_slot. Used by topk_kernel and by the decode kernel
// that selects its own unit's blocks.
//
// Thread t owns PER consecutive blocks [t*PER, t*PER + PER): their 32-bit
// orderable keys stay in registers for the whole kernel, so the bucket (and,
// when needed, radix) passes are register compares plus LDS histogram atomics,
// and the ascending compaction is one workgroup prefix scan.
//
// SOFTMAX: scores are the Eq. 6 form, the sum over the group's heads of each
// head's softmax, from per-head logits and per-chunk (max, sum exp) partials.
// EPB = 4: logits of compressed entries (4 per block; a block's score is the
// max over its 3 inside entries), chunks of kSoftmaxChunk entries. EPB = 1:
// one logit per block (block statistics), chunks of kStatChunk blocks; a
// block whose every head's logit is -inf has no score.
template <int G, bool SOFTMAX, int NT, int PER, int EPB = 4>
__device__ __forceinline__ void topk_unit(
    int unit, int Hkv, int64_t T_cap, int64_t nb_cap, const int32_t *__restrict__ seq_lens,
    int top_k, int n_init, int n_local, const float *__restrict__ logits, int64_t nc_pad,
    const float2 *__restrict__ stats, int n_chunks, const float *__restrict__ bscore_in,
    float *__restrict__ bscore_out, int32_t *row, int idx_cap, int32_t *cnt_slot,
    int use_buckets) {
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_hist2[256];
    __shared__ uint32_t s_kmin[NT / 64], s_kmax[NT / 64];
    __shared__ float s_M[G], s_Zinv[G];
    __shared__ float2 s_st[G * 64];
    constexpr int kSelWords = NT * PER / 32;        // one bit per block this workgroup covers
    __shared__ int s_wave[NT / 64];
    __shared__ uint32_t s_digit, s_above, s_bcnt, s_nbnd;
    __shared__ float s_lo[NT / 64], s_hi[NT / 64];
    __shared__ uint32_t s_sel[kSelWords];
    __shared__ uint32_t s_bkey[kBoundaryCap];
    __shared__ int s_bblk[kBoundaryCap];
    const int b = unit / Hkv;
    const int tid = threadIdx.x;
    const int64_t L = clamp_len(seq_lens[b], T_cap);
    const int64_t nc = n_compressed(L);
    const int nb = (int)n_blocks(L);
    const int init_hi = n_init < nb ? n_init : nb;
    const int local_lo = nb - n_local > 0 ? nb - n_local : 0;
    const int cand_lo = init_hi;
    const int cand_hi = local_lo > cand_lo ? local_lo : cand_lo;
    const int n_cand = cand_hi - cand_lo;
    const int blk0 = tid * PER;                     // first block of this thread

    static_assert(EPB == 4 || EPB == 1, "entries per block");
    float score[PER];
    if constexpr (SOFTMAX) {
        // per-head softmax max / denominator from the chunk partials (<= 64 chunks
        // staged in LDS)
        const int used = EPB == 4 ? (int)((nc + kSoftmaxChunk - 1) / kSoftmaxChunk)
                                  : (int)((L / kBlock + kStatChunk - 1) / kStatChunk);
        if (used <= 64) {
            for (int i = tid; i < G * used; i += NT)
                s_st[i] = stats[((int64_t)unit * G + i / used) * n_chunks + i % used];
            __syncthreads();
        }
        if (tid < G) {
            float M = -INFINITY, Z = 0.f;
            const float2 *st = stats + ((int64_t)unit * G + tid) * n_chunks;
            for (int c = 0; c < used; ++c) {
                const float2 v = used <= 64 ? s_st[tid * used + c] : st[c];   // > 64: long contexts
                merge_ms(M, Z, v.x, v.y);
            }
            s_M[tid] = M;
            s_Zinv[tid] = Z > 0.f ? 1.f / Z : 0.f;
        }
        __syncthreads();
        if constexpr (EPB == 1) {
            // blocks blk0 .. blk0 + PER - 1, four at a time (rows padded to a
            // multiple of 4 blocks; nc_pad is the row stride)
#pragma unroll
            for (int q0 = 0; q0 < PER; q0 += 4) {
                float S[4] = {0.f, 0.f, 0.f, 0.f};
                bool any[4] = {false, false, false, false};
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                    if (blk0 + q0 < nc_pad)
                        v = *reinterpret_cast<const float4 *>(logits + ((int64_t)unit * G + h) * nc_pad +
                                                              blk0 + q0);
                    const float x[4] = {v.x, v.y, v.z, v.w};
                    const float Mh = s_M[h], Zi = s_Zinv[h];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (x[e] != -INFINITY) {
                            S[e] += hw_exp(x[e] - Mh) * Zi;
                            any[e] = true;
                        }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) score[q0 + e] = (blk0 + q0 + e < nb && any[e]) ? S[e] : -INFINITY;
            }
        } else {
        // entries 4*blk0 .. 4*blk0 + 4*PER - 1, eight blocks (32 entries) at a time
#pragma unroll
        for (int sub = 0; sub < PER; sub += 8) {
            float S[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) S[k] = 0.f;
            const int64_t j0 = 4 * (int64_t)(blk0 + sub);
#pragma unroll
            for (int g0 = 0; g0 < G; g0 += (G >= 8 ? 2 : (G < 4 ? G : 4))) {
                constexpr int GC = G >= 8 ? 2 : (G < 4 ? G : 4);   // heads per load group
                float4 lg[GC][8];
#pragma unroll
                for (int gg = 0; gg < GC; ++gg)
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        lg[gg][q] = (j0 + 4 * q < nc)
                                        ? *reinterpret_cast<const float4 *>(
                                              logits + ((int64_t)unit * G + g0 + gg) * nc_pad + j0 + 4 * q)
                                        : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
                for (int gg = 0; gg < GC; ++gg) {
                    const float Mg = s_M[g0 + gg], Zi = s_Zinv[g0 + gg];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        S[4 * q + 0] += hw_exp(lg[gg][q].x - Mg) * Zi;
                        S[4 * q + 1] += hw_exp(lg[gg][q].y - Mg) * Zi;
                        S[4 * q + 2] += hw_exp(lg[gg][q].z - Mg) * Zi;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float best = -INFINITY;
#pragma unroll
                for (int e = 0; e < 3; ++e)
                    if (j0 + 4 * q + e < nc) best = fmaxf(best, S[4 * q + e]);
                score[sub + q] = (blk0 + sub + q < nb) ? best : -INFINITY;
            }
        }
        }
    } else {
#pragma unroll
        for (int q = 0; q < PER; q += 4) {
            float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (blk0 + q + 3 < nb_cap)
                v = *reinterpret_cast<const float4 *>(bscore_in + (int64_t)unit * nb_cap + blk0 + q);
            else {
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    t[e] = (blk0 + q + e < nb_cap) ? bscore_in[(int64_t)unit * nb_cap + blk0 + q + e] : -INFINITY;
                v = make_float4(t[0], t[1], t[2], t[3]);
            }
            score[q] = v.x; score[q + 1] = v.y; score[q + 2] = v.z; score[q + 3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (blk0 + q >= nb) score[q] = -INFINITY;
    }
    uint32_t key[PER];
    bool cand[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int blk = blk0 + q;
        if (bscore_out && blk < nb_cap) bscore_out[(int64_t)unit * nb_cap + blk] = score[q];
        key[q] = orderable(score[q]);
        cand[q] = blk >= cand_lo && blk < cand_hi;
    }

    const bool take_all = top_k >= n_cand;
    const bool take_none = top_k <= 0;
    const bool choose = !take_all && !take_none;

    // Bin of histogram h that holds the `remaining`-th largest counted key
    // (bins scanned from the top), the count of keys in the bins above it and
    // the bin's own count.
    auto boundary_bin = [&](const uint32_t *h, int remaining) {
        if (tid < 64) {
            // lane l owns bins 4l .. 4l+3; keys in bins owned by higher lanes
            // = wave total - inclusive prefix over lanes 0..l
            const uint32_t hb[4] = {h[4 * tid], h[4 * tid + 1], h[4 * tid + 2], h[4 * tid + 3]};
            const uint32_t c = hb[0] + hb[1] + hb[2] + hb[3];
            const uint32_t incl = wave_incl_sum(c);
            uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
#pragma unroll
            for (int k = 3; k >= 0; --k) {
                if (above < (uint32_t)remaining && above + hb[k] >= (uint32_t)remaining) {
                    s_digit = 4 * tid + k;
                    s_above = above;
                    s_bcnt = hb[k];
                }
                above += hb[k];
            }
        }
        __syncthreads();
    };

    // Fast path (grids of many units, where the kernel is throughput bound;
    // with few units its longer chain of dependent steps costs more than the
    // radix passes it saves): 256 equal-width value buckets over the
    // candidates' [min, max].
    // A bucket index is a monotone function of the score (fp32 subtraction of
    // a constant and multiplication by a positive constant are monotone under
    // rounding), so every candidate in a bucket above the one holding the k-th
    // largest score is taken, and only that boundary bucket's candidates are
    // ranked exactly (score, then lower block id) in LDS. Degenerate ranges
    // (all scores equal, non-finite) and boundary buckets above kBoundaryCap
    // fall back to the radix select of the exact k-th key below.
    int bin[PER];
    bool fast = false;
    int bstar = 0;
    if (choose && use_buckets) {
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (cand[q]) {
                lo = fminf(lo, score[q]);
                hi = fmaxf(hi, score[q]);
            }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            lo = fminf(lo, shfl_xor(lo, off));
            hi = fmaxf(hi, shfl_xor(hi, off));
        }
        if ((tid & 63) == 0) {
            s_lo[tid >> 6] = lo;
            s_hi[tid >> 6] = hi;
        }
        for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
        for (int i = tid; i < kSelWords; i += NT) s_sel[i] = 0;
        if (tid == 0) s_nbnd = 0;
        __syncthreads();
        lo = s_lo[0];
        hi = s_hi[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) {
            lo = fminf(lo, s_lo[w]);
            hi = fmaxf(hi, s_hi[w]);
        }
        const float range = hi - lo;
        const float inv = 256.f / range;
        fast = range > 0.f && range <= FLT_MAX && inv <= FLT_MAX;   // same on every thread
        if (fast) {
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                int bq = -1;
                if (cand[q]) {
                    bq = (int)((score[q] - lo) * inv);
                    bq = bq < 0 ? 0 : (bq > 255 ? 255 : bq);
                    atomicAdd(&s_hist[bq], 1u);
                }
                bin[q] = bq;
            }
            __syncthreads();
            boundary_bin(s_hist, top_k);
            bstar = (int)s_digit;
            const int c = (int)s_bcnt;                      // the boundary bucket's count
            const int r = top_k - (int)s_above;             // taken from the boundary bucket, >= 1
            if (c <= kBoundaryCap) {
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    if (bin[q] == bstar) {
                        const uint32_t slot = atomicAdd(&s_nbnd, 1u);
                        s_bkey[slot] = key[q];
                        s_bblk[slot] = blk0 + q;
                    }
                __syncthreads();
                for (int i = tid; i < c; i += NT) {
                    const uint32_t ki = s_bkey[i];
                    const int bi = s_bblk[i];
                    int rank = 0;
                    for (int j = 0; j < c; ++j) {
                        const uint32_t kj = s_bkey[j];
                        rank += (kj > ki || (kj == ki && s_bblk[j] < bi)) ? 1 : 0;
                    }
                    if (rank < r) atomicOr(&s_sel[bi >> 5], 1u << (bi & 31));
                }
                __syncthreads();
            } else {
                fast = false;
            }
        }
    }

    // Fallback: radix select of the top_k-th largest key among the candidates,
    // 8-bit digits from the most significant bit in which the candidates'
    // keys differ (the bits above it are common to every candidate: those of
    // the smallest and largest key agree there). The passes stop early once
    // the boundary bin holds exactly the keys still to take: every key whose
    // digits so far match (prefix under mask) is then taken, so the classes
    // compared below are those of the masked key. A digit that reaches below
    // bit 0 starts at bit 0 instead; its upper bits are already fixed by the
    // prefix, so the bins stay in key order. Two histograms alternate, so a
    // pass clears the next pass's one and needs two barriers.
    uint32_t prefix = 0, mask = 0;
    int remaining = top_k;
    bool whole_class = false;           // every key of the boundary class is taken
    if (choose && !fast) {
        uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (cand[q]) {
                kmin = key[q] < kmin ? key[q] : kmin;
                kmax = key[q] > kmax ? key[q] : kmax;
            }
        kmin = wave_min_u32(kmin);
        kmax = wave_max_u32(kmax);
        if ((tid & 63) == 0) {
            s_kmin[tid >> 6] = kmin;
            s_kmax[tid >> 6] = kmax;
        }
        for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            kmin = s_kmin[w] < kmin ? s_kmin[w] : kmin;
            kmax = s_kmax[w] > kmax ? s_kmax[w] : kmax;
        }
        const uint32_t diff = kmin ^ kmax;               // same on every thread
        if (diff == 0u) {
            prefix = kmin;                               // one class: ranked by id below
            mask = ~0u;
        } else {
            const int hb = 31 - __builtin_clz(diff);     // highest differing bit
            mask = hb == 31 ? 0u : (~0u << (hb + 1));
            prefix = kmin & mask;
            int shift = hb - 7 > 0 ? hb - 7 : 0;
#pragma unroll 1
            for (int pass = 0;; ++pass) {
                uint32_t *h = (pass & 1) ? s_hist2 : s_hist;
                uint32_t *h_next = (pass & 1) ? s_hist : s_hist2;
                for (int i = tid; i < 256; i += NT) h_next[i] = 0;
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    if (cand[q] && (key[q] & mask) == prefix) atomicAdd(&h[(key[q] >> shift) & 255u], 1u);
                __syncthreads();
                boundary_bin(h, remaining);
                prefix |= s_digit << shift;
                mask |= 255u << shift;
                remaining -= (int)s_above;
                if ((int)s_bcnt == remaining) {
                    whole_class = true;
                    break;
                }
                if (shift == 0) break;
                shift = shift - 8 > 0 ? shift - 8 : 0;
            }
        }
    }
    const uint32_t thr = prefix;        // masked key of the k-th largest candidate
    const int take_eq = remaining;      // keys of thr's class taken, lowest ids first
    int rank = 0;
    if (choose && !fast && !whole_class) {
        int n_eq = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) n_eq += (cand[q] && key[q] == thr) ? 1 : 0;
        int unused;
        rank = wg_exclusive_scan<NT>(n_eq, s_wave, unused);
    }

    // ascending compaction over this thread's consecutive blocks
    bool in[PER];
    int n_in = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int blk = blk0 + q;
        bool x;
        if (blk >= nb) x = false;
        else if (blk < init_hi || blk >= local_lo) x = true;
        else if (take_none) x = false;
        else if (take_all) x = true;
        else if (fast) x = bin[q] > bstar || (bin[q] == bstar && ((s_sel[blk >> 5] >> (blk & 31)) & 1u));
        else if ((key[q] & mask) > thr) x = true;
        else if ((key[q] & mask) == thr) x = whole_class || rank++ < take_eq;
        else x = false;
        in[q] = x;
        n_in += x ? 1 : 0;
    }
    int total;
    int pos = wg_exclusive_scan<NT>(n_in, s_wave, total);
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (in[q]) {
            if (pos < idx_cap) row[pos] = blk0 + q;
            ++pos;
        }
    for (int i = total + tid; i < idx_cap; i += NT) row[i] = -1;
    if (tid == 0) *cnt_slot = total < idx_cap ? total : idx_cap;
}

}  // namespace sa
