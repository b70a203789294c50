// Block selection with a second-order block statistic.
//
// Page: the abstract on "CoSA: Accelerating Long-Context Inference via
// Proxy-Kernel Co-Designed Sparse Attention" (COBS): ranking blocks by
// attention mass, a cumulant expansion of that mass, and a compressed
// second-order statistic stored per block. The pages give no formula; the
// reading implemented here: for a query q and block B the log-mass is
// log 64 + q . mu_B + 1/2 q^T Sigma_B q + ..., and the stored statistic is the
// per-channel variance (the diagonal of Sigma_B), so a block's estimate is
//   q . mu_B + 1/2 sum_c q_c^2 var_{B,c}      (log 64 is common and dropped).
//
// Statistics (per complete 64-token block, in the key dtype): the fp64 mean
// and population variance of each channel over the block's 64 keys, each
// rounded once (to nearest, ties to even) to the key dtype. fp64 sums of 64
// bf16 or fp32 keys of ordinary range are exact, and the variance's are
// within about 2^-46 relative, so the stored values are those of the plain
// definition up to one unit in the last place (in practice identical).
// Layout [B, Hkv, nb_cap, 2, d]: mean row, then variance row.
//
// Kernels (HBM or latency bound; no matrix cores):
//   cobs_stats_kernel    four 16-lane row groups per block (one per quarter of
//                        16 keys), 8 channels per lane; the keys stay in
//                        registers for both passes, fp64 partial sums meet in
//                        LDS
//   cobs_score_kernel    one row group per block: the group's estimates for
//                        every selector head (fp32; bf16 mean terms by dot2
//                        products), reduced over the 16 lanes; exponentials on
//                        the hardware exp2.
//                        Raw-sum mode writes the sum over heads as the block
//                        score; softmax mode writes per-head logits and each
//                        chunk's (max, sum exp) per head
// The top-k and Eq. 1 union reuse the block path's top-k (in softmax mode it
// merges the chunk statistics and forms block score = sum over heads of each
// head's softmax over the blocks, the Eq. 6 form, from the logits), either as
// its own launch or inside the decode step's attention workgroups.
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"
#include "topk_device.h"

namespace sa {

constexpr int kCobsThreads = 256;
constexpr int kCobsGroups = kCobsThreads / kRowLanes;       // 16 blocks in flight per workgroup
constexpr int kCobsChunk = kStatChunk;                      // blocks per scoring workgroup

CobsWorkspace cobs_workspace_layout(int B, int Hkv, int G, int64_t T_cap, int score_mode) {
    CobsWorkspace w{};
    const int64_t units = (int64_t)B * Hkv;
    w.nb_cap = n_blocks(T_cap);
    w.n_chunks = (int)((w.nb_cap + kCobsChunk - 1) / kCobsChunk);
    if (w.n_chunks < 1) w.n_chunks = 1;
    w.nb_pad = (int64_t)w.n_chunks * kCobsChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    w.bscore_off = take((size_t)units * w.nb_cap * sizeof(float) + 4);
    if (score_mode == SA_SCORE_SOFTMAX_SUM) {
        w.logits_off = take((size_t)units * G * w.nb_pad * sizeof(float));
        w.stats_off = take((size_t)units * G * w.n_chunks * sizeof(float2));
    }
    w.total = off;
    return w;
}

// ---------------------------------------------------------------- statistics

// fp64 -> key dtype, one rounding to nearest with ties to even. bf16 keeps 8
// significant bits with fp32's exponent range: the spacing of bf16 values
// near x is 2^(e - 7) for 2^e <= |x| < 2^(e+1), and 2^-133 below 2^-126; x is
// scaled by the inverse spacing (exact), rounded to an integer (rint: ties to
// even) and scaled back, which is then exactly a bf16 value (or past the
// largest, which the fp32 conversion turns into an infinity).
__device__ __forceinline__ float round_once_key(double x, float *) { return (float)x; }
__device__ __forceinline__ float round_once_key(double x, bf16_t *) {
    int e = ilogb(x);
    e = (e < -126 ? -126 : e) - 7;
    return (float)ldexp(rint(ldexp(x, -e)), e);
}
template <typename T>
__device__ __forceinline__ void store_once(T *p, const double (&x)[8]) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = round_once_key(x[e], (T *)nullptr);
    store8(p, f);                           // exact: each value is already one of T
}

// Four row groups per block, one per quarter (16 consecutive keys); each keeps
// its 16 keys in registers, so the block is read once. Quarter sums (fp64)
// meet in LDS and give the block mean; then the quarter sums of squared
// deviations from it meet the same way.
constexpr int kStatsBlocksPerWG = kCobsGroups / 4;

template <typename T>
__global__ __launch_bounds__(kCobsThreads) void cobs_stats_kernel(
    const T *__restrict__ K, T *__restrict__ stats, int64_t T_cap, int64_t nb_cap,
    const int32_t *__restrict__ lens_prev, const int32_t *__restrict__ lens_now, int Hkv) {
    __shared__ double s_part[kStatsBlocksPerWG][4][kRowLanes][8];
    const int unit = blockIdx.y;
    const int b = unit / Hkv;
    const int lane16 = threadIdx.x & (kRowLanes - 1), group = threadIdx.x / kRowLanes;
    const int slot = group >> 2, quarter = group & 3;
    const int64_t L0 = clamp_len(lens_prev[b], T_cap), L1 = clamp_len(lens_now[b], T_cap);
    const int64_t lo = L0 / kBlock, hi = L1 / kBlock;       // complete blocks only
    const int64_t blk = lo + (int64_t)blockIdx.x * kStatsBlocksPerWG + slot;
    const bool valid = blk < hi && blk < nb_cap;            // uniform per row group
    const T *src = K + ((int64_t)unit * T_cap + blk * kBlock + quarter * 16) * kD + lane16 * kLaneElems;
    Raw8<T> r[16];
    double p[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
    if (valid) {
#pragma unroll
        for (int t = 0; t < 16; ++t) load_raw(src + (int64_t)t * kD, r[t]);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float x[8];
            unpack(r[t], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] += (double)x[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_part[slot][quarter][lane16][e] = p[e];
    __syncthreads();
    double m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        m[e] = ((s_part[slot][0][lane16][e] + s_part[slot][1][lane16][e]) +
                (s_part[slot][2][lane16][e] + s_part[slot][3][lane16][e])) * 0.015625;   // 2^-6, exact
    double q[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
    if (valid) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float x[8];
            unpack(r[t], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double dv = (double)x[e] - m[e];
                q[e] += dv * dv;
            }
        }
    }
    __syncthreads();                                        // every group has read the sums
#pragma unroll
    for (int e = 0; e < 8; ++e) s_part[slot][quarter][lane16][e] = q[e];
    __syncthreads();
    if (!valid || quarter != 0) return;
    double v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = ((s_part[slot][0][lane16][e] + s_part[slot][1][lane16][e]) +
                (s_part[slot][2][lane16][e] + s_part[slot][3][lane16][e])) * 0.015625;
    T *dst = stats + ((int64_t)unit * nb_cap + blk) * 2 * kD + lane16 * kLaneElems;
    store_once(dst, m);
    store_once(dst + kD, v);
}

// ---------------------------------------------------------------- scores

// Sum over the 16 lanes of a row with DPP. The partner sequence (quad xor 1,
// quad xor 2, half mirror, mirror) pairs only sums of equal terms, so every
// lane of the row ends with the same bits.
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppRowHalfMirror>(v);
    v += dpp<kDppRowMirror>(v);
    return v;
}

template <typename T, int G, bool SOFTMAX, int ORDER>
__global__ __launch_bounds__(kCobsThreads) void cobs_score_kernel(
    const T *__restrict__ sel, int H_sel, const T *__restrict__ stats, int64_t stats_nb,
    int Hkv, int64_t nb_cap, int64_t T_cap, const int32_t *__restrict__ seq_lens,
    float *__restrict__ bscore,
    float *__restrict__ logits, int64_t nb_pad, float2 *__restrict__ cstats, int n_chunks) {
    __shared__ float2 s_ms[kCobsGroups][G];
    const int unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int lane16 = threadIdx.x & (kRowLanes - 1), group = threadIdx.x / kRowLanes;
    const int64_t L = clamp_len(seq_lens[b], T_cap);
    const int64_t nbc = L / kBlock;                         // blocks with statistics
    const int64_t chunk0 = (int64_t)blockIdx.x * kCobsChunk;

    // selector slices: q_h and 1/2 q_h^2 for this lane's 8 channels (bf16:
    // q_h also as packed pairs for the mean term's dot2 products, which are
    // exact in fp32 and leave the mean row unconverted)
    constexpr bool kBf16 = sizeof(T) == 2;
    float qv[G][8], q2[G][8];
    uint32_t qp[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const T *qs = sel + ((int64_t)b * H_sel + (int64_t)kvh * G + h) * kD + lane16 * kLaneElems;
        load8(qs, qv[h]);
        if constexpr (kBf16) {
            const uint4 r = *reinterpret_cast<const uint4 *>(qs);
            qp[h][0] = r.x; qp[h][1] = r.y; qp[h][2] = r.z; qp[h][3] = r.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) q2[h][e] = 0.5f * (qv[h][e] * qv[h][e]);
    }
    float run_m[G], run_s[G];                               // this group's (max, sum exp) per head
#pragma unroll
    for (int h = 0; h < G; ++h) {
        run_m[h] = -INFINITY;
        run_s[h] = 0.f;
    }
    // the unit's statistics rows of blocks < nbc; rows past them read as zeros
    constexpr uint32_t kRowBytes = kD * sizeof(T);
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(stats + (int64_t)unit * stats_nb * 2 * kD,
                                                (uint32_t)(nbc * 2 * kRowBytes));
    const uint32_t lane_off = lane16 * kLaneElems * sizeof(T);
    constexpr int kPer = kCobsChunk / kCobsGroups;          // 16 blocks per row group
    constexpr int kBatch = G >= 8 ? 4 : 8;                 // blocks in flight per row group
#pragma unroll 1
    for (int i0 = 0; i0 < kPer; i0 += kBatch) {
        Raw8<T> mu[kBatch], va[kBatch];
        int64_t blk[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            blk[j] = chunk0 + (int64_t)(i0 + j) * kCobsGroups + group;
            load_raw_nt(rS, row_offset(2 * blk[j], kRowBytes, lane_off), mu[j]);
            if constexpr (ORDER == 2) load_raw_nt(rS, row_offset(2 * blk[j] + 1, kRowBytes, lane_off), va[j]);
        }
        float a[kBatch][G];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            float m8[8], v8[8];
            if constexpr (!kBf16) unpack(mu[j], m8);
            if constexpr (ORDER == 2) unpack(va[j], v8);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float acc = 0.f;
                if constexpr (kBf16) {
                    const uint4 &r = reinterpret_cast<const uint4 &>(mu[j]);
                    acc = dot2_bf16(qp[h][0], r.x, acc);
                    acc = dot2_bf16(qp[h][1], r.y, acc);
                    acc = dot2_bf16(qp[h][2], r.z, acc);
                    acc = dot2_bf16(qp[h][3], r.w, acc);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = fmaf(qv[h][e], m8[e], acc);
                }
                if constexpr (ORDER == 2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = fmaf(q2[h][e], v8[e], acc);
                }
                a[j][h] = row_sum16(acc);
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t k = blk[j];
            const bool has = k < nbc;
            if constexpr (!SOFTMAX) {
                float tot = a[j][0];
#pragma unroll
                for (int h = 1; h < G; ++h) tot += a[j][h];
                if (lane16 == 0 && k < nb_cap) bscore[(int64_t)unit * nb_cap + k] = has ? tot : -INFINITY;
            } else if (lane16 < G && k < nb_pad) {
                float v = a[j][0];
#pragma unroll
                for (int h = 1; h < G; ++h)
                    if (lane16 == h) v = a[j][h];
                logits[((int64_t)unit * G + lane16) * nb_pad + k] = has ? v : -INFINITY;
            }
        }
        if constexpr (SOFTMAX) {                            // one rescale per batch and head
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float bm = -INFINITY;
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    if (blk[j] < nbc) bm = fmaxf(bm, a[j][h]);
                if (bm == -INFINITY) continue;
                const float mn = fmaxf(run_m[h], bm);
                float ssum = run_m[h] == -INFINITY ? 0.f : run_s[h] * hw_exp(run_m[h] - mn);
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    if (blk[j] < nbc) ssum += hw_exp(a[j][h] - mn);
                run_m[h] = mn;
                run_s[h] = ssum;
            }
        }
    }
    if constexpr (SOFTMAX) {
        if (lane16 == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) s_ms[group][h] = make_float2(run_m[h], run_s[h]);
        }
        __syncthreads();
        if (threadIdx.x < G) {
            float2 r = s_ms[0][threadIdx.x];
            for (int g2 = 1; g2 < kCobsGroups; ++g2)
                merge_ms(r.x, r.y, s_ms[g2][threadIdx.x].x, s_ms[g2][threadIdx.x].y);
            cstats[((int64_t)unit * G + threadIdx.x) * n_chunks + blockIdx.x] = r;
        }
    }
}

// ---------------------------------------------------------------- launchers

int launch_cobs_stats(const void *K, void *stats, int dtype, int B, int Hkv, int64_t T_cap,
                      int64_t nb_cap, const int32_t *lens_prev, const int32_t *lens_now,
                      int32_t max_new_blocks, hipStream_t stream) {
    const dim3 grid((unsigned)((max_new_blocks + kStatsBlocksPerWG - 1) / kStatsBlocksPerWG),
                    (unsigned)(B * Hkv));
    if (dtype == SA_BF16)
        hipLaunchKernelGGL(cobs_stats_kernel<bf16_t>, grid, dim3(kCobsThreads), 0, stream,
                           (const bf16_t *)K, (bf16_t *)stats, T_cap, nb_cap, lens_prev, lens_now, Hkv);
    else
        hipLaunchKernelGGL(cobs_stats_kernel<float>, grid, dim3(kCobsThreads), 0, stream,
                           (const float *)K, (float *)stats, T_cap, nb_cap, lens_prev, lens_now, Hkv);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

template <typename T, int G>
static void launch_cobs_g(const void *sel, int H_sel, const void *stats, int64_t stats_nb, int B,
                          int Hkv, int64_t T_cap, const int32_t *seq_lens, const sa_select_params &p,
                          int order, float *bscore, const CobsWorkspace &w, char *ws,
                          hipStream_t stream) {
    const dim3 grid((unsigned)w.n_chunks, (unsigned)(B * Hkv));
    float *logits = (float *)(ws + w.logits_off);
    float2 *cst = (float2 *)(ws + w.stats_off);
#define SA_COBS(SM, ORD)                                                                          \
    hipLaunchKernelGGL((cobs_score_kernel<T, G, SM, ORD>), grid, dim3(kCobsThreads), 0, stream,    \
                       (const T *)sel, H_sel, (const T *)stats, stats_nb, Hkv, w.nb_cap, T_cap,     \
                       seq_lens, bscore, logits, w.nb_pad, cst, w.n_chunks)
    if (p.score_mode == SA_SCORE_SOFTMAX_SUM) {
        if (order == 2) SA_COBS(true, 2);
        else SA_COBS(true, 1);
    } else {
        if (order == 2) SA_COBS(false, 2);
        else SA_COBS(false, 1);
    }
#undef SA_COBS
}

int launch_cobs_select(const void *sel, int G, const void *stats, int64_t stats_nb, int dtype,
                       int B, int Hkv, int64_t T_cap, const int32_t *seq_lens,
                       const sa_select_params &p,
                       int order, int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                       float *block_scores_out, void *workspace, hipStream_t stream,
                       FusedSelect *fs) {
    const CobsWorkspace w = cobs_workspace_layout(B, Hkv, G, T_cap, p.score_mode);
    char *ws = (char *)workspace;
    const bool softmax = p.score_mode == SA_SCORE_SOFTMAX_SUM;
    // raw sum: the scorer writes block scores (to the caller's buffer when one
    // is given); softmax: the top-k forms them from the logits and writes them
    // out when asked
    float *bscore = (block_scores_out && !softmax) ? block_scores_out : (float *)(ws + w.bscore_off);
    const int H_sel = G * Hkv;
#define SA_COBS_CASE(GG)                                                                          \
    case GG:                                                                                      \
        if (dtype == SA_BF16)                                                                     \
            launch_cobs_g<bf16_t, GG>(sel, H_sel, stats, stats_nb, B, Hkv, T_cap, seq_lens, p,    \
                                      order, bscore, w, ws, stream);                              \
        else                                                                                      \
            launch_cobs_g<float, GG>(sel, H_sel, stats, stats_nb, B, Hkv, T_cap, seq_lens, p,     \
                                     order, bscore, w, ws, stream);                               \
        break;
    switch (G) {
        SA_COBS_CASE(1)
        SA_COBS_CASE(2)
        SA_COBS_CASE(4)
        SA_COBS_CASE(8)
        default: return SA_ERR_UNSUPPORTED;
    }
#undef SA_COBS_CASE
    float *logits = (float *)(ws + w.logits_off);
    const float2 *cst = (const float2 *)(ws + w.stats_off);
    if (fs) {                                       // the decode workgroups take the top-k
        fs->nb_cap = w.nb_cap;
        fs->top_k = p.top_k;
        fs->n_init = p.n_init;
        fs->n_local = p.n_local;
        fs->bscore = softmax ? nullptr : bscore;
        fs->logits = softmax ? logits : nullptr;
        fs->nc_pad = softmax ? w.nb_pad : 0;
        fs->stats = softmax ? cst : nullptr;
        fs->n_chunks = softmax ? w.n_chunks : 0;
        fs->idx_out = idx_out;
        fs->cnt_out = cnt_out;
        fs->use_buckets = B * Hkv >= kBucketMinUnits ? 1 : 0;
        fs->epb = 1;
    } else if (softmax) {
        launch_topk_block_softmax(B * Hkv, G, Hkv, T_cap, w.nb_cap, seq_lens, p, logits, w.nb_pad,
                                  cst, w.n_chunks, block_scores_out, idx_out, idx_cap, cnt_out,
                                  stream);
    } else {
        launch_topk_raw(B * Hkv, Hkv, T_cap, w.nb_cap, seq_lens, p, bscore, idx_out, idx_cap,
                        cnt_out, stream);
    }
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
