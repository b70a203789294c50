// Block selection: scoring of compressed keys, block aggregation, exact top-k
// and the union with the initial and local blocks.
//
// Page: "SparDA: Sparse Decoupled Attention for Efficient Long-Context LLM
// Inference" (picx.dev summary). Eq. 1 (union of init, local and top-k sets),
// Eq. 4 (raw scores of one Forecast vector per GQA group, "Compact Forecast
// Indexer": no per-head loop, no softmax) and Eq. 6 (the query-driven
// selector: sum over the G heads of a group of each head's softmax over the
// compressed entries).
//
// Kernels (all HBM or latency bound, no matrix cores: scoring is a
// matrix-vector product per group):
//   score_raw_kernel      RAW_SUM. The group's selector vectors are summed
//                         once, then every block's three inside entries
//                         (4b, 4b+1, 4b+2) are scored and max-reduced; the
//                         straddling entry 4b+3 belongs to no block and is not
//                         read. Writes one fp32 score per block.
//   score_softmax_kernel  SOFTMAX_SUM. G dot products per entry, written as
//                         fp32 logits, plus per 512-entry chunk and head the
//                         running (max, sum of exp) for the softmax denominator.
//   topk_kernel           one workgroup per (sequence, KV head): merges the
//                         chunk denominators, forms block scores, buckets the
//                         candidates by value (256 buckets over their range),
//                         ranks the boundary bucket exactly in LDS (a 4-pass
//                         8-bit radix select of the exact k-th (score, -index)
//                         key when the bucketing degenerates), and writes the
//                         union in ascending block order with a prefix scan.
#include <float.h>
#include <math.h>
#include <type_traits>

#include "compress_device.h"
#include "sa_device.h"
#include "sa_internal.h"
#include "topk_device.h"

namespace sa {

constexpr int kSelThreads = 256;
constexpr int kRawChunkBlocks = 256;                // blocks per workgroup (raw mode)
constexpr int kAppendColumn = 1;                    // the append as an extra column of workgroups
constexpr int kAppendInFirst = 2;                   // the append by each unit's first workgroup
constexpr int64_t kMaxTopkBlocks = 32768;           // 1024 threads x 32 blocks

SelectWorkspace select_workspace_layout(int B, int Hkv, int G, int64_t T_cap, int score_mode) {
    SelectWorkspace w{};
    const int64_t units = (int64_t)B * Hkv;
    const int64_t nc_cap = n_compressed(T_cap);
    w.n_chunks = (int)((nc_cap + kSoftmaxChunk - 1) / kSoftmaxChunk);
    w.nc_pad = (int64_t)w.n_chunks * kSoftmaxChunk;
    w.nb_cap = n_blocks(T_cap);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    if (score_mode == SA_SCORE_SOFTMAX_SUM) {
        w.logits_bytes = (size_t)units * G * w.nc_pad * sizeof(float);
        w.logits_off = take(w.logits_bytes);
        w.stats_bytes = (size_t)units * G * (w.n_chunks > 0 ? w.n_chunks : 1) * sizeof(float2);
        w.stats_off = take(w.stats_bytes);
    } else {
        w.bscore_bytes = (size_t)units * (w.nb_cap > 0 ? w.nb_cap : 1) * sizeof(float);
        w.bscore_off = take(w.bscore_bytes);
    }
    w.total = off;
    return w;
}

// ---------------------------------------------------------------- raw scores

template <typename T>
struct RawIter {                         // one iteration: 4 blocks x 3 inside entries per row group
    Raw8<T> r[12];
};

// APPEND: the launch has one more column of workgroups, which write the
// compressed entries completed between lens_prev and seq_lens (the decode
// step's append) while the other columns score. Scoring then reads only the
// entries that existed before (j < n_c(lens_prev)) from Kc and forms any newer
// entry it needs from K itself, with the same arithmetic, so it never depends
// on the concurrent writes.
template <typename T, bool APPEND>
__global__ __launch_bounds__(kSelThreads) void score_raw_kernel(
    const T *__restrict__ sel, int H_sel, int Gs, const T *__restrict__ Kc, int Hkv,
    int64_t nc_cap, int64_t T_cap, const int32_t *__restrict__ seq_lens, float *__restrict__ bscore,
    int64_t nb_cap, const T *__restrict__ K, T *__restrict__ Kc_w,
    const int32_t *__restrict__ lens_prev, int n_local, int app_mode) {
    const int unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int64_t L = clamp_len(seq_lens[b], T_cap);
    const int64_t nc = n_compressed(L);
    const int lane = threadIdx.x & 63;
    const int lane16 = threadIdx.x & 15;
    const int group = threadIdx.x >> 4;                 // 0..15
    constexpr uint32_t kRowBytes = kD * sizeof(T);
    int64_t nc_old = nc;                                // entries readable from Kc
    if constexpr (APPEND) {
        int64_t Lp = lens_prev[b];
        Lp = Lp < 0 ? 0 : (Lp > L ? L : Lp);
        nc_old = n_compressed(Lp);
        if (app_mode == kAppendColumn && blockIdx.x == gridDim.x - 1) {   // the append column
            const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
            T *Kcu = Kc_w + (int64_t)unit * nc_cap * kD + lane16 * kLaneElems;
            for (int64_t j = nc_old + group; j < nc; j += 16) {   // few keys in flight
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
    const int64_t chunk0 = (int64_t)blockIdx.x * kRawChunkBlocks;
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

    // iterations of 64 blocks; the next iteration's rows are in flight while
    // the current ones are reduced (sched_barrier keeps the prefetch in place)
    constexpr int kIters = kRawChunkBlocks / 64;
#pragma unroll
    for (int it = 0; it < kIters; it += 2) {
        const int64_t b0 = chunk0 + it * 64 + group * 4;
        if (it + 1 < kIters) issue(bufB, b0 + 64);
        __builtin_amdgcn_sched_barrier(0);
        process(bufA, b0);
        if (it + 1 < kIters) {
            if (it + 2 < kIters) issue(bufA, b0 + 128);
            __builtin_amdgcn_sched_barrier(0);
            process(bufB, b0 + 64);
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
                const int64_t b0 = chunk0 + it * 64 + group * 4;
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
    // kAppendInFirst (bf16, chosen when the caller expects at most one new
    // entry per unit): after its own blocks, the unit's first workgroup loads
    // the new entry's 32 keys (two per row group, all in flight at once),
    // stages them in LDS and one row group sums them in token order. (Loads
    // issued before the main loop, under a condition, cost the loop its exact
    // wait counts.) If the length grew by more than expected, the workgroup
    // forms every new entry one row group at a time, so Kc never has gaps.
    constexpr bool kInFirst = APPEND && sizeof(T) == 2;
    if constexpr (kInFirst) {
        if (app_mode == kAppendInFirst && blockIdx.x == 0 && nc_old + 1 < nc) {   // uniform
            const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
            T *Kcu = Kc_w + (int64_t)unit * nc_cap * kD + lane16 * kLaneElems;
            for (int64_t j = nc_old + group; j < nc; j += 16) {
                Raw8<T> r;
                compress_entry_raw(Ku, j, r);
                store_raw(Kcu + j * kD, r);
            }
        } else if (app_mode == kAppendInFirst && blockIdx.x == 0 && nc_old < nc) {
            __shared__ uint4 s_rows[2 * kCmpStride][16];
            const T *Ka = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
            Raw8<T> app_rows[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                load_raw(Ka + (nc_old * kCmpStride + 2 * group + i) * kD, app_rows[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) s_rows[2 * group + i][lane16] = app_rows[i].v;
            __syncthreads();
            if (group == 0) {
                Raw8<T> e;
                entry_from_rows(s_rows, lane16, e);
                store_raw(Kc_w + ((int64_t)unit * nc_cap + nc_old) * kD + lane16 * kLaneElems, e);
            }
        }
    }
}

// ---------------------------------------------------------------- softmax scores

// APPEND (one-call decode step): entries completed between lens_prev and
// seq_lens are not read from Kc; the group that owns such an entry forms it
// from the keys (the append's arithmetic), writes it to Kc and scores it in
// extra iterations after the main loop. A lane's new entries come after all of
// its old ones in the main loop's order, so every running (max, sum) sees the
// same values in the same order as with a separate append before the launch.
template <typename T, int G, bool APPEND>
__global__ __launch_bounds__(kSelThreads) void score_softmax_kernel(
    const T *__restrict__ sel, int H_sel, const T *__restrict__ Kc, int Hkv, int64_t nc_cap,
    int64_t T_cap, const int32_t *__restrict__ seq_lens, float *__restrict__ logits, int64_t nc_pad,
    float2 *__restrict__ stats, int n_chunks, const T *__restrict__ K, T *__restrict__ Kc_w,
    const int32_t *__restrict__ lens_prev) {
    constexpr int EPI = 16 / G;                         // entries per row group per iteration
    constexpr int PER_IT = 16 * EPI;                     // entries per workgroup iteration
    __shared__ float2 s_ms[4][G];
    const int unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int64_t L = clamp_len(seq_lens[b], T_cap);
    const int64_t nc = n_compressed(L);
    int64_t nc_old = nc;                                // entries readable from Kc
    if constexpr (APPEND) {
        int64_t Lp = lens_prev[b];
        Lp = Lp < 0 ? 0 : (Lp > L ? L : Lp);
        nc_old = n_compressed(Lp);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lane16 = threadIdx.x & 15;
    const int group = threadIdx.x >> 4;
    float q[G][8];
    {
        const T *sp = sel + ((int64_t)b * H_sel + (int64_t)kvh * G) * kD + lane16 * kLaneElems;
#pragma unroll
        for (int g = 0; g < G; ++g) load8(sp + (int64_t)g * kD, q[g]);
    }
    const T *Kcu = Kc + (int64_t)unit * nc_cap * kD + lane16 * kLaneElems;
    const int my_e = lane16 / G, my_g = lane16 % G;     // value this lane ends up holding
    float *lrow = logits + ((int64_t)unit * G + my_g) * nc_pad;
    float m = -INFINITY, ssum = 0.f;
    const int64_t base = (int64_t)blockIdx.x * kSoftmaxChunk;
    // one iteration: dot products, reduction, online update over the entries
    // read from Kc (below nc_old) or, with FORM, the new ones formed from the keys
    // bf16 with a single new entry: its 32 keys staged in LDS (see below)
    __shared__ uint4 s_rows[2 * kCmpStride][16];
    const bool one_new = APPEND && nc == nc_old + 1;
    auto iteration = [&](int it, auto form) {
        constexpr bool FORM = decltype(form)::value;
        auto live = [&](int64_t je) { return FORM ? (je >= nc_old && je < nc) : je < nc_old; };
        const int64_t j0 = base + it * PER_IT + group * EPI;
        Raw8<T> r[EPI];
#pragma unroll
        for (int e = 0; e < EPI; ++e) {
            const int64_t je = j0 + e;
            if (live(je)) {
                if constexpr (APPEND) {
                    if constexpr (FORM) {
                        const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
                        if constexpr (sizeof(T) == 2) {
                            if (one_new) entry_from_rows(s_rows, lane16, r[e]);
                            else compress_entry_raw(Ku, je, r[e]);
                        } else {
                            compress_entry_raw(Ku, je, r[e]);
                        }
                        store_raw(Kc_w + ((int64_t)unit * nc_cap + je) * kD + lane16 * kLaneElems, r[e]);
                        continue;
                    }
                }
                load_raw(Kcu + je * kD, r[e]);
            }
        }
        float v[16];
#pragma unroll
        for (int e = 0; e < EPI; ++e) {
            float x[8];
            if (live(j0 + e)) unpack(r[e], x);
            else {
#pragma unroll
                for (int c = 0; c < 8; ++c) x[c] = 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc = fmaf(q[g][c], x[c], acc);
                v[e * G + g] = acc;
            }
        }
        transpose_reduce16<16>(v, lane);
        const int64_t j = j0 + my_e;
        if (live(j)) {
            const float x = v[0];
            lrow[j] = x;
            if (x > m) {
                ssum = ssum * hw_exp(m - x) + 1.f;
                m = x;
            } else {
                ssum += hw_exp(x - m);
            }
        }
    };
#pragma unroll 1
    for (int it = 0; it < kSoftmaxChunk / PER_IT; ++it) iteration(it, std::false_type{});
    if constexpr (APPEND) {
        // the iterations of this chunk that hold new entries (uniform per workgroup)
        const int64_t a = nc_old > base ? nc_old : base;
        const int64_t z = nc < base + kSoftmaxChunk ? nc : base + kSoftmaxChunk;
        // bf16, one new entry: the workgroup loads its 32 keys (two per row
        // group, all in flight at once) into LDS, and the owning group sums
        // them in token order (per-lane loads of all 32 would wait in turn)
        if constexpr (sizeof(T) == 2) {
            if (a < z && one_new) {                      // uniform per workgroup
                const T *Ka = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
                Raw8<T> rows[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    load_raw(Ka + (nc_old * kCmpStride + 2 * group + i) * kD, rows[i]);
#pragma unroll
                for (int i = 0; i < 2; ++i) s_rows[2 * group + i][lane16] = rows[i].v;
                __syncthreads();
            }
        }
#pragma unroll 1
        for (int it = (int)((a - base) / PER_IT); a < z && it <= (int)((z - 1 - base) / PER_IT); ++it)
            iteration(it, std::true_type{});
    }
    // merge (max, sum) over lanes holding the same head: lane bits >= log2(G)
#pragma unroll
    for (int bit = G; bit < 64; bit <<= 1) {
        const float m2 = shfl_xor(m, bit);
        const float s2 = shfl_xor(ssum, bit);
        merge_ms(m, ssum, m2, s2);
    }
    if (lane < G) s_ms[wave][lane] = make_float2(m, ssum);
    __syncthreads();
    if (threadIdx.x < G) {
        float2 a = s_ms[0][threadIdx.x];
        for (int w = 1; w < 4; ++w) merge_ms(a.x, a.y, s_ms[w][threadIdx.x].x, s_ms[w][threadIdx.x].y);
        stats[((int64_t)unit * G + threadIdx.x) * n_chunks + blockIdx.x] = a;
    }
}

// ---------------------------------------------------------------- top-k + union

template <int G, bool SOFTMAX, int NT, int PER, int EPB>
__global__ __launch_bounds__(NT) void topk_kernel(
    int Hkv, int64_t T_cap, int64_t nb_cap, const int32_t *__restrict__ seq_lens, int top_k,
    int n_init, int n_local, const float *__restrict__ logits, int64_t nc_pad,
    const float2 *__restrict__ stats, int n_chunks, const float *__restrict__ bscore_in,
    float *__restrict__ bscore_out, int32_t *__restrict__ idx_out, int idx_cap,
    int32_t *__restrict__ cnt_out, int use_buckets) {
    const int unit = blockIdx.x;
    topk_unit<G, SOFTMAX, NT, PER, EPB>(unit, Hkv, T_cap, nb_cap, seq_lens, top_k, n_init, n_local,
                                   logits, nc_pad, stats, n_chunks, bscore_in, bscore_out,
                                   idx_out + (int64_t)unit * idx_cap, idx_cap, cnt_out + unit,
                                   use_buckets);
}

// Launch shape for the block count: keys of PER consecutive blocks per thread.
template <int G, bool SOFTMAX, int EPB = 4>
static void launch_topk(int n_units, int Hkv, int64_t T_cap, int64_t nb_cap, const int32_t *seq_lens,
                        const sa_select_params &p, const float *logits, int64_t nc_pad,
                        const float2 *stats, int n_chunks, const float *bscore, float *bs_out,
                        int32_t *idx_out, int idx_cap, int32_t *cnt_out, hipStream_t stream) {
    const int use_buckets = n_units >= kBucketMinUnits ? 1 : 0;
#define SA_TOPK(NT, PER)                                                                          \
    hipLaunchKernelGGL((topk_kernel<G, SOFTMAX, NT, PER, EPB>), dim3((unsigned)n_units), dim3(NT), 0, \
                       stream, Hkv, T_cap, nb_cap, seq_lens, p.top_k, p.n_init, p.n_local, logits, \
                       nc_pad, stats, n_chunks, bscore, bs_out, idx_out, idx_cap, cnt_out,          \
                       use_buckets)
    if (nb_cap <= 256 * 8) SA_TOPK(256, 8);
    else if (nb_cap <= 1024 * 8) SA_TOPK(1024, 8);
    else SA_TOPK(1024, 32);
#undef SA_TOPK
}

// Top-k + union over precomputed raw block scores, one workgroup per unit
// (used by the prefill path: a unit is one (query, KV head) there, with its
// own visible length in seq_lens).
void launch_topk_raw(int n_units, int Hkv, int64_t T_cap, int64_t nb_cap, const int32_t *seq_lens,
                     const sa_select_params &p, const float *bscore, int32_t *idx_out, int idx_cap,
                     int32_t *cnt_out, hipStream_t stream) {
    launch_topk<1, false>(n_units, Hkv, T_cap, nb_cap, seq_lens, p, nullptr, 0, nullptr, 0, bscore,
                          nullptr, idx_out, idx_cap, cnt_out, stream);
}

// Top-k + union over per-head logits of whole blocks (one logit per block and
// head, chunk partials of kStatChunk blocks): the second-order selection.
void launch_topk_block_softmax(int n_units, int G, int Hkv, int64_t T_cap, int64_t nb_cap,
                               const int32_t *seq_lens, const sa_select_params &p,
                               const float *logits, int64_t nb_pad, const float2 *stats,
                               int n_chunks, float *bs_out, int32_t *idx_out, int idx_cap,
                               int32_t *cnt_out, hipStream_t stream) {
#define SA_TBS(GG)                                                                                \
    launch_topk<GG, true, 1>(n_units, Hkv, T_cap, nb_cap, seq_lens, p, logits, nb_pad, stats,     \
                             n_chunks, nullptr, bs_out, idx_out, idx_cap, cnt_out, stream)
    if (G == 1) SA_TBS(1);
    else if (G == 2) SA_TBS(2);
    else if (G == 4) SA_TBS(4);
    else SA_TBS(8);
#undef SA_TBS
}

template <typename T, int G>
static void launch_softmax(const void *sel, int H_sel, const void *Kc, int B, int Hkv, int64_t T_cap,
                           int64_t nc_cap, const int32_t *seq_lens, const sa_select_params &p,
                           int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out, float *bs_out,
                           const SelectWorkspace &w, char *ws, hipStream_t stream,
                           FusedSelect *fs, const void *K = nullptr,
                           const int32_t *lens_prev = nullptr) {
    float *logits = (float *)(ws + w.logits_off);
    float2 *stats = (float2 *)(ws + w.stats_off);
    const unsigned units = (unsigned)(B * Hkv);
    if (w.n_chunks > 0) {
        if (lens_prev)                                  // scoring + the step's append
            hipLaunchKernelGGL((score_softmax_kernel<T, G, true>), dim3((unsigned)w.n_chunks, units),
                               dim3(kSelThreads), 0, stream, (const T *)sel, H_sel, (const T *)Kc,
                               Hkv, nc_cap, T_cap, seq_lens, logits, w.nc_pad, stats, w.n_chunks,
                               (const T *)K, (T *)Kc, lens_prev);
        else
            hipLaunchKernelGGL((score_softmax_kernel<T, G, false>), dim3((unsigned)w.n_chunks, units),
                               dim3(kSelThreads), 0, stream, (const T *)sel, H_sel, (const T *)Kc,
                               Hkv, nc_cap, T_cap, seq_lens, logits, w.nc_pad, stats, w.n_chunks,
                               (const T *)nullptr, (T *)nullptr, (const int32_t *)nullptr);
    }
    if (fs) {
        fs->logits = logits;
        fs->nc_pad = w.nc_pad;
        fs->stats = stats;
        fs->n_chunks = w.n_chunks;
        return;
    }
    launch_topk<G, true>(B * Hkv, Hkv, T_cap, w.nb_cap, seq_lens, p, logits, w.nc_pad, stats,
                         w.n_chunks, nullptr, bs_out, idx_out, idx_cap, cnt_out, stream);
}

template <typename T>
static void launch_raw(const void *sel, int H_sel, int Gs, const void *Kc, int B, int Hkv,
                       int64_t T_cap, int64_t nc_cap, const int32_t *seq_lens,
                       const sa_select_params &p, int32_t *idx_out, int32_t idx_cap,
                       int32_t *cnt_out, float *bs_out, const SelectWorkspace &w, char *ws,
                       hipStream_t stream, const void *K = nullptr,
                       const int32_t *lens_prev = nullptr, FusedSelect *fs = nullptr,
                       int32_t max_new_tokens = 1 << 30) {
    float *bscore = (float *)(ws + w.bscore_off);
    const unsigned units = (unsigned)(B * Hkv);
    const unsigned chunks = (unsigned)((w.nb_cap + kRawChunkBlocks - 1) / kRawChunkBlocks);
    if (lens_prev) {
        // scoring + the step's append in one launch: with at most one new entry
        // per unit (bf16) the unit's first workgroup writes it; otherwise an
        // extra column of workgroups does (which leaves the grid uneven over the
        // CUs: measured ~2.4 us at 128K)
        const int mode = (sizeof(T) == 2 && max_new_tokens <= kCmpStride) ? kAppendInFirst
                                                                           : kAppendColumn;
        const unsigned cols = chunks + (mode == kAppendColumn ? 1 : 0);
        hipLaunchKernelGGL((score_raw_kernel<T, true>), dim3(cols, units), dim3(kSelThreads), 0,
                           stream, (const T *)sel, H_sel, Gs, (const T *)Kc, Hkv, nc_cap, T_cap,
                           seq_lens, bscore, w.nb_cap, (const T *)K, (T *)Kc, lens_prev, p.n_local,
                           mode);
    } else if (chunks > 0)
        hipLaunchKernelGGL((score_raw_kernel<T, false>), dim3(chunks, units), dim3(kSelThreads), 0,
                           stream, (const T *)sel, H_sel, Gs, (const T *)Kc, Hkv, nc_cap, T_cap,
                           seq_lens, bscore, w.nb_cap, (const T *)nullptr, (T *)nullptr,
                           (const int32_t *)nullptr, 0, 0);
    if (fs) {
        fs->bscore = bscore;
        return;
    }
    launch_topk<1, false>(B * Hkv, Hkv, T_cap, w.nb_cap, seq_lens, p, nullptr, 0, nullptr, 0,
                          bscore, bs_out, idx_out, idx_cap, cnt_out, stream);
}

int launch_select(const void *sel, int G, const void *Kc, int dtype, int B, int Hkv,
                  int64_t T_cap, int64_t nc_cap, const int32_t *seq_lens,
                  const sa_select_params &p, int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                  float *block_scores_out, void *workspace, hipStream_t stream, const void *K,
                  const int32_t *lens_prev, FusedSelect *fs, int32_t max_new_tokens) {
    const SelectWorkspace w = select_workspace_layout(B, Hkv, G, T_cap, p.score_mode);
    if (w.nb_cap > kMaxTopkBlocks) return SA_ERR_UNSUPPORTED;
    char *ws = (char *)workspace;
    const int H_sel = G * Hkv;
    if (fs) {
        fs->nb_cap = w.nb_cap;
        fs->top_k = p.top_k;
        fs->n_init = p.n_init;
        fs->n_local = p.n_local;
        fs->bscore = nullptr;
        fs->logits = nullptr;
        fs->stats = nullptr;
        fs->nc_pad = 0;
        fs->n_chunks = 0;
        fs->idx_out = idx_out;
        fs->cnt_out = cnt_out;
        fs->use_buckets = B * Hkv >= kBucketMinUnits ? 1 : 0;
        fs->epb = 4;
    }
    if (p.score_mode == SA_SCORE_RAW_SUM) {
        if (dtype == SA_BF16)
            launch_raw<bf16_t>(sel, H_sel, G, Kc, B, Hkv, T_cap, nc_cap, seq_lens, p, idx_out, idx_cap,
                               cnt_out, block_scores_out, w, ws, stream, K, lens_prev, fs,
                               max_new_tokens);
        else
            launch_raw<float>(sel, H_sel, G, Kc, B, Hkv, T_cap, nc_cap, seq_lens, p, idx_out, idx_cap,
                              cnt_out, block_scores_out, w, ws, stream, K, lens_prev, fs,
                              max_new_tokens);
    } else {
#define SA_SOFTMAX_CASE(GG)                                                                       \
    case GG:                                                                                      \
        if (dtype == SA_BF16)                                                                     \
            launch_softmax<bf16_t, GG>(sel, H_sel, Kc, B, Hkv, T_cap, nc_cap, seq_lens, p, idx_out, \
                                       idx_cap, cnt_out, block_scores_out, w, ws, stream, fs, K,  \
                                       lens_prev);                                                \
        else                                                                                      \
            launch_softmax<float, GG>(sel, H_sel, Kc, B, Hkv, T_cap, nc_cap, seq_lens, p, idx_out,  \
                                      idx_cap, cnt_out, block_scores_out, w, ws, stream, fs, K,   \
                                      lens_prev);                                                 \
        break;
        switch (G) {
            SA_SOFTMAX_CASE(1)
            SA_SOFTMAX_CASE(2)
            SA_SOFTMAX_CASE(4)
            SA_SOFTMAX_CASE(8)
            default: return SA_ERR_UNSUPPORTED;
        }
#undef SA_SOFTMAX_CASE
    }
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
