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
#include "score_raw_device.h"
#include "topk_device.h"

namespace sa {

constexpr int kSelThreads = 256;
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

template <typename T, bool APPEND>
__global__ __launch_bounds__(kSelThreads) void score_raw_kernel(
    const T *__restrict__ sel, int H_sel, int Gs, const T *__restrict__ Kc, int Hkv,
    int64_t nc_cap, int64_t T_cap, const int32_t *__restrict__ seq_lens, float *__restrict__ bscore,
    int64_t nb_cap, const T *__restrict__ K, T *__restrict__ Kc_w,
    const int32_t *__restrict__ lens_prev, int n_local, int app_mode) {
    score_raw_chunk<T, APPEND, kSelThreads / 16>(
        sel, H_sel, Gs, Kc, Hkv, nc_cap, T_cap, seq_lens, bscore, nb_cap, K, Kc_w, lens_prev,
        n_local, app_mode, (int)blockIdx.x, (int)blockIdx.y,
        APPEND && app_mode == kAppendColumn && blockIdx.x == gridDim.x - 1);
}

// ---------------------------------------------------------------- softmax scores

// APPEND (one-call decode step): entries completed between lens_prev and
// seq_lens are not read from Kc; they are formed from the keys (the append's
// arithmetic), written to Kc and scored in extra iterations after the main
// loop. A lane's new entries come after all of its old ones in the main loop's
// order, so every running (max, sum) sees the same values in the same order as
// with a separate append before the launch. bf16: the workgroup stages each
// new entry's 32 keys in LDS (two per row group, all in flight at once) and the
// row group that scores the entry sums them in token order, once, before the
// scoring iterations (formation inside the unrolled iteration would set the
// register count, and with it the occupancy, of every workgroup of the launch);
// the group takes the chunk's last new entry from LDS and earlier ones from its
// own stores. fp32: formed in the iteration from per-lane key loads.
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
    // bf16 appends: a new entry's 32 keys staged in LDS, the chunk's last new entry
    __shared__ uint4 s_rows[2 * kCmpStride][16];
    __shared__ uint4 s_last[16];
    int64_t j_last = -1;
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
                        T *kw = Kc_w + ((int64_t)unit * nc_cap + je) * kD + lane16 * kLaneElems;
                        if constexpr (sizeof(T) == 2) {          // formed before the iterations
                            if (je == j_last) r[e].v = s_last[lane16];
                            else load_raw(kw, r[e]);
                        } else {
                            compress_entry_raw(K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems, je, r[e]);
                            store_raw(kw, r[e]);
                        }
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
        if constexpr (sizeof(T) == 2) {
            const T *Ka = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
#pragma unroll 1
            for (int64_t j = a; j < z; ++j) {             // uniform per workgroup
                Raw8<T> rows[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) load_raw(Ka + (j * kCmpStride + 2 * group + i) * kD, rows[i]);
#pragma unroll
                for (int i = 0; i < 2; ++i) s_rows[2 * group + i][lane16] = rows[i].v;
                __syncthreads();
                if (group == (int)(((j - base) % PER_IT) / EPI)) {     // the group that scores entry j
                    Raw8<T> t;
                    entry_from_rows(s_rows, lane16, t);
                    store_raw(Kc_w + ((int64_t)unit * nc_cap + j) * kD + lane16 * kLaneElems, t);
                    if (j == z - 1) s_last[lane16] = t.v;
                }
                __syncthreads();                          // s_rows is refilled for the next entry
            }
            j_last = z - 1;
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
        // the step's append: with at most one new entry per unit (bf16) and
        // the attention launch next (fs), that launch's last split workgroup of
        // each unit writes it, in the shadow of its top-k (in the scoring
        // launch it made the unit's chunk-0 workgroup the last one: measured
        // ~2 us of tail at 128K); without fs the unit's first scoring
        // workgroup writes it; otherwise an extra column of scoring workgroups
        // does (which leaves the grid uneven over the CUs: ~2.4 us at 128K)
        const bool small = sizeof(T) == 2 && max_new_tokens <= kCmpStride;
        const int mode = small ? (fs ? kAppendElsewhere : kAppendInFirst) : kAppendColumn;
        if (fs && mode == kAppendElsewhere) {
            fs->app_K = K;
            fs->app_Kc = const_cast<void *>(Kc);
            fs->app_lens_prev = lens_prev;
            fs->app_nc_cap = nc_cap;
        }
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
        fs->app_K = nullptr;
        fs->app_Kc = nullptr;
        fs->app_lens_prev = nullptr;
        fs->app_nc_cap = 0;
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
