// Token-level selection with one index shared by several layers.
//
// Pages: the CLSA abstract on "HySparse2: Hybrid Sparse Attention with
// Two-Level KV Sharing" (one indexer computes a top-k over individual tokens
// once; every layer that shares the KV cache reuses that index) and the JSSA
// item on the "Sparse Attention" topic page (tokens scored in a shared
// low-dimensional query-key space, a separate token set per KV head). The
// score is the raw form of Eq. 4 on the SparDA summary page ("Methodology",
// one vector per group and no softmax as in its "Compact Forecast Indexer"),
// taken against each token's index key Ki_t (the keys themselves, d_i = 128,
// or a 64-dimensional projection of them); the first n_init and last n_local
// visible tokens are always kept (the token counterpart of Eq. 1).
//
// Per (sequence b, KV head kvh) = unit, with T up to 128K tokens, one
// workgroup cannot hold the keys, so the exact top-k is a grid-wide radix
// select over 32-bit orderable keys, 8 bits per pass, with per-unit global
// histograms. Every kernel covers 4096 tokens of one unit per workgroup
// (grid: chunks x units):
//   tok_zero_kernel    clears the per-unit histograms (no memset: the call may
//                      be captured in a graph)
//   tok_score_kernel   scores every visible token with the group-summed
//                      selector (one index-key row per 16 or 8 lanes, fp32
//                      products, transposed DPP reduction), writes the keys
//                      of the candidates and counts their top 8 bits
//   tok_radix_kernel   passes 2..4: each workgroup re-derives the digits
//                      chosen so far from the histograms, then counts the
//                      next 8 bits of the keys that share that prefix
//   tok_count_kernel   the exact k-th key and how many keys equal to it are
//                      taken (ties to the lower token); per chunk the count of
//                      surely-taken tokens and of keys equal to the k-th
//   tok_write_kernel   ascending compaction: a chunk's tokens land after those
//                      of earlier chunks (prefix over the chunk counts), equal
//                      keys are taken in token order
// The keys pass (4 B per token) stays in the last-level cache between the
// passes; HBM traffic is dominated by the index-key scan.
#include <float.h>
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"
#include "tok_positions.h"

namespace sa {

constexpr int kTokThreads = 256;
constexpr int kTokChunk = 4096;                       // tokens per workgroup
constexpr int kTokPer = kTokChunk / kTokThreads;      // consecutive tokens per thread
constexpr int kTokPasses = 4;                         // 8-bit digits of a 32-bit key

TokenWorkspace token_workspace_layout(int B, int Hkv, int64_t T_cap) {
    TokenWorkspace w{};
    const int64_t units = (int64_t)B * Hkv;
    const int64_t chunks = (T_cap + kTokChunk - 1) / kTokChunk;
    w.n_chunks = (int)(chunks > 0 ? chunks : 1);      // chunk 0 always runs: it writes the counts
    w.t_pad = (int64_t)w.n_chunks * kTokChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    w.keys_off = take((size_t)units * w.t_pad * sizeof(uint32_t));
    w.hist_off = take((size_t)kTokPasses * units * 256 * sizeof(uint32_t));
    w.counts_off = take((size_t)units * w.n_chunks * 2 * sizeof(int32_t));
    w.info_off = take((size_t)units * 4 * sizeof(uint32_t));
    w.total = off;
    return w;
}

// Kept and candidate windows of a unit at visible length L.
struct TokWindows {
    int64_t L, init_hi, local_lo, n_cand;
    bool choose, take_all;
};
__device__ __forceinline__ TokWindows tok_windows(int64_t L, int top_k, int n_init, int n_local) {
    TokWindows w;
    w.L = L;
    w.init_hi = n_init < L ? n_init : L;
    const int64_t lo = L - n_local;
    w.local_lo = lo > w.init_hi ? lo : w.init_hi;
    w.n_cand = w.local_lo - w.init_hi;
    w.take_all = top_k >= w.n_cand;
    w.choose = !w.take_all && top_k > 0;
    return w;
}

// Wave 0 finds the bin of the 256-bin LDS histogram s_h that holds the
// `remaining`-th largest counted key (bins scanned from the top), the number
// of keys in the bins above it and the bin's own count (tok_digit_seq states
// the same search sequentially); every thread reads them after the barrier.
__device__ __forceinline__ void tok_digit(const uint32_t *s_h, int remaining, uint32_t *s_digit,
                                          uint32_t *s_above, uint32_t *s_bcnt) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        if (tid == 0) {                 // defined even if no bin qualifies (inconsistent counts)
            *s_digit = 0;
            *s_above = 0;
            *s_bcnt = 0xffffffffu;
        }
        const uint32_t hb[4] = {s_h[4 * tid], s_h[4 * tid + 1], s_h[4 * tid + 2], s_h[4 * tid + 3]};
        const uint64_t c = (uint64_t)hb[0] + hb[1] + hb[2] + hb[3];
        uint64_t incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint64_t t = __shfl_down(incl, off, 64);
            if (tid + off < 64) incl += t;
        }
        uint64_t above = incl - c;                   // keys in bins owned by higher lanes
#pragma unroll
        for (int k = 3; k >= 0; --k) {
            if (tok_bin_holds(above, hb[k], remaining)) {   // at most one bin of the whole wave
                *s_digit = 4 * tid + k;
                *s_above = (uint32_t)above;
                *s_bcnt = hb[k];
            }
            above += hb[k];
        }
    }
    __syncthreads();
}

// The digits chosen by the first `passes` passes of a unit: prefix (the chosen
// high bits), mask, and how many of the top_k remain to be found below them.
// The digits stop early (whole = true) once the boundary bin holds exactly the
// keys still to take: every key whose masked bits equal the prefix is then
// taken, and later passes have nothing to count.
__device__ __forceinline__ void tok_prefix(const uint32_t *hist_unit, int64_t hist_stride,
                                           int passes, int top_k, uint32_t *s_h, uint32_t *s_digit,
                                           uint32_t *s_above, uint32_t *s_bcnt, uint32_t &prefix,
                                           uint32_t &mask, int &remaining, bool &whole) {
    prefix = 0;
    mask = 0;
    remaining = top_k;
    whole = false;
    for (int p = 0; p < passes; ++p) {
        s_h[threadIdx.x] = hist_unit[p * hist_stride + threadIdx.x];   // 256 threads, 256 bins
        __syncthreads();
        tok_digit(s_h, remaining, s_digit, s_above, s_bcnt);
        const int shift = 24 - 8 * p;
        prefix |= *s_digit << shift;
        mask |= 255u << shift;
        remaining = tok_remaining_after(remaining, *s_above);
        const bool done = *s_bcnt == (uint32_t)remaining;              // same on every thread
        __syncthreads();                                               // s_h and the scalars reused
        if (done) {
            whole = true;
            break;
        }
    }
}

__global__ __launch_bounds__(kTokThreads) void tok_zero_kernel(uint32_t *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kTokThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kTokThreads)
        p[i] = 0u;
}

// ---------------------------------------------------------------- scores

// Index-key rows of DI elements: LPR = DI / 8 lanes per row, each lane 8
// elements (16 B for bf16). A row group of LPR lanes takes NR rows per
// iteration; the rows of one load instruction are consecutive across the
// wave's row groups (row = base + q * NG + group), so each instruction reads
// one contiguous span.
template <typename T, int DI>
struct TokScoreShape {
    static constexpr int LPR = DI / 8;
    static constexpr int NG = kTokThreads / LPR;                    // row groups per workgroup
    static constexpr int NR = (LPR == 16 && sizeof(T) == 2) ? 16 : 8;
    static constexpr int RPI = NG * NR;                              // rows per iteration
    static constexpr int ITERS = kTokChunk / RPI;
};

template <typename T, int DI>
__global__ __launch_bounds__(kTokThreads) void tok_score_kernel(
    const T *__restrict__ sel, int H_sel, int Gs, const T *__restrict__ Ki, int Hkv, int64_t T_cap,
    const int32_t *__restrict__ seq_lens, int top_k, int n_init, int n_local,
    uint32_t *__restrict__ keys, int64_t t_pad, uint32_t *__restrict__ hist1,
    float *__restrict__ scores_out) {
    using S = TokScoreShape<T, DI>;
    __shared__ uint32_t s_hist[256];
    const int unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int pos = tid & (S::LPR - 1), grp = tid / S::LPR;
    const TokWindows w = tok_windows(clamp_len(seq_lens[b], T_cap), top_k, n_init, n_local);
    const int64_t t0 = (int64_t)blockIdx.x * kTokChunk;
    if (t0 >= w.L) {                                   // no visible token in this chunk
        if (scores_out)
            for (int i = tid; i < kTokChunk; i += kTokThreads)
                if (t0 + i < T_cap) scores_out[(int64_t)unit * T_cap + t0 + i] = -INFINITY;
        return;
    }
    s_hist[tid] = 0;

    // group-summed selector slice of this lane (sum in head order, fp32)
    float s[8];
    {
        const T *sp = sel + ((int64_t)b * H_sel + (int64_t)kvh * Gs) * DI + pos * 8;
        load8(sp, s);
        for (int g = 1; g < Gs; ++g) {
            float x[8];
            load8(sp + (int64_t)g * DI, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = s[e] + x[e];
        }
    }
    constexpr uint32_t kRowBytes = DI * sizeof(T);
    // rows at or past L read as zeros (and are not counted)
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(Ki + (int64_t)unit * T_cap * DI,
                                                (uint32_t)(w.L * kRowBytes));
    const uint32_t lane_off = pos * 8 * sizeof(T);
    uint32_t *krow = keys + (int64_t)unit * t_pad;
    __syncthreads();                                   // s_hist cleared

#pragma unroll 1
    for (int it = 0; it < S::ITERS; ++it) {
        const int64_t base = t0 + (int64_t)it * S::RPI + grp;
        if (base >= w.L) break;                        // uniform per row group only: no barrier inside
        Raw8<T> r[S::NR];
#pragma unroll
        for (int q = 0; q < S::NR; ++q)
            load_raw_nt(rK, row_offset(base + (int64_t)q * S::NG, kRowBytes, lane_off), r[q]);
        float v[S::NR];
#pragma unroll
        for (int q = 0; q < S::NR; ++q) {
            float x[8];
            unpack(r[q], x);
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaf(s[e], x[e], a);
            v[q] = a;
        }
        // sum over the LPR lanes of each row: lane position pos ends with the
        // total of value vi (16 lanes, 16 values: vi = pos; 16 lanes, 8
        // values: vi = pos / 2, both lanes of a pair hold it; 8 lanes, 8
        // values: vi = pos)
        int vi;
        bool writer;
        if constexpr (S::LPR == 16) {
            transpose_reduce16<S::NR>(v, lane);
            vi = S::NR == 16 ? pos : (pos >> 1);
            writer = S::NR == 16 || (pos & 1) == 0;
        } else {
            transpose_reduce_step<1, S::NR, S::NR>(v, lane & 15);
            vi = pos;
            writer = true;
        }
        const int64_t t = base + (int64_t)vi * S::NG;
        if (writer && t < w.L) {
            const bool cand = t >= w.init_hi && t < w.local_lo;
            const uint32_t key = cand ? orderable(v[0]) : 0u;
            krow[t] = key;
            if (scores_out) scores_out[(int64_t)unit * T_cap + t] = v[0];
            if (cand && w.choose) atomicAdd(&s_hist[key >> 24], 1u);
        }
    }
    if (scores_out)
        for (int i = tid; i < kTokChunk; i += kTokThreads)
            if (t0 + i >= w.L && t0 + i < T_cap) scores_out[(int64_t)unit * T_cap + t0 + i] = -INFINITY;
    __syncthreads();
    if (w.choose && s_hist[tid] != 0) atomicAdd(&hist1[(int64_t)unit * 256 + tid], s_hist[tid]);
}

// ---------------------------------------------------------------- radix passes 2..4

// Loads this thread's kTokPer consecutive keys of the chunk and flags the
// candidates among them.
__device__ __forceinline__ void tok_load_keys(const uint32_t *krow, int64_t t0, const TokWindows &w,
                                              uint32_t (&key)[kTokPer], bool (&cand)[kTokPer]) {
    const int64_t tb = t0 + (int64_t)threadIdx.x * kTokPer;
    const uint4 *src = reinterpret_cast<const uint4 *>(krow + tb);
#pragma unroll
    for (int i = 0; i < kTokPer / 4; ++i) {
        const uint4 v = src[i];
        key[4 * i] = v.x; key[4 * i + 1] = v.y; key[4 * i + 2] = v.z; key[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
        const int64_t t = tb + i;
        cand[i] = t >= w.init_hi && t < w.local_lo;
    }
}

__global__ __launch_bounds__(kTokThreads) void tok_radix_kernel(
    int pass, int Hkv, int64_t T_cap, const int32_t *__restrict__ seq_lens, int top_k, int n_init,
    int n_local, const uint32_t *__restrict__ keys, int64_t t_pad, uint32_t *__restrict__ hist,
    int64_t hist_stride) {
    __shared__ uint32_t s_h[256];
    __shared__ uint32_t s_digit, s_above, s_bcnt;
    const int unit = blockIdx.y;
    const int b = unit / Hkv;
    const TokWindows w = tok_windows(clamp_len(seq_lens[b], T_cap), top_k, n_init, n_local);
    const int64_t t0 = (int64_t)blockIdx.x * kTokChunk;
    // uniform per workgroup: nothing to choose, or no candidate in the chunk
    if (!w.choose || t0 >= w.local_lo || t0 + kTokChunk <= w.init_hi) return;
    const uint32_t *hu = hist + (int64_t)unit * 256;
    uint32_t prefix, mask;
    int remaining;
    bool whole;
    tok_prefix(hu, hist_stride, pass, top_k, s_h, &s_digit, &s_above, &s_bcnt, prefix, mask,
               remaining, whole);
    if (whole) return;                                         // the set is already decided
    uint32_t key[kTokPer];
    bool cand[kTokPer];
    tok_load_keys(keys + (int64_t)unit * t_pad, t0, w, key, cand);
    s_h[threadIdx.x] = 0;
    __syncthreads();
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int i = 0; i < kTokPer; ++i)
        if (cand[i] && (key[i] & mask) == prefix) atomicAdd(&s_h[(key[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (s_h[threadIdx.x] != 0)
        atomicAdd(&hist[pass * hist_stride + (int64_t)unit * 256 + threadIdx.x], s_h[threadIdx.x]);
}

// ---------------------------------------------------------------- counts and compaction

// Taken here: the kept initial/local tokens, every candidate when top_k
// covers them all, else candidates whose key is above the exact k-th key; and
// keys equal to it in token order while take_eq lasts.
__global__ __launch_bounds__(kTokThreads) void tok_count_kernel(
    int Hkv, int64_t T_cap, const int32_t *__restrict__ seq_lens, int top_k, int n_init,
    int n_local, const uint32_t *__restrict__ keys, int64_t t_pad,
    const uint32_t *__restrict__ hist, int64_t hist_stride, int n_chunks,
    int32_t *__restrict__ counts, uint32_t *__restrict__ info) {
    __shared__ uint32_t s_h[256];
    __shared__ uint32_t s_digit, s_above, s_bcnt;
    __shared__ int s_red[2][kTokThreads / 64];
    const int unit = blockIdx.y;
    const int b = unit / Hkv;
    const TokWindows w = tok_windows(clamp_len(seq_lens[b], T_cap), top_k, n_init, n_local);
    const int64_t t0 = (int64_t)blockIdx.x * kTokChunk;
    if (t0 >= w.L) return;                                     // chunk never read
    uint32_t thr = 0, mask = 0xffffffffu;
    int take_eq = 0;
    bool whole = false;
    if (w.choose)
        tok_prefix(hist + (int64_t)unit * 256, hist_stride, kTokPasses, top_k, s_h, &s_digit,
                   &s_above, &s_bcnt, thr, mask, take_eq, whole);
    uint32_t key[kTokPer];
    bool cand[kTokPer];
    tok_load_keys(keys + (int64_t)unit * t_pad, t0, w, key, cand);
    int n_sure = 0, n_eq = 0;
    const int64_t tb = t0 + (int64_t)threadIdx.x * kTokPer;
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
        const int64_t t = tb + i;
        if (t >= w.L) continue;
        if (!cand[i]) ++n_sure;                                 // kept initial / local token
        else if (w.take_all || (w.choose && (key[i] & mask) > thr)) ++n_sure;
        else if (w.choose && (key[i] & mask) == thr) ++n_eq;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        n_sure += __shfl_xor(n_sure, off, 64);
        n_eq += __shfl_xor(n_eq, off, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_red[0][wave] = n_sure;
        s_red[1][wave] = n_eq;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int a = 0, e = 0;
        for (int k = 0; k < kTokThreads / 64; ++k) {
            a += s_red[0][k];
            e += s_red[1][k];
        }
        counts[((int64_t)unit * n_chunks + blockIdx.x) * 2] = a;
        counts[((int64_t)unit * n_chunks + blockIdx.x) * 2 + 1] = e;
        if (blockIdx.x == 0) {
            info[unit * 4] = thr;
            info[unit * 4 + 1] = (uint32_t)take_eq;
            info[unit * 4 + 2] = mask;
        }
    }
}

__global__ __launch_bounds__(kTokThreads) void tok_write_kernel(
    int Hkv, int64_t T_cap, const int32_t *__restrict__ seq_lens, int top_k, int n_init,
    int n_local, const uint32_t *__restrict__ keys, int64_t t_pad,
    const int32_t *__restrict__ counts, int n_chunks, const uint32_t *__restrict__ info,
    int32_t *__restrict__ idx_out, int idx_cap, int32_t *__restrict__ cnt_out) {
    __shared__ int s_wave[kTokThreads / 64];
    __shared__ int64_t s_red[2][kTokThreads / 64];
    const int unit = blockIdx.y;
    const int b = unit / Hkv;
    const int tid = threadIdx.x;
    const TokWindows w = tok_windows(clamp_len(seq_lens[b], T_cap), top_k, n_init, n_local);
    const int64_t t0 = (int64_t)blockIdx.x * kTokChunk;
    const int n_used = (int)((w.L + kTokChunk - 1) / kTokChunk);
    const uint32_t thr = w.choose ? info[unit * 4] : 0u;
    const uint32_t mask = w.choose ? info[unit * 4 + 2] : 0xffffffffu;
    const int take_eq = w.choose ? tok_take_eq(info[unit * 4 + 1]) : 0;
    int32_t *row = idx_out + (int64_t)unit * idx_cap;
    const int32_t *cu = counts + (int64_t)unit * n_chunks * 2;

    // sums over chunks [0, upto) of the surely-taken and the equal-key counts
    auto chunk_sums = [&](int upto, int64_t &sure, int64_t &eq) {
        int64_t a = 0, e = 0;
        for (int c = tid; c < upto; c += kTokThreads) {
            a += cu[2 * c];
            e += cu[2 * c + 1];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            a += __shfl_xor(a, off, 64);
            e += __shfl_xor(e, off, 64);
        }
        if ((tid & 63) == 0) {
            s_red[0][tid >> 6] = a;
            s_red[1][tid >> 6] = e;
        }
        __syncthreads();
        sure = 0;
        eq = 0;
        for (int k = 0; k < kTokThreads / 64; ++k) {
            sure += s_red[0][k];
            eq += s_red[1][k];
        }
        __syncthreads();
    };
    if (blockIdx.x == 0) {                                   // count and padding of the row
        int64_t sure, eq;
        chunk_sums(n_used, sure, eq);
        const int total = tok_row_total(sure, eq, take_eq, idx_cap);
        for (int i = total + tid; i < idx_cap; i += kTokThreads) row[i] = -1;
        if (tid == 0) cnt_out[unit] = total;
    }
    if (t0 >= w.L) return;
    int64_t sure_before, eq_before;
    chunk_sums((int)blockIdx.x, sure_before, eq_before);
    uint32_t key[kTokPer];
    bool cand[kTokPer];
    tok_load_keys(keys + (int64_t)unit * t_pad, t0, w, key, cand);
    const int64_t tb = t0 + (int64_t)tid * kTokPer;
    int n_eq = 0;
#pragma unroll
    for (int i = 0; i < kTokPer; ++i)
        n_eq += (w.choose && tb + i < w.L && cand[i] && (key[i] & mask) == thr) ? 1 : 0;
    int unused;
    int64_t eq_rank = eq_before + wg_exclusive_scan<kTokThreads>(n_eq, s_wave, unused);
    bool in[kTokPer];
    int n_in = 0;
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
        const int64_t t = tb + i;
        bool x;
        if (t >= w.L) x = false;
        else if (!cand[i]) x = true;
        else if (w.take_all) x = true;
        else if (!w.choose) x = false;
        else if ((key[i] & mask) > thr) x = true;
        else if ((key[i] & mask) == thr) x = eq_rank++ < take_eq;
        else x = false;
        in[i] = x;
        n_in += x ? 1 : 0;
    }
    int64_t pos = tok_first_pos(sure_before, eq_before, take_eq,
                                wg_exclusive_scan<kTokThreads>(n_in, s_wave, unused));
#pragma unroll
    for (int i = 0; i < kTokPer; ++i)
        if (in[i]) {
            if (tok_slot_ok(pos, idx_cap)) row[pos] = (int32_t)(tb + i);
            ++pos;
        }
}

template <typename T, int DI>
static void launch_tok_score(const void *sel, int H_sel, int Gs, const void *Ki, int B, int Hkv,
                             int64_t T_cap, const int32_t *seq_lens, int top_k, int n_init,
                             int n_local, const TokenWorkspace &w, char *ws, float *scores_out,
                             hipStream_t stream) {
    hipLaunchKernelGGL((tok_score_kernel<T, DI>), dim3((unsigned)w.n_chunks, (unsigned)(B * Hkv)),
                       dim3(kTokThreads), 0, stream, (const T *)sel, H_sel, Gs, (const T *)Ki, Hkv,
                       T_cap, seq_lens, top_k, n_init, n_local, (uint32_t *)(ws + w.keys_off),
                       w.t_pad, (uint32_t *)(ws + w.hist_off), scores_out);
}

int launch_token_select(const void *sel, int H_sel, const void *Ki, int dtype, int B, int Hkv,
                        int d_i, int64_t T_cap, const int32_t *seq_lens, int top_k, int n_init,
                        int n_local, int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                        float *scores_out, void *workspace, hipStream_t stream) {
    const TokenWorkspace w = token_workspace_layout(B, Hkv, T_cap);
    char *ws = (char *)workspace;
    const int units = B * Hkv;
    const int Gs = H_sel / Hkv;
    const int64_t hist_stride = (int64_t)units * 256;
    uint32_t *hist = (uint32_t *)(ws + w.hist_off);
    const int64_t n_hist = kTokPasses * hist_stride;
    const unsigned zero_blocks = (unsigned)((n_hist + kTokThreads - 1) / kTokThreads < 1024
                                                ? (n_hist + kTokThreads - 1) / kTokThreads : 1024);
    hipLaunchKernelGGL(tok_zero_kernel, dim3(zero_blocks), dim3(kTokThreads), 0, stream, hist, n_hist);
    if (dtype == SA_BF16) {
        if (d_i == 128)
            launch_tok_score<bf16_t, 128>(sel, H_sel, Gs, Ki, B, Hkv, T_cap, seq_lens, top_k, n_init,
                                          n_local, w, ws, scores_out, stream);
        else
            launch_tok_score<bf16_t, 64>(sel, H_sel, Gs, Ki, B, Hkv, T_cap, seq_lens, top_k, n_init,
                                         n_local, w, ws, scores_out, stream);
    } else {
        if (d_i == 128)
            launch_tok_score<float, 128>(sel, H_sel, Gs, Ki, B, Hkv, T_cap, seq_lens, top_k, n_init,
                                         n_local, w, ws, scores_out, stream);
        else
            launch_tok_score<float, 64>(sel, H_sel, Gs, Ki, B, Hkv, T_cap, seq_lens, top_k, n_init,
                                        n_local, w, ws, scores_out, stream);
    }
    const dim3 grid((unsigned)w.n_chunks, (unsigned)units);
    const uint32_t *keys = (const uint32_t *)(ws + w.keys_off);
    for (int pass = 1; pass < kTokPasses; ++pass)
        hipLaunchKernelGGL(tok_radix_kernel, grid, dim3(kTokThreads), 0, stream, pass, Hkv, T_cap,
                           seq_lens, top_k, n_init, n_local, keys, w.t_pad, hist, hist_stride);
    int32_t *counts = (int32_t *)(ws + w.counts_off);
    uint32_t *info = (uint32_t *)(ws + w.info_off);
    hipLaunchKernelGGL(tok_count_kernel, grid, dim3(kTokThreads), 0, stream, Hkv, T_cap, seq_lens,
                       top_k, n_init, n_local, keys, w.t_pad, (const uint32_t *)hist, hist_stride,
                       w.n_chunks, counts, info);
    hipLaunchKernelGGL(tok_write_kernel, grid, dim3(kTokThreads), 0, stream, Hkv, T_cap, seq_lens,
                       top_k, n_init, n_local, keys, w.t_pad, (const int32_t *)counts, w.n_chunks,
                       (const uint32_t *)info, idx_out, idx_cap, cnt_out);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
