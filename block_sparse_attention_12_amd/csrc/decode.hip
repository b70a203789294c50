// Gathered split-K sparse decode attention (Eq. 5 of the SparDA summary page,
// "Methodology": the attention query attends only to the keys and values of the
// selected blocks).
//
// Work unit: (sequence b, KV head kvh, split s). The unit's selected blocks
// idx[b, kvh, 0..cnt) are divided into n_split contiguous shares; each
// 256-thread workgroup streams its share's K and V blocks (64 rows x 256 B
// each for bf16, contiguous in HBM) once and serves all G query heads of the
// group from that single read (attend_device.h: GQA packing for G = 1, 2, 4
// or 8, both products on the matrix cores for bf16 block lists, online
// softmax without workgroup barriers inside the block loop).
//
// Split merge: every workgroup writes (max, sum, weighted values) for its G
// heads with device-scope stores and counts itself in its unit's counter word
// (handoff_device.h); the unit's last workgroup merges the n_split partials
// with log-sum-exp weights and writes O and LSE. No second launch and no
// cache-writeback fence (a release fence per workgroup would write back the
// die's L2: measured, it serialised the grid). With n_split = 1 the workgroup
// writes O directly.
#include <math.h>

#include "attend_device.h"
#include "compress_device.h"
#include "handoff_device.h"
#include "sa_device.h"
#include "sa_internal.h"
#include "topk_device.h"

namespace sa {

constexpr int kDecThreads = 256;
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

// workspace: the split partials [B * Hq][n_split][kPartStride] fp32, then the
// hand-off words: [0] epoch, [1] units merged, [2 + unit] the unit's arrivals
__host__ __device__ static inline size_t partial_bytes(int B, int Hq, int32_t n_split) {
    return ((size_t)B * Hq * n_split * kPartStride * sizeof(float) + 255) & ~(size_t)255;
}
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int32_t n_split) {
    if (n_split <= 1) return 0;
    return partial_bytes(B, Hq, n_split) + (2 + (size_t)B * Hkv) * sizeof(uint64_t);
}

// The last workgroup of a unit: merges the unit's n_split partial rows (read
// with device-scope loads, eight splits at a time with all their loads in
// flight) of its G heads, writes O and LSE.
template <int G, int NT>
__device__ __forceinline__ void merge_partials(const float *part, int64_t row_base, int n_split,
                                               void *O, int out_bf16, float *lse) {
    for (int pair = threadIdx.x; pair < G * (kD / 2); pair += NT) {
        const int g = pair / (kD / 2);
        const int c2 = (pair % (kD / 2)) * 2;
        const int64_t row = row_base + g;
        const float *pr = part + row * n_split * kPartStride;
        float M = -INFINITY, lsum = 0.f, a0 = 0.f, a1 = 0.f;
        for (int s0 = 0; s0 < n_split; s0 += 8) {
            float mk[8], lk[8], xk[8], yk[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float *ps = pr + (int64_t)(s0 + k) * kPartStride;
                const bool in = s0 + k < n_split;
                mk[k] = in ? load_dev(ps + kD) : -INFINITY;
                lk[k] = in ? load_dev(ps + kD + 1) : 0.f;
                xk[k] = in ? load_dev(ps + c2) : 0.f;
                yk[k] = in ? load_dev(ps + c2 + 1) : 0.f;
            }
            float Mc = M;
#pragma unroll
            for (int k = 0; k < 8; ++k) Mc = fmaxf(Mc, mk[k]);
            if (Mc == -INFINITY) continue;                  // nothing seen yet
            const float w_old = (M == -INFINITY) ? 0.f : exp2f(M - Mc);
            lsum *= w_old;
            a0 *= w_old;
            a1 *= w_old;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float wt = (mk[k] == -INFINITY) ? 0.f : exp2f(mk[k] - Mc);
                lsum = fmaf(wt, lk[k], lsum);
                a0 = fmaf(wt, xk[k], a0);
                a1 = fmaf(wt, yk[k], a1);
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
        if (lse && c2 == 0) lse[row] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
    }
}

// ROWS = false: idx lists 64-token blocks (contiguous rows). ROWS = true: idx
// lists single tokens (the token-level index); 64 consecutive list entries
// form a tile that is processed exactly like a block, except that each lane
// loads its 4 rows from the token ids of its entries (prefetched three tiles
// ahead with the buffer that uses them).
// SG > 0: the workgroup first takes its own unit's top-k (topk_unit, with SG
// selector heads per group, SSOFT for the softmax-sum form) from the scoring
// kernels' output into LDS; every split of a unit computes the same set (the
// redundant work replaces a separate top-k launch on the critical path) and
// split 0 writes it out.
// One workgroup's share of a unit: split `split` of unit `unit` out of n_units.
template <typename T, int G, bool DIRECT, bool ROWS, int SG, bool SSOFT>
__device__ __forceinline__ void decode_unit(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, int Hq, int Hkv,
    int64_t T_cap, const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int idx_cap, float qscale, int n_split,
    float *__restrict__ part, void *__restrict__ O, int out_bf16,
    float *__restrict__ lse, const FusedSelect &fs, int split, int unit, int n_units) {
    __shared__ AttendSmem<G, 4> sm;
    __shared__ uint32_t s_arrive;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int tid = threadIdx.x;
    // split merge hand-off words after the partials (see decode_workspace_bytes)
    uint64_t *sync = DIRECT ? nullptr
                            : (uint64_t *)((char *)part + partial_bytes(n_units / Hkv, Hq, n_split));
    const uint64_t tag = DIRECT ? 0 : call_tag(sync);
    int64_t L = seq_lens[b];
    L = L < 0 ? 0 : (L > T_cap ? T_cap : L);
    // the group's queries: loaded first, so the load overlaps the top-k below
    // (bf16: in the matrix-core operand layout)
    constexpr bool kMfma = __is_same(T, bf16_t);
    const T *Qg = Q + ((int64_t)b * Hq + (int64_t)kvh * G) * kD;
    QFrag<T, G> q;
    QMfma qm;
    if constexpr (kMfma) load_q_mfma<G>(Qg, tid & 63, qm);
    else load_q<G>(Qg + (tid & 15) * kLaneElems, q);
    int n;
    const int32_t *idx_row;
    if constexpr (SG > 0) {
        __shared__ int32_t s_list[kFusedMaxCap];
        __shared__ int32_t s_cnt;
        // The step's append (raw-sum, bf16): the unit's last split writes the
        // compressed entries completed between lens_prev and seq_lens (Eq. 2;
        // the same sums in the same order as the compress kernel). One new
        // entry: its 32 keys are loaded here, two per 16-lane row group, stay
        // in flight during the top-k, are staged in LDS and summed in token
        // order by one row group. More (a length jump beyond the caller's
        // hint): one entry per row group at a time from per-lane key loads.
        constexpr bool kApp = !SSOFT && __is_same(T, bf16_t);
        __shared__ uint4 s_app[kApp ? 2 * kCmpStride : 1][16];
        const int app_group = tid >> 4, app_lane = tid & 15;
        const bool app = kApp && fs.app_Kc != nullptr && split == n_split - 1;   // uniform
        int64_t app_lo = 0, app_hi = 0;
        Raw8<bf16_t> app_rows[2];
        if constexpr (kApp) {
            if (app) {
                int64_t Lp = fs.app_lens_prev[b];
                Lp = Lp < 0 ? 0 : (Lp > L ? L : Lp);
                app_lo = n_compressed(Lp);
                app_hi = n_compressed(L);
                if (app_hi == app_lo + 1) {
                    const bf16_t *Ka = (const bf16_t *)fs.app_K +
                                       ((int64_t)unit * T_cap + app_lo * kCmpStride + 2 * app_group) * kD +
                                       app_lane * kLaneElems;
                    load_raw(Ka, app_rows[0]);
                    load_raw(Ka + kD, app_rows[1]);
                }
            }
        }
        topk_unit<SG, SSOFT, kDecThreads, kFusedMaxBlocks / kDecThreads>(
            unit, Hkv, T_cap, fs.nb_cap, seq_lens, fs.top_k, fs.n_init, fs.n_local, fs.logits,
            fs.nc_pad, fs.stats, fs.n_chunks, fs.bscore, nullptr, s_list, idx_cap, &s_cnt,
            fs.use_buckets);
        if constexpr (kApp) {
            if (app && app_hi == app_lo + 1) {
                s_app[2 * app_group][app_lane] = app_rows[0].v;
                s_app[2 * app_group + 1][app_lane] = app_rows[1].v;
            }
        }
        __syncthreads();
        if constexpr (kApp) {
            if (app) {
                bf16_t *Kcu = (bf16_t *)fs.app_Kc + (int64_t)unit * fs.app_nc_cap * kD +
                              app_lane * kLaneElems;
                if (app_hi == app_lo + 1) {
                    if (app_group == 0) {
                        Raw8<bf16_t> e;
                        entry_from_rows(s_app, app_lane, e);
                        store_raw(Kcu + app_lo * kD, e);
                    }
                } else {
                    const bf16_t *Ku = (const bf16_t *)fs.app_K + (int64_t)unit * T_cap * kD +
                                       app_lane * kLaneElems;
                    for (int64_t j = app_lo + app_group; j < app_hi; j += kDecThreads / 16) {
                        Raw8<bf16_t> r;
                        compress_entry_raw(Ku, j, r);
                        store_raw(Kcu + j * kD, r);
                    }
                }
            }
        }
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
    const AttendOut out{part, n_split, split, O, out_bf16, lse};
    const int64_t row_base = (int64_t)b * Hq + (int64_t)kvh * G;
    constexpr int kMode = DIRECT ? kAttendDirect : kAttendPartialCoherent;
    if constexpr (kMfma)
        attend_share_mfma<G, ROWS, 4, kMode>(qm, K, V, T_cap, unit, L,
                                             idx_row + (ROWS ? 0 : e_lo), n, e_lo, nblk, qscale,
                                             row_base, out, sm);
    else
        attend_share<T, G, ROWS, 4, kMode>(q, K, V, T_cap, unit, L, idx_row + (ROWS ? 0 : e_lo), n,
                                           e_lo, nblk, qscale, row_base, out, sm);
    if constexpr (!DIRECT) {
        wait_own_stores();
        __syncthreads();
        if (tid == 0) s_arrive = arrive(sync + 2 + unit, tag);
        __syncthreads();
        if (s_arrive != (uint32_t)(n_split - 1)) return;
        // the unit's last split
        if (tid == 0) arm(sync + 2 + unit, tag);
        merge_partials<G, kDecThreads>(part, row_base, n_split, O, out_bf16, lse);
        // every workgroup has counted itself (so read the epoch) once the last
        // unit is merged: the call's tag becomes the epoch
        if (tid == 0 && arrive(sync + 1, tag) == (uint32_t)(n_units - 1)) {
            arm(sync + 1, tag);
            store_dev(sync, tag);
        }
    }
}

template <typename T, int G, bool DIRECT, bool ROWS, int SG = 0, bool SSOFT = false>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, int Hq, int Hkv,
    int64_t T_cap, const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int idx_cap, float qscale, int n_split,
    float *__restrict__ part, void *__restrict__ O, int out_bf16,
    float *__restrict__ lse, FusedSelect fs) {
    decode_unit<T, G, DIRECT, ROWS, SG, SSOFT>(Q, K, V, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap,
                                               qscale, n_split, part, O, out_bf16, lse, fs,
                                               (int)blockIdx.x, (int)blockIdx.y, (int)gridDim.y);
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
