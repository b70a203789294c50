// C ABI entry points of libsparse_attn: argument validation, workspace sizing
// and dispatch to the kernel launchers. Every check runs on the host before
// any HIP call, so an invalid call enqueues nothing and returns a status.
#include <stddef.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_internal.h"

using namespace sa;

namespace {

bool dtype_ok(int dt) { return dt == SA_F32 || dt == SA_BF16; }

// query heads per KV head the decode attention kernels are built for
bool attn_group_ok(int Hq, int Hkv) {
    const int G = Hq / Hkv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

int check_params(const sa_select_params *p) {
    if (!p) return SA_ERR_INVALID_ARG;
    if (p->top_k < 0 || p->n_init < 0 || p->n_local < 0) return SA_ERR_INVALID_ARG;
    if (p->score_mode != SA_SCORE_SOFTMAX_SUM && p->score_mode != SA_SCORE_RAW_SUM)
        return SA_ERR_INVALID_ARG;
    if (p->block_size != kBlock || p->cmp_kernel != kCmpKernel || p->cmp_stride != kCmpStride)
        return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

int64_t union_cap(const sa_select_params *p) {
    return (int64_t)p->top_k + p->n_init + p->n_local;
}

}  // namespace

extern "C" {

int sparse_attn_abi_version(void) { return SPARSE_ATTN_ABI_VERSION; }

const char *sparse_attn_status_string(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARG: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SA_ERR_WORKSPACE: return "workspace missing or too small";
        case SA_ERR_CAPACITY: return "output or cache capacity too small";
        case SA_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int sparse_attn_compress(const void *K, void *Kc, int dtype, int B, int Hkv, int d, int64_t T_cap,
                         int64_t nc_cap, const int32_t *lens_prev, const int32_t *lens_now,
                         int32_t max_new_entries, void *stream) {
    if (!K || !Kc || !lens_prev || !lens_now) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || B <= 0 || Hkv <= 0 || d <= 0 || T_cap < 0 || nc_cap < 0)
        return SA_ERR_INVALID_ARG;
    if (max_new_entries < 0) return SA_ERR_INVALID_ARG;
    if (d != kD) return SA_ERR_UNSUPPORTED;
    if (nc_cap < n_compressed(T_cap)) return SA_ERR_CAPACITY;
    if ((int64_t)B * Hkv > 0x7fffffff) return SA_ERR_UNSUPPORTED;
    if (max_new_entries == 0 || T_cap == 0) return SA_OK;
    return launch_compress(K, Kc, dtype, B, Hkv, T_cap, nc_cap, lens_prev, lens_now,
                           max_new_entries, (hipStream_t)stream);
}

size_t sparse_attn_select_workspace_size(int B, int Hkv, int H_sel, int64_t T_cap,
                                         const sa_select_params *p) {
    if (!p || B <= 0 || Hkv <= 0 || H_sel <= 0 || H_sel % Hkv || T_cap < 0) return 0;
    const int G = H_sel / Hkv;
    return select_workspace_layout(B, Hkv, G, T_cap, p->score_mode).total;
}

int sparse_attn_select(const void *sel, int H_sel, const void *Kc, int dtype, int B, int Hkv,
                       int d, int64_t T_cap, int64_t nc_cap, const int32_t *seq_lens,
                       const sa_select_params *p, int32_t *idx_out, int32_t idx_cap,
                       int32_t *cnt_out, float *block_scores_out, void *workspace,
                       size_t ws_bytes, void *stream) {
    if (!sel || !Kc || !seq_lens || !idx_out || !cnt_out) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || B <= 0 || Hkv <= 0 || H_sel <= 0 || d <= 0 || T_cap < 0 || nc_cap < 0)
        return SA_ERR_INVALID_ARG;
    int st = check_params(p);
    if (st) return st;
    if (H_sel % Hkv) return SA_ERR_INVALID_ARG;
    const int G = H_sel / Hkv;
    if (d != kD) return SA_ERR_UNSUPPORTED;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return SA_ERR_UNSUPPORTED;
    if (n_blocks(T_cap) > 32768) return SA_ERR_UNSUPPORTED;
    if (nc_cap < n_compressed(T_cap)) return SA_ERR_CAPACITY;
    if (idx_cap < union_cap(p) || idx_cap <= 0) return SA_ERR_CAPACITY;
    const size_t need = select_workspace_layout(B, Hkv, G, T_cap, p->score_mode).total;
    if (need > 0 && (!workspace || ws_bytes < need)) return SA_ERR_WORKSPACE;
    return launch_select(sel, G, Kc, dtype, B, Hkv, T_cap, nc_cap, seq_lens, *p, idx_out, idx_cap,
                         cnt_out, block_scores_out, workspace, (hipStream_t)stream);
}

size_t sparse_attn_decode_workspace_size(int B, int Hq, int Hkv, int32_t idx_cap, int32_t n_split) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || idx_cap <= 0) return 0;
    int s = n_split > 0 ? n_split : decode_auto_split(B, Hkv, idx_cap);
    if (s < decode_min_split(idx_cap)) s = decode_min_split(idx_cap);
    return decode_workspace_bytes(B, Hq, Hkv, s);
}

int sparse_attn_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                       int Hkv, int d, int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                       const int32_t *cnt, int32_t idx_cap, float scale, void *O, int out_dtype,
                       float *lse_out, int32_t n_split, void *workspace, size_t ws_bytes,
                       void *stream) {
    if (!Q || !K || !V || !seq_lens || !idx || !cnt || !O) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype) || B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 ||
        T_cap < 0 || idx_cap <= 0)
        return SA_ERR_INVALID_ARG;
    if (Hq % Hkv) return SA_ERR_INVALID_ARG;
    if (!(scale == scale)) return SA_ERR_INVALID_ARG;
    if (d != kD || !attn_group_ok(Hq, Hkv)) return SA_ERR_UNSUPPORTED;
    if (n_split > kMaxSplit || idx_cap > 64 * kMaxSplit) return SA_ERR_UNSUPPORTED;
    if ((int64_t)T_cap * d * (dtype == SA_BF16 ? 2 : 4) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    int s = n_split > 0 ? n_split : decode_auto_split(B, Hkv, idx_cap);
    if (s < decode_min_split(idx_cap)) s = decode_min_split(idx_cap);
    const size_t need = decode_workspace_bytes(B, Hq, Hkv, s);
    if (need > 0 && (!workspace || ws_bytes < need)) return SA_ERR_WORKSPACE;
    return launch_decode(Q, K, V, dtype, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap, scale, O,
                         out_dtype, lse_out, s, workspace, (hipStream_t)stream);
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int decode_splits(int B, int Hkv, int32_t idx_cap, int32_t n_split) {
    int s = n_split > 0 ? n_split : decode_auto_split(B, Hkv, idx_cap);
    return s < decode_min_split(idx_cap) ? decode_min_split(idx_cap) : s;
}

}  // namespace

size_t sparse_attn_decode_step_workspace_size(int B, int Hq, int Hkv, int H_sel, int64_t T_cap,
                                              const sa_select_params *p, int32_t idx_cap,
                                              int32_t n_split) {
    if (!p || B <= 0 || Hq <= 0 || Hkv <= 0 || H_sel <= 0 || H_sel % Hkv || T_cap < 0 ||
        idx_cap <= 0)
        return 0;
    const size_t sel = select_workspace_layout(B, Hkv, H_sel / Hkv, T_cap, p->score_mode).total;
    return align256(sel) + decode_workspace_bytes(B, Hq, Hkv, decode_splits(B, Hkv, idx_cap, n_split));
}

int32_t sparse_attn_decode_step_splits(int dtype, int B, int Hkv, int64_t T_cap,
                                       const sa_select_params *p, int32_t idx_cap,
                                       int32_t max_new_tokens, int32_t n_split) {
    if (!p || !dtype_ok(dtype) || B <= 0 || Hkv <= 0 || T_cap < 0 || idx_cap <= 0 || n_split < 0 ||
        max_new_tokens < 0)
        return 0;
    (void)T_cap;
    (void)max_new_tokens;
    return decode_splits(B, Hkv, idx_cap, n_split);
}

int sparse_attn_decode_step(const void *Q, const void *sel, int H_sel, const void *K, const void *V,
                            void *Kc, int dtype, int B, int Hq, int Hkv, int d, int64_t T_cap,
                            int64_t nc_cap, const int32_t *lens_prev, const int32_t *lens_now,
                            int32_t max_new_tokens, const sa_select_params *p, float scale,
                            int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out, void *O,
                            int out_dtype, float *lse_out, int32_t n_split, void *workspace,
                            size_t ws_bytes, void *stream) {
    if (!Q || !sel || !K || !V || !Kc || !lens_prev || !lens_now || !idx_out || !cnt_out || !O)
        return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype) || B <= 0 || Hq <= 0 || Hkv <= 0 || H_sel <= 0 ||
        d <= 0 || T_cap <= 0 || nc_cap < 0 || idx_cap <= 0 || max_new_tokens < 0)
        return SA_ERR_INVALID_ARG;
    int st = check_params(p);
    if (st) return st;
    if (Hq % Hkv || H_sel % Hkv || !(scale == scale)) return SA_ERR_INVALID_ARG;
    const int G = H_sel / Hkv;
    if (d != kD || !attn_group_ok(Hq, Hkv)) return SA_ERR_UNSUPPORTED;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return SA_ERR_UNSUPPORTED;
    if (n_blocks(T_cap) > 32768 || (int64_t)B * Hkv > 65535) return SA_ERR_UNSUPPORTED;
    if (n_split > kMaxSplit || idx_cap > 64 * kMaxSplit) return SA_ERR_UNSUPPORTED;
    if (T_cap * d * (dtype == SA_BF16 ? 2 : 4) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    if (nc_cap < n_compressed(T_cap)) return SA_ERR_CAPACITY;
    if (idx_cap < union_cap(p)) return SA_ERR_CAPACITY;
    const hipStream_t hs = (hipStream_t)stream;
    const size_t sel_bytes = align256(select_workspace_layout(B, Hkv, G, T_cap, p->score_mode).total);
    const int s = decode_splits(B, Hkv, idx_cap, n_split);
    const size_t need = sel_bytes + decode_workspace_bytes(B, Hq, Hkv, s);
    if (!workspace || ws_bytes < need) return SA_ERR_WORKSPACE;
    // up to 2048 blocks, each decode workgroup takes its unit's top-k itself
    // from the block scores (no separate top-k launch between scoring and
    // attention); not for 8 selector heads a group, whose softmax top-k would
    // take the attention kernel past 256 VGPRs
    FusedSelect fs{};
    const bool fused = n_blocks(T_cap) <= kFusedMaxBlocks && idx_cap <= kFusedMaxCap &&
                       (p->score_mode == SA_SCORE_RAW_SUM || G <= 4);
    FusedSelect *fsp = fused ? &fs : nullptr;
    if (p->score_mode == SA_SCORE_RAW_SUM) {
        // the scorer reads only the entries that existed before the step (a
        // candidate block holding a new one is rescored with it formed from the
        // keys); the new entries are written by the attention launch (bf16, at
        // most 16 new tokens, fused top-k: fs->app_*) or by the scoring launch
        st = launch_select(sel, G, Kc, dtype, B, Hkv, T_cap, nc_cap, lens_now, *p, idx_out, idx_cap,
                           cnt_out, nullptr, workspace, hs, K, lens_prev, fsp, max_new_tokens);
    } else {
        // the scorer forms the new entries itself (they enter every head's
        // softmax denominator in the order a separate append would give) and
        // writes them to Kc
        st = launch_select(sel, G, Kc, dtype, B, Hkv, T_cap, nc_cap, lens_now, *p, idx_out, idx_cap,
                           cnt_out, nullptr, workspace, hs, K, lens_prev, fsp);
    }
    if (st) return st;
    if (fused)
        return launch_decode_select(Q, K, V, dtype, B, Hq, Hkv, T_cap, lens_now, idx_cap, scale, O,
                                    out_dtype, lse_out, s, (char *)workspace + sel_bytes, fs, G,
                                    p->score_mode != SA_SCORE_RAW_SUM, hs);
    return launch_decode(Q, K, V, dtype, B, Hq, Hkv, T_cap, lens_now, idx_out, cnt_out, idx_cap,
                         scale, O, out_dtype, lse_out, s, (char *)workspace + sel_bytes, hs);
}

int32_t sparse_attn_prefill_tile_cap(int64_t q_start, int64_t Tq, const sa_select_params *p) {
    if (!p || q_start < 0 || Tq <= 0) return 0;
    return prefill_tile_cap(q_start, Tq, *p);
}

size_t sparse_attn_prefill_workspace_size(int Hq, int Hkv, int64_t q_start, int64_t Tq,
                                          const sa_select_params *p) {
    if (!p || Hq <= 0 || Hkv <= 0 || Hq % Hkv || q_start < 0 || Tq <= 0) return 0;
    return prefill_workspace_bytes(Hq, Hkv, q_start, Tq, *p);
}

int sparse_attn_prefill_chunk(const void *Q, int64_t q_start, int64_t Tq, const void *K,
                              const void *V, const void *Kc, int dtype, int Hq, int Hkv, int d,
                              int64_t T_cap, int64_t nc_cap, const sa_select_params *p,
                              float scale, void *O, int out_dtype, float *lse_out,
                              int32_t *tile_idx_out, int32_t tile_idx_cap, int32_t *tile_cnt_out,
                              void *workspace, size_t ws_bytes, void *stream) {
    if (!Q || !K || !V || !Kc || !O || !tile_idx_out || !tile_cnt_out) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype) || Hq <= 0 || Hkv <= 0 || d <= 0 || Tq <= 0 ||
        q_start < 0 || T_cap < 0 || nc_cap < 0)
        return SA_ERR_INVALID_ARG;
    if (q_start % kBlock) return SA_ERR_INVALID_ARG;
    if (Hq % Hkv) return SA_ERR_INVALID_ARG;
    if (!(scale == scale)) return SA_ERR_INVALID_ARG;
    int st = check_params(p);
    if (st) return st;
    if (d != kD || Hq / Hkv != 4 || dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (n_blocks(q_start + Tq) > 32768) return SA_ERR_UNSUPPORTED;
    if (T_cap * d * 2 > 0x7fffffffLL || nc_cap * d * 2 > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    // a tile's per-query block scores (64 queries x Hkv x blocks, fp32) take 32-bit offsets
    if ((63 * (int64_t)Hkv + 1) * n_blocks(q_start + Tq) * 4 > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    if (T_cap < q_start + Tq) return SA_ERR_CAPACITY;
    if (nc_cap < n_compressed(q_start + Tq)) return SA_ERR_CAPACITY;
    if (tile_idx_cap < prefill_tile_cap(q_start, Tq, *p)) return SA_ERR_CAPACITY;
    const size_t need = prefill_workspace_bytes(Hq, Hkv, q_start, Tq, *p);
    if (need > 0 && (!workspace || ws_bytes < need)) return SA_ERR_WORKSPACE;
    return launch_prefill(Q, q_start, Tq, K, V, Kc, Hq, Hkv, T_cap, nc_cap, *p, scale, O, out_dtype,
                          lse_out, tile_idx_out, tile_idx_cap, tile_cnt_out, workspace,
                          (hipStream_t)stream);
}

int sparse_attn_prefill_attend(const void *Q, int64_t q_start, int64_t Tq, const void *K,
                               const void *V, int dtype, int Hq, int Hkv, int d, int64_t T_cap,
                               const int32_t *tile_idx, int32_t tile_idx_cap,
                               const int32_t *tile_cnt, float scale, void *O, int out_dtype,
                               float *lse_out, void *stream) {
    if (!Q || !K || !V || !O || !tile_idx || !tile_cnt) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype) || Hq <= 0 || Hkv <= 0 || d <= 0 || Tq <= 0 ||
        q_start < 0 || T_cap < 0 || tile_idx_cap <= 0)
        return SA_ERR_INVALID_ARG;
    if (q_start % kBlock) return SA_ERR_INVALID_ARG;
    if (Hq % Hkv) return SA_ERR_INVALID_ARG;
    if (!(scale == scale)) return SA_ERR_INVALID_ARG;
    if (d != kD || Hq / Hkv != 4 || dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (T_cap * d * 2 > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    if (T_cap < q_start + Tq) return SA_ERR_CAPACITY;
    return launch_prefill_attend(Q, q_start, Tq, K, V, Hq, Hkv, T_cap, tile_idx, tile_idx_cap,
                                 tile_cnt, scale, O, out_dtype, lse_out, (hipStream_t)stream);
}

size_t sparse_attn_token_select_workspace_size(int B, int Hkv, int64_t T_cap) {
    if (B <= 0 || Hkv <= 0 || T_cap < 0) return 0;
    return token_workspace_layout(B, Hkv, T_cap).total;
}

int sparse_attn_token_select(const void *sel, int H_sel, const void *Ki, int dtype, int B, int Hkv,
                             int d_i, int64_t T_cap, const int32_t *seq_lens, int32_t top_k,
                             int32_t n_init, int32_t n_local, int32_t *idx_out, int32_t idx_cap,
                             int32_t *cnt_out, float *scores_out, void *workspace,
                             size_t ws_bytes, void *stream) {
    if (!sel || !Ki || !seq_lens || !idx_out || !cnt_out) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || B <= 0 || Hkv <= 0 || H_sel <= 0 || d_i <= 0 || T_cap < 0)
        return SA_ERR_INVALID_ARG;
    if (top_k < 0 || n_init < 0 || n_local < 0 || H_sel % Hkv) return SA_ERR_INVALID_ARG;
    if (d_i != 64 && d_i != 128) return SA_ERR_UNSUPPORTED;
    if (H_sel / Hkv > 64 || (int64_t)B * Hkv > 65535) return SA_ERR_UNSUPPORTED;
    if (T_cap * d_i * (dtype == SA_BF16 ? 2 : 4) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    if (idx_cap <= 0 || idx_cap < (int64_t)top_k + n_init + n_local) return SA_ERR_CAPACITY;
    const size_t need = token_workspace_layout(B, Hkv, T_cap).total;
    if (!workspace || ws_bytes < need) return SA_ERR_WORKSPACE;
    return launch_token_select(sel, H_sel, Ki, dtype, B, Hkv, d_i, T_cap, seq_lens, top_k, n_init,
                               n_local, idx_out, idx_cap, cnt_out, scores_out, workspace,
                               (hipStream_t)stream);
}

size_t sparse_attn_token_decode_workspace_size(int B, int Hq, int Hkv, int32_t idx_cap,
                                               int32_t n_split) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || idx_cap <= 0) return 0;
    const int32_t tiles = (idx_cap + 63) / 64;
    int s = n_split > 0 ? n_split : decode_auto_split(B, Hkv, tiles);
    if (s < decode_min_split(tiles)) s = decode_min_split(tiles);
    return decode_workspace_bytes(B, Hq, Hkv, s);
}

int sparse_attn_token_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                             int Hkv, int d, int64_t T_cap, const int32_t *seq_lens,
                             const int32_t *idx, const int32_t *cnt, int32_t idx_cap, float scale,
                             void *O, int out_dtype, float *lse_out, int32_t n_split,
                             void *workspace, size_t ws_bytes, void *stream) {
    if (!Q || !K || !V || !seq_lens || !idx || !cnt || !O) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype) || B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 ||
        T_cap < 0 || idx_cap <= 0)
        return SA_ERR_INVALID_ARG;
    if (Hq % Hkv) return SA_ERR_INVALID_ARG;
    if (!(scale == scale)) return SA_ERR_INVALID_ARG;
    if (d != kD || !attn_group_ok(Hq, Hkv)) return SA_ERR_UNSUPPORTED;
    const int32_t tiles = (int32_t)(((int64_t)idx_cap + 63) / 64);
    if (n_split > kMaxSplit || tiles > 64 * kMaxSplit) return SA_ERR_UNSUPPORTED;
    if ((int64_t)T_cap * d * (dtype == SA_BF16 ? 2 : 4) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    int s = n_split > 0 ? n_split : decode_auto_split(B, Hkv, tiles);
    if (s < decode_min_split(tiles)) s = decode_min_split(tiles);
    const size_t need = decode_workspace_bytes(B, Hq, Hkv, s);
    if (need > 0 && (!workspace || ws_bytes < need)) return SA_ERR_WORKSPACE;
    return launch_decode_rows(Q, K, V, dtype, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap, scale,
                              O, out_dtype, lse_out, s, workspace, (hipStream_t)stream);
}

int sparse_attn_cobs_stats(const void *K, void *stats, int dtype, int B, int Hkv, int d,
                           int64_t T_cap, int64_t nb_cap, const int32_t *lens_prev,
                           const int32_t *lens_now, int32_t max_new_blocks, void *stream) {
    if (!K || !stats || !lens_prev || !lens_now) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || B <= 0 || Hkv <= 0 || d <= 0 || T_cap < 0 || nb_cap < 0)
        return SA_ERR_INVALID_ARG;
    if (max_new_blocks < 0) return SA_ERR_INVALID_ARG;
    if (d != kD) return SA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv > 65535) return SA_ERR_UNSUPPORTED;
    if (nb_cap < T_cap / kBlock) return SA_ERR_CAPACITY;
    if (max_new_blocks == 0 || T_cap < kBlock) return SA_OK;
    return launch_cobs_stats(K, stats, dtype, B, Hkv, T_cap, nb_cap, lens_prev, lens_now,
                             max_new_blocks, (hipStream_t)stream);
}

size_t sparse_attn_cobs_select_workspace_size(int B, int Hkv, int H_sel, int64_t T_cap,
                                              const sa_select_params *p) {
    if (!p || B <= 0 || Hkv <= 0 || H_sel <= 0 || H_sel % Hkv || T_cap < 0) return 0;
    return cobs_workspace_layout(B, Hkv, H_sel / Hkv, T_cap, p->score_mode).total;
}

int sparse_attn_cobs_select(const void *sel, int H_sel, const void *stats, int dtype, int B,
                            int Hkv, int d, int64_t T_cap, int64_t nb_cap,
                            const int32_t *seq_lens, const sa_select_params *p, int32_t order,
                            int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                            float *block_scores_out, void *workspace, size_t ws_bytes,
                            void *stream) {
    if (!sel || !stats || !seq_lens || !idx_out || !cnt_out) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || B <= 0 || Hkv <= 0 || H_sel <= 0 || d <= 0 || T_cap < 0 || nb_cap < 0)
        return SA_ERR_INVALID_ARG;
    int st = check_params(p);
    if (st) return st;
    if (H_sel % Hkv || (order != 1 && order != 2)) return SA_ERR_INVALID_ARG;
    const int G = H_sel / Hkv;
    if (d != kD) return SA_ERR_UNSUPPORTED;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return SA_ERR_UNSUPPORTED;
    if (n_blocks(T_cap) > 32768 || (int64_t)B * Hkv > 65535) return SA_ERR_UNSUPPORTED;
    if (nb_cap < n_blocks(T_cap)) return SA_ERR_CAPACITY;
    if (idx_cap < union_cap(p) || idx_cap <= 0) return SA_ERR_CAPACITY;
    const size_t need = cobs_workspace_layout(B, Hkv, G, T_cap, p->score_mode).total;
    if (!workspace || ws_bytes < need) return SA_ERR_WORKSPACE;
    if (T_cap == 0) return SA_ERR_INVALID_ARG;
    return launch_cobs_select(sel, G, stats, nb_cap, dtype, B, Hkv, T_cap, seq_lens, *p, order, idx_out,
                              idx_cap, cnt_out, block_scores_out, workspace, (hipStream_t)stream);
}

size_t sparse_attn_cobs_decode_step_workspace_size(int B, int Hq, int Hkv, int H_sel,
                                                   int64_t T_cap, const sa_select_params *p,
                                                   int32_t idx_cap, int32_t n_split) {
    if (!p || B <= 0 || Hq <= 0 || Hkv <= 0 || H_sel <= 0 || H_sel % Hkv || T_cap < 0 ||
        idx_cap <= 0)
        return 0;
    const size_t sel = cobs_workspace_layout(B, Hkv, H_sel / Hkv, T_cap, p->score_mode).total;
    return align256(sel) + decode_workspace_bytes(B, Hq, Hkv, decode_splits(B, Hkv, idx_cap, n_split));
}

int sparse_attn_cobs_decode_step(const void *Q, const void *sel, int H_sel, const void *K,
                                 const void *V, void *stats, int dtype, int B, int Hq, int Hkv,
                                 int d, int64_t T_cap, int64_t nb_cap, const int32_t *lens_prev,
                                 const int32_t *lens_now, int32_t max_new_blocks,
                                 const sa_select_params *p, int32_t order, float scale,
                                 int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out, void *O,
                                 int out_dtype, float *lse_out, int32_t n_split, void *workspace,
                                 size_t ws_bytes, void *stream) {
    if (!Q || !sel || !K || !V || !stats || !lens_prev || !lens_now || !idx_out || !cnt_out || !O)
        return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype) || B <= 0 || Hq <= 0 || Hkv <= 0 || H_sel <= 0 ||
        d <= 0 || T_cap <= 0 || nb_cap < 0 || idx_cap <= 0 || max_new_blocks < 0)
        return SA_ERR_INVALID_ARG;
    int st = check_params(p);
    if (st) return st;
    if (Hq % Hkv || H_sel % Hkv || (order != 1 && order != 2) || !(scale == scale))
        return SA_ERR_INVALID_ARG;
    const int G = H_sel / Hkv;
    if (d != kD || !attn_group_ok(Hq, Hkv)) return SA_ERR_UNSUPPORTED;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return SA_ERR_UNSUPPORTED;
    if (n_blocks(T_cap) > 32768 || (int64_t)B * Hkv > 65535) return SA_ERR_UNSUPPORTED;
    if (n_split > kMaxSplit || idx_cap > 64 * kMaxSplit) return SA_ERR_UNSUPPORTED;
    if (T_cap * d * (dtype == SA_BF16 ? 2 : 4) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    if (nb_cap < n_blocks(T_cap)) return SA_ERR_CAPACITY;
    if (idx_cap < union_cap(p)) return SA_ERR_CAPACITY;
    const size_t sel_bytes =
        align256(cobs_workspace_layout(B, Hkv, G, T_cap, p->score_mode).total);
    const int s = decode_splits(B, Hkv, idx_cap, n_split);
    if (!workspace || ws_bytes < sel_bytes + decode_workspace_bytes(B, Hq, Hkv, s))
        return SA_ERR_WORKSPACE;
    const hipStream_t hs = (hipStream_t)stream;
    if (max_new_blocks > 0 && T_cap >= kBlock) {     // statistics of newly completed blocks
        st = launch_cobs_stats(K, stats, dtype, B, Hkv, T_cap, nb_cap, lens_prev, lens_now,
                               max_new_blocks, hs);
        if (st) return st;
    }
    // raw sum: the attention workgroups take the top-k from the block scores
    // (as in sparse_attn_decode_step). Softmax sum: every workgroup would read
    // all G heads' logits (G x 8 KB at 2048 blocks) and exponentiate them, which
    // measured slower than the separate top-k launch (64 workgroups).
    const bool softmax = p->score_mode != SA_SCORE_RAW_SUM;
    FusedSelect fs{};
    const bool fused = n_blocks(T_cap) <= kFusedMaxBlocks && idx_cap <= kFusedMaxCap && !softmax;
    st = launch_cobs_select(sel, G, stats, nb_cap, dtype, B, Hkv, T_cap, lens_now, *p, order,
                            idx_out, idx_cap, cnt_out, nullptr, workspace, hs,
                            fused ? &fs : nullptr);
    if (st) return st;
    if (fused)
        return launch_decode_select(Q, K, V, dtype, B, Hq, Hkv, T_cap, lens_now, idx_cap, scale, O,
                                    out_dtype, lse_out, s, (char *)workspace + sel_bytes, fs, G,
                                    softmax, hs);
    return launch_decode(Q, K, V, dtype, B, Hq, Hkv, T_cap, lens_now, idx_out, cnt_out, idx_cap,
                         scale, O, out_dtype, lse_out, s, (char *)workspace + sel_bytes, hs);
}

size_t sparse_attn_block_mass_workspace_size(int B, int Hq, int64_t mass_cap) {
    if (B <= 0 || Hq <= 0 || mass_cap <= 0) return 0;
    return block_mass_workspace_bytes(B, Hq, mass_cap);
}

int sparse_attn_block_mass(const void *Q, const void *K, int dtype, int B, int Hq, int Hkv, int d,
                           int64_t T_cap, const int32_t *seq_lens, float scale, float *mass_out,
                           int64_t mass_cap, const int32_t *idx, const int32_t *cnt,
                           int32_t idx_cap, float *recall_out, void *workspace, size_t ws_bytes,
                           void *stream) {
    if (!Q || !K || !seq_lens || !mass_out) return SA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || B <= 0 || Hq <= 0 || Hkv <= 0 || T_cap <= 0) return SA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0 || !(scale == scale)) return SA_ERR_INVALID_ARG;
    if (idx && (!cnt || !recall_out || idx_cap <= 0)) return SA_ERR_INVALID_ARG;
    if (d != kD || Hq / Hkv != 4) return SA_ERR_UNSUPPORTED;       // measurement kernel: G = 4
    if (T_cap * d * (dtype == SA_BF16 ? 2 : 4) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
    if (mass_cap < n_blocks(T_cap)) return SA_ERR_CAPACITY;
    if (!workspace || ws_bytes < block_mass_workspace_bytes(B, Hq, mass_cap)) return SA_ERR_WORKSPACE;
    return launch_block_mass(Q, K, dtype, B, Hq, Hkv, T_cap, seq_lens, scale, mass_out, mass_cap,
                             idx, cnt, idx_cap, recall_out, workspace, (hipStream_t)stream);
}

int sparse_attn_stream_read_blocks(void) { return kStreamReadBlocks; }

int sparse_attn_stream_read(const void *buf, size_t bytes, uint32_t *xor_out, void *stream) {
    if (!buf || !xor_out || bytes == 0 || bytes % 16 != 0) return SA_ERR_INVALID_ARG;
    if ((uintptr_t)buf % 16 != 0) return SA_ERR_INVALID_ARG;
    return launch_stream_read(buf, bytes, xor_out, (hipStream_t)stream);
}

}  // extern "C"
