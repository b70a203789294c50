// Host-side launchers of libsparse_attn (one per kernel family). Argument
// validation happens in sparse_attn_api.hip before any of these is called;
// the launchers only size grids and enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"

namespace sa {

// Scratch layout of sparse_attn_select (offsets in bytes inside the workspace).
struct SelectWorkspace {
    size_t logits_off, logits_bytes;   // [units][G][nc_pad] fp32 (softmax mode)
    size_t stats_off, stats_bytes;     // [units][G][n_chunks] float2 (max, sum exp)
    size_t bscore_off, bscore_bytes;   // [units][nb_cap] fp32
    size_t total;
    int64_t nc_pad;                    // row stride of the logits
    int64_t nb_cap;
    int n_chunks;
};
SelectWorkspace select_workspace_layout(int B, int Hkv, int G, int64_t T_cap, int score_mode);

int launch_compress(const void *K, void *Kc, int dtype, int B, int Hkv, int64_t T_cap,
                    int64_t nc_cap, const int32_t *lens_prev, const int32_t *lens_now,
                    int32_t max_new_entries, hipStream_t stream);

// What a decode kernel needs to take the top-k of its own (sequence, KV head)
// from the scoring kernels' output (raw-sum block scores, or softmax-mode
// logits and chunk statistics), and where to write the block sets.
struct FusedSelect {
    int64_t nb_cap;
    int top_k, n_init, n_local;
    const float *bscore;               // raw-sum mode
    const float *logits;               // softmax mode
    int64_t nc_pad;                    // logits row stride
    const float2 *stats;
    int n_chunks;
    int32_t *idx_out, *cnt_out;
    int use_buckets;
    int epb;                           // softmax logits per block: 4 (compressed entries) or 1
    // the step's append by the attention launch (raw-sum, bf16 keys): when
    // app_Kc is set, the last split workgroup of each unit writes the
    // compressed entries completed between app_lens_prev and seq_lens, formed
    // from app_K (the scoring launch read none of them)
    const void *app_K;
    void *app_Kc;
    const int32_t *app_lens_prev;
    int64_t app_nc_cap;
};

// With K and lens_prev, the compressed entries completed between lens_prev
// and seq_lens are written in the same step (raw-sum mode: max_new_tokens is
// an upper bound on lens_now - lens_prev; up to 16 with bf16 keys and fs, the
// attention launch writes them (fs->app_*) and the scorer reads only older
// entries; otherwise the scoring launch writes them; softmax mode: the
// scoring workgroup owning a new entry forms, scores and writes it).
// With fs, only the scoring kernel(s) run and fs describes their output (the
// top-k is left to the caller's next launch).
int launch_select(const void *sel, int G, const void *Kc, int dtype, int B, int Hkv,
                  int64_t T_cap, int64_t nc_cap, const int32_t *seq_lens,
                  const sa_select_params &p, int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                  float *block_scores_out, void *workspace, hipStream_t stream,
                  const void *K = nullptr, const int32_t *lens_prev = nullptr,
                  FusedSelect *fs = nullptr, int32_t max_new_tokens = 1 << 30);
// Decode attention whose workgroups first take their unit's top-k themselves
// (fs from launch_select or launch_cobs_select): needs ceil(T_cap / 64) <= 2048,
// idx_cap <= 1024 and, for the softmax-sum form, G <= 4 and logits of
// compressed entries (epb 4; per-block logits are not taken here).
constexpr int64_t kFusedMaxBlocks = 2048;
constexpr int kFusedMaxCap = 1024;
int launch_decode_select(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                         int Hkv, int64_t T_cap, const int32_t *seq_lens, int32_t idx_cap,
                         float scale, void *O, int out_dtype, float *lse_out, int32_t n_split,
                         void *workspace, const FusedSelect &fs, int G, bool softmax,
                         hipStream_t stream);

void launch_topk_block_softmax(int n_units, int G, int Hkv, int64_t T_cap, int64_t nb_cap,
                               const int32_t *seq_lens, const sa_select_params &p,
                               const float *logits, int64_t nb_pad, const float2 *stats,
                               int n_chunks, float *bs_out, int32_t *idx_out, int idx_cap,
                               int32_t *cnt_out, hipStream_t stream);
void launch_topk_raw(int n_units, int Hkv, int64_t T_cap, int64_t nb_cap, const int32_t *seq_lens,
                     const sa_select_params &p, const float *bscore, int32_t *idx_out, int idx_cap,
                     int32_t *cnt_out, hipStream_t stream);

int decode_auto_split(int B, int Hkv, int32_t idx_cap);
int decode_min_split(int32_t idx_cap);
// split partials [B * Hq][n_split][132] fp32 and the split-merge hand-off
// words (0 bytes for one split)
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int32_t n_split);
int launch_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq, int Hkv,
                  int64_t T_cap, const int32_t *seq_lens, const int32_t *idx, const int32_t *cnt,
                  int32_t idx_cap, float scale, void *O, int out_dtype, float *lse_out,
                  int32_t n_split, void *workspace, hipStream_t stream);

// Token-level selection: scratch layout and launcher (offsets in bytes).
struct TokenWorkspace {
    size_t keys_off;                   // [units][t_pad] uint32 orderable keys
    size_t hist_off;                   // [4 passes][units][256] uint32
    size_t counts_off;                 // [units][n_chunks][2] int32
    size_t info_off;                   // [units][2] uint32 (k-th key, equal keys taken)
    size_t total;
    int64_t t_pad;
    int n_chunks;
};
TokenWorkspace token_workspace_layout(int B, int Hkv, int64_t T_cap);
int launch_token_select(const void *sel, int H_sel, const void *Ki, int dtype, int B, int Hkv,
                        int d_i, int64_t T_cap, const int32_t *seq_lens, int top_k, int n_init,
                        int n_local, int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                        float *scores_out, void *workspace, hipStream_t stream);
// Decode attention over per-(b, kvh) token lists (gathered single rows).
int launch_decode_rows(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                       int Hkv, int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                       const int32_t *cnt, int32_t idx_cap, float scale, void *O, int out_dtype,
                       float *lse_out, int32_t n_split, void *workspace, hipStream_t stream);

// Second-order block statistic selection: scratch layout and launchers.
struct CobsWorkspace {
    size_t bscore_off;                 // [units][nb_cap] fp32 block scores
    size_t logits_off;                 // [units][G][nb_pad] fp32 (softmax mode)
    size_t stats_off;                  // [units][G][n_chunks] float2 (max, sum exp)
    size_t total;
    int64_t nb_cap, nb_pad;
    int n_chunks;
};
CobsWorkspace cobs_workspace_layout(int B, int Hkv, int G, int64_t T_cap, int score_mode);
int launch_cobs_stats(const void *K, void *stats, int dtype, int B, int Hkv, int64_t T_cap,
                      int64_t nb_cap, const int32_t *lens_prev, const int32_t *lens_now,
                      int32_t max_new_blocks, hipStream_t stream);
int launch_cobs_select(const void *sel, int G, const void *stats, int64_t stats_nb, int dtype,
                       int B, int Hkv, int64_t T_cap, const int32_t *seq_lens,
                       const sa_select_params &p,
                       int order, int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                       float *block_scores_out, void *workspace, hipStream_t stream,
                       FusedSelect *fs = nullptr);

int32_t prefill_tile_cap(int64_t q_start, int64_t Tq, const sa_select_params &p);
size_t prefill_workspace_bytes(int Hq, int Hkv, int64_t q_start, int64_t Tq,
                               const sa_select_params &p);
int launch_prefill(const void *Q, int64_t q_start, int64_t Tq, const void *K, const void *V,
                   const void *Kc, int Hq, int Hkv, int64_t T_cap, int64_t nc_cap,
                   const sa_select_params &p, float scale, void *O, int out_dtype, float *lse_out,
                   int32_t *tile_idx, int32_t tile_idx_cap, int32_t *tile_cnt, void *workspace,
                   hipStream_t stream);

int launch_prefill_attend(const void *Q, int64_t q_start, int64_t Tq, const void *K, const void *V,
                          int Hq, int Hkv, int64_t T_cap, const int32_t *tile_idx,
                          int32_t tile_idx_cap, const int32_t *tile_cnt, float scale, void *O,
                          int out_dtype, float *lse_out, hipStream_t stream);

size_t block_mass_workspace_bytes(int B, int Hq, int64_t nb_cap);
int launch_block_mass(const void *Q, const void *K, int dtype, int B, int Hq, int Hkv, int64_t T_cap,
                      const int32_t *seq_lens, float scale, float *mass, int64_t nb_cap,
                      const int32_t *idx, const int32_t *cnt, int idx_cap, float *recall,
                      void *workspace, hipStream_t stream);

constexpr int kStreamReadBlocks = 2048;   // workgroups of the stream-read grid
constexpr int kMaxSplit = 64;              // decode workgroups per (b, kvh); 64 blocks per split
int launch_stream_read(const void *buf, size_t bytes, uint32_t *xor_out, hipStream_t stream);

}  // namespace sa
