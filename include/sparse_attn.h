/*
 * sparse_attn.h - C ABI of the MI355X (gfx950) block-sparse attention library
 * (libsparse_attn.so).
 *
 * The method: keys are mean-pooled into compressed keys, a query (or one
 * Forecast vector per GQA group) scores them, scores are aggregated to
 * 64-token blocks, the top-k blocks are unioned with the initial and local
 * blocks, and attention with an online softmax runs over only that union.
 * Sources: the page "SparDA: Sparse Decoupled Attention for Efficient
 * Long-Context LLM Inference" (picx.dev summary), sections "Theoretical
 * Foundation" (Eq. 1, Eq. 2) and "Methodology" (Eq. 4, Eq. 5, "Compact
 * Forecast Indexer", Eq. 6); tile-shared prefill selection and cross-layer
 * index reuse follow the Kascade and CLSA abstracts on the pages "CoSA ..."
 * and "HySparse2 ...".
 *
 * Common rules for every entry point:
 *  - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *    The library never allocates or frees memory; scratch memory is a
 *    caller-provided device workspace whose size the *_workspace_size
 *    functions return (0 means no workspace is needed; then it may be NULL).
 *  - Tensors are dense, row-major, innermost dimension last (the ABI takes
 *    no strides: every kernel addresses a (sequence, KV head) slice as one
 *    contiguous [T_cap, d] window through a single buffer resource whose
 *    hardware range check bounds every access; callers with strided caches
 *    pass a dense copy or a dense per-layer allocation):
 *      K, V  [B, Hkv, T_cap, d]     (prefill: B = 1)
 *      Kc    [B, Hkv, nc_cap, d]    compressed keys, same dtype as K
 *      Q     [B, Hq, d] (decode) or [Tq, Hq, d] (prefill chunk of one sequence)
 *      sel   [B, H_sel, d]          selector vectors (Q itself, or Forecast F)
 *    Every row of d elements starts 16-byte aligned (true for dense tensors
 *    with d = 128). Only d = 128 is supported.
 *  - dtype is SA_F32 or SA_BF16 and applies to all of Q, K, V, Kc and sel.
 *    Arithmetic is fp32 (products, sums, softmax), outputs O are fp32 or bf16
 *    (out_dtype), log-sum-exp outputs are fp32 natural logarithms.
 *  - GQA: G = Hq / Hkv query heads share a KV head; query head h uses KV head
 *    h / G. Hq must be a multiple of Hkv. Decode attention (sparse_attn_decode,
 *    the decode steps, sparse_attn_token_decode) takes G in {1, 2, 4, 8};
 *    prefill and the block-mass measurement take G = 4.
 *  - seq_lens is a DEVICE int32 array [B]: the visible length L of each
 *    sequence, 0 <= L <= T_cap. Kernels clamp values outside that range into
 *    it so that no access leaves the tensors; the results are then undefined.
 *  - Every call only enqueues work on the given hipStream_t (NULL = the
 *    default stream) and returns without synchronising. Outputs are valid once
 *    the stream reaches that point. Calls that share a workspace must be
 *    ordered on one stream.
 *  - Arguments are validated on the host before any HIP call. Every function
 *    returns SA_OK (0) or a negative status; sparse_attn_status_string gives
 *    its text. On an error nothing has been enqueued. A launch failure
 *    reported by HIP returns SA_ERR_HIP.
 *  - No global mutable state; calls on different streams with different
 *    buffers may run concurrently.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_ABI_VERSION 1

/* status codes */
#define SA_OK               0
#define SA_ERR_INVALID_ARG (-1)  /* null pointer, bad size, inconsistent shapes */
#define SA_ERR_UNSUPPORTED (-2)  /* valid but not implemented (d != 128, GQA ratio, ...) */
#define SA_ERR_WORKSPACE   (-3)  /* workspace missing or smaller than required */
#define SA_ERR_CAPACITY    (-4)  /* an output or cache capacity is too small */
#define SA_ERR_HIP         (-5)  /* a HIP launch reported an error */

/* element types */
#define SA_F32  0
#define SA_BF16 1

/* how the G selector heads of a group combine their scores of a compressed entry */
#define SA_SCORE_SOFTMAX_SUM 0  /* sum over heads of each head's softmax over all entries (Eq. 6 form) */
#define SA_SCORE_RAW_SUM     1  /* sum over heads of raw dot products (Eq. 4; one Forecast: its dot) */

typedef struct sa_select_params {
    int32_t block_size;  /* tokens per KV block: must be 64 */
    int32_t cmp_kernel;  /* compression window l of Eq. 2: must be 32 */
    int32_t cmp_stride;  /* compression stride s of Eq. 2: must be 16 */
    int32_t top_k;       /* blocks chosen by score, >= 0 */
    int32_t n_init;      /* initial blocks always kept, >= 0 */
    int32_t n_local;     /* most recent blocks always kept, >= 0 */
    int32_t score_mode;  /* SA_SCORE_SOFTMAX_SUM or SA_SCORE_RAW_SUM */
} sa_select_params;

/* Returns SPARSE_ATTN_ABI_VERSION of the loaded library. */
int sparse_attn_abi_version(void);

/* Static text for a status code (never NULL). */
const char *sparse_attn_status_string(int status);

/*
 * sparse_attn_compress - Eq. 2: compressed entry j is the mean of keys
 * 16j .. 16j+31 (kernel 32, stride 16). Only complete windows exist:
 * n_c(L) = (L - 32) / 16 + 1 for L >= 32, else 0.
 *
 * Writes, for every sequence b, the entries j in [n_c(lens_prev[b]),
 * n_c(lens_now[b])) of Kc from K; other entries are left untouched. A bulk
 * build passes lens_prev = 0; a decode-time append passes the previous
 * lengths, so only windows completed by the new tokens are formed.
 * Each entry is one exact value: the window sum is the fp32 sum of two fp32
 * partial sums of 16 consecutive keys each, accumulated in token order, then
 * multiplied by 1/32 and rounded to the key dtype (round to nearest even).
 *
 *   K          [B, Hkv, T_cap, d] device, read
 *   Kc         [B, Hkv, nc_cap, d] device, written; nc_cap >= n_c(T_cap)
 *   lens_prev, lens_now   device int32 [B], lens_prev <= lens_now <= T_cap
 *   max_new_entries  host hint: an upper bound on n_c(lens_now) - n_c(lens_prev)
 *                    over the batch; sizes the launch only (any value >= 1
 *                    gives correct results; pass n_c(T_cap) for a bulk build)
 * Errors: SA_ERR_INVALID_ARG (null pointers, sizes <= 0, bad dtype),
 *         SA_ERR_UNSUPPORTED (d != 128), SA_ERR_CAPACITY (nc_cap < n_c(T_cap)).
 */
int sparse_attn_compress(const void *K, void *Kc, int dtype, int B, int Hkv, int d,
                         int64_t T_cap, int64_t nc_cap, const int32_t *lens_prev,
                         const int32_t *lens_now, int32_t max_new_entries, void *stream);

/* Workspace bytes needed by sparse_attn_select (may be 0). */
size_t sparse_attn_select_workspace_size(int B, int Hkv, int H_sel, int64_t T_cap,
                                         const sa_select_params *p);

/*
 * sparse_attn_select - Eq. 4 / Eq. 6 scoring and top-k, Eq. 1 union, per
 * (sequence b, KV head kvh) at visible length L = seq_lens[b].
 *
 * Scores: with H_sel = G * Hkv selector heads (the decode queries, G = Hq/Hkv)
 * or H_sel = Hkv (one Forecast vector per group, "Compact Forecast Indexer"),
 * the group's heads score every compressed entry j < n_c(L):
 *   SOFTMAX_SUM: S_j = sum_h softmax_j(sel_h . Kc_j)    (softmax over j < n_c(L))
 *   RAW_SUM:     S_j = sum_h sel_h . Kc_j
 * Block b's score is the max of S_j over the entries whose window lies wholly
 * inside the block (4b, 4b+1, 4b+2). With nb = ceil(L / 64) visible blocks,
 * init = [0, min(n_init, nb)), local = [max(0, nb - n_local), nb), and the
 * top_k blocks by score among the rest (ties to the lower block index) are
 * unioned with init and local.
 *
 *   sel        [B, H_sel, d] device
 *   Kc         [B, Hkv, nc_cap, d] device, valid for j < n_c(seq_lens[b])
 *   T_cap      largest possible L; nc_cap >= n_c(T_cap)
 *   idx_out    [B, Hkv, idx_cap] device int32: the union in ascending block
 *              order, padded with -1; idx_cap >= top_k + n_init + n_local
 *   cnt_out    [B, Hkv] device int32: number of valid entries of each row
 *   block_scores_out  optional [B, Hkv, ceil(T_cap/64)] device fp32: each
 *              block's score (-inf when no complete window lies inside it)
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d != 128, H_sel not Hkv or
 *         a multiple of it with G in {1,2,4,8}, parameters other than
 *         64/32/16, ceil(T_cap/64) > 32768), SA_ERR_CAPACITY (idx_cap, nc_cap),
 *         SA_ERR_WORKSPACE.
 */
int sparse_attn_select(const void *sel, int H_sel, const void *Kc, int dtype, int B, int Hkv,
                       int d, int64_t T_cap, int64_t nc_cap, const int32_t *seq_lens,
                       const sa_select_params *p, int32_t *idx_out, int32_t idx_cap,
                       int32_t *cnt_out, float *block_scores_out, void *workspace,
                       size_t ws_bytes, void *stream);

/* Workspace bytes needed by sparse_attn_decode for this split count
 * (n_split <= 0 asks the library's choice for this shape). */
size_t sparse_attn_decode_workspace_size(int B, int Hq, int Hkv, int32_t idx_cap,
                                         int32_t n_split);

/*
 * sparse_attn_decode - Eq. 5 for one new token per sequence: query heads of
 * KV head kvh attend, with softmax scale `scale`, to the tokens t < L of the
 * blocks listed in idx[b, kvh, 0 .. cnt[b, kvh]) (any order, no duplicates).
 * The query sits at position L - 1. The work of each (b, kvh) is split over
 * n_split workgroups whose partial (max, sum, weighted values) are merged
 * with log-sum-exp weights.
 *
 *   Q          [B, Hq, d] device
 *   K, V       [B, Hkv, T_cap, d] device
 *   idx, cnt   as written by sparse_attn_select (idx_cap columns)
 *   O          [B, Hq, d] device, out_dtype SA_F32 or SA_BF16
 *   lse_out    optional [B, Hq] device fp32: natural log of the softmax
 *              denominator incl. scale (-inf when no token is selected)
 *   n_split    workgroups per (b, kvh), at most 64; <= 0 lets the library
 *              choose. A split holds at most 64 blocks, so the count is
 *              raised to at least ceil(idx_cap / 64) (idx_cap <= 4096).
 *   workspace  required when the split count is above 1: the split
 *              partials (fp32), merged by a second kernel on the same stream.
 * A (b, kvh) with cnt = 0 yields O = 0 and LSE = -inf.
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d != 128, G not 1, 2, 4
 *         or 8, n_split > 64, idx_cap > 4096, one (b, kvh) cache slice of
 *         T_cap * d elements taking 2 GiB or more),
 *         SA_ERR_WORKSPACE.
 */
int sparse_attn_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                       int Hkv, int d, int64_t T_cap, const int32_t *seq_lens,
                       const int32_t *idx, const int32_t *cnt, int32_t idx_cap, float scale,
                       void *O, int out_dtype, float *lse_out, int32_t n_split,
                       void *workspace, size_t ws_bytes, void *stream);

/* Split-K workgroups per (b, kvh) that sparse_attn_decode_step uses for the
 * attention with these arguments (n_split as passed to it: 0 = automatic); 0
 * for invalid arguments. sparse_attn_decode with this n_split over the step's
 * block sets gives the step's outputs up to fp32 summation order. */
int32_t sparse_attn_decode_step_splits(int dtype, int B, int Hkv, int64_t T_cap,
                                       const sa_select_params *p, int32_t idx_cap,
                                       int32_t max_new_tokens, int32_t n_split);

/* Workspace bytes needed by sparse_attn_decode_step (select and decode scratch). */
size_t sparse_attn_decode_step_workspace_size(int B, int Hq, int Hkv, int H_sel, int64_t T_cap,
                                              const sa_select_params *p, int32_t idx_cap,
                                              int32_t n_split);

/*
 * sparse_attn_decode_step - one whole decode step of the hot path in one call:
 * sparse_attn_compress over [lens_prev, lens_now) (Eq. 2 append), then
 * sparse_attn_select at L = lens_now (Eq. 1, Eq. 4 / Eq. 6), then
 * sparse_attn_decode (Eq. 5) with n_split = sparse_attn_decode_step_splits:
 * identical block sets and compressed keys, outputs equal up to fp32
 * summation order (the same kernels; the attention is one launch with the
 * top-k, see below).
 * In RAW_SUM mode the scorer reads the entries that existed at lens_prev
 * from Kc and forms any newer entry a candidate block needs from K with the
 * same arithmetic; the new entries are written to Kc by the attention launch
 * (see max_new_tokens) or by workgroups of the scoring launch. In
 * SOFTMAX_SUM mode the workgroup that owns a new entry forms it from K after
 * the entries it read from Kc, scores it
 * (so every head's running max / sum sees the same values in the same order
 * as after a separate append) and writes it to Kc.
 * With at most 2048 blocks (T_cap <= 131072), idx_cap <= 1024 and, in
 * SOFTMAX_SUM mode, at most 4 selector heads per KV head, there is no
 * separate top-k launch: every attention workgroup of a (b, kvh) takes that
 * unit's top-k and union from the block scores itself (the same device code
 * as the top-k kernel, so the same sets), and the unit's first workgroup
 * writes idx_out / cnt_out.
 *
 *   Q [B, Hq, d]; sel [B, H_sel, d]; K, V [B, Hkv, T_cap, d]; Kc [B, Hkv,
 *   nc_cap, d] (updated in place); lens_prev, lens_now device int32 [B];
 *   max_new_tokens host hint, the expected bound on lens_now - lens_prev:
 *   it only picks how the append is scheduled, never what is computed (in
 *   RAW_SUM mode, up to 16 with bf16 keys and the top-k inside the attention
 *   launch, each unit's last attention workgroup writes the new entries
 *   while it takes the top-k; otherwise, up to 16 with bf16 keys, each unit's
 *   first scoring workgroup, else an extra column of scoring workgroups);
 *   every entry in [n_c(lens_prev), n_c(lens_now)) is written in both modes
 *   whatever the hint;
 *   idx_out / cnt_out as in sparse_attn_select; O / lse_out as in
 *   sparse_attn_decode. Workspace: sparse_attn_decode_step_workspace_size.
 * Errors: those of the three calls it stands for.
 */
int sparse_attn_decode_step(const void *Q, const void *sel, int H_sel, const void *K, const void *V,
                            void *Kc, int dtype, int B, int Hq, int Hkv, int d, int64_t T_cap,
                            int64_t nc_cap, const int32_t *lens_prev, const int32_t *lens_now,
                            int32_t max_new_tokens, const sa_select_params *p, float scale,
                            int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out, void *O,
                            int out_dtype, float *lse_out, int32_t n_split, void *workspace,
                            size_t ws_bytes, void *stream);

/*
 * sparse_attn_decode_step_noalloc - for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): sparse_attn_decode_step with the same arguments except
 * the workspace, and the same results. Its scratch memory is a fixed array of
 * SA_NOALLOC_SCRATCH_BYTES per GPU inside the library (held until the process
 * ends); the call allocates nothing. Calls that overlap on one GPU (other
 * streams or host threads) share that array and race: order them.
 * Errors: those of sparse_attn_decode_step; SA_ERR_WORKSPACE when the step
 *         needs more scratch than SA_NOALLOC_SCRATCH_BYTES
 *         (sparse_attn_decode_step_workspace_size tells); SA_ERR_HIP when the
 *         array's device address cannot be obtained.
 */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int sparse_attn_decode_step_noalloc(const void *Q, const void *sel, int H_sel, const void *K,
                                    const void *V, void *Kc, int dtype, int B, int Hq, int Hkv,
                                    int d, int64_t T_cap, int64_t nc_cap,
                                    const int32_t *lens_prev, const int32_t *lens_now,
                                    int32_t max_new_tokens, const sa_select_params *p,
                                    float scale, int32_t *idx_out, int32_t idx_cap,
                                    int32_t *cnt_out, void *O, int out_dtype, float *lse_out,
                                    int32_t n_split, void *stream);

/* Columns needed per tile row of the prefill block sets: min(ceil(T/64),
 * 64 * top_k + n_init + n_local) for a context of T = q_start + Tq tokens. */
int32_t sparse_attn_prefill_tile_cap(int64_t q_start, int64_t Tq, const sa_select_params *p);

/* Workspace bytes needed by sparse_attn_prefill_chunk. */
size_t sparse_attn_prefill_workspace_size(int Hq, int Hkv, int64_t q_start, int64_t Tq,
                                          const sa_select_params *p);

/*
 * sparse_attn_prefill_chunk - causal prefill of Tq new queries at positions
 * q_start .. q_start+Tq-1 of one sequence whose context ends with them
 * (L = q_start + Tq). q_start must be a multiple of 64. Tile t holds queries
 * q_start+64t .. q_start+64t+63 (the last tile may be shorter), all inside
 * block bt = q_start/64 + t.
 *
 * Selection per query p (L = p + 1), per KV head: Eq. 4 / Eq. 6 scores over
 * entries j < n_c(p+1) with params->score_mode, block scores as in
 * sparse_attn_select, top_k among blocks other than init and the local window
 * [bt - n_local + 1, bt]. The tile's set is the union of its queries' top-k
 * sets, init and the local window (ascending). Each query of the tile then
 * attends causally (token t <= p) to that set, on matrix cores.
 *
 *   Q          [Tq, Hq, d] device
 *   K, V       [Hkv, T_cap, d] device, T_cap >= q_start + Tq
 *   Kc         [Hkv, nc_cap, d] device holding entries j < n_c(q_start + Tq)
 *              (run sparse_attn_compress over the chunk first)
 *   O          [Tq, Hq, d] device (out_dtype); lse_out optional [Tq, Hq] fp32
 *   tile_idx_out [n_tiles, Hkv, tile_idx_cap] device int32, written (ascending,
 *              -1 padded); tile_cnt_out [n_tiles, Hkv] device int32, written;
 *              tile_idx_cap >= sparse_attn_prefill_tile_cap(...)
 * Errors: SA_ERR_INVALID_ARG (incl. q_start % 64 != 0), SA_ERR_UNSUPPORTED
 *         (d != 128, G != 4, dtype != SA_BF16, parameters other than 64/32/16,
 *         more than 32768 blocks, or (63 Hkv + 1) * nb * 4 bytes of one tile's
 *         per-query block scores beyond 2^31 - 1), SA_ERR_CAPACITY,
 *         SA_ERR_WORKSPACE.
 */
int sparse_attn_prefill_chunk(const void *Q, int64_t q_start, int64_t Tq, const void *K,
                              const void *V, const void *Kc, int dtype, int Hq, int Hkv, int d,
                              int64_t T_cap, int64_t nc_cap, const sa_select_params *p,
                              float scale, void *O, int out_dtype, float *lse_out,
                              int32_t *tile_idx_out, int32_t tile_idx_cap, int32_t *tile_cnt_out,
                              void *workspace, size_t ws_bytes, void *stream);

/*
 * sparse_attn_prefill_attend - the attention half of sparse_attn_prefill_chunk
 * over caller-given tile block sets, e.g. the sets one anchor layer selected,
 * reused by the following layers (top-k indices computed in anchor layers and
 * reused in later layers, for prefill and decode: Kascade abstract on the page
 * "CoSA ..."). Each query of tile t attends causally (t <= p) to the blocks
 * tile_idx[t, kvh, 0 .. tile_cnt[t, kvh]) (ascending, each <= the tile's
 * block, no duplicates).
 *
 *   Q [Tq, Hq, d], K/V [Hkv, T_cap, d] device bf16; O [Tq, Hq, d] (out_dtype),
 *   lse_out optional [Tq, Hq] fp32; tile_idx [n_tiles, Hkv, tile_idx_cap],
 *   tile_cnt [n_tiles, Hkv] device int32.
 * Errors: SA_ERR_INVALID_ARG (incl. q_start % 64 != 0), SA_ERR_UNSUPPORTED
 *         (d != 128, G != 4, dtype != SA_BF16), SA_ERR_CAPACITY (T_cap).
 */
int sparse_attn_prefill_attend(const void *Q, int64_t q_start, int64_t Tq, const void *K,
                               const void *V, int dtype, int Hq, int Hkv, int d, int64_t T_cap,
                               const int32_t *tile_idx, int32_t tile_idx_cap,
                               const int32_t *tile_cnt, float scale, void *O, int out_dtype,
                               float *lse_out, void *stream);

/* Workspace bytes needed by sparse_attn_token_select. */
size_t sparse_attn_token_select_workspace_size(int B, int Hkv, int64_t T_cap);

/*
 * sparse_attn_token_select - token-level index, computed once and meant to be
 * reused by every layer that shares the KV cache (CLSA abstract on the page
 * "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing"; tokens
 * scored in a shared low-dimensional query-key space with one token set per
 * KV head: JSSA item on the "Sparse Attention" topic page).
 *
 * Per (sequence b, KV head kvh) at visible length L = seq_lens[b]: every
 * token t < L gets the raw score of Eq. 4 (SparDA summary page, one vector per
 * group, no softmax) against its index key, s_t = sum over the group's
 * selector vectors of sel . Ki_t, summed in fp32. The first n_init and the
 * last n_local visible tokens are always kept; the top_k of the other visible
 * tokens by score (exact; ties to the lower token index) are added.
 *
 *   sel        [B, H_sel, d_i] device: H_sel = Hkv (one Forecast per group) or
 *              a multiple of Hkv (the group's query heads, summed; at most 64)
 *   Ki         [B, Hkv, T_cap, d_i] device: index keys (the keys themselves
 *              with d_i = 128, or a 64-dimensional projection of them),
 *              valid for t < L
 *   idx_out    [B, Hkv, idx_cap] device int32: the kept and chosen token ids
 *              ascending, padded with -1; idx_cap >= top_k + n_init + n_local
 *   cnt_out    [B, Hkv] device int32: number of valid entries of each row
 *   scores_out optional [B, Hkv, T_cap] device fp32: s_t (-inf for t >= L)
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d_i not 64 or 128, more
 *         than 64 selector heads per group, B * Hkv > 65535, a (b, kvh) slice
 *         of T_cap * d_i elements taking 2 GiB or more), SA_ERR_CAPACITY,
 *         SA_ERR_WORKSPACE.
 */
int sparse_attn_token_select(const void *sel, int H_sel, const void *Ki, int dtype, int B, int Hkv,
                             int d_i, int64_t T_cap, const int32_t *seq_lens, int32_t top_k,
                             int32_t n_init, int32_t n_local, int32_t *idx_out, int32_t idx_cap,
                             int32_t *cnt_out, float *scores_out, void *workspace,
                             size_t ws_bytes, void *stream);

/* Workspace bytes needed by sparse_attn_token_decode for this split count
 * (n_split <= 0 asks the library's choice for this shape). */
size_t sparse_attn_token_decode_workspace_size(int B, int Hq, int Hkv, int32_t idx_cap,
                                               int32_t n_split);

/*
 * sparse_attn_token_decode - Eq. 5 for one new token per sequence over a
 * token list: the query heads of KV head kvh attend, with softmax scale
 * `scale`, to the tokens idx[b, kvh, 0 .. cnt[b, kvh]) (any order, no
 * duplicates; ids outside [0, L) are ignored), e.g. the list written by
 * sparse_attn_token_select and shared by several layers. Rows are gathered
 * one token at a time; 64 list entries form a tile, and tiles are split over
 * n_split workgroups per (b, kvh) whose partials are merged with log-sum-exp
 * weights, as in sparse_attn_decode.
 *
 *   Q [B, Hq, d], K/V [B, Hkv, T_cap, d] device; idx [B, Hkv, idx_cap] and
 *   cnt [B, Hkv] device int32; O [B, Hq, d] (out_dtype); lse_out optional
 *   [B, Hq] fp32 natural log of the softmax denominator (-inf when empty).
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d != 128, G not 1, 2, 4
 *         or 8, n_split > 64, idx_cap > 262144, a (b, kvh) cache slice of
 *         T_cap * d elements taking 2 GiB or more), SA_ERR_WORKSPACE.
 */
int sparse_attn_token_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq,
                             int Hkv, int d, int64_t T_cap, const int32_t *seq_lens,
                             const int32_t *idx, const int32_t *cnt, int32_t idx_cap, float scale,
                             void *O, int out_dtype, float *lse_out, int32_t n_split,
                             void *workspace, size_t ws_bytes, void *stream);

/*
 * sparse_attn_cobs_stats - per-block statistics for selection with a
 * second-order term (the COBS abstract on the page "CoSA: Accelerating
 * Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention":
 * block selection by attention mass, a cumulant expansion of it, and a
 * compressed second-order statistic stored per block; the pages give no
 * formula, and the reading here is the block mean plus the per-channel
 * variance, i.e. the diagonal of the keys' covariance).
 *
 * For every sequence b and every complete 64-token block j with
 * lens_prev[b] / 64 <= j < lens_now[b] / 64, writes
 *   stats[b, kvh, j, 0, :] = mean of keys 64j .. 64j+63
 *   stats[b, kvh, j, 1, :] = mean of (key - mean)^2 over the same keys
 * each a sum in a fixed fp32 order (the four 16-key quarter sums, each in
 * token order, added in quarter order) times 2^-6 (the variance uses the fp32
 * mean), rounded to the key dtype: one exact value. Other rows are left
 * untouched. Partial blocks get no statistics.
 *
 *   K          [B, Hkv, T_cap, d] device; stats [B, Hkv, nb_cap, 2, d] device,
 *              K's dtype, nb_cap >= T_cap / 64
 *   lens_prev, lens_now   device int32 [B]
 *   max_new_blocks  host hint: an upper bound on the new complete blocks per
 *              sequence (sizes the launch; pass nb_cap for a bulk build)
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d != 128, B * Hkv > 65535),
 *         SA_ERR_CAPACITY.
 */
int sparse_attn_cobs_stats(const void *K, void *stats, int dtype, int B, int Hkv, int d,
                           int64_t T_cap, int64_t nb_cap, const int32_t *lens_prev,
                           const int32_t *lens_now, int32_t max_new_blocks, void *stream);

/* Workspace bytes needed by sparse_attn_cobs_select. */
size_t sparse_attn_cobs_select_workspace_size(int B, int Hkv, int H_sel, int64_t T_cap,
                                              const sa_select_params *p);

/*
 * sparse_attn_cobs_select - block selection by the estimated attention mass
 * of each block (same reading as sparse_attn_cobs_stats): for selector head h
 * and a block with statistics, the estimated log-mass (less the common log 64)
 *   order 1:  e_h = sel_h . mean
 *   order 2:  e_h = sel_h . mean + 1/2 sum_c sel_hc^2 var_c
 * and the group's block score is, with params->score_mode,
 *   SOFTMAX_SUM: sum_h softmax over the blocks of e_h   (Eq. 6 form)
 *   RAW_SUM:     sum_h e_h                             (one Forecast: its e)
 * Blocks without statistics (the partial last block) score -inf. Then, as in
 * sparse_attn_select, the top_k candidate blocks (ties to the lower index)
 * are unioned with the initial and local blocks (Eq. 1 on the SparDA summary
 * page). idx_out / cnt_out / block_scores_out as in sparse_attn_select.
 *
 *   sel        [B, H_sel, d] device (H_sel = G * Hkv, G in {1, 2, 4, 8})
 *   stats      [B, Hkv, nb_cap, 2, d] device, written by sparse_attn_cobs_stats
 *              for the complete blocks of seq_lens[b]; nb_cap >= ceil(T_cap/64)
 *   order      1 or 2
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d != 128, G, parameters
 *         other than 64/32/16, ceil(T_cap/64) > 32768), SA_ERR_CAPACITY,
 *         SA_ERR_WORKSPACE.
 */
int sparse_attn_cobs_select(const void *sel, int H_sel, const void *stats, int dtype, int B,
                            int Hkv, int d, int64_t T_cap, int64_t nb_cap,
                            const int32_t *seq_lens, const sa_select_params *p, int32_t order,
                            int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out,
                            float *block_scores_out, void *workspace, size_t ws_bytes,
                            void *stream);

/* Workspace bytes needed by sparse_attn_cobs_decode_step (select and decode scratch). */
size_t sparse_attn_cobs_decode_step_workspace_size(int B, int Hq, int Hkv, int H_sel,
                                                   int64_t T_cap, const sa_select_params *p,
                                                   int32_t idx_cap, int32_t n_split);

/*
 * sparse_attn_cobs_decode_step - one decode step selected by block statistics
 * in one call: sparse_attn_cobs_stats over [lens_prev, lens_now) (statistics
 * of the blocks the new tokens complete), then sparse_attn_cobs_select at
 * L = lens_now, then sparse_attn_decode (Eq. 5); results identical to those
 * three calls. In RAW_SUM mode with at most 2048 blocks (T_cap <= 131072)
 * and idx_cap <= 1024 there is no separate top-k launch: every attention
 * workgroup of a (b, kvh) takes that unit's top-k and union from the block
 * scores itself (the same device code as the top-k kernel), and the unit's
 * first workgroup writes idx_out / cnt_out.
 *
 *   Q [B, Hq, d]; sel [B, H_sel, d]; K, V [B, Hkv, T_cap, d]; stats
 *   [B, Hkv, nb_cap, 2, d] (updated in place); lens_prev, lens_now device
 *   int32 [B]; max_new_blocks host hint as in sparse_attn_cobs_stats (0 = no
 *   statistics update); order 1 or 2; idx_out / cnt_out as in
 *   sparse_attn_cobs_select; O / lse_out / n_split as in sparse_attn_decode.
 *   Workspace: sparse_attn_cobs_decode_step_workspace_size.
 * Errors: those of the three calls it stands for.
 */
int sparse_attn_cobs_decode_step(const void *Q, const void *sel, int H_sel, const void *K,
                                 const void *V, void *stats, int dtype, int B, int Hq, int Hkv,
                                 int d, int64_t T_cap, int64_t nb_cap, const int32_t *lens_prev,
                                 const int32_t *lens_now, int32_t max_new_blocks,
                                 const sa_select_params *p, int32_t order, float scale,
                                 int32_t *idx_out, int32_t idx_cap, int32_t *cnt_out, void *O,
                                 int out_dtype, float *lse_out, int32_t n_split, void *workspace,
                                 size_t ws_bytes, void *stream);

/*
 * sparse_attn_block_mass - selection quality, not a step of the sparse path:
 * the exact attention mass of every 64-token block for the decode query of
 * each head (the sum of the block's dense attention probabilities, the
 * quantity the CoSA abstract on the page "CoSA ..." reduces block selection
 * to), and optionally the recall of a selected block set (the mass it
 * captures: one minus the rest bucket of Eq. 7 on the page "SparDA ...",
 * section "Training"). Reads every visible key.
 *
 *   Q [B, Hq, d], K [B, Hkv, T_cap, d] device, dtype SA_F32 or SA_BF16; the
 *   query of sequence b sits at position seq_lens[b] - 1 and sees t < seq_lens[b]
 *   (lengths clamped to [0, T_cap]); probabilities softmax_t(scale * q . k_t).
 *   mass_out  [B, Hq, mass_cap] device fp32, written (0 past a sequence's
 *             block count); mass_cap >= ceil(T_cap / 64)
 *   idx, cnt  optional block sets as produced by sparse_attn_select
 *             ([B, Hkv, idx_cap], [B, Hkv]); then recall_out [B, Hq] device
 *             fp32 is written (ids outside the sequence's blocks count 0)
 *   workspace >= sparse_attn_block_mass_workspace_size(B, Hq, mass_cap) bytes
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (d != 128, G != 4),
 *         SA_ERR_CAPACITY (mass_cap), SA_ERR_WORKSPACE.
 */
size_t sparse_attn_block_mass_workspace_size(int B, int Hq, int64_t mass_cap);
int sparse_attn_block_mass(const void *Q, const void *K, int dtype, int B, int Hq, int Hkv, int d,
                           int64_t T_cap, const int32_t *seq_lens, float scale, float *mass_out,
                           int64_t mass_cap, const int32_t *idx, const int32_t *cnt,
                           int32_t idx_cap, float *recall_out, void *workspace, size_t ws_bytes,
                           void *stream);

/*
 * sparse_attn_stream_read - measurement utility, not a step of the method: reads
 * a device buffer once with a whole-GPU grid (the HBM stream-read ceiling that
 * the bandwidth-bound kernels are compared against, next to the vendor peak).
 * Each of the sparse_attn_stream_read_blocks() workgroups writes the XOR of the
 * 32-bit words it read to xor_out[workgroup]; the XOR over all of xor_out is the
 * XOR of the whole buffer.
 *
 *   buf      device pointer, 16-byte aligned, caller-owned, read only
 *   bytes    > 0, multiple of 16
 *   xor_out  device uint32 [sparse_attn_stream_read_blocks()], written
 * Errors: SA_ERR_INVALID_ARG (null pointer, size or alignment), SA_ERR_HIP.
 */
int sparse_attn_stream_read_blocks(void);
int sparse_attn_stream_read(const void *buf, size_t bytes, uint32_t *xor_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
