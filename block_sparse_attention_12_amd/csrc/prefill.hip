// Chunked sparse prefill on matrix cores.
//
// Page "SparDA: Sparse Decoupled Attention for Efficient Long-Context LLM
// Inference" (picx.dev summary): per query, Eq. 6's group-summed softmax
// scores over the compressed keys (or raw Eq. 4 scores), block scores, top-k
// and the Eq. 1 union; Eq. 5 attention over the chosen blocks. Sharing one
// block set per 64-query tile follows the Kascade abstract on the page
// "CoSA ..." ("tile-level operations" for prefill).
//
// One sequence, queries q_start .. q_start+Tq-1 (q_start a multiple of 64).
// Tile t = queries q_start+64t .. +63, all inside block bt = q_start/64 + t.
// A workgroup owns one (tile, KV head): 64 queries x 4 heads = 256 rows
// (row = 4 * query + head). Both the scoring and the attention kernel give
// each of 8 waves (two per SIMD) 32 rows.
//
// Both dense contractions use v_mfma_f32_16x16x32_bf16 in the transposed form
// S^T = K Q^T (keys as M, rows as N), so each lane ends up with the scores of a
// single row and no data movement is needed between the score and the value
// products: O^T = V^T P^T, with P converted in registers to the B operand. The
// key order inside each K = 32 step is permuted identically on both operands.
// K (or compressed-key) tiles sit in LDS row-major with an XOR swizzle of their
// 16-byte chunks (conflict-free 16-row reads); V tiles row-major with their own
// swizzle, read as V^T operands with ds_read_b64_tr_b16.
//
// Softmax: a row's reference (log2 units) is the max of its first half block;
// probabilities are taken against it without rescaling the accumulators. In
// the attention kernel the row sums come from the matrix cores (the value
// product with an all-ones tile), and a pass whose row sum passes 2^64 is void:
// a pass that tracks the rows' maxima follows, then one against the raised
// references (the result does not depend on the reference, only overflow does).
//
// Kernels:
//   prefill_score_kernel  per (tile, KV head), two software-pipelined sweeps
//                         over the compressed keys: per-row softmax sum over
//                         the entries the row's query can see (lazy per-lane
//                         references), then the group-summed probabilities,
//                         max-reduced over each block's three inside entries,
//                         written as one score per (query, KV head, block).
//   topk (select.hip)     per (query, KV head): top-k among the blocks that
//                         are neither initial nor in the local window, plus
//                         init and local.
//   prefill_union_kernel  per (tile, KV head): union of its 64 queries' sets.
//   prefill_attn_kernel   per (tile, KV head): causal attention over the union,
//                         blocks staged through a 3-stage LDS ring (loads of
//                         the block after next in registers during the current
//                         one),
//                         softmax in fp32, P rounded to bf16 for the value
//                         product, fp32 accumulation.
// Workgroups are numbered tile * Hkv + kvh so the tiles of one KV head land on
// the same XCD (round-robin dispatch over 8 XCDs) and share its L2.
#include <math.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kPfThreads = 256;
constexpr int kPfG = 4;
constexpr float kLog2eF = 1.44269504088896340736f;
constexpr float kLn2F = 0.69314718055994530942f;

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &v) { return __builtin_bit_cast(bf16x8_t, v); }

// A operand (rows as M) from a swizzled LDS tile: row m_row, channels 32 ks + 8 g .. +8
__device__ __forceinline__ bf16x8_t lds_frag_rows(const bf16_t *lds, int m_row, int ks, int g) {
    const int chunk = (4 * ks + g) ^ (m_row & 15);
    return as_bf16x8(*reinterpret_cast<const uint4 *>(lds + m_row * kD + chunk * 8));
}

// V tiles use their own swizzle: chunk c of row r at c ^ 2 (r % 8). A transposed
// read of 8 rows x 32 bytes (one half of a ds_read_b64_tr_b16) then touches 16
// distinct chunks, all 64 banks once.
__device__ __forceinline__ int vt_swizzle(int row) { return 2 * (row & 7); }

// A operand of V^T for the value product from a swizzled row-major V tile
// (the attention kernel's v_frag): channel row 16 ct + (l%16), permuted keys
// of step kk: slots 0..3 hold keys 32kk + 4g .. +3, slots 4..7 keys 32kk + 16
// + 4g .. +3. ds_read_b64_tr_b16 transposes inside each 16-lane group: output
// lane i, element j comes from source lane 4j + i/4, element i%4, so source
// lane s reads key row key0 + s/4 at channels 16 ct + 4 (s%4) .. +3.
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Two fp32 values to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// Row mapping shared by the scoring and attention kernels: 8 waves per
// workgroup (two per SIMD, so one wave's vector work overlaps the other's
// matrix work), each owning 32 rows = 8 queries x 4 heads of the tile as two
// 16-row tiles (row = 4 * query + head).
constexpr int kAtWaves = 8;
constexpr int kAtThreads = 64 * kAtWaves;
constexpr int kAtRt = 2;
constexpr int kPfTileElems = 64 * kD;             // one 64 x 128 bf16 tile (16 KB)


// This wave's query rows as B operands: qf[rt][ks] = Q[row 16 rt + (l%16)][32 ks + 8 g .. +8]
// (zeros for queries past the chunk); qloc[rt] = the lane's query offset in the tile.
__device__ __forceinline__ void load_q_frags(bf16x8_t (&qf)[kAtRt][4], int (&qloc)[kAtRt], const bf16_t *Q,
                                             int Hq, int kvh, int64_t q_first, int64_t Tq, int wave,
                                             int lane) {
    const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) {
        qloc[rt] = 8 * wave + 4 * rt + (c16 >> 2);
        const int64_t qi = q_first + qloc[rt];
        const int h = c16 & 3;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qi < Tq)
                v = *reinterpret_cast<const uint4 *>(Q + (qi * Hq + (int64_t)kvh * kPfG + h) * kD +
                                                     32 * ks + 8 * g);
            qf[rt][ks] = as_bf16x8(v);
        }
    }
}

// A 64 x 128 tile staged global -> registers -> LDS: this thread's two 16-byte
// chunks, thread t's load r filling chunk slot 512 r + t of the tile, each slot
// fetching the source chunk that the swizzle puts there (K swizzle c ^ (r%16),
// or the V swizzle). Rows outside the buffer read as zeros.
struct TileRegs {
    Raw8<bf16_t> c[2];
};
__device__ __forceinline__ int vt_swizzle(int row);
template <bool V_SWIZZLE>
__device__ __forceinline__ void load_tile_regs(TileRegs &tr, __amdgpu_buffer_rsrc_t src, int64_t row0,
                                               int tid) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int slot = kAtThreads * r + tid;
        const int row = slot >> 4;
        const int sw = V_SWIZZLE ? vt_swizzle(row) : (row & 15);
        load_raw(src, row_offset(row0 + row, kD * 2, ((slot & 15) ^ sw) * 16), tr.c[r]);
    }
}
__device__ __forceinline__ void store_tile_lds(bf16_t *lds, const TileRegs &tr, int tid) {
#pragma unroll
    for (int r = 0; r < 2; ++r) *reinterpret_cast<uint4 *>(lds + (kAtThreads * r + tid) * 8) = tr.c[r].v;
}

// The attention kernel keeps the K swizzle (measured free of LDS bank
// conflicts; rows padded to 272 bytes instead measured a 2-way conflict on
// these 16-byte reads) and stages V unswizzled in rows padded to 288 bytes: a
// transposed read of 8 rows x 32 bytes then starts 8 banks further per row
// (measured conflict-free), and every V fragment address is one per-lane base
// plus a constant.
constexpr int kAtKRow = 2 * kD;
constexpr int kAtVRow = 2 * kD + 32;
// Thread t loads the 16-byte chunks t % 16 of rows t / 16 and 32 + t / 16 of
// a 64-row block starting blk_bytes into src (the block offset in the scalar
// offset, the lane part fixed).
__device__ __forceinline__ void load_tile_rows(TileRegs &tr, __amdgpu_buffer_rsrc_t src, uint32_t blk_bytes,
                                               uint32_t lane_off) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const sa_v4i v = __builtin_amdgcn_raw_buffer_load_b128(src, (int)lane_off, (int)(blk_bytes + r * 32 * 2 * kD), 0);
        tr.c[r].v = make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
    }
}

// Scores S^T = K Q^T of half a tile (keys 32hh .. 32hh+31) for this wave's rows:
// s[j][rt][i] = score of row 16 rt + (l%16) with key 32hh + 16j + 4g + i.
__device__ __forceinline__ void half_scores(f32x4_t (&s)[2][kAtRt], const bf16_t *sK,
                                            const bf16x8_t (&qf)[kAtRt][4], int hh, int g, int c16) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) s[j][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8_t a = lds_frag_rows(sK, 32 * hh + 16 * j + c16, ks, g);
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) s[j][rt] = mfma16(a, qf[rt][ks], s[j][rt]);
        }
}

// ------------------------------------------------------------------ scoring

// Visible compressed entries for a query at position p: n_c(p + 1). The
// compressed keys go through a 2-stage LDS ring of 64-entry chunks, and each
// sweep is software-pipelined: the matrix products of chunk c + 1 sit in the
// same straight-line block as the vector work on chunk c's scores, so one
// wave keeps its matrix and vector pipes busy together (chunk c + 2's loads
// are in registers meanwhile). Chunks below what the tile's first query sees
// need no visibility mask; the rest take it.
//
// Softmax denominators (sweep 1) use a lazy reference per lane: the max of the
// lane's scores in chunk 0 (log2 units); every term is exp2(x - ref) with no
// running max. The sum does not depend on the reference beyond rounding; only
// overflow does, so a lane whose sum exceeds 2^64 (some later score above its
// reference by more than 64) makes the workgroup rerun sweep 1 with a running
// max. Sweep 2 takes each probability as exp2(x - (m + log2 z)) of the row's
// merged (m, z).
constexpr float kScoreSumLimit = 18446744073709551616.f;   // 2^64

template <bool RAW>
__global__ __launch_bounds__(kAtThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_score_kernel(
    const bf16_t *__restrict__ Q, const bf16_t *__restrict__ Kc, int Hq, int Hkv, int64_t q_start,
    int64_t Tq, int64_t nc_cap, float *__restrict__ bscore, int64_t nb_cap,
    int32_t *__restrict__ qlens) {
    __shared__ __align__(16) bf16_t ring[2 * kPfTileElems];
    const int tile = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t q_first = (int64_t)tile * 64;                  // query index of the tile start
    const int64_t bt = q_start / kBlock + tile;
    if (kvh == 0 && tid < 64 && q_first + tid < Tq) qlens[q_first + tid] = (int32_t)(q_start + q_first + tid + 1);

    int qloc[kAtRt];
    bf16x8_t qf[kAtRt][4];
    load_q_frags(qf, qloc, Q, Hq, kvh, q_first, Tq, wave, lane);
    int nvis[kAtRt];                                             // visible entries of the lane's row
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) {
        const int64_t qi = q_first + qloc[rt];
        nvis[rt] = qi < Tq ? (int)n_compressed(q_start + qi + 1) : 0;
    }
    const __amdgpu_buffer_rsrc_t rKc = make_rsrc(Kc + (int64_t)kvh * nc_cap * kD,
                                                (uint32_t)(nc_cap * kD * 2));
    // block scores of this tile's queries for this KV head: query qloc at byte
    // qloc * Hkv * nb_cap * 4 (the launcher checks the span fits 31 bits);
    // queries past the chunk fall outside the resource and are not written
    const int64_t nq = Tq - q_first < 64 ? Tq - q_first : 64;
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(
        bscore + (q_first * Hkv + kvh) * nb_cap, (uint32_t)(((nq - 1) * Hkv + 1) * nb_cap * 4));
    uint32_t qoff[kAtRt];
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) qoff[rt] = (uint32_t)((int64_t)qloc[rt] * Hkv * nb_cap * 4);
    const int n_chunks = (int)(bt / 16) + 1;                     // every block <= bt is covered
    const int vis_min = (int)n_compressed(q_start + q_first + 1);
    const int n_full = vis_min / 64 < n_chunks ? vis_min / 64 : n_chunks;
    const int nbc = (int)nb_cap;                                 // <= 32768 blocks

    // scores of a staged chunk: s[mt][rt][i] for entry 16 mt + 4g + i of it
    auto chunk_scores = [&](f32x4_t (&s)[4][kAtRt], const bf16_t *sK) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            f32x4_t h[2][kAtRt];
            half_scores(h, sK, qf, hh, g, c16);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int rt = 0; rt < kAtRt; ++rt) s[2 * hh + j][rt] = h[j][rt];
        }
    };
    // entries of chunk c past the row's visible count become -inf
    auto mask = [&](f32x4_t (&s)[4][kAtRt], int c) {
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) {
            const int lim = nvis[rt] - 64 * c - 4 * g;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * mt + i >= lim) s[mt][rt][i] = -INFINITY;
        }
    };
    // one sweep: first(s) on chunk 0's scores, then body(s, c) for every chunk
    auto sweep = [&](auto first, auto body) {
        TileRegs rk;
        load_tile_regs<false>(rk, rKc, 0, tid);
        store_tile_lds(ring, rk, tid);
        load_tile_regs<false>(rk, rKc, 64, tid);                 // rows past the buffer read zeros
        __syncthreads();
        f32x4_t cur[4][kAtRt];
        chunk_scores(cur, ring);
        if (n_full == 0) mask(cur, 0);
        first(cur);
        store_tile_lds(ring + kPfTileElems, rk, tid);
        // Loads, stores and products past the last chunk are not skipped (rows
        // past the buffer read zeros; their slots and scores go unused), which
        // keeps the products and the vector work in one branch-free block.
        for (int c = 0; c < n_chunks; ++c) {
            __syncthreads();                       // chunk c + 1 staged; chunk c's slot is free
            load_tile_regs<false>(rk, rKc, (int64_t)(c + 2) * 64, tid);
            if (c >= n_full) mask(cur, c);
            f32x4_t nxt[4][kAtRt];
            chunk_scores(nxt, ring + ((c + 1) & 1) * kPfTileElems);
            body(cur, c);
            store_tile_lds(ring + (c & 1) * kPfTileElems, rk, tid);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int rt = 0; rt < kAtRt; ++rt) cur[mt][rt] = nxt[mt][rt];
        }
        __syncthreads();                           // ring free for the next sweep
    };

    // sweep 1 (softmax mode): per-row max and sum of exp over visible entries
    // (base 2), per lane, then merged over the 4 lanes sharing a row
    float m[kAtRt], z[kAtRt];
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) { m[rt] = -INFINITY; z[rt] = 0.f; }
    if constexpr (!RAW) {
        sweep([&](f32x4_t (&s)[4][kAtRt]) {
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) {
                float mx = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][rt][i]);
                m[rt] = mx == -INFINITY ? 0.f : mx * kLog2eF;        // lane with nothing visible: z stays 0
            }
        }, [&](f32x4_t (&s)[4][kAtRt], int) {
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) {
                float acc = z[rt];
                const float nm = -m[rt];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc += __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][rt][i], kLog2eF, nm));
                z[rt] = acc;
            }
        });
        bool over = false;
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) over |= !(z[rt] <= kScoreSumLimit);
        if (__syncthreads_or(over)) {
            // rerun with a running max (scores spread far beyond the references)
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) { m[rt] = -INFINITY; z[rt] = 0.f; }
            sweep([&](f32x4_t (&)[4][kAtRt]) {}, [&](f32x4_t (&s)[4][kAtRt], int) {
#pragma unroll
                for (int rt = 0; rt < kAtRt; ++rt) {
                    float x[16];
                    float mx = m[rt];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            x[4 * mt + i] = s[mt][rt][i] * kLog2eF;
                            mx = fmaxf(mx, x[4 * mt + i]);
                        }
                    if (mx != -INFINITY) {
                        float acc = z[rt] * __builtin_amdgcn_exp2f(m[rt] - mx);
#pragma unroll
                        for (int k = 0; k < 16; ++k) acc += __builtin_amdgcn_exp2f(x[k] - mx);
                        z[rt] = acc;
                        m[rt] = mx;
                    }
                }
            });
        }
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) {
            if (!(z[rt] > 0.f)) m[rt] = -INFINITY;                      // nothing visible in this lane
#pragma unroll
            for (int sh = 16; sh <= 32; sh <<= 1) {
                const float m2 = shfl_xor(m[rt], sh), z2 = shfl_xor(z[rt], sh);
                const float mn = fmaxf(m[rt], m2);
                if (mn != -INFINITY) {
                    z[rt] = z[rt] * __builtin_amdgcn_exp2f(m[rt] - mn) + z2 * __builtin_amdgcn_exp2f(m2 - mn);
                    m[rt] = mn;
                }
            }
        }
    }
    // probability of a score: exp2(x log2 e - bias), bias = m + log2 z (+inf
    // for a row that sees nothing, so every probability is 0)
    float nbias[kAtRt];
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) nbias[rt] = z[rt] > 0.f ? -(m[rt] + log2f(z[rt])) : -INFINITY;

    // sweep 2: probabilities (or raw scores) summed over the 4 heads of a query
    // (lanes 4k .. 4k+3 of a row group), max over each block's inside entries
    // 4b, 4b+1, 4b+2 (lane g holds block 16c + 4mt + g), one score per
    // (query, KV head, block). Masked entries give probability 0 (raw: -inf in
    // every head's sum); a block whose first inside entry is masked is -inf.
    sweep([&](f32x4_t (&)[4][kAtRt]) {}, [&](f32x4_t (&s)[4][kAtRt], int c) {
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float v[3];
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    float pv = RAW ? s[mt][rt][i]
                                   : __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][rt][i], kLog2eF, nbias[rt]));
                    pv += dpp<kDppQuadXor1>(pv);
                    pv += dpp<kDppQuadXor2>(pv);
                    v[i] = pv;
                }
                const int blk = 16 * c + 4 * mt + g;
                float bs = fmaxf(fmaxf(v[0], v[1]), v[2]);
                if (!RAW) bs = 4 * blk >= nvis[rt] ? -INFINITY : bs;
                const uint32_t off = ((c16 & 3) == 0 && blk < nbc) ? qoff[rt] + 4u * (uint32_t)blk
                                                                     : 0xffffffffu;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bs), rB, (int)off, 0, 0);
            }
        }
    });
}

// ------------------------------------------------------------------ union

__global__ __launch_bounds__(kPfThreads) void prefill_union_kernel(
    const int32_t *__restrict__ qidx, const int32_t *__restrict__ qcnt, int qcap, int Hkv,
    int64_t q_start, int64_t Tq, int32_t *__restrict__ tile_idx, int tile_cap,
    int32_t *__restrict__ tile_cnt) {
    __shared__ uint32_t s_bits[32768 / 32];
    __shared__ int s_wave[kPfThreads / 64];
    const int tile = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
    const int tid = threadIdx.x;
    const int64_t bt = q_start / kBlock + tile;
    const int nb = (int)bt + 1;
    const int words = (nb + 31) / 32;
    for (int w = tid; w < words; w += kPfThreads) s_bits[w] = 0u;
    __syncthreads();
    const int64_t q_first = (int64_t)tile * 64;
    const int nq = (int)(Tq - q_first < 64 ? Tq - q_first : 64);
    for (int e = tid; e < nq * qcap; e += kPfThreads) {
        const int q = e / qcap, k = e % qcap;
        const int64_t unit = (q_first + q) * Hkv + kvh;
        if (k < qcnt[unit]) {
            const int blk = qidx[unit * qcap + k];
            if (blk >= 0 && blk < nb) atomicOr(&s_bits[blk >> 5], 1u << (blk & 31));
        }
    }
    __syncthreads();
    // ascending compaction: thread t owns words t*per .. t*per+per-1
    const int per = (words + kPfThreads - 1) / kPfThreads;
    const int lo = tid * per < words ? tid * per : words;
    const int hi = lo + per < words ? lo + per : words;
    int n = 0;
    for (int w = lo; w < hi; ++w) n += __popc(s_bits[w]);
    // workgroup exclusive scan
    const int lane = tid & 63, wave = tid >> 6;
    int v = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPfThreads / 64; ++w) {
        if (w < wave) base += s_wave[w];
        total += s_wave[w];
    }
    int pos = base + v - n;
    int32_t *row = tile_idx + (int64_t)blockIdx.x * tile_cap;
    for (int w = lo; w < hi; ++w) {
        uint32_t bits = s_bits[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            if (pos < tile_cap) row[pos] = w * 32 + b;
            ++pos;
        }
    }
    for (int i = total + tid; i < tile_cap; i += kPfThreads) row[i] = -1;
    if (tid == 0) tile_cnt[blockIdx.x] = total < tile_cap ? total : tile_cap;
}

// ------------------------------------------------------------------ attention

// A pass is kept when every row sum of probabilities (against the row's
// reference, log2 units) stays within 2^kRescaleSlack: every probability is then
// below it too, far from fp32 / bf16 overflow. The result does not depend on the
// reference: numerator and denominator share it.
constexpr float kRescaleSlack = 64.f;
constexpr float kSumLimit = 18446744073709551616.f;     // 2^kRescaleSlack
// Passes over a tile's blocks: at most fast, tracking, fast (the cap only
// bounds the loop).
constexpr int kPfMaxPasses = 4;

__global__ __launch_bounds__(kAtThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(
    const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ V,
    int Hq, int Hkv, int64_t q_start, int64_t Tq, int64_t T_cap, const int32_t *__restrict__ tile_idx,
    int tile_cap, const int32_t *__restrict__ tile_cnt, float qscale, void *__restrict__ O,
    int out_bf16, float *__restrict__ lse) {
    // three K stages, then three V stages (block e in stage e % 3 of each),
    // rows of kAtKRow / kAtVRow bytes
    __shared__ __align__(16) char ring[3 * 64 * (kAtKRow + kAtVRow)];
    __shared__ int s_redo[kPfMaxPasses];
    constexpr uint32_t kKTile = 64 * kAtKRow, kVTile = 64 * kAtVRow, kVStages = 3 * kKTile;
    const int tile = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t q_first = (int64_t)tile * 64;
    const int64_t bt = q_start / kBlock + tile;
    if (tid < kPfMaxPasses) s_redo[tid] = 0;

    int qloc[kAtRt];                               // query offset inside the tile, per row tile
    bf16x8_t qf[kAtRt][4];
    load_q_frags(qf, qloc, Q, Hq, kvh, q_first, Tq, wave, lane);

    f32x4_t o[8][kAtRt];
    // per row tile: the row sums (every element of a lane holds its row's sum),
    // reference (log2 units), running max (tracking passes only)
    f32x4_t osum[kAtRt];
    float m[kAtRt], mrun[kAtRt];
    const bf16x8_t ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) m[rt] = -INFINITY;

    const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + (int64_t)kvh * T_cap * kD, (uint32_t)(T_cap * kD * 2));
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + (int64_t)kvh * T_cap * kD, (uint32_t)(T_cap * kD * 2));
    typedef const __attribute__((address_space(4))) int32_t const_i32_t;   // scalar loads
    const_i32_t *ids = (const_i32_t *)(tile_idx + (int64_t)blockIdx.x * tile_cap);
    int n = tile_cnt[blockIdx.x];
    n = n < 0 ? 0 : (n > tile_cap ? tile_cap : n);
    auto blk_at = [&](int e) -> int64_t { return ids[__builtin_amdgcn_readfirstlane(e)]; };

    // Per-lane LDS byte offsets, fixed for the kernel: every fragment read and
    // staging store below is one of these plus a constant (stage, key rows,
    // channels), which the LDS instructions take as their immediate offset.
    // K fragment of channel step ks: key row c16 (+ 32hh + 16j), swizzled
    // chunk (4ks + g) ^ c16. V^T fragment: key row vrow (+ 32kk + 16 half),
    // channels 4 (c16 % 4) .. +3 (+ 16ct). Staging: row tid / 16 (+ 32r),
    // 16-byte chunk slot tid % 16, which for K holds the source chunk the
    // swizzle puts there.
    const int vrow = 4 * g + (c16 >> 2);
    uint32_t koff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = (uint32_t)(c16 * kAtKRow + (((4 * ks + g) ^ c16) << 4));
    uint32_t voff = kVStages + (uint32_t)(vrow * kAtVRow + 8 * (c16 & 3));
    uint32_t kst = (uint32_t)(tid * 16);
    uint32_t vst = kVStages + (uint32_t)((tid >> 4) * kAtVRow + (tid & 15) * 16);
    // global lane offsets in a block (K: the swizzled source chunk)
    uint32_t gofs_k = (uint32_t)((tid >> 4) * 2 * kD + (((tid & 15) ^ ((tid >> 4) & 15)) << 4));
    uint32_t gofs_v = (uint32_t)((tid >> 4) * 2 * kD + (tid & 15) * 16);
    char *lds = ring;
    auto k_frag = [&](uint32_t off) { return as_bf16x8(*reinterpret_cast<const uint4 *>(lds + off)); };
    auto v_frag = [&](uint32_t off) {                  // rows off and off + 16 rows, transposed
        const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(lds + off));
        const s16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(lds + off + 16 * kAtVRow));
        typedef __attribute__((ext_vector_type(8))) short s16x8_t;
        const s16x8_t v = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        return __builtin_bit_cast(bf16x8_t, v);
    };

    // causal mask inside the tile's own block: key <= query
    auto mask_causal = [&](f32x4_t (&s)[2][kAtRt], int hh) {
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) {
            int q = qloc[rt] - 32 * hh - 4 * g;
            asm volatile("" : "+v"(q));            // compared here, not hoisted as lane masks
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * j + i > q) s[j][rt][i] = -INFINITY;
        }
    };
    // Exponents against the row references (TRACK: running max kept),
    // probabilities as bf16 B operands (keys 32hh + 4g + i for j = 0, then
    // 32hh + 16 + 4g + i). The row sums are taken by the value product.
    auto half_probs = [&](bf16x8_t (&pb)[kAtRt], const f32x4_t (&s)[2][kAtRt], auto track) {
        constexpr bool TRACK = decltype(track)::value;
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) {
            const float nm = -m[rt];
            float p[2][4];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[j][i] = __builtin_fmaf(s[j][rt][i], qscale, nm);
            if constexpr (TRACK)
                mrun[rt] = fmaxf(fmaxf(fmaxf(mrun[rt], fmaxf(p[0][0], p[0][1])), fmaxf(p[0][2], p[0][3])),
                                 fmaxf(fmaxf(p[1][0], p[1][1]), fmaxf(p[1][2], p[1][3])));
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[j][i] = __builtin_amdgcn_exp2f(p[j][i]);
            pb[rt] = as_bf16x8(make_uint4(cvt_pk_bf16(p[0][0], p[0][1]), cvt_pk_bf16(p[0][2], p[0][3]),
                                          cvt_pk_bf16(p[1][0], p[1][1]), cvt_pk_bf16(p[1][2], p[1][3])));
        }
    };
    // Scores of half hh (keys 32hh .. 32hh + 31) of the block staged at K
    // offsets kb (koff plus the stage): s[j][rt].
    auto half_scores_at = [&](f32x4_t (&s)[2][kAtRt], const uint32_t (&kb)[4], int hh) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) s[j][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8_t a = k_frag(kb[ks] + (uint32_t)(32 * hh + 16 * j) * kAtKRow);
#pragma unroll
                for (int rt = 0; rt < kAtRt; ++rt) s[j][rt] = mfma16(a, qf[rt][ks], s[j][rt]);
            }
    };
    // Probabilities of half hh's scores, then the value product O^T += V^T P^T
    // over its 32 keys from the V tile at offset vb (voff plus the stage), and
    // the row sums as one more product with an all-ones V^T tile (the sums of
    // the bf16 probabilities the value product weighs, on the matrix cores
    // instead of 16 vector additions per row tile and block).
    auto half_values = [&](const f32x4_t (&s)[2][kAtRt], uint32_t vb, int hh, auto track) {
        bf16x8_t pb[kAtRt];
        half_probs(pb, s, track);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const bf16x8_t a = v_frag(vb + 32 * ct + (uint32_t)(32 * hh) * kAtVRow);
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) o[ct][rt] = mfma16(a, pb[rt], o[ct][rt]);
        }
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) osum[rt] = mfma16(ones, pb[rt], osum[rt]);
    };
    // Issue order of one half step for the scheduler: the score products,
    // each pair after its K fragment read (reads run two ahead) and followed
    // by a share of the probabilities' vector work, then the value products
    // with their V fragment reads.
    auto half_step_order = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         // LDS reads
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);     // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);     // VALU
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    };

    // Blocks go through a 3-stage LDS ring (block e in stage e % 3), and the
    // loop is software-pipelined in half blocks: while one half's scores turn
    // into probabilities (vector work), the next half's scores are computed
    // (matrix products) in the same straight-line code, followed by the
    // first half's value product. Block e + 2's loads are in registers during
    // block e and go into the stage block e - 1 used; one barrier ends each
    // block. Loads, products and stores past the last block are not skipped
    // (they repeat the last block; their results go unused). The stage is one
    // offset added to the lane bases per block.
    // The reference of a row is the max of its first half block; a pass in
    // which some row's sum of probabilities passes 2^64 is void and the
    // workgroup runs its blocks again (accumulators are never rescaled; see the
    // end of the pass). The tile's own block, last in the ascending set, takes
    // the causal mask.
    const bool last_diag = n > 0 && blk_at(n - 1) == bt;
    bool track = false;                            // this pass keeps the running maxima
    for (int pass = 0; pass < kPfMaxPasses; ++pass) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) o[ct][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < kAtRt; ++rt) { osum[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; mrun[rt] = -INFINITY; }
        TileRegs rk, rv;
        auto load_block = [&](int64_t blk) {
            const uint32_t bb = (uint32_t)blk * (kBlock * 2 * kD);
            load_tile_rows(rk, rK, bb, gofs_k);
            load_tile_rows(rv, rV, bb, gofs_v);
        };
        auto store_block = [&](int st) {
            uint32_t kb = kst + (uint32_t)st * kKTile, vb = vst + (uint32_t)st * kVTile;
            asm volatile("" : "+v"(kb), "+v"(vb));
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                *reinterpret_cast<uint4 *>(lds + kb + r * 32 * kAtKRow) = rk.c[r].v;
                *reinterpret_cast<uint4 *>(lds + vb + r * 32 * kAtVRow) = rv.c[r].v;
            }
        };
        if (n > 0) {
            load_block(blk_at(0));
            store_block(0);
        }
        if (n > 1) {
            load_block(blk_at(1));
            store_block(1);
        }
        __syncthreads();
        f32x4_t sa[2][kAtRt], sb[2][kAtRt];        // scores of the first / second half
        half_scores_at(sa, koff, 0);
        if (n == 1 && last_diag) mask_causal(sa, 0);
        if (pass == 0 && n > 0) {                  // references from the first half block
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) {
                float mx = fmaxf(fmaxf(fmaxf(sa[0][rt][0], sa[0][rt][1]), fmaxf(sa[0][rt][2], sa[0][rt][3])),
                                 fmaxf(fmaxf(sa[1][rt][0], sa[1][rt][1]), fmaxf(sa[1][rt][2], sa[1][rt][3]))) *
                           qscale;
                mx = fmaxf(mx, shfl_xor(mx, 16));
                mx = fmaxf(mx, shfl_xor(mx, 32));
                m[rt] = mx == -INFINITY ? 0.f : mx;
            }
        }
        auto blocks = [&](auto trk) {
        for (int e = 0; e < n; ++e) {
            const int st = e % 3, st1 = st == 2 ? 0 : st + 1, st2 = st == 0 ? 2 : st - 1;
            const bool diag = e == n - 1 && last_diag;
            if (diag) {                            // a branch, not selects in every block
                asm volatile("");
                mask_causal(sa, 0);
            }
            // this block's stage bases, one register each: every read below
            // is a base plus an immediate (kept opaque so the compiler does
            // not rebuild each address from the loop counter)
            uint32_t kb0[4], kb1[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kb0[ks] = koff[ks] + (uint32_t)st * kKTile;
                kb1[ks] = koff[ks] + (uint32_t)st1 * kKTile;
            }
            uint32_t vb0 = voff + (uint32_t)st * kVTile;
            asm volatile("" : "+v"(kb0[0]), "+v"(kb0[1]), "+v"(kb0[2]), "+v"(kb0[3]), "+v"(kb1[0]),
                              "+v"(kb1[1]), "+v"(kb1[2]), "+v"(kb1[3]), "+v"(vb0));
            load_block(blk_at(e + 2 < n ? e + 2 : n - 1));
            half_scores_at(sb, kb0, 1);
            half_values(sa, vb0, 0, trk);
            half_step_order();
            if (diag) {
                asm volatile("");
                mask_causal(sb, 1);
            }
            half_scores_at(sa, kb1, 0);
            half_values(sb, vb0, 1, trk);
            half_step_order();
            store_block(st2);
            __syncthreads();                       // block e + 2 staged; stage e % 3 free
        }
        };
        if (track) blocks(std::true_type{});
        else blocks(std::false_type{});
        // end of pass. A pass whose row sums stay within 2^kRescaleSlack is
        // final. Otherwise a tracking pass follows (same references, running
        // maxima kept), after which every row's reference is raised to its
        // maximum and a last pass runs (probabilities <= 1 there).
        bool redo = false;
        if (track) {
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt) {
                float mx = mrun[rt];
                mx = fmaxf(mx, shfl_xor(mx, 16));
                mx = fmaxf(mx, shfl_xor(mx, 32));
                if (mx > 0.f) m[rt] += mx;
            }
            redo = true;
        } else {
#pragma unroll
            for (int rt = 0; rt < kAtRt; ++rt)
                if (!(osum[rt][0] <= kSumLimit)) redo = true;         // also catches inf / NaN
        }
        __syncthreads();
        if (redo) s_redo[pass] = 1;
        __syncthreads();
        if (s_redo[pass] == 0) break;
        track = !track;
    }

    // finish: normalise by the row sums and write
#pragma unroll
    for (int rt = 0; rt < kAtRt; ++rt) {
        const float l = osum[rt][0];
        const int64_t qi = q_first + qloc[rt];
        if (qi >= Tq) continue;
        const int h = c16 & 3;
        const int64_t orow = qi * Hq + (int64_t)kvh * kPfG + h;
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int ch = 16 * ct + 4 * g;
            const f32x4_t &v = o[ct][rt];
            if (out_bf16) {
                uint2 w = make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
                *reinterpret_cast<uint2 *>(reinterpret_cast<bf16_t *>(O) + orow * kD + ch) = w;
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(O) + orow * kD + ch) =
                    make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            }
        }
        if (lse && g == 0) lse[orow] = l > 0.f ? (m[rt] + log2f(l)) * kLn2F : -INFINITY;
    }
}

// ------------------------------------------------------------------ host side

int32_t prefill_tile_cap(int64_t q_start, int64_t Tq, const sa_select_params &p) {
    const int64_t nb = n_blocks(q_start + Tq);
    const int64_t u = 64 * (int64_t)p.top_k + p.n_init + p.n_local;
    return (int32_t)(nb < u ? nb : u);
}

struct PrefillWorkspace {
    size_t bscore_off, qlens_off, qidx_off, qcnt_off, total;
    int64_t nb_cap;
    int qcap;
};

static PrefillWorkspace prefill_layout(int Hkv, int64_t q_start, int64_t Tq, const sa_select_params &p) {
    PrefillWorkspace w{};
    w.nb_cap = n_blocks(q_start + Tq);
    w.qcap = p.top_k + p.n_init + p.n_local;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    w.bscore_off = take((size_t)Tq * Hkv * w.nb_cap * sizeof(float));
    w.qlens_off = take((size_t)Tq * sizeof(int32_t));
    w.qidx_off = take((size_t)Tq * Hkv * w.qcap * sizeof(int32_t));
    w.qcnt_off = take((size_t)Tq * Hkv * sizeof(int32_t));
    w.total = off;
    return w;
}

size_t prefill_workspace_bytes(int Hq, int Hkv, int64_t q_start, int64_t Tq, const sa_select_params &p) {
    (void)Hq;
    return prefill_layout(Hkv, q_start, Tq, p).total;
}

int launch_prefill(const void *Q, int64_t q_start, int64_t Tq, const void *K, const void *V,
                   const void *Kc, int Hq, int Hkv, int64_t T_cap, int64_t nc_cap,
                   const sa_select_params &p, float scale, void *O, int out_dtype, float *lse_out,
                   int32_t *tile_idx, int32_t tile_idx_cap, int32_t *tile_cnt, void *workspace,
                   hipStream_t stream) {
    const PrefillWorkspace w = prefill_layout(Hkv, q_start, Tq, p);
    char *ws = (char *)workspace;
    float *bscore = (float *)(ws + w.bscore_off);
    int32_t *qlens = (int32_t *)(ws + w.qlens_off);
    int32_t *qidx = (int32_t *)(ws + w.qidx_off);
    int32_t *qcnt = (int32_t *)(ws + w.qcnt_off);
    const int n_tiles = (int)((Tq + 63) / 64);
    const dim3 grid((unsigned)(n_tiles * Hkv));
    if (p.score_mode == SA_SCORE_RAW_SUM)
        hipLaunchKernelGGL(prefill_score_kernel<true>, grid, dim3(kAtThreads), 0, stream, (const bf16_t *)Q,
                           (const bf16_t *)Kc, Hq, Hkv, q_start, Tq, nc_cap, bscore, w.nb_cap, qlens);
    else
        hipLaunchKernelGGL(prefill_score_kernel<false>, grid, dim3(kAtThreads), 0, stream, (const bf16_t *)Q,
                           (const bf16_t *)Kc, Hq, Hkv, q_start, Tq, nc_cap, bscore, w.nb_cap, qlens);
    launch_topk_raw((int)(Tq * Hkv), Hkv, q_start + Tq, w.nb_cap, qlens, p, bscore, qidx, w.qcap,
                    qcnt, stream);
    hipLaunchKernelGGL(prefill_union_kernel, grid, dim3(kPfThreads), 0, stream, (const int32_t *)qidx,
                       (const int32_t *)qcnt, w.qcap, Hkv, q_start, Tq, tile_idx, tile_idx_cap, tile_cnt);
    return launch_prefill_attend(Q, q_start, Tq, K, V, Hq, Hkv, T_cap, tile_idx, tile_idx_cap,
                                 tile_cnt, scale, O, out_dtype, lse_out, stream);
}

int launch_prefill_attend(const void *Q, int64_t q_start, int64_t Tq, const void *K, const void *V,
                          int Hq, int Hkv, int64_t T_cap, const int32_t *tile_idx,
                          int32_t tile_idx_cap, const int32_t *tile_cnt, float scale, void *O,
                          int out_dtype, float *lse_out, hipStream_t stream) {
    const int n_tiles = (int)((Tq + 63) / 64);
    hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)(n_tiles * Hkv)), dim3(kAtThreads), 0,
                       stream, (const bf16_t *)Q, (const bf16_t *)K, (const bf16_t *)V, Hq, Hkv,
                       q_start, Tq, T_cap, tile_idx, tile_idx_cap, tile_cnt, scale * kLog2eF, O,
                       out_dtype == SA_BF16 ? 1 : 0, lse_out);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
