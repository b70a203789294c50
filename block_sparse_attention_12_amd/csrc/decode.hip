// Gathered split-K sparse decode attention (Eq. 5 of the SparDA summary page,
// "Methodology": the attention query attends only to the keys and values of the
// selected blocks).
//
// Work unit: (sequence b, KV head kvh, split s). The unit's selected blocks
// idx[b, kvh, 0..cnt) are divided into n_split contiguous shares; each
// workgroup streams its share's K and V blocks (64 rows x 256 B each for bf16,
// contiguous in HBM) once and serves all G = 4 query heads of the group from
// that single read (GQA packing).
//
// Mapping of a 256-thread workgroup: wave w owns rows 16w .. 16w+15 of every
// block; inside a wave, row group r = lane / 16 takes rows 16w + 4i + r
// (i = 0..3) and each lane owns 8 channels. One block costs each lane 4 K and
// 4 V loads of 16 B, all issued before any arithmetic. Logits for 4 rows x 4
// heads are reduced across the 16 lanes of a row by the DPP transposed
// reduction, leaving one logit per lane; the online softmax keeps a running
// max per head (wave-uniform) and per-lane partial sums, so no workgroup
// barrier is needed inside the block loop. Probabilities reach the lanes that
// hold the matching V rows through a wave-private LDS slot. The four waves'
// states are merged once at the end through LDS.
//
// With n_split > 1 each workgroup writes (max, sum, weighted values) to the
// workspace and combine_kernel merges them with log-sum-exp weights; with
// n_split = 1 the workgroup writes O directly. Logits are kept in base-2 units
// (q is pre-multiplied by scale * log2 e) so every exponential is one exp2.
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kDecThreads = 256;
constexpr int kDecG = 4;
constexpr int kPartStride = kD + 4;          // acc[128], max, sum, 2 pad (16 B aligned rows)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

int decode_auto_split(int B, int Hkv, int32_t idx_cap) {
    const int units = B * Hkv;
    const int target = 2048;                              // workgroups in flight over 256 CUs
    int s = (target + units - 1) / units;
    int max_s = idx_cap / 2 > 1 ? idx_cap / 2 : 1;       // at least ~2 blocks per split
    if (s > max_s) s = max_s;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return s;
}

size_t decode_workspace_bytes(int B, int Hq, int32_t n_split) {
    if (n_split <= 1) return 0;
    return (size_t)B * Hq * n_split * kPartStride * sizeof(float);
}

template <int G>
__device__ __forceinline__ float pick(const float (&a)[G], int i) {
    float r = a[0];
#pragma unroll
    for (int g = 1; g < G; ++g) r = (i == g) ? a[g] : r;
    return r;
}

__device__ __forceinline__ void store_out(float *O, int64_t i, float x) { O[i] = x; }

template <typename T, bool DIRECT>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, int Hq, int Hkv,
    int64_t T_cap, const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int idx_cap, float qscale, int n_split,
    float *__restrict__ part, void *__restrict__ O, int out_bf16, float *__restrict__ lse) {
    constexpr int G = kDecG;
    __shared__ __align__(16) float s_p[4][64];
    __shared__ float s_m[4][G], s_l[4][G];
    __shared__ __align__(16) float s_acc[4][G][kD];

    const int split = blockIdx.x, unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lane16 = lane & 15, rgrp = lane >> 4;
    int64_t L = seq_lens[b];
    L = L < 0 ? 0 : (L > T_cap ? T_cap : L);
    int n = cnt[unit];
    n = n < 0 ? 0 : (n > idx_cap ? idx_cap : n);
    const int per = (n + n_split - 1) / n_split;
    const int e_lo = split * per;
    const int e_hi = e_lo + per < n ? e_lo + per : n;

    float q[G][8];
    {
        const T *qp = Q + ((int64_t)b * Hq + (int64_t)kvh * G) * kD + lane16 * kLaneElems;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            load8(qp + (int64_t)g * kD, q[g]);
#pragma unroll
            for (int c = 0; c < 8; ++c) q[g][c] *= qscale;
        }
    }
    float m_run[G], acc[G][8];
    float l_lane = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = -INFINITY;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
    }
    const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
    const T *Vu = V + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
    const int32_t *irow = idx + (int64_t)unit * idx_cap;
    const int my_head = lane16 & 3;
    const int my_row = 16 * wave + 4 * (lane16 >> 2) + rgrp;   // row of the logit this lane holds

#pragma unroll 1
    for (int e = e_lo; e < e_hi; ++e) {
        const int64_t t0 = (int64_t)irow[e] * kBlock;
        Raw8<T> kr[4], vr[4];
        bool ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + 16 * wave + 4 * i + rgrp;
            ok[i] = t >= 0 && t < L;
            if (ok[i]) {
                load_raw(Ku + t * kD, kr[i]);
                load_raw(Vu + t * kD, vr[i]);
            }
        }
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float k8[8];
            if (ok[i]) unpack(kr[i], k8);
            else {
#pragma unroll
                for (int c = 0; c < 8; ++c) k8[c] = 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float a = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) a = fmaf(q[g][c], k8[c], a);
                v[i * G + g] = a;
            }
        }
        transpose_reduce16<16>(v, lane);
        const int64_t my_t = t0 + my_row;
        const float x = (my_t >= 0 && my_t < L) ? v[0] : -INFINITY;
        // block max per head over the wave (lanes sharing lane & 3)
        float mx = fmaxf(x, dpp<kDppRowRor4>(x));
        mx = fmaxf(mx, dpp<kDppRowRor8>(mx));
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        float alpha[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mb = __shfl(mx, g, 64);
            const float mn = fmaxf(m_run[g], mb);
            alpha[g] = (m_run[g] == -INFINITY) ? 0.f : exp2f(m_run[g] - mn);
            m_run[g] = mn;
        }
        const float my_m = pick<G>(m_run, my_head);
        const float p = (x == -INFINITY) ? 0.f : exp2f(x - my_m);
        l_lane = l_lane * pick<G>(alpha, my_head) + p;
        s_p[wave][lane] = p;
        __builtin_amdgcn_wave_barrier();
        float pr[16];
        {
            const float4 *src = reinterpret_cast<const float4 *>(&s_p[wave][rgrp * 16]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 t = src[k];
                pr[4 * k] = t.x; pr[4 * k + 1] = t.y; pr[4 * k + 2] = t.z; pr[4 * k + 3] = t.w;
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[g][c] *= alpha[g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!ok[i]) continue;
            float v8[8];
            unpack(vr[i], v8);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pg = pr[i * G + g];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(pg, v8[c], acc[g][c]);
            }
        }
    }

    // ---- merge inside the wave: l over lanes of one head, acc over row groups
    float l = l_lane;
    l += dpp<kDppRowRor4>(l);
    l += dpp<kDppRowRor8>(l);
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float a = acc[g][c];
            a += shfl_xor(a, 16);
            a += shfl_xor(a, 32);
            acc[g][c] = a;
        }
    if (rgrp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float4 *dst = reinterpret_cast<float4 *>(&s_acc[wave][g][lane16 * 8]);
            dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
    }
    if (lane < G) {
        s_m[wave][lane] = pick<G>(m_run, lane);
        s_l[wave][lane] = l;                    // lane g < 4 holds head g's sum
    }
    __syncthreads();

    // ---- merge the four waves: thread -> (head g, channels 2c, 2c+1)
    const int g = tid >> 6;
    const int c2 = (tid & 63) * 2;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
    float lsum = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float mw = s_m[w][g];
        const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        lsum = fmaf(wt, s_l[w][g], lsum);
        a0 = fmaf(wt, s_acc[w][g][c2], a0);
        a1 = fmaf(wt, s_acc[w][g][c2 + 1], a1);
    }
    const int64_t row = (int64_t)b * Hq + (int64_t)kvh * G + g;   // query head row
    if constexpr (DIRECT) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if (out_bf16) {
            uint32_t w = f32_to_bf16_bits(a0 * inv) | (f32_to_bf16_bits(a1 * inv) << 16);
            reinterpret_cast<uint32_t *>(O)[(row * kD + c2) / 2] = w;
        } else {
            reinterpret_cast<float2 *>(O)[(row * kD + c2) / 2] = make_float2(a0 * inv, a1 * inv);
        }
        if (lse && (tid & 63) == 0) lse[row] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
    } else {
        float *dst = part + (row * n_split + split) * kPartStride;
        reinterpret_cast<float2 *>(dst)[c2 / 2] = make_float2(a0, a1);
        if ((tid & 63) == 0) {
            dst[kD] = M;
            dst[kD + 1] = lsum;
        }
    }
}

__global__ __launch_bounds__(kD) void combine_kernel(const float *__restrict__ part, int n_split,
                                                     void *__restrict__ O, int out_bf16,
                                                     float *__restrict__ lse) {
    const int64_t row = blockIdx.x;
    const int c = threadIdx.x;
    const float *p = part + row * n_split * kPartStride;
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, p[s * kPartStride + kD]);
    float lsum = 0.f, a = 0.f;
    for (int s = 0; s < n_split; ++s) {
        const float ms = p[s * kPartStride + kD];
        const float wt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
        lsum = fmaf(wt, p[s * kPartStride + kD + 1], lsum);
        a = fmaf(wt, p[s * kPartStride + c], a);
    }
    const float o = lsum > 0.f ? a / lsum : 0.f;
    if (out_bf16) reinterpret_cast<bf16_t *>(O)[row * kD + c] = (bf16_t)f32_to_bf16_bits(o);
    else reinterpret_cast<float *>(O)[row * kD + c] = o;
    if (lse && c == 0) lse[row] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
}

template <typename T>
static void launch_decode_t(const void *Q, const void *K, const void *V, int B, int Hq, int Hkv,
                            int64_t T_cap, const int32_t *seq_lens, const int32_t *idx,
                            const int32_t *cnt, int32_t idx_cap, float scale, void *O,
                            int out_bf16, float *lse, int32_t n_split, void *ws,
                            hipStream_t stream) {
    const dim3 grid((unsigned)n_split, (unsigned)(B * Hkv));
    const float qscale = scale * kLog2e;
    if (n_split == 1) {
        hipLaunchKernelGGL((decode_kernel<T, true>), grid, dim3(kDecThreads), 0, stream,
                           (const T *)Q, (const T *)K, (const T *)V, Hq, Hkv, T_cap, seq_lens, idx,
                           cnt, idx_cap, qscale, 1, (float *)nullptr, O, out_bf16, lse);
    } else {
        hipLaunchKernelGGL((decode_kernel<T, false>), grid, dim3(kDecThreads), 0, stream,
                           (const T *)Q, (const T *)K, (const T *)V, Hq, Hkv, T_cap, seq_lens, idx,
                           cnt, idx_cap, qscale, n_split, (float *)ws, (void *)nullptr, 0,
                           (float *)nullptr);
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(B * Hq)), dim3(kD), 0, stream,
                           (const float *)ws, n_split, O, out_bf16, lse);
    }
}

int launch_decode(const void *Q, const void *K, const void *V, int dtype, int B, int Hq, int Hkv,
                  int64_t T_cap, const int32_t *seq_lens, const int32_t *idx, const int32_t *cnt,
                  int32_t idx_cap, float scale, void *O, int out_dtype, float *lse_out,
                  int32_t n_split, void *workspace, hipStream_t stream) {
    const int out_bf16 = out_dtype == SA_BF16 ? 1 : 0;
    if (dtype == SA_BF16)
        launch_decode_t<bf16_t>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap, scale, O,
                                out_bf16, lse_out, n_split, workspace, stream);
    else
        launch_decode_t<float>(Q, K, V, B, Hq, Hkv, T_cap, seq_lens, idx, cnt, idx_cap, scale, O,
                               out_bf16, lse_out, n_split, workspace, stream);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
