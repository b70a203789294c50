// Selection quality: exact per-block attention mass of the decode query and the
// recall of a selected block set.
//
// Page "CoSA: Accelerating Long-Context Inference via Proxy-Kernel Co-Designed
// Sparse Attention" (abstract): a block's attention mass is the sum of its
// attention probabilities; selecting the blocks of largest mass recovers dense
// attention. The recall of a set is the mass it captures (one minus the rest
// bucket of Eq. 7 on the SparDA page).
//
// This reads every key (it is the dense reference the selection approximates),
// so it is a measurement, not a step of the sparse path.
//
//   block_lse_kernel   grid (chunks of 16 blocks, units (b, kvh)): for each of
//                      the chunk's blocks and each of the G = 4 heads, the block
//                      max m and sum z of 2^(s - m) over its visible tokens
//                      (s = scale * log2(e) * q . k); wave w takes blocks
//                      w, w+4, ...; a row of K is read by 16 lanes as in the
//                      decode kernel, 4 rows per load instruction.
//   block_mass_kernel  one workgroup per (b, head): M = max m, Z = sum z 2^(m-M),
//                      mass = z 2^(m-M) / Z; recall = sum of the masses of the
//                      head's KV-head set.
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kBmThreads = 256;
constexpr int kBmChunk = 16;         // blocks per workgroup of the first kernel
constexpr int kBmG = 4;

template <typename T> struct QRow;
template <> struct QRow<bf16_t> { uint32_t w[kBmG][4]; };
template <> struct QRow<float> { float w[kBmG][8]; };

__device__ __forceinline__ void load_qrow(const bf16_t *p, QRow<bf16_t> &q) {
#pragma unroll
    for (int g = 0; g < kBmG; ++g) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p + (int64_t)g * kD);
        q.w[g][0] = v.x; q.w[g][1] = v.y; q.w[g][2] = v.z; q.w[g][3] = v.w;
    }
}
__device__ __forceinline__ void load_qrow(const float *p, QRow<float> &q) {
#pragma unroll
    for (int g = 0; g < kBmG; ++g) load8(p + (int64_t)g * kD, q.w[g]);
}
__device__ __forceinline__ float dotq(const QRow<bf16_t> &q, int g, const Raw8<bf16_t> &k) {
    float a = dot2_bf16(q.w[g][0], k.v.x, 0.f);
    a = dot2_bf16(q.w[g][1], k.v.y, a);
    a = dot2_bf16(q.w[g][2], k.v.z, a);
    return dot2_bf16(q.w[g][3], k.v.w, a);
}
__device__ __forceinline__ float dotq(const QRow<float> &q, int g, const Raw8<float> &k) {
    float x[8];
    unpack(k, x);
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a = fmaf(q.w[g][c], x[c], a);
    return a;
}

// (m, z) pairs in log2 units: merge b into a
__device__ __forceinline__ void merge_mz(float &m, float &z, float m2, float z2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    z = (m == -INFINITY ? 0.f : z * exp2f(m - mn)) + (m2 == -INFINITY ? 0.f : z2 * exp2f(m2 - mn));
    m = mn;
}

template <typename T>
__global__ __launch_bounds__(kBmThreads) void block_lse_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, int Hq, int Hkv, int64_t T_cap,
    const int32_t *__restrict__ seq_lens, float qscale, int64_t nb_cap, float *__restrict__ bm,
    float *__restrict__ bz) {
    const int unit = blockIdx.y;
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane >> 4, lane16 = lane & 15;
    int64_t L = seq_lens[b];
    L = L < 0 ? 0 : (L > T_cap ? T_cap : L);
    const int nb = (int)n_blocks(L);
    const int blk_lo = blockIdx.x * kBmChunk;
    const int blk_hi = blk_lo + kBmChunk < nb ? blk_lo + kBmChunk : nb;
    if (blk_lo >= blk_hi) return;
    QRow<T> q;
    load_qrow(Q + ((int64_t)b * Hq + (int64_t)kvh * kBmG) * kD + lane16 * kLaneElems, q);
    constexpr uint32_t kRowBytes = kD * sizeof(T);
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + (int64_t)unit * T_cap * kD, (uint32_t)(L * kRowBytes));
    const uint32_t lane_off = lane16 * kLaneElems * sizeof(T);
    for (int blk = blk_lo + wave; blk < blk_hi; blk += kBmThreads / 64) {
        float m[kBmG], z[kBmG];
#pragma unroll
        for (int g = 0; g < kBmG; ++g) { m[g] = -INFINITY; z[g] = 0.f; }
#pragma unroll 4
        for (int it = 0; it < kBlock / 4; ++it) {
            const int64_t t = (int64_t)blk * kBlock + 4 * it + rg;      // this row group's token
            Raw8<T> k;
            load_raw_nt(rK, row_offset(t, kRowBytes, lane_off), k);
            float s[kBmG];
#pragma unroll
            for (int g = 0; g < kBmG; ++g) {
                float v = dotq(q, g, k);
#pragma unroll
                for (int off = 8; off >= 1; off >>= 1) v += shfl_xor(v, off);   // over the 16 lanes
                s[g] = t < L ? v * qscale : -INFINITY;
            }
#pragma unroll
            for (int g = 0; g < kBmG; ++g) merge_mz(m[g], z[g], s[g], 1.f);
        }
        // the 4 row groups of the wave
#pragma unroll
        for (int g = 0; g < kBmG; ++g) {
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float m2 = shfl_xor(m[g], off), z2 = shfl_xor(z[g], off);
                merge_mz(m[g], z[g], m2, z2);
            }
        }
        if (lane < kBmG) {
            float mm = m[0], zz = z[0];
#pragma unroll
            for (int g = 1; g < kBmG; ++g)
                if (lane == g) { mm = m[g]; zz = z[g]; }
            const int64_t o = ((int64_t)b * Hq + (int64_t)kvh * kBmG + lane) * nb_cap + blk;
            bm[o] = mm;
            bz[o] = zz;
        }
    }
}

__global__ __launch_bounds__(kBmThreads) void block_mass_kernel(
    int Hq, int Hkv, int64_t T_cap, const int32_t *__restrict__ seq_lens, int64_t nb_cap,
    const float *__restrict__ bm, const float *__restrict__ bz, float *__restrict__ mass,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, int idx_cap,
    float *__restrict__ recall) {
    __shared__ float s_m[kBmThreads / 64], s_z[kBmThreads / 64];
    const int bh = blockIdx.x;                     // b * Hq + h
    const int b = bh / Hq, h = bh % Hq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t L = seq_lens[b];
    L = L < 0 ? 0 : (L > T_cap ? T_cap : L);
    const int nb = (int)n_blocks(L);
    const float *m_row = bm + (int64_t)bh * nb_cap;
    const float *z_row = bz + (int64_t)bh * nb_cap;
    float M = -INFINITY, Z = 0.f;
    for (int i = tid; i < nb; i += kBmThreads) merge_mz(M, Z, m_row[i], z_row[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = shfl_xor(M, off), z2 = shfl_xor(Z, off);
        merge_mz(M, Z, m2, z2);
    }
    if (lane == 0) { s_m[wave] = M; s_z[wave] = Z; }
    __syncthreads();
    M = s_m[0];
    Z = s_z[0];
#pragma unroll
    for (int w = 1; w < kBmThreads / 64; ++w) merge_mz(M, Z, s_m[w], s_z[w]);
    const float inv = Z > 0.f ? 1.f / Z : 0.f;
    float *out = mass + (int64_t)bh * nb_cap;
    for (int64_t i = tid; i < nb_cap; i += kBmThreads)
        out[i] = (i < nb && m_row[i] != -INFINITY) ? z_row[i] * exp2f(m_row[i] - M) * inv : 0.f;
    if (idx) {
        const int unit = b * Hkv + h / (Hq / Hkv);
        int n = cnt[unit];
        n = n < 0 ? 0 : (n > idx_cap ? idx_cap : n);
        float r = 0.f;
        for (int i = tid; i < n; i += kBmThreads) {
            const int blk = idx[(int64_t)unit * idx_cap + i];
            if (blk >= 0 && blk < nb && m_row[blk] != -INFINITY) r += z_row[blk] * exp2f(m_row[blk] - M) * inv;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) r += shfl_xor(r, off);
        __syncthreads();
        if (lane == 0) s_z[wave] = r;
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < kBmThreads / 64; ++w) t += s_z[w];
            recall[bh] = t;
        }
    }
}

size_t block_mass_workspace_bytes(int B, int Hq, int64_t nb_cap) {
    return 2 * (size_t)B * Hq * nb_cap * sizeof(float);
}

int launch_block_mass(const void *Q, const void *K, int dtype, int B, int Hq, int Hkv, int64_t T_cap,
                      const int32_t *seq_lens, float scale, float *mass, int64_t nb_cap,
                      const int32_t *idx, const int32_t *cnt, int idx_cap, float *recall,
                      void *workspace, hipStream_t stream) {
    float *bm = (float *)workspace;
    float *bz = bm + (size_t)B * Hq * nb_cap;
    const float qscale = scale * 1.44269504088896340736f;
    const int64_t nb_max = n_blocks(T_cap);
    const dim3 grid((unsigned)((nb_max + kBmChunk - 1) / kBmChunk), (unsigned)(B * Hkv));
    // every block below a sequence's block count is written by the first kernel
    // and only those are read by the second
    if (dtype == SA_BF16)
        hipLaunchKernelGGL(block_lse_kernel<bf16_t>, grid, dim3(kBmThreads), 0, stream,
                           (const bf16_t *)Q, (const bf16_t *)K, Hq, Hkv, T_cap, seq_lens, qscale,
                           nb_cap, bm, bz);
    else
        hipLaunchKernelGGL(block_lse_kernel<float>, grid, dim3(kBmThreads), 0, stream,
                           (const float *)Q, (const float *)K, Hq, Hkv, T_cap, seq_lens, qscale,
                           nb_cap, bm, bz);
    hipLaunchKernelGGL(block_mass_kernel, dim3((unsigned)(B * Hq)), dim3(kBmThreads), 0, stream, Hq,
                       Hkv, T_cap, seq_lens, nb_cap, (const float *)bm, (const float *)bz, mass, idx,
                       cnt, idx_cap, recall);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
