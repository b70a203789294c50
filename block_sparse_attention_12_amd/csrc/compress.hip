// Compressed-key build and append (Eq. 2 of the SparDA summary page,
// "Theoretical Foundation": mean pooling with kernel 32, stride 16).
//
// Entry j = (P_j + P_{j+1}) * 2^-5, rounded to the key dtype, where P_m is the
// fp32 sum of keys 16m .. 16m+15 accumulated in token order. The file is built
// with -ffp-contract=off so the adds are never fused or reassociated: every
// entry is one exact value, reproducible by a CPU implementation.
//
// Layout: one workgroup row of 16 lanes per run of R consecutive entries; each
// lane owns 8 channels. A lane streams the 16 keys of a half-window with 16
// independent 16 B (bf16) loads, so the wave keeps 4 rows x 16 tokens in
// flight. Consecutive entries share a half-window, which is carried in
// registers. HBM bound: every key is read once (the half-window at a run
// boundary is read twice, usually from L2).
#include "compress_device.h"
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kCompressThreads = 256;
constexpr int kCompressRun = 4;                              // entries per row group
constexpr int kCompressEntriesPerWG = (kCompressThreads / kRowLanes) * kCompressRun;

template <typename T>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(
    const T *__restrict__ K, T *__restrict__ Kc, int Hkv, int64_t T_cap, int64_t nc_cap,
    const int32_t *__restrict__ lens_prev, const int32_t *__restrict__ lens_now) {
    const int unit = blockIdx.x;                 // b * Hkv + kvh
    const int b = unit / Hkv;
    int64_t Lp = lens_prev[b], Ln = lens_now[b];
    Ln = Ln < 0 ? 0 : (Ln > T_cap ? T_cap : Ln);
    Lp = Lp < 0 ? 0 : (Lp > Ln ? Ln : Lp);
    const int64_t j_begin = n_compressed(Lp);
    const int64_t j_end = n_compressed(Ln);
    const int group = threadIdx.x / kRowLanes;
    const int lane16 = threadIdx.x % kRowLanes;
    const T *Ku = K + (int64_t)unit * T_cap * kD + lane16 * kLaneElems;
    T *Kcu = Kc + (int64_t)unit * nc_cap * kD + lane16 * kLaneElems;
    const int64_t step = (int64_t)gridDim.y * kCompressEntriesPerWG;
    for (int64_t j0 = j_begin + ((int64_t)blockIdx.y * (kCompressThreads / kRowLanes) + group) *
                                    kCompressRun;
         j0 < j_end; j0 += step) {
        compress_run<T, kCompressRun>(Ku, Kcu, j0, j_end);
    }
}

int launch_compress(const void *K, void *Kc, int dtype, int B, int Hkv, int64_t T_cap,
                    int64_t nc_cap, const int32_t *lens_prev, const int32_t *lens_now,
                    int32_t max_new_entries, hipStream_t stream) {
    int64_t wgs = (max_new_entries + kCompressEntriesPerWG - 1) / kCompressEntriesPerWG;
    if (wgs < 1) wgs = 1;
    if (wgs > 65535) wgs = 65535;
    dim3 grid((unsigned)(B * Hkv), (unsigned)wgs);
    if (dtype == SA_BF16)
        hipLaunchKernelGGL(compress_kernel<bf16_t>, grid, dim3(kCompressThreads), 0, stream,
                           (const bf16_t *)K, (bf16_t *)Kc, Hkv, T_cap, nc_cap, lens_prev, lens_now);
    else
        hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kCompressThreads), 0, stream,
                           (const float *)K, (float *)Kc, Hkv, T_cap, nc_cap, lens_prev, lens_now);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
