// sparse_attn_decode_step_noalloc: the one-call decode step with its scratch
// memory in a fixed device array of the library instead of a caller
// workspace, for callers that cannot allocate (code under graph capture,
// serving loops, harnesses that forbid allocation). It allocates nothing.
//
// The array `scratch` is a file-scope device array, one copy per GPU the
// library runs on, held until the process ends. Its name is a host-side
// stand-in in host code, so host code never uses it directly: the first call
// on a device (with that device current) asks the runtime for the device
// address of that GPU's copy (hipGetSymbolAddress) and keeps it per device;
// kernels receive that address as their workspace argument, exactly as they
// receive a caller workspace in sparse_attn_decode_step.
//
// Every call on a GPU shares its copy: calls that overlap on one GPU (other
// streams, other host threads) race. The step's kernels write every scratch
// word they read within the same call (block scores, logits, split partials),
// so nothing has to start at zero.
#include <atomic>

#include "sa_device.h"
#include "sa_internal.h"

using namespace sa;

namespace {

constexpr size_t kScratchBytes = SA_NOALLOC_SCRATCH_BYTES;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch` (looked up once
// per device; concurrent first calls look up the same address).
int scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SA_ERR_HIP;
    if (dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SA_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SA_OK;
}

}  // namespace

extern "C" {

int sparse_attn_decode_step_noalloc(const void *Q, const void *sel, int H_sel, const void *K,
                                    const void *V, void *Kc, int dtype, int B, int Hq, int Hkv,
                                    int d, int64_t T_cap, int64_t nc_cap,
                                    const int32_t *lens_prev, const int32_t *lens_now,
                                    int32_t max_new_tokens, const sa_select_params *p,
                                    float scale, int32_t *idx_out, int32_t idx_cap,
                                    int32_t *cnt_out, void *O, int out_dtype, float *lse_out,
                                    int32_t n_split, void *stream) {
    if (!p) return SA_ERR_INVALID_ARG;
    const size_t need =
        sparse_attn_decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap, p, idx_cap, n_split);
    if (need > kScratchBytes) return SA_ERR_WORKSPACE;
    void *ws = nullptr;
    const int st = scratch_for_current_device(&ws);
    if (st) return st;
    return sparse_attn_decode_step(Q, sel, H_sel, K, V, Kc, dtype, B, Hq, Hkv, d, T_cap, nc_cap,
                                   lens_prev, lens_now, max_new_tokens, p, scale, idx_out, idx_cap,
                                   cnt_out, O, out_dtype, lse_out, n_split, ws, kScratchBytes,
                                   stream);
}

}  // extern "C"
