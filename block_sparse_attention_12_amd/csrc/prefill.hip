// Chunked sparse prefill (placeholder until the matrix-core kernels land).
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

int32_t prefill_tile_cap(int64_t q_start, int64_t Tq, const sa_select_params &p) {
    const int64_t nb = n_blocks(q_start + Tq);
    const int64_t u = 64 * (int64_t)p.top_k + p.n_init + p.n_local;
    return (int32_t)(nb < u ? nb : u);
}

size_t prefill_workspace_bytes(int, int, int64_t, int64_t, const sa_select_params &) { return 0; }

int launch_prefill(const void *, int64_t, int64_t, const void *, const void *, const void *, int,
                   int, int64_t, int64_t, const sa_select_params &, float, void *, int, float *,
                   int32_t *, int32_t, int32_t *, void *, hipStream_t) {
    return SA_ERR_UNSUPPORTED;
}

}  // namespace sa
