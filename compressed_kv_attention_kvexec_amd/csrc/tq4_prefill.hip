// tq4_prefill.hip -- chunked-prefill attention over TQ4 pages (gfx950).
#include "tq4_device.h"
#include "tq4_launch.h"

namespace tq4 {

PrefillPlan plan_prefill(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads, int32_t n_kv_heads) {
    PrefillPlan pl{};
    pl.group = n_q_heads / n_kv_heads;
    pl.workspace_bytes = 256;
    (void)prior_len;
    (void)chunk_len;
    return pl;
}

hipError_t launch_prefill(const PrefillParams &, const PrefillPlan &, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace tq4
