// Chunked prefill of the KDA mixer (under construction).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

size_t prefill_workspace_bytes(const kda_shape&, int32_t, int64_t) { return 0; }

int launch_prefill(const kda_shape&, const PrefillArgs&, hipStream_t) {
    return KDA_ERR_UNSUPPORTED;
}

}  // namespace kda
