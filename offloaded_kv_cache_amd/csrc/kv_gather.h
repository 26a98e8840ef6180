// kv_gather.h - launcher of the multi-layer page-in copy with HIP events recorded at the
// kernel's own start and end (either may be NULL).
#pragma once

#include "kv_internal.h"

namespace kvc {

hipError_t launch_gather_multi_timed(const MultiGatherBatch& batch, int64_t page_bytes, hipStream_t stream,
                                     hipEvent_t start, hipEvent_t stop);

}  // namespace kvc
