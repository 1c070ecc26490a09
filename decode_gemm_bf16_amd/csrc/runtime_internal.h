// Internal entry points of runtime.cpp shared with other sources of the library.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/uw.h"

namespace uw {

// The SwiGLU layer behind uw_mlp_forward, with fused_only restricting every
// projection to the fused direct-palette kernels (no allocation anywhere).
uw_status mlp_forward_impl(uw_handle gate, uw_handle up, uw_handle down, const int32_t* pipelines,
                           const uint16_t* x_dev, float* y_dev, int64_t tokens, void* work_dev, size_t work_bytes,
                           bool fused_only);

// Sets the thread-local error text read by uw_last_error and returns st.
uw_status set_error(uw_status st, const char* msg);

}  // namespace uw
