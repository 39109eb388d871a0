// Launcher of the acceptance-label kernels (tv.hip) behind the C ABI
// (arguments already validated).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dspark {

size_t tv_workspace_bytes(int B, int gamma, int V);
hipError_t launch_tv_label(int B, int gamma, int V, int rank, int dtype, const void* target,
                           const void* U, const void* W1, const void* W2,
                           const int32_t* anchor, const int32_t* tokens, const float* row_max,
                           const float* row_logZ, const float* temperature, float* tv,
                           float* label, int32_t* status, void* ws, hipStream_t stream);

}  // namespace dspark
