// Internal host-side launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

constexpr int kMaxVocab = 262144;   // largest vocabulary the kernels take

size_t draft_workspace_bytes(int B, int gamma, int V, int rank, int dtype);
// 0 = automatic (persistent kernel when possible), 1 = multi-launch only,
// 2 = persistent only (fails with hipErrorNotSupported where it cannot run),
// 3 / 4 = persistent only with 8 / 4 waves per work-group
int set_draft_path(int path);   // returns the previous setting
int get_draft_path();
// compute units of the current device (cached per device)
int device_cu_count();
hipError_t launch_draft_block(int B, int gamma, int V, int rank, int dtype, const void* U,
                              const void* W1, const void* W2, const int32_t* anchor,
                              const float* temperature, const float* uniforms, int32_t* tokens,
                              float* q_tok, float* row_max, float* row_logZ, int32_t* status,
                              void* ws, hipStream_t stream);

hipError_t launch_confidence(int B, int gamma, int H, int V, int rank, int dtype,
                             const void* hidden, const void* W1, const int32_t* anchor,
                             const int32_t* tokens, const float* w, float bias, float* conf,
                             int32_t* status, hipStream_t stream);

constexpr int kScheduleMaxKeys = 8192;
constexpr int kScheduleMergeKeys = 4096;   // candidates ranked by run searches
size_t schedule_workspace_bytes(int R, int gamma);

size_t verify_workspace_bytes(int B, int gamma, int V, int rank, int dtype);
hipError_t launch_verify(int B, int gamma, int V, int rank, int dtype, const void* target,
                         const void* U, const void* W1, const void* W2, const int32_t* anchor,
                         const int32_t* tokens, const float* q_tok, const float* row_max,
                         const float* row_logZ, const float* temperature, const float* uniforms,
                         const int32_t* ell, int32_t* out_tokens, int32_t* n_accepted,
                         float* ratio, int32_t* status, void* ws, hipStream_t stream);

}  // namespace dspark
