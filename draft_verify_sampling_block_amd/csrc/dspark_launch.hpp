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
// 3 / 4 = persistent only with 8 / 4 waves per work-group, 5 = the pipelined
// kernel only
int set_draft_path(int path);   // returns the previous setting
int get_draft_path();
// The pipelined single-launch draft kernel (draft_pipe.hip): workspace
// bytes, and the launch on a device with P compute units;
// hipErrorNotSupported where it cannot run.  `hdr`: its start-barrier
// header (kDraftPipeHeaderBytes, at the same place for every call and
// zero-filled before the first; nothing else writes it); `ws`: its exchange
// words (any content).
constexpr size_t kDraftPipeHeaderBytes = 1536;
// The confidence head evaluated alongside the draft: hidden [B,gamma,H]
// (the draft's dtype), w [H+rank], bias, temps [gamma] or NULL, out conf
// [B,gamma].
struct ConfIn {
  const void* hidden;
  const float* w;
  float bias;
  const float* temps;
  float* conf;
  int H;
};
size_t draft_pipe_workspace_bytes(int B, int V);
hipError_t draft_pipe(int B, int gamma, int V, int rank, int P, long long spin_cap,
                      const uint16_t* U, const uint16_t* W1, const uint16_t* W2,
                      const int32_t* anchor, const float* temperature, const float* uniforms,
                      int32_t* tokens, float* q_tok, float* row_max, float* row_logZ,
                      int32_t* status, uint32_t* hdr, void* ws, const ConfIn* cf, bool coop,
                      hipStream_t stream);
// compute units of the current device (cached per device)
int device_cu_count();
hipError_t launch_draft_block(int B, int gamma, int V, int rank, int dtype, const void* U,
                              const void* W1, const void* W2, const int32_t* anchor,
                              const float* temperature, const float* uniforms, int32_t* tokens,
                              float* q_tok, float* row_max, float* row_logZ, int32_t* status,
                              void* ws, hipStream_t stream, const ConfIn* cf = nullptr);

// RNN head (rnn.hip, draft.hip): the recurrence's workspace (pre-activations
// of the hidden part for every position, two state buffers), its launches,
// and the whole block draft (the draft workspace plus the recurrence's)
size_t rnn_workspace_bytes(int B, int gamma, int rank);
hipError_t launch_rnn_hidden(int B, int gamma, int rank, int H, int dtype, const void* hidden,
                             const void* Wr, const float* br, void* ws, hipStream_t stream);
hipError_t launch_rnn_state(int k, int B, int gamma, int V, int rank, int H, int dtype,
                            const void* Wr, const void* W1, const int32_t* anchor,
                            const int32_t* tokens, void* emb, float* state_out, int32_t* status,
                            void* ws, hipStream_t stream);
size_t draft_rnn_workspace_bytes(int B, int gamma, int V, int rank, int H, int dtype);
hipError_t launch_draft_block_rnn(int B, int gamma, int V, int rank, int H, int dtype,
                                  const void* U, const void* W1, const void* W2,
                                  const void* hidden, const void* Wr, const float* br,
                                  const int32_t* anchor, const float* temperature,
                                  const float* uniforms, int32_t* tokens, float* q_tok,
                                  float* row_max, float* row_logZ, void* emb, float* state,
                                  int32_t* status, void* ws, hipStream_t stream);

hipError_t launch_confidence(int B, int gamma, int H, int V, int rank, int dtype,
                             const void* hidden, const void* W1, const int32_t* anchor,
                             const int32_t* tokens, const float* w, float bias,
                             const float* temps, float* conf, int32_t* status,
                             hipStream_t stream);   // temps [gamma] or NULL

constexpr int kScheduleMaxKeys = 8192;
constexpr int kScheduleMergeKeys = 4096;   // candidates ranked by run searches
size_t schedule_workspace_bytes(int R, int gamma);

size_t verify_workspace_bytes(int B, int gamma, int V, int rank, int dtype);
hipError_t launch_verify(int B, int gamma, int V, int rank, int dtype, const void* target,
                         const void* U, const void* W1, const void* W2, const int32_t* anchor,
                         const int32_t* tokens, const float* q_tok, const float* row_max,
                         const float* row_logZ, const float* temperature, const float* uniforms,
                         const int32_t* ell, int32_t* out_tokens, int32_t* n_accepted,
                         float* ratio, int32_t* status, void* ws, hipStream_t stream,
                         bool emb_rows = false);
// emb_rows: W1 is the RNN head's emb [B, gamma, rank], and the q recompute of
// request b at slot j takes its bias row b * gamma + j (not the W1 row of the
// previous token)

}  // namespace dspark
