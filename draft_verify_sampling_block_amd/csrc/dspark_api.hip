// C ABI of libdspark: host-side validation, then the kernel launchers.
// Every check runs before anything is enqueued; a failed check returns a
// negative status, enqueues nothing and records a message for
// dspark_last_error().
#include <stdarg.h>
#include <stdio.h>

#include "../../include/dspark.h"
#include "dspark_launch.hpp"
#include "schedule_launch.hpp"
#include "tv_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                      \
  do {                                                                      \
    if (!(p)) return fail(DSPARK_EINVAL, "%s: '%s' is NULL", fn, #p);       \
    if (!aligned16(p)) return fail(DSPARK_EALIGN, "%s: '%s' is not 16-byte aligned", fn, #p); \
  } while (0)

#define OPT_PTR(p)                                                          \
  do {                                                                      \
    if ((p) && !aligned16(p))                                               \
      return fail(DSPARK_EALIGN, "%s: '%s' is not 16-byte aligned", fn, #p); \
  } while (0)

int check_dims(const char* fn, int B, int gamma, int V, int rank, int dtype) {
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16)
    return fail(DSPARK_EDTYPE, "%s: dtype %d is neither DSPARK_F32 nor DSPARK_BF16", fn, dtype);
  if (B < 1) return fail(DSPARK_EINVAL, "%s: B=%d must be >= 1", fn, B);
  if (gamma < 1 || gamma > 64) return fail(DSPARK_EINVAL, "%s: gamma=%d outside [1,64]", fn, gamma);
  if (V < 8 || V % 8) return fail(DSPARK_EINVAL, "%s: V=%d must be a positive multiple of 8", fn, V);
  if (V > dspark::kMaxVocab)
    return fail(DSPARK_EUNSUPPORTED, "%s: V=%d exceeds %d", fn, V, dspark::kMaxVocab);
  if (dtype == DSPARK_BF16 && rank != 32 && rank != 64 && rank != 128 && rank != 256)
    return fail(DSPARK_EINVAL, "%s: bf16 rank=%d must be 32, 64, 128 or 256", fn, rank);
  if (rank < 32 || rank > 512 || rank % 32)
    return fail(DSPARK_EINVAL, "%s: rank=%d must be a multiple of 32 in [32,512]", fn, rank);
  if ((long long)B * (gamma + 1) > (1LL << 31) / 2)
    return fail(DSPARK_EUNSUPPORTED, "%s: B*(gamma+1) too large", fn);
  return DSPARK_OK;
}

int hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(DSPARK_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return DSPARK_OK;
}

}  // namespace

extern "C" {

const char* dspark_status_str(int status) {
  switch (status) {
    case DSPARK_OK: return "DSPARK_OK";
    case DSPARK_EINVAL: return "DSPARK_EINVAL: invalid argument";
    case DSPARK_EDTYPE: return "DSPARK_EDTYPE: unknown dtype";
    case DSPARK_EALIGN: return "DSPARK_EALIGN: pointer not 16-byte aligned";
    case DSPARK_EWORKSPACE: return "DSPARK_EWORKSPACE: workspace missing or too small";
    case DSPARK_EUNSUPPORTED: return "DSPARK_EUNSUPPORTED: outside supported sizes";
    case DSPARK_EHIP: return "DSPARK_EHIP: HIP runtime error";
    default: return "unknown dspark status";
  }
}

const char* dspark_last_error(void) { return g_err; }

const char* dspark_version(void) { return "libdspark 0.1 gfx950"; }

int dspark_set_draft_path(int path) {
  if (path < 0 || path > 6)
    return fail(DSPARK_EINVAL, "dspark_set_draft_path: path %d is not in 0..6", path);
  const int old = dspark::set_draft_path(path);
  return old;
}

size_t dspark_draft_block_workspace(int B, int gamma, int V, int rank, int dtype) {
  if (check_dims("dspark_draft_block_workspace", B, gamma, V, rank, dtype) != DSPARK_OK) return 0;
  return dspark::draft_workspace_bytes(B, gamma, V, rank, dtype);
}

int dspark_draft_block(int B, int gamma, int V, int rank, int dtype, const void* U, const void* W1,
                       const void* W2, const int32_t* anchor, const float* temperature,
                       const float* uniforms, int32_t* tokens, float* q_tok, float* row_max,
                       float* row_logZ, int32_t* status, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  const char* fn = "dspark_draft_block";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  REQUIRE_PTR(U); REQUIRE_PTR(W1); REQUIRE_PTR(W2); REQUIRE_PTR(anchor);
  REQUIRE_PTR(temperature); REQUIRE_PTR(uniforms); REQUIRE_PTR(tokens); REQUIRE_PTR(q_tok);
  REQUIRE_PTR(row_max); REQUIRE_PTR(row_logZ); OPT_PTR(status);
  if (!status && dspark::get_draft_path() >= 2)
    return fail(DSPARK_EINVAL, "%s: the persistent-only draft paths need a status word (a "
                "timed-out wait is reported there only)", fn);
  const size_t need = dspark::draft_workspace_bytes(B, gamma, V, rank, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  return hip_status(fn, dspark::launch_draft_block(B, gamma, V, rank, dtype, U, W1, W2, anchor,
                                                   temperature, uniforms, tokens, q_tok, row_max,
                                                   row_logZ, status, workspace, stream));
}

int dspark_draft_block_conf(int B, int gamma, int V, int rank, int H, int dtype, const void* U,
                            const void* W1, const void* W2, const int32_t* anchor,
                            const float* temperature, const float* uniforms, const void* hidden,
                            const float* w, float bias, const float* temps, int32_t* tokens,
                            float* q_tok, float* row_max, float* row_logZ, float* conf,
                            int32_t* status, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const char* fn = "dspark_draft_block_conf";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  if (H < 8 || H % 8) return fail(DSPARK_EINVAL, "%s: H=%d must be a positive multiple of 8", fn, H);
  REQUIRE_PTR(U); REQUIRE_PTR(W1); REQUIRE_PTR(W2); REQUIRE_PTR(anchor);
  REQUIRE_PTR(temperature); REQUIRE_PTR(uniforms); REQUIRE_PTR(hidden); REQUIRE_PTR(w);
  REQUIRE_PTR(tokens); REQUIRE_PTR(q_tok); REQUIRE_PTR(row_max); REQUIRE_PTR(row_logZ);
  REQUIRE_PTR(conf); OPT_PTR(temps); OPT_PTR(status);
  if (!status && dspark::get_draft_path() >= 2)
    return fail(DSPARK_EINVAL, "%s: the persistent-only draft paths need a status word (a "
                "timed-out wait is reported there only)", fn);
  const size_t need = dspark::draft_workspace_bytes(B, gamma, V, rank, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  const dspark::ConfIn cf{hidden, w, bias, temps, conf, H};
  return hip_status(fn, dspark::launch_draft_block(B, gamma, V, rank, dtype, U, W1, W2, anchor,
                                                   temperature, uniforms, tokens, q_tok, row_max,
                                                   row_logZ, status, workspace, stream, &cf));
}

size_t dspark_draft_block_rnn_workspace(int B, int gamma, int V, int rank, int H, int dtype) {
  if (check_dims("dspark_draft_block_rnn_workspace", B, gamma, V, rank, dtype) != DSPARK_OK)
    return 0;
  if (H < 8 || H % 8) return 0;
  return dspark::draft_rnn_workspace_bytes(B, gamma, V, rank, H, dtype);
}

int dspark_draft_block_rnn(int B, int gamma, int V, int rank, int H, int dtype, const void* U,
                           const void* W1, const void* W2, const void* hidden, const void* Wr,
                           const float* br, const int32_t* anchor, const float* temperature,
                           const float* uniforms, int32_t* tokens, float* q_tok,
                           float* row_max, float* row_logZ, void* emb, float* state,
                           int32_t* status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const char* fn = "dspark_draft_block_rnn";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  if (H < 8 || H % 8) return fail(DSPARK_EINVAL, "%s: H=%d must be a positive multiple of 8", fn, H);
  REQUIRE_PTR(U); REQUIRE_PTR(W1); REQUIRE_PTR(W2); REQUIRE_PTR(hidden); REQUIRE_PTR(Wr);
  REQUIRE_PTR(br); REQUIRE_PTR(anchor); REQUIRE_PTR(temperature); REQUIRE_PTR(uniforms);
  REQUIRE_PTR(tokens); REQUIRE_PTR(q_tok); REQUIRE_PTR(row_max); REQUIRE_PTR(row_logZ);
  REQUIRE_PTR(emb); OPT_PTR(state); OPT_PTR(status);
  const size_t need = dspark::draft_rnn_workspace_bytes(B, gamma, V, rank, H, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  return hip_status(fn, dspark::launch_draft_block_rnn(B, gamma, V, rank, H, dtype, U, W1, W2,
                                                       hidden, Wr, br, anchor, temperature,
                                                       uniforms, tokens, q_tok, row_max,
                                                       row_logZ, emb, state, status, workspace,
                                                       stream));
}

int dspark_confidence(int B, int gamma, int H, int V, int rank, int dtype, const void* hidden,
                      const void* W1, const int32_t* anchor, const int32_t* tokens,
                      const float* w, float bias, float* conf, int32_t* status,
                      hipStream_t stream) {
  const char* fn = "dspark_confidence";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  if (H < 8 || H % 8) return fail(DSPARK_EINVAL, "%s: H=%d must be a positive multiple of 8", fn, H);
  REQUIRE_PTR(hidden); REQUIRE_PTR(W1); REQUIRE_PTR(anchor); REQUIRE_PTR(tokens);
  REQUIRE_PTR(w); REQUIRE_PTR(conf); OPT_PTR(status);
  return hip_status(fn, dspark::launch_confidence(B, gamma, H, V, rank, dtype, hidden, W1, anchor,
                                                  tokens, w, bias, nullptr, conf, status, stream));
}

int dspark_confidence_sts(int B, int gamma, int H, int V, int rank, int dtype,
                          const void* hidden, const void* W1, const int32_t* anchor,
                          const int32_t* tokens, const float* w, float bias, const float* temps,
                          float* conf, int32_t* status, hipStream_t stream) {
  const char* fn = "dspark_confidence_sts";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  if (H < 8 || H % 8) return fail(DSPARK_EINVAL, "%s: H=%d must be a positive multiple of 8", fn, H);
  REQUIRE_PTR(hidden); REQUIRE_PTR(W1); REQUIRE_PTR(anchor); REQUIRE_PTR(tokens);
  REQUIRE_PTR(w); REQUIRE_PTR(temps); REQUIRE_PTR(conf); OPT_PTR(status);
  return hip_status(fn, dspark::launch_confidence(B, gamma, H, V, rank, dtype, hidden, W1, anchor,
                                                  tokens, w, bias, temps, conf, status, stream));
}

size_t dspark_schedule_workspace(int R, int gamma) {
  if (R < 1 || gamma < 1 || gamma > 64) return 0;
  return dspark::schedule_workspace_bytes(R, gamma);
}

// checks shared by the scheduler entry points (all but the workspace);
// static: file-local despite the C linkage of this block
static int check_schedule_args(const char* fn, int R, int gamma, const float* conf,
                               int32_t* ell, int32_t* order, double* stats, int32_t* status) {
  if (R < 1) return fail(DSPARK_EINVAL, "%s: R=%d must be >= 1", fn, R);
  if (gamma < 1 || gamma > 64) return fail(DSPARK_EINVAL, "%s: gamma=%d outside [1,64]", fn, gamma);
  if ((long long)R * gamma > dspark::kScheduleMaxKeys)
    return fail(DSPARK_EUNSUPPORTED, "%s: R*gamma=%lld exceeds %d candidates", fn,
                (long long)R * gamma, dspark::kScheduleMaxKeys);
  REQUIRE_PTR(conf); REQUIRE_PTR(ell); OPT_PTR(order); OPT_PTR(stats); OPT_PTR(status);
  return DSPARK_OK;
}
static int check_schedule(const char* fn, int R, int gamma, const float* conf, int32_t* ell,
                          int32_t* order, double* stats, int32_t* status, void* workspace,
                          size_t workspace_bytes) {
  const int rc = check_schedule_args(fn, R, gamma, conf, ell, order, stats, status);
  if (rc) return rc;
  const size_t need = dspark::schedule_workspace_bytes(R, gamma);
  if (need && (!workspace || workspace_bytes < need))
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
  if (need && !aligned16(workspace))
    return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  return DSPARK_OK;
}

int dspark_schedule(int R, int gamma, const float* conf, const double* sps, int sps_len,
                    int32_t* ell, int32_t* order, double* stats, int32_t* status,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dspark_schedule";
  if (sps_len < 1) return fail(DSPARK_EINVAL, "%s: sps_len=%d must be >= 1", fn, sps_len);
  REQUIRE_PTR(sps);
  int rc = check_schedule(fn, R, gamma, conf, ell, order, stats, status, workspace,
                          workspace_bytes);
  if (rc) return rc;
  return hip_status(fn, dspark::launch_schedule(R, gamma, conf, sps, sps_len, dspark::kSchedTheta,
                                                0.0, nullptr, ell, order, stats, status,
                                                workspace, stream));
}

int dspark_schedule_noalloc(int R, int gamma, const float* conf, const double* sps, int sps_len,
                            int32_t* ell, int32_t* order, double* stats, int32_t* status,
                            hipStream_t stream) {
  const char* fn = "dspark_schedule_noalloc";
  if (sps_len < 1) return fail(DSPARK_EINVAL, "%s: sps_len=%d must be >= 1", fn, sps_len);
  REQUIRE_PTR(sps);
  int rc = check_schedule_args(fn, R, gamma, conf, ell, order, stats, status);
  if (rc) return rc;
  const size_t need = dspark::schedule_workspace_bytes(R, gamma);
  if (need > dspark::schedule_scratch_bytes())
    return fail(DSPARK_EUNSUPPORTED,
                "%s: R*gamma=%lld needs %zu bytes of scratch, more than the %zu bytes the "
                "allocation-free variant holds", fn, (long long)R * gamma, need,
                dspark::schedule_scratch_bytes());
  int32_t* scr = nullptr;
  if (need) {
    hipError_t e = hipSuccess;
    scr = dspark::schedule_scratch(&e);
    if (!scr) return hip_status(fn, e != hipSuccess ? e : hipErrorInvalidSymbol);
  }
  return hip_status(fn, dspark::launch_schedule(R, gamma, conf, sps, sps_len, dspark::kSchedTheta,
                                                0.0, nullptr, ell, order, stats, status, scr,
                                                stream, /*traced=*/false));
}

int dspark_schedule_capacity(int R, int gamma, const float* conf, const double* capacity,
                             int32_t* ell, int32_t* order, double* stats, int32_t* status,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dspark_schedule_capacity";
  int rc = check_schedule(fn, R, gamma, conf, ell, order, stats, status, workspace,
                          workspace_bytes);
  if (rc) return rc;
  if (!capacity) return fail(DSPARK_EINVAL, "%s: 'capacity' is NULL", fn);
  if (reinterpret_cast<uintptr_t>(capacity) & 7u)
    return fail(DSPARK_EALIGN, "%s: 'capacity' is not 8-byte aligned", fn);
  return hip_status(fn, dspark::launch_schedule(R, gamma, conf, nullptr, 0,
                                                dspark::kSchedCapacity, 0.0, capacity, ell,
                                                order, stats, status, workspace, stream));
}

int dspark_schedule_threshold(int R, int gamma, const float* conf, double threshold,
                              int32_t* ell, int32_t* order, double* stats, int32_t* status,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dspark_schedule_threshold";
  int rc = check_schedule(fn, R, gamma, conf, ell, order, stats, status, workspace,
                          workspace_bytes);
  if (rc) return rc;
  return hip_status(fn, dspark::launch_schedule(R, gamma, conf, nullptr, 0,
                                                dspark::kSchedThreshold, threshold, nullptr,
                                                ell, order, stats, status, workspace, stream));
}

size_t dspark_verify_workspace(int B, int gamma, int V, int rank, int dtype) {
  if (check_dims("dspark_verify_workspace", B, gamma, V, rank, dtype) != DSPARK_OK) return 0;
  return dspark::verify_workspace_bytes(B, gamma, V, rank, dtype);
}

int dspark_verify(int B, int gamma, int V, int rank, int dtype, const void* target, const void* U,
                  const void* W1, const void* W2, const int32_t* anchor, const int32_t* tokens,
                  const float* q_tok, const float* row_max, const float* row_logZ,
                  const float* temperature, const float* uniforms, const int32_t* ell,
                  int32_t* out_tokens, int32_t* n_accepted, float* ratio, int32_t* status,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dspark_verify";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  REQUIRE_PTR(target); REQUIRE_PTR(U); REQUIRE_PTR(W1); REQUIRE_PTR(W2); REQUIRE_PTR(anchor);
  REQUIRE_PTR(tokens); REQUIRE_PTR(q_tok); REQUIRE_PTR(row_max); REQUIRE_PTR(row_logZ);
  REQUIRE_PTR(temperature); REQUIRE_PTR(uniforms); REQUIRE_PTR(ell); REQUIRE_PTR(out_tokens);
  REQUIRE_PTR(n_accepted); OPT_PTR(ratio); OPT_PTR(status);
  const size_t need = dspark::verify_workspace_bytes(B, gamma, V, rank, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  return hip_status(fn, dspark::launch_verify(B, gamma, V, rank, dtype, target, U, W1, W2, anchor,
                                              tokens, q_tok, row_max, row_logZ, temperature,
                                              uniforms, ell, out_tokens, n_accepted, ratio, status,
                                              workspace, stream));
}

}  // extern "C"

int dspark_verify_rnn(int B, int gamma, int V, int rank, int dtype, const void* target,
                      const void* U, const void* emb, const void* W2, const int32_t* anchor,
                      const int32_t* tokens, const float* q_tok, const float* row_max,
                      const float* row_logZ, const float* temperature, const float* uniforms,
                      const int32_t* ell, int32_t* out_tokens, int32_t* n_accepted, float* ratio,
                      int32_t* status, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  const char* fn = "dspark_verify_rnn";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  REQUIRE_PTR(target); REQUIRE_PTR(U); REQUIRE_PTR(emb); REQUIRE_PTR(W2); REQUIRE_PTR(anchor);
  REQUIRE_PTR(tokens); REQUIRE_PTR(q_tok); REQUIRE_PTR(row_max); REQUIRE_PTR(row_logZ);
  REQUIRE_PTR(temperature); REQUIRE_PTR(uniforms); REQUIRE_PTR(ell); REQUIRE_PTR(out_tokens);
  REQUIRE_PTR(n_accepted); OPT_PTR(ratio); OPT_PTR(status);
  const size_t need = dspark::verify_workspace_bytes(B, gamma, V, rank, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  return hip_status(fn, dspark::launch_verify(B, gamma, V, rank, dtype, target, U, emb, W2,
                                              anchor, tokens, q_tok, row_max, row_logZ,
                                              temperature, uniforms, ell, out_tokens, n_accepted,
                                              ratio, status, workspace, stream,
                                              /*emb_rows=*/true));
}

size_t dspark_tv_label_workspace(int B, int gamma, int V, int rank, int dtype) {
  if (check_dims("dspark_tv_label_workspace", B, gamma, V, rank, dtype) != DSPARK_OK) return 0;
  return dspark::tv_workspace_bytes(B, gamma, V);
}

int dspark_tv_label(int B, int gamma, int V, int rank, int dtype, const void* target,
                    const void* U, const void* W1, const void* W2, const int32_t* anchor,
                    const int32_t* tokens, const float* row_max, const float* row_logZ,
                    const float* temperature, float* tv, float* label, int32_t* status,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dspark_tv_label";
  int rc = check_dims(fn, B, gamma, V, rank, dtype);
  if (rc) return rc;
  REQUIRE_PTR(target); REQUIRE_PTR(U); REQUIRE_PTR(W1); REQUIRE_PTR(W2); REQUIRE_PTR(anchor);
  REQUIRE_PTR(tokens); REQUIRE_PTR(row_max); REQUIRE_PTR(row_logZ); REQUIRE_PTR(temperature);
  REQUIRE_PTR(tv); OPT_PTR(label); OPT_PTR(status);
  const size_t need = dspark::tv_workspace_bytes(B, gamma, V);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSPARK_EALIGN, "%s: workspace not 16-byte aligned", fn);
  return hip_status(fn, dspark::launch_tv_label(B, gamma, V, rank, dtype, target, U, W1, W2,
                                                anchor, tokens, row_max, row_logZ, temperature,
                                                tv, label, status, workspace, stream));
}
