// dspark_confidence: c[b,k] = sigmoid(w_h . h[b,k] + w_e . W1[prev_k] + bias).
//
// [weigao] part 3 / [billytse] 5: a linear layer over the position's hidden
// state and the Markov embedding of the previous token, squashed by a
// sigmoid.  [xhh] non-anticipation note: position k reads x_{k-1} (the
// anchor for k = 0), never x_k.  One wave per (b, k): the H + rank dot
// product is read with 16-byte loads and reduced across the wave in fp32
// (conf_row.hpp, which the single-launch draft kernel's draw waves share).
//
// With per-position temperatures (dspark_confidence_sts: sequential
// temperature scaling, [billytse] 5.2; [weigao] part 3) the logit of
// position k is divided by temps[k] before the sigmoid; a temperature that
// is not finite and positive leaves the logit unchanged and is flagged.
#include "conf_row.hpp"
#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "trace.hpp"

namespace dspark {

template <typename T>
__global__ __launch_bounds__(256) void confidence_kernel(
    int B, int gamma, int H, int V, int rank, const T* __restrict__ hidden,
    const T* __restrict__ W1, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ w, float bias,
    const float* __restrict__ temps, float* __restrict__ conf, int32_t* status) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= B * gamma) return;
  const int b = row / gamma, k = row % gamma;
  int prev = (k == 0) ? anchor[b] : tokens[(size_t)b * gamma + k - 1];
  prev = clamp_token(prev, V, status);
  const float dot = conf_dot_wave<T>(hidden + (size_t)row * H, W1 + (size_t)prev * rank, w, H,
                                     rank, lane);
  if (lane == 0) conf[row] = conf_from_dot(dot, bias, temps, k, status);
}

hipError_t launch_confidence(int B, int gamma, int H, int V, int rank, int dtype,
                             const void* hidden, const void* W1, const int32_t* anchor,
                             const int32_t* tokens, const float* w, float bias,
                             const float* temps, float* conf, int32_t* status,
                             hipStream_t stream) {
  const int rows = B * gamma;
  const dim3 grid((rows + 3) / 4), blk(256);
  TraceScope ts("confidence_kernel", stream);
  if (dtype == DSPARK_BF16)
    confidence_kernel<uint16_t><<<grid, blk, 0, stream>>>(
        B, gamma, H, V, rank, static_cast<const uint16_t*>(hidden),
        static_cast<const uint16_t*>(W1), anchor, tokens, w, bias, temps, conf, status);
  else
    confidence_kernel<float><<<grid, blk, 0, stream>>>(
        B, gamma, H, V, rank, static_cast<const float*>(hidden), static_cast<const float*>(W1),
        anchor, tokens, w, bias, temps, conf, status);
  return hipGetLastError();
}

}  // namespace dspark
