// dspark_confidence: c[b,k] = sigmoid(w_h . h[b,k] + w_e . W1[prev_k] + bias).
//
// [weigao] part 3 / [billytse] 5: a linear layer over the position's hidden
// state and the Markov embedding of the previous token, squashed by a
// sigmoid.  [xhh] non-anticipation note: position k reads x_{k-1} (the
// anchor for k = 0), never x_k.  One wave per (b, k): the H + rank dot
// product is read with 16-byte loads and reduced across the wave in fp32.
//
// With per-position temperatures (dspark_confidence_sts: sequential
// temperature scaling, [billytse] 5.2; [weigao] part 3) the logit of
// position k is divided by temps[k] before the sigmoid; a temperature that
// is not finite and positive leaves the logit unchanged and is flagged.
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
  const T* hrow = hidden + (size_t)row * H;
  const T* erow = W1 + (size_t)prev * rank;
  float s = 0.f;
  for (int i = 8 * lane; i < H; i += 8 * kWave) {
    float hv[8];
    load8_f32_stream(hrow + i, hv);
    const float4 w0 = *reinterpret_cast<const float4*>(w + i);
    const float4 w1 = *reinterpret_cast<const float4*>(w + i + 4);
    s += hv[0] * w0.x + hv[1] * w0.y + hv[2] * w0.z + hv[3] * w0.w;
    s += hv[4] * w1.x + hv[5] * w1.y + hv[6] * w1.z + hv[7] * w1.w;
  }
  for (int i = 8 * lane; i < rank; i += 8 * kWave) {
    float ev[8];
    load8_f32(erow + i, ev);
    const float* we = w + H + i;
#pragma unroll
    for (int t = 0; t < 8; ++t) s += ev[t] * we[t];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) {
    float z = s + bias;
    if (temps) {
      const float t = temps[k];
      if (t > 0.f && t <= 3.0e38f)
        z = z / t;
      else
        flag(status, DSPARK_DEV_BAD_CONF);
    }
    conf[row] = 1.f / (1.f + expf(-z));
  }
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
