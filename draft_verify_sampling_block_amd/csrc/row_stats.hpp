// Softmax statistics of one row of logits by one 256-thread work-group,
// shared by the verification and the acceptance-label kernels.
#pragma once

#include "dspark_common.hpp"

namespace dspark {

struct RowStats {
  float M;     // max of y = t * scale
  double Z;    // sum of exp(y - M) (0 for a greedy row)
  int arg;     // lowest index attaining M (greedy rows only; else 0x7fffffff)
};

// Every thread of the work-group calls it (`red`: 8 doubles of shared
// memory).  Each thread reads groups of kU chunks of 8 consecutive entries
// with all loads of a group in flight together; the running max and exp-sum
// are fp32 (the sum is rescaled when the max grows) and are combined across
// threads in fp64.
template <typename T>
__device__ inline RowStats row_stats(const T* __restrict__ row, int V, float scale, bool greedy,
                                     double* red) {
  constexpr int kU = 8;
  const int tid = threadIdx.x;
  float m = -INFINITY;
  float s32 = 0.f;
  int arg = 0x7fffffff;
  const int stride = 8 * 256;
  for (int base = 8 * tid; base < V; base += kU * stride) {
    // the loads are unconditional (chunks past the row re-read chunk 0 and
    // are masked afterwards) so that all kU are in flight together
    float y[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * stride;
      load8_f32_stream(row + (i < V ? i : 0), y[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (base + u * stride >= V) {
#pragma unroll
        for (int t = 0; t < 8; ++t) y[u][t] = -INFINITY;
      }
    }
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        y[u][t] *= scale;
        gm = fmaxf(gm, y[u][t]);
      }
    }
    if (gm > m) {
      if (greedy) {
#pragma unroll
        for (int u = kU - 1; u >= 0; --u) {
#pragma unroll
          for (int t = 7; t >= 0; --t)
            if (y[u][t] == gm) arg = base + u * stride + t;
        }
      } else if (s32 > 0.f) {
        s32 *= __expf(m - gm);
      }
      m = gm;
    }
    if (!greedy) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int t = 0; t < 8; ++t) s32 += __expf(y[u][t] - m);
      }
    }
  }
  const double s = (double)s32;
  const float M = block_max(m, red);
  int a = 0x7fffffff;
  if (greedy) a = (m == M) ? arg : 0x7fffffff;
  a = block_min_int(a, red);
  const double mine = (!greedy && m > -INFINITY) ? s * exp((double)m - (double)M) : 0.0;
  const double Zt = block_sum(mine, red);
  return RowStats{M, Zt, a};
}

}  // namespace dspark
