// Per-tile statistics of the draft kernels (gfx950): the first level of the
// two-level inverse-CDF draw ([billytse] 3.3: each position's token is
// sampled from softmax(U_k + W1[prev] W2)).  A 64-entry vocabulary tile of
// one request reduces to (max, sum of exp((y - max) / T), lowest argmax);
// the per-request draw scans these words and recomputes only the tile where
// the cumulative mass crosses u * Z.
#pragma once

#include "dspark_common.hpp"

namespace dspark {

struct TileStats {
  uint64_t* ms;   // [B][nT] (max, sum) as two fp32: max over the tile of y' = z + bias
                  // (unscaled logits), sum over the tile of exp((y' - max) / T)
  int32_t* arg;   // [B][nT] lowest vocabulary index attaining the max (greedy rows only)
};
__device__ inline uint64_t pack_ms(float mx, float s) {
  return (uint64_t)__float_as_uint(mx) | ((uint64_t)__float_as_uint(s) << 32);
}
__device__ inline float ms_max(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ inline float ms_sum(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

// inverse temperature of a request; 0 marks greedy
__device__ inline float inv_temp(float T) { return (T > 0.f) ? 1.f / T : 0.f; }

// Summand of the tile mass: exp((y' - m') / T) as 2^(y' ce - m' ce) with
// ce = log2(e) / T and mc = m' ce.  The statistics pass and the sampler's
// recompute evaluate exactly this expression.
__device__ inline float tile_term(float yp, float ce, float mc) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(yp, ce, -mc));
}

// Reduction of one block-tile for this lane's request (column c): acc holds
// y' = base logit + bias (-inf past V); gives the tile max, lowest argmax
// (when `any_greedy`, which is wave-uniform) and exp-sum, combined over the
// two half-waves so both lanes of the request hold them.  `it` is the lane's
// inverse temperature (0 = greedy).
struct TileStat {
  float mx, s;
  int arg;
};
__device__ inline TileStat tile_reduce(const f32x16_t acc[kSub], int vt, float it,
                                       bool any_greedy) {
  const int h = (threadIdx.x & 63) >> 5;
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, acc[t][j]);
  }
  float lo, hi;
  half_pair(mx, lo, hi);
  mx = fmaxf(lo, hi);
  int arg = 0x7fffffff;
  if (any_greedy) {
    int off = 0x7fffffff;   // lowest in-lane offset 32t + j attaining the max
#pragma unroll
    for (int t = kSub - 1; t >= 0; --t) {
#pragma unroll
      for (int j = 15; j >= 0; --j) off = (acc[t][j] == mx) ? 32 * t + j : off;
    }
    arg = off == 0x7fffffff ? off : vt * kTileV + 16 * h + off;
    int alo, ahi;
    half_pair(arg, alo, ahi);
    arg = min(alo, ahi);
  }
  const float ce = it * kLog2e, mc = mx * ce;
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s += tile_term(acc[t][j], ce, mc);
  }
  half_pair(s, lo, hi);
  return TileStat{mx, lo + hi, arg};
}

// store the statistics of request b (< B) for tile vt (device-coherent);
// the argmax only for a greedy request (inverse temperature `it` 0)
__device__ inline void store_tile_stat(const TileStats& ts, int b, int nT, int vt,
                                       const TileStat& st, float it) {
  const size_t i = (size_t)b * nT + vt;
  st_dev(ts.ms + i, pack_ms(st.mx, st.s));
  if (!(it > 0.f)) st_dev(ts.arg + i, st.arg);
}

}  // namespace dspark

namespace dspark {

// Reduction of ONE 32-entry sub-tile (sub-tile `t` of tile vt) for this
// lane's request: accumulator element j of lane (c, h) is entry
// vt * 64 + 32 t + 16 h + j.  Same outputs as tile_reduce over half a tile.
__device__ inline TileStat half_reduce(const f32x16_t& acc, int vt, int t, float it,
                                       bool any_greedy) {
  const int h = (threadIdx.x & 63) >> 5;
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) mx = fmaxf(mx, acc[j]);
  float lo, hi;
  half_pair(mx, lo, hi);
  mx = fmaxf(lo, hi);
  int arg = 0x7fffffff;
  if (any_greedy) {
    int off = 0x7fffffff;
#pragma unroll
    for (int j = 15; j >= 0; --j) off = (acc[j] == mx) ? j : off;
    arg = off == 0x7fffffff ? off : vt * kTileV + 32 * t + 16 * h + off;
    int alo, ahi;
    half_pair(arg, alo, ahi);
    arg = min(alo, ahi);
  }
  const float ce = it * kLog2e, mc = mx * ce;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += tile_term(acc[j], ce, mc);
  half_pair(s, lo, hi);
  return TileStat{mx, lo + hi, arg};
}

}  // namespace dspark
