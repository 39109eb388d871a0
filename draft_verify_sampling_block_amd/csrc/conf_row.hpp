// The confidence head's value for one (request, position), computed by one
// wave ([weigao] part 3; [billytse] 5: a linear layer over the position's
// hidden state and the Markov embedding of the previous token, through a
// sigmoid; with sequential temperature scaling ([billytse] 5.2) the logit is
// divided by the position's temperature first).  Shared by the standalone
// head's kernel and the draw waves of the single-launch draft kernel, so the
// two give the same bits.
//
// Lane l takes entries 8l .. 8l+7 of every 512-entry block of the hidden
// row (16-byte loads), up to kConfBlocks blocks (4096 entries) held at once:
// all of a chunk's loads are issued before the first is used, and the draft
// kernel issues them before it waits for a position's statistics and adds
// them up afterwards.  Then the embedding part, then the 64 partial sums are
// added across the wave.
#pragma once

#include "dspark_common.hpp"

namespace dspark {

constexpr int kConfBlocks = 8;   // 512-entry blocks of a hidden row per chunk

// 8 hidden entries as loaded (streamed: each is read once)
template <typename T>
struct HBlk;
template <>
struct HBlk<uint16_t> {
  u32x4_t v;
};
template <>
struct HBlk<float> {
  f32x4_t a, b;
};
__device__ inline void hblk_load(const uint16_t* p, HBlk<uint16_t>& h) {
  h.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ inline void hblk_load(const float* p, HBlk<float>& h) {
  h.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  h.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + 1);
}
__device__ inline void hblk_f32(const HBlk<uint16_t>& h, float out[8]) {
  const uint32_t w[4] = {h.v.x, h.v.y, h.v.z, h.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void hblk_f32(const HBlk<float>& h, float out[8]) {
  out[0] = h.a.x; out[1] = h.a.y; out[2] = h.a.z; out[3] = h.a.w;
  out[4] = h.b.x; out[5] = h.b.y; out[6] = h.b.z; out[7] = h.b.w;
}

// one chunk's loads: blocks i0, i0 + 512, ... (indices past H read a valid
// entry, which the sum skips)
template <typename T>
__device__ inline void conf_chunk_load(const T* hrow, int H, int i0, HBlk<T> (&h)[kConfBlocks]) {
#pragma unroll
  for (int u = 0; u < kConfBlocks; ++u) hblk_load(hrow + min(i0 + u * 8 * kWave, H - 8), h[u]);
}
// s += w[i] * hidden[i] over the chunk's entries, block by block
template <typename T>
__device__ inline float conf_chunk_add(const HBlk<T> (&h)[kConfBlocks], const float* w, int H,
                                       int i0, float s) {
#pragma unroll
  for (int u = 0; u < kConfBlocks; ++u) {
    const int i = i0 + u * 8 * kWave;
    if (i < H) {
      float hv[8];
      hblk_f32(h[u], hv);
      const float4 w0 = *reinterpret_cast<const float4*>(w + i);
      const float4 w1 = *reinterpret_cast<const float4*>(w + i + 4);
      s += hv[0] * w0.x + hv[1] * w0.y + hv[2] * w0.z + hv[3] * w0.w;
      s += hv[4] * w1.x + hv[5] * w1.y + hv[6] * w1.z + hv[7] * w1.w;
    }
  }
  return s;
}
// then the embedding part and the sum over the wave
template <typename T>
__device__ inline float conf_finish_dot(const T* erow, const float* w, int H, int rank, int lane,
                                        float s) {
  for (int i = 8 * lane; i < rank; i += 8 * kWave) {
    float ev[8];
    load8_f32(erow + i, ev);
    const float* we = w + H + i;
#pragma unroll
    for (int t = 0; t < 8; ++t) s += ev[t] * we[t];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  return s;
}

// w[0:H] . hrow + w[H:H+rank] . erow, every lane holding the sum (H a
// multiple of 8)
template <typename T>
__device__ inline float conf_dot_wave(const T* hrow, const T* erow, const float* w, int H,
                                      int rank, int lane) {
  float s = 0.f;
  for (int i0 = 8 * lane; i0 - 8 * lane < H; i0 += kConfBlocks * 8 * kWave) {
    HBlk<T> h[kConfBlocks];
    conf_chunk_load(hrow, H, i0, h);
    s = conf_chunk_add(h, w, H, i0, s);
  }
  return conf_finish_dot(erow, w, H, rank, lane, s);
}

// sigmoid((dot + bias) / temps[k]); temps NULL: no scaling.  A temperature
// that is not finite and positive leaves the logit unchanged and is flagged.
__device__ inline float conf_from_dot(float dot, float bias, const float* temps, int k,
                                      int32_t* status) {
  float z = dot + bias;
  if (temps) {
    const float t = temps[k];
    if (t > 0.f && t <= 3.0e38f)
      z = z / t;
    else
      flag(status, DSPARK_DEV_BAD_CONF);
  }
  return 1.f / (1.f + expf(-z));
}

}  // namespace dspark
