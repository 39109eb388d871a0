// Device-side building blocks shared by the libdspark kernels (gfx950).
//
// Tiling used by every vocabulary-streaming kernel
// -------------------------------------------------
// A wave owns a "wave tile" of 32 requests x 256 vocabulary entries.  The
// Markov bias of the tile is one 32 x 256 x rank contraction on the bf16
// matrix cores: v_mfma_f32_32x32x16_bf16, 8 output sub-tiles of 32 x 32,
// rank/16 k-steps each.  Operand layout of that instruction (lane l, c =
// l % 32, h = l / 32):
//     A: row c,    k = 8h .. 8h+7 of the k-step      (8 bf16 per lane)
//     B: column c, k = 8h .. 8h+7 of the k-step      (8 bf16 per lane)
//     D: column c, rows 8*(j/4) + 4h + (j%4) for j = 0..15
// Rows are requests (A = gathered W1 rows), columns are vocabulary entries
// (B = W2t rows, which are k-contiguous).  Column c of sub-tile t is mapped
// to vocabulary entry v0 + 8c + t, so after the contraction each lane holds,
// for each of its 16 requests, 8 CONSECUTIVE vocabulary entries: the base
// logits U are then read as one 16-byte load per (lane, request), and the
// 32 lanes of a half-wave cover 512 contiguous bytes of a U row.
//
// A "chunk" is 64 consecutive vocabulary entries (lanes c = 8q..8q+7 of a
// half-wave); 4 chunks make the 256-entry tile.  Sampling is two-level:
// per-chunk partial sums are written by the streaming kernel, and the
// per-request kernel scans them in fp64 and recomputes only the one chunk
// where the cumulative sum crosses u * Z.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

constexpr int kWave = 64;
constexpr int kTileM = 32;        // requests per wave tile
constexpr int kTileV = 256;       // vocabulary entries per wave tile
constexpr int kChunk = 64;        // vocabulary entries per sampling chunk
constexpr int kChunksPerTile = kTileV / kChunk;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline int n_tiles(int V) { return (V + kTileV - 1) / kTileV; }
__host__ __device__ inline int n_chunks(int V) { return n_tiles(V) * kChunksPerTile; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// 8 consecutive elements -> fp32 (bf16 path: one 16-byte load)
__device__ inline void load8_f32(const uint16_t* p, float out[8]) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void load8_f32(const float* p, float out[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
// streamed (read-once) variants: non-temporal so they do not evict W2t
__device__ inline void load8_f32_stream(const uint16_t* p, float out[8]) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void load8_f32_stream(const float* p, float out[8]) {
  f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + 1);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ inline bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ inline void flag(int32_t* status, int bits) {
  if (status) atomicOr(reinterpret_cast<int*>(status), bits);
}

__device__ inline int clamp_token(int t, int V, int32_t* status) {
  if (t < 0 || t >= V) {
    flag(status, DSPARK_DEV_BAD_TOKEN);
    return t < 0 ? 0 : V - 1;
  }
  return t;
}

// request row m(j) of accumulator element j for half-wave h (D layout above)
__device__ inline int acc_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

// ---------------------------------------------------------------------------
// Markov bias of one wave tile.
//   acc[t][j] = sum_k W1[prevs[m(j)]][k] * W2t[v0 + 8c + t][k]
// prevs[0..31] are the W1 rows of the wave's 32 request rows (-1 = empty
// row, contributes zeros).  Lanes whose column c lies outside
// [col_lo, col_hi) feed zeros for B: this recomputes a single chunk
// bit-identically, because each output element depends only on its own A
// row and B column and the k-step order is fixed.
// Must be called by all 64 lanes of the wave (matrix instructions).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline void bias_tile(const T* __restrict__ W1, const int* prevs,
                                 const T* __restrict__ W2t, int v0, int V, int rank,
                                 int col_lo, int col_hi, f32x16_t acc[8]);

template <>
__device__ inline void bias_tile<uint16_t>(const uint16_t* __restrict__ W1, const int* prevs,
                                           const uint16_t* __restrict__ W2t, int v0, int V,
                                           int rank, int col_lo, int col_hi, f32x16_t acc[8]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x16_t{};
  const bool col_ok = (c >= col_lo) && (c < col_hi);
  const uint16_t* brow[8];
  bool bok[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    int v = v0 + 8 * c + t;
    bok[t] = col_ok && (v < V);
    brow[t] = W2t + (size_t)(bok[t] ? v : 0) * rank + 8 * h;
  }
  const int pa = prevs[c];
  const bool aok = pa >= 0;
  const uint16_t* ap = W1 + (size_t)(aok ? pa : 0) * rank + 8 * h;
  const bf16x8_t zero = bf16x8_t{};
  for (int ks = 0; ks < rank; ks += 16) {
    bf16x8_t a = load_bf16x8(ap + ks);
    a = aok ? a : zero;
    bf16x8_t b[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      b[t] = load_bf16x8(brow[t] + ks);
      b[t] = bok[t] ? b[t] : zero;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[t], acc[t], 0, 0, 0);
  }
}

// fp32 inputs: plain FMA dot products (k ascending) in the same layout.
template <>
__device__ inline void bias_tile<float>(const float* __restrict__ W1, const int* prevs,
                                        const float* __restrict__ W2t, int v0, int V, int rank,
                                        int col_lo, int col_hi, f32x16_t acc[8]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  const bool col_ok = (c >= col_lo) && (c < col_hi);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    int v = v0 + 8 * c + t;
    bool vok = col_ok && v < V;
    const float* brow = W2t + (size_t)(vok ? v : 0) * rank;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int p = prevs[acc_row(j, h)];
      float s = 0.f;
      if (vok && p >= 0) {
        const float* arow = W1 + (size_t)p * rank;
        for (int i = 0; i < rank; ++i) s = fmaf(arow[i], brow[i], s);
      }
      acc[t][j] = s;
    }
  }
}

}  // namespace dspark

namespace dspark {

// ---------------------------------------------------------------------------
// Block-wide reductions / scans for 256-thread work-groups (4 waves).
// `scratch` must hold at least 8 doubles of shared memory.  All threads of
// the block must call them.
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ inline int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ inline int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline float block_max(float v, double* scratch) {
  float* s = reinterpret_cast<float*>(scratch);
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, s[w]);
  return r;
}
__device__ inline int block_min_int(int v, double* scratch) {
  int* s = reinterpret_cast<int*>(scratch);
  v = wave_min_int(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = s[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = min(r, s[w]);
  return r;
}
__device__ inline int block_max_int(int v, double* scratch) {
  int* s = reinterpret_cast<int*>(scratch);
  v = wave_max_int(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = s[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = max(r, s[w]);
  return r;
}
__device__ inline double block_sum(double v, double* scratch) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += scratch[w];
  return r;
}
// Prefix sum over threads in thread order.  Thread i gets [*start, *end):
// the running total before and after its own value.  The intervals of
// consecutive threads share their end points bit for bit (each end is
// computed once and reused as the next start), so they tile [0, total)
// exactly; returns the block total.  Deterministic association.
__device__ inline double block_scan_interval(double v, double* scratch, double* start,
                                             double* end) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  __syncthreads();
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  double base = 0.0, tot = 0.0;
  const int nw = (int)(blockDim.x >> 6);
  for (int w = 0; w < nw; ++w) {
    if (w == wave) base = tot;
    tot = tot + scratch[w];
  }
  *start = (lane == 0) ? base : base + excl;
  *end = (lane == 63) ? ((wave == nw - 1) ? tot : base + incl) : base + incl;
  return tot;
}

}  // namespace dspark
