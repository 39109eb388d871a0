// Device-side building blocks shared by the libdspark kernels (gfx950).
//
// Tiling used by every vocabulary-streaming kernel
// -------------------------------------------------
// A wave owns a "wave tile" of 32 requests x 128 vocabulary entries.  The
// Markov bias of the tile is one 32 x 128 x rank contraction on the bf16
// matrix cores: v_mfma_f32_32x32x16_bf16, 4 output sub-tiles of 32 x 32,
// rank/16 k-steps each.  Operand layout of that instruction (lane l, c =
// l % 32, h = l / 32):
//     A: row c,    k = 8h .. 8h+7 of the k-step      (8 bf16 per lane)
//     B: column c, k = 8h .. 8h+7 of the k-step      (8 bf16 per lane)
//     D: column c, rows 8*(j/4) + 4h + (j%4) for j = 0..15
// Rows are requests (A = gathered W1 rows), columns are vocabulary entries
// (B = W2t rows, which are k-contiguous).  Column c of sub-tile t is mapped
// to vocabulary entry v0 + 4c + t, so after the contraction each lane holds,
// for each of its 16 requests, 4 CONSECUTIVE vocabulary entries: the base
// logits are read as one 8-byte load per (lane, request) and a half-wave
// covers 256 contiguous bytes of a row.
//
// The W2t rows of a tile (128 x rank bf16, 64 KB at rank 256) are staged
// once per work-group into LDS with global->LDS DMA loads and shared by the
// work-group's 4 waves (one 32-request block each).  LDS rows keep their 16
// byte k-chunks XOR-swizzled by (row/4) so that the 16 lanes of a matrix
// operand read hit 16 distinct bank groups.
//
// A "chunk" is 64 consecutive vocabulary entries (lanes c = 16q..16q+15 of
// a half-wave); 2 chunks make the 128-entry tile.  Sampling is two-level:
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
constexpr int kTileV = 128;       // vocabulary entries per tile
constexpr int kSub = 4;           // 32-column matrix sub-tiles per tile
constexpr int kChunk = 64;        // vocabulary entries per sampling chunk
constexpr int kChunksPerTile = kTileV / kChunk;
constexpr int kMaxKSteps = 16;    // rank <= 256
constexpr int kLdsTileBytes = kTileV * kMaxKSteps * 2 * 16;   // 64 KB

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline int n_tiles(int V) { return (V + kTileV - 1) / kTileV; }
__host__ __device__ inline int n_chunks(int V) { return n_tiles(V) * kChunksPerTile; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// 4 consecutive elements -> fp32 (streamed, read-once: non-temporal)
__device__ inline void load4_f32_stream(const uint16_t* p, float out[4]) {
  u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  out[0] = __uint_as_float(v.x << 16);
  out[1] = __uint_as_float(v.x & 0xFFFF0000u);
  out[2] = __uint_as_float(v.y << 16);
  out[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
__device__ inline void load4_f32_stream(const float* p, float out[4]) {
  f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
// raw 4-element loads kept in registers until the epilogue (8 bytes for
// bf16, 16 bytes for fp32)
template <typename T> struct Raw4;
template <> struct Raw4<uint16_t> { using type = u32x2_t; };
template <> struct Raw4<float> { using type = u32x4_t; };
template <typename T> using raw4_t = typename Raw4<T>::type;

__device__ inline u32x4_t load4_raw(const float* p) {
  f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return __builtin_bit_cast(u32x4_t, v);
}
__device__ inline u32x2_t load4_raw(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}
__device__ inline void unpack4(const u32x2_t& r, float out[4]) {
  out[0] = __uint_as_float(r.x << 16);
  out[1] = __uint_as_float(r.x & 0xFFFF0000u);
  out[2] = __uint_as_float(r.y << 16);
  out[3] = __uint_as_float(r.y & 0xFFFF0000u);
}
__device__ inline void unpack4(const u32x4_t& r, float out[4]) {
  out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
  out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
}

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
// accumulator element that holds request row m for half-wave (m/4)%2
__device__ inline int row_half(int m) { return (m >> 2) & 1; }
__device__ inline int row_elem(int m) { return 4 * (m >> 3) + (m & 3); }

// ---------------------------------------------------------------------------
// W2t tile in LDS: 128 rows (tile-local vocabulary index r) of rank bf16,
// i.e. nq = rank/8 chunks of 16 bytes per row, chunk q stored at slot
// q ^ swz(r).  Row r is read by lane column c = r/4 of sub-tile t = r%4.
// ---------------------------------------------------------------------------
__device__ inline int lds_swz(int r, int nq) { return ((r >> 2) & 15) & (nq - 1); }
__device__ inline int lds_off(int r, int q, int nq) { return (r * nq + (q ^ lds_swz(r, nq))) * 16; }

// Issue DMA loads of tile rows [row_lo, row_lo + nrows) into `lds`; every
// wave of the work-group takes part.  Rows past V read row V-1 (their
// columns are masked later).  Completion: s_waitcnt + barrier by the caller.
__device__ inline void stage_w2_rows(const uint16_t* __restrict__ W2t, int v0, int V, int rank,
                                     char* lds, int row_lo, int nrows) {
  const int nq = rank >> 3;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int nslots = nrows * nq;           // a multiple of 64 (nrows in {64,128}, nq >= 4)
  const int s_lo = row_lo * nq;
  for (int g = wave; g * 64 < nslots; g += nwaves) {
    const int s = s_lo + g * 64 + lane;
    const int r = s / nq, p = s - (s / nq) * nq;
    const int q = p ^ lds_swz(r, nq);
    int v = v0 + r;
    v = v < V ? v : V - 1;
    const uint16_t* src = W2t + (size_t)v * rank + q * 8;
    __builtin_amdgcn_global_load_lds(src, lds + (size_t)(s_lo + g * 64) * 16, 16, 0, 0);
  }
}

// Markov bias of one wave tile with B read from the LDS tile.
//   acc[t][j] = sum_k W1[prev(m(j))][k] * W2t[v0 + 4c + t][k]
// `afrag` holds this lane's A operand for every k-step (its row c =
// request c of the block, zeros for an empty row).  Lanes whose column c lies
// outside [col_lo, col_hi) feed zeros for B: this recomputes a single chunk
// bit-identically (each output element depends only on its own A row and B
// column, and the k-step order is fixed).  All 64 lanes must call it.
template <int KS>
__device__ inline void bias_tile_lds(const bf16x8_t afrag[KS], const char* lds, int col_lo,
                                     int col_hi, f32x16_t acc[kSub]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  constexpr int nq = 2 * KS;
  const bool col_ok = (c >= col_lo) && (c < col_hi);
  const bf16x8_t zero = bf16x8_t{};
#pragma unroll
  for (int t = 0; t < kSub; ++t) acc[t] = f32x16_t{};
  // B fragments double-buffered: the LDS reads of k-step ks+1 are issued
  // before the matrix instructions of k-step ks; the scheduling barrier
  // keeps the compiler from hoisting further reads (register pressure)
  bf16x8_t bcur[kSub], bnext[kSub];
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
    bcur[t] = *reinterpret_cast<const bf16x8_t*>(lds + lds_off(4 * c + t, h, nq));
    bcur[t] = col_ok ? bcur[t] : zero;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) {
#pragma unroll
      for (int t = 0; t < kSub; ++t) {
        bnext[t] = *reinterpret_cast<const bf16x8_t*>(lds + lds_off(4 * c + t, 2 * (ks + 1) + h, nq));
        bnext[t] = col_ok ? bnext[t] : zero;
      }
    }
#pragma unroll
    for (int t = 0; t < kSub; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ks], bcur[t], acc[t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kSub; ++t) bcur[t] = bnext[t];
  }
}

// this lane's A operand (row c = request `tok` or empty) for all k-steps
template <int KS>
__device__ inline void load_afrag(const uint16_t* __restrict__ W1, int tok, bf16x8_t afrag[KS]) {
  const int h = (threadIdx.x & 63) >> 5;
  const bf16x8_t zero = bf16x8_t{};
  const uint16_t* arow = W1 + (size_t)(tok >= 0 ? tok : 0) * (16 * KS) + 8 * h;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    afrag[ks] = load_bf16x8(arow + 16 * ks);
    afrag[ks] = tok >= 0 ? afrag[ks] : zero;
  }
}

// fp32 inputs: plain FMA dot products (k ascending) in the same layout.
// `tok` is this lane's A row (request c of the block, -1 = empty); the rows
// of the lane's outputs are fetched from the owning lanes.  All 64 lanes.
__device__ inline void bias_tile_f32(const float* __restrict__ W1, int tok,
                                     const float* __restrict__ W2t, int v0, int V, int rank,
                                     int col_lo, int col_hi, f32x16_t acc[kSub]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  const bool col_ok = (c >= col_lo) && (c < col_hi);
  int prow[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) prow[j] = __shfl(tok, acc_row(j, h), kWave);
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
    const int v = v0 + 4 * c + t;
    const bool vok = col_ok && v < V;
    const float* brow = W2t + (size_t)(vok ? v : 0) * rank;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int p = prow[j];
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
