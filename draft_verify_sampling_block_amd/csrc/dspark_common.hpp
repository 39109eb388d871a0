// Device-side building blocks shared by the libdspark kernels (gfx950).
//
// Tiling used by every vocabulary-streaming kernel
// -------------------------------------------------
// The vocabulary is cut into 64-entry tiles.  A "block-tile" is one tile x
// 32 requests: its Markov bias is a 64 x 32 x rank contraction on the bf16
// matrix cores, v_mfma_f32_32x32x16_bf16, as 2 output sub-tiles of 32 x 32
// with rank/16 k-steps each.  Operand layout of that instruction (lane l,
// c = l % 32, h = l / 32):
//     A: row c,    k = 8h .. 8h+7 of the k-step      (8 bf16 per lane)
//     B: column c, k = 8h .. 8h+7 of the k-step      (8 bf16 per lane)
//     D: column c, rows 8*(j/4) + 4h + (j%4) for j = 0..15
// Rows are vocabulary entries (A = W2 columns, 8 consecutive k) and columns are
// requests (B = the W1 rows of the requests' previous tokens).  Matrix row
// i of sub-tile t stands for vocabulary entry v0 + 32t + sub_row_vocab(i),
// chosen so that accumulator element j of lane (c, h) is entry
// v0 + 32t + 16h + j of request c: every lane ends up with 2 runs of 16
// CONSECUTIVE vocabulary entries of ONE request.  The base logits are read
// as 16-byte loads straight into that layout, the temperature is the
// lane's own, and the per-tile reductions run inside the lane with one
// exchange between the two half-waves.
//
// W2 tiles staged in LDS are stored transposed, k-contiguous per
// vocabulary entry, in matrix-row order (LDS row
// 32t + i holds entry v0 + 32t + sub_row_vocab(i)), each row padded by one
// 16-byte chunk, so that the 16 lanes of each quarter-wave, which read 16
// consecutive rows at one k-chunk, hit 16 distinct bank groups.  The per-tile statistics (max, lowest argmax, sum of exp(y - max))
// are the first level of the two-level inverse-CDF draw; the per-request
// sampler scans them in fp64 and recomputes only the one tile where the
// cumulative mass crosses u * Z, with the same instructions on the same
// operands, hence bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dspark.h"
#include "dspark_launch.hpp"

namespace dspark {

constexpr int kWave = 64;
constexpr int kTileM = 32;        // requests per block
constexpr int kTileV = 64;        // vocabulary entries per tile
constexpr int kSub = 2;           // 32-column matrix sub-tiles per tile
constexpr int kMaxKSteps = 16;    // rank <= 256
constexpr int kLdsTileBytes = kTileV * (2 * kMaxKSteps + 1) * 16;   // 33 KB (padded rows)
constexpr int kMaxTiles = kMaxVocab / kTileV;     // 4096 (kMaxVocab: dspark_launch.hpp)
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline int n_tiles(int V) { return (V + kTileV - 1) / kTileV; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// This lane's base logits of one block-tile: for sub-tile t the 16
// consecutive entries v0 + 32t + 16h + [0, 16), kept raw (16-byte loads,
// streamed and read once: non-temporal) until the epilogue.
template <typename T> struct URow;
template <> struct URow<uint16_t> {
  static constexpr int kLoads = 2;   // 8 bf16 per load
  u32x4_t w[kSub][kLoads];
};
template <> struct URow<float> {
  static constexpr int kLoads = 4;   // 4 fp32 per load
  u32x4_t w[kSub][kLoads];
};

// `row` is the start of a length-V row.  A load that `ok` false or the end
// of the row excludes reads `safe` (any valid 16-byte-aligned address)
// instead, so no load is predicated; its values are meaningless and every
// caller discards them (entries past V start at -inf in init_acc, lanes of
// absent requests are never stored).  Nothing selects on the loaded values
// here, so the loads stay in flight until their first real use.  V % 8 == 0
// keeps every 16-byte load wholly inside or outside the row.
template <typename T>
__device__ inline void load_urow(URow<T>& u, const T* __restrict__ row, int v0, int V, bool ok,
                                 const T* __restrict__ safe) {
  const int h = (threadIdx.x & 63) >> 5;
  constexpr int per = 16 / (int)sizeof(T);
  const int vb = v0 + 16 * h, rem = V - vb;
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
#pragma unroll
    for (int q = 0; q < URow<T>::kLoads; ++q) {
      const bool in = ok && (32 * t + q * per < rem);
      const T* p = in ? row + vb + 32 * t + q * per : safe;
      u.w[t][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    }
  }
}
__device__ inline float urow_at(const URow<uint16_t>& u, int t, int j) {
  const uint32_t w = u.w[t][j >> 3][(j >> 1) & 3];
  return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}
__device__ inline float urow_at(const URow<float>& u, int t, int j) {
  return __uint_as_float(u.w[t][j >> 2][j & 3]);
}
// Start value of a block-tile accumulator: the base logits, -inf for the
// entries at or past V.  `rem` = V - (v0 + 16h) for this lane.
template <typename T>
__device__ inline void init_acc(const URow<T>& u, int rem, f32x16_t acc[kSub]) {
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t][j] = (32 * t + j < rem) ? urow_at(u, t, j) : -INFINITY;
  }
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

// Loads and stores of data exchanged between work-groups of one running
// kernel: relaxed atomics at device scope, so each access is coherent across
// the chip's L2 slices without whole-cache write-backs or invalidations.
// Ordering comes from the flag protocol around them (stores complete before
// a flag is raised; loads issue after the flag is seen).
template <typename X>
__device__ inline X ld_dev(const X* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename X>
__device__ inline void st_dev(X* p, X v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// lane l receives (x of lane l % 32, x of lane l % 32 + 32): the two
// half-waves' values in the same order on every lane
__device__ inline void half_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ inline void half_pair(int x, int& lo, int& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  lo = (int)r[0];
  hi = (int)r[1];
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

// vocabulary offset, within a 32-entry sub-tile, of matrix row i (the
// inverse of: accumulator element j of half-wave h holds offset 16h + j)
__host__ __device__ inline int sub_row_vocab(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// vocabulary offset within the tile of tile row r (r in [0, 64))
__host__ __device__ inline int tile_row_vocab(int r) { return (r & 32) + sub_row_vocab(r & 31); }

// ---------------------------------------------------------------------------
// Rows of rank bf16 in LDS (transposed W2 tiles, or gathered W1 rows): nq = rank/8
// chunks of 16 bytes per row plus one pad chunk, so a row takes nq + 1
// chunks.  nq + 1 is odd, so 16 consecutive rows read at one chunk land in
// 16 distinct 16-byte bank groups, and chunk q of row r sits at the fixed
// offset (r (nq + 1) + q) 16: a k-step's operand address is the row base
// plus an immediate.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int lds_row_bytes(int nq) { return (nq + 1) * 16; }
__device__ inline int lds_off(int r, int q, int nq) { return r * lds_row_bytes(nq) + q * 16; }

// DMA nrows rows into `lds` (row r <- src row row_of(r)); the pad chunk of
// each row is filled with the row's chunk 0.  Every wave of the work-group
// takes part.  Completion: s_waitcnt + barrier by the caller.
template <typename RowOf>
__device__ inline void stage_rows_lds(const uint16_t* __restrict__ src, int rank, char* lds,
                                      int nrows, RowOf&& row_of) {
  const int nq = rank >> 3, nc = nq + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int nslots = nrows * nc;
  for (int g = wave; g * 64 < nslots; g += nwaves) {
    const int s = g * 64 + lane;
    if (s < nslots) {
      const int r = s / nc, q = s - r * nc;
      __builtin_amdgcn_global_load_lds(src + (size_t)row_of(r) * rank + (q < nq ? q : 0) * 8,
                                       lds + (size_t)(g * 64) * 16, 16, 0, 0);
    }
  }
}

// Matrix row of the tile (the inverse of tile_row_vocab): vocabulary offset
// o in [0, 64) sits in tile row (o & 32) + 8 ((o >> 2) & 3) + 4 ((o >> 4) & 1)
// + (o & 3).
__host__ __device__ inline int tile_vocab_row(int o) {
  return (o & 32) | (((o >> 2) & 3) << 3) | (((o >> 4) & 1) << 2) | (o & 3);
}

// ---------------------------------------------------------------------------
// W2 is stored [rank, V]: row k holds coordinate k's weights over the whole
// vocabulary, so the 64 entries of one tile at one k are 128 contiguous
// bytes.  The matrix-core operand wants 8 consecutive k of ONE entry per
// lane, so a tile is transposed on its way into LDS: a thread loads a block
// of 4 k-rows x 8 entries (four 16-byte loads) and writes it as eight 8-byte
// k-runs, one per entry, into the padded k-contiguous image that the LDS
// operand readers use (LDS row r = entry v0 + tile_row_vocab(r); chunk q =
// k 8q .. 8q + 7).  A tile has (rank / 4) x 8 blocks.
// ---------------------------------------------------------------------------
struct W2Block {
  u32x4_t r[4];   // r[i] = W2[4 kb + i][v0 + 8 vb .. + 8)
};
__host__ __device__ inline int w2_blocks(int rank) { return (rank >> 2) * 8; }
// block s: kb = s / 8, vb = s % 8; a block past V reads entries V-8 .. V-1
// instead (any valid address: rows past V start at -inf, so their bias is
// never used).  V % 8 == 0 keeps a block wholly inside or outside the row.
__device__ inline void w2_block_load(const uint16_t* __restrict__ W2, int V, int v0, int s,
                                     W2Block& blk) {
  const int kb = s >> 3, vb = s & 7;
  const int v = min(v0 + 8 * vb, V - 8);
  const uint16_t* p = W2 + (size_t)(4 * kb) * V + v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    blk.r[i] = *reinterpret_cast<const u32x4_t*>(p + (size_t)i * V);
}
__device__ inline void w2_block_store(const W2Block& blk, int s, char* lds, int nq) {
  const int kb = s >> 3, vb = s & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = j >> 1;
    uint32_t lo, hi;   // (k0, k1) and (k2, k3) of entry 8 vb + j
    if (j & 1) {
      lo = (blk.r[0][m] >> 16) | (blk.r[1][m] & 0xFFFF0000u);
      hi = (blk.r[2][m] >> 16) | (blk.r[3][m] & 0xFFFF0000u);
    } else {
      lo = (blk.r[0][m] & 0xFFFFu) | (blk.r[1][m] << 16);
      hi = (blk.r[2][m] & 0xFFFFu) | (blk.r[3][m] << 16);
    }
    const int r = tile_vocab_row(8 * vb + j);
    *reinterpret_cast<u32x2_t*>(lds + r * lds_row_bytes(nq) + kb * 8) = u32x2_t{lo, hi};
  }
}

// The padded k-contiguous LDS image of W2 tile v0 (see above), written by
// every thread of the work-group (loads, then LDS stores).  Completion:
// barrier by the caller.
__device__ inline void stage_tile(const uint16_t* __restrict__ W2, int v0, int V, int rank,
                                  char* lds) {
  const int nq = rank >> 3, nb = w2_blocks(rank);
  for (int s = threadIdx.x; s < nb; s += blockDim.x) {
    W2Block blk;
    w2_block_load(W2, V, v0, s, blk);
    w2_block_store(blk, s, lds, nq);
  }
}

// Raw W2 rows of ONE tile in LDS, for the single-tile recomputes of the
// samplers: k-row k (the tile's 64 entries, 128 bytes) at byte
// raw_off(k) = 128 k + 16 (k / 8).  The rows arrive by DMA, eight per
// instruction (each 1 KB run followed by a 16-byte gap, so that rows k and
// k + 8, read together by the two half-waves, fall on different banks); the
// matrix operand is then gathered from them 16 bits at a time.
constexpr int kRawTileBytes = kMaxKSteps * 16 * 128 + kMaxKSteps * 2 * 16;   // rank 256
__host__ __device__ inline int raw_off(int k) { return 128 * k + 16 * (k >> 3); }
// DMA of tile v0's rows (rank multiple of 8); every wave of the group takes
// part.  Completion: s_waitcnt + barrier by the caller.
__device__ inline void dma_tile_raw(const uint16_t* __restrict__ W2, int V, int v0, int rank,
                                    char* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int g = wave; g < rank / 8; g += nwaves) {   // rows 8g .. 8g + 7
    const int s = g * 64 + lane;
    const int k = s >> 3, pc = s & 7;
    const int v = min(v0 + 8 * pc, V - 8);           // pieces past V: any valid address
    __builtin_amdgcn_global_load_lds(W2 + (size_t)k * V + v, lds + g * (1024 + 16), 16, 0, 0);
  }
}
// This lane's A operand of sub-tile t, k-step ks, from the raw rows: the
// 8 consecutive k of entry 32 t + sub_row_vocab(c) (the values the tile
// images hold, bit for bit).
__device__ inline bf16x8_t raw_frag(const char* lds, int t, int ks) {
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const int k0 = 16 * ks + 8 * h;
  const char* base = lds + raw_off(k0) + 2 * (32 * t + sub_row_vocab(c));
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = *reinterpret_cast<const uint16_t*>(base + 256 * i);
    const uint32_t hi = *reinterpret_cast<const uint16_t*>(base + 256 * i + 128);
    w[i] = lo | (hi << 16);
  }
  return __builtin_bit_cast(bf16x8_t, w);
}

// Gathered rows: LDS row r <- src row ids[r] (ids in LDS or memory).
__device__ inline void stage_gather(const uint16_t* __restrict__ src, const int* ids, int rank,
                                    char* lds, int nrows) {
  stage_rows_lds(src, rank, lds, nrows, [&](int r) { return ids[r]; });
}

// DMA nchunks consecutive 16-byte chunks from src (16-byte aligned) to
// lds; every wave of the work-group takes part.  kCoherent reads at device
// scope (data written by other work-groups of the running kernel).
// Completion: s_waitcnt + barrier by the caller.
template <bool kCoherent>
__device__ inline void dma_copy(const void* src, char* lds, int nchunks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const char* s = static_cast<const char*>(src);
  for (int g = wave; g * 64 < nchunks; g += nwaves) {
    const int ch = g * 64 + lane;
    if (ch < nchunks)
      __builtin_amdgcn_global_load_lds(s + (size_t)ch * 16, lds + (size_t)(g * 64) * 16, 16, 0,
                                       kCoherent ? 16 : 0);
  }
}

__device__ inline bf16x8_t lds_frag(const char* lds, int r, int q, int nq) {
  return *reinterpret_cast<const bf16x8_t*>(lds + lds_off(r, q, nq));
}

// Markov bias of one block-tile with the W2 tile (A) read from its LDS image and the
// request operand (B) given per k-step by `bfrag`, accumulated onto acc:
//   acc[t][j] += sum_k W2[k][v0 + 32t + 16h + j] * Wrow_c[k]
// (k-steps in ascending order) where Wrow_c is the W1 row fed by the lanes
// of column c.  The callers start acc at the base logits (init_acc), so the
// result is the biased logit itself.  Each output element depends only on
// its own A row, its own B column, its own start value and the fixed k-step
// order, so feeding zeros to the other columns recomputes one request's
// values bit for bit.  All 64 lanes must call it.
template <int KS, typename BF>
__device__ inline void bias_tile_ldsA(BF&& bfrag, const char* ldsA, f32x16_t acc[kSub]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  constexpr int nq = 2 * KS;
  bf16x8_t acur[kSub], anext[kSub];
#pragma unroll
  for (int t = 0; t < kSub; ++t) acur[t] = lds_frag(ldsA, 32 * t + c, h, nq);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) {
#pragma unroll
      for (int t = 0; t < kSub; ++t) anext[t] = lds_frag(ldsA, 32 * t + c, 2 * (ks + 1) + h, nq);
    }
    const bf16x8_t bv = bfrag(ks);
#pragma unroll
    for (int t = 0; t < kSub; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[t], bv, acc[t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kSub; ++t) acur[t] = anext[t];
  }
}

// Sub-tile t alone of the same contraction (the identical instruction chain
// that bias_tile_ldsA runs for acc[t]).
template <int KS, typename BF>
__device__ inline void bias_subtile_ldsA(BF&& bfrag, const char* ldsA, int t, f32x16_t& acc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  constexpr int nq = 2 * KS;
  bf16x8_t acur = lds_frag(ldsA, 32 * t + c, h, nq), anext;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) anext = lds_frag(ldsA, 32 * t + c, 2 * (ks + 1) + h, nq);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur, bfrag(ks), acc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    acur = anext;
  }
}

// Sub-tile t of the contraction with both operands given per k-step (the
// instruction chain bias_subtile_ldsA runs; any source of the same operand
// values gives the same result bit for bit).
template <int KS, typename AF, typename BF>
__device__ inline void bias_subtile(AF&& afrag, BF&& bfrag, f32x16_t& acc) {
  bf16x8_t acur = afrag(0), anext;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) anext = afrag(ks + 1);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur, bfrag(ks), acc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    acur = anext;
  }
}

// The same contraction with the W2 tile operands held in registers (see
// wreg_from_lds).
template <int KS, typename BF>
__device__ inline void bias_tile_regA(BF&& bfrag, const bf16x8_t (&wreg)[KS][kSub],
                                      f32x16_t acc[kSub]) {
  bf16x8_t bcur = bfrag(0), bnext;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) bnext = bfrag(ks + 1);
#pragma unroll
    for (int t = 0; t < kSub; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[ks][t], bcur, acc[t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep later operand reads from being hoisted
    bcur = bnext;
  }
}

// This lane's A operand of a tile for every k-step, read from the tile's
// LDS image (stage_tile): the operands bias_tile_ldsA reads, bit for bit.
template <int KS>
__device__ inline void wreg_from_lds(const char* img, bf16x8_t (&wreg)[KS][kSub]) {
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wreg[ks][t] = lds_frag(img, 32 * t + c, 2 * ks + h, 2 * KS);
  }
}

// this lane's B operand (the W1 row of token `tok`, or zeros for tok < 0)
// for all k-steps, straight from global memory
template <int KS>
__device__ inline void load_bfrag(const uint16_t* __restrict__ W1, int tok, bf16x8_t bfrag[KS]) {
  const int h = (threadIdx.x & 63) >> 5;
  const bf16x8_t zero = bf16x8_t{};
  const uint16_t* row = W1 + (size_t)(tok >= 0 ? tok : 0) * (16 * KS) + 8 * h;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bfrag[ks] = load_bf16x8(row + 16 * ks);
    bfrag[ks] = tok >= 0 ? bfrag[ks] : zero;
  }
}

// fp32 inputs: plain FMA dot products (k ascending) in the same layout,
// accumulated onto acc.  `tok` is the W1 row of this lane's request column
// (-1 = nothing added).  W2 is [rank, V]: per k the lane's 16 consecutive
// entries are four 16-byte loads of row k; the 16 entries' chains advance
// together (each k ascending, one fma per k).
__device__ inline void bias_tile_f32(const float* __restrict__ W1, int tok,
                                     const float* __restrict__ W2, int v0, int V, int rank,
                                     f32x16_t acc[kSub]) {
  if (tok < 0) return;
  const int h = (threadIdx.x & 63) >> 5;
  const float* arow = W1 + (size_t)tok * rank;
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
    const int vb = v0 + 32 * t + 16 * h;
    // column of each group of 4 entries; groups past V read column 0 (V % 4
    // == 0 keeps a group wholly inside or outside): computed, not kept
    int col[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) col[q] = vb + 4 * q < V ? vb + 4 * q : 0;
    float s[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = acc[t][j];
    for (int i = 0; i < rank; i += 4) {
      const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(arow + i);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float* row = W2 + (size_t)(i + kk) * V;
        const float ak = a4[kk];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(row + col[q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * q + e] = fmaf(ak, b4[e], s[4 * q + e]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (vb + j < V) acc[t][j] = s[j];
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
