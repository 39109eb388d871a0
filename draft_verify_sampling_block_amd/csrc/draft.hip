// dspark_draft_block kernels: sequential Markov-head sampling over a block.
//
// [billytse] 3.2-3.3: position k's distribution is softmax(U_k + W1[prev] W2)
// where prev is the token sampled at position k-1 (the anchor for k = 0);
// positions are sampled left to right.  [weigao] part 2: rank-r factors.
//
// Two implementations with identical results:
//
//  * persistent (bf16, rank <= 256, one work-group per compute unit, launched
//    cooperatively so all work-groups are resident): each work-group owns a
//    fixed set of 64-entry vocabulary tiles for the whole block; the W2
//    rows of those tiles stay resident (8 tiles in registers, one per wave,
//    the rest in LDS) across all gamma positions, so W2 is read from memory
//    once per call.  Per position: gather the W1 rows of the previous
//    tokens into LDS, compute every (tile, 32-request block) on the matrix
//    cores with the streamed base logits, publish per-tile statistics, then
//    the work-group that owns request b draws token b as soon as every
//    work-group has published (flags in memory, bounded spins), and
//    publishes it for the next position.
//
//  * multi-launch (any dtype / fallback): per position one
//    vocabulary-parallel launch (draft_stats_kernel) and one request-parallel
//    launch (draft_sample_kernel) doing the same two steps.
#include <atomic>
#include <type_traits>

#include "dspark_common.hpp"
#include "draft_tile.hpp"
#include "dspark_launch.hpp"
#include "trace.hpp"

namespace dspark {

template <typename T>
constexpr bool kIsBf16 = std::is_same<T, uint16_t>::value;

// Shared-memory state of the per-request sampler (block-wide).
struct SampShared {
  double red[8];
  double before, scale;
  int tile;
  float se[kTileV];
  __attribute__((aligned(16))) char arow[kMaxKSteps * 32];  // W1 row of the request (bf16)
  __attribute__((aligned(16))) char useg[kTileV * 4];        // base logits of the crossing tile
};
// LDS the sampler needs besides SampShared: the crossing tile's W2 rows,
// then a copy of the request's tile statistics
constexpr int kSampScratchBytes = kLdsTileBytes + 2 * kMaxTiles * 4;

// Draw draft token k of request b from the tile statistics (all threads of
// the work-group call this).  `scratch` is kSampScratchBytes of LDS.
// Writes tokens (device-coherent store) and q_tok/row_max/row_logZ.
template <typename T, int KS, int NTHR>
__device__ void sample_request(int b, int k, int B, int gamma, int V, int rank, int prev,
                               const T* __restrict__ U, const T* __restrict__ W1,
                               const T* __restrict__ W2, const float* __restrict__ temperature,
                               const float* __restrict__ uniforms, const TileStats& ts,
                               int32_t* tokens, float* q_tok, float* row_max, float* row_logZ,
                               int32_t* status, char* scratch, SampShared& sh,
                               uint32_t* tok_flag) {
  static_assert(NTHR >= 256, "the statistics loads assume >= 256 threads");
  // thread 0: the token, published first (flag word (k + 1) << 24 | token
  // when tok_flag is given, so that waiting work-groups read it with the
  // flag itself), then the other outputs
  auto emit = [&](int tok, float q, float rmax, float rlz) {
    if (tok_flag) st_dev(tok_flag + b, ((uint32_t)(k + 1) << 24) | (uint32_t)tok);
    tokens[(size_t)b * gamma + k] = tok;
    q_tok[(size_t)b * gamma + k] = q;
    row_max[(size_t)b * gamma + k] = rmax;
    row_logZ[(size_t)b * gamma + k] = rlz;
  };
  const int tid = threadIdx.x, nthr = NTHR;
  const int nT = n_tiles(V);
  // the request's packed tile statistics, copied to LDS (device-coherent
  // reads); the row starts `shift` entries into the copy when it is not
  // 16-byte aligned
  const uint64_t* cms;
  {
    const size_t first = (size_t)b * nT;
    const int shift = (int)(first & 1);
    cms = reinterpret_cast<const uint64_t*>(scratch + kLdsTileBytes) + shift;
    dma_copy<true>(ts.ms + (first - shift), scratch + kLdsTileBytes, (nT + shift + 1) / 2);
  }
  auto cm = [&](int t) { return ms_max(cms[t]); };
  auto cs = [&](int t) { return ms_sum(cms[t]); };
  const float Tb = temperature[b];
  const double u = (double)uniforms[((size_t)b * (gamma + 1) + k) * 2 + 0];
  const bool greedy = !(Tb > 0.f);
  const size_t out = (size_t)b * gamma + k;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  float m = -INFINITY;
  for (int t = tid; t < nT; t += nthr) m = fmaxf(m, cm(t));
  m = block_max(m, sh.red);

  if (greedy) {
    int a = 0x7fffffff;
    for (int t = tid; t < nT; t += nthr)
      if (cm(t) == m) a = min(a, ld_dev(ts.arg + (size_t)b * nT + t));
    a = block_min_int(a, sh.red);
    if (tid == 0) {
      if (!(m == m) || a < 0 || a >= V) {  // NaN logits leave no argmax
        flag(status, DSPARK_DEV_NONFINITE);
        a = 0;
      }
      emit(a, 1.f, m, 0.f);
    }
    __syncthreads();
    return;
  }

  // mass of tile t relative to the row max: cs[t] * 2^((cm[t] - m) ce),
  // factor in fp32, accumulation in fp64 over each thread's contiguous range
  const float scale = 1.f / Tb;
  const float ce = scale * kLog2e;
  const int per = (nT + nthr - 1) / nthr;
  const int c0 = min(nT, tid * per), c1 = min(nT, c0 + per);
  double local = 0.0;
  for (int t = c0; t < c1; ++t)
    local += (double)cs(t) * (double)__builtin_amdgcn_exp2f((cm(t) - m) * ce);
  double start, end;
  const double Z = block_scan_interval(local, sh.red, &start, &end);
  // u * Z can round up to Z: the target is kept below Z, so exactly one
  // thread's interval [start, end) holds it (the intervals tile [0, Z))
  double target = u * Z;
  if (!(target < Z)) target = nextafter(Z, 0.0);
  const bool finite = isfinite(m) && isfinite(Z) && Z > 0.0;

  if (tid == 0) sh.tile = -1;
  __syncthreads();
  if (finite && local > 0.0 && start <= target && target < end) {
    double run = start, before = start, lastb = start;
    int found = -1, lastt = -1;
    for (int t = c0; t < c1; ++t) {
      const double st = (double)cs(t) * (double)__builtin_amdgcn_exp2f((cm(t) - m) * ce);
      if (st > 0.0) { lastt = t; lastb = run; }
      if (st > 0.0 && target < run + st) { found = t; before = run; break; }
      run += st;
    }
    if (found < 0) { found = lastt; before = lastb; }
    sh.tile = found;
    sh.before = before;
    sh.scale = (double)__builtin_amdgcn_exp2f((cm(found) - m) * ce);
  }
  __syncthreads();
  const int vt = sh.tile;
  const float ms = m * scale;    // row max of the scaled logits
  if (!finite || vt < 0) {
    if (tid == 0) {
      flag(status, DSPARK_DEV_NONFINITE);
      emit(0, 0.f, ms, __logf((float)Z));
    }
    __syncthreads();
    return;
  }
  const float mc = cm(vt) * ce;
  __syncthreads();   // the statistics copy is dead from here: the tile rows may land

  // recompute the crossing tile exactly as the statistics pass did: same
  // operands, request b in its own column b % 32, one sub-tile at a time
  const int v0 = vt * kTileV;
  const int mrow = b % kTileM;
  const int lane = tid & 63, c = lane & 31, h = lane >> 5;
  const bool mine = tid < kWave && c == mrow;
  const int rem = V - (v0 + 16 * h);   // usable entries: j < rem - 32t
  if constexpr (kIsBf16<T>) {
    // the request's W1 row and base logits of the tile by DMA, the tile's
    // transposed W2 image by every thread; waves 0 and 1 then recompute
    // sub-tiles 0 and 1
    dma_copy<false>(W1 + (size_t)prev * rank, sh.arow, rank / 8);
    dma_copy<false>(U + out * V + v0, sh.useg, min(kTileV, V - v0) / 8);
    stage_tile(W2, v0, V, rank, scratch);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid < kSub * kWave) {
      const int t = tid >> 6;
      const bool own = c == mrow;
      const uint16_t* useg = reinterpret_cast<const uint16_t*>(sh.useg) + 32 * t + 16 * h;
      const bf16x8_t zero = bf16x8_t{};
      auto bfrag = [&](int ks) {
        const bf16x8_t f = *reinterpret_cast<const bf16x8_t*>(sh.arow + 16 * (2 * ks + h));
        return own ? f : zero;
      };
      f32x16_t acc;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = (32 * t + j < rem) ? bf16_to_f32(useg[j]) : -INFINITY;
      bias_subtile_ldsA<KS>(bfrag, scratch, t, acc);
      if (own) {
        float* se = sh.se + 32 * t + 16 * h;
#pragma unroll
        for (int j = 0; j < 16; ++j) se[j] = tile_term(acc[j], ce, mc);
      }
    }
  } else {
    URow<T> ur;
    load_urow<T>(ur, U + out * V, v0, V, mine, U);
    if (tid < kWave) {
      f32x16_t acc[kSub];
      init_acc<T>(ur, rem, acc);
      bias_tile_f32(reinterpret_cast<const float*>(W1), mine ? prev : -1,
                    reinterpret_cast<const float*>(W2), v0, V, rank, acc);
      if (mine) {
#pragma unroll
        for (int t = 0; t < kSub; ++t) {
          float* se = sh.se + 32 * t + 16 * h;
#pragma unroll
          for (int j = 0; j < 16; ++j) se[j] = tile_term(acc[t][j], ce, mc);
        }
      }
    }
  }
  __syncthreads();
  // inverse CDF inside the tile on wave 0: lane i holds entry i; prefix
  // sums over the wave, the first entry whose running mass exceeds r wins
  // (the last positive one if rounding leaves r past the total)
  if (tid < kWave) {
    const double r = (target - sh.before) / sh.scale;
    const double e = (double)sh.se[tid];
    double incl = e;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double n = __shfl_up(incl, o, kWave);
      if (tid >= o) incl += n;
    }
    const unsigned long long hit = __ballot(e > 0.0 && r < incl);
    const unsigned long long pos = __ballot(e > 0.0);
    const int pick = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
    if (tid == 0)
      emit(v0 + pick, (float)((double)sh.se[pick] * sh.scale / Z), ms, __logf((float)Z));
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Multi-launch path
// ---------------------------------------------------------------------------

// The bias row of request b: row prev_src[b * prev_stride] of W1 (the Markov
// head: the previous token's embedding), or with emb_k >= 0 row
// b * gamma + emb_k of the table passed as W1 (the RNN head's projected
// vectors emb [B, gamma, rank]).
template <typename T, int KS>
__global__ __launch_bounds__(256) void draft_stats_kernel(
    int B, int gamma, int V, int rank, int k, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2, const int32_t* __restrict__ prev_src, int prev_stride, int emb_k,
    const float* __restrict__ temperature, TileStats ts, int32_t* status) {
  __shared__ __attribute__((aligned(16))) char w2s[kIsBf16<T> ? kLdsTileBytes : 16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nRB = (B + kTileM - 1) / kTileM;
  const int nT = n_tiles(V);
  const int vt = blockIdx.x, v0 = vt * kTileV;

  if constexpr (kIsBf16<T>) stage_tile(W2, v0, V, rank, w2s);
  int rb = wave;
  bf16x8_t bfrag[KS];
  URow<T> ur;
  int tok = -1;
  float it = 0.f;
  auto setup = [&](int blk) {
    const int b = blk * kTileM + c;
    tok = -1;
    it = 0.f;
    if (b < B) {
      tok = emb_k >= 0 ? b * gamma + emb_k
                       : clamp_token(prev_src[(size_t)b * prev_stride], V, h == 0 ? status : nullptr);
      it = inv_temp(temperature[b]);
    }
    if constexpr (kIsBf16<T>) load_bfrag<KS>(W1, tok, bfrag);
    load_urow<T>(ur, U + ((size_t)b * gamma + k) * V, v0, V, b < B, U);
  };
  if (rb < nRB) setup(rb);
  if constexpr (kIsBf16<T>) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int rem = V - (v0 + 16 * h);
  while (rb < nRB) {
    f32x16_t acc[kSub];
    init_acc<T>(ur, rem, acc);
    if constexpr (kIsBf16<T>)
      bias_tile_ldsA<KS>([&](int ks) { return bfrag[ks]; }, w2s, acc);
    else
      bias_tile_f32(reinterpret_cast<const float*>(W1), tok, reinterpret_cast<const float*>(W2),
                    v0, V, rank, acc);
    const int b = rb * kTileM + c;
    const bool any_greedy = __ballot((b < B) && !(it > 0.f)) != 0;
    const TileStat st = tile_reduce(acc, vt, it, any_greedy);
    if (b < B && h == 0) store_tile_stat(ts, b, nT, vt, st, it);
    rb += 4;
    if (rb < nRB) setup(rb);
  }
}

template <typename T, int KS>
__global__ __launch_bounds__(256) void draft_sample_kernel(
    int B, int gamma, int V, int rank, int k, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2, const int32_t* __restrict__ prev_src, int prev_stride, int emb_k,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, TileStats ts,
    int32_t* __restrict__ tokens, float* __restrict__ q_tok, float* __restrict__ row_max,
    float* __restrict__ row_logZ, int32_t* status) {
  __shared__ __attribute__((aligned(16))) char scratch[kSampScratchBytes];
  __shared__ SampShared sh;
  const int b = blockIdx.x;
  const int prev = emb_k >= 0 ? b * gamma + emb_k
                              : clamp_token(prev_src[(size_t)b * prev_stride], V, nullptr);
  sample_request<T, KS, 256>(b, k, B, gamma, V, rank, prev, U, W1, W2, temperature, uniforms,
                             ts, tokens, q_tok, row_max, row_logZ, status, scratch, sh, nullptr);
}

// ---------------------------------------------------------------------------
// Persistent path (bf16)
// ---------------------------------------------------------------------------

constexpr int kPdRegTiles = 8;              // resident tiles in registers per group
constexpr int kPdLdsTiles = 2;              // extra resident tiles in LDS
constexpr int kPdMaxRows = 128;             // W1 rows gathered per chunk
constexpr int kPdFlagStride = 32;           // 128-byte spacing of per-group flags
constexpr int kPdMaxGroups = 4096;
constexpr int kPdRowBytes = kPdMaxRows * (2 * kMaxKSteps + 1) * 16;   // 66 KB (padded rows)
static_assert(kPdRowBytes >= kSampScratchBytes, "the sampler reuses the W1 row area");

struct PdArgs {
  int B, gamma, V, rank, P;
  const uint16_t* U;
  const uint16_t* W1;
  const uint16_t* W2;
  const int32_t* anchor;
  const float* temperature;
  const float* uniforms;
  int32_t* tokens;
  float* q_tok;
  float* row_max;
  float* row_logZ;
  int32_t* status;
  TileStats ts;
  uint32_t* stats_flag;  // [P * kPdFlagStride]: positions whose statistics group p published
  uint32_t* tok_flag;    // [B]: ((k + 1) << 24) | token k of request b, once drawn
  long long spin_cap;    // wall-clock ticks a wait may last
};

// Flag protocol between the work-groups of the running kernel.  Data and
// flags are device-scope (agent) relaxed atomics: each access is coherent
// across the chip's L2 slices.  A producer waits for its data stores to
// complete (s_waitcnt, every wave, then a work-group barrier) before thread 0
// stores the flag; a consumer issues its data loads only after it has seen
// the flag.  The hardware waits give the ordering; compiler-only fences on
// both sides keep the compiler from moving the data accesses across the flag
// access.  (Agent-scope release/acquire would add a whole-L2 write-back or
// invalidate per hop, which measured tens of microseconds per position.)
__device__ inline uint32_t ld_flag(const uint32_t* p) { return ld_dev(p); }
__device__ inline void st_flag(uint32_t* p, uint32_t v) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  st_dev(p, v);
}

// Wave 0 waits until flags[i*stride] >= want for all i < n; then the group
// synchronises.  With `low` given (n <= kPdMaxRows), the low 24 bits of each
// flag as finally read are left in low[i].  The wait is bounded: past
// `cap_ticks` of the device wall clock it raises DSPARK_DEV_TIMEOUT and gives
// up, and any group that sees that flag already raised gives up at once, so a
// kernel whose groups cannot all make progress still drains.  All threads of
// the work-group call it.
__device__ inline void wait_flags(const uint32_t* flags, int n, int stride, uint32_t want,
                                  long long cap_ticks, int32_t* status, int* low = nullptr) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const long long t0 = wall_clock64();
    for (int it = 0;; ++it) {
      bool ok = true;
      for (int i = lane; i < n; i += kWave) {
        const uint32_t v = ld_flag(flags + (size_t)i * stride);
        ok &= v >= want;
        if (low) low[i] = (int)(v & 0xFFFFFFu);
      }
      if (__all(ok)) break;
      if ((it & 15) == 15) {
        const bool late = wall_clock64() - t0 > cap_ticks;
        const bool gave_up = status && (ld_dev(status) & DSPARK_DEV_TIMEOUT);
        if (late || gave_up) {
          if (late && lane == 0) flag(status, DSPARK_DEV_TIMEOUT);
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // data loads stay after the flags
}

// Every wave waits for its own stores to complete, then the group
// synchronises; thread 0 may then raise a flag.
__device__ inline void stores_done_group() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// NW waves per group; each wave holds R = kPdRegTiles / NW W2 tiles in
// registers (NW = 8: two waves per SIMD, 128 registers of tile each at rank
// 256; NW = 4: one wave per SIMD with two tiles, the tiles and the
// accumulators split over the architectural and accumulation registers).
// PF: the groups that draw no token warm the caches with the next
// position's base logits while the owners draw.
template <int KS, int NW, bool PF>
__global__ __launch_bounds__(NW * 64, 1) void pdraft_kernel(PdArgs a) {
  constexpr int nq = 2 * KS;
  constexpr int R = kPdRegTiles / NW;
  __shared__ __attribute__((aligned(16))) char ldsL[kPdLdsTiles * kLdsTileBytes];
  __shared__ __attribute__((aligned(16))) char ldsA[kPdRowBytes];
  __shared__ int s_tok[kPdMaxRows];
  __shared__ float s_it[kPdMaxRows];   // inverse temperatures of the chunk
  // statistics of the chunk's block-tasks, per resident tile slot (register
  // tile i of wave w: slot w + NW i; LDS tile i: slot kPdRegTiles + i) and
  // chunk row; written to memory once the chunk is done
  constexpr int kSlots = kPdRegTiles + kPdLdsTiles;
  __shared__ float s_mx[kSlots][kPdMaxRows], s_sum[kSlots][kPdMaxRows];
  __shared__ int s_arg[kSlots][kPdMaxRows];
  __shared__ SampShared sh;
  // sink of the cache-warming loads (never read)
  __shared__ uint32_t s_pf[1];

  const int p = blockIdx.x, P = a.P;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int B = a.B, V = a.V, gamma = a.gamma;
  const int nT = n_tiles(V);

  // Resident W2 tiles: group p owns the contiguous tiles [tbase, tbase +
  // tcount) (the first nT % P groups one more), so that its statistics of a
  // request form one contiguous run.  Tile slot s is tile tbase + s:
  // register tile i of wave w is slot w + NW i, LDS tile i slot
  // kPdRegTiles + i; slots >= tcount are empty.
  const int tcount = nT / P + (p < nT % P ? 1 : 0);
  const int tbase = p * (nT / P) + min(p, nT % P);
  auto slot_tile = [&](int slot) { return slot < tcount ? tbase + slot : nT; };  // nT: none
  // W2 is [rank, V]: every resident tile passes through its transposed LDS
  // image.  The blocks of the eight register tiles are loaded in one shot;
  // they pass four at a time through the four image areas (the two LDS tile
  // areas and the W1 row area), the LDS tiles' blocks loading while the
  // first four images are read; then the LDS tiles are staged in place.
  // Blocks of slots without a tile load (clamped, in-bounds) addresses and
  // are never stored.
  static_assert(kPdRowBytes >= 2 * kLdsTileBytes && kPdRegTiles == 8 && kPdLdsTiles == 2,
                "four tile images at a time");
  auto img = [&](int j) {   // image area j of 4
    return j < 2 ? ldsL + j * kLdsTileBytes : ldsA + (j - 2) * kLdsTileBytes;
  };
  const int nbk = w2_blocks(a.rank);
  const int nthr = NW * 64;
  // block threadIdx.x + nthr q of slot s, for every q with a block there
  constexpr int kQ = (32 * KS + NW * 64 - 1) / (NW * 64);   // blocks per slot (rank 16 KS)
  auto load_slot = [&](int sl, W2Block (&bk)[kQ]) {
    const int tl = min(slot_tile(sl), nT - 1);
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      w2_block_load(a.W2, V, tl * kTileV, min((int)threadIdx.x + nthr * q, nbk - 1), bk[q]);
  };
  auto store_slot = [&](int sl, const W2Block (&bk)[kQ], char* dst) {
    if (slot_tile(sl) < nT) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int sb = (int)threadIdx.x + nthr * q;
        if (sb < nbk) w2_block_store(bk[q], sb, dst, 2 * KS);
      }
    }
  };
  auto read_round = [&](int s0, bf16x8_t (&wr)[R][KS][kSub]) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int sl = wave + NW * i;
      if (sl >= s0 && sl < s0 + 4) wreg_from_lds<KS>(img(sl - s0), wr[i]);
    }
  };
  bf16x8_t wreg[R][KS][kSub];
  {
    W2Block blk[kPdRegTiles][kQ];
#pragma unroll
    for (int j = 0; j < kPdRegTiles; ++j) load_slot(j, blk[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) store_slot(j, blk[j], img(j));
    __syncthreads();
    W2Block lblk[kPdLdsTiles][kQ];
#pragma unroll
    for (int j = 0; j < kPdLdsTiles; ++j) load_slot(kPdRegTiles + j, lblk[j]);
    read_round(0, wreg);
    __syncthreads();
#pragma unroll
    for (int j = 4; j < 8; ++j) store_slot(j, blk[j], img(j - 4));
    __syncthreads();
    read_round(4, wreg);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPdLdsTiles; ++j) store_slot(kPdRegTiles + j, lblk[j], img(j));
  }
  int nL = 0;
  for (int i = 0; i < kPdLdsTiles; ++i) nL += slot_tile(kPdRegTiles + i) < nT ? 1 : 0;
  __syncthreads();

  // Block-tasks of this wave for one position, in order: per chunk of up to
  // kPdMaxRows requests, its register tiles x every block of the chunk, then
  // its round-robin share (from `start`, step NW) of the (LDS tile, block)
  // pairs.  Register tiles of a wave that lie inside the vocabulary form a
  // prefix i < nreg; R <= 2 and kPdLdsTiles == 2 keep the index maths free
  // of divisions.
  static_assert(R <= 2 && kPdLdsTiles == 2, "task indexing assumes at most two of each");
  const int nch = (B + kPdMaxRows - 1) / kPdMaxRows;
  int nreg = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) nreg += (slot_tile(wave + NW * i) < nT) ? 1 : 0;
  auto chunk_blocks = [&](int ch) {
    return (min(kPdMaxRows, B - ch * kPdMaxRows) + kTileM - 1) / kTileM;
  };
  auto chunk_tasks = [&](int ch, int start) {
    const int nblk = chunk_blocks(ch);
    const int nlds = nL * nblk;
    return nreg * nblk + (start < nlds ? (nlds - start + NW - 1) / NW : 0);
  };
  // A ring of D prefetched tasks: base logits (they do not depend on the
  // drafted tokens, so the first ones of a position are requested before
  // its tokens are known) and the task's tile / block / W2 location
  // (which: -1 - i = register tile i, >= 0 = LDS tile).  One slot ahead is
  // enough at two waves per SIMD; one wave per SIMD keeps two.
  constexpr int D = NW >= 8 ? 1 : 2;
  struct Slot {
    URow<uint16_t> u;
    int tile, rb, which;
  };
  Slot ring[D];
  int fch = 0, fidx = 0;   // next task to fetch: chunk, index in the chunk
  // tile / request block / A source of task fi of chunk ch
  auto task_at = [&](int ch, int fi, int start, int& tile, int& rb, int& which) {
    const int nblk = chunk_blocks(ch);
    const int rbase = ch * (kPdMaxRows / kTileM);
    if (fi < nreg * nblk) {
      const int i = (R == 2 && fi >= nblk) ? 1 : 0;
      rb = rbase + fi - i * nblk;
      tile = slot_tile(wave + NW * i);
      which = -1 - i;
    } else {
      const int li = start + (fi - nreg * nblk) * NW;
      const int w = li >= nblk ? 1 : 0;
      rb = rbase + li - w * nblk;
      tile = slot_tile(kPdRegTiles + w);
      which = w;
    }
  };
  // Past the last task the slot still issues its loads (of a safe
  // address): a fixed count of loads per task lets the in-order memory
  // counter wait for exactly the slot it needs, not for every later one.
  auto fetch_next = [&](Slot& sl, int start, int k) {
    if (fch >= nch) {
#pragma unroll
      for (int t = 0; t < kSub; ++t) {
#pragma unroll
        for (int q = 0; q < URow<uint16_t>::kLoads; ++q)   // four distinct 16-byte words
          sl.u.w[t][q] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(a.W2) + t * URow<uint16_t>::kLoads + q);
      }
      return;
    }
    task_at(fch, fidx, start, sl.tile, sl.rb, sl.which);
    const int b = sl.rb * kTileM + c;
    load_urow<uint16_t>(sl.u, a.U + ((size_t)b * gamma + k) * V, sl.tile * kTileV, V, b < B,
                        a.U);
    if (++fidx == chunk_tasks(fch, start)) {
      fidx = 0;
      ++fch;
      while (fch < nch && chunk_tasks(fch, start) == 0) ++fch;
    }
  };

  // put the first D tasks of position kk in flight
  auto prime = [&](int kk) {
    const int st = (wave + kk) % NW;
    fch = 0;
    fidx = 0;
    while (fch < nch && chunk_tasks(fch, st) == 0) ++fch;
#pragma unroll
    for (int d = 0; d < D; ++d) fetch_next(ring[d], st, kk);
  };

  for (int k = 0; k < gamma; ++k) {
    const int start = (wave + k) % NW;   // rotate who takes the LDS extras
    prime(k);
    // tokens of position k - 1: flag words (k << 24) | token; with one chunk
    // the wait leaves them in s_tok directly
    const bool tok_in_lds = k > 0 && nch == 1;
    if (k > 0)
      wait_flags(a.tok_flag, B, 1, (uint32_t)k << 24, a.spin_cap, a.status,
                 tok_in_lds ? s_tok : nullptr);

    // run the task in slot sl: start the accumulators at its base logits,
    // refill the slot with the task D ahead, add the bias, reduce
    auto run_task = [&](Slot& sl) {
      const int tile = sl.tile, rb = sl.rb, which = sl.which;
      const int b = rb * kTileM + c;
      const int v0 = tile * kTileV;
      const int lrow = (rb % (kPdMaxRows / kTileM)) * kTileM + c;   // row in the gathered chunk
      const float it = s_it[lrow];
      const bool any_greedy = __ballot((b < B) && !(it > 0.f)) != 0;
      auto bfrag = [&](int ks) { return lds_frag(ldsA, lrow, 2 * ks + h, nq); };
      // Each A source runs its own start / contraction / reduction, so the
      // accumulators of one never meet those of the other at a merge point
      // (which would cost register copies and a second accumulator set).
      auto finish = [&](f32x16_t (&acc)[kSub], int slot) {
        const TileStat st = tile_reduce(acc, tile, it, any_greedy);
        if (h == 0) {
          s_mx[slot][lrow] = st.mx;
          s_sum[slot][lrow] = st.s;
          s_arg[slot][lrow] = st.arg;
        }
      };
      // start the accumulators at the base logits, then refill the slot
      // (no global load after that: a later load would make the in-order
      // memory counter wait for the prefetch just issued)
      auto start_acc = [&](f32x16_t (&acc)[kSub]) {
        if (v0 + kTileV <= V) {
#pragma unroll
          for (int t = 0; t < kSub; ++t) {
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[t][j] = urow_at(sl.u, t, j);
          }
        } else {
          init_acc<uint16_t>(sl.u, V - (v0 + 16 * h), acc);
        }
        fetch_next(sl, start, k);
      };
      if (which >= 0) {
        f32x16_t acc[kSub];
        start_acc(acc);
        bias_tile_ldsA<KS>(bfrag, ldsL + which * kLdsTileBytes, acc);
        finish(acc, kPdRegTiles + which);
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (which == -1 - i) {
            f32x16_t acc[kSub];
            start_acc(acc);
            bias_tile_regA<KS>(bfrag, wreg[i], acc);
            finish(acc, wave + NW * i);
          }
        }
      }
    };
    // write the finished chunk's statistics (all waves done: caller synced)
    auto flush = [&](int chd) {
      const int r0 = chd * kPdMaxRows;
      const int nrows = min(kPdMaxRows, B - r0);
      for (int e = threadIdx.x; e < kSlots * kPdMaxRows; e += blockDim.x) {
        const int slot = e % kSlots, row = e / kSlots;
        const int tile = slot_tile(slot);
        if (row < nrows && tile < nT)
          store_tile_stat(a.ts, r0 + row, nT, tile,
                          TileStat{s_mx[slot][row], s_sum[slot][row], s_arg[slot][row]},
                          s_it[row]);
      }
    };

    // stage chunk ch: its previous tokens' W1 rows and inverse temperatures
    auto load_chunk = [&](int ch) {
      const int r0 = ch * kPdMaxRows;
      const int nrows = min(kPdMaxRows, B - r0);
      const int nblk = chunk_blocks(ch);
      for (int r = threadIdx.x; r < nblk * kTileM; r += blockDim.x) {
        int t = 0;
        float it = 0.f;
        if (r < nrows) {
          const int b = r0 + r;
          t = (k == 0) ? a.anchor[b]
                       : tok_in_lds ? s_tok[r] : (int)(ld_dev(a.tok_flag + b) & 0xFFFFFFu);
          t = clamp_token(t, V, k == 0 ? a.status : nullptr);
          it = inv_temp(a.temperature[b]);
        }
        s_tok[r] = t;
        s_it[r] = it;
      }
      __syncthreads();
      stage_gather(a.W1, s_tok, a.rank, ldsA, nblk * kTileM);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    // Every wave stages every chunk in order (the barriers match), switching
    // chunk whenever its next task lies in the following one.  The task loop
    // is unrolled by the ring depth so each slot stays in fixed registers
    // and its loads stay in flight until the slot's task runs.
    int ch = -1, chunk_end = 0, g = 0;
    auto enter = [&]() {
      while (g == chunk_end && ch + 1 < nch) {
        if (ch >= 0) {
          __syncthreads();  // chunk ch done: the row area and statistics are reused
          flush(ch);
        }
        ++ch;
        load_chunk(ch);
        chunk_end += chunk_tasks(ch, start);
      }
    };
    const int ntot = [&] {
      int n = 0;
      for (int cc = 0; cc < nch; ++cc) n += chunk_tasks(cc, start);
      return n;
    }();
    while (g < ntot) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (d > 0 && g >= ntot) break;
        enter();
        run_task(ring[d]);
        ++g;
      }
    }
    while (ch + 1 < nch) {   // chunks after this wave's last task
      if (ch >= 0) {
        __syncthreads();
        flush(ch);
      }
      ++ch;
      load_chunk(ch);
    }
    __syncthreads();  // the W1 row area is reused by the sampler
    flush(ch);
    // publish this group's statistics of position k
    stores_done_group();
    if (threadIdx.x == 0) st_flag(a.stats_flag + (size_t)p * kPdFlagStride, (uint32_t)(k + 1));

    // Groups that draw no token are idle until the tokens of position k
    // arrive: they touch the next position's base logits (one dword per
    // 32 bytes, DMA'd into LDS the group never reads) of their own tiles and
    // of an owner group's tiles, so those rows sit in the caches (the
    // Infinity Cache, and the L2 of the XCD both groups run on) when the
    // tasks of position k + 1 stream them.  Wave 0 keeps polling flags.
    if constexpr (PF) {
      const int nown = min(B, P);
      if (k + 1 < gamma && p >= nown && wave > 0) {
        const int other = p - nown;     // owner group covered by this one, if any
        const int nsl = (other < nown) ? 2 : 1;
        constexpr int kSeg = 16;        // bf16 entries per 32-byte segment
        auto slice = [&](int sl, int& v0, int& v1) {
          const int q = sl == 0 ? p : other;
          const int tc = nT / P + (q < nT % P ? 1 : 0);
          const int tb = q * (nT / P) + min(q, nT % P);
          v0 = tb * kTileV;
          v1 = min(V, (tb + tc) * kTileV);
        };
        int s0a, s0b, s1a = 0, s1b = 0;
        slice(0, s0a, s0b);
        if (nsl == 2) slice(1, s1a, s1b);
        const int n0 = (s0b - s0a + kSeg - 1) / kSeg, n1 = (s1b - s1a + kSeg - 1) / kSeg;
        const int per_req = n0 + n1;
        const int total = per_req * B;
        // eight loads in flight per lane per round; their XOR is kept only
        // so that the loads are issued (and the wave waits for them here,
        // while wave 0 is still polling)
        constexpr int kPfU = 8;
        uint32_t x = 0;
        for (int g0 = (wave - 1) * 64; g0 < total; g0 += (NW - 1) * 64 * kPfU) {
          uint32_t w[kPfU];
#pragma unroll
          for (int u = 0; u < kPfU; ++u) {
            const int g = min(g0 + u * (NW - 1) * 64 + lane, total - 1);
            const int b = g / per_req, j = g - b * per_req;
            const int v = j < n0 ? s0a + j * kSeg : s1a + (j - n0) * kSeg;
            w[u] = *reinterpret_cast<const uint32_t*>(a.U + ((size_t)b * gamma + k + 1) * V + v);
          }
#pragma unroll
          for (int u = 0; u < kPfU; ++u) x ^= w[u];
        }
        if (x == 0x7fc00001u) s_pf[0] = x;   // practically never true
      }
    }

    // draw the tokens of the requests this group owns
    bool waited = false;
    for (int b = p; b < B; b += P) {
      if (!waited) {
        wait_flags(a.stats_flag, P, kPdFlagStride, (uint32_t)(k + 1), a.spin_cap, a.status);
        waited = true;
      }
      const int prev = clamp_token(
          k == 0 ? a.anchor[b] : (int)(ld_dev(a.tok_flag + b) & 0xFFFFFFu), V, nullptr);
      sample_request<uint16_t, KS, NW * 64>(b, k, B, gamma, V, a.rank, prev, a.U, a.W1, a.W2,
                                            a.temperature, a.uniforms, a.ts, a.tokens, a.q_tok,
                                            a.row_max, a.row_logZ, a.status, ldsA, sh,
                                            a.tok_flag);
    }
  }
}

// zero the statistics flags [0, n0) and the token flags [0, n1)
__global__ void pdraft_reset_kernel(uint32_t* f0, int n0, uint32_t* f1, int n1) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n0) f0[i] = 0u;
  if (i < n1) f1[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {
// 0 auto, 1 multi-launch, 2-4 the earlier persistent kernel only (3: 8
// waves, 4: 4 waves), 5 the pipelined kernel only, 6 the same by a
// cooperative launch; process-wide, read by every call
std::atomic<int> g_draft_path{0};

struct DevInfo {
  int cus = 0;
  bool coop = false;
  int wall_khz = 100000;  // rate of the device wall clock read by wall_clock64()
};
DevInfo dev_info() {
  static thread_local int cached_dev = -1;
  static thread_local DevInfo info;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DevInfo{};
  if (dev != cached_dev) {
    info = DevInfo{};
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      info.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess)
      info.coop = v != 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) == hipSuccess && v > 0)
      info.wall_khz = v;
    cached_dev = dev;
  }
  return info;
}
}  // namespace

int set_draft_path(int path) { return g_draft_path.exchange(path); }
int device_cu_count() { return dev_info().cus; }
int get_draft_path() { return g_draft_path.load(); }

static size_t stats_bytes(int B, int V) { return align256((size_t)B * n_tiles(V) * 4); }

// The workspace: a header holding the pipelined kernel's start barrier (at
// the same place for every shape, zero-filled before the first call; nothing
// else writes there), the statistics and flags of the multi-launch and
// earlier persistent kernels (cleared by those paths), then the pipelined
// kernel's exchange words (zeroed by that kernel before use).
constexpr size_t kWsHeader = kDraftPipeHeaderBytes;
static size_t persistent_ws_bytes(int B, int V) {
  const size_t flags = align256((size_t)kPdMaxGroups * kPdFlagStride * 4) + align256((size_t)B * 4);
  return 3 * stats_bytes(B, V) + flags;
}

size_t draft_workspace_bytes(int B, int gamma, int V, int rank, int dtype) {
  (void)gamma; (void)rank; (void)dtype;
  return kWsHeader + persistent_ws_bytes(B, V) + draft_pipe_workspace_bytes(B, V);
}

static TileStats carve_stats(void* ws, int B, int V) {
  char* w = static_cast<char*>(ws) + kWsHeader;
  TileStats ts;
  ts.ms = reinterpret_cast<uint64_t*>(w);                          // 2 x stats_bytes
  ts.arg = reinterpret_cast<int32_t*>(w + 2 * stats_bytes(B, V));
  return ts;
}

template <typename T, int KS>
static hipError_t draft_multi(int B, int gamma, int V, int rank, const T* U, const T* W1,
                              const T* W2, const int32_t* anchor, const float* temperature,
                              const float* uniforms, int32_t* tokens, float* q_tok,
                              float* row_max, float* row_logZ, int32_t* status, void* ws,
                              hipStream_t stream) {
  const TileStats ts = carve_stats(ws, B, V);
  const dim3 blk(256);
  for (int k = 0; k < gamma; ++k) {
    const int32_t* prev = (k == 0) ? anchor : tokens + (k - 1);
    const int stride = (k == 0) ? 1 : gamma;
    {
      TraceScope t("draft_stats_kernel", stream);
      draft_stats_kernel<T, KS><<<dim3((unsigned)n_tiles(V)), blk, 0, stream>>>(
          B, gamma, V, rank, k, U, W1, W2, prev, stride, -1, temperature, ts, status);
    }
    TraceScope t("draft_sample_kernel", stream);
    draft_sample_kernel<T, KS><<<dim3(B), blk, 0, stream>>>(B, gamma, V, rank, k, U, W1, W2,
                                                           prev, stride, -1, temperature,
                                                           uniforms, ts, tokens, q_tok, row_max,
                                                           row_logZ, status);
  }
  return hipGetLastError();
}

// Returns hipErrorNotSupported when the persistent kernel cannot run here.
template <int KS>
static hipError_t draft_persistent(int B, int gamma, int V, int rank, const uint16_t* U,
                                   const uint16_t* W1, const uint16_t* W2,
                                   const int32_t* anchor, const float* temperature,
                                   const float* uniforms, int32_t* tokens, float* q_tok,
                                   float* row_max, float* row_logZ, int32_t* status, void* ws,
                                   hipStream_t stream) {
  const DevInfo di = dev_info();
  const int P = di.cus;
  if (!di.coop || P < 1 || P > kPdMaxGroups) return hipErrorNotSupported;
  if ((long long)n_tiles(V) > (long long)P * (kPdRegTiles + kPdLdsTiles))
    return hipErrorNotSupported;
  // waves per group: 8 (one register tile each, two waves per SIMD, which
  // overlap one wave's reductions with the other's matrix instructions)
  // unless 4 (two tiles each) are asked for
  const int nw = get_draft_path() == 4 ? 4 : 8;
  const void* kern = nw == 8 ? reinterpret_cast<const void*>(pdraft_kernel<KS, 8, true>)
                             : reinterpret_cast<const void*>(pdraft_kernel<KS, 4, false>);
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, nw * 64, 0) != hipSuccess ||
      occ < 1)
    return hipErrorNotSupported;
  PdArgs a;
  a.B = B; a.gamma = gamma; a.V = V; a.rank = rank; a.P = P;
  a.U = U; a.W1 = W1; a.W2 = W2; a.anchor = anchor; a.temperature = temperature;
  a.uniforms = uniforms; a.tokens = tokens; a.q_tok = q_tok; a.row_max = row_max;
  a.row_logZ = row_logZ; a.status = status;
  a.ts = carve_stats(ws, B, V);
  char* fl = static_cast<char*>(ws) + kWsHeader + 3 * stats_bytes(B, V);
  a.stats_flag = reinterpret_cast<uint32_t*>(fl);
  a.tok_flag = reinterpret_cast<uint32_t*>(fl + align256((size_t)kPdMaxGroups * kPdFlagStride * 4));
  a.spin_cap = 200LL * di.wall_khz;  // 0.2 s: reached only if a group never arrives
  {
    TraceScope t("pdraft_reset_kernel", stream);
    const int nflags = P * kPdFlagStride;
    const int n = nflags > B ? nflags : B;
    pdraft_reset_kernel<<<dim3((n + 255) / 256), dim3(256), 0, stream>>>(a.stats_flag, nflags,
                                                                         a.tok_flag, B);
  }
  TraceScope t("pdraft_kernel", stream);
  void* args[] = {&a};
  return hipLaunchCooperativeKernel(kern, dim3(P), dim3(nw * 64), args, 0, stream);
}

static hipError_t draft_block_only(int B, int gamma, int V, int rank, int dtype, const void* U,
                                   const void* W1, const void* W2, const int32_t* anchor,
                                   const float* temperature, const float* uniforms,
                                   int32_t* tokens, float* q_tok, float* row_max,
                                   float* row_logZ, int32_t* status, void* ws,
                                   hipStream_t stream);

// With `cf`, the confidence head too: inside the pipelined kernel (its draw
// waves evaluate it), else by the head's own launch after the draft.
hipError_t launch_draft_block(int B, int gamma, int V, int rank, int dtype, const void* U,
                              const void* W1, const void* W2, const int32_t* anchor,
                              const float* temperature, const float* uniforms, int32_t* tokens,
                              float* q_tok, float* row_max, float* row_logZ, int32_t* status,
                              void* ws, hipStream_t stream, const ConfIn* cf) {
  // the single-launch kernels report a timed-out wait through the status
  // word only, so without one the per-position launches (which never wait)
  // run; the pipelined kernel first (automatic setting, or 5), then the
  // earlier persistent kernel (automatic, or 2-4)
  const int path = get_draft_path();
  const bool persist = path != 1 && status != nullptr;
  if (dtype == DSPARK_BF16 && persist && (path == 0 || path == 5 || path == 6)) {
    const DevInfo di = dev_info();
    hipError_t e = hipErrorNotSupported;
    if (di.cus > 0 && (path != 6 || di.coop))
      e = draft_pipe(B, gamma, V, rank, di.cus, 200LL * di.wall_khz, static_cast<const uint16_t*>(U),
                     static_cast<const uint16_t*>(W1), static_cast<const uint16_t*>(W2), anchor,
                     temperature, uniforms, tokens, q_tok, row_max, row_logZ, status,
                     static_cast<uint32_t*>(ws),
                     static_cast<char*>(ws) + kWsHeader + persistent_ws_bytes(B, V), cf,
                     path == 6, stream);
    if (e != hipErrorNotSupported || path >= 5) return e;
  }
  hipError_t e = draft_block_only(B, gamma, V, rank, dtype, U, W1, W2, anchor, temperature,
                                  uniforms, tokens, q_tok, row_max, row_logZ, status, ws, stream);
  if (e != hipSuccess || !cf) return e;
  return launch_confidence(B, gamma, cf->H, V, rank, dtype, cf->hidden, W1, anchor, tokens, cf->w,
                           cf->bias, cf->temps, cf->conf, status, stream);
}

// the draft by the earlier persistent kernel or the per-position launches
static hipError_t draft_block_only(int B, int gamma, int V, int rank, int dtype, const void* U,
                                   const void* W1, const void* W2, const int32_t* anchor,
                                   const float* temperature, const float* uniforms,
                                   int32_t* tokens, float* q_tok, float* row_max,
                                   float* row_logZ, int32_t* status, void* ws,
                                   hipStream_t stream) {
  const int path = get_draft_path();
  const bool persist = path != 1 && status != nullptr;
  if (dtype == DSPARK_BF16) {
    auto* u = static_cast<const uint16_t*>(U);
    auto* w1 = static_cast<const uint16_t*>(W1);
    auto* w2 = static_cast<const uint16_t*>(W2);
#define DSPARK_DRAFT_KS(KS)                                                                     \
  {                                                                                             \
    if (persist) {                                                                              \
      hipError_t e = draft_persistent<KS>(B, gamma, V, rank, u, w1, w2, anchor, temperature,    \
                                          uniforms, tokens, q_tok, row_max, row_logZ, status,   \
                                          ws, stream);                                          \
      if (e != hipErrorNotSupported || path >= 2) return e;                                     \
    }                                                                                           \
    return draft_multi<uint16_t, KS>(B, gamma, V, rank, u, w1, w2, anchor, temperature,         \
                                     uniforms, tokens, q_tok, row_max, row_logZ, status, ws,    \
                                     stream);                                                   \
  }
    switch (rank) {
      case 32: DSPARK_DRAFT_KS(2)
      case 64: DSPARK_DRAFT_KS(4)
      case 128: DSPARK_DRAFT_KS(8)
      default: DSPARK_DRAFT_KS(16)
    }
#undef DSPARK_DRAFT_KS
  }
  return draft_multi<float, 1>(B, gamma, V, rank, static_cast<const float*>(U),
                               static_cast<const float*>(W1), static_cast<const float*>(W2),
                               anchor, temperature, uniforms, tokens, q_tok, row_max, row_logZ,
                               status, ws, stream);
}

// ---------------------------------------------------------------------------
// RNN head: per position, the recurrence (rnn.hip) produces emb[:, k], then
// the statistics and draw launches take their bias rows from it
// ---------------------------------------------------------------------------

size_t draft_rnn_workspace_bytes(int B, int gamma, int V, int rank, int H, int dtype) {
  (void)H;
  return draft_workspace_bytes(B, gamma, V, rank, dtype) + rnn_workspace_bytes(B, gamma, rank);
}

template <typename T, int KS>
static hipError_t draft_rnn_impl(int B, int gamma, int V, int rank, int H, int dtype,
                                 const T* U, const T* W1, const T* W2, const void* hidden,
                                 const void* Wr, const float* br, const int32_t* anchor,
                                 const float* temperature, const float* uniforms, int32_t* tokens,
                                 float* q_tok, float* row_max, float* row_logZ, T* emb,
                                 float* state, int32_t* status, void* ws, hipStream_t stream) {
  const TileStats ts = carve_stats(ws, B, V);
  void* rws = static_cast<char*>(ws) + draft_workspace_bytes(B, gamma, V, rank, dtype);
  hipError_t e = launch_rnn_hidden(B, gamma, rank, H, dtype, hidden, Wr, br, rws, stream);
  if (e != hipSuccess) return e;
  const dim3 blk(256);
  for (int k = 0; k < gamma; ++k) {
    e = launch_rnn_state(k, B, gamma, V, rank, H, dtype, Wr, W1, anchor, tokens, emb, state,
                         status, rws, stream);
    if (e != hipSuccess) return e;
    {
      TraceScope t("draft_stats_kernel", stream);
      draft_stats_kernel<T, KS><<<dim3((unsigned)n_tiles(V)), blk, 0, stream>>>(
          B, gamma, V, rank, k, U, emb, W2, anchor, 1, k, temperature, ts, status);
    }
    TraceScope t("draft_sample_kernel", stream);
    draft_sample_kernel<T, KS><<<dim3(B), blk, 0, stream>>>(B, gamma, V, rank, k, U, emb, W2,
                                                           anchor, 1, k, temperature, uniforms,
                                                           ts, tokens, q_tok, row_max, row_logZ,
                                                           status);
  }
  return hipGetLastError();
}

hipError_t launch_draft_block_rnn(int B, int gamma, int V, int rank, int H, int dtype,
                                  const void* U, const void* W1, const void* W2,
                                  const void* hidden, const void* Wr, const float* br,
                                  const int32_t* anchor, const float* temperature,
                                  const float* uniforms, int32_t* tokens, float* q_tok,
                                  float* row_max, float* row_logZ, void* emb, float* state,
                                  int32_t* status, void* ws, hipStream_t stream) {
  if (dtype == DSPARK_BF16) {
    auto* u = static_cast<const uint16_t*>(U);
    auto* w1 = static_cast<const uint16_t*>(W1);
    auto* w2 = static_cast<const uint16_t*>(W2);
    auto* em = static_cast<uint16_t*>(emb);
#define DSPARK_RNN_KS(KS)                                                                       \
  return draft_rnn_impl<uint16_t, KS>(B, gamma, V, rank, H, dtype, u, w1, w2, hidden, Wr, br,  \
                                      anchor, temperature, uniforms, tokens, q_tok, row_max,    \
                                      row_logZ, em, state, status, ws, stream)
    switch (rank) {
      case 32: DSPARK_RNN_KS(2);
      case 64: DSPARK_RNN_KS(4);
      case 128: DSPARK_RNN_KS(8);
      default: DSPARK_RNN_KS(16);
    }
#undef DSPARK_RNN_KS
  }
  return draft_rnn_impl<float, 1>(B, gamma, V, rank, H, dtype, static_cast<const float*>(U),
                                  static_cast<const float*>(W1), static_cast<const float*>(W2),
                                  hidden, Wr, br, anchor, temperature, uniforms, tokens, q_tok,
                                  row_max, row_logZ, static_cast<float*>(emb), state, status, ws,
                                  stream);
}

}  // namespace dspark
