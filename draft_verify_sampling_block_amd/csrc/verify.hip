// dspark_verify: lossless speculative rejection sampling.
//
// [billytse] 1 and [xhh] acceptance-rule Q&A: draft token x_k ~ q is
// accepted with probability min(1, p(x_k)/q(x_k)); the first rejection ends
// the scan and one token is drawn there from norm(max(0, p - q)); if all
// verified tokens pass, one bonus token is drawn from the next target slot.
//
// Launches:
//   verify_rows_kernel    one work-group per (slot k, request b), k-major, for
//                         k <= ell[b]: target-row max / argmax / log-sum-exp,
//                         p(x_k), ratio and the accept flag; the first
//                         rejected slot is read off the flags afterwards.
//   verify_tile_stats     (bf16, B <= 128) or verify_plan +
//   / verify_final_stats  verify_final_stats: vocabulary-parallel tiles (as
//                         in drafting): per-chunk sums of the residual
//                         max(0, p_j - q_j) (q_j recomputed bit-identically
//                         on the matrix cores) or of the bonus slot's p.
//   verify_finish_kernel  per request: fp64 scan of the chunk sums, exact
//                         recompute of the crossing chunk, the drawn token,
//                         and the outputs.
#include <algorithm>
#include <type_traits>

#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "row_stats.hpp"
#include "trace.hpp"

namespace dspark {

namespace {

struct VerifyWs {
  float* rM;           // [B][gamma+1] target row max of y = t/T (max t when greedy)
  float* rLZ;          // [B][gamma+1] log sum exp(y - max)
  int32_t* rArg;       // [B][gamma+1] lowest argmax
  float* wratio;       // [B][gamma]
  int32_t* wacc;       // [B][gamma]
  float* fchunk;       // [B][nC] residual (or bonus p) chunk sums
  float* pchunk;       // [B][nC] p chunk sums of the residual slot (fallback)
  int4* plan;          // [B] final draw of the request: (mode, slot, prev, -)
  int32_t* any_res;    // [1] nonzero when some request draws from a residual
  int emb_rows;        // the bias row of (b, j) is row b * gamma + j (RNN head)
};

VerifyWs carve(void* ws, int B, int gamma, int V) {
  char* p = static_cast<char*>(ws);
  const size_t nC = n_tiles(V);
  VerifyWs w;
  w.rM = reinterpret_cast<float*>(p); p += align256((size_t)B * (gamma + 1) * 4);
  w.rLZ = reinterpret_cast<float*>(p); p += align256((size_t)B * (gamma + 1) * 4);
  w.rArg = reinterpret_cast<int32_t*>(p); p += align256((size_t)B * (gamma + 1) * 4);
  w.wratio = reinterpret_cast<float*>(p); p += align256((size_t)B * gamma * 4);
  w.wacc = reinterpret_cast<int32_t*>(p); p += align256((size_t)B * gamma * 4);
  w.fchunk = reinterpret_cast<float*>(p); p += align256((size_t)B * nC * 4);
  w.pchunk = reinterpret_cast<float*>(p); p += align256((size_t)B * nC * 4);
  w.plan = reinterpret_cast<int4*>(p); p += align256((size_t)B * 16);
  w.any_res = reinterpret_cast<int32_t*>(p); p += 256;
  w.emb_rows = 0;
  return w;
}

__device__ inline int clamp_ell(const int32_t* ell, int b, int gamma, int32_t* status) {
  int L = ell[b];
  if (L < 0 || L > gamma) {
    flag(status, DSPARK_DEV_BAD_ELL);
    L = L < 0 ? 0 : gamma;
  }
  return L;
}

__device__ inline float inv_temp(float T) { return (T > 0.f) ? 1.f / T : 0.f; }

// first rejected slot of request b among its L verified slots (L when all
// pass), from the accept flags verify_rows_kernel wrote for every k < L
// The flags are requested eight at a time (independent loads, indices
// clamped to L - 1), so a row costs one memory round trip per eight slots.
__device__ inline int first_reject(const VerifyWs& ws, int b, int gamma, int L) {
  const int32_t* acc = ws.wacc + (size_t)b * gamma;
  for (int k0 = 0; k0 < L; k0 += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = acc[min(k0 + u, L - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < L && v[u] == 0) return k0 + u;
  }
  return L;
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void verify_rows_kernel(
    int B, int gamma, int V, const T* __restrict__ target, const int32_t* __restrict__ tokens,
    const float* __restrict__ q_tok, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, const int32_t* __restrict__ ell, VerifyWs ws,
    int32_t* status) {
  __shared__ double red[8];
  const int k = blockIdx.x / B, b = blockIdx.x % B;
  const int tid = threadIdx.x;
  // the residual flag starts clear; verify_plan_kernel, which runs after
  // this launch, raises it
  if (blockIdx.x == 0 && tid == 0) *ws.any_res = 0;
  const int L = clamp_ell(ell, b, gamma, tid == 0 ? status : nullptr);
  if (k > L) return;  // uniform: every thread reads the same ell[b]

  const float it = inv_temp(temperature[b]);
  const bool greedy = !(it > 0.f);
  const float scale = greedy ? 1.f : it;
  const T* row = target + ((size_t)b * (gamma + 1) + k) * V;

  const RowStats rs = row_stats<T>(row, V, scale, greedy, red);
  const float M = rs.M;
  const double Zt = rs.Z;
  const int a = rs.arg;

  if (tid == 0) {
    const size_t sk = (size_t)b * (gamma + 1) + k;
    const bool fin = (M == M) && M > -INFINITY && M < INFINITY && (greedy || (Zt > 0.0 && Zt < INFINITY));
    if (!fin) flag(status, DSPARK_DEV_NONFINITE);
    ws.rM[sk] = M;
    ws.rLZ[sk] = greedy ? 0.f : (float)log(Zt);
    ws.rArg[sk] = (a >= 0 && a < V) ? a : 0;
    if (k < L) {
      const size_t bk = (size_t)b * gamma + k;
      const int x = clamp_token(tokens[bk], V, status);
      float p;
      if (greedy) {
        p = (x == a) ? 1.f : 0.f;
      } else {
        float tx;
        if constexpr (sizeof(T) == 2) tx = bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[x]);
        else tx = reinterpret_cast<const float*>(row)[x];
        p = (float)((double)__expf(tx * scale - M) / Zt);
      }
      const float q = q_tok[bk];
      const float u = uniforms[((size_t)b * (gamma + 1) + k) * 2 + 1];
      const bool accept = u * q < p;
      ws.wratio[bk] = p / q;
      ws.wacc[bk] = accept ? 1 : 0;
    }
  }
}

// per-element residual / bonus weight; identical expression in both kernels
__device__ inline void final_weight(float yt, float yq, float M, float LZ, float mq, float lzq,
                                    bool residual, float& r, float& p) {
  p = __expf(yt - M - LZ);
  if (residual) {
    const float q = __expf(yq - mq - lzq);
    r = fmaxf(0.f, p - q);
  } else {
    r = p;
  }
}

// Final-draw row of request b: mode 0 = nothing to stream (greedy), 1 =
// residual at the first rejected slot j, 2 = bonus at slot L.
struct FinalRow {
  int mode, slot, prev;
};
__device__ inline FinalRow final_row(int b, int B, int gamma, int V, const int32_t* ell,
                                     const float* temperature, const int32_t* anchor,
                                     const int32_t* tokens, const VerifyWs& ws) {
  FinalRow f{0, 0, -1};
  if (b >= B) return f;
  const int L = clamp_ell(ell, b, gamma, nullptr);
  if (!(temperature[b] > 0.f)) return f;
  const int j = first_reject(ws, b, gamma, L);
  if (j < L) {
    f.mode = 1;
    f.slot = j;
    f.prev = ws.emb_rows ? b * gamma + j
                         : clamp_token(j == 0 ? anchor[b] : tokens[(size_t)b * gamma + j - 1],
                                       V, nullptr);
  } else {
    f.mode = 2;
    f.slot = L;
  }
  return f;
}

// the final draw of every request, once the first rejections are known
__global__ void verify_plan_kernel(int B, int gamma, int V, const int32_t* __restrict__ ell,
                                   const float* __restrict__ temperature,
                                   const int32_t* __restrict__ anchor,
                                   const int32_t* __restrict__ tokens, VerifyWs ws) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const FinalRow f = final_row(b, B, gamma, V, ell, temperature, anchor, tokens, ws);
  ws.plan[b] = make_int4(f.mode, f.slot, f.prev, 0);
  if (f.mode == 1) atomicOr(ws.any_res, 1);
}

// Per-request constants of the final weights (mode 0: nothing to sum).
struct FinalParams {
  int mode;
  float it, M, LZ, mq, lzq;
};
__device__ inline FinalParams final_params(const FinalRow& mine, int b, int gamma,
                                           const float* __restrict__ row_max,
                                           const float* __restrict__ row_logZ,
                                           const float* __restrict__ temperature,
                                           const VerifyWs& ws) {
  FinalParams f{mine.mode, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mine.mode != 0) {
    f.it = 1.f / temperature[b];
    const size_t sk = (size_t)b * (gamma + 1) + mine.slot;
    f.M = ws.rM[sk];
    f.LZ = ws.rLZ[sk];
    if (mine.mode == 1) {
      f.mq = row_max[(size_t)b * gamma + mine.slot];
      f.lzq = row_logZ[(size_t)b * gamma + mine.slot];
    }
  }
  return f;
}
// Residual and p mass of one 32-entry sub-tile for the lane's request: the
// lane's 16 entries (target logits yt, q logits yq; `rem` usable entries of
// the lane) summed in order, then the two half-waves' sums added.
__device__ inline void subtile_sums(const FinalParams& f, const float (&yt)[16],
                                    const f32x16_t& yq, int rem, float& sr, float& sp) {
  sr = 0.f;
  sp = 0.f;
  if (f.mode != 0) {
    const bool res = f.mode == 1;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < rem) {
        float r, p;
        final_weight(yt[j] * f.it, res ? yq[j] * f.it : 0.f, f.M, f.LZ, f.mq, f.lzq, res, r, p);
        sr += r;
        sp += p;
      }
    }
  }
  float lo, hi;
  half_pair(sr, lo, hi);
  sr = lo + hi;
  half_pair(sp, lo, hi);
  sp = lo + hi;
}

// One (64-entry tile, 32-request block) task of the final statistics for
// the lane's request b (column c): the q logits of residual requests start
// at the base logits and get the Markov bias on the matrix cores (A = the
// W2 tile in LDS, B = the W1 rows of the previous tokens), then the
// residual and p masses of the tile are summed per request.  All 64 lanes
// call it; tp holds the lane's target entries and acc starts at its base
// logits (init_acc).
template <typename T, int KS>
__device__ inline void final_task(const FinalRow& mine, int b, int vt, int V, int gamma, int nT,
                                  int rank, const URow<T>& tp, f32x16_t (&acc)[kSub],
                                  const bf16x8_t (&bfrag)[KS], const char* w2s,
                                  const T* __restrict__ W1, const T* __restrict__ W2,
                                  const float* __restrict__ row_max,
                                  const float* __restrict__ row_logZ,
                                  const float* __restrict__ temperature, const VerifyWs& ws) {
  constexpr bool bf = sizeof(T) == 2;
  const int h = (threadIdx.x & 63) >> 5;
  const int v0 = vt * kTileV;
  const bool blk_res = __ballot(mine.mode == 1) != 0;
  if (blk_res) {
    if constexpr (bf)
      bias_tile_ldsA<KS>([&](int ks) { return bfrag[ks]; }, w2s, acc);
    else
      bias_tile_f32(reinterpret_cast<const float*>(W1), mine.mode == 1 ? mine.prev : -1,
                    reinterpret_cast<const float*>(W2), v0, V, rank, acc);
  }
  float sr = 0.f, sp = 0.f;
  const FinalParams fp = final_params(mine, b, gamma, row_max, row_logZ, temperature, ws);
#pragma unroll
  for (int t = 0; t < kSub; ++t) {
    float yt[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) yt[j] = urow_at(tp, t, j);
    float r, p;
    subtile_sums(fp, yt, acc[t], V - (v0 + 32 * t + 16 * h), r, p);
    sr += r;
    sp += p;
  }
  if (mine.mode != 0 && h == 0) {
    const size_t ci = (size_t)b * nT + vt;
    ws.fchunk[ci] = sr;
    ws.pchunk[ci] = sp;
  }
}

// one work-group per 64-entry tile; waves take 32-request blocks
template <typename T, int KS>
__global__ __launch_bounds__(256) void verify_final_stats_kernel(
    int B, int gamma, int V, int rank, const T* __restrict__ target, const T* __restrict__ U,
    const T* __restrict__ W1, const T* __restrict__ W2, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ row_max,
    const float* __restrict__ row_logZ, const float* __restrict__ temperature,
    const int32_t* __restrict__ ell, VerifyWs ws, int32_t* status) {
  constexpr bool bf = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) char w2s[bf ? kLdsTileBytes : 16];
  __shared__ __attribute__((aligned(16))) char s_stg[bf ? 4 : 1][bf ? kTileM * 128 : 16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nRB = (B + kTileM - 1) / kTileM;
  const int nT = n_tiles(V);
  const int vt = blockIdx.x, v0 = vt * kTileV;

  // does any request of the batch need the q recompute (a residual draw)?
  const bool any_res = *ws.any_res != 0;
  if (bf && any_res) stage_tile(reinterpret_cast<const uint16_t*>(W2), v0, V, rank, w2s);

  auto plan_of = [&](int r) {   // the final-draw plan of request r (mode 0 past the batch)
    FinalRow f{0, 0, -1};
    if (r < B) {
      const int4 pl = ws.plan[r];
      f = FinalRow{pl.x, pl.y, pl.z};
    }
    return f;
  };

  if constexpr (bf) {
    // One pass per 32-request block rb (lane column c = request b), one
    // block ahead: the block's target and base-logit rows of the tile are
    // loaded as whole 128-byte rows (load j: block row 8 (j % 4) + lane / 8,
    // entries 8 (lane % 8) + [0, 8)), with the plans they need requested one
    // block earlier still, and passed to the matrix layout through the
    // wave's 4 KB of LDS (16-byte pieces swizzled by row).  A load whose
    // lanes each take 16 bytes of another row (32 rows per instruction)
    // moves about half as many bytes per second on this chip.
    const uint16_t* tg = reinterpret_cast<const uint16_t*>(target);
    const uint16_t* ub = reinterpret_cast<const uint16_t*>(U);
    const int lr = lane >> 3, lp = lane & 7;
    char* stg = s_stg[wave];
    struct Plans {
      FinalRow mine;      // the lane's request
      int2 rows[4];       // (mode, slot) of the rows the lane loads
    };
    auto plans = [&](int rb, Plans& pl) {
      pl.mine = plan_of(rb < nRB ? rb * kTileM + c : B);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const FinalRow f = plan_of(rb < nRB ? rb * kTileM + 8 * j + lr : B);
        pl.rows[j] = make_int2(f.mode, f.slot);
      }
    };
    auto fetch = [&](u32x4_t (&ld)[8], int rb, const Plans& pl) {
      const int e = v0 + 8 * lp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = rb * kTileM + 8 * j + lr;
        const int md = pl.rows[j].x, sl = pl.rows[j].y;   // mode 0 for rows past the batch
        const bool in = e < V;
        ld[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            in && md != 0 ? tg + ((size_t)r * (gamma + 1) + sl) * V + e : tg));
        ld[4 + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            in && md == 1 ? ub + ((size_t)r * gamma + sl) * V + e : ub));
      }
    };
    // registers -> LDS (row r's piece q at q ^ (r % 8)) -> lane (c, h):
    // sub-tile st, load q of URow = piece 4 st + 2 h + q of row c
    auto restage = [&](const u32x4_t (&ld)[8], URow<uint16_t>& tp, URow<uint16_t>& up) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<u32x4_t*>(stg + (8 * j + lr) * 128 + 16 * (lp ^ lr)) = ld[4 * a + j];
        asm volatile("" ::: "memory");   // the wave's LDS accesses stay in this order
        URow<uint16_t>& dst = a == 0 ? tp : up;
#pragma unroll
        for (int st = 0; st < kSub; ++st) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int pc = 4 * st + 2 * h + q;
            dst.w[st][q] =
                *reinterpret_cast<const u32x4_t*>(stg + c * 128 + 16 * (pc ^ (c & 7)));
          }
        }
        asm volatile("" ::: "memory");
      }
    };

    Plans pl, pl_next;
    plans(wave, pl);
    u32x4_t ld[8];
    fetch(ld, wave, pl);
    plans(wave + 4, pl_next);
    for (int rb = wave; rb < nRB || (rb == wave); rb += 4) {
      // the first pass of every wave also joins the barrier that publishes
      // the LDS tile
      const bool live = rb < nRB;
      const int b = rb * kTileM + c;
      const FinalRow mine = pl.mine;
      // the block's W1 rows (previous tokens of residual requests) loaded as
      // whole 128-byte segments, 8 rows per load (pass q, load j: row
      // 8 j + lane / 8, piece 8 q + lane % 8 of the row's 2 KS pieces of 16
      // bytes), then passed to the B-operand layout through the wave's LDS
      // area like the target rows: lane (c, h) takes pieces 2 ks + h of row c
      // (rank 32: rows of 64 bytes, loaded per lane as before)
      constexpr int kW1 = KS >= 4 ? KS : 1;
      const int tokc = mine.mode == 1 ? mine.prev : -1;
      u32x4_t w1raw[kW1];
      if constexpr (KS >= 4) {
        const uint16_t* w1 = reinterpret_cast<const uint16_t*>(W1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tr = __shfl(tokc, 8 * j + lr, kWave);   // lane r < 32 holds request r
          const uint16_t* row = w1 + (size_t)(tr >= 0 ? tr : 0) * (16 * KS) + 8 * lp;
#pragma unroll
          for (int q = 0; q < KS / 4; ++q)
            w1raw[4 * q + j] = *reinterpret_cast<const u32x4_t*>(row + 64 * q);
        }
      }
      URow<uint16_t> tp, up;
      restage(ld, tp, up);
      fetch(ld, rb + 4, pl_next);
      bf16x8_t bfrag[KS];
      if constexpr (KS < 4) load_bfrag<KS>(reinterpret_cast<const uint16_t*>(W1), tokc, bfrag);
#pragma unroll
      for (int q = 0; q < KS / 4; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<u32x4_t*>(stg + (8 * j + lr) * 128 + 16 * (lp ^ lr)) = w1raw[4 * q + j];
        asm volatile("" ::: "memory");   // the wave's LDS accesses stay in this order
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int pc = 2 * kk + h;
          bfrag[4 * q + kk] = tokc >= 0
              ? *reinterpret_cast<const bf16x8_t*>(stg + c * 128 + 16 * (pc ^ (c & 7)))
              : bf16x8_t{};
        }
        asm volatile("" ::: "memory");
      }
      pl = pl_next;
      plans(rb + 8, pl_next);
      if (rb == wave) {
        if (any_res) __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      if (!live) break;
      f32x16_t acc[kSub];
      init_acc<uint16_t>(up, V - (v0 + 16 * h), acc);   // q logits start at the base logits
      final_task<T, KS>(mine, b, vt, V, gamma, nT, rank, tp, acc, bfrag, w2s, W1, W2, row_max,
                        row_logZ, temperature, ws);
    }
  } else {
    for (int rb = wave; rb < nRB; rb += 4) {
      const int b = rb * kTileM + c;
      const FinalRow mine = plan_of(b);
      bf16x8_t bfrag[KS];   // unused: fp32 adds the bias with plain FMAs
      URow<T> tp, up;
      load_urow<T>(tp, target + ((size_t)b * (gamma + 1) + mine.slot) * V, v0, V,
                   mine.mode != 0, target);
      load_urow<T>(up, U + ((size_t)b * gamma + mine.slot) * V, v0, V, mine.mode == 1, U);
      f32x16_t acc[kSub];
      init_acc<T>(up, V - (v0 + 16 * h), acc);   // q logits start at the base logits
      final_task<T, KS>(mine, b, vt, V, gamma, nT, rank, tp, acc, bfrag, w2s, W1, W2, row_max,
                        row_logZ, temperature, ws);
    }
  }
}

// The same statistics in tile-loop form (bf16, at most kVtMaxRows
// requests): one work-group of 8 waves per compute unit.  Work-group p owns
// the contiguous tiles [tbase, tbase + tcount) and walks them one by one;
// wave w computes sub-tile w % 2 of 32-request block w / 2 (A = the W2 tile
// in LDS, B = the W1 row of the lane's previous token, held in registers),
// so each element is computed exactly as verify_final_stats_kernel computes
// it and the sub-tile sums are combined in the same order.  The next tile's
// W2 rows are loaded into registers while the current one is processed and
// written to the other LDS buffer; the chunk sums collect in LDS and are
// written out every kVtOutTiles tiles.
//
// The target and base-logit entries a wave needs (32 rows x 64 bytes per
// tile) are loaded 16 rows per instruction, four lanes to a row's 64 bytes,
// and passed through a per-wave LDS area to the lanes of the matrix layout
// (lane = request, 32 bytes each).  A load whose lanes each touch another
// row (32 rows per instruction) moves about two thirds as many bytes per
// second on this chip at the same occupancy.
constexpr int kVtWaves = 8;
constexpr int kVtMaxRows = 4 * kTileM;
constexpr int kVtOutTiles = 16;
constexpr int kVtStageRow = 80;   // 64 bytes of one row's entries + 16 of padding
template <int KS>
__global__ __launch_bounds__(kVtWaves * 64, 1) void verify_tile_stats_kernel(
    int B, int gamma, int V, int rank, const uint16_t* __restrict__ target,
    const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ row_max,
    const float* __restrict__ row_logZ, const float* __restrict__ temperature,
    const int32_t* __restrict__ ell, VerifyWs ws) {
  constexpr int nq = 2 * KS, nc = nq + 1;
  constexpr int kRowB = nc * 16;                 // bytes of one padded LDS row
  constexpr int kThr = kVtWaves * 64;
  constexpr int kBlocks = 32 * KS;               // 4 x 8 blocks of one tile (rank 16 KS)
  constexpr int kPer = (kBlocks + kThr - 1) / kThr;
  __shared__ __attribute__((aligned(16))) char w2s[2][kTileV * kRowB];
  // per wave: [target | base logits][32 rows][kVtStageRow]
  __shared__ __attribute__((aligned(16))) char s_stage[kVtWaves][2][kTileM][kVtStageRow];
  __shared__ float s_part[2][kSub][kVtMaxRows][2];
  __shared__ float s_out[2][kVtOutTiles][kVtMaxRows];
  __shared__ int s_mode[kVtMaxRows], s_slot[kVtMaxRows], s_prv[kVtMaxRows];
  __shared__ int s_any;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const int t = wave & 1, rb = wave >> 1;
  const int P = gridDim.x, p = blockIdx.x;
  const int nT = n_tiles(V);
  const int tcount = nT / P + (p < nT % P ? 1 : 0);
  const int tbase = p * (nT / P) + min(p, nT % P);
  // every request's plan (the rows the waves load for one another)
  if (tid == 0) s_any = 0;
  __syncthreads();
  for (int r = tid; r < kVtMaxRows; r += kThr) {
    FinalRow f{0, 0, -1};
    if (r < B) f = final_row(r, B, gamma, V, ell, temperature, anchor, tokens, ws);
    if (f.mode == 1) s_any = 1;
    s_mode[r] = f.mode;
    s_slot[r] = f.slot;
    s_prv[r] = f.prev;
  }
  __syncthreads();
  const bool any_res = s_any != 0;   // some request of the batch draws from a residual

  // tile vt's transposed image (as stage_tile writes it): thread blocks
  // tid + kThr j of 4 k-rows x 8 entries of W2 [rank, V].  Two register
  // stages: tile i + 1 waits in one while tile i + 2 loads into the other.
  W2Block stA[kPer], stB[kPer];
  auto load_tile = [&](W2Block (&st)[kPer], int vt) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      w2_block_load(W2, V, vt * kTileV, min(tid + kThr * j, kBlocks - 1), st[j]);
  };
  auto write_tile = [&](const W2Block (&st)[kPer], int buf) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int sb = tid + kThr * j;
      if (kBlocks % kThr == 0 || sb < kBlocks) w2_block_store(st[j], sb, w2s[buf], nq);
    }
  };
  // every load below is issued unconditionally (safe or clamped addresses
  // where there is nothing to read): with a fixed count of loads per step
  // the in-order memory counter waits for exactly the data it needs
  const int tlast = tbase + tcount - 1;
  // this wave's request column
  const int b = rb * kTileM + c;
  const bool active = rb * kTileM < B;

  // The rows this lane loads for its wave: block rows 16 g + lane / 4
  // (g = 0, 1), 16 bytes at entry 32 t + 8 (lane % 4) of the tile.
  const int lr = lane >> 2, lq = lane & 3;
  const uint16_t* lt[2];
  const uint16_t* lu[2];
  bool lt_on[2], lu_on[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int r = rb * kTileM + 16 * g + lr;
    const bool own = active && r < B;
    const int md = own ? s_mode[r] : 0;
    const int sl = own ? s_slot[r] : 0;
    lt_on[g] = md != 0;
    lu_on[g] = md == 1;
    lt[g] = target + ((size_t)(own ? r : 0) * (gamma + 1) + sl) * V;
    lu[g] = U + ((size_t)(own ? r : 0) * gamma + sl) * V;
  }
  // two register sets, like the tile stages: step i stages one and fills
  // the other, so no loaded register is ever copied (a copy would wait for
  // it).  Set element j: j / 2 = target or base logits, j % 2 = g.
  u32x4_t ldA[4], ldB[4];
  auto fetch = [&](u32x4_t (&ld)[4], int vt) {
    const int e = vt * kTileV + 32 * t + 8 * lq;
    const bool in = vt <= tlast && e < V;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      ld[g] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(in && lt_on[g] ? lt[g] + e : target));
      ld[2 + g] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(in && lu_on[g] ? lu[g] + e : U));
    }
  };
  // the first tile's entries, W2 rows and W1 fragments requested together
  fetch(ldA, tbase);
  if (any_res) {
    load_tile(stA, tbase);
    write_tile(stA, 0);
  }

  // plan, weights' constants, the W1 row of the previous token (zero
  // unless the request draws from a residual)
  FinalRow mine{0, 0, -1};
  if (active && b < B) mine = FinalRow{s_mode[b], s_slot[b], s_prv[b]};
  const FinalParams fpar = final_params(mine, b, gamma, row_max, row_logZ, temperature, ws);
  const bool blk_res = any_res && __ballot(mine.mode == 1) != 0;
  bf16x8_t bfrag[KS];
  load_bfrag<KS>(W1, (any_res && mine.mode == 1) ? mine.prev : -1, bfrag);
  __builtin_amdgcn_s_waitcnt(0);   // the first tile's operands have landed
  __syncthreads();

  // registers -> this wave's LDS area -> the matrix layout: lane (c, h)
  // takes entries 32 t + 16 h + [0, 16) of request row c
  char (*stg)[kTileM][kVtStageRow] = s_stage[wave];
  auto restage = [&](const u32x4_t (&ld)[4], u32x4_t (&tq)[2], u32x4_t (&uq)[2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4_t*>(&stg[j >> 1][16 * (j & 1) + lr][16 * lq]) = ld[j];
    asm volatile("" ::: "memory");   // the wave's LDS accesses stay in this order
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      tq[q] = *reinterpret_cast<const u32x4_t*>(&stg[0][c][16 * (2 * h + q)]);
      uq[q] = *reinterpret_cast<const u32x4_t*>(&stg[1][c][16 * (2 * h + q)]);
    }
    asm volatile("" ::: "memory");
  };

  auto flush = [&](int first, int n) {   // s_out rows of tiles [first, first + n)
    for (int e = tid; e < n * kVtMaxRows; e += kThr) {
      const int r = e / n, i = e - r * n;
      if (r < B) {
        const size_t ci = (size_t)r * nT + tbase + first + i;
        ws.fchunk[ci] = s_out[0][(first + i) % kVtOutTiles][r];
        ws.pchunk[ci] = s_out[1][(first + i) % kVtOutTiles][r];
      }
    }
  };
  // the tile walk, with (kRes) or without the bias on the matrix cores
  auto walk = [&](auto res_tag) {
    constexpr bool kRes = decltype(res_tag)::value;
    if constexpr (kRes) load_tile(stB, min(tbase + 1, tlast));
    // tile i from LDS buffer i & 1; `next` holds tile i + 1, `after`
    // receives tile i + 2; `ld` holds tile i's entries, `ld1` receives
    // tile i + 1's
    auto step = [&](int i, const W2Block (&next)[kPer], W2Block (&after)[kPer],
                    const u32x4_t (&ld)[4], u32x4_t (&ld1)[4]) {
      const int vt = tbase + i;
      u32x4_t tq[2], uq[2];
      restage(ld, tq, uq);
      f32x16_t acc;
      float yt[16];
      const int rem = V - (vt * kTileV + 32 * t + 16 * h);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t wu = uq[j >> 3][(j >> 1) & 3], wt = tq[j >> 3][(j >> 1) & 3];
        const float fu = (j & 1) ? __uint_as_float(wu & 0xFFFF0000u) : __uint_as_float(wu << 16);
        yt[j] = (j & 1) ? __uint_as_float(wt & 0xFFFF0000u) : __uint_as_float(wt << 16);
        acc[j] = j < rem ? fu : -INFINITY;   // q logits start at the base logits
      }
      fetch(ld1, vt + 1);
      if constexpr (kRes) load_tile(after, min(vt + 2, tlast));
      if (active) {
        if (kRes && blk_res)
          bias_subtile_ldsA<KS>([&](int ks) { return bfrag[ks]; }, w2s[i & 1], t, acc);
        float sr, sp;
        subtile_sums(fpar, yt, acc, rem, sr, sp);
        if (h == 0) {
          s_part[i & 1][t][b][0] = sr;
          s_part[i & 1][t][b][1] = sp;
        }
      }
      if constexpr (kRes) {
        if (i + 1 < tcount) write_tile(next, (i + 1) & 1);
      }
      __syncthreads();
      // the tile's chunk sums: sub-tile 0 + sub-tile 1, as in final_task
      if (tid < kVtMaxRows) {
        s_out[0][i % kVtOutTiles][tid] = s_part[i & 1][0][tid][0] + s_part[i & 1][1][tid][0];
        s_out[1][i % kVtOutTiles][tid] = s_part[i & 1][0][tid][1] + s_part[i & 1][1][tid][1];
      }
      if ((i + 1) % kVtOutTiles == 0 || i + 1 == tcount) {
        __syncthreads();
        const int first = i - i % kVtOutTiles;
        flush(first, i + 1 - first);
        __syncthreads();
      }
    };
    for (int i = 0; i < tcount; i += 2) {
      step(i, stB, stA, ldA, ldB);
      if (i + 1 < tcount) step(i + 1, stA, stB, ldB, ldA);
    }
  };
  if (any_res) walk(std::true_type{});
  else walk(std::false_type{});
}

constexpr int kFinPer = kMaxTiles / 256;   // chunk sums per thread of the finish kernel

template <typename T, int KS>
__global__ __launch_bounds__(256) void verify_finish_kernel(
    int B, int gamma, int V, int rank, const T* __restrict__ target, const T* __restrict__ U,
    const T* __restrict__ W1, const T* __restrict__ W2, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ row_max,
    const float* __restrict__ row_logZ, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, const int32_t* __restrict__ ell, VerifyWs ws,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ n_accepted,
    float* __restrict__ ratio, int32_t* status) {
  constexpr bool bf = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) char w2s[bf ? kRawTileBytes : 16];
  __shared__ double red[8];
  __shared__ int s_tile, s_pick;
  __shared__ double s_before;
  __shared__ float se[kTileV];
  __shared__ int s_j, s_prev;

  const int b = blockIdx.x, tid = threadIdx.x;
  const int nT = n_tiles(V);
  // Everything that does not wait for the first rejection is requested at
  // once: the verify length, the temperature, the request's accept flags
  // and drafted tokens (wave 0, one slot per lane), the anchor, this
  // thread's residual chunk sums and the draw uniform.
  const int L = clamp_ell(ell, b, gamma, nullptr);
  const float Tb = temperature[b];
  const bool greedy = !(Tb > 0.f);
  const int per = (nT + blockDim.x - 1) / blockDim.x;   // <= kFinPer
  const int c0 = min(nT, tid * per), c1 = min(nT, c0 + per);
  const float* fc = ws.fchunk + (size_t)b * nT;
  const float* pc = ws.pchunk + (size_t)b * nT;
  float fcv[kFinPer];
#pragma unroll
  for (int i = 0; i < kFinPer; ++i) fcv[i] = (!greedy && c0 + i < c1) ? fc[c0 + i] : 0.f;
  const double u = (double)uniforms[((size_t)b * (gamma + 1) + gamma) * 2 + 0];
  if (tid < kWave) {
    const int lane = tid;
    const int acc = lane < gamma ? ws.wacc[(size_t)b * gamma + lane] : 1;
    const int tok = lane < gamma ? tokens[(size_t)b * gamma + lane] : 0;
    const int anc = anchor[b];
    // the first slot among the L tested whose flag is 0 (L when all pass)
    const unsigned long long rej = __ballot(lane < L && acc == 0);
    const int jj = rej ? __builtin_ctzll(rej) : L;
    const int tk = __shfl(tok, jj > 0 ? jj - 1 : 0, kWave);
    if (lane == 0) {
      s_j = jj;
      s_prev = jj < L ? (ws.emb_rows ? b * gamma + jj : clamp_token(jj == 0 ? anc : tk, V, nullptr))
                      : -1;
    }
  }
  __syncthreads();
  const int j = s_j;
  const bool residual = j < L;
  const int slot = residual ? j : L;
  const int n = residual ? j : L;
  const size_t sk = (size_t)b * (gamma + 1) + slot;

  int y = 0;
  if (greedy) {
    y = ws.rArg[sk];
  } else {
    // the crossing tile's recompute operands that do not wait for the scan:
    // the weights' constants and the previous token's W1 row
    const int mrow = b % kTileM;
    const int lane = tid & 63, c = lane & 31, h = lane >> 5;
    const bool mine = tid < (bf ? kSub : 1) * kWave && c == mrow;
    const int prev = s_prev;
    const float it = 1.f / Tb;
    const float M = ws.rM[sk], LZ = ws.rLZ[sk];
    const float mq = residual ? row_max[(size_t)b * gamma + slot] : 0.f;
    const float lzq = residual ? row_logZ[(size_t)b * gamma + slot] : 0.f;
    bf16x8_t bfrag[bf ? KS : 1];
    if constexpr (bf) {
      if (residual && tid < kSub * kWave)
        load_bfrag<KS>(reinterpret_cast<const uint16_t*>(W1), mine ? prev : -1, bfrag);
    }
    // residual tile sums; fall back to p when the residual has no mass
    double local = 0.0;
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
      if (c0 + i < c1) local += (double)fcv[i];
    double start, end;
    double S = block_scan_interval(local, red, &start, &end);
    bool use_p = false;
    if (!(S > 0.0) && residual) {
      use_p = true;
      if (tid == 0) flag(status, DSPARK_DEV_DEGENERATE);
      local = 0.0;
#pragma unroll
      for (int i = 0; i < kFinPer; ++i) {
        fcv[i] = c0 + i < c1 ? pc[c0 + i] : 0.f;
        if (c0 + i < c1) local += (double)fcv[i];
      }
      S = block_scan_interval(local, red, &start, &end);
    }
    const double tgt = u * S;
    const bool finite = S > 0.0 && isfinite(S);
    const int last_pos = block_max_int(local > 0.0 ? tid : -1, red);
    if (tid == 0) s_tile = -1;
    __syncthreads();
    if (finite && local > 0.0 &&
        ((start <= tgt && tgt < end) || (tid == last_pos && tgt >= end))) {
      double run = start, before = start, lastb = start;
      int found = -1, lastc = -1;
#pragma unroll
      for (int i = 0; i < kFinPer; ++i) {   // the thread's chunks, in order
        const int cc = c0 + i;
        const double sc = (double)fcv[i];
        if (cc < c1 && found < 0) {
          if (sc > 0.0) { lastc = cc; lastb = run; }
          if (sc > 0.0 && tgt < run + sc) { found = cc; before = run; }
          run += sc;
        }
      }
      if (found < 0) { found = lastc; before = lastb; }
      s_tile = found;
      s_before = before;
    }
    __syncthreads();
    const int vt = s_tile;
    if (vt < 0) {
      if (tid == 0) flag(status, DSPARK_DEV_NONFINITE);
      y = 0;
    } else {
      // recompute the crossing tile exactly as verify_final_stats did:
      // same operands, request b in its own column b % 32; bf16: waves 0
      // and 1 take sub-tiles 0 and 1 (A gathered from the tile's raw W2
      // rows), fp32: wave 0 takes both
      const int v0 = vt * kTileV;
      const int tw = tid >> 6;   // bf16: the sub-tile of waves 0 and 1
      URow<T> tr, ur;
      load_urow<T>(tr, target + sk * V, v0, V, mine, target);
      load_urow<T>(ur, U + ((size_t)b * gamma + slot) * V, v0, V, mine && residual, U);
      f32x16_t acc[kSub];
      init_acc<T>(ur, V - (v0 + 16 * h), acc);
      if (residual) {
        if constexpr (bf) {
          dma_tile_raw(reinterpret_cast<const uint16_t*>(W2), V, v0, rank, w2s);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
          auto bf_ = [&](int ks) { return bfrag[ks]; };
          if (tw == 0)
            bias_subtile<KS>([&](int ks) { return raw_frag(w2s, 0, ks); }, bf_, acc[0]);
          else if (tw == 1)
            bias_subtile<KS>([&](int ks) { return raw_frag(w2s, 1, ks); }, bf_, acc[1]);
        } else {
          if (tid < kWave)
            bias_tile_f32(reinterpret_cast<const float*>(W1), mine ? prev : -1,
                          reinterpret_cast<const float*>(W2), v0, V, rank, acc);
        }
      }
      if (mine) {
        const int rem = V - (v0 + 16 * h);
#pragma unroll
        for (int t = 0; t < kSub; ++t) {
          if (bf && t != tw) continue;
          float* so = se + 32 * t + 16 * h;
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            float r = 0.f, p = 0.f;
            if (32 * t + jj < rem) {
              const float yt = urow_at(tr, t, jj) * it;
              const float yq = residual ? acc[t][jj] * it : 0.f;
              final_weight(yt, yq, M, LZ, mq, lzq, residual, r, p);
            }
            so[jj] = use_p ? p : r;
          }
        }
      }
      __syncthreads();
      // the entry: the first with positive weight whose running sum passes
      // the target (else the last positive one), one entry per lane of
      // wave 0 with the running sums as a wave scan
      if (tid < kWave) {
        const double rr = tgt - s_before;
        const double e = (double)se[tid];
        double run = e;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const double nb = __shfl_up(run, o, kWave);
          if (tid >= o) run += nb;
        }
        const unsigned long long hit = __ballot(e > 0.0 && rr < run);
        const unsigned long long pos = __ballot(e > 0.0);
        const int pick = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
        if (tid == 0) s_pick = v0 + pick;
      }
      __syncthreads();
      y = s_pick;
    }
  }

  // outputs: accepted prefix, the drawn token, -1 padding; ratios of tested slots
  for (int i = tid; i <= gamma; i += blockDim.x) {
    int v = -1;
    if (i < n) v = tokens[(size_t)b * gamma + i];
    else if (i == n) v = y;
    out_tokens[(size_t)b * (gamma + 1) + i] = v;
  }
  if (ratio) {
    for (int i = tid; i < gamma; i += blockDim.x)
      ratio[(size_t)b * gamma + i] = (i < L && i <= j) ? ws.wratio[(size_t)b * gamma + i] : NAN;
  }
  if (tid == 0) n_accepted[b] = n;
}

size_t verify_workspace_bytes(int B, int gamma, int V, int rank, int dtype) {
  (void)rank; (void)dtype;
  const size_t nC = n_tiles(V);
  return 3 * align256((size_t)B * (gamma + 1) * 4) +
         2 * align256((size_t)B * gamma * 4) + 2 * align256((size_t)B * nC * 4) +
         align256((size_t)B * 16) + 256;
}

template <typename T, int KS>
static hipError_t verify_impl(int B, int gamma, int V, int rank, const T* target, const T* U,
                              const T* W1, const T* W2, const int32_t* anchor,
                              const int32_t* tokens, const float* q_tok, const float* row_max,
                              const float* row_logZ, const float* temperature,
                              const float* uniforms, const int32_t* ell, int32_t* out_tokens,
                              int32_t* n_accepted, float* ratio, int32_t* status, void* wsp,
                              hipStream_t stream, bool emb_rows) {
  VerifyWs ws = carve(wsp, B, gamma, V);
  ws.emb_rows = emb_rows ? 1 : 0;
  {
    TraceScope t1("verify_rows_kernel", stream);
    verify_rows_kernel<T><<<dim3(B * (gamma + 1)), dim3(256), 0, stream>>>(
        B, gamma, V, target, tokens, q_tok, temperature, uniforms, ell, ws, status);
  }

  // bf16 with at most 128 requests: the tile-loop form
  bool tiles = false;
  if constexpr (sizeof(T) == 2) {
    const int cus = device_cu_count();
    if (B <= kVtMaxRows && cus > 0) {
      const int P = std::min(cus, n_tiles(V));
      TraceScope t2("verify_tile_stats_kernel", stream);
      verify_tile_stats_kernel<KS><<<dim3(P), dim3(kVtWaves * 64), 0, stream>>>(
          B, gamma, V, rank, target, U, W1, W2, anchor, tokens, row_max, row_logZ, temperature,
          ell, ws);
      tiles = true;
    }
  }
  if (!tiles) {
    {
      TraceScope tp("verify_plan_kernel", stream);
      verify_plan_kernel<<<dim3((B + 255) / 256), dim3(256), 0, stream>>>(B, gamma, V, ell,
                                                                          temperature, anchor,
                                                                          tokens, ws);
    }
    TraceScope t2("verify_final_stats_kernel", stream);
    verify_final_stats_kernel<T, KS><<<dim3(n_tiles(V)), dim3(256), 0, stream>>>(
        B, gamma, V, rank, target, U, W1, W2, anchor, tokens, row_max, row_logZ, temperature,
        ell, ws, status);
  }
  TraceScope t3("verify_finish_kernel", stream);
  verify_finish_kernel<T, KS><<<dim3(B), dim3(256), 0, stream>>>(
      B, gamma, V, rank, target, U, W1, W2, anchor, tokens, row_max, row_logZ, temperature,
      uniforms, ell, ws, out_tokens, n_accepted, ratio, status);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int gamma, int V, int rank, int dtype, const void* target,
                         const void* U, const void* W1, const void* W2, const int32_t* anchor,
                         const int32_t* tokens, const float* q_tok, const float* row_max,
                         const float* row_logZ, const float* temperature, const float* uniforms,
                         const int32_t* ell, int32_t* out_tokens, int32_t* n_accepted,
                         float* ratio, int32_t* status, void* ws, hipStream_t stream,
                         bool emb_rows) {
  if (dtype == DSPARK_BF16) {
    auto* tg = static_cast<const uint16_t*>(target);
    auto* u = static_cast<const uint16_t*>(U);
    auto* w1 = static_cast<const uint16_t*>(W1);
    auto* w2 = static_cast<const uint16_t*>(W2);
#define DSPARK_VERIFY_KS(KS)                                                                  \
  return verify_impl<uint16_t, KS>(B, gamma, V, rank, tg, u, w1, w2, anchor, tokens, q_tok,    \
                                   row_max, row_logZ, temperature, uniforms, ell, out_tokens,  \
                                   n_accepted, ratio, status, ws, stream, emb_rows)
    switch (rank) {
      case 32: DSPARK_VERIFY_KS(2);
      case 64: DSPARK_VERIFY_KS(4);
      case 128: DSPARK_VERIFY_KS(8);
      default: DSPARK_VERIFY_KS(16);
    }
#undef DSPARK_VERIFY_KS
  }
  return verify_impl<float, 1>(B, gamma, V, rank, static_cast<const float*>(target),
                               static_cast<const float*>(U), static_cast<const float*>(W1),
                               static_cast<const float*>(W2), anchor, tokens, q_tok, row_max,
                               row_logZ, temperature, uniforms, ell, out_tokens, n_accepted, ratio,
                               status, ws, stream, emb_rows);
}

}  // namespace dspark
