// dspark_tv_label kernels: per drafted position, the total variation between
// the draft and target distributions and the acceptance label 1 - TV.
//
// [weigao] part 3 (the confidence head's training target) and [billytse]
// 5.1: c*_k = 1 - 0.5 * ||p^d_k - p^t_k||_1, which equals the probability
// that the accept-or-resample test keeps drafted token k.  The draft
// distribution of position k is softmax((U[b,k] + W1[prev] W2) / T) with
// prev the anchor or drafted token k-1 (the distribution token k was drawn
// from); the target one is softmax(target[b,k] / T).  Greedy requests
// (T <= 0): one-hot q at the drafted token, one-hot p at the target's
// lowest-index argmax, label 1 when they agree.
//
// Launches:
//   tv_rows_kernel    one work-group per (request, position): target-row
//                     max / log-sum-exp / argmax (shared row_stats).
//   tv_tile_kernel    one work-group per 64-entry vocabulary tile, waves over
//                     (32-request block, position) tasks: the draft logits
//                     are recomputed exactly as the draft computed them (base
//                     logits + Markov bias on the matrix cores, W2 tile in
//                     LDS) and normalised with the draft's stored row max and
//                     log-sum-exp; each request's |p - q| over the tile goes
//                     to a per-(row, tile) partial.
//   tv_finish_kernel  one wave per row: fp64 sum of the partials.
#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "row_stats.hpp"
#include "trace.hpp"
#include "tv_launch.hpp"

namespace dspark {

namespace {

struct TvWs {
  float* M;       // [B*gamma] target row max of t/T (max t when greedy)
  float* LZ;      // [B*gamma] log sum exp(t/T - M)
  int32_t* arg;   // [B*gamma] lowest argmax of the target row
  float* part;    // [B*gamma][nT] sum over the tile of |p - q|
};

TvWs carve_tv(void* ws, int B, int gamma, int V) {
  char* p = static_cast<char*>(ws);
  const size_t rows = (size_t)B * gamma;
  TvWs w;
  w.M = reinterpret_cast<float*>(p); p += align256(rows * 4);
  w.LZ = reinterpret_cast<float*>(p); p += align256(rows * 4);
  w.arg = reinterpret_cast<int32_t*>(p); p += align256(rows * 4);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

__device__ inline float tv_inv_temp(float T) { return (T > 0.f) ? 1.f / T : 0.f; }

}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void tv_rows_kernel(int B, int gamma, int V,
                                                      const T* __restrict__ target,
                                                      const float* __restrict__ temperature,
                                                      TvWs ws, int32_t* status) {
  __shared__ double red[8];
  const int row = blockIdx.x;   // b * gamma + k
  const int b = row / gamma, k = row - b * gamma;
  const float it = tv_inv_temp(temperature[b]);
  const bool greedy = !(it > 0.f);
  const RowStats rs = row_stats<T>(target + ((size_t)b * (gamma + 1) + k) * V, V,
                                   greedy ? 1.f : it, greedy, red);
  if (threadIdx.x == 0) {
    const bool fin = (rs.M == rs.M) && rs.M > -INFINITY && rs.M < INFINITY &&
                     (greedy || (rs.Z > 0.0 && rs.Z < INFINITY));
    if (!fin) flag(status, DSPARK_DEV_NONFINITE);
    ws.M[row] = rs.M;
    ws.LZ[row] = greedy ? 0.f : (float)log(rs.Z);
    ws.arg[row] = (rs.arg >= 0 && rs.arg < V) ? rs.arg : 0;
  }
}

// One work-group (4 waves) per tile vt; task t = (request block t / gamma,
// position t % gamma).  Lane column c is request b of the block; h picks the
// lane's 16-entry halves, as in the draft's block-tiles.
//
// bf16: a wave loads its task's 32 target rows and 32 base-logit rows of the
// tile as whole 128-byte rows (8 rows per instruction) two tasks ahead, with
// the lane's temperature and previous token, and passes the entries to the
// matrix layout through its own 4 KB of LDS (16-byte pieces swizzled by row).
// A load whose lanes each take a piece of another row (32 rows per
// instruction) moves about half as many bytes per second on this chip.  The
// rows of greedy requests are read too (their temperatures are not known
// when the loads issue; their lanes discard them).
constexpr int kTvStageBytes = kTileM * 128;
// (two work-groups per compute unit: two waves per SIMD)
template <typename T, int KS>
__global__ __launch_bounds__(256, 2) void tv_tile_kernel(
    int B, int gamma, int V, int rank, const T* __restrict__ target, const T* __restrict__ U,
    const T* __restrict__ W1, const T* __restrict__ W2, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ row_max,
    const float* __restrict__ row_logZ, const float* __restrict__ temperature, TvWs ws) {
  constexpr bool bf = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) char w2s[bf ? kLdsTileBytes : 16];
  __shared__ __attribute__((aligned(16))) char s_stg[bf ? 4 : 1][bf ? kTvStageBytes : 16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nRB = (B + kTileM - 1) / kTileM;
  const int nT = n_tiles(V);
  const int vt = blockIdx.x, v0 = vt * kTileV;
  const int ntask = nRB * gamma;

  if constexpr (bf) stage_tile(reinterpret_cast<const uint16_t*>(W2), v0, V, rank, w2s);

  // the label partial of the lane's request over this tile (acc: its draft
  // logits, tp: its target entries)
  auto finish_task = [&](int b, int k, float it, bool sampled, const URow<T>& tp,
                         const f32x16_t (&acc)[kSub]) {
    float s = 0.f;
    if (sampled) {
      const size_t row = (size_t)b * gamma + k;
      const float M = ws.M[row], LZ = ws.LZ[row];
      const float mq = row_max[row], lzq = row_logZ[row];
      // exp(y / T - M - log Z) as 2^(y (log2 e / T) - (M + log Z) log2 e):
      // one fused multiply-add and the hardware base-2 exponential per term
      constexpr float kLog2e = 1.4426950408889634f;
      const float a = it * kLog2e;
      const float cp = (M + LZ) * kLog2e, cq = (mq + lzq) * kLog2e;
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        const int rem = V - (v0 + 32 * st + 16 * h);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < rem) {
            const float p = __builtin_amdgcn_exp2f(fmaf(urow_at(tp, st, j), a, -cp));
            const float q = __builtin_amdgcn_exp2f(fmaf(acc[st][j], a, -cq));
            s += fabsf(p - q);
          }
        }
      }
    }
    float lo, hi;
    half_pair(s, lo, hi);
    if (sampled && h == 0) ws.part[((size_t)b * gamma + k) * nT + vt] = lo + hi;
  };

  if constexpr (bf) {
    const uint16_t* tg = reinterpret_cast<const uint16_t*>(target);
    const uint16_t* ub = reinterpret_cast<const uint16_t*>(U);
    const int lr = lane >> 3, lp = lane & 7;   // loads: block row 8 j + lr, piece lp
    char* stg = s_stg[wave];
    // task tt's rows: u32x4 j < 4 target, j >= 4 base logits, row 8 (j % 4) + lr
    auto fetch = [&](u32x4_t (&ld)[8], int tt) {
      const bool lv = tt < ntask;
      const int rb = lv ? tt / gamma : 0, k = lv ? tt - rb * gamma : 0;
      const int e = v0 + 8 * lp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = rb * kTileM + 8 * j + lr;
        const bool on = lv && r < B && e < V;
        ld[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            on ? tg + ((size_t)r * (gamma + 1) + k) * V + e : tg));
        ld[4 + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            on ? ub + ((size_t)r * gamma + k) * V + e : ub));
      }
    };
    // the lane's request of task tt: temperature and previous token
    auto head = [&](int tt, float& temp, int& tok) {
      temp = 0.f;
      tok = 0;
      if (tt < ntask) {
        const int rb = tt / gamma, k = tt - rb * gamma;
        const int b = rb * kTileM + c;
        if (b < B) {
          temp = temperature[b];
          tok = k == 0 ? anchor[b] : tokens[(size_t)b * gamma + k - 1];
        }
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

    // task t of this wave: its entries in ld, its temperature and previous
    // token in temp_n / tok_n; those of task t + 8 are requested in their
    // place (two tasks in flight per wave).  False once the wave is done.
    auto task = [&](int t, u32x4_t (&ld)[8], float& temp_n, int& tok_n) {
      // the first pass of every wave also joins the barrier that publishes
      // the LDS tile
      const bool live = t < ntask;
      const int rb = live ? t / gamma : 0, k = live ? t - rb * gamma : 0;
      const int b = rb * kTileM + c;
      const bool in = live && b < B;
      const float it = in ? tv_inv_temp(temp_n) : 0.f;
      const bool sampled = in && it > 0.f;   // greedy rows need no stream
      const int prev = sampled ? clamp_token(tok_n, V, nullptr) : -1;
      bf16x8_t bfrag[KS];
      load_bfrag<KS>(reinterpret_cast<const uint16_t*>(W1), prev, bfrag);
      URow<uint16_t> tp, up;
      restage(ld, tp, up);
      head(t + 8, temp_n, tok_n);
      fetch(ld, t + 8);
      if (t == wave) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      if (!live) return false;
      f32x16_t acc[kSub];
      init_acc<uint16_t>(up, V - (v0 + 16 * h), acc);   // draft logits start at the base logits
      if (__ballot(sampled) != 0)
        bias_tile_ldsA<KS>([&](int ks) { return bfrag[ks]; }, w2s, acc);
      finish_task(b, k, it, sampled, tp, acc);
      return true;
    };
    u32x4_t ldA[8], ldB[8];
    float tA, tB;
    int kA, kB;
    head(wave, tA, kA);
    fetch(ldA, wave);
    head(wave + 4, tB, kB);
    fetch(ldB, wave + 4);
    for (int t = wave;; t += 8) {
      if (!task(t, ldA, tA, kA)) break;
      if (!task(t + 4, ldB, tB, kB)) break;
    }
  } else {
    for (int t = wave; t < ntask; t += 4) {
      const int rb = t / gamma, k = t - rb * gamma;
      const int b = rb * kTileM + c;
      const bool in = b < B;
      const float it = in ? tv_inv_temp(temperature[b]) : 0.f;
      const bool sampled = in && it > 0.f;
      int prev = -1;
      if (sampled)
        prev = clamp_token(k == 0 ? anchor[b] : tokens[(size_t)b * gamma + k - 1], V, nullptr);
      URow<T> tp, up;
      load_urow<T>(tp, target + ((size_t)b * (gamma + 1) + k) * V, v0, V, sampled, target);
      load_urow<T>(up, U + ((size_t)b * gamma + k) * V, v0, V, sampled, U);
      f32x16_t acc[kSub];
      init_acc<T>(up, V - (v0 + 16 * h), acc);
      if (__ballot(sampled) != 0)
        bias_tile_f32(reinterpret_cast<const float*>(W1), prev,
                      reinterpret_cast<const float*>(W2), v0, V, rank, acc);
      finish_task(b, k, it, sampled, tp, acc);
    }
  }
}

__global__ __launch_bounds__(256) void tv_finish_kernel(int B, int gamma, int V,
                                                        const int32_t* __restrict__ tokens,
                                                        const float* __restrict__ temperature,
                                                        TvWs ws, float* __restrict__ tv,
                                                        float* __restrict__ label) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= B * gamma) return;   // wave-uniform
  const int b = row / gamma;
  const int nT = n_tiles(V);
  float d;
  if (!(temperature[b] > 0.f)) {
    d = (tokens[row] == ws.arg[row]) ? 0.f : 1.f;
  } else {
    double acc = 0.0;
    for (int t = lane; t < nT; t += kWave) acc += (double)ws.part[(size_t)row * nT + t];
    acc = wave_sum(acc);
    d = (float)(0.5 * acc);
  }
  if (lane == 0) {
    tv[row] = d;
    if (label) label[row] = 1.f - d;
  }
}

size_t tv_workspace_bytes(int B, int gamma, int V) {
  const size_t rows = (size_t)B * gamma;
  return 3 * align256(rows * 4) + align256(rows * (size_t)n_tiles(V) * 4);
}

template <typename T, int KS>
static hipError_t tv_impl(int B, int gamma, int V, int rank, const T* target, const T* U,
                          const T* W1, const T* W2, const int32_t* anchor, const int32_t* tokens,
                          const float* row_max, const float* row_logZ, const float* temperature,
                          float* tv, float* label, int32_t* status, void* wsp,
                          hipStream_t stream) {
  const TvWs ws = carve_tv(wsp, B, gamma, V);
  {
    TraceScope t1("tv_rows_kernel", stream);
    tv_rows_kernel<T><<<dim3(B * gamma), dim3(256), 0, stream>>>(B, gamma, V, target,
                                                                 temperature, ws, status);
  }
  {
    TraceScope t2("tv_tile_kernel", stream);
    tv_tile_kernel<T, KS><<<dim3(n_tiles(V)), dim3(256), 0, stream>>>(
        B, gamma, V, rank, target, U, W1, W2, anchor, tokens, row_max, row_logZ, temperature,
        ws);
  }
  TraceScope t3("tv_finish_kernel", stream);
  tv_finish_kernel<<<dim3((B * gamma + 3) / 4), dim3(256), 0, stream>>>(B, gamma, V, tokens,
                                                                         temperature, ws, tv,
                                                                         label);
  return hipGetLastError();
}

hipError_t launch_tv_label(int B, int gamma, int V, int rank, int dtype, const void* target,
                           const void* U, const void* W1, const void* W2,
                           const int32_t* anchor, const int32_t* tokens, const float* row_max,
                           const float* row_logZ, const float* temperature, float* tv,
                           float* label, int32_t* status, void* ws, hipStream_t stream) {
  if (dtype == DSPARK_BF16) {
    auto* tg = static_cast<const uint16_t*>(target);
    auto* u = static_cast<const uint16_t*>(U);
    auto* w1 = static_cast<const uint16_t*>(W1);
    auto* w2 = static_cast<const uint16_t*>(W2);
#define DSPARK_TV_KS(KS)                                                                    \
  return tv_impl<uint16_t, KS>(B, gamma, V, rank, tg, u, w1, w2, anchor, tokens, row_max,    \
                               row_logZ, temperature, tv, label, status, ws, stream)
    switch (rank) {
      case 32: DSPARK_TV_KS(2);
      case 64: DSPARK_TV_KS(4);
      case 128: DSPARK_TV_KS(8);
      default: DSPARK_TV_KS(16);
    }
#undef DSPARK_TV_KS
  }
  return tv_impl<float, 1>(B, gamma, V, rank, static_cast<const float*>(target),
                           static_cast<const float*>(U), static_cast<const float*>(W1),
                           static_cast<const float*>(W2), anchor, tokens, row_max, row_logZ,
                           temperature, tv, label, status, ws, stream);
}

}  // namespace dspark
