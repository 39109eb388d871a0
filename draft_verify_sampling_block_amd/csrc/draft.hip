// dspark_draft_block kernels: sequential Markov-head sampling over a block.
//
// [billytse] 3.2-3.3: position k's distribution is softmax(U_k + W1[prev] W2)
// where prev is the token sampled at position k-1 (the anchor for k = 0);
// positions are sampled left to right.  [weigao] part 2: rank-r factors.
//
// Per position k two launches:
//   draft_stats_kernel   vocabulary-parallel: one work-group per 128-entry
//                        vocabulary tile stages the tile's W2t rows in LDS
//                        (DMA), and each wave takes 32-request blocks: bias
//                        tile on the matrix cores, streamed base logits added,
//                        per-tile max / argmax and per-64-entry-chunk sums of
//                        exp(y - tile max) written out.
//   draft_sample_kernel  request-parallel: combines the tile statistics in
//                        fp64, finds the chunk where the cumulative mass
//                        crosses u * Z, recomputes that one chunk
//                        bit-identically, and picks the token.
#include <type_traits>

#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "trace.hpp"

namespace dspark {

template <typename T>
constexpr bool kIsBf16 = std::is_same<T, uint16_t>::value;

// Per-lane state of one 32-request block: A operand, streamed logits and
// the lane's own row token / inverse temperature.
template <typename T, int KS>
struct BlockIn {
  bf16x8_t afrag[KS];
  raw4_t<T> up[16];
  int tok;
  float itc;
};

template <typename T, int KS>
__device__ inline void block_prefetch(BlockIn<T, KS>& in, int rb, int B, int gamma, int V, int k,
                                      int vt, const T* __restrict__ U, const T* __restrict__ W1,
                                      const int32_t* __restrict__ prev_src, int prev_stride,
                                      const float* __restrict__ temperature, int32_t* status) {
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const int bc = rb * kTileM + c;
  in.tok = -1;
  in.itc = 0.f;
  if (bc < B) {
    in.tok = clamp_token(prev_src[(size_t)bc * prev_stride], V, h == 0 ? status : nullptr);
    const float Tb = temperature[bc];
    in.itc = (Tb > 0.f) ? 1.f / Tb : 0.f;
  }
  if constexpr (kIsBf16<T>) load_afrag<KS>(W1, in.tok, in.afrag);
  const int vb = vt * kTileV + 4 * c;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int b = rb * kTileM + acc_row(j, h);
    in.up[j] = (b < B && vb < V) ? load4_raw(U + ((size_t)b * gamma + k) * V + vb) : raw4_t<T>{};
  }
}

template <typename T, int KS>
__global__ __launch_bounds__(256) void draft_stats_kernel(
    int B, int gamma, int V, int rank, int k, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2t, const int32_t* __restrict__ prev_src, int prev_stride,
    const float* __restrict__ temperature, float* __restrict__ tile_max,
    int32_t* __restrict__ tile_arg, float* __restrict__ chunk_sum, int32_t* status) {
  __shared__ __attribute__((aligned(16))) char w2s[kIsBf16<T> ? kLdsTileBytes : 16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nRB = (B + kTileM - 1) / kTileM;
  const int nT = n_tiles(V), nC = n_chunks(V);
  const int vt = blockIdx.x, v0 = vt * kTileV;

  if constexpr (kIsBf16<T>) stage_w2_rows(W2t, v0, V, rank, w2s, 0, kTileV);
  BlockIn<T, KS> in;
  int rb = wave;
  if (rb < nRB)
    block_prefetch<T, KS>(in, rb, B, gamma, V, k, vt, U, W1, prev_src, prev_stride, temperature,
                          status);
  if constexpr (kIsBf16<T>) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int vb = v0 + 4 * c;
  const bool vok = vb < V;
  while (rb < nRB) {
    f32x16_t acc[kSub];
    if constexpr (kIsBf16<T>)
      bias_tile_lds<KS>(in.afrag, w2s, 0, 32, acc);
    else
      bias_tile_f32(reinterpret_cast<const float*>(W1), in.tok, reinterpret_cast<const float*>(W2t),
                    v0, V, rank, 0, 32, acc);
    // does any row of this block sample greedily (needs the argmax)?
    const bool any_greedy = __ballot((rb * kTileM + c < B) && !(in.itc > 0.f)) != 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = acc_row(j, h);
      const int b = rb * kTileM + m;
      const bool bok = b < B;
      const float it = __shfl(in.itc, m, kWave);
      const float scale = (it > 0.f) ? it : 1.f;
      float y[4];
      unpack4(in.up[j], y);
#pragma unroll
      for (int t = 0; t < kSub; ++t) y[t] = (bok && vok) ? (y[t] + acc[t][j]) * scale : -INFINITY;
      float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      int arg = 0x7fffffff;
      if (any_greedy) {
#pragma unroll
        for (int t = kSub - 1; t >= 0; --t)
          if (y[t] == mx) arg = vb + t;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) arg = min(arg, __shfl_xor(arg, o, kWave));
      }
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < kSub; ++t) s += __expf(y[t] - mx);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, kWave);
      if (bok) {
        if (c == 0) {
          tile_max[(size_t)b * nT + vt] = mx;
          tile_arg[(size_t)b * nT + vt] = arg;
        }
        if ((c & 15) == 0) chunk_sum[(size_t)b * nC + vt * kChunksPerTile + (c >> 4)] = s;
      }
    }
    rb += 4;
    if (rb < nRB)
      block_prefetch<T, KS>(in, rb, B, gamma, V, k, vt, U, W1, prev_src, prev_stride,
                            temperature, status);
  }
}

template <typename T, int KS>
__global__ __launch_bounds__(256) void draft_sample_kernel(
    int B, int gamma, int V, int rank, int k, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2t, const int32_t* __restrict__ prev_src, int prev_stride,
    const float* __restrict__ temperature, const float* __restrict__ uniforms,
    const float* __restrict__ tile_max, const int32_t* __restrict__ tile_arg,
    const float* __restrict__ chunk_sum, int32_t* __restrict__ tokens, float* __restrict__ q_tok,
    float* __restrict__ row_max, float* __restrict__ row_logZ, int32_t* status) {
  __shared__ __attribute__((aligned(16))) char w2s[kIsBf16<T> ? kLdsTileBytes : 16];
  __shared__ double red[8];
  __shared__ int s_chunk;
  __shared__ double s_before, s_scale;
  __shared__ float se[kChunk];

  const int b = blockIdx.x, tid = threadIdx.x;
  const int nT = n_tiles(V), nC = n_chunks(V);
  const float* tm = tile_max + (size_t)b * nT;
  const float Tb = temperature[b];
  const bool greedy = !(Tb > 0.f);
  const size_t out = (size_t)b * gamma + k;

  float m = -INFINITY;
  for (int t = tid; t < nT; t += blockDim.x) m = fmaxf(m, tm[t]);
  m = block_max(m, red);

  if (greedy) {
    int a = 0x7fffffff;
    for (int t = tid; t < nT; t += blockDim.x)
      if (tm[t] == m) a = min(a, tile_arg[(size_t)b * nT + t]);
    a = block_min_int(a, red);
    if (tid == 0) {
      if (!(m == m) || a < 0 || a >= V) {  // NaN logits leave no argmax
        flag(status, DSPARK_DEV_NONFINITE);
        a = 0;
      }
      tokens[out] = a;
      q_tok[out] = 1.f;
      row_max[out] = m;
      row_logZ[out] = 0.f;
    }
    return;
  }

  // fp64 mass of each thread's contiguous range of chunks
  const int per = (nC + blockDim.x - 1) / blockDim.x;
  const int c0 = min(nC, tid * per), c1 = min(nC, c0 + per);
  const float* cs = chunk_sum + (size_t)b * nC;
  const double md = (double)m;
  double local = 0.0;
  {
    int tcur = -1;
    double sc_t = 0.0;
    for (int cc = c0; cc < c1; ++cc) {
      const int t = cc / kChunksPerTile;
      if (t != tcur) { tcur = t; sc_t = exp((double)tm[t] - md); }
      local += (double)cs[cc] * sc_t;
    }
  }
  double start, end;
  const double Z = block_scan_interval(local, red, &start, &end);
  const double u = (double)uniforms[((size_t)b * (gamma + 1) + k) * 2 + 0];
  const double target = u * Z;
  const bool finite = isfinite(m) && isfinite(Z) && Z > 0.0;
  const int last_pos = block_max_int(local > 0.0 ? tid : -1, red);

  if (tid == 0) s_chunk = -1;
  __syncthreads();
  if (finite && local > 0.0 &&
      ((start <= target && target < end) || (tid == last_pos && target >= end))) {
    double run = start;
    int found = -1, lastc = -1;
    double before = start, lastb = start;
    int tcur = -1;
    double sc_t = 0.0;
    for (int cc = c0; cc < c1; ++cc) {
      const int t = cc / kChunksPerTile;
      if (t != tcur) { tcur = t; sc_t = exp((double)tm[t] - md); }
      const double sc = (double)cs[cc] * sc_t;
      if (sc > 0.0) { lastc = cc; lastb = run; }
      if (sc > 0.0 && target < run + sc) { found = cc; before = run; break; }
      run += sc;
    }
    if (found < 0) { found = lastc; before = lastb; }
    s_chunk = found;
    s_before = before;
    s_scale = exp((double)tm[found / kChunksPerTile] - md);
  }
  __syncthreads();
  const int cstar = s_chunk;
  if (!finite || cstar < 0) {
    if (tid == 0) {
      flag(status, DSPARK_DEV_NONFINITE);
      tokens[out] = 0;
      q_tok[out] = 0.f;
      row_max[out] = m;
      row_logZ[out] = (float)log(Z);
    }
    return;
  }

  // recompute the crossing chunk exactly as draft_stats_kernel computed it
  const int vt = cstar / kChunksPerTile, q = cstar % kChunksPerTile;
  const int v0 = vt * kTileV;
  const int mrow = b % kTileM;
  const int prev = clamp_token(prev_src[(size_t)b * prev_stride], V, nullptr);
  const int lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int c_lo = 16 * q, c_hi = 16 * q + 16;
  const bool mine = tid < kWave && h == row_half(mrow) && c >= c_lo && c < c_hi;
  const int vb = v0 + 4 * c;
  raw4_t<T> uraw = raw4_t<T>{};
  if (mine && vb < V) uraw = load4_raw(U + out * V + vb);
  f32x16_t acc[kSub];
  if constexpr (kIsBf16<T>) {
    stage_w2_rows(W2t, v0, V, rank, w2s, kChunk * q, kChunk);
    bf16x8_t afrag[KS];
    if (tid < kWave) load_afrag<KS>(W1, c == mrow ? prev : -1, afrag);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid < kWave) bias_tile_lds<KS>(afrag, w2s, c_lo, c_hi, acc);
  } else {
    if (tid < kWave)
      bias_tile_f32(reinterpret_cast<const float*>(W1), c == mrow ? prev : -1,
                    reinterpret_cast<const float*>(W2t), v0, V, rank, c_lo, c_hi, acc);
  }
  if (mine) {
    const int jm = row_elem(mrow);
    const float scale = 1.f / Tb;
    const float tmax = tm[vt];
    float y[4];
    unpack4(uraw, y);
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
      const float yy = (vb < V) ? (y[t] + acc[t][jm]) * scale : -INFINITY;
      se[(c - c_lo) * kSub + t] = __expf(yy - tmax);
    }
  }
  __syncthreads();
  if (tid == 0) {
    const double r = (target - s_before) / s_scale;
    double run = 0.0;
    int pick = -1, lastp = -1;
    for (int i = 0; i < kChunk; ++i) {
      const double e = (double)se[i];
      if (e > 0.0) lastp = i;
      run += e;
      if (e > 0.0 && r < run) { pick = i; break; }
    }
    if (pick < 0) pick = lastp < 0 ? 0 : lastp;
    const int x = v0 + q * kChunk + pick;
    tokens[out] = x;
    q_tok[out] = (float)((double)se[pick] * s_scale / Z);
    row_max[out] = m;
    row_logZ[out] = (float)log(Z);
  }
}

size_t draft_workspace_bytes(int B, int gamma, int V, int rank, int dtype) {
  (void)gamma; (void)rank; (void)dtype;
  size_t nT = n_tiles(V), nC = n_chunks(V);
  return align256((size_t)B * nT * 4) * 2 + align256((size_t)B * nC * 4);
}

template <typename T, int KS>
static hipError_t draft_impl(int B, int gamma, int V, int rank, const T* U, const T* W1,
                             const T* W2t, const int32_t* anchor, const float* temperature,
                             const float* uniforms, int32_t* tokens, float* q_tok, float* row_max,
                             float* row_logZ, int32_t* status, void* ws, hipStream_t stream) {
  const size_t nT = n_tiles(V);
  char* w = static_cast<char*>(ws);
  float* tile_max = reinterpret_cast<float*>(w);
  int32_t* tile_arg = reinterpret_cast<int32_t*>(w + align256((size_t)B * nT * 4));
  float* chunk_sum = reinterpret_cast<float*>(w + 2 * align256((size_t)B * nT * 4));
  const dim3 blk(256);
  for (int k = 0; k < gamma; ++k) {
    const int32_t* prev = (k == 0) ? anchor : tokens + (k - 1);
    const int stride = (k == 0) ? 1 : gamma;
    {
      TraceScope ts("draft_stats_kernel", stream);
      draft_stats_kernel<T, KS><<<dim3((unsigned)nT), blk, 0, stream>>>(
          B, gamma, V, rank, k, U, W1, W2t, prev, stride, temperature, tile_max, tile_arg,
          chunk_sum, status);
    }
    TraceScope ts("draft_sample_kernel", stream);
    draft_sample_kernel<T, KS><<<dim3(B), blk, 0, stream>>>(
        B, gamma, V, rank, k, U, W1, W2t, prev, stride, temperature, uniforms, tile_max, tile_arg,
        chunk_sum, tokens, q_tok, row_max, row_logZ, status);
  }
  return hipGetLastError();
}

hipError_t launch_draft_block(int B, int gamma, int V, int rank, int dtype, const void* U,
                              const void* W1, const void* W2t, const int32_t* anchor,
                              const float* temperature, const float* uniforms, int32_t* tokens,
                              float* q_tok, float* row_max, float* row_logZ, int32_t* status,
                              void* ws, hipStream_t stream) {
  if (dtype == DSPARK_BF16) {
    auto* u = static_cast<const uint16_t*>(U);
    auto* w1 = static_cast<const uint16_t*>(W1);
    auto* w2 = static_cast<const uint16_t*>(W2t);
#define DSPARK_DRAFT_KS(KS)                                                                   \
  return draft_impl<uint16_t, KS>(B, gamma, V, rank, u, w1, w2, anchor, temperature, uniforms, \
                                  tokens, q_tok, row_max, row_logZ, status, ws, stream)
    switch (rank) {
      case 32: DSPARK_DRAFT_KS(2);
      case 64: DSPARK_DRAFT_KS(4);
      case 128: DSPARK_DRAFT_KS(8);
      default: DSPARK_DRAFT_KS(16);
    }
#undef DSPARK_DRAFT_KS
  }
  return draft_impl<float, 1>(B, gamma, V, rank, static_cast<const float*>(U),
                              static_cast<const float*>(W1), static_cast<const float*>(W2t),
                              anchor, temperature, uniforms, tokens, q_tok, row_max, row_logZ,
                              status, ws, stream);
}

}  // namespace dspark
