// dspark_draft_block kernels: sequential Markov-head sampling over a block.
//
// [billytse] 3.2-3.3: position k's distribution is softmax(U_k + W1[prev] W2)
// where prev is the token sampled at position k-1 (the anchor for k = 0);
// positions are sampled left to right.  [weigao] part 2: rank-r factors.
//
// Per position k two launches:
//   draft_stats_kernel   vocabulary-parallel: for every (32-request block,
//                        256-entry vocabulary tile) one wave computes the bias
//                        tile on the matrix cores, adds the streamed base
//                        logits, and writes per-tile max / argmax and
//                        per-64-entry-chunk sums of exp(y - tile max).
//   draft_sample_kernel  request-parallel: combines the tile statistics in
//                        fp64, finds the chunk where the cumulative mass
//                        crosses u * Z, recomputes that one chunk
//                        bit-identically, and picks the token.
#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "trace.hpp"

namespace dspark {

template <typename T>
__global__ __launch_bounds__(256) void draft_stats_kernel(
    int B, int gamma, int V, int rank, int k, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2t, const int32_t* __restrict__ prev_src, int prev_stride,
    const float* __restrict__ temperature, float* __restrict__ tile_max,
    int32_t* __restrict__ tile_arg, float* __restrict__ chunk_sum, int32_t* status) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nRB = (B + kTileM - 1) / kTileM;
  const int nT = n_tiles(V), nC = n_chunks(V);
  const int task = blockIdx.x * 4 + wave;
  const bool active = task < nT * nRB;
  const int vt = active ? task / nRB : 0, rb = active ? task % nRB : 0;
  const int v0 = vt * kTileV;

  __shared__ int sprev[4][kTileM];
  __shared__ float sinvT[4][kTileM];
  if (h == 0) {
    int b = rb * kTileM + c;
    int p = -1;
    float it = 0.f;
    if (active && b < B) {
      p = clamp_token(prev_src[(size_t)b * prev_stride], V, status);
      float Tb = temperature[b];
      it = (Tb > 0.f) ? 1.f / Tb : 0.f;
    }
    sprev[wave][c] = p;
    sinvT[wave][c] = it;
  }
  __syncthreads();
  if (!active) return;

  f32x16_t acc[8];
  bias_tile<T>(W1, sprev[wave], W2t, v0, V, rank, 0, 32, acc);

  // does any row of this block sample greedily (needs the argmax)?
  bool any_greedy = false;
  for (int m = 0; m < kTileM; ++m)
    any_greedy |= (rb * kTileM + m < B) && !(sinvT[wave][m] > 0.f);

  const int vb = v0 + 8 * c;
  const bool vok = vb < V;
#pragma unroll 4
  for (int j = 0; j < 16; ++j) {
    const int m = acc_row(j, h);
    const int b = rb * kTileM + m;
    const bool bok = b < B;
    const float it = sinvT[wave][m];
    const float scale = (it > 0.f) ? it : 1.f;
    float y[8];
    if (bok && vok) {
      load8_f32_stream(U + ((size_t)b * gamma + k) * V + vb, y);
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = (y[t] + acc[t][j]) * scale;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = -INFINITY;
    }
    float mx = y[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) mx = fmaxf(mx, y[t]);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    int arg = 0x7fffffff;
    if (any_greedy) {
#pragma unroll
      for (int t = 7; t >= 0; --t)
        if (y[t] == mx) arg = vb + t;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) arg = min(arg, __shfl_xor(arg, o, kWave));
    }
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) s += __expf(y[t] - mx);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) s += __shfl_xor(s, o, kWave);
    if (bok) {
      if (c == 0) {
        tile_max[(size_t)b * nT + vt] = mx;
        tile_arg[(size_t)b * nT + vt] = arg;
      }
      if ((c & 7) == 0) chunk_sum[(size_t)b * nC + vt * kChunksPerTile + (c >> 3)] = s;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void draft_sample_kernel(
    int B, int gamma, int V, int rank, int k, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2t, const int32_t* __restrict__ prev_src, int prev_stride,
    const float* __restrict__ temperature, const float* __restrict__ uniforms,
    const float* __restrict__ tile_max, const int32_t* __restrict__ tile_arg,
    const float* __restrict__ chunk_sum, int32_t* __restrict__ tokens, float* __restrict__ q_tok,
    float* __restrict__ row_max, float* __restrict__ row_logZ, int32_t* status) {
  __shared__ double red[8];
  __shared__ int s_chunk;
  __shared__ double s_before, s_scale;
  __shared__ int sprev[kTileM];
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
  for (int cc = c0; cc < c1; ++cc) local += (double)cs[cc] * exp((double)tm[cc >> 2] - md);
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
    for (int cc = c0; cc < c1; ++cc) {
      double sc = (double)cs[cc] * exp((double)tm[cc >> 2] - md);
      if (sc > 0.0) { lastc = cc; lastb = run; }
      if (sc > 0.0 && target < run + sc) { found = cc; before = run; break; }
      run += sc;
    }
    if (found < 0) { found = lastc; before = lastb; }
    s_chunk = found;
    s_before = before;
    s_scale = exp((double)tm[found >> 2] - md);
  }
  if (tid < kTileM) sprev[tid] = -1;
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
  const int vt = cstar >> 2, q = cstar & 3;
  const int mrow = b % kTileM;
  if (tid == 0) sprev[mrow] = clamp_token(prev_src[(size_t)b * prev_stride], V, status);
  __syncthreads();
  if (tid < kWave) {  // wave 0 recomputes the chunk exactly as draft_stats_kernel did
    const int lane = tid, c = lane & 31, h = lane >> 5;
    const int v0 = vt * kTileV;
    f32x16_t acc[8];
    bias_tile<T>(W1, sprev, W2t, v0, V, rank, 8 * q, 8 * q + 8, acc);
    const int hm = (mrow >> 2) & 1;
    const int jm = 4 * (mrow >> 3) + (mrow & 3);
    if (h == hm && c >= 8 * q && c < 8 * q + 8) {
      const int vb = v0 + 8 * c;
      const float scale = 1.f / Tb;
      const float tmax = tm[vt];
      float y[8];
      if (vb < V) {
        load8_f32(U + out * V + vb, y);
#pragma unroll
        for (int t = 0; t < 8; ++t) y[t] = (y[t] + acc[t][jm]) * scale;
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) y[t] = -INFINITY;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) se[(c - 8 * q) * 8 + t] = __expf(y[t] - tmax);
    }
  }
  __syncthreads();
  if (tid == 0) {
    const double r = (target - s_before) / s_scale;
    double run = 0.0;
    int pick = -1, lastp = -1;
    for (int i = 0; i < kChunk; ++i) {
      double e = (double)se[i];
      if (e > 0.0) lastp = i;
      run += e;
      if (e > 0.0 && r < run) { pick = i; break; }
    }
    if (pick < 0) pick = lastp < 0 ? 0 : lastp;
    const int x = vt * kTileV + q * kChunk + pick;
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

template <typename T>
static hipError_t draft_impl(int B, int gamma, int V, int rank, const T* U, const T* W1,
                             const T* W2t, const int32_t* anchor, const float* temperature,
                             const float* uniforms, int32_t* tokens, float* q_tok, float* row_max,
                             float* row_logZ, int32_t* status, void* ws, hipStream_t stream) {
  const size_t nT = n_tiles(V);
  char* w = static_cast<char*>(ws);
  float* tile_max = reinterpret_cast<float*>(w);
  int32_t* tile_arg = reinterpret_cast<int32_t*>(w + align256((size_t)B * nT * 4));
  float* chunk_sum = reinterpret_cast<float*>(w + 2 * align256((size_t)B * nT * 4));
  const int nRB = (B + kTileM - 1) / kTileM;
  const int tasks = (int)nT * nRB;
  const dim3 g1((tasks + 3) / 4), blk(256);
  for (int k = 0; k < gamma; ++k) {
    const int32_t* prev = (k == 0) ? anchor : tokens + (k - 1);
    const int stride = (k == 0) ? 1 : gamma;
    {
    TraceScope ts("draft_stats_kernel", stream);
    draft_stats_kernel<T><<<g1, blk, 0, stream>>>(B, gamma, V, rank, k, U, W1, W2t, prev, stride,
                                                  temperature, tile_max, tile_arg, chunk_sum,
                                                  status);
    }
    TraceScope ts("draft_sample_kernel", stream);
    draft_sample_kernel<T><<<dim3(B), blk, 0, stream>>>(
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
  if (dtype == DSPARK_BF16)
    return draft_impl<uint16_t>(B, gamma, V, rank, static_cast<const uint16_t*>(U),
                                static_cast<const uint16_t*>(W1),
                                static_cast<const uint16_t*>(W2t), anchor, temperature, uniforms,
                                tokens, q_tok, row_max, row_logZ, status, ws, stream);
  return draft_impl<float>(B, gamma, V, rank, static_cast<const float*>(U),
                           static_cast<const float*>(W1), static_cast<const float*>(W2t), anchor,
                           temperature, uniforms, tokens, q_tok, row_max, row_logZ, status, ws,
                           stream);
}

}  // namespace dspark
