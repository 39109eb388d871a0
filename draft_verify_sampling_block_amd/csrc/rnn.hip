// dspark_draft_block_rnn kernels: the RNN head's recurrence.
//
// [weigao] "DSpark 的核心设计" part 2 (the _rnn_step description): the
// previous state, the previous token's embedding and the position's hidden
// state pass through one linear layer whose output splits into gate,
// candidate and output; state_k = gate * state_{k-1} + (1 - gate) *
// candidate, and the position's bias is W2 applied to tanh(output).
// [billytse] 3.3: the recurrence lets each position see the whole block
// prefix.  Layer Wr [3r, 2r + H] (rows gate | candidate | output, columns
// state | embedding | hidden), bias br [3r]; gate = sigmoid, candidate and
// output = tanh; the state starts at zero in each block; the embedding of a
// token is its W1 row.
//
//  * rnn_hidden_kernel (once per call): P[b gamma + k, :] = Wr[:, 2r:] h[b,k]
//    + br for every position at once -- the hidden states do not depend on
//    the drafted tokens.  bf16: one dense GEMM on the matrix cores
//    (v_mfma_f32_32x32x16_bf16), fp32 out.
//  * rnn_state_kernel (per position k): pre = P[b gamma + k] + Wr[:, :r]
//    s_{k-1} + Wr[:, r:2r] W1[x_{k-1}], then the activations, the state update
//    and emb[b, k] = tanh(output) (rounded to the input dtype: the B operand
//    of the position's bias contraction).  bf16: a 32-row matrix block holds
//    the gate, candidate and output rows of 8 state elements in the order
//    that leaves each lane the three pre-activations of 4 elements of one
//    request, so the recurrence finishes in registers; the fp32 state enters
//    the contraction as two bf16 parts (hi + lo, ~2^-17 relative).
#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "trace.hpp"

namespace dspark {

namespace {

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// ---------------------------------------------------------------------------
// P = hidden . Wr[:, koff:]^T + br
// ---------------------------------------------------------------------------

// bf16: one work-group of 4 waves per 32 x 32 block of P; wave w takes the
// k-steps [w ks4, (w + 1) ks4) of the contraction (A = hidden rows m, B = Wr
// rows j, both 8 consecutive k per lane), requesting kHidUnroll steps'
// operands at a time; the four partial blocks are summed through LDS in wave
// order.  Accumulator lane (c, h): column j0 + c, rows m0 + 8 (i / 4) + 4 h +
// i % 4.
constexpr int kHidUnroll = 8;
__global__ __launch_bounds__(256) void rnn_hidden_kernel_bf16(
    int M, int N, int H, int ldw, int koff, const uint16_t* __restrict__ hidden,
    const uint16_t* __restrict__ Wr, const float* __restrict__ br, float* __restrict__ P) {
  __shared__ f32x16_t s_part[3][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const uint16_t* arow = hidden + (size_t)min(m0 + c, M - 1) * H;
  const uint16_t* brow = Wr + (size_t)min(j0 + c, N - 1) * ldw + koff;
  const bf16x8_t zero = bf16x8_t{};
  const int nks = (H + 15) / 16;
  const int ks4 = (nks + 3) / 4;
  const int kb = wave * ks4, ke = min(nks, kb + ks4);
  f32x16_t acc = {};
  for (int ks0 = kb; ks0 < ke; ks0 += kHidUnroll) {
    bf16x8_t a[kHidUnroll], b[kHidUnroll];
#pragma unroll
    for (int u = 0; u < kHidUnroll; ++u) {
      const int k = 16 * (ks0 + u) + 8 * h;   // H % 8 == 0: 8 entries wholly in or out
      const bool in = ks0 + u < ke && k < H;
      a[u] = in ? load_bf16x8(arow + k) : zero;
      b[u] = in ? load_bf16x8(brow + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < kHidUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
  }
  if (wave > 0) s_part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += s_part[w][lane];
  const int j = j0 + c;
  if (j >= N) return;
  const float bj = br[j];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (m < M) P[(size_t)m * N + j] = acc[i] + bj;
  }
}

// fp32: one thread per entry, k ascending
__global__ __launch_bounds__(256) void rnn_hidden_kernel_f32(
    int M, int N, int H, int ldw, int koff, const float* __restrict__ hidden,
    const float* __restrict__ Wr, const float* __restrict__ br, float* __restrict__ P) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= M * N) return;
  const int m = e / N, j = e - m * N;
  const float* a = hidden + (size_t)m * H;
  const float* w = Wr + (size_t)j * ldw + koff;
  float s = 0.f;
  for (int k = 0; k < H; ++k) s = fmaf(a[k], w[k], s);
  P[e] = s + br[j];
}

// ---------------------------------------------------------------------------
// One position of the recurrence
// ---------------------------------------------------------------------------

struct RnnPos {
  int B, gamma, rank, k, ldw;
  const float* P;          // [B gamma, 3r]
  const float* s_prev;     // [B, r]  (unused at k = 0: the state starts at zero)
  float* s_next;           // [B, r]
  float* state_out;        // [B, gamma, r] or NULL
  const int32_t* anchor;
  const int32_t* tokens;   // [B, gamma]: position k - 1's tokens
  int V;
};

// the three pre-activations of element `el` of request b finish here
__device__ inline void rnn_finish(const RnnPos& a, int b, int el, float pg, float pc, float po,
                                  void* emb, bool bf) {
  const int r = a.rank;
  const size_t row = (size_t)b * a.gamma + a.k;
  const float* Pr = a.P + row * 3 * r;
  pg += Pr[el];
  pc += Pr[r + el];
  po += Pr[2 * r + el];
  const float g = sigmoid_f(pg), cnd = tanhf(pc), o = tanhf(po);
  const float s_old = a.k > 0 ? a.s_prev[(size_t)b * r + el] : 0.f;
  const float s_new = g * s_old + (1.f - g) * cnd;
  a.s_next[(size_t)b * r + el] = s_new;
  if (a.state_out) a.state_out[row * r + el] = s_new;
  if (bf)
    static_cast<uint16_t*>(emb)[row * r + el] = f32_to_bf16_rne(o);
  else
    static_cast<float*>(emb)[row * r + el] = o;
}

// bf16: grid (r / 8 element groups, ceil(B / 32) request blocks), one
// work-group of 4 waves each.  Matrix row R of the block is part R / 8 (0
// gate, 1 candidate, 2 output, 3 unused) of element 8 g + R % 8; the
// contraction runs over K = 3r: the state's bf16 high parts, its low parts
// (both against the layer's state columns), then the embedding (W1 row of
// the previous token) against the embedding columns.  Wave w takes k-steps
// [w kPer, (w + 1) kPer) with all their operands requested at once; the four
// partial blocks are summed through LDS in wave order, and wave 0 finishes.
template <int KS>   // r = 16 KS
__global__ __launch_bounds__(256) void rnn_state_kernel_bf16(RnnPos a, const uint16_t* __restrict__ Wr,
                                                             const uint16_t* __restrict__ W1,
                                                             uint16_t* __restrict__ emb,
                                                             int32_t* status) {
  constexpr int r = 16 * KS;
  constexpr int nks = 3 * KS;
  constexpr int kPer = (nks + 3) / 4;
  __shared__ f32x16_t s_part[3][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const int g = blockIdx.x, rb = blockIdx.y;
  // A: matrix row c
  const int part = c >> 3, el_a = 8 * g + (c & 7);
  const bool arow_on = part < 3;
  const uint16_t* wrow = Wr + (size_t)(arow_on ? part * r + el_a : 0) * a.ldw;
  // B: request column c
  const int b = rb * kTileM + c;
  const bool bon = b < a.B;
  const int bb = bon ? b : 0;
  int prev = a.k == 0 ? a.anchor[bb] : a.tokens[(size_t)bb * a.gamma + a.k - 1];
  prev = clamp_token(prev, a.V, (bon && h == 0 && g == 0 && wave == 0) ? status : nullptr);
  const float* srow = a.s_prev + (size_t)bb * r;
  const uint16_t* erow = W1 + (size_t)prev * r;
  const bf16x8_t zero = bf16x8_t{};
  const bool first = a.k == 0;

  auto afrag = [&](int ks) -> bf16x8_t {
    const int kk = 16 * ks + 8 * h;          // in [0, 3r)
    const int col = kk < 2 * r ? (kk < r ? kk : kk - r) : kk - r;   // state | state | emb cols
    const bf16x8_t f = load_bf16x8(wrow + col);
    return arow_on ? f : zero;
  };
  // the raw B data of k-step ks: 8 state values (fp32) or 8 embedding values
  struct BRaw {
    f32x4_t x0, x1;
    bf16x8_t e;
  };
  auto bload = [&](int ks, BRaw& d) {
    const int kk = 16 * ks + 8 * h;
    if (kk >= 2 * r) {
      d.e = load_bf16x8(erow + (kk - 2 * r));
    } else {
      const int off = kk < r ? kk : kk - r;
      d.x0 = *reinterpret_cast<const f32x4_t*>(srow + off);
      d.x1 = *reinterpret_cast<const f32x4_t*>(srow + off + 4);
    }
  };
  auto bfrag = [&](int ks, const BRaw& d) -> bf16x8_t {
    const int kk = 16 * ks + 8 * h;
    if (kk >= 2 * r) return bon ? d.e : zero;
    if (first || !bon) return zero;
    const bool lo = kk >= r;
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t q[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = 2 * i + t;
        const float x = e < 4 ? d.x0[e] : d.x1[e - 4];
        const uint16_t hi = f32_to_bf16_rne(x);
        q[t] = lo ? f32_to_bf16_rne(x - bf16_to_f32(hi)) : hi;
      }
      w[i] = q[0] | (q[1] << 16);
    }
    return __builtin_bit_cast(bf16x8_t, w);
  };
  f32x16_t acc = {};
  {
    bf16x8_t af[kPer];
    BRaw bd[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int ks = min(wave * kPer + u, nks - 1);
      af[u] = afrag(ks);
      bload(ks, bd[u]);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int ks = wave * kPer + u;
      if (ks < nks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u], bfrag(ks, bd[u]), acc,
                                                                  0, 0, 0);
    }
  }
  if (wave > 0) s_part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += s_part[w][lane];
  // lane (c, h): column b; element i holds row 8 (i / 4) + 4 h + i % 4, i.e.
  // part i / 4 of element 8 g + 4 h + i % 4
  if (!bon) return;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    rnn_finish(a, b, 8 * g + 4 * h + e, acc[e], acc[4 + e], acc[8 + e], emb, true);
}

// fp32: one work-group per request, one thread per state element; k ascending
__global__ __launch_bounds__(256) void rnn_state_kernel_f32(RnnPos a, const float* __restrict__ Wr,
                                                           const float* __restrict__ W1,
                                                           float* __restrict__ emb,
                                                           int32_t* status) {
  const int b = blockIdx.x, r = a.rank;
  int prev = a.k == 0 ? a.anchor[b] : a.tokens[(size_t)b * a.gamma + a.k - 1];
  prev = clamp_token(prev, a.V, threadIdx.x == 0 ? status : nullptr);
  const float* e = W1 + (size_t)prev * r;
  const float* s = a.s_prev + (size_t)b * r;
  for (int el = threadIdx.x; el < r; el += blockDim.x) {
    float pre[3];
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const float* w = Wr + (size_t)(part * r + el) * a.ldw;
      float acc = 0.f;
      if (a.k > 0)
        for (int j = 0; j < r; ++j) acc = fmaf(w[j], s[j], acc);
      for (int j = 0; j < r; ++j) acc = fmaf(w[r + j], e[j], acc);
      pre[part] = acc;
    }
    rnn_finish(a, b, el, pre[0], pre[1], pre[2], emb, false);
  }
}

}  // namespace

size_t rnn_workspace_bytes(int B, int gamma, int rank) {
  return align256((size_t)B * gamma * 3 * rank * 4) + 2 * align256((size_t)B * rank * 4);
}

hipError_t launch_rnn_hidden(int B, int gamma, int rank, int H, int dtype, const void* hidden,
                             const void* Wr, const float* br, void* ws, hipStream_t stream) {
  const int M = B * gamma, N = 3 * rank, ldw = 2 * rank + H;
  float* P = static_cast<float*>(ws);
  TraceScope t("rnn_hidden_kernel", stream);
  if (dtype == DSPARK_BF16) {
    rnn_hidden_kernel_bf16<<<dim3((M + 31) / 32, (N + 31) / 32), dim3(256), 0, stream>>>(
        M, N, H, ldw, 2 * rank, static_cast<const uint16_t*>(hidden),
        static_cast<const uint16_t*>(Wr), br, P);
  } else {
    const long long n = (long long)M * N;
    rnn_hidden_kernel_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
        M, N, H, ldw, 2 * rank, static_cast<const float*>(hidden), static_cast<const float*>(Wr),
        br, P);
  }
  return hipGetLastError();
}

hipError_t launch_rnn_state(int k, int B, int gamma, int V, int rank, int H, int dtype,
                            const void* Wr, const void* W1, const int32_t* anchor,
                            const int32_t* tokens, void* emb, float* state_out, int32_t* status,
                            void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  RnnPos a;
  a.B = B; a.gamma = gamma; a.rank = rank; a.k = k; a.ldw = 2 * rank + H; a.V = V;
  a.P = reinterpret_cast<const float*>(w);
  float* s0 = reinterpret_cast<float*>(w + align256((size_t)B * gamma * 3 * rank * 4));
  float* s1 = reinterpret_cast<float*>(reinterpret_cast<char*>(s0) +
                                       align256((size_t)B * rank * 4));
  a.s_prev = (k & 1) ? s0 : s1;
  a.s_next = (k & 1) ? s1 : s0;
  a.state_out = state_out;
  a.anchor = anchor;
  a.tokens = tokens;
  TraceScope t("rnn_state_kernel", stream);
  if (dtype == DSPARK_BF16) {
    const dim3 grid(rank / 8, (B + kTileM - 1) / kTileM);
    auto* wr = static_cast<const uint16_t*>(Wr);
    auto* w1 = static_cast<const uint16_t*>(W1);
    auto* e = static_cast<uint16_t*>(emb);
    switch (rank) {
      case 32: rnn_state_kernel_bf16<2><<<grid, dim3(256), 0, stream>>>(a, wr, w1, e, status); break;
      case 64: rnn_state_kernel_bf16<4><<<grid, dim3(256), 0, stream>>>(a, wr, w1, e, status); break;
      case 128: rnn_state_kernel_bf16<8><<<grid, dim3(256), 0, stream>>>(a, wr, w1, e, status); break;
      default: rnn_state_kernel_bf16<16><<<grid, dim3(256), 0, stream>>>(a, wr, w1, e, status); break;
    }
  } else {
    rnn_state_kernel_f32<<<dim3(B), dim3(256), 0, stream>>>(
        a, static_cast<const float*>(Wr), static_cast<const float*>(W1), static_cast<float*>(emb),
        status);
  }
  return hipGetLastError();
}

}  // namespace dspark
