// dspark_schedule: hardware-aware prefix scheduler in one work-group.
//
// [weigao] part 4 / [billytse] 6: survival a[r,j] = prod_{i<=j} c[r,i];
// rank every extendable position by survival and add them one at a time
// while Theta = tau * SPS(Bt) rises, Bt = sum_r (1 + l_r) and tau = sum_r
// (1 + sum_{j<=l_r} a[r,j]).  [xhh] scheduler Q&A: stop once Theta no longer
// rises (strict rise to admit).  [billytse] 7: stopping early keeps the
// admission of position j independent of later positions' confidences.
//
// Layout: 1024 threads, keys (fp64 survival) and flat ids in LDS (<= 8192
// keys = 96 KB), padded to a power of two >= 1024.  Steps:
//   1. per-request cumulative product, left to right in fp64 (one thread per
//      request; bit-identical to a sequential product);
//   2. order by (a desc, flat id asc) -- a total order, so the order is
//      exact: a request's survivals never increase along its positions, so
//      a candidate's rank is the sum over the R runs of one binary search
//      each (schedule_rank_kernel, many compute units, up to 4096
//      candidates); beyond that a bitonic sort with the keys in registers
//      (shuffles within a wave, LDS for strides 64..512);
//   3. tau_n = R + sum of the first n ranked survivals, computed as a
//      double-double prefix scan and rounded once (the exact sum up to
//      ~1e-30 relative; independent of association);
//   4. candidate n is admitted iff Bt+1 is inside the table, SPS > 0 there,
//      and tau_{n+1} * SPS[R+n+1] > tau_n * SPS[R+n]; the number admitted is
//      the first n that fails (block min-reduction) -- no sequential loop.
//
// Two further stop rules share steps 1-3 and admit a prefix of the same
// ranking: capacity ([billytse] 7, [weigao] part 4 asynchronous scheduling:
// the batch size K is fixed from older predictions, the current candidates
// are still ranked by their latest survival; the first K are taken) and
// threshold ([billytse] 8 threshold sweep: every candidate whose survival is
// at least the threshold).
#include <mutex>

#include "dspark_common.hpp"
#include "dspark_launch.hpp"
#include "schedule_launch.hpp"
#include "trace.hpp"

namespace dspark {

namespace {

// candidates per thread of the 1024-thread group (kScheduleMaxKeys / 1024)
constexpr int kSchedPer = kScheduleMaxKeys / 1024;

struct dd {
  double hi, lo;
};
// sum of two double-doubles (inputs are non-negative: no cancellation)
__device__ inline dd dd_add(dd a, dd b) {
  double s = a.hi + b.hi;
  double bb = s - a.hi;
  double e = (a.hi - (s - bb)) + (b.hi - bb);
  e += a.lo + b.lo;
  double hi = s + e;
  double lo = e - (hi - s);
  return dd{hi, lo};
}
__device__ inline dd shfl_up_dd(dd v, int o) {
  return dd{__shfl_up(v.hi, o, kWave), __shfl_up(v.lo, o, kWave)};
}

// rank order of candidates: survival descending, then flat id ascending
__device__ inline bool rank_before(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Bitonic sort of the P = 1024 E keys in key[] / idx[] (LDS) into rank
// order, 1024 threads.  Thread t holds elements t + 1024 e in registers;
// compare-exchange partners at distance >= 1024 sit in the same thread,
// below 64 in the same wave (exchanged by shuffles), and in between they
// meet through LDS.  Every element keeps the rank-first of itself and its
// partner when (it is the lower of the pair) == (its run sorts in rank
// order), else the rank-second.
template <int E>
__device__ void bitonic_sort(double* key, int* idx) {
  const int tid = threadIdx.x;
  constexpr int P = 1024 * E;
  double k[E];
  int id[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = key[tid + 1024 * e];
    id[e] = idx[tid + 1024 * e];
  }
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 1024) {
        const int es = stride >> 10;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int f = e ^ es;
          if (f > e) {
            const int i = tid + 1024 * e;
            const bool up = (i & size) == 0;
            const bool first_is_hi = rank_before(k[f], id[f], k[e], id[e]);
            if (first_is_hi == up) {
              const double tk = k[e]; k[e] = k[f]; k[f] = tk;
              const int ti = id[e]; id[e] = id[f]; id[f] = ti;
            }
          }
        }
      } else {
        double ko[E];
        int io[E];
        if (stride >= 64) {
          __syncthreads();   // earlier readers are done with the arrays
#pragma unroll
          for (int e = 0; e < E; ++e) {
            key[tid + 1024 * e] = k[e];
            idx[tid + 1024 * e] = id[e];
          }
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) {
            ko[e] = key[(tid + 1024 * e) ^ stride];
            io[e] = idx[(tid + 1024 * e) ^ stride];
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            ko[e] = __shfl_xor(k[e], stride, kWave);
            io[e] = __shfl_xor(id[e], stride, kWave);
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid + 1024 * e;
          const bool up = (i & size) == 0;
          const bool lower = (i & stride) == 0;
          const bool mine_first = rank_before(k[e], id[e], ko[e], io[e]);
          const bool keep_first = (up == lower);
          if (mine_first != keep_first) {
            k[e] = ko[e];
            id[e] = io[e];
          }
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[tid + 1024 * e] = k[e];
    idx[tid + 1024 * e] = id[e];
  }
  __syncthreads();
}

}  // namespace

// Survival of every candidate, exactly as schedule_kernel forms it: the
// confidence clamped into [0, 1] (flagging is left to schedule_kernel), then
// each request's running product left to right in fp64.
__device__ inline void survival_keys(int R, int gamma, const float* __restrict__ conf,
                                     double* key) {
  const int N = R * gamma;
  // eight loads per thread in flight at a time (indices clamped into the
  // array), then the stores
  constexpr int kU = 8;
  const int nt = blockDim.x, t = threadIdx.x;
  for (int i0 = 0; i0 < N; i0 += kU * nt) {
    float c[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) c[u] = conf[min(i0 + u * nt + t, N - 1)];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * nt + t;
      if (i < N) key[i] = (double)((c[u] >= 0.f) ? fminf(c[u], 1.f) : 0.f);   // NaN -> 0
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    double acc = 1.0;
    for (int j = 0; j < gamma; ++j) {
      acc = acc * key[r * gamma + j];
      key[r * gamma + j] = acc;
    }
  }
  __syncthreads();
}

// Rank of every candidate in the order (survival desc, flat id asc), for
// up to kScheduleMergeKeys candidates, spread over compute units: a
// candidate's rank is the number of entries ranked ahead of it in every
// request's run.  A run is already in rank order (a request's survival never
// rises along its positions and equal ones keep ascending flat ids), so each
// run's count is one binary search.  kRankSplit lanes share a candidate,
// each searching every kRankSplit-th run with kRankRuns searches advancing
// together, and their counts are added by shuffles.  The order is total, so
// the ranks are a permutation of [0, N).
constexpr int kRankRuns = 16;
constexpr int kRankSplit = 16;
constexpr int kRankThreads = 256;   // kRankThreads / kRankSplit candidates per group
__global__ __launch_bounds__(kRankThreads) void schedule_rank_kernel(
    int R, int gamma, const float* __restrict__ conf, int32_t* __restrict__ rank_out) {
  __shared__ double key[kScheduleMergeKeys];
  survival_keys(R, gamma, conf, key);
  const int N = R * gamma;
  const int i = blockIdx.x * (kRankThreads / kRankSplit) + threadIdx.x / kRankSplit;
  const int part = threadIdx.x % kRankSplit;
  const int ic = min(i, N - 1);   // lanes past N search too, then drop their count
  const double ki = key[ic];
  int steps = 0;
  while ((1 << steps) <= gamma) ++steps;   // searches over gamma entries
  int rank = 0;
  for (int r0 = part; r0 < R; r0 += kRankRuns * kRankSplit) {
    int lo[kRankRuns], hi[kRankRuns];
#pragma unroll
    for (int u = 0; u < kRankRuns; ++u) {
      lo[u] = 0;
      hi[u] = r0 + u * kRankSplit < R ? gamma : 0;
    }
    for (int st = 0; st < steps; ++st) {
#pragma unroll
      for (int u = 0; u < kRankRuns; ++u) {
        if (lo[u] < hi[u]) {
          const int mid = (lo[u] + hi[u]) >> 1;
          const int f = (r0 + u * kRankSplit) * gamma + mid;
          if (rank_before(key[f], f, ki, ic)) lo[u] = mid + 1;
          else hi[u] = mid;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRankRuns; ++u) rank += lo[u];
  }
#pragma unroll
  for (int o = 1; o < kRankSplit; o <<= 1) rank += __shfl_xor(rank, o, kWave);
  if (part == 0 && i < N) rank_out[i] = rank;
}

__global__ __launch_bounds__(1024) void schedule_kernel(int R, int gamma,
                                                        const float* __restrict__ conf,
                                                        const double* __restrict__ sps,
                                                        int sps_len, int mode, double thr,
                                                        const double* __restrict__ cap,
                                                        int32_t* __restrict__ ell,
                                                        int32_t* __restrict__ order,
                                                        double* __restrict__ stats,
                                                        const int32_t* __restrict__ ranks,
                                                        int32_t* status) {
  __shared__ double key_a[kScheduleMaxKeys];
  __shared__ int idx_a[kScheduleMaxKeys];
  __shared__ double key_b[kScheduleMergeKeys];   // candidates placed by rank
  __shared__ int idx_b[kScheduleMergeKeys];
  double* key = key_a;
  int* idx = idx_a;
  __shared__ double wsum_hi[16], wsum_lo[16];
  __shared__ double s_tau, s_theta;

  const int tid = threadIdx.x, nthr = blockDim.x;   // 1024
  const int N = R * gamma;
  int P = 1024;
  while (P < N) P <<= 1;

  // 1. survival products: the confidences are read by the whole group at
  //    once (clamped into [0, 1], a bad value flagged), then each request's
  //    running product is taken in LDS
  for (int i = tid; i < N; i += nthr) {
    float c = conf[i];
    if (!(c >= 0.f)) {  // negative or NaN
      flag(status, DSPARK_DEV_BAD_CONF);
      c = 0.f;
    } else if (c > 1.f) {
      flag(status, DSPARK_DEV_BAD_CONF);
      c = 1.f;
    }
    key[i] = (double)c;
    idx[i] = i;
  }
  __syncthreads();
  for (int r = tid; r < R; r += nthr) {
    double acc = 1.0;
    for (int j = 0; j < gamma; ++j) {
      acc = acc * key[r * gamma + j];
      key[r * gamma + j] = acc;
    }
  }
  for (int i = N + tid; i < P; i += nthr) {
    key[i] = -1.0;
    idx[i] = 0x7fffffff;
  }
  // the SPS entries this thread's admission tests read (R + n for n in its
  // block and one past it), requested now and used after the ranking
  const int per = (N + nthr - 1) / nthr;
  const int c0 = min(N, tid * per), c1 = min(N, c0 + per);
  double spv[kSchedPer + 1];
#pragma unroll
  for (int u = 0; u <= kSchedPer; ++u) {
    const int i = R + c0 + u;
    spv[u] = (mode == kSchedTheta && u <= per && i < sps_len) ? sps[i] : 0.0;
  }
  // capacity: K floored and clamped to [0, N]; NaN or below 1 takes nothing
  int kcap = 0;
  if (mode == kSchedCapacity) {
    const double K = cap[0];
    kcap = K >= 1.0 ? (K >= (double)N ? N : (int)floor(K)) : 0;
  }
  __syncthreads();

  // 2. rank order (survival desc, flat id asc): placed by the ranks
  //    schedule_rank_kernel computed, or (beyond its buffer) a bitonic sort
  if (ranks) {
    for (int i = tid; i < N; i += nthr) {
      const int q = ranks[i];
      key_b[q] = key_a[i];
      idx_b[q] = i;
    }
    key = key_b;
    idx = idx_b;
    __syncthreads();
  } else {
    switch (P) {
      case 1024: bitonic_sort<1>(key, idx); break;
      case 2048: bitonic_sort<2>(key, idx); break;
      case 4096: bitonic_sort<4>(key, idx); break;
      default: bitonic_sort<8>(key, idx); break;
    }
  }

  // 3. double-double prefix sums over ranked survivals, in thread-contiguous
  //    blocks of `per` candidates
  dd local{0.0, 0.0};
  for (int i = c0; i < c1; ++i) local = dd_add(local, dd{key[i], 0.0});
  const int lane = tid & 63, wave = tid >> 6;
  dd incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    dd n = shfl_up_dd(incl, o);
    if (lane >= o) incl = dd_add(n, incl);
  }
  dd excl = shfl_up_dd(incl, 1);
  if (lane == 0) excl = dd{0.0, 0.0};
  if (lane == 63) { wsum_hi[wave] = incl.hi; wsum_lo[wave] = incl.lo; }
  __syncthreads();
  dd base{(double)R, 0.0};
  for (int w = 0; w < wave; ++w) base = dd_add(base, dd{wsum_hi[w], wsum_lo[w]});
  dd run = dd_add(base, excl);

  // 4. admission test of each candidate n in this thread's block
  int fail = N;
  if (mode == kSchedCapacity) {
    fail = kcap;
  } else if (mode == kSchedThreshold) {
    // survivals are ranked descending: the first one below the threshold
    for (int n = c0; n < c1; ++n) {
      if (!(key[n] >= thr)) {
        fail = n;
        break;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kSchedPer; ++u) {
      const int n = c0 + u;
      if (n >= c1 || fail != N) break;
      const double tau_n = run.hi + run.lo;
      run = dd_add(run, dd{key[n], 0.0});
      const double tau_n1 = run.hi + run.lo;
      const int nb = R + n + 1;   // SPS at nb is spv[u + 1], at nb - 1 spv[u]
      bool ok = nb < sps_len && spv[u + 1] > 0.0;
      if (ok) {
        const double theta_n = tau_n * spv[u];
        ok = tau_n1 * spv[u + 1] > theta_n;
      }
      if (!ok) fail = n;
    }
  }
  // first failing candidate overall
  fail = block_min_int(fail, reinterpret_cast<double*>(wsum_hi));
  const int nadm = fail;
  // tau and Theta after the last admitted candidate (thread holding n = nadm-1,
  // or the start value when nothing is admitted)
  if (tid == 0 && nadm == 0) {
    s_tau = (double)R;
    s_theta = R < sps_len ? (double)R * spv[0] : 0.0;   // thread 0: spv[0] = SPS[R]
    if (mode != kSchedTheta) s_theta = __builtin_nan("");
  }
  if (nadm > 0 && nadm - 1 >= c0 && nadm - 1 < c1) {
    dd r2 = dd_add(base, excl);
    for (int n = c0; n < nadm; ++n) r2 = dd_add(r2, dd{key[n], 0.0});
    const double tau = r2.hi + r2.lo;
    double sp_last = 0.0;   // SPS[R + nadm] = spv[nadm - c0]
#pragma unroll
    for (int u = 0; u <= kSchedPer; ++u)
      if (u == nadm - c0) sp_last = spv[u];
    s_tau = tau;
    s_theta = mode == kSchedTheta ? tau * sp_last : __builtin_nan("");
  }
  __syncthreads();

  // 5. outputs: the ranked order, and ell[r] = the admitted candidates of
  //    request r, which are a prefix of its positions (its survival never
  //    rises with j and ties keep the flat order), read off their ranks
  int* rank = reinterpret_cast<int*>(key);   // the keys are no longer read
  for (int i = tid; i < N; i += nthr) {
    const int id = idx[i];
    if (order) order[i] = id;
    rank[id] = i;
  }
  __syncthreads();
  for (int r = tid; r < R; r += nthr) {
    int L = 0;
    while (L < gamma && rank[r * gamma + L] < nadm) ++L;
    ell[r] = L;
  }
  if (tid == 0 && stats) {
    stats[0] = (double)nadm;
    stats[1] = s_tau;
    stats[2] = s_theta;
  }
}

// the candidates' ranks (int32) when schedule_rank_kernel runs
size_t schedule_workspace_bytes(int R, int gamma) {
  const long long N = (long long)R * gamma;
  return N <= kScheduleMergeKeys ? align256((size_t)N * 4) : 0;
}

hipError_t launch_schedule(int R, int gamma, const float* conf, const double* sps, int sps_len,
                           int mode, double threshold, const double* capacity, int32_t* ell,
                           int32_t* order, double* stats, int32_t* status, void* ws,
                           hipStream_t stream, bool traced) {
  const int N = R * gamma;
  int32_t* ranks = nullptr;
  if (N <= kScheduleMergeKeys) {
    ranks = static_cast<int32_t*>(ws);
    TraceScope tr(traced ? "schedule_rank_kernel" : nullptr, stream);
    constexpr int kPerGroup = kRankThreads / kRankSplit;
    schedule_rank_kernel<<<dim3((N + kPerGroup - 1) / kPerGroup), dim3(kRankThreads), 0,
                           stream>>>(R, gamma, conf, ranks);
  }
  TraceScope ts(traced ? "schedule_kernel" : nullptr, stream);
  schedule_kernel<<<dim3(1), dim3(1024), 0, stream>>>(R, gamma, conf, sps, sps_len, mode,
                                                      threshold, capacity, ell, order, stats,
                                                      ranks, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (dspark_schedule_noalloc): the
// candidates' ranks, int32, for up to kScheduleMergeKeys candidates (16 KB;
// larger batches rank inside the one work-group and need none).  Every
// device the library runs on holds one copy until the process ends; all
// calls on a device share it, so calls that overlap on one device race.
// Nothing in it needs clearing: the ranking kernel writes every rank the
// scheduler kernel then reads.  In host code the array's name stands for a
// host-side shadow, not a device address: host code only ever uses the
// address schedule_scratch() looked up for the current device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int32_t scratch[kScheduleMergeKeys];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

size_t schedule_scratch_bytes() { return (size_t)kScheduleMergeKeys * sizeof(int32_t); }

int32_t* schedule_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kScratchDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {   // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

}  // namespace dspark
