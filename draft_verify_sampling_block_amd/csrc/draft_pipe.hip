// Pipelined single-launch draft kernel (bf16, rank <= 256).
//
// [billytse] 3.2-3.3: position k's token is drawn from softmax(U_k + W1[prev]
// W2), prev being the token drawn at position k - 1 (the anchor at k = 0);
// positions are sampled left to right, requests independently of each other.
//
// One cooperative launch with two roles:
//
//  * tile groups (work-groups 0 .. Pt-1): each owns a contiguous run of
//    64-entry vocabulary tiles whose W2 rows stay on chip for the whole block
//    (8 tiles in registers, one per wave, up to 2 more in LDS).  The requests
//    are cut into windows of 32; the windows of all positions are processed
//    in order (position-major).  Per window every wave runs its block-task
//    (tile x 32 requests: bias on the matrix cores with the accumulators
//    started at the base logits, then the tile reduction; an LDS tile is
//    split into two half tasks), and the statistics go out as one 8-byte word
//    per (request, tile) plus one per (request, group): the group's max and
//    its exp-sum relative to that max, tagged with the parity of the
//    position.
//
//  * draw groups (work-groups Pt .. Pt+Pd-1): one wave per request draws its
//    token as soon as every tile group's word of that request is in: an fp64
//    scan over the Pt group words finds the group where the cumulative mass
//    crosses u * Z, a scan over that group's tile words the tile, and a
//    recompute of that one tile's 64 logits (W2 rows, the previous token's W1
//    row and the base logits) the entry.  The token goes out in the request's
//    flag word.
//
// While a window's tokens are drawn the tile groups already run the next
// window (other requests), so with two or more windows per position the
// draws and the exchanges stay off the critical path; the tile groups wait
// only when a window's previous tokens are not in yet.
//
// The exchange words live in the caller's workspace and need no clearing
// launch: every work-group zeroes the words it writes (a tile group its tile
// words and its column of group words, a draw wave its requests' token
// flags), then arrives at a start barrier, and no exchange word is read
// before every work-group has arrived.  A zero word carries tag 0, which
// position 0 (tag 1) never takes as written.  The barrier lives in a header
// at a fixed place in the workspace: a call number E (read by everyone at
// the start, advanced by the first draw group once everyone has arrived)
// and one arrival word per work-group, set to E + 1, so no two work-groups
// write the same word and no arrival of an earlier call passes for one of
// this call.
// The workspace only has to be zero-filled once, before its first use.
//
// Waits between work-groups are bounded by the device wall clock; a wait
// that gives up raises DSPARK_DEV_TIMEOUT, after which every other wait gives
// up at once so the grid always drains (results are then undefined but every
// output stays in range, and the workspace must be zero-filled again).
#include <algorithm>
#include <type_traits>

#include "conf_row.hpp"
#include "dspark_common.hpp"
#include "draft_tile.hpp"
#include "dspark_launch.hpp"
#include "trace.hpp"

namespace dspark {

constexpr int kPpWaves = 8;
constexpr int kBufferDword3 = 0x00020000;   // buffer descriptor word 3 (CDNA: raw bytes)
constexpr int kPpRegTiles = 8;                          // register tiles (one per wave)
constexpr int kPpLdsTiles = 2;                          // LDS tiles per tile group
constexpr int kPpMaxTiles = kPpRegTiles + kPpLdsTiles;  // tiles per tile group
constexpr int kPpSlots = kPpRegTiles + 2 * kPpLdsTiles; // statistics slots (LDS tiles by half)
constexpr int kPpRowBytes = kTileM * (2 * kMaxKSteps + 1) * 16;   // W1 rows of one window
constexpr int kPpMaxTileGroups = 256;                   // group words: 4 per lane of a wave
constexpr int kPpMaxDrawGroups = 16;
constexpr int kPpDrawLds = 1024;                        // per draw wave: W1 row + 64 masses
static_assert(kPpWaves * kPpDrawLds <= kLdsTileBytes, "draw scratch lives in ldsX");

struct PpArgs {
  int B, gamma, V, rank;
  int Pt, Pd;   // tile groups [0, Pt), draw groups [Pt, Pt + Pd)
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
  uint64_t* tw;         // [nT][B] tile words (max, exp-sum | parity << 63); a window's
                        // 32 requests write 256 contiguous bytes per tile
  uint64_t* gw;         // [B][Pt] group words (max, exp-sum or argmax | parity << 63)
  uint32_t* tok_flag;   // [B] ((k + 1) << 24) | token k
  uint32_t* hdr;        // start barrier: [0] call number, [64 + g] arrival of group g
  long long spin_cap;   // wall-clock ticks a wait may last
  // the confidence head (conf NULL: not evaluated)
  const uint16_t* hidden;   // [B][gamma][H]
  const float* cw;          // [H + rank]
  const float* temps;       // [gamma] or NULL
  float* conf;              // [B][gamma]
  float cbias;
  int H;
};

// tiles of tile group q (contiguous, the first nT % Pt groups one more)
__host__ __device__ inline int pp_tcount(int q, int nT, int Pt) {
  return nT / Pt + (q < nT % Pt ? 1 : 0);
}
__host__ __device__ inline int pp_tbase(int q, int nT, int Pt) {
  return q * (nT / Pt) + (q < nT % Pt ? q : nT % Pt);
}

// Cross-lane steps of the draw, none through the LDS crossbar: DPP moves
// within 16-lane rows, the row broadcasts and the whole-wave shift, the
// row-pair and half-wave swaps, and reads of one lane into a scalar.
// DPP control words: quad_perm p0 | p1 << 2 | p2 << 4 | p3 << 6, row_shr:n
// 0x110 + n, row_ror:n 0x120 + n, wave_shr:1 0x138, row_bcast:15 0x142,
// row_bcast:31 0x143.
template <int Ctrl, int RowMask = 0xf>
__device__ inline uint32_t dpp_u(uint32_t x) {   // lanes without a source read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, Ctrl, RowMask, 0xf, true);
}
template <int Ctrl, int RowMask = 0xf>
__device__ inline double dpp_d(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t lo = dpp_u<Ctrl, RowMask>((uint32_t)b);
  const uint64_t hi = dpp_u<Ctrl, RowMask>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
template <int Ctrl>
__device__ inline float dpp_f(float x) {
  return __uint_as_float(dpp_u<Ctrl>(__float_as_uint(x)));
}
// lane l's value (l wave-uniform)
__device__ inline int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ inline float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ inline double lane_d(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)((hi << 32) | lo));
}
// values of the even (lo) and odd (hi) 16-lane row of this lane's row pair
__device__ inline void row_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// inclusive prefix sum over the wave's 64 lanes (within each row by
// doubling steps, then the rows' totals carried into the rows after them)
__device__ inline double wave_incl_scan(double v) {
  v += dpp_d<0x111>(v);
  v += dpp_d<0x112>(v);
  v += dpp_d<0x114>(v);
  v += dpp_d<0x118>(v);
  v += dpp_d<0x142, 0xa>(v);
  v += dpp_d<0x143, 0xc>(v);
  return v;
}
// the preceding lane's value (0 in lane 0)
__device__ inline double wave_prev(double v) { return dpp_d<0x138>(v); }
__device__ inline float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  float lo, hi;
  row_pair(v, lo, hi);
  v = fmaxf(lo, hi);
  half_pair(v, lo, hi);
  return fmaxf(lo, hi);
}

// Bounded wait of one wave: true once done() holds on every lane; false
// when the wall-clock cap passed (DSPARK_DEV_TIMEOUT raised here) or another
// wait already gave up.
template <typename Done>
__device__ inline bool pp_wait(Done&& done, long long cap, int32_t* status) {
  const long long t0 = wall_clock64();
  for (int it = 0;; ++it) {
    if (__all(done())) return true;
    if ((it & 15) == 15) {
      const bool late = wall_clock64() - t0 > cap;
      const bool gave_up = ld_dev(status) & DSPARK_DEV_TIMEOUT;
      if (late || gave_up) {
        if (late && (threadIdx.x & 63) == 0) flag(status, DSPARK_DEV_TIMEOUT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Start barrier (see the top of the file).  pp_call: the call number, read
// by wave 0 before anything else; pp_arrive: once this work-group's zeroing
// stores are complete, thread 0 marks it arrived; pp_wait_all: the first
// draw group (idle until the first statistics arrive) waits until every
// arrival word reads E + 1 and then advances the call number (every
// work-group read it before arriving), which is what the other work-groups
// wait for.  Each work-group reads the header from one wave, and only that
// draw group reads the arrival words, so the few header lines are not
// swamped by reads from every wave of the grid.
constexpr int kPpHdrArrive = 64;   // header word of work-group 0's arrival
static_assert((kPpHdrArrive + kPpMaxTileGroups + kPpMaxDrawGroups) * 4 <= kDraftPipeHeaderBytes,
              "the header holds every work-group's arrival word");
__device__ inline bool pp_wave0() {   // a wave-uniform (scalar) test
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
}
__device__ inline uint32_t pp_call(const PpArgs& a) {
  return pp_wave0() ? __builtin_amdgcn_readfirstlane(ld_dev(a.hdr)) : 0u;
}
// (The zeroing stores are device-scope stores like every other exchange
// word's; each wave waits until its own have completed, so the arrival is
// marked after all of the work-group's.)
__device__ inline void pp_arrive(const PpArgs& a, uint32_t E) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's zeroing stores are complete
  __syncthreads();
  if (threadIdx.x == 0) st_dev(a.hdr + kPpHdrArrive + blockIdx.x, E + 1u);
}
__device__ inline void pp_wait_all(const PpArgs& a, uint32_t E) {
  const int G = a.Pt + a.Pd, lane = threadIdx.x & 63;
  if (pp_wave0()) {
    if ((int)blockIdx.x == a.Pt) {
      const bool ok = pp_wait(
          [&]() {
            bool in = true;
            for (int g = lane; g < G; g += kWave) in &= ld_dev(a.hdr + kPpHdrArrive + g) == E + 1u;
            return in;
          },
          a.spin_cap, a.status);
      if (ok && lane == 0) st_dev(a.hdr, E + 1u);
    } else {
      pp_wait([&]() { return ld_dev(a.hdr) == E + 1u; }, a.spin_cap, a.status);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Draw role: one wave draws token k of request b
// ---------------------------------------------------------------------------
template <int KS>
__device__ void pp_draw(const PpArgs& a, int b, int k, char* wl) {
  const int lane = threadIdx.x & 63;
  const int B = a.B, V = a.V, gamma = a.gamma, rank = a.rank, Pt = a.Pt;
  const int nT = n_tiles(V);
  (void)B;
  // the previous token: the anchor, or the flag word this wave's lane 0
  // stored for position k - 1 (read back by the same lane)
  int pv = 0;
  if (lane == 0) pv = k == 0 ? a.anchor[b] : (int)(ld_dev(a.tok_flag + b) & 0xFFFFFFu);
  const int prev = clamp_token(lane_i(pv, 0), V, nullptr);
  // the previous token's W1 row into this wave's LDS (needed only by the
  // crossing-tile recompute; requested first so it is in by then)
  if (lane < rank / 8)
    __builtin_amdgcn_global_load_lds(a.W1 + (size_t)prev * rank + 8 * lane, wl, 16, 0, 0);
  // The confidence of (b, k) needs only the previous token, known now: the
  // wave evaluates it while the position's statistics are still being
  // formed (the same code, hence the same bits, as the head's own kernel).
  if (a.conf) {
    const float dot = conf_dot_wave<uint16_t>(a.hidden + ((size_t)b * gamma + k) * a.H,
                                              a.W1 + (size_t)prev * rank, a.cw, a.H, rank, lane);
    if (lane == 0)
      a.conf[(size_t)b * gamma + k] = conf_from_dot(dot, a.cbias, a.temps, k, a.status);
  }
  const float Tb = a.temperature[b];
  const bool greedy = !(Tb > 0.f);
  const double u = (double)a.uniforms[((size_t)b * (gamma + 1) + k) * 2 + 0];
  const size_t out = (size_t)b * gamma + k;
  auto emit = [&](int tok, float q, float rmax, float rlz) {
    if (lane == 0) {
      st_dev(a.tok_flag + b, ((uint32_t)(k + 1) << 24) | (uint32_t)tok);
      a.tokens[out] = tok;
      a.q_tok[out] = q;
      a.row_max[out] = rmax;
      a.row_logZ[out] = rlz;
    }
  };

  // the group words of (b, k): lane l holds groups 4l .. 4l + 3.  Two
  // polls are kept in flight (each checked while the next is under way), so
  // words that land between polls are seen half a round trip sooner.
  const uint64_t want = (uint64_t)((k + 1) & 1);
  const uint64_t* gwb = a.gw + (size_t)b * Pt;
  uint64_t r[4], ra[4], rb[4];
  auto issue = [&](uint64_t (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * lane + i < Pt) ? ld_dev(gwb + 4 * lane + i) : (want << 63);
  };
  auto ready = [&](const uint64_t (&x)[4]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) ok &= (x[i] >> 63) == want;
    return __all(ok) != 0;
  };
  {
    const long long t0 = wall_clock64();
    issue(ra);
    for (int it = 0;; ++it) {
      issue(rb);
      if (ready(ra)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = ra[i];
        break;
      }
      issue(ra);
      if (ready(rb)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = rb[i];
        break;
      }
      if ((it & 7) == 7) {
        const bool late = wall_clock64() - t0 > a.spin_cap;
        if (late || (ld_dev(a.status) & DSPARK_DEV_TIMEOUT)) {
          if (late && lane == 0) flag(a.status, DSPARK_DEV_TIMEOUT);
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = rb[i];
          break;
        }
      }
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // tile-word loads stay after the group words

  float gm[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gm[i] = (4 * lane + i < Pt) ? __uint_as_float((uint32_t)r[i]) : -INFINITY;
    mloc = fmaxf(mloc, gm[i]);
  }
  const float M = wave_max_dpp(mloc);
  auto payload = [&](int i) { return (uint32_t)(r[i] >> 32) & 0x7FFFFFFFu; };

  if (greedy) {
    // the lowest group attaining the max holds the lowest argmax
    int fi = 4;
#pragma unroll
    for (int i = 3; i >= 0; --i)
      if (4 * lane + i < Pt && gm[i] == M) fi = i;
    const unsigned long long hit = __ballot(fi < 4);
    int tok = 0;
    if (hit) {
      const int src = __builtin_ctzll(hit);
      uint32_t pl = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i == fi) pl = payload(i);
      tok = lane_i((int)pl, src);
    }
    if (!hit || !(M == M) || tok < 0 || tok >= V) {
      if (lane == 0) flag(a.status, DSPARK_DEV_NONFINITE);
      tok = 0;
    }
    emit(tok, 1.f, M, 0.f);
    return;
  }

  // mass of group q relative to the row max, in fp64; scan over the groups
  const float scale = 1.f / Tb;
  const float ce = scale * kLog2e;
  double gmass[4];
  double lsum = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gmass[i] = (4 * lane + i < Pt)
                   ? (double)__uint_as_float(payload(i)) *
                         (double)__builtin_amdgcn_exp2f((gm[i] - M) * ce)
                   : 0.0;
    lsum += gmass[i];
  }
  const double incl = wave_incl_scan(lsum);
  const double excl = wave_prev(incl);
  const double Z = lane_d(incl, kWave - 1);
  // u * Z can round up to Z: the target is kept below Z, so exactly one
  // lane's interval [excl, incl) holds it (consecutive intervals share ends)
  double target = u * Z;
  if (!(target < Z)) target = nextafter(Z, 0.0);
  const float ms = M * scale;
  const bool finite = isfinite(M) && isfinite(Z) && Z > 0.0;
  const bool mine = finite && lsum > 0.0 && excl <= target && target < incl;
  int fg = -1;
  double before = excl;
  if (mine) {
    double run = excl, lastb = excl;
    int lastg = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (gmass[i] > 0.0) {
        lastg = i;
        lastb = run;
        if (fg < 0 && target < run + gmass[i]) {
          fg = i;
          before = run;
        }
      }
      run += gmass[i];
    }
    if (fg < 0) {
      fg = lastg;
      before = lastb;
    }
  }
  const unsigned long long gh = __ballot(mine);
  if (!gh) {
    if (lane == 0) flag(a.status, DSPARK_DEV_NONFINITE);
    emit(0, 0.f, ms, __logf((float)Z));
    return;
  }
  const int gsrc = __builtin_ctzll(gh);
  const int gq = 4 * gsrc + lane_i(fg, gsrc);
  const double gbefore = lane_d(before, gsrc);

  // that group's tile words: lane t holds tile tb + t
  const int tb = pp_tbase(gq, nT, Pt), tc = pp_tcount(gq, nT, Pt);
  // (tagged with the position's parity like the group words; stored before
  // them, so normally in already)
  uint64_t w = 0;
  pp_wait(
      [&]() {
        if (lane >= tc) return true;
        w = ld_dev(a.tw + (size_t)(tb + lane) * B + b);
        return (w >> 63) == want;
      },
      a.spin_cap, a.status);
  float tm = -INFINITY;
  double tmass = 0.0;
  if (lane < tc) {
    tm = ms_max(w);
    tmass = (double)__uint_as_float((uint32_t)(w >> 32) & 0x7FFFFFFFu) *
            (double)__builtin_amdgcn_exp2f((tm - M) * ce);
  }
  const double tincl = wave_incl_scan(tmass);
  const double texcl = wave_prev(tincl);
  const double rt = target - gbefore;
  const unsigned long long th = __ballot(tmass > 0.0 && rt < tincl);
  const unsigned long long tpos = __ballot(tmass > 0.0);
  if (!tpos) {
    if (lane == 0) flag(a.status, DSPARK_DEV_NONFINITE);
    emit(0, 0.f, ms, __logf((float)Z));
    return;
  }
  const int tl = th ? __builtin_ctzll(th) : 63 - __builtin_clzll(tpos);
  const int vt = tb + tl;
  const float mvt = lane_f(tm, tl);
  const double tbefore = gbefore + lane_d(texcl, tl);
  const double tscale = (double)__builtin_amdgcn_exp2f((mvt - M) * ce);
  const float mc = mvt * ce;

  // recompute tile vt: lane (g, rho) sums k-rows rho, rho + 8, ... for the
  // entries v0 + 8g .. + 7; the eight partial sums of an entry are then
  // added across the lanes of the same g
  const int v0 = vt * kTileV;
  const int g8 = lane & 7, rho = lane >> 3;
  const int col = min(v0 + 8 * g8, V - 8);   // pieces past V: any valid address
  constexpr int NR = 2 * KS;                 // k-rows per lane (rank / 8)
  // (buffer loads: one per-lane byte offset plus a scalar one per k-row step,
  // where 64-bit addresses for every step would be held in registers across
  // the draw loop)
  u32x4_t wv[NR];
  {
    const __amdgpu_buffer_rsrc_t w2r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.W2), (short)0, rank * V * 2, kBufferDword3);
    const int vo = (rho * V + col) * 2;
#pragma unroll
    for (int m = 0; m < NR; ++m) wv[m] = __builtin_amdgcn_raw_buffer_load_b128(w2r, vo, m * 16 * V, 0);
  }
  const u32x4_t uv = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(a.U + out * V + col));
  const uint16_t* wrow = reinterpret_cast<const uint16_t*>(wl);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const float ak = bf16_to_f32(wrow[rho + 8 * m]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wd = wv[m][e >> 1];
      const float w2 = (e & 1) ? __uint_as_float(wd & 0xFFFF0000u) : __uint_as_float(wd << 16);
      acc[e] = __builtin_fmaf(ak, w2, acc[e]);
    }
  }
  // the partial sums of lanes g8, g8 + 8, ..., g8 + 56 added in pairs:
  // across half rows (row_ror:8), across the rows of a pair, across halves
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += dpp_f<0x128>(acc[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float lo, hi;
    row_pair(acc[e], lo, hi);
    acc[e] = lo + hi;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float lo, hi;
    half_pair(acc[e], lo, hi);
    acc[e] = lo + hi;
  }
  float* es = reinterpret_cast<float*>(wl + 512);
  if (rho == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wd = uv[e >> 1];
      const float ub = (e & 1) ? __uint_as_float(wd & 0xFFFF0000u) : __uint_as_float(wd << 16);
      const float z = ub + acc[e];
      es[8 * g8 + e] = (v0 + 8 * g8 + e < V) ? tile_term(z, ce, mc) : 0.f;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const double ej = (double)es[lane];
  const double rr = (target - tbefore) / tscale;
  const double eincl = wave_incl_scan(ej);
  const unsigned long long hit = __ballot(ej > 0.0 && rr < eincl);
  const unsigned long long pos = __ballot(ej > 0.0);
  const int pick = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
  const double epick = lane_d(ej, pick);
  emit(v0 + pick, (float)(epick * tscale / Z), ms, __logf((float)Z));
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int KS>
__global__ __launch_bounds__(kPpWaves * 64, 1) void pdraft_pipe_kernel(PpArgs a) {
  constexpr int nq = 2 * KS;
  constexpr int nc = nq + 1;   // 16-byte chunks per padded LDS row
  __shared__ __attribute__((aligned(16))) char ldsL[kPpLdsTiles * kLdsTileBytes];
  // W1 rows of the current and the next window: two separate arrays, so
  // that the compiler can tell a gather into one from the reads of the
  // other and lets them overlap
  __shared__ __attribute__((aligned(16))) char ldsR0[kPpRowBytes];
  __shared__ __attribute__((aligned(16))) char ldsR1[kPpRowBytes];
  // third W2 tile image while the resident tiles are staged; then 4 KB per
  // wave for passing the base logits to the matrix layout (tile groups) or
  // the draw waves' scratch
  __shared__ __attribute__((aligned(16))) char ldsX[kLdsTileBytes];
  // per window parity: statistics of the window's block-tasks per slot and
  // row (register tile of wave w: slot w; half t of LDS tile i: slot 8 + 2i + t)
  __shared__ float s_mx[2][kPpSlots][kTileM], s_sum[2][kPpSlots][kTileM];
  __shared__ int s_arg[2][kPpSlots][kTileM];
  // inverse temperatures of a window's requests, by window index mod 3 (the
  // group words of window j - 1, the tasks of window j and the gather for window
  // j + 1 overlap)
  __shared__ float s_it[3][kTileM];
  __shared__ int s_done[2];   // waves done with the window of each parity

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the lane id from the mbcnt instructions (rematerialised where needed
  // instead of held in a register the task loop would have to spill)
  const int lane = __lane_id();

  if ((int)blockIdx.x >= a.Pt) {
    // draw role: wave w of draw group g draws requests g + Pd (w + 8 m),
    // m = 0, 1, ... of every position, in the order the tile groups complete
    // them; consecutive requests go to different draw groups, so a window's
    // draws (and their W2 reads) spread over all of them
    const int g = (int)blockIdx.x - a.Pt;
    char* wl = ldsX + wave * kPpDrawLds;

    const uint32_t E = pp_call(a);
    // this wave's requests' token flags start at zero
    for (int b = g + a.Pd * wave; b < a.B; b += a.Pd * kPpWaves)
      if (lane == 0) st_dev(a.tok_flag + b, 0u);
    pp_arrive(a, E);
    pp_wait_all(a, E);
    for (int k = 0; k < a.gamma; ++k)
      for (int b = g + a.Pd * wave; b < a.B; b += a.Pd * kPpWaves) pp_draw<KS>(a, b, k, wl);
    return;
  }

  const int p = blockIdx.x, Pt = a.Pt;
  const int c = lane & 31, h = lane >> 5;
  const int B = a.B, V = a.V, gamma = a.gamma, rank = a.rank;
  const int nT = n_tiles(V);
  const int tcount = pp_tcount(p, nT, Pt), tbase = pp_tbase(p, nT, Pt);
  auto slot_tile = [&](int slot) { return slot < tcount ? tbase + slot : nT; };


  // Resident W2 tiles (W2 is [rank, V]): the blocks of the eight register
  // tiles are loaded in one shot and pass three at a time through three LDS
  // images (the two LDS tile areas and ldsX) into registers; then the LDS
  // tiles are staged in place.
  auto img = [&](int j) { return j < 2 ? ldsL + j * kLdsTileBytes : ldsX; };
  const int nbk = w2_blocks(rank);
  constexpr int nthr = kPpWaves * 64;
  constexpr int kQ = (32 * KS + nthr - 1) / nthr;
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
        if (sb < nbk) w2_block_store(bk[q], sb, dst, nq);
      }
    }
  };
  // This group zeroes its tile words and its column of group words and
  // arrives at the start barrier before anything else (the stores' wait then
  // holds no W2 loads); it waits for the others once its W2 tiles are staged
  // (outside the window loop's function, whose registers it would crowd).
  const uint32_t E = pp_call(a);
  for (int i = (int)threadIdx.x; i < B * tcount; i += kPpWaves * 64)
    st_dev(a.tw + (size_t)tbase * B + i, (uint64_t)0);   // rows tbase .. + tcount - 1
  for (int bq = (int)threadIdx.x; bq < B; bq += kPpWaves * 64)
    st_dev(a.gw + (size_t)bq * Pt + p, (uint64_t)0);
  pp_arrive(a, E);
  bf16x8_t wreg[KS][kSub];
  {
    W2Block blk[kPpRegTiles][kQ];
#pragma unroll
    for (int j = 0; j < kPpRegTiles; ++j) load_slot(j, blk[j]);
    W2Block lblk[kPpLdsTiles][kQ];
#pragma unroll
    for (int r0 = 0; r0 < kPpRegTiles; r0 += 3) {
#pragma unroll
      for (int j = r0; j < r0 + 3 && j < kPpRegTiles; ++j) store_slot(j, blk[j], img(j - r0));
      if (r0 + 3 >= kPpRegTiles) {
#pragma unroll
        for (int j = 0; j < kPpLdsTiles; ++j) load_slot(kPpRegTiles + j, lblk[j]);
      }
      __syncthreads();
      if (wave >= r0 && wave < r0 + 3) wreg_from_lds<KS>(img(wave - r0), wreg);
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kPpLdsTiles; ++j) store_slot(kPpRegTiles + j, lblk[j], img(j));
  }
  // the statistics slots this group has no task for hold empty statistics
  // (both parities, written once; tasks write only their own slots)
  for (int e = (int)threadIdx.x; e < 2 * kPpSlots * kTileM; e += kPpWaves * 64) {
    const int sl = (e / kTileM) % kPpSlots, pe = e / (kPpSlots * kTileM), cc = e % kTileM;
    const int ti = sl < kPpRegTiles ? sl : kPpRegTiles + ((sl - kPpRegTiles) >> 1);
    if (ti >= tcount) {
      s_mx[pe][sl][cc] = -INFINITY;
      s_sum[pe][sl][cc] = 0.f;
      s_arg[pe][sl][cc] = 0x7fffffff;
    }
  }
  pp_wait_all(a, E);   // every work-group has zeroed its words (and the barrier
                       // makes the empty statistics visible)
  const int nL = (tcount > kPpRegTiles ? 1 : 0) + (tcount > kPpRegTiles + 1 ? 1 : 0);
  const bool hasreg = wave < tcount;
  // half-tasks of a window: 2 per LDS tile; half i goes to wave i + 4
  const int hidx = (wave + 4) & 7;
  const bool hashalf = hidx < 2 * nL;
  const int ntask = (hasreg ? 1 : 0) + (hashalf ? 1 : 0);   // per window, every window

  // windows: position-major, 32 requests each
  const int nch = (B + kTileM - 1) / kTileM;
  const int nwin = gamma * nch;

  // one-task ring of base logits (they do not depend on drafted tokens);
  // past the last task the slot loads a safe address, so every task issues
  // the same four loads
  struct Slot {
    URow<uint16_t> u;
  };
  Slot ring;
  int fj = 0, ft = 0;   // next task to fetch (window, index in the window)
  auto fetch_next = [&](Slot& sl) __attribute__((always_inline)) {
    if (ft >= ntask) {
      ++fj;
      ft = 0;
    }
    const bool real = fj < nwin && ntask > 0;
    const bool reg = hasreg && ft == 0;
    const int k = real ? fj / nch : 0;
    const int b = (real ? (fj % nch) * kTileM : 0) + c;
    const int tile = reg ? tbase + wave : tbase + kPpRegTiles + (hidx >> 1);
    const int sub = reg ? -1 : (hidx & 1);
    const int v0 = tile * kTileV;
    // whole 128-byte row pieces: load i covers rows 8i .. 8i + 7 of the
    // block, lane L taking 16 bytes (chunk L % 8) of row 8i + L / 8; a half
    // task's sub-tile (64 bytes per row) takes loads 0 and 1, 16 rows each,
    // and loads 2 and 3 read a safe address (every task issues four loads)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = reg ? 8 * i + (lane >> 3) : 16 * i + (lane >> 2);
      const int off = reg ? 8 * (lane & 7) : 32 * sub + 8 * (lane & 3);
      const int bq = b - c + r;
      const bool in = real && (reg || i < 2) && bq < B && v0 + off < V;
      const uint16_t* pp = in ? a.U + ((size_t)bq * gamma + k) * V + v0 + off : a.U + 8 * i;
      sl.u.w[i >> 1][i & 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pp));
    }
    ++ft;
  };
  // The ring slot's row pieces passed to the matrix layout through this
  // wave's 4 KB of LDS (row r at 128 r, chunk q at 16 (q ^ (r % 8)), so that
  // eight consecutive rows read at one chunk hit eight distinct bank groups):
  // lane (c, h) gets the entries 32 t + 16 h .. + 15 of request c for t = 0, 1
  // (a half task: its sub-tile's entries 16 h .. + 15 in part 0).
  char* rs = ldsX + wave * 4096;
  // `vb` is the task's first vocabulary entry (the tile, or a half task's
  // sub-tile): a lane whose 8-entry chunk lies at or past V writes -inf
  // there, so the accumulators start at -inf past the vocabulary with no
  // per-entry test (V % 8 == 0: a chunk is wholly inside or outside).
  auto restage = [&](const URow<uint16_t>& in, bool reg, int vb, URow<uint16_t>& out) __attribute__((always_inline)) {
    const int q = reg ? (lane & 7) : (lane & 3);
    const bool past = vb + 8 * q >= V;
    const u32x4_t ninf = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};   // bf16 -inf
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (reg || i < 2) {
        const int r = reg ? 8 * i + (lane >> 3) : 16 * i + (lane >> 2);
        *reinterpret_cast<u32x4_t*>(rs + r * 128 + 16 * (q ^ (r & 7))) =
            past ? ninf : in.w[i >> 1][i & 1];
      }
    }
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int q = (reg ? 4 * t : 0) + 2 * h + e;
        if (reg || t == 0)
          out.w[t][e] = *reinterpret_cast<const u32x4_t*>(rs + c * 128 + 16 * (q ^ (c & 7)));
      }
    }
  };

  // Gather of window jn's rows into `dst` by waves 0..3, eight rows each
  // (previous tokens `tok` and temperatures `tv` in lanes 0..7, the latter
  // loaded ahead by temp_issue; lanes past the window's requests hold
  // token 0 and inverse temperature 0).  Waves 4..7, which run the LDS
  // tiles' half tasks, issue no row DMA: a wave with a DMA in flight waits
  // for it before its next LDS read.  Completion: the caller's wait.
  constexpr int kGw = 4, kRpw = kTileM / kGw;   // gathering waves, rows each
  auto gather = [&](int jn, char* dst, int tok, float tv) __attribute__((always_inline)) {
    const int nrows = min(kTileM, B - (jn % nch) * kTileM);
    const int row = wave * kRpw + lane;
    if (lane < kRpw) s_it[jn % 3][row] = row < nrows ? inv_temp(tv) : 0.f;
    char* wd = dst + (size_t)(wave * kRpw) * nc * 16;
    constexpr int nslots = kRpw * nc;
    constexpr int ng = (nslots + 63) / 64;
    // every slot's token requested before the first is used (one wait)
    int tk[ng];
#pragma unroll
    for (int g = 0; g < ng; ++g) tk[g] = __shfl(tok, min((g * 64 + lane) / nc, kRpw - 1), kWave);
#pragma unroll
    for (int g = 0; g < ng; ++g) {
      const int s = g * 64 + lane;
      const int rl = s / nc, q = s - rl * nc;
      if (s < nslots)
        __builtin_amdgcn_global_load_lds(a.W1 + (size_t)tk[g] * rank + (q < nq ? q : 0) * 8,
                                         wd + g * 1024, 16, 0, 0);
    }
  };
  // Temperatures of this wave's rows of window jn (lanes 0..7), loaded well
  // before the gather that takes them.
  auto temp_issue = [&](int jn) __attribute__((always_inline)) {
    const int row = wave * kRpw + lane;
    const int bq = (jn % nch) * kTileM + row;
    return (lane < kRpw && bq < B) ? a.temperature[bq] : 0.f;
  };
  // Previous tokens of this wave's rows of window jn (lanes 0..7): issue
  // one flag load per lane, then (later, so the load is in flight meanwhile)
  // check that every one is in and take the tokens.  Position 0 takes the
  // anchors.
  auto poll_issue = [&](int jn) __attribute__((always_inline)) {
    const int row = wave * kRpw + lane;
    const int bq = (jn % nch) * kTileM + row;
    const bool real = lane < kRpw && bq < B;
    if (jn / nch == 0) return real ? (uint32_t)a.anchor[bq] : 0u;
    return real ? ld_dev(a.tok_flag + bq) : 0xFFFFFFFFu;
  };
  auto poll_check = [&](int jn, uint32_t v, int& tok) __attribute__((always_inline)) {
    const int kn = jn / nch;
    const int row = wave * kRpw + lane;
    const bool real = lane < kRpw && (jn % nch) * kTileM + row < B;
    if (kn == 0) {
      tok = real ? clamp_token((int)v, V, a.status) : 0;
      return true;
    }
    tok = real ? clamp_token((int)(v & 0xFFFFFFu), V, nullptr) : 0;
    return __all(v >= ((uint32_t)kn << 24)) != 0;
  };
  auto wait_tokens = [&](int jn, int& tok) __attribute__((always_inline)) {
    pp_wait([&]() { return poll_check(jn, poll_issue(jn), tok); }, a.spin_cap, a.status);
  };
  const bool gathers = wave < kGw;

  // Window j's group words, written by the last wave to finish its tasks
  // (column c = the window's request c): the LDS tiles' tile words (their
  // two halves combined here) and per request the group's max and exp-sum
  // relative to it (the argmax for a greedy request), tagged with the
  // position's parity (bit 63).  The register tiles' words went out from
  // their tasks.  The two half-waves split the tiles: half h takes register
  // tiles 4h .. 4h + 3 and LDS tile 8 + h, and the halves' maxima, sums and
  // argmax candidates are exchanged once.
  static_assert(kPpRegTiles == 8 && kPpLdsTiles == 2, "the split assumes 8 + 2 tiles");
  auto finish_window = [&](int j) __attribute__((always_inline)) {
    const int pb = j & 1;
    const int r0 = (j % nch) * kTileM;
    const uint64_t tag = (uint64_t)(((j / nch) + 1) & 1) << 63;   // parity of the position
    const bool act = r0 + c < B;
    const int bq = r0 + c;
    const float it = act ? s_it[j % 3][c] : 0.f;
    const bool greedy = !(it > 0.f);
    const float ce = it * kLog2e;
    // this half's slots, read at once: register tiles 4h + i, then the two
    // halves of LDS tile 8 + h (a slot the group has no tile for holds the
    // empty statistics written before the first window: max -inf, sum 0)
    float lmx[6], lsm[6];
    int lag[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int sl = i < 4 ? 4 * h + i : kPpRegTiles + 2 * h + (i - 4);
      lmx[i] = s_mx[pb][sl][c];
      lsm[i] = s_sum[pb][sl][c];
      lag[i] = s_arg[pb][sl][c];
    }
    float tmx[5], tsm[5];
    int targ[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tmx[i] = lmx[i];
      tsm[i] = lsm[i];
      targ[i] = lag[i];
    }
    {
      const int tl = kPpRegTiles + h;   // this half's LDS tile
      const float m0 = lmx[4], m1 = lmx[5];
      const float m = fmaxf(m0, m1);
      tmx[4] = m;
      targ[4] = (m0 == m) ? lag[4] : lag[5];
      tsm[4] = (greedy || !(m > -INFINITY))
                   ? 0.f
                   : lsm[4] * __builtin_amdgcn_exp2f((m0 - m) * ce) +
                         lsm[5] * __builtin_amdgcn_exp2f((m1 - m) * ce);
      if (act && tl < tcount && !greedy)
        st_dev(a.tw + (size_t)(tbase + tl) * B + bq,
               (uint64_t)((pack_ms(m, tsm[4]) & ~(1ull << 63)) | tag));
    }
    // tile index (within the group) of entry i of this half
    auto tidx = [&](int i) { return i < 4 ? 4 * h + i : kPpRegTiles + h; };
    float hmx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 5; ++i) hmx = fmaxf(hmx, tmx[i]);
    if (!act) hmx = -INFINITY;
    float mlo, mhi;
    half_pair(hmx, mlo, mhi);
    const float gmx = fmaxf(mlo, mhi);
    uint32_t pl = 0;
    if (greedy) {
      // the lowest tile index attaining the max, then its argmax
      int bi = 0x7fffffff, ba = 0x7fffffff;
#pragma unroll
      for (int i = 4; i >= 0; --i)
        if (tmx[i] == gmx && tidx(i) < bi) {
          bi = tidx(i);
          ba = targ[i];
        }
      int bilo, bihi, balo, bahi;
      half_pair(bi, bilo, bihi);
      half_pair(ba, balo, bahi);
      pl = (uint32_t)(bilo <= bihi ? balo : bahi);
    } else {
      float hs = 0.f;
#pragma unroll
      for (int i = 0; i < 5; ++i)
        hs += tsm[i] * __builtin_amdgcn_exp2f((tmx[i] - gmx) * ce);
      float slo, shi;
      half_pair(hs, slo, shi);
      pl = __float_as_uint(slo + shi);
    }
    if (act && h == 0)
      st_dev(a.gw + (size_t)bq * Pt + p,
             (uint64_t)(((uint64_t)__float_as_uint(gmx) | ((uint64_t)(pl & 0x7FFFFFFFu) << 32)) | tag));
  };
  // waves with tasks in every window; the one whose count completes a
  // window writes its group words
  const int nwt = tcount < kPpWaves ? tcount : kPpWaves;
  // (relaxed LDS atomic: the work-group's LDS serves each wave's accesses in
  // order, so the statistics a wave stored before its count are in place
  // for the wave that reads the full count; acquire/release would also
  // wait for this wave's base-logit loads in flight)
  auto task_done = [&](int j) __attribute__((always_inline)) {
    int prev = 0;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&s_done[j & 1], 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP);
    prev = lane_i(prev, 0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (prev == nwt - 1) {
      if (lane == 0)
        __hip_atomic_store(&s_done[j & 1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      finish_window(j);
    }
  };

  // run the wave's task `ft_run` of window j (parity buffers PB), taking the
  // base logits from the ring slot and refilling it with the next task
  auto run_task = [&](auto pbc, int j, bool reg) __attribute__((always_inline)) {
    constexpr int pb = decltype(pbc)::value;
    const char* rows = pb ? ldsR1 : ldsR0;
    const int b = (j % nch) * kTileM + c;
    const float it = s_it[j % 3][c];
    const bool any_greedy = __ballot((b < B) && !(it > 0.f)) != 0;
    auto bfrag = [&](int ks) { return lds_frag(rows, c, 2 * ks + h, nq); };
    if (reg) {
      const int tile = tbase + wave;
      const int v0 = tile * kTileV;
      URow<uint16_t> u;
      restage(ring.u, true, v0, u);
      fetch_next(ring);
      f32x16_t acc[kSub];
#pragma unroll
      for (int t = 0; t < kSub; ++t) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc[t][jj] = urow_at(u, t, jj);
      }
      bias_tile_regA<KS>(bfrag, wreg, acc);
      const TileStat st = tile_reduce(acc, tile, it, any_greedy);
      if (h == 0) {
        s_mx[pb][wave][c] = st.mx;
        s_sum[pb][wave][c] = st.s;
        s_arg[pb][wave][c] = st.arg;
        if (b < B && it > 0.f)
          st_dev(a.tw + (size_t)tile * B + b,
                 (uint64_t)((pack_ms(st.mx, st.s) & ~(1ull << 63)) |
                            ((uint64_t)(((j / nch) + 1) & 1) << 63)));
      }
    } else {
      const int li = hidx >> 1, t = hidx & 1;
      const int tile = tbase + kPpRegTiles + li;
      const int v0 = tile * kTileV;
      URow<uint16_t> u;
      restage(ring.u, false, v0 + 32 * t, u);
      fetch_next(ring);
      f32x16_t acc;   // the sub-tile's entries sit in part 0
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) acc[jj] = urow_at(u, 0, jj);
      bias_subtile_ldsA<KS>(bfrag, ldsL + li * kLdsTileBytes, t, acc);
      const TileStat st = half_reduce(acc, tile, t, it, any_greedy);
      if (h == 0) {
        const int slot = kPpRegTiles + 2 * li + t;
        s_mx[pb][slot][c] = st.mx;
        s_sum[pb][slot][c] = st.s;
        s_arg[pb][slot][c] = st.arg;
      }
    }
  };

  constexpr int kWaitAll = 0;   // s_waitcnt immediate: every counter at zero

  // One window of parity PB.  With two or more windows per position the
  // next window's previous tokens were drawn from statistics published one
  // or more windows ago: they are polled at the top, the rows gathered into
  // the other buffer as soon as they are in (mid-window), and only a late
  // draw makes the window end wait.  With one window per position the next
  // window needs this window's own draws: wait, gather, then go on.
  // `gc`: whether this wave gathers rows (waves 0..3).  The two kinds of
  // wave run separate copies of the loop, so that no row DMA appears in the
  // code the other waves run (the compiler makes every LDS access after a
  // possible DMA wait for all loads in flight, the base-logit ring included).
  auto window = [&](auto pbc, auto gc, int j) __attribute__((always_inline)) {
    constexpr int pb = decltype(pbc)::value;
    constexpr bool gat = decltype(gc)::value;
    char* nxt = pb ? ldsR0 : ldsR1;
    const bool more = j + 1 < nwin;
    if constexpr (gat) {
      int tok = 0;
      bool staged = !more || nch == 1;
      // the flag and temperature loads stay in flight during the register task
      const uint32_t pv = staged ? 0u : poll_issue(j + 1);
      const float tv = more ? temp_issue(j + 1) : 0.f;
      if (hasreg) run_task(pbc, j, true);
      if (ntask > 0) task_done(j);   // before the DMA: LDS accesses after it wait for it
      if (!staged) {
        if (!poll_check(j + 1, pv, tok)) wait_tokens(j + 1, tok);
        gather(j + 1, nxt, tok, tv);
      }
      __builtin_amdgcn_s_waitcnt(kWaitAll);   // this wave's rows are in
      __syncthreads();
      if (nch == 1 && more) {
        wait_tokens(j + 1, tok);
        gather(j + 1, nxt, tok, tv);
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        __syncthreads();
      }
    } else {
      if (hasreg) run_task(pbc, j, true);
      if (hashalf) run_task(pbc, j, false);
      if (ntask > 0) task_done(j);
      __syncthreads();
      if (nch == 1 && more) __syncthreads();
    }
  };

  // window 0: the anchors' rows
  if (threadIdx.x < 2) s_done[threadIdx.x] = 0;
  fetch_next(ring);
  auto run = [&](auto gc) __attribute__((always_inline)) {
    constexpr bool gat = decltype(gc)::value;
    if constexpr (gat) {
      int tok = 0;
      const float tv = temp_issue(0);
      poll_check(0, poll_issue(0), tok);
      gather(0, ldsR0, tok, tv);
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    for (int j = 0; j < nwin; j += 2) {
      window(std::integral_constant<int, 0>{}, gc, j);
      if (j + 1 < nwin) window(std::integral_constant<int, 1>{}, gc, j + 1);
    }
  };
  if (gathers) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

size_t draft_pipe_workspace_bytes(int B, int V) {
  return align256((size_t)B * n_tiles(V) * 8) + align256((size_t)B * kPpMaxTileGroups * 8) +
         align256((size_t)B * 4);
}

// Pt / Pd for this shape on a device with P compute units; false when the
// pipelined kernel cannot run (too few groups to keep every W2 tile on chip).
bool draft_pipe_plan(int B, int V, int P, int& Pt, int& Pd) {
  const int nT = n_tiles(V);
  Pd = min(kPpMaxDrawGroups, (B + kPpWaves - 1) / kPpWaves);
  Pt = min(min(P - Pd, nT), kPpMaxTileGroups);
  return Pd >= 1 && Pt >= 1 && (long long)Pt * kPpMaxTiles >= nT;
}

// Every work-group must be resident at once (they wait for one another):
// the grid is at most one work-group per compute unit and the occupancy
// check admits one per unit.  A plain launch on the stream's queue places
// them all as soon as the units are free; a cooperative launch guarantees
// it even beside other work on the device, but goes through a queue of its
// own, whose hand-over costs about 10 us on each side of the kernel.
template <int KS>
static hipError_t launch_pipe(const PpArgs& a0, bool coop, hipStream_t stream) {
  PpArgs a = a0;
  const void* kern = reinterpret_cast<const void*>(pdraft_pipe_kernel<KS>);
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kPpWaves * 64, 0) != hipSuccess ||
      occ < 1)
    return hipErrorNotSupported;
  TraceScope t("pdraft_pipe_kernel", stream);
  void* args[] = {&a};
  if (coop)
    return hipLaunchCooperativeKernel(kern, dim3(a.Pt + a.Pd), dim3(kPpWaves * 64), args, 0,
                                      stream);
  return hipLaunchKernel(kern, dim3(a.Pt + a.Pd), dim3(kPpWaves * 64), args, 0, stream);
}

hipError_t draft_pipe(int B, int gamma, int V, int rank, int P, long long spin_cap,
                      const uint16_t* U, const uint16_t* W1, const uint16_t* W2,
                      const int32_t* anchor, const float* temperature, const float* uniforms,
                      int32_t* tokens, float* q_tok, float* row_max, float* row_logZ,
                      int32_t* status, uint32_t* hdr, void* ws, const ConfIn* cf, bool coop,
                      hipStream_t stream) {
  PpArgs a;
  if (!draft_pipe_plan(B, V, P, a.Pt, a.Pd)) return hipErrorNotSupported;
  a.B = B; a.gamma = gamma; a.V = V; a.rank = rank;
  a.U = U; a.W1 = W1; a.W2 = W2; a.anchor = anchor; a.temperature = temperature;
  a.uniforms = uniforms; a.tokens = tokens; a.q_tok = q_tok; a.row_max = row_max;
  a.row_logZ = row_logZ; a.status = status;
  char* w = static_cast<char*>(ws);
  a.tw = reinterpret_cast<uint64_t*>(w);
  w += align256((size_t)B * n_tiles(V) * 8);
  a.gw = reinterpret_cast<uint64_t*>(w);
  w += align256((size_t)B * kPpMaxTileGroups * 8);
  a.tok_flag = reinterpret_cast<uint32_t*>(w);
  a.hdr = hdr;
  a.hidden = cf ? static_cast<const uint16_t*>(cf->hidden) : nullptr;
  a.cw = cf ? cf->w : nullptr;
  a.temps = cf ? cf->temps : nullptr;
  a.conf = cf ? cf->conf : nullptr;
  a.cbias = cf ? cf->bias : 0.f;
  a.H = cf ? cf->H : 0;
  a.spin_cap = spin_cap;
  switch (rank) {
    case 32: return launch_pipe<2>(a, coop, stream);
    case 64: return launch_pipe<4>(a, coop, stream);
    case 128: return launch_pipe<8>(a, coop, stream);
    default: return launch_pipe<16>(a, coop, stream);
  }
}

}  // namespace dspark
