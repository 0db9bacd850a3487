// libspecverify: batched speculative-sampling verification on gfx950.
//
// One persistent kernel, `flow_kernel`, serves the three verification entry
// points.  The work of a call is cut into units that workgroups claim from a
// shared counter:
//
//   statistics units (claimed first, in sequence order) -- stream a quarter
//       row (4 slices of 16384 tokens) once from HBM, double-buffered, and
//       reduce it to an exact base-2 softmax (reference, sum) pair
//       (spec_device.hpp).  They never wait for anything.
//   draw units -- published when the last statistics unit of a sequence
//       finishes: that workgroup merges the sequence's statistics, takes
//       every accept decision ([LT] §5.1, [CA] Key design 3), finds the first
//       rejection A and publishes one draw unit per slice.  A draw unit writes
//       per-512-token sub-tile masses of the sampling weights of the row pair
//       A ((pt - pd)+, or Cactus's (h - pd)+) or of the bonus row pt; the last
//       one to finish finds the inverse-CDF crossing and re-reads the single
//       sub-tile that holds it ([LT] §9.1: accepted length and the resampled
//       or bonus token).
//   gamma units -- published when every statistics unit of one position has
//       finished: sum_x min(pt, pd_i) over one slice for all N drafters (the
//       target slice stays in registers); the last one of a sequence forms
//       the HedgeSpec estimator and loss ([NB] Key designs 1-3).
//
// Published units go to a queue whose slots follow the statistics units in
// claim order, so a workgroup only ever waits when every statistics unit has
// been claimed and no published work is left.  A draw or gamma unit's
// sequence had its statistics streamed moments earlier, so its re-reads are
// served by the Infinity Cache.  Counters are reset by the last unit of each
// sequence and the claim counters by the last workgroup to exit, so the
// workspace counters are zero again when the kernel ends.
//
// [LT] "Speculative Decoding 为什么是 Lossless 的 -- 详细证明教程";
// [NB] HedgeSpec note "Not-a-Bandit: Provably No-Regret Drafter Selection ...";
// [CA] Cactus note; [NH] Chaudhuri, Freund, Hsu 2009 (NormalHedge).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_device.hpp"
#include "spec_verify.h"

namespace specv {

enum : uint32_t { ST_ACCEPT = 1, ST_REJECT = 2, ST_INVALID = 3 };
enum : int { MODE_VERIFY = 0, MODE_GAMMA = 1 };
// Sampling-weight modes of the draw passes.
enum : int { W_RESID = 0, W_TARGET_H = 1, W_TARGET = 2 };

constexpr int kTilesPerSlice = 8;
constexpr int kSliceTok = kTile * kTilesPerSlice;   // 16384 tokens per slice
constexpr int kSliceChunks = kSliceTok / kVec;      // 16-byte chunks per slice
constexpr int kSlicesPerUnit = 4;                   // slices one statistics unit streams
constexpr int kMaxSlices = (kMaxV + kSliceTok - 1) / kSliceTok;  // slices of the longest row
constexpr unsigned long long kWaitTicks = 200000000ull;  // bounded queue wait: 2 s of the 100 MHz clock
constexpr int kDecWords = 12;
enum : int { DYN_DRAW = 1, DYN_GAMMA = 2 };

// Everything a lane needs to turn logits into sampling weights (fp64).
struct WeightCtx {
  float c;
  float kt, kd;           // row references
  double inv_st, inv_sd;  // 1 / row sums
  double s_scale;         // Cactus rescale s of the non-candidate tokens (1.0 for SpS)
  double gstar;           // Cactus gamma* (the candidate's target mass)
  int n;                  // candidate token
  int special;            // 1: token n carries gamma* (delta > 0)
  int mode;               // W_RESID, W_TARGET_H, W_TARGET
};

struct Params {
  const uint16_t* target;
  int64_t t_stride;
  int t_rows;  // target rows per sequence in memory
  const uint16_t* draft;
  int64_t d_stride;
  int64_t drafter_stride;
  const int32_t* tokens;
  const float* r;
  const float* u;
  const int32_t* traj;
  const int32_t* sel;
  int B, K, N, V;
  float c;  // log2(e) / T
  double delta;
  int mode;
  int fused;
  // units
  int R;     // statistic rows per sequence
  int RT;    // of which target rows
  int S;     // slices per row
  int Q;     // statistics units per row (kSlicesPerUnit slices each)
  int nsub;  // 512-token sub-tiles per row
  int U1;    // statistics units per sequence
  int U3;    // final steps per sequence (estimator and / or draw)
  int n_static, total_units;
  int queue_cap;  // queue slots in the workspace
  // outputs
  int32_t* accepted_len;
  int32_t* out_token;
  uint8_t* accept_mask;
  float* gamma_star;
  float* gamma;
  float* est_len;
  float* loss;
  // workspace: counters
  uint32_t* work;    // [0] claim counter, [1] exit counter, [2] queue tail, [3] fault flag
  uint32_t* p1cnt;   // [B][K+1] finished statistics units per (sequence, position)
  uint32_t* p1all;   // [B] finished statistics units per sequence
  uint32_t* p2cnt;   // [B] finished draw units
  uint32_t* p2gcnt;  // [B] finished gamma units
  uint32_t* done;    // [B] finished final steps
  unsigned long long* queue;  // published units (0 = slot not yet filled)
  // workspace: scratch
  float* stat_k;   // [B][R][Q]
  double* stat_s;  // [B][R][Q]
  double* subsum;  // [B][nsub]
  double* gpart;   // [B][K][N][S]
  double* dec;     // [B][kDecWords]
};

__device__ __forceinline__ const uint4* as_chunks(const uint16_t* row) { return reinterpret_cast<const uint4*>(row); }

__device__ __forceinline__ const uint16_t* target_row(const Params& p, int b, int k) {
  return p.target + (static_cast<int64_t>(b) * p.t_rows + k) * p.t_stride;
}
__device__ __forceinline__ const uint16_t* draft_row(const Params& p, int b, int i, int k) {
  return p.draft + static_cast<int64_t>(i) * p.drafter_stride + (static_cast<int64_t>(b) * p.K + k) * p.d_stride;
}
// Statistic row r of a sequence: r < RT target row r, else drafter (r - RT) / K, position (r - RT) % K.
__device__ __forceinline__ const uint16_t* stat_row(const Params& p, int b, int r) {
  if (r < p.RT) return target_row(p, b, r);
  const int j = r - p.RT;
  return draft_row(p, b, j / p.K, j % p.K);
}
__device__ __forceinline__ int counter_of(const Params& p, int r) {
  if (p.mode == MODE_VERIFY) return 0;
  return r < p.RT ? r : (r - p.RT) % p.K;
}
__device__ __forceinline__ uint32_t p1_target(const Params& p, int k) {
  if (p.mode == MODE_VERIFY) return static_cast<uint32_t>(p.R * p.Q);
  return static_cast<uint32_t>((1 + p.N) * p.Q);  // k < K
}

// Merge the per-unit statistics of one row into (k, s): exact power-of-two rescaling.
__device__ __forceinline__ RowStats merge_row(const Params& p, int b, int r) {
  const size_t base = (static_cast<size_t>(b) * p.R + r) * p.Q;
  uint32_t* kp = reinterpret_cast<uint32_t*>(p.stat_k + base);
  float km = kNoRef;
  for (int s = 0; s < p.Q; ++s) km = fmaxf(km, __uint_as_float(ld_agent(kp + s)));
  double tot = 0.0;
  for (int s = 0; s < p.Q; ++s) {
    const float ks = __uint_as_float(ld_agent(kp + s));
    tot += ldexp(ld_agent_d(p.stat_s + base + s), static_cast<int>(fmaxf(ks - km, -2000.0f)));
  }
  return RowStats{km, tot};
}

// ---------------------------------------------------------------------------
// Sampling weights, sub-tile search and token search
// ---------------------------------------------------------------------------

// Sampling weight of one token:
//   W_RESID    (h - pd)+ with h = s * pt, h_n = gamma*   ([LT] §2.2 / [CA] Key design 2)
//   W_TARGET_H h          (a rejection with zero residual mass)
//   W_TARGET   pt         (bonus token)
__device__ __forceinline__ double weight1(const WeightCtx& w, float zt, float zd, int tok) {
  const double pt = static_cast<double>(fast_exp2(fmaf(zt, w.c, -w.kt))) * w.inv_st;
  if (w.mode == W_TARGET) return pt;
  double h = w.s_scale * pt;
  if (w.special && tok == w.n) h = w.gstar;
  if (w.mode == W_TARGET_H) return h;
  const double pd = static_cast<double>(fast_exp2(fmaf(zd, w.c, -w.kd))) * w.inv_sd;
  return fmax(h - pd, 0.0);
}

// Weights of eight consecutive tokens starting at `tok0`.
__device__ __forceinline__ void weights8(const WeightCtx& w, const float zt[8], const float zd[8], int tok0,
                                         double out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = weight1(w, zt[e], zd[e], tok0 + e);
}

// Wave 0: the sub-tile holding the crossing of x = u * Z, Z = sum of subsum[].
// Returns false when Z is not positive.  x_rel is x minus the mass before the
// sub-tile, or +inf when rounding left no crossing (the last positive-mass
// token is then taken).
__device__ __forceinline__ bool find_subtile(const double* subsum, int nsub, double u, int& s_star, double& x_rel) {
  const int lane = lane_id();
  const int per = (nsub + 63) / 64;
  const int lo = min(lane * per, nsub), hi = min(lo + per, nsub);
  double ls = 0.0;
  for (int s = lo; s < hi; ++s) ls += subsum[s];
  const double incl = wave_incl_scan(ls);
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  const double Z = __shfl(incl, 63, 64);
  if (!(Z > 0.0)) return false;
  const double x = u * Z;
  const unsigned long long m = __ballot(incl > x);
  const bool clamp = (m == 0ull);
  int L;
  if (!clamp) {
    L = __ffsll(static_cast<long long>(m)) - 1;
  } else {
    const unsigned long long pos = __ballot(ls > 0.0);
    L = 63 - __clzll(static_cast<long long>(pos));
  }
  int ss = -1;
  double P = 0.0;
  int lane_clamp = 0;
  if (lane == L) {
    double run = excl;
    if (!clamp) {
      for (int s = lo; s < hi; ++s) {
        const double nr = run + subsum[s];
        if (nr > x) {
          ss = s;
          P = run;
          break;
        }
        run = nr;
      }
    }
    if (ss < 0) {
      lane_clamp = 1;
      run = excl;
      for (int s = lo; s < hi; ++s) {
        if (subsum[s] > 0.0) {
          ss = s;
          P = run;
        }
        run += subsum[s];
      }
    }
  }
  s_star = __shfl(ss, L, 64);
  P = __shfl(P, L, 64);
  lane_clamp = __shfl(lane_clamp, L, 64);
  x_rel = (clamp || lane_clamp) ? __builtin_inf() : x - P;
  return s_star >= 0;
}

// Wave 0: the token in sub-tile s_star where the running mass passes x_rel
// (or the sub-tile's last positive-mass token when x_rel is +inf).  Recomputes
// the sub-tile's weights and lane scan exactly as the draw pass did.
template <bool PAIR>
__device__ __forceinline__ int find_token(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w, int s_star,
                          double x_rel) {
  const int lane = lane_id();
  const int nchunks = (V + kVec - 1) / kVec;
  const int ci = s_star * 64 + lane;
  double wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  double ls = 0.0;
  if (ci < nchunks) {
    const int valid = V - ci * kVec;
    float zt[8], zd[8];
    unpack8(as_chunks(trow)[ci], zt, valid);
    if (PAIR)
      unpack8(as_chunks(drow)[ci], zd, valid);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) zd[e] = -__builtin_inff();
    weights8(w, zt, zd, ci * kVec, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e) ls += wv[e];
  }
  const double incl = wave_incl_scan(ls);
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  const unsigned long long pos = __ballot(ls > 0.0);
  if (pos == 0ull) return -1;
  const unsigned long long m = __ballot(incl > x_rel);
  const bool clamp = (m == 0ull);
  const int L = clamp ? 63 - __clzll(static_cast<long long>(pos)) : __ffsll(static_cast<long long>(m)) - 1;
  int tok = -1;
  if (lane == L) {
    // first element whose running mass passes x_rel; else the lane's last positive element
    int e_star = -1, e_last = -1;
    double run = excl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (wv[e] > 0.0) e_last = e;
      run += wv[e];
      if (!clamp && e_star < 0 && wv[e] > 0.0 && run > x_rel) e_star = e;
    }
    if (e_star < 0) e_star = e_last;
    tok = e_star >= 0 ? ci * kVec + e_star : -1;
  }
  tok = __shfl(tok, L, 64);
  if (tok < 0) {  // rounding put the crossing on a zero-mass lane: last positive token of the sub-tile
    const int Lp = 63 - __clzll(static_cast<long long>(pos));
    int t2 = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (wv[e] > 0.0) t2 = ci * kVec + e;
    tok = __shfl(t2, Lp, 64);
  }
  return tok;
}

// Per-sub-tile masses of the sampling weights over tiles [t0, t0 + ntiles) of a
// row (pair); lane 63 of each wave stores the sub-tile's inclusive scan total.
// Used for a draw slice (to global memory) and for the whole-row fallback (to LDS).
template <bool PAIR, bool TO_GLOBAL>
__device__ __forceinline__ void weight_subtiles(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w,
                                                int t0, int ntiles, double* subsum, int nsub) {
  const uint4* tr = as_chunks(trow);
  const uint4* dr = as_chunks(drow);
  const int nchunks = (V + kVec - 1) / kVec;
  const int tid = threadIdx.x;
  constexpr int kBatch = 4;
#pragma unroll 1
  for (int j0 = 0; j0 < ntiles; j0 += kBatch) {
    uint4 vt[kBatch], vd[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int ci = (t0 + j0 + q) * kThreads + tid;
      if (j0 + q < ntiles && ci < nchunks) {
        vt[q] = tr[ci];
        if (PAIR) vd[q] = dr[ci];
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (j0 + q >= ntiles) break;  // uniform over the workgroup
      const int jt = t0 + j0 + q;
      const int ci = jt * kThreads + tid;
      double lsum = 0.0;
      if (ci < nchunks) {
        const int valid = V - ci * kVec;
        float zt[8], zd[8];
        unpack8(vt[q], zt, valid);
        if (PAIR)
          unpack8(vd[q], zd, valid);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) zd[e] = -__builtin_inff();
        // same element order as find_token's lane sum, so the two agree bit for bit
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum += weight1(w, zt[e], zd[e], ci * kVec + e);
      }
      const double incl = wave_incl_scan(lsum);
      const int s = jt * kWaves + wave_id();
      if (lane_id() == 63 && s < nsub) {
        if (TO_GLOBAL)
          st_agent_d(&subsum[s], incl);
        else
          subsum[s] = incl;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-sequence decisions (block-wide)
// ---------------------------------------------------------------------------

struct Decision {
  WeightCtx w;
  int A;         // accepted length; -1 invalid
  int draw_row;  // position of the draw row (A, or K for the bonus)
  int pair;      // 1: residual over (target A, draft A); 0: pt of target row K
};

struct DecideLds {
  float rk[2 * SPEC_MAX_K + 1];
  double rs[2 * SPEC_MAX_K + 1];
  uint32_t state[SPEC_MAX_K];
  double ct[SPEC_MAX_K];
  double gs[SPEC_MAX_K];
  Decision d;
};

// Merge the statistics of target rows 0..K and drafter `drafter`'s rows 0..K-1,
// take every accept decision, and describe the draw.  Writes accept_mask and
// gamma_star when `write_outputs`.  The result is in L.d after the call.
__device__ __forceinline__ void decide(const Params& p, int b, int drafter, bool write_outputs, DecideLds& L) {
  const int K = p.K, V = p.V;
  const int t = threadIdx.x;
  const bool bad_sel = drafter < 0 || drafter >= p.N;
  if (!bad_sel && t < 2 * K + 1) {
    const int r = t <= K ? t : p.RT + drafter * K + (t - K - 1);
    const RowStats st = merge_row(p, b, r);
    L.rk[t] = st.k;
    L.rs[t] = st.s;
  }
  __syncthreads();
  if (t < K) {
    uint32_t state = ST_INVALID;
    bool acc = false;
    const int n = p.tokens[b * K + t];
    if (!bad_sel && n >= 0 && n < V) {
      const RowStats st{L.rk[t], L.rs[t]};
      const RowStats sd{L.rk[K + 1 + t], L.rs[K + 1 + t]};
      // [CA] Key design 3 with the verifier's probability c of the candidate; delta = 0 is SpS.
      const double ct = fmin(token_prob(bf16_at(target_row(p, b, t), n), p.c, st), 1.0);
      const double cd = token_prob(bf16_at(draft_row(p, b, drafter, t), n), p.c, sd);
      const double gs = fmin(ct + sqrt(2.0 * p.delta * ct * (1.0 - ct)), 1.0);
      const double ratio = cd > 0.0 ? gs / cd : (gs > 0.0 ? __builtin_inf() : 0.0);
      acc = static_cast<double>(p.r[b * K + t]) < ratio;  // [LT] §5.1: strict
      state = acc ? ST_ACCEPT : ST_REJECT;
      L.ct[t] = ct;
      L.gs[t] = gs;
      if (write_outputs && p.gamma_star) p.gamma_star[b * K + t] = static_cast<float>(gs);
    }
    if (write_outputs && p.accept_mask) p.accept_mask[b * K + t] = acc ? 1 : 0;
    L.state[t] = state;
  }
  __syncthreads();
  if (t == 0) {
    Decision d;
    int A = K;
    bool bad = bad_sel;
    for (int q = 0; q < K; ++q) {
      bad |= (L.state[q] == ST_INVALID);
      if (L.state[q] == ST_REJECT && A == K) A = q;
    }
    WeightCtx w;
    w.c = p.c;
    w.kd = 0.0f;
    w.inv_sd = 1.0;
    w.s_scale = 1.0;
    w.gstar = 0.0;
    w.n = -1;
    w.special = 0;
    if (bad) {
      d.A = -1;
      d.draw_row = 0;
      d.pair = 0;
      w.mode = W_TARGET;
      w.kt = 0.0f;
      w.inv_st = 1.0;
    } else if (A < K) {
      // [LT] §9.1: the first rejection A is resampled from the residual of its row pair
      const double ct = L.ct[A], gs = L.gs[A];
      d.A = A;
      d.draw_row = A;
      d.pair = 1;
      w.mode = W_RESID;
      w.kt = L.rk[A];
      w.inv_st = 1.0 / L.rs[A];
      w.kd = L.rk[K + 1 + A];
      w.inv_sd = 1.0 / L.rs[K + 1 + A];
      w.s_scale = ct < 1.0 ? (1.0 - gs) / (1.0 - ct) : 0.0;  // [CA] Key design 2 (1.0 exactly at delta = 0)
      w.gstar = gs;
      w.n = p.tokens[b * K + A];
      w.special = p.delta > 0.0 ? 1 : 0;
    } else {
      // every draft kept: bonus token from target row K
      d.A = K;
      d.draw_row = K;
      d.pair = 0;
      w.mode = W_TARGET;
      w.kt = L.rk[K];
      w.inv_st = 1.0 / L.rs[K];
    }
    d.w = w;
    L.d = d;
  }
  __syncthreads();
}

__device__ __forceinline__ void store_decision(double* rec, const Decision& d) {
  st_agent_d(rec + 0, static_cast<double>(d.A));
  st_agent_d(rec + 1, static_cast<double>(d.draw_row));
  st_agent_d(rec + 2, static_cast<double>(d.pair));
  st_agent_d(rec + 3, static_cast<double>(d.w.kt));
  st_agent_d(rec + 4, static_cast<double>(d.w.kd));
  st_agent_d(rec + 5, d.w.inv_st);
  st_agent_d(rec + 6, d.w.inv_sd);
  st_agent_d(rec + 7, d.w.s_scale);
  st_agent_d(rec + 8, d.w.gstar);
  st_agent_d(rec + 9, static_cast<double>(d.w.n));
  st_agent_d(rec + 10, static_cast<double>(d.w.special));
  st_agent_d(rec + 11, static_cast<double>(d.w.mode));
}

__device__ __forceinline__ Decision load_decision(double* rec, float c) {
  Decision d;
  d.A = static_cast<int>(ld_agent_d(rec + 0));
  d.draw_row = static_cast<int>(ld_agent_d(rec + 1));
  d.pair = static_cast<int>(ld_agent_d(rec + 2));
  d.w.c = c;
  d.w.kt = static_cast<float>(ld_agent_d(rec + 3));
  d.w.kd = static_cast<float>(ld_agent_d(rec + 4));
  d.w.inv_st = ld_agent_d(rec + 5);
  d.w.inv_sd = ld_agent_d(rec + 6);
  d.w.s_scale = ld_agent_d(rec + 7);
  d.w.gstar = ld_agent_d(rec + 8);
  d.w.n = static_cast<int>(ld_agent_d(rec + 9));
  d.w.special = static_cast<int>(ld_agent_d(rec + 10));
  d.w.mode = static_cast<int>(ld_agent_d(rec + 11));
  return d;
}

// ---------------------------------------------------------------------------
// Units
// ---------------------------------------------------------------------------

struct Lds {
  double subsum[kMaxSub];
  double scratch[2 * kWaves];
  double part[SPEC_MAX_N * kWaves];
  float lt;
  float ld[SPEC_MAX_N];
  DecideLds dl;
  int flag;
  unsigned long long desc;
};

__device__ __forceinline__ void load_slice(const uint4* rc, int c0, int nchunks, uint4 v[kTilesPerSlice]) {
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    const int ci = c0 + t * kThreads + static_cast<int>(threadIdx.x);
    if (ci < nchunks) v[t] = rc[ci];
  }
}

__device__ __forceinline__ void acc_slice(const uint4 v[kTilesPerSlice], int c0, int nchunks, int V, float c,
                                          RowAcc& a) {
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    const int ci = c0 + t * kThreads + static_cast<int>(threadIdx.x);
    if (ci < nchunks) {
      float z[8];
      unpack8(v[t], z, V - ci * kVec);
      row_acc_add8(a, z, c);
    }
  }
}

__device__ __forceinline__ int draw_drafter(const Params& p, int b) { return p.mode == MODE_VERIFY ? 0 : p.sel[b]; }

__device__ __forceinline__ unsigned long long dyn_desc(int type, int b, int k, int s) {
  return (static_cast<unsigned long long>(type) << 56) | (static_cast<unsigned long long>(b) << 32) |
         (static_cast<unsigned long long>(k) << 16) | static_cast<unsigned long long>(s);
}

// Thread 0: append a unit to the queue.  A slot past the capacity can only come from
// counters that did not start at zero: it is not written, and the fault flag is set.
__device__ __forceinline__ void publish(const Params& p, int type, int b, int k, int s) {
  const uint32_t slot = ticket(&p.work[2]);
  if (slot < static_cast<uint32_t>(p.queue_cap))
    st_agent_u64(&p.queue[slot], dyn_desc(type, b, k, s));
  else
    st_agent(&p.work[3], 3u);
}

// Thread 0 after a sequence's final step: the last one resets the sequence's counters
// (by then every other unit of the sequence has finished).
__device__ __forceinline__ void finish_sequence(const Params& p, int b) {
  const uint32_t old = ticket(&p.done[b]);
  if (old == static_cast<uint32_t>(p.U3 - 1)) {
    for (int k = 0; k <= p.K; ++k) st_agent(&p.p1cnt[b * (p.K + 1) + k], 0u);
    st_agent(&p.p1all[b], 0u);
    st_agent(&p.p2cnt[b], 0u);
    st_agent(&p.p2gcnt[b], 0u);
    st_agent(&p.done[b], 0u);
  }
}

// A sequence's statistics are complete: take its decisions (block-wide), record
// them, and publish its draw units.
__device__ __forceinline__ void start_draws(const Params& p, int b, Lds& L) {
  decide(p, b, draw_drafter(p, b), true, L.dl);
  if (threadIdx.x == 0) {
    store_decision(p.dec + static_cast<size_t>(b) * kDecWords, L.dl.d);
    stores_complete();
    for (int s = 0; s < p.S; ++s) publish(p, DYN_DRAW, b, 0, s);
  }
}

// Statistics unit: slices [j * kSlicesPerUnit, ...) of statistic row r of sequence b,
// double-buffered.  Thread 0 issues the next claim once the first loads are out.
__device__ __forceinline__ void unit_stats(const Params& p, int b, int r, int j, Lds& L, uint32_t* claim) {
  const uint4* rc = as_chunks(stat_row(p, b, r));
  const int nchunks = (p.V + kVec - 1) / kVec;
  const int s0 = j * kSlicesPerUnit;
  const int cnt = min(kSlicesPerUnit, p.S - s0);
  uint4 va[kTilesPerSlice], vb[kTilesPerSlice];
  RowAcc a = row_acc_init();
  load_slice(rc, s0 * kSliceChunks, nchunks, va);
  if (threadIdx.x == 0) *claim = ticket(&p.work[0]);
#pragma unroll 1
  for (int q = 0; q < cnt; q += 2) {
    if (q + 1 < cnt) load_slice(rc, (s0 + q + 1) * kSliceChunks, nchunks, vb);
    acc_slice(va, (s0 + q) * kSliceChunks, nchunks, p.V, p.c, a);
    if (q + 1 < cnt) {
      if (q + 2 < cnt) load_slice(rc, (s0 + q + 2) * kSliceChunks, nchunks, va);
      acc_slice(vb, (s0 + q + 1) * kSliceChunks, nchunks, p.V, p.c, a);
    }
  }
  const RowStats st = block_row_stats(a, L.scratch);
  if (threadIdx.x == 0) {
    const size_t idx = (static_cast<size_t>(b) * p.R + r) * p.Q + j;
    st_agent(reinterpret_cast<uint32_t*>(p.stat_k + idx), __float_as_uint(st.k));
    st_agent_d(p.stat_s + idx, st.s);
    stores_complete();
    int fl = 0;
    if (p.mode == MODE_VERIFY) {
      if (ticket(&p.p1cnt[b * (p.K + 1)]) == static_cast<uint32_t>(p.R * p.Q - 1)) fl |= 1;
    } else {
      if (r < p.K || r >= p.RT) {  // a row of position k < K: target row k or a drafter row
        const int k = counter_of(p, r);
        if (ticket(&p.p1cnt[b * (p.K + 1) + k]) == p1_target(p, k) - 1) {
          for (int s = 0; s < p.S; ++s) publish(p, DYN_GAMMA, b, k, s);
        }
      }
      if (p.fused && ticket(&p.p1all[b]) == static_cast<uint32_t>(p.R * p.Q - 1)) fl |= 1;
    }
    L.flag = fl;
  }
  __syncthreads();
  if (L.flag & 1) start_draws(p, b, L);
}

// Last draw unit of a sequence: the inverse-CDF crossing and the output token.
__device__ __forceinline__ void draw_final(const Params& p, int b, const Decision& d, Lds& L) {
  const bool ok = d.A >= 0;
  int token = -1;
  if (ok) {
    for (int q = threadIdx.x; q < p.nsub; q += kThreads)
      L.subsum[q] = ld_agent_d(p.subsum + static_cast<size_t>(b) * p.nsub + q);
    __syncthreads();
    const uint16_t* trow = target_row(p, b, d.draw_row);
    const uint16_t* drow = d.pair ? draft_row(p, b, draw_drafter(p, b), d.draw_row) : trow;
    const double uu = static_cast<double>(p.u[b * (p.K + 1) + d.draw_row]);
    if (wave_id() == 0) {
      int s_star = -1;
      double x_rel = 0.0;
      const bool found = find_subtile(L.subsum, p.nsub, uu, s_star, x_rel);
      int tok = -2;  // -2: no mass (zero residual)
      if (found)
        tok = d.pair ? find_token<true>(trow, drow, p.V, d.w, s_star, x_rel)
                     : find_token<false>(trow, drow, p.V, d.w, s_star, x_rel);
      if (lane_id() == 0) L.flag = tok;
    }
    __syncthreads();
    token = L.flag;
    __syncthreads();
    if (token == -2) {
      // zero residual mass on a rejection: draw from the position's target h instead (whole row, rare)
      WeightCtx wh = d.w;
      wh.mode = W_TARGET_H;
      const int ntiles = (p.V + kTile - 1) / kTile;
      weight_subtiles<false, false>(trow, trow, p.V, wh, 0, ntiles, L.subsum, p.nsub);
      __syncthreads();
      if (wave_id() == 0) {
        int s_star = -1;
        double x_rel = 0.0;
        int tok = -1;
        if (find_subtile(L.subsum, p.nsub, uu, s_star, x_rel))
          tok = find_token<false>(trow, trow, p.V, wh, s_star, x_rel);
        if (lane_id() == 0) L.flag = tok;
      }
      __syncthreads();
      token = L.flag;
    }
  }
  if (threadIdx.x == 0) {
    const bool good = ok && token >= 0;
    p.accepted_len[b] = good ? d.A : -1;
    p.out_token[b] = good ? token : -1;
    finish_sequence(p, b);
  }
}

// Draw unit: sub-tile masses of slice s of sequence b's draw row(s).
__device__ __forceinline__ void unit_draw(const Params& p, int b, int s, Lds& L) {
  if (threadIdx.x == 0) {
    Decision d = load_decision(p.dec + static_cast<size_t>(b) * kDecWords, p.c);
    // a record is used only if it describes a draw row of this call
    if (d.A < -1 || d.A > p.K || d.draw_row < 0 || d.draw_row > p.K || (d.pair && d.draw_row >= p.K)) {
      d.A = -1;
      st_agent(&p.work[3], 4u);
    }
    L.dl.d = d;
  }
  __syncthreads();
  const Decision d = L.dl.d;
  if (d.A >= 0) {
    const uint16_t* trow = target_row(p, b, d.draw_row);
    double* out = p.subsum + static_cast<size_t>(b) * p.nsub;
    const int t0 = s * kTilesPerSlice;
    if (d.pair)
      weight_subtiles<true, true>(trow, draft_row(p, b, draw_drafter(p, b), d.draw_row), p.V, d.w, t0,
                                  kTilesPerSlice, out, p.nsub);
    else
      weight_subtiles<false, true>(trow, trow, p.V, d.w, t0, kTilesPerSlice, out, p.nsub);
  }
  stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) L.flag = ticket(&p.p2cnt[b]) == static_cast<uint32_t>(p.S - 1) ? 1 : 0;
  __syncthreads();
  if (L.flag) draw_final(p, b, d, L);
}

// Last gamma unit of a sequence: gamma, the estimator and the loss of every drafter.
__device__ __forceinline__ void estimate(const Params& p, int b) {
  const int tid = threadIdx.x;
  if (tid < p.N) {
    const int i = tid, K = p.K;
    // [NB] Key design 2 (reading: L = 1 + sum_k gamma_k prod_{j<k} a_j) and Key design 3 (f = K + 1 - L)
    double Lh = 1.0, prod = 1.0;
    for (int k = 0; k < K; ++k) {
      double g = 0.0;
      const size_t gi = ((static_cast<size_t>(b) * K + k) * p.N + i) * p.S;
      for (int s = 0; s < p.S; ++s) g += ld_agent_d(p.gpart + gi + s);
      p.gamma[(b * K + k) * p.N + i] = static_cast<float>(g);
      Lh += g * prod;
      if (k < K - 1) {
        double a;
        const int x = p.traj[b * K + k];
        if (x < 0 || x >= p.V) {
          a = __builtin_nan("");
        } else {
          const RowStats st = merge_row(p, b, k);
          const RowStats sd = merge_row(p, b, p.RT + i * K + k);
          const double ptx = token_prob(bf16_at(target_row(p, b, k), x), p.c, st);
          const double pdx = token_prob(bf16_at(draft_row(p, b, i, k), x), p.c, sd);
          a = ptx > 0.0 ? fmin(1.0, pdx / ptx) : (pdx > 0.0 ? 1.0 : 0.0);
        }
        prod *= a;
      }
    }
    p.est_len[b * p.N + i] = static_cast<float>(Lh);
    p.loss[b * p.N + i] = static_cast<float>(static_cast<double>(K + 1) - Lh);
  }
  __syncthreads();
  if (tid == 0) finish_sequence(p, b);
}

// Gamma unit: sum_x min(pt_k, pd_{i,k}) over slice s for every drafter i.
__device__ __forceinline__ void unit_gamma(const Params& p, int b, int k, int s, Lds& L) {
  const int tid = threadIdx.x;
  // log2 normalisers L = k + log2(s) of the target row and the N drafter rows
  if (tid <= p.N) {
    const int r = tid == 0 ? k : p.RT + (tid - 1) * p.K + k;
    const RowStats st = merge_row(p, b, r);
    const float lv = static_cast<float>(static_cast<double>(st.k) + log2(st.s));
    if (tid == 0)
      L.lt = lv;
    else
      L.ld[tid - 1] = lv;
  }
  for (int i = tid; i < p.N * kWaves; i += kThreads) L.part[i] = 0.0;
  __syncthreads();
  const float c = p.c, lt = L.lt;
  const int nchunks = (p.V + kVec - 1) / kVec;
  const uint4* tr = as_chunks(target_row(p, b, k));
  constexpr int kHalf = kTilesPerSlice / 2;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    const int c0 = s * kSliceChunks + h * kHalf * kThreads;
    uint4 vt[kHalf], vd[kHalf], vn[kHalf];
#pragma unroll
    for (int t = 0; t < kHalf; ++t) {
      const int ci = c0 + t * kThreads + tid;
      if (ci < nchunks) {
        vt[t] = tr[ci];
        vd[t] = as_chunks(draft_row(p, b, 0, k))[ci];
      }
    }
#pragma unroll 1
    for (int i = 0; i < p.N; ++i) {
      if (i + 1 < p.N) {  // prefetch the next drafter's half-slice
        const uint4* dn = as_chunks(draft_row(p, b, i + 1, k));
#pragma unroll
        for (int t = 0; t < kHalf; ++t) {
          const int ci = c0 + t * kThreads + tid;
          if (ci < nchunks) vn[t] = dn[ci];
        }
      }
      const float ld = L.ld[i];
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < kHalf; ++t) {
        const int ci = c0 + t * kThreads + tid;
        if (ci < nchunks) {
          const int valid = p.V - ci * kVec;
          float zt[8], zd[8], e[8];
          unpack8(vt[t], zt, valid);
          unpack8(vd[t], zd, valid);
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = fast_exp2(fminf(fmaf(zt[q], c, -lt), fmaf(zd[q], c, -ld)));
          acc += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        }
      }
      const double g = wave_sum(static_cast<double>(acc));
      if (lane_id() == 0) L.part[i * kWaves + wave_id()] += g;
#pragma unroll
      for (int t = 0; t < kHalf; ++t) vd[t] = vn[t];
    }
  }
  __syncthreads();
  if (tid < p.N) {
    double g = 0.0;
    for (int w = 0; w < kWaves; ++w) g += L.part[tid * kWaves + w];
    st_agent_d(p.gpart + ((static_cast<size_t>(b) * p.K + k) * p.N + tid) * p.S + s, g);
  }
  stores_complete();
  __syncthreads();
  if (tid == 0) L.flag = ticket(&p.p2gcnt[b]) == static_cast<uint32_t>(p.K * p.S - 1) ? 1 : 0;
  __syncthreads();
  if (L.flag) estimate(p, b);
}

// ---------------------------------------------------------------------------
// The persistent kernel
// ---------------------------------------------------------------------------

#ifdef SPEC_TRACE
// Diagnostic build only: per-unit timestamps (start, end) and workgroup.
__device__ unsigned long long g_trace[1 << 17][3];
#endif

// Statistics unit h: sequence-major; within a sequence, verify rows in order, gamma rows
// grouped by position (target row k, then every drafter's row k), the bonus row last.
__device__ __forceinline__ void run_static(const Params& p, int h, Lds& L, uint32_t* claim) {
  const int b = h / p.U1, loc = h % p.U1;
  const int slot = loc / p.Q, j = loc % p.Q;
  int r;
  if (p.mode == MODE_VERIFY) {
    r = slot;
  } else if (slot < p.K * (1 + p.N)) {
    const int k = slot / (1 + p.N), t = slot % (1 + p.N);
    r = t == 0 ? k : p.RT + (t - 1) * p.K + k;
  } else {
    r = p.K;  // fused: target row K (bonus)
  }
  unit_stats(p, b, r, j, L, claim);
}

// SPEC_FLOW_WAVES_PER_EU (compile time) caps registers for that many waves per SIMD.
#ifdef SPEC_FLOW_WAVES_PER_EU
__global__ __launch_bounds__(kThreads, SPEC_FLOW_WAVES_PER_EU) void flow_kernel(Params p) {
#else
__global__ __launch_bounds__(kThreads) void flow_kernel(Params p) {
#endif
  __shared__ Lds L;
  __shared__ int sh_unit;
  if (threadIdx.x == 0) sh_unit = static_cast<int>(ticket(&p.work[0]));
  __syncthreads();
  int u = sh_unit;
  while (u < p.total_units) {
    __syncthreads();
#ifdef SPEC_TRACE
    const unsigned long long t_start = wall_clock64();
#endif
    uint32_t nxt = 0;
    if (u < p.n_static) {
      run_static(p, u, L, &nxt);
    } else {
      if (threadIdx.x == 0) {
        nxt = ticket(&p.work[0]);
        // a queue slot: wait until its unit is published (only when nothing else is left)
        unsigned long long* slot = &p.queue[u - p.n_static];
        unsigned long long d = ld_agent_u64(slot);
        const unsigned long long t0 = wall_clock64();
        while (d == 0ull) {
          if (wall_clock64() - t0 > kWaitTicks) {
            st_agent(&p.work[3], 1u);  // fault: a published unit never arrived
            break;
          }
          __builtin_amdgcn_s_sleep(2);
          d = ld_agent_u64(slot);
        }
        st_agent_u64(slot, 0ull);
        L.desc = d;
      }
      __syncthreads();
      const unsigned long long d = L.desc;
      if (d != 0ull) {
        const int type = static_cast<int>(d >> 56);
        const int b = static_cast<int>((d >> 32) & 0xffffffull);
        const int k = static_cast<int>((d >> 16) & 0xffffull);
        const int s = static_cast<int>(d & 0xffffull);
        // a descriptor is used only if every field is in range (a corrupt slot sets the fault flag)
        const bool ok = b < p.B && s < p.S &&
                        ((type == DYN_DRAW && (p.mode == MODE_VERIFY || p.fused)) ||
                         (type == DYN_GAMMA && p.mode == MODE_GAMMA && k < p.K));
        if (!ok) {
          if (threadIdx.x == 0) st_agent(&p.work[3], 2u);
        } else if (type == DYN_DRAW) {
          unit_draw(p, b, s, L);
        } else {
          unit_gamma(p, b, k, s, L);
        }
      }
    }
    __syncthreads();
#ifdef SPEC_TRACE
    if (threadIdx.x == 0 && u < (1 << 17)) {
      g_trace[u][0] = t_start;
      g_trace[u][1] = wall_clock64();
      g_trace[u][2] = blockIdx.x;
    }
#endif
    if (threadIdx.x == 0) sh_unit = static_cast<int>(nxt);
    __syncthreads();
    u = sh_unit;
  }
  if (threadIdx.x == 0) {
    if (ticket(&p.work[1]) == gridDim.x - 1) {  // every other workgroup has left
      st_agent(&p.work[0], 0u);
      st_agent(&p.work[1], 0u);
      st_agent(&p.work[2], 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// NormalHedge ([NH]); one wave per sequence, lane i = drafter i.
// ---------------------------------------------------------------------------
constexpr int kHedgeBisect = 64;

__global__ __launch_bounds__(64) void hedge_kernel(double* R, double* W, const float* loss, const uint8_t* has,
                                                   float scale, const float* v, int32_t* sel, int N) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool act = i < N;
  const int idx = b * N + i;
  double wfinal = act ? W[idx] : 0.0;
  if (has == nullptr || has[b] != 0) {
    const double l = act ? static_cast<double>(loss[idx]) * static_cast<double>(scale) : 0.0;
    const double wi = act ? W[idx] : 0.0;
    const double lhat = wave_sum(wi * l);
    const double Ri = act ? R[idx] + (lhat - l) : 0.0;
    const double rp = act ? fmax(Ri, 0.0) : 0.0;
    double M = rp;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmax(M, __shfl_xor(M, m, 64));
    double wn;
    if (M > 0.0) {
      // (1/N) sum exp(rp^2 / 2c) = e, bisection on [M^2 / (2 (1 + ln N)), M^2 / 2]
      double lo = M * M / (2.0 * (1.0 + log(static_cast<double>(N))));
      double hi = M * M / 2.0;
      for (int it = 0; it < kHedgeBisect; ++it) {
        const double mid = 0.5 * (lo + hi);
        const double f = wave_sum(act ? exp(rp * rp / (2.0 * mid)) : 0.0) / static_cast<double>(N);
        if (f > 2.71828182845904523536)
          lo = mid;
        else
          hi = mid;
      }
      const double cc = 0.5 * (lo + hi);
      const double wu = act ? (rp / cc) * exp(rp * rp / (2.0 * cc)) : 0.0;
      wn = wu / wave_sum(wu);
    } else {
      wn = 1.0 / static_cast<double>(N);
    }
    if (act) {
      R[idx] = Ri;
      W[idx] = wn;
    }
    wfinal = act ? wn : 0.0;
  }
  if (v != nullptr) {
    // next drafter: inverse CDF of the weights at v (ascending drafter index);
    // every lane runs the same loop over shuffled weights, lane 0 stores.
    const double wcur = wfinal;
    double tot = 0.0;
    for (int q = 0; q < N; ++q) tot += __shfl(wcur, q, 64);
    const double x = static_cast<double>(v[b]) * tot;
    double run = 0.0;
    int pick = -1, last_pos = -1;
    for (int q = 0; q < N; ++q) {
      const double wq = __shfl(wcur, q, 64);
      if (wq > 0.0) last_pos = q;
      run += wq;
      if (pick < 0 && run > x) pick = q;
    }
    if (i == 0) sel[b] = pick >= 0 ? pick : last_pos;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t q = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < n; q += stride) p[q] = 0u;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

struct Shape {
  int B, K, N, V, mode, fused;
  int R, RT, S, Q, nsub, U1, U3;
  int64_t n_static, n_dyn;
};

static Shape make_shape(int B, int K, int N, int V, int mode, int fused) {
  Shape s;
  s.B = B;
  s.K = K;
  s.N = N;
  s.V = V;
  s.mode = mode;
  s.fused = fused;
  s.RT = mode == MODE_VERIFY ? K + 1 : K + fused;
  s.R = s.RT + N * K;
  s.S = (V + kSliceTok - 1) / kSliceTok;
  s.Q = (s.S + kSlicesPerUnit - 1) / kSlicesPerUnit;
  s.nsub = (V + kSub - 1) / kSub;
  s.U1 = s.R * s.Q;
  s.U3 = mode == MODE_VERIFY ? 1 : 1 + fused;
  s.n_static = static_cast<int64_t>(B) * s.U1;
  const int64_t dyn_per_seq = mode == MODE_VERIFY ? s.S : static_cast<int64_t>(K) * s.S + (fused ? s.S : 0);
  s.n_dyn = static_cast<int64_t>(B) * dyn_per_seq;
  return s;
}

struct WsLayout {
  size_t work, p1cnt, p1all, p2cnt, p2gcnt, done, queue, zero_end, stat_k, stat_s, subsum, gpart, dec, total;
};

// Queue slots one call can publish at most: B * (K + 1) * (slices of the longest row)
// covers B * S draw units and B * K * S gamma units for any V.
static size_t queue_capacity(int B, int K) {
  return static_cast<size_t>(B) * (static_cast<size_t>(K) + 1) * kMaxSlices;
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Counters first (they must read zero at launch), scratch after them.
static WsLayout ws_layout(const Shape& s) {
  WsLayout L;
  const size_t B = static_cast<size_t>(s.B), K1 = static_cast<size_t>(s.K) + 1;
  const size_t cells = B * static_cast<size_t>(s.R) * static_cast<size_t>(s.Q);
  size_t o = 0;
  L.work = o;
  o = align256(o + 16);
  L.p1cnt = o;
  o = align256(o + 4 * B * K1);
  L.p1all = o;
  o = align256(o + 4 * B);
  L.p2cnt = o;
  o = align256(o + 4 * B);
  L.p2gcnt = o;
  o = align256(o + 4 * B);
  L.done = o;
  o = align256(o + 4 * B);
  L.queue = o;  // slots are zero between calls, like the counters
  o = align256(o + 8 * queue_capacity(s.B, s.K));
  // Everything before zero_end must read zero at launch; it depends on B and K only,
  // so a workspace can serve any V without being cleared again.
  L.zero_end = o;
  L.stat_k = o;
  o = align256(o + 4 * cells);
  L.stat_s = o;
  o = align256(o + 8 * cells);
  L.subsum = o;
  o = align256(o + 8 * B * static_cast<size_t>(s.nsub));
  L.gpart = o;
  o = align256(o + (s.mode == MODE_GAMMA ? 8 * B * s.K * s.N * s.S : 0));
  L.dec = o;
  o = align256(o + 8 * B * kDecWords);
  L.total = o;
  return L;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool stride_ok(int64_t s, int V) { return s >= V && (s % 8) == 0; }

static int bind_workspace(Params& p, const Shape& s, void* ws, size_t bytes) {
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return SPEC_ERR_WORKSPACE;
  const WsLayout L = ws_layout(s);
  if (bytes < L.total) return SPEC_ERR_WORKSPACE;
  if (static_cast<size_t>(s.n_dyn) > queue_capacity(s.B, s.K)) return SPEC_ERR_SHAPE;
  p.queue_cap = static_cast<int>(queue_capacity(s.B, s.K));
  char* base = static_cast<char*>(ws);
  p.work = reinterpret_cast<uint32_t*>(base + L.work);
  p.p1cnt = reinterpret_cast<uint32_t*>(base + L.p1cnt);
  p.p1all = reinterpret_cast<uint32_t*>(base + L.p1all);
  p.p2cnt = reinterpret_cast<uint32_t*>(base + L.p2cnt);
  p.p2gcnt = reinterpret_cast<uint32_t*>(base + L.p2gcnt);
  p.done = reinterpret_cast<uint32_t*>(base + L.done);
  p.queue = reinterpret_cast<unsigned long long*>(base + L.queue);
  p.stat_k = reinterpret_cast<float*>(base + L.stat_k);
  p.stat_s = reinterpret_cast<double*>(base + L.stat_s);
  p.subsum = reinterpret_cast<double*>(base + L.subsum);
  p.gpart = reinterpret_cast<double*>(base + L.gpart);
  p.dec = reinterpret_cast<double*>(base + L.dec);
  return SPEC_OK;
}

// Resident workgroups the device holds (memoised per device: a device property, not call state).
static int resident_workgroups() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int ncu = 0, per = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, flow_kernel, kThreads, 0) != hipSuccess) return 0;
  const int g = ncu * (per > 0 ? per : 1);
  if (dev >= 0 && dev < 64) cache[dev] = g;
  return g;
}

// Statistics units first (in claim order), then one queue slot per published unit.
static void plan_units(Params& p, const Shape& s) {
  p.R = s.R;
  p.RT = s.RT;
  p.S = s.S;
  p.Q = s.Q;
  p.nsub = s.nsub;
  p.U1 = s.U1;
  p.U3 = s.U3;
  p.n_static = static_cast<int>(s.n_static);
  p.total_units = static_cast<int>(s.n_static + s.n_dyn);
}

static int launch_flow(Params& p, const Shape& s, hipStream_t stream) {
  const int64_t total = s.n_static + s.n_dyn;
  if (total > 0x3fffffffLL) return SPEC_ERR_SHAPE;
  int grid = resident_workgroups();
  if (grid <= 0) return SPEC_ERR_HIP;
  if (grid > total) grid = static_cast<int>(total);
  plan_units(p, s);
  hipLaunchKernelGGL(flow_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

static int check_common(int B, int K, int V, float T) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return SPEC_ERR_SHAPE;
  if (B > SPEC_MAX_B) return SPEC_ERR_SHAPE;
  if (!(T > 0.0f) || !isfinite(T)) return SPEC_ERR_PARAM;
  return SPEC_OK;
}

static float log2e_over(float T) { return static_cast<float>(1.4426950408889634074 / static_cast<double>(T)); }

static int verify_common(const spec_bf16* target, int64_t ts, const spec_bf16* draft, int64_t ds,
                         const int32_t* tokens, const float* r, const float* u, int B, int K, int V, double delta,
                         float T, int32_t* A, int32_t* tok, uint8_t* mask, float* gstar, void* ws, size_t wsb,
                         hipStream_t stream) {
  int st = check_common(B, K, V, T);
  if (st != SPEC_OK) return st;
  if (!target || !draft || !tokens || !r || !u || !A || !tok) return SPEC_ERR_NULL;
  if (!stride_ok(ts, V) || !stride_ok(ds, V)) return SPEC_ERR_SHAPE;
  if (!aligned16(target) || !aligned16(draft)) return SPEC_ERR_ALIGN;
  const Shape s = make_shape(B, K, 1, V, MODE_VERIFY, 0);
  Params p{};
  st = bind_workspace(p, s, ws, wsb);
  if (st != SPEC_OK) return st;
  p.target = target;
  p.t_stride = ts;
  p.t_rows = K + 1;
  p.draft = draft;
  p.d_stride = ds;
  p.drafter_stride = 0;
  p.tokens = tokens;
  p.r = r;
  p.u = u;
  p.B = B;
  p.K = K;
  p.N = 1;
  p.V = V;
  p.c = log2e_over(T);
  p.delta = delta;
  p.mode = MODE_VERIFY;
  p.accepted_len = A;
  p.out_token = tok;
  p.accept_mask = mask;
  p.gamma_star = gstar;
  return launch_flow(p, s, stream);
}

}  // namespace specv

using namespace specv;

extern "C" {

const char* spec_status_str(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_NULL: return "required pointer is NULL";
    case SPEC_ERR_SHAPE: return "size or stride out of range";
    case SPEC_ERR_PARAM: return "temperature / delta / loss_scale not finite or out of range";
    case SPEC_ERR_ALIGN: return "logits base pointer not 16-byte aligned";
    case SPEC_ERR_WORKSPACE: return "workspace NULL, misaligned or too small";
    case SPEC_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t spec_workspace_counter_bytes(int B, int K) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || B > SPEC_MAX_B) return 0;
  return ws_layout(make_shape(B, K, 1, 1, MODE_VERIFY, 0)).zero_end;
}

size_t spec_workspace_bytes(int B, int K, int N) {
  if (B < 1 || K < 1 || N < 1 || K > SPEC_MAX_K || N > SPEC_MAX_N || B > SPEC_MAX_B) return 0;
  // the layout grows with V: size it for the largest vocabulary a call may use
  const size_t v = ws_layout(make_shape(B, K, 1, SPEC_MAX_V, MODE_VERIFY, 0)).total;
  const size_t g = ws_layout(make_shape(B, K, N, SPEC_MAX_V, MODE_GAMMA, 1)).total;
  return v > g ? v : g;
}

int spec_workspace_init(void* workspace, size_t bytes, spec_stream_t stream) {
  if (workspace == nullptr) return SPEC_ERR_WORKSPACE;
  const size_t words = bytes / 4;
  if (words == 0) return SPEC_OK;
  const int grid = static_cast<int>(words / 256 + 1 < 1024 ? words / 256 + 1 : 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(workspace), words);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_verify(const spec_bf16* target, int64_t target_row_stride, const spec_bf16* draft, int64_t draft_row_stride,
                const int32_t* draft_tokens, const float* r_accept, const float* u_resample, int B, int K, int V,
                float temperature, int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask, void* workspace,
                size_t workspace_bytes, spec_stream_t stream) {
  return verify_common(target, target_row_stride, draft, draft_row_stride, draft_tokens, r_accept, u_resample, B, K,
                       V, 0.0, temperature, accepted_len, out_token, accept_mask, nullptr, workspace,
                       workspace_bytes, stream);
}

int spec_cactus_verify(const spec_bf16* verifier, int64_t verifier_row_stride, const spec_bf16* draft,
                       int64_t draft_row_stride, const int32_t* draft_tokens, const float* r_accept,
                       const float* u_resample, int B, int m, int V, float delta, float temperature,
                       int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask, float* gamma_star,
                       void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  if (!(delta >= 0.0f) || !isfinite(delta)) return SPEC_ERR_PARAM;
  return verify_common(verifier, verifier_row_stride, draft, draft_row_stride, draft_tokens, r_accept, u_resample, B,
                       m, V, static_cast<double>(delta), temperature, accepted_len, out_token, accept_mask,
                       gamma_star, workspace, workspace_bytes, stream);
}

int spec_counterfactual_gamma(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                              const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                              const int32_t* traj_tokens, int B, int K, int N, int V, float temperature, float* gamma,
                              float* est_len, float* loss, const int32_t* sel, const int32_t* draft_tokens,
                              const float* r_accept, const float* u_resample, int32_t* accepted_len,
                              int32_t* out_token, uint8_t* accept_mask, void* workspace, size_t workspace_bytes,
                              spec_stream_t stream) {
  int st = check_common(B, K, V, temperature);
  if (st != SPEC_OK) return st;
  if (N < 1 || N > SPEC_MAX_N) return SPEC_ERR_SHAPE;
  if (!target || !drafts || !traj_tokens || !gamma || !est_len || !loss) return SPEC_ERR_NULL;
  const bool fused = sel != nullptr;
  if (fused && (!draft_tokens || !r_accept || !u_resample || !accepted_len || !out_token)) return SPEC_ERR_NULL;
  if (target_rows_per_seq < K + (fused ? 1 : 0)) return SPEC_ERR_SHAPE;
  if (!stride_ok(target_row_stride, V) || !stride_ok(draft_row_stride, V)) return SPEC_ERR_SHAPE;
  if (drafter_stride < 0 || (drafter_stride % 8) != 0 || (N > 1 && drafter_stride == 0)) return SPEC_ERR_SHAPE;
  if (!aligned16(target) || !aligned16(drafts)) return SPEC_ERR_ALIGN;
  const Shape s = make_shape(B, K, N, V, MODE_GAMMA, fused ? 1 : 0);
  Params p{};
  st = bind_workspace(p, s, workspace, workspace_bytes);
  if (st != SPEC_OK) return st;
  p.target = target;
  p.t_stride = target_row_stride;
  p.t_rows = target_rows_per_seq;
  p.draft = drafts;
  p.d_stride = draft_row_stride;
  p.drafter_stride = drafter_stride;
  p.tokens = draft_tokens;
  p.r = r_accept;
  p.u = u_resample;
  p.traj = traj_tokens;
  p.sel = sel;
  p.B = B;
  p.K = K;
  p.N = N;
  p.V = V;
  p.c = log2e_over(temperature);
  p.delta = 0.0;
  p.mode = MODE_GAMMA;
  p.fused = fused ? 1 : 0;
  p.accepted_len = accepted_len;
  p.out_token = out_token;
  p.accept_mask = accept_mask;
  p.gamma = gamma;
  p.est_len = est_len;
  p.loss = loss;
  return launch_flow(p, s, stream);
}

int hedge_update(double* cum_regret, double* weights, const float* loss, const uint8_t* has_loss, float loss_scale,
                 const float* v_select, int32_t* sel_out, int B, int N, spec_stream_t stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_N) return SPEC_ERR_SHAPE;
  if (!cum_regret || !weights || !loss) return SPEC_ERR_NULL;
  if (v_select && !sel_out) return SPEC_ERR_NULL;
  if (!(loss_scale >= 0.0f) || !isfinite(loss_scale)) return SPEC_ERR_PARAM;
  hipLaunchKernelGGL(hedge_kernel, dim3(B), dim3(64), 0, stream, cum_regret, weights, loss, has_loss, loss_scale,
                     v_select, sel_out, N);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // extern "C"
