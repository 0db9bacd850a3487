// libspecverify: batched speculative-sampling verification on gfx950.
//
// One kernel, `row_kernel`, serves the three verification entry points.  A
// workgroup owns one "job": a (sequence b, position k) row pair -- target row
// k and one draft row -- or the bonus row (target row K of a sequence).
//
//   pass 1  streams the row pair once from HBM and reduces each row to its
//           base-2 softmax statistics (k, s) (see spec_device.hpp);
//   scalar  one lane forms the fp64 accept ratio at the drafted token
//           ([LT] §5.1 / [CA] Key design 3), the realised-token ratio of the
//           HedgeSpec estimator, and publishes the position's decision;
//   pass 2  only where its result can be used: the residual (pt - pd)+ (or
//           Cactus's (h - pd)+) of a rejected position with no earlier
//           rejection already known, the bonus row's pt, and the HedgeSpec
//           acceptance mass sum_x min(pt, pd).  It re-reads the pair (from
//           cache when it is still resident) and leaves per-sub-tile masses of
//           the sampling weights in LDS;
//   pass 3  one wave re-reads the single 512-token sub-tile that holds the
//           inverse-CDF crossing and finds the token;
//   tickets the last workgroup of a sequence (or of a (sequence, drafter)
//           pair) folds the per-position results into the accepted length and
//           output token (or the acceptance-length estimator and loss) and
//           resets its counters, so the workspace is zero again on exit.
//
// [LT] "Speculative Decoding 为什么是 Lossless 的 -- 详细证明教程";
// [NB] HedgeSpec note "Not-a-Bandit ..."; [CA] Cactus note;
// [NH] Chaudhuri, Freund, Hsu 2009 (NormalHedge).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_device.hpp"
#include "spec_verify.h"

namespace specv {

enum : uint32_t { ST_UNKNOWN = 0, ST_ACCEPT = 1, ST_REJECT = 2, ST_INVALID = 3 };
enum : int { MODE_VERIFY = 0, MODE_GAMMA = 1 };
// Sampling-weight modes of pass 2 / pass 3.
enum : int { W_RESID = 0, W_TARGET_H = 1, W_TARGET = 2 };

struct Params {
  const uint16_t* target;
  int64_t t_stride;
  int t_rows;  // target rows per sequence
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
  int32_t* accepted_len;
  int32_t* out_token;
  uint8_t* accept_mask;
  float* gamma_star;
  float* gamma;
  float* est_len;
  float* loss;
  uint32_t* seq_ticket;
  uint32_t* seq_state;
  int32_t* seq_cand;
  uint32_t* est_ticket;
  double* est_g;
  double* est_a;
};

struct Job {
  int b, k, i;
  bool pair;    // has a draft row
  bool verify;  // accept test (k < K) or bonus draw (k == K)
  bool bonus;
  bool gamma;   // HedgeSpec evaluation role
};

__device__ __forceinline__ Job decode_job(const Params& p, int j) {
  Job J;
  if (p.mode == MODE_VERIFY) {
    J.b = j / (p.K + 1);
    J.k = j % (p.K + 1);
    J.i = 0;
    J.bonus = (J.k == p.K);
    J.pair = !J.bonus;
    J.verify = true;
    J.gamma = false;
  } else {
    const int nk = p.K * p.N;
    if (j < p.B * nk) {
      J.b = j / nk;
      const int rem = j % nk;
      J.k = rem / p.N;
      J.i = rem % p.N;
      J.pair = true;
      J.gamma = true;
      J.bonus = false;
      J.verify = p.fused && p.sel[J.b] == J.i;
    } else {
      J.b = j - p.B * nk;
      J.k = p.K;
      J.i = -1;
      J.pair = false;
      J.gamma = false;
      J.bonus = true;
      J.verify = true;
    }
  }
  return J;
}

// Everything a lane needs to turn logits into sampling weights (fp64).
struct WeightCtx {
  float c;
  float kt, kd;          // row references
  double inv_st, inv_sd; // 1 / row sums
  double s_scale;        // Cactus rescale s of the non-candidate tokens (1.0 for SpS)
  double gstar;          // Cactus gamma* (the candidate's target mass)
  int n;                 // candidate token
  int special;           // 1: token n carries gamma* (delta > 0)
  int mode;              // W_RESID, W_TARGET_H, W_TARGET
};

// Sampling weights of eight consecutive tokens starting at `tok0`:
//   W_RESID    (h - pd)+ with h = s * pt, h_n = gamma*   ([LT] §2.2 / [CA] Key design 2)
//   W_TARGET_H h          (a rejection with zero residual mass)
//   W_TARGET   pt         (bonus token)
// Optionally adds sum min(pt, pd) of the eight tokens to *gmin ([LT] §6.3).
template <bool GMIN>
__device__ __forceinline__ void weights8(const WeightCtx& w, const float zt[8], const float zd[8], int tok0,
                                         double out[8], double* gmin) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double pt = static_cast<double>(fast_exp2(fmaf(zt[e], w.c, -w.kt))) * w.inv_st;
    if (w.mode == W_TARGET) {
      out[e] = pt;
      continue;
    }
    double h = w.s_scale * pt;
    if (w.special && tok0 + e == w.n) h = w.gstar;
    if (w.mode == W_TARGET_H && !GMIN) {
      out[e] = h;
      continue;
    }
    const double pd = static_cast<double>(fast_exp2(fmaf(zd[e], w.c, -w.kd))) * w.inv_sd;
    out[e] = fmax(h - pd, 0.0);
    if (GMIN) *gmin += fmin(pt, pd);
  }
}

__device__ __forceinline__ const uint4* as_chunks(const uint16_t* row) { return reinterpret_cast<const uint4*>(row); }

// Pass 1: softmax statistics of the target row (and the draft row when PAIR).
template <bool PAIR>
__device__ __forceinline__ void stats_pass(const uint16_t* trow, const uint16_t* drow, int V, float c, RowAcc& at,
                                           RowAcc& ad) {
  const uint4* tr = as_chunks(trow);
  const uint4* dr = as_chunks(drow);
  const int nchunks = (V + kVec - 1) / kVec;
  const int tid = threadIdx.x;
  for (int base = 0; base < nchunks; base += kThreads * kUnroll) {
    uint4 vt[kUnroll], vd[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ci = base + u * kThreads + tid;
      if (ci < nchunks) {
        vt[u] = tr[ci];
        if (PAIR) vd[u] = dr[ci];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ci = base + u * kThreads + tid;
      if (ci < nchunks) {
        const int valid = V - ci * kVec;
        float z[8];
        unpack8(vt[u], z, valid);
        row_acc_add8(at, z, c);
        if (PAIR) {
          unpack8(vd[u], z, valid);
          row_acc_add8(ad, z, c);
        }
      }
    }
  }
}

// Pass 2 for the HedgeSpec mass alone: sum_x 2^min(log2 pt(x), log2 pd(x)), one exp per token.
__device__ __forceinline__ double gamma_pass(const uint16_t* trow, const uint16_t* drow, int V, float c, float lt,
                                             float ld) {
  const uint4* tr = as_chunks(trow);
  const uint4* dr = as_chunks(drow);
  const int nchunks = (V + kVec - 1) / kVec;
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int base = 0; base < nchunks; base += kThreads * kUnroll) {
    uint4 vt[kUnroll], vd[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ci = base + u * kThreads + tid;
      if (ci < nchunks) {
        vt[u] = tr[ci];
        vd[u] = dr[ci];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ci = base + u * kThreads + tid;
      if (ci < nchunks) {
        const int valid = V - ci * kVec;
        float zt[8], zd[8], e[8];
        unpack8(vt[u], zt, valid);
        unpack8(vd[u], zd, valid);
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fminf(fmaf(zt[i], c, -lt), fmaf(zd[i], c, -ld)));
        acc += static_cast<double>(((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
      }
    }
  }
  return acc;
}

// Pass 2 with sampling weights: per-sub-tile masses into subsum[], optional sum min(pt, pd).
template <bool PAIR, bool GMIN>
__device__ __forceinline__ void weight_pass(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w,
                                            double* subsum, double* gmin) {
  const uint4* tr = as_chunks(trow);
  const uint4* dr = as_chunks(drow);
  const int nchunks = (V + kVec - 1) / kVec;
  const int ntiles = (nchunks + kThreads - 1) / kThreads;
  const int nsub = (V + kSub - 1) / kSub;
  const int tid = threadIdx.x;
  for (int j0 = 0; j0 < ntiles; j0 += kUnroll) {
    uint4 vt[kUnroll], vd[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ci = (j0 + u) * kThreads + tid;
      if (ci < nchunks) {
        vt[u] = tr[ci];
        if (PAIR) vd[u] = dr[ci];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int jt = j0 + u;
      if (jt >= ntiles) break;  // uniform over the workgroup
      const int ci = jt * kThreads + tid;
      double lsum = 0.0;
      if (ci < nchunks) {
        const int valid = V - ci * kVec;
        float zt[8], zd[8];
        unpack8(vt[u], zt, valid);
        if (PAIR) unpack8(vd[u], zd, valid);
        double wv[8];
        weights8<GMIN>(w, zt, zd, ci * kVec, wv, gmin);
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum += wv[e];
      }
      const double incl = wave_incl_scan(lsum);
      const int s = jt * kWaves + wave_id();
      if (lane_id() == 63 && s < nsub) subsum[s] = incl;
    }
  }
}

// Wave 0: the sub-tile holding the crossing of x = u * Z, Z = sum of subsum[].
// Returns false when Z is not positive.  x_rel is x minus the mass before the
// sub-tile, or +inf when rounding left no crossing (the last positive-mass
// token is then taken).
__device__ bool find_subtile(const double* subsum, int nsub, double u, int& s_star, double& x_rel) {
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
  unsigned long long m = __ballot(incl > x);
  bool clamp = (m == 0ull);
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

// Wave 0, pass 3: the token in sub-tile s_star where the running mass passes
// x_rel (or the sub-tile's last positive-mass token when x_rel is +inf).
template <bool PAIR>
__device__ int find_token(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w, int s_star,
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
    if (PAIR) unpack8(as_chunks(drow)[ci], zd, valid);
    weights8<false>(w, zt, zd, ci * kVec, wv, nullptr);
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

// Inverse-CDF draw over one row (pair) with weights mode w.mode and uniform u.
template <bool PAIR>
__device__ int draw_token(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w, double u,
                          double* subsum, bool* ok) {
  double dummy = 0.0;
  weight_pass<PAIR, false>(trow, drow, V, w, subsum, &dummy);
  __syncthreads();
  __shared__ int sh_tok;
  __shared__ int sh_ok;
  if (wave_id() == 0) {
    int s_star = -1;
    double x_rel = 0.0;
    const bool found = find_subtile(subsum, (V + kSub - 1) / kSub, u, s_star, x_rel);
    int tok = -1;
    if (found) tok = find_token<PAIR>(trow, drow, V, w, s_star, x_rel);
    if (lane_id() == 0) {
      sh_tok = tok;
      sh_ok = found ? 1 : 0;
    }
  }
  __syncthreads();
  *ok = sh_ok != 0;
  const int t = sh_tok;
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kThreads) void row_kernel(Params p) {
  __shared__ double subsum[kMaxSub];
  __shared__ double scratch[2 * kWaves];
  __shared__ WeightCtx sh_w;
  __shared__ int sh_flags;  // bit0 residual draw, bit1 bonus draw, bit2 gamma pass
  __shared__ float sh_lt, sh_ld;
  __shared__ double sh_a;

  const int j = logical_job(blockIdx.x, gridDim.x);
  const Job J = decode_job(p, j);
  const int V = p.V, K = p.K;
  const float c = p.c;

  if (p.mode == MODE_GAMMA && J.bonus) {
    const int s = p.sel[J.b];
    if (s < 0 || s >= p.N) {  // invalid selection: the whole sequence reports -1
      if (threadIdx.x == 0) {
        p.accepted_len[J.b] = -1;
        p.out_token[J.b] = -1;
      }
      return;
    }
  }

  const uint16_t* trow = p.target + (static_cast<int64_t>(J.b) * p.t_rows + J.k) * p.t_stride;
  const uint16_t* drow = nullptr;
  if (J.pair) {
    const int di = (p.mode == MODE_GAMMA) ? J.i : 0;
    drow = p.draft + static_cast<int64_t>(di) * p.drafter_stride + (static_cast<int64_t>(J.b) * K + J.k) * p.d_stride;
  }

  // ---- pass 1 -------------------------------------------------------------
  RowAcc at = row_acc_init(), ad = row_acc_init();
  if (J.pair)
    stats_pass<true>(trow, drow, V, c, at, ad);
  else
    stats_pass<false>(trow, drow, V, c, at, ad);
  const RowStats st = block_row_stats(at, scratch);
  RowStats sd{0.0f, 1.0};
  if (J.pair) sd = block_row_stats(ad, scratch);

  // ---- scalar decisions (one lane) ----------------------------------------
  if (threadIdx.x == 0) {
    WeightCtx w;
    w.c = c;
    w.kt = st.k;
    w.kd = sd.k;
    w.inv_st = 1.0 / st.s;
    w.inv_sd = 1.0 / sd.s;
    w.s_scale = 1.0;
    w.gstar = 0.0;
    w.n = -1;
    w.special = 0;
    w.mode = W_TARGET;
    int flags = 0;
    const int sbase = J.b * (K + 1);
    if (J.verify && !J.bonus) {
      const int n = p.tokens[J.b * K + J.k];
      uint32_t state;
      bool acc = false;
      if (n < 0 || n >= V) {
        state = ST_INVALID;
      } else {
        // [CA] Key design 3 with the verifier's probability c of the candidate; delta = 0 is SpS.
        const double ct = fmin(token_prob(bf16_at(trow, n), c, st), 1.0);
        const double cd = token_prob(bf16_at(drow, n), c, sd);
        const double gs = fmin(ct + sqrt(2.0 * p.delta * ct * (1.0 - ct)), 1.0);
        const double ratio = cd > 0.0 ? gs / cd : (gs > 0.0 ? __builtin_inf() : 0.0);
        acc = static_cast<double>(p.r[J.b * K + J.k]) < ratio;  // [LT] §5.1: strict
        state = acc ? ST_ACCEPT : ST_REJECT;
        w.s_scale = ct < 1.0 ? (1.0 - gs) / (1.0 - ct) : 0.0;
        w.gstar = gs;
        w.n = n;
        w.special = p.delta > 0.0 ? 1 : 0;
        w.mode = W_RESID;
        if (p.gamma_star) p.gamma_star[J.b * K + J.k] = static_cast<float>(gs);
      }
      if (p.accept_mask) p.accept_mask[J.b * K + J.k] = acc ? 1 : 0;
      st_agent(&p.seq_state[sbase + J.k], state);
      if (state == ST_REJECT) {
        // The residual is needed only at the first rejection; skip if an earlier one is already known.
        bool earlier = false;
        for (int q = 0; q < J.k; ++q) earlier |= (ld_agent(&p.seq_state[sbase + q]) == ST_REJECT);
        if (!earlier) flags |= 1;
      }
    } else if (J.bonus) {
      bool known = false;
      for (int q = 0; q < K; ++q) {
        const uint32_t s = ld_agent(&p.seq_state[sbase + q]);
        known |= (s == ST_REJECT || s == ST_INVALID);
      }
      if (!known) flags |= 2;
      w.mode = W_TARGET;
    }
    if (J.gamma) {
      flags |= 4;
      // realised-token ratio a_k = min(1, pd(x_k) / pt(x_k)) of the estimator ([NB] Key design 2)
      double a = 1.0;
      if (J.k < K - 1) {
        const int x = p.traj[J.b * K + J.k];
        if (x < 0 || x >= V) {
          a = __builtin_nan("");
        } else {
          const double ptx = token_prob(bf16_at(trow, x), c, st);
          const double pdx = token_prob(bf16_at(drow, x), c, sd);
          a = ptx > 0.0 ? fmin(1.0, pdx / ptx) : (pdx > 0.0 ? 1.0 : 0.0);
        }
      }
      sh_a = a;
      sh_lt = static_cast<float>(static_cast<double>(st.k) + log2(st.s));
      sh_ld = static_cast<float>(static_cast<double>(sd.k) + log2(sd.s));
    }
    sh_w = w;
    sh_flags = flags;
  }
  __syncthreads();
  const int flags = sh_flags;
  const WeightCtx w = sh_w;

  // ---- pass 2 / 3 ---------------------------------------------------------
  int token = -1;
  double gamma = 0.0;
  if (flags & 1) {
    // residual draw at a rejected position (and, when evaluating, the mass in the same pass)
    double gl = 0.0;
    if (flags & 4)
      weight_pass<true, true>(trow, drow, V, w, subsum, &gl);
    else
      weight_pass<true, false>(trow, drow, V, w, subsum, &gl);
    if (flags & 4) {
      const double g = wave_sum(gl);
      if (lane_id() == 0) scratch[wave_id()] = g;
    }
    __syncthreads();
    if (flags & 4) {
      for (int q = 0; q < kWaves; ++q) gamma += scratch[q];
    }
    __shared__ int sh_tok;
    __shared__ int sh_found;
    if (wave_id() == 0) {
      int s_star = -1;
      double x_rel = 0.0;
      const double uu = static_cast<double>(p.u[J.b * (K + 1) + J.k]);
      const bool found = find_subtile(subsum, (V + kSub - 1) / kSub, uu, s_star, x_rel);
      int tok = -1;
      if (found) tok = find_token<true>(trow, drow, V, w, s_star, x_rel);
      if (lane_id() == 0) {
        sh_tok = tok;
        sh_found = found ? 1 : 0;
      }
    }
    __syncthreads();
    token = sh_tok;
    const bool found = sh_found != 0;
    __syncthreads();
    if (!found) {
      // zero residual mass on a rejection: draw from the position's target h instead
      WeightCtx wh = w;
      wh.mode = W_TARGET_H;
      bool ok = false;
      token = draw_token<false>(trow, drow, V, wh, static_cast<double>(p.u[J.b * (K + 1) + J.k]), subsum, &ok);
      if (!ok) token = -1;
    }
  } else {
    if (flags & 4) {
      const double gl = gamma_pass(trow, drow, V, c, sh_lt, sh_ld);
      const double g = wave_sum(gl);
      if (lane_id() == 0) scratch[wave_id()] = g;
      __syncthreads();
      for (int q = 0; q < kWaves; ++q) gamma += scratch[q];
      __syncthreads();
    }
    if (flags & 2) {
      bool ok = false;
      token = draw_token<false>(trow, drow, V, w, static_cast<double>(p.u[J.b * (K + 1) + K]), subsum, &ok);
      if (!ok) token = -1;
    }
  }

  // ---- publish + completion tickets ---------------------------------------
  if (threadIdx.x != 0) return;
  if (J.gamma) {
    const int idx = (J.b * K + J.k) * p.N + J.i;
    p.gamma[idx] = static_cast<float>(gamma);
    st_agent_d(&p.est_g[idx], gamma);
    st_agent_d(&p.est_a[idx], sh_a);
    __threadfence();
    const uint32_t old = ticket(&p.est_ticket[J.b * p.N + J.i]);
    if (old == static_cast<uint32_t>(K - 1)) {
      __threadfence();
      // [NB] Key design 2 (reading: L = 1 + sum_k gamma_k prod_{j<k} a_j) and Key design 3 (f = K + 1 - L)
      double L = 1.0, prod = 1.0;
      for (int q = 0; q < K; ++q) {
        const int qi = (J.b * K + q) * p.N + J.i;
        L += ld_agent_d(&p.est_g[qi]) * prod;
        prod *= ld_agent_d(&p.est_a[qi]);
      }
      p.est_len[J.b * p.N + J.i] = static_cast<float>(L);
      p.loss[J.b * p.N + J.i] = static_cast<float>(static_cast<double>(K + 1) - L);
      for (int q = 0; q < K; ++q) {
        const int qi = (J.b * K + q) * p.N + J.i;
        st_agent_d(&p.est_g[qi], 0.0);
        st_agent_d(&p.est_a[qi], 0.0);
      }
      st_agent(&p.est_ticket[J.b * p.N + J.i], 0u);
    }
  }
  if (J.verify) {
    const int sbase = J.b * (K + 1);
    st_agent_i(&p.seq_cand[sbase + J.k], token);
    __threadfence();
    const uint32_t old = ticket(&p.seq_ticket[J.b]);
    if (old == static_cast<uint32_t>(K)) {
      __threadfence();
      // [LT] §9.1: keep drafts up to the first rejection A, then the resample at A or the bonus.
      int A = K;
      bool bad = false;
      for (int q = 0; q < K; ++q) {
        const uint32_t s = ld_agent(&p.seq_state[sbase + q]);
        bad |= (s == ST_INVALID);
        if (s == ST_REJECT && A == K) A = q;
      }
      int tok = ld_agent_i(&p.seq_cand[sbase + A]);
      if (bad || tok < 0) {
        A = -1;
        tok = -1;
      }
      p.accepted_len[J.b] = A;
      p.out_token[J.b] = tok;
      for (int q = 0; q <= K; ++q) {
        st_agent(&p.seq_state[sbase + q], 0u);
        st_agent_i(&p.seq_cand[sbase + q], 0);
      }
      st_agent(&p.seq_ticket[J.b], 0u);
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
    double Ri = act ? R[idx] + (lhat - l) : 0.0;
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
struct WsLayout {
  size_t seq_ticket, seq_state, seq_cand, est_ticket, est_g, est_a, total;
};

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static WsLayout ws_layout(int B, int K, int N) {
  WsLayout L;
  size_t o = 0;
  const size_t b = static_cast<size_t>(B), k1 = static_cast<size_t>(K) + 1, n = static_cast<size_t>(N);
  L.seq_ticket = o;
  o = align256(o + 4 * b);
  L.seq_state = o;
  o = align256(o + 4 * b * k1);
  L.seq_cand = o;
  o = align256(o + 4 * b * k1);
  L.est_ticket = o;
  o = align256(o + 4 * b * n);
  L.est_g = o;
  o = align256(o + 8 * b * static_cast<size_t>(K) * n);
  L.est_a = o;
  o = align256(o + 8 * b * static_cast<size_t>(K) * n);
  L.total = o;
  return L;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool stride_ok(int64_t s, int V) { return s >= V && (s % 8) == 0; }

static int bind_workspace(Params& p, void* ws, size_t bytes, int B, int K, int N) {
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return SPEC_ERR_WORKSPACE;
  const WsLayout L = ws_layout(B, K, N);
  if (bytes < L.total) return SPEC_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  p.seq_ticket = reinterpret_cast<uint32_t*>(base + L.seq_ticket);
  p.seq_state = reinterpret_cast<uint32_t*>(base + L.seq_state);
  p.seq_cand = reinterpret_cast<int32_t*>(base + L.seq_cand);
  p.est_ticket = reinterpret_cast<uint32_t*>(base + L.est_ticket);
  p.est_g = reinterpret_cast<double*>(base + L.est_g);
  p.est_a = reinterpret_cast<double*>(base + L.est_a);
  return SPEC_OK;
}

static int launch_rows(const Params& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(row_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

static int check_common(int B, int K, int V, float T) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return SPEC_ERR_SHAPE;
  if (static_cast<int64_t>(B) * (K + 1) * SPEC_MAX_N > 0x7fffffffLL) return SPEC_ERR_SHAPE;
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
  Params p{};
  st = bind_workspace(p, ws, wsb, B, K, 1);
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
  return launch_rows(p, B * (K + 1), stream);
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

size_t spec_workspace_bytes(int B, int K, int N) {
  if (B < 1 || K < 1 || N < 1) return 0;
  return ws_layout(B, K, N).total;
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
  const int64_t jobs = static_cast<int64_t>(B) * K * N + (fused ? B : 0);
  if (jobs > 0x7fffffffLL) return SPEC_ERR_SHAPE;
  Params p{};
  st = bind_workspace(p, workspace, workspace_bytes, B, K, N);
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
  return launch_rows(p, static_cast<int>(jobs), stream);
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
