// libspecverify: batched speculative-sampling verification on gfx950.
//
// Three persistent kernels: `verify_kernel` serves spec_verify, spec_cactus_verify
// and (an instance of its own) spec_cactus_kl_verify, `gamma_kernel` serves
// spec_counterfactual_gamma, and `tree_kernel` serves spec_tree_gamma (its
// phases are described where it is defined).  A grid is the number of
// workgroups the device holds at once (G), and every workgroup g runs its
// phases on a fixed schedule; nothing is claimed from a shared counter.  Small
// one-wave kernels serve the learners: hedge_update, hedge_exp_update and
// hedge_queue_update (the delayed-feedback queue resident on the device), and
// spec_acceptance_loss.
//
//   gamma groups -- (gamma calls) slots of S workgroups stream a position's
//       target row and its N drafter rows once (gamma_groups).
//   phase 0 -- (verify and draft-tree calls) statistics slices of the call's
//       slice list, dealt to the workgroups on a fixed schedule weighted by how
//       fast the hardware serves each dispatch slot of them (static_phase).  A
//       slice is 16384 tokens of one row, streamed once from HBM with 128-bit
//       loads while the next slice's loads are in flight.  Each wave reduces its
//       share to an exact base-2 softmax pair (reference k, sum s) and publishes
//       it as one 64-bit word.  The list is sequence-major, so sequences finish
//       their statistics one after another.  It holds the rows the decisions
//       need (target and draft rows of positions 0..K-1): the bonus row K is
//       read only by the draw units of a sequence that accepts every draft.
//   phase 1 -- units g, g + G, ... of the draw list, one per slice of a
//       sequence's rows.  A draw unit merges the sequence's statistics, takes
//       every accept decision ([LT] §5.1, [CA] Key design 3), finds the first
//       rejection A and computes per-512-token sub-tile masses of the sampling
//       weights of its slice of the row pair A ((pt - pd)+, Cactus's (h - pd)+)
//       or of the bonus row pt (at references of its own, since that row has no
//       statistics).  It publishes its slice's total, reads the other slices'
//       totals, and the unit whose slice holds the inverse-CDF crossing ([LT]
//       §9.1) finds the token in the rows it still holds in registers.
//   phase 2 -- (gamma calls) units g, g + G, ... of the HedgeSpec estimator and
//       loss ([NB] Key designs 1-3).
//
// A draw unit reads phase-0 words and the totals of its own sequence's draw
// units, and a phase-2 unit reads words of earlier phases; every workgroup
// finishes a phase before it starts the next, and the draw units of a sequence
// are at most one round of the grid apart, so every wait ends (a wait is also
// bounded by the wall clock; a timeout sets the workspace's fault word).
//
// Cross-workgroup data is published with device-scope 64-bit stores of words
// that are never zero, into a workspace that is zero before the call; a reader
// polls a word with device-scope loads until it is non-zero.  No counter, queue
// or fence sits on the streaming path.  Every word is cleared once all its
// readers are done with it (by its only reader, or by the step that knows the
// others are done), so the workspace is zero again when the kernel ends.
//
// [LT] "Speculative Decoding 为什么是 Lossless 的 -- 详细证明教程";
// [NB] HedgeSpec note "Not-a-Bandit: Provably No-Regret Drafter Selection ...";
// [CA] Cactus note; [NH] Chaudhuri, Freund, Hsu 2009 (NormalHedge).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "spec_device.hpp"
#include "spec_verify.h"

namespace specv {

enum : uint32_t { ST_ACCEPT = 1, ST_REJECT = 2, ST_INVALID = 3 };
enum : int { MODE_VERIFY = 0, MODE_GAMMA = 1, MODE_TREE = 2 };
// Sampling-weight modes of the draw passes.
enum : int { W_RESID = 0, W_TARGET_H = 1, W_TARGET = 2 };

constexpr int kTilesPerSlice = 8;
constexpr int kSliceTok = kTile * kTilesPerSlice;   // 16384 tokens per slice
constexpr int kSliceChunks = kSliceTok / kVec;      // 16-byte chunks per slice
constexpr int kMaxSlices = (kMaxV + kSliceTok - 1) / kSliceTok;  // slices of the longest row
constexpr unsigned long long kWaitTicks = 200000000ull;  // bounded wait: 2 s of the 100 MHz clock
constexpr unsigned long long kValid = 1ull << 63;        // published bit of an fp64 word
constexpr int kStage = 8 * kThreads;  // statistics words staged in LDS at once
constexpr int kRowCap = 256;          // merged rows held in LDS at once
constexpr int kNoK = INT32_MIN;       // statistics word of a share with no finite logit
constexpr int kNoToken = INT32_MIN;   // no preloaded drafted token
constexpr int kMaxQueue = 256;        // slots of a learner's delayed-feedback queue

// Everything a lane needs to turn logits into sampling weights.  Weights are kept
// in units of 1/st (st the target row's sum): an inverse-CDF draw depends only on
// ratios of weights, so the target normaliser never has to be applied per token.
struct WeightCtx {
  float c;
  float kt, kd;    // row references
  double r;        // st / sd: a draft term 2^(zd c - kd) in units of 1/st
  double s_scale;  // Cactus rescale s of the non-candidate tokens (1.0 for SpS)
  double hn;       // Cactus gamma* * st: the candidate's h in units of 1/st
  int n;           // candidate token
  int special;     // 1: token n carries gamma* (delta > 0)
  int mode;        // W_RESID, W_TARGET_H, W_TARGET
};

// The censoring learner's round (hedge_censored_update, and the learner step of a
// fused HedgeSpec round): its state, the previous round's outputs it reads, and
// the selections it writes.
struct CensoredArgs {
  double* S;          // [B][N] the learner's state (regret, or cumulative loss)
  double* W;          // [B][N] weights
  double* qloss;      // [B][Q][N] queued scaled losses
  int32_t* qtok;      // [B][Q] tokens verified since each queued round (-1: empty slot)
  int32_t* round;     // [B] rounds done
  const float* loss;  // [B][N] the previous round's losses
  const int32_t* alen;  // [B] the previous round's accepted lengths
  int K, learner;
  float eta, scale;
  const float* v;     // [T][B] selection uniforms
  int32_t* sel;       // [B] out: this round's drafters
  int32_t* sel_hist;  // [T][B] out
  int B, N, Q, T;
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
  int kl_exact;  // Cactus gamma*: 0 the Taylor form, 1 the exact root of the KL budget (verify_kernel<true, *>)
  int mode;
  int fused;
  // schedule
  int R;       // statistic rows per sequence
  int RT;      // of which target rows
  int S;       // slices per row
  int nsub;    // 512-token sub-tiles per row
  int P1;      // phase-1 (draw) units per sequence
  int P2;      // phase-2 (estimator) units per sequence
  int nlast;   // gamma calls: steps per sequence that read its statistics (0: verify calls)
  int RS;      // statistics slices per sequence (R * S)
  int total0;  // slices of the statistics list (verify and draft-tree calls: B * R * S; gamma calls: 0)
  int ngroups; // gamma groups (B * K): a position's target row and its N drafter rows
  int ncu;     // compute units; workgroup g sits in dispatch slot g / ncu
  int slots;   // workgroups per compute unit in this launch (1: no weighting)
  int topk;    // draft-tree calls: children per node (1..kMaxTopk)
  // outputs
  int32_t* accepted_len;
  int32_t* out_token;
  uint8_t* accept_mask;
  float* gamma_star;
  float* gamma;
  float* est_len;
  float* loss;
  // workspace (all zero between calls)
  uint32_t* flags;            // [3]: fault word
  uint32_t* done;             // [B] tickets of a gamma call's last steps
  unsigned long long* part;   // [B][R][S][kWaves] statistics words
  unsigned long long* tot;    // [B][kMaxSlices][kMaxSlices] draw slice totals, [reader][writer] (fp64 | kValid)
  unsigned long long* gpart;  // [B][K][N][S][kWaves] gamma partial sums (fp64 | kValid)
  unsigned long long* cand;   // draft-tree calls: [B][K][N][pieces][topk] piece records
  unsigned long long* pstat;  // gamma calls: [slots][S][kWaves] a slot's private statistics words (prefix target row)
  uint32_t* pdone;            // gamma calls: [slots] tickets of the members done with those words
  // fused HedgeSpec rounds (spec_hedgespec_round), whose learner arguments come as
  // the kernel's second argument; both nullptr in every other call
  unsigned long long* selw;  // [B] the round's drafter + 1, published by the learner to the sequence's draw units
  unsigned long long* lrnw;  // [B] non-zero once the learner has read the previous round's loss
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
__device__ __forceinline__ unsigned long long* part_row(const Params& p, int b, int r) {
  return p.part + (static_cast<size_t>(b) * p.R + r) * static_cast<size_t>(p.S) * kWaves;
}

// Statistic row streamed i-th within a sequence of the phase-0 list.  Verify
// calls: target 0, draft 0, target 1, draft 1, ...  Draft-tree calls: target rows
// 0..K-1.  (Gamma calls have no list: their groups stream every row.)
__device__ __forceinline__ int order_row(const Params& p, int i) {
  if (p.mode == MODE_TREE) return i;
  const int k = i >> 1;
  return (i & 1) ? p.RT + k : k;
}

// ---------------------------------------------------------------------------
// Published words
// ---------------------------------------------------------------------------

// Statistics word: low 32 bits the fp32 sum s (>= 1/2 whenever a finite logit was
// seen), high 32 bits the integer reference k, or kNoK with s = 0.  Never zero.
__device__ __forceinline__ unsigned long long pack_stats(float km, double s) {
  if (!(km > kNoRef)) return static_cast<unsigned long long>(static_cast<uint32_t>(kNoK)) << 32;
  const int k = static_cast<int>(fminf(fmaxf(km, -1.0e9f), 1.0e9f));
  return (static_cast<unsigned long long>(static_cast<uint32_t>(k)) << 32) |
         static_cast<unsigned long long>(__float_as_uint(static_cast<float>(s)));
}
__device__ __forceinline__ int stats_k(unsigned long long w) { return static_cast<int>(static_cast<uint32_t>(w >> 32)); }
__device__ __forceinline__ double stats_s(unsigned long long w) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(w)));
}
__device__ __forceinline__ unsigned long long pack_f64(double v) {
  return static_cast<unsigned long long>(__double_as_longlong(v)) | kValid;
}
__device__ __forceinline__ double unpack_f64(unsigned long long w) {
  return __longlong_as_double(static_cast<long long>(w & ~kValid));
}

// Re-read a word until it is published.  After the wait bound (or once another
// wait has timed out) the fault word is set and 0 is returned.
template <int kSleep = 2>
__device__ __forceinline__ unsigned long long poll_word(uint32_t* flags, unsigned long long* a) {
  unsigned long long w = ld_agent_u64(a);
  if (w != 0ull) return w;
  const unsigned long long t0 = wall_clock64();
  for (uint32_t n = 1;; ++n) {
    if ((n & 7u) == 0u && ld_agent(&flags[3]) != 0u) return 0ull;  // another wait timed out
    __builtin_amdgcn_s_sleep(kSleep);
    w = ld_agent_u64(a);
    if (w != 0ull) return w;
    if (wall_clock64() - t0 > kWaitTicks) {
      st_agent(&flags[3], 1u);
      return 0ull;
    }
  }
}

// LDS written by some lanes of this wave is then read by others: the writes
// complete first.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Phase 0: statistics slices
// ---------------------------------------------------------------------------

struct SliceLoc {
  __amdgpu_buffer_rsrc_t row;  // the row's chunks (loads past its last chunk read zero)
  int c0;                   // first chunk of the slice
  int full;                 // every chunk of the slice lies inside the row and holds 8 tokens
  unsigned long long* out;  // the slice's kWaves statistics words
};

// Slice `sig` of the list: sequence-major, then statistic row in streaming order,
// then slice, rotated by the row's position so that a workgroup whose list
// entries share one residue modulo S does not always get the same (and, for the
// last slice, shorter) slice of its rows.
__device__ __forceinline__ SliceLoc slice_loc(const Params& p, int sig) {
  if (sig >= p.total0) {
    // no slice: a buffer of no bytes, whose loads read zero without touching memory
    SliceLoc none;
    none.row = row_buffer(p.target, 0u);
    none.c0 = 0;
    none.full = 1;
    none.out = nullptr;
    return none;
  }
  const int b = sig / p.RS;
  const int q = sig - b * p.RS;
  const int i = q / p.S;
  int x = q - i * p.S + i % p.S;
  if (x >= p.S) x -= p.S;
  const int r = order_row(p, i);
  SliceLoc L;
  L.row = row_buffer(stat_row(p, b, r), static_cast<uint32_t>((p.V + kVec - 1) / kVec) * 16u);
  L.c0 = x * kSliceChunks;
  L.full = (x + 1) * kSliceTok <= p.V;
  L.out = part_row(p, b, r) + static_cast<size_t>(x) * kWaves;
  return L;
}

// A slice's chunks past the row's end read zero; slice_finish masks their tokens.
__device__ __forceinline__ void slice_load(const Params& p, const SliceLoc& L, uint4 v[kTilesPerSlice]) {
  const uint32_t lane_off = threadIdx.x * 16u;
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t)
    v[t] = stream_load16(L.row, lane_off, static_cast<uint32_t>(L.c0 + t * kThreads) * 16u);
}

// One reference per lane and half slice: the maximum over the lane's 32 logits
// first (three-input max instructions, 0.5 per logit), then 2^(z c - k) summed in
// fp32 groups of eight and in fp64 beyond.  A lane with no finite logit keeps
// k = kNoRef and s = 0.  The halves then meet at the larger reference.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

constexpr int kHalfTiles = kTilesPerSlice / 2;

__device__ __forceinline__ void half_stats(const Params& p, const SliceLoc& L, const uint4 v[kTilesPerSlice], int t0,
                                           float& k, double& s) {
  float z[kHalfTiles][8];
  if (L.full) {
#pragma unroll
    for (int t = 0; t < kHalfTiles; ++t) unpack8(v[t0 + t], z[t], 8);
  } else {
    const int nchunks = (p.V + kVec - 1) / kVec;
#pragma unroll
    for (int t = 0; t < kHalfTiles; ++t) {
      const int ci = L.c0 + (t0 + t) * kThreads + static_cast<int>(threadIdx.x);
      unpack8(v[t0 + t], z[t], ci < nchunks ? p.V - ci * kVec : 0);
    }
  }
  float m = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < kHalfTiles; ++t)
    m = max3f(max3f(z[t][0], z[t][1], z[t][2]), max3f(z[t][3], z[t][4], z[t][5]), max3f(z[t][6], z[t][7], m));
  const float c = p.c;
  k = fmaxf(kNoRef, ceilf(m * c));
  s = 0.0;
#pragma unroll
  for (int t = 0; t < kHalfTiles; ++t) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fmaf(z[t][i], c, -k));
    s += static_cast<double>(((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
  }
}

__device__ __forceinline__ void slice_finish(const Params& p, const SliceLoc& L, const uint4 v[kTilesPerSlice]) {
  float k1, k2;
  double s1, s2;
  half_stats(p, L, v, 0, k1, s1);
  half_stats(p, L, v, kHalfTiles, k2, s2);
  const float k = fmaxf(k1, k2);
  const double s = ldexp(s1, static_cast<int>(fmaxf(k1 - k, -2000.0f))) + ldexp(s2, static_cast<int>(fmaxf(k2 - k, -2000.0f)));
  const float km = wave_max(k);
  const double sw = wave_sum(ldexp(s, static_cast<int>(fmaxf(k - km, -2000.0f))));
  if (lane_id() == 0) st_agent_u64(L.out + wave_id(), pack_stats(km, sw));
}

// ---------------------------------------------------------------------------
// Merging published statistics (block-wide)
// ---------------------------------------------------------------------------

struct MergeLds {
  unsigned long long stage[kStage];
  float rk[kRowCap];   // merged reference of row i
  double rs[kRowCap];  // merged sum of row i
};

// Rows row_of(0..nrows) of sequence b (nrows <= kRowCap) -> M.rk / M.rs.
template <class RowFn>
__device__ __forceinline__ void merge_rows(const Params& p, int b, int nrows, RowFn row_of, MergeLds& M) {
  const int W = p.S * kWaves;
  const int per = kStage / W > 0 ? kStage / W : 1;
  const int tid = threadIdx.x;
  for (int i0 = 0; i0 < nrows; i0 += per) {
    const int nb = min(per, nrows - i0);
    const int nw = nb * W;
    unsigned long long w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = tid + e * kThreads;
      w[e] = 1ull;
      if (q < nw) w[e] = ld_agent_u64(part_row(p, b, row_of(i0 + q / W)) + q % W);
    }
    bool missing = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = tid + e * kThreads;
      if (q < nw) M.stage[q] = w[e];
      missing |= w[e] == 0ull;
    }
    if (missing) {  // not yet published (rare): wait for each missing word
      for (int q = tid; q < nw; q += kThreads)
        if (M.stage[q] == 0ull) M.stage[q] = poll_word(p.flags, part_row(p, b, row_of(i0 + q / W)) + q % W);
    }
    __syncthreads();
    // four rows per wave at once, one per row of 16 lanes (lane l16 of it taking
    // words l16, l16 + 16, ...)
    const int r16 = lane_id() >> 4, l16 = lane_id() & 15;
    for (int j0 = wave_id() * 4; j0 < nb; j0 += kWaves * 4) {
      const int i = j0 + r16;
      const bool valid = i < nb;
      const unsigned long long* st = M.stage + (valid ? i : 0) * W;
      int km = kNoK;
      if (valid)
        for (int q = l16; q < W; q += 16) km = max(km, stats_k(st[q]));
      km = row16_max_i(km);
      double s = 0.0;
      if (valid)
        for (int q = l16; q < W; q += 16) {
          const int kq = stats_k(st[q]);
          if (kq != kNoK) s += ldexp(stats_s(st[q]), max(kq - km, -2000));
        }
      s = row16_sum(s);
      if (valid && l16 == 0) {
        M.rk[i0 + i] = km == kNoK ? kNoRef : static_cast<float>(km);
        M.rs[i0 + i] = s;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sampling weights, sub-tile search and token search
// ---------------------------------------------------------------------------

// Sampling weight of one token in units of 1/st, with MODE and SPECIAL (Cactus's
// candidate rule, delta > 0) fixed at compile time so that a lane's tokens form
// straight-line code the scheduler can interleave:
//   W_RESID    (h - pd)+ with h = s * pt, h_n = gamma*   ([LT] §2.2 / [CA] Key design 2)
//   W_TARGET_H h          (a rejection with zero residual mass)
//   W_TARGET   pt         (bonus token)
// Without SPECIAL, h = pt (s = 1 exactly when delta = 0).
template <int MODE, bool SPECIAL>
__device__ __forceinline__ double weight1(const WeightCtx& w, float zt, float zd, int tok) {
  const double et = static_cast<double>(fast_exp2(fmaf(zt, w.c, -w.kt)));
  if (MODE == W_TARGET) return et;
  const double h = SPECIAL ? (tok == w.n ? w.hn : w.s_scale * et) : et;
  if (MODE == W_TARGET_H) return h;
  const double ed = static_cast<double>(fast_exp2(fmaf(zd, w.c, -w.kd)));
  return fmax(fma(-w.r, ed, h), 0.0);
}

// Weights of eight consecutive tokens starting at `tok0`.
template <int MODE, bool SPECIAL>
__device__ __forceinline__ void weights8(const WeightCtx& w, const float zt[8], const float zd[8], int tok0,
                                         double out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = weight1<MODE, SPECIAL>(w, zt[e], zd[e], tok0 + e);
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
  const double excl = lane_prev(incl);
  const double Z = readlane_f64(incl, 63);
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
  s_star = __builtin_amdgcn_readlane(ss, L);
  P = readlane_f64(P, L);
  lane_clamp = __builtin_amdgcn_readlane(lane_clamp, L);
  x_rel = (clamp || lane_clamp) ? __builtin_inf() : x - P;
  return s_star >= 0;
}

// Weights of one lane's 8-token chunk (chunk index ci; zero past the row's end)
// and their sum in token order.  The mass pass and the token search both use it,
// so a sub-tile's mass and its re-scan agree bit for bit.
template <int MODE, bool SPECIAL>
__device__ __forceinline__ double chunk_weights(uint4 ct, uint4 cd, int ci, int V, const WeightCtx& w,
                                                double wv[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) wv[e] = 0.0;
  double ls = 0.0;
  const int nchunks = (V + kVec - 1) / kVec;
  if (ci < nchunks) {
    const int valid = V - ci * kVec;
    float zt[8], zd[8];
    unpack8(ct, zt, valid);
    if (MODE == W_RESID)
      unpack8(cd, zd, valid);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) zd[e] = -__builtin_inff();
    weights8<MODE, SPECIAL>(w, zt, zd, ci * kVec, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e) ls += wv[e];
  }
  return ls;
}

// One wave over one sub-tile, lane l holding chunk ci (ct, cd): the token where
// the running mass passes x_rel, or the sub-tile's last positive-mass token when
// x_rel is +inf or rounding left no crossing; -1 when the sub-tile has no mass.
template <int MODE, bool SPECIAL>
__device__ __forceinline__ int subtile_token(uint4 ct, uint4 cd, int ci, int V, const WeightCtx& w, double x_rel) {
  const int lane = lane_id();
  double wv[8];
  const double ls = chunk_weights<MODE, SPECIAL>(ct, cd, ci, V, w, wv);
  const double incl = wave_incl_scan(ls);
  const double excl = lane_prev(incl);
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
  tok = __builtin_amdgcn_readlane(tok, L);
  if (tok < 0) {  // rounding put the crossing on a zero-mass lane: last positive token of the sub-tile
    const int Lp = 63 - __clzll(static_cast<long long>(pos));
    int t2 = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (wv[e] > 0.0) t2 = ci * kVec + e;
    tok = __builtin_amdgcn_readlane(t2, Lp);
  }
  return tok;
}

// Wave 0: the token in sub-tile s_star of a row (pair), read again from memory.
template <int MODE, bool SPECIAL>
__device__ __forceinline__ int find_token(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w,
                                          int s_star, double x_rel) {
  const int nchunks = (V + kVec - 1) / kVec;
  const int ci = s_star * 64 + lane_id();
  uint4 ct = make_uint4(0u, 0u, 0u, 0u), cd = ct;
  if (ci < nchunks) {
    ct = as_chunks(trow)[ci];
    if (MODE == W_RESID) cd = as_chunks(drow)[ci];
  }
  return subtile_token<MODE, SPECIAL>(ct, cd, ci, V, w, x_rel);
}

// Per-sub-tile masses of the sampling weights over tiles [0, ntiles) of a row
// into LDS (the whole-row draw of a rejection whose residual has no mass).
template <int MODE, bool SPECIAL>
__device__ __forceinline__ void row_subtiles(const uint16_t* trow, const uint16_t* drow, int V, const WeightCtx& w,
                                             int ntiles, double* lds_sub, int nsub) {
  constexpr int kBatch = 4;
  const uint4* tr = as_chunks(trow);
  const uint4* dr = as_chunks(drow);
  const int nchunks = (V + kVec - 1) / kVec;
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int j0 = 0; j0 < ntiles; j0 += kBatch) {
    uint4 vt[kBatch], vd[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int ci = (j0 + q) * kThreads + tid;
      vt[q] = make_uint4(0u, 0u, 0u, 0u);
      vd[q] = vt[q];
      if (j0 + q < ntiles && ci < nchunks) {
        vt[q] = tr[ci];
        if (MODE == W_RESID) vd[q] = dr[ci];
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (j0 + q >= ntiles) break;  // uniform over the workgroup
      double wv[8];
      const double lsum = chunk_weights<MODE, SPECIAL>(vt[q], vd[q], (j0 + q) * kThreads + tid, V, w, wv);
      const double incl = wave_incl_scan(lsum);
      const int s = (j0 + q) * kWaves + wave_id();
      if (lane_id() == 63 && s < nsub) lds_sub[s] = incl;
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
  Decision d;
  double ct[SPEC_MAX_K];  // exact-KL Cactus: pt(n) of every position (-1: no valid token)
};

struct Lds {
  MergeLds m;
  DecideLds dl;
  double subsum[kMaxSub];
  float wref[kMaxSub / kTilesPerSlice];  // bonus draws: each wave's reference, per slice of the unit
  double tot[kMaxSlices];
  int tk[kMaxSlices];                    // bonus draws: each slice's reference
  double gsum[kRowCap];
  double arat[kRowCap];
  int flag;
  int32_t qtok[kWaves][kMaxQueue];  // fused HedgeSpec rounds: each wave's learner queue counts
};

__device__ __forceinline__ int draw_drafter(const Params& p, int b) { return p.mode == MODE_VERIFY ? 0 : p.sel[b]; }

__device__ __forceinline__ int censored_round(const CensoredArgs& a, int b, int32_t* tok);

// The drafter whose rows unit x of sequence b verifies: 0 in verify calls, sel[b]
// in gamma calls, and in a fused HedgeSpec round the learner's choice for this
// round, which learner_steps published at the kernel's start.
template <bool LEARN>
__device__ __forceinline__ int unit_drafter(const Params& p, int b, int x, Lds& L) {
  if (p.mode == MODE_VERIFY) return 0;
  if (!LEARN) return p.sel[b];
  if (threadIdx.x == 0) {
    const unsigned long long w = poll_word(p.flags, &p.selw[b]);
    L.flag = static_cast<int>(static_cast<uint32_t>(w)) - 1;  // a timeout leaves -1: no valid drafter
  }
  __syncthreads();
  const int d = __builtin_amdgcn_readfirstlane(L.flag);  // the same in every lane: scalar for the row buffers
  __syncthreads();
  return d;
}

// Fused HedgeSpec rounds ([NB] overall framework: select, then verify): the
// learner steps of every sequence, taken at the kernel's start by the waves of
// gamma slot 0 (workgroups 0 .. S-1, which take no gamma rows: row_chunk with
// skip0), wave w of workgroup g taking sequences g kWaves + w, + S kWaves, ...
// Each publishes the sequence's drafter (+1) to its draw units and, once it has
// read the previous round's loss, the word that lets the estimator overwrite it.
__device__ __forceinline__ void learner_steps(const Params& p, const CensoredArgs& a, Lds& L) {
  const int S = p.S, g = blockIdx.x, w = wave_id();
  const int span = (gridDim.x / S >= 2 ? S : static_cast<int>(gridDim.x)) * kWaves;
  for (int b = g * kWaves + w; b < p.B; b += span) {
    const int pick = censored_round(a, b, L.qtok[w]);
    if (lane_id() == 0) {
      st_agent_u64(&p.lrnw[b], 1ull);
      st_agent_u64(&p.selw[b], static_cast<unsigned long long>(static_cast<uint32_t>(pick)) + 1ull);
    }
    wave_lds_sync();
  }
}

// One outcome's part of a two-outcome KL divergence, c * phi(1 + x) with
// phi(t) = t ln t - t + 1 >= 0 and x = (g - c) / c: `plain` is its direct form
// g ln(1 + x) - (g - c), whose two parts cancel when x is small; there phi(1 + x)
// is the series x^2 / 2 - x^3 / 6 + x^4 / 12 - ... (the k-th term
// (-1)^k x^k / (k (k - 1))), through x^8: below 1e-15 of the sum for |x| < 0.01.
__host__ __device__ inline double kl_share(double c, double x, double plain) {
  if (!(fabs(x) < 0.01)) return plain;
  const double q = 1.0 / 30 + x * (-1.0 / 42 + x * (1.0 / 56));
  return c * (x * x * (0.5 + x * (-1.0 / 6 + x * (1.0 / 12 + x * (-1.0 / 20 + x * q)))));
}

// [CA] Key designs 1-2 with the KL divergence, before Key design 3's Taylor
// step: the largest g in [c, 1] whose target h (h_n = g, the other tokens pt
// scaled by (1 - g) / (1 - c)) keeps KL(h || pt) <= delta.  For that h the
// divergence is the two-outcome f(g) = g ln(g / c) + (1 - g) ln((1 - g) / (1 - c)),
// evaluated as c phi(g / c) + (1 - c) phi((1 - g) / (1 - c)) (kl_share: the same
// sum as two non-negative parts), with f'(g) = ln(g / c) - ln((1 - g) / (1 - c)).
// f is increasing and convex on [c, 1], so Newton steps from above the root
// descend to it, and one from below lands above it; a step that leaves the
// bracket [lo, hi] (f(lo) <= delta < f(hi)) is replaced by the bracket's
// geometric midpoint (the root can sit many decades below 1).  The Taylor value
// starts it, its product taken as two square roots so that it does not underflow.
// It stops once a step is below 1e-8 of min(g - c, 1 - g): Newton's error after
// such a step is of the order of its square over that distance (f' vanishes at
// c and f'' grows near 1), so g - c, g and 1 - g (the scale s of the other tokens)
// are then exact to about 1e-16 relative.  `iters` (host checks) receives the
// number of steps taken.
constexpr int kKlMaxSteps = 100;
constexpr int kKlFloatSteps = 24;
__host__ __device__ inline double gamma_star_kl(double c, double delta, int* iters = nullptr) {
  if (iters) *iters = 0;
  if (!(delta > 0.0) || !(c > 0.0)) return c;
  if (c >= 1.0) return 1.0;
  const double lc = log(c);
  if (-lc <= delta) return 1.0;  // the one-hot target fits the budget
  const double c1 = 1.0 - c, rc = 1.0 / c, rc1 = 1.0 / c1;
  double lo = c, hi = 1.0;
  // a point strictly inside the bracket, or lo when none is left (adjacent doubles)
  auto mid = [&] {
    const double m = sqrt(lo) * sqrt(hi), a = 0.5 * (lo + hi);
    return m > lo && m < hi ? m : a > lo && a < hi ? a : lo;
  };
  double g = c + sqrt(2.0 * delta) * sqrt(c * c1);
  if (g == c) return c;  // the Taylor step is below half an ulp of c: so is the root's
  if (!(g < hi)) g = mid();
  // A start from single-precision Newton steps on the same f, whose logarithms cost
  // a small fraction of the double ones (the double steps below, which decide the
  // root, then take about two steps instead of five, and a root near 1 no longer
  // costs them a run of midpoints).  Only where the Taylor step is not already
  // close (its relative step above 1e-3) and c is a normal float; kept only if it
  // lies strictly inside (c, 1).
  if (g - c > 1e-3 * c && c > 1e-30) {
    const float cf = static_cast<float>(c), lcf = static_cast<float>(lc), df = static_cast<float>(delta);
    const float lc1f = log1pf(-cf);  // ln(1 - c)
    float lof = cf, hif = 1.0f, gf = static_cast<float>(g);
    for (int it = 0; it < kKlFloatSteps; ++it) {
      if (!(gf > lof && gf < hif)) {
        const float m = sqrtf(lof) * sqrtf(hif);
        gf = m > lof && m < hif ? m : 0.5f * (lof + hif);
        if (!(gf > lof && gf < hif)) break;  // the float bracket is exhausted
      }
      const float l1 = logf(gf) - lcf;      // ln(g / c)
      const float l2 = log1pf(-gf) - lc1f;  // ln((1 - g) / (1 - c))
      const float fv = gf * l1 + (1.0f - gf) * l2 - df;
      if (fv <= 0.0f)
        lof = gf;
      else
        hif = gf;
      const float gn = gf - fv / (l1 - l2);
      const bool done = fabsf(gn - gf) <= 1e-5f * fminf(gf - cf, 1.0f - gf);
      gf = gn;
      if (done) break;
    }
    const double gd = static_cast<double>(gf);
    if (gd > c && gd < 1.0) g = gd;
  }
  for (int it = 0; it < kKlMaxSteps; ++it) {
    if (iters) *iters = it + 1;
    const double d = g - c, x = d * rc, y = -d * rc1;
    const double l1 = x < 1e300 ? log1p(x) : log(g) - lc;  // ln(g / c)
    const double l2 = log1p(y);                            // ln((1 - g) / (1 - c))
    const double f = kl_share(c, x, g * l1 - d) + kl_share(c1, y, (1.0 - g) * l2 + d) - delta;
    if (f <= 0.0)
      lo = g;
    else
      hi = g;
    const double gn = g - f / (l1 - l2);
    // converged: the step is within the tolerance (g may itself be lo or hi)
    if (fabs(gn - g) <= 1e-8 * fmin(d, 1.0 - g)) return gn >= lo && gn <= hi ? gn : g;
    g = gn > lo && gn < hi ? gn : mid();
    if (g == lo) return lo;  // the bracket is down to adjacent doubles
  }
  return lo;
}

// The divergence f(g) of gamma_star_kl itself, for 0 < c < 1 and c <= g < 1.
__host__ __device__ inline double kl_divergence(double g, double c) {
  const double c1 = 1.0 - c, d = g - c, x = d / c, y = -d / c1;
  const double l1 = x < 1e300 ? log1p(x) : log(g) - log(c);
  return kl_share(c, x, g * l1 - d) + kl_share(c1, y, (1.0 - g) * log1p(y) + d);
}

// Merge the statistics of target rows 0..K-1 and drafter `drafter`'s rows 0..K-1
// (0 for verify calls; a drafter id out of range makes the sequence invalid),
// take every accept decision, and describe the draw (the bonus row K has no
// statistics: its draw finds its own references).  Writes accept_mask and
// gamma_star when `write_outputs`.  The result is in L.dl.d after the call.
template <bool KL = false>
__device__ __forceinline__ void decide(const Params& p, int b, bool write_outputs, int pre_n, int drafter, Lds& L) {
  const int K = p.K, V = p.V;
  const int t = threadIdx.x;
  const bool bad_sel = drafter < 0 || drafter >= p.N;
  const int dsafe = bad_sel ? 0 : drafter;
  // thread t < K: the drafted token of position t, its uniform and its two logits,
  // loaded first so that these loads overlap the statistics words' (every thread
  // loads, those past K position K - 1's, and the logits stay bf16 patterns until
  // the decisions, so that no wait for them comes before the words' loads)
  const int tc = min(t, K - 1);
  const int n = pre_n != kNoToken ? pre_n : p.tokens[b * K + tc];
  const bool tok_ok = t < K && !bad_sel && n >= 0 && n < V;
  const int nc = min(max(n, 0), V - 1);
  const float rr = p.r[b * K + tc];
  const uint32_t zt_bits = target_row(p, b, tc)[nc];
  const uint32_t zd_bits = draft_row(p, b, dsafe, tc)[nc];
  // rows 0..K-1: target rows 0..K-1; rows K..2K-1: the drafter's rows 0..K-1
  merge_rows(p, b, 2 * K, [&](int i) { return i < K ? i : p.RT + dsafe * K + (i - K); }, L.m);
  // threads t < K (all in wave 0): the accept test of position t
  uint32_t state = ST_INVALID;
  double ct = 0.0, gs = 0.0;
  if (t < K) {
    bool acc = false;
    if (tok_ok) {
      const RowStats st{L.m.rk[t], L.m.rs[t]};
      const RowStats sd{L.m.rk[K + t], L.m.rs[K + t]};
      const float zt = __uint_as_float(zt_bits << 16), zd = __uint_as_float(zd_bits << 16);
      // [CA] Key design 3 with the verifier's probability c of the candidate; delta = 0 is SpS.
      ct = fmin(token_prob(zt, p.c, st), 1.0);
      const double cd = token_prob(zd, p.c, sd);
      if (KL && p.delta > 0.0) {
        // accept iff r pd(n) < gamma*, decided without the root: gamma* >= c,
        // gamma* <= 1, and the divergence grows on [c, 1], so x = r pd(n) in [c, 1)
        // lies below gamma* exactly when its divergence is below delta (c = 0
        // leaves gamma* = 0, which nothing lies below).  The draw finds gamma*.
        const double xr = static_cast<double>(rr) * cd;
        acc = ct > 0.0 && (xr < ct || (xr < 1.0 && kl_divergence(xr, ct) < p.delta));
      } else {
        gs = fmin(ct + sqrt(2.0 * p.delta * ct * (1.0 - ct)), 1.0);
        const double ratio = cd > 0.0 ? gs / cd : (gs > 0.0 ? __builtin_inf() : 0.0);
        acc = static_cast<double>(rr) < ratio;  // [LT] §5.1: strict
        if (write_outputs && p.gamma_star) p.gamma_star[b * K + t] = static_cast<float>(gs);
      }
      state = acc ? ST_ACCEPT : ST_REJECT;
    }
    if (KL) L.dl.ct[t] = tok_ok ? ct : -1.0;
    if (write_outputs && p.accept_mask) p.accept_mask[b * K + t] = acc ? 1 : 0;
  }
  // wave 0: the first rejection A (ballots over the positions) and the draw
  if (wave_id() == 0) {
    const unsigned long long rej = __ballot(t < K && state == ST_REJECT);
    const unsigned long long inv = __ballot(t < K && state == ST_INVALID);
    const int A = rej != 0ull ? __ffsll(static_cast<long long>(rej)) - 1 : K;
    const double ctA = readlane_f64(ct, A < K ? A : 0);
    const double gsA = readlane_f64(gs, A < K ? A : 0);
    const int nA = __builtin_amdgcn_readlane(n, A < K ? A : 0);
    if (t == 0) {
      Decision d;
      WeightCtx w;
      w.c = p.c;
      w.kd = 0.0f;
      w.r = 0.0;
      w.s_scale = 1.0;
      w.hn = 0.0;
      w.n = -1;
      w.special = 0;
      if (bad_sel || inv != 0ull) {
        d.A = -1;
        d.draw_row = 0;
        d.pair = 0;
        w.mode = W_TARGET;
        w.kt = 0.0f;
      } else if (A < K) {
        // [LT] §9.1: the first rejection A is resampled from the residual of its row pair
        d.A = A;
        d.draw_row = A;
        d.pair = 1;
        w.mode = W_RESID;
        w.kt = L.m.rk[A];
        w.kd = L.m.rk[K + A];
        w.r = L.m.rs[A] / L.m.rs[K + A];
        // [CA] Key design 2 (1.0 exactly at delta = 0); with the exact-KL gamma*
        // the draw sets both once it has gamma* (kl_positions)
        w.s_scale = ctA < 1.0 ? (1.0 - gsA) / (1.0 - ctA) : 0.0;
        w.hn = gsA * L.m.rs[A];
        w.n = nA;
        w.special = p.delta > 0.0 ? 1 : 0;
      } else {
        // every draft kept: bonus token from target row K (the draw sets the references)
        d.A = K;
        d.draw_row = K;
        d.pair = 0;
        w.mode = W_TARGET;
        w.kt = 0.0f;
      }
      d.w = w;
      L.dl.d = d;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Units
// ---------------------------------------------------------------------------

// A sequence's last step: clear its statistics words once every step that reads
// them is done.  In a verify call (nlast = 0) the draw unit passed as `clearer`
// knows this, having read every draw unit's total (each unit publishes its total
// after its last read of the words).  In a gamma call, the steps that read them
// (nlast: the draw units of a fused call and the estimator) take a ticket and
// the last one clears.  LEARN: a fused HedgeSpec round, whose drafter word is
// cleared with them.
template <bool LEARN = false>
__device__ __forceinline__ void finish_sequence(const Params& p, int b, bool clearer, Lds& L) {
  int last = clearer ? 1 : 0;
  if (p.nlast == 1) {
    last = 1;
  } else if (p.nlast > 1) {
    stores_complete();  // this step's own words are out before it takes its ticket
    __syncthreads();
    if (threadIdx.x == 0) {
      const int l = ticket(&p.done[b]) == static_cast<uint32_t>(p.nlast - 1) ? 1 : 0;
      if (l) st_agent(&p.done[b], 0u);
      L.flag = l;
    }
    __syncthreads();
    last = L.flag;
  }
  if (last) {
    unsigned long long* w = part_row(p, b, 0);
    const int n = p.R * p.S * kWaves;
    for (int q = threadIdx.x; q < n; q += kThreads) st_agent_u64(w + q, 0ull);
    if (LEARN && threadIdx.x == 0) st_agent_u64(&p.selw[b], 0ull);  // every draw unit has read it
  }
  __syncthreads();
}

// Wave: the inverse-CDF crossing among up to 64 masses, lane i holding mass i
// (0 past the last): the first i whose running mass (a wave scan) passes x, with
// x made relative to the mass before it; when rounding leaves no crossing, the
// last i with mass and x = +inf.  -1 when there is no mass.  Every wave that
// calls it on the same masses gets the same answer.
__device__ __forceinline__ int wave_crossing(double m, double incl, double& x) {
  const unsigned long long hit = __ballot(incl > x);
  if (hit != 0ull) {
    const int i = __ffsll(static_cast<long long>(hit)) - 1;
    x -= readlane_f64(lane_prev(incl), i);
    return i;
  }
  const unsigned long long pos = __ballot(m > 0.0);
  x = __builtin_inf();
  return pos == 0ull ? -1 : 63 - __clzll(static_cast<long long>(pos));
}

// Wave: the crossing slice of a sequence's draw, lane i holding slice i's total:
// x = u * Z with Z the sum of the totals.  -1 when Z is not positive.
__device__ __forceinline__ int crossing_slice(double t, double u, double& x_rel) {
  const double incl = wave_incl_scan(t);
  const double Z = readlane_f64(incl, 63);
  if (!(Z > 0.0)) return -1;
  x_rel = u * Z;
  return wave_crossing(t, incl, x_rel);
}

constexpr int kSliceSub = kTilesPerSlice * kWaves;  // 512-token sub-tiles of a slice

// Draw unit x of a sequence takes slices x, x + P1, x + 2 P1, ... < S (P1 the
// sequence's draw units: S when the grid holds a unit per slice, fewer
// otherwise, so that no workgroup runs two units one after the other).
__device__ __forceinline__ int unit_slices(const Params& p, int x) {
  return p.P1 == p.S ? 1 : (p.S - x + p.P1 - 1) / p.P1;
}
// The draw unit that takes slice s.
__device__ __forceinline__ int slice_unit(const Params& p, int s) { return p.P1 == p.S ? s : s % p.P1; }

// Draw unit x publishes the total of each of its slices s (the wave scan of the
// slice's sub-tile masses, L.subsum[j kSliceSub ..] for its j-th slice) to each
// unit y of its sequence as word tot[b][y][s], reads the S words addressed to it
// (clearing them: it is their only reader), and returns the crossing slice of
// the sequence's draw (-1 for none), with x_rel the draw's point relative to the
// mass before that slice.
// REF (bonus draws, whose row has no merged statistics): a wave's sub-tile masses
// are in units of 2^-k_w, k_w its own reference (L.wref), so a slice's total is
// published as a statistics word at the slice's reference (the largest of its
// waves'), the reader brings the totals to the largest slice reference before
// the scan, and x_rel is returned in units of the crossing slice's reference
// (kx, from the crossing slice's word).
template <bool MULTI = false, bool REF = false>
__device__ __forceinline__ int exchange_totals(const Params& p, int b, int x, double u, double& x_rel, Lds& L,
                                               int& kx) {
  const int tid = threadIdx.x;
  unsigned long long* tw = p.tot + static_cast<size_t>(b) * kMaxSlices * kMaxSlices;
  if (tid < 64) {  // wave 0
    auto publish = [&](int j) {
      double m = tid < kSliceSub ? L.subsum[j * kSliceSub + tid] : 0.0;
      float ks = 0.0f;
      if (REF) {
        const float* wr = L.wref + j * kWaves;
        ks = fmaxf(fmaxf(wr[0], wr[1]), fmaxf(wr[2], wr[3]));
        if (tid < kSliceSub) m = ldexp(m, static_cast<int>(fmaxf(wr[tid & (kWaves - 1)] - ks, -2000.0f)));
      }
      const double T = readlane_f64(wave_incl_scan(m), 63);
      if (tid < p.P1) st_agent_u64(tw + tid * kMaxSlices + x + j * p.P1, REF ? pack_stats(ks, T) : pack_f64(T));
    };
    publish(0);
    if (MULTI)
      for (int j = 1; j < unit_slices(p, x); ++j) publish(j);
  }
  if (tid < p.S) {
    unsigned long long* src = tw + x * kMaxSlices + tid;
    unsigned long long w = ld_agent_u64(src);
    if (w == 0ull) w = poll_word(p.flags, src);
    if (REF) {
      L.tk[tid] = stats_k(w);
      L.tot[tid] = stats_s(w);
    } else {
      L.tot[tid] = unpack_f64(w);
    }
    st_agent_u64(src, 0ull);
  }
  __syncthreads();
  const int lane = lane_id();
  if (!REF) return crossing_slice(lane < p.S ? L.tot[lane] : 0.0, u, x_rel);
  const int kq = lane < p.S ? L.tk[lane] : kNoK;
  const int km = wave_max_i(kq);
  const double t = kq != kNoK ? ldexp(L.tot[lane], max(kq - km, -2000)) : 0.0;
  const int xs = crossing_slice(t, u, x_rel);
  if (xs >= 0) {
    kx = L.tk[xs];
    x_rel = ldexp(x_rel, min(km - kx, 2000));
  }
  return xs;
}

// Draw unit x of sequence b, decision d made: the sub-tile masses of slice x of
// the draw row (pair), the totals exchanged, and, if the crossing falls in this
// slice, the token from the rows still held in registers.  Returns the crossing
// slice (-1: the draw has no mass).
// Exact-KL Cactus: gamma* of every position, lane t < K solving position t (K <=
// 64; every wave does the same work, so none waits for another).  Unit 0 writes
// them out (`write`); the result is gamma* of position A (0 if A is none).
__device__ __forceinline__ double kl_positions(const Params& p, int b, bool write, int A, const Lds& L) {
  const int t = lane_id();
  const double ct = t < p.K ? L.dl.ct[t] : -1.0;
  double gsv = 0.0;
  if (ct >= 0.0) gsv = gamma_star_kl(ct, p.delta);
  if (write && wave_id() == 0 && ct >= 0.0 && p.gamma_star) p.gamma_star[b * p.K + t] = static_cast<float>(gsv);
  return A >= 0 && A < p.K ? readlane_f64(gsv, A) : 0.0;
}

// With KL (exact-KL Cactus, delta > 0), the residual's gamma* is found here, while
// the slice's loads are in flight, and completes d.w; a bonus draw's unit 0 finds
// every position's gamma* (outputs only) at the same point.
// MULTI: the unit may take several slices (P1 < S); without it, slice x only,
// in straight-line code.
// W_TARGET (the bonus row, which has no merged statistics): each wave weighs its
// share of a slice at its own reference k_w = ceil(max z c) over that share
// (L.wref), and exchange_totals brings the slices to a common one.
// LEARN (fused HedgeSpec rounds): `drafter` is the learner's pick for the round;
// the other calls look theirs up here (0, or sel[b]), each instance on its own,
// which keeps the residual draws' row loads inside their own instances (a drafter
// shared by both made the compiler hoist them above the choice between the two,
// measured 2% slower).
template <int MODE, bool SPECIAL, bool KL = false, bool MULTI = false, bool LEARN = false>
__device__ __forceinline__ int draw_slice(const Params& p, int b, int x, Decision& d, int drafter, Lds& L) {
  const int tid = threadIdx.x, wave = wave_id();
  const uint16_t* trow = target_row(p, b, d.draw_row);
  const uint16_t* drow = d.pair ? draft_row(p, b, LEARN ? drafter : draw_drafter(p, b), d.draw_row) : trow;
  const uint32_t row_bytes = static_cast<uint32_t>((p.V + kVec - 1) / kVec) * 16u;
  const __amdgpu_buffer_rsrc_t tr = row_buffer(trow, row_bytes);
  const __amdgpu_buffer_rsrc_t dr = row_buffer(drow, row_bytes);
  // the unit's slices one after another; the last one's rows stay in registers
  const int ns = MULTI ? unit_slices(p, x) : 1;
  uint4 vt[kTilesPerSlice], vd[kTilesPerSlice];
  auto slice_masses = [&](int j) {
    const int sl = x + j * p.P1;
    const int c0 = sl * kTilesPerSlice * kThreads + tid;  // this lane's chunk of the slice's first tile
    // chunks past the row's end read zero and weigh nothing (chunk_weights)
#pragma unroll
    for (int q = 0; q < kTilesPerSlice; ++q) {
      const uint32_t uo = static_cast<uint32_t>((sl * kTilesPerSlice + q) * kThreads) * 16u;
      vt[q] = buffer_load16(tr, tid * 16u, uo);
      vd[q] = MODE == W_RESID ? buffer_load16(dr, tid * 16u, uo) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (KL && MODE == W_TARGET && j == 0 && x == 0 && p.delta > 0.0 && p.gamma_star)
      kl_positions(p, b, true, -1, L);  // the outputs only: a bonus draw needs no gamma*
    if (KL && MODE == W_RESID && SPECIAL && j == 0) {
      const double gsA = kl_positions(p, b, x == 0, d.A, L);
      const double ctA = L.dl.ct[d.A];
      d.w.s_scale = ctA < 1.0 ? (1.0 - gsA) / (1.0 - ctA) : 0.0;
      d.w.hn = gsA * L.m.rs[d.A];
    }
    if (MODE == W_TARGET) {
      const int nchunks = (p.V + kVec - 1) / kVec;
      float mx = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < kTilesPerSlice; ++q) {
        const int ci = c0 + q * kThreads;
        float z[8];
        unpack8(vt[q], z, ci < nchunks ? p.V - ci * kVec : 0);
        mx = max3f(max3f(z[0], z[1], z[2]), max3f(z[3], z[4], z[5]), max3f(z[6], z[7], mx));
      }
      d.w.kt = fmaxf(kNoRef, ceilf(wave_max(mx) * p.c));
      if (lane_id() == 0) L.wref[j * kWaves + wave] = d.w.kt;
    }
#pragma unroll
    for (int q = 0; q < kTilesPerSlice; ++q) {
      double wv[8];
      const double ls = chunk_weights<MODE, SPECIAL>(vt[q], vd[q], c0 + q * kThreads, p.V, d.w, wv);
      const double incl = wave_incl_scan(ls);
      if (lane_id() == 63) L.subsum[j * kSliceSub + q * kWaves + wave] = incl;
    }
  };
  // the first slice as straight-line code (the only one when the grid holds a
  // unit per slice), the others, if any, in a loop
  slice_masses(0);
  if (MULTI)
    for (int j = 1; j < ns; ++j) slice_masses(j);
  __syncthreads();
  double x_rel = 0.0;
  int kx = 0;
  const int xs = exchange_totals<MULTI, MODE == W_TARGET>(p, b, x, static_cast<double>(p.u[b * (p.K + 1) + d.draw_row]),
                                                         x_rel, L, kx);
  if (xs < 0 || (MULTI ? slice_unit(p, xs) : xs) != x) return xs;
  // the crossing slice is this unit's j-th; its total is positive, so one of its
  // sub-tiles has mass; the scan is the one that formed the total
  const int js = (xs - x) / p.P1;
  double m = lane_id() < kSliceSub ? L.subsum[js * kSliceSub + lane_id()] : 0.0;
  float kw = 0.0f;
  if (MODE == W_TARGET) {  // every sub-tile at the slice's reference kx, as its published total
    const float* wr = L.wref + js * kWaves;
    m = ldexp(m, static_cast<int>(fmaxf(wr[lane_id() & (kWaves - 1)] - static_cast<float>(kx), -2000.0f)));
    kw = wr[wave];
  }
  const int ss = wave_crossing(m, wave_incl_scan(m), x_rel);
  const int qs = ss / kWaves;
  if (wave == ss - qs * kWaves) {
    if (MODE == W_TARGET) {  // this wave's own units
      d.w.kt = kw;
      x_rel = ldexp(x_rel, static_cast<int>(fminf(static_cast<float>(kx) - kw, 2000.0f)));
    }
    const int c0 = xs * kTilesPerSlice * kThreads + tid;
    uint4 ct = vt[0], cd = vd[0];
    if (!MULTI || js == ns - 1) {  // the last slice: its rows are still in registers
#pragma unroll
      for (int q = 1; q < kTilesPerSlice; ++q)
        if (q == qs) {
          ct = vt[q];
          cd = vd[q];
        }
    } else {  // an earlier slice: its crossing tile is read again
      const uint32_t uo = static_cast<uint32_t>((xs * kTilesPerSlice + qs) * kThreads) * 16u;
      ct = buffer_load16(tr, tid * 16u, uo);
      cd = MODE == W_RESID ? buffer_load16(dr, tid * 16u, uo) : make_uint4(0u, 0u, 0u, 0u);
    }
    const int tok = subtile_token<MODE, SPECIAL>(ct, cd, c0 + qs * kThreads, p.V, d.w, x_rel);
    if (lane_id() == 0) {
      p.accepted_len[b] = tok >= 0 ? d.A : -1;
      p.out_token[b] = tok >= 0 ? tok : -1;
    }
  }
  return xs;
}

// A rejection whose residual has no mass: the token is drawn from the position's
// target h instead (whole row; rare).
template <bool SPECIAL>
__device__ __forceinline__ void target_h_draw(const Params& p, int b, const Decision& d, Lds& L) {
  const uint16_t* trow = target_row(p, b, d.draw_row);
  const double uu = static_cast<double>(p.u[b * (p.K + 1) + d.draw_row]);
  WeightCtx wh = d.w;
  wh.mode = W_TARGET_H;
  __syncthreads();  // every thread is done with the slice's masses in LDS
  row_subtiles<W_TARGET_H, SPECIAL>(trow, trow, p.V, wh, (p.V + kTile - 1) / kTile, L.subsum, p.nsub);
  __syncthreads();
  if (wave_id() == 0) {
    int s_star = -1;
    double x_rel = 0.0;
    int tok = -1;
    if (find_subtile(L.subsum, p.nsub, uu, s_star, x_rel))
      tok = find_token<W_TARGET_H, SPECIAL>(trow, trow, p.V, wh, s_star, x_rel);
    if (lane_id() == 0) {
      p.accepted_len[b] = tok >= 0 ? d.A : -1;
      p.out_token[b] = tok >= 0 ? tok : -1;
    }
  }
}

// Draw unit x of sequence b.  Unit 0 also writes the per-position outputs, the
// outputs of a sequence with no valid draw, and the outputs of a draw with no
// mass.  `pre_n`: the drafted token of position min(threadIdx.x, K - 1), loaded ahead of
// time, or kNoToken.  MULTI: units of several slices (a kernel instance of its
// own, so that the other launches keep the single-slice code alone).
// LEARN: a fused HedgeSpec round (the learner step in the sequence's first unit).
template <bool KL = false, bool MULTI = false, bool LEARN = false>
__device__ __forceinline__ void unit_draw(const Params& p, int b, int x, int pre_n, Lds& L) {
  const int drafter = unit_drafter<LEARN>(p, b, x, L);
  decide<KL>(p, b, x == 0, pre_n, drafter, L);
  Decision d = L.dl.d;
  // exact-KL gamma* outputs of a sequence with no draw (a bonus draw finds them
  // while its loads are in flight, a residual draw as it completes its weights)
  if (KL && x == 0 && p.delta > 0.0 && p.gamma_star && d.A < 0) kl_positions(p, b, true, -1, L);
  int xs;
  if (d.A < 0) {
    // no draw: the totals are still exchanged, so that unit 0 knows when to clear
    for (int q = threadIdx.x; q < (MULTI ? unit_slices(p, x) : 1) * kSliceSub; q += kThreads) L.subsum[q] = 0.0;
    __syncthreads();
    double x_rel = 0.0;
    int kx = 0;
    xs = exchange_totals<MULTI>(p, b, x, 0.0, x_rel, L, kx);
    if (x == 0 && threadIdx.x == 0) {
      p.accepted_len[b] = -1;
      p.out_token[b] = -1;
    }
  } else {
    xs = !d.pair       ? draw_slice<W_TARGET, false, KL, MULTI, LEARN>(p, b, x, d, drafter, L)
         : d.w.special ? draw_slice<W_RESID, true, KL, MULTI, LEARN>(p, b, x, d, drafter, L)
                       : draw_slice<W_RESID, false, false, MULTI, LEARN>(p, b, x, d, drafter, L);
    if (xs < 0 && x == 0) {
      if (d.w.special)
        target_h_draw<true>(p, b, d, L);
      else
        target_h_draw<false>(p, b, d, L);
    }
  }
  // the unit that holds the crossing slice (unit 0 when there is none) has read
  // every unit's totals
  finish_sequence<LEARN>(p, b, (xs < 0 ? 0 : MULTI ? slice_unit(p, xs) : xs) == x, L);
}

// ---------------------------------------------------------------------------
// Gamma groups: statistics and gamma in one pass
// ---------------------------------------------------------------------------
//
// Group (b, k) is position k of sequence b: the target row k and the N drafter
// rows k.  A slot of S workgroups takes a group at a time; member x streams slice
// x of each of the N + 1 rows once, keeping the lane's 64 exponentials of the
// target slice and of the current drafter slice in registers.  After publishing
// a row slice's statistics it waits for the other members' words of that row
// (they stream the same rows in the same order), turns the exponentials into
// probabilities with the row's normaliser, and publishes its slice's share of
// gamma_i = sum_x min(pt, pd_i) ([NB] Key design 1), without reading the row
// again.  The next row's loads are in flight meanwhile.

// Lane statistics of one slice whose tokens past the row's end are already -inf
// (mask_tail): the lane's reference k, the ceiling of its largest z c (a
// three-input max pass first), and s = sum 2^(z c - k) over its 64 logits, the
// terms kept in e.  (A single pass with a reference from the first eight logits
// and a fallback for the rare lane it does not fit measured 15 % slower: the
// fallback path's registers spilled to scratch.)
__device__ __forceinline__ float lane_exps(const Params& p, const uint4 v[kTilesPerSlice], float e[kTilesPerSlice][8],
                                           double& s) {
  const float c = p.c;
  float m = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    float z[8];
    unpack8(v[t], z, 8);
    m = max3f(max3f(z[0], z[1], z[2]), max3f(z[3], z[4], z[5]), max3f(z[6], z[7], m));
  }
  const float k = fmaxf(kNoRef, ceilf(m * c));
  s = 0.0;
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    float z[8];
    // (forcing a fresh unpack here with an empty asm on the loads measured 12-15 %
    // slower: it also pins the schedule)
    unpack8(v[t], z, 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[t][i] = fast_exp2(fmaf(z[i], c, -k));
    s += static_cast<double>(((e[t][0] + e[t][1]) + (e[t][2] + e[t][3])) + ((e[t][4] + e[t][5]) + (e[t][6] + e[t][7])));
  }
  return k;
}

// Wave: publish its share of a slice's statistics (one word per wave).
__device__ __forceinline__ void publish_slice_stats(unsigned long long* row_words, int x, float k, double s) {
  const float km = wave_max(k);
  const double sw = wave_sum(ldexp(s, static_cast<int>(fmaxf(k - km, -2000.0f))));
  if (lane_id() == 0) st_agent_u64(row_words + static_cast<size_t>(x) * kWaves + wave_id(), pack_stats(km, sw));
}

// Wave: a row's statistics words, loaded (issue) and then, once the loads are
// back, waited for where still missing and merged (finish).  Between the two the
// wave can do other work while the loads fly.
constexpr int kRowWordsPerLane = kMaxSlices * kWaves / 64;

__device__ __forceinline__ void wave_row_issue(const Params& p, const unsigned long long* row_words,
                                               unsigned long long wv[kRowWordsPerLane]) {
  const int W = p.S * kWaves;
  // every lane loads (lanes past the row's words reload word 0, and
  // wave_row_finish ignores them): loads behind a branch would blur the count of
  // loads in flight that the waits for the slice loads rely on
#pragma unroll
  for (int j = 0; j < kRowWordsPerLane; ++j) {
    const int q = lane_id() + 64 * j;
    wv[j] = ld_agent_u64(const_cast<unsigned long long*>(row_words) + (q < W ? q : 0));
  }
  // keep the loads here: the compiler would otherwise sink them to their use,
  // behind loads that a wait for them would then also wait for
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ RowStats wave_row_finish(const Params& p, const unsigned long long* row_words,
                                                    unsigned long long wv[kRowWordsPerLane]) {
  const int W = p.S * kWaves;
  int km = kNoK;
#pragma unroll
  for (int j = 0; j < kRowWordsPerLane; ++j) {
    const int q = lane_id() + 64 * j;
    if (q < W && wv[j] == 0ull) wv[j] = poll_word(p.flags, const_cast<unsigned long long*>(row_words) + q);
    if (q < W) km = max(km, stats_k(wv[j]));
  }
  km = wave_max_i(km);
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < kRowWordsPerLane; ++j) {
    const int q = lane_id() + 64 * j;
    if (q < W) {
      const int kq = stats_k(wv[j]);
      if (kq != kNoK) s += ldexp(stats_s(wv[j]), max(kq - km, -2000));
    }
  }
  s = wave_sum(s);
  return RowStats{km == kNoK ? kNoRef : static_cast<float>(km), s};
}

// Factor turning a lane's terms (reference kl) into probabilities of the row.
__device__ __forceinline__ float lane_scale(float kl, const RowStats& r) {
  if (kl == kNoRef || !(r.s > 0.0)) return 0.0f;
  return static_cast<float>(ldexp(1.0 / r.s, static_cast<int>(fmaxf(kl - r.k, -2000.0f))));
}

// The target slice's 64 terms per lane, in LDS as 16 float4 per lane (terms
// 4j .. 4j + 3 in pt[j][lane]: conflict-free, consecutive lanes reading
// consecutive 16-byte words), while the drafters' slices stream through
// registers.  Four terms per read keep few reads in flight for the registers
// the step leaves free.
struct GammaLds {
  float4 pt[kTilesPerSlice * 2][kThreads];
  int last;  // the member that clears its slot's private words
};

// A slice that runs past the row's end: chunks beyond it become -inf logits and
// the last chunk's tokens beyond it too, so that the reductions need no bounds.
__device__ __forceinline__ void mask_tail(uint4 v[kTilesPerSlice], int ci0, int V) {
  // the bounds are the same every step: recompute them here rather than let the
  // compiler keep 64 lane masks live across the loop (they would spill)
  asm volatile("" : "+v"(ci0));
  const int nchunks = (V + kVec - 1) / kVec;
  constexpr uint32_t kNegInf2 = 0xff80ff80u;  // two bf16 -inf
  // selects, not branches: a branch would join into copies of the load registers,
  // and the copies would wait for loads issued after these
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    const int ci = ci0 + t * kThreads;
    const int valid = V - ci * kVec;  // tokens of this chunk inside the row
    uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = 2 * d < valid ? (w[d] & 0x0000ffffu) : (kNegInf2 & 0x0000ffffu);
      const uint32_t hi = 2 * d + 1 < valid ? (w[d] & 0xffff0000u) : (kNegInf2 & 0xffff0000u);
      w[d] = lo | hi;
    }
    v[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Shares of the workgroups by dispatch slot.  A compute unit holds `slots`
// workgroups, dispatched in slot order (workgroup g in slot g / ncu), and waves
// dispatched first win the arbitration for the compute unit's issue slots and
// memory, so slot 0 runs fastest.  Slot c >= 1 takes slot_share(slots, c) / 11 of
// an even share of the work and slot 0 the rest, so that the slots finish
// together.  Both kernels run two slots (measured: the second takes 9/11 of
// phase 0, and 8/11 of the gamma groups' rows below); the shares of three and four
// slots are rougher measurements, kept for devices where more fit.
constexpr int kMaxSlots = 4;
constexpr int kShareDen = 11;
__host__ __device__ constexpr int slot_share(int P, int c) {
  return P == 2 ? (c == 1 ? 9 : 11) : P == 3 ? (c == 1 ? 11 : c == 2 ? 9 : 11) : P == 4 ? 11 - c : 11;
}
// The gamma groups' shares: with two slots the second takes 8/11 (measured: its
// members' steps run about a quarter slower than the first slot's, since they
// also wait longer for the other members' words); other slot counts as above.
__host__ __device__ constexpr int gamma_share(int P, int c) {
  return P == 2 ? (c == 1 ? 8 : 11) : slot_share(P, c);
}

// The rows of all groups, group by group (row 0 the target row k, row 1 + i
// drafter i's row k), are cut into Q chunks, one per slot, in proportion to the
// slots' weights (slot_weights).  A chunk that starts inside a group begins with
// that group's target row once more (a prefix job, whose statistics words are the
// slot's own), so that its drafter rows meet the target's probabilities.
struct RowChunk {
  int64_t j0, j1;  // the chunk's rows [j0, j1) of the sequence
  int prefix;      // 1: job 0 is the target row of group j0 / R1, on private words
  int njobs;
};

// Total weight of the gamma slots 0 .. q-1 (S members each, workgroups q S ..
// q S + S - 1): a slot weighs the share of the last dispatch slot among its
// members, which sets its pace (every member waits for the others' words of each
// row).  P dispatch slots of ncu workgroups; P = 1 weighs every slot alike.
__host__ __device__ inline int64_t slot_weights(int q, int S, int ncu, int P) {
  if (P <= 1) return static_cast<int64_t>(q) * kShareDen;
  int64_t w = 0;
  int done = 0;  // slots counted so far
#pragma unroll
  for (int c = 0; c < kMaxSlots; ++c) {
    if (c >= P) break;
    // slots whose last member lies in dispatch slot c or before: (q' + 1) S <= (c + 1) ncu
    const int upto = c == P - 1 ? q : min(q, static_cast<int>(static_cast<int64_t>(c + 1) * ncu / S));
    if (upto > done) {
      w += static_cast<int64_t>(upto - done) * gamma_share(P, c);
      done = upto;
    }
  }
  return w;
}

// skip0 (Q >= 2): slot 0 takes no rows (in a fused HedgeSpec round its members
// take the learner steps instead) and the other slots share them as above.
__host__ __device__ inline RowChunk row_chunk(int64_t J, int R1, int Q, int slot, int S, int ncu, int P,
                                              bool skip0 = false) {
  RowChunk c;
  const int64_t w0 = skip0 && Q >= 2 ? slot_weights(1, S, ncu, P) : 0;
  const int64_t WQ = slot_weights(Q, S, ncu, P) - w0;
  c.j0 = J * max(slot_weights(slot, S, ncu, P) - w0, static_cast<int64_t>(0)) / WQ;
  c.j1 = J * max(slot_weights(slot + 1, S, ncu, P) - w0, static_cast<int64_t>(0)) / WQ;
  c.prefix = c.j0 < c.j1 && (c.j0 % R1) != 0 ? 1 : 0;
  c.njobs = c.j0 < c.j1 ? static_cast<int>(c.j1 - c.j0) + c.prefix : 0;
  return c;
}

// Job n of a chunk -> group q (nG past the last job), row r, private words.
__host__ __device__ inline void chunk_job(const RowChunk& c, int R1, int nG, int n, int& q, int& r, bool& priv) {
  if (n >= c.njobs) {
    q = nG;
    r = 0;
    priv = false;
    return;
  }
  const int64_t j = c.prefix ? (n == 0 ? c.j0 - c.j0 % R1 : c.j0 + n - 1) : c.j0 + n;
  q = static_cast<int>(j / R1);
  r = static_cast<int>(j - static_cast<int64_t>(q) * R1);
  priv = c.prefix && n == 0;
}

// FULL: the member's slice lies inside the row (every member but the last of a
// ragged row), so its loop carries no masking.  LEARN: a fused HedgeSpec round
// (slot 0 takes no rows).
template <bool FULL, bool LEARN>
__device__ __forceinline__ void gamma_member(const Params& p, GammaLds& GL, int slot, int x) {
  const int S = p.S, Q = gridDim.x / S;
  const int K = p.K, N = p.N, R1 = N + 1, nG = p.ngroups;
  const int ci0 = x * kSliceChunks + static_cast<int>(threadIdx.x);
  const int nchunks = (p.V + kVec - 1) / kVec;
  const int tid = threadIdx.x;
  // dispatch slots as phase 0 counts them (all of them in the grid, else one)
  const int P = (p.slots >= 1 && p.slots <= kMaxSlots && p.ncu * p.slots == static_cast<int>(gridDim.x)) ? p.slots : 1;
  const RowChunk ch = row_chunk(static_cast<int64_t>(nG) * R1, R1, Q, slot, S, p.ncu, P, LEARN);
  if (ch.njobs == 0) return;
  const int prefix = ch.prefix, njobs = ch.njobs;
  unsigned long long* own_words = p.pstat + static_cast<size_t>(slot) * S * kWaves;
  // jobs n and n + 1 advance one row at a time (no division per step): the
  // cursor holds job n + 1's group and row, and how many jobs are left after it
  int nq, nr, left;
  bool npriv;
  chunk_job(ch, R1, nG, 0, nq, nr, npriv);
  left = njobs - 1;
  auto advance = [&](int& q, int& r, bool& priv) {  // returns job n + 1 into (q, r, priv)
    q = nq;
    r = nr;
    priv = npriv;
    if (left <= 0) {
      nq = nG;
      nr = 0;
    } else if (npriv) {  // after the prefix: the chunk's first row
      nq = static_cast<int>(ch.j0 / R1);
      nr = static_cast<int>(ch.j0 - static_cast<int64_t>(nq) * R1);
    } else if (++nr == R1) {
      nr = 0;
      ++nq;
    }
    npriv = false;
    --left;
  };
  // row r of group q: 0 the target row k, 1 + i drafter i's row k
  auto row_index = [&](int k, int r) { return r == 0 ? k : p.RT + (r - 1) * K + k; };
  auto words_of = [&](int q, int r, bool priv) -> unsigned long long* {
    if (priv) return own_words;
    const int b = q / K, k = q - b * K;
    return part_row(p, b, row_index(k, r));
  };
  // Unconditional buffer loads: chunks past the row's end read zero (mask_tail
  // then masks their tokens), so no load sits behind a branch whose join would
  // copy, and therefore wait for, the registers it fills.
  const uint32_t row_bytes = static_cast<uint32_t>(nchunks) * 16u;
  auto load = [&](int q, int r, uint4 (&v)[kTilesPerSlice]) {
    const bool none = q >= nG;
    const int b = none ? 0 : q / K, k = none ? 0 : q - b * K;
    const __amdgpu_buffer_rsrc_t rs = row_buffer(stat_row(p, b, row_index(k, none ? 0 : r)), none ? 0u : row_bytes);
#pragma unroll
    for (int t = 0; t < kTilesPerSlice; ++t)
      v[t] = stream_load16(rs, tid * 16u, static_cast<uint32_t>(x * kSliceChunks + t * kThreads) * 16u);
  };
  // The previous row slice's terms wait in registers until its row's normaliser
  // is known: the other members' words of that row are loaded at the start of
  // the next step and used after that step's own statistics pass, so the
  // exchange between the members overlaps work.
  int pq = -1, pr = 0;
  float pkl = 0.0f;
  // finish the previous row slice (terms in `ep`) once its row is known
  auto finish_prev = [&](const RowStats& rs, const float (&ep)[kTilesPerSlice][8]) {
    const int b = pq / K, k = pq - b * K;
    const float sc = lane_scale(pkl, rs);
    if (pr == 0) {  // the target's terms become probabilities
#pragma unroll
      for (int j = 0; j < kTilesPerSlice * 2; ++j) {
        float4 a = GL.pt[j][tid];
        a.x *= sc;
        a.y *= sc;
        a.z *= sc;
        a.w *= sc;
        GL.pt[j][tid] = a;
      }
      return;
    }
    double gs = 0.0;
    // the next tile's terms are read before this tile's are used, so that two
    // tiles' reads are in flight rather than one
    float4 na = GL.pt[0][tid], nb = GL.pt[1][tid];
#pragma unroll
    for (int t = 0; t < kTilesPerSlice; ++t) {
      const float4 a = na, b = nb;
      if (t + 1 < kTilesPerSlice) {
        na = GL.pt[2 * t + 2][tid];
        nb = GL.pt[2 * t + 3][tid];
      }
      const float pt8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float mn[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) mn[i] = min_nonneg(pt8[i], ep[t][i] * sc);
      gs += static_cast<double>(((mn[0] + mn[1]) + (mn[2] + mn[3])) + ((mn[4] + mn[5]) + (mn[6] + mn[7])));
    }
    gs = wave_sum(gs);
    if (lane_id() == 0)
      st_agent_u64(p.gpart + ((((static_cast<size_t>(b) * K + k) * N + (pr - 1)) * S + x) * kWaves + wave_id()),
                   pack_f64(gs));
  };
  // job n: reduce its row from `cur` into `ec` while job n + 1's loads go to
  // `nxt`, then finish the previous row slice (terms in `ep`)
  unsigned long long* pw = nullptr;
  int cq, cr;  // the current job (job n)
  bool cpriv;
  auto step = [&](uint4 (&cur)[kTilesPerSlice], uint4 (&nxt)[kTilesPerSlice], float (&ec)[kTilesPerSlice][8],
                  float (&ep)[kTilesPerSlice][8]) {
    const int q = cq, r = cr;
    const bool priv = cpriv;
    int q1, r1;
    bool priv1;
    advance(q1, r1, priv1);
    // the previous row's words first: vmcnt retires in order, so waiting for them
    // later must not also wait for the next slice's loads
    unsigned long long wv[kRowWordsPerLane];
    if (pq >= 0) wave_row_issue(p, pw, wv);
    load(q1, r1, nxt);  // unconditional (no job: a buffer of no bytes), as in static_phase
    if (!FULL) mask_tail(cur, ci0, p.V);
    double sl;
    const float kl = lane_exps(p, cur, ec, sl);
    unsigned long long* words = words_of(q, r, priv);
    publish_slice_stats(words, x, kl, sl);
    if (pq >= 0) finish_prev(wave_row_finish(p, pw, wv), ep);
    if (r == 0) {  // the target's terms wait in LDS for the row's normaliser
#pragma unroll
      for (int t = 0; t < kTilesPerSlice; ++t) {
        GL.pt[2 * t][tid] = make_float4(ec[t][0], ec[t][1], ec[t][2], ec[t][3]);
        GL.pt[2 * t + 1][tid] = make_float4(ec[t][4], ec[t][5], ec[t][6], ec[t][7]);
      }
    }
    pq = q;
    pr = r;
    pkl = kl;
    pw = words;
    cq = q1;
    cr = r1;
    cpriv = priv1;
  };
  uint4 va[kTilesPerSlice], vb[kTilesPerSlice];
  float ea[kTilesPerSlice][8], eb[kTilesPerSlice][8];
  advance(cq, cr, cpriv);  // job 0
  load(cq, cr, va);
  bool last_in_a = true;
  int n = 0;
#pragma unroll 1
  while (true) {
    step(va, vb, ea, eb);
    last_in_a = true;
    if (++n >= njobs) break;
    step(vb, va, eb, ea);
    last_in_a = false;
    if (++n >= njobs) break;
  }
  // the last row slice's terms are in ea or eb, whichever the last step filled
  {
    unsigned long long wv[kRowWordsPerLane];
    wave_row_issue(p, pw, wv);
    const RowStats rs = wave_row_finish(p, pw, wv);
    if (last_in_a)
      finish_prev(rs, ea);
    else
      finish_prev(rs, eb);
  }
  if (prefix) {
    // the slot's private words: every member has read them once it is done; the
    // last member to finish clears them (and its ticket)
    stores_complete();
    __syncthreads();
    if (tid == 0) {
      const int l = ticket(&p.pdone[slot]) == static_cast<uint32_t>(S - 1) ? 1 : 0;
      if (l) st_agent(&p.pdone[slot], 0u);
      GL.last = l;
    }
    __syncthreads();
    if (GL.last)
      for (int q = tid; q < S * kWaves; q += kThreads) st_agent_u64(own_words + q, 0ull);
    __syncthreads();
  }
}

// Slot g / S of the workgroups, member g % S (workgroups beyond the last full slot
// and slots beyond the last group have no group work).
// LEARN: a fused HedgeSpec round, whose slot 0 takes no rows.
template <bool LEARN>
__device__ __forceinline__ void gamma_groups(const Params& p, GammaLds& GL) {
  const int S = p.S, Q = gridDim.x / S, g = blockIdx.x;
  if (g >= Q * S) return;
  const int x = g % S;
  if ((x + 1) * kSliceTok <= p.V)
    gamma_member<true, LEARN>(p, GL, g / S, x);
  else
    gamma_member<false, LEARN>(p, GL, g / S, x);
}


// Estimator step of a sequence: gamma, the estimator and the loss of every drafter,
// positions in chunks whose rows fit the LDS arrays.  LEARN: a fused HedgeSpec
// round (the loss buffer is the learner's input too).
template <bool LEARN>
__device__ __forceinline__ void unit_estimate(const Params& p, int b, Lds& L) {
  const int tid = threadIdx.x, K = p.K, N = p.N;
  const int J = max(1, min(K, kRowCap / (N + 1)));
  const int nw = p.S * kWaves;  // gamma words of a (position, drafter) pair: one per (slice, wave)
  // [NB] Key design 2 (reading: L = 1 + sum_k gamma_k prod_{j<k} a_j) and Key design 3 (f = K + 1 - L)
  double Lh = 1.0, prod = 1.0;
  for (int k0 = 0; k0 < K; k0 += J) {
    const int nk = min(J, K - k0);
    const int npair = nk * N;  // pair tid = (position k0 + tid / N, drafter tid % N)
    const int kl = tid / N, di = tid - kl * N, kk = k0 + kl;
    // the pair's trajectory token and its two logits, issued first so that these
    // loads overlap the words' below
    const bool has_tok = tid < npair && kk < K - 1;
    const int x = has_tok ? p.traj[b * K + kk] : 0;
    const bool x_ok = x >= 0 && x < p.V;
    uint32_t ztb = 0u, zdb = 0u;
    if (has_tok && x_ok) {
      ztb = target_row(p, b, kk)[x];
      zdb = draft_row(p, b, di, kk)[x];
    }
    // gamma words of the chunk's pairs (contiguous: pair by pair, nw each), read by
    // the whole workgroup through LDS, kStage at a time; thread tid < npair sums its
    // pair's words in order
    const unsigned long long* src = p.gpart + (static_cast<size_t>(b) * K + k0) * N * nw;
    const int total = npair * nw;
    double g = 0.0;
    for (int q0 = 0; q0 < total; q0 += kStage) {
      const int nq = min(kStage, total - q0);
      unsigned long long w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = ld_agent_u64(const_cast<unsigned long long*>(src) + q0 + min(tid + e * kThreads, nq - 1));
      bool missing = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = tid + e * kThreads;
        if (q < nq) L.m.stage[q] = w[e];
        missing |= q < nq && w[e] == 0ull;
      }
      if (missing) {  // not yet published (rare): wait for each missing word
        for (int q = tid; q < nq; q += kThreads)
          if (L.m.stage[q] == 0ull) L.m.stage[q] = poll_word(p.flags, const_cast<unsigned long long*>(src) + q0 + q);
      }
      __syncthreads();
      if (tid < npair) {
        const int lo = max(tid * nw, q0), hi = min((tid + 1) * nw, q0 + nq);
        for (int q = lo; q < hi; ++q) g += unpack_f64(L.m.stage[q - q0]);
      }
      __syncthreads();
    }
    if (tid < npair) {
      L.gsum[tid] = g;
      p.gamma[(b * K + kk) * N + di] = static_cast<float>(g);
    }
    // statistics of the chunk's rows: (target kk, drafter 0 kk, ..., drafter N-1 kk)
    merge_rows(p, b, nk * (N + 1),
               [&](int i) {
                 const int k2 = k0 + i / (N + 1), m = i % (N + 1);
                 return m == 0 ? k2 : p.RT + (m - 1) * K + k2;
               },
               L.m);
    // realised-token acceptance a = min(1, pd(x)/pt(x)) at x = traj[kk]
    if (tid < npair) {
      double a = 1.0;
      if (kk < K - 1) {
        if (!x_ok) {
          a = __builtin_nan("");
        } else {
          const RowStats st{L.m.rk[kl * (N + 1)], L.m.rs[kl * (N + 1)]};
          const RowStats sd{L.m.rk[kl * (N + 1) + 1 + di], L.m.rs[kl * (N + 1) + 1 + di]};
          const double ptx = token_prob(__uint_as_float(ztb << 16), p.c, st);
          const double pdx = token_prob(__uint_as_float(zdb << 16), p.c, sd);
          a = ptx > 0.0 ? fmin(1.0, pdx / ptx) : (pdx > 0.0 ? 1.0 : 0.0);
        }
      }
      L.arat[tid] = a;
    }
    __syncthreads();
    if (tid < N) {
      for (int k1 = 0; k1 < nk; ++k1) {
        Lh += L.gsum[k1 * N + tid] * prod;
        prod *= L.arat[k1 * N + tid];
      }
    }
    __syncthreads();
  }
  if (LEARN) {
    // fused HedgeSpec round: the learner reads the previous round's loss from the
    // same buffer; overwrite it only once the learner is done with it (its only
    // reader here: clear the word)
    if (tid == 0) {
      poll_word(p.flags, &p.lrnw[b]);
      st_agent_u64(&p.lrnw[b], 0ull);
    }
    __syncthreads();
  }
  if (tid < N) {
    p.est_len[b * N + tid] = static_cast<float>(Lh);
    p.loss[b * N + tid] = static_cast<float>(static_cast<double>(K + 1) - Lh);
  }
  // every gamma unit of the sequence has published (all were read above): clear them
  unsigned long long* gw = p.gpart + static_cast<size_t>(b) * K * N * p.S * kWaves;
  for (int q = tid; q < K * N * p.S * kWaves; q += kThreads) st_agent_u64(gw + q, 0ull);
  finish_sequence<LEARN>(p, b, false, L);
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool is_draw_unit(const Params& p, int u) { return p.P1 > 0; }

template <bool MULTI, bool LEARN>
__device__ __forceinline__ void run_unit1(const Params& p, int u, int pre_n, Lds& L) {
  const int b = u / p.P1;
  unit_draw<false, MULTI, LEARN>(p, b, u - b * p.P1, pre_n, L);
}

template <bool LEARN>
__device__ __forceinline__ void run_unit2(const Params& p, int v, Lds& L) {
  unit_estimate<LEARN>(p, v / p.P2, L);
}

// The list is dealt in levels, the slowest slot first.  Level l covers slots
// 0..P-1-l for rounds[l] rounds of slices (one per workgroup of those slots and
// round, in workgroup order); after the last level, slot 0 takes the rest of the
// list round-robin.  A slot c >= 1 thus takes the rounds of levels 0..P-1-c.
struct Split {
  int P, C, T0;
  int rounds[kMaxSlots];
};

__host__ __device__ inline Split make_split(int T0, int ncu, int slots, int G) {
  Split sp;
  sp.T0 = T0;
  sp.P = (slots >= 1 && slots <= kMaxSlots && ncu * slots == G) ? slots : 1;
  sp.C = sp.P > 1 ? ncu : G;
  // n[c]: slices of a slot-c workgroup, c >= 1
  // loops over the constant kMaxSlots, fully unrolled: the arrays stay in registers
  int n[kMaxSlots + 1];
#pragma unroll
  for (int c = 0; c <= kMaxSlots; ++c)
    n[c] = c >= 1 && c < sp.P
               ? static_cast<int>(static_cast<int64_t>(sp.T0) * slot_share(sp.P, c) / (static_cast<int64_t>(G) * kShareDen))
               : 0;
#pragma unroll
  for (int l = 0; l < kMaxSlots; ++l) {
    int r = 0;
#pragma unroll
    for (int hi = 1; hi < kMaxSlots; ++hi)
      if (hi == sp.P - 1 - l) r = n[hi] - n[hi + 1];  // the slowest slot of level l is hi
    sp.rounds[l] = r > 0 ? r : 0;
  }
  return sp;
}

// Draft-tree calls: the whole list to the first dispatch slot.  Their statistics
// are the target rows' alone (a few percent of the bytes), and a second-slot
// workgroup that streams none of them starts on the drafter rows' pieces at once
// (measured against the slot-weighted split: hedge_eval_tree 4% and pool21_tree
// 1.4% faster).
__host__ __device__ inline Split tree_split(int T0, int ncu, int slots, int G) {
  Split sp = make_split(T0, ncu, slots, G);
#pragma unroll
  for (int l = 0; l < kMaxSlots; ++l) sp.rounds[l] = 0;
  return sp;
}

// k-th statistics slice of workgroup g (T0 when it has no more).  32-bit
// arithmetic throughout (a 64-bit compare runs on the vector unit and needs
// registers that may still be the destinations of loads in flight): every
// intermediate is below T0 + (k + 1) C, and the launch bounds T0 and callers ask
// for at most a few slices past a workgroup's count.
__host__ __device__ inline int static_slice(const Split& sp, int k, int g) {
  const int c = g / sp.C;
  int base = 0;
#pragma unroll
  for (int l = 0; l + 1 < kMaxSlots; ++l) {
    if (l + 1 >= sp.P) break;
    if (c > sp.P - 1 - l) return sp.T0;
    const int width = (sp.P - l) * sp.C;
    if (k < sp.rounds[l]) return base + k * width + g;
    k -= sp.rounds[l];
    base += sp.rounds[l] * width;
  }
  if (c > 0) return sp.T0;
  const int s = base + k * sp.C + g;
  return s < sp.T0 ? s : sp.T0;
}

// Phase 0: workgroup g streams its statistics slices of the sequence-major slice
// list in order.  kStaticDepth slices are in flight: the loads of the next
// kStaticDepth - 1 slices are outstanding while the current one is reduced.
constexpr int kStaticDepth = 2;

__device__ __forceinline__ void static_phase(const Params& p, int G, int g) {
  const int T0 = p.total0;
  const Split sp = p.mode == MODE_TREE ? tree_split(p.total0, p.ncu, p.slots, G) : make_split(p.total0, p.ncu, p.slots, G);
  auto slice = [&](int k) { return static_slice(sp, k, g); };
  uint4 va[kTilesPerSlice], vb[kTilesPerSlice];
  // Every load is issued unconditionally (a missing slice's loads read a buffer of
  // no bytes): a load behind a branch leaves the join with two possible counts of
  // loads in flight, and the wait for the current slice then also waits for the
  // first loads of the next one.
  int k = 0;
  int sa = slice(0), sb = slice(1);
  SliceLoc la = slice_loc(p, sa), lb{};
  slice_load(p, la, va);
  while (sa < T0) {
    lb = slice_loc(p, sb);
    slice_load(p, lb, vb);
    slice_finish(p, la, va);
    if (sb >= T0) break;
    const int sc = slice(k + 2);
    la = slice_loc(p, sc);
    slice_load(p, la, va);
    slice_finish(p, lb, vb);
    sa = sc;
    sb = slice(k + 3);
    k += 2;
  }
}

// The gamma groups (gamma calls), phase 0 (static_phase), then phase 1 and phase
// 2: units g, g + G, ... of each list.  A draw unit waits for phase-0 words and
// for the totals of its sequence's other draw units, which are less than one
// round of the grid away; a phase-2 unit waits only for earlier phases' words.
// LDS of the units, or of the gamma groups (which run before any unit)
union KernelLds {
  Lds units;
  GammaLds gamma;
};

// MULTI: draw units of several slices (fused calls whose B S exceeds the grid).
// LEARN: fused HedgeSpec rounds (spec_hedgespec_round), an instance of its own so
// that the other gamma calls keep the leaner code; the learner's arguments a are a
// second kernel argument (unused by the other instances), which keeps them out of
// the Params every kernel takes.
template <bool MULTI, bool LEARN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gamma_kernel(Params p,
                                                                                                       CensoredArgs a) {
  __shared__ KernelLds KL;
  Lds& L = KL.units;
  const int G = gridDim.x, g = blockIdx.x;
  const int T1 = p.B * p.P1;
  // the drafted token of this workgroup's first draw unit (position
  // min(threadIdx.x, K - 1)), loaded now so that the unit's decisions do not wait
  // for it (nothing waits for the load here)
  int pre_n = kNoToken;
  if (g < T1 && is_draw_unit(p, g)) pre_n = p.tokens[(g / p.P1) * p.K + min(static_cast<int>(threadIdx.x), p.K - 1)];
  if (LEARN) {
    // slot 0's workgroups (all of the grid's, when it holds one slot) take the
    // learner steps first; their LDS is then handed to the groups
    if (g < (gridDim.x / p.S >= 2 ? p.S : static_cast<int>(gridDim.x))) learner_steps(p, a, L);
    __syncthreads();
  }
  if (p.mode == MODE_GAMMA) gamma_groups<LEARN>(p, KL.gamma);
  static_phase(p, G, g);
  for (int u = g; u < T1; u += G) {
    __syncthreads();
    run_unit1<MULTI, LEARN>(p, u, u == g ? pre_n : kNoToken, L);
  }
  // the estimator units start on the workgroups after the draw units' (workgroup
  // g takes units (g - T1) mod G, + G, ...), so that where the grid has room they
  // run beside the draws rather than after them
  const int T2 = p.B * p.P2;
  for (int v = (g + G - T1 % G) % G; v < T2; v += G) {
    __syncthreads();
    run_unit2<LEARN>(p, v, L);
  }
}

// Verify calls (spec_verify, spec_cactus_verify): phase 0, then the draw units
// g, g + G, ...  It is the gamma kernel without the groups and the estimator, so
// it holds less LDS and fewer registers.
// KL: Cactus gamma* as the exact root of the KL budget (spec_cactus_kl_verify), a
// separate instance so that the other calls keep the leaner code.  MULTI: draw
// units of several slices, for calls whose B S exceeds the grid (an instance of
// its own too: the single-slice code measured 1% slower beside it).
template <bool KL, bool MULTI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void verify_kernel(Params p) {
  __shared__ Lds L;
  const int G = gridDim.x, g = blockIdx.x;
  const int T1 = p.B * p.P1;
  // the drafted token of this workgroup's first draw unit (position
  // min(threadIdx.x, K - 1)), loaded now so that the unit's decisions do not wait
  // for it (nothing waits for the load here)
  int pre_n = kNoToken;
  if (g < T1) pre_n = p.tokens[(g / p.P1) * p.K + min(static_cast<int>(threadIdx.x), p.K - 1)];
  static_phase(p, G, g);
  for (int u = g; u < T1; u += G) {
    __syncthreads();
    const int b = u / p.P1;
    unit_draw<KL, MULTI>(p, b, u - b * p.P1, u == g ? pre_n : kNoToken, L);
  }
}

// ---------------------------------------------------------------------------
// Draft-tree gamma ([NB] Key design 1, the greedy draft-tree case)
// ---------------------------------------------------------------------------
//
// gamma[b][k][i] = sum of pt_k over the topk tokens of drafter i's row k (logit
// descending, ties to the smaller id): the target's probability of landing on one
// of the children drafter i keeps at the node.  Phase 0 streams the target rows
// 0..K-1 for their statistics (static_phase).  A piece unit -- one wave, a piece
// of kPieceTok tokens of drafter i's row k -- streams the piece once and
// publishes its topk best tokens, with wave operations only (no workgroup
// barrier, so the four waves of a workgroup stream independently, the next
// piece's loads in flight while one is ranked).  A merge unit (b, k, i) takes the
// row's topk from its pieces' records, gathers their target logits and sums pt.
// Piece units wait for nothing, merge units only for piece units and phase 0,
// and every workgroup runs its piece units before its merge units, so every
// wait ends.
//
// A token is ranked by one 32-bit key inside a piece, (order-preserving key of
// its bf16 logit) << 16 | (0xffff - its offset in the piece), and by one 64-bit
// record across pieces, key << 32 | (0xffffffff - token id): larger is better,
// and ties of the logit go to the smaller id.  Records are never zero, so each
// one is its own "published" flag, and a piece's record count, min(topk, tokens
// of the piece inside the row), is known to its reader.

constexpr int kMaxTopk = 64;
constexpr int kPieceTok = 64 * kVec * kTilesPerSlice;   // 4096 tokens: 8 loads of 16 bytes per lane
constexpr int kPieceChunks = kPieceTok / kVec;
constexpr int kMaxPieces = kMaxV / kPieceTok;
constexpr int kWaveCand = 512;                          // a piece's candidates held in LDS

constexpr int kWaveRec = 1024;   // records a merge wave gathers in LDS (beyond: the exact pass)
constexpr int kRecPerLane = 8;  // rows with at most 64 x this many records keep them in registers

struct TreeLds {
  uint32_t cand[kWaves][kWaveCand + 16];  // (+16: zeros after the last, for reads of 16 keys)
  uint32_t ranked[kWaves][kMaxTopk];      // a piece's best keys in rank order
  int ncand[kWaves];
  unsigned long long rec[kWaves][kWaveRec];  // a merge wave's records at or above its bound
};

// Order-preserving 16-bit key of a bf16 logit; -0 counts as +0.
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  b = b == 0x8000u ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

// Piece keys of one chunk: token offset off0 + e in the piece, `valid` of its 8
// tokens inside the row (the rest key 0, below every token).
__device__ __forceinline__ void chunk_keys(const uint4 w, int off0, int valid, uint32_t k[8]) {
  const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t b = (h[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    k[e] = e < valid ? (bf16_key(b) << 16) | (0xffffu - static_cast<uint32_t>(off0 + e)) : 0u;
  }
}

// The same key of a bf16 value held as a float (low 16 bits zero), and back.
__device__ __forceinline__ uint32_t float_key16(float f) { return bf16_key(__float_as_uint(f) >> 16); }
__device__ __forceinline__ float key16_float(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
  return __uint_as_float(b << 16);
}

// The kk-th largest (1 <= kk <= 64) of the wave's 16-bit keys, one per lane, by
// radix selection from the top bit: the largest T with at least kk keys >= T.
// Ballots and scalar counts only (no LDS round trip).
__device__ __forceinline__ uint32_t wave_kth_largest16(uint32_t key, int kk) {
  uint32_t T = 0u;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    if (__popcll(__ballot(key >= c)) >= kk) T = c;
  }
  return T;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o)));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}


// The piece's keys at or above `tau` (nonzero), counted over the wave.
__device__ __forceinline__ int wave_count_at_least(const uint4 v[kTilesPerSlice], int base, int V, uint32_t tau) {
  int c = 0;
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    const int off0 = (t * 64 + lane_id()) * kVec;
    uint32_t k[8];
    chunk_keys(v[t], off0, min(max(V - (base + off0), 0), kVec), k);
#pragma unroll
    for (int e = 0; e < 8; ++e) c += (k[e] != 0u && k[e] >= tau) ? 1 : 0;
  }
  return wave_sum_i(c);
}

// Piece x of row (b K + k) N + i: loads of its 4096 tokens (lane l, load t:
// tokens (64 t + l) 8 .. + 8 of the piece).  none: a unit past the last, whose
// loads read a buffer of no bytes (zero, without touching memory); row and x are
// then any valid piece, and only the byte count is a select.
__device__ __forceinline__ void piece_load(const Params& p, int row, int x, bool none, uint4 v[kTilesPerSlice]) {
  const int i = row % p.N, bk = row / p.N, k = bk % p.K, b = bk / p.K;
  const uint32_t row_bytes = none ? 0u : static_cast<uint32_t>((p.V + kVec - 1) / kVec) * 16u;
  const __amdgpu_buffer_rsrc_t dr = row_buffer(draft_row(p, b, i, k), row_bytes);
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t)
    v[t] = stream_load16(dr, lane_id() * 16u, static_cast<uint32_t>(x * kPieceChunks + t * 64) * 16u);
}

// A piece's records, one per lane (lane r: the record of rank r), stored after the
// next piece's loads are issued: loads and stores retire in order, so a store
// issued before them would make the wait for the next piece also wait for it.
// A lane without a record stores past the end of its buffer, which drops it, so
// the store is one unconditional instruction that the waits can count.
struct PieceRecords {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off;
  unsigned long long val;
};
constexpr int kStoreAgent = 16;  // sc1: written through to where other compute units read it

__device__ __forceinline__ PieceRecords no_records(const Params& p) {
  return PieceRecords{row_buffer(p.cand, 0u), 0u, 0ull};
}
__device__ __forceinline__ void store_records(const PieceRecords& r) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 d = {static_cast<uint32_t>(r.val), static_cast<uint32_t>(r.val >> 32)};
  __builtin_amdgcn_raw_buffer_store_b64(d, r.rs, r.off, 0, kStoreAgent);
}

// Piece unit u (one wave): the topk best tokens of the piece (logits in v), as
// records in rank order (returned, to be stored by the caller).  Candidates are
// the tokens whose logit reaches the topk-th best lane maximum (topk lanes, so
// topk tokens, at or above it; lanes with no token inside the row count as -inf,
// which only lowers it).  Their exact 32-bit keys (ties to the smaller id) then
// rank them.  Ranks are counted against values read back from LDS (16-byte
// broadcast reads), not lane by lane.  FULL: every token of the piece lies inside
// the row (all pieces but a row's last, unless V is a multiple of the piece).
template <bool FULL>
__device__ __forceinline__ PieceRecords piece_unit(const Params& p, int row, int x, const uint4 (&v)[kTilesPerSlice],
                                                  TreeLds& L) {
  const int V = p.V, kk = p.topk;
  const int P = (V + kPieceTok - 1) / kPieceTok;
  const int w = wave_id(), lane = lane_id();
  const int base = x * kPieceTok;
  uint32_t* cand = L.cand[w];
  auto valid_of = [&](int off0) { return FULL ? kVec : min(max(V - (base + off0), 0), kVec); };
  // the lane's best logit
  float m = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < kTilesPerSlice; ++t) {
    float z[8];
    unpack8(v[t], z, valid_of((t * 64 + lane) * kVec));
    m = max3f(max3f(z[0], z[1], z[2]), max3f(z[3], z[4], z[5]), max3f(z[6], z[7], m));
  }
  // tau: the topk-th best lane maximum (lanes without a token inside the row hold
  // -inf, which only lowers it), selected on the maxima's exact bf16 keys
  const float tau = key16_float(wave_kth_largest16(float_key16(m), kk));
  int C;
  if (FULL && tau > 0.0f) {
    // Candidates (logit >= tau) element position by element position, on the raw
    // words: one compare per bf16 value gives the wave's mask of lanes holding a
    // candidate there, and nearly every mask is empty.  The high half of a word
    // needs no unpacking: read as a float, the word is its high bf16 value plus
    // less than one bf16 step of that value's size (the low half's bits extend
    // the mantissa), so for tau > 0, a bf16 value itself, it reaches tau exactly
    // when the high value does.  A lane writes its candidate at the running count
    // plus its rank in the mask: no atomics, no LDS round trip.
    C = 0;
    auto put = [&](unsigned long long mask, int t, int e, uint32_t bits) {
      if ((mask >> lane) & 1ull) {
        const int q = C + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                              static_cast<uint32_t>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
        if (q < kWaveCand)
          cand[q] = (bf16_key(bits) << 16) | (0xffffu - static_cast<uint32_t>((t * 64 + lane) * kVec + e));
      }
      C += __popcll(mask);
    };
#pragma unroll
    for (int t = 0; t < kTilesPerSlice; ++t) {
      const uint32_t wd[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned long long mlo = __builtin_amdgcn_ballot_w64(__uint_as_float(wd[d] << 16) >= tau);
        const unsigned long long mhi = __builtin_amdgcn_ballot_w64(__uint_as_float(wd[d]) >= tau);
        if ((mlo | mhi) == 0ull) continue;
        if (mlo != 0ull) put(mlo, t, 2 * d, wd[d] & 0xffffu);
        if (mhi != 0ull) put(mhi, t, 2 * d + 1, wd[d] >> 16);
      }
    }
  } else {
    if (lane == 0) L.ncand[w] = 0;
    wave_lds_sync();
    // candidates (logit >= tau, inside the row) to LDS, with their exact keys; a
    // load without any in the wave costs one ballot
#pragma unroll
    for (int t = 0; t < kTilesPerSlice; ++t) {
      const int off0 = (t * 64 + lane) * kVec;
      const int valid = valid_of(off0);
      float z[8];
      unpack8(v[t], z, 8);
      uint32_t hit = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) hit |= ((FULL || e < valid) && z[e] >= tau) ? (1u << e) : 0u;
      if (__builtin_amdgcn_ballot_w64(hit != 0u) == 0ull) continue;
      const uint4 wv = v[t];
      while (hit != 0u) {
        const int e = __builtin_ctz(hit);
        hit &= hit - 1u;
        // element e's bf16 bits by selects (an index into z would put z in scratch)
        const uint32_t word = e < 4 ? (e < 2 ? wv.x : wv.y) : (e < 6 ? wv.z : wv.w);
        const uint32_t bits = (e & 1) ? (word >> 16) : (word & 0xffffu);
        const int q = atomicAdd(&L.ncand[w], 1);
        if (q < kWaveCand) cand[q] = (bf16_key(bits) << 16) | (0xffffu - static_cast<uint32_t>(off0 + e));
      }
    }
    wave_lds_sync();
    C = L.ncand[w];
  }
  if (C > kWaveCand) {
    // rare: the exact topk-th best key by bisection (C > kWaveCand >= topk keys reach
    // tau), then its candidates again
    uint32_t lo = 0u, hi = 0xffffffffu;
    while (lo < hi) {
      const uint32_t mid = static_cast<uint32_t>((static_cast<uint64_t>(lo) + hi + 1u) / 2u);  // in (lo, hi]
      if (wave_count_at_least(v, base, V, mid) >= kk)
        lo = mid;
      else
        hi = mid - 1u;
    }
    if (lane == 0) L.ncand[w] = 0;
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < kTilesPerSlice; ++t) {
      const int off0 = (t * 64 + lane) * kVec;
      uint32_t kv[8];
      chunk_keys(v[t], off0, valid_of(off0), kv);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kv[e] != 0u && kv[e] >= lo) cand[atomicAdd(&L.ncand[w], 1)] = kv[e];  // exactly topk of them
    }
    wave_lds_sync();
    C = L.ncand[w];
  }
  if (lane < 16) cand[C + lane] = 0u;  // below every key
  wave_lds_sync();
  // rank of each candidate among them; the topk best go to `ranked` in rank order
  // (16 keys per round: four 16-byte broadcast reads issued together)
  for (int q0 = 0; q0 < C; q0 += 64) {
    const int q = q0 + lane;
    const uint32_t me = q < C ? cand[q] : 0u;
    int r = 0;
    for (int j = 0; j < C; j += 16) {
      const uint4 o0 = *reinterpret_cast<const uint4*>(cand + j);
      const uint4 o1 = *reinterpret_cast<const uint4*>(cand + j + 4);
      const uint4 o2 = *reinterpret_cast<const uint4*>(cand + j + 8);
      const uint4 o3 = *reinterpret_cast<const uint4*>(cand + j + 12);
      r += (o0.x > me ? 1 : 0) + (o0.y > me ? 1 : 0) + (o0.z > me ? 1 : 0) + (o0.w > me ? 1 : 0);
      r += (o1.x > me ? 1 : 0) + (o1.y > me ? 1 : 0) + (o1.z > me ? 1 : 0) + (o1.w > me ? 1 : 0);
      r += (o2.x > me ? 1 : 0) + (o2.y > me ? 1 : 0) + (o2.z > me ? 1 : 0) + (o2.w > me ? 1 : 0);
      r += (o3.x > me ? 1 : 0) + (o3.y > me ? 1 : 0) + (o3.z > me ? 1 : 0) + (o3.w > me ? 1 : 0);
    }
    if (q < C && r < kk) L.ranked[w][r] = me;
  }
  wave_lds_sync();
  // lane r: the record of rank r
  const int nrec = min(kk, C);
  const uint32_t me = lane < nrec ? L.ranked[w][lane] : 0u;
  const uint32_t tok = static_cast<uint32_t>(base) + (0xffffu - (me & 0xffffu));
  PieceRecords rec;
  rec.rs = row_buffer(p.cand + (static_cast<size_t>(row) * P + x) * static_cast<size_t>(kk), static_cast<uint32_t>(kk) * 8u);
  rec.off = static_cast<uint32_t>(lane < nrec ? lane : kk) * 8u;
  rec.val = (static_cast<unsigned long long>(me >> 16) << 32) | (0xffffffffu - tok);
  return rec;
}

// Records a piece publishes: min(topk, its tokens inside the row).
__device__ __forceinline__ int piece_records(const Params& p, int x) {
  return min(p.topk, min(kPieceTok, p.V - x * kPieceTok));
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
  const uint32_t h = wave_max_u32(static_cast<uint32_t>(x >> 32));
  const uint32_t l = wave_max_u32(static_cast<uint32_t>(x >> 32) == h ? static_cast<uint32_t>(x) : 0u);
  return (static_cast<unsigned long long>(h) << 32) | l;
}

// Bits of a record that can differ: the 16-bit logit key (bits 32..47) and the
// token id's complement below 2^20 (bits 0..19); bits 20..31 are all ones and
// 48..63 zero in every record of a row of at most 2^20 tokens.
__device__ __forceinline__ int record_bit(int j) { return j < 16 ? 47 - j : 19 - (j - 16); }
constexpr int kRecordBits = 36;

// The kk-th best of a set of distinct records, by radix selection from the top
// bit: the largest T with at least kk records >= T (0 when the set holds at most
// kk).  count_ge(T) counts the set's records >= T over the wave.
template <class CountGe>
__device__ __forceinline__ unsigned long long kth_best_record(int kk, CountGe count_ge) {
  unsigned long long T = 0x00000000fff00000ull;  // the bits every record holds
  if (count_ge(T) <= kk) return 0ull;
#pragma unroll 1
  for (int j = 0; j < kRecordBits; ++j) {
    const unsigned long long c = T | (1ull << record_bit(j));
    if (count_ge(c) >= kk) T = c;
  }
  return T;
}

// Merge unit v = (b K + k) N + i, one wave (no workgroup barrier): the row's topk
// best records over its pieces, and gamma = the target probability of their
// tokens.  A bound at or below the row's topk-th best record is the best topk-th
// record of the pieces with topk records; the records at or above it (1-2 topk on
// these rows) go to LDS, and the exact topk-th best among them is selected bit by
// bit with ballots.  Too many records at or above the bound (ties over many
// pieces) select over all the row's records instead.
__device__ __forceinline__ void tree_merge(const Params& p, int v, TreeLds& L) {
  const int K = p.K, N = p.N, kk = p.topk;
  const int P = (p.V + kPieceTok - 1) / kPieceTok;
  const int bk = v / N, k = bk % K, b = bk / K;
  const int w = wave_id(), lane = lane_id();
  unsigned long long* recs = p.cand + static_cast<size_t>(v) * P * static_cast<size_t>(kk);
  unsigned long long* wrec = L.rec[w];
  // the target row's statistics words, issued first (phase 0)
  unsigned long long* row_words = part_row(p, b, k);
  unsigned long long wv[kRowWordsPerLane];
  wave_row_issue(p, row_words, wv);
  const int nall = P * kk;
  const uint16_t* trow = target_row(p, b, k);
  RowStats st{};
  double s = 0.0;
  auto add_token = [&](unsigned long long r) {
    const uint32_t tok = 0xffffffffu - static_cast<uint32_t>(r);
    if (tok < static_cast<uint32_t>(p.V))
      s += token_prob(bf16_at(trow, static_cast<int>(tok)), p.c, st);
    else
      st_agent(&p.flags[3], 1u);  // not a record of this call: the fault word, never an index
  };
  // a record slot q of the row that its piece writes (piece x = q / kk, rank q % kk)
  auto written = [&](int q) { return q < nall && q - (q / kk) * kk < piece_records(p, q / kk); };
  if (nall <= 64 * kRecPerLane) {
    // every record of the row in registers, loaded together (a slot no piece
    // writes reads slot 0 and counts as none), then the exact topk-th best
    unsigned long long rr[kRecPerLane];
#pragma unroll
    for (int j = 0; j < kRecPerLane; ++j) {
      const int q = j * 64 + lane;
      rr[j] = ld_agent_u64(recs + (written(q) ? q : 0));
    }
#pragma unroll
    for (int j = 0; j < kRecPerLane; ++j) {
      const int q = j * 64 + lane;
      if (!written(q))
        rr[j] = 0ull;
      else if (rr[j] == 0ull)
        rr[j] = poll_word(p.flags, recs + q);
    }
    st = wave_row_finish(p, row_words, wv);
    const int nrl = (nall + 63) / 64;
    const unsigned long long T = kth_best_record(kk, [&](unsigned long long t) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < kRecPerLane; ++j)
        if (j < nrl) c += __popcll(__builtin_amdgcn_ballot_w64(rr[j] != 0ull && rr[j] >= t));
      return c;
    });
#pragma unroll
    for (int j = 0; j < kRecPerLane; ++j)
      if (rr[j] != 0ull && rr[j] >= T) add_token(rr[j]);
  } else {
    // the bound: the best topk-th record of the pieces with topk records
    unsigned long long tw = 0ull;
    for (int x = lane; x < P; x += 64)
      if (piece_records(p, x) == kk) tw = max(tw, poll_word(p.flags, recs + static_cast<size_t>(x) * kk + (kk - 1)));
    tw = wave_max_u64(tw);
    // the records at or above it, compacted to LDS in lane order (every record the
    // pieces write is read)
    int C = 0;
    for (int q0 = 0; q0 < nall; q0 += 64) {
      const int q = q0 + lane;
      unsigned long long r = 0ull;
      if (written(q)) r = poll_word(p.flags, recs + q);
      const bool in = r != 0ull && r >= tw;
      const unsigned long long m = __builtin_amdgcn_ballot_w64(in);
      if (in) {
        const int at = C + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
        if (at < kWaveRec) wrec[at] = r;
      }
      C += __popcll(m);
    }
    st = wave_row_finish(p, row_words, wv);
    if (C <= kWaveRec) {
      wave_lds_sync();
      // the gathered records, up to 16 per lane, in registers for the selection
      constexpr int kPer = kWaveRec / 64;
      unsigned long long g[kPer];
      const int nper = (C + 63) / 64;
#pragma unroll
      for (int j = 0; j < kPer; ++j) g[j] = (j < nper && j * 64 + lane < C) ? wrec[j * 64 + lane] : 0ull;
      const unsigned long long T = kth_best_record(kk, [&](unsigned long long t) {
        int c = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (j < nper) c += __popcll(__builtin_amdgcn_ballot_w64(g[j] >= t));
        return c;
      });
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (j < nper && g[j] != 0ull && g[j] >= T) add_token(g[j]);
    } else {
      // rare: select over every record of the row, read again from memory (each is
      // published: all were read above)
      auto rec_at = [&](int q) -> unsigned long long { return written(q) ? ld_agent_u64(recs + q) : 0ull; };
      const unsigned long long T = kth_best_record(kk, [&](unsigned long long t) {
        int c = 0;
        for (int q0 = 0; q0 < nall; q0 += 64) {
          const unsigned long long r = rec_at(q0 + lane);
          c += __popcll(__builtin_amdgcn_ballot_w64(r != 0ull && r >= t));
        }
        return c;
      });
      for (int q0 = 0; q0 < nall; q0 += 64) {
        const unsigned long long r = rec_at(q0 + lane);
        if (r != 0ull && r >= T) add_token(r);
      }
    }
  }
  s = wave_sum(s);
  if (lane == 0) p.gamma[v] = static_cast<float>(s);
  // every record of the row back to zero
  for (int q = lane; q < nall; q += 64)
    if (written(q)) st_agent_u64(recs + q, 0ull);
  // the last of the row's N merge units clears its statistics words
  stores_complete();
  int last = 0;
  if (lane == 0) {
    last = ticket(&p.done[bk]) == static_cast<uint32_t>(N - 1) ? 1 : 0;
    if (last) st_agent(&p.done[bk], 0u);
  }
  if (__builtin_amdgcn_readfirstlane(last))
    for (int q = lane; q < p.S * kWaves; q += 64) st_agent_u64(row_words + q, 0ull);
}

// Draft-tree calls (spec_tree_gamma): phase 0 over the target rows, then the piece
// units (one per wave at a time), then the merge units g, g + G, ...
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void tree_kernel(Params p) {
  __shared__ TreeLds L;
  const int G = gridDim.x, g = blockIdx.x;
  static_phase(p, G, g);
  // whole-piece units of wave w: u = g kWaves + w, + G kWaves, ... (row u / Pw,
  // piece u % Pw); the next unit's loads are in flight while one is ranked
  const int rows = p.B * p.K * p.N;
  const int Pw = p.V / kPieceTok;  // whole pieces per row
  const int T1 = rows * Pw, GW = G * kWaves;
  uint4 va[kTilesPerSlice], vb[kTilesPerSlice];
  int u = g * kWaves + wave_id();
  PieceRecords rec = no_records(p);
  // (a unit past the last loads the last unit's descriptor with no bytes: no
  // branch around the division, whose join would keep a flag in a register that
  // the in-order load counter then makes wait for the loads in flight)
  auto load_unit = [&](int uu, uint4 (&v)[kTilesPerSlice]) {
    const int uc = min(uu, T1 - 1);
    piece_load(p, uc / Pw, uc % Pw, uu >= T1, v);
  };
  if (T1 > 0) load_unit(u, va);
  while (u < T1) {
    load_unit(u + GW, vb);
    store_records(rec);
    rec = piece_unit<true>(p, u / Pw, u % Pw, va, L);
    u += GW;
    if (u >= T1) break;
    load_unit(u + GW, va);
    store_records(rec);
    rec = piece_unit<true>(p, u / Pw, u % Pw, vb, L);
    u += GW;
  }
  store_records(rec);
  // a row's last piece when V is not a multiple of the piece: one per row
  if (Pw * kPieceTok < p.V) {
    for (int r = g * kWaves + wave_id(); r < rows; r += GW) {
      piece_load(p, r, Pw, false, va);
      store_records(piece_unit<false>(p, r, Pw, va, L));
    }
  }
  // merge units: one per wave, v = g kWaves + w, + G kWaves, ...
  const int T2 = p.B * p.K * p.N;
  for (int v = g * kWaves + wave_id(); v < T2; v += GW) tree_merge(p, v, L);
}

// ---------------------------------------------------------------------------
// NormalHedge ([NH]); one wave per sequence, lane i = drafter i.
// ---------------------------------------------------------------------------
constexpr int kHedgeNewtonSteps = 64;  // most Newton steps for the NormalHedge scale

// One NormalHedge step of a wave, lane i = drafter i (act: i < N): with the loss l
// (already scaled), lhat = sum_i w_i l_i, R_i += lhat - l_i, then the weights
// from [R]+ ([NH]; uniform when every [R_i]+ is 0).  Every lane of the wave must
// call it: the wave sums read all 64 lanes.
__device__ __forceinline__ void normalhedge_step(double& R, double& w, double l, bool act, int N) {
  const double lhat = wave_sum(act ? w * l : 0.0);
  R = act ? R + (lhat - l) : 0.0;
  const double rp = act ? fmax(R, 0.0) : 0.0;
  double M = rp;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmax(M, __shfl_xor(M, m, 64));
  if (M > 0.0) {
    // the scale c > 0 with (1/N) sum exp(rp^2 / 2c) = e, found in s = 1 / (2c):
    // psi(s) = log sum exp(rp^2 s) - log(N e) is a log-sum-exp of lines, so convex and
    // increasing (slope: the exp-weighted mean of rp^2), with psi >= 0 at
    // s = (1 + ln N) / M^2 (c at the bracket's left end M^2 / (2 (1 + ln N))) and
    // psi <= 0 at s = 1 / M^2 (c = M^2 / 2).  Newton steps from the first descend to
    // the root without passing it; once a step is below 1e-8 of s the error left is
    // of the order of its square.  Exponents are taken against M^2 (all <= 0).
    const double M2 = M * M;
    const double lnNe = log(static_cast<double>(N)) + 1.0;
    const double s_lo = 1.0 / M2;
    double sv = lnNe / M2;
    for (int it = 0; it < kHedgeNewtonSteps; ++it) {
      const double q = act ? rp * rp : 0.0;
      const double e = act ? exp((q - M2) * sv) : 0.0;
      const double S = wave_sum(e);
      const double psi = M2 * sv + log(S) - lnNe;
      const double dpsi = wave_sum(q * e) / S;
      if (!(psi > 0.0) || !(dpsi > 0.0)) break;   // at (or, by rounding, past) the root
      const double sn = fmax(sv - psi / dpsi, s_lo);
      if (!(sn < sv)) break;
      const bool done = sv - sn <= 1e-8 * sn;
      sv = sn;
      if (done) break;
    }
    const double cc = 1.0 / (2.0 * sv);
    const double wu = act ? (rp / cc) * exp(rp * rp / (2.0 * cc)) : 0.0;
    const double tot = wave_sum(wu);  // every lane takes part (lanes past N add 0)
    w = act ? wu / tot : 0.0;
  } else {
    w = act ? 1.0 / static_cast<double>(N) : 0.0;
  }
}

// Next drafter of sequence b: inverse CDF of the weights at v[b] (ascending
// drafter index), lane q holding drafter q's weight; every lane runs the same
// loop over shuffled weights, lane 0 stores.  Every lane returns the pick.
__device__ __forceinline__ int hedge_select(double wcur, const float* v, int32_t* sel, int b, int N) {
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
  const int s = pick >= 0 ? pick : last_pos;
  if (lane_id() == 0) sel[b] = s;
  return s;
}

__global__ __launch_bounds__(64) void hedge_kernel(double* R, double* W, const float* loss, const uint8_t* has,
                                                   float scale, const float* v, int32_t* sel, int N) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool act = i < N;
  const int idx = b * N + i;
  double wfinal = act ? W[idx] : 0.0;
  if (has == nullptr || has[b] != 0) {
    double Ri = act ? R[idx] : 0.0;
    const double l = act ? static_cast<double>(loss[idx]) * static_cast<double>(scale) : 0.0;
    normalhedge_step(Ri, wfinal, l, act, N);
    if (act) {
      R[idx] = Ri;
      W[idx] = wfinal;
    }
  }
  if (v != nullptr) hedge_select(wfinal, v, sel, b, N);
}

// [NB] Key design 3's other learner: exponential-weights Hedge.  One step of a
// wave, lane i = drafter i (act: i < N): cumulative loss L_i += l_i (already
// scaled), weights proportional to exp(-eta L_i), taken against min L (which
// leaves them unchanged).  Every lane of the wave must call it.
__device__ __forceinline__ void hedge_exp_step(double& L, double& w, double l, double eta, bool act) {
  L = act ? L + l : 0.0;
  double mn = act ? L : __builtin_inf();
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mn = fmin(mn, __shfl_xor(mn, m, 64));
  const double u = act ? exp(-eta * (L - mn)) : 0.0;
  const double tot = wave_sum(u);
  w = act ? u / tot : 0.0;
}

// One wave per sequence: hedge_exp_step, then the selection as hedge_kernel's.
__global__ __launch_bounds__(64) void hedge_exp_kernel(double* L, double* W, const float* loss, const uint8_t* has,
                                                       float scale, float eta, const float* v, int32_t* sel, int N) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool act = i < N;
  const int idx = b * N + i;
  double wfinal = act ? W[idx] : 0.0;
  if (has == nullptr || has[b] != 0) {
    double Li = act ? L[idx] : 0.0;
    const double l = act ? static_cast<double>(loss[idx]) * static_cast<double>(scale) : 0.0;
    hedge_exp_step(Li, wfinal, l, static_cast<double>(eta), act);
    if (act) {
      L[idx] = Li;
      W[idx] = wfinal;
    }
  }
  if (v != nullptr) hedge_select(wfinal, v, sel, b, N);
}

// [NB] Key design 3's delayed feedback, resident on the device: one wave per
// sequence b, lane i = drafter i.  round[b] counts the calls of sequence b.  A
// call at round t (t = round[b]):
//   1. pushes round t - 1's loss (when t > 0) into ring slot (t - 1) % Q with its
//      usable round t + d (d = delays[(t - 1) B + b], -1: never);
//   2. applies every queued loss usable at t, one NormalHedge step each, in order
//      of (usable round, origin round), and frees their slots;
//   3. draws round t's drafter: sel[b] = inverse CDF of the weights at
//      v[t B + b], also kept in sel_hist[t B + b];
//   4. round[b] = t + 1.
// The same queue and order as the host-side DelayedNormalHedge.  Slots hold the
// scaled loss (fp64) and the usable round (-1: free); the usable rounds are worked
// on in LDS during the call.  Delays of at most Q - 2 rounds keep a slot from
// being reused before its loss is applied (Q >= 2K + 2 covers the note's 2K).
__global__ __launch_bounds__(64) void hedge_queue_kernel(double* R, double* W, double* qloss, int32_t* qdue,
                                                         int32_t* round, const float* loss, const int32_t* delays,
                                                         float scale, const float* v, int32_t* sel, int32_t* sel_hist,
                                                         int B, int N, int Q, int T) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool act = i < N;
  const int idx = b * N + i;
  const int t = round[b];
  if (t >= T) return;  // the schedules are exhausted: nothing more (never reached by a well-formed loop)
  __shared__ int32_t due[kMaxQueue];
  double Ri = act ? R[idx] : 0.0, wi = act ? W[idx] : 0.0;
  int32_t* gdue = qdue + static_cast<size_t>(b) * Q;
  double* ql = qloss + static_cast<size_t>(b) * Q * N;
  for (int q = i; q < Q; q += 64) due[q] = gdue[q];
  __syncthreads();
  // this call's push stays in a register too: reading the slot back from global
  // memory in the same call is not relied on
  int pslot = -1;
  double pushed = 0.0;
  if (t > 0) {
    const int d = delays[(t - 1) * B + b];
    pslot = (t - 1) % Q;
    pushed = act ? static_cast<double>(loss[idx]) * static_cast<double>(scale) : 0.0;
    if (act) ql[pslot * N + i] = pushed;
    if (i == 0) due[pslot] = d >= 0 ? t + d : -1;
  }
  __syncthreads();
  // ready slots, earliest (usable round, origin round) first; origin of slot q is the
  // latest round r <= t - 1 with r % Q == q
  for (;;) {
    int best = -1;
    long long key = 0x7fffffffffffffffLL;
    for (int q = 0; q < Q; ++q) {
      const int u = due[q];
      if (u < 0 || u > t) continue;
      const int origin = (t - 1) - (((t - 1) % Q - q) % Q + Q) % Q;
      const long long k2 = (static_cast<long long>(u) << 32) | static_cast<uint32_t>(origin);
      if (k2 < key) {
        key = k2;
        best = q;
      }
    }
    if (best < 0) break;
    normalhedge_step(Ri, wi, act ? (best == pslot ? pushed : ql[best * N + i]) : 0.0, act, N);
    __syncthreads();
    if (i == 0) due[best] = -1;
    __syncthreads();
  }
  if (act) {
    R[idx] = Ri;
    W[idx] = wi;
  }
  for (int q = i; q < Q; q += 64) gdue[q] = due[q];
  const int pick = hedge_select(wi, v + static_cast<size_t>(t) * B, sel, b, N);
  if (i == 0) {
    sel_hist[static_cast<size_t>(t) * B + b] = pick;
    round[b] = t + 1;
  }
}

// [NB] Key design 3's delay from censoring, resident on the device: round s's
// loss is usable once K more tokens have been verified after round s (each round
// verifies its accepted drafts plus one token).  One wave per sequence b, lane i
// = drafter i; slots hold the scaled loss (fp64) and the tokens verified since
// its round (-1: free).  A call at round t (t = round[b] < T):
//   1. when t > 0, adds round t - 1's accepted_len[b] + 1 tokens (none when it is
//      negative: nothing was verified) to every queued loss;
//   2. applies every queued loss that has reached K tokens, oldest round first
//      (they all become usable now, so this is (usable round, origin) order), one
//      learner step each, and frees their slots;
//   3. when t > 0, queues round t - 1's loss in slot (t - 1) % Q with 0 tokens
//      (a loss still queued there, from round t - 1 - Q, never arrives: only
//      rounds that verified nothing can leave one that long);
//   4. draws round t's drafter (sel[b], sel_hist[t B + b]) and sets round[b] = t + 1.
// The learner is NormalHedge (state: cumulative regret) or exponential-weights
// Hedge with rate eta (state: cumulative loss).
enum : int { LEARNER_NORMALHEDGE = 0, LEARNER_HEDGE = 1 };

// One wave (lane i: drafter i), sequence b: one round of the censoring learner.
// `tok` (LDS, Q entries) holds the queue's counts during the round.  Returns the
// round's drafter (sel[b] as it stands once the schedules are exhausted).
__device__ __forceinline__ int censored_round(const CensoredArgs& a, int b, int32_t* tok) {
  const int i = lane_id();
  const int N = a.N, Q = a.Q, K = a.K;
  const bool act = i < N;
  const int idx = b * N + i;
  const int t = a.round[b];
  if (t >= a.T) return a.sel[b];  // the schedules are exhausted: nothing more
  double Si = act ? a.S[idx] : 0.0, wi = act ? a.W[idx] : 0.0;
  int32_t* gtok = a.qtok + static_cast<size_t>(b) * Q;
  double* ql = a.qloss + static_cast<size_t>(b) * Q * N;
  const int add = t > 0 && a.alen[b] >= 0 ? a.alen[b] + 1 : 0;
  for (int q = i; q < Q; q += 64) {
    const int32_t c = gtok[q];
    tok[q] = c >= 0 ? min(c + add, K) : -1;  // counts stop at K: reaching it is all that matters
  }
  wave_lds_sync();
  if (t > 0) {
    // queued slots hold rounds t - 1 - Q .. t - 2; slot q holds the latest r <= t - 2 with r % Q == q
    const int newest = ((t - 2) % Q + Q) % Q;  // slot of round t - 2 (when t = 1 nothing is queued)
    for (;;) {
      int best = -1, best_age = -1;
      for (int q = 0; q < Q; ++q) {
        if (tok[q] < K) continue;
        const int age = ((newest - q) % Q + Q) % Q;  // rounds before t - 2
        if (age > best_age) {
          best_age = age;
          best = q;
        }
      }
      if (best < 0) break;
      const double l = act ? ql[best * N + i] : 0.0;
      if (a.learner == LEARNER_NORMALHEDGE)
        normalhedge_step(Si, wi, l, act, N);
      else
        hedge_exp_step(Si, wi, l, static_cast<double>(a.eta), act);
      wave_lds_sync();
      if (i == 0) tok[best] = -1;
      wave_lds_sync();
    }
    const int pslot = (t - 1) % Q;
    if (act) ql[pslot * N + i] = static_cast<double>(a.loss[idx]) * static_cast<double>(a.scale);
    if (i == 0) tok[pslot] = 0;
    wave_lds_sync();
  }
  if (act) {
    a.S[idx] = Si;
    a.W[idx] = wi;
  }
  for (int q = i; q < Q; q += 64) gtok[q] = tok[q];
  const int pick = hedge_select(wi, a.v + static_cast<size_t>(t) * a.B, a.sel, b, N);
  if (i == 0) {
    a.sel_hist[static_cast<size_t>(t) * a.B + b] = pick;
    a.round[b] = t + 1;
  }
  return pick;
}

__global__ __launch_bounds__(64) void hedge_censored_kernel(CensoredArgs a) {
  __shared__ int32_t tok[kMaxQueue];
  censored_round(a, blockIdx.x, tok);
}

// [NB] Key design 3's acceptance-probability loss of a chunk: the sum over its K
// positions of 1 - gamma (fp64), per sequence and drafter.
__global__ void acceptance_loss_kernel(const float* gamma, float* loss, int B, int K, int N) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * N) return;
  const int b = idx / N, i = idx - b * N;
  double s = 0.0;
  for (int k = 0; k < K; ++k) s += 1.0 - static_cast<double>(gamma[(static_cast<size_t>(b) * K + k) * N + i]);
  loss[idx] = static_cast<float>(s);
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
  int topk;  // draft-tree calls
  int R, RT, S, nsub, P1, P2, nlast;
  int64_t RS, total0, ngroups;  // checked below 2^31 before a launch
};

static Shape make_shape(int B, int K, int N, int V, int mode, int fused) {
  Shape s;
  s.B = B;
  s.K = K;
  s.N = N;
  s.V = V;
  s.mode = mode;
  s.fused = fused;
  s.topk = 0;
  // statistics rows: the target rows 0..K-1 and the drafters' rows; the bonus row K
  // (needed only when every draft is accepted) is read by the draw units of such
  // a sequence alone
  s.RT = K;
  s.R = s.RT + N * K;
  if (mode == MODE_TREE) s.R = s.RT = K;  // the statistics list holds the target rows only
  s.S = (V + kSliceTok - 1) / kSliceTok;
  s.nsub = (V + kSub - 1) / kSub;
  s.P1 = mode == MODE_VERIFY || fused ? s.S : 0;
  s.P2 = mode == MODE_VERIFY ? 0 : 1;
  s.nlast = mode == MODE_VERIFY ? 0 : s.P1 + s.P2;
  if (mode == MODE_TREE) {
    s.P1 = s.P2 = 0;
    s.nlast = N;  // merge units per target row (tickets per row)
  }
  s.RS = static_cast<int64_t>(s.R) * s.S;
  // gamma calls: the groups take every statistics row, so the list is empty
  s.total0 = mode == MODE_VERIFY ? static_cast<int64_t>(B) * s.RS : 0;
  s.ngroups = mode == MODE_VERIFY ? 0 : static_cast<int64_t>(B) * K;
  if (mode == MODE_TREE) {
    s.total0 = static_cast<int64_t>(B) * s.RS;
    s.ngroups = 0;
  }
  return s;
}

// Byte offsets of the workspace regions.  They depend on (B, K, N, mode) only
// (every region is sized for the longest row), so one workspace serves every V.
struct WsLayout {
  size_t flags, done, part, tot, gpart, cand, pstat, pdone, selw, lrnw, total;
};

// Most workgroups of a gamma call (its slots' private words are sized for it).
constexpr int kMaxGrid = 4096;

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static WsLayout ws_layout(const Shape& s) {
  WsLayout L;
  const size_t B = static_cast<size_t>(s.B);
  size_t o = 0;
  L.flags = o;
  o = align256(o + 16);
  L.done = o;
  o = align256(o + 4 * B * (s.mode == MODE_TREE ? static_cast<size_t>(s.K) : 1));  // tree: a ticket per target row
  L.part = o;
  o = align256(o + 8 * B * static_cast<size_t>(s.R) * kMaxSlices * kWaves);
  L.tot = o;
  o = align256(o + 8 * B * static_cast<size_t>(kMaxSlices) * kMaxSlices);
  L.gpart = o;
  o = align256(o + (s.mode == MODE_GAMMA ? 8 * B * static_cast<size_t>(s.K) * s.N * kMaxSlices * kWaves : 0));
  L.cand = o;
  // draft-tree records: sized by the call's V (a workspace for V serves every smaller V)
  o = align256(o + (s.mode == MODE_TREE ? 8 * B * static_cast<size_t>(s.K) * s.N * ((s.V + kPieceTok - 1) / kPieceTok) * s.topk : 0));
  // gamma calls: a slot's private statistics words and its ticket (at most one
  // word per wave of the grid)
  L.pstat = o;
  o = align256(o + (s.mode == MODE_GAMMA ? 8 * static_cast<size_t>(kMaxGrid) * kWaves : 0));
  L.pdone = o;
  o = align256(o + (s.mode == MODE_GAMMA ? 4 * static_cast<size_t>(kMaxGrid) : 0));
  // fused HedgeSpec rounds: each sequence's drafter word and learner word
  L.selw = o;
  o = align256(o + (s.mode == MODE_GAMMA ? 8 * B : 0));
  L.lrnw = o;
  o = align256(o + (s.mode == MODE_GAMMA ? 8 * B : 0));
  L.total = o;
  return L;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool stride_ok(int64_t s, int V) { return s >= V && (s % 8) == 0; }

static int bind_workspace(Params& p, const Shape& s, void* ws, size_t bytes) {
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return SPEC_ERR_WORKSPACE;
  const WsLayout L = ws_layout(s);
  if (bytes < L.total) return SPEC_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  p.flags = reinterpret_cast<uint32_t*>(base + L.flags);
  p.done = reinterpret_cast<uint32_t*>(base + L.done);
  p.part = reinterpret_cast<unsigned long long*>(base + L.part);
  p.tot = reinterpret_cast<unsigned long long*>(base + L.tot);
  p.gpart = reinterpret_cast<unsigned long long*>(base + L.gpart);
  p.cand = reinterpret_cast<unsigned long long*>(base + L.cand);
  p.pstat = reinterpret_cast<unsigned long long*>(base + L.pstat);
  p.pdone = reinterpret_cast<uint32_t*>(base + L.pdone);
  // the learner's words: gamma calls only (a verify or draft-tree layout has no room
  // for them, and a null selw tells the kernels there is no learner)
  p.selw = s.mode == MODE_GAMMA ? reinterpret_cast<unsigned long long*>(base + L.selw) : nullptr;
  p.lrnw = s.mode == MODE_GAMMA ? reinterpret_cast<unsigned long long*>(base + L.lrnw) : nullptr;
  return SPEC_OK;
}

// Resident workgroups the device holds (memoised per device: a device property, not call state).
// Compute units of the current device (memoised per device).
static int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev] = ncu;
  return ncu;
}

template <class Kernel>
static int resident_workgroups(Kernel kernel, int which) {
  static int cache[10][64] = {{0}};  // [which kernel][device]
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[which][dev] > 0) return cache[which][dev];
  int ncu = 0, per = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, 0) != hipSuccess) return 0;
  const int g = ncu * (per > 0 ? per : 1);
  if (dev >= 0 && dev < 64) cache[which][dev] = g;
  return g;
}

static void plan_units(Params& p, const Shape& s) {
  p.R = s.R;
  p.RT = s.RT;
  p.S = s.S;
  p.nsub = s.nsub;
  p.P1 = s.P1;
  p.P2 = s.P2;
  p.nlast = s.nlast;
  p.RS = static_cast<int>(s.RS);
  p.total0 = static_cast<int>(s.total0);
  p.ngroups = static_cast<int>(s.ngroups);
}

// lrn: the learner of a fused HedgeSpec round (gamma calls), else nullptr.
static int launch_flow(Params& p, const Shape& s, hipStream_t stream, const CensoredArgs* lrn = nullptr) {
  // a slice is 32 KB of logits, so 2^31 slices exceed any device's memory; the
  // limit keeps the schedule in 32-bit arithmetic (with room for j * G + g)
  if (s.total0 > 0x3fffffffLL || static_cast<int64_t>(s.B) * s.P1 > 0x3fffffffLL || s.ngroups > 0x3fffffffLL ||
      static_cast<int64_t>(s.B) * s.K * s.N * ((s.V + kPieceTok - 1) / kPieceTok) > 0x1fffffffLL)
    return SPEC_ERR_SHAPE;
  const bool verify = s.mode == MODE_VERIFY;
  const bool tree = s.mode == MODE_TREE;
  int grid = tree     ? resident_workgroups(tree_kernel, 3)
             : verify ? (p.kl_exact ? resident_workgroups(verify_kernel<true, false>, 2)
                                    : resident_workgroups(verify_kernel<false, false>, 0))
                      : (lrn ? resident_workgroups(gamma_kernel<false, true>, 7)
                                     : resident_workgroups(gamma_kernel<false>, 1));
  if (grid <= 0) return SPEC_ERR_HIP;
  const int ncu = compute_units();
  const int slots = ncu > 0 && grid % ncu == 0 ? grid / ncu : 1;
  int64_t want = s.total0;
  // gamma calls: a slot of S workgroups per row chunk, up to one chunk per row
  if (s.ngroups * (s.N + 1) * s.S > want) want = s.ngroups * (s.N + 1) * s.S;
  if (static_cast<int64_t>(s.B) * s.P1 > want) want = static_cast<int64_t>(s.B) * s.P1;
  if (static_cast<int64_t>(s.B) * s.P2 > want) want = static_cast<int64_t>(s.B) * s.P2;
  // piece units, four per workgroup at a time
  const int64_t tree_units = tree ? (static_cast<int64_t>(s.B) * s.K * s.N * ((s.V + kPieceTok - 1) / kPieceTok) + 3) / 4 : 0;
  if (tree_units > want) want = tree_units;
  if (grid > want) grid = static_cast<int>(want);
  // every workgroup is resident at once (the schedule's waits rely on it); a gamma
  // slot needs S workgroups at once
  if (s.mode == MODE_GAMMA && grid < s.S) return SPEC_ERR_SHAPE;
  if (grid > kMaxGrid) grid = kMaxGrid;  // the workspace's per-workgroup regions are sized for it
  plan_units(p, s);
  // draw units: one per slice of a sequence when the grid holds them all; else as
  // many per sequence as the grid holds (each taking several slices), so that no
  // workgroup runs a second draw unit after its first
  const bool multi = s.P1 > 0 && static_cast<int64_t>(s.B) * s.P1 > grid;
  if (multi) {
    // the instance with units of several slices holds as many workgroups
    const int g2 = verify ? (p.kl_exact ? resident_workgroups(verify_kernel<true, true>, 6)
                                        : resident_workgroups(verify_kernel<false, true>, 4))
                          : (lrn ? resident_workgroups(gamma_kernel<true, true>, 8)
                                         : resident_workgroups(gamma_kernel<true>, 5));
    if (g2 <= 0) return SPEC_ERR_HIP;
    if (g2 < grid) grid = g2;
    if (s.mode == MODE_GAMMA && grid < s.S) return SPEC_ERR_SHAPE;
    p.P1 = grid / s.B > 1 ? grid / s.B : 1;
    if (p.P1 > s.P1) p.P1 = s.P1;
    if (s.mode != MODE_VERIFY) p.nlast = p.P1 + p.P2;
  }
  p.ncu = ncu;
  p.slots = slots;  // make_split weights the slots only when the grid is all of them
  if (s.mode == MODE_GAMMA) {
    void (*kernel)(Params, CensoredArgs) = lrn ? (multi ? gamma_kernel<true, true> : gamma_kernel<false, true>)
                                               : (multi ? gamma_kernel<true> : gamma_kernel<false>);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, p, lrn ? *lrn : CensoredArgs{});
  } else {
    void (*kernel)(Params) = tree                  ? tree_kernel
                             : verify && p.kl_exact ? (multi ? verify_kernel<true, true> : verify_kernel<true, false>)
                                                    : (multi ? verify_kernel<false, true> : verify_kernel<false, false>);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  }
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
                         int kl_exact, float T, int32_t* A, int32_t* tok, uint8_t* mask, float* gstar, void* ws,
                         size_t wsb, hipStream_t stream) {
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
  p.kl_exact = kl_exact;
  p.mode = MODE_VERIFY;
  p.accepted_len = A;
  p.out_token = tok;
  p.accept_mask = mask;
  p.gamma_star = gstar;
  return launch_flow(p, s, stream);
}

// The workspace of spec_verify_noalloc: a device array of the library, one copy
// per device, zero when the code object is loaded.  Host code never passes its
// name to a kernel (on the host it is only a stand-in for the symbol); each
// device's address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocBytes = static_cast<size_t>(SPEC_NOALLOC_MAX_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[64] = {nullptr};

// This device's copy of `scratch` (nullptr on failure).
static void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
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
    case SPEC_ERR_TOO_LARGE: return "call needs more scratch than SPEC_NOALLOC_MAX_BYTES";
    default: return "unknown status";
  }
}

size_t spec_workspace_bytes(int B, int K, int N) {
  if (B < 1 || K < 1 || N < 1 || K > SPEC_MAX_K || N > SPEC_MAX_N || B > SPEC_MAX_B) return 0;
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
                       V, 0.0, 0, temperature, accepted_len, out_token, accept_mask, nullptr, workspace,
                       workspace_bytes, stream);
}

int spec_verify_noalloc(const spec_bf16* target, int64_t target_row_stride, const spec_bf16* draft,
                        int64_t draft_row_stride, const int32_t* draft_tokens, const float* r_accept,
                        const float* u_resample, int B, int K, int V, float temperature, int32_t* accepted_len,
                        int32_t* out_token, uint8_t* accept_mask, spec_stream_t stream) {
  int st = check_common(B, K, V, temperature);
  if (st != SPEC_OK) return st;
  const size_t need = ws_layout(make_shape(B, K, 1, V, MODE_VERIFY, 0)).total;
  if (need > kNoAllocBytes) return SPEC_ERR_TOO_LARGE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return SPEC_ERR_HIP;
  // clear what this call reads as unpublished: the regions of its layout (a kernel
  // node, never a memset node, so that the call can be captured in a graph)
  const size_t words = need / 4;
  const int grid = static_cast<int>(words / 256 + 1 < 1024 ? words / 256 + 1 : 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(ws), words);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  return verify_common(target, target_row_stride, draft, draft_row_stride, draft_tokens, r_accept, u_resample, B, K,
                       V, 0.0, 0, temperature, accepted_len, out_token, accept_mask, nullptr, ws, need, stream);
}

int spec_cactus_verify(const spec_bf16* verifier, int64_t verifier_row_stride, const spec_bf16* draft,
                       int64_t draft_row_stride, const int32_t* draft_tokens, const float* r_accept,
                       const float* u_resample, int B, int m, int V, float delta, float temperature,
                       int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask, float* gamma_star,
                       void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  if (!(delta >= 0.0f) || !isfinite(delta)) return SPEC_ERR_PARAM;
  return verify_common(verifier, verifier_row_stride, draft, draft_row_stride, draft_tokens, r_accept, u_resample, B,
                       m, V, static_cast<double>(delta), 0, temperature, accepted_len, out_token, accept_mask,
                       gamma_star, workspace, workspace_bytes, stream);
}

int spec_cactus_kl_verify(const spec_bf16* verifier, int64_t verifier_row_stride, const spec_bf16* draft,
                          int64_t draft_row_stride, const int32_t* draft_tokens, const float* r_accept,
                          const float* u_resample, int B, int m, int V, float delta, float temperature,
                          int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask, float* gamma_star,
                          void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  if (!(delta >= 0.0f) || !isfinite(delta)) return SPEC_ERR_PARAM;
  return verify_common(verifier, verifier_row_stride, draft, draft_row_stride, draft_tokens, r_accept, u_resample, B,
                       m, V, static_cast<double>(delta), 1, temperature, accepted_len, out_token, accept_mask,
                       gamma_star, workspace, workspace_bytes, stream);
}

static int gamma_call(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                              const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                              const int32_t* traj_tokens, int B, int K, int N, int V, float temperature, float* gamma,
                              float* est_len, float* loss, const int32_t* sel, const int32_t* draft_tokens,
                              const float* r_accept, const float* u_resample, int32_t* accepted_len,
                              int32_t* out_token, uint8_t* accept_mask, void* workspace, size_t workspace_bytes,
                              spec_stream_t stream, const CensoredArgs* lrn) {
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
  if (lrn == nullptr) p.selw = p.lrnw = nullptr;  // no learner step: the kernel reads neither word
  return launch_flow(p, s, stream, lrn);
}

int spec_counterfactual_gamma(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                              const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                              const int32_t* traj_tokens, int B, int K, int N, int V, float temperature, float* gamma,
                              float* est_len, float* loss, const int32_t* sel, const int32_t* draft_tokens,
                              const float* r_accept, const float* u_resample, int32_t* accepted_len,
                              int32_t* out_token, uint8_t* accept_mask, void* workspace, size_t workspace_bytes,
                              spec_stream_t stream) {
  return gamma_call(target, target_row_stride, target_rows_per_seq, drafts, draft_row_stride, drafter_stride,
                    traj_tokens, B, K, N, V, temperature, gamma, est_len, loss, sel, draft_tokens, r_accept,
                    u_resample, accepted_len, out_token, accept_mask, workspace, workspace_bytes, stream, nullptr);
}

int spec_hedgespec_round(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                         const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                         const int32_t* traj_tokens, int B, int K, int N, int V, float temperature, float* gamma,
                         float* est_len, float* loss, const int32_t* draft_tokens, const float* r_accept,
                         const float* u_resample, int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                         double* state, double* weights, double* queue_loss, int32_t* queue_tokens, int32_t* round,
                         int learner, float eta, float loss_scale, const float* v_select, int32_t* sel,
                         int32_t* sel_hist, int Q, int T, void* workspace, size_t workspace_bytes,
                         spec_stream_t stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_N || K < 1 || K > SPEC_MAX_K || Q < K + 1 || Q > kMaxQueue || T < 1)
    return SPEC_ERR_SHAPE;
  if (!state || !weights || !queue_loss || !queue_tokens || !round || !v_select || !sel || !sel_hist || !accepted_len ||
      !loss)
    return SPEC_ERR_NULL;
  if (learner != SPEC_LEARNER_NORMALHEDGE && learner != SPEC_LEARNER_HEDGE) return SPEC_ERR_PARAM;
  if (!(loss_scale >= 0.0f) || !isfinite(loss_scale) || !(eta >= 0.0f) || !isfinite(eta)) return SPEC_ERR_PARAM;
  const CensoredArgs a{state, weights, queue_loss, queue_tokens, round, loss, accepted_len, K, learner, eta,
                       loss_scale, v_select, sel, sel_hist, B, N, Q, T};
  return gamma_call(target, target_row_stride, target_rows_per_seq, drafts, draft_row_stride, drafter_stride,
                    traj_tokens, B, K, N, V, temperature, gamma, est_len, loss, sel, draft_tokens, r_accept,
                    u_resample, accepted_len, out_token, accept_mask, workspace, workspace_bytes, stream, &a);
}

size_t spec_tree_workspace_bytes(int B, int K, int N, int V, int topk) {
  if (B < 1 || K < 1 || N < 1 || K > SPEC_MAX_K || N > SPEC_MAX_N || B > SPEC_MAX_B || topk < 1 || topk > kMaxTopk ||
      V < 1 || V > SPEC_MAX_V)
    return 0;
  Shape sh = make_shape(B, K, N, V, MODE_TREE, 0);
  sh.topk = topk;
  return ws_layout(sh).total;
}

int spec_tree_gamma(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                    const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride, int B, int K, int N,
                    int V, int topk, float temperature, float* gamma, void* workspace, size_t workspace_bytes,
                    spec_stream_t stream) {
  int st = check_common(B, K, V, temperature);
  if (st != SPEC_OK) return st;
  if (N < 1 || N > SPEC_MAX_N) return SPEC_ERR_SHAPE;
  if (topk < 1 || topk > kMaxTopk) return SPEC_ERR_PARAM;
  if (!target || !drafts || !gamma) return SPEC_ERR_NULL;
  if (target_rows_per_seq < K) return SPEC_ERR_SHAPE;
  if (!stride_ok(target_row_stride, V) || !stride_ok(draft_row_stride, V)) return SPEC_ERR_SHAPE;
  if (drafter_stride < 0 || (drafter_stride % 8) != 0 || (N > 1 && drafter_stride == 0)) return SPEC_ERR_SHAPE;
  if (!aligned16(target) || !aligned16(drafts)) return SPEC_ERR_ALIGN;
  Shape s = make_shape(B, K, N, V, MODE_TREE, 0);
  s.topk = topk;
  Params p{};
  st = bind_workspace(p, s, workspace, workspace_bytes);
  if (st != SPEC_OK) return st;
  p.target = target;
  p.t_stride = target_row_stride;
  p.t_rows = target_rows_per_seq;
  p.draft = drafts;
  p.d_stride = draft_row_stride;
  p.drafter_stride = drafter_stride;
  p.B = B;
  p.K = K;
  p.N = N;
  p.V = V;
  p.c = log2e_over(temperature);
  p.mode = MODE_TREE;
  p.topk = topk;
  p.gamma = gamma;
  return launch_flow(p, s, stream);
}

int hedge_exp_update(double* cum_loss, double* weights, const float* loss, const uint8_t* has_loss, float loss_scale,
                     float eta, const float* v_select, int32_t* sel_out, int B, int N, spec_stream_t stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_N) return SPEC_ERR_SHAPE;
  if (!cum_loss || !weights || !loss) return SPEC_ERR_NULL;
  if (v_select && !sel_out) return SPEC_ERR_NULL;
  if (!(loss_scale >= 0.0f) || !isfinite(loss_scale) || !(eta >= 0.0f) || !isfinite(eta)) return SPEC_ERR_PARAM;
  hipLaunchKernelGGL(hedge_exp_kernel, dim3(B), dim3(64), 0, stream, cum_loss, weights, loss, has_loss, loss_scale, eta,
                     v_select, sel_out, N);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int hedge_queue_update(double* cum_regret, double* weights, double* queue_loss, int32_t* queue_due, int32_t* round,
                       const float* loss, const int32_t* delays, float loss_scale, const float* v_select,
                       int32_t* sel_out, int32_t* sel_hist, int B, int N, int Q, int T, spec_stream_t stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_N || Q < 2 || Q > kMaxQueue || T < 1) return SPEC_ERR_SHAPE;
  if (!cum_regret || !weights || !queue_loss || !queue_due || !round || !loss || !delays || !v_select || !sel_out ||
      !sel_hist)
    return SPEC_ERR_NULL;
  if (!(loss_scale >= 0.0f) || !isfinite(loss_scale)) return SPEC_ERR_PARAM;
  hipLaunchKernelGGL(hedge_queue_kernel, dim3(B), dim3(64), 0, stream, cum_regret, weights, queue_loss, queue_due,
                     round, loss, delays, loss_scale, v_select, sel_out, sel_hist, B, N, Q, T);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int hedge_censored_update(double* state, double* weights, double* queue_loss, int32_t* queue_tokens, int32_t* round,
                          const float* loss, const int32_t* accepted_len, int K, int learner, float eta,
                          float loss_scale, const float* v_select, int32_t* sel_out, int32_t* sel_hist, int B, int N,
                          int Q, int T, spec_stream_t stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_N || K < 1 || K > SPEC_MAX_K || Q < K + 1 || Q > kMaxQueue || T < 1)
    return SPEC_ERR_SHAPE;
  if (!state || !weights || !queue_loss || !queue_tokens || !round || !loss || !accepted_len || !v_select || !sel_out ||
      !sel_hist)
    return SPEC_ERR_NULL;
  if (learner != SPEC_LEARNER_NORMALHEDGE && learner != SPEC_LEARNER_HEDGE) return SPEC_ERR_PARAM;
  if (!(loss_scale >= 0.0f) || !isfinite(loss_scale) || !(eta >= 0.0f) || !isfinite(eta)) return SPEC_ERR_PARAM;
  const CensoredArgs a{state, weights, queue_loss, queue_tokens, round, loss, accepted_len, K, learner, eta,
                       loss_scale, v_select, sel_out, sel_hist, B, N, Q, T};
  hipLaunchKernelGGL(hedge_censored_kernel, dim3(B), dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_acceptance_loss(const float* gamma, float* loss, int B, int K, int N, spec_stream_t stream) {
  if (B < 1 || K < 1 || N < 1 || B > SPEC_MAX_B || K > SPEC_MAX_K || N > SPEC_MAX_N) return SPEC_ERR_SHAPE;
  if (!gamma || !loss) return SPEC_ERR_NULL;
  const int n = B * N;
  hipLaunchKernelGGL(acceptance_loss_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, gamma, loss, B, K, N);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
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
