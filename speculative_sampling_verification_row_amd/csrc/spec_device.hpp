// Device building blocks for full-vocabulary speculative-sampling verification
// on gfx950 (CDNA4, wave64).
//
// Rows are bf16 logits streamed with 128-bit loads: a workgroup of kThreads
// lanes covers a tile of kTile = kThreads * 8 consecutive tokens per load
// instruction, lane t of the tile owning tokens [8t, 8t + 8).  Wave w's share of
// a tile is a "sub-tile" of 512 consecutive tokens, so tile order, then wave,
// then lane, then element is ascending token order -- the order of every
// cumulative sum used by the inverse-CDF draws.
//
// Softmax statistics are kept in base 2.  Each lane carries an integer-valued
// float reference k and an fp64 sum s of 2^(z*c - k), c = log2(e) / T.  When a
// larger logit arrives, k moves up to ceil(z*c) and s is rescaled by an exact
// power of two (ldexp), so the running reference never adds rounding error.
// Each term is exp2 of one fused multiply-add, evaluated in fp32; sums of eight
// terms are formed in fp32 and accumulated in fp64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;             // lanes per workgroup
constexpr int kWaves = kThreads / 64;     // wave64
constexpr int kVec = 8;                   // bf16 per 16-byte load
constexpr int kTile = kThreads * kVec;    // tokens per tile
constexpr int kSub = 64 * kVec;           // tokens per wave sub-tile
constexpr int kUnroll = 4;                // tiles in flight per row
constexpr int kMaxV = 1 << 20;
constexpr int kMaxSub = kMaxV / kSub;     // sub-tiles per row at most
constexpr float kNoRef = -1.0e30f;        // initial reference: "no finite logit seen"

struct RowAcc {
  float k;   // integer-valued reference exponent (base 2)
  double s;  // sum of 2^(z*c - k)
};

__device__ __forceinline__ RowAcc row_acc_init() { return RowAcc{kNoRef, 0.0}; }

// Eight bf16 (one 16-byte chunk) -> fp32, ascending token order.  Tokens at or
// beyond `valid` (< 8 only in a row's last chunk) become -inf.
__device__ __forceinline__ void unpack8(const uint4 v, float z[8], int valid) {
  z[0] = __uint_as_float(v.x << 16);
  z[1] = __uint_as_float(v.x & 0xffff0000u);
  z[2] = __uint_as_float(v.y << 16);
  z[3] = __uint_as_float(v.y & 0xffff0000u);
  z[4] = __uint_as_float(v.z << 16);
  z[5] = __uint_as_float(v.z & 0xffff0000u);
  z[6] = __uint_as_float(v.w << 16);
  z[7] = __uint_as_float(v.w & 0xffff0000u);
  if (valid < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= valid) z[e] = -__builtin_inff();
  }
}

// Raw buffer access to a row: the descriptor covers `bytes` bytes from `base`,
// and a load past them reads zero.  A load names its address as a per-lane byte
// offset plus a wave-uniform one, so eight loads of a lane share one address
// register.  Word 3 of the descriptor is the gfx9 raw-buffer format (32-bit
// data format, no swizzle, no index stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t uniform_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(lane_off), static_cast<int>(uniform_off), 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Streaming loads (every logit is read once): the non-temporal cache policy
// (bit 1 of the buffer instruction's cache-policy operand), which streams 5 %
// faster than the default on MI355X (measured with the streaming-read probe).
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ uint4 stream_load16(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t uniform_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(lane_off), static_cast<int>(uniform_off),
                                                       kStreamPolicy);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// min of two floats known to be >= +0 (not NaN): their bit patterns order as
// unsigned integers, so one integer min does it (fminf would first quiet each
// operand read from memory, one more instruction per operand).
__device__ __forceinline__ float min_nonneg(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}

__device__ __forceinline__ float bf16_at(const uint16_t* row, int idx) {
  return __uint_as_float(static_cast<uint32_t>(row[idx]) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold eight logits into a lane accumulator.
__device__ __forceinline__ void row_acc_add8(RowAcc& a, const float z[8], float c) {
  const float gm = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
  const float kn = fmaxf(a.k, ceilf(gm * c));
  a.s = ldexp(a.s, static_cast<int>(fmaxf(a.k - kn, -2000.0f)));
  a.k = kn;
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fmaf(z[i], c, -kn));
  a.s += static_cast<double>(((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
}

// ---------------------------------------------------------------------------
// Wave / workgroup reductions
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave's index in the workgroup, as a scalar (the compiler cannot tell that
// threadIdx.x >> 6 is the same in every lane of a wave: without readfirstlane,
// addresses derived from it become per-lane values, and a buffer descriptor built
// from them is issued through a loop over the lanes' distinct values).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Cross-lane moves use DPP (data-parallel primitives of the VALU) rather than
// LDS permutes: quad permutations and row mirrors combine lanes within a row of
// 16, row shifts and row broadcasts build prefix sums, and readlane collects the
// four row results.  64-bit values move as two 32-bit halves.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3
constexpr int kDppWaveShr1 = 0x138;    // lane i <- lane i - 1
__host__ __device__ constexpr int dpp_row_shr(int n) { return 0x110 + n; }

// Lane values moved by a DPP control; lanes with no source (or outside the row
// mask) read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL, ROW_MASK>(__float_as_int(v)));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL, ROW_MASK>(static_cast<int>(b));
  const int hi = dpp_i32<CTRL, ROW_MASK>(static_cast<int>(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Maximum over the 64 lanes (every lane gets it).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i32<kDppQuadXor1>(v));
  v = max(v, dpp_i32<kDppQuadXor2>(v));
  v = max(v, dpp_i32<kDppRowHalfMirror>(v));
  v = max(v, dpp_i32<kDppRowMirror>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Maximum and sum over each row of 16 lanes (every lane of the row gets its row's):
// the first four steps of the wave reductions, without the readlanes.
__device__ __forceinline__ int row16_max_i(int v) {
  v = max(v, dpp_i32<kDppQuadXor1>(v));
  v = max(v, dpp_i32<kDppQuadXor2>(v));
  v = max(v, dpp_i32<kDppRowHalfMirror>(v));
  return max(v, dpp_i32<kDppRowMirror>(v));
}
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowHalfMirror>(v);
  return v + dpp_f64<kDppRowMirror>(v);
}

// Sum over the 64 lanes in a fixed order (every lane gets it).
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowHalfMirror>(v);
  v += dpp_f64<kDppRowMirror>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Inclusive prefix sum over the 64 lanes (ascending lane order): Hillis-Steele
// within each row of 16, then the row totals carried across rows.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_f64<dpp_row_shr(1)>(v);
  v += dpp_f64<dpp_row_shr(2)>(v);
  v += dpp_f64<dpp_row_shr(4)>(v);
  v += dpp_f64<dpp_row_shr(8)>(v);
  v += dpp_f64<kDppRowBcast15, 0xa>(v);
  v += dpp_f64<kDppRowBcast31, 0xc>(v);
  return v;
}

// The value of lane i - 1 (0 in lane 0).
__device__ __forceinline__ double lane_prev(double v) { return dpp_f64<kDppWaveShr1>(v); }

struct RowStats {
  float k;       // row reference (max over lanes), integer-valued
  double s;      // sum of 2^(z*c - k) over the row
};

// Combine the lanes' accumulators of one row into the row's (k, s).
// Every lane of the workgroup must call it; `scratch` holds 2 * kWaves doubles.
__device__ __forceinline__ RowStats block_row_stats(const RowAcc a, double* scratch) {
  float km = wave_max(a.k);
  float* kf = reinterpret_cast<float*>(scratch);
  if (lane_id() == 0) kf[wave_id()] = km;
  __syncthreads();
  km = kf[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) km = fmaxf(km, kf[w]);
  __syncthreads();
  double s = ldexp(a.s, static_cast<int>(fmaxf(a.k - km, -2000.0f)));
  s = wave_sum(s);
  if (lane_id() == 0) scratch[wave_id()] = s;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += scratch[w];
  __syncthreads();
  return RowStats{km, tot};
}

// fp64 probability of one token of a row: 2^(z*c - k) / s (z*c is exact in fp64).
__device__ __forceinline__ double token_prob(float z, float c, const RowStats& st) {
  return exp2(static_cast<double>(z) * static_cast<double>(c) - static_cast<double>(st.k)) / st.s;
}

// XCD-aware mapping: the dispatcher hands workgroup x to XCD x % 8.  Give each
// XCD a contiguous block of logical jobs so that jobs that share rows (the N
// drafters of one position share its target row) run under one L2.
__device__ __forceinline__ int logical_job(int x, int G) {
  const int per = G / 8, rem = G % 8;
  const int xcd = x % 8, q = x / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + q;
}

// Cross-workgroup protocol.  Every value one workgroup hands to another is
// written and read with device-scope atomic stores / loads, which the hardware
// keeps coherent across the XCDs' L2 caches without any cache maintenance.  A
// producer waits until its own stores have completed (vmcnt counts stores on
// gfx9, and a device-scope store completes once it is visible device-wide),
// passes a workgroup barrier, then bumps a completion counter with a relaxed
// atomic; a consumer polls that counter with device-scope loads.  No
// agent-scope fence is used: on this target it writes back and invalidates the
// whole L2, which costs far more than the data it protects.
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_i(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent_i(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_d(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent_d(double* p) {
  return __longlong_as_double(static_cast<long long>(
      __hip_atomic_load(reinterpret_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
}
__device__ __forceinline__ void st_agent_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent_u64(unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ticket(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ticket_n(uint32_t* p, uint32_t n) {
  return __hip_atomic_fetch_add(p, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void stores_complete() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace specv
