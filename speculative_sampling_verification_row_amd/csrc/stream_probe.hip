// libstreamprobe: a plain streaming read of device memory with the access pattern
// of the verification kernels' statistics phase, and no arithmetic beyond folding
// the loaded words, so that its bandwidth is the ceiling that phase can reach.
//
// The buffer is cut into slices of kThreads x kLoads x 16 bytes (32 KB).  A
// persistent grid of G workgroups streams slices g, g + G, g + 2G, ... in order,
// each lane issuing kLoads 128-bit buffer loads per slice, with the next slice's
// loads in flight while the current one is folded -- the same two-deep pipeline,
// load width, descriptor-based addressing and non-temporal cache policy as the
// statistics slices.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stream_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 8;
constexpr uint32_t kSliceBytes = kThreads * kLoads * 16u;
constexpr int kPolicy = 2;  // bit 1 of the buffer load's cache-policy operand: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_buffer(const unsigned char* base, uint64_t off,
                                                               uint64_t bytes) {
  // a descriptor of the slice's bytes (none past the buffer's end: such loads read zero)
  const uint64_t left = off < bytes ? bytes - off : 0;
  const uint32_t n = static_cast<uint32_t>(left < kSliceBytes ? left : kSliceBytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base + (off < bytes ? off : 0)), 0,
                                           static_cast<int>(n), 0x00020000);
}

__device__ __forceinline__ void slice_issue(__amdgpu_buffer_rsrc_t r, uint4 v[kLoads]) {
#pragma unroll
  for (int t = 0; t < kLoads; ++t) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(threadIdx.x * 16u),
                                                         static_cast<int>(t * kThreads * 16u), kPolicy);
    v[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ uint32_t fold(const uint4 v[kLoads]) {
  uint32_t a = 0;
#pragma unroll
  for (int t = 0; t < kLoads; ++t) a ^= (v[t].x + v[t].y) ^ (v[t].z + v[t].w);
  return a;
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const unsigned char* buf, uint64_t bytes,
                                                               uint32_t* out) {
  const uint64_t nslices = (bytes + kSliceBytes - 1) / kSliceBytes;
  const uint64_t G = gridDim.x;
  uint64_t j = blockIdx.x;
  uint4 va[kLoads], vb[kLoads];
  uint32_t acc = 0;
  slice_issue(slice_buffer(buf, j * kSliceBytes, bytes), va);
  while (j < nslices) {
    slice_issue(slice_buffer(buf, (j + G) * kSliceBytes, bytes), vb);
    acc ^= fold(va);
    j += G;
    if (j >= nslices) break;
    slice_issue(slice_buffer(buf, (j + G) * kSliceBytes, bytes), va);
    acc ^= fold(vb);
    j += G;
  }
  out[static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int stream_read_probe(const void* buf, uint64_t bytes, uint32_t* out, int grid, stream_probe_stream_t stream) {
  if (buf == nullptr || out == nullptr || bytes == 0 || grid < 1) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (bytes & 15u) != 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(buf), bytes, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
