/*
 * stream_probe.h -- C ABI of libstreamprobe.so, a measurement aid beside
 * libspecverify.so: a plain streaming read of device memory in 32 KB slices with
 * the statistics phase's access pattern (persistent grid, 128-bit buffer loads,
 * two slices in flight per workgroup), folding the words it reads and nothing
 * else.  Its bandwidth is the read ceiling the verification kernels can reach.
 */
#ifndef STREAM_PROBE_H
#define STREAM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* stream_probe_stream_t;

/*
 * Read `bytes` bytes from device buffer `buf` (16-byte aligned, bytes a multiple
 * of 16) with `grid` workgroups of 256 lanes on `stream`; workgroup g streams
 * slices g, g + grid, ...  `out` [grid * 256] uint32 (device) receives each lane's
 * fold of its words (so that the loads are not removed).  Returns 0, -1 for bad
 * arguments (nothing launched), -6 if the launch failed.
 */
int stream_read_probe(const void* buf, uint64_t bytes, uint32_t* out, int grid, stream_probe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_PROBE_H */
