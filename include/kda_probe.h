/*
 * kda_probe.h -- HBM stream probes exported by libkda.so (measurement only).
 *
 * Plain read, write and copy kernels over a device buffer. The grid-stride
 * ones use the same 16-byte non-temporal accesses the core kernel uses for its
 * state stream and serve as kernels of exactly known traffic for calibrating
 * the HBM byte counters (FETCH_SIZE, WRITE_SIZE). The _runs variants give each
 * workgroup one contiguous run with plain stores, the fastest write shape
 * measured; with the read probe they give the achievable HBM bandwidth on the
 * machine at hand. None of them is part of the KDA method.
 *
 * All pointers are device pointers, 16-byte aligned; `bytes` is a positive
 * multiple of 16. Calls are asynchronous on `hip_stream`. Return values are
 * kda_status codes (include/kda.h): KDA_OK, KDA_ERR_NULL, KDA_ERR_ALIGN
 * (pointer or size), KDA_ERR_HIP. Nothing is enqueued on error.
 */
#ifndef KDA_PROBE_H
#define KDA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i] for `bytes` bytes (reads and writes `bytes` each). */
int kda_probe_copy(void* dst, const void* src, int64_t bytes, void* hip_stream);

/* Fills `bytes` bytes of dst with the fp32 value `value` (writes only). */
int kda_probe_write(void* dst, int64_t bytes, float value, void* hip_stream);

/* kda_probe_copy and kda_probe_write over one contiguous run per workgroup
 * (4096 workgroups), plain stores. */
int kda_probe_copy_runs(void* dst, const void* src, int64_t bytes, void* hip_stream);
int kda_probe_write_runs(void* dst, int64_t bytes, float value, void* hip_stream);

/* Reads `bytes` bytes of src; writes one fp32 partial sum per workgroup to
 * sink (sink holds at least kda_probe_sink_floats() floats). */
int kda_probe_read(const void* src, int64_t bytes, float* sink, void* hip_stream);

/* Number of floats kda_probe_read writes to its sink. */
int32_t kda_probe_sink_floats(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H */
