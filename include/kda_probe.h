/*
 * kda_probe.h -- HBM stream probes exported by libkda_probe.so (measurement
 * only; a library of its own, apart from the product library libkda.so).
 *
 * Plain read, write and copy kernels over a device buffer. The grid-stride
 * ones use the same 16-byte non-temporal accesses the core kernel uses for its
 * state stream and serve as kernels of exactly known traffic for calibrating
 * the HBM byte counters (FETCH_SIZE, WRITE_SIZE). The _runs variants give each
 * workgroup one contiguous run with plain stores, the fastest write shape
 * measured; with the read probe they give the achievable HBM bandwidth on the
 * machine at hand. kda_probe_state_stream replays the core kernel's state
 * traffic alone. None of them is part of the KDA method.
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

/* The state traffic of kda_decode / kda_verify alone, for the ceiling of that
 * access pattern: the core kernel's grid (one workgroup per (request, head)
 * with the core's 8 or 16 waves, the same order of units over the XCDs), its
 * lane layout and its load and store flavours, and no other work. Workgroup (r, h) reads
 * the 64 KiB fp32 tile state[src][h] and, for t = 0 .. tokens-1, writes
 * c^(t+1) times it to state[dst[t]][h], c = 0.999f applied once per token in
 * fp32. Slots as in kda_verify: dst[t] = slots[r * slots_row_stride + t],
 * src = dst[accepted[r] - 1], or src = dst[0] when accepted is NULL (the
 * decode case, in place when tokens == 1). A request with a slot outside
 * [0, num_slots) or an accepted count outside [1, tokens] is skipped. Conv
 * windows, projected rows and core_out are not touched.
 *
 * state: fp32 pool, 16-byte aligned; state_slot_stride in elements, a
 * multiple of 4 and >= heads * 16384. slots, accepted: int32, 4-byte aligned.
 * 1 <= tokens <= 8, slots_row_stride >= tokens, 1 <= heads <= 4096,
 * requests >= 0 (0 enqueues nothing), requests * heads <= INT32_MAX.
 *
 * options (bit set):
 *   KDA_PROBE_BARRIER         a workgroup barrier between the tile's loads and
 *                             the first store (every wave's loads returned
 *                             first, as at the core kernel's first barrier);
 *   KDA_PROBE_CORE_OCCUPANCY  residency held to the core kernel's (one 16-wave
 *                             or two 8-wave workgroups a compute unit) by a
 *                             static LDS allocation.
 * The fastest of the four variants is the ceiling of the access pattern.
 * Returns KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE (also unknown option bits),
 * KDA_ERR_ALIGN or KDA_ERR_HIP; nothing is enqueued on error. Overwrites the
 * destination tiles. */
#define KDA_PROBE_BARRIER 1
#define KDA_PROBE_CORE_OCCUPANCY 2
int kda_probe_state_stream(float* state, int64_t state_slot_stride, int32_t num_slots,
                           const int32_t* slots, int64_t slots_row_stride,
                           const int32_t* accepted, int32_t requests, int32_t tokens,
                           int32_t heads, int32_t options, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H */
