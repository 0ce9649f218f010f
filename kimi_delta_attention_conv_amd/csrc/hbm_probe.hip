// HBM stream probes (measurement only; see include/kda_probe.h; built into
// libkda_probe.so, apart from the product library): grid-stride
// read, write and copy with 16-byte non-temporal accesses, sized to keep every
// CU's memory pipeline busy (256 CUs x 8 workgroups of 256 threads), write
// and copy over one contiguous run per workgroup with plain stores (4096
// workgroups of 256 threads), the fastest write shape measured on MI355X, and
// the core kernel's state traffic with none of its arithmetic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"
#include "kda_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlocks = 2048;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void probe_copy(f32x4* __restrict__ dst,
                                                       const f32x4* __restrict__ src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kThreads) void probe_write(f32x4* __restrict__ dst, int64_t n,
                                                        float value) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const f32x4 v = {value, value, value, value};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(v, dst + i);
}

__global__ __launch_bounds__(kThreads) void probe_read(const f32x4* __restrict__ src, int64_t n,
                                                       float* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    float acc = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const f32x4 v = __builtin_nontemporal_load(src + i);
        acc += (v.x + v.y) + (v.z + v.w);
    }
    __shared__ float part[kThreads / 64];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) s += part[w];
        sink[blockIdx.x] = s;
    }
}

// Workgroup b covers float4 elements [b * per, min((b + 1) * per, n)).
__global__ __launch_bounds__(kThreads) void probe_write_runs(f32x4* __restrict__ dst, int64_t n,
                                                             int64_t per, float value) {
    const f32x4 v = {value, value, value, value};
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < n ? lo + per : n;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) dst[i] = v;
}

__global__ __launch_bounds__(kThreads) void probe_copy_runs(f32x4* __restrict__ dst,
                                                            const f32x4* __restrict__ src,
                                                            int64_t n, int64_t per) {
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < n ? lo + per : n;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) dst[i] = src[i];
}

// The core kernel's state traffic alone (kda_probe_state_stream): one
// workgroup per (request, head) unit with the core's waves a unit, units
// blocked by XCD (workgroup b runs on XCD b % 8), the core's lane layout (8
// waves: lane l holds rows 16w + (l >> 3) and 16w + 8 + (l >> 3); 16 waves:
// row 8w + (l >> 3); columns 32m + 4(l & 7) .. +3), non-temporal loads for one
// token and plain loads otherwise, non-temporal stores, one tile written per
// token. BARRIER: a workgroup barrier after the loads (it waits for every
// wave's loads, as the core kernel's first barrier does), so that no store of
// a workgroup starts before all of its loads have returned. CAP: a static LDS
// allocation that holds residency to the core kernel's own (one 16-wave or
// two 8-wave workgroups a compute unit of 160 KB); without it the probe, far
// lighter in registers, runs more workgroups a CU than the core kernel can.
constexpr int kTile = 128;
template <int L, int WAVES, bool BARRIER, bool CAP>
__global__ __launch_bounds__(64 * WAVES) void probe_state_stream(float* __restrict__ state,
                                                          int64_t slot_stride, int num_slots,
                                                          const int32_t* __restrict__ slots,
                                                          int64_t row_stride,
                                                          const int32_t* __restrict__ accepted,
                                                          int requests, int heads) {
    // 96 KB (one workgroup a CU) or 56 KB (two); 4 bytes when not capped
    constexpr int kPad = !CAP ? 1 : (WAVES == 16 ? 24576 : 14336);
    __shared__ float pad[kPad];
    if (CAP && num_slots < 0) {   // never taken (num_slots >= 1): keeps the allocation
        pad[threadIdx.x % kPad] = 0.0f;
        __syncthreads();
        state[0] = pad[(threadIdx.x + 1) % kPad];
    }
    int unit = blockIdx.x;
    const int q = (requests * heads) >> 3;
    if ((int)blockIdx.x < 8 * q) unit = (blockIdx.x & 7) * q + (blockIdx.x >> 3);
    const int r = unit / heads, h = unit - r * heads;
    const int32_t* srow = slots + (int64_t)r * row_stride;
    const int a = accepted != nullptr ? accepted[r] : 1;
    int dst[L];
    bool ok = a >= 1 && a <= L;
    int src = srow[0];
#pragma unroll
    for (int t = 0; t < L; ++t) {
        dst[t] = srow[t];
        ok = ok && (unsigned)dst[t] < (unsigned)num_slots;
        if (t == a - 1) src = dst[t];
    }
    if (!ok) return;   // uniform across the workgroup: no wave reaches the barrier
    constexpr int RW = kTile / WAVES, G = RW / 8;   // rows a wave, 8-row groups a lane
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t off = (int64_t)h * kTile * kTile + (int64_t)(wave * RW + (lane >> 3)) * kTile +
                        (lane & 7) * 4;
    f32x4 S[G][4];
    const float* sb = state + (int64_t)src * slot_stride + off;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4* ptr = reinterpret_cast<const f32x4*>(sb + g * 8 * kTile + 32 * m);
            S[g][m] = (L == 1) ? __builtin_nontemporal_load(ptr) : *ptr;
        }
    if (BARRIER) __syncthreads();
#pragma unroll
    for (int t = 0; t < L; ++t) {
        float* dp = state + (int64_t)dst[t] * slot_stride + off;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                S[g][m] *= 0.999f;
                __builtin_nontemporal_store(S[g][m], reinterpret_cast<f32x4*>(dp + g * 8 * kTile + 32 * m));
            }
    }
}

// The core kernel's choice of waves a unit: 16 for one token or at most one
// unit a compute unit, else 8.
template <int L, bool BARRIER, bool CAP>
void launch_state_stream_v(float* state, int64_t slot_stride, int num_slots, const int32_t* slots,
                           int64_t row_stride, const int32_t* accepted, int requests, int heads,
                           int cu_count, hipStream_t s) {
    const dim3 grid((unsigned)(requests * heads));
    if (L == 1 || (int64_t)requests * heads <= cu_count)
        hipLaunchKernelGGL((probe_state_stream<L, 16, BARRIER, CAP>), grid, dim3(1024), 0, s, state,
                           slot_stride, num_slots, slots, row_stride, accepted, requests, heads);
    else
        hipLaunchKernelGGL((probe_state_stream<L, 8, BARRIER, CAP>), grid, dim3(512), 0, s, state,
                           slot_stride, num_slots, slots, row_stride, accepted, requests, heads);
}

template <int L>
void launch_state_stream(float* state, int64_t slot_stride, int num_slots, const int32_t* slots,
                         int64_t row_stride, const int32_t* accepted, int requests, int heads,
                         int cu_count, int options, hipStream_t s) {
    const bool barrier = (options & KDA_PROBE_BARRIER) != 0, cap = (options & KDA_PROBE_CORE_OCCUPANCY) != 0;
    if (barrier && cap)
        launch_state_stream_v<L, true, true>(state, slot_stride, num_slots, slots, row_stride, accepted,
                                             requests, heads, cu_count, s);
    else if (barrier)
        launch_state_stream_v<L, true, false>(state, slot_stride, num_slots, slots, row_stride, accepted,
                                              requests, heads, cu_count, s);
    else if (cap)
        launch_state_stream_v<L, false, true>(state, slot_stride, num_slots, slots, row_stride, accepted,
                                              requests, heads, cu_count, s);
    else
        launch_state_stream_v<L, false, false>(state, slot_stride, num_slots, slots, row_stride, accepted,
                                               requests, heads, cu_count, s);
}

constexpr int kRunBlocks = 4096;

bool ok16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

}  // namespace

extern "C" {

int32_t kda_probe_sink_floats(void) { return kBlocks; }

int kda_probe_copy(void* dst, const void* src, int64_t bytes, void* hip_stream) {
    if (dst == nullptr || src == nullptr) return KDA_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || !ok16(dst) || !ok16(src)) return KDA_ERR_ALIGN;
    hipLaunchKernelGGL(probe_copy, dim3(kBlocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<f32x4*>(dst),
                       static_cast<const f32x4*>(src), bytes / 16);
    return launched();
}

int kda_probe_write(void* dst, int64_t bytes, float value, void* hip_stream) {
    if (dst == nullptr) return KDA_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || !ok16(dst)) return KDA_ERR_ALIGN;
    hipLaunchKernelGGL(probe_write, dim3(kBlocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<f32x4*>(dst), bytes / 16,
                       value);
    return launched();
}

int kda_probe_write_runs(void* dst, int64_t bytes, float value, void* hip_stream) {
    if (dst == nullptr) return KDA_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || !ok16(dst)) return KDA_ERR_ALIGN;
    const int64_t n = bytes / 16, per = (n + kRunBlocks - 1) / kRunBlocks;
    hipLaunchKernelGGL(probe_write_runs, dim3(kRunBlocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<f32x4*>(dst), n, per,
                       value);
    return launched();
}

int kda_probe_copy_runs(void* dst, const void* src, int64_t bytes, void* hip_stream) {
    if (dst == nullptr || src == nullptr) return KDA_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || !ok16(dst) || !ok16(src)) return KDA_ERR_ALIGN;
    const int64_t n = bytes / 16, per = (n + kRunBlocks - 1) / kRunBlocks;
    hipLaunchKernelGGL(probe_copy_runs, dim3(kRunBlocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<f32x4*>(dst),
                       static_cast<const f32x4*>(src), n, per);
    return launched();
}

int kda_probe_state_stream(float* state, int64_t state_slot_stride, int32_t num_slots,
                           const int32_t* slots, int64_t slots_row_stride,
                           const int32_t* accepted, int32_t requests, int32_t tokens,
                           int32_t heads, int32_t options, void* hip_stream) {
    if (tokens < 1 || tokens > 8 || heads < 1 || heads > 4096 || requests < 0 ||
        num_slots < 1 || slots_row_stride < tokens)
        return KDA_ERR_SHAPE;
    if ((options & ~(KDA_PROBE_BARRIER | KDA_PROBE_CORE_OCCUPANCY)) != 0) return KDA_ERR_SHAPE;
    if ((int64_t)requests * heads > INT32_MAX) return KDA_ERR_SHAPE;
    if (state_slot_stride < (int64_t)heads * kTile * kTile) return KDA_ERR_SHAPE;
    if (requests == 0) return KDA_OK;
    if (state == nullptr || slots == nullptr) return KDA_ERR_NULL;
    if (!ok16(state) || state_slot_stride % 4 != 0 ||
        (reinterpret_cast<uintptr_t>(slots) & 3) != 0 ||
        (reinterpret_cast<uintptr_t>(accepted) & 3) != 0)
        return KDA_ERR_ALIGN;
    int device = 0, cus = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return KDA_ERR_HIP;
    using Launch = void (*)(float*, int64_t, int, const int32_t*, int64_t, const int32_t*, int,
                            int, int, int, hipStream_t);
    static const Launch kLaunch[8] = {launch_state_stream<1>, launch_state_stream<2>,
                                      launch_state_stream<3>, launch_state_stream<4>,
                                      launch_state_stream<5>, launch_state_stream<6>,
                                      launch_state_stream<7>, launch_state_stream<8>};
    kLaunch[tokens - 1](state, state_slot_stride, num_slots, slots, slots_row_stride, accepted,
                        requests, heads, cus, options, static_cast<hipStream_t>(hip_stream));
    return launched();
}

int kda_probe_read(const void* src, int64_t bytes, float* sink, void* hip_stream) {
    if (src == nullptr || sink == nullptr) return KDA_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || !ok16(src) || !ok16(sink)) return KDA_ERR_ALIGN;
    hipLaunchKernelGGL(probe_read, dim3(kBlocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const f32x4*>(src),
                       bytes / 16, sink);
    return launched();
}

}  // extern "C"
