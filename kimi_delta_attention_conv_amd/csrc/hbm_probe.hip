// HBM stream probes (measurement only; see include/kda_probe.h): grid-stride
// read, write and copy with 16-byte non-temporal accesses, sized to keep every
// CU's memory pipeline busy (256 CUs x 8 workgroups of 256 threads), and write
// and copy over one contiguous run per workgroup with plain stores (4096
// workgroups of 256 threads), the fastest write shape measured on MI355X.
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

int kda_probe_read(const void* src, int64_t bytes, float* sink, void* hip_stream) {
    if (src == nullptr || sink == nullptr) return KDA_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || !ok16(src) || !ok16(sink)) return KDA_ERR_ALIGN;
    hipLaunchKernelGGL(probe_read, dim3(kBlocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const f32x4*>(src),
                       bytes / 16, sink);
    return launched();
}

}  // extern "C"
