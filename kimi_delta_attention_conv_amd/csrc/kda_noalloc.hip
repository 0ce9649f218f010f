// kda_linear_noalloc: kda_linear for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops or harnesses that
// forbid hipMalloc). The K split's fp32 partial tiles, which kda_linear takes
// in a caller's workspace, go instead to a static device array of this file,
// `scratch`, of kScratchBytes. Each GPU the library runs on holds its own copy
// of the array from module load until the process ends.
//
// Host code never passes the array's name to a kernel: in host code that name
// is a host-side stand-in, not a device address. The first call on a device
// (with that device current) asks the runtime for the device address with
// hipGetSymbolAddress and keeps it per device; every launch takes that
// pointer.
//
// Every call on a GPU shares that GPU's array. The split kernels overwrite
// each partial they later read, so nothing needs clearing between calls, but
// two calls that overlap in time on one GPU (other streams, other threads)
// race on the array: callers serialise them, for instance on one stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr int64_t kScratchBytes = int64_t{KDA_NOALLOC_SCRATCH_BYTES};
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (set-up on first use).
hipError_t scratch_for(int device, float** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = ptr;
    }
    *out = static_cast<float*>(g_scratch_ptr[device]);
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t kda_noalloc_scratch_bytes(void) { return (size_t)kScratchBytes; }

kda_status kda_linear_noalloc(const void* x, int64_t x_pitch, const void* w, void* y,
                              int64_t y_pitch, int32_t M, int32_t N, int32_t K,
                              void* hip_stream) {
    // the same validation as kda_linear, before anything else
    if (M < 0 || N < 1 || K < 8 || K % 8 != 0) return KDA_ERR_SHAPE;
    if (M > (1 << 20)) return KDA_ERR_SHAPE;
    if ((int64_t)M * N > ((int64_t)1 << 43)) return KDA_ERR_SHAPE;
    if (M == 0) return KDA_OK;
    if (x == nullptr || w == nullptr || y == nullptr) return KDA_ERR_NULL;
    if (x_pitch < K || y_pitch < N) return KDA_ERR_SHAPE;
    const auto al = [](const void* p, uintptr_t a) {
        return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
    };
    if (x_pitch % 8 != 0 || !al(x, 16) || !al(w, 16) || !al(y, 2)) return KDA_ERR_ALIGN;
    const int64_t need = kda::linear_workspace_floats(M, N, K) * (int64_t)sizeof(float);
    if (need > kScratchBytes) return KDA_ERR_SCRATCH;

    kda::LinearParams p{};
    p.X = static_cast<const uint16_t*>(x);
    p.x_pitch = x_pitch;
    p.W = static_cast<const uint16_t*>(w);
    p.Y = static_cast<uint16_t*>(y);
    p.y_pitch = y_pitch;
    p.M = M;
    p.N = N;
    p.K = K;
    p.cu_count = kda::current_device_cus();
    if (need > 0) {
        int device = -1;
        hipError_t e = hipGetDevice(&device);
        float* ptr = nullptr;
        if (e == hipSuccess) e = scratch_for(device, &ptr);
        if (e != hipSuccess) {
            kda::record_hip_error(e, "kda_linear_noalloc scratch");
            return KDA_ERR_HIP;
        }
        p.part = ptr;
        p.part_floats = kScratchBytes / (int64_t)sizeof(float);
    }
    const hipError_t e = kda::launch_linear(p, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) {
        kda::record_hip_error(e, "kda_linear_noalloc launch");
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

}  // extern "C"
