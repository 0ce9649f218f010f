// Internal interface between the host library (kda_api.cpp) and the gfx950
// kernels (kda_core.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kHeadDim = 128;   // dk = dv
constexpr int kFaRank = 128;    // f_a width
constexpr int kWidth = 4;       // conv taps
constexpr int kMaxTokens = 8;   // verify length bound

// Weights in the layout the core kernel reads, owned by a handle.
struct PreparedWeights {
    float* conv_w;        // fp32 [3D][W]: tap j of channel c at c * W + j (one 16-byte row a channel)
    float* conv_b;        // fp32 [3D] (zeros when the layer has no conv bias)
    uint16_t* f_b;        // bf16 [D][128]
    float* a_exp;         // fp32 [H] = exp(A_log)
    float* dt_bias;       // fp32 [D]
    float* norm_w;        // fp32 [H][128]
};

// Everything one launch of the core kernel reads, by value.
struct CoreParams {
    const uint16_t* projected;  // bf16 rows, pitch elements apart
    int64_t pitch;
    const int32_t* slots;
    int64_t slots_row_stride;
    const int32_t* accepted;    // nullptr: decode (src = dst = slots[r])
    uint16_t* conv;
    int64_t conv_slot_stride, conv_dim_stride, conv_pos_stride;
    float* state;
    int64_t state_slot_stride;
    const float* conv_w;
    const float* conv_b;
    const uint16_t* f_b;
    const float* a_exp;
    const float* dt_bias;
    const float* norm_w;
    uint16_t* out;
    int32_t* err_count;
    int32_t heads;
    int32_t requests;
    int32_t num_slots;
    float lb;
    float q_scale;
    float norm_eps;
    float l2_eps;
    int32_t conv_dim_first16;   // conv pool is dim first [slots][3D][3], 16-byte aligned
    int32_t handoff_bf16;       // round conv out, g1 and o to bf16 where produced
    int32_t fa_u16;             // f_a columns only 2-byte aligned (odd pitch or base)
    int32_t cu_count;           // compute units of the device (host side: waves a unit)
    const int32_t* claims;      // per-slot destination counts of this call, or nullptr
};

// Raw inputs of the weight re-layout kernel (device pointers).
struct PrepareParams {
    const uint16_t* conv_weight;  // bf16 [3D][1][W]
    const uint16_t* conv_bias;    // bf16 [3D] or nullptr
    const uint16_t* f_b;          // bf16 [D][128]
    const void* A_log;            // [H]
    const void* dt_bias;          // [D]
    const void* norm_weight;      // [128] or [H][128]
    int32_t norm_head_stride;
    int32_t heads;
    int32_t A_log_bf16, dt_bias_bf16, norm_weight_bf16;   // element type bf16 (else fp32)
};

// Y[M][N] = X[M][K] W[N][K]^T (bf16 in, fp32 accumulate, bf16 out).
struct LinearParams {
    const uint16_t* X;   // rows x_pitch elements apart, 16-byte aligned
    int64_t x_pitch;
    const uint16_t* W;   // dense [N][K]
    uint16_t* Y;         // rows y_pitch elements apart
    int64_t y_pitch;
    int32_t M, N, K;     // K a multiple of 8
    float* part;         // fp32 workspace for a K split, or null
    int64_t part_floats; // its capacity in floats
    int32_t cu_count;    // compute units of the current device (0: unknown)
};

hipError_t launch_prepare(const PrepareParams& in, const PreparedWeights& out, hipStream_t s);
// n int32 zeros at p (a kernel, so that the clear can sit in a captured graph).
hipError_t launch_zero(int32_t* p, int64_t n, hipStream_t s);
// Destination claims of one call (p.claims non-null): add one per (valid
// request, token) to claims[dst] (clear = false), or store zero there (clear =
// true, after the core kernel). A request is valid under the core kernel's
// rules (slots in range, accepted count in 1 .. L).
hipError_t launch_claims(int tokens, const CoreParams& p, int32_t* claims, bool clear, hipStream_t s);
hipError_t launch_linear(const LinearParams& p, hipStream_t s);
// Compute units of the current device, read once per device (0 if the query fails).
int32_t current_device_cus();
// Workspace floats launch_linear uses for a K split of this shape (0: none).
int64_t linear_workspace_floats(int32_t M, int32_t N, int32_t K);
hipError_t launch_core(int tokens, const CoreParams& p, hipStream_t s);
// Records a failed HIP call for kda_last_hip_error (this thread).
void record_hip_error(hipError_t e, const char* what);

}  // namespace kda
