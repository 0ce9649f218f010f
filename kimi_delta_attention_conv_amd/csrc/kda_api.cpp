// Host side of the C ABI declared in include/kda.h: argument validation (all
// of it before anything is enqueued), the handle and its device memory, and
// the stream-ordered launches of the gfx950 kernels.
//
// The call shapes follow page
// "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.prepared":
// PreparedKda.__init__ / prepare_caches (kda_prepare) and PreparedKda.run
// (kda_decode: slots [B]; kda_verify: slots [>= B, q] and accepted [>= B]).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>

#include "kda.h"
#include "kda_internal.h"

static thread_local char g_last_hip_error[256] = "";

void kda::record_hip_error(hipError_t e, const char* what) {
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s (%d)", what,
                  hipGetErrorString(e), (int)e);
}

struct kda_handle_s {
    int device = 0;
    int32_t cu_count = 0;        // compute units of `device` (the core's choice of waves a unit)
    int32_t heads = 0;
    void* dev_mem = nullptr;
    kda::PreparedWeights w{};
    int32_t* err_count = nullptr;
    int32_t* claims = nullptr;   // [num_slots] destination counts (check_distinct), else null
    kda_caches caches{};
    float lb = 0.0f, norm_eps = 0.0f, l2_eps = 0.0f;
    int32_t rounding = KDA_ROUND_FUSED;
};

namespace {

kda_status hip_fail(hipError_t e, const char* what) {
    kda::record_hip_error(e, what);
    return KDA_ERR_HIP;
}

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The handle's pointers belong to the device kda_prepare ran on.
kda_status check_device(const kda_handle_s* h) {
    int d = -1;
    hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    return d == h->device ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status check_call(const kda_handle_s* h, const void* projected, int64_t pitch,
                      int32_t requests, const int32_t* slots, const void* core_out) {
    if (h == nullptr) return KDA_ERR_NULL;
    if (requests < 0) return KDA_ERR_SHAPE;
    if (requests == 0) return KDA_OK;
    if (projected == nullptr || slots == nullptr || core_out == nullptr) return KDA_ERR_NULL;
    const int64_t D = (int64_t)h->heads * kda::kHeadDim;
    if (pitch < 4 * D + kda::kFaRank + h->heads) return KDA_ERR_SHAPE;
    if (!aligned(projected, 2) || !aligned(core_out, 4) || !aligned(slots, 4)) return KDA_ERR_ALIGN;
    // the grid is requests x heads workgroups
    if ((int64_t)requests * h->heads > INT32_MAX) return KDA_ERR_SHAPE;
    return KDA_OK;
}

kda::CoreParams core_params(const kda_handle_s* h, const void* projected, int64_t pitch,
                            int32_t requests, const int32_t* slots, int64_t slots_row_stride,
                            const int32_t* accepted, void* core_out) {
    kda::CoreParams p{};
    p.projected = static_cast<const uint16_t*>(projected);
    p.pitch = pitch;
    p.slots = slots;
    p.slots_row_stride = slots_row_stride;
    p.accepted = accepted;
    p.conv = static_cast<uint16_t*>(h->caches.conv);
    p.conv_slot_stride = h->caches.conv_slot_stride;
    p.conv_dim_stride = h->caches.conv_dim_stride;
    p.conv_pos_stride = h->caches.conv_pos_stride;
    p.state = h->caches.state;
    p.state_slot_stride = h->caches.state_slot_stride;
    p.conv_w = h->w.conv_w;
    p.conv_b = h->w.conv_b;
    p.f_b = h->w.f_b;
    p.a_exp = h->w.a_exp;
    p.dt_bias = h->w.dt_bias;
    p.norm_w = h->w.norm_w;
    p.out = static_cast<uint16_t*>(core_out);
    p.err_count = h->err_count;
    p.heads = h->heads;
    p.requests = requests;
    p.num_slots = h->caches.num_slots;
    p.lb = h->lb;
    p.q_scale = 1.0f / std::sqrt((float)kda::kHeadDim);
    p.norm_eps = h->norm_eps;
    p.l2_eps = h->l2_eps;
    p.handoff_bf16 = h->rounding == KDA_ROUND_BF16_HANDOFF;
    // f_a is read as 4-byte words when every row starts 4-byte aligned
    p.fa_u16 = (pitch % 2 != 0) || !aligned(projected, 4);
    p.cu_count = h->cu_count;
    p.claims = h->claims;
    // the dim-first pool [slots][3D][3] with 16-byte aligned slots takes the
    // kernel's coalesced window stores (each head's q, k, v windows are three
    // contiguous 768-byte runs whose starts are multiples of 16 bytes)
    p.conv_dim_first16 = h->caches.conv_pos_stride == 1 && h->caches.conv_dim_stride == 3 &&
                         h->caches.conv_slot_stride % 8 == 0 && aligned(h->caches.conv, 16);
    return p;
}

// The core launch, with the distinct-destination check around it when the
// handle has one: claims, the core kernel (which skips every request naming a
// slot claimed more than once), then the claims' reset. All three are kernels
// on the caller's stream, so the sequence can be captured in a graph.
hipError_t run_core(const kda_handle_s* h, int tokens, const kda::CoreParams& p, hipStream_t s) {
    if (h->claims == nullptr) return kda::launch_core(tokens, p, s);
    hipError_t e = kda::launch_claims(tokens, p, h->claims, false, s);
    if (e != hipSuccess) return e;
    e = kda::launch_core(tokens, p, s);
    // the reset is enqueued even when the core launch failed, so that the
    // claims are zero again for the next call
    const hipError_t c = kda::launch_claims(tokens, p, h->claims, true, s);
    return e != hipSuccess ? e : c;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "a count, size, pitch or stride is out of range";
        case KDA_ERR_ALIGN: return "a pointer, pitch or stride is misaligned";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration (conv width must be 4, tokens <= 8)";
        case KDA_ERR_HIP: return "a HIP runtime call failed";
        case KDA_ERR_NOMEM: return "out of memory";
        case KDA_ERR_DEVICE: return "the current device is not the handle's device";
        case KDA_ERR_SCRATCH: return "the shape needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

const char* kda_last_hip_error(void) { return g_last_hip_error; }

kda_status kda_prepare(const kda_weights* w, const kda_caches* c, void* hip_stream,
                       kda_handle* out) {
    if (w == nullptr || c == nullptr || out == nullptr) return KDA_ERR_NULL;
    if (w->conv_weight == nullptr || w->f_b == nullptr || w->A_log == nullptr ||
        w->dt_bias == nullptr || w->norm_weight == nullptr || c->conv == nullptr ||
        c->state == nullptr)
        return KDA_ERR_NULL;
    if (w->heads < 1 || w->heads > 4096) return KDA_ERR_SHAPE;
    if (w->conv_width != kda::kWidth) return KDA_ERR_UNSUPPORTED;
    if (w->norm_head_stride != 0 && w->norm_head_stride != kda::kHeadDim) return KDA_ERR_SHAPE;
    // both epsilons strictly positive: with zero, an all-zero q, k or o row
    // would divide zero by zero
    if (!std::isfinite(w->gate_lower_bound) || !std::isfinite(w->norm_eps) ||
        !std::isfinite(w->l2_eps) || !(w->norm_eps > 0.0f) || !(w->l2_eps > 0.0f))
        return KDA_ERR_SHAPE;
    if (w->rounding != KDA_ROUND_FUSED && w->rounding != KDA_ROUND_BF16_HANDOFF)
        return KDA_ERR_SHAPE;
    for (int32_t dt : {w->A_log_dtype, w->dt_bias_dtype, w->norm_weight_dtype})
        if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_SHAPE;
    const int64_t H = w->heads, D = H * kda::kHeadDim, C = 3 * D;
    if (c->num_slots < 1) return KDA_ERR_SHAPE;
    if (c->check_distinct != 0 && c->check_distinct != 1) return KDA_ERR_SHAPE;
    if (c->conv_slot_stride < 0 || c->conv_dim_stride < 0 || c->conv_pos_stride < 0)
        return KDA_ERR_SHAPE;
    // every (channel, position) of a slot must be addressable without overlap in
    // at least the channel-major sense: the slot stride spans the window block
    if (c->conv_slot_stride < (C - 1) * c->conv_dim_stride + (kda::kWidth - 2) * c->conv_pos_stride + 1)
        return KDA_ERR_SHAPE;
    if (c->state_slot_stride < H * kda::kHeadDim * kda::kHeadDim) return KDA_ERR_SHAPE;
    if (c->state_slot_stride % 4 != 0 || !aligned(c->state, 16)) return KDA_ERR_ALIGN;
    if (!aligned(c->conv, 2) || !aligned(w->conv_weight, 2) || !aligned(w->f_b, 2) ||
        (w->conv_bias != nullptr && !aligned(w->conv_bias, 2)) ||
        !aligned(w->A_log, w->A_log_dtype == KDA_BF16 ? 2 : 4) ||
        !aligned(w->dt_bias, w->dt_bias_dtype == KDA_BF16 ? 2 : 4) ||
        !aligned(w->norm_weight, w->norm_weight_dtype == KDA_BF16 ? 2 : 4))
        return KDA_ERR_ALIGN;

    kda_handle_s* h = new (std::nothrow) kda_handle_s();
    if (h == nullptr) return KDA_ERR_NOMEM;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "hipGetDevice");
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "hipDeviceGetAttribute");
    }
    h->cu_count = cus;
    const int64_t b_conv_w = align_up(C * kda::kWidth * 4), b_conv_b = align_up(C * 4),
                  b_fb = align_up(D * kda::kFaRank * 2), b_a = align_up(H * 4),
                  b_dt = align_up(D * 4), b_nw = align_up(H * kda::kHeadDim * 4),
                  b_err = kAlign, b_claims = c->check_distinct ? align_up((int64_t)c->num_slots * 4) : 0;
    const int64_t total = b_conv_w + b_conv_b + b_fb + b_a + b_dt + b_nw + b_err + b_claims;
    e = hipMalloc(&h->dev_mem, (size_t)total);
    if (e != hipSuccess) {
        delete h;
        return e == hipErrorOutOfMemory ? KDA_ERR_NOMEM : hip_fail(e, "hipMalloc");
    }
    char* base = static_cast<char*>(h->dev_mem);
    h->w.conv_w = reinterpret_cast<float*>(base);
    base += b_conv_w;
    h->w.conv_b = reinterpret_cast<float*>(base);
    base += b_conv_b;
    h->w.f_b = reinterpret_cast<uint16_t*>(base);
    base += b_fb;
    h->w.a_exp = reinterpret_cast<float*>(base);
    base += b_a;
    h->w.dt_bias = reinterpret_cast<float*>(base);
    base += b_dt;
    h->w.norm_w = reinterpret_cast<float*>(base);
    base += b_nw;
    h->err_count = reinterpret_cast<int32_t*>(base);
    base += b_err;
    h->claims = c->check_distinct ? reinterpret_cast<int32_t*>(base) : nullptr;
    h->heads = w->heads;
    h->caches = *c;
    h->lb = w->gate_lower_bound;
    h->norm_eps = w->norm_eps;
    h->l2_eps = w->l2_eps;
    h->rounding = w->rounding;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    kda::PrepareParams in{};
    in.conv_weight = static_cast<const uint16_t*>(w->conv_weight);
    in.conv_bias = static_cast<const uint16_t*>(w->conv_bias);
    in.f_b = static_cast<const uint16_t*>(w->f_b);
    in.A_log = w->A_log;
    in.dt_bias = w->dt_bias;
    in.norm_weight = w->norm_weight;
    in.norm_head_stride = w->norm_head_stride;
    in.heads = w->heads;
    in.A_log_bf16 = w->A_log_dtype == KDA_BF16;
    in.dt_bias_bf16 = w->dt_bias_dtype == KDA_BF16;
    in.norm_weight_bf16 = w->norm_weight_dtype == KDA_BF16;
    // counters start at zero (kernels, not memsets: graph-safe everywhere)
    e = kda::launch_zero(h->err_count, 1, s);
    if (e == hipSuccess && h->claims != nullptr) e = kda::launch_zero(h->claims, c->num_slots, s);
    if (e == hipSuccess) e = kda::launch_prepare(in, h->w, s);
    if (e != hipSuccess) {
        kda_status st = hip_fail(e, "prepare launch");
        (void)hipFree(h->dev_mem);
        delete h;
        return st;
    }
    *out = h;
    return KDA_OK;
}

kda_status kda_decode(kda_handle h, const void* projected, int64_t pitch, int32_t batch,
                      const int32_t* slots, void* core_out, void* hip_stream) {
    kda_status st = check_call(h, projected, pitch, batch, slots, core_out);
    if (st != KDA_OK || batch == 0) return st;
    if ((st = check_device(h)) != KDA_OK) return st;
    const kda::CoreParams p = core_params(h, projected, pitch, batch, slots, 1, nullptr, core_out);
    hipError_t e = run_core(h, 1, p, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? KDA_OK : hip_fail(e, "kda_decode launch");
}

kda_status kda_verify(kda_handle h, const void* projected, int64_t pitch, int32_t requests,
                      int32_t tokens, const int32_t* slots, int64_t slots_row_stride,
                      const int32_t* accepted, void* core_out, void* hip_stream) {
    if (h == nullptr) return KDA_ERR_NULL;
    if (tokens < 1) return KDA_ERR_SHAPE;
    if (tokens > kda::kMaxTokens) return KDA_ERR_UNSUPPORTED;
    if (slots_row_stride < tokens) return KDA_ERR_SHAPE;
    kda_status st = check_call(h, projected, pitch, requests, slots, core_out);
    if (st != KDA_OK || requests == 0) return st;
    if (accepted == nullptr) return KDA_ERR_NULL;
    if (!aligned(accepted, 4)) return KDA_ERR_ALIGN;
    if ((int64_t)requests * tokens > INT32_MAX) return KDA_ERR_SHAPE;
    if ((st = check_device(h)) != KDA_OK) return st;
    const kda::CoreParams p =
        core_params(h, projected, pitch, requests, slots, slots_row_stride, accepted, core_out);
    hipError_t e = run_core(h, tokens, p, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? KDA_OK : hip_fail(e, "kda_verify launch");
}

kda_status kda_linear(const void* x, int64_t x_pitch, const void* w, void* y, int64_t y_pitch,
                      int32_t M, int32_t N, int32_t K, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
    if (M < 0 || N < 1 || K < 8 || K % 8 != 0) return KDA_ERR_SHAPE;
    if (M > (1 << 20)) return KDA_ERR_SHAPE;   // grid y limit at 64 rows a workgroup
    // one workgroup per tile of at least 128 x 64 outputs above 64 rows: M N <= 2^43
    // keeps every grid within 2^31 workgroups
    if ((int64_t)M * N > ((int64_t)1 << 43)) return KDA_ERR_SHAPE;
    if (M == 0) return KDA_OK;
    if (x == nullptr || w == nullptr || y == nullptr) return KDA_ERR_NULL;
    if (x_pitch < K || y_pitch < N) return KDA_ERR_SHAPE;
    if (x_pitch % 8 != 0 || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 2) ||
        !aligned(workspace, 16))
        return KDA_ERR_ALIGN;
    kda::LinearParams p{};
    p.X = static_cast<const uint16_t*>(x);
    p.x_pitch = x_pitch;
    p.W = static_cast<const uint16_t*>(w);
    p.Y = static_cast<uint16_t*>(y);
    p.y_pitch = y_pitch;
    p.M = M;
    p.N = N;
    p.K = K;
    p.part = static_cast<float*>(workspace);
    p.part_floats = workspace == nullptr ? 0 : (int64_t)(workspace_bytes / sizeof(float));
    p.cu_count = kda::current_device_cus();
    hipError_t e = kda::launch_linear(p, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? KDA_OK : hip_fail(e, "kda_linear launch");
}

size_t kda_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || N < 1 || K < 8 || K % 8 != 0 || M > (1 << 20)) return 0;
    return (size_t)kda::linear_workspace_floats(M, N, K) * sizeof(float);
}

kda_status kda_in_proj(const void* x, int64_t x_pitch, const void* w_in, void* projected,
                       int64_t pitch, int32_t rows, int32_t hidden, int32_t heads,
                       void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (heads < 1 || heads > 4096) return KDA_ERR_SHAPE;
    const int32_t N = 4 * heads * kda::kHeadDim + kda::kFaRank + heads;
    return kda_linear(x, x_pitch, w_in, projected, pitch, rows, N, hidden, workspace,
                      workspace_bytes, hip_stream);
}

kda_status kda_o_proj(const void* core, int64_t core_pitch, const void* w_o, void* out,
                      int64_t out_pitch, int32_t rows, int32_t heads, int32_t hidden,
                      void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (heads < 1 || heads > 4096) return KDA_ERR_SHAPE;
    return kda_linear(core, core_pitch, w_o, out, out_pitch, rows, hidden,
                      heads * kda::kHeadDim, workspace, workspace_bytes, hip_stream);
}

kda_status kda_device_errors(kda_handle h, int32_t* count_out, void* hip_stream) {
    if (h == nullptr || count_out == nullptr) return KDA_ERR_NULL;
    const kda_status st = check_device(h);
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    int32_t host = 0;
    hipError_t e = hipMemcpyAsync(&host, h->err_count, sizeof host, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = kda::launch_zero(h->err_count, 1, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "kda_device_errors");
    *count_out = host;
    return KDA_OK;
}

kda_status kda_destroy(kda_handle h) {
    if (h == nullptr) return KDA_OK;
    int caller = -1;
    hipError_t c = hipGetDevice(&caller);
    if (c == hipSuccess && caller != h->device) c = hipSetDevice(h->device);
    if (c != hipSuccess) return hip_fail(c, "kda_destroy device");   // handle kept: retry possible
    hipError_t e = hipDeviceSynchronize();
    hipError_t f = hipFree(h->dev_mem);
    delete h;
    hipError_t r = caller != -1 ? hipSetDevice(caller) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "kda_destroy sync");
    if (f != hipSuccess) return hip_fail(f, "kda_destroy free");
    if (r != hipSuccess) return hip_fail(r, "kda_destroy restore device");
    return KDA_OK;
}

}  // extern "C"
