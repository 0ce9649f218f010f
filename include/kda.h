/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA decode / spec-verify core.
 *
 * One call runs, for R requests x L tokens (S = R L rows) and H heads of 128
 * channels, the core of a Kimi Delta Attention layer between the packed input
 * projection and the gated core output:
 *   1. the causal width-4 conv update with SiLU of the packed q|k|v channels
 *      against a per-slot conv window cache;
 *   2. the channel-wise decay gate g = lb * sigmoid(exp(A_log_h) *
 *      (f_b f_a + dt_bias)) and beta = sigmoid(beta_raw);
 *   3. l2-normalised q and k, q scaled by 128^-0.5;
 *   4. the gated delta rule on a 128 x 128 fp32 state per (slot, head):
 *      S <- diag(e^g) S;  S <- S + beta k (v - S^T k)^T;  o = S^T q,
 *      with a state written for every token;
 *   5. the head-wise gated RMSNorm o_norm(o) * sigmoid(gate) into bf16.
 *
 * Sources (page titles; sections named, no line numbers):
 *   [kda]      "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.kda":
 *              module docstring (kernel K1 kda_pre; the role table's "kda
 *              tasks" row names the steps above and their order) and the host
 *              launcher entry kda_pre (the two conv cache layouts).
 *   [prepared] "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.prepared":
 *              PreparedKda.__init__ (weights, fp32 norm weight, the scalars
 *              gate_lower_bound, 128^-0.5, o_norm.eps), _operands (the packed
 *              projection row and the operand set), prepare_caches and run
 *              (decode: slots [B]; verify: slots [>= B, q], accepted [>= B]).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers on the device that is
 *     current when kda_prepare runs; every later call on the handle must be
 *     made with that device current (else KDA_ERR_DEVICE).
 *   - Sizes and strides are in elements unless a name says bytes.
 *   - Calls are asynchronous and stream ordered: they enqueue work on
 *     `hip_stream` (a hipStream_t, NULL = the null stream) and return.
 *   - Every argument is validated on the host before anything is enqueued
 *     (the only HIP call before that asks which device is current). On a
 *     non-KDA_OK status nothing was enqueued and no device memory changed,
 *     except for KDA_ERR_HIP (a HIP call failed; see kda_last_hip_error).
 *   - Nothing unwinds across the ABI; no function allocates on the host per
 *     call. Only kda_prepare allocates device memory; kda_destroy frees it.
 *     kda_linear_noalloc uses a static per-GPU buffer of the library instead
 *     of a workspace and allocates nothing.
 *   - Within one call every (request, token) must name its own destination
 *     slot ([prepared] run: a block-table slice). A slot named twice races and
 *     has no defined result, unless the caches were registered with
 *     check_distinct, which turns such requests into skipped, counted ones.
 *   - No call records a memset: counters and claims are cleared by kernels, so
 *     kda_decode, kda_verify and the projections can be captured in a HIP graph.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128   /* dk = dv = 128 ([prepared] PreparedKda.__init__: dim = 128 * heads) */
#define KDA_FA_RANK 128    /* f_a width ([prepared] _operands: projected[:, 4D : 4D + 128]) */
#define KDA_CONV_WIDTH 4   /* the only supported conv width W (conv state holds W - 1 = 3 inputs) */
#define KDA_MAX_TOKENS 8   /* largest verify length L */

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* a count, size, pitch or stride is out of range */
    KDA_ERR_ALIGN = -3,       /* a pointer, pitch or stride breaks the alignment rules */
    KDA_ERR_UNSUPPORTED = -4, /* valid but not supported: conv width != 4, L > 8 */
    KDA_ERR_HIP = -5,         /* a HIP runtime call failed (kda_last_hip_error names it) */
    KDA_ERR_NOMEM = -6,       /* device or host allocation failed in kda_prepare */
    KDA_ERR_DEVICE = -7,      /* the current HIP device is not the one the handle was prepared on */
    KDA_ERR_SCRATCH = -8      /* kda_linear_noalloc: the shape needs more scratch than
                                 KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef struct kda_handle_s* kda_handle;

/* Where intermediate values are rounded ([kda] module docstring, its sentence
 * on rounding: the fused kernels are to round as the unfused kernels did
 * wherever those passed bf16 tensors to one another).
 *   KDA_ROUND_FUSED         every intermediate stays fp32 inside the kernel;
 *   KDA_ROUND_BF16_HANDOFF  the values an unfused pipeline hands over in bf16
 *                           are rounded to bf16 (RNE) where produced: the conv
 *                           + SiLU outputs q|k|v, g1 = f_b f_a before the gate,
 *                           and the recurrence output o before the RMSNorm.
 * The state stays fp32 and core_out bf16 in both modes. */
typedef enum {
    KDA_ROUND_FUSED = 0,
    KDA_ROUND_BF16_HANDOFF = 1
} kda_rounding;

/* Element type of the small per-head and per-channel weights (A_log, dt_bias,
 * norm_weight). The library converts them to fp32 at prepare time ([prepared]
 * PreparedKda.__init__ casts them to float); bf16 values convert exactly. */
typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Attention weights of one layer ([prepared] PreparedKda.__init__). Borrowed
 * only during kda_prepare: the library copies and re-lays them out into its
 * own device memory on `hip_stream`; the caller may free them once that
 * stream has passed the kda_prepare call. All pointers are device pointers. */
typedef struct {
    int32_t heads;            /* H >= 1 heads of 128 channels; D = 128 H */
    int32_t conv_width;       /* W; must be KDA_CONV_WIDTH */
    const void* conv_weight;  /* bf16 [3D][1][W], the nn.Conv1d layout (q, k, v channel
                                 blocks of D); kept in that order as fp32 in the
                                 handle. 2-byte aligned. */
    const void* conv_bias;    /* bf16 [3D], or NULL for no conv bias (taken as zero) */
    const void* f_b;          /* bf16 [D][128], row i = output channel i. 2-byte aligned. */
    const void* A_log;        /* [H], one per head ([prepared]: heads = A_log.numel());
                                 element type A_log_dtype */
    const void* dt_bias;      /* [D]; element type dt_bias_dtype */
    const void* norm_weight;  /* o_norm weight: [128] shared by all heads (norm_head_stride
                                 0) or [H][128] (stride 128); element type norm_weight_dtype */
    int32_t norm_head_stride; /* 0 or 128 */
    float gate_lower_bound;   /* lb (e.g. -5); finite */
    float norm_eps;           /* o_norm.eps (e.g. 1e-6); finite and > 0 */
    float l2_eps;             /* epsilon inside the l2norm square root (1e-6); finite and > 0
                                 (with 0, an all-zero q or k row would give 0 / 0) */
    int32_t rounding;         /* a kda_rounding value; zero-initialised = KDA_ROUND_FUSED */
    int32_t A_log_dtype;      /* kda_dtype of A_log; zero-initialised = KDA_F32 */
    int32_t dt_bias_dtype;    /* kda_dtype of dt_bias */
    int32_t norm_weight_dtype;/* kda_dtype of norm_weight */
} kda_weights;

/* The per-slot caches of one layer ([kda] kda_pre launcher: conv_state
 * [slots, dim, state_len] or a transposed view; [prepared] prepare_caches).
 * Borrowed for the handle's lifetime: the library records the pointers and
 * strides; the caller keeps the memory alive and changes it only through
 * these calls (or between calls, stream ordered).
 *
 *   conv  : bf16 windows of the last W - 1 = 3 q|k|v inputs, oldest first.
 *           Element (slot, channel c < 3D, position m < 3) lives at
 *           conv + slot * conv_slot_stride + c * conv_dim_stride + m * conv_pos_stride.
 *           Dim first [slots][3D][3]: strides (9D, 3, 1). Transposed view of
 *           storage [slots][3][3D]: strides (9D, 1, 3D). Any non-negative
 *           strides are accepted; those two are the fast paths.
 *   state : fp32 [slots][H][128 v][128 k] per slot, slot stride
 *           state_slot_stride >= H * 128 * 128; row v of a head is
 *           contiguous over k. Base 16-byte aligned, stride a multiple of 4.
 *
 *   check_distinct : 0 (default) or 1. With 1, every kda_decode / kda_verify
 *           call first counts, per slot, how many (valid request, token)
 *           pairs name it as a destination, and every request naming a slot
 *           counted more than once (twice in its own row included) is skipped
 *           entirely and counted in kda_device_errors, like a request with an
 *           invalid index; the counts are reset at the end of the call. Costs
 *           num_slots * 4 bytes of handle memory and two small kernels a call.
 *           With 0 the distinct destinations are a precondition, not checked. */
typedef struct {
    void* conv;
    int64_t conv_slot_stride;
    int64_t conv_dim_stride;
    int64_t conv_pos_stride;
    float* state;
    int64_t state_slot_stride;
    int32_t num_slots;        /* >= 1; valid slot indices are 0 .. num_slots - 1 */
    int32_t check_distinct;   /* 0 or 1 (above); zero-initialised = no check */
} kda_caches;

/* Creates a handle: validates, allocates the handle's device memory, re-lays
 * the weights out on `hip_stream` ([prepared] PreparedKda.__init__) and records
 * the caches. *out is set only on KDA_OK.
 * Errors: KDA_ERR_NULL (w, c, out, a weight or cache pointer), KDA_ERR_SHAPE
 * (heads < 1, num_slots < 1, a stride too small or negative, norm_head_stride
 * not 0 or 128, a non-finite scalar or an epsilon <= 0, rounding not a
 * kda_rounding value, a dtype not a kda_dtype value, check_distinct not 0 or
 * 1), KDA_ERR_ALIGN (a weight
 * pointer not aligned to its element size, the state base or stride),
 * KDA_ERR_UNSUPPORTED (conv_width != 4),
 * KDA_ERR_NOMEM, KDA_ERR_HIP. */
kda_status kda_prepare(const kda_weights* w, const kda_caches* c, void* hip_stream,
                       kda_handle* out);

/* One decode step of `batch` requests, one token each ([prepared] run with
 * slots [B] and no accepted counts). Request b reads and writes its state and
 * conv window in place at slot slots[b].
 *   projected : device bf16 [batch][pitch], row b = q|k|v (3D) | gate (D) |
 *               f_a (128) | beta_raw (H) | padding ([prepared] _operands).
 *               pitch >= 4D + 128 + H (any parity); base 2-byte aligned.
 *   slots     : device int32 [batch].
 *   core_out  : device bf16 [batch][D]; base 4-byte aligned.
 * A request whose slot is outside 0 .. num_slots - 1 is skipped entirely (no
 * read, no write, its core_out row untouched) and counted in the device error
 * counter (kda_device_errors); so is, with check_distinct, a request whose
 * slot another request of the call also names. batch == 0 is a no-op.
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE (batch < 0, pitch too small),
 * KDA_ERR_ALIGN, KDA_ERR_DEVICE (called with another device current than the
 * one kda_prepare ran on), KDA_ERR_HIP. */
kda_status kda_decode(kda_handle h, const void* projected, int64_t pitch, int32_t batch,
                      const int32_t* slots, void* core_out, void* hip_stream);

/* One speculative-verify step of `requests` x `tokens` rows ([prepared] run
 * with slots [>= B, q] and accepted [>= B]; [kda] kda tasks: a state written
 * per token). Row r L + t of `projected` / `core_out` is token t of request r.
 *   slots     : device int32; token t of request r writes its state and conv
 *               window to slot slots[r * slots_row_stride + t]
 *               (slots_row_stride >= tokens, so a block-table slice passes
 *               without a copy).
 *   accepted  : device int32 [requests], each in 1 .. tokens: the carried state
 *               and window are read from slot slots[r * slots_row_stride +
 *               accepted[r] - 1], the one written for the last accepted token
 *               of the previous step.
 * Other arguments as kda_decode. tokens in 1 .. KDA_MAX_TOKENS. Invalid slot or
 * accepted values skip the request as in kda_decode. requests == 0 is a no-op.
 * Errors: as kda_decode, plus KDA_ERR_UNSUPPORTED (tokens > 8) and
 * KDA_ERR_SHAPE (tokens < 1, slots_row_stride < tokens). */
kda_status kda_verify(kda_handle h, const void* projected, int64_t pitch, int32_t requests,
                      int32_t tokens, const int32_t* slots, int64_t slots_row_stride,
                      const int32_t* accepted, void* core_out, void* hip_stream);

/* ---- projections around the core ------------------------------------------
 * The dense contraction y = x W^T of an nn.Linear layer without bias: bf16
 * inputs, fp32 accumulation (MFMA), bf16 output rounded to nearest even.
 * One rank's share of the layer's projections on each side of the core:
 *   in_proj  ([kda] module docstring, gemv role: in_proj -> q|k|v|g|f_a|beta):
 *            hidden rows [S][hidden] x W_in [4D + 128 + H][hidden] -> the
 *            packed projection rows [S][pitch] that kda_decode / kda_verify read;
 *   o_proj   (page "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.back",
 *            module docstring: o_proj with K = 1536 local): core_out rows
 *            [S][D] x W_o [hidden][D] -> this rank's partial [S][hidden],
 *            before the tensor-parallel all-reduce (not part of this library).
 * Layouts: x rows x_pitch elements apart, base and rows 16-byte aligned
 * (x_pitch a multiple of 8); W dense [N][K] (the nn.Linear weight), 16-byte
 * aligned, K a multiple of 8; y rows y_pitch >= N elements apart, 2-byte
 * aligned; only columns 0 .. N-1 of each y row are written. All pointers are
 * device pointers borrowed for the call; the call is asynchronous on
 * hip_stream.
 * Workspace: optional device memory (16-byte aligned) of workspace_bytes
 * bytes. For the shapes kda_linear_workspace_bytes answers non-zero (33 to 256
 * rows, K >= 4096 and a multiple of 256), a workspace of at least that size
 * lets the call split K over 4 slices of workgroups: fp32 partial tiles go to
 * the workspace and a second kernel on the same stream adds them in slice
 * order. Its contents are undefined before and after the call; it must not be
 * in use by another call still in flight (stream order is enough). NULL, or
 * too small a size, runs the unsplit kernel.
 * The result is deterministic for a given shape and choice of path (each
 * path sums in a fixed order; the two paths may differ in the last bit).
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE (M < 0 or > 2^20, N < 1, M N > 2^43,
 * K < 8, K not a multiple of 8, a pitch too small), KDA_ERR_ALIGN (also a
 * misaligned workspace),
 * KDA_ERR_HIP. M == 0 is a no-op. */
kda_status kda_linear(const void* x, int64_t x_pitch, const void* w, void* y, int64_t y_pitch,
                      int32_t M, int32_t N, int32_t K, void* workspace, size_t workspace_bytes,
                      void* hip_stream);

/* Bytes of workspace with which kda_linear splits K for this shape; 0 when
 * the shape is never split (or the shape is invalid). Host-only. */
size_t kda_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* Size of the static scratch buffer of kda_linear_noalloc, per GPU. */
#define KDA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/* kda_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the same
 * kernels and results as kda_linear given a workspace of
 * kda_linear_workspace_bytes(M, N, K), with the K split's fp32 partial tiles
 * in a static device buffer of the library instead (KDA_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the library's load until the process ends; enough for
 * in_proj's split up to 256 rows). It calls no allocator. Every call on one
 * GPU shares that GPU's buffer: calls that overlap in time on one GPU (other
 * streams or threads) race and must be serialised by the caller (one stream
 * is enough). Arguments, layouts and errors as kda_linear, plus
 * KDA_ERR_SCRATCH when kda_linear_workspace_bytes(M, N, K) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES (nothing is enqueued then). */
kda_status kda_linear_noalloc(const void* x, int64_t x_pitch, const void* w, void* y,
                              int64_t y_pitch, int32_t M, int32_t N, int32_t K,
                              void* hip_stream);

/* KDA_NOALLOC_SCRATCH_BYTES, as the library was built. Host-only. */
size_t kda_noalloc_scratch_bytes(void);

/* in_proj: N = 4D + 128 + H packed outputs (D = 128 heads), K = hidden;
 * projected rows are `pitch` elements apart (pitch >= N). Workspace as for
 * kda_linear with that N and K. */
kda_status kda_in_proj(const void* x, int64_t x_pitch, const void* w_in, void* projected,
                       int64_t pitch, int32_t rows, int32_t hidden, int32_t heads,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* o_proj: N = hidden, K = D = 128 heads; core rows `core_pitch` elements
 * apart (core_pitch >= D, a multiple of 8), out rows `out_pitch` apart.
 * Workspace as for kda_linear with that N and K. */
kda_status kda_o_proj(const void* core, int64_t core_pitch, const void* w_o, void* out,
                      int64_t out_pitch, int32_t rows, int32_t heads, int32_t hidden,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* Number of requests skipped for an out-of-range slot or accepted count since
 * the last read. Waits for `hip_stream`, copies the counter to *count_out and
 * resets it to zero. Errors: KDA_ERR_NULL, KDA_ERR_DEVICE, KDA_ERR_HIP. */
kda_status kda_device_errors(kda_handle h, int32_t* count_out, void* hip_stream);

/* Frees the handle and its device memory, after waiting for the handle's
 * device (made current for the call; the caller's current device is restored).
 * NULL is a no-op. The borrowed caches are not touched. */
kda_status kda_destroy(kda_handle h);

/* Static description of a status code. */
const char* kda_status_string(kda_status s);

/* The HIP error string of the last KDA_ERR_HIP on this thread, or "". */
const char* kda_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
