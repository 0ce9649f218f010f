/*
 * KDA decode / spec-verify core -- plain sequential CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The GPU library shares no code, header,
 * table or helper with it, and neither side includes or links the other.
 *
 * Page abbreviations used in the citations below:
 *   [kda]      page "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.kda"
 *              (K1 kda_pre: module docstring with the role table, function list)
 *   [prepared] page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.prepared"
 *              (PreparedKda, decode_conv_weight)
 *
 * The pages name the steps and their order ([kda] module docstring, "kda tasks"
 * row: conv update, f_b MFMA + lower-bound gate, l2norm, the recurrence on
 * 16-row state chunks with a state written per token, gated RMSNorm ->
 * core_out) and the operand layout ([prepared] PreparedKda._operands). They
 * print no formula; the formulas below are the plain readings of those steps.
 *
 * Arithmetic: every step is evaluated in IEEE double, in the order written.
 * Values are rounded where they are stored: the recurrent state to fp32
 * (round-to-nearest-even) after every token, core_out to bf16 (RNE), conv
 * windows copied exactly (they hold bf16 inputs). Carrying the fp32-rounded
 * state makes a verify call over L tokens equal L chained decode calls bit
 * for bit.
 *
 * Two rounding modes. Fused (handoff_bf16 = 0): nothing else is rounded.
 * Hand-off (handoff_bf16 = 1): three values that an unfused stack of kernels
 * would pass to the next kernel as bf16 tensors are rounded to bf16 (RNE)
 * where they are produced -- the conv + SiLU outputs q|k|v, g1 = f_b f_a, and
 * the recurrence output o ([kda] module docstring, the sentence on rounding:
 * the fused kernels round as the unfused ones did wherever those exchanged
 * bf16 data).
 *
 * Destination slots. Each (request, token) of a call writes its own slot; a
 * slot named twice in one call has no defined result, so such a call is
 * rejected, or, when the problem asks for it (check_distinct), every request
 * involved is skipped and counted like a request with an invalid index.
 *
 * kda_ref_run is the definition. kda_ref_handoff_ties, further down, is
 * checker instrumentation for the hand-off mode's parity bars: it replays a
 * call read-only and counts values that lie near a bf16 rounding boundary.
 *
 * Parity status: every step has a pin in the CPU tests (closed forms,
 * invariants, library routines, brute force). Parity unpinned: three readings
 * that no printed value fixes -- the l2norm epsilon (1e-6 inside the square
 * root), the norm weight shared by all heads, and which three values the
 * hand-off mode rounds -- rest on this build's reading of the pages alone.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_REF_HEAD_DIM 128 /* dk = dv = 128 ([prepared] PreparedKda.__init__: dim = 128 * heads) */
#define KDA_REF_FA_RANK 128  /* f_a columns ([prepared] _operands: projected[:, 4d : 4d + 128]) */

/* ---------------------------------------------------------------------- */
/* Number formats                                                          */
/* ---------------------------------------------------------------------- */

double kda_ref_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Direct round-to-nearest-even of a double to bf16 (8 significant bits,
 * fp32's exponent range, subnormals kept). No intermediate float rounding. */
uint16_t kda_ref_double_to_bf16(double x)
{
    if (isnan(x)) return (uint16_t)0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7f80);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    int qexp = e - 8;                   /* quantum of an 8-bit significand */
    if (qexp < -133) qexp = -133;       /* bf16 subnormal quantum 2^-133 */
    double q = ldexp(1.0, qexp);
    double r = nearbyint(a / q) * q;    /* a / q exact; nearbyint ties to even */
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (r > bf16_max) return (uint16_t)(sign | 0x7f80);
    float f = (float)r;                 /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7fff));
}

/* ---------------------------------------------------------------------- */
/* Step functions (double in, double out)                                  */
/* ---------------------------------------------------------------------- */

/* Logistic sigmoid, written as 1 / (1 + e^-x) so that large |x| saturates to
 * 0 or 1 without overflow. */
double kda_ref_sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/* Causal short-conv update of one token for C channels, then SiLU
 * ([kda] module docstring, kda tasks: "conv update of the owned channels";
 * function kda_conv: the spec conv update of a request's L tokens).
 *
 * w is the nn.Conv1d weight [C][1][W] read as [C][W] ([prepared]
 * decode_conv_weight takes the [3 * D, 1, width] weight). nn.Conv1d is a
 * cross-correlation: with left padding W - 1, tap j multiplies the input
 * W - 1 - j steps back, so tap W - 1 is the current input x and taps
 * 0 .. W - 2 the cached window, oldest first.
 *
 * win is [C][W - 1], oldest input first; it is shifted in place to hold the
 * last W - 1 inputs including x. bias may be NULL (no conv bias: zero). */
void kda_ref_conv_token(int32_t C, int32_t W, const double* w, const double* bias,
                        double* win, const double* x, double* y)
{
    for (int32_t c = 0; c < C; ++c) {
        const double* wc = w + (int64_t)c * W;
        double* wn = win + (int64_t)c * (W - 1);
        double pre = bias ? bias[c] : 0.0;
        for (int32_t m = 0; m < W - 1; ++m) pre += wc[m] * wn[m];
        pre += wc[W - 1] * x[c];
        y[c] = pre * kda_ref_sigmoid(pre);           /* SiLU */
        for (int32_t m = 0; m + 1 < W - 1; ++m) wn[m] = wn[m + 1];
        if (W > 1) wn[W - 2] = x[c];
    }
}

/* Channel-wise decay gate of one token for all H heads ([kda] kda tasks:
 * "f_b MFMA + lower-bound gate"; function kda_gates: g1 = f_b f_a).
 *   g1[i] = sum_m f_b[i][m] * f_a[m]               (f_b is [D][128])
 *   g[i]  = lb * sigmoid(exp(A_log[i / 128]) * (g1[i] + dt_bias[i]))
 * A_log has one value per head ([prepared] PreparedKda.__init__: heads =
 * A_log.numel()); dt_bias has one per channel. With round_g1, g1 is rounded
 * to bf16 before the gate (the hand-off mode). */
void kda_ref_gate(int32_t H, const double* f_b, const double* f_a, const double* A_log,
                  const double* dt_bias, double lb, int32_t round_g1, double* g)
{
    const int32_t D = H * KDA_REF_HEAD_DIM;
    for (int32_t i = 0; i < D; ++i) {
        double g1 = 0.0;
        for (int32_t m = 0; m < KDA_REF_FA_RANK; ++m)
            g1 += f_b[(int64_t)i * KDA_REF_FA_RANK + m] * f_a[m];
        if (round_g1) g1 = kda_ref_bf16_to_double(kda_ref_double_to_bf16(g1));   /* hand-off */
        double a = exp(A_log[i / KDA_REF_HEAD_DIM]);
        g[i] = lb * kda_ref_sigmoid(a * (g1 + dt_bias[i]));
    }
}

/* l2 normalisation with the epsilon inside the square root, then a scale
 * ([kda] kda tasks: "l2norm"; the 128^-0.5 q scale is the second of the
 * scalars in [prepared] PreparedKda.__init__):
 *   out = x * scale / sqrt(sum x^2 + eps). With eps > 0 a zero vector maps to
 * zero (the GPU library rejects eps <= 0). */
void kda_ref_l2norm(int32_t n, const double* x, double eps, double scale, double* out)
{
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int32_t i = 0; i < n; ++i) out[i] = x[i] * inv * scale;
}

/* One token of the gated delta rule on one head's state ([kda] kda tasks:
 * "the recurrence on 16 state rows"; function kda_recur: state rows of head
 * h, the recurrence over the L tokens).
 *
 * Storage: S is [dv][dk], row j = value channel j (the pages split the state
 * into 16-row v-chunks), column i = key channel i. In matrix terms, with
 * M = S^T ([dk][dv]):  M <- diag(e^g) M;  M <- M + beta k (v - M^T k)^T;
 * o = M^T q. Row by row, in that order:
 *   S[j][i] *= exp(g[i])
 *   u = v[j] - sum_i S[j][i] k[i]
 *   S[j][i] += (beta * u) * k[i]
 *   o[j] = sum_i S[j][i] q[i]                                            */
void kda_ref_recur_token(int32_t dk, int32_t dv, double* S, const double* g, const double* k,
                         const double* q, const double* v, double beta, double* o)
{
    for (int32_t j = 0; j < dv; ++j) {
        double* row = S + (int64_t)j * dk;
        for (int32_t i = 0; i < dk; ++i) row[i] *= exp(g[i]);
        double kS = 0.0;
        for (int32_t i = 0; i < dk; ++i) kS += row[i] * k[i];
        double bu = beta * (v[j] - kS);
        for (int32_t i = 0; i < dk; ++i) row[i] += bu * k[i];
        double acc = 0.0;
        for (int32_t i = 0; i < dk; ++i) acc += row[i] * q[i];
        o[j] = acc;
    }
}

/* Head-wise gated RMSNorm of one head's n outputs ([kda] kda tasks: "gated
 * RMSNorm -> core_out"; function kda_norm: over the head's 128):
 *   rstd = 1 / sqrt(mean_j o[j]^2 + eps);  y[j] = o[j] * rstd * w[j] * sigmoid(gate[j]) */
void kda_ref_gated_rmsnorm(int32_t n, const double* o, const double* gate, const double* w,
                           double eps, double* y)
{
    double ss = 0.0;
    for (int32_t j = 0; j < n; ++j) ss += o[j] * o[j];
    double rstd = 1.0 / sqrt(ss / (double)n + eps);
    for (int32_t j = 0; j < n; ++j) y[j] = o[j] * rstd * w[j] * kda_ref_sigmoid(gate[j]);
}

/* ---------------------------------------------------------------------- */
/* One decode or verify call                                               */
/* ---------------------------------------------------------------------- */

typedef struct {
    int32_t heads;              /* H; head dim 128, D = 128 H */
    int32_t width;              /* conv taps W (>= 1) */
    int32_t requests;           /* R */
    int32_t tokens;             /* L tokens a request; S = R L rows */
    const uint16_t* projected;  /* bf16 [S][pitch]: q|k|v (3D), gate (D), f_a (128), beta (H) */
    int64_t pitch;              /* elements */
    const int32_t* slots;       /* slots[r * slots_row_stride + t] */
    int64_t slots_row_stride;
    const int32_t* accepted;    /* [R] in 1..L (verify), or NULL (decode: L == 1) */
    int32_t num_slots;
    uint16_t* conv;             /* bf16 conv-window pool, element strides below */
    int64_t conv_slot_stride, conv_dim_stride, conv_pos_stride;
    float* state;               /* fp32 [num_slots][slot stride]; [h][v][k] within a slot */
    int64_t state_slot_stride;
    const uint16_t* conv_weight;/* bf16 [3D][1][W] (nn.Conv1d layout) */
    const uint16_t* conv_bias;  /* bf16 [3D], or NULL */
    const uint16_t* f_b;        /* bf16 [D][128] */
    const float* A_log;         /* [H] */
    const float* dt_bias;       /* [D] */
    const float* norm_weight;   /* [128] shared (stride 0) or [H][128] (stride 128) */
    int32_t norm_head_stride;
    double gate_lower_bound;
    double q_scale;             /* 128^-0.5 */
    double norm_eps;
    double l2_eps;
    uint16_t* core_out;         /* bf16 [S][D] */
    double* core_out_f64;       /* optional [S][D]: the value before the bf16 rounding */
    int32_t handoff_bf16;       /* 0 fused; 1 bf16 hand-offs (conv out, g1, o) */
    int32_t check_distinct;     /* 0: a repeated destination makes the call undefined (-1);
                                   1: requests with a repeated destination are skipped */
} kda_ref_problem;

/* Slot resolution ([prepared] PreparedKda.run and _operands: slots [B] for a
 * decode step; slots [>= B, q] with accepted [>= B] for a verify step).
 * Decode: the state is read and written in place at slots[r]. Verify: the
 * carried state is the one written for the last accepted token of the
 * previous step, slots[r][accepted[r] - 1]; token t writes slots[r][t].
 * Returns 0 when every index is in range, else -1 (the request is skipped). */
static int resolve_slots(const kda_ref_problem* p, int32_t r, int32_t* src, int32_t* dst)
{
    const int32_t L = p->tokens;
    const int32_t* row = p->slots + (int64_t)r * p->slots_row_stride;
    for (int32_t t = 0; t < L; ++t) {
        dst[t] = row[t];
        if (dst[t] < 0 || dst[t] >= p->num_slots) return -1;
    }
    if (p->accepted == NULL) {
        *src = dst[0];
    } else {
        int32_t a = p->accepted[r];
        if (a < 1 || a > L) return -1;
        *src = row[a - 1];
    }
    return 0;
}

/* Destination collisions. A call writes one state and one conv window per
 * (request, token) to the slot the slots operand names; the pages give each
 * token of each request its own slot ([prepared] run: a block-table slice of
 * distinct cache lines), and a slot named twice in one call would receive two
 * writes with no order between them. collide[r] is set for every request
 * whose indices are all valid and one of whose destination slots is named
 * more than once by such requests (twice in its own row included). Returns
 * how many requests collide, or -1 when out of memory. */
static int32_t find_collisions(const kda_ref_problem* p, int32_t* collide)
{
    const int32_t R = p->requests, L = p->tokens;
    int32_t* count = calloc((size_t)p->num_slots, sizeof(int32_t));
    int32_t* dst = malloc(sizeof(int32_t) * (size_t)L);
    if (count == NULL || dst == NULL) { free(count); free(dst); return -1; }
    int32_t src;
    for (int32_t r = 0; r < R; ++r)
        if (resolve_slots(p, r, &src, dst) == 0)
            for (int32_t t = 0; t < L; ++t) ++count[dst[t]];
    int32_t n = 0;
    for (int32_t r = 0; r < R; ++r) {
        collide[r] = 0;
        if (resolve_slots(p, r, &src, dst) != 0) continue;
        for (int32_t t = 0; t < L; ++t)
            if (count[dst[t]] > 1) collide[r] = 1;
        n += collide[r];
    }
    free(count);
    free(dst);
    return n;
}

/* The whole-problem checks kda_ref_run and kda_ref_handoff_ties share. */
static int problem_ok(const kda_ref_problem* p)
{
    const int32_t H = p->heads, W = p->width, R = p->requests, L = p->tokens;
    if (H <= 0 || W < 1 || R < 0 || L < 1 || p->pitch < 0 || p->num_slots < 0) return 0;
    if (p->accepted == NULL && L != 1) return 0;
    return p->pitch >= 4 * (int64_t)H * KDA_REF_HEAD_DIM + KDA_REF_FA_RANK + H;
}

/* Runs one call. The conv and state pools are updated in place; core_out rows
 * of skipped requests are left untouched. Returns the number of skipped
 * requests (an index out of range, or with check_distinct a repeated
 * destination), or -1 on an invalid problem -- a repeated destination
 * without check_distinct included, in which case nothing is written. */
int32_t kda_ref_run(const kda_ref_problem* p)
{
    if (!problem_ok(p)) return -1;
    const int32_t H = p->heads, W = p->width, R = p->requests, L = p->tokens;
    const int32_t N = KDA_REF_HEAD_DIM, D = H * N, C = 3 * D;

    int32_t* collide = malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
    if (collide == NULL) return -1;
    const int32_t n_collide = find_collisions(p, collide);
    if (n_collide < 0 || (n_collide > 0 && !p->check_distinct)) {
        free(collide);
        return -1;
    }

    /* Weights in double, nn.Conv1d weight [C][1][W] read as [C][W]. */
    double* w = malloc(sizeof(double) * (size_t)C * W);
    double* b = p->conv_bias ? malloc(sizeof(double) * (size_t)C) : NULL;
    double* fb = malloc(sizeof(double) * (size_t)D * KDA_REF_FA_RANK);
    double* alog = malloc(sizeof(double) * (size_t)H);
    double* dtb = malloc(sizeof(double) * (size_t)D);
    double* nw = malloc(sizeof(double) * (size_t)H * N);
    double* win = malloc(sizeof(double) * (size_t)C * (W > 1 ? W - 1 : 1));
    double* S = malloc(sizeof(double) * (size_t)H * N * N);
    double* x = malloc(sizeof(double) * (size_t)p->pitch);
    double* y = malloc(sizeof(double) * (size_t)C);
    double* g = malloc(sizeof(double) * (size_t)D);
    double* qh = malloc(sizeof(double) * (size_t)N);
    double* kh = malloc(sizeof(double) * (size_t)N);
    double* o = malloc(sizeof(double) * (size_t)N);
    double* gate = malloc(sizeof(double) * (size_t)N);
    double* yo = malloc(sizeof(double) * (size_t)N);
    int32_t* dst = malloc(sizeof(int32_t) * (size_t)L);
    const int hand = p->handoff_bf16 != 0;
    for (int64_t i = 0; i < (int64_t)C * W; ++i) w[i] = kda_ref_bf16_to_double(p->conv_weight[i]);
    if (b)
        for (int32_t c = 0; c < C; ++c) b[c] = kda_ref_bf16_to_double(p->conv_bias[c]);
    for (int64_t i = 0; i < (int64_t)D * KDA_REF_FA_RANK; ++i) fb[i] = kda_ref_bf16_to_double(p->f_b[i]);
    for (int32_t h = 0; h < H; ++h) alog[h] = (double)p->A_log[h];
    for (int32_t i = 0; i < D; ++i) dtb[i] = (double)p->dt_bias[i];
    for (int32_t h = 0; h < H; ++h)
        for (int32_t j = 0; j < N; ++j)
            nw[(int64_t)h * N + j] = (double)p->norm_weight[(int64_t)h * p->norm_head_stride + j];

    int32_t skipped = 0;
    for (int32_t r = 0; r < R; ++r) {
        int32_t src;
        if (resolve_slots(p, r, &src, dst) != 0 || collide[r]) { ++skipped; continue; }

        /* Read the carried conv window and state before any write. */
        for (int32_t c = 0; c < C; ++c)
            for (int32_t m = 0; m < W - 1; ++m)
                win[(int64_t)c * (W - 1) + m] = kda_ref_bf16_to_double(
                    p->conv[src * p->conv_slot_stride + c * p->conv_dim_stride + m * p->conv_pos_stride]);
        for (int64_t e = 0; e < (int64_t)H * N * N; ++e)
            S[e] = (double)p->state[src * p->state_slot_stride + e];

        for (int32_t t = 0; t < L; ++t) {
            const int64_t row = (int64_t)r * L + t;
            const uint16_t* xr = p->projected + row * p->pitch;
            for (int64_t e = 0; e < p->pitch; ++e) x[e] = kda_ref_bf16_to_double(xr[e]);

            /* conv update + SiLU over q|k|v; the new window goes to dst[t] */
            kda_ref_conv_token(C, W, w, b, win, x, y);
            if (hand)
                for (int32_t c = 0; c < C; ++c)
                    y[c] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(y[c]));   /* hand-off */
            for (int32_t c = 0; c < C; ++c)
                for (int32_t m = 0; m < W - 1; ++m)
                    p->conv[dst[t] * p->conv_slot_stride + c * p->conv_dim_stride + m * p->conv_pos_stride] =
                        kda_ref_double_to_bf16(win[(int64_t)c * (W - 1) + m]);

            /* decay gate from f_a = projected[4D : 4D + 128] */
            kda_ref_gate(H, fb, x + 4 * (int64_t)D, alog, dtb, p->gate_lower_bound, hand, g);

            for (int32_t h = 0; h < H; ++h) {
                /* beta = sigmoid(projected[4D + 128 + h]), one per (token, head) */
                double beta = kda_ref_sigmoid(x[4 * (int64_t)D + KDA_REF_FA_RANK + h]);
                kda_ref_l2norm(N, y + (int64_t)h * N, p->l2_eps, p->q_scale, qh);
                kda_ref_l2norm(N, y + D + (int64_t)h * N, p->l2_eps, 1.0, kh);
                const double* v = y + 2 * (int64_t)D + (int64_t)h * N;
                double* Sh = S + (int64_t)h * N * N;
                kda_ref_recur_token(N, N, Sh, g + (int64_t)h * N, kh, qh, v, beta, o);
                if (hand)
                    for (int32_t j = 0; j < N; ++j)
                        o[j] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(o[j]));   /* hand-off */

                /* the state written for this token, rounded to fp32 and carried */
                float* out_state = p->state + dst[t] * p->state_slot_stride + (int64_t)h * N * N;
                for (int64_t e = 0; e < (int64_t)N * N; ++e) {
                    float f = (float)Sh[e];
                    out_state[e] = f;
                    Sh[e] = (double)f;
                }

                /* gated RMSNorm with gate = projected[3D + 128 h + j] */
                for (int32_t j = 0; j < N; ++j) gate[j] = x[3 * (int64_t)D + (int64_t)h * N + j];
                kda_ref_gated_rmsnorm(N, o, gate, nw + (int64_t)h * N, p->norm_eps, yo);
                for (int32_t j = 0; j < N; ++j) {
                    int64_t oi = row * D + (int64_t)h * N + j;
                    p->core_out[oi] = kda_ref_double_to_bf16(yo[j]);
                    if (p->core_out_f64) p->core_out_f64[oi] = yo[j];
                }
            }
        }
    }

    free(w); free(b); free(fb); free(alog); free(dtb); free(nw); free(win); free(S); free(x);
    free(y); free(g); free(qh); free(kh); free(o); free(gate); free(yo); free(dst); free(collide);
    return skipped;
}

/* ---------------------------------------------------------------------- */
/* Near ties of the hand-off mode (checker instrumentation, not the method) */
/* ---------------------------------------------------------------------- */

/* Another implementation computes each value it rounds to bf16 in its own
 * precision, so where the value lies close to a bf16 rounding boundary its
 * rounding can differ from the oracle's. Given a margin m for a value x (a
 * bound on that implementation's error in x), x counts as a near tie when
 * x - m and x + m round to different bf16 values. Margins are a relative
 * factor times a magnitude:
 *   conv out y = SiLU(pre):  |SiLU'(pre)| (|bias| + sum |w * input|) + (1 + |pre|) |y|
 *       (the pre-activation's rounding scaled by the slope, plus SiLU's own
 *       evaluation, whose exponential sees an argument rounded relative to |pre|);
 *   g1 = sum_m f_b[m] f_a[m]:  sum |f_b f_a|, or zero when every term is a
 *       multiple of one quantum Q and the sum of |terms| is at most 2^24 Q
 *       (then every fp32 summation order is exact);
 *   o:  sum_i |S_dec q_i| + |beta| (|v| + sum_i |S_dec k_i|) sum_i |k_i q_i|,
 *       S_dec the decayed state row;
 *   core_out value y:  |y|. */

static int near_tie(double x, double m)
{
    return m > 0.0 && kda_ref_double_to_bf16(x - m) != kda_ref_double_to_bf16(x + m);
}

/* The lowest set bit of a nonzero double: |a| = M 2^k with M odd gives 2^k. */
static double lowest_bit(double a)
{
    int e;
    double m = frexp(fabs(a), &e);      /* |a| = m 2^e, m in [0.5, 1) */
    int64_t M = (int64_t)ldexp(m, 53);  /* exact: 53 significant bits */
    int k = e - 53;
    while ((M & 1) == 0) { M >>= 1; ++k; }
    return ldexp(1.0, k);
}

/* Margin of g1 = sum_m f_b[m] f_a[m] for an fp32 implementation: zero when
 * the sum is exact in fp32 in any order, else rel * sum |terms|. */
static double g1_margin(const double* fbrow, const double* fa, double rel)
{
    double mag = 0.0, q = INFINITY;
    for (int32_t m = 0; m < KDA_REF_FA_RANK; ++m) {
        const double t = fbrow[m] * fa[m];
        if (t == 0.0) continue;
        mag += fabs(t);
        const double qt = lowest_bit(fbrow[m]) * lowest_bit(fa[m]);
        if (qt < q) q = qt;
    }
    if (mag == 0.0 || mag <= ldexp(q, 24)) return 0.0;
    return rel * mag;
}

/* Counts, per (request, head), the near ties among the values that the
 * hand-off mode rounds -- conv out, g1, o -- and among core_out, under the
 * relative margins rel[0..3] (conv, g1, o, core_out). ties is [R][H][4],
 * zeroed by the caller. The call is the one kda_ref_run(p) performs with
 * handoff_bf16 = 1, replayed with the same step functions on private copies:
 * the pools are only read, so this runs before kda_ref_run on the same
 * problem. Returns what kda_ref_run would (skipped count, or -1). */
int32_t kda_ref_handoff_ties(const kda_ref_problem* p, const double* rel, int32_t* ties)
{
    if (!problem_ok(p)) return -1;
    const int32_t H = p->heads, W = p->width, R = p->requests, L = p->tokens;
    const int32_t N = KDA_REF_HEAD_DIM, D = H * N, C = 3 * D;

    int32_t* collide = malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
    if (collide == NULL) return -1;
    const int32_t n_collide = find_collisions(p, collide);
    if (n_collide < 0 || (n_collide > 0 && !p->check_distinct)) {
        free(collide);
        return -1;
    }

    double* w = malloc(sizeof(double) * (size_t)C * W);
    double* b = p->conv_bias ? malloc(sizeof(double) * (size_t)C) : NULL;
    double* fb = malloc(sizeof(double) * (size_t)D * KDA_REF_FA_RANK);
    double* alog = malloc(sizeof(double) * (size_t)H);
    double* dtb = malloc(sizeof(double) * (size_t)D);
    double* nw = malloc(sizeof(double) * (size_t)H * N);
    double* win = malloc(sizeof(double) * (size_t)C * (W > 1 ? W - 1 : 1));
    double* S = malloc(sizeof(double) * (size_t)H * N * N);
    double* x = malloc(sizeof(double) * (size_t)p->pitch);
    double* y = malloc(sizeof(double) * (size_t)C);
    double* g = malloc(sizeof(double) * (size_t)D);
    double* qh = malloc(sizeof(double) * (size_t)N);
    double* kh = malloc(sizeof(double) * (size_t)N);
    double* o = malloc(sizeof(double) * (size_t)N);
    double* gate = malloc(sizeof(double) * (size_t)N);
    double* yo = malloc(sizeof(double) * (size_t)N);
    double* cmag = malloc(sizeof(double) * (size_t)C);
    double* omag = malloc(sizeof(double) * (size_t)N);
    int32_t* dst = malloc(sizeof(int32_t) * (size_t)L);
    for (int64_t i = 0; i < (int64_t)C * W; ++i) w[i] = kda_ref_bf16_to_double(p->conv_weight[i]);
    if (b)
        for (int32_t c = 0; c < C; ++c) b[c] = kda_ref_bf16_to_double(p->conv_bias[c]);
    for (int64_t i = 0; i < (int64_t)D * KDA_REF_FA_RANK; ++i) fb[i] = kda_ref_bf16_to_double(p->f_b[i]);
    for (int32_t h = 0; h < H; ++h) alog[h] = (double)p->A_log[h];
    for (int32_t i = 0; i < D; ++i) dtb[i] = (double)p->dt_bias[i];
    for (int32_t h = 0; h < H; ++h)
        for (int32_t j = 0; j < N; ++j)
            nw[(int64_t)h * N + j] = (double)p->norm_weight[(int64_t)h * p->norm_head_stride + j];

    int32_t skipped = 0;
    for (int32_t r = 0; r < R; ++r) {
        int32_t src;
        if (resolve_slots(p, r, &src, dst) != 0 || collide[r]) { ++skipped; continue; }
        int32_t* tr = ties + (int64_t)r * H * 4;
        for (int32_t c = 0; c < C; ++c)
            for (int32_t m = 0; m < W - 1; ++m)
                win[(int64_t)c * (W - 1) + m] = kda_ref_bf16_to_double(
                    p->conv[src * p->conv_slot_stride + c * p->conv_dim_stride + m * p->conv_pos_stride]);
        for (int64_t e = 0; e < (int64_t)H * N * N; ++e)
            S[e] = (double)p->state[src * p->state_slot_stride + e];

        for (int32_t t = 0; t < L; ++t) {
            const int64_t row = (int64_t)r * L + t;
            const uint16_t* xr = p->projected + row * p->pitch;
            for (int64_t e = 0; e < p->pitch; ++e) x[e] = kda_ref_bf16_to_double(xr[e]);

            /* conv out: margins from the window before this token's shift */
            for (int32_t c = 0; c < C; ++c) {
                double mg = b ? fabs(b[c]) : 0.0, pre = b ? b[c] : 0.0;
                for (int32_t m = 0; m < W - 1; ++m) {
                    const double term = w[(int64_t)c * W + m] * win[(int64_t)c * (W - 1) + m];
                    mg += fabs(term);
                    pre += term;
                }
                const double term = w[(int64_t)c * W + W - 1] * x[c];
                mg += fabs(term);
                pre += term;
                const double sg = kda_ref_sigmoid(pre);
                const double slope = sg * (1.0 + pre * (1.0 - sg));   /* SiLU'(pre) */
                cmag[c] = fabs(slope) * mg + (1.0 + fabs(pre)) * fabs(pre * sg);
            }
            kda_ref_conv_token(C, W, w, b, win, x, y);
            for (int32_t c = 0; c < C; ++c) {
                if (near_tie(y[c], rel[0] * cmag[c])) ++tr[((c % D) / N) * 4 + 0];
                y[c] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(y[c]));
            }

            /* g1 */
            const double* fa = x + 4 * (int64_t)D;
            for (int32_t i = 0; i < D; ++i) {
                const double* fbrow = fb + (int64_t)i * KDA_REF_FA_RANK;
                double g1 = 0.0;
                for (int32_t m = 0; m < KDA_REF_FA_RANK; ++m) g1 += fbrow[m] * fa[m];
                if (near_tie(g1, g1_margin(fbrow, fa, rel[1]))) ++tr[(i / N) * 4 + 1];
            }
            kda_ref_gate(H, fb, fa, alog, dtb, p->gate_lower_bound, 1, g);

            for (int32_t h = 0; h < H; ++h) {
                double beta = kda_ref_sigmoid(x[4 * (int64_t)D + KDA_REF_FA_RANK + h]);
                kda_ref_l2norm(N, y + (int64_t)h * N, p->l2_eps, p->q_scale, qh);
                kda_ref_l2norm(N, y + D + (int64_t)h * N, p->l2_eps, 1.0, kh);
                const double* v = y + 2 * (int64_t)D + (int64_t)h * N;
                double* Sh = S + (int64_t)h * N * N;
                const double* gh = g + (int64_t)h * N;
                double kq = 0.0;
                for (int32_t i = 0; i < N; ++i) kq += fabs(kh[i] * qh[i]);
                for (int32_t j = 0; j < N; ++j) {
                    double aq = 0.0, ak = 0.0;
                    for (int32_t i = 0; i < N; ++i) {
                        const double sd = Sh[(int64_t)j * N + i] * exp(gh[i]);
                        aq += fabs(sd * qh[i]);
                        ak += fabs(sd * kh[i]);
                    }
                    omag[j] = aq + fabs(beta) * (fabs(v[j]) + ak) * kq;
                }
                kda_ref_recur_token(N, N, Sh, gh, kh, qh, v, beta, o);
                for (int32_t j = 0; j < N; ++j) {
                    if (near_tie(o[j], rel[2] * omag[j])) ++tr[h * 4 + 2];
                    o[j] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(o[j]));
                }
                for (int64_t e = 0; e < (int64_t)N * N; ++e) Sh[e] = (double)(float)Sh[e];
                for (int32_t j = 0; j < N; ++j) gate[j] = x[3 * (int64_t)D + (int64_t)h * N + j];
                kda_ref_gated_rmsnorm(N, o, gate, nw + (int64_t)h * N, p->norm_eps, yo);
                for (int32_t j = 0; j < N; ++j)
                    if (near_tie(yo[j], rel[3] * fabs(yo[j]))) ++tr[h * 4 + 3];
            }
        }
    }

    free(w); free(b); free(fb); free(alog); free(dtb); free(nw); free(win); free(S); free(x);
    free(y); free(g); free(qh); free(kh); free(o); free(gate); free(yo); free(cmag); free(omag);
    free(dst); free(collide);
    return skipped;
}

/* ---------------------------------------------------------------------- */
/* Projections around the core (in_proj before it, o_proj after it)       */
/* ---------------------------------------------------------------------- */

/* y[m][n] = sum_k x[m][k] * w[n][k] for the rows of `rows` (or all M rows
 * when rows == NULL), in double, k ascending; the nn.Linear weight layout
 * [N][K] ([kda] module docstring, gemv role: in_proj -> q|k|v|g|f_a|beta;
 * page "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.back",
 * module docstring: o_proj with K = 1536 local). x rows are x_pitch apart,
 * y rows y_pitch apart; y gets bf16 (round to nearest even from double) and,
 * when y_f64 is not NULL, the unrounded value (y_f64 rows are N apart). */
void kda_ref_linear(int32_t M, int32_t N, int32_t K, const uint16_t* x, int64_t x_pitch,
                    const uint16_t* w, uint16_t* y, int64_t y_pitch, double* y_f64)
{
    double* xr = malloc(sizeof(double) * (size_t)K);
    for (int32_t m = 0; m < M; ++m) {
        for (int32_t k = 0; k < K; ++k) xr[k] = kda_ref_bf16_to_double(x[(int64_t)m * x_pitch + k]);
        for (int32_t n = 0; n < N; ++n) {
            const uint16_t* wr = w + (int64_t)n * K;
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k) acc += xr[k] * kda_ref_bf16_to_double(wr[k]);
            y[(int64_t)m * y_pitch + n] = kda_ref_double_to_bf16(acc);
            if (y_f64) y_f64[(int64_t)m * N + n] = acc;
        }
    }
    free(xr);
}

/* The same contraction for a list of (m, n) entries only (sampled checks at
 * full size): out[i] = sum_k x[ms[i]][k] * w[ns[i]][k], in double. */
void kda_ref_linear_entries(int32_t K, const uint16_t* x, int64_t x_pitch, const uint16_t* w,
                            int32_t count, const int32_t* ms, const int32_t* ns, double* out)
{
    for (int32_t i = 0; i < count; ++i) {
        const uint16_t* xr = x + (int64_t)ms[i] * x_pitch;
        const uint16_t* wr = w + (int64_t)ns[i] * K;
        double acc = 0.0;
        for (int32_t k = 0; k < K; ++k)
            acc += kda_ref_bf16_to_double(xr[k]) * kda_ref_bf16_to_double(wr[k]);
        out[i] = acc;
    }
}
