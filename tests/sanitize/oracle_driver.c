/* Drives the oracle through decode, verify (with skipped requests), repeated
 * destinations (rejected, or skipped when checked), the hand-off mode with its
 * near-tie replay and the projection reference, on small pseudo-random inputs. */
#include <stdlib.h>
#include <stdio.h>
#include <string.h>
#include "kda_oracle.c"

static uint32_t rng_state = 12345u;
static double urand(void) { rng_state = rng_state * 1664525u + 1013904223u; return (rng_state >> 8) * (1.0 / 16777216.0); }
static uint16_t bf(double x) { return kda_ref_double_to_bf16(x); }
static uint16_t* bf_array(size_t n, double scale) {
    uint16_t* a = malloc(n * sizeof *a);
    for (size_t i = 0; i < n; ++i) a[i] = bf((urand() * 2.0 - 1.0) * scale);
    return a;
}
static float* f_array(size_t n, double lo, double hi) {
    float* a = malloc(n * sizeof *a);
    for (size_t i = 0; i < n; ++i) a[i] = (float)(lo + (hi - lo) * urand());
    return a;
}

static int run_case(int H, int R, int L, int verify, int dim_first, int with_bias, int per_head,
                    int handoff, int bad_request, int dup, int check) {
    const int N = 128, D = H * N, C = 3 * D, W = 4, slots_n = R * L + 3;
    const int64_t pitch = 4 * (int64_t)D + 128 + H + 6, S = (int64_t)R * L;
    uint16_t* projected = bf_array((size_t)(S * pitch), 1.0);
    uint16_t* conv = bf_array((size_t)slots_n * C * (W - 1), 1.0);
    float* state = f_array((size_t)slots_n * H * N * N, -0.05, 0.05);
    uint16_t* cw = bf_array((size_t)C * W, 0.5);
    uint16_t* cb = with_bias ? bf_array((size_t)C, 0.1) : NULL;
    uint16_t* fb = bf_array((size_t)D * 128, 0.09);
    float* alog = f_array((size_t)H, -1.0, 1.0);
    float* dtb = f_array((size_t)D, -1.0, 1.0);
    float* nw = f_array((size_t)(per_head ? D : N), 0.5, 1.5);
    int32_t* slots = malloc(sizeof(int32_t) * (size_t)R * (L + 1));
    for (int i = 0; i < R * (L + 1); ++i) slots[i] = i % slots_n;
    int32_t* acc = malloc(sizeof(int32_t) * (size_t)R);
    for (int r = 0; r < R; ++r) acc[r] = 1 + r % L;
    if (bad_request) { if (verify) acc[0] = L + 1; else slots[0] = slots_n + 5; }
    if (dup) slots[2 * (L + 1)] = slots[L + 1];   /* requests 1 and 2 share a destination */
    uint16_t* out = calloc((size_t)(S * D), sizeof *out);
    double* out64 = calloc((size_t)(S * D), sizeof *out64);
    int32_t* ties = calloc((size_t)R * H * 4, sizeof *ties);

    kda_ref_problem p;
    memset(&p, 0, sizeof p);
    p.heads = H; p.width = W; p.requests = R; p.tokens = L;
    p.projected = projected; p.pitch = pitch;
    p.slots = slots; p.slots_row_stride = L + 1; p.accepted = verify ? acc : NULL;
    p.num_slots = slots_n; p.conv = conv;
    p.conv_slot_stride = (int64_t)C * (W - 1);
    p.conv_dim_stride = dim_first ? W - 1 : 1;
    p.conv_pos_stride = dim_first ? 1 : C;
    p.state = state; p.state_slot_stride = (int64_t)H * N * N;
    p.conv_weight = cw; p.conv_bias = cb; p.f_b = fb; p.A_log = alog; p.dt_bias = dtb;
    p.norm_weight = nw; p.norm_head_stride = per_head ? N : 0;
    p.gate_lower_bound = -5.0; p.q_scale = 1.0 / sqrt(128.0); p.norm_eps = 1e-6; p.l2_eps = 1e-6;
    p.core_out = out; p.core_out_f64 = out64;
    p.handoff_bf16 = handoff; p.check_distinct = check;
    const double rel[4] = {1e-6, 1e-6, 1e-6, 1e-6};
    const int32_t expect = dup ? (check ? 2 + bad_request : -1) : bad_request;
    int bad = 0;
    if (handoff) bad |= kda_ref_handoff_ties(&p, rel, ties) != expect;
    const int32_t skipped = kda_ref_run(&p);
    free(projected); free(conv); free(state); free(cw); free(cb); free(fb); free(alog);
    free(dtb); free(nw); free(slots); free(acc); free(out); free(out64); free(ties);
    return bad || skipped != expect;
}

int main(void) {
    int bad = 0;
    bad |= run_case(2, 3, 1, 0, 1, 1, 0, 0, 0, 0, 0);
    bad |= run_case(2, 3, 1, 0, 0, 0, 1, 0, 1, 0, 0);
    bad |= run_case(1, 2, 3, 1, 1, 1, 0, 0, 0, 0, 0);
    bad |= run_case(3, 2, 8, 1, 0, 1, 1, 0, 1, 0, 0);
    bad |= run_case(2, 2, 4, 1, 1, 1, 0, 1, 0, 0, 0);
    bad |= run_case(1, 4, 2, 1, 1, 1, 0, 1, 1, 1, 0);
    bad |= run_case(1, 4, 2, 1, 0, 1, 0, 1, 1, 1, 1);
    bad |= run_case(2, 3, 1, 0, 1, 0, 0, 0, 0, 1, 1);
    {   /* projection reference, with a padded x pitch */
        const int M = 5, Nn = 7, K = 24;
        uint16_t* x = bf_array((size_t)M * (K + 8), 1.0);
        uint16_t* w = bf_array((size_t)Nn * K, 0.2);
        uint16_t* y = calloc((size_t)M * (Nn + 1), sizeof *y);
        double* y64 = calloc((size_t)M * Nn, sizeof *y64);
        int32_t ms[3] = {0, 4, 2}, ns[3] = {6, 0, 3};
        double e[3];
        kda_ref_linear(M, Nn, K, x, K + 8, w, y, Nn + 1, y64);
        kda_ref_linear_entries(K, x, K + 8, w, 3, ms, ns, e);
        for (int i = 0; i < 3; ++i) bad |= e[i] != y64[ms[i] * Nn + ns[i]];
        free(x); free(w); free(y); free(y64);
    }
    printf("oracle under sanitizers: %s\n", bad ? "FAIL" : "ok");
    return bad;
}
