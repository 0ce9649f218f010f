/* Host-side validation of the C ABI, run under AddressSanitizer and UBSan: every call
 * here fails validation before any HIP call, so no GPU is touched. */
#include <stdio.h>
#include <string.h>
#include "kda.h"
#include "kda_probe.h"
int main(void) {
    kda_handle h = 0;
    kda_weights w; kda_caches c;
    memset(&w, 0, sizeof w); memset(&c, 0, sizeof c);
    int bad = 0;
    bad |= kda_prepare(NULL, &c, NULL, &h) != KDA_ERR_NULL;
    w.heads = 2; w.conv_width = 4; w.conv_weight = (void*)0x10000; w.f_b = (void*)0x10000;
    w.A_log = (void*)0x10000; w.dt_bias = (void*)0x10000; w.norm_weight = (void*)0x10000;
    w.norm_eps = 1e-6f; w.l2_eps = 1e-6f;
    c.conv = (void*)0x20000; c.state = (float*)0x40000; c.num_slots = 4;
    c.conv_slot_stride = 9 * 256; c.conv_dim_stride = 3; c.conv_pos_stride = 1;
    c.state_slot_stride = 2 * 128 * 128;
    w.conv_width = 3; bad |= kda_prepare(&w, &c, NULL, &h) != KDA_ERR_UNSUPPORTED; w.conv_width = 4;
    w.rounding = 7; bad |= kda_prepare(&w, &c, NULL, &h) != KDA_ERR_SHAPE; w.rounding = 0;
    w.l2_eps = 0.0f; bad |= kda_prepare(&w, &c, NULL, &h) != KDA_ERR_SHAPE; w.l2_eps = 1e-6f;
    c.check_distinct = 3; bad |= kda_prepare(&w, &c, NULL, &h) != KDA_ERR_SHAPE; c.check_distinct = 0;
    c.state = (float*)0x40004; bad |= kda_prepare(&w, &c, NULL, &h) != KDA_ERR_ALIGN;
    bad |= h != 0;
    bad |= kda_decode(NULL, (void*)0x1000, 1154, 1, (void*)0x2000, (void*)0x3000, NULL) != KDA_ERR_NULL;
    bad |= kda_verify(NULL, (void*)0x1000, 1154, 1, 4, (void*)0x2000, 4, (void*)0x4000, (void*)0x3000, NULL) != KDA_ERR_NULL;
    bad |= kda_linear((void*)0x1000, 64, (void*)0x2000, (void*)0x3000, 16, -1, 16, 64, NULL, 0, NULL) != KDA_ERR_SHAPE;
    bad |= kda_linear((void*)0x1008, 64, (void*)0x2000, (void*)0x3000, 16, 4, 16, 64, NULL, 0, NULL) != KDA_ERR_ALIGN;
    bad |= kda_linear_workspace_bytes(64, 6284, 7168) != 4u * 50 * 64 * 128 * 4;
    bad |= kda_linear_noalloc((void*)0x1000, 4096, (void*)0x2000, (void*)0x3000, 40000, 256,
                              40000, 4096, NULL) != KDA_ERR_SCRATCH;
    bad |= kda_linear_noalloc(NULL, 64, (void*)0x2000, (void*)0x3000, 16, 4, 16, 64, NULL) != KDA_ERR_NULL;
    bad |= kda_noalloc_scratch_bytes() != KDA_NOALLOC_SCRATCH_BYTES;
    bad |= kda_probe_copy(NULL, (void*)0x1000, 16, NULL) != KDA_ERR_NULL;
    for (int s = 0; s >= -9; --s) bad |= kda_status_string((kda_status)s) == NULL;
    bad |= strlen(kda_last_hip_error()) != 0;
    bad |= kda_destroy(NULL) != KDA_OK;
    printf("host validation under sanitizers: %s\n", bad ? "FAIL" : "ok");
    return bad;
}
