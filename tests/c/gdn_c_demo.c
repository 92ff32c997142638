/*
 * gdn_c_demo.c -- the library driven from plain C: device buffers from
 * hipMalloc, every call through include/gdn.h, no Python and no torch.
 *
 * One value head (NV = NK = 1) at D = 4 from a zero state.  The token's inputs
 * come from the command line: k[4] q[4] v[4] alpha beta gn[4] z[4] eps.  The
 * program prints, one line each, the raw o of gdn_decode and the state's key
 * column 0 after it, then y of gdn_decode_norm (from a fresh zero state), and
 * the status names of two calls the library must reject before any launch.
 * The expected values are the test's to check.
 *
 * Build (the package's build step does this):
 *   gcc -std=c11 -O2 -D__HIP_PLATFORM_AMD__ -I include -I /opt/rocm/include \
 *       tests/c/gdn_c_demo.c -o tests/c/gdn_c_demo \
 *       -L gated_deltanet_decode_delta_amd -lgdn -L /opt/rocm/lib -lamdhip64 \
 *       -Wl,-rpath,'$ORIGIN/../../gated_deltanet_decode_delta_amd' -Wl,-rpath,/opt/rocm/lib
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

#define D 4

static int hip_ok(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 0;
    }
    return 1;
}

static void *dev_copy(const float *h, size_t n) {
    void *p = NULL;
    if (!hip_ok(hipMalloc(&p, n * sizeof(float)), "hipMalloc")) return NULL;
    if (h && !hip_ok(hipMemcpy(p, h, n * sizeof(float), hipMemcpyHostToDevice), "hipMemcpy")) return NULL;
    if (!h && !hip_ok(hipMemset(p, 0, n * sizeof(float)), "hipMemset")) return NULL;
    return p;
}

static void print_row(const char *name, const float *x, int n) {
    printf("%s:", name);
    for (int i = 0; i < n; ++i) printf(" %.9g", x[i]);
    printf("\n");
}

int main(int argc, char **argv) {
    if (argc != 1 + 4 + 4 + 4 + 2 + 4 + 4 + 1) {
        fprintf(stderr, "usage: %s k[4] q[4] v[4] alpha beta gn[4] z[4] eps\n", argv[0]);
        return 2;
    }
    float in[23];
    for (int i = 0; i < 23; ++i) in[i] = strtof(argv[1 + i], NULL);
    const float *k = in, *q = in + 4, *v = in + 8, *gn = in + 14, *z = in + 18;
    const float alpha = in[12], beta = in[13], eps = in[22];

    float *dk = dev_copy(k, D), *dq = dev_copy(q, D), *dv = dev_copy(v, D);
    float *da = dev_copy(&alpha, 1), *db = dev_copy(&beta, 1);
    float *dgn = dev_copy(gn, D), *dz = dev_copy(z, D);
    float *st1 = dev_copy(NULL, D * D), *st2 = dev_copy(NULL, D * D);
    float *o = dev_copy(NULL, D), *y = dev_copy(NULL, D);
    if (!dk || !dq || !dv || !da || !db || !dgn || !dz || !st1 || !st2 || !o || !y) return 1;

    /* raw o on state 1 (batch 1: the strides are not stepped, the widths serve) */
    gdn_status s = gdn_decode(st1, D * D, dq, dk, D, dv, D, da, db, 1, o, D, 1, 1, 1, D, D, NULL);
    if (s != GDN_OK) {
        fprintf(stderr, "gdn_decode: %s (hip %d)\n", gdn_status_string(s), gdn_last_hip_error());
        return 1;
    }
    /* y on state 2 */
    s = gdn_decode_norm(st2, D * D, dq, dk, D, dv, D, da, db, 1, dz, D, dgn, eps, y, GDN_F32, D,
                        1, 1, 1, D, D, NULL);
    if (s != GDN_OK) {
        fprintf(stderr, "gdn_decode_norm: %s (hip %d)\n", gdn_status_string(s), gdn_last_hip_error());
        return 1;
    }
    if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 1;

    float ho[D], hy[D], hs[D * D];
    if (!hip_ok(hipMemcpy(ho, o, sizeof ho, hipMemcpyDeviceToHost), "hipMemcpy") ||
        !hip_ok(hipMemcpy(hy, y, sizeof hy, hipMemcpyDeviceToHost), "hipMemcpy") ||
        !hip_ok(hipMemcpy(hs, st1, sizeof hs, hipMemcpyDeviceToHost), "hipMemcpy"))
        return 1;
    float col0[D];
    for (int i = 0; i < D; ++i) col0[i] = hs[i * D];   /* row i = value index, key index 0 */
    print_row("o", ho, D);
    print_row("state_col0", col0, D);
    print_row("y", hy, D);

    /* rejected before any launch: 3 value heads over 2 key heads, and a state
       pointer off its 16-byte alignment */
    s = gdn_decode(st1, D * D, dq, dk, D, dv, D, da, db, 1, o, D, 1, 2, 3, D, D, NULL);
    printf("status_shape: %s\n", gdn_status_string(s));
    s = gdn_decode(st1 + 1, D * D, dq, dk, D, dv, D, da, db, 1, o, D, 1, 1, 1, D, D, NULL);
    printf("status_align: %s\n", gdn_status_string(s));

    void *bufs[] = {dk, dq, dv, da, db, dgn, dz, st1, st2, o, y};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) hipFree(bufs[i]);
    return 0;
}
