/*
 * gdn_oracle.c -- plain, slow CPU oracle of the gated delta rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header, table or constant with the HIP library, and it is
 * written from the definitions on the pages, not from the kernels.
 *
 * Arithmetic is IEEE double throughout.  Storage is what the caller hands in:
 * fp32 state (rounded to nearest-even after every step, as a fp32 state pool
 * would be) or IEEE binary16 state (same, to binary16).  Outputs are returned in
 * double, before any rounding to an output dtype.
 *
 * Sources (page title, then the part of it followed):
 *  - logicaffeine "codegen_cuda/gdn.rs", kernel `gdn_step`: the per-row update
 *    of one value head's D x D memory (u = S.k, w = S.q, coef = beta(v - alpha u),
 *    S <- alpha S + coef k^T, output scaled by 1/sqrt(D)), the tiled key-head
 *    pairing g = h mod NK, and the note that the 1/sqrt(D) scale does not cancel
 *    under the norm.
 *  - same page, kernel `gdn_gate_norm`: per-head RMS norm over the head's
 *    outputs with eps inside the square root, times the shared weight, THEN
 *    times silu(z).
 *  - metrale "layers/ops/ssm_gdn_a.rs", launchers `gdn_decode`,
 *    `gdn_decode_f32_strided_norm`, `gdn_decode_f16_strided_norm`,
 *    `gdn_prefill_regresident` and the two `ssm_h_state_*` converters: per-
 *    sequence row strides, the fp16 state pool with a slot pitch in halves,
 *    round-to-nearest-even narrowing, and the token-sequential recurrence.
 *  - logicaffeine "codegen_cuda/gdn.rs", kernels `gk_conv_silu_l2` and
 *    `gk_gdn_gates`, and metrale `gdn_decode_f32_conv_norm`: the input stage
 *    fused in front of the decode (conv ring, silu, per-head L2 of q and k, the
 *    write-strength and decay gates).
 *  - logicaffeine "codegen_cuda/gdn.rs", kernel `gdn_gate_norm_q`: int8
 *    quantisation of the normed output in groups of 32.
 *
 * What is computed (the plain definition, not the kernels' factoring): for value
 * head h of sequence b, with key head g = h mod NK,
 *     S' = alpha * S (I - beta k k^T) + beta v k^T       (textbook delta rule)
 *     o  = S' q / sqrt(Dk)                               (read from the UPDATED state)
 * The first line is evaluated term by term as
 *     S'_ij = alpha S_ij - alpha beta (S k)_i k_j + beta v_i k_j,
 * and o is a second matrix-vector product over S'.  The kernels instead use the
 * algebraically equal o = (alpha S q + coef (k.q)) / sqrt(Dk); keeping the two
 * forms apart is what makes a formula slip on either side show up.
 *
 * Layout readings (logicaffeine's `gdn_step` indexes the memory value-row major,
 * while metrale's comments describe the transposed [k_dim, v_dim] order; the
 * sizes agree because Dk = Dv, and this follows the first page's arithmetic):
 *   state slot of (b, h) at  b*pitch + h*Dv*Dk,  row i = value index, column j =
 *   key index (key index contiguous);  token row r = b*T + t;  q/k element
 *   r*qk_stride + g*Dk + j;  v/z/out element r*stride + h*Dv + i;  alpha/beta
 *   element r*ab_stride + h.  All strides are in elements.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Storage conversions, written from the IEEE 754 definitions.               */
/* ------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Round to nearest, ties to even, from an exact double value.  Scaling by a
 * power of two is exact in double, and nearbyint() rounds to nearest-even in
 * the default rounding mode, so each branch below rounds exactly once. */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);          /* quiet NaN */
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {                                /* subnormal range */
        double m = nearbyint(ldexp(a, 24));                   /* units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)m);                /* m == 1024 is the smallest normal */
    }
    int e2;
    (void)frexp(a, &e2);                                      /* a = f 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                                           /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, 10 - e));                   /* 11 significant bits */
    if (m >= 2048.0) { m = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7c00u);            /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

double orc_f16_to_f64(uint16_t h)
{
    double s = (h & 0x8000u) ? -1.0 : 1.0;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    if (e == 0x1f) return f ? NAN : s * INFINITY;
    if (e == 0) return s * ldexp((double)f, -24);
    return s * ldexp((double)(1024 + f), e - 25);
}

/* bfloat16: the top 16 bits of binary32 (8 exponent bits, 7 fraction bits).
 * Round to nearest-even from a double, including the subnormal range. */
uint16_t orc_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0u);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
    if (a < ldexp(1.0, -126)) {
        double m = nearbyint(ldexp(a, 133));                  /* units of 2^-133 */
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e2;
    (void)frexp(a, &e2);
    int e = e2 - 1;
    double m = nearbyint(ldexp(a, 7 - e));                    /* 8 significant bits */
    if (m >= 256.0) { m = 128.0; e += 1; }
    if (e > 127) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (uint16_t)((e + 127) << 7) | (uint16_t)(m - 128.0));
}

void orc_f32_to_f16_array(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_f64_to_f16((double)src[i]);
}

void orc_f16_to_f32_array(const uint16_t *src, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = (float)orc_f16_to_f64(src[i]);
}

void orc_f64_to_bf16_array(const double *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_f64_to_bf16(src[i]);
}

/* ------------------------------------------------------------------------- */
/* The recurrence in double.                                                 */
/* ------------------------------------------------------------------------- */

/* One step of one value head.  S is Dv x Dk, row-major (row = value index),
 * updated in place to S'; o (length Dv) receives S' q / sqrt(Dk).
 * Source: logicaffeine codegen_cuda/gdn.rs, kernel `gdn_step`, restated as the
 * delta rule alpha S (I - beta k k^T) + beta v k^T. */
void orc_head_step(double *S, const double *q, const double *k, const double *v,
                   double alpha, double beta, int Dk, int Dv, double *o)
{
    for (int i = 0; i < Dv; ++i) {
        double *row = S + (int64_t)i * Dk;
        double sk = 0.0;                                      /* (S k)_i, old state */
        for (int j = 0; j < Dk; ++j) sk += row[j] * k[j];
        for (int j = 0; j < Dk; ++j)
            row[j] = alpha * row[j] - alpha * beta * sk * k[j] + beta * v[i] * k[j];
    }
    double scale = 1.0 / sqrt((double)Dk);
    for (int i = 0; i < Dv; ++i) {
        const double *row = S + (int64_t)i * Dk;
        double acc = 0.0;
        for (int j = 0; j < Dk; ++j) acc += row[j] * q[j];
        o[i] = acc * scale;
    }
}

/* Gated RMS norm of one head's output.
 * Source: logicaffeine codegen_cuda/gdn.rs, kernel `gdn_gate_norm`:
 *   r = sqrt(mean_i o_i^2 + eps),  y_i = (gn_i o_i / r) * z_i * sigmoid(z_i). */
void orc_gated_rmsnorm(const double *o, const double *z, const double *gn, double eps,
                       int Dv, double *y)
{
    double ss = 0.0;
    for (int i = 0; i < Dv; ++i) ss += o[i] * o[i];
    double r = sqrt(ss / (double)Dv + eps);
    for (int i = 0; i < Dv; ++i) {
        double silu = z[i] / (1.0 + exp(-z[i]));
        y[i] = (gn[i] * o[i] / r) * silu;
    }
}

/* ------------------------------------------------------------------------- */
/* Strided, storage-typed driver: T tokens of one (sequence b, value head h).  */
/* ------------------------------------------------------------------------- */

enum { ORC_STATE_F32 = 0, ORC_STATE_F16 = 1 };

/* Runs tokens t = 0..T-1 of head (b, h).  T = 1 is the single-token decode.
 * The slot is widened to double at the start; after every step it is rounded to
 * its storage type (and widened back), so that each step starts from exactly
 * what a state pool would hold.  out may be NULL (state only).  z NULL means
 * raw output o; otherwise out receives the gated-norm output y.
 * Returns 0, or -1 on bad arguments or allocation failure. */
int orc_seq_head(int b, int h, int T, int state_kind, void *state, int64_t pitch,
                 const float *q, const float *k, int64_t qk_stride,
                 const float *v, int64_t v_stride,
                 const float *alpha, const float *beta, int64_t ab_stride,
                 const float *z, int64_t z_stride, const float *gn, double eps,
                 double *out, int64_t out_stride,
                 int NK, int NV, int Dk, int Dv)
{
    if (T < 0 || NK <= 0 || NV <= 0 || Dk <= 0 || Dv <= 0 || h < 0 || h >= NV || b < 0)
        return -1;
    int g = h % NK;                                           /* tiled pairing */
    int64_t nel = (int64_t)Dv * Dk;
    int64_t slot = (int64_t)b * pitch + (int64_t)h * nel;
    double *S = (double *)malloc(sizeof(double) * (size_t)nel);
    double *qd = (double *)malloc(sizeof(double) * (size_t)Dk);
    double *kd = (double *)malloc(sizeof(double) * (size_t)Dk);
    double *vd = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *zd = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *gd = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *od = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *yd = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!S || !qd || !kd || !vd || !zd || !gd || !od || !yd) {
        free(S); free(qd); free(kd); free(vd); free(zd); free(gd); free(od); free(yd);
        return -1;
    }
    if (state_kind == ORC_STATE_F32) {
        const float *s32 = (const float *)state + slot;
        for (int64_t e = 0; e < nel; ++e) S[e] = (double)s32[e];
    } else {
        const uint16_t *s16 = (const uint16_t *)state + slot;
        for (int64_t e = 0; e < nel; ++e) S[e] = orc_f16_to_f64(s16[e]);
    }
    if (z) for (int i = 0; i < Dv; ++i) gd[i] = (double)gn[i];

    for (int t = 0; t < T; ++t) {
        int64_t r = (int64_t)b * T + t;
        for (int j = 0; j < Dk; ++j) {
            qd[j] = (double)q[r * qk_stride + (int64_t)g * Dk + j];
            kd[j] = (double)k[r * qk_stride + (int64_t)g * Dk + j];
        }
        for (int i = 0; i < Dv; ++i) vd[i] = (double)v[r * v_stride + (int64_t)h * Dv + i];
        double a = (double)alpha[r * ab_stride + h];
        double be = (double)beta[r * ab_stride + h];

        orc_head_step(S, qd, kd, vd, a, be, Dk, Dv, od);

        const double *res = od;
        if (z) {
            for (int i = 0; i < Dv; ++i) zd[i] = (double)z[r * z_stride + (int64_t)h * Dv + i];
            orc_gated_rmsnorm(od, zd, gd, eps, Dv, yd);
            res = yd;
        }
        if (out)
            for (int i = 0; i < Dv; ++i) out[r * out_stride + (int64_t)h * Dv + i] = res[i];

        /* the state pool holds storage-precision values between steps */
        for (int64_t e = 0; e < nel; ++e) {
            if (state_kind == ORC_STATE_F32) S[e] = (double)(float)S[e];
            else S[e] = orc_f16_to_f64(orc_f64_to_f16(S[e]));
        }
    }

    if (state_kind == ORC_STATE_F32) {
        float *s32 = (float *)state + slot;
        for (int64_t e = 0; e < nel; ++e) s32[e] = (float)S[e];
    } else {
        uint16_t *s16 = (uint16_t *)state + slot;
        for (int64_t e = 0; e < nel; ++e) s16[e] = orc_f64_to_f16(S[e]);
    }
    free(S); free(qd); free(kd); free(vd); free(zd); free(gd); free(od); free(yd);
    return 0;
}

/* Every (b, h) of a batch, sequence by sequence.  T = 1 is one decode call. */
int orc_seq(int B, int T, int state_kind, void *state, int64_t pitch,
            const float *q, const float *k, int64_t qk_stride,
            const float *v, int64_t v_stride,
            const float *alpha, const float *beta, int64_t ab_stride,
            const float *z, int64_t z_stride, const float *gn, double eps,
            double *out, int64_t out_stride,
            int NK, int NV, int Dk, int Dv)
{
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < NV; ++h) {
            int rc = orc_seq_head(b, h, T, state_kind, state, pitch, q, k, qk_stride, v, v_stride,
                                  alpha, beta, ab_stride, z, z_stride, gn, eps, out, out_stride,
                                  NK, NV, Dk, Dv);
            if (rc) return rc;
        }
    return 0;
}

/* A list of (b, h) heads, one after the other (a driver for timing the oracle
 * on several host threads: each thread takes its own list, and distinct heads
 * touch disjoint state and output). */
int orc_seq_head_list(int n, const int *bs, const int *hs, int T, int state_kind, void *state,
                      int64_t pitch, const float *q, const float *k, int64_t qk_stride,
                      const float *v, int64_t v_stride,
                      const float *alpha, const float *beta, int64_t ab_stride,
                      const float *z, int64_t z_stride, const float *gn, double eps,
                      double *out, int64_t out_stride,
                      int NK, int NV, int Dk, int Dv)
{
    for (int i = 0; i < n; ++i) {
        int rc = orc_seq_head(bs[i], hs[i], T, state_kind, state, pitch, q, k, qk_stride, v,
                              v_stride, alpha, beta, ab_stride, z, z_stride, gn, eps, out,
                              out_stride, NK, NV, Dk, Dv);
        if (rc) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Front end of the decode step: conv ring, silu, L2 of q and k, the gates.   */
/* ------------------------------------------------------------------------- */

/* One token of one sequence through the layer's input stage, in double.
 * Source: logicaffeine codegen_cuda/gdn.rs, kernels `gk_conv_silu_l2` and
 * `gk_gdn_gates`, and the GDN layer sequence of codegen_cuda/qwen38.rs
 * (`emit_qwen38_generate`: the conv runs over the q|k|v channels of the
 * projection row, the leading 2*NK head blocks are L2-normalised); metrale
 * layers/ops/ssm_gdn_a.rs, `gdn_decode_f32_conv_norm` (the same steps fused
 * into the decode launch, with separate L2 and norm epsilons).
 *
 *  channels  C = 2*NK*D + NV*D: q heads, then k heads, then v heads.
 *  ring      taps rows of C floats, row 0 the oldest input.  The token shifts
 *            every row up by one (row 0 is dropped) and stores x in row taps-1;
 *            ring is updated in place (fp32 copies, exact).
 *  conv      y_c = silu( sum_t ring'[t][c] * w[t][c] ),  w is [taps][C].
 *  L2        each q and k head block (D channels) is divided by
 *            sqrt(sum of its squares + l2_eps); v is not normalised.
 *  gates     beta_h = sigmoid(br_h);  alpha_h = (1 + exp(ar_h + dt_h))^rate_h
 *            (rate already holds the negative decay rate, so it is used as is).
 * Outputs q, k ([NK*D]), v ([NV*D]), alpha, beta ([NV]) in double. */
int orc_frontend_token(int NK, int NV, int D, int taps,
                       float *ring, const float *x, const float *w,
                       const float *br, const float *ar, const float *dt, const float *rate,
                       double l2_eps,
                       double *q, double *k, double *v, double *alpha, double *beta)
{
    if (NK <= 0 || NV <= 0 || D <= 0 || taps <= 0) return -1;
    int64_t C = (int64_t)(2 * NK + NV) * D;
    for (int64_t c = 0; c < C; ++c) {
        for (int t = 0; t + 1 < taps; ++t) ring[(int64_t)t * C + c] = ring[(int64_t)(t + 1) * C + c];
        ring[(int64_t)(taps - 1) * C + c] = x[c];
    }
    double *y = (double *)malloc(sizeof(double) * (size_t)C);
    if (!y) return -1;
    for (int64_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int t = 0; t < taps; ++t)
            acc += (double)ring[(int64_t)t * C + c] * (double)w[(int64_t)t * C + c];
        y[c] = acc / (1.0 + exp(-acc));
    }
    for (int blk = 0; blk < 2 * NK; ++blk) {
        const double *src = y + (int64_t)blk * D;
        double ss = 0.0;
        for (int j = 0; j < D; ++j) ss += src[j] * src[j];
        double den = sqrt(ss + l2_eps);
        double *dst = blk < NK ? q + (int64_t)blk * D : k + (int64_t)(blk - NK) * D;
        for (int j = 0; j < D; ++j) dst[j] = src[j] / den;
    }
    for (int64_t i = 0; i < (int64_t)NV * D; ++i) v[i] = y[(int64_t)2 * NK * D + i];
    for (int h = 0; h < NV; ++h) {
        beta[h] = 1.0 / (1.0 + exp(-(double)br[h]));
        alpha[h] = pow(1.0 + exp((double)ar[h] + (double)dt[h]), (double)rate[h]);
    }
    free(y);
    return 0;
}

/* The fused decode: front end, then the step and the gated norm of every value
 * head, for B sequences.  Strides are in elements: x rows x_stride apart,
 * ring slots ring_stride apart, br/ar rows g_stride apart, z and out rows
 * z_stride / out_stride apart.  The fp32 state is rounded once, after the step
 * (one token).  z NULL gives the raw output o.  The q, k, v, alpha, beta that
 * the front end produced may be returned (any of them NULL to skip), as
 * [B][NK*D], [B][NV*D] and [B][NV]. */
int orc_fused_decode(int B, int NK, int NV, int D, int taps,
                     float *state, int64_t pitch,
                     float *ring, int64_t ring_stride,
                     const float *x, int64_t x_stride, const float *w,
                     const float *br, const float *ar, int64_t g_stride,
                     const float *dt, const float *rate, double l2_eps,
                     const float *z, int64_t z_stride, const float *gn, double eps,
                     double *out, int64_t out_stride,
                     double *q_out, double *k_out, double *v_out, double *a_out, double *b_out)
{
    if (B < 0 || NK <= 0 || NV <= 0 || NV % NK || D <= 0 || taps <= 0) return -1;
    int64_t nel = (int64_t)D * D;
    double *q = (double *)malloc(sizeof(double) * (size_t)NK * D);
    double *k = (double *)malloc(sizeof(double) * (size_t)NK * D);
    double *v = (double *)malloc(sizeof(double) * (size_t)NV * D);
    double *al = (double *)malloc(sizeof(double) * (size_t)NV);
    double *be = (double *)malloc(sizeof(double) * (size_t)NV);
    double *S = (double *)malloc(sizeof(double) * (size_t)nel);
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    double *yy = (double *)malloc(sizeof(double) * (size_t)D);
    double *zd = (double *)malloc(sizeof(double) * (size_t)D);
    double *gd = (double *)malloc(sizeof(double) * (size_t)D);
    int rc = (!q || !k || !v || !al || !be || !S || !o || !yy || !zd || !gd) ? -1 : 0;
    if (!rc && z) for (int i = 0; i < D; ++i) gd[i] = (double)gn[i];
    for (int b = 0; b < B && !rc; ++b) {
        rc = orc_frontend_token(NK, NV, D, taps, ring + (int64_t)b * ring_stride,
                                x + (int64_t)b * x_stride, w, br + (int64_t)b * g_stride,
                                ar + (int64_t)b * g_stride, dt, rate, l2_eps, q, k, v, al, be);
        if (rc) break;
        if (q_out) memcpy(q_out + (int64_t)b * NK * D, q, sizeof(double) * (size_t)NK * D);
        if (k_out) memcpy(k_out + (int64_t)b * NK * D, k, sizeof(double) * (size_t)NK * D);
        if (v_out) memcpy(v_out + (int64_t)b * NV * D, v, sizeof(double) * (size_t)NV * D);
        if (a_out) memcpy(a_out + (int64_t)b * NV, al, sizeof(double) * (size_t)NV);
        if (b_out) memcpy(b_out + (int64_t)b * NV, be, sizeof(double) * (size_t)NV);
        for (int h = 0; h < NV; ++h) {
            int g = h % NK;
            float *slot = state + (int64_t)b * pitch + (int64_t)h * nel;
            for (int64_t e = 0; e < nel; ++e) S[e] = (double)slot[e];
            orc_head_step(S, q + (int64_t)g * D, k + (int64_t)g * D, v + (int64_t)h * D,
                          al[h], be[h], D, D, o);
            const double *res = o;
            if (z) {
                for (int i = 0; i < D; ++i) zd[i] = (double)z[(int64_t)b * z_stride + (int64_t)h * D + i];
                orc_gated_rmsnorm(o, zd, gd, eps, D, yy);
                res = yy;
            }
            for (int i = 0; i < D; ++i) out[(int64_t)b * out_stride + (int64_t)h * D + i] = res[i];
            for (int64_t e = 0; e < nel; ++e) slot[e] = (float)S[e];
        }
    }
    free(q); free(k); free(v); free(al); free(be); free(S); free(o); free(yy); free(zd); free(gd);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* int8 group quantisation of the normed output.                             */
/* ------------------------------------------------------------------------- */

/* Symmetric int8 quantisation in groups of 32 consecutive values.
 * Source: logicaffeine codegen_cuda/gdn.rs, kernel `gdn_gate_norm_q`: per group
 * the absolute maximum a, scale s = a / 127 (s = 1 when a == 0), and each code
 * the value divided by s, rounded to the nearest integer with ties to even.
 * Every decision is taken in binary32, as that kernel takes it: the input is
 * the fp32 output vector, and a/127 and y/s are single-precision operations
 * (this file is compiled without contraction, and x86-64 evaluates float
 * expressions in float).  n must be a multiple of 32. */
int orc_quant_groups32(const float *y, int64_t n, int8_t *codes, float *scales)
{
    if (n < 0 || n % 32) return -1;
    for (int64_t g0 = 0; g0 < n; g0 += 32) {
        float a = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float m = fabsf(y[g0 + i]);
            if (m > a) a = m;
        }
        float s = a > 0.0f ? a / 127.0f : 1.0f;
        scales[g0 / 32] = s;
        for (int i = 0; i < 32; ++i) {
            float r = nearbyintf(y[g0 + i] / s);
            codes[g0 + i] = (int8_t)(int)r;
        }
    }
    return 0;
}
