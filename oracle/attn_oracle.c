/*
 * attn_oracle.c -- plain, slow fp64 CPU reference for attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP kernels behind attn_fwd_bf16) never calls, links or includes it,
 * and this file shares no code, header, table or constant with that path.
 *
 * What it computes (sources are the web pages the method is described on):
 *
 *   - The operation is the fused softmax(Q K^T * scale) V of a transformer
 *     attention layer, bf16 inputs, head dimension 128, BSHD or BHSD layout,
 *     any query / key length (MoonMath AI MI300X attention article, opening
 *     paragraphs describing the kernel and its interface).  Head dimension
 *     64, the other size the HipKittens summary's kernel suite covers, is a
 *     parameter here (any D from 1 to 256).
 *   - The output is bf16 and the rounding to bf16 is selectable among
 *     round-to-nearest-even, round-to-nearest-ties-away and round-toward-zero
 *     (same article, paragraph on limitations and numerics, and the
 *     benchmark section that measures each of the three modes).
 *
 * The plain definition is evaluated in two passes per query row, in fp64,
 * with no blocking, no online rescaling and no reordering:
 *     s_j   = scale * sum_d q_d k_{j,d}            (d ascending)
 *     m     = max_j s_j
 *     p_j   = exp(s_j - m)
 *     l     = sum_j p_j                            (j ascending)
 *     o_d   = (sum_j p_j v_{j,d}) / l
 * Alongside it goes sigma_d = sqrt(sum_j p_j^2 v_{j,d}^2) / l, the RMS size
 * of the terms the p.V contraction adds up; the accuracy gate uses it as the
 * floor of the ULP scale for outputs that cancel to near zero.
 *
 * "Method" companion (an approximation the kernel makes, not the definition):
 * the probabilities enter the p.V matrix product as bf16 (the article runs
 * O += P V on the matrix cores; the AITER docs index names the bf16
 * 16x16x32 MFMA for both attention products on gfx950).  This file writes
 * that step out directly from the pages' order of operations, with the
 * reading documented in the design notes: x_j = s_j log2(e), M = ceil(max x),
 * pt_j = bf16(2^(x_j - M)), and
 *     o_method_d = sum_j pt_j v_{j,d} / L,  L = sum_j 2^(x_j - M)
 * (or L = sum_j pt_j when l_from_rounded is set).  Because M only rescales by
 * an exact power of two, pt_j does not depend on how keys are tiled.  The
 * bf16 rounding of pt_j is to nearest-even unless p_round names another mode:
 * the article measures each output rounding mode at a different speed, which
 * reads as the weights being rounded in the loop with the selected mode too,
 * so that reading is selectable.
 *
 * Two extensions the pages list as limitations of the kernel they describe
 * (MoonMath article, limitations paragraph: no causal masking, no grouped-
 * query attention), kept separate from the plain entry point:
 *   - grouped-query attention: Hq query heads share Hkv key/value heads, query
 *     head h reading key/value head h / (Hq / Hkv);
 *   - a causal mask aligned at the bottom-right: query i (of Sq) may attend
 *     key j (of Skv) iff j <= i + (Skv - Sq), i.e. the queries are the last Sq
 *     positions of the key sequence.  A row with no admissible key (possible
 *     only when Sq > Skv) is defined as all zeros, with sigma zero.
 * Masked keys are left out of the sums; nothing else changes.
 *
 * Optionally the row's log-sum-exp of the scaled scores is returned as well,
 * lse = m + log(sum_j exp(s_j - m)) over the admissible keys (natural log;
 * -inf for a row with no admissible key): the intermediate the FlyDSL
 * procedure article (debugging advice) suggests comparing against a
 * reference, and the side output a backward pass consumes.
 *
 * Rounding of the fp64 result to bf16 is done directly (no fp32 step) and
 * exactly, by locating the value on the bf16 grid; NaN maps to 0x7FC0.
 *
 * Build: plain C99, no -ffast-math, -ffp-contract=off (so IEEE NaN/Inf rules
 * hold and no multiply-add is fused), OpenMP across rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DMAX 256   /* largest head dimension */

enum { OR_LAYOUT_BSHD = 0, OR_LAYOUT_BHSD = 1 };
enum { OR_RTNE = 0, OR_RTNA = 1, OR_RTZ = 2 };

int oracle_version(void) { return 1; }

/* bf16 bit pattern -> exact double. */
static double bf16_to_double(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_double(uint16_t h) { return bf16_to_double(h); }

/*
 * Round an fp64 value to bf16 under the selected mode, exactly.
 *
 * bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored fraction bits.
 * For |x| in the binade [2^e, 2^(e+1)) the spacing of bf16 values is
 * 2^(e-7); below 2^-126 the spacing stays 2^-133 (subnormals).  x / spacing
 * is exact in fp64 (division by a power of two), its integer part n and the
 * fraction f = x/spacing - n are exact as well, and the mode picks n or n+1.
 */
uint16_t oracle_round_bf16(double x, int mode) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    const double two128 = ldexp(1.0, 128);
    if (a >= two128) {                      /* beyond the largest binade */
        return (mode == OR_RTZ) ? (uint16_t)(sign | 0x7F7F) : (uint16_t)(sign | 0x7F80);
    }
    int e2;
    frexp(a, &e2);                          /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                         /* floor(log2 a) */
    if (e < -126) e = -126;                 /* subnormal spacing */
    double spacing = ldexp(1.0, e - 7);
    double n = a / spacing;                 /* exact */
    double fl = floor(n);
    double fr = n - fl;                     /* exact */
    double m = fl;
    if (mode == OR_RTNE) {
        if (fr > 0.5) m = fl + 1.0;
        else if (fr == 0.5) m = (fmod(fl, 2.0) == 1.0) ? fl + 1.0 : fl;
    } else if (mode == OR_RTNA) {
        if (fr >= 0.5) m = fl + 1.0;
    } /* OR_RTZ keeps fl */
    double v = m * spacing;                 /* exact: m has at most 9 bits */
    if (v >= two128) return sign | 0x7F80;  /* rounded up past the max finite */
    if (v == 0.0) return sign;
    /* encode v */
    if (v < ldexp(1.0, -126)) {
        uint16_t frac = (uint16_t)(v / ldexp(1.0, -133));  /* 1..127 */
        return sign | frac;
    }
    frexp(v, &e2);
    int ev = e2 - 1;
    double mant = v / ldexp(1.0, ev);       /* in [1, 2), 7 fraction bits */
    uint16_t frac = (uint16_t)((mant - 1.0) * 128.0);
    return (uint16_t)(sign | ((uint16_t)(ev + 127) << 7) | frac);
}

void oracle_round_bf16_array(const double* x, uint16_t* out, int64_t n, int mode) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_round_bf16(x[i], mode);
}

/* Element offset of row (b, h, i) of a [*, D] tensor in the given layout. */
static int64_t row_offset(int layout, int64_t b, int64_t h, int64_t i, int64_t H, int64_t S, int64_t D) {
    if (layout == OR_LAYOUT_BSHD) return ((b * S + i) * H + h) * D;
    return ((b * H + h) * S + i) * D;
}

/* Round to bf16 in the given mode and back, for the method companion's probabilities. */
static double round_trip_bf16(double x, int mode) { return bf16_to_double(oracle_round_bf16(x, mode)); }

/*
 * Evaluate rows of attention.
 *   q         : bf16 bit patterns [B,Sq,Hq,D] or [B,Hq,Sq,D];
 *   k, v      : [B,Skv,Hkv,D] or [B,Hkv,Skv,D]; Hq a multiple of Hkv;
 *               D the head dimension (1 .. 256).
 *   causal    : 0 = every key, 1 = bottom-right aligned causal mask.
 *   rows      : flat query-row ids r = (b*Hq + h)*Sq + i, or NULL for all
 *               B*Hq*Sq rows in that order; nrows is the count.
 *   o_exact, sigma            : [nrows, D] doubles (required).
 *   o_method, sigma_method    : [nrows, D] doubles, or NULL to skip.
 *   lse                       : [nrows] doubles, or NULL to skip.
 *   l_from_rounded            : method companion's normaliser (see header).
 *   p_round                   : OR_RTNE / OR_RTNA / OR_RTZ for the method
 *                               companion's bf16 probabilities.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attention_gqa(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                         float scale, int causal, const int64_t* rows, int64_t nrows,
                         double* o_exact, double* sigma,
                         double* o_method, double* sigma_method, double* lse,
                         int l_from_rounded, int p_round, int nthreads) {
    if (!q || !k || !v || !o_exact || !sigma) return -1;
    if (p_round != OR_RTNE && p_round != OR_RTNA && p_round != OR_RTZ) return -1;
    if (layout != OR_LAYOUT_BSHD && layout != OR_LAYOUT_BHSD) return -1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1 || D > ORACLE_DMAX) return -1;
    if (Hq % Hkv != 0 || (causal != 0 && causal != 1)) return -1;
    const int64_t H = Hq, group = Hq / Hkv;
    if (rows == NULL) nrows = B * H * Sq;
    if (nrows < 0) return -1;
    const double sc = (double)scale;
    const double log2e = 1.4426950408889634073599246810018921;  /* 1/ln 2 */
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
        double* kk = (double*)malloc(sizeof(double) * D);
        if (!s || !kk) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < nrows; t++) {
            if (!s || !kk) continue;
            int64_t r = rows ? rows[t] : t;
            int64_t i = r % Sq, bh = r / Sq, h = bh % H, b = bh / H;
            int64_t hk = h / group;                       /* key/value head of query head h */
            /* admissible keys: j < n_keys (all of them unless causal) */
            int64_t n_keys = Skv;
            if (causal) {
                n_keys = i + (Skv - Sq) + 1;
                if (n_keys > Skv) n_keys = Skv;
            }
            double* oe = o_exact + t * D;
            double* sg = sigma + t * D;
            if (n_keys <= 0) {                            /* no admissible key: zeros */
                if (lse) lse[t] = -INFINITY;
                for (int d = 0; d < D; d++) {
                    oe[d] = 0.0;
                    sg[d] = 0.0;
                    if (o_method) o_method[t * D + d] = 0.0;
                    if (o_method && sigma_method) sigma_method[t * D + d] = 0.0;
                }
                continue;
            }
            double qq[ORACLE_DMAX];
            const uint16_t* qp = q + row_offset(layout, b, h, i, H, Sq, D);
            for (int d = 0; d < D; d++) qq[d] = bf16_to_double(qp[d]);

            /* pass 1: scores and their maximum (NaN propagates into m) */
            double m = -INFINITY;
            for (int64_t j = 0; j < n_keys; j++) {
                const uint16_t* kp = k + row_offset(layout, b, hk, j, Hkv, Skv, D);
                for (int d = 0; d < D; d++) kk[d] = bf16_to_double(kp[d]);
                double acc = 0.0;
                for (int d = 0; d < D; d++) acc += qq[d] * kk[d];
                s[j] = sc * acc;
                if (!isnan(m) && (isnan(s[j]) || s[j] > m)) m = s[j];
            }

            /* pass 2: weights, normaliser, weighted sums */
            double num[ORACLE_DMAX], sq[ORACLE_DMAX], numm[ORACLE_DMAX], sqm[ORACLE_DMAX];
            for (int d = 0; d < D; d++) { num[d] = 0.0; sq[d] = 0.0; numm[d] = 0.0; sqm[d] = 0.0; }
            double l = 0.0, lm = 0.0, lm_rounded = 0.0;
            double xmax = m * log2e;
            double M = ceil(xmax);
            for (int64_t j = 0; j < n_keys; j++) {
                const uint16_t* vp = v + row_offset(layout, b, hk, j, Hkv, Skv, D);
                double p = exp(s[j] - m);
                l += p;
                double pt = 0.0, pm = 0.0;
                if (o_method) {
                    pm = exp2(s[j] * log2e - M);
                    pt = round_trip_bf16(pm, p_round);
                    lm += pm;
                    lm_rounded += pt;
                }
                for (int d = 0; d < D; d++) {
                    double vv = bf16_to_double(vp[d]);
                    num[d] += p * vv;
                    sq[d] += (p * vv) * (p * vv);
                    if (o_method) {
                        numm[d] += pt * vv;
                        sqm[d] += (pt * vv) * (pt * vv);
                    }
                }
            }
            for (int d = 0; d < D; d++) {
                oe[d] = num[d] / l;
                sg[d] = sqrt(sq[d]) / l;
            }
            if (lse) lse[t] = m + log(l);
            if (o_method) {
                double L = l_from_rounded ? lm_rounded : lm;
                double* om = o_method + t * D;
                double* sm = sigma_method ? sigma_method + t * D : NULL;
                for (int d = 0; d < D; d++) {
                    om[d] = numm[d] / L;
                    if (sm) sm[d] = sqrt(sqm[d]) / L;
                }
            }
        }
        free(s);
        free(kk);
    }
    return failed ? -1 : 0;
}

/* The plain operation: every query head has its own key/value head, no mask. */
int oracle_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int layout, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                     float scale, const int64_t* rows, int64_t nrows,
                     double* o_exact, double* sigma,
                     double* o_method, double* sigma_method,
                     int l_from_rounded, int nthreads) {
    return oracle_attention_gqa(q, k, v, layout, B, H, H, Sq, Skv, 128, scale, 0, rows, nrows,
                                o_exact, sigma, o_method, sigma_method, NULL, l_from_rounded, OR_RTNE, nthreads);
}

/*
 * Backward pass of the same operation (NEXT to the forward: the gradients a
 * training step needs; the HipKittens summary's kernel suite pairs attention
 * forward with its backward).  With a loss L and dO = dL/dO given, the chain
 * rule on the plain definition gives, per (batch, head), with p the softmax
 * weights and causal-masked pairs left out:
 *     dv_j = sum_i p_ij do_i
 *     dp_ij = <do_i, v_j>
 *     ds_ij = p_ij (dp_ij - delta_i),    delta_i = sum_j p_ij dp_ij = <do_i, o_i>
 *     dq_i = scale sum_j ds_ij k_j,     dk_j = scale sum_i ds_ij q_i
 * delta_i is evaluated as <do_i, o_i> with the o the caller passes (the
 * forward's stored bf16 output, as a backward pass that starts from the saved
 * output does), or with the exact o when o is NULL; the two agree up to o's
 * rounding.  Everything in fp64, rows in ascending order, no blocking.
 *
 *   q, o, dO : [B,Sq,H,D] or [B,H,Sq,D] bf16 bits (o may be NULL);
 *   k, v     : [B,Skv,Hkv,D] or [B,Hkv,Skv,D]; query head h reads key/value
 *              head h / (H / Hkv), H a multiple of Hkv (Hkv = H: plain heads)
 *   dq, sdq  : [B*H*Sq, D] doubles, rows (b*H + h)*Sq + i: the gradient and
 *              the RMS size of the terms its sum adds (scale |ds_ij k_jd|)
 *   dk, sdk, dv, sdv : [B*Hkv*Skv, D] doubles, rows (b*Hkv + hk)*Skv + j; a
 *              key/value head's gradient sums the terms of all its query heads
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                         const uint16_t* dO, int layout, int64_t B, int64_t H, int64_t Hkv, int64_t Sq,
                         int64_t Skv, int64_t D, float scale, int causal,
                         double* dq, double* sdq, double* dk, double* sdk, double* dv, double* sdv,
                         int nthreads) {
    if (!q || !k || !v || !dO || !dq || !sdq || !dk || !sdk || !dv || !sdv) return -1;
    if (layout != OR_LAYOUT_BSHD && layout != OR_LAYOUT_BHSD) return -1;
    if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Sq < 1 || Skv < 1 || D < 1 || D > ORACLE_DMAX) return -1;
    if (causal != 0 && causal != 1) return -1;
    const int64_t group = H / Hkv;   /* query head h reads key/value head h / group */
    const double sc = (double)scale;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    double* P = (double*)malloc(sizeof(double) * (size_t)(Sq * Skv));
    double* dS = (double*)malloc(sizeof(double) * (size_t)(Sq * Skv));
    if (!P || !dS) { free(P); free(dS); return -1; }
    /* dk, dv (and the sums of squares behind sdk, sdv) add up over the query
       heads of each key/value head */
    for (int64_t r = 0; r < B * Hkv * Skv * D; r++) { dk[r] = 0.0; sdk[r] = 0.0; dv[r] = 0.0; sdv[r] = 0.0; }
    for (int64_t b = 0; b < B; b++) {
        for (int64_t h = 0; h < H; h++) {
            const int64_t kvh = h / group;
            /* weights p_ij (masked pairs 0), per row */
#pragma omp parallel for schedule(dynamic, 8)
            for (int64_t i = 0; i < Sq; i++) {
                int64_t n_keys = Skv;
                if (causal) {
                    n_keys = i + (Skv - Sq) + 1;
                    if (n_keys > Skv) n_keys = Skv;
                    if (n_keys < 0) n_keys = 0;
                }
                const uint16_t* qp = q + row_offset(layout, b, h, i, H, Sq, D);
                double m = -INFINITY;
                double* pr = P + i * Skv;
                for (int64_t j = 0; j < Skv; j++) {
                    if (j >= n_keys) { pr[j] = 0.0; continue; }
                    const uint16_t* kp = k + row_offset(layout, b, kvh, j, Hkv, Skv, D);
                    double acc = 0.0;
                    for (int d = 0; d < D; d++) acc += bf16_to_double(qp[d]) * bf16_to_double(kp[d]);
                    pr[j] = sc * acc;
                    if (!isnan(m) && (isnan(pr[j]) || pr[j] > m)) m = pr[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < n_keys; j++) { pr[j] = exp(pr[j] - m); l += pr[j]; }
                for (int64_t j = 0; j < n_keys; j++) pr[j] /= l;
                /* delta_i = <do_i, o_i> (given o, or the exact o = sum_j p_ij v_j) */
                const uint16_t* gp = dO + row_offset(layout, b, h, i, H, Sq, D);
                double delta = 0.0;
                for (int d = 0; d < D; d++) {
                    double od;
                    if (o) {
                        od = bf16_to_double(o[row_offset(layout, b, h, i, H, Sq, D) + d]);
                    } else {
                        od = 0.0;
                        for (int64_t j = 0; j < n_keys; j++)
                            od += pr[j] * bf16_to_double(v[row_offset(layout, b, kvh, j, Hkv, Skv, D) + d]);
                    }
                    delta += bf16_to_double(gp[d]) * od;
                }
                /* ds_ij = p_ij (<do_i, v_j> - delta_i) */
                double* dr = dS + i * Skv;
                for (int64_t j = 0; j < Skv; j++) {
                    if (j >= n_keys) { dr[j] = 0.0; continue; }
                    const uint16_t* vp = v + row_offset(layout, b, kvh, j, Hkv, Skv, D);
                    double dp = 0.0;
                    for (int d = 0; d < D; d++) dp += bf16_to_double(gp[d]) * bf16_to_double(vp[d]);
                    dr[j] = pr[j] * (dp - delta);
                }
            }
            /* dq_i = scale sum_j ds_ij k_j */
#pragma omp parallel for schedule(dynamic, 8)
            for (int64_t i = 0; i < Sq; i++) {
                double* g = dq + ((b * H + h) * Sq + i) * D;
                double* sg = sdq + ((b * H + h) * Sq + i) * D;
                for (int d = 0; d < D; d++) { g[d] = 0.0; sg[d] = 0.0; }
                for (int64_t j = 0; j < Skv; j++) {
                    const double w = dS[i * Skv + j];
                    if (w == 0.0) continue;
                    const uint16_t* kp = k + row_offset(layout, b, kvh, j, Hkv, Skv, D);
                    for (int d = 0; d < D; d++) {
                        const double t = sc * w * bf16_to_double(kp[d]);
                        g[d] += t;
                        sg[d] += t * t;
                    }
                }
                for (int d = 0; d < D; d++) sg[d] = sqrt(sg[d]);
            }
            /* dk_j = scale sum_i ds_ij q_i,  dv_j = sum_i p_ij do_i */
#pragma omp parallel for schedule(dynamic, 8)
            for (int64_t j = 0; j < Skv; j++) {
                double* gk = dk + ((b * Hkv + kvh) * Skv + j) * D;
                double* sk = sdk + ((b * Hkv + kvh) * Skv + j) * D;
                double* gv = dv + ((b * Hkv + kvh) * Skv + j) * D;
                double* sv = sdv + ((b * Hkv + kvh) * Skv + j) * D;
                for (int64_t i = 0; i < Sq; i++) {
                    const double w = dS[i * Skv + j], pw = P[i * Skv + j];
                    const uint16_t* qp = q + row_offset(layout, b, h, i, H, Sq, D);
                    const uint16_t* gp = dO + row_offset(layout, b, h, i, H, Sq, D);
                    for (int d = 0; d < D; d++) {
                        const double tk = sc * w * bf16_to_double(qp[d]);
                        const double tv = pw * bf16_to_double(gp[d]);
                        gk[d] += tk; sk[d] += tk * tk;
                        gv[d] += tv; sv[d] += tv * tv;
                    }
                }
            }
        }
    }
    for (int64_t r = 0; r < B * Hkv * Skv * D; r++) { sdk[r] = sqrt(sdk[r]); sdv[r] = sqrt(sdv[r]); }
    free(P);
    free(dS);
    return 0;
}
