/*
 * ggq_oracle.c -- plain, slow CPU reference for the fused dequantize-and-multiply
 * path over GGUF block-quantized weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header, table or constant with the GPU library.
 *
 * What the method computes, and where it is stated:
 *  - Phobos README (githubhelp mirror), section "Inference": GGUF models at Q8_0
 *    and Q4_K_M run on the GPU ("quantized GGUF models on Phobos kernels"), decode
 *    is a matrix-vector product per token, and a mixture-of-experts layer routes
 *    each token to a few experts.  The section's note says the host backend is the
 *    slow verification oracle and both backends produce the same logits.
 *  - Phobos README, "Examples" table (backend_check, batch_check): every device op
 *    is checked against the host; a batched pass is checked against single passes.
 *  - The pages name Q8_0 and Q4_K but print neither their arithmetic nor their
 *    bytes.  This file follows the plain reading used throughout the library:
 *      Q8_0: 32 int8 q + one fp16 d per block, w = d*q.
 *      Q4_K: 256-weight super-block, fp16 d and dmin, eight 32-weight sub-blocks
 *            with 6-bit scale sc and min m packed in 12 bytes, 4-bit q,
 *            w = d*sc*q - dmin*m.
 *    with the GGUF on-disk byte layout (the engine loads GGUF files and was
 *    verified token-for-token against llama.cpp, README "Inference").
 *
 * Precision: everything is accumulated in fp64, in ascending index order, with no
 * blocking or reordering.  Dequantized weights are the exact fp32 value of the
 * definition (see the notes at each function).
 *
 * Parity status of each function (pins live in tests/test_oracle_*.py):
 *   ggo_half_to_float     pinned: exhaustive vs numpy's binary16 conversion
 *   ggo_q4_k_scale_min    pinned: per-byte exhaustive vs an independent bit map
 *   ggo_dequant_*         pinned: hand-built blocks, brute force, exact rationals
 *   ggo_gemv, ggo_matvec  pinned: one-hot columns, exact integer cases, Fractions
 *   ggo_router/topk/probs pinned: hand-built ties, zero router, permutations
 *   ggo_moe               pinned: dense-sum invariant, top_k = E, brute force
 *   ggo_gemm              pinned: M=1 vs matvec, exact integer cases
 *   Agreement of the byte layout with real GGUF files: parity unpinned (no GGUF
 *   file and no printed block exists to pin it against).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GGO_Q8_0 8
#define GGO_Q4_K 12

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 -> binary32, from the format's definition:
 *   e == 0        : (-1)^s * f * 2^-24           (zero and subnormals)
 *   0 < e < 31    : (-1)^s * (1024 + f) * 2^(e-25)
 *   e == 31       : infinity (f == 0) or NaN
 * Every finite binary16 value is exact in binary32. */
float ggo_half_to_float(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e < 31)
        v = ldexp((double)(1024 + f), e - 25);
    else
        v = f ? (double)NAN : (double)INFINITY;
    return (float)(s ? -v : v);
}

static float half_at(const uint8_t *p) { return ggo_half_to_float((uint16_t)(p[0] | (p[1] << 8))); }

/* ------------------------------------------------------------------------- */
/* Q4_K packed scales: 12 bytes hold eight 6-bit scales sc[0..7] and eight 6-bit
 * mins m[0..7].  Sub-blocks 0..3 keep all six bits in bytes 0..3 (scales) and
 * 4..7 (mins).  Sub-blocks 4..7 keep their low four bits in the nibbles of bytes
 * 8..11 (scale low nibble, min high nibble) and their top two bits in the top two
 * bits of bytes 0..3 (scales) and 4..7 (mins). */
void ggo_q4_k_scale_min(const uint8_t s[12], int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* One Q8_0 block (34 bytes) -> 32 floats.  d*q is a product of an 11-bit and an
 * 8-bit significand, exact in fp64 and in fp32. */
static void dequant_q8_0_block(const uint8_t *blk, float *out)
{
    double d = (double)half_at(blk);
    for (int j = 0; j < 32; ++j)
        out[j] = (float)(d * (double)(int8_t)blk[2 + j]);
}

/* One Q4_K super-block (144 bytes) -> 256 floats.
 * Weight i (0..255) lives in quant byte qs[32*(i/64) + i%32]: the low nibble for
 * (i%64) < 32, the high nibble otherwise; its sub-block is j = i/32.
 * d*sc*q (<= 21 significant bits) and dmin*m (<= 17 bits) are exact in fp64, and
 * their difference spans at most 50 bits (binary16 exponents differ by <= 29), so
 * the fp64 difference is exact and the cast to fp32 is the single rounding of
 * the exact value. */
static void dequant_q4_k_block(const uint8_t *blk, float *out)
{
    double d = (double)half_at(blk);
    double dmin = (double)half_at(blk + 2);
    const uint8_t *s = blk + 4;
    const uint8_t *qs = blk + 16;
    for (int i = 0; i < 256; ++i) {
        int j = i / 32;
        int byte = qs[32 * (i / 64) + i % 32];
        int q = ((i % 64) < 32) ? (byte & 15) : (byte >> 4);
        int sc, m;
        ggo_q4_k_scale_min(s, j, &sc, &m);
        out[i] = (float)(d * (double)sc * (double)q - dmin * (double)m);
    }
}

static int64_t row_bytes(int fmt, int64_t k)
{
    if (fmt == GGO_Q8_0) return k / 32 * 34;
    if (fmt == GGO_Q4_K) return k / 256 * 144;
    return -1;
}

/* Dequantize one row of k weights. Returns 0, or -1 on a bad format/size. */
int ggo_dequant_row(int fmt, const uint8_t *row, int64_t k, float *out)
{
    if (fmt == GGO_Q8_0 && k % 32 == 0) {
        for (int64_t b = 0; b < k / 32; ++b)
            dequant_q8_0_block(row + b * 34, out + b * 32);
        return 0;
    }
    if (fmt == GGO_Q4_K && k % 256 == 0) {
        for (int64_t b = 0; b < k / 256; ++b)
            dequant_q4_k_block(row + b * 144, out + b * 256);
        return 0;
    }
    return -1;
}

/* Dequantize rows [r0, r1) of an n x k matrix into out[(r - r0) * k + c]. */
int ggo_dequant(int fmt, const uint8_t *w, int64_t n, int64_t k, int64_t r0, int64_t r1, float *out)
{
    int64_t rb = row_bytes(fmt, k);
    if (rb < 0 || r0 < 0 || r1 > n || r0 > r1) return -1;
    for (int64_t r = r0; r < r1; ++r)
        if (ggo_dequant_row(fmt, w + r * rb, k, out + (r - r0) * k) != 0) return -1;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Matrix-vector product, fp64:  y[b][r] = sum_k w[r][k] * x[b][k]  and
 * s[b][r] = sum_k |w[r][k] * x[b][k]|, for rows [r0, r1), batches 0..nb-1,
 * summed in ascending k.  Each product of an fp32 weight and an fp32 activation
 * is exact in fp64.  y, s are indexed [b * ldy + r]. s may be NULL. */
int ggo_gemv(int fmt, const uint8_t *w, int64_t n, int64_t k, const float *x, int64_t ldx,
             int64_t nb, int64_t r0, int64_t r1, double *y, double *s, int64_t ldy)
{
    int64_t rb = row_bytes(fmt, k);
    if (rb < 0 || r0 < 0 || r1 > n || r0 > r1) return -1;
    float *wr = (float *)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
    if (!wr) return -2;
    for (int64_t r = r0; r < r1; ++r) {
        if (ggo_dequant_row(fmt, w + r * rb, k, wr) != 0) { free(wr); return -1; }
        for (int64_t b = 0; b < nb; ++b) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                double p = (double)wr[c] * (double)x[b * ldx + c];
                acc += p;
                aabs += fabs(p);
            }
            y[b * ldy + r] = acc;
            if (s) s[b * ldy + r] = aabs;
        }
    }
    free(wr);
    return 0;
}

/* Same product with an fp64 input vector v[k] (one batch), used for the expert
 * down projection of a hidden state held in fp64.  If absw != 0 the weights are
 * replaced by their magnitudes (for propagated error bounds). */
int ggo_matvec_f64(int fmt, const uint8_t *w, int64_t n, int64_t k, const double *v,
                   int absw, double *y, double *s)
{
    int64_t rb = row_bytes(fmt, k);
    if (rb < 0) return -1;
    float *wr = (float *)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
    if (!wr) return -2;
    for (int64_t r = 0; r < n; ++r) {
        if (ggo_dequant_row(fmt, w + r * rb, k, wr) != 0) { free(wr); return -1; }
        double acc = 0.0, aabs = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            double wc = absw ? fabs((double)wr[c]) : (double)wr[c];
            double p = wc * v[c];
            acc += p;
            aabs += fabs(p);
        }
        y[r] = acc;
        if (s) s[r] = aabs;
    }
    free(wr);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Router: logits[t][e] = sum_h wr[e][h] * x[t][h] in fp64, s = sum |.|. */
void ggo_router_logits(const float *wr, int64_t e, int64_t h, const float *x, int64_t t,
                       double *logits, double *s)
{
    for (int64_t ti = 0; ti < t; ++ti)
        for (int64_t ei = 0; ei < e; ++ei) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t c = 0; c < h; ++c) {
                double p = (double)wr[ei * h + c] * (double)x[ti * h + c];
                acc += p;
                aabs += fabs(p);
            }
            logits[ti * e + ei] = acc;
            if (s) s[ti * e + ei] = aabs;
        }
}

/* Top-k by logit.  Softmax is strictly increasing in the logit, so the k largest
 * softmax probabilities are the k largest logits.  Output is in rank order
 * (largest first); equal logits rank the lower expert index first. */
void ggo_topk_f64(const double *l, int64_t t, int64_t e, int k, int32_t *idx)
{
    char *taken = (char *)calloc((size_t)e, 1);
    for (int64_t ti = 0; ti < t; ++ti) {
        memset(taken, 0, (size_t)e);
        const double *row = l + ti * e;
        for (int s = 0; s < k; ++s) {
            int64_t best = -1;
            for (int64_t i = 0; i < e; ++i)
                if (!taken[i] && (best < 0 || row[i] > row[best])) best = i;
            taken[best] = 1;
            idx[ti * k + s] = (int32_t)best;
        }
    }
    free(taken);
}

/* The same selection on fp32 logits (used to check the device's own choice
 * against its own logits, compared exactly). */
void ggo_topk_f32(const float *l, int64_t t, int64_t e, int k, int32_t *idx)
{
    char *taken = (char *)calloc((size_t)e, 1);
    for (int64_t ti = 0; ti < t; ++ti) {
        memset(taken, 0, (size_t)e);
        const float *row = l + ti * e;
        for (int s = 0; s < k; ++s) {
            int64_t best = -1;
            for (int64_t i = 0; i < e; ++i)
                if (!taken[i] && (best < 0 || row[i] > row[best])) best = i;
            taken[best] = 1;
            idx[ti * k + s] = (int32_t)best;
        }
    }
    free(taken);
}

/* Routing weights: softmax over all e logits (max-subtracted, fp64), then the
 * selected k probabilities renormalised to sum to one.  This equals a softmax
 * over the selected logits alone. */
void ggo_route_probs(const double *l, int64_t t, int64_t e, const int32_t *idx, int k, double *p)
{
    double *pf = (double *)malloc(sizeof(double) * (size_t)e);
    for (int64_t ti = 0; ti < t; ++ti) {
        const double *row = l + ti * e;
        double mx = row[0];
        for (int64_t i = 1; i < e; ++i) if (row[i] > mx) mx = row[i];
        double z = 0.0;
        for (int64_t i = 0; i < e; ++i) { pf[i] = exp(row[i] - mx); z += pf[i]; }
        for (int64_t i = 0; i < e; ++i) pf[i] /= z;
        double sel = 0.0;
        for (int s = 0; s < k; ++s) sel += pf[idx[ti * k + s]];
        for (int s = 0; s < k; ++s) p[ti * k + s] = pf[idx[ti * k + s]] / sel;
    }
    free(pf);
}

/* ------------------------------------------------------------------------- */
/* One expert's feed-forward on one token, fp64:
 *   g = Wg[e] x,  u = Wu[e] x,  h = silu(g) * u with silu(g) = g / (1 + exp(-g)),
 *   y = Wd[e] h.
 * Expert e of a stacked tensor starts at byte e * rows * row_bytes.
 * Optional outputs (any may be NULL): g, u, sg = sum|Wg x|, su = sum|Wu x|
 * (each [f]), h [f], y [hdim], sy = sum|Wd h| [hdim]. */
int ggo_expert_ffn(int fmt, const uint8_t *wg, const uint8_t *wu, const uint8_t *wd,
                   int64_t e, int64_t hdim, int64_t f, const float *x,
                   double *g, double *u, double *sg, double *su, double *h,
                   double *y, double *sy)
{
    int64_t rbh = row_bytes(fmt, hdim), rbf = row_bytes(fmt, f);
    if (rbh < 0 || rbf < 0) return -1;
    double *gg = (double *)malloc(sizeof(double) * (size_t)f * 5);
    double *uu = gg + f, *sgg = gg + 2 * f, *suu = gg + 3 * f, *hh = gg + 4 * f;
    int rc = 0;
    rc |= ggo_gemv(fmt, wg + e * f * rbh, f, hdim, x, hdim, 1, 0, f, gg, sgg, f);
    rc |= ggo_gemv(fmt, wu + e * f * rbh, f, hdim, x, hdim, 1, 0, f, uu, suu, f);
    for (int64_t i = 0; i < f; ++i)
        hh[i] = gg[i] / (1.0 + exp(-gg[i])) * uu[i];
    if (y) rc |= ggo_matvec_f64(fmt, wd + e * hdim * rbf, hdim, f, hh, 0, y, sy);
    if (g) memcpy(g, gg, sizeof(double) * (size_t)f);
    if (u) memcpy(u, uu, sizeof(double) * (size_t)f);
    if (sg) memcpy(sg, sgg, sizeof(double) * (size_t)f);
    if (su) memcpy(su, suu, sizeof(double) * (size_t)f);
    if (h) memcpy(h, hh, sizeof(double) * (size_t)f);
    free(gg);
    return rc;
}

/* Gate and up projections of a dense gated feed-forward on one token, fp64:
 *   g = Wg x,  u = Wu x,  h = silu(g) * u with silu(g) = g / (1 + exp(-g))
 * -- the first half of the expert feed-forward above, for Wg, Wu of n rows and
 * k columns.  Outputs [n] each: g, u, sg = sum|Wg x|, su = sum|Wu x|, h. */
int ggo_gated_ffn(int fmt, const uint8_t *wg, const uint8_t *wu, int64_t n, int64_t k,
                  const float *x, double *g, double *u, double *sg, double *su, double *h)
{
    int rc = 0;
    rc |= ggo_gemv(fmt, wg, n, k, x, k, 1, 0, n, g, sg, n);
    rc |= ggo_gemv(fmt, wu, n, k, x, k, 1, 0, n, u, su, n);
    for (int64_t i = 0; i < n; ++i)
        h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
    return rc;
}

/* Routed mixture-of-experts layer for tokens [t0, t1):
 *   y[t] = sum over the k selected experts of p[t][s] * (Wd[e] h_e(x[t]))
 * Only the selected experts' weights are read.  The sum runs over the selected
 * experts in ascending expert index (so that it equals, bit for bit, the dense
 * sum over all experts in index order with zero weight on the others).
 * hout (optional) receives h for each (t, slot) as [t][k][f]. */
int ggo_moe(int fmt, const uint8_t *wg, const uint8_t *wu, const uint8_t *wd,
            int64_t e, int64_t hdim, int64_t f, const float *x, int64_t t0, int64_t t1,
            const int32_t *idx, const double *p, int k, double *y, double *hout)
{
    double *ye = (double *)malloc(sizeof(double) * (size_t)hdim);
    double *he = (double *)malloc(sizeof(double) * (size_t)f);
    int rc = 0;
    for (int64_t ti = t0; ti < t1; ++ti) {
        double *yt = y + ti * hdim;
        for (int64_t r = 0; r < hdim; ++r) yt[r] = 0.0;
        for (int64_t ei = 0; ei < e; ++ei) {
            for (int s = 0; s < k; ++s) {
                if (idx[ti * k + s] != ei) continue;
                rc |= ggo_expert_ffn(fmt, wg, wu, wd, ei, hdim, f, x + ti * hdim,
                                     NULL, NULL, NULL, NULL, he, ye, NULL);
                for (int64_t r = 0; r < hdim; ++r) yt[r] += p[ti * k + s] * ye[r];
                if (hout) memcpy(hout + (ti * k + s) * f, he, sizeof(double) * (size_t)f);
            }
        }
    }
    free(ye);
    free(he);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Matrix product C[m][n] = sum_k a[m][k] * w[n][k] (fp64) and S = sum |a w| for
 * m in [m0, m1), n in [n0, n1); c and s indexed [m * ldc + n].  The weight row
 * is dequantized once per n and dotted against each activation row in
 * ascending k. */
int ggo_gemm(int fmt, const uint8_t *w, int64_t n, int64_t k, const float *a, int64_t lda,
             int64_t m0, int64_t m1, int64_t n0, int64_t n1, double *c, double *s, int64_t ldc)
{
    int64_t rb = row_bytes(fmt, k);
    if (rb < 0 || n0 < 0 || n1 > n || n0 > n1 || m0 > m1) return -1;
    float *wr = (float *)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
    if (!wr) return -2;
    for (int64_t nn = n0; nn < n1; ++nn) {
        if (ggo_dequant_row(fmt, w + nn * rb, k, wr) != 0) { free(wr); return -1; }
        for (int64_t mm = m0; mm < m1; ++mm) {
            const float *ar = a + mm * lda;
            double acc = 0.0, aabs = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) {
                double p = (double)wr[kk] * (double)ar[kk];
                acc += p;
                aabs += fabs(p);
            }
            c[mm * ldc + nn] = acc;
            if (s) s[mm * ldc + nn] = aabs;
        }
    }
    free(wr);
    return 0;
}
