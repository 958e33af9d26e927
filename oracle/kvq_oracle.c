/*
 * kvq_oracle.c -- plain, slow CPU oracle for KIVI-style asymmetric low-bit
 * KV-cache quantization and for decode attention over the dequantized cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or helper with it; the two meet only through the
 * seeded input generators and the comparison in the tests.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (contraction off so every fp32 step below is one IEEE operation, as written).
 *
 * Sources (cited by page title and section):
 *  [P1] "KV cache compression: quantization, eviction and sparse attention",
 *       section 3.2 (KIVI: keys per-channel over G-token groups, values
 *       per-token, full-precision residual of the most recent R tokens, a
 *       group is quantized once it is full), section 3.4 (paged blocks),
 *       section 8.1 (byte accounting), section 2.2 (sum of weights is 1).
 *  [P3] "KV Cache compression lab", experiment 01 (grid of 2^bits lines between
 *       min and max, spacing (max-min)/(2^bits-1), each value snaps to the
 *       nearest line, zero = starting point of the grid).
 *  [P1] section 3.1: 8-bit KV (FP8 E4M3 with a static per-tensor or per-head
 *       scale, or INT8 with a dynamic per-token scale) as the first 2x.
 *  [P1] section 3.3 (KVQuant: quantize keys before RoPE, apply RoPE when
 *       reading; non-uniform grids with levels at quantiles of the
 *       distribution, like NF4) and section 2 (RoPE rotates pairs of
 *       dimensions, keeping each pair's norm).
 *  [P3] experiment 03: RoPE treats two adjacent dimensions as one plane;
 *       KVQuant keeps the few extreme key values in fp16 as a sparse matrix
 *       and quantizes the rest.
 *  [P2] "KV compression and quantization", part B.1 (FP8 E4M3/E5M2 and INT8
 *       at 0.5x the fp16 bytes).
 *  [P4] "KV cache compression" (jaedaily), formula paragraph: per-channel key
 *       dequant k = round((k - z_c)/s_c) s_c + z_c, per-token value dequant,
 *       M_KV = 2 L H_kv n d_h b, attention softmax(q k^T / sqrt(d_h)).
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): scale and zero are computed in fp32 and stored as fp16 (round to
 * nearest even); codes are computed from the STORED scale and zero as
 * clamp(rint((x - z) * (1/s)), 0, 2^b - 1) with ties to even; a group whose
 * stored scale is 0 gets all-zero codes; min and max are canonicalised so a
 * -0 extreme becomes +0; the residual keeps at least R tokens, and a group
 * is quantized only once it lies wholly outside them, so
 * n_q = G * floor(max(0, n - R) / G).
 * 8-bit formats: INT8 is the same min/max quantizer with 8 bits applied to
 * every key and value token over its d channels (asymmetric, like the rest
 * of the method); FP8 takes the nearest E4M3 value (ties to even) of
 * x * (1/scale) clamped to +-448, with one static fp32 scale per kv head for
 * keys and one for values supplied by the caller; both keep the residual
 * window and the group flush of the low-bit format.
 *
 * Parity pins (tests that tie this file to something other than itself) live
 * in tests/test_oracle_pins.py.  Every function below is pinned there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 codec, written from the format's definition:           */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds */
/* subnormals (fraction * 2^-24), exponent 31 holds inf / NaN.              */
/* ------------------------------------------------------------------------ */

float orc_h2f(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac + 1024), expo - 25);
    return (float)(sign ? -v : v);
}

/* Round a float to the nearest binary16 value, ties to even. */
uint16_t orc_f2h(float xf)
{
    double x = (double)xf; /* exact */
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(x))
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-24, m an integer 0..1024 */
        double m = rint(ldexp(a, 24)); /* exact scaling; rint is ties-to-even */
        return (uint16_t)(sign | (uint16_t)m); /* m == 1024 is the smallest normal */
    }
    int e2;
    frexp(a, &e2);             /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;            /* a in [2^e, 2^(e+1)) */
    double m = rint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7c00); /* overflow rounds to infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* ------------------------------------------------------------------------ */
/* Asymmetric uniform min/max quantizer of one set of fp16 values.          */
/* [P3] exp. 01: 2^b grid lines between min and max, spacing                 */
/* s = (max - min)/(2^b - 1), zero = min, each value snaps to the nearest   */
/* line.  [P4]: dequant q*s + z.                                             */
/* ------------------------------------------------------------------------ */

static void quantize_set(const uint16_t *x, int count, long stride, int bits,
                         uint8_t *codes, long code_stride, uint16_t *s_out, uint16_t *z_out)
{
    const int qmax = (1 << bits) - 1;
    float mn = orc_h2f(x[0]);
    float mx = mn;
    for (int i = 1; i < count; ++i) {
        float v = orc_h2f(x[(long)i * stride]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    mn = mn + 0.0f; /* -0 + +0 = +0 under round-to-nearest */
    mx = mx + 0.0f;
    float s32 = (mx - mn) / (float)qmax;
    uint16_t s16 = orc_f2h(s32);
    uint16_t z16 = orc_f2h(mn); /* exact: mn is an fp16 value */
    float s = orc_h2f(s16);
    float z = orc_h2f(z16);
    float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
    for (int i = 0; i < count; ++i) {
        float v = orc_h2f(x[(long)i * stride]);
        float t = (v - z) * inv;
        float r = rintf(t);
        if (r < 0.0f) r = 0.0f;
        if (r > (float)qmax) r = (float)qmax;
        codes[(long)i * code_stride] = (uint8_t)r;
    }
    *s_out = s16;
    *z_out = z16;
}

/* Number of quantized tokens of a sequence holding n tokens ([P1] 3.2:
 * a group of G tokens is quantized only once it is full and outside the
 * most recent R tokens). */
int orc_num_quantized(int n, int G, int R)
{
    int over = n - R;
    if (over <= 0) return 0;
    return G * (over / G);
}

/* Keys of one group, per channel over the group's G tokens ([P1] 3.2, [P4]).
 * x, codes: [G][d] row-major; s, z: [d]. */
void orc_quantize_key_group(const uint16_t *x, int G, int d, int bits,
                            uint8_t *codes, uint16_t *s, uint16_t *z)
{
    for (int c = 0; c < d; ++c)
        quantize_set(x + c, G, d, bits, codes + c, d, &s[c], &z[c]);
}

/* Values of one token, over its d channels ([P1] 3.2, [P4]). */
void orc_quantize_value_token(const uint16_t *x, int d, int bits,
                              uint8_t *codes, uint16_t *s, uint16_t *z)
{
    quantize_set(x, d, 1, bits, codes, 1, s, z);
}

/* Whole-sequence quantization of one (sequence, kv-head) stream holding n
 * tokens: groups [0, n_q) are quantized, [n_q, n) stay fp16 (the caller keeps
 * them).  k, v: [n][d]; kcodes, vcodes: [n_q][d]; ks, kz: [n_q/G][d];
 * vs, vz: [n_q].  Returns n_q. */
int orc_prefill_stream(const uint16_t *k, const uint16_t *v, int n, int d,
                       int kbits, int vbits, int G, int R,
                       uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                       uint8_t *vcodes, uint16_t *vs, uint16_t *vz)
{
    int nq = orc_num_quantized(n, G, R);
    for (int g = 0; g < nq / G; ++g)
        orc_quantize_key_group(k + (long)g * G * d, G, d, kbits,
                               kcodes + (long)g * G * d, ks + (long)g * d, kz + (long)g * d);
    for (int t = 0; t < nq; ++t)
        orc_quantize_value_token(v + (long)t * d, d, vbits, vcodes + (long)t * d, vs + t, vz + t);
    return nq;
}

/* Incremental form ([P1] 3.2, [P4] deployment step (c)): append one fp16
 * token to a stream's state; when the full-precision tail reaches R + G
 * tokens, its oldest G tokens form a full group outside the most recent R
 * and are quantized.  State: *n, *nq; hist_k/hist_v [cap][d] hold every
 * appended fp16 token at its position (the oracle keeps the whole history;
 * only [nq, n) is treated as residual); the quantized arrays are indexed as
 * in orc_prefill_stream.  Returns 1 if a group was flushed, 0 otherwise,
 * -1 if cap would be exceeded. */
int orc_append_stream(uint16_t *hist_k, uint16_t *hist_v, int cap, int *n, int *nq,
                      const uint16_t *k_new, const uint16_t *v_new, int d,
                      int kbits, int vbits, int G, int R,
                      uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                      uint8_t *vcodes, uint16_t *vs, uint16_t *vz)
{
    if (*n >= cap) return -1;
    memcpy(hist_k + (long)(*n) * d, k_new, sizeof(uint16_t) * d);
    memcpy(hist_v + (long)(*n) * d, v_new, sizeof(uint16_t) * d);
    *n += 1;
    if (*n - *nq == R + G) {
        int g = *nq / G;
        orc_quantize_key_group(hist_k + (long)(*nq) * d, G, d, kbits,
                               kcodes + (long)(*nq) * d, ks + (long)g * d, kz + (long)g * d);
        for (int t = *nq; t < *nq + G; ++t)
            orc_quantize_value_token(hist_v + (long)t * d, d, vbits,
                                     vcodes + (long)t * d, vs + t, vz + t);
        *nq += G;
        return 1;
    }
    return 0;
}

/* Dequantized stream ([P4]: x = q*s + z, one fp32 rounding via fma; the
 * residual tokens are the fp16 values themselves).  out_k, out_v: [n][d]. */
void orc_dequantize_stream(const uint16_t *k, const uint16_t *v, int n, int nq, int d, int G,
                           const uint8_t *kcodes, const uint16_t *ks, const uint16_t *kz,
                           const uint8_t *vcodes, const uint16_t *vs, const uint16_t *vz,
                           float *out_k, float *out_v)
{
    for (int t = 0; t < n; ++t) {
        for (int c = 0; c < d; ++c) {
            long i = (long)t * d + c;
            if (t < nq) {
                long gi = (long)(t / G) * d + c;
                out_k[i] = fmaf((float)kcodes[i], orc_h2f(ks[gi]), orc_h2f(kz[gi]));
                out_v[i] = fmaf((float)vcodes[i], orc_h2f(vs[t]), orc_h2f(vz[t]));
            } else {
                out_k[i] = orc_h2f(k[i]);
                out_v[i] = orc_h2f(v[i]);
            }
        }
    }
}

/* Scaled dot-product attention of gq query rows against n key/value rows,
 * accumulated in fp64 ([P4]: softmax(q k^T / sqrt(d_h)) weighting v; the
 * softmax subtracts the row maximum before exponentiating, which leaves its
 * value unchanged).  One function serves fp32 keys (kf) and fp64 keys (kd,
 * e.g. keys rotated by orc_rope_rotate): exactly one of the two is non-NULL.
 * q: [gq][d]; keys, vh: [n][d]; out: [gq][d]; weights (optional, may be
 * NULL): [gq][n].  n == 0 gives out = 0. */
static void attention_core(const float *q, int gq, const float *kf, const double *kd, const float *vh,
                           int n, int d, float scale, double *out, double *weights)
{
    double *logit = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    for (int h = 0; h < gq; ++h) {
        double *o = out + (long)h * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        if (n == 0) continue;
        double m = -INFINITY;
        for (int t = 0; t < n; ++t) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) {
                long i = (long)t * d + c;
                acc += (double)q[(long)h * d + c] * (kf ? (double)kf[i] : kd[i]);
            }
            logit[t] = (double)scale * acc;
            if (logit[t] > m) m = logit[t];
        }
        double l = 0.0;
        for (int t = 0; t < n; ++t) {
            logit[t] = exp(logit[t] - m);
            l += logit[t];
        }
        for (int t = 0; t < n; ++t) {
            double p = logit[t] / l;
            if (weights) weights[(long)h * n + t] = p;
            for (int c = 0; c < d; ++c) o[c] += p * (double)vh[(long)t * d + c];
        }
    }
    free(logit);
}

/* Attention over fp32 keys (the dequantized cache). */
void orc_attention(const float *q, int gq, const float *kh, const float *vh, int n, int d,
                   float scale, double *out, double *weights)
{
    attention_core(q, gq, kh, NULL, vh, n, d, scale, out, weights);
}

/* ------------------------------------------------------------------------ */
/* Non-uniform grid ("codebook" mode; [P1] section 3.3: KVQuant places the   */
/* levels at quantiles of the distribution, like NF4).  The 2^b levels sit   */
/* at the standard-normal quantiles of the centres of 2^b equal-probability  */
/* bins, c_k = Phi^-1((k + 1/2) / 2^b), mapped affinely onto each set's      */
/* [min, max] like the uniform grid's levels (so min and max stay exact): in */
/* grid steps of the uniform grid, L_k = Q (c_k - c_0) / (c_Q - c_0), rounded */
/* to the nearest multiple of 1/F_b (ties to even), F_b the largest power of */
/* two with F_b Q <= 255.  Scale, zero and 1/s are the uniform grid's; a      */
/* value goes to the nearest level (ties to the even code) and dequantizes   */
/* to L_code * s + z.  With L_k = k this is exactly the uniform rule.        */
/* ------------------------------------------------------------------------ */

/* Standard normal quantile: bisection on the cdf 0.5 erfc(-x / sqrt 2). */
static double normal_quantile(double p)
{
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        if (0.5 * erfc(-mid / sqrt(2.0)) < p)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

int orc_codebook_scale(int bits)
{
    int Q = (1 << bits) - 1, F = 1;
    while (2 * F * Q <= 255) F *= 2;
    return F;
}

/* Levels L_0 .. L_Q of the b-bit codebook, in uniform grid steps. */
void orc_codebook_levels(int bits, double *levels)
{
    int n = 1 << bits, Q = n - 1;
    double F = (double)orc_codebook_scale(bits);
    double c[256];
    for (int k = 0; k < n; ++k) c[k] = normal_quantile((k + 0.5) / n);
    for (int k = 0; k < n; ++k)
        levels[k] = nearbyint(F * Q * (c[k] - c[0]) / (c[Q] - c[0])) / F; /* round half to even */
}

/* Set quantizer on the codebook lev[] (see quantize_set for s, z, inv). */
static void quantize_set_cb(const uint16_t *x, int count, long stride, int bits, const double *lev,
                            uint8_t *codes, long code_stride, uint16_t *s_out, uint16_t *z_out)
{
    const int qmax = (1 << bits) - 1;
    float mn = orc_h2f(x[0]);
    float mx = mn;
    for (int i = 1; i < count; ++i) {
        float v = orc_h2f(x[(long)i * stride]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    float s32 = (mx - mn) / (float)qmax;
    uint16_t s16 = orc_f2h(s32);
    uint16_t z16 = orc_f2h(mn);
    float s = orc_h2f(s16);
    float z = orc_h2f(z16);
    float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
    for (int i = 0; i < count; ++i) {
        float v = orc_h2f(x[(long)i * stride]);
        float t = (v - z) * inv;
        /* nearest level: count the midpoints below t; a tie at the midpoint
         * between levels k and k+1 goes to whichever of the two is even */
        int code = 0;
        for (int k = 0; k < qmax; ++k) {
            float m = (float)(0.5 * (lev[k] + lev[k + 1])); /* exact */
            if ((k % 2 == 0) ? (t > m) : (t >= m)) code += 1;
        }
        codes[(long)i * code_stride] = (uint8_t)code;
    }
    *s_out = s16;
    *z_out = z16;
}

void orc_quantize_key_group_cb(const uint16_t *x, int G, int d, int bits, const double *lev,
                               uint8_t *codes, uint16_t *s, uint16_t *z)
{
    for (int c = 0; c < d; ++c)
        quantize_set_cb(x + c, G, d, bits, lev, codes + c, d, &s[c], &z[c]);
}

void orc_quantize_value_token_cb(const uint16_t *x, int d, int bits, const double *lev,
                                 uint8_t *codes, uint16_t *s, uint16_t *z)
{
    quantize_set_cb(x, d, 1, bits, lev, codes, 1, s, z);
}

/* orc_prefill_stream / orc_append_stream / orc_dequantize_stream on the
 * codebooks of kbits and vbits. */
int orc_prefill_stream_cb(const uint16_t *k, const uint16_t *v, int n, int d,
                          int kbits, int vbits, int G, int R,
                          uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                          uint8_t *vcodes, uint16_t *vs, uint16_t *vz)
{
    double klev[256], vlev[256];
    orc_codebook_levels(kbits, klev);
    orc_codebook_levels(vbits, vlev);
    int nq = orc_num_quantized(n, G, R);
    for (int g = 0; g < nq / G; ++g)
        orc_quantize_key_group_cb(k + (long)g * G * d, G, d, kbits, klev,
                                  kcodes + (long)g * G * d, ks + (long)g * d, kz + (long)g * d);
    for (int t = 0; t < nq; ++t)
        orc_quantize_value_token_cb(v + (long)t * d, d, vbits, vlev, vcodes + (long)t * d, vs + t, vz + t);
    return nq;
}

int orc_append_stream_cb(uint16_t *hist_k, uint16_t *hist_v, int cap, int *n, int *nq,
                         const uint16_t *k_new, const uint16_t *v_new, int d,
                         int kbits, int vbits, int G, int R,
                         uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                         uint8_t *vcodes, uint16_t *vs, uint16_t *vz)
{
    if (*n >= cap) return -1;
    memcpy(hist_k + (long)(*n) * d, k_new, sizeof(uint16_t) * d);
    memcpy(hist_v + (long)(*n) * d, v_new, sizeof(uint16_t) * d);
    *n += 1;
    if (*n - *nq == R + G) {
        double klev[256], vlev[256];
        orc_codebook_levels(kbits, klev);
        orc_codebook_levels(vbits, vlev);
        int g = *nq / G;
        orc_quantize_key_group_cb(hist_k + (long)(*nq) * d, G, d, kbits, klev,
                                  kcodes + (long)(*nq) * d, ks + (long)g * d, kz + (long)g * d);
        for (int t = *nq; t < *nq + G; ++t)
            orc_quantize_value_token_cb(hist_v + (long)t * d, d, vbits, vlev,
                                        vcodes + (long)t * d, vs + t, vz + t);
        *nq += G;
        return 1;
    }
    return 0;
}

void orc_dequantize_stream_cb(const uint16_t *k, const uint16_t *v, int n, int nq, int d, int G,
                              int kbits, int vbits,
                              const uint8_t *kcodes, const uint16_t *ks, const uint16_t *kz,
                              const uint8_t *vcodes, const uint16_t *vs, const uint16_t *vz,
                              float *out_k, float *out_v)
{
    double klev[256], vlev[256];
    orc_codebook_levels(kbits, klev);
    orc_codebook_levels(vbits, vlev);
    for (int t = 0; t < n; ++t) {
        for (int c = 0; c < d; ++c) {
            long i = (long)t * d + c;
            if (t < nq) {
                long gi = (long)(t / G) * d + c;
                out_k[i] = fmaf((float)klev[kcodes[i]], orc_h2f(ks[gi]), orc_h2f(kz[gi]));
                out_v[i] = fmaf((float)vlev[vcodes[i]], orc_h2f(vs[t]), orc_h2f(vz[t]));
            } else {
                out_k[i] = orc_h2f(k[i]);
                out_v[i] = orc_h2f(v[i]);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Dense-and-sparse keys ([P3] exp. 03, closing paragraph: KVQuant keeps the  */
/* few extreme values in fp16 as a sparse matrix and quantizes the rest).    */
/* Per key group of G tokens (one kv head): the n_out entries of largest     */
/* magnitude |x| (ties: the lower position t*d + c first) are kept exactly;  */
/* each channel's min, max, scale and zero are taken over its other values  */
/* (none left: s = z = 0) and those values are quantized with the group     */
/* quantizer above; a kept position's code is 0 and it dequantizes to the    */
/* kept value.                                                               */
/* ------------------------------------------------------------------------ */

struct mag_pos {
    float mag;
    int pos;
};

/* larger magnitude first, then the lower position */
static int cmp_magnitude_desc(const void *a, const void *b)
{
    const struct mag_pos *p = (const struct mag_pos *)a, *q = (const struct mag_pos *)b;
    if (p->mag != q->mag) return p->mag > q->mag ? -1 : 1;
    return p->pos < q->pos ? -1 : (p->pos > q->pos ? 1 : 0);
}

static int cmp_int_asc(const void *a, const void *b)
{
    int i = *(const int *)a, j = *(const int *)b;
    return i < j ? -1 : (i > j ? 1 : 0);
}

/* x, codes: [G][d]; s, z: [d]; out_pos (t*d + c, ascending), out_val (fp16
 * bits): [n_out].  lev: the codebook's levels, or NULL for the uniform grid. */
void orc_quantize_key_group_ds(const uint16_t *x, int G, int d, int bits, int n_out, const double *lev,
                               uint8_t *codes, uint16_t *s, uint16_t *z,
                               uint16_t *out_pos, uint16_t *out_val)
{
    const int n = G * d, qmax = (1 << bits) - 1;
    struct mag_pos *e = (struct mag_pos *)malloc(sizeof(struct mag_pos) * n);
    int *idx = (int *)malloc(sizeof(int) * n_out);
    char *kept = (char *)calloc(n, 1);
    for (int i = 0; i < n; ++i) {
        e[i].mag = fabsf(orc_h2f(x[i]));
        e[i].pos = i;
    }
    qsort(e, n, sizeof(struct mag_pos), cmp_magnitude_desc);
    for (int k = 0; k < n_out; ++k) idx[k] = e[k].pos;
    qsort(idx, n_out, sizeof(int), cmp_int_asc);
    for (int k = 0; k < n_out; ++k) {
        kept[idx[k]] = 1;
        out_pos[k] = (uint16_t)idx[k];
        out_val[k] = x[idx[k]];
    }
    free(e);
    for (int c = 0; c < d; ++c) {
        int any = 0;
        float mn = 0.0f, mx = 0.0f;
        for (int t = 0; t < G; ++t) {
            if (kept[t * d + c]) continue;
            float v = orc_h2f(x[t * d + c]);
            if (!any || v < mn) mn = v;
            if (!any || v > mx) mx = v;
            any = 1;
        }
        mn = mn + 0.0f;
        mx = mx + 0.0f;
        float s32 = (mx - mn) / (float)qmax;
        uint16_t s16 = orc_f2h(s32);
        uint16_t z16 = orc_f2h(mn);
        float sf = orc_h2f(s16);
        float zf = orc_h2f(z16);
        float inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;
        for (int t = 0; t < G; ++t) {
            if (kept[t * d + c]) {
                codes[t * d + c] = 0;
                continue;
            }
            float v = orc_h2f(x[t * d + c]);
            float tt = (v - zf) * inv;
            if (lev) { /* nearest codebook level, ties to the even code (quantize_set_cb) */
                int code = 0;
                for (int k = 0; k < qmax; ++k) {
                    float m = (float)(0.5 * (lev[k] + lev[k + 1]));
                    if ((k % 2 == 0) ? (tt > m) : (tt >= m)) code += 1;
                }
                codes[t * d + c] = (uint8_t)code;
                continue;
            }
            float r = rintf(tt);
            if (r < 0.0f) r = 0.0f;
            if (r > (float)qmax) r = (float)qmax;
            codes[t * d + c] = (uint8_t)r;
        }
        s[c] = s16;
        z[c] = z16;
    }
    free(idx);
    free(kept);
}

/* One value token on the uniform grid (grid 0) or the codebook (grid 1). */
static void quantize_value_token_grid(const uint16_t *x, int d, int bits, int grid, uint8_t *codes,
                                      uint16_t *s, uint16_t *z)
{
    if (grid) {
        double lev[256];
        orc_codebook_levels(bits, lev);
        orc_quantize_value_token_cb(x, d, bits, lev, codes, s, z);
    } else {
        orc_quantize_value_token(x, d, bits, codes, s, z);
    }
}

/* Whole stream with dense-and-sparse keys (n_out kept entries per key
 * group) on the uniform grid (grid 0) or the codebook (grid 1); values as in
 * orc_prefill_stream(_cb).  opos, oval: [n_q/G][n_out]. */
int orc_prefill_stream_ds(const uint16_t *k, const uint16_t *v, int n, int d,
                          int kbits, int vbits, int G, int R, int n_out, int grid,
                          uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                          uint8_t *vcodes, uint16_t *vs, uint16_t *vz,
                          uint16_t *opos, uint16_t *oval)
{
    double klev[256];
    if (grid) orc_codebook_levels(kbits, klev);
    int nq = orc_num_quantized(n, G, R);
    for (int g = 0; g < nq / G; ++g)
        orc_quantize_key_group_ds(k + (long)g * G * d, G, d, kbits, n_out, grid ? klev : NULL,
                                  kcodes + (long)g * G * d, ks + (long)g * d, kz + (long)g * d,
                                  opos + (long)g * n_out, oval + (long)g * n_out);
    for (int t = 0; t < nq; ++t)
        quantize_value_token_grid(v + (long)t * d, d, vbits, grid, vcodes + (long)t * d, vs + t, vz + t);
    return nq;
}

int orc_append_stream_ds(uint16_t *hist_k, uint16_t *hist_v, int cap, int *n, int *nq,
                         const uint16_t *k_new, const uint16_t *v_new, int d,
                         int kbits, int vbits, int G, int R, int n_out, int grid,
                         uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                         uint8_t *vcodes, uint16_t *vs, uint16_t *vz,
                         uint16_t *opos, uint16_t *oval)
{
    if (*n >= cap) return -1;
    memcpy(hist_k + (long)(*n) * d, k_new, sizeof(uint16_t) * d);
    memcpy(hist_v + (long)(*n) * d, v_new, sizeof(uint16_t) * d);
    *n += 1;
    if (*n - *nq == R + G) {
        int g = *nq / G;
        double klev[256];
        if (grid) orc_codebook_levels(kbits, klev);
        orc_quantize_key_group_ds(hist_k + (long)(*nq) * d, G, d, kbits, n_out, grid ? klev : NULL,
                                  kcodes + (long)(*nq) * d, ks + (long)g * d, kz + (long)g * d,
                                  opos + (long)g * n_out, oval + (long)g * n_out);
        for (int t = *nq; t < *nq + G; ++t)
            quantize_value_token_grid(hist_v + (long)t * d, d, vbits, grid, vcodes + (long)t * d, vs + t, vz + t);
        *nq += G;
        return 1;
    }
    return 0;
}

void orc_dequantize_stream_ds(const uint16_t *k, const uint16_t *v, int n, int nq, int d, int G, int n_out,
                              int kbits, int vbits, int grid,
                              const uint8_t *kcodes, const uint16_t *ks, const uint16_t *kz,
                              const uint8_t *vcodes, const uint16_t *vs, const uint16_t *vz,
                              const uint16_t *opos, const uint16_t *oval,
                              float *out_k, float *out_v)
{
    if (grid)
        orc_dequantize_stream_cb(k, v, n, nq, d, G, kbits, vbits, kcodes, ks, kz, vcodes, vs, vz, out_k, out_v);
    else
        orc_dequantize_stream(k, v, n, nq, d, G, kcodes, ks, kz, vcodes, vs, vz, out_k, out_v);
    for (int g = 0; g < nq / G; ++g)
        for (int e = 0; e < n_out; ++e) {
            int p = opos[(long)g * n_out + e];
            out_k[(long)g * G * d + p] = orc_h2f(oval[(long)g * n_out + e]);
        }
}

/* ------------------------------------------------------------------------ */
/* 8-bit KV formats ([P1] section 3.1: FP8 E4M3 with a static per-tensor or  */
/* per-head scale, or INT8 with a dynamic per-token scale, dequantized by    */
/* the attention kernel as it reads; [P2] part B.1: FP8 and INT8 hold the    */
/* cache at half the fp16 bytes).  Tokens [0, n_q) are quantized, every      */
/* token on its own (no per-channel key groups).  With no residual window    */
/* (R = 0) every token is quantized as it is written, n_q = n: a per-token   */
/* quantizer needs no group to be complete, and the pages' 8-bit cache      */
/* stores each token in 8 bits.  With R > 0 the low-bit format's residual    */
/* window and group flushes apply.                                           */
/* ------------------------------------------------------------------------ */

#define ORC_FMT_INT8 1
#define ORC_FMT_FP8_E4M3 2

/* FP8 E4M3 (the OCP "FN" variant): 1 sign bit, 4 exponent bits (bias 7), 3
 * fraction bits; exponent 0 holds subnormals (fraction * 2^-9); there is no
 * infinity, and only exponent 15 with fraction 7 is NaN, so the largest
 * finite value is 1.75 * 2^8 = 448. */
float orc_fp8_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int expo = (c >> 3) & 0xf;
    int frac = c & 7;
    double v;
    if (expo == 15 && frac == 7)
        v = NAN;
    else if (expo == 0)
        v = ldexp((double)frac, -9);
    else
        v = ldexp((double)(frac + 8), expo - 10);
    return (float)(sign ? -v : v);
}

/* Nearest E4M3 value of a float, ties to even, saturating at +-448; the sign
 * of a value that rounds to zero is kept (code 0x80 for -0). */
uint8_t orc_fp8_e4m3_encode(float xf)
{
    double x = (double)xf;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint8_t)(sign | 0x7f);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7e);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9 with m an integer 0..8 */
        double m = rint(ldexp(a, 9)); /* exact scaling; ties to even */
        return (uint8_t)(sign | (uint8_t)m); /* m == 8 is the smallest normal */
    }
    int e2;
    frexp(a, &e2);
    int e = e2 - 1;                    /* a in [2^e, 2^(e+1)), -6 <= e <= 8 */
    double m = rint(ldexp(a, 3 - e));  /* in [8, 16] */
    if (m == 16.0) {
        m = 8.0;
        e += 1;
    }
    /* a < 448 rounds to at most 448 = 1.75 * 2^8 (e = 8, m = 14) */
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)((int)m - 8));
}

/* One token under a static scale: code = E4M3(x * (1/scale)), the quotient
 * clamped to +-448 first.  A scale that is not positive gives 1/scale := 0
 * (all codes +0). */
void orc_quantize_token_fp8(const uint16_t *x, int d, float scale, uint8_t *codes)
{
    float inv = (scale > 0.0f) ? 1.0f / scale : 0.0f;
    for (int c = 0; c < d; ++c) {
        float t = orc_h2f(x[c]) * inv;
        if (t > 448.0f) t = 448.0f;
        if (t < -448.0f) t = -448.0f;
        codes[c] = orc_fp8_e4m3_encode(t);
    }
}

/* One key or value token of an 8-bit format.  INT8: the min/max quantizer
 * above with 8 bits over the token's d channels (dynamic, per token), scale
 * and zero in *s, *z.  FP8: the static scale; *s = *z = 0. */
static void quantize_token8(int fmt, const uint16_t *x, int d, float scale,
                            uint8_t *codes, uint16_t *s, uint16_t *z)
{
    if (fmt == ORC_FMT_FP8_E4M3) {
        orc_quantize_token_fp8(x, d, scale, codes);
        *s = 0;
        *z = 0;
    } else {
        quantize_set(x, d, 1, 8, codes, 1, s, z);
    }
}

/* Quantized tokens of an 8-bit stream holding n tokens (see above). */
int orc_num_quantized8(int n, int G, int R)
{
    if (R == 0) return n > 0 ? n : 0;
    return orc_num_quantized(n, G, R);
}

/* Whole-stream quantization in an 8-bit format (fmt 1 = INT8 per token,
 * 2 = FP8 E4M3 with static scales kscale / vscale of this kv head).
 * k, v: [n][d]; kcodes, vcodes: [n_q][d]; ks, kz, vs, vz: [n_q] (INT8 only,
 * zeros for FP8).  Returns n_q. */
int orc_prefill_stream8(int fmt, const uint16_t *k, const uint16_t *v, int n, int d, int G, int R,
                        float kscale, float vscale,
                        uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                        uint8_t *vcodes, uint16_t *vs, uint16_t *vz)
{
    int nq = orc_num_quantized8(n, G, R);
    for (int t = 0; t < nq; ++t) {
        quantize_token8(fmt, k + (long)t * d, d, kscale, kcodes + (long)t * d, ks + t, kz + t);
        quantize_token8(fmt, v + (long)t * d, d, vscale, vcodes + (long)t * d, vs + t, vz + t);
    }
    return nq;
}

/* Incremental form of orc_prefill_stream8: with R = 0 the new token is
 * quantized at once; otherwise the same flush rule as orc_append_stream (the
 * oldest G tail tokens once the tail holds R + G).  Returns 1 when tokens
 * were quantized. */
int orc_append_stream8(int fmt, uint16_t *hist_k, uint16_t *hist_v, int cap, int *n, int *nq,
                       const uint16_t *k_new, const uint16_t *v_new, int d, int G, int R,
                       float kscale, float vscale,
                       uint8_t *kcodes, uint16_t *ks, uint16_t *kz,
                       uint8_t *vcodes, uint16_t *vs, uint16_t *vz)
{
    if (*n >= cap) return -1;
    memcpy(hist_k + (long)(*n) * d, k_new, sizeof(uint16_t) * d);
    memcpy(hist_v + (long)(*n) * d, v_new, sizeof(uint16_t) * d);
    *n += 1;
    if (R == 0) {
        int t = *n - 1;
        quantize_token8(fmt, hist_k + (long)t * d, d, kscale, kcodes + (long)t * d, ks + t, kz + t);
        quantize_token8(fmt, hist_v + (long)t * d, d, vscale, vcodes + (long)t * d, vs + t, vz + t);
        *nq = *n;
        return 1;
    }
    if (*n - *nq == R + G) {
        for (int t = *nq; t < *nq + G; ++t) {
            quantize_token8(fmt, hist_k + (long)t * d, d, kscale, kcodes + (long)t * d, ks + t, kz + t);
            quantize_token8(fmt, hist_v + (long)t * d, d, vscale, vcodes + (long)t * d, vs + t, vz + t);
        }
        *nq += G;
        return 1;
    }
    return 0;
}

/* Dequantized stream of an 8-bit format.  INT8: fmaf(code, s_t, z_t); FP8:
 * E4M3(code) * scale, one fp32 rounding; residual tokens as stored. */
void orc_dequantize_stream8(int fmt, const uint16_t *k, const uint16_t *v, int n, int nq, int d,
                            float kscale, float vscale,
                            const uint8_t *kcodes, const uint16_t *ks, const uint16_t *kz,
                            const uint8_t *vcodes, const uint16_t *vs, const uint16_t *vz,
                            float *out_k, float *out_v)
{
    for (int t = 0; t < n; ++t) {
        for (int c = 0; c < d; ++c) {
            long i = (long)t * d + c;
            if (t < nq && fmt == ORC_FMT_FP8_E4M3) {
                out_k[i] = orc_fp8_e4m3_decode(kcodes[i]) * kscale;
                out_v[i] = orc_fp8_e4m3_decode(vcodes[i]) * vscale;
            } else if (t < nq) {
                out_k[i] = fmaf((float)kcodes[i], orc_h2f(ks[t]), orc_h2f(kz[t]));
                out_v[i] = fmaf((float)vcodes[i], orc_h2f(vs[t]), orc_h2f(vz[t]));
            } else {
                out_k[i] = orc_h2f(k[i]);
                out_v[i] = orc_h2f(v[i]);
            }
        }
    }
}

/* Bytes of one stream in an 8-bit format: one byte per code, plus (INT8) an
 * fp16 (scale, zero) pair per quantized key token and per value token, plus
 * the fp16 residual.  FP8's static scales belong to the layer, not to a
 * stream, and are not counted. */
double orc_stream_bytes8(int fmt, long n, int d, int G, int R)
{
    long nq = orc_num_quantized8((int)n, G, R);
    double codes = (double)nq * d * 2.0;
    double meta = fmt == ORC_FMT_INT8 ? (double)nq * 8.0 : 0.0;
    double resid = (double)(n - nq) * d * 2.0 * 2.0;
    return codes + meta + resid;
}

void orc_fp8_decode_array(const uint8_t *c, float *f, long count)
{
    for (long i = 0; i < count; ++i) f[i] = orc_fp8_e4m3_decode(c[i]);
}

void orc_fp8_encode_array(const float *f, uint8_t *c, long count)
{
    for (long i = 0; i < count; ++i) c[i] = orc_fp8_e4m3_encode(f[i]);
}

/* ------------------------------------------------------------------------ */
/* Pre-RoPE keys ([P1] section 3.3: quantize the keys before the rotary      */
/* position embedding, whose rotation makes an outlier channel's values vary */
/* from token to token and widens the per-channel ranges, and apply RoPE to  */
/* the keys when they are read; [P1] section 2: RoPE rotates each pair of     */
/* dimensions and keeps the pair's norm; [P3] exp. 03: the two dimensions of */
/* a pair are adjacent).  Token t's pair i = (2i, 2i+1) is rotated by the    */
/* angle t * theta_i, theta_i = base^(-2i/d), counter-clockwise:             */
/*   k'[2i]   = k[2i] cos(a) - k[2i+1] sin(a)                                 */
/*   k'[2i+1] = k[2i] sin(a) + k[2i+1] cos(a)                                 */
/* (the rotary embedding's own definition), all in fp64.                     */
/* ------------------------------------------------------------------------ */

/* Rotates rows [0, n) of k (fp32, [n][d]) as tokens at positions
 * pos0 .. pos0 + n - 1 into out (fp64 [n][d]). */
void orc_rope_rotate(const float *k, int n, int d, long pos0, double base, double *out)
{
    for (int t = 0; t < n; ++t) {
        for (int i = 0; i < d / 2; ++i) {
            double theta = pow(base, -2.0 * (double)i / (double)d);
            double a = (double)(pos0 + t) * theta;
            double c = cos(a), s = sin(a);
            double x0 = (double)k[(long)t * d + 2 * i];
            double x1 = (double)k[(long)t * d + 2 * i + 1];
            out[(long)t * d + 2 * i] = x0 * c - x1 * s;
            out[(long)t * d + 2 * i + 1] = x0 * s + x1 * c;
        }
    }
}

/* Attention over fp64 keys (e.g. keys rotated by orc_rope_rotate): the same
 * function as orc_attention, reading the keys in fp64. */
void orc_attention_d(const float *q, int gq, const double *kh, const float *vh, int n, int d,
                     float scale, double *out)
{
    attention_core(q, gq, NULL, kh, vh, n, d, scale, out, NULL);
}

/* ------------------------------------------------------------------------ */
/* Byte accounting ([P4] M_KV = 2 L H_kv n d_h b; [P1] 8.1 per-token table).  */
/* ------------------------------------------------------------------------ */

/* Bytes of one (sequence, kv-head) stream holding n tokens in the KIVI
 * format: packed key and value codes for the n_q quantized tokens, one fp16
 * (scale, zero) pair per (key group, channel) and per quantized value token,
 * and fp16 keys and values for the n - n_q residual tokens.  Bit widths of 16
 * mean "not quantized" (plain fp16 cache, no metadata). */
double orc_stream_bytes(long n, int d, int kbits, int vbits, int G, int R)
{
    if (kbits == 16 && vbits == 16) return 2.0 * (double)n * d * 2.0;
    long nq = orc_num_quantized((int)n, G, R);
    double codes = (double)nq * d * (kbits + vbits) / 8.0;
    double kmeta = (double)(nq / G) * d * 4.0;
    double vmeta = (double)nq * 4.0;
    double resid = (double)(n - nq) * d * 2.0 * 2.0;
    return codes + kmeta + vmeta + resid;
}

/* [P4] closed form for an unquantized cache: 2 * L * H_kv * n * d_h * b. */
double orc_kv_bytes_closed_form(long L, long Hkv, long n, long d, double bytes_per_elem)
{
    return 2.0 * (double)L * (double)Hkv * (double)n * (double)d * bytes_per_elem;
}

/* Array helpers so the tests can run the codec over every bit pattern. */
void orc_h2f_array(const uint16_t *h, float *f, long count)
{
    for (long i = 0; i < count; ++i) f[i] = orc_h2f(h[i]);
}

void orc_f2h_array(const float *f, uint16_t *h, long count)
{
    for (long i = 0; i < count; ++i) h[i] = orc_f2h(f[i]);
}
