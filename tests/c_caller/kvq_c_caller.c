/*
 * A plain C caller of the library's C ABI (include/kvq.h): device memory from
 * hipMalloc, no Python and no torch, so the boundary is exercised the way a
 * C or C++ serving loop would use it.
 *
 * Two caches: contiguous (INT2 keys, INT4 values, G = 32, R = 64) and paged
 * (INT4 keys, INT2 values, G = 16, R = 32), whose block table this program
 * keeps as the header asks of a caller: a block id from a shuffled pool for
 * every key group before the call that quantizes it (the prefill, or the
 * append that flushes the group).  For each, it quantizes a small seeded
 * batch (kv_quantize_prefill), appends tokens across group flushes
 * (kv_append_token), reads the cache back (kv_dequantize) and runs decode
 * attention (kv_decode_attention, and the no-allocation form), then checks
 * against the oracle (oracle/kvq_oracle.c, test infrastructure, linked into
 * this test program only):
 *   - dequantized keys and values bit for bit, zeros past each sequence;
 *   - attention within max-abs 2e-3 and per-row cosine 0.9999 of the
 *     oracle's fp64 attention over the same dequantized cache;
 *   - the no-allocation call equal to the workspace call bit for bit.
 * Method: "KV cache compression: quantization, eviction and sparse
 * attention", section 3.2 (per-channel key groups, per-token values, fp16
 * residual window); the attention definition from "KV cache compression"
 * (jaedaily), formula paragraph.
 *
 * Exit status 0 when every check passes, 1 otherwise (2: a call failed).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvq.h"

/* oracle (test infrastructure) */
float orc_h2f(uint16_t h);
uint16_t orc_f2h(float x);
int orc_prefill_stream(const uint16_t *k, const uint16_t *v, int n, int d, int kbits, int vbits, int G, int R,
                       uint8_t *kcodes, uint16_t *ks, uint16_t *kz, uint8_t *vcodes, uint16_t *vs, uint16_t *vz);
int orc_append_stream(uint16_t *hist_k, uint16_t *hist_v, int cap, int *n, int *nq, const uint16_t *k_new,
                      const uint16_t *v_new, int d, int kbits, int vbits, int G, int R, uint8_t *kcodes,
                      uint16_t *ks, uint16_t *kz, uint8_t *vcodes, uint16_t *vs, uint16_t *vz);
void orc_dequantize_stream(const uint16_t *k, const uint16_t *v, int n, int nq, int d, int G,
                           const uint8_t *kcodes, const uint16_t *ks, const uint16_t *kz, const uint8_t *vcodes,
                           const uint16_t *vs, const uint16_t *vz, float *out_k, float *out_v);
void orc_attention(const float *q, int gq, const float *kh, const float *vh, int n, int d, float scale,
                   double *out, double *weights);

enum { B = 3, H = 2, GQ = 4, HQ = H * GQ, D = 128, CAP = 400, MAXG = 64 };

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
            exit(2);                                                                \
        }                                                                           \
    } while (0)
#define KVQ_OK_(x)                                                                  \
    do {                                                                            \
        kvq_status s_ = (x);                                                        \
        if (s_ != KVQ_OK) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #x, kvq_status_string(s_));          \
            exit(2);                                                                \
        }                                                                           \
    } while (0)

/* seeded inputs: xorshift64*, sums of uniforms (roughly normal), a few
 * channels of each kv head scaled up like the outlier channels of keys */
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform01(void)
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normalish(void)
{
    double s = 0.0;
    for (int i = 0; i < 4; ++i) s += uniform01();
    return (float)((s - 2.0) * 1.7320508075688772);
}

static int num_quantized(int n, int G, int R)
{
    return n <= R ? 0 : G * ((n - R) / G);
}

/* One cache: prefill, STEPS appends, read back, attention, checks.  Returns
 * 0 when every check passes. */
static int run(int paged, int KB, int VB, int G, int R)
{
    const int STEPS = 2 * G + R / 2 + 5;
    const int lens0[B] = {150, 0, 77};
    int T = 0;
    for (int b = 0; b < B; ++b)
        if (lens0[b] + STEPS > T) T = lens0[b] + STEPS;
    /* every token of every stream, [B][H][T][D] fp16 */
    const long all = (long)B * H * T * D;
    uint16_t *Kh = malloc(sizeof(uint16_t) * all), *Vh = malloc(sizeof(uint16_t) * all);
    for (long i = 0; i < all; ++i) {
        const int c = (int)(i % D);
        Kh[i] = orc_f2h(normalish() * ((c % 37) == 5 ? 12.0f : 1.0f));
        Vh[i] = orc_f2h(normalish());
    }
    uint16_t qh[B * HQ * D];
    for (int i = 0; i < B * HQ * D; ++i) qh[i] = orc_f2h(normalish());

    kvq_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.num_seqs = B;
    cfg.num_kv_heads = H;
    cfg.head_dim = D;
    cfg.k_bits = KB;
    cfg.v_bits = VB;
    cfg.group_size = G;
    cfg.residual = R;
    cfg.max_tokens = paged ? 0 : CAP;
    if (paged) {
        cfg.block_size = G;
        cfg.max_blocks_per_seq = MAXG;
        cfg.num_blocks = B * MAXG;
    }
    cfg.kv_format = KVQ_FORMAT_KIVI;
    cfg.grid = KVQ_GRID_UNIFORM;
    kvq_sizes sz;
    KVQ_OK_(kvq_buffer_sizes(&cfg, &sz));

    kvq_cache cache;
    memset(&cache, 0, sizeof cache);
    HIP_OK(hipMalloc(&cache.packed, sz.packed_bytes));
    HIP_OK(hipMalloc(&cache.k_res, sz.residual_bytes));
    HIP_OK(hipMalloc(&cache.v_res, sz.residual_bytes));
    HIP_OK(hipMalloc((void **)&cache.n_tokens, sz.counter_bytes));
    HIP_OK(hipMalloc((void **)&cache.n_quant, sz.counter_bytes));
    HIP_OK(hipMalloc((void **)&cache.arrivals, sz.counter_bytes));
    HIP_OK(hipMemset(cache.arrivals, 0, sz.counter_bytes));
    HIP_OK(hipMemset(cache.n_tokens, 0, sz.counter_bytes));
    HIP_OK(hipMemset(cache.n_quant, 0, sz.counter_bytes));
    /* paged: the block table and a pool handed out in a seeded shuffled order */
    int32_t table[B * MAXG], assigned[B] = {0}, pool[B * MAXG], pool_next = 0;
    int32_t *dtable = NULL;
    if (paged) {
        for (int i = 0; i < B * MAXG; ++i) {
            table[i] = -1;
            pool[i] = i;
        }
        for (int i = B * MAXG - 1; i > 0; --i) {
            const int j = (int)(uniform01() * (i + 1));
            const int32_t t = pool[i];
            pool[i] = pool[j];
            pool[j] = t;
        }
        HIP_OK(hipMalloc((void **)&dtable, sz.block_table_bytes));
        cache.block_table = dtable;
    }
    /* every sequence gets a block for each key group it will hold after the
     * next call, before that call */
#define ASSIGN_BLOCKS(NEXT_LEN)                                                           \
    do {                                                                                \
        if (!paged) break;                                                              \
        for (int b_ = 0; b_ < B; ++b_)                                                  \
            for (int g_ = assigned[b_]; g_ < num_quantized((NEXT_LEN)[b_], G, R) / G; ++g_) \
                table[b_ * MAXG + g_] = pool[pool_next++];                              \
        for (int b_ = 0; b_ < B; ++b_)                                                  \
            assigned[b_] = num_quantized((NEXT_LEN)[b_], G, R) / G;                    \
        HIP_OK(hipMemcpy(dtable, table, sizeof table, hipMemcpyHostToDevice));          \
    } while (0)

    /* prefill: the first lens0[b] tokens, as [B][H][L][D] with L = max lens0 */
    int L = 0;
    for (int b = 0; b < B; ++b)
        if (lens0[b] > L) L = lens0[b];
    uint16_t *kp = malloc(sizeof(uint16_t) * B * H * L * D), *vp = malloc(sizeof(uint16_t) * B * H * L * D);
    for (int bh = 0; bh < B * H; ++bh)
        for (int t = 0; t < L; ++t) {
            memcpy(kp + ((long)bh * L + t) * D, Kh + ((long)bh * T + t) * D, sizeof(uint16_t) * D);
            memcpy(vp + ((long)bh * L + t) * D, Vh + ((long)bh * T + t) * D, sizeof(uint16_t) * D);
        }
    void *dk, *dv, *dlens, *dkn, *dvn, *dq, *dout, *dout2, *dws, *dko, *dvo;
    HIP_OK(hipMalloc(&dk, sizeof(uint16_t) * B * H * L * D));
    HIP_OK(hipMalloc(&dv, sizeof(uint16_t) * B * H * L * D));
    HIP_OK(hipMalloc(&dlens, sizeof(int32_t) * B));
    HIP_OK(hipMemcpy(dk, kp, sizeof(uint16_t) * B * H * L * D, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, vp, sizeof(uint16_t) * B * H * L * D, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dlens, lens0, sizeof(int32_t) * B, hipMemcpyHostToDevice));
    ASSIGN_BLOCKS(lens0);
    KVQ_OK_(kv_quantize_prefill(&cfg, &cache, dk, dv, L, (const int32_t *)dlens, NULL));

    /* appends: token lens0[b] + s of every stream at step s */
    HIP_OK(hipMalloc(&dkn, sizeof(uint16_t) * B * H * D));
    HIP_OK(hipMalloc(&dvn, sizeof(uint16_t) * B * H * D));
    uint16_t kn[B * H * D], vn[B * H * D];
    for (int s = 0; s < STEPS; ++s) {
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h) {
                const long src = (((long)b * H + h) * T + lens0[b] + s) * D;
                memcpy(kn + (b * H + h) * D, Kh + src, sizeof(uint16_t) * D);
                memcpy(vn + (b * H + h) * D, Vh + src, sizeof(uint16_t) * D);
            }
        HIP_OK(hipMemcpy(dkn, kn, sizeof kn, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dvn, vn, sizeof vn, hipMemcpyHostToDevice));
        int next[B];
        for (int b = 0; b < B; ++b) next[b] = lens0[b] + s + 1;
        ASSIGN_BLOCKS(next);
        KVQ_OK_(kv_append_token(&cfg, &cache, dkn, dvn, NULL));
    }

    /* read back, and attention */
    const int OT = T + G;   /* past every sequence: must read back as zeros */
    HIP_OK(hipMalloc(&dko, sizeof(float) * B * H * OT * D));
    HIP_OK(hipMalloc(&dvo, sizeof(float) * B * H * OT * D));
    KVQ_OK_(kv_dequantize(&cfg, &cache, (float *)dko, (float *)dvo, OT, NULL));
    const size_t wsb = kv_decode_attention_workspace_bytes(&cfg, HQ);
    if (wsb == 0) {
        fprintf(stderr, "kv_decode_attention_workspace_bytes returned 0\n");
        return 2;
    }
    HIP_OK(hipMalloc(&dws, wsb));
    HIP_OK(hipMalloc(&dq, sizeof qh));
    HIP_OK(hipMalloc(&dout, sizeof(float) * B * HQ * D));
    HIP_OK(hipMalloc(&dout2, sizeof(float) * B * HQ * D));
    HIP_OK(hipMemcpy(dq, qh, sizeof qh, hipMemcpyHostToDevice));
    const float scale = 1.0f / sqrtf((float)D);
    KVQ_OK_(kv_decode_attention(&cfg, &cache, dq, HQ, scale, (float *)dout, dws, wsb, NULL));
    KVQ_OK_(kv_decode_attention_noalloc(&cfg, &cache, dq, HQ, scale, (float *)dout2, NULL));
    HIP_OK(hipDeviceSynchronize());
    float *ko = malloc(sizeof(float) * B * H * OT * D), *vo = malloc(sizeof(float) * B * H * OT * D);
    float out[B * HQ * D], out2[B * HQ * D];
    HIP_OK(hipMemcpy(ko, dko, sizeof(float) * B * H * OT * D, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(vo, dvo, sizeof(float) * B * H * OT * D, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out2, dout2, sizeof out2, hipMemcpyDeviceToHost));

    /* oracle: prefill then the same appends, per stream */
    int bad = 0;
    double max_err = 0.0, min_cos = 1.0;
    uint8_t *kc = malloc(CAP * D), *vc = malloc(CAP * D);
    uint16_t *ks = malloc(sizeof(uint16_t) * CAP * D / G + 2), *kz = malloc(sizeof(uint16_t) * CAP * D / G + 2);
    uint16_t vs[CAP], vz[CAP];
    uint16_t *hk = malloc(sizeof(uint16_t) * CAP * D), *hv = malloc(sizeof(uint16_t) * CAP * D);
    float *ok = malloc(sizeof(float) * CAP * D), *ov = malloc(sizeof(float) * CAP * D);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const long base = ((long)b * H + h) * T * D;
            int n = lens0[b];
            memcpy(hk, Kh + base, sizeof(uint16_t) * n * D);
            memcpy(hv, Vh + base, sizeof(uint16_t) * n * D);
            int nq = orc_prefill_stream(hk, hv, n, D, KB, VB, G, R, kc, ks, kz, vc, vs, vz);
            for (int s = 0; s < STEPS; ++s) {
                const long src = base + (long)(lens0[b] + s) * D;
                if (orc_append_stream(hk, hv, CAP, &n, &nq, Kh + src, Vh + src, D, KB, VB, G, R, kc, ks, kz, vc,
                                      vs, vz) < 0) {
                    fprintf(stderr, "oracle capacity exceeded\n");
                    return 2;
                }
            }
            orc_dequantize_stream(hk, hv, n, nq, D, G, kc, ks, kz, vc, vs, vz, ok, ov);
            const float *gk = ko + ((long)b * H + h) * OT * D, *gv = vo + ((long)b * H + h) * OT * D;
            if (memcmp(gk, ok, sizeof(float) * n * D) || memcmp(gv, ov, sizeof(float) * n * D)) {
                fprintf(stderr, "dequantized values differ: sequence %d, kv head %d\n", b, h);
                bad = 1;
            }
            for (long i = (long)n * D; i < (long)OT * D; ++i)
                if (gk[i] != 0.0f || gv[i] != 0.0f) {
                    fprintf(stderr, "nonzero past the end: sequence %d, kv head %d\n", b, h);
                    bad = 1;
                    break;
                }
            float qf[GQ * D];
            for (int i = 0; i < GQ * D; ++i) qf[i] = orc_h2f(qh[((long)b * HQ + h * GQ) * D + i]);
            double ref[GQ * D];
            orc_attention(qf, GQ, ok, ov, n, D, scale, ref, NULL);
            for (int r = 0; r < GQ; ++r) {
                const float *g = out + ((long)b * HQ + h * GQ + r) * D;
                double dot = 0.0, ng = 0.0, nr = 0.0;
                for (int c = 0; c < D; ++c) {
                    const double e = fabs((double)g[c] - ref[r * D + c]);
                    if (e > max_err) max_err = e;
                    dot += (double)g[c] * ref[r * D + c];
                    ng += (double)g[c] * g[c];
                    nr += ref[r * D + c] * ref[r * D + c];
                }
                const double cs = (ng == 0.0 && nr == 0.0) ? 1.0 : dot / sqrt(ng * nr);
                if (cs < min_cos) min_cos = cs;
            }
        }
    if (max_err > 2e-3 || min_cos < 0.9999) {
        fprintf(stderr, "attention outside the bar: max-abs %.3g, min cosine %.8f\n", max_err, min_cos);
        bad = 1;
    }
    if (memcmp(out, out2, sizeof out)) {
        fprintf(stderr, "the no-allocation call differs from the workspace call\n");
        bad = 1;
    }
    printf("c caller, %s: B=%d H=%d gq=%d k%d/v%d G=%d R=%d, %d appends: dequantized %s, attention max-abs %.3g "
           "min cosine %.8f, no-allocation call %s\n",
           paged ? "paged" : "contiguous", B, H, GQ, KB, VB, G, R, STEPS, bad ? "CHECK FAILED" : "bit-exact",
           max_err, min_cos, memcmp(out, out2, sizeof out) ? "differs" : "identical");
    void *bufs[] = {cache.packed, cache.k_res, cache.v_res, cache.n_tokens, cache.n_quant, cache.arrivals, dtable,
                    dk, dv, dlens, dkn, dvn, dq, dout, dout2, dws, dko, dvo};
    for (unsigned i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    free(Kh); free(Vh); free(kp); free(vp); free(ko); free(vo); free(kc); free(vc); free(ks); free(kz);
    free(hk); free(hv); free(ok); free(ov);
    return bad;
}

int main(void)
{
    int bad = run(0, 2, 4, 32, 64);
    bad |= run(1, 4, 2, 16, 32);
    return bad;
}
