// kvq_attn.hip -- split-K decode attention over the packed KIVI cache (gfx950).
//
// What it computes ("KV cache compression" (jaedaily), formula paragraph;
// "KV cache compression: quantization, eviction and sparse attention",
// sections 3.1, 3.2, 3.4 and 8.2): for every query head h of sequence b,
//   out = sum_t softmax_t(scale * q . k_t) v_t
// over the dequantized keys/values of the quantized groups and the fp16
// residual tokens.  The kernel dequantizes while it reads; the quantized part
// and the residual are processed by different workgroups and merged.
//
// Dequantization is folded into the arithmetic instead of materialised:
//   q . k_t  = sum_c (q_c s_c) code_tc + sum_c q_c z_c        (key group scales)
//   sum_t p_t v_t = sum_t (p_t s_t) code_t + (sum_t p_t z_t)    (value token scales)
// so each packed code costs one multiply-add per query head.  All query heads
// of one kv head (the GQA group) are served by the same workgroup, so every
// packed byte is read from HBM once per step.
//
// Split-K: each stream (b, kv head) is cut into `splits` ranges of key groups
// plus one workgroup for the residual ring; each writes (m, l, acc) partials,
// which attn_merge_kernel combines by log-sum-exp.
#include "kvq_device.h"

namespace kvq {

constexpr int kWaves = 4;
constexpr int kPartStride = kD + 2;   // partial: acc[128], m, l
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float x) {
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int GQ>
struct AttnSmem {
    float qt[kWaves][GQ][4][36];   // per wave: folded query (or raw query for the residual)
    float w[kWaves][GQ][16];       // per wave: p_t * s_t of the current 16 tokens
    float m[kWaves][GQ], l[kWaves][GQ], pz[kWaves][GQ];
};

// Per-wave online-softmax state.  Values in log2 units (query pre-scaled by
// scale * log2(e)), so exp2 is the exponential.
template <int GQ>
struct WaveState {
    float m[GQ], l[GQ], pz[GQ];
    float2 acc[GQ];   // channels 2*lane, 2*lane+1
};

// Update with the logits lg[hh] of 16 tokens held by lanes (token tl = lane/4,
// part = lane%4; all 4 parts hold the same value).  valid: token exists.
// vs, vz: value scale/zero of the lane's token.  Writes w = p*s to LDS.
template <int GQ>
__device__ __forceinline__ void softmax_16(WaveState<GQ>& st, float (&lg)[GQ], bool valid, float vs, float vz,
                                           float (*wbuf)[16], int tl, int part) {
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        const float x = valid ? lg[hh] : -INFINITY;
        const float mp = wave_max(x);
        const float mnew = fmaxf(st.m[hh], mp);
        float alpha, p;
        if (mnew == -INFINITY) {
            alpha = 1.0f;
            p = 0.0f;
        } else {
            alpha = exp2f(st.m[hh] - mnew);
            p = valid ? exp2f(x - mnew) : 0.0f;
        }
        st.m[hh] = mnew;
        st.l[hh] = st.l[hh] * alpha + (part == 0 ? p : 0.0f);
        st.pz[hh] = st.pz[hh] * alpha + (part == 0 ? p * vz : 0.0f);
        st.acc[hh].x *= alpha;
        st.acc[hh].y *= alpha;
        if (part == 0) wbuf[hh][tl] = p * vs;
    }
}

template <int KB>
__device__ __forceinline__ float kcode(const uint4& u, int i) {
    if (KB == 2) {
        const uint32_t w = i < 16 ? u.x : u.y;
        return (float)((w >> ((i & 15) * 2)) & 3u);
    } else {
        const uint32_t w = i < 8 ? u.x : (i < 16 ? u.y : (i < 24 ? u.z : u.w));
        return (float)((w >> ((i & 7) * 4)) & 15u);
    }
}

template <int GQ, int KB, int VB>
__device__ void attend_group(AttnSmem<GQ>& sm, WaveState<GQ>& st, const Layout& L, const uint8_t* __restrict__ rec,
                             const float2 (&qs)[GQ], int wave, int lane) {
    const int tl = lane >> 2, part = lane & 3;
    // Fold the group's key scales into the query; key zeros give a per-head bias.
    const uint2 km = *(const uint2*)(rec + L.kmeta_off + 8 * lane);
    const float s0 = h2f(km.x & 0xffffu), z0 = h2f(km.x >> 16);
    const float s1 = h2f(km.y & 0xffffu), z1 = h2f(km.y >> 16);
    float bias[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        *(float2*)&sm.qt[wave][hh][lane >> 4][(2 * lane) & 31] = make_float2(qs[hh].x * s0, qs[hh].y * s1);
        bias[hh] = wave_sum(qs[hh].x * z0 + qs[hh].y * z1);
    }
    wave_sync();

    for (int pass = 0; pass < L.G / 16; ++pass) {
        const int t = pass * 16 + tl;
        uint4 kc;
        if (KB == 2) {
            const uint2 x = *(const uint2*)(rec + t * 32 + part * 8);
            kc = make_uint4(x.x, x.y, 0, 0);
        } else {
            kc = *(const uint4*)(rec + t * 64 + part * 16);
        }
        const uint32_t vm = *(const uint32_t*)(rec + L.vmeta_off + 4 * t);
        float dot[GQ];
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) dot[hh] = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            const float c0 = kcode<KB>(kc, i), c1 = kcode<KB>(kc, i + 1);
            const float c2 = kcode<KB>(kc, i + 2), c3 = kcode<KB>(kc, i + 3);
#pragma unroll
            for (int hh = 0; hh < GQ; ++hh) {
                const float4 qv = *(const float4*)&sm.qt[wave][hh][part][i];
                dot[hh] += qv.x * c0 + qv.y * c1 + qv.z * c2 + qv.w * c3;
            }
        }
        float lg[GQ];
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
            float x = dot[hh];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            lg[hh] = x + bias[hh];
        }
        softmax_16<GQ>(st, lg, true, h2f(vm & 0xffffu), h2f(vm >> 16), sm.w[wave], tl, part);
        wave_sync();
        // values: lane owns channels 2*lane, 2*lane+1; units (pass, c) are adjacent
        uint32_t u0[2], u1[2];
        if (VB == 2) {
            const uint2 x = *(const uint2*)(rec + L.vcode_off + (pass * kD + 2 * lane) * 4);
            u0[0] = x.x; u1[0] = x.y;
        } else {
            const uint4 x = *(const uint4*)(rec + L.vcode_off + (pass * kD + 2 * lane) * 8);
            u0[0] = x.x; u0[1] = x.y; u1[0] = x.z; u1[1] = x.w;
        }
#pragma unroll
        for (int tt = 0; tt < 16; tt += 4) {
            float a[4], bb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = tt + j;
                if (VB == 2) {
                    a[j] = (float)((u0[0] >> (2 * k)) & 3u);
                    bb[j] = (float)((u1[0] >> (2 * k)) & 3u);
                } else {
                    a[j] = (float)((u0[k >> 3] >> (4 * (k & 7))) & 15u);
                    bb[j] = (float)((u1[k >> 3] >> (4 * (k & 7))) & 15u);
                }
            }
#pragma unroll
            for (int hh = 0; hh < GQ; ++hh) {
                const float4 wv = *(const float4*)&sm.w[wave][hh][tt];
                st.acc[hh].x += wv.x * a[0] + wv.y * a[1] + wv.z * a[2] + wv.w * a[3];
                st.acc[hh].y += wv.x * bb[0] + wv.y * bb[1] + wv.z * bb[2] + wv.w * bb[3];
            }
        }
        wave_sync();
    }
}

// Residual ring: tokens [nq, n) of stream sh, 16 per pass, spread over waves.
template <int GQ>
__device__ void attend_residual(AttnSmem<GQ>& sm, WaveState<GQ>& st, const Layout& L, const kvq_cache& c,
                                long sh, int nq, int n, const float2 (&qs)[GQ], int wave, int lane) {
    const int tl = lane >> 2, part = lane & 3;
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
        *(float2*)&sm.qt[wave][hh][lane >> 4][(2 * lane) & 31] = qs[hh];
    wave_sync();
    const half_t* kr = (const half_t*)c.k_res + sh * L.ring * kD;
    const half_t* vr = (const half_t*)c.v_res + sh * L.ring * kD;
    for (int base = nq + wave * 16; base < n; base += kWaves * 16) {
        const int t = base + tl;
        const bool valid = t < n;
        const int slot = (valid ? t : base) % L.ring;
        float dot[GQ];
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) dot[hh] = 0.0f;
        const uint4* krow = (const uint4*)(kr + (long)slot * kD + part * 32);
#pragma unroll
        for (int i = 0; i < 32; i += 8) {
            const uint4 x = krow[i / 8];
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
            float kv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kv[2 * j] = h2f(xs[j] & 0xffffu);
                kv[2 * j + 1] = h2f(xs[j] >> 16);
            }
#pragma unroll
            for (int hh = 0; hh < GQ; ++hh) {
                const float4 qa = *(const float4*)&sm.qt[wave][hh][part][i];
                const float4 qb = *(const float4*)&sm.qt[wave][hh][part][i + 4];
                dot[hh] += qa.x * kv[0] + qa.y * kv[1] + qa.z * kv[2] + qa.w * kv[3] +
                           qb.x * kv[4] + qb.y * kv[5] + qb.z * kv[6] + qb.w * kv[7];
            }
        }
        float lg[GQ];
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
            float x = dot[hh];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            lg[hh] = x;
        }
        softmax_16<GQ>(st, lg, valid, 1.0f, 0.0f, sm.w[wave], tl, part);
        wave_sync();
        for (int tt = 0; tt < 16; ++tt) {
            const int tok = base + tt;
            if (tok >= n) break;
            const uint32_t x = ((const uint32_t*)(vr + (long)(tok % L.ring) * kD))[lane];
            const float va = h2f(x & 0xffffu), vb = h2f(x >> 16);
#pragma unroll
            for (int hh = 0; hh < GQ; ++hh) {
                const float wv = sm.w[wave][hh][tt];
                st.acc[hh].x += wv * va;
                st.acc[hh].y += wv * vb;
            }
        }
        wave_sync();
    }
}

template <int GQ, int KB, int VB>
__global__ __launch_bounds__(256) void attn_split_kernel(Layout L, kvq_cache c, const half_t* __restrict__ q,
                                                         float qscale, float* __restrict__ ws, int splits,
                                                         int gps) {
    __shared__ AttnSmem<GQ> sm;
    const int sp = blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // counters written by this library satisfy 0 <= nq <= n <= nq + ring; clamp
    // so that no other value can index outside the records or the ring
    const int nq = max(c.n_quant[b], 0);
    const int n = min(max(c.n_tokens[b], nq), nq + L.ring);
    const int Hq = L.H * GQ;

    float2 qs[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        const uint32_t x = ((const uint32_t*)(q + ((long)b * Hq + h * GQ + hh) * kD))[lane];
        qs[hh] = make_float2(h2f(x & 0xffffu) * qscale, h2f(x >> 16) * qscale);
    }
    WaveState<GQ> st;
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        st.m[hh] = -INFINITY;
        st.l[hh] = 0.0f;
        st.pz[hh] = 0.0f;
        st.acc[hh] = make_float2(0.0f, 0.0f);
    }

    if (sp < splits) {
        const int ng = nq / L.G;
        const int g0 = sp * gps;
        const int g1 = min(g0 + gps, ng);
        for (int g = g0 + wave; g < g1; g += kWaves) {
            const uint8_t* rec = record_at(L, c.packed, c.block_table, b, h, g);
            if (rec) attend_group<GQ, KB, VB>(sm, st, L, rec, qs, wave, lane);
        }
    } else {
        attend_residual<GQ>(sm, st, L, c, sh, nq, n, qs, wave, lane);
    }

    // Combine the four waves.
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        const float lt = wave_sum(st.l[hh]);
        const float pzt = wave_sum(st.pz[hh]);
        if (lane == 0) {
            sm.m[wave][hh] = st.m[hh];
            sm.l[wave][hh] = lt;
            sm.pz[wave][hh] = pzt;
        }
    }
    __syncthreads();
    float* accbuf = &sm.qt[0][0][0][0];   // reuse: [wave][GQ][128] fits in qt
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        float M = -INFINITY;
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][hh]);
        const float f = (M == -INFINITY || st.m[hh] == -INFINITY) ? 0.0f : exp2f(st.m[hh] - M);
        *(float2*)&accbuf[((wave * GQ) + hh) * kD + 2 * lane] = make_float2(st.acc[hh].x * f, st.acc[hh].y * f);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < GQ * kD; i += 256) {
        const int hh = i / kD, ch = i % kD;
        float M = -INFINITY;
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][hh]);
        float lsum = 0.0f, pzs = 0.0f, a = 0.0f;
        for (int w = 0; w < kWaves; ++w) {
            const float f = (M == -INFINITY || sm.m[w][hh] == -INFINITY) ? 0.0f : exp2f(sm.m[w][hh] - M);
            lsum += sm.l[w][hh] * f;
            pzs += sm.pz[w][hh] * f;
            a += accbuf[((w * GQ) + hh) * kD + ch];
        }
        float* part = ws + (((long)b * Hq + h * GQ + hh) * (splits + 1) + sp) * kPartStride;
        part[ch] = a + pzs;
        if (ch == 0) {
            part[kD] = M;
            part[kD + 1] = lsum;
        }
    }
}

// out[b][hq][c] = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M); 0 if empty.
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ ws, float* __restrict__ out,
                                                         int nparts) {
    const long row = blockIdx.x;
    const float* p = ws + row * nparts * kPartStride;
    float M = -INFINITY;
    for (int s = 0; s < nparts; ++s) M = fmaxf(M, p[s * kPartStride + kD]);
    float L = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < nparts; ++s) {
            const float m = p[s * kPartStride + kD];
            const float f = m == -INFINITY ? 0.0f : exp2f(m - M);
            L += p[s * kPartStride + kD + 1] * f;
            o += p[s * kPartStride + threadIdx.x] * f;
        }
    }
    out[row * kD + threadIdx.x] = L > 0.0f ? o / L : 0.0f;
}

AttnPlan plan_attention(const Layout& L, int num_q_heads) {
    AttnPlan P;
    const int streams = L.B * L.H;
    const int maxg = L.paged ? L.max_blocks : L.groups;
    // Aim for ~2048 workgroups over the chip, at least 8 groups per wave.
    int splits = (2048 + streams - 1) / streams;
    const int cap = maxg / (kWaves * 8);
    if (splits > cap) splits = cap;
    if (splits < 1) splits = 1;
    if (const char* e = getenv("KVQ_SPLITS")) {
        const int v = atoi(e);
        if (v >= 1) splits = v;
    }
    P.splits = splits;
    P.groups_per_split = maxg > 0 ? (maxg + splits - 1) / splits : 0;
    P.workspace = (size_t)L.B * num_q_heads * (splits + 1) * kPartStride * sizeof(float);
    return P;
}

hipError_t launch_attention(const Layout& L, const AttnPlan& P, const kvq_cache& c, const half_t* q,
                            int num_q_heads, float scale, float* out, void* ws, hipStream_t s) {
    const int gq = num_q_heads / L.H;
    const float qscale = scale * kLog2e;
    dim3 grid(P.splits + 1, L.B * L.H);
#define KVQ_ATT(GQ, KB, VB) hipLaunchKernelGGL((attn_split_kernel<GQ, KB, VB>), grid, dim3(256), 0, s, L, c, q, \
                                               qscale, (float*)ws, P.splits, P.groups_per_split)
#define KVQ_ATT_B(GQ)                                              \
    if (L.kbits == 2 && L.vbits == 2) KVQ_ATT(GQ, 2, 2);            \
    else if (L.kbits == 2 && L.vbits == 4) KVQ_ATT(GQ, 2, 4);       \
    else if (L.kbits == 4 && L.vbits == 2) KVQ_ATT(GQ, 4, 2);       \
    else KVQ_ATT(GQ, 4, 4);
    switch (gq) {
        case 1: KVQ_ATT_B(1); break;
        case 2: KVQ_ATT_B(2); break;
        case 4: KVQ_ATT_B(4); break;
        case 8: KVQ_ATT_B(8); break;
        case 16: KVQ_ATT_B(16); break;
        default: return hipErrorInvalidValue;
    }
#undef KVQ_ATT_B
#undef KVQ_ATT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(L.B * num_q_heads), dim3(kD), 0, s, (const float*)ws, out,
                       P.splits + 1);
    return hipGetLastError();
}

}  // namespace kvq
