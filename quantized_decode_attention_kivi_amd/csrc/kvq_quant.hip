// kvq_quant.hip -- quantize-prefill, append/flush, dequantize and code export
// kernels of libkvq (gfx950).
//
// Method ("KV cache compression: quantization, eviction and sparse attention",
// section 3.2; "KV cache compression" (jaedaily), formula paragraph; "KV Cache
// compression lab", experiment 01): keys are quantized per channel over each
// group of G tokens, values per token over their 128 channels, each set with
// its own min/max scale and zero; the newest R tokens stay fp16 and a group
// is quantized once it is full and outside them.
#include "kvq_device.h"

namespace kvq {

// Shared memory of one group quantization (G tokens x 128 channels).
template <int G>
struct QuantSmem {
    uint32_t ktile[G][kD / 2];     // fp16 pairs, token-major
    uint32_t vtile[G][kD / 2];
    float4 red[4][kD / 2];         // per token slice: (min0, min1, max0, max1)
    float kz[kD], kinv[kD];
    uint8_t vcode[kD][G];          // value codes, channel-major
};

// Quantize G consecutive fp16 rows of keys (ksrc) and values (vsrc) into one
// record.  Called by all 256 threads of a workgroup.
template <int G>
__device__ void quantize_group(QuantSmem<G>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                               const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec) {
    const int tid = threadIdx.x;
    const int cp = tid & 63;   // channel pair
    const int ts = tid >> 6;   // token slice
    const float kq = (float)((1 << L.kbits) - 1);
    const float vq = (float)((1 << L.vbits) - 1);

    // Phase A: stage both tiles in LDS; per-channel key min/max over the group.
    float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
    const uint32_t* k32 = (const uint32_t*)ksrc;
    const uint32_t* v32 = (const uint32_t*)vsrc;
    for (int t = ts; t < G; t += 4) {
        const uint32_t kx = k32[t * (kD / 2) + cp];
        const uint32_t vx = v32[t * (kD / 2) + cp];
        sm.ktile[t][cp] = kx;
        sm.vtile[t][cp] = vx;
        const float a = h2f(kx & 0xffffu), b = h2f(kx >> 16);
        mn0 = fminf(mn0, a); mx0 = fmaxf(mx0, a);
        mn1 = fminf(mn1, b); mx1 = fmaxf(mx1, b);
    }
    sm.red[ts][cp] = make_float4(mn0, mn1, mx0, mx1);
    __syncthreads();
    if (ts == 0) {
        for (int j = 1; j < 4; ++j) {
            const float4 r = sm.red[j][cp];
            mn0 = fminf(mn0, r.x); mn1 = fminf(mn1, r.y);
            mx0 = fmaxf(mx0, r.z); mx1 = fmaxf(mx1, r.w);
        }
        const QParams p0 = make_qparams(mn0, mx0, L.kbits);
        const QParams p1 = make_qparams(mn1, mx1, L.kbits);
        sm.kz[2 * cp] = p0.z; sm.kinv[2 * cp] = p0.inv;
        sm.kz[2 * cp + 1] = p1.z; sm.kinv[2 * cp + 1] = p1.inv;
        *(uint2*)(rec + L.kmeta_off + 8 * cp) = make_uint2(p0.sz_bits, p1.sz_bits);
    }
    __syncthreads();

    // Phase B: key codes, one unit = (token t, 16 channels), token-major rows.
    // Phase C: value min/max per token (8 lanes per token), value codes.
    for (int u = tid; u < G * 8; u += 256) {
        const int t = u >> 3, ch = u & 7;
        // keys
        uint32_t lo = 0, hi = 0;
        for (int i = 0; i < 8; ++i) {
            const uint32_t x = sm.ktile[t][ch * 8 + i];
            const int c = ch * 16 + 2 * i;
            const uint32_t q0 = quant_code(h2f(x & 0xffffu), sm.kz[c], sm.kinv[c], kq);
            const uint32_t q1 = quant_code(h2f(x >> 16), sm.kz[c + 1], sm.kinv[c + 1], kq);
            if (L.kbits == 2) {
                lo |= (q0 | (q1 << 2)) << (4 * i);
            } else {
                const uint32_t pair = q0 | (q1 << 4);
                if (i < 4) lo |= pair << (8 * i); else hi |= pair << (8 * (i - 4));
            }
        }
        if (L.kbits == 2)
            *(uint32_t*)(rec + t * 32 + ch * 4) = lo;
        else
            *(uint2*)(rec + t * 64 + ch * 8) = make_uint2(lo, hi);

        // values: this token's min/max over its 128 channels
        float vals[16];
        float vmn = INFINITY, vmx = -INFINITY;
        for (int i = 0; i < 8; ++i) {
            const uint32_t x = sm.vtile[t][ch * 8 + i];
            vals[2 * i] = h2f(x & 0xffffu);
            vals[2 * i + 1] = h2f(x >> 16);
            vmn = fminf(vmn, fminf(vals[2 * i], vals[2 * i + 1]));
            vmx = fmaxf(vmx, fmaxf(vals[2 * i], vals[2 * i + 1]));
        }
        for (int off = 1; off < 8; off <<= 1) {
            vmn = fminf(vmn, __shfl_xor(vmn, off));
            vmx = fmaxf(vmx, __shfl_xor(vmx, off));
        }
        const QParams pv = make_qparams(vmn, vmx, L.vbits);
        for (int i = 0; i < 16; ++i)
            sm.vcode[ch * 16 + i][t] = (uint8_t)quant_code(vals[i], pv.z, pv.inv, vq);
        if (ch == 0) *(uint32_t*)(rec + L.vmeta_off + 4 * t) = pv.sz_bits;
    }
    __syncthreads();

    // Phase D: value code units (16 tokens of one channel).
    for (int u = tid; u < (G / 16) * kD; u += 256) {
        const int j = u >> 7, c = u & 127;
        const uint4 w = *(const uint4*)&sm.vcode[c][16 * j];
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
        if (L.vbits == 2) {
            uint32_t packed = 0;
            for (int i = 0; i < 16; ++i) packed |= ((wv[i >> 2] >> (8 * (i & 3))) & 3u) << (2 * i);
            *(uint32_t*)(rec + L.vcode_off + u * 4) = packed;
        } else {
            uint32_t lo = 0, hi = 0;
            for (int i = 0; i < 8; ++i) lo |= ((wv[i >> 2] >> (8 * (i & 3))) & 15u) << (4 * i);
            for (int i = 8; i < 16; ++i) hi |= ((wv[i >> 2] >> (8 * (i & 3))) & 15u) << (4 * (i - 8));
            *(uint2*)(rec + L.vcode_off + u * 8) = make_uint2(lo, hi);
        }
    }
    __syncthreads();  // LDS may be reused by the caller
}

// ---------------------------------------------------------------------------
// Prefill: grid (ceil(max_len / G), B*H); one workgroup per (group, stream).
// ---------------------------------------------------------------------------

__device__ __forceinline__ int clamped_len(const Layout& L, const int32_t* seq_lens, int b, int max_len) {
    int n = seq_lens[b];
    n = n < 0 ? 0 : n;
    n = n > max_len ? max_len : n;
    n = n > L.capacity ? L.capacity : n;
    return n;
}

template <int G>
__global__ __launch_bounds__(256) void prefill_groups_kernel(Layout L, kvq_cache c, const half_t* k,
                                                             const half_t* v, int max_len,
                                                             const int32_t* seq_lens) {
    __shared__ QuantSmem<G> sm;
    const int g = blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = num_quantized(n, G, L.R);
    if (g * G >= nq) return;
    uint8_t* rec = record_at(L, c.packed, c.block_table, b, h, g);
    if (!rec) return;
    const long base = ((long)sh * max_len + (long)g * G) * kD;
    quantize_group<G>(sm, L, k + base, v + base, rec);
}

// Residual copy and counters: grid (B*H), 256 threads.
__global__ __launch_bounds__(256) void prefill_tail_kernel(Layout L, kvq_cache c, const half_t* k,
                                                           const half_t* v, int max_len,
                                                           const int32_t* seq_lens) {
    const int sh = blockIdx.x;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = num_quantized(n, L.G, L.R);
    const uint32_t* k32 = (const uint32_t*)(k + (long)sh * max_len * kD);
    const uint32_t* v32 = (const uint32_t*)(v + (long)sh * max_len * kD);
    uint32_t* kr = (uint32_t*)c.k_res + (long)sh * L.ring * (kD / 2);
    uint32_t* vr = (uint32_t*)c.v_res + (long)sh * L.ring * (kD / 2);
    for (int i = nq + (threadIdx.x >> 6); i < n; i += 4) {
        const int slot = i % L.ring;
        const int cp = threadIdx.x & 63;
        kr[slot * (kD / 2) + cp] = k32[(long)i * (kD / 2) + cp];
        vr[slot * (kD / 2) + cp] = v32[(long)i * (kD / 2) + cp];
    }
    if (h == 0 && threadIdx.x == 0) {
        c.n_tokens[b] = n;
        c.n_quant[b] = nq;
    }
}

// ---------------------------------------------------------------------------
// Append one token per (sequence, head) and flush a full group: grid (B).
// ---------------------------------------------------------------------------

template <int G>
__global__ __launch_bounds__(256) void append_kernel(Layout L, kvq_cache c, const half_t* knew,
                                                     const half_t* vnew) {
    __shared__ QuantSmem<G> sm;
    const int b = blockIdx.x;
    const int n = c.n_tokens[b];
    const int nq = c.n_quant[b];
    // counters written by this library satisfy 0 <= nq <= n, nq % G == 0;
    // anything else is treated as a full cache (nothing is written)
    const bool sane = nq >= 0 && n >= nq && (nq % G) == 0;
    const bool room = sane && (n - nq) < L.ring && n < L.capacity;
    const bool flush = room && (n + 1 - nq == L.R + G);
    bool flushed = flush;
    for (int h = 0; h < L.H; ++h) {
        const long sh = (long)b * L.H + h;
        if (room && threadIdx.x < 64) {
            const int slot = n % L.ring;
            ((uint32_t*)c.k_res)[(sh * L.ring + slot) * (kD / 2) + threadIdx.x] =
                ((const uint32_t*)knew)[sh * (kD / 2) + threadIdx.x];
            ((uint32_t*)c.v_res)[(sh * L.ring + slot) * (kD / 2) + threadIdx.x] =
                ((const uint32_t*)vnew)[sh * (kD / 2) + threadIdx.x];
        }
        __syncthreads();
        if (flush) {
            uint8_t* rec = record_at(L, c.packed, c.block_table, b, h, nq / G);
            if (rec) {
                const long row = (sh * L.ring + (nq % L.ring)) * kD;
                quantize_group<G>(sm, L, (const half_t*)c.k_res + row, (const half_t*)c.v_res + row, rec);
            } else {
                flushed = false;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0 && room) {
        c.n_tokens[b] = n + 1;
        c.n_quant[b] = nq + (flushed ? G : 0);
    }
}

// ---------------------------------------------------------------------------
// Dequantize / export: grid (out_tokens / 16, B*H), 256 threads, 16 tokens
// per block; thread -> token t = tid/16, channels (tid%16)*8 .. +8.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t kcode_at(const uint8_t* rec, int kbits, int t, int c) {
    const int bit = (t * kD + c) * kbits;
    return (rec[bit >> 3] >> (bit & 7)) & ((1u << kbits) - 1);
}
__device__ __forceinline__ uint32_t vcode_at(const uint8_t* rec, const Layout& L, int t, int c) {
    const int unit = (t >> 4) * kD + c;
    const int bit = unit * 16 * L.vbits + (t & 15) * L.vbits;
    return (rec[L.vcode_off + (bit >> 3)] >> (bit & 7)) & ((1u << L.vbits) - 1);
}

__global__ __launch_bounds__(256) void dequantize_kernel(Layout L, kvq_cache c, float* ko, float* vo,
                                                         int out_tokens) {
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c0 = (threadIdx.x & 15) * 8;
    if (t >= out_tokens) return;
    const int nq = max(c.n_quant[b], 0);
    const int n = min(max(c.n_tokens[b], nq), nq + L.ring);
    float* kd = ko + ((long)sh * out_tokens + t) * kD + c0;
    float* vd = vo + ((long)sh * out_tokens + t) * kD + c0;
    const uint8_t* rec = t < nq ? record_at(L, c.packed, c.block_table, b, h, t / L.G) : nullptr;
    for (int i = 0; i < 8; ++i) {
        const int ch = c0 + i;
        float kv = 0.0f, vv = 0.0f;
        if (t < nq) {
            if (rec) {
                const int tg = t % L.G;
                const uint32_t km = *(const uint32_t*)(rec + L.kmeta_off + 4 * ch);
                const uint32_t vm = *(const uint32_t*)(rec + L.vmeta_off + 4 * tg);
                kv = fmaf((float)kcode_at(rec, L.kbits, tg, ch), h2f(km & 0xffffu), h2f(km >> 16));
                vv = fmaf((float)vcode_at(rec, L, tg, ch), h2f(vm & 0xffffu), h2f(vm >> 16));
            }
        } else if (t < n) {
            const long row = ((long)sh * L.ring + (t % L.ring)) * kD + ch;
            kv = (float)((const half_t*)c.k_res)[row];
            vv = (float)((const half_t*)c.v_res)[row];
        }
        kd[i] = kv;
        vd[i] = vv;
    }
}

__global__ __launch_bounds__(256) void export_kernel(Layout L, kvq_cache c, uint8_t* kc, uint8_t* vc,
                                                     uint16_t* ks, uint16_t* kz, uint16_t* vs,
                                                     uint16_t* vz, int out_tokens) {
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c0 = (threadIdx.x & 15) * 8;
    if (t >= out_tokens) return;
    const int nq = max(c.n_quant[b], 0);
    const uint8_t* rec = t < nq ? record_at(L, c.packed, c.block_table, b, h, t / L.G) : nullptr;
    const int tg = t % L.G;
    const long e = ((long)sh * out_tokens + t) * kD + c0;
    for (int i = 0; i < 8; ++i) {
        kc[e + i] = rec ? (uint8_t)kcode_at(rec, L.kbits, tg, c0 + i) : 0;
        vc[e + i] = rec ? (uint8_t)vcode_at(rec, L, tg, c0 + i) : 0;
    }
    if (tg == 0) {  // key metadata row of this group
        const long gi = ((long)sh * (out_tokens / L.G) + t / L.G) * kD + c0;
        for (int i = 0; i < 8; ++i) {
            const uint32_t km = rec ? *(const uint32_t*)(rec + L.kmeta_off + 4 * (c0 + i)) : 0u;
            ks[gi + i] = (uint16_t)(km & 0xffffu);
            kz[gi + i] = (uint16_t)(km >> 16);
        }
    }
    if (c0 == 0) {
        const uint32_t vm = rec ? *(const uint32_t*)(rec + L.vmeta_off + 4 * tg) : 0u;
        vs[(long)sh * out_tokens + t] = (uint16_t)(vm & 0xffffu);
        vz[(long)sh * out_tokens + t] = (uint16_t)(vm >> 16);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

#define KVQ_DISPATCH_G(G_, F)          \
    switch (G_) {                      \
        case 16: F(16); break;         \
        case 32: F(32); break;         \
        case 64: F(64); break;         \
        default: return hipErrorInvalidValue; \
    }

hipError_t launch_prefill(const Layout& L, const kvq_cache& c, const half_t* k, const half_t* v,
                          int max_len, const int32_t* seq_lens, hipStream_t s) {
    const int ngroups = (max_len + L.G - 1) / L.G;
    if (ngroups > 0) {
        dim3 grid(ngroups, L.B * L.H);
#define KVQ_PF(GG) hipLaunchKernelGGL(prefill_groups_kernel<GG>, grid, dim3(256), 0, s, L, c, k, v, max_len, seq_lens)
        KVQ_DISPATCH_G(L.G, KVQ_PF);
#undef KVQ_PF
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(prefill_tail_kernel, dim3(L.B * L.H), dim3(256), 0, s, L, c, k, v, max_len, seq_lens);
    return hipGetLastError();
}

hipError_t launch_append(const Layout& L, const kvq_cache& c, const half_t* k, const half_t* v,
                         hipStream_t s) {
#define KVQ_AP(GG) hipLaunchKernelGGL(append_kernel<GG>, dim3(L.B), dim3(256), 0, s, L, c, k, v)
    KVQ_DISPATCH_G(L.G, KVQ_AP);
#undef KVQ_AP
    return hipGetLastError();
}

hipError_t launch_dequantize(const Layout& L, const kvq_cache& c, float* ko, float* vo, int out_tokens,
                             hipStream_t s) {
    if (out_tokens <= 0) return hipSuccess;
    dim3 grid((out_tokens + 15) / 16, L.B * L.H);
    hipLaunchKernelGGL(dequantize_kernel, grid, dim3(256), 0, s, L, c, ko, vo, out_tokens);
    return hipGetLastError();
}

hipError_t launch_export(const Layout& L, const kvq_cache& c, uint8_t* kc, uint8_t* vc, uint16_t* ks,
                         uint16_t* kz, uint16_t* vs, uint16_t* vz, int out_tokens, hipStream_t s) {
    if (out_tokens <= 0) return hipSuccess;
    dim3 grid((out_tokens + 15) / 16, L.B * L.H);
    hipLaunchKernelGGL(export_kernel, grid, dim3(256), 0, s, L, c, kc, vc, ks, kz, vs, vz, out_tokens);
    return hipGetLastError();
}

}  // namespace kvq
