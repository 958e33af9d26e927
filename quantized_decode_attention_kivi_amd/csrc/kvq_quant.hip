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

template <int G>
struct QuantSmem {
    float kmn[16][kD], kmx[16][kD];   // per token slice, per channel
    float kz[kD], kinv[kD];
    uint8_t vcode[G][kD];             // value codes before packing
};

// Code of x on the set's grid: uniform (rint), or the normal-quantile
// codebook's nearest level (CB; mid: its midpoints).
template <bool CB, int BITS>
__device__ __forceinline__ uint32_t code_of(float x, float z, float inv, const float (&mid)[15]) {
    if constexpr (CB) {
#pragma clang fp contract(off)
        return cb_code<(1 << BITS) - 1>((x - z) * inv, mid);
    } else {
        return quant_code(x, z, inv, (float)((1 << BITS) - 1));
    }
}

// Quantize G consecutive fp16 rows of keys (ksrc) and values (vsrc) into one
// record.  Called by all 256 threads of a workgroup.  Thread (ts = tid/16,
// cg = tid%16) holds channels 8cg..8cg+7 of tokens ts, ts+16, ...  CB: the
// normal-quantile codebook grid instead of the uniform one.
template <int G, int KB, int VB, bool CB>
__device__ void quantize_group(QuantSmem<G>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                               const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec) {
    constexpr int NT = G / 16;
    constexpr float kq = (float)((1 << KB) - 1);
    constexpr float vq = (float)((1 << VB) - 1);
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;

    float kx[NT][8], vx[NT][8];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        const uint4 a = *(const uint4*)(ksrc + t * kD + 8 * cg);
        const uint4 b = *(const uint4*)(vsrc + t * kD + 8 * cg);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kx[j][2 * e] = h2f(aw[e] & 0xffffu);
            kx[j][2 * e + 1] = h2f(aw[e] >> 16);
            vx[j][2 * e] = h2f(bw[e] & 0xffffu);
            vx[j][2 * e + 1] = h2f(bw[e] >> 16);
        }
    }

    // Key statistics: per channel over the G tokens.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float mn = kx[0][e], mx = kx[0][e];
#pragma unroll
        for (int j = 1; j < NT; ++j) {
            mn = fminf(mn, kx[j][e]);
            mx = fmaxf(mx, kx[j][e]);
        }
        sm.kmn[ts][8 * cg + e] = mn;
        sm.kmx[ts][8 * cg + e] = mx;
    }

    // Value statistics: per token over its 128 channels (16 lanes of a row).
    QParams pv[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        float mn = vx[j][0], mx = vx[j][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) {
            mn = fminf(mn, vx[j][e]);
            mx = fmaxf(mx, vx[j][e]);
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, off));
            mx = fmaxf(mx, __shfl_xor(mx, off));
        }
        pv[j] = make_qparams(mn, mx, VB);
        if (cg == 0) {
            const int t = ts + 16 * j;
            const int pos = vmeta_pos(L, t);
            *(uint16_t*)(rec + pos) = pv[j].s_bits;
            *(uint16_t*)(rec + pos + 2 * L.spt) = pv[j].z_bits;
        }
    }
    __syncthreads();
    if (tid < kD) {
        float mn = sm.kmn[0][tid], mx = sm.kmx[0][tid];
        for (int j = 1; j < 16; ++j) {
            mn = fminf(mn, sm.kmn[j][tid]);
            mx = fmaxf(mx, sm.kmx[j][tid]);
        }
        const QParams p = make_qparams(mn, mx, KB);
        sm.kz[tid] = p.z;
        sm.kinv[tid] = p.inv;
        *(uint16_t*)(rec + L.kmeta_off + 2 * tid) = p.s_bits;
        *(uint16_t*)(rec + L.kmeta_off + 2 * kD + 2 * tid) = p.z_bits;
    }
    __syncthreads();

    // Key codes: the 8 channels of a thread are one INT4 word, half an INT2 word.
    float kzr[8], kir[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        kzr[e] = sm.kz[8 * cg + e];
        kir[e] = sm.kinv[8 * cg + e];
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t q = code_of<CB, KB>(kx[j][e], kzr[e], kir[e], L.kmid);
            w |= q << (KB == 4 ? code_bit(4, e) : code_bit(2, e + 8 * (cg & 1)));
        }
        if (KB == 4) {
            *(uint32_t*)(rec + t * 64 + 4 * cg) = w;
        } else {
            w |= __shfl_xor(w, 1);
            if ((cg & 1) == 0) *(uint32_t*)(rec + t * 32 + 2 * cg) = w;
        }
        // value codes of the same token into LDS, channel order
        uint32_t v0 = 0, v1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v0 |= code_of<CB, VB>(vx[j][e], pv[j].z, pv[j].inv, L.vmid) << (8 * e);
            v1 |= code_of<CB, VB>(vx[j][e + 4], pv[j].z, pv[j].inv, L.vmid) << (8 * e);
        }
        *(uint2*)&sm.vcode[t][8 * cg] = make_uint2(v0, v1);
    }
    __syncthreads();

    // Value code words, lane-major in decode-operand order.
    constexpr int SPT = G == 16 ? 4 : 8;
    constexpr int WPL = SPT * VB / 4;        // words per lane
    constexpr int CPW = 32 / VB;             // codes per word
    for (int D = tid; D < 64 * WPL; D += 256) {
        const int lane = D / WPL, wi = D % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < CPW; ++e) {
            const int q = wi * CPW + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = (slot >> 2) * 16 + 4 * g + (slot & 3);
            w |= (uint32_t)sm.vcode[t][16 * ct + n] << code_bit(VB, e);
        }
        *(uint32_t*)(rec + L.vcode_off + lane * SPT * VB + 4 * wi) = w;
    }
    __syncthreads();  // LDS may be reused by the caller
}

// The same for the 8-bit formats ("KV cache compression: ...", section 3.1):
// every key and value token on its own.  F = kFmtInt8: the min/max grid with
// 8 bits over the token's 128 channels (the 16 threads of a row reduce it);
// F = kFmtFp8: E4M3 codes under the kv head's static scales (inverses kinv,
// vinv).  Key bytes go straight to the record in channel order; value bytes
// through LDS into the lane-major operand order.
template <int G, int F>
__device__ void quantize_group8(QuantSmem<G>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                                const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec, float kinv,
                                float vinv) {
    constexpr int NT = G / 16;
    constexpr int SPT = G == 16 ? 4 : 8;
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        const uint4 a = *(const uint4*)(ksrc + t * kD + 8 * cg);
        const uint4 b = *(const uint4*)(vsrc + t * kD + 8 * cg);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
        float kx[8], vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kx[2 * e] = h2f(aw[e] & 0xffffu);
            kx[2 * e + 1] = h2f(aw[e] >> 16);
            vx[2 * e] = h2f(bw[e] & 0xffffu);
            vx[2 * e + 1] = h2f(bw[e] >> 16);
        }
        uint32_t kw[2], vw[2];
        if (F == kFmtInt8) {
            float kmn = kx[0], kmx = kx[0], vmn = vx[0], vmx = vx[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) {
                kmn = fminf(kmn, kx[e]);
                kmx = fmaxf(kmx, kx[e]);
                vmn = fminf(vmn, vx[e]);
                vmx = fmaxf(vmx, vx[e]);
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                kmn = fminf(kmn, __shfl_xor(kmn, off));
                kmx = fmaxf(kmx, __shfl_xor(kmx, off));
                vmn = fminf(vmn, __shfl_xor(vmn, off));
                vmx = fmaxf(vmx, __shfl_xor(vmx, off));
            }
            const QParams pk = make_qparams(kmn, kmx, 8);
            const QParams pv = make_qparams(vmn, vmx, 8);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kw[h] = vw[h] = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kw[h] |= quant_code(kx[4 * h + e], pk.z, pk.inv, 255.0f) << (8 * e);
                    vw[h] |= quant_code(vx[4 * h + e], pv.z, pv.inv, 255.0f) << (8 * e);
                }
            }
            if (cg == 0) {
                const int kp = tmeta_pos(L, L.kmeta_off, t), vp = tmeta_pos(L, L.vmeta_off, t);
                *(uint16_t*)(rec + kp) = pk.s_bits;
                *(uint16_t*)(rec + kp + 2 * SPT) = pk.z_bits;
                *(uint16_t*)(rec + vp) = pv.s_bits;
                *(uint16_t*)(rec + vp + 2 * SPT) = pv.z_bits;
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kw[h] = fp8_code2(kx[4 * h], kx[4 * h + 1], kinv) | fp8_code2(kx[4 * h + 2], kx[4 * h + 3], kinv) << 16;
                vw[h] = fp8_code2(vx[4 * h], vx[4 * h + 1], vinv) | fp8_code2(vx[4 * h + 2], vx[4 * h + 3], vinv) << 16;
            }
        }
        *(uint2*)(rec + t * kD + 8 * cg) = make_uint2(kw[0], kw[1]);
        *(uint2*)&sm.vcode[t][8 * cg] = make_uint2(vw[0], vw[1]);
    }
    __syncthreads();

    // Value bytes, lane-major: lane l = 16g + n holds, at byte ct*SPT + slot
    // of its SPT*8 bytes, the code of channel 16ct + n for the slot's token.
    constexpr int WPL = SPT * 2;   // words per lane
    for (int D = tid; D < 64 * WPL; D += 256) {
        const int lane = D / WPL, wi = D % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = wi * 4 + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = (slot >> 2) * 16 + 4 * g + (slot & 3);
            w |= (uint32_t)sm.vcode[t][16 * ct + n] << (8 * e);
        }
        *(uint32_t*)(rec + L.vcode_off + lane * SPT * 8 + 4 * wi) = w;
    }
    __syncthreads();  // LDS may be reused by the caller
}

// Quantizes one group of the format F (kFmtKivi: key bits KB, value bits VB).
template <int G, int KB, int VB, int F>
__device__ __forceinline__ void quantize_any(QuantSmem<G>& sm, const Layout& L, const kvq_cache& c, int h,
                                             const half_t* ksrc, const half_t* vsrc, uint8_t* rec) {
    if (F == kFmtKivi) {
        if (L.grid == KVQ_GRID_NORMAL_QUANTILE) quantize_group<G, KB, VB, true>(sm, L, ksrc, vsrc, rec);
        else quantize_group<G, KB, VB, false>(sm, L, ksrc, vsrc, rec);
    } else {
        const float kinv = F == kFmtFp8 ? fp8_inv_scale(c.k_scale[h]) : 0.0f;
        const float vinv = F == kFmtFp8 ? fp8_inv_scale(c.v_scale[h]) : 0.0f;
        quantize_group8<G, F>(sm, L, ksrc, vsrc, rec, kinv, vinv);
    }
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

template <int G, int KB, int VB, int F>
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
    quantize_any<G, KB, VB, F>(sm, L, c, h, k + base, v + base, rec);
}

// Residual copy and counters: grid (B*H), 256 threads.
__global__ __launch_bounds__(256) void prefill_tail_kernel(Layout L, kvq_cache c, const half_t* k,
                                                           const half_t* v, int max_len,
                                                           const int32_t* seq_lens) {
    const int sh = blockIdx.x;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = num_quantized(n, L.G, L.R);
    const uint4* k16 = (const uint4*)(k + (long)sh * max_len * kD);
    const uint4* v16 = (const uint4*)(v + (long)sh * max_len * kD);
    uint4* kr = (uint4*)c.k_res + (long)sh * L.ring * (kD / 8);
    uint4* vr = (uint4*)c.v_res + (long)sh * L.ring * (kD / 8);
    const int cp = threadIdx.x & 15;
    for (int i = nq + (threadIdx.x >> 4); i < n; i += 16) {
        const int slot = i % L.ring;
        kr[slot * (kD / 8) + cp] = k16[(long)i * (kD / 8) + cp];
        vr[slot * (kD / 8) + cp] = v16[(long)i * (kD / 8) + cp];
    }
    if (h == 0 && threadIdx.x == 0) {
        c.n_tokens[b] = n;
        c.n_quant[b] = nq;
    }
}

// ---------------------------------------------------------------------------
// Append one token per (sequence, head) and flush a full group: grid (B).
// ---------------------------------------------------------------------------

template <int G, int KB, int VB, int F>
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
                quantize_any<G, KB, VB, F>(sm, L, c, h, (const half_t*)c.k_res + row,
                                           (const half_t*)c.v_res + row, rec);
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
    const int tg = t % L.G;
    for (int i = 0; i < 8; ++i) {
        const int ch = c0 + i;
        float kv = 0.0f, vv = 0.0f;
        if (t < nq) {
            if (rec && L.fmt == kFmtFp8) {
#pragma clang fp contract(off)
                kv = fp8_value(kcode_at(L, rec, tg, ch)) * c.k_scale[h];
                vv = fp8_value(vcode_at(L, rec, tg, ch)) * c.v_scale[h];
            } else if (rec) {
                const bool tok = L.fmt == kFmtInt8;   // per-token key scale and zero
                const bool cb = L.grid == KVQ_GRID_NORMAL_QUANTILE;
                const uint32_t kcd = kcode_at(L, rec, tg, ch), vcd = vcode_at(L, rec, tg, ch);
                kv = fmaf(cb ? cb_level(L.klut, kcd, L.kbits) : (float)kcd,
                          h2f(tok ? ktok_scale_bits(L, rec, tg) : kscale_bits(L, rec, ch)),
                          h2f(tok ? ktok_zero_bits(L, rec, tg) : kzero_bits(L, rec, ch)));
                vv = fmaf(cb ? cb_level(L.vlut, vcd, L.vbits) : (float)vcd, h2f(vscale_bits(L, rec, tg)),
                          h2f(vzero_bits(L, rec, tg)));
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
        kc[e + i] = rec ? (uint8_t)kcode_at(L, rec, tg, c0 + i) : 0;
        vc[e + i] = rec ? (uint8_t)vcode_at(L, rec, tg, c0 + i) : 0;
    }
    if (L.fmt == kFmtFp8) return;   // no scale/zero tables
    if (L.fmt == kFmtInt8) {
        if (c0 == 0) {
            ks[(long)sh * out_tokens + t] = rec ? ktok_scale_bits(L, rec, tg) : 0;
            kz[(long)sh * out_tokens + t] = rec ? ktok_zero_bits(L, rec, tg) : 0;
        }
    } else if (tg == 0) {  // key metadata row of this group
        const long gi = ((long)sh * (out_tokens / L.G) + t / L.G) * kD + c0;
        for (int i = 0; i < 8; ++i) {
            ks[gi + i] = rec ? kscale_bits(L, rec, c0 + i) : 0;
            kz[gi + i] = rec ? kzero_bits(L, rec, c0 + i) : 0;
        }
    }
    if (c0 == 0) {
        vs[(long)sh * out_tokens + t] = rec ? vscale_bits(L, rec, tg) : 0;
        vz[(long)sh * out_tokens + t] = rec ? vzero_bits(L, rec, tg) : 0;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

#define KVQ_DISPATCH(L_, F)                                                    \
    do {                                                                       \
        switch (layout_key(L_)) {                                              \
            case 1622: F(16, 2, 2, kFmtKivi); break;                           \
            case 1624: F(16, 2, 4, kFmtKivi); break;                           \
            case 1642: F(16, 4, 2, kFmtKivi); break;                           \
            case 1644: F(16, 4, 4, kFmtKivi); break;                           \
            case 3222: F(32, 2, 2, kFmtKivi); break;                           \
            case 3224: F(32, 2, 4, kFmtKivi); break;                           \
            case 3242: F(32, 4, 2, kFmtKivi); break;                           \
            case 3244: F(32, 4, 4, kFmtKivi); break;                           \
            case 11688: F(16, 8, 8, kFmtInt8); break;                          \
            case 13288: F(32, 8, 8, kFmtInt8); break;                          \
            case 21688: F(16, 8, 8, kFmtFp8); break;                           \
            case 23288: F(32, 8, 8, kFmtFp8); break;                           \
            default: return hipErrorInvalidValue;                              \
        }                                                                      \
    } while (0)

hipError_t launch_prefill(const Layout& L, const kvq_cache& c, const half_t* k, const half_t* v,
                          int max_len, const int32_t* seq_lens, hipStream_t s) {
    const int ngroups = (max_len + L.G - 1) / L.G;
    if (ngroups > 0) {
        dim3 grid(ngroups, L.B * L.H);
#define KVQ_PF(GG, KB, VB, FF)                                                                               \
    hipLaunchKernelGGL((prefill_groups_kernel<GG, KB, VB, FF>), grid, dim3(256), 0, s, L, c, k, v, max_len, \
                       seq_lens)
        KVQ_DISPATCH(L, KVQ_PF);
#undef KVQ_PF
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(prefill_tail_kernel, dim3(L.B * L.H), dim3(256), 0, s, L, c, k, v, max_len, seq_lens);
    return hipGetLastError();
}

hipError_t launch_append(const Layout& L, const kvq_cache& c, const half_t* k, const half_t* v,
                         hipStream_t s) {
#define KVQ_AP(GG, KB, VB, FF) \
    hipLaunchKernelGGL((append_kernel<GG, KB, VB, FF>), dim3(L.B), dim3(256), 0, s, L, c, k, v)
    KVQ_DISPATCH(L, KVQ_AP);
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
