// kvq_device.h -- device helpers of libkvq: record addressing, the fp32
// quantizer step, code positions inside a record.  gfx950 only.
#pragma once

#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half_t;

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f2h_bits(float x) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Record of key group g of stream (b, h); nullptr if it lies outside the
// cache (contiguous: g >= groups; paged: g >= max_blocks or a block id
// outside [0, num_blocks)).  PG: the cache is paged (L.paged).
template <bool PG>
__device__ __forceinline__ uint8_t* record_at_t(const Layout& L, void* packed, const int32_t* bt, int b, int h,
                                                int g) {
    long idx;
    if (PG) {
        if (g < 0 || g >= L.max_blocks) return nullptr;
        // read through the constant address space: a scalar load when the
        // index is wave uniform (the table does not change during a kernel)
        const int id = *(const __attribute__((address_space(4))) int32_t*)(bt + (long)b * L.max_blocks + g);
        if (id < 0 || id >= L.num_blocks) return nullptr;
        idx = (long)id * L.H + h;
    } else {
        if (g < 0 || g >= L.groups) return nullptr;
        idx = ((long)b * L.H + h) * L.groups + g;
    }
    return (uint8_t*)packed + idx * (long)L.record;
}
__device__ __forceinline__ uint8_t* record_at(const Layout& L, void* packed, const int32_t* bt, int b, int h,
                                              int g) {
    return L.paged ? record_at_t<true>(L, packed, bt, b, h, g) : record_at_t<false>(L, packed, bt, b, h, g);
}

// Grid parameters of one quantized set ("KV Cache compression lab",
// experiment 01: 2^b levels from min to max, spacing (max-min)/(2^b-1)).
// Computed in fp32, stored in fp16; the codes use the stored values.
struct QParams {
    float z, inv;
    uint16_t s_bits, z_bits;
};

// RN(x / Q) for Q = 2^bits - 1 (3, 15 or 255) and 0 <= x <= 131008 (the
// difference of two finite fp16 values): the product with RN(1/Q), then one
// fma correction by the exact remainder.  Equal to IEEE division for every
// fp32 x in that range (checked exhaustively on the host), at a third of its
// instructions.
__device__ __forceinline__ float div_by_levels(float x, int bits) {
#pragma clang fp contract(off)
    const float d = (float)((1 << bits) - 1);
    const float r = bits == 2 ? (float)(1.0 / 3.0) : bits == 4 ? (float)(1.0 / 15.0) : (float)(1.0 / 255.0);
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, d, x);
    return __builtin_fmaf(e, r, q0);
}

// RN(1 / s) for s > 0 an fp16 value: the hardware reciprocal (within 1 ulp)
// and one Newton step.  Equal to IEEE division for every positive fp16 s and
// every starting value within 1 ulp (checked exhaustively on the host).
__device__ __forceinline__ float recip_fp16(float s) {
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

__device__ __forceinline__ QParams make_qparams(float mn, float mx, int bits) {
#pragma clang fp contract(off)
    mn = mn + 0.0f;  // a -0 extreme becomes +0
    mx = mx + 0.0f;
    float s32 = div_by_levels(mx - mn, bits);
    // The quotient is rounded to fp32 and then to fp16.  Without this
    // register fence the compiler fuses the last fma with the conversion
    // (v_fma_mixlo_f16), which rounds once, straight to fp16, and differs at
    // quotients on an fp16 rounding midpoint.
    asm volatile("" : "+v"(s32));
    const uint16_t sb = f2h_bits(s32);
    const uint16_t zb = f2h_bits(mn);
    const float s = h2f(sb);
    QParams p;
    p.z = h2f(zb);
    p.inv = s > 0.0f ? recip_fp16(s) : 0.0f;
    p.s_bits = sb;
    p.z_bits = zb;
    return p;
}

// code = clamp(rint((x - z) * inv), 0, 2^b - 1), ties to even.
__device__ __forceinline__ uint32_t quant_code(float x, float z, float inv, float qmax) {
#pragma clang fp contract(off)
    const float t = (x - z) * inv;
    const float r = __builtin_rintf(t);
    return (uint32_t)fminf(fmaxf(r, 0.0f), qmax);
}

// FP8 E4M3 (OCP): value of a code, exact (every E4M3 value is an fp16 value).
__device__ __forceinline__ float fp8_value(uint32_t code) {
    return (float)__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, false)[0];
}

// FP8 E4M3 code of x * inv: the product clamped to +-448 (the largest finite
// value), then rounded to the nearest code, ties to even, by the hardware
// conversion.  inv = 1/scale, or 0 for a scale that is not positive.
__device__ __forceinline__ float fp8_inv_scale(float scale) { return scale > 0.0f ? 1.0f / scale : 0.0f; }
__device__ __forceinline__ uint32_t fp8_code2(float x0, float x1, float inv) {
#pragma clang fp contract(off)
    const float a = __builtin_amdgcn_fmed3f(x0 * inv, -448.0f, 448.0f);
    const float b = __builtin_amdgcn_fmed3f(x1 * inv, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;   // bytes: a, b
}

// Normal-quantile codebook: code of t = (x - z) * inv (grid steps) as the
// nearest level, counting the midpoints below t; a tie at the midpoint of
// levels k and k + 1 goes to the even one of the two (k even: '>', odd: '>=').
template <int Q>
__device__ __forceinline__ uint32_t cb_code(float t, const float (&mid)[15]) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < Q; ++k) c += (k & 1) ? (t >= mid[k] ? 1u : 0u) : (t > mid[k] ? 1u : 0u);
    return c;
}

// Level of code c (grid steps) from a codebook byte table (byte c = F * L_c).
__device__ __forceinline__ float cb_level(const uint32_t (&lut)[4], uint32_t c, int bits) {
    const uint32_t w = c < 4 ? lut[0] : c < 8 ? lut[1] : c < 12 ? lut[2] : lut[3];
    const float invF = bits == 2 ? 1.0f / 64.0f : 1.0f / 16.0f;
    return (float)((w >> (8 * (c & 3))) & 0xffu) * invF;
}

// ---------------------------------------------------------------------------
// Positions inside a record (see kvq_internal.h for the layout).
// ---------------------------------------------------------------------------

// Byte offset and bit of key code (token t, channel c).
__device__ __forceinline__ void kcode_pos(const Layout& L, int t, int c, int* byte, int* bit) {
    if (L.kbits == 8) {   // (channels 4j .. 4j+3 of a token are one word)
        *byte = k8_byte(t, c & ~3);
        *bit = 8 * (c & 3);
        return;
    }
    const int cpw = 32 / L.kbits;           // codes per word
    const int q = c & 31;
    *byte = t * 16 * L.kbits + 4 * L.kbits * (c >> 5) + 4 * (q / cpw);
    *bit = code_bit(L.kbits, q % cpw);
}

// Byte offset (from the record start) and bit of value code (token t, channel c).
__device__ __forceinline__ void vcode_pos(const Layout& L, int t, int c, int* byte, int* bit) {
    int g, slot;
    vslot(t, &g, &slot);
    const int cpw = 32 / L.vbits;
    const int lane = 16 * g + (c & 15);
    const int q = (c >> 4) * L.spt + slot;
    *byte = L.vcode_off + vlane_byte(L.spt * L.vbits, lane, 4 * (q / cpw));
    *bit = code_bit(L.vbits, q % cpw);
}

// Byte offset of the fp16 scale of token t in a per-token table starting at
// `off` (the value table; the INT8 key table); its zero follows 2*spt bytes on.
__device__ __forceinline__ int tmeta_pos(const Layout& L, int off, int t) {
    int g, slot;
    vslot(t, &g, &slot);
    return off + g * 4 * L.spt + 2 * slot;
}
__device__ __forceinline__ int vmeta_pos(const Layout& L, int t) { return tmeta_pos(L, L.vmeta_off, t); }

__device__ __forceinline__ uint32_t kcode_at(const Layout& L, const uint8_t* rec, int t, int c) {
    int by, bi;
    kcode_pos(L, t, c, &by, &bi);
    return (*(const uint32_t*)(rec + by) >> bi) & ((1u << L.kbits) - 1);
}
__device__ __forceinline__ uint32_t vcode_at(const Layout& L, const uint8_t* rec, int t, int c) {
    int by, bi;
    vcode_pos(L, t, c, &by, &bi);
    return (*(const uint32_t*)(rec + by) >> bi) & ((1u << L.vbits) - 1);
}
__device__ __forceinline__ uint16_t kscale_bits(const Layout& L, const uint8_t* rec, int c) {
    return *(const uint16_t*)(rec + L.kmeta_off + 2 * c);
}
__device__ __forceinline__ uint16_t kzero_bits(const Layout& L, const uint8_t* rec, int c) {
    return *(const uint16_t*)(rec + L.kmeta_off + 2 * kD + 2 * c);
}
// INT8 format: per-token key scale and zero.
__device__ __forceinline__ uint16_t ktok_scale_bits(const Layout& L, const uint8_t* rec, int t) {
    return *(const uint16_t*)(rec + tmeta_pos(L, L.kmeta_off, t));
}
__device__ __forceinline__ uint16_t ktok_zero_bits(const Layout& L, const uint8_t* rec, int t) {
    return *(const uint16_t*)(rec + tmeta_pos(L, L.kmeta_off, t) + 2 * L.spt);
}
__device__ __forceinline__ uint16_t vscale_bits(const Layout& L, const uint8_t* rec, int t) {
    return *(const uint16_t*)(rec + vmeta_pos(L, t));
}
__device__ __forceinline__ uint16_t vzero_bits(const Layout& L, const uint8_t* rec, int t) {
    return *(const uint16_t*)(rec + vmeta_pos(L, t) + 2 * L.spt);
}

}  // namespace kvq
