// kvq_device.h -- device helpers of libkvq: record addressing, the fp32
// quantizer step, code extraction.  gfx950 only.
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
// outside [0, num_blocks)).
__device__ __forceinline__ uint8_t* record_at(const Layout& L, void* packed, const int32_t* bt,
                                              int b, int h, int g) {
    long idx;
    if (L.paged) {
        if (g < 0 || g >= L.max_blocks) return nullptr;
        int id = bt[(long)b * L.max_blocks + g];
        if (id < 0 || id >= L.num_blocks) return nullptr;
        idx = (long)id * L.H + h;
    } else {
        if (g < 0 || g >= L.groups) return nullptr;
        idx = ((long)b * L.H + h) * L.groups + g;
    }
    return (uint8_t*)packed + idx * (long)L.record;
}

// Grid parameters of one quantized set ("KV Cache compression lab",
// experiment 01: 2^b levels from min to max, spacing (max-min)/(2^b-1)).
// Computed in fp32, stored in fp16; the codes use the stored values.
struct QParams {
    float z, inv;
    uint32_t sz_bits;  // fp16 s in the low half, fp16 z in the high half
};

__device__ __forceinline__ QParams make_qparams(float mn, float mx, int bits) {
#pragma clang fp contract(off)
    mn = mn + 0.0f;  // a -0 extreme becomes +0
    mx = mx + 0.0f;
    const float s32 = (mx - mn) / (float)((1 << bits) - 1);
    const uint16_t sb = f2h_bits(s32);
    const uint16_t zb = f2h_bits(mn);
    const float s = h2f(sb);
    QParams p;
    p.z = h2f(zb);
    p.inv = s > 0.0f ? 1.0f / s : 0.0f;
    p.sz_bits = (uint32_t)sb | ((uint32_t)zb << 16);
    return p;
}

// code = clamp(rint((x - z) * inv), 0, 2^b - 1), ties to even.
__device__ __forceinline__ uint32_t quant_code(float x, float z, float inv, float qmax) {
#pragma clang fp contract(off)
    const float t = (x - z) * inv;
    const float r = __builtin_rintf(t);
    return (uint32_t)fminf(fmaxf(r, 0.0f), qmax);
}

}  // namespace kvq
