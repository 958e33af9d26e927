// kvq_internal.h -- layout of the packed cache and launcher declarations shared
// by the HIP translation units of libkvq (gfx950).  Not part of the public ABI.
//
// Packed cache: one RECORD per (key group of G tokens, kv head).  A record holds
// everything the decode kernel needs for those G tokens ("KV cache compression:
// quantization, eviction and sparse attention", section 3.4: a block carries its
// codes and its scale/zero tables, the key group is aligned to the block):
//
//   [0, kcode)            key codes, token-major, LSB-first:
//                         element (t, c) at bit (t*128 + c) * k_bits
//   [vcode_off, +vcode)   value codes in 16-token units: unit (j = t/16, c) is
//                         16*v_bits bits at unit index j*128 + c; token t%16
//                         at bit (t%16) * v_bits of the unit
//   [kmeta_off, +512)     128 key (s, z) fp16 pairs, channel c at 4*c
//   [vmeta_off, +4G)      G value (s, z) fp16 pairs, token t at 4*t
//
// Contiguous caches address record (b, h, g) at ((b*H + h)*groups + g); paged
// caches at (block_table[b][g]*H + h).  The fp16 residual ring of (b, h) holds
// token i at slot i % (R + G).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kD = 128;          // head dim (only size implemented)
constexpr int kMaxGq = 16;       // query heads per kv head

struct Layout {
    int B, H, kbits, vbits, G, R, ring;
    int paged, num_blocks, max_blocks, groups;   // groups: record slots per sequence
    int capacity;                                 // max tokens a sequence may hold
    int kcode, vcode, vcode_off, kmeta_off, vmeta_off, record;
};

// Fills *L from cfg; returns KVQ_OK or the validation error.
kvq_status make_layout(const kvq_config* cfg, Layout* L);

// Largest n_q a sequence may reach.
__host__ __device__ inline int num_quantized(int n, int G, int R) {
    int over = n - R;
    return over <= 0 ? 0 : G * (over / G);
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_prefill(const Layout& L, const kvq_cache& c, const _Float16* k, const _Float16* v,
                          int max_len, const int32_t* seq_lens, hipStream_t s);
hipError_t launch_append(const Layout& L, const kvq_cache& c, const _Float16* k, const _Float16* v,
                         hipStream_t s);
hipError_t launch_dequantize(const Layout& L, const kvq_cache& c, float* ko, float* vo, int out_tokens,
                             hipStream_t s);
hipError_t launch_export(const Layout& L, const kvq_cache& c, uint8_t* kc, uint8_t* vc, uint16_t* ks,
                         uint16_t* kz, uint16_t* vs, uint16_t* vz, int out_tokens, hipStream_t s);

struct AttnPlan {
    int splits;        // quantized-part splits per stream (plus one residual split)
    int groups_per_split;
    size_t workspace;  // bytes
};
AttnPlan plan_attention(const Layout& L, int num_q_heads);
hipError_t launch_attention(const Layout& L, const AttnPlan& P, const kvq_cache& c, const _Float16* q,
                            int num_q_heads, float scale, float* out, void* ws, hipStream_t s);

}  // namespace kvq
