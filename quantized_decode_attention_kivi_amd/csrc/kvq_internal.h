// kvq_internal.h -- layout of the packed cache and launcher declarations shared
// by the HIP translation units of libkvq (gfx950).  Not part of the public ABI.
//
// Packed cache: one RECORD per (key group of G tokens, kv head), G = 16 or 32.
// A record holds everything the decode kernel needs for those G tokens ("KV
// cache compression: quantization, eviction and sparse attention", section
// 3.4: a block carries its codes and its scale/zero tables, the key group is
// aligned to the block).  Its sections are laid out for the decode kernel's
// matrix-core operands (16x16 f16 MFMA tiles, wave64: lane l = 16*g + n with
// lane group g = l/16 and row/column n = l%16):
//
//   [0, kcode)            key codes, token-major, 16*kb bytes per token.  Inside
//                         a token the 32 channels 32g..32g+31 of lane group g
//                         occupy 4*kb bytes at offset 4*kb*g, in code order
//                         q = channel - 32g packed by code_bit().
//   [vcode_off, +vcode)   value codes: lane l = 16g + n owns SPT*vb bytes
//                         holding, in code order q = ct*SPT + slot (ct = 0..7,
//                         slot = 0..SPT-1), the code of channel 16*ct + n for
//                         the token of that slot (vslot()).  SPT = 8 for
//                         G = 32, 4 for G = 16.  Lanes of at most 32 bytes are
//                         contiguous (offset l*SPT*vb); the 64-byte lanes of
//                         the 8-bit formats at G = 32 are cut into 16-byte
//                         chunks, chunk k of lane l at 1024*k + 16*l
//                         (vlane_byte()), so that each 16-byte load per lane
//                         reads 1 KiB of whole cache lines.
//   [kmeta_off, +512)     key scales s[128] then key zeros z[128], fp16,
//                         channel order.
//   [vmeta_off, +4G)      per lane group g: SPT value scales then SPT value
//                         zeros, fp16, slot order (4*SPT bytes per group).
//
// Code order inside a 32-bit word (code_bit): 8-bit code q (0..3) in byte q;
// INT4 code q (0..7) sits at nibble
// {0,2,4,6,1,3,5,7}[q]; INT2 code q (0..15) at bit 4*(q%8) + 2*(q/8).  These
// are the orders in which the gfx950 fp8 / fp4 conversion instructions return
// nibbles, so the decode kernel unpacks a word straight into operand order.
//
// 8-bit formats (INT8, FP8 E4M3) keep the same sections with one byte per
// code (code_bit(8, q) = 8q, so a lane's value bytes are in code order).
// Their key bytes are stored in 16-byte pieces, the piece of token t holding
// channels 16h .. 16h+15 (h = c/16) at 1024*(2*(t/16) + h%2) + 16*(16*(h/2) +
// t%16) (k8_byte()): piece k of lane l = 16g + n at 1024*k + 16*l is the
// lane's 16-byte key operand for token 16*(k/2) + n, channels 32g + 16*(k%2),
// so that each 16-byte load per lane reads 1 KiB of whole cache lines; their key scale/zero table is per token, laid
// out like the value table (kmeta_off, 4G bytes, INT8 only), and FP8 records
// carry no tables at all (its scales are per kv head, outside the records).
//
// Dense-and-sparse keys add, after the value table, G 4-byte entries
// (position t*128 + c in the low half, the fp16 key in the high half), in
// ascending position order: the group's kept extreme keys.
//
// Contiguous caches address record (b, h, g) at ((b*H + h)*groups + g); paged
// caches at (block_table[b][g]*H + h).  The fp16 residual ring of (b, h) holds
// token i at slot i % (R + G), token-major, 128 channels per slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kD = 128;          // head dim (only size implemented)
constexpr int kMaxGq = 16;       // query heads per kv head

// Cache formats (KVQ_FORMAT_*).
constexpr int kFmtKivi = KVQ_FORMAT_KIVI;
constexpr int kFmtInt8 = KVQ_FORMAT_INT8;
constexpr int kFmtFp8 = KVQ_FORMAT_FP8_E4M3;

struct Layout {
    int fmt;
    float rope_theta;                             // > 0: keys are pre-RoPE, rotated on read
    int grid;                                     // KVQ_GRID_*
    uint32_t klut[4], vlut[4];                    // codebook: byte k = F_b * L_k (key / value bits)
    float kmid[15], vmid[15];                     // codebook: midpoints of consecutive levels, grid steps
    int sparse;                                   // dense-and-sparse keys: G kept (pos, fp16) pairs per record
    int sparse_off;                               // their offset in the record (after the value table)
    int B, H, kbits, vbits, G, R, ring;
    int onwrite;                                  // 8-bit format without a residual window:
                                                  // every token quantized as it is written
    int paged, num_blocks, max_blocks, groups;   // groups: record slots per sequence
    int capacity;                                 // max tokens a sequence may hold
    int spt;                                      // value-code slots per lane and column tile
    int kcode, vcode, vcode_off, kmeta_off, vmeta_off, record;
};

// Fills *L from cfg; returns KVQ_OK or the validation error.
kvq_status make_layout(const kvq_config* cfg, Layout* L);

// Offset inside the key codes of the 8-bit formats of the byte of token t,
// channel c.
__host__ __device__ inline int k8_byte(int t, int c) {
    return 1024 * (2 * (t >> 4) + ((c >> 4) & 1)) + 16 * (16 * (c >> 5) + (t & 15)) + (c & 15);
}

// Offset inside the value codes of byte b of lane `lane`'s lane_bytes bytes.
__host__ __device__ inline int vlane_byte(int lane_bytes, int lane, int b) {
    return lane_bytes <= 32 ? lane * lane_bytes + b : 1024 * (b >> 4) + 16 * lane + (b & 15);
}

// Quantized tokens of a sequence holding n: whole groups outside the
// newest R tokens.
__host__ __device__ inline int num_quantized(int n, int G, int R) {
    int over = n - R;
    return over <= 0 ? 0 : G * (over / G);
}

// The same for layout L: with quantize-on-write (L.onwrite) all n tokens,
// the last group possibly partial.
__host__ __device__ inline int quantized_count(const Layout& L, int n) {
    return L.onwrite ? (n > 0 ? n : 0) : num_quantized(n, L.G, L.R);
}

// Codebook levels of b bits (2 or 4) in 1/F_b grid steps, F_b = 64 or 16:
// levels16[k] = F_b * L_k; returns F_b (0 for other widths).
int codebook_levels16(int bits, int* levels16);

// Instantiation key of a layout: format * 10000 + G * 100 + kbits * 10 + vbits.
inline int layout_key(const Layout& L) { return L.fmt * 10000 + L.G * 100 + L.kbits * 10 + L.vbits; }

// Bit offset of code q inside its 32-bit word.
__host__ __device__ inline int code_bit(int bits, int q) {
    if (bits == 8) return 8 * q;
    if (bits == 4) {
        const int nib = (q & 3) * 2 + ((q >> 2) & 1);   // {0,2,4,6,1,3,5,7}[q]
        return 4 * nib;
    }
    return 4 * (q & 7) + 2 * ((q >> 3) & 1);
}

// Lane group and slot of record token t in the value-code and value-meta
// sections; inverse: t = (slot/4)*16 + 4*g + slot%4.
__host__ __device__ inline void vslot(int t, int* g, int* slot) {
    *g = (t & 15) >> 2;
    *slot = ((t >> 4) << 2) | (t & 3);
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
hipError_t launch_export_outliers(const Layout& L, const kvq_cache& c, uint16_t* pos, uint16_t* val, int out_tokens,
                                  hipStream_t s);

struct AttnPlan {
    int nwg;             // attention workgroups (each an equal share of the batch's units)
    long slots;          // partial-result slots: nwg + streams - 1
    size_t part_floats;  // floats of one partial result (Hq/H heads x (128 + 4))
    size_t meta_off;     // bytes: T (units of the batch), then each stream's first unit, after the slots
    size_t workspace;    // bytes
    bool fits;           // the batch's units at capacity fit the kernel's 32-bit positions
};
AttnPlan plan_attention(const Layout& L, int num_q_heads);
hipError_t launch_attention_partials(const Layout& L, const AttnPlan& P, const kvq_cache& c, const _Float16* q,
                                     int num_q_heads, float scale, void* ws, hipStream_t s);
hipError_t launch_attention_merge(const Layout& L, const AttnPlan& P, const kvq_cache& c, int num_q_heads,
                                  const void* ws, float* out, hipStream_t s);

}  // namespace kvq
