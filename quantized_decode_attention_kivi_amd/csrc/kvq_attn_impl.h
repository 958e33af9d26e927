// kvq_attn_impl.h -- split-K decode attention over the packed KV cache (gfx950):
// the kernel templates.  Each format family is instantiated in a translation
// unit of its own (kvq_attn_*.hip), compiled in parallel; kvq_attn.hip holds
// the split planning, the dispatch and the merge kernels.
//
// What it computes ("KV cache compression" (jaedaily), formula paragraph;
// "KV cache compression: quantization, eviction and sparse attention",
// sections 3.1, 3.2, 3.4 and 8.2): for every query head h of sequence b,
//   out = sum_t softmax_t(scale * q . k_t) v_t
// over the dequantized keys/values of the quantized groups and the fp16
// residual tokens.  The kernel dequantizes while it reads; the quantized part
// and the residual are processed by different workgroups and merged.
//
// Dequantization is folded into the contractions instead of materialised:
//   q . k_t      = sum_c (q_c s_c) code_tc + sum_c q_c z_c        (key group)
//   sum_t p_t v_t = sum_t (p_t s_t) code_t + sum_t p_t z_t        (value tokens)
// For one kv head and 32 tokens both are small dense products between the
// query heads of the GQA group (up to 16, padded to 16) and the codes, so they
// run on the matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation):
//   keys:   C[token][head]  = codes[token][c] . (q s)[c][head]
//   values: acc[head][c]   += (p s)[head][token] . codes[token][c]
// Codes are exact small integers in fp16.  q s is the exact product of two
// fp16 numbers (22 significant bits), so it is split exactly into an fp16
// high and low part and contracted twice; p s is split the same way (to 22
// bits).  The key zero points enter as one more product, z[c] . q[c][head],
// whose result seeds the key accumulator.  The vector ALU only unpacks codes
// and runs the online softmax.
//
// Work split: each stream (b, kv head) is cut into `splits` ranges of 32-token
// units plus one workgroup for the fp16 residual ring.  Waves walk their units
// independently (two units in flight per wave), combine in LDS, and every
// workgroup writes a partial (max, sum, output) to the workspace.  A second,
// small kernel merges the partials of each (stream, head) by log-sum-exp.
// The kernel boundary makes the partials visible to it; a per-workgroup
// device-scope release would write back the XCD's L2 once per workgroup.
#pragma once

#include <algorithm>
#include <type_traits>

#include "kvq_device.h"

namespace kvq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kPart = kD + 4;          // floats per head in a partial: out[128], m, l, pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ __forceinline__ uint32_t as_u32(h2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ h8 make_h8(h2 a, h2 b, h2 c, h2 d) {
    return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ h8 words_h8(uint4 w) {
    return make_h8(as_h2(w.x), as_h2(w.y), as_h2(w.z), as_h2(w.w));
}

// Maximum of two logits (finite, or -inf for nothing seen): one max
// instruction (these sources are built without NaN semantics, so no operand
// is quieted first, and a move from another lane folds into it as DPP).
__device__ __forceinline__ float max_logit(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = max_logit(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const uint32_t v = __builtin_bit_cast(uint32_t, x);
    auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max_logit(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}
// x(l) + x(l ^ 32): the first step of group_sum.
__device__ __forceinline__ float add_group_pairs(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
}
__device__ __forceinline__ float group_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
    const uint32_t v = __builtin_bit_cast(uint32_t, x);
    auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// Code unpacking (word layout: code_bit()).  INT4: byte-spread nibbles read as
// fp8 e4m3 are c * 2^-9 (exact, subnormals included), scaled by 512.  INT2:
// codes 0..3 in the low bits of a nibble read as fp4 e2m1 are c / 2, scaled by 2.
__device__ __forceinline__ h8 unpack4(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    return make_h8(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true));
}
__device__ __forceinline__ h8 unpack2_half(uint32_t w, bool upper) {
    const uint32_t x = (upper ? (w >> 2) : w) & 0x33333333u;
    return make_h8(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 0),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 1),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 2),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 3));
}
// Codes 8j..8j+7 of a lane's code sequence held in words w[].
template <int BITS>
__device__ __forceinline__ h8 codes8(const uint32_t* w, int j) {
    if (BITS == 4) return unpack4(w[j]);
    return unpack2_half(w[j >> 1], j & 1);
}

// Normal-quantile codebook: the same codes, looked up in the byte table lut
// (byte c = F * L_c, F = 64 for 2 bits, 16 for 4) and returned as the exact
// fp16 levels L_c in the same operand order.  Bytes become fp16 numbers
// 1024 + F L_c by pairing them with 0x64 (v_perm_b32), and one packed fma
// scales them to L_c exactly.
__device__ __forceinline__ uint32_t lut16(uint32_t x, const uint32_t (&lut)[4]) {   // x: a code in each byte
    const uint32_t s7 = x & 0x07070707u;
    const uint32_t a = __builtin_amdgcn_perm(lut[1], lut[0], s7);   // entries 0-7
    const uint32_t b = __builtin_amdgcn_perm(lut[3], lut[2], s7);   // entries 8-15
    const uint32_t m = ((x >> 3) & 0x01010101u) * 0xffu;             // bytes with code >= 8
    return (m & b) | (~m & a);
}
template <int BITS>
__device__ __forceinline__ h8 bytes_levels(uint32_t b0123, uint32_t b4567) {
    constexpr float invF = BITS == 2 ? 1.0f / 64.0f : 1.0f / 16.0f;
    const h2 sc = h2{(_Float16)invF, (_Float16)invF};
    const h2 off = h2{(_Float16)(-1024.0f * invF), (_Float16)(-1024.0f * invF)};
    const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, b0123, 0x04010400u)) * sc + off;
    const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, b0123, 0x04030402u)) * sc + off;
    const h2 c = as_h2(__builtin_amdgcn_perm(0x64646464u, b4567, 0x04010400u)) * sc + off;
    const h2 d = as_h2(__builtin_amdgcn_perm(0x64646464u, b4567, 0x04030402u)) * sc + off;
    return make_h8(a, b, c, d);
}
template <int BITS, bool CB>
__device__ __forceinline__ h8 levels8(const uint32_t* w, int j, const uint32_t (&lut)[4]) {
    if constexpr (!CB) {
        return codes8<BITS>(w, j);
    } else if constexpr (BITS == 4) {
        // codes 0-3 in the low nibbles of the bytes, 4-7 in the high ones
        return bytes_levels<4>(lut16(w[j] & 0x0F0F0F0Fu, lut), lut16((w[j] >> 4) & 0x0F0F0F0Fu, lut));
    } else {
        // nibble k holds code k (codes 8-15: bits 2-3); even codes -> bytes of
        // e, odd ones -> bytes of o; the 4-entry table is lut[0]
        const uint32_t y = (j & 1) ? (w[j >> 1] >> 2) : w[j >> 1];
        const uint32_t le = __builtin_amdgcn_perm(0u, lut[0], y & 0x03030303u);
        const uint32_t lo = __builtin_amdgcn_perm(0u, lut[0], (y >> 4) & 0x03030303u);
        return bytes_levels<2>(__builtin_amdgcn_perm(lo, le, 0x05010400u), __builtin_amdgcn_perm(lo, le, 0x07030602u));
    }
}

// a * b - c elementwise with one fp16 rounding (the exact low part of a * b
// when c is its rounded value), one packed fma per word with the
// subtrahend's sign in the instruction's negate modifiers.  Written with the
// compiler's fma (not inline assembly) so that its hazard tracking covers
// these instructions next to the matrix products.
__device__ __forceinline__ h2 fma_sub_h2(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_elementwise_fma(as_h2(a), as_h2(b), -as_h2(c));
}
__device__ __forceinline__ h8 fma_sub_h8(h8 a, h8 b, h8 c) {
    const u32x4 x = __builtin_bit_cast(u32x4, a), y = __builtin_bit_cast(u32x4, b), z = __builtin_bit_cast(u32x4, c);
    return make_h8(fma_sub_h2(x[0], y[0], z[0]), fma_sub_h2(x[1], y[1], z[1]), fma_sub_h2(x[2], y[2], z[2]),
                   fma_sub_h2(x[3], y[3], z[3]));
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One 32-token unit (NR = 32/G records) staged in LDS by the buffer unit's
// direct-to-LDS loads: each load instruction moves 16 bytes per lane from any
// record offset to LDS slot (base + 16*lane), so the next unit's codes are in
// flight without occupying registers.  Byte offsets inside one stage buffer:
//   KC   key codes.  16-bit keys (INT4): the 16 bytes lane (g, n) feeds the
//        key product of row tile rt sit at KC + rt*1024 + 16*lane.  INT2: the 8
//        bytes of (g, n, rt) sit at KC + rt*512 + 16*((g/2)*16 + n) + 8*(g%2).
//   VC   value codes.  G = 32: lane l's words 0-3 at VC + 16l, words 4-7 (INT4)
//        at VC + 1024 + 16l.  G = 16: record i's words of lane l at
//        VC + i*64*VW*4 + VW*4*l (VW words per lane and record).
//   META record i's key scale/zero table (512 B) then its value scale/zero
//        table (4G B) at META + i*MREC; SP (dense-and-sparse keys): then its
//        G kept-key entries (4G B).
template <int G, int KB, int VB, bool SP = false>
struct Stage {
    static constexpr int NR = 32 / G;
    static constexpr int SPT = G == 16 ? 4 : 8;
    static constexpr int VW = SPT * VB / 4;          // value words per lane and record
    static constexpr int KC = 0;
    static constexpr int VC = 512 * KB;
    static constexpr int META = VC + 512 * VB;
    static constexpr int MREC = 512 + 4 * G + (SP ? 4 * G : 0);
    static constexpr int BYTES = META + NR * MREC;
    // 16-byte aligned and large enough to hold a wave's [16][128] fp32
    // accumulators at the end (two waves per stage array)
    static constexpr int PITCH = BYTES < 4096 ? 4096 : (BYTES + 15) / 16 * 16;
    // direct-to-LDS load instructions per unit (the wait counts below)
    static constexpr int LOADS = G == 32 ? KB / 2 + VB / 2 + 1 : 6;
};

// s_waitcnt immediate that waits for all LDS operations of the wave.
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations of this wave are outstanding; other counters untouched.
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Buffer descriptor of one record, wave uniform (hardware range check: an
// absent record gets num_records = 0 and every load from it returns zeros).
__device__ __forceinline__ u32x4 record_desc(const uint8_t* rec, int bytes) {
    const uint64_t a = (uint64_t)rec;
    u32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    d[2] = __builtin_amdgcn_readfirstlane(rec ? (uint32_t)bytes : 0u);
    d[3] = 0x00020000u;
    return d;
}

// 16 bytes per lane from record offset `off` to LDS address lds + 16*lane.
// Issued from inline assembly so that the compiler inserts no waits of its
// own for the LDS write (it cannot tell the two stage buffers apart and would
// drain the prefetch); the kernel waits explicitly before reading a buffer.
// The load carries the non-temporal policy (nt): the cache is read once per
// call (7-12 % faster on the INT4 and paged layers).  With it, lanes of 64
// bytes read 16 bytes at a time (each load touching a quarter of every line
// it reaches) were much slower (8-bit G = 32 layout before its codes were
// stored in 16-byte chunks: INT8 layer 106 -> 145 us); lanes of 32 bytes read
// in two halves are not (INT4 values at G = 32; 8-bit values at G = 16:
// INT8 and FP8 8 x 32K layers at G = 16, 89.5 and 84.1 us with nt, 89.4 and
// 84.7 us without, same box).  The compiler's hazard tracking does not see
// inside the assembly, so the one wait state this chip family needs between a
// scalar write of M0 and a direct-to-LDS load reading it is written here.
__device__ __forceinline__ void lds_load16(u32x4 desc, lds_u8* dst, int off) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(off), "s"(desc), "{m0}"(m0)
                 : "memory");
}
// The same with the instruction's offset field K, which moves the LDS
// destination (m0 + K + 16*lane) and the record offset alike: loads whose LDS
// offsets inside the stage buffer equal their record offsets share one M0
// value (one scalar write and one wait state per unit instead of one per
// load).  off >= K in every lane; FIRST: the load right after M0 is written.
template <int K, bool FIRST>
__device__ __forceinline__ void lds_load16_at(u32x4 desc, uint32_t m0, int off) {
    static_assert(K >= 0 && K < 4096, "the offset field holds 12 bits");
    if constexpr (FIRST)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%3 nt lds" ::"v"(off - K), "s"(desc),
                     "{m0}"(m0), "n"(K)
                     : "memory");
    else
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%3 nt lds" ::"v"(off - K), "s"(desc), "{m0}"(m0),
                     "n"(K)
                     : "memory");
}

// Issues the direct-to-LDS loads of one unit into stage buffer `buf` (wave
// uniform address) and returns which of its records exist.  Every call issues
// exactly Stage::LOADS load instructions, so the wait counts stay exact.
template <int G, int KB, int VB, bool PG, bool SP = false>
__device__ __forceinline__ uint32_t issue_unit(lds_u8* buf, const Layout& L, const kvq_cache& c, int b, int h,
                                               int unit, int ngroups, int lane) {
    using S = Stage<G, KB, VB, SP>;
    const int g = lane >> 4, n = lane & 15;
    // The buffer's LDS address, made opaque here so that the per-load M0
    // values are formed next to each load rather than hoisted out of the unit
    // loop into scalar registers of their own.
    uint32_t base = (uint32_t)(uintptr_t)buf;
    asm volatile("" : "+s"(base));
    buf = (lds_u8*)(uintptr_t)base;
    uint32_t has = 0;
#pragma unroll
    for (int i = 0; i < S::NR; ++i) {
        const int grp = unit * S::NR + i;
        const uint8_t* rec = grp < ngroups ? record_at_t<PG>(L, c.packed, c.block_table, b, h, grp) : nullptr;
        has |= (rec != nullptr) << i;
        const u32x4 rs = record_desc(rec, L.record);
        if constexpr (G == 32 && KB == 2 && VB == 2) {
            // record sections at the same offsets as in the stage buffer
            // (key codes 0, value codes 1024, tables 2048): one M0 value
            const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)buf);
            const int rt = lane >> 5, gh = (lane >> 4) & 1;
            lds_load16_at<S::KC, true>(rs, m0, (16 * rt + n) * 32 + 16 * gh);
            lds_load16_at<S::VC, false>(rs, m0, L.vcode_off + S::VW * 4 * lane);
            // tables: lanes past them read out of range (zeros into the
            // stage buffer's unused tail, below PITCH) rather than branch,
            // so that the three loads stay in one block under one M0 write
            static_assert(S::META + 16 * 64 <= S::PITCH, "the table load's idle lanes land in the stage");
            const int nt = 32 + (SP ? G / 2 : G / 4);
            lds_load16_at<S::META, false>(rs, m0, lane < 32   ? L.kmeta_off + 16 * lane
                                                  : lane < nt ? L.vmeta_off + 16 * (lane - 32)
                                                              : 0x40000000);
            continue;
        }
        if (G == 32) {
            if (KB == 4) {
                lds_load16(rs, buf + S::KC, n * 64 + 16 * g);
                lds_load16(rs, buf + S::KC + 1024, (16 + n) * 64 + 16 * g);
            } else {
                // slot l = rt*32 + gh*16 + n  <-  token 16rt + n, lane groups 2gh, 2gh+1
                const int rt = lane >> 5, gh = (lane >> 4) & 1;
                lds_load16(rs, buf + S::KC, (16 * rt + n) * 32 + 16 * gh);
            }
            lds_load16(rs, buf + S::VC, L.vcode_off + S::VW * 4 * lane);
            if (VB == 4) lds_load16(rs, buf + S::VC + 1024, L.vcode_off + S::VW * 4 * lane + 16);
        } else {
            if (KB == 4) {
                lds_load16(rs, buf + S::KC + i * 1024, n * 64 + 16 * g);
            } else if (lane < 32) {
                const int gh = lane >> 4;
                lds_load16(rs, buf + S::KC + i * 512, n * 32 + 16 * gh);
            }
            if (VB == 4) {
                lds_load16(rs, buf + S::VC + i * 1024, L.vcode_off + 16 * lane);
            } else if (lane < 32) {
                lds_load16(rs, buf + S::VC + i * 512, L.vcode_off + 16 * lane);
            }
        }
        // key table, value table (and kept keys): contiguous in the record
        if (lane < 32 + (SP ? G / 2 : G / 4))
            lds_load16(rs, buf + S::META + i * S::MREC,
                       lane < 32 ? L.kmeta_off + 16 * lane : L.vmeta_off + 16 * (lane - 32));
    }
    return has;
}

// 8-bit formats (INT8, FP8 E4M3): one 32-token unit (NR = 32/G records)
// staged the same way, byte offsets inside one stage buffer:
//   KC   key bytes: load i = 2rt + half puts the 16 bytes lane (g, n) feeds
//        the key product of row tile rt (token 16rt + n, channels
//        32g + 16half .. +15) at KC + 1024 i + 16 lane.
//   VC   value bytes.  G = 32: bytes 16i .. 16i+15 of lane l's 64 at
//        VC + 1024 i + 16 l.  G = 16: record r's lane-l bytes 16half .. at
//        VC + 1024 (2r + half) + 16 l.
//   META INT8 only: record r's per-token key table (4G bytes) then its value
//        table (4G bytes) at META + 8G r.
template <int G, int F>
struct Stage8 {
    static constexpr int NR = 32 / G;
    static constexpr int SPT = G == 16 ? 4 : 8;
    static constexpr int KC = 0;
    static constexpr int VC = 4096;
    static constexpr int META = 8192;
    static constexpr int MREC = F == kFmtInt8 ? 8 * G : 0;
    static constexpr int BYTES = META + NR * MREC;
    static constexpr int PITCH = (BYTES + 15) / 16 * 16;
    static constexpr int LOADS = 8 + (F == kFmtInt8 ? NR : 0);
};

template <int G, int F, bool PG>
__device__ __forceinline__ uint32_t issue_unit8(lds_u8* buf, const Layout& L, const kvq_cache& c, int b, int h,
                                                int unit, int ngroups, int lane) {
    using S = Stage8<G, F>;
    uint32_t base = (uint32_t)(uintptr_t)buf;
    asm volatile("" : "+s"(base));
    buf = (lds_u8*)(uintptr_t)base;
    uint32_t has = 0;
#pragma unroll
    for (int i = 0; i < S::NR; ++i) {
        const int grp = unit * S::NR + i;
        const uint8_t* rec = grp < ngroups ? record_at_t<PG>(L, c.packed, c.block_table, b, h, grp) : nullptr;
        has |= (rec != nullptr) << i;
        const u32x4 rs = record_desc(rec, L.record);
        if (G == 32) {
#pragma unroll
            for (int k = 0; k < 4; ++k)   // k = 2rt + half
                lds_load16(rs, buf + S::KC + 1024 * k, 1024 * k + 16 * lane);
#pragma unroll
            for (int k = 0; k < 4; ++k) lds_load16(rs, buf + S::VC + 1024 * k, L.vcode_off + 1024 * k + 16 * lane);
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                lds_load16(rs, buf + S::KC + 1024 * (2 * i + hf), 1024 * hf + 16 * lane);
                lds_load16(rs, buf + S::VC + 1024 * (2 * i + hf), L.vcode_off + 32 * lane + 16 * hf);
            }
        }
        if (F == kFmtInt8 && lane < G / 2) lds_load16(rs, buf + S::META + i * S::MREC, L.kmeta_off + 16 * lane);
    }
    return has;
}

// Per-wave online-softmax state and value accumulators.
struct WaveAcc {
    f4 acc[8];        // acc[ct][i]: head 4g+i, channel 16ct+n
    float m;          // running max of head n (log2 units), same in all lane groups
    float l, pz;      // this lane's share of sum p and sum p*z for head n
};

__device__ __forceinline__ void acc_init(WaveAcc& A) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) A.acc[ct] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    A.m = kNegInf;
    A.l = 0.0f;
    A.pz = 0.0f;
}

// Moves the running max of every lane to mnew (>= A.m).  Only when it rose
// in some lane are the accumulators scaled, each row by its head's
// exp2(m - mnew): 1 where the max did not move, 0 where nothing was seen
// yet (m = -inf, the accumulators still zero).
__device__ __forceinline__ void raise_max(WaveAcc& A, float mnew, int lane) {
    if (__builtin_amdgcn_ballot_w64(mnew > A.m)) {
        const float alpha = mnew > A.m ? __builtin_amdgcn_exp2f(A.m - mnew) : 1.0f;
        // rows of acc are columns 4g+i; column j's alpha lives in lanes with n == j
        const int base = (lane & 48) | ((lane >> 4) << 2);
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, base + i);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) A.acc[ct][i] *= ai[i];
        A.l *= alpha;
        A.pz *= alpha;
    }
    A.m = mnew;
}

// Online-softmax step over the 8 logits x[] (raw q.k, slot order) of this
// lane's column, then the value contraction with operands vop(ct).  vs/vz:
// value scale/zero of each slot; valid: slot holds a token.  The weights p*s
// are split into fp16 high and low parts (22 bits).  LP (limb-packed): rows
// 0-7 of the value product take the high parts and rows 8-15 the low parts of
// heads 0-7, one product per column tile; otherwise each part is a product of
// its own over rows = heads.
template <bool LP, typename VOp>
__device__ __forceinline__ void softmax_and_values(WaveAcc& A, const float (&x)[8], const float (&vs)[8],
                                                   const float (&vz)[8], const bool (&valid)[8], float sl2,
                                                   int lane, VOp vop) {
    float cm = kNegInf;
#pragma unroll
    for (int k = 0; k < 8; ++k) cm = valid[k] ? max_logit(cm, x[k]) : cm;
    cm = group_max(cm);
    const float mnew = max_logit(A.m, cm * sl2);
    raise_max(A, mnew, lane);
    float w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        // invalid slots (masked tokens, missing records) contribute nothing,
        // whatever their (possibly non-finite) scale and zero bits
        const float p = valid[k] ? __builtin_amdgcn_exp2f(fmaf(x[k], sl2, -mnew)) : 0.0f;
        A.l += p;
        A.pz = valid[k] ? fmaf(p, vz[k], A.pz) : A.pz;
        w[k] = valid[k] ? p * vs[k] : 0.0f;
    }
    // fp16 high parts (w rounded) and low parts (w - hi, exact in fp32,
    // rounded), two weights per packed conversion
    h2 hp[4], lp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hp[j] = __builtin_convertvector((f2){w[2 * j], w[2 * j + 1]}, h2);
        lp[j] = __builtin_convertvector((f2){w[2 * j] - (float)hp[j][0], w[2 * j + 1] - (float)hp[j][1]}, h2);
    }
    const h8 whi = make_h8(hp[0], hp[1], hp[2], hp[3]), wlo = make_h8(lp[0], lp[1], lp[2], lp[3]);
    if (LP) {
        const h8 wop = (lane & 8) ? wlo : whi;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) A.acc[ct] = mfma(wop, vop(ct), A.acc[ct]);
    } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const h8 bop = vop(ct);
            A.acc[ct] = mfma(whi, bop, A.acc[ct]);
            A.acc[ct] = mfma(wlo, bop, A.acc[ct]);
        }
    }
}

// LP: the two limb partials of a logit sit in columns n and n^8 of the same
// 16-lane row; one DPP rotation by 8 brings them together.
__device__ __forceinline__ float add_limb_partner(float x) {
    // bound_ctrl with a zero "old" lets the compiler fold the move into the add
    const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128 /* row_ror:8 */, 0xf, 0xf, true);
    return x + __builtin_bit_cast(float, y);
}

// DPP rotation of a 32-bit value by 8 lanes within each 16-lane row: lane n
// receives lane n ^ 8's value.  Every source lane exists, so the zero "old"
// value with bound control is never used; it lets the compiler fold the move
// into the instruction that consumes it.
__device__ __forceinline__ uint32_t ror8(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128 /* row_ror:8 */, 0xf, 0xf, true);
}
__device__ __forceinline__ float ror8f(float x) { return __builtin_bit_cast(float, ror8(__builtin_bit_cast(uint32_t, x))); }

// Limb-packed rows split the unit's 8 slots between the two lanes of a head:
// lane n (< 8, the high limb) owns slots 0-3 (row tile 0), lane n + 8 (the
// low limb) slots 4-7 (row tile 1).  own_logit() forms the lane's full logit
// of slot (4 rt + i) for its own rt from the two row tiles' results: with
// `partnered`, the two lanes hold the high and low limb parts of the same
// logit (one DPP rotation adds the partner's); otherwise both hold it whole.
__device__ __forceinline__ bool high_limb_lane(int lane) { return (lane & 8) == 0; }
__device__ __forceinline__ float own_logit(float c0, float c1, int lane, bool partnered) {
    const bool hi = high_limb_lane(lane);
    const float own = hi ? c0 : c1;
    return partnered ? own + ror8f(hi ? c1 : c0) : own;
}

// Online-softmax step and value contraction of a limb-packed lane over its 4
// own slots (x[]: raw q.k, vs/vz: value scale/zero, valid: holds a token).
// Each lane evaluates the weights p s of its own slots only and forms both
// fp16 limbs of them (high part and low part: 22 bits); the lanes of a head
// then trade the limbs the other needs by DPP, so that row n of the value
// product gets the high parts of all 8 slots and row n + 8 the low parts,
// with each weight evaluated once.  A.l and A.pz hold the lane's share (its
// own slots): the two lanes of a head are added at the end.  TS, TZ:
// _Float16 where the scales and zeros are stored fp16 values, float
// otherwise.
template <typename TS, typename TZ, typename VOp>
__device__ __forceinline__ void softmax_and_values_lp(WaveAcc& A, const float (&x)[4], const TS (&vs)[4],
                                                      const TZ (&vz)[4], const bool (&valid)[4], float sl2,
                                                      int lane, VOp vop) {
    float cm = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k) cm = valid[k] ? max_logit(cm, x[k]) : cm;
    cm = max_logit(cm, ror8f(cm));   // the partner's 4 slots
    cm = group_max(cm);
    const float mnew = max_logit(A.m, cm * sl2);
    raise_max(A, mnew, lane);
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // invalid slots (masked tokens, missing records) contribute nothing,
        // whatever their (possibly non-finite) scale and zero bits
        const float p = valid[k] ? __builtin_amdgcn_exp2f(fmaf(x[k], sl2, -mnew)) : 0.0f;
        A.l += p;
        A.pz = valid[k] ? fmaf(p, (float)vz[k], A.pz) : A.pz;
        w[k] = valid[k] ? p * (float)vs[k] : 0.0f;
    }
    // the weights as fp16 high parts (w rounded) and low parts (w - hi, exact
    // in fp32, rounded): 22 bits, two weights per packed conversion
    h2 hp[2], lp[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        hp[j] = __builtin_convertvector((f2){w[2 * j], w[2 * j + 1]}, h2);
        lp[j] = __builtin_convertvector((f2){w[2 * j] - (float)hp[j][0], w[2 * j + 1] - (float)hp[j][1]}, h2);
    }
    uint32_t d[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t H = as_u32(hp[j]);
        const uint32_t Lw = as_u32(lp[j]);
        // slots 0-3: the high lane keeps its own high limbs; the low lane
        // (lanes 8-15 of the row, banks 2-3) takes its partner's low limbs
        d[j] = (uint32_t)__builtin_amdgcn_update_dpp((int)H, (int)Lw, 0x128 /* row_ror:8 */, 0xf, 0xc, false);
        // slots 4-7: the low lane keeps its own low limbs; the high lane
        // (banks 0-1) takes its partner's high limbs
        d[2 + j] = (uint32_t)__builtin_amdgcn_update_dpp((int)Lw, (int)H, 0x128, 0xf, 0x3, false);
    }
    const h8 wop = make_h8(as_h2(d[0]), as_h2(d[1]), as_h2(d[2]), as_h2(d[3]));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) A.acc[ct] = mfma(wop, vop(ct), A.acc[ct]);
}

// Token packing (limb-packed, at most 4 query heads per kv head): columns
// 4-7 and 12-15 of the products carry no head, so the second 16-token tile's
// logits move there, column c then holding head c & 3, tile (c >> 2) & 1 and
// limb c >> 3.  One DPP shift by 4 columns, written only to those columns
// (bank mask), does the move; every lane then has 4 logits instead of 8.
__device__ __forceinline__ float pack_second_tile(float first, float second) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, first),
                                                                 __builtin_bit_cast(int, second),
                                                                 0x114 /* row_shr:4 */, 0xf, 0xa, false));
}

// Online-softmax step and value contraction of a token-packed lane: 4 logits
// x[] (raw q.k) of its tile, value scale/zero vs/vz of those tokens.  The
// running max is shared by the head's four columns (one rotation by 4 pairs
// the tiles; the limb columns hold copies).  The value operand holds the
// lane's weights in its tile's half of the 8 token slots and zeros in the
// other half, so accumulator rows c, c + 4, c + 8, c + 12 add up to head c.
template <typename VOp>
__device__ __forceinline__ void softmax_and_values_tp(WaveAcc& A, const float (&x)[4], const float (&vs)[4],
                                                      const float (&vz)[4], const bool (&valid)[4], float sl2,
                                                      int lane, VOp vop) {
    float cm = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k) cm = valid[k] ? max_logit(cm, x[k]) : cm;
    cm = max_logit(cm, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, cm),
                                                                              0x124 /* row_ror:4 */, 0xf, 0xf, true)));
    cm = group_max(cm);
    const float mnew = max_logit(A.m, cm * sl2);
    raise_max(A, mnew, lane);
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float p = valid[k] ? __builtin_amdgcn_exp2f(fmaf(x[k], sl2, -mnew)) : 0.0f;
        A.l += p;
        A.pz = valid[k] ? fmaf(p, vz[k], A.pz) : A.pz;
        w[k] = valid[k] ? p * vs[k] : 0.0f;
    }
    // the lane's limb of each weight, two weights per packed conversion: the
    // high part (w rounded), or the low part (w - hi, exact in fp32, rounded)
    const bool lo = lane & 8;
    h2 part[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const h2 hi = __builtin_convertvector((f2){w[2 * j], w[2 * j + 1]}, h2);
        const h2 lw = __builtin_convertvector((f2){w[2 * j] - (float)hi[0], w[2 * j + 1] - (float)hi[1]}, h2);
        part[j] = as_h2(lo ? as_u32(lw) : as_u32(hi));
    }
    const h2 a = part[0], b = part[1], z = h2{(_Float16)0.0f, (_Float16)0.0f};
    const h8 wop = (lane & 4) ? make_h8(z, z, a, b) : make_h8(a, b, z, z);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) A.acc[ct] = mfma(wop, vop(ct), A.acc[ct]);
}

// Query operand of lane (g, n): q[head n][32g + 8j + e], zero for heads >= gq.
struct QOps {
    h8 q[4];
};

template <typename T>
__device__ __forceinline__ T lds_read(const lds_u8* p) {
    return *(const __attribute__((address_space(3))) T*)p;
}

// ---------------------------------------------------------------------------
// Pre-RoPE keys rotated on read ("KV cache compression: ...", section 3.3:
// KVQuant quantizes keys before the rotary embedding and applies it when
// reading; section 2: RoPE rotates pairs of dimensions).  Pair i = (2i, 2i+1)
// of token t turns by t * theta_i, theta_i = base^(-i/64).  The rotation
// depends on the token, so it cannot be folded into the query operand: each
// dequantized key element is rotated in fp32, split exactly into fp16 high
// and low parts, and both parts go through the key product with the plain
// fp16 query (its dequantization included: k = code * s + z per channel).
//
// Angles: phi_i = theta_i / 2pi turns per token as a 0.64 fixed-point
// fraction, so t * phi_i mod 1 is an exact integer product at any position;
// the (cos, sin) of a unit's first token comes from sincospi of that, those
// of its tokens t0 + r from a per-workgroup table of (cos, sin)(r theta_i),
// r <= 16, by the angle-addition formula.
// ---------------------------------------------------------------------------
// Attention instantiation formats beyond the cache formats: the low-bit
// format with pre-RoPE keys (3), with the codebook grid (4), with both (5).
constexpr int kFmtRope = 3;
constexpr int kFmtKiviCb = 4;
constexpr int kFmtRopeCb = 5;
constexpr int kFmtKiviSp = 6;     // dense-and-sparse keys, uniform grid
constexpr int kFmtKiviCbSp = 7;   // dense-and-sparse keys, codebook grid
constexpr bool low_bit(int F) { return F == kFmtKivi || F >= kFmtRope; }
constexpr bool rope_fmt(int F) { return F == kFmtRope || F == kFmtRopeCb; }
constexpr bool cb_fmt(int F) { return F == kFmtKiviCb || F == kFmtRopeCb || F == kFmtKiviCbSp; }
constexpr bool sp_fmt(int F) { return F == kFmtKiviSp || F == kFmtKiviCbSp; }
constexpr int kTabPitch = 66;     // float2 per table row: rows of lanes n = 0..15 hit distinct banks

struct RopeLds {
    uint64_t phi[64];                 // turns per token of pair i, 0.64 fixed point
    f2 tab[17][kTabPitch];            // (cos, sin)(r theta_i), r = 0..16
    f2 base[kWaves][2][64];           // per wave: (cos, sin) at the unit's tokens t0 and t0 + 16
};

// (sin, cos) of the angle a / 2^64 turns (the top 32 bits, signed: |turns| <= 1/2).
__device__ __forceinline__ void turns_sincos(uint64_t a, float* s, float* c) {
    const int hi = (int)(uint32_t)(a >> 32);
    sincospif((float)hi * 0x1p-31f, s, c);
}

// Workgroup prologue: phi and the table.  All threads.
__device__ void rope_setup(RopeLds& R, float theta, int tid) {
    if (tid < 64) {
        const double th = pow((double)theta, -(double)tid / 64.0);
        R.phi[tid] = (uint64_t)(th * (18446744073709551616.0 / 6.283185307179586476925));
    }
    __syncthreads();
    for (int e = tid; e < 17 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float sn, cs;
        turns_sincos((uint64_t)r * R.phi[i], &sn, &cs);
        R.tab[r][i] = f2{cs, sn};
    }
    __syncthreads();
}

// The wave's (cos, sin) at tokens t0 and t0 + 16 for every pair (lane = pair).
// The (cos, sin) pairs are stored halved, so the keys come out of the
// rotation at half their value (exactly: a power of two), which keeps their
// fp16 parts finite; the caller's logit scale is doubled to match.
__device__ __forceinline__ void rope_unit_base(RopeLds* R, int wave, int lane, int t0) {
    float sn, cs;
    turns_sincos((uint64_t)(uint32_t)t0 * R->phi[lane], &sn, &cs);
    sn *= 0.5f;
    cs *= 0.5f;
    const f2 t16 = R->tab[16][lane];
    R->base[wave][0][lane] = f2{cs, sn};
    R->base[wave][1][lane] = f2{cs * t16[0] - sn * t16[1], sn * t16[0] + cs * t16[1]};
    wave_sync();
}

// Key logits of both row tiles (token t0 + 16rt + n of lane (g, n), rt = 0, 1)
// against the lane's column head: getx(rt, j, x) gives the pre-RoPE key
// values x[0..7] of channels 32g + 8j .. + 7 (pairs i = 16g + 4j + p).  The
// lane's table entries (row n) are read once for both tiles.
template <typename GetX>
__device__ __forceinline__ void rope_key_tiles(const RopeLds* R, int wave, int lane, const QOps& Q, f4 (&C)[2],
                                               GetX getx) {
    const int g = lane >> 4, n = lane & 15;
    C[0] = C[1] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i0 = 16 * g + 4 * j;
        const f4 ts[2] = {*(const __attribute__((address_space(3))) f4*)&R->tab[n][i0],
                          *(const __attribute__((address_space(3))) f4*)&R->tab[n][i0 + 2]};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float x[8];
            getx(rt, j, x);
            const f4 bs[2] = {*(const __attribute__((address_space(3))) f4*)&R->base[wave][rt][i0],
                              *(const __attribute__((address_space(3))) f4*)&R->base[wave][rt][i0 + 2]};
            h2 hi[4], lo[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f4 b = bs[p >> 1], t = ts[p >> 1];
                const int o = 2 * (p & 1);
                const float Cs = b[o] * t[o] - b[o + 1] * t[o + 1];
                const float Sn = b[o + 1] * t[o] + b[o] * t[o + 1];
                const float k0 = Cs * x[2 * p] - Sn * x[2 * p + 1];
                const float k1 = Sn * x[2 * p] + Cs * x[2 * p + 1];
                // the pair's fp16 high parts (one packed conversion) and low
                // parts k - hi (exact in fp32), rounded
                hi[p] = __builtin_convertvector((f2){k0, k1}, h2);
                lo[p] = __builtin_convertvector((f2){k0 - (float)hi[p][0], k1 - (float)hi[p][1]}, h2);
            }
            C[rt] = mfma(make_h8(hi[0], hi[1], hi[2], hi[3]), Q.q[j], C[rt]);
            C[rt] = mfma(make_h8(lo[0], lo[1], lo[2], lo[3]), Q.q[j], C[rt]);
        }
    }
}

// ---------------------------------------------------------------------------
// Dense-and-sparse keys ("KV Cache compression lab", experiment 03: KVQuant
// keeps the few extreme keys in fp16 as a sparse matrix and quantizes the
// rest).  A kept entry's code is 0, so the dense product gave it the
// channel's zero z; its logit correction is q[head][c] * (x - z) for every
// query head.  The unit's entries are sorted by token, so each entry lane
// marks where its token's run starts and ends; then lane t (one per token)
// sums its run's corrections for all heads in registers and writes them to a
// per-wave [token][head] tile, from which each lane adds its logit slots'.
// No atomics: LDS atomics serialise across lanes.
// ---------------------------------------------------------------------------
struct SparseLds {
    _Float16 q[kD][16];               // the segment's query, [channel][head]
    float corr[kWaves][32][16];       // per wave: logit corrections [token of the unit][head]
    uint8_t run[kWaves][2][32];       // per wave: first and one-past-last entry of each token
};

template <int G, int MREC>
__device__ __forceinline__ void sparse_corrections(const lds_u8* meta, SparseLds* SPL, int wave, int lane) {
    // entry o = i*G + l of the unit (record i, entry l; ascending tokens)
    uint8_t(&run)[2][32] = SPL->run[wave];
    if (lane < 16) ((uint32_t*)&run[0][0])[lane] = 0u;   // empty runs
    int tok = 255;
    if (lane < 32) {
        const int i = lane / G, l = lane % G;
        const uint32_t e = lds_read<uint32_t>(meta + i * MREC + 512 + 4 * G + 4 * l);
        // (a position outside the group, possible only in a record this
        // library did not write, is ignored)
        if ((e & 0xffffu) < (uint32_t)(G * kD)) tok = i * G + (int)((e & 0xffffu) >> 7);
    }
    const int prev = __shfl_up(tok, 1), next = __shfl_down(tok, 1);
    if (lane < 32 && tok < 32) {
        if (lane == 0 || prev != tok) run[0][tok] = (uint8_t)lane;
        if (lane == 31 || next != tok) run[1][tok] = (uint8_t)(lane + 1);
    }
    wave_sync();
    if (lane < 32) {
        float acc[16];
#pragma unroll
        for (int h = 0; h < 16; ++h) acc[h] = 0.0f;
        const int o1 = run[1][lane];
        for (int o = run[0][lane]; o < o1; ++o) {
            const lds_u8* m = meta + (o / G) * MREC;
            const uint32_t e = lds_read<uint32_t>(m + 512 + 4 * G + 4 * (o % G));
            const int ch = (int)(e & (kD - 1));
            const float d = h2f(e >> 16) - h2f(lds_read<uint16_t>(m + 256 + 2 * ch));
            const h8 qa = __builtin_bit_cast(h8, *(const __attribute__((address_space(3))) u32x4*)&SPL->q[ch][0]);
            const h8 qb = __builtin_bit_cast(h8, *(const __attribute__((address_space(3))) u32x4*)&SPL->q[ch][8]);
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                acc[h] = fmaf((float)qa[h], d, acc[h]);
                acc[h + 8] = fmaf((float)qb[h], d, acc[h + 8]);
            }
        }
        f4* row = (f4*)&SPL->corr[wave][lane][0];
#pragma unroll
        for (int k = 0; k < 4; ++k) row[k] = f4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
    }
    wave_sync();
}

// One staged unit (see Stage): key logits on the matrix cores, then the
// online-softmax step and the value product.  RP: pre-RoPE keys (R, wave:
// the rotation tables; t0: the unit's first token).
template <int G, int KB, int VB, bool LP, bool RP, bool CB, bool SP, bool TP>
__device__ __forceinline__ void process_unit(const lds_u8* buf, uint32_t has, WaveAcc& A, const QOps& Q, float sl2,
                                             int lane, RopeLds* R, int wave, int t0, const Layout& L,
                                             SparseLds* SPL, int gq) {
    using S = Stage<G, KB, VB, SP>;
    constexpr int SPT = S::SPT;
    const int g = lane >> 4, n = lane & 15;
    const bool lo_limb = LP && (lane & 8);

    // Key side: accumulators start from sum_c z[c] q[c][head] (every row; LP:
    // high-limb columns only), then add codes . (q s) with q s split exactly
    // into fp16 high and low parts (LP: the part of the lane's column).
    f4 C[2];
    if constexpr (RP) {
        // pre-RoPE: dequantize, rotate, split, contract with the plain query
        rope_unit_base(R, wave, lane, t0);
        uint32_t kc[2][KB];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (KB == 4) {
                const u32x4 x = lds_read<u32x4>(buf + S::KC + rt * 1024 + 16 * lane);
                kc[rt][0] = x[0]; kc[rt][1] = x[1]; kc[rt][2] = x[2]; kc[rt][3] = x[3];
            } else {
                const u32x2 x = lds_read<u32x2>(buf + S::KC + rt * 512 + 16 * ((g >> 1) * 16 + n) + 8 * (g & 1));
                kc[rt][0] = x[0]; kc[rt][1] = x[1];
            }
        }
        rope_key_tiles(R, wave, lane, Q, C, [&](int rt, int j, float* x) {
            // the record's channel scales and zeros (one record for both
            // tiles when G = 32, record rt when G = 16)
            const lds_u8* km = buf + S::META + (S::NR == 2 ? rt : 0) * S::MREC;
            const h8 a = levels8<KB, CB>(kc[rt], j, L.klut);
            const h8 sj = __builtin_bit_cast(h8, lds_read<u32x4>(km + 16 * (4 * g + j)));
            const h8 zj = __builtin_bit_cast(h8, lds_read<u32x4>(km + 256 + 16 * (4 * g + j)));
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = fmaf((float)a[e], (float)sj[e], (float)zj[e]);
        });
    } else {
    // the unit's key codes are read first, so that their LDS latency overlaps
    // the scale/zero tables' reads and the q s products
    uint32_t kc[2][KB];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        if constexpr (KB == 4) {
            const u32x4 x = lds_read<u32x4>(buf + S::KC + rt * 1024 + 16 * lane);
            kc[rt][0] = x[0]; kc[rt][1] = x[1]; kc[rt][2] = x[2]; kc[rt][3] = x[3];
        } else {
            const u32x2 x = lds_read<u32x2>(buf + S::KC + rt * 512 + 16 * ((g >> 1) * 16 + n) + 8 * (g & 1));
            kc[rt][0] = x[0]; kc[rt][1] = x[1];
        }
    }
    // G = 16: both records' zero-point sums from one set of products, record
    // 0's zeros in rows 0-7 (lanes n < 8) and record 1's in rows 8-15; lane
    // groups 0-1 then hold record 0's sums and 2-3 record 1's, and one swap
    // of the wave's halves gives every lane both (the same products and
    // order as one record at a time: the same sums).
    float czr[S::NR];
    if constexpr (S::NR == 2) {
        const lds_u8* kz = buf + S::META + (n >= 8 ? S::MREC : 0) + 256;
        f4 c2 = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) c2 = mfma(__builtin_bit_cast(h8, lds_read<u32x4>(kz + 16 * (4 * g + j))), Q.q[j], c2);
        const uint32_t u = __builtin_bit_cast(uint32_t, c2[0]);
        const auto hv = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        czr[0] = __builtin_bit_cast(float, (uint32_t)hv[0]);
        czr[1] = __builtin_bit_cast(float, (uint32_t)hv[1]);
    }
    if constexpr (TP && S::NR == 2) {
        // Token packing at G = 16: column n carries head n & 3 of row tile
        // (n >> 2) & 1, whose tokens are that record's, so each lane forms
        // the q s limbs of its own column's record only (one set of products
        // instead of one per record) and both tiles' products use them: row
        // tile rt's logits are right in the columns of tile rt.
        const lds_u8* km = buf + S::META + ((n >> 2) & 1) * S::MREC;
        h8 qop[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h8 s = __builtin_bit_cast(h8, lds_read<u32x4>(km + 16 * (4 * g + j)));
            {
#pragma clang fp contract(off)
                qop[j] = Q.q[j] * s;
            }
        }
        if (lo_limb) {
            // low-limb columns (a divergent branch): q s - hi(q s), no bias
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 s = __builtin_bit_cast(h8, lds_read<u32x4>(km + 16 * (4 * g + j)));
                qop[j] = fma_sub_h8(Q.q[j], s, qop[j]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float z = lo_limb ? 0.0f : czr[rt];
            f4 acc = f4{z, z, z, z};
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = mfma(levels8<KB, CB>(kc[rt], j, L.klut), qop[j], acc);
            C[rt] = acc;
        }
    } else {
#pragma unroll
    for (int i = 0; i < S::NR; ++i) {
        const lds_u8* km = buf + S::META + i * S::MREC;
        f4 cz = S::NR == 2 ? f4{czr[i], czr[i], czr[i], czr[i]} : f4{0.0f, 0.0f, 0.0f, 0.0f};
        h8 qhi[4], qlo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h8 s = __builtin_bit_cast(h8, lds_read<u32x4>(km + 16 * (4 * g + j)));
            if constexpr (S::NR == 1) {
                const h8 z = __builtin_bit_cast(h8, lds_read<u32x4>(km + 256 + 16 * (4 * g + j)));
                cz = mfma(z, Q.q[j], cz);
            }
            {
#pragma clang fp contract(off)
                const h8 hi = Q.q[j] * s;
                qhi[j] = hi;
                if (!LP) qlo[j] = fma_sub_h8(Q.q[j], s, hi);
            }
        }
        if (LP && lo_limb) {
            // low-limb columns (a divergent branch: only these lanes pay for
            // it): the exact low parts q s - hi(q s), and no bias
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 s = __builtin_bit_cast(h8, lds_read<u32x4>(km + 16 * (4 * g + j)));
                qhi[j] = fma_sub_h8(Q.q[j], s, qhi[j]);
            }
            cz = f4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (S::NR == 2 && rt != i) continue;
            f4 acc = cz;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 a = levels8<KB, CB>(kc[rt], j, L.klut);
                acc = mfma(a, qhi[j], acc);
                if (!LP) acc = mfma(a, qlo[j], acc);
            }
            C[rt] = acc;
        }
    }
    }
    }

    // value codes of this lane (per record)
    uint32_t vc[S::NR][S::VW];
    if (G == 32) {
        const u32x4 x = lds_read<u32x4>(buf + S::VC + 16 * lane);
        vc[0][0] = x[0]; vc[0][1] = x[1]; vc[0][2] = x[2]; vc[0][3] = x[3];
        if (VB == 4) {
            const u32x4 y = lds_read<u32x4>(buf + S::VC + 1024 + 16 * lane);
            vc[0][4] = y[0]; vc[0][5] = y[1]; vc[0][6] = y[2]; vc[0][7] = y[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < S::NR; ++i) {
            if (VB == 4) {
                const u32x4 x = lds_read<u32x4>(buf + S::VC + i * 1024 + 16 * lane);
                vc[i][0] = x[0]; vc[i][1] = x[1]; vc[i][2] = x[2]; vc[i][3] = x[3];
            } else {
                const u32x2 x = lds_read<u32x2>(buf + S::VC + i * 512 + 8 * lane);
                vc[i][0] = x[0]; vc[i][1] = x[1];
            }
        }
    }

    // dense-and-sparse keys: the kept entries' corrections q . (x - z) to
    // their tokens' logits, gathered per (head, token) in the wave's tile
    if constexpr (SP) sparse_corrections<G, S::MREC>(buf + S::META, SPL, wave, lane);

    auto vop = [&](int ct) -> h8 {
        if (S::NR == 1) return levels8<VB, CB>(vc[0], ct, L.vlut);
        // G = 16: 4 slots of each record; code q = 4ct + slot
        const h8 a = levels8<VB, CB>(vc[0], ct >> 1, L.vlut);
        const h8 b = levels8<VB, CB>(vc[1], ct >> 1, L.vlut);
        const int o = 4 * (ct & 1);
        return h8{a[o], a[o + 1], a[o + 2], a[o + 3], b[o], b[o + 1], b[o + 2], b[o + 3]};
    };
    if constexpr (TP) {
        static_assert(LP && !RP && !SP, "token packing: limb-packed, post-RoPE keys, no kept keys");
        // the lane's tile (columns with bit 2 set: the second 16 tokens) and
        // its 4 logits, value scales and zeros
        const int rt = (lane >> 2) & 1;
        const int rec = S::NR == 2 ? rt : 0;
        const lds_u8* vm = buf + S::META + rec * S::MREC + 512 + g * 4 * SPT;
        float x[4], vs[4], vz[4];
        bool valid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = S::NR == 2 ? i : 4 * rt + i;
            // G = 16: each tile's logits are already in its own columns (the
            // limb partner n ^ 8 is in the same tile)
            x[i] = S::NR == 2 ? add_limb_partner(rt ? C[1][i] : C[0][i])
                              : pack_second_tile(add_limb_partner(C[0][i]), add_limb_partner(C[1][i]));
            vs[i] = h2f(lds_read<uint16_t>(vm + 2 * slot));
            vz[i] = h2f(lds_read<uint16_t>(vm + 2 * (SPT + slot)));
            valid[i] = S::NR == 1 || ((has >> rec) & 1);
        }
        softmax_and_values_tp(A, x, vs, vz, valid, sl2, lane, vop);
        return;
    }

    if constexpr (LP) {
        // the lane's own 4 slots: row tile rt = 0 (high limb lane) or 1 (low);
        // slot 4rt + i <-> token 16rt + 4g + i (pre-RoPE: both limb columns
        // already hold the head's full logit)
        const int rt = high_limb_lane(lane) ? 0 : 1;
        const int rec = S::NR == 2 ? rt : 0;
        const lds_u8* vm = buf + S::META + rec * S::MREC + 512 + g * 4 * SPT;
        float x[4];
        _Float16 vs[4], vz[4];
        bool valid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = S::NR == 2 ? i : 4 * rt + i;
            x[i] = own_logit(C[0][i], C[1][i], lane, !RP);
            if constexpr (SP) x[i] += SPL->corr[wave][16 * rt + 4 * g + i][n & 7];
            vs[i] = lds_read<_Float16>(vm + 2 * slot);
            vz[i] = lds_read<_Float16>(vm + 2 * (SPT + slot));
            valid[i] = S::NR == 1 || ((has >> rec) & 1);
        }
        softmax_and_values_lp(A, x, vs, vz, valid, sl2, lane, vop);
        return;
    }
    // value scale/zero of the lane's 8 slots: slot k = 4*rt + i <-> token 16rt + 4g + i
    float x[8], vs[8], vz[8];
    bool valid[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int rec = S::NR == 2 ? rt : 0;
        const lds_u8* vm = buf + S::META + rec * S::MREC + 512 + g * 4 * SPT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 4 * rt + i;
            const int slot = S::NR == 2 ? i : k;
            x[k] = C[rt][i];
            if constexpr (SP) x[k] += SPL->corr[wave][16 * rt + 4 * g + i][n];
            vs[k] = h2f(lds_read<uint16_t>(vm + 2 * slot));
            vz[k] = h2f(lds_read<uint16_t>(vm + 2 * (SPT + slot)));
            valid[k] = S::NR == 1 || ((has >> rec) & 1);
        }
    }
    softmax_and_values<false>(A, x, vs, vz, valid, sl2, lane, vop);
}

// Eight 8-bit codes (words w0, w1, byte order) as an fp16 operand.  INT8:
// code - 128, exact: v_perm_b32 pairs each byte with 0x64 into the fp16
// number 1024 + code, and one packed subtraction recentres it.  FP8: the
// E4M3 values themselves (exact in fp16).
template <int F>
__device__ __forceinline__ h8 conv8(uint32_t w0, uint32_t w1) {
    if (F == kFmtInt8) {
        const h2 off = h2{(_Float16)-1152.0f, (_Float16)-1152.0f};
        const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u)) + off;
        const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u)) + off;
        const h2 c = as_h2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u)) + off;
        const h2 d = as_h2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u)) + off;
        return make_h8(a, b, c, d);
    }
    return make_h8(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
}

// One staged unit of an 8-bit format.  The query is an exact fp16 operand
// and so are the codes, so each key product is one MFMA per 32 channels with
// no high/low split; the per-token dequantization acts on the finished dot
// products:
//   INT8  q . k_t = s_t (q . (code_t - 128)) + (z_t + 128 s_t) sum_c q_c
//   FP8   q . k_t = s_k (q . e_t)       (s_k folded into sl2 by the caller)
// and on the value side p s_t multiplies the code operand as in the low-bit
// format, with z_t + 128 s_t (INT8) or 0 (FP8) as the zero term.  LP: the
// columns n and n + 8 hold the same head, so both lane halves compute the
// same logits and need no limb partner.  qsum: sum_c q_c of the lane's head;
// vscl: the static value scale (FP8).
template <int G, int F, bool LP>
__device__ __forceinline__ void process_unit8(const lds_u8* buf, uint32_t has, WaveAcc& A, const QOps& Q,
                                              float sl2, float qsum, float vscl, int lane, int nvalid) {
    using S = Stage8<G, F>;
    constexpr int SPT = S::SPT;
    const int g = lane >> 4;

    f4 C[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const u32x4 x0 = lds_read<u32x4>(buf + S::KC + 1024 * (2 * rt) + 16 * lane);
        const u32x4 x1 = lds_read<u32x4>(buf + S::KC + 1024 * (2 * rt + 1) + 16 * lane);
        f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
        acc = mfma(conv8<F>(x0[0], x0[1]), Q.q[0], acc);
        acc = mfma(conv8<F>(x0[2], x0[3]), Q.q[1], acc);
        acc = mfma(conv8<F>(x1[0], x1[1]), Q.q[2], acc);
        acc = mfma(conv8<F>(x1[2], x1[3]), Q.q[3], acc);
        C[rt] = acc;
    }

    // value words of this lane: w[2][8]; column tile ct uses w[0][ct] and
    // w[1][ct] (G = 32: the slot halves 0-3 and 4-7 of the same record;
    // G = 16: slots 0-3 of records 0 and 1)
    uint32_t w[2][8];
    if (G == 32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4 v = lds_read<u32x4>(buf + S::VC + 1024 * k + 16 * lane);
            w[0][2 * k] = v[0];
            w[1][2 * k] = v[1];
            w[0][2 * k + 1] = v[2];
            w[1][2 * k + 1] = v[3];
        }
    } else {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const u32x4 v = lds_read<u32x4>(buf + S::VC + 1024 * (2 * r + hf) + 16 * lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) w[r][4 * hf + e] = v[e];
            }
    }

    auto vop = [&](int ct) -> h8 { return conv8<F>(w[0][ct], w[1][ct]); };
    // Per-token dequantization of row tile rt's 4 logits c[] of this lane
    // (slot 4rt + i <-> token 16rt + 4g + i), with their value scales and zeros.
    auto tile = [&](int rt, f4 c, float (&x)[4], float (&vs)[4], float (&vz)[4], bool (&valid)[4]) {
        const int rec = S::NR == 2 ? rt : 0;
        float ks4[4], kz4[4], vs4[4], vz4[4];
        if (F == kFmtInt8) {
            // the record's tables: per lane group g, SPT scales then SPT zeros
            const lds_u8* km = buf + S::META + rec * S::MREC + g * 4 * SPT;
            const lds_u8* vm = km + 4 * G;
            const int s0 = S::NR == 2 ? 0 : 4 * rt;   // first slot of this row tile
            const u32x2 a = lds_read<u32x2>(km + 2 * s0);
            const u32x2 bz = lds_read<u32x2>(km + 2 * SPT + 2 * s0);
            const u32x2 cv = lds_read<u32x2>(vm + 2 * s0);
            const u32x2 dz = lds_read<u32x2>(vm + 2 * SPT + 2 * s0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ks4[i] = h2f((a[i >> 1] >> (16 * (i & 1))) & 0xffffu);
                kz4[i] = h2f((bz[i >> 1] >> (16 * (i & 1))) & 0xffffu);
                vs4[i] = h2f((cv[i >> 1] >> (16 * (i & 1))) & 0xffffu);
                vz4[i] = h2f((dz[i >> 1] >> (16 * (i & 1))) & 0xffffu);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (F == kFmtInt8) {
                x[i] = fmaf(ks4[i], c[i], fmaf(128.0f, ks4[i], kz4[i]) * qsum);
                vs[i] = vs4[i];
                vz[i] = fmaf(128.0f, vs4[i], vz4[i]);
            } else {
                x[i] = c[i];
                vs[i] = vscl;
                vz[i] = 0.0f;
            }
            // (quantize-on-write: the unit may end inside its last record;
            // its later slots hold zero tokens, masked here)
            valid[i] = (S::NR == 1 || ((has >> rec) & 1)) && 16 * rt + 4 * g + i < nvalid;
        }
    };
    if constexpr (LP) {
        // both limb columns hold the head's full logits: each lane takes its
        // own row tile (0 for the high limb lane, 1 for the low), reading
        // that tile's tables at a per-lane address
        const bool hi = high_limb_lane(lane);
        f4 co;
#pragma unroll
        for (int i = 0; i < 4; ++i) co[i] = hi ? C[0][i] : C[1][i];
        float x[4], vs[4], vz[4];
        bool valid[4];
        tile(hi ? 0 : 1, co, x, vs, vz, valid);
        softmax_and_values_lp(A, x, vs, vz, valid, sl2, lane, vop);
        return;
    }
    float x[8], vs[8], vz[8];
    bool valid[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float xt[4], vst[4], vzt[4];
        bool vt[4];
        tile(rt, C[rt], xt, vst, vzt, vt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[4 * rt + i] = xt[i];
            vs[4 * rt + i] = vst[i];
            vz[4 * rt + i] = vzt[i];
            valid[4 * rt + i] = vt[i];
        }
    }
    softmax_and_values<false>(A, x, vs, vz, valid, sl2, lane, vop);
}

// Ring slot of token t0 + r (0 <= r < 32) given slot0 = t0 % ring; ring >= 16.
__device__ __forceinline__ int ring_slot(int slot0, int r, int ring) {
    int s = slot0 + r;
    s -= s >= ring ? ring : 0;
    s -= s >= ring ? ring : 0;
    return s;
}

// One 32-token unit of the fp16 residual ring: tokens t0 .. t0+31 (< n).
// Keys and query are exact fp16, so the key product needs one part (LP: the
// high-limb columns carry it, the low-limb columns add zero).  The value rows
// go straight to LDS (rows 0-15 to sva, 16-31 to svb, 256 bytes each; rows at
// or past n read as zeros), from where each lane gathers its operand columns.
template <bool LP, bool RP, bool TP>
__device__ __forceinline__ void process_residual(WaveAcc& A, const Layout& L, const kvq_cache& c, long sh, int t0,
                                                 int n, const QOps& Q, float sl2, int lane, lds_u8* sva,
                                                 lds_u8* svb, RopeLds* R, int wave) {
    const int g = lane >> 4, n16 = lane & 15;
    const int slot0 = t0 % L.ring;
    {
        const uint8_t* vbase = (const uint8_t*)c.v_res + sh * L.ring * kD * 2;
        const u32x4 vd = record_desc(vbase, L.ring * kD * 2);
        __builtin_amdgcn_s_waitcnt(kLgkmZero);   // earlier reads of these buffers returned
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int off = t0 + r < n ? ring_slot(slot0, r, L.ring) * (kD * 2) + 16 * n16 : 0x40000000;
            lds_load16(vd, i < 4 ? sva + 1024 * i : svb + 1024 * (i - 4), off);
        }
    }
    const half_t* kr = (const half_t*)c.k_res + sh * L.ring * kD;
    f4 C[2];
    if constexpr (RP) {
        rope_unit_base(R, wave, lane, t0);
        rope_key_tiles(R, wave, lane, Q, C, [&](int rt, int j, float* x) {
            const int r = 16 * rt + n16;
            const uint32_t keep = t0 + r < n ? 0xffffffffu : 0u;
            const uint4* row =
                (const uint4*)(kr + (long)(t0 + r < n ? ring_slot(slot0, r, L.ring) : slot0) * kD + 32 * g);
            uint4 w = row[j];
            w.x &= keep; w.y &= keep; w.z &= keep; w.w &= keep;
            const h8 k8 = words_h8(w);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)k8[e];
        });
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = 16 * rt + n16;
        f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t keep = t0 + r < n ? 0xffffffffu : 0u;
        const uint4* row = (const uint4*)(kr + (long)(t0 + r < n ? ring_slot(slot0, r, L.ring) : slot0) * kD + 32 * g);
        if constexpr (RP) {
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint4 w = row[j];
                w.x &= keep; w.y &= keep; w.z &= keep; w.w &= keep;
                acc = mfma(words_h8(w), Q.q[j], acc);
            }
            C[rt] = LP && (lane & 8) ? f4{0.0f, 0.0f, 0.0f, 0.0f} : acc;
        }
    }
    auto vop = [&](int ct) -> h8 {
        h8 b;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const lds_u8* rows = (k >> 2) ? svb : sva;
            b[k] = __builtin_bit_cast(_Float16, lds_read<uint16_t>(rows + (4 * g + (k & 3)) * (kD * 2) +
                                                                   (16 * ct + n16) * 2));
        }
        return b;
    };
    if constexpr (TP) {
        // token-packed columns, as in the quantized units
        const int rt = (lane >> 2) & 1;
        float x[4], vs[4], vz[4];
        bool valid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = pack_second_tile(add_limb_partner(C[0][i]), add_limb_partner(C[1][i]));
            vs[i] = 1.0f;
            vz[i] = 0.0f;
            valid[i] = t0 + rt * 16 + 4 * g + i < n;
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the value rows are in LDS
        wave_sync();
        softmax_and_values_tp(A, x, vs, vz, valid, sl2, lane, vop);
        return;
    }
    if constexpr (LP) {
        // own slots, as in the quantized units (the low limb lanes' key
        // products are zero unless pre-RoPE keys made both limbs whole)
        const int rt = high_limb_lane(lane) ? 0 : 1;
        float x[4], vs[4], vz[4];
        bool valid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = own_logit(C[0][i], C[1][i], lane, !RP);
            vs[i] = 1.0f;
            vz[i] = 0.0f;
            valid[i] = t0 + rt * 16 + 4 * g + i < n;
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the value rows are in LDS
        wave_sync();
        softmax_and_values_lp(A, x, vs, vz, valid, sl2, lane, vop);
        return;
    }
    float x[8], vs[8], vz[8];
    bool valid[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        x[k] = C[k >> 2][k & 3];
        vs[k] = 1.0f;
        vz[k] = 0.0f;
        valid[k] = t0 + (k >> 2) * 16 + 4 * g + (k & 3) < n;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the value rows are in LDS
    wave_sync();
    softmax_and_values<false>(A, x, vs, vz, valid, sl2, lane, vop);
}

// A wave's [16][128] fp32 accumulator image after the unit loop.
// Rows of a wave's accumulator image: limb-packed waves add the low-limb
// rows (head hh + 8) to the high ones in registers before writing it, token
// packing also the second token tile (hh + 4), so that the image holds one
// row per head.
template <bool LP, bool TP>
constexpr int acc_rows() { return TP ? 4 : LP ? 8 : 16; }
// Images per stage array (kWaves * pitch bytes): 4 (all in stage_a) or 2.
template <int ROWS>
constexpr int acc_per_array(int pitch) { return kWaves * pitch / (ROWS * kD * 4) >= kWaves ? kWaves : 2; }
template <int ROWS>
__device__ __forceinline__ float* wave_acc(uint8_t* stage_a, uint8_t* stage_b, int w, int pitch) {
    const int per = acc_per_array<ROWS>(pitch);
    return (float*)((w < per ? stage_a : stage_b) + (w % per) * ROWS * kD * 4);
}

// The workgroup reduction's per-wave totals (running max, weight sum, sum of
// p z per head); the kernel's prologue uses the same memory for its scan.
struct WaveRed {
    float m[kWaves][16], l[kWaves][16], pz[kWaves][16];
};

// Wave priority from the share of this wave's units still to do (3: more
// than 3/4 left ... 0: under 1/4).  Waves issue oldest-first, so without
// this the first workgroup placed on a CU runs ahead and the CU spends the
// end of the kernel with few waves; lagging waves now win arbitration and
// the workgroups of a CU finish close together.  Level k is reached while
// (4 left - 1) / total >= k, i.e. left >= ceil((k total + 1) / 4): the three
// thresholds are formed once per segment, so the unit loop only compares.
struct ProgressPrio {
    int t1, t2, t3;
};
__device__ __forceinline__ ProgressPrio progress_prio(int total) {
    return ProgressPrio{(total + 4) / 4, (2 * total + 4) / 4, (3 * total + 4) / 4};
}
__device__ __forceinline__ void set_progress_prio(int left, const ProgressPrio& p) {
    if (left >= p.t3) __builtin_amdgcn_s_setprio(3);
    else if (left >= p.t2) __builtin_amdgcn_s_setprio(2);
    else if (left >= p.t1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}
// The same levels, set only where the level changes (left is one of the
// thresholds, or the first unit): one scalar compare in the other units.
__device__ __forceinline__ void update_progress_prio(int left, bool first, const ProgressPrio& p) {
    if (first || left == p.t3 - 1 || left == p.t2 - 1 || left == p.t1 - 1) set_progress_prio(left, p);
}

// 32-token units of sequence b: its quantized groups first (G = 16: two
// records per unit), then its fp16 residual tokens.  Counters written by this
// library satisfy 0 <= nq <= n <= nq + ring; the clamps keep any other value
// inside the records and the ring.
// In the flattened work split a residual unit counts kResCost times a
// quantized one (its fp16 rows are gathered with plain loads, without the
// staged prefetch): `cost` is the stream's length in those terms.
constexpr int kResCost = 3;
struct SeqUnits {
    int nq, n, ngroups, uq, units, cost;
};
__device__ __forceinline__ SeqUnits seq_units(const Layout& L, const kvq_cache& c, int b) {
    SeqUnits u;
    u.nq = max(c.n_quant[b], 0);
    u.n = min(max(c.n_tokens[b], u.nq), u.nq + L.ring);
    u.ngroups = (u.nq + L.G - 1) / L.G;   // (the last one partial only when quantized on write)
    u.uq = (u.ngroups * L.G + 31) / 32;
    u.units = u.uq + (u.n - u.nq + 31) / 32;
    u.cost = u.uq + kResCost * (u.units - u.uq);
    return u;
}
// First unit whose cost position is >= x (a unit belongs to the workgroup
// that holds its first cost position).
__device__ __forceinline__ int unit_at(const SeqUnits& u, int x) {
    return x <= u.uq ? x : u.uq + (x - u.uq + kResCost - 1) / kResCost;
}

// Stage layout, unit issue and unit processing of a format.
template <int G, int KB, int VB, int F>
using StageT = typename std::conditional<low_bit(F), Stage<G, KB, VB, sp_fmt(F)>, Stage8<G, F>>::type;

template <int G, int KB, int VB, int F, bool PG>
__device__ __forceinline__ uint32_t issue_any(lds_u8* buf, const Layout& L, const kvq_cache& c, int b, int h,
                                              int unit, int ngroups, int lane) {
    if constexpr (low_bit(F)) return issue_unit<G, KB, VB, PG, sp_fmt(F)>(buf, L, c, b, h, unit, ngroups, lane);
    else return issue_unit8<G, F, PG>(buf, L, c, b, h, unit, ngroups, lane);
}

template <int G, int KB, int VB, int F, bool LP, bool TP>
__device__ __forceinline__ void process_any(const lds_u8* buf, uint32_t has, WaveAcc& A, const QOps& Q, float sl2,
                                            float qsum, float vscl, int lane, RopeLds* R, int wave, int t0,
                                            const Layout& L, SparseLds* SPL, int gq, int nq) {
    if constexpr (low_bit(F))
        process_unit<G, KB, VB, LP, rope_fmt(F), cb_fmt(F), sp_fmt(F), TP>(buf, has, A, Q, sl2, lane, R, wave, t0,
                                                                           L, SPL, gq);
    else process_unit8<G, F, LP>(buf, has, A, Q, sl2, qsum, vscl, lane, nq - t0);
}

// Units [lo, hi) of stream (b, h) by the four waves of the workgroup (wave w
// takes lo + w, lo + w + 4, ...), combined into one partial result (heads
// < gq: output[128] unnormalised, running max in log2 units, weight sum) at
// `part`.  Called by every thread of the workgroup.
template <int G, int KB, int VB, int F, bool LP, bool TP, bool PG, int NS>
__device__ __forceinline__ void attend_segment(uint8_t* stage_a, uint8_t* stage_b, uint8_t* stage_c, uint8_t* stage_d,
                                               WaveRed* red, const Layout& L, const kvq_cache& c,
                                               const half_t* __restrict__ q, float sl2, int gq, int b, int h,
                                               const SeqUnits& su, int lo, int hi, float* __restrict__ part,
                                               int lane, int wave, RopeLds* R, SparseLds* SPL) {
    using S = StageT<G, KB, VB, F>;
    // The lane index, produced afresh: per-lane addresses derived from it are
    // formed here, once per segment, instead of being hoisted out of the
    // segment loop and held (or spilled) across every unit loop.
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    const int g = lane >> 4, n16 = lane & 15;
    const int tid = wave * 64 + lane;
    const int Hq = L.H * gq;
    const long sh = (long)b * L.H + h;

    // The first unit's loads go out before the query's, so that the two
    // latencies overlap (the wait below covers both).
    const int q1 = min(hi, su.uq);
    int u = lo + wave;
    lds_u8* s0 = (lds_u8*)(stage_a + wave * S::PITCH);
    uint32_t h0 = 0;
    if (u < q1) h0 = issue_any<G, KB, VB, F, PG>(s0, L, c, b, h, u, su.ngroups, lane);

    QOps Q;
    {
        // column n: head n (LP: head n%8, high limb for n < 8, low limb above;
        // token packing at G = 16: head n%4, columns 4-7 and 12-15 for the
        // second row tile's record)
        const int hd = TP && G == 16 ? (n16 & 3) : LP ? (n16 & 7) : n16;
        const bool hv = hd < gq;
        const uint4* qp = (const uint4*)(q + ((long)b * Hq + h * gq + (hv ? hd : 0)) * kD + 32 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) Q.q[j] = words_h8(hv ? qp[j] : make_uint4(0, 0, 0, 0));
        // The unit loop's loads are invisible to the compiler's wait counting:
        // retire these here (with the first unit's) so that it places no wait
        // on them inside the loop.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    // Logit scale of the units' products (log2 units).  The low-bit keys are
    // contracted with q s formed in fp16: the query is first scaled by an
    // exact power of two 2^-k (k >= 0, one for the whole segment) that brings
    // every |q| below 1, so |q s| < s stays inside the fp16 range for any
    // finite scale s; 2^k moves into the logit scale.  Pre-RoPE keys are
    // rotated in fp32 and split into fp16 parts at half their value (a
    // rotated pair can reach sqrt(2) times the largest fp16), so their scale
    // doubles.
    float sl2s = sl2;
    _Float16 qscale = (_Float16)1.0f;
    if constexpr (rope_fmt(F)) {
        sl2s = 2.0f * sl2;
    } else if constexpr (low_bit(F)) {
        h2 m2 = h2{(_Float16)0.0f, (_Float16)0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                m2 = __builtin_elementwise_max(m2, __builtin_elementwise_abs(h2{Q.q[j][2 * e], Q.q[j][2 * e + 1]}));
        float m = group_max(fmaxf((float)m2[0], (float)m2[1]));
        // over the 16 columns of a row: lane ^ 8, ^ 4, ^ 2, ^ 1 (swizzle in
        // bit mode: and-mask 0x1f, xor-mask in bits 10-14)
        m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, m), 0x201f)));
        m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, m), 0x101f)));
        m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, m), 0x081f)));
        m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, m), 0x041f)));
        // m = f 2^e with f in [1/2, 1): k = max(e, 0) leaves max |q| 2^-k < 1
        const int k = __builtin_amdgcn_readfirstlane(max(__builtin_amdgcn_frexp_expf(m), 0));
        if (k > 0) {
            qscale = (_Float16)__builtin_ldexpf(1.0f, -k);
            const h8 f = h8{qscale, qscale, qscale, qscale, qscale, qscale, qscale, qscale};
#pragma unroll
            for (int j = 0; j < 4; ++j) Q.q[j] = Q.q[j] * f;
            sl2s = __builtin_ldexpf(sl2, k);
        }
    }
    if constexpr (sp_fmt(F)) {
        // the segment's query for the kept-key corrections, [channel][head],
        // scaled like the query operands
        for (int idx = tid; idx < kD * 16; idx += 256) {
            const int ch = idx >> 4, hh = idx & 15;
            SPL->q[ch][hh] = hh < gq ? q[((long)b * Hq + h * gq + hh) * kD + ch] * qscale : (_Float16)0.0f;
        }
        __syncthreads();
    }
    // 8-bit formats: sum_c q_c of the lane's head (INT8), the kv head's
    // static scales (FP8; the key scale joins the logit scale)
    float qsum = 0.0f, vscl = 0.0f, sl2q = sl2s;
    if (F == kFmtInt8) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) t += (float)Q.q[j][e];
        qsum = group_sum(t);
    } else if (F == kFmtFp8) {
        sl2q = sl2 * c.k_scale[h];
        vscl = c.v_scale[h];
    }
    WaveAcc A;
    acc_init(A);

    {
        const int ntot = max(1, (q1 - (lo + wave) + kWaves - 1) / kWaves);   // this wave's units
        const ProgressPrio prio = progress_prio(ntot);
        int left = ntot;   // units of this wave from u on
        if (u < q1) {
            // Direct-to-LDS loads: the next NS - 1 units of the wave are in
            // flight, each in a stage buffer of its own, while unit u is
            // processed from its buffer; the buffers rotate.  The waits are
            // explicit (vmcnt counts this wave's outstanding loads, in issue
            // order).  Unit u's loads were issued above.
            lds_u8* sb[NS];
            uint32_t hb[NS] = {};
            sb[0] = s0;
            hb[0] = h0;
            uint8_t* const arrays[4] = {stage_a, stage_b, stage_c, stage_d};
#pragma unroll
            for (int i = 1; i < NS; ++i) sb[i] = (lds_u8*)(arrays[i] + wave * S::PITCH);
            // units u + kWaves .. u + (NS - 2) kWaves go out now, the one
            // NS - 1 ahead at the top of each iteration
#pragma unroll
            for (int i = 1; i + 1 < NS; ++i)
                if (u + i * kWaves < q1) hb[i] = issue_any<G, KB, VB, F, PG>(sb[i], L, c, b, h, u + i * kWaves, su.ngroups, lane);
            for (;;) {
                // issue the unit NS - 1 ahead into the buffer freed last
                const int ahead = u + (NS - 1) * kWaves;
                if (ahead < q1) {
                    __builtin_amdgcn_s_waitcnt(kLgkmZero);   // last reads of that buffer returned
                    hb[NS - 1] = issue_any<G, KB, VB, F, PG>(sb[NS - 1], L, c, b, h, ahead, su.ngroups, lane);
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * S::LOADS));
                } else {
                    // the wave's later units still in flight: min(NS - 2, those left)
                    const int left = min((q1 - 1 - u) / kWaves, NS - 2);
                    if (NS >= 4 && left >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * S::LOADS));
                    else if (NS >= 3 && left >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(S::LOADS));
                    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                }
                wave_sync();
                update_progress_prio(left, left == ntot, prio);
                --left;
                process_any<G, KB, VB, F, LP, TP>(sb[0], hb[0], A, Q, sl2q, qsum, vscl, lane, R, wave, 32 * u, L, SPL, gq,
                                                  su.nq);
                u += kWaves;
                if (u >= q1) break;
                // rotate: the buffer just processed is the next to be refilled
                lds_u8* const t = sb[0];
#pragma unroll
                for (int i = 0; i + 1 < NS; ++i) {
                    sb[i] = sb[i + 1];
                    hb[i] = hb[i + 1];
                }
                sb[NS - 1] = t;
            }
        }
    }
    for (int u = lo + wave; u < hi; u += kWaves)
        if (u >= su.uq)
            process_residual<LP, rope_fmt(F), TP>(A, L, c, sh, su.nq + 32 * (u - su.uq), su.n, Q, sl2s, lane,
                                                (lds_u8*)(stage_a + wave * S::PITCH),
                                                (lds_u8*)(stage_b + wave * S::PITCH), R, wave);
    __builtin_amdgcn_s_setprio(0);

    // Wave results -> LDS: totals over the lane groups, accumulators by head.
    // The accumulators reuse the stage buffers: every wave has consumed its
    // staged units and has no load in flight once all have passed the barrier.
    // (limb-packed without token packing: the two lanes of a head each hold
    // the sums over their own slots)
    float lt = group_sum(A.l);
    float pzt = group_sum(A.pz);
    if (LP && !TP) {
        lt += ror8f(lt);
        pzt += ror8f(pzt);
    }
    __syncthreads();
    // TP: columns hh and hh + 4 hold the two token tiles of head hh
    const float lh = TP ? lt + __shfl(lt, (lane + 4) & 15) : lt;
    const float pzh = TP ? pzt + __shfl(pzt, (lane + 4) & 15) : pzt;
    if (lane < 16) {
        red->m[wave][lane] = A.m;
        red->l[wave][lane] = lh;
        red->pz[wave][lane] = pzh;
    }
    {
        // LP: row 4g + i + 8 (lane group g + 2) onto row 4g + i; TP: all
        // four lane groups onto group 0
        constexpr int ROWS = acc_rows<LP, TP>();
        if constexpr (LP) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) A.acc[ct][i] = TP ? group_sum(A.acc[ct][i]) : add_group_pairs(A.acc[ct][i]);
        }
        float* wacc = wave_acc<ROWS>(stage_a, stage_b, wave, S::PITCH);
        if (4 * g < ROWS) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) wacc[(4 * g + i) * kD + 16 * ct + n16] = A.acc[ct][i];
        }
    }
    __syncthreads();

    // Workgroup partial (heads < gq) -> workspace.
    for (int idx = tid; idx < gq * kD; idx += 256) {
        const int hh = idx >> 7, ch = idx & (kD - 1);
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red->m[w][hh]);
        float o = 0.0f, Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = red->m[w][hh];
            const float f = mw == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            const float a = wave_acc<acc_rows<LP, TP>()>(stage_a, stage_b, w, S::PITCH)[hh * kD + ch];
            o += (a + red->pz[w][hh]) * f;
            Ls += red->l[w][hh] * f;
        }
        part[hh * kPart + ch] = o;
        if (ch == 0) {
            part[hh * kPart + kD] = M;
            part[hh * kPart + kD + 1] = Ls;
        }
    }
    __syncthreads();   // the stage buffers are staged into again by the next segment
}

// Decode attention over the whole batch as one flattened sequence of work:
// sequence b contributes H streams (b, h) of cost_b each (its units, residual
// ones weighted kResCost), in (b, h) order, T in all, and workgroup w takes
// positions [w T / nwg, (w+1) T / nwg), a unit going to the workgroup holding
// its first position, whatever the sequence lengths (ragged batches and long
// single streams are balanced alike).  It writes one partial per stream segment it covers, at
// slot w + s for stream s (unique: along the workgroup order the covered
// streams never decrease).  The first workgroup of each stream records the
// stream's flattened start, and workgroup 0 records T; from these the merge
// finds the stream's workgroups.
// Waves per SIMD each instantiation is compiled for: four (at most 128
// registers) where that fits without spilling, else three.  A kernel that
// spills runs with scratch memory and far slower; the build rejects any
// attention kernel that uses scratch, so this table is checked.  Four waves
// fit the limb-packed kernels with INT2 values; without limb packing the
// separate high/low query operands take 16 more registers, INT4 values more
// than INT2 ones.  (Three waves lose little where the kernel waits on HBM.)
// The 8-bit formats stage twice the bytes per unit: their LDS allows two
// workgroups per CU, two waves per SIMD.
// Stage buffers per wave (the unit loop takes 2 to 4).  Two everywhere: more
// units in flight per wave cost workgroups per CU through LDS, and measured
// no faster (INT4 8 x 32K layer: 65.4 us with two, 65.7 with three, 66.2
// with four; INT2 1 x 128K: 30.0, 30.3, 31.8; paged batch: 152, 152, 163).
constexpr int attn_stages(int G, int KB, int VB, int F) { return 2; }

// Pre-RoPE keys take registers for the rotation: three waves.
constexpr int attn_waves(int G, int KB, int VB, int F, bool LP, bool PG) {
    return rope_fmt(F) ? 3 : !low_bit(F) ? 2 : F != kFmtKivi ? 3 : LP && VB == 2 && !(G == 16 && KB == 2) ? 4 : 3;
}

template <int G, int KB, int VB, int F, bool LP, bool TP, bool PG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves(G, KB, VB, F, LP, PG)))) void attn_kernel(
    Layout L, kvq_cache c, const half_t* __restrict__ q, float sl2, float* __restrict__ ws, int gq, int nwg,
    long meta_off) {
    using S = StageT<G, KB, VB, F>;
    // Two stage buffers per wave (ping-pong), in two arrays: the compiler
    // treats them as separate objects.  After the unit loop the same memory
    // holds the waves' accumulator images (all four in stage_a when they are
    // 4 KB, as with limb packing; else waves 0-1 in stage_a, 2-3 in stage_b).
    __shared__ __attribute__((aligned(16))) uint8_t stage_a[kWaves * S::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t stage_b[kWaves * S::PITCH];
    constexpr int NS = attn_stages(G, KB, VB, F);
    uint8_t* stage_c = nullptr;
    uint8_t* stage_d = nullptr;
    if constexpr (NS >= 3) {
        __shared__ __attribute__((aligned(16))) uint8_t stage_c_lds[kWaves * S::PITCH];
        stage_c = stage_c_lds;
    }
    if constexpr (NS >= 4) {
        __shared__ __attribute__((aligned(16))) uint8_t stage_d_lds[kWaves * S::PITCH];
        stage_d = stage_d_lds;
    }
    // The reduction totals: in stage_b where all four accumulator images fit
    // in stage_a (limb-packed kernels; their workgroups then take
    // 2 * kWaves * PITCH bytes of LDS), else an array of their own.
    WaveRed* red;
    if constexpr (acc_per_array<acc_rows<LP, TP>()>(S::PITCH) == kWaves) {
        static_assert(sizeof(WaveRed) <= kWaves * S::PITCH, "reduction totals fit a stage array");
        red = (WaveRed*)stage_b;
    } else {
        __shared__ WaveRed red_lds;
        red = &red_lds;
    }
    int* const wsum = (int*)red;            // [kWaves]
    int* const first = wsum + kWaves;       // sequence holding unit w T / nwg, flattened start of that sequence
    const int w = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
    SparseLds* SPL = nullptr;
    if constexpr (sp_fmt(F)) {
        __shared__ __attribute__((aligned(16))) SparseLds sparse_lds;
        SPL = &sparse_lds;
    }
    RopeLds* R = nullptr;
    if constexpr (rope_fmt(F)) {
        __shared__ __attribute__((aligned(16))) RopeLds rope_lds;
        rope_setup(rope_lds, L.rope_theta, tid);
        R = &rope_lds;
    }

    // Units per sequence, prefix over the batch (each thread a run of
    // consecutive sequences, then a scan over the threads).  Flattened
    // positions fit in 32 bits (the host rejects larger batches).
    const int per = (L.B + 255) / 256;
    const int b0 = min(tid * per, L.B), b1 = min(b0 + per, L.B);
    int mine = 0;
    for (int b = b0; b < b1; ++b) mine += L.H * seq_units(L, c, b).cost;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int T = 0, below = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int v = wsum[i];
        below += i < wave ? v : 0;
        T += v;
    }
    T = __builtin_amdgcn_readfirstlane(T);
    const int excl = below + incl - mine;
    const int start = __builtin_amdgcn_readfirstlane((int)((long)w * T / nwg));
    const int end = __builtin_amdgcn_readfirstlane((int)((long)(w + 1) * T / nwg));
    if (start < end && excl <= start && start < excl + mine) {
        int p = excl;
        for (int b = b0; b < b1; ++b) {
            const int f = L.H * seq_units(L, c, b).cost;
            if (start < p + f) {
                first[0] = b;
                first[1] = p;
                break;
            }
            p += f;
        }
    }
    __syncthreads();
    int* meta = (int*)((uint8_t*)ws + meta_off);
    if (w == 0 && tid == 0) meta[0] = T;
    if (start >= end) return;   // fewer units than workgroups

    int b = __builtin_amdgcn_readfirstlane(first[0]);
    const int pb = __builtin_amdgcn_readfirstlane(first[1]);
    __syncthreads();   // first[] read by every wave before stage buffers (which may hold it) are written
    SeqUnits su = seq_units(L, c, b);
    // (the division runs on the vector ALU: bring the result back to a scalar
    // register, or everything derived from it becomes per-lane)
    int h = __builtin_amdgcn_readfirstlane((start - pb) / su.cost);
    int ps = pb + h * su.cost;   // flattened start of stream (b, h)
    for (;;) {
        const int lo = __builtin_amdgcn_readfirstlane(max(start - ps, 0));
        const int hi = __builtin_amdgcn_readfirstlane(min(end - ps, su.cost));
        const int s = b * L.H + h;
        if (lo == 0 && wave == 0) {
            // the merge finds the stream's workgroups from its flattened start
            int l0;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l0));
            if (l0 == 0) meta[1 + s] = ps;
        }
        attend_segment<G, KB, VB, F, LP, TP, PG, NS>(stage_a, stage_b, stage_c, stage_d, red, L, c, q, sl2, gq, b, h, su,
                                          unit_at(su, lo), unit_at(su, hi), ws + ((long)w + s) * gq * kPart,
                                          lane, wave, R, SPL);
        if (ps + hi >= end) break;
        // next stream that has work (x < end <= T guarantees one)
        ps += su.cost;
        if (++h == L.H) {
            h = 0;
            do su = seq_units(L, c, ++b);
            while (su.units == 0);
        }
    }
}

// Resident attention workgroups on the current device: CUs x workgroups per
// CU for this instantiation (from its register and LDS footprint).  Falls
// back to 256 CUs x 3 when no device is visible (host-only size queries).
template <int G, int KB, int VB, int F, bool LP, bool TP, bool PG>
int attn_slots_for() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * 3;
    if (cached[dev]) return cached[dev];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)attn_kernel<G, KB, VB, F, LP, TP, PG>, 256, 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 3;
    (void)hipGetLastError();
    cached[dev] = cus * per_cu;
    return cached[dev];
}

// Limb packing: with at most 8 query heads per kv head, the high and low
// fp16 parts of q*s and p*s share one 16-column product.
static inline bool limb_packed(int gq) { return gq <= 8; }

// Launch of one (G, KB, VB, format) family: limb packing from the query
// heads per kv head, paged addressing from the layout.
// Token packing (see pack_second_tile): the uniform low-bit format with at
// most 4 query heads per kv head.
template <int F>
static inline bool token_packed(int gq) {
    return F == kFmtKivi && gq <= 4;
}

template <int G, int KB, int VB, int F>
hipError_t launch_attn_family(const Layout& L, const AttnPlan& P, const kvq_cache& c, const half_t* q, int gq,
                              float sl2, void* ws, hipStream_t s) {
#define KVQ_ATT3(LP, TP, PG)                                                                                 \
    hipLaunchKernelGGL((attn_kernel<G, KB, VB, F, LP, TP, PG>), dim3(P.nwg), dim3(256), 0, s, L, c, q, sl2, \
                       (float*)ws, gq, P.nwg, (long)P.meta_off)
    if (limb_packed(gq) && token_packed<F>(gq)) {
        if constexpr (F == kFmtKivi) {
            if (L.paged) KVQ_ATT3(true, true, true);
            else KVQ_ATT3(true, true, false);
        }
    } else if (limb_packed(gq)) {
        if (L.paged) KVQ_ATT3(true, false, true);
        else KVQ_ATT3(true, false, false);
    } else {
        if (L.paged) KVQ_ATT3(false, false, true);
        else KVQ_ATT3(false, false, false);
    }
#undef KVQ_ATT3
    return hipGetLastError();
}

// Resident workgroups of the family's instantiation for this launch.
template <int G, int KB, int VB, int F>
int attn_family_slots(const Layout& L, int gq) {
    if (limb_packed(gq) && token_packed<F>(gq)) {
        if constexpr (F == kFmtKivi)
            return L.paged ? attn_slots_for<G, KB, VB, F, true, true, true>()
                           : attn_slots_for<G, KB, VB, F, true, true, false>();
    }
    if (limb_packed(gq))
        return L.paged ? attn_slots_for<G, KB, VB, F, true, false, true>()
                       : attn_slots_for<G, KB, VB, F, true, false, false>();
    return L.paged ? attn_slots_for<G, KB, VB, F, false, false, true>()
                   : attn_slots_for<G, KB, VB, F, false, false, false>();
}

// Families and where they are instantiated: X(G, KB, VB, F).
#define KVQ_LOW_BIT_FAMILIES(X, F)                                                                      \
    X(16, 2, 2, F) X(16, 2, 4, F) X(16, 4, 2, F) X(16, 4, 4, F) X(32, 2, 2, F) X(32, 2, 4, F) X(32, 4, 2, F) \
    X(32, 4, 4, F)
#define KVQ_8BIT_FAMILIES(X) X(16, 8, 8, kFmtInt8) X(32, 8, 8, kFmtInt8) X(16, 8, 8, kFmtFp8) X(32, 8, 8, kFmtFp8)
#define KVQ_ALL_FAMILIES(X)                                                                             \
    KVQ_LOW_BIT_FAMILIES(X, kFmtKivi) KVQ_LOW_BIT_FAMILIES(X, kFmtRope) KVQ_LOW_BIT_FAMILIES(X, kFmtKiviCb) \
    KVQ_LOW_BIT_FAMILIES(X, kFmtRopeCb) KVQ_LOW_BIT_FAMILIES(X, kFmtKiviSp)                                 \
    KVQ_LOW_BIT_FAMILIES(X, kFmtKiviCbSp) KVQ_8BIT_FAMILIES(X)

#define KVQ_INSTANTIATE_FAMILY(GG, KB, VB, FF)                                                                     \
    template hipError_t launch_attn_family<GG, KB, VB, FF>(const Layout&, const AttnPlan&, const kvq_cache&,        \
                                                           const half_t*, int, float, void*, hipStream_t);        \
    template int attn_family_slots<GG, KB, VB, FF>(const Layout&, int);
#define KVQ_DECLARE_FAMILY(GG, KB, VB, FF)                                                                         \
    extern template hipError_t launch_attn_family<GG, KB, VB, FF>(const Layout&, const AttnPlan&, const kvq_cache&, \
                                                                  const half_t*, int, float, void*, hipStream_t); \
    extern template int attn_family_slots<GG, KB, VB, FF>(const Layout&, int);

}  // namespace kvq
