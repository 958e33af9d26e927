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
#include "kvq_device.h"

namespace kvq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

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

// Max over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const uint32_t v = __builtin_bit_cast(uint32_t, x);
    auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
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

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Raw loads of one 32-token unit: NR records (1 for G = 32, 2 for G = 16).
template <int G, int KB, int VB>
struct UnitRaw {
    static constexpr int NR = 32 / G;
    static constexpr int SPT = G == 16 ? 4 : 8;
    static constexpr int VW = SPT * VB / 4;    // value words per lane and record
    uint32_t kc[2][KB];                        // per row tile: this lane's 32 key codes
    uint32_t vc[NR][VW];                       // per record: this lane's value codes
    uint2 km[NR];                              // per record: 8 bytes of key meta
    uint4 vm[NR];                              // per record: 16 bytes of value meta (some lanes)
    bool has[NR];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over one record (hardware range check: an absent record
// gets num_records = 0 and every load from it returns zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const uint8_t* rec, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, rec ? bytes : 0, 0x00020000);
}

template <int G, int KB, int VB>
__device__ __forceinline__ void load_unit(UnitRaw<G, KB, VB>& r, const Layout& L, const kvq_cache& c, int b, int h,
                                          int unit, int ngroups, int lane) {
    // Buffer loads: every call issues the same loads (so the wait counts stay
    // exact and the next unit's loads overlap this unit's arithmetic), and the
    // compiler does not re-issue them at their point of use.
    using R = UnitRaw<G, KB, VB>;
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int i = 0; i < R::NR; ++i) {
        const int grp = unit * R::NR + i;
        const uint8_t* rec = grp < ngroups ? record_at(L, c.packed, c.block_table, b, h, grp) : nullptr;
        r.has[i] = rec != nullptr;
        const __amdgpu_buffer_rsrc_t rs = record_rsrc(rec, L.record);
        const u32x2 km = __builtin_amdgcn_raw_buffer_load_b64(rs, L.kmeta_off + 8 * lane, 0, 0);
        r.km[i] = make_uint2(km[0], km[1]);
        const u32x4 vm = __builtin_amdgcn_raw_buffer_load_b128(rs, L.vmeta_off + 16 * (lane < G / 4 ? lane : 0), 0, 0);
        r.vm[i] = make_uint4(vm[0], vm[1], vm[2], vm[3]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (R::NR == 2 && rt != i) continue;
            const int t = R::NR == 2 ? n : 16 * rt + n;
            const int off = t * 16 * KB + 4 * KB * g;
            if (KB == 4) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
                r.kc[rt][0] = x[0]; r.kc[rt][1] = x[1]; r.kc[rt][2] = x[2]; r.kc[rt][3] = x[3];
            } else {
                const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
                r.kc[rt][0] = x[0]; r.kc[rt][1] = x[1];
            }
        }
        const int pv = L.vcode_off + lane * R::VW * 4;
#pragma unroll
        for (int w = 0; w < R::VW; w += 4) {
            if (w + 4 <= R::VW) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, pv + 4 * w, 0, 0);
                r.vc[i][w] = x[0]; r.vc[i][w + 1] = x[1]; r.vc[i][w + 2] = x[2]; r.vc[i][w + 3] = x[3];
            } else {
                const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, pv + 4 * w, 0, 0);
                r.vc[i][w] = x[0]; r.vc[i][w + 1] = x[1];
            }
        }
    }
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
    for (int k = 0; k < 8; ++k) cm = valid[k] ? fmaxf(cm, x[k]) : cm;
    cm = group_max(cm);
    const float mnew = fmaxf(A.m, cm * sl2);
    const float alpha = mnew == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(A.m - mnew);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
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
    h8 whi, wlo;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const _Float16 hi = (_Float16)w[k];
        whi[k] = hi;
        wlo[k] = (_Float16)(w[k] - (float)hi);
    }
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
    const int y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128 /* row_ror:8 */, 0xf, 0xf, false);
    return x + __builtin_bit_cast(float, y);
}

template <int G>
struct AttnSmem {
    // per wave: key meta (2 records x 512 B) and value meta (2 records x 128 B)
    uint32_t kmeta[kWaves][2][kD];
    uint32_t vmeta[kWaves][2][32];
    float wm[kWaves][16], wl[kWaves][16], wpz[kWaves][16];
    float wacc[kWaves][16][kD];
};

// Query operand of lane (g, n): q[head n][32g + 8j + e], zero for heads >= gq.
struct QOps {
    h8 q[4];
};

template <int G, int KB, int VB, bool LP>
__device__ __forceinline__ void process_unit(AttnSmem<G>& sm, WaveAcc& A, const UnitRaw<G, KB, VB>& r,
                                             const QOps& Q, float sl2, int wave, int lane) {
    using R = UnitRaw<G, KB, VB>;
    constexpr int SPT = R::SPT;
    const int g = lane >> 4;
    const bool lo_limb = LP && (lane & 8);
    // stage the records' scale/zero tables
#pragma unroll
    for (int i = 0; i < R::NR; ++i) {
        *(uint2*)&sm.kmeta[wave][i][2 * lane] = r.km[i];
        if (lane < G / 4) *(uint4*)&sm.vmeta[wave][i][4 * lane] = r.vm[i];
    }
    wave_sync();

    // Key side: accumulators start from sum_c z[c] q[c][head] (every row; LP:
    // high-limb columns only), then add codes . (q s) with q s split exactly
    // into fp16 high and low parts (LP: the part of the lane's column).
    f4 C[2];
#pragma unroll
    for (int i = 0; i < R::NR; ++i) {
        const uint4* km = (const uint4*)&sm.kmeta[wave][i][0];
        f4 cz = f4{0.0f, 0.0f, 0.0f, 0.0f};
        h8 qhi[4], qlo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h8 s = words_h8(km[4 * g + j]);
            const h8 z = words_h8(km[16 + 4 * g + j]);
            cz = mfma(z, Q.q[j], cz);
            {
#pragma clang fp contract(off)
                const h8 hi = Q.q[j] * s;
                const h8 lo = __builtin_elementwise_fma(Q.q[j], s, -hi);
                qhi[j] = LP ? (lo_limb ? lo : hi) : hi;
                qlo[j] = lo;
            }
        }
        if (LP && lo_limb) cz = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (R::NR == 2 && rt != i) continue;
            f4 acc = cz;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 a = codes8<KB>(r.kc[rt], j);
                acc = mfma(a, qhi[j], acc);
                if (!LP) acc = mfma(a, qlo[j], acc);
            }
            C[rt] = acc;
        }
    }

    // value scale/zero of the lane's 8 slots: slot k = 4*rt + i <-> token 16rt + 4g + i
    float x[8], vs[8], vz[8];
    bool valid[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int rec = R::NR == 2 ? rt : 0;
        const uint16_t* vm = (const uint16_t*)&sm.vmeta[wave][rec][0] + g * 2 * SPT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 4 * rt + i;
            const int slot = R::NR == 2 ? i : k;
            x[k] = LP ? add_limb_partner(C[rt][i]) : C[rt][i];
            vs[k] = h2f(vm[slot]);
            vz[k] = h2f(vm[SPT + slot]);
            valid[k] = R::NR == 1 || r.has[rec];
        }
    }
    softmax_and_values<LP>(A, x, vs, vz, valid, sl2, lane, [&](int ct) -> h8 {
        if (R::NR == 1) return codes8<VB>(r.vc[0], ct);
        // G = 16: 4 slots of each record; code q = 4ct + slot
        const h8 a = codes8<VB>(r.vc[0], ct >> 1);
        const h8 b = codes8<VB>(r.vc[1], ct >> 1);
        const int o = 4 * (ct & 1);
        return h8{a[o], a[o + 1], a[o + 2], a[o + 3], b[o], b[o + 1], b[o + 2], b[o + 3]};
    });
    wave_sync();   // LDS meta slots are rewritten by the next unit
}

// One 32-token unit of the fp16 residual ring: tokens t0 .. t0+31 (< n).
// Keys and query are exact fp16, so the key product needs one part (LP: the
// high-limb columns carry it, the low-limb columns add zero).
template <bool LP>
__device__ __forceinline__ void process_residual(WaveAcc& A, const Layout& L, const kvq_cache& c, long sh, int t0,
                                                 int n, const QOps& Q, float sl2, int lane) {
    const int g = lane >> 4, n16 = lane & 15;
    const half_t* kr = (const half_t*)c.k_res + sh * L.ring * kD;
    const half_t* vr = (const half_t*)c.v_res + sh * L.ring * kD;
    f4 C[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int t = t0 + 16 * rt + n16;
        f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t keep = t < n ? 0xffffffffu : 0u;
        const uint4* row = (const uint4*)(kr + (long)((t < n ? t : t0) % L.ring) * kD + 32 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 w = row[j];
            w.x &= keep; w.y &= keep; w.z &= keep; w.w &= keep;
            acc = mfma(words_h8(w), Q.q[j], acc);
        }
        C[rt] = LP && (lane & 8) ? f4{0.0f, 0.0f, 0.0f, 0.0f} : acc;
    }
    float x[8], vs[8], vz[8];
    bool valid[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        x[k] = LP ? add_limb_partner(C[k >> 2][k & 3]) : C[k >> 2][k & 3];
        vs[k] = 1.0f;
        vz[k] = 0.0f;
        valid[k] = t0 + (k >> 2) * 16 + 4 * g + (k & 3) < n;
    }
    softmax_and_values<LP>(A, x, vs, vz, valid, sl2, lane, [&](int ct) -> h8 {
        h8 b;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = t0 + (k >> 2) * 16 + 4 * g + (k & 3);
            const _Float16 x = vr[(long)((t < n ? t : t0) % L.ring) * kD + 16 * ct + n16];
            b[k] = t < n ? x : (_Float16)0.0f;
        }
        return b;
    });
}

template <int G, int KB, int VB, bool LP>
__global__ __launch_bounds__(256) void attn_kernel(Layout L, kvq_cache c, const half_t* __restrict__ q,
                                                   float sl2, float* __restrict__ ws,
                                                   int gq, int splits, int ups) {
    __shared__ AttnSmem<G> sm;
    const int sp = blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int g = lane >> 4, n16 = lane & 15;
    // counters written by this library satisfy 0 <= nq <= n <= nq + ring; clamp
    // so that no other value can index outside the records or the ring
    const int nq = max(c.n_quant[b], 0);
    const int n = min(max(c.n_tokens[b], nq), nq + L.ring);
    const int Hq = L.H * gq;
    const int parts = splits;

    QOps Q;
    {
        // column n: head n (LP: head n%8, high limb for n < 8, low limb above)
        const int hd = LP ? (n16 & 7) : n16;
        const bool hv = hd < gq;
        const uint4* qp = (const uint4*)(q + ((long)b * Hq + h * gq + (hv ? hd : 0)) * kD + 32 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) Q.q[j] = words_h8(hv ? qp[j] : make_uint4(0, 0, 0, 0));
    }
    WaveAcc A;
    acc_init(A);

    // Units of this stream: the quantized ones first, then the 32-token units
    // of the fp16 residual ring; split sp takes units [sp*ups, sp*ups + ups).
    const int ngroups = nq / L.G;
    const int uq = (ngroups * L.G + 31) / 32;
    const int units = uq + (n - nq + 31) / 32;
    const int u0 = sp * ups, u1 = min(u0 + ups, units);
    {
        const int q1 = min(u1, uq);
        int u = u0 + wave;
        if (u < q1) {
            UnitRaw<G, KB, VB> ra, rb;
            load_unit(ra, L, c, b, h, u, ngroups, lane);
            for (;;) {
                load_unit(rb, L, c, b, h, u + kWaves < q1 ? u + kWaves : u, ngroups, lane);
                process_unit<G, KB, VB, LP>(sm, A, ra, Q, sl2, wave, lane);
                u += kWaves;
                if (u >= q1) break;
                load_unit(ra, L, c, b, h, u + kWaves < q1 ? u + kWaves : u, ngroups, lane);
                process_unit<G, KB, VB, LP>(sm, A, rb, Q, sl2, wave, lane);
                u += kWaves;
                if (u >= q1) break;
            }
        }
    }
    for (int u = u0 + wave; u < u1; u += kWaves)
        if (u >= uq) process_residual<LP>(A, L, c, sh, nq + 32 * (u - uq), n, Q, sl2, lane);

    // Wave results -> LDS: totals over the lane groups, accumulators by head.
    const float lt = group_sum(A.l);
    const float pzt = group_sum(A.pz);
    if (lane < 16) {
        sm.wm[wave][lane] = A.m;
        sm.wl[wave][lane] = lt;
        sm.wpz[wave][lane] = pzt;
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.wacc[wave][4 * g + i][16 * ct + n16] = A.acc[ct][i];
    __syncthreads();

    // Workgroup partial (heads < gq) -> workspace.
    float* part = ws + ((long)sh * parts + sp) * gq * kPart;
    for (int idx = threadIdx.x; idx < gq * kD; idx += 256) {
        const int hh = idx >> 7, ch = idx & (kD - 1);
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][hh]);
        float o = 0.0f, Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm.wm[w][hh];
            const float f = mw == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            // LP: rows hh and hh+8 hold the high- and low-limb sums of head hh
            const float a = LP ? sm.wacc[w][hh][ch] + sm.wacc[w][hh + 8][ch] : sm.wacc[w][hh][ch];
            o += (a + sm.wpz[w][hh]) * f;
            Ls += sm.wl[w][hh] * f;
        }
        part[hh * kPart + ch] = o;
        if (ch == 0) {
            part[hh * kPart + kD] = M;
            part[hh * kPart + kD + 1] = Ls;
        }
    }
}

// Split merge: grid (B*H, gq), 1024 threads.  Log-sum-exp over the parts of
// one (stream, head): out = sum_p o_p e^(m_p-M) / sum_p l_p e^(m_p-M), 0 for
// an empty sequence.  Every load (outputs of up to 32 parts per thread, and
// the parts' max and sum) is issued before any is used: one memory round trip.
constexpr int kMaxParts = 256;
constexpr int kMergeThreads = 1024;
constexpr int kMergeSlices = kMergeThreads / kD;
constexpr int kMergePer = kMaxParts / kMergeSlices;
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float* __restrict__ ws,
                                                                  float* __restrict__ out, int parts, int gq) {
    __shared__ float fac[kMaxParts];
    __shared__ float red[kMergeThreads / 64][2];
    __shared__ float acc[kMergeSlices][kD];
    const int sh = blockIdx.x, hh = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int slice = tid >> 7, ch = tid & (kD - 1);
    const long stride = (long)gq * kPart;
    const float* p = ws + ((long)sh * parts * gq + hh) * kPart;
    float o[kMergePer];
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) {
        const int i = slice + j * kMergeSlices;
        o[j] = i < parts ? p[i * stride + ch] : 0.0f;
    }
    float m = kNegInf, l = 0.0f;
    if (tid < parts) {
        m = p[tid * stride + kD];
        l = p[tid * stride + kD + 1];
    }
    float M = m;
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0) red[wv][0] = M;
    __syncthreads();
    M = red[0][0];
    for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w][0]);
    const float f = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    if (tid < parts) fac[tid] = f;
    float Ls = l * f;
    for (int off = 32; off >= 1; off >>= 1) Ls += __shfl_xor(Ls, off);
    if (lane == 0) red[wv][1] = Ls;
    __syncthreads();
    Ls = 0.0f;
    for (int w = 0; w < kMergeThreads / 64; ++w) Ls += red[w][1];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) {
        const int i = slice + j * kMergeSlices;
        if (i < parts) sum = fmaf(o[j], fac[i], sum);
    }
    acc[slice][ch] = sum;
    __syncthreads();
    if (slice == 0) {
        float s = acc[0][ch];
        for (int k = 1; k < kMergeSlices; ++k) s += acc[k][ch];
        out[((long)sh * gq + hh) * kD + ch] = Ls > 0.0f ? s / Ls : 0.0f;
    }
}

// Resident attention workgroups on the current device: CUs x workgroups per
// CU for this instantiation (from its register and LDS footprint).  Falls
// back to 256 CUs x 3 when no device is visible (host-only size queries).
template <int G, int KB, int VB, bool LP>
static int attn_slots_for() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * 3;
    if (cached[dev]) return cached[dev];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)attn_kernel<G, KB, VB, LP>, 256, 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 3;
    (void)hipGetLastError();
    cached[dev] = cus * per_cu;
    return cached[dev];
}

// Limb packing: with at most 8 query heads per kv head, the high and low
// fp16 parts of q*s and p*s share one 16-column product.
static inline bool limb_packed(int gq) { return gq <= 8; }

template <bool LP>
static int attn_slots_lp(const Layout& L) {
    switch (L.G * 100 + L.kbits * 10 + L.vbits) {
        case 1622: return attn_slots_for<16, 2, 2, LP>();
        case 1624: return attn_slots_for<16, 2, 4, LP>();
        case 1642: return attn_slots_for<16, 4, 2, LP>();
        case 1644: return attn_slots_for<16, 4, 4, LP>();
        case 3222: return attn_slots_for<32, 2, 2, LP>();
        case 3224: return attn_slots_for<32, 2, 4, LP>();
        case 3242: return attn_slots_for<32, 4, 2, LP>();
        default: return attn_slots_for<32, 4, 4, LP>();
    }
}
static int attn_slots(const Layout& L, int gq) {
    return limb_packed(gq) ? attn_slots_lp<true>(L) : attn_slots_lp<false>(L);
}

AttnPlan plan_attention(const Layout& L, int num_q_heads) {
    AttnPlan P;
    const int gq = num_q_heads / L.H;
    const int streams = L.B * L.H;
    const int maxg = L.paged ? L.max_blocks : L.groups;
    // 32-token units at capacity: quantized groups, then the residual ring
    const int maxu = (maxg * L.G + 31) / 32 + (L.R + L.G - 1 + 31) / 32;
    // One round of resident workgroups when the work allows it: all splits
    // are the same length, so a round with a partly filled tail is avoided.
    // At least one unit per wave, at most 128 units (32 per wave) per split.
    const int slots = attn_slots(L, gq);
    int splits = slots / streams;
    if (splits < 1) splits = 1;
    const int minsplit = (maxu + 3) / 4;
    if (splits > minsplit) splits = minsplit;
    int ups = (maxu + splits - 1) / splits;
    if (ups > 128) splits = (maxu + 127) / 128;
    if (const char* e = getenv("KVQ_UNITS_PER_SPLIT")) {
        const int v = atoi(e);
        if (v >= 1) splits = (maxu + v - 1) / v;
    }
    if (splits > kMaxParts) splits = kMaxParts;
    if (splits < 1) splits = 1;
    P.splits = splits;
    P.units_per_split = (maxu + splits - 1) / splits;
    P.parts = splits;
    P.part_floats = (size_t)gq * kPart;
    P.workspace = (size_t)streams * P.parts * P.part_floats * sizeof(float);
    return P;
}

hipError_t launch_attention_partials(const Layout& L, const AttnPlan& P, const kvq_cache& c, const half_t* q,
                                     int num_q_heads, float scale, void* ws, hipStream_t s) {
    const int gq = num_q_heads / L.H;
    const float sl2 = scale * kLog2e;
    dim3 grid(P.parts, L.B * L.H);
#define KVQ_ATT2(GG, KB, VB, LP)                                                                           \
    hipLaunchKernelGGL((attn_kernel<GG, KB, VB, LP>), grid, dim3(256), 0, s, L, c, q, sl2, (float*)ws, gq, \
                       P.splits, P.units_per_split)
#define KVQ_ATT(GG, KB, VB)              \
    if (limb_packed(gq))                  \
        KVQ_ATT2(GG, KB, VB, true);       \
    else                                  \
        KVQ_ATT2(GG, KB, VB, false)
    const int key = L.G * 100 + L.kbits * 10 + L.vbits;
    switch (key) {
        case 1622: KVQ_ATT(16, 2, 2); break;
        case 1624: KVQ_ATT(16, 2, 4); break;
        case 1642: KVQ_ATT(16, 4, 2); break;
        case 1644: KVQ_ATT(16, 4, 4); break;
        case 3222: KVQ_ATT(32, 2, 2); break;
        case 3224: KVQ_ATT(32, 2, 4); break;
        case 3242: KVQ_ATT(32, 4, 2); break;
        case 3244: KVQ_ATT(32, 4, 4); break;
        default: return hipErrorInvalidValue;
    }
#undef KVQ_ATT
#undef KVQ_ATT2
    return hipGetLastError();
}

hipError_t launch_attention_merge(const Layout& L, const AttnPlan& P, int num_q_heads, const void* ws, float* out,
                                  hipStream_t s) {
    const int gq = num_q_heads / L.H;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(L.B * L.H, gq), dim3(kMergeThreads), 0, s, (const float*)ws, out,
                       P.parts, gq);
    return hipGetLastError();
}

}  // namespace kvq
