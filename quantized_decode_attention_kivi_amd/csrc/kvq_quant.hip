// kvq_quant.hip -- quantize-prefill, append/flush, dequantize and code export
// kernels of libkvq (gfx950).
//
// Method ("KV cache compression: quantization, eviction and sparse attention",
// section 3.2; "KV cache compression" (jaedaily), formula paragraph; "KV Cache
// compression lab", experiment 01): keys are quantized per channel over each
// group of G tokens, values per token over their 128 channels, each set with
// its own min/max scale and zero; the newest R tokens stay fp16 and a group
// is quantized once it is full and outside them.
#include <type_traits>

#include "kvq_device.h"

namespace kvq {

// Shared memory of the codebook and dense-and-sparse quantizers (about 17 KB
// at G = 32).  The channel extremes of each token slice are kept as the fp16
// values they are: min and max are exact in any precision, and half the
// bytes of fp32 let more workgroups share a compute unit (24 -> 17 KB:
// dense-and-sparse 8B-layer prefill 490 -> 458 us).
template <int G>
struct QuantSmem {
    uint16_t kmn[16][kD], kmx[16][kD];   // per token slice, per channel: fp16 bits (exact: fp16
                                         // inputs, or infinities for kept extremes)
    float kz[kD], kinv[kD];
    uint8_t vcode[G][kD];             // value codes before packing
    int red[2][4];                    // dense-and-sparse: per-wave counts (double-buffered)
    uint32_t kept[G * kD / 32];       // dense-and-sparse: kept positions, one bit each
    uint32_t cand[8 * G];             // dense-and-sparse: each wave's candidates (2G slots per wave)
    int wtot[2];                      // dense-and-sparse: kept count of the first two words' waves
    uint2 cb4[240];                   // 4-bit codebook: per 1/16 of a grid step (threshold bits, code)
};

// Shared memory of the uniform-grid and 8-bit quantizers: the same fp16
// extremes without the codebook table and the selection's arrays (about
// 14 KB: eight workgroups fit a compute unit).
template <int G>
struct QuantSmemU {
    uint16_t kmn[16][kD], kmx[16][kD];   // per token slice, per channel (fp16 bits)
    float kz[kD], kinv[kD];
    uint8_t vcode[G][kD];                 // value codes before packing
    uint32_t vmeta[G];                    // image of the record's value scale/zero table
};

// Quantizer variants (compile-time): the 8-bit formats kFmtInt8 and kFmtFp8,
// and the low-bit format on the uniform grid (kQUniform), the codebook
// grid (kQCodebook), each with dense-and-sparse keys (kQSparse, kQCodebookSparse).
constexpr int kQUniform = 0, kQCodebook = 4, kQSparse = 6, kQCodebookSparse = 7;
__host__ __device__ constexpr bool q_low_bit(int F) { return F == kQUniform || F >= kQCodebook; }
// Shared memory of variant F.
template <int G, int F>
using QSmem = typename std::conditional<F == kQUniform || !q_low_bit(F), QuantSmemU<G>, QuantSmem<G>>::type;

// 16 bytes of a source row, read once: a non-temporal load.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once16(const half_t* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A record word written once (non-temporal store).
__device__ __forceinline__ void store_once(uint8_t* p, uint32_t w) { __builtin_nontemporal_store(w, (uint32_t*)p); }
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_once8(uint8_t* p, uint32_t a, uint32_t b) {
    __builtin_nontemporal_store(u32x2{a, b}, (u32x2*)p);
}

// Dense-and-sparse keys ("KV Cache compression lab", experiment 03: KVQuant
// keeps the few extreme keys in fp16 as a sparse matrix).  Marks in kbit[]
// the group's G entries of largest |x| (ties: lower position) and writes
// them, in ascending position order, as (position, fp16) pairs at `sparse`.
// Each entry's key ((|x| bits) << 12 | (4095 - position)) is unique, so a
// threshold found bit by bit from the top, by counting keys at or above each
// candidate, selects exactly G entries.  All 256 threads.
template <int G>
__device__ __forceinline__ void select_extremes(QuantSmem<G>& sm, const uint32_t (&kb)[G / 16][8],
                                                uint32_t (&kbit)[G / 16], const half_t* __restrict__ ksrc,
                                                uint32_t* __restrict__ sparse) {
    constexpr int NT = G / 16;
    const int tid = threadIdx.x, cg = tid & 15, ts = tid >> 4, lane = tid & 63, wave = tid >> 6;
    uint32_t key[NT][8];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            key[j][e] = ((kb[j][e] & 0x7fffu) << 12) | (4095u - (uint32_t)((ts + 16 * j) * kD + 8 * cg + e));
    // the kept-position words start empty (first read after the barriers below)
    for (int i = tid; i < G * kD / 32; i += 256) sm.kept[i] = 0;
    // The group's G largest keys are among the G largest of each wave's
    // quarter.  Each wave finds a threshold with between G and 2G of its keys
    // at or above it (counts by ballot: no barrier; the search stops at the
    // first candidate threshold in that range), writes those keys to its 2G
    // slots in LDS (zeros, below every key, in the rest), and the first wave
    // finds the G-th largest of the candidates, which is the group's.
    uint32_t Tw = 0;
    int nw = 0;
    for (int bit = 26; bit >= 0; --bit) {
        const uint32_t cand = Tw | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j][e] >= cand));
        if (cnt >= G) {
            Tw = cand;
            nw = cnt;
            if (cnt <= 2 * G) break;   // the wave's G largest, and at most G others
        }
    }
    // (the search always stops in the range: its last step up leaves exactly
    // G keys at or above, the keys being distinct; the slot bound below only
    // keeps the writes inside the wave's 2G slots)
    uint32_t* const cands = sm.cand + wave * 2 * G;
    int base = 0;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool up = key[j][e] >= Tw;
            const uint64_t m = __builtin_amdgcn_ballot_w64(up);
            const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (up && base + below < 2 * G) cands[base + below] = key[j][e];
            base += (int)__builtin_popcountll(m);
        }
    for (int i = min(nw, 2 * G) + lane; i < 2 * G; i += 64) cands[i] = 0u;
    __syncthreads();
    if (wave == 0) {
        constexpr int PL = 8 * G / 64;   // candidate slots per lane: 4 (G = 32) or 2
        uint32_t c[PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) c[i] = sm.cand[64 * i + lane];
        uint32_t T = 0;
        for (int bit = 26; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < PL; ++i) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c[i] >= cand));
            if (cnt >= G) {
                T = cand;
                if (cnt == G) break;   // exactly G at or above
            }
        }
        // the G-th largest candidate itself (the smallest of the G at or above
        // T), so that no key outside the candidates reaches the threshold
        uint32_t mn = 0xffffffffu;
#pragma unroll
        for (int i = 0; i < PL; ++i) mn = c[i] >= T ? min(mn, c[i]) : mn;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        if (lane == 0) sm.red[0][0] = (int)mn;
    }
    __syncthreads();
    const uint32_t T = (uint32_t)sm.red[0][0];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        kbit[j] = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (key[j][e] >= T) {
                kbit[j] |= 1u << e;
                const int pos = (ts + 16 * j) * kD + 8 * cg + e;
                atomicOr(&sm.kept[pos >> 5], 1u << (pos & 31));
            }
    }
    __syncthreads();
    // ordered compaction: word i covers positions 32i .. 32i + 31
    constexpr int W = G * kD / 32;   // 64 or 128 words: the first one or two waves
    const int mine = tid < W ? __builtin_popcount(sm.kept[tid]) : 0;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63 && wave < 2) sm.wtot[wave] = incl;
    __syncthreads();
    if (tid < W) {
        int idx = incl - mine + (wave == 1 ? sm.wtot[0] : 0);
        uint32_t w = sm.kept[tid];
        while (w) {
            const int b = __builtin_ctz(w);
            w &= w - 1;
            const int pos = 32 * tid + b;
            const uint32_t val = __builtin_bit_cast(uint16_t, ksrc[pos]);
            sparse[idx++] = (val << 16) | (uint32_t)pos;
        }
    }
}

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

// The 4-bit codebook code by table: t = (x - z) * inv falls in bin
// i = floor(16 t) (exact: a power-of-two scale), clamped to [0, 239]; the
// code counts the midpoints passed, which is the count at the bin's start
// plus at most one more (neighbouring midpoints are more than 1/16 of a
// step apart), passed when t exceeds the bin's threshold: the next midpoint
// m, or for a midpoint whose tie goes up (odd index, t >= m) the float just
// below it.  Equal to cb_code for every fp32 t.  Built by threads 0..239.
__device__ __forceinline__ void cb4_table(uint2 (&tab)[240], const float (&mid)[15], int tid) {
    if (tid < 240) {
        const float a = (float)tid * 0.0625f;
        const uint32_t lo = cb_code<15>(a, mid);
        uint32_t thr = 0x7f800000u;   // +inf: no midpoint left
        if (lo < 15) {
            const uint32_t mb = __builtin_bit_cast(uint32_t, mid[lo]);
            thr = (lo & 1) ? mb - 1 : mb;   // (mid > 0: the next float below is bits - 1)
        }
        tab[tid] = make_uint2(thr, lo);
    }
}
__device__ __forceinline__ uint32_t cb4_code(float x, float z, float inv, const uint2 (&tab)[240]) {
#pragma clang fp contract(off)
    const float t = (x - z) * inv;
    const int i = min(max((int)(t * 16.0f), 0), 239);
    const uint2 e = tab[i];
    return e.y + (t > __builtin_bit_cast(float, e.x) ? 1u : 0u);
}

// Quantize G consecutive fp16 rows of keys (ksrc) and values (vsrc) into one
// record.  Called by all 256 threads of a workgroup.  Thread (ts = tid/16,
// cg = tid%16) holds channels 8cg..8cg+7 of tokens ts, ts+16, ...  CB: the
// normal-quantile codebook grid instead of the uniform one.
template <int G, int KB, int VB, bool CB, bool SP>
__device__ void quantize_group(QuantSmem<G>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                               const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec) {
    constexpr int NT = G / 16;
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;

    float kx[NT][8], vx[NT][8];
    uint32_t kraw[NT][8];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        const uint4 a = load_once16(ksrc + t * kD + 8 * cg);
        const uint4 b = load_once16(vsrc + t * kD + 8 * cg);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kraw[j][2 * e] = aw[e] & 0xffffu;
            kraw[j][2 * e + 1] = aw[e] >> 16;
            kx[j][2 * e] = h2f(aw[e] & 0xffffu);
            kx[j][2 * e + 1] = h2f(aw[e] >> 16);
            vx[j][2 * e] = h2f(bw[e] & 0xffffu);
            vx[j][2 * e + 1] = h2f(bw[e] >> 16);
        }
    }
    // 4-bit codebook: its bin table (read after the barriers below)
    if constexpr (CB && (KB == 4 || VB == 4)) cb4_table(sm.cb4, KB == 4 ? L.kmid : L.vmid, tid);
    // dense-and-sparse: the kept extremes leave the channels' ranges
    uint32_t kbit[NT] = {};
    if constexpr (SP) select_extremes<G>(sm, kraw, kbit, ksrc, (uint32_t*)(rec + L.sparse_off));

    // Key statistics: per channel over the G tokens (without kept extremes).
    constexpr float kInf = __builtin_huge_valf();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float mn = kInf, mx = -kInf;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const bool k = SP && ((kbit[j] >> e) & 1);
            mn = fminf(mn, k ? kInf : kx[j][e]);
            mx = fmaxf(mx, k ? -kInf : kx[j][e]);
        }
        sm.kmn[ts][8 * cg + e] = __builtin_bit_cast(uint16_t, (_Float16)mn);
        sm.kmx[ts][8 * cg + e] = __builtin_bit_cast(uint16_t, (_Float16)mx);
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
        float mn = h2f(sm.kmn[0][tid]), mx = h2f(sm.kmx[0][tid]);
        for (int j = 1; j < 16; ++j) {
            mn = fminf(mn, h2f(sm.kmn[j][tid]));
            mx = fmaxf(mx, h2f(sm.kmx[j][tid]));
        }
        if (mn > mx) mn = mx = 0.0f;   // every value of the channel kept: s = z = 0
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
            const uint32_t q = SP && ((kbit[j] >> e) & 1) ? 0u
                               : CB && KB == 4 ? cb4_code(kx[j][e], kzr[e], kir[e], sm.cb4)
                                               : code_of<CB, KB>(kx[j][e], kzr[e], kir[e], L.kmid);
            w |= q << (KB == 4 ? code_bit(4, e) : code_bit(2, e + 8 * (cg & 1)));
        }
        if (KB == 4) {
            store_once(rec + t * 64 + 4 * cg, w);
        } else {
            w |= __shfl_xor(w, 1);
            if ((cg & 1) == 0) store_once(rec + t * 32 + 2 * cg, w);
        }
        // value codes of the same token into LDS, channel order
        uint32_t v0 = 0, v1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (CB && VB == 4) {
                v0 |= cb4_code(vx[j][e], pv[j].z, pv[j].inv, sm.cb4) << (8 * e);
                v1 |= cb4_code(vx[j][e + 4], pv[j].z, pv[j].inv, sm.cb4) << (8 * e);
            } else {
                v0 |= code_of<CB, VB>(vx[j][e], pv[j].z, pv[j].inv, L.vmid) << (8 * e);
                v1 |= code_of<CB, VB>(vx[j][e + 4], pv[j].z, pv[j].inv, L.vmid) << (8 * e);
            }
        }
        *(uint2*)&sm.vcode[t][8 * cg] = make_uint2(v0, v1);
    }
    __syncthreads();

    // Value code words, lane-major in decode-operand order.
    constexpr int SPT = G == 16 ? 4 : 8;
    constexpr int WPL = SPT * VB / 4;        // words per lane
    constexpr int CPW = 32 / VB;             // codes per word
    for (int D = tid; D < 64 * WPL; D += 256) {
        // (lanes over 32 bytes: D runs chunk-major, so writes follow the layout)
        const int lane = WPL > 8 ? (D >> 2) & 63 : D / WPL;
        const int wi = WPL > 8 ? 4 * (D >> 8) + (D & 3) : D % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < CPW; ++e) {
            const int q = wi * CPW + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = (slot >> 2) * 16 + 4 * g + (slot & 3);
            w |= (uint32_t)sm.vcode[t][16 * ct + n] << code_bit(VB, e);
        }
        store_once(rec + L.vcode_off + vlane_byte(SPT * VB, lane, 4 * wi), w);
    }
    __syncthreads();  // LDS may be reused by the caller
}

// The uniform grid without kept keys (the plain method), written for the
// vector ALU's issue budget: the same codes, scales and zeros as
// quantize_group, with fewer instructions per element.
//  - x - z is one mixed-precision fma, x * 1 + (-z), reading x straight from
//    its fp16 half: one rounding, exactly (float)x - z.
//  - t = (x - z) * inv clamped to [0, Q], then v_cvt_pk_u8_f32 rounds it to
//    the nearest integer, ties to even (the conversion follows the default
//    round-to-nearest-even mode and saturates to [0, 255]; the GPU parity
//    tests put keys and values on exact ties at every bit width), and drops
//    it into its byte of a word: clamping before
//    rounding gives the same integer as clamp(rint(t), 0, Q), since 0 and Q
//    are integers and rounding is monotonic.  Code words are assembled
//    from those byte words (code_bit: INT4 codes 0-3 are bytes 0-3 and codes
//    4-7 the same bytes' high nibbles; INT2 codes 0-7 are nibbles 0-7, even
//    codes in low nibbles, and codes 8-15 the same nibbles shifted by 2).
//  - value extremes: packed fp16 min/max over the thread's 8 channels, then
//    the 16 lanes of a row by DPP (quad swaps, half-row and row mirrors).
template <int HI>
__device__ __forceinline__ float minus_z(uint32_t w, float nz) {
    float r;
    if (HI) asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(nz));
    else asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(nz));
    return r;
}

// Code of the fp16 half HI of w as a byte of `acc` (byte `pos`).
template <int HI>
__device__ __forceinline__ uint32_t code_byte(uint32_t w, float nz, float inv, float qmax, int pos, uint32_t acc) {
#pragma clang fp contract(off)
    const float t = minus_z<HI>(w, nz) * inv;
    return __builtin_amdgcn_cvt_pk_u8_f32(fminf(fmaxf(t, 0.0f), qmax), pos, acc);
}

// The same with the byte conversion's saturation to [0, 255] as the clamp
// (8-bit codes).
template <int HI>
__device__ __forceinline__ uint32_t code_byte_sat(uint32_t w, float nz, float inv, int pos, uint32_t acc) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_cvt_pk_u8_f32(minus_z<HI>(w, nz) * inv, pos, acc);
}

typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(hh2, a), __builtin_bit_cast(hh2, b)));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(hh2, a), __builtin_bit_cast(hh2, b)));
}

// Min (MAX = false) or max over the 16 lanes of each row.
template <bool MAX, int CTRL>
__device__ __forceinline__ float row_step(float x) {
    const float y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf,
                                                                        0xf, false));
    return MAX ? fmaxf(x, y) : fminf(x, y);
}
template <bool MAX>
__device__ __forceinline__ float row16(float x) {
    x = row_step<MAX, 0xB1>(x);    // quad_perm [1,0,3,2]
    x = row_step<MAX, 0x4E>(x);    // quad_perm [2,3,0,1]
    x = row_step<MAX, 0x141>(x);   // row_half_mirror
    return row_step<MAX, 0x140>(x);   // row_mirror
}

template <int G, int KB, int VB>
__device__ void quantize_group_uniform(QuantSmemU<G>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                                       const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec) {
    constexpr int NT = G / 16;
    // Metadata stores: with INT2 keys, non-temporal, the value table written
    // as whole words from an LDS image; with INT4 keys, plain stores from the
    // lanes that compute them (each the faster choice in same-box timing of
    // the two layouts).
    constexpr bool kMetaOnce = KB == 2;
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;

    uint32_t kw[NT][4], vw[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        const uint4 a = load_once16(ksrc + t * kD + 8 * cg);
        const uint4 b = load_once16(vsrc + t * kD + 8 * cg);
        kw[j][0] = a.x; kw[j][1] = a.y; kw[j][2] = a.z; kw[j][3] = a.w;
        vw[j][0] = b.x; vw[j][1] = b.y; vw[j][2] = b.z; vw[j][3] = b.w;
    }

    // Key statistics: per channel over the thread's tokens (packed fp16),
    // then over the 16 token slices.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t mn = kw[0][i], mx = kw[0][i];
#pragma unroll
        for (int j = 1; j < NT; ++j) {
            mn = pk_min(mn, kw[j][i]);
            mx = pk_max(mx, kw[j][i]);
        }
        *(uint32_t*)&sm.kmn[ts][8 * cg + 2 * i] = mn;
        *(uint32_t*)&sm.kmx[ts][8 * cg + 2 * i] = mx;
    }

    // Value statistics and codes: per token over its 128 channels.
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const uint32_t m2 = pk_min(pk_min(vw[j][0], vw[j][1]), pk_min(vw[j][2], vw[j][3]));
        const uint32_t x2 = pk_max(pk_max(vw[j][0], vw[j][1]), pk_max(vw[j][2], vw[j][3]));
        const float mn = row16<false>(fminf(h2f(m2 & 0xffffu), h2f(m2 >> 16)));
        const float mx = row16<true>(fmaxf(h2f(x2 & 0xffffu), h2f(x2 >> 16)));
        const QParams p = make_qparams(mn, mx, VB);
        const int t = ts + 16 * j;
        if (cg == 0) {
            const int pos = vmeta_pos(L, t);
            if constexpr (kMetaOnce) {   // into the table's image; written out whole below
                uint16_t* img = (uint16_t*)sm.vmeta;
                img[(pos - L.vmeta_off) / 2] = p.s_bits;
                img[(pos - L.vmeta_off) / 2 + L.spt] = p.z_bits;
            } else {
                *(uint16_t*)(rec + pos) = p.s_bits;
                *(uint16_t*)(rec + pos + 2 * L.spt) = p.z_bits;
            }
        }
        const float nz = -p.z, qv = (float)((1 << VB) - 1);
        uint32_t v0 = 0, v1 = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            v0 = code_byte<0>(vw[j][i], nz, p.inv, qv, 2 * i, v0);
            v0 = code_byte<1>(vw[j][i], nz, p.inv, qv, 2 * i + 1, v0);
            v1 = code_byte<0>(vw[j][i + 2], nz, p.inv, qv, 2 * i, v1);
            v1 = code_byte<1>(vw[j][i + 2], nz, p.inv, qv, 2 * i + 1, v1);
        }
        *(uint2*)&sm.vcode[t][8 * cg] = make_uint2(v0, v1);
    }
    __syncthreads();
    if (tid < kD) {
        float mn = h2f(sm.kmn[0][tid]), mx = h2f(sm.kmx[0][tid]);
        for (int j = 1; j < 16; ++j) {
            mn = fminf(mn, h2f(sm.kmn[j][tid]));
            mx = fmaxf(mx, h2f(sm.kmx[j][tid]));
        }
        const QParams p = make_qparams(mn, mx, KB);
        sm.kz[tid] = -p.z;   // (negated: the fma's addend)
        sm.kinv[tid] = p.inv;
        if constexpr (kMetaOnce) {
            __builtin_nontemporal_store(p.s_bits, (uint16_t*)(rec + L.kmeta_off + 2 * tid));
            __builtin_nontemporal_store(p.z_bits, (uint16_t*)(rec + L.kmeta_off + 2 * kD + 2 * tid));
        } else {
            *(uint16_t*)(rec + L.kmeta_off + 2 * tid) = p.s_bits;
            *(uint16_t*)(rec + L.kmeta_off + 2 * kD + 2 * tid) = p.z_bits;
        }
    } else if (kMetaOnce && tid < kD + G) {
        __builtin_nontemporal_store(sm.vmeta[tid - kD], (uint32_t*)(rec + L.vmeta_off) + (tid - kD));
    }
    __syncthreads();

    // Key codes: channels 8cg .. 8cg+7 of the thread's tokens.
    float nzr[8], kir[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        nzr[e] = sm.kz[8 * cg + e];
        kir[e] = sm.kinv[8 * cg + e];
    }
    const float qk = (float)((1 << KB) - 1);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        if (KB == 4) {
            // bytes of codes 0-3 (channel pairs of words 0, 1) and 4-7 (words 2, 3)
            uint32_t a = 0, b = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a = code_byte<0>(kw[j][i], nzr[2 * i], kir[2 * i], qk, 2 * i, a);
                a = code_byte<1>(kw[j][i], nzr[2 * i + 1], kir[2 * i + 1], qk, 2 * i + 1, a);
                b = code_byte<0>(kw[j][i + 2], nzr[2 * i + 4], kir[2 * i + 4], qk, 2 * i, b);
                b = code_byte<1>(kw[j][i + 2], nzr[2 * i + 5], kir[2 * i + 5], qk, 2 * i + 1, b);
            }
            store_once(rec + t * 64 + 4 * cg, a | (b << 4));
        } else {
            // even codes (channel 2i: low halves) and odd codes (high halves),
            // nibble e of the half word; this thread's 8 codes are codes
            // 8 (cg & 1) .. of the word shared with its neighbour
            uint32_t ev = 0, od = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ev = code_byte<0>(kw[j][i], nzr[2 * i], kir[2 * i], qk, i, ev);
                od = code_byte<1>(kw[j][i], nzr[2 * i + 1], kir[2 * i + 1], qk, i, od);
            }
            uint32_t w = (ev | (od << 4)) << (2 * (cg & 1));
            w |= __shfl_xor(w, 1);
            if ((cg & 1) == 0) store_once(rec + t * 32 + 2 * cg, w);
        }
    }
    __syncthreads();

    // Value code words, lane-major in decode-operand order.
    constexpr int SPT = G == 16 ? 4 : 8;
    constexpr int WPL = SPT * VB / 4;        // words per lane
    constexpr int CPW = 32 / VB;             // codes per word
    for (int D = tid; D < 64 * WPL; D += 256) {
        // (lanes over 32 bytes: D runs chunk-major, so writes follow the layout)
        const int lane = WPL > 8 ? (D >> 2) & 63 : D / WPL;
        const int wi = WPL > 8 ? 4 * (D >> 8) + (D & 3) : D % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < CPW; ++e) {
            const int q = wi * CPW + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = (slot >> 2) * 16 + 4 * g + (slot & 3);
            w |= (uint32_t)sm.vcode[t][16 * ct + n] << code_bit(VB, e);
        }
        store_once(rec + L.vcode_off + vlane_byte(SPT * VB, lane, 4 * wi), w);
    }
    __syncthreads();  // LDS may be reused by the caller
}

// Two consecutive 16-token records of one stream on the uniform grid in one
// workgroup (bulk quantization of G = 16 layouts): the same arithmetic as
// quantize_group_uniform, record by record, with the per-record work (the
// 128 channel extremes and scales) spread over all four waves.  Thread
// (ts, cg) holds channels 8cg .. 8cg+7 of token ts of each record.  A null
// record pointer: that record is skipped (its rows are not read).
struct QuantSmemPair {
    uint16_t kmn[2][16][kD], kmx[2][16][kD];   // fp16 extremes per record, token, channel
    float kz[2][kD], kinv[2][kD];
    uint8_t vcode[32][kD];
};

template <int KB, int VB>
__device__ void quantize_pair16(QuantSmemPair& sm, const Layout& L, const half_t* __restrict__ ksrc,
                                const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec0,
                                uint8_t* __restrict__ rec1) {
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;
    uint8_t* const recs[2] = {rec0, rec1};

    uint32_t kw[2][4], vw[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = ts + 16 * j;
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (recs[j]) {
            a = load_once16(ksrc + t * kD + 8 * cg);
            b = load_once16(vsrc + t * kD + 8 * cg);
        }
        kw[j][0] = a.x; kw[j][1] = a.y; kw[j][2] = a.z; kw[j][3] = a.w;
        vw[j][0] = b.x; vw[j][1] = b.y; vw[j][2] = b.z; vw[j][3] = b.w;
        // key extremes: this token's values, reduced over the record's 16 tokens below
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(uint32_t*)&sm.kmn[j][ts][8 * cg + 2 * i] = kw[j][i];
            *(uint32_t*)&sm.kmx[j][ts][8 * cg + 2 * i] = kw[j][i];
        }
    }

    // Value statistics and codes: per token over its 128 channels.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t m2 = pk_min(pk_min(vw[j][0], vw[j][1]), pk_min(vw[j][2], vw[j][3]));
        const uint32_t x2 = pk_max(pk_max(vw[j][0], vw[j][1]), pk_max(vw[j][2], vw[j][3]));
        const float mn = row16<false>(fminf(h2f(m2 & 0xffffu), h2f(m2 >> 16)));
        const float mx = row16<true>(fmaxf(h2f(x2 & 0xffffu), h2f(x2 >> 16)));
        const QParams p = make_qparams(mn, mx, VB);
        if (cg == 0 && recs[j]) {
            const int pos = vmeta_pos(L, ts);
            *(uint16_t*)(recs[j] + pos) = p.s_bits;
            *(uint16_t*)(recs[j] + pos + 2 * L.spt) = p.z_bits;
        }
        const float nz = -p.z, qv = (float)((1 << VB) - 1);
        uint32_t v0 = 0, v1 = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            v0 = code_byte<0>(vw[j][i], nz, p.inv, qv, 2 * i, v0);
            v0 = code_byte<1>(vw[j][i], nz, p.inv, qv, 2 * i + 1, v0);
            v1 = code_byte<0>(vw[j][i + 2], nz, p.inv, qv, 2 * i, v1);
            v1 = code_byte<1>(vw[j][i + 2], nz, p.inv, qv, 2 * i + 1, v1);
        }
        *(uint2*)&sm.vcode[ts + 16 * j][8 * cg] = make_uint2(v0, v1);
    }
    __syncthreads();
    {
        // channel ch of record j: all four waves, one (record, channel) each
        const int j = tid >> 7, ch = tid & (kD - 1);
        // (reduced in fp32 in the single-record order: the same extremes)
        float mn = h2f(sm.kmn[j][0][ch]), mx = h2f(sm.kmx[j][0][ch]);
        for (int r = 1; r < 16; ++r) {
            mn = fminf(mn, h2f(sm.kmn[j][r][ch]));
            mx = fmaxf(mx, h2f(sm.kmx[j][r][ch]));
        }
        const QParams p = make_qparams(mn, mx, KB);
        sm.kz[j][ch] = -p.z;   // (negated: the fma's addend)
        sm.kinv[j][ch] = p.inv;
        if (recs[j]) {
            *(uint16_t*)(recs[j] + L.kmeta_off + 2 * ch) = p.s_bits;
            *(uint16_t*)(recs[j] + L.kmeta_off + 2 * kD + 2 * ch) = p.z_bits;
        }
    }
    __syncthreads();

    // Key codes: channels 8cg .. 8cg+7 of token ts of each record.
    const float qk = (float)((1 << KB) - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float nzr[8], kir[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            nzr[e] = sm.kz[j][8 * cg + e];
            kir[e] = sm.kinv[j][8 * cg + e];
        }
        if (KB == 4) {
            uint32_t a = 0, b = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a = code_byte<0>(kw[j][i], nzr[2 * i], kir[2 * i], qk, 2 * i, a);
                a = code_byte<1>(kw[j][i], nzr[2 * i + 1], kir[2 * i + 1], qk, 2 * i + 1, a);
                b = code_byte<0>(kw[j][i + 2], nzr[2 * i + 4], kir[2 * i + 4], qk, 2 * i, b);
                b = code_byte<1>(kw[j][i + 2], nzr[2 * i + 5], kir[2 * i + 5], qk, 2 * i + 1, b);
            }
            if (recs[j]) store_once(recs[j] + ts * 64 + 4 * cg, a | (b << 4));
        } else {
            uint32_t ev = 0, od = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ev = code_byte<0>(kw[j][i], nzr[2 * i], kir[2 * i], qk, i, ev);
                od = code_byte<1>(kw[j][i], nzr[2 * i + 1], kir[2 * i + 1], qk, i, od);
            }
            uint32_t w = (ev | (od << 4)) << (2 * (cg & 1));
            w |= __shfl_xor(w, 1);
            if ((cg & 1) == 0 && recs[j]) store_once(recs[j] + ts * 32 + 2 * cg, w);
        }
    }

    // Value code words of each record, lane-major in decode-operand order
    // (the codes of LDS rows 16j .. 16j+15).
    constexpr int SPT = 4;
    constexpr int WPL = SPT * VB / 4;        // words per lane
    constexpr int CPW = 32 / VB;             // codes per word
    for (int D = tid; D < 2 * 64 * WPL; D += 256) {
        const int j = D / (64 * WPL), Dj = D % (64 * WPL);
        const int lane = Dj / WPL, wi = Dj % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < CPW; ++e) {
            const int q = wi * CPW + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = 4 * g + slot;
            w |= (uint32_t)sm.vcode[16 * j + t][16 * ct + n] << code_bit(VB, e);
        }
        if (recs[j]) store_once(recs[j] + L.vcode_off + vlane_byte(SPT * VB, lane, 4 * wi), w);
    }
    __syncthreads();  // LDS may be reused by the caller
}

// Codebook grid at G = 16: two consecutive groups of a stream per workgroup,
// each thread holding channels 8cg..8cg+7 of token ts of both records (as
// quantize_group does for the two halves of a G = 32 group), so every thread
// quantizes 16 elements instead of 8 (8B-layer shape at G = 16: 416 -> 352
// us).  Each record gets exactly the bytes quantize_group<16> writes: the
// same reductions (min and max are exact in any order) and the same code
// arithmetic.  rec1 may be null (the stream's last group); its rows are then
// neither read nor written.  (With dense-and-sparse keys the two selections
// run one after the other and the pairing gained nothing: those keep one
// group per workgroup.)
struct QuantSmemPairG {
    uint16_t kmn[2][16][kD], kmx[2][16][kD];   // per record, token, channel: fp16 bits
    float kz[2][kD], kinv[2][kD];
    uint8_t vcode[32][kD];                     // value codes, rows 16j + ts
    uint2 cb4[240];                            // 4-bit codebook bin table
};

template <int KB, int VB>
__device__ void quantize_pair16cb(QuantSmemPairG& sm, const Layout& L, const half_t* __restrict__ ksrc,
                                 const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec0,
                                 uint8_t* __restrict__ rec1) {
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;
    uint8_t* const recs[2] = {rec0, rec1};

    float kx[2][8], vx[2][8];
    uint32_t kraw[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = ts + 16 * j;
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (recs[j]) {
            a = load_once16(ksrc + t * kD + 8 * cg);
            b = load_once16(vsrc + t * kD + 8 * cg);
        }
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kraw[j][2 * e] = aw[e] & 0xffffu;
            kraw[j][2 * e + 1] = aw[e] >> 16;
            kx[j][2 * e] = h2f(aw[e] & 0xffffu);
            kx[j][2 * e + 1] = h2f(aw[e] >> 16);
            vx[j][2 * e] = h2f(bw[e] & 0xffffu);
            vx[j][2 * e + 1] = h2f(bw[e] >> 16);
        }
    }
    if constexpr (KB == 4 || VB == 4) cb4_table(sm.cb4, KB == 4 ? L.kmid : L.vmid, tid);

    // Key statistics: this token's values per record, reduced over the
    // record's 16 tokens below.
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sm.kmn[j][ts][8 * cg + e] = (uint16_t)kraw[j][e];
            sm.kmx[j][ts][8 * cg + e] = (uint16_t)kraw[j][e];
        }

    // Value statistics: per token over its 128 channels (16 lanes of a row).
    QParams pv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
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
        if (cg == 0 && recs[j]) {
            const int pos = vmeta_pos(L, ts);
            *(uint16_t*)(recs[j] + pos) = pv[j].s_bits;
            *(uint16_t*)(recs[j] + pos + 2 * L.spt) = pv[j].z_bits;
        }
    }
    __syncthreads();
    {
        // channel ch of record j: all four waves, one (record, channel) each
        const int j = tid >> 7, ch = tid & (kD - 1);
        float mn = h2f(sm.kmn[j][0][ch]), mx = h2f(sm.kmx[j][0][ch]);
        for (int r = 1; r < 16; ++r) {
            mn = fminf(mn, h2f(sm.kmn[j][r][ch]));
            mx = fmaxf(mx, h2f(sm.kmx[j][r][ch]));
        }
        const QParams p = make_qparams(mn, mx, KB);
        sm.kz[j][ch] = p.z;
        sm.kinv[j][ch] = p.inv;
        if (recs[j]) {
            *(uint16_t*)(recs[j] + L.kmeta_off + 2 * ch) = p.s_bits;
            *(uint16_t*)(recs[j] + L.kmeta_off + 2 * kD + 2 * ch) = p.z_bits;
        }
    }
    __syncthreads();

    // Key codes (token ts of each record) and the value codes into LDS.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float kzr[8], kir[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kzr[e] = sm.kz[j][8 * cg + e];
            kir[e] = sm.kinv[j][8 * cg + e];
        }
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t q = KB == 4 ? cb4_code(kx[j][e], kzr[e], kir[e], sm.cb4)
                                       : code_of<true, KB>(kx[j][e], kzr[e], kir[e], L.kmid);
            w |= q << (KB == 4 ? code_bit(4, e) : code_bit(2, e + 8 * (cg & 1)));
        }
        if (KB == 4) {
            if (recs[j]) store_once(recs[j] + ts * 64 + 4 * cg, w);
        } else {
            w |= __shfl_xor(w, 1);
            if ((cg & 1) == 0 && recs[j]) store_once(recs[j] + ts * 32 + 2 * cg, w);
        }
        uint32_t v0 = 0, v1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (VB == 4) {
                v0 |= cb4_code(vx[j][e], pv[j].z, pv[j].inv, sm.cb4) << (8 * e);
                v1 |= cb4_code(vx[j][e + 4], pv[j].z, pv[j].inv, sm.cb4) << (8 * e);
            } else {
                v0 |= code_of<true, VB>(vx[j][e], pv[j].z, pv[j].inv, L.vmid) << (8 * e);
                v1 |= code_of<true, VB>(vx[j][e + 4], pv[j].z, pv[j].inv, L.vmid) << (8 * e);
            }
        }
        *(uint2*)&sm.vcode[16 * j + ts][8 * cg] = make_uint2(v0, v1);
    }
    __syncthreads();

    // Value code words of each record, lane-major in decode-operand order
    // (the codes of LDS rows 16j .. 16j+15).
    constexpr int SPT = 4;
    constexpr int WPL = SPT * VB / 4;        // words per lane
    constexpr int CPW = 32 / VB;             // codes per word
    for (int D = tid; D < 2 * 64 * WPL; D += 256) {
        const int j = D / (64 * WPL), Dj = D % (64 * WPL);
        const int lane = Dj / WPL, wi = Dj % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < CPW; ++e) {
            const int q = wi * CPW + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = 4 * g + slot;
            w |= (uint32_t)sm.vcode[16 * j + t][16 * ct + n] << code_bit(VB, e);
        }
        if (recs[j]) store_once(recs[j] + L.vcode_off + vlane_byte(SPT * VB, lane, 4 * wi), w);
    }
    __syncthreads();  // LDS may be reused by the caller
}

// The same for the 8-bit formats ("KV cache compression: ...", section 3.1):
// every key and value token on its own.  F = kFmtInt8: the min/max grid with
// 8 bits over the token's 128 channels (the 16 threads of a row reduce it);
// F = kFmtFp8: E4M3 codes under the kv head's static scales (inverses kinv,
// vinv).  Key bytes go straight to the record in channel order; value bytes
// through LDS into the lane-major operand order.  rows: tokens present (a
// partial group when quantized on write); the others are not read and are
// stored as zero tokens (codes 0, INT8 scale and zero 0).
template <int G, int F>
__device__ void quantize_group8(QuantSmemU<G>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                                const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec, float kinv,
                                float vinv, int rows) {
    constexpr int NT = G / 16;
    constexpr int SPT = G == 16 ? 4 : 8;
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = ts + 16 * j;
        const uint4 z4 = make_uint4(0, 0, 0, 0);
        const uint4 a = t < rows ? load_once16(ksrc + t * kD + 8 * cg) : z4;
        const uint4 b = t < rows ? load_once16(vsrc + t * kD + 8 * cg) : z4;
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t kw[2], vw[2];
        if (F == kFmtInt8) {
            // extremes of the token's 8 channels (packed fp16), then of its
            // row of 16 lanes
            const uint32_t km = pk_min(pk_min(aw[0], aw[1]), pk_min(aw[2], aw[3]));
            const uint32_t kM = pk_max(pk_max(aw[0], aw[1]), pk_max(aw[2], aw[3]));
            const uint32_t vm = pk_min(pk_min(bw[0], bw[1]), pk_min(bw[2], bw[3]));
            const uint32_t vM = pk_max(pk_max(bw[0], bw[1]), pk_max(bw[2], bw[3]));
            const float kmn = row16<false>(fminf(h2f(km & 0xffffu), h2f(km >> 16)));
            const float kmx = row16<true>(fmaxf(h2f(kM & 0xffffu), h2f(kM >> 16)));
            const float vmn = row16<false>(fminf(h2f(vm & 0xffffu), h2f(vm >> 16)));
            const float vmx = row16<true>(fmaxf(h2f(vM & 0xffffu), h2f(vM >> 16)));
            const QParams pk = make_qparams(kmn, kmx, 8);
            const QParams pv = make_qparams(vmn, vmx, 8);
            // codes: the byte conversion rounds to nearest even and saturates
            // to [0, 255], which is the clamp itself
            const float nk = -pk.z, nv = -pv.z;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kw[h] = vw[h] = 0;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    kw[h] = code_byte_sat<0>(aw[2 * h + i], nk, pk.inv, 2 * i, kw[h]);
                    kw[h] = code_byte_sat<1>(aw[2 * h + i], nk, pk.inv, 2 * i + 1, kw[h]);
                    vw[h] = code_byte_sat<0>(bw[2 * h + i], nv, pv.inv, 2 * i, vw[h]);
                    vw[h] = code_byte_sat<1>(bw[2 * h + i], nv, pv.inv, 2 * i + 1, vw[h]);
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
            float kx[8], vx[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kx[2 * e] = h2f(aw[e] & 0xffffu);
                kx[2 * e + 1] = h2f(aw[e] >> 16);
                vx[2 * e] = h2f(bw[e] & 0xffffu);
                vx[2 * e + 1] = h2f(bw[e] >> 16);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kw[h] = fp8_code2(kx[4 * h], kx[4 * h + 1], kinv) | fp8_code2(kx[4 * h + 2], kx[4 * h + 3], kinv) << 16;
                vw[h] = fp8_code2(vx[4 * h], vx[4 * h + 1], vinv) | fp8_code2(vx[4 * h + 2], vx[4 * h + 3], vinv) << 16;
            }
        }
        store_once8(rec + k8_byte(t, 8 * cg), kw[0], kw[1]);
        *(uint2*)&sm.vcode[t][8 * cg] = make_uint2(vw[0], vw[1]);
    }
    __syncthreads();

    // Value bytes, lane-major: lane l = 16g + n holds, at byte ct*SPT + slot
    // of its SPT*8 bytes, the code of channel 16ct + n for the slot's token.
    constexpr int WPL = SPT * 2;   // words per lane
    for (int D = tid; D < 64 * WPL; D += 256) {
        // (lanes over 32 bytes: D runs chunk-major, so writes follow the layout)
        const int lane = WPL > 8 ? (D >> 2) & 63 : D / WPL;
        const int wi = WPL > 8 ? 4 * (D >> 8) + (D & 3) : D % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = wi * 4 + e;
            const int ct = q / SPT, slot = q % SPT;
            const int t = (slot >> 2) * 16 + 4 * g + (slot & 3);
            w |= (uint32_t)sm.vcode[t][16 * ct + n] << (8 * e);
        }
        store_once(rec + L.vcode_off + vlane_byte(SPT * 8, lane, 4 * wi), w);
    }
    __syncthreads();  // LDS may be reused by the caller
}

// FP8 E4M3 at G = 16: two consecutive groups of a stream per workgroup, each
// thread holding channels 8cg..8cg+7 of token ts of both records, with the
// arithmetic of quantize_group8<16> (every token on its own, so each record
// gets exactly the bytes that one writes; 8B-layer shape at G = 16: 320 ->
// 272 us).  rows0, rows1: tokens present in each record (a partial last
// record when quantized on write); rec1 may be null.  (INT8 measured no
// faster this way and keeps one group per workgroup.)
__device__ void quantize_pair16_fp8(QuantSmemU<32>& sm, const Layout& L, const half_t* __restrict__ ksrc,
                                  const half_t* __restrict__ vsrc, uint8_t* __restrict__ rec0,
                                  uint8_t* __restrict__ rec1, float kinv, float vinv, int rows0, int rows1) {
    constexpr int SPT = 4;
    const int tid = threadIdx.x;
    const int cg = tid & 15;
    const int ts = tid >> 4;
    uint8_t* const recs[2] = {rec0, rec1};
    const int rows[2] = {rows0, rows1};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint8_t* const rec = recs[j];
        const int t = ts + 16 * j;   // row of the pair; token ts of record j
        const uint4 z4 = make_uint4(0, 0, 0, 0);
        const bool here = rec && ts < rows[j];
        const uint4 a = here ? load_once16(ksrc + t * kD + 8 * cg) : z4;
        const uint4 b = here ? load_once16(vsrc + t * kD + 8 * cg) : z4;
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t kw[2], vw[2];
        {
            float kx[8], vx[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kx[2 * e] = h2f(aw[e] & 0xffffu);
                kx[2 * e + 1] = h2f(aw[e] >> 16);
                vx[2 * e] = h2f(bw[e] & 0xffffu);
                vx[2 * e + 1] = h2f(bw[e] >> 16);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kw[h] = fp8_code2(kx[4 * h], kx[4 * h + 1], kinv) | fp8_code2(kx[4 * h + 2], kx[4 * h + 3], kinv) << 16;
                vw[h] = fp8_code2(vx[4 * h], vx[4 * h + 1], vinv) | fp8_code2(vx[4 * h + 2], vx[4 * h + 3], vinv) << 16;
            }
        }
        if (rec) store_once8(rec + k8_byte(ts, 8 * cg), kw[0], kw[1]);
        *(uint2*)&sm.vcode[t][8 * cg] = make_uint2(vw[0], vw[1]);
    }
    __syncthreads();

    // Value bytes of each record, lane-major (LDS rows 16j .. 16j+15).
    constexpr int WPL = SPT * 2;   // words per lane
    for (int D = tid; D < 2 * 64 * WPL; D += 256) {
        const int j = D / (64 * WPL), Dj = D % (64 * WPL);
        const int lane = Dj / WPL, wi = Dj % WPL;
        const int g = lane >> 4, n = lane & 15;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = wi * 4 + e;
            const int ct = q / SPT, slot = q % SPT;
            w |= (uint32_t)sm.vcode[16 * j + 4 * g + slot][16 * ct + n] << (8 * e);
        }
        if (recs[j]) store_once(recs[j] + L.vcode_off + vlane_byte(SPT * 8, lane, 4 * wi), w);
    }
    __syncthreads();  // LDS may be reused by the caller
}

// Variant of a layout (host).
inline int quant_variant(const Layout& L) {
    if (L.fmt != kFmtKivi) return L.fmt;
    const bool cb = L.grid == KVQ_GRID_NORMAL_QUANTILE;
    return L.sparse ? (cb ? kQCodebookSparse : kQSparse) : (cb ? kQCodebook : kQUniform);
}

// Quantizes one group in variant F (low-bit: key bits KB, value bits VB).
// rows: tokens of the group present (8-bit formats quantized on write; the
// low-bit formats always quantize whole groups).
template <int G, int KB, int VB, int F>
__device__ __forceinline__ void quantize_any(QSmem<G, F>& sm, const Layout& L, const kvq_cache& c, int h,
                                             const half_t* ksrc, const half_t* vsrc, uint8_t* rec, int rows = G) {
    if constexpr (F == kQUniform) {
        quantize_group_uniform<G, KB, VB>(sm, L, ksrc, vsrc, rec);
    } else if constexpr (q_low_bit(F)) {
        quantize_group<G, KB, VB, F == kQCodebook || F == kQCodebookSparse, F == kQSparse || F == kQCodebookSparse>(
            sm, L, ksrc, vsrc, rec);
    } else {
        const float kinv = F == kFmtFp8 ? fp8_inv_scale(c.k_scale[h]) : 0.0f;
        const float vinv = F == kFmtFp8 ? fp8_inv_scale(c.v_scale[h]) : 0.0f;
        quantize_group8<G, F>(sm, L, ksrc, vsrc, rec, kinv, vinv, rows);
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
    __shared__ QSmem<G, F> sm;
    const int g = blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = quantized_count(L, n);
    if (g * G >= nq) return;
    uint8_t* rec = record_at(L, c.packed, c.block_table, b, h, g);
    if (!rec) return;
    const long base = ((long)sh * max_len + (long)g * G) * kD;
    quantize_any<G, KB, VB, F>(sm, L, c, h, k + base, v + base, rec, min(G, nq - g * G));
}

// Uniform grid, G = 16: grid (ceil(max_len / 32), B*H); one workgroup per two
// consecutive groups of a stream.
template <int KB, int VB>
__global__ __launch_bounds__(256) void prefill_pairs16_kernel(Layout L, kvq_cache c, const half_t* k,
                                                              const half_t* v, int max_len,
                                                              const int32_t* seq_lens) {
    __shared__ QuantSmemPair sm;
    const int g = 2 * blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = num_quantized(n, 16, L.R);
    if (g * 16 >= nq) return;
    uint8_t* rec0 = record_at(L, c.packed, c.block_table, b, h, g);
    uint8_t* rec1 = (g + 1) * 16 < nq ? record_at(L, c.packed, c.block_table, b, h, g + 1) : nullptr;
    if (!rec0 && !rec1) return;
    const long base = ((long)sh * max_len + (long)g * 16) * kD;
    quantize_pair16<KB, VB>(sm, L, k + base, v + base, rec0, rec1);
}

// Codebook grid, G = 16: grid (ceil(max_len / 32), B*H); one workgroup per
// two consecutive groups of a stream.
template <int KB, int VB>
__global__ __launch_bounds__(256) void prefill_pairs16cb_kernel(Layout L, kvq_cache c, const half_t* k,
                                                                const half_t* v, int max_len,
                                                                const int32_t* seq_lens) {
    __shared__ QuantSmemPairG sm;
    const int g = 2 * blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = num_quantized(n, 16, L.R);
    if (g * 16 >= nq) return;
    uint8_t* rec0 = record_at(L, c.packed, c.block_table, b, h, g);
    uint8_t* rec1 = (g + 1) * 16 < nq ? record_at(L, c.packed, c.block_table, b, h, g + 1) : nullptr;
    if (!rec0 && !rec1) return;
    const long base = ((long)sh * max_len + (long)g * 16) * kD;
    quantize_pair16cb<KB, VB>(sm, L, k + base, v + base, rec0, rec1);
}

// FP8, G = 16: grid (ceil(max_len / 32), B*H); one workgroup per two
// consecutive groups of a stream.
__global__ __launch_bounds__(256) void prefill_pairs16_fp8_kernel(Layout L, kvq_cache c, const half_t* k,
                                                                  const half_t* v, int max_len,
                                                                  const int32_t* seq_lens) {
    __shared__ QuantSmemU<32> sm;
    const int g = 2 * blockIdx.x;
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = quantized_count(L, n);
    if (g * 16 >= nq) return;
    uint8_t* rec0 = record_at(L, c.packed, c.block_table, b, h, g);
    uint8_t* rec1 = (g + 1) * 16 < nq ? record_at(L, c.packed, c.block_table, b, h, g + 1) : nullptr;
    if (!rec0 && !rec1) return;
    const long base = ((long)sh * max_len + (long)g * 16) * kD;
    quantize_pair16_fp8(sm, L, k + base, v + base, rec0, rec1, fp8_inv_scale(c.k_scale[h]),
                        fp8_inv_scale(c.v_scale[h]), min(16, nq - g * 16), min(16, nq - (g + 1) * 16));
}

// Residual copy and counters: grid (B*H), 256 threads.
__global__ __launch_bounds__(256) void prefill_tail_kernel(Layout L, kvq_cache c, const half_t* k,
                                                           const half_t* v, int max_len,
                                                           const int32_t* seq_lens) {
    const int sh = blockIdx.x;
    const int b = sh / L.H, h = sh % L.H;
    const int n = clamped_len(L, seq_lens, b, max_len);
    const int nq = quantized_count(L, n);
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
        if (c.arrivals) c.arrivals[b] = 0;
    }
}

// ---------------------------------------------------------------------------
// Append one token per (sequence, head) and flush a full group: grid (B, H),
// then the counters: grid (ceil(B / 256)).
// ---------------------------------------------------------------------------

// State of sequence b before an append.  Counters written by this library
// satisfy 0 <= nq <= n, nq % G == 0 (quantize-on-write layouts: nq = n);
// anything else is treated as a full cache (nothing is written).  A flush
// happens when the new token brings the ring to R + G tokens: its oldest G
// leave the residual window.  On write, the new token goes straight into
// the record of group n / G, which must exist (write).
struct AppendState {
    int n, nq;
    bool room, flush, write;
};
__device__ __forceinline__ AppendState append_state(const Layout& L, const kvq_cache& c, int b) {
    AppendState a;
    a.n = c.n_tokens[b];
    a.nq = c.n_quant[b];
    if (L.onwrite) {
        a.room = a.n >= 0 && a.nq == a.n && a.n < L.capacity;
        a.flush = false;
        a.write = a.room && record_at(L, c.packed, c.block_table, b, 0, a.n / L.G) != nullptr;
        return a;
    }
    const bool sane = a.nq >= 0 && a.n >= a.nq && (a.nq % L.G) == 0;
    a.room = sane && (a.n - a.nq) < L.ring && a.n < L.capacity;
    a.flush = a.room && (a.n + 1 - a.nq == L.R + L.G);
    a.write = false;
    return a;
}

// Counters after an append in state a (the record of a flushed or written
// group exists for every head or for none).
__device__ __forceinline__ void advance_counters(const Layout& L, const kvq_cache& c, int b, const AppendState& a) {
    if (L.onwrite) {
        if (!a.write) return;   // no block for the token's group: nothing was appended
        c.n_tokens[b] = a.n + 1;
        c.n_quant[b] = a.n + 1;
        return;
    }
    const bool flushed = a.flush && record_at(L, c.packed, c.block_table, b, 0, a.nq / L.G) != nullptr;
    c.n_tokens[b] = a.n + 1;
    c.n_quant[b] = a.nq + (flushed ? L.G : 0);
}

// One token of an 8-bit format quantized into slot t of its group's record
// (quantize-on-write), by the 16 threads of one DPP row, thread cg holding
// channels 8cg .. 8cg+7: the same per-token arithmetic as quantize_group8.
template <int F>
__device__ void quantize_token8(const Layout& L, const half_t* __restrict__ krow, const half_t* __restrict__ vrow,
                                uint8_t* __restrict__ rec, int t, int cg, float kinv, float vinv) {
    const uint4 a = *(const uint4*)(krow + 8 * cg);
    const uint4 bb = *(const uint4*)(vrow + 8 * cg);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
    uint32_t kw[2], vw[2];
    if (F == kFmtInt8) {
        const uint32_t km = pk_min(pk_min(aw[0], aw[1]), pk_min(aw[2], aw[3]));
        const uint32_t kM = pk_max(pk_max(aw[0], aw[1]), pk_max(aw[2], aw[3]));
        const uint32_t vm = pk_min(pk_min(bw[0], bw[1]), pk_min(bw[2], bw[3]));
        const uint32_t vM = pk_max(pk_max(bw[0], bw[1]), pk_max(bw[2], bw[3]));
        const float kmn = row16<false>(fminf(h2f(km & 0xffffu), h2f(km >> 16)));
        const float kmx = row16<true>(fmaxf(h2f(kM & 0xffffu), h2f(kM >> 16)));
        const float vmn = row16<false>(fminf(h2f(vm & 0xffffu), h2f(vm >> 16)));
        const float vmx = row16<true>(fmaxf(h2f(vM & 0xffffu), h2f(vM >> 16)));
        const QParams pk = make_qparams(kmn, kmx, 8);
        const QParams pv = make_qparams(vmn, vmx, 8);
        const float nk = -pk.z, nv = -pv.z;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kw[h] = vw[h] = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                kw[h] = code_byte_sat<0>(aw[2 * h + i], nk, pk.inv, 2 * i, kw[h]);
                kw[h] = code_byte_sat<1>(aw[2 * h + i], nk, pk.inv, 2 * i + 1, kw[h]);
                vw[h] = code_byte_sat<0>(bw[2 * h + i], nv, pv.inv, 2 * i, vw[h]);
                vw[h] = code_byte_sat<1>(bw[2 * h + i], nv, pv.inv, 2 * i + 1, vw[h]);
            }
        }
        if (cg == 0) {
            const int kp = tmeta_pos(L, L.kmeta_off, t), vp = tmeta_pos(L, L.vmeta_off, t);
            *(uint16_t*)(rec + kp) = pk.s_bits;
            *(uint16_t*)(rec + kp + 2 * L.spt) = pk.z_bits;
            *(uint16_t*)(rec + vp) = pv.s_bits;
            *(uint16_t*)(rec + vp + 2 * L.spt) = pv.z_bits;
        }
    } else {
        float kx[8], vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kx[2 * e] = h2f(aw[e] & 0xffffu);
            kx[2 * e + 1] = h2f(aw[e] >> 16);
            vx[2 * e] = h2f(bw[e] & 0xffffu);
            vx[2 * e + 1] = h2f(bw[e] >> 16);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kw[h] = fp8_code2(kx[4 * h], kx[4 * h + 1], kinv) | fp8_code2(kx[4 * h + 2], kx[4 * h + 3], kinv) << 16;
            vw[h] = fp8_code2(vx[4 * h], vx[4 * h + 1], vinv) | fp8_code2(vx[4 * h + 2], vx[4 * h + 3], vinv) << 16;
        }
    }
    *(uint2*)(rec + k8_byte(t, 8 * cg)) = make_uint2(kw[0], kw[1]);
    // value bytes: each to its place in the lane-major operand layout
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int by, bi;
        vcode_pos(L, t, 8 * cg + e, &by, &bi);
        rec[by + bi / 8] = (uint8_t)(vw[e >> 2] >> (8 * (e & 3)));
    }
}

// Append: grid (B, H), one workgroup per (sequence, kv head), so the heads'
// flushes run side by side.  The new token goes into the ring; on a flush
// the oldest G ring tokens (the new one among them when R = 0) are quantized
// into the group's record.  Every head reads the counters first; they then
// advance (n + 1, and n_q + G when the group was flushed: it has a record,
// which exists for every head or for none) once all heads of the sequence
// have read them: with c.arrivals, by the last of the sequence's workgroups
// to arrive (an agent-scope atomic counter that it resets), else by
// append_counters_kernel after this kernel.
template <int G, int KB, int VB, int F>
__global__ __launch_bounds__(256) void append_kernel(Layout L, kvq_cache c, const half_t* knew,
                                                     const half_t* vnew) {
    __shared__ QSmem<G, F> sm;
    const int b = blockIdx.x, h = blockIdx.y;
    const AppendState a = append_state(L, c, b);
    if (!a.room) return;   // (the same for every head of b: none arrives)
    const long sh = (long)b * L.H + h;
    if constexpr (!q_low_bit(F)) {
        if (L.onwrite) {
            // quantize-on-write: the token goes straight into its group's
            // record; a group's first token finds the record cleared to zero
            // tokens first, so its unwritten slots read as zero codes
            uint8_t* rec = a.write ? record_at(L, c.packed, c.block_table, b, h, a.n / G) : nullptr;
            if (rec) {
                if (a.n % G == 0) {
                    for (int i = threadIdx.x; i < L.record / 16; i += 256)
                        ((uint4*)rec)[i] = make_uint4(0, 0, 0, 0);
                    __syncthreads();
                }
                if (threadIdx.x < 16) {
                    const float kinv = F == kFmtFp8 ? fp8_inv_scale(c.k_scale[h]) : 0.0f;
                    const float vinv = F == kFmtFp8 ? fp8_inv_scale(c.v_scale[h]) : 0.0f;
                    quantize_token8<F>(L, knew + sh * kD, vnew + sh * kD, rec, a.n % G, threadIdx.x, kinv, vinv);
                }
            }
        }
    }
    if (!L.onwrite) {
        if (threadIdx.x < 64) {
            const int slot = a.n % L.ring;
            ((uint32_t*)c.k_res)[(sh * L.ring + slot) * (kD / 2) + threadIdx.x] =
                ((const uint32_t*)knew)[sh * (kD / 2) + threadIdx.x];
            ((uint32_t*)c.v_res)[(sh * L.ring + slot) * (kD / 2) + threadIdx.x] =
                ((const uint32_t*)vnew)[sh * (kD / 2) + threadIdx.x];
        }
        uint8_t* rec = a.flush ? record_at(L, c.packed, c.block_table, b, h, a.nq / G) : nullptr;
        if (rec) {   // (no block for the group: the counters do not advance it either)
            __syncthreads();   // the new token's row is visible to the whole workgroup
            const long row = (sh * L.ring + (a.nq % L.ring)) * kD;
            quantize_any<G, KB, VB, F>(sm, L, c, h, (const half_t*)c.k_res + row, (const half_t*)c.v_res + row, rec);
        }
    }
    if (!c.arrivals) return;
    __syncthreads();   // every thread of this workgroup has read the counters
    if (threadIdx.x == 0) {
        // (relaxed: the other heads' counter reads completed before their
        // arrivals, and no data of theirs is read here)
        const int before = __hip_atomic_fetch_add(&c.arrivals[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == L.H - 1) {   // every head of b has read the counters
            __hip_atomic_store(&c.arrivals[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            advance_counters(L, c, b, a);
        }
    }
}

// Counters after an append without c.arrivals (one thread per sequence,
// after append_kernel): as above.
__global__ __launch_bounds__(256) void append_counters_kernel(Layout L, kvq_cache c) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= L.B) return;
    const AppendState a = append_state(L, c, b);
    if (!a.room) return;
    advance_counters(L, c, b, a);
}

// ---------------------------------------------------------------------------
// Dequantize / export: grid (out_tokens / 16, B*H), 256 threads, 16 tokens
// per block; thread -> token t = tid/16, channels (tid%16)*8 .. +8.
// ---------------------------------------------------------------------------

// Largest record of any format (INT8 at G = 32; at G = 16 two records of a
// 32-token block take the same bytes).
constexpr int kMaxRecordBytes = 8448;

// Value of key (token tg of the record, channel ch) from a record in LDS; the
// arithmetic of the quantizer's dequantization (one fma, or code times the
// static FP8 scale).
__device__ __forceinline__ float deq_key(const Layout& L, const kvq_cache& c, const uint8_t* rec, int h, int tg,
                                         int ch) {
    const uint32_t kcd = kcode_at(L, rec, tg, ch);
    if (L.fmt == kFmtFp8) {
#pragma clang fp contract(off)
        return fp8_value(kcd) * c.k_scale[h];
    }
    const bool tok = L.fmt == kFmtInt8;   // per-token key scale and zero
    const bool cb = L.grid == KVQ_GRID_NORMAL_QUANTILE;
    return fmaf(cb ? cb_level(L.klut, kcd, L.kbits) : (float)kcd,
                h2f(tok ? ktok_scale_bits(L, rec, tg) : kscale_bits(L, rec, ch)),
                h2f(tok ? ktok_zero_bits(L, rec, tg) : kzero_bits(L, rec, ch)));
}
__device__ __forceinline__ float deq_value(const Layout& L, const kvq_cache& c, const uint8_t* rec, int h, int tg,
                                           int ch) {
    const uint32_t vcd = vcode_at(L, rec, tg, ch);
    if (L.fmt == kFmtFp8) {
#pragma clang fp contract(off)
        return fp8_value(vcd) * c.v_scale[h];
    }
    const bool cb = L.grid == KVQ_GRID_NORMAL_QUANTILE;
    return fmaf(cb ? cb_level(L.vlut, vcd, L.vbits) : (float)vcd, h2f(vscale_bits(L, rec, tg)),
                h2f(vzero_bits(L, rec, tg)));
}

// kv_dequantize: 32 tokens of one stream per workgroup (grid
// (ceil(out_tokens / 32), B*H), 256 threads).  The records holding them
// (32 / G) are copied to LDS with 16-byte loads; then each thread writes 4
// consecutive channels of a token per 16-byte store, keys and values, 4 of
// each: quantized tokens from the records, ring tokens converted from fp16,
// zeros past the sequence's end.
// KB, VB, G, F, CB: the layout's bit widths, group size, format and grid,
// fixed at compile time (written into a copy of the layout, so that the
// position helpers fold to shifts and masks).
template <int KB, int VB, int G, int F, bool CB>
__global__ __launch_bounds__(256) void dequantize_kernel(Layout L, kvq_cache c, float* ko, float* vo,
                                                         int out_tokens) {
    L.kbits = KB;
    L.vbits = VB;
    L.G = G;
    L.spt = G == 16 ? 4 : 8;
    L.fmt = F;
    L.grid = CB ? KVQ_GRID_NORMAL_QUANTILE : KVQ_GRID_UNIFORM;
    __shared__ __align__(16) uint8_t srec[kMaxRecordBytes];
    const int sh = blockIdx.y;
    const int b = sh / L.H, h = sh % L.H;
    const int t0 = blockIdx.x * 32;
    const int tid = threadIdx.x;
    const int nq = max(c.n_quant[b], 0);
    const int n = min(max(c.n_tokens[b], nq), nq + L.ring);
    const int nr = 32 / L.G;
    uint32_t has = 0;
    for (int r = 0; r < nr; ++r) {
        const int tr = t0 + r * L.G;
        const uint8_t* rec = tr < nq ? record_at(L, c.packed, c.block_table, b, h, tr / L.G) : nullptr;
        if (!rec) continue;
        has |= 1u << r;
        uint4* dst = (uint4*)(srec + r * L.record);
        for (int i = tid; i < L.record / 16; i += 256) dst[i] = ((const uint4*)rec)[i];
    }
    __syncthreads();
#pragma unroll 1
    for (int side = 0; side < 2; ++side) {
        float* out = side ? vo : ko;
        const half_t* res = (const half_t*)(side ? c.v_res : c.k_res);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + 256 * k;   // (token, channel quad) of the block
            const int t = t0 + (idx >> 5), c4 = (idx & 31) * 4;
            if (t >= out_tokens) continue;
            float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (t < nq) {
                const int r = (t - t0) / L.G;
                if ((has >> r) & 1) {
                    const uint8_t* rec = srec + r * L.record;
                    const int tg = t % L.G;
                    float e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        e[i] = side ? deq_value(L, c, rec, h, tg, c4 + i) : deq_key(L, c, rec, h, tg, c4 + i);
                    o = make_float4(e[0], e[1], e[2], e[3]);
                }
            } else if (t < n) {
                const half_t* row = res + ((long)sh * L.ring + (t % L.ring)) * kD + c4;
                o = make_float4((float)row[0], (float)row[1], (float)row[2], (float)row[3]);
            }
            const u32x4 ob = u32x4{__float_as_uint(o.x), __float_as_uint(o.y), __float_as_uint(o.z),
                                   __float_as_uint(o.w)};
            __builtin_nontemporal_store(ob, (u32x4*)(out + ((long)sh * out_tokens + t) * kD + c4));
        }
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

// Dense-and-sparse keys: kept entries of group g of stream sh (grid
// (groups, B*H), G threads).  restore: write them over the dequantized keys;
// export: the logical (position, value) lists.
__global__ void restore_outliers_kernel(Layout L, kvq_cache c, float* ko, int out_tokens) {
    const int g = blockIdx.x, sh = blockIdx.y, e = threadIdx.x;
    const int b = sh / L.H, h = sh % L.H;
    const int nq = max(c.n_quant[b], 0);
    if ((g + 1) * L.G > nq || e >= L.G) return;
    const uint8_t* rec = record_at(L, c.packed, c.block_table, b, h, g);
    if (!rec) return;
    const uint32_t w = ((const uint32_t*)(rec + L.sparse_off))[e];
    const int pos = (int)(w & 0xffffu);
    const int t = g * L.G + (pos >> 7);
    if (pos < L.G * kD && t < out_tokens) ko[((long)sh * out_tokens + t) * kD + (pos & (kD - 1))] = h2f(w >> 16);
}

__global__ void export_outliers_kernel(Layout L, kvq_cache c, uint16_t* pos, uint16_t* val, int out_tokens) {
    const int g = blockIdx.x, sh = blockIdx.y, e = threadIdx.x;
    const int b = sh / L.H, h = sh % L.H;
    if (e >= L.G) return;
    const long o = ((long)sh * (out_tokens / L.G) + g) * L.G + e;
    const int nq = max(c.n_quant[b], 0);
    const uint8_t* rec = (g + 1) * L.G <= nq ? record_at(L, c.packed, c.block_table, b, h, g) : nullptr;
    const uint32_t w = rec ? ((const uint32_t*)(rec + L.sparse_off))[e] : 0u;
    pos[o] = (uint16_t)(w & 0xffffu);
    val[o] = (uint16_t)(w >> 16);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

#define KVQ_LOW_BIT_Q(F, Q)                                                                                   \
    case Q * 10000 + 1622: F(16, 2, 2, Q); break;                                                           \
    case Q * 10000 + 1624: F(16, 2, 4, Q); break;                                                           \
    case Q * 10000 + 1642: F(16, 4, 2, Q); break;                                                           \
    case Q * 10000 + 1644: F(16, 4, 4, Q); break;                                                           \
    case Q * 10000 + 3222: F(32, 2, 2, Q); break;                                                           \
    case Q * 10000 + 3224: F(32, 2, 4, Q); break;                                                           \
    case Q * 10000 + 3242: F(32, 4, 2, Q); break;                                                           \
    case Q * 10000 + 3244: F(32, 4, 4, Q); break;
#define KVQ_DISPATCH(L_, F)                                                                                    \
    do {                                                                                                       \
        switch (quant_variant(L_) * 10000 + (L_).G * 100 + (L_).kbits * 10 + (L_).vbits) {                    \
            KVQ_LOW_BIT_Q(F, kQUniform)                                                                        \
            KVQ_LOW_BIT_Q(F, kQCodebook)                                                                       \
            KVQ_LOW_BIT_Q(F, kQSparse)                                                                         \
            KVQ_LOW_BIT_Q(F, kQCodebookSparse)                                                                 \
            case 11688: F(16, 8, 8, kFmtInt8); break;                                                          \
            case 13288: F(32, 8, 8, kFmtInt8); break;                                                          \
            case 21688: F(16, 8, 8, kFmtFp8); break;                                                           \
            case 23288: F(32, 8, 8, kFmtFp8); break;                                                           \
            default: return hipErrorInvalidValue;                                                              \
        }                                                                                                      \
    } while (0)

hipError_t launch_prefill(const Layout& L, const kvq_cache& c, const half_t* k, const half_t* v,
                          int max_len, const int32_t* seq_lens, hipStream_t s) {
    const int ngroups = (max_len + L.G - 1) / L.G;
    if (ngroups > 0 && L.G == 16 && quant_variant(L) == kQUniform) {
        dim3 grid((ngroups + 1) / 2, L.B * L.H);
#define KVQ_PP(KB, VB)                                                                                      \
    hipLaunchKernelGGL((prefill_pairs16_kernel<KB, VB>), grid, dim3(256), 0, s, L, c, k, v, max_len, seq_lens)
        switch (L.kbits * 10 + L.vbits) {
            case 22: KVQ_PP(2, 2); break;
            case 24: KVQ_PP(2, 4); break;
            case 42: KVQ_PP(4, 2); break;
            case 44: KVQ_PP(4, 4); break;
            default: return hipErrorInvalidValue;
        }
#undef KVQ_PP
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (ngroups > 0 && L.G == 16 && L.fmt == kFmtFp8) {
        dim3 grid((ngroups + 1) / 2, L.B * L.H);
        hipLaunchKernelGGL(prefill_pairs16_fp8_kernel, grid, dim3(256), 0, s, L, c, k, v, max_len, seq_lens);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (ngroups > 0 && L.G == 16 && quant_variant(L) == kQCodebook) {
        dim3 grid((ngroups + 1) / 2, L.B * L.H);
#define KVQ_PC(KB, VB) \
    hipLaunchKernelGGL((prefill_pairs16cb_kernel<KB, VB>), grid, dim3(256), 0, s, L, c, k, v, max_len, seq_lens)
        switch (L.kbits * 10 + L.vbits) {
            case 22: KVQ_PC(2, 2); break;
            case 24: KVQ_PC(2, 4); break;
            case 42: KVQ_PC(4, 2); break;
            case 44: KVQ_PC(4, 4); break;
            default: return hipErrorInvalidValue;
        }
#undef KVQ_PC
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (ngroups > 0) {
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
    hipLaunchKernelGGL((append_kernel<GG, KB, VB, FF>), dim3(L.B, L.H), dim3(256), 0, s, L, c, k, v)
    KVQ_DISPATCH(L, KVQ_AP);
#undef KVQ_AP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!c.arrivals) hipLaunchKernelGGL(append_counters_kernel, dim3((L.B + 255) / 256), dim3(256), 0, s, L, c);
    return hipGetLastError();
}

hipError_t launch_dequantize(const Layout& L, const kvq_cache& c, float* ko, float* vo, int out_tokens,
                             hipStream_t s) {
    if (out_tokens <= 0) return hipSuccess;
    static_assert(kMaxRecordBytes % 16 == 0, "records are copied in 16-byte pieces");
    if (L.record > kMaxRecordBytes * L.G / 32) return hipErrorInvalidValue;
    dim3 grid((out_tokens + 31) / 32, L.B * L.H);
    const bool cb = L.grid == KVQ_GRID_NORMAL_QUANTILE;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, L, c, ko, vo, out_tokens); };
#define KVQ_DEQ_G(KB, VB, F, CB) \
    (L.G == 16 ? go(dequantize_kernel<KB, VB, 16, F, CB>) : go(dequantize_kernel<KB, VB, 32, F, CB>))
#define KVQ_DEQ_LOWBIT(KB, VB) (cb ? KVQ_DEQ_G(KB, VB, kFmtKivi, true) : KVQ_DEQ_G(KB, VB, kFmtKivi, false))
    if (L.fmt == kFmtInt8) KVQ_DEQ_G(8, 8, kFmtInt8, false);
    else if (L.fmt == kFmtFp8) KVQ_DEQ_G(8, 8, kFmtFp8, false);
    else if (L.kbits == 2 && L.vbits == 2) KVQ_DEQ_LOWBIT(2, 2);
    else if (L.kbits == 2) KVQ_DEQ_LOWBIT(2, 4);
    else if (L.vbits == 2) KVQ_DEQ_LOWBIT(4, 2);
    else KVQ_DEQ_LOWBIT(4, 4);
#undef KVQ_DEQ_LOWBIT
#undef KVQ_DEQ_G
    if (L.sparse) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(restore_outliers_kernel, dim3((out_tokens + L.G - 1) / L.G, L.B * L.H), dim3(L.G), 0, s, L,
                           c, ko, out_tokens);
    }
    return hipGetLastError();
}

hipError_t launch_export_outliers(const Layout& L, const kvq_cache& c, uint16_t* pos, uint16_t* val, int out_tokens,
                                  hipStream_t s) {
    if (out_tokens <= 0) return hipSuccess;
    hipLaunchKernelGGL(export_outliers_kernel, dim3(out_tokens / L.G, L.B * L.H), dim3(L.G), 0, s, L, c, pos, val,
                       out_tokens);
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
