// kvq_attn.hip -- decode attention: split planning, dispatch to the kernel
// families (instantiated in kvq_attn_*.hip) and the log-sum-exp merge
// kernels (gfx950).
#include "kvq_attn_impl.h"

namespace kvq {

KVQ_ALL_FAMILIES(KVQ_DECLARE_FAMILY)

// Workgroup w of nwg covers units [w T / nwg, (w + 1) T / nwg): empty when
// there are fewer units than workgroups; an empty one writes no partial.
__device__ __forceinline__ bool covers_units(long w, long T, long nwg) {
    // (with at least as many units as workgroups every share is non-empty:
    // no divisions in the common case)
    return T >= nwg || w * T / nwg != (w + 1) * T / nwg;
}

// Split merge: grid (B*H, gq), 1024 threads.  Log-sum-exp over the partials
// of one (stream, head): out = sum_p o_p e^(m_p-M) / sum_p l_p e^(m_p-M); 0 for
// an empty sequence (no partials).  The stream's partials are in the slots
// w + s of the workgroups w0 <= w <= w1 that cover its units (those with an
// empty share wrote none and are skipped); w1 - w0 < nwg <= kMaxParts.
constexpr int kMaxParts = 1024;
constexpr int kMergeThreads = 1024;
constexpr int kMergeSlices = kMergeThreads / kD;
constexpr int kMergeBatch = 16;   // partial outputs in flight per thread
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(Layout L, kvq_cache c, const float* __restrict__ ws,
                                                                  float* __restrict__ out, int gq, int nwg,
                                                                  long meta_off) {
    __shared__ float fac[kMaxParts];
    __shared__ float red[kMergeThreads / 64][2];
    __shared__ float acc[kMergeSlices][kD];
    const int s = blockIdx.x, hh = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int slice = tid >> 7, ch = tid & (kD - 1);
    float* orow = out + ((long)s * gq + hh) * kD;   // query head (s % H) * gq + hh of sequence s / H
    if (seq_units(L, c, s / L.H).units == 0) {
        if (tid < kD) orow[tid] = 0.0f;
        return;
    }
    // Workgroups covering the stream's units [P, P + units) of the T in all:
    // w covers [w T / nwg, (w + 1) T / nwg), so unit x lies in
    // ceil((x + 1) nwg / T) - 1 (clamped: a slot outside the workspace is
    // never read).
    const int* meta = (const int*)((const uint8_t*)ws + meta_off);
    const long T = max(meta[0], 1);
    const long P = meta[1 + s];
    const long units = seq_units(L, c, s / L.H).cost;   // (cost positions)
    const int w0 = (int)min(max(((P + 1) * nwg - 1) / T, 0L), (long)nwg - 1);
    const int w1 = (int)min(max(((P + units) * nwg - 1) / T, (long)w0), (long)nwg - 1);
    const int parts = w1 - w0 + 1;
    const long stride = (long)gq * kPart;
    const float* p = ws + ((long)(w0 + s) * gq + hh) * kPart;

    // The first batch of outputs is read together with the maxima and sums
    // (the partials of workgroups with an empty share are not read).
    float o0[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
        const int i = slice + j * kMergeSlices;
        o0[j] = i < parts && covers_units(w0 + i, T, nwg) ? p[i * stride + ch] : 0.0f;
    }
    float m = kNegInf, l = 0.0f;
    if (tid < parts && covers_units(w0 + tid, T, nwg)) {
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
    for (int j = 0; j < kMergeBatch; ++j) {
        const int i = slice + j * kMergeSlices;
        if (i < parts) sum = fmaf(o0[j], fac[i], sum);
    }
    for (int i0 = slice + kMergeSlices * kMergeBatch; i0 < parts; i0 += kMergeSlices * kMergeBatch) {
        float o[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const int i = i0 + j * kMergeSlices;
            o[j] = i < parts && fac[i] != 0.0f ? p[i * stride + ch] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const int i = i0 + j * kMergeSlices;
            if (i < parts) sum = fmaf(o[j], fac[i], sum);
        }
    }
    acc[slice][ch] = sum;
    __syncthreads();
    if (slice == 0) {
        float t = acc[0][ch];
        for (int k = 1; k < kMergeSlices; ++k) t += acc[k][ch];
        orow[ch] = Ls > 0.0f ? t / Ls : 0.0f;
    }
}

// Split merge for batches of many streams with few partials each: one wave
// per (stream, head) row, four rows per workgroup; lane l produces channels
// 2l and 2l+1.  Same arithmetic as attn_merge_kernel.
constexpr int kRowsPerMerge = 4;
__global__ __launch_bounds__(256) void attn_merge_rows_kernel(Layout L, kvq_cache c, const float* __restrict__ ws,
                                                              float* __restrict__ out, int gq, int nwg,
                                                              long meta_off) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * kRowsPerMerge + wave;
    if (row >= (long)L.B * L.H * gq) return;   // (no workgroup barrier below)
    const int s = (int)(row / gq), hh = (int)(row % gq);
    float2* orow = (float2*)(out + row * kD);
    const long units = seq_units(L, c, s / L.H).cost;   // (cost positions)
    if (units == 0) {
        orow[lane] = make_float2(0.0f, 0.0f);
        return;
    }
    const int* meta = (const int*)((const uint8_t*)ws + meta_off);
    const long T = max(meta[0], 1);
    const long P = meta[1 + s];
    const int w0 = (int)min(max(((P + 1) * nwg - 1) / T, 0L), (long)nwg - 1);
    const int w1 = (int)min(max(((P + units) * nwg - 1) / T, (long)w0), (long)nwg - 1);
    const int parts = w1 - w0 + 1;
    const long stride = (long)gq * kPart;
    const float* p = ws + ((long)(w0 + s) * gq + hh) * kPart;

    // Chunks of 16 partials, each read in one go (partial i0 + j's max and
    // weight sum by lanes j, j + 16, ..., its outputs by all lanes) and merged
    // into running sums rescaled to the running max: one round trip per chunk.
    float M = kNegInf, Ls = 0.0f;
    float2 acc = make_float2(0.0f, 0.0f);
    for (int i0 = 0; i0 < parts; i0 += 16) {
        const int i = i0 + (lane & 15);
        const bool mine = i < parts && covers_units(w0 + i, T, nwg);
        float2 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = i0 + j < parts && covers_units(w0 + i0 + j, T, nwg)
                       ? *(const float2*)(p + (long)(i0 + j) * stride + 2 * lane)
                       : make_float2(0.0f, 0.0f);
        const float mi = mine ? p[(long)i * stride + kD] : kNegInf;
        const float li = mine ? p[(long)i * stride + kD + 1] : 0.0f;
        float cm = mi;
        for (int off = 8; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
        const float Mn = fmaxf(M, cm);
        if (Mn == kNegInf) continue;   // nothing in this chunk or before it
        const float r = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        const float f = mi == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mi - Mn);
        // (every 16-lane group holds the chunk's 16 partials: sums within a
        // group give every lane the chunk's total)
        float lf = li * f;
        for (int off = 8; off >= 1; off >>= 1) lf += __shfl_xor(lf, off);
        Ls = Ls * r + lf;
        acc.x *= r;
        acc.y *= r;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float fj = __shfl(f, j);
            acc.x = fmaf(v[j].x, fj, acc.x);
            acc.y = fmaf(v[j].y, fj, acc.y);
        }
        M = Mn;
    }
    orow[lane] = Ls > 0.0f ? make_float2(acc.x / Ls, acc.y / Ls) : make_float2(0.0f, 0.0f);
}

// Instantiation key of the attention kernels: as layout_key, with the low-bit
// format's pre-RoPE variant as format kFmtRope.
static inline int attn_key(const Layout& L) {
    if (L.fmt != kFmtKivi) return layout_key(L);
    const bool rp = L.rope_theta > 0.0f, cb = L.grid == KVQ_GRID_NORMAL_QUANTILE;
    const int f = L.sparse ? (cb ? kFmtKiviCbSp : kFmtKiviSp)
                           : rp ? (cb ? kFmtRopeCb : kFmtRope) : (cb ? kFmtKiviCb : kFmtKivi);
    return layout_key(L) + f * 10000;
}

static int attn_slots(const Layout& L, int gq) {
    switch (attn_key(L)) {
#define KVQ_SLOTS_CASE(GG, KB, VB, FF) \
    case FF * 10000 + GG * 100 + KB * 10 + VB: return attn_family_slots<GG, KB, VB, FF>(L, gq);
        KVQ_ALL_FAMILIES(KVQ_SLOTS_CASE)
#undef KVQ_SLOTS_CASE
        default: return 256 * 3;
    }
}

// Compute units of the current device (256 when none is visible).
static int device_cus() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        (void)hipGetLastError();
        cached[dev] = cus;
    }
    return cached[dev];
}

AttnPlan plan_attention(const Layout& L, int num_q_heads) {
    AttnPlan P;
    const int gq = num_q_heads / L.H;
    const long streams = (long)L.B * L.H;
    const int maxg = L.paged ? L.max_blocks : L.groups;
    // 32-token units per stream at capacity: quantized groups, then the residual
    const long maxu = ((long)maxg * L.G + 31) / 32 + (L.R + L.G - 1 + 31) / 32;
    // One round of resident workgroups (the flattened split balances any
    // mix of lengths), no more than 1 per 8 units of the batch at capacity,
    // and never more partials per stream than the merge holds.
    long nwg = attn_slots(L, gq);
    // Uniform low-bit grid in a contiguous cache: two workgroups per CU keep
    // the split-K kernel as fast as a full round and halve the partials, so
    // the merge reads one chunk per row; so no more than about 8 partials
    // per stream, and no fewer than two workgroups per CU (70B layer, 8
    // streams: whole call 39.0-39.9 -> 37.3-37.5 us; 8B layer, 64 streams:
    // within run-to-run spread; the 80-layer cache, paged batches and the
    // heavier formats keep a full round, which they need).
    if (attn_key(L) / 10000 == kFmtKivi && !L.paged)
        nwg = std::min(nwg, std::max(2L * device_cus(), 8 * streams));
    nwg = std::min(nwg, std::max(1L, (streams * maxu + 7) / 8));
    if (const char* e = getenv("KVQ_WORKGROUPS")) {
        const int v = atoi(e);
        if (v >= 1) nwg = v;
    }
    nwg = std::min(nwg, (long)kMaxParts);
    P.nwg = (int)nwg;
    P.fits = streams * maxu < (1L << 31);   // flattened unit positions are 32-bit
    P.slots = nwg + streams - 1;
    P.part_floats = (size_t)gq * kPart;
    P.meta_off = (P.slots * P.part_floats * sizeof(float) + 255) / 256 * 256;
    P.workspace = P.meta_off + (size_t)(1 + streams) * sizeof(int32_t);
    return P;
}

hipError_t launch_attention_partials(const Layout& L, const AttnPlan& P, const kvq_cache& c, const half_t* q,
                                     int num_q_heads, float scale, void* ws, hipStream_t s) {
    const int gq = num_q_heads / L.H;
    const float sl2 = scale * kLog2e;
    switch (attn_key(L)) {
#define KVQ_LAUNCH_CASE(GG, KB, VB, FF) \
    case FF * 10000 + GG * 100 + KB * 10 + VB: return launch_attn_family<GG, KB, VB, FF>(L, P, c, q, gq, sl2, ws, s);
        KVQ_ALL_FAMILIES(KVQ_LAUNCH_CASE)
#undef KVQ_LAUNCH_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attention_merge(const Layout& L, const AttnPlan& P, const kvq_cache& c, int num_q_heads,
                                  const void* ws, float* out, hipStream_t s) {
    const int gq = num_q_heads / L.H;
    const long streams = (long)L.B * L.H;
    // partials per stream when the lengths are equal: a few -> one wave per
    // row; many -> a workgroup per row to keep all their loads in flight
    const long expect = (P.nwg + streams - 1) / streams + 2;
    if (expect <= 16) {
        const long rows = streams * gq;
        hipLaunchKernelGGL(attn_merge_rows_kernel, dim3((unsigned)((rows + kRowsPerMerge - 1) / kRowsPerMerge)),
                           dim3(64 * kRowsPerMerge), 0, s, L, c, (const float*)ws, out, gq, P.nwg, (long)P.meta_off);
    } else {
        hipLaunchKernelGGL(attn_merge_kernel, dim3(L.B * L.H, gq), dim3(kMergeThreads), 0, s, L, c,
                           (const float*)ws, out, gq, P.nwg, (long)P.meta_off);
    }
    return hipGetLastError();
}

}  // namespace kvq
