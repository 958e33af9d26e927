// kvq_api.hip -- C ABI of libkvq: host-side validation, sizes and dispatch.
// Every entry point validates its arguments before anything is enqueued and
// never allocates device memory.
#include <cmath>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include "kvq_internal.h"

namespace kvq {

static thread_local char g_last_error[256] = "";

// Fixed device scratch of kv_decode_attention_noalloc: one copy per GPU the
// library runs on, held until the process ends.  In host code the array's
// name is only a stand-in for the symbol, never a device address: the
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed to
// kernels.
constexpr size_t kScratchBytes = (size_t)KVQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

static kvq_status hip_status(hipError_t e) {
    if (e == hipSuccess) return KVQ_OK;
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return KVQ_EHIP;
}

// Standard normal quantile: Newton's method on Phi(x) - p from x = 0
// (Phi(x) = erfc(-x / sqrt 2) / 2, Phi'(x) = exp(-x^2 / 2) / sqrt(2 pi)); the
// codebook needs p in [1/32, 31/32], where it converges in a few steps.
static double normal_quantile(double p) {
    double x = 0.0;
    for (int it = 0; it < 60; ++it) {
        const double f = 0.5 * std::erfc(-x * M_SQRT1_2) - p;
        const double d = std::exp(-0.5 * x * x) * 0.3989422804014326779;
        x -= f / d;
    }
    return x;
}

int codebook_levels16(int bits, int* levels16) {
    if (bits != 2 && bits != 4) return 0;
    const int n = 1 << bits, Q = n - 1;
    const int F = bits == 2 ? 64 : 16;   // largest power of two with F * Q <= 255
    double c[16];
    for (int k = 0; k < n; ++k) c[k] = normal_quantile((k + 0.5) / n);
    for (int k = 0; k < n; ++k) levels16[k] = (int)std::nearbyint(F * Q * (c[k] - c[0]) / (c[Q] - c[0]));
    return F;
}

// The kernels' tables of a codebook grid: byte levels (lut) and the
// midpoints between neighbouring levels (mid).  They depend on the bit width
// alone, so they are computed once per width (the quantiles cost tens of
// microseconds, far more than a decode call's launch).
struct CodebookTables {
    uint32_t lut[4];
    float mid[15];
};

static CodebookTables make_codebook_tables(int bits) {
    CodebookTables t;
    int lev[16] = {0};
    const int F = codebook_levels16(bits, lev);
    const int n = 1 << bits;
    for (int w = 0; w < 4; ++w) t.lut[w] = 0;
    for (int k = 0; k < n; ++k) t.lut[k >> 2] |= (uint32_t)lev[k] << (8 * (k & 3));
    for (int k = 0; k < 15; ++k) t.mid[k] = k + 1 < n ? (float)(lev[k] + lev[k + 1]) / (float)(2 * F) : 0.0f;
    return t;
}

static void fill_codebook(int bits, uint32_t* lut, float* mid) {
    static const CodebookTables t2 = make_codebook_tables(2), t4 = make_codebook_tables(4);   // (thread-safe init)
    const CodebookTables& t = bits == 2 ? t2 : t4;
    for (int w = 0; w < 4; ++w) lut[w] = t.lut[w];
    for (int k = 0; k < 15; ++k) mid[k] = t.mid[k];
}

kvq_status make_layout(const kvq_config* cfg, Layout* L) {
    if (!cfg || !L) return KVQ_EINVAL;
    if (cfg->num_seqs < 1 || cfg->num_kv_heads < 1) return KVQ_EINVAL;
    if (cfg->head_dim != kD) return KVQ_EUNSUPPORTED;
    if (cfg->kv_format == kFmtKivi) {
        if ((cfg->k_bits != 2 && cfg->k_bits != 4) || (cfg->v_bits != 2 && cfg->v_bits != 4))
            return KVQ_EUNSUPPORTED;
    } else if (cfg->kv_format == kFmtInt8 || cfg->kv_format == kFmtFp8) {
        if (cfg->k_bits != 8 || cfg->v_bits != 8) return KVQ_EINVAL;
    } else {
        return KVQ_EINVAL;
    }
    const int G = cfg->group_size;
    if (G != 16 && G != 32) return KVQ_EUNSUPPORTED;
    if (cfg->residual < 0 || cfg->residual % G != 0) return KVQ_EINVAL;
    if (cfg->residual > (1 << 20)) return KVQ_EINVAL;
    if (!(cfg->rope_theta >= 0.0f) || cfg->rope_theta > 1e30f) return KVQ_EINVAL;   // also rejects NaN
    if (cfg->rope_theta > 0.0f && (cfg->kv_format != kFmtKivi || cfg->rope_theta <= 1.0f)) return KVQ_EUNSUPPORTED;
    L->rope_theta = cfg->rope_theta;
    if (cfg->grid != KVQ_GRID_UNIFORM && cfg->grid != KVQ_GRID_NORMAL_QUANTILE) return KVQ_EINVAL;
    if (cfg->grid == KVQ_GRID_NORMAL_QUANTILE && cfg->kv_format != kFmtKivi) return KVQ_EUNSUPPORTED;
    L->grid = cfg->grid;
    for (int i = 0; i < 4; ++i) L->klut[i] = L->vlut[i] = 0;
    for (int i = 0; i < 15; ++i) L->kmid[i] = L->vmid[i] = 0.0f;
    if (L->grid == KVQ_GRID_NORMAL_QUANTILE) {
        fill_codebook(cfg->k_bits, L->klut, L->kmid);
        fill_codebook(cfg->v_bits, L->vlut, L->vmid);
    }
    if (cfg->sparse_keys != 0 && cfg->sparse_keys != 1) return KVQ_EINVAL;
    if (cfg->sparse_keys && (cfg->kv_format != kFmtKivi || cfg->rope_theta > 0.0f)) return KVQ_EUNSUPPORTED;
    L->sparse = cfg->sparse_keys;
    L->fmt = cfg->kv_format;
    L->B = cfg->num_seqs;
    L->H = cfg->num_kv_heads;
    L->kbits = cfg->k_bits;
    L->vbits = cfg->v_bits;
    L->G = G;
    L->R = cfg->residual;
    L->ring = cfg->residual + G;
    // 8-bit formats quantize each token on its own: without a residual
    // window a token is quantized when written (the group's record fills up
    // token by token)
    L->onwrite = cfg->kv_format != kFmtKivi && cfg->residual == 0;
    L->paged = cfg->block_size != 0;
    if (L->paged) {
        if (cfg->block_size != G) return KVQ_EINVAL;
        if (cfg->num_blocks < 1 || cfg->max_blocks_per_seq < 1) return KVQ_EINVAL;
        L->num_blocks = cfg->num_blocks;
        L->max_blocks = cfg->max_blocks_per_seq;
        L->groups = cfg->max_blocks_per_seq;
        const long cap = L->onwrite ? (long)L->max_blocks * G : (long)L->R + (long)(L->max_blocks + 1) * G - 1;
        L->capacity = cap > 0x7fffffffL ? 0x7fffffff : (int)cap;
    } else {
        if (cfg->max_tokens < 0) return KVQ_EINVAL;
        L->num_blocks = 0;
        L->max_blocks = 0;
        L->groups = L->onwrite ? (cfg->max_tokens + G - 1) / G : num_quantized(cfg->max_tokens, G, L->R) / G;
        L->capacity = cfg->max_tokens;
    }
    L->spt = G == 16 ? 4 : 8;
    L->kcode = G * kD * L->kbits / 8;
    L->vcode = G * kD * L->vbits / 8;
    L->vcode_off = L->kcode;
    L->kmeta_off = L->vcode_off + L->vcode;
    // key table: per (group, channel) for KIVI, per token for INT8, none for FP8
    const int kmeta = L->fmt == kFmtKivi ? kD * 4 : L->fmt == kFmtInt8 ? G * 4 : 0;
    L->vmeta_off = L->kmeta_off + kmeta;
    L->sparse_off = L->vmeta_off + (L->fmt == kFmtFp8 ? 0 : G * 4);
    L->record = L->sparse_off + (L->sparse ? G * 4 : 0);
    return KVQ_OK;
}

static kvq_status check_cache(const Layout& L, const kvq_cache* c) {
    if (!c || !c->packed || !c->k_res || !c->v_res || !c->n_tokens || !c->n_quant) return KVQ_EINVAL;
    if ((uintptr_t)c->arrivals & 3) return KVQ_EINVAL;
    if (L.paged && !c->block_table) return KVQ_EINVAL;
    if (((uintptr_t)c->packed & 15) || ((uintptr_t)c->k_res & 15) || ((uintptr_t)c->v_res & 15))
        return KVQ_EINVAL;
    if (L.fmt == kFmtFp8 && (!c->k_scale || !c->v_scale || ((uintptr_t)c->k_scale & 3) ||
                             ((uintptr_t)c->v_scale & 3)))
        return KVQ_EINVAL;
    return KVQ_OK;
}

// Device address of the scratch array on the device that `stream` belongs to
// (the current device for the null stream), looked up on the first call for
// that device with the device made current for the lookup.
static kvq_status scratch_address(hipStream_t stream, void** out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    dev = cur;
    if (stream && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return KVQ_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t restore = dev != cur ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return hip_status(e);
        if (restore != hipSuccess) return hip_status(restore);
        if (!p || ((uintptr_t)p & 255)) {
            snprintf(g_last_error, sizeof(g_last_error), "scratch array of device %d at a bad address %p", dev, p);
            return KVQ_EHIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

#pragma GCC visibility push(default)
extern "C" {

kvq_status kvq_buffer_sizes(const kvq_config* cfg, kvq_sizes* out) {
    Layout L;
    if (!out) return KVQ_EINVAL;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    const size_t nrec = L.paged ? (size_t)L.num_blocks * L.H : (size_t)L.B * L.H * L.groups;
    out->record_bytes = (size_t)L.record;
    out->packed_bytes = nrec * L.record;
    out->residual_bytes = (size_t)L.B * L.H * L.ring * kD * 2;
    out->counter_bytes = (size_t)L.B * sizeof(int32_t);
    out->block_table_bytes = L.paged ? (size_t)L.B * L.max_blocks * sizeof(int32_t) : 0;
    out->groups_per_seq = L.groups;
    out->residual_slots = L.ring;
    return KVQ_OK;
}

kvq_status kv_quantize_prefill(const kvq_config* cfg, const kvq_cache* cache, const void* k, const void* v,
                               int32_t max_len, const int32_t* seq_lens, void* stream) {
    Layout L;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, cache)) != KVQ_OK) return st;
    if (!k || !v || !seq_lens || max_len < 0) return KVQ_EINVAL;
    if (((uintptr_t)k & 15) || ((uintptr_t)v & 15)) return KVQ_EINVAL;
    return hip_status(launch_prefill(L, *cache, (const _Float16*)k, (const _Float16*)v, max_len, seq_lens,
                                     (hipStream_t)stream));
}

kvq_status kv_append_token(const kvq_config* cfg, const kvq_cache* cache, const void* k_new, const void* v_new,
                           void* stream) {
    Layout L;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, cache)) != KVQ_OK) return st;
    if (!k_new || !v_new || ((uintptr_t)k_new & 3) || ((uintptr_t)v_new & 3)) return KVQ_EINVAL;
    return hip_status(launch_append(L, *cache, (const _Float16*)k_new, (const _Float16*)v_new,
                                    (hipStream_t)stream));
}

kvq_status kv_dequantize(const kvq_config* cfg, const kvq_cache* cache, float* k_out, float* v_out,
                         int32_t out_tokens, void* stream) {
    Layout L;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, cache)) != KVQ_OK) return st;
    if (!k_out || !v_out || out_tokens < 0) return KVQ_EINVAL;
    return hip_status(launch_dequantize(L, *cache, k_out, v_out, out_tokens, (hipStream_t)stream));
}

size_t kv_decode_attention_workspace_bytes(const kvq_config* cfg, int32_t num_q_heads) {
    Layout L;
    if (make_layout(cfg, &L) != KVQ_OK) return 0;
    if (num_q_heads < L.H || num_q_heads % L.H) return 0;
    const AttnPlan P = plan_attention(L, num_q_heads);
    return P.fits ? P.workspace : 0;
}

static kvq_status check_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t num_q_heads,
                                  float softmax_scale, const void* workspace, size_t workspace_bytes, Layout* L,
                                  AttnPlan* P) {
    kvq_status st = make_layout(cfg, L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(*L, cache)) != KVQ_OK) return st;
    if (!q || !workspace || ((uintptr_t)q & 15) || ((uintptr_t)workspace & 255)) return KVQ_EINVAL;
    if (num_q_heads < L->H || num_q_heads % L->H) return KVQ_EINVAL;
    const int gq = num_q_heads / L->H;
    if (gq < 1 || gq > kMaxGq) return KVQ_EUNSUPPORTED;
    if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return KVQ_EINVAL;
    *P = plan_attention(*L, num_q_heads);
    if (!P->fits) return KVQ_EUNSUPPORTED;
    if (workspace_bytes < P->workspace) return KVQ_ECAPACITY;
    return KVQ_OK;
}

kvq_status kv_decode_attention_partials(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                        int32_t num_q_heads, float softmax_scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    Layout L;
    AttnPlan P;
    kvq_status st = check_attention(cfg, cache, q, num_q_heads, softmax_scale, workspace, workspace_bytes, &L, &P);
    if (st != KVQ_OK) return st;
    return hip_status(launch_attention_partials(L, P, *cache, (const _Float16*)q, num_q_heads, softmax_scale,
                                                workspace, (hipStream_t)stream));
}

kvq_status kv_decode_attention_merge(const kvq_config* cfg, const kvq_cache* cache, int32_t num_q_heads,
                                     const void* workspace, size_t workspace_bytes, float* out, void* stream) {
    Layout L;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, cache)) != KVQ_OK) return st;
    if (!workspace || !out || ((uintptr_t)workspace & 255)) return KVQ_EINVAL;
    if (num_q_heads < L.H || num_q_heads % L.H) return KVQ_EINVAL;
    const int gq = num_q_heads / L.H;
    if (gq < 1 || gq > kMaxGq) return KVQ_EUNSUPPORTED;
    const AttnPlan P = plan_attention(L, num_q_heads);
    if (!P.fits) return KVQ_EUNSUPPORTED;
    if (workspace_bytes < P.workspace) return KVQ_ECAPACITY;
    return hip_status(launch_attention_merge(L, P, *cache, num_q_heads, workspace, out, (hipStream_t)stream));
}

kvq_status kv_decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t num_q_heads,
                               float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
    Layout L;
    AttnPlan P;
    kvq_status st = check_attention(cfg, cache, q, num_q_heads, softmax_scale, workspace, workspace_bytes, &L, &P);
    if (st != KVQ_OK) return st;
    if (!out) return KVQ_EINVAL;
    st = hip_status(launch_attention_partials(L, P, *cache, (const _Float16*)q, num_q_heads, softmax_scale,
                                              workspace, (hipStream_t)stream));
    if (st != KVQ_OK) return st;
    return hip_status(launch_attention_merge(L, P, *cache, num_q_heads, workspace, out, (hipStream_t)stream));
}

kvq_status kv_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                       int32_t num_q_heads, float softmax_scale, float* out, void* stream) {
    Layout L;
    AttnPlan P;
    // validation first, with a stand-in workspace address: the size and
    // argument checks need no device and enqueue nothing
    kvq_status st = check_attention(cfg, cache, q, num_q_heads, softmax_scale, (const void*)(uintptr_t)256,
                                    kScratchBytes, &L, &P);
    if (st == KVQ_ECAPACITY || (st == KVQ_OK && P.workspace > kScratchBytes)) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "kv_decode_attention_noalloc: this call needs %zu bytes of scratch, the fixed array holds %zu",
                 (size_t)P.workspace, kScratchBytes);
        return KVQ_ECAPACITY;
    }
    if (st != KVQ_OK) return st;
    if (!out) return KVQ_EINVAL;
    void* ws = nullptr;
    if ((st = scratch_address((hipStream_t)stream, &ws)) != KVQ_OK) return st;
    st = hip_status(launch_attention_partials(L, P, *cache, (const _Float16*)q, num_q_heads, softmax_scale, ws,
                                              (hipStream_t)stream));
    if (st != KVQ_OK) return st;
    return hip_status(launch_attention_merge(L, P, *cache, num_q_heads, ws, out, (hipStream_t)stream));
}

kvq_status kv_export_codes(const kvq_config* cfg, const kvq_cache* cache, uint8_t* k_codes, uint8_t* v_codes,
                           uint16_t* k_s, uint16_t* k_z, uint16_t* v_s, uint16_t* v_z, int32_t out_tokens,
                           void* stream) {
    Layout L;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, cache)) != KVQ_OK) return st;
    if (!k_codes || !v_codes) return KVQ_EINVAL;
    if (L.fmt != kFmtFp8 && (!k_s || !k_z || !v_s || !v_z)) return KVQ_EINVAL;
    if (out_tokens < 0 || out_tokens % L.G) return KVQ_EINVAL;
    return hip_status(launch_export(L, *cache, k_codes, v_codes, k_s, k_z, v_s, v_z, out_tokens,
                                    (hipStream_t)stream));
}

kvq_status kv_export_outliers(const kvq_config* cfg, const kvq_cache* cache, uint16_t* pos, uint16_t* val,
                              int32_t out_tokens, void* stream) {
    Layout L;
    kvq_status st = make_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, cache)) != KVQ_OK) return st;
    if (!L.sparse || !pos || !val || out_tokens < 0 || out_tokens % L.G) return KVQ_EINVAL;
    return hip_status(launch_export_outliers(L, *cache, pos, val, out_tokens, (hipStream_t)stream));
}

kvq_status kvq_codebook_levels(int32_t bits, float* levels_host) {
    if (!levels_host) return KVQ_EINVAL;
    int lev[16];
    const int F = codebook_levels16(bits, lev);
    if (!F) return KVQ_EUNSUPPORTED;
    for (int k = 0; k < (1 << bits); ++k) levels_host[k] = (float)lev[k] / (float)F;
    return KVQ_OK;
}

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid argument";
        case KVQ_EUNSUPPORTED: return "unsupported configuration";
        case KVQ_ECAPACITY: return "buffer or workspace too small";
        case KVQ_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* kvq_last_error(void) { return g_last_error; }

}  // extern "C"
#pragma GCC visibility pop
