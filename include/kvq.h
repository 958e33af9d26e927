/*
 * kvq.h -- C ABI of the MI355X (gfx950) KIVI-style quantized KV-cache library.
 *
 * The method (cited by page title and section):
 *  - "KV cache compression: quantization, eviction and sparse attention",
 *    section 3.2 (KIVI): keys are quantized per channel over groups of G
 *    tokens, values per token, with a min/max scale and zero point; the most
 *    recent R tokens stay in full precision and a group is quantized once it
 *    is full; attention is computed over the quantized part and the
 *    full-precision part and the two are merged.  Section 3.4: paged blocks of
 *    16 tokens carry their own scale/zero tables, the key group is aligned to
 *    the block, and the attention kernel dequantizes while it reads.
 *  - "KV Cache compression lab", experiment 01: 2^b equally spaced levels
 *    between min and max, spacing (max - min)/(2^b - 1), zero = the grid's
 *    start, every value goes to its nearest level.
 *  - "KV cache compression" (jaedaily), formula paragraph: the per-channel
 *    key and per-token value dequantization q*s + z, and attention
 *    softmax(q k^T / sqrt(d_h)).
 *  - "KV cache compression: ...", section 3.3 (KVQuant): keys quantized
 *    before the rotary position embedding, which is applied by the attention
 *    kernel when it reads them; levels placed at quantiles of the
 *    distribution (like NF4) instead of evenly; section 2: RoPE rotates
 *    pairs of dimensions.
 *  - "KV Cache compression lab", experiment 03: KVQuant keeps the few
 *    extreme key values in fp16 as a sparse matrix and quantizes the rest.
 *  - "KV cache compression: ...", section 3.1, and "KV compression and
 *    quantization", part B.1: 8-bit caches at half the fp16 bytes, either
 *    FP8 E4M3 under a static per-head scale or INT8 under a dynamic
 *    per-token scale, dequantized by the attention kernel while it reads.
 *
 * Numeric contract (identical on every entry point):
 *   n_q  = G * floor(max(0, n - R) / G) quantized tokens; [n_q, n) stay fp16.
 *   For each key (group, channel) and each value token: mn, mx = min, max of
 *   the fp16 inputs (as fp32, -0 canonicalised to +0); s = fp16_rn((mx - mn)
 *   / (2^b - 1)); z = fp16(mn); inv = s > 0 ? 1/s : 0 (IEEE division);
 *   code = clamp(rint((x - z) * inv), 0, 2^b - 1) in fp32, ties to even.
 *   Dequantized value: fmaf(code, s, z).
 *   8-bit formats (kv_format): INT8 applies the same quantizer with b = 8 to
 *   every key and every value token over its 128 channels; FP8 E4M3 stores
 *   code = E4M3_rn(clamp(x * (1/scale), -448, 448)) (ties to even, the sign
 *   of a zero kept) with one static fp32 scale per kv head for keys and one
 *   for values, dequantized as E4M3(code) * scale.  Both keep n_q, the
 *   residual ring and the group flush above; only the codes differ.
 *   Attention: out[b][h] = sum_t softmax_t(scale * q[b][h] . k_t) v_t over all
 *   n tokens (dequantized part and fp16 residual), query head h reading kv
 *   head h / (Hq / H).  n = 0 gives out = 0.
 *   Codebook grid (grid = KVQ_GRID_NORMAL_QUANTILE, low-bit format): the 2^b
 *   levels are L_k = Q (c_k - c_0) / (c_Q - c_0), c_k = Phi^-1((k + 1/2) / 2^b)
 *   the standard normal quantiles, rounded to the nearest multiple of 1/F
 *   (F = 64 for 2 bits, 16 for 4; ties to even); s, z and inv as above;
 *   code = the nearest level to (x - z) * inv, a tie at a midpoint going to
 *   the even code; dequantized value fmaf(L_code, s, z).  kvq_codebook_levels
 *   returns the levels.
 *   Dense-and-sparse keys (sparse_keys = 1, low-bit format): in each key
 *   group the G entries of largest |x| (ties: lower position t*128 + c) are
 *   kept exactly in fp16; each channel's mn, mx (hence s, z) are taken over
 *   its other values (none left: s = z = 0); kept positions carry code 0 and
 *   dequantize to the kept value.
 *   Pre-RoPE keys (rope_theta > 0): the cache holds keys before the rotary
 *   embedding and attention uses RoPE_t(k_t) in place of k_t, pair
 *   (2i, 2i+1) of token t (0-based position in its sequence) rotated by the
 *   angle t * rope_theta^(-2i/128): (k0 cos - k1 sin, k0 sin + k1 cos).  The
 *   query is passed already rotated to its own position, as usual.
 *
 * Conventions for every call below:
 *   - Pointers named *_host are host memory; every other data pointer is a
 *     device pointer owned by the caller.  The library allocates and frees
 *     nothing and keeps no pointer to caller memory after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *     device work is enqueued asynchronously on it; the call returns once the
 *     work is enqueued.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns KVQ_EINVAL (or KVQ_EUNSUPPORTED for a valid but
 *     unimplemented shape) and enqueues nothing.  A failed launch returns
 *     KVQ_EHIP; kvq_last_error() then holds the HIP error text.
 *   - Inputs must be finite fp16; this is not checked on the hot path.
 *   - Calls on one cache must be ordered (same stream, or caller-synchronised).
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_HEAD_DIM 128

/* Cache formats (kvq_config.kv_format). */
#define KVQ_FORMAT_KIVI 0     /* keys per channel over G-token groups, values per
                                 token; k_bits, v_bits in {2, 4}                 */
#define KVQ_FORMAT_INT8 1     /* keys and values per token, 8-bit min/max grid
                                 computed at write time; k_bits = v_bits = 8     */
/* Level grids of the low-bit format (kvq_config.grid). */
#define KVQ_GRID_UNIFORM 0         /* 2^b evenly spaced levels (KIVI)              */
#define KVQ_GRID_NORMAL_QUANTILE 1 /* levels at normal quantiles, table dequant    */

#define KVQ_FORMAT_FP8_E4M3 2 /* keys and values FP8 E4M3 under static per-kv-head
                                 scales (kvq_cache.k_scale / v_scale);
                                 k_bits = v_bits = 8                             */

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_EINVAL = 1,        /* malformed argument (null pointer, bad size)      */
    KVQ_EUNSUPPORTED = 2,  /* well-formed but not implemented (e.g. d != 128)  */
    KVQ_ECAPACITY = 3,     /* buffer or workspace too small                    */
    KVQ_EHIP = 4           /* HIP runtime error while enqueueing               */
} kvq_status;

/* Shape of one quantized cache (one attention layer, or several layers folded
 * into the sequence axis). */
typedef struct kvq_config {
    int32_t num_seqs;           /* B >= 1                                        */
    int32_t num_kv_heads;       /* H >= 1                                        */
    int32_t head_dim;           /* d, must be 128                                */
    int32_t k_bits;             /* key code width: 2 or 4 (8 in 8-bit formats)   */
    int32_t v_bits;             /* value code width: 2 or 4 (8 in 8-bit formats) */
    int32_t group_size;         /* G: 16 or 32 tokens per key group              */
    int32_t residual;           /* R >= 0, a multiple of G.  8-bit formats with
                                   R = 0 quantize every token as it is written
                                   (n_q = n, the last group filling up)         */
    int32_t max_tokens;         /* contiguous mode: per-sequence capacity        */
    int32_t block_size;         /* 0 = contiguous; otherwise paged, == G         */
    int32_t num_blocks;         /* paged: blocks in the pool                     */
    int32_t max_blocks_per_seq; /* paged: length of one block-table row          */
    int32_t kv_format;          /* KVQ_FORMAT_*                                  */
    float rope_theta;           /* 0: keys used as given.  > 0: keys are stored
                                   before RoPE and rotated on read with this base
                                   (10000, 500000, ...); low-bit format only     */
    int32_t grid;               /* KVQ_GRID_*; the codebook grid needs the
                                   low-bit format                                */
    int32_t sparse_keys;        /* 1: dense-and-sparse keys (low-bit format, not
                                   with pre-RoPE keys); 0: off                   */
} kvq_config;

/* Device buffers of one cache.  Sizes come from kvq_buffer_sizes(). */
typedef struct kvq_cache {
    void *packed;               /* group records (codes + fp16 scale/zero)       */
    void *k_res;                /* fp16 key residual ring   [B][H][R+G][d]       */
    void *v_res;                /* fp16 value residual ring [B][H][R+G][d]       */
    int32_t *n_tokens;          /* [B] tokens held per sequence (n)              */
    int32_t *n_quant;           /* [B] quantized tokens per sequence (n_q)       */
    const int32_t *block_table; /* paged: [B][max_blocks_per_seq] block ids; a
                                   sequence's key group g lives in block
                                   block_table[b][g].  NULL in contiguous mode. */
    const float *k_scale;       /* FP8 format: [H] static key scale per kv head,
                                   positive and finite (caller-calibrated, e.g.
                                   max |k| / 448); ignored by other formats      */
    const float *v_scale;       /* FP8 format: [H] static value scale, likewise  */
    int32_t *arrivals;          /* optional [B] int32 (counter_bytes), 4-byte
                                   aligned: zero before the first
                                   kv_append_token (kv_quantize_prefill zeroes
                                   it) and left zero by the library.  With it an
                                   append is one kernel, whose last workgroup of
                                   each sequence advances that sequence's
                                   counters; NULL: a second kernel does that     */
} kvq_cache;

/* Byte sizes of the buffers of kvq_cache and of one group record.
 * Record = one (key group, kv head): G*d*k_bits/8 key-code bytes,
 * G*d*v_bits/8 value-code bytes, d fp16 key scales and d fp16 key zeros,
 * G fp16 value scales and G fp16 value zeros (INT8: G fp16 key scales and
 * zeros instead of d; FP8: no scales or zeros; dense-and-sparse keys: plus G
 * (position, fp16 value) pairs of 4 bytes), arranged inside the record in
 * the order the decode kernel consumes them (an internal format: use
 * kv_export_codes / kv_dequantize for a logical view).  Contiguous mode holds B*H*floor(max(0,max_tokens-R)/G)
 * records; paged mode holds num_blocks*H records. */
typedef struct kvq_sizes {
    size_t packed_bytes;
    size_t record_bytes;
    size_t residual_bytes;     /* each of k_res and v_res                        */
    size_t counter_bytes;      /* each of n_tokens, n_quant and arrivals         */
    size_t block_table_bytes;  /* paged mode only, else 0                        */
    int32_t groups_per_seq;    /* key groups one sequence can hold               */
    int32_t residual_slots;    /* R + G                                          */
} kvq_sizes;

/* Host only, no device work.  Validates cfg and fills *out. */
kvq_status kvq_buffer_sizes(const kvq_config *cfg, kvq_sizes *out);

/* Bulk quantization of whole sequences ("KV cache compression" (jaedaily),
 * deployment step (c); "KV cache compression: ...", section 3.2).
 * k, v: fp16 [B][H][max_len][d]; seq_lens: device int32 [B], the number of
 * valid tokens of each sequence.  Overwrites the cache state: for every
 * sequence, groups [0, n_q) are quantized into records and tokens [n_q, n)
 * are copied into the residual ring; n_tokens = n and n_quant = n_q (8-bit
 * formats with R = 0: n_q = n, the last group's record holding its tokens
 * and zero tokens after them).
 * Preconditions (caller): 0 <= seq_lens[b] <= max_len, seq_lens[b] within the
 * capacity (max_tokens, or max_blocks_per_seq*G with block_table rows filled
 * for every quantized group).  The kernels clamp a violating length to the
 * capacity and skip a record whose block id is outside [0, num_blocks), so no
 * access leaves the buffers; the cache content is then unspecified. */
kvq_status kv_quantize_prefill(const kvq_config *cfg, const kvq_cache *cache,
                               const void *k, const void *v, int32_t max_len,
                               const int32_t *seq_lens, void *stream);

/* Append one fp16 token to every sequence ("KV cache compression: ...",
 * section 3.2: the newest tokens stay full precision; once the full-precision
 * tail holds R + G tokens its oldest G tokens form a full group outside the
 * most recent R, which is quantized into a record and leaves the ring).
 * k_new, v_new: fp16 [B][H][d].  n_tokens and n_quant are updated on the
 * device, so a sequence of appends needs no host synchronisation: by the
 * append kernel itself when cache->arrivals is given (the last of a
 * sequence's kv-head workgroups to finish, counted by an agent-scope atomic
 * on arrivals[b], advances the counters once every head has read them, and
 * resets the count), else by a second one-thread-per-sequence kernel.
 * 8-bit formats with R = 0 quantize the new token at once into slot n % G
 * of its group's record (the group's first token clears the record first)
 * and advance n_q with n.
 * Preconditions (caller): n + 1 within capacity; in paged mode
 * block_table[b][n_q/G] holds a free block before the append that flushes
 * (8-bit formats with R = 0: block_table[b][n/G] before the append of each
 * group's first token; without it nothing is appended).
 * A flush that would leave the buffers is skipped (no write) and the token is
 * still appended to the ring only if the ring has room. */
kvq_status kv_append_token(const kvq_config *cfg, const kvq_cache *cache,
                           const void *k_new, const void *v_new, void *stream);

/* Dequantize the whole cache ("KV cache compression" (jaedaily), formula
 * paragraph: q*s + z, one fp32 rounding).  k_out, v_out: fp32
 * [B][H][out_tokens][d]; token t < n_tokens[b] receives its dequantized
 * (t < n_q) or exact fp16 (t >= n_q) value, later positions receive 0.
 * Tokens beyond out_tokens are not written. */
kvq_status kv_dequantize(const kvq_config *cfg, const kvq_cache *cache,
                         float *k_out, float *v_out, int32_t out_tokens, void *stream);

/* Workspace bytes kv_decode_attention needs for num_q_heads query heads.
 * Host only.  Returns 0 for an invalid cfg. */
size_t kv_decode_attention_workspace_bytes(const kvq_config *cfg, int32_t num_q_heads);

/* Decode attention of one query token per sequence over the whole cache
 * ("KV cache compression: ...", sections 3.1, 3.2 and 8.2: the kernel
 * dequantizes while it reads, the quantized part and the full-precision
 * residual are computed separately and merged).  q: fp16 [B][Hq][d];
 * out: fp32 [B][Hq][d]; Hq a multiple of H with Hq/H <= 16; softmax_scale is
 * normally 1/sqrt(d).  q must be 16-byte aligned.  Any finite fp16 query
 * and cache give a finite result: the kernel scales the query by a power of
 * two before it forms q * s in fp16 (and pre-RoPE keys before their fp16
 * split), and moves the factor into the softmax scale.  Accuracy is that of
 * fp32 accumulation: logits carrying terms far above 65504 (key groups
 * spanning most of the fp16 range against large query elements) keep the
 * fp32 rounding of those terms.
 * workspace: 256-byte aligned device memory of at least
 * kv_decode_attention_workspace_bytes(cfg, Hq) bytes that receives the
 * partial results (no initialisation needed, content not preserved between
 * calls).  Two kernels are enqueued: the attention, in which every workgroup
 * takes an equal share of all (sequence, kv head, 32-token unit) work of the
 * batch whatever the sequence lengths, and the log-sum-exp merge that writes
 * out; calls sharing a workspace must be ordered on one stream. */
kvq_status kv_decode_attention(const kvq_config *cfg, const kvq_cache *cache,
                               const void *q, int32_t num_q_heads, float softmax_scale,
                               float *out, void *workspace, size_t workspace_bytes,
                               void *stream);

/* The two steps of kv_decode_attention, for callers that place the merge
 * themselves (for example after gathering partials of a sequence split over
 * several devices: every partial is a (max, sum, output) triple that merges
 * by log-sum-exp).
 *
 * kv_decode_attention_partials: same arguments and checks as
 * kv_decode_attention without `out`; writes partial results of Hq/H heads x
 * 132 floats each (output[128] unnormalised, running max in log2 units, sum
 * of weights, pad) into the workspace, every (sequence, kv head) with
 * tokens getting one or more, and records per (sequence, kv head) where its
 * partials are.
 *
 * kv_decode_attention_merge: reads those partials for the same cfg, cache
 * counters and num_q_heads (the cache must not change in between) and writes
 * out fp32 [B][Hq][d] (0 for an empty sequence). */
kvq_status kv_decode_attention_partials(const kvq_config *cfg, const kvq_cache *cache,
                                        const void *q, int32_t num_q_heads, float softmax_scale,
                                        void *workspace, size_t workspace_bytes, void *stream);
kvq_status kv_decode_attention_merge(const kvq_config *cfg, const kvq_cache *cache,
                                     int32_t num_q_heads, const void *workspace,
                                     size_t workspace_bytes, float *out, void *stream);

/* kv_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments (minus the
 * workspace), checks and result as kv_decode_attention; the partial results
 * go to a fixed device array of KVQ_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends.  The call allocates
 * nothing: on its first use on a device it looks up that device's array
 * (the device of `stream`, or the current device for the null stream).
 * A call whose partials need more than the array holds
 * (kv_decode_attention_workspace_bytes(cfg, num_q_heads) above the limit)
 * returns KVQ_ECAPACITY with the sizes in kvq_last_error(), enqueueing
 * nothing.  Nothing in the array needs clearing between calls (every slot
 * the merge reads is written first in the same call), but every call on a
 * GPU uses that GPU's one array: calls that overlap on one GPU (different
 * streams, or threads without ordering) race and give wrong results. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kv_decode_attention_noalloc(const kvq_config *cfg, const kvq_cache *cache,
                                       const void *q, int32_t num_q_heads, float softmax_scale,
                                       float *out, void *stream);

/* Logical view of the quantized part (test hook).  k_codes, v_codes: uint8
 * [B][H][out_tokens][d], one code per element for t < n_q[b], 0 elsewhere;
 * k_s, k_z: fp16 bits [B][H][out_tokens/G][d] for groups < n_q[b]/G, 0
 * elsewhere; v_s, v_z: fp16 bits [B][H][out_tokens] for t < n_q[b], 0
 * elsewhere.  INT8 format: k_s, k_z are per token, [B][H][out_tokens] like
 * v_s, v_z.  FP8 format: the four scale/zero arrays are not written and may
 * be NULL.  out_tokens must be a multiple of G. */
kvq_status kv_export_codes(const kvq_config *cfg, const kvq_cache *cache,
                           uint8_t *k_codes, uint8_t *v_codes,
                           uint16_t *k_s, uint16_t *k_z, uint16_t *v_s, uint16_t *v_z,
                           int32_t out_tokens, void *stream);

/* Dense-and-sparse keys (test hook): the kept entries of every quantized key
 * group.  pos, val: uint16 [B][H][out_tokens/G][G], ascending positions
 * t*128 + c within the group and their fp16 values for groups < n_q[b]/G, 0
 * elsewhere.  out_tokens must be a multiple of G; KVQ_EINVAL unless the
 * cache has sparse_keys. */
kvq_status kv_export_outliers(const kvq_config *cfg, const kvq_cache *cache, uint16_t *pos, uint16_t *val,
                              int32_t out_tokens, void *stream);

/* Host only: the 2^bits levels L_0..L_Q (in steps of the uniform grid, so
 * the uniform grid's are 0..Q) of the normal-quantile codebook for bits 2
 * or 4, written to levels_host[0 .. 2^bits - 1]. */
kvq_status kvq_codebook_levels(int32_t bits, float *levels_host);

/* Static description of a status code. */
const char *kvq_status_string(kvq_status status);

/* Text of the last KVQ_EHIP error raised on the calling thread ("" if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
