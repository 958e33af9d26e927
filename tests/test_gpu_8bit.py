"""GPU parity of the 8-bit cache formats ("KV cache compression: quantization,
eviction and sparse attention", section 3.1: FP8 E4M3 under a static
per-head scale, INT8 under a dynamic per-token scale, dequantized by the
attention kernel while it reads): the HIP path through the C ABI against
the CPU oracle on the same seeded inputs.  Codes, scales, zeros and
dequantized values bit-exact; attention within max-abs 2e-3 and per-row
cosine 0.9999.
"""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_decode_attention_kivi_amd import kvq, synth
from parity_util import (compare_attention, compare_codes, make_cache, oracle_attention, oracle_states,
                         to_bits)

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5
FORMATS = {"int8": kvq.FORMAT_INT8, "fp8": kvq.FORMAT_FP8_E4M3}


def _w(fmt, **kw):
    base = dataclasses.replace(synth.WORKLOADS_8BIT["llama3_8b_layer_b8_32k_int8"], kv_format=FORMATS[fmt])
    return dataclasses.replace(base, **kw)


# several key groups, several splits, ragged tails; G = 16 with an odd group
# count (half-empty last unit); more than 8 query heads per kv head (no limb
# packing); no residual window; a paged pool
SMALL = {
    "gqa4_g32_ragged": dict(name="e4", num_seqs=3, context=2048 + 37, tag=51),
    "gqa1_g16_odd": dict(name="e1", num_seqs=3, num_q_heads=3, num_kv_heads=3, group_size=16, residual=16,
                         context=16 * 37 + 9, tag=52),
    "gqa16_g16": dict(name="e16", num_seqs=2, num_q_heads=32, num_kv_heads=2, group_size=16, residual=32,
                      context=777, tag=53),
    "gqa8_g32_r0": dict(name="e8", num_seqs=2, num_q_heads=16, num_kv_heads=2, residual=0, context=1000,
                        tag=54),
    "paged_g16": dict(name="ep", num_seqs=5, group_size=16, residual=128, context=1500, min_context=30,
                      paged=True, tag=55),
}


def _prefill(w, lens=None):
    lens = synth.seq_lengths(w) if lens is None else np.asarray(lens, np.int64)
    L = int(max(int(np.max(lens)), 1))
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    scales = synth.calibrate_fp8_scales(K, V) if w.kv_format == kvq.FORMAT_FP8_E4M3 else None
    cache = make_cache(w, lens, shuffle_seed=9, scales=scales)
    print("prefill %s fmt=%d B=%d H=%d L=%d" % (w.name, w.kv_format, w.num_seqs, w.num_kv_heads, L), flush=True)
    cache.prefill(K, V, lens)
    torch.cuda.synchronize()
    states = oracle_states(to_bits(K), to_bits(V), lens, w, cap=L + 256, scales=scales)
    return cache, states, K, V, scales


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("case", list(SMALL))
def test_prefill_codes_and_attention_8bit(fmt, case):
    w = _w(fmt, **SMALL[case])
    cache, states, _, _, _ = _prefill(w)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_edge_lengths_8bit(fmt):
    G, R = 32, 64
    lens = [0, 1, R - 1, R, R + 1, R + G - 1, R + G, R + G + 1, 5 * G + R + 3]
    w = _w(fmt, name="e8edge", num_seqs=len(lens), num_q_heads=8, num_kv_heads=2, residual=R,
           context=max(lens), tag=56)
    cache, states, _, _, _ = _prefill(w, lens)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    assert np.all(out[0] == 0)
    compare_attention(out, oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_append_sequence_8bit(fmt):
    """prefill(m) then appends crossing several flushes equal the oracle's
    incremental state (FP8: appended tokens beyond the calibrated range
    saturate at +-448 scale on both sides)."""
    w = _w(fmt, name="e8app", num_seqs=3, num_q_heads=8, num_kv_heads=2, group_size=16, residual=32,
           context=400, tag=57)
    m, steps = 250, 3 * 16 + 5
    lens0 = np.array([m, m - 17, m - 40], np.int64)
    K, V = synth.make_kv(w, max_len=m + steps, device="cuda")
    # calibrate on the prefilled part only, so the appended tokens can exceed it
    scales = synth.calibrate_fp8_scales(K[:, :, :m - 40], V[:, :, :m - 40]) \
        if w.kv_format == kvq.FORMAT_FP8_E4M3 else None
    cache = make_cache(w, lens0 + steps + 1, max_tokens=m + steps + 8, scales=scales)
    cache.prefill(K[:, :, :m].contiguous(), V[:, :, :m].contiguous(), lens0)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :m], vb[:, :, :m], lens0, w, cap=m + steps + 8, scales=scales)
    for s in range(steps):
        kn = torch.stack([K[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        vn = torch.stack([V[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        cache.append(kn, vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(kb[b, h, int(lens0[b])], vb[b, h, int(lens0[b])])
        lens0 += 1
        if s % 16 == 15 or s == steps - 1:
            compare_codes(cache, states)
    q = synth.make_query(w, device="cuda", step=3)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("G,paged", [(16, False), (32, False), (16, True), (32, True)])
def test_quantized_on_write_8bit(fmt, G, paged):
    """Without a residual window the 8-bit formats quantize every token as it
    is written ("KV cache compression: quantization, eviction and sparse
    attention", section 3.1): after a prefill of ragged lengths and after
    every append n_q = n, the partial last group included; codes, scales,
    zeros and dequantized values bit-exact against the oracle, attention
    within the bar (paged: each group's block is handed out when its first
    token is written)."""
    w = _w(fmt, name="e8ow", num_seqs=3, num_q_heads=8, num_kv_heads=2, group_size=G, residual=0,
           context=300, tag=59 + G, paged=paged)
    m, steps = 200, G + 7
    lens0 = np.array([m, m - 5, m - G - 3], np.int64)
    K, V = synth.make_kv(w, max_len=m + steps, device="cuda")
    scales = synth.calibrate_fp8_scales(K, V) if w.kv_format == kvq.FORMAT_FP8_E4M3 else None
    cache = make_cache(w, lens0 + steps + 1, max_tokens=m + steps + 8, shuffle_seed=13, scales=scales)
    print("on-write %s G=%d paged=%d" % (fmt, G, paged), flush=True)
    cache.prefill(K[:, :, :m].contiguous(), V[:, :, :m].contiguous(), lens0)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :m], vb[:, :, :m], lens0, w, cap=m + steps + 8, scales=scales)
    torch.cuda.synchronize()
    assert np.array_equal(cache.n_quant.cpu().numpy(), lens0) and np.array_equal(cache.n_tokens.cpu().numpy(), lens0)
    compare_codes(cache, states)
    for s in range(steps):
        kn = torch.stack([K[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        vn = torch.stack([V[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        cache.append(kn, vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(kb[b, h, int(lens0[b])], vb[b, h, int(lens0[b])])
        lens0 += 1
        if s in (0, 2, G - 3, steps - 1):
            torch.cuda.synchronize()
            assert np.array_equal(cache.n_quant.cpu().numpy(), lens0)
            compare_codes(cache, states)
    q = synth.make_query(w, device="cuda", step=5)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_fp8_codes_are_the_e4m3_encoding_of_every_value():
    """Every E4M3 code (both signs, subnormals, 448) and the midpoints between
    neighbouring codes go through the device quantizer: inputs x = v * s with
    s a power of two so x * (1/s) is exact, and the codes must be the
    oracle's encoding (ties to even, saturation beyond 448)."""
    import oracle
    w = _w("fp8", name="e8grid", num_seqs=1, num_q_heads=1, num_kv_heads=1, residual=0, context=512, tag=58)
    codes = np.concatenate([np.arange(0, 0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    vals = np.sort(oracle.fp8_decode(codes[:0x7F]).astype(np.float64))
    mids = (vals[:-1] + vals[1:]) / 2
    pool = np.concatenate([oracle.fp8_decode(codes).astype(np.float64), mids, -mids, [460.0, -500.0, 1e4]])
    s = 2.0 ** -4
    x = (pool * s).astype(np.float16)                    # every value here is exact in fp16
    assert np.array_equal(x.astype(np.float64), pool * s)
    n = 512
    flat = np.resize(x, n * 128).reshape(1, 1, n, 128)
    K = torch.from_numpy(flat).cuda()
    V = torch.from_numpy(flat[:, :, ::-1].copy()).cuda()
    scales = (torch.full((1,), s, device="cuda"), torch.full((1,), s, device="cuda"))
    cache = make_cache(w, [n], scales=scales)
    cache.prefill(K, V, [n])
    states = oracle_states(to_bits(K), to_bits(V), [n], w, cap=n + 64, scales=scales)
    compare_codes(cache, states)
    kc = cache.export_codes(n)[0][0, 0].cpu().numpy()
    assert set(np.unique(kc).tolist()) >= set(codes.tolist())   # every code occurs


@pytest.mark.parametrize("name", list(synth.WORKLOADS_8BIT))
def test_full_size_8bit_workload(name):
    """The 8B-layer workload (8 x 32K tokens, 32 q / 8 kv heads) in each
    8-bit format at full size: sampled streams bit-exact, every attention row."""
    w = synth.WORKLOADS_8BIT[name]
    cache, states, _, _, _ = _prefill(w)
    compare_codes(cache, states, streams=[(0, 0), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))
