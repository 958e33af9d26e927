"""GPU parity of pre-RoPE keys rotated on read ("KV cache compression:
quantization, eviction and sparse attention", section 3.3: keys quantized
before the rotary embedding, which the attention kernel applies when it
reads them): the HIP path through the C ABI against the CPU oracle (fp64
rotation of the dequantized keys, fp64 attention).  Codes, scales, zeros and
dequantized (pre-RoPE) values bit-exact; attention within max-abs 2e-3 and
per-row cosine 0.9999.
"""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_decode_attention_kivi_amd import synth
from parity_util import (compare_attention, compare_codes, make_cache, oracle_attention, oracle_states,
                         to_bits)

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


def _w(base, **kw):
    return dataclasses.replace(synth.workload(base), **kw)


# every bit-width pair and both group sizes; ragged tails, more than 8 query
# heads per kv head, no residual window, a paged pool; positions up to 128K
SMALL = {
    "k4v4_g32_gq4": _w("llama3_8b_layer_b8_32k_int4_prerope", name="r44", num_seqs=3, context=2048 + 37, tag=61),
    "k2v2_g32_gq8": _w("llama3_70b_layer_b1_128k_int2_prerope", name="r22", num_seqs=2, context=4096 + 5, tag=62),
    "k2v4_g32_r0": _w("llama3_8b_layer_b8_32k_int4_prerope", name="r24", num_seqs=2, num_q_heads=4, num_kv_heads=2,
                      k_bits=2, v_bits=4, residual=0, context=1500, tag=63, rope_theta=10000.0),
    "k4v2_g16_gq16": _w("llama3_8b_layer_b8_32k_int4_prerope", name="r42", num_seqs=2, num_q_heads=32, num_kv_heads=2,
                        k_bits=4, v_bits=2, group_size=16, residual=32, context=777, tag=64),
    "k2v2_g16_odd_gq1": _w("llama3_8b_layer_b8_32k_int4_prerope", name="r1", num_seqs=3, num_q_heads=3,
                           num_kv_heads=3, k_bits=2, v_bits=2, group_size=16, residual=16, context=16 * 37 + 9,
                           tag=65),
    "paged_k4v2_g16": _w("llama3_8b_layer_b8_32k_int4_prerope", name="rp", num_seqs=5, k_bits=4, v_bits=2,
                         group_size=16, residual=128, context=1500, min_context=30, paged=True, tag=66),
}


def _prefill(w, lens=None):
    lens = synth.seq_lengths(w) if lens is None else np.asarray(lens, np.int64)
    L = int(max(int(np.max(lens)), 1))
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens, shuffle_seed=13)
    print("prefill %s rope=%g B=%d H=%d L=%d" % (w.name, w.rope_theta, w.num_seqs, w.num_kv_heads, L), flush=True)
    cache.prefill(K, V, lens)
    torch.cuda.synchronize()
    states = oracle_states(to_bits(K), to_bits(V), lens, w, cap=L + 256)
    return cache, states, K, V


@pytest.mark.parametrize("case", list(SMALL))
def test_prefill_and_rotated_attention(case):
    w = SMALL[case]
    cache, states, _, _ = _prefill(w)
    compare_codes(cache, states)        # the cache holds the pre-RoPE keys
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE, rope_base=w.rope_theta))


def test_rope_edges_and_appends():
    """Empty and short sequences, flush boundaries, then appends that cross
    flushes (the rotation follows each token's position through the move
    from the ring to a record)."""
    G, R = 32, 64
    lens = np.array([0, 1, R - 1, R + G, R + G + 1, 5 * G + R + 3], np.int64)
    w = _w("llama3_8b_layer_b8_32k_int4_prerope", name="redge", num_seqs=len(lens), num_q_heads=8, num_kv_heads=2,
           k_bits=2, v_bits=4, residual=R, context=int(lens.max()) + 80, tag=67)
    steps = 2 * G + 3
    K, V = synth.make_kv(w, max_len=int(lens.max()) + steps, device="cuda")
    cache = make_cache(w, lens + steps + 1, max_tokens=int(lens.max()) + steps + 8)
    cache.prefill(K[:, :, :int(lens.max())].contiguous(), V[:, :, :int(lens.max())].contiguous(), lens)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb, vb, lens, w, cap=int(lens.max()) + steps + 8)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    assert np.all(out[0] == 0)
    compare_attention(out, oracle_attention(to_bits(q), states, SCALE, rope_base=w.rope_theta))
    for s in range(steps):
        kn = torch.stack([K[b, :, int(lens[b])] for b in range(w.num_seqs)]).contiguous()
        vn = torch.stack([V[b, :, int(lens[b])] for b in range(w.num_seqs)]).contiguous()
        cache.append(kn, vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(kb[b, h, int(lens[b])], vb[b, h, int(lens[b])])
        lens += 1
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda", step=5)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE, rope_base=w.rope_theta))


def test_rope_at_position_zero_only_is_plain_attention():
    """A one-token cache: the key sits at position 0, where RoPE is the
    identity, so the output is that token's value whatever the base."""
    w = _w("llama3_8b_layer_b8_32k_int4_prerope", name="r0", num_seqs=2, num_q_heads=4, num_kv_heads=2, context=1,
           tag=68)
    cache, states, K, V = _prefill(w, [1, 1])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    exp = np.repeat(V[:, :, 0].float().cpu().numpy(), 2, axis=1)
    assert np.abs(out - exp).max() == 0


@pytest.mark.parametrize("name", list(synth.WORKLOADS_ROPE))
def test_full_size_rope_workload(name):
    """The 8B-layer (8 x 32K) and 70B-layer (1 x 128K, positions up to
    131071) shapes with pre-RoPE keys at full size: sampled streams
    bit-exact, every attention row against the oracle's fp64 rotation."""
    w = synth.WORKLOADS_ROPE[name]
    cache, states, _, _ = _prefill(w)
    compare_codes(cache, states, streams=[(0, 0), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE, rope_base=w.rope_theta))
