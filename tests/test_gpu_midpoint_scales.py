"""GPU parity of scales whose quotient (max - min) / (2^b - 1) lies exactly
halfway between two fp16 numbers ("KV Cache compression lab", experiment 01:
the scale of a set is its range over 2^b - 1, kept in fp16).  The scale is
the fp16 rounding of the correctly rounded fp32 quotient, which on these sets
is the even neighbour; keys (per channel over a group) and values (per
token) are built on such extremes for every quantizer kernel: the uniform
grid at G = 32 and G = 16, the codebook grid, INT8 per token, and a flush
from the residual window on append.  Codes, scales, zeros and dequantized
values bit-exact against the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

from midpoint_extremes import MIDPOINT_EXTREMES
from quantized_decode_attention_kivi_amd import kvq, synth
from parity_util import compare_codes, make_cache, oracle_states, to_bits

pytestmark = pytest.mark.gpu


def _on_extremes(rng, n_sets, size, bits):
    """[n_sets][size] fp16 values; set i spans one pair of extremes (both
    present, at random places), the rest uniform in between."""
    pairs = MIDPOINT_EXTREMES[bits]
    out = np.empty((n_sets, size), np.float16)
    for i in range(n_sets):
        mn, mx = pairs[int(rng.integers(len(pairs)))]
        x = rng.uniform(mn, mx, size)
        a, b = rng.choice(size, 2, replace=False)
        x[a], x[b] = mn, mx
        out[i] = np.clip(x, mn, mx).astype(np.float16)
    return out


def _kv(w, L, seed):
    """Keys whose every (group, channel) set and values whose every token set
    lies on midpoint extremes (INT8: keys per token as well)."""
    rng = np.random.default_rng(seed)
    B, H, G, d = w.num_seqs, w.num_kv_heads, w.group_size, w.head_dim
    bits = 8 if w.kv_format == kvq.FORMAT_INT8 else w.k_bits
    K = np.empty((B, H, L, d), np.float16)
    if w.kv_format == kvq.FORMAT_INT8:
        K[:] = _on_extremes(rng, B * H * L, d, 8).reshape(B, H, L, d)
    else:
        ng = (L + G - 1) // G
        sets = _on_extremes(rng, B * H * ng * d, G, bits).reshape(B, H, ng, d, G)
        K[:] = sets.transpose(0, 1, 2, 4, 3).reshape(B, H, ng * G, d)[:, :, :L]
    vbits = 8 if w.kv_format == kvq.FORMAT_INT8 else w.v_bits
    V = _on_extremes(rng, B * H * L, d, vbits).reshape(B, H, L, d)
    return torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()


def _w(base, **kw):
    return dataclasses.replace(synth.workload(base), **kw)


CASES = {
    "uniform_g32": _w("llama3_8b_layer_b8_32k_int4", name="m32", num_seqs=2, num_q_heads=8, num_kv_heads=2,
                      residual=32, context=700, tag=91),
    "uniform_g16": _w("llama3_8b_layer_b8_32k_int4", name="m16", num_seqs=2, num_q_heads=8, num_kv_heads=2,
                      group_size=16, residual=16, context=16 * 29 + 5, tag=92),
    "codebook_g32": _w("llama3_8b_layer_b8_32k_int4_codebook", name="mcb", num_seqs=2, num_q_heads=8,
                       num_kv_heads=2, residual=32, context=700, tag=93),
    "int8_g32": _w("llama3_8b_layer_b8_32k_int8", name="m8", num_seqs=2, num_q_heads=8, num_kv_heads=2,
                   residual=32, context=700, tag=94),
}


@pytest.mark.parametrize("case", list(CASES))
def test_midpoint_scales_prefill(case):
    w = CASES[case]
    lens = np.array([w.context, w.context - 77], np.int64)
    L = int(lens.max())
    K, V = _kv(w, L, seed=w.tag)
    cache = make_cache(w, lens)
    print("prefill %s L=%d" % (w.name, L), flush=True)
    cache.prefill(K, V, lens)
    torch.cuda.synchronize()
    compare_codes(cache, oracle_states(to_bits(K), to_bits(V), lens, w, cap=L + 64))


@pytest.mark.parametrize("case", ["uniform_g32", "int8_g32"])
def test_midpoint_scales_append_flush(case):
    w = CASES[case]
    m, steps = 300, 2 * w.group_size + 3
    lens0 = np.array([m, m - 21], np.int64)
    K, V = _kv(w, m + steps, seed=w.tag + 100)
    cache = make_cache(w, lens0 + steps + 1, max_tokens=m + steps + 8)
    cache.prefill(K[:, :, :m].contiguous(), V[:, :, :m].contiguous(), lens0)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :m], vb[:, :, :m], lens0, w, cap=m + steps + 8)
    print("append %s steps=%d" % (w.name, steps), flush=True)
    for _ in range(steps):
        kn = torch.stack([K[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        vn = torch.stack([V[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        cache.append(kn, vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(kb[b, h, int(lens0[b])], vb[b, h, int(lens0[b])])
        lens0 += 1
    compare_codes(cache, states)
