"""GPU parity of dense-and-sparse keys ("KV Cache compression lab",
experiment 03: KVQuant keeps the few extreme key values in fp16 as a sparse
matrix and quantizes the rest): the HIP path through the C ABI against the
CPU oracle.  Codes, scales, zeros, kept (position, value) pairs and
dequantized values bit-exact; attention within max-abs 2e-3 and per-row
cosine 0.9999.
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


SMALL = {
    "k4v4_g32_gq4": _w("llama3_8b_layer_b8_32k_int4_sparse", name="s44", num_seqs=3, context=2048 + 37, tag=81),
    "k2v2_g32_gq8": _w("llama3_70b_layer_b1_128k_int2_sparse", name="s22", num_seqs=2, context=4096 + 5, tag=82),
    "k2v4_g32_r0": _w("llama3_8b_layer_b8_32k_int4_sparse", name="s24", num_seqs=2, num_q_heads=4, num_kv_heads=2,
                      k_bits=2, v_bits=4, residual=0, context=1500, tag=83),
    "k4v2_g16_gq16": _w("llama3_8b_layer_b8_32k_int4_sparse", name="s42", num_seqs=2, num_q_heads=32,
                        num_kv_heads=2, k_bits=4, v_bits=2, group_size=16, residual=32, context=777, tag=84),
    "k2v2_g16_odd_gq1": _w("llama3_8b_layer_b8_32k_int4_sparse", name="s1", num_seqs=3, num_q_heads=3,
                           num_kv_heads=3, k_bits=2, v_bits=2, group_size=16, residual=16, context=16 * 37 + 9,
                           tag=85),
    "paged_k4v2_g16": _w("llama3_8b_layer_b8_32k_int4_sparse", name="sp", num_seqs=5, k_bits=4, v_bits=2,
                         group_size=16, residual=128, context=1500, min_context=30, paged=True, tag=86),
    "codebook_k2v2_g32": _w("llama3_70b_layer_b1_128k_int2_sparse", name="scb", num_seqs=2, context=3000, tag=87,
                            grid=1),
}


def _prefill(w, lens=None, K=None, V=None):
    lens = synth.seq_lengths(w) if lens is None else np.asarray(lens, np.int64)
    L = int(max(int(np.max(lens)), 1))
    if K is None:
        K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens, shuffle_seed=19)
    print("prefill %s sparse grid=%d B=%d H=%d L=%d" % (w.name, w.grid, w.num_seqs, w.num_kv_heads, L), flush=True)
    cache.prefill(K, V, lens)
    torch.cuda.synchronize()
    states = oracle_states(to_bits(K), to_bits(V), lens, w, cap=L + 256)
    return cache, states, K, V


@pytest.mark.parametrize("case", list(SMALL))
def test_sparse_prefill_and_attention(case):
    w = SMALL[case]
    cache, states, _, _ = _prefill(w)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_sparse_ties_and_concentrated_extremes():
    """Groups whose extremes crowd into one token or one channel, and equal
    magnitudes at the selection boundary (ties go to the lower position)."""
    w = _w("llama3_8b_layer_b8_32k_int4_sparse", name="stie", num_seqs=1, num_q_heads=2, num_kv_heads=1,
           residual=0, context=256, tag=88)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((256, 128))
    k[5, :40] = 30.0 + np.arange(40)          # one token holds more than G extremes
    k[32:64, 77] = 60.0 - np.arange(32)       # one channel of a whole group kept
    k[64:96][np.arange(32), (7 * np.arange(32)) % 128] = 25.0   # equal magnitudes, more than G
    k[70, 3] = -25.0
    K = torch.from_numpy(k.astype(np.float16)).reshape(1, 1, 256, 128).cuda()
    V = torch.from_numpy(rng.standard_normal((1, 1, 256, 128)).astype(np.float16)).cuda()
    cache, states, _, _ = _prefill(w, [256], K, V)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_sparse_appends_across_flushes():
    w = _w("llama3_8b_layer_b8_32k_int4_sparse", name="sapp", num_seqs=3, num_q_heads=8, num_kv_heads=2,
           k_bits=4, v_bits=2, group_size=16, residual=32, context=400, tag=89)
    m, steps = 250, 3 * 16 + 5
    lens0 = np.array([m, m - 17, m - 40], np.int64)
    K, V = synth.make_kv(w, max_len=m + steps, device="cuda")
    cache = make_cache(w, lens0 + steps + 1, max_tokens=m + steps + 8)
    cache.prefill(K[:, :, :m].contiguous(), V[:, :, :m].contiguous(), lens0)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :m], vb[:, :, :m], lens0, w, cap=m + steps + 8)
    for s in range(steps):
        kn = torch.stack([K[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        vn = torch.stack([V[b, :, int(lens0[b])] for b in range(w.num_seqs)]).contiguous()
        cache.append(kn, vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(kb[b, h, int(lens0[b])], vb[b, h, int(lens0[b])])
        lens0 += 1
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda", step=3)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("name", list(synth.WORKLOADS_SPARSE))
def test_full_size_sparse_workload(name):
    w = synth.WORKLOADS_SPARSE[name]
    cache, states, _, _ = _prefill(w)
    compare_codes(cache, states, streams=[(0, 0), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))
