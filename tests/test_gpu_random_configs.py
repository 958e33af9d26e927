"""GPU parity over seeded random configurations: every format and option
mixed with group sizes, residual windows, query heads per kv head, ragged
lengths (empty sequences included) and contiguous or paged caches.  Each
configuration is prefilled, then appended until every sequence has flushed
at least one group, and compared with the oracle: codes, scales, zeros and dequantized values
bit for bit, attention within max-abs 2e-3 and per-row cosine 0.9999; the
split entry points (partials, then merge) and the no-allocation entry point
must equal the combined call bit for bit.
The configurations come from a fixed seed, so the set is the same on every
run; each one prints its parameters before touching the GPU."""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_decode_attention_kivi_amd import kvq, synth
from parity_util import (compare_attention, compare_codes, make_cache, oracle_attention, oracle_states,
                         to_bits)

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5
N_CONFIGS = 96
N_LONG_CONFIGS = 24


def _config(i, long_context=False):
    rng = np.random.Generator(np.random.PCG64((0x10C9 if long_context else 0x5EED) + 7919 * i))
    fmt = int(rng.choice([kvq.FORMAT_KIVI] * 4 + [kvq.FORMAT_INT8, kvq.FORMAT_FP8_E4M3]))
    G = int(rng.choice([16, 32]))
    H = int(rng.integers(1, 4))
    gq = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    B = int(rng.integers(1, 5))
    R = int(rng.choice([0, G, 4 * G]))
    paged = bool(rng.integers(0, 2))
    kb = vb = 8
    theta, grid, sparse = 0.0, 0, 0
    if fmt == kvq.FORMAT_KIVI:
        kb, vb = int(rng.choice([2, 4])), int(rng.choice([2, 4]))
        option = int(rng.integers(0, 4))   # plain, codebook, pre-RoPE, dense-and-sparse
        grid = 1 if option == 1 or (option == 3 and rng.integers(0, 2)) else 0
        theta = 10000.0 if option == 2 else 0.0
        sparse = 1 if option == 3 else 0
    lens = rng.integers(0, 6000 if long_context else 900, size=B)
    if not long_context or B > 1:
        lens[int(rng.integers(0, B))] = int(rng.integers(0, 3))   # an empty or nearly empty sequence
    base = synth.WORKLOADS["llama3_8b_layer_b8_32k_int4"]
    w = dataclasses.replace(base, name="rnd%s%d" % ("L" if long_context else "", i), num_seqs=B, num_q_heads=H * gq, num_kv_heads=H, k_bits=kb,
                            v_bits=vb, group_size=G, residual=R, context=int(lens.max()) + 1, paged=paged,
                            min_context=0, tag=(300 if long_context else 200) + i, kv_format=fmt, rope_theta=theta, grid=grid,
                            sparse_keys=sparse)
    return w, lens.astype(np.int64), R + G + 1   # every sequence, the empty one too, flushes a group


@pytest.mark.parametrize("i", range(N_CONFIGS))
def test_random_configuration(i):
    _check_configuration(i, *_config(i))


@pytest.mark.parametrize("i", range(N_LONG_CONFIGS))
def test_random_long_configuration(i):
    """Lengths up to 6000 tokens: streams split over several workgroups."""
    _check_configuration(i, *_config(i, long_context=True))


def _check_configuration(i, w, lens0, steps):
    print("config %d: fmt=%d k%d/v%d G=%d R=%d B=%d H=%d gq=%d paged=%s theta=%g grid=%d sparse=%d lens=%s"
          % (i, w.kv_format, w.k_bits, w.v_bits, w.group_size, w.residual, w.num_seqs, w.num_kv_heads, w.gq,
             w.paged, w.rope_theta, w.grid, w.sparse_keys, list(lens0)), flush=True)
    L = int(lens0.max()) + steps
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    scales = synth.calibrate_fp8_scales(K, V) if w.kv_format == kvq.FORMAT_FP8_E4M3 else None
    cache = make_cache(w, lens0 + steps + 1, max_tokens=L + 8, shuffle_seed=i, scales=scales)
    m = int(max(int(lens0.max()), 1))
    cache.prefill(K[:, :, :m].contiguous(), V[:, :, :m].contiguous(), lens0)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :m], vb[:, :, :m], lens0, w, cap=L + 8, scales=scales)
    compare_codes(cache, states)
    lens = lens0.copy()
    for _ in range(steps):
        kn = torch.stack([K[b, :, int(lens[b])] for b in range(w.num_seqs)]).contiguous()
        vn = torch.stack([V[b, :, int(lens[b])] for b in range(w.num_seqs)]).contiguous()
        cache.append(kn, vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(kb[b, h, int(lens[b])], vb[b, h, int(lens[b])])
        lens += 1
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda", step=i)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE, rope_base=w.rope_theta))
    # the split entry points and the no-allocation entry point compute the
    # same thing as the combined call, bit for bit
    ev = tuple(torch.cuda.Event() for _ in range(3))
    split = cache.decode_attention(q, SCALE, split_events=ev)
    noalloc = torch.empty_like(out)
    kvq.kv_decode_attention_noalloc(cache.cfg, cache.cache, q, w.num_q_heads, SCALE, noalloc)
    torch.cuda.synchronize()
    assert torch.equal(split, out) and torch.equal(noalloc, out)
