"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.  Codes, scales, zeros and dequantized values must
match bit for bit; attention within max-abs 2e-3 and per-row cosine 0.9999.

Sizes: small cases span several key groups, several splits and a ragged tail;
the full-size cases are the five measured workloads themselves.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_kivi_amd import synth
from quantized_decode_attention_kivi_amd.kvq import num_quantized as kvq_num_quantized
from parity_util import (compare_attention, compare_codes, compare_stream_codes, make_cache, oracle_attention,
                         oracle_states, to_bits)

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


def _w(base, **kw):
    return dataclasses.replace(synth.WORKLOADS[base], **kw)


SMALL = {
    "single_head_1k_int2": _w("single_head_1k_int2"),
    "gqa4_int4_ragged": _w("llama3_8b_layer_b8_32k_int4", num_seqs=3, context=2048 + 37),
    "gqa8_int2_ragged": _w("llama3_70b_layer_b1_128k_int2", num_seqs=2, context=4096 + 5),
    "gqa2_k2v4_r64": _w("llama3_8b_layer_b8_32k_int4", name="k2v4", num_seqs=2, num_q_heads=4, num_kv_heads=2,
                        k_bits=2, v_bits=4, group_size=32, residual=64, context=1500, tag=21),
    "gqa1_k4v4_g16_odd": _w("llama3_8b_layer_b8_32k_int4", name="g16odd", num_seqs=3, num_q_heads=3,
                            num_kv_heads=3, k_bits=4, v_bits=4, group_size=16, residual=16, context=16 * 37 + 9,
                            tag=24),
    "gqa16_k4v2_g16": _w("llama3_8b_layer_b8_32k_int4", name="gq16", num_seqs=2, num_q_heads=32,
                         num_kv_heads=2, k_bits=4, v_bits=2, group_size=16, residual=32, context=777, tag=22),
    "mha_g32_r0": _w("llama3_8b_layer_b8_32k_int4", name="mha", num_seqs=2, num_q_heads=4, num_kv_heads=4,
                     k_bits=4, v_bits=2, group_size=32, residual=0, context=1000, tag=23),
    "paged_k4v2_g16": _w("paged_64seq_1k_16k_k4v2", name="pga", num_seqs=3, context=700, min_context=200, tag=25),
}


def _run_prefill(w, lens=None, paged_shuffle=7):
    lens = synth.seq_lengths(w) if lens is None else np.asarray(lens, np.int64)
    L = int(max(int(np.max(lens)), 1))
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens, shuffle_seed=paged_shuffle)
    print("prefill %s B=%d H=%d L=%d lens=%s" % (w.name, w.num_seqs, w.num_kv_heads, L, list(lens)[:8]), flush=True)
    cache.prefill(K, V, lens)
    torch.cuda.synchronize()
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb, vb, lens, w, cap=L + 256)
    return cache, states, kb, vb


@pytest.mark.parametrize("case", list(SMALL))
def test_prefill_codes_and_attention(case):
    w = SMALL[case]
    cache, states, _, _ = _run_prefill(w)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    ref = oracle_attention(to_bits(q), states, SCALE)
    compare_attention(out.cpu().numpy(), ref)


def test_edge_lengths_in_one_batch():
    """Empty sequence, shorter than the residual, exactly at the flush
    boundaries and one past them, all in the same batch."""
    base = _w("llama3_8b_layer_b8_32k_int4", name="edges", num_kv_heads=2, num_q_heads=8, k_bits=2, v_bits=4,
              group_size=32, residual=64, tag=31)
    G, R = 32, 64
    lens = [0, 1, R - 1, R, R + 1, R + G - 1, R + G, R + G + 1, 5 * G + R + 3]
    w = dataclasses.replace(base, num_seqs=len(lens), context=max(lens))
    cache, states, _, _ = _run_prefill(w, lens)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    assert np.all(out[0] == 0)  # n = 0 gives 0
    ref = oracle_attention(to_bits(q), states, SCALE)
    compare_attention(out, ref)


@pytest.mark.parametrize("paged", [False, True])
def test_many_short_sequences(paged):
    """3000 sequences of 0 to 400 tokens in one batch (6000 streams, more
    than one workgroup round): the per-sequence prefix every workgroup
    computes in its prologue, the flattened split across many streams, the
    merge, and appends of 3000 sequences per launch across a group flush.
    Attention of every row against the oracle after the prefill and after
    the appends; codes of a sample of sequences bit for bit."""
    B = 3000
    w = _w("paged_64seq_1k_16k_k4v2" if paged else "llama3_8b_layer_b8_32k_int4", name="many%d" % paged,
           num_seqs=B, num_q_heads=8, num_kv_heads=2, k_bits=2, v_bits=4, group_size=16 if paged else 32,
           residual=32, context=400, min_context=0, tag=35 + paged)
    lens = np.random.Generator(np.random.PCG64(35 + paged)).integers(0, 401, size=B).astype(np.int64)
    steps = w.group_size + 1   # every sequence flushes a group at most once, most none
    L = int(lens.max()) + steps
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens + steps, shuffle_seed=7)
    print("many sequences: B=%d paged=%s steps=%d" % (B, paged, steps), flush=True)
    cache.prefill(K[:, :, :int(lens.max())].contiguous(), V[:, :, :int(lens.max())].contiguous(), lens)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :int(lens.max())], vb[:, :, :int(lens.max())], lens, w, cap=L + 64)
    rng = np.random.Generator(np.random.PCG64(7))
    sample = [(int(b), h) for b in rng.choice(B, 40, replace=False) for h in range(2)]
    compare_codes(cache, states, sample)
    q = synth.make_query(w, device="cuda")
    compare_attention(cache.decode_attention(q, SCALE).cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))
    # appends: one kernel launch for all 3000 sequences per step
    n = lens.copy()
    for _ in range(steps):
        idx = torch.as_tensor(n, device="cuda")
        ar = torch.arange(B, device="cuda")
        cache.append(K[ar, :, idx].contiguous(), V[ar, :, idx].contiguous())
        for b in range(B):
            for h in range(2):
                states[b][h].append(kb[b, h, n[b]], vb[b, h, n[b]])
        n += 1
    compare_codes(cache, states, sample)
    q = synth.make_query(w, device="cuda", step=1)
    compare_attention(cache.decode_attention(q, SCALE).cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_cache_without_group_capacity():
    """A contiguous cache too short ever to flush a group (max_tokens below
    R + G): it holds no group records, every token stays in the residual
    window.  Prefill, appends, exports through sequence and stream views, and
    attention all work on it; the views hand over the cache's placeholder
    record buffer, since a zero-size slice has no address."""
    G, R, cap = 32, 32, 43
    w = _w("llama3_8b_layer_b8_32k_int4", name="nogroups", num_seqs=3, num_kv_heads=2, num_q_heads=8, k_bits=2,
           v_bits=2, group_size=G, residual=R, context=cap, tag=34)
    lens0, steps = np.array([0, 20, 7], np.int64), 20
    K, V = synth.make_kv(w, max_len=cap, device="cuda")
    cache = make_cache(w, lens0 + steps, max_tokens=cap)
    assert cache.sizes.packed_bytes == 0
    print("no-group cache: lens=%s steps=%d cap=%d" % (list(lens0), steps, cap), flush=True)
    m = int(lens0.max())
    cache.prefill(K[:, :, :m].contiguous(), V[:, :, :m].contiguous(), lens0)
    kb, vb = to_bits(K), to_bits(V)
    states = oracle_states(kb[:, :, :m], vb[:, :, :m], lens0, w, cap=cap)
    lens = lens0.copy()
    for _ in range(steps):
        cache.append(torch.stack([K[b, :, int(lens[b])] for b in range(3)]).contiguous(),
                     torch.stack([V[b, :, int(lens[b])] for b in range(3)]).contiguous())
        for b in range(3):
            for h in range(2):
                states[b][h].append(kb[b, h, int(lens[b])], vb[b, h, int(lens[b])])
        lens += 1
    assert all(st.nq == 0 for row in states for st in row)
    compare_codes(cache, states)
    compare_stream_codes(cache, 1, 1, states[1][1])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    compare_attention(out, oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("case,arrivals", [("gqa4_int4_ragged", True), ("gqa16_k4v2_g16", True),
                                           ("mha_g32_r0", True), ("paged_k4v2_g16", True),
                                           ("gqa4_int4_ragged", False), ("paged_k4v2_g16", False)])
def test_append_sequence_matches_prefill(case, arrivals):
    """prefill(m) followed by appends that cross several flushes must equal
    the oracle's incremental state, step by step (paged: each flush's block
    is handed out from a shuffled pool and written into the device table
    between calls).  arrivals: the counters advance inside the append kernel
    (per-sequence arrival counts, left zero), else in a second kernel."""
    w = SMALL[case]
    m = 300 if w.residual < 300 else w.residual + 5
    steps = 3 * w.group_size + 7
    lens0 = np.full(w.num_seqs, m, np.int64)
    lens0[-1] = max(0, m - 17)  # ragged
    K, V = synth.make_kv(w, max_len=m + steps, device="cuda")
    cache = make_cache(w, lens0 + steps + 1, max_tokens=m + steps + 8, shuffle_seed=5)
    if not arrivals:
        cache.cache.arrivals = None
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
        if s % 16 == 15 or s == steps - 1:
            compare_codes(cache, states)
    assert not cache.arrivals.any()
    q = synth.make_query(w, device="cuda", step=3)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_paged_matches_contiguous_and_oracle():
    w = _w("paged_64seq_1k_16k_k4v2", num_seqs=6, context=1200, min_context=40)
    lens = synth.seq_lengths(w)
    cache, states, kb, vb = _run_prefill(w, lens, paged_shuffle=11)
    compare_codes(cache, states)
    q = synth.make_query(w, device="cuda")
    outp = cache.decode_attention(q, SCALE)
    wc = dataclasses.replace(w, paged=False)
    K = torch.from_numpy(kb.view(np.float16)).cuda()
    V = torch.from_numpy(vb.view(np.float16)).cuda()
    cc = make_cache(wc, lens)
    cc.prefill(K, V, lens)
    outc = cc.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    # the same records read through the block table give the same result up
    # to the order of the split merge
    assert (outp - outc).abs().max().item() <= 1e-5
    compare_attention(outp.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_constant_values_give_constant_output():
    """All value rows equal -> every weight sum equals 1 -> out = that row
    (weights are internal to the kernel, so this is how their sum is seen)."""
    w = _w("llama3_70b_layer_b1_128k_int2", name="constv", num_seqs=2, context=3000, tag=41)
    lens = [3000, 2111]
    K, V = synth.make_kv(w, max_len=3000, device="cuda")
    # grid-aligned rows (spacing 1/4, both extreme codes present) quantize exactly
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    codes = torch.randint(0, 4, (w.num_kv_heads, 1, 128), generator=gen, device="cuda")
    codes[:, :, 0], codes[:, :, 1] = 0, 3
    row = (codes.float() * 0.25 - 0.5).to(torch.float16)
    V = row.unsqueeze(0).expand(2, -1, 3000, -1).contiguous()
    cache = make_cache(w, lens)
    cache.prefill(K, V, lens)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    exp = np.repeat(row[:, 0].float().cpu().numpy(), w.gq, axis=0)
    for b in range(2):
        assert np.abs(out[b] - exp).max() < 1e-5


@pytest.mark.parametrize("name", ["llama3_8b_layer_b8_32k_int4", "llama3_70b_layer_b1_128k_int2"])
def test_full_size_workload(name):
    """The measured single-layer workloads at full size, every output row."""
    w = synth.WORKLOADS[name]
    cache, states, _, _ = _run_prefill(w)
    compare_codes(cache, states, streams=[(0, 0), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("name", ["llama3_8b_layer_b8_32k_int4", "llama3_70b_layer_b1_128k_int2"])
def test_full_size_decode_steps(name):
    """The single-layer workloads at full size through the decode steps the
    benchmark times: prefill, then 40 appends (every stream flushes one group
    at the 32nd), then attention; sampled streams bit-exact and every
    attention row against the oracle's incremental state."""
    w = synth.WORKLOADS[name]
    lens = synth.seq_lengths(w)
    L = int(lens.max())
    steps = 40
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens, max_tokens=L + steps + 8)
    print("prefill %s, then %d appends" % (w.name, steps), flush=True)
    cache.prefill(K, V, lens)
    kb, vb = to_bits(K), to_bits(V)
    del K, V
    states = oracle_states(kb, vb, lens, w, cap=L + steps + 8)
    del kb, vb
    for s in range(steps):
        kn, vn = synth.make_tokens(w, s, device="cuda")
        cache.append(kn.contiguous(), vn.contiguous())
        knb, vnb = to_bits(kn), to_bits(vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(knb[b, h], vnb[b, h])
    assert all(states[b][h].nq == lens[b] - w.residual + w.group_size
               for b in range(w.num_seqs) for h in range(w.num_kv_heads))
    compare_codes(cache, states, streams=[(0, 0), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda", step=7)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_full_size_paged_workload():
    """The paged workload at full size (64 sequences of 1K-16K tokens, G = 16
    blocks handed out from a shuffled pool): sampled sequences bit-exact,
    every attention row."""
    w = synth.WORKLOADS["paged_64seq_1k_16k_k4v2"]
    cache, states, _, _ = _run_prefill(w)
    compare_codes(cache, states, streams=[(0, 0), (17, 3), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


def test_full_size_paged_decode_steps():
    """The paged workload at full size through decode steps: prefill from a
    shuffled pool, then 20 appends (every sequence crosses at least one
    16-token flush, its block written into the device table between calls),
    then attention; sampled sequences bit-exact, every attention row."""
    w = synth.WORKLOADS["paged_64seq_1k_16k_k4v2"]
    lens = synth.seq_lengths(w).astype(np.int64)
    L = int(lens.max())
    steps = 20
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens + steps + 1, shuffle_seed=9)
    print("prefill %s, then %d appends" % (w.name, steps), flush=True)
    cache.prefill(K, V, lens)
    kb, vb = to_bits(K), to_bits(V)
    del K, V
    states = oracle_states(kb, vb, lens, w, cap=L + steps + 8)
    del kb, vb
    for s in range(steps):
        kn, vn = synth.make_tokens(w, s, device="cuda")
        cache.append(kn.contiguous(), vn.contiguous())
        knb, vnb = to_bits(kn), to_bits(vn)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                states[b][h].append(knb[b, h], vnb[b, h])
    flushed = [states[b][0].nq > kvq_num_quantized(int(lens[b]), w.group_size, w.residual)
               for b in range(w.num_seqs)]
    assert all(flushed)
    compare_codes(cache, states, streams=[(0, 0), (17, 3), (w.num_seqs - 1, w.num_kv_heads - 1)])
    q = synth.make_query(w, device="cuda", step=5)
    out = cache.decode_attention(q, SCALE)
    torch.cuda.synchronize()
    compare_attention(out.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.timeout(600)
def test_full_size_80_layer_cache():
    """The 80-layer, 128K-token INT2 cache with the layers folded into the
    batch (43 GB of fp16 input, 7 GB packed), every stream: each layer's
    input is pulled back and the oracle quantizes all of its 8 (layer, kv
    head) streams from the same bits on the host thread pool; the 64 query
    rows of every layer (5120 in all) must match the oracle's attention, and
    kv head (layer mod 8) of every layer -- 80 streams, kv heads 0-7 ten times
    each -- must match bit for bit in codes, scales, zeros and dequantized
    values."""
    from concurrent.futures import ThreadPoolExecutor
    from parity_util import THREADS
    w = synth.WORKLOADS["llama3_70b_cache_80l_128k_int2"]
    lens = synth.seq_lengths(w)
    L = int(lens.max())
    B, H, gq = w.num_seqs, w.num_kv_heads, w.gq
    print("generating %s (%d x %d x %d x 128 fp16, K and V)" % (w.name, B, H, L), flush=True)
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens)
    cache.prefill(K, V, lens)
    q = synth.make_query(w, device="cuda")
    out = cache.decode_attention(q, SCALE).cpu().numpy()
    qf = oracle.h2f(to_bits(q))
    ref = np.empty(out.shape, np.float64)

    def one(job):
        b, h, kb, vb = job
        st = oracle.StreamState.prefill(kb, vb, w.k_bits, w.v_bits, w.group_size, w.residual)
        kh, vh = st.dequantize()
        ref[b, h * gq:(h + 1) * gq] = oracle.attention(qf[b, h * gq:(h + 1) * gq], kh, vh, SCALE)
        return st if h == b % H else None

    per = max(1, THREADS // H)   # layers per round: one stream per pool thread
    with ThreadPoolExecutor(THREADS) as ex:
        for b0 in range(0, B, per):
            bs = range(b0, min(b0 + per, B))
            kb = to_bits(K[b0:bs[-1] + 1])
            vb = to_bits(V[b0:bs[-1] + 1])
            jobs = [(b, h, kb[b - b0, h, :lens[b]], vb[b - b0, h, :lens[b]]) for b in bs for h in range(H)]
            for st, (b, h, _, _) in zip(ex.map(one, jobs), jobs):
                if st is not None:
                    compare_stream_codes(cache, b, h, st)
            if b0 % 16 == 0:
                print("layers %d-%d checked" % (b0, bs[-1]), flush=True)
    del K, V
    torch.cuda.empty_cache()
    compare_attention(out, ref)
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nwg", [1, 2, 5, 13, 64, 300, 1024])
def test_any_workgroup_count(nwg):
    """The flattened split gives the oracle's result for any number of
    attention workgroups: workgroups spanning several streams, streams spread
    over many workgroups, more workgroups than units, and empty sequences at
    the start, in the middle and at the end of the batch (both merge kernels
    are used across these counts)."""
    base = _w("llama3_8b_layer_b8_32k_int4", name="flat", num_kv_heads=2, num_q_heads=8, k_bits=4, v_bits=2,
              group_size=32, residual=64, tag=32)
    lens = [0, 700, 33, 0, 2100, 64, 0]
    w = dataclasses.replace(base, num_seqs=len(lens), context=max(lens))
    cache, states, _, _ = _run_prefill(w, lens)
    q = synth.make_query(w, device="cuda")
    os.environ["KVQ_WORKGROUPS"] = str(nwg)
    try:
        out = cache.decode_attention(q, SCALE).cpu().numpy()
    finally:
        del os.environ["KVQ_WORKGROUPS"]
    for b in (0, 3, 6):
        assert np.all(out[b] == 0)
    compare_attention(out, oracle_attention(to_bits(q), states, SCALE))


def test_split_entry_points_equal_combined_call():
    """kv_decode_attention_partials followed by kv_decode_attention_merge is
    the same computation as kv_decode_attention (bit for bit)."""
    w = SMALL["gqa8_int2_ragged"]
    cache, states, _, _ = _run_prefill(w)
    q = synth.make_query(w, device="cuda", step=2)
    a = cache.decode_attention(q, SCALE).clone()
    ev = tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
    b = cache.decode_attention(q, SCALE, split_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    compare_attention(b.cpu().numpy(), oracle_attention(to_bits(q), states, SCALE))


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 32), (2, 2, 32), (4, 2, 16), (2, 4, 16), (8, 8, 32), (8, 8, 16)])
def test_prefill_ties_on_power_of_two_grids(kb, vb, G):
    """Keys on a per-channel grid (INT8: per-token, like the values) and
    values on a per-token grid, both with a power-of-two step and both
    extremes present, at half steps: t = (x - z)/s is exact and every odd
    multiple of 1/2 is a tie, which rounds to even.  Codes, scales and zeros
    bit-exact against the oracle."""
    Q = (1 << kb) - 1
    R = G
    B, H, L = 2, 2, 5 * G + R + 3
    w = _w("llama3_8b_layer_b8_32k_int4", name="ties", num_seqs=B, num_q_heads=2 * H, num_kv_heads=H, k_bits=kb,
           v_bits=vb, group_size=G, residual=R, context=L, tag=43, kv_format=1 if kb == 8 else 0)
    rng = np.random.Generator(np.random.PCG64(17))

    def per_token(Qb):
        # token t holds base_t + (k/2) s_t over its channels, channels 0/1 at the extremes
        kk = rng.integers(0, 2 * Qb + 1, (B, H, L, 128))
        kk[..., 0], kk[..., 1] = 0, 2 * Qb
        st = 2.0 ** -rng.integers(2, 6, (B, H, L, 1))
        return kk, rng.integers(-8, 8, (B, H, L, 1)) * 0.125 + kk * 0.5 * st

    if kb == 8:
        k, K = per_token(Q)
    else:
        # channel c of every group holds base_c + (k/2) s_c, k in [0, 2Q],
        # the group's first two tokens at k = 0 and k = 2Q
        k = rng.integers(0, 2 * Q + 1, (B, H, L, 128))
        g0 = np.arange(L) % G
        k[:, :, g0 == 0, :] = 0
        k[:, :, g0 == 1, :] = 2 * Q
        sk = 2.0 ** -rng.integers(2, 6, (B, H, 1, 128))
        K = rng.integers(-8, 8, (B, H, 1, 128)) * 0.125 + k * 0.5 * sk
    kv, V = per_token((1 << vb) - 1)
    Kt = torch.from_numpy(K.astype(np.float16)).cuda()
    Vt = torch.from_numpy(V.astype(np.float16)).cuda()
    assert np.array_equal(Kt.cpu().numpy().astype(np.float64), K)   # every value exact in fp16
    assert np.array_equal(Vt.cpu().numpy().astype(np.float64), V)
    lens = np.array([L, L - G - 2])
    cache = make_cache(w, lens)
    print("ties kb=%d vb=%d G=%d" % (kb, vb, G), flush=True)
    cache.prefill(Kt, Vt, lens)
    states = oracle_states(to_bits(Kt), to_bits(Vt), lens, w, cap=L + 256)
    # the constructed data has ties: half of the elements sit on one
    odd = (k % 2 == 1).mean()
    assert odd > 0.3
    compare_codes(cache, states)


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 32), (2, 2, 16), (4, 2, 32), (8, 8, 32)])
def test_prefill_degenerate_sets(kb, vb, G):
    """Sets whose scale is 0 or an fp16 subnormal, and signed zeros: key
    channels constant over a group (0 and -0 among them) or spanning a few
    subnormal steps; value rows (and INT8 key rows) constant, of mixed +-0,
    or of subnormals.  Codes, scales, zeros and dequantized values bit-exact
    against the oracle."""
    B, H, R = 2, 2, G
    L = 6 * G + R + 5
    w = _w("llama3_8b_layer_b8_32k_int4", name="degenerate", num_seqs=B, num_q_heads=2 * H, num_kv_heads=H,
           k_bits=kb, v_bits=vb, group_size=G, residual=R, context=L, tag=44, kv_format=1 if kb == 8 else 0)
    rng = np.random.Generator(np.random.PCG64(23))
    K = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    V = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    # fp16 subnormals: a span of 5 steps (the scale rounds to 0 or one step)
    # or of up to 399 (a subnormal scale)
    tiny = lambda shape, top=400: (rng.integers(0, top, shape) * 2.0 ** -24).astype(np.float16)
    signed_zero = lambda shape: np.where(rng.integers(0, 2, shape) == 1, np.float16(-0.0), np.float16(0.0))
    g0 = (np.arange(L) // G) * G
    K[..., 0:6] = K[:, :, g0, 0:6]              # constant over each group
    K[..., 6:10] = signed_zero((B, H, L, 4))    # +-0 only
    K[..., 10:12] = tiny((B, H, L, 2), 6)       # a few subnormal steps
    K[..., 12:14] = tiny((B, H, L, 2))
    K[..., 14:18] = (1.0 + rng.integers(0, 3, (B, H, L, 4)) * 2.0 ** -10).astype(np.float16)
    for rows, fill in ((np.arange(L) % 7 == 0, "const"), (np.arange(L) % 11 == 0, "zero"),
                       (np.arange(L) % 13 == 0, "tiny")):
        for T in ((K, V) if kb == 8 else (V,)):
            if fill == "const":
                T[:, :, rows, :] = T[:, :, rows, :1]
            elif fill == "zero":
                T[:, :, rows, :] = signed_zero((B, H, int(rows.sum()), 128))
            else:
                T[:, :, rows, :] = tiny((B, H, int(rows.sum()), 128))
    Kt = torch.from_numpy(K).cuda()
    Vt = torch.from_numpy(V).cuda()
    lens = np.array([L, L - G - 3])
    cache = make_cache(w, lens)
    print("degenerate kb=%d vb=%d G=%d" % (kb, vb, G), flush=True)
    cache.prefill(Kt, Vt, lens)
    states = oracle_states(to_bits(Kt), to_bits(Vt), lens, w, cap=L + 256)
    compare_codes(cache, states)


def _fp32_attention(q32, kh, vh, scale):
    """Attention with the logits summed in fp32 over the channels (products
    of the fp32 query and dequantized keys, rounded to fp32 one by one), the
    rest in fp64: what plain fp32 arithmetic gives on these logits."""
    lg = np.zeros((q32.shape[0], kh.shape[0]), np.float32)
    for c in range(kh.shape[1]):
        lg = lg + (q32[:, c:c + 1].astype(np.float64) * kh[None, :, c]).astype(np.float32)
    lg = lg.astype(np.float64) * np.float32(scale)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    return (p @ vh.astype(np.float64)) / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("kb,vb,gq,rope", [(2, 2, 8, 0.0), (4, 4, 4, 0.0), (4, 2, 16, 0.0), (2, 2, 8, 10000.0)])
def test_wide_range_keys_and_large_queries(kb, vb, gq, rope):
    """Key groups spanning most of the fp16 range: channel 5 holds -60000 on
    two tokens of every 32 and +60000 on the rest, so its scale is 40000
    (INT2) or 8000 (INT4), and the query's element on it (2 or 10) makes
    |q s| = 80000, beyond the largest fp16 (the fp16 products overflowed
    before the query was scaled).  Pre-RoPE keys: channels 4 and 5 both at
    +-60000, whose rotation reaches 84852; the query is 0 there, so the keys'
    fp16 parts must stay finite for the logits to.  Attention must be finite
    and match the oracle.

    Bar: max-abs 2e-3 and row cosine 0.9999 for INT2 and pre-RoPE keys.  For
    INT4 the inputs that overflowed carry a logit term of at least
    65504 * 15 / 2 = 5 10^5, whose fp32 rounding alone puts plain fp32
    attention over the same dequantized cache (logits summed in fp32)
    outside that bar on this data; these rows are held to twice the error
    of that plain fp32 attention instead (and to the bar where it is looser)."""
    B, H, G, R = 2, 2, 32, 32
    lens = np.array([600, 417])
    L = int(lens.max())
    w = _w("llama3_8b_layer_b8_32k_int4", name="wide", num_seqs=B, num_q_heads=H * gq, num_kv_heads=H, k_bits=kb,
           v_bits=vb, group_size=G, residual=R, context=L, tag=47, rope_theta=rope)
    rng = np.random.Generator(np.random.PCG64(48))
    K = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    V = (rng.standard_normal((B, H, L, 128)) * 0.25).astype(np.float16)
    wide = np.where(np.arange(L) % G < 2, np.float16(-60000.0), np.float16(60000.0))
    K[:, :, :, 5] = wide
    if rope:
        K[:, :, :, 4] = wide
    q = (rng.standard_normal((B, H * gq, 128)) * (3.0 if kb == 2 else 1.0)).astype(np.float16)
    if rope:
        q[:, :, 4:6] = 0
    else:
        q[:, :, 5] = 2.0 if kb == 2 else 10.0
    Kt, Vt, qt = (torch.from_numpy(a).cuda() for a in (K, V, q))
    cache = make_cache(w, lens)
    print("wide-range keys kb=%d vb=%d gq=%d rope=%g" % (kb, vb, gq, rope), flush=True)
    cache.prefill(Kt, Vt, lens)
    out = cache.decode_attention(qt, SCALE)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    states = oracle_states(to_bits(Kt), to_bits(Vt), lens, w, cap=L + 64)
    if not rope:
        st = states[0][0]
        assert np.array_equal(st.key_meta()[0][:, 5], np.full(st.nq // G, np.float16(120000.0 / ((1 << kb) - 1))
                                                               .view(np.uint16)))
    ref = oracle_attention(to_bits(qt), states, SCALE, rope_base=rope)
    if kb == 2:
        compare_attention(out, ref)
        return
    qf = oracle.h2f(to_bits(qt))
    for b in range(B):
        for h in range(H):
            kh, vh = states[b][h].dequantize()
            rows = slice(h * gq, (h + 1) * gq)
            plain = _fp32_attention(qf[b, rows], kh, vh, SCALE)
            r, o = ref[b, rows], out[b, rows].astype(np.float64)
            cos = lambda x: (x * r).sum(-1) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(r, axis=-1))
            tol = max(2e-3, 2 * np.abs(plain - r).max())
            assert np.abs(o - r).max() <= tol, (b, h, np.abs(o - r).max(), tol)
            assert cos(o).min() >= min(0.9999, 1 - 2 * (1 - cos(plain).min())), (b, h, cos(o).min(), cos(plain).min())


