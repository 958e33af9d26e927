"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run
the oracle on the same seeded inputs, compare.

The bar: codes, scales, zeros and dequantized values bit-exact; attention
within max-abs 2e-3 of the oracle (fp64) with per-row cosine >= 0.9999.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from quantized_decode_attention_kivi_amd import kvq, synth

ATOL = 2e-3
MIN_COS = 0.9999
THREADS = min(16, os.cpu_count() or 1)


def make_cache(w: synth.Workload, lens, max_tokens=None, num_blocks=None, shuffle_seed=None, scales=None):
    """scales: FP8 format, the (k_scale, v_scale) pair of per-head tensors.
    w.rope_theta > 0: the keys are pre-RoPE and attention rotates them."""
    G, R = w.group_size, w.residual
    if w.paged:
        mb = max(1, (int(np.max(lens)) + 64 - R) // G + 1)
        onwrite = w.kv_format != kvq.FORMAT_KIVI and R == 0
        nb = num_blocks if num_blocks is not None else int(sum(kvq.groups_held(int(n) + 64, G, R, onwrite)
                                                               for n in lens)) + 4
        shape = kvq.CacheShape(w.num_seqs, w.num_kv_heads, w.k_bits, w.v_bits, G, R, paged=True,
                               num_blocks=nb, max_blocks_per_seq=mb, kv_format=w.kv_format,
                               rope_theta=w.rope_theta, grid=w.grid,
                               sparse_keys=w.sparse_keys)
    else:
        shape = kvq.CacheShape(w.num_seqs, w.num_kv_heads, w.k_bits, w.v_bits, G, R,
                               max_tokens=max_tokens if max_tokens is not None else int(np.max(lens)) + 64,
                               kv_format=w.kv_format, rope_theta=w.rope_theta, grid=w.grid,
                               sparse_keys=w.sparse_keys)
    ks, vs = scales if scales is not None else (None, None)
    c = kvq.QuantizedKVCache(shape, k_scale=ks, v_scale=vs)
    if w.paged and shuffle_seed is not None:
        c.shuffle_free_blocks(shuffle_seed)
    return c


def oracle_states(kb: np.ndarray, vb: np.ndarray, lens, w: synth.Workload, cap=None, scales=None):
    """kb, vb: uint16 [B][H][L][d] -> StreamState per (b, h).  scales: FP8
    format, the per-head (k_scale, v_scale) tensors the cache was given."""
    ks = vs = None
    if scales is not None:
        ks, vs = (t.detach().cpu().numpy().astype(np.float32) for t in scales)
    return oracle.prefill_batch(kb, vb, lens, w.k_bits, w.v_bits, w.group_size, w.residual,
                                cap=cap, threads=THREADS, fmt=w.kv_format, kscales=ks, vscales=vs, grid=w.grid,
                                sparse=bool(w.sparse_keys))


def _compare_exported(view, hix, states_of_heads, b):
    """Exports view (a one-sequence cache) and compares its heads hix[i]
    with states_of_heads[i]."""
    G = view.G
    T = int(view.lens.max()) + G     # a group past the end: must read back as zeros
    fmt = view.shape.kv_format
    kc, vc, ks, kz, vs, vz = [None if t is None else t[0].cpu().numpy() for t in view.export_codes(T)]
    if fmt != kvq.FORMAT_FP8_E4M3:
        ks, kz, vs, vz = (a.view(np.uint16) for a in (ks, kz, vs, vz))
    kd, vd = [t[0].cpu().numpy() for t in view.dequantize(T)]
    nt = int(view.n_tokens.cpu()[0])
    nqs = int(view.n_quant.cpu()[0])
    if view.shape.sparse_keys:
        opos, oval = [t[0].cpu().numpy().view(np.uint16) for t in view.export_outliers(T)]
    for h, st in zip(hix, states_of_heads):
        assert nt == st.n and nqs == st.nq, (b, nt, st.n, nqs, st.nq)
        nq, n = st.nq, st.n
        assert np.array_equal(kc[h, :nq], st.key_codes()), ("key codes", b, h)
        assert np.array_equal(vc[h, :nq], st.value_codes()), ("value codes", b, h)
        if fmt != kvq.FORMAT_FP8_E4M3:
            nk = nq // G if fmt == kvq.FORMAT_KIVI else nq   # per group or per token
            oks, okz = st.key_meta()
            assert np.array_equal(ks[h, :nk], oks), ("key scales", b, h)
            assert np.array_equal(kz[h, :nk], okz), ("key zeros", b, h)
            ovs, ovz = st.value_meta()
            assert np.array_equal(vs[h, :nq], ovs), ("value scales", b, h)
            assert np.array_equal(vz[h, :nq], ovz), ("value zeros", b, h)
        if view.shape.sparse_keys:
            sp, sv = st.outliers()
            assert np.array_equal(opos[h, :nq // G], sp), ("kept key positions", b, h)
            assert np.array_equal(oval[h, :nq // G], sv), ("kept key values", b, h)
            assert not opos[h, nq // G:].any() and not oval[h, nq // G:].any()
        okd, ovd = st.dequantize()
        assert np.array_equal(kd[h, :n], okd), ("dequantized keys", b, h)
        assert np.array_equal(vd[h, :n], ovd), ("dequantized values", b, h)
        assert np.all(kd[h, n:] == 0) and np.all(vd[h, n:] == 0)


def compare_codes(cache: kvq.QuantizedKVCache, states, streams=None):
    """Bit-exact comparison of codes, scales, zeros and dequantized values of
    the (b, h) streams (default: all), exported one sequence at a time through
    read-only sequence views of the cache."""
    torch.cuda.synchronize()
    B, H = cache.shape.num_seqs, cache.shape.num_kv_heads
    streams = streams if streams is not None else [(b, h) for b in range(B) for h in range(H)]
    by_seq = {}
    for b, h in streams:
        by_seq.setdefault(b, []).append(h)
    for b, heads in sorted(by_seq.items()):
        _compare_exported(cache.sequence_view(b), heads, [states[b][h] for h in heads], b)


def compare_stream_codes(cache: kvq.QuantizedKVCache, b: int, h: int, st):
    """compare_codes for one stream of a contiguous cache, exported through a
    one-stream view (only that stream's bytes leave the device)."""
    torch.cuda.synchronize()
    _compare_exported(cache.stream_view(b, h), [0], [st], b)


def oracle_attention(q16: np.ndarray, states, scale, rows=None, rope_base=0.0):
    """q16: uint16 fp16 bits [B][Hq][d] -> fp64 [B][Hq][d] (rows: list of
    (b, hq) to compute, others NaN).  rope_base > 0: pre-RoPE keys rotated on
    read."""
    qf = oracle.h2f(q16)
    B, Hq, d = qf.shape
    H = len(states[0])
    gq = Hq // H
    out = np.full((B, Hq, d), np.nan)
    if rows is None:
        return oracle.decode_attention_batch(qf, states, scale, threads=THREADS, rope_base=rope_base)
    from concurrent.futures import ThreadPoolExecutor
    by_stream = {}
    for b, hq in rows:
        by_stream.setdefault((b, hq // gq), []).append(hq)

    def one(item):
        (b, h), hqs = item
        kh, vh = states[b][h].dequantize()
        o = oracle.attention_rope(qf[b, hqs], kh, vh, scale, rope_base) if rope_base > 0 \
            else oracle.attention(qf[b, hqs], kh, vh, scale)
        for i, hq in enumerate(hqs):
            out[b, hq] = o[i]

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, by_stream.items()))
    return out


def compare_attention(got: np.ndarray, ref: np.ndarray, rows=None):
    got = got.astype(np.float64)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        got, ref = got[idx], ref[idx]
    else:
        got = got.reshape(-1, got.shape[-1])
        ref = ref.reshape(-1, ref.shape[-1])
    err = np.abs(got - ref).max()
    ng = np.linalg.norm(got, axis=-1)
    nr = np.linalg.norm(ref, axis=-1)
    both_zero = (ng == 0) & (nr == 0)
    cos = np.where(both_zero, 1.0, (got * ref).sum(-1) / np.maximum(ng * nr, 1e-300))
    assert err <= ATOL, "max abs error %.3g > %.1g" % (err, ATOL)
    assert cos.min() >= MIN_COS, "min row cosine %.8f < %.4f" % (cos.min(), MIN_COS)
    return err, float(cos.min())


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)
