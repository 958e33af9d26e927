"""Host-side tests of the C ABI (no GPU): the library loads and exports every
entry point include/kvq.h declares, the size queries agree with the oracle's
byte accounting of the packed format ("KV cache compression: quantization,
eviction and sparse attention", section 8.1; per-token value metadata as in
its section 3.2), and malformed arguments are rejected before anything is
enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _kvq():
    from quantized_decode_attention_kivi_amd import kvq
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"defined", "sizeof", "if", "ifdef", "extern"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["kv_quantize_prefill", "kv_append_token", "kv_dequantize", "kv_decode_attention",
              "kvq_buffer_sizes", "kv_decode_attention_workspace_bytes", "kv_export_codes"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    kvq = _kvq()
    lib = ctypes.CDLL(kvq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(kvq.EXPORTED) <= set(declared_functions())


def _cfg(kvq, **kw):
    d = dict(num_seqs=2, num_kv_heads=3, head_dim=128, k_bits=4, v_bits=2, group_size=32, residual=64,
             max_tokens=1000, block_size=0, num_blocks=0, max_blocks_per_seq=0, kv_format=0, rope_theta=0.0,
             grid=0, sparse_keys=0)
    d.update(kw)
    return kvq.kvq_config(**d)


@pytest.mark.parametrize("kb,vb,G,R,T", [(4, 4, 32, 128, 32768), (2, 2, 32, 128, 131072), (4, 2, 16, 128, 4000),
                                         (2, 4, 32, 0, 33), (4, 4, 16, 16, 15)])
def test_buffer_sizes_match_oracle_bytes(orc, kb, vb, G, R, T):
    kvq = _kvq()
    cfg = _cfg(kvq, num_seqs=3, num_kv_heads=2, k_bits=kb, v_bits=vb, group_size=G, residual=R, max_tokens=T)
    sz = kvq.kvq_buffer_sizes(cfg)
    groups = max(0, (T - R) // G)
    assert sz.groups_per_seq == groups
    assert sz.residual_slots == R + G
    # one record = the oracle's bytes of one more quantized group of G tokens
    # (codes + per-channel key pairs + per-token value pairs)
    one_group = orc.stream_bytes(R + 2 * G, 128, kb, vb, G, R) - orc.stream_bytes(R + G, 128, kb, vb, G, R)
    assert sz.record_bytes == one_group
    assert sz.packed_bytes == 3 * 2 * groups * sz.record_bytes
    assert sz.residual_bytes == 3 * 2 * (R + G) * 128 * 2
    assert sz.counter_bytes == 3 * 4
    assert sz.block_table_bytes == 0


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("G,R,T", [(32, 128, 32768), (16, 0, 4000), (16, 16, 15)])
def test_buffer_sizes_8bit_match_oracle_bytes(orc, fmt, G, R, T):
    """8-bit formats: one record = one more quantized group in the oracle's
    accounting (a byte per code; INT8 adds a per-token fp16 pair for keys
    and for values; FP8 none)."""
    kvq = _kvq()
    cfg = _cfg(kvq, num_seqs=2, num_kv_heads=3, k_bits=8, v_bits=8, group_size=G, residual=R, max_tokens=T,
               kv_format=fmt)
    sz = kvq.kvq_buffer_sizes(cfg)
    one_group = orc.stream_bytes(R + 2 * G, 128, 8, 8, G, R, fmt=fmt) - orc.stream_bytes(R + G, 128, 8, 8, G, R,
                                                                                         fmt=fmt)
    assert sz.record_bytes == one_group == G * 256 + (8 * G if fmt == 1 else 0)
    groups = max(0, (T - R) // G)
    assert sz.packed_bytes == 2 * 3 * groups * sz.record_bytes
    assert sz.residual_slots == R + G


@pytest.mark.parametrize("kw,status", [
    (dict(kv_format=1, k_bits=4, v_bits=4), "KVQ_EINVAL"),     # 8-bit formats take 8-bit codes only
    (dict(kv_format=2, k_bits=8, v_bits=4), "KVQ_EINVAL"),
    (dict(kv_format=3, k_bits=8, v_bits=8), "KVQ_EINVAL"),     # unknown format
    (dict(kv_format=-1), "KVQ_EINVAL"),
    (dict(kv_format=0, k_bits=8, v_bits=8), "KVQ_EUNSUPPORTED"),
    (dict(kv_format=1, k_bits=8, v_bits=8, group_size=64), "KVQ_EUNSUPPORTED"),
])
def test_format_validation(kw, status):
    kvq = _kvq()
    cfg = _cfg(kvq, **kw)
    out = kvq.kvq_sizes()
    assert kvq.lib().kvq_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)) == getattr(kvq, status)


@pytest.mark.skipif("not _no_gpu()", reason="argument rejection is exercised only where no kernel can launch")
def test_fp8_calls_need_static_scales():
    kvq = _kvq()
    L = kvq.lib()
    cfg = _cfg(kvq, k_bits=8, v_bits=8, kv_format=2)
    good = 0x10000
    vp = ctypes.c_void_p
    by = ctypes.byref
    no_scales = kvq.kvq_cache(good, good, good, good, good, None, None, None)
    one_scale = kvq.kvq_cache(good, good, good, good, good, None, good, None)
    odd = kvq.kvq_cache(good, good, good, good, good, None, good, good + 2)
    for c in (no_scales, one_scale, odd):
        assert L.kv_quantize_prefill(by(cfg), by(c), vp(good), vp(good), 10, vp(good), None) == kvq.KVQ_EINVAL
        assert L.kv_append_token(by(cfg), by(c), vp(good), vp(good), None) == kvq.KVQ_EINVAL
        assert L.kv_dequantize(by(cfg), by(c), vp(good), vp(good), 4, None) == kvq.KVQ_EINVAL
    # export: FP8 writes no scale/zero tables, so they may be null; INT8 needs them
    c8 = kvq.kvq_cache(good, good, good, good, good, None, None, None)
    icfg = _cfg(kvq, k_bits=8, v_bits=8, kv_format=1)
    assert L.kv_export_codes(by(icfg), by(c8), vp(good), vp(good), None, None, None, None, 32, None) == \
        kvq.KVQ_EINVAL


def test_fp8_cache_needs_scales_on_host():
    kvq = _kvq()
    shape = kvq.CacheShape(2, 3, 8, 8, 32, 64, max_tokens=300, kv_format=kvq.FORMAT_FP8_E4M3)
    with pytest.raises(ValueError):
        kvq.QuantizedKVCache(shape, device="cpu")
    c = kvq.QuantizedKVCache(shape, device="cpu", k_scale=[0.1, 0.2, 0.3], v_scale=[1.0, 2.0, 3.0])
    assert c.cache.k_scale == c.k_scale.data_ptr() and c.cache.v_scale == c.v_scale.data_ptr()
    assert c.sequence_view(1).cache.k_scale == c.cache.k_scale


@pytest.mark.parametrize("bits", [2, 4])
def test_codebook_levels_equal_oracle(orc, bits):
    """The library's normal-quantile codebook (computed on the host by its
    own quantile routine) is the oracle's, level for level."""
    kvq = _kvq()
    import numpy as np
    assert np.array_equal(kvq.kvq_codebook_levels(bits).astype(np.float64), orc.codebook_levels(bits))


@pytest.mark.parametrize("kw,status", [
    (dict(grid=2), "KVQ_EINVAL"),
    (dict(grid=-1), "KVQ_EINVAL"),
    (dict(grid=1, kv_format=1, k_bits=8, v_bits=8), "KVQ_EUNSUPPORTED"),   # low-bit format only
])
def test_grid_validation(kw, status):
    kvq = _kvq()
    cfg = _cfg(kvq, **kw)
    out = kvq.kvq_sizes()
    assert kvq.lib().kvq_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)) == getattr(kvq, status)
    bad = (ctypes.c_float * 16)()
    assert kvq.lib().kvq_codebook_levels(3, bad) == kvq.KVQ_EUNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(sparse_keys=2), "KVQ_EINVAL"),
    (dict(sparse_keys=1, kv_format=2, k_bits=8, v_bits=8), "KVQ_EUNSUPPORTED"),
    (dict(sparse_keys=1, rope_theta=10000.0), "KVQ_EUNSUPPORTED"),
])
def test_sparse_validation(kw, status):
    kvq = _kvq()
    cfg = _cfg(kvq, **kw)
    out = kvq.kvq_sizes()
    assert kvq.lib().kvq_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)) == getattr(kvq, status)


@pytest.mark.parametrize("G", [16, 32])
def test_sparse_record_size(G):
    """Dense-and-sparse keys add G (position, fp16) pairs of 4 bytes to every
    record."""
    kvq = _kvq()
    a = kvq.kvq_buffer_sizes(_cfg(kvq, group_size=G, residual=2 * G))
    b = kvq.kvq_buffer_sizes(_cfg(kvq, group_size=G, residual=2 * G, sparse_keys=1))
    assert b.record_bytes == a.record_bytes + 4 * G and b.packed_bytes == a.packed_bytes // a.record_bytes * b.record_bytes


def test_paged_sizes():
    kvq = _kvq()
    cfg = _cfg(kvq, group_size=16, residual=128, max_tokens=0, block_size=16, num_blocks=100,
               max_blocks_per_seq=20)
    sz = kvq.kvq_buffer_sizes(cfg)
    assert sz.packed_bytes == 100 * 3 * sz.record_bytes
    assert sz.block_table_bytes == 2 * 20 * 4
    assert sz.groups_per_seq == 20


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, "KVQ_EUNSUPPORTED"),
    ("k_bits", 3, "KVQ_EUNSUPPORTED"),
    ("v_bits", 8, "KVQ_EUNSUPPORTED"),
    ("group_size", 64, "KVQ_EUNSUPPORTED"),
    ("residual", 40, "KVQ_EINVAL"),    # not a multiple of G = 16
    ("residual", -32, "KVQ_EINVAL"),
    ("num_seqs", 0, "KVQ_EINVAL"),
    ("num_kv_heads", 0, "KVQ_EINVAL"),
    ("block_size", 32, "KVQ_EINVAL"),   # paged block must equal G (16 here)
])
def test_config_validation(field, value, status):
    kvq = _kvq()
    base = dict(group_size=16, residual=32)
    base[field] = value
    cfg = _cfg(kvq, **base)
    out = kvq.kvq_sizes()
    got = kvq.lib().kvq_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out))
    assert got == getattr(kvq, status)
    assert kvq.kv_decode_attention_workspace_bytes(cfg, 12) == 0


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif("not _no_gpu()", reason="argument rejection is exercised only where no kernel can launch")
def test_calls_reject_bad_arguments_before_launch():
    """Every call below is malformed in exactly one way and must return the
    validation status (the fake pointers are never dereferenced)."""
    kvq = _kvq()
    L = kvq.lib()
    cfg = _cfg(kvq)
    good = 0x10000
    cache = kvq.kvq_cache(good, good, good, good, good, None)
    vp = ctypes.c_void_p
    by = ctypes.byref
    # null cache pointer
    bad = kvq.kvq_cache(good, None, good, good, good, None)
    assert L.kv_quantize_prefill(by(cfg), by(bad), vp(good), vp(good), 10, vp(good), None) == kvq.KVQ_EINVAL
    # misaligned k (kernels use 128-bit loads)
    assert L.kv_quantize_prefill(by(cfg), by(cache), vp(good + 4), vp(good), 10, vp(good), None) == kvq.KVQ_EINVAL
    # negative max_len
    assert L.kv_quantize_prefill(by(cfg), by(cache), vp(good), vp(good), -1, vp(good), None) == kvq.KVQ_EINVAL
    # append: null token
    assert L.kv_append_token(by(cfg), by(cache), None, vp(good), None) == kvq.KVQ_EINVAL
    # dequantize: negative token count
    assert L.kv_dequantize(by(cfg), by(cache), vp(good), vp(good), -5, None) == kvq.KVQ_EINVAL
    # attention: Hq not a multiple of H, too many query heads per kv head, tiny workspace
    ws = kvq.kv_decode_attention_workspace_bytes(cfg, 6)
    assert ws > 0
    assert L.kv_decode_attention(by(cfg), by(cache), vp(good), 7, ctypes.c_float(0.088), vp(good), vp(good),
                                 ws, None) == kvq.KVQ_EINVAL
    assert L.kv_decode_attention(by(cfg), by(cache), vp(good), 3 * 17, ctypes.c_float(0.088), vp(good),
                                 vp(good), 10 ** 9, None) == kvq.KVQ_EUNSUPPORTED
    assert L.kv_decode_attention(by(cfg), by(cache), vp(good), 6, ctypes.c_float(0.088), vp(good), vp(good),
                                 ws - 1, None) == kvq.KVQ_ECAPACITY
    assert L.kv_decode_attention(by(cfg), by(cache), vp(good), 6, ctypes.c_float(-1.0), vp(good), vp(good),
                                 ws, None) == kvq.KVQ_EINVAL
    # export: token count not a multiple of G
    assert L.kv_export_codes(by(cfg), by(cache), *[vp(good)] * 6, 33, None) == kvq.KVQ_EINVAL
    # paged cache without block table
    pcfg = _cfg(kvq, group_size=16, residual=32, max_tokens=0, block_size=16, num_blocks=8, max_blocks_per_seq=4)
    assert L.kv_append_token(by(pcfg), by(cache), vp(good), vp(good), None) == kvq.KVQ_EINVAL
    assert L.kvq_status_string(kvq.KVQ_ECAPACITY).decode() == "buffer or workspace too small"


def test_noalloc_rejects_oversized_calls_before_any_device_work():
    """The no-allocation entry point checks the scratch its partials need
    against its fixed array on the host: an oversized batch is refused with
    KVQ_ECAPACITY and both sizes in the error text (no device is touched:
    this runs on a machine without a GPU); a malformed call is refused as by
    kv_decode_attention."""
    kvq = _kvq()
    L = kvq.lib()
    good = 0x10000
    cache = kvq.kvq_cache(good, good, good, good, good, None)
    vp, by = ctypes.c_void_p, ctypes.byref
    cfg = _cfg(kvq, num_seqs=4096, num_kv_heads=8, max_tokens=4096)
    need = kvq.kv_decode_attention_workspace_bytes(cfg, 128)
    assert need > 16 << 20
    st = L.kv_decode_attention_noalloc(by(cfg), by(cache), vp(good), 128, ctypes.c_float(0.088), vp(good), None)
    assert st == kvq.KVQ_ECAPACITY
    msg = L.kvq_last_error().decode()
    assert str(need) in msg and str(16 << 20) in msg
    small = _cfg(kvq)
    assert L.kv_decode_attention_noalloc(by(small), by(cache), vp(good), 7, ctypes.c_float(0.088), vp(good),
                                         None) == kvq.KVQ_EINVAL
    assert L.kv_decode_attention_noalloc(by(small), by(cache), vp(good), 6, ctypes.c_float(0.088), None,
                                         None) == kvq.KVQ_EINVAL


@pytest.mark.parametrize("paged", [False, True])
def test_sequence_view_offsets(paged):
    """A sequence view is the one-sequence cache at fixed offsets of the
    parent's buffers (host tensors here; no kernel is called)."""
    kvq = _kvq()
    if paged:
        shape = kvq.CacheShape(5, 3, 4, 2, 16, 32, paged=True, num_blocks=40, max_blocks_per_seq=9)
    else:
        shape = kvq.CacheShape(5, 3, 4, 2, 32, 64, max_tokens=700)
    c = kvq.QuantizedKVCache(shape, device="cpu")
    one = kvq.kvq_buffer_sizes(kvq.CacheShape(**{**shape.__dict__, "num_seqs": 1}).config())
    for b in (0, 2, 4):
        v = c.sequence_view(b)
        assert v.cfg.num_seqs == 1
        if paged:
            assert v.cache.packed == c.cache.packed
            assert v.cache.block_table == c.cache.block_table + b * shape.max_blocks_per_seq * 4
        else:
            assert v.cache.packed == c.cache.packed + b * one.packed_bytes
        assert v.cache.k_res == c.cache.k_res + b * one.residual_bytes
        assert v.cache.v_res == c.cache.v_res + b * one.residual_bytes
        assert v.cache.n_tokens == c.cache.n_tokens + 4 * b
        assert v.cache.n_quant == c.cache.n_quant + 4 * b
    with pytest.raises(kvq.KVQError):
        c.sequence_view(1).append(None, None)
    with pytest.raises(IndexError):
        c.sequence_view(5)


def test_prefill_block_assignment():
    """Paged prefill hands the whole pool out again, sequence by sequence, in
    the pool's order: the same table as taking blocks one at a time from a
    fresh free list; the table is rewritten only when it changes; appends
    continue from what is left (host bookkeeping only, no kernel)."""
    kvq = _kvq()
    G, R = 16, 32
    shape = kvq.CacheShape(4, 2, 4, 2, G, R, paged=True, num_blocks=60, max_blocks_per_seq=20)
    c = kvq.QuantizedKVCache(shape, device="cpu")
    c.shuffle_free_blocks(7)
    for lens in ([300, 47, 0, 200], [40, 300, 200, 17], [0, 0, 0, 0]):
        lens = np.array(lens)
        c._prefill_blocks(lens)
        free = list(c._block_order)
        want = np.full((4, 20), -1, np.int32)
        for b, n in enumerate(lens):
            for i in range(kvq.num_quantized(int(n), G, R) // G):
                want[b, i] = free.pop()
        assert np.array_equal(c._bt_host, want)
        assert np.array_equal(c.block_table.numpy(), want)
        assert c._free == free
    # unchanged table: no rewrite (the device copy is left alone)
    lens = np.array([300, 47, 0, 200])
    c._prefill_blocks(lens)
    c.block_table.fill_(-5)
    c._prefill_blocks(lens)
    assert int(c.block_table.min()) == -5
    # an append that crosses a group boundary takes the next free block
    c.block_table.copy_(torch.from_numpy(c._bt_host))
    nxt = c._free[-1]
    grow = lens.copy()
    grow[2] = R + G   # sequence 2's first group becomes full
    c._ensure_blocks(grow)
    assert c._bt_host[2, 0] == nxt and c.block_table[2, 0] == nxt
    assert np.array_equal(c.block_table.numpy(), c._bt_host)
    # several sequences, several groups at once: the next blocks in pool
    # order, in sequence order, and only those entries are written
    free = list(c._free)
    c.block_table[c.block_table < 0] = -7          # marks the entries that must stay unwritten
    before = c.block_table.clone()
    grow2 = grow + np.array([16, 0, 3 * G, 2 * G])
    c._ensure_blocks(grow2)
    want = {}
    for b, n in enumerate(grow2):
        for g in range(int(np.count_nonzero(before[b].numpy() >= 0)), kvq.num_quantized(int(n), G, R) // G):
            want[(b, g)] = free.pop()
    assert c._free == free and len(want) == 6   # 1 + 3 + 2 new groups
    tab = c.block_table.numpy()
    for (b, g), blk in want.items():
        assert tab[b, g] == blk and c._bt_host[b, g] == blk
    untouched = np.ones(tab.shape, bool)
    for (b, g) in want:
        untouched[b, g] = False
    assert np.array_equal(tab[untouched], before.numpy()[untouched])
    with pytest.raises(kvq.KVQError):
        c._prefill_blocks(np.array([340, 340, 340, 340]))   # 19 blocks each > 60 in the pool
