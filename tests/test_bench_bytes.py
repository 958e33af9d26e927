"""The benchmark's byte counts (the numerators of every GB/s it reports)
against the library's own record layout (kvq_buffer_sizes, the C
implementation) and against closed forms.  Host only: no kernel is called."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_decode_attention_kivi_amd import kvq, synth  # noqa: E402

ALL = [name for table in synth._TABLES for name in table]


def _record_bytes(w):
    shape = kvq.CacheShape(1, w.num_kv_heads, w.k_bits, w.v_bits, w.group_size, w.residual,
                           max_tokens=w.group_size + w.residual, kv_format=w.kv_format, grid=w.grid,
                           sparse_keys=w.sparse_keys)
    return kvq.kvq_buffer_sizes(shape.config()).record_bytes


@pytest.mark.parametrize("name", ALL)
def test_attention_bytes_are_the_records_read(name):
    """Per (sequence, kv head): its n_q / G records as laid out by the
    library, its fp16 residual keys and values; per sequence the fp16 query
    and the fp32 output."""
    w = synth.workload(name)
    lens = synth.seq_lengths(w).astype(np.int64)
    rec = _record_bytes(w)
    want = 0
    for n in lens:
        nq = kvq.num_quantized(int(n), w.group_size, w.residual)
        want += w.num_kv_heads * ((nq // w.group_size) * rec + (int(n) - nq) * 128 * 2 * 2)
        want += w.num_q_heads * 128 * (2 + 4)
    assert bench.attention_bytes(lens, w) == want


@pytest.mark.parametrize("name", ALL)
def test_prefill_bytes_are_input_plus_records(name):
    """fp16 keys and values read once; records and the fp16 residual written."""
    w = synth.workload(name)
    lens = synth.seq_lengths(w).astype(np.int64)
    rec = _record_bytes(w)
    want = 0
    for n in lens:
        nq = kvq.num_quantized(int(n), w.group_size, w.residual)
        want += w.num_kv_heads * (int(n) * 128 * 4 + (nq // w.group_size) * rec + (int(n) - nq) * 128 * 4)
    assert bench.prefill_bytes(lens, w) == want


def test_80_layer_int2_cache_closed_form():
    """80 layers x 8 kv heads x 131072 tokens, INT2 keys and values, G = 32,
    R = 128: per quantized token and head 2 x 128 x 2 / 8 = 64 code bytes,
    128 x 4 / 32 = 16 bytes of key scale/zero and 4 of value scale/zero;
    128 fp16 residual tokens of keys and values; 64 query heads per layer."""
    w = synth.workload("llama3_70b_cache_80l_128k_int2")
    lens = synth.seq_lengths(w).astype(np.int64)
    assert w.num_seqs == 80 and w.num_kv_heads == 8 and int(lens.min()) == int(lens.max()) == 131072
    nq = 131072 - 128
    want = 80 * (8 * (nq * (64 + 16 + 4) + 128 * 512) + 64 * 128 * 6)
    assert bench.attention_bytes(lens, w) == want
    assert abs(want / 1e9 - 7.09) < 0.01


@pytest.mark.parametrize("name", ALL)
def test_dequantize_bytes_are_records_and_fp32_output(name):
    """kv_dequantize of one sequence: its records and fp16 residual read (the
    attention bytes without query and output), its fp32 keys and values
    written (2 x 4 bytes per element)."""
    w = synth.workload(name)
    n = int(synth.seq_lengths(w)[0])
    rec = _record_bytes(w)
    nq = kvq.num_quantized(n, w.group_size, w.residual)
    want = w.num_kv_heads * ((nq // w.group_size) * rec + (n - nq) * 128 * 2 * 2 + n * 128 * 4 * 2)
    assert bench.dequantize_bytes(n, w) == want


def test_dequantize_bytes_closed_form_80_layer_cache():
    """One layer of one sequence of the 80-layer INT2 cache: 8 kv heads x
    (131072 - 128 quantized tokens x 84 bytes + 128 fp16 residual tokens x
    512 bytes + 131072 tokens x 1024 bytes of fp32 keys and values)."""
    w = synth.workload("llama3_70b_cache_80l_128k_int2")
    assert bench.dequantize_bytes(131072, w) == 8 * ((131072 - 128) * 84 + 128 * 512 + 131072 * 1024)
