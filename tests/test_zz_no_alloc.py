"""kv_decode_attention_noalloc (partials in the library's fixed device
scratch, nothing allocated) against kv_decode_attention with a caller
workspace: the same kernels and the same split, so the outputs must be
identical bit for bit.  Two calls in a row, the second on a smaller cache
(fewer sequences and tokens), so the second reuses the array the first left
behind; then a paged batch."""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_decode_attention_kivi_amd import kvq, synth
from parity_util import make_cache

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


def _compare(w, lens, step):
    lens = np.asarray(lens, np.int64)
    L = int(lens.max())
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    cache = make_cache(w, lens, shuffle_seed=3)
    print("noalloc %s B=%d lens=%s" % (w.name, w.num_seqs, list(lens)[:6]), flush=True)
    cache.prefill(K, V, lens)
    q = synth.make_query(w, device="cuda", step=step)
    ref = cache.decode_attention(q, SCALE)
    out = torch.full_like(ref, float("nan"))
    kvq.kv_decode_attention_noalloc(cache.cfg, cache.cache, q, w.num_q_heads, SCALE, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.isfinite(out).all()


def test_noalloc_equals_workspace_call_twice_then_smaller():
    big = dataclasses.replace(synth.WORKLOADS["llama3_70b_layer_b1_128k_int2"], name="na_big", num_seqs=4,
                              context=20000 + 17, tag=61)
    _compare(big, [20017, 9000, 131, 15000], 0)
    small = dataclasses.replace(synth.WORKLOADS["llama3_8b_layer_b8_32k_int4"], name="na_small", num_seqs=2,
                                context=1500, tag=62)
    _compare(small, [1500, 700], 1)


def test_noalloc_paged_and_full_8b_layer():
    _compare(synth.WORKLOADS["llama3_8b_layer_b8_32k_int4"], synth.seq_lengths(synth.WORKLOADS[
        "llama3_8b_layer_b8_32k_int4"]), 2)
    w = dataclasses.replace(synth.WORKLOADS["paged_64seq_1k_16k_k4v2"], name="na_paged", num_seqs=6, context=3000,
                            min_context=100, tag=63)
    _compare(w, synth.seq_lengths(w), 3)
