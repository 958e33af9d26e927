"""A decode step captured in a HIP graph: kv_append_token then
kv_decode_attention (and the no-allocation form), recorded once with
torch.cuda.graph and replayed step after step.  The library enqueues kernels
only (no memset, copy or allocation on the stream), so the captured step is
the eager step; every replay is checked against the same calls made eagerly
on a second cache built from the same tokens: outputs and, at the end, the
caches' codes, scales and zeros bit for bit.  Between replays the program
does its own eager work (new token and query rows copied into the captured
buffers, the eager step, a synchronisation).  Paged caches get their blocks
for all the steps before the capture, since handing out a block is host
work."""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_decode_attention_kivi_amd import kvq, synth
from parity_util import make_cache

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


def _w(base, **kw):
    return dataclasses.replace(synth.WORKLOADS[base], **kw)


CASES = {
    "gqa8_int2": _w("llama3_70b_layer_b1_128k_int2", num_seqs=2, context=700 + 5),
    "gqa4_int4_g32_r64": _w("llama3_8b_layer_b8_32k_int4", name="gr", num_seqs=3, context=640 + 19, residual=64,
                             tag=31),
    "paged_k4v2_g16": _w("paged_64seq_1k_16k_k4v2", name="gpg", num_seqs=3, context=500, min_context=150, tag=32),
}


def _step_rows(K, V, lens):
    kn = torch.stack([K[b, :, int(lens[b])] for b in range(len(lens))]).contiguous()
    vn = torch.stack([V[b, :, int(lens[b])] for b in range(len(lens))]).contiguous()
    return kn, vn


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("case", list(CASES))
def test_decode_step_graph_replays_equal_eager(case, noalloc):
    w = CASES[case]
    steps = w.group_size + 9          # crosses a group flush
    lens0 = synth.seq_lengths(w).astype(np.int64)
    L = int(lens0.max()) + steps
    K, V = synth.make_kv(w, max_len=L, device="cuda")
    caches = []
    for _ in range(2):
        c = make_cache(w, lens0 + steps + 1, max_tokens=L + 8, shuffle_seed=3)
        c.prefill(K[:, :, :int(lens0.max())].contiguous(), V[:, :, :int(lens0.max())].contiguous(), lens0)
        c._ensure_blocks(lens0 + steps)   # every block the steps will need, handed out now (paged)
        caches.append(c)
    eager, graphed = caches
    Hq = w.num_q_heads
    kn = torch.empty((w.num_seqs, w.num_kv_heads, 128), dtype=torch.float16, device="cuda")
    vn = torch.empty_like(kn)
    q = torch.empty((w.num_seqs, Hq, 128), dtype=torch.float16, device="cuda")
    out_g = torch.empty((w.num_seqs, Hq, 128), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)
    ws_g = graphed.workspace(Hq)
    ws_e = eager.workspace(Hq)
    q.zero_()
    torch.cuda.synchronize()

    def attend(cache, ws, out):
        if noalloc:
            kvq.kv_decode_attention_noalloc(cache.cfg, cache.cache, q, Hq, SCALE, out)
        else:
            kvq.kv_decode_attention(cache.cfg, cache.cache, q, Hq, SCALE, out, ws)

    def step(cache, ws, out):
        kvq.kv_append_token(cache.cfg, cache.cache, kn, vn)
        attend(cache, ws, out)

    # one eager call first: the library's one-time set-up per device (the
    # scratch array's address, the device's CU count) stays out of the capture
    attend(eager, ws_e, out_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graphed, ws_g, out_g)
    torch.cuda.synchronize()
    lens = lens0.copy()
    print("graph %s noalloc=%s B=%d lens=%s steps=%d" % (case, noalloc, w.num_seqs, list(lens0), steps), flush=True)
    for s in range(steps):
        a, b = _step_rows(K, V, lens)
        kn.copy_(a)
        vn.copy_(b)
        q.copy_(synth.make_query(w, device="cuda", step=s))
        step(eager, ws_e, out_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d differs from the eager step" % s
        lens += 1
    for t_e, t_g in zip(eager.export_codes(L), graphed.export_codes(L)):
        if t_e is not None:
            assert torch.equal(t_e, t_g)
    assert torch.equal(eager.n_tokens, graphed.n_tokens) and torch.equal(eager.n_quant, graphed.n_quant)
    assert np.array_equal(graphed.n_tokens.cpu().numpy(), lens)
