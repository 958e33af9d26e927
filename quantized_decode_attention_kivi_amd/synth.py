"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the quantization method: it only draws
random numbers with the structure the pages describe for real K/V caches and
names the workloads.

Structure ("KV cache compression: quantization, eviction and sparse
attention", section 2.1; "KV Cache compression lab", experiment 03):
  * keys carry a few fixed outlier channels, tens of times larger than the
    rest, at the same channels for every token -> 4 seed-chosen channels per
    (layer, kv head) scaled x20 (section 3.1 of the first page uses 20x);
  * values have no channel outliers; their large entries come by token row ->
    for the long-context workloads 1% of the token rows per (sequence, kv head)
    are scaled x5;
  * everything else, and the query, is N(0, 1), cast to fp16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BASE_SEED = 0x4B495649


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    k_bits: int
    v_bits: int
    group_size: int
    residual: int
    context: int                 # tokens per sequence (max for the paged mix)
    head_dim: int = 128
    paged: bool = False
    min_context: int = 0         # paged mix: lengths uniform in [min_context, context]
    v_outlier_frac: float = 0.01
    layers: int = 1              # layers folded into the sequence axis
    tag: int = 0                 # distinguishes seeds between workloads
    kv_format: int = 0           # 0 low-bit KIVI, 1 INT8 per token, 2 FP8 E4M3 static
    rope_theta: float = 0.0      # > 0: the keys are pre-RoPE (rotated on read with this base)
    grid: int = 0                # 0 uniform levels, 1 normal-quantile codebook (low-bit format)
    sparse_keys: int = 0         # 1: dense-and-sparse keys (G kept fp16 keys per group)

    @property
    def gq(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# The five workloads the method is measured on (sizes from the task's
# statement of the problem; readings of unstated parameters are explained in
# the design notes: paged G = block size = 16 with R = 128; the full-cache
# workload uses R = 128).
WORKLOADS = {
    "single_head_1k_int2": Workload(
        "single_head_1k_int2", num_seqs=1, num_q_heads=1, num_kv_heads=1, k_bits=2, v_bits=2,
        group_size=32, residual=32, context=1024, v_outlier_frac=0.0, tag=1),
    "llama3_8b_layer_b8_32k_int4": Workload(
        "llama3_8b_layer_b8_32k_int4", num_seqs=8, num_q_heads=32, num_kv_heads=8, k_bits=4,
        v_bits=4, group_size=32, residual=128, context=32768, tag=2),
    "llama3_70b_layer_b1_128k_int2": Workload(
        "llama3_70b_layer_b1_128k_int2", num_seqs=1, num_q_heads=64, num_kv_heads=8, k_bits=2,
        v_bits=2, group_size=32, residual=128, context=131072, tag=3),
    "paged_64seq_1k_16k_k4v2": Workload(
        "paged_64seq_1k_16k_k4v2", num_seqs=64, num_q_heads=32, num_kv_heads=8, k_bits=4,
        v_bits=2, group_size=16, residual=128, context=16384, min_context=1024, paged=True, tag=4),
    "llama3_70b_cache_80l_128k_int2": Workload(
        "llama3_70b_cache_80l_128k_int2", num_seqs=80, num_q_heads=64, num_kv_heads=8, k_bits=2,
        v_bits=2, group_size=32, residual=128, context=131072, layers=80, tag=5),
}

# The 8-bit formats on the shape and data of the 8B-layer workload (same
# seeds): "KV cache compression: ...", section 3.1.
WORKLOADS_8BIT = {
    "llama3_8b_layer_b8_32k_fp8": Workload(
        "llama3_8b_layer_b8_32k_fp8", num_seqs=8, num_q_heads=32, num_kv_heads=8, k_bits=8,
        v_bits=8, group_size=32, residual=128, context=32768, tag=2, kv_format=2),
    "llama3_8b_layer_b8_32k_int8": Workload(
        "llama3_8b_layer_b8_32k_int8", num_seqs=8, num_q_heads=32, num_kv_heads=8, k_bits=8,
        v_bits=8, group_size=32, residual=128, context=32768, tag=2, kv_format=1),
}


# Pre-RoPE keys rotated on read ("KV cache compression: ...", section 3.3) on
# the 8B-layer and 70B-layer shapes and data (same seeds); base 500000 (the
# Llama-3 family's).  The generated keys are taken as the pre-RoPE keys.
WORKLOADS_ROPE = {
    "llama3_8b_layer_b8_32k_int4_prerope": Workload(
        "llama3_8b_layer_b8_32k_int4_prerope", num_seqs=8, num_q_heads=32, num_kv_heads=8, k_bits=4,
        v_bits=4, group_size=32, residual=128, context=32768, tag=2, rope_theta=500000.0),
    "llama3_70b_layer_b1_128k_int2_prerope": Workload(
        "llama3_70b_layer_b1_128k_int2_prerope", num_seqs=1, num_q_heads=64, num_kv_heads=8, k_bits=2,
        v_bits=2, group_size=32, residual=128, context=131072, tag=3, rope_theta=500000.0),
}


# The normal-quantile codebook grid ("KV cache compression: ...", section
# 3.3) on the same two shapes and data.
WORKLOADS_CODEBOOK = {
    "llama3_8b_layer_b8_32k_int4_codebook": Workload(
        "llama3_8b_layer_b8_32k_int4_codebook", num_seqs=8, num_q_heads=32, num_kv_heads=8, k_bits=4,
        v_bits=4, group_size=32, residual=128, context=32768, tag=2, grid=1),
    "llama3_70b_layer_b1_128k_int2_codebook": Workload(
        "llama3_70b_layer_b1_128k_int2_codebook", num_seqs=1, num_q_heads=64, num_kv_heads=8, k_bits=2,
        v_bits=2, group_size=32, residual=128, context=131072, tag=3, grid=1),
}

# Dense-and-sparse keys ("KV Cache compression lab", experiment 03) on the
# same two shapes and data.
WORKLOADS_SPARSE = {
    "llama3_8b_layer_b8_32k_int4_sparse": Workload(
        "llama3_8b_layer_b8_32k_int4_sparse", num_seqs=8, num_q_heads=32, num_kv_heads=8, k_bits=4,
        v_bits=4, group_size=32, residual=128, context=32768, tag=2, sparse_keys=1),
    "llama3_70b_layer_b1_128k_int2_sparse": Workload(
        "llama3_70b_layer_b1_128k_int2_sparse", num_seqs=1, num_q_heads=64, num_kv_heads=8, k_bits=2,
        v_bits=2, group_size=32, residual=128, context=131072, tag=3, sparse_keys=1),
}

_TABLES = (WORKLOADS, WORKLOADS_8BIT, WORKLOADS_ROPE, WORKLOADS_CODEBOOK, WORKLOADS_SPARSE)


def workload(name: str) -> Workload:
    """A named workload of any table."""
    for table in _TABLES:
        if name in table:
            return table[name]
    raise KeyError("unknown workload %r (known: %s)" % (name, ", ".join(k for t in _TABLES for k in t)))


def seed_for(tag: int, *parts: int) -> int:
    """Deterministic 63-bit seed for (workload tag, layer, tensor, ...)."""
    ss = np.random.SeedSequence([BASE_SEED, tag, *parts])
    return int(ss.generate_state(2, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def seq_lengths(w: Workload) -> np.ndarray:
    """Per-sequence token counts (uniform mix for the paged workload)."""
    if not w.paged and w.min_context == 0:
        return np.full(w.num_seqs, w.context, np.int32)
    rng = np.random.Generator(np.random.PCG64(seed_for(w.tag, 99)))
    return rng.integers(w.min_context, w.context + 1, size=w.num_seqs).astype(np.int32)


def outlier_channels(w: Workload, layer: int, head: int, count: int = 4) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_for(w.tag, layer, 7, head)))
    return np.sort(rng.permutation(w.head_dim)[:count])


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_kv(w: Workload, seqs=None, max_len=None, device="cpu", layer_of_seq=None,
            k_outlier=20.0, v_outlier=5.0):
    """fp16 K and V tensors [S][H][max_len][d] for the sequences `seqs`
    (default: all).  Sequence b belongs to layer layer_of_seq(b) (default:
    b // (num_seqs / layers)); its outlier channels come from that layer."""
    lens = seq_lengths(w)
    seqs = list(range(w.num_seqs)) if seqs is None else list(seqs)
    L = int(max_len if max_len is not None else max(int(lens[b]) for b in seqs))
    H, d = w.num_kv_heads, w.head_dim
    per_layer = max(1, w.num_seqs // w.layers)
    lay = layer_of_seq or (lambda b: b // per_layer)
    K = torch.empty((len(seqs), H, L, d), dtype=torch.float16, device=device)
    V = torch.empty((len(seqs), H, L, d), dtype=torch.float16, device=device)
    for i, b in enumerate(seqs):
        n = min(int(lens[b]), L)
        for h in range(H):
            g = _gen(device, seed_for(w.tag, lay(b), 1, b, h))
            kk = torch.randn((L, d), generator=g, device=device, dtype=torch.float32)
            ch = torch.as_tensor(outlier_channels(w, lay(b), h), device=device)
            kk[:, ch] *= k_outlier
            K[i, h] = kk.to(torch.float16)
            g = _gen(device, seed_for(w.tag, lay(b), 2, b, h))
            vv = torch.randn((L, d), generator=g, device=device, dtype=torch.float32)
            nrows = int(w.v_outlier_frac * n)
            if nrows > 0:
                rng = np.random.Generator(np.random.PCG64(seed_for(w.tag, lay(b), 3, b, h)))
                rows = torch.as_tensor(rng.choice(n, size=nrows, replace=False), device=device)
                vv[rows] *= v_outlier
            V[i, h] = vv.to(torch.float16)
    return K, V


def make_query(w: Workload, device="cpu", step: int = 0, seqs=None):
    """fp16 query [S][Hq][d]."""
    S = w.num_seqs if seqs is None else len(list(seqs))
    g = _gen(device, seed_for(w.tag, 0, 4, step))
    return torch.randn((S, w.num_q_heads, w.head_dim), generator=g, device=device,
                       dtype=torch.float32).to(torch.float16)


def make_tokens(w: Workload, step: int, device="cpu", k_outlier=20.0):
    """One new fp16 (k, v) token per (sequence, kv head): [B][H][d] each, with
    the same outlier channels as the cache it is appended to."""
    B, H, d = w.num_seqs, w.num_kv_heads, w.head_dim
    g = _gen(device, seed_for(w.tag, 0, 5, step))
    k = torch.randn((B, H, d), generator=g, device=device, dtype=torch.float32)
    k *= torch.as_tensor(_outlier_gain(w, k_outlier), device=device)
    v = torch.randn((B, H, d), generator=g, device=device, dtype=torch.float32)
    return k.to(torch.float16), v.to(torch.float16)


_GAIN_CACHE = {}


def _outlier_gain(w: Workload, k_outlier: float) -> np.ndarray:
    """[B][H][d] multipliers: k_outlier on each (sequence, head)'s outlier
    channels (those of the sequence's layer), 1 elsewhere."""
    key = (w, k_outlier)
    if key not in _GAIN_CACHE:
        per_layer = max(1, w.num_seqs // w.layers)
        gain = np.ones((w.num_seqs, w.num_kv_heads, w.head_dim), np.float32)
        for b in range(w.num_seqs):
            for h in range(w.num_kv_heads):
                gain[b, h, outlier_channels(w, b // per_layer, h)] = k_outlier
        _GAIN_CACHE[key] = gain
    return _GAIN_CACHE[key]


def calibrate_fp8_scales(K: torch.Tensor, V: torch.Tensor):
    """Static FP8 scales for the inputs: per kv head, the largest |value| of
    the given keys (values) over every sequence, token and channel, divided
    by 448 so that it lands on the largest E4M3 value.  This stands in for an
    offline calibration set ("KV compression and quantization", part B.3:
    static scales are fixed beforehand from calibration data); K, V:
    [S][H][L][d].  -> two float32 tensors [H] on K's device."""
    ks = K.abs().amax(dim=(0, 2, 3)).float() / 448.0
    vs = V.abs().amax(dim=(0, 2, 3)).float() / 448.0
    return ks, vs


def random_fp16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) fp16 bit patterns (numpy, for small host tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape) * scale).astype(np.float16).view(np.uint16)
