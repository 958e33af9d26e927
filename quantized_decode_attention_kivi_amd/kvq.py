"""ctypes binding of libkvq (the C ABI in include/kvq.h).

Argument marshalling only: the functions below carry the C names, turn torch
tensors into device pointers and the current HIP stream into a void*, and
raise on a non-OK status.  Every step of the computation runs in the HIP
kernels of libkvq.so; if the library is not built, loading fails loudly --
there is no fallback.

`QuantizedKVCache` allocates the caller-owned buffers with torch (device
memory and streams are all torch provides here) and keeps the host-side copy
of the per-sequence token counts that argument validation needs.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")
_lib = None

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ECAPACITY, KVQ_EHIP = range(5)
HEAD_DIM = 128
# cache formats (KVQ_FORMAT_*) and level grids (KVQ_GRID_*)
FORMAT_KIVI, FORMAT_INT8, FORMAT_FP8_E4M3 = 0, 1, 2
GRID_UNIFORM, GRID_NORMAL_QUANTILE = 0, 1


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_kv_heads", "head_dim", "k_bits", "v_bits", "group_size", "residual",
        "max_tokens", "block_size", "num_blocks", "max_blocks_per_seq", "kv_format")] + \
        [("rope_theta", ctypes.c_float), ("grid", ctypes.c_int32), ("sparse_keys", ctypes.c_int32)]


class kvq_cache(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
                ("n_tokens", ctypes.c_void_p), ("n_quant", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("arrivals", ctypes.c_void_p)]


class kvq_sizes(ctypes.Structure):
    _fields_ = [("packed_bytes", ctypes.c_size_t), ("record_bytes", ctypes.c_size_t),
                ("residual_bytes", ctypes.c_size_t), ("counter_bytes", ctypes.c_size_t),
                ("block_table_bytes", ctypes.c_size_t), ("groups_per_seq", ctypes.c_int32),
                ("residual_slots", ctypes.c_int32)]


EXPORTED = ["kvq_buffer_sizes", "kv_quantize_prefill", "kv_append_token", "kv_dequantize",
            "kv_decode_attention_workspace_bytes", "kv_decode_attention", "kv_decode_attention_partials",
            "kv_decode_attention_merge", "kv_decode_attention_noalloc", "kv_export_codes", "kv_export_outliers", "kvq_codebook_levels",
            "kvq_status_string",
            "kvq_last_error"]


class KVQError(RuntimeError):
    def __init__(self, status, where):
        msg = "%s: %s" % (where, lib().kvq_status_string(status).decode())
        if status == KVQ_EHIP:
            msg += " (" + lib().kvq_last_error().decode() + ")"
        super().__init__(msg)
        self.status = status


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        L.kvq_buffer_sizes.argtypes = [P(kvq_config), P(kvq_sizes)]
        L.kvq_buffer_sizes.restype = ctypes.c_int
        L.kv_quantize_prefill.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, ctypes.c_int32, vp, vp]
        L.kv_quantize_prefill.restype = ctypes.c_int
        L.kv_append_token.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, vp]
        L.kv_append_token.restype = ctypes.c_int
        L.kv_dequantize.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, ctypes.c_int32, vp]
        L.kv_dequantize.restype = ctypes.c_int
        L.kv_decode_attention_workspace_bytes.argtypes = [P(kvq_config), ctypes.c_int32]
        L.kv_decode_attention_workspace_bytes.restype = ctypes.c_size_t
        L.kv_decode_attention.argtypes = [P(kvq_config), P(kvq_cache), vp, ctypes.c_int32, ctypes.c_float,
                                          vp, vp, ctypes.c_size_t, vp]
        L.kv_decode_attention.restype = ctypes.c_int
        L.kv_decode_attention_partials.argtypes = [P(kvq_config), P(kvq_cache), vp, ctypes.c_int32, ctypes.c_float,
                                                   vp, ctypes.c_size_t, vp]
        L.kv_decode_attention_partials.restype = ctypes.c_int
        L.kv_decode_attention_merge.argtypes = [P(kvq_config), P(kvq_cache), ctypes.c_int32, vp, ctypes.c_size_t,
                                                vp, vp]
        L.kv_decode_attention_merge.restype = ctypes.c_int
        L.kv_decode_attention_noalloc.argtypes = [P(kvq_config), P(kvq_cache), vp, ctypes.c_int32, ctypes.c_float,
                                                  vp, vp]
        L.kv_decode_attention_noalloc.restype = ctypes.c_int
        L.kv_export_codes.argtypes = [P(kvq_config), P(kvq_cache)] + [vp] * 6 + [ctypes.c_int32, vp]
        L.kv_export_codes.restype = ctypes.c_int
        L.kv_export_outliers.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, ctypes.c_int32, vp]
        L.kv_export_outliers.restype = ctypes.c_int
        L.kvq_codebook_levels.argtypes = [ctypes.c_int32, P(ctypes.c_float)]
        L.kvq_codebook_levels.restype = ctypes.c_int
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != KVQ_OK:
        raise KVQError(status, where)


# ---------------------------------------------------------------------------
# C-ABI functions, same names
# ---------------------------------------------------------------------------

def kvq_buffer_sizes(cfg: kvq_config) -> kvq_sizes:
    out = kvq_sizes()
    _check(lib().kvq_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)), "kvq_buffer_sizes")
    return out


def kv_quantize_prefill(cfg, cache, k, v, max_len, seq_lens, stream=None):
    _check(lib().kv_quantize_prefill(ctypes.byref(cfg), ctypes.byref(cache), _ptr(k), _ptr(v), int(max_len),
                                     _ptr(seq_lens), _stream(stream)), "kv_quantize_prefill")


def kv_append_token(cfg, cache, k_new, v_new, stream=None):
    _check(lib().kv_append_token(ctypes.byref(cfg), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
                                 _stream(stream)), "kv_append_token")


def kv_dequantize(cfg, cache, k_out, v_out, out_tokens, stream=None):
    _check(lib().kv_dequantize(ctypes.byref(cfg), ctypes.byref(cache), _ptr(k_out), _ptr(v_out),
                               int(out_tokens), _stream(stream)), "kv_dequantize")


def kv_decode_attention_workspace_bytes(cfg, num_q_heads) -> int:
    return int(lib().kv_decode_attention_workspace_bytes(ctypes.byref(cfg), int(num_q_heads)))


def kv_decode_attention(cfg, cache, q, num_q_heads, softmax_scale, out, workspace, stream=None):
    _check(lib().kv_decode_attention(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q), int(num_q_heads),
                                     ctypes.c_float(softmax_scale), _ptr(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "kv_decode_attention")


def kv_decode_attention_partials(cfg, cache, q, num_q_heads, softmax_scale, workspace, stream=None):
    _check(lib().kv_decode_attention_partials(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q), int(num_q_heads),
                                              ctypes.c_float(softmax_scale), _ptr(workspace),
                                              workspace.numel() * workspace.element_size(), _stream(stream)),
           "kv_decode_attention_partials")


def kv_decode_attention_merge(cfg, cache, num_q_heads, workspace, out, stream=None):
    _check(lib().kv_decode_attention_merge(ctypes.byref(cfg), ctypes.byref(cache), int(num_q_heads), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _ptr(out),
                                           _stream(stream)), "kv_decode_attention_merge")


def kv_decode_attention_noalloc(cfg, cache, q, num_q_heads, softmax_scale, out, stream=None):
    _check(lib().kv_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q), int(num_q_heads),
                                             ctypes.c_float(softmax_scale), _ptr(out), _stream(stream)),
           "kv_decode_attention_noalloc")


def kv_export_codes(cfg, cache, k_codes, v_codes, k_s, k_z, v_s, v_z, out_tokens, stream=None):
    _check(lib().kv_export_codes(ctypes.byref(cfg), ctypes.byref(cache), _ptr(k_codes), _ptr(v_codes),
                                 _ptr(k_s), _ptr(k_z), _ptr(v_s), _ptr(v_z), int(out_tokens),
                                 _stream(stream)), "kv_export_codes")


def kv_export_outliers(cfg, cache, pos, val, out_tokens, stream=None):
    _check(lib().kv_export_outliers(ctypes.byref(cfg), ctypes.byref(cache), _ptr(pos), _ptr(val), int(out_tokens),
                                    _stream(stream)), "kv_export_outliers")


def kvq_codebook_levels(bits) -> np.ndarray:
    out = (ctypes.c_float * (1 << int(bits)))()
    _check(lib().kvq_codebook_levels(int(bits), out), "kvq_codebook_levels")
    return np.array(out[:], np.float32)


# ---------------------------------------------------------------------------
# Buffer owner
# ---------------------------------------------------------------------------

def num_quantized(n, G, R, onwrite=False):
    """Quantized tokens of a sequence holding n: whole groups outside the
    newest R tokens; every token when quantized on write (8-bit formats with
    R = 0)."""
    if onwrite:
        return max(int(n), 0)
    return 0 if n <= R else G * ((n - R) // G)


def groups_held(n, G, R, onwrite=False):
    """Key groups (records, paged blocks) a sequence holding n uses."""
    return -(-num_quantized(n, G, R, onwrite) // G)


@dataclass
class CacheShape:
    num_seqs: int
    num_kv_heads: int
    k_bits: int
    v_bits: int
    group_size: int
    residual: int
    max_tokens: int = 0
    paged: bool = False
    num_blocks: int = 0
    max_blocks_per_seq: int = 0
    kv_format: int = FORMAT_KIVI
    rope_theta: float = 0.0      # > 0: keys are pre-RoPE, rotated on read with this base
    grid: int = 0                # GRID_UNIFORM or GRID_NORMAL_QUANTILE (low-bit format)
    sparse_keys: int = 0         # 1: dense-and-sparse keys (G kept fp16 keys per group)

    def config(self) -> kvq_config:
        return kvq_config(self.num_seqs, self.num_kv_heads, HEAD_DIM, self.k_bits, self.v_bits,
                          self.group_size, self.residual, self.max_tokens if not self.paged else 0,
                          self.group_size if self.paged else 0, self.num_blocks, self.max_blocks_per_seq,
                          self.kv_format, self.rope_theta, self.grid, self.sparse_keys)


class QuantizedKVCache:
    """Device buffers of one quantized cache plus host-side bookkeeping of the
    token counts (used only to validate calls and size exports).  In paged
    mode a simple host free-list hands out blocks ahead of the device flushes."""

    def __init__(self, shape: CacheShape, device="cuda", k_scale=None, v_scale=None):
        """k_scale, v_scale: FP8 format only, the static per-kv-head scales
        (float sequences or tensors of H positive values)."""
        self.shape = shape
        self.cfg = shape.config()
        self.sizes = kvq_buffer_sizes(self.cfg)
        self.device = torch.device(device)
        sz = self.sizes
        self.packed = torch.empty(max(sz.packed_bytes, 16), dtype=torch.uint8, device=self.device)
        self.k_res = torch.zeros(sz.residual_bytes // 2, dtype=torch.float16, device=self.device)
        self.v_res = torch.zeros(sz.residual_bytes // 2, dtype=torch.float16, device=self.device)
        self.n_tokens = torch.zeros(shape.num_seqs, dtype=torch.int32, device=self.device)
        self.n_quant = torch.zeros(shape.num_seqs, dtype=torch.int32, device=self.device)
        # per-sequence arrival counters of the append kernel (kept zero by the library)
        self.arrivals = torch.zeros(shape.num_seqs, dtype=torch.int32, device=self.device)
        self.block_table = None
        if shape.paged:
            self.block_table = torch.full((shape.num_seqs, shape.max_blocks_per_seq), -1, dtype=torch.int32,
                                          device=self.device)
            self._bt_host = np.full((shape.num_seqs, shape.max_blocks_per_seq), -1, np.int32)
            self._block_order = list(range(shape.num_blocks - 1, -1, -1))  # pop() hands out 0, 1, 2, ...
            self._free = list(self._block_order)
            self._nblk = np.zeros(shape.num_seqs, np.int64)   # blocks held per sequence (table prefix)
        self.lens = np.zeros(shape.num_seqs, np.int64)
        self.k_scale = self.v_scale = None
        if shape.kv_format == FORMAT_FP8_E4M3:
            if k_scale is None or v_scale is None:
                raise ValueError("the FP8 format needs static k_scale and v_scale per kv head")
            H = shape.num_kv_heads
            self.k_scale = torch.as_tensor(k_scale, dtype=torch.float32).reshape(H).to(self.device).contiguous()
            self.v_scale = torch.as_tensor(v_scale, dtype=torch.float32).reshape(H).to(self.device).contiguous()
        self.cache = self._make_cache()
        self._ws = None

    def _make_cache(self):
        return kvq_cache(self.packed.data_ptr(), self.k_res.data_ptr(), self.v_res.data_ptr(),
                         self.n_tokens.data_ptr(), self.n_quant.data_ptr(),
                         self.block_table.data_ptr() if self.block_table is not None else None,
                         self.k_scale.data_ptr() if self.k_scale is not None else None,
                         self.v_scale.data_ptr() if self.v_scale is not None else None,
                         self.arrivals.data_ptr())

    def sequence_view(self, b: int) -> "QuantizedKVCache":
        """Read-only cache of sequence b alone, sharing this cache's memory.

        A sequence of a cache is itself a valid one-sequence cache: its
        records (contiguous mode; paged mode keeps the shared block pool and
        uses the sequence's block-table row), its residual ring and its two
        counters sit at fixed offsets.  Used to export or dequantize single
        sequences of caches too large to export whole."""
        if not 0 <= b < self.shape.num_seqs:
            raise IndexError(b)
        v = object.__new__(QuantizedKVCache)
        v.shape = replace(self.shape, num_seqs=1)
        v.cfg = v.shape.config()
        v.sizes = kvq_buffer_sizes(v.cfg)
        v.device = self.device
        v._parent = self
        v._view = True
        per_ring = v.sizes.residual_bytes // 2
        if self.shape.paged:
            v.packed = self.packed
        else:
            per = v.sizes.packed_bytes
            # no group records at this capacity: the parent's placeholder
            # (a zero-size slice has no address to hand over)
            v.packed = self.packed[b * per:(b + 1) * per] if per else self.packed
        v.k_res = self.k_res[b * per_ring:(b + 1) * per_ring]
        v.v_res = self.v_res[b * per_ring:(b + 1) * per_ring]
        v.n_tokens = self.n_tokens[b:b + 1]
        v.n_quant = self.n_quant[b:b + 1]
        v.arrivals = self.arrivals[b:b + 1]
        v.block_table = self.block_table[b:b + 1] if self.block_table is not None else None
        v.lens = self.lens[b:b + 1].copy()
        v.k_scale, v.v_scale = self.k_scale, self.v_scale
        v.cache = v._make_cache()
        v._ws = None
        return v

    def stream_view(self, b: int, h: int) -> "QuantizedKVCache":
        """Read-only cache of stream (sequence b, kv head h) alone, sharing
        this cache's memory (contiguous mode).  In a contiguous cache the
        records of one (sequence, kv head) are consecutive and so is its
        residual ring, so the stream is itself a valid cache of one sequence
        and one kv head; its counters are the sequence's."""
        if self.shape.paged:
            raise ValueError("stream_view: contiguous caches only")
        if not (0 <= b < self.shape.num_seqs and 0 <= h < self.shape.num_kv_heads):
            raise IndexError((b, h))
        v = object.__new__(QuantizedKVCache)
        v.shape = replace(self.shape, num_seqs=1, num_kv_heads=1)
        v.cfg = v.shape.config()
        v.sizes = kvq_buffer_sizes(v.cfg)
        v.device = self.device
        v._parent = self
        v._view = True
        s = b * self.shape.num_kv_heads + h
        per = v.sizes.packed_bytes
        v.packed = self.packed[s * per:(s + 1) * per] if per else self.packed
        per_ring = v.sizes.residual_bytes // 2
        v.k_res = self.k_res[s * per_ring:(s + 1) * per_ring]
        v.v_res = self.v_res[s * per_ring:(s + 1) * per_ring]
        v.n_tokens = self.n_tokens[b:b + 1]
        v.n_quant = self.n_quant[b:b + 1]
        v.arrivals = self.arrivals[b:b + 1]
        v.block_table = None
        v.lens = self.lens[b:b + 1].copy()
        v.k_scale = self.k_scale[h:h + 1] if self.k_scale is not None else None
        v.v_scale = self.v_scale[h:h + 1] if self.v_scale is not None else None
        v.cache = v._make_cache()
        v._ws = None
        return v

    def _writable(self, what):
        if getattr(self, "_view", False):
            raise KVQError(KVQ_EINVAL, "%s on a read-only sequence view" % what)

    @property
    def G(self):
        return self.shape.group_size

    @property
    def R(self):
        return self.shape.residual

    @property
    def onwrite(self):
        """8-bit format without a residual window: tokens quantized as written."""
        return self.shape.kv_format != FORMAT_KIVI and self.shape.residual == 0

    def capacity(self):
        s = self.shape
        if s.paged:
            if self.onwrite:
                return s.max_blocks_per_seq * s.group_size
            return s.residual + (s.max_blocks_per_seq + 1) * s.group_size - 1
        return s.max_tokens

    # -- paged block bookkeeping (host) ------------------------------------
    def _ensure_blocks(self, lens_after):
        """Give every sequence a block for each key group it will hold.  Only
        the new entries go to the device table: a copy from pinned memory and
        an indexed store, both ordered on the current stream before the call
        that reads them, so the host does not wait for the device."""
        if not self.shape.paged:
            return
        need = np.array([groups_held(int(n), self.G, self.R, self.onwrite) for n in np.atleast_1d(lens_after)],
                        np.int64)
        short = np.nonzero(need > self._nblk)[0]
        if len(short) == 0:
            return
        if int(need.max()) > self._bt_host.shape[1]:
            raise KVQError(KVQ_ECAPACITY, "paged cache: a sequence needs more than max_blocks_per_seq blocks")
        rows, cols, vals = [], [], []
        for b in short:
            for g in range(int(self._nblk[b]), int(need[b])):
                if not self._free:
                    raise KVQError(KVQ_ECAPACITY, "paged cache out of blocks")
                blk = self._free.pop()
                self._bt_host[b, g] = blk
                rows.append(int(b))
                cols.append(g)
                vals.append(blk)
            self._nblk[b] = need[b]
        upd = torch.tensor([rows, cols, vals], dtype=torch.int64)
        if self.device.type == "cuda":
            upd = upd.pin_memory().to(self.device, non_blocking=True)
        self.block_table[upd[0], upd[1]] = upd[2].to(torch.int32)

    def _prefill_blocks(self, lens):
        """Block table after a prefill: the whole pool is free again and each
        sequence in turn takes a block per key group from the pool, in the
        order the pool hands them out.  The device table is rewritten only if
        it changes (a rewrite waits for the device: in-flight calls may read
        the table)."""
        need = np.array([groups_held(int(n), self.G, self.R, self.onwrite) for n in lens], np.int64)
        total = int(need.sum())
        if total > len(self._block_order) or (len(need) and int(need.max()) > self._bt_host.shape[1]):
            raise KVQError(KVQ_ECAPACITY, "paged cache out of blocks")
        order = np.asarray(self._block_order[::-1][:total], np.int32)   # pop() order
        table = np.full_like(self._bt_host, -1)
        start = 0
        for b, k in enumerate(need):
            table[b, :k] = order[start:start + k]
            start += int(k)
        self._free = self._block_order[:len(self._block_order) - total]
        self._nblk = need.copy()
        if not np.array_equal(table, self._bt_host):
            self._bt_host[:] = table
            self.block_table.copy_(torch.from_numpy(self._bt_host))

    def shuffle_free_blocks(self, seed):
        """Hand blocks out in a seeded random order (so paged parity tests do
        not see an accidentally contiguous pool)."""
        rng = np.random.Generator(np.random.PCG64(seed))
        self._block_order = [int(i) for i in rng.permutation(self.shape.num_blocks)]
        self._free = list(self._block_order)

    # -- calls --------------------------------------------------------------
    def prefill(self, k, v, seq_lens, stream=None, seq_lens_device=None):
        """k, v: fp16 [B][H][max_len][d] on the device; seq_lens: ints [B]
        (host).  seq_lens_device: optional int32 device copy of seq_lens,
        reused instead of a fresh host-to-device copy."""
        self._writable("prefill")
        lens = np.asarray(seq_lens, np.int64)
        B, H, max_len, d = k.shape
        if (B, H, d) != (self.shape.num_seqs, self.shape.num_kv_heads, HEAD_DIM) or k.shape != v.shape:
            raise ValueError("k/v shape %s does not match the cache" % (tuple(k.shape),))
        if k.dtype != torch.float16 or v.dtype != torch.float16 or not k.is_contiguous() or not v.is_contiguous():
            raise ValueError("k and v must be contiguous fp16")
        if np.any(lens < 0) or np.any(lens > max_len) or np.any(lens > self.capacity()):
            raise ValueError("sequence length outside [0, min(max_len, capacity)]")
        if self.shape.paged:
            self._prefill_blocks(lens)
        sl = seq_lens_device
        if sl is None:
            sl = torch.as_tensor(lens.astype(np.int32), device=self.device)
        kv_quantize_prefill(self.cfg, self.cache, k, v, max_len, sl, stream)
        self.lens = lens.copy()
        self._keep = sl  # keep alive until the stream has consumed it

    def append(self, k_new, v_new, stream=None):
        """k_new, v_new: fp16 [B][H][d] on the device."""
        self._writable("append")
        if np.any(self.lens + 1 > self.capacity()):
            raise KVQError(KVQ_ECAPACITY, "kv_append_token: a sequence is full")
        self._ensure_blocks(self.lens + 1)
        kv_append_token(self.cfg, self.cache, k_new, v_new, stream)
        self.lens = self.lens + 1

    def dequantize(self, out_tokens=None, stream=None):
        T = int(out_tokens if out_tokens is not None else max(int(self.lens.max()), 1))
        B, H = self.shape.num_seqs, self.shape.num_kv_heads
        ko = torch.empty((B, H, T, HEAD_DIM), dtype=torch.float32, device=self.device)
        vo = torch.empty_like(ko)
        kv_dequantize(self.cfg, self.cache, ko, vo, T, stream)
        return ko, vo

    def export_codes(self, out_tokens=None, stream=None):
        G = self.G
        T = int(out_tokens if out_tokens is not None else max(int(self.lens.max()), 1))
        T = (T + G - 1) // G * G
        B, H = self.shape.num_seqs, self.shape.num_kv_heads
        dev = self.device
        kc = torch.empty((B, H, T, HEAD_DIM), dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        fmt = self.shape.kv_format
        if fmt == FORMAT_FP8_E4M3:   # no scale/zero tables
            ks = kz = vs = vz = None
        else:
            kshape = (B, H, T // G, HEAD_DIM) if fmt == FORMAT_KIVI else (B, H, T)
            ks = torch.empty(kshape, dtype=torch.int16, device=dev)
            kz = torch.empty_like(ks)
            vs = torch.empty((B, H, T), dtype=torch.int16, device=dev)
            vz = torch.empty_like(vs)
        kv_export_codes(self.cfg, self.cache, kc, vc, ks, kz, vs, vz, T, stream)
        return kc, vc, ks, kz, vs, vz

    def export_outliers(self, out_tokens=None, stream=None):
        """Dense-and-sparse keys: (positions, fp16 values) [B][H][T/G][G]."""
        G = self.G
        T = int(out_tokens if out_tokens is not None else max(int(self.lens.max()), 1))
        T = (T + G - 1) // G * G
        B, H = self.shape.num_seqs, self.shape.num_kv_heads
        pos = torch.empty((B, H, T // G, G), dtype=torch.int16, device=self.device)
        val = torch.empty_like(pos)
        kv_export_outliers(self.cfg, self.cache, pos, val, T, stream)
        return pos, val

    def workspace(self, num_q_heads):
        nb = kv_decode_attention_workspace_bytes(self.cfg, num_q_heads)
        if nb == 0:
            raise KVQError(KVQ_EINVAL, "kv_decode_attention_workspace_bytes")
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode_attention(self, q, softmax_scale=None, out=None, stream=None, split_events=None):
        """q: fp16 [B][Hq][d] -> fp32 [B][Hq][d].  split_events: optional
        (start, mid, end) torch.cuda.Event triple recorded around the two
        kernels (partials, merge) on the stream."""
        B, Hq, d = q.shape
        if B != self.shape.num_seqs or d != HEAD_DIM or q.dtype != torch.float16 or not q.is_contiguous():
            raise ValueError("q must be contiguous fp16 [B][Hq][128]")
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=self.device)
        ws = self.workspace(Hq)
        if split_events is None:
            kv_decode_attention(self.cfg, self.cache, q, Hq, softmax_scale, out, ws, stream)
            return out
        st = stream if stream is not None else torch.cuda.current_stream()
        split_events[0].record(st)
        kv_decode_attention_partials(self.cfg, self.cache, q, Hq, softmax_scale, ws, stream)
        split_events[1].record(st)
        kv_decode_attention_merge(self.cfg, self.cache, Hq, ws, out, stream)
        split_events[2].record(st)
        return out
