"""CPU oracle for KIVI-style KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU library never
imports, links or runs anything here.

The arithmetic lives in ``kvq_oracle.c`` (plain C99, fp32 quantizer exactly as
the fixed formula states, fp64 attention).  This module compiles it with gcc
when asked (``build()``), loads it with ctypes and offers numpy-level helpers
that loop over (sequence, kv-head) streams.  Nothing here does arithmetic of
the method itself beyond bookkeeping of which tokens belong to which stream.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")
_lib = None
_lock = threading.Lock()

_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile kvq_oracle.c into libkvq_oracle.so (plain gcc, no fast-math,
    no contraction, so every fp32 operation is one IEEE rounding)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fno-builtin", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """Load the oracle library, compiling it first if no build exists or the
    source is newer than the build."""
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_LIB_PATH)
            L.orc_h2f.restype = ctypes.c_float
            L.orc_h2f.argtypes = [ctypes.c_uint16]
            L.orc_f2h.restype = ctypes.c_uint16
            L.orc_f2h.argtypes = [ctypes.c_float]
            L.orc_h2f_array.argtypes = [_u16p, _f32p, ctypes.c_long]
            L.orc_f2h_array.argtypes = [_f32p, _u16p, ctypes.c_long]
            L.orc_num_quantized.restype = ctypes.c_int
            L.orc_num_quantized.argtypes = [ctypes.c_int] * 3
            L.orc_num_quantized8.restype = ctypes.c_int
            L.orc_num_quantized8.argtypes = [ctypes.c_int] * 3
            L.orc_quantize_key_group.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 _u8p, _u16p, _u16p]
            L.orc_quantize_value_token.argtypes = [_u16p, ctypes.c_int, ctypes.c_int,
                                                   _u8p, _u16p, _u16p]
            L.orc_prefill_stream.restype = ctypes.c_int
            L.orc_prefill_stream.argtypes = [_u16p, _u16p] + [ctypes.c_int] * 6 + \
                [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p]
            L.orc_append_stream.restype = ctypes.c_int
            L.orc_append_stream.argtypes = [_u16p, _u16p, ctypes.c_int, _i32p, _i32p,
                                            _u16p, _u16p] + [ctypes.c_int] * 5 + \
                [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p]
            L.orc_dequantize_stream.argtypes = [_u16p, _u16p] + [ctypes.c_int] * 4 + \
                [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _f32p, _f32p]
            L.orc_attention.argtypes = [_f32p, ctypes.c_int, _f32p, _f32p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float, _f64p, _f64p]
            L.orc_fp8_e4m3_decode.restype = ctypes.c_float
            L.orc_fp8_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.orc_fp8_e4m3_encode.restype = ctypes.c_uint8
            L.orc_fp8_e4m3_encode.argtypes = [ctypes.c_float]
            L.orc_fp8_decode_array.argtypes = [_u8p, _f32p, ctypes.c_long]
            L.orc_fp8_encode_array.argtypes = [_f32p, _u8p, ctypes.c_long]
            L.orc_quantize_token_fp8.argtypes = [_u16p, ctypes.c_int, ctypes.c_float, _u8p]
            L.orc_prefill_stream8.restype = ctypes.c_int
            L.orc_prefill_stream8.argtypes = [ctypes.c_int, _u16p, _u16p] + [ctypes.c_int] * 4 + \
                [ctypes.c_float] * 2 + [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p]
            L.orc_append_stream8.restype = ctypes.c_int
            L.orc_append_stream8.argtypes = [ctypes.c_int, _u16p, _u16p, ctypes.c_int, _i32p, _i32p,
                                             _u16p, _u16p] + [ctypes.c_int] * 3 + \
                [ctypes.c_float] * 2 + [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p]
            L.orc_dequantize_stream8.argtypes = [ctypes.c_int, _u16p, _u16p] + [ctypes.c_int] * 3 + \
                [ctypes.c_float] * 2 + [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _f32p, _f32p]
            L.orc_stream_bytes8.restype = ctypes.c_double
            L.orc_stream_bytes8.argtypes = [ctypes.c_int, ctypes.c_long] + [ctypes.c_int] * 3
            L.orc_rope_rotate.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_double,
                                          _f64p]
            L.orc_attention_d.argtypes = [_f32p, ctypes.c_int, _f64p, _f32p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_float, _f64p]
            L.orc_codebook_scale.restype = ctypes.c_int
            L.orc_codebook_scale.argtypes = [ctypes.c_int]
            L.orc_codebook_levels.argtypes = [ctypes.c_int, _f64p]
            L.orc_quantize_key_group_cb.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p,
                                                    _u8p, _u16p, _u16p]
            L.orc_quantize_value_token_cb.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _f64p,
                                                      _u8p, _u16p, _u16p]
            L.orc_prefill_stream_cb.restype = ctypes.c_int
            L.orc_prefill_stream_cb.argtypes = L.orc_prefill_stream.argtypes
            L.orc_append_stream_cb.restype = ctypes.c_int
            L.orc_append_stream_cb.argtypes = L.orc_append_stream.argtypes
            L.orc_dequantize_stream_cb.argtypes = [_u16p, _u16p] + [ctypes.c_int] * 6 + \
                [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _f32p, _f32p]
            L.orc_quantize_key_group_ds.argtypes = [_u16p] + [ctypes.c_int] * 4 + [_f64p, _u8p, _u16p, _u16p,
                                                                                 _u16p, _u16p]
            L.orc_prefill_stream_ds.restype = ctypes.c_int
            L.orc_prefill_stream_ds.argtypes = [_u16p, _u16p] + [ctypes.c_int] * 8 + \
                [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _u16p, _u16p]
            L.orc_append_stream_ds.restype = ctypes.c_int
            L.orc_append_stream_ds.argtypes = [_u16p, _u16p, ctypes.c_int, _i32p, _i32p, _u16p, _u16p] + \
                [ctypes.c_int] * 7 + [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _u16p, _u16p]
            L.orc_dequantize_stream_ds.argtypes = [_u16p, _u16p] + [ctypes.c_int] * 8 + \
                [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _u16p, _u16p, _f32p, _f32p]
            L.orc_stream_bytes.restype = ctypes.c_double
            L.orc_stream_bytes.argtypes = [ctypes.c_long] + [ctypes.c_int] * 5
            L.orc_kv_bytes_closed_form.restype = ctypes.c_double
            L.orc_kv_bytes_closed_form.argtypes = [ctypes.c_long] * 4 + [ctypes.c_double]
            _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


# --------------------------------------------------------------------------
# fp16 codec
# --------------------------------------------------------------------------

def h2f(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().orc_h2f_array(_p(bits, _u16p), _p(out, _f32p), bits.size)
    return out


def f2h(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f2h_array(_p(x, _f32p), _p(out, _u16p), x.size)
    return out


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().orc_fp8_decode_array(_p(c, _u8p), _p(out, _f32p), c.size)
    return out


def fp8_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_fp8_encode_array(_p(x, _f32p), _p(out, _u8p), x.size)
    return out


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

# cache formats: the low-bit KIVI format, and the two 8-bit formats
FMT_KIVI, FMT_INT8, FMT_FP8 = 0, 1, 2
# level grids of the low-bit format: uniform, normal-quantile codebook
GRID_UNIFORM, GRID_CODEBOOK = 0, 1


def codebook_levels(bits: int) -> np.ndarray:
    """Levels L_0..L_Q of the b-bit normal-quantile codebook, in grid steps."""
    out = np.empty(1 << bits, np.float64)
    lib().orc_codebook_levels(int(bits), _p(out, _f64p))
    return out


def quantize_key_group_cb(x_bits: np.ndarray, bits: int, levels=None):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    G, d = x.shape
    lev = np.ascontiguousarray(codebook_levels(bits) if levels is None else levels, np.float64)
    codes = np.empty((G, d), np.uint8)
    s = np.empty(d, np.uint16)
    z = np.empty(d, np.uint16)
    lib().orc_quantize_key_group_cb(_p(x, _u16p), G, d, bits, _p(lev, _f64p), _p(codes, _u8p), _p(s, _u16p),
                                    _p(z, _u16p))
    return codes, s, z


def quantize_key_group_ds(x_bits: np.ndarray, bits: int, n_out: int):
    """Dense-and-sparse key group: -> (codes [G][d], s [d], z [d],
    kept positions [n_out] ascending, kept fp16 bits [n_out])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    G, d = x.shape
    codes = np.empty((G, d), np.uint8)
    s = np.empty(d, np.uint16)
    z = np.empty(d, np.uint16)
    pos = np.empty(n_out, np.uint16)
    val = np.empty(n_out, np.uint16)
    lib().orc_quantize_key_group_ds(_p(x, _u16p), G, d, bits, n_out, None, _p(codes, _u8p), _p(s, _u16p),
                                    _p(z, _u16p), _p(pos, _u16p), _p(val, _u16p))
    return codes, s, z, pos, val


def quantize_value_token_cb(x_bits: np.ndarray, bits: int, levels=None):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    lev = np.ascontiguousarray(codebook_levels(bits) if levels is None else levels, np.float64)
    codes = np.empty(x.shape[0], np.uint8)
    s = np.empty(1, np.uint16)
    z = np.empty(1, np.uint16)
    lib().orc_quantize_value_token_cb(_p(x, _u16p), x.shape[0], bits, _p(lev, _f64p), _p(codes, _u8p),
                                      _p(s, _u16p), _p(z, _u16p))
    return codes, int(s[0]), int(z[0])

def num_quantized(n: int, G: int, R: int, fmt: int = 0) -> int:
    """Quantized tokens of a stream holding n (fmt: FMT_KIVI, or an 8-bit
    format, whose streams with R = 0 quantize every token on write)."""
    if fmt:
        return int(lib().orc_num_quantized8(int(n), int(G), int(R)))
    return int(lib().orc_num_quantized(int(n), int(G), int(R)))


def quantize_key_group(x_bits: np.ndarray, bits: int):
    """x_bits: uint16 fp16 bit patterns [G][d] -> (codes [G][d], s [d], z [d])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    G, d = x.shape
    codes = np.empty((G, d), np.uint8)
    s = np.empty(d, np.uint16)
    z = np.empty(d, np.uint16)
    lib().orc_quantize_key_group(_p(x, _u16p), G, d, bits, _p(codes, _u8p), _p(s, _u16p), _p(z, _u16p))
    return codes, s, z


def quantize_token_fp8(x_bits: np.ndarray, scale: float):
    """x_bits: uint16 [d] -> E4M3 codes [d] under a static scale."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.empty(x.shape[0], np.uint8)
    lib().orc_quantize_token_fp8(_p(x, _u16p), x.shape[0], ctypes.c_float(scale), _p(codes, _u8p))
    return codes


def quantize_value_token(x_bits: np.ndarray, bits: int):
    """x_bits: uint16 [d] -> (codes [d], s, z)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    d = x.shape[0]
    codes = np.empty(d, np.uint8)
    s = np.empty(1, np.uint16)
    z = np.empty(1, np.uint16)
    lib().orc_quantize_value_token(_p(x, _u16p), d, bits, _p(codes, _u8p), _p(s, _u16p), _p(z, _u16p))
    return codes, int(s[0]), int(z[0])


class StreamState:
    """Quantized state of one (sequence, kv-head) stream, as the oracle
    defines it: codes and fp16 metadata for tokens [0, nq), fp16 history for
    every token (only [nq, n) is the residual).

    fmt FMT_KIVI: kbits/vbits in {2, 4}, key scale/zero per (group, channel),
    value scale/zero per token.  FMT_INT8: 8-bit codes, key and value
    scale/zero per token.  FMT_FP8: E4M3 codes under the static scales
    kscale / vscale of the stream's kv head, no per-token metadata."""

    def __init__(self, d, kbits, vbits, G, R, cap, fmt=FMT_KIVI, kscale=0.0, vscale=0.0, grid=GRID_UNIFORM,
                 sparse=False):
        self.d, self.kbits, self.vbits, self.G, self.R, self.cap = d, kbits, vbits, G, R, cap
        self.fmt, self.kscale, self.vscale = fmt, float(kscale), float(vscale)
        self.grid = grid
        self.sparse = sparse          # dense-and-sparse keys: G kept entries per key group
        self.opos = np.zeros((cap // G + 1, G), np.uint16)
        self.oval = np.zeros((cap // G + 1, G), np.uint16)
        self.n = 0
        self.nq = 0
        self.hist_k = np.zeros((cap, d), np.uint16)
        self.hist_v = np.zeros((cap, d), np.uint16)
        self.kcodes = np.zeros((cap, d), np.uint8)
        self.vcodes = np.zeros((cap, d), np.uint8)
        if fmt == FMT_KIVI:
            ng = cap // G + 1
            self.ks = np.zeros((ng, d), np.uint16)
            self.kz = np.zeros((ng, d), np.uint16)
        else:
            self.ks = np.zeros(cap, np.uint16)
            self.kz = np.zeros(cap, np.uint16)
        self.vs = np.zeros(cap, np.uint16)
        self.vz = np.zeros(cap, np.uint16)

    def _arrays(self):
        return (_p(self.kcodes, _u8p), _p(self.ks, _u16p), _p(self.kz, _u16p),
                _p(self.vcodes, _u8p), _p(self.vs, _u16p), _p(self.vz, _u16p))

    @classmethod
    def prefill(cls, k_bits, v_bits, kbits, vbits, G, R, cap=None, fmt=FMT_KIVI, kscale=0.0, vscale=0.0,
                grid=GRID_UNIFORM, sparse=False):
        k = np.ascontiguousarray(k_bits, np.uint16)
        v = np.ascontiguousarray(v_bits, np.uint16)
        n, d = k.shape
        st = cls(d, kbits, vbits, G, R, cap if cap is not None else max(n, 1), fmt, kscale, vscale, grid, sparse)
        st.hist_k[:n] = k
        st.hist_v[:n] = v
        if sparse:
            st.nq = int(lib().orc_prefill_stream_ds(
                _p(k, _u16p), _p(v, _u16p), n, d, kbits, vbits, G, R, G, int(grid), *st._arrays(),
                _p(st.opos, _u16p), _p(st.oval, _u16p)))
        elif fmt == FMT_KIVI and grid == GRID_CODEBOOK:
            st.nq = int(lib().orc_prefill_stream_cb(
                _p(k, _u16p), _p(v, _u16p), n, d, kbits, vbits, G, R, *st._arrays()))
        elif fmt == FMT_KIVI:
            st.nq = int(lib().orc_prefill_stream(
                _p(k, _u16p), _p(v, _u16p), n, d, kbits, vbits, G, R, *st._arrays()))
        else:
            st.nq = int(lib().orc_prefill_stream8(
                fmt, _p(k, _u16p), _p(v, _u16p), n, d, G, R,
                ctypes.c_float(st.kscale), ctypes.c_float(st.vscale), *st._arrays()))
        st.n = n
        return st

    def append(self, k_new_bits, v_new_bits) -> int:
        kn = np.ascontiguousarray(k_new_bits, np.uint16)
        vn = np.ascontiguousarray(v_new_bits, np.uint16)
        n = ctypes.c_int(self.n)
        nq = ctypes.c_int(self.nq)
        if self.sparse:
            r = lib().orc_append_stream_ds(
                _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), self.cap,
                ctypes.byref(n), ctypes.byref(nq), _p(kn, _u16p), _p(vn, _u16p),
                self.d, self.kbits, self.vbits, self.G, self.R, self.G, int(self.grid), *self._arrays(),
                _p(self.opos, _u16p), _p(self.oval, _u16p))
        elif self.fmt == FMT_KIVI:
            fn = lib().orc_append_stream_cb if self.grid == GRID_CODEBOOK else lib().orc_append_stream
            r = fn(
                _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), self.cap,
                ctypes.byref(n), ctypes.byref(nq), _p(kn, _u16p), _p(vn, _u16p),
                self.d, self.kbits, self.vbits, self.G, self.R, *self._arrays())
        else:
            r = lib().orc_append_stream8(
                self.fmt, _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), self.cap,
                ctypes.byref(n), ctypes.byref(nq), _p(kn, _u16p), _p(vn, _u16p),
                self.d, self.G, self.R, ctypes.c_float(self.kscale), ctypes.c_float(self.vscale),
                *self._arrays())
        if r < 0:
            raise ValueError("oracle stream capacity exceeded")
        self.n, self.nq = n.value, nq.value
        return r

    def dequantize(self):
        """-> (k_hat, v_hat) float32 [n][d]."""
        n, d = self.n, self.d
        ok = np.empty((max(n, 1), d), np.float32)
        ov = np.empty((max(n, 1), d), np.float32)
        if self.sparse:
            lib().orc_dequantize_stream_ds(
                _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), n, self.nq, d, self.G, self.G, self.kbits,
                self.vbits, int(self.grid), *self._arrays(), _p(self.opos, _u16p), _p(self.oval, _u16p),
                _p(ok, _f32p), _p(ov, _f32p))
        elif self.fmt == FMT_KIVI and self.grid == GRID_CODEBOOK:
            lib().orc_dequantize_stream_cb(
                _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), n, self.nq, d, self.G, self.kbits, self.vbits,
                *self._arrays(), _p(ok, _f32p), _p(ov, _f32p))
        elif self.fmt == FMT_KIVI:
            lib().orc_dequantize_stream(
                _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), n, self.nq, d, self.G,
                *self._arrays(), _p(ok, _f32p), _p(ov, _f32p))
        else:
            lib().orc_dequantize_stream8(
                self.fmt, _p(self.hist_k, _u16p), _p(self.hist_v, _u16p), n, self.nq, d,
                ctypes.c_float(self.kscale), ctypes.c_float(self.vscale),
                *self._arrays(), _p(ok, _f32p), _p(ov, _f32p))
        return ok[:n], ov[:n]

    # logical views used by the parity tests
    def key_codes(self):
        return self.kcodes[: self.nq]

    def value_codes(self):
        return self.vcodes[: self.nq]

    def key_meta(self):
        """KIVI: per (group, channel) [nq/G][d]; INT8 / FP8: per token [nq]."""
        if self.fmt == FMT_KIVI:
            g = self.nq // self.G
            return self.ks[:g], self.kz[:g]
        return self.ks[: self.nq], self.kz[: self.nq]

    def value_meta(self):
        return self.vs[: self.nq], self.vz[: self.nq]

    def outliers(self):
        """Dense-and-sparse keys: kept positions (t*d + c within the group,
        ascending) and fp16 values, [nq/G][G]."""
        g = self.nq // self.G
        return self.opos[:g], self.oval[:g]

    def residual(self):
        return self.hist_k[self.nq: self.n], self.hist_v[self.nq: self.n]


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float,
              want_weights: bool = False):
    """q: float32 [gq][d]; k_hat, v_hat: float32 [n][d] -> out float64 [gq][d]
    (and weights [gq][n] if asked)."""
    q = np.ascontiguousarray(q, np.float32)
    kh = np.ascontiguousarray(k_hat, np.float32)
    vh = np.ascontiguousarray(v_hat, np.float32)
    gq, d = q.shape
    n = kh.shape[0]
    if n == 0:
        kh = np.zeros((1, d), np.float32)
        vh = np.zeros((1, d), np.float32)
    out = np.empty((gq, d), np.float64)
    w = np.empty((gq, max(n, 1)), np.float64) if want_weights else None
    lib().orc_attention(_p(q, _f32p), gq, _p(kh, _f32p), _p(vh, _f32p), n, d,
                        ctypes.c_float(scale), _p(out, _f64p),
                        _p(w, _f64p) if w is not None else None)
    if want_weights:
        return out, w[:, :n]
    return out


def rope_rotate(k: np.ndarray, base: float, pos0: int = 0) -> np.ndarray:
    """k: float32 [n][d] keys at positions pos0.. -> fp64 rotated keys."""
    k = np.ascontiguousarray(k, np.float32)
    n, d = k.shape
    out = np.empty((max(n, 1), d), np.float64)
    if n:
        lib().orc_rope_rotate(_p(k, _f32p), n, d, int(pos0), float(base), _p(out, _f64p))
    return out[:n]


def attention_rope(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float, base: float):
    """Attention over pre-RoPE keys k_hat (float32 [n][d], token t at
    position t) rotated on read: softmax(q . RoPE_t(k_t) * scale) v."""
    q = np.ascontiguousarray(q, np.float32)
    vh = np.ascontiguousarray(v_hat, np.float32)
    gq, d = q.shape
    n = k_hat.shape[0]
    kr = rope_rotate(k_hat, base) if n else np.zeros((1, d))
    if n == 0:
        vh = np.zeros((1, d), np.float32)
    kr = np.ascontiguousarray(kr, np.float64)
    out = np.empty((gq, d), np.float64)
    lib().orc_attention_d(_p(q, _f32p), gq, _p(kr, _f64p), _p(vh, _f32p), n, d, ctypes.c_float(scale),
                          _p(out, _f64p))
    return out


def stream_bytes(n, d, kbits, vbits, G, R, fmt=FMT_KIVI) -> float:
    if fmt != FMT_KIVI:
        return float(lib().orc_stream_bytes8(fmt, int(n), d, G, R))
    return float(lib().orc_stream_bytes(int(n), d, kbits, vbits, G, R))


def kv_bytes_closed_form(L, Hkv, n, d, bytes_per_elem) -> float:
    return float(lib().orc_kv_bytes_closed_form(int(L), int(Hkv), int(n), int(d), float(bytes_per_elem)))


# --------------------------------------------------------------------------
# batch helpers: loop over (sequence, kv-head) streams
# --------------------------------------------------------------------------

def prefill_batch(k_bits, v_bits, seq_lens, kbits, vbits, G, R, cap=None, threads=1,
                  fmt=FMT_KIVI, kscales=None, vscales=None, grid=GRID_UNIFORM, sparse=False):
    """k_bits, v_bits: uint16 [B][H][L][d]; seq_lens: [B]; kscales, vscales:
    FP8 static scales per kv head [H].
    -> list (per sequence) of lists (per kv-head) of StreamState."""
    B, H = k_bits.shape[:2]

    def one(bh):
        b, h = bh
        n = int(seq_lens[b])
        ks = float(kscales[h]) if kscales is not None else 0.0
        vs = float(vscales[h]) if vscales is not None else 0.0
        return StreamState.prefill(k_bits[b, h, :n], v_bits[b, h, :n], kbits, vbits, G, R,
                                   cap=cap if cap is not None else max(n, 1), fmt=fmt,
                                   kscale=ks, vscale=vs, grid=grid, sparse=sparse)

    jobs = [(b, h) for b in range(B) for h in range(H)]
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(one, jobs))
    else:
        res = [one(j) for j in jobs]
    return [[res[b * H + h] for h in range(H)] for b in range(B)]


def decode_attention_batch(q_f32, states, scale, threads=1, rope_base=0.0):
    """q_f32: float32 [B][Hq][d]; states from prefill_batch -> float64 [B][Hq][d].
    Query head h reads kv head h // (Hq / H).  rope_base > 0: the cached keys
    are pre-RoPE and are rotated on read (attention_rope)."""
    B, Hq, d = q_f32.shape
    H = len(states[0])
    gq = Hq // H
    out = np.zeros((B, Hq, d), np.float64)

    def one(bh):
        b, h = bh
        kh, vh = states[b][h].dequantize()
        qs = q_f32[b, h * gq:(h + 1) * gq]
        out[b, h * gq:(h + 1) * gq] = attention_rope(qs, kh, vh, scale, rope_base) if rope_base > 0 \
            else attention(qs, kh, vh, scale)

    jobs = [(b, h) for b in range(B) for h in range(H)]
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out
