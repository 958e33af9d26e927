"""Pins of the CPU oracle to facts that do not come from the oracle itself:
an independent fp16 implementation (numpy), closed forms and numbers the
pages print, constructed inputs whose answer is known exactly, invariants of
the method, and special cases of attention with a closed-form answer.

Each test names the passage it follows.  A plausible slip in the oracle (a
transposed key/value granularity, a wrong group index, a dropped zero point,
a wrong rounding rule, a softmax over the wrong axis) breaks at least one of
them; test_pin_catches_planted_mistakes checks that on purpose-built broken
copies of the oracle.
"""
import json
import os
import subprocess

import numpy as np
import pytest

from midpoint_extremes import MIDPOINT_EXTREMES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f16bits(vals):
    return np.asarray(vals, np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# fp16 codec against numpy's float16 (an independent implementation)
# --------------------------------------------------------------------------

def test_f16_decode_every_bit_pattern(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.h2f(pats)
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(1)
    mant = rng.random(200000).astype(np.float64) + 1.0
    expo = rng.integers(-30, 18, size=mant.size)
    x = (mant * np.exp2(expo) * rng.choice([-1.0, 1.0], size=mant.size)).astype(np.float32)
    # exact halfway points between adjacent fp16 values (ties), both parities
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -14, 2.0 ** -24,
                      2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 1e-10, np.inf, -np.inf],
                     np.float32)
    for arr in (x, ties, edges, -ties):
        ours = orc.f2h(arr)
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float16).view(np.uint16)
        assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------
# Quantizer: closed form of the scale and grid-aligned inputs
# "KV Cache compression lab", experiment 01: s = (max - min)/(2^b - 1),
# zero = the grid's start; "KV cache compression" (jaedaily), formula
# paragraph: per-channel keys, per-token values, dequant q*s + z.
# --------------------------------------------------------------------------

def _grid_aligned(rng, count, bits):
    """Codes in [0, Q] with both ends present, a power-of-two spacing and a
    zero that is a multiple of it, so every value is an exact fp16 number."""
    Q = (1 << bits) - 1
    codes = rng.integers(0, Q + 1, size=count)
    i, j = rng.choice(count, size=2, replace=False)
    codes[i], codes[j] = 0, Q
    s = 2.0 ** int(rng.integers(-6, 3))
    z = s * int(rng.integers(-40, 40))
    return codes.astype(np.uint8), s, z


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("G", [16, 32])
def test_key_group_grid_aligned_per_channel(orc, bits, G):
    rng = np.random.default_rng(10 + bits + G)
    d = 128
    codes = np.zeros((G, d), np.uint8)
    x = np.zeros((G, d), np.float64)
    S = np.zeros(d)
    Z = np.zeros(d)
    for c in range(d):  # every channel has its own scale and zero
        cc, s, z = _grid_aligned(rng, G, bits)
        codes[:, c] = cc
        x[:, c] = z + cc * s
        S[c], Z[c] = s, z
    got_codes, got_s, got_z = orc.quantize_key_group(f16bits(x), bits)
    assert np.array_equal(got_codes, codes)
    assert np.array_equal(got_s, f16bits(S))
    assert np.array_equal(got_z, f16bits(Z))


@pytest.mark.parametrize("bits", [2, 4])
def test_value_tokens_grid_aligned_per_token(orc, bits):
    rng = np.random.default_rng(20 + bits)
    d, n = 128, 70
    x = np.zeros((n, d))
    exp_codes = np.zeros((n, d), np.uint8)
    S = np.zeros(n)
    Z = np.zeros(n)
    for t in range(n):  # every token has its own scale and zero
        cc, s, z = _grid_aligned(rng, d, bits)
        exp_codes[t] = cc
        x[t] = z + cc * s
        S[t], Z[t] = s, z
        got, gs, gz = orc.quantize_value_token(f16bits(x[t]), bits)
        assert np.array_equal(got, cc)
        assert gs == f16bits([s])[0] and gz == f16bits([z])[0]


def test_ties_to_even_golden(orc):
    g = _golden("tie_to_even_int2.json")
    vals = np.array(g["values"])
    x = np.tile(vals[:, None], (1, 128))  # same 5 values in every channel
    codes, s, z = orc.quantize_key_group(f16bits(x), g["bits"])
    assert codes[:, 0].tolist() == g["expected_codes"]
    assert np.all(codes == codes[:, :1])
    assert np.all(orc.h2f(s) == g["expected_scale"])
    assert np.all(orc.h2f(z) == g["expected_zero"])
    # per-token form on the same five values padded with copies of the ends
    tok = np.concatenate([vals, np.full(123, 3.0)])
    c2, s2, z2 = orc.quantize_value_token(f16bits(tok), g["bits"])
    assert c2[:5].tolist() == g["expected_codes"]


def _even_neighbour_of_midpoint(mn, mx, bits):
    from fractions import Fraction
    q = (Fraction(mx) - Fraction(mn)) / ((1 << bits) - 1)
    lo = np.float16(float(q))
    lo = lo if Fraction(float(lo)) < q else np.nextafter(lo, np.float16(-np.inf))
    hi = np.nextafter(lo, np.float16(np.inf))
    assert Fraction(float(lo)) < q < Fraction(float(hi)) and 2 * q == Fraction(float(lo)) + Fraction(float(hi))
    return lo if int(lo.view(np.uint16)) % 2 == 0 else hi


@pytest.mark.parametrize("bits", [4, 8])
def test_scale_on_fp16_midpoint_goes_to_even(orc, bits):
    """The scale is the fp16 rounding of (max - min) / (2^b - 1); for the
    sets whose quotient lies exactly halfway between two fp16 numbers it is
    the even one of the two (checked here in exact rational arithmetic)."""
    for mn, mx in MIDPOINT_EXTREMES[bits]:
        want = _even_neighbour_of_midpoint(mn, mx, bits)
        x = np.linspace(mn, mx, 32)
        x[0], x[-1] = mn, mx
        if bits == 4:
            _, s, z = orc.quantize_key_group(f16bits(np.tile(x[:, None], (1, 128))), bits)
            assert np.all(s == want.view(np.uint16)) and np.all(orc.h2f(z) == np.float32(np.float16(mn)))
            tok = np.concatenate([x, np.full(96, mn)])
            _, sv, _ = orc.quantize_value_token(f16bits(tok), bits)
            assert sv == want.view(np.uint16)
        else:
            tok = np.concatenate([x, np.full(96, mx)])
            st = orc.StreamState.prefill(np.tile(f16bits(tok), (32, 1)), np.tile(f16bits(tok), (32, 1)),
                                         8, 8, 32, 0, fmt=orc.FMT_INT8)
            assert np.all(st.key_meta()[0] == want.view(np.uint16))
            assert np.all(st.value_meta()[0] == want.view(np.uint16))


def test_outlier_crowds_levels_golden(orc):
    g = _golden("outlier_levels_int4.json")
    vals = np.array(g["normal_values"] + [g["outlier_value"]] + [0.0] * (128 - 16))
    codes, _, _ = orc.quantize_value_token(f16bits(vals), g["bits"])
    used = np.unique(codes[: len(g["normal_values"])])
    assert len(used) <= g["max_levels_used_by_normal_values"]
    assert codes[len(g["normal_values"])] == (1 << g["bits"]) - 1
    # without the outlier the same fifteen values use (almost) the whole grid
    vals2 = np.array(g["normal_values"] + [0.0] * (128 - 15))
    codes2, _, _ = orc.quantize_value_token(f16bits(vals2), g["bits"])
    assert len(np.unique(codes2[:15])) >= 10


def test_degenerate_group_zero_scale(orc):
    x = np.full((32, 128), 1.5)
    codes, s, z = orc.quantize_key_group(f16bits(x), 2)
    assert np.all(codes == 0) and np.all(s == 0) and np.all(orc.h2f(z) == 1.5)
    st = orc.StreamState.prefill(f16bits(np.full((64, 128), -2.25)), f16bits(np.full((64, 128), 7.0)),
                                 2, 4, 32, 0)
    kh, vh = st.dequantize()
    assert np.all(kh == -2.25) and np.all(vh == 7.0)


def test_negative_zero_extremes_canonicalised(orc):
    x = np.zeros((32, 128), np.float16)
    x[::2] = np.float16(-0.0)
    codes, s, z = orc.quantize_key_group(x.view(np.uint16), 4)
    assert np.all(z == 0) and np.all(s == 0) and np.all(codes == 0)
    y = np.abs(np.random.default_rng(3).standard_normal((32, 128))).astype(np.float16)
    y[5] = np.float16(-0.0)  # -0 is the minimum of every channel
    codes, s, z = orc.quantize_key_group(y.view(np.uint16), 4)
    assert np.all(z == 0)


# --------------------------------------------------------------------------
# Invariants on random data with the pages' structure
# --------------------------------------------------------------------------

def _roundtrip_bound(x, s16, z16, bits):
    """|x - x_hat| <= s/2 + Q*|s32 - s| + 4 ulp-scale terms: s/2 from snapping
    to the nearest level ("KV Cache compression lab", experiment 01); the
    clamp can bind at the top because s is the fp16-rounded spacing; the rest
    covers the fp32 roundings of (x - z), *inv and the fma."""
    Q = (1 << bits) - 1
    s = s16.astype(np.float64)
    z = z16.astype(np.float64)
    return s / 2 + Q * s * 2.0 ** -11 + 4 * 2.0 ** -24 * (np.abs(x) + np.abs(z) + Q * s) + 1e-30


@pytest.mark.parametrize("kbits,vbits,G,R", [(2, 2, 32, 32), (4, 4, 32, 128), (4, 2, 16, 128)])
def test_roundtrip_bound_and_extreme_codes(orc, kbits, vbits, G, R):
    from quantized_decode_attention_kivi_amd import synth
    w = synth.Workload("t", 1, 4, 2, kbits, vbits, G, R, context=2048 + 37, tag=77)
    K, V = synth.make_kv(w)
    kb = K.numpy().view(np.uint16)
    vb = V.numpy().view(np.uint16)
    for h in range(2):
        st = orc.StreamState.prefill(kb[0, h], vb[0, h], kbits, vbits, G, R)
        n, nq = st.n, st.nq
        assert nq == G * ((n - R) // G)
        kh, vh = st.dequantize()
        xk = orc.h2f(kb[0, h, :n]).astype(np.float64)
        xv = orc.h2f(vb[0, h, :n]).astype(np.float64)
        ks, kz = st.key_meta()
        vs, vz = st.value_meta()
        ksf = np.repeat(orc.h2f(ks), G, axis=0)
        kzf = np.repeat(orc.h2f(kz), G, axis=0)
        errk = np.abs(xk[:nq] - kh[:nq])
        assert np.all(errk <= _roundtrip_bound(xk[:nq], ksf, kzf, kbits))
        vsf = orc.h2f(vs)[:, None]
        vzf = orc.h2f(vz)[:, None]
        errv = np.abs(xv[:nq] - vh[:nq])
        assert np.all(errv <= _roundtrip_bound(xv[:nq], vsf, vzf, vbits))
        # residual tokens are exact
        assert np.array_equal(kh[nq:], xk[nq:].astype(np.float32))
        assert np.array_equal(vh[nq:], xv[nq:].astype(np.float32))
        # every non-degenerate key channel-group uses code 0 (its min) and Q (its max)
        kc = st.key_codes().reshape(-1, G, 128)
        assert np.all(kc.min(axis=1) == 0) and np.all(kc.max(axis=1) == (1 << kbits) - 1)
        vc = st.value_codes()
        assert np.all(vc.min(axis=1) == 0) and np.all(vc.max(axis=1) == (1 << vbits) - 1)


def test_granularity_matches_structure(orc):
    """"KV Cache compression lab", experiment 03: on keys with outlier
    channels per-channel grouping beats per-token grouping, on values with
    outlier rows per-token grouping wins."""
    from quantized_decode_attention_kivi_amd import synth
    w = synth.Workload("t", 1, 1, 1, 2, 2, 32, 0, context=1024, v_outlier_frac=0.05, tag=78)
    K, V = synth.make_kv(w)
    kb = K.numpy().view(np.uint16)[0, 0]
    vb = V.numpy().view(np.uint16)[0, 0]

    def rel_mse(xb, per_channel):
        x = orc.h2f(xb).astype(np.float64)
        xh = np.zeros_like(x)
        if per_channel:
            for g in range(x.shape[0] // 32):
                c, s, z = orc.quantize_key_group(xb[g * 32:(g + 1) * 32], 2)
                xh[g * 32:(g + 1) * 32] = c * orc.h2f(s)[None, :] + orc.h2f(z)[None, :]
        else:
            for t in range(x.shape[0]):
                c, s, z = orc.quantize_value_token(xb[t], 2)
                xh[t] = c * orc.h2f(np.array([s], np.uint16))[0] + orc.h2f(np.array([z], np.uint16))[0]
        return np.mean((x - xh) ** 2) / np.mean(x ** 2)

    assert rel_mse(kb, True) < 0.5 * rel_mse(kb, False)
    assert rel_mse(vb, False) < rel_mse(vb, True)


# --------------------------------------------------------------------------
# Residual window and flush ("KV cache compression: ...", section 3.2;
# "KV cache compression" (jaedaily), deployment step (c))
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G,R", [(32, 32), (32, 128), (16, 128), (16, 0), (64, 64)])
def test_num_quantized_closed_form(orc, G, R):
    for n in list(range(0, 400)) + [1023, 1024, 131072]:
        nq = orc.num_quantized(n, G, R)
        assert nq % G == 0 and 0 <= nq <= n
        if n >= R:
            assert R <= n - nq <= R + G - 1  # the newest R tokens always stay fp16
        else:
            assert nq == 0


@pytest.mark.parametrize("kbits,vbits,G,R", [(2, 2, 32, 32), (4, 2, 16, 128), (4, 4, 32, 0)])
def test_prefill_equals_prefill_plus_appends(orc, kbits, vbits, G, R):
    rng_seed = 5 + G + R
    n_total, m = 500, 137
    kb = np.random.default_rng(rng_seed).standard_normal((n_total, 128)).astype(np.float16).view(np.uint16)
    vb = np.random.default_rng(rng_seed + 1).standard_normal((n_total, 128)).astype(np.float16).view(np.uint16)
    full = orc.StreamState.prefill(kb, vb, kbits, vbits, G, R, cap=n_total)
    inc = orc.StreamState.prefill(kb[:m], vb[:m], kbits, vbits, G, R, cap=n_total)
    flushes = 0
    for t in range(m, n_total):
        flushes += inc.append(kb[t], vb[t])
        assert inc.nq == orc.num_quantized(inc.n, G, R)
    assert flushes == (full.nq - orc.num_quantized(m, G, R)) // G
    assert inc.n == full.n and inc.nq == full.nq
    assert np.array_equal(inc.key_codes(), full.key_codes())
    assert np.array_equal(inc.value_codes(), full.value_codes())
    for a, b in zip(inc.key_meta() + inc.value_meta(), full.key_meta() + full.value_meta()):
        assert np.array_equal(a, b)


def test_dequantize_grid_aligned_multi_group_exact(orc):
    """Grid-aligned keys and values with a different (s, z) per (group,
    channel) and per token: dequantization must give back the input exactly,
    which fixes the group index (t // G) and the per-token value metadata."""
    rng = np.random.default_rng(31)
    G, R, n, bits = 32, 32, 32 * 5 + 40, 4
    x = np.zeros((n, 128))
    for g in range(n // G + 1):
        for c in range(128):
            cc, s, z = _grid_aligned(rng, G, bits)
            seg = x[g * G:(g + 1) * G, c]
            x[g * G:(g + 1) * G, c] = (z + cc * s)[: seg.shape[0]]
    v = np.zeros((n, 128))
    for t in range(n):
        cc, s, z = _grid_aligned(rng, 128, bits)
        v[t] = z + cc * s
    st = orc.StreamState.prefill(f16bits(x), f16bits(v), bits, bits, G, R)
    assert st.nq == 32 * 5
    kh, vh = st.dequantize()
    assert np.array_equal(kh, x.astype(np.float32))
    assert np.array_equal(vh, v.astype(np.float32))


# --------------------------------------------------------------------------
# Attention special cases ("KV cache compression: ...", section 2.2: the
# weights sum to 1; "KV cache compression" (jaedaily): softmax(q k^T/sqrt(d)))
# --------------------------------------------------------------------------

def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_attention_weights_sum_to_one(orc):
    q = _rand((8, 128), 1)
    k = _rand((300, 128), 2, 3.0)
    v = _rand((300, 128), 3)
    out, w = orc.attention(q, k, v, 128 ** -0.5, want_weights=True)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
    assert np.all(w >= 0)
    # the output is the weighted mean of the value rows
    assert np.allclose(out, w @ v.astype(np.float64), rtol=0, atol=1e-12)


def test_attention_constant_values(orc):
    q = _rand((4, 128), 4)
    k = _rand((77, 128), 5, 4.0)
    c = _rand((1, 128), 6)
    out = orc.attention(q, k, np.repeat(c, 77, axis=0), 0.1)
    assert np.allclose(out, np.repeat(c, 4, axis=0), atol=1e-6, rtol=0)


def test_attention_constant_keys_is_mean(orc):
    q = _rand((3, 128), 7)
    k = np.repeat(_rand((1, 128), 8), 50, axis=0)
    v = _rand((50, 128), 9)
    out = orc.attention(q, k, v, 128 ** -0.5)
    assert np.allclose(out, np.repeat(v.astype(np.float64).mean(axis=0, keepdims=True), 3, axis=0),
                       atol=1e-12, rtol=0)


def test_attention_single_token_and_empty(orc):
    q = _rand((2, 128), 10)
    k = _rand((1, 128), 11)
    v = _rand((1, 128), 12)
    assert np.array_equal(orc.attention(q, k, v, 0.3), np.repeat(v.astype(np.float64), 2, axis=0))
    out0 = orc.attention(q, np.zeros((0, 128), np.float32), np.zeros((0, 128), np.float32), 0.3)
    assert np.all(out0 == 0)


def test_attention_two_tokens_logistic(orc):
    """Two tokens: the weight of token 0 is the logistic function of the
    logit difference."""
    q = np.zeros((1, 128), np.float32)
    q[0, 3] = 1.0
    k = np.zeros((2, 128), np.float32)
    k[0, 3], k[1, 3] = 2.0, -1.0
    v = _rand((2, 128), 13)
    scale = 0.5
    out = orc.attention(q, k, v, scale)
    a = 1.0 / (1.0 + np.exp(-(scale * 2.0 - scale * -1.0)))
    assert np.allclose(out[0], a * v[0] + (1 - a) * v[1], atol=1e-13, rtol=0)


def test_attention_dominant_token_and_permutation(orc):
    q = _rand((2, 128), 14)
    k = _rand((64, 128), 15) * 0.01
    k[17] = q[0] * 50.0
    v = _rand((64, 128), 16)
    out = orc.attention(q, k, v, 1.0)
    assert np.allclose(out[0], v[17], atol=1e-9)
    perm = np.random.default_rng(17).permutation(64)
    out_p = orc.attention(q, k[perm], v[perm], 1.0)
    assert np.allclose(out, out_p, atol=1e-13, rtol=0)


def test_grid_aligned_quantized_attention_equals_unquantized(orc):
    """If every key and value lies on its own grid, quantization is lossless
    and attention over the quantized cache equals attention over the fp16
    inputs bit for bit."""
    rng = np.random.default_rng(41)
    G, R, n, bits = 16, 16, 16 * 6 + 9, 2
    x = np.zeros((n, 128))
    for g in range(n // G + 1):
        for c in range(128):
            cc, s, z = _grid_aligned(rng, G, bits)
            x[g * G:(g + 1) * G, c] = (z + cc * s)[: x[g * G:(g + 1) * G, c].shape[0]]
    v = np.zeros((n, 128))
    for t in range(n):
        cc, s, z = _grid_aligned(rng, 128, bits)
        v[t] = z + cc * s
    st = orc.StreamState.prefill(f16bits(x), f16bits(v), bits, bits, G, R)
    kh, vh = st.dequantize()
    q = _rand((4, 128), 42)
    assert np.array_equal(orc.attention(q, kh, vh, 0.125),
                          orc.attention(q, x.astype(np.float32), v.astype(np.float32), 0.125))


# --------------------------------------------------------------------------
# Byte accounting ("KV cache compression: ...", section 8.1;
# "KV cache compression" (jaedaily): M_KV = 2 L H_kv n d_h b)
# --------------------------------------------------------------------------

def test_bytes_closed_forms_golden(orc):
    g = _golden("bytes_70b_shape.json")
    L, H, d = g["shape"]["layers"], g["shape"]["kv_heads"], g["shape"]["head_dim"]
    assert orc.kv_bytes_closed_form(L, H, 1, d, 2) == g["bf16_bytes_per_token"]
    n = g["tokens_128k_section_8_1"]
    assert orc.kv_bytes_closed_form(L, H, n, d, 2) == g["bf16_total_at_128k_gib"] * 2 ** 30
    assert orc.kv_bytes_closed_form(L, H, 1, d, 1) == g["fp8_kib_per_token"] * 1024
    assert abs(orc.kv_bytes_closed_form(L, H, g["tokens_jaedaily"], d, 2) / 1e9
               - g["jaedaily_total_gb_approx"]) < 2.0
    # per-stream accounting summed over the 640 (layer, head) streams equals
    # the closed form for an unquantized cache
    assert orc.stream_bytes(n, d, 16, 16, 32, 128) * L * H == orc.kv_bytes_closed_form(L, H, n, d, 2)
    # INT4, G = 32, R = 128: codes 80 KiB per token (section 8.1)
    per_stream = orc.stream_bytes(n, d, 4, 4, 32, 128)
    nq = orc.num_quantized(n, 32, 128)
    codes = nq * d * 8 / 8
    assert codes * L * H / n == pytest.approx(g["int4_code_kib_per_token"] * 1024, rel=2e-3)
    kmeta = (nq // 32) * d * 4
    vmeta = nq * 4
    # the page's metadata formula counts per-channel pairs for K and V; the
    # key half of it is our key metadata
    assert kmeta * L * H / nq == g["int4_metadata_formula_kib_per_token"] * 1024 / 2
    assert vmeta * L * H / nq == 2.5 * 1024
    resid = (n - nq) * d * 4
    assert per_stream == codes + kmeta + vmeta + resid
    # 128 residual tokens of the 70B shape are 40 MiB (section 8.1, "40 MB")
    assert 128 * L * H * d * 4 == 40 * 2 ** 20


# --------------------------------------------------------------------------
# 8-bit formats ("KV cache compression: ...", section 3.1: FP8 E4M3 with a
# static per-head scale, or INT8 with a dynamic per-token scale; "KV
# compression and quantization", part B.1: both at half the fp16 bytes).
# The E4M3 codec is checked against torch's float8_e4m3fn conversion, an
# independent implementation of the same format.
# --------------------------------------------------------------------------

def _torch_e4m3(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_decode_every_code(orc):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # facts of the format: largest finite 448, smallest subnormal 2^-9, 1.0 = 0x38
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_fp8_encode_matches_torch(orc):
    rng = np.random.default_rng(8)
    mant = rng.random(200000) + 1.0
    expo = rng.integers(-12, 9, size=mant.size)
    x = mant * np.exp2(expo) * rng.choice([-1.0, 1.0], size=mant.size)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    # exact halfway points between neighbouring codes (ties, both parities)
    # and the floats just beside them
    vals = np.sort(orc.fp8_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64))
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1000))])
    edges = np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11,
                      2.0 ** -6, 1e-30], np.float32)
    for arr in (x, mid, -mid, near, -near, edges):
        assert np.array_equal(orc.fp8_encode(arr), _torch_e4m3(arr))
    # beyond the largest finite value the encoder saturates (the quantizer
    # clamps before encoding, so only +-448 itself reaches it from there)
    big = np.array([448.5, 464.0, 1e6, np.inf], np.float32)
    assert np.all(orc.fp8_encode(big) == 0x7E) and np.all(orc.fp8_encode(-big) == 0xFE)


def _fp8_bound(x, scale):
    """|x - x_hat| for one element under a static scale: half a step of a
    3-bit fraction (2^-4 relative) in the normal range, half the subnormal
    spacing (2^-10 scale) below it, plus the fp32 roundings of x/s and e*s."""
    return np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10) * (1 + 2.0 ** -20) + 1e-30


@pytest.mark.parametrize("G,R", [(32, 0), (16, 128)])
def test_fp8_roundtrip_bound_and_saturation(orc, G, R):
    rng = np.random.default_rng(81 + G)
    n = 300
    k = (rng.standard_normal((n, 128)) * np.exp2(rng.integers(-8, 6, size=(n, 1)))).astype(np.float16)
    v = (rng.standard_normal((n, 128)) * 3).astype(np.float16)
    ks, vs = 0.0125, 0.75    # about 5.6 and 336 at the top of the grid: k saturates in places
    st = orc.StreamState.prefill(k.view(np.uint16), v.view(np.uint16), 8, 8, G, R,
                                 fmt=orc.FMT_FP8, kscale=ks, vscale=vs)
    nq = st.nq
    assert nq == orc.num_quantized(n, G, R, orc.FMT_FP8) == (n if R == 0 else orc.num_quantized(n, G, R))
    kh, vh = st.dequantize()
    for x16, xh, sc in ((k, kh, ks), (v, vh, vs)):
        x = x16[:nq].astype(np.float64)
        sat = np.abs(x) > 448 * sc
        assert np.all(np.abs(x - xh[:nq])[~sat] <= _fp8_bound(x, sc)[~sat])
        assert np.array_equal(xh[:nq][sat], (np.sign(x[sat]) * np.float32(448 * sc)).astype(np.float32))
        assert np.array_equal(xh[nq:], x16[nq:].astype(np.float32))
    assert (np.abs(k[:nq].astype(np.float64)) > 448 * ks).any()
    # no per-token metadata in this format
    assert not st.key_meta()[0].any() and not st.value_meta()[0].any()


def test_fp8_grid_aligned_exact(orc):
    """Inputs that are E4M3 values times a power-of-two scale come back
    exactly, with the codes they were built from; the key and value scales
    are kept apart."""
    rng = np.random.default_rng(82)
    G, R, n = 16, 16, 16 * 6 + 5
    ks, vs = 2.0 ** -3, 2.0 ** 2
    ok = np.concatenate([np.arange(0, 0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    kc = rng.choice(ok, size=(n, 128)).astype(np.uint8)
    vc = rng.choice(ok, size=(n, 128)).astype(np.uint8)
    kx = (orc.fp8_decode(kc).astype(np.float64) * ks).astype(np.float16)
    vx = (orc.fp8_decode(vc).astype(np.float64) * vs).astype(np.float16)
    st = orc.StreamState.prefill(kx.view(np.uint16), vx.view(np.uint16), 8, 8, G, R,
                                 fmt=orc.FMT_FP8, kscale=ks, vscale=vs)
    nq = st.nq
    assert np.array_equal(st.key_codes(), kc[:nq]) and np.array_equal(st.value_codes(), vc[:nq])
    kh, vh = st.dequantize()
    assert np.array_equal(kh, kx.astype(np.float32)) and np.array_equal(vh, vx.astype(np.float32))


def test_int8_per_token_grid_aligned(orc):
    """INT8 is per token for keys as well as values: every key token gets its
    own (s, z), so tokens built on different grids come back with exactly
    the codes they were built from (a per-channel key grid would not)."""
    rng = np.random.default_rng(83)
    G, R, n = 32, 0, 32 * 3
    kx = np.zeros((n, 128))
    vx = np.zeros((n, 128))
    codes = {}
    meta = {}
    for name, x in (("k", kx), ("v", vx)):
        cs, S, Z = [], [], []
        for t in range(n):
            c, s, z = _grid_aligned(rng, 128, 8)
            x[t] = z + c * s
            cs.append(c)
            S.append(s)
            Z.append(z)
        codes[name] = np.array(cs)
        meta[name] = (f16bits(S), f16bits(Z))
    st = orc.StreamState.prefill(f16bits(kx), f16bits(vx), 8, 8, G, R, fmt=orc.FMT_INT8)
    assert st.nq == n
    assert np.array_equal(st.key_codes(), codes["k"]) and np.array_equal(st.value_codes(), codes["v"])
    for got, want in zip(st.key_meta() + st.value_meta(), meta["k"] + meta["v"]):
        assert np.array_equal(got, want)
    kh, vh = st.dequantize()
    assert np.array_equal(kh, kx.astype(np.float32)) and np.array_equal(vh, vx.astype(np.float32))


def test_int8_ties_to_even(orc):
    # s = 1, z = 0: the token spans 0..255; x.5 goes to the even neighbour
    tok = np.full(128, 7.0)
    tok[:8] = [0.0, 255.0, 0.5, 1.5, 2.5, 254.5, 127.5, 128.5]
    st = orc.StreamState.prefill(np.tile(f16bits(tok), (32, 1)), np.tile(f16bits(tok), (32, 1)),
                                 8, 8, 32, 0, fmt=orc.FMT_INT8)
    want = [0, 255, 0, 2, 2, 254, 128, 128]
    assert st.key_codes()[5, :8].tolist() == want and st.value_codes()[9, :8].tolist() == want
    assert orc.h2f(st.key_meta()[0][:1])[0] == 1.0 and orc.h2f(st.key_meta()[1][:1])[0] == 0.0


def test_int8_roundtrip_bound_and_extreme_codes(orc):
    from quantized_decode_attention_kivi_amd import synth
    w = synth.Workload("t", 1, 4, 2, 8, 8, 32, 128, context=1024 + 45, tag=84)
    K, V = synth.make_kv(w)
    kb = K.numpy().view(np.uint16)
    vb = V.numpy().view(np.uint16)
    for h in range(2):
        st = orc.StreamState.prefill(kb[0, h], vb[0, h], 8, 8, 32, 128, fmt=orc.FMT_INT8)
        nq = st.nq
        kh, vh = st.dequantize()
        for xb, xh, (s16, z16), c in ((kb[0, h], kh, st.key_meta(), st.key_codes()),
                                      (vb[0, h], vh, st.value_meta(), st.value_codes())):
            x = orc.h2f(xb[:nq]).astype(np.float64)
            s = orc.h2f(s16)[:, None]
            z = orc.h2f(z16)[:, None]
            assert np.all(np.abs(x - xh[:nq]) <= _roundtrip_bound(x, s, z, 8))
            assert np.all(c.min(axis=1) == 0) and np.all(c.max(axis=1) == 255)


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("G,R", [(32, 0), (16, 128), (32, 128)])
def test_8bit_prefill_equals_prefill_plus_appends(orc, fmt, G, R):
    n_total, m = 420, 101
    rng = np.random.default_rng(85 + G + R + fmt)
    kb = (rng.standard_normal((n_total, 128)) * 4).astype(np.float16).view(np.uint16)
    vb = rng.standard_normal((n_total, 128)).astype(np.float16).view(np.uint16)
    kw = dict(fmt=fmt, kscale=0.02, vscale=0.01)
    full = orc.StreamState.prefill(kb, vb, 8, 8, G, R, cap=n_total, **kw)
    inc = orc.StreamState.prefill(kb[:m], vb[:m], 8, 8, G, R, cap=n_total, **kw)
    for t in range(m, n_total):
        inc.append(kb[t], vb[t])
        assert inc.nq == orc.num_quantized(inc.n, G, R, fmt)
        assert inc.nq == (inc.n if R == 0 else orc.num_quantized(inc.n, G, R))
    assert inc.n == full.n and inc.nq == full.nq
    assert np.array_equal(inc.key_codes(), full.key_codes())
    assert np.array_equal(inc.value_codes(), full.value_codes())
    for a, b in zip(inc.key_meta() + inc.value_meta(), full.key_meta() + full.value_meta()):
        assert np.array_equal(a, b)
    ka, va = inc.dequantize()
    kf, vf = full.dequantize()
    assert np.array_equal(ka, kf) and np.array_equal(va, vf)


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("G", [16, 32])
def test_8bit_quantized_on_write_without_residual(orc, fmt, G):
    """8-bit formats with R = 0 ("KV cache compression: quantization,
    eviction and sparse attention", section 3.1: the FP8 / INT8 cache holds
    every token in 8 bits): every token is quantized when it is written,
    whatever the group size, by the per-token quantizer alone (INT8: the
    8-bit min/max set quantizer over the token's channels; FP8: E4M3 under
    the static scale), and the stream keeps no fp16 token."""
    n, m = 2 * G + 5, G - 3        # ragged: neither count is a multiple of G
    rng = np.random.default_rng(90 + G + fmt)
    kb = (rng.standard_normal((n, 128)) * 3).astype(np.float16).view(np.uint16)
    vb = rng.standard_normal((n, 128)).astype(np.float16).view(np.uint16)
    kw = dict(fmt=fmt, kscale=0.02, vscale=0.01)
    st = orc.StreamState.prefill(kb[:m], vb[:m], 8, 8, G, 0, cap=n, **kw)
    assert (st.n, st.nq) == (m, m)
    for t in range(m, n):
        st.append(kb[t], vb[t])
        assert st.nq == st.n == t + 1
    for t in range(n):
        for x, codes, meta, sc in ((kb[t], st.key_codes()[t], st.key_meta(), kw["kscale"]),
                                   (vb[t], st.value_codes()[t], st.value_meta(), kw["vscale"])):
            if fmt == orc.FMT_INT8:
                c, s16, z16 = orc.quantize_value_token(x, 8)
                assert np.array_equal(codes, c) and meta[0][t] == s16 and meta[1][t] == z16
            else:
                assert np.array_equal(codes, orc.quantize_token_fp8(x, sc))
    kh, vh = st.dequantize()
    assert st.residual()[0].shape[0] == 0
    # no token is returned exactly as stored: every one went through its codes
    assert not np.array_equal(kh, orc.h2f(kb)) and not np.array_equal(vh, orc.h2f(vb))


def test_8bit_bytes_golden(orc):
    """FP8 holds 160 KiB per token for the 80-layer, 8-kv-head, d = 128 shape
    (section 8.1), half the fp16 cache (part B.1); INT8 adds two fp16 pairs
    per token and head."""
    g = _golden("bytes_70b_shape.json")
    L, H, d = g["shape"]["layers"], g["shape"]["kv_heads"], g["shape"]["head_dim"]
    n = 4096
    fp8 = orc.stream_bytes(n, d, 8, 8, 32, 0, fmt=orc.FMT_FP8)
    int8 = orc.stream_bytes(n, d, 8, 8, 32, 0, fmt=orc.FMT_INT8)
    assert fp8 * L * H / n == g["fp8_kib_per_token"] * 1024
    assert fp8 == orc.kv_bytes_closed_form(1, 1, n, d, 1)
    assert fp8 / orc.stream_bytes(n, d, 16, 16, 32, 0) == 0.5
    assert int8 == fp8 + n * 8
    # with a residual window the newest tokens are counted at fp16
    assert orc.stream_bytes(n, d, 8, 8, 32, 128, fmt=orc.FMT_FP8) == (n - 128) * 256 + 128 * 512


# --------------------------------------------------------------------------
# Pre-RoPE keys rotated on read ("KV cache compression: ...", section 3.3:
# quantize keys before RoPE, apply RoPE when reading; section 2: RoPE rotates
# pairs of dimensions and keeps each pair's norm; "KV Cache compression lab",
# experiment 03: the pair is two adjacent dimensions).  The rotation is
# checked against complex multiplication by exp(i t theta_i), a formulation
# of its own, and against the properties that define RoPE.
# --------------------------------------------------------------------------

def _rope_complex(k, base, pos0=0):
    """Independent formulation: pair (2i, 2i+1) as the complex number
    k[2i] + i k[2i+1], multiplied by exp(i t base^(-i/64)) (d = 128)."""
    n, d = k.shape
    z = k[:, 0::2].astype(np.float64) + 1j * k[:, 1::2].astype(np.float64)
    freq = np.power(float(base), -np.arange(d // 2) / (d / 2))
    t = (pos0 + np.arange(n))[:, None].astype(np.float64)
    r = z * np.exp(1j * t * freq[None, :])
    out = np.empty((n, d))
    out[:, 0::2], out[:, 1::2] = r.real, r.imag
    return out


@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_rope_unit_pairs_closed_form(orc, base):
    for i in (0, 1, 17, 32, 63):
        for pos in (0, 1, 5, 1000, 131071):
            th = base ** (-i / 64.0)
            for which, want in ((0, (np.cos(pos * th), np.sin(pos * th))), (1, (-np.sin(pos * th), np.cos(pos * th)))):
                k = np.zeros((1, 128), np.float32)
                k[0, 2 * i + which] = 1.0
                r = orc.rope_rotate(k, base, pos0=pos)[0]
                assert abs(r[2 * i] - want[0]) < 1e-12 and abs(r[2 * i + 1] - want[1]) < 1e-12
                r[2 * i: 2 * i + 2] = 0
                assert not r.any()


def test_rope_matches_complex_rotation_norms_and_identity(orc):
    rng = np.random.default_rng(90)
    k = (rng.standard_normal((300, 128)) * 3).astype(np.float32)
    for base, pos0 in ((10000.0, 0), (500000.0, 77777)):
        r = orc.rope_rotate(k, base, pos0=pos0)
        assert np.allclose(r, _rope_complex(k, base, pos0), rtol=0, atol=1e-9)
        kk = k.astype(np.float64)
        assert np.allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, kk[:, 0::2] ** 2 + kk[:, 1::2] ** 2, atol=1e-9)
    assert np.array_equal(orc.rope_rotate(k[:1], 10000.0, pos0=0)[0], k[0].astype(np.float64))


def test_rope_relative_position(orc):
    """RoPE(q, m) . RoPE(k, n) depends on m - n only."""
    rng = np.random.default_rng(91)
    q = rng.standard_normal((1, 128)).astype(np.float32)
    k = rng.standard_normal((1, 128)).astype(np.float32)
    for m, n in ((10, 3), (5000, 4993), (131000, 130993)):
        a = orc.rope_rotate(q, 500000.0, m)[0] @ orc.rope_rotate(k, 500000.0, n)[0]
        b = orc.rope_rotate(q, 500000.0, m - n)[0] @ k[0].astype(np.float64)
        assert abs(a - b) < 1e-8 * (1 + abs(b))


def test_attention_rope_matches_rotated_keys(orc):
    """Attention over pre-RoPE keys rotated on read equals plain fp64
    attention over keys rotated beforehand (complex formulation), with
    positions 0 .. n-1."""
    rng = np.random.default_rng(92)
    n, gq = 70, 3
    q = rng.standard_normal((gq, 128)).astype(np.float32)
    k = (rng.standard_normal((n, 128)) * 2).astype(np.float32)
    v = rng.standard_normal((n, 128)).astype(np.float32)
    got = orc.attention_rope(q, k, v, 128 ** -0.5, 500000.0)
    kr = _rope_complex(k, 500000.0)
    lg = (q.astype(np.float64) @ kr.T) * np.float64(np.float32(128 ** -0.5))
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(got, p @ v.astype(np.float64), rtol=0, atol=1e-12)


def test_attention_rope_single_token_constant_values_and_empty(orc):
    """Pre-RoPE attention, cases fixed whatever the rotation does: one token
    gives its value row; equal value rows give that row; no tokens give 0."""
    rng = np.random.default_rng(94)
    q = rng.standard_normal((3, 128)).astype(np.float32)
    k = (rng.standard_normal((1, 128)) * 5).astype(np.float32)
    v = rng.standard_normal((1, 128)).astype(np.float32)
    assert np.array_equal(orc.attention_rope(q, k, v, 0.3, 10000.0), np.repeat(v.astype(np.float64), 3, axis=0))
    k = (rng.standard_normal((90, 128)) * 5).astype(np.float32)
    c = rng.standard_normal((1, 128)).astype(np.float32)
    out = orc.attention_rope(q, k, np.repeat(c, 90, axis=0), 128 ** -0.5, 500000.0)
    assert np.allclose(out, np.repeat(c.astype(np.float64), 3, axis=0), atol=1e-6, rtol=0)
    e = np.zeros((0, 128), np.float32)
    assert np.all(orc.attention_rope(q, e, e, 0.3, 10000.0) == 0)


def test_attention_rope_zero_and_counter_rotated_keys_give_the_mean(orc):
    """All rotated keys equal -> equal logits -> the mean value row.  Zero
    keys stay zero under any rotation; keys built as one vector turned back
    by their own position's angles (complex multiplication by
    exp(-i t theta_j)) come out of the rotation as that vector again."""
    rng = np.random.default_rng(95)
    n, base = 200, 10000.0
    q = (rng.standard_normal((2, 128)) * 3).astype(np.float32)
    v = rng.standard_normal((n, 128)).astype(np.float32)
    mean = np.repeat(v.astype(np.float64).mean(axis=0, keepdims=True), 2, axis=0)
    out = orc.attention_rope(q, np.zeros((n, 128), np.float32), v, 128 ** -0.5, base)
    assert np.allclose(out, mean, atol=1e-12, rtol=0)
    c = rng.standard_normal(128)
    z = c[0::2] + 1j * c[1::2]
    freq = np.power(base, -np.arange(64) / 64.0)
    back = z[None, :] * np.exp(-1j * np.arange(n)[:, None] * freq[None, :])
    k = np.empty((n, 128))
    k[:, 0::2], k[:, 1::2] = back.real, back.imag
    out = orc.attention_rope(q, k.astype(np.float32), v, 128 ** -0.5, base)
    assert np.allclose(out, mean, atol=1e-5, rtol=0)
    # the plain attention over the same (unrotated) keys is not the mean
    assert np.abs(orc.attention(q, k.astype(np.float32), v, 128 ** -0.5) - mean).max() > 1e-2


def test_attention_rope_two_tokens_logistic(orc):
    """Two tokens at positions 0 and 1, keys on one channel pair: token 0 is
    not rotated, token 1's pair i turns by theta_i = base^(-i/64) radians.
    The weight of token 0 is the logistic function of the logit difference
    worked out by hand for each pair and channel."""
    scale = 0.5
    for base in (10000.0, 500000.0):
        for i in (0, 5, 63):
            th = base ** (-i / 64.0)
            for ch, a, b in ((2 * i, 3.0, 2.0), (2 * i + 1, -1.0, 4.0)):
                q = np.zeros((1, 128), np.float32)
                q[0, ch] = 1.0
                k = np.zeros((2, 128), np.float32)
                k[0, 2 * i], k[1, 2 * i] = a, b          # both keys on the pair's first channel
                v = _rand((2, 128), 96 + i)
                # rotated token 1: (b cos th, b sin th) on channels (2i, 2i+1)
                l0 = a if ch == 2 * i else 0.0
                l1 = b * np.cos(th) if ch == 2 * i else b * np.sin(th)
                w0 = 1.0 / (1.0 + np.exp(-scale * (l0 - l1)))
                out = orc.attention_rope(q, k, v, scale, base)
                assert np.allclose(out[0], w0 * v[0] + (1 - w0) * v[1], atol=1e-12, rtol=0), (base, i, ch)


def test_pre_rope_quantization_narrows_key_ranges(orc):
    """Section 3.3's reason for quantizing before RoPE: on keys whose outlier
    channels are consistently large (the "bright vertical lines" of
    experiment 03), per-channel 2-bit quantization of the pre-RoPE keys,
    rotated afterwards, errs less than quantizing the rotated keys."""
    rng = np.random.default_rng(93)
    n, G, base = 32 * 32, 32, 10000.0
    k = rng.standard_normal((n, 128))
    for c in (4, 9, 70, 101):                         # fixed outlier channels, same sign every token
        k[:, c] = 20.0 + rng.standard_normal(n)
    k16 = k.astype(np.float16)
    kf = k16.astype(np.float32)
    exact = orc.rope_rotate(kf, base)

    def quant_groups(x16):
        out = np.zeros(x16.shape, np.float64)
        xb = x16.view(np.uint16)
        for g in range(n // G):
            c, s, z = orc.quantize_key_group(xb[g * G:(g + 1) * G], 2)
            out[g * G:(g + 1) * G] = c * orc.h2f(s)[None, :].astype(np.float64) + orc.h2f(z)[None, :]
        return out

    pre = orc.rope_rotate(quant_groups(k16).astype(np.float32), base)
    post = quant_groups(exact.astype(np.float16))
    err_pre = np.mean((pre - exact) ** 2)
    err_post = np.mean((post - exact) ** 2)
    assert err_pre < 0.5 * err_post, (err_pre, err_post)


# --------------------------------------------------------------------------
# Non-uniform grid ("KV cache compression: ...", section 3.3: KVQuant's
# levels at quantiles of the distribution, like NF4).  The levels are checked
# against scipy's normal quantile function (an implementation of its own),
# the quantizer against the uniform rule it reduces to with levels 0..Q, and
# the grid's purpose: lower 2-bit error than the uniform grid on normal data.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_levels_are_normal_quantiles(orc, bits):
    from scipy.special import ndtri
    n, Q = 1 << bits, (1 << bits) - 1
    F = orc.lib().orc_codebook_scale(bits)
    assert F * Q <= 255 < 2 * F * Q and F & (F - 1) == 0
    c = ndtri((np.arange(n) + 0.5) / n)
    want = np.rint(F * Q * (c - c[0]) / (c[-1] - c[0])) / F
    lev = orc.codebook_levels(bits)
    assert np.array_equal(lev, want)
    assert lev[0] == 0 and lev[-1] == Q and np.all(np.diff(lev) > 0)
    assert np.array_equal(lev + lev[::-1], np.full(n, float(Q)))      # symmetric, like the normal


@pytest.mark.parametrize("bits", [2, 4])
def test_codebook_with_identity_levels_is_the_uniform_rule(orc, bits):
    rng = np.random.default_rng(100 + bits)
    x = rng.standard_normal((32, 128)).astype(np.float16).view(np.uint16)
    ident = np.arange(1 << bits, dtype=np.float64)
    a = orc.quantize_key_group(x, bits)
    b = orc.quantize_key_group_cb(x, bits, levels=ident)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    g = _golden("tie_to_even_int2.json")           # ties included
    vals = np.tile(np.array(g["values"])[:, None], (1, 128))
    codes, _, _ = orc.quantize_key_group_cb(f16bits(vals), 2, levels=np.arange(4.0))
    assert codes[:, 0].tolist() == g["expected_codes"]


@pytest.mark.parametrize("bits", [2, 4])
def test_codebook_grid_aligned_and_ties(orc, bits):
    """Values on the codebook's levels (power-of-two step, exact in fp16)
    come back with their codes and exactly; values on a midpoint between two
    levels go to the even code."""
    rng = np.random.default_rng(110 + bits)
    lev = orc.codebook_levels(bits)
    Q = (1 << bits) - 1
    s, z = 2.0 ** -3, -1.5
    codes = rng.integers(0, Q + 1, size=(32, 128))
    codes[0], codes[1] = 0, Q
    x = z + s * lev[codes]
    got, gs, gz = orc.quantize_key_group_cb(f16bits(x), bits)
    assert np.array_equal(got, codes)
    assert np.all(orc.h2f(gs) == s) and np.all(orc.h2f(gz) == z)
    mids = (lev[:-1] + lev[1:]) / 2
    tok = np.concatenate([[z, z + s * Q], z + s * mids, np.full(128 - 2 - Q, z)])
    c2, _, _ = orc.quantize_value_token_cb(f16bits(tok), bits)
    k = np.arange(Q)
    assert c2[2:2 + Q].tolist() == np.where(k % 2 == 0, k, k + 1).tolist()


def test_codebook_beats_uniform_at_2_bits(orc):
    """The quantile grid's purpose: lower 2-bit error than the uniform grid
    on normally distributed key groups (32 tokens per channel) and value
    tokens (128 channels)."""
    rng = np.random.default_rng(120)
    k = rng.standard_normal((32 * 64, 128)).astype(np.float16)
    v = rng.standard_normal((256, 128)).astype(np.float16)

    def rel(x16, xh):
        x = x16.astype(np.float64)
        return np.mean((x - xh) ** 2) / np.mean(x ** 2)

    for cb in (False, True):
        st = orc.StreamState.prefill(k.view(np.uint16), np.resize(v, k.shape).view(np.uint16), 2, 2, 32, 0,
                                     grid=orc.GRID_CODEBOOK if cb else orc.GRID_UNIFORM)
        kh, vh = st.dequantize()
        if cb:
            ek_cb, ev_cb = rel(k, kh), rel(np.resize(v, k.shape), vh)
        else:
            ek_u, ev_u = rel(k, kh), rel(np.resize(v, k.shape), vh)
    assert ek_cb < 0.97 * ek_u and ev_cb < 0.93 * ev_u, (ek_cb, ek_u, ev_cb, ev_u)


@pytest.mark.parametrize("kbits,vbits,G,R", [(2, 2, 32, 32), (4, 2, 16, 128), (4, 4, 32, 0)])
def test_codebook_roundtrip_and_prefill_equals_appends(orc, kbits, vbits, G, R):
    n_total, m = 400, 111
    rng = np.random.default_rng(130 + G + R)
    kb = (rng.standard_normal((n_total, 128)) * 3).astype(np.float16).view(np.uint16)
    vb = rng.standard_normal((n_total, 128)).astype(np.float16).view(np.uint16)
    cb = orc.GRID_CODEBOOK
    full = orc.StreamState.prefill(kb, vb, kbits, vbits, G, R, cap=n_total, grid=cb)
    inc = orc.StreamState.prefill(kb[:m], vb[:m], kbits, vbits, G, R, cap=n_total, grid=cb)
    for t in range(m, n_total):
        inc.append(kb[t], vb[t])
    assert inc.nq == full.nq == orc.num_quantized(n_total, G, R)
    for a, b in zip((inc.key_codes(), inc.value_codes()) + inc.key_meta() + inc.value_meta(),
                    (full.key_codes(), full.value_codes()) + full.key_meta() + full.value_meta()):
        assert np.array_equal(a, b)
    kh, vh = full.dequantize()
    nq = full.nq
    for xb, xh, bits, (s16, z16), per_tok, codes in (
            (kb, kh, kbits, full.key_meta(), False, full.key_codes()),
            (vb, vh, vbits, full.value_meta(), True, full.value_codes())):
        lev = orc.codebook_levels(bits)
        gap = np.max(np.diff(lev))
        x = orc.h2f(xb[:nq]).astype(np.float64)
        sf = orc.h2f(s16)[:, None] if per_tok else np.repeat(orc.h2f(s16), G, axis=0)
        zf = orc.h2f(z16)[:, None] if per_tok else np.repeat(orc.h2f(z16), G, axis=0)
        bound = sf * gap / 2 + (1 << bits) * sf * 2.0 ** -11 + 4 * 2.0 ** -24 * (np.abs(x) + np.abs(zf) + 16 * sf)
        assert np.all(np.abs(x - xh[:nq]) <= bound)
        c = codes.reshape(-1, G, 128) if not per_tok else codes
        ax = 1 if not per_tok else 1
        assert np.all(c.min(axis=ax) == 0) and np.all(c.max(axis=ax) == (1 << bits) - 1)


# --------------------------------------------------------------------------
# Dense-and-sparse keys ("KV Cache compression lab", experiment 03, closing
# paragraph: KVQuant keeps the few extreme values in fp16 as a sparse matrix
# and quantizes the rest).  Selection checked by brute force (numpy's own
# sort), the dense part against the plain set quantizer on what is left.
# --------------------------------------------------------------------------

def _ds_group(rng, G, outlier_channels=(3, 70), gain=20.0):
    x = rng.standard_normal((G, 128))
    for c in outlier_channels:
        x[:, c] *= gain
    x[0, 5] = x[1, 5] = 7.0          # equal magnitudes: ties broken by position
    x[2, 6] = -7.0
    return x.astype(np.float16)


@pytest.mark.parametrize("G", [16, 32])
def test_ds_selection_is_the_largest_magnitudes(orc, G):
    rng = np.random.default_rng(140 + G)
    for trial in range(5):
        x = _ds_group(rng, G, gain=[1.0, 20.0, 3.0, 20.0, 50.0][trial])
        codes, s16, z16, pos, val = orc.quantize_key_group_ds(x.view(np.uint16), 2, G)
        mag = np.abs(x.astype(np.float64)).ravel()
        order = np.lexsort((np.arange(mag.size), -mag))        # by |x| descending, then position
        want = np.sort(order[:G])
        assert np.array_equal(pos.astype(np.int64), want)
        assert np.array_equal(val, x.view(np.uint16).ravel()[want])
        assert np.all(codes.ravel()[want] == 0)


def test_ds_ties_at_the_boundary_go_to_the_lower_position(orc):
    """G - 1 clearly largest entries, then three of equal magnitude (+-50)
    competing for the last place: the lowest position wins."""
    G = 32
    x = np.random.default_rng(152).standard_normal((G, 128))
    big = [(t, (7 * t) % 128) for t in range(G - 1)]
    for i, (t, c) in enumerate(big):
        x[t, c] = 100.0 + i
    x[20, 100], x[5, 64], x[9, 1] = 50.0, -50.0, 50.0
    codes, s16, z16, pos, val = orc.quantize_key_group_ds(x.astype(np.float16).view(np.uint16), 2, G)
    want = sorted([t * 128 + c for t, c in big] + [5 * 128 + 64])
    assert pos.tolist() == want


def test_ds_dense_part_is_the_set_quantizer_on_the_rest(orc):
    rng = np.random.default_rng(150)
    G = 32
    x = _ds_group(rng, G)
    xb = x.view(np.uint16)
    codes, s16, z16, pos, val = orc.quantize_key_group_ds(xb, 2, G)
    kept = np.zeros(G * 128, bool)
    kept[pos] = True
    kept = kept.reshape(G, 128)
    for c in range(128):
        rest = xb[~kept[:, c], c]
        if rest.size == 0:
            assert s16[c] == 0 and z16[c] == 0
            continue
        cc, s, z = orc.quantize_value_token(rest, 2)       # the plain min/max set quantizer
        assert np.array_equal(codes[~kept[:, c], c], cc) and s16[c] == s and z16[c] == z


def test_ds_channel_with_no_dense_values(orc):
    """A channel whose every value is among the group's largest keeps them
    all; its scale and zero are 0."""
    G = 16
    x = np.random.default_rng(151).standard_normal((G, 128)).astype(np.float16)
    x[:, 9] = (100 + np.arange(G)).astype(np.float16)
    codes, s16, z16, pos, val = orc.quantize_key_group_ds(x.view(np.uint16), 4, G)
    assert np.array_equal(pos, np.arange(G) * 128 + 9)
    assert s16[9] == 0 and z16[9] == 0


@pytest.mark.parametrize("G,R", [(32, 0), (16, 128), (32, 64)])
def test_ds_stream_roundtrip_and_appends(orc, G, R):
    n_total, m = 420, 97
    rng = np.random.default_rng(160 + G + R)
    k = rng.standard_normal((n_total, 128))
    k[:, [3, 77]] *= 20
    kb = k.astype(np.float16).view(np.uint16)
    vb = rng.standard_normal((n_total, 128)).astype(np.float16).view(np.uint16)
    full = orc.StreamState.prefill(kb, vb, 2, 2, G, R, cap=n_total, sparse=True)
    inc = orc.StreamState.prefill(kb[:m], vb[:m], 2, 2, G, R, cap=n_total, sparse=True)
    for t in range(m, n_total):
        inc.append(kb[t], vb[t])
    assert inc.nq == full.nq
    for a, b in zip((inc.key_codes(), inc.value_codes()) + inc.key_meta() + inc.value_meta() + inc.outliers(),
                    (full.key_codes(), full.value_codes()) + full.key_meta() + full.value_meta() + full.outliers()):
        assert np.array_equal(a, b)
    kh, _ = full.dequantize()
    nq = full.nq
    opos, oval = full.outliers()
    xk = orc.h2f(kb[:nq]).astype(np.float64)
    kept = np.zeros((nq // G, G * 128), bool)
    for g in range(nq // G):
        kept[g, opos[g]] = True
    kept = kept.reshape(nq, 128)
    assert np.array_equal(kh[:nq][kept], xk[kept].astype(np.float32))      # kept entries exact
    s = np.repeat(orc.h2f(full.key_meta()[0]), G, axis=0)
    z = np.repeat(orc.h2f(full.key_meta()[1]), G, axis=0)
    err = np.abs(xk - kh[:nq])
    assert np.all(err[~kept] <= _roundtrip_bound(xk, s, z, 2)[~kept])


def test_ds_codebook_dense_part_is_the_codebook_on_the_rest(orc):
    """Dense-and-sparse on the codebook grid: the kept extremes as on the
    uniform grid, the rest of each channel on the codebook quantizer."""
    rng = np.random.default_rng(153)
    G = 32
    x = _ds_group(rng, G)
    xb = x.view(np.uint16)
    st = orc.StreamState.prefill(xb, xb, 2, 2, G, 0, sparse=True, grid=orc.GRID_CODEBOOK)
    pos, val = st.outliers()
    u = orc.quantize_key_group_ds(xb, 2, G)
    assert np.array_equal(pos[0], u[3]) and np.array_equal(val[0], u[4])
    kept = np.zeros(G * 128, bool)
    kept[pos[0]] = True
    kept = kept.reshape(G, 128)
    codes = st.key_codes()
    s16, z16 = st.key_meta()
    for c in range(128):
        rest = xb[~kept[:, c], c]
        if rest.size:
            cc, s, z = orc.quantize_value_token_cb(rest, 2)
            assert np.array_equal(codes[~kept[:, c], c], cc) and s16[0, c] == s and z16[0, c] == z


def test_ds_lowers_key_error(orc):
    """The purpose: at 2 bits, keeping the few extreme keys exact lowers the
    key error of the synthetic keys (outlier channels) against per-channel
    quantization of everything."""
    from quantized_decode_attention_kivi_amd import synth
    w = synth.Workload("t", 1, 4, 1, 2, 2, 32, 0, context=2048, tag=79)
    K, _ = synth.make_kv(w)
    kb = K.numpy().view(np.uint16)[0, 0]
    x = orc.h2f(kb).astype(np.float64)
    errs = []
    for sparse in (False, True):
        st = orc.StreamState.prefill(kb, kb, 2, 2, 32, 0, sparse=sparse)
        kh, _ = st.dequantize()
        errs.append(np.mean((x - kh) ** 2))
    assert errs[1] < 0.8 * errs[0], errs


# --------------------------------------------------------------------------
# Mutation check: planted mistakes in a copy of the oracle must be caught
# --------------------------------------------------------------------------

MUTATIONS = [
    ("rintf(t)", "floorf(t + 0.5f)", "ties"),                           # wrong rounding rule
    ("if (R == 0) return n > 0 ? n : 0;", "if (0) return n;", "onwrite"),  # 8-bit waits for whole groups
    ("codes[(long)i * code_stride] = (uint8_t)r;",
     "codes[(long)i * code_stride] = (uint8_t)r; if (0) {}", None),     # no-op (control)
    ("(long)(t / G) * d + c", "(long)(t / G) * d", "dequant"),          # dropped channel index
    ("fmaf((float)vcodes[i], orc_h2f(vs[t]), orc_h2f(vz[t]))",
     "fmaf((float)vcodes[i], orc_h2f(vs[t]), 0.0f)", "dequant"),        # dropped zero point
    ("if (*n - *nq == R + G)", "if (*n - *nq == R)", "append"),         # wrong flush condition
    ("logit[t] = exp(logit[t] - m);", "logit[t] = exp(logit[t]);", None),  # still exact (no overflow here)
    ("p = logit[t] / l;", "p = logit[t];", "attn"),                     # dropped normalisation
    ("p = logit[t] / l;", "p = logit[t];", "attnrope"),                 # the same, seen by the pre-RoPE pins
    ("(kf ? (double)kf[i] : kd[i])", "(kf ? (double)kf[i] : 0.5 * kd[i])", "attnrope"),  # fp64 keys misread
    ("logit[t] = (double)scale * acc;", "logit[t] = acc;", "attnrope"),   # softmax scale dropped
    ("logit[t] = (double)scale * acc;", "logit[t] = acc;", "attn2"),      # the same, plain attention
    ("mn = mn + 0.0f;", "mn = mn;", "negzero"),                        # -0 not canonicalised
    ("double m = rint(ldexp(a, 3 - e));", "double m = floor(ldexp(a, 3 - e) + 0.5);", "fp8enc"),  # ties away
    ("v = ldexp((double)(frac + 8), expo - 10);", "v = ldexp((double)(frac + 8), expo - 9);", "fp8dec"),
    ("quantize_token8(fmt, k + (long)t * d, d, kscale,", "quantize_token8(fmt, k + (long)t * d, d, vscale,",
     "fp8grid"),                                                        # key/value scales swapped
    ("out_k[i] = orc_fp8_e4m3_decode(kcodes[i]) * kscale;",
     "out_k[i] = orc_fp8_e4m3_decode(kcodes[i]);", "fp8grid"),          # scale not applied
    ("quantize_set(x, d, 1, 8, codes, 1, s, z);", "quantize_set(x, d, 1, 7, codes, 1, s, z);", "int8grid"),
    ("out[(long)t * d + 2 * i] = x0 * c - x1 * s;", "out[(long)t * d + 2 * i] = x0 * c + x1 * s;",
     "rope"),                                                           # rotation sign
    ("double theta = pow(base, -2.0 * (double)i / (double)d);",
     "double theta = pow(base, -1.0 * (double)i / (double)d);", "rope"),  # wrong frequencies
    ("double a = (double)(pos0 + t) * theta;", "double a = (double)(pos0 + t + 1) * theta;", "rope"),  # positions from 1
    ("if ((k % 2 == 0) ? (t > m) : (t >= m)) code += 1;", "if (t > m) code += 1;", "cbtie"),  # ties always down
    ("for (int k = 0; k < n; ++k) c[k] = normal_quantile((k + 0.5) / n);",
     "for (int k = 0; k < n; ++k) c[k] = normal_quantile((k + 1.0) / (n + 1));", "cblev"),  # other quantiles
    ("out_k[i] = fmaf((float)klev[kcodes[i]], orc_h2f(ks[gi]), orc_h2f(kz[gi]));",
     "out_k[i] = fmaf((float)kcodes[i], orc_h2f(ks[gi]), orc_h2f(kz[gi]));", "cbdeq"),  # LUT skipped
    ("return p->pos < q->pos ? -1 : (p->pos > q->pos ? 1 : 0);",
     "return p->pos > q->pos ? -1 : (p->pos < q->pos ? 1 : 0);", "dssel"),   # ties to the higher position
    ("            if (kept[t * d + c]) continue;\n            float v = orc_h2f(x[t * d + c]);",
     "            float v = orc_h2f(x[t * d + c]);", "dsdense"),                 # kept values in the range
    ("out_k[(long)g * G * d + p] = orc_h2f(oval[(long)g * n_out + e]);",
     "(void)p;", "dsdeq"),                                                    # kept values not restored
]


def test_pin_catches_planted_mistakes(tmp_path):
    """Build broken copies of the oracle and check the pins above fail on
    them (the control mutations must keep passing)."""
    src = open(os.path.join(os.path.dirname(__file__), "..", "oracle", "kvq_oracle.c")).read()
    here = os.path.dirname(__file__)
    sel = {
        "ties": "test_ties_to_even_golden",
        "dequant": "test_dequantize_grid_aligned_multi_group_exact",
        "append": "test_prefill_equals_prefill_plus_appends",
        "attn": "test_attention_weights_sum_to_one",
        "attn2": "test_attention_two_tokens_logistic",
        "attnrope": "attention_rope",
        "negzero": "test_negative_zero_extremes_canonicalised",
        "fp8enc": "test_fp8_encode_matches_torch",
        "fp8dec": "test_fp8_decode_every_code",
        "fp8grid": "test_fp8_grid_aligned_exact",
        "int8grid": "test_int8_per_token_grid_aligned",
        "rope": "test_rope_unit_pairs_closed_form",
        "cbtie": "test_codebook_grid_aligned_and_ties",
        "cblev": "test_codebook_levels_are_normal_quantiles",
        "cbdeq": "test_codebook_roundtrip_and_prefill_equals_appends",
        "dssel": "test_ds_ties_at_the_boundary_go_to_the_lower_position",
        "dsdense": "test_ds_dense_part_is_the_set_quantizer_on_the_rest",
        "dsdeq": "test_ds_stream_roundtrip_and_appends",
        "onwrite": "test_8bit_quantized_on_write_without_residual",
    }
    for i, (old, new, which) in enumerate(MUTATIONS):
        assert old in src, old
        if which is None:
            continue
        d = tmp_path / ("m%d" % i)
        d.mkdir()
        (d / "oracle").mkdir()
        (d / "oracle" / "kvq_oracle.c").write_text(src.replace(old, new, 1))
        py = open(os.path.join(here, "..", "oracle", "__init__.py")).read()
        (d / "oracle" / "__init__.py").write_text(py)
        env = dict(os.environ, PYTHONPATH=str(d) + os.pathsep + os.path.join(here, ".."))
        code = ("import sys; sys.path.insert(0, %r); import oracle; oracle.build();"
                "import importlib; import pytest;"
                "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r, '-k', %r,"
                " '--rootdir', %r]))") % (str(d), os.path.join(here, "test_oracle_pins.py"),
                                          sel[which], str(d))
        r = subprocess.run(["python", "-c", code], env=env, capture_output=True, text=True, cwd=str(d))
        assert r.returncode != 0, "mutation %d (%s) was not caught:\n%s" % (i, new, r.stdout[-2000:])
