"""Host checks of the two fp32 identities the HIP quantizer uses in place of
IEEE division when it forms a set's scale and reciprocal (the fixed formula
asks for s = fp16((max - min) / (2^b - 1)) and inv = 1/s, both correctly
rounded):

  * RN(x / Q) for Q = 3, 15, 255 equals q1 = fma(fma(-q0, Q, x), r, q0)
    with r = RN(1/Q) and q0 = RN(x r), for EVERY fp32 x in [0, 131008] (the
    range of max - min over finite fp16 inputs);
  * RN(1 / s) equals r1 = fma(fma(-s, r0, 1), r0, r0) for every positive
    finite fp16 s and EVERY starting value r0 within 1 ulp of 1/s (the
    hardware reciprocal's documented accuracy), whatever r0 it returns.

The reference quotients come from fp64 division rounded to fp32, which is
the correctly rounded fp32 quotient here: x / Q and 1 / s never fall on an
fp32 rounding midpoint (a midpoint has a finite binary expansion; x / Q for
Q odd has one only when Q divides x's integer significand, and then it is an
fp32 number of at most 24 bits; 1 / s likewise).  The check is plain C with
hardware or library fmaf, run over all inputs (about 3.6e9 quotients and
95,000 reciprocals)."""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(void) {
    long bad = 0;
    const float ds[3] = {3.0f, 15.0f, 255.0f};
    const uint32_t top = u_of(131008.0f);
    for (int k = 0; k < 3; ++k) {
        const float d = ds[k];
        const float r = (float)(1.0 / (double)d);
        long b = 0;
#pragma omp parallel for reduction(+ : b) schedule(static)
        for (long u = 0; u <= (long)top; ++u) {
            const float x = f_of((uint32_t)u);
            const float q0 = x * r;
            const float e = fmaf(-q0, d, x);
            const float q1 = fmaf(e, r, q0);
            const float want = (float)((double)x / (double)d);
            b += u_of(q1) != u_of(want);
        }
        bad += b;
    }
    for (uint32_t h = 1; h < 0x7c00; ++h) {
        const uint32_t e = (h >> 10) & 31, f = h & 1023;
        const double s = e ? ldexp(1.0 + f / 1024.0, (int)e - 15) : ldexp((double)f, -24);
        const float sf = (float)s;
        const float want = (float)(1.0 / s);
        for (int dl = -1; dl <= 1; ++dl) {
            const float r0 = f_of(u_of(want) + dl);
            const float r1 = fmaf(fmaf(-sf, r0, 1.0f), r0, r0);
            bad += u_of(r1) != u_of(want);
        }
    }
    printf("mismatches %ld\n", bad);
    return bad != 0;
}
"""


def test_division_free_scale_and_reciprocal_equal_ieee_division(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "divcheck.c"
    exe = tmp_path / "divcheck"
    src.write_text(SRC)
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    if b"fma" in open("/proc/cpuinfo", "rb").read():
        flags.append("-mfma")   # hardware fmaf (the library's is exact too, only slower)
    subprocess.run([gcc, *flags, "-o", str(exe), str(src), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0 and "mismatches 0" in r.stdout, r.stdout + r.stderr


CB4_SRC = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float mid[15];
/* the count of midpoints passed, ties to the even code */
static unsigned count_code(float t) {
    unsigned c = 0;
    for (int k = 0; k < 15; ++k) c += (k & 1) ? (t >= mid[k]) : (t > mid[k]);
    return c;
}
int main(int argc, char** argv) {
    for (int k = 0; k < 15; ++k) mid[k] = strtof(argv[1 + k], NULL);
    uint32_t thr[240], lo[240];
    for (int i = 0; i < 240; ++i) {
        lo[i] = count_code((float)i * 0.0625f);
        thr[i] = lo[i] < 15 ? ((lo[i] & 1) ? u_of(mid[lo[i]]) - 1 : u_of(mid[lo[i]])) : 0x7f800000u;
    }
    long bad = 0;
    /* every fp32 t in [-2, 18]: negative ones, then non-negative ones */
    const uint32_t neg_top = u_of(-2.0f), pos_top = u_of(18.0f);
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (long u = 0; u <= (long)pos_top + (long)(neg_top - 0x80000000u) + 1; ++u) {
        const uint32_t bits = u <= (long)pos_top ? (uint32_t)u : 0x80000000u + (uint32_t)(u - pos_top - 1);
        const float t = f_of(bits);
        int i = (int)(t * 16.0f);
        i = i < 0 ? 0 : i > 239 ? 239 : i;
        const unsigned got = lo[i] + (t > f_of(thr[i]));
        bad += got != count_code(t);
    }
    printf("mismatches %ld\n", bad);
    return bad != 0;
}
"""


def test_codebook_4bit_bin_table_equals_midpoint_count(tmp_path):
    """The 4-bit codebook quantizer's table form (bin floor(16 t) clamped to
    [0, 239], the count of midpoints passed at the bin's start, one more when
    t exceeds the bin's threshold) against the plain count of midpoints
    passed with ties to the even code, for every fp32 t in [-2, 18], on the
    library's 4-bit levels (the midpoints of neighbouring levels)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import numpy as np
    from quantized_decode_attention_kivi_amd import kvq
    lev = kvq.kvq_codebook_levels(4).astype(np.float32)
    mids = [(np.float32(lev[k]) + np.float32(lev[k + 1])) / np.float32(2) for k in range(15)]
    assert all(m > 0 for m in mids) and all(b - a > 1 / 16 for a, b in zip(mids, mids[1:]))
    src = tmp_path / "cb4.c"
    exe = tmp_path / "cb4"
    src.write_text(CB4_SRC)
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-fopenmp", "-o", str(exe), str(src)], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    r = subprocess.run([str(exe)] + ["%.9g" % m for m in mids], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0 and "mismatches 0" in r.stdout, r.stdout + r.stderr
