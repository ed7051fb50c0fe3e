"""The quantiser's division on the GPU computes fp32(x / s) as a multiply by
r = fp32(1 / s) followed by two FMA corrections (Markstein's FMA division).
This CPU test checks that identity against IEEE fp32 division, in C with the
host's correctly rounded fmaf: every finite bf16 x against thousands of
divisors s = fp32(a / 127) (a the row absmax), random fp32 x, and x built to
fall next to half-integer quotients, where a wrong last bit would change the
rounded int8 value."""
import os
import subprocess
import textwrap

import pytest

SRC = textwrap.dedent(r"""
    #include <math.h>
    #include <stdint.h>
    #include <stdio.h>
    #include <string.h>

    static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
    static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

    /* the device sequence, written out: q0 = x r; q1 = fma(fma(-q0, s, x), r, q0); q2 likewise */
    static float quotient_fma(float x, float s, float r) {
        volatile float q0 = x * r;
        float q1 = fmaf(fmaf(-q0, s, x), r, q0);
        return fmaf(fmaf(-q1, s, x), r, q1);
    }

    static uint64_t rng = 0x9E3779B97F4A7C15ull;
    static uint64_t next(void) {  /* SplitMix64 */
        uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }

    static long bad = 0, checked = 0, naive_bad = 0, one_step_bad = 0;
    static void check(float x, float s, float r) {
        /* only |x| <= 127.5 s matters (|x| <= absmax) and |x / s| >= 1/4 (else the value rounds to 0) */
        volatile float want = x / s;
        float got = quotient_fma(x, s, r);
        volatile float q0 = x * r;
        float q1 = fmaf(fmaf(-q0, s, x), r, q0);
        naive_bad += u_of(q0) != u_of(want);       /* the plain product: wrong in some cases */
        one_step_bad += u_of(q1) != u_of(want);    /* one correction: counted, for the record */
        ++checked;
        if (u_of(got) != u_of(want)) {
            if (bad < 5) printf("mismatch x=%a s=%a want=%a got=%a\n", x, s, want, got);
            ++bad;
        }
    }

    int main(void) {
        /* divisors: s = fp32(a / 127) for absmax a = every bf16 in [1e-5, 3e38) sampled, plus random fp32 a */
        float as[6000];
        int na = 0;
        for (uint32_t b = 0x3728; b < 0x7F00 && na < 3000; b += 5) as[na++] = f_of(b << 16);
        while (na < 6000) { float a = f_of((uint32_t)(next() & 0x7FFFFFFFu)); if (isfinite(a) && a >= 1e-5f && a < 1e37f) as[na++] = a; }
        for (int i = 0; i < na; ++i) {
            volatile float s = as[i] / 127.0f;
            volatile float r = 1.0f / s;
            float lim = as[i];
            /* every bf16 with 1/4 s <= |x| <= a */
            for (uint32_t h = 0; h < 0x7F80; ++h) {
                float x = f_of(h << 16);
                if (x > lim || x < 0.25f * s) continue;
                check(x, s, r);
                check(-x, s, r);
            }
            /* random fp32 x in [-a, a] */
            for (int j = 0; j < 300; ++j) {
                float t = (float)((next() >> 11) * 0x1.0p-53) * 2.0f - 1.0f;
                check(t * lim, s, r);
            }
            /* next to half-integer quotients: x = fp32((k + 1/2) s) and its fp32 neighbours */
            for (int k = 0; k < 127; ++k) {
                float x = (float)(k + 0.5) * s;
                for (int d = -3; d <= 3; ++d) {
                    float y = f_of(u_of(x) + d);
                    if (y <= lim) check(y, s, r);
                }
            }
        }
        printf("checked %ld bad %ld naive_bad %ld one_step_bad %ld\n", checked, bad, naive_bad, one_step_bad);
        return bad != 0;
    }
    """)


def test_fma_quotient_equals_ieee_division(tmp_path):
    c = tmp_path / "quotient.c"
    exe = tmp_path / "quotient"
    c.write_text(SRC)
    cc = os.environ.get("CC", "gcc")
    r = subprocess.run([cc, "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", str(c), "-o", str(exe), "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"no C compiler: {r.stderr[:200]}")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    assert " bad 0 " in r.stdout
    naive_bad = int(r.stdout.split("naive_bad ")[1].split()[0])
    assert naive_bad > 0, "the check must be able to fail: x * fp32(1/s) alone is not always correctly rounded"
