"""The reciprocal division the mass kernel relies on (host check, no GPU).

The pooling average at interior positions divides by the window count n
through y = RN(1/n): q = RN(a*y), r = fma(-n, q, a), RN(q + r*y).  The EMA
sweep and the prefix scan divide by a head's fixed totals the same way in
fp64.  For a reciprocal within half an ulp and a quotient q within one ulp,
the residual is exact and the corrected quotient is the correctly rounded
a/n (Markstein's theorem); the kernel uses the fp32 form only for sums in
[2^-80, 2^100], where no intermediate is subnormal.  This test compiles a
small C program with the host compiler and compares the identity against
IEEE division: every fp32 value in that range for n = 7 (the kernel's
pooling kernel) and n = 63 (the largest window), and sampled fp64 pairs of the kind
the sweeps divide (u64 totals up to 2^64), near-midpoint quotients included.
"""
import os
import shutil
import subprocess
import textwrap

import pytest

SOURCE = textwrap.dedent(r"""
    #include <math.h>
    #include <stdint.h>
    #include <stdio.h>
    #include <string.h>

    static uint64_t s = 88172645463325252ull;
    static uint64_t xr(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }

    static long check_f32(int n) {  /* every float in [2^-80, 2^100] */
      long bad = 0;
      volatile float nv = (float)n;
      const float y = 1.0f / nv;
      for (uint32_t b = 0x17800000u; b <= 0x71800000u; ++b) {
        float a; memcpy(&a, &b, 4);
        const float q = a * y;
        const float g = fmaf(fmaf(-nv, q, a), y, q);
        if (g != a / nv) ++bad;
      }
      return bad;
    }

    static long check_f64(long pairs) {
      long bad = 0;
      for (long i = 0; i < pairs; ++i) {
        const int db = 1 + (int)(xr() % 64);
        const uint64_t D = (xr() >> (64 - db)) | 1ull << (db - 1);
        const double d = (double)D, y = 1.0 / d;
        uint64_t A;
        if (i & 1) {
          A = xr() % (D + 1);
        } else {  /* a quotient next to a rounding midpoint */
          const double q0 = ldexp(1.0 + (double)(xr() >> 12) * 0x1p-52, -(int)(xr() % 40));
          const long double m = (long double)q0 + ldexpl(1.0L, ilogb(q0) - 53);
          const long double al = (long double)d * m;
          if (al >= 18446744073709551615.0L || al < 1) continue;
          A = (uint64_t)al + (xr() % 3) - 1;
          if (A > D) continue;
        }
        const double a = (double)A;
        const double q = a * y;
        const double g = fma(fma(-d, q, a), y, q);
        if (g != a / d) ++bad;
      }
      return bad;
    }

    int main(void) {
      const int ns[] = {7, 63};
      long bad = 0;
      for (int i = 0; i < 2; ++i) {
        const long b = check_f32(ns[i]);
        printf("f32 n=%d mismatches %ld\n", ns[i], b);
        bad += b;
      }
      const long b = check_f64(20000000);
      printf("f64 mismatches %ld\n", b);
      return (bad + b) != 0;
    }
""")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_reciprocal_division_is_correctly_rounded(tmp_path):
    src = tmp_path / "recip.c"
    exe = tmp_path / "recip"
    src.write_text(SOURCE)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), str(src), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert r.stdout.count("mismatches 0") == 3, r.stdout
