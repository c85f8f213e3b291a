"""The quantize kernel divides max − min by the code range 2^b − 1 (3 or 15)
as q = RN(x·y), y = RN(1/d), then fma(fma(−q, d, x), y, q), and takes q
itself for ±0 and non-finite x. This checks that the sequence equals the
IEEE (correctly rounded) division bit for bit, run on the host in C:

* every fp32 pattern of the binades where the steps need not scale by
  powers of two: the subnormals and the normal binades below 2^-119 (the
  quotient can be subnormal there) and the top two binades (q·d can
  overflow);
* every pattern of one middle binade, [1, 2). Between those edges x and q
  are normal, the remainder x − q·d is a multiple of 2^-149 (q normal, d an
  integer) and so exact, and the correcting fma rounds once: scaling x by
  2^k scales every step by 2^k, so the middle binades behave alike;
* ±0, ±inf and NaN through the guard.

A mismatch anywhere fails with the first few inputs printed.
"""
import os
import shutil
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
    static float kernel_div(float x, float d, float y) {
      if (x == 0.0f || !isfinite(x)) return x * y;        /* the guard */
      const float q = x * y;
      const float r = fmaf(-q, d, x);
      return fmaf(r, y, q);
    }
    static long check_range(uint32_t lo, uint32_t hi, float d, float y) {
      long bad = 0;
      #pragma omp parallel for reduction(+ : bad) schedule(static, 65536)
      for (int64_t u = lo; u < (int64_t)hi; ++u)
        for (int s = 0; s < 2; ++s) {
          const float x = f_of((uint32_t)u | (s ? 0x80000000u : 0u));
          const float want = x / d, got = kernel_div(x, d, y);
          if (u_of(want) != u_of(got) && !(isnan(want) && isnan(got))) {
            if (bad < 5) printf("d=%g x=%a want=%a got=%a\n", d, x, want, got);
            ++bad;
          }
        }
      return bad;
    }
    int main(void) {
      long bad = 0;
      for (int k = 0; k < 2; ++k) {
        const float d = k ? 15.0f : 3.0f;
        volatile float dv = d;
        const float y = 1.0f / dv;
        const uint32_t B = 1u << 23;                      /* patterns per binade */
        bad += check_range(0, 8 * B, d, y);               /* subnormals .. 2^-119 */
        bad += check_range(127 * B, 128 * B, d, y);       /* [1, 2) */
        bad += check_range(253 * B, 255 * B, d, y);       /* [2^126, 2^128) */
        bad += check_range(255 * B, 255 * B + 2, d, y);   /* inf, a NaN */
      }
      printf("mismatches %ld\n", bad);
      return bad != 0;
    }
""")


def test_code_range_division_matches_ieee(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "div.c"
    src.write_text(SRC)
    exe = tmp_path / "div"
    # the host's fused multiply-add inline when it has one (else libm's fmaf,
    # also correctly rounded, but slower)
    with open("/proc/cpuinfo") as fh:
        fma = " fma " in fh.read().replace("\n", " ")
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    *(["-mfma"] if fma else []), str(src), "-o", str(exe), "-lm"], check=True)
    threads = str(max(1, min(8, len(os.sched_getaffinity(0)))))
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                       env={**os.environ, "OMP_NUM_THREADS": threads})
    assert r.returncode == 0, r.stdout[-2000:]
    assert "mismatches 0" in r.stdout
