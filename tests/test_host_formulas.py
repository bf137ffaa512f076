"""Host checks of arithmetic identities the kernels rely on (no GPU): the
three-operation correctly rounded division by 6 used for single-level P
block scales (device_common.h, div6_rn), compared with IEEE binary32
division for every binary32 in several binades.  The device executes the
same IEEE operations (v_mul_f32, v_fma_f32 with round-to-nearest-even)."""
import os
import subprocess
import tempfile

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
  const float r = 1.0f / 6.0f;
  long bad = 0, n = 0;
  const int exps[] = {-30, -10, -1, 0, 1, 7};
  for (int k = 0; k < 6; ++k)
    for (uint32_t m = 0; m < (1u << 23); ++m) {
      uint32_t bits = ((uint32_t)(127 + exps[k]) << 23) | m;
      float a;
      memcpy(&a, &bits, 4);
      float q1 = a * r;
      float rem = fmaf(-q1, 6.0f, a);
      float q2 = fmaf(rem, r, q1);
      volatile float want = a / 6.0f;
      ++n;
      if (q2 != want) ++bad;
    }
  printf("%ld %ld\n", n, bad);
  return 0;
}
"""


def test_div6_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "div6.c")
        exe = os.path.join(td, "div6")
        open(c, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", c, "-o", exe, "-lm"], check=True)
        n, bad = map(int, subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split())
    assert n == 6 * (1 << 23) and bad == 0
