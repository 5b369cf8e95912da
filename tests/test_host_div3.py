"""The pack kernels' division by 3 (the TQ3 scale rule s = fp16(fl32(a / 3))):
fl32(a / 3) as the product with fl32(1/3) corrected by two fmas.  Checked here
against IEEE fp32 division for every finite non-negative fp32 a (about 17 s of
C on one core), with the fmas of the host's libm, which are correctly rounded
like the GPU's."""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
  const float c = 0x1.555556p-2f;
  uint64_t bad = 0;
  for (uint64_t u = 0; u < 0x7f800000ull; ++u) {
    float a, q, q1, ref;
    uint32_t v = (uint32_t)u, b1, b2;
    memcpy(&a, &v, 4);
    q = a * c;
    q1 = fmaf(fmaf(-3.0f, q, a), c, q);
    ref = a / 3.0f;
    memcpy(&b1, &q1, 4);
    memcpy(&b2, &ref, 4);
    bad += b1 != b2;
  }
  printf("%llu\n", (unsigned long long)bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_div3_rn_equals_ieee_division_for_every_finite_float():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div3.c"), os.path.join(d, "div3")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=300).stdout
    assert int(out.strip()) == 0
