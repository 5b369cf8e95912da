"""The pack kernel's code-space coding (mkv_demote.hip), compiled for the host
and checked against the TQ3 code rule written out here: every E4M3 byte
(NaN codes aside, they are outside the input contract) against every
non-negative finite fp16 group scale at layer scale 1, a spread of other
layer scales with the kernel's approximate reciprocal off by up to one ulp,
and the assembly of codes into triple words for the K and V thread layouts.
The kernel's helper text is extracted from the source, so this checks the
code the GPU runs; the GPU intrinsics it uses are emulated from their
definitions (v_bitop3: truth-table bit (a b c), a the most significant;
v_perm_b32: selector 0-3 picks a byte of the second operand, 4-7 of the
first; the E4M3 decode), and the bit-exact GPU tests of the pack check that
the hardware agrees."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = os.path.join(HERE, "..", "mixed_format_paged_amd", "csrc", "mkv_demote.hip")


def _between(text, start, end):
    i = text.index(start)
    return text[i:text.index(end, i)]


PRELUDE = r"""
#include <cstdint>
#include <cstring>
#include <cmath>
#include <cstdio>
#include <random>
#include <vector>
static inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static float e4m3_value(uint32_t c) {            // E4M3FN, exact; 0x7f / 0xff are NaN
  c &= 0xff;
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  if ((c & 0x7f) == 0x7f) return NAN;
  const float v = e == 0 ? m * 0x1p-9f : ldexpf(1.0f + m / 8.0f, (int)e - 7);
  return (c & 0x80) ? -v : v;
}
struct F2 { float v[2]; float operator[](int i) const { return v[i]; } };
static inline F2 __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(uint32_t w, float, bool hi) {
  return {{e4m3_value(w >> (hi ? 16 : 0)), e4m3_value(w >> (hi ? 24 : 8))}};
}
static inline float __fmul_rn(float a, float b) { volatile float r = a * b; return r; }
static inline uint32_t __builtin_amdgcn_bitop3_b32(uint32_t a, uint32_t b, uint32_t c, uint32_t t) {
  uint32_t r = 0;
  for (int i = 0; i < 32; ++i) {
    const uint32_t idx = ((a >> i) & 1) << 2 | ((b >> i) & 1) << 1 | ((c >> i) & 1);
    r |= ((t >> idx) & 1) << i;
  }
  return r;
}
static inline uint32_t __builtin_amdgcn_perm(uint32_t a, uint32_t b, uint32_t sel) {
  const uint64_t d = ((uint64_t)a << 32) | b;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) r |= (uint32_t)((d >> (8 * ((sel >> (8 * i)) & 0xff))) & 0xff) << (8 * i);
  return r;
}
"""

MAIN = r"""
static float fp16_value(uint32_t h) {
  const uint32_t e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf(1.0f + m / 1024.0f, (int)e - 15);
}
// The TQ3 code u = q + 4 of x against scale s: q the integer nearest x / s,
// ties to even, clamped to [-3, 3]; as exact compares with s/2, 3s/2, 5s/2
// (s = 0: u = 4).
static uint32_t rule_code(float x, float s) {
  if (s == 0.0f) return 4;
  const float ax = fabsf(x);
  const int m = (ax > 0.5f * s) + (ax >= 1.5f * s) + (ax > 2.5f * s);
  return (uint32_t)(std::signbit(x) ? 4 - m : 4 + m);
}
static uint32_t code_of_byte(const Planes& p, int i) {
  return (uint32_t)!((p.n >> (8 * i + 7)) & 1) << 2 | ((p.u1 >> (8 * i + 7)) & 1) << 1 | ((p.u0 >> (8 * i + 7)) & 1);
}
static uint32_t rep(uint32_t k) { return k * 0x01010101u; }
int main() {
  long bad = 0, n = 0;
  // layer scale 1: every byte, every fp16 scale (a group of all-zero values has s = 0)
  for (uint32_t hb = 0; hb < 0x7c00; ++hb) {
    const float s = fp16_value(hb);
    const Keys k = group_keys<false>(thresholds(s), 1.0f, 1.0f);
    for (uint32_t b = 0; b < 256; ++b) {
      if ((b & 0x7f) == 0x7f || (hb == 0 && (b & 0x7f))) continue;
      const Planes p = code_planes(b * 0x01010101u, rep(k.k1), rep(k.k2), rep(k.k3));
      ++n;
      bad += code_of_byte(p, (int)(b % 4)) != rule_code(e4m3_value(b), s);
    }
  }
  // other layer scales, with the reciprocal off by -1, 0 and +1 ulp
  const float scales[] = {0.37f, 2.5f, 0.02f, 0.05f, 100.0f, 0.001f, 37.0f, 0x1p-20f, 1500.0f, 300.0f, 1e-30f, 1e30f};
  for (float scl : scales)
    for (int ulp = -1; ulp <= 1; ++ulp) {
      const float rscl = __uint_as_float(__float_as_uint(1.0f / scl) + ulp);
      for (uint32_t hb = 0; hb < 0x7c00; hb += 3) {
        const float s = fp16_value(hb);
        const Keys k = group_keys<true>(thresholds(s), scl, rscl);
        for (uint32_t b = 0; b < 256; ++b) {
          if ((b & 0x7f) == 0x7f || (hb == 0 && (b & 0x7f))) continue;
          const Planes p = code_planes(b * 0x01010101u, rep(k.k1), rep(k.k2), rep(k.k3));
          ++n;
          bad += code_of_byte(p, 0) != rule_code(__fmul_rn(e4m3_value(b), scl), s);
        }
      }
    }
  // triple words: K (two groups' dwords) and V (four tokens' dwords, regrouped)
  std::mt19937 rng(1);
  long bad_words = 0;
  for (int it = 0; it < 100000; ++it) {
    uint32_t x[4];
    float s[4];
    Keys k[4];
    for (int r = 0; r < 4; ++r) {
      x[r] = rng();
      for (int q = 0; q < 4; ++q)
        if (((x[r] >> (8 * q)) & 0x7f) == 0x7f) x[r] ^= 1u << (8 * q);
      s[r] = fp16_value(1 + rng() % 0x7bff);
      k[r] = group_keys<false>(thresholds(s[r]), 1.0f, 1.0f);
    }
    uint32_t ref = 0;
    for (int i = 0; i < 4; ++i)
      ref |= rule_code(e4m3_value(x[0] >> (8 * i)), s[0]) << (6 * i) | rule_code(e4m3_value(x[1] >> (8 * i)), s[1]) << (6 * i + 3);
    const uint32_t wk = compact_fields(pair_fields(code_planes(x[0], bytes4(k[0].k1), bytes4(k[0].k2), bytes4(k[0].k3)),
                                                   code_planes(x[1], bytes4(k[1].k1), bytes4(k[1].k2), bytes4(k[1].k3))));
    bad_words += wk != ref;
    uint32_t k1 = 0, k2 = 0, k3 = 0;
    for (int r = 0; r < 4; ++r) { k1 |= k[r].k1 << (8 * r); k2 |= k[r].k2 << (8 * r); k3 |= k[r].k3 << (8 * r); }
    const uint32_t e01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u), e23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
    const uint32_t f01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u), f23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
    const uint32_t w[2] = {
        compact_fields(pair_fields(code_planes(__builtin_amdgcn_perm(e23, e01, 0x05040100u), k1, k2, k3),
                                   code_planes(__builtin_amdgcn_perm(e23, e01, 0x07060302u), k1, k2, k3))),
        compact_fields(pair_fields(code_planes(__builtin_amdgcn_perm(f23, f01, 0x05040100u), k1, k2, k3),
                                   code_planes(__builtin_amdgcn_perm(f23, f01, 0x07060302u), k1, k2, k3)))};
    for (int h = 0; h < 2; ++h) {
      uint32_t rv = 0;
      for (int r = 0; r < 4; ++r)
        rv |= rule_code(e4m3_value(x[r] >> (16 * h)), s[r]) << (6 * r) | rule_code(e4m3_value(x[r] >> (16 * h + 8)), s[r]) << (6 * r + 3);
      bad_words += w[h] != rv;
    }
  }
  printf("%ld %ld %ld\n", n, bad, bad_words);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_pack_code_space_matches_the_code_rule():
    src = open(KERNEL).read()
    helpers = (_between(src, "struct Thresholds {", "// Largest |decode| of 16 FP8 bytes.")
               + _between(src, "// ---- codes from the FP8 bytes, four at a time", "// Workgroup of 128 threads"))
    code = PRELUDE + helpers.replace("__device__ inline", "static inline").replace("__device__ ", "static ") + MAIN
    with tempfile.TemporaryDirectory() as d:
        path, exe = os.path.join(d, "pack_codes.cpp"), os.path.join(d, "pack_codes")
        with open(path, "w") as f:
            f.write(code)
        subprocess.run(["g++", "-O2", "-std=c++17", "-fno-fast-math", "-ffp-contract=off", path, "-o", exe],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=300).stdout.split()
    n, bad, bad_words = map(int, out)
    assert n > 40_000_000
    assert bad == 0 and bad_words == 0, (bad, bad_words)
