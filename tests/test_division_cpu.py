"""The smoothing division used by the device kernels, checked exhaustively on the CPU.

The kernels compute x / scale (the exercise page's smoothing, "Formula and conventions"
item 1) as q0 = RN(x * y) with y = RN(1 / scale), followed by two Newton-Markstein
corrections q <- fma(fma(-s, q, x), y, q), falling back to IEEE division when a
quotient, an input or the scale leaves [2^-90, 2^90]. That claim ("equals the correctly
rounded quotient") is tested here against the C library's IEEE float division for every
positive finite bfloat16 x and every smoothing scale of the five workloads, plus random
binary32 inputs. gcc's fmaf is correctly rounded, like the GPU's v_fma_f32.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

from workloads import WORKLOADS, make_inputs

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float div_rn(float x, float s, float y) {
  float q = x * y;
  float r = fmaf(-s, q, x);
  q = fmaf(r, y, q);
  r = fmaf(-s, q, x);
  q = fmaf(r, y, q);
  float aq = fabsf(q), ax = fabsf(x);
  if (!(aq >= 0x1p-90f && aq <= 0x1p90f && ax >= 0x1p-90f)) q = x / s;
  return q;
}
static float recip(float s) { return (s >= 0x1p-90f && s <= 0x1p90f) ? 1.0f / s : 0.0f; }
static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)st; }
int main(int argc, char** argv) {
  FILE* f = fopen(argv[1], "rb");
  fseek(f, 0, SEEK_END); long n = ftell(f) / 4; fseek(f, 0, SEEK_SET);
  float* sc = malloc(n * 4); if (fread(sc, 4, n, f) != (size_t)n) return 2; fclose(f);
  long bad = 0, total = 0;
  for (long i = 0; i < n; i++) {           /* every positive finite bf16 x, both signs */
    float s = sc[i], y = recip(s);
    for (uint32_t h = 1; h < 0x7F80; h++) {
      uint32_t u = h << 16; float x; memcpy(&x, &u, 4);
      float a = div_rn(x, s, y), b = x / s, c = div_rn(-x, s, y), d = -x / s;
      if (memcmp(&a, &b, 4) || memcmp(&c, &d, 4)) { if (bad < 5) printf("bad x=%a s=%a got %a want %a\n", x, s, a, b); bad++; }
      total += 2;
    }
  }
  for (long i = 0; i < 20000000; i++) {   /* random binary32 x and scales */
    uint32_t ux = rnd() & 0xFFFFFFFFu, us = (rnd() & 0x007FFFFFu) | ((100u + rnd() % 55u) << 23);
    float x, s; memcpy(&x, &ux, 4); memcpy(&s, &us, 4);
    if (!isfinite(x)) continue;
    float y = recip(s), a = div_rn(x, s, y), b = x / s;
    if (memcmp(&a, &b, 4)) { if (bad < 5) printf("bad x=%a s=%a got %a want %a\n", x, s, a, b); bad++; }
    total++;
  }
  printf("%ld %ld\n", bad, total);
  return 0;
}
"""


def test_fast_division_matches_ieee_division():
    scales = [make_inputs(cid, B=min(WORKLOADS[cid].B, 256))[2] for cid in WORKLOADS]
    rng = np.random.default_rng(0)
    extra = np.ldexp(rng.random(2000) + 0.5, rng.integers(-95, 96, 2000)).astype(np.float32)
    edge = np.array([2.0**-90, 2.0**90, float.fromhex("0x1.fffffep-91"), 1.0, 3.0, 0.1, 1e-30, 1e30], np.float32)
    allsc = np.unique(np.concatenate(scales + [extra, edge]).astype(np.float32))
    with tempfile.TemporaryDirectory() as d:
        src, exe, dat = os.path.join(d, "t.c"), os.path.join(d, "t"), os.path.join(d, "s.bin")
        open(src, "w").write(C_SRC)
        allsc.tofile(dat)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe, dat], capture_output=True, text=True, check=True, timeout=600).stdout
    bad, total = map(int, out.strip().splitlines()[-1].split())
    assert total > 5e8
    assert bad == 0, out
