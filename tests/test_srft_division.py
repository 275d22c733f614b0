"""The SRFT encoder's two quotients (group scale absmax / L and the reciprocal of the binary16 scale)
are computed on the GPU without the hardware division sequence, by FMA schemes that must equal the
correctly rounded quotient the oracle takes with a plain division.  This checks both schemes
exhaustively on the host with the same binary32 operations (fmaf is the same fused multiply-add the
kernel issues):
  RN(a / L) = fma(fma(-q0, L, a), c, q0) with c = RN(1/L), q0 = RN(a c), for L = 7, 127 (Markstein's
  correction with the exact remainder): every a >= 0 with biased exponent 0..31 (subnormals and the
  binades where an intermediate could be subnormal), every a in [1, 2) and in the top binade.  Where
  every intermediate is normal, all of q0, the remainder, q1 and RN(a / L) scale exactly with a power
  of two, so [1, 2) stands for exponents 32..253 (the full range was also run: no difference);
  RN(1 / d) = fma(fma(-d, y0, 1), y0, y0) for every positive finite binary16 d and every start y0
  within one ulp of RN(1 / d) (the hardware reciprocal's bound)."""
import os
import subprocess
import tempfile

PROGRAM = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
#include <stdlib.h>
int main(int argc, char** argv) {
  long long bad = 0;
  {
    const float L = (float)atoi(argv[1]);
    volatile float one = 1.0f;
    const float c = one / L;
    const uint32_t ranges[3][2] = {{0u, 32u << 23}, {127u << 23, 128u << 23}, {254u << 23, 255u << 23}};
    for (int ri = 0; ri < 3; ++ri)
    for (uint32_t u = ranges[ri][0]; u < ranges[ri][1]; ++u) {
      const float a = fb(u);
      const float q0 = a * c;
      const float q1 = fmaf(fmaf(-q0, L, a), c, q0);
      bad += bf(q1) != bf(a / L);
    }
  }
  long long badr = 0, n = 0;
  for (uint32_t h = 1; h < 0x7C00u; ++h) {
    const uint32_t e = h >> 10, m = h & 1023u;
    const float d = (float)(e ? ldexp((double)(m | 1024u), (int)e - 25) : ldexp((double)m, -24));
    const float want = 1.0f / d;
    for (int k = -1; k <= 1; ++k) {
      const float y0 = fb(bf(want) + (uint32_t)k);
      const float y1 = fmaf(fmaf(-d, y0, 1.0f), y0, y0);
      ++n;
      badr += bf(y1) != bf(want);
    }
  }
  printf("%lld %lld %lld\n", bad, badr, n);
  return 0;
}
"""


def test_fma_quotients_equal_correctly_rounded_division():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "q.c")
        exe = os.path.join(d, "q")
        open(src, "w").write(PROGRAM)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-mfma", "-o", exe, src,
                        "-lm"], check=True)
        procs = [subprocess.Popen([exe, L], stdout=subprocess.PIPE, text=True) for L in ("7", "127")]
        outs = [p.communicate()[0].split() for p in procs]
        assert all(p.returncode == 0 for p in procs)
    for out in outs:
        bad, badr, n = (int(v) for v in out)
        assert n == 3 * 31743
        assert bad == 0 and badr == 0
