"""Pins of the oracle's Philox4x32-10 (the counter-based generator behind the signs D and the dither).

Two independent references:
* the known-answer vectors published with the generator's definition (Salmon, Moraes, Dror, Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC'11, Random123 distribution), and
* rocRAND's Philox4x32-10 engine (``/opt/rocm/include/rocrand/rocrand_philox4x32_10.h``), compiled here
  for the host and driven to arbitrary counters through its subsequence/offset arguments.
"""
import os
import subprocess

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        v = [int(t, 16) for t in line.split()]
        rows.append((tuple(v[0:4]), tuple(v[4:6]), tuple(v[6:10])))
    return rows


KAT = _kat()


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(orc, ctr, key, want):
    assert tuple(int(v) for v in orc.philox4x32_10(ctr, key)) == want


PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // args: x y z w k0 k1 (hex); counter (x,y,z,w) reached through offset = 4 (x + y 2^32) and
  // subsequence = z + w 2^32 from a zero counter.
  unsigned long long v[6];
  for (int i = 0; i < 6; ++i) v[i] = strtoull(argv[1 + i], 0, 16);
  unsigned long long seed = v[4] | (v[5] << 32);
  unsigned long long offset = 4ull * (v[0] | (v[1] << 32));
  unsigned long long subseq = v[2] | (v[3] << 32);
  rocrand_device::philox4x32_10_engine e(seed, subseq, offset);
  uint4 r = e.next4();
  printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
}
"""


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    if not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers not installed")
    d = tmp_path_factory.mktemp("rocrand")
    src = d / "probe.cpp"
    src.write_text(PROBE)
    exe = d / "probe"
    subprocess.run(["hipcc", "-O1", "-o", str(exe), str(src)], check=True, capture_output=True)
    return str(exe)


def test_philox_matches_rocrand(orc, rocrand_probe):
    rng = np.random.default_rng(123)
    cases = [(0, 0, 0, 0, 0, 0), (1, 0, 0, 0, 7, 0), (3, 5, 0, 1, 0xDEADBEEF, 0x12345678)]
    # counters of the forms the codec uses: (0,0,0,0) for the signs, (octet, tile lo, tile hi, 1)
    # for the dither; plus random words.
    cases += [(o, t, 0, 1, s & 0xFFFFFFFF, s >> 32) for o, t, s in [(5, 1000, 0x0000000100000002), (15, 262143, 77)]]
    for _ in range(12):
        c = [int(v) for v in rng.integers(0, 2**32, size=6, dtype=np.uint64)]
        c[1] &= (1 << 29) - 1  # the probe reaches counter word 1 through a 64-bit offset 4 (x + y 2^32)
        cases.append(tuple(c))
    for c in cases:
        out = subprocess.run([rocrand_probe] + [f"{v:x}" for v in c], check=True, capture_output=True,
                             text=True).stdout.split()
        want = tuple(int(w, 16) for w in out)
        got = tuple(int(v) for v in orc.philox4x32_10(c[:4], c[4:]))
        assert got == want, c


def test_signs_are_philox_bits_and_balanced(orc):
    # D_i = -1 iff bit i of the 128-bit Philox output (counter 0, key = seed) is set.
    for seed in (0, 1, 2**40 + 3):
        d = orc.signs(seed)
        w = orc.philox4x32_10((0, 0, 0, 0), (seed & 0xFFFFFFFF, seed >> 32))
        bits = np.array([(int(w[i >> 5]) >> (i & 31)) & 1 for i in range(128)])
        assert np.array_equal(d, np.where(bits == 1, -1.0, 1.0).astype(np.float32))
    # over many seeds, each coordinate's sign is a fair coin
    neg = np.array([(orc.signs(s) < 0) for s in range(2000)], dtype=np.float64)
    m = neg.mean(axis=0)
    assert np.all(np.abs(m - 0.5) < 5 * 0.5 / np.sqrt(2000))
    assert abs(neg.mean() - 0.5) < 5 * 0.5 / np.sqrt(2000 * 128)


def test_dither_halfwords_uniform(orc):
    # the dither's 16-bit uniforms: moments of b = 2h/65536 over many octets
    seed = 99
    vals = np.array([orc.dither_octet(seed, t, o, orc.LAT_Z) for t in range(400) for o in range(16)])
    # for Z, U = b - rint(b) is uniform on [-1/2, 1/2]: mean 0, variance 1/12
    assert abs(vals.mean()) < 5 * np.sqrt(1 / 12 / vals.size)
    assert abs(vals.var() - 1 / 12) < 0.02 * (1 / 12)
    assert vals.min() >= -0.5 and vals.max() <= 0.5


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_round_count_is_a_prefix_of_the_pinned_rounds(orc, ctr, key, want):
    """Philox4x32-R with R = 7 (a dither format option) is the first 7 rounds of the function the
    known answers pin: running rounds 7..9 on its output gives the 10-round answer."""
    r7 = orc.philox4x32_span(ctr, key, 0, 7)
    assert tuple(int(v) for v in orc.philox4x32_span(r7, key, 7, 10)) == want
    assert tuple(int(v) for v in orc.philox4x32_span(ctr, key, 0, 10)) == want
    assert tuple(int(v) for v in r7) != want
