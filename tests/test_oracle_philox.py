"""Pins of the oracle's Philox4x32-10 and token draw.

Pin 1: rocRAND's Philox4x32-10 engine (the installed ROCm header, compiled for
the host CPU) on 10^5 counters, including the counter layout used for canvas
tokens and weights.  Pin 2: chi-square uniformity of token ids.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle import philox

ROCRAND_PROG = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>
#include <vector>
int main(int argc, char** argv) {
  unsigned long long seed = strtoull(argv[1], 0, 0);
  FILE* f = fopen(argv[2], "rb"); FILE* g = fopen(argv[3], "wb");
  uint32_t c[4];
  while (fread(c, 4, 4, f) == 4) {
    unsigned long long offset = ((((unsigned long long)c[1]) << 32) | c[0]) * 4ull;
    unsigned long long subseq = (((unsigned long long)c[3]) << 32) | c[2];
    rocrand_device::philox4x32_10_engine e(seed, subseq, offset);
    uint32_t r[4] = {e.next(), e.next(), e.next(), e.next()};
    fwrite(r, 4, 4, g);
  }
  fclose(f); fclose(g); return 0;
}
"""


def _rocrand_available():
    return os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h") and shutil.which("g++")


@pytest.mark.skipif(not _rocrand_available(), reason="ROCm rocRAND headers or g++ missing")
def test_philox_matches_rocrand_engine():
    rng = np.random.default_rng(11)
    n = 100_000
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    # the engine takes the low 64 counter bits as a count of 32-bit outputs
    # (4 per counter), so c1 must stay below 2^30 for the mapping to be exact
    ctr[:, 1] >>= 2
    # the layouts actually used: (pos, step, block, req|tag<<24) and weights
    ctr[:1000, 0] = np.arange(1000) % 256
    ctr[:1000, 1] = np.arange(1000) // 256
    ctr[:1000, 2] = 3
    ctr[:1000, 3] = 5
    ctr[1000:2000, 0] = np.arange(1000)
    ctr[1000:2000, 1] = 0
    ctr[1000:2000, 2] = 17
    ctr[1000:2000, 3] = 1 << 24
    ctr[2000] = [0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF]
    ctr[2001] = [0, 0, 0, 0]
    seeds = [0, 1, 0xDEADBEEFCAFEF00D]
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "p.cpp")
        exe = os.path.join(td, "p")
        open(src, "w").write(ROCRAND_PROG)
        subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", src, "-o", exe], check=True)
        fin = os.path.join(td, "in.bin")
        ctr.tofile(fin)
        for seed in seeds:
            fout = os.path.join(td, "out.bin")
            subprocess.run([exe, str(seed), fin, fout], check=True)
            ref = np.fromfile(fout, dtype=np.uint32).reshape(n, 4)
            k0, k1 = philox.seed_key(seed)
            got = np.stack(philox.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], k0, k1), axis=1)
            assert np.array_equal(got, ref), f"seed {seed}: {np.argwhere(got != ref)[:5]}"


def test_token_draw_uniform_chi_square():
    V = 4096
    ids = np.concatenate([philox.token_draw(1, np.arange(256), t, 0, 0, V) for t in range(200)])
    assert ids.min() >= 0 and ids.max() < V
    counts = np.bincount(ids, minlength=V)
    chi2 = ((counts - ids.size / V) ** 2 / (ids.size / V)).sum()
    p = stats.chi2.sf(chi2, V - 1)
    assert 1e-4 < p < 1 - 1e-4


def test_token_draw_is_top_bits_for_power_of_two_vocab():
    # floor(r0 * V / 2^32) with V = 2^18 is r0 >> 14: checks the scaling and
    # that the draw depends on every key and counter word.
    k0, k1 = philox.seed_key(9)
    r0 = philox.philox4x32_10(np.arange(256), 4, 2, 3, k0, k1)[0]
    ids = philox.token_draw(9, np.arange(256), 4, 2, 3, 262144)
    assert np.array_equal(ids, (r0 >> 14).astype(np.int64))
    base = philox.token_draw(9, np.arange(256), 4, 2, 3, 262144)
    for args in [(8, 4, 2, 3), (9, 5, 2, 3), (9, 4, 1, 3), (9, 4, 2, 4)]:
        s, st, b, r = args
        other = philox.token_draw(s, np.arange(256), st, b, r, 262144)
        assert (other != base).mean() > 0.99
