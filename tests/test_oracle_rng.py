"""Pins for the oracle's random numbers (Philox4x32-10, uniform map, Gumbel).

The pages are silent on the random number generator; the reading is
Philox4x32-10 (Salmon et al., SC'11) with counter (v>>2, k, r, stream).  The
oracle's implementation is pinned to rocRAND's published engine (a separate
implementation of the same definition), and the derived variates to the
closed-form laws of the uniform and Gumbel distributions.
"""
import ctypes
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp()
    so = os.path.join(d, "rocrand_ref.so")
    subprocess.check_call([hipcc, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-O2", "-fPIC", "-shared", "-o", so,
                           os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp")])
    L = ctypes.CDLL(so)
    P = ctypes.POINTER(ctypes.c_uint32)
    L.ref_philox4x32_10.argtypes = [ctypes.c_uint32, ctypes.c_uint32, P, P]

    def ref(k0, k1, ctr):
        c = np.ascontiguousarray(np.asarray(ctr, np.uint32))
        o = np.zeros(4, np.uint32)
        L.ref_philox4x32_10(k0, k1, c.ctypes.data_as(P), o.ctypes.data_as(P))
        return o
    yield ref
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand(oracle, rocrand_ref):
    rng = np.random.default_rng(123)
    for i in range(3000):
        k0, k1 = (int(x) for x in rng.integers(0, 2**32, 2, dtype=np.uint64))
        ctr = rng.integers(0, 2**32, 4, dtype=np.uint64)
        ctr[1] %= 2**30   # keeps rocRAND's 64-bit offset = 4*(c0 | c1<<32) from wrapping
        if i < 4:
            ctr[:] = [0, 0, 0, 0] if i == 0 else ctr
        np.testing.assert_array_equal(oracle.philox(k0, k1, ctr), rocrand_ref(k0, k1, ctr))


def test_word_counter_layout(oracle):
    """Element (stream, r, k, v) takes word v&3 of the block at counter (v>>2, k, r, stream)."""
    seed = 0x0123456789ABCDEF
    for (s, r, k, v) in [(0, 0, 1, 0), (0, 5, 3, 7), (1, 2, 4, 0), (2, 9, 16, 151935), (3, 511, 17, 262143)]:
        blk = oracle.philox(seed & 0xFFFFFFFF, seed >> 32, [v >> 2, k, r, s])
        assert oracle.word(seed, s, r, k, v) == blk[v & 3]
    w = oracle.words(seed, 0, 3, 2, 10, 6)
    assert list(w) == [oracle.word(seed, 0, 3, 2, v) for v in range(10, 16)]


def test_uniform_map_exact():
    """u = ((w>>9) + 1/2) 2^-23: endpoints 2^-24 and 1-2^-24, exact in binary32."""
    from oracle import oracle as O
    assert O.uniform(0) == 2.0 ** -24
    assert O.uniform(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert O.uniform(511) == O.uniform(0)           # low 9 bits ignored
    for w in [1 << 9, 12345 << 9, 0x80000000, 0xDEADBEEF]:
        u = O.uniform(w)
        assert float(np.float32(u)) == u            # representable in binary32
        assert u == ((w >> 9) + 0.5) / 2.0 ** 23


def test_uniform_moments(oracle):
    w = oracle.words(7, 1, 0, 0, 0, 200_000)
    u = np.array([oracle.uniform(int(x)) for x in w[:50_000]])
    assert abs(u.mean() - 0.5) < 4 * math.sqrt(1 / 12 / u.size)
    assert abs(u.var() - 1 / 12) < 0.002
    # uniformity of the full 32-bit words over 256 byte bins
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_gumbel_law(oracle):
    """Gumbel draws follow exp(-exp(-g)): KS test, mean Euler-gamma, variance pi^2/6."""
    w = oracle.words(99, 0, 4, 5, 0, 100_000)
    g = np.array([oracle.gumbel(int(x)) for x in w])
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-4
    assert abs(g.mean() - np.euler_gamma) < 4 * math.sqrt(math.pi ** 2 / 6 / g.size)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    # bounded support from the uniform grid
    assert oracle.gumbel(0xFFFFFFFF) == pytest.approx(-math.log(-math.log1p(-2.0 ** -24)), rel=1e-12)
    assert oracle.gumbel(0xFFFFFFFF) < 16.64 and oracle.gumbel(0) > -2.82


def test_streams_are_distinct(oracle):
    """Different (stream, r, k) give unrelated words (no repeats in a sample)."""
    seen = set()
    for s in range(4):
        for r in range(3):
            for k in range(1, 4):
                seen.update(int(x) for x in oracle.words(5, s, r, k, 0, 64))
    assert len(seen) > 0.999 * 4 * 3 * 3 * 64
