"""Pins for the oracle's Philox4x32-10 and its 53-bit uniforms.

The pages fix no generator; the reading is Philox4x32-10 (Salmon et al., SC'11). The oracle's numpy
implementation is pinned to an independent implementation: the open-source rocRAND engine header,
compiled host-only at test time (tests/golden/philox_kat.cpp).
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_kat(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc or the rocRAND header is not available")
    exe = str(tmp_path_factory.mktemp("kat") / "philox_kat")
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-O1", os.path.join(HERE, "golden", "philox_kat.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(rows):
        text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(x) for x in line.split()] for line in out.strip().splitlines()], dtype=np.uint64)

    return run


def test_philox_matches_rocrand(rocrand_kat):
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 2**32, size=(1500, 6), dtype=np.uint64)
    # structured counters used by the sampler: (m, h, b, tag) with small values, and extreme words
    extra = [[0, 0, 0, 0, 0, 0], [2**32 - 1] * 6, [5, 3, 1, 0, 1, 0], [0, 31, 7, 1, 12345, 0],
             [127, 27, 0, 2, 2**32 - 1, 1], [1023, 0, 3, 2 + 256 * 3, 42, 9]]
    rows = np.vstack([rows, np.array(extra, dtype=np.uint64)])
    want = rocrand_kat(rows)
    got = np.stack(philox.philox4x32_10(rows[:, 0], rows[:, 1], rows[:, 2], rows[:, 3], rows[:, 4], rows[:, 5]),
                   axis=1).astype(np.uint64)
    assert np.array_equal(got, want)


def test_seed_key_split():
    assert philox.seed_key(0x0123456789ABCDEF) == (0x89ABCDEF, 0x01234567)
    assert philox.seed_key(5) == (5, 0)


def test_u53_is_exact_top_bits():
    x0 = np.array([0, 0xFFFFFFFF, 0x80000000, 0x12345678], dtype=np.uint32)
    x1 = np.array([0, 0xFFFFFFFF, 0, 0x9ABCDEF0], dtype=np.uint32)
    u = philox.u53_from_words(x0, x1)
    assert u[0] == 0.0
    assert u[1] == 1.0 - 2.0**-53          # largest value, strictly below 1
    assert u[2] == 0.5
    w = (0x12345678 << 32) | 0x9ABCDEF0
    assert u[3] == (w >> 11) / 2.0**53


def test_u53_uniform_chi_square():
    u = philox.uniforms(3, np.arange(1 << 16), 5, 2, philox.TAG_POINT)
    assert u.min() >= 0.0 and u.max() < 1.0
    counts, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
    expected = u.size / 64
    chi2 = np.sum((counts - expected) ** 2 / expected)
    assert chi2 < 120.0  # 63 dof: the 99.99% quantile is about 117


def test_counter_words_are_independent_streams():
    m = np.arange(4096)
    base = philox.uniforms(11, m, 0, 0, 0)
    for other in (philox.uniforms(11, m, 1, 0, 0), philox.uniforms(11, m, 0, 1, 0), philox.uniforms(11, m, 0, 0, 1),
                  philox.uniforms(12, m, 0, 0, 0)):
        assert not np.any(base == other)
        assert abs(np.corrcoef(base, other)[0, 1]) < 0.06
