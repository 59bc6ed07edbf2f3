"""Pins for the oracle's Philox4x32-10 and uniform mapping (CPU only).

* Published known-answer vectors (tests/golden/philox4x32_10_kat.txt).
* rocRAND's Philox4x32-10 engine, built here as a host program from its
  MIT-licensed header, run as an independent implementation of the same
  stream convention (key = seed, counter words 2-3 = subsequence, word index t
  = block t // 4, lane t % 4).
* Statistical sanity of 2**20 words and the exhaustive uniform mapping.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([int(t, 16) for t in line.split()])
    return rows


def test_known_answers():
    rows = _kat_rows()
    assert len(rows) == 3
    for r in rows:
        assert philox.philox4x32_10(r[0:4], r[4:6]) == tuple(r[6:10])


def test_vectorised_words_match_scalar_block():
    for seed, sub, start, count in [(0, 0, 0, 9), (2**64 - 1, 2**64 - 1, 2**33 - 3, 7),
                                    (123456789, 5, 1, 13), (3 << 32, 4096, 0, 6)]:
        got = philox.words(seed, sub, count, start=start)
        want = [philox.word(seed, sub, t) for t in range(start, start + count)]
        assert [int(v) for v in got] == want


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc or rocRAND header not available")
    exe = str(tmp_path_factory.mktemp("rocrand") / "philox_rocrand_ref")
    src = os.path.join(HERE, "philox_rocrand_ref.cpp")
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o", exe],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("could not build the rocRAND comparator: " + r.stderr[-400:])
    return exe


@pytest.mark.parametrize("seed,sub,off,count", [
    (0, 0, 0, 64),
    (1, 0, 0, 17),
    (3 << 32, 0, 0, 6),
    (12345678901234567, 4096, 0, 40),
    (2**64 - 1, 2**64 - 1, 0, 12),
    (42, 2**40 + 32 * 7, 3, 25),
    (7, 11, (1 << 34) - 5, 20),          # block index crosses 2**32
])
def test_matches_rocrand(rocrand_ref, seed, sub, off, count):
    out = subprocess.run([rocrand_ref, str(seed), str(sub), str(off), str(count)],
                         capture_output=True, text=True, check=True).stdout.split()
    want = [int(v) for v in out]
    got = [int(v) for v in philox.words(seed, sub, count, start=off)]
    assert got == want


def test_word_statistics():
    w = philox.words(20240601, 9, 1 << 20)
    # byte histogram chi-square, 255 dof: mean 255, sd ~22.6
    bytes_ = w.view(np.uint8)
    hist = np.bincount(bytes_, minlength=256).astype(np.float64)
    exp = bytes_.size / 256.0
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert 150 < chi2 < 380, chi2
    # serial correlation of consecutive words (as uniforms)
    u = philox.uniform(w)
    c = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(c) < 5e-3
    # distinct subsequences are not shifted copies of each other
    w2 = philox.words(20240601, 10, 1 << 12)
    assert not np.array_equal(w[: 1 << 12], w2)
    assert abs(np.mean(u) - 0.5) < 2e-3


def test_uniform_mapping_exhaustive():
    codes = np.arange(1 << 23, dtype=np.uint64)
    w = codes << np.uint64(9)
    u = philox.uniform(w)
    assert u[0] == 2.0 ** -24 and u[-1] == 1.0 - 2.0 ** -24
    assert np.all(np.diff(u) > 0)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)   # exact in float32
    # low 9 bits are ignored
    assert np.array_equal(philox.uniform(w | np.uint64(0x1FF)), u)
    # u * q < q for every positive float32 q (so q == p always accepts)
    q = np.abs(np.random.default_rng(0).standard_normal(4096)).astype(np.float32).astype(np.float64) + 1e-30
    assert np.all(u[-1] * q < q)
    assert np.array_equal(philox.uniform_code(w).astype(np.float64) * 2.0 ** -24, u)
