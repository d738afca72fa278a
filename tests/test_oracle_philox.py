"""Pins of the oracle's Philox4x32-10 and token draw.

* Independent implementation: rocRAND's Philox4x32-10 (installed ROCm
  library, host code) must agree bit for bit on random counters and keys.
* token(r) = floor(r V / 2^32) is exactly r >> (32 - log2 V) for power-of-two V
  and is uniform (chi-square).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp(prefix="philox_ref_")
    exe = os.path.join(d, "ref")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "philox_rocrand_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def run_ref(exe, rows):
    inp = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()], dtype=np.uint64)


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(123)
    rows = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 2, 3, 4, 5, 6)]
    for _ in range(300):
        c = rng.integers(0, 2**32, size=4, dtype=np.uint64)
        c[1] &= np.uint64(0x3FFFFFFF)
        k = rng.integers(0, 2**32, size=2, dtype=np.uint64)
        rows.append((*c, *k))
    # the counter layout the method uses: (pos, step, block, purpose)
    for pos in (0, 1, 255):
        for step in (0, 47):
            rows.append((pos, step, 3, 1, 0, 0))
            rows.append((pos, step, 0, 0, 7, 0))
    ref = run_ref(rocrand_ref, rows)
    for r, want in zip(rows, ref):
        got = philox.philox4x32_10(tuple(np.uint64(v) for v in r[:4]), (r[4], r[5]))
        assert [int(g) for g in got] == [int(w) for w in want], r


def test_token_is_top_bits_for_power_of_two_vocab():
    rng = np.random.default_rng(1)
    r = rng.integers(0, 2**32, size=100000, dtype=np.uint64)
    for logv in (12, 18):
        assert np.array_equal(philox.token_from_word(r, 1 << logv), (r >> np.uint64(32 - logv)).astype(np.int64))


def test_token_range_non_power_of_two():
    r = np.array([0, 1, 2**31, 2**32 - 1], dtype=np.uint64)
    t = philox.token_from_word(r, 1000)
    assert t.min() >= 0 and t.max() <= 999 and t[-1] == 999 and t[0] == 0


@pytest.mark.parametrize("vocab", [4096, 262144])
def test_draws_are_uniform(vocab):
    pos = np.arange(1 << 18)
    t = philox.draw_tokens(7, pos, 3, 1, philox.PURPOSE_RENOISE, vocab)
    bins = 256
    counts = np.bincount(t * bins // vocab, minlength=bins)
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4, p


def test_purposes_steps_blocks_are_distinct_streams():
    pos = np.arange(256)
    a = philox.draw_tokens(0, pos, 0, 0, philox.PURPOSE_INIT, 262144)
    b = philox.draw_tokens(0, pos, 0, 0, philox.PURPOSE_RENOISE, 262144)
    c = philox.draw_tokens(0, pos, 1, 0, philox.PURPOSE_RENOISE, 262144)
    d = philox.draw_tokens(0, pos, 0, 1, philox.PURPOSE_RENOISE, 262144)
    e = philox.draw_tokens(1, pos, 0, 0, philox.PURPOSE_RENOISE, 262144)
    for x, y in [(a, b), (b, c), (b, d), (b, e)]:
        assert (x != y).mean() > 0.99
    assert np.array_equal(philox.init_canvas(0, 256, 0, 262144), a)
