"""The seeded input generator: reproducible, moments as documented, bf16 rounding."""
import math

import numpy as np

import synthetic as S


def test_mix64_matches_scalar_and_vector():
    idx = np.arange(100, dtype=np.uint64)
    h = S.hash64(5, 9, idx)
    key = S.stream_key(5, 9)
    for i in (0, 1, 99):
        assert int(h[i]) == S.mix64(key + (i + 1) * S.GOLDEN)


def test_normal_moments_and_bounds():
    v = S.normal_f32(0, 1, 1 << 20, 2.0)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 2.0) < 0.01
    assert np.abs(v).max() <= 2.0 * 131070 / S.SD4 + 1e-5


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 3.0e-3], dtype=np.float32)
    b = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
    assert b[0] == 1.0 and b[1] == 1.0  # halfway -> even
    assert b[2] == np.float32(1.0 + 2**-7)
    assert b[3] == -2.5
    assert abs(b[4] - 3.0e-3) / 3.0e-3 < 2**-8


def test_planted_logits():
    planted, col = S.peak_rows(0, 0, 4096, 262144)
    assert abs(planted.mean() - 0.7) < 0.03
    rows = S.planted_logits_rows(0, 0, 16, 1024, [0, 1, 2])
    assert rows.shape == (3, 1024)
    again = S.planted_logits_rows(0, 0, 16, 1024, [2])
    assert np.array_equal(rows[2], again[0])


def test_twelve_field_background():
    """The planted logits' background: mean 0, standard deviation sigma, tails past the four-field
    bound (3.46 sigma), and values equal to the sum of the twelve 16-bit fields of the hashes of
    3 i, 3 i + 1, 3 i + 2 recomputed here with Python integers."""
    v = S.normal12_f32(5, 77, np.arange(262144, dtype=np.uint64), 3.0).astype(np.float64)
    assert abs(v.mean()) < 0.03 and abs(v.std() - 3.0) < 0.03
    assert 3.8 * 3.0 < np.abs(v).max() < 6.0 * 3.0
    for i in (0, 1, 12345):
        s = 0
        for q in range(3):
            h = int(S.hash64(5, 77, np.array([3 * i + q], dtype=np.uint64))[0])
            s += sum((h >> (16 * f)) & 0xFFFF for f in range(4))
        want = np.float32(s - 393210) * np.float32(3.0 / math.sqrt(65536.0 * 65536.0 - 1.0))
        assert v[i] == np.float64(want)
