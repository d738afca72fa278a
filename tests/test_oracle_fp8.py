"""Pins of the oracle's FP8 E4M3 weight storage (OCP 8-bit floating point, E4M3 without infinities).

Pins that do not reuse the oracle's own arithmetic: code values fixed by the
format's definition (bias 7, subnormals m * 2^-9, S.1111.111 = NaN, largest
finite 448); torch's float8_e4m3fn conversions as an independent library
routine (decode of all 256 codes, and rounding of in-range values, which it
does to nearest-even); a brute-force nearest-code search over the 253 finite
values; the rounding error bound of the format.
"""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import model as OM

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])


def test_format_anchor_codes():
    d = fp8.decode([0x00, 0x01, 0x07, 0x08, 0x38, 0x40, 0x7E, 0xB8, 0xFE])
    assert list(d) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 2.0, 448.0, -1.0, -448.0]
    assert np.isnan(fp8.decode([0x7F, 0xFF])).all()
    assert np.signbit(fp8.decode([0x80]))[0]


def test_decode_matches_torch_on_every_code():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    d = fp8.decode(np.arange(256))
    assert np.array_equal(np.isnan(t), np.isnan(d))
    assert np.array_equal(t[~np.isnan(t)], d[~np.isnan(d)])


def test_round_trip_of_every_finite_code():
    assert np.array_equal(fp8.encode(fp8.decode(FINITE).astype(np.float32)), FINITE.astype(np.uint8))


def test_ties_go_to_even_mantissa():
    x = [1.0625, 1.1875, 0.5 * 2 ** -9, 1.5 * 2 ** -9, 2.5 * 2 ** -9, 7.5 * 2 ** -9]
    got = [int(c) for c in fp8.encode(x)]
    assert got == [0x38, 0x3A, 0x00, 0x02, 0x02, 0x08]


def test_saturates_beyond_the_largest_finite_value():
    big = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e6, 3e38], dtype=np.float32)
    assert (fp8.encode(big) == 0x7E).all()
    assert (fp8.encode(-big) == 0xFE).all()


def _brute_force(x):
    vals = fp8.decode(FINITE)
    out = []
    for v in np.asarray(x, dtype=np.float32).astype(np.float64):
        if abs(v) >= 448.0:
            out.append(0xFE if v < 0 else 0x7E)
            continue
        err = np.abs(vals - v)
        best = np.flatnonzero(err == err.min())
        codes = FINITE[best]
        codes = codes[(codes & 0x80) == (0x80 if np.signbit(v) else 0)] if len(codes) > 1 else codes
        even = [c for c in codes if c % 2 == 0]
        out.append(int(even[0] if even else codes[0]))
    return np.array(out, dtype=np.uint8)


def test_encode_is_the_nearest_code_with_ties_to_even():
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-12, np.log2(460.0), 4000))
    x = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    mids = (fp8.decode(FINITE[:-1]) + fp8.decode(FINITE[1:])) / 2  # exact midpoints of neighbours
    mids = mids[np.isfinite(mids) & (np.abs(mids) < 448)].astype(np.float32)
    x = np.concatenate([x, mids])
    assert np.array_equal(fp8.encode(x), _brute_force(x))


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * rng.choice([1e-3, 0.1, 10.0, 100.0], 200000)).astype(np.float32)
    x = x[np.abs(x) < 448.0]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(x), t)


def test_row_quantization_error_bound_and_extremes():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    w[3] = 0.0
    codes, s = fp8.quantize_rows(w)
    assert s.dtype == np.float32 and s[3] == 1.0 and (codes[3] == 0).all()
    # the largest magnitude of each non-zero row lands on +-448
    r = np.arange(64) != 3
    amax = np.argmax(np.abs(w), axis=1)
    assert (codes[r, amax[r]] & 0x7F == 0x7E).all()
    deq = fp8.dequantize(codes, s)
    # half a unit in the last place: 2^-4 relative above 2^-6 * s, 2^-10 * s absolute below
    bound = np.maximum(np.abs(w) * 2.0 ** -4, s[:, None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - w) <= bound).all()
    # 3 fraction bits: the mean error is about a quarter unit, 2^-5 of the magnitude
    assert np.abs(deq - w).mean() < 0.04 * np.abs(w).mean()


def test_fp8_view_only_touches_routed_experts():
    rng = np.random.default_rng(1)
    lw = {"wq": rng.standard_normal((4, 4)), "sh_up": rng.standard_normal((3, 4)),
          "experts": [{n: rng.standard_normal(sh).astype(np.float32).astype(np.float64)
                       for n, sh in (("gate", (6, 4)), ("up", (6, 4)), ("down", (4, 6)))} for _ in range(2)]}
    W = {"embed": rng.standard_normal((10, 4)), "layers": [lw]}
    V = fp8.Fp8Weights(W)
    assert V["embed"] is W["embed"] and V["layers"][0]["wq"] is lw["wq"]
    for n in ("gate", "up", "down"):
        q = V["layers"][0]["experts"][1][n]
        src = lw["experts"][1][n]
        assert q.shape == src.shape and not np.array_equal(q, src)
        assert np.allclose(q, src, rtol=2 ** -4, atol=np.abs(src).max() * 2 ** -12)
    h = rng.standard_normal((5, 4))
    a = OM.ffn(h, V["layers"][0]["experts"][0], True)
    b = OM.ffn(h, lw["experts"][0], True)
    assert np.allclose(a, b, rtol=0.3, atol=0.1 * np.abs(b).max())
