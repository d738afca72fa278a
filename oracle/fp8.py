"""FP8 E4M3 storage of the routed experts' weights (an opt-in mode of the library).

Source: [P2] "24GB GPU: practical adoption and running conditions" lists
quantised GGUF builds of the model (the 8-bit one at about half the bf16
footprint) and [P1] "Summary" points local runs at them; the pages fix no
format for this library. Reading taken: the OCP 8-bit floating-point E4M3
format ("OFP8", the variant with no infinities): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448. Values are rounded to nearest,
ties to an even mantissa, and magnitudes beyond the rounding range of 448
saturate to 448.

Each output row of an expert matrix (a gate / up feature, a down output) has
its own float32 scale s = max|w| / 448 (1 for an all-zero row); the stored
code is the E4M3 rounding of the float32 quotient w / s, and the weight the
model computes with is decode(code) * s. Test infrastructure: only tests/,
the package's smoke entry and the benchmark's CPU baseline use this module.
"""
from __future__ import annotations

import numpy as np

MAX_E4M3 = 448.0


def decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def encode(x) -> np.ndarray:
    """E4M3 codes of float32 values: round to nearest, ties to even, saturating at +-448."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    # subnormal range (below the smallest normal 2^-6): units of 2^-9; 8 units is the code 0x08
    sub = np.rint(a * 512.0).astype(np.int64)
    # normal range: a = f * 2^e with f in [1, 2); keep 3 fraction bits, a carry bumps the exponent
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex.astype(np.int64) - 1
    m = np.rint((np.ldexp(np.where(a > 0, a, 1.0), -e) - 1.0) * 8.0).astype(np.int64)
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    norm = np.clip((e + 7) * 8 + m, 0, 0x7E)
    mag = np.where(a < 2.0 ** -6, sub, norm)
    mag = np.where(a >= 464.0, 0x7E, mag)  # 464 is the midpoint to 480 (NaN's place): saturate
    return (sign | mag).astype(np.uint8)


def row_scales(w) -> np.ndarray:
    """float32 scale per row: max|w| / 448, or 1 for an all-zero row."""
    w = np.asarray(w, dtype=np.float32)
    mx = np.abs(w).max(axis=-1)
    return np.where(mx > 0, mx / np.float32(MAX_E4M3), np.float32(1.0)).astype(np.float32)


def quantize_rows(w):
    """(codes [R, K] uint8, scales [R] float32) of a matrix of float32 (bf16-valued) weights."""
    w = np.asarray(w, dtype=np.float32)
    s = row_scales(w)
    q = (w / s[:, None]).astype(np.float32)  # float32 division, as the device does
    return encode(q), s


def dequantize(codes, scales) -> np.ndarray:
    """The weights the FP8 mode computes with: decode(code) * scale, float64."""
    return decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def dequantize_matrix(w) -> np.ndarray:
    """float64 weights after the round trip: per-row scales, E4M3 codes, decode times scale."""
    codes, s = quantize_rows(w)
    return dequantize(codes, s)


class _Experts:
    def __init__(self, experts):
        self.src = experts
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            src = self.src[e]
            names = ("gate", "up", "down")
            out = {}
            for n in names:
                try:
                    out[n] = dequantize_matrix(src[n])
                except KeyError:
                    pass
            self.cache[e] = out
        return self.cache[e]


class _Layer:
    def __init__(self, lw):
        self.lw = lw
        self.experts = _Experts(lw["experts"])

    def __getitem__(self, key):
        return self.experts if key == "experts" else self.lw[key]


class _Layers:
    def __init__(self, layers):
        self.src = layers
        self.cache = {}

    def __getitem__(self, l):
        if l not in self.cache:
            self.cache[l] = _Layer(self.src[l])
        return self.cache[l]


class Fp8Weights:
    """View of a weight set whose routed experts (only) compute with FP8-stored weights.

    Gate and up matrices [F, D] have one scale per feature row, the down
    matrix [D, F] one per output row; every other tensor is passed through.
    """

    def __init__(self, W):
        self.W = W
        self.layers = _Layers(W["layers"])

    def __getitem__(self, key):
        return self.layers if key == "layers" else self.W[key]
