"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module holds no arithmetic of the denoising method. It only turns a
(seed, tensor id, element index) triple into a reproducible value, so that the
oracle and the HIP library can be fed identical bytes without either one
importing the other.

Generator (all integer / exactly rounded arithmetic, so a device twin can be
bit-identical):

* ``mix64`` is the SplitMix64 output finaliser (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014; constants as
  published by Vigna).
* ``hash64(seed, tid, i) = mix64(mix64(seed * G + tid) + (i + 1) * G)`` with
  ``G = 0x9E3779B97F4A7C15``, all modulo 2**64.
* "Normal" values use the Irwin-Hall sum of the four 16-bit fields of the
  hash: ``c = sum(fields) - 131070`` (an exact integer), scaled by one
  correctly rounded float32 multiply, ``value = f32(c) * f32(sigma / SD4)``
  with ``SD4 = sqrt((65536**2 - 1) / 3)``. The result has mean 0 and standard
  deviation ``sigma`` and is bounded by about 3.46 sigma.
* The background of the planted-peak logits uses twelve 16-bit fields, those of
  the hashes of indices 3 i, 3 i + 1 and 3 i + 2: ``c = sum - 393210``,
  ``value = f32(c) * f32(sigma / SD12)`` with ``SD12 = sqrt(65536**2 - 1)``.
  Its tails reach 6 sigma; the largest of 262144 draws is about 4.2 sigma
  (a normal's: 4.55 sigma; four fields': 3.3 sigma), which is what decides
  how often a planted peak is the row's argmax.
* bf16 values are the float32 value rounded to nearest-even on its upper 16
  bits.
* Uniform ids are ``((hash >> 32) * V) >> 32``.

The device twin lives in the HIP library (``dg_synth_*``); the GPU tests check
that both produce the same bits.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
SD4 = math.sqrt((65536.0 * 65536.0 - 1.0) / 3.0)
SD12 = math.sqrt(65536.0 * 65536.0 - 1.0)

# tensor-id namespaces (kept disjoint by the high bits)
TID_EMBED = 1
TID_SC_W1 = 2
TID_SC_W2 = 3
TID_PROMPT = 10
TID_X_INPUT = 11
TID_KV_INPUT = 12
TID_LOGITS = 20
TID_PEAK = 21
TID_LAYER_BASE = 1 << 20   # + layer * 64 + kind
TID_EXPERT_BASE = 1 << 32  # + (layer * 1024 + expert) * 8 + kind

# per-layer dense tensor kinds
K_WQ, K_WK, K_WV, K_WO, K_WR, K_SH_GATE, K_SH_UP, K_SH_DOWN = range(8)
# per-expert tensor kinds
E_GATE, E_UP, E_DOWN = range(3)


def layer_tid(layer: int, kind: int) -> int:
    return TID_LAYER_BASE + layer * 64 + kind


def expert_tid(layer: int, expert: int, kind: int) -> int:
    return TID_EXPERT_BASE + (layer * 1024 + expert) * 8 + kind


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tid: int) -> int:
    return mix64((seed * GOLDEN + tid) & MASK64)


def hash64(seed: int, tid: int, idx: np.ndarray) -> np.ndarray:
    """64-bit hash of element indices ``idx`` (any int array) in stream (seed, tid)."""
    key = np.uint64(stream_key(seed, tid))
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (i + np.uint64(1)) * np.uint64(GOLDEN)
    return _mix64_np(z)


def normal_scale(sigma: float) -> np.float32:
    return np.float32(sigma / SD4)


def _irwin_hall4(h: np.ndarray) -> np.ndarray:
    f = np.uint64(0xFFFF)
    s = (h & f) + ((h >> np.uint64(16)) & f) + ((h >> np.uint64(32)) & f) + (h >> np.uint64(48))
    return (s.astype(np.int64) - 131070).astype(np.float32)


def normal_f32(seed: int, tid: int, n_or_idx, sigma: float) -> np.ndarray:
    """float32 'normal' values (Irwin-Hall of four 16-bit uniforms)."""
    idx = np.arange(n_or_idx, dtype=np.uint64) if np.isscalar(n_or_idx) else n_or_idx
    c = _irwin_hall4(hash64(seed, tid, idx))
    return c * normal_scale(sigma)


def _fields_sum(h: np.ndarray) -> np.ndarray:
    f = np.uint64(0xFFFF)
    return (h & f) + ((h >> np.uint64(16)) & f) + ((h >> np.uint64(32)) & f) + (h >> np.uint64(48))


def normal12_f32(seed: int, tid: int, idx: np.ndarray, sigma: float) -> np.ndarray:
    """float32 'normal' values from twelve 16-bit uniforms (hashes of 3 i, 3 i + 1, 3 i + 2)."""
    i3 = np.asarray(idx, dtype=np.uint64) * np.uint64(3)
    s = (_fields_sum(hash64(seed, tid, i3)) + _fields_sum(hash64(seed, tid, i3 + np.uint64(1)))
         + _fields_sum(hash64(seed, tid, i3 + np.uint64(2))))
    c = (s.astype(np.int64) - 393210).astype(np.float32)
    return c * np.float32(sigma / SD12)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(seed: int, tid: int, n_or_idx, sigma: float) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, tid, n_or_idx, sigma))


def uniform_ids(seed: int, tid: int, n: int, vocab: int) -> np.ndarray:
    h = hash64(seed, tid, np.arange(n, dtype=np.uint64))
    with np.errstate(over="ignore"):
        return (((h >> np.uint64(32)) * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)


# ---------------------------------------------------------------------------
# Planted-peak logits: background "normal" sigma (twelve fields), and in a
# fraction of rows +peak added at one uniformly chosen column, then rounded to
# bf16.
# ---------------------------------------------------------------------------
PEAK_FRACTION_NUM = 3006477107  # floor(0.7 * 2**32)


def peak_rows(seed: int, step: int, rows: int, vocab: int):
    """(planted mask [rows] bool, column [rows] int64) for one logits buffer."""
    h = hash64(seed, TID_PEAK + (step << 8), np.arange(rows, dtype=np.uint64))
    planted = (h & np.uint64(0xFFFFFFFF)) < np.uint64(PEAK_FRACTION_NUM)
    with np.errstate(over="ignore"):
        col = ((h >> np.uint64(32)) * np.uint64(vocab)) >> np.uint64(32)
    return planted, col.astype(np.int64)


def planted_logits_rows(seed: int, step: int, rows: int, vocab: int, row_ids,
                        sigma: float = 3.0, peak: float = 12.0) -> np.ndarray:
    """bf16 bit patterns [len(row_ids), vocab] of the selected rows."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    planted, col = peak_rows(seed, step, rows, vocab)
    out = np.empty((len(row_ids), vocab), dtype=np.uint16)
    cols = np.arange(vocab, dtype=np.uint64)
    for j, r in enumerate(row_ids):
        v = normal12_f32(seed, TID_LOGITS + (step << 8), np.uint64(r) * np.uint64(vocab) + cols, sigma)
        if planted[r]:
            v[col[r]] = np.float32(v[col[r]] + np.float32(peak))
        out[j] = f32_to_bf16_bits(v)
    return out


# ---------------------------------------------------------------------------
# Model weights (random init, sigma 0.02), generated lazily per tensor.
# Layout of every matrix is [out_features, in_features].
# ---------------------------------------------------------------------------
class _Lazy(dict):
    """dict whose missing entries are produced by a factory and cached."""

    def __init__(self, factory, cache=True):
        super().__init__()
        self._factory = factory
        self._cache = cache

    def __missing__(self, key):
        v = self._factory(key)
        if self._cache:
            self[key] = v
        return v


class SyntheticWeights:
    """Oracle-facing view of the synthetic weights as float64 arrays.

    ``W["embed"]``, ``W["sc_w1"]``, ``W["sc_w2"]``, ``W["layers"][l][name]`` and
    ``W["layers"][l]["experts"][e][name]`` mirror the tensors the HIP library
    fills on the device for the same (seed, shape, dtype).
    shape keys: n_layers, d_model, n_q_heads, n_kv_heads, head_dim, n_experts,
    d_expert, d_shared, gated, vocab, d_selfcond.
    """

    def __init__(self, shape: dict, seed: int = 0, dtype: str = "bf16", sigma: float = 0.02,
                 cache_experts: bool = True):
        self.s = dict(shape)
        self.seed = seed
        self.dtype = dtype
        self.sigma = sigma
        self.cache_experts = cache_experts
        self._top = _Lazy(self._make_top)
        self._layers = _Lazy(self._make_layer)

    def values(self, tid: int, n: int) -> np.ndarray:
        if self.dtype == "bf16":
            v = bf16_bits_to_f32(normal_bf16_bits(self.seed, tid, n, self.sigma))
        else:
            v = normal_f32(self.seed, tid, n, self.sigma)
        return v.astype(np.float64)

    def mat(self, tid: int, rows: int, cols: int) -> np.ndarray:
        return self.values(tid, rows * cols).reshape(rows, cols)

    def _make_top(self, key):
        s = self.s
        if key == "embed":
            return self.mat(TID_EMBED, s["vocab"], s["d_model"])
        if key == "sc_w1":
            return self.mat(TID_SC_W1, s["d_selfcond"], s["d_model"])
        if key == "sc_w2":
            return self.mat(TID_SC_W2, s["d_model"], s["d_selfcond"])
        if key == "layers":
            return self._layers
        raise KeyError(key)

    def _make_layer(self, l):
        s = self.s
        d, hd = s["d_model"], s["head_dim"]
        shapes = {
            "wq": (K_WQ, s["n_q_heads"] * hd, d),
            "wk": (K_WK, s["n_kv_heads"] * hd, d),
            "wv": (K_WV, s["n_kv_heads"] * hd, d),
            "wo": (K_WO, d, s["n_q_heads"] * hd),
            "wr": (K_WR, s["n_experts"], d),
            "sh_gate": (K_SH_GATE, s["d_shared"], d),
            "sh_up": (K_SH_UP, s["d_shared"], d),
            "sh_down": (K_SH_DOWN, d, s["d_shared"]),
        }

        def make(name):
            if name == "experts":
                return _Lazy(lambda e: self._make_expert(l, e), cache=self.cache_experts)
            if name == "sh_gate" and not s["gated"]:
                raise KeyError(name)
            kind, r, c = shapes[name]
            return self.mat(layer_tid(l, kind), r, c)

        return _Lazy(make)

    def _make_expert(self, l, e):
        s = self.s
        d, f = s["d_model"], s["d_expert"]
        shapes = {"gate": (E_GATE, f, d), "up": (E_UP, f, d), "down": (E_DOWN, d, f)}

        def make(name):
            if name == "gate" and not s["gated"]:
                raise KeyError(name)
            kind, r, c = shapes[name]
            return self.mat(expert_tid(l, e, kind), r, c)

        return _Lazy(make)

    def __getitem__(self, key):
        return self._top[key]
