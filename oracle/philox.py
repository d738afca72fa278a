"""Philox4x32-10 counter-based generator and the uniform token draw.

The pages only say that initial tokens and re-noised tokens are drawn
uniformly from the whole vocabulary ([P3] "Masked Diffusion vs Uniform State
Diffusion"; [P4] "How Uniform State Diffusion works", where a noised position
takes x ~ Uniform(V)). The generator is Philox4x32 with 10 rounds from its
published definition (Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11): each round multiplies words 0 and 2 of
the counter by two fixed odd constants, keeps the 64-bit products' high and
low halves, and xors the high halves with the other two words and the
round key; the key is bumped by two Weyl constants between rounds.

Reading taken (the oracle and the device code implement it separately):
key = (seed low 32 bits, seed high 32 bits);
counter = (position, step, block, purpose) with purpose 0 = canvas init and
1 = re-noise; the draw uses output word 0;
token(r) = floor(r * V / 2**32), which for a power-of-two V is r >> (32 - log2 V)
and therefore exactly uniform.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

PURPOSE_INIT = 0
PURPOSE_RENOISE = 1
PURPOSE_GUMBEL = 2  # categorical sampling: purpose word 2 + 4 * (token // 4), output word token % 4


def philox4x32_10(ctr, key):
    """Ten Philox rounds on counters ``ctr`` (4 arrays or ints) with key (k0, k1).

    Works elementwise on NumPy arrays (uint64 holding 32-bit words) or ints.
    Returns the four output words as uint64 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & np.uint64(MASK32) for c in ctr)
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    lo_mask = np.uint64(MASK32)
    s32 = np.uint64(32)
    for rnd in range(10):
        if rnd:
            k0 = np.uint64((int(k0) + W0) & MASK32)
            k1 = np.uint64((int(k1) + W1) & MASK32)
        p0 = m0 * c0  # < 2**64, exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> s32, p0 & lo_mask
        hi1, lo1 = p1 >> s32, p1 & lo_mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def seed_key(seed: int):
    seed &= (1 << 64) - 1
    return seed & MASK32, seed >> 32


def token_from_word(r, vocab: int):
    """Map a 32-bit word to a token id in [0, vocab): floor(r * vocab / 2**32)."""
    r = np.asarray(r, dtype=np.uint64)
    return ((r * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


def draw_tokens(seed: int, positions, step: int, block: int, purpose: int, vocab: int):
    """Uniform token ids for ``positions`` keyed on (seed; pos, step, block, purpose)."""
    pos = np.asarray(positions, dtype=np.uint64)
    z = np.zeros_like(pos)
    w0, _, _, _ = philox4x32_10((pos, z + np.uint64(step), z + np.uint64(block), z + np.uint64(purpose)),
                                seed_key(seed))
    return token_from_word(w0, vocab)


def init_canvas(seed: int, canvas: int, block: int, vocab: int):
    """Canvas initialisation: every position a uniform random token.

    [P3] "Inference mechanism" (the entropy-bounded sampler starts from
    uniformly random tokens); [P4] "Reverse diffusion process", step 1.
    """
    return draw_tokens(seed, np.arange(canvas), 0, block, PURPOSE_INIT, vocab)


def uniform24(seed: int, positions, step: int, block: int, vocab: int):
    """[len(positions), vocab] uniforms in (0, 1) for categorical sampling: token v of position i
    takes output word v % 4 of the counter (i, step, block, 2 + 4 (v // 4)), keeps its top 24 bits
    r and maps them to (r + 1/2) / 2**24 (exactly representable in float32 and float64)."""
    pos = np.asarray(positions, dtype=np.uint64)
    ng = (vocab + 3) // 4
    P = np.repeat(pos[:, None], ng, axis=1)
    G = np.repeat(np.arange(ng, dtype=np.uint64)[None, :], pos.size, axis=0)
    z = np.zeros_like(P)
    words = philox4x32_10((P, z + np.uint64(step), z + np.uint64(block), np.uint64(PURPOSE_GUMBEL) + np.uint64(4) * G),
                          seed_key(seed))
    w = np.stack(words, axis=-1).reshape(pos.size, ng * 4)[:, :vocab]
    return ((w >> np.uint64(8)).astype(np.float64) + 0.5) / float(1 << 24)
