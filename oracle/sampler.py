"""Logits scheduler, entropy-bounded sampler and the two-fold adaptive stop.

Sources:
* [P4] "Standard sampling settings" (table): at most 48 denoising steps,
  temperature decaying linearly from 0.8 to 0.4, entropy bound 0.1, adaptive
  stopping threshold 0.005 on the canvas mean entropy.
* [P4] "Two-Fold Adaptive Stopping": stop only when both conditions hold at
  once: (1) the canvas mean entropy is below the threshold, (2) the prediction
  matched the previous one two consecutive times (t-2 == t-1 == t).
* [P3] "Inference mechanism": the logits scheduler sharpens with temperature
  (explore early, converge late); the entropy-bounded sampler accepts tokens
  by an entropy-based confidence and re-noises the rest with random tokens.
* [P4] "Reverse diffusion process": keep confident tokens, re-noise the
  others, re-evaluate the whole canvas every step (nothing is frozen).

Readings taken where the pages are silent (also listed with the project's design notes):
* temperature index runs over the step budget: T(s) = t0 + (t1 - t0) s/(S-1),
  evaluated in double and rounded once to float32 (T(0)=t0, T(S-1)=t1);
* entropy in nats of the tempered distribution softmax(l / T);
* the accepted token is the argmax (lowest index on ties), per position,
  accept iff H <= bound (inclusive);
* "predictions" compared by the stop rule are the argmax vector;
* the stable counter counts consecutive equal argmax vectors; it is reset at
  step 0 and whenever a vector changes; two equalities are needed.

Variants the pages also describe, each behind a Schedule flag (defaults off):
* stop_either: [P3] "Inference mechanism" lets either condition stop the
  canvas (stability for N steps, or the entropy threshold) where [P4] needs
  both;
* accept_cumulative: [P3] "Inference mechanism" accepts token groups by an
  entropy-based confidence. Reading taken: positions are taken in increasing
  entropy (lower position first on ties) and the group accepted is the
  longest such run whose summed entropy stays within the bound (it may be
  empty); the rest are re-noised.
* categorical: [P4] "Standard sampling settings" explains the temperature
  schedule as exploring early and settling late, i.e. sampling from the
  tempered distribution. Reading taken: an accepted position keeps a token
  drawn from softmax(l / T) (Gumbel-max: argmax_v l_v / T - ln(-ln u_v), u
  from Philox, philox.uniform24) instead of the argmax; the predictions the
  stop rule compares, and the committed block, stay the argmax.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox


@dataclass
class Schedule:
    """Sampler settings; defaults are the pages' recommended values."""
    max_steps: int = 48
    t_start: float = 0.8
    t_end: float = 0.4
    entropy_bound: float = 0.1
    stop_mean_entropy: float = 0.005
    stable_needed: int = 2
    seed: int = 0
    stop_either: bool = False
    accept_cumulative: bool = False
    categorical: bool = False


def temperature(step: int, sched: Schedule) -> float:
    """Linear temperature decay over the step budget, as a float32 value."""
    t0 = float(np.float32(sched.t_start))
    t1 = float(np.float32(sched.t_end))
    if sched.max_steps <= 1:
        return float(np.float32(t0))
    return float(np.float32(t0 + (t1 - t0) * (step / (sched.max_steps - 1))))


def tempered_probs(logits: np.ndarray, T: float) -> np.ndarray:
    """softmax(l / T) per row, float64."""
    z = np.asarray(logits, dtype=np.float64) / np.float64(T)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def entropy_nats(p: np.ndarray) -> np.ndarray:
    """H = -sum p ln p per row, with 0 ln 0 = 0."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0.0, p * np.log(np.where(p > 0.0, p, 1.0)), 0.0)
    return -t.sum(axis=-1)


def cumulative_accept(H: np.ndarray, bound: float) -> np.ndarray:
    """Group acceptance: walk the positions in increasing entropy (ties: lower position first),
    adding each entropy to a running total; every position visited while the total is still
    <= bound is accepted, and the walk ends at the first one that takes it past the bound."""
    H = np.asarray(H, dtype=np.float64)
    order = sorted(range(H.size), key=lambda i: (H[i], i))
    accept = np.zeros(H.size, dtype=bool)
    total = 0.0
    for i in order:
        total += H[i]
        if total > bound:
            break
        accept[i] = True
    return accept


def gumbel_sample(logits: np.ndarray, T: float, seed: int, step: int, block: int) -> np.ndarray:
    """One token per row drawn from softmax(l / T) by the Gumbel-max rule: the index of the largest
    l_v / T + g_v, g_v = -ln(-ln u_v), u_v from philox.uniform24 (lowest index on ties)."""
    logits = np.asarray(logits, dtype=np.float64)
    C, V = logits.shape
    u = philox.uniform24(seed, np.arange(C), step, block, V)
    g = -np.log(-np.log(u))
    return np.argmax(logits / np.float64(T) + g, axis=-1).astype(np.int64)


@dataclass
class StepResult:
    entropy: np.ndarray      # [C] float64
    pred: np.ndarray         # [C] int64, argmax
    accept: np.ndarray       # [C] bool
    next_canvas: np.ndarray  # [C] int64
    mean_entropy: float
    stable: int
    stop: bool
    probs: np.ndarray | None = None  # [C, V] tempered probabilities (for self-conditioning)


def sample_step(logits: np.ndarray, step: int, block: int, sched: Schedule,
                prev_pred: np.ndarray | None, stable: int, keep_probs: bool = False,
                T: float | None = None) -> StepResult:
    """One entropy-bounded sampling step over a canvas of logits [C, V]."""
    logits = np.asarray(logits, dtype=np.float64)
    C, V = logits.shape
    if T is None:
        T = temperature(step, sched)
    p = tempered_probs(logits, T)
    H = entropy_nats(p)
    pred = np.argmax(logits, axis=-1).astype(np.int64)  # first maximum = lowest index
    accept = cumulative_accept(H, sched.entropy_bound) if sched.accept_cumulative else H <= sched.entropy_bound
    noise = philox.draw_tokens(sched.seed, np.arange(C), step, block, philox.PURPOSE_RENOISE, V)
    keep = gumbel_sample(logits, T, sched.seed, step, block) if sched.categorical else pred
    nxt = np.where(accept, keep, noise)
    meanH = float(H.mean())
    if step > 0 and prev_pred is not None and np.array_equal(pred, prev_pred):
        stable = stable + 1
    else:
        stable = 0
    confident, steady = meanH < sched.stop_mean_entropy, stable >= sched.stable_needed
    stop = (confident or steady) if sched.stop_either else (confident and steady)
    return StepResult(H, pred, accept, nxt, meanH, stable, bool(stop), p if keep_probs else None)
