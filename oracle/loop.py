"""The denoising loop of one canvas and block-autoregressive generation.

* [P4] "Reverse diffusion process": start from a canvas of random tokens,
  read it bidirectionally, compute per-position distributions, keep confident
  tokens, re-noise the rest, repeat, and fix the block once it is stable.
* [P4] "Two-Fold Adaptive Stopping": stop early when both conditions hold;
  otherwise run to the step budget ([P4] "Standard sampling settings").
* [P3] "Inference mechanism": self-conditioning feeds the previous step's
  probability-weighted embedding into the next step.
* [P4] "Block Diffusion": generate a 256-token block, append it to the
  context, update the KV cache, denoise the next canvas.

Readings: the committed block is the argmax vector of the final step (for
both a natural stop and the step-budget exit); the self-conditioning input at
step 0 is zero.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import model as M
from . import philox
from .sampler import Schedule, sample_step, temperature


@dataclass
class BlockTrace:
    block_ids: np.ndarray
    steps: int
    stopped: bool
    canvases: list = field(default_factory=list)   # canvas fed to each step
    results: list = field(default_factory=list)    # sampler StepResult per step
    temperatures: list = field(default_factory=list)


def denoise_block(step_fn, sched: Schedule, block: int, canvas_len: int, vocab: int) -> BlockTrace:
    """Run the loop with ``step_fn(step, canvas, prev_result, T_prev) -> logits``.

    ``step_fn`` is the model; a scripted function can stand in for it.
    """
    canvas = philox.init_canvas(sched.seed, canvas_len, block, vocab)
    prev_pred, stable = None, 0
    prev_res, prev_T = None, None
    tr = BlockTrace(np.zeros(canvas_len, np.int64), 0, False)
    for s in range(sched.max_steps):
        T = temperature(s, sched)
        logits = step_fn(s, canvas, prev_res, prev_T)
        res = sample_step(logits, s, block, sched, prev_pred, stable, keep_probs=True, T=T)
        tr.canvases.append(canvas.copy())
        tr.results.append(res)
        tr.temperatures.append(T)
        if res.stop or s == sched.max_steps - 1:
            tr.block_ids = res.pred.copy()
            tr.steps = s + 1
            tr.stopped = res.stop
            break
        prev_pred, stable = res.pred, res.stable
        prev_res, prev_T = res, T
        canvas = res.next_canvas
    return tr


def model_step_fn(W, cache: M.KVCache, shape: M.ModelShape):
    """Denoiser step with self-conditioning from the previous step's tempered probabilities."""
    def fn(s, canvas, prev_res, prev_T):
        sc = None if prev_res is None else M.self_condition(W, prev_res.probs)
        return M.denoise_step(W, cache, canvas, sc, shape)
    return fn


def generate(W, shape: M.ModelShape, sched: Schedule, prompt_ids, n_blocks: int, capacity: int):
    """Prefill the prompt, then denoise and commit ``n_blocks`` canvases."""
    cache = M.KVCache.empty(shape, capacity)
    M.encode(W, cache, prompt_ids, shape)
    traces = []
    for b in range(n_blocks):
        tr = denoise_block(model_step_fn(W, cache, shape), sched, b, shape.canvas, shape.vocab)
        M.encode(W, cache, tr.block_ids, shape)
        traces.append(tr)
    return cache, traces
