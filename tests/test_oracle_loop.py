"""Block-autoregressive loop of the oracle on a tiny random model.

Pins: the committed cache equals a fresh prefill of prompt + committed blocks
([P4] "Block Diffusion": the KV cache must accumulate correctly), every block
is the final step's argmax, and a random-init model never meets the stop
(entropy stays near ln V), so each canvas uses the whole step budget.
"""
import math

import numpy as np

import synthetic
from oracle import model as M
from oracle.loop import generate
from oracle.sampler import Schedule


def test_generate_tiny_model():
    s = dict(n_layers=1, d_model=16, n_q_heads=2, n_kv_heads=1, head_dim=8, n_experts=4, d_expert=8,
             d_shared=8, gated=0, vocab=64, d_selfcond=16)
    shape = M.ModelShape(n_layers=1, d_model=16, n_q_heads=2, n_kv_heads=1, head_dim=8, n_experts=4, top_k=2,
                         d_expert=8, d_shared=8, gated=False, vocab=64, d_selfcond=16, canvas=8)
    W = synthetic.SyntheticWeights(s, seed=0, dtype="f32")
    prompt = synthetic.uniform_ids(1, synthetic.TID_PROMPT, 6, 64)
    sched = Schedule(max_steps=4)
    cache, traces = generate(W, shape, sched, prompt, n_blocks=2, capacity=6 + 16)
    assert cache.length == 22
    for tr in traces:
        assert tr.steps == 4 and not tr.stopped
        assert np.array_equal(tr.block_ids, tr.results[-1].pred)
        for r in tr.results:
            assert abs(r.mean_entropy - math.log(64)) < 0.05
    fresh = M.KVCache.empty(shape, 22)
    M.encode(W, fresh, np.concatenate([prompt, traces[0].block_ids, traces[1].block_ids]), shape)
    np.testing.assert_allclose(fresh.k[0], cache.k[0], atol=1e-12)
    np.testing.assert_allclose(fresh.v[0], cache.v[0], atol=1e-12)
