"""Pins of the oracle's scheduler, entropy-bounded sampler and stop rule.

Pinned against: the settings the pages print (tests/golden/sampling_settings.json),
closed forms of the entropy (uniform -> ln V, one-hot -> 0, k-way tie -> ln k,
two-level row), the monotonicity of entropy in temperature, and a scripted
truth table of the two-fold stop.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import philox
from oracle.loop import denoise_block
from oracle.sampler import Schedule, cumulative_accept, entropy_nats, sample_step, temperature, tempered_probs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sampling_settings.json")))


def test_defaults_are_the_pages_settings():
    s = Schedule()
    assert s.max_steps == GOLDEN["max_steps"]
    assert s.t_start == GOLDEN["t_start"] and s.t_end == GOLDEN["t_end"]
    assert s.entropy_bound == GOLDEN["entropy_bound"]
    assert s.stop_mean_entropy == GOLDEN["stop_mean_entropy"]
    assert s.stable_needed == GOLDEN["stable_matches"]


@pytest.mark.parametrize("S", [48, 8, 2])
def test_temperature_endpoints_and_linearity(S):
    s = Schedule(max_steps=S)
    T = [temperature(i, s) for i in range(S)]
    assert T[0] == float(np.float32(0.8))
    assert T[-1] == float(np.float32(0.4))
    assert all(a > b for a, b in zip(T, T[1:]))
    for i, t in enumerate(T):  # linear in the step index, up to one float32 rounding
        exact = 0.8 + (0.4 - 0.8) * i / (S - 1)
        assert abs(t - exact) <= 2 * np.finfo(np.float32).eps * exact


def test_temperature_single_step_budget():
    assert temperature(0, Schedule(max_steps=1)) == float(np.float32(0.8))


@pytest.mark.parametrize("V", [4096, 262144])
@pytest.mark.parametrize("T", [0.8, 0.4, 0.5791])
def test_uniform_entropy_is_log_v(V, T):
    row = np.full((1, V), 3.25)
    H = entropy_nats(tempered_probs(row, T))
    assert abs(H[0] - math.log(V)) < 1e-9


def test_one_hot_entropy_is_zero():
    V = 4096
    row = np.full((1, V), -1000.0)
    row[0, 1234] = 0.0
    res = sample_step(row, 5, 0, Schedule(), None, 0)
    assert res.entropy[0] == 0.0
    assert res.pred[0] == 1234 and res.accept[0] and res.next_canvas[0] == 1234


@pytest.mark.parametrize("k", [2, 3, 7])
def test_k_way_tie_entropy_and_lowest_index(k):
    V = 4096
    rng = np.random.default_rng(k)
    idx = np.sort(rng.choice(V, size=k, replace=False))
    row = np.full((1, V), -1000.0)
    row[0, idx] = 5.0
    res = sample_step(row, 3, 0, Schedule(), None, 0)
    assert abs(res.entropy[0] - math.log(k)) < 1e-12
    assert res.pred[0] == idx[0]


@given(a=st.floats(-20, 20), b=st.floats(-20, 20), T=st.floats(0.3, 1.0), V=st.sampled_from([2, 17, 4096]))
@settings(max_examples=200, deadline=None)
def test_two_level_row_closed_form(a, b, T, V):
    row = np.full((1, V), b)
    row[0, 0] = a
    H = entropy_nats(tempered_probs(row, T))[0]
    pa = 1.0 / (1.0 + (V - 1) * math.exp((b - a) / T))
    pb = (1.0 - pa) / (V - 1)
    want = -(pa * math.log(pa) if pa > 0 else 0.0) - (V - 1) * (pb * math.log(pb) if pb > 0 else 0.0)
    assert abs(H - want) < 1e-9


@given(seed=st.integers(0, 2**31), T1=st.floats(0.3, 1.5), T2=st.floats(0.3, 1.5))
@settings(max_examples=100, deadline=None)
def test_entropy_non_decreasing_in_temperature(seed, T1, T2):
    rng = np.random.default_rng(seed)
    row = rng.normal(0, 3, size=(4, 257))
    lo, hi = min(T1, T2), max(T1, T2)
    assert np.all(entropy_nats(tempered_probs(row, lo)) <= entropy_nats(tempered_probs(row, hi)) + 1e-12)


def test_accept_is_inclusive_and_renoise_is_philox():
    V, C = 4096, 64
    rng = np.random.default_rng(0)
    logits = rng.normal(0, 3, size=(C, V))
    logits[::2, 5] += 60.0  # even rows confident
    sched = Schedule(seed=11)
    T = temperature(7, sched)
    H = entropy_nats(tempered_probs(logits, T))
    # place the bound exactly on row 0's entropy: inclusive -> accepted
    sched.entropy_bound = float(H[0])
    res = sample_step(logits, 7, 2, sched, None, 0)
    assert res.accept[0]
    assert np.array_equal(res.accept, H <= H[0])
    noise = philox.draw_tokens(11, np.arange(C), 7, 2, philox.PURPOSE_RENOISE, V)
    assert np.array_equal(res.next_canvas[res.accept], res.pred[res.accept])
    assert np.array_equal(res.next_canvas[~res.accept], noise[~res.accept])
    assert res.mean_entropy == pytest.approx(H.mean(), abs=0)


def _scripted(preds_per_step, V=512, C=16, confident=True):
    """step_fn returning logits whose argmax follows ``preds_per_step``."""
    def fn(s, canvas, prev_res, prev_T):
        p = preds_per_step(s)
        logits = np.zeros((C, V))
        logits[np.arange(C), p] = 1000.0 if confident else 0.05
        return logits
    return fn


def test_stop_needs_both_conditions_earliest_step_two():
    C = 16
    fixed = np.arange(C) * 3
    tr = denoise_block(_scripted(lambda s: fixed), Schedule(), 0, C, 512)
    assert tr.stopped and tr.steps == 3  # t-2 == t-1 == t first holds at s = 2
    assert np.array_equal(tr.block_ids, fixed)


def test_low_entropy_but_changing_predictions_never_stops():
    C = 16
    tr = denoise_block(_scripted(lambda s: (np.arange(C) + s) % 512), Schedule(), 0, C, 512)
    assert not tr.stopped and tr.steps == 48
    assert all(r.mean_entropy == 0.0 for r in tr.results)


def test_stable_predictions_but_high_entropy_never_stops():
    C = 16
    fixed = np.arange(C)
    tr = denoise_block(_scripted(lambda s: fixed, confident=False), Schedule(max_steps=8), 0, C, 512)
    assert not tr.stopped and tr.steps == 8
    assert tr.results[-1].stable == 7
    assert all(r.mean_entropy > 0.005 for r in tr.results)


def test_prediction_change_resets_the_count():
    C = 16
    a, b = np.arange(C), np.arange(C) + 100
    tr = denoise_block(_scripted(lambda s: a if s < 3 else b), Schedule(), 0, C, 512)
    # a,a,a would stop at s=2; use a change at s=1 instead
    tr = denoise_block(_scripted(lambda s: a if s == 0 else b), Schedule(), 0, C, 512)
    assert [r.stable for r in tr.results] == [0, 0, 1, 2]
    assert tr.steps == 4 and np.array_equal(tr.block_ids, b)


def test_threshold_is_strict():
    C, V = 8, 64
    logits = np.zeros((C, V))
    logits[:, 0] = 12.0
    H = entropy_nats(tempered_probs(logits, temperature(2, Schedule())))
    sched = Schedule(stop_mean_entropy=float(H.mean()))
    prev = np.zeros(C, dtype=np.int64)
    assert not sample_step(logits, 2, 0, sched, prev, 1).stop   # mean == threshold: not below
    sched.stop_mean_entropy = float(np.nextafter(H.mean(), 1.0))
    assert sample_step(logits, 2, 0, sched, prev, 1).stop


def test_single_match_variant():
    C = 16
    fixed = np.arange(C)
    tr = denoise_block(_scripted(lambda s: fixed), Schedule(stable_needed=1), 0, C, 512)
    assert tr.steps == 2


def test_budget_exit_commits_final_prediction():
    C = 16
    tr = denoise_block(_scripted(lambda s: (np.arange(C) * 7 + s) % 512), Schedule(max_steps=5), 1, C, 512)
    assert tr.steps == 5 and not tr.stopped
    assert np.array_equal(tr.block_ids, (np.arange(C) * 7 + 4) % 512)
    # the first canvas is the block's Philox initialisation
    assert np.array_equal(tr.canvases[0], philox.init_canvas(0, C, 1, 512))


# ------------------------------------------------------------- sampler variants
# Either-condition stop ([P3] "Inference mechanism") and group acceptance by summed entropy
# ([P3] same section: "token groups"); the readings are in the oracle's header.

def test_either_stop_fires_on_entropy_alone():
    C = 16
    tr = denoise_block(_scripted(lambda s: (np.arange(C) + s) % 512), Schedule(stop_either=True), 0, C, 512)
    assert tr.stopped and tr.steps == 1  # confident from step 0, predictions never repeat


def test_either_stop_fires_on_stability_alone():
    C = 16
    fixed = np.arange(C)
    tr = denoise_block(_scripted(lambda s: fixed, confident=False), Schedule(max_steps=8, stop_either=True), 0, C, 512)
    assert tr.stopped and tr.steps == 3  # two equalities reached at s = 2; entropy stays high
    assert all(r.mean_entropy > 0.005 for r in tr.results)


def test_either_stop_needs_one_condition():
    C = 16
    tr = denoise_block(_scripted(lambda s: (np.arange(C) + s) % 512, confident=False),
                       Schedule(max_steps=6, stop_either=True), 0, C, 512)
    assert not tr.stopped and tr.steps == 6


def test_group_acceptance_worked_example():
    # increasing entropy: 0.01 (pos 1), 0.03 (pos 3), 0.04 (pos 4), 0.05 (pos 0), 0.2 (pos 2);
    # running totals 0.01, 0.04, 0.08, 0.13 -> the fourth passes 0.1: positions 1, 3, 4 accepted
    H = np.array([0.05, 0.01, 0.2, 0.03, 0.04])
    assert cumulative_accept(H, 0.1).tolist() == [False, True, False, True, True]


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_group_acceptance_equal_entropies_take_lowest_positions(k):
    # eight positions of entropy 0.1 / k + tiny: exactly k - 1 fit when the unit is just above 0.1 / k
    e = 0.1 / k * (1 + 1e-9)
    H = np.full(8, e)
    acc = cumulative_accept(H, 0.1)
    assert acc.tolist() == [True] * (k - 1) + [False] * (9 - k)
    # and exactly k when the unit is just below
    acc = cumulative_accept(np.full(8, 0.1 / k * (1 - 1e-9)), 0.1)
    assert acc.tolist() == [True] * k + [False] * (8 - k)


def test_group_acceptance_edge_cases():
    assert not cumulative_accept(np.array([0.5, 0.2, 0.3]), 0.1).any()        # nothing fits
    assert cumulative_accept(np.zeros(6), 0.1).all()                           # zero entropy always fits
    assert cumulative_accept(np.array([0.0, 0.1, 0.0]), 0.1).all()             # inclusive bound


@given(seed=st.integers(0, 2**31), n=st.integers(1, 40), bound=st.floats(0.0, 2.0))
@settings(max_examples=200, deadline=None)
def test_group_acceptance_is_the_longest_fitting_prefix(seed, n, bound):
    rng = np.random.default_rng(seed)
    H = rng.choice([0.0, 0.02, 0.05, 0.1, 0.3], size=n) * rng.random(n).round(1)
    acc = cumulative_accept(H, bound)
    order = np.lexsort((np.arange(n), H))  # increasing entropy, lower position first on ties
    # brute force over prefix lengths, each sum computed afresh
    best = max(L for L in range(n + 1) if all(H[order[:j]].sum() <= bound for j in range(1, L + 1)))
    assert acc.sum() == best
    assert set(np.nonzero(acc)[0]) == set(order[:best].tolist())


def test_group_acceptance_in_a_sampling_step():
    C, V = 6, 64
    logits = np.zeros((C, V))
    logits[[0, 2, 5], [3, 7, 9]] = 1000.0   # one-hot rows: entropy 0
    logits[4, :2] = 1000.0                   # two-way tie: ln 2 > bound
    sched = Schedule(seed=3, accept_cumulative=True)
    res = sample_step(logits, 4, 1, sched, None, 0)
    assert res.accept.tolist() == [True, False, True, False, False, True]
    noise = philox.draw_tokens(3, np.arange(C), 4, 1, philox.PURPOSE_RENOISE, V)
    assert np.array_equal(res.next_canvas, np.where(res.accept, res.pred, noise))


def test_categorical_frequencies_follow_the_tempered_softmax():
    # the same four-token row at 4096 positions x 4 steps: Gumbel-max draws must follow softmax(l / T)
    from scipy import stats
    from oracle.sampler import gumbel_sample
    l = np.array([0.0, 1.0, 2.0, 0.5])
    T = 0.8
    rows = np.tile(l, (4096, 1))
    counts = np.zeros(4)
    for step in range(4):
        counts += np.bincount(gumbel_sample(rows, T, 21, step, 3), minlength=4)
    p = np.exp(l / T) / np.exp(l / T).sum()
    chi2 = ((counts - counts.sum() * p) ** 2 / (counts.sum() * p)).sum()
    assert stats.chi2.sf(chi2, 3) > 1e-3, (counts / counts.sum(), p)
    # the untempered distribution is clearly rejected (the draws do depend on T)
    q = np.exp(l) / np.exp(l).sum()
    chi2q = ((counts - counts.sum() * q) ** 2 / (counts.sum() * q)).sum()
    assert stats.chi2.sf(chi2q, 3) < 1e-6


def test_categorical_limits():
    from oracle.sampler import gumbel_sample
    rng = np.random.default_rng(2)
    logits = rng.normal(0, 3, size=(64, 300))
    # T -> 0: the draw is the argmax
    assert np.array_equal(gumbel_sample(logits, 1e-6, 7, 0, 0), np.argmax(logits, axis=1))
    # a one-hot row always draws its peak
    oh = np.full((16, 300), -1000.0)
    oh[np.arange(16), np.arange(16) * 7] = 0.0
    for step in range(5):
        assert np.array_equal(gumbel_sample(oh, 0.8, 7, step, 1), np.arange(16) * 7)
    # draws differ between steps at a flat row (fresh noise every step)
    flat = np.zeros((64, 300))
    draws = [gumbel_sample(flat, 0.8, 7, s, 0) for s in range(3)]
    assert not np.array_equal(draws[0], draws[1]) and not np.array_equal(draws[1], draws[2])


def test_uniform24_is_uniform_on_a_24_bit_grid():
    from scipy import stats
    u = philox.uniform24(99, np.arange(64), 5, 2, 1000).ravel()
    k = u * (1 << 24) - 0.5
    assert np.array_equal(k, np.round(k)) and k.min() >= 0 and k.max() < (1 << 24)
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_categorical_step_keeps_draws_only_where_accepted():
    from oracle.sampler import gumbel_sample
    C, V = 8, 64
    logits = np.zeros((C, V))
    logits[0:4, 5] = 1000.0                     # confident rows
    logits[4:, :] = np.linspace(0, 1, V)       # flat-ish rows
    sched = Schedule(seed=5, categorical=True)
    res = sample_step(logits, 2, 1, sched, None, 0)
    T = temperature(2, sched)
    draws = gumbel_sample(logits, T, 5, 2, 1)
    noise = philox.draw_tokens(5, np.arange(C), 2, 1, philox.PURPOSE_RENOISE, V)
    assert res.accept.tolist() == [True] * 4 + [False] * 4
    assert np.array_equal(res.next_canvas, np.where(res.accept, draws, noise))
    assert np.array_equal(res.pred, np.argmax(logits, axis=1))
