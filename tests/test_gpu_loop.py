"""GPU parity of self-conditioning at the benchmark's split and of a whole denoising trajectory.

* Self-conditioning ([P3] "Inference mechanism": the previous step's probabilities times the token
  embeddings, through a small FFN, into the next step) at d_model 2816 and a vocabulary of 16384:
  the P E product then runs exactly as at the benchmark size, 11 column blocks x 23 vocabulary
  shares on a 256-workgroup XCD-mapped grid with 3 padding workgroups and a 23-partial in-order
  sum. The self-conditioning vector of every canvas row is compared with the oracle, teacher-forced
  on the GPU's step-0 logits and row statistics, and so are the step-1 logits.
* The tiny fp32 configuration (1 layer, d_model 256, 16 experts top-2 with plain GeLU FFNs, vocab
  4096, 64 prompt tokens, 8 steps with the temperature falling linearly from 0.8 to 0.4; [P4]
  "Standard sampling settings", "Two-Fold Adaptive Stopping", "Block Diffusion") run step by step
  through the runtime loop: every step's self-conditioning vector and logits against the oracle
  teacher-forced on the GPU's canvas and previous logits, every sampler decision against the oracle
  on the GPU's logits, the whole trajectory against the oracle's own untethered loop, then the
  native dg_generate_block reproducing the loop bit for bit and committing the block.
"""
import numpy as np
import pytest

import synthetic
from oracle import loop as OL
from oracle import model as OM
from oracle import sampler as OS

from gpu_util import announce, need_gpu, to_f64, torch
from test_gpu_model import assert_close, check_routes, gpu_routes, ids_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    need_gpu()
    from canvas_denoising_amd import _lib, configs, runtime
    return _lib, configs, runtime


def _shape(desc, OM=OM):
    return OM.ModelShape(n_layers=desc.n_layers, d_model=desc.d_model, n_q_heads=desc.n_q_heads,
                         n_kv_heads=desc.n_kv_heads, head_dim=desc.head_dim, n_experts=desc.n_experts,
                         top_k=desc.top_k, d_expert=desc.d_expert, d_shared=desc.d_shared, gated=bool(desc.gated),
                         vocab=desc.vocab, d_selfcond=desc.d_selfcond, canvas=desc.canvas,
                         rms_eps=desc.rms_eps)


def test_self_conditioning_at_the_benchmark_split(libs):
    L, configs, runtime = libs
    announce("self-conditioning at d_model 2816, vocab 16384 (23 shares x 11 column blocks)")
    desc = configs.desc(1, 2816, 16, 8, 128, 8, 2, 128, 256, 1, 16384, 2816, L.DG_BF16, canvas=256)
    model = runtime.Model(desc, 64 + 256, seed=7, sigma=0.02)
    W = synthetic.SyntheticWeights(configs.shape_dict(desc), seed=7, dtype="bf16", sigma=0.02)
    shape = _shape(desc)
    prompt = ids_tensor(3, 64, desc.vocab)
    model.prefill(prompt)
    sched = L.make_sched(max_steps=48, seed=2)
    st = runtime.SamplerState(desc.canvas, desc.vocab)
    st.init(sched, 0)
    canvas0 = st.canvas.clone()
    logits0 = model.denoise_step(canvas0, 0).clone()
    st.sample(logits0, sched, 0, 0)
    T0 = L.dg_temperature(sched, 0)
    canvas1 = st.canvas.clone()
    logits1 = model.denoise_step(canvas1, 1, logits0, st.row_stats, T0, logits=torch.empty_like(logits0))
    torch.cuda.synchronize()
    routes1 = gpu_routes(L, model, desc.canvas)
    sc_gpu = to_f64(model.buffer(L.DG_BUF_SC, torch.float32, (desc.canvas, desc.d_model)))

    cache = OM.KVCache.empty(shape, 64 + 256)
    OM.encode(W, cache, prompt.cpu().numpy(), shape)  # one layer: its K/V do not depend on routing
    g0 = to_f64(logits0)
    # the sampler's row statistics, which the kernel turns back into probabilities
    stats = to_f64(st.row_stats)
    m_ref = g0.max(axis=1)
    lnz_ref = np.log(np.exp((g0 - m_ref[:, None]) / T0).sum(axis=1))
    assert np.array_equal(stats[:, 0], m_ref)
    np.testing.assert_allclose(stats[:, 1], lnz_ref, atol=1e-5)
    sc_ref = OM.self_condition(W, OS.tempered_probs(g0, T0))
    assert_close(sc_gpu, sc_ref, 2e-2, "self-conditioning vector (all 256 rows)")
    ref1, _, infos = OM.denoise_step(W, cache.copy(), canvas1.cpu().numpy(), sc_ref, shape, return_info=True,
                                     forced_sel=routes1)
    check_routes(routes1, infos, shape.top_k, "self-conditioned step")
    assert_close(to_f64(logits1), ref1, 2e-2, "self-conditioned step logits")
    model.close()


def test_tiny_config_trajectory(libs):
    L, configs, runtime = libs
    w = configs.tiny_f32()
    d = w.desc
    C, V, S = d.canvas, d.vocab, w.max_steps
    announce(f"tiny fp32 configuration: {S}-step trajectory, then the native loop and the commit")
    model = runtime.Model(d, w.capacity, seed=0, sigma=0.02)
    W = synthetic.SyntheticWeights(configs.shape_dict(d), seed=0, dtype="f32", sigma=0.02)
    shape = _shape(d)
    prompt = ids_tensor(1, w.prompt, V)
    model.prefill(prompt)
    cache = OM.KVCache.empty(shape, w.capacity)
    OM.encode(W, cache, prompt.cpu().numpy(), shape)
    torch.cuda.synchronize()
    gk, gv = model.kv_view()
    assert_close(to_f64(gk[0, :, :w.prompt]), cache.k[0][:, :w.prompt], 2e-4, "prompt K")
    assert_close(to_f64(gv[0, :, :w.prompt]), cache.v[0][:, :w.prompt], 2e-4, "prompt V")
    del gk, gv

    # the runtime loop, step by step, recording what each step saw and produced
    sched = L.make_sched(max_steps=S, seed=0)
    osched = OS.Schedule(max_steps=S, seed=0)
    st = runtime.SamplerState(C, V)
    st.init(sched, 0)
    logits = torch.empty(C, V, dtype=torch.float32, device="cuda")
    rec = []
    prev_pred, stable = None, 0
    for s in range(S):
        T = L.dg_temperature(sched, s)
        assert T == np.float32(OS.temperature(s, osched))
        canvas_in = st.canvas.clone()
        prev_logits = logits.clone() if s > 0 else None
        if s == 0:
            model.denoise_step(st.canvas, s, logits=logits)
        else:
            model.denoise_step(st.canvas, s, logits, st.row_stats, L.dg_temperature(sched, s - 1), logits=logits)
        st.sample(logits, sched, s, 0)
        torch.cuda.synchronize()
        sc = to_f64(model.buffer(L.DG_BUF_SC, torch.float32, (C, d.d_model))) if s > 0 else None
        r = dict(canvas=canvas_in.cpu().numpy().astype(np.int64), logits=to_f64(logits), sc=sc,
                 prev_logits=None if prev_logits is None else to_f64(prev_logits),
                 routes=gpu_routes(L, model, C), pred=st.pred.cpu().numpy().astype(np.int64),
                 accept=st.accept.cpu().numpy().astype(bool), next=st.canvas.cpu().numpy().astype(np.int64),
                 entropy=to_f64(st.entropy), stop=st.stop_state())
        rec.append(r)
        # teacher-forced model step: the GPU's canvas and previous logits
        sc_ref = None
        if s > 0:
            sc_ref = OM.self_condition(W, OS.tempered_probs(r["prev_logits"], OS.temperature(s - 1, osched)))
            assert_close(r["sc"], sc_ref, 2e-4, f"step {s} self-conditioning vector")
        ref, _, infos = OM.denoise_step(W, cache.copy(), r["canvas"], sc_ref, shape, return_info=True,
                                        forced_sel=r["routes"])
        check_routes(r["routes"], infos, shape.top_k, f"step {s}")
        assert_close(r["logits"], ref, 2e-4, f"step {s} logits")
        # teacher-forced sampler: the GPU's logits, previous prediction and stability count
        res = OS.sample_step(r["logits"], s, 0, osched, prev_pred, stable)
        flag = np.abs(res.entropy - osched.entropy_bound) <= 1e-4
        assert np.array_equal(r["pred"], res.pred), f"step {s} argmax"
        assert np.array_equal(r["accept"][~flag], res.accept[~flag]), f"step {s} accept mask"
        assert np.array_equal(r["next"][~flag], res.next_canvas[~flag]), f"step {s} next canvas"
        assert np.abs(r["entropy"] - res.entropy).max() < 1e-3, f"step {s} entropy"
        assert abs(r["stop"]["mean_entropy"] - res.mean_entropy) < 1e-3
        assert r["stop"]["stable_count"] == res.stable and r["stop"]["stopped"] == int(res.stop)
        assert r["stop"]["steps_run"] == s + 1
        prev_pred, stable = r["pred"], res.stable
        if res.stop:
            break
    steps = len(rec)
    print(f"trajectory: {steps} steps, mean entropy {rec[-1]['stop']['mean_entropy']:.3f} "
          f"(ln V = {np.log(V):.3f}), accepted {[int(r['accept'].sum()) for r in rec]}")
    assert steps == S  # a random-init model never reaches the stop (entropy ~ ln V)

    # the oracle's own, untethered trajectory: the same canvases and stop decisions; argmax equal
    # except where the oracle's two largest logits are closer than fp32 rounding can separate
    tr = OL.denoise_block(OL.model_step_fn(W, cache.copy(), shape), osched, 0, C, V)
    assert tr.steps == steps and tr.stopped == bool(rec[-1]["stop"]["stopped"])
    for s, (r, res) in enumerate(zip(rec, tr.results)):
        assert np.array_equal(r["canvas"], tr.canvases[s]), f"step {s} canvas (untethered)"
        top2 = -np.sort(-r["logits"], axis=1)[:, :2]
        near = (top2[:, 0] - top2[:, 1]) <= 1e-4 * np.sqrt((r["logits"] ** 2).mean(axis=1))
        assert np.array_equal(r["pred"][~near], res.pred[~near]), f"step {s} argmax (untethered)"
        flag = np.abs(res.entropy - osched.entropy_bound) <= 1e-4
        assert np.array_equal(r["next"][~flag], res.next_canvas[~flag]), f"step {s} next canvas (untethered)"
        assert np.abs(r["entropy"] - res.entropy).max() < 1e-3

    # the native loop reproduces the runtime loop bit for bit, then commits the block
    final_logits = logits.clone()
    out = torch.empty(C, dtype=torch.int32, device="cuda")
    n = model.generate_block(sched, 0, out, commit=True)
    torch.cuda.synchronize()
    assert n == steps
    assert np.array_equal(out.cpu().numpy(), rec[-1]["pred"])
    assert torch.equal(model.logits, final_logits)
    stop = runtime.stop_dict(model.buffer(L.DG_BUF_STOP, torch.int32, (4,)))
    assert stop == rec[-1]["stop"]
    assert model.length == w.prompt + C
    OM.encode(W, cache, out.cpu().numpy(), shape)
    gk, gv = model.kv_view()
    assert_close(to_f64(gk[0, :, :model.length]), cache.k[0][:, :model.length], 2e-4, "committed K")
    assert_close(to_f64(gv[0, :, :model.length]), cache.v[0][:, :model.length], 2e-4, "committed V")
    model.close()


@pytest.mark.parametrize("stable_needed,mode", [(3, 0), (2, 0), (0, 0), (3, 1)])
def test_pipelined_loops_stop_where_the_step_loop_stops(libs, stable_needed, mode):
    """The Python runtime's denoise_canvas and the native dg_generate_block read a step's stop state
    only when that step could have stopped ([P4] "Two-Fold Adaptive Stopping": the stable count is 0
    on step 0 and grows by one a step at most), launching the other steps back to back. With all
    weights zero every row's logits are equal, so the argmax (lowest index) never changes and the
    stable count is the step index; with a mean-entropy threshold above ln V the two-fold rule stops
    the canvas on step stable_needed (either rule: on step 0). Both loops must stop on that step,
    run no step after it, and leave the state the step-by-step loop (a read-back after every step)
    leaves."""
    L, configs, runtime = libs
    w = configs.tiny_f32()
    d = w.desc
    C, V, S = d.canvas, d.vocab, w.max_steps
    announce(f"pipelined stop read-back: stable_needed {stable_needed}, mode {mode}")
    model = runtime.Model(d, w.capacity, seed=None)
    model.weights.zero_()
    model.prefill(ids_tensor(1, w.prompt, V))
    sched = L.make_sched(max_steps=S, seed=0, stop_mean_entropy=1e9, stable_needed=stable_needed,
                         mode=L.DG_SCHED_STOP_EITHER if mode else 0)
    want = 1 if mode else stable_needed + 1
    assert want < S
    st = runtime.SamplerState(C, V)
    logits = model.logits

    # the step-by-step loop
    st.init(sched, 0)
    s = 0
    while True:
        if s > 0:
            model.denoise_step(st.canvas, s, logits, st.row_stats, L.dg_temperature(sched, s - 1), logits=logits)
        else:
            model.denoise_step(st.canvas, s, logits=logits)
        st.sample(logits, sched, s, 0)
        stop = st.stop_state()
        s += 1
        if stop["stopped"] or s == S:
            break
    assert s == want and stop["stopped"] == 1 and stop["steps_run"] == want
    ref = dict(pred=st.pred.clone(), canvas=st.canvas.clone(), logits=logits.clone(), stop=stop)

    # the runtime's pipelined loop
    logits.fill_(float("nan"))
    steps, stopped = model.denoise_canvas(st, sched, 0)
    torch.cuda.synchronize()
    assert (steps, stopped) == (want, True)
    assert st.stop_state() == ref["stop"]
    assert torch.equal(st.pred, ref["pred"]) and torch.equal(st.canvas, ref["canvas"])
    assert torch.equal(logits, ref["logits"])

    # the native loop
    logits.fill_(float("nan"))
    out = torch.empty(C, dtype=torch.int32, device="cuda")
    n = model.generate_block(sched, 0, out, commit=False)
    torch.cuda.synchronize()
    assert n == want
    assert torch.equal(out, ref["pred"])
    assert torch.equal(logits, ref["logits"])
    assert runtime.stop_dict(model.buffer(L.DG_BUF_STOP, torch.int32, (4,))) == ref["stop"]
    model.close()
