"""GPU parity of the LM head that also produces the sampler's split-row records.

With dg_ctx_fuse_sampler_stats the LM head ([P3] "Encoder-denoiser design": logits at every canvas
position) folds its logits, as stored, into the entropy-bounded sampler's records (max, sum 2^u,
sum u 2^u, first argmax; [P3] "Inference mechanism", [P4] "Standard sampling settings") for every
row and 256-token vocabulary block, and dg_sample_canvas_fused samples from those records without
reading the logits again. Checked here:

* the logits are bit-identical to the plain LM head's;
* the decisions (argmax, accept mask, re-noised ids, stop state) equal the sampler pass's on the
  same logits and the oracle's, except rows whose entropy lies within 1e-4 of the bound; entropies
  and row statistics agree to float rounding;
* a vocabulary that is not a multiple of 256 (a last block with idle waves);
* the runtime loop and the native dg_generate_block give the same trajectory with the records;
* the argument checks (fp32 model, categorical sampling, another schedule).
"""
import numpy as np
import pytest

from oracle import sampler as OS

from gpu_util import announce, need_gpu, to_f64, torch
from test_gpu_model import ids_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    need_gpu()
    from canvas_denoising_amd import _lib, configs, runtime
    return _lib, configs, runtime


def _model(libs, vocab, canvas=64, seed=5):
    L, configs, runtime = libs
    desc = configs.desc(1, 256, 4, 2, 64, 8, 2, 128, 256, 1, vocab, 256, L.DG_BF16, canvas=canvas)
    model = runtime.Model(desc, 64 + 2 * canvas, seed=seed, sigma=0.05)
    model.prefill(ids_tensor(3, 64, vocab))
    return desc, model


def _same_decisions(a, b, entropy, bound=0.1):
    """a, b: SamplerStates after sampling the same logits; entropy: the reference entropies."""
    flag = np.abs(entropy - bound) <= 1e-4
    assert torch.equal(a.pred, b.pred)
    assert np.array_equal(a.accept.cpu().numpy()[~flag], b.accept.cpu().numpy()[~flag])
    assert np.array_equal(a.canvas.cpu().numpy()[~flag], b.canvas.cpu().numpy()[~flag])
    return flag


@pytest.mark.parametrize("vocab", [16384, 4160])
def test_records_from_the_lm_head_match_the_sampler_pass(libs, vocab):
    L, configs, runtime = libs
    announce(f"LM head with sampler records, vocab {vocab}")
    desc, model = _model(libs, vocab)
    C, V = desc.canvas, desc.vocab
    sched = L.make_sched(max_steps=48, seed=11)
    st = runtime.SamplerState(C, V)
    st.init(sched, 0)
    canvas0 = st.canvas.clone()
    plain0 = model.denoise_step(canvas0, 0).clone()
    st.sample(plain0, sched, 0, 0)
    canvas1 = st.canvas.clone()
    stats0 = st.row_stats.clone()
    T0 = L.dg_temperature(sched, 0)
    plain1 = model.denoise_step(canvas1, 1, plain0, stats0, T0, logits=torch.empty_like(plain0)).clone()

    model.fuse_sampler_stats(sched)
    for step, canvas, prev in ((0, canvas0, None), (1, canvas1, plain0)):
        out = torch.empty_like(plain0)
        if prev is None:
            model.denoise_step(canvas, step, logits=out)
        else:
            model.denoise_step(canvas, step, prev, stats0, T0, logits=out)
        torch.cuda.synchronize()
        plain = plain0 if step == 0 else plain1
        assert torch.equal(out, plain), "the LM head's logits change when it also makes the records"
        a, b = runtime.SamplerState(C, V), runtime.SamplerState(C, V)
        for s_ in (a, b):
            s_.init(sched, 0)
            s_.canvas.copy_(canvas)
        a.sample_fused(model.ctx, sched, step, 0)
        b.sample(out, sched, step, 0)
        torch.cuda.synchronize()
        res = OS.sample_step(to_f64(out), step, 0, OS.Schedule(seed=11), None, 0)
        flag = _same_decisions(a, b, res.entropy)
        assert np.array_equal(a.pred.cpu().numpy(), res.pred)
        assert np.array_equal(a.canvas.cpu().numpy()[~flag], res.next_canvas[~flag])
        assert np.abs(to_f64(a.entropy) - to_f64(b.entropy)).max() < 1e-5
        assert np.abs(to_f64(a.entropy) - res.entropy).max() < 1e-3
        assert np.allclose(to_f64(a.row_stats), to_f64(b.row_stats), rtol=1e-5, atol=1e-5)
        sa, sb = a.stop_state(), b.stop_state()
        assert sa["stable_count"] == sb["stable_count"] and sa["stopped"] == sb["stopped"]
        assert abs(sa["mean_entropy"] - sb["mean_entropy"]) < 1e-5
        print(f"step {step}: mean entropy {sa['mean_entropy']:.4f}, {int(flag.sum())} rows near the bound")
    model.fuse_sampler_stats(None)
    model.close()


def test_loops_with_records_from_the_lm_head(libs):
    """Four steps through the runtime loop with and without the records: step 0 is identical, later
    steps agree up to the self-conditioning's rounding; the native loop reproduces the runtime loop
    with the records bit for bit."""
    L, configs, runtime = libs
    announce("loops with the LM head's sampler records")
    desc, model = _model(libs, 16384)
    C, V = desc.canvas, desc.vocab
    sched = L.make_sched(max_steps=4, seed=3)
    st = runtime.SamplerState(C, V)
    logits = model.logits

    steps, _ = model.denoise_canvas(st, sched, 0, limit=1)
    ref0 = dict(pred=st.pred.clone(), canvas=st.canvas.clone(), logits=logits.clone())
    steps, _ = model.denoise_canvas(st, sched, 0)
    torch.cuda.synchronize()
    ref = dict(pred=st.pred.clone(), logits=logits.clone(), steps=steps)

    model.fuse_sampler_stats(sched)
    model.denoise_canvas(st, sched, 0, limit=1)
    torch.cuda.synchronize()
    assert torch.equal(st.pred, ref0["pred"]) and torch.equal(st.canvas, ref0["canvas"])
    assert torch.equal(logits, ref0["logits"])
    steps, _ = model.denoise_canvas(st, sched, 0)
    torch.cuda.synchronize()
    assert steps == ref["steps"]
    got = dict(pred=st.pred.clone(), canvas=st.canvas.clone(), logits=logits.clone(), stop=st.stop_state())
    d = (to_f64(got["logits"]) - to_f64(ref["logits"])).__abs__().max()
    assert d < 2e-2 * to_f64(ref["logits"]).__abs__().max(), f"self-conditioned logits moved by {d}"
    # the native loop with the records: the same trajectory, bit for bit
    logits.fill_(float("nan"))
    out = torch.empty(C, dtype=torch.int32, device="cuda")
    n = model.generate_block(sched, 0, out, commit=False)
    torch.cuda.synchronize()
    assert n == steps
    assert torch.equal(out, got["pred"]) and torch.equal(logits, got["logits"])
    assert runtime.stop_dict(model.buffer(L.DG_BUF_STOP, torch.int32, (4,))) == got["stop"]
    # another schedule's temperatures do not match the records
    other = L.make_sched(max_steps=4, seed=3, t_start=0.9)
    with pytest.raises(L.DGError):
        model.generate_block(other, 0, out, commit=False)
    model.fuse_sampler_stats(None)
    model.close()


def test_records_refused_where_they_cannot_serve(libs):
    L, configs, runtime = libs
    announce("sampler records: argument checks")
    desc, model = _model(libs, 4096)
    with pytest.raises(L.DGError):
        model.fuse_sampler_stats(L.make_sched(max_steps=8, seed=0, mode=L.DG_SCHED_SAMPLE))
    st = runtime.SamplerState(desc.canvas, desc.vocab)
    sched = L.make_sched(max_steps=8, seed=0)
    st.init(sched, 0)
    with pytest.raises(L.DGError):  # no records yet: the context does not make them
        st.sample_fused(model.ctx, sched, 0, 0)
    model.close()
    w = configs.tiny_f32()
    m32 = runtime.Model(w.desc, w.capacity, seed=None)
    with pytest.raises(L.DGError):
        m32.fuse_sampler_stats(L.make_sched(max_steps=8, seed=0))
    m32.close()
