"""GPU checks of dg_ctx_set_weights and the runtime's load-time choice among copies of the weights.

A context pointed at a device copy of its weights computes bit-identical logits (the step graph is
re-captured), no longer reads the old buffer, and rejects NULL and misaligned buffers.
Model.place_weights keeps the buffer its measure() ranks fastest.
"""
import pytest

from gpu_util import announce, need_gpu, torch
from test_gpu_model import ids_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    need_gpu()
    from canvas_denoising_amd import _lib, configs, runtime
    return _lib, configs, runtime


def _model(libs):
    L, configs, runtime = libs
    desc = configs.desc(2, 256, 4, 2, 64, 8, 2, 128, 256, 1, 4096, 256, L.DG_BF16, canvas=64)
    model = runtime.Model(desc, 64 + 2 * 64, seed=7, sigma=0.05)
    model.prefill(ids_tensor(5, 64, 4096))
    return desc, model


def test_copy_of_the_weights_gives_the_same_logits(libs):
    L, configs, runtime = libs
    announce("dg_ctx_set_weights: a copy of the weights")
    desc, model = _model(libs)
    canvas = ids_tensor(9, desc.canvas, desc.vocab)
    ref = model.denoise_step(canvas, 0).clone()
    old = model.weights
    copy = torch.empty_like(old)
    copy.copy_(old)
    model.set_weights(copy)
    got = model.denoise_step(canvas, 0).clone()
    assert torch.equal(got, ref)
    old.zero_()  # the old buffer is no longer read
    got = model.denoise_step(canvas, 0).clone()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    with pytest.raises(L.DGError):
        L.dg_ctx_set_weights(model.ctx, None)
    with pytest.raises(L.DGError):
        L.dg_ctx_set_weights(model.ctx, copy[16:])
    assert torch.equal(model.denoise_step(canvas, 0), ref)  # a refused call changes nothing
    model.close()


def test_place_weights_keeps_the_fastest(libs):
    L, configs, runtime = libs
    announce("Model.place_weights")
    desc, model = _model(libs)
    canvas = ids_tensor(9, desc.canvas, desc.vocab)
    ref = model.denoise_step(canvas, 0).clone()
    seen = []
    fake = iter([3.0, 1.0, 2.0])

    def measure():
        seen.append(model.weights.data_ptr())
        model.denoise_step(canvas, 0)
        torch.cuda.synchronize()
        return next(fake)

    times, kept = model.place_weights(measure, tries=3)
    assert times == [3.0, 1.0, 2.0] and kept == 1
    assert len(set(seen)) == 3 and model.weights.data_ptr() == seen[1]
    assert torch.equal(model.denoise_step(canvas, 0), ref)
    model.close()
