"""dg_sample_canvas_static (no workspace argument: the library's static device scratch) against
dg_sample_canvas with a caller workspace, through the C ABI: two calls in a row, the second on a
smaller input (the shared scratch keeps the first call's records), every output bit for bit; and a
shape whose records exceed the static scratch is refused before anything runs."""
import numpy as np
import pytest

from gpu_util import announce, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    need_gpu()
    from canvas_denoising_amd import _lib
    return _lib


def _outputs(rows, dev="cuda"):
    return dict(canvas=torch.zeros(rows, dtype=torch.int32, device=dev),
                pred=torch.full((rows,), -1, dtype=torch.int32, device=dev),
                accept=torch.zeros(rows, dtype=torch.uint8, device=dev),
                entropy=torch.zeros(rows, dtype=torch.float32, device=dev),
                stats=torch.zeros(rows, 2, dtype=torch.float32, device=dev),
                stop=torch.zeros(4, dtype=torch.int32, device=dev))


def _run(L, logits, dtype, rows, vocab, sched, step, block, o, prev_pred, workspace=None):
    o["pred"].copy_(prev_pred)
    L.dg_init_canvas(sched, block, rows, vocab, o["canvas"], o["stop"])
    args = (logits, dtype, rows, vocab, sched, step, block, o["canvas"], o["pred"], o["accept"], o["entropy"],
            o["stats"], o["stop"])
    if workspace is None:
        L.dg_sample_canvas_static(*args)
    else:
        L.dg_sample_canvas(*args, workspace, workspace.numel())


@pytest.mark.parametrize("order", ["large_then_small"])
def test_static_scratch_sampler_matches_workspace_sampler(L, order):
    announce("dg_sample_canvas_static: 256 x 262144 bf16, then 37 x 4096 fp32")
    cases = []
    # call 1: a full canvas at the benchmark vocabulary, planted-peak bf16 logits (the sampler workload)
    big = torch.empty(256, 262144, dtype=torch.bfloat16, device="cuda")
    L.dg_synth_planted_logits(0, 5, 256, 262144, 3.0, 12.0, big)
    cases.append((big, L.DG_BF16, 256, 262144, 5))
    # call 2: smaller and in fp32, with rows of sharply peaked logits so some positions are accepted
    rng = np.random.default_rng(1)
    x = rng.normal(0, 2, size=(37, 4096)).astype(np.float32)
    x[::2, 11] += 60.0
    cases.append((torch.from_numpy(x).cuda(), L.DG_F32, 37, 4096, 3))
    sched = L.make_sched(max_steps=48, seed=9)
    for logits, dtype, rows, vocab, step in cases:
        prev = torch.from_numpy(np.arange(rows, dtype=np.int32) % vocab).cuda()
        ws = torch.zeros(max(256, L.dg_sample_workspace_size(rows, vocab)), dtype=torch.uint8, device="cuda")
        a, b = _outputs(rows), _outputs(rows)
        _run(L, logits, dtype, rows, vocab, sched, step, 1, a, prev, workspace=ws)
        _run(L, logits, dtype, rows, vocab, sched, step, 1, b, prev)
        torch.cuda.synchronize()
        for k in a:
            assert torch.equal(a[k], b[k]), f"{rows}x{vocab}: {k} differs"
        print(f"{rows}x{vocab}: accepted {int(b['accept'].sum())}, stop state {b['stop'].cpu().tolist()}")
    assert int(b["accept"].sum()) > 0  # the second call exercised acceptance
    # records beyond the 1 MiB static scratch: refused, nothing written
    rows, vocab = 65535, 8192
    assert L.dg_sample_workspace_size(rows, vocab) > (1 << 20)
    o = _outputs(rows)
    before = {k: v.clone() for k, v in o.items()}
    with pytest.raises(L.DGError) as err:
        L.dg_sample_canvas_static(torch.zeros(rows, vocab, dtype=torch.bfloat16, device="cuda"), L.DG_BF16, rows,
                                  vocab, sched, 0, 0, o["canvas"], o["pred"], o["accept"], o["entropy"], o["stats"],
                                  o["stop"])
    assert err.value.code == L.DG_ERR_CAPACITY
    torch.cuda.synchronize()
    for k in o:
        assert torch.equal(o[k], before[k])
