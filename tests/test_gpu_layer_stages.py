"""Stage-by-stage parity of one layer (dg_forward_layer) against the oracle.

Queries, attention output, post-attention normalised activations, router
logits, shared-expert activation, gated per-slot routed-expert outputs
(teacher-forced on the GPU's routing) and the layer output are each compared
with the float64 oracle, so a failure names the stage that broke.
"""
import numpy as np
import pytest

import synthetic
from oracle import model as OM

from gpu_util import announce, need_gpu, to_f64, torch
from test_gpu_model import assert_close, build, check_routes, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    need_gpu()
    from canvas_denoising_amd import _lib, configs, runtime
    return _lib, configs, runtime


@pytest.mark.parametrize("dtype,gated,causal,M,past,renorm,E", [
    ("bf16", 1, False, 64, 40, 0, 8), ("bf16", 1, True, 64, 0, 0, 8), ("bf16", 0, True, 50, 77, 0, 8),
    ("f32", 0, False, 64, 40, 0, 8), ("f32", 1, True, 37, 5, 0, 8), ("bf16", 1, False, 64, 40, 1, 8),
    ("f32", 0, True, 37, 5, 1, 8),
    # wider routings: 64 experts; 128 with 37 rows and renormalised gates; 192, ungated and causal
    ("bf16", 1, False, 64, 40, 0, 64), ("bf16", 1, True, 37, 5, 1, 128), ("bf16", 0, True, 50, 77, 0, 192)])
def test_layer_stages(libs, dtype, gated, causal, M, past, renorm, E):
    """renorm = 1: gates renormalised over the k chosen experts (dg_model_desc.renorm_gates)."""
    L, configs, runtime = libs
    announce(f"layer stages {dtype} gated={gated} causal={causal} M={M} past={past} renorm={renorm} E={E}")
    model, W, shape = build(libs, dtype=dtype, gated=gated, n_layers=1, canvas=64, capacity=256, renorm=renorm, E=E)
    tol = tol_for(dtype)
    rng = np.random.default_rng(M + past)
    if past:
        model.kv_write(0, torch.from_numpy(rng.normal(size=(shape.n_kv_heads, past, shape.head_dim))).cuda(),
                       torch.from_numpy(rng.normal(size=(shape.n_kv_heads, past, shape.head_dim))).cuda(), 0)
    L.dg_kv_set_length(model.ctx, past)
    x = torch.from_numpy(rng.normal(size=(M, shape.d_model)).astype(np.float32)).cuda()
    x0 = to_f64(x)
    model.forward_layer(0, x, M, causal)
    torch.cuda.synchronize()
    K, V = model.kv_view()

    lw = W["layers"][0]
    hd, Hq, Hkv, D = shape.head_dim, shape.n_q_heads, shape.n_kv_heads, shape.d_model
    QW = Hq * hd
    h = OM.rms_norm(x0, shape.rms_eps)
    q = h @ lw["wq"].T
    q_gpu = to_f64(model.buffer(L.DG_BUF_Q, model.dtype, (64, QW)))[:M]
    assert_close(q_gpu, q, tol, "queries")
    k = (h @ lw["wk"].T).reshape(M, Hkv, hd).transpose(1, 0, 2)
    v = (h @ lw["wv"].T).reshape(M, Hkv, hd).transpose(1, 0, 2)
    kc = np.concatenate([to_f64(K[0, :, :past]), k], axis=1)
    vc = np.concatenate([to_f64(V[0, :, :past]), v], axis=1)
    assert_close(to_f64(K[0, :, past:past + M]), k, tol, "written K")
    assert_close(to_f64(V[0, :, past:past + M]), v, tol, "written V")
    o = OM.attention(q.reshape(M, Hq, hd).transpose(1, 0, 2), kc, vc, past, causal).transpose(1, 0, 2).reshape(M, QW)
    o_gpu = to_f64(model.buffer(L.DG_BUF_ATTN, model.dtype, (64, QW)))[:M]
    assert_close(o_gpu, o, tol, "attention output")
    x1 = x0 + o @ lw["wo"].T
    h2 = OM.rms_norm(x1, shape.rms_eps)
    r = h2 @ lw["wr"].T
    r_gpu = to_f64(model.buffer(L.DG_BUF_ROUTER_LOGITS, torch.float32, (64, shape.n_experts)))[:M]
    assert_close(r_gpu, r, tol, "router logits")
    sel = model.buffer(L.DG_BUF_SEL, torch.int32, (64, shape.top_k)).cpu().numpy()[:M]
    assert np.array_equal(OM.topk_from_logits(r_gpu, shape.top_k), sel)
    up = h2 @ lw["sh_up"].T
    sh = (OM.gelu(h2 @ lw["sh_gate"].T) * up) if gated else OM.gelu(up)
    sh_gpu = to_f64(model.buffer(L.DG_BUF_SHARED_ACT, model.dtype, (64, shape.d_shared)))[:M]
    assert_close(sh_gpu, sh, tol, "shared-expert activation")
    gates = np.take_along_axis(OM.softmax(r_gpu), sel, axis=1)
    if renorm:
        gates = gates / gates.sum(axis=1, keepdims=True)
    gate_gpu = to_f64(model.buffer(L.DG_BUF_GATE, torch.float32, (64, shape.top_k)))[:M]
    np.testing.assert_allclose(gate_gpu, gates, rtol=2e-5, atol=1e-7)
    slot_of = model.buffer(L.DG_BUF_SLOT_OF, torch.int32, (64, shape.top_k)).cpu().numpy()[:M]
    assert sorted(slot_of.ravel().tolist()) == list(range(M * shape.top_k))
    slot_out = to_f64(model.buffer(L.DG_BUF_SLOT_OUT, torch.float32, (64 * shape.top_k, D)))
    want = np.zeros((M * shape.top_k, D))
    for t in range(M):
        for j in range(shape.top_k):
            want[slot_of[t, j]] = gates[t, j] * OM.ffn(h2[t:t + 1], lw["experts"][int(sel[t, j])], bool(gated))[0]
    assert_close(slot_out[:M * shape.top_k], want, tol, "routed expert outputs")
    # slots are expert-major and token-ascending
    order = sorted(range(M * shape.top_k), key=lambda p: (sel.ravel()[p], p // shape.top_k))
    assert [slot_of.ravel()[p] for p in order] == list(range(M * shape.top_k))
    # the experts' first slots, then the experts by decreasing token count (lower index on ties)
    E = shape.n_experts
    offs = model.buffer(L.DG_BUF_OFFSETS, torch.int32, (2 * E + 1,)).cpu().numpy()
    counts = np.bincount(sel.ravel(), minlength=E)
    assert np.array_equal(offs[:E + 1], np.concatenate([[0], np.cumsum(counts)]))
    assert offs[E + 1:].tolist() == sorted(range(E), key=lambda e: (-counts[e], e))
    y_ref, info = OM.layer_forward(lw, x0, np.concatenate([to_f64(K[0, :, :past]),
                                                        np.zeros((Hkv, 256 - past, hd))], axis=1),
                                np.concatenate([to_f64(V[0, :, :past]), np.zeros((Hkv, 256 - past, hd))], axis=1),
                                past, shape, causal, forced_sel=sel)
    # the oracle teacher-forced on the GPU's experts (its own near-tie choices may differ)
    check_routes([sel], [info], shape.top_k, "layer")
    assert_close(to_f64(x), y_ref, tol, "layer output")
    # the layer leaves h = RMSNorm(its output), the next layer's input
    h_gpu = to_f64(model.buffer(L.DG_BUF_H, model.dtype, (64, D)))[:M]
    assert_close(h_gpu, OM.rms_norm(y_ref, shape.rms_eps), tol, "output RMSNorm")
    # a second launch on the same input, with the routing outputs cleared first, routes again
    # identically
    model.buffer(L.DG_BUF_SEL, torch.int32, (64, shape.top_k)).zero_()
    model.buffer(L.DG_BUF_SLOT_OF, torch.int32, (64, shape.top_k)).zero_()
    L.dg_kv_set_length(model.ctx, past)
    model.forward_layer(0, torch.from_numpy(x0.astype(np.float32)).cuda(), M, causal)
    torch.cuda.synchronize()
    assert np.array_equal(model.buffer(L.DG_BUF_SEL, torch.int32, (64, shape.top_k)).cpu().numpy()[:M], sel)
    assert np.array_equal(model.buffer(L.DG_BUF_SLOT_OF, torch.int32, (64, shape.top_k)).cpu().numpy()[:M], slot_of)
    model.close()
