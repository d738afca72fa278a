"""GPU parity of the FP8 (E4M3) routed-expert mode against the oracle (oracle/fp8.py).

* Quantization: codes and float32 scales bit-exact against the oracle's per-row
  quantization of the same bf16 weights (both sides divide in float32,
  correctly rounded, and round to E4M3 nearest-even with saturation).
* Computation: layer outputs and logits against the oracle computing with the
  dequantized expert weights (code * scale in float64), to the bf16 tolerance
  (row relative error 2e-2, tests/test_gpu_model.assert_close); router
  near-ties flagged as in the bf16 tests. The FP8 results must also be closer
  to that oracle than to the bf16-weight oracle, so the mode is really in use.
* Switching back to the bf16 weights reproduces the bf16 results bit for bit.
* Full size (d_model 2816, 128 experts of width 704): codes and scales of
  sampled rows, and the layer output on sampled rows.
"""
import numpy as np
import pytest

import synthetic
from oracle import fp8 as OF
from oracle import model as OM

from gpu_util import announce, need_gpu, to_f64, torch
from test_gpu_model import ROUTER_TIE, assert_close, build, ids_tensor, router_flags

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    need_gpu()
    from canvas_denoising_amd import _lib, configs, runtime
    return _lib, configs, runtime


def fp8_index(R, K, which, gr, gw):
    """[R, K] byte positions of a matrix inside its expert's FP8 code region (the paired-tile order
    of include/dg.h): 1 KiB block (row group, column-tile pair, row block) holds, at 16 l .. 16 l + 15,
    slot l's 8 codes of the even column tile then its 8 codes of the odd one; slot l is row l % 16,
    columns 8 (l // 16) .. + 7 of a 32-column tile."""
    r = np.arange(R)[:, None]
    k = np.arange(K)[None, :]
    rb, kb = r // 16, k // 32
    block = ((rb // gr) * (K // 64) + kb // 2) * (gr * gw) + which * gr + rb % gr
    slot = r % 16 + 16 * ((k % 32) // 8)
    return block * 1024 + slot * 16 + (kb % 2) * 8 + k % 8


def device_codes(L, model, kind, layer, expert, R, K, which, gr, gw, rows=None):
    code_off, scale_off = L.dg_expert_fp8_tensor(model.desc, kind, layer, expert)
    n = gw * R * K
    region = model.expert_fp8[code_off:code_off + n].cpu().numpy()
    idx = fp8_index(R, K, which, gr, gw)
    if rows is not None:
        idx = idx[rows]
    scales = model.expert_fp8[scale_off:scale_off + 4 * R].view(torch.float32).cpu().numpy()
    return region[idx], scales if rows is None else scales[rows]


def matrices(L, d, gated):
    """(name, kind, R, K, which, gr, gw) of an expert's three matrices."""
    gw = 2 if gated else 1
    out = [("up", L.DG_W_EX_UP, d.d_expert, d.d_model, 1 if gated else 0, 2, gw),
           ("down", L.DG_W_EX_DOWN, d.d_model, d.d_expert, 0, 4, 1)]
    if gated:
        out.insert(0, ("gate", L.DG_W_EX_GATE, d.d_expert, d.d_model, 0, 2, gw))
    return out


@pytest.mark.parametrize("gated", [1, 0])
def test_quantize_matches_oracle(libs, gated):
    L, configs, runtime = libs
    announce(f"fp8 quantize gated={gated}")
    model, W, shape = build(libs, dtype="bf16", gated=gated, n_layers=2, E=8, F=128)
    model.use_expert_fp8(True)
    torch.cuda.synchronize()
    d = model.desc
    for layer in range(2):
        for e in range(d.n_experts):
            for name, kind, R, K, which, gr, gw in matrices(L, d, gated):
                codes, scales = device_codes(L, model, kind, layer, e, R, K, which, gr, gw)
                want_c, want_s = OF.quantize_rows(W["layers"][layer]["experts"][e][name].astype(np.float32))
                assert np.array_equal(scales.view(np.uint32), want_s.view(np.uint32)), (layer, e, name)
                bad = np.nonzero(codes != want_c)
                assert bad[0].size == 0, f"{layer} {e} {name}: {bad[0].size} codes differ, first at {bad[0][0], bad[1][0]}"
    # the codes use the whole range: saturating maxima, zeros and subnormals all occur
    allc = model.expert_fp8.cpu().numpy()
    assert (allc == 0x7E).any() and (allc == 0xFE).any()
    model.close()


def _err(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("gated", [1, 0])
def test_fp8_layer_matches_oracle(libs, gated):
    """One layer over 256 rows (top-2 of 4 experts: ~128 tokens per expert, several passes)."""
    L, configs, runtime = libs
    announce(f"fp8 forward_layer gated={gated}")
    model, W, shape = build(libs, dtype="bf16", gated=gated, n_layers=1, E=4, k=2, canvas=256, capacity=512,
                            d=128, Hq=2, Hkv=1, hd=64, F=192, Fs=128, V=256, dsc=64)
    rng = np.random.default_rng(11)
    x0 = rng.normal(size=(256, shape.d_model)).astype(np.float32)
    x_bf = torch.from_numpy(x0).cuda()
    model.forward_layer(0, x_bf, 256, False)
    model.use_expert_fp8(True)
    x = torch.from_numpy(x0).cuda()
    model.forward_layer(0, x, 256, False)
    torch.cuda.synchronize()
    V8 = OF.Fp8Weights(W)
    kv = OM.KVCache.empty(shape, 512)
    ref8, info = OM.layer_forward(V8["layers"][0], x0.astype(np.float64), kv.k[0], kv.v[0], 0, shape, False)
    kv = OM.KVCache.empty(shape, 512)
    ref16, _ = OM.layer_forward(W["layers"][0], x0.astype(np.float64), kv.k[0], kv.v[0], 0, shape, False)
    keep = OM.router_margin(info["router_logits"], shape.top_k) > ROUTER_TIE
    got = to_f64(x)[keep]
    assert_close(got, ref8[keep], 2e-2, "fp8 layer output")
    # the step from the input is what the experts changed: compare those deltas
    d8, d16, dg = ref8[keep] - x0[keep], ref16[keep] - x0[keep], got - x0[keep]
    e8, e16 = _err(dg, d8), _err(dg, d16)
    print(f"layer delta error vs fp8 oracle {e8:.3g}, vs bf16 oracle {e16:.3g}")
    assert e8 < 0.5 * e16
    assert not torch.equal(x, x_bf)
    model.close()


def test_fp8_step_and_switch_back(libs):
    L, configs, runtime = libs
    announce("fp8 denoise step, switch back to bf16")
    model, W, shape = build(libs, dtype="bf16", gated=1, n_layers=2, E=8, k=2, F=128)
    n_prompt = 80
    prompt = ids_tensor(1, n_prompt, shape.vocab)
    model.prefill(prompt)
    canvas = ids_tensor(2, shape.canvas, shape.vocab)
    a = model.denoise_step(canvas, 0).clone()
    model.use_expert_fp8(True)
    b = model.denoise_step(canvas, 0).clone()
    b2 = model.denoise_step(canvas, 0).clone()  # graph replay of the FP8 step
    model.use_expert_fp8(False)
    c = model.denoise_step(canvas, 0).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, c)
    assert torch.equal(b, b2)
    assert not torch.equal(a, b)
    cache = OM.KVCache.empty(shape, 512)
    OM.encode(W, cache, prompt.cpu().numpy(), shape)
    ref8, _, infos = OM.denoise_step(OF.Fp8Weights(W), cache.copy(), canvas.cpu().numpy(), None, shape,
                                     return_info=True)
    flag = router_flags(infos, shape.top_k)
    print(f"canvas router near-ties: {int(flag.sum())} of {shape.canvas}")
    assert_close(to_f64(b)[~flag], ref8[~flag], 2e-2, "fp8 step logits")
    model.close()


def test_fp8_errors(libs):
    L, configs, runtime = libs
    announce("fp8 error paths")
    model, W, shape = build(libs, dtype="f32", gated=0, n_layers=1)
    assert L.dg_expert_fp8_bytes(model.desc) == 0
    with pytest.raises(RuntimeError):
        L.dg_ctx_use_expert_fp8(model.ctx, torch.empty(256, dtype=torch.uint8, device="cuda"))
    model.close()
    model, W, shape = build(libs, dtype="bf16", gated=1, n_layers=1)
    buf = torch.empty(L.dg_expert_fp8_bytes(model.desc) + 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        L.dg_quantize_experts_fp8(model.desc, model.weights, buf[1:])
    with pytest.raises(RuntimeError):
        L.dg_ctx_use_expert_fp8(model.ctx, buf[1:])
    model.close()


def test_fp8_moe_layer_full_size(libs):
    L, configs, runtime = libs
    announce("fp8 full-size MoE layer (d 2816, 128 experts of 704)")
    w = configs.moe_layer_bf16()
    d = w.desc
    model = runtime.Model(d, w.capacity, seed=0, sigma=0.02)
    model.use_expert_fp8(True)
    C, D = d.canvas, d.d_model
    x0 = synthetic.normal_f32(2, synthetic.TID_X_INPUT, C * D, 1.0).reshape(C, D)
    x = torch.from_numpy(x0.copy()).cuda()
    model.forward_layer(0, x, C, False)  # no cached positions: the canvas attends to itself
    torch.cuda.synchronize()
    W = synthetic.SyntheticWeights(configs.shape_dict(d), seed=0, dtype="bf16", sigma=0.02, cache_experts=False)
    # codes and scales of sampled rows of two experts
    rows_of = {"gate": np.array([0, 17, 703]), "up": np.array([5, 702]), "down": np.array([0, 1234, 2815])}
    for e in (3, 127):
        ex = W["layers"][0]["experts"][e]
        for name, kind, R, K, which, gr, gw in matrices(L, d, True):
            rows = rows_of[name]
            codes, scales = device_codes(L, model, kind, 0, e, R, K, which, gr, gw, rows=rows)
            want_c, want_s = OF.quantize_rows(ex[name][rows].astype(np.float32))
            assert np.array_equal(scales.view(np.uint32), want_s.view(np.uint32)), (e, name)
            assert np.array_equal(codes, want_c), (e, name)
    # the layer on sampled rows, experts with dequantized weights
    lw = OF.Fp8Weights(W)["layers"][0]
    shape = OM.ModelShape(n_layers=1, d_model=D, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads, head_dim=d.head_dim,
                          n_experts=d.n_experts, top_k=d.top_k, d_expert=d.d_expert, d_shared=d.d_shared,
                          gated=True, vocab=d.vocab, d_selfcond=d.d_selfcond)
    xf = x0.astype(np.float64)
    h = OM.rms_norm(xf, shape.rms_eps)
    hd, G = d.head_dim, d.n_q_heads // d.n_kv_heads
    k = (h @ lw["wk"].T).reshape(C, d.n_kv_heads, hd).transpose(1, 0, 2)
    v = (h @ lw["wv"].T).reshape(C, d.n_kv_heads, hd).transpose(1, 0, 2)
    rows = np.arange(3, C, 13)
    q = (h[rows] @ lw["wq"].T).reshape(len(rows), d.n_q_heads, hd).transpose(1, 0, 2)
    o = np.stack([OM.softmax(q[j] @ k[j // G].T / np.sqrt(hd)) @ v[j // G] for j in range(d.n_q_heads)])
    x1 = xf[rows] + o.transpose(1, 0, 2).reshape(len(rows), -1) @ lw["wo"].T
    h2 = OM.rms_norm(x1, shape.rms_eps)
    r = h2 @ lw["wr"].T
    # the whole layer on the first 2 candidate rows whose k-th / (k+1)-th router logits are no near-tie
    pick = np.flatnonzero(OM.router_margin(r, d.top_k) > ROUTER_TIE)[:2]
    print(f"rows through the whole layer: {rows[pick].tolist()} ({len(pick)} of {len(rows)} candidates)")
    assert len(pick) == 2
    rows, x1, h2, r = rows[pick], x1[pick], h2[pick], r[pick]
    sel = OM.topk_from_logits(r, d.top_k)
    gates = np.take_along_axis(OM.softmax(r), sel, axis=1)
    y = OM.ffn(h2, lw, True, prefix="sh_")
    for i in range(len(rows)):
        for j in range(d.top_k):
            y[i] += gates[i, j] * OM.ffn(h2[i:i + 1], lw["experts"][int(sel[i, j])], True)[0]
    assert_close(to_f64(x)[rows], x1 + y, 2e-2, "fp8 layer output (sampled rows)")
    model.close()


def test_fp8_with_prefill_chunks(libs):
    """FP8 experts in a 1024-row prefill chunk (the token-tiled GEMMs over E4M3 codes, converted as
    they leave LDS), then a denoising step (the FP8 weight streams); against the oracle with the
    dequantised experts."""
    L, configs, runtime = libs
    announce("fp8 experts, prefill of 1500 tokens in 1024-row chunks")
    desc = configs.desc(2, 256, 4, 2, 64, 8, 2, 128, 256, 1, 512, 128, L.DG_BF16, canvas=64, prefill_rows=1024)
    model = runtime.Model(desc, 1600, seed=3, sigma=0.05)
    model.use_expert_fp8(True)
    W = synthetic.SyntheticWeights(configs.shape_dict(desc), seed=3, dtype="bf16", sigma=0.05)
    V8 = OF.Fp8Weights(W)
    shape = OM.ModelShape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, n_experts=8, top_k=2,
                          d_expert=128, d_shared=256, gated=True, vocab=512, d_selfcond=128, canvas=64)
    n = 1500
    prompt = ids_tensor(1, n, shape.vocab)
    model.prefill(prompt)
    canvas = ids_tensor(2, shape.canvas, shape.vocab)
    logits = model.denoise_step(canvas, 0)
    torch.cuda.synchronize()
    cache = OM.KVCache.empty(shape, 1600)
    infos = []
    OM.encode(V8, cache, prompt.cpu().numpy(), shape, infos=infos)
    keep = ~router_flags(infos, shape.top_k)
    K, _ = model.kv_view()
    k_gpu = to_f64(K[1, :, :n])  # layer 1 keys depend on layer 0's experts
    assert_close(k_gpu[:, keep], cache.k[1][:, :n][:, keep], 2e-2, "layer-1 keys after an FP8 chunked prefill")
    ref, _, cinfo = OM.denoise_step(V8, cache.copy(), canvas.cpu().numpy(), None, shape, return_info=True)
    cflag = router_flags(cinfo, shape.top_k)
    assert_close(to_f64(logits)[~cflag], ref[~cflag], 2e-2, "fp8 step logits after a chunked prefill")
    model.close()
