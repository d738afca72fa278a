"""Parity at the benchmark's full sizes, on sampled outputs the oracle computes one by one.

* One MoE denoiser layer (d_model 2816, 16q/8kv x 128 heads, 128 experts top-8 of
  width 704 gated + shared 2816) over a 256-row canvas attending to 4096 cached
  positions plus the canvas: canvas K for every row, router logits for every row
  (exact top-8 teacher-forced on the GPU's logits), every one of the 2048 gated
  routed-expert slot outputs (all 128 experts of the dominant kernel's launch)
  and the layer output of every row, the oracle teacher-forced on the GPU's
  expert choice.
* The 30-layer, 262144-vocab step: the sampler teacher-forced on the GPU's
  logits (exact), LM-head logits on sampled (row, vocab) pairs from the GPU's
  final normalised activations, the self-conditioning vector of sampled rows
  (the embedding streamed through the host in vocabulary chunks), and the
  committed block's K/V in deeper layers at sampled positions, teacher-forced
  on the GPU's caches of the layers below.
"""
import concurrent.futures as cf

import numpy as np
import pytest

import synthetic
from oracle import model as OM
from oracle import sampler as OS

from gpu_util import announce, need_gpu, to_f64, torch
from test_gpu_model import ROUTER_TIE, assert_close, check_routes, gpu_routes

pytestmark = pytest.mark.gpu

POOL = 16  # host threads for generating weights (NumPy releases the GIL inside its array operations)


def expert_ffns(W, layer, rows_of, h, gated=True):
    """{expert: FFN_e(h[rows])} for the experts in rows_of (expert -> row indices), weights generated
    on a thread pool and dropped after use."""
    def one(e):
        ex = W["layers"][layer]["experts"][e]
        return e, OM.ffn(h[rows_of[e]], {k: ex[k] for k in (("gate", "up", "down") if gated else ("up", "down"))},
                         gated)
    with cf.ThreadPoolExecutor(POOL) as pool:
        return dict(pool.map(one, sorted(rows_of)))


def embed_rows(ids, D, seed=0):
    """Rows of the synthetic embedding (as the device fills it), float64."""
    idx = (np.asarray(ids, dtype=np.uint64)[:, None] * np.uint64(D) + np.arange(D, dtype=np.uint64)[None, :]).ravel()
    return synthetic.bf16_bits_to_f32(synthetic.normal_bf16_bits(seed, synthetic.TID_EMBED, idx, 0.02)).astype(
        np.float64).reshape(len(ids), D)


def probs_times_embedding(p, V, D, chunk=16384, seed=0):
    """u = p E for p [rows x V], E streamed in vocabulary chunks generated on a thread pool."""
    def part(c0):
        c1 = min(V, c0 + chunk)
        return p[:, c0:c1] @ embed_rows(np.arange(c0, c1), D, seed)
    with cf.ThreadPoolExecutor(POOL) as pool:
        parts = list(pool.map(part, range(0, V, chunk)))
    u = np.zeros((p.shape[0], D))
    for x in parts:  # fixed order
        u += x
    return u


@pytest.fixture(scope="module")
def libs():
    need_gpu()
    from canvas_denoising_amd import _lib, configs, runtime
    return _lib, configs, runtime


@pytest.mark.parametrize("rope", [0.0, 10000.0])
def test_moe_layer_full_size(libs, rope):
    L, configs, runtime = libs
    announce(f"full-size MoE layer (d 2816, 128 experts, 4096 cached) rope={rope}")
    w = configs.moe_layer_bf16()
    d = w.desc
    d.rope_theta = rope
    model = runtime.Model(d, w.capacity, seed=0, sigma=0.02)
    past, C, D, hd = w.prompt, d.canvas, d.d_model, d.head_dim
    kv_n = d.n_kv_heads * past * hd
    kb = synthetic.normal_bf16_bits(3, synthetic.TID_KV_INPUT, kv_n, 1.0).reshape(d.n_kv_heads, past, hd)
    vb = synthetic.normal_bf16_bits(3, synthetic.TID_KV_INPUT + 1, kv_n, 1.0).reshape(d.n_kv_heads, past, hd)
    model.kv_write(0, torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16),
                   torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16), 0)
    L.dg_kv_set_length(model.ctx, past)
    x0 = synthetic.normal_f32(2, synthetic.TID_X_INPUT, C * D, 1.0).reshape(C, D)
    x = torch.from_numpy(x0.copy()).cuda()
    model.forward_layer(0, x, C, False)
    torch.cuda.synchronize()
    K, V = model.kv_view()

    W = synthetic.SyntheticWeights(configs.shape_dict(d), seed=0, dtype="bf16", sigma=0.02, cache_experts=False)
    lw = W["layers"][0]
    shape = OM.ModelShape(n_layers=1, d_model=D, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads, head_dim=hd,
                          n_experts=d.n_experts, top_k=d.top_k, d_expert=d.d_expert, d_shared=d.d_shared,
                          gated=True, vocab=d.vocab, d_selfcond=d.d_selfcond)
    xf = x0.astype(np.float64)
    h = OM.rms_norm(xf, shape.rms_eps)
    k = (h @ lw["wk"].T).reshape(C, d.n_kv_heads, hd).transpose(1, 0, 2)
    v = (h @ lw["wv"].T).reshape(C, d.n_kv_heads, hd).transpose(1, 0, 2)
    if rope > 0:
        k = OM.rope(k, past + np.arange(C), rope)
    assert_close(to_f64(K[0, :, past:past + C]), k, 2e-2, "canvas K (all rows)")
    kc = np.concatenate([synthetic.bf16_bits_to_f32(kb).astype(np.float64), k], axis=1)
    vc = np.concatenate([synthetic.bf16_bits_to_f32(vb).astype(np.float64), v], axis=1)
    # teacher-forced routing on every row
    r_gpu = to_f64(model.buffer(L.DG_BUF_ROUTER_LOGITS, torch.float32, (C, d.n_experts)))
    sel_gpu = model.buffer(L.DG_BUF_SEL, torch.int32, (C, d.top_k)).cpu().numpy()
    assert np.array_equal(OM.topk_from_logits(r_gpu, d.top_k), sel_gpu)
    counts = np.bincount(sel_gpu.ravel(), minlength=d.n_experts)
    print(f"tokens per expert: min {counts.min()} max {counts.max()}, experts used {int((counts > 0).sum())}")
    # every row through attention (the oracle's float64 over all 4352 keys)
    q = (h @ lw["wq"].T).reshape(C, d.n_q_heads, hd).transpose(1, 0, 2)
    if rope > 0:
        q = OM.rope(q, past + np.arange(C), rope)
    o = OM.attention(q, kc, vc, past, causal=False).transpose(1, 0, 2).reshape(C, d.n_q_heads * hd)
    x1 = xf + o @ lw["wo"].T
    h2 = OM.rms_norm(x1, shape.rms_eps)
    r = h2 @ lw["wr"].T
    assert_close(r_gpu, r, 2e-2, "router logits (all rows)")
    check_routes([sel_gpu], [{"router_logits": r}], d.top_k, "full-size layer")
    # every routed slot, teacher-forced on the GPU's experts: gate x FFN_e(h2) against DG_BUF_SLOT_OUT
    gates = np.take_along_axis(OM.softmax(r), sel_gpu, axis=1)
    rows_of = {}
    for t in range(C):
        for j in range(d.top_k):
            rows_of.setdefault(int(sel_gpu[t, j]), []).append(t)
    outs = expert_ffns(W, 0, {e: np.array(v) for e, v in rows_of.items()}, h2)
    slot_of = model.buffer(L.DG_BUF_SLOT_OF, torch.int32, (C, d.top_k)).cpu().numpy()
    assert sorted(slot_of.ravel().tolist()) == list(range(C * d.top_k))
    order = sorted(range(C * d.top_k), key=lambda p: (sel_gpu.ravel()[p], p // d.top_k))
    assert [slot_of.ravel()[p] for p in order] == list(range(C * d.top_k)), "slots expert-major, token-ascending"
    E = d.n_experts
    offs = model.buffer(L.DG_BUF_OFFSETS, torch.int32, (2 * E + 1,)).cpu().numpy()
    counts = np.bincount(sel_gpu.ravel(), minlength=E)
    assert np.array_equal(offs[:E + 1], np.concatenate([[0], np.cumsum(counts)]))
    assert offs[E + 1:].tolist() == sorted(range(E), key=lambda e: (-counts[e], e)), "experts by token count"
    want = np.zeros((C * d.top_k, D))
    y = OM.ffn(h2, lw, True, prefix="sh_")
    pos_in = {e: {t: i for i, t in enumerate(v)} for e, v in rows_of.items()}
    for t in range(C):
        for j in range(d.top_k):
            e = int(sel_gpu[t, j])
            val = gates[t, j] * outs[e][pos_in[e][t]]
            want[slot_of[t, j]] = val
            y[t] += val
    slot_out = to_f64(model.buffer(L.DG_BUF_SLOT_OUT, torch.float32, (C * d.top_k, D)))
    assert_close(slot_out, want, 2e-2, "routed-expert slot outputs (all 2048 slots, all 128 experts)")
    assert_close(to_f64(x), x1 + y, 2e-2, "layer output (all rows)")
    model.close()


@pytest.mark.slow
def test_full_step_sampled(libs):
    L, configs, runtime = libs
    w = configs.full_loop_bf16()
    d = w.desc
    d.prefill_rows = 2048  # as bench.py runs it: the prompt prefilled in 2048-row chunks
    C, V, D = d.canvas, d.vocab, d.d_model
    announce("full-size 30-layer step: prefill 8192, denoise, sample, self-conditioned step, commit")
    model = runtime.Model(d, w.prompt + 2 * C, seed=0, sigma=0.02)
    prompt = torch.from_numpy(synthetic.uniform_ids(4, synthetic.TID_PROMPT, w.prompt, V)).cuda()
    model.prefill(prompt)
    sched = L.make_sched(max_steps=48, seed=0)
    st = runtime.SamplerState(C, V)
    st.init(sched, 0)
    canvas0 = st.canvas.clone()
    logits = model.denoise_step(st.canvas, 0)
    torch.cuda.synchronize()
    # LM head on sampled (row, vocab) pairs from the GPU's final normalised activations
    h = to_f64(model.buffer(L.DG_BUF_H, torch.bfloat16, (C, D)))
    rng = np.random.default_rng(0)
    cols = np.sort(rng.choice(V, size=2048, replace=False))
    idx = (cols[:, None].astype(np.uint64) * np.uint64(D) + np.arange(D, dtype=np.uint64)[None, :]).ravel()
    E_cols = synthetic.bf16_bits_to_f32(synthetic.normal_bf16_bits(0, synthetic.TID_EMBED, idx, 0.02))
    E_cols = E_cols.astype(np.float64).reshape(len(cols), D)
    assert_close(to_f64(logits[:, torch.from_numpy(cols).cuda()]), h @ E_cols.T, 2e-2, "LM head (sampled vocab)")
    # sampler teacher-forced on the GPU's logits: exact discrete outputs
    st.sample(logits, sched, 0, 0)
    torch.cuda.synchronize()
    lg = to_f64(logits)
    res = OS.sample_step(lg, 0, 0, OS.Schedule(seed=0), None, 0)
    assert np.array_equal(st.pred.cpu().numpy(), res.pred)
    flag = np.abs(res.entropy - 0.1) <= 1e-4
    assert np.array_equal(st.canvas.cpu().numpy()[~flag], res.next_canvas[~flag])
    assert np.abs(to_f64(st.entropy) - res.entropy).max() < 1e-3
    print(f"mean entropy {res.mean_entropy:.3f} (ln V = {np.log(V):.3f}), accepted {int(res.accept.sum())}")
    # the LM head making the sampler's records itself (1024 vocabulary blocks a row, merged 64 at a
    # time): the same logits, and the same decisions without a second read of them
    model.fuse_sampler_stats(sched)
    logits_f = model.denoise_step(canvas0, 0, logits=torch.empty_like(logits))
    stf = runtime.SamplerState(C, V)
    stf.init(sched, 0)
    stf.sample_fused(model.ctx, sched, 0, 0)
    torch.cuda.synchronize()
    assert torch.equal(logits_f, logits)
    assert np.array_equal(stf.pred.cpu().numpy(), res.pred)
    assert np.array_equal(stf.canvas.cpu().numpy()[~flag], res.next_canvas[~flag])
    assert np.abs(to_f64(stf.entropy) - to_f64(st.entropy)).max() < 1e-5
    assert np.allclose(to_f64(stf.row_stats), to_f64(st.row_stats), rtol=1e-5, atol=1e-5)
    model.fuse_sampler_stats(None)
    # a self-conditioned step at full size: the self-conditioning vector of sampled rows against
    # the oracle's p E (E streamed through the host in vocabulary chunks), teacher-forced on the
    # GPU's step-0 logits
    T0 = L.dg_temperature(sched, 0)
    logits1 = model.denoise_step(st.canvas, 1, logits, st.row_stats, T0, logits=torch.empty_like(logits))
    torch.cuda.synchronize()
    assert torch.isfinite(logits1.float()).all()
    sc = to_f64(model.buffer(L.DG_BUF_SC, torch.float32, (C, D)))
    rows = np.array([0, 1, 37, 100, 128, 200, 254, 255])
    p = OS.tempered_probs(lg[rows], T0)
    u = probs_times_embedding(p, V, D)
    W = synthetic.SyntheticWeights(configs.shape_dict(d), seed=0, dtype="bf16", sigma=0.02, cache_experts=False)
    sc_ref = OM.gelu(u @ W["sc_w1"].T) @ W["sc_w2"].T
    assert_close(sc[rows], sc_ref, 2e-2, "self-conditioning vector (sampled rows, V = 262144)")
    del lg, p
    # the block commit, and the committed K/V of deeper layers at sampled positions: each layer's
    # output for those positions from the oracle, teacher-forced on the GPU's cache of that layer
    # (keys 0 .. p, checked at the positions below) and on the GPU's expert choice
    block = st.pred.clone()
    model.commit(block)
    torch.cuda.synchronize()
    assert model.length == w.prompt + C
    routes = gpu_routes(L, model, C)
    ids = block.cpu().numpy().astype(np.int64)
    pick = np.array([0, 77, 190, 255])
    pos = w.prompt + pick
    K, Vc = model.kv_view()
    shape = OM.ModelShape(n_layers=d.n_layers, d_model=D, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                          head_dim=d.head_dim, n_experts=d.n_experts, top_k=d.top_k, d_expert=d.d_expert,
                          d_shared=d.d_shared, gated=True, vocab=V, d_selfcond=d.d_selfcond)
    x = embed_rows(ids[pick], D)
    G = d.n_q_heads // d.n_kv_heads
    hd = d.head_dim
    for l in range(4):
        lw = W["layers"][l]
        h = OM.rms_norm(x, shape.rms_eps)
        k_ref = (h @ lw["wk"].T).reshape(len(pick), d.n_kv_heads, hd)
        v_ref = (h @ lw["wv"].T).reshape(len(pick), d.n_kv_heads, hd)
        p_t = torch.from_numpy(pos).cuda()
        assert_close(to_f64(K[l][:, p_t].permute(1, 0, 2)), k_ref, 2e-2, f"committed K of layer {l}")
        assert_close(to_f64(Vc[l][:, p_t].permute(1, 0, 2)), v_ref, 2e-2, f"committed V of layer {l}")
        if l == 3:
            break
        q = (h @ lw["wq"].T).reshape(len(pick), d.n_q_heads, hd)
        kl = to_f64(K[l][:, :model.length])
        vl = to_f64(Vc[l][:, :model.length])
        o = np.empty((len(pick), d.n_q_heads, hd))
        for i, pp in enumerate(pos):  # causal: keys 0 .. pp
            for j in range(d.n_q_heads):
                sc_ = kl[j // G, :pp + 1] @ q[i, j] / np.sqrt(hd)
                o[i, j] = OM.softmax(sc_) @ vl[j // G, :pp + 1]
        x1 = x + o.reshape(len(pick), -1) @ lw["wo"].T
        h2 = OM.rms_norm(x1, shape.rms_eps)
        r = h2 @ lw["wr"].T
        sel = routes[l][pick]
        check_routes([sel], [{"router_logits": r}], d.top_k, f"commit layer {l}")
        gates = np.take_along_axis(OM.softmax(r), sel, axis=1)
        rows_of = {}
        for i in range(len(pick)):
            for j in range(d.top_k):
                rows_of.setdefault(int(sel[i, j]), []).append(i)
        outs = expert_ffns(W, l, {e: np.array(v) for e, v in rows_of.items()}, h2)
        y = OM.ffn(h2, lw, True, prefix="sh_")
        for i in range(len(pick)):
            for j in range(d.top_k):
                e = int(sel[i, j])
                y[i] += gates[i, j] * outs[e][rows_of[e].index(i)]
        x = x1 + y
    model.close()


def _layer0_kv(ids, d):
    """Layer-0 K and V of tokens `ids` at any positions: they depend only on the token itself
    (RMSNorm of its embedding row times W_k / W_v; no positional encoding)."""
    D, hd, H = d.d_model, d.head_dim, d.n_kv_heads
    idx = (np.asarray(ids, dtype=np.uint64)[:, None] * np.uint64(D) + np.arange(D, dtype=np.uint64)[None, :]).ravel()
    E = synthetic.bf16_bits_to_f32(synthetic.normal_bf16_bits(0, synthetic.TID_EMBED, idx, 0.02))
    h = OM.rms_norm(E.astype(np.float64).reshape(len(ids), D), 1e-6)
    n = H * hd * D
    wk = synthetic.bf16_bits_to_f32(synthetic.normal_bf16_bits(0, synthetic.layer_tid(0, 1), n, 0.02))
    wv = synthetic.bf16_bits_to_f32(synthetic.normal_bf16_bits(0, synthetic.layer_tid(0, 2), n, 0.02))
    k = h @ wk.astype(np.float64).reshape(H * hd, D).T
    v = h @ wv.astype(np.float64).reshape(H * hd, D).T
    return k.reshape(len(ids), H, hd), v.reshape(len(ids), H, hd)


def test_block_ar_full_size(libs):
    """The block-autoregressive configuration at its full size: a 32768-token prompt, then canvases
    of 256 committed one after another until the KV cache (32768 + 9 x 256 positions) is exactly full;
    one more commit is refused. Checked: layer-0 K/V of sampled prompt and committed positions
    (exact function of the token), the committed lengths, the sampler teacher-forced on the last
    canvas's logits (exact), and the capacity error leaving the cache as it was."""
    L, configs, runtime = libs
    w = configs.block_ar_bf16()
    d = w.desc
    d.prefill_rows = 2048  # as bench.py runs it
    C, V = d.canvas, d.vocab
    announce(f"block-AR full size: prompt {w.prompt}, capacity {w.capacity}")
    model = runtime.Model(d, w.capacity, seed=0, sigma=0.02)
    ids = synthetic.uniform_ids(5, synthetic.TID_PROMPT, w.prompt, V)
    model.prefill(torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    assert model.length == w.prompt
    rng = np.random.default_rng(4)
    pos = np.sort(np.concatenate([[0, 1, w.prompt - 1], rng.choice(w.prompt, size=61, replace=False)]))
    k_ref, v_ref = _layer0_kv(ids[pos], d)
    K, Vc = model.kv_view()
    p_t = torch.from_numpy(pos).cuda()
    assert_close(to_f64(K[0][:, p_t].permute(1, 0, 2)), k_ref, 2e-2, "layer-0 K of prompt positions")
    assert_close(to_f64(Vc[0][:, p_t].permute(1, 0, 2)), v_ref, 2e-2, "layer-0 V of prompt positions")
    del K, Vc
    sched = L.make_sched(max_steps=48, seed=0)
    out = torch.empty(C, dtype=torch.int32, device="cuda")
    n_fit = (w.capacity - w.prompt) // C
    committed = []
    for b in range(n_fit):
        steps = model.generate_block(sched, b, out, commit=True)
        torch.cuda.synchronize()
        assert 1 <= steps <= 48
        committed.append(out.cpu().numpy().copy())
        assert model.length == w.prompt + (b + 1) * C
    assert model.length == w.capacity
    # the last canvas's final logits, sampler teacher-forced: exact discrete outputs
    st = runtime.SamplerState(C, V)
    st.init(sched, n_fit - 1)
    st.sample(model.logits, sched, 47, n_fit - 1)
    torch.cuda.synchronize()
    res = OS.sample_step(to_f64(model.logits), 47, n_fit - 1, OS.Schedule(seed=0), None, 0)
    assert np.array_equal(st.pred.cpu().numpy(), res.pred)
    # committed blocks: layer-0 K/V at sampled positions of every block
    K, Vc = model.kv_view()
    for b, blk in enumerate(committed):
        j = np.sort(rng.choice(C, size=8, replace=False))
        k_ref, v_ref = _layer0_kv(blk[j].astype(np.int64), d)
        p_t = torch.from_numpy(w.prompt + b * C + j).cuda()
        assert_close(to_f64(K[0][:, p_t].permute(1, 0, 2)), k_ref, 2e-2, f"layer-0 K of block {b}")
        assert_close(to_f64(Vc[0][:, p_t].permute(1, 0, 2)), v_ref, 2e-2, f"layer-0 V of block {b}")
    del K, Vc
    # the cache is full: the next canvas has no room and nothing changes
    before = model.kv.clone()
    with pytest.raises(L.DGError) as err:
        model.generate_block(sched, n_fit, out, commit=True)
    assert err.value.code == L.DG_ERR_CAPACITY
    torch.cuda.synchronize()
    assert model.length == w.capacity
    assert torch.equal(model.kv, before)
    model.close()


def test_moe_layer_full_size_prefill_chunk(libs):
    """A 2048-row causal chunk at full size (128 experts, ~128 tokens each): routing of 2048 rows and
    the token-tiled expert GEMMs, on sampled rows."""
    L, configs, runtime = libs
    announce("full-size 2048-row causal chunk (token-tiled experts), 1024 cached")
    w = configs.moe_layer_bf16()
    d = w.desc
    d.prefill_rows = 2048
    past, M, D, hd = 1024, 2048, d.d_model, d.head_dim
    model = runtime.Model(d, past + M, seed=0, sigma=0.02)
    kv_n = d.n_kv_heads * past * hd
    kb = synthetic.normal_bf16_bits(3, synthetic.TID_KV_INPUT, kv_n, 1.0).reshape(d.n_kv_heads, past, hd)
    vb = synthetic.normal_bf16_bits(3, synthetic.TID_KV_INPUT + 1, kv_n, 1.0).reshape(d.n_kv_heads, past, hd)
    model.kv_write(0, torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16),
                   torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16), 0)
    L.dg_kv_set_length(model.ctx, past)
    x0 = synthetic.normal_f32(5, synthetic.TID_X_INPUT, M * D, 1.0).reshape(M, D)
    x = torch.from_numpy(x0.copy()).cuda()
    model.forward_layer(0, x, M, True)
    torch.cuda.synchronize()
    W = synthetic.SyntheticWeights(configs.shape_dict(d), seed=0, dtype="bf16", sigma=0.02, cache_experts=False)
    lw = W["layers"][0]
    shape = OM.ModelShape(n_layers=1, d_model=D, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads, head_dim=hd,
                          n_experts=d.n_experts, top_k=d.top_k, d_expert=d.d_expert, d_shared=d.d_shared,
                          gated=True, vocab=d.vocab, d_selfcond=d.d_selfcond)
    xf = x0.astype(np.float64)
    h = OM.rms_norm(xf, shape.rms_eps)
    k = (h @ lw["wk"].T).reshape(M, d.n_kv_heads, hd).transpose(1, 0, 2)
    v = (h @ lw["wv"].T).reshape(M, d.n_kv_heads, hd).transpose(1, 0, 2)
    kc = np.concatenate([synthetic.bf16_bits_to_f32(kb).astype(np.float64), k], axis=1)
    vc = np.concatenate([synthetic.bf16_bits_to_f32(vb).astype(np.float64), v], axis=1)
    rows = np.arange(5, M, 97)
    q = (h[rows] @ lw["wq"].T).reshape(len(rows), d.n_q_heads, hd).transpose(1, 0, 2)
    G = d.n_q_heads // d.n_kv_heads
    o = np.empty((d.n_q_heads, len(rows), hd))
    for j in range(d.n_q_heads):
        for i, r in enumerate(rows):  # causal: keys 0 .. past + r
            s = q[j, i] @ kc[j // G, :past + r + 1].T / np.sqrt(hd)
            o[j, i] = OM.softmax(s) @ vc[j // G, :past + r + 1]
    x1 = xf[rows] + o.transpose(1, 0, 2).reshape(len(rows), -1) @ lw["wo"].T
    h2 = OM.rms_norm(x1, shape.rms_eps)
    r = h2 @ lw["wr"].T
    pick = np.flatnonzero(OM.router_margin(r, d.top_k) > ROUTER_TIE)[:3]
    print(f"rows through the whole layer: {rows[pick].tolist()} ({len(pick)} of {len(rows)} candidates)")
    assert len(pick) == 3
    rows, x1, h2, r = rows[pick], x1[pick], h2[pick], r[pick]
    sel = OM.topk_from_logits(r, d.top_k)
    gates = np.take_along_axis(OM.softmax(r), sel, axis=1)
    y = OM.ffn(h2, lw, True, prefix="sh_")
    for i in range(len(rows)):
        for j in range(d.top_k):
            y[i] += gates[i, j] * OM.ffn(h2[i:i + 1], lw["experts"][int(sel[i, j])], True)[0]
    assert_close(to_f64(x)[rows], x1 + y, 2e-2, "layer output of a 2048-row chunk (sampled rows)")
    model.close()
