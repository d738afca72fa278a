"""Pins of the oracle's attention, MoE, self-conditioning, encoder and step.

Pinned against brute-force loops on tiny shapes (written independently of the
vectorised oracle), closed forms (all keys equal -> mean of V; one key -> V;
top_k = E -> the dense softmax mixture; one-hot / uniform probabilities in
self-conditioning), GeLU's textbook values, and structural identities of the
method (prefill + commit == prefill of the concatenation; bidirectional step is
permutation-equivariant without positional encoding; causal queries ignore
later keys).
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synthetic
from oracle import model as M


def brute_attention(q, k, v, q_pos0, causal):
    Hq, Mq, hd = q.shape
    Hkv, L, _ = k.shape
    out = np.zeros_like(q)
    for j in range(Hq):
        kv = j * Hkv // Hq
        for i in range(Mq):
            scores = []
            for t in range(L):
                if causal and t > q_pos0 + i:
                    continue
                s = 0.0
                for c in range(hd):
                    s += q[j, i, c] * k[kv, t, c]
                scores.append((t, s / math.sqrt(hd)))
            mx = max(s for _, s in scores)
            w = [(t, math.exp(s - mx)) for t, s in scores]
            z = sum(e for _, e in w)
            for t, e in w:
                for c in range(hd):
                    out[j, i, c] += e / z * v[kv, t, c]
    return out


@given(seed=st.integers(0, 10**6), Hkv=st.sampled_from([1, 2]), g=st.sampled_from([1, 2]),
       Mq=st.integers(1, 6), past=st.integers(0, 8), hd=st.sampled_from([1, 4, 8]), causal=st.booleans())
@settings(max_examples=60, deadline=None)
def test_attention_brute_force(seed, Hkv, g, Mq, past, hd, causal):
    rng = np.random.default_rng(seed)
    Hq = Hkv * g
    L = past + Mq
    q = rng.normal(size=(Hq, Mq, hd))
    k = rng.normal(size=(Hkv, L, hd)) * 2
    v = rng.normal(size=(Hkv, L, hd))
    np.testing.assert_allclose(M.attention(q, k, v, past, causal), brute_attention(q, k, v, past, causal),
                               rtol=1e-12, atol=1e-12)


def test_attention_equal_keys_gives_mean_of_values():
    rng = np.random.default_rng(0)
    q = rng.normal(size=(4, 5, 8))
    k = np.repeat(rng.normal(size=(2, 1, 8)), 9, axis=1)
    v = rng.normal(size=(2, 9, 8))
    out = M.attention(q, k, v, 4, causal=False)
    for j in range(4):
        np.testing.assert_allclose(out[j], np.broadcast_to(v[j // 2].mean(axis=0), (5, 8)), atol=1e-13)


def test_attention_single_key_and_causal_first_query():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(2, 3, 4))
    k = rng.normal(size=(2, 3, 4))
    v = rng.normal(size=(2, 3, 4))
    out = M.attention(q[:, :1], k[:, :1], v[:, :1], 0, causal=False)
    np.testing.assert_allclose(out[:, 0], v[:, 0], atol=1e-15)
    out = M.attention(q, k, v, 0, causal=True)
    np.testing.assert_allclose(out[:, 0], v[:, 0], atol=1e-15)  # position 0 sees only key 0
    k2, v2 = k.copy(), v.copy()
    k2[:, 2] += 5.0
    v2[:, 2] -= 3.0
    out2 = M.attention(q, k2, v2, 0, causal=True)
    np.testing.assert_allclose(out2[:, :2], out[:, :2], atol=0)  # later keys are invisible


def test_gelu_textbook_values():
    # x * Phi(x) with Phi the standard normal CDF
    assert M.gelu(np.array(1.0)) == pytest.approx(0.8413447460685429, abs=1e-15)
    assert M.gelu(np.array(-1.0)) == pytest.approx(-0.15865525393145707, abs=1e-15)
    x = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(M.gelu(x) - M.gelu(-x), x, atol=1e-14)
    assert M.gelu(np.array(0.0)) == 0.0


def test_rms_norm_closed_form():
    x = np.array([[3.0, 3.0, 3.0, 3.0], [1.0, -1.0, 1.0, -1.0]])
    y = M.rms_norm(x, 1e-6)
    np.testing.assert_allclose(y[0], 3.0 / math.sqrt(9.0 + 1e-6))
    np.testing.assert_allclose(y[1], x[1] / math.sqrt(1.0 + 1e-6))


TINY = dict(n_layers=2, d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=4, n_experts=6, d_expert=8,
            d_shared=12, gated=1, vocab=40, d_selfcond=10)


def tiny_shape(top_k=2, gated=True, **kw):
    s = dict(TINY, gated=int(gated), **kw)
    return s, M.ModelShape(n_layers=s["n_layers"], d_model=s["d_model"], n_q_heads=s["n_q_heads"],
                           n_kv_heads=s["n_kv_heads"], head_dim=s["head_dim"], n_experts=s["n_experts"],
                           top_k=top_k, d_expert=s["d_expert"], d_shared=s["d_shared"], gated=gated,
                           vocab=s["vocab"], d_selfcond=s["d_selfcond"], canvas=8)


def brute_moe(h, lw, shape):
    E = shape.n_experts
    out = np.zeros_like(h)
    for t in range(h.shape[0]):
        r = [sum(h[t, c] * lw["wr"][e, c] for c in range(h.shape[1])) for e in range(E)]
        mx = max(r)
        z = sum(math.exp(x - mx) for x in r)
        p = [math.exp(x - mx) / z for x in r]
        chosen = []
        for _ in range(shape.top_k):  # repeated selection of the largest, lowest index first
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or r[e] > r[best]:
                    best = e
            chosen.append(best)
        mass = sum(p[e] for e in chosen) if shape.renorm_gates else 1.0
        for e in chosen:
            w = lw["experts"][e]
            out[t] += p[e] / mass * _brute_ffn(h[t], w, shape.gated, "")
        out[t] += _brute_ffn(h[t], lw, shape.gated, "sh_")
    return out


def _brute_ffn(x, w, gated, pre):
    up = w[pre + "up"] @ x
    if gated:
        g = w[pre + "gate"] @ x
        a = np.array([0.5 * gi * (1 + math.erf(gi / math.sqrt(2))) * ui for gi, ui in zip(g, up)])
    else:
        a = np.array([0.5 * ui * (1 + math.erf(ui / math.sqrt(2))) for ui in up])
    return w[pre + "down"] @ a


@pytest.mark.parametrize("gated,top_k", [(True, 2), (False, 2), (True, 1), (True, 6)])
def test_moe_brute_force(gated, top_k):
    s, shape = tiny_shape(top_k=top_k, gated=gated)
    W = synthetic.SyntheticWeights(s, seed=3, dtype="f32", sigma=0.5)
    rng = np.random.default_rng(0)
    h = rng.normal(size=(7, s["d_model"]))
    y, info = M.moe(h, W["layers"][0], shape)
    np.testing.assert_allclose(y, brute_moe(h, W["layers"][0], shape), rtol=1e-10, atol=1e-12)


def test_moe_all_experts_is_dense_softmax_mixture():
    s, shape = tiny_shape(top_k=6)
    W = synthetic.SyntheticWeights(s, seed=4, dtype="f32", sigma=0.5)
    lw = W["layers"][1]
    h = np.random.default_rng(2).normal(size=(5, s["d_model"]))
    p = M.softmax(h @ lw["wr"].T)
    dense = sum(p[:, [e]] * M.ffn(h, lw["experts"][e], True) for e in range(6)) + M.ffn(h, lw, True, "sh_")
    y, _ = M.moe(h, lw, shape)
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-13)


def test_router_dominant_column_and_ties():
    r = np.array([[0.0, 5.0, 5.0, 1.0, 5.0], [100.0, 1.0, 2.0, 3.0, 4.0]])
    sel = M.topk_from_logits(r, 2)
    assert sel[0].tolist() == [1, 2]  # ties: lowest index first
    assert sel[1, 0] == 0
    s, shape = tiny_shape(top_k=1)
    W = synthetic.SyntheticWeights(s, seed=5, dtype="f32", sigma=0.5)
    src = W["layers"][0]
    lw = {k: src[k] for k in ("sh_gate", "sh_up", "sh_down")}
    lw["experts"] = src["experts"]
    hh = np.abs(np.random.default_rng(3).normal(size=(4, s["d_model"])))  # positive rows
    lw["wr"] = np.zeros((6, s["d_model"]))
    lw["wr"][4] = 100.0  # expert 4's logit dominates every row by >= 100
    y, info = M.moe(hh, lw, shape)
    assert (info["sel"][:, 0] == 4).all()
    want = info["gates"][:, [0]] * M.ffn(hh, lw["experts"][4], True) + M.ffn(hh, lw, True, "sh_")
    np.testing.assert_allclose(y, want, rtol=1e-12)


def test_self_conditioning_one_hot_and_uniform():
    s, shape = tiny_shape()
    W = synthetic.SyntheticWeights(s, seed=6, dtype="f32", sigma=0.5)
    V = s["vocab"]
    p = np.zeros((3, V))
    p[0, 7] = 1.0
    p[1, :] = 1.0 / V
    p[2, [1, 2]] = 0.5
    E = W["embed"]
    u_want = np.stack([E[7], E.mean(axis=0), 0.5 * (E[1] + E[2])])
    sc = M.self_condition(W, p)
    want = M.gelu(u_want @ W["sc_w1"].T) @ W["sc_w2"].T
    np.testing.assert_allclose(sc, want, rtol=1e-12, atol=1e-14)


def test_prefill_then_commit_equals_prefill_of_concatenation():
    s, shape = tiny_shape()
    W = synthetic.SyntheticWeights(s, seed=7, dtype="f32", sigma=0.3)
    prompt = synthetic.uniform_ids(1, synthetic.TID_PROMPT, 9, s["vocab"])
    block = synthetic.uniform_ids(2, synthetic.TID_PROMPT, 8, s["vocab"])
    a = M.KVCache.empty(shape, 32)
    M.encode(W, a, prompt, shape)
    M.encode(W, a, block, shape)
    b = M.KVCache.empty(shape, 32)
    M.encode(W, b, np.concatenate([prompt, block]), shape)
    c = M.KVCache.empty(shape, 32)
    for t in np.concatenate([prompt, block]):  # token by token
        M.encode(W, c, [t], shape)
    assert a.length == b.length == c.length == 17
    for l in range(shape.n_layers):
        np.testing.assert_allclose(a.k[l], b.k[l], atol=1e-12)
        np.testing.assert_allclose(a.v[l], b.v[l], atol=1e-12)
        np.testing.assert_allclose(c.k[l], b.k[l], atol=1e-12)


def test_capacity_is_enforced():
    s, shape = tiny_shape()
    W = synthetic.SyntheticWeights(s, seed=7, dtype="f32")
    cache = M.KVCache.empty(shape, 10)
    with pytest.raises(ValueError):
        M.encode(W, cache, np.arange(11) % s["vocab"], shape)
    assert cache.length == 0


def test_denoise_step_is_permutation_equivariant_and_leaves_length():
    s, shape = tiny_shape()
    W = synthetic.SyntheticWeights(s, seed=8, dtype="f32", sigma=0.3)
    cache = M.KVCache.empty(shape, 32)
    M.encode(W, cache, synthetic.uniform_ids(1, synthetic.TID_PROMPT, 5, s["vocab"]), shape)
    canvas = synthetic.uniform_ids(3, synthetic.TID_PROMPT, 8, s["vocab"])
    perm = np.random.default_rng(0).permutation(8)
    l1 = M.denoise_step(W, cache, canvas, None, shape)
    l2 = M.denoise_step(W, cache, canvas[perm], None, shape)
    np.testing.assert_allclose(l2, l1[perm], rtol=1e-10, atol=1e-12)
    assert cache.length == 5


def test_denoise_step_canvas_attends_bidirectionally():
    s, shape = tiny_shape()
    W = synthetic.SyntheticWeights(s, seed=9, dtype="f32", sigma=0.3)
    cache = M.KVCache.empty(shape, 32)
    canvas = synthetic.uniform_ids(4, synthetic.TID_PROMPT, 8, s["vocab"])
    l1 = M.denoise_step(W, cache, canvas, None, shape)
    c2 = canvas.copy()
    c2[-1] = (c2[-1] + 1) % s["vocab"]
    l2 = M.denoise_step(W, cache, c2, None, shape)
    assert np.abs(l1[0] - l2[0]).max() > 1e-9  # the first position sees the last one


# ------------------------------------------------------------------ rotary position embedding
def test_rope_closed_forms():
    x = np.array([[[1.0, 0.0]]])  # hd = 2: one pair, frequency theta^0 = 1
    for p in (0.0, 1.0, 2.5, 1000.0):
        assert np.allclose(M.rope(x, [p], 10000.0)[0, 0], [np.cos(p), np.sin(p)], atol=1e-12)
    rng = np.random.default_rng(0)
    y = rng.normal(size=(3, 5, 8))
    assert np.array_equal(M.rope(y, np.zeros(5), 10000.0), y)  # position 0 is the identity
    # hd = 4: the second pair turns at theta^(-1/2) per position, and pairs are (0, 2) and (1, 3)
    z = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    w = 100.0 ** -0.5 * 3.0
    assert np.allclose(M.rope(z, [3.0], 100.0)[0, 0], [0.0, np.cos(w), 0.0, np.sin(w)], atol=1e-12)


def test_rope_is_a_rotation_and_depends_on_relative_position():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(2, 6, 16))
    k = rng.normal(size=(2, 6, 16))
    pq = rng.integers(0, 5000, 6)
    pk = rng.integers(0, 5000, 6)
    rq = M.rope(q, pq, 10000.0)
    # norms of every (j, j + hd/2) pair are kept
    n0 = q[..., :8] ** 2 + q[..., 8:] ** 2
    n1 = rq[..., :8] ** 2 + rq[..., 8:] ** 2
    assert np.allclose(n0, n1)
    # composition: turning by a then by b is turning by a + b
    assert np.allclose(M.rope(M.rope(q, pq, 500.0), pk, 500.0), M.rope(q, pq + pk, 500.0))
    # scores depend on the positions only through their difference
    s0 = np.einsum("hmd,hmd->hm", rq, M.rope(k, pk, 10000.0))
    s1 = np.einsum("hmd,hmd->hm", M.rope(q, pq + 777, 10000.0), M.rope(k, pk + 777, 10000.0))
    assert np.allclose(s0, s1)


def test_layer_with_rope_rotates_cached_keys_and_queries():
    import dataclasses
    s, shape0 = tiny_shape()
    shape = dataclasses.replace(shape0, rope_theta=10000.0)
    W = synthetic.SyntheticWeights(s, seed=9, dtype="f32", sigma=0.5)
    lw = W["layers"][0]
    rng = np.random.default_rng(4)
    x = rng.normal(size=(5, shape.d_model))
    ck = np.zeros((shape.n_kv_heads, 16, shape.head_dim))
    cv = np.zeros_like(ck)
    M.layer_forward(lw, x, ck, cv, 7, shape, causal=True)
    h = M.rms_norm(x, shape.rms_eps)
    k = (h @ lw["wk"].T).reshape(5, shape.n_kv_heads, shape.head_dim).transpose(1, 0, 2)
    assert np.allclose(ck[:, 7:12], M.rope(k, np.arange(7, 12), 10000.0))
    assert not np.allclose(ck[:, 7:12], k)
    # without rope the same layer stores the plain keys
    ck0 = np.zeros_like(ck)
    M.layer_forward(lw, x, ck0, np.zeros_like(ck), 7, shape0, causal=True)
    assert np.allclose(ck0[:, 7:12], k)


# ------------------------------------------------------------------ the step's wiring, by brute force
# A loops-only statement of one layer, the encoder pass and the denoising step, written without the
# oracle's helpers (rms_norm, layer_forward, lm_head, self_condition, denoise_step): per-element
# loops for the norms and the residual adds, matrix-vector products row by row, the brute-force
# attention and MoE above. It fixes where self-conditioning enters (added to the input embedding,
# before the first norm), the pre-norm placement before attention and before the MoE, both
# residual adds, and the final norm before the tied LM head ([P3] "Encoder-denoiser design",
# "Inference mechanism"; [P4] "Gemma-based MoE backbone"; readings 10 and 12).
def _brute_rms(v, eps):
    ms = sum(float(a) * float(a) for a in v) / len(v)
    return np.array([a / math.sqrt(ms + eps) for a in v])


def _brute_layer(lw, xs, ck, cv, pos0, shape, causal):
    """xs: list of residual rows at positions pos0 ..; writes K/V into ck/cv [Hkv, cap, hd]."""
    hd, Hq, Hkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    Mr = len(xs)
    hs = [_brute_rms(x, shape.rms_eps) for x in xs]
    q = np.zeros((Hq, Mr, hd))
    for i, h in enumerate(hs):
        qv, kv, vv = lw["wq"] @ h, lw["wk"] @ h, lw["wv"] @ h
        for j in range(Hq):
            q[j, i] = qv[j * hd:(j + 1) * hd]
        for j in range(Hkv):
            ck[j, pos0 + i] = kv[j * hd:(j + 1) * hd]
            cv[j, pos0 + i] = vv[j * hd:(j + 1) * hd]
    o = brute_attention(q, ck[:, :pos0 + Mr], cv[:, :pos0 + Mr], pos0, causal)
    out_rows, h2s = [], []
    for i in range(Mr):
        ocat = np.concatenate([o[j, i] for j in range(Hq)])
        proj = lw["wo"] @ ocat
        x1 = np.array([xs[i][c] + proj[c] for c in range(len(xs[i]))])
        h2s.append(_brute_rms(x1, shape.rms_eps))
        out_rows.append(x1)
    y = brute_moe(np.array(h2s), lw, shape)
    return [np.array([out_rows[i][c] + y[i, c] for c in range(len(out_rows[i]))]) for i in range(Mr)]


def _brute_encode(W, ck, cv, length, ids, shape):
    xs = [np.array(W["embed"][int(t)]) for t in ids]
    for l in range(shape.n_layers):
        xs = _brute_layer(W["layers"][l], xs, ck[l], cv[l], length, shape, causal=True)
    return length + len(ids)


def brute_denoise_step(W, ck, cv, length, canvas, sc, shape):
    E = W["embed"]
    xs = []
    for i, t in enumerate(canvas):
        row = np.array(E[int(t)], dtype=np.float64)
        if sc is not None:
            row = np.array([row[c] + sc[i, c] for c in range(len(row))])
        xs.append(row)
    for l in range(shape.n_layers):
        xs = _brute_layer(W["layers"][l], xs, ck[l], cv[l], length, shape, causal=False)
    logits = np.zeros((len(canvas), E.shape[0]))
    for i, x in enumerate(xs):
        hf = _brute_rms(x, shape.rms_eps)
        for v in range(E.shape[0]):
            logits[i, v] = sum(hf[c] * E[v, c] for c in range(len(hf)))
    return logits


def brute_self_condition(W, p):
    """u = sum_v p_v E[v] (loops over the vocabulary), then GeLU(u W1^T) W2^T."""
    E = W["embed"]
    out = np.zeros((p.shape[0], E.shape[1]))
    for i in range(p.shape[0]):
        u = np.zeros(E.shape[1])
        for v in range(E.shape[0]):
            u += p[i, v] * E[v]
        a = W["sc_w1"] @ u
        a = np.array([0.5 * z * (1 + math.erf(z / math.sqrt(2))) for z in a])
        out[i] = W["sc_w2"] @ a
    return out


def _wiring_case(seed=11, rope=0.0, renorm=False, gated=True):
    import dataclasses
    s, shape = tiny_shape(top_k=2, gated=gated)
    shape = dataclasses.replace(shape, canvas=6, renorm_gates=renorm)
    W = synthetic.SyntheticWeights(s, seed=seed, dtype="f32", sigma=0.4)
    prompt = synthetic.uniform_ids(seed, synthetic.TID_PROMPT, 5, s["vocab"])
    canvas = synthetic.uniform_ids(seed + 1, synthetic.TID_PROMPT, 6, s["vocab"])
    sc = np.random.default_rng(seed).normal(size=(6, s["d_model"]))
    return s, shape, W, prompt, canvas, sc


@pytest.mark.parametrize("with_sc", [False, True])
@pytest.mark.parametrize("gated,renorm", [(True, False), (False, False), (True, True)])
def test_denoise_step_matches_brute_force(with_sc, gated, renorm):
    s, shape, W, prompt, canvas, sc = _wiring_case(gated=gated, renorm=renorm)
    sc = sc if with_sc else None
    cache = M.KVCache.empty(shape, 16)
    M.encode(W, cache, prompt, shape)
    ck = [np.zeros((shape.n_kv_heads, 16, shape.head_dim)) for _ in range(shape.n_layers)]
    cv = [np.zeros_like(a) for a in ck]
    n = _brute_encode(W, ck, cv, 0, prompt, shape)
    assert n == cache.length == 5
    for l in range(shape.n_layers):  # encoder pass: same K/V in every layer
        np.testing.assert_allclose(cache.k[l][:, :5], ck[l][:, :5], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(cache.v[l][:, :5], cv[l][:, :5], rtol=1e-10, atol=1e-12)
    got = M.denoise_step(W, cache, canvas, sc, shape)
    want = brute_denoise_step(W, ck, cv, 5, canvas, sc, shape)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_self_condition_matches_brute_force():
    s, shape, W, *_ = _wiring_case()
    rng = np.random.default_rng(3)
    p = rng.random((4, s["vocab"]))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(M.self_condition(W, p), brute_self_condition(W, p), rtol=1e-10, atol=1e-13)


def test_renormalised_gates_are_the_softmax_over_the_chosen_logits():
    """With renormalisation the k gates sum to 1 and equal softmax over the k chosen logits alone
    (softmax restricted to a subset is the full softmax divided by its mass on that subset)."""
    rng = np.random.default_rng(5)
    h = rng.normal(size=(9, 12))
    wr = rng.normal(size=(7, 12))
    r, sel, g = M.route(h, wr, 3, renorm=True)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-14)
    chosen = np.take_along_axis(r, sel, axis=1)
    e = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    np.testing.assert_allclose(g, e / e.sum(axis=1, keepdims=True), rtol=1e-13)
    r0, sel0, g0 = M.route(h, wr, 3, renorm=False)
    assert np.array_equal(sel, sel0) and np.array_equal(r, r0)
    assert (g0.sum(axis=1) < 1.0).all()
    # k = E: the renormalised gates are the plain softmax
    _, _, gall = M.route(h, wr, 7, renorm=True)
    _, sall, pall = M.route(h, wr, 7, renorm=False)
    np.testing.assert_allclose(gall, pall, rtol=1e-13)


def test_forced_routing_is_the_identity_on_the_own_choice():
    """Teacher forcing with the router's own choice changes nothing; forcing other experts takes
    this router's softmax probabilities of those experts as gates."""
    s, shape, W, prompt, canvas, sc = _wiring_case()
    lw = W["layers"][0]
    h = np.random.default_rng(8).normal(size=(5, s["d_model"]))
    y, info = M.moe(h, lw, shape)
    y2, info2 = M.moe(h, lw, shape, forced_sel=info["sel"])
    np.testing.assert_array_equal(y, y2)
    other = (info["sel"] + 1) % shape.n_experts
    _, info3 = M.moe(h, lw, shape, forced_sel=other)
    assert np.array_equal(info3["sel"], other)
    np.testing.assert_allclose(info3["gates"], np.take_along_axis(M.softmax(info["router_logits"]), other, axis=1))


# Plausible wiring mistakes, planted in the oracle (on the CPU): each must make the brute-force
# comparison fail, so the pin above is shown to see them.
def _mut_no_final_norm(monkeypatch):
    monkeypatch.setattr(M, "lm_head", lambda W, x, shape: x @ W["embed"].T)


def _faulty_layer(lw, x, ck, cv, pos0, shape, causal, forced_sel=None, h_extra=None, attn_residual=True,
                  moe_norm=True):
    """The oracle's layer with one of its wiring choices switched: something added to the normalised
    attention input, the attention residual dropped, or the MoE fed the un-normalised residual."""
    Mr = x.shape[0]
    hd, Hq, Hkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    h = M.rms_norm(x, shape.rms_eps)
    if h_extra is not None:
        h = h + h_extra
    q = (h @ lw["wq"].T).reshape(Mr, Hq, hd).transpose(1, 0, 2)
    ck[:, pos0:pos0 + Mr] = (h @ lw["wk"].T).reshape(Mr, Hkv, hd).transpose(1, 0, 2)
    cv[:, pos0:pos0 + Mr] = (h @ lw["wv"].T).reshape(Mr, Hkv, hd).transpose(1, 0, 2)
    o = M.attention(q, ck[:, :pos0 + Mr], cv[:, :pos0 + Mr], pos0, causal).transpose(1, 0, 2).reshape(Mr, -1)
    x = (x if attn_residual else 0.0) + o @ lw["wo"].T
    y, info = M.moe(M.rms_norm(x, shape.rms_eps) if moe_norm else x, lw, shape, forced_sel)
    return x + y, info


def _mut_sc_after_norm(monkeypatch):
    def step(W, cache, canvas, sc, shape, return_info=False, forced_sel=None):
        x = np.asarray(W["embed"])[np.asarray(canvas, dtype=np.int64)]  # sc not added to the embedding
        for l in range(shape.n_layers):
            x, _ = _faulty_layer(W["layers"][l], x, cache.k[l], cache.v[l], cache.length, shape, False,
                                 h_extra=sc if l == 0 else None)  # ... but to the first normalised input
        return M.lm_head(W, x, shape)
    monkeypatch.setattr(M, "denoise_step", step)


def _mut_no_attention_residual(monkeypatch):
    monkeypatch.setattr(M, "layer_forward", lambda *a, **k: _faulty_layer(*a, attn_residual=False, **k))


def _mut_no_moe_norm(monkeypatch):
    monkeypatch.setattr(M, "layer_forward", lambda *a, **k: _faulty_layer(*a, moe_norm=False, **k))


def _mut_gates_renormalised(monkeypatch):
    orig = M.route
    monkeypatch.setattr(M, "route", lambda h, wr, k, renorm=False, forced_sel=None: orig(h, wr, k, True, forced_sel))


def _mut_sc_scaled(monkeypatch):
    orig = M.self_condition
    monkeypatch.setattr(M, "self_condition", lambda W, p: orig(W, p) * 0.5)


def _mut_sc_no_gelu(monkeypatch):
    monkeypatch.setattr(M, "self_condition", lambda W, p: ((p @ W["embed"]) @ W["sc_w1"].T) @ W["sc_w2"].T)


@pytest.mark.parametrize("mutation", [_mut_no_final_norm, _mut_sc_after_norm, _mut_no_attention_residual,
                                      _mut_no_moe_norm, _mut_gates_renormalised])
def test_brute_force_step_catches_planted_wiring_mistakes(monkeypatch, mutation):
    s, shape, W, prompt, canvas, sc = _wiring_case()
    ck = [np.zeros((shape.n_kv_heads, 16, shape.head_dim)) for _ in range(shape.n_layers)]
    cv = [np.zeros_like(a) for a in ck]
    _brute_encode(W, ck, cv, 0, prompt, shape)
    want = brute_denoise_step(W, [a.copy() for a in ck], [a.copy() for a in cv], 5, canvas, sc, shape)
    cache = M.KVCache([a.copy() for a in ck], [a.copy() for a in cv], 5)
    mutation(monkeypatch)
    got = M.denoise_step(W, cache, canvas, sc, shape)
    assert not np.allclose(got, want, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("mutation", [_mut_sc_scaled, _mut_sc_no_gelu])
def test_brute_force_self_condition_catches_planted_mistakes(monkeypatch, mutation):
    s, shape, W, *_ = _wiring_case()
    p = np.random.default_rng(3).random((3, s["vocab"]))
    p /= p.sum(axis=1, keepdims=True)
    want = brute_self_condition(W, p)
    mutation(monkeypatch)
    assert not np.allclose(M.self_condition(W, p), want, rtol=1e-6, atol=1e-8)


def test_faulty_layer_without_a_fault_is_the_oracle_layer():
    s, shape, W, prompt, canvas, sc = _wiring_case()
    lw = W["layers"][1]
    x = np.random.default_rng(2).normal(size=(4, s["d_model"]))
    c1 = [np.zeros((shape.n_kv_heads, 8, shape.head_dim)) for _ in range(2)]
    c2 = [a.copy() for a in c1]
    y1, _ = M.layer_forward(lw, x, c1[0], c1[1], 3, shape, True)
    y2, _ = _faulty_layer(lw, x, c2[0], c2[1], 3, shape, True)
    np.testing.assert_array_equal(y1, y2)
