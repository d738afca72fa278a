"""Denoiser and encoder forward passes, float64, unblocked.

What the pages fix:
* [P3] "Encoder-denoiser design": the model switches between an encoder mode
  (the query is processed the standard, causal way and its key/value cache is
  shared with the denoiser, no cross-attention) and a denoiser mode (causal
  attention becomes bidirectional over the whole noisy canvas and logits are
  produced at every canvas position).
* [P4] "Gemma-based MoE backbone" (table): sparse MoE with 128 experts, 8
  active plus 1 shared; canvas 256 tokens.
* [P4] "From decoder-only to a hybrid structure": the denoising decoder sees
  context on both sides inside the canvas; the KV cache carries the prompt
  and earlier blocks.
* [P3] "Inference mechanism": self-conditioning multiplies the previous
  step's softmax probabilities with the token embeddings and passes the
  probability-weighted representation through a small feed-forward network
  into the next step.
* [P4] "Block Diffusion" / [P3] "Inference mechanism": a finished 256-token
  block is appended to the prompt and the encoder KV cache is extended.

Readings where the pages are silent (parity of these against the real model
is unpinned; they are internal definitions shared with the HIP path and
listed with the project's design notes): pre-norm RMSNorm (unit gain, eps) before attention, before the MoE and before
the LM head; no positional encoding by default (rope_theta = 0), or, as an
option, rotary position embedding of queries and keys at their cache
positions (see rope below); no biases; attention scale 1/sqrt(hd);
GQA query head j reads KV head floor(j * Hkv / Hq); router = softmax over
all experts, top-k chosen on the router logits (lowest index on ties), gate =
the selected softmax probability (not renormalised), shared expert weight 1;
expert FFN gated GeLU (GeLU(h Wg) * (h Wu)) Wd, or plain GeLU(h Wu) Wd when
not gated; GeLU is the exact erf form; tied embedding/LM head;
self-conditioning u = p E with the sampler's tempered p, sc = GeLU(u W1) W2,
added to the next step's input embedding (zero at step 0); the commit
re-encodes the block causally.
All matrices are stored [out_features, in_features], so y = x @ W.T.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf


@dataclass
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    gated: bool
    vocab: int
    d_selfcond: int
    canvas: int = 256
    rms_eps: float = 1e-6
    renorm_gates: bool = False
    rope_theta: float = 0.0


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GeLU, x * Phi(x)."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    z = z - z.max(axis=axis, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=axis, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos0: int, causal: bool) -> np.ndarray:
    """Scaled dot-product attention with grouped KV heads.

    q: [Hq, M, hd] for queries at absolute positions q_pos0 .. q_pos0+M-1;
    k, v: [Hkv, L, hd] for key positions 0 .. L-1. Bidirectional (denoiser
    mode) attends to every key; causal (encoder mode) lets the query at
    position p see keys 0..p.
    """
    Hq, M, hd = q.shape
    Hkv, L, _ = k.shape
    out = np.empty_like(q)
    for j in range(Hq):
        kv = (j * Hkv) // Hq
        s = (q[j] @ k[kv].T) / np.sqrt(hd)
        if causal:
            qpos = q_pos0 + np.arange(M)[:, None]
            s = np.where(np.arange(L)[None, :] <= qpos, s, -np.inf)
        out[j] = softmax(s, axis=-1) @ v[kv]
    return out


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotary position embedding of x [..., M, hd] at the given M positions.

    The pages give no positional scheme; they name a Gemma backbone ([P3]
    "Encoder-denoiser design") with a context of up to 256K tokens ([P4]
    "Gemma-based MoE backbone", table). Reading: the rotary embedding of the
    Gemma family in its "rotate half" form: for j < hd/2 the pair
    (x_j, x_{j+hd/2}) is turned by the angle pos * theta^(-2j/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def ffn(h: np.ndarray, w: dict, gated: bool, prefix: str = "") -> np.ndarray:
    up = h @ w[prefix + "up"].T
    if gated:
        a = gelu(h @ w[prefix + "gate"].T) * up
    else:
        a = gelu(up)
    return a @ w[prefix + "down"].T


def route(h: np.ndarray, wr: np.ndarray, top_k: int, renorm: bool = False, forced_sel=None):
    """Router: logits, selected experts (descending logit, lowest index on ties), gates.

    ``forced_sel`` [M, top_k] (teacher forcing, for comparisons where another
    implementation's rounding legitimately picked a different expert at a
    near-tie): use these experts instead of this router's own choice; the
    gates are still this router's softmax probabilities of them.
    """
    r = h @ wr.T
    if forced_sel is None:
        order = np.argsort(-r, axis=-1, kind="stable")[:, :top_k]
    else:
        order = np.asarray(forced_sel, dtype=np.int64).reshape(r.shape[0], top_k)
    p = softmax(r, axis=-1)
    gates = np.take_along_axis(p, order, axis=-1)
    if renorm:
        gates = gates / gates.sum(axis=-1, keepdims=True)
    return r, order, gates


def topk_from_logits(r: np.ndarray, top_k: int):
    """Top-k expert ids (descending, lowest index on ties) from given router logits."""
    return np.argsort(-np.asarray(r, dtype=np.float64), axis=-1, kind="stable")[:, :top_k]


def moe(h: np.ndarray, lw: dict, shape: ModelShape, forced_sel=None):
    """Sparse MoE FFN: sum over the k selected experts of gate * FFN_e(h), plus the shared expert.

    ``forced_sel``: teacher-forced expert choice (see ``route``)."""
    r, sel, gates = route(h, lw["wr"], shape.top_k, shape.renorm_gates, forced_sel)
    y = np.zeros_like(h)
    for e in np.unique(sel):
        rows, slot = np.nonzero(sel == e)
        y[rows] += gates[rows, slot][:, None] * ffn(h[rows], lw["experts"][int(e)], shape.gated)
    y += ffn(h, lw, shape.gated, prefix="sh_")
    return y, {"router_logits": r, "sel": sel, "gates": gates}


@dataclass
class KVCache:
    """Per-layer keys/values [Hkv, capacity, hd] and the committed length."""
    k: list
    v: list
    length: int = 0

    @classmethod
    def empty(cls, shape: ModelShape, capacity: int) -> "KVCache":
        z = lambda: np.zeros((shape.n_kv_heads, capacity, shape.head_dim))
        return cls([z() for _ in range(shape.n_layers)], [z() for _ in range(shape.n_layers)], 0)

    def copy(self) -> "KVCache":
        return KVCache([a.copy() for a in self.k], [a.copy() for a in self.v], self.length)


def layer_forward(lw: dict, x: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray, pos0: int,
                  shape: ModelShape, causal: bool, forced_sel=None):
    """One transformer layer over M rows placed at positions pos0 .. pos0+M-1.

    The rows' keys/values are written into cache_k/cache_v (modified in place)
    at those positions, and attention reads positions 0 .. pos0+M-1.
    ``forced_sel``: teacher-forced expert choice of the MoE (see ``route``).
    Returns (new x, info dict with the router decisions).
    """
    M = x.shape[0]
    hd, Hq, Hkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    h = rms_norm(x, shape.rms_eps)
    q = (h @ lw["wq"].T).reshape(M, Hq, hd).transpose(1, 0, 2)
    k = (h @ lw["wk"].T).reshape(M, Hkv, hd).transpose(1, 0, 2)
    v = (h @ lw["wv"].T).reshape(M, Hkv, hd).transpose(1, 0, 2)
    if shape.rope_theta > 0:
        pos = pos0 + np.arange(M)
        q = rope(q, pos, shape.rope_theta)
        k = rope(k, pos, shape.rope_theta)
    cache_k[:, pos0:pos0 + M] = k
    cache_v[:, pos0:pos0 + M] = v
    L = pos0 + M
    o = attention(q, cache_k[:, :L], cache_v[:, :L], pos0, causal)
    o = o.transpose(1, 0, 2).reshape(M, Hq * hd)
    x = x + o @ lw["wo"].T
    h2 = rms_norm(x, shape.rms_eps)
    y, info = moe(h2, lw, shape, forced_sel)
    info["h_attn"] = h
    info["h_moe"] = h2
    return x + y, info


def embed(W, ids) -> np.ndarray:
    return np.asarray(W["embed"])[np.asarray(ids, dtype=np.int64)]


def lm_head(W, x: np.ndarray, shape: ModelShape) -> np.ndarray:
    """Logits at every row: final RMSNorm then the tied embedding transposed."""
    return rms_norm(x, shape.rms_eps) @ W["embed"].T


def self_condition(W, probs: np.ndarray) -> np.ndarray:
    """Probability-weighted embedding u = p E, then sc = GeLU(u W1) W2."""
    u = probs @ W["embed"]
    return gelu(u @ W["sc_w1"].T) @ W["sc_w2"].T


def denoise_step(W, cache: KVCache, canvas, sc: np.ndarray | None, shape: ModelShape,
                 return_info: bool = False, forced_sel=None):
    """Denoiser mode: bidirectional pass over the canvas, logits at every position.

    The canvas keys/values go to positions cache.length .. +C as scratch; the
    committed length is not changed. ``forced_sel``: None, or a list with one
    teacher-forced expert choice [C, top_k] (or None) per layer.
    """
    x = embed(W, canvas)
    if sc is not None:
        x = x + sc
    infos = []
    for l in range(shape.n_layers):
        fs = None if forced_sel is None else forced_sel[l]
        x, info = layer_forward(W["layers"][l], x, cache.k[l], cache.v[l], cache.length, shape, causal=False,
                                forced_sel=fs)
        infos.append(info)
    logits = lm_head(W, x, shape)
    return (logits, x, infos) if return_info else logits


def encode(W, cache: KVCache, ids, shape: ModelShape, infos: list | None = None, forced_sel=None) -> None:
    """Encoder mode: causal pass over ``ids`` appended at cache.length; extends the cache.

    Used for the prompt prefill and for committing a finished block. When
    ``infos`` is a list, each layer's router decisions are appended to it.
    ``forced_sel``: as in ``denoise_step``, one entry per layer.
    """
    ids = np.asarray(ids, dtype=np.int64)
    n = len(ids)
    if cache.length + n > cache.k[0].shape[1]:
        raise ValueError("KV capacity exceeded")
    x = embed(W, ids)
    for l in range(shape.n_layers):
        fs = None if forced_sel is None else forced_sel[l]
        x, info = layer_forward(W["layers"][l], x, cache.k[l], cache.v[l], cache.length, shape, causal=True,
                                forced_sel=fs)
        if infos is not None:
            infos.append(info)
    cache.length += n


def router_margin(router_logits: np.ndarray, top_k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest router logit per row (inf when k == E).

    Rows with a small gap are near-ties whose expert choice any rounding can flip.
    """
    r = -np.sort(-np.asarray(router_logits, dtype=np.float64), axis=-1)
    if top_k >= r.shape[-1]:
        return np.full(r.shape[:-1], np.inf)
    return r[..., top_k - 1] - r[..., top_k]
