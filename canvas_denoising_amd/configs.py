"""Model shapes and workloads used by the benchmark and the tests.

The five workloads follow the pages' setting: a 256-token canvas, 8 of 128
experts plus one shared expert ([P4] "Gemma-based MoE backbone", table) and
the recommended sampler settings ([P4] "Standard sampling settings"). Sizes
of the synthetic stand-ins (d_model 2816, 16 query / 8 KV heads of 128, expert
width 704, shared width 2816, vocab 262144) are the benchmark's own choice;
weights are random-init N(0, 0.02)-like, inputs seeded and synthetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import _lib as L


def desc(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, n_experts, top_k, d_expert, d_shared, gated, vocab,
         d_selfcond, dtype, canvas=256, rms_eps=1e-6, renorm_gates=0, rope_theta=0.0,
         prefill_rows=0) -> L.dg_model_desc:
    return L.dg_model_desc(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, n_experts, top_k, d_expert, d_shared,
                           gated, vocab, canvas, d_selfcond, dtype, rms_eps, renorm_gates, rope_theta, prefill_rows)


def shape_dict(d: L.dg_model_desc) -> dict:
    """Shape keys of the seeded weight generator."""
    return dict(n_layers=d.n_layers, d_model=d.d_model, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                head_dim=d.head_dim, n_experts=d.n_experts, d_expert=d.d_expert, d_shared=d.d_shared,
                gated=d.gated, vocab=d.vocab, d_selfcond=d.d_selfcond)


@dataclass
class Workload:
    name: str
    desc: L.dg_model_desc
    prompt: int = 0
    blocks: int = 1
    max_steps: int = 48
    capacity: int = 0
    notes: str = ""


def tiny_f32() -> Workload:
    """1 layer, d 256, 4 x 64 heads, 16 experts top-2 (FFN 512, GeLU) + shared 512, vocab 4096, fp32."""
    d = desc(1, 256, 4, 4, 64, 16, 2, 512, 512, 0, 4096, 256, L.DG_F32)
    return Workload("tiny-fp32", d, prompt=64, blocks=1, max_steps=8, capacity=64 + 2 * 256)


def moe_layer_bf16() -> Workload:
    """One MoE denoiser layer: d 2816, 16q/8kv x 128, 128 experts top-8 (704, gated) + shared 2816."""
    d = desc(1, 2816, 16, 8, 128, 128, 8, 704, 2816, 1, 256, 256, L.DG_BF16)
    return Workload("moe-layer-bf16", d, prompt=4096, capacity=4096 + 256)


def full_loop_bf16(n_layers: int = 30) -> Workload:
    """30 layers of the MoE layer, tied vocab 262144, self-conditioning FFN 2816, prompt 8192."""
    d = desc(n_layers, 2816, 16, 8, 128, 128, 8, 704, 2816, 1, 262144, 2816, L.DG_BF16)
    return Workload("full-loop-bf16", d, prompt=8192, blocks=1, max_steps=48, capacity=8192 + 2 * 256)


def block_ar_bf16() -> Workload:
    """Same model, prompt 32768, 8 canvases of 256 committed block by block."""
    w = full_loop_bf16()
    return Workload("block-ar-bf16", w.desc, prompt=32768, blocks=8, max_steps=48, capacity=32768 + 8 * 256 + 256)
