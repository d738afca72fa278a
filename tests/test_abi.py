"""The C ABI on the CPU: every symbol include/dg.h declares is exported, and
argument validation rejects bad calls before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from canvas_denoising_amd import _lib
    return _lib


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L.lib, n), n
        assert n in L._SIGS, f"{n} has no ctypes signature"


def test_temperature_matches_pages_schedule(L):
    s = L.make_sched()
    assert L.dg_temperature(s, 0) == np.float32(0.8)
    assert L.dg_temperature(s, 47) == np.float32(0.4)
    assert np.isnan(L.lib.dg_temperature(None, 0))


def test_sampler_validation_errors(L):
    s = L.make_sched()
    fake = 1 << 20  # never dereferenced: validation fails first
    cases = [
        (dict(d_logits=None), L.DG_ERR_INVALID),
        (dict(rows=0), L.DG_ERR_SHAPE),
        (dict(vocab=0), L.DG_ERR_SHAPE),
        (dict(dtype=7), L.DG_ERR_INVALID),
        (dict(step=48), L.DG_ERR_INVALID),
        (dict(step=-1), L.DG_ERR_INVALID),
        (dict(ws_bytes=16), L.DG_ERR_CAPACITY),
        (dict(d_logits=fake + 2), L.DG_ERR_INVALID),
        (dict(d_workspace=fake + 16), L.DG_ERR_INVALID),
        (dict(d_stop=None), L.DG_ERR_INVALID),
    ]
    for over, code in cases:
        a = dict(d_logits=fake, dtype=0, rows=256, vocab=262144, step=0, ws_bytes=1 << 20, d_stop=fake,
                 d_workspace=fake)
        a.update(over)
        with pytest.raises(L.DGError) as ei:
            L.dg_sample_canvas(a["d_logits"], a["dtype"], a["rows"], a["vocab"], s, a["step"], 0, fake, fake,
                               None, None, None, a["d_stop"], a["d_workspace"], a["ws_bytes"])
        assert ei.value.code == code, (over, ei.value)


def test_sched_validation(L):
    for bad in (dict(max_steps=0), dict(t_start=0.0), dict(t_end=float("nan")), dict(stable_needed=-1)):
        s = L.make_sched(**bad)
        with pytest.raises(L.DGError) as ei:
            L.dg_init_canvas(s, 0, 256, 4096, 1 << 20, None)
        assert ei.value.code == L.DG_ERR_INVALID


def test_workspace_size(L):
    assert L.dg_sample_workspace_size(0, 10) == 0
    assert L.dg_sample_workspace_size(256, 262144) >= 256 * 16
    assert 16 <= L.dg_sample_workspace_size(1, 1) <= 4096


def test_fp8_expert_buffer_layout_and_validation(L):
    from canvas_denoising_amd import configs
    d = configs.full_loop_bf16().desc
    E, F, D, nl = d.n_experts, d.d_expert, d.d_model, d.n_layers
    per_layer = 3 * E * F * D + 4 * E * (2 * F + D)  # codes, then scales; every part a multiple of 256 here
    assert L.dg_expert_fp8_bytes(d) == nl * per_layer
    assert L.dg_expert_fp8_bytes(configs.desc(1, 256, 4, 2, 64, 8, 2, 128, 256, 1, 512, 128, L.DG_F32)) == 0
    assert L.dg_expert_fp8_bytes(configs.desc(1, 256, 4, 2, 64, 8, 2, 96, 256, 1, 512, 128, L.DG_BF16)) == 0
    gate = L.dg_expert_fp8_tensor(d, L.DG_W_EX_GATE, 1, 5)
    up = L.dg_expert_fp8_tensor(d, L.DG_W_EX_UP, 1, 5)
    down = L.dg_expert_fp8_tensor(d, L.DG_W_EX_DOWN, 1, 5)
    assert gate[0] == up[0] == per_layer + 5 * 2 * F * D  # gate and up share the expert's region
    assert up[1] - gate[1] == 4 * F
    assert down[0] == per_layer + 2 * E * F * D + 5 * D * F
    assert down[1] == per_layer + 3 * E * F * D + 4 * E * 2 * F + 4 * 5 * D
    for bad in [(L.DG_W_Q, 0, 0), (L.DG_W_EX_UP, nl, 0), (L.DG_W_EX_UP, 0, E)]:
        with pytest.raises(L.DGError):
            L.dg_expert_fp8_tensor(d, *bad)
    with pytest.raises(L.DGError):
        L.dg_quantize_experts_fp8(d, None, None)
    with pytest.raises(L.DGError):
        L.dg_ctx_use_expert_fp8(None, None)


def test_prefill_rows_and_rope_validation(L):
    from canvas_denoising_amd import configs
    base = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, n_experts=8, top_k=2, d_expert=128,
                d_shared=256, gated=1, vocab=512, d_selfcond=128, dtype=L.DG_BF16)

    def mk(**kw):
        a = dict(base, **kw)
        return configs.desc(a["n_layers"], a["d_model"], a["n_q_heads"], a["n_kv_heads"], a["head_dim"],
                            a["n_experts"], a["top_k"], a["d_expert"], a["d_shared"], a["gated"], a["vocab"],
                            a["d_selfcond"], a["dtype"], canvas=64, rope_theta=a.get("rope", 0.0),
                            prefill_rows=a.get("prefill_rows", 0))
    ws0 = L.dg_workspace_size(mk(), 4096)
    assert ws0 > 0
    ws1 = L.dg_workspace_size(mk(prefill_rows=1024), 4096)
    assert ws1 > ws0  # activations, routing tables and expert buffers grow with the chunk
    assert L.dg_workspace_size(mk(prefill_rows=32), 4096) == 0      # below the canvas
    assert L.dg_workspace_size(mk(prefill_rows=5000), 8192) == 0    # above 4096
    assert L.dg_workspace_size(mk(prefill_rows=1024, n_experts=192), 4096) == 0  # > 256 rows needs E <= 128
    assert L.dg_workspace_size(mk(prefill_rows=256, n_experts=192), 4096) > 0
    # the rotary table is one (cos, sin) pair per cache position and frequency
    assert L.dg_workspace_size(mk(rope=10000.0), 4096) - ws0 >= 4096 * 32 * 8
    assert L.dg_workspace_size(mk(rope=-1.0), 4096) == 0


@pytest.mark.parametrize("hd,dtype,es", [(128, 0, 2), (64, 0, 2), (64, 1, 4)])
def test_kv_bytes_carry_the_documented_tail(L, hd, dtype, es):
    """dg_kv_bytes = K and V of every layer and head, plus the tail dg.h documents: the attention
    kernel's largest key stage (128) minus one V block (32) = 96 head_dim-wide positions."""
    from canvas_denoising_amd import configs
    d = configs.desc(3, 256, 4, 2, hd, 8, 2, 128, 256, 1, 512, 128, dtype, canvas=64)
    for cap in (64, 224, 4096):
        assert L.dg_kv_bytes(d, cap) - 2 * 3 * 2 * cap * hd * es == 96 * hd * es
