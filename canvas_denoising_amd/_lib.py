"""ctypes binding of libdg (include/dg.h): argument marshalling only.

Every function keeps the C name and argument order. Device buffers may be
passed as torch tensors (their data_ptr is used) or as raw integer
addresses; ``stream=None`` means torch's current HIP stream when torch has a
GPU, else the default stream. A non-zero status raises DGError with the
library's message. Importing this module fails loudly when libdg.so has not
been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

DG_OK, DG_ERR_INVALID, DG_ERR_SHAPE, DG_ERR_CAPACITY, DG_ERR_UNSUPPORTED, DG_ERR_HIP = 0, -1, -2, -3, -4, -5
DG_BF16, DG_F32 = 0, 1


class DGError(RuntimeError):
    def __init__(self, name: str, code: int, msg: str):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m canvas_denoising_amd.build`")
lib = ctypes.CDLL(LIB_PATH)


class dg_model_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k", "d_expert",
        "d_shared", "gated", "vocab", "canvas", "d_selfcond", "dtype")] + [
        ("rms_eps", ctypes.c_float), ("renorm_gates", ctypes.c_int32), ("rope_theta", ctypes.c_float),
        ("prefill_rows", ctypes.c_int32)]


class dg_sched(ctypes.Structure):
    _fields_ = [("max_steps", ctypes.c_int32), ("t_start", ctypes.c_float), ("t_end", ctypes.c_float),
                ("entropy_bound", ctypes.c_float), ("stop_mean_entropy", ctypes.c_float),
                ("stable_needed", ctypes.c_int32), ("seed", ctypes.c_uint64), ("mode", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class dg_stop_state(ctypes.Structure):
    _fields_ = [("mean_entropy", ctypes.c_float), ("stable_count", ctypes.c_int32),
                ("stopped", ctypes.c_int32), ("steps_run", ctypes.c_int32)]


assert ctypes.sizeof(dg_sched) == 40 and ctypes.sizeof(dg_stop_state) == 16 and ctypes.sizeof(dg_model_desc) == 72

_P = ctypes.c_void_p
_I32, _I64, _U64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "dg_last_error": (ctypes.c_char_p, []),
    "dg_version": (ctypes.c_char_p, []),
    "dg_temperature": (_F32, [ctypes.POINTER(dg_sched), _I32]),
    "dg_profile_enable": (ctypes.c_int, [_I32, _I32]),
    "dg_profile_only": (ctypes.c_int, [ctypes.c_char_p]),
    "dg_profile_report": (ctypes.c_int, [ctypes.c_char_p, _SZ]),
    "dg_sample_workspace_size": (_SZ, [_I32, _I32]),
    "dg_init_canvas": (ctypes.c_int, [ctypes.POINTER(dg_sched), _I32, _I32, _I32, _P, _P, _P]),
    "dg_sample_canvas": (ctypes.c_int, [_P, _I32, _I32, _I32, ctypes.POINTER(dg_sched), _I32, _I32,
                                        _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_sample_canvas_static": (ctypes.c_int, [_P, _I32, _I32, _I32, ctypes.POINTER(dg_sched), _I32, _I32,
                                               _P, _P, _P, _P, _P, _P, _P]),
    "dg_synth_normal": (ctypes.c_int, [_U64, _U64, _I64, _F32, _I32, _P, _P]),
    "dg_synth_uniform_ids": (ctypes.c_int, [_U64, _U64, _I64, _I32, _P, _P]),
    "dg_stream_read": (ctypes.c_int, [_P, _I64, _P, _I32, _P]),
    "dg_synth_planted_logits": (ctypes.c_int, [_U64, _I32, _I32, _I32, _F32, _F32, _P, _P]),
    "dg_synth_fill_weights": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _U64, _F32, _P, _P]),
    "dg_weights_bytes": (_SZ, [ctypes.POINTER(dg_model_desc)]),
    "dg_weight_tensor": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _I32, _I32, _I32, ctypes.POINTER(_SZ),
                                        ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "dg_load_weight": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _I32, _I32, _I32, _P, _P, _P]),
    "dg_prepare_weights": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _P, _P]),
    "dg_expert_fp8_bytes": (_SZ, [ctypes.POINTER(dg_model_desc)]),
    "dg_expert_fp8_tensor": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _I32, _I32, _I32, ctypes.POINTER(_SZ),
                                            ctypes.POINTER(_SZ)]),
    "dg_quantize_experts_fp8": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _P, _P, _P]),
    "dg_kv_bytes": (_SZ, [ctypes.POINTER(dg_model_desc), _I64]),
    "dg_workspace_size": (_SZ, [ctypes.POINTER(dg_model_desc), _I64]),
    "dg_ctx_create": (ctypes.c_int, [ctypes.POINTER(dg_model_desc), _P, _P, _I64, _P, _SZ, ctypes.POINTER(_P)]),
    "dg_ctx_destroy": (ctypes.c_int, [_P]),
    "dg_ctx_use_graphs": (ctypes.c_int, [_P, _I32]),
    "dg_ctx_set_weights": (ctypes.c_int, [_P, _P]),
    "dg_ctx_use_expert_fp8": (ctypes.c_int, [_P, _P]),
    "dg_ctx_fuse_sampler_stats": (ctypes.c_int, [_P, ctypes.POINTER(dg_sched)]),
    "dg_sample_canvas_fused": (ctypes.c_int, [_P, ctypes.POINTER(dg_sched), _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                              _SZ, _P]),
    "dg_kv_length": (_I64, [_P]),
    "dg_ctx_graph_captures": (_I64, [_P]),
    "dg_kv_set_length": (ctypes.c_int, [_P, _I64]),
    "dg_prefill_kv": (ctypes.c_int, [_P, _P, _I32, _P]),
    "dg_denoise_step": (ctypes.c_int, [_P, _P, _I32, _P, _P, _F32, _P, _P]),
    "dg_commit_block": (ctypes.c_int, [_P, _P, _P]),
    "dg_forward_layer": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P]),
    "dg_generate_block": (ctypes.c_int, [_P, ctypes.POINTER(dg_sched), _I32, _P, _P, _I32, ctypes.POINTER(_I32), _P]),
    "dg_ctx_buffer": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_SZ)]),
}

# weight kinds / context buffers (include/dg.h)
(DG_W_EMBED, DG_W_EMBED_T, DG_W_SC1, DG_W_SC2, DG_W_Q, DG_W_K, DG_W_V, DG_W_O, DG_W_ROUTER, DG_W_SH_GATE,
 DG_W_SH_UP, DG_W_SH_DOWN, DG_W_EX_GATE, DG_W_EX_UP, DG_W_EX_DOWN) = range(15)
(DG_BUF_X, DG_BUF_H, DG_BUF_ROUTER_LOGITS, DG_BUF_SEL, DG_BUF_GATE, DG_BUF_SC, DG_BUF_CANVAS, DG_BUF_PRED,
 DG_BUF_STOP, DG_BUF_ENTROPY, DG_BUF_ROW_STATS, DG_BUF_ACCEPT, DG_BUF_Q, DG_BUF_ATTN, DG_BUF_SHARED_ACT,
 DG_BUF_SLOT_OUT, DG_BUF_SLOT_OF, DG_BUF_SEL_LAYERS, DG_BUF_OFFSETS) = range(19)

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def ptr(x):
    """Device address of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def stream_handle(stream=None):
    if stream is not None:
        return stream if isinstance(stream, int) else getattr(stream, "cuda_stream", stream)
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except Exception:  # pragma: no cover - torch without HIP
        pass
    return None


def _check(name: str, rc: int) -> int:
    if rc != DG_OK:
        raise DGError(name, rc, dg_last_error())
    return rc


DG_SCHED_STOP_EITHER, DG_SCHED_ACCEPT_GROUP, DG_SCHED_SAMPLE = 1, 2, 4


def make_sched(max_steps=48, t_start=0.8, t_end=0.4, entropy_bound=0.1, stop_mean_entropy=0.005,
               stable_needed=2, seed=0, mode=0) -> dg_sched:
    return dg_sched(max_steps, t_start, t_end, entropy_bound, stop_mean_entropy, stable_needed, seed, mode, 0)


# ------------------------------------------------------------------ calls
def dg_last_error() -> str:
    return lib.dg_last_error().decode()


def dg_version() -> str:
    return lib.dg_version().decode()


def dg_temperature(sched: dg_sched, step: int) -> float:
    return lib.dg_temperature(ctypes.byref(sched), step)


def dg_profile_enable(on: bool, max_launches: int = 0):
    return _check("dg_profile_enable", lib.dg_profile_enable(int(on), max_launches))


def dg_profile_only(name=None):
    return _check("dg_profile_only", lib.dg_profile_only(name.encode() if name else None))


def dg_profile_report() -> dict:
    import json
    buf = ctypes.create_string_buffer(1 << 16)
    _check("dg_profile_report", lib.dg_profile_report(buf, len(buf)))
    return json.loads(buf.value.decode())


def dg_sample_workspace_size(rows: int, vocab: int) -> int:
    return lib.dg_sample_workspace_size(rows, vocab)


def dg_init_canvas(sched, block, canvas, vocab, d_canvas, d_stop, stream=None):
    return _check("dg_init_canvas", lib.dg_init_canvas(ctypes.byref(sched), block, canvas, vocab, ptr(d_canvas),
                                                       ptr(d_stop), stream_handle(stream)))


def dg_sample_canvas(d_logits, dtype, rows, vocab, sched, step, block, d_canvas, d_pred, d_accept, d_entropy,
                     d_row_stats, d_stop, d_workspace, ws_bytes, stream=None):
    return _check("dg_sample_canvas", lib.dg_sample_canvas(
        ptr(d_logits), dtype, rows, vocab, ctypes.byref(sched), step, block, ptr(d_canvas), ptr(d_pred),
        ptr(d_accept), ptr(d_entropy), ptr(d_row_stats), ptr(d_stop), ptr(d_workspace), ws_bytes,
        stream_handle(stream)))


def dg_sample_canvas_static(d_logits, dtype, rows, vocab, sched, step, block, d_canvas, d_pred, d_accept, d_entropy,
                            d_row_stats, d_stop, stream=None):
    return _check("dg_sample_canvas_static", lib.dg_sample_canvas_static(
        ptr(d_logits), dtype, rows, vocab, ctypes.byref(sched), step, block, ptr(d_canvas), ptr(d_pred),
        ptr(d_accept), ptr(d_entropy), ptr(d_row_stats), ptr(d_stop), stream_handle(stream)))


def dg_synth_normal(seed, tid, n, sigma, dtype, d_out, stream=None):
    return _check("dg_synth_normal", lib.dg_synth_normal(seed, tid, n, sigma, dtype, ptr(d_out),
                                                         stream_handle(stream)))


def dg_synth_uniform_ids(seed, tid, n, vocab, d_out, stream=None):
    return _check("dg_synth_uniform_ids", lib.dg_synth_uniform_ids(seed, tid, n, vocab, ptr(d_out),
                                                                   stream_handle(stream)))


def dg_stream_read(d_src, nbytes, d_sink, blocks, stream=None):
    return _check("dg_stream_read", lib.dg_stream_read(ptr(d_src), nbytes, ptr(d_sink), blocks, stream_handle(stream)))


def dg_synth_planted_logits(seed, step, rows, vocab, sigma, peak, d_out, stream=None):
    return _check("dg_synth_planted_logits", lib.dg_synth_planted_logits(seed, step, rows, vocab, sigma, peak,
                                                                         ptr(d_out), stream_handle(stream)))


def dg_synth_fill_weights(desc, seed, sigma, d_weights, stream=None):
    return _check("dg_synth_fill_weights", lib.dg_synth_fill_weights(ctypes.byref(desc), seed, sigma, ptr(d_weights),
                                                                     stream_handle(stream)))


def dg_weights_bytes(desc) -> int:
    return lib.dg_weights_bytes(ctypes.byref(desc))


def dg_weight_tensor(desc, kind, layer=0, expert=0):
    """(byte offset, rows, cols) of one tensor in the packed weight buffer."""
    off, r, c = _SZ(), _I64(), _I64()
    _check("dg_weight_tensor", lib.dg_weight_tensor(ctypes.byref(desc), kind, layer, expert, ctypes.byref(off),
                                                    ctypes.byref(r), ctypes.byref(c)))
    return off.value, r.value, c.value


def dg_load_weight(desc, kind, layer, expert, d_src, d_weights, stream=None):
    return _check("dg_load_weight", lib.dg_load_weight(ctypes.byref(desc), kind, layer, expert, ptr(d_src),
                                                       ptr(d_weights), stream_handle(stream)))


def dg_prepare_weights(desc, d_weights, stream=None):
    return _check("dg_prepare_weights", lib.dg_prepare_weights(ctypes.byref(desc), ptr(d_weights),
                                                               stream_handle(stream)))


def dg_expert_fp8_bytes(desc) -> int:
    return lib.dg_expert_fp8_bytes(ctypes.byref(desc))


def dg_expert_fp8_tensor(desc, kind, layer=0, expert=0):
    """(code byte offset, scale byte offset) of one routed-expert matrix in the FP8 expert buffer."""
    code, scale = _SZ(), _SZ()
    _check("dg_expert_fp8_tensor", lib.dg_expert_fp8_tensor(ctypes.byref(desc), kind, layer, expert,
                                                            ctypes.byref(code), ctypes.byref(scale)))
    return code.value, scale.value


def dg_quantize_experts_fp8(desc, d_weights, d_fp8, stream=None):
    return _check("dg_quantize_experts_fp8", lib.dg_quantize_experts_fp8(ctypes.byref(desc), ptr(d_weights),
                                                                         ptr(d_fp8), stream_handle(stream)))


def dg_kv_bytes(desc, capacity) -> int:
    return lib.dg_kv_bytes(ctypes.byref(desc), capacity)


def dg_workspace_size(desc, capacity) -> int:
    return lib.dg_workspace_size(ctypes.byref(desc), capacity)


def dg_ctx_create(desc, d_weights, d_kv, capacity, d_workspace, ws_bytes) -> int:
    out = _P()
    _check("dg_ctx_create", lib.dg_ctx_create(ctypes.byref(desc), ptr(d_weights), ptr(d_kv), capacity,
                                              ptr(d_workspace), ws_bytes, ctypes.byref(out)))
    return out.value


def dg_ctx_destroy(ctx):
    return _check("dg_ctx_destroy", lib.dg_ctx_destroy(ctx))


def dg_ctx_use_graphs(ctx, on: bool):
    return _check("dg_ctx_use_graphs", lib.dg_ctx_use_graphs(ctx, int(on)))


def dg_ctx_set_weights(ctx, d_weights):
    return _check("dg_ctx_set_weights", lib.dg_ctx_set_weights(ctx, ptr(d_weights)))


def dg_ctx_use_expert_fp8(ctx, d_fp8):
    return _check("dg_ctx_use_expert_fp8", lib.dg_ctx_use_expert_fp8(ctx, ptr(d_fp8)))


def dg_ctx_fuse_sampler_stats(ctx, sched):
    """sched: a dg_sched (the LM head then also produces the sampler's records at its temperatures), or None."""
    return _check("dg_ctx_fuse_sampler_stats",
                  lib.dg_ctx_fuse_sampler_stats(ctx, ctypes.byref(sched) if sched is not None else None))


def dg_sample_canvas_fused(ctx, sched, step, block, d_canvas, d_pred, d_accept, d_entropy, d_row_stats, d_stop,
                           d_workspace, ws_bytes, stream=None):
    return _check("dg_sample_canvas_fused", lib.dg_sample_canvas_fused(
        ctx, ctypes.byref(sched), step, block, ptr(d_canvas), ptr(d_pred), ptr(d_accept), ptr(d_entropy),
        ptr(d_row_stats), ptr(d_stop), ptr(d_workspace), ws_bytes, stream_handle(stream)))


def dg_kv_length(ctx) -> int:
    return lib.dg_kv_length(ctx)


def dg_ctx_graph_captures(ctx) -> int:
    return lib.dg_ctx_graph_captures(ctx)


def dg_kv_set_length(ctx, length):
    return _check("dg_kv_set_length", lib.dg_kv_set_length(ctx, length))


def dg_prefill_kv(ctx, d_prompt_ids, n_prompt, stream=None):
    return _check("dg_prefill_kv", lib.dg_prefill_kv(ctx, ptr(d_prompt_ids), n_prompt, stream_handle(stream)))


def dg_denoise_step(ctx, d_canvas, step, d_prev_logits, d_prev_row_stats, prev_temperature, d_logits, stream=None):
    return _check("dg_denoise_step", lib.dg_denoise_step(ctx, ptr(d_canvas), step, ptr(d_prev_logits),
                                                         ptr(d_prev_row_stats), prev_temperature, ptr(d_logits),
                                                         stream_handle(stream)))


def dg_commit_block(ctx, d_block_ids, stream=None):
    return _check("dg_commit_block", lib.dg_commit_block(ctx, ptr(d_block_ids), stream_handle(stream)))


def dg_forward_layer(ctx, layer, d_x, rows, causal, stream=None):
    return _check("dg_forward_layer", lib.dg_forward_layer(ctx, layer, ptr(d_x), rows, int(causal),
                                                           stream_handle(stream)))


def dg_generate_block(ctx, sched, block, d_logits, d_block_out, commit=True, stream=None) -> int:
    steps = _I32()
    _check("dg_generate_block", lib.dg_generate_block(ctx, ctypes.byref(sched), block, ptr(d_logits),
                                                      ptr(d_block_out), int(commit), ctypes.byref(steps),
                                                      stream_handle(stream)))
    return steps.value


def dg_ctx_buffer(ctx, which):
    """(device address, bytes) of a context buffer."""
    p, n = _P(), _SZ()
    _check("dg_ctx_buffer", lib.dg_ctx_buffer(ctx, which, ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value
