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
        ("rms_eps", ctypes.c_float), ("renorm_gates", ctypes.c_int32)]


class dg_sched(ctypes.Structure):
    _fields_ = [("max_steps", ctypes.c_int32), ("t_start", ctypes.c_float), ("t_end", ctypes.c_float),
                ("entropy_bound", ctypes.c_float), ("stop_mean_entropy", ctypes.c_float),
                ("stable_needed", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class dg_stop_state(ctypes.Structure):
    _fields_ = [("mean_entropy", ctypes.c_float), ("stable_count", ctypes.c_int32),
                ("stopped", ctypes.c_int32), ("steps_run", ctypes.c_int32)]


assert ctypes.sizeof(dg_sched) == 32 and ctypes.sizeof(dg_stop_state) == 16 and ctypes.sizeof(dg_model_desc) == 64

_P = ctypes.c_void_p
_I32, _I64, _U64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "dg_last_error": (ctypes.c_char_p, []),
    "dg_version": (ctypes.c_char_p, []),
    "dg_temperature": (_F32, [ctypes.POINTER(dg_sched), _I32]),
    "dg_profile_enable": (ctypes.c_int, [_I32, _I32]),
    "dg_profile_report": (ctypes.c_int, [ctypes.c_char_p, _SZ]),
    "dg_sample_workspace_size": (_SZ, [_I32, _I32]),
    "dg_init_canvas": (ctypes.c_int, [ctypes.POINTER(dg_sched), _I32, _I32, _I32, _P, _P, _P]),
    "dg_sample_canvas": (ctypes.c_int, [_P, _I32, _I32, _I32, ctypes.POINTER(dg_sched), _I32, _I32,
                                        _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_synth_normal": (ctypes.c_int, [_U64, _U64, _I64, _F32, _I32, _P, _P]),
    "dg_synth_uniform_ids": (ctypes.c_int, [_U64, _U64, _I64, _I32, _P, _P]),
    "dg_synth_planted_logits": (ctypes.c_int, [_U64, _I32, _I32, _I32, _F32, _F32, _P, _P]),
}

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


def make_sched(max_steps=48, t_start=0.8, t_end=0.4, entropy_bound=0.1, stop_mean_entropy=0.005,
               stable_needed=2, seed=0) -> dg_sched:
    return dg_sched(max_steps, t_start, t_end, entropy_bound, stop_mean_entropy, stable_needed, seed)


# ------------------------------------------------------------------ calls
def dg_last_error() -> str:
    return lib.dg_last_error().decode()


def dg_version() -> str:
    return lib.dg_version().decode()


def dg_temperature(sched: dg_sched, step: int) -> float:
    return lib.dg_temperature(ctypes.byref(sched), step)


def dg_profile_enable(on: bool, max_launches: int = 0):
    return _check("dg_profile_enable", lib.dg_profile_enable(int(on), max_launches))


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


def dg_synth_normal(seed, tid, n, sigma, dtype, d_out, stream=None):
    return _check("dg_synth_normal", lib.dg_synth_normal(seed, tid, n, sigma, dtype, ptr(d_out),
                                                         stream_handle(stream)))


def dg_synth_uniform_ids(seed, tid, n, vocab, d_out, stream=None):
    return _check("dg_synth_uniform_ids", lib.dg_synth_uniform_ids(seed, tid, n, vocab, ptr(d_out),
                                                                   stream_handle(stream)))


def dg_synth_planted_logits(seed, step, rows, vocab, sigma, peak, d_out, stream=None):
    return _check("dg_synth_planted_logits", lib.dg_synth_planted_logits(seed, step, rows, vocab, sigma, peak,
                                                                         ptr(d_out), stream_handle(stream)))
