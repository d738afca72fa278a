"""Helpers shared by the GPU tests (not collected by pytest)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says which one it was."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits_of(t) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
