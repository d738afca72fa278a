"""Device-buffer plumbing around libdg, using torch for memory and streams.

Nothing here computes a step of the method: every call goes through libdg.
"""
from __future__ import annotations

import torch

from . import _lib as L


def torch_dtype(dg_dtype: int) -> torch.dtype:
    return torch.bfloat16 if dg_dtype == L.DG_BF16 else torch.float32


class SamplerState:
    """Buffers for dg_sample_canvas on one canvas: canvas, argmax, accept mask,
    entropies, row statistics, the 16-byte stop state and the sampler scratch."""

    def __init__(self, rows: int, vocab: int, device="cuda"):
        self.rows, self.vocab = rows, vocab
        self.canvas = torch.zeros(rows, dtype=torch.int32, device=device)
        self.pred = torch.full((rows,), -1, dtype=torch.int32, device=device)
        self.accept = torch.zeros(rows, dtype=torch.uint8, device=device)
        self.entropy = torch.zeros(rows, dtype=torch.float32, device=device)
        self.row_stats = torch.zeros(rows, 2, dtype=torch.float32, device=device)
        self.stop = torch.zeros(4, dtype=torch.int32, device=device)  # dg_stop_state
        self.ws_bytes = max(256, L.dg_sample_workspace_size(rows, vocab))
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def init(self, sched, block: int, stream=None):
        L.dg_init_canvas(sched, block, self.rows, self.vocab, self.canvas, self.stop, stream)

    def sample(self, logits: torch.Tensor, sched, step: int, block: int, stream=None):
        dt = L.DG_BF16 if logits.dtype == torch.bfloat16 else L.DG_F32
        L.dg_sample_canvas(logits, dt, self.rows, self.vocab, sched, step, block, self.canvas, self.pred,
                           self.accept, self.entropy, self.row_stats, self.stop, self.workspace, self.ws_bytes,
                           stream)

    def stop_state(self) -> dict:
        s = self.stop.cpu()
        return {"mean_entropy": s[0:1].view(torch.float32).item(), "stable_count": int(s[1]),
                "stopped": int(s[2]), "steps_run": int(s[3])}
