"""Device-buffer plumbing around libdg, using torch for memory and streams.

Nothing here computes a step of the method: every call goes through libdg.
"""
from __future__ import annotations

import torch

from . import _lib as L


def torch_dtype(dg_dtype: int) -> torch.dtype:
    return torch.bfloat16 if dg_dtype == L.DG_BF16 else torch.float32



# slot of position p % 32 inside a V cache block (include/dg.h)
V_SLOT_OF_POS = [((p & 15) >> 2) * 8 + (p >> 4) * 4 + (p & 3) for p in range(32)]

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
        self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)  # counters start at zero

    def init(self, sched, block: int, stream=None):
        L.dg_init_canvas(sched, block, self.rows, self.vocab, self.canvas, self.stop, stream)

    def sample(self, logits: torch.Tensor, sched, step: int, block: int, stream=None):
        dt = L.DG_BF16 if logits.dtype == torch.bfloat16 else L.DG_F32
        if not hasattr(self, "_ptrs"):  # device addresses never change: marshal them once
            self._ptrs = tuple(t.data_ptr() for t in (self.canvas, self.pred, self.accept, self.entropy,
                                                      self.row_stats, self.stop, self.workspace))
        L.dg_sample_canvas(logits.data_ptr(), dt, self.rows, self.vocab, sched, step, block, *self._ptrs,
                           self.ws_bytes, stream)

    def sample_fused(self, ctx, sched, step: int, block: int, stream=None):
        """dg_sample_canvas_fused: the same outputs, from the records the context's LM head made."""
        if not hasattr(self, "_ptrs"):
            self._ptrs = tuple(t.data_ptr() for t in (self.canvas, self.pred, self.accept, self.entropy,
                                                      self.row_stats, self.stop, self.workspace))
        L.dg_sample_canvas_fused(ctx, sched, step, block, *self._ptrs, self.ws_bytes, stream)

    def stop_state(self) -> dict:
        return stop_dict(self.stop)


def stop_dict(stop: torch.Tensor) -> dict:
    s = stop.cpu()
    return {"mean_entropy": s[0:1].view(torch.float32).item(), "stable_count": int(s[1]),
            "stopped": int(s[2]), "steps_run": int(s[3])}


class Model:
    """A libdg context over torch-allocated weights, KV cache and workspace."""

    def __init__(self, desc, capacity: int, seed: int | None = 0, sigma: float = 0.02, device="cuda"):
        self.desc = desc
        self.capacity = capacity
        self.dtype = torch_dtype(desc.dtype)
        self.weights = torch.empty(L.dg_weights_bytes(desc), dtype=torch.uint8, device=device)
        if seed is not None:
            L.dg_synth_fill_weights(desc, seed, sigma, self.weights)
        self.kv = torch.zeros(L.dg_kv_bytes(desc, capacity), dtype=torch.uint8, device=device)
        self.ws_bytes = L.dg_workspace_size(desc, capacity)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        self.ctx = L.dg_ctx_create(desc, self.weights, self.kv, capacity, self.workspace, self.ws_bytes)
        self.logits = torch.empty(desc.canvas, desc.vocab, dtype=self.dtype, device=device)

    def close(self):
        if self.ctx:
            L.dg_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # --- views
    def tensor(self, kind, layer=0, expert=0) -> torch.Tensor:
        """Row-major [rows, cols] view of one weight tensor (the embedding and the routed-expert tensors
        are tiled: use load_weight)."""
        if kind in (L.DG_W_EMBED, L.DG_W_EX_GATE, L.DG_W_EX_UP, L.DG_W_EX_DOWN):
            raise ValueError("the embedding and routed-expert weights are stored fragment-tiled; "
                             "write them with load_weight")
        off, r, c = L.dg_weight_tensor(self.desc, kind, layer, expert)
        es = 2 if self.desc.dtype == L.DG_BF16 else 4
        return self.weights[off:off + r * c * es].view(self.dtype).view(r, c)

    def load_weight(self, kind, src: torch.Tensor, layer=0, expert=0):
        """Store a row-major device tensor of the model dtype as weight (kind, layer, expert)."""
        _, r, c = L.dg_weight_tensor(self.desc, kind, layer, expert)
        if tuple(src.shape) != (r, c) or src.dtype != self.dtype or not src.is_cuda or not src.is_contiguous():
            raise ValueError(f"expected a contiguous {self.dtype} CUDA tensor of shape ({r}, {c})")
        L.dg_load_weight(self.desc, kind, layer, expert, src, self.weights)

    def set_weights(self, weights: torch.Tensor):
        """Compute from another buffer holding the same weights (dg_ctx_set_weights); views taken
        earlier with tensor() then refer to the old buffer."""
        if weights.dtype != torch.uint8 or weights.numel() != self.weights.numel() or not weights.is_cuda:
            raise ValueError("expected a uint8 CUDA buffer of dg_weights_bytes bytes")
        L.dg_ctx_set_weights(self.ctx, weights)
        self.weights = weights

    def place_weights(self, measure, tries: int = 3):
        """Keep the fastest of `tries` allocations of the weights.

        How fast the weight streams run depends on where their allocation lies in device memory, and
        an allocation keeps its speed. The current buffer and tries - 1 device copies are each timed
        with measure() (seconds, lower is better; it runs model work and synchronizes), the fastest
        is kept and the others are freed (fewer copies when device memory would not hold another with
        1 GiB to spare). Views taken earlier with tensor() keep the buffer they came from alive and no
        longer reach the model; take them again afterwards. Returns (times, index of the kept buffer)."""
        cands, times = [self.weights], [float(measure())]
        for _ in range(1, tries):
            free, _total = torch.cuda.mem_get_info(self.weights.device)
            if free < self.weights.numel() + (1 << 30):  # no room for another copy: keep the best so far
                break
            cands.append(torch.empty_like(self.weights))
            cands[-1].copy_(self.weights)
            torch.cuda.synchronize()
            self.set_weights(cands[-1])
            times.append(float(measure()))
        best = min(range(len(times)), key=times.__getitem__)
        self.set_weights(cands[best])
        cands.clear()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return times, best

    def use_expert_fp8(self, on: bool = True):
        """Quantize the routed experts to FP8 (once) and compute with them; False returns to the
        model-dtype weights."""
        if on:
            if getattr(self, "expert_fp8", None) is None:
                self.expert_fp8 = torch.empty(L.dg_expert_fp8_bytes(self.desc), dtype=torch.uint8,
                                              device=self.weights.device)
                L.dg_quantize_experts_fp8(self.desc, self.weights, self.expert_fp8)
            L.dg_ctx_use_expert_fp8(self.ctx, self.expert_fp8)
        else:
            L.dg_ctx_use_expert_fp8(self.ctx, None)

    def _kv_raw(self):
        d = self.desc
        t = self.kv.view(self.dtype)
        n = d.n_layers * d.n_kv_heads * self.capacity * d.head_dim
        k = t[:n].view(d.n_layers, d.n_kv_heads, self.capacity, d.head_dim)
        v = t[n:2 * n].view(d.n_layers, d.n_kv_heads, self.capacity // 32, d.head_dim, 32)
        return k, v

    def kv_view(self):
        """(K, V) as [n_layers, n_kv_heads, capacity, head_dim]: K is a view of the cache, V a
        copy un-tiled from its 32-position transposed blocks (include/dg.h)."""
        k, v = self._kv_raw()
        d = self.desc
        slots = torch.tensor(V_SLOT_OF_POS, device=v.device)
        vv = v.index_select(4, slots).permute(0, 1, 2, 4, 3).reshape(d.n_layers, d.n_kv_heads, self.capacity,
                                                                     d.head_dim)
        return k, vv

    def kv_write(self, layer, k_rows, v_rows, start=0):
        """Write positions start .. start+n-1 of one layer: k_rows / v_rows [n_kv_heads, n, head_dim]."""
        k, v = self._kv_raw()
        n = k_rows.shape[1]
        k[layer, :, start:start + n] = k_rows.to(self.dtype)
        pos = torch.arange(start, start + n, device=v.device)
        slot = torch.tensor(V_SLOT_OF_POS, device=v.device)[pos % 32]
        v[layer][:, pos // 32, :, slot] = v_rows.to(self.dtype).permute(1, 0, 2)

    def buffer(self, which, dtype, shape) -> torch.Tensor:
        ptr, nbytes = L.dg_ctx_buffer(self.ctx, which)
        base = self.workspace.data_ptr()
        off = ptr - base
        return self.workspace[off:off + nbytes].view(dtype).view(*shape)

    @property
    def length(self) -> int:
        return L.dg_kv_length(self.ctx)

    # --- calls
    def prefill(self, ids: torch.Tensor):
        L.dg_prefill_kv(self.ctx, ids, ids.numel())

    def denoise_step(self, canvas, step, prev_logits=None, prev_row_stats=None, prev_temperature=0.0, logits=None):
        out = self.logits if logits is None else logits
        L.dg_denoise_step(self.ctx, canvas, step, prev_logits, prev_row_stats, prev_temperature, out)
        return out

    def commit(self, ids):
        L.dg_commit_block(self.ctx, ids)

    def forward_layer(self, layer, x, rows, causal=False):
        L.dg_forward_layer(self.ctx, layer, x, rows, causal)

    def fuse_sampler_stats(self, sched):
        """With a schedule, the LM head also produces the sampler's records at its temperatures and
        denoise_canvas samples from them (dg_ctx_fuse_sampler_stats); None turns that off."""
        L.dg_ctx_fuse_sampler_stats(self.ctx, sched)
        self._fused_sched = sched

    def generate_block(self, sched, block, block_out, commit=True) -> int:
        return L.dg_generate_block(self.ctx, sched, block, self.logits, block_out, commit)

    _STOP_SLOTS = 16

    def denoise_canvas(self, st, sched, block, limit=None, logits=None):
        """Denoising steps of one canvas, from its initial state, until it stops or `limit` steps ran
        (at most sched.max_steps); returns (steps, stopped). Each step's stop state is copied to a
        pinned slot behind the step, and the host reads a step's copy only when that step could have
        stopped: under the two-fold rule the stable count is 0 on step 0 and grows by at most one a
        step, so steps whose count cannot have reached stable_needed are launched back to back."""
        out = self.logits if logits is None else logits
        n = sched.max_steps if limit is None else min(limit, sched.max_steps)
        if not hasattr(self, "_stop_host"):
            self._stop_host = torch.zeros(self._STOP_SLOTS, 4, dtype=torch.int32, pin_memory=True)
            self._stop_ev = [torch.cuda.Event() for _ in range(self._STOP_SLOTS)]
        host, ev, k = self._stop_host, self._stop_ev, self._STOP_SLOTS
        either = (sched.mode & L.DG_SCHED_STOP_EITHER) != 0
        st.init(sched, block)
        known, c_known, enq = -1, 0, 0
        while True:
            j = known + 1
            while j < enq:
                cap = j if known < 0 else c_known + (j - known)  # most the stable count can be at step j
                if either or cap >= sched.stable_needed:
                    break
                j += 1
            if j == enq and enq - known > k - 1:
                j = known + 1
            if j < enq:
                ev[j % k].synchronize()
                known, c_known = j, int(host[j % k, 1])
                if int(host[j % k, 2]):
                    return j + 1, True
                continue
            if enq == n:
                return enq, False
            s = enq
            if s > 0:
                self.denoise_step(st.canvas, s, out, st.row_stats, L.dg_temperature(sched, s - 1), logits=out)
            else:
                self.denoise_step(st.canvas, s, logits=out)
            if getattr(self, "_fused_sched", None) is not None:
                st.sample_fused(self.ctx, sched, s, block)
            else:
                st.sample(out, sched, s, block)
            host[s % k].copy_(st.stop, non_blocking=True)
            ev[s % k].record()
            enq += 1
