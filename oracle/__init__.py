"""CPU oracle of the canvas-denoising hot path. TEST INFRASTRUCTURE ONLY.

A plain, slow NumPy float64 statement of what one uniform-state discrete
diffusion denoising step computes, written from the pages that describe
DiffusionGemma (cited per function). It exists to check the HIP library:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product package never imports it, and this
package imports nothing from the product package.

Sources (cited by page title and section throughout):

* [P1] molayo1419.me, "Running the diffusion LLM DiffusionGemma on Modal and
  visualising the denoising steps in a browser".
* [P2] axbrief.com, "DiffusionGemma: Google's 26B MoE model that generates text
  like images".
* [P3] juhoplayground.github.io, "DiffusionGemma - parallel text generation and
  diffusion-based language models".
* [P4] marrrang.tistory.com, "[AI] DiffusionGemma deep dive - Uniform State
  Diffusion and inference architecture".

Precision: every intermediate is float64 and never rounded; weights and inputs
enter as the exact values the GPU stores (bf16 or fp32 promoted to float64).

Parity pins live in ``tests/test_oracle_*.py``. Functions without an
independent pin are marked "parity unpinned" in their docstring.
"""
from . import philox, sampler, model, loop  # noqa: F401
