"""Plain, slow, fp64 CPU oracle of the early-skip denoising step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP library (no kernels, headers, helpers or tables)
and imports nothing from it.

Sources (the gist.science summary pages, read as the specification):

* ES-dLLM: Efficient Inference for Diffusion Large Language Models by
  Early-Skipping -- technical summary section 1 (whole-sequence iterative
  denoising, highest-confidence unmasking), section 2A (importance score
  eq. I), section 2B (top-k selection with k = (1 - r_l)|S|, early skip,
  K/V/hidden caches updated in place by scatter for selected rows and reused
  for skipped rows, periodic full refresh, skip at 1/8 and 1/4 of depth).
* DyLLM: Efficient Diffusion LLM Inference via Saliency-based Token Selection
  and Partial Attention -- technical summary section 2A (cosine similarity of
  a token's vector between adjacent steps; salient when it falls below a
  threshold).

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/`` against
closed forms, invariants, hand-worked values under ``tests/golden/`` or
library routines; the module docstring of ``esdllm`` lists the readings taken
where the pages are silent.
"""
from .esdllm import *  # noqa: F401,F403
