"""Seeded synthetic workloads for the early-skip denoising path.

This module only *draws* inputs: shapes, schedules and random tensors.  It holds
none of the method's arithmetic (no norm, attention, score, selection or
unmasking), so both the oracle under ``oracle/`` and the HIP path can take their
inputs from it without sharing any computation.

The pages (ES-dLLM on gist.science, technical summary sections 2 and 4) give no
sizes.  The five workloads below are the plain readings used throughout:

* ``tiny``   -- 2-layer fp32 model, d=64, 4x16 heads, FFN 172, vocab 512,
  16 prompt + 48 masked tokens, 8 steps x 6 tokens, skip layer 1, keep 16 of
  64, relative-L2-plus-inverse-confidence score.  Drawn on the host.
* ``layer8b`` -- one 8B-class layer (d 4096, 32x128 heads, FFN 11008), S=512,
  cached hidden state ~N(0,1), current state = cache + N(0,0.5^2) on a random
  20% of rows and N(0,0.01^2) on the rest, K/V cache ~N(0,1), confidences
  ~U(0,1); eq.(I) score; keep swept over {1, 1/2, 1/4, 1/8}.
* ``full8b`` -- 32 such layers, vocab 126464, 256 uniform prompt tokens + 256
  masked, blocks of 32, 256 steps x 1 token, skip layer 4, keep 1/4.
* ``batch8b`` -- the full8b model, batch 16, prompt lengths ~U{128..1024}
  (right-padded), 256 generated each, blocks of 32, 128 steps x 2 tokens.
* ``long8b`` -- the full8b model, 4096 prompt + 512 masked, blocks of 64,
  512 steps x 1 token, keep 1/8 (576 of 4608 rows).

Weights are N(0, 0.02); RMSNorm gains are 1; there are no biases and the LM
head is untied.  Large tensors are drawn with torch's seeded generator on the
device the caller names (the device's Philox stream), small ones on the host;
whichever device draws them, both sides of a parity check consume the same
bytes (the oracle gets exact host copies).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

__all__ = [
    "ModelDims", "Schedule", "Workload", "WORKLOADS", "workload",
    "make_model", "make_prompt", "make_layer_state", "generator",
]


@dataclasses.dataclass(frozen=True)
class ModelDims:
    d: int
    n_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    n_layers: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0

    @property
    def mask_id(self) -> int:
        # The [MASK] token is the last vocabulary id (511 for the tiny model).
        return self.vocab - 1

    def layer_params(self) -> int:
        return 4 * self.d * self.d + 3 * self.d * self.d_ffn

    def model_params(self) -> int:
        return self.n_layers * self.layer_params() + 2 * self.vocab * self.d


@dataclasses.dataclass(frozen=True)
class Schedule:
    """Semi-autoregressive unmasking schedule and the skip knobs."""
    gen_len: int           # masked positions appended after each prompt
    block_len: int         # positions per semi-autoregressive block
    steps: int             # total denoising steps over the whole generation
    skip_layer: int        # layers [0, skip_layer) run on all rows
    keep: float            # keep ratio (fraction of valid rows recomputed)
    score: str             # "esdllm" | "rell2_invconf" | "cosine"
    alpha: float = 0.5
    refresh_interval: int = 0   # 0: refresh only at each block's first step
    skip_layer2: int = 0        # second skip layer (0: one level); skip_layer < skip_layer2 <= n_layers
    keep2: float = 1.0          # keep ratio at the second skip layer
    response_interval: int = 0  # > 0: full-context skip steps every N in-block steps, response rows only otherwise
    score_tensor: str = "hidden"  # tensor whose change is scored: "hidden" (layer-s input), "key" or "value" of layer s
    per_layer: bool = False     # DyLLM-style re-selection at every layer >= skip_layer by the context change
    keep_layer: float = 0.0     # keep ratio of that re-selection (0: same as keep)

    @property
    def n_blocks(self) -> int:
        return self.gen_len // self.block_len

    @property
    def steps_per_block(self) -> int:
        return self.steps // self.n_blocks

    @property
    def per_step(self) -> int:
        return self.block_len // self.steps_per_block


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: ModelDims
    dtype: str                   # storage type: "f32" or "bf16"
    seed: int
    batch: int
    prompt_len: Optional[int]    # fixed prompt length, or None for ragged
    prompt_range: Optional[tuple]  # (lo, hi) inclusive for ragged prompts
    sched: Optional[Schedule]
    draw_device: str             # where the large tensors are drawn


_D8B = dict(d=4096, n_heads=32, head_dim=128, d_ffn=11008)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", ModelDims(d=64, n_heads=4, head_dim=16, d_ffn=172, vocab=512, n_layers=2),
        dtype="f32", seed=0, batch=1, prompt_len=16, prompt_range=None,
        sched=Schedule(gen_len=48, block_len=48, steps=8, skip_layer=1, keep=0.25,
                       score="rell2_invconf"),
        draw_device="cpu"),
    "layer8b": Workload(
        "layer8b", ModelDims(vocab=126464, n_layers=1, **_D8B),
        dtype="bf16", seed=1, batch=1, prompt_len=512, prompt_range=None,
        sched=None, draw_device="cuda"),
    "full8b": Workload(
        "full8b", ModelDims(vocab=126464, n_layers=32, **_D8B),
        dtype="bf16", seed=2, batch=1, prompt_len=256, prompt_range=None,
        sched=Schedule(gen_len=256, block_len=32, steps=256, skip_layer=4, keep=0.25,
                       score="esdllm"),
        draw_device="cuda"),
    "batch8b": Workload(
        "batch8b", ModelDims(vocab=126464, n_layers=32, **_D8B),
        dtype="bf16", seed=3, batch=16, prompt_len=None, prompt_range=(128, 1024),
        sched=Schedule(gen_len=256, block_len=32, steps=128, skip_layer=4, keep=0.25,
                       score="esdllm"),
        draw_device="cuda"),
    "long8b": Workload(
        "long8b", ModelDims(vocab=126464, n_layers=32, **_D8B),
        dtype="bf16", seed=4, batch=1, prompt_len=4096, prompt_range=None,
        sched=Schedule(gen_len=512, block_len=64, steps=512, skip_layer=4, keep=0.125,
                       score="esdllm"),
        draw_device="cuda"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def generator(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g: torch.Generator, shape, std: float, device: str) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(mean=0.0, std=std, generator=g)
    return t


def _store(t: torch.Tensor, dtype: str) -> torch.Tensor:
    # bf16 storage: round-to-nearest-even by torch's conversion.
    return t.to(torch.bfloat16) if dtype == "bf16" else t


LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def make_model(dims: ModelDims, seed: int, dtype: str, device: str,
               n_layers: Optional[int] = None, std: float = 0.02) -> dict:
    """Draw a random-init model.

    Draw order: E, then per layer (Wq, Wk, Wv, Wo, Wg, Wu, Wd), then W_lm.
    Matrices are [out, in] row-major.  Gains are ones (not drawn).
    ``n_layers`` may truncate the draw (the first layers are identical to those
    of the full draw, since the stream is consumed in order).
    """
    L = dims.n_layers if n_layers is None else n_layers
    g = generator(seed, device)
    d, F, V = dims.d, dims.d_ffn, dims.vocab
    model = {"embed": _store(_normal(g, (V, d), std, device), dtype), "layers": []}
    ones = torch.ones(d, dtype=torch.float32, device=device)
    for _ in range(L):
        lw = {"attn_norm": _store(ones.clone(), dtype), "ffn_norm": _store(ones.clone(), dtype)}
        for key, shape in (("wq", (d, d)), ("wk", (d, d)), ("wv", (d, d)), ("wo", (d, d)),
                           ("w_gate", (F, d)), ("w_up", (F, d)), ("w_down", (d, F))):
            lw[key] = _store(_normal(g, shape, std, device), dtype)
        model["layers"].append(lw)
    # W_lm is drawn after all n_layers of the full model, so a truncated draw
    # skips it (truncation is only for layer-level workloads).
    if L == dims.n_layers:
        model["final_norm"] = _store(ones.clone(), dtype)
        model["lm_head"] = _store(_normal(g, (V, d), std, device), dtype)
    return model


def make_prompt(wl: Workload, device: str = "cpu"):
    """Prompt token ids and lengths.

    Returns (prompts: list of int64 tensors, prompt_lens: list of int).
    Prompt ids are uniform over the whole vocabulary (the [MASK] id included:
    prompt positions are never masked whatever their id).  Drawn on the host
    with its own stream (seed * 1000 + 7) so that the prompt does not depend on
    how many weights were drawn.
    """
    g = generator(wl.seed * 1000 + 7, "cpu")
    if wl.prompt_len is not None:
        lens = [wl.prompt_len] * wl.batch
    else:
        lo, hi = wl.prompt_range
        lens = torch.randint(lo, hi + 1, (wl.batch,), generator=g).tolist()
    prompts = [torch.randint(0, wl.dims.vocab, (n,), generator=g, dtype=torch.int64) for n in lens]
    return [p.to(device) for p in prompts], lens


def make_layer_state(wl: Workload, device: str, S: Optional[int] = None,
                     changed_frac: float = 0.2, big_std: float = 0.5, small_std: float = 0.01):
    """Single-layer step state (layer8b workload).

    h_prev ~ N(0,1) [S,d]; h_cur = h_prev + N(0, big_std^2) on a random
    ``changed_frac`` of rows and + N(0, small_std^2) on the others; K/V cache
    ~N(0,1) [S,d]; conf ~ U(0,1) [S].  Draw order: h_prev, noise, row subset,
    K, V, conf, from the seed's stream offset by 1 (the weights use the seed's
    stream itself).  h_prev/h_cur/K/V are stored in the workload's dtype.
    """
    S = wl.prompt_len if S is None else S
    d = wl.dims.d
    g = generator(wl.seed * 1000 + 1, device)
    h_prev = _normal(g, (S, d), 1.0, device)
    noise = _normal(g, (S, d), 1.0, device)
    perm = torch.randperm(S, generator=g, device=device)
    n_big = int(round(changed_frac * S))
    scale = torch.full((S, 1), small_std, dtype=torch.float32, device=device)
    scale[perm[:n_big]] = big_std
    h_cur = h_prev + noise * scale
    k = _normal(g, (S, d), 1.0, device)
    v = _normal(g, (S, d), 1.0, device)
    conf = torch.rand((S,), generator=g, device=device, dtype=torch.float32)
    dt = wl.dtype
    return {"h_prev": _store(h_prev, dt), "h_cur": _store(h_cur, dt), "k": _store(k, dt),
            "v": _store(v, dt), "conf": conf, "changed_rows": perm[:n_big].sort().values}


def host_f64(t: torch.Tensor):
    """Exact host copy as float64 numpy (bf16/fp32 widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
