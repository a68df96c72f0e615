"""Device-side decoding driver over libdtsk: owns the caches as torch tensors
(device memory only) and calls dl_denoise_step once per denoising step.

The semi-autoregressive schedule (ES-dLLM section 1: a few most-confident
masked tokens are unmasked per step; section 2B: a full refresh pass at set
intervals) is host bookkeeping: which block is current, how many tokens to
unmask, whether this step is a refresh step.  Everything computed per token
runs in the library.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib as L


PRODUCT_WEIGHTS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def pack_model(tensors: dict, free_source: bool = False, stream=None) -> dict:
    """The same model with its product weights (every layer's wq, wk, wv, wo,
    w_gate, w_up, w_down and the LM head, if the dict has one) in the blocked order
    (DL_WEIGHTS_BLOCKED), written by dl_pack_weights into new device tensors;
    the embedding table and norm gains are shared.  With ``free_source`` the
    dict's row-major tensors are dropped as their copies are made (the caller
    must hold no other reference for the memory to be released)."""
    def packed(t):
        out = torch.empty_like(t)
        L.dl_pack_weights(t, out, stream)
        return out
    out = {k: v for k, v in tensors.items() if k not in ("layers", "lm_head")}
    layers = []
    for i, lw in enumerate(tensors["layers"]):
        nl = {k: (packed(v) if k in PRODUCT_WEIGHTS else v) for k, v in lw.items()}
        layers.append(nl)
        if free_source:
            tensors["layers"][i] = {k: v for k, v in lw.items() if k not in PRODUCT_WEIGHTS}
            del lw
    out["layers"] = layers
    if "lm_head" in tensors:
        out["lm_head"] = packed(tensors["lm_head"])
        if free_source:
            del tensors["lm_head"]
    return out


class DeviceModel:
    """Weights on the device plus the dl_model struct that points at them.
    ``weight_layout``: "row_major", or "blocked" for tensors from pack_model."""

    def __init__(self, tensors: dict, n_heads: int, head_dim: int, dtype: str, rms_eps: float = 1e-5,
                 rope_base: float = 10000.0, weight_layout: str = "row_major"):
        self.t = tensors
        self.weight_layout = weight_layout
        emb = tensors["embed"]
        self.vocab, self.d = emb.shape
        self.d_ffn = tensors["layers"][0]["w_gate"].shape[0]
        self.n_layers = len(tensors["layers"])
        self.n_heads, self.head_dim = n_heads, head_dim
        self.dtype = dtype
        self.rms_eps, self.rope_base = rms_eps, rope_base
        self._layers = (L.LayerW * self.n_layers)(*[L.layer_struct(lw) for lw in tensors["layers"]])

    def dims(self, B: int, S: int) -> L.Dims:
        return L.make_dims(B, S, self.d, self.n_heads, self.head_dim, self.d_ffn, self.vocab, self.n_layers,
                           self.dtype, self.rms_eps, self.rope_base, self.weight_layout)

    def struct(self, B: int, S: int) -> L.Model:
        return L.Model(self.dims(B, S), L.ptr(self.t["embed"]), L.ptr(self.t["final_norm"]),
                       L.ptr(self.t["lm_head"]), self._layers)


def is_refresh_step(step: int, steps_per_block: int, refresh_interval: int) -> bool:
    sib = step % steps_per_block
    return sib == 0 or (refresh_interval > 0 and sib % refresh_interval == 0)


def is_full_context_step(step: int, steps_per_block: int, response_interval: int) -> bool:
    """DyLLM response-only strategy: with an interval N > 0 only every N-th
    in-block step takes the prompt rows too."""
    return response_interval <= 0 or (step % steps_per_block) % response_interval == 0


class Decoder:
    """Caches of a batch of sequences: prompt + gen_len masked positions each,
    right-padded to S = max length."""

    def __init__(self, model: DeviceModel, prompts: Sequence[torch.Tensor], sched, keep_logits: bool = False,
                 device: str = "cuda", mask_id: Optional[int] = None):
        self.m = model
        self.sched = sched
        self.B = len(prompts)
        self.prompt_lens = [int(len(p)) for p in prompts]
        self.seq_lens = [n + sched.gen_len for n in self.prompt_lens]
        self.S = max(self.seq_lens)
        B, S, d = self.B, self.S, model.d
        mid = model.vocab - 1 if mask_id is None else mask_id
        tdt = L.TORCH_DTYPES[L.DTYPES[model.dtype]]
        tokens = torch.zeros((B, S), dtype=torch.int32)
        masked = torch.zeros((B, S), dtype=torch.uint8)
        for b, p in enumerate(prompts):
            n = len(p)
            tokens[b, :n] = p.to(torch.int32).cpu()
            tokens[b, n:n + sched.gen_len] = mid
            masked[b, n:n + sched.gen_len] = 1
        self.tokens0, self.masked0 = tokens.to(device), masked.to(device)
        self.tokens, self.masked = self.tokens0.clone(), self.masked0.clone()
        self.seq_len = torch.tensor(self.seq_lens, dtype=torch.int32, device=device)
        self.prompt_len = torch.tensor(self.prompt_lens, dtype=torch.int32, device=device)
        self.h_prev = torch.zeros((B, S, d), dtype=tdt, device=device)
        self.k_cache = torch.zeros((model.n_layers, B, S, d), dtype=tdt, device=device)
        self.v_cache = torch.zeros((model.n_layers, B, S, d), dtype=tdt, device=device)
        self.h_final = torch.zeros((B, S, d), dtype=tdt, device=device)
        self.conf = torch.zeros((B, S), dtype=torch.float32, device=device)
        self.argmax = torch.zeros((B, S), dtype=torch.int32, device=device)
        self.scores = torch.zeros((B, S), dtype=torch.float32, device=device)
        self.logits = torch.zeros((B, S, model.vocab), dtype=torch.float32, device=device) if keep_logits else None
        self.sel = L.SelectionTensors(B, S, device)
        two = getattr(sched, "skip_layer2", 0) > 0
        self.h_prev2 = torch.zeros((B, S, d), dtype=tdt, device=device) if two else None
        self.scores2 = torch.zeros((B, S), dtype=torch.float32, device=device) if two else None
        self.sel2 = L.SelectionTensors(B, S, device) if two else None
        per_layer = bool(getattr(sched, "per_layer", False))
        Ln = model.n_layers
        self.q_cache = torch.zeros((Ln, B, S, d), dtype=tdt, device=device) if per_layer else None
        self.ctx_cache = torch.zeros((Ln, B, S, d), dtype=torch.float32, device=device) if per_layer else None
        self.lse_cache = (torch.zeros((Ln, B, S, model.n_heads), dtype=torch.float32, device=device)
                          if per_layer else None)
        self.y_cache = torch.zeros((Ln, B, S, d), dtype=torch.float32, device=device) if per_layer else None
        self.layer_scores = torch.zeros((B, S), dtype=torch.float32, device=device) if per_layer else None
        self.sel_l = L.SelectionTensors(B, S, device) if per_layer else None
        self.dims = model.dims(B, S)
        self.model_struct = model.struct(B, S)
        self.ws = L.workspace(self.dims, sum(self.seq_lens), device)
        self._seq_len_host = (ctypes.c_int32 * B)(*self.seq_lens)
        self._prompt_len_host = (ctypes.c_int32 * B)(*self.prompt_lens)
        self.state = L.State(L.ptr(self.tokens), L.ptr(self.masked), L.ptr(self.seq_len), L.ptr(self.prompt_len),
                             L.ptr(self.h_prev), L.ptr(self.k_cache), L.ptr(self.v_cache), L.ptr(self.h_final),
                             L.ptr(self.conf), L.ptr(self.argmax), L.ptr(self.logits), L.ptr(self.scores),
                             self.sel.struct(), L.ptr(self.h_prev2), L.ptr(self.scores2),
                             self.sel2.struct() if two else L.Selection(), L.ptr(self.q_cache),
                             L.ptr(self.ctx_cache), L.ptr(self.lse_cache), L.ptr(self.y_cache),
                             L.ptr(self.layer_scores), self.sel_l.struct() if per_layer else L.Selection())
        self.steps_per_block = sched.steps // (sched.gen_len // sched.block_len)
        self.per_step = sched.block_len // self.steps_per_block

    def reset(self):
        """Back to the initial tokens and mask (caches are rebuilt by step 0's refresh)."""
        self.tokens.copy_(self.tokens0)
        self.masked.copy_(self.masked0)

    def params(self, step: int, force_refresh: Optional[bool] = None, keep: Optional[float] = None,
               mode: int = L.DL_SEL_TOPK, threshold: float = 0.0, n_unmask: Optional[int] = None,
               response_only: Optional[bool] = None, keep2: Optional[float] = None, mode2: int = L.DL_SEL_TOPK,
               threshold2: float = 0.0, mode_l: int = L.DL_SEL_TOPK, threshold_l: float = 0.0) -> L.StepParams:
        s = self.sched
        refresh = (is_refresh_step(step, self.steps_per_block, s.refresh_interval) if force_refresh is None
                   else force_refresh)
        if response_only is None:
            response_only = not is_full_context_step(step, self.steps_per_block, getattr(s, "response_interval", 0))
        s2 = getattr(s, "skip_layer2", 0)
        return L.StepParams(step // self.steps_per_block, s.block_len,
                            self.per_step if n_unmask is None else n_unmask, s.skip_layer, int(bool(refresh)),
                            L.SCORE_KINDS[s.score], s.alpha, mode, s.keep if keep is None else keep, threshold,
                            ctypes.cast(self._seq_len_host, ctypes.POINTER(ctypes.c_int32)),
                            int(bool(response_only) and not refresh),
                            ctypes.cast(self._prompt_len_host, ctypes.POINTER(ctypes.c_int32)), s2, mode2,
                            getattr(s, "keep2", 1.0) if keep2 is None else keep2, threshold2,
                            L.SCORE_TENSORS[getattr(s, "score_tensor", "hidden")],
                            int(bool(getattr(s, "per_layer", False))), mode_l,
                            getattr(s, "keep_layer", 0.0) or s.keep, threshold_l)

    def step(self, step: int, **kw):
        L.dl_denoise_step(self.model_struct, self.state, self.params(step, **kw), self.ws)

    def run(self, n_steps: Optional[int] = None, **kw):
        for t in range(self.sched.steps if n_steps is None else n_steps):
            self.step(t, **kw)
