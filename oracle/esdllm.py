"""fp64 reference of the early-skip / partial-recompute denoising loop.

TEST INFRASTRUCTURE (see the package docstring): plain numpy, float64
arithmetic, one obvious step at a time.  Library primitives used as steps:
``numpy.matmul`` (dense products), ``numpy.exp/sqrt/sin/cos``, ``numpy.argsort``
with a stable key (selection).  Nothing is fused, blocked or reordered beyond
what the definitions state.

Where a floating-point value decides an integer (top-k selection, unmasking,
argmax) the decision is taken on the value rounded to float32, the precision
the GPU kernels decide in.

Model (a bidirectional pre-RMSNorm transformer; the pages only say the whole
sequence is reprocessed each step, ES-dLLM section 1 / DyLLM section 1):

    n(x)  = x / sqrt(mean(x^2) + eps) * g
    q,k,v = n(x) Wq^T, n(x) Wk^T, n(x) Wv^T ;  q,k rotated by RoPE at the
            token's absolute position (rotate-half pairs (j, j + dh/2),
            angle pos * base^(-2j/dh))
    h     = x + softmax(q k^T / sqrt(dh)) v Wo^T   (per head, all valid keys)
    y     = h + (silu(n(h) Wg^T) * n(h) Wu^T) Wd^T
    logits= n_final(x_L) Wlm^T

Readings taken where the pages are silent or disagree (each is repeated in the
function that uses it):

* The varied tensor H in eq. I is the *input hidden state of the skip layer s*
  (the pages allow hidden states, keys or values).  H^(t-1) is the previous
  step's value for every row: layers below s run on all rows every step.
* c^(t-1) is the cached maximum softmax probability of every row (stale for
  rows skipped at the previous step); it enters eq. I with a + sign as printed
  (one page's prose says confident tokens change less; the formula wins).
* k = ceil(keep * |S|) on the sequence's valid length, computed exactly from
  the float32 keep value, clamped to [1, |S|].  Ties in the score go to the
  lower index; the selected set is returned in ascending index order.
* A refresh step (every row through every layer) runs at each block's first
  step, and every ``refresh_interval`` steps inside a block when non-zero.
* Selected rows write their fresh K/V into the layer's cache *before*
  attention; skipped rows' K/V, confidence, argmax and final hidden state are
  reused untouched.
* Unmasking takes, among still-masked positions of the current block, the n
  highest cached confidences (lower index on ties) and writes the cached argmax.
* The tiny workload's own text defines a second score: relative L2 change plus
  (1 - c).  DyLLM's saliency (cosine similarity) gives a third: 1 - cos.
* Two skip layers (ES-dLLM section 2B: skipping at layers 4 and 8 of 32, a
  skip ratio r_l per layer): the second level scores the rows kept by the
  first, at the input of layer s2, against a second cache H2 of that input,
  and keeps k2 = ceil(keep2 * |S|) of them (|S| as for the first level, capped
  at the first level's count).  H2 is rewritten for every row on a refresh
  step and for the first level's rows on a skip step.
* Keys or values as the varied tensor (ES-dLLM section 2A allows hidden
  states, keys or values): H is then the key (rotated, as cached) or value row
  of layer s, computed from X_s for every candidate row; h_prev holds its
  previous value instead of the hidden state.
* Per-layer re-selection (DyLLM section 2B): at every layer from s on, the
  active rows (those whose layer input was recomputed: the ES selection at
  layer s, the previous layer's salient rows above it) get fresh q/K/V and
  exact attention; every other row's context is updated as C + S dV with S
  from its cached query and normaliser and the active rows' previous keys.
  The rows with the largest 1 - cos(C_new, C_cached) (top-k at keep_layer, or
  above a threshold) go through Wo and the FFN; the others keep their cached
  layer output.  The context cache takes C_new for every row; query and
  normaliser caches change for the active rows only.
* Response-only steps (DyLLM section 2B, strategy 3): on a skip step that is
  not a full-context step, only the response rows (positions >= prompt length)
  go through the prefix layers, are scored and can be kept; |S| is then the
  response length.  Prompt rows keep every cache (their K/V at every layer
  serve as keys).  Full-context steps are those whose in-block index is a
  multiple of the interval; refresh steps are always full context.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "rms_norm", "rope", "attention", "silu", "layer_forward", "lm_logits",
    "conf_argmax", "score_rows", "keep_count", "select_topk", "select_threshold",
    "unmask", "SeqState", "init_state", "denoise_step", "decode",
    "is_refresh_step", "is_full_context_step", "candidate_rows", "level2_count", "scored_tensor", "FLT_MIN",
    "attention_lse", "finish_layer", "layer_parts", "approx_context", "layer_input_rows",
]

F64 = np.float64
FLT_MIN = float(np.finfo(np.float32).tiny)   # smallest normal float32


# ----------------------------------------------------------------------------
# Model pieces
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm: x / sqrt(mean(x^2) + eps) * g."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, F64)


def rope(x: np.ndarray, pos: np.ndarray, n_heads: int, head_dim: int, base: float) -> np.ndarray:
    """Rotary position embedding, rotate-half form, per head.

    For pair j in [0, dh/2): theta = pos * base^(-2j/dh);
    (x_j, x_{j+dh/2}) -> (x_j cos - x_{j+dh/2} sin, x_{j+dh/2} cos + x_j sin).
    """
    x = np.asarray(x, F64)
    n = x.shape[0]
    half = head_dim // 2
    j = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * j / head_dim)
    ang = np.asarray(pos, F64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    xh = x.reshape(n, n_heads, head_dim)
    x1, x2 = xh[..., :half], xh[..., half:]
    out = np.empty_like(xh)
    out[..., :half] = x1 * c - x2 * s
    out[..., half:] = x2 * c + x1 * s
    return out.reshape(n, n_heads * head_dim)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_heads: int, head_dim: int) -> np.ndarray:
    """Bidirectional multi-head attention of query rows against all given keys.

    q: [n, H*dh]; K, V: [m, H*dh] (the sequence's valid keys).  Per head:
    softmax over keys of q.k / sqrt(dh) (max-subtracted), times V.
    """
    q = np.asarray(q, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    n = q.shape[0]
    out = np.empty((n, n_heads * head_dim), F64)
    scale = 1.0 / math.sqrt(head_dim)
    for h in range(n_heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        s = (q[:, sl] @ K[:, sl].T) * scale          # [n, m]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, sl] = p @ V[:, sl]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def layer_forward(x: np.ndarray, pos: np.ndarray, lw: dict, K_cache: np.ndarray,
                  V_cache: np.ndarray, n_valid: int, dims) -> np.ndarray:
    """One layer on the rows ``x`` (positions ``pos``) of one sequence.

    The rows' fresh K/V are written into ``K_cache``/``V_cache`` (this layer,
    this sequence, [S, d]) at ``pos`` *before* attention, so every row attends
    over keys 0..n_valid-1 with fresh values for the rows recomputed now and
    cached values for the rest (ES-dLLM section 2B: in-place cache update for
    selected tokens, direct reuse for skipped ones).
    """
    H, dh = dims.n_heads, dims.head_dim
    xn = rms_norm(x, lw["attn_norm"], dims.rms_eps)
    q = xn @ np.asarray(lw["wq"], F64).T
    k = xn @ np.asarray(lw["wk"], F64).T
    v = xn @ np.asarray(lw["wv"], F64).T
    q = rope(q, pos, H, dh, dims.rope_base)
    k = rope(k, pos, H, dh, dims.rope_base)
    K_cache[pos] = k
    V_cache[pos] = v
    o = attention(q, K_cache[:n_valid], V_cache[:n_valid], H, dh)
    h = x + o @ np.asarray(lw["wo"], F64).T
    hn = rms_norm(h, lw["ffn_norm"], dims.rms_eps)
    a = silu(hn @ np.asarray(lw["w_gate"], F64).T) * (hn @ np.asarray(lw["w_up"], F64).T)
    return h + a @ np.asarray(lw["w_down"], F64).T


# ----------------------------------------------------------------------------
# DyLLM pieces (DyLLM section 2B): per-layer intermediates and the approximate
# context update of rows whose query did not change
# ----------------------------------------------------------------------------

def attention_lse(q: np.ndarray, K: np.ndarray, n_heads: int, head_dim: int) -> np.ndarray:
    """Per row and head, log sum_j exp(q.k_j / sqrt(dh)) over the given keys:
    the softmax normaliser of ``attention`` in log form.  [n, H]."""
    q = np.asarray(q, F64)
    K = np.asarray(K, F64)
    scale = 1.0 / math.sqrt(head_dim)
    out = np.empty((q.shape[0], n_heads), F64)
    for h in range(n_heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        s = (q[:, sl] @ K[:, sl].T) * scale
        m = s.max(axis=1)
        out[:, h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def finish_layer(x: np.ndarray, ctx: np.ndarray, lw: dict, dims) -> np.ndarray:
    """The rest of a layer from its attention context (before Wo):
    h = x + ctx Wo^T; y = h + (silu(n(h) Wg^T) * n(h) Wu^T) Wd^T."""
    h = np.asarray(x, F64) + np.asarray(ctx, F64) @ np.asarray(lw["wo"], F64).T
    hn = rms_norm(h, lw["ffn_norm"], dims.rms_eps)
    a = silu(hn @ np.asarray(lw["w_gate"], F64).T) * (hn @ np.asarray(lw["w_up"], F64).T)
    return h + a @ np.asarray(lw["w_down"], F64).T


def layer_parts(x: np.ndarray, pos: np.ndarray, lw: dict, K_cache: np.ndarray, V_cache: np.ndarray,
                n_valid: int, dims):
    """``layer_forward`` with its intermediates: returns (y, q, ctx, lse) where
    q is the rows' rotated query, ctx their attention context (before Wo) and
    lse its per-head log normaliser.  Writes the rows' K/V first, as there."""
    H, dh = dims.n_heads, dims.head_dim
    xn = rms_norm(x, lw["attn_norm"], dims.rms_eps)
    q = rope(xn @ np.asarray(lw["wq"], F64).T, pos, H, dh, dims.rope_base)
    k = rope(xn @ np.asarray(lw["wk"], F64).T, pos, H, dh, dims.rope_base)
    v = xn @ np.asarray(lw["wv"], F64).T
    K_cache[pos] = k
    V_cache[pos] = v
    ctx = attention(q, K_cache[:n_valid], V_cache[:n_valid], H, dh)
    lse = attention_lse(q, K_cache[:n_valid], H, dh)
    return finish_layer(x, ctx, lw, dims), q, ctx, lse


def approx_context(C: np.ndarray, q: np.ndarray, lse: np.ndarray, K_act: np.ndarray, dV_act: np.ndarray,
                   n_heads: int, head_dim: int) -> np.ndarray:
    """DyLLM's saliency-aware approximate attention for rows with cached context
    C, query q and normaliser lse: C + S dV, with S_ij = exp(q_i.k_j/sqrt(dh) -
    lse_i) the cached attention probability of key j and dV_j the change of its
    value row, over the active rows j (keys K_act as they were when C was
    formed).  Exact when only those value rows changed."""
    C = np.array(C, F64, copy=True)
    q = np.asarray(q, F64)
    K_act = np.asarray(K_act, F64)
    dV_act = np.asarray(dV_act, F64)
    scale = 1.0 / math.sqrt(head_dim)
    for h in range(n_heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        S = np.exp((q[:, sl] @ K_act[:, sl].T) * scale - np.asarray(lse, F64)[:, h:h + 1])
        C[:, sl] += S @ dV_act[:, sl]
    return C


def layer_input_rows(st, X_s: np.ndarray, layer: int, s_layer: int, rows: np.ndarray) -> np.ndarray:
    """Inputs of ``rows`` at ``layer`` in a per-layer step: the fresh skip-layer
    input at layer s, else the cached output of the layer below (rewritten
    this step for the rows that layer recomputed)."""
    return np.asarray(X_s, F64)[rows] if layer == s_layer else st.Y[layer - 1][rows]


def lm_logits(x: np.ndarray, final_norm: np.ndarray, lm_head: np.ndarray, eps: float) -> np.ndarray:
    return rms_norm(x, final_norm, eps) @ np.asarray(lm_head, F64).T


def conf_argmax(logits: np.ndarray):
    """Confidence = maximum softmax probability = 1 / sum_v exp(l_v - max l).

    The argmax is taken on the logits rounded to float32, lowest id on ties.
    Returns (conf fp64 [n], argmax int64 [n]).
    """
    logits = np.asarray(logits, F64)
    m = logits.max(axis=1, keepdims=True)
    conf = 1.0 / np.exp(logits - m).sum(axis=1)
    l32 = logits.astype(np.float32)
    amax = np.argmax(l32, axis=1).astype(np.int64)   # first maximum = lowest id
    return conf, amax


# ----------------------------------------------------------------------------
# Importance score and selection (ES-dLLM section 2A/2B, DyLLM section 2A)
# ----------------------------------------------------------------------------

def score_rows(kind: str, x_cur: np.ndarray, h_prev: np.ndarray, conf: np.ndarray,
               alpha: float = 0.5) -> np.ndarray:
    """Per-row importance score, fp64.

    esdllm        : alpha*c + (1-alpha) * ||x - h||_1 / (sqrt(d) * ||h||_2)   (eq. I)
    rell2_invconf : ||x - h||_2 / ||h||_2 + (1 - c)      (the tiny workload's text)
    cosine        : 1 - x.h / (||x||_2 ||h||_2)            (DyLLM saliency)

    Denominators are floored at FLT_MIN so an all-zero cached row scores finite.
    """
    x = np.asarray(x_cur, F64)
    h = np.asarray(h_prev, F64)
    c = np.asarray(conf, F64)
    d = x.shape[1]
    diff = x - h
    if kind == "esdllm":
        l1 = np.abs(diff).sum(axis=1)
        den = np.maximum(math.sqrt(d) * np.sqrt((h * h).sum(axis=1)), FLT_MIN)
        return alpha * c + (1.0 - alpha) * l1 / den
    if kind == "rell2_invconf":
        num = np.sqrt((diff * diff).sum(axis=1))
        den = np.maximum(np.sqrt((h * h).sum(axis=1)), FLT_MIN)
        return num / den + (1.0 - c)
    if kind == "cosine":
        den = np.maximum(np.sqrt((x * x).sum(axis=1)) * np.sqrt((h * h).sum(axis=1)), FLT_MIN)
        return 1.0 - (x * h).sum(axis=1) / den
    raise ValueError(f"unknown score kind {kind!r}")


def keep_count(keep: float, n: int) -> int:
    """k = (1 - r)|S| with keep = 1 - r: ceil(keep * n), clamped to [1, n].

    ``keep`` is taken as a float32 (the value a caller passes over the C ABI);
    the product of a float32 and an integer below 2^29 is exact in float64,
    so the ceiling has no rounding drift.
    """
    if n <= 0:
        return 0
    k = math.ceil(float(np.float32(keep)) * n)
    return max(1, min(n, k))


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k highest scores (decided in float32), ascending.

    Order key (-score, index): among equal scores the lower index is taken.
    A NaN score is an error here (the GPU ranks NaN last).
    """
    s32 = np.asarray(scores, F64).astype(np.float32)
    assert not np.isnan(s32).any(), "NaN importance score"
    n = s32.shape[0]
    order = np.lexsort((np.arange(n), -s32.astype(F64)))   # primary: -score, then index
    return np.sort(order[:k]).astype(np.int64)


def select_threshold(scores: np.ndarray, tau: float) -> np.ndarray:
    """Rows whose float32 score is strictly above float32 tau, ascending."""
    s32 = np.asarray(scores, F64).astype(np.float32)
    assert not np.isnan(s32).any(), "NaN importance score"
    return np.nonzero(s32 > np.float32(tau))[0].astype(np.int64)


def unmask(masked: np.ndarray, conf: np.ndarray, lo: int, hi: int, n: int) -> np.ndarray:
    """Positions to unmask: the n most confident still-masked ones in [lo, hi).

    Decided on float32 confidence, lower index on ties; returned ascending.
    """
    cand = np.nonzero(masked[lo:hi])[0] + lo
    if cand.size == 0 or n <= 0:
        return np.zeros(0, np.int64)
    c32 = np.asarray(conf, F64)[cand].astype(np.float32)
    order = np.lexsort((cand, -c32.astype(F64)))
    return np.sort(cand[order[:min(n, cand.size)]]).astype(np.int64)


# ----------------------------------------------------------------------------
# Decode state and the denoising step
# ----------------------------------------------------------------------------

@dataclass
class SeqState:
    """Per-sequence caches (all rows of the sequence, valid length n)."""
    tokens: np.ndarray            # [n] int64
    masked: np.ndarray            # [n] bool
    prompt_len: int
    conf: np.ndarray              # [n] fp64, max softmax probability
    argmax: np.ndarray            # [n] int64
    h_prev: np.ndarray            # [n, d] previous value of the scored tensor (the skip-layer input by default)
    K: List[np.ndarray]           # per layer [n, d] (rotated keys)
    V: List[np.ndarray]           # per layer [n, d]
    h_final: np.ndarray           # [n, d] last layer output (before final norm)
    logits: Optional[np.ndarray] = None   # [n, V] when kept
    h_prev2: Optional[np.ndarray] = None  # [n, d] input of the second skip layer
    # per-layer caches of the DyLLM variant (layers >= s): rotated query,
    # attention context, its per-head log normaliser, layer output
    Q: Optional[List[np.ndarray]] = None      # per layer [n, d]
    C: Optional[List[np.ndarray]] = None      # per layer [n, d]
    LSE: Optional[List[np.ndarray]] = None    # per layer [n, H]
    Y: Optional[List[np.ndarray]] = None      # per layer [n, d]


def init_state(prompt: np.ndarray, gen_len: int, dims, mask_id: Optional[int] = None,
               keep_logits: bool = False) -> SeqState:
    P = int(len(prompt))
    n = P + gen_len
    mid = dims.vocab - 1 if mask_id is None else mask_id
    tokens = np.concatenate([np.asarray(prompt, np.int64), np.full(gen_len, mid, np.int64)])
    masked = np.zeros(n, bool)
    masked[P:] = True
    d = dims.d
    return SeqState(tokens=tokens, masked=masked, prompt_len=P,
                    conf=np.zeros(n, F64), argmax=np.zeros(n, np.int64),
                    h_prev=np.zeros((n, d), F64),
                    K=[np.zeros((n, d), F64) for _ in range(dims.n_layers)],
                    V=[np.zeros((n, d), F64) for _ in range(dims.n_layers)],
                    h_final=np.zeros((n, d), F64),
                    logits=np.zeros((n, dims.vocab), F64) if keep_logits else None,
                    h_prev2=np.zeros((n, d), F64),
                    Q=[np.zeros((n, d), F64) for _ in range(dims.n_layers)],
                    C=[np.zeros((n, d), F64) for _ in range(dims.n_layers)],
                    LSE=[np.zeros((n, dims.n_heads), F64) for _ in range(dims.n_layers)],
                    Y=[np.zeros((n, d), F64) for _ in range(dims.n_layers)])


def is_refresh_step(step: int, sched) -> bool:
    """Refresh at each block's first step, and every refresh_interval steps."""
    sib = step % sched.steps_per_block
    if sib == 0:
        return True
    return sched.refresh_interval > 0 and sib % sched.refresh_interval == 0


def scored_tensor(which: str, x: np.ndarray, pos: np.ndarray, lw: dict, dims) -> np.ndarray:
    """The tensor whose change eq. I measures, for rows x = X_s at positions pos
    (ES-dLLM section 2A: hidden states, keys or values): X_s itself, or layer
    s's key rows RoPE(n(X_s) Wk^T) / value rows n(X_s) Wv^T."""
    if which == "hidden":
        return np.asarray(x, F64)
    xn = rms_norm(x, lw["attn_norm"], dims.rms_eps)
    if which == "key":
        return rope(xn @ np.asarray(lw["wk"], F64).T, pos, dims.n_heads, dims.head_dim, dims.rope_base)
    if which == "value":
        return xn @ np.asarray(lw["wv"], F64).T
    raise ValueError(f"unknown scored tensor {which!r}")


def is_full_context_step(step: int, sched) -> bool:
    """DyLLM response-only strategy: with an interval N > 0, a skip step takes
    every row only when its in-block index is a multiple of N."""
    N = getattr(sched, "response_interval", 0)
    return N <= 0 or (step % sched.steps_per_block) % N == 0


def candidate_rows(st: SeqState, response_only: bool) -> np.ndarray:
    """Rows that go through the prefix layers and may be kept: every row, or
    the response rows [prompt_len, n) on a response-only step."""
    n = st.tokens.shape[0]
    return np.arange(st.prompt_len if response_only else 0, n, dtype=np.int64)


def level2_count(keep2: float, n_cand: int, n_kept1: int) -> int:
    """Rows kept at the second skip layer: k = (1 - r_l)|S| on the step's
    candidate count, never more than the first level kept."""
    if n_kept1 <= 0:
        return 0
    return min(keep_count(keep2, n_cand), n_kept1)


@dataclass
class StepInfo:
    refresh: bool
    selected: np.ndarray          # rows recomputed in layers >= s (ascending)
    scores: Optional[np.ndarray]  # fp64 scores [n] (skip steps only; -inf for non-candidates)
    unmasked: np.ndarray          # positions unmasked by this step
    selected2: Optional[np.ndarray] = None   # rows recomputed in layers >= s2 (two levels)
    scores2: Optional[np.ndarray] = None     # fp64 second-level scores [n] (-inf outside `selected`)
    response_only: bool = False
    layer_selected: Optional[list] = None    # per-layer variant: rows through O-proj + FFN of each layer >= s
    layer_scores: Optional[list] = None      # per-layer variant: 1 - cos of each layer's context change


def _positions_in(rows_all: np.ndarray, chosen) -> np.ndarray:
    """Indices into the ascending array ``rows_all`` of the ascending subset
    ``chosen`` (an error if ``chosen`` is not such a subset)."""
    chosen = np.asarray(chosen, np.int64)
    idx = np.searchsorted(rows_all, chosen)
    assert idx.size == 0 or (idx.max() < rows_all.size and np.array_equal(rows_all[idx], chosen)), \
        "forced rows are not a subset of the candidates"
    assert np.all(np.diff(chosen) > 0), "forced rows must be strictly ascending"
    return idx.astype(np.int64)


def denoise_step(model: dict, dims, st: SeqState, step: int, sched, mode: str = "topk",
                 threshold: float = 0.0, force_refresh: Optional[bool] = None,
                 keep: Optional[float] = None, response_only: Optional[bool] = None,
                 mode2: str = "topk", threshold2: float = 0.0, mode_l: str = "topk",
                 threshold_l: float = 0.0, force_sel=None, force_sel2=None,
                 force_layer_sel=None, x_s=None) -> StepInfo:
    """One denoising step of one sequence (ES-dLLM section 2B).

    Refresh step: every row through every layer; all caches rewritten.
    Skip step: layers [0, s) on the candidate rows (every row, or the response
    rows on a response-only step) give X_s; score X_s against h_prev with the
    cached confidence; keep the top-k (or threshold) rows; h_prev <- X_s for
    the candidates; layers [s, L) on the kept rows only, each layer scattering
    their fresh K/V into its cache first; LM head on the kept rows; scatter
    conf, argmax, h_final (and logits) for kept rows only.  Then unmask.
    With a second skip layer s2, layers [s, s2) run on the first level's rows,
    which are scored again at the input of s2 against h_prev2; only the second
    level's rows go through [s2, L) and the LM head.  With the per-layer
    variant (DyLLM section 2B), every layer from s on re-selects its salient
    rows by the change of the attention context (``_per_layer``).

    ``force_sel`` / ``force_sel2`` / ``force_layer_sel`` (one array per layer
    from s) belong to the comparison protocol, not to the method: a skip step
    then keeps the given rows instead of deciding them itself.  The scores are
    still computed and returned, so a caller can check the given sets against
    them; every other computation is unchanged.  ``x_s`` (comparison protocol
    as well) gives the skip layer's input of the candidate rows [n_cand, d]:
    layers [0, s) are then not run (their caches are per-step scratch) and the
    step goes on from those rows, so that a later stage can be compared from
    the same input as another implementation's.
    """
    n = st.tokens.shape[0]
    s_layer = sched.skip_layer
    s2 = getattr(sched, "skip_layer2", 0)
    L = dims.n_layers
    refresh = is_refresh_step(step, sched) if force_refresh is None else force_refresh
    if response_only is None:
        response_only = not is_full_context_step(step, sched)
    response_only = bool(response_only) and not refresh
    keep = sched.keep if keep is None else keep
    cand = candidate_rows(st, response_only)

    if x_s is None:
        x = np.asarray(model["embed"], F64)[st.tokens[cand]]     # [n_cand, d]
        for li in range(s_layer):
            x = layer_forward(x, cand, model["layers"][li], st.K[li], st.V[li], n, dims)
    else:
        x = np.array(x_s, F64, copy=True)
        assert x.shape == (cand.size, dims.d), "x_s must hold the skip-layer input of every candidate row"

    which = getattr(sched, "score_tensor", "hidden")
    assert which == "hidden" or s_layer < L, "a key/value score needs layer s to exist"
    T = scored_tensor(which, x, cand, model["layers"][s_layer], dims) if which != "hidden" else x
    scores = None
    if refresh:
        idx = np.arange(cand.size, dtype=np.int64)
    else:
        sc = score_rows(sched.score, T, st.h_prev[cand], st.conf[cand], sched.alpha)
        scores = np.full(n, -np.inf)
        scores[cand] = sc
        if force_sel is not None:
            idx = _positions_in(cand, force_sel)
        elif mode == "topk":
            idx = select_topk(sc, keep_count(keep, cand.size))
        else:
            idx = select_threshold(sc, threshold)
    sel = cand[idx]
    st.h_prev[cand] = T                                       # every candidate row

    xr = x[idx]
    if getattr(sched, "per_layer", False):
        assert s_layer < L and getattr(sched, "skip_layer2", 0) == 0 and not response_only
        rows, xr, lsel, lsc = _per_layer(model, dims, st, sched, sel, xr, x, refresh, mode_l, threshold_l,
                                         force_layer_sel)
        return _finish_step(model, dims, st, step, sched, rows, xr, StepInfo(
            refresh=refresh, selected=sel, scores=scores, unmasked=None, layer_selected=lsel, layer_scores=lsc))
    sel2, scores2, l_rest = None, None, s_layer
    if s2 > 0:
        for li in range(s_layer, s2):
            xr = layer_forward(xr, sel, model["layers"][li], st.K[li], st.V[li], n, dims)
        if refresh:
            idx2 = np.arange(sel.size, dtype=np.int64)
        else:
            sc2 = score_rows(sched.score, xr, st.h_prev2[sel], st.conf[sel], sched.alpha)
            scores2 = np.full(n, -np.inf)
            scores2[sel] = sc2
            if force_sel2 is not None:
                idx2 = _positions_in(sel, force_sel2)
            elif mode2 == "topk":
                idx2 = select_topk(sc2, level2_count(sched.keep2, cand.size, sel.size))
            else:
                idx2 = select_threshold(sc2, threshold2)
        st.h_prev2[sel] = xr                                  # every first-level row
        sel2 = sel[idx2]
        xr = xr[idx2]
        l_rest = s2
    rows = sel if sel2 is None else sel2
    for li in range(l_rest, L):
        xr = layer_forward(xr, rows, model["layers"][li], st.K[li], st.V[li], n, dims)
    return _finish_step(model, dims, st, step, sched, rows, xr, StepInfo(
        refresh=refresh, selected=sel, scores=scores, unmasked=None, selected2=sel2, scores2=scores2,
        response_only=response_only))


def _finish_step(model, dims, st, step, sched, rows, xr, info: StepInfo) -> StepInfo:
    """LM head on the rows that went through every layer, scatter of their
    confidence, argmax, final state (and logits), then unmasking."""
    n = st.tokens.shape[0]
    if rows.size:
        logits = lm_logits(xr, model["final_norm"], model["lm_head"], dims.rms_eps)
        conf, amax = conf_argmax(logits)
        st.conf[rows] = conf
        st.argmax[rows] = amax
        st.h_final[rows] = xr
        if st.logits is not None:
            st.logits[rows] = logits

    b = step // sched.steps_per_block
    lo = st.prompt_len + b * sched.block_len
    hi = min(lo + sched.block_len, n)
    pos = unmask(st.masked, st.conf, lo, hi, sched.per_step)
    st.tokens[pos] = st.argmax[pos]
    st.masked[pos] = False
    info.unmasked = pos
    return info


def _per_layer(model, dims, st, sched, A, xA, X_s, refresh, mode_l, threshold_l, force_layer_sel=None):
    """Layers [s, L) of the per-layer variant (DyLLM section 2B).  A: the rows
    whose input of layer s is fresh (every row on a refresh step), xA their
    inputs.  Returns (rows through the last layer, their outputs, the salient
    rows of each layer, each layer's scores).  ``force_layer_sel[l - s]``,
    when given, replaces the salient set of layer l (comparison protocol)."""
    n = st.tokens.shape[0]
    H, dh = dims.n_heads, dims.head_dim
    s_layer, L = sched.skip_layer, dims.n_layers
    keep_l = getattr(sched, "keep_layer", 0.0) or sched.keep
    lsel, lsc = [], []
    for li in range(s_layer, L):
        lw = model["layers"][li]
        if refresh:
            y, q, ctx, lse = layer_parts(xA, A, lw, st.K[li], st.V[li], n, dims)
            st.Q[li][A], st.C[li][A], st.LSE[li][A], st.Y[li][A] = q, ctx, lse, y
            lsel.append(A)
            lsc.append(None)
            xA = y
            continue
        K_old = st.K[li][A].copy()
        V_old = st.V[li][A].copy()
        y_unused, q, ctx, lse = layer_parts(xA, A, lw, st.K[li], st.V[li], n, dims)
        C_new = approx_context(st.C[li], st.Q[li], st.LSE[li], K_old, st.V[li][A] - V_old, H, dh)
        C_new[A] = ctx
        sig = score_rows("cosine", C_new, st.C[li], st.conf)
        if force_layer_sel is not None:
            R = _positions_in(np.arange(n, dtype=np.int64), force_layer_sel[li - s_layer])
        elif mode_l == "topk":
            R = select_topk(sig, keep_count(keep_l, n))
        else:
            R = select_threshold(sig, threshold_l)
        st.C[li] = C_new
        st.Q[li][A] = q
        st.LSE[li][A] = lse
        y = finish_layer(layer_input_rows(st, X_s, li, s_layer, R), C_new[R], lw, dims)
        st.Y[li][R] = y
        lsel.append(R)
        lsc.append(sig)
        A, xA = R, y
    return A, xA, lsel, lsc


def decode(model: dict, dims, prompt: np.ndarray, sched, n_steps: Optional[int] = None,
           vanilla: bool = False, keep_logits: bool = False, mode: str = "topk",
           threshold: float = 0.0, mode2: str = "topk", threshold2: float = 0.0, mode_l: str = "topk",
           threshold_l: float = 0.0):
    """Run the decode loop.  ``vanilla`` refreshes every step (full recompute)."""
    st = init_state(prompt, sched.gen_len, dims, keep_logits=keep_logits)
    infos = []
    T = sched.steps if n_steps is None else n_steps
    for t in range(T):
        infos.append(denoise_step(model, dims, st, t, sched, mode=mode, threshold=threshold,
                                  force_refresh=True if vanilla else None, mode2=mode2,
                                  threshold2=threshold2, mode_l=mode_l, threshold_l=threshold_l))
    return st, infos
