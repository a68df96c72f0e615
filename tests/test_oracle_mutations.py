"""Planted mistakes in the oracle must each make some pin fail.

Every mutant below is a plausible slip (a dropped term, a wrong sign, a wrong
index or tie rule, a cache written after use, a transposed operand).  The
mutant is planted in the oracle module, on the CPU, for the duration of one
test; the test passes only if at least one pin raises.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import esdllm as E

_orig = {name: getattr(E, name) for name in ("score_rows", "rms_norm", "rope", "attention", "select_topk",
                                             "unmask", "keep_count", "conf_argmax", "silu", "layer_forward",
                                             "select_threshold", "candidate_rows", "level2_count",
                                             "is_full_context_step", "scored_tensor", "approx_context",
                                             "attention_lse", "layer_input_rows", "finish_layer",
                                             "is_refresh_step", "_positions_in")}


def m_score_l2(kind, x, h, c, alpha=0.5):          # L2 instead of L1 in eq. I
    if kind != "esdllm":
        return _orig["score_rows"](kind, x, h, c, alpha)
    d = x.shape[1]
    num = np.sqrt(((x - h) ** 2).sum(1))
    return alpha * c + (1 - alpha) * num / np.maximum(np.sqrt(d) * np.sqrt((h * h).sum(1)), E.FLT_MIN)


def m_score_csign(kind, x, h, c, alpha=0.5):       # confidence enters with the wrong sign
    return _orig["score_rows"](kind, x, h, -np.asarray(c) if kind == "esdllm" else c, alpha)


def m_score_nosqrtd(kind, x, h, c, alpha=0.5):     # sqrt(d) dropped from the denominator
    s = _orig["score_rows"](kind, x, h, c, alpha)
    if kind == "esdllm":
        s = alpha * np.asarray(c) + (s - alpha * np.asarray(c)) * np.sqrt(x.shape[1])
    return s


def m_rms_noeps(x, g, eps):
    return _orig["rms_norm"](x, g, 0.0)


def m_rope_sign(x, pos, H, dh, base):              # rotation by -theta
    return _orig["rope"](x, -np.asarray(pos), H, dh, base)


def m_rope_pairs(x, pos, H, dh, base):             # wrong frequency index (j+1)
    return _orig["rope"](x, pos, H, dh, base * 1.5)


def m_attn_noscale(q, K, V, H, dh):
    return _orig["attention"](np.asarray(q) * np.sqrt(dh), K, V, H, dh)


def m_attn_swap(q, K, V, H, dh):                   # keys and values transposed in role
    return _orig["attention"](q, V, K, H, dh)


def m_topk_hi_tie(scores, k):                      # ties to the higher index
    s32 = np.asarray(scores).astype(np.float32)
    n = len(s32)
    order = np.lexsort((-np.arange(n), -s32.astype(np.float64)))
    return np.sort(order[:k])


def m_topk_low(scores, k):                         # the k lowest instead of the highest
    return _orig["select_topk"](-np.asarray(scores), k)


def m_unmask_noblock(masked, conf, lo, hi, n):     # ignores the block boundary
    return _orig["unmask"](masked, conf, 0, len(masked), n)


def m_unmask_lowconf(masked, conf, lo, hi, n):
    return _orig["unmask"](masked, -np.asarray(conf), lo, hi, n)


def m_keep_floor(keep, n):
    return max(1, min(n, int(np.floor(float(np.float32(keep)) * n))))


def m_conf_maxlogit(logits):                       # softmax forgotten
    c, a = _orig["conf_argmax"](logits)
    return np.asarray(logits).max(1), a


def m_silu_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def m_layer_kv_late(x, pos, lw, K_cache, V_cache, n_valid, dims):   # cache written after attention
    Kold, Vold = K_cache.copy(), V_cache.copy()
    _orig["layer_forward"](x, pos, lw, K_cache, V_cache, n_valid, dims)   # fills the fresh rows
    Knew, Vnew = K_cache.copy(), V_cache.copy()
    H, dh = dims.n_heads, dims.head_dim
    xn = E.rms_norm(x, lw["attn_norm"], dims.rms_eps)
    q = E.rope(xn @ np.asarray(lw["wq"]).T, pos, H, dh, dims.rope_base)
    o = E.attention(q, Kold[:n_valid], Vold[:n_valid], H, dh)          # stale keys for the fresh rows
    h = x + o @ np.asarray(lw["wo"]).T
    hn = E.rms_norm(h, lw["ffn_norm"], dims.rms_eps)
    K_cache[:], V_cache[:] = Knew, Vnew
    return h + (E.silu(hn @ np.asarray(lw["w_gate"]).T) * (hn @ np.asarray(lw["w_up"]).T)) @ np.asarray(lw["w_down"]).T


def m_threshold_ge(scores, tau):
    s32 = np.asarray(scores).astype(np.float32)
    return np.nonzero(s32 >= np.float32(tau) - np.float32(0.05))[0]


def m_cand_all(st, response_only):                  # prompt rows scored on response-only steps
    return _orig["candidate_rows"](st, False)


def m_cand_shift(st, response_only):                # response rows start one late
    c = _orig["candidate_rows"](st, response_only)
    return c[1:] if response_only else c


def m_full_context_always(step, sched):             # response-only steps never happen
    return True


def m_level2_of_kept(keep2, n_cand, n_kept1):       # second ratio taken of the first level's count
    return _orig["keep_count"](keep2, n_kept1) if n_kept1 > 0 else 0


def m_key_from_wq(which, x, pos, lw, dims):         # query projection scored as the key
    if which == "key":
        lw = dict(lw, wk=lw["wq"])
    return _orig["scored_tensor"](which, x, pos, lw, dims)


def m_key_unrotated(which, x, pos, lw, dims):       # keys scored before RoPE
    if which == "key":
        return E.rms_norm(x, lw["attn_norm"], dims.rms_eps) @ np.asarray(lw["wk"]).T
    return _orig["scored_tensor"](which, x, pos, lw, dims)


def m_kv_unnormed(which, x, pos, lw, dims):         # projection of X_s without its RMSNorm
    if which == "value":
        return np.asarray(x) @ np.asarray(lw["wv"]).T
    return _orig["scored_tensor"](which, x, pos, lw, dims)


def m_approx_sign(C, q, lse, K_act, dV_act, H, dh):   # the value change subtracted
    return _orig["approx_context"](C, q, lse, K_act, -np.asarray(dV_act), H, dh)


def m_approx_nolse(C, q, lse, K_act, dV_act, H, dh):  # probabilities left unnormalised
    return _orig["approx_context"](C, q, np.zeros_like(np.asarray(lse)), K_act, dV_act, H, dh)


def m_lse_noscale(q, K, H, dh):                       # normaliser of unscaled scores
    return _orig["attention_lse"](np.asarray(q) * np.sqrt(dh), K, H, dh)


def m_input_always_xs(st, X_s, layer, s_layer, rows):  # every layer fed the skip-layer input
    return np.asarray(X_s)[rows]


def m_finish_noresid(x, ctx, lw, dims):               # attention residual dropped
    return _orig["finish_layer"](np.zeros_like(np.asarray(x)), ctx, lw, dims)


def m_refresh_no_interval(step, sched):            # the refresh interval ignored
    return step % sched.steps_per_block == 0


def m_refresh_interval_off_by_one(step, sched):    # every (N+1)-th in-block step instead of every N-th
    sib = step % sched.steps_per_block
    return sib == 0 or (sched.refresh_interval > 0 and sib % (sched.refresh_interval + 1) == 0)


def m_forced_shift(rows_all, chosen):               # forced rows taken one candidate late
    idx = _orig["_positions_in"](rows_all, chosen)
    return np.minimum(idx + 1, len(rows_all) - 1)


MUTANTS = [
    ("score_rows", m_score_l2), ("score_rows", m_score_csign), ("score_rows", m_score_nosqrtd),
    ("rms_norm", m_rms_noeps), ("rope", m_rope_sign), ("rope", m_rope_pairs),
    ("attention", m_attn_noscale), ("attention", m_attn_swap),
    ("select_topk", m_topk_hi_tie), ("select_topk", m_topk_low),
    ("unmask", m_unmask_noblock), ("unmask", m_unmask_lowconf), ("keep_count", m_keep_floor),
    ("conf_argmax", m_conf_maxlogit), ("silu", m_silu_sigmoid), ("layer_forward", m_layer_kv_late),
    ("select_threshold", m_threshold_ge),
    ("candidate_rows", m_cand_all), ("candidate_rows", m_cand_shift),
    ("is_full_context_step", m_full_context_always), ("level2_count", m_level2_of_kept),
    ("scored_tensor", m_key_from_wq), ("scored_tensor", m_key_unrotated), ("scored_tensor", m_kv_unnormed),
    ("approx_context", m_approx_sign), ("approx_context", m_approx_nolse), ("attention_lse", m_lse_noscale),
    ("layer_input_rows", m_input_always_xs), ("finish_layer", m_finish_noresid),
    ("is_refresh_step", m_refresh_no_interval), ("is_refresh_step", m_refresh_interval_off_by_one),
    ("_positions_in", m_forced_shift),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(E, name, mutant)
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:  # a crash also exposes the mutant
            failed.append(f"{pin.__name__}:{type(e).__name__}")
    assert failed, f"no pin caught mutant {mutant.__name__} of {name}"
