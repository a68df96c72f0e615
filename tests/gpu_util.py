"""Helpers shared by the GPU parity tests: model conversion, the per-row
relative error, and the tie-band comparison of selections."""
from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import esdllm as E


def np_model(m: dict) -> dict:
    """Exact float64 host copy of a model dict of torch tensors."""
    out = {k: workloads.host_f64(v) for k, v in m.items() if k != "layers"}
    out["layers"] = [{k: workloads.host_f64(v) for k, v in lw.items()} for lw in m["layers"]]
    return out


def to_device(m: dict, device="cuda") -> dict:
    out = {k: v.to(device) for k, v in m.items() if k != "layers"}
    out["layers"] = [{k: v.to(device) for k, v in lw.items()} for lw in m["layers"]]
    return out


def row_rel_err(gpu, ref) -> float:
    """max over rows of ||g - o||_inf / max(||o||_inf, 1e-6)."""
    g = np.asarray(gpu, np.float64).reshape(len(gpu), -1) if np.ndim(gpu) > 1 else np.asarray(gpu, np.float64)[:, None]
    o = np.asarray(ref, np.float64).reshape(g.shape)
    if g.size == 0:
        return 0.0
    num = np.abs(g - o).max(axis=1)
    den = np.maximum(np.abs(o).max(axis=1), 1e-6)
    return float((num / den).max())


def lse_err(gpu, ref) -> float:
    """max over elements of |g - o| / max(|o|, 1): log normalisers are
    compared absolutely near zero and relatively beyond."""
    g = np.asarray(gpu, np.float64)
    o = np.asarray(ref, np.float64).reshape(g.shape)
    if g.size == 0:
        return 0.0
    return float((np.abs(g - o) / np.maximum(np.abs(o), 1.0)).max())


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


# Selected sets may differ only on ties within this band of the k-th score
# (1e-4 absolute), decided on identical inputs: the oracle's score function
# applied to the very rows the kernels scored.
SEL_BAND = 1e-4


def topk_within_band(g_rows, cand, scores, k, band=SEL_BAND):
    """g_rows (ascending positions) against the top-k of ``scores`` (one per
    position of ``cand``; decided in float32, lower index on ties): they may
    differ only on positions whose score lies within ``band`` of the k-th.
    Returns (ok, number of differing positions, the oracle's set)."""
    cand = np.asarray(cand, np.int64)
    o_rows = cand[E.select_topk(scores, k)]
    a, b = set(map(int, g_rows)), set(map(int, o_rows))
    if a == b:
        return True, 0, o_rows
    s32 = dict(zip(cand.tolist(), np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)))
    kth = np.sort(np.array(list(s32.values())))[::-1][k - 1]
    bad = [i for i in a ^ b if i not in s32 or abs(s32[i] - kth) > band]
    return not bad, len(a ^ b), o_rows


def threshold_within_band(g_rows, cand, scores, tau, band=SEL_BAND):
    """g_rows against {cand : float32 score > float32 tau}, except rows whose
    score lies within ``band`` of tau."""
    cand = np.asarray(cand, np.int64)
    o_rows = cand[E.select_threshold(scores, tau)]
    a, b = set(map(int, g_rows)), set(map(int, o_rows))
    s32 = dict(zip(cand.tolist(), np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)))
    bad = [i for i in a ^ b if i not in s32 or abs(s32[i] - float(np.float32(tau))) > band]
    return not bad, len(a ^ b), o_rows


def check_scores_exact_inputs(g_scores, x_now, h_before, conf_before, kind, alpha, cand, rtol=1e-5):
    """The kernel's scores of the rows ``cand`` against the oracle's score
    function on the kernel's own inputs (x_now: the scored rows as the kernel
    read them, h_before / conf_before: the caches before the step).  Returns
    the oracle's scores (fp64, one per position of cand)."""
    cand = np.asarray(cand, np.int64)
    s = E.score_rows(kind, np.asarray(x_now)[cand], np.asarray(h_before)[cand], np.asarray(conf_before)[cand],
                     alpha)
    g = np.asarray(g_scores, np.float64)[cand]
    err = np.abs(g - s).max(initial=0.0)
    assert err <= rtol * max(1.0, np.abs(s).max(initial=0.0)), f"scores differ by {err}"
    return s


def implied_band_ok(g_rows, o_rows, s_exact, s_orc, cand, k):
    """The oracle's own selection (from its own inputs) against the GPU's.
    Both score functions are the oracle's; they differ only through their
    inputs, by at most delta = max |s_exact - s_orc|.  The GPU's set is the
    top-k of s_exact within SEL_BAND, so every differing row's own score lies
    within SEL_BAND + 2 delta of the oracle's k-th score.  Returns (ok, delta)."""
    cand = np.asarray(cand, np.int64)
    s_orc = np.asarray(s_orc, np.float64)
    delta = float(np.abs(np.asarray(s_exact, np.float64) - s_orc).max(initial=0.0))
    a, b = set(map(int, g_rows)), set(map(int, o_rows))
    if a == b:
        return True, delta
    s32 = dict(zip(cand.tolist(), s_orc.astype(np.float32).astype(np.float64)))
    kth = np.sort(np.array(list(s32.values())))[::-1][k - 1]
    band = SEL_BAND + 2.0 * delta + 1e-7 * max(1.0, abs(kth))
    bad = [i for i in a ^ b if abs(s32[i] - kth) > band]
    return not bad, delta


def check_unmask_exact_inputs(masked_before, tokens_before, masked_after, tokens_after, conf_after, argmax_after,
                              lo, hi, n_unmask):
    """The positions the GPU unmasked are exactly the oracle's unmask of the
    GPU's own confidences (float32, lower index on ties, current block only),
    and each took the GPU's argmax.  Returns those positions."""
    want = E.unmask(np.asarray(masked_before, bool), np.asarray(conf_after, np.float64), lo, hi, n_unmask)
    got = np.nonzero(np.asarray(masked_before, bool) & ~np.asarray(masked_after, bool))[0]
    assert got.tolist() == want.tolist(), (got.tolist(), want.tolist())
    assert not (~np.asarray(masked_before, bool) & np.asarray(masked_after, bool)).any()
    exp_tok = np.asarray(tokens_before).copy()
    exp_tok[want] = np.asarray(argmax_after)[want]
    assert np.array_equal(np.asarray(tokens_after), exp_tok)
    return got


def check_lm_rows_exact_inputs(logits_rows, conf_rows, argmax_rows, rtol=1e-5):
    """Confidence and argmax of the LM epilogue against the oracle's
    conf_argmax of the GPU's own fp32 logits."""
    c, a = E.conf_argmax(np.asarray(logits_rows, np.float64))
    assert np.array_equal(np.asarray(argmax_rows, np.int64), a)
    if c.size:
        err = float(np.abs(np.asarray(conf_rows, np.float64) - c).max() / max(c.max(), 1e-30))
        assert err <= rtol, err


def snapshot(dec, names=("tokens", "masked", "h_prev", "h_prev2", "conf", "argmax", "ctx_cache", "y_cache")):
    """Host float64 / integer copies of the decode state before a step."""
    out = {}
    for k in names:
        v = getattr(dec, k, None)
        if v is None:
            continue
        out[k] = v.detach().cpu().numpy() if not v.is_floating_point() else host(v)
    return out


def sync_from_oracle(dec, b: int, st) -> None:
    """Overwrite sequence b of the GPU decode state with the oracle's state
    (rounded to the storage type): the next step then starts from the same
    inputs on both sides.  Data flows oracle -> GPU only."""
    n = len(st.tokens)
    dev = dec.tokens.device
    dt = dec.h_prev.dtype

    def put(dst, src, dtype=None):
        dst.copy_(torch.as_tensor(np.asarray(src), device=dev).to(dtype or dst.dtype))

    put(dec.tokens[b, :n], st.tokens.astype(np.int32))
    put(dec.masked[b, :n], st.masked.astype(np.uint8))
    put(dec.conf[b, :n], st.conf.astype(np.float32))
    put(dec.argmax[b, :n], st.argmax.astype(np.int32))
    put(dec.h_prev[b, :n], st.h_prev.astype(np.float32), dt)
    put(dec.h_final[b, :n], st.h_final.astype(np.float32), dt)
    for li in range(len(st.K)):
        put(dec.k_cache[li, b, :n], st.K[li].astype(np.float32), dt)
        put(dec.v_cache[li, b, :n], st.V[li].astype(np.float32), dt)
    if dec.logits is not None and st.logits is not None:
        put(dec.logits[b, :n], st.logits.astype(np.float32))
    if getattr(dec, "h_prev2", None) is not None and st.h_prev2 is not None:
        put(dec.h_prev2[b, :n], st.h_prev2.astype(np.float32), dt)
    if getattr(dec, "ctx_cache", None) is not None and st.C is not None:
        for li in range(len(st.C)):
            put(dec.q_cache[li, b, :n], st.Q[li].astype(np.float32), dt)
            put(dec.ctx_cache[li, b, :n], st.C[li].astype(np.float32))
            put(dec.lse_cache[li, b, :n], st.LSE[li].astype(np.float32))
            put(dec.y_cache[li, b, :n], st.Y[li].astype(np.float32))
def _rows_same_band(g_rows, o_rows, s_exact, s_orc, cand, k, what):
    ok, delta = implied_band_ok(g_rows, o_rows, s_exact, s_orc, cand, k)
    assert ok, f"{what}: the oracle's own selection differs outside SEL_BAND + 2 delta (delta {delta})"
    return delta


def bf16_step(dec, m_np, dims, sts, t, sched, tol=2e-2):
    """One step of every sequence, compared with the oracle from a shared
    snapshot (the bf16 protocol):

    1. the oracle's state is copied to the GPU (oracle -> GPU only) and the
       GPU runs the step;
    2. exact inputs: the GPU's scores equal the oracle's score function on the
       rows the GPU scored (h_prev after the step) against the caches before
       it, and its kept sets are their top-k within SEL_BAND; likewise the
       second level; the unmasked positions are exactly the oracle's unmask of
       the GPU's confidences; conf / argmax follow the GPU's logits;
    3. the oracle runs the same step with the GPU's kept sets forced, and
       every value is compared (scored rows, K/V of every layer, final hidden
       state, logits and confidence of the recomputed rows) within ``tol``;
       the oracle's own selections and unmasking may differ from the GPU's only
       within SEL_BAND + twice the measured score difference.
    Returns the largest measured score difference of the step."""
    two = getattr(sched, "skip_layer2", 0) > 0
    for b, st in enumerate(sts):
        sync_from_oracle(dec, b, st)
    before = snapshot(dec)
    dec.step(t)
    torch.cuda.synchronize()
    after = snapshot(dec, ("tokens", "masked", "h_prev", "h_prev2", "conf", "argmax", "scores", "scores2"))
    lg = host(dec.logits)
    g1 = dec.sel.rows()
    g2 = dec.sel2.rows() if two else g1
    refresh = E.is_refresh_step(t, sched)
    resp = (not refresh) and not E.is_full_context_step(t, sched)
    deltas = [0.0]
    for b, st in enumerate(sts):
        n = len(st.tokens)
        cand = np.arange(st.prompt_len if resp else 0, n, dtype=np.int64)
        kw = {}
        if refresh:
            assert g1[b] == list(range(n)) and g2[b] == list(range(n)), (t, b)
        else:
            s1 = check_scores_exact_inputs(after["scores"][b], after["h_prev"][b], before["h_prev"][b],
                                           before["conf"][b], sched.score, sched.alpha, cand)
            assert np.all(np.isneginf(after["scores"][b][np.setdiff1d(np.arange(n), cand)])), (t, b)
            k1 = E.keep_count(sched.keep, cand.size)
            ok, _, _ = topk_within_band(g1[b], cand, s1, k1)
            assert ok, (t, b, "level 1 against its own inputs")
            kw["force_sel"] = np.asarray(g1[b], np.int64)
            if two:
                r1 = np.asarray(g1[b], np.int64)
                s2 = check_scores_exact_inputs(after["scores2"][b], after["h_prev2"][b], before["h_prev2"][b],
                                               before["conf"][b], sched.score, sched.alpha, r1)
                k2 = E.level2_count(sched.keep2, cand.size, r1.size)
                ok, _, _ = topk_within_band(g2[b], r1, s2, k2)
                assert ok, (t, b, "level 2 against its own inputs")
                assert set(g2[b]) <= set(g1[b])
                kw["force_sel2"] = np.asarray(g2[b], np.int64)
        info = E.denoise_step(m_np, dims, st, t, sched, **kw)
        if not refresh:
            deltas.append(_rows_same_band(g1[b], cand[E.select_topk(info.scores[cand], k1)], s1, info.scores[cand],
                                          cand, k1, f"step {t} seq {b} level 1"))
            if two:
                r1 = np.asarray(g1[b], np.int64)
                deltas.append(_rows_same_band(g2[b], r1[E.select_topk(info.scores2[r1], k2)], s2, info.scores2[r1],
                                              r1, k2, f"step {t} seq {b} level 2"))
        rows = np.asarray(g2[b], np.int64)
        # values of the same step on both sides
        assert row_rel_err(after["h_prev"][b, :n], st.h_prev) <= tol, (t, b, "h_prev")
        if two:
            assert row_rel_err(after["h_prev2"][b, :n], st.h_prev2) <= tol, (t, b, "h_prev2")
        for li in range(dims.n_layers):
            assert row_rel_err(host(dec.k_cache[li, b, :n]), st.K[li]) <= tol, (t, b, li, "K")
            assert row_rel_err(host(dec.v_cache[li, b, :n]), st.V[li]) <= tol, (t, b, li, "V")
        assert row_rel_err(host(dec.h_final[b, :n])[rows], st.h_final[rows]) <= tol, (t, b, "h_final")
        assert row_rel_err(lg[b, :n][rows], st.logits[rows]) <= tol, (t, b, "logits")
        assert row_rel_err(after["conf"][b, :n][rows], st.conf[rows]) <= tol, (t, b, "conf")
        check_lm_rows_exact_inputs(lg[b, :n][rows], after["conf"][b, :n][rows], after["argmax"][b, :n][rows])
        # unmasking: exact on the GPU's confidences; the oracle's own choice
        # within the band of the confidences' measured difference
        blk = t // sched.steps_per_block
        lo = st.prompt_len + blk * sched.block_len
        hi = min(lo + sched.block_len, n)
        got = check_unmask_exact_inputs(before["masked"][b, :n], before["tokens"][b, :n], after["masked"][b, :n],
                                        after["tokens"][b, :n], after["conf"][b, :n], after["argmax"][b, :n], lo,
                                        hi, sched.per_step)
        assert len(got) == len(info.unmasked)
        mc = np.nonzero(before["masked"][b, :n].astype(bool))[0]
        mc = mc[(mc >= lo) & (mc < hi)]
        if mc.size and len(got):
            _rows_same_band(got, info.unmasked, after["conf"][b, :n][mc], st.conf[mc], mc, len(got),
                            f"step {t} seq {b} unmask")
    return max(deltas)
