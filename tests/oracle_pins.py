"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
hand-worked value (``tests/golden/``), a closed form, a brute force on tiny
inputs, a torch library routine (``libref``), or an invariant the pages fix.
They look the oracle up through the module object at call time, so the
planted-mistake test can patch a function and check that some pin fails.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

import libref
import workloads
from oracle import esdllm as E

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "score_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def micro_dims(n_layers=3):
    return workloads.ModelDims(d=32, n_heads=2, head_dim=16, d_ffn=48, vocab=40, n_layers=n_layers)


def np_model(dims, seed=5):
    m = workloads.make_model(dims, seed, "f32", "cpu")
    out = {"embed": workloads.host_f64(m["embed"]), "final_norm": workloads.host_f64(m["final_norm"]),
           "lm_head": workloads.host_f64(m["lm_head"]), "layers": []}
    for lw in m["layers"]:
        out["layers"].append({k: workloads.host_f64(v) for k, v in lw.items()})
    return out


def micro_sched(**kw):
    base = dict(gen_len=12, block_len=6, steps=6, skip_layer=1, keep=0.35, score="esdllm")
    base.update(kw)
    return workloads.Schedule(**base)


def close(a, b, rtol=1e-12, atol=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b).max() if a.size else 0.0
    assert err <= atol + rtol * (np.abs(b).max() if b.size else 0.0), f"max abs err {err}"


# --------------------------------------------------------------------------
# score, selection, unmasking
# --------------------------------------------------------------------------

def pin_score_golden():
    for c in golden()["cases"]:
        x = np.array([c["x"]], float)
        h = np.array([c["h"]], float)
        for kind in ("esdllm", "rell2_invconf", "cosine"):
            got = E.score_rows(kind, x, h, np.array([c["c"]]), c["alpha"])[0]
            assert abs(got - c[kind]) < 1e-12, (kind, c["why"], got, c[kind])


def pin_score_closed_forms():
    rng = np.random.default_rng(11)
    n, d = 7, 24
    h = rng.normal(size=(n, d))
    c = rng.uniform(size=n)
    # no change: only the confidence terms remain
    close(E.score_rows("esdllm", h, h, c, 0.5), 0.5 * c)
    close(E.score_rows("rell2_invconf", h, h, c), 1.0 - c)
    close(E.score_rows("cosine", h, h, c), np.zeros(n), atol=1e-14)
    # constant rows a*1 vs b*1: L1/(sqrt(d)*L2) = |a-b|/|b| = relative L2
    a, b = 1.75, -0.5
    xs, hs = np.full((1, d), a), np.full((1, d), b)
    close(E.score_rows("esdllm", xs, hs, np.zeros(1), 0.0), [abs(a - b) / abs(b)])
    close(E.score_rows("rell2_invconf", xs, hs, np.ones(1)), [abs(a - b) / abs(b)])
    # pure scaling x = (1+eps) h: relative L2 = |eps|, cosine distance 0
    for eps in (0.3, -0.2):
        close(E.score_rows("rell2_invconf", (1 + eps) * h, h, np.ones(n)), np.full(n, abs(eps)))
        close(E.score_rows("cosine", (1 + eps) * h, h, c), np.zeros(n), atol=1e-14)
    # the variation term of eq. I is scale invariant; alpha=1 keeps only c
    x = h + rng.normal(size=(n, d))
    close(E.score_rows("esdllm", 3 * x, 3 * h, c, 0.0), E.score_rows("esdllm", x, h, c, 0.0))
    close(E.score_rows("esdllm", x, h, c, 1.0), c)
    # a zero cached row stays finite (floored denominator)
    z = E.score_rows("esdllm", np.ones((1, 4)), np.zeros((1, 4)), np.zeros(1))
    assert np.isfinite(z).all() and z[0] > 1e30


def pin_keep_count():
    for c in golden()["keep_count"]:
        assert E.keep_count(c["keep"], c["n"]) == c["k"], c
    assert E.keep_count(0.5, 0) == 0


def _brute_topk(s, k):
    s32 = np.asarray(s, np.float64).astype(np.float32)
    order = sorted(range(len(s32)), key=lambda i: (-float(s32[i]), i))
    return sorted(order[:k])


def pin_select_topk():
    for c in golden()["topk"]:
        assert E.select_topk(np.array(c["scores"]), c["k"]).tolist() == c["selected"], c
    rng = np.random.default_rng(3)
    for trial in range(300):
        n = int(rng.integers(1, 17))
        s = rng.choice(np.array([0.1, 0.2, 0.2, 0.5, 0.9, -1.0]), size=n) if trial % 2 else rng.normal(size=n)
        for k in range(0, n + 1):
            got = E.select_topk(s, k).tolist()
            assert got == _brute_topk(s, k), (s, k, got)
    # exhaustive over all 3-valued score vectors of length 5
    for s in itertools.product((0.0, 0.5, 1.0), repeat=5):
        for k in range(6):
            assert E.select_topk(np.array(s), k).tolist() == _brute_topk(s, k)


def pin_select_threshold():
    rng = np.random.default_rng(4)
    for _ in range(100):
        n = int(rng.integers(0, 20))
        s = rng.normal(size=n)
        tau = float(rng.normal())
        want = [i for i in range(n) if np.float32(s[i]) > np.float32(tau)]
        assert E.select_threshold(s, tau).tolist() == want


def pin_unmask():
    for c in golden()["unmask"]:
        got = E.unmask(np.array(c["masked"]), np.array(c["conf"]), c["lo"], c["hi"], c["n"]).tolist()
        assert got == c["positions"], (c, got)
    rng = np.random.default_rng(6)
    for _ in range(200):
        n = int(rng.integers(1, 15))
        masked = rng.uniform(size=n) < 0.6
        conf = rng.choice(np.array([0.1, 0.3, 0.3, 0.8]), size=n)
        lo = int(rng.integers(0, n))
        hi = int(rng.integers(lo, n + 1))
        m = int(rng.integers(0, 5))
        cand = [i for i in range(lo, hi) if masked[i]]
        want = sorted(sorted(cand, key=lambda i: (-float(np.float32(conf[i])), i))[:m])
        assert E.unmask(masked, conf, lo, hi, m).tolist() == want


# --------------------------------------------------------------------------
# model pieces vs torch library routines and closed forms
# --------------------------------------------------------------------------

def pin_rms_norm():
    rng = np.random.default_rng(7)
    x = rng.normal(size=(5, 64)) * 3
    g = rng.normal(size=64)
    close(E.rms_norm(x, g, 1e-5), libref.rms(libref.t(x), libref.t(g), 1e-5).numpy())
    y = E.rms_norm(x, np.ones(64), 1e-5)
    ms = (x * x).mean(axis=1)
    close(np.sqrt((y * y).mean(axis=1)), np.sqrt(ms / (ms + 1e-5)))
    a = 0.01
    close(E.rms_norm(np.full((1, 8), a), np.ones(8), 1e-5), np.full((1, 8), a / math.sqrt(a * a + 1e-5)))


def pin_rope():
    rng = np.random.default_rng(8)
    H, dh = 3, 8
    x = rng.normal(size=(6, H * dh))
    pos = np.array([0, 1, 2, 5, 77, 4095])
    y = E.rope(x, pos, H, dh, 10000.0)
    close(y[0], x[0])                                      # position 0 is the identity
    close(np.linalg.norm(y.reshape(6, H, dh), axis=2), np.linalg.norm(x.reshape(6, H, dh), axis=2))
    close(y, libref.rope(libref.t(x), pos, H, dh, 10000.0).numpy())
    # q.k depends only on the position difference
    q, k = rng.normal(size=(1, dh)), rng.normal(size=(1, dh))
    dots = [(E.rope(q, np.array([p + 9]), 1, dh, 10000.0) @ E.rope(k, np.array([p]), 1, dh, 10000.0).T).item()
            for p in (0, 3, 100)]
    close(dots, [dots[0]] * 3)
    # head_dim 2: a plain rotation by angle pos
    z = E.rope(np.array([[1.0, 0.0]]), np.array([1]), 1, 2, 10000.0)
    close(z, [[math.cos(1.0), math.sin(1.0)]])


def pin_attention():
    rng = np.random.default_rng(9)
    H, dh = 2, 8
    q = rng.normal(size=(4, H * dh))
    K = rng.normal(size=(9, H * dh))
    V = rng.normal(size=(9, H * dh))
    close(E.attention(q, K, V, H, dh), libref.attn(libref.t(q), libref.t(K), libref.t(V), H, dh).numpy())
    close(E.attention(q, K[:1], V[:1], H, dh), np.repeat(V[:1], 4, axis=0))     # one key
    Ke = np.repeat(K[:1], 9, axis=0)
    close(E.attention(q, Ke, V, H, dh), np.repeat(V.mean(axis=0, keepdims=True), 4, axis=0))
    close(E.attention(np.zeros_like(q), K, V, H, dh), np.repeat(V.mean(axis=0, keepdims=True), 4, axis=0))


def pin_conf_argmax():
    V = 37
    c, a = E.conf_argmax(np.zeros((2, V)))
    close(c, [1.0 / V] * 2)
    assert a.tolist() == [0, 0]
    rng = np.random.default_rng(10)
    lg = rng.normal(size=(6, V)) * 4
    lg[3, 5] = lg[3, 20] = lg[3].max() + 1.0     # exact tie: lowest id wins
    c, a = E.conf_argmax(lg)
    tl = torch.as_tensor(lg)
    close(c, torch.softmax(tl, dim=1).max(dim=1).values.numpy())
    assert a[3] == 5
    assert a.tolist()[:3] == tl[:3].argmax(dim=1).tolist()
    assert np.all(c >= 1.0 / V) and np.all(c <= 1.0)


def pin_layer_full():
    dims = micro_dims()
    m = np_model(dims)
    rng = np.random.default_rng(12)
    n = 11
    x = rng.normal(size=(n, dims.d))
    K = np.zeros((n, dims.d))
    V = np.zeros((n, dims.d))
    y = E.layer_forward(x, np.arange(n), m["layers"][1], K, V, n, dims)
    close(y, libref.full_layer(libref.t(x), m["layers"][1], dims).numpy(), rtol=1e-11)


def pin_layer_partial():
    """Selected rows attend over a cache whose other rows are stale."""
    dims = micro_dims()
    m = np_model(dims)
    rng = np.random.default_rng(13)
    n = 13
    rows = np.array([1, 4, 5, 11])
    x = rng.normal(size=(len(rows), dims.d))
    K0 = rng.normal(size=(n, dims.d))
    V0 = rng.normal(size=(n, dims.d))
    K, V = K0.copy(), V0.copy()
    y = E.layer_forward(x, rows, m["layers"][2], K, V, n, dims)
    y_ref, K_ref, V_ref = libref.partial_layer(libref.t(x), rows, m["layers"][2], K0, V0, dims)
    close(y, y_ref.numpy(), rtol=1e-11)
    close(K, K_ref.numpy())
    close(V, V_ref.numpy())
    other = np.setdiff1d(np.arange(n), rows)
    assert np.array_equal(K[other], K0[other]) and np.array_equal(V[other], V0[other])


# --------------------------------------------------------------------------
# the decode loop: invariants the pages fix
# --------------------------------------------------------------------------

def _micro_run(sched, vanilla=False, seed=5, n_steps=None):
    dims = micro_dims()
    m = np_model(dims, seed)
    g = torch.Generator().manual_seed(seed)
    prompt = torch.randint(0, dims.vocab, (9,), generator=g).numpy()
    st, infos = E.decode(m, dims, prompt, sched, vanilla=vanilla, keep_logits=True, n_steps=n_steps)
    return dims, m, prompt, st, infos


def pin_refresh_is_full_forward():
    sched = micro_sched()
    dims = micro_dims()
    m = np_model(dims)
    prompt = np.arange(9) % dims.vocab
    st = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    tokens0 = st.tokens.copy()
    E.denoise_step(m, dims, st, 0, sched)
    xs = libref.forward(tokens0, m, dims, n_layers=sched.skip_layer).numpy()
    xL = libref.forward(tokens0, m, dims).numpy()
    lg = libref.logits(libref.t(xL), m, dims)
    close(st.h_prev, xs, rtol=1e-11)
    close(st.h_final, xL, rtol=1e-11)
    close(st.logits, lg.numpy(), rtol=1e-10)
    close(st.conf, torch.softmax(lg, 1).max(1).values.numpy(), rtol=1e-10)


def pin_skip_step_semantics():
    """A skip step: h_prev <- X_s for all rows; the top-k by eq. I are the rows
    recomputed; skipped rows keep every cached byte; recomputed rows follow the
    stale-cache partial layers."""
    sched = micro_sched()
    dims = micro_dims()
    m = np_model(dims)
    prompt = (np.arange(9) * 7) % dims.vocab
    st = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    E.denoise_step(m, dims, st, 0, sched)                    # refresh
    before = {k: (getattr(st, k).copy()) for k in ("conf", "argmax", "h_final", "logits", "h_prev")}
    Kb = [k.copy() for k in st.K]
    Vb = [v.copy() for v in st.V]
    tokens1 = st.tokens.copy()
    info = E.denoise_step(m, dims, st, 1, sched)
    assert not info.refresh
    n = len(tokens1)
    k = E.keep_count(sched.keep, n)
    sel = info.selected
    assert len(sel) == k and np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < n
    # h_prev is the fresh skip-layer input of every row
    xs = libref.forward(tokens1, m, dims, n_layers=sched.skip_layer)
    close(st.h_prev, xs.numpy(), rtol=1e-11)
    # the selection is the brute-force top-k of eq. I (scores recomputed in torch)
    d = dims.d
    hp = libref.t(before["h_prev"])
    sc = 0.5 * libref.t(before["conf"]) + 0.5 * (xs - hp).abs().sum(1) / (math.sqrt(d) * hp.norm(dim=1))
    assert sel.tolist() == _brute_topk(sc.numpy(), k)
    # skipped rows: bit-identical caches
    other = np.setdiff1d(np.arange(n), sel)
    for key in ("conf", "argmax", "h_final", "logits"):
        assert np.array_equal(getattr(st, key)[other], before[key][other]), key
    for li in range(sched.skip_layer, dims.n_layers):
        assert np.array_equal(st.K[li][other], Kb[li][other])
        assert np.array_equal(st.V[li][other], Vb[li][other])
    # recomputed rows: partial layers against stale caches, by torch
    xr = xs[torch.as_tensor(sel)]
    for li in range(sched.skip_layer, dims.n_layers):
        xr, Kn, Vn = libref.partial_layer(xr, sel, m["layers"][li], Kb[li], Vb[li], dims)
        close(st.K[li], Kn.numpy(), rtol=1e-11)
        close(st.V[li], Vn.numpy(), rtol=1e-11)
    close(st.h_final[sel], xr.numpy(), rtol=1e-11)
    lg = libref.logits(xr, m, dims)
    close(st.conf[sel], torch.softmax(lg, 1).max(1).values.numpy(), rtol=1e-10)


def pin_refresh_interval_schedule():
    """Which steps are full refreshes (ES-dLLM section 2B; ES-dLLM*: more
    frequent refreshes), written out by hand for two blocks of six steps: a
    refresh at each block's first step, and with an interval N also at every
    in-block index that is a multiple of N."""
    expected = {0: "RSSSSS" "RSSSSS", 2: "RSRSRS" "RSRSRS", 4: "RSSSRS" "RSSSRS", 5: "RSSSSR" "RSSSSR"}
    for interval, kinds in expected.items():
        sched = micro_sched(gen_len=12, block_len=6, steps=12, refresh_interval=interval)
        assert sched.steps_per_block == 6
        got = "".join("R" if E.is_refresh_step(t, sched) else "S" for t in range(sched.steps))
        assert got == kinds, (interval, got)
        _, _, _, _, infos = _micro_run(sched)
        assert "".join("R" if i.refresh else "S" for i in infos) == kinds, interval


def pin_forced_selection_changes_only_the_decision():
    """The comparison protocol's hook: a skip step told to keep its own
    selection is bit-identical to the step left alone; told to keep another
    set, it recomputes exactly that set with the stale-cache partial layers
    (torch) and still reports its own scores; told to keep every row, it equals
    the keep = 100% step bit for bit."""
    import copy
    sched = micro_sched()
    dims = micro_dims()
    m = np_model(dims)
    prompt = (np.arange(9) * 5) % dims.vocab
    st0 = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    E.denoise_step(m, dims, st0, 0, sched)                   # refresh
    fields = ("tokens", "masked", "conf", "argmax", "h_prev", "h_final", "logits")

    def same(a, b):
        for key in fields:
            assert np.array_equal(getattr(a, key), getattr(b, key)), key
        for li in range(dims.n_layers):
            assert np.array_equal(a.K[li], b.K[li]) and np.array_equal(a.V[li], b.V[li]), li

    st_a, st_b = copy.deepcopy(st0), copy.deepcopy(st0)
    ia = E.denoise_step(m, dims, st_a, 1, sched)
    ib = E.denoise_step(m, dims, st_b, 1, sched, force_sel=ia.selected)
    assert np.array_equal(ia.selected, ib.selected) and np.array_equal(ia.scores, ib.scores)
    same(st_a, st_b)
    # another set of the same size: the complement's lowest rows
    n = len(st0.tokens)
    other = np.setdiff1d(np.arange(n), ia.selected)[:len(ia.selected)]
    st_c = copy.deepcopy(st0)
    tokens1 = st0.tokens.copy()
    ic = E.denoise_step(m, dims, st_c, 1, sched, force_sel=other)
    assert np.array_equal(ic.selected, other)
    close(ic.scores, ia.scores, rtol=0, atol=0)
    xs = libref.forward(tokens1, m, dims, n_layers=sched.skip_layer)
    xr = xs[torch.as_tensor(other)]
    for li in range(sched.skip_layer, dims.n_layers):
        xr, Kn, Vn = libref.partial_layer(xr, other, m["layers"][li], st0.K[li], st0.V[li], dims)
        close(st_c.K[li], Kn.numpy(), rtol=1e-11)
    close(st_c.h_final[other], xr.numpy(), rtol=1e-11)
    rest = np.setdiff1d(np.arange(n), other)
    assert np.array_equal(st_c.h_final[rest], st0.h_final[rest])
    # every row forced == keep = 100%
    st_d, st_e = copy.deepcopy(st0), copy.deepcopy(st0)
    E.denoise_step(m, dims, st_d, 1, sched, force_sel=np.arange(n))
    E.denoise_step(m, dims, st_e, 1, sched, keep=1.0)
    same(st_d, st_e)


def pin_stage_input_hook():
    """The comparison protocol's second hook: a step given its own skip-layer
    input is bit-identical to the step left alone (prefix caches aside, which
    are per-step scratch); given another input, it scores that input by eq. I
    and runs the partial layers (torch) from it."""
    import copy
    sched = micro_sched()
    dims = micro_dims()
    m = np_model(dims)
    prompt = (np.arange(9) * 3) % dims.vocab
    st0 = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    E.denoise_step(m, dims, st0, 0, sched)
    st_a, st_b = copy.deepcopy(st0), copy.deepcopy(st0)
    ia = E.denoise_step(m, dims, st_a, 1, sched)
    ib = E.denoise_step(m, dims, st_b, 1, sched, x_s=st_a.h_prev)
    assert np.array_equal(ia.selected, ib.selected) and np.array_equal(ia.scores, ib.scores)
    for key in ("tokens", "masked", "conf", "argmax", "h_prev", "h_final", "logits"):
        assert np.array_equal(getattr(st_a, key), getattr(st_b, key)), key
    for li in range(sched.skip_layer, dims.n_layers):
        assert np.array_equal(st_a.K[li], st_b.K[li]) and np.array_equal(st_a.V[li], st_b.V[li])
    # another input: X_s shifted by a constant row
    n = len(st0.tokens)
    x2 = st_a.h_prev + 0.05 * np.sin(np.arange(dims.d))[None, :]
    st_c = copy.deepcopy(st0)
    ic = E.denoise_step(m, dims, st_c, 1, sched, x_s=x2)
    hp = libref.t(st0.h_prev)
    xt = libref.t(x2)
    sc = 0.5 * libref.t(st0.conf) + 0.5 * (xt - hp).abs().sum(1) / (math.sqrt(dims.d) * hp.norm(dim=1))
    close(ic.scores, sc.numpy(), rtol=1e-12)
    sel = ic.selected
    assert sel.tolist() == _brute_topk(sc.numpy(), E.keep_count(sched.keep, n))
    close(st_c.h_prev, x2, rtol=0, atol=0)
    xr = xt[torch.as_tensor(sel)]
    for li in range(sched.skip_layer, dims.n_layers):
        xr, Kn, Vn = libref.partial_layer(xr, sel, m["layers"][li], st0.K[li], st0.V[li], dims)
        close(st_c.K[li], Kn.numpy(), rtol=1e-11)
    close(st_c.h_final[sel], xr.numpy(), rtol=1e-11)


def pin_keep_all_equals_vanilla():
    """keep = 100% is full recomputation, bit for bit, over a whole decode."""
    sched = micro_sched(keep=1.0)
    _, _, _, st_a, inf_a = _micro_run(sched)
    _, _, _, st_b, inf_b = _micro_run(sched, vanilla=True)
    assert any(not i.refresh for i in inf_a) and all(i.refresh for i in inf_b)
    for key in ("tokens", "masked", "conf", "argmax", "h_prev", "h_final", "logits"):
        assert np.array_equal(getattr(st_a, key), getattr(st_b, key)), key
    for li in range(len(st_a.K)):
        assert np.array_equal(st_a.K[li], st_b.K[li]) and np.array_equal(st_a.V[li], st_b.V[li])


def pin_unmask_schedule():
    for sched in (micro_sched(), micro_sched(block_len=12, steps=4), micro_sched(keep=0.1, refresh_interval=2)):
        dims, m, prompt, st, infos = _micro_run(sched)
        P = len(prompt)
        assert np.array_equal(st.tokens[:P], prompt)
        assert not st.masked.any()
        seen = set()
        for t, inf in enumerate(infos):
            assert len(inf.unmasked) == sched.per_step
            b = t // sched.steps_per_block
            lo, hi = P + b * sched.block_len, P + (b + 1) * sched.block_len
            assert all(lo <= p < hi for p in inf.unmasked)
            seen.update(inf.unmasked.tolist())
            sib = t % sched.steps_per_block
            assert inf.refresh == (sib == 0 or (sched.refresh_interval and sib % sched.refresh_interval == 0))
        assert seen == set(range(P, P + sched.gen_len))


def pin_fresh_cache_skip_is_exact():
    """With caches fresh and no token changed, recomputed rows equal the full
    result and the score reduces to its confidence term."""
    sched = workloads.Schedule(gen_len=12, block_len=12, steps=12, skip_layer=1, keep=0.5, score="esdllm")
    dims = micro_dims()
    m = np_model(dims)
    st = E.init_state(np.arange(9), sched.gen_len, dims, keep_logits=True)
    tokens0, masked0 = st.tokens.copy(), st.masked.copy()
    E.denoise_step(m, dims, st, 0, sched)                    # refresh, then unmasks
    full = st.h_final.copy()
    conf0 = st.conf.copy()
    st.tokens[:] = tokens0                                  # undo the unmasking only
    st.masked[:] = masked0
    info = E.denoise_step(m, dims, st, 1, sched)
    assert not info.refresh
    close(info.scores, 0.5 * conf0, rtol=1e-14)
    close(st.h_final[info.selected], full[info.selected], rtol=1e-11)


# --------------------------------------------------------------------------
# two skip levels (ES-dLLM section 2B: skipping at two early layers, a skip
# ratio per layer)
# --------------------------------------------------------------------------

def _eq1(conf, x, h, d):
    """Eq. I with alpha = 0.5, written in torch."""
    x, h = libref.t(x), libref.t(h)
    return (0.5 * libref.t(conf) + 0.5 * (x - h).abs().sum(1) / (math.sqrt(d) * h.norm(dim=1))).numpy()


def pin_nested_keep2_all_is_one_level():
    """A second level that keeps everything the first kept changes nothing."""
    one = micro_sched(keep=0.35)
    two = micro_sched(keep=0.35, skip_layer2=2, keep2=1.0)
    _, _, _, st_a, inf_a = _micro_run(one)
    _, _, _, st_b, inf_b = _micro_run(two)
    for key in ("tokens", "masked", "conf", "argmax", "h_prev", "h_final", "logits"):
        assert np.array_equal(getattr(st_a, key), getattr(st_b, key)), key
    for li in range(len(st_a.K)):
        assert np.array_equal(st_a.K[li], st_b.K[li]) and np.array_equal(st_a.V[li], st_b.V[li])
    for ia, ib in zip(inf_a, inf_b):
        assert np.array_equal(ia.selected, ib.selected2)


def pin_nested_full_first_level_is_one_level_at_s2():
    """Keeping every row at s1 makes the second level a single skip at s2 whose
    cached input is h_prev2."""
    two = micro_sched(skip_layer=1, keep=1.0, skip_layer2=2, keep2=0.35)
    one = micro_sched(skip_layer=2, keep=0.35)
    _, _, _, st_a, inf_a = _micro_run(two)
    _, _, _, st_b, inf_b = _micro_run(one)
    assert any(not i.refresh for i in inf_b)
    for key in ("tokens", "masked", "conf", "argmax", "h_final", "logits"):
        assert np.array_equal(getattr(st_a, key), getattr(st_b, key)), key
    assert np.array_equal(st_a.h_prev2, st_b.h_prev)
    for li in range(len(st_a.K)):
        assert np.array_equal(st_a.K[li], st_b.K[li]) and np.array_equal(st_a.V[li], st_b.V[li])
    for ia, ib in zip(inf_a, inf_b):
        assert np.array_equal(ia.selected2, ib.selected)
        if not ib.refresh:
            assert np.array_equal(ia.scores2, ib.scores)


def pin_nested_step_semantics():
    """One two-level skip step against torch: R1 = top-k1 of eq. I at s1,
    layers [s1, s2) on R1 against stale caches, h_prev2 <- their s2 input,
    R2 = top-k2 of eq. I at s2 among R1, layers [s2, L) on R2; every other row
    keeps every cached byte."""
    sched = micro_sched(skip_layer=1, keep=0.6, skip_layer2=2, keep2=0.3)
    dims = micro_dims()
    m = np_model(dims)
    prompt = (np.arange(9) * 5 + 2) % dims.vocab
    st = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    tokens0 = st.tokens.copy()
    E.denoise_step(m, dims, st, 0, sched)                    # refresh
    close(st.h_prev2, libref.forward(tokens0, m, dims, n_layers=2).numpy(), rtol=1e-11)
    before = {k: getattr(st, k).copy() for k in ("conf", "argmax", "h_final", "logits", "h_prev", "h_prev2")}
    Kb = [k.copy() for k in st.K]
    Vb = [v.copy() for v in st.V]
    tokens1 = st.tokens.copy()
    info = E.denoise_step(m, dims, st, 1, sched)
    assert not info.refresh
    n, d = len(tokens1), dims.d
    k1 = E.keep_count(0.6, n)
    k2 = min(E.keep_count(0.3, n), k1)
    R1, R2 = info.selected, info.selected2
    assert len(R1) == k1 and len(R2) == k2 and set(R2.tolist()) <= set(R1.tolist())
    assert np.all(np.diff(R2) > 0)
    xs = libref.forward(tokens1, m, dims, n_layers=1)
    assert R1.tolist() == _brute_topk(_eq1(before["conf"], xs, before["h_prev"], d), k1)
    xr, K1, V1 = libref.partial_layer(xs[torch.as_tensor(R1)], R1, m["layers"][1], Kb[1], Vb[1], dims)
    close(st.K[1], K1.numpy(), rtol=1e-11)
    close(st.V[1], V1.numpy(), rtol=1e-11)
    close(st.h_prev2[R1], xr.numpy(), rtol=1e-11)
    out1 = np.setdiff1d(np.arange(n), R1)
    assert np.array_equal(st.h_prev2[out1], before["h_prev2"][out1])
    sc2 = _eq1(before["conf"][R1], xr, before["h_prev2"][R1], d)
    close(info.scores2[R1], sc2, rtol=1e-11)
    assert np.all(np.isneginf(info.scores2[out1]))
    assert R2.tolist() == R1[_brute_topk(sc2, k2)].tolist()
    x2 = xr[torch.as_tensor(np.searchsorted(R1, R2))]
    for li in range(2, dims.n_layers):
        x2, Kn, Vn = libref.partial_layer(x2, R2, m["layers"][li], Kb[li], Vb[li], dims)
        close(st.K[li], Kn.numpy(), rtol=1e-11)
        close(st.V[li], Vn.numpy(), rtol=1e-11)
    close(st.h_final[R2], x2.numpy(), rtol=1e-11)
    lg = libref.logits(x2, m, dims)
    close(st.conf[R2], torch.softmax(lg, 1).max(1).values.numpy(), rtol=1e-10)
    out2 = np.setdiff1d(np.arange(n), R2)
    for key in ("conf", "argmax", "h_final", "logits"):
        assert np.array_equal(getattr(st, key)[out2], before[key][out2]), key


# --------------------------------------------------------------------------
# response-only steps (DyLLM section 2B, strategy 3)
# --------------------------------------------------------------------------

def pin_response_only_without_prompt_is_full_context():
    """With no prompt every row is a response row: the response-only schedule
    decodes exactly like the full-context one."""
    dims = micro_dims()
    m = np_model(dims)
    runs = []
    for sched in (micro_sched(keep=0.4), micro_sched(keep=0.4, response_interval=2)):
        st, infos = E.decode(m, dims, np.zeros(0, np.int64), sched, keep_logits=True)
        runs.append((st, infos))
    (st_a, inf_a), (st_b, inf_b) = runs
    assert any(i.response_only for i in inf_b)
    for key in ("tokens", "masked", "conf", "argmax", "h_prev", "h_final", "logits"):
        assert np.array_equal(getattr(st_a, key), getattr(st_b, key)), key
    for ia, ib in zip(inf_a, inf_b):
        assert np.array_equal(ia.selected, ib.selected)


def pin_response_only_step_semantics():
    """A response-only step against torch: the response rows go through the
    prefix against the cached prompt K/V, are scored, and k = ceil(keep * n_resp)
    of them are kept; prompt rows keep every cached byte."""
    sched = micro_sched(keep=0.5, response_interval=2)
    dims = micro_dims()
    m = np_model(dims)
    prompt = (np.arange(9) * 3 + 1) % dims.vocab
    P = len(prompt)
    st = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    E.denoise_step(m, dims, st, 0, sched)                    # refresh
    before = {k: getattr(st, k).copy() for k in ("conf", "argmax", "h_final", "logits", "h_prev")}
    Kb = [k.copy() for k in st.K]
    Vb = [v.copy() for v in st.V]
    tokens1 = st.tokens.copy()
    info = E.denoise_step(m, dims, st, 1, sched)
    assert info.response_only and not info.refresh
    n, d = len(tokens1), dims.d
    cand = np.arange(P, n)
    x = libref.t(m["embed"])[torch.as_tensor(tokens1[cand])]
    for li in range(sched.skip_layer):
        x, Kn, Vn = libref.partial_layer(x, cand, m["layers"][li], Kb[li], Vb[li], dims)
        close(st.K[li], Kn.numpy(), rtol=1e-11)
        assert np.array_equal(st.K[li][:P], Kb[li][:P]) and np.array_equal(st.V[li][:P], Vb[li][:P])
    close(st.h_prev[cand], x.numpy(), rtol=1e-11)
    assert np.array_equal(st.h_prev[:P], before["h_prev"][:P])
    sc = _eq1(before["conf"][cand], x, before["h_prev"][cand], d)
    close(info.scores[cand], sc, rtol=1e-11)
    assert np.all(np.isneginf(info.scores[:P]))
    k = E.keep_count(0.5, n - P)
    sel = info.selected
    assert sel.tolist() == (cand[_brute_topk(sc, k)]).tolist()
    xr = x[torch.as_tensor(sel - P)]
    for li in range(sched.skip_layer, dims.n_layers):
        xr, Kn, Vn = libref.partial_layer(xr, sel, m["layers"][li], Kb[li], Vb[li], dims)
        close(st.K[li], Kn.numpy(), rtol=1e-11)
    close(st.h_final[sel], xr.numpy(), rtol=1e-11)
    other = np.setdiff1d(np.arange(n), sel)
    for key in ("conf", "argmax", "h_final", "logits"):
        assert np.array_equal(getattr(st, key)[other], before[key][other]), key


def pin_response_only_schedule():
    """Refresh steps are full context; other steps are full context every
    response_interval in-block steps and response-only otherwise."""
    sched = micro_sched(keep=0.4, block_len=6, steps=8, gen_len=12, response_interval=3)
    dims, m, prompt, st, infos = _micro_run(sched)
    P, n = len(prompt), len(prompt) + sched.gen_len
    kinds = []
    for t, inf in enumerate(infos):
        sib = t % sched.steps_per_block
        kinds.append("R" if inf.refresh else ("r" if inf.response_only else "F"))
        assert inf.response_only == (not inf.refresh and sib % 3 != 0)
        if inf.response_only:
            assert inf.selected.min() >= P and len(inf.selected) == E.keep_count(0.4, n - P)
        elif not inf.refresh:
            assert len(inf.selected) == E.keep_count(0.4, n)
    assert kinds == list("RrrFRrrF"), kinds


# --------------------------------------------------------------------------
# keys or values as the scored tensor (ES-dLLM section 2A)
# --------------------------------------------------------------------------

def _kv_step(which, model_fix=None):
    sched = micro_sched(keep=0.4, score_tensor=which)
    dims = micro_dims()
    m = np_model(dims)
    if model_fix:
        model_fix(m, dims)
    prompt = (np.arange(9) * 4 + 3) % dims.vocab
    st = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    tokens0 = st.tokens.copy()
    E.denoise_step(m, dims, st, 0, sched)                    # refresh
    h0 = st.h_prev.copy()
    conf0 = st.conf.copy()
    tokens1 = st.tokens.copy()
    info = E.denoise_step(m, dims, st, 1, sched)
    return sched, dims, m, tokens0, tokens1, h0, conf0, st, info


def pin_value_score_with_identity_projection():
    """Layer s's Wv = I (gains 1): the scored value rows are RMSNorm(X_s)."""
    def fix(m, dims):
        m["layers"][1]["wv"] = np.eye(dims.d)
    sched, dims, m, tokens0, tokens1, h0, conf0, st, info = _kv_step("value", fix)
    def rn(tokens):
        x = libref.forward(tokens, m, dims, n_layers=sched.skip_layer)
        return libref.rms(x, libref.t(np.ones(dims.d)), dims.rms_eps)
    v0, v1 = rn(tokens0), rn(tokens1)
    close(h0, v0.numpy(), rtol=1e-11)
    close(st.h_prev, v1.numpy(), rtol=1e-11)
    close(info.scores, _eq1(conf0, v1, v0, dims.d), rtol=1e-11)
    assert info.selected.tolist() == _brute_topk(info.scores, E.keep_count(sched.keep, len(tokens1)))


def pin_key_and_value_scores_against_torch():
    """Keys (rotated, as cached) or values of layer s, from torch's projection
    and complex-multiplication RoPE, at the refresh and at the next step."""
    for which, slot in (("key", 1), ("value", 2)):
        sched, dims, m, tokens0, tokens1, h0, conf0, st, info = _kv_step(which)
        s = sched.skip_layer
        def tens(tokens):
            x = libref.forward(tokens, m, dims, n_layers=s)
            return libref.qkv(x, torch.arange(len(tokens)), m["layers"][s], dims)[slot]
        t0, t1 = tens(tokens0), tens(tokens1)
        close(h0, t0.numpy(), rtol=1e-11)
        close(st.h_prev, t1.numpy(), rtol=1e-11)
        close(info.scores, _eq1(conf0, t1, t0, dims.d), rtol=1e-11)
        assert info.selected.tolist() == _brute_topk(info.scores, E.keep_count(sched.keep, len(tokens1)))


# --------------------------------------------------------------------------
# per-layer re-selection with approximate attention (DyLLM section 2B)
# --------------------------------------------------------------------------

def _rand_attn(seed=3, n=11, m=13, H=2, dh=8):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(n, H * dh)), rng.normal(size=(m, H * dh)), rng.normal(size=(m, H * dh)), H, dh


def pin_attention_lse_torch():
    q, K, _, H, dh = _rand_attn()
    lse = E.attention_lse(q, K, H, dh)
    qt, Kt = libref.t(q), libref.t(K)
    for h in range(H):
        sl = slice(h * dh, (h + 1) * dh)
        close(lse[:, h], torch.logsumexp(qt[:, sl] @ Kt[:, sl].T / math.sqrt(dh), dim=1).numpy())


def pin_approx_context_exact_when_only_values_change():
    """Delta C = S Delta V holds exactly when only value rows change (keys and
    queries fixed): checked against torch's attention before and after."""
    q, K, V, H, dh = _rand_attn(seed=4)
    A = np.array([1, 4, 5, 11])
    V2 = V.copy()
    V2[A] += np.random.default_rng(9).normal(size=(len(A), V.shape[1]))
    C0 = libref.attn(libref.t(q), libref.t(K), libref.t(V), H, dh).numpy()
    C1 = libref.attn(libref.t(q), libref.t(K), libref.t(V2), H, dh).numpy()
    got = E.approx_context(C0, q, E.attention_lse(q, K, H, dh), K[A], V2[A] - V[A], H, dh)
    close(got, C1, rtol=1e-12, atol=1e-12)
    assert np.abs(C1 - C0).max() > 1e-3


def pin_layer_parts_against_torch():
    dims = micro_dims()
    m = np_model(dims)
    lw = m["layers"][1]
    n = 14
    x = np.random.default_rng(2).normal(size=(n, dims.d))
    pos = np.arange(n)
    K = np.zeros((n, dims.d))
    V = np.zeros((n, dims.d))
    y, q, ctx, lse = E.layer_parts(x, pos, lw, K, V, n, dims)
    qt, kt, vt = libref.qkv(libref.t(x), torch.as_tensor(pos), lw, dims)
    close(q, qt.numpy(), rtol=1e-12)
    close(ctx, libref.attn(qt, kt, vt, dims.n_heads, dims.head_dim).numpy(), rtol=1e-11)
    close(y, libref.full_layer(libref.t(x), lw, dims).numpy(), rtol=1e-11)
    close(E.finish_layer(x, ctx, lw, dims), y, rtol=1e-13)
    K2, V2 = np.zeros_like(K), np.zeros_like(V)
    assert np.array_equal(E.layer_forward(x, pos, lw, K2, V2, n, dims), y)


def pin_per_layer_keep_all_is_vanilla():
    """Every row kept at layer s and at every layer: the per-layer variant is
    full recomputation, bit for bit, over a whole decode."""
    sched = micro_sched(keep=1.0, per_layer=True, keep_layer=1.0)
    _, _, _, st_a, inf_a = _micro_run(sched)
    _, _, _, st_b, _ = _micro_run(micro_sched(keep=1.0), vanilla=True)
    assert any(not i.refresh for i in inf_a)
    for key in ("tokens", "masked", "conf", "argmax", "h_prev", "h_final", "logits"):
        assert np.array_equal(getattr(st_a, key), getattr(st_b, key)), key
    for li in range(len(st_a.K)):
        assert np.array_equal(st_a.K[li], st_b.K[li]) and np.array_equal(st_a.V[li], st_b.V[li])


def pin_per_layer_step_against_torch():
    """One per-layer step after a refresh, layer by layer in torch: fresh q/K/V
    and exact attention for the active rows; C + S dV for the others from the
    cached query, normaliser and previous keys; salient rows = brute-force
    top-k of 1 - cos; Wo + FFN on them from the right inputs; caches."""
    sched = micro_sched(keep=0.4, per_layer=True, keep_layer=0.3)
    dims = micro_dims()
    m = np_model(dims)
    H, dh, d = dims.n_heads, dims.head_dim, dims.d
    prompt = (np.arange(9) * 2 + 5) % dims.vocab
    st = E.init_state(prompt, sched.gen_len, dims, keep_logits=True)
    tokens0 = st.tokens.copy()
    E.denoise_step(m, dims, st, 0, sched)                    # refresh: every cache of every layer
    s = sched.skip_layer
    x = libref.forward(tokens0, m, dims, n_layers=s)
    for li in range(s, dims.n_layers):
        lw = m["layers"][li]
        q, k, v = libref.qkv(x, torch.arange(len(tokens0)), lw, dims)
        close(st.Q[li], q.numpy(), rtol=1e-11)
        close(st.C[li], libref.attn(q, k, v, H, dh).numpy(), rtol=1e-11)
        x = libref.full_layer(x, lw, dims)
        close(st.Y[li], x.numpy(), rtol=1e-11)
    old = {k: [a.copy() for a in getattr(st, k)] for k in ("K", "V", "Q", "C", "LSE", "Y")}
    before = {k: getattr(st, k).copy() for k in ("conf", "h_prev", "h_final", "argmax")}
    tokens1 = st.tokens.copy()
    info = E.denoise_step(m, dims, st, 1, sched)
    n = len(tokens1)
    Xs = libref.forward(tokens1, m, dims, n_layers=s)
    A = np.array(_brute_topk(_eq1(before["conf"], Xs, before["h_prev"], d), E.keep_count(0.4, n)))
    assert info.selected.tolist() == A.tolist()
    xA = Xs[torch.as_tensor(A)]
    k_l = E.keep_count(0.3, n)
    for i, li in enumerate(range(s, dims.n_layers)):
        lw = m["layers"][li]
        q, k, v = libref.qkv(xA, torch.as_tensor(A), lw, dims)
        Kn, Vn = libref.t(old["K"][li]).clone(), libref.t(old["V"][li]).clone()
        Kn[A], Vn[A] = k, v
        C = libref.t(old["C"][li]).clone()
        Qc, lse = libref.t(old["Q"][li]), libref.t(old["LSE"][li])
        dV = v - libref.t(old["V"][li][A])
        for h in range(H):
            sl = slice(h * dh, (h + 1) * dh)
            P = torch.exp(Qc[:, sl] @ libref.t(old["K"][li][A])[:, sl].T / math.sqrt(dh) - lse[:, h:h + 1])
            C[:, sl] += P @ dV[:, sl]
        C[A] = libref.attn(q, Kn, Vn, H, dh)
        sig = (1.0 - torch.nn.functional.cosine_similarity(C, libref.t(old["C"][li]), dim=1)).numpy()
        R = np.array(_brute_topk(sig, k_l))
        assert info.layer_selected[i].tolist() == R.tolist(), li
        close(info.layer_scores[i], sig, rtol=1e-10, atol=1e-12)
        close(st.C[li], C.numpy(), rtol=1e-11)
        close(st.K[li], Kn.numpy(), rtol=1e-11)
        x_in = Xs[torch.as_tensor(R)] if li == s else libref.t(st.Y[li - 1][R])
        y = libref.finish_layer(x_in, C[torch.as_tensor(R)], lw, dims)
        close(st.Y[li][R], y.numpy(), rtol=1e-11)
        other = np.setdiff1d(np.arange(n), R)
        assert np.array_equal(st.Y[li][other], old["Y"][li][other])
        A, xA = R, y
    close(st.h_final[A], xA.numpy(), rtol=1e-11)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
