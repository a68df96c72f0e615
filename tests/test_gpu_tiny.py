"""GPU parity on the tiny workload (2 layers, d=64, vocab 512): the whole
8-step decode in fp32 against the oracle, every bf16 step from the oracle's state,
and device-side invariants (keep-all == refresh, skipped rows untouched,
determinism)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_util import (bf16_step, check_scores_exact_inputs, host, np_model, row_rel_err, snapshot,
                      to_device, topk_within_band)
from oracle import esdllm as E

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def _setup(dtype, sched=None, keep_logits=True):
    from dynamic_token_skipping_amd import Decoder, DeviceModel
    wl = workloads.workload("tiny")
    sched = sched or wl.sched
    m_cpu = workloads.make_model(wl.dims, wl.seed, dtype, "cpu")
    prompts, _ = workloads.make_prompt(wl)
    dev = DeviceModel(to_device(m_cpu), wl.dims.n_heads, wl.dims.head_dim, dtype)
    dec = Decoder(dev, prompts, sched, keep_logits=keep_logits)
    st = E.init_state(prompts[0].numpy(), sched.gen_len, wl.dims, keep_logits=True)
    return wl, sched, np_model(m_cpu), dec, st


def _compare_step_f32(dec, st, info, before, wl, sched, t):
    """fp32 whole trajectory: the GPU's scores against the oracle's score
    function on its own inputs, the kept set equal to the oracle's, and every
    value within 1e-5."""
    d = wl.dims
    n = len(st.tokens)
    sel = dec.sel.rows()[0]
    rows = info.selected
    if not info.refresh:
        cand = np.arange(n)
        s_ex = check_scores_exact_inputs(host(dec.scores[0]), host(dec.h_prev[0]), before["h_prev"][0],
                                         before["conf"][0], sched.score, sched.alpha, cand)
        ok, _, _ = topk_within_band(sel, cand, s_ex, E.keep_count(sched.keep, n))
        assert ok, f"step {t}: selection against its own inputs"
        assert np.abs(host(dec.scores[0])[:n] - info.scores).max() <= 1e-5 * max(1.0, np.abs(info.scores).max())
    assert sel == list(rows), f"step {t}"
    assert row_rel_err(host(dec.h_final[0])[rows], st.h_final[rows]) <= TOL_F32, f"step {t} h_final"
    assert row_rel_err(host(dec.logits[0])[rows], st.logits[rows]) <= TOL_F32, f"step {t} logits"
    assert row_rel_err(host(dec.conf[0])[rows][:, None], st.conf[rows][:, None]) <= TOL_F32, f"step {t} conf"
    assert row_rel_err(host(dec.h_prev[0]), st.h_prev) <= TOL_F32, f"step {t} h_prev"
    for li in range(sched.skip_layer, d.n_layers):
        assert row_rel_err(host(dec.k_cache[li, 0])[rows], st.K[li][rows]) <= TOL_F32, f"step {t} K{li}"
        assert row_rel_err(host(dec.v_cache[li, 0])[rows], st.V[li][rows]) <= TOL_F32, f"step {t} V{li}"


@pytest.mark.parametrize("refresh_interval", [0, 2])
def test_tiny_fp32_full_decode_matches_oracle(refresh_interval):
    """The whole decode; with refresh_interval 2 every other step inside a
    block is a full refresh as well (ES-dLLM*'s more frequent refresh)."""
    wl = workloads.workload("tiny")
    wl, sched, m_np, dec, st = _setup("f32", dataclasses.replace(wl.sched, refresh_interval=refresh_interval))
    refreshes = 0
    for t in range(sched.steps):
        before = snapshot(dec)
        info = E.denoise_step(m_np, wl.dims, st, t, sched)
        refreshes += bool(info.refresh)
        dec.step(t)
        torch.cuda.synchronize()
        _compare_step_f32(dec, st, info, before, wl, sched, t)
        assert np.array_equal(dec.tokens[0].cpu().numpy(), st.tokens), f"tokens differ after step {t}"
        assert np.array_equal(dec.masked[0].cpu().numpy().astype(bool), st.masked)
        assert np.array_equal(dec.argmax[0].cpu().numpy()[info.selected], st.argmax[info.selected])
    assert not dec.masked.any()
    n_blocks = -(-sched.gen_len // sched.block_len)
    assert refreshes > n_blocks if refresh_interval else refreshes == n_blocks


def test_tiny_bf16_decode_steps():
    """bf16 storage, every step from the oracle's state with the GPU's kept
    set forced into the oracle: selection and unmasking exact on the GPU's own
    inputs (1e-4 band), every value within 2e-2 at every step."""
    wl, sched, m_np, dec, st = _setup("bf16")
    for t in range(sched.steps):
        bf16_step(dec, m_np, wl.dims, [st], t, sched, TOL_BF16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_keep_all_equals_refresh_on_device(dtype):
    sched = dataclasses.replace(workloads.workload("tiny").sched, keep=1.0)
    _, _, _, a, _ = _setup(dtype, sched)
    _, _, _, b, _ = _setup(dtype, sched)
    for t in range(4):
        a.step(t)
        b.step(t, force_refresh=True)
    torch.cuda.synchronize()
    for name in ("tokens", "masked", "h_prev", "k_cache", "v_cache", "h_final", "conf", "argmax", "logits"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_skipped_rows_bit_identical_and_deterministic(dtype):
    wl, sched, _, dec, _ = _setup(dtype)
    dec.step(0)
    dec.step(1)
    torch.cuda.synchronize()
    before = {n: getattr(dec, n).clone() for n in ("k_cache", "v_cache", "h_final", "conf", "argmax", "logits")}
    snap = {n: getattr(dec, n).clone() for n in ("tokens", "masked", "h_prev", "k_cache", "v_cache", "h_final",
                                                 "conf", "argmax", "logits")}
    dec.step(2)
    torch.cuda.synchronize()
    sel = dec.sel.rows()[0]
    assert len(sel) == E.keep_count(sched.keep, dec.seq_lens[0])
    other = sorted(set(range(dec.seq_lens[0])) - set(sel))
    s = sched.skip_layer
    for n, v in before.items():
        now = getattr(dec, n)
        if n in ("k_cache", "v_cache"):
            assert torch.equal(now[s:, 0, other], v[s:, 0, other]), n
        else:
            assert torch.equal(now[0, other], v[0, other]), n
    after = {n: getattr(dec, n).clone() for n in snap}
    # determinism: replay step 2 from the same state
    for n, v in snap.items():
        getattr(dec, n).copy_(v)
    dec.step(2)
    torch.cuda.synchronize()
    for n, v in after.items():
        assert torch.equal(getattr(dec, n), v), n
