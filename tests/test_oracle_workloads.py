"""The oracle on the tiny workload (whole decode) and on reduced shapes of the
8B-class workloads: schedule counts, selection sizes and the keep-all identity."""
import numpy as np
import pytest

import oracle_pins
import workloads
from oracle import esdllm as E


def _np_model(m):
    out = {k: workloads.host_f64(v) for k, v in m.items() if k != "layers"}
    out["layers"] = [{k: workloads.host_f64(v) for k, v in lw.items()} for lw in m["layers"]]
    return out


def test_tiny_workload_decode():
    wl = workloads.workload("tiny")
    m = _np_model(workloads.make_model(wl.dims, wl.seed, wl.dtype, "cpu"))
    prompts, lens = workloads.make_prompt(wl)
    sched = wl.sched
    st, infos = E.decode(m, wl.dims, prompts[0].numpy(), sched)
    assert sched.per_step == 6 and sched.steps_per_block == 8
    assert [len(i.unmasked) for i in infos] == [6] * 8
    assert infos[0].refresh and not any(i.refresh for i in infos[1:])
    assert all(len(i.selected) == 16 for i in infos[1:])
    assert not st.masked.any()
    assert np.array_equal(st.tokens[:16], prompts[0].numpy())
    # deterministic
    st2, _ = E.decode(m, wl.dims, prompts[0].numpy(), sched)
    assert np.array_equal(st.tokens, st2.tokens)


def test_tiny_workload_keep_all_is_vanilla():
    wl = workloads.workload("tiny")
    m = _np_model(workloads.make_model(wl.dims, wl.seed, wl.dtype, "cpu"))
    prompts, _ = workloads.make_prompt(wl)
    import dataclasses
    sched = dataclasses.replace(wl.sched, keep=1.0)
    a, _ = E.decode(m, wl.dims, prompts[0].numpy(), sched)
    b, _ = E.decode(m, wl.dims, prompts[0].numpy(), sched, vanilla=True)
    assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.h_final, b.h_final)


@pytest.mark.parametrize("name", ["full8b", "batch8b", "long8b"])
def test_schedules_of_8b_workloads(name):
    s = workloads.workload(name).sched
    assert s.n_blocks * s.steps_per_block == s.steps
    assert s.per_step * s.steps_per_block == s.block_len
    assert {"full8b": 1, "batch8b": 2, "long8b": 1}[name] == s.per_step
    n = {"full8b": 512, "long8b": 4608}.get(name)
    if n:
        assert E.keep_count(s.keep, n) == {"full8b": 128, "long8b": 576}[name]


def test_batch_prompt_lengths():
    wl = workloads.workload("batch8b")
    prompts, lens = workloads.make_prompt(wl)
    assert len(lens) == 16 and all(128 <= n <= 1024 for n in lens)
    assert all(len(p) == n for p, n in zip(prompts, lens))
