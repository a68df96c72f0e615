"""Degenerate inputs of scoring and selection (ES-dLLM technical summary
section 2A eq. I and 2B top-k; DyLLM section 2A threshold), on the GPU
against the oracle's score function and a brute-force sort:

* exact ties (identical rows) go to the lower index, for every k;
* a zero-norm cached row is guarded by FLT_MIN (eq. I's L1 term overflows to
  +inf in float32 when the current row is not zero, and is 0 when it is);
* a NaN score (a NaN confidence) ranks below every number, NaN rows among
  themselves by index;
* k = 1 and k = len; a threshold equal to a score keeps that row out (strict);
* an empty sequence selects nothing.

Every scoring kernel is covered: behind dl_score_select the one-wave-per-row
kernel (d = 256) and, in bf16 with d a multiple of 512, the
one-workgroup-per-row kernel; and the fused one of the decode step."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import host, np_model, to_device
from oracle import esdllm as E

pytestmark = pytest.mark.gpu


def _expected(scores, cand, k):
    """Brute-force top-k of float32 scores with NaN last and the lower index
    first among equal keys; ascending positions."""
    s32 = np.asarray(scores, np.float64).astype(np.float32)
    nan = np.isnan(s32)
    key = np.where(nan, -np.inf, s32.astype(np.float64))
    order = sorted(range(len(cand)), key=lambda j: (nan[j], -key[j], cand[j]))
    return sorted(int(cand[j]) for j in order[:k])


def _inputs(B, S, d, lens, seed):
    g = np.random.default_rng(seed)
    h_prev = g.standard_normal((B, S, d)).astype(np.float32)
    h_cur = (h_prev + 0.3 * g.standard_normal((B, S, d))).astype(np.float32)
    conf = g.uniform(size=(B, S)).astype(np.float32)
    # sequence 0: exact ties -- rows 4..7 copies of row 2, rows 12, 13 copies of row 11
    for r in (4, 5, 6, 7):
        h_prev[0, r], h_cur[0, r], conf[0, r] = h_prev[0, 2], h_cur[0, 2], conf[0, 2]
    for r in (12, 13):
        h_prev[0, r], h_cur[0, r], conf[0, r] = h_prev[0, 11], h_cur[0, 11], conf[0, 11]
    # zero-norm cached rows: 20 (current row non-zero: +inf in float32) and 21 (both zero: alpha*c)
    h_prev[0, 20] = 0.0
    h_prev[0, 21] = 0.0
    h_cur[0, 21] = 0.0
    h_prev[0, 30] = 0.0                        # a second +inf, tied with row 20
    # NaN scores: rows 25 and 9 of sequence 0, row 3 of sequence 2
    conf[0, 25] = np.nan
    conf[0, 9] = np.nan
    conf[2, 3] = np.nan
    return h_prev, h_cur, conf


@pytest.mark.parametrize("dtype,d", [("f32", 256), ("bf16", 256), ("bf16", 512), ("bf16", 2560)])
def test_score_select_degenerate_inputs(dtype, d):
    import dynamic_token_skipping_amd as D
    B, S = 3, 40
    lens = [40, 0, 17]
    h_prev, h_cur, conf = _inputs(B, S, d, lens, seed=11)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    hp = torch.as_tensor(h_prev).to(tdt).cuda()
    hc = torch.as_tensor(h_cur).to(tdt).cuda()
    cf = torch.as_tensor(conf).cuda()
    hp64, hc64 = host(hp), host(hc)             # exactly what the kernel reads
    dims = D.make_dims(B, S, d, d // 128, 128, 512, 1024, 1, dtype)
    ws = D.workspace(dims, B * S)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sel = D.SelectionTensors(B, S)
    scores = torch.full((B, S), 7.0, dtype=torch.float32, device="cuda")
    with np.errstate(over="ignore", invalid="ignore"):
        o = [E.score_rows("esdllm", hc64[b, :n], hp64[b, :n], conf[b, :n].astype(np.float64), 0.5)
             for b, n in enumerate(lens)]
    assert np.isinf(np.float32(o[0][20])) and np.isinf(np.float32(o[0][30]))
    assert o[0][21] == 0.5 * np.float64(conf[0, 21])
    for keep in (1e-3, 1.0, 0.1, 0.2, 0.3, 0.95):
        ks = [E.keep_count(keep, n) for n in lens]
        assert keep != 1e-3 or ks == [1, 0, 1]
        assert keep != 1.0 or ks == lens
        D.dl_score_select(dims, hc, hp, cf, seq, "esdllm", 0.5, D.DL_SEL_TOPK, keep, 0.0, sel, scores=scores, ws=ws)
        torch.cuda.synchronize()
        got = sel.rows()
        g_sc = host(scores)
        for b, n in enumerate(lens):
            assert len(got[b]) == ks[b]
            if n == 0:
                continue
            # scores against the oracle's on the same inputs: NaN and +inf (float32) where it has them
            nan = np.isnan(o[b])
            inf = np.isinf(np.float32(o[b])) & ~nan
            assert np.array_equal(np.isnan(g_sc[b, :n]), nan)
            assert np.array_equal(np.isinf(g_sc[b, :n]), inf)
            num = ~nan & ~inf
            err = np.abs(g_sc[b, :n][num] - o[b][num]).max(initial=0.0)
            assert err <= 1e-5 * max(1.0, np.abs(o[b][num]).max(initial=0.0))
            # the kept set: exactly the brute force on the kernel's own float32 scores, and on the oracle's
            assert got[b] == _expected(g_sc[b, :n], np.arange(n), ks[b]), (keep, b)
            assert got[b] == _expected(o[b], np.arange(n), ks[b]), (keep, b)
        assert torch.all(scores[1] == 7.0) and torch.all(scores[2, 17:] == 7.0)   # padding is not written
    # the tie groups: with k cutting inside a group, its lowest indices are kept
    s0 = host(scores)[0, :40]
    assert len(set(s0[[2, 4, 5, 6, 7]].tolist())) == 1 and s0[11] == s0[12] == s0[13]
    # threshold equal to a score: strict, so that row (and its ties) stay out
    for tau_row in (2, 11, 15):
        tau = float(s0[tau_row])
        D.dl_score_select(dims, hc, hp, cf, seq, "esdllm", 0.5, D.DL_SEL_THRESHOLD, 1.0, tau, sel, ws=ws)
        torch.cuda.synchronize()
        got = sel.rows()
        for b, n in enumerate(lens):
            want = [i for i in range(n) if not np.isnan(g_sc[b, i]) and np.float32(g_sc[b, i]) > np.float32(tau)]
            assert got[b] == want, (tau_row, b)
        assert tau_row not in got[0]


def test_fused_scoring_degenerate_rows_in_a_decode():
    """The decode step's fused scoring pass (d = 512): zero-norm cached rows
    and NaN confidences planted before a skip step; the kept set follows the
    brute force on the kernel's own scores (NaN last, lower index on ties),
    which equal the oracle's score function on the same inputs."""
    from dynamic_token_skipping_amd import Decoder, DeviceModel
    dims = workloads.ModelDims(d=512, n_heads=4, head_dim=128, d_ffn=1024, vocab=1024, n_layers=3)
    sched = workloads.Schedule(gen_len=32, block_len=16, steps=8, skip_layer=1, keep=0.25, score="esdllm")
    m_cpu = workloads.make_model(dims, 21, "bf16", "cpu")
    g = torch.Generator().manual_seed(21)
    prompts = [torch.randint(0, dims.vocab, (n,), generator=g) for n in (9, 45, 96)]
    dec = Decoder(DeviceModel(to_device(m_cpu), dims.n_heads, dims.head_dim, "bf16"), prompts, sched)
    dec.step(0)
    torch.cuda.synchronize()
    dec.h_prev[0, 3] = 0                       # +inf (current row not zero)
    dec.h_prev[0, 30] = 0                      # tied +inf
    dec.h_prev[1, 50] = 0
    dec.conf[0, 7] = float("nan")
    dec.conf[2, 0] = float("nan")
    dec.conf[2, 1] = float("nan")
    hp_before, cf_before = host(dec.h_prev), host(dec.conf)
    dec.step(1)
    torch.cuda.synchronize()
    got = dec.sel.rows()
    g_sc = host(dec.scores)
    hp_after = host(dec.h_prev)
    for b, n in enumerate(dec.seq_lens):
        k = E.keep_count(sched.keep, n)
        assert got[b] == _expected(g_sc[b, :n], np.arange(n), k), b
        with np.errstate(over="ignore", invalid="ignore"):
            o = E.score_rows("esdllm", hp_after[b, :n], hp_before[b, :n], cf_before[b, :n], 0.5)
        assert np.array_equal(np.isnan(g_sc[b, :n]), np.isnan(o))
        o32 = np.float32(o)
        assert np.array_equal(np.isinf(g_sc[b, :n]), np.isinf(o32) & ~np.isnan(o))
        fin = np.isfinite(o32)
        assert np.abs(g_sc[b, :n][fin] - o[fin]).max() <= 1e-5 * max(1.0, np.abs(o[fin]).max())
        assert got[b] == _expected(o, np.arange(n), k), b
    assert 3 in got[0] and 30 in got[0] and 7 not in got[0]
    assert 0 not in got[2] and 1 not in got[2]


def test_select_beyond_register_capacity():
    """More candidates than the selection kernel holds in registers (over 8
    per thread of its 1024): 10000 rows of one sequence, top-k and threshold,
    against the brute force on the kernel's own scores and the oracle's."""
    import dynamic_token_skipping_amd as D
    S, d = 10000, 512
    g = np.random.default_rng(23)
    h_prev = g.standard_normal((1, S, d)).astype(np.float32)
    h_cur = (h_prev + 0.3 * g.standard_normal((1, S, d))).astype(np.float32)
    conf = g.uniform(size=(1, S)).astype(np.float32)
    h_prev[0, 100:110] = h_prev[0, 99]                    # a tie group
    h_cur[0, 100:110] = h_cur[0, 99]
    conf[0, 100:110] = conf[0, 99]
    hp = torch.as_tensor(h_prev).to(torch.bfloat16).cuda()
    hc = torch.as_tensor(h_cur).to(torch.bfloat16).cuda()
    cf = torch.as_tensor(conf).cuda()
    dims = D.make_dims(1, S, d, 4, 128, 512, 1024, 1, "bf16")
    ws = D.workspace(dims, S)
    seq = torch.tensor([S], dtype=torch.int32, device="cuda")
    sel = D.SelectionTensors(1, S)
    scores = torch.zeros((1, S), dtype=torch.float32, device="cuda")
    o = E.score_rows("esdllm", host(hc[0]), host(hp[0]), conf[0].astype(np.float64), 0.5)
    for keep in (0.3, 0.0101, 1.0):
        k = E.keep_count(keep, S)
        D.dl_score_select(dims, hc, hp, cf, seq, "esdllm", 0.5, D.DL_SEL_TOPK, keep, 0.0, sel, scores=scores, ws=ws)
        torch.cuda.synchronize()
        g_sc = host(scores[0])
        assert np.abs(g_sc - o).max() <= 1e-5 * np.abs(o).max()
        got = sel.rows()[0]
        assert got == _expected(g_sc, np.arange(S), k), keep
    tau = float(np.sort(g_sc)[S // 2])
    D.dl_score_select(dims, hc, hp, cf, seq, "esdllm", 0.5, D.DL_SEL_THRESHOLD, 1.0, tau, sel, ws=ws)
    torch.cuda.synchronize()
    assert sel.rows()[0] == [i for i in range(S) if np.float32(g_sc[i]) > np.float32(tau)]
