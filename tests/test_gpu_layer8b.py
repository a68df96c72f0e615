"""GPU parity at the 8B-class layer shape (d 4096, 32x128 heads, FFN 11008,
S 512): the standalone entry points against the oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import host, lse_err, row_rel_err, topk_within_band
from oracle import esdllm as E

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def lay():
    import dynamic_token_skipping_amd as D
    wl = workloads.workload("layer8b")
    m = workloads.make_model(wl.dims, wl.seed, "bf16", "cuda")
    st = workloads.make_layer_state(wl, "cuda")
    S = wl.prompt_len
    dims = D.make_dims(1, S, wl.dims.d, wl.dims.n_heads, wl.dims.head_dim, wl.dims.d_ffn, wl.dims.vocab, 1, "bf16")
    ws = D.workspace(dims, S)
    seq_len = torch.tensor([S], dtype=torch.int32, device="cuda")
    lw_np = {k: host(v) for k, v in m["layers"][0].items()}
    return dict(wl=wl, m=m, st=st, S=S, dims=dims, ws=ws, seq_len=seq_len, lw_np=lw_np, D=D,
                h_prev=host(st["h_prev"]), h_cur=host(st["h_cur"]), conf=host(st["conf"]))


@pytest.mark.parametrize("keep", [1.0, 0.5, 0.25, 0.125])
def test_score_select_matches_oracle(lay, keep):
    D = lay["D"]
    sel = D.SelectionTensors(1, lay["S"])
    scores = torch.zeros((1, lay["S"]), dtype=torch.float32, device="cuda")
    D.dl_score_select(lay["dims"], lay["st"]["h_cur"], lay["st"]["h_prev"], lay["st"]["conf"], lay["seq_len"],
                      "esdllm", 0.5, D.DL_SEL_TOPK, keep, 0.0, sel, scores=scores, ws=lay["ws"])
    torch.cuda.synchronize()
    o_sc = E.score_rows("esdllm", lay["h_cur"], lay["h_prev"], lay["conf"], 0.5)
    g_sc = host(scores[0])
    assert np.abs(g_sc - o_sc).max() <= 1e-5 * np.abs(o_sc).max()
    k = E.keep_count(keep, lay["S"])
    g_sel = sel.rows()[0]
    assert len(g_sel) == k and g_sel == sorted(g_sel)
    assert int(sel.row_off[1]) == k
    ok, nd, _ = topk_within_band(g_sel, np.arange(lay["S"]), o_sc, k)
    assert ok and nd == 0, f"{nd} rows differ"


def test_changed_rows_win_when_confidence_is_flat(lay):
    """With every confidence equal, eq. I ranks rows by their relative L1
    change alone, so keeping as many rows as were given the large change keeps
    exactly those rows."""
    D = lay["D"]
    sel = D.SelectionTensors(1, lay["S"])
    flat = torch.full_like(lay["st"]["conf"], 0.5)
    changed = lay["st"]["changed_rows"].tolist()
    keep = len(changed) / lay["S"]                       # 102/512, exact in float32
    D.dl_score_select(lay["dims"], lay["st"]["h_cur"], lay["st"]["h_prev"], flat, lay["seq_len"], "esdllm", 0.5,
                      D.DL_SEL_TOPK, keep, 0.0, sel, ws=lay["ws"])
    torch.cuda.synchronize()
    assert len(changed) == E.keep_count(keep, lay["S"])
    assert sel.rows()[0] == changed


def test_threshold_select(lay):
    D = lay["D"]
    sel = D.SelectionTensors(1, lay["S"])
    o_sc = E.score_rows("esdllm", lay["h_cur"], lay["h_prev"], lay["conf"], 0.5)
    tau = float(np.sort(o_sc)[::-1][99] + np.sort(o_sc)[::-1][100]) / 2     # between the 100th and 101st
    D.dl_score_select(lay["dims"], lay["st"]["h_cur"], lay["st"]["h_prev"], lay["st"]["conf"], lay["seq_len"],
                      "esdllm", 0.5, D.DL_SEL_THRESHOLD, 1.0, tau, sel, ws=lay["ws"])
    torch.cuda.synchronize()
    assert sel.rows()[0] == E.select_threshold(o_sc, tau).tolist()


@pytest.mark.parametrize("keep", [1.0, 0.75, 0.55, 0.25, 0.125, 0.078, 0.04])
def test_partial_layer_matches_oracle(lay, keep):
    """Attention + FFN sub-blocks on the selected rows against stale K/V.
    384 and 282 rows leave the second 256-row tile of the gate|up and split-K
    products full up to one epilogue pass, and ragged inside it; 40 rows run
    the 128-row tiles mostly empty, 21 rows the weight-streaming kernel.
    The rows' log softmax normalisers (dl_partial_attn's optional output)
    against the oracle's, and asking for them leaves the layer output
    bit-identical."""
    D = lay["D"]
    wl, S, d = lay["wl"], lay["S"], lay["wl"].dims.d
    o_sc = E.score_rows("esdllm", lay["h_cur"], lay["h_prev"], lay["conf"], 0.5)
    rows = E.select_topk(o_sc, E.keep_count(keep, S))
    k = len(rows)
    sel = D.SelectionTensors(1, S)
    sel.sel_idx[0, :k] = torch.as_tensor(rows, dtype=torch.int32)
    sel.sel_count[0] = k
    sel.row_off[1] = k
    x = lay["st"]["h_cur"][0:S].float()[torch.as_tensor(rows, device="cuda")].contiguous()
    kc = lay["st"]["k"].clone().reshape(1, S, d)
    vc = lay["st"]["v"].clone().reshape(1, S, d)
    lw = lay["m"]["layers"][0]
    x_plain = x.clone()
    lse = torch.full((k, wl.dims.n_heads), float("nan"), dtype=torch.float32, device="cuda")
    D.dl_partial_attn(lay["dims"], lw, x, sel, lay["seq_len"], k, kc, vc, lay["ws"], lse=lse)
    D.dl_ffn_rows(lay["dims"], lw, x, sel, k, lay["ws"])
    D.dl_partial_attn(lay["dims"], lw, x_plain, sel, lay["seq_len"], k, kc.clone(), vc.clone(), lay["ws"])
    D.dl_ffn_rows(lay["dims"], lw, x_plain, sel, k, lay["ws"])
    torch.cuda.synchronize()
    assert torch.equal(x, x_plain)
    K = host(lay["st"]["k"])
    V = host(lay["st"]["v"])
    y, _, _, o_lse = E.layer_parts(lay["h_cur"][rows], rows, lay["lw_np"], K, V, S, wl.dims)
    assert row_rel_err(host(x), y) <= TOL
    assert lse_err(host(lse), o_lse) <= TOL
    assert row_rel_err(host(kc[0])[rows], K[rows]) <= TOL
    assert row_rel_err(host(vc[0])[rows], V[rows]) <= TOL
    other = np.setdiff1d(np.arange(S), rows)
    assert torch.equal(kc[0][other], lay["st"]["k"][other]) and torch.equal(vc[0][other], lay["st"]["v"][other])


def test_lm_head_rows_matches_oracle(lay):
    D = lay["D"]
    S, d, V = lay["S"], lay["wl"].dims.d, lay["wl"].dims.vocab
    rows = np.arange(3, S, 4)                              # 128 rows
    k = len(rows)
    sel = D.SelectionTensors(1, S)
    sel.sel_idx[0, :k] = torch.as_tensor(rows, dtype=torch.int32)
    sel.sel_count[0] = k
    sel.row_off[1] = k
    x = lay["st"]["h_cur"].float()[torch.as_tensor(rows, device="cuda")].contiguous()
    conf = torch.full((1, S), -1.0, device="cuda")
    amax = torch.full((1, S), -1, dtype=torch.int32, device="cuda")
    hfin = torch.zeros((1, S, d), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros((1, S, V), dtype=torch.float32, device="cuda")
    D.dl_lm_head_rows(lay["dims"], lay["m"]["final_norm"], lay["m"]["lm_head"], x, sel, k, conf, amax, hfin, logits,
                      lay["ws"])
    torch.cuda.synchronize()
    lg = E.lm_logits(lay["h_cur"][rows], host(lay["m"]["final_norm"]), host(lay["m"]["lm_head"]), 1e-5)
    c, a = E.conf_argmax(lg)
    assert row_rel_err(host(logits[0])[rows], lg) <= TOL
    assert np.abs(host(conf[0])[rows] - c).max() <= TOL * c.max()
    srt = np.sort(lg, axis=1)
    clear = (srt[:, -1] - srt[:, -2]) > 1e-2 * np.abs(lg).max(axis=1)
    assert clear.sum() > k // 2
    assert np.array_equal(amax[0].cpu().numpy()[rows][clear], a[clear])
    other = np.setdiff1d(np.arange(S), rows)
    assert (conf[0][other] == -1).all() and (amax[0][other] == -1).all()
    assert torch.equal(hfin[0][torch.as_tensor(rows, device="cuda")], x.to(torch.bfloat16))


def test_gather_scatter_roundtrip(lay):
    D = lay["D"]
    S, d = lay["S"], lay["wl"].dims.d
    g = torch.Generator(device="cuda").manual_seed(5)
    rows = torch.randperm(S, generator=g, device="cuda")[:77].sort().values.to(torch.int32)
    sel = D.SelectionTensors(1, S)
    sel.sel_idx[0, :77] = rows
    sel.sel_count[0] = 77
    sel.row_off[1] = 77
    src = lay["st"]["h_cur"].reshape(1, S, d)
    dst = torch.empty((77, d), dtype=torch.bfloat16, device="cuda")
    D.dl_gather(lay["dims"], src, d, D.DL_BF16, sel, 77, dst)
    cache = torch.zeros((1, S, d), dtype=torch.bfloat16, device="cuda")
    D.dl_scatter_cache(lay["dims"], dst, d, D.DL_BF16, sel, 77, cache)
    torch.cuda.synchronize()
    assert torch.equal(dst, src[0][rows.long()])
    assert torch.equal(cache[0][rows.long()], dst)
    mask = torch.ones(S, dtype=torch.bool, device="cuda")
    mask[rows.long()] = False
    assert (cache[0][mask] == 0).all()


def test_unmask_matches_oracle(lay):
    D = lay["D"]
    S = lay["S"]
    rng = np.random.default_rng(9)
    conf = rng.choice(np.array([0.1, 0.2, 0.2, 0.5, 0.9], np.float32), size=S)
    masked = (rng.uniform(size=S) < 0.7).astype(np.uint8)
    masked[:100] = 0
    prompt = torch.tensor([100], dtype=torch.int32, device="cuda")
    for block, bl, n in ((0, 32, 1), (2, 32, 5), (3, 64, 64), (0, 412, 7)):
        tok = torch.full((1, S), 7, dtype=torch.int32, device="cuda")
        am = torch.arange(S, dtype=torch.int32, device="cuda").reshape(1, S)
        msk = torch.as_tensor(masked).reshape(1, S).cuda()
        D.dl_unmask(lay["dims"], tok, msk, torch.as_tensor(conf).reshape(1, S).cuda(), am, prompt, lay["seq_len"],
                    block, bl, n)
        torch.cuda.synchronize()
        lo = 100 + block * bl
        want = E.unmask(masked.astype(bool), conf.astype(np.float64), lo, min(lo + bl, S), n)
        got = np.nonzero(masked.astype(bool) & ~msk[0].cpu().numpy().astype(bool))[0]
        assert got.tolist() == want.tolist()
        assert (tok[0].cpu().numpy()[want] == want).all()


def test_timing_counts_products_and_keeps_results(lay):
    """Sampled kernel timing (events bound to the products' dispatch packets):
    with stride 1 the four products of a kept-row layer are each timed once,
    their algorithmic bytes add up to the closed form, and the layer's output
    is bit-identical to an untimed run."""
    D = lay["D"]
    S, d, F = lay["S"], lay["wl"].dims.d, lay["wl"].dims.d_ffn
    k = 128
    rows = np.arange(0, S, S // k)[:k]
    sel = D.SelectionTensors(1, S)
    sel.sel_idx[0, :k] = torch.as_tensor(rows, dtype=torch.int32)
    sel.sel_count[0] = k
    sel.row_off[1] = k
    lw = lay["m"]["layers"][0]
    x0 = lay["st"]["h_cur"][0:S].float()[torch.as_tensor(rows, device="cuda")].contiguous()

    def run(timed):
        x = x0.clone()
        kc = lay["st"]["k"].clone().reshape(1, S, d)
        vc = lay["st"]["v"].clone().reshape(1, S, d)
        D.dl_timing_reset()
        D.dl_timing_enable(D.DL_KC_GEMM, 1 if timed else 0)
        D.dl_partial_attn(lay["dims"], lw, x, sel, lay["seq_len"], k, kc, vc, lay["ws"])
        D.dl_ffn_rows(lay["dims"], lw, x, sel, k, lay["ws"])
        torch.cuda.synchronize()
        t = D.dl_timing_read(D.DL_KC_GEMM)
        D.dl_timing_enable(D.DL_KC_GEMM, 0)
        return x, t

    x_plain, t_plain = run(False)
    x_timed, t = run(True)
    assert t_plain["launches"] == 0
    assert torch.equal(x_plain, x_timed)
    assert t["launches"] == 4 and t["dropped"] == 0
    assert 0 < t["ms"] < 10.0
    gemm = lambda M, N, K: 2.0 * (N * K + M * K + M * N)        # bf16 weights + rows in + rows out
    want = gemm(k, 3 * d, d) + gemm(k, d, d) + gemm(k, 2 * F, d) + gemm(k, d, F)
    assert t["bytes"] == pytest.approx(want, rel=1e-12)
    assert t["flops"] == pytest.approx(2.0 * k * d * (3 * d + d + 2 * F) + 2.0 * k * F * d, rel=1e-12)


def test_pack_weights_is_the_blocked_permutation(lay):
    """dl_pack_weights puts element (n, k) of a row-major [N, K] matrix at
    ((n/8)(K/64) + k/64)*512 + (n%8)*64 + k%64: the matrix cut into 8 x 64
    blocks, blocks of a row group in K order."""
    D = lay["D"]
    for w in (lay["m"]["layers"][0]["wq"], lay["m"]["layers"][0]["w_down"], lay["m"]["lm_head"][:4104]):
        w = w.contiguous()
        N, K = w.shape
        out = torch.empty_like(w)
        D.dl_pack_weights(w, out)
        torch.cuda.synchronize()
        want = w.view(torch.int16).reshape(N // 8, 8, K // 64, 64).permute(0, 2, 1, 3).reshape(N, K)
        assert torch.equal(out.view(torch.int16), want)


@pytest.mark.parametrize("keep", [1.0, 0.25, 0.04])
def test_blocked_weights_bit_identical(lay, keep):
    """The one-layer entry points with the layer's product weights and the
    LM head in the blocked order give the same rows, caches and LM outputs,
    bit for bit, as with row-major weights (512 rows on the 128-row tiles, 128
    kept rows, 21 rows on the weight-streaming kernel)."""
    from dynamic_token_skipping_amd import pack_model
    D = lay["D"]
    wl, S, d = lay["wl"], lay["S"], lay["wl"].dims.d
    dm = wl.dims
    o_sc = E.score_rows("esdllm", lay["h_cur"], lay["h_prev"], lay["conf"], 0.5)
    rows = E.select_topk(o_sc, E.keep_count(keep, S))
    k = len(rows)
    sel = D.SelectionTensors(1, S)
    sel.sel_idx[0, :k] = torch.as_tensor(rows, dtype=torch.int32)
    sel.sel_count[0] = k
    sel.row_off[1] = k
    x0 = lay["st"]["h_cur"][0:S].float()[torch.as_tensor(rows, device="cuda")].contiguous()
    one = {"layers": [lay["m"]["layers"][0]], "lm_head": lay["m"]["lm_head"], "final_norm": lay["m"]["final_norm"]}
    packed = pack_model(one)
    outs = []
    for layout, mw in (("row_major", one), ("blocked", packed)):
        dims = D.make_dims(1, S, d, dm.n_heads, dm.head_dim, dm.d_ffn, dm.vocab, 1, "bf16", weight_layout=layout)
        x = x0.clone()
        kc = lay["st"]["k"].clone().reshape(1, S, d)
        vc = lay["st"]["v"].clone().reshape(1, S, d)
        conf = torch.zeros((1, S), dtype=torch.float32, device="cuda")
        am = torch.zeros((1, S), dtype=torch.int32, device="cuda")
        hf = torch.zeros((1, S, d), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((1, S, dm.vocab), dtype=torch.float32, device="cuda")
        lw = mw["layers"][0]
        D.dl_partial_attn(dims, lw, x, sel, lay["seq_len"], k, kc, vc, lay["ws"])
        D.dl_ffn_rows(dims, lw, x, sel, k, lay["ws"])
        D.dl_lm_head_rows(dims, mw["final_norm"], mw["lm_head"], x, sel, k, conf, am, hf, lg, lay["ws"])
        torch.cuda.synchronize()
        outs.append((x, kc, vc, conf, am, hf, lg))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    del packed, outs


@pytest.mark.parametrize("keep", [1.0, 0.25, 0.04])
def test_row_map_reuse_is_bit_identical(lay, keep):
    """A selection carrying its own row map (filled by dl_score_select with
    row_off in one launch) gives the row entry points exactly the results of
    one without (each call building its map in the workspace); the map holds
    each packed row's flat position and sequence, -1 / 0 past the last row,
    and the 64-row attention tiles in order."""
    D = lay["D"]
    S, d, V = lay["S"], lay["wl"].dims.d, lay["wl"].dims.vocab
    st = lay["st"]
    sels = [D.SelectionTensors(1, S), D.SelectionTensors(1, S, row_map=True)]
    for sel in sels:
        D.dl_score_select(lay["dims"], st["h_cur"], st["h_prev"], st["conf"], lay["seq_len"], "esdllm", 0.5,
                          D.DL_SEL_TOPK, keep, 0.0, sel, ws=lay["ws"])
    torch.cuda.synchronize()
    a, b = sels
    assert torch.equal(a.sel_idx, b.sel_idx) and torch.equal(a.sel_count, b.sel_count)
    assert torch.equal(a.row_off, b.row_off)
    k = int(a.sel_count[0])
    assert k == E.keep_count(keep, S)
    m = b.row_map.cpu().numpy()
    T = (S + 63) // 64 + 1
    assert len(m) == 1 + 2 * S + 2 * T and m[0] == k
    assert np.array_equal(m[1:1 + k], a.sel_idx[0, :k].cpu().numpy()) and (m[1 + k:1 + S] == -1).all()
    assert (m[1 + S:1 + 2 * S] == 0).all()
    n_t = (k + 63) // 64
    t0, tr = m[1 + 2 * S:1 + 2 * S + T], m[1 + 2 * S + T:]
    assert np.array_equal(t0[:n_t], np.arange(n_t) * 64) and tr[:n_t].sum() == k and (tr[n_t:] == 0).all()
    rows = a.sel_idx[0, :k].long()
    lw = lay["m"]["layers"][0]
    outs = []
    for sel in sels:
        x = st["h_cur"][0:S].float()[rows].contiguous()
        kc = st["k"].clone().reshape(1, S, d)
        vc = st["v"].clone().reshape(1, S, d)
        D.dl_partial_attn(lay["dims"], lw, x, sel, lay["seq_len"], k, kc, vc, lay["ws"])
        D.dl_ffn_rows(lay["dims"], lw, x, sel, k, lay["ws"])
        conf = torch.full((1, S), -1.0, device="cuda")
        amax = torch.full((1, S), -1, dtype=torch.int32, device="cuda")
        hfin = torch.zeros((1, S, d), dtype=torch.bfloat16, device="cuda")
        logits = torch.zeros((1, S, V), dtype=torch.float32, device="cuda")
        D.dl_lm_head_rows(lay["dims"], lay["m"]["final_norm"], lay["m"]["lm_head"], x, sel, k, conf, amax, hfin,
                          logits, lay["ws"])
        torch.cuda.synchronize()
        outs.append((x, kc, vc, conf, amax, hfin, logits))
    for u, v in zip(*outs):
        assert torch.equal(u, v)
    del outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("keep,extra", [(0.25, 64), (0.25, 8), (0.04, 64)])
def test_stale_tail_rows_and_workspace_do_not_leak(lay, keep, extra):
    """The row kernels may read packed rows past the selection's count (up to
    k_total_max) and stale workspace bytes before the device-side row count
    arrives; what they store must not depend on them.  NaN in the tail rows
    of x_rows and in every workspace byte leaves the first k rows, the K/V
    caches, h_final, the logits and the confidence statistics bit-identical
    to a run over zeroed buffers, and the tail rows unwritten."""
    D = lay["D"]
    S, d, V = lay["S"], lay["wl"].dims.d, lay["wl"].dims.vocab
    st = lay["st"]
    sel = D.SelectionTensors(1, S, row_map=True)
    D.dl_score_select(lay["dims"], st["h_cur"], st["h_prev"], st["conf"], lay["seq_len"], "esdllm", 0.5,
                      D.DL_SEL_TOPK, keep, 0.0, sel, ws=lay["ws"])
    torch.cuda.synchronize()
    k = int(sel.sel_count[0])
    kmax = min(S, k + extra)
    assert k == E.keep_count(keep, S) and kmax > k
    rows = sel.sel_idx[0, :k].long()
    lw = lay["m"]["layers"][0]
    outs = []
    for poison in (False, True):
        ws = D.workspace(lay["dims"], kmax)
        ws.fill_(255 if poison else 0)                # 0xff bytes: NaN in fp32 and bf16
        x = torch.full((kmax, d), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
        x[:k] = st["h_cur"][0:S].float()[rows]
        kc = st["k"].clone().reshape(1, S, d)
        vc = st["v"].clone().reshape(1, S, d)
        D.dl_partial_attn(lay["dims"], lw, x, sel, lay["seq_len"], kmax, kc, vc, ws)
        D.dl_ffn_rows(lay["dims"], lw, x, sel, kmax, ws)
        conf = torch.full((1, S), -1.0, device="cuda")
        amax = torch.full((1, S), -1, dtype=torch.int32, device="cuda")
        hfin = torch.zeros((1, S, d), dtype=torch.bfloat16, device="cuda")
        logits = torch.zeros((1, S, V), dtype=torch.float32, device="cuda")
        D.dl_lm_head_rows(lay["dims"], lay["m"]["final_norm"], lay["m"]["lm_head"], x, sel, kmax, conf, amax, hfin,
                          logits, ws)
        torch.cuda.synchronize()
        if poison:
            assert torch.isnan(x[k:]).all()              # tail rows read at most, never written
        assert torch.isfinite(x[:k]).all()
        outs.append((x[:k].clone(), kc, vc, conf, amax, hfin, logits))
        del ws
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    del outs
