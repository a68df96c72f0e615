"""GPU parity of the attention sub-block on a ragged batch at sizes where the
matrix-core kernel splits the keys of each sequence into chunks (and, at
keep 1, where it does not), and with 32 heads, where enough (query tile,
head) pairs take the single-pass kernel that covers every key of a pair in
one workgroup: dl_partial_attn + dl_ffn_rows against the oracle layer on
every selected row, and the K/V rows it must leave alone."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import host, lse_err, row_rel_err
from oracle import esdllm as E

pytestmark = pytest.mark.gpu
TOL = 2e-2
DIMS = workloads.ModelDims(d=512, n_heads=4, head_dim=128, d_ffn=1024, vocab=256, n_layers=1)
S = 640
LENS = (640, 333, 77)     # full, ragged last chunk, shorter than one chunk


# 32 heads: 448 + 333 + 77 rows make 15 query tiles, 480 (tile, head) pairs
DIMS32 = workloads.ModelDims(d=4096, n_heads=32, head_dim=128, d_ffn=1024, vocab=256, n_layers=1)
LENS32 = (448, 333, 77)


@pytest.fixture(scope="module", params=["4_heads", "32_heads"])
def setup(request):
    import dynamic_token_skipping_amd as D
    DIMS, S, LENS = (globals()["DIMS"], globals()["S"], globals()["LENS"]) if request.param == "4_heads" else (
        DIMS32, max(LENS32), LENS32)
    m = workloads.make_model(DIMS, 31, "bf16", "cuda")
    g = torch.Generator(device="cuda").manual_seed(32)
    B = len(LENS)
    kc0 = (torch.randn((B, S, DIMS.d), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    vc0 = torch.randn((B, S, DIMS.d), generator=g, device="cuda").to(torch.bfloat16)
    x0 = torch.randn((B, S, DIMS.d), generator=g, device="cuda")
    dims = D.make_dims(B, S, DIMS.d, DIMS.n_heads, DIMS.head_dim, DIMS.d_ffn, DIMS.vocab, 1, "bf16")
    ws = D.workspace(dims, B * S)
    seq_len = torch.tensor(LENS, dtype=torch.int32, device="cuda")
    lw_np = {k: host(v) for k, v in m["layers"][0].items()}
    return dict(D=D, m=m, kc0=kc0, vc0=vc0, x0=x0, dims=dims, ws=ws, seq_len=seq_len, lw_np=lw_np, DIMS=DIMS, S=S,
                LENS=LENS)


@pytest.mark.parametrize("keep", [1.0, 0.75, 0.5, 0.25, 0.05])
def test_ragged_partial_layer_matches_oracle(setup, keep):
    D = setup["D"]
    DIMS, S, LENS = setup["DIMS"], setup["S"], setup["LENS"]
    B = len(LENS)
    sel = D.SelectionTensors(B, S)
    rows = []
    for b, n in enumerate(LENS):
        k = E.keep_count(keep, n)
        r = np.unique(np.linspace(0, n - 1, k).round().astype(np.int64))
        rows.append(r)
        sel.sel_idx[b, :len(r)] = torch.as_tensor(r, dtype=torch.int32)
        sel.sel_count[b] = len(r)
    off = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    sel.row_off.copy_(torch.as_tensor(off, dtype=torch.int32))
    R = int(off[-1])
    x = torch.cat([setup["x0"][b, torch.as_tensor(rows[b], device="cuda")] for b in range(B)]).contiguous()
    kc, vc = setup["kc0"].clone(), setup["vc0"].clone()
    lw = setup["m"]["layers"][0]
    lse = torch.full((R + 3, DIMS.n_heads), float("nan"), dtype=torch.float32, device="cuda")
    D.dl_partial_attn(setup["dims"], lw, x, sel, setup["seq_len"], R, kc, vc, setup["ws"], lse=lse)
    D.dl_ffn_rows(setup["dims"], lw, x, sel, R, setup["ws"])
    torch.cuda.synchronize()
    xg = host(x)
    lg = host(lse)
    assert np.isnan(lg[R:]).all()                      # rows past row_off[B] untouched
    for b, n in enumerate(LENS):
        K = host(setup["kc0"][b, :n])
        V = host(setup["vc0"][b, :n])
        y, _, _, o_lse = E.layer_parts(host(setup["x0"][b])[rows[b]], rows[b], setup["lw_np"], K, V, n, DIMS)
        assert row_rel_err(xg[off[b]:off[b + 1]], y) <= TOL, f"sequence {b}"
        assert lse_err(lg[off[b]:off[b + 1]], o_lse) <= TOL, f"sequence {b}"
        assert row_rel_err(host(kc[b])[rows[b]], K[rows[b]]) <= TOL
        assert row_rel_err(host(vc[b])[rows[b]], V[rows[b]]) <= TOL
        other = np.setdiff1d(np.arange(S), rows[b])
        assert torch.equal(kc[b][other], setup["kc0"][b][other])
        assert torch.equal(vc[b][other], setup["vc0"][b][other])


@pytest.mark.parametrize("keep", [1.0, 0.25, 0.05])
def test_ragged_row_map_reuse_is_bit_identical(setup, keep):
    """A ragged batch selected by dl_score_select with and without the
    selection's own row map: the map holds b * S + position and b for every
    packed row (-1 / 0 past the last), and each sequence's rows in 64-row
    attention tiles in order; dl_partial_attn and dl_ffn_rows give
    bit-identical rows and caches either way."""
    D = setup["D"]
    DIMS, S, LENS = setup["DIMS"], setup["S"], setup["LENS"]
    B = len(LENS)
    g = torch.Generator(device="cuda").manual_seed(41)
    h_prev = torch.randn((B, S, DIMS.d), generator=g, device="cuda").to(torch.bfloat16)
    h_cur = (h_prev.float() + 0.3 * torch.randn((B, S, DIMS.d), generator=g, device="cuda")).to(torch.bfloat16)
    conf = torch.rand((B, S), generator=g, device="cuda")
    sels = [D.SelectionTensors(B, S), D.SelectionTensors(B, S, row_map=True)]
    for sel in sels:
        D.dl_score_select(setup["dims"], h_cur, h_prev, conf, setup["seq_len"], "esdllm", 0.5, D.DL_SEL_TOPK, keep,
                          0.0, sel, ws=setup["ws"])
    torch.cuda.synchronize()
    a, b_ = sels
    assert torch.equal(a.sel_idx, b_.sel_idx) and torch.equal(a.sel_count, b_.sel_count)
    assert torch.equal(a.row_off, b_.row_off)
    cnt = a.sel_count.cpu().tolist()
    assert cnt == [E.keep_count(keep, n) for n in LENS]
    off = a.row_off.cpu().tolist()
    R = off[-1]
    m = b_.row_map.cpu().numpy()
    BS = B * S
    T = (BS + 63) // 64 + B
    assert len(m) == 1 + 2 * BS + 2 * T and m[0] == R
    idx = a.sel_idx.cpu().numpy()
    want_pos = np.concatenate([bb * S + idx[bb, :c] for bb, c in enumerate(cnt)])
    want_seq = np.concatenate([np.full(c, bb) for bb, c in enumerate(cnt)])
    assert np.array_equal(m[1:1 + R], want_pos) and (m[1 + R:1 + BS] == -1).all()
    assert np.array_equal(m[1 + BS:1 + BS + R], want_seq) and (m[1 + BS + R:1 + 2 * BS] == 0).all()
    t0, tr = m[1 + 2 * BS:1 + 2 * BS + T], m[1 + 2 * BS + T:]
    want_t0, want_tr = [], []
    for bb, c in enumerate(cnt):
        for j in range(0, c, 64):
            want_t0.append(off[bb] + j)
            want_tr.append(min(64, c - j))
    nt = len(want_t0)
    assert np.array_equal(t0[:nt], want_t0) and np.array_equal(tr[:nt], want_tr) and (tr[nt:] == 0).all()
    lw = setup["m"]["layers"][0]
    outs = []
    for sel in sels:
        rows = [idx[bb, :c] for bb, c in enumerate(cnt)]
        x = torch.cat([setup["x0"][bb, torch.as_tensor(rows[bb], device="cuda", dtype=torch.long)]
                       for bb in range(B)]).contiguous()
        kc, vc = setup["kc0"].clone(), setup["vc0"].clone()
        D.dl_partial_attn(setup["dims"], lw, x, sel, setup["seq_len"], R, kc, vc, setup["ws"])
        D.dl_ffn_rows(setup["dims"], lw, x, sel, R, setup["ws"])
        torch.cuda.synchronize()
        outs.append((x, kc, vc))
    for u, v in zip(*outs):
        assert torch.equal(u, v)


def test_fp32_partial_attn_lse_matches_oracle():
    """fp32 storage (the SIMT attention kernel): dl_partial_attn's rows and
    their log softmax normalisers on a ragged batch of two sequences against
    the oracle layer, within 1e-5."""
    import dynamic_token_skipping_amd as D
    dims = workloads.ModelDims(d=64, n_heads=2, head_dim=32, d_ffn=128, vocab=64, n_layers=1)
    lens = (40, 17)
    B, S = len(lens), max(lens)
    m = workloads.make_model(dims, 7, "f32", "cuda")
    g = torch.Generator(device="cuda").manual_seed(8)
    kc0 = torch.randn((B, S, dims.d), generator=g, device="cuda")
    vc0 = torch.randn((B, S, dims.d), generator=g, device="cuda")
    x0 = torch.randn((B, S, dims.d), generator=g, device="cuda")
    sel = D.SelectionTensors(B, S)
    rows = []
    for b, n in enumerate(lens):
        r = np.arange(1, n, 2)
        rows.append(r)
        sel.sel_idx[b, :len(r)] = torch.as_tensor(r, dtype=torch.int32)
        sel.sel_count[b] = len(r)
    off = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    sel.row_off.copy_(torch.as_tensor(off, dtype=torch.int32))
    R = int(off[-1])
    x = torch.cat([x0[b, torch.as_tensor(rows[b], device="cuda")] for b in range(B)]).contiguous()
    dl = D.make_dims(B, S, dims.d, dims.n_heads, dims.head_dim, dims.d_ffn, dims.vocab, 1, "f32")
    ws = D.workspace(dl, R)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kc, vc = kc0.clone(), vc0.clone()
    lse = torch.full((R, dims.n_heads), float("nan"), dtype=torch.float32, device="cuda")
    lw = m["layers"][0]
    D.dl_partial_attn(dl, lw, x, sel, seq_len, R, kc, vc, ws, lse=lse)
    D.dl_ffn_rows(dl, lw, x, sel, R, ws)
    torch.cuda.synchronize()
    lw_np = {k: host(v) for k, v in lw.items()}
    xg, lg = host(x), host(lse)
    for b, n in enumerate(lens):
        K = host(kc0[b, :n])
        V = host(vc0[b, :n])
        y, _, _, o_lse = E.layer_parts(host(x0[b])[rows[b]], rows[b], lw_np, K, V, n, dims)
        assert row_rel_err(xg[off[b]:off[b + 1]], y) <= 1e-5, f"sequence {b}"
        assert lse_err(lg[off[b]:off[b + 1]], o_lse) <= 1e-5, f"sequence {b}"


# (model, sequence lengths, cached keys zero below this position, key size
# factor after it).  keep < 1, so that most keys stay the cached ones (a
# selected row's key is recomputed); the scores then reach 23-31 (log2
# units) and each case sees a few hundred jumps of more than 8 and many
# smaller rises, with about 1% of the increment from bf16 rounding alone
JUMP_CASES = {
    "key_chunks": (DIMS, (1600, 1111), 700, 15.0),     # > 1024 keys: k_attn_mfma, keys in chunks
    "rows_16q": (DIMS, (1000, 777), 400, 15.0),        # k_attn_rows, 16 queries x 8 key parts
    "rows_64q": (DIMS32, (900, 333), 400, 7.0),        # k_attn_rows, 64 queries x 2 key parts
}


@pytest.mark.parametrize("case,keep", [("key_chunks", 0.5), ("key_chunks", 0.25), ("rows_16q", 0.25),
                                       ("rows_64q", 0.5)])
def test_attention_with_jumping_scores(case, keep):
    """The attention kernels rescale their softmax lazily: a query's
    reference max moves only when a tile brings a score more than 8 (log2
    units) above it, and the probabilities of the other tiles stay relative
    to the old max (up to 2^8).  Cached keys that are exactly zero up to a
    position and a few times the usual size after it make every query's max
    jump by more than 8 inside a key range and then drift by less; the
    attention increment of each row and the log normalisers still match the
    oracle, ragged sequences (a last tile masked, or keys all zero) included.
    Each case drives one kernel shape (at keep 0.5 the key-chunk kernel runs
    in one chunk over 1356 rows, at keep 0.25 in chunks merged afterwards)."""
    import dynamic_token_skipping_amd as D
    dm, lens, zero_until, kmul = JUMP_CASES[case]
    S_l, B = max(lens), len(lens)
    m = workloads.make_model(dm, 41, "bf16", "cuda")
    g = torch.Generator(device="cuda").manual_seed(42)
    kscale = torch.full((1, S_l, 1), kmul * 0.5, device="cuda")
    kscale[:, :zero_until] = 0.0
    kc0 = (torch.randn((B, S_l, dm.d), generator=g, device="cuda") * kscale).to(torch.bfloat16)
    vc0 = torch.randn((B, S_l, dm.d), generator=g, device="cuda").to(torch.bfloat16)
    x0 = torch.randn((B, S_l, dm.d), generator=g, device="cuda")
    dims = D.make_dims(B, S_l, dm.d, dm.n_heads, dm.head_dim, dm.d_ffn, dm.vocab, 1, "bf16")
    ws = D.workspace(dims, B * S_l)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lw_np = {k: host(v) for k, v in m["layers"][0].items()}
    sel = D.SelectionTensors(B, S_l)
    rows = []
    for b, n in enumerate(lens):
        r = np.unique(np.linspace(0, n - 1, E.keep_count(keep, n)).round().astype(np.int64))
        rows.append(r)
        sel.sel_idx[b, :len(r)] = torch.as_tensor(r, dtype=torch.int32)
        sel.sel_count[b] = len(r)
    off = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    sel.row_off.copy_(torch.as_tensor(off, dtype=torch.int32))
    R = int(off[-1])
    x = torch.cat([x0[b, torch.as_tensor(rows[b], device="cuda")] for b in range(B)]).contiguous()
    kc, vc = kc0.clone(), vc0.clone()
    lse = torch.full((R, dm.n_heads), float("nan"), dtype=torch.float32, device="cuda")
    D.dl_partial_attn(dims, m["layers"][0], x, sel, seq_len, R, kc, vc, ws, lse=lse)
    torch.cuda.synchronize()
    xg, lg = host(x), host(lse)
    for b, n in enumerate(lens):
        K, V = host(kc0[b, :n]), host(vc0[b, :n])
        xb = host(x0[b])[rows[b]]
        _, _, ctx, o_lse = E.layer_parts(xb, rows[b], lw_np, K, V, n, dm)
        # the sub-block adds Wo(attention) to x: compare that increment itself
        # (bf16 rounding of q, K and V alone accounts for about 1% of it here)
        att = ctx @ np.asarray(lw_np["wo"], np.float64).T
        assert row_rel_err(xg[off[b]:off[b + 1]] - xb, att) <= TOL, f"sequence {b}"
        assert lse_err(lg[off[b]:off[b + 1]], o_lse) <= TOL, f"sequence {b}"
