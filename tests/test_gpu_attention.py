"""GPU parity of the attention sub-block on a ragged batch at sizes where the
matrix-core kernel splits the keys of each sequence into chunks (and, at
keep 1, where it does not): dl_partial_attn + dl_ffn_rows against the oracle
layer on every selected row, and the K/V rows it must leave alone."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import host, row_rel_err
from oracle import esdllm as E

pytestmark = pytest.mark.gpu
TOL = 2e-2
DIMS = workloads.ModelDims(d=512, n_heads=4, head_dim=128, d_ffn=1024, vocab=256, n_layers=1)
S = 640
LENS = (640, 333, 77)     # full, ragged last chunk, shorter than one chunk


@pytest.fixture(scope="module")
def setup():
    import dynamic_token_skipping_amd as D
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
    return dict(D=D, m=m, kc0=kc0, vc0=vc0, x0=x0, dims=dims, ws=ws, seq_len=seq_len, lw_np=lw_np)


@pytest.mark.parametrize("keep", [1.0, 0.5, 0.25, 0.05])
def test_ragged_partial_layer_matches_oracle(setup, keep):
    D = setup["D"]
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
    D.dl_partial_attn(setup["dims"], lw, x, sel, setup["seq_len"], R, kc, vc, setup["ws"])
    D.dl_ffn_rows(setup["dims"], lw, x, sel, R, setup["ws"])
    torch.cuda.synchronize()
    xg = host(x)
    for b, n in enumerate(LENS):
        K = host(setup["kc0"][b, :n])
        V = host(setup["vc0"][b, :n])
        y = E.layer_forward(host(setup["x0"][b])[rows[b]], rows[b], setup["lw_np"], K, V, n, DIMS)
        assert row_rel_err(xg[off[b]:off[b + 1]], y) <= TOL, f"sequence {b}"
        assert row_rel_err(host(kc[b])[rows[b]], K[rows[b]]) <= TOL
        assert row_rel_err(host(vc[b])[rows[b]], V[rows[b]]) <= TOL
        other = np.setdiff1d(np.arange(S), rows[b])
        assert torch.equal(kc[b][other], setup["kc0"][b][other])
        assert torch.equal(vc[b][other], setup["vc0"][b][other])
