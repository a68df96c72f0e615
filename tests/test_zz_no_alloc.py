"""The no-allocation denoising step (dl_denoise_step_noalloc, the library's
built-in scratch as workspace) against the workspace entry point on
identical states through the C ABI: bit-identical results over refresh and
skip steps, for two inputs in a row, the second smaller; and a step larger
than the scratch rejected before anything is enqueued."""
import ctypes

import pytest
import torch

import workloads
from gpu_util import to_device

pytestmark = pytest.mark.gpu

DIMS = workloads.ModelDims(d=256, n_heads=2, head_dim=128, d_ffn=512, vocab=1024, n_layers=3)
SCHED = workloads.Schedule(gen_len=32, block_len=16, steps=8, skip_layer=1, keep=0.25, score="esdllm")
FIELDS = ("tokens", "masked", "h_prev", "k_cache", "v_cache", "h_final", "conf", "argmax", "logits", "scores")


def _pair(prompt_lens, seed, sched=SCHED):
    from dynamic_token_skipping_amd import Decoder, DeviceModel
    m = to_device(workloads.make_model(DIMS, seed, "bf16", "cpu"))
    g = torch.Generator().manual_seed(seed)
    prompts = [torch.randint(0, DIMS.vocab, (n,), generator=g) for n in prompt_lens]
    dm = DeviceModel(m, DIMS.n_heads, DIMS.head_dim, "bf16")
    return Decoder(dm, prompts, sched, keep_logits=True), Decoder(dm, prompts, sched, keep_logits=True)


def _same(a, b, what):
    for f in FIELDS:
        assert torch.equal(getattr(a, f), getattr(b, f)), (what, f)
    assert a.sel.rows() == b.sel.rows(), what


@pytest.mark.parametrize("case", [((9, 45, 96), 21, 4), ((5, 20), 22, 3)], ids=["three_seqs", "two_shorter"])
def test_noalloc_step_matches_workspace_step(case):
    """Both inputs run in one process, the larger first (parametrised in that
    order), so the second call meets the scratch holding the first's bytes."""
    import dynamic_token_skipping_amd as D
    lens, seed, steps = case
    a, b = _pair(lens, seed)
    assert D.workspace_bytes(a.dims, sum(a.seq_lens)) <= D.NOALLOC_SCRATCH_BYTES
    for t in range(steps):
        a.step(t)
        D.dl_denoise_step_noalloc(b.model_struct, b.state, b.params(t))
        torch.cuda.synchronize()
        _same(a, b, (lens, t))
    assert a.sel.rows() != [list(range(n)) for n in a.seq_lens]   # the last step was a skip step


def test_noalloc_two_calls_in_a_row_second_smaller():
    """A larger step then a smaller one through the no-allocation entry
    point, each against the workspace entry point."""
    import dynamic_token_skipping_amd as D
    for lens, seed in (((40, 70, 120), 31), ((3,), 32)):
        a, b = _pair(lens, seed)
        for t in range(3):
            a.step(t)
            D.dl_denoise_step_noalloc(b.model_struct, b.state, b.params(t))
            torch.cuda.synchronize()
            _same(a, b, (lens, t))


def test_noalloc_rejects_a_step_beyond_its_scratch():
    """The long-context 8B-class shape needs about 1.2 GB of workspace: the
    call returns DL_E_WORKSPACE and touches nothing (every pointer below
    refers to one small buffer, which stays unchanged)."""
    import dynamic_token_skipping_amd as D
    from dynamic_token_skipping_amd import _lib as L
    buf = torch.full((4096,), 7, dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    dims = L.make_dims(1, 4608, 4096, 32, 128, 11008, 126464, 32, "bf16")
    assert D.workspace_bytes(dims, 4608) > D.NOALLOC_SCRATCH_BYTES
    layers = (L.LayerW * 32)(*[L.LayerW(*([p] * 9)) for _ in range(32)])
    model = L.Model(dims, p, p, p, layers)
    sel = L.Selection(p, p, p)
    state = L.State(p, p, p, p, p, p, p, p, p, p, None, None, sel, None, None, L.Selection(), None, None, None, None,
                    None, L.Selection())
    lens = (ctypes.c_int32 * 1)(4608)
    prompt = (ctypes.c_int32 * 1)(4096)
    lp = ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32))
    pp = ctypes.cast(prompt, ctypes.POINTER(ctypes.c_int32))
    params = L.StepParams(0, 64, 1, 4, 0, L.DL_SCORE_ESDLLM, 0.5, L.DL_SEL_TOPK, 0.125, 0.0, lp, 0, pp, 0,
                          L.DL_SEL_TOPK, 1.0, 0.0, L.DL_TENSOR_HIDDEN, 0, L.DL_SEL_TOPK, 0.125, 0.0)
    with pytest.raises(L.DLError) as e:
        D.dl_denoise_step_noalloc(model, state, params)
    torch.cuda.synchronize()
    assert e.value.status == -5 and "scratch" in str(e.value)
    assert bool((buf == 7).all())
