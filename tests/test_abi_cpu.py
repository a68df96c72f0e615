"""The C ABI without a GPU: the library loads, exports every symbol that
include/dl.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from dynamic_token_skipping_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "dl.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\S.*?\b(dl_[a-z_]+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_abi_version(lib):
    assert lib.dl_abi_version() == 5


def test_status_strings(lib):
    for code in range(-7, 1):
        assert lib.dl_status_string(code)


def _dims(**kw):
    base = dict(B=1, S=512, d=4096, n_heads=32, head_dim=128, d_ffn=11008, vocab=126464, n_layers=32, dtype="bf16")
    base.update(kw)
    return L.make_dims(**base)


def test_workspace_bytes(lib):
    a = L.workspace_bytes(_dims(), 128)
    b = L.workspace_bytes(_dims(), 512)
    assert 0 < a < b
    assert L.workspace_bytes(_dims(d=4000)) == 0          # d != H*dh


@pytest.mark.parametrize("kw,code", [
    (dict(d=4000), -2), (dict(head_dim=127, d=32 * 127), -2), (dict(dtype=7), -3), (dict(B=0), -1),
    (dict(S=9000, dtype="f32"), -7), (dict(B=2000), -7),
    (dict(vocab=262144), -7), (dict(S=261632), -7),
    (dict(weight_layout=2), -1), (dict(weight_layout="blocked", dtype="f32", S=512), -3),
    (dict(weight_layout="blocked", d_ffn=11000), -2), (dict(weight_layout="blocked", vocab=126463), -2),
])
def test_bad_dims_rejected(lib, kw, code):
    d = _dims(**kw)
    s = L.Selection(16, 16, 16)
    r = lib.dl_score_select(ctypes.byref(d), 16, 32, 16, 16, 0, 0.5, 0, 0.25, 0.0, ctypes.byref(s), None, 16, 1 << 30,
                            None)
    assert r == code, lib.dl_last_error()


def test_blocked_layout_accepted(lib):
    """The 8B-class shape takes blocked weights: d, d_ffn multiples of 64,
    vocab of 8."""
    assert L.workspace_bytes(_dims(weight_layout="blocked"), 128) == L.workspace_bytes(_dims(), 128) > 0


@pytest.mark.parametrize("args,code", [
    ((0, 1 << 20, 8, 64, 1), -1),                 # NULL src
    ((1 << 20, 1 << 24, 8, 64, 0), -3),           # fp32
    ((1 << 20, 1 << 24, 12, 64, 1), -2),          # N % 8
    ((1 << 20, 1 << 24, 8, 96, 1), -2),           # K % 64
    ((1 << 20, (1 << 20) + 512, 8, 64, 1), -1),   # dst overlaps src (8 x 64 bf16 = 1 KiB)
    ((1 << 20, (1 << 24) + 8, 8, 64, 1), -4),     # dst not 16-byte aligned
    ((1 << 20, 1 << 24, 0, 64, 1), -1),
])
def test_pack_weights_validation(lib, args, code):
    src, dst, N, K, dt = args
    assert lib.dl_pack_weights(src, dst, N, K, dt, None) == code, lib.dl_last_error()


def test_row_map_size(lib):
    """A selection's row map: n_rows, row_pos and row_seq for B*S rows, and two
    arrays over the attention tile capacity (B*S / 64 rounded up, plus one per
    sequence); 0 for an empty shape."""
    assert lib.dl_row_map_ints(1, 512) == 1 + 2 * 512 + 2 * (8 + 1)
    assert lib.dl_row_map_ints(16, 1280) == 1 + 2 * 16 * 1280 + 2 * (320 + 16)
    assert lib.dl_row_map_ints(3, 65) == 1 + 2 * 195 + 2 * (4 + 3)
    assert lib.dl_row_map_ints(0, 512) == 0 and lib.dl_row_map_ints(2, 0) == 0
    assert ctypes.sizeof(L.Selection) == 4 * ctypes.sizeof(ctypes.c_void_p)


def test_misaligned_row_map_rejected(lib):
    d = _dims()
    s = L.Selection(16, 16, 16, 18)
    r = lib.dl_score_select(ctypes.byref(d), 16, 32, 16, 16, 0, 0.5, 0, 0.25, 0.0, ctypes.byref(s), None, 16, 1 << 30,
                            None)
    assert r == -4 and b"row_map" in lib.dl_last_error()


def test_buffer_range_limits():
    """bf16: one weight matrix and one sequence's keys (plus 512 rows of
    prefetch slack) must stay below 2 GiB, the span of one buffer read; the
    largest accepted shapes sit one row below the limit."""
    assert L.workspace_bytes(_dims(vocab=262143), 64) > 0         # 262143 * 4096 * 2 < 2^31
    assert L.workspace_bytes(_dims(vocab=262144), 64) == 0        # = 2^31
    assert L.workspace_bytes(_dims(S=261631), 64) > 0             # (S + 512) * 4096 * 2 < 2^31
    assert L.workspace_bytes(_dims(S=261632), 64) == 0
    assert L.workspace_bytes(_dims(vocab=262144, dtype="f32"), 64) > 0   # fp32 products index with 64 bits


def test_null_and_alignment(lib):
    d = _dims()
    s = L.Selection(16, 16, 16)
    assert lib.dl_score_select(ctypes.byref(d), None, 32, 16, 16, 0, 0.5, 0, 0.25, 0.0, ctypes.byref(s), None, 16,
                               1 << 30, None) == -1
    assert b"h_cur" in lib.dl_last_error()
    assert lib.dl_score_select(ctypes.byref(d), 18, 32, 16, 16, 0, 0.5, 0, 0.25, 0.0, ctypes.byref(s), None, 16,
                               1 << 30, None) == -4
    assert lib.dl_score_select(ctypes.byref(d), 32, 32, 16, 16, 0, 0.5, 0, 0.25, 0.0, ctypes.byref(s), None, 16,
                               1 << 30, None) == -1                    # aliasing
    assert lib.dl_score_select(ctypes.byref(d), 16, 32, 16, 16, 0, 0.5, 0, 1.5, 0.0, ctypes.byref(s), None, 16,
                               1 << 30, None) == -1                    # keep > 1
    assert lib.dl_score_select(ctypes.byref(d), 16, 32, 16, 16, 9, 0.5, 0, 0.5, 0.0, ctypes.byref(s), None, 16,
                               1 << 30, None) == -1                    # score kind
    assert lib.dl_score_select(ctypes.byref(d), 16, 32, 16, 16, 0, 0.5, 0, 0.5, 0.0, ctypes.byref(s), None, 16,
                               8, None) == -5                          # workspace


def test_step_validation(lib):
    d = _dims(n_layers=2)
    lw = (L.LayerW * 2)(*[L.LayerW(*([16] * 9)) for _ in range(2)])
    m = L.Model(d, 16, 16, 16, lw)
    st = L.State(16, 16, 16, 16, 16, 16, 16, 16, 16, 16, None, None, L.Selection(16, 16, 16))
    lens = (ctypes.c_int32 * 1)(512)
    p = L.StepParams(0, 32, 1, 3, 0, 0, 0.5, 0, 0.25, 0.0, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    assert lib.dl_denoise_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(p), 16, 1 << 40, None) == -1
    assert b"skip_layer" in lib.dl_last_error()
    p.skip_layer = 1
    lens[0] = 600
    assert lib.dl_denoise_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(p), 16, 1 << 40, None) == -2
    lens[0] = 512
    assert lib.dl_denoise_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(p), 16, 64, None) == -5
    p.block_len = 4096
    assert lib.dl_denoise_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(p), 16, 1 << 40, None) == -7


def test_step_validation_two_levels_and_response_only(lib):
    d = _dims(n_layers=4)
    lw = (L.LayerW * 4)(*[L.LayerW(*([16] * 9)) for _ in range(4)])
    m = L.Model(d, 16, 16, 16, lw)
    lens = (ctypes.c_int32 * 1)(512)
    plen = (ctypes.c_int32 * 1)(256)

    def state(h_prev2=48, sel2=(64, 64, 64)):
        return L.State(16, 16, 16, 16, 16, 16, 16, 16, 16, 16, None, None, L.Selection(16, 16, 16), h_prev2, None,
                       L.Selection(*sel2))

    def params(**kw):
        p = L.StepParams(0, 32, 1, 1, 0, 0, 0.5, 0, 0.5, 0.0, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)),
                         0, ctypes.cast(plen, ctypes.POINTER(ctypes.c_int32)), 2, 0, 0.25, 0.0)
        for k, v in kw.items():
            setattr(p, k, v)
        return p

    def run(st, p, ws_bytes=1 << 40):
        return lib.dl_denoise_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(p), 16, ws_bytes, None)

    assert run(state(), params(), 64) == -5                      # valid up to the workspace size
    assert run(state(), params(skip_layer2=1)) == -1             # s2 must exceed s
    assert b"skip_layer2" in lib.dl_last_error()
    assert run(state(), params(skip_layer2=5)) == -1             # beyond n_layers
    assert run(state(), params(keep_ratio2=0.75)) == -1          # keeps more than the first level
    assert run(state(), params(keep_ratio2=0.0)) == -1
    assert run(state(), params(mode2=7)) == -1
    assert run(state(h_prev2=None), params()) == -1              # h_prev2 needed with two levels
    assert run(state(h_prev2=16), params()) == -1                # aliases h_prev
    assert run(state(sel2=(16, 64, 64)), params()) == -1         # sel2 aliases sel
    assert b"alias" in lib.dl_last_error()
    assert run(state(h_prev2=None), params(skip_layer2=0), 64) == -5   # one level: h_prev2 unused
    p = params(skip_layer2=0, response_only=1, prompt_len_host=None)
    assert run(state(), p) == -1                                 # response-only needs host prompt lengths
    plen[0] = 600
    assert run(state(), params(skip_layer2=0, response_only=1)) == -2
    plen[0] = 256
    assert run(state(), params(skip_layer2=0, response_only=1), 64) == -5
    assert run(state(), params(score_tensor=3)) == -1             # unknown scored tensor
    assert run(state(), params(skip_layer2=0, score_tensor=1), 64) == -5
    p = params(skip_layer2=0, score_tensor=2)
    p.skip_layer = 4                                              # no layer s to take keys / values from
    assert run(state(), p) == -1 and b"key/value" in lib.dl_last_error()
