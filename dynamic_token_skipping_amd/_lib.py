"""ctypes binding of libdtsk (include/dl.h): argument marshalling only.

Every function here has the name of the C entry point it wraps, takes torch
tensors (device memory) or plain numbers, passes their addresses and the
current HIP stream, and raises DLError on a non-zero status.  No arithmetic of
the method happens on this side.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_size_t, c_void_p
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdtsk.so")

DL_F32, DL_BF16 = 0, 1
DL_SCORE_ESDLLM, DL_SCORE_RELL2_INVCONF, DL_SCORE_COSINE = 0, 1, 2
DL_SEL_TOPK, DL_SEL_THRESHOLD = 0, 1
DL_TENSOR_HIDDEN, DL_TENSOR_KEY, DL_TENSOR_VALUE = 0, 1, 2
SCORE_TENSORS = {"hidden": DL_TENSOR_HIDDEN, "key": DL_TENSOR_KEY, "value": DL_TENSOR_VALUE}
SCORE_KINDS = {"esdllm": DL_SCORE_ESDLLM, "rell2_invconf": DL_SCORE_RELL2_INVCONF, "cosine": DL_SCORE_COSINE}
DTYPES = {"f32": DL_F32, "bf16": DL_BF16}
TORCH_DTYPES = {DL_F32: torch.float32, DL_BF16: torch.bfloat16}

EXPORTS = ("dl_score_select", "dl_gather", "dl_scatter_cache", "dl_partial_attn", "dl_ffn_rows", "dl_lm_head_rows",
           "dl_unmask", "dl_denoise_step", "dl_denoise_step_noalloc", "dl_workspace_bytes", "dl_status_string",
           "dl_last_error",
           "dl_abi_version", "dl_row_map_ints", "dl_pack_weights", "dl_timing_enable", "dl_timing_reset",
           "dl_timing_read")
DL_KC_GEMM, DL_KC_ATTN, DL_KC_LMHEAD, DL_KC_GEMM_TILED, DL_KC_APPROX = 0, 1, 2, 3, 4


class Dims(Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("d", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
                ("d_ffn", c_int32), ("vocab", c_int32), ("n_layers", c_int32), ("dtype", c_int32),
                ("rms_eps", c_float), ("rope_base", c_float), ("weight_layout", c_int32)]


class Selection(Structure):
    _fields_ = [("sel_idx", c_void_p), ("sel_count", c_void_p), ("row_off", c_void_p), ("row_map", c_void_p)]


class LayerW(Structure):
    _fields_ = [(k, c_void_p) for k in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up",
                                        "w_down")]


class Model(Structure):
    _fields_ = [("dims", Dims), ("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("layers", POINTER(LayerW))]


class State(Structure):
    _fields_ = [("tokens", c_void_p), ("masked", c_void_p), ("seq_len", c_void_p), ("prompt_len", c_void_p),
                ("h_prev", c_void_p), ("k_cache", c_void_p), ("v_cache", c_void_p), ("h_final", c_void_p),
                ("conf", c_void_p), ("argmax", c_void_p), ("logits", c_void_p), ("scores", c_void_p),
                ("sel", Selection), ("h_prev2", c_void_p), ("scores2", c_void_p), ("sel2", Selection),
                ("q_cache", c_void_p), ("ctx_cache", c_void_p), ("lse_cache", c_void_p), ("y_cache", c_void_p),
                ("layer_scores", c_void_p), ("sel_l", Selection)]


class StepParams(Structure):
    _fields_ = [("block", c_int32), ("block_len", c_int32), ("n_unmask", c_int32), ("skip_layer", c_int32),
                ("full_refresh", c_int32), ("score", c_int32), ("alpha", c_float), ("mode", c_int32),
                ("keep_ratio", c_float), ("threshold", c_float), ("seq_len_host", POINTER(c_int32)),
                ("response_only", c_int32), ("prompt_len_host", POINTER(c_int32)), ("skip_layer2", c_int32),
                ("mode2", c_int32), ("keep_ratio2", c_float), ("threshold2", c_float), ("score_tensor", c_int32),
                ("per_layer", c_int32), ("mode_l", c_int32), ("keep_ratio_l", c_float), ("threshold_l", c_float)]


class Timing(Structure):
    _fields_ = [("launches", ctypes.c_int64), ("dropped", ctypes.c_int64), ("ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


class DLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libdtsk status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libdtsk.so from the package directory (built by build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dynamic_token_skipping_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    st = c_int32
    lib.dl_score_select.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_int32,
                                    c_float, c_float, POINTER(Selection), c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dl_gather.argtypes = [POINTER(Dims), c_void_p, c_int32, c_int32, POINTER(Selection), c_int32, c_void_p,
                              c_void_p]
    lib.dl_scatter_cache.argtypes = [POINTER(Dims), c_void_p, c_int32, c_int32, POINTER(Selection), c_int32,
                                     c_void_p, c_void_p]
    lib.dl_partial_attn.argtypes = [POINTER(Dims), POINTER(LayerW), c_void_p, POINTER(Selection), c_void_p, c_int32,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dl_ffn_rows.argtypes = [POINTER(Dims), POINTER(LayerW), c_void_p, POINTER(Selection), c_int32, c_void_p,
                                c_size_t, c_void_p]
    lib.dl_lm_head_rows.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, POINTER(Selection), c_int32,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dl_unmask.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                              c_int32, c_int32, c_void_p]
    lib.dl_denoise_step.argtypes = [POINTER(Model), POINTER(State), POINTER(StepParams), c_void_p, c_size_t,
                                    c_void_p]
    lib.dl_denoise_step_noalloc.argtypes = [POINTER(Model), POINTER(State), POINTER(StepParams), c_void_p]
    lib.dl_workspace_bytes.argtypes = [POINTER(Dims), c_int32]
    lib.dl_workspace_bytes.restype = c_size_t
    lib.dl_status_string.argtypes = [c_int32]
    lib.dl_status_string.restype = c_char_p
    lib.dl_last_error.argtypes = []
    lib.dl_last_error.restype = c_char_p
    lib.dl_abi_version.argtypes = []
    lib.dl_abi_version.restype = c_int32
    lib.dl_row_map_ints.argtypes = [c_int32, c_int32]
    lib.dl_row_map_ints.restype = ctypes.c_int64
    lib.dl_pack_weights.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p]
    lib.dl_timing_enable.argtypes = [c_int32, c_int32]
    lib.dl_timing_reset.argtypes = []
    lib.dl_timing_read.argtypes = [c_int32, POINTER(Timing)]
    for name in ("dl_score_select", "dl_gather", "dl_scatter_cache", "dl_partial_attn", "dl_ffn_rows",
                 "dl_lm_head_rows", "dl_unmask", "dl_denoise_step", "dl_denoise_step_noalloc", "dl_pack_weights",
                 "dl_timing_enable",
                 "dl_timing_reset",
                 "dl_timing_read"):
        getattr(lib, name).restype = st
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load()
        raise DLError(status, f"{lib.dl_status_string(status).decode()}: {lib.dl_last_error().decode()}")


def ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def stream_handle(stream=None) -> Optional[int]:
    if not torch.cuda.is_available():
        return None
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


WEIGHT_LAYOUTS = {"row_major": 0, "blocked": 1}


def make_dims(B, S, d, n_heads, head_dim, d_ffn, vocab, n_layers, dtype, rms_eps=1e-5, rope_base=10000.0,
              weight_layout="row_major") -> Dims:
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    wl = WEIGHT_LAYOUTS[weight_layout] if isinstance(weight_layout, str) else int(weight_layout)
    return Dims(B, S, d, n_heads, head_dim, d_ffn, vocab, n_layers, dt, rms_eps, rope_base, wl)


class SelectionTensors:
    """Device arrays of a selection: sel_idx [B,S], sel_count [B], row_off [B+1]
    (int32) and, with ``row_map=True``, the row map that dl_score_select fills
    for the row entry points (leave it off for selections a decode step writes)."""

    def __init__(self, B: int, S: int, device="cuda", row_map: bool = False):
        self.sel_idx = torch.zeros((B, S), dtype=torch.int32, device=device)
        self.sel_count = torch.zeros((B,), dtype=torch.int32, device=device)
        self.row_off = torch.zeros((B + 1,), dtype=torch.int32, device=device)
        self.row_map = (torch.zeros((int(load().dl_row_map_ints(B, S)),), dtype=torch.int32, device=device)
                        if row_map else None)

    def struct(self) -> Selection:
        return Selection(ptr(self.sel_idx), ptr(self.sel_count), ptr(self.row_off),
                         ptr(self.row_map) if self.row_map is not None else None)

    def rows(self):
        """Host list of selected positions per sequence (synchronises)."""
        cnt = self.sel_count.cpu().tolist()
        idx = self.sel_idx.cpu()
        return [idx[b, :c].tolist() for b, c in enumerate(cnt)]


def layer_struct(lw: dict) -> LayerW:
    return LayerW(*[ptr(lw[k]) for k in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up",
                                         "w_down")])


def workspace_bytes(dims: Dims, max_rows: int = 0) -> int:
    return int(load().dl_workspace_bytes(ctypes.byref(dims), int(max_rows)))


def workspace(dims: Dims, max_rows: int = 0, device="cuda") -> torch.Tensor:
    n = workspace_bytes(dims, max_rows)
    if n == 0:
        _check(-1)
    return torch.empty((n,), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def dl_score_select(dims: Dims, h_cur, h_prev, conf, seq_len, kind, alpha, mode, keep_ratio, threshold,
                    sel: SelectionTensors, scores=None, ws=None, stream=None):
    k = SCORE_KINDS[kind] if isinstance(kind, str) else int(kind)
    s = sel.struct()
    _check(load().dl_score_select(ctypes.byref(dims), ptr(h_cur), ptr(h_prev), ptr(conf), ptr(seq_len), k,
                                  float(alpha), int(mode), float(keep_ratio), float(threshold), ctypes.byref(s),
                                  ptr(scores), ptr(ws), 0 if ws is None else ws.numel(), stream_handle(stream)))


def dl_gather(dims: Dims, src, w: int, dtype: int, sel: SelectionTensors, k_total_max: int, dst, stream=None):
    s = sel.struct()
    _check(load().dl_gather(ctypes.byref(dims), ptr(src), int(w), int(dtype), ctypes.byref(s), int(k_total_max),
                            ptr(dst), stream_handle(stream)))


def dl_scatter_cache(dims: Dims, rows, w: int, dtype: int, sel: SelectionTensors, k_total_max: int, cache,
                     stream=None):
    s = sel.struct()
    _check(load().dl_scatter_cache(ctypes.byref(dims), ptr(rows), int(w), int(dtype), ctypes.byref(s),
                                   int(k_total_max), ptr(cache), stream_handle(stream)))


def dl_partial_attn(dims: Dims, layer: dict, x_rows, sel: SelectionTensors, seq_len, k_total_max: int, k_cache,
                    v_cache, ws, stream=None, lse=None):
    """``lse``: optional fp32 [k_total_max, n_heads] tensor for the rows' log
    softmax normalisers."""
    lw = layer_struct(layer)
    s = sel.struct()
    _check(load().dl_partial_attn(ctypes.byref(dims), ctypes.byref(lw), ptr(x_rows), ctypes.byref(s), ptr(seq_len),
                                  int(k_total_max), ptr(k_cache), ptr(v_cache), ptr(lse), ptr(ws), ws.numel(),
                                  stream_handle(stream)))


def dl_ffn_rows(dims: Dims, layer: dict, x_rows, sel: SelectionTensors, k_total_max: int, ws, stream=None):
    lw = layer_struct(layer)
    s = sel.struct()
    _check(load().dl_ffn_rows(ctypes.byref(dims), ctypes.byref(lw), ptr(x_rows), ctypes.byref(s), int(k_total_max),
                              ptr(ws), ws.numel(), stream_handle(stream)))


def dl_lm_head_rows(dims: Dims, final_norm, lm_head, x_rows, sel: SelectionTensors, k_total_max: int, conf, argmax,
                    h_final, logits, ws, stream=None):
    s = sel.struct()
    _check(load().dl_lm_head_rows(ctypes.byref(dims), ptr(final_norm), ptr(lm_head), ptr(x_rows), ctypes.byref(s),
                                  int(k_total_max), ptr(conf), ptr(argmax), ptr(h_final), ptr(logits), ptr(ws),
                                  ws.numel(), stream_handle(stream)))


def dl_unmask(dims: Dims, tokens, masked, conf, argmax, prompt_len, seq_len, block: int, block_len: int,
              n_unmask: int, stream=None):
    _check(load().dl_unmask(ctypes.byref(dims), ptr(tokens), ptr(masked), ptr(conf), ptr(argmax), ptr(prompt_len),
                            ptr(seq_len), int(block), int(block_len), int(n_unmask), stream_handle(stream)))


def dl_denoise_step(model: Model, state: State, params: StepParams, ws, stream=None):
    _check(load().dl_denoise_step(ctypes.byref(model), ctypes.byref(state), ctypes.byref(params), ptr(ws),
                                  ws.numel(), stream_handle(stream)))


def dl_denoise_step_noalloc(model: Model, state: State, params: StepParams, stream=None):
    """dl_denoise_step with the library's built-in scratch as its workspace
    (nothing is allocated; see include/dl.h for the size limit)."""
    _check(load().dl_denoise_step_noalloc(ctypes.byref(model), ctypes.byref(state), ctypes.byref(params),
                                          stream_handle(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def dl_pack_weights(src, dst, stream=None):
    """dst (same shape, device) <- the blocked copy of the row-major [N, K]
    bf16 matrix src."""
    N, K = src.shape
    dt = {torch.bfloat16: DL_BF16, torch.float32: DL_F32}.get(src.dtype, -1)
    _check(load().dl_pack_weights(ptr(src), ptr(dst), int(N), int(K), dt, stream_handle(stream)))


def dl_abi_version() -> int:
    return int(load().dl_abi_version())


def dl_row_map_ints(B: int, S: int) -> int:
    return int(load().dl_row_map_ints(int(B), int(S)))


def dl_timing_enable(kc: int, stride: int = 1):
    """Time about one launch in `stride` of class kc (1: every launch, 0 or False: off)."""
    _check(load().dl_timing_enable(int(kc), int(stride)))


def dl_timing_reset():
    _check(load().dl_timing_reset())


def dl_timing_read(kc: int) -> dict:
    t = Timing()
    _check(load().dl_timing_read(int(kc), ctypes.byref(t)))
    return {"launches": t.launches, "dropped": t.dropped, "ms": t.ms, "bytes": t.bytes, "flops": t.flops}
