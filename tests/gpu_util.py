"""Helpers shared by the GPU parity tests: model conversion, the per-row
relative error, and the tie-band comparison of selections."""
from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import esdllm as E


def np_model(m: dict) -> dict:
    """Exact float64 host copy of a model dict of torch tensors."""
    out = {k: workloads.host_f64(v) for k, v in m.items() if k != "layers"}
    out["layers"] = [{k: workloads.host_f64(v) for k, v in lw.items()} for lw in m["layers"]]
    return out


def to_device(m: dict, device="cuda") -> dict:
    out = {k: v.to(device) for k, v in m.items() if k != "layers"}
    out["layers"] = [{k: v.to(device) for k, v in lw.items()} for lw in m["layers"]]
    return out


def row_rel_err(gpu, ref) -> float:
    """max over rows of ||g - o||_inf / max(||o||_inf, 1e-6)."""
    g = np.asarray(gpu, np.float64).reshape(len(gpu), -1) if np.ndim(gpu) > 1 else np.asarray(gpu, np.float64)[:, None]
    o = np.asarray(ref, np.float64).reshape(g.shape)
    if g.size == 0:
        return 0.0
    num = np.abs(g - o).max(axis=1)
    den = np.maximum(np.abs(o).max(axis=1), 1e-6)
    return float((num / den).max())


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def selection_diff_ok(gpu_sel, oracle_sel, oracle_scores, k, band_abs=1e-4, band_rel=0.0):
    """Selections agree except on rows whose oracle score is within the band of
    the k-th largest oracle score (decided in float32)."""
    a, b = set(map(int, gpu_sel)), set(map(int, oracle_sel))
    if a == b:
        return True, 0
    s32 = np.asarray(oracle_scores, np.float64).astype(np.float32).astype(np.float64)
    kth = np.sort(s32)[::-1][k - 1]
    band = band_abs + band_rel * abs(kth)
    bad = [i for i in a ^ b if abs(s32[i] - kth) > band]
    return len(bad) == 0, len(a ^ b)


def unmask_diff_ok(gpu_pos, oracle_pos, oracle_conf, band_rel=2e-2):
    """Unmasked sets agree except on positions whose oracle confidence is within
    band_rel of the smallest confidence the oracle unmasked."""
    a, b = set(map(int, gpu_pos)), set(map(int, oracle_pos))
    if a == b:
        return True, 0
    if not b:
        return False, len(a ^ b)
    c = np.asarray(oracle_conf, np.float64)
    edge = min(c[i] for i in b)
    bad = [i for i in a ^ b if abs(c[i] - edge) > band_rel * abs(edge)]
    return len(bad) == 0, len(a ^ b)


def sync_from_oracle(dec, b: int, st) -> None:
    """Overwrite sequence b of the GPU decode state with the oracle's state
    (rounded to the storage type): the next step then starts from the same
    inputs on both sides.  Data flows oracle -> GPU only."""
    n = len(st.tokens)
    dev = dec.tokens.device
    dt = dec.h_prev.dtype

    def put(dst, src, dtype=None):
        dst.copy_(torch.as_tensor(np.asarray(src), device=dev).to(dtype or dst.dtype))

    put(dec.tokens[b, :n], st.tokens.astype(np.int32))
    put(dec.masked[b, :n], st.masked.astype(np.uint8))
    put(dec.conf[b, :n], st.conf.astype(np.float32))
    put(dec.argmax[b, :n], st.argmax.astype(np.int32))
    put(dec.h_prev[b, :n], st.h_prev.astype(np.float32), dt)
    put(dec.h_final[b, :n], st.h_final.astype(np.float32), dt)
    for li in range(len(st.K)):
        put(dec.k_cache[li, b, :n], st.K[li].astype(np.float32), dt)
        put(dec.v_cache[li, b, :n], st.V[li].astype(np.float32), dt)
    if dec.logits is not None and st.logits is not None:
        put(dec.logits[b, :n], st.logits.astype(np.float32))
    if getattr(dec, "h_prev2", None) is not None and st.h_prev2 is not None:
        put(dec.h_prev2[b, :n], st.h_prev2.astype(np.float32), dt)
    if getattr(dec, "ctx_cache", None) is not None and st.C is not None:
        for li in range(len(st.C)):
            put(dec.q_cache[li, b, :n], st.Q[li].astype(np.float32), dt)
            put(dec.ctx_cache[li, b, :n], st.C[li].astype(np.float32))
            put(dec.lse_cache[li, b, :n], st.LSE[li].astype(np.float32))
            put(dec.y_cache[li, b, :n], st.Y[li].astype(np.float32))
