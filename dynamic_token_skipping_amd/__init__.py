"""Early-skip partial-recompute denoising step for masked-diffusion LLMs on
AMD Instinct MI355X: a HIP library (libdtsk, C ABI in include/dl.h) and its
thin Python binding."""
from ._lib import (DLError, DL_BF16, DL_F32, DL_SCORE_COSINE, DL_SCORE_ESDLLM, DL_SCORE_RELL2_INVCONF,  # noqa: F401
                   DL_SEL_THRESHOLD, DL_SEL_TOPK, EXPORTS, SelectionTensors, dl_abi_version, dl_denoise_step,
                   dl_denoise_step_noalloc, NOALLOC_SCRATCH_BYTES,
                   dl_ffn_rows, dl_gather, dl_lm_head_rows, dl_pack_weights, dl_partial_attn, dl_row_map_ints,
                   dl_scatter_cache,
                   dl_score_select,
                   dl_unmask, load, make_dims, workspace, workspace_bytes, dl_timing_enable, dl_timing_read,
                   dl_timing_reset, DL_KC_GEMM, DL_KC_ATTN, DL_KC_LMHEAD,
                   DL_KC_GEMM_TILED, DL_KC_APPROX)
from .decode import Decoder, DeviceModel, is_refresh_step, pack_model  # noqa: F401
