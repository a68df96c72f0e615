/*
 * dl.h -- C ABI of the early-skip partial-recompute step of masked-diffusion
 * LLM decoding, for AMD Instinct MI355X (gfx950).
 *
 * The method (ES-dLLM: Efficient Inference for Diffusion Large Language Models
 * by Early-Skipping, technical summary sections 1-2; DyLLM: Efficient Diffusion
 * LLM Inference via Saliency-based Token Selection and Partial Attention,
 * technical summary section 2):
 *   at each denoising step the first s layers run on every token; at layer s
 *   each token gets an importance score from the change of its hidden state
 *   since the previous step and its previous confidence; only the top-k tokens
 *   (k = (1 - r)|S|) go through layers s..L-1, whose key/value caches are
 *   updated in place for those rows (scatter) and reused for the others; the
 *   most confident masked tokens of the current block are then unmasked.  A
 *   full pass over every token (refresh) runs at set intervals.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; scratch memory comes from the
 *     caller's workspace (size from dl_workspace_bytes).
 *   - Layouts are row-major and contiguous.  Weight matrices are [out, in].
 *     Per-sequence tensors are padded to [B, S, ...]; row i of sequence b is at
 *     flat row b*S + i.  Every pointer must be 16-byte aligned.
 *   - Storage type (dims.dtype) applies to weights, embeddings, gains, the
 *     K/V/hidden caches and the inter-kernel activations; accumulation is fp32.
 *     The residual stream of rows in flight (x_rows) is always fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls validate on
 *     the host, enqueue, and return; device faults surface at the caller's next
 *     synchronisation.
 *   - On a failed validation a call returns a negative dl_status, enqueues
 *     nothing and writes nothing.  A launch failure returns DL_E_HIP.
 *     dl_last_error() returns a thread-local text for the last failure.
 *   - Packed rows: a selection lists, per sequence b, sel_count[b] ascending
 *     positions in sel_idx[b*S ...]; packed row r of sequence b is
 *     row_off[b] + j for its j-th selected position.  Row buffers such as
 *     x_rows are [k_total_max, width]; only the first row_off[B] rows are
 *     written (row_off lives on the device, so threshold selections need no
 *     host synchronisation), and kernels may read any of the k_total_max rows
 *     before the row count arrives.
 */
#ifndef DL_H
#define DL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DL_ABI_VERSION 5

typedef enum {
  DL_OK = 0,
  DL_E_ARG = -1,        /* null pointer, bad enum, non-positive size */
  DL_E_SHAPE = -2,      /* inconsistent dimensions (d != H*dh, k > S, ...) */
  DL_E_DTYPE = -3,      /* unsupported storage type for this entry point */
  DL_E_ALIGN = -4,      /* pointer not 16-byte aligned */
  DL_E_WORKSPACE = -5,  /* workspace too small (see dl_workspace_bytes) */
  DL_E_HIP = -6,        /* HIP runtime error (text in dl_last_error) */
  DL_E_UNSUPPORTED = -7 /* valid request outside what this build implements */
} dl_status;

typedef enum { DL_F32 = 0, DL_BF16 = 1 } dl_dtype;

/* Importance score of a row, from its current skip-layer input x, its cached
 * previous-step input h and its cached confidence c (max softmax probability):
 *   DL_SCORE_ESDLLM        alpha*c + (1-alpha)*||x-h||_1 / (sqrt(d)*||h||_2)
 *                          (ES-dLLM, section 2A, eq. I; alpha = 0.5 there)
 *   DL_SCORE_RELL2_INVCONF ||x-h||_2 / ||h||_2 + (1 - c)
 *   DL_SCORE_COSINE        1 - x.h / (||x||_2 ||h||_2)
 *                          (DyLLM, section 2A: low similarity = salient)
 * Denominators are floored at FLT_MIN.  Larger score = more important. */
typedef enum { DL_SCORE_ESDLLM = 0, DL_SCORE_RELL2_INVCONF = 1, DL_SCORE_COSINE = 2 } dl_score_kind;

/* DL_SEL_TOPK: per sequence the k = ceil(keep * len) rows (clamped to
 * [1, len], keep read as float32) with the largest scores, lower index first
 * among equal scores, NaN ranked last (ES-dLLM section 2B: k = (1 - r_l)|S|).
 * DL_SEL_THRESHOLD: every row with score > threshold (DyLLM section 2A). */
typedef enum { DL_SEL_TOPK = 0, DL_SEL_THRESHOLD = 1 } dl_select_mode;

/* The tensor whose change between steps the score measures (ES-dLLM section
 * 2A: hidden states, keys or values may serve): the input of the skip layer
 * s, or layer s's key rows RoPE(n(x) Wk^T) (rotated, as cached) or value rows
 * n(x) Wv^T, n = RMSNorm with layer s's attn_norm.  state.h_prev holds the
 * previous value of that tensor. */
typedef enum { DL_TENSOR_HIDDEN = 0, DL_TENSOR_KEY = 1, DL_TENSOR_VALUE = 2 } dl_score_tensor;

/* Storage order of the product weights (wq, wk, wv, wo, w_gate, w_up,
 * w_down and lm_head; the embedding table and the norm gains are always
 * plain).  Each is logically an [N, K] matrix (N output rows of K inputs):
 *   DL_WEIGHTS_ROW_MAJOR  element (n, k) at n*K + k.
 *   DL_WEIGHTS_BLOCKED    blocks of 8 rows x 64 inputs, each block contiguous
 *                         (row-major inside, 1 KiB in bf16), the blocks of an
 *                         8-row group in input order, the groups in row order:
 *                         element (n, k) at ((n/8)*(K/64) + k/64)*512 +
 *                         (n%8)*64 + k%64.  bf16 only; needs N % 8 == 0 and
 *                         K % 64 == 0 (d and d_ffn multiples of 64, vocab of 8).
 * Both give bit-identical results; the blocked order lets a product's
 * per-step weight reads be 1 KiB runs instead of 128-byte pieces of rows
 * K*2 bytes apart.  dl_pack_weights writes it. */
typedef enum { DL_WEIGHTS_ROW_MAJOR = 0, DL_WEIGHTS_BLOCKED = 1 } dl_weight_layout;

typedef struct {
  int32_t B;          /* sequences in the batch */
  int32_t S;          /* padded row capacity per sequence */
  int32_t d;          /* hidden size = n_heads * head_dim */
  int32_t n_heads;
  int32_t head_dim;   /* even */
  int32_t d_ffn;      /* SwiGLU inner size */
  int32_t vocab;
  int32_t n_layers;
  dl_dtype dtype;
  float rms_eps;      /* RMSNorm epsilon */
  float rope_base;    /* RoPE base (rotate-half pairs (j, j + head_dim/2)) */
  int32_t weight_layout; /* dl_weight_layout of the product weights */
} dl_dims;

typedef struct {
  int32_t *sel_idx;   /* [B, S] device: ascending positions, first sel_count[b] valid */
  int32_t *sel_count; /* [B] device */
  int32_t *row_off;   /* [B + 1] device: exclusive prefix sum of sel_count */
  int32_t *row_map;   /* optional device array of dl_row_map_ints(B, S) int32: the packed
                         rows' map (each row's flat position and sequence, the attention
                         query tiles).  dl_score_select writes it with row_off in the same
                         launch; dl_partial_attn, dl_ffn_rows and dl_lm_head_rows then read
                         it instead of building one in their workspace.  It describes the
                         selection as dl_score_select last wrote it: a selection written by
                         other means (dl_denoise_step neither reads nor writes row_map)
                         leaves it stale, so pass NULL there.  NULL: each call builds its
                         own. */
} dl_selection;

/* One layer's weights (device, storage dtype).  Norm gains are [d]; wq, wk,
 * wv, wo are [d, d]; w_gate, w_up are [d_ffn, d]; w_down is [d, d_ffn]. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo;
  const void *ffn_norm, *w_gate, *w_up, *w_down;
} dl_layer_w;

typedef struct {
  dl_dims dims;
  const void *embed;          /* [vocab, d] device */
  const void *final_norm;     /* [d] device */
  const void *lm_head;        /* [vocab, d] device (untied) */
  const dl_layer_w *layers;   /* HOST array of n_layers entries */
} dl_model;

/* Decoding state, all device memory owned by the caller. */
typedef struct {
  int32_t *tokens;            /* [B, S] current ids ([MASK] id where masked) */
  uint8_t *masked;            /* [B, S] 1 = still masked */
  const int32_t *seq_len;     /* [B] valid rows (prompt + generation) */
  const int32_t *prompt_len;  /* [B] */
  void *h_prev;               /* [B, S, d] previous value of the scored tensor (the skip-layer
                                 input unless params.score_tensor says otherwise) */
  void *k_cache, *v_cache;    /* [L, B, S, d] rotated keys / values per layer
                                 (layers < skip layer are per-step scratch) */
  void *h_final;              /* [B, S, d] last-layer output (before final norm) */
  float *conf;                /* [B, S] max softmax probability */
  int32_t *argmax;            /* [B, S] most likely id (lowest id on ties) */
  float *logits;              /* [B, S, vocab] fp32, or NULL to skip writing them */
  float *scores;              /* [B, S] this step's scores, or NULL (-inf for rows that were
                                 not candidates: prompt rows of a response-only step) */
  dl_selection sel;           /* this step's recomputed rows (written by the step) */
  /* second skip level (used when params.skip_layer2 > 0; may be NULL otherwise) */
  void *h_prev2;              /* [B, S, d] input of layer skip_layer2 as last computed */
  float *scores2;             /* [B, S] second-level scores (-inf outside sel), or NULL */
  dl_selection sel2;          /* rows recomputed in layers [skip_layer2, L) and the LM head */
  /* per-layer re-selection (used when params.per_layer != 0; may be NULL
   * otherwise).  Layers below skip_layer are not used. */
  void *q_cache;              /* [L, B, S, d] rotated queries of each layer */
  float *ctx_cache;           /* [L, B, S, d] fp32 attention contexts (before Wo) */
  float *lse_cache;           /* [L, B, S, n_heads] fp32 log softmax normalisers of those contexts */
  float *y_cache;             /* [L, B, S, d] fp32 layer outputs */
  float *layer_scores;        /* [B, S] the last layer's saliency 1 - cos, or NULL */
  dl_selection sel_l;         /* rows through the last layer and the LM head */
} dl_state;

typedef struct {
  int32_t block;              /* current block: unmask window starts at prompt_len + block*block_len */
  int32_t block_len;
  int32_t n_unmask;           /* tokens unmasked per sequence this step */
  int32_t skip_layer;         /* s: layers [0, s) on every row; 1 <= s <= n_layers */
  int32_t full_refresh;       /* nonzero: every row through every layer */
  dl_score_kind score;
  float alpha;
  dl_select_mode mode;
  float keep_ratio;           /* in (0, 1] for DL_SEL_TOPK */
  float threshold;            /* for DL_SEL_THRESHOLD */
  const int32_t *seq_len_host;/* [B] HOST copy of state.seq_len, used for grid sizing only */
  /* DyLLM response-only step (technical summary section 2B, strategy 3): on a
   * skip step, only positions [prompt_len[b], seq_len[b]) go through layers
   * [0, s), are scored and can be kept, and keep_ratio applies to their count;
   * prompt rows keep every cache.  Ignored on a refresh step. */
  int32_t response_only;
  const int32_t *prompt_len_host; /* [B] HOST copy of state.prompt_len (response_only only) */
  /* Second skip level (ES-dLLM technical summary section 2B: skipping at two
   * early layers with a skip ratio per layer).  0: one level.  Otherwise
   * skip_layer < skip_layer2 <= n_layers: the rows in sel go through layers
   * [s, s2); at the input of s2 they are scored against state.h_prev2 (same
   * score kind and cached confidence) and h_prev2 is rewritten for them; the
   * DL_SEL_TOPK level keeps ceil(keep_ratio2 * count) of them, count being
   * what keep_ratio applies to, at most as many as sel holds (keep_ratio2 <=
   * keep_ratio when the first level is also DL_SEL_TOPK); only those go
   * through [s2, L) and the LM head.  A refresh step rewrites h_prev2 for
   * every row. */
  int32_t skip_layer2;
  dl_select_mode mode2;
  float keep_ratio2;
  float threshold2;
  /* Tensor scored at the first level (DL_TENSOR_KEY / DL_TENSOR_VALUE need
   * skip_layer < n_layers).  The second level always scores hidden states. */
  dl_score_tensor score_tensor;
  /* DyLLM per-layer re-selection (technical summary section 2B): from layer
   * skip_layer on, the active rows (sel at layer s, then the previous layer's
   * salient rows) get fresh q/K/V and exact attention; every other row's
   * context is updated approximately as C + S dV, S_ij = exp(q_i.k_j /
   * sqrt(dh) - lse_i) from its cached query and normaliser and the active
   * rows' previous keys, dV_j the change of their values; the rows with the
   * largest 1 - cos(C_new, C_cached) (top-k of keep_ratio_l of the valid
   * length, or above threshold_l) go through Wo and the FFN, the others keep
   * their cached output.  ctx_cache takes every row's new context; q_cache
   * and lse_cache change for the active rows.  A refresh step fills every
   * cache for every row.  Needs skip_layer < n_layers, one skip level and
   * full-context steps. */
  int32_t per_layer;
  dl_select_mode mode_l;
  float keep_ratio_l;
  float threshold_l;
} dl_step_params;

/* ---------------------------------------------------------------------------
 * Score and select (ES-dLLM section 2A eq. I and 2B top-k; DyLLM section 2A
 * threshold).  h_cur and h_prev are [B, S, d] in dims.dtype, conf is [B, S].
 * Writes `out` (device arrays sized as in dl_selection) and, if non-NULL,
 * scores[B, S] (fp32; padding rows untouched).  Reads only; h_prev is not
 * updated.  Needs dl_workspace_bytes(dims, 0) bytes of workspace.
 * ------------------------------------------------------------------------- */
dl_status dl_score_select(const dl_dims *dims, const void *h_cur, const void *h_prev, const float *conf,
                          const int32_t *seq_len, dl_score_kind kind, float alpha, dl_select_mode mode,
                          float keep_ratio, float threshold, dl_selection *out, float *scores_or_null,
                          void *ws, size_t ws_bytes, void *stream);

/* Gather selected rows (ES-dLLM section 2B: only the top-k tokens go on):
 * dst[row_off[b] + j, :] = src[b, sel_idx[b][j], :]; src is [B, S, w] and dst
 * [k_total_max, w], both of `dtype` (DL_F32 or DL_BF16). */
dl_status dl_gather(const dl_dims *dims, const void *src, int32_t w, dl_dtype dtype, const dl_selection *sel,
                    int32_t k_total_max, void *dst, void *stream);

/* Scatter packed rows back into a cache (ES-dLLM section 2B: in-place update
 * of the selected rows; other rows keep every byte):
 * cache[b, sel_idx[b][j], :] = rows[row_off[b] + j, :]. */
dl_status dl_scatter_cache(const dl_dims *dims, const void *rows, int32_t w, dl_dtype dtype,
                           const dl_selection *sel, int32_t k_total_max, void *cache, void *stream);

/* Attention sub-block of one layer on the selected rows (ES-dLLM section 2B,
 * DyLLM section 2B): x_rows (fp32 [k_total_max, d], in/out) +=
 *   Wo * Attn(RoPE(Wq n(x)), K, V), where the rows' fresh RoPE(Wk n(x)) and
 * Wv n(x) are first written into k_cache/v_cache ([B, S, d] of this layer) at
 * their positions, and each row attends over keys 0..seq_len[b]-1 of its own
 * sequence (bidirectional).  n = RMSNorm with layer->attn_norm.
 * lse_or_null (device fp32 [k_total_max, n_heads], or NULL): for each packed
 * row r < row_off[B] and head h, the log of that row's softmax normaliser,
 * log sum_j exp(q_rh . k_jh / sqrt(head_dim)) over the same keys (the cached
 * normaliser of DyLLM's approximate attention, DyLLM section 2B); rows from
 * row_off[B] on are not written.  Asking for it changes no other output. */
dl_status dl_partial_attn(const dl_dims *dims, const dl_layer_w *layer, float *x_rows, const dl_selection *sel,
                          const int32_t *seq_len, int32_t k_total_max, void *k_cache, void *v_cache,
                          float *lse_or_null, void *ws, size_t ws_bytes, void *stream);

/* SwiGLU FFN sub-block on packed rows: x += Wd (silu(Wg n(x)) * Wu n(x)),
 * n = RMSNorm with layer->ffn_norm.  x_rows is fp32 [k_total_max, d]; the
 * rows actually processed are the first sel->row_off[B]. */
dl_status dl_ffn_rows(const dl_dims *dims, const dl_layer_w *layer, float *x_rows, const dl_selection *sel,
                      int32_t k_total_max, void *ws, size_t ws_bytes, void *stream);

/* Final norm + LM head on packed rows, then confidence (max softmax
 * probability = 1 / sum exp(l - max)) and argmax (lowest id on ties), scattered
 * with h_final (= x_rows in storage dtype) and, if non-NULL, the fp32 logits
 * into the [B, S] caches at the selected positions (ES-dLLM section 2A: c is
 * the maximum probability; section 2B: caches of skipped rows are reused). */
dl_status dl_lm_head_rows(const dl_dims *dims, const void *final_norm, const void *lm_head, const float *x_rows,
                          const dl_selection *sel, int32_t k_total_max, float *conf, int32_t *argmax,
                          void *h_final, float *logits_or_null, void *ws, size_t ws_bytes, void *stream);

/* Unmask (ES-dLLM section 1: only the most confident masked tokens are
 * unmasked each step): per sequence, among masked positions in
 * [prompt_len + block*block_len, +block_len) (clipped to seq_len), the
 * n_unmask with the highest conf (lower index on ties) get tokens = argmax
 * and masked = 0. */
dl_status dl_unmask(const dl_dims *dims, int32_t *tokens, uint8_t *masked, const float *conf,
                    const int32_t *argmax, const int32_t *prompt_len, const int32_t *seq_len, int32_t block,
                    int32_t block_len, int32_t n_unmask, void *stream);

/* One whole denoising step: embed; layers [0, s) on every valid row (on the
 * response rows only on a response-only step); then
 *   refresh: layers [s, L) on every row, h_prev <- layer-s input of every row
 *            (and h_prev2 <- layer-s2 input of every row with two levels);
 *   skip:    score the candidate rows against h_prev, h_prev <- their layer-s
 *            input, select, layers [s, L) on the selected rows only (with two
 *            levels: [s, s2) on sel, second score and selection, [s2, L) on
 *            sel2);
 * LM head + scatter for the rows that went through every layer; unmask.
 * state->sel receives the selection (all rows on a refresh step), and
 * state->sel2 the second-level selection when there is one. */
dl_status dl_denoise_step(const dl_model *model, dl_state *state, const dl_step_params *params, void *ws,
                          size_t ws_bytes, void *stream);

/* The same step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the workspace is a file-scope device array of DL_NOALLOC_SCRATCH_BYTES
 * inside the library, which each device the library runs on holds until the
 * process ends, instead of the caller's.  The call allocates nothing.
 * Arguments and results are those of dl_denoise_step; the current device must
 * be the device of `stream`.  A step whose workspace (dl_workspace_bytes of
 * its valid rows) exceeds the array is rejected with DL_E_WORKSPACE before
 * anything is enqueued (the 8B-class shapes need the workspace entry point).
 * Every call on one device shares that device's array: calls that overlap on
 * one device (other streams, other threads) race and must be serialised by
 * the caller. */
#define DL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dl_status dl_denoise_step_noalloc(const dl_model *model, dl_state *state, const dl_step_params *params,
                                  void *stream);

/* ---------------------------------------------------------------------------
 * Kernel timing (measurement support, not part of the method).  While a class
 * is enabled with sampling stride n >= 1, about one launch in n of that class
 * (chosen by a fixed hash of the launch's sequence number, so that launches of
 * every shape are sampled) is timed by two HIP events bound to its kernels'
 * own dispatch packets on the launch's stream (from the start of its first
 * kernel to the end of its last, as hipExtLaunchKernel records them, so no
 * marker packet sits between the kernels), and that launch's algorithmic
 * bytes and FLOPs are added up (for a product: weights + input rows + output rows in the storage
 * type, 2*M*N*K FLOPs; for attention: Q + K/V rows read + output,
 * 4*rows*keys*d FLOPs).  n = 1 times every launch; n = 0 disables the class.
 * dl_timing_read synchronises on the recorded events and returns the sums
 * since dl_timing_reset.  Up to 65536 launches per class are timed; launches
 * not timed (not sampled, or the event pool is full) are counted in
 * `dropped`.  Not thread-safe.
 * ------------------------------------------------------------------------- */
typedef enum {
  DL_KC_GEMM = 0,        /* layer products on at most 128 rows (the kept rows of a skip step) */
  DL_KC_ATTN = 1,        /* attention */
  DL_KC_LMHEAD = 2,      /* LM head product with its confidence statistics */
  DL_KC_GEMM_TILED = 3,  /* layer products on more rows (prefix layers, refresh steps) */
  DL_KC_APPROX = 4,      /* approximate context update of the per-layer variant */
  DL_KC_COUNT = 5
} dl_kernel_class;

typedef struct {
  int64_t launches;     /* launches timed */
  int64_t dropped;      /* launches of the class not timed (not sampled, or pool full) */
  double ms;            /* summed kernel time */
  double bytes;         /* summed algorithmic bytes */
  double flops;         /* summed algorithmic FLOPs */
} dl_timing;

dl_status dl_timing_enable(dl_kernel_class kc, int32_t stride);
dl_status dl_timing_reset(void);
dl_status dl_timing_read(dl_kernel_class kc, dl_timing *out);

/* Workspace bytes for any entry point above on a batch whose valid rows sum
 * to at most max_rows (0: B*S). */
size_t dl_workspace_bytes(const dl_dims *dims, int32_t max_rows);

const char *dl_status_string(dl_status s);
const char *dl_last_error(void);
int32_t dl_abi_version(void);

/* Size, in int32 elements, of a selection's row map (dl_selection.row_map)
 * for B sequences of row capacity S; 0 when B or S is below 1. */
int64_t dl_row_map_ints(int32_t B, int32_t S);

/* The DL_WEIGHTS_BLOCKED copy of a row-major [N, K] weight: dst (device,
 * N*K elements, not overlapping src) receives src (device) in blocked order.
 * bf16 only (DL_E_DTYPE otherwise); N % 8 and K % 64 must be 0 (DL_E_SHAPE).
 * Enqueued on `stream`; src is only read. */
dl_status dl_pack_weights(const void *src, void *dst, int32_t N, int32_t K, dl_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DL_H */
