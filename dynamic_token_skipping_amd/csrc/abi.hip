// The C ABI of libdtsk: host-side validation, workspace layout and the
// orchestration of one denoising step from the kernels of k_rows / k_gemm /
// k_attn.  Nothing here allocates or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "launch.h"

using namespace dtsk;

namespace dtsk {
thread_local DispatchEvents* g_region_events = nullptr;
}

namespace {

thread_local char g_err[512] = "";

dl_status fail(dl_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

#define DL_CHECK_HIP(expr)                                                              \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(DL_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define DL_TRY(expr)               \
  do {                             \
    dl_status s_ = (expr);         \
    if (s_ != DL_OK) return s_;    \
  } while (0)

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t esize(dl_dtype t) { return t == DL_BF16 ? 2 : 4; }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

constexpr int kTileRows = 64;       // attention query tile
constexpr int kLmChunk = 512;       // LM-head rows per product (bounds the logits buffer)

dl_status check_ptr(const void* p, const char* what) {
  if (!p) return fail(DL_E_ARG, "%s is NULL", what);
  if (((uintptr_t)p) & 15) return fail(DL_E_ALIGN, "%s is not 16-byte aligned", what);
  return DL_OK;
}

dl_status check_dims(const dl_dims* d) {
  if (!d) return fail(DL_E_ARG, "dims is NULL");
  if (d->B < 1 || d->S < 1 || d->d < 1 || d->n_heads < 1 || d->head_dim < 2 || d->d_ffn < 1 || d->vocab < 1 ||
      d->n_layers < 1)
    return fail(DL_E_ARG, "dims: every size must be positive");
  if (d->dtype != DL_F32 && d->dtype != DL_BF16) return fail(DL_E_DTYPE, "dims.dtype %d unknown", (int)d->dtype);
  if (d->n_heads * d->head_dim != d->d)
    return fail(DL_E_SHAPE, "d (%d) != n_heads (%d) * head_dim (%d)", d->d, d->n_heads, d->head_dim);
  if (d->head_dim % 2) return fail(DL_E_SHAPE, "head_dim must be even");
  if (d->B > 1024) return fail(DL_E_UNSUPPORTED, "B > 1024");
  if (!(d->rms_eps > 0.f)) return fail(DL_E_ARG, "rms_eps must be positive");
  if (!(d->rope_base > 0.f)) return fail(DL_E_ARG, "rope_base must be positive");
  if (!attention_supported(d->dtype, d->S, d->head_dim))
    return fail(DL_E_UNSUPPORTED, "attention for S=%d head_dim=%d not built", d->S, d->head_dim);
  if ((size_t)d->d * esize(d->dtype) % 16 != 0) return fail(DL_E_SHAPE, "d * element size must be a multiple of 16 bytes");
  if (d->dtype == DL_BF16) {
    // The bf16 products read one weight matrix (vocab, d_ffn or d rows of d
    // columns, or d rows of d_ffn) through one buffer resource, and the
    // attention kernels one sequence's keys or values (S rows of d, plus the
    // tiles their prefetch runs past the end): 32-bit byte offsets.
    const long long wmax = (long long)std::max(std::max(d->vocab, d->d_ffn), d->d) * d->d * 2;
    const long long kv = ((long long)d->S + 512) * d->d * 2;
    if (wmax > kMaxBufBytes)
      return fail(DL_E_UNSUPPORTED, "a bf16 weight matrix of %lld bytes: one product reads at most 2 GiB - 1", wmax);
    if (kv > kMaxBufBytes)
      return fail(DL_E_UNSUPPORTED, "one sequence's keys (S=%d, d=%d) exceed what one attention read spans (2 GiB)",
                  d->S, d->d);
  }
  if (d->weight_layout != DL_WEIGHTS_ROW_MAJOR && d->weight_layout != DL_WEIGHTS_BLOCKED)
    return fail(DL_E_ARG, "dims.weight_layout %d unknown", (int)d->weight_layout);
  if (d->weight_layout == DL_WEIGHTS_BLOCKED) {
    if (d->dtype != DL_BF16) return fail(DL_E_DTYPE, "blocked weights are bf16 only");
    if (d->d % 64 || d->d_ffn % 64 || d->vocab % 8)
      return fail(DL_E_SHAPE, "blocked weights need d (%d) and d_ffn (%d) multiples of 64 and vocab (%d) of 8", d->d,
                  d->d_ffn, d->vocab);
  }
  return DL_OK;
}

dl_status check_sel(const dl_selection* s, const char* what) {
  if (!s) return fail(DL_E_ARG, "%s is NULL", what);
  DL_TRY(check_ptr(s->sel_idx, "sel_idx"));
  DL_TRY(check_ptr(s->sel_count, "sel_count"));
  DL_TRY(check_ptr(s->row_off, "row_off"));
  if (((uintptr_t)s->row_map) & 3) return fail(DL_E_ALIGN, "%s.row_map is not 4-byte aligned", what);
  return DL_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct RowMapMem {
  size_t row_pos, row_seq, n_rows, tile_row0, tile_rows;
};

struct Layout {
  int R;                    // row capacity (valid rows over the batch)
  int T;                    // attention tile capacity
  size_t sel_idx, sel_count, row_off;  // the step's candidate rows (every valid row, or the response rows)
  RowMapMem map_all, map_sel, map_sel2;
  size_t x_all, x_sel, x_sel2;  // fp32 [R, d]
  size_t t_rows;            // fp32 [R, d]: key / value rows of the skip layer when they are scored
  // per-layer re-selection
  size_t k_act, v_old, dv;  // T [R, d]: the active rows' previous keys / values, their value change
  size_t ctx_new;           // fp32 [R, d]: every row's new context, packed over all rows
  size_t lsel_idx[2], lsel_count[2], lsel_off[2];  // two selections used in turn
  RowMapMem map_l[2];
  size_t inv;               // int32 [B*S]: packed row of a flat position
  size_t scores2;           // fp32 [B*S]
  size_t act;               // T [R, d] normalised rows
  size_t ffn_act;           // T [R, F] silu(gate) * up
  size_t q, attn;           // T [R, d]
  size_t P;                 // fp32 GEMM partials
  size_t lm_part;           // float4 [min(R, kLmChunk)][ceil(V / 128)]
  int R_part;               // rows of the attention key-chunk partials (0: none)
  int attn_splits;          // key chunks the partials have room for
  size_t attn_o;            // fp32 [attn_splits][R_part][d]
  size_t attn_ml;           // float2 [attn_splits][R_part][n_heads]
  size_t scores;            // fp32 [B*S]
  size_t rope;              // float2 [S, head_dim/2]
  size_t total;
};

constexpr int kAttnPartRows = 1024;  // packed-row bound for split-key attention

size_t gemm_partial_floats(const dl_dims& d, int R, int N, int K, int epi) {
  // worst case over every row bound the planner can see (1..R)
  size_t best = 0;
  for (int m : {16, 32, 64}) {
    if (m >= R) break;
    const GemmPlan p = plan_gemm(d.dtype, m, N, K, epi, d.head_dim, d.d_ffn);
    best = std::max(best, (size_t)p.splits * (size_t)m * (size_t)N);
  }
  for (int m = 128;; m += 128) {
    const int M = std::min(m, R);
    const GemmPlan p = plan_gemm(d.dtype, M, N, K, epi, d.head_dim, d.d_ffn);
    best = std::max(best, (size_t)p.splits * (size_t)M * (size_t)N);
    if (M == R) break;
  }
  return best;
}

Layout make_layout(const dl_dims& d, int R) {
  Layout L{};
  const int B = d.B, S = d.S;
  L.R = std::max(R, 1);
  L.T = cdiv(L.R, kTileRows) + B;
  const size_t es = esize(d.dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.sel_idx = take(sizeof(int32_t) * (size_t)B * S);
  L.sel_count = take(sizeof(int32_t) * B);
  L.row_off = take(sizeof(int32_t) * (B + 1));
  for (RowMapMem* m : {&L.map_all, &L.map_sel, &L.map_sel2, &L.map_l[0], &L.map_l[1]}) {
    m->row_pos = take(sizeof(int32_t) * L.R);
    m->row_seq = take(sizeof(int32_t) * L.R);
    m->n_rows = take(sizeof(int32_t));
    m->tile_row0 = take(sizeof(int32_t) * L.T);
    m->tile_rows = take(sizeof(int32_t) * L.T);
  }
  L.x_all = take(sizeof(float) * (size_t)L.R * d.d);
  L.x_sel = take(sizeof(float) * (size_t)L.R * d.d);
  L.x_sel2 = take(sizeof(float) * (size_t)L.R * d.d);
  L.t_rows = take(sizeof(float) * (size_t)L.R * d.d);
  L.k_act = take(es * (size_t)L.R * d.d);
  L.v_old = take(es * (size_t)L.R * d.d);
  L.dv = take(es * (size_t)L.R * d.d);
  L.ctx_new = take(sizeof(float) * (size_t)L.R * d.d);
  for (int i = 0; i < 2; ++i) {
    L.lsel_idx[i] = take(sizeof(int32_t) * (size_t)B * S);
    L.lsel_count[i] = take(sizeof(int32_t) * B);
    L.lsel_off[i] = take(sizeof(int32_t) * (B + 1));
  }
  L.inv = take(sizeof(int32_t) * (size_t)B * S);
  L.scores2 = take(sizeof(float) * (size_t)B * S);
  L.act = take(es * (size_t)L.R * d.d);
  L.ffn_act = take(es * (size_t)L.R * d.d_ffn);
  L.q = take(es * (size_t)L.R * d.d);
  L.attn = take(es * (size_t)L.R * d.d);
  size_t pf = 0;
  pf = std::max(pf, gemm_partial_floats(d, L.R, 3 * d.d, d.d, EPI_QKV));
  pf = std::max(pf, gemm_partial_floats(d, L.R, d.d, d.d, EPI_NONE));
  pf = std::max(pf, gemm_partial_floats(d, L.R, 2 * d.d_ffn, d.d, EPI_SWIGLU));
  pf = std::max(pf, gemm_partial_floats(d, L.R, d.d, d.d_ffn, EPI_NONE));
  pf = std::max(pf, gemm_partial_floats(d, std::min(L.R, kLmChunk), d.vocab, d.d, EPI_LM));
  L.P = take(sizeof(float) * pf);
  L.lm_part = take(16 * (size_t)std::min(L.R, kLmChunk) * cdiv(d.vocab, 128));
  L.attn_splits = std::min(kAttnMaxSplits, std::max(1, S / 128));
  L.R_part = (d.dtype == DL_BF16 && d.head_dim == 128 && L.attn_splits > 1) ? std::min(L.R, kAttnPartRows) : 0;
  L.attn_o = take(sizeof(float) * (size_t)L.attn_splits * L.R_part * d.d);
  L.attn_ml = take(sizeof(float) * 2 * (size_t)L.attn_splits * L.R_part * d.n_heads);
  L.scores = take(sizeof(float) * (size_t)B * S);
  L.rope = take(sizeof(float) * 2 * (size_t)S * (d.head_dim / 2));
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// A selection's own row map (dl_selection.row_map): n_rows, then row_pos and
// row_seq for B*S rows, then tile_row0 and tile_rows for the tile capacity.
int64_t row_map_tiles(int B, int S) { return cdiv((long long)B * S, kTileRows) + B; }

RowMap rowmap_of_sel(const dl_selection* sel, int B, int S, int R_max) {
  const int64_t bs = (int64_t)B * S, tc = row_map_tiles(B, S);
  RowMap r;
  r.n_rows = sel->row_map;
  r.row_pos = sel->row_map + 1;
  r.row_seq = sel->row_map + 1 + bs;
  r.tile_row0 = sel->row_map + 1 + 2 * bs;
  r.tile_rows = sel->row_map + 1 + 2 * bs + tc;
  r.R_max = R_max;
  // tiles fill in order, so the first cdiv(R_max, kTileRows) + B hold every row of R_max
  r.T_max = (int)std::min<int64_t>(tc, cdiv(R_max, kTileRows) + B);
  r.tq = kTileRows;
  return r;
}

RowMap rowmap_at(void* ws, const RowMapMem& m, int R_max, int T_max) {
  RowMap r;
  r.row_pos = at<int32_t>(ws, m.row_pos);
  r.row_seq = at<int32_t>(ws, m.row_seq);
  r.n_rows = at<int32_t>(ws, m.n_rows);
  r.tile_row0 = at<int32_t>(ws, m.tile_row0);
  r.tile_rows = at<int32_t>(ws, m.tile_rows);
  r.R_max = R_max;
  r.T_max = T_max;
  r.tq = kTileRows;
  return r;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
constexpr int kTimingPool = 1 << 16;

struct TimingClass {
  bool enabled = false;
  uint32_t stride = 1;            // sample about one launch in `stride`
  uint32_t seq = 0;               // launches seen since reset
  std::vector<hipEvent_t> ev;     // 2 per launch
  int used = 0;                   // pairs recorded since reset
  int64_t dropped = 0;
  double bytes = 0, flops = 0;
};
TimingClass g_timing[DL_KC_COUNT];

// Runs `launch`; when the class is enabled and the launch is sampled, the
// region's kernels carry the event pair on their dispatch packets.
template <typename F>
hipError_t timed(dl_kernel_class kc, hipStream_t st, double bytes, double flops, F&& launch) {
  (void)st;  // the events follow the kernels' own stream
  TimingClass& t = g_timing[kc];
  if (!t.enabled) return launch();
  const uint32_t i = t.seq++;
  if (t.used >= kTimingPool || (t.stride > 1 && ((i * 2654435761u) >> 13) % t.stride != 0)) {
    ++t.dropped;
    return launch();
  }
  DispatchEvents de{t.ev[2 * t.used], t.ev[2 * t.used + 1]};
  g_region_events = &de;
  const hipError_t e = launch();
  g_region_events = nullptr;
  if (e != hipSuccess) return e;
  if (de.start != nullptr) {  // no kernel of the region took the events
    ++t.dropped;
    return hipSuccess;
  }
  ++t.used;
  t.bytes += bytes;
  t.flops += flops;
  return hipSuccess;
}

double gemm_bytes(const dl_dims& d, long long M, long long N, long long K) {
  const double es = (double)esize(d.dtype);
  return es * ((double)N * K + (double)M * K + (double)M * N);
}

// ---------------------------------------------------------------------------
// layer pieces on packed rows
// ---------------------------------------------------------------------------
struct Ctx {
  const dl_dims* d;
  void* ws;
  const Layout* L;
  hipStream_t st;
  long long keys_total;   // sum of valid keys over the batch (host bound, timing only)
  long long rows_x_keys;  // sum over sequences of rows x keys (host bound, timing only)
};

dl_status check_layer(const dl_layer_w* w) {
  if (!w) return fail(DL_E_ARG, "layer weights are NULL");
  DL_TRY(check_ptr(w->attn_norm, "attn_norm"));
  DL_TRY(check_ptr(w->wq, "wq"));
  DL_TRY(check_ptr(w->wk, "wk"));
  DL_TRY(check_ptr(w->wv, "wv"));
  DL_TRY(check_ptr(w->wo, "wo"));
  DL_TRY(check_ptr(w->ffn_norm, "ffn_norm"));
  DL_TRY(check_ptr(w->w_gate, "w_gate"));
  DL_TRY(check_ptr(w->w_up, "w_up"));
  DL_TRY(check_ptr(w->w_down, "w_down"));
  return DL_OK;
}

Epilogue epi_base(const Ctx& c, int kind, const RowMap& rm, int m_base) {
  Epilogue e{};
  e.kind = kind;
  e.row_pos = rm.row_pos + m_base;
  e.row_seq = rm.row_seq + m_base;
  e.S = c.d->S;
  e.d = c.d->d;
  e.head_dim = c.d->head_dim;
  e.F = c.d->d_ffn;
  e.V = c.d->vocab;
  e.rope = at<float2>(c.ws, c.L->rope);
  return e;
}

// One product of rows [m_base, m_base + rows) of A with the weight segments,
// followed by its epilogue: fused into the product on the matrix-core paths,
// as separate kernels on the SIMT path.  EPI_NONE products leave fp32
// partials in the workspace for launch_reduce_rows.  Returns the K split.
dl_status product(const Ctx& c, dl_kernel_class kc, const void* A, const RowMap& rm, int m_base, int rows, int K,
                  const void* const* seg, int n_seg, int N, const Epilogue& e, int* splits_out,
                  float* conf = nullptr, int32_t* argmax = nullptr) {
  const dl_dims& d = *c.d;
  float* P = at<float>(c.ws, c.L->P);
  const GemmPlan p = plan_gemm(d.dtype, rows, N, K, e.kind, d.head_dim, d.d_ffn);
  if (splits_out) *splits_out = p.splits;
  if (kc == DL_KC_GEMM && rows > 128) kc = DL_KC_GEMM_TILED;
  Epilogue ge = e;
  if (p.sep_epi && e.kind != EPI_NONE) ge.kind = EPI_NONE;   // partials; the epilogue kernel finishes
  if (e.kind == EPI_LM) ge.lm_tiles = cdiv(N, p.bn);          // statistics per column tile of the plan
  // the timed region holds the product and, when it has one, its separate
  // epilogue kernel (rows addressed through the full row map)
  DL_CHECK_HIP(timed(kc, c.st, gemm_bytes(d, rows, N, K), 2.0 * rows * N * K, [&] {
    hipError_t err = launch_gemm(d.dtype, p, A, rows, rm.n_rows, m_base, K, seg, n_seg, N, P, ge, c.st,
                                 d.weight_layout);
    if (err != hipSuccess || !p.sep_epi) return err;
    switch (e.kind) {
      case EPI_QKV:
        return launch_epi_qkv(d.dtype, P, p.splits, rm, d.S, d.d, d.head_dim, e.rope, e.q_out, e.k_cache, e.v_cache,
                              c.st);
      case EPI_SWIGLU: return launch_epi_swiglu(d.dtype, P, p.splits, rm, d.d_ffn, e.act_out, c.st);
      case EPI_LM: return launch_lm_reduce(P, p.splits, rm, m_base, rows, d.vocab, conf, argmax, e.logits, c.st);
      default: return hipSuccess;
    }
  }));
  if (!p.sep_epi && e.kind == EPI_LM) {
    DL_CHECK_HIP(launch_lm_merge(e.lm_part, ge.lm_tiles, rm, m_base, rows, conf, argmax, c.st));
  }
  return DL_OK;
}

// Attention sub-block.  On entry act holds RMSNorm(x, attn_norm) if act_ready.
// On exit x has the attention residual added and act = RMSNorm(x, ffn_norm).
// lse_rows (optional): each packed row's per-head log softmax normaliser.
dl_status attn_block(const Ctx& c, const dl_layer_w* w, float* x, const RowMap& rm, const int32_t* seq_len,
                     void* kc, void* vc, bool act_ready, float* lse_rows = nullptr) {
  const dl_dims& d = *c.d;
  void* act = at<void>(c.ws, c.L->act);
  void* q = at<void>(c.ws, c.L->q);
  void* attn = at<void>(c.ws, c.L->attn);
  if (!act_ready) DL_CHECK_HIP(launch_rmsnorm(d.dtype, x, w->attn_norm, rm, d.d, d.rms_eps, act, c.st));
  {
    const void* seg[4] = {w->wq, w->wk, w->wv, w->wv};
    Epilogue e = epi_base(c, EPI_QKV, rm, 0);
    e.q_out = q;
    e.k_cache = kc;
    e.v_cache = vc;
    DL_TRY(product(c, DL_KC_GEMM, act, rm, 0, rm.R_max, d.d, seg, d.d, 3 * d.d, e, nullptr));
  }
  {
    // algorithmic: q rows + every valid key/value row of the sequences once + output rows
    const double es = (double)esize(d.dtype);
    const double keys = (double)c.keys_total;
    DL_CHECK_HIP(timed(DL_KC_ATTN, c.st, es * ((double)rm.R_max * d.d * 2 + 2.0 * keys * d.d),
                       4.0 * (double)c.rows_x_keys * d.d,
                       [&] {
                         const int splits = std::min(
                             c.L->attn_splits, attention_splits(d.dtype, d.head_dim, d.S, d.n_heads, rm, c.L->R_part));
                         return launch_attention(d.dtype, q, kc, vc, seq_len, rm, d.S, d.n_heads, d.head_dim, splits,
                                                 at<float>(c.ws, c.L->attn_o), at<float2>(c.ws, c.L->attn_ml),
                                                 c.L->R_part, attn, c.st, nullptr, nullptr, nullptr, lse_rows, d.B);
                       }));
  }
  {
    const void* seg[4] = {w->wo, w->wo, w->wo, w->wo};
    const Epilogue e = epi_base(c, EPI_NONE, rm, 0);
    int splits = 1;
    DL_TRY(product(c, DL_KC_GEMM, attn, rm, 0, rm.R_max, d.d, seg, d.d, d.d, e, &splits));
    DL_CHECK_HIP(launch_reduce_rows(d.dtype, at<float>(c.ws, c.L->P), splits, rm, d.d, x, w->ffn_norm, d.rms_eps,
                                    act, c.st));
  }
  return DL_OK;
}

// FFN sub-block; act = RMSNorm(x, ffn_norm) on entry.  On exit x has the FFN
// residual added and, if next_norm != nullptr, act = RMSNorm(x, next_norm).
dl_status ffn_block(const Ctx& c, const dl_layer_w* w, float* x, const RowMap& rm, const void* next_norm) {
  const dl_dims& d = *c.d;
  void* act = at<void>(c.ws, c.L->act);
  void* ffn_act = at<void>(c.ws, c.L->ffn_act);
  {
    const void* seg[4] = {w->w_gate, w->w_up, w->w_up, w->w_up};
    Epilogue e = epi_base(c, EPI_SWIGLU, rm, 0);
    e.act_out = ffn_act;
    DL_TRY(product(c, DL_KC_GEMM, act, rm, 0, rm.R_max, d.d, seg, d.d_ffn, 2 * d.d_ffn, e, nullptr));
  }
  {
    const void* seg[4] = {w->w_down, w->w_down, w->w_down, w->w_down};
    const Epilogue e = epi_base(c, EPI_NONE, rm, 0);
    int splits = 1;
    DL_TRY(product(c, DL_KC_GEMM, ffn_act, rm, 0, rm.R_max, d.d_ffn, seg, d.d, d.d, e, &splits));
    DL_CHECK_HIP(launch_reduce_rows(d.dtype, at<float>(c.ws, c.L->P), splits, rm, d.d, x, next_norm, d.rms_eps, act,
                                    c.st));
  }
  return DL_OK;
}

// Layers [l0, l1) on the rows of rm.  act_ready: act already holds
// RMSNorm(x, attn_norm of l0).  next_after: the gain normalised into act after
// the last layer (nullptr: none).
dl_status run_layers(const Ctx& c, const dl_model* model, int l0, int l1, float* x, const RowMap& rm,
                     const int32_t* seq_len, char* k_cache, char* v_cache, bool act_ready, const void* next_after) {
  const size_t lstride = (size_t)c.d->B * c.d->S * c.d->d * esize(c.d->dtype);
  for (int l = l0; l < l1; ++l) {
    const dl_layer_w* w = &model->layers[l];
    DL_TRY(attn_block(c, w, x, rm, seq_len, k_cache + (size_t)l * lstride, v_cache + (size_t)l * lstride, act_ready));
    const void* nn = l + 1 < l1 ? model->layers[l + 1].attn_norm : next_after;
    DL_TRY(ffn_block(c, w, x, rm, nn));
    act_ready = nn != nullptr;
  }
  return DL_OK;
}

dl_status lm_block(const Ctx& c, const void* final_norm, const void* lm_head, const float* x, const RowMap& rm,
                   float* conf, int32_t* argmax, void* h_final, float* logits, bool act_ready) {
  const dl_dims& d = *c.d;
  void* act = at<void>(c.ws, c.L->act);
  if (!act_ready) DL_CHECK_HIP(launch_rmsnorm(d.dtype, x, final_norm, rm, d.d, d.rms_eps, act, c.st));
  const void* seg[4] = {lm_head, lm_head, lm_head, lm_head};
  for (int m0 = 0; m0 < rm.R_max; m0 += kLmChunk) {
    const int rows = std::min(kLmChunk, rm.R_max - m0);
    const void* A = static_cast<const char*>(act) + (size_t)m0 * d.d * esize(d.dtype);
    Epilogue e = epi_base(c, EPI_LM, rm, m0);
    e.lm_part = at<float>(c.ws, c.L->lm_part);
    e.lm_tiles = cdiv(d.vocab, 128);
    e.logits = logits;
    DL_TRY(product(c, DL_KC_LMHEAD, A, rm, m0, rows, d.d, seg, d.vocab, d.vocab, e, nullptr, conf, argmax));
  }
  DL_CHECK_HIP(launch_store_rows(d.dtype, x, d.d, rm, h_final, c.st));
  return DL_OK;
}

size_t layer_stride_bytes(const dl_dims& d) { return (size_t)d.B * d.S * d.d * esize(d.dtype); }

// Layers [s, L) of the per-layer variant (DyLLM section 2B).  The active rows
// (sel_A / rm_A, inputs x_A packed in fp32, act = their RMSNorm for layer s
// when act_ready) are every row on a refresh step, the first selection
// otherwise.  rm_all / all_off: every valid row, packed by sequence offsets
// (x_all holds their layer-s inputs).  On return *rows / *x_rows / *sel_out
// describe the rows through the last layer, and act holds their final norm.
struct LayerSel {
  int32_t *idx, *cnt, *off;
};

dl_status per_layer_layers(const Ctx& c, const dl_model* model, const dl_state* s, const dl_step_params* p,
                           bool refresh, LayerSel sel_A, RowMap rm_A, float* x_A, bool act_ready,
                           const RowMap& rm_all, const int32_t* all_off, float* x_all, long long R_l,
                           long long A_x_keys, long long R_x_keys, RowMap* rows_out, float** x_out,
                           LayerSel* sel_out) {
  const dl_dims& d = *c.d;
  const Layout& L = *c.L;
  const size_t es = esize(d.dtype);
  const size_t lstride = (size_t)d.B * d.S * d.d * es;
  const size_t fstride = (size_t)d.B * d.S * d.d;
  const size_t hstride = (size_t)d.B * d.S * d.n_heads;
  void* act = at<void>(c.ws, L.act);
  void* q = at<void>(c.ws, L.q);
  void* attn = at<void>(c.ws, L.attn);
  void* k_act = at<void>(c.ws, L.k_act);
  void* v_old = at<void>(c.ws, L.v_old);
  void* dv = at<void>(c.ws, L.dv);
  float* ctx_new = at<float>(c.ws, L.ctx_new);
  int32_t* inv = at<int32_t>(c.ws, L.inv);
  float* lscores = s->layer_scores ? s->layer_scores : at<float>(c.ws, L.scores2);
  float* xbuf[2] = {at<float>(c.ws, L.x_sel), at<float>(c.ws, L.x_sel2)};
  int turn = x_A == xbuf[0] ? 1 : 0;             // the salient rows never land on the active rows' buffer
  const int sl = p->skip_layer;
  for (int l = sl; l < d.n_layers; ++l) {
    const long long ax = l == sl ? A_x_keys : R_x_keys;   // sum over sequences of active rows x keys (timing)
    const dl_layer_w* w = &model->layers[l];
    char* kc = static_cast<char*>(s->k_cache) + (size_t)l * lstride;
    char* vc = static_cast<char*>(s->v_cache) + (size_t)l * lstride;
    char* qc = static_cast<char*>(s->q_cache) + (size_t)l * lstride;
    float* ctx_l = s->ctx_cache + (size_t)l * fstride;
    float* lse_l = s->lse_cache + (size_t)l * hstride;
    float* y_l = s->y_cache + (size_t)l * fstride;
    if (!act_ready) DL_CHECK_HIP(launch_rmsnorm(d.dtype, x_A, w->attn_norm, rm_A, d.d, d.rms_eps, act, c.st));
    if (!refresh) {
      // the active rows' keys and values as the cached contexts saw them
      DL_CHECK_HIP(launch_gather(es, kc, nullptr, d.S, d.d, rm_A, k_act, c.st));
      DL_CHECK_HIP(launch_gather(es, vc, nullptr, d.S, d.d, rm_A, v_old, c.st));
    }
    {  // fresh q / k / v of the active rows; their K/V rows into the caches
      const void* seg[4] = {w->wq, w->wk, w->wv, w->wv};
      Epilogue e = epi_base(c, EPI_QKV, rm_A, 0);
      e.q_out = q;
      e.k_cache = kc;
      e.v_cache = vc;
      DL_TRY(product(c, DL_KC_GEMM, act, rm_A, 0, rm_A.R_max, d.d, seg, d.d, 3 * d.d, e, nullptr));
    }
    // exact contexts (fp32, packed over all rows) and normalisers of the active rows
    {
      const double kk = (double)c.keys_total;
      DL_CHECK_HIP(timed(DL_KC_ATTN, c.st, (double)es * ((double)rm_A.R_max * d.d * 2 + 2.0 * kk * d.d),
                         4.0 * (double)ax * d.d, [&] {
                           const int splits = std::min(L.attn_splits, attention_splits(d.dtype, d.head_dim, d.S,
                                                                                      d.n_heads, rm_A, L.R_part));
                           return launch_attention(d.dtype, q, kc, vc, s->seq_len, rm_A, d.S, d.n_heads, d.head_dim,
                                                   splits, at<float>(c.ws, L.attn_o), at<float2>(c.ws, L.attn_ml),
                                                   L.R_part, attn, c.st, ctx_new, all_off, lse_l);
                         }));
    }
    RowMap rm_R = rm_A;
    LayerSel sel_R = sel_A;
    float* x_R = x_A;
    if (refresh) {
      DL_CHECK_HIP(launch_scatter(sizeof(float), ctx_new, d.d, rm_all, ctx_l, c.st));
    } else {
      // approximate contexts of every other row, then saliency and ctx cache <- new
      DL_CHECK_HIP(launch_value_change(d.dtype, vc, v_old, rm_A, d.d, dv, c.st));
      DL_CHECK_HIP(launch_inv_rows(rm_A, d.B * d.S, inv, c.st));
      DL_CHECK_HIP(timed(DL_KC_APPROX, c.st,
                         (double)es * ((double)rm_all.R_max * d.d + 2.0 * rm_A.R_max * d.d) +
                             8.0 * rm_all.R_max * d.d,
                         4.0 * (double)ax * d.d, [&] {
                           return launch_attention_approx(d.dtype, qc, k_act, dv, sel_A.off, sel_A.cnt, lse_l, inv,
                                                          ctx_l, ctx_new, rm_all, d.S, d.n_heads, d.head_dim, c.st);
                         }));
      DL_CHECK_HIP(launch_score(DL_F32, nullptr, ctx_new, all_off, ctx_l, s->conf, s->seq_len, d.B, d.S, d.d,
                                DL_SCORE_COSINE, 0.f, lscores, c.st));
      const int tsel = turn;
      sel_R = LayerSel{at<int32_t>(c.ws, L.lsel_idx[tsel]), at<int32_t>(c.ws, L.lsel_count[tsel]),
                       at<int32_t>(c.ws, L.lsel_off[tsel])};
      DL_CHECK_HIP(launch_select(lscores, s->seq_len, d.B, d.S, p->mode_l, p->keep_ratio_l, p->threshold_l, sel_R.idx,
                                 sel_R.cnt, c.st));
      rm_R = rowmap_at(c.ws, L.map_l[tsel], (int)R_l, std::min(L.T, cdiv(R_l, kTileRows) + d.B));
      DL_CHECK_HIP(launch_row_off_map(sel_R.idx, sel_R.cnt, sel_R.off, d.B, d.S, rm_R, c.st));
      // inputs of the salient rows: X_s at layer s, the cached output of the layer below above it
      x_R = xbuf[tsel];
      if (l == sl)
        DL_CHECK_HIP(launch_gather(sizeof(float), x_all, all_off, d.S, d.d, rm_R, x_R, c.st));
      else
        DL_CHECK_HIP(launch_gather(sizeof(float), s->y_cache + (size_t)(l - 1) * fstride, nullptr, d.S, d.d, rm_R,
                                   x_R, c.st));
      turn ^= 1;
    }
    // the active rows' queries into the cache
    DL_CHECK_HIP(launch_scatter(es, q, d.d, rm_A, qc, c.st));
    // Wo and the FFN on the salient rows, from their new contexts
    DL_CHECK_HIP(launch_gather_cvt(d.dtype, ctx_new, all_off, d.S, d.d, rm_R, attn, c.st));
    {
      const void* seg[4] = {w->wo, w->wo, w->wo, w->wo};
      const Epilogue e = epi_base(c, EPI_NONE, rm_R, 0);
      int splits = 1;
      DL_TRY(product(c, DL_KC_GEMM, attn, rm_R, 0, rm_R.R_max, d.d, seg, d.d, d.d, e, &splits));
      DL_CHECK_HIP(launch_reduce_rows(d.dtype, at<float>(c.ws, L.P), splits, rm_R, d.d, x_R, w->ffn_norm, d.rms_eps,
                                      act, c.st));
    }
    const void* nn = l + 1 < d.n_layers ? model->layers[l + 1].attn_norm : model->final_norm;
    DL_TRY(ffn_block(c, w, x_R, rm_R, nn));
    DL_CHECK_HIP(launch_scatter(sizeof(float), x_R, d.d, rm_R, y_l, c.st));
    rm_A = rm_R;
    sel_A = sel_R;
    x_A = x_R;
    act_ready = true;
  }
  *rows_out = rm_A;
  *x_out = x_A;
  *sel_out = sel_A;
  return DL_OK;
}

// The key (rotated) or value rows of layer l for the packed rows of rm, in
// fp32, from act = RMSNorm(x, attn_norm of l) (already in the workspace):
// one product with Wk or Wv, its split-K partials summed in order, then RoPE
// at each row's position for keys.
dl_status scored_kv_rows(const Ctx& c, const dl_layer_w* w, dl_score_tensor which, const RowMap& rm, float* t) {
  const dl_dims& d = *c.d;
  const void* W = which == DL_TENSOR_KEY ? w->wk : w->wv;
  const void* seg[4] = {W, W, W, W};
  const Epilogue e = epi_base(c, EPI_NONE, rm, 0);
  int splits = 1;
  DL_TRY(product(c, DL_KC_GEMM, at<void>(c.ws, c.L->act), rm, 0, rm.R_max, d.d, seg, d.d, d.d, e, &splits));
  DL_CHECK_HIP(launch_fill_i32(reinterpret_cast<int32_t*>(t), 0, (size_t)rm.R_max * d.d, c.st));
  DL_CHECK_HIP(launch_reduce_rows(d.dtype, at<float>(c.ws, c.L->P), splits, rm, d.d, t, nullptr, d.rms_eps, nullptr,
                                  c.st));
  if (which == DL_TENSOR_KEY)
    DL_CHECK_HIP(launch_rope_rows(t, rm, d.S, d.d, d.head_dim, at<float2>(c.ws, c.L->rope), c.st));
  return DL_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// the no-allocation step's workspace: a file-scope device array.  Each device
// the library runs on holds its own copy until the process ends.  In host code
// the array's name is only a stand-in; host code passes the device address
// that hipGetSymbolAddress gives for the current device.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = DL_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
dl_status scratch_on_current_device(void** out) {
  int dev = 0;
  DL_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DL_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DL_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(DL_E_HIP, "hipGetSymbolAddress gave no address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DL_OK;
}
}  // namespace

// ===========================================================================
// exported entry points
// ===========================================================================
extern "C" {

int32_t dl_abi_version(void) { return DL_ABI_VERSION; }

dl_status dl_pack_weights(const void* src, void* dst, int32_t N, int32_t K, dl_dtype dtype, void* stream) {
  DL_TRY(check_ptr(src, "src"));
  DL_TRY(check_ptr(dst, "dst"));
  if (N < 1 || K < 1) return fail(DL_E_ARG, "N and K must be positive");
  if (dtype != DL_BF16) return fail(DL_E_DTYPE, "blocked weights are bf16 only");
  if (N % 8 || K % 64) return fail(DL_E_SHAPE, "blocked weights need N %% 8 == 0 and K %% 64 == 0 (N=%d, K=%d)", N, K);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, n = (uintptr_t)N * (uintptr_t)K * 2;
  if (a < b + n && b < a + n) return fail(DL_E_ARG, "dst overlaps src");
  if ((a | b) & 15) return fail(DL_E_ALIGN, "src and dst must be 16-byte aligned");
  DL_CHECK_HIP(launch_pack_weights(src, dst, N, K, (hipStream_t)stream));
  return DL_OK;
}

int64_t dl_row_map_ints(int32_t B, int32_t S) {
  if (B < 1 || S < 1) return 0;
  return 1 + 2 * (int64_t)B * S + 2 * row_map_tiles(B, S);
}

dl_status dl_timing_enable(dl_kernel_class kc, int32_t stride) {
  if (kc < 0 || kc >= DL_KC_COUNT) return fail(DL_E_ARG, "kernel class %d unknown", (int)kc);
  if (stride < 0) return fail(DL_E_ARG, "sampling stride %d < 0", (int)stride);
  TimingClass& t = g_timing[kc];
  if (stride && t.ev.empty()) {
    t.ev.resize(2 * kTimingPool);
    for (auto& e : t.ev) DL_CHECK_HIP(hipEventCreate(&e));
  }
  t.enabled = stride != 0;
  t.stride = stride ? (uint32_t)stride : 1u;
  return DL_OK;
}

dl_status dl_timing_reset(void) {
  for (auto& t : g_timing) {
    t.used = 0;
    t.seq = 0;
    t.dropped = 0;
    t.bytes = t.flops = 0;
  }
  return DL_OK;
}

dl_status dl_timing_read(dl_kernel_class kc, dl_timing* out) {
  if (kc < 0 || kc >= DL_KC_COUNT) return fail(DL_E_ARG, "kernel class %d unknown", (int)kc);
  if (!out) return fail(DL_E_ARG, "out is NULL");
  TimingClass& t = g_timing[kc];
  double ms = 0;
  for (int i = 0; i < t.used; ++i) {
    DL_CHECK_HIP(hipEventSynchronize(t.ev[2 * i + 1]));
    float m = 0.f;
    DL_CHECK_HIP(hipEventElapsedTime(&m, t.ev[2 * i], t.ev[2 * i + 1]));
    ms += m;
  }
  out->launches = t.used;
  out->dropped = t.dropped;
  out->ms = ms;
  out->bytes = t.bytes;
  out->flops = t.flops;
  return DL_OK;
}

const char* dl_last_error(void) { return g_err; }

const char* dl_status_string(dl_status s) {
  switch (s) {
    case DL_OK: return "ok";
    case DL_E_ARG: return "invalid argument";
    case DL_E_SHAPE: return "inconsistent shape";
    case DL_E_DTYPE: return "unsupported dtype";
    case DL_E_ALIGN: return "misaligned pointer";
    case DL_E_WORKSPACE: return "workspace too small";
    case DL_E_HIP: return "HIP runtime error";
    case DL_E_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

size_t dl_workspace_bytes(const dl_dims* dims, int32_t max_rows) {
  if (check_dims(dims) != DL_OK) return 0;
  const int R = max_rows > 0 ? max_rows : dims->B * dims->S;
  return make_layout(*dims, R).total;
}

dl_status dl_score_select(const dl_dims* dims, const void* h_cur, const void* h_prev, const float* conf,
                          const int32_t* seq_len, dl_score_kind kind, float alpha, dl_select_mode mode,
                          float keep_ratio, float threshold, dl_selection* out, float* scores_or_null, void* ws,
                          size_t ws_bytes, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_ptr(h_cur, "h_cur"));
  DL_TRY(check_ptr(h_prev, "h_prev"));
  DL_TRY(check_ptr(conf, "conf"));
  DL_TRY(check_ptr(seq_len, "seq_len"));
  DL_TRY(check_sel(out, "out"));
  if (h_cur == h_prev) return fail(DL_E_ARG, "h_cur and h_prev alias");
  if (kind < DL_SCORE_ESDLLM || kind > DL_SCORE_COSINE) return fail(DL_E_ARG, "score kind %d unknown", (int)kind);
  if (mode != DL_SEL_TOPK && mode != DL_SEL_THRESHOLD) return fail(DL_E_ARG, "select mode %d unknown", (int)mode);
  if (mode == DL_SEL_TOPK && !(keep_ratio > 0.f && keep_ratio <= 1.f))
    return fail(DL_E_ARG, "keep_ratio %g outside (0, 1]", (double)keep_ratio);
  float* scores = scores_or_null;
  if (scores) DL_TRY(check_ptr(scores, "scores"));
  const size_t need = dl_workspace_bytes(dims, 1);
  if (!scores) {
    DL_TRY(check_ptr(ws, "ws"));
    if (ws_bytes < need) return fail(DL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    scores = at<float>(ws, make_layout(*dims, 1).scores);
  }
  hipStream_t st = (hipStream_t)stream;
  DL_CHECK_HIP(launch_score(dims->dtype, h_cur, nullptr, nullptr, const_cast<void*>(h_prev), conf, seq_len, dims->B,
                            dims->S, dims->d, kind, alpha, scores, st));
  RowMap rm{};
  if (out->row_map) rm = rowmap_of_sel(out, dims->B, dims->S, dims->B * dims->S);
  if (dims->B == 1) {   // one sequence: row_off (and the map) from the selection's own launch
    DL_CHECK_HIP(launch_select(scores, seq_len, 1, dims->S, mode, keep_ratio, threshold, out->sel_idx,
                               out->sel_count, st, nullptr, nullptr, nullptr, out->row_off,
                               out->row_map ? &rm : nullptr));
    return DL_OK;
  }
  DL_CHECK_HIP(launch_select(scores, seq_len, dims->B, dims->S, mode, keep_ratio, threshold, out->sel_idx,
                             out->sel_count, st));
  if (out->row_map)
    DL_CHECK_HIP(launch_row_off_map(out->sel_idx, out->sel_count, out->row_off, dims->B, dims->S, rm, st));
  else
    DL_CHECK_HIP(launch_row_off(out->sel_count, out->row_off, dims->B, st));
  return DL_OK;
}

dl_status dl_gather(const dl_dims* dims, const void* src, int32_t w, dl_dtype dtype, const dl_selection* sel,
                    int32_t k_total_max, void* dst, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_ptr(src, "src"));
  DL_TRY(check_ptr(dst, "dst"));
  DL_TRY(check_sel(sel, "sel"));
  if (w < 1 || k_total_max < 0) return fail(DL_E_ARG, "w must be positive and k_total_max non-negative");
  if (dtype != DL_F32 && dtype != DL_BF16) return fail(DL_E_DTYPE, "dtype %d unknown", (int)dtype);
  if (k_total_max > dims->B * dims->S) return fail(DL_E_SHAPE, "k_total_max > B*S");
  DL_CHECK_HIP(launch_gather_sel(esize(dtype), src, w, sel->sel_idx, sel->row_off, dims->B, dims->S, k_total_max,
                                 dst, (hipStream_t)stream));
  return DL_OK;
}

dl_status dl_scatter_cache(const dl_dims* dims, const void* rows, int32_t w, dl_dtype dtype, const dl_selection* sel,
                           int32_t k_total_max, void* cache, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_ptr(rows, "rows"));
  DL_TRY(check_ptr(cache, "cache"));
  DL_TRY(check_sel(sel, "sel"));
  if (w < 1 || k_total_max < 0) return fail(DL_E_ARG, "w must be positive and k_total_max non-negative");
  if (dtype != DL_F32 && dtype != DL_BF16) return fail(DL_E_DTYPE, "dtype %d unknown", (int)dtype);
  if (k_total_max > dims->B * dims->S) return fail(DL_E_SHAPE, "k_total_max > B*S");
  DL_CHECK_HIP(launch_scatter_sel(esize(dtype), rows, w, sel->sel_idx, sel->row_off, dims->B, dims->S, k_total_max,
                                  cache, (hipStream_t)stream));
  return DL_OK;
}

static dl_status prep_rows(const dl_dims* dims, const dl_selection* sel, int32_t k_total_max, void* ws,
                           size_t ws_bytes, Layout* L, RowMap* rm, hipStream_t st) {
  DL_TRY(check_sel(sel, "sel"));
  DL_TRY(check_ptr(ws, "ws"));
  if (k_total_max < 0 || k_total_max > dims->B * dims->S) return fail(DL_E_SHAPE, "k_total_max outside [0, B*S]");
  *L = make_layout(*dims, k_total_max);
  if (ws_bytes < L->total) return fail(DL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L->total);
  if (sel->row_map) {   // written by dl_score_select with row_off
    *rm = rowmap_of_sel(sel, dims->B, dims->S, k_total_max);
    return DL_OK;
  }
  *rm = rowmap_at(ws, L->map_sel, k_total_max, std::min(L->T, cdiv(k_total_max, kTileRows) + dims->B));
  DL_CHECK_HIP(launch_rowmap(sel->sel_idx, sel->sel_count, sel->row_off, dims->B, dims->S, *rm, st));
  return DL_OK;
}

dl_status dl_partial_attn(const dl_dims* dims, const dl_layer_w* layer, float* x_rows, const dl_selection* sel,
                          const int32_t* seq_len, int32_t k_total_max, void* k_cache, void* v_cache,
                          float* lse_or_null, void* ws, size_t ws_bytes, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_layer(layer));
  DL_TRY(check_ptr(x_rows, "x_rows"));
  DL_TRY(check_ptr(seq_len, "seq_len"));
  DL_TRY(check_ptr(k_cache, "k_cache"));
  DL_TRY(check_ptr(v_cache, "v_cache"));
  hipStream_t st = (hipStream_t)stream;
  Layout L;
  RowMap rm;
  DL_TRY(prep_rows(dims, sel, k_total_max, ws, ws_bytes, &L, &rm, st));
  if (k_total_max == 0) return DL_OK;
  // the rows' RMSNorm and the RoPE table in one launch
  DL_CHECK_HIP(launch_rmsnorm_rope(dims->dtype, x_rows, layer->attn_norm, rm, dims->d, dims->rms_eps,
                                   at<void>(ws, L.act), dims->S, dims->head_dim, dims->rope_base,
                                   at<float2>(ws, L.rope), st));
  Ctx c{dims, ws, &L, st, (long long)dims->B * dims->S, (long long)k_total_max * dims->S};
  DL_TRY(attn_block(c, layer, x_rows, rm, seq_len, k_cache, v_cache, true, lse_or_null));
  return DL_OK;
}

dl_status dl_ffn_rows(const dl_dims* dims, const dl_layer_w* layer, float* x_rows, const dl_selection* sel,
                      int32_t k_total_max, void* ws, size_t ws_bytes, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_layer(layer));
  DL_TRY(check_ptr(x_rows, "x_rows"));
  hipStream_t st = (hipStream_t)stream;
  Layout L;
  RowMap rm;
  DL_TRY(prep_rows(dims, sel, k_total_max, ws, ws_bytes, &L, &rm, st));
  if (k_total_max == 0) return DL_OK;
  Ctx c{dims, ws, &L, st, 0, 0};
  DL_CHECK_HIP(launch_rmsnorm(dims->dtype, x_rows, layer->ffn_norm, rm, dims->d, dims->rms_eps, at<void>(ws, L.act),
                              st));
  return ffn_block(c, layer, x_rows, rm, nullptr);
}

dl_status dl_lm_head_rows(const dl_dims* dims, const void* final_norm, const void* lm_head, const float* x_rows,
                          const dl_selection* sel, int32_t k_total_max, float* conf, int32_t* argmax, void* h_final,
                          float* logits_or_null, void* ws, size_t ws_bytes, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_ptr(final_norm, "final_norm"));
  DL_TRY(check_ptr(lm_head, "lm_head"));
  DL_TRY(check_ptr(x_rows, "x_rows"));
  DL_TRY(check_ptr(conf, "conf"));
  DL_TRY(check_ptr(argmax, "argmax"));
  DL_TRY(check_ptr(h_final, "h_final"));
  if (logits_or_null) DL_TRY(check_ptr(logits_or_null, "logits"));
  hipStream_t st = (hipStream_t)stream;
  Layout L;
  RowMap rm;
  DL_TRY(prep_rows(dims, sel, k_total_max, ws, ws_bytes, &L, &rm, st));
  if (k_total_max == 0) return DL_OK;
  Ctx c{dims, ws, &L, st, 0, 0};
  return lm_block(c, final_norm, lm_head, x_rows, rm, conf, argmax, h_final, logits_or_null, false);
}

dl_status dl_unmask(const dl_dims* dims, int32_t* tokens, uint8_t* masked, const float* conf, const int32_t* argmax,
                    const int32_t* prompt_len, const int32_t* seq_len, int32_t block, int32_t block_len,
                    int32_t n_unmask, void* stream) {
  DL_TRY(check_dims(dims));
  DL_TRY(check_ptr(tokens, "tokens"));
  DL_TRY(check_ptr(masked, "masked"));
  DL_TRY(check_ptr(conf, "conf"));
  DL_TRY(check_ptr(argmax, "argmax"));
  DL_TRY(check_ptr(prompt_len, "prompt_len"));
  DL_TRY(check_ptr(seq_len, "seq_len"));
  if (block < 0 || block_len < 1 || n_unmask < 0) return fail(DL_E_ARG, "block/block_len/n_unmask out of range");
  if (block_len > 1024) return fail(DL_E_UNSUPPORTED, "block_len > 1024");
  DL_CHECK_HIP(launch_unmask(tokens, masked, conf, argmax, prompt_len, seq_len, dims->B, dims->S, block, block_len,
                             n_unmask, (hipStream_t)stream));
  return DL_OK;
}

dl_status dl_denoise_step(const dl_model* model, dl_state* s, const dl_step_params* p, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!model || !s || !p) return fail(DL_E_ARG, "model, state and params must be non-NULL");
  const dl_dims* dims = &model->dims;
  DL_TRY(check_dims(dims));
  const dl_dims& d = *dims;
  DL_TRY(check_ptr(model->embed, "embed"));
  DL_TRY(check_ptr(model->final_norm, "final_norm"));
  DL_TRY(check_ptr(model->lm_head, "lm_head"));
  if (!model->layers) return fail(DL_E_ARG, "model.layers is NULL");
  for (int l = 0; l < d.n_layers; ++l) DL_TRY(check_layer(&model->layers[l]));
  DL_TRY(check_ptr(s->tokens, "tokens"));
  DL_TRY(check_ptr(s->masked, "masked"));
  DL_TRY(check_ptr(s->seq_len, "seq_len"));
  DL_TRY(check_ptr(s->prompt_len, "prompt_len"));
  DL_TRY(check_ptr(s->h_prev, "h_prev"));
  DL_TRY(check_ptr(s->k_cache, "k_cache"));
  DL_TRY(check_ptr(s->v_cache, "v_cache"));
  DL_TRY(check_ptr(s->h_final, "h_final"));
  DL_TRY(check_ptr(s->conf, "conf"));
  DL_TRY(check_ptr(s->argmax, "argmax"));
  if (s->logits) DL_TRY(check_ptr(s->logits, "logits"));
  if (s->scores) DL_TRY(check_ptr(s->scores, "scores"));
  DL_TRY(check_sel(&s->sel, "state.sel"));
  DL_TRY(check_ptr(ws, "ws"));
  if (!p->seq_len_host) return fail(DL_E_ARG, "params.seq_len_host is NULL");
  if (p->skip_layer < 1 || p->skip_layer > d.n_layers)
    return fail(DL_E_ARG, "skip_layer %d outside [1, %d]", p->skip_layer, d.n_layers);
  if (p->score < DL_SCORE_ESDLLM || p->score > DL_SCORE_COSINE) return fail(DL_E_ARG, "score kind unknown");
  if (p->mode != DL_SEL_TOPK && p->mode != DL_SEL_THRESHOLD) return fail(DL_E_ARG, "select mode unknown");
  if (p->mode == DL_SEL_TOPK && !(p->keep_ratio > 0.f && p->keep_ratio <= 1.f))
    return fail(DL_E_ARG, "keep_ratio %g outside (0, 1]", (double)p->keep_ratio);
  if (p->block < 0 || p->block_len < 1 || p->n_unmask < 0) return fail(DL_E_ARG, "block schedule out of range");
  if (p->block_len > 1024) return fail(DL_E_UNSUPPORTED, "block_len > 1024");
  const bool refresh = p->full_refresh != 0;
  const bool two = p->skip_layer2 != 0;
  if (two) {
    if (p->skip_layer2 <= p->skip_layer || p->skip_layer2 > d.n_layers)
      return fail(DL_E_ARG, "skip_layer2 %d outside (%d, %d]", p->skip_layer2, p->skip_layer, d.n_layers);
    if (p->mode2 != DL_SEL_TOPK && p->mode2 != DL_SEL_THRESHOLD) return fail(DL_E_ARG, "select mode2 unknown");
    if (p->mode2 == DL_SEL_TOPK && !(p->keep_ratio2 > 0.f && p->keep_ratio2 <= 1.f))
      return fail(DL_E_ARG, "keep_ratio2 %g outside (0, 1]", (double)p->keep_ratio2);
    if (p->mode == DL_SEL_TOPK && p->mode2 == DL_SEL_TOPK && p->keep_ratio2 > p->keep_ratio)
      return fail(DL_E_ARG, "keep_ratio2 %g above keep_ratio %g", (double)p->keep_ratio2, (double)p->keep_ratio);
    DL_TRY(check_ptr(s->h_prev2, "h_prev2"));
    DL_TRY(check_sel(&s->sel2, "state.sel2"));
    if (s->scores2) DL_TRY(check_ptr(s->scores2, "scores2"));
    if (s->h_prev2 == s->h_prev) return fail(DL_E_ARG, "h_prev2 and h_prev alias");
    if (s->sel2.sel_idx == s->sel.sel_idx || s->sel2.sel_count == s->sel.sel_count ||
        s->sel2.row_off == s->sel.row_off)
      return fail(DL_E_ARG, "state.sel2 and state.sel alias");
  }
  if (p->score_tensor < DL_TENSOR_HIDDEN || p->score_tensor > DL_TENSOR_VALUE)
    return fail(DL_E_ARG, "score_tensor %d unknown", (int)p->score_tensor);
  const bool kv = p->score_tensor != DL_TENSOR_HIDDEN;
  if (kv && p->skip_layer >= d.n_layers)
    return fail(DL_E_ARG, "a key/value score needs skip_layer (%d) < n_layers (%d)", p->skip_layer, d.n_layers);
  const bool resp = p->response_only != 0 && !refresh;
  if (resp && !p->prompt_len_host) return fail(DL_E_ARG, "params.prompt_len_host is NULL on a response-only step");
  const bool per_layer = p->per_layer != 0;
  if (per_layer) {
    if (p->skip_layer >= d.n_layers)
      return fail(DL_E_ARG, "per-layer re-selection needs skip_layer (%d) < n_layers (%d)", p->skip_layer,
                  d.n_layers);
    if (two) return fail(DL_E_UNSUPPORTED, "per-layer re-selection with a second skip level");
    if (p->response_only) return fail(DL_E_UNSUPPORTED, "per-layer re-selection on a response-only step");
    if (p->mode_l != DL_SEL_TOPK && p->mode_l != DL_SEL_THRESHOLD) return fail(DL_E_ARG, "select mode_l unknown");
    if (p->mode_l == DL_SEL_TOPK && !(p->keep_ratio_l > 0.f && p->keep_ratio_l <= 1.f))
      return fail(DL_E_ARG, "keep_ratio_l %g outside (0, 1]", (double)p->keep_ratio_l);
    DL_TRY(check_ptr(s->q_cache, "q_cache"));
    DL_TRY(check_ptr(s->ctx_cache, "ctx_cache"));
    DL_TRY(check_ptr(s->lse_cache, "lse_cache"));
    DL_TRY(check_ptr(s->y_cache, "y_cache"));
    if (s->layer_scores) DL_TRY(check_ptr(s->layer_scores, "layer_scores"));
    DL_TRY(check_sel(&s->sel_l, "state.sel_l"));
    if (s->sel_l.sel_idx == s->sel.sel_idx || s->sel_l.sel_count == s->sel.sel_count ||
        s->sel_l.row_off == s->sel.row_off)
      return fail(DL_E_ARG, "state.sel_l and state.sel alias");
  }

  // Host row bounds (grid sizing; exact for top-k): candidates, first and second level.
  auto topk_count = [](float keep, long long base) -> long long {
    if (base <= 0) return 0;
    const double kk = ceil((double)keep * (double)base);
    return kk < 1.0 ? 1 : (kk > (double)base ? base : (long long)kk);
  };
  long long R_all = 0, R_cand = 0, R_sel = 0, R_sel2 = 0, R_l = 0;
  long long cand_x_keys = 0, sel_x_keys = 0, sel2_x_keys = 0, l_x_keys = 0;
  for (int b = 0; b < d.B; ++b) {
    const int n = p->seq_len_host[b];
    if (n < 0 || n > d.S) return fail(DL_E_SHAPE, "seq_len_host[%d] = %d outside [0, S=%d]", b, n, d.S);
    const int P0 = resp ? p->prompt_len_host[b] : 0;
    if (P0 < 0 || P0 > n) return fail(DL_E_SHAPE, "prompt_len_host[%d] = %d outside [0, %d]", b, P0, n);
    const long long nc = n - P0;
    const long long k1 = p->mode == DL_SEL_TOPK && !refresh ? topk_count(p->keep_ratio, nc) : nc;
    const long long k2 = two && p->mode2 == DL_SEL_TOPK && !refresh ? std::min(topk_count(p->keep_ratio2, nc), k1) : k1;
    R_all += n;
    R_cand += nc;
    R_sel += k1;
    R_sel2 += k2;
    const long long kl = per_layer && p->mode_l == DL_SEL_TOPK && !refresh ? topk_count(p->keep_ratio_l, n) : n;
    R_l += kl;
    l_x_keys += kl * n;
    cand_x_keys += nc * n;
    sel_x_keys += k1 * n;
    sel2_x_keys += k2 * n;
  }
  const Layout L = make_layout(d, (int)R_all);
  if (ws_bytes < L.total) return fail(DL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);

  hipStream_t st = (hipStream_t)stream;
  Ctx c{dims, ws, &L, st, R_all, cand_x_keys};
  const int sl = p->skip_layer;
  const int s2 = two ? p->skip_layer2 : 0;
  int32_t* all_idx = at<int32_t>(ws, L.sel_idx);
  int32_t* all_cnt = at<int32_t>(ws, L.sel_count);
  int32_t* all_off = at<int32_t>(ws, L.row_off);
  int32_t* inv = at<int32_t>(ws, L.inv);
  auto tiles = [&](long long R) { return std::min(L.T, cdiv(R, kTileRows) + d.B); };
  const RowMap rm_all = rowmap_at(ws, L.map_all, (int)R_cand, tiles(R_cand));
  float* x_all = at<float>(ws, L.x_all);

  // the step's candidate rows: every valid row, or the response rows
  DL_CHECK_HIP(launch_identity_sel(s->seq_len, d.B, d.S, all_idx, all_cnt, st, resp ? s->prompt_len : nullptr));
  DL_CHECK_HIP(launch_row_off_map(all_idx, all_cnt, all_off, d.B, d.S, rm_all, st));
  DL_CHECK_HIP(launch_rope_table(d.S, d.head_dim, d.rope_base, at<float2>(ws, L.rope), st));
  DL_CHECK_HIP(launch_embed(d.dtype, s->tokens, rm_all, model->embed, d.d, x_all, st));

  char* kcache = static_cast<char*>(s->k_cache);
  char* vcache = static_cast<char*>(s->v_cache);
  float* scores = s->scores ? s->scores : at<float>(ws, L.scores);
  float* scores2 = s->scores2 ? s->scores2 : at<float>(ws, L.scores2);
  auto copy_sel = [&](const dl_selection& dst) -> dl_status {
    DL_CHECK_HIP(hipMemcpyAsync(dst.sel_idx, all_idx, sizeof(int32_t) * (size_t)d.B * d.S, hipMemcpyDeviceToDevice,
                                st));
    DL_CHECK_HIP(hipMemcpyAsync(dst.sel_count, all_cnt, sizeof(int32_t) * d.B, hipMemcpyDeviceToDevice, st));
    DL_CHECK_HIP(hipMemcpyAsync(dst.row_off, all_off, sizeof(int32_t) * (d.B + 1), hipMemcpyDeviceToDevice, st));
    return DL_OK;
  };
  if (refresh) {
    // every row through every layer; h_prev <- the layer-s input (h_prev2 <- the layer-s2 input)
    auto norm_of = [&](int l) { return l < d.n_layers ? model->layers[l].attn_norm : model->final_norm; };
    DL_TRY(run_layers(c, model, 0, sl, x_all, rm_all, s->seq_len, kcache, vcache, false, norm_of(sl)));
    if (kv) {
      float* t = at<float>(ws, L.t_rows);
      DL_TRY(scored_kv_rows(c, &model->layers[sl], p->score_tensor, rm_all, t));
      DL_CHECK_HIP(launch_store_rows(d.dtype, t, d.d, rm_all, s->h_prev, st));
    } else {
      DL_CHECK_HIP(launch_store_rows(d.dtype, x_all, d.d, rm_all, s->h_prev, st));
    }
    int l0 = sl;
    if (two) {
      DL_TRY(run_layers(c, model, sl, s2, x_all, rm_all, s->seq_len, kcache, vcache, true, norm_of(s2)));
      DL_CHECK_HIP(launch_store_rows(d.dtype, x_all, d.d, rm_all, s->h_prev2, st));
      l0 = s2;
    }
    if (per_layer) {
      RowMap rm_out;
      float* x_out;
      LayerSel so;
      DL_TRY(per_layer_layers(c, model, s, p, true, LayerSel{all_idx, all_cnt, all_off}, rm_all, x_all, true, rm_all,
                              all_off, x_all, R_all, cand_x_keys, cand_x_keys, &rm_out, &x_out, &so));
      DL_TRY(copy_sel(s->sel_l));
    } else {
      DL_TRY(run_layers(c, model, l0, d.n_layers, x_all, rm_all, s->seq_len, kcache, vcache, true,
                        model->final_norm));
    }
    DL_TRY(copy_sel(s->sel));
    if (two) DL_TRY(copy_sel(s->sel2));
    DL_TRY(lm_block(c, model->final_norm, model->lm_head, x_all, rm_all, s->conf, s->argmax, s->h_final, s->logits,
                    true));
  } else {
    DL_TRY(run_layers(c, model, 0, sl, x_all, rm_all, s->seq_len, kcache, vcache, false,
                      kv ? model->layers[sl].attn_norm : nullptr));
    // score against h_prev and overwrite it with this step's value of the scored tensor
    const float* xs = x_all;
    if (kv) {
      float* t = at<float>(ws, L.t_rows);
      DL_TRY(scored_kv_rows(c, &model->layers[sl], p->score_tensor, rm_all, t));
      xs = t;
    }
    const RowMap rm_sel = rowmap_at(ws, L.map_sel, (int)R_sel, tiles(R_sel));
    // one sequence: the selection's launch writes row_off and the map too
    int32_t* one_off = d.B == 1 ? s->sel.row_off : nullptr;
    const RowMap* one_map = d.B == 1 ? &rm_sel : nullptr;
    if (!resp) {
      DL_CHECK_HIP(launch_score(d.dtype, nullptr, xs, all_off, s->h_prev, s->conf, s->seq_len, d.B, d.S, d.d,
                                p->score, p->alpha, scores, st));
      DL_CHECK_HIP(launch_select(scores, s->seq_len, d.B, d.S, p->mode, p->keep_ratio, p->threshold, s->sel.sel_idx,
                                 s->sel.sel_count, st, nullptr, nullptr, nullptr, one_off, one_map));
    } else {
      DL_CHECK_HIP(launch_fill_scores(scores, -INFINITY, s->seq_len, d.B, d.S, st));
      DL_CHECK_HIP(launch_score(d.dtype, nullptr, xs, nullptr, s->h_prev, s->conf, s->seq_len, d.B, d.S, d.d,
                                p->score, p->alpha, scores, st, &rm_all));
      DL_CHECK_HIP(launch_select(scores, s->seq_len, d.B, d.S, p->mode, p->keep_ratio, p->threshold, s->sel.sel_idx,
                                 s->sel.sel_count, st, all_idx, all_cnt, all_cnt, one_off, one_map));
    }
    if (d.B != 1)
      DL_CHECK_HIP(launch_row_off_map(s->sel.sel_idx, s->sel.sel_count, s->sel.row_off, d.B, d.S, rm_sel, st));
    float* x_sel = at<float>(ws, L.x_sel);
    if (!resp) {
      DL_CHECK_HIP(launch_gather(sizeof(float), x_all, all_off, d.S, d.d, rm_sel, x_sel, st));
    } else {
      DL_CHECK_HIP(launch_inv_rows(rm_all, d.B * d.S, inv, st));
      DL_CHECK_HIP(launch_gather(sizeof(float), x_all, nullptr, d.S, d.d, rm_sel, x_sel, st, inv));
    }
    c.rows_x_keys = sel_x_keys;
    if (per_layer) {
      RowMap rm_out;
      float* x_out;
      LayerSel so;
      DL_TRY(per_layer_layers(c, model, s, p, false, LayerSel{s->sel.sel_idx, s->sel.sel_count, s->sel.row_off},
                              rm_sel, x_sel, false, rm_all, all_off, x_all, R_l, sel_x_keys, l_x_keys, &rm_out,
                              &x_out, &so));
      DL_CHECK_HIP(hipMemcpyAsync(s->sel_l.sel_idx, so.idx, sizeof(int32_t) * (size_t)d.B * d.S,
                                  hipMemcpyDeviceToDevice, st));
      DL_CHECK_HIP(hipMemcpyAsync(s->sel_l.sel_count, so.cnt, sizeof(int32_t) * d.B, hipMemcpyDeviceToDevice, st));
      DL_CHECK_HIP(hipMemcpyAsync(s->sel_l.row_off, so.off, sizeof(int32_t) * (d.B + 1), hipMemcpyDeviceToDevice, st));
      DL_TRY(lm_block(c, model->final_norm, model->lm_head, x_out, rm_out, s->conf, s->argmax, s->h_final, s->logits,
                      true));
    } else if (!two) {
      DL_TRY(run_layers(c, model, sl, d.n_layers, x_sel, rm_sel, s->seq_len, kcache, vcache, false,
                        model->final_norm));
      DL_TRY(lm_block(c, model->final_norm, model->lm_head, x_sel, rm_sel, s->conf, s->argmax, s->h_final, s->logits,
                      sl < d.n_layers));
    } else {
      // layers [s, s2) on sel; second score against h_prev2 (rewritten for sel) and selection among sel
      DL_TRY(run_layers(c, model, sl, s2, x_sel, rm_sel, s->seq_len, kcache, vcache, false, nullptr));
      DL_CHECK_HIP(launch_fill_scores(scores2, -INFINITY, s->seq_len, d.B, d.S, st));
      DL_CHECK_HIP(launch_score(d.dtype, nullptr, x_sel, nullptr, s->h_prev2, s->conf, s->seq_len, d.B, d.S, d.d,
                                p->score, p->alpha, scores2, st, &rm_sel));
      DL_CHECK_HIP(launch_select(scores2, s->seq_len, d.B, d.S, p->mode2, p->keep_ratio2, p->threshold2,
                                 s->sel2.sel_idx, s->sel2.sel_count, st, s->sel.sel_idx, s->sel.sel_count, all_cnt));
      const RowMap rm_sel2 = rowmap_at(ws, L.map_sel2, (int)R_sel2, tiles(R_sel2));
      DL_CHECK_HIP(launch_row_off_map(s->sel2.sel_idx, s->sel2.sel_count, s->sel2.row_off, d.B, d.S, rm_sel2,
                                      st));
      float* x_sel2 = at<float>(ws, L.x_sel2);
      DL_CHECK_HIP(launch_inv_rows(rm_sel, d.B * d.S, inv, st));
      DL_CHECK_HIP(launch_gather(sizeof(float), x_sel, nullptr, d.S, d.d, rm_sel2, x_sel2, st, inv));
      c.rows_x_keys = sel2_x_keys;
      DL_TRY(run_layers(c, model, s2, d.n_layers, x_sel2, rm_sel2, s->seq_len, kcache, vcache, false,
                        model->final_norm));
      DL_TRY(lm_block(c, model->final_norm, model->lm_head, x_sel2, rm_sel2, s->conf, s->argmax, s->h_final,
                      s->logits, s2 < d.n_layers));
    }
  }
  DL_CHECK_HIP(launch_unmask(s->tokens, s->masked, s->conf, s->argmax, s->prompt_len, s->seq_len, d.B, d.S, p->block,
                             p->block_len, p->n_unmask, st));
  return DL_OK;
}

dl_status dl_denoise_step_noalloc(const dl_model* model, dl_state* state, const dl_step_params* params,
                                  void* stream) {
  void* ws = nullptr;
  DL_TRY(scratch_on_current_device(&ws));
  const dl_status st = dl_denoise_step(model, state, params, ws, kScratchBytes, stream);
  if (st == DL_E_WORKSPACE) {
    char detail[sizeof g_err];
    snprintf(detail, sizeof detail, "%s", g_err);
    return fail(DL_E_WORKSPACE, "the no-allocation step's scratch holds %zu bytes (%s)", kScratchBytes, detail);
  }
  return st;
}

}  // extern "C"
