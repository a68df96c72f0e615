// Host-side launchers of libdtsk's kernels (internal; not part of the ABI).
#pragma once

#include "common.h"

namespace dtsk {

// ---- selections and row maps ------------------------------------------------
// Positions [start[b], seq_len[b]) of each sequence (start == nullptr: from 0).
hipError_t launch_identity_sel(const int32_t* seq_len, int B, int S, int32_t* sel_idx, int32_t* sel_count,
                               hipStream_t st, const int32_t* start = nullptr);
// row_off = exclusive prefix of sel_count.
hipError_t launch_row_off(const int32_t* sel_count, int32_t* row_off, int B, hipStream_t st);
// Packed-row maps and attention query tiles of a selection with row_off set.
hipError_t launch_rowmap(const int32_t* sel_idx, const int32_t* sel_count, const int32_t* row_off, int B, int S,
                         const RowMap& rm, hipStream_t st);
// row_off, the row maps and the attention tiles of a selection in one launch
// (launch_row_off followed by launch_rowmap, same outputs).
hipError_t launch_row_off_map(const int32_t* sel_idx, const int32_t* sel_count, int32_t* row_off, int B, int S,
                              const RowMap& rm, hipStream_t st);
// Selection-driven gather / scatter (no row map needed): packed row r of
// sequence b <-> flat row b*S + sel_idx[b*S + r - row_off[b]].
hipError_t launch_gather_sel(size_t elem_bytes, const void* src, int w, const int32_t* sel_idx,
                             const int32_t* row_off, int B, int S, int R_max, void* dst, hipStream_t st);
hipError_t launch_scatter_sel(size_t elem_bytes, const void* rows, int w, const int32_t* sel_idx,
                              const int32_t* row_off, int B, int S, int R_max, void* cache, hipStream_t st);

// ---- scores and selection -----------------------------------------------------
// Score of each valid row.  If x_packed != nullptr, the current input is the
// fp32 packed row x_packed[off_all[b] + i] rounded to the storage type, and
// h_prev is overwritten with it after scoring (one pass); otherwise h_cur is read.
// With a row map, only its packed rows are scored: input x_packed[r], flat row
// rm->row_pos[r] of scores and h_prev.
hipError_t launch_score(dl_dtype dt, const void* h_cur, const float* x_packed, const int32_t* off_all, void* h_prev,
                        const float* conf, const int32_t* seq_len, int B, int S, int d, dl_score_kind kind,
                        float alpha, float* scores, hipStream_t st, const RowMap* rm = nullptr);
// Selection among every valid row, or among the candidate lists (cand_idx,
// cand_cnt: ascending positions per sequence, a selection's layout); top-k
// keeps ceil(keep * k_base[b]) (default base: the candidate count), at most
// the candidate count.  sel_idx must not alias cand_idx.  With B == 1 the
// same launch can also write row_off (if non-null) and the row map rm (if
// non-null; as launch_row_off_map writes it).
hipError_t launch_select(const float* scores, const int32_t* seq_len, int B, int S, dl_select_mode mode, float keep,
                         float threshold, int32_t* sel_idx, int32_t* sel_count, hipStream_t st,
                         const int32_t* cand_idx = nullptr, const int32_t* cand_cnt = nullptr,
                         const int32_t* k_base = nullptr, int32_t* row_off = nullptr, const RowMap* rm = nullptr);
// v at positions [0, seq_len[b]) of a [B, S] array.
hipError_t launch_fill_scores(float* scores, float v, const int32_t* seq_len, int B, int S, hipStream_t st);

// ---- row movement -------------------------------------------------------------
hipError_t launch_embed(dl_dtype dt, const int32_t* tokens, const RowMap& rm, const void* E, int d, float* x,
                        hipStream_t st);
// dst[r] = src[src_row(r)]: src_row = src_inv[row_pos] when src_inv != nullptr
// (rows whose entry is negative are left alone), else off[row_seq] +
// (row_pos - row_seq*S) when src_off != nullptr (packed source), else row_pos
// (padded [B,S,w] source).
hipError_t launch_gather(size_t elem_bytes, const void* src, const int32_t* src_off, int S, int w, const RowMap& rm,
                         void* dst, hipStream_t st, const int32_t* src_inv = nullptr);
// dst[r] = T(src[src_off[b] + position of r]): fp32 rows packed by sequence
// offsets, converted to the storage type, for the packed rows of rm.
hipError_t launch_gather_cvt(dl_dtype dt, const float* src, const int32_t* src_off, int S, int d, const RowMap& rm,
                             void* dst, hipStream_t st);
// dv[r] = V[row_pos[r]] - v_old[r] (storage type, difference in fp32).
hipError_t launch_value_change(dl_dtype dt, const void* V, const void* v_old, const RowMap& rm, int d, void* dv,
                               hipStream_t st);
// inv[p] = the packed row of flat position p in the row map, -1 for positions
// outside it (inv has BS = B*S entries).
hipError_t launch_inv_rows(const RowMap& rm, int BS, int32_t* inv, hipStream_t st);
// cache[row_pos[r]] = rows[r] (same type)
hipError_t launch_scatter(size_t elem_bytes, const void* rows, int w, const RowMap& rm, void* cache, hipStream_t st);
// dst[row_pos[r]] = T(x[r]) for fp32 rows x
hipError_t launch_store_rows(dl_dtype dt, const float* x, int w, const RowMap& rm, void* dst, hipStream_t st);

// ---- normalisation and epilogues ------------------------------------------------
hipError_t launch_rmsnorm(dl_dtype dt, const float* x, const void* g, const RowMap& rm, int d, float eps, void* out,
                          hipStream_t st);
hipError_t launch_rope_table(int S, int head_dim, float base, float2* table, hipStream_t st);
// launch_rmsnorm and launch_rope_table in one launch (the table's blocks after
// the rows').
hipError_t launch_rmsnorm_rope(dl_dtype dt, const float* x, const void* g, const RowMap& rm, int d, float eps,
                               void* out, int S, int head_dim, float base, float2* table, hipStream_t st);
// RoPE in place on fp32 packed rows [R_max, d] of the row map, at each row's position.
hipError_t launch_rope_rows(float* x, const RowMap& rm, int S, int d, int head_dim, const float2* rope,
                            hipStream_t st);
hipError_t launch_epi_qkv(dl_dtype dt, const float* P, int splits, const RowMap& rm, int S, int d, int head_dim,
                          const float2* rope, void* q_out, void* k_cache, void* v_cache, hipStream_t st);
hipError_t launch_epi_residual(const float* P, int splits, const RowMap& rm, int N, float* x, hipStream_t st);
hipError_t launch_epi_swiglu(dl_dtype dt, const float* P, int splits, const RowMap& rm, int F, void* out,
                             hipStream_t st);

// ---- GEMM with fused epilogue -----------------------------------------------------
enum EpiKind { EPI_NONE = 0, EPI_QKV = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_LM = 4 };

// What the last workgroup of a column tile does with the summed tile.  Row m
// of the product is packed row m of the row map (pointers already offset to
// the product's first row).
struct Epilogue {
  int kind;
  float* x;                       // EPI_RESID: x[m][n] += C[m][n] (row stride N)
  void* q_out;                    // EPI_QKV: rotated q rows [M, d]
  void* k_cache;                  // EPI_QKV: this layer's [B*S, d]
  void* v_cache;
  const int32_t* row_pos;         // flat [B*S] row of packed row m
  const int32_t* row_seq;
  int S, d, head_dim;
  const float2* rope;             // (cos, sin) [S, head_dim/2]
  void* act_out;                  // EPI_SWIGLU: silu(gate) * up rows [M, F]
  int F;
  float* lm_part;                 // EPI_LM: float4 (max, sum exp, argmax bits, 0) [M][lm_tiles]
  int lm_tiles;
  float* logits;                  // EPI_LM: optional fp32 logits [B*S, V] at row_pos
  int V;
};

enum GemmKind { GEMM_SIMT = 0, GEMM_LARGE = 1, GEMM_SKINNY = 2 };
struct GemmPlan {
  int kind;
  int splits;  // > 1 only with EPI_NONE: fp32 partials reduced by launch_reduce_rows
  int bn;      // column tile
  int mi;      // skinny: 16-row blocks of A
  int wmode;   // weight-row order: 0 segmented, 1 gate|up interleaved, 2 RoPE pairs,
               // 3 gate|up interleaved over `tiles` ragged column tiles
  int sep_epi; // 1: the product writes fp32 partials and the separate epilogue kernels finish
  int tiles;   // column tiles when they are not N / bn (wmode 3), else 0
  int bm;      // GEMM_LARGE row tile: 256 (8 waves) or 0 for 128
  int nw;      // GEMM_LARGE 128-row tiles: 8 waves, or 0 for the default
};
// The epilogue kind decides the tile the fused epilogue needs; a GEMM_SIMT
// plan leaves the epilogue to the separate kernels below.
GemmPlan plan_gemm(dl_dtype dt, int M, int N, int K, int epi_kind, int head_dim, int F);
// Rows [m_base, m_base + M_max) of A (A points at row m_base); rows at or
// beyond *n_rows are skipped.  With EPI_NONE or a GEMM_SIMT plan, P receives
// [splits][M_max][N] fp32 partials; otherwise the epilogue consumes the tile.
hipError_t launch_gemm(dl_dtype dt, const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows,
                       int m_base, int K, const void* const* Wseg, int n_seg, int N, float* P, const Epilogue& epi,
                       hipStream_t st, int w_layout);
// dst = the DL_WEIGHTS_BLOCKED copy of the row-major [N, K] bf16 matrix src
// (N % 8 == 0, K % 64 == 0).
hipError_t launch_pack_weights(const void* src, void* dst, int N, int K, hipStream_t st);
// x[r] += sum over splits of P[s][r] (in split order); then, if g != nullptr,
// out[r] = T(x[r] / sqrt(mean(x[r]^2) + eps) * g).  Packed rows of the map.
hipError_t launch_reduce_rows(dl_dtype dt, const float* P, int splits, const RowMap& rm, int d, float* x,
                              const void* g, float eps, void* out, hipStream_t st);
// Merge the per-tile LM statistics of rows [m_base, m_base + M_max) into conf / argmax.
hipError_t launch_lm_merge(const float* lm_part, int lm_tiles, const RowMap& rm, int m_base, int M_max, float* conf,
                           int32_t* argmax, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t st);

// ---- attention ---------------------------------------------------------------------
bool attention_supported(dl_dtype dt, int S, int head_dim);
// Key chunks for the matrix-core kernel: enough workgroups to fill the chip,
// at most kAttnMaxSplits, and only when every packed row fits the R_part rows
// of the partial buffers.
constexpr int kAttnMaxSplits = 8;
constexpr int kAttnTargetBlocks = 2048;
int attention_splits(dl_dtype dt, int head_dim, int S, int n_heads, const RowMap& rm, int R_part);
// o_part [kAttnMaxSplits][R_part][d] fp32, ml_part [kAttnMaxSplits][R_part][n_heads].
// With ctx_out, the normalised context goes there in fp32 instead of `out`, at
// row ctx_off[b] + position (the packed row of an all-rows map), and each
// (row, head)'s log normaliser to lse_out[row_pos * n_heads + head].  Without
// ctx_out, lse_rows (if set) takes that normaliser at the packed row,
// lse_rows[row * n_heads + head], beside `out`.  n_seq: the sequences of the
// caches when known (1 spares the kernels a dependent load), else 0.
hipError_t launch_attention(dl_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_len, const RowMap& rm, int S, int n_heads, int head_dim, int splits,
                            float* o_part, float2* ml_part, int R_part, void* out, hipStream_t st,
                            float* ctx_out = nullptr, const int32_t* ctx_off = nullptr, float* lse_out = nullptr,
                            float* lse_rows = nullptr, int n_seq = 0);
// Approximate context of every row of rm_all that is not active (inv < 0):
// ctx_new[r] = ctx_cache[pos] + sum_j exp(q_cache[pos].k_j / sqrt(dh) - lse[pos]) dv_j
// per head, j over the active rows of the row's sequence (k_act / dv_act packed
// by key_off, key_cnt of them).
hipError_t launch_attention_approx(dl_dtype dt, const void* q_cache, const void* k_act, const void* dv_act,
                                   const int32_t* key_off, const int32_t* key_cnt, const float* lse,
                                   const int32_t* inv, const float* ctx_cache, float* ctx_new, const RowMap& rm_all,
                                   int S, int n_heads, int head_dim, hipStream_t st);

// ---- LM head reduction and unmasking -------------------------------------------------
// Packed rows [m_base, m_base + M_max) of the row map; P is [splits][M_max][V].
hipError_t launch_lm_reduce(const float* P, int splits, const RowMap& rm, int m_base, int M_max, int V, float* conf,
                            int32_t* argmax, float* logits_out, hipStream_t st);
hipError_t launch_unmask(int32_t* tokens, uint8_t* masked, const float* conf, const int32_t* argmax,
                         const int32_t* prompt_len, const int32_t* seq_len, int B, int S, int block, int block_len,
                         int n_unmask, hipStream_t st);

}  // namespace dtsk
