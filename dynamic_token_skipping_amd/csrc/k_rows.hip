// Row-level kernels: selections and row maps, importance score, top-k /
// threshold selection, embedding, gathers and scatters, RMSNorm, GEMM
// epilogues (RoPE + K/V cache scatter, residual add, SwiGLU), LM-head
// confidence reduction and block unmasking.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "launch.h"

namespace dtsk {

namespace {

constexpr int kRowThreads = 256;

// ---------------------------------------------------------------------------
// selections
// ---------------------------------------------------------------------------
// positions [start[b], seq_len[b]) of each sequence (start = 0 without `start`)
__global__ void k_identity_sel(const int32_t* __restrict__ seq_len, const int32_t* __restrict__ start, int S,
                               int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count) {
  const int b = blockIdx.y;
  const int n = seq_len[b];
  const int p0 = start ? min(max(start[b], 0), n) : 0;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < S; j += gridDim.x * blockDim.x)
    sel_idx[(size_t)b * S + j] = j < n - p0 ? p0 + j : 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) sel_count[b] = n - p0;
}

// One block: exclusive prefix of sel_count (B <= 1024).
__global__ void k_row_off(const int32_t* __restrict__ sel_count, int32_t* __restrict__ row_off, int B) {
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int b = 0; b < B; ++b) {
      row_off[b] = acc;
      acc += sel_count[b];
    }
    row_off[B] = acc;
  }
}

constexpr int kMaxMapSeqs = 1024;   // sequences the one-launch row map holds in LDS

// One block: the row count and the attention query tiles (tq rows each,
// never crossing a sequence), from an existing row_off.
__global__ void k_tiles(const int32_t* __restrict__ sel_count, const int32_t* __restrict__ row_off, int B,
                        int32_t* __restrict__ n_rows, int32_t* __restrict__ tile_row0,
                        int32_t* __restrict__ tile_rows, int T_max, int tq) {
  __shared__ int32_t toff[1025];
  const int t = threadIdx.x;
  if (t == 0) {
    int tacc = 0;
    for (int b = 0; b < B; ++b) {
      toff[b] = tacc;
      tacc += (sel_count[b] + tq - 1) / tq;
    }
    toff[B] = tacc;
    *n_rows = row_off[B];
  }
  __syncthreads();
  for (int s = t; s < T_max; s += blockDim.x) {
    int r0 = 0, rows = 0;
    if (s < toff[B]) {
      int lo = 0, hi = B - 1;  // last b with toff[b] <= s
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (toff[mid] <= s) lo = mid; else hi = mid - 1;
      }
      const int b = lo;
      const int j0 = (s - toff[b]) * tq;
      r0 = row_off[b] + j0;
      rows = min(tq, sel_count[b] - j0);
    }
    tile_row0[s] = r0;
    tile_rows[s] = rows;
  }
}

__global__ void k_rowmap(const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ row_off, int B, int S,
                         int R_max, int32_t* __restrict__ row_pos, int32_t* __restrict__ row_seq) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R_max) return;
  const int n = row_off[B];
  if (r >= n) {
    row_pos[r] = -1;
    row_seq[r] = 0;
    return;
  }
  int lo = 0, hi = B - 1;  // last b with row_off[b] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (row_off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  row_pos[r] = b * S + sel_idx[(size_t)b * S + (r - row_off[b])];
  row_seq[r] = b;
}

// row_off, the row map and the attention tiles of a selection in one launch:
// every block forms row_off in LDS from sel_count; the last block writes it
// out with n_rows and the tiles, the others fill row_pos / row_seq for 256
// packed rows each.  Same outputs as k_row_off, k_tiles and k_rowmap.
__global__ __launch_bounds__(256) void k_rowmap_all(const int32_t* __restrict__ sel_idx,
                                                    const int32_t* __restrict__ sel_count, int B, int S, int R_max,
                                                    int32_t* __restrict__ row_off, int32_t* __restrict__ n_rows,
                                                    int32_t* __restrict__ row_pos, int32_t* __restrict__ row_seq,
                                                    int32_t* __restrict__ tile_row0, int32_t* __restrict__ tile_rows,
                                                    int T_max, int tq) {
  __shared__ int32_t roff[kMaxMapSeqs + 1], toff[kMaxMapSeqs + 1];
  const int t = threadIdx.x;
  const bool last = blockIdx.x == gridDim.x - 1;
  if (t == 0) {
    int acc = 0, tacc = 0;
    for (int b = 0; b < B; ++b) {
      roff[b] = acc;
      toff[b] = tacc;
      acc += sel_count[b];
      tacc += (sel_count[b] + tq - 1) / tq;
    }
    roff[B] = acc;
    toff[B] = tacc;
  }
  __syncthreads();
  if (!last) {
    const int r = blockIdx.x * 256 + t;
    if (r >= R_max) return;
    if (r >= roff[B]) {
      row_pos[r] = -1;
      row_seq[r] = 0;
      return;
    }
    int lo = 0, hi = B - 1;  // last b with roff[b] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (roff[mid] <= r) lo = mid; else hi = mid - 1;
    }
    row_pos[r] = lo * S + sel_idx[(size_t)lo * S + (r - roff[lo])];
    row_seq[r] = lo;
    return;
  }
  for (int b = t; b <= B; b += 256) row_off[b] = roff[b];
  if (t == 0) *n_rows = roff[B];
  for (int s = t; s < T_max; s += 256) {
    int r0 = 0, rows = 0;
    if (s < toff[B]) {
      int lo = 0, hi = B - 1;  // last b with toff[b] <= s
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (toff[mid] <= s) lo = mid; else hi = mid - 1;
      }
      const int j0 = (s - toff[lo]) * tq;
      r0 = roff[lo] + j0;
      rows = min(tq, sel_count[lo] - j0);
    }
    tile_row0[s] = r0;
    tile_rows[s] = rows;
  }
}

// ---------------------------------------------------------------------------
// importance score (one wave per row)
// ---------------------------------------------------------------------------
// Which row a scoring wave takes: with a row map (rm_pos != nullptr) wave w of
// block x takes packed row r = 4x + w, i.e. flat row rm_pos[r] and input row
// x_packed[r]; otherwise position i = 4x + w of sequence blockIdx.y, input row
// x_packed[off_all[b] + i].  Returns false when the wave has no row.
__device__ __forceinline__ bool score_row(const int32_t* __restrict__ rm_pos, const int32_t* __restrict__ rm_n,
                                          const int32_t* __restrict__ off_all, const int32_t* __restrict__ seq_len,
                                          int S, size_t* row, size_t* xrow) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rm_pos) {
    if (w >= *rm_n) return false;
    *row = (size_t)rm_pos[w];
    *xrow = (size_t)w;
    return true;
  }
  const int b = blockIdx.y;
  if (w >= seq_len[b]) return false;
  *row = (size_t)b * S + w;
  *xrow = off_all ? (size_t)(off_all[b] + w) : 0;
  return true;
}

template <typename T, bool kFused>
__global__ __launch_bounds__(256) void k_score(const T* __restrict__ h_cur, const float* __restrict__ x_packed,
                                               const int32_t* __restrict__ off_all,
                                               const int32_t* __restrict__ rm_pos, const int32_t* __restrict__ rm_n,
                                               T* __restrict__ h_prev, const float* __restrict__ conf,
                                               const int32_t* __restrict__ seq_len, int S, int d, int kind,
                                               float alpha, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  size_t row, xrow;
  if (!score_row(rm_pos, rm_n, off_all, seq_len, S, &row, &xrow)) return;
  const T* hp = h_prev + row * d;
  float l1 = 0.f, dd = 0.f, hh = 0.f, xx = 0.f, xh = 0.f;
  if constexpr (kFused) {
    const float* xr = x_packed + xrow * d;
    T* hw = h_prev + row * d;
    for (int c = lane; c < d; c += 64) {
      const T xt = from_f32<T>(xr[c]);
      const float x = to_f32(xt), h = to_f32(hp[c]);
      const float df = x - h;
      l1 += fabsf(df);
      dd += df * df;
      hh += h * h;
      xx += x * x;
      xh += x * h;
      hw[c] = xt;  // each element is read before this lane overwrites it
    }
  } else {
    const T* xc = h_cur + row * d;
    for (int c = lane; c < d; c += 64) {
      const float x = to_f32(xc[c]), h = to_f32(hp[c]);
      const float df = x - h;
      l1 += fabsf(df);
      dd += df * df;
      hh += h * h;
      xx += x * x;
      xh += x * h;
    }
  }
  l1 = warp_sum(l1);
  dd = warp_sum(dd);
  hh = warp_sum(hh);
  xx = warp_sum(xx);
  xh = warp_sum(xh);
  if (lane == 0) {
    const float c = conf[row];
    float s;
    if (kind == DL_SCORE_ESDLLM) {
      s = alpha * c + (1.f - alpha) * (l1 / fmaxf(sqrtf((float)d) * sqrtf(hh), FLT_MIN));
    } else if (kind == DL_SCORE_RELL2_INVCONF) {
      s = sqrtf(dd) / fmaxf(sqrtf(hh), FLT_MIN) + (1.f - c);
    } else {
      s = 1.f - xh / fmaxf(sqrtf(xx) * sqrtf(hh), FLT_MIN);
    }
    scores[row] = s;
  }
}

// score_row for one workgroup per row: row blockIdx.x of the map, or
// position blockIdx.x of sequence blockIdx.y.
__device__ __forceinline__ bool score_row_wg(const int32_t* __restrict__ rm_pos, const int32_t* __restrict__ rm_n,
                                             const int32_t* __restrict__ off_all,
                                             const int32_t* __restrict__ seq_len, int S, size_t* row,
                                             size_t* xrow) {
  const int w = blockIdx.x;
  if (rm_pos) {
    if (w >= *rm_n) return false;
    *row = (size_t)rm_pos[w];
    *xrow = (size_t)w;
    return true;
  }
  const int b = blockIdx.y;
  if (w >= seq_len[b]) return false;
  *row = (size_t)b * S + w;
  *xrow = off_all ? (size_t)(off_all[b] + w) : 0;
  return true;
}

// bf16 storage, d a multiple of 512: one 256-thread workgroup per row (a
// 512-row step fills 512 workgroups, two per CU), thread t owning 8
// consecutive columns of every 2048-column slice.  kFused: X comes from the
// packed fp32 rows, rounded to bf16, and replaces H_prev in the same pass
// (the slices are taken four at a time: every load of a group is issued
// before any of the group's H_prev stores); otherwise X is the bf16 tensor
// h_cur and nothing is written but the score.  Each thread's sums, then the
// four waves' sums added in wave order through LDS.  Same sums as k_score in a
// different summation order.
template <bool kFused>
__global__ __launch_bounds__(256) void k_score_bf16x8(const float* __restrict__ x_packed,
                                                      const uint16_t* __restrict__ h_cur,
                                                      const int32_t* __restrict__ off_all,
                                                      const int32_t* __restrict__ rm_pos,
                                                      const int32_t* __restrict__ rm_n, bf16_t* __restrict__ h_prev,
                                                      const float* __restrict__ conf,
                                                      const int32_t* __restrict__ seq_len, int S, int d, int kind,
                                                      float alpha, float* __restrict__ scores) {
  constexpr int G = 4;                                // slices per load group
  __shared__ float red[4][5];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  size_t row, xrow;
  if (!score_row_wg(rm_pos, rm_n, off_all, seq_len, S, &row, &xrow)) return;   // uniform over the workgroup
  uint16_t* hp = reinterpret_cast<uint16_t*>(h_prev) + row * d;
  const float* xr = kFused ? x_packed + xrow * d : nullptr;
  const uint16_t* xc = kFused ? nullptr : h_cur + row * d;
  float l1 = 0.f, dd = 0.f, hh = 0.f, xx = 0.f, xh = 0.f;
  const int n_slices = (d + 2047) / 2048;
  for (int s0 = 0; s0 < n_slices; s0 += G) {
    float4 xa[G], xb[G];
    uint4 hv[G], xv[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int c = (s0 + gi) * 2048 + t * 8;
      if (s0 + gi < n_slices && c < d) {
        if constexpr (kFused) {
          xa[gi] = *reinterpret_cast<const float4*>(xr + c);
          xb[gi] = *reinterpret_cast<const float4*>(xr + c + 4);
        } else {
          xv[gi] = *reinterpret_cast<const uint4*>(xc + c);
        }
        hv[gi] = *reinterpret_cast<const uint4*>(hp + c);
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int c = (s0 + gi) * 2048 + t * 8;
      if (!kFused && s0 + gi < n_slices && c < d) {
        const uint32_t xw[4] = {xv[gi].x, xv[gi].y, xv[gi].z, xv[gi].w};
        const uint32_t hw[4] = {hv[gi].x, hv[gi].y, hv[gi].z, hv[gi].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xf[2] = {__uint_as_float(xw[e] << 16), __uint_as_float(xw[e] & 0xffff0000u)};
          const float hf[2] = {__uint_as_float(hw[e] << 16), __uint_as_float(hw[e] & 0xffff0000u)};
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float df = xf[q] - hf[q];
            l1 += fabsf(df);
            dd += df * df;
            hh += hf[q] * hf[q];
            xx += xf[q] * xf[q];
            xh += xf[q] * hf[q];
          }
        }
      }
      if (kFused && s0 + gi < n_slices && c < d) {
        const float xs[8] = {xa[gi].x, xa[gi].y, xa[gi].z, xa[gi].w, xb[gi].x, xb[gi].y, xb[gi].z, xb[gi].w};
        const uint32_t hw[4] = {hv[gi].x, hv[gi].y, hv[gi].z, hv[gi].w};
        uint32_t ow[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16_t x0 = from_f32<bf16_t>(xs[2 * e]), x1 = from_f32<bf16_t>(xs[2 * e + 1]);
          const float xf[2] = {to_f32(x0), to_f32(x1)};
          const float hf[2] = {__uint_as_float(hw[e] << 16), __uint_as_float(hw[e] & 0xffff0000u)};
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float df = xf[q] - hf[q];
            l1 += fabsf(df);
            dd += df * df;
            hh += hf[q] * hf[q];
            xx += xf[q] * xf[q];
            xh += xf[q] * hf[q];
          }
          ow[e] = (uint32_t)x0.u | ((uint32_t)x1.u << 16);
        }
        *reinterpret_cast<uint4*>(hp + c) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
  }
  l1 = warp_sum(l1);
  dd = warp_sum(dd);
  hh = warp_sum(hh);
  xx = warp_sum(xx);
  xh = warp_sum(xh);
  if (lane == 0) {
    red[w][0] = l1;
    red[w][1] = dd;
    red[w][2] = hh;
    red[w][3] = xx;
    red[w][4] = xh;
  }
  __syncthreads();
  if (t == 0) {
    l1 = dd = hh = xx = xh = 0.f;
    for (int i = 0; i < 4; ++i) {
      l1 += red[i][0];
      dd += red[i][1];
      hh += red[i][2];
      xx += red[i][3];
      xh += red[i][4];
    }
    const float c = conf[row];
    float s;
    if (kind == DL_SCORE_ESDLLM) {
      s = alpha * c + (1.f - alpha) * (l1 / fmaxf(sqrtf((float)d) * sqrtf(hh), FLT_MIN));
    } else if (kind == DL_SCORE_RELL2_INVCONF) {
      s = sqrtf(dd) / fmaxf(sqrtf(hh), FLT_MIN) + (1.f - c);
    } else {
      s = 1.f - xh / fmaxf(sqrtf(xx) * sqrtf(hh), FLT_MIN);
    }
    scores[row] = s;
  }
}

// ---------------------------------------------------------------------------
// top-k / threshold selection: one 1024-thread block per sequence
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  if (isnan(f)) return 0u;           // NaN ranks last
  if (f == 0.f) f = 0.f;             // -0 and +0 compare equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 1024;

// Exclusive block scan of one int per thread (fixed order).
constexpr int kSelRegs = 8;   // candidates per thread held in registers by k_select

__device__ __forceinline__ int block_excl_scan(int v, int* buf, int* total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) buf[w] = incl;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int i = 0; i < kSelThreads / 64; ++i) {
      const int x = buf[i];
      buf[i] = acc;
      acc += x;
    }
    buf[kSelThreads / 64] = acc;
  }
  __syncthreads();
  *total = buf[kSelThreads / 64];
  return buf[w] + incl - v;
}

// With one sequence, the selection's row offsets and row map can come out of
// the same launch (what k_rowmap_all writes for B = 1): row_off null = none;
// row_pos null = row_off only.
struct SelMap {
  int32_t* row_off;
  int32_t* n_rows;
  int32_t* row_pos;
  int32_t* row_seq;
  int32_t* tile_row0;
  int32_t* tile_rows;
  int R_max, T_max, tq;
};

// Row offsets and the map's rows from tot and tiles, by the block of a
// one-sequence selection (the kept rows' own entries are written as they are
// found).
__device__ void sel_map_finish(const SelMap& m, int tot) {
  const int t = threadIdx.x;
  if (t == 0) {
    m.row_off[0] = 0;
    m.row_off[1] = tot;
  }
  if (!m.row_pos) return;
  if (t == 0) *m.n_rows = tot;
  for (int r = tot + t; r < m.R_max; r += kSelThreads) {
    m.row_pos[r] = -1;
    m.row_seq[r] = 0;
  }
  for (int s = t; s < m.T_max; s += kSelThreads) {
    const int j0 = s * m.tq;
    m.tile_row0[s] = j0 < tot ? j0 : 0;
    m.tile_rows[s] = j0 < tot ? min(m.tq, tot - j0) : 0;
  }
}

// Candidates of sequence b: positions 0..seq_len[b]-1, or with a candidate
// list the cand_cnt[b] ascending positions cand_idx[b*S ...].  Top-k keeps
// k = ceil(keep * base) of them, clamped to [1, base] and to the candidate
// count, where base = k_base[b] (default: the candidate count).
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ seq_len, int S, int mode,
                                                        float keep, float threshold,
                                                        const int32_t* __restrict__ cand_idx,
                                                        const int32_t* __restrict__ cand_cnt,
                                                        const int32_t* __restrict__ k_base,
                                                        int32_t* __restrict__ sel_idx,
                                                        int32_t* __restrict__ sel_count, SelMap map) {
  __shared__ int hist[256];
  __shared__ int scan_buf[kSelThreads / 64 + 1];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int b = blockIdx.x, t = threadIdx.x;
  const int n = cand_idx ? cand_cnt[b] : seq_len[b];     // candidates
  const float* sc = scores + (size_t)b * S;
  const int32_t* cl = cand_idx ? cand_idx + (size_t)b * S : nullptr;
  auto pos = [&](int j) { return cl ? cl[j] : j; };
  const int chunk = (n + kSelThreads - 1) / kSelThreads;
  const int i0 = min(n, t * chunk), i1 = min(n, i0 + chunk);
  // Each thread's keys stay in registers when they fit (up to kSelRegs per
  // thread, n <= 8192): the radix passes and the output pass then read no
  // memory.  SEL_FOR_KEYS(body) runs body with (i, key) for the thread's
  // candidates i0 .. i1-1 in order.
  const bool in_regs = chunk <= kSelRegs;             // uniform
  uint32_t kr[kSelRegs];
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kSelRegs; ++q) kr[q] = i0 + q < i1 ? score_key(sc[pos(i0 + q)]) : 0u;
  }
#define SEL_FOR_KEYS(...)                                             \
  if (in_regs) {                                                      \
    _Pragma("unroll") for (int q = 0; q < kSelRegs; ++q) {            \
      if (i0 + q < i1) {                                              \
        const int i = i0 + q;                                         \
        const uint32_t key = kr[q];                                   \
        (void)i;                                                      \
        __VA_ARGS__                                                   \
      }                                                               \
    }                                                                 \
  } else {                                                            \
    for (int i = i0; i < i1; ++i) {                                   \
      const uint32_t key = score_key(sc[pos(i)]);                     \
      __VA_ARGS__                                                     \
    }                                                                 \
  }

  uint32_t thr;       // selected: key > thr, plus the first `need_eq` with key == thr
  int need_eq;
  if (mode == DL_SEL_TOPK) {
    int k = 0;
    const int base = k_base ? k_base[b] : n;
    if (base > 0 && n > 0) {
      const double kk = ceil((double)keep * (double)base);
      k = kk < 1.0 ? 1 : (kk > (double)base ? base : (int)kk);
      k = min(k, n);
    }
    if (k == 0) {
      if (t == 0) sel_count[b] = 0;
      if (map.row_off) sel_map_finish(map, 0);
      return;
    }
    // radix select of the k-th largest key, 8 bits at a time from the top
    if (t == 0) {
      s_prefix = 0u;
      s_need = k;
    }
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
      for (int j = t; j < 256; j += kSelThreads) hist[j] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix;
      SEL_FOR_KEYS(if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);)
      __syncthreads();
      if (t < 64) {
        // wave 0 finds the digit holding the need-th largest key: lane l owns
        // digits 4l..4l+3; a suffix scan gives the count of keys above them
        const int need = s_need;
        const int h0 = hist[4 * t], h1 = hist[4 * t + 1], h2 = hist[4 * t + 2], h3 = hist[4 * t + 3];
        const int own = h0 + h1 + h2 + h3;
        int incl = own;                     // keys in lanes >= t
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_down(incl, o, 64);
          if (t + o < 64) incl += u;
        }
        int above = incl - own;             // keys with a digit above 4t + 3
        const int hs[4] = {h3, h2, h1, h0};
        int found = -1, rest = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {       // digits 4t+3 down to 4t
          if (found < 0 && above < need && need <= above + hs[q]) {
            found = 4 * t + 3 - q;
            rest = need - above;
          }
          above += hs[q];
        }
        if (found >= 0) {                   // exactly one lane and digit qualify
          s_prefix = prefix | ((uint32_t)found << shift);
          s_need = rest;
        }
      }
      __syncthreads();
    }
    thr = s_prefix;
    need_eq = s_need;  // how many rows with key == thr are taken (lowest indices)
  } else {
    thr = score_key(threshold);
    need_eq = 0;
    if (isnan(threshold)) thr = 0xffffffffu;
  }
  // Rows with key == thr are taken in index order until need_eq of them are
  // in: the rank of an equal row is the number of equal rows before it.
  const bool topk = mode == DL_SEL_TOPK;
  int n_eq = 0;
  SEL_FOR_KEYS(n_eq += key == thr;)
  int tot;
  const int eq_base = block_excl_scan(n_eq, scan_buf, &tot);
  int n_sel = 0, er = eq_base;
  SEL_FOR_KEYS(if (key > thr) {
    ++n_sel;
  } else if (topk && key == thr) {
    n_sel += er < need_eq;
    ++er;
  })
  int out = block_excl_scan(n_sel, scan_buf, &tot);
  int32_t* dst = sel_idx + (size_t)b * S;
  er = eq_base;
  const bool rows_too = map.row_pos != nullptr;     // one sequence: b = 0, row position = pos
  SEL_FOR_KEYS(bool take = key > thr;
               if (!take && topk && key == thr) take = er++ < need_eq;
               if (take) {
                 if (rows_too) {
                   map.row_pos[out] = pos(i);
                   map.row_seq[out] = 0;
                 }
                 dst[out++] = pos(i);
               })
#undef SEL_FOR_KEYS
  if (t == 0) sel_count[b] = tot;
  if (map.row_off) sel_map_finish(map, tot);
}

// ---------------------------------------------------------------------------
// embeddings, gathers, scatters
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_embed(const int32_t* __restrict__ tokens,
                                                       const int32_t* __restrict__ row_pos,
                                                       const T* __restrict__ E, int d, float* __restrict__ x) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const T* e = E + (size_t)tokens[p] * d;
  float* xr = x + (size_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) xr[c] = to_f32(e[c]);
}

// 16-byte granular copy when the row width allows it, else element-wise.
template <int kBytes>
__global__ __launch_bounds__(kRowThreads) void k_gather(const char* __restrict__ src,
                                                        const int32_t* __restrict__ src_off,
                                                        const int32_t* __restrict__ src_inv, int S, size_t row_bytes,
                                                        const int32_t* __restrict__ row_pos,
                                                        const int32_t* __restrict__ row_seq,
                                                        char* __restrict__ dst) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  size_t srow = (size_t)p;
  if (src_inv) {
    const int q = src_inv[p];
    if (q < 0) return;
    srow = (size_t)q;
  } else if (src_off) {
    const int b = row_seq[r];
    srow = (size_t)src_off[b] + (size_t)(p - b * S);
  }
  const char* s = src + srow * row_bytes;
  char* o = dst + (size_t)r * row_bytes;
  using V = typename std::conditional<kBytes == 16, uint4, uint8_t>::type;
  const size_t n = row_bytes / kBytes;
  for (size_t c = threadIdx.x; c < n; c += blockDim.x) reinterpret_cast<V*>(o)[c] = reinterpret_cast<const V*>(s)[c];
}

template <int kBytes>
__global__ __launch_bounds__(kRowThreads) void k_scatter(const char* __restrict__ rows, size_t row_bytes,
                                                         const int32_t* __restrict__ row_pos,
                                                         char* __restrict__ cache) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const char* s = rows + (size_t)r * row_bytes;
  char* o = cache + (size_t)p * row_bytes;
  using V = typename std::conditional<kBytes == 16, uint4, uint8_t>::type;
  const size_t n = row_bytes / kBytes;
  for (size_t c = threadIdx.x; c < n; c += blockDim.x) reinterpret_cast<V*>(o)[c] = reinterpret_cast<const V*>(s)[c];
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_store_rows(const float* __restrict__ x, int w,
                                                            const int32_t* __restrict__ row_pos,
                                                            T* __restrict__ dst) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const float* s = x + (size_t)r * w;
  T* o = dst + (size_t)p * w;
  for (int c = threadIdx.x; c < w; c += blockDim.x) o[c] = from_f32<T>(s[c]);
}

// Selection-driven row copies (ABI-level gather / scatter).
__device__ __forceinline__ int sel_flat_row(int r, const int32_t* __restrict__ sel_idx,
                                            const int32_t* __restrict__ row_off, int B, int S) {
  if (r >= row_off[B]) return -1;
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (row_off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo * S + sel_idx[(size_t)lo * S + (r - row_off[lo])];
}

template <int kBytes, bool kToCache>
__global__ __launch_bounds__(kRowThreads) void k_copy_sel(const char* __restrict__ src, size_t row_bytes,
                                                          const int32_t* __restrict__ sel_idx,
                                                          const int32_t* __restrict__ row_off, int B, int S,
                                                          char* __restrict__ dst) {
  const int r = blockIdx.x;
  const int p = sel_flat_row(r, sel_idx, row_off, B, S);
  if (p < 0) return;
  const char* s = src + (kToCache ? (size_t)r : (size_t)p) * row_bytes;
  char* o = dst + (kToCache ? (size_t)p : (size_t)r) * row_bytes;
  using V = typename std::conditional<kBytes == 16, uint4, uint8_t>::type;
  const size_t n = row_bytes / kBytes;
  for (size_t c = threadIdx.x; c < n; c += blockDim.x) reinterpret_cast<V*>(o)[c] = reinterpret_cast<const V*>(s)[c];
}

// ---------------------------------------------------------------------------
// RMSNorm: out = T(x / sqrt(mean(x^2) + eps) * g)
// ---------------------------------------------------------------------------

// Split sum + residual + (optional) RMSNorm of the next sub-block, one block
// per packed row: x += sum_s P[s]; out = T(x / sqrt(mean(x^2) + eps) * g).
// 4 consecutive storage-type values <-> float4
template <typename T>
__device__ __forceinline__ float4 load4(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const float4*>(p);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
  }
}
template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = v;
  } else {
    const uint32_t a = (uint32_t)from_f32<T>(v.x).u | ((uint32_t)from_f32<T>(v.y).u << 16);
    const uint32_t b = (uint32_t)from_f32<T>(v.z).u | ((uint32_t)from_f32<T>(v.w).u << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
  }
}

// Row copies four columns at a time (widths a multiple of 4, so every row
// start is 8-byte aligned in bf16 and 16-byte aligned in fp32): the embedding
// lookup and the fp32 -> storage-type row store.  Same conversions as the
// element-wise kernels.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_embed4(const int32_t* __restrict__ tokens,
                                                        const int32_t* __restrict__ row_pos,
                                                        const T* __restrict__ E, int d, float* __restrict__ x) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const T* e = E + (size_t)tokens[p] * d;
  float* xr = x + (size_t)r * d;
#pragma unroll 4
  for (int c = threadIdx.x * 4; c < d; c += kRowThreads * 4) *reinterpret_cast<float4*>(xr + c) = load4(e + c);
}
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_store_rows4(const float* __restrict__ x, int w,
                                                             const int32_t* __restrict__ row_pos,
                                                             T* __restrict__ dst) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const float* s = x + (size_t)r * w;
  T* o = dst + (size_t)p * w;
#pragma unroll 4
  for (int c = threadIdx.x * 4; c < w; c += kRowThreads * 4) store4(o + c, *reinterpret_cast<const float4*>(s + c));
}

// threads of the row reduction at d = 4096 (512: two float4 per thread; 256
// and 1024 measured 0.4% slower per decode step)
#ifndef DTSK_RED_THREADS
#define DTSK_RED_THREADS 512
#endif
constexpr int kRedSplits = 8;   // partials loaded together (more are added in a second loop)

// RoPE table entry idx of S * half: (cos, sin) of pos * base^(-2j/dh),
// pos = idx / half, j = idx % half, computed in double.
__device__ __forceinline__ void rope_entry(int idx, int half, int head_dim, double base, float2* __restrict__ tab) {
  const int pos = idx / half, j = idx % half;
  const double inv = pow(base, -2.0 * (double)j / (double)head_dim);
  double sn, cs;
  sincos((double)pos * inv, &sn, &cs);
  tab[idx] = make_float2((float)cs, (float)sn);
}

// Optional work of a row-reduction launch: the RoPE table, in the blocks past
// the rows (block M_max + i fills entries i * blockDim .. + blockDim), so that
// a call that needs both pays one launch.
struct RopeJob {
  float2* tab;      // nullptr: no table
  int n;            // entries (S * half)
  int half;
  int head_dim;
  double base;
};
__device__ __forceinline__ void rope_block(const RopeJob& rj, int blk) {
  const int idx = blk * (int)blockDim.x + (int)threadIdx.x;
  if (rj.tab && idx < rj.n) rope_entry(idx, rj.half, rj.head_dim, rj.base, rj.tab);
}

template <typename T, int kChunks, int NT = kRowThreads>
__global__ __launch_bounds__(NT) void k_reduce_rows(const float* __restrict__ P, int splits, int M_max,
                                                    const int32_t* __restrict__ n_rows, int d, float* __restrict__ x,
                                                    const T* __restrict__ g, float eps, T* __restrict__ out,
                                                    RopeJob rj) {
  // d == kChunks * 4 * NT: every thread owns kChunks float4 of the
  // row; its row, partial and gain loads are all issued before the first is
  // used, and the partials are added in split order
  __shared__ float red[16];
  const int r = blockIdx.x;
  if (r >= M_max) {
    rope_block(rj, r - M_max);
    return;
  }
  // rows r < M_max are in every buffer: their loads go out before the row
  // count arrives, which then decides whether anything is stored
  const size_t sstride = (size_t)M_max * d;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)r * d);
  const float4* pr = reinterpret_cast<const float4*>(P + (size_t)r * d);
  float4 v[kChunks], ps[kRedSplits][kChunks], gv[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) v[c] = xr[threadIdx.x + c * NT];
#pragma unroll
  for (int s = 0; s < kRedSplits; ++s)
    if (s < splits)
#pragma unroll
      for (int c = 0; c < kChunks; ++c) ps[s][c] = pr[s * (sstride / 4) + threadIdx.x + c * NT];
  if (g)
#pragma unroll
    for (int c = 0; c < kChunks; ++c) gv[c] = load4(g + (threadIdx.x + c * NT) * 4);
  if (r >= *n_rows) return;                          // uniform over the workgroup
  auto add = [&](float4& a, const float4& b) {
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  };
#pragma unroll
  for (int s = 0; s < kRedSplits; ++s)
    if (s < splits)
#pragma unroll
      for (int c = 0; c < kChunks; ++c) add(v[c], ps[s][c]);
  for (int s = kRedSplits; s < splits; ++s)
#pragma unroll
    for (int c = 0; c < kChunks; ++c) add(v[c], pr[s * (sstride / 4) + threadIdx.x + c * NT]);
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (splits > 0) xr[threadIdx.x + c * NT] = v[c];
    ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
  }
  if (!g) return;
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  T* o = out + (size_t)r * d;
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    store4(o + (threadIdx.x + c * NT) * 4,
           make_float4(v[c].x * inv * gv[c].x, v[c].y * inv * gv[c].y, v[c].z * inv * gv[c].z,
                       v[c].w * inv * gv[c].w));
}

// Any width: the plain loop.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_reduce_rows_any(const float* __restrict__ P, int splits, int M_max,
                                                                 const int32_t* __restrict__ n_rows, int d,
                                                                 float* __restrict__ x, const T* __restrict__ g,
                                                                 float eps, T* __restrict__ out, RopeJob rj) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  if (r >= M_max) {
    rope_block(rj, r - M_max);
    return;
  }
  if (r >= *n_rows) return;
  const size_t sstride = (size_t)M_max * d;
  float* xr = x + (size_t)r * d;
  const float* pr = P + (size_t)r * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float v = xr[c];
    if (splits > 0) {
      float acc = 0.f;
      for (int s = 0; s < splits; ++s) acc += pr[s * sstride + c];
      v += acc;
      xr[c] = v;
    }
    ss += v * v;
  }
  if (!g) return;
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  T* o = out + (size_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) o[c] = from_f32<T>(xr[c] * inv * to_f32(g[c]));
}

// RoPE table: (cos, sin) of pos * base^(-2j/dh), computed in double.
__global__ void k_rope_table(int S, int half, int head_dim, double base, float2* __restrict__ tab) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= S * half) return;
  rope_entry(idx, half, head_dim, base, tab);
}

// q/k/v epilogue: sum the split-K partials, rotate q and k, write q rows and
// scatter k/v into this layer's caches at the rows' positions.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_epi_qkv(const float* __restrict__ P, int splits, int M_max,
                                                         const int32_t* __restrict__ n_rows,
                                                         const int32_t* __restrict__ row_pos,
                                                         const int32_t* __restrict__ row_seq, int S, int d,
                                                         int head_dim, const float2* __restrict__ rope,
                                                         T* __restrict__ q_out, T* __restrict__ k_cache,
                                                         T* __restrict__ v_cache) {
  const int r = blockIdx.x;
  if (r >= *n_rows) return;
  const int p = row_pos[r];
  const int pos = p - row_seq[r] * S;
  const int N = 3 * d;
  const int half = head_dim >> 1;
  const size_t stride = (size_t)M_max * N;
  const float* base = P + (size_t)r * N;
  // q and k: pairs (j, j + half) of each head
  for (int pi = threadIdx.x; pi < d; pi += blockDim.x) {   // d/2 pairs for q, d/2 for k
    const int which = pi / (d >> 1);                        // 0 = q, 1 = k
    const int pr = pi % (d >> 1);
    const int h = pr / half, j = pr % half;
    const int c1 = which * d + h * head_dim + j, c2 = c1 + half;
    float a = 0.f, bb = 0.f;
    for (int s = 0; s < splits; ++s) {
      a += base[s * stride + c1];
      bb += base[s * stride + c2];
    }
    const float2 cs = rope[pos * half + j];
    const float o1 = a * cs.x - bb * cs.y;
    const float o2 = bb * cs.x + a * cs.y;
    const int col = h * head_dim + j;
    if (which == 0) {
      q_out[(size_t)r * d + col] = from_f32<T>(o1);
      q_out[(size_t)r * d + col + half] = from_f32<T>(o2);
    } else {
      k_cache[(size_t)p * d + col] = from_f32<T>(o1);
      k_cache[(size_t)p * d + col + half] = from_f32<T>(o2);
    }
  }
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += base[s * stride + 2 * d + c];
    v_cache[(size_t)p * d + c] = from_f32<T>(v);
  }
}

// The same epilogue with one workgroup per (packed row, segment, head):
// thread j takes the pair (j, j + head_dim/2) of its head (for v, those two
// dims), loads every split's partial before the first add, sums them in split
// order from 0 (the result equals k_epi_qkv's bit for bit) and writes.
constexpr int kEpiMaxSplits = 8;
template <typename T>
__global__ __launch_bounds__(64) void k_epi_qkv_heads(const float* __restrict__ P, int splits, int M_max,
                                                      const int32_t* __restrict__ n_rows,
                                                      const int32_t* __restrict__ row_pos,
                                                      const int32_t* __restrict__ row_seq, int S, int d, int n_heads,
                                                      int head_dim, const float2* __restrict__ rope,
                                                      T* __restrict__ q_out, T* __restrict__ k_cache,
                                                      T* __restrict__ v_cache) {
  const int r = blockIdx.x;
  if (r >= *n_rows) return;
  const int seg = blockIdx.y / n_heads, h = blockIdx.y - seg * n_heads;
  const int half = head_dim >> 1, j = threadIdx.x;
  if (j >= half) return;
  const int p = row_pos[r];
  const size_t stride = (size_t)M_max * 3 * d;
  const float* base = P + (size_t)r * 3 * d + seg * d + h * head_dim + j;
  float v1[kEpiMaxSplits], v2[kEpiMaxSplits];
#pragma unroll
  for (int s = 0; s < kEpiMaxSplits; ++s)
    if (s < splits) {
      v1[s] = base[s * stride];
      v2[s] = base[s * stride + half];
    }
  float a = 0.f, bb = 0.f;
#pragma unroll
  for (int s = 0; s < kEpiMaxSplits; ++s)
    if (s < splits) {
      a += v1[s];
      bb += v2[s];
    }
  const size_t col = (size_t)h * head_dim + j;
  if (seg == 2) {
    v_cache[(size_t)p * d + col] = from_f32<T>(a);
    v_cache[(size_t)p * d + col + half] = from_f32<T>(bb);
    return;
  }
  const int pos = p - row_seq[r] * S;
  const float2 cs = rope[pos * half + j];
  const float o1 = a * cs.x - bb * cs.y;
  const float o2 = bb * cs.x + a * cs.y;
  T* dst = seg == 0 ? q_out + (size_t)r * d : k_cache + (size_t)p * d;
  dst[col] = from_f32<T>(o1);
  dst[col + half] = from_f32<T>(o2);
}

// The same epilogue with four RoPE pairs per thread (16-byte partial loads):
// one workgroup per (packed row, q|k|v segment); thread t owns dims
// [c, c + 4) and [half + c, half + c + 4) of head t / (half / 4), with
// c = 4 (t % (half / 4)).  Same sums in the same order as k_epi_qkv_heads.
template <typename T>
__global__ __launch_bounds__(1024) void k_epi_qkv_rows4(const float* __restrict__ P, int splits, int M_max,
                                                        const int32_t* __restrict__ n_rows,
                                                        const int32_t* __restrict__ row_pos,
                                                        const int32_t* __restrict__ row_seq, int S, int d,
                                                        int head_dim, const float2* __restrict__ rope,
                                                        T* __restrict__ q_out, T* __restrict__ k_cache,
                                                        T* __restrict__ v_cache) {
  const int r = blockIdx.x;
  const int seg = blockIdx.y, t = threadIdx.x;
  const int half = head_dim >> 1, tph = half >> 2;   // threads per head
  if (t >= d >> 3) return;                           // d / 8 = heads x threads per head
  const int h = t / tph, c = (t - h * tph) * 4;
  const size_t stride = (size_t)M_max * 3 * d;
  const float* base = P + (size_t)r * 3 * d + (size_t)seg * d + (size_t)h * head_dim + c;
  float4 v1[kEpiMaxSplits], v2[kEpiMaxSplits];
#pragma unroll
  for (int s = 0; s < kEpiMaxSplits; ++s)
    if (s < splits) {
      v1[s] = *reinterpret_cast<const float4*>(base + s * stride);
      v2[s] = *reinterpret_cast<const float4*>(base + s * stride + half);
    }
  // rows r < M_max are in the partials and the row map: their loads go out
  // before the row count arrives, which then decides whether anything is stored
  const int p = row_pos[r], sq = row_seq[r];
  if (r >= *n_rows) return;                          // uniform over the workgroup
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
#pragma unroll
  for (int s = 0; s < kEpiMaxSplits; ++s)
    if (s < splits) {
      a.x += v1[s].x; a.y += v1[s].y; a.z += v1[s].z; a.w += v1[s].w;
      b.x += v2[s].x; b.y += v2[s].y; b.z += v2[s].z; b.w += v2[s].w;
    }
  const size_t col = (size_t)h * head_dim + c;
  if (seg == 2) {
    store4(v_cache + (size_t)p * d + col, a);
    store4(v_cache + (size_t)p * d + col + half, b);
    return;
  }
  const int pos = p - sq * S;
  const float4 c01 = *reinterpret_cast<const float4*>(rope + (size_t)pos * half + c);       // (cos, sin) of c, c + 1
  const float4 c23 = *reinterpret_cast<const float4*>(rope + (size_t)pos * half + c + 2);   // of c + 2, c + 3
  const float4 o1 = make_float4(a.x * c01.x - b.x * c01.y, a.y * c01.z - b.y * c01.w, a.z * c23.x - b.z * c23.y,
                                a.w * c23.z - b.w * c23.w);
  const float4 o2 = make_float4(b.x * c01.x + a.x * c01.y, b.y * c01.z + a.y * c01.w, b.z * c23.x + a.z * c23.y,
                                b.w * c23.z + a.w * c23.w);
  T* dst = seg == 0 ? q_out + (size_t)r * d : k_cache + (size_t)p * d;
  store4(dst + col, o1);
  store4(dst + col + half, o2);
}

__global__ __launch_bounds__(kRowThreads) void k_epi_residual(const float* __restrict__ P, int splits, int M_max,
                                                              const int32_t* __restrict__ n_rows, int N,
                                                              float* __restrict__ x) {
  const int r = blockIdx.x;
  if (r >= *n_rows) return;
  const size_t stride = (size_t)M_max * N;
  const float* base = P + (size_t)r * N;
  float* xr = x + (size_t)r * N;
  for (int c = threadIdx.x; c < N; c += blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += base[s * stride + c];
    xr[c] += v;
  }
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_epi_swiglu(const float* __restrict__ P, int splits, int M_max,
                                                            const int32_t* __restrict__ n_rows, int F,
                                                            T* __restrict__ out) {
  const int r = blockIdx.x;
  if (r >= *n_rows) return;
  const int N = 2 * F;
  const size_t stride = (size_t)M_max * N;
  const float* base = P + (size_t)r * N;
  for (int c = threadIdx.x; c < F; c += blockDim.x) {
    float g = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
      g += base[s * stride + c];
      u += base[s * stride + F + c];
    }
    const float a = g / (1.f + expf(-g)) * u;
    out[(size_t)r * F + c] = from_f32<T>(a);
  }
}

// The same with four columns per thread: 16-byte partial loads, all of them
// issued before the row count arrives (rows r < M_max are in the partials);
// the same sums in the same order.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_epi_swiglu4(const float* __restrict__ P, int splits, int M_max,
                                                             const int32_t* __restrict__ n_rows, int F,
                                                             T* __restrict__ out) {
  const int r = blockIdx.x, c = (blockIdx.y * kRowThreads + threadIdx.x) * 4;
  if (c >= F) return;
  const int N = 2 * F;
  const size_t stride = (size_t)M_max * N;
  const float* base = P + (size_t)r * N + c;
  float4 gv[kEpiMaxSplits], uv[kEpiMaxSplits];
#pragma unroll
  for (int s = 0; s < kEpiMaxSplits; ++s)
    if (s < splits) {
      gv[s] = *reinterpret_cast<const float4*>(base + s * stride);
      uv[s] = *reinterpret_cast<const float4*>(base + s * stride + F);
    }
  if (r >= *n_rows) return;
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
#pragma unroll
  for (int s = 0; s < kEpiMaxSplits; ++s)
    if (s < splits) {
      g.x += gv[s].x; g.y += gv[s].y; g.z += gv[s].z; g.w += gv[s].w;
      u.x += uv[s].x; u.y += uv[s].y; u.z += uv[s].z; u.w += uv[s].w;
    }
  store4(out + (size_t)r * F + c,
         make_float4(g.x / (1.f + expf(-g.x)) * u.x, g.y / (1.f + expf(-g.y)) * u.y,
                     g.z / (1.f + expf(-g.z)) * u.z, g.w / (1.f + expf(-g.w)) * u.w));
}

// ---------------------------------------------------------------------------
// LM head: per row, max / argmax (lowest id) / sum exp over the vocabulary
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRowThreads) void k_lm_reduce(const float* __restrict__ P, int splits, int M_max,
                                                           const int32_t* __restrict__ n_rows, int m_base,
                                                           const int32_t* __restrict__ row_pos, int V,
                                                           float* __restrict__ conf, int32_t* __restrict__ argmax,
                                                           float* __restrict__ logits_out) {
  __shared__ float sm[kRowThreads / 64], ss[kRowThreads / 64];
  __shared__ int si[kRowThreads / 64];
  const int r = blockIdx.x;
  if (m_base + r >= *n_rows) return;
  const int p = row_pos[m_base + r];
  const size_t stride = (size_t)M_max * V;
  const float* base = P + (size_t)r * V;
  float m = -INFINITY, sum = 0.f;
  int am = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float l = 0.f;
    for (int s = 0; s < splits; ++s) l += base[s * stride + v];
    if (logits_out) logits_out[(size_t)p * V + v] = l;
    if (l > m) {
      sum = sum * expf(m - l) + 1.f;
      m = l;
      am = v;
    } else {
      sum += expf(l - m);
    }
  }
  // combine within the wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(sum, o, 64);
    const int a2 = __shfl_xor(am, o, 64);
    const float mn = fmaxf(m, m2);
    const float sn = (m == -INFINITY ? 0.f : sum * expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
    const int an = (m2 > m || (m2 == m && a2 < am)) ? a2 : am;
    m = mn;
    sum = sn;
    am = an;
  }
  if (lane == 0) {
    sm[w] = m;
    ss[w] = sum;
    si[w] = am;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], Ssum = ss[0];
    int A = si[0];
    for (int i = 1; i < kRowThreads / 64; ++i) {
      const float mn = fmaxf(M, sm[i]);
      Ssum = Ssum * expf(M - mn) + ss[i] * expf(sm[i] - mn);
      if (sm[i] > M || (sm[i] == M && si[i] < A)) A = si[i];
      M = mn;
    }
    conf[p] = 1.f / Ssum;
    argmax[p] = A;
  }
}

// Merge per-tile (max, sum exp, argmax) statistics of a row, in tile order.
__device__ __forceinline__ void lm_merge(float& m, float& s, int& a, float m2, float s2, int a2) {
  const float mn = fmaxf(m, m2);
  const float sn = (m == -INFINITY ? 0.f : s * expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
  a = (m2 > m || (m2 == m && a2 < a)) ? a2 : a;
  m = mn;
  s = sn;
}

__global__ __launch_bounds__(kRowThreads) void k_lm_merge(const float4* __restrict__ part, int tiles,
                                                          const int32_t* __restrict__ n_rows, int m_base,
                                                          const int32_t* __restrict__ row_pos,
                                                          float* __restrict__ conf, int32_t* __restrict__ argmax) {
  __shared__ float sm[kRowThreads / 64], ss[kRowThreads / 64];
  __shared__ int sa[kRowThreads / 64];
  const int r = blockIdx.x;
  if (m_base + r >= *n_rows) return;
  float m = -INFINITY, s = 0.f;
  int a = 0x7fffffff;
  const float4* pr = part + (size_t)r * tiles;
  for (int i = threadIdx.x; i < tiles; i += blockDim.x) {
    const float4 v = pr[i];
    lm_merge(m, s, a, v.x, v.y, __float_as_int(v.z));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    const int a2 = __shfl_xor(a, o, 64);
    lm_merge(m, s, a, m2, s2, a2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sm[w] = m;
    ss[w] = s;
    sa[w] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], Ssum = ss[0];
    int A = sa[0];
    for (int i = 1; i < kRowThreads / 64; ++i) lm_merge(M, Ssum, A, sm[i], ss[i], sa[i]);
    const int p = row_pos[m_base + r];
    conf[p] = 1.f / Ssum;
    argmax[p] = A;
  }
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// inv[row_pos[r]] = r for the packed rows of a row map
__global__ void k_inv_rows(const int32_t* __restrict__ row_pos, const int32_t* __restrict__ n_rows, int R_max,
                           int32_t* __restrict__ inv) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R_max && r < *n_rows) inv[row_pos[r]] = r;
}

// RoPE applied in place to fp32 packed rows [R, d] of a row map (rotate-half
// pairs (j, j + dh/2) of every head, angle table (cos, sin) [S, dh/2] at the
// row's position in its sequence).
__global__ __launch_bounds__(kRowThreads) void k_rope_rows(float* __restrict__ x, const int32_t* __restrict__ row_pos,
                                                           const int32_t* __restrict__ row_seq, int S, int d,
                                                           int head_dim, const float2* __restrict__ tab) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const int pos = p - row_seq[r] * S;
  const int half = head_dim / 2;
  float* xr = x + (size_t)r * d;
  for (int idx = threadIdx.x; idx < d / 2; idx += blockDim.x) {
    const int h = idx / half, j = idx - h * half;
    float* xh = xr + h * head_dim;
    const float a = xh[j], b = xh[j + half];
    const float2 cs = tab[(size_t)pos * half + j];
    xh[j] = a * cs.x - b * cs.y;
    xh[j + half] = b * cs.x + a * cs.y;
  }
}

// dst[r] = T(src[src_off[b] + position]) for the packed rows of a row map
// (fp32 rows packed by sequence offsets -> storage-type rows).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_gather_cvt(const float* __restrict__ src,
                                                            const int32_t* __restrict__ src_off, int S, int d,
                                                            const int32_t* __restrict__ row_pos,
                                                            const int32_t* __restrict__ row_seq, T* __restrict__ dst) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const int b = row_seq[r];
  const float* sr = src + ((size_t)src_off[b] + (size_t)(p - b * S)) * d;
  T* o = dst + (size_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) o[c] = from_f32<T>(sr[c]);
}

// dv[r] = T(V[row_pos[r]] - v_old[r]): the change of an active row's value
// (the layer's cache already holds the new one), difference taken in fp32.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_value_change(const T* __restrict__ V, const T* __restrict__ v_old,
                                                              const int32_t* __restrict__ row_pos, int d,
                                                              T* __restrict__ dv) {
  const int r = blockIdx.x;
  const int p = row_pos[r];
  if (p < 0) return;
  const T* vn = V + (size_t)p * d;
  const T* vo = v_old + (size_t)r * d;
  T* o = dv + (size_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) o[c] = from_f32<T>(to_f32(vn[c]) - to_f32(vo[c]));
}

// v at the valid positions of every sequence ([B, S] array)
__global__ void k_fill_valid(float* __restrict__ p, float v, const int32_t* __restrict__ seq_len, int S) {
  const int b = blockIdx.y, i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < seq_len[b]) p[(size_t)b * S + i] = v;
}

// ---------------------------------------------------------------------------
// unmask: rank each masked candidate of the block by (conf desc, index asc)
// ---------------------------------------------------------------------------
constexpr int kMaxBlockLen = 1024;
__global__ __launch_bounds__(kMaxBlockLen) void k_unmask(int32_t* __restrict__ tokens, uint8_t* __restrict__ masked,
                                                         const float* __restrict__ conf,
                                                         const int32_t* __restrict__ argmax,
                                                         const int32_t* __restrict__ prompt_len,
                                                         const int32_t* __restrict__ seq_len, int S, int block,
                                                         int block_len, int n_unmask) {
  __shared__ float c[kMaxBlockLen];
  __shared__ uint8_t m[kMaxBlockLen];
  const int b = blockIdx.x, t = threadIdx.x;
  const int lo = prompt_len[b] + block * block_len;
  const int hi = min(lo + block_len, seq_len[b]);
  const int len = max(0, hi - lo);
  const size_t base = (size_t)b * S + lo;
  if (t < len) {
    c[t] = conf[base + t];
    m[t] = masked[base + t];
  }
  __syncthreads();
  if (t < len && m[t]) {
    int rank = 0;
    const float ct = c[t];
    for (int j = 0; j < len; ++j)
      if (m[j] && (c[j] > ct || (c[j] == ct && j < t))) ++rank;
    if (rank < n_unmask) {
      tokens[base + t] = argmax[base + t];
      masked[base + t] = 0;
    }
  }
}

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

// ===========================================================================
// launchers
// ===========================================================================
hipError_t launch_identity_sel(const int32_t* seq_len, int B, int S, int32_t* sel_idx, int32_t* sel_count,
                               hipStream_t st, const int32_t* start) {
  dim3 grid(cdiv(S, 256), B);
  DTSK_LAUNCH(k_identity_sel, grid, dim3(256), 0, st, seq_len, start, S, sel_idx, sel_count);
  return hipGetLastError();
}

hipError_t launch_row_off(const int32_t* sel_count, int32_t* row_off, int B, hipStream_t st) {
  DTSK_LAUNCH(k_row_off, dim3(1), dim3(64), 0, st, sel_count, row_off, B);
  return hipGetLastError();
}

hipError_t launch_rowmap(const int32_t* sel_idx, const int32_t* sel_count, const int32_t* row_off, int B, int S,
                         const RowMap& rm, hipStream_t st) {
  DTSK_LAUNCH(k_tiles, dim3(1), dim3(256), 0, st, sel_count, row_off, B, rm.n_rows, rm.tile_row0,
                     rm.tile_rows, rm.T_max, rm.tq);
  DTSK_LAUNCH(k_rowmap, dim3(cdiv(rm.R_max, 256)), dim3(256), 0, st, sel_idx, row_off, B, S, rm.R_max,
                     rm.row_pos, rm.row_seq);
  return hipGetLastError();
}

hipError_t launch_row_off_map(const int32_t* sel_idx, const int32_t* sel_count, int32_t* row_off, int B, int S,
                              const RowMap& rm, hipStream_t st) {
  if (B > kMaxMapSeqs) {   // more sequences than the one-launch kernel holds in LDS
    hipError_t e = launch_row_off(sel_count, row_off, B, st);
    return e != hipSuccess ? e : launch_rowmap(sel_idx, sel_count, row_off, B, S, rm, st);
  }
  DTSK_LAUNCH(k_rowmap_all, dim3(cdiv(std::max(rm.R_max, 0), 256) + 1), dim3(256), 0, st, sel_idx, sel_count, B, S,
              rm.R_max, row_off, rm.n_rows, rm.row_pos, rm.row_seq, rm.tile_row0, rm.tile_rows, rm.T_max, rm.tq);
  return hipGetLastError();
}

hipError_t launch_gather_sel(size_t elem_bytes, const void* src, int w, const int32_t* sel_idx,
                             const int32_t* row_off, int B, int S, int R_max, void* dst, hipStream_t st) {
  if (R_max <= 0) return hipSuccess;
  const size_t rb = elem_bytes * (size_t)w;
  if (rb % 16 == 0)
    DTSK_LAUNCH((k_copy_sel<16, false>), dim3(R_max), dim3(kRowThreads), 0, st, (const char*)src, rb, sel_idx,
                       row_off, B, S, (char*)dst);
  else
    DTSK_LAUNCH((k_copy_sel<1, false>), dim3(R_max), dim3(kRowThreads), 0, st, (const char*)src, rb, sel_idx,
                       row_off, B, S, (char*)dst);
  return hipGetLastError();
}

hipError_t launch_scatter_sel(size_t elem_bytes, const void* rows, int w, const int32_t* sel_idx,
                              const int32_t* row_off, int B, int S, int R_max, void* cache, hipStream_t st) {
  if (R_max <= 0) return hipSuccess;
  const size_t rb = elem_bytes * (size_t)w;
  if (rb % 16 == 0)
    DTSK_LAUNCH((k_copy_sel<16, true>), dim3(R_max), dim3(kRowThreads), 0, st, (const char*)rows, rb, sel_idx,
                       row_off, B, S, (char*)cache);
  else
    DTSK_LAUNCH((k_copy_sel<1, true>), dim3(R_max), dim3(kRowThreads), 0, st, (const char*)rows, rb, sel_idx,
                       row_off, B, S, (char*)cache);
  return hipGetLastError();
}

hipError_t launch_score(dl_dtype dt, const void* h_cur, const float* x_packed, const int32_t* off_all, void* h_prev,
                        const float* conf, const int32_t* seq_len, int B, int S, int d, dl_score_kind kind,
                        float alpha, float* scores, hipStream_t st, const RowMap* rm) {
  const int32_t* rp = rm ? rm->row_pos : nullptr;
  const int32_t* rn = rm ? rm->n_rows : nullptr;
  if (rm && (!x_packed || rm->R_max <= 0)) return rm->R_max <= 0 ? hipSuccess : hipErrorInvalidValue;
  dim3 grid = rm ? dim3(cdiv(rm->R_max, 4)) : dim3(cdiv(S, 4), B);
  if (dt == DL_F32) {
    if (x_packed)
      DTSK_LAUNCH((k_score<float, true>), grid, dim3(256), 0, st, (const float*)h_cur, x_packed, off_all, rp,
                         rn, (float*)h_prev, conf, seq_len, S, d, (int)kind, alpha, scores);
    else
      DTSK_LAUNCH((k_score<float, false>), grid, dim3(256), 0, st, (const float*)h_cur, x_packed, off_all, rp,
                         rn, (float*)h_prev, conf, seq_len, S, d, (int)kind, alpha, scores);
  } else {
    if (d % 512 == 0) {   // one workgroup per row
      if (x_packed)
        DTSK_LAUNCH(k_score_bf16x8<true>, rm ? dim3(rm->R_max) : dim3(S, B), dim3(256), 0, st, x_packed,
                    (const uint16_t*)nullptr, off_all, rp, rn, (bf16_t*)h_prev, conf, seq_len, S, d, (int)kind, alpha,
                    scores);
      else
        DTSK_LAUNCH(k_score_bf16x8<false>, rm ? dim3(rm->R_max) : dim3(S, B), dim3(256), 0, st, x_packed,
                    (const uint16_t*)h_cur, off_all, rp, rn, (bf16_t*)h_prev, conf, seq_len, S, d, (int)kind, alpha,
                    scores);
    } else if (x_packed)
      DTSK_LAUNCH((k_score<bf16_t, true>), grid, dim3(256), 0, st, (const bf16_t*)h_cur, x_packed, off_all, rp,
                         rn, (bf16_t*)h_prev, conf, seq_len, S, d, (int)kind, alpha, scores);
    else
      DTSK_LAUNCH((k_score<bf16_t, false>), grid, dim3(256), 0, st, (const bf16_t*)h_cur, x_packed, off_all,
                         rp, rn, (bf16_t*)h_prev, conf, seq_len, S, d, (int)kind, alpha, scores);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, const int32_t* seq_len, int B, int S, dl_select_mode mode, float keep,
                         float threshold, int32_t* sel_idx, int32_t* sel_count, hipStream_t st,
                         const int32_t* cand_idx, const int32_t* cand_cnt, const int32_t* k_base, int32_t* row_off,
                         const RowMap* rm) {
  SelMap m{};
  if (row_off) {
    if (B != 1) return hipErrorInvalidValue;
    m.row_off = row_off;
    if (rm) {
      m.n_rows = rm->n_rows;
      m.row_pos = rm->row_pos;
      m.row_seq = rm->row_seq;
      m.tile_row0 = rm->tile_row0;
      m.tile_rows = rm->tile_rows;
      m.R_max = rm->R_max;
      m.T_max = rm->T_max;
      m.tq = rm->tq;
    }
  }
  DTSK_LAUNCH(k_select, dim3(B), dim3(kSelThreads), 0, st, scores, seq_len, S, (int)mode, keep, threshold,
                     cand_idx, cand_cnt, k_base, sel_idx, sel_count, m);
  return hipGetLastError();
}

hipError_t launch_embed(dl_dtype dt, const int32_t* tokens, const RowMap& rm, const void* E, int d, float* x,
                        hipStream_t st) {
  if (d % 4 == 0) {
    if (dt == DL_F32)
      DTSK_LAUNCH(k_embed4<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, tokens, rm.row_pos, (const float*)E, d,
                  x);
    else
      DTSK_LAUNCH(k_embed4<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, tokens, rm.row_pos, (const bf16_t*)E,
                  d, x);
    return hipGetLastError();
  }
  if (dt == DL_F32)
    DTSK_LAUNCH(k_embed<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, tokens, rm.row_pos,
                       (const float*)E, d, x);
  else
    DTSK_LAUNCH(k_embed<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, tokens, rm.row_pos,
                       (const bf16_t*)E, d, x);
  return hipGetLastError();
}

hipError_t launch_gather(size_t elem_bytes, const void* src, const int32_t* src_off, int S, int w, const RowMap& rm,
                         void* dst, hipStream_t st, const int32_t* src_inv) {
  if (rm.R_max <= 0) return hipSuccess;
  const size_t rb = elem_bytes * (size_t)w;
  if (rb % 16 == 0)
    DTSK_LAUNCH(k_gather<16>, dim3(rm.R_max), dim3(kRowThreads), 0, st, (const char*)src, src_off, src_inv, S,
                       rb, rm.row_pos, rm.row_seq, (char*)dst);
  else
    DTSK_LAUNCH(k_gather<1>, dim3(rm.R_max), dim3(kRowThreads), 0, st, (const char*)src, src_off, src_inv, S,
                       rb, rm.row_pos, rm.row_seq, (char*)dst);
  return hipGetLastError();
}

hipError_t launch_inv_rows(const RowMap& rm, int BS, int32_t* inv, hipStream_t st) {
  DTSK_LAUNCH(k_fill_i32, dim3(cdiv(BS, 256)), dim3(256), 0, st, inv, -1, (size_t)BS);
  if (rm.R_max > 0)
    DTSK_LAUNCH(k_inv_rows, dim3(cdiv(rm.R_max, 256)), dim3(256), 0, st, rm.row_pos, rm.n_rows, rm.R_max, inv);
  return hipGetLastError();
}

hipError_t launch_rope_rows(float* x, const RowMap& rm, int S, int d, int head_dim, const float2* rope,
                            hipStream_t st) {
  if (rm.R_max <= 0) return hipSuccess;
  DTSK_LAUNCH(k_rope_rows, dim3(rm.R_max), dim3(kRowThreads), 0, st, x, rm.row_pos, rm.row_seq, S, d, head_dim,
                     rope);
  return hipGetLastError();
}

hipError_t launch_gather_cvt(dl_dtype dt, const float* src, const int32_t* src_off, int S, int d, const RowMap& rm,
                             void* dst, hipStream_t st) {
  if (rm.R_max <= 0) return hipSuccess;
  if (dt == DL_F32)
    DTSK_LAUNCH(k_gather_cvt<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, src, src_off, S, d, rm.row_pos,
                       rm.row_seq, (float*)dst);
  else
    DTSK_LAUNCH(k_gather_cvt<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, src, src_off, S, d,
                       rm.row_pos, rm.row_seq, (bf16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_value_change(dl_dtype dt, const void* V, const void* v_old, const RowMap& rm, int d, void* dv,
                               hipStream_t st) {
  if (rm.R_max <= 0) return hipSuccess;
  if (dt == DL_F32)
    DTSK_LAUNCH(k_value_change<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, (const float*)V,
                       (const float*)v_old, rm.row_pos, d, (float*)dv);
  else
    DTSK_LAUNCH(k_value_change<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, (const bf16_t*)V,
                       (const bf16_t*)v_old, rm.row_pos, d, (bf16_t*)dv);
  return hipGetLastError();
}

hipError_t launch_fill_scores(float* scores, float v, const int32_t* seq_len, int B, int S, hipStream_t st) {
  DTSK_LAUNCH(k_fill_valid, dim3(cdiv(S, 256), B), dim3(256), 0, st, scores, v, seq_len, S);
  return hipGetLastError();
}

hipError_t launch_scatter(size_t elem_bytes, const void* rows, int w, const RowMap& rm, void* cache, hipStream_t st) {
  const size_t rb = elem_bytes * (size_t)w;
  if (rb % 16 == 0)
    DTSK_LAUNCH(k_scatter<16>, dim3(rm.R_max), dim3(kRowThreads), 0, st, (const char*)rows, rb, rm.row_pos,
                       (char*)cache);
  else
    DTSK_LAUNCH(k_scatter<1>, dim3(rm.R_max), dim3(kRowThreads), 0, st, (const char*)rows, rb, rm.row_pos,
                       (char*)cache);
  return hipGetLastError();
}

hipError_t launch_store_rows(dl_dtype dt, const float* x, int w, const RowMap& rm, void* dst, hipStream_t st) {
  if (w % 4 == 0) {
    if (dt == DL_F32)
      DTSK_LAUNCH(k_store_rows4<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, x, w, rm.row_pos, (float*)dst);
    else
      DTSK_LAUNCH(k_store_rows4<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, x, w, rm.row_pos, (bf16_t*)dst);
    return hipGetLastError();
  }
  if (dt == DL_F32)
    DTSK_LAUNCH(k_store_rows<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, x, w, rm.row_pos, (float*)dst);
  else
    DTSK_LAUNCH(k_store_rows<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, x, w, rm.row_pos,
                       (bf16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(dl_dtype dt, const float* x, const void* g, const RowMap& rm, int d, float eps, void* out,
                          hipStream_t st) {
  // the kernels of the split-sum reduction with no splits: the normalised rows
  // come out bit-identical to the ones the reduction after a sub-block writes
  return launch_reduce_rows(dt, nullptr, 0, rm, d, const_cast<float*>(x), g, eps, out, st);
}

hipError_t launch_rope_table(int S, int head_dim, float base, float2* table, hipStream_t st) {
  const int half = head_dim / 2;
  DTSK_LAUNCH(k_rope_table, dim3(cdiv((long long)S * half, 256)), dim3(256), 0, st, S, half, head_dim,
                     (double)base, table);
  return hipGetLastError();
}

hipError_t launch_epi_qkv(dl_dtype dt, const float* P, int splits, const RowMap& rm, int S, int d, int head_dim,
                          const float2* rope, void* q_out, void* k_cache, void* v_cache, hipStream_t st) {
  if (rm.R_max <= 0) return hipSuccess;
  if (head_dim % 8 == 0 && d % head_dim == 0 && d / 8 <= 1024 && splits >= 1 && splits <= kEpiMaxSplits) {
    const dim3 grid(rm.R_max, 3), block((d / 8 + 63) / 64 * 64);
    if (dt == DL_F32)
      DTSK_LAUNCH(k_epi_qkv_rows4<float>, grid, block, 0, st, P, splits, rm.R_max, rm.n_rows, rm.row_pos,
                  rm.row_seq, S, d, head_dim, rope, (float*)q_out, (float*)k_cache, (float*)v_cache);
    else
      DTSK_LAUNCH(k_epi_qkv_rows4<bf16_t>, grid, block, 0, st, P, splits, rm.R_max, rm.n_rows, rm.row_pos,
                  rm.row_seq, S, d, head_dim, rope, (bf16_t*)q_out, (bf16_t*)k_cache, (bf16_t*)v_cache);
    return hipGetLastError();
  }
  if (head_dim <= 128 && d % head_dim == 0 && splits >= 1 && splits <= kEpiMaxSplits) {
    const dim3 grid(rm.R_max, 3 * (d / head_dim));
    if (dt == DL_F32)
      DTSK_LAUNCH(k_epi_qkv_heads<float>, grid, dim3(64), 0, st, P, splits, rm.R_max, rm.n_rows, rm.row_pos,
                         rm.row_seq, S, d, d / head_dim, head_dim, rope, (float*)q_out, (float*)k_cache,
                         (float*)v_cache);
    else
      DTSK_LAUNCH(k_epi_qkv_heads<bf16_t>, grid, dim3(64), 0, st, P, splits, rm.R_max, rm.n_rows, rm.row_pos,
                         rm.row_seq, S, d, d / head_dim, head_dim, rope, (bf16_t*)q_out, (bf16_t*)k_cache,
                         (bf16_t*)v_cache);
    return hipGetLastError();
  }
  if (dt == DL_F32)
    DTSK_LAUNCH(k_epi_qkv<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, P, splits, rm.R_max, rm.n_rows,
                       rm.row_pos, rm.row_seq, S, d, head_dim, rope, (float*)q_out, (float*)k_cache,
                       (float*)v_cache);
  else
    DTSK_LAUNCH(k_epi_qkv<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, P, splits, rm.R_max, rm.n_rows,
                       rm.row_pos, rm.row_seq, S, d, head_dim, rope, (bf16_t*)q_out, (bf16_t*)k_cache,
                       (bf16_t*)v_cache);
  return hipGetLastError();
}

hipError_t launch_epi_residual(const float* P, int splits, const RowMap& rm, int N, float* x, hipStream_t st) {
  DTSK_LAUNCH(k_epi_residual, dim3(rm.R_max), dim3(kRowThreads), 0, st, P, splits, rm.R_max, rm.n_rows, N, x);
  return hipGetLastError();
}

hipError_t launch_epi_swiglu(dl_dtype dt, const float* P, int splits, const RowMap& rm, int F, void* out,
                             hipStream_t st) {
  if (F % 4 == 0 && splits <= kEpiMaxSplits) {
    const dim3 grid(rm.R_max, cdiv(F / 4, kRowThreads));
    if (dt == DL_F32)
      DTSK_LAUNCH(k_epi_swiglu4<float>, grid, dim3(kRowThreads), 0, st, P, splits, rm.R_max, rm.n_rows, F,
                  (float*)out);
    else
      DTSK_LAUNCH(k_epi_swiglu4<bf16_t>, grid, dim3(kRowThreads), 0, st, P, splits, rm.R_max, rm.n_rows, F,
                  (bf16_t*)out);
    return hipGetLastError();
  }
  if (dt == DL_F32)
    DTSK_LAUNCH(k_epi_swiglu<float>, dim3(rm.R_max), dim3(kRowThreads), 0, st, P, splits, rm.R_max,
                       rm.n_rows, F, (float*)out);
  else
    DTSK_LAUNCH(k_epi_swiglu<bf16_t>, dim3(rm.R_max), dim3(kRowThreads), 0, st, P, splits, rm.R_max,
                       rm.n_rows, F, (bf16_t*)out);
  return hipGetLastError();
}

hipError_t launch_lm_reduce(const float* P, int splits, const RowMap& rm, int m_base, int M_max, int V, float* conf,
                            int32_t* argmax, float* logits_out, hipStream_t st) {
  if (M_max <= 0) return hipSuccess;
  DTSK_LAUNCH(k_lm_reduce, dim3(M_max), dim3(kRowThreads), 0, st, P, splits, M_max, rm.n_rows, m_base,
                     rm.row_pos, V, conf, argmax, logits_out);
  return hipGetLastError();
}

template <typename T>
static hipError_t reduce_rows_t(const float* P, int splits, const RowMap& rm, int d, float* x, const void* g,
                                float eps, void* out, hipStream_t st, const RopeJob& rj) {
  const T* gg = (const T*)g;
  T* oo = (T*)out;
  // the rows, then the table's blocks (if any) of the same width
  const auto blocks = [&](int nt) { return rm.R_max + (rj.tab ? cdiv(rj.n, nt) : 0); };
  if (d == 4096)
    DTSK_LAUNCH((k_reduce_rows<T, 4096 / 4 / DTSK_RED_THREADS, DTSK_RED_THREADS>), dim3(blocks(DTSK_RED_THREADS)),
                dim3(DTSK_RED_THREADS), 0, st, P, splits, rm.R_max, rm.n_rows, d, x, gg, eps, oo, rj);
  else if (d == 2048)
    DTSK_LAUNCH((k_reduce_rows<T, 2>), dim3(blocks(kRowThreads)), dim3(kRowThreads), 0, st, P, splits, rm.R_max,
                rm.n_rows, d, x, gg, eps, oo, rj);
  else if (d == 1024)
    DTSK_LAUNCH((k_reduce_rows<T, 1>), dim3(blocks(kRowThreads)), dim3(kRowThreads), 0, st, P, splits, rm.R_max,
                rm.n_rows, d, x, gg, eps, oo, rj);
  else
    DTSK_LAUNCH(k_reduce_rows_any<T>, dim3(blocks(kRowThreads)), dim3(kRowThreads), 0, st, P, splits, rm.R_max,
                rm.n_rows, d, x, gg, eps, oo, rj);
  return hipGetLastError();
}

hipError_t launch_reduce_rows(dl_dtype dt, const float* P, int splits, const RowMap& rm, int d, float* x,
                              const void* g, float eps, void* out, hipStream_t st) {
  if (rm.R_max <= 0) return hipSuccess;
  const RopeJob none{nullptr, 0, 1, 2, 1.0};
  if (dt == DL_F32) return reduce_rows_t<float>(P, splits, rm, d, x, g, eps, out, st, none);
  return reduce_rows_t<bf16_t>(P, splits, rm, d, x, g, eps, out, st, none);
}

hipError_t launch_rmsnorm_rope(dl_dtype dt, const float* x, const void* g, const RowMap& rm, int d, float eps,
                               void* out, int S, int head_dim, float base, float2* table, hipStream_t st) {
  if (rm.R_max <= 0) return launch_rope_table(S, head_dim, base, table, st);
  const RopeJob rj{table, S * (head_dim / 2), head_dim / 2, head_dim, (double)base};
  if (dt == DL_F32) return reduce_rows_t<float>(nullptr, 0, rm, d, const_cast<float*>(x), g, eps, out, st, rj);
  return reduce_rows_t<bf16_t>(nullptr, 0, rm, d, const_cast<float*>(x), g, eps, out, st, rj);
}

hipError_t launch_lm_merge(const float* lm_part, int lm_tiles, const RowMap& rm, int m_base, int M_max, float* conf,
                           int32_t* argmax, hipStream_t st) {
  if (M_max <= 0) return hipSuccess;
  DTSK_LAUNCH(k_lm_merge, dim3(M_max), dim3(kRowThreads), 0, st, (const float4*)lm_part, lm_tiles, rm.n_rows,
                     m_base, rm.row_pos, conf, argmax);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>(1024, (n + 255) / 256);
  DTSK_LAUNCH(k_fill_i32, dim3(blocks), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

hipError_t launch_unmask(int32_t* tokens, uint8_t* masked, const float* conf, const int32_t* argmax,
                         const int32_t* prompt_len, const int32_t* seq_len, int B, int S, int block, int block_len,
                         int n_unmask, hipStream_t st) {
  DTSK_LAUNCH(k_unmask, dim3(B), dim3(kMaxBlockLen), 0, st, tokens, masked, conf, argmax, prompt_len, seq_len,
                     S, block, block_len, n_unmask);
  return hipGetLastError();
}

}  // namespace dtsk
