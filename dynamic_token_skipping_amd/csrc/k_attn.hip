// Partial attention: the packed query rows of a layer attend over every valid
// key of their own sequence (bidirectional), keys and values read from the
// layer's [B, S, d] caches after the rows' fresh K/V were scattered in.
//
//  * k_attn_mfma (bf16, head_dim 128): flash-style.  A workgroup (4 waves)
//    takes 64 query rows of one sequence and one head; each wave owns 16
//    rows.  Key/value tiles of 64 rows are staged in LDS (V transposed).  The
//    wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16, so that each
//    lane holds, for its query (lane % 16), keys 4g..4g+3 and 16+4g..16+4g+3
//    of every 32-key chunk (g = lane / 16): exactly the B operand of
//    O^T = V^T P^T when the MFMA reduction index is ordered the same way on
//    the V^T side.  Online softmax in fp32 (exp2 with the scale folded in).
//  * k_attn_simt: one workgroup per (query row, head); scores staged in LDS,
//    max-subtracted softmax in fp32.  Used for fp32 storage and head sizes the
//    matrix-core kernel does not cover.
#include <math.h>

#include "launch.h"

namespace dtsk {

namespace {

constexpr int kSimtThreads = 128;
constexpr int kMaxKeysSimt = 8192;

// Optional fp32 outputs of the exact attention: the normalised context of a
// query row goes to ctx[row(r) * d + ...] (row = ctx_off[b] + position in the
// sequence, i.e. the packed row of an all-rows map) instead of the storage-type
// output, and its per-head log normaliser log sum_j exp(q.k_j * scale) to
// lse[row_pos[r] * n_heads + h].
struct CtxOut {
  float* ctx;
  float* lse;
  const int32_t* row_pos;
  const int32_t* ctx_off;
  __device__ __forceinline__ size_t row(int r, int b, int S) const {
    return (size_t)ctx_off[b] + (size_t)(row_pos[r] - b * S);
  }
};

// Inputs of the approximate context update (see k_attn_approx_simt).
struct ApproxIn {
  const void* q;              // [B*S, d] cached rotated queries of the layer
  const void* k;              // packed previous keys of the active rows
  const void* dv;             // packed value changes of the active rows
  const int32_t* key_off;     // [B + 1] active rows' packed offsets
  const int32_t* key_cnt;     // [B] active rows per sequence
  const float* lse;           // [B*S, H] cached log normalisers
  const int32_t* inv;         // [B*S] packed active row of a position, -1 if none
  const float* ctx_cache;     // [B*S, d] cached contexts
  float* ctx_new;             // [R_all, d] new contexts, packed like the query map
  const int32_t* n_rows;      // query map (every valid row)
  const int32_t* row_pos;
  const int32_t* row_seq;
};

template <typename T>
__global__ __launch_bounds__(kSimtThreads) void k_attn_simt(const T* __restrict__ q, const T* __restrict__ Kc,
                                                            const T* __restrict__ Vc,
                                                            const int32_t* __restrict__ seq_len,
                                                            const int32_t* __restrict__ n_rows,
                                                            const int32_t* __restrict__ row_seq, int S, int d,
                                                            int head_dim, float scale, T* __restrict__ out,
                                                            CtxOut co) {
  __shared__ float qs[128];
  __shared__ float sc[kMaxKeysSimt];
  __shared__ float red[16];
  const int r = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (r >= *n_rows) return;
  const int b = row_seq[r];
  const int n = seq_len[b];
  const size_t col0 = (size_t)h * head_dim;
  for (int e = t; e < head_dim; e += blockDim.x) qs[e] = to_f32(q[(size_t)r * d + col0 + e]);
  __syncthreads();
  const T* Kb = Kc + (size_t)b * S * d + col0;
  const T* Vb = Vc + (size_t)b * S * d + col0;
  float m = -INFINITY;
  for (int j = t; j < n; j += blockDim.x) {
    const T* kr = Kb + (size_t)j * d;
    float s = 0.f;
    for (int e = 0; e < head_dim; ++e) s = fmaf(qs[e], to_f32(kr[e]), s);
    s *= scale;
    sc[j] = s;
    m = fmaxf(m, s);
  }
  // block max
  m = warp_max(m);
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  float sum = 0.f;
  for (int j = t; j < n; j += blockDim.x) {
    const float p = expf(sc[j] - m);
    sc[j] = p;
    sum += p;
  }
  __syncthreads();
  sum = block_sum(sum, red + 8);
  const float inv = 1.f / sum;
  float* crow = co.ctx ? co.ctx + co.row(r, b, S) * d + col0 : nullptr;
  for (int e = t; e < head_dim; e += blockDim.x) {
    float o = 0.f;
    for (int j = 0; j < n; ++j) o = fmaf(sc[j], to_f32(Vb[(size_t)j * d + e]), o);
    if (crow) crow[e] = o * inv;
    else out[(size_t)r * d + col0 + e] = from_f32<T>(o * inv);
  }
  if (co.lse && t == 0) co.lse[(size_t)co.row_pos[r] * gridDim.y + h] = m + logf(sum);
}

// Approximate context of rows whose query is unchanged (fp32, any head size):
// C_new = C_cached + sum_j exp(q.k_j * scale - lse) dV_j over the active rows j
// of the row's sequence (keys and value changes packed by the active rows'
// selection offsets).  One workgroup per (packed row of the all-rows map,
// head); active rows (inv >= 0) are left to the exact path.
template <typename T>
__global__ __launch_bounds__(kSimtThreads) void k_attn_approx_simt(ApproxIn a, int S, int d, int head_dim,
                                                                   float scale) {
  __shared__ float qs[128];
  __shared__ float sc[kMaxKeysSimt];
  const int r = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (r >= *a.n_rows) return;
  const int pos = a.row_pos[r];
  if (a.inv[pos] >= 0) return;
  const int b = a.row_seq[r];
  const int n = a.key_cnt[b];
  const size_t col0 = (size_t)h * head_dim;
  const T* qc = reinterpret_cast<const T*>(a.q) + (size_t)pos * d + col0;
  for (int e = t; e < head_dim; e += blockDim.x) qs[e] = to_f32(qc[e]);
  __syncthreads();
  const float lse = a.lse[(size_t)pos * gridDim.y + h];
  const T* Kb = reinterpret_cast<const T*>(a.k) + (size_t)a.key_off[b] * d + col0;
  const T* Vb = reinterpret_cast<const T*>(a.dv) + (size_t)a.key_off[b] * d + col0;
  for (int j = t; j < n; j += blockDim.x) {
    const T* kr = Kb + (size_t)j * d;
    float s = 0.f;
    for (int e = 0; e < head_dim; ++e) s = fmaf(qs[e], to_f32(kr[e]), s);
    sc[j] = expf(s * scale - lse);
  }
  __syncthreads();
  const float* cold = a.ctx_cache + (size_t)pos * d + col0;
  float* cnew = a.ctx_new + (size_t)r * d + col0;
  for (int e = t; e < head_dim; e += blockDim.x) {
    float o = 0.f;
    for (int j = 0; j < n; ++j) o = fmaf(sc[j], to_f32(Vb[(size_t)j * d + e]), o);
    cnew[e] = cold[e] + o;
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDh = 128;          // head_dim of the MFMA kernel
constexpr int kTQ = 64;           // query rows per workgroup (16 per wave)
constexpr int kTK = 64;           // keys per LDS tile
constexpr int kKStride = kDh + 8; // LDS row stride of K (bf16 elements)
constexpr int kVStride = kTK + 8; // LDS row stride of V^T (bf16 elements)

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)from_f32<bf16_t>(a).u | ((uint32_t)from_f32<bf16_t>(b).u << 16);
}

// V^T tile: row = dim (kVStride bf16), 32-bit word = a pair of keys.  Pair
// kp of dim row `dim` lives in word slot kp ^ (((dim >> 3) & 7) << 2): the
// stores of one instruction (4 key pairs x 16 dim chunks) then hit 32
// distinct banks, and the readers' 8-byte pair loads stay contiguous because
// the XOR leaves bit 0 of the slot alone.
__device__ __forceinline__ int vt_word(int dim, int kp) { return dim * (kVStride / 2) + (kp ^ (((dim >> 3) & 7) << 2)); }

// One workgroup = (64-query tile, head, key chunk [kbeg, kbeg + chunk)).
// With one chunk the normalised output goes straight to `out` (or in fp32 to
// co.ctx with the log normaliser to co.lse); with several, the chunk's
// unnormalised O and its (running max, sum) go to o_part/ml_part and
// k_attn_combine merges them.
// kApprox: the approximate context update instead (DyLLM's saliency-aware
// approximate attention): the query tiles are those of the all-rows map, each
// row's cached query is read at its position, the keys and values are the
// active rows' previous keys and value changes (packed, a.key_off / a.key_cnt),
// and the softmax has the row's cached normaliser in place of the running one:
// C_new = C_cached + sum_j 2^(s_j - lse2) dV_j, written for non-active rows.
template <bool kApprox>
__global__ __launch_bounds__(256) void k_attn_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
                                                   const uint16_t* __restrict__ Vc,
                                                   const int32_t* __restrict__ seq_len,
                                                   const int32_t* __restrict__ row_seq,
                                                   const int32_t* __restrict__ tile_row0,
                                                   const int32_t* __restrict__ tile_rows, int S, int d, int n_heads,
                                                   float scale_log2, int chunk, int n_split, int n_tiles,
                                                   uint16_t* __restrict__ out, float* __restrict__ o_part,
                                                   float2* __restrict__ ml_part, int R_part, CtxOut co, ApproxIn a) {
  __shared__ __align__(16) uint16_t Ks[kTK * kKStride];
  __shared__ __align__(16) uint32_t Vt[kDh * kVStride / 2];
  // Block order: (head, chunk) pair p runs on XCD p % 8, and on that XCD the
  // query tiles of one pair get consecutive block ids, so the tiles that read
  // the same keys and values do so through one L2.
  const int xcd = blockIdx.x & 7, rb = blockIdx.x >> 3;
  const int pq = rb / n_tiles, tile = rb - pq * n_tiles;
  const int pair = pq * 8 + xcd;
  if (pair >= n_heads * n_split) return;
  const int h = pair % n_heads, split = pair / n_heads;
  const int nrows = tile_rows[tile];
  if (nrows <= 0) return;
  const int r0 = tile_row0[tile];
  const int b = row_seq[r0];
  const int n = kApprox ? a.key_cnt[b] : seq_len[b];
  const int kbeg = split * chunk;
  if (!kApprox && kbeg >= n) return;               // the combine only reads chunks below n
  const int kend = min(n, kbeg + chunk);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ql = lane & 15, g = lane >> 4;
  const int qrow = wave * 16 + ql;                 // query row within the tile
  const bool qvalid = qrow < nrows;
  const size_t col0 = (size_t)h * kDh;

  // Q^T fragments (B operand): query ql, dims c*32 + g*8 .. +8
  size_t qsrc_row = (size_t)(r0 + qrow);
  const uint16_t* qsrc = q;
  float lse2 = 0.f;                                // kApprox: the row's cached normaliser (log2 units)
  if constexpr (kApprox) {
    qsrc = static_cast<const uint16_t*>(a.q);
    qsrc_row = qvalid ? (size_t)a.row_pos[r0 + qrow] : 0;
    if (qvalid) lse2 = a.lse[qsrc_row * n_heads + h] * 1.4426950408889634f;
  }
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qvalid) v = *reinterpret_cast<const uint4*>(qsrc + qsrc_row * d + col0 + c * 32 + g * 8);
    qf[c] = __builtin_bit_cast(bf16x8, v);
  }

  f32x4 o[8];  // O^T blocks: dims blk*16 + g*4 + i, query ql
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* Kb = kApprox ? static_cast<const uint16_t*>(a.k) + (size_t)a.key_off[b] * d + col0
                               : Kc + (size_t)b * S * d + col0;
  const uint16_t* Vb = kApprox ? static_cast<const uint16_t*>(a.dv) + (size_t)a.key_off[b] * d + col0
                               : Vc + (size_t)b * S * d + col0;
  // per thread and tile: 4 K chunks (key c >> 4, dims (c & 15) * 8) and 2 x 2 V
  // chunks (keys 2kp, 2kp + 1 of key pair kp = c >> 4, dims (c & 15) * 8)
  uint4 kr[4], va[2], vb[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t + i * 256;
      const int key = k0 + (c >> 4), dc = (c & 15) * 8;
      kr[i] = key < kend ? *reinterpret_cast<const uint4*>(Kb + (size_t)key * d + dc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + i * 256;
      const int key = k0 + (c >> 4) * 2, dc = (c & 15) * 8;
      va[i] = key < kend ? *reinterpret_cast<const uint4*>(Vb + (size_t)key * d + dc) : make_uint4(0, 0, 0, 0);
      vb[i] = key + 1 < kend ? *reinterpret_cast<const uint4*>(Vb + (size_t)(key + 1) * d + dc)
                             : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kTK) {
    lds_barrier();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t + i * 256;
      *reinterpret_cast<uint4*>(Ks + (c >> 4) * kKStride + (c & 15) * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + i * 256;
      const int kp = c >> 4, dc = (c & 15) * 8;
      const uint32_t aw[4] = {va[i].x, va[i].y, va[i].z, va[i].w}, bw[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[vt_word(dc + 2 * e, kp)] = (aw[e] & 0xffffu) | (bw[e] << 16);          // dim dc+2e:   keys 2kp, 2kp+1
        Vt[vt_word(dc + 2 * e + 1, kp)] = (aw[e] >> 16) | (bw[e] & 0xffff0000u);  // dim dc+2e+1
      }
    }
    if (k0 + kTK < kend) fetch(k0 + kTK);          // next tile in flight during this one's math
    lds_barrier();

    // S^T blocks: keys kb*16 + g*4 + i (i < 4), query ql
    f32x4 st[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 kv = *reinterpret_cast<const uint4*>(Ks + (kb * 16 + ql) * kKStride + c * 32 + g * 8);
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qf[c], st[kb], 0, 0, 0);
      }
    }
    if constexpr (kApprox) {
      // cached probabilities: 2^(s - lse2), no running normaliser
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kb * 16 + g * 4 + i;
          st[kb][i] = key < kend ? exp2f(st[kb][i] * scale_log2 - lse2) : 0.f;
        }
    } else {
    // online softmax for query ql over this tile
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kb * 16 + g * 4 + i;
        float v = st[kb][i] * scale_log2;
        if (key >= kend) v = -INFINITY;
        st[kb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float corr = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(st[kb][i] - m_new);
        st[kb][i] = p;
        psum += p;
      }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) o[blk] *= corr;
    }
    // O^T += V^T P^T over the two 32-key chunks
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint4 pw;
      pw.x = pack_bf16x2(st[2 * c][0], st[2 * c][1]);
      pw.y = pack_bf16x2(st[2 * c][2], st[2 * c][3]);
      pw.z = pack_bf16x2(st[2 * c + 1][0], st[2 * c + 1][1]);
      pw.w = pack_bf16x2(st[2 * c + 1][2], st[2 * c + 1][3]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int dim = blk * 16 + ql;
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[vt_word(dim, c * 16 + g * 2)]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[vt_word(dim, c * 16 + 8 + g * 2)]);
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[blk], 0, 0, 0);
      }
    }
  }
  if constexpr (kApprox) {
    if (!qvalid) return;
    const int r = r0 + qrow;
    const size_t pos = (size_t)a.row_pos[r];
    if (a.inv[pos] >= 0) return;                   // active rows take the exact path
    const float* cold = a.ctx_cache + pos * d + col0;
    float* cnew = a.ctx_new + (size_t)r * d + col0;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const float4 c = *reinterpret_cast<const float4*>(cold + blk * 16 + g * 4);
      *reinterpret_cast<float4*>(cnew + blk * 16 + g * 4) =
          make_float4(c.x + o[blk][0], c.y + o[blk][1], c.z + o[blk][2], c.w + o[blk][3]);
    }
    return;
  }
  // full row sum over the 4 lanes sharing this query
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const int r = r0 + qrow;
  if (n_split == 1 && co.ctx) {
    const float inv = 1.f / l_run;
    float* crow = co.ctx + co.row(r, b, S) * d + col0;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
      *reinterpret_cast<float4*>(crow + blk * 16 + g * 4) =
          make_float4(o[blk][0] * inv, o[blk][1] * inv, o[blk][2] * inv, o[blk][3] * inv);
    if (g == 0) co.lse[(size_t)co.row_pos[r] * n_heads + h] = (m_run + log2f(l_run)) * 0.6931471805599453f;
    return;
  }
  if (n_split == 1) {
    const float inv = 1.f / l_run;
    uint16_t* orow = out + (size_t)r * d + col0;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      uint2 w;
      w.x = pack_bf16x2(o[blk][0] * inv, o[blk][1] * inv);
      w.y = pack_bf16x2(o[blk][2] * inv, o[blk][3] * inv);
      *reinterpret_cast<uint2*>(orow + blk * 16 + g * 4) = w;
    }
    return;
  }
  float* prow = o_part + ((size_t)split * R_part + r) * d + col0;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
    *reinterpret_cast<float4*>(prow + blk * 16 + g * 4) = make_float4(o[blk][0], o[blk][1], o[blk][2], o[blk][3]);
  if (g == 0) ml_part[((size_t)split * R_part + r) * n_heads + h] = make_float2(m_run, l_run);
}

// Merge the key chunks of each (row, head): O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// Grid (packed row, 256-column group); thread t covers 4 columns.
__global__ __launch_bounds__(64) void k_attn_combine(const float* __restrict__ o_part,
                                                     const float2* __restrict__ ml_part,
                                                     const int32_t* __restrict__ n_rows,
                                                     const int32_t* __restrict__ row_seq,
                                                     const int32_t* __restrict__ seq_len, int d, int n_heads,
                                                     int chunk, int splits, int R_part, uint16_t* __restrict__ out,
                                                     CtxOut co, int S) {
  const int r = blockIdx.x;
  const int col = blockIdx.y * 256 + threadIdx.x * 4;
  if (r >= *n_rows || col >= d) return;
  const int n = seq_len[row_seq[r]];
  const int ns = min(splits, (n + chunk - 1) / chunk);
  const int h = col / kDh;
  float2 ml[kAttnMaxSplits];
  float4 v[kAttnMaxSplits];
#pragma unroll
  for (int c = 0; c < kAttnMaxSplits; ++c) {      // all loads first
    if (c < ns) {
      ml[c] = ml_part[((size_t)c * R_part + r) * n_heads + h];
      v[c] = *reinterpret_cast<const float4*>(o_part + ((size_t)c * R_part + r) * d + col);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < kAttnMaxSplits; ++c)
    if (c < ns) M = fmaxf(M, ml[c].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int c = 0; c < kAttnMaxSplits; ++c) {
    if (c < ns) {
      const float w = exp2f(ml[c].x - M);
      L += w * ml[c].y;
      acc.x += w * v[c].x;
      acc.y += w * v[c].y;
      acc.z += w * v[c].z;
      acc.w += w * v[c].w;
    }
  }
  const float inv = 1.f / L;
  if (co.ctx) {
    const int b = row_seq[r];
    *reinterpret_cast<float4*>(co.ctx + co.row(r, b, S) * d + col) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (col % kDh == 0) co.lse[(size_t)co.row_pos[r] * n_heads + h] = (M + log2f(L)) * 0.6931471805599453f;
    return;
  }
  uint2 w2;
  w2.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  w2.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(out + (size_t)r * d + col) = w2;
}

}  // namespace

static bool use_mfma_attention(dl_dtype dt, int head_dim) { return dt == DL_BF16 && head_dim == kDh; }

bool attention_supported(dl_dtype dt, int S, int head_dim) {
  if (use_mfma_attention(dt, head_dim)) return true;
  return head_dim <= 128 && head_dim % 2 == 0 && S <= kMaxKeysSimt;
}

#ifndef DTSK_ATTN_SPLIT_CAP
#define DTSK_ATTN_SPLIT_CAP kAttnMaxSplits
#endif

int attention_splits(dl_dtype dt, int head_dim, int S, int n_heads, const RowMap& rm, int R_part) {
  if (!use_mfma_attention(dt, head_dim) || rm.R_max > R_part) return 1;
  const int base = std::max(1, rm.T_max * n_heads);
  int s = std::min(std::min(kAttnMaxSplits, DTSK_ATTN_SPLIT_CAP), std::max(1, kAttnTargetBlocks / base));
  s = std::min(s, std::max(1, S / (2 * kTK)));     // at least two key tiles per chunk
  return s;
}

hipError_t launch_attention(dl_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_len, const RowMap& rm, int S, int n_heads, int head_dim, int splits,
                            float* o_part, float2* ml_part, int R_part, void* out, hipStream_t st, float* ctx_out,
                            const int32_t* ctx_off, float* lse_out) {
  const int d = n_heads * head_dim;
  const float scale = 1.f / sqrtf((float)head_dim);
  const CtxOut co{ctx_out, lse_out, rm.row_pos, ctx_off};
  if (ctx_out && (!lse_out || !ctx_off)) return hipErrorInvalidValue;
  if (use_mfma_attention(dt, head_dim)) {
    if (rm.tq != kTQ || rm.T_max <= 0) return rm.T_max < 0 ? hipErrorInvalidValue : hipSuccess;
    if (splits < 1 || splits > kAttnMaxSplits || (splits > 1 && (!o_part || !ml_part || rm.R_max > R_part)))
      return hipErrorInvalidValue;
    const int chunk = (S + splits * kTK - 1) / (splits * kTK) * kTK;
    const float scale_log2 = scale * 1.4426950408889634f;
    const int grid = (n_heads * splits + 7) / 8 * 8 * rm.T_max;
    DTSK_LAUNCH(k_attn_mfma<false>, dim3(grid), dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, seq_len, rm.row_seq, rm.tile_row0, rm.tile_rows, S, d, n_heads,
                       scale_log2, chunk, splits, rm.T_max, (uint16_t*)out, o_part, ml_part, R_part, co, ApproxIn{});
    if (splits > 1 && rm.R_max > 0)
      DTSK_LAUNCH(k_attn_combine, dim3(rm.R_max, (d + 255) / 256), dim3(64), 0, st, o_part, ml_part,
                         rm.n_rows, rm.row_seq, seq_len, d, n_heads, chunk, splits, R_part, (uint16_t*)out, co, S);
    return hipGetLastError();
  }
  dim3 grid(rm.R_max, n_heads);
  if (rm.R_max <= 0) return hipSuccess;
  if (dt == DL_F32)
    DTSK_LAUNCH(k_attn_simt<float>, grid, dim3(kSimtThreads), 0, st, (const float*)q, (const float*)k_cache,
                       (const float*)v_cache, seq_len, rm.n_rows, rm.row_seq, S, d, head_dim, scale, (float*)out, co);
  else
    DTSK_LAUNCH(k_attn_simt<bf16_t>, grid, dim3(kSimtThreads), 0, st, (const bf16_t*)q,
                       (const bf16_t*)k_cache, (const bf16_t*)v_cache, seq_len, rm.n_rows, rm.row_seq, S, d,
                       head_dim, scale, (bf16_t*)out, co);
  return hipGetLastError();
}

hipError_t launch_attention_approx(dl_dtype dt, const void* q_cache, const void* k_act, const void* dv_act,
                                   const int32_t* key_off, const int32_t* key_cnt, const float* lse,
                                   const int32_t* inv, const float* ctx_cache, float* ctx_new, const RowMap& rm_all,
                                   int S, int n_heads, int head_dim, hipStream_t st) {
  const int d = n_heads * head_dim;
  const float scale = 1.f / sqrtf((float)head_dim);
  const ApproxIn a{q_cache, k_act, dv_act, key_off, key_cnt, lse, inv, ctx_cache, ctx_new,
                   rm_all.n_rows, rm_all.row_pos, rm_all.row_seq};
  if (rm_all.R_max <= 0) return hipSuccess;
  if (use_mfma_attention(dt, head_dim)) {
    if (rm_all.tq != kTQ || rm_all.T_max <= 0) return rm_all.T_max < 0 ? hipErrorInvalidValue : hipSuccess;
    const float scale_log2 = scale * 1.4426950408889634f;
    const int grid = (n_heads + 7) / 8 * 8 * rm_all.T_max;
    DTSK_LAUNCH(k_attn_mfma<true>, dim3(grid), dim3(256), 0, st, nullptr, nullptr, nullptr, nullptr,
                       rm_all.row_seq, rm_all.tile_row0, rm_all.tile_rows, S, d, n_heads, scale_log2, S, 1,
                       rm_all.T_max, nullptr, nullptr, nullptr, 0, CtxOut{}, a);
    return hipGetLastError();
  }
  if (S > kMaxKeysSimt) return hipErrorInvalidValue;
  dim3 grid(rm_all.R_max, n_heads);
  if (dt == DL_F32)
    DTSK_LAUNCH(k_attn_approx_simt<float>, grid, dim3(kSimtThreads), 0, st, a, S, d, head_dim, scale);
  else
    DTSK_LAUNCH(k_attn_approx_simt<bf16_t>, grid, dim3(kSimtThreads), 0, st, a, S, d, head_dim, scale);
  return hipGetLastError();
}

}  // namespace dtsk
