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
//    With key chunks over several workgroups, k_attn_combine merges them.
//  * k_attn_rows (bf16, head_dim 128, up to kRowsMaxKeys keys): every key of
//    a (query rows, head) in one workgroup, the key range split over the
//    waves within each tile and the waves' softmax states merged in LDS, so
//    nothing is merged afterwards.  64 queries per workgroup over 64-key
//    tiles when the query tiles fill the chip; else 16 queries over 128-key
//    tiles with 8 waves (the kept rows of one sequence).
//  * K/V tiles come through buffer loads whose range ends at the sequence's
//    last key (zeros past it, no branches), several tiles ahead in registers.
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
// lse[row_pos[r] * n_heads + h].  Without ctx, lse_rows (if set) takes the
// same normaliser at the packed row, lse_rows[r * n_heads + h], beside the
// storage-type output.
struct CtxOut {
  float* ctx;
  float* lse;
  const int32_t* row_pos;
  const int32_t* ctx_off;
  float* lse_rows;
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
  if (t == 0) {
    const float ls = m + logf(sum);
    if (co.lse) co.lse[(size_t)co.row_pos[r] * gridDim.y + h] = ls;
    if (co.lse_rows) co.lse_rows[(size_t)r * gridDim.y + h] = ls;
  }
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

// Two fp32 values to a bf16 pair, round to nearest even: one
// v_cvt_pk_bf16_f32 (the same bits as from_f32<bf16_t> for every non-NaN
// value; a NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
// 2^x for the softmax: one v_exp_f32 (2^-inf = 0).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// V^T tile: row = dim (kVStride bf16), 32-bit word = a pair of keys.  Pair
// kp of dim row `dim` lives in word slot kp ^ (((dim >> 3) & 7) << 2): the
// stores of one instruction (4 key pairs x 16 dim chunks) then hit 32
// distinct banks, and the readers' 8-byte pair loads stay contiguous because
// the XOR leaves bit 0 of the slot alone.
template <int TK>   // keys per tile: a V^T row holds TK + 8 bf16
__device__ __forceinline__ int vt_word_t(int dim, int kp) { return dim * ((TK + 8) / 2) + (kp ^ (((dim >> 3) & 7) << 2)); }
__device__ __forceinline__ int vt_word(int dim, int kp) { return vt_word_t<kTK>(dim, kp); }
// The V^T words of two keys' rows a (key 2kp) and b (key 2kp + 1), each
// holding dims 2e, 2e + 1: low halves (dim 2e) and high halves (dim 2e + 1),
// key 2kp in the low half of the word.  One v_perm_b32 each.
__device__ __forceinline__ uint32_t vt_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t vt_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Unit (head, or (head, key chunk) pair) of the pq-th block group on XCD
// `xcd`, or -1 past the last: unit pq * 8 + xcd, so that units x, x + 8, ...
// run on XCD x and the query tiles of one unit share that XCD's L2.
// (Consecutive units per XCD, which put a head's 256-byte K/V row slices in
// other L2 channels, measured the same.)
__device__ __forceinline__ int unit_on_xcd(int pq, int xcd, int n_units) {
  const int u = pq * 8 + xcd;
  return u < n_units ? u : -1;
}

// Waves per SIMD the key-chunk kernel is built for: 3 (168 VGPRs, no
// spills, against 184 and 2 waves left to the compiler) lets the softmax
// vector work of one wave overlap the matrix-core work of the others; 0:
// the compiler's choice.
#ifndef DTSK_ATTN_MFMA_OCC
#define DTSK_ATTN_MFMA_OCC 3
#endif
#if DTSK_ATTN_MFMA_OCC > 0
#define DTSK_ATTN_MFMA_BOUNDS __launch_bounds__(256, DTSK_ATTN_MFMA_OCC)
#else
#define DTSK_ATTN_MFMA_BOUNDS __launch_bounds__(256)
#endif

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
__global__ DTSK_ATTN_MFMA_BOUNDS void k_attn_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
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
  const int pair = unit_on_xcd(pq, xcd, n_heads * n_split);
  if (pair < 0) return;
  const int h = pair % n_heads, split = pair / n_heads;
  const int nrows = __builtin_amdgcn_readfirstlane(tile_rows[tile]);
  if (nrows <= 0) return;
  const int r0 = __builtin_amdgcn_readfirstlane(tile_row0[tile]);
  const int b = __builtin_amdgcn_readfirstlane(row_seq[r0]);   // uniform: the resources below stay scalar
  const int n = __builtin_amdgcn_readfirstlane(kApprox ? a.key_cnt[b] : seq_len[b]);
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

  const int koff_b = kApprox ? __builtin_amdgcn_readfirstlane(a.key_off[b]) : 0;
  const uint16_t* Kb = kApprox ? static_cast<const uint16_t*>(a.k) + (size_t)koff_b * d : Kc + (size_t)b * S * d;
  const uint16_t* Vb = kApprox ? static_cast<const uint16_t*>(a.dv) + (size_t)koff_b * d : Vc + (size_t)b * S * d;
  // K and V rows of the sequence through buffer resources ending at key kend
  // (the chunk's end): keys past it read as zeros with no branch, so the next
  // tile's loads stay in flight during this tile's math.  Per thread and
  // tile: 4 K chunks (key c >> 4, dims (c & 15) * 8 of head h) and 2 x 2 V
  // chunks (keys 2kp, 2kp + 1 of key pair kp = c >> 4).
  // The per-lane offsets within a tile are fixed; each tile moves the
  // resources' base (scalar arithmetic only) and shrinks their range to the
  // keys left before kend.
  const uint32_t row_bytes = (uint32_t)d * 2;
  const uint32_t coff = (uint32_t)(col0 + (t & 15) * 8) * 2;
  uint32_t kofs[4], vofs[2], vofs1[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) kofs[i] = (uint32_t)((t >> 4) + i * 16) * row_bytes + coff;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    vofs[i] = (uint32_t)((t >> 4) * 2 + i * 32) * row_bytes + coff;
    vofs1[i] = vofs[i] + row_bytes;
  }
  uint4 kr[4], va[2], vb[2];
  auto fetch = [&](int k0) {
    // keys left as a signed max (a scalar instruction; an unsigned "a < b ?
    // b - a : 0" becomes a vector-only saturating subtract, and a resource
    // in vector registers costs a waterfall loop around every load)
    const uint32_t tb = (uint32_t)k0 * row_bytes;
    const uint32_t rec = (uint32_t)max(kend - k0, 0) * row_bytes;
    const __amdgpu_buffer_rsrc_t k_rs = buf_rsrc(reinterpret_cast<const char*>(Kb) + tb, rec);
    const __amdgpu_buffer_rsrc_t v_rs = buf_rsrc(reinterpret_cast<const char*>(Vb) + tb, rec);
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = buf_load16(k_rs, kofs[i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      va[i] = buf_load16(v_rs, vofs[i]);
      vb[i] = buf_load16(v_rs, vofs1[i]);
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
        Vt[vt_word(dc + 2 * e, kp)] = vt_lo(aw[e], bw[e]);       // dim dc+2e:   keys 2kp, 2kp+1
        Vt[vt_word(dc + 2 * e + 1, kp)] = vt_hi(aw[e], bw[e]);   // dim dc+2e+1
      }
    }
    fetch(k0 + kTK);                               // next tile in flight during this one's math (past kend: zeros)
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
      // cached probabilities: 2^(s - lse2), no running normaliser; keys past
      // kend masked only in the tile that crosses it (uniform)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[kb][i] = exp2_fast(fmaf(st[kb][i], scale_log2, -lse2));
      if (k0 + kTK > kend) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + kb * 16 + g * 4 + i >= kend) st[kb][i] = 0.f;
      }
    } else {
    // online softmax for query ql over this tile
    // unscaled scores, their max scaled once, the scale of each probability
    // in one fma (as in k_attn_rows)
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, st[kb][i]);
    if (k0 + kTK > kend) {                          // the tile that crosses kend (uniform): mask the keys past it
      tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (k0 + kb * 16 + g * 4 + i >= kend) st[kb][i] = -INFINITY;
          tmax = fmaxf(tmax, st[kb][i]);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    tmax *= scale_log2;
    // Lazy rescale (as in k_attn_rows): the reference max m_run moves only
    // when a tile brings a score more than 8 above it, so p <= 2^8 and O, l
    // stay relative to m_run; a wave rescales only when one of its queries
    // moved.  The softmax vector work per score roughly halves.
    const bool grow = tmax > m_run + 8.f;
    const float m_new = grow ? tmax : m_run;
    if (__builtin_amdgcn_ballot_w64(grow)) {        // uniform over the wave
      const float corr = grow ? exp2_fast(m_run - m_new) : 1.f;
      l_run *= corr;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) o[blk] *= corr;
    }
    m_run = m_new;
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;   // no key seen yet: every p is 2^-inf = 0
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_fast(fmaf(st[kb][i], scale_log2, -m_ref));
        st[kb][i] = p;
        psum += p;
      }
    l_run += psum;
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
    if (co.lse_rows && g == 0)
      co.lse_rows[(size_t)r * n_heads + h] = (m_run + log2f(l_run)) * 0.6931471805599453f;
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

// Attention over every key without key chunks: one workgroup = (16 G queries
// of a 64-row query tile, head), G x H waves.  Wave w serves the 16 queries
// of group w % G and part p = w / G of every 64-key tile (keys p * 64 / H to
// (p + 1) * 64 / H - 1 of each tile); the tile's K and V^T are staged once in
// LDS for all waves, and the next A tiles are in flight in registers
// meanwhile.  At the end the H parts' softmax states (m, l, O) of each query
// are merged through LDS: O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.
// No partial results leave the workgroup.  Same S^T = K Q^T / O^T += V^T P^T
// fragments as k_attn_mfma; with 16 keys per wave (H = 4) the P^T operand of
// a lane is exactly the four probabilities its S^T block left it (keys
// 4g .. 4g + 3 of query ql), fed to the 16x16x16 MFMA.
// G = 4, H = 2: 64 queries per workgroup, for many query rows.  G = 1, H = 8
// (128-key tiles): four workgroups per query tile, for few query rows (the
// kept rows of one sequence), where it replaces the key chunks and their
// merge kernel.  With lse_rows set, each query's log normaliser
// (M + log2 den) ln 2 of the merged state goes to lse_rows[row * n_heads + h].
#ifndef DTSK_ROWS_MAX_KEYS
#define DTSK_ROWS_MAX_KEYS 1024
#endif
constexpr int kRowsMaxKeys = DTSK_ROWS_MAX_KEYS;  // longer sequences take the key-chunk kernel
constexpr int kRowsMinBlocks = 256; // (query tile, head) pairs from which 64-query workgroups fill the chip
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int G, int H, int A, int TK>   // A: key tiles in flight beyond the one in LDS; TK keys per tile
__global__ __launch_bounds__(G * H * 64) void k_attn_rows(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ Kc,
                                                          const uint16_t* __restrict__ Vc,
                                                          const int32_t* __restrict__ seq_len,
                                                          const int32_t* __restrict__ row_seq,
                                                          const int32_t* __restrict__ tile_row0,
                                                          const int32_t* __restrict__ tile_rows, int S, int d,
                                                          int n_heads, float scale_log2, int n_tiles,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse_rows, int one_seq) {
  constexpr int NT = G * H * 64;               // threads
  constexpr int KW = TK / H;                   // keys of a tile per wave
  constexpr int NSB = KW / 16;                 // S^T blocks per wave and tile
  constexpr int SUB = kTQ / (16 * G);          // workgroups per 64-row query tile
  constexpr int KC = TK * 16 / NT;             // 16-byte K chunks per thread and tile
  constexpr int VC = TK * 8 / NT;              // V key-pair chunks per thread and tile
  static_assert((NSB == 1 || NSB == 2) && SUB >= 1 && KC >= 1 && VC >= 1, "workgroup shape");
  // one LDS block: the K tile and the V^T tile, later the other parts' O^T
  constexpr int kKsBytes = TK * kKStride * 2, kVtBytes = kDh * (TK + 8) * 2;
  // Merge through LDS: when every part's O^T fits (kAllMerge), all waves
  // write theirs and each then merges 8 / H of the 8 dim blocks; otherwise
  // parts 1 .. H-1 write and part 0 merges all blocks.
  constexpr bool kAllMerge = H * G * 8 * 16 * 16 * 4 <= kKsBytes + kVtBytes;
  constexpr int kMergeParts = kAllMerge ? H : H - 1;   // parts whose state goes through LDS
  static_assert(kMergeParts * G * 8 * 16 * 16 * 4 <= kKsBytes + kVtBytes, "merge buffer");
  static_assert(!kAllMerge || 8 % H == 0, "dim blocks per wave");
  __shared__ __align__(16) char smem[kKsBytes + kVtBytes];
  __shared__ float merge_ml[kMergeParts * G][16][2];   // (m, l) of the parts' queries
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint32_t* Vt = reinterpret_cast<uint32_t*>(smem + kKsBytes);
  // Block order: head p runs on XCD p % 8 and its query tiles (and their
  // sub-tiles) get consecutive block ids there, so the workgroups reading the
  // same keys share one L2.
  const int xcd = blockIdx.x & 7, rb = blockIdx.x >> 3;
  const int pq = rb / (n_tiles * SUB), rem = rb - pq * (n_tiles * SUB);
  const int tile = rem / SUB, sub = rem - tile * SUB;
  const int h = unit_on_xcd(pq, xcd, n_heads);
  if (h < 0) return;
  // With one sequence its key count is read beside the tile's entries
  // instead of after the row's sequence: one dependent load fewer before the
  // first key tile.
  const int nrows = __builtin_amdgcn_readfirstlane(tile_rows[tile]);
  const int r0 = __builtin_amdgcn_readfirstlane(tile_row0[tile]);
  const int n_one = one_seq ? __builtin_amdgcn_readfirstlane(seq_len[0]) : 0;
  if (nrows <= sub * 16 * G) return;               // also an unused tile (0 rows)
  const int b = one_seq ? 0 : __builtin_amdgcn_readfirstlane(row_seq[r0]);   // uniform: the resources below stay scalar
  const int n = one_seq ? n_one : __builtin_amdgcn_readfirstlane(seq_len[b]);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int grp = wave % G, part = wave / G;
  const int ql = lane & 15, g = lane >> 4;
  const int qrow = sub * 16 * G + grp * 16 + ql;   // query row within the 64-row tile
  const bool qvalid = qrow < nrows;
  const size_t col0 = (size_t)h * kDh;

  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qvalid) v = *reinterpret_cast<const uint4*>(q + (size_t)(r0 + qrow) * d + col0 + c * 32 + g * 8);
    qf[c] = __builtin_bit_cast(bf16x8, v);
  }
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // K and V rows of this sequence through buffer resources ending at key n:
  // keys >= n (the last tile's tail, the tiles fetched past the end) read as
  // zeros with no branch, so the loads of every ring slot stay countable and
  // in flight together.  Per thread and tile: KC K chunks (chunk c = t + i NT:
  // key c >> 4, dims (c & 15) * 8 of head h) and VC V key pairs (the two keys
  // of pair c >> 4, same dims).
  // The per-lane offsets within a tile are fixed; each tile moves the
  // resources' base (scalar arithmetic only) and shrinks their range to the
  // keys left before n.
  const uint32_t row_bytes = (uint32_t)d * 2;
  const char* kseq = reinterpret_cast<const char*>(Kc + (size_t)b * S * d);
  const char* vseq = reinterpret_cast<const char*>(Vc + (size_t)b * S * d);
  const uint32_t coff = (uint32_t)(col0 + (t & 15) * 8) * 2;
  uint32_t kofs[KC], vofs[VC], vofs1[VC];
#pragma unroll
  for (int i = 0; i < KC; ++i) kofs[i] = (uint32_t)((t >> 4) + i * (NT >> 4)) * row_bytes + coff;
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    vofs[i] = (uint32_t)((t >> 4) * 2 + i * (NT >> 3)) * row_bytes + coff;
    vofs1[i] = vofs[i] + row_bytes;
  }
  uint4 kr[A + 1][KC], va[A + 1][VC], vb[A + 1][VC];
  auto fetch = [&](int k0, int slot) {
    const uint32_t tb = (uint32_t)k0 * row_bytes;
    const uint32_t rec = (uint32_t)max(n - k0, 0) * row_bytes;   // scalar (see k_attn_mfma)
    const __amdgpu_buffer_rsrc_t k_rs = buf_rsrc(kseq + tb, rec);
    const __amdgpu_buffer_rsrc_t v_rs = buf_rsrc(vseq + tb, rec);
#pragma unroll
    for (int i = 0; i < KC; ++i) kr[slot][i] = buf_load16(k_rs, kofs[i]);
#pragma unroll
    for (int i = 0; i < VC; ++i) {
      va[slot][i] = buf_load16(v_rs, vofs[i]);
      vb[slot][i] = buf_load16(v_rs, vofs1[i]);
    }
  };
  const int n_kt = (n + TK - 1) / TK;
  constexpr int kRing = A + 1;
#pragma unroll
  for (int a = 0; a < A; ++a) {
    fetch(a * TK, a);
    __builtin_amdgcn_sched_barrier(0);   // slot by slot, the order the ring's waits count in
  }
  // Unrolled by the ring length so that every ring slot is a fixed register
  // set.  The ring runs over whole ring lengths of tiles: every pass issues
  // and consumes its loads on every path (the tiles past n_kt read zeros), so
  // the count of loads in flight is the same at every join and the waits stay
  // partial; only the math of a tile past the end is skipped.
  for (int kt0 = 0; kt0 < n_kt; kt0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
    const int kt = kt0 + u;
    const int k0 = kt * TK;
    fetch((kt + A) * TK, (u + A) % kRing);   // past the end: zeros, no memory access
    lds_barrier();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = t + i * NT;
      *reinterpret_cast<uint4*>(Ks + (c >> 4) * kKStride + (c & 15) * 8) = kr[u][i];
    }
#pragma unroll
    for (int i = 0; i < VC; ++i) {
      const int c = t + i * NT;
      const int kp = c >> 4, dc = (c & 15) * 8;
      const uint32_t aw[4] = {va[u][i].x, va[u][i].y, va[u][i].z, va[u][i].w};
      const uint32_t bw[4] = {vb[u][i].x, vb[u][i].y, vb[u][i].z, vb[u][i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[vt_word_t<TK>(dc + 2 * e, kp)] = vt_lo(aw[e], bw[e]);
        Vt[vt_word_t<TK>(dc + 2 * e + 1, kp)] = vt_hi(aw[e], bw[e]);
      }
    }
    lds_barrier();
    if (kt >= n_kt) continue;                      // uniform over the workgroup
    // this wave's keys of the tile: S^T blocks kb = NSB part + j, keys kb*16 + g*4 + i
    f32x4 st[NSB];
#pragma unroll
    for (int j = 0; j < NSB; ++j) {
      const int kb = NSB * part + j;
      st[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 kv = *reinterpret_cast<const uint4*>(Ks + (kb * 16 + ql) * kKStride + c * 32 + g * 8);
        st[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qf[c], st[j], 0, 0, 0);
      }
    }
    // scores stay unscaled: the max is taken on them and scaled once (the
    // scale is positive, so that is the max of the scaled scores exactly),
    // and each probability takes its scale in one fma below
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < NSB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, st[j][i]);
    if (k0 + TK > n) {                            // the tile that crosses n (uniform): mask the keys past it
      tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < NSB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (k0 + (NSB * part + j) * 16 + g * 4 + i >= n) st[j][i] = -INFINITY;
          tmax = fmaxf(tmax, st[j][i]);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    tmax *= scale_log2;
    // Lazy rescale: the reference max m_run of a query moves only when a tile
    // brings a score more than 8 above it, so p = 2^(s - m_run) <= 2^8 (exact
    // range in fp32 and bf16) and O, l stay relative to m_run; the normalised
    // output O / l is the same for any reference.  A wave rescales only when
    // one of its queries moved.  A part that has seen no key keeps m_run =
    // -inf and p = 0.
    const bool grow = tmax > m_run + 8.f;
    const float m_new = grow ? tmax : m_run;
    if (__builtin_amdgcn_ballot_w64(grow)) {      // uniform over the wave
      const float corr = grow ? exp2_fast(m_run - m_new) : 1.f;
      l_run *= corr;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) o[blk] *= corr;
    }
    m_run = m_new;
    // a query that has seen no key yet (m = -inf) has only masked scores
    // here: a finite reference makes each of them 2^-inf = 0
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < NSB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_fast(fmaf(st[j][i], scale_log2, -m_ref));
        st[j][i] = p;
        psum += p;
      }
    l_run += psum;
    if constexpr (NSB == 2) {
      // O^T += V^T P^T over this wave's 32 keys: key pairs 16 part + 2g, +1 (block 0) and 16 part + 8 + 2g, +1
      uint4 pw;
      pw.x = pack_bf16x2(st[0][0], st[0][1]);
      pw.y = pack_bf16x2(st[0][2], st[0][3]);
      pw.z = pack_bf16x2(st[1][0], st[1][1]);
      pw.w = pack_bf16x2(st[1][2], st[1][3]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int dim = blk * 16 + ql;
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[vt_word_t<TK>(dim, part * 16 + g * 2)]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[vt_word_t<TK>(dim, part * 16 + 8 + g * 2)]);
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[blk], 0, 0, 0);
      }
    } else {
      // O^T += V^T P^T over this wave's 16 keys: lane (g, ql) holds keys 4g .. 4g + 3 (key pairs 8 part + 2g, +1)
      uint2 pw;
      pw.x = pack_bf16x2(st[0][0], st[0][1]);
      pw.y = pack_bf16x2(st[0][2], st[0][3]);
      const s16x4 pf = __builtin_bit_cast(s16x4, pw);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int dim = blk * 16 + ql;
        const uint2 vv = *reinterpret_cast<const uint2*>(&Vt[vt_word_t<TK>(dim, part * 8 + g * 2)]);
        o[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pf, o[blk], 0, 0, 0);
      }
    }
  }
  }
  // row sums over the 4 lanes sharing a query
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  lds_barrier();                                  // the last tile's V^T reads are done: reuse the K/V space
  if constexpr (kAllMerge) {
    // every part hands (m, l, O) over; part p then merges dim blocks p * 8 / H .. of its group's queries
    float* mo = reinterpret_cast<float*>(smem);   // [part][grp][blk][g*4 + i][ql]
    const int slot = part * G + grp;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) mo[((slot * 8 + blk) * 16 + g * 4 + i) * 16 + ql] = o[blk][i];
    if (g == 0) {
      merge_ml[slot][ql][0] = m_run;
      merge_ml[slot][ql][1] = l_run;
    }
    lds_barrier();
    if (!qvalid) return;
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < H; ++p) M = fmaxf(M, merge_ml[p * G + grp][ql][0]);
    float w[H], den = 0.f;
#pragma unroll
    for (int p = 0; p < H; ++p) {
      const float mp = merge_ml[p * G + grp][ql][0];
      w[p] = mp == -INFINITY ? 0.f : exp2f(mp - M);
      den += w[p] * merge_ml[p * G + grp][ql][1];
    }
    const float inv = 1.f / den;
    if (lse_rows && part == 0 && g == 0)
      lse_rows[(size_t)(r0 + qrow) * n_heads + h] = (M + log2f(den)) * 0.6931471805599453f;
    uint16_t* orow = out + (size_t)(r0 + qrow) * d + col0;
    constexpr int BPW = 8 / H;
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
      const int blk = part * BPW + bb;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int p = 0; p < H; ++p) acc += w[p] * mo[(((p * G + grp) * 8 + blk) * 16 + g * 4 + i) * 16 + ql];
        v[i] = acc * inv;
      }
      uint2 wv;
      wv.x = pack_bf16x2(v[0], v[1]);
      wv.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(orow + blk * 16 + g * 4) = wv;
    }
    return;
  }
  // parts 1 .. H-1 hand (m, l, O) to part 0's wave of the same group
  float* mo = reinterpret_cast<float*>(smem);     // O^T of parts 1 ..: [part-1][grp][blk][g*4 + i][ql]
  if (part > 0) {
    const int slot = (part - 1) * G + grp;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) mo[((slot * 8 + blk) * 16 + g * 4 + i) * 16 + ql] = o[blk][i];
    if (g == 0) {
      merge_ml[slot][ql][0] = m_run;
      merge_ml[slot][ql][1] = l_run;
    }
  }
  lds_barrier();
  if (part > 0 || !qvalid) return;
  float M = m_run;
#pragma unroll
  for (int p = 1; p < H; ++p) M = fmaxf(M, merge_ml[(p - 1) * G + grp][ql][0]);
  float w[H];
  w[0] = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
  float den = w[0] * l_run;
#pragma unroll
  for (int p = 1; p < H; ++p) {
    const float mp = merge_ml[(p - 1) * G + grp][ql][0];
    w[p] = mp == -INFINITY ? 0.f : exp2f(mp - M);
    den += w[p] * merge_ml[(p - 1) * G + grp][ql][1];
  }
  const float inv = 1.f / den;
  if (lse_rows && g == 0) lse_rows[(size_t)(r0 + qrow) * n_heads + h] = (M + log2f(den)) * 0.6931471805599453f;
  uint16_t* orow = out + (size_t)(r0 + qrow) * d + col0;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = w[0] * o[blk][i];
#pragma unroll
      for (int p = 1; p < H; ++p) s += w[p] * mo[((((p - 1) * G + grp) * 8 + blk) * 16 + g * 4 + i) * 16 + ql];
      v[i] = s * inv;
    }
    uint2 wv;
    wv.x = pack_bf16x2(v[0], v[1]);
    wv.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(orow + blk * 16 + g * 4) = wv;
  }
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
  if (co.lse_rows && col % kDh == 0) co.lse_rows[(size_t)r * n_heads + h] = (M + log2f(L)) * 0.6931471805599453f;
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

#ifndef DTSK_ATTN_ROWS
#define DTSK_ATTN_ROWS 1
#endif
#ifndef DTSK_ATTN_Q16
#define DTSK_ATTN_Q16 1
#endif
#ifndef DTSK_ROWS_AHEAD
#define DTSK_ROWS_AHEAD 2
#endif
#ifndef DTSK_Q16_PARTS
#define DTSK_Q16_PARTS 8
#endif
#ifndef DTSK_Q16_AHEAD
#define DTSK_Q16_AHEAD 3
#endif
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
                            const int32_t* ctx_off, float* lse_out, float* lse_rows, int n_seq) {
  const int d = n_heads * head_dim;
  const float scale = 1.f / sqrtf((float)head_dim);
  const CtxOut co{ctx_out, lse_out, rm.row_pos, ctx_off, lse_rows};
  if (ctx_out && (!lse_out || !ctx_off)) return hipErrorInvalidValue;
  if (ctx_out && lse_rows) return hipErrorInvalidValue;
  if (use_mfma_attention(dt, head_dim)) {
    if (rm.tq != kTQ || rm.T_max <= 0) return rm.T_max < 0 ? hipErrorInvalidValue : hipSuccess;
    if (splits < 1 || splits > kAttnMaxSplits || (splits > 1 && (!o_part || !ml_part || rm.R_max > R_part)))
      return hipErrorInvalidValue;
    const float scale_log2 = scale * 1.4426950408889634f;
    // Every key of a (query rows, head) in one workgroup, with nothing to
    // merge afterwards: 64 queries per workgroup when the query tiles alone
    // give the chip enough workgroups, else 16 (the kept rows of one
    // sequence: 2 tiles x 32 heads x 4); key chunks plus a merge kernel only
    // past kRowsMaxKeys keys or for a context output.
    const long long query_tiles = ((long long)rm.R_max + kTQ - 1) / kTQ;
    if (DTSK_ATTN_ROWS && !ctx_out && S <= kRowsMaxKeys) {
      const int grid = (n_heads + 7) / 8 * 8 * rm.T_max;
      if (query_tiles * n_heads >= kRowsMinBlocks) {
        DTSK_LAUNCH((k_attn_rows<4, 2, DTSK_ROWS_AHEAD, 64>), dim3(grid), dim3(512), 0, st, (const uint16_t*)q, (const uint16_t*)k_cache,
                    (const uint16_t*)v_cache, seq_len, rm.row_seq, rm.tile_row0, rm.tile_rows, S, d, n_heads,
                    scale_log2, rm.T_max, (uint16_t*)out, lse_rows, n_seq == 1);
        return hipGetLastError();
      }
      if (DTSK_ATTN_Q16) {
        DTSK_LAUNCH((k_attn_rows<1, DTSK_Q16_PARTS, DTSK_Q16_AHEAD, DTSK_Q16_PARTS * 16>), dim3(grid * (kTQ / 16)), dim3(DTSK_Q16_PARTS * 64), 0, st, (const uint16_t*)q,
                    (const uint16_t*)k_cache, (const uint16_t*)v_cache, seq_len, rm.row_seq, rm.tile_row0,
                    rm.tile_rows, S, d, n_heads, scale_log2, rm.T_max, (uint16_t*)out, lse_rows, n_seq == 1);
        return hipGetLastError();
      }
    }
    const int chunk = (S + splits * kTK - 1) / (splits * kTK) * kTK;
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
