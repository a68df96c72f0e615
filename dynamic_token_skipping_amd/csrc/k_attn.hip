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

template <typename T>
__global__ __launch_bounds__(kSimtThreads) void k_attn_simt(const T* __restrict__ q, const T* __restrict__ Kc,
                                                            const T* __restrict__ Vc,
                                                            const int32_t* __restrict__ seq_len,
                                                            const int32_t* __restrict__ n_rows,
                                                            const int32_t* __restrict__ row_seq, int S, int d,
                                                            int head_dim, float scale, T* __restrict__ out) {
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
  for (int e = t; e < head_dim; e += blockDim.x) {
    float o = 0.f;
    for (int j = 0; j < n; ++j) o = fmaf(sc[j], to_f32(Vb[(size_t)j * d + e]), o);
    out[(size_t)r * d + col0 + e] = from_f32<T>(o * inv);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDh = 128;          // head_dim of the MFMA kernel
constexpr int kTQ = 64;           // query rows per workgroup (16 per wave)
constexpr int kTK = 64;           // keys per LDS tile
constexpr int kKStride = kDh + 8; // LDS row stride of K (bf16 elements)
constexpr int kVStride = kTK + 8; // LDS row stride of V^T

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)from_f32<bf16_t>(a).u | ((uint32_t)from_f32<bf16_t>(b).u << 16);
}

__global__ __launch_bounds__(256) void k_attn_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
                                                   const uint16_t* __restrict__ Vc,
                                                   const int32_t* __restrict__ seq_len,
                                                   const int32_t* __restrict__ row_seq,
                                                   const int32_t* __restrict__ tile_row0,
                                                   const int32_t* __restrict__ tile_rows, int S, int d,
                                                   float scale_log2, uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint16_t Ks[kTK * kKStride];
  __shared__ __align__(16) uint16_t Vt[kDh * kVStride];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int nrows = tile_rows[tile];
  if (nrows <= 0) return;
  const int r0 = tile_row0[tile];
  const int b = row_seq[r0];
  const int n = seq_len[b];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ql = lane & 15, g = lane >> 4;
  const int qrow = wave * 16 + ql;                 // query row within the tile
  const bool qvalid = qrow < nrows;
  const size_t col0 = (size_t)h * kDh;

  // Q^T fragments (B operand): query ql, dims c*32 + g*8 .. +8
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qvalid) v = *reinterpret_cast<const uint4*>(q + (size_t)(r0 + qrow) * d + col0 + c * 32 + g * 8);
    qf[c] = __builtin_bit_cast(bf16x8, v);
  }

  f32x4 o[8];  // O^T blocks: dims blk*16 + g*4 + i, query ql
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* Kb = Kc + (size_t)b * S * d + col0;
  const uint16_t* Vb = Vc + (size_t)b * S * d + col0;
  for (int k0 = 0; k0 < n; k0 += kTK) {
    lds_barrier();  // previous tile fully consumed
    // K tile: 64 keys x 128 dims, 16 B per thread-chunk
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t + i * 256;
      const int key = c >> 4, dc = (c & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k0 + key < n) v = *reinterpret_cast<const uint4*>(Kb + (size_t)(k0 + key) * d + dc);
      *reinterpret_cast<uint4*>(Ks + key * kKStride + dc) = v;
    }
    // V tile transposed: pairs of keys packed into 32-bit words of V^T[dim][key]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + i * 256;                    // 512 items: 32 key pairs x 16 dim chunks
      const int kp = c >> 4, dc = (c & 15) * 8;
      const int key = kp * 2;
      uint4 a = make_uint4(0, 0, 0, 0), bq = make_uint4(0, 0, 0, 0);
      if (k0 + key < n) a = *reinterpret_cast<const uint4*>(Vb + (size_t)(k0 + key) * d + dc);
      if (k0 + key + 1 < n) bq = *reinterpret_cast<const uint4*>(Vb + (size_t)(k0 + key + 1) * d + dc);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (aw[e] & 0xffffu) | (bw[e] << 16);          // dim dc+2e:   keys key, key+1
        const uint32_t hi = (aw[e] >> 16) | (bw[e] & 0xffff0000u);      // dim dc+2e+1: keys key, key+1
        *reinterpret_cast<uint32_t*>(Vt + (dc + 2 * e) * kVStride + key) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (dc + 2 * e + 1) * kVStride + key) = hi;
      }
    }
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
    // online softmax for query ql over this tile
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kb * 16 + g * 4 + i;
        float v = st[kb][i] * scale_log2;
        if (key >= n) v = -INFINITY;
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
        const uint16_t* vr = Vt + (blk * 16 + ql) * kVStride + c * 32 + g * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[blk], 0, 0, 0);
      }
    }
  }
  // full row sum over the 4 lanes sharing this query
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const float inv = 1.f / l_run;
  uint16_t* orow = out + (size_t)(r0 + qrow) * d + col0;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    uint2 w;
    w.x = pack_bf16x2(o[blk][0] * inv, o[blk][1] * inv);
    w.y = pack_bf16x2(o[blk][2] * inv, o[blk][3] * inv);
    *reinterpret_cast<uint2*>(orow + blk * 16 + g * 4) = w;
  }
}

}  // namespace

static bool use_mfma_attention(dl_dtype dt, int head_dim) { return dt == DL_BF16 && head_dim == kDh; }

bool attention_supported(dl_dtype dt, int S, int head_dim) {
  if (use_mfma_attention(dt, head_dim)) return true;
  return head_dim <= 128 && head_dim % 2 == 0 && S <= kMaxKeysSimt;
}

hipError_t launch_attention(dl_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_len, const RowMap& rm, int S, int n_heads, int head_dim, void* out,
                            hipStream_t st) {
  const int d = n_heads * head_dim;
  const float scale = 1.f / sqrtf((float)head_dim);
  if (use_mfma_attention(dt, head_dim)) {
    if (rm.tq != kTQ) return hipErrorInvalidValue;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL(k_attn_mfma, dim3(rm.T_max, n_heads), dim3(256), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k_cache, (const uint16_t*)v_cache, seq_len, rm.row_seq, rm.tile_row0,
                       rm.tile_rows, S, d, scale_log2, (uint16_t*)out);
    return hipGetLastError();
  }
  dim3 grid(rm.R_max, n_heads);
  if (dt == DL_F32)
    hipLaunchKernelGGL(k_attn_simt<float>, grid, dim3(kSimtThreads), 0, st, (const float*)q, (const float*)k_cache,
                       (const float*)v_cache, seq_len, rm.n_rows, rm.row_seq, S, d, head_dim, scale, (float*)out);
  else
    hipLaunchKernelGGL(k_attn_simt<bf16_t>, grid, dim3(kSimtThreads), 0, st, (const bf16_t*)q,
                       (const bf16_t*)k_cache, (const bf16_t*)v_cache, seq_len, rm.n_rows, rm.row_seq, S, d,
                       head_dim, scale, (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace dtsk
