// Partial attention: the packed query rows of a layer attend over every valid
// key of their own sequence (bidirectional), keys and values read from the
// layer's [B, S, d] caches after the rows' fresh K/V were scattered in.
//
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

}  // namespace

bool attention_supported(dl_dtype dt, int S, int head_dim) {
  (void)dt;
  return head_dim <= 128 && head_dim % 2 == 0 && S <= kMaxKeysSimt;
}

hipError_t launch_attention(dl_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_len, const RowMap& rm, int S, int n_heads, int head_dim, void* out,
                            hipStream_t st) {
  const int d = n_heads * head_dim;
  const float scale = 1.f / sqrtf((float)head_dim);
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
