// Dense products of packed rows with weight matrices: P = A W^T.
//
// A [M, K] holds the packed rows (storage dtype), W [N, K] the weights as
// stored ([out, in]), given as up to four row segments so that Wq|Wk|Wv and
// Wgate|Wup run as one product.  The output is fp32 partial sums, one slice
// per K split, reduced in a fixed order by the epilogue kernels.
//
//  * k_gemm_mfma: bf16 operands on the gfx950 matrix cores
//    (v_mfma_f32_16x16x32_bf16), 256 threads as a 2x2 grid of waves, A and W
//    tiles staged through LDS with a double buffer.
//  * k_gemm_simt: fp32 FMA fallback for fp32 storage and shapes the MFMA
//    tiling does not cover.
#include "launch.h"

namespace dtsk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct WSeg {
  const void* p[4];
};

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Spread consecutive tiles over the 8 XCDs in contiguous runs: hardware hands
// workgroup i to XCD i % 8, so tile t runs on XCD (t / per_xcd).
__device__ __forceinline__ int xcd_swizzle(int bid, int nb) {
  if ((nb & 7) != 0) return bid;
  return (bid & 7) * (nb >> 3) + (bid >> 3);
}

// ---------------------------------------------------------------------------
// MFMA bf16 GEMM
// ---------------------------------------------------------------------------
template <int BM, int BN>
struct MfmaCfg {
  static constexpr int BK = 64;
  static constexpr int LDS_STRIDE = BK + 8;       // bf16 elements per LDS row (16-byte skew)
  static constexpr int WM = BM / 2, WN = BN / 2;  // per-wave tile
  static constexpr int MI = WM / 16, NI = WN / 16;
  static constexpr int A_CHUNKS = BM * BK / 8 / 256;  // uint4 loads per thread
  static constexpr int W_CHUNKS = BN * BK / 8 / 256;
  static constexpr int LDS_BYTES = 2 * (BM + BN) * LDS_STRIDE * 2;
};

template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_mfma(const uint16_t* __restrict__ A, int M_max,
                                                   const int32_t* __restrict__ n_rows, int m_base, int K, WSeg W,
                                                   int n_seg,
                                                   int N, int k_per_split, int n_mt, int n_nt,
                                                   float* __restrict__ P) {
  using C = MfmaCfg<BM, BN>;
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* As = lds;                                   // [2][BM][LDS_STRIDE]
  uint16_t* Ws = lds + 2 * BM * C::LDS_STRIDE;          // [2][BN][LDS_STRIDE]

  const int bid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int mt = bid % n_mt;
  const int nt = (bid / n_mt) % n_nt;
  const int split = bid / (n_mt * n_nt);
  const int M = min(*n_rows - m_base, M_max);
  const int m0 = mt * BM;
  if (m0 >= M) return;
  const int n0 = nt * BN;
  const int k_begin = split * k_per_split;
  const int k_end = min(K, k_begin + k_per_split);
  const int nk = (k_end - k_begin) / C::BK;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm0 = (wave >> 1) * C::WM, wn0 = (wave & 1) * C::WN;

  // global -> register staging
  uint4 ra[C::A_CHUNKS], rw[C::W_CHUNKS];
  auto load_tiles = [&](int kt) {
    const int kb = k_begin + kt * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int c = t + i * 256;
      const int row = c >> 3, kc = (c & 7) * 8;
      const int m = m0 + row;
      if (m < M)
        ra[i] = *reinterpret_cast<const uint4*>(A + (size_t)m * K + kb + kc);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::W_CHUNKS; ++i) {
      const int c = t + i * 256;
      const int row = c >> 3, kc = (c & 7) * 8;
      const int n = n0 + row;
      const int sg = n / n_seg;
      const uint16_t* wp = reinterpret_cast<const uint16_t*>(W.p[sg]) + (size_t)(n - sg * n_seg) * K;
      rw[i] = *reinterpret_cast<const uint4*>(wp + kb + kc);
    }
  };
  auto store_tiles = [&](int buf) {
    uint16_t* a = As + buf * BM * C::LDS_STRIDE;
    uint16_t* w = Ws + buf * BN * C::LDS_STRIDE;
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int c = t + i * 256;
      *reinterpret_cast<uint4*>(a + (c >> 3) * C::LDS_STRIDE + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::W_CHUNKS; ++i) {
      const int c = t + i * 256;
      *reinterpret_cast<uint4*>(w + (c >> 3) * C::LDS_STRIDE + (c & 7) * 8) = rw[i];
    }
  };

  f32x4 acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
    const uint16_t* a = As + buf * BM * C::LDS_STRIDE;
    const uint16_t* w = Ws + buf * BN * C::LDS_STRIDE;
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const int koff = ks * 32 + (lane >> 4) * 8;
      bf16x8 fa[C::MI], fb[C::NI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(a + (wm0 + i * 16 + (lane & 15)) * C::LDS_STRIDE + koff);
        fa[i] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < C::NI; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(w + (wn0 + j * 16 + (lane & 15)) * C::LDS_STRIDE + koff);
        fb[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // C fragment: lane holds rows (lane/16)*4 + e, column lane%16 of each 16x16 block
  float* Pout = P + (size_t)split * M_max * N;
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm0 + i * 16 + (lane >> 4) * 4 + e;
        const int n = n0 + wn0 + j * 16 + (lane & 15);
        if (m < M) Pout[(size_t)m * N + n] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// SIMT fallback: 64x64 tile, 4x4 outputs per thread, fp32 FMA
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_gemm_simt(const T* __restrict__ A, int M_max,
                                                   const int32_t* __restrict__ n_rows, int m_base, int K, WSeg W,
                                                   int n_seg, int N, float* __restrict__ P) {
  constexpr int TB = 64, BK = 16;
  __shared__ float As[BK][TB + 4];
  __shared__ float Ws[BK][TB + 4];
  const int M = min(*n_rows - m_base, M_max);
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  if (m0 >= M) return;
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int c = t; c < TB * BK; c += 256) {
      const int row = c / BK, kk = c % BK;
      const int m = m0 + row, n = n0 + row, k = k0 + kk;
      float av = 0.f, wv = 0.f;
      if (m < M && k < K) av = to_f32(A[(size_t)m * K + k]);
      if (n < N && k < K) {
        const int sg = n / n_seg;
        wv = to_f32(reinterpret_cast<const T*>(W.p[sg])[(size_t)(n - sg * n_seg) * K + k]);
      }
      As[kk][row] = av;
      Ws[kk][row] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        w[i] = Ws[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) P[(size_t)m * N + n] = acc[i][j];
    }
}

constexpr int kBM = 128, kBN = 128;

}  // namespace

GemmPlan plan_gemm(dl_dtype dt, int M, int N, int K) {
  GemmPlan p{1, 0};
  if (dt == DL_BF16 && K % 64 == 0 && N % kBN == 0) {
    p.kind = 1;
    // Split K until the grid covers the 256 CUs about once (at most 8 ways,
    // each split a whole number of 64-wide K steps).
    const int tiles = cdiv(M, kBM) * (N / kBN);
    int s = 1;
    while (tiles * s < 256 && s < 8 && (K / 64) % (s * 2) == 0) s *= 2;
    p.splits = s;
  }
  return p;
}

hipError_t launch_gemm(dl_dtype dt, const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows,
                       int m_base, int K, const void* const* Wseg, int n_seg, int N, float* P, hipStream_t st) {
  WSeg w;
  for (int i = 0; i < 4; ++i) w.p[i] = Wseg[i];
  if (M_max <= 0) return hipSuccess;
  if (plan.kind == 1) {
    using C = MfmaCfg<kBM, kBN>;
    static bool attr_set = false;  // the tile needs more than the default 64 KiB of LDS
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)k_gemm_mfma<kBM, kBN>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const int n_mt = cdiv(M_max, kBM), n_nt = N / kBN;
    const int kps = K / plan.splits;
    const int grid = n_mt * n_nt * plan.splits;
    hipLaunchKernelGGL((k_gemm_mfma<kBM, kBN>), dim3(grid), dim3(256), C::LDS_BYTES, st, (const uint16_t*)A, M_max,
                       n_rows, m_base, K, w, n_seg, N, kps, n_mt, n_nt, P);
  } else {
    dim3 grid(cdiv(N, 64), cdiv(M_max, 64));
    if (dt == DL_F32)
      hipLaunchKernelGGL(k_gemm_simt<float>, grid, dim3(256), 0, st, (const float*)A, M_max, n_rows, m_base, K, w,
                         n_seg, N, P);
    else
      hipLaunchKernelGGL(k_gemm_simt<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)A, M_max, n_rows, m_base, K, w,
                         n_seg, N, P);
  }
  return hipGetLastError();
}

}  // namespace dtsk
