// Dense products of packed rows with weight matrices, C = A W^T, with the
// consumer's epilogue fused in.
//
// A [M, K] holds the packed rows (storage dtype), W [N, K] the weights as
// stored ([out, in]).  Weights may be given as up to four row segments so
// that Wq|Wk|Wv run as one product (segmented: segment = n / n_seg), and
// Wgate|Wup as one product whose every column tile holds gate rows in its
// first half and the matching up rows in its second half (interleaved), so
// that SwiGLU needs nothing outside the tile.  On up to 128 rows the gate|up
// product is cut into exactly one column tile per compute unit, each holding
// d_ffn / 256 gate rows and the matching up rows (ragged, the rest of the
// tile empty), so that every unit streams the same share of the weights.
//
//  * k_gemm_skinny (bf16, M <= 128): the weight-streaming regime.  Each of
//    the 4 waves owns BN/4 output columns for all M rows; its weight rows go
//    from HBM straight into a ring of registers kDepth 64-wide K steps ahead
//    (v_mfma_f32_16x16x32_bf16 B operand layout), while the A rows of each K
//    step are staged once per workgroup in LDS (double buffer).
//  * k_gemm_mfma<BN, BM, waves, depth> (bf16): BM x BN tiles, A and W
//    through LDS; 128 x 128 for many rows, 128 x 64 for up to 128 rows (twice
//    the column tiles), 256-row tiles with 8 waves for gate|up (192-wide
//    ragged tiles) and the split-K products on 257..512 rows, 128 x 256
//    tiles with 16 waves for the LM head.
//  * k_gemm_simt: fp32 FMA fallback (fp32 storage, odd shapes); its results
//    go through the separate epilogue kernels of k_rows.
//
// Products whose epilogue needs only the tile's own columns (QKV + RoPE + K/V
// scatter, gate/up + SwiGLU, LM-head statistics) run without a K split: the
// finished tile goes to LDS and the workgroup applies the epilogue.  Products
// with too few column tiles (the d x d and d x F projections) split K and
// write fp32 partials; a row kernel then sums the splits in split order and
// applies residual + RMSNorm.  No workgroup waits on another one.
#include "launch.h"

namespace dtsk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Weight row of output column n.
//  mode 0 segmented:   segment n / n_seg, row n % n_seg
//  mode 1 interleaved: each BN-wide tile holds rows [t*BN/2, (t+1)*BN/2) of
//                      segment 0 then the same rows of segment 1 (gate | up)
//  mode 2 rope pairs:  segmented, and inside each 128-row head a 64-wide tile
//                      holds dims [32p, 32p+32) then [64+32p, 64+32p+32), so
//                      that RoPE partners j and j+64 share the tile
//  mode 3 ragged interleaved: the n_seg rows of each of the two segments are
//                      cut into n_tiles runs, run t = [t*n_seg/n_tiles,
//                      (t+1)*n_seg/n_tiles) of at most BN/2 rows; tile t holds
//                      run t of segment 0 from column 0 and run t of segment 1
//                      from column BN/2; the columns past each run are empty
//                      (their weights read as zeros).  With n_tiles = the
//                      compute units, every unit streams the same share.
struct WMap {
  const void* p[4];
  int mode;
  int n_seg;
  int seg_bytes;  // bytes of one segment (buffer range of the skinny path)
  int n_tiles;    // mode 3: column tiles
  int blocked;    // 1: segments in 8-row x 64-input blocks (DL_WEIGHTS_BLOCKED)
};

// Byte offset of element (r, k) in a bf16 weight segment of K inputs per row.
// Row-major: (r K + k) 2.  Blocked: 8 x 64 blocks of 1 KB, an 8-row group's
// blocks in K order: ((r / 8) (K / 64) + k / 64) 1024 + (r % 8) 128 + (k % 64) 2.
// Within a block the 64 inputs of a row are contiguous, so the 16-byte pieces
// of one 64-wide K step sit at the same offsets in both orders; a K step moves
// a row's offset by w_step bytes.
__device__ __forceinline__ uint32_t w_offset(bool blocked, int r, int k, int K) {
  return blocked ? (uint32_t)((((r >> 3) * (K >> 6) + (k >> 6)) << 10) + ((r & 7) << 7) + ((k & 63) << 1))
                 : (uint32_t)((r * K + k) * 2);
}
__device__ __forceinline__ uint32_t w_step(bool blocked) { return blocked ? 1024u : 128u; }

// Mode 3: the rows [a, a + h) of each segment that tile t holds.
__device__ __forceinline__ void ragged_run(const WMap& w, int t, int& a, int& h) {
  if ((unsigned)w.n_seg < (1u << 23) && (unsigned)w.n_tiles <= 256u) {   // (t + 1) n_seg < 2^31
    a = (int)((unsigned)t * (unsigned)w.n_seg / (unsigned)w.n_tiles);
    h = (int)((unsigned)(t + 1) * (unsigned)w.n_seg / (unsigned)w.n_tiles) - a;
    return;
  }
  a = (int)((long long)t * w.n_seg / w.n_tiles);
  h = (int)((long long)(t + 1) * w.n_seg / w.n_tiles) - a;
}

// r < 0: an empty column of a mode 3 tile.
template <int BN>
__device__ __forceinline__ void wrow_index(const WMap& w, int n, int& sg, int& r) {
  if (w.mode == 3) {
    const int c = n % BN;
    int a, h;
    ragged_run(w, n / BN, a, h);
    sg = c / (BN / 2);
    const int j = c % (BN / 2);
    r = j < h ? a + j : -1;
    return;
  }
  if (w.mode == 1) {
    const int c = n % BN;
    sg = c / (BN / 2);
    r = (n / BN) * (BN / 2) + c % (BN / 2);
    return;
  }
  sg = n / w.n_seg;
  r = n - sg * w.n_seg;
  if (w.mode == 2) {      // 64-wide tiles inside 128-dim heads
    const int head = r >> 7, part = (r >> 6) & 1, c = r & 63;
    r = head * 128 + (c >> 5) * 64 + part * 32 + (c & 31);
  }
}

template <int BN>
__device__ __forceinline__ const uint16_t* wrow(const WMap& w, int n, int K) {
  int sg, r;
  wrow_index<BN>(w, n, sg, r);
  return reinterpret_cast<const uint16_t*>(w.p[sg]) + (size_t)r * K;
}

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// fused epilogues on a finished tile held in LDS: T[m][c], rows [0, M),
// tile columns c whose output column is n0 + c in W-map order
// ---------------------------------------------------------------------------
// SWIGLU_ONLY: a tile shape that only gate|up products use (the other
// branches are left out of its code).
template <int BN, int TS, int NT = 256, int MAXM = 128, bool SWIGLU_ONLY = false>
__device__ __forceinline__ void tile_epilogue(const Epilogue& e, float* __restrict__ T, const WMap& w, int n0, int M) {
  const int t = threadIdx.x;
  if (SWIGLU_ONLY || e.kind == EPI_SWIGLU) {   // modes 1, 3: gate in [0, BN/2), up in [BN/2, BN)
    constexpr int H = BN / 2;
    int a = (n0 / BN) * H, h = H;         // the tile's inner columns [a, a + h)
    if (w.mode == 3) ragged_run(w, n0 / BN, a, h);
    uint16_t* out = reinterpret_cast<uint16_t*>(e.act_out);
    // one column per lane, the rows over the waves: no division in the loop.
    // silu(g) = g / (1 + 2^(-g log2 e)) through the hardware exp2 and
    // reciprocal (about 1 ulp each, far below the bf16 rounding of the output)
    static_assert(NT % 64 == 0, "whole waves");
    for (int c = t & 63; c < h; c += 64)
#pragma unroll 4
      for (int m = t >> 6; m < M; m += NT / 64) {
        const float gt = T[m * TS + c], up = T[m * TS + H + c];
        const float sg = gt * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(gt * -1.4426950408889634f));
        out[(size_t)m * e.F + a + c] = from_f32<bf16_t>(sg * up).u;
      }
    return;
  }
  if constexpr (SWIGLU_ONLY) return;
  if (e.kind == EPI_QKV) {
    int sg, r0;
    wrow_index<BN>(w, n0, sg, r0);                  // segment of the tile: 0 q, 1 k, 2 v
    const int hd = e.head_dim, half = hd / 2;
    // each row's cache position and sequence position, read once into the
    // tile's padding columns, so that the loops below issue no dependent loads
    int* Ti = reinterpret_cast<int*>(T);
    for (int m = t; m < M; m += NT) {
      const int p = e.row_pos[m];
      Ti[m * TS + BN] = p;
      Ti[m * TS + BN + 1] = p - e.row_seq[m] * e.S;
    }
    lds_barrier();
    if constexpr (BN == 192) {
      if (w.mode == 2 && hd == 128) {
        // Rope-pair tile of several 64-column groups: group g holds dims
        // r0_g + [0, 32) and r0_g + 64 + [0, 32) of one head of its own
        // segment (a tile may cross from q to k or k to v between groups).
        // Pair p of the tile: group p / 32, columns (64 g + i, 64 g + 32 + i),
        // i = p % 32, rows r0_g + i and r0_g + i + 64.
        constexpr int NG = BN / 64, NP = BN / 2;
        constexpr int kIt = (MAXM * NP + NT - 1) / NT;
        int gsg[NG], gr0[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) wrow_index<BN>(w, n0 + g * 64, gsg[g], gr0[g]);
        float2 cs[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {            // every rotation factor first: independent loads
          const int idx = t + it * NT;
          cs[it] = make_float2(1.f, 0.f);
          if (idx < M * NP) {
            const int m = idx / NP, pr = idx - m * NP, g = pr >> 5;
            if (gsg[g] != 2) cs[it] = e.rope[Ti[m * TS + BN + 1] * half + (gr0[g] + (pr & 31)) % hd];
          }
        }
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
          const int idx = t + it * NT;
          if (idx < M * NP) {
            const int m = idx / NP, pr = idx - m * NP, g = pr >> 5, i = pr & 31;
            const int c1 = g * 64 + i, r1 = gr0[g] + i;
            const float a = T[m * TS + c1], b = T[m * TS + c1 + 32];
            const size_t pos = (size_t)Ti[m * TS + BN];
            if (gsg[g] == 2) {
              uint16_t* vc = reinterpret_cast<uint16_t*>(e.v_cache) + pos * e.d;
              vc[r1] = from_f32<bf16_t>(a).u;
              vc[r1 + half] = from_f32<bf16_t>(b).u;
            } else {
              uint16_t* dst = reinterpret_cast<uint16_t*>(gsg[g] == 0 ? e.q_out : e.k_cache) +
                              (gsg[g] == 0 ? (size_t)m * e.d : pos * e.d);
              dst[r1] = from_f32<bf16_t>(a * cs[it].x - b * cs[it].y).u;
              dst[r1 + half] = from_f32<bf16_t>(b * cs[it].x + a * cs[it].y).u;
            }
          }
        }
        return;
      }
    }
    // Fast column map: a 64-wide rope-pair tile (mode 2) holds dims r0 + [0, 32)
    // and r0 + 64 + [0, 32) of one head; a BN-wide segmented tile with
    // head_dim == BN holds one whole head r0 + [0, BN).  Other shapes take the
    // general map.
    const bool fast = (w.mode == 2 && BN == 64 && hd == 128) || (w.mode == 0 && hd == BN);
    if (sg == 2) {
      uint16_t* vc = reinterpret_cast<uint16_t*>(e.v_cache);
      for (int idx = t; idx < M * BN; idx += NT) {
        const int m = idx / BN, c = idx % BN;
        int r;
        if (fast) {
          r = w.mode == 2 ? r0 + ((c >> 5) << 6) + (c & 31) : r0 + c;
        } else {
          int s2;
          wrow_index<BN>(w, n0 + c, s2, r);
        }
        vc[(size_t)Ti[m * TS + BN] * e.d + r] = from_f32<bf16_t>(T[m * TS + c]).u;
      }
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(sg == 0 ? e.q_out : e.k_cache);
      constexpr int kIt = (MAXM * (BN / 2) + NT - 1) / NT;   // pairs per thread
      // pair pr: tile columns (c1, c2) and the weight row r1 of c1 (dim j = r1 % hd
      // of its head; the partner dim is j + half)
      auto pair_map = [&](int pr, int& c1, int& c2, int& r1) {
        if (fast) {
          c1 = pr;
          c2 = pr + BN / 2;
          r1 = r0 + pr;
          return;
        }
        if (w.mode == 2) {
          c1 = pr;
          c2 = pr + BN / 2;
        } else {
          c1 = (pr / half) * hd + pr % half;
          c2 = c1 + half;
        }
        int s2;
        wrow_index<BN>(w, n0 + c1, s2, r1);
      };
      const int j0 = fast ? r0 % hd : 0;
      float2 cs[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it) {            // every rotation factor first: independent loads
        const int idx = t + it * NT;
        cs[it] = make_float2(1.f, 0.f);
        if (idx < M * (BN / 2)) {
          const int m = idx / (BN / 2), pr = idx % (BN / 2);
          int c1, c2, r1;
          pair_map(pr, c1, c2, r1);
          const int j = fast ? j0 + pr : r1 % hd;
          cs[it] = e.rope[Ti[m * TS + BN + 1] * half + j];
        }
      }
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int idx = t + it * NT;
        if (idx < M * (BN / 2)) {
          const int m = idx / (BN / 2), pr = idx % (BN / 2);
          int c1, c2, r1;
          pair_map(pr, c1, c2, r1);
          const float a = T[m * TS + c1], b = T[m * TS + c2];
          const float o1 = a * cs[it].x - b * cs[it].y, o2 = b * cs[it].x + a * cs[it].y;
          const size_t rowoff = sg == 0 ? (size_t)m * e.d : (size_t)Ti[m * TS + BN] * e.d;
          dst[rowoff + r1] = from_f32<bf16_t>(o1).u;
          dst[rowoff + r1 + half] = from_f32<bf16_t>(o2).u;
        }
      }
    }
  } else if (e.kind == EPI_LM) {
    // per row: (max, sum exp(l - max), lowest argmax) over this tile's columns
    const int lane = t & 63, wave = t >> 6;
    const int tile = n0 / BN;
    for (int m = wave; m < M; m += NT / 64) {
      float mx = -INFINITY, sm = 0.f;
      int am = 0x7fffffff;
      for (int c = lane; c < BN; c += 64) {
        const float l = T[m * TS + c];
        if (e.logits) e.logits[(size_t)e.row_pos[m] * e.V + n0 + c] = l;
        if (l > mx) {
          sm = sm * expf(mx - l) + 1.f;
          mx = l;
          am = n0 + c;
        } else {
          sm += expf(l - mx);
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(sm, o, 64);
        const int a2 = __shfl_xor(am, o, 64);
        const float mn = fmaxf(mx, m2);
        const float sn = (mx == -INFINITY ? 0.f : sm * expf(mx - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
        am = (m2 > mx || (m2 == mx && a2 < am)) ? a2 : am;
        mx = mn;
        sm = sn;
      }
      if (lane == 0)
        reinterpret_cast<float4*>(e.lm_part)[(size_t)m * e.lm_tiles + tile] =
            make_float4(mx, sm, __int_as_float(am), 0.f);
    }
  }
}

// Workgroup order: the splits of one column tile get block ids that are equal
// mod 8, i.e. run on the same XCD (hardware deals block i to XCD i % 8), so
// that they share the rows of A in that XCD's L2.
__device__ __forceinline__ void tile_of_block(int bid, int splits, int& tile, int& split) {
  const int xcd = bid & 7, r = bid >> 3;
  split = r % splits;
  tile = (r / splits) * 8 + xcd;
}

// Tiled kernel: which (row tile, column tile, K split) block `bid` computes
// (hardware deals block i to XCD i % 8).
//  * Without a K split, column tile nt runs on XCD nt % 8, and the row tiles
//    of one column tile get consecutive block ids there, so they run together
//    and read that column tile's weights through one L2.
//  * With a K split in 2, 4 or 8, XCD x takes split x % splits only, for every
//    (8 / splits)-th column tile: each XCD's L2 then holds the rows of A of one
//    K range, not all of them (with the splits of a column tile on one XCD,
//    every XCD fetched the whole of A).
__device__ __forceinline__ bool split_major(int splits) { return splits > 1 && 8 % splits == 0; }

__device__ __forceinline__ void tile_of_block_mn(int bid, int n_mt, int splits, int& mt, int& nt, int& split) {
  const int xcd = bid & 7, r = bid >> 3;
  if (split_major(splits)) {
    split = xcd % splits;
    mt = r % n_mt;
    nt = (r / n_mt) * (8 / splits) + xcd / splits;
    return;
  }
  const int per_nt = n_mt * splits;
  const int q = r / per_nt, rem = r - q * per_nt;
  nt = q * 8 + xcd;
  mt = rem / splits;
  split = rem - mt * splits;
}

// ---------------------------------------------------------------------------
// skinny weight-streaming GEMM (M <= 16 * MI <= 128)
// ---------------------------------------------------------------------------
constexpr uint32_t kOob = 0x80000000u;   // byte offset past every buffer (< 2 GiB each)
#ifndef DTSK_SKINNY_DEPTH
#define DTSK_SKINNY_DEPTH 4
#endif
#ifndef DTSK_LARGE_DEPTH
#define DTSK_LARGE_DEPTH 4
#endif
#ifndef DTSK_LDS_SWIZZLE
#define DTSK_LDS_SWIZZLE 1
#endif
#ifndef DTSK_TILED_SMALL
#define DTSK_TILED_SMALL 1
#endif
// the tiled kernel from this many rows up (fewer go to the skinny kernel)
#ifndef DTSK_TILED_MIN_ROWS
#define DTSK_TILED_MIN_ROWS 32
#endif
#ifndef DTSK_T128_MIN_TILES
#define DTSK_T128_MIN_TILES 160
#endif
// the LM head on up to 128 rows through the tiled kernel (else the skinny one)
#ifndef DTSK_TILED_LM
#define DTSK_TILED_LM 1
#endif
#ifndef DTSK_QKV_SPLIT
#define DTSK_QKV_SPLIT 1
#endif
#ifndef DTSK_RAGGED
#define DTSK_RAGGED 1
#endif
#ifndef DTSK_KROT
#define DTSK_KROT 1
#endif
// products on more than 256 rows through 256-row tiles
#ifndef DTSK_BIG_TILES
#define DTSK_BIG_TILES 1
#endif
#ifndef DTSK_LM256
#define DTSK_LM256 1
#endif
#ifndef DTSK_LM_NW
#define DTSK_LM_NW 16
#endif
// waves and register-ring depth of the 128-row tiles on up to 128 rows
#ifndef DTSK_SMALL_NW
#define DTSK_SMALL_NW 8
#endif
#ifndef DTSK_SMALL_NW128
#define DTSK_SMALL_NW128 DTSK_SMALL_NW
#endif
#ifndef DTSK_GU96
#define DTSK_GU96 1
#endif
#ifndef DTSK_QKV96
#define DTSK_QKV96 1
#endif
#ifndef DTSK_QKV192
#define DTSK_QKV192 1
#endif
// the tiled kernel skips the fragment reads and MFMAs of padding K steps
#ifndef DTSK_SKIP_PAD
#define DTSK_SKIP_PAD 1
#endif
// weights of the tiled products loaded with the non-temporal hint
#ifndef DTSK_W_NT
#define DTSK_W_NT 1
#endif
#ifndef DTSK_SMALL_DEPTH
#define DTSK_SMALL_DEPTH 4
#endif
// waves of the 128 x 128 tiles on more than 128 rows
#ifndef DTSK_MID_NW
#define DTSK_MID_NW 8
#endif
#ifndef DTSK_BIG_NW128
#define DTSK_BIG_NW128 8
#endif
#ifndef DTSK_BIG_DEPTH192
#define DTSK_BIG_DEPTH192 3
#endif


// K-step order of a tile.  Weight rows are K*2 bytes apart (a power of two in
// the 8B-class shapes); if every tile walked K from the same start, all of
// them would address the same low address bits at the same time.  Starting
// each tile at its own K step spreads the requests over the HBM channels.
// The order is a fixed function of the tile, so results stay deterministic.
__device__ __forceinline__ int k_rotation(int tile, int nk) {
#if DTSK_KROT
  return nk > 0 ? (int)(((unsigned)tile * 2654435761u) >> 16) % nk : 0;
#else
  return 0;
#endif
}
constexpr int kDepth = DTSK_SKINNY_DEPTH;      // 64-wide K steps fetched ahead (even)
constexpr int kDepthL = DTSK_LARGE_DEPTH;
constexpr int kBigDepth192 = DTSK_BIG_DEPTH192;   // register ring of the 256 x 192 tile
static_assert(kDepth % 2 == 0, "the skinny kernel's LDS double buffer needs an even pipeline depth");

// LDS layout of a 64-wide bf16 K step: row r, 16-byte chunk c.  With the XOR
// swizzle a row is 128 bytes and chunk c lives in slot c ^ ((r >> 1) & 7):
// 16 lanes reading one chunk of 16 consecutive rows, or 8 lanes writing the 8
// chunks of a row, touch 16 (8) distinct 16-byte slots of the 256-byte bank
// row.  Without it rows are padded to 144 bytes.
#if DTSK_LDS_SWIZZLE
constexpr int kRowElems = 64;
__device__ __forceinline__ int lds_idx(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }
#else
constexpr int kRowElems = 72;
__device__ __forceinline__ int lds_idx(int r, int c) { return r * 72 + (c << 3); }
#endif

// The K steps of a split are padded up to a multiple of kDepth; padding steps
// and rows >= M read through out-of-range buffer offsets, which return zeros
// without a memory access, so the pipeline below has no data-dependent
// branches and every wait on the load counter is exact.
template <int MI, int BN>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t* __restrict__ A, int M_max,
                                                     const int32_t* __restrict__ n_rows, int m_base, int K, WMap W,
                                                     int N, int splits, int n_nt, float* __restrict__ P,
                                                     Epilogue epi) {
  constexpr int NB = BN / 64;               // 16-column blocks per wave
  constexpr int MP = MI * 16;               // padded rows
  constexpr int AS = kRowElems;             // LDS row stride (bf16)
  constexpr int A_ITEMS = MP * 8;           // 16-byte items per A step
  constexpr int AP = (A_ITEMS + 255) / 256; // A items per thread per step
  constexpr int TS = BN + 4;                // LDS row stride of the finished tile (fp32)
  constexpr int A_BYTES = 2 * MP * AS * 2, T_BYTES = MP * TS * 4;
  __shared__ __align__(16) char lds_raw[A_BYTES > T_BYTES ? A_BYTES : T_BYTES];
  uint16_t (*As)[MP * AS] = reinterpret_cast<uint16_t (*)[MP * AS]>(lds_raw);

  int tile, split;
  tile_of_block(blockIdx.x, splits, tile, split);
  if (tile >= n_nt) return;
  const int M = min(*n_rows - m_base, M_max);
  if (M <= 0) return;
  const int n0 = tile * BN;
  const int nk_all = K / 64;
  const int ks0 = split * nk_all / splits, ks1 = (split + 1) * nk_all / splits;
  const int nk = ks1 - ks0;
  const int nk_pad = (nk + kDepth - 1) / kDepth * kDepth;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, l16 = lane & 15;

  // weight rows of this wave: 16-row runs inside one segment (the planner
  // checks the tiling); rows of block nb are row0[nb] + l16
  const int ncol0 = n0 + wave * (BN / 4);
  int seg, row0[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wrow_index<BN>(W, ncol0 + nb * 16, seg, row0[nb]);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(W.p[seg]), (short)0,
                                                                      W.seg_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), (short)0,
                                                                      M * K * 2, kBufWord3);
  uint32_t woff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) woff[nb] = w_offset(W.blocked, row0[nb] + l16, ks0 * 64 + g * 8, K);
  const uint32_t wst = w_step(W.blocked);
  uint32_t aoff[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    const int c = t + i * 256;
    aoff[i] = (uint32_t)((((c >> 3) * K) + ks0 * 64 + (c & 7) * 8) * 2);
  }

  uint4 ring[kDepth][NB][2];
  uint4 aring[kDepth][AP];
  const int rot = k_rotation(tile, nk);
  auto issue = [&](int step, uint4 (&w)[NB][2], uint4 (&a)[AP]) {
    const bool in = step < nk;
    const int sr = step + rot >= nk ? step + rot - nk : step + rot;
    const uint32_t ks = (uint32_t)sr * 128u, ksw = (uint32_t)sr * wst;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t o = in ? woff[nb] + ksw : kOob;
      w[nb][0] = DTSK_W_NT ? buf_load16_nt(wr, o) : buf_load16(wr, o);
      w[nb][1] = DTSK_W_NT ? buf_load16_nt(wr, in ? o + 64u : kOob) : buf_load16(wr, in ? o + 64u : kOob);
    }
#pragma unroll
    for (int i = 0; i < AP; ++i) a[i] = buf_load16(ar, in ? aoff[i] + ks : kOob);
  };
  auto store_a = [&](int buf, const uint4 (&a)[AP]) {
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int c = t + i * 256;
      if (A_ITEMS % 256 == 0 || c < A_ITEMS) *reinterpret_cast<uint4*>(&As[buf][lds_idx(c >> 3, c & 7)]) = a[i];
    }
  };

  f32x4 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < kDepth - 1; ++s) issue(s, ring[s], aring[s]);
  store_a(0, aring[0]);
  lds_barrier();

  for (int kt = 0; kt < nk_pad; kt += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      issue(kt + u + kDepth - 1, ring[(u + kDepth - 1) % kDepth], aring[(u + kDepth - 1) % kDepth]);
      const uint16_t* a = As[u & 1];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const uint4 av = *reinterpret_cast<const uint4*>(a + lds_idx(i * 16 + l16, kc * 4 + g));
          const bf16x8 fa = __builtin_bit_cast(bf16x8, av);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8, ring[u][nb][kc]),
                                                                 acc[i][nb], 0, 0, 0);
        }
      }
      store_a((u + 1) & 1, aring[(u + 1) % kDepth]);
      lds_barrier();
    }
  }

  // C fragment: rows i*16 + g*4 + r, column l16 of each 16-column block
  if (epi.kind == EPI_NONE) {              // partial sums of this split
    float* Ps = P + (size_t)split * M_max * N;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = i * 16 + g * 4 + r;
          if (m < M) Ps[(size_t)m * N + n0 + wave * (BN / 4) + nb * 16 + l16] = acc[i][nb][r];
        }
    return;
  }
  float* T = reinterpret_cast<float*>(lds_raw);   // the A buffers are free after the last barrier
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) T[(i * 16 + g * 4 + r) * TS + wave * (BN / 4) + nb * 16 + l16] = acc[i][nb][r];
  lds_barrier();
  tile_epilogue<BN, TS, 256, MP>(epi, T, W, n0, M);
}

// ---------------------------------------------------------------------------
// register-tiled GEMM for few rows (M <= 16 * MI <= 128): the 4 waves of a
// workgroup split the K steps of the tile (wave w takes steps w, w+4, ...);
// each wave loads its A-row and weight fragments straight into registers
// (B/A operand layouts of v_mfma_f32_16x16x32_bf16) with no LDS traffic and
// no barrier in the main loop, every A fragment feeding NBW products and
// every weight fragment MI.  The four partial tiles are summed through LDS
// in wave order at the end.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Tiled MFMA GEMM: BM-row x BN-column tiles.  BM = 128 with 4 waves (2 x 2,
// each 64 x BN/2), or BM = 256 with 8 waves (4 x 2, each 64 x BN/2) for
// products on more than 256 rows, where the larger tile halves the weight
// re-reads per output.  A and W tiles go through LDS (double buffer),
// fetched DEPTH - 1 steps ahead into register rings with buffer loads (rows
// >= M and padding steps read as zeros).
// ---------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kBigBM = 256, kBigWaves = 8;   // the 256-row tile
constexpr int kRaggedTiles = 256;   // ragged column tiles: one per compute unit
constexpr int kBigRagged = 128;     // ragged gate|up tiles of the 256-row tile
constexpr int kLds = kRowElems;
// rows of the finished tile that one epilogue pass stages in LDS
template <int BM>
constexpr int epi_rows() { return BM > 128 ? 128 : BM; }
// dynamic LDS of the tiled kernel: the A/W double buffers, or one epilogue
// pass of the finished fp32 tile, whichever is larger
// W tile rows in LDS: BN rounded up to whole load items of NW waves (8 rows
// per wave), so that a partial last item stores unconditionally (its rows
// past BN are never read)
template <int BN, int NW>
constexpr int w_lds_rows() { return (BN + NW * 8 - 1) / (NW * 8) * (NW * 8); }
template <int BN, int BM, int NW>
constexpr int large_lds() {
  return 2 * (BM + w_lds_rows<BN, NW>()) * kLds * 2 > epi_rows<BM>() * (BN + 4) * 4
             ? 2 * (BM + w_lds_rows<BN, NW>()) * kLds * 2
             : epi_rows<BM>() * (BN + 4) * 4;
}

// WNT: weights loaded with the non-temporal hint (for products whose weight
// tiles are read by few row tiles; with many, the L2 copy serves the others)
template <int BN, int BM, int NW, int DEPTH, bool WNT = true>
__global__ __launch_bounds__(NW * 64) void k_gemm_mfma(const uint16_t* __restrict__ A, int M_max,
                                                       const int32_t* __restrict__ n_rows, int m_base, int K, WMap W,
                                                       int N, int splits, int n_mt, int n_nt, float* __restrict__ P,
                                                       Epilogue epi) {
  constexpr int NT = NW * 64;                  // threads
  constexpr int WM = BM / (NW / 2), WN = BN / 2, MI = WM / 16, NI = WN / 16;
  constexpr int IR = NT / 8;                   // tile rows per load item (8 threads per 128-byte row)
  constexpr int CH = BM / IR;                  // 16-byte A items per thread per step
  constexpr int CW = (BN + IR - 1) / IR;       // 16-byte W items per thread per step (the last may be partial)
  constexpr int CM = CH > CW ? CH : CW;
  static_assert(BM % IR == 0 && BN % 8 == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* As = lds;                          // [2][BM][kLds]
  constexpr int WR = w_lds_rows<BN, NW>();     // W tile rows in LDS (>= BN)
  uint16_t* Ws = lds + 2 * BM * kLds;          // [2][WR][kLds]

  int mt, nt, split;
  tile_of_block_mn(blockIdx.x, n_mt, splits, mt, nt, split);
  if (nt >= n_nt) return;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  const int nk_all = K / kBK;
  const int ks0 = split * nk_all / splits, ks1 = (split + 1) * nk_all / splits;
  const int nk = ks1 - ks0;
  const int nk_pad = (nk + DEPTH - 1) / DEPTH * DEPTH;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

  // item i of thread t covers tile row (t >> 3) + IR i, columns ((t & 7) * 8, +8);
  // the 8 rows a wave loads for one item never straddle a weight segment
  // (segments and the gate/up halves of a tile start at multiples of 8 rows).
  // The per-lane offsets are fixed; each K step moves the buffer descriptors'
  // base (scalar arithmetic only), and a padding step gets descriptors with no
  // records, so every lane reads zeros through the range check.
  // A's rows up to M_max are read (rows >= M_max are past the records at
  // every step): a row at or past the row count feeds only its own output
  // row, which is never stored, so the first loads need not wait for *n_rows
  const char* abase = reinterpret_cast<const char*>(A + (size_t)m0 * K);
  const int arec = max(min(M_max - m0, BM), 0) * K * 2;
  const char* wbase[CW];
  uint32_t aoff[CH], woff[CW];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int row = (t >> 3) + IR * i, kc = (t & 7) * 8;
    aoff[i] = (uint32_t)((row * K + ks0 * kBK + kc) * 2);
  }
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int row = (t >> 3) + IR * i, kc = (t & 7) * 8;
    int sg, r;
    wrow_index<BN>(W, n0 + row, sg, r);
    sg = __builtin_amdgcn_readfirstlane(sg);
    wbase[i] = static_cast<const char*>(W.p[sg]);
    // empty columns, and rows past BN of a partial last item (whole waves),
    // read zeros without a memory access
    woff[i] = r < 0 || row >= BN ? kOob : w_offset(W.blocked, r, ks0 * kBK + kc, K);
  }
  const int wst = (int)w_step(W.blocked);
  uint4 ra[DEPTH][CH], rw[DEPTH][CW];
  // K order: with one row tile, each column tile starts at its own K step
  // (its weight rows spread over the HBM channels); with several, every tile
  // on an XCD starts at that XCD's step, so the tiles sharing its L2 walk the
  // rows of A together instead of pulling all of A through it at once.
  const int rot = k_rotation(n_mt > 1 ? (int)(blockIdx.x & 7) : nt, nk);
  auto issue = [&](int step, uint4 (&a)[CH], uint4 (&w)[CW]) {
    const bool in = step < nk;
    const int sr = step + rot >= nk ? step + rot - nk : step + rot;
    const int ks = in ? sr * (kBK * 2) : 0, ksw = in ? sr * wst : 0;
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(abase) + ks, (short)0,
                                                                         in ? arec - ks : 0, kBufWord3);
#pragma unroll
    for (int i = 0; i < CM; ++i) {
      if (i < CH) a[i] = buf_load16(ar, aoff[i]);
      if (i < CW) {
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(wbase[i]) + ksw, (short)0, in ? (int)W.seg_bytes - ksw : 0, kBufWord3);
        w[i] = WNT && DTSK_W_NT ? buf_load16_nt(wr, woff[i]) : buf_load16(wr, woff[i]);
      }
    }
  };
  auto store = [&](int buf, const uint4 (&a)[CH], const uint4 (&w)[CW]) {
#pragma unroll
    for (int i = 0; i < CM; ++i) {
      const int row = (t >> 3) + IR * i, kc = (t & 7) * 8;
      if (i < CH) *reinterpret_cast<uint4*>(As + buf * BM * kLds + lds_idx(row, kc >> 3)) = a[i];
      if (i < CW) *reinterpret_cast<uint4*>(Ws + buf * WR * kLds + lds_idx(row, kc >> 3)) = w[i];
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s) issue(s, ra[s], rw[s]);
  // the row count decides the early exit and which rows are stored
  const int M = min(*n_rows - m_base, M_max);
  if (m0 >= M) return;
  store(0, ra[0], rw[0]);
  lds_barrier();
  for (int kt = 0; kt < nk_pad; kt += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      issue(kt + u + DEPTH - 1, ra[(u + DEPTH - 1) % DEPTH], rw[(u + DEPTH - 1) % DEPTH]);
      const int buf = (DEPTH % 2 == 0) ? (u & 1) : ((kt + u) & 1);   // LDS buffer of step kt + u
      const uint16_t* a = As + buf * BM * kLds;
      const uint16_t* w = Ws + buf * WR * kLds;
      // a padding step (past this split's K steps; its tiles are zeros) adds
      // nothing: skip its fragment reads and MFMAs (uniform branch)
      if (DTSK_SKIP_PAD && kt + u >= nk) {
        store(buf ^ 1, ra[(u + 1) % DEPTH], rw[(u + 1) % DEPTH]);
        lds_barrier();
        continue;
      }
#pragma unroll
      for (int ks = 0; ks < kBK / 32; ++ks) {
        const int kch = ks * 4 + (lane >> 4);
        bf16x8 fa[MI], fb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
          fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a + lds_idx(wm0 + i * 16 + (lane & 15), kch)));
#pragma unroll
        for (int j = 0; j < NI; ++j)
          fb[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(w + lds_idx(wn0 + j * 16 + (lane & 15), kch)));
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      store(buf ^ 1, ra[(u + 1) % DEPTH], rw[(u + 1) % DEPTH]);
      lds_barrier();
    }
  }

  if (epi.kind == EPI_NONE) {
    float* Ps = P + (size_t)split * M_max * N;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 16 + (lane >> 4) * 4 + r;
          if (m < M) Ps[(size_t)m * N + n0 + wn0 + j * 16 + (lane & 15)] = acc[i][j][r];
        }
    return;
  }
  // finished tile to LDS in passes of ER rows (rows relative to the pass),
  // then the epilogue on a view whose row 0 is the pass's first packed row
  constexpr int TS = BN + 4, ER = epi_rows<BM>();
  float* T = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int pass = 0; pass < BM / ER; ++pass) {
    const int r0 = m0 + pass * ER;
    if (r0 >= M) continue;                     // uniform over the workgroup (and every later pass too)
    if (pass > 0) lds_barrier();               // the previous pass has read T
    if (wm0 / ER == pass) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            T[(wm0 - pass * ER + i * 16 + (lane >> 4) * 4 + r) * TS + wn0 + j * 16 + (lane & 15)] = acc[i][j][r];
    }
    lds_barrier();
    Epilogue e = epi;
    const int Mt = min(ER, M - r0);
    if (e.kind == EPI_SWIGLU) e.act_out = reinterpret_cast<uint16_t*>(e.act_out) + (size_t)r0 * e.F;
    if (e.kind == EPI_QKV) e.q_out = reinterpret_cast<uint16_t*>(e.q_out) + (size_t)r0 * e.d;
    if (e.row_pos) e.row_pos += r0;
    if (e.row_seq) e.row_seq += r0;
    if (e.kind == EPI_LM) e.lm_part += (size_t)r0 * e.lm_tiles * 4;
    tile_epilogue<BN, TS, NT, ER, (BN == 192 && BM == kBigBM)>(e, T, W, n0, Mt);
  }
}

// ---------------------------------------------------------------------------
// SIMT fallback: 64x64 tile, 4x4 outputs per thread, fp32 FMA, no epilogue
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_gemm_simt(const T* __restrict__ A, int M_max,
                                                   const int32_t* __restrict__ n_rows, int m_base, int K, WMap W,
                                                   int N, float* __restrict__ P) {
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
        const int sg = n / W.n_seg, r = n - sg * W.n_seg;
        const size_t idx = W.blocked ? ((size_t)(r >> 3) * (K >> 6) + (k >> 6)) * 512 + (r & 7) * 64 + (k & 63)
                                     : (size_t)r * K + k;
        wv = to_f32(reinterpret_cast<const T*>(W.p[sg])[idx]);
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

template <int MI, int BN>
hipError_t launch_skinny(const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows, int m_base, int K,
                         const WMap& w, int N, float* P, const Epilogue& epi, hipStream_t st) {
  const int n_nt = N / BN;
  const int grid = cdiv(n_nt, 8) * 8 * plan.splits;
  DTSK_LAUNCH((k_gemm_skinny<MI, BN>), dim3(grid), dim3(256), 0, st, (const uint16_t*)A, M_max, n_rows, m_base,
                     K, w, N, plan.splits, n_nt, P, epi);
  return hipGetLastError();
}

template <int BN>
hipError_t launch_skinny_bn(const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows, int m_base, int K,
                            const WMap& w, int N, float* P, const Epilogue& epi, hipStream_t st) {
  switch (plan.mi) {
    case 1: return launch_skinny<1, BN>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    case 2: return launch_skinny<2, BN>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    case 4: return launch_skinny<4, BN>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    default: return launch_skinny<8, BN>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
  }
}

// Row tiles up to which the weights are loaded non-temporal: on the kept rows
// (one row tile) and on 512 rows in 256-row tiles they are read once or
// twice and the hint keeps the activation rows cached; with more row tiles
// each weight tile is read again by the others, from L2 if it stayed there.
#ifndef DTSK_NT_MAX_ROW_TILES
#define DTSK_NT_MAX_ROW_TILES 2
#endif
constexpr int kNtMaxRowTiles = DTSK_NT_MAX_ROW_TILES;

template <int BN, int BM, int NW, int DEPTH, bool WNT>
hipError_t launch_tiled_k(const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows, int m_base, int K,
                          const WMap& w, int N, float* P, const Epilogue& epi, hipStream_t st) {
  constexpr int lds_bytes = large_lds<BN, BM, NW>();
  static bool attr_set = false;  // the tile may need more than the default 64 KiB of LDS
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_mfma<BN, BM, NW, DEPTH, WNT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_mt = cdiv(M_max, BM), n_nt = plan.tiles > 0 ? plan.tiles : N / BN;
  // one block per (row tile, column tile, split), in tile_of_block_mn's order
  const bool by_split = plan.splits > 1 && 8 % plan.splits == 0;
  const int grid = by_split ? cdiv(n_nt, 8 / plan.splits) * n_mt * 8 : cdiv(n_nt, 8) * 8 * n_mt * plan.splits;
  DTSK_LAUNCH((k_gemm_mfma<BN, BM, NW, DEPTH, WNT>), dim3(grid), dim3(NW * 64), lds_bytes, st, (const uint16_t*)A,
              M_max, n_rows, m_base, K, w, N, plan.splits, n_mt, n_nt, P, epi);
  return hipGetLastError();
}

template <int BN, int BM = kBM, int NW = 4, int DEPTH = kDepthL>
hipError_t launch_tiled(const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows, int m_base, int K,
                        const WMap& w, int N, float* P, const Epilogue& epi, hipStream_t st) {
  if (cdiv(M_max, BM) <= kNtMaxRowTiles)
    return launch_tiled_k<BN, BM, NW, DEPTH, true>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
  return launch_tiled_k<BN, BM, NW, DEPTH, false>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
}

}  // namespace

GemmPlan plan_gemm(dl_dtype dt, int M, int N, int K, int epi_kind, int head_dim, int F) {
  const GemmPlan simt{GEMM_SIMT, 1, 128, 8, 0, 1};
  GemmPlan p = simt;
  if (dt != DL_BF16 || K % 64 != 0 || M <= 0) return p;
  const int nk = K / 64;
  const int n_seg = epi_kind == EPI_QKV ? N / 3 : epi_kind == EPI_SWIGLU ? N / 2 : N;
  // 33..128 rows: one row of 128-row tiles of the tiled kernel when the shape
  // allows it (at 64 rows it beat the skinny kernel by 7% per layer); fewer
  // rows go to the skinny kernel
  const bool tiled_small = DTSK_TILED_SMALL && M > DTSK_TILED_MIN_ROWS && M <= 128 &&
                           (DTSK_TILED_LM || epi_kind != EPI_LM) &&
                           N % 64 == 0 && (epi_kind != EPI_LM || N % 128 == 0) &&
                           (epi_kind != EPI_QKV || (head_dim == 128 && n_seg % 128 == 0)) &&
                           (epi_kind != EPI_SWIGLU || F % 32 == 0);
  if (tiled_small) {
    p.kind = GEMM_LARGE;
    p.sep_epi = 0;
    // 128-wide column tiles when there are enough of them to spread over the
    // chip; else 64-wide ones (twice the workgroups)
    // (the LM statistics are kept per 128-wide column tile)
    const bool wide = epi_kind == EPI_LM || (N % 128 == 0 && N / 128 >= DTSK_T128_MIN_TILES && epi_kind != EPI_QKV &&
                                             (epi_kind != EPI_SWIGLU || F % 64 == 0));
    p.bn = wide ? 128 : 64;
    // the LM head: 256-wide tiles (DTSK_LM_NW = 16 waves of 16 x 128), which
    // read the rows of A half as often as 128-wide ones
    if (DTSK_LM256 && epi_kind == EPI_LM && N % 256 == 0) p.bn = 256;
    if (p.bn != 256) p.nw = p.bn == 128 ? DTSK_SMALL_NW128 : DTSK_SMALL_NW;
    p.wmode = epi_kind == EPI_SWIGLU ? 1 : epi_kind == EPI_QKV ? 2 : 0;
    // Wq|Wk|Wv: 128-wide tiles of natural column order and a K split in two
    // (192 workgroups, half the A rows each); k_epi_qkv_rows4 sums the two
    // partials and applies RoPE and the cache writes
    if (DTSK_QKV_SPLIT && epi_kind == EPI_QKV && head_dim <= 128 && n_seg % 128 == 0 && (N / 128) * 2 <= 256 &&
        nk >= 2) {
      p.bn = 128;
      // 96-wide tiles when they make whole rounds of 256 workgroups (d =
      // 4096: 128 tiles x 2 splits, against 96 x 2 on 128-wide tiles); the
      // partials stay in natural column order for the separate epilogue
      if (DTSK_QKV96 && p.nw == 8 && N % 96 == 0 && (N / 96) * 2 <= 256 && (N / 96) * 2 > (N / 128) * 2) p.bn = 96;
      p.wmode = 0;
      p.sep_epi = 1;
      p.splits = 2;
      return p;
    }
    // gate|up: one ragged column tile per compute unit (each holding F / 256
    // gate rows and the matching up rows) when that is at least 32 rows
    if (DTSK_RAGGED && epi_kind == EPI_SWIGLU && F >= 32 * kRaggedTiles && F <= 64 * kRaggedTiles) {
      p.bn = 128;
      p.wmode = 3;
      p.tiles = kRaggedTiles;
      // up to 48 gate rows per tile: 96-wide tiles (43 + 43 live columns of
      // 96 at F = 11008 instead of 128), a quarter fewer weight requests,
      // LDS stores and MFMAs on empty columns
      if (DTSK_GU96 && F <= 48 * kRaggedTiles && p.nw == 8) p.bn = 96;
    }
    if (epi_kind == EPI_NONE) {
      const int tiles = N / p.bn;
      int s = 1;
      while (tiles * s < 256 && s < 8 && s * 2 <= nk) s *= 2;
      p.splits = s;
    }
    return p;
  }
  if (M <= 128 && (long long)n_seg * K * 2 < 0x7fff0000LL && 128LL * K * 2 < 0x7fff0000LL) {
    p.kind = GEMM_SKINNY;
    p.sep_epi = 0;
    p.mi = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
    switch (epi_kind) {
      case EPI_QKV:
        if (head_dim == 128 && n_seg % 128 == 0) {
          p.bn = 64;
          p.wmode = 2;
        } else if (head_dim % 2 == 0 && 128 % head_dim == 0 && n_seg % 128 == 0) {
          p.bn = 128;
        } else {
          return simt;
        }
        break;
      case EPI_SWIGLU:
        if (F % 32 != 0) return simt;
        p.bn = 64;
        p.wmode = 1;
        break;
      case EPI_LM:
        p.bn = 128;
        break;
      default: {  // partial sums: split K until the grid covers the CUs about once
        p.bn = 64;
        if (N % 64 != 0) return simt;
        const int tiles = N / 64;
        p.splits = std::max(1, std::min(std::min((256 + tiles - 1) / tiles, 16), nk));
      }
    }
    if (N % p.bn != 0) return simt;
    return p;
  }
  if (N % kBN != 0) return p;
  if (epi_kind == EPI_SWIGLU && F % (kBN / 2) != 0) return p;
  if (epi_kind == EPI_QKV && !(head_dim % 2 == 0 && 128 % head_dim == 0 && (N / 3) % kBN == 0)) return p;
  p.kind = GEMM_LARGE;
  p.sep_epi = 0;
  p.bn = kBN;
  p.wmode = epi_kind == EPI_SWIGLU ? 1 : 0;
  if (DTSK_LM256 && epi_kind == EPI_LM && N % 256 == 0) p.bn = 256;   // as on fewer rows
  if (p.bn == kBN) p.nw = DTSK_MID_NW;
  // More than 256 rows, gate|up and the split-K products: 256-row tiles,
  // which read every weight tile half as often as 128-row tiles; gate|up on
  // kBigRagged ragged 192-wide tiles (up to 96 gate rows and the matching up
  // rows each), so that at 512 rows the two row tiles fill 256 compute units.
  // (QKV and the LM head ran slower on 256-row tiles at 512 rows, QKV also at
  // 4608 rows.)
  const bool big = DTSK_BIG_TILES && M > kBigBM && (epi_kind == EPI_SWIGLU || epi_kind == EPI_NONE);
  if (big) {
    p.bm = kBigBM;
    if (epi_kind == EPI_SWIGLU && F <= 96 * kBigRagged) {
      p.bn = 192;
      p.wmode = 3;
      p.tiles = kBigRagged;
    }
  }
  // QKV on 385..512 rows: 192-wide tiles in rope-pair order, 64 column tiles
  // x 4 row tiles = 256 workgroups in one round (128-wide tiles make 96 x 4 =
  // 384, a round and a half)
  if (DTSK_QKV192 && epi_kind == EPI_QKV && head_dim == 128 && n_seg % 64 == 0 && N % 192 == 0 &&
      M > 3 * kBM && M <= 4 * kBM && (N / 192) * 4 <= 256) {
    p.bn = 192;
    p.wmode = 2;
    p.nw = 8;
  }
  if (epi_kind == EPI_NONE) {
    const int tiles = cdiv(M, big ? kBigBM : kBM) * (N / kBN);
    int s = 1;
    while (tiles * s < 256 && s < 8 && s * 2 <= nk) s *= 2;
    p.splits = s;
  }
  return p;
}

hipError_t launch_gemm(dl_dtype dt, const GemmPlan& plan, const void* A, int M_max, const int32_t* n_rows,
                       int m_base, int K, const void* const* Wseg, int n_seg, int N, float* P, const Epilogue& epi,
                       hipStream_t st, int w_layout) {
  WMap w;
  for (int i = 0; i < 4; ++i) w.p[i] = Wseg[i];
  w.mode = plan.wmode;
  w.n_seg = n_seg;
  w.blocked = w_layout == DL_WEIGHTS_BLOCKED;
  // blocked weights: whole 8-row groups and 64-wide K steps (the dims check
  // refuses other shapes)
  if (w.blocked && (dt != DL_BF16 || K % 64 != 0 || n_seg % 8 != 0)) return hipErrorInvalidValue;
  const long long seg_bytes = (long long)(plan.wmode == 1 || plan.wmode == 3 ? N / 2 : n_seg) * K * 2;
  // the tiled and skinny kernels address a segment through one buffer
  // resource with 32-bit offsets; larger segments are refused by the dims check
  if (plan.kind != GEMM_SIMT && seg_bytes > kMaxBufBytes) return hipErrorInvalidValue;
  w.seg_bytes = (int)std::min<long long>(seg_bytes, kMaxBufBytes);
  w.n_tiles = plan.tiles;
  if (plan.wmode == 3) w.n_seg = N / 2;
  if (M_max <= 0) return hipSuccess;
  if (plan.kind == GEMM_SKINNY) {
    if (plan.bn == 64) return launch_skinny_bn<64>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    return launch_skinny_bn<128>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
  }
  if (plan.kind == GEMM_LARGE) {
    if (plan.bm == kBigBM) {
      if (plan.bn == 192) {   // the 192-wide tile carries only the SwiGLU epilogue
        if (epi.kind != EPI_SWIGLU) return hipErrorInvalidValue;
        return launch_tiled<192, kBigBM, kBigWaves, kBigDepth192>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
      }
      return launch_tiled<kBN, kBigBM, DTSK_BIG_NW128>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    }
    if (plan.bn == 256) return launch_tiled<256, kBM, DTSK_LM_NW>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
#if DTSK_SMALL_NW128 == 16
    if (plan.nw == 16 && plan.bn == kBN)
      return launch_tiled<kBN, kBM, 16, DTSK_SMALL_DEPTH>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
#endif
    if (plan.nw == 8) {
      if (plan.bn == 192)  // QKV in rope-pair order
        return launch_tiled<192, kBM, 8, DTSK_SMALL_DEPTH>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
      if (plan.bn == 96)   // the ragged gate|up tiles only
        return launch_tiled<96, kBM, 8, DTSK_SMALL_DEPTH>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
      if (plan.bn == 64)
        return launch_tiled<64, kBM, 8, DTSK_SMALL_DEPTH>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
      return launch_tiled<kBN, kBM, 8, DTSK_SMALL_DEPTH>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    }
    if (plan.bn == 64) return launch_tiled<64>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
    return launch_tiled<kBN>(plan, A, M_max, n_rows, m_base, K, w, N, P, epi, st);
  }
  dim3 grid(cdiv(N, 64), cdiv(M_max, 64));
  if (dt == DL_F32)
    DTSK_LAUNCH(k_gemm_simt<float>, grid, dim3(256), 0, st, (const float*)A, M_max, n_rows, m_base, K, w, N,
                       P);
  else
    DTSK_LAUNCH(k_gemm_simt<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)A, M_max, n_rows, m_base, K, w, N,
                       P);
  return hipGetLastError();
}

// Blocked copy of a row-major [N, K] bf16 matrix (N % 8 == 0, K % 64 == 0):
// one thread moves one 16-byte piece (8 inputs of a row), which stays
// contiguous in the blocked order.
__global__ __launch_bounds__(256) void k_pack_w8x64(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    long long items, int K) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= items) return;
  const int pieces = K >> 3;                     // 16-byte pieces per row
  const long long r = i / pieces;
  const int k = (int)(i - r * pieces) << 3;
  const long long e = ((r >> 3) * (K >> 6) + (k >> 6)) * 512 + (r & 7) * 64 + (k & 63);
  dst[e >> 3] = src[i];
}

hipError_t launch_pack_weights(const void* src, void* dst, int N, int K, hipStream_t st) {
  const long long items = (long long)N * (K / 8);
  if (items <= 0) return hipSuccess;
  const long long blocks = (items + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  DTSK_LAUNCH(k_pack_w8x64, dim3((unsigned)blocks), dim3(256), 0, st, (const uint4*)src, (uint4*)dst, items, K);
  return hipGetLastError();
}

}  // namespace dtsk
