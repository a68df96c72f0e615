// Internal helpers shared by the HIP kernels of libdtsk (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dl.h"

namespace dtsk {

// Storage types.  bf16 is kept as raw 16-bit patterns; conversions are done
// here so that every rounding point is explicit (round to nearest even).
struct bf16_t {
  uint16_t u;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x.u) << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) {
  uint32_t u = __float_as_uint(f);
  bf16_t r;
  if ((u & 0x7fffffffu) > 0x7f800000u) {  // NaN stays a (quiet) NaN
    r.u = (uint16_t)((u >> 16) | 0x40u);
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    r.u = (uint16_t)(u >> 16);
  }
  return r;
}

// Kernel timing by dispatch timestamps.  While a timed region of the calling
// thread is open, `g_region_events` points at its event pair: every launch
// through DTSK_LAUNCH then binds `stop` to its own dispatch packet, and the
// first one also binds `start` (which it clears), so the pair spans the
// region's kernels from the first one's start to the last one's end, with no
// marker packets between the launches.
struct DispatchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local DispatchEvents* g_region_events;

template <typename F, typename... Args>
inline void launch_with_events(DispatchEvents* ev, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                               Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev->start, ev->stop, 0u, args...);
  ev->start = nullptr;
}

#define DTSK_LAUNCH(kernel, grid, block, lds, st, ...)                                              \
  do {                                                                                              \
    if (::dtsk::DispatchEvents* ev_ = ::dtsk::g_region_events)                                      \
      ::dtsk::launch_with_events(ev_, kernel, dim3(grid), dim3(block), (uint32_t)(lds), st, __VA_ARGS__); \
    else                                                                                            \
      hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);                                \
  } while (0)

// Round an fp32 value to the storage type and back (what a store + load does).
template <typename T>
__device__ __forceinline__ float round_to(float f) { return to_f32(from_f32<T>(f)); }

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024).  Fixed order, so
// the result does not depend on timing.  `red` must hold 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = warp_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// not for its global loads, so loads prefetched ahead stay in flight across
// the barrier (a plain __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer loads.  A resource covers `bytes` bytes from `base`; a 16-byte
// load whose byte offset runs past them returns zeros without touching
// memory (the range check of raw buffer addressing), so a masked load needs
// no branch.  That matters for prefetch rings: a load under an exec branch
// leaves the compiler unable to count the loads in flight, and it then waits
// for all of them (vmcnt(0)) right after issuing the next tile's.  Offsets
// and sizes are 32-bit: one resource spans less than 2 GiB.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;   // resource word 3 on CDNA: 32-bit data format, no swizzle
constexpr long long kMaxBufBytes = 0x7fffffffLL;   // the largest range one resource here covers

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same with the non-temporal hint (cache policy bit nt): for data read
// once, such as a product's weights, so that it does not push the operands
// that are read again (the activation rows) out of the caches.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Row maps of a packed selection: for packed row r, the flat [B,S] row
// b*S + i it came from, and its sequence b.  Built on the device.
struct RowMap {
  int32_t* row_pos;   // [R_max]  (-1 beyond row_off[B])
  int32_t* row_seq;   // [R_max]
  int32_t* n_rows;    // [1]      = row_off[B]
  int32_t* tile_row0; // [T_max]  attention query tiles: first packed row
  int32_t* tile_rows; // [T_max]  rows in the tile (0 = unused)
  int32_t R_max;
  int32_t T_max;
  int32_t tq;         // query rows per attention tile
};

}  // namespace dtsk
