// Shared device helpers and the workspace layout of the EntmaxKV HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/entmaxkv.h"

namespace ekv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Workspace layout.  The control words come first and are zero when idle
// (ekv_workspace_init zeroes the whole buffer; every kernel that changes a
// control word restores it before the step ends).
// ---------------------------------------------------------------------------
struct Layout {
  size_t status;    // u32 device status bits
  size_t max_key;   // u32 [B*Hq] running max of the decode scores (ordered key, 0 = empty)
  size_t scores;    // f32 [B*Hkv*max_pages] bounding-box page scores
  size_t stats;     // float4 [B*Hq*max_pages] Gaussian (mean_Y, sd_Y, e_hat, n_p)
  size_t tau_hat;   // f64 [B*Hq]
  size_t item_cnt;  // i32 [B*Hq*max_pages] candidates kept by each decode work item
  size_t item_max;  // f32 [B*Hq*max_pages] per item maximum score
  size_t cand_x;    // f32 [B*Hq*max_pages*P] candidate scores, one region per item
  size_t cand_t;    // i32 [B*Hq*max_pages*P] candidate logical token ids
  size_t ovf_x;     // f32 [B*Hq*max_pages*P] compacted candidates (large sets)
  size_t ovf_t;     // i32 [B*Hq*max_pages*P]
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout make_layout(int B, int Hkv, int Hq, int max_pages, int P) {
  Layout L{};
  size_t off = 0;
  const size_t bh = size_t(B) * Hq;
  const size_t tok = size_t(max_pages) * P;
  L.status = off;   off = align256(off + 4);
  L.max_key = off;  off = align256(off + 4 * bh);
  L.scores = off;   off = align256(off + 4 * size_t(B) * Hkv * max_pages);
  L.stats = off;    off = align256(off + 16 * bh * max_pages);
  L.tau_hat = off;  off = align256(off + 8 * bh);
  L.item_cnt = off; off = align256(off + 4 * bh * max_pages);
  L.item_max = off; off = align256(off + 4 * bh * max_pages);
  L.cand_x = off;   off = align256(off + 4 * bh * tok);
  L.cand_t = off;   off = align256(off + 4 * bh * tok);
  L.ovf_x = off;    off = align256(off + 4 * bh * tok);
  L.ovf_t = off;    off = align256(off + 4 * bh * tok);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Storage formats.  A lane always loads 16 contiguous bytes.
// ---------------------------------------------------------------------------
template <int DT> struct Elem;
template <> struct Elem<EKV_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  __device__ static __forceinline__ void unpack(const uint4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load1(const void* base, size_t i) {
    return reinterpret_cast<const float*>(base)[i];
  }
};
template <> struct Elem<EKV_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  // bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
  __device__ static __forceinline__ void unpack(const uint4& w, float* f) {
    f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
    f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
    f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
  }
  __device__ static __forceinline__ float load1(const void* base, size_t i) {
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(base)[i]) << 16);
  }
};

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 is
// mapped like +0 so equal values give equal keys.  Key 0 is below every
// non-NaN float and marks "empty".
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bits) {
  atomicOr(status, bits);
}

// ---------------------------------------------------------------------------
// Reductions.  Fixed butterfly order, so results do not depend on timing.
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <typename T> __device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, kWave));
  return v;
}
template <typename T> __device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, kWave));
  return v;
}

// Block-wide reductions for blockDim.x a multiple of 64 (<= 1024).  `red`
// is shared scratch of >= 16 elements; every thread gets the result.
template <typename T> __device__ T block_sum(T v, T* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
  for (int i = 1; i < nw; ++i) r += red[i];
  return r;
}
template <typename T> __device__ T block_max(T v, T* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
  for (int i = 1; i < nw; ++i) r = max(r, red[i]);
  return r;
}
template <typename T> __device__ T block_min(T v, T* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_min(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
  for (int i = 1; i < nw; ++i) r = min(r, red[i]);
  return r;
}

// Exclusive prefix sum over the block (blockDim.x multiple of 64, <= 1024);
// `red` holds >= 17 ints.  Returns the exclusive prefix, *total the sum.
__device__ inline int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  *total = tot;
  return before + inc - v;
}

// Number of pages of a sequence of length L.
__device__ __forceinline__ int pages_of(int L, int P) { return (L + P - 1) / P; }

}  // namespace ekv
