// Shared device helpers and the workspace layout of the EntmaxKV HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/entmaxkv.h"

namespace ekv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Workspace layout.  The status word comes first; ekv_workspace_init zeroes
// the whole buffer.  Every other region is fully rewritten by the step that
// reads it, so nothing carries over between calls.
// ---------------------------------------------------------------------------
constexpr int kItemTokens = 64;  // tokens of one decode work item

struct Layout {
  // regions every call may touch, at offsets that depend only on the shape
  size_t status;    // u32 device status bits
  size_t sel_done;  // u32 [B*Hq] per-unit arrival counters of the selection stage (zero between calls)
  size_t scores;    // f32 [B*Hq][score_stride] bounding-box page scores (unit rows)
  size_t musd;      // float2 [B*Hq*max_pages] Gaussian page score (mean_Y, sd_Y)
  size_t ehat;      // f32 [B*Hq*max_pages] estimated page maximum
  size_t tau_hat;   // f64 [B*Hq]
  size_t smx_part;  // f32 [B*Hq][kSmxMaxSlots][head_dim + 2] softmax block partials
  size_t keep_bits; // u64 [B*Hq][keep_words(max_pages)] Gaussian keep decisions per query head
  size_t cand;      // u64 [B*Hkv][cand_lists(max_pages)][kCandPerList] per 64 pages, their
                    // largest scores as (key << 32 | page), in page order, zero-padded
  size_t cand_cut;  // u32 [B*Hkv][cand_lists(max_pages)] largest key a list left out (0: none)
  // the entmax decode's per-item regions, sized for lists of item_pages pages
  size_t item_cnt;  // i32 [B*Hq*max_items] candidates kept by each decode work item
  size_t item_max;  // f32 [B*Hq*max_items] per item maximum score
  size_t item_lb;   // f32 [B*Hq*max_items] per item lower bound on the head's threshold
  size_t cand_x;    // f32 [B*Hq*max_items*64] candidate scores, one region per item
  size_t cand_t;    // i32 [...] candidate logical token ids
  size_t cand_r;    // i32 [...] candidate physical rows (page * P + slot)
  size_t ovf_x;     // f32 [B*Hq*max_items*64] compacted candidates (large sets)
  size_t ovf_t;     // i32 [...]
  size_t ovf_r;     // i32 [...]
  size_t item_lvl;  // u32 [B*Hq*max_items] per item: its scores at or above max - 1/32, - 1/16, - 1/8 (8 bits each;
                    // written and read for heads of more than 1024 items only)
  size_t total;
  size_t max_items; // per (sequence, query head)
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// row stride of the internal page-score buffer: 16-byte aligned rows
inline int score_stride(int max_pages) { return (max_pages + 3) & ~3; }
// 64-page words of a query head's keep bitmap
inline int keep_words(int max_pages) { return (max_pages + 63) / 64; }
// Top-k candidate lists: every kCandListPages pages (one wave of a scoring
// block of kCandBlockPages pages) keep their kCandPerList largest scores for
// the top-k select.
constexpr int kCandBlockPages = 256;
constexpr int kCandListPages = 64;
constexpr int kCandPerList = 8;
inline int cand_lists(int max_pages) {
  return (max_pages + kCandBlockPages - 1) / kCandBlockPages * (kCandBlockPages / kCandListPages);
}

constexpr int kSmxMaxSlots = 256;  // softmax decode blocks per (sequence, KV head), at most

// The entmax decode's per-item regions for B * Hq query heads and lists of
// up to item_pages pages, carved from offset `off` on.
inline size_t carve_items(Layout& L, size_t off, size_t bh, int P, int item_pages) {
  L.max_items = (size_t(item_pages) * P + kItemTokens - 1) / kItemTokens;
  const size_t tok = L.max_items * kItemTokens;
  L.item_cnt = off; off = align256(off + 4 * bh * L.max_items);
  L.item_max = off; off = align256(off + 4 * bh * L.max_items);
  L.item_lb = off;  off = align256(off + 4 * bh * L.max_items);
  L.cand_x = off;   off = align256(off + 4 * bh * tok);
  L.cand_t = off;   off = align256(off + 4 * bh * tok);
  L.cand_r = off;   off = align256(off + 4 * bh * tok);
  L.ovf_x = off;    off = align256(off + 4 * bh * tok);
  L.ovf_t = off;    off = align256(off + 4 * bh * tok);
  L.ovf_r = off;    off = align256(off + 4 * bh * tok);
  L.item_lvl = off; off = align256(off + 4 * bh * L.max_items);
  return off;
}

// item_pages: the longest page list an entmax decode on this workspace
// reads (the list capacity of sparse calls; max_pages for the full cache).
// Everything before item_cnt is independent of it.
inline Layout make_layout(int B, int Hkv, int Hq, int max_pages, int P, int D, int item_pages) {
  Layout L{};
  size_t off = 0;
  const size_t bh = size_t(B) * Hq;
  L.status = off;   off = align256(off + 4);
  // selection units are (sequence, KV head), or (sequence, query head) in
  // per-query-head mode: size the per-unit arrays for the larger count
  L.sel_done = off; off = align256(off + 4 * bh);
  L.scores = off;   off = align256(off + 4 * bh * score_stride(max_pages));
  L.musd = off;     off = align256(off + 8 * bh * max_pages);
  L.ehat = off;     off = align256(off + 4 * bh * max_pages);
  L.tau_hat = off;  off = align256(off + 8 * bh);
  L.smx_part = off; off = align256(off + 4 * bh * kSmxMaxSlots * size_t(D + 2));
  L.keep_bits = off; off = align256(off + 8 * bh * size_t(keep_words(max_pages)));
  // candidate lists exist for shared (sequence, KV head) selections only
  const size_t bk = size_t(B) * Hkv * cand_lists(max_pages);
  L.cand = off;     off = align256(off + 8 * bk * kCandPerList);
  L.cand_cut = off; off = align256(off + 4 * bk);
  L.total = carve_items(L, off, bh, P, item_pages);
  return L;
}

// Only what the entmax decode uses: the status word, then the per-item
// regions (the selection and softmax regions are left out).
inline Layout make_decode_layout(int B, int Hq, int P, int item_pages) {
  Layout L{};
  L.status = 0;
  L.total = carve_items(L, 256, size_t(B) * Hq, P, item_pages);
  return L;
}

// ---------------------------------------------------------------------------
// Matrix-core helpers (gfx950 v_mfma_f32_16x16x32_bf16).  Lane l holds
// A[row l%16][k 8(l/16)..+8), B[k 8(l/16)..+8][col l%16] and returns
// D[rows 4(l/16)..+4][col l%16].
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Split c into three bf16 limbs with c = l0 + l1 + l2 up to 2^-24 |c|: each
// limb is the bf16 rounding of what the previous ones left, and the fp32
// subtractions are exact.  limb(i) returns the bits of limb i.
__device__ __forceinline__ void split3_bf16(float c, uint32_t* l0, uint32_t* l1, uint32_t* l2) {
  *l0 = bf16_rne_bits(c);
  const float r1 = c - __uint_as_float(*l0 << 16);
  *l1 = bf16_rne_bits(r1);
  const float r2 = r1 - __uint_as_float(*l1 << 16);
  *l2 = bf16_rne_bits(r2);
}

// A operand of a 16-row limb product: chunk (kb, ln) holds, for row ln%16 =
// 4h + l and k = 32 kb + 8 (ln/16) + j (j < 8), limb l of coefficient
// coef(h, k); rows with h >= G or l = 3 are zero.  Groups of more than 4
// heads take NH = ceil(G/4) such operands, operand hh holding heads
// 4 hh .. 4 hh + 3 in s_a[hh KB + kb].  Thread t owns chunks t, t +
// blockDim, ...; limb_fetch reads the raw values its chunks need (issue it
// before other loads so it is not queued behind them) and limb_build writes
// each chunk with one conflict-free 16-byte LDS store.
template <int KB, int NH = 1> struct LimbChunks {
  static constexpr int kPerThread = (NH * KB * kWave + 255) / 256;  // for 256-thread blocks
  float v[kPerThread][8];
};

template <int KB, int G, int NH = 1, typename Fetch8>
__device__ __forceinline__ void limb_fetch(LimbChunks<KB, NH>& lc, Fetch8 fetch8) {
#pragma unroll
  for (int i = 0; i < LimbChunks<KB, NH>::kPerThread; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int hh = c / (KB * kWave), cc = c - hh * (KB * kWave);
    const int kb = cc >> 6, ln = cc & 63, row = ln & 15, kg = ln >> 4, h = 4 * hh + (row >> 2);
    if (c < NH * KB * kWave && h < G && (row & 3) < 3) fetch8(h, 32 * kb + 8 * kg, lc.v[i]);
  }
}

template <int KB, int G, int NH = 1, typename Coef>
__device__ __forceinline__ void limb_build(u32x4_t (*s_a)[kWave], const LimbChunks<KB, NH>& lc, Coef coef) {
#pragma unroll
  for (int i = 0; i < LimbChunks<KB, NH>::kPerThread; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c >= NH * KB * kWave) break;
    const int hh = c / (KB * kWave), cc = c - hh * (KB * kWave);
    const int kb = cc >> 6, ln = cc & 63, row = ln & 15, kg = ln >> 4;
    const int h = 4 * hh + (row >> 2), limb = row & 3;
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
    if (h < G && limb < 3) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t l0, l1, l2;
        split3_bf16(coef(32 * kb + 8 * kg + j, lc.v[i][j]), &l0, &l1, &l2);
        const uint32_t bits = limb == 0 ? l0 : (limb == 1 ? l1 : l2);
        wv[j >> 1] |= (bits & 0xffffu) << (16 * (j & 1));
      }
    }
    s_a[hh * KB + kb][ln] = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
  }
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
// Wave-wide reductions on the DPP row network (no LDS traffic): within each
// 16-lane row, xor-1 and xor-2 quad permutes, then the half-row and row
// mirrors (after the quad steps every lane of a quad holds the same value,
// so a mirror adds the other quad / half-row); the four row results are read
// with readlane and combined in a fixed order, so every lane gets the same,
// reproducible value.  The whole wave must be active.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

template <int CTRL> __device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL, typename T> __device__ __forceinline__ T dpp(T v) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t r = ((uint64_t)dpp32<CTRL>((uint32_t)(u >> 32)) << 32) | dpp32<CTRL>((uint32_t)u);
    return __builtin_bit_cast(T, r);
  } else {
    return __builtin_bit_cast(T, dpp32<CTRL>(__builtin_bit_cast(uint32_t, v)));
  }
}
template <typename T> __device__ __forceinline__ T lane_value(T v, int l) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  }
}
// Reduction over aligned groups of 4, 8 or 16 lanes (every lane of a group
// gets the group's value).
template <int N, typename T, typename Op> __device__ __forceinline__ T group_reduce(T v, Op op) {
  static_assert(N == 4 || N == 8 || N == 16, "group size");
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  if constexpr (N >= 8) v = op(v, dpp<kDppRowHalfMirror>(v));
  if constexpr (N >= 16) v = op(v, dpp<kDppRowMirror>(v));
  return v;
}
template <typename T, typename Op> __device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = group_reduce<16>(v, op);
  const T r0 = lane_value(v, 0), r1 = lane_value(v, 16), r2 = lane_value(v, 32), r3 = lane_value(v, 48);
  return op(op(r0, r1), op(r2, r3));
}
template <typename T> __device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T x, T y) { return x + y; });
}
template <typename T> __device__ __forceinline__ T wave_max(T v) {
  return wave_reduce(v, [](T x, T y) { return max(x, y); });
}
template <typename T> __device__ __forceinline__ T wave_min(T v) {
  return wave_reduce(v, [](T x, T y) { return min(x, y); });
}

// Store that is visible to every block of the device once it completes
// (device-scope relaxed atomic store; written through the L2).
template <typename T> __device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this wave issued has completed.  After
// st_dev stores, a later atomic by the same block orders after them.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// K sums at once; `red` holds >= K * (waves per block) doubles.
template <int K> __device__ inline void block_sums(double (&v)[K], double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = wave_sum(v[k]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[K * w + k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = red[k];
  for (int i = 1; i < nw; ++i) {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] += red[K * i + k];
  }
}
__device__ inline void block_sum3(double& a, double& b, double& c, double* red) {
  double v[3] = {a, b, c};
  block_sums<3>(v, red);
  a = v[0]; b = v[1]; c = v[2];
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

// Inclusive prefix sum across the wave: row shifts by 1, 2, 4, 8 (lanes
// without a source add 0), then lane 15 of rows 0 and 2 is added to rows 1
// and 3 and lane 31 to rows 2 and 3 (row broadcasts).  Whole wave active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// The same scan on unsigned words (sums wrap modulo 2^32, so several small
// counts can share one word in disjoint bit fields).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}

// Exclusive prefix sum over the block (blockDim.x multiple of 64, <= 1024);
// `red` holds >= 17 ints.  Returns the exclusive prefix, *total the sum.
__device__ inline int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(v);
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

// block_exclusive_scan on unsigned words (modulo 2^32); `red` holds >= 16.
__device__ inline uint32_t block_exclusive_scan_u32(uint32_t v, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t inc = wave_incl_scan_u32(v);
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  *total = tot;
  return before + inc - v;
}

// p[i] for i < n, else `fill`, read from p[min(i, n - 1)] (p[0] when n is
// 0, which must be readable) without a branch: guarded loads written this
// way are issued back to back, where a branch around each load costs a
// wait for it.
template <typename T> __device__ __forceinline__ T load_or(const T* p, int i, int n, T fill) {
  const T v = p[i < n ? i : (n > 0 ? n - 1 : 0)];
  return i < n ? v : fill;
}

// Number of pages of a sequence of length L.
__device__ __forceinline__ int pages_of(int L, int P) { return (L + P - 1) / P; }

}  // namespace ekv
