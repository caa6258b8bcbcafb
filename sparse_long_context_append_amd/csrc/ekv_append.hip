// append_kv: write new tokens into their page slots and keep the per-page
// metadata current (EntmaxKV summary sec. 2.A keeps k_min/k_max and the key
// moments per page; sec. 1: the cache grows by one token per decode step).
//
// A (touched page, KV head, sequence) is one unit.  Each thread of a unit
// owns one 16-byte vector of key coordinates (8 bf16 or 4 fp32 values), so
// every load and store is 16 bytes, and folds the page's new tokens into
// its coordinates' min, max, mean and squared-deviation sum in token order:
// one call with n tokens and n calls with one token produce the same bits.
// The loads of four tokens are issued before the first is folded.  Units
// are packed 256 threads to a block, KV heads fastest, so the threads of a
// block read neighbouring rows of the new tokens.
#include "ekv_kernels.h"

namespace ekv {

constexpr int kAppendThreads = 256;
constexpr int kAppendAhead = 4;  // tokens whose loads are in flight together

template <int DT, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a, int touched) {
  using E = Elem<DT>;
  constexpr int EPL = E::kPerVec;      // coordinates per thread
  constexpr int TPU = D / EPL;         // threads per unit
  constexpr int UPB = kAppendThreads / TPU;
  const int b = blockIdx.y;
  const int unit = blockIdx.x * UPB + (int)threadIdx.x / TPU;
  const int c = (int)threadIdx.x % TPU;  // coordinates [c EPL, c EPL + EPL)
  const int Hkv = a.n_kv_heads, P = a.page_size;
  if (unit >= touched * Hkv) return;
  const int j = unit / Hkv, g = unit - j * Hkv;
  const int L = a.seq_lens[b];
  if (L < 0 || (long long)L + a.n_new > (long long)a.max_pages * P) {
    if (unit == 0 && c == 0) set_status(a.status, EKV_DEV_BAD_LENGTH);
    return;
  }
  const int lp = L / P + j;
  const int t0 = max(L, lp * P), t1 = min(L + a.n_new, (lp + 1) * P);
  if (t0 >= t1) return;
  const int phys = a.page_table[(size_t)b * a.max_pages + lp];
  if (phys < 0 || phys >= a.n_phys) {
    if (g == 0 && c == 0) set_status(a.status, EKV_DEV_BAD_PAGE);
    return;
  }
  const int slot0 = t0 - lp * P;
  const size_t page_base = (size_t)phys * Hkv + g;
  const int i0 = c * EPL;
  char* kc = reinterpret_cast<char*>(a.k);
  char* vc = reinterpret_cast<char*>(a.v);
  const char* kn = reinterpret_cast<const char*>(a.k_new);
  const char* vn = reinterpret_cast<const char*>(a.v_new);
  float mn[EPL], mx[EPL], mean[EPL], m2[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) { mn[e] = INFINITY; mx[e] = -INFINITY; mean[e] = 0.f; m2[e] = 0.f; }
  if (slot0 > 0) {  // continue an existing page
    if (a.k_box) {
      const char* bx = reinterpret_cast<const char*>(a.k_box);
      E::unpack(ldg16(bx + ((page_base * 2 + 0) * D + i0) * E::kBytes), mn);
      E::unpack(ldg16(bx + ((page_base * 2 + 1) * D + i0) * E::kBytes), mx);
    }
    if (a.k_moments) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 mu4 = *reinterpret_cast<const float4*>(a.k_moments + (page_base * 2 + 0) * D + i0 + e);
        const float4 m24 = *reinterpret_cast<const float4*>(a.k_moments + (page_base * 2 + 1) * D + i0 + e);
        mean[e] = mu4.x; mean[e + 1] = mu4.y; mean[e + 2] = mu4.z; mean[e + 3] = mu4.w;
        m2[e] = m24.x; m2[e + 1] = m24.y; m2[e + 2] = m24.z; m2[e + 3] = m24.w;
      }
    }
  }
  int n = slot0;
  for (int tb = t0; tb < t1; tb += kAppendAhead) {
    uint4 kr[kAppendAhead], vr[kAppendAhead];
#pragma unroll
    for (int u = 0; u < kAppendAhead; ++u) {
      if (tb + u < t1) {
        const size_t src = ((((size_t)b * a.n_new + (tb + u - L)) * Hkv + g) * D + i0) * E::kBytes;
        kr[u] = ldg16(kn + src);
        vr[u] = ldg16(vn + src);
      }
    }
#pragma unroll
    for (int u = 0; u < kAppendAhead; ++u) {
      const int t = tb + u;
      if (t >= t1) break;
      const size_t dst = ((page_base * P + (t - lp * P)) * D + i0) * E::kBytes;
      *reinterpret_cast<uint4*>(kc + dst) = kr[u];
      *reinterpret_cast<uint4*>(vc + dst) = vr[u];
      float kf[EPL];
      E::unpack(kr[u], kf);
      n += 1;
      const float rn = float(n);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        mn[e] = fminf(mn[e], kf[e]);
        mx[e] = fmaxf(mx[e], kf[e]);
        // Welford's update of the mean and the sum of squared deviations
        const float delta = kf[e] - mean[e];
        mean[e] += delta / rn;
        m2[e] += delta * (kf[e] - mean[e]);
      }
    }
  }
  if (a.k_box) {
    char* bx = reinterpret_cast<char*>(a.k_box);
    uint4 wmn, wmx;
    if (DT == EKV_BF16) {
      // min/max of bf16 values are bf16 values: the top 16 bits are exact
      uint32_t pm[4], px[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pm[e] = (__float_as_uint(mn[2 * e]) >> 16) | (__float_as_uint(mn[2 * e + 1]) & 0xffff0000u);
        px[e] = (__float_as_uint(mx[2 * e]) >> 16) | (__float_as_uint(mx[2 * e + 1]) & 0xffff0000u);
      }
      wmn = make_uint4(pm[0], pm[1], pm[2], pm[3]);
      wmx = make_uint4(px[0], px[1], px[2], px[3]);
    } else {
      wmn = make_uint4(__float_as_uint(mn[0]), __float_as_uint(mn[1]), __float_as_uint(mn[2]), __float_as_uint(mn[3]));
      wmx = make_uint4(__float_as_uint(mx[0]), __float_as_uint(mx[1]), __float_as_uint(mx[2]), __float_as_uint(mx[3]));
    }
    *reinterpret_cast<uint4*>(bx + ((page_base * 2 + 0) * D + i0) * E::kBytes) = wmn;
    *reinterpret_cast<uint4*>(bx + ((page_base * 2 + 1) * D + i0) * E::kBytes) = wmx;
  }
  if (a.k_moments) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      *reinterpret_cast<float4*>(a.k_moments + (page_base * 2 + 0) * D + i0 + e) =
          make_float4(mean[e], mean[e + 1], mean[e + 2], mean[e + 3]);
      *reinterpret_cast<float4*>(a.k_moments + (page_base * 2 + 1) * D + i0 + e) =
          make_float4(m2[e], m2[e + 1], m2[e + 2], m2[e + 3]);
    }
  }
}

template <int DT, int D>
static hipError_t append_dispatch(const AppendArgs& a, int touched, hipStream_t s) {
  constexpr int UPB = kAppendThreads / (D / Elem<DT>::kPerVec);
  const long long units = (long long)touched * a.n_kv_heads;
  const dim3 grid((unsigned)((units + UPB - 1) / UPB), a.batch), block(kAppendThreads);
  hipLaunchKernelGGL((append_kernel<DT, D>), grid, block, 0, s, a, touched);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n_new <= 0) return hipSuccess;
  const int touched = (a.n_new + a.page_size - 1) / a.page_size + 1;
  if (a.kv_dtype == EKV_BF16)
    return a.head_dim == 128 ? append_dispatch<EKV_BF16, 128>(a, touched, s) : append_dispatch<EKV_BF16, 64>(a, touched, s);
  return a.head_dim == 128 ? append_dispatch<EKV_F32, 128>(a, touched, s) : append_dispatch<EKV_F32, 64>(a, touched, s);
}

}  // namespace ekv
