// append_kv: write new tokens into their page slots and keep the per-page
// metadata current (EntmaxKV summary sec. 2.A keeps k_min/k_max and the key
// moments per page; sec. 1: the cache grows by one token per decode step).
//
// One workgroup per (KV head, touched page, sequence); thread i owns key
// coordinate i.  The workgroup folds the page's new tokens in token order,
// so one call with n tokens and n calls with one token produce the same bits.
#include "ekv_kernels.h"

namespace ekv {

template <int DT>
__global__ void append_kernel(AppendArgs a) {
  using E = Elem<DT>;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int i = threadIdx.x;  // coordinate
  const int P = a.page_size, D = a.head_dim, Hkv = a.n_kv_heads;
  const int L = a.seq_lens[b];
  if (L < 0 || (long long)L + a.n_new > (long long)a.max_pages * P) {
    if (i == 0 && g == 0 && j == 0) set_status(a.status, EKV_DEV_BAD_LENGTH);
    return;
  }
  const int lp = L / P + j;
  const int t0 = max(L, lp * P), t1 = min(L + a.n_new, (lp + 1) * P);
  if (t0 >= t1) return;
  const int phys = a.page_table[(size_t)b * a.max_pages + lp];
  if (phys < 0 || phys >= a.n_phys) {
    if (i == 0 && g == 0) set_status(a.status, EKV_DEV_BAD_PAGE);
    return;
  }
  if (i >= D) return;
  const int slot0 = t0 - lp * P;
  const size_t page_base = ((size_t)phys * Hkv + g);
  float mn = INFINITY, mx = -INFINITY, mean = 0.f, m2 = 0.f;
  if (slot0 > 0) {  // continue an existing page
    if (a.k_box) {
      mn = E::load1(a.k_box, (page_base * 2 + 0) * D + i);
      mx = E::load1(a.k_box, (page_base * 2 + 1) * D + i);
    }
    if (a.k_moments) {
      mean = a.k_moments[(page_base * 2 + 0) * D + i];
      m2 = a.k_moments[(page_base * 2 + 1) * D + i];
    }
  }
  int n = slot0;
  for (int t = t0; t < t1; ++t) {
    const size_t src = (((size_t)b * a.n_new + (t - L)) * Hkv + g) * D + i;
    const size_t dst = (page_base * P + (t - lp * P)) * D + i;
    float kf;
    if (DT == EKV_BF16) {
      const uint16_t kb = reinterpret_cast<const uint16_t*>(a.k_new)[src];
      const uint16_t vb = reinterpret_cast<const uint16_t*>(a.v_new)[src];
      reinterpret_cast<uint16_t*>(a.k)[dst] = kb;
      reinterpret_cast<uint16_t*>(a.v)[dst] = vb;
      kf = __uint_as_float(uint32_t(kb) << 16);
    } else {
      kf = reinterpret_cast<const float*>(a.k_new)[src];
      reinterpret_cast<float*>(a.k)[dst] = kf;
      reinterpret_cast<float*>(a.v)[dst] = reinterpret_cast<const float*>(a.v_new)[src];
    }
    mn = fminf(mn, kf);
    mx = fmaxf(mx, kf);
    // Welford's update of the mean and the sum of squared deviations.
    n += 1;
    const float delta = kf - mean;
    mean += delta / float(n);
    m2 += delta * (kf - mean);
  }
  if (a.k_box) {
    if (DT == EKV_BF16) {
      // min/max of bf16 values are bf16 values: the top 16 bits are exact.
      reinterpret_cast<uint16_t*>(a.k_box)[(page_base * 2 + 0) * D + i] = uint16_t(__float_as_uint(mn) >> 16);
      reinterpret_cast<uint16_t*>(a.k_box)[(page_base * 2 + 1) * D + i] = uint16_t(__float_as_uint(mx) >> 16);
    } else {
      reinterpret_cast<float*>(a.k_box)[(page_base * 2 + 0) * D + i] = mn;
      reinterpret_cast<float*>(a.k_box)[(page_base * 2 + 1) * D + i] = mx;
    }
  }
  if (a.k_moments) {
    a.k_moments[(page_base * 2 + 0) * D + i] = mean;
    a.k_moments[(page_base * 2 + 1) * D + i] = m2;
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n_new <= 0) return hipSuccess;
  const int touched = (a.n_new + a.page_size - 1) / a.page_size + 1;
  dim3 grid(touched, a.n_kv_heads, a.batch), block(a.head_dim);
  if (a.kv_dtype == EKV_BF16)
    hipLaunchKernelGGL(append_kernel<EKV_BF16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<EKV_F32>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ekv
