// Page scoring and candidate selection (EntmaxKV summary sec. 2.A and 2.B).
//
// score_bbox   streams every page's k_min/k_max record once, coalesced, and
//              forms the box upper bound of q.k for each query head of the
//              KV head's group; the page score is the group maximum.
// topk         per (sequence, KV head): radix select of the k-th largest
//              score on order-preserving integer keys, then an ordered
//              compaction (lower page id first among equal scores).
// score_gauss  streams every page's (mean, M2) record once and forms the
//              Gaussian score model (mean_Y, sd_Y, estimated max) per head.
// tau_hat      per (sequence, query head): Newton's method on the expected
//              entmax mass F(t) = sum_p n_p E[(Y_p - t)_+^(1/(alpha-1))] = 1.
// gauss_keep   per (sequence, KV head): keep pages whose estimated maximum
//              beats tau_hat - delta for some head of the group.
#include "ekv_kernels.h"

namespace ekv {

constexpr int kScoreThreads = 256;
constexpr int kBboxPagesPerBlock = 64;
constexpr int kGaussPagesPerBlock = 32;
constexpr int kSelThreads = 1024;

__device__ __forceinline__ int clamp_len(int L, int max_pages, int P, uint32_t* status) {
  if (L < 0 || (long long)L > (long long)max_pages * P) {
    set_status(status, EKV_DEV_BAD_LENGTH);
    return L < 0 ? 0 : max_pages * P;
  }
  return L;
}

// ---------------------------------------------------------------------------
// Bounding-box scoring.  A page record is k_min[D] followed by k_max[D].
// Lane `sub` of the LPP lanes that cover one record holds 16 bytes of either
// half; its coefficients are min(q,0) for the k_min half and max(q,0) for the
// k_max half, so the record's dot product with those coefficients is
// sum_i max(q_i kmin_i, q_i kmax_i) (for q_i >= 0 the max takes kmax_i, for
// q_i < 0 it takes kmin_i).  Accumulation is float64, reductions in a fixed
// butterfly order.
// ---------------------------------------------------------------------------
template <int DT, int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_bbox_kernel(SelectArgs a) {
  using E = Elem<DT>;
  constexpr int EPL = E::kPerVec;
  constexpr int LPH = D / EPL;
  constexpr int LPP = 2 * LPH;
  static_assert(LPP <= kWave && kWave % LPP == 0, "page record must tile a wave");
  constexpr int PPW = kWave / LPP;
  constexpr int NW = kScoreThreads / kWave;
  const int b = blockIdx.z, g = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = lane % LPP, half = sub / LPH, dim0 = (sub % LPH) * EPL;
  const int P = a.page_size, Hkv = a.n_kv_heads;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);

  double c[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G + h) * D + dim0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const double qv = qh[e];
      c[h][e] = half ? fmax(qv, 0.0) : fmin(qv, 0.0);
    }
  }
  float* out = a.scores + ((size_t)b * Hkv + g) * a.max_pages;
  const int p_begin = blockIdx.x * kBboxPagesPerBlock;
  for (int base = p_begin; base < p_begin + kBboxPagesPerBlock; base += NW * PPW) {
    const int p = base + w * PPW + lane / LPP;
    bool valid = p < n_b;
    double acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0;
    if (valid) {
      const int phys = a.page_table[(size_t)b * a.max_pages + p];
      if (phys < 0 || phys >= a.n_phys) {
        set_status(a.status, EKV_DEV_BAD_PAGE);
        valid = false;
      } else {
        const char* rec = reinterpret_cast<const char*>(a.k_box) +
                          (((size_t)phys * Hkv + g) * 2 + half) * D * E::kBytes + (size_t)dim0 * E::kBytes;
        float f[EPL];
        E::unpack(ldg16(rec), f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const double kv = f[e];
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = fma(c[h][e], kv, acc[h]);
        }
      }
    }
#pragma unroll
    for (int m = 1; m < LPP; m <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] += __shfl_xor(acc[h], m, kWave);
    }
    if (sub == 0 && p < a.max_pages && p < p_begin + kBboxPagesPerBlock) {
      double s = acc[0];
#pragma unroll
      for (int h = 1; h < G; ++h) s = fmax(s, acc[h]);
      out[p] = valid ? float(s * (double)a.scale) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k.  One block per (KV head, sequence).  Each thread owns a contiguous
// run of pages so the final compaction writes ascending page ids.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_and_u32(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v &= __shfl_xor(v, m, kWave);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int i = 1; i < nw; ++i) r &= red[i];
  return r;
}
__device__ __forceinline__ uint32_t block_or_u32(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m, kWave);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int i = 1; i < nw; ++i) r |= red[i];
  return r;
}

__global__ __launch_bounds__(kSelThreads) void topk_kernel(SelectArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int unit = b * a.n_kv_heads + g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = a.page_size;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);
  const int k_eff = min(a.top_k, n_b);
  const float* s = a.scores + (size_t)unit * a.max_pages;
  int32_t* out = a.sel + (size_t)unit * a.cap;
  if (k_eff >= n_b) {
    for (int p = tid; p < n_b; p += blockDim.x) out[p] = p;
    if (tid == 0) a.sel_count[unit] = n_b;
    return;
  }
  __shared__ uint32_t hist[256];
  __shared__ uint32_t red[16];
  __shared__ int redi[17];
  __shared__ uint32_t sh_digit, sh_above;
  const int per = (n_b + blockDim.x - 1) / blockDim.x;
  const int e0 = min(tid * per, n_b), e1 = min(e0 + per, n_b);

  uint32_t kand = 0xffffffffu, kor = 0u;
  for (int e = e0; e < e1; ++e) {
    const uint32_t k = f2key(s[e]);
    kand &= k;
    kor |= k;
  }
  kand = block_and_u32(kand, red);
  kor = block_or_u32(kor, red);
  const uint32_t diff = kand ^ kor;
  uint32_t prefix, mask;
  int rem = k_eff;
  if (diff == 0u) {
    prefix = kand;  // every score equal: the k lowest page ids
  } else {
    const int top = 31 - __clz(diff);
    const int start = (top / 8) * 8;
    mask = (start + 8 >= 32) ? 0u : ~((1u << (start + 8)) - 1u);
    prefix = kand & mask;
    for (int shift = start; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0u;
      __syncthreads();
      for (int e = e0; e < e1; ++e) {
        const uint32_t k = f2key(s[e]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (w == 0) {
        const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                       c3 = hist[4 * lane + 3];
        // suffix sum over lanes: S_l = sum of bins >= 4 l
        uint32_t S = c0 + c1 + c2 + c3;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(S, o, kWave);
          if (lane + o < 64) S += t;
        }
        uint32_t Snext = __shfl_down(S, 1, kWave);
        if (lane == 63) Snext = 0u;
        if (S >= (uint32_t)rem && Snext < (uint32_t)rem) {
          uint32_t above = Snext;
          const uint32_t cs[4] = {c0, c1, c2, c3};
          int digit = 4 * lane;
          for (int bin = 3; bin >= 0; --bin) {
            if (above + cs[bin] >= (uint32_t)rem) { digit = 4 * lane + bin; break; }
            above += cs[bin];
          }
          sh_digit = (uint32_t)digit;
          sh_above = above;
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      mask |= 0xffu << shift;
      rem -= (int)sh_above;
      __syncthreads();
    }
  }
  const uint32_t kstar = prefix;  // key of the k-th largest score
  // rem = how many pages with key == kstar to take (the lowest ids first)
  int c_eq = 0;
  for (int e = e0; e < e1; ++e) c_eq += (f2key(s[e]) == kstar);
  int tot;
  const int eq_before = block_exclusive_scan(c_eq, redi, &tot);
  int c_sel = 0, r = eq_before;
  for (int e = e0; e < e1; ++e) {
    const uint32_t k = f2key(s[e]);
    if (k > kstar) ++c_sel;
    else if (k == kstar) { if (r < rem) ++c_sel; ++r; }
  }
  int pos = block_exclusive_scan(c_sel, redi, &tot);
  r = eq_before;
  for (int e = e0; e < e1; ++e) {
    const uint32_t k = f2key(s[e]);
    bool take = k > kstar;
    if (k == kstar) { take = r < rem; ++r; }
    if (take) out[pos++] = e;
  }
  if (tid == 0) a.sel_count[unit] = tot;
}

// ---------------------------------------------------------------------------
// Gaussian scoring.  A page record is mean[D] followed by M2[D] (float32).
// Lanes of the mean half accumulate sum_i q_i mean_i, lanes of the M2 half
// sum_i q_i^2 M2_i; after the in-half butterfly one exchange gives every lane
// both sums.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_gauss_kernel(SelectArgs a) {
  constexpr int EPL = 4;
  constexpr int LPH = D / EPL;
  constexpr int LPP = 2 * LPH;
  static_assert(LPP <= kWave && kWave % LPP == 0 && G <= LPP, "layout");
  constexpr int PPW = kWave / LPP;
  constexpr int NW = kScoreThreads / kWave;
  const int b = blockIdx.z, g = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = lane % LPP, half = sub / LPH, dim0 = (sub % LPH) * EPL;
  const int P = a.page_size, Hkv = a.n_kv_heads;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);
  const double a1s = ((double)a.alpha - 1.0) * (double)a.scale;

  double c[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G + h) * D + dim0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const double qv = qh[e];
      c[h][e] = half ? qv * qv : qv;
    }
  }
  const int p_begin = blockIdx.x * kGaussPagesPerBlock;
  for (int base = p_begin; base < p_begin + kGaussPagesPerBlock; base += NW * PPW) {
    const int p = base + w * PPW + lane / LPP;
    bool valid = p < n_b;
    double acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0;
    if (valid) {
      const int phys = a.page_table[(size_t)b * a.max_pages + p];
      if (phys < 0 || phys >= a.n_phys) {
        set_status(a.status, EKV_DEV_BAD_PAGE);
        valid = false;
      } else {
        const float* rec = a.k_moments + (((size_t)phys * Hkv + g) * 2 + half) * D + dim0;
        const float4 v = *reinterpret_cast<const float4*>(rec);
        const double f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = fma(c[h][e], f[e], acc[h]);
      }
    }
#pragma unroll
    for (int m = 1; m < LPH; m <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] += __shfl_xor(acc[h], m, kWave);
    }
    double other[G];
#pragma unroll
    for (int h = 0; h < G; ++h) other[h] = __shfl_xor(acc[h], LPH, kWave);
    if (sub < G && p < a.max_pages && p < p_begin + kGaussPagesPerBlock) {
      double A = 0.0, Bv = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (h == sub) { A = half ? other[h] : acc[h]; Bv = half ? acc[h] : other[h]; }
      const int hq = g * G + sub;
      float4 r;
      if (valid) {
        const int np = min(P, L - p * P);
        const double mu = a1s * A;
        const double var = a1s * a1s * Bv / (double)np;
        const double sd = sqrt(fmax(var, 0.0));
        const double ehat = mu + sd * sqrt(2.0 * log((double)np));
        r = make_float4((float)mu, (float)sd, (float)ehat, (float)np);
      } else {
        r = make_float4(0.f, 0.f, -INFINITY, 0.f);
      }
      a.stats[((size_t)b * a.n_q_heads + hq) * a.max_pages + p] = r;
    }
  }
}

// ---------------------------------------------------------------------------
// tau_hat: Newton's method on F(t) = sum_p n_p E_p(t) - 1.  F is convex and
// decreasing, and F(max mu - 1) >= 0 (the top page alone contributes at
// least n_p * 1^e by Jensen's inequality), so Newton iterates started there
// increase monotonically to the root.  With u = (mu - t)/sd:
//   exponent 1 (alpha=2):   E = a Phi(u) + sd phi(u),               E' = -Phi(u)
//   exponent 2 (alpha=1.5): E = (a^2 + sd^2) Phi(u) + a sd phi(u),  E' = -2 (a Phi + sd phi)
// with a = mu - t; a page with sd = 0 contributes (a)_+^e.  Pages more than
// 10 standard deviations below t contribute less than 1e-23 sd^e and are
// skipped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void tau_hat_kernel(SelectArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int P = a.page_size;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);
  const size_t bh = (size_t)b * a.n_q_heads + h;
  const float4* st = a.stats + bh * a.max_pages;
  __shared__ double redd[16];
  if (n_b == 0) {
    if (tid == 0) {
      a.tau_hat[bh] = 0.0;
      if (a.tau_hat_out) a.tau_hat_out[bh] = 0.f;
    }
    return;
  }
  double mu_max = -INFINITY;
  for (int p = tid; p < n_b; p += blockDim.x) mu_max = fmax(mu_max, (double)st[p].x);
  mu_max = block_max(mu_max, redd);
  const bool quad = a.alpha == 1.5f;
  const double kInvSqrt2 = 0.70710678118654752440, kInvSqrt2Pi = 0.39894228040143267794;
  double t = mu_max - 1.0;
  for (int it = 0; it < 100; ++it) {
    double F = 0.0, dF = 0.0;
    for (int p = tid; p < n_b; p += blockDim.x) {
      const float4 s = st[p];
      const double mu = s.x, sd = s.y, n = s.w;
      const double am = mu - t;
      if (sd <= 0.0) {
        if (am > 0.0) {
          if (quad) { F += n * am * am; dF -= n * 2.0 * am; }
          else { F += n * am; dF -= n; }
        }
        continue;
      }
      const double u = am / sd;
      if (u < -10.0) continue;
      const double Phi = 0.5 * erfc(-u * kInvSqrt2);
      const double phi = exp(-0.5 * u * u) * kInvSqrt2Pi;
      const double e1 = am * Phi + sd * phi;  // E[(Y - t)_+]
      if (quad) {
        F += n * ((am * am + sd * sd) * Phi + am * sd * phi);
        dF -= n * 2.0 * e1;
      } else {
        F += n * e1;
        dF -= n * Phi;
      }
    }
    F = block_sum(F, redd);
    dF = block_sum(dF, redd);
    const double step = (F - 1.0) / (-dF);
    if (!(step > 0.0)) break;
    t += step;
    if (step <= 1e-14 * fmax(1.0, fabs(t))) break;
  }
  if (tid == 0) {
    a.tau_hat[bh] = t;
    if (a.tau_hat_out) a.tau_hat_out[bh] = (float)t;
  }
}

// ---------------------------------------------------------------------------
// Keep pages whose estimated maximum beats tau_hat - delta for some head of
// the group; ordered compaction; at least one page (the best margin, lowest
// id on ties).
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kSelThreads) void gauss_keep_kernel(SelectArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int unit = b * a.n_kv_heads + g;
  const int tid = threadIdx.x;
  const int P = a.page_size;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);
  int32_t* out = a.sel + (size_t)unit * a.cap;
  __shared__ int redi[17];
  __shared__ double redd[16];
  __shared__ int redp[16];
  if (n_b == 0) {
    if (tid == 0) a.sel_count[unit] = 0;
    return;
  }
  double tau[G];
  const float4* st[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
    tau[h] = a.tau_hat[bh];
    st[h] = a.stats + bh * a.max_pages;
  }
  const double ndelta = -(double)a.delta;
  const int per = (n_b + blockDim.x - 1) / blockDim.x;
  const int e0 = min(tid * per, n_b), e1 = min(e0 + per, n_b);
  auto margin = [&](int p) {
    double m = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) m = fmax(m, (double)st[h][p].z - tau[h]);
    return m;
  };
  int c = 0;
  double best = -INFINITY;
  int best_p = 0x7fffffff;
  for (int p = e0; p < e1; ++p) {
    const double m = margin(p);
    if (m > ndelta) ++c;
    if (m > best) { best = m; best_p = p; }
  }
  int tot;
  int pos = block_exclusive_scan(c, redi, &tot);
  if (tot > 0) {
    for (int p = e0; p < e1; ++p)
      if (margin(p) > ndelta) out[pos++] = p;
    if (tid == 0) a.sel_count[unit] = tot;
    return;
  }
  // floor: the single best page
  const double bm = block_max(best, redd);
  int cand = (best == bm) ? best_p : 0x7fffffff;
  const int lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  cand = wave_min(cand);
  __syncthreads();
  if (lane == 0) redp[w] = cand;
  __syncthreads();
  if (tid == 0) {
    int pbest = redp[0];
    for (int i = 1; i < nw; ++i) pbest = min(pbest, redp[i]);
    out[0] = pbest == 0x7fffffff ? 0 : pbest;  // every page invalid: page 0
    a.sel_count[unit] = 1;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int DT, int D>
static hipError_t bbox_dispatch_g(const SelectArgs& a, dim3 grid, hipStream_t s) {
  switch (a.group) {
    case 1: hipLaunchKernelGGL((score_bbox_kernel<DT, D, 1>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_bbox_kernel<DT, D, 2>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_bbox_kernel<DT, D, 4>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_bbox_kernel<DT, D, 8>), grid, dim3(kScoreThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_bbox(const SelectArgs& a, hipStream_t s) {
  dim3 grid((a.max_pages + kBboxPagesPerBlock - 1) / kBboxPagesPerBlock, a.n_kv_heads, a.batch);
  if (a.kv_dtype == EKV_BF16)
    return a.head_dim == 128 ? bbox_dispatch_g<EKV_BF16, 128>(a, grid, s) : bbox_dispatch_g<EKV_BF16, 64>(a, grid, s);
  return a.head_dim == 128 ? bbox_dispatch_g<EKV_F32, 128>(a, grid, s) : bbox_dispatch_g<EKV_F32, 64>(a, grid, s);
}

hipError_t launch_topk(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_kv_heads, a.batch), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t gauss_dispatch_g(const SelectArgs& a, dim3 grid, hipStream_t s) {
  switch (a.group) {
    case 1: hipLaunchKernelGGL((score_gauss_kernel<D, 1>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_gauss_kernel<D, 2>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_gauss_kernel<D, 4>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_gauss_kernel<D, 8>), grid, dim3(kScoreThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_gauss(const SelectArgs& a, hipStream_t s) {
  dim3 grid((a.max_pages + kGaussPagesPerBlock - 1) / kGaussPagesPerBlock, a.n_kv_heads, a.batch);
  return a.head_dim == 128 ? gauss_dispatch_g<128>(a, grid, s) : gauss_dispatch_g<64>(a, grid, s);
}

hipError_t launch_tau_hat(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(tau_hat_kernel, dim3(a.n_q_heads, a.batch), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gauss_keep(const SelectArgs& a, hipStream_t s) {
  dim3 grid(a.n_kv_heads, a.batch), block(kSelThreads);
  switch (a.group) {
    case 1: hipLaunchKernelGGL(gauss_keep_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(gauss_keep_kernel<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(gauss_keep_kernel<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(gauss_keep_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ekv
