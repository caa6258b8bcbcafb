// Sparse (or full-cache) exact alpha-entmax decode (EntmaxKV summary
// sec. 2.C: load only the selected pages' keys and values and compute the
// alpha-entmax weights over that reduced set).
//
// gather_score  persistent grid over work items; an item is up to `ppi`
//               consecutive entries of a (sequence, KV head)'s page list.
//               Each K row is read once with 16-byte lane loads and scored
//               against every query head of the group (x = (alpha-1) scale
//               q.k, float32).  The item keeps only candidates that can be
//               in the support: x > m - 1, where m is a lower bound on the
//               head's maximum (its own maximum, or the running maximum
//               published with an integer atomic) - the threshold satisfies
//               tau >= max x - 1 because the top token's weight is at most 1.
// tau_v         one block per (sequence, query head): collects the
//               candidates above (final max) - 1, finds the exact threshold
//               and support, and accumulates sum_j p_j v_j over the support
//               (rows split across the block, fixed-order combine).
#include "ekv_kernels.h"

namespace ekv {

constexpr int kDecThreads = 256;
constexpr int kTauThreads = 256;

__device__ __forceinline__ int dec_len(const DecodeArgs& a, int b) {
  const int L = a.seq_lens[b];
  if (L < 0 || (long long)L > (long long)a.max_pages * a.page_size) return L < 0 ? 0 : a.max_pages * a.page_size;
  return L;
}

// Number of page-list entries of unit u = b * Hkv + g.
__device__ __forceinline__ int unit_pages(const DecodeArgs& a, int u) {
  const int b = u / a.n_kv_heads;
  const int n_b = pages_of(dec_len(a, b), a.page_size);
  if (!a.sel) return n_b;
  return min(max(a.sel_count[u], 0), min(a.cap, n_b));
}

template <int DT, int D, int G>
__global__ __launch_bounds__(kDecThreads) void gather_score_kernel(DecodeArgs a) {
  using E = Elem<DT>;
  constexpr int EPL = E::kPerVec;
  constexpr int LPR = D / EPL;         // lanes per K row
  static_assert(LPR <= kWave && G <= LPR, "layout");
  constexpr int RPW = kWave / LPR;     // rows per wave load
  constexpr int NW = kDecThreads / kWave;
  constexpr int RPI = NW * RPW;        // rows per block iteration
  // dynamic LDS: prefix[n_units + 1] | x[G][ppi * P] | phys[ppi] | np[ppi] | lp[ppi]
  extern __shared__ int smem[];
  __shared__ int redi[17];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane % LPR, dim0 = sub * EPL, rloc = lane / LPR;
  const int P = a.page_size, Hkv = a.n_kv_heads, ppi = a.ppi;
  const int n_units = a.batch * Hkv;
  const int tpi = ppi * P;
  const size_t max_tok = (size_t)a.max_pages * P;
  int* s_prefix = smem;
  float* s_xall = reinterpret_cast<float*>(smem + n_units + 1);
  int* s_phys = smem + n_units + 1 + G * tpi;
  int* s_np = s_phys + ppi;
  int* s_lp = s_np + ppi;

  // item prefix over units (same on every block)
  int running = 0;
  for (int u0 = 0; u0 < n_units; u0 += kDecThreads) {
    const int u = u0 + tid;
    const int items = u < n_units ? (unit_pages(a, u) + ppi - 1) / ppi : 0;
    int tot;
    const int ex = block_exclusive_scan(items, redi, &tot);
    if (u < n_units) s_prefix[u] = running + ex;
    running += tot;
  }
  if (tid == 0) s_prefix[n_units] = running;
  __syncthreads();
  const int total_items = running;

  int cur_u = -1;
  float qr[G][EPL];
  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    // unit of this item: last u with s_prefix[u] <= item
    int lo = 0, hi = n_units;  // invariant: s_prefix[lo] <= item < s_prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_prefix[mid] <= item) lo = mid; else hi = mid;
    }
    const int u = lo, j = item - s_prefix[u];
    const int b = u / Hkv, g = u % Hkv;
    const int L = dec_len(a, b);
    const int n_b = pages_of(L, P);
    const int npu = unit_pages(a, u);
    const int k0 = j * ppi, npg = min(k0 + ppi, npu) - k0;
    if (tid < npg) {
      int lp = a.sel ? a.sel[(size_t)u * a.cap + k0 + tid] : k0 + tid;
      int phys = -1, np = 0;
      if (lp < 0 || lp >= n_b) {
        set_status(a.status, EKV_DEV_BAD_PAGE);
        lp = 0;
      } else {
        phys = a.page_table[(size_t)b * a.max_pages + lp];
        if (phys < 0 || phys >= a.n_phys) {
          set_status(a.status, EKV_DEV_BAD_PAGE);
          phys = -1;
        } else {
          np = min(P, L - lp * P);
        }
      }
      s_lp[tid] = lp;
      s_phys[tid] = phys;
      s_np[tid] = np;
    }
    if (u != cur_u) {
      cur_u = u;
      const float qs = (a.alpha - 1.f) * a.scale;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float* qh = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G + h) * D + dim0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) qr[h][e] = qh[e] * qs;
      }
    }
    __syncthreads();
    const int ntok = npg * P;
    for (int r0 = 0; r0 < ntok; r0 += RPI) {
      const int r = r0 + w * RPW + rloc;
      const int kk = r / P, slot = r - kk * P;
      const bool valid = r < ntok && slot < s_np[min(kk, npg - 1)];
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      if (valid) {
        const char* row = reinterpret_cast<const char*>(a.k) +
                          ((((size_t)s_phys[kk] * Hkv + g) * P + slot) * D + dim0) * E::kBytes;
        float f[EPL];
        E::unpack(ldg16(row), f);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = fmaf(qr[h][e], f[e], acc[h]);
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] += __shfl_xor(acc[h], m, kWave);
      }
      if (r < ntok && sub < G) {
        float v = acc[0];
#pragma unroll
        for (int h = 1; h < G; ++h) if (sub == h) v = acc[h];
        s_xall[sub * tpi + r] = valid ? v : -INFINITY;
      }
    }
    __syncthreads();
    // per head: item maximum, candidate threshold, ordered compaction
    for (int h = w; h < G; h += NW) {
      float m = -INFINITY;
      for (int r = lane; r < ntok; r += kWave) m = fmaxf(m, s_xall[h * tpi + r]);
      m = wave_max(m);
      const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
      int cnt = 0;
      if (m > -INFINITY) {
        uint32_t old = 0;
        if (lane == 0) old = atomicMax(&a.max_key[bh], f2key(m));
        old = __shfl(old, 0, kWave);
        const double thr = (double)fmaxf(m, old ? key2f(old) : m) - 1.0;
        const size_t region = bh * max_tok + (size_t)j * ppi * P;
        for (int r0 = 0; r0 < ntok; r0 += kWave) {
          const int r = r0 + lane;
          const float x = r < ntok ? s_xall[h * tpi + r] : -INFINITY;
          const bool keep = (double)x > thr;
          const unsigned long long bal = __ballot(keep);
          if (keep) {
            const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
            const int kk = r / P;
            a.cand_x[region + pos] = x;
            a.cand_t[region + pos] = s_lp[kk] * P + (r - kk * P);
          }
          cnt += __popcll(bal);
        }
      }
      if (lane == 0) {
        a.item_cnt[bh * a.max_pages + j] = cnt;
        a.item_max[bh * a.max_pages + j] = m;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Exact threshold over the candidates (float64).  Let S(t) = {x_j > t}.  The
// solve keeps t <= tau and S(t) a superset of the support:
//   * closed form on S(t): alpha=2: r = (sum x - 1)/|S|; alpha=1.5: r solves
//     sum (x - r)^2 = 1 (smaller root).  If r < min over S(t) of x, S(t) is
//     the support and tau = r (the sort-based criterion: a top-k set passes
//     exactly when it is the support).  Otherwise the smallest member is not
//     in the support and t may move up to it.
//   * Newton's step on f(t) = sum (x - t)_+^e - 1 (convex, decreasing) from
//     the left also never passes tau.
// t takes the larger of the two, so every failed round drops >= 1 element.
// For other alpha only Newton runs, to convergence.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(kTauThreads) void tau_v_kernel(DecodeArgs a) {
  using E = Elem<DT>;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int G = a.group, g = h / G, Hkv = a.n_kv_heads, P = a.page_size;
  const int u = b * Hkv + g;
  const size_t bh = (size_t)b * a.n_q_heads + h;
  const size_t max_tok = (size_t)a.max_pages * P;
  __shared__ float lx[kLdsCands];
  __shared__ int lt[kLdsCands];
  __shared__ double redd[16];
  __shared__ int redi[17];
  __shared__ float vpart[kTauThreads / (D / E::kPerVec)][D];

  const int ppi = a.ppi;
  const int npu = unit_pages(a, u);
  const int n_items = (npu + ppi - 1) / ppi;
  const uint32_t mk = a.max_key[bh];
  __syncthreads();
  if (tid == 0) a.max_key[bh] = 0u;  // leave the control word clean for the next step
  float* out = a.out + bh * D;
  if (n_items == 0 || mk == 0u) {
    for (int e = tid; e < D; e += blockDim.x) out[e] = 0.f;
    if (tid == 0) {
      if (a.tau) a.tau[bh] = -INFINITY;
      if (a.support_count) a.support_count[bh] = 0;
      if (a.psum) a.psum[bh] = 0.f;
    }
    return;
  }
  const double m = key2f(mk);
  const double thr = m - 1.0;
  const int32_t* icnt = a.item_cnt + bh * a.max_pages;
  const float* cx = a.cand_x + bh * max_tok;
  const int32_t* ct = a.cand_t + bh * max_tok;

  // ---- collect candidates above m - 1, in item order ----
  int N = 0;
  for (int j0 = 0; j0 < n_items; j0 += kTauThreads) {
    const int j = j0 + tid;
    int c = 0;
    if (j < n_items) {
      const size_t base = (size_t)j * ppi * P;
      const int n = icnt[j];
      for (int i = 0; i < n; ++i) c += (double)cx[base + i] > thr;
    }
    int tot;
    block_exclusive_scan(c, redi, &tot);
    N += tot;
  }
  const bool in_lds = N <= kLdsCands;
  float* xs = in_lds ? lx : a.ovf_x + bh * max_tok;
  int32_t* ts = in_lds ? lt : a.ovf_t + bh * max_tok;
  int run = 0;
  for (int j0 = 0; j0 < n_items; j0 += kTauThreads) {
    const int j = j0 + tid;
    int c = 0, n = 0;
    size_t base = 0;
    if (j < n_items) {
      base = (size_t)j * ppi * P;
      n = icnt[j];
      for (int i = 0; i < n; ++i) c += (double)cx[base + i] > thr;
    }
    int tot;
    int pos = run + block_exclusive_scan(c, redi, &tot);
    for (int i = 0; i < n; ++i) {
      const float x = cx[base + i];
      if ((double)x > thr) { xs[pos] = x; ts[pos] = ct[base + i]; ++pos; }
    }
    run += tot;
  }
  __syncthreads();

  // ---- threshold ----
  const double alpha = a.alpha;
  const bool sparsemax = a.alpha == 2.0f, ent15 = a.alpha == 1.5f;
  const double beta = 1.0 / (alpha - 1.0);
  double t = thr, tau = thr, t_prev = thr;
  for (int it = 0; it < 4096; ++it) {
    tau = t;  // fallback if the iteration cap is ever reached
    double s1 = 0.0, s2 = 0.0, f = 0.0, fd = 0.0, xmin = INFINITY;
    double cnt = 0.0;
    for (int i = tid; i < N; i += blockDim.x) {
      const double x = xs[i];
      if (x > t) {
        const double y = x - m, d = x - t;
        cnt += 1.0; s1 += y; s2 += y * y; xmin = fmin(xmin, x);
        if (sparsemax) { f += d; fd += 1.0; }
        else if (ent15) { f += d * d; fd += 2.0 * d; }
        else { const double pw = pow(d, beta); f += pw; fd += beta * pw / d; }
      }
    }
    cnt = block_sum(cnt, redd);
    s1 = block_sum(s1, redd);
    s2 = block_sum(s2, redd);
    f = block_sum(f, redd);
    fd = block_sum(fd, redd);
    xmin = block_min(xmin, redd);
    if (cnt == 0.0) { tau = t_prev; break; }  // only reachable through rounding
    t_prev = t;
    if (sparsemax || ent15) {
      bool ok = false;
      double r = 0.0;
      if (sparsemax) {
        r = m + (s1 - 1.0) / cnt;
        ok = true;
      } else {
        const double mu = s1 / cnt;
        const double disc = (1.0 - cnt * (s2 / cnt - mu * mu)) / cnt;
        if (disc >= 0.0) { r = m + mu - sqrt(disc); ok = true; }
      }
      if (ok && r < xmin) { tau = r; break; }
      const double tn = t + (f - 1.0) / fd;
      t = fmax(tn, xmin);
    } else {
      const double step = (f - 1.0) / fd;
      if (!(step > 0.0)) { tau = t; break; }
      t += step;
      tau = t;
      if (step <= 1e-15 * fmax(1.0, fabs(t))) break;
    }
  }

  // ---- support, weights, compaction in place (p replaces x) ----
  double ps = 0.0;
  int nsup = 0;
  for (int i0 = 0; i0 < N; i0 += kTauThreads) {
    const int i = i0 + tid;
    float x = 0.f;
    int tok = 0;
    bool in = false;
    if (i < N) { x = xs[i]; tok = ts[i]; in = (double)x > tau; }
    double p = 0.0;
    if (in) {
      const double d = (double)x - tau;
      p = sparsemax ? d : (ent15 ? d * d : pow(d, beta));
      ps += p;
    }
    int tot;
    const int pos = nsup + block_exclusive_scan(in ? 1 : 0, redi, &tot);  // syncs before writing
    if (in) {
      xs[pos] = (float)p;
      ts[pos] = tok;
      if (a.support_idx && pos < a.support_cap) a.support_idx[bh * a.support_cap + pos] = tok;
    }
    nsup += tot;
    __syncthreads();
  }
  ps = block_sum(ps, redd);

  // ---- sum_j p_j v_j ----
  constexpr int EPL = E::kPerVec;
  constexpr int LPR = D / EPL;
  constexpr int RPB = kTauThreads / LPR;
  const int rr = tid / LPR, sub = tid % LPR;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int s = rr; s < nsup; s += RPB) {
    const int tok = ts[s];
    const float p = xs[s];
    const int lp = tok / P, slot = tok - lp * P;
    const int phys = a.page_table[(size_t)b * a.max_pages + lp];
    if (phys < 0 || phys >= a.n_phys) continue;
    const char* row = reinterpret_cast<const char*>(a.v) +
                      ((((size_t)phys * Hkv + g) * P + slot) * D + (size_t)sub * EPL) * E::kBytes;
    float f[EPL];
    E::unpack(ldg16(row), f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, f[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) vpart[rr][sub * EPL + e] = acc[e];
  __syncthreads();
  for (int e = tid; e < D; e += blockDim.x) {
    float o = 0.f;
    for (int r = 0; r < RPB; ++r) o += vpart[r][e];
    out[e] = o;
  }
  if (tid == 0) {
    if (a.tau) a.tau[bh] = (float)tau;
    if (a.support_count) a.support_count[bh] = nsup;
    if (a.psum) a.psum[bh] = (float)ps;
  }
}

size_t gather_lds_bytes(int n_units, int group, int ppi, int page_size) {
  return 4 * ((size_t)n_units + 1 + (size_t)group * ppi * page_size + 3 * (size_t)ppi);
}

template <int DT, int D>
static hipError_t decode_dispatch(const DecodeArgs& a, int grid_items, hipStream_t s) {
  const dim3 g1(grid_items), b1(kDecThreads);
  const size_t lds = gather_lds_bytes(a.batch * a.n_kv_heads, a.group, a.ppi, a.page_size);
  switch (a.group) {
    case 1: hipLaunchKernelGGL((gather_score_kernel<DT, D, 1>), g1, b1, lds, s, a); break;
    case 2: hipLaunchKernelGGL((gather_score_kernel<DT, D, 2>), g1, b1, lds, s, a); break;
    case 4: hipLaunchKernelGGL((gather_score_kernel<DT, D, 4>), g1, b1, lds, s, a); break;
    case 8: hipLaunchKernelGGL((gather_score_kernel<DT, D, 8>), g1, b1, lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tau_v_kernel<DT, D>), dim3(a.n_q_heads, a.batch), dim3(kTauThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int grid_items, hipStream_t s) {
  if (a.kv_dtype == EKV_BF16)
    return a.head_dim == 128 ? decode_dispatch<EKV_BF16, 128>(a, grid_items, s)
                             : decode_dispatch<EKV_BF16, 64>(a, grid_items, s);
  return a.head_dim == 128 ? decode_dispatch<EKV_F32, 128>(a, grid_items, s)
                           : decode_dispatch<EKV_F32, 64>(a, grid_items, s);
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace ekv
