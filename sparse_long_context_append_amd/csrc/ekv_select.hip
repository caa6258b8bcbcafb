// Page scoring and candidate selection (EntmaxKV summary sec. 2.A and 2.B).
//
// score_bbox   streams every page's k_min/k_max record once and forms the
//              box upper bound of q.k for each query head of the KV head's
//              group; the page score is the group maximum.  For bf16 records
//              and groups of up to 4 heads the dot products run on the
//              matrix cores (q split into three bf16 limbs, see below);
//              otherwise on the vector ALUs in float64.
// topk         per (sequence, KV head): radix select of the k-th largest
//              score on order-preserving integer keys held in registers,
//              then an ordered compaction (lower page id first on ties).
// score_gauss  streams every page's (mean, M2) record once and forms the
//              Gaussian score model (mean_Y, sd_Y, estimated max) per head.
// tau_hat      per (sequence, query head): Newton's method on the expected
//              entmax mass F(t) = sum_p n_p E[(Y_p - t)_+^(1/(alpha-1))] = 1.
// gauss_keep   per (sequence, KV head): keep pages whose estimated maximum
//              beats tau_hat - delta for some head of the group.
#include "ekv_kernels.h"

namespace ekv {

constexpr int kScoreThreads = 256;
constexpr int kBboxPagesPerBlock = 64;   // 16 pages per wave
constexpr int kGaussPagesPerBlock = 64;  // 8 lane groups per wave, 2 pages each
constexpr int kSelThreads = 1024;
constexpr int kTauHatThreads = 1024;
constexpr int kTauHatLive = 8192;        // pages alive at the start point kept in LDS
constexpr int kTauHatLiveBig = 16384;    // the same for sequences of more than 8192 pages (one block per CU)

__device__ __forceinline__ int clamp_len(int L, int max_pages, int P, uint32_t* status) {
  if (L < 0 || (long long)L > (long long)max_pages * P) {
    set_status(status, EKV_DEV_BAD_LENGTH);
    return L < 0 ? 0 : max_pages * P;
  }
  return L;
}

// Physical page of logical page p of sequence b.  The table entry is read
// before the sequence length is known (p < max_pages keeps it inside the
// table), so the two loads travel together; the length check follows.
__device__ __forceinline__ int page_phys_spec(const SelectArgs& a, int b, int p, int* n_b_out) {
  const int raw = p < a.max_pages ? a.page_table[(size_t)b * a.max_pages + p] : -1;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, a.page_size, a.status);
  const int n_b = pages_of(L, a.page_size);
  *n_b_out = n_b;
  if (p >= n_b) return -1;
  if (raw < 0 || raw >= a.n_phys) {
    set_status(a.status, EKV_DEV_BAD_PAGE);
    return -1;
  }
  return raw;
}

__device__ __forceinline__ int page_phys(const SelectArgs& a, int b, int p, int n_b) {
  if (p >= n_b) return -1;
  const int phys = a.page_table[(size_t)b * a.max_pages + p];
  if (phys < 0 || phys >= a.n_phys) {
    set_status(a.status, EKV_DEV_BAD_PAGE);
    return -1;
  }
  return phys;
}

// Top-k candidate list of one wave's kCandListPages pages, one page per
// lane: key is the lane's page score key (0 past the sequence end).  The
// values v = (key << 6 | 63 - lane) are distinct and order the pages by
// score, ties to the lower page.  The (kCandPerList + 1)-th largest value is
// found bit by bit (one ballot per bit, from the highest bit where the values
// differ until one value is left); the pages above it are listed in page
// order with zero padding, and its key is the list's cut (0 when no page is
// left out).
__device__ __forceinline__ void write_candidates(const SelectArgs& a, uint32_t key, int unit, int list, int page0) {
  static_assert(kCandListPages == kWave, "one page per lane");
  const int lane = threadIdx.x & 63;
  const uint64_t v = (uint64_t)key << 6 | (uint32_t)(kCandListPages - 1 - lane);
  const uint32_t vhi = (uint32_t)(v >> 32), vlo = (uint32_t)v;
  // the highest bit where the values differ is the highest bit of max ^ min
  // (every value lies between them); equal keys differ in the low 6 bits
  const uint32_t kmax = wave_max(key), kmin = wave_min(key);
  int bit = kmax != kmin ? 31 - __clz(kmax ^ kmin) + 6 : 5;
  uint64_t alive = ~0ull;  // lanes whose value agrees with the wanted one on the bits so far
  int want = kCandPerList + 1;  // rank of the wanted value among the alive ones, 1 = largest
  int n_alive = kCandListPages;
  // eight bits per round: the ballots do not depend on the search, so they
  // are issued together and only the scalar counts run in sequence.  Bits
  // past the last one (and bits after one value is left) keep the alive set
  for (; bit >= 0 && n_alive > 1; bit -= 8) {
    uint64_t B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bb = bit - i;
      const uint32_t word = bb >= 32 ? vhi : vlo;
      const uint64_t past = (uint64_t)((int64_t)bb >> 63);  // all ones below bit 0
      B[i] = __ballot((word >> (bb & 31)) & 1u) & ~past;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t x1 = alive & B[i], x0 = alive ^ x1;  // alive values with this bit 1, 0
      const int c1 = __popcll(x1);
      const bool one = c1 >= want;
      alive = one ? x1 : x0;
      want = one ? want : want - c1;
      n_alive = one ? c1 : n_alive - c1;
    }
  }
  const int l = __ffsll((long long)alive) - 1;  // the one value left
  const uint64_t kw = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)vhi, l) << 32 |
                      (uint32_t)__builtin_amdgcn_readlane((int)vlo, l);
  const bool in = v > kw && (v >> 6) != 0ull;
  const uint64_t I = __ballot(in);
  const int pos = __popcll(I & ((1ull << lane) - 1ull)), tot = __popcll(I);
  const size_t row = (size_t)unit * a.cand_lists + list;
  uint64_t* cl = a.cand + row * kCandPerList;
  if (in) cl[pos] = (v >> 6) << 32 | (uint32_t)(page0 + lane);
  if (lane >= tot && lane < kCandPerList) cl[lane] = 0ull;
  if (lane == 0) a.cand_cut[row] = (uint32_t)(kw >> 6);
}

// ---------------------------------------------------------------------------
// Bounding-box score on the matrix cores.
//
// The box bound is linear in the record: with c_h = [min(q_h,0) | max(q_h,0)]
// over the record [k_min | k_max], sum_i max(q_i kmin_i, q_i kmax_i) = c_h .
// record (q_i >= 0 picks kmax_i, q_i < 0 picks kmin_i).  So the scores of 16
// pages are one 16 x 2D by 2D x 16 product.  The A rows are 4h + l, holding
// limb l of c_h: c = l0 + l1 + l2 in bf16 with the remainder below 2^-24 |c|,
// and bf16 x bf16 products are exact in fp32, so the products carry the full
// fp32 coefficient.  Each 32-wide k block is accumulated from zero by the
// matrix core and the block sums are added in float64.  A group of 8 heads
// takes two such operands against the same record fragment.
// ---------------------------------------------------------------------------
template <int D, int G, int NG>
__global__ __launch_bounds__(kScoreThreads) void score_bbox_mfma_kernel(SelectArgs a) {
  constexpr int K = 2 * D;   // record length (bf16 elements)
  constexpr int KB = K / 32;  // k blocks
  constexpr int NH = (G + 3) / 4;  // 16-row operands (four heads each)
  __shared__ u32x4_t s_a[NH * KB][kWave];
  __shared__ uint32_t s_key[NG == 4 ? kCandBlockPages : 1];  // the block's page score keys (top-k lists)
  const int b = blockIdx.z, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = a.n_kv_heads;
  // wave w handles page groups ng*4 + w (16 pages each) of this block
  const int p0 = blockIdx.x * (64 * NG) + col;

  // loads, in order: q for the A operand, page-table entries, page records
  const float* qg = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * D;
  LimbChunks<KB, NH> lc;
  limb_fetch<KB, G, NH>(lc, [&](int h, int k0, float* v) {
    const int half = k0 >= D;
    const float4* qv = reinterpret_cast<const float4*>(qg + (size_t)h * D + (k0 - half * D));
    const float4 q0 = qv[0], q1 = qv[1];
    v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w; v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  });
  int phys[NG];
  int n_b = 0;
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) phys[ng] = page_phys_spec(a, b, p0 + (ng * 4 + w) * 16, &n_b);
  u32x4_t bv[NG][KB];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    if (phys[ng] >= 0) {
      const uint16_t* rec = reinterpret_cast<const uint16_t*>(a.k_box) + ((size_t)phys[ng] * a.hkv_mem + (g >> a.kv_shift)) * K + 8 * grp;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) bv[ng][kb] = *reinterpret_cast<const u32x4_t*>(rec + 32 * kb);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) bv[ng][kb] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // coefficients [min(q,0) | max(q,0)] over the record, as bf16 limbs
  limb_build<KB, G, NH>(s_a, lc, [](int k, float qv) { return k >= D ? fmaxf(qv, 0.f) : fminf(qv, 0.f); });
  __syncthreads();

#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    double U[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      U[hh] = 0.0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f32x4_t c = mfma_bf16(s_a[hh * KB + kb][lane], bv[ng][kb], f32x4_t{0.f, 0.f, 0.f, 0.f});
        U[hh] += ((double)c[0] + (double)c[1]) + (double)c[2];
      }
    }
    // lane holds heads grp, grp + 4, ... of page `col`; the shared page
    // score is the group maximum, the per-head score the lane's own values
    const int p = p0 + (ng * 4 + w) * 16;
    if (a.per_head_scores) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int h = 4 * hh + grp;
        if (h < G && p < a.max_pages)
          a.scores[((size_t)b * a.n_q_heads + (size_t)g * G + h) * a.score_stride + p] =
              phys[ng] >= 0 ? float(U[hh] * (double)a.scale) : -INFINITY;
      }
      continue;
    }
    double S = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) S = 4 * hh + grp < G ? fmax(S, U[hh]) : S;
    S = fmax(S, __shfl_xor(S, 16, kWave));
    S = fmax(S, __shfl_xor(S, 32, kWave));
    const float sc = phys[ng] >= 0 ? float(S * (double)a.scale) : -INFINITY;
    if (grp == 0 && p < a.max_pages) a.scores[((size_t)b * Hkv + g) * a.score_stride + p] = sc;
    if (NG == 4 && grp == 0) s_key[NG == 4 ? (ng * 4 + w) * 16 + col : 0] = p < n_b ? f2key(sc) : 0u;
  }
  if (NG == 4 && a.cand_lists > 0) {
    // wave w lists the block's pages 64 w .. 64 w + 63, one per lane
    __syncthreads();
    write_candidates(a, s_key[NG == 4 ? w * kCandListPages + lane : 0], b * Hkv + g, blockIdx.x * 4 + w,
                     blockIdx.x * kCandBlockPages + w * kCandListPages);
  }
}

// ---------------------------------------------------------------------------
// Bounding-box score on the vector ALUs (fp32 records): four
// lanes per page record, each lane walks a quarter of the record in 16-byte
// loads issued together; coefficients min(q,0) / max(q,0) as above, float64
// accumulation, a two-step reduction across the four lanes.
// ---------------------------------------------------------------------------
template <int DT, int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_bbox_valu_kernel(SelectArgs a) {
  using E = Elem<DT>;
  constexpr int EPL = E::kPerVec;
  constexpr int VEC = 2 * D / EPL;  // 16-byte vectors per record
  constexpr int NL = VEC / 4;       // loads per lane (four lanes per record)
  const int b = blockIdx.z, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane & 3;
  const int Hkv = a.n_kv_heads;
  const int p = blockIdx.x * kBboxPagesPerBlock + w * 16 + (lane >> 2);
  int n_b;
  const int phys = page_phys_spec(a, b, p, &n_b);
  uint4 v[NL];
  if (phys >= 0) {
    const char* rec = reinterpret_cast<const char*>(a.k_box) + ((size_t)phys * a.hkv_mem + (g >> a.kv_shift)) * 2 * D * E::kBytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = ldg16(rec + 16 * (sub + 4 * i));
  }
  double acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.0;
  if (phys >= 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float f[EPL];
      E::unpack(v[i], f);
      const int e0 = EPL * (sub + 4 * i);
      const bool half = e0 >= D;
      const int dim0 = e0 - (half ? D : 0);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float* qh = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G + h) * D + dim0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const double qv = qh[e];
          acc[h] = fma(half ? fmax(qv, 0.0) : fmin(qv, 0.0), (double)f[e], acc[h]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc[h] = group_reduce<4>(acc[h], [](double u, double v) { return u + v; });
  }
  if (sub == 0 && p < a.max_pages && a.per_head_scores) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      a.scores[((size_t)b * a.n_q_heads + (size_t)g * G + h) * a.score_stride + p] =
          phys >= 0 ? float(acc[h] * (double)a.scale) : -INFINITY;
  } else if (sub == 0 && p < a.max_pages) {
    double s = acc[0];
#pragma unroll
    for (int h = 1; h < G; ++h) s = fmax(s, acc[h]);
    a.scores[((size_t)b * Hkv + g) * a.score_stride + p] = phys >= 0 ? float(s * (double)a.scale) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Top-k.  One 1024-thread block per (KV head, sequence).  With E > 0 thread
// t owns the page slots [t E, t E + E) of the score row (E chosen on the host
// from the table width, E * 1024 >= max_pages), and its keys stay in
// registers; they are requested before the sequence length is known and the
// slots at or past it are masked afterwards.  With E == 0 (more than 16384
// pages) thread t owns ceil(n / 1024) pages and re-reads them from L2.
// ---------------------------------------------------------------------------
struct RadixSmem {
  uint32_t hist[2][256];
  uint32_t red[4][16];
  uint32_t redu[16];
  uint32_t digit[2], above[2], bucket[2];
};

// The k-th largest key, resolved as far as the selection needs: every key k
// with (k & mask) > prefix is taken, and `rem` of those with (k & mask) ==
// prefix, lowest page id first.  prefix is at most every taken key.
struct KthKey {
  uint32_t prefix, mask;
  int rem;
};

__device__ __forceinline__ void radix_clear(RadixSmem& r) {
  for (int i = threadIdx.x; i < 512; i += blockDim.x) (&r.hist[0][0])[i] = 0u;
}

// Radix select over the block's keys, given their AND and OR over the block.
// for_keys(f) calls f(key) for each key this thread holds.  Digits of up to 8
// bits, the first ending at the highest bit where the keys differ (the bits
// above it are common to all keys), so the first histogram spreads the keys
// over all its bins.  The histograms are zero on entry and on return.  Needs
// k_eff <= the number of keys.
template <class ForKeys>
__device__ __forceinline__ KthKey radix_kth(RadixSmem& r, ForKeys&& for_keys, uint32_t kand, uint32_t kor,
                                            int k_eff) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t diff = kand ^ kor;
  if (diff == 0u) return KthKey{kand, 0xffffffffu, k_eff};  // every key equal: the k lowest page ids
  const int top = 31 - __clz(diff);
  uint32_t mask = top >= 31 ? 0u : ~((2u << top) - 1u);
  uint32_t prefix = kand & mask;
  int rem = k_eff;
  int buf = 0;
  for (int hi = top; hi >= 0; hi -= 8, buf ^= 1) {
    const int shift = max(hi - 7, 0);
    const uint32_t dmask = (2u << (hi - shift)) - 1u;  // hi - shift <= 7
    uint32_t* hb = r.hist[buf];
    for_keys([&](uint32_t k) {
      if ((k & mask) == prefix) atomicAdd(&hb[(k >> shift) & dmask], 1u);
    });
    __syncthreads();
    if (w == 0) {
      const uint32_t c0 = hb[4 * lane], c1 = hb[4 * lane + 1], c2 = hb[4 * lane + 2], c3 = hb[4 * lane + 3];
      // this histogram is used again two passes later: clear it now
      hb[4 * lane] = 0u; hb[4 * lane + 1] = 0u; hb[4 * lane + 2] = 0u; hb[4 * lane + 3] = 0u;
      // suffix sums over lanes (bins >= 4 lane, and >= 4 lane + 4) from
      // the inclusive prefix and the total
      const uint32_t c = c0 + c1 + c2 + c3;
      const uint32_t inc = (uint32_t)wave_incl_scan((int)c);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      const uint32_t Snext = total - inc;
      const uint32_t S = Snext + c;
      if (S >= (uint32_t)rem && Snext < (uint32_t)rem) {
        uint32_t above = Snext;
        const uint32_t cs[4] = {c0, c1, c2, c3};
        int digit = 4 * lane;
        uint32_t bucket = 0u;
#pragma unroll
        for (int bin = 3; bin >= 0; --bin) {
          if (above + cs[bin] >= (uint32_t)rem) { digit = 4 * lane + bin; bucket = cs[bin]; break; }
          above += cs[bin];
        }
        r.digit[buf] = (uint32_t)digit;
        r.above[buf] = above;
        r.bucket[buf] = bucket;
      }
    }
    __syncthreads();
    prefix |= r.digit[buf] << shift;
    mask |= dmask << shift;
    rem -= (int)r.above[buf];
    // the chosen bucket holds exactly the keys still wanted: all of it is
    // taken, and its lower digits need not be resolved
    if (r.bucket[buf] == (uint32_t)rem) break;
  }
  return KthKey{prefix, mask, rem};
}

// Writes the selected pages in page order.  for_keys(f) calls f(key, page)
// for this thread's keys in page order, and the threads' keys follow one
// another in page order.  One scan of (greater, equal) counts packed in the
// low and high 16 bits of an unsigned word: each prefix is at most
// n <= 65535, so neither field carries into the other, and the high field is
// read without sign extension.
template <class ForKeys>
__device__ __forceinline__ void topk_emit(RadixSmem& r, ForKeys&& for_keys, const KthKey& kk, int32_t* out) {
  uint32_t c_gt = 0u, c_eq = 0u;
  for_keys([&](uint32_t k, int) {
    const uint32_t km = k & kk.mask;
    c_gt += (km > kk.prefix);
    c_eq += (km == kk.prefix);
  });
  uint32_t tot;
  const uint32_t packed = block_exclusive_scan_u32(c_gt | (c_eq << 16), r.redu, &tot);
  const int gt_before = (int)(packed & 0xffffu), eq_before = (int)(packed >> 16);
  int pos = gt_before + min(eq_before, kk.rem);
  int rr = eq_before;
  for_keys([&](uint32_t k, int page) {
    const uint32_t km = k & kk.mask;
    bool take = km > kk.prefix;
    if (km == kk.prefix) { take = rr < kk.rem; ++rr; }
    if (take) out[pos++] = page;
  });
}

template <int E>  // keys per thread held in registers (0: read from memory)
__device__ __forceinline__ void topk_block(const SelectArgs& a, const float* s, const uint32_t (&kin)[E > 0 ? E : 1], int n_b,
                           int k_eff, int32_t* out, int unit) {
  constexpr int KE = E > 0 ? E : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  __shared__ RadixSmem rs;
  const int per = E > 0 ? E : (n_b + blockDim.x - 1) / blockDim.x;
  const int e0 = min(tid * per, n_b), e1 = min(e0 + per, n_b);
  const int cnt = e1 - e0;
  uint32_t keys[KE];
#pragma unroll
  for (int i = 0; i < KE; ++i) keys[i] = kin[i];
  // this thread's keys in page order: from registers (E > 0, loop fully
  // unrolled so the array stays in registers) or from memory (E == 0)
  auto for_keys = [&](auto&& f) {
    if (E > 0) {
#pragma unroll
      for (int i = 0; i < KE; ++i)
        if (i < cnt) f(keys[i], e0 + i);
    } else {
      for (int i = 0; i < cnt; ++i) f(f2key(s[e0 + i]), e0 + i);
    }
  };
  // bits shared by every key (AND and OR in one reduction) and cleared histograms
  uint32_t kand = 0xffffffffu, kor = 0u;
  for_keys([&](uint32_t k, int) { kand &= k; kor |= k; });
  kand = wave_reduce(kand, [](uint32_t u, uint32_t v) { return u & v; });
  kor = wave_reduce(kor, [](uint32_t u, uint32_t v) { return u | v; });
  radix_clear(rs);
  if (lane == 0) { rs.red[0][w] = kand; rs.red[1][w] = kor; }
  __syncthreads();
  kand = rs.red[0][0];
  kor = rs.red[1][0];
  for (int i = 1; i < nw; ++i) { kand &= rs.red[0][i]; kor |= rs.red[1][i]; }
  const KthKey kk = radix_kth(rs, [&](auto&& f) { for_keys([&](uint32_t k, int) { f(k); }); }, kand, kor, k_eff);
  topk_emit(rs, for_keys, kk, out);
  if (tid == 0) a.sel_count[unit] = k_eff;
}

template <int E>
__global__ __launch_bounds__(kSelThreads) void topk_kernel(SelectArgs a) {
  constexpr int KE = E > 0 ? E : 1;
  const int g = blockIdx.x, b = blockIdx.y;
  const int unit = b * a.n_kv_heads + g;
  const int tid = threadIdx.x;
  const int P = a.page_size;
  const float* s = a.scores + (size_t)unit * a.score_stride;
  // the score row's slots, requested with the length: the stride is a
  // multiple of 4 and the row 16-byte aligned, so an index clamped to the
  // row's last vector keeps every load inside the row
  uint32_t keys[KE];
  if (E > 0) {
#pragma unroll
    for (int i = 0; i < KE; i += 4) {
      const int at = min(tid * KE + i, a.score_stride - 4);
      const float4 v = *reinterpret_cast<const float4*>(s + at);
      keys[i] = f2key(v.x); keys[(i + 1) % KE] = f2key(v.y);
      keys[(i + 2) % KE] = f2key(v.z); keys[(i + 3) % KE] = f2key(v.w);
    }
  } else {
    keys[0] = 0u;  // unused: the keys are read from memory
  }
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);
  const int k_eff = min(a.top_k, n_b);
  int32_t* out = a.sel + (size_t)unit * a.cap;
  if (k_eff >= n_b) {
    for (int p = tid; p < n_b; p += blockDim.x) out[p] = p;
    if (tid == 0) a.sel_count[unit] = n_b;
    return;
  }
  if (n_b > 65535) {  // packed 16-bit counts would overflow: the host rejects such shapes
    set_status(a.status, EKV_DEV_OVERFLOW);
    if (tid == 0) a.sel_count[unit] = 0;
    return;
  }
  topk_block<E>(a, s, keys, n_b, k_eff, out, unit);
}

// ---------------------------------------------------------------------------
// Top-k over the scoring's candidate lists.  Every kCandListPages pages
// listed their kCandPerList largest scores (ties to the lower page) in page
// order, and the list's cut: the largest score it left out.  The k largest
// entries of the lists are the k largest pages of the row whenever every cut
// lies below all of them, since a page left out then scores below every
// selected page.  That fails only when kCandListPages pages hold more than
// kCandPerList of the k pages (clustered or equal scores); the block then
// selects over the whole score row as topk_kernel does.  Empty list slots
// hold key 0, below every score.
// ---------------------------------------------------------------------------
template <int EU, int E>  // list entries per thread; score keys per thread for the whole row
__global__ __launch_bounds__(kSelThreads) void topk_cand_kernel(SelectArgs a) {
  constexpr int KE = E > 0 ? E : 1;
  static_assert(EU % 2 == 0, "entries are loaded in pairs");
  __shared__ RadixSmem rs;
  const int g = blockIdx.x, b = blockIdx.y;
  const int unit = b * a.n_kv_heads + g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  const int nc = a.cand_lists * kCandPerList;  // even, and <= EU * blockDim.x
  // the lists and the cuts, requested with the length; an index clamped to
  // the last pair keeps every load inside the unit's lists
  const uint64_t* cl = a.cand + (size_t)unit * nc;
  uint32_t keys[EU];
  int pid[EU];
#pragma unroll
  for (int i = 0; i < EU; i += 2) {
    const int at = tid * EU + i;
    const uint4 v = *reinterpret_cast<const uint4*>(cl + min(at, nc - 2));
    const bool ok = at < nc;
    keys[i] = ok ? v.y : 0u;
    pid[i] = (int)v.x;
    keys[i + 1] = ok ? v.w : 0u;
    pid[i + 1] = (int)v.z;
  }
  uint32_t cmax = tid < a.cand_lists ? a.cand_cut[(size_t)unit * a.cand_lists + tid] : 0u;  // lists <= threads
  const int L = clamp_len(a.seq_lens[b], a.max_pages, a.page_size, a.status);
  const int n_b = pages_of(L, a.page_size);
  const int k_eff = min(a.top_k, n_b);
  int32_t* out = a.sel + (size_t)unit * a.cap;
  if (k_eff >= n_b) {
    for (int p = tid; p < n_b; p += blockDim.x) out[p] = p;
    if (tid == 0) a.sel_count[unit] = n_b;
    return;
  }
  if (n_b > 65535) {  // packed 16-bit counts would overflow: the host rejects such shapes
    set_status(a.status, EKV_DEV_OVERFLOW);
    if (tid == 0) a.sel_count[unit] = 0;
    return;
  }
  // listed pages in page order (empty slots skipped)
  auto for_cand = [&](auto&& f) {
#pragma unroll
    for (int i = 0; i < EU; ++i)
      if (keys[i] != 0u) f(keys[i], pid[i]);
  };
  uint32_t kand = 0xffffffffu, kor = 0u, nlist = 0u;
  for_cand([&](uint32_t k, int) { kand &= k; kor |= k; ++nlist; });
  kand = wave_reduce(kand, [](uint32_t u, uint32_t v) { return u & v; });
  kor = wave_reduce(kor, [](uint32_t u, uint32_t v) { return u | v; });
  nlist = wave_sum(nlist);
  cmax = wave_max(cmax);
  radix_clear(rs);
  if (lane == 0) { rs.red[0][w] = kand; rs.red[1][w] = kor; rs.red[2][w] = nlist; rs.red[3][w] = cmax; }
  __syncthreads();
  kand = rs.red[0][0]; kor = rs.red[1][0]; nlist = rs.red[2][0]; cmax = rs.red[3][0];
  for (int i = 1; i < nw; ++i) {
    kand &= rs.red[0][i]; kor |= rs.red[1][i]; nlist += rs.red[2][i]; cmax = max(cmax, rs.red[3][i]);
  }
  if ((int)nlist >= k_eff) {  // fewer listed pages than k: some block left out a page, use the row
    const KthKey kk = radix_kth(rs, [&](auto&& f) { for_cand([&](uint32_t k, int) { f(k); }); }, kand, kor, k_eff);
    if (cmax < kk.prefix) {  // every page left out scores below every selected page
      topk_emit(rs, for_cand, kk, out);
      if (tid == 0) a.sel_count[unit] = k_eff;
      return;
    }
  }
  const float* s = a.scores + (size_t)unit * a.score_stride;
  uint32_t rk[KE];
  if (E > 0) {
#pragma unroll
    for (int i = 0; i < KE; i += 4) {
      const int at = min(tid * KE + i, a.score_stride - 4);
      const float4 v = *reinterpret_cast<const float4*>(s + at);
      rk[i] = f2key(v.x); rk[(i + 1) % KE] = f2key(v.y);
      rk[(i + 2) % KE] = f2key(v.z); rk[(i + 3) % KE] = f2key(v.w);
    }
  } else {
    rk[0] = 0u;  // unused: the keys are read from memory
  }
  topk_block<E>(a, s, rk, n_b, k_eff, out, unit);
}

// ---------------------------------------------------------------------------
// Gaussian scoring.  A page record is mean[D] followed by M2[D] (float32).
// Eight lanes per record; lane s loads the 16-byte vectors s, s+8, s+16, ...
// so each load instruction covers 128 contiguous bytes of 8 records.  Mean
// vectors accumulate sum_i q_i mean_i, M2 vectors sum_i q_i^2 M2_i (fp32
// within the lane, float64 across the eight lanes).
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_gauss_kernel(SelectArgs a) {
  constexpr int VEC = 2 * D / 4;  // 16-byte vectors per record
  constexpr int NL = VEC / 8;     // loads per lane per page
  constexpr int NLH = NL / 2;     // of them in the mean half
  constexpr int NP = kGaussPagesPerBlock / 32;  // pages per lane group
  const int b = blockIdx.z, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane & 7;
  const int P = a.page_size, Hkv = a.n_kv_heads;
  // lane group (lane / 8) of wave w takes pages base + 32 n + 8 w + lane / 8
  const int pbase = blockIdx.x * kGaussPagesPerBlock + w * 8 + (lane >> 3);
  // the group's queries, staged once per block in LDS (every lane reads
  // its 16-float slice of each head from there, not through the L1)
  __shared__ float4 s_q[G * D / 4];
  float4 qload = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* qg = reinterpret_cast<const float4*>(a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * D);
  if (tid < G * D / 4) qload = qg[tid];
  int phys[NP];
  int n_b = 0;
#pragma unroll
  for (int n = 0; n < NP; ++n) phys[n] = page_phys_spec(a, b, pbase + 32 * n, &n_b);
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  float4 v[NP][NL];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    if (phys[n] >= 0) {
      const float4* rec = reinterpret_cast<const float4*>(a.k_moments + ((size_t)phys[n] * a.hkv_mem + (g >> a.kv_shift)) * 2 * D);
#pragma unroll
      for (int i = 0; i < NL; ++i) v[n][i] = rec[sub + 8 * i];
    }
  }
  if (tid < G * D / 4) s_q[tid] = qload;
  __syncthreads();
  const double a1s = ((double)a.alpha - 1.0) * (double)a.scale;
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    float fa[G], fb[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      fa[h] = 0.f;
      fb[h] = 0.f;
      if (phys[n] >= 0) {
#pragma unroll
        for (int i = 0; i < NLH; ++i) {
          const float4 q4 = s_q[h * (D / 4) + sub + 8 * i], mv = v[n][i], sv = v[n][i + NLH];
          fa[h] = fmaf(q4.x, mv.x, fa[h]); fa[h] = fmaf(q4.y, mv.y, fa[h]);
          fa[h] = fmaf(q4.z, mv.z, fa[h]); fa[h] = fmaf(q4.w, mv.w, fa[h]);
          fb[h] = fmaf(q4.x * q4.x, sv.x, fb[h]); fb[h] = fmaf(q4.y * q4.y, sv.y, fb[h]);
          fb[h] = fmaf(q4.z * q4.z, sv.z, fb[h]); fb[h] = fmaf(q4.w * q4.w, sv.w, fb[h]);
        }
      }
    }
    double A[G], Bv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      A[h] = fa[h];
      Bv[h] = fb[h];
      A[h] = group_reduce<8>(A[h], [](double u, double v) { return u + v; });
      Bv[h] = group_reduce<8>(Bv[h], [](double u, double v) { return u + v; });
    }
    const int p = pbase + 32 * n;
    if (sub < G && p < a.max_pages) {
      double As = 0.0, Bs = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (h == sub) { As = A[h]; Bs = Bv[h]; }
      float mu = 0.f, sd = 0.f, eh = -INFINITY, npf = 0.f;
      if (phys[n] >= 0) {
        const int np = min(P, L - p * P);
        const double mud = a1s * As;
        const double var = a1s * a1s * Bs / (double)np;
        const double sdd = sqrt(fmax(var, 0.0));
        mu = (float)mud;
        sd = (float)sdd;
        eh = (float)(mud + sdd * sqrt(2.0 * log((double)np)));
        npf = (float)np;
      }
      const size_t at = ((size_t)b * a.n_q_heads + (size_t)g * G + sub) * a.max_pages + p;
      a.musd[at] = make_float2(mu, sd);
      a.ehat[at] = eh;
      if (a.stats_out) a.stats_out[at] = make_float4(mu, sd, eh, npf);
    }
  }
}

// ---------------------------------------------------------------------------
// tau_hat solves F(t) = sum_p n_p E_p(t) = 1 for one (sequence, query head),
// where E_p(t) is the expected value of (Y - t)_+^e for the page's Gaussian
// score Y ~ N(mu, sd^2) and e = 1/(alpha-1).  With a = mu - t, u = a / sd:
//   e = 1 (alpha=2):   E = a Phi(u) + sd phi(u),               E' = -Phi(u)
//   e = 2 (alpha=1.5): E = (a^2 + sd^2) Phi(u) + a sd phi(u),  E' = -2 (a Phi + sd phi)
// and E = (a)_+^e when sd = 0.  F is continuous and strictly decreasing
// where positive, so the root is unique.
//
// Other alpha in [1.1, 2] use the quadrature of gauss_mass_general below.
//
// Start: E_p(t) >= (mu_p - t)_+^e (Jensen, e >= 1), so every page alone
// bounds the root from below by mu_p - n_p^{-(alpha-1)}; the largest of
// these is t0.  t only matters above t0, where a page with u < -7
// contributes below 2e-13 n_p sd^e: such pages are dropped once, at t0.
// The iteration is Halley's method on log F (alpha 1.5 and 2, where F'' is
// at hand) or Newton's (other alpha), kept inside a bracket [lo, hi] with
// F(lo) >= 1 > F(hi) and replaced by bisection whenever it would leave it.
// Per-page terms are evaluated in fp32 and summed in fp64; the iteration
// stops once a step moves t by at most 2e-7 max(1, |t|).  Near the root
// Halley's method converges cubically (each step about the cube of the one
// before, in units of the root's scale): a Halley step of at most
// 1e-4 max(1, |t|) that is also at most 1/100 of the step before it (the
// iteration is in that regime, not crossing the kink of a page with zero
// variance) leaves an error far below the tolerance, so it is taken as the
// last step, without one more evaluation of F to confirm it.
//
// Each head marks the pages whose estimated maximum beats its tau_hat -
// delta in a bitmap; the last block of a (sequence, KV head) to finish
// (arrival counter) keeps the pages some head of the group marked, in
// ascending order, at least one page (the best margin, lowest id on ties).
// ---------------------------------------------------------------------------
// The standard normal density and distribution function at u from one
// exponential.  erfc is the Chebyshev fit of Press, Teukolsky, Vetterling
// and Flannery, Numerical Recipes (2nd ed.) sec. 6.2: erfc(z) = t exp(-z^2 +
// P(t)), t = 1 / (1 + z/2), fractional error below 1.2e-7.  Here z^2 = u^2/2
// is carried as an exact two-float sum, and exp(-z^2) comes from a
// Cody-Waite reduction onto the hardware exp2 (about 1e-7 relative), which
// the density exp(-u^2/2) / sqrt(2 pi) shares.  In fp32 the density and
// Phi(u <= 0) come out within about 5e-7 relative, Phi(u > 0) within 2e-7
// absolute, against 50 + 20 instructions for erfcf and expf.
__device__ __forceinline__ void normal_pdf_cdf(float u, float& pdf, float& cdf) {
  const float kInvSqrt2 = 0.70710678118654752440f, kInvSqrt2Pi = 0.39894228040143267794f;
  const float kLog2e = 1.4426950408889634f, kLog2eHi = 1.44269502162933349609375f, kLog2eLo = 1.925963033500011e-08f;
  const float z = fabsf(u) * kInvSqrt2;
  const float t = __builtin_amdgcn_rcpf(1.f + 0.5f * z);
  float p = 0.17087277f;
  p = fmaf(t, p, -0.82215223f);
  p = fmaf(t, p, 1.48851587f);
  p = fmaf(t, p, -1.13520398f);
  p = fmaf(t, p, 0.27886807f);
  p = fmaf(t, p, -0.18628806f);
  p = fmaf(t, p, 0.09678418f);
  p = fmaf(t, p, 0.37409196f);
  p = fmaf(t, p, 1.00002368f);
  p = fmaf(t, p, -1.26551223f);
  const float u2h = u * u, u2l = fmaf(u, u, -u2h);  // u^2 = u2h + u2l exactly
  const float z2h = 0.5f * u2h, z2l = 0.5f * u2l;
  const float n = __builtin_rintf(-z2h * kLog2eHi);
  const float fr = fmaf(-z2h, kLog2eHi, -n) - z2h * kLog2eLo;
  const float e1 = __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(fr), (int)n);  // exp(-z2h)
  const float erfc = t * e1 * __builtin_amdgcn_exp2f((p - z2l) * kLog2e);
  pdf = e1 * (1.f - z2l) * kInvSqrt2Pi;
  cdf = u <= 0.f ? 0.5f * erfc : 1.f - 0.5f * erfc;
}

__device__ __forceinline__ void gauss_mass(float mu, float sd, float tf, bool quad, float& e, float& de,
                                           float& dde) {
  const float am = mu - tf;
  if (sd <= 0.f) {
    const float pos = fmaxf(am, 0.f);
    e = quad ? pos * pos : pos;
    de = quad ? -2.f * pos : (am > 0.f ? -1.f : 0.f);
    dde = quad && am > 0.f ? 2.f : 0.f;
    return;
  }
  const float rsd = __builtin_amdgcn_rcpf(sd);
  const float u = am * rsd;
  if (u < -7.f) {
    e = de = dde = 0.f;
    return;
  }
  float phi, Phi;
  normal_pdf_cdf(u, phi, Phi);
  const float e1 = am * Phi + sd * phi;
  if (quad) {
    e = (am * am + sd * sd) * Phi + am * sd * phi;
    de = -2.f * e1;
    dde = 2.f * Phi;
  } else {
    e = e1;
    de = -Phi;
    dde = phi * rsd;
  }
}

// Other alpha in [1.1, 2] (e = 1/(alpha-1) in [1, 10]): with z = (Y - t)/sd,
// E = sd^e M_e(u) and E' = -e sd^(e-1) M_(e-1)(u), where M_b(u) is the
// integral over z > 0 of z^b phi(z - u).  The log integrand f(z) = e ln z -
// (z - u)^2 / 2 peaks at zs = (u + sqrt(u^2 + 4e)) / 2.  Two 16-point
// Gauss-Legendre rules cover it, the right one up to where f has dropped by
// 30 (three Newton steps on the concave f), the left one down to zs - sqrt(60)
// widths, or from 0 with z = s^2 when that end would pass 0 (the integrand
// then behaves like s^(2e+1), smooth enough for the rule).  Node weights
// are taken relative to the peak, exp(f(z) - f(zs)), from differences that
// keep their precision in fp32; the peak factor is applied in fp64.  The
// relative error is about 1e-7 over u in [-7, 40].  Beyond u = 40 the
// truncation is negligible and E = a^e (1 + C(e,2)/u^2 + 3 C(e,4)/u^4 +
// 15 C(e,6)/u^6), the moments of N(u, 1) to order u^-6.
__constant__ float kGL16[8][2] = {
    {0.095012510f, 0.189450610f}, {0.281603551f, 0.182603415f}, {0.458016778f, 0.169156519f},
    {0.617876244f, 0.149595989f}, {0.755404408f, 0.124628971f}, {0.865631202f, 0.095158512f},
    {0.944575023f, 0.062253524f}, {0.989400935f, 0.027152459f}};

__device__ __forceinline__ float normal_power_series(float b, float u) {
  const float v = 1.f / (u * u);
  const float t2 = 0.5f * b * (b - 1.f);               // C(b,2)
  const float t4 = 0.25f * t2 * (b - 2.f) * (b - 3.f);  // 3 C(b,4)
  const float t6 = t4 * (b - 4.f) * (b - 5.f) / 6.f;    // 15 C(b,6)
  return 1.f + v * (t2 + v * (t4 + v * t6));
}

__device__ void gauss_mass_general(float mu, float sd, float tf, float beta, float& e, float& de) {
  const float am = mu - tf;
  if (sd <= 0.f) {
    if (am <= 0.f) { e = de = 0.f; return; }
    e = exp2f(beta * log2f(am));
    de = -beta * e / am;
    return;
  }
  const float u = am / sd;
  if (u < -7.f) {
    e = de = 0.f;
    return;
  }
  if (u > 40.f) {
    const float la = log2f(am);
    e = exp2f(beta * la) * normal_power_series(beta, u);
    de = -beta * exp2f((beta - 1.f) * la) * normal_power_series(beta - 1.f, u);
    return;
  }
  const float zs = 0.5f * (u + sqrtf(u * u + 4.f * beta));
  const float rzs = 1.f / zs;
  const float kLog2e = 1.44269504089f, kDrop = 30.f, kSpan = 7.745966692f;  // sqrt(2 kDrop)
  // (f(z) - f(zs)) / ln 2 from differences; the node weights use the
  // hardware exp2 / log2 / reciprocal (about 1 ulp), which the 1e-7 budget
  // of the rule absorbs
  const float hb = 0.5f * kLog2e;
  auto rel2 = [&](float z) {
    return beta * __builtin_amdgcn_logf(z * rzs) - hb * (z - zs) * (z + zs - 2.f * u);
  };
  float zr = zs + kSpan;
#pragma unroll
  for (int i = 0; i < 3; ++i) zr -= (rel2(zr) * 0.69314718056f + kDrop) / (beta / zr - (zr - u));
  const float zl = zs - kSpan * rsqrtf(beta * rzs * rzs + 1.f);
  float m = 0.f, m1 = 0.f;  // relative to the peak: M_e and M_(e-1)
  {
    const float h = 0.5f * (zr - zs), c = zs + h;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int sg = -1; sg <= 1; sg += 2) {
        const float z = c + (float)sg * h * kGL16[i][0];
        const float v = kGL16[i][1] * __builtin_amdgcn_exp2f(rel2(z));
        m += v;
        m1 += v * __builtin_amdgcn_rcpf(z);
      }
    }
    m *= h;
    m1 *= h;
  }
  if (zl > 0.f) {
    const float h = 0.5f * (zs - zl), c = zl + h;
    float ml = 0.f, ml1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int sg = -1; sg <= 1; sg += 2) {
        const float z = c + (float)sg * h * kGL16[i][0];
        const float v = kGL16[i][1] * __builtin_amdgcn_exp2f(rel2(z));
        ml += v;
        ml1 += v * __builtin_amdgcn_rcpf(z);
      }
    }
    m += h * ml;
    m1 += h * ml1;
  } else {  // z = s^2 over s in [0, sqrt(zs)]: dz = 2 s ds
    const float h = 0.5f * sqrtf(zs);
    float ml = 0.f, ml1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int sg = -1; sg <= 1; sg += 2) {
        const float sv = h + (float)sg * h * kGL16[i][0];
        const float z = sv * sv;
        const float v = kGL16[i][1] * 2.f * sv * __builtin_amdgcn_exp2f(rel2(z));
        ml += v;
        ml1 += v * __builtin_amdgcn_rcpf(z);
      }
    }
    m += h * ml;
    m1 += h * ml1;
  }
  // peak factor exp(f(zs)) sd^e / sqrt(2 pi)
  const double zd = zs, ud = u;
  const double sc = exp((double)beta * log(zd * (double)sd) - 0.5 * (zd - ud) * (zd - ud)) * 0.3989422804014327;
  e = (float)(sc * (double)m);
  de = (float)(-(double)beta * sc / (double)sd * (double)m1);
}

// Other alpha, per page and Newton step: log M_e and log M_(e-1) are
// tabulated once per block on the grid u = -7 + i/32 (1536 nodes up to
// u = 40.97; the step is a power of two, so the nodes are exact in fp32)
// with the quadrature above; a page's expectation is then a four-point
// Lagrange interpolation of the logs (log M is smooth in u: error near
// 1e-8) and two exponentials, split into 2^k times a hardware exp2 of the
// fraction.  Zero variance and u > 40 keep the closed forms above.
constexpr int kMomNodes = 1536;
constexpr float kMomU0 = -7.f;
constexpr double kMomInvH = 32.0;

template <bool GEN> struct MomTable {
  double lm[kMomNodes], lm1[kMomNodes];
};
template <> struct MomTable<false> {};  // the closed-form instance needs no table

__device__ void mom_table_build(MomTable<true>& T, float beta) {
  for (int i = threadIdx.x; i < kMomNodes; i += blockDim.x) {
    float e, de;
    gauss_mass_general(kMomU0 + (float)i * (1.f / 32.f), 1.f, 0.f, beta, e, de);  // M_e(u), -e M_(e-1)(u)
    T.lm[i] = log((double)e);
    T.lm1[i] = log(-(double)de / (double)beta);
  }
}

// e^y with fp32 relative accuracy: 2^k times the hardware 2^f, f in [0, 1)
__device__ __forceinline__ float exp_split(double y) {
  const double x = y * 1.4426950408889634;
  const double k = floor(x);
  return __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f((float)(x - k)), (int)k);
}

__device__ void gauss_mass_table(float mu, float sd, float tf, float beta, const MomTable<true>& T, float& e,
                                 float& de) {
  const float am = mu - tf;
  if (sd <= 0.f || am > 40.f * sd) {  // a single point, or beyond the table: closed forms
    gauss_mass_general(mu, sd, tf, beta, e, de);
    return;
  }
  const float u = am / sd;
  if (u < -7.f) {
    e = de = 0.f;
    return;
  }
  const double x = ((double)u - (double)kMomU0) * kMomInvH;
  const int i = max(0, min((int)x - 1, kMomNodes - 4));
  const double s = x - (double)i;  // position among the nodes i .. i + 3
  const double w0 = -(s - 1.0) * (s - 2.0) * (s - 3.0) * (1.0 / 6.0), w1 = s * (s - 2.0) * (s - 3.0) * 0.5,
               w2 = -s * (s - 1.0) * (s - 3.0) * 0.5, w3 = s * (s - 1.0) * (s - 2.0) * (1.0 / 6.0);
  const double lm = ((w0 * T.lm[i] + w1 * T.lm[i + 1]) + w2 * T.lm[i + 2]) + w3 * T.lm[i + 3];
  const double lm1 = ((w0 * T.lm1[i] + w1 * T.lm1[i + 1]) + w2 * T.lm1[i + 2]) + w3 * T.lm1[i + 3];
  const double ls = log((double)sd);
  e = exp_split((double)beta * ls + lm);
  de = -beta * exp_split(((double)beta - 1.0) * ls + lm1);
}

// live-list entries carry the partial last page as sd -> -sd - 1.
// mode: 0 alpha = 2, 1 alpha = 1.5, 2 other alpha (beta = 1/(alpha-1);
// no second derivative, ddF is left unchanged).
template <bool GEN>
__device__ __forceinline__ void live_term(float2 v, float P, float last_n, float tf, int mode, float beta,
                                          const MomTable<GEN>& T, double& F, float& dF, float& ddF) {
  float n = P, sd = v.y;
  if (sd < 0.f) { sd = -sd - 1.f; n = last_n; }
  float e, de, dde = 0.f;
  if constexpr (GEN) gauss_mass_table(v.x, sd, tf, beta, T, e, de);
  else gauss_mass(v.x, sd, tf, mode == 1, e, de, dde);
  F += (double)n * (double)e;
  dF = fmaf(n, de, dF);
  ddF = fmaf(n, dde, ddF);
}

// The single page of the largest margin max_h (e_hat - tau_hat) (lowest id
// on ties), for a group that keeps no page.
template <int G>
__device__ void gauss_floor_unit(const SelectArgs& a, int b, int g, int n_b, int32_t* out, int unit) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  __shared__ double redd[16];
  __shared__ int redp[16];
  double tau[G];
  const float* eh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
    tau[h] = __hip_atomic_load(a.tau_hat + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // written by the group's other blocks
    eh[h] = a.ehat + bh * a.max_pages;
  }
  double best = -INFINITY;
  int best_p = 0x7fffffff;
  for (int p = tid; p < n_b; p += blockDim.x) {
    double mg = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) mg = fmax(mg, (double)eh[h][p] - tau[h]);
    if (mg > best) { best = mg; best_p = p; }
  }
  const double bm = block_max(best, redd);
  int cand = (best == bm) ? best_p : 0x7fffffff;
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

// GEN: alpha other than 1.5 and 2 (a separate instance, so that the
// quadrature's registers do not weigh on the closed-form one)
// The closed-form instance with the 8192-page list is held to 64 registers
// so that two blocks share a compute unit (its LDS, 65 KB, allows two).
template <int G, bool GEN, int LIVE>
__global__ __launch_bounds__(kTauHatThreads)
__attribute__((amdgpu_waves_per_eu(!GEN && LIVE <= kTauHatLive ? 8 : 4))) void tau_hat_kernel(SelectArgs a) {
  // pages per thread held in registers: as many as the live list holds
  // (n_b <= LIVE), which keeps the 8192-page instance within 64 registers
  constexpr int PPT = LIVE / kTauHatThreads;
  constexpr int NW = kTauHatThreads / kWave;
  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / G, unit = b * a.n_kv_heads + g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = a.page_size;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, P, a.status);
  const int n_b = pages_of(L, P);
  const size_t bh = (size_t)b * a.n_q_heads + h;
  const float2* st = a.musd + bh * a.max_pages;
  __shared__ float2 live[LIVE];
  __shared__ MomTable<GEN> mom;
  __shared__ double part[2][NW][3];
  __shared__ double redd[16];
  __shared__ int redi[17];
  __shared__ int s_last;
  double t = 0.0;
  const bool in_regs = n_b <= PPT * kTauHatThreads;
  const float* eh_row = a.ehat + bh * a.max_pages;
  float ehv[PPT];  // this head's estimated maxima (pages tid, tid + 1024, ...), for its keep decisions
  if (n_b > 0) {
    const int mode = GEN ? 2 : (a.alpha == 1.5f ? 1 : 0);
    const float beta = 1.f / (a.alpha - 1.f);
    const float Pf = (float)P;
    const float last_n = (float)(L - (n_b - 1) * P);  // tokens of the last page
    // (other alpha: the moment tables first, while few registers are live;
    // the barriers of block_max below publish them)
    if constexpr (GEN) mom_table_build(mom, beta);
    // thread t owns pages t, t + 1024, ...: one round of coalesced loads
    float2 ms[PPT];
    double lb = -INFINITY;
    // n^-(alpha-1) for a full page and for the last one, once per thread
    auto count_term = [&](double n) {
      return mode == 0 ? 1.0 / n : (mode == 1 ? 1.0 / sqrt(n) : pow(n, -(double)(a.alpha - 1.f)));
    };
    const double r_full = count_term((double)P), r_last = count_term((double)last_n);
    auto bound = [&](float2 v, int p) { return (double)v.x - (p == n_b - 1 ? r_last : r_full); };
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int p = i * kTauHatThreads + tid;
        ms[i] = p < n_b ? st[p] : make_float2(-INFINITY, 0.f);
        if (p < n_b) lb = fmax(lb, bound(ms[i], p));
      }
    } else {
      for (int p = tid; p < n_b; p += kTauHatThreads) lb = fmax(lb, bound(st[p], p));
    }
    const double t0 = block_max(lb, redd);
    const float t0f = (float)t0;
    auto alive = [&](float2 v) { return v.y > 0.f ? (v.x - t0f) > -7.f * v.y : v.x > t0f; };
    // live pages at t0, compacted (thread-major order, fixed for given inputs)
    int n_live = 0;
    bool use_live = false;
    if (in_regs) {
      int c = 0;
#pragma unroll
      for (int i = 0; i < PPT; ++i) c += (i * kTauHatThreads + tid < n_b) && alive(ms[i]);
      int pos = block_exclusive_scan(c, redi, &n_live);
      use_live = n_live <= LIVE;
      if (use_live) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
          const int p = i * kTauHatThreads + tid;
          if (p < n_b && alive(ms[i])) {
            float2 v = ms[i];
            if (p == n_b - 1 && last_n != Pf) v.y = -v.y - 1.f;
            live[pos++] = v;
          }
        }
      }
      // the estimated maxima are requested now, in the registers of the
      // page records (no longer needed); they arrive while the iteration runs
#pragma unroll
      for (int i = 0; i < PPT; ++i) ehv[i] = load_or(eh_row, i * kTauHatThreads + tid, n_b, -INFINITY);
      __syncthreads();
    }
    double lo = -INFINITY, hi = INFINITY;
    double prev_step = 0.0;  // the last step's size (wave 0)
    t = t0;
    for (int it = 0; it < 200; ++it) {
      const float tf = (float)t;
      // F in fp64 (it decides the root); its derivatives only shape the
      // step, so their sums within a wave are fp32
      double F = 0.0;
      float dFf = 0.f, ddFf = 0.f;
      if (use_live) {
        for (int i = tid; i < n_live; i += kTauHatThreads)
          live_term<GEN>(live[i], Pf, last_n, tf, mode, beta, mom, F, dFf, ddFf);
      } else {
        for (int p = tid; p < n_b; p += kTauHatThreads) {
          float2 v = st[p];
          if (p == n_b - 1 && last_n != Pf) v.y = -v.y - 1.f;
          live_term<GEN>(v, Pf, last_n, tf, mode, beta, mom, F, dFf, ddFf);
        }
      }
      // wave partials -> wave 0 computes the step -> every wave reads it
      F = wave_sum(F);
      double dF = wave_sum(dFf), ddF = wave_sum(ddFf);
      if (lane == 0) {
        part[0][w][0] = F;
        part[0][w][1] = dF;
        part[0][w][2] = ddF;
      }
      __syncthreads();
      if (w == 0) {
        // lane i < NW takes wave i's partials; a fixed-order wave sum
        double pf = lane < NW ? part[0][lane][0] : 0.0;
        double pd = lane < NW ? part[0][lane][1] : 0.0;
        double pdd = lane < NW ? part[0][lane][2] : 0.0;
        static_assert(NW == 16, "one partial per lane of the first row");
        auto add = [](double u, double v) { return u + v; };
        pf = group_reduce<16>(pf, add);
        pd = group_reduce<16>(pd, add);
        pdd = group_reduce<16>(pdd, add);
        F = pf; dF = pd; ddF = pdd;
        int stop = 0;
        if (F == 1.0) {
          stop = 1;
        } else {
          if (F > 1.0) lo = t; else hi = t;
          const double tol = 2e-7 * fmax(1.0, fabs(t));
          // Halley's method on g = log F (cubic near the root), else Newton's
          // on g, else bisection of the bracket.  Near the root g comes from
          // its series in F - 1; farther away a float logarithm suffices.
          double cand = t;
          bool ok = false, halley = false;
          if (F > 0.0 && dF < 0.0) {
            const double x = F - 1.0;
            const double gl = fabs(x) < 1e-3 ? x * (1.0 - x * (0.5 - x * (1.0 / 3.0 - 0.25 * x)))
                                             : (double)logf((float)F);
            const double iF = 1.0 / F;
            const double g1 = dF * iF, g2 = ddF * iF - g1 * g1;
            const double cn = t - gl / g1;
            const float r = mode == 2 ? 0.f : (float)(gl * g2 / (g1 * g1));  // 0: Newton
            const float den = 1.f - 0.5f * r;
            const double ch = den > 0.f ? t + (cn - t) * (double)(1.f / den) : cn;  // Halley = Newton / (1 - r/2)
            if (den > 0.f && ch > lo && ch < hi) { cand = ch; ok = true; halley = mode != 2; }
            else if (cn > lo && cn < hi) { cand = cn; ok = true; }
            else if (fabs(cn - t) <= tol) { cand = cn; ok = true; }
          }
          const double step = fabs(cand - t);
          if (ok && (step <= tol || (halley && step <= 1e-4 * fmax(1.0, fabs(t)) && step <= 0.01 * prev_step))) {
            stop = 1;
          } else if (!ok) {
            if (lo > -INFINITY && hi < INFINITY) cand = 0.5 * (lo + hi);
            else if (hi < INFINITY) cand = hi - fmax(1.0, fabs(hi));
            else cand = lo + fmax(1.0, fabs(lo));
          }
          if (!stop && hi - lo <= tol) stop = 1;
          prev_step = ok ? step : 0.0;
          t = cand;
        }
        if (lane == 0) {
          part[1][0][0] = t;
          part[1][0][1] = stop ? 1.0 : 0.0;
        }
      }
      __syncthreads();
      t = part[1][0][0];
      const bool stop = part[1][0][1] != 0.0;
      if (stop) break;
    }
  }
  // this head's keep decisions, e_hat - tau_hat > -delta, one word per
  // 64-page chunk (a ballot of one wave; pages past n_b are never kept),
  // read by the group's last block
  if (n_b > 0) {
    uint64_t* kb = a.keep_bits + bh * a.keep_words;
    const double ndelta = -(double)a.delta;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int c = i * NW + w;  // pages 64 c .. 64 c + 63
        const uint64_t m = __ballot((double)ehv[i] - t > ndelta);
        if (lane == 0 && 64 * c < n_b) st_dev(kb + c, m);
      }
    } else {
      for (int c = w; 64 * c < n_b; c += NW) {
        const uint64_t m = __ballot((double)load_or(eh_row, 64 * c + lane, n_b, -INFINITY) - t > ndelta);
        if (lane == 0) st_dev(kb + c, m);
      }
    }
  }
  if (tid == 0) {
    st_dev(a.tau_hat + bh, t);  // read by the group's last block
    if (a.tau_hat_out) a.tau_hat_out[bh] = (float)t;
  }
  wait_mem();  // every wave's device-scope stores have completed
  __syncthreads();
  if (tid == 0) {
    // release: tau_hat above is visible at agent scope before the arrival is
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    s_last = atomicAdd(a.done + unit, 1u) == (uint32_t)(G - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // The last block reads the other heads' keep words (and, for the floor,
  // their tau_hat) with agent-scope atomic loads, which return the coherent
  // value: each writer's stores completed before its release and arrival,
  // and this block saw every arrival.  (An acquire fence here would
  // invalidate this compute unit's caches and slow the loads below by
  // microseconds.)
  if (tid == 0) st_dev(a.done + unit, 0u);  // ready for the next call

  // ---- the group's last block: the pages some head keeps, ascending ids.
  // Pages go in chunks of 64 (chunk c: pages 64 c .. 64 c + 63, one keep
  // word per head), thread c taking chunk c; one scan over the chunks'
  // counts places every kept page.  Sequences of more than 64 Ki pages go in
  // passes of 1024 chunks. ----
  int32_t* out = a.sel + (size_t)unit * a.cap;
  if (n_b == 0) {
    if (tid == 0) a.sel_count[unit] = 0;
    return;
  }
  const uint64_t* kb0 = a.keep_bits + ((size_t)b * a.n_q_heads + (size_t)g * G) * a.keep_words;
  uint64_t* s_mask = reinterpret_cast<uint64_t*>(live);  // the live list is no longer needed
  int* s_off = reinterpret_cast<int*>(s_mask + kTauHatThreads);
  static_assert(LIVE * sizeof(float2) >= kTauHatThreads * (sizeof(uint64_t) + sizeof(int)), "union scratch");
  __syncthreads();  // every wave is done with the live list
  int run = 0;
  for (int base = 0; base < n_b; base += 64 * kTauHatThreads) {  // block-uniform
    const int nch = min(kTauHatThreads, (n_b - base + 63) / 64);
    // a page is kept when some head of the group keeps it: the OR of the
    // heads' words, read with agent-scope atomic loads
    if (tid < nch) {
      uint64_t m = 0;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        m |= __hip_atomic_load(kb0 + (size_t)hh * a.keep_words + base / 64 + tid, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      s_mask[tid] = m;
    }
    __syncthreads();
    const int cnt = tid < nch ? __popcll(s_mask[tid]) : 0;
    int tot;
    const int off = block_exclusive_scan(cnt, redi, &tot);
    if (tid < nch) s_off[tid] = run + off;
    __syncthreads();
    for (int c = w; c < nch; c += NW) {
      const uint64_t m = s_mask[c];
      if ((m >> lane) & 1ull) out[s_off[c] + __popcll(m & ((1ull << lane) - 1ull))] = base + 64 * c + lane;
    }
    run += tot;
    __syncthreads();  // s_mask / s_off are rewritten by the next pass
  }
  if (run > 0) {
    if (tid == 0) a.sel_count[unit] = run;
    return;
  }
  gauss_floor_unit<G>(a, b, g, n_b, out, unit);
}

// ---------------------------------------------------------------------------
// At least min_pages pages per unit (min_pages > 1; the threshold kernel's
// last block already guarantees one).  When the keep rule kept fewer than
// m = min(min_pages, n_b) pages, the unit's list becomes the m pages of
// largest margin max_h (e_hat_h - tau_hat_h), lower page id first on equal
// margins, in ascending order: a superset of the kept pages, whose margins
// are above -delta while every other page's is not.  One 1024-thread block
// per unit; the margins (rounded to float) go through the top-k block.
// ---------------------------------------------------------------------------
template <int G, int E>
__global__ __launch_bounds__(kSelThreads) void gauss_floor_kernel(SelectArgs a) {
  constexpr int KE = E > 0 ? E : 1;
  const int g = blockIdx.x, b = blockIdx.y;
  const int unit = b * a.n_kv_heads + g;
  const int tid = threadIdx.x;
  const int L = clamp_len(a.seq_lens[b], a.max_pages, a.page_size, a.status);
  const int n_b = pages_of(L, a.page_size);
  const int m = min(a.min_pages, n_b);
  if (a.sel_count[unit] >= m) return;  // block-uniform
  int32_t* out = a.sel + (size_t)unit * a.cap;
  if (m == n_b) {  // every page
    for (int p = tid; p < n_b; p += blockDim.x) out[p] = p;
    if (tid == 0) a.sel_count[unit] = n_b;
    return;
  }
  double tau[G];
  const float* eh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
    tau[h] = a.tau_hat[bh];
    eh[h] = a.ehat + bh * a.max_pages;
  }
  auto margin = [&](int p) {
    double mg = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) mg = fmax(mg, (double)eh[h][p] - tau[h]);
    return (float)mg;
  };
  uint32_t keys[KE];
  float* s = a.scores + (size_t)unit * a.score_stride;
  if (E > 0) {
#pragma unroll
    for (int i = 0; i < KE; ++i) {
      const int p = tid * KE + i;
      keys[i] = p < n_b ? f2key(margin(p)) : 0u;
    }
  } else {
    keys[0] = 0u;  // unused: the keys are read back from the score row
    for (int p = tid; p < n_b; p += blockDim.x) s[p] = margin(p);
    __syncthreads();  // the row is read by other threads of the block next
  }
  topk_block<E>(a, s, keys, n_b, m, out, unit);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// bf16 records are scored four 16-page groups per wave (256 pages per block)
// when that still leaves >= 512 blocks
static bool bbox_fat(const SelectArgs& a) {
  return a.kv_dtype == EKV_BF16 && (long long)a.max_pages * a.n_kv_heads * a.batch >= 512LL * 256;
}

// Candidate lists per unit that the scoring writes for the top-k, or 0:
// lists need the 256-page scoring blocks and a shared selection, fit the
// top-k block's registers, and are used when they hold at least four times
// the k pages (at most two of the k pages per list on average, so that no
// list is likely to hold fewer than its share).
static int topk_cand_lists(const SelectArgs& a) {
  if (!a.cand || !a.cand_cut || a.per_head_scores || !bbox_fat(a)) return 0;
  const int nl = cand_lists(a.max_pages);
  const long long nc = (long long)nl * kCandPerList;
  if (nl > kSelThreads || nc > 8LL * kSelThreads || 4LL * a.top_k > nc) return 0;
  return nl;
}

template <int DT, int D>
static hipError_t bbox_dispatch(const SelectArgs& a0, hipStream_t s) {
  const dim3 blk(kScoreThreads);
  SelectArgs a = a0;
  a.cand_lists = topk_cand_lists(a0);
  if (DT == EKV_BF16) {
    const bool fat = bbox_fat(a);
    const int ppb = fat ? 256 : 64;
    const dim3 grid((a.max_pages + ppb - 1) / ppb, a.n_kv_heads, a.batch);
#define EKV_BBOX(GG)                                                                                 \
  if (fat) hipLaunchKernelGGL((score_bbox_mfma_kernel<D, GG, 4>), grid, blk, 0, s, a);              \
  else hipLaunchKernelGGL((score_bbox_mfma_kernel<D, GG, 1>), grid, blk, 0, s, a);
    switch (a.group) {
      case 1: EKV_BBOX(1); break;
      case 2: EKV_BBOX(2); break;
      case 4: EKV_BBOX(4); break;
      default: EKV_BBOX(8); break;
    }
#undef EKV_BBOX
    return hipGetLastError();
  }
  const dim3 grid((a.max_pages + kBboxPagesPerBlock - 1) / kBboxPagesPerBlock, a.n_kv_heads, a.batch);
  switch (a.group) {
    case 1: hipLaunchKernelGGL((score_bbox_valu_kernel<DT, D, 1>), grid, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_bbox_valu_kernel<DT, D, 2>), grid, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_bbox_valu_kernel<DT, D, 4>), grid, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_bbox_valu_kernel<DT, D, 8>), grid, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_bbox(const SelectArgs& a, hipStream_t s) {
  if (a.kv_dtype == EKV_BF16)
    return a.head_dim == 128 ? bbox_dispatch<EKV_BF16, 128>(a, s) : bbox_dispatch<EKV_BF16, 64>(a, s);
  return a.head_dim == 128 ? bbox_dispatch<EKV_F32, 128>(a, s) : bbox_dispatch<EKV_F32, 64>(a, s);
}

template <int EU>
static void topk_cand_dispatch(const SelectArgs& a, dim3 grid, int per, hipStream_t s) {
  if (per <= 16) hipLaunchKernelGGL((topk_cand_kernel<EU, 16>), grid, dim3(kSelThreads), 0, s, a);
  else hipLaunchKernelGGL((topk_cand_kernel<EU, 0>), grid, dim3(kSelThreads), 0, s, a);
}

hipError_t launch_topk(const SelectArgs& a0, hipStream_t s) {
  SelectArgs a = a0;
  a.cand_lists = topk_cand_lists(a0);  // the scoring launch decided the same
  const dim3 grid(a.n_kv_heads, a.batch);
  const int per = (a.max_pages + kSelThreads - 1) / kSelThreads;
  if (a.cand_lists > 0) {
    const int nc = a.cand_lists * kCandPerList;
    if (nc <= 2 * kSelThreads) topk_cand_dispatch<2>(a, grid, per, s);
    else if (nc <= 4 * kSelThreads) topk_cand_dispatch<4>(a, grid, per, s);
    else topk_cand_dispatch<8>(a, grid, per, s);
    return hipGetLastError();
  }
  if (per <= 4) hipLaunchKernelGGL((topk_kernel<4>), grid, dim3(kSelThreads), 0, s, a);
  else if (per <= 16) hipLaunchKernelGGL((topk_kernel<16>), grid, dim3(kSelThreads), 0, s, a);
  else hipLaunchKernelGGL((topk_kernel<0>), grid, dim3(kSelThreads), 0, s, a);
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

template <bool GEN, int LIVE>
static hipError_t tau_hat_dispatch(const SelectArgs& a, hipStream_t s) {
  const dim3 grid(a.n_q_heads, a.batch), block(kTauHatThreads);
  switch (a.group) {
    case 1: hipLaunchKernelGGL((tau_hat_kernel<1, GEN, LIVE>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((tau_hat_kernel<2, GEN, LIVE>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((tau_hat_kernel<4, GEN, LIVE>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((tau_hat_kernel<8, GEN, LIVE>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The live-page list holds 8192 pages (two blocks per compute unit) unless a
// sequence can have more pages; then 16384 (128 KB of LDS, one block per
// unit), so that long sequences keep iterating on chip.
template <int E>
static hipError_t gauss_floor_dispatch(const SelectArgs& a, hipStream_t s) {
  const dim3 grid(a.n_kv_heads, a.batch), block(kSelThreads);
  switch (a.group) {
    case 1: hipLaunchKernelGGL((gauss_floor_kernel<1, E>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gauss_floor_kernel<2, E>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gauss_floor_kernel<4, E>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((gauss_floor_kernel<8, E>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Needs max_pages <= 65535 (the top-k block's limit, checked on the host).
hipError_t launch_gauss_floor(const SelectArgs& a, hipStream_t s) {
  const int per = (a.max_pages + kSelThreads - 1) / kSelThreads;
  if (per <= 4) return gauss_floor_dispatch<4>(a, s);
  if (per <= 16) return gauss_floor_dispatch<16>(a, s);
  return gauss_floor_dispatch<0>(a, s);
}

hipError_t launch_tau_hat(const SelectArgs& a, hipStream_t s) {
  const bool gen = !(a.alpha == 1.5f || a.alpha == 2.0f);
  if (a.max_pages > kTauHatLive)
    return gen ? tau_hat_dispatch<true, kTauHatLiveBig>(a, s) : tau_hat_dispatch<false, kTauHatLiveBig>(a, s);
  return gen ? tau_hat_dispatch<true, kTauHatLive>(a, s) : tau_hat_dispatch<false, kTauHatLive>(a, s);
}

}  // namespace ekv
