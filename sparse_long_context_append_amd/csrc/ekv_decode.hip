// Sparse (or full-cache) exact alpha-entmax decode (EntmaxKV summary
// sec. 2.C: load only the selected pages' keys and values and compute the
// alpha-entmax weights over that reduced set).
//
// gather_score  grid of (slot, unit) blocks over work items of 64 consecutive
//               tokens of a (sequence, KV head)'s page list.  Each K row is read once
//               and scored against every query head of the group,
//               x = (alpha-1) scale q.k.  For bf16 keys and groups of up to
//               4 heads the scores come from the matrix cores (16 tokens x
//               4 heads x 3 limbs of q per instruction), otherwise from the
//               vector ALUs.  An item keeps only tokens that can be in the
//               support: x > (item max) - 1, since the threshold satisfies
//               tau >= (head max) - 1 >= (item max) - 1 (the top token's
//               weight is at most 1).
// tau_v         one block per (sequence, query head): collects the
//               candidates above (head max) - 1 (skipping items whose
//               maximum is not above it), finds the exact threshold and
//               support in float64, and accumulates sum_j p_j v_j over the
//               support rows (rows split across the block, fixed-order
//               combine, so results are bitwise reproducible).
#include "ekv_kernels.h"

#include <type_traits>

namespace ekv {

constexpr int kDecThreads = 256;
constexpr int kTauThreads = 256;
// A head of at most this many items keeps its item records in the threshold
// kernel's registers (four per thread); only larger heads use the per-item
// level counts, so the gather computes them only where some unit may have
// more (chosen on the host from the list capacity).
constexpr int kTauFewItems = 4 * kTauThreads;
constexpr int kTauItemChunk = 1024;
constexpr int kCollectU = 16;  // items per wave per on-chip collection round
constexpr int kVRows = 8;      // V rows in flight per thread in the weighted sum
constexpr int kSolveBatch = 8; // scores loaded at once per thread in a threshold pass

// A stored length clamped to [0, max_pages * P].
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int L) {
  if (L < 0 || (long long)L > (long long)a.max_pages * a.page_size) return L < 0 ? 0 : a.max_pages * a.page_size;
  return L;
}

__device__ __forceinline__ int dec_len(const DecodeArgs& a, int b) { return clamp_len(a, a.seq_lens[b]); }

// Number of page-list entries of a unit from its sequence's stored length
// and its list's stored count (ignored without lists).
__device__ __forceinline__ int unit_pages_of(const DecodeArgs& a, int L, int cnt) {
  const int n_b = pages_of(clamp_len(a, L), a.page_size);
  return a.sel ? min(max(cnt, 0), min(a.cap, n_b)) : n_b;
}

// The stored list count of unit u, read without a branch (the length of
// sequence 0 stands in without lists).
__device__ __forceinline__ int unit_count_raw(const DecodeArgs& a, int u) {
  const int32_t* p = a.sel ? a.sel_count : a.seq_lens;
  return p[a.sel ? (u >> a.sel_shift) : 0];
}

// Number of page-list entries of unit u = b * Hkv + g.
__device__ __forceinline__ int unit_pages(const DecodeArgs& a, int u) {
  return unit_pages_of(a, a.seq_lens[u / a.n_kv_heads], unit_count_raw(a, u));
}

__device__ __forceinline__ int unit_items(const DecodeArgs& a, int u) {
  return (int)(((long long)unit_pages(a, u) * a.page_size + kItemTokens - 1) / kItemTokens);
}

// Token r of item j of unit u: its physical row (page * P + slot), logical
// token id, and whether it holds a valid key.
struct TokenRef {
  int phys, slot, logical;
  bool valid;
};

__device__ __forceinline__ TokenRef token_ref(const DecodeArgs& a, int u, int b, int L, int n_b, int npu, int j,
                                              int r) {
  TokenRef t{-1, 0, 0, false};
  const int P = a.page_size;
  const long long T = (long long)j * kItemTokens + r;
  if (T >= (long long)npu * P) return t;
  const int k = (int)(T >> __builtin_ctz(P));  // P is a power of two
  t.slot = (int)(T & (P - 1));
  const int lp = a.sel ? a.sel[(size_t)(u >> a.sel_shift) * a.cap + k] : k;
  if (lp < 0 || lp >= n_b) {
    set_status(a.status, EKV_DEV_BAD_PAGE);
    return t;
  }
  const int phys = a.page_table[(size_t)b * a.max_pages + lp];
  if (phys < 0 || phys >= a.n_phys) {
    set_status(a.status, EKV_DEV_BAD_PAGE);
    return t;
  }
  t.phys = phys;
  t.logical = lp * P + t.slot;
  t.valid = t.slot < L - lp * P;
  return t;
}

// Sizes of one unit (sequence b, KV head g) of a (slot, unit) grid.
struct UnitCtx {
  int L, n_b, npu, n_items;
};

// References of token r in items j0 .. j0+SUB-1 of unit u, resolved in two
// dependent rounds whose loads all travel together: round one (refs_list)
// reads the page-list entries (and, when `first`, the sequence length and
// selection count), round two (refs_table) the page-table entries.  Entries
// are range-checked against the table before the length is known and
// against the length afterwards (refs_finish).  Split in three so that a
// kernel can keep the next super-item's rounds in flight behind its current
// work.
template <int SUB> struct RefPipe {
  int lp[SUB], ph[SUB];
  int j0, r, L, cnt, b;
  bool first;
};

template <int SUB>
__device__ __forceinline__ void refs_list(const DecodeArgs& a, int u, int b, int j0, int r, bool first,
                                          RefPipe<SUB>& rp) {
  const int P = a.page_size;
  const int capk = a.sel ? min(a.cap, a.max_pages) : a.max_pages;
  rp.b = b;
  rp.j0 = j0;
  rp.r = r;
  rp.first = first;
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    const long long T = (long long)(j0 + s) * kItemTokens + r;
    const int k = (int)(T >> __builtin_ctz(P));  // P is a power of two
    // read from a clamped index and masked afterwards (no branch per load)
    const int v = a.sel ? a.sel[(size_t)(u >> a.sel_shift) * a.cap + min(k, capk - 1)] : k;
    rp.lp[s] = k < capk ? v : -1;
  }
  if (first) {
    rp.L = a.seq_lens[b];
    rp.cnt = a.sel ? a.sel_count[u >> a.sel_shift] : 0;
  }
}

template <int SUB>
__device__ __forceinline__ void refs_table(const DecodeArgs& a, RefPipe<SUB>& rp) {
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    const bool in = rp.lp[s] >= 0 && rp.lp[s] < a.max_pages;
    const int v = a.page_table[(size_t)rp.b * a.max_pages + (in ? rp.lp[s] : 0)];
    rp.ph[s] = in ? v : -1;
  }
}

template <int SUB>
__device__ __forceinline__ void refs_finish(const DecodeArgs& a, const RefPipe<SUB>& rp, UnitCtx* ctx, TokenRef* tr) {
  const int P = a.page_size;
  if (rp.first) {
    int L = rp.L;
    if (L < 0 || (long long)L > (long long)a.max_pages * P) L = L < 0 ? 0 : a.max_pages * P;
    ctx->L = L;
    ctx->n_b = pages_of(L, P);
    ctx->npu = a.sel ? min(max(rp.cnt, 0), min(a.cap, ctx->n_b)) : ctx->n_b;
    ctx->n_items = (int)(((long long)ctx->npu * P + kItemTokens - 1) / kItemTokens);
  }
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    const long long T = (long long)(rp.j0 + s) * kItemTokens + rp.r;
    const int k = (int)(T >> __builtin_ctz(P));  // P is a power of two
    const int slot = (int)(T & (P - 1));
    tr[s] = TokenRef{-1, slot, 0, false};
    if (T >= (long long)ctx->npu * P) continue;
    if (rp.lp[s] < 0 || rp.lp[s] >= ctx->n_b || rp.ph[s] < 0 || rp.ph[s] >= a.n_phys) {
      set_status(a.status, EKV_DEV_BAD_PAGE);
      continue;
    }
    tr[s].phys = rp.ph[s];
    tr[s].logical = rp.lp[s] * P + slot;
    tr[s].valid = slot < ctx->L - rp.lp[s] * P;
  }
}

template <int SUB>
__device__ __forceinline__ void resolve_refs(const DecodeArgs& a, int u, int b, int j0, int r, bool first,
                                             UnitCtx* ctx, TokenRef* tr) {
  RefPipe<SUB> rp;
  refs_list<SUB>(a, u, b, j0, r, first, rp);
  refs_table<SUB>(a, rp);
  refs_finish<SUB>(a, rp, ctx, tr);
}

// ---------------------------------------------------------------------------
// Matrix-core gather (bf16 keys).  Grid (slots, units): block
// (s, u) takes super-items s, s + slots, ... of unit u, a super-item being
// SUB consecutive 64-token items whose loads are all issued before any is
// used.  A rows 4h + l hold limb l of q_h (alpha-1) scale; B columns are the
// 16 tokens of a wave; the fp32 accumulator runs over the D/32 k blocks.
// Lane l ends with head l/16 of token l%16: x = (c0 + c1) + c2.  Groups of
// 8 heads take a second operand (heads 4..7) against the same K fragment.
// ---------------------------------------------------------------------------
// n^-(alpha-1): the largest distance below a level shared by n scores at
// which their weights alone reach 1.
// Evaluated in float and rounded up by a relative 1e-5, so the bound
// stays below the exact one.
// The hardware reciprocal, reciprocal square root, exp2 and log2 are within
// a few ulp (about 1e-6 relative for the exp2/log2 pair), well inside the
// 1e-5 rounding up.
__device__ __forceinline__ double count_pow(int n, float alpha) {
  const float nf = (float)n;
  float v;
  if (alpha == 2.0f) v = __builtin_amdgcn_rcpf(nf);
  else if (alpha == 1.5f) v = __builtin_amdgcn_rsqf(nf);
  else v = __builtin_amdgcn_exp2f(-(alpha - 1.f) * __builtin_amdgcn_logf(nf));
  return (double)v * (1.0 + 1e-5);
}

// Balanced assignment (BAL): the super-items of all units are numbered
// unit by unit, and block i takes the contiguous range [i C, i C + C),
// C = ceil(total / blocks), so every block gets the same work whatever the
// units' sizes and most blocks stay inside one unit.  Every wave computes
// the numbering itself from the units' sizes (lane l: units 8 l .. 8 l + 7,
// at most 512 units), without a block barrier.
struct UnitWalk {
  int incl;     // inclusive count of super-items through this lane's units
  int pre[8];   // first super-item of each of this lane's units
  int sup[8];   // super-items of each
};

template <int SUB>
__device__ __forceinline__ int unit_walk(const DecodeArgs& a, UnitWalk* uw) {
  const int lane = threadIdx.x & 63, units = a.batch * a.n_kv_heads;
  int len[8], cnt[8];  // every load first (the last unit stands in past the end)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int u = min(8 * lane + k, units - 1);
    len[k] = a.seq_lens[u / a.n_kv_heads];
    cnt[k] = unit_count_raw(a, u);
  }
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int items = (int)(((long long)unit_pages_of(a, len[k], cnt[k]) * a.page_size + kItemTokens - 1) / kItemTokens);
    uw->sup[k] = 8 * lane + k < units ? (items + SUB - 1) / SUB : 0;
    sum += uw->sup[k];
  }
  uw->incl = wave_incl_scan(sum);
  int run = uw->incl - sum;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uw->pre[k] = run;
    run += uw->sup[k];
  }
  return __builtin_amdgcn_readlane(uw->incl, 63);
}

// The unit holding super-item gs (gs < total) and gs's index inside it.
__device__ __forceinline__ void unit_locate(const UnitWalk& uw, int gs, int* u, int* sj) {
  const int owner = __popcll(__ballot(uw.incl <= gs));  // lanes whose units all end at or before gs
  int k = 0;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) k += __builtin_amdgcn_readlane(uw.pre[kk] + uw.sup[kk], owner) <= gs;
  int p = 0;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) p = kk == k ? uw.pre[kk] : p;
  *u = 8 * owner + k;
  *sj = gs - __builtin_amdgcn_readlane(p, owner);
}

// LVL: some unit may have more than kTauFewItems items, whose per-item level
// counts the threshold kernel reads (every unit's are written then)
template <int D, int G, int SUB, bool BAL, bool LVL>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(BAL || G > 4 ? 2 : 4))) void gather_mfma_kernel(
    DecodeArgs a, int slots) {
  constexpr int KB = D / 32;
  constexpr int NH = (G + 3) / 4;  // 16-row operands (four heads each)
  __shared__ u32x4_t s_a[NH * KB][kWave];
  // per-wave item maxima and kept counts, [head operand][item][head][wave]:
  // a lane reads the four waves' values of its head in one 16-byte load
  __shared__ float4 s_max[NH][SUB][4];
  __shared__ int4 s_cnt[NH][SUB][4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = a.n_kv_heads;
  const size_t tok_per_bh = (size_t)a.max_items * kItemTokens;
  const int r = 16 * w + col;  // this lane's token within an item
  int u, sj, gs = 0, gs_end = 0;
  UnitWalk uw;
  if (BAL) {
    const int total = unit_walk<SUB>(a, &uw);
    const int C = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    gs = (int)blockIdx.x * C;
    gs_end = min(gs + C, total);
    if (gs >= gs_end) return;  // block-uniform: nothing left for this block
    unit_locate(uw, gs, &u, &sj);
  } else {
    u = blockIdx.y;
    sj = blockIdx.x;
  }
  int b = u / Hkv, g = u - b * Hkv;

  // loads, in order: q for the A operand, then the first super-item's
  // references (resolved speculatively with the unit's size)
  const float qs = (a.alpha - 1.f) * a.scale;
  LimbChunks<KB, NH> lc;
  auto fetch_q = [&]() {
    const float* qg = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * D;
    limb_fetch<KB, G, NH>(lc, [&](int h, int k0, float* v) {
      const float4* qv = reinterpret_cast<const float4*>(qg + (size_t)h * D + k0);
      const float4 q0 = qv[0], q1 = qv[1];
      v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w; v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    });
  };
  fetch_q();
  UnitCtx ctx;
  TokenRef tr[SUB];
  resolve_refs<SUB>(a, u, b, sj * SUB, r, true, &ctx, tr);
  bool a_ready = false;
  const int n_super = (ctx.n_items + SUB - 1) / SUB;
  RefPipe<SUB> nxt;  // the next super-item's references, in flight behind this one
  while (BAL || sj < n_super) {
    // every lane loads (a lane without a token reads row 0 of the cache and
    // zeroes the values), so the loads carry no branches and the first
    // product waits only for its own item's keys
    u32x4_t bv[SUB][KB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      const bool has = tr[s].phys >= 0;
      const size_t rowi = has ? ((size_t)tr[s].phys * a.hkv_mem + (g >> a.kv_shift)) * a.page_size + tr[s].slot : 0;
      const uint16_t* row = reinterpret_cast<const uint16_t*>(a.k) + rowi * D + 8 * grp;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + 32 * kb);
        bv[s][kb] = has ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    // the next super-item of this block, and its page-list round
    int nu = u, nsj;
    bool has_next;
    if (BAL) {
      has_next = gs + 1 < gs_end;
      if (has_next) unit_locate(uw, gs + 1, &nu, &nsj);
    } else {
      nsj = sj + slots;
      has_next = nsj < n_super;
    }
    if (has_next) refs_list<SUB>(a, nu, nu / Hkv, nsj * SUB, r, BAL, nxt);
    if (!a_ready) {  // q limbs: coefficients q_h (alpha-1) scale (block-uniform)
      limb_build<KB, G, NH>(s_a, lc, [qs](int, float qv) { return qv * qs; });
      __syncthreads();
      a_ready = true;
    }
    // lane holds heads grp + 4 hh (hh < NH) of token col
    float x[NH][SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) c = mfma_bf16(s_a[hh * KB + kb][lane], bv[s][kb], c);
        x[hh][s] = tr[s].valid && 4 * hh + grp < G ? (c[0] + c[1]) + c[2] : -INFINITY;
        // per-head item maximum (the 16 lanes of one head share grp)
        const float m = group_reduce<16>(x[hh][s], [](float u, float v) { return fmaxf(u, v); });
        if (col == 0) reinterpret_cast<float*>(&s_max[hh][s][grp])[w] = m;
      }
    }
    // this super-item's token ids and rows, kept aside so that the next
    // super-item's references can be finished before the stores below (a
    // later wait on them would also wait for those stores)
    int ct_cur[SUB], cr_cur[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      ct_cur[s] = tr[s].logical;
      cr_cur[s] = tr[s].phys * a.page_size + tr[s].slot;
    }
    const int n_items_cur = ctx.n_items;
    if (has_next) refs_table<SUB>(a, nxt);  // its page-list entries are in by now
    __syncthreads();
    // candidates: above a lower bound on tau (tokens at or below it have
    // weight 0).  The super-item maximum gives msup - 1 (the top token alone
    // has weight at most 1).  More generally, if n tokens lie at or above a
    // level l, tau >= l - n^-(alpha-1) (a subset's threshold never exceeds
    // the full set's); this wave's tokens of the head are counted at
    // l = msup - 1/8, - 1/4, - 1/2.
    float m[NH][SUB];
    double lb[NH];
    float msup[NH];
    bool keep[NH][SUB];
    uint32_t bits[NH][SUB];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const bool hv = 4 * hh + grp < G;
      msup[hh] = -INFINITY;
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const float4 mv = s_max[hh][s][grp];
        m[hh][s] = fmaxf(fmaxf(mv.x, mv.y), fmaxf(mv.z, mv.w));
        msup[hh] = fmaxf(msup[hh], m[hh][s]);
      }
      lb[hh] = (double)msup[hh] - 1.0;
#pragma unroll
      for (int ci = 0; ci < 3; ++ci) {
        const float lvl = msup[hh] - 0.125f * (float)(1 << ci);
        int n = 0;
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          const unsigned long long bal = __ballot(hv && x[hh][s] >= lvl);
          n += __popc((uint32_t)(bal >> (16 * grp)) & 0xffffu);
        }
        if (n > 0) lb[hh] = fmax(lb[hh], (double)lvl - count_pow(n, a.alpha));
      }
      lb[hh] -= 1e-6 * fmax(1.0, fabs((double)msup[hh]));  // margin for the rounding of x
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        keep[hh][s] = hv && msup[hh] > -INFINITY && (double)x[hh][s] > lb[hh];
        const unsigned long long bal = __ballot(keep[hh][s]);
        bits[hh][s] = (uint32_t)(bal >> (16 * grp)) & 0xffffu;
        // with LVL, the item's scores at or above its maximum - 1/32, - 1/16,
        // - 1/8 (the threshold kernel's count bound on heads of many items),
        // packed beside the kept count in 8-bit fields (at most 16 per wave,
        // 64 per item)
        uint32_t pk = __popc(bits[hh][s]);
        if (LVL) {
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const float lv = m[hh][s] - 0.03125f * (float)(1 << k);
            const unsigned long long bl = __ballot(hv && x[hh][s] >= lv);
            pk |= (uint32_t)__popc((uint32_t)(bl >> (16 * grp)) & 0xffffu) << (8 * (k + 1));
          }
        }
        if (col == 0) reinterpret_cast<int*>(&s_cnt[hh][s][grp])[w] = (int)pk;
      }
    }
    if (has_next) refs_finish<SUB>(a, nxt, &ctx, tr);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int h = 4 * hh + grp;
      if (h >= G) continue;
      const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int j = sj * SUB + s;
        if (j >= n_items_cur) break;
        const int4 cv = s_cnt[hh][s][grp];
        constexpr int FM = LVL ? 0xff : -1;  // the kept-count field (LVL packs level counts above it)
        const int off = (w > 0 ? cv.x & FM : 0) + (w > 1 ? cv.y & FM : 0) + (w > 2 ? cv.z & FM : 0);
        const uint32_t pks = (uint32_t)((cv.x + cv.y) + (cv.z + cv.w));  // the fields' sums (<= 64 each)
        const int tot = (int)(pks & (uint32_t)FM);
        if (keep[hh][s]) {
          const int pos = off + __popc(bits[hh][s] & ((1u << col) - 1u));
          const size_t at = bh * tok_per_bh + (size_t)j * kItemTokens + pos;
          a.cand_x[at] = x[hh][s];
          a.cand_t[at] = ct_cur[s];
          a.cand_r[at] = cr_cur[s];
        }
        if (w == 0 && col == 0) {
          a.item_cnt[bh * a.max_items + j] = tot;
          a.item_max[bh * a.max_items + j] = m[hh][s];
          a.item_lb[bh * a.max_items + j] = msup[hh] > -INFINITY ? __double2float_rd(lb[hh]) : -INFINITY;
          if (LVL) a.item_lvl[bh * a.max_items + j] = pks >> 8;
        }
      }
    }
    __syncthreads();  // s_max / s_cnt (and s_a on a unit change) are rewritten next
    if (!has_next) break;
    if (BAL) {
      ++gs;
      if (nu != u) {  // the next unit's queries
        u = nu;
        b = u / Hkv;
        g = u - b * Hkv;
        fetch_q();
        a_ready = false;
      }
    }
    sj = nsj;
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU gather (fp32 keys): LPR lanes per K row, every
// load of the item issued up front, fp32 dot products reduced across the
// row's lanes; scores staged in LDS, then one wave per head compacts.
// ---------------------------------------------------------------------------
template <int DT, int D, int G>
__global__ __launch_bounds__(kDecThreads) void gather_valu_kernel(DecodeArgs a, int slots) {
  using E = Elem<DT>;
  constexpr int EPL = E::kPerVec;
  constexpr int LPR = D / EPL;           // lanes per K row
  static_assert(LPR <= kWave && G <= LPR, "layout");
  constexpr int RPW = kWave / LPR;       // rows per wave load
  constexpr int RPI = 4 * RPW;           // rows per block load
  constexpr int NIT = kItemTokens / RPI; // loads per lane per item
  __shared__ float s_x[G][kItemTokens];
  __shared__ int s_t[kItemTokens], s_r[kItemTokens];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane % LPR, dim0 = sub * EPL, rloc = lane / LPR;
  const int u = blockIdx.y, Hkv = a.n_kv_heads;
  const int b = u / Hkv, g = u - b * Hkv;
  const size_t tok_per_bh = (size_t)a.max_items * kItemTokens;
  UnitCtx ctx;
  TokenRef tr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    resolve_refs<1>(a, u, b, blockIdx.x, it * RPI + w * RPW + rloc, it == 0, &ctx, &tr[it]);
  float qr[G][EPL];
  const float qs = (a.alpha - 1.f) * a.scale;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G + h) * D + dim0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[h][e] = qh[e] * qs;
  }
  for (int j = blockIdx.x; j < ctx.n_items; j += slots) {
    if (j != (int)blockIdx.x) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) resolve_refs<1>(a, u, b, j, it * RPI + w * RPW + rloc, false, &ctx, &tr[it]);
    }
    uint4 v[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + w * RPW + rloc;
      if (tr[it].phys >= 0)
        v[it] = ldg16(reinterpret_cast<const char*>(a.k) +
                      ((((size_t)tr[it].phys * a.hkv_mem + (g >> a.kv_shift)) * a.page_size + tr[it].slot) * D + dim0) * E::kBytes);
      if (sub == 0) {
        s_t[r] = tr[it].logical;
        s_r[r] = tr[it].phys * a.page_size + tr[it].slot;
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + w * RPW + rloc;
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      if (tr[it].valid) {
        float f[EPL];
        E::unpack(v[it], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = fmaf(qr[h][e], f[e], acc[h]);
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] += __shfl_xor(acc[h], m, kWave);
      if (sub < G) {
        float xv = acc[0];
#pragma unroll
        for (int h = 1; h < G; ++h) if (sub == h) xv = acc[h];
        s_x[sub][r] = tr[it].valid ? xv : -INFINITY;
      }
    }
    __syncthreads();
    for (int h = w; h < G; h += 4) {
      const float x = s_x[h][lane];
      const float m = wave_max(x);
      const bool keep = m > -INFINITY && (double)x > (double)m - 1.0;
      const unsigned long long bal = __ballot(keep);
      const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
      if (keep) {
        const int pos = __popcll(bal & ((1ull << lane) - 1ull));
        const size_t at = bh * tok_per_bh + (size_t)j * kItemTokens + pos;
        a.cand_x[at] = x;
        a.cand_t[at] = s_t[lane];
        a.cand_r[at] = s_r[lane];
      }
      uint32_t lv3 = 0u;  // scores at or above m - 1/32, - 1/16, - 1/8 (heads of many items)
      if (ctx.n_items > kTauFewItems) {  // block-uniform
#pragma unroll
        for (int k = 0; k < 3; ++k) lv3 |= (uint32_t)__popcll(__ballot(x >= m - 0.03125f * (float)(1 << k))) << (8 * k);
      }
      if (lane == 0) {
        a.item_cnt[bh * a.max_items + j] = __popcll(bal);
        a.item_max[bh * a.max_items + j] = m;
        a.item_lb[bh * a.max_items + j] = m > -INFINITY ? __double2float_rd((double)m - 1.0) : -INFINITY;
        if (ctx.n_items > kTauFewItems) a.item_lvl[bh * a.max_items + j] = m > -INFINITY ? lv3 : 0u;
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
// (d)^(1/(alpha-1)) for d > 0: AK = 0 for alpha 2, 1 for alpha 1.5, 2 otherwise
// (compile-time, so the common cases carry no pow).
template <int AK> __device__ __forceinline__ double entmax_pow(double d, double beta) {
  if (AK == 0) return d;
  if (AK == 1) return d * d;
  return pow(d, beta);
}

// Exact threshold of the N candidate scores xs (all threads of the calling
// wave, or of the block, take part; every one gets the result).  Other
// alpha, whole block: when the fp32 steps end, the scores that can still
// matter are copied to prune_buf (room for prune_cap) if they fit there.
template <bool WAVE, int AK>
__device__ double solve_threshold(const float* xs, int N, double m, double thr, float alpha_f, double* redd,
                                  float* prune_buf = nullptr, int prune_cap = 0) {
  const int idx = WAVE ? (threadIdx.x & 63) : threadIdx.x;
  const int stride = WAVE ? kWave : blockDim.x;
  constexpr bool sparsemax = AK == 0, ent15 = AK == 1;
  const double beta = 1.0 / ((double)alpha_f - 1.0);
  const float beta_f = (float)beta;
  double t = thr, tau = thr, t_prev = thr;
  // other alpha: the powers are first taken in fp32 (hardware exp2/log2)
  // while the steps are large, then in fp64 for the last steps
  bool coarse = AK == 2;
  for (int it = 0; it < 4096; ++it) {
    tau = t;  // fallback if the iteration cap is ever reached
    double s1 = 0.0, s2 = 0.0, f = 0.0, fd = 0.0, xmin = INFINITY, cnt = 0.0;
    // kSolveBatch scores per thread loaded at once (the list may be in
    // global memory), then taken in the same order as one at a time
    for (int i0 = idx; i0 < N; i0 += kSolveBatch * stride) {
      float xb[kSolveBatch];
#pragma unroll
      for (int u = 0; u < kSolveBatch; ++u) xb[u] = load_or(xs, i0 + u * stride, N, -INFINITY);
#pragma unroll
      for (int u = 0; u < kSolveBatch; ++u) {
        const double x = xb[u];
        if (x > t) {
          const double y = x - m, d = x - t;
          cnt += 1.0; s1 += y; s2 += y * y; xmin = fmin(xmin, x);
          const double pw = AK == 2 && coarse
                                ? (double)__builtin_amdgcn_exp2f(beta_f * __builtin_amdgcn_logf((float)d))
                                : entmax_pow<AK>(d, beta);
          f += pw;
          fd += sparsemax ? 1.0 : (ent15 ? 2.0 * d : beta * pw / d);
        }
      }
    }
    if (WAVE) {
      cnt = wave_sum(cnt);
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      f = wave_sum(f);
      fd = wave_sum(fd);
      xmin = wave_min(xmin);
    } else if (AK == 2) {  // (other alpha needs neither the moments nor xmin)
      double v[3] = {cnt, f, fd};
      block_sums<3>(v, redd);
      cnt = v[0];
      f = v[1];
      fd = v[2];
    } else {  // the sums in one reduction (same order as one at a time)
      double v[5] = {cnt, s1, s2, f, fd};
      block_sums<5>(v, redd);
      cnt = v[0];
      s1 = v[1];
      s2 = v[2];
      f = v[3];
      fd = v[4];
      xmin = block_min(xmin, redd);
    }
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
      // Newton's method on f^(1/e) - 1 (f^(1/e) is the e-norm of (x - t)_+,
      // convex and decreasing in t, and linear for a single score): from
      // below tau the steps stay below it and converge quadratically.  A
      // step may cross tau only through the rounding of the fp32 phase; the
      // next one then comes back from the right.
      if (!(fd > 0.0)) { tau = t_prev; break; }
      const double step = beta * (f - pow(f, 1.0 - 1.0 / beta)) / fd;
      t += step;
      tau = t;
      const double size = fabs(step), scale_t = fmax(1.0, fabs(t));
      if (coarse) {
        if (size <= 1e-6 * scale_t) {
          coarse = false;
          if (!WAVE && AK == 2 && prune_buf) {
            // t is now within about 1e-6 of tau and the fp64 steps stay
            // there: a score at or below cut = t - 1e-4 max(1, |t|) adds
            // nothing to any later pass, so the others are listed apart
            // (in order: contiguous ranges, one scan), when they fit
            const double cut = t - 1e-4 * scale_t;
            const int E = (N + stride - 1) / stride;
            const int e0 = min(idx * E, N), e1 = min(e0 + E, N);
            int c = 0;
            for (int i0 = e0; i0 < e1; i0 += kSolveBatch) {
              float xb[kSolveBatch];
#pragma unroll
              for (int u = 0; u < kSolveBatch; ++u) xb[u] = load_or(xs, i0 + u, e1, -INFINITY);
#pragma unroll
              for (int u = 0; u < kSolveBatch; ++u) c += (double)xb[u] > cut;
            }
            int total;
            int pos = block_exclusive_scan(c, reinterpret_cast<int*>(redd), &total);
            if (total <= prune_cap) {
              for (int i0 = e0; i0 < e1; i0 += kSolveBatch) {
                float xb[kSolveBatch];
#pragma unroll
                for (int u = 0; u < kSolveBatch; ++u) xb[u] = load_or(xs, i0 + u, e1, -INFINITY);
#pragma unroll
                for (int u = 0; u < kSolveBatch; ++u)
                  if ((double)xb[u] > cut) prune_buf[pos++] = xb[u];
              }
              __syncthreads();
              xs = prune_buf;
              N = total;
            }
          }
        }
      } else if (size <= 1e-15 * scale_t || it > 4000) {
        break;
      }
    }
  }
  return tau;
}

// tau from the support's count c and the sums s1, s2 of (x - m) and
// (x - m)^2 over it: sum_S (x - tau) = 1 (alpha 2), sum_S (x - tau)^2 = 1
// (alpha 1.5, the larger root of the quadratic).
template <int AK> __device__ __forceinline__ double support_tau(double c, double s1, double s2, double m) {
  if (AK == 0) return m + (s1 - 1.0) / c;
  const double mu = s1 / c;
  const double disc = (1.0 - c * (s2 / c - mu * mu)) / c;
  return m + mu - sqrt(fmax(disc, 0.0));
}

// Exact threshold of at most blockDim.x candidates (in LDS) by the pairwise
// support test, alpha 2 and 1.5: with f(t) = sum_j (x_j - t)_+^e decreasing
// and f(tau) = 1, x_i is in the support iff f(x_i) < 1.  Thread i evaluates
// f(x_i); tau follows from the closed form on the support.  All threads of
// the block take part and get the result.
template <int AK>
__device__ double solve_pairwise(const float* lx, int N, double m, double* red) {
  static_assert(AK == 0 || AK == 1, "closed forms for alpha 2 and 1.5 only");
  const int i = threadIdx.x;
  const bool has = i < N;
  const float xif = has ? lx[i] : 0.f;
  // f in float32 (its rounding, about N 2^-24 f, only matters for scores
  // that lie within that distance of tau), the x_j in ascending j; every
  // lane reads four of them with one broadcast LDS load
  float ff = 0.f;
  auto acc = [&](float xj) {
    const float d = fmaxf(xj - xif, 0.f);
    ff += AK == 0 ? d : d * d;
  };
  const float4* x4 = reinterpret_cast<const float4*>(lx);
  const int n4 = N >> 2;
#pragma unroll 4
  for (int q = 0; q < n4; ++q) {
    const float4 v = x4[q];
    acc(v.x);
    acc(v.y);
    acc(v.z);
    acc(v.w);
  }
  for (int j = 4 * n4; j < N; ++j) acc(lx[j]);
  const bool in = has && (double)ff < 1.0;
  const double y = (double)xif - m;
  double c = in ? 1.0 : 0.0, s1 = in ? y : 0.0, s2 = in ? y * y : 0.0;
  block_sum3(c, s1, s2, red);
  return support_tau<AK>(c, s1, s2, m);
}

// On-chip scratch of the threshold stage (one instance per block), with room
// for CAP candidates: kLdsCands, or kLdsCandsBig (about 115 KB) when every
// block of the launch has a compute unit of its own anyway.
constexpr int kLdsCandsBig = 8192;
constexpr int kWaveCands = 128;  // candidates the single-wave threshold path takes (two per lane)
template <int CAP> struct TauSmem {
  alignas(16) float lx[CAP];  // (read four at a time by the pairwise test)
  int lt[CAP];
  int lr[CAP];
  int s_pre[kTauItemChunk + 1];
  int s_item[kTauItemChunk];
  int s_icnt[kTauItemChunk];  // candidate counts of the listed items (on-chip collection)
  int s_tab[2][65];  // per-item kept counts of a collection round (rounds alternate halves)
  float vpart[2048];  // row-group partial outputs (RPB x D <= 2048)
  double redd[48];  // block reductions (up to three values per wave)
  int redi[17];
  double s_tau;
  double s_ps;  // the single-wave threshold path's outputs
  int s_nsup;
  float pc[kWaveCands];  // its weights by candidate (0 off the support), when waves 1..3 prefetch the V rows
  uint32_t s_mkey[4];
  int s_kcnt[4];
  int s_flag;
};

// Threshold, support and output of query head h of sequence b from the
// candidate lists of its unit; the whole block takes part.
template <int DT, int D, int AK, int CAP>
__device__ __forceinline__ void tau_v_block(const DecodeArgs& a, int b, int h, TauSmem<CAP>& sm) {
  using E = Elem<DT>;
  const int tid = threadIdx.x;
  const int G = a.group, g = h / G, Hkv = a.n_kv_heads, P = a.page_size;
  const int u = b * Hkv + g;
  const size_t bh = (size_t)b * a.n_q_heads + h;
  const size_t tok_per_bh = (size_t)a.max_items * kItemTokens;
  float* lx = sm.lx;
  int* lt = sm.lt;
  int* lr = sm.lr;
  int* s_pre = sm.s_pre;
  double* redd = sm.redd;
  int* redi = sm.redi;
  constexpr int EPL = E::kPerVec;
  constexpr int LPR = D / EPL;
  constexpr int RPB = kTauThreads / LPR;
  __syncthreads();  // sm may still be in use by the caller

  const int32_t* icnt = a.item_cnt + bh * a.max_items;
  const float* imax = a.item_max + bh * a.max_items;
  const float* ilb = a.item_lb + bh * a.max_items;
  const uint32_t* ilv = a.item_lvl + bh * a.max_items;
  // the first IPT * kTauThreads items' records are requested before the
  // unit's size is known (indices clamped to the unit's item slots, the
  // values past the unit's items masked once it is)
  constexpr int IPT = kTauFewItems / kTauThreads;  // items per thread with few items
  int loc[IPT];
  float lmx[IPT], lbv[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int jj = min(IPT * threadIdx.x + i, a.max_items - 1);
    loc[i] = icnt[jj];
    lmx[i] = imax[jj];
    lbv[i] = ilb[jj];
  }
  const int n_items = unit_items(a, u);
  float* out = a.out + bh * D;
  const float* cx = a.cand_x + bh * tok_per_bh;
  const int32_t* ct = a.cand_t + bh * tok_per_bh;
  const int32_t* cr = a.cand_r + bh * tok_per_bh;

  // ---- item counts and maxima (one round of loads) ----
  constexpr int RPT = 16;  // raw candidates per thread per round of the workspace path
  const int tid_w = tid >> 6;
  const bool few_items = n_items <= kTauFewItems;
  float lmax = -INFINITY, llb = -INFINITY;
  if (few_items) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (IPT * tid + i >= n_items) {
        loc[i] = 0;
        lmx[i] = -INFINITY;
        lbv[i] = -INFINITY;
      }
      llb = fmaxf(llb, lbv[i]);
      lmax = fmaxf(lmax, lmx[i]);
    }
  } else {
    // eight loads in flight per thread per round
    for (int j0 = tid; j0 < n_items; j0 += 8 * kTauThreads) {
      float vm[8], vl[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kTauThreads;
        vm[u] = load_or(imax, j, n_items, -INFINITY);
        vl[u] = load_or(ilb, j, n_items, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lmax = fmaxf(lmax, vm[u]);
        llb = fmaxf(llb, vl[u]);
      }
    }
  }
  // the largest item maximum and the largest item bound in one block
  // reduction (one pair of barriers)
  float mf, lbf;
  {
    constexpr int NWV = kTauThreads / kWave;
    float* rf = reinterpret_cast<float*>(redd);  // 2 NWV floats
    const float wm = wave_max(lmax), wl = wave_max(llb);
    __syncthreads();
    if ((tid & 63) == 0) {
      rf[tid_w] = wm;
      rf[NWV + tid_w] = wl;
    }
    __syncthreads();
    mf = rf[0];
    lbf = rf[NWV];
#pragma unroll
    for (int i = 1; i < NWV; ++i) {
      mf = max(mf, rf[i]);
      lbf = max(lbf, rf[NWV + i]);
    }
  }
  if (!(mf > -INFINITY)) {  // no pages, or every page invalid (flagged): empty result
    for (int e = tid; e < D; e += blockDim.x) out[e] = 0.f;
    if (tid == 0) {
      if (a.tau) a.tau[bh] = -INFINITY;
      if (a.support_count) a.support_count[bh] = 0;
      if (a.psum) a.psum[bh] = 0.f;
    }
    return;
  }
  const double m = mf;
  // Lower bound on tau: the largest of the items' own bounds (each at least
  // its item's maximum - 1, so this is at least m - 1), and the count bound
  // on the item maxima: n items with maximum at or above a level l hold n
  // scores there, so tau >= l - n^-(alpha-1); levels m - 1/32 .. m - 1/4.
  double thr = fmax(m - 1.0, (double)lbf);
  // With few items, those above this first bound are listed in the same
  // pair of barriers as the count bound's sums (a superset of the items
  // above the final bound, whose candidates the collection filters); n_pre
  // is their number, or -1 when they are too many for one collection round
  // and are listed against the final bound instead.
  int n_pre = -1;
  if (!few_items) {  // block-uniform
    // A head of many items (a long context of clustered keys) may have its
    // top score standing alone, with the mass lower down: levels m - 1/32,
    // - 1/16, - 1/8 and m - 1/4 .. m - 3/4 in steps of 1/8, and each item
    // adds the most scores it is known to hold at or above a level: its
    // counts at its own maximum M - 1/32, - 1/16, - 1/8 (the gather's, at the
    // same float levels) where those lie at or above the level, else one
    // score when M does.
    constexpr int NL = 8;
    float lvl[NL];
    int nk[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      lvl[k] = mf - (k < 3 ? 0.03125f * (float)(1 << k) : 0.125f * (float)(k - 1));  // exact in float
      nk[k] = 0;
    }
    for (int j0 = tid; j0 < n_items; j0 += 8 * kTauThreads) {
      float vm[8];
      uint32_t vv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kTauThreads;
        vm[u] = load_or(imax, j, n_items, -INFINITY);
        vv[u] = load_or(ilv, j, n_items, 0u);
      }
#pragma unroll 1
      for (int u = 0; u < 8; ++u) {  // (not unrolled: keeps the kernel's code compact)
        const float M = vm[u];
        const float l1 = M - 0.03125f, l2 = M - 0.0625f, l3 = M - 0.125f;
        const uint32_t lv = vv[u];
        const int c1 = (int)(lv & 0xffu), c2 = (int)((lv >> 8) & 0xffu), c3 = (int)((lv >> 16) & 0xffu);
#pragma unroll
        for (int k = 0; k < NL; ++k)
          nk[k] += l3 >= lvl[k] ? c3 : l2 >= lvl[k] ? c2 : l1 >= lvl[k] ? c1 : M >= lvl[k] ? 1 : 0;
      }
    }
    // integer block sums of the level counts (one pair of barriers; the
    // collection's table is free here)
    constexpr int NWV = kTauThreads / kWave;
    static_assert(NL * NWV <= 65, "level sums in one table half");
#pragma unroll
    for (int k = 0; k < NL; ++k) nk[k] = wave_sum(nk[k]);
    __syncthreads();
    if ((tid & 63) == 0) {
#pragma unroll
      for (int k = 0; k < NL; ++k) sm.s_tab[1][NL * tid_w + k] = nk[k];
    }
    __syncthreads();
    double cb = -INFINITY;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      int t = 0;
#pragma unroll
      for (int i = 0; i < NWV; ++i) t += sm.s_tab[1][NL * i + k];
      if (t > 0) cb = fmax(cb, (double)lvl[k] - count_pow(t, a.alpha));
    }
    thr = fmax(thr, cb - 1e-6 * fmax(1.0, fabs(m)));
  } else {
    float lvl[4];
    int nk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lvl[k] = mf - 0.03125f * (float)(1 << k);
      nk[k] = 0;
    }
    if (few_items) {
#pragma unroll
      for (int i = 0; i < IPT; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) nk[k] += lmx[i] >= lvl[k];
    } else {
      for (int j0 = tid; j0 < n_items; j0 += 8 * kTauThreads) {
        float vm[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = j0 + u * kTauThreads;
          vm[u] = load_or(imax, j, n_items, -INFINITY);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int k = 0; k < 4; ++k) nk[k] += vm[u] >= lvl[k];
      }
    }
    // this thread's items above the first bound (few items)
    int nz0 = 0;
    if (few_items) {
#pragma unroll
      for (int i = 0; i < IPT; ++i) nz0 += loc[i] > 0 && (double)lmx[i] > thr;
    }
    // integer block sums of the four counts and, with few items, the
    // exclusive scan of nz0 (one pair of barriers)
    constexpr int NWV = kTauThreads / kWave;
    const int inc0 = wave_incl_scan(nz0);
    {
#pragma unroll
      for (int k = 0; k < 4; ++k) nk[k] = wave_sum(nk[k]);
      __syncthreads();
      if ((tid & 63) == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) redi[4 * tid_w + k] = nk[k];
      }
      if ((tid & 63) == 63) sm.s_tab[0][tid_w] = inc0;  // (the collection's table is free here)
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int t = 0;
#pragma unroll
        for (int i = 0; i < NWV; ++i) t += redi[4 * i + k];
        nk[k] = t;
      }
    }
    double cb = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (nk[k] > 0) cb = fmax(cb, (double)lvl[k] - count_pow(nk[k], a.alpha));
    const double thr0 = thr;
    thr = fmax(thr, cb - 1e-6 * fmax(1.0, fabs(m)));
    if (few_items) {
      int before = 0, n0 = 0;
#pragma unroll
      for (int i = 0; i < NWV; ++i) {
        const int t = sm.s_tab[0][i];
        before += i < tid_w ? t : 0;
        n0 += t;
      }
      if (n0 <= 4 * kCollectU) {  // block-uniform: one collection round takes them all
        int rank = before + inc0 - nz0;
#pragma unroll
        for (int i = 0; i < IPT; ++i)
          if (loc[i] > 0 && (double)lmx[i] > thr0) {
            sm.s_item[rank] = IPT * tid + i;
            sm.s_icnt[rank] = min(loc[i], kItemTokens);
            ++rank;
          }
        n_pre = n0;
      }
    }
  }

  // Kept candidates (above thr) of the listed items s_item[0, n_list),
  // whose candidate counts are in s_icnt, appended in item and token order
  // to the on-chip list from position N.  One wave per item, lane r reading
  // the item's candidate r, so a wave's loads are contiguous; lanes past the
  // item's count read its last candidate again, so an item of c candidates
  // costs the cache lines of c, not of 64.  kCollectU items per wave per
  // round, and one wave scans the round's 4 kCollectU per-item counts.
  // False, with the list abandoned, once it would exceed CAP.
  auto collect_lds = [&](int n_list, int& N) -> bool {
    constexpr int U = kCollectU;
    const int lane = tid & 63;
    for (int r0 = 0; r0 < n_list; r0 += 4 * U) {
      float xv[U];
      int tv[U], rv[U], cv[U], iv[U];
      // the round's items and counts first, then every load (one wait for
      // the LDS reads, not one per item)
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int k = r0 + tid_w * U + j;
        const int kk = k < n_list ? k : n_list - 1;
        iv[j] = sm.s_item[kk];
        cv[j] = sm.s_icnt[kk];
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int k = r0 + tid_w * U + j;
        const int c = cv[j];
        // (within the unit's item slots; c >= 1 for a listed item)
        const size_t at = (size_t)iv[j] * kItemTokens + min(lane, max(c - 1, 0));
        cv[j] = k < n_list ? c : 0;
        xv[j] = cx[at];
        tv[j] = ct[at];
        rv[j] = cr[at];
      }
      uint64_t mk[U];
      int mine = 0;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        mk[j] = __ballot(lane < cv[j] && (double)xv[j] > thr);
        mine = lane == j ? __popcll(mk[j]) : mine;
      }
      // the round's 4 U = 64 counts go to one half of the table (rounds
      // alternate halves, so a round's writes never meet a slower wave's
      // reads of the round before); after one barrier every wave scans all
      // of them itself
      static_assert(4 * U == kWave, "one count per lane");
      int* tab = sm.s_tab[(r0 / (4 * U)) & 1];
      if (lane < U) tab[tid_w * U + lane] = mine;
      __syncthreads();
      const int v = tab[lane];
      const int inc = wave_incl_scan(v);
      const int n_end = N + __builtin_amdgcn_readlane(inc, 63);
      if (n_end > CAP) return false;
      const int ex = inc - v;
      int off[U];
#pragma unroll
      for (int j = 0; j < U; ++j) off[j] = N + __shfl(ex, tid_w * U + j, kWave);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if ((mk[j] >> lane) & 1ull) {
          const int pos = off[j] + __popcll(mk[j] & ((1ull << lane) - 1ull));
          lx[pos] = xv[j];
          lt[pos] = tv[j];
          lr[pos] = rv[j];
        }
      }
      N = n_end;
    }
    return true;
  };

  // ---- collect candidates above thr, in item order (an item whose
  // maximum is at most thr holds none) ----
  int N = 0;
  bool in_lds = true, done = false, lds_full = false;
  if (few_items) {
    int n_ne = n_pre;
    if (n_pre < 0) {  // block-uniform
      int nz = 0;
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        if (!((double)lmx[i] > thr)) loc[i] = 0;
        nz += loc[i] > 0;
      }
      // the non-empty items, in order: one scan
      int rank = block_exclusive_scan(nz, redi, &n_ne);
#pragma unroll
      for (int i = 0; i < IPT; ++i)
        if (loc[i] > 0) {
          sm.s_item[rank] = IPT * tid + i;
          sm.s_icnt[rank] = min(loc[i], kItemTokens);
          ++rank;
        }
    }
    __syncthreads();
    done = collect_lds(n_ne, N);
    if (!done) {
      lds_full = true;
      N = 0;
    }
  }
  if (!done) {
    // general case.  The items above thr are listed (s_item) and collected
    // on chip as above; when their kept candidates do not fit there, or the
    // items are too many to list at once, the raw candidates of the listed
    // items (with their first candidate's rank in s_pre) are read RPT per
    // thread per round (one round of loads, one scan), and the kept ones
    // appended to the workspace list, which is copied on chip afterwards
    // when it fits.
    float* ox = a.ovf_x + bh * tok_per_bh;
    int32_t* ot = a.ovf_t + bh * tok_per_bh;
    int32_t* orow = a.ovf_r + bh * tok_per_bh;
    int run = 0;
    auto read_rounds = [&](int n_ne, int raw_tot) {
      for (int r0 = 0; r0 < raw_tot; r0 += RPT * kTauThreads) {
        // scores, token ids and rows in one round of loads (the ids and rows
        // of the few that pass are then at hand for the stores)
        float xv[RPT];
        int tv[RPT], rv[RPT];
        // addresses first (the last candidate stands in past the end), then
        // the loads, unconditionally
        const int i0 = r0 + RPT * tid;
        int lo = 0, hi = n_ne;  // s_pre[lo] <= min(i0, raw_tot - 1) < s_pre[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_pre[mid] <= min(i0, raw_tot - 1)) lo = mid; else hi = mid;
        }
        int k = lo;
        size_t at[RPT];
#pragma unroll
        for (int c = 0; c < RPT; ++c) {
          const int i = min(i0 + c, raw_tot - 1);
          while (s_pre[k + 1] <= i) ++k;
          at[c] = (size_t)sm.s_item[k] * kItemTokens + (i - s_pre[k]);
        }
#pragma unroll
        for (int c = 0; c < RPT; ++c) {
          xv[c] = cx[at[c]];
          tv[c] = ct[at[c]];
          rv[c] = cr[at[c]];
        }
#pragma unroll
        for (int c = 0; c < RPT; ++c)
          if (i0 + c >= raw_tot) xv[c] = -INFINITY;
        int kc = 0;
#pragma unroll
        for (int c = 0; c < RPT; ++c) kc += (double)xv[c] > thr;
        int tot;
        int pos = run + block_exclusive_scan(kc, redi, &tot);
#pragma unroll
        for (int c = 0; c < RPT; ++c)
          if ((double)xv[c] > thr) { ox[pos] = xv[c]; ot[pos] = tv[c]; orow[pos] = rv[c]; ++pos; }
        run += tot;
      }
    };
    // Usually few items reach above thr (it lies close to the top score):
    // list them all at once, in item order.  Thread t takes the contiguous
    // items [t E, t E + E), E <= 64, and marks the ones above thr in a bit
    // mask; one scan places them.
    bool listed = false;
    if (n_items <= 64 * kTauThreads) {
      const int E = (n_items + kTauThreads - 1) / kTauThreads;
      const int e0 = min(tid * E, n_items), e1 = min(e0 + E, n_items);
      uint64_t smask = 0;
      int scount = 0;
      for (int i0 = e0; i0 < e1; i0 += 8) {
        float vm[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) vm[q] = load_or(imax, i0 + q, e1, -INFINITY);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if ((double)vm[q] > thr) { smask |= 1ull << (i0 + q - e0); ++scount; }
      }
      int n_sv;
      int spos = block_exclusive_scan(scount, redi, &n_sv);
      if (n_sv <= kTauItemChunk) {
        listed = true;
        while (smask) {
          const int k = __ffsll((unsigned long long)smask) - 1;
          smask &= smask - 1;
          sm.s_item[spos++] = e0 + k;
        }
        __syncthreads();
        if (!lds_full) {
          for (int k = tid; k < n_sv; k += kTauThreads) sm.s_icnt[k] = min(icnt[sm.s_item[k]], kItemTokens);
          __syncthreads();
          done = collect_lds(n_sv, N);
          if (!done) N = 0;
        }
      }
      if (listed && !done) {
        // their raw counts and first ranks: thread t takes listed items 4t .. 4t+3
        int lc[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = 4 * tid + q;
          const int c = icnt[sm.s_item[k < n_sv ? k : (n_sv > 0 ? n_sv - 1 : 0)]];
          lc[q] = k < n_sv ? c : 0;
          sum += lc[q];
        }
        int raw_tot;
        int base = block_exclusive_scan(sum, redi, &raw_tot);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = 4 * tid + q;
          if (k < n_sv) s_pre[k] = base;
          base += lc[q];
        }
        if (tid == 0) s_pre[n_sv] = raw_tot;
        __syncthreads();
        read_rounds(n_sv, raw_tot);
      }
    }
    // otherwise chunks of up to 1024 items, each listing its non-empty items
    // above thr (one scan)
    for (int c0 = 0; !listed && c0 < n_items; c0 += kTauItemChunk) {
      const int nc = min(kTauItemChunk, n_items - c0);
      int lc[4], sum = 0, nz = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = 4 * tid + i;
        const float mx = load_or(imax + c0, jj, nc, -INFINITY);
        const int c = load_or(icnt + c0, jj, nc, 0);
        lc[i] = (double)mx > thr ? c : 0;
        sum += lc[i];
        nz += lc[i] > 0;
      }
      int packed_tot;
      const int packed = block_exclusive_scan((nz << 17) | sum, redi, &packed_tot);
      const int raw_tot = packed_tot & 0x1ffff, n_ne = packed_tot >> 17;
      int base = packed & 0x1ffff, rank = packed >> 17;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (lc[i] > 0) {
          s_pre[rank] = base;
          sm.s_item[rank] = c0 + 4 * tid + i;
          ++rank;
        }
        base += lc[i];
      }
      if (tid == 0) s_pre[n_ne] = raw_tot;
      __syncthreads();
      read_rounds(n_ne, raw_tot);
      __syncthreads();  // s_pre / s_item are rewritten by the next chunk
    }
    if (!done) {
      N = run;
      in_lds = N <= CAP;
      wait_mem();  // this thread's list entries are written before others read them
      __syncthreads();
      if (in_lds)
        for (int i = tid; i < N; i += kTauThreads) { lx[i] = ox[i]; lt[i] = ot[i]; lr[i] = orow[i]; }
    }
  }
  __syncthreads();
  if (in_lds && N > kTauThreads) {
    // Count bound on the candidates themselves.  Bin j holds the candidates
    // with (m - x) 64 in [j, j + 1) (the last bin everything lower); the
    // n_j candidates in bins 0..j lie above m - (j + 1)/64, so, one bin of
    // slack covering the rounding of the bin index, above L_j = m - (j + 2)/64,
    // and tau >= L_j - n_j^-(alpha-1).  The candidates above the best of
    // these bounds are kept, in order; usually few enough for the pairwise
    // test below, where the iterative solve would take a pass per step.
    int* hist = sm.s_pre;  // (free here)
    for (int i = tid; i < 256; i += kTauThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += kTauThreads) {
      const float d = (mf - lx[i]) * 64.f;
      atomicAdd(&hist[d < 255.f ? (int)d : 255], 1);
    }
    __syncthreads();
    const int c = tid < 256 ? hist[tid] : 0;
    int tot;
    const int excl = block_exclusive_scan(c, redi, &tot);
    double bnd = -INFINITY;
    if (tid < 255 && excl + c > 0)
      bnd = (double)(mf - (float)(tid + 2) * (1.f / 64.f)) - count_pow(excl + c, a.alpha);
    bnd = block_max(bnd, redd) - 1e-6 * fmax(1.0, fabs(m));
    if (bnd > thr) {  // block-uniform
      thr = bnd;
      constexpr int EW = CAP / kTauThreads;
      const int E = (N + kTauThreads - 1) / kTauThreads;
      const int e0 = min(tid * E, N), e1 = min(e0 + E, N);
      float xv[EW];
      int tv[EW], rv[EW];
      int kept = 0;
#pragma unroll
      for (int k = 0; k < EW; ++k) {
        xv[k] = -INFINITY;
        tv[k] = rv[k] = 0;
        if (k < E && e0 + k < e1) {
          xv[k] = lx[e0 + k];
          tv[k] = lt[e0 + k];
          rv[k] = lr[e0 + k];
        }
        kept += (double)xv[k] > thr;
      }
      int n2;
      int pos = block_exclusive_scan(kept, redi, &n2);  // every read above is done
#pragma unroll
      for (int k = 0; k < EW; ++k) {
        if ((double)xv[k] > thr) {
          lx[pos] = xv[k];
          lt[pos] = tv[k];
          lr[pos] = rv[k];
          ++pos;
        }
      }
      N = n2;
      __syncthreads();
    }
  }
  float* xs = in_lds ? lx : a.ovf_x + bh * tok_per_bh;
  int32_t* ts = in_lds ? lt : a.ovf_t + bh * tok_per_bh;
  int32_t* rs = in_lds ? lr : a.ovf_r + bh * tok_per_bh;

  // ---- threshold: one wave when the candidates are few, else the block ----
  double tau;
  double& s_tau = sm.s_tau;
  const double beta = 1.0 / ((double)a.alpha - 1.0);
  double ps = 0.0;
  int nsup = 0;
  auto emit = [&](int pos, double p, int tok) {
    if (a.support_idx && pos < a.support_cap) a.support_idx[bh * a.support_cap + pos] = tok;
    if (a.support_p && pos < a.support_cap) a.support_p[bh * a.support_cap + pos] = (float)p;
  };
  // V rows prefetched by waves 1..3 during the single-wave solve: VGR row
  // groups of LPR lanes, VPR rows each (every candidate of the single-wave
  // path at d = 128 in bf16)
  constexpr int VGR = (kTauThreads - kWave) / LPR;
  constexpr int VPR = (kWaveCands + VGR - 1) / VGR < 12 ? (kWaveCands + VGR - 1) / VGR : 12;
  bool vpre = false;
  uint4 vq[VPR];
  if (AK != 2 && in_lds && N >= 1 && N <= kWaveCands) {
    // At most 128 candidates (alpha 2 and 1.5), on chip: wave 0 holds them,
    // candidate l + 64 r in slot r of lane l, and takes the pairwise support
    // test, tau and the weights by itself, with lane exchanges and ballots
    // instead of block barriers.  Same tests and closed forms as the block
    // path, the support in the same (candidate) order.  Meanwhile, when the
    // candidates are few enough, waves 1..3 load every candidate's V row
    // (most are in the support); wave 0 then leaves the list in place and
    // hands over the weights by candidate.  Otherwise waves 1..3 wait at the
    // barrier, and wave 0 compacts the list in place for the usual V sum.
    vpre = N <= VPR * VGR;  // block-uniform
    if (tid_w == 0) {
      constexpr int K = kWaveCands / kWave;
      const int l = tid & 63;
      float xf[K];
      int tk[K], rw[K];
      bool has[K];
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const int i = l + kWave * r;
        has[r] = i < N;
        xf[r] = has[r] ? lx[i] : 0.f;
        tk[r] = has[r] ? lt[i] : 0;
        rw[r] = has[r] ? lr[i] : 0;
      }
      // f(x) = sum_j (x_j - x)_+^e over the candidates in ascending j, the
      // x_j read four at a time with broadcast LDS loads; the second slot
      // only when there are more than 64 candidates
      float ff[K];
#pragma unroll
      for (int r = 0; r < K; ++r) ff[r] = 0.f;
      auto pass = [&](auto nslots) {
        constexpr int KS = decltype(nslots)::value;
        auto acc = [&](float xj) {
#pragma unroll
          for (int r = 0; r < KS; ++r) {
            const float d = fmaxf(xj - xf[r], 0.f);
            ff[r] += AK == 0 ? d : d * d;
          }
        };
        const float4* x4 = reinterpret_cast<const float4*>(lx);
        const int n4 = N >> 2;
#pragma unroll 2
        for (int q = 0; q < n4; ++q) {
          const float4 v = x4[q];
          acc(v.x);
          acc(v.y);
          acc(v.z);
          acc(v.w);
        }
        for (int j = 4 * n4; j < N; ++j) acc(lx[j]);
      };
      if (N > kWave) pass(std::integral_constant<int, K>{});
      else pass(std::integral_constant<int, 1>{});
      double c = 0.0, s1 = 0.0, s2 = 0.0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        if (has[r] && (double)ff[r] < 1.0) {
          const double y = (double)xf[r] - m;
          c += 1.0;
          s1 += y;
          s2 += y * y;
        }
      }
      c = wave_sum(c);
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      tau = support_tau<AK>(c, s1, s2, m);
      double p[K];
      int pos[K], base = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const bool sup = has[r] && (double)xf[r] > tau;
        const uint64_t bal = __ballot(sup);
        pos[r] = sup ? base + __popcll(bal & ((1ull << l) - 1ull)) : -1;
        base += __popcll(bal);
        p[r] = sup ? entmax_pow<AK>((double)xf[r] - tau, beta) : 0.0;
      }
      double pl = 0.0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        pl += p[r];
        if (pos[r] >= 0) emit(pos[r], p[r], tk[r]);
        if (vpre) {
          if (l + kWave * r < N) sm.pc[l + kWave * r] = (float)p[r];
        } else if (pos[r] >= 0) {
          // every lane has read its candidates above, so the list is
          // rewritten in place (p replaces x)
          lx[pos[r]] = (float)p[r];
          lt[pos[r]] = tk[r];
          lr[pos[r]] = rw[r];
        }
      }
      ps = wave_sum(pl);
      if (l == 0) {
        s_tau = tau;
        sm.s_nsup = base;
        sm.s_ps = ps;
      }
    } else if (vpre) {
      // candidate gq + VGR q's row, the lane's 16 bytes of it (the last
      // candidate stands in past the end; lr is not rewritten on this path)
      const int gq = (tid - kWave) / LPR, sub = tid % LPR;
#pragma unroll
      for (int q = 0; q < VPR; ++q) {
        const int row = lr[min(gq + VGR * q, N - 1)];
        const int phys = row >> __builtin_ctz(P), slot = row & (P - 1);  // P is a power of two
        vq[q] = ldg16(reinterpret_cast<const char*>(a.v) +
                      ((((size_t)phys * a.hkv_mem + (g >> a.kv_shift)) * P + slot) * D + (size_t)sub * EPL) * E::kBytes);
      }
    }
    __syncthreads();
    tau = s_tau;
    nsup = sm.s_nsup;
    ps = sm.s_ps;
  } else {  // the block path
  // (other alpha: the pairwise test would take N^2 fp64 powers; Newton's
  // method takes a few passes instead)
  bool pairwise = false;
  if constexpr (AK != 2) {
    if (N <= kTauThreads) {  // (then the list is on chip)
      tau = solve_pairwise<AK>(lx, N, m, redd);
      pairwise = true;
    }
  }
  if (!pairwise) {
    if (N <= 8 * kWave) {
      if (tid_w == 0) {
        tau = solve_threshold<true, AK>(xs, N, m, thr, a.alpha, redd);
        if ((tid & 63) == 0) s_tau = tau;
      }
      __syncthreads();
      tau = s_tau;
    } else {
      tau = solve_threshold<false, AK>(xs, N, m, thr, a.alpha, redd, sm.vpart, 2048);  // vpart is free until the output
    }
  }

  // ---- support, weights, compaction in place (p replaces x) ----
  if (in_lds) {
    // on chip (N <= CAP, at most EW per thread): thread t holds the
    // contiguous candidates [t E, t E + E) in registers, one scan places its
    // kept ones
    constexpr int EW = CAP / kTauThreads;
    static_assert(CAP % kTauThreads == 0, "candidates per thread");
    const int E = (N + kTauThreads - 1) / kTauThreads;
    const int e0 = min(tid * E, N), e1 = min(e0 + E, N);
    float xv[EW];
    int tv[EW], rv[EW];
    int c = 0;
#pragma unroll
    for (int k = 0; k < EW; ++k) {
      xv[k] = -INFINITY;
      tv[k] = rv[k] = 0;
      if (k < E) {  // block-uniform: no read past the slots in use
        const int i = min(e0 + k, CAP - 1);  // in the LDS list; masked below
        xv[k] = xs[i];
        tv[k] = ts[i];
        rv[k] = rs[i];
        if (!(e0 + k < e1)) xv[k] = -INFINITY;
      }
      c += (double)xv[k] > tau;
    }
    int pos = block_exclusive_scan(c, redi, &nsup);  // every read above is done
#pragma unroll
    for (int k = 0; k < EW; ++k) {
      if ((double)xv[k] > tau) {
        if (AK == 2) {
          xs[pos] = xv[k];  // the power is taken below, over the support only
        } else {
          const double p = entmax_pow<AK>((double)xv[k] - tau, beta);
          ps += p;
          xs[pos] = (float)p;
          emit(pos, p, tv[k]);
        }
        ts[pos] = tv[k];
        rs[pos] = rv[k];
        ++pos;
      }
    }
    __syncthreads();
  } else {
    // in the workspace: rounds of kSolveBatch contiguous candidates per
    // thread (loaded at once), one scan per round; a kept candidate moves to
    // a position at or below its own, so no write reaches a later round's
    constexpr int WB = kSolveBatch;
    for (int i0 = 0; i0 < N; i0 += WB * kTauThreads) {
      const int e0 = i0 + WB * tid;
      float xv[WB];
      int tv[WB], rv[WB];
      int c = 0;
#pragma unroll
      for (int k = 0; k < WB; ++k) {
        xv[k] = load_or(xs, e0 + k, N, -INFINITY);
        tv[k] = load_or(ts, e0 + k, N, 0);
        rv[k] = load_or(rs, e0 + k, N, 0);
      }
#pragma unroll
      for (int k = 0; k < WB; ++k) c += (double)xv[k] > tau;
      int tot;
      int pos = nsup + block_exclusive_scan(c, redi, &tot);  // every read of the round is done
#pragma unroll
      for (int k = 0; k < WB; ++k) {
        if ((double)xv[k] > tau) {
          if (AK == 2) {
            xs[pos] = xv[k];  // the power is taken below, over the support only
          } else {
            const double p = entmax_pow<AK>((double)xv[k] - tau, beta);
            ps += p;
            xs[pos] = (float)p;
            emit(pos, p, tv[k]);
          }
          ts[pos] = tv[k];
          rs[pos] = rv[k];
          ++pos;
        }
      }
      nsup += tot;
      wait_mem();  // workspace list entries are read by other threads next
      __syncthreads();
    }
  }
  if (AK == 2) {
    // other alpha: the fp64 powers over the compacted support, every lane
    // busy (p replaces x)
    for (int i = tid; i < nsup; i += kTauThreads) {
      const double p = entmax_pow<AK>((double)xs[i] - tau, beta);
      ps += p;
      xs[i] = (float)p;
      emit(i, p, ts[i]);
    }
    if (!in_lds) wait_mem();  // read by other threads next
    __syncthreads();
  }
  ps = block_sum(ps, redd);
  }  // the block path

  // ---- sum_j p_j v_j ----
  const int rr = tid / LPR, sub = tid % LPR;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  if (vpre) {
    // the rows loaded during the solve, weighted by candidate (0 off the
    // support), in candidate order
    if (tid_w > 0) {
      const int gq = (tid - kWave) / LPR;
#pragma unroll
      for (int q = 0; q < VPR; ++q) {
        const int i = gq + VGR * q;
        if (i < N) {
          const float pw = sm.pc[i];
          float f[EPL];
          E::unpack(vq[q], f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pw, f[e], acc[e]);
        }
      }
    }
  }
  // kVRows rows in flight per thread: every load of a round first (the last
  // row stands in past the end), then the products in row order
  for (int s0 = rr; !vpre && s0 < nsup; s0 += kVRows * RPB) {
    uint4 vv[kVRows];
    float pv[kVRows];
#pragma unroll
    for (int i = 0; i < kVRows; ++i) {
      const int s = min(s0 + i * RPB, nsup - 1);
      const int row = rs[s];
      pv[i] = xs[s];
      const int phys = row >> __builtin_ctz(P), slot = row & (P - 1);  // P is a power of two
      const char* vrow = reinterpret_cast<const char*>(a.v) +
                         ((((size_t)phys * a.hkv_mem + (g >> a.kv_shift)) * P + slot) * D + (size_t)sub * EPL) * E::kBytes;
      vv[i] = ldg16(vrow);
    }
#pragma unroll
    for (int i = 0; i < kVRows; ++i) {
      if (s0 + i * RPB < nsup) {
        float f[EPL];
        E::unpack(vv[i], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pv[i], f[e], acc[e]);
      }
    }
  }
  // the wave's row groups (lanes sub, sub + LPR, ...) by lane exchanges,
  // then the four waves' partials in order
#pragma unroll
  for (int mask = LPR; mask < kWave; mask <<= 1)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], mask, kWave);
  constexpr int NWV = kTauThreads / kWave;
  static_assert(NWV * D <= 2048, "vpart");
  if ((tid & 63) < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm.vpart[tid_w * D + sub * EPL + e] = acc[e];
  }
  __syncthreads();
  for (int e = tid; e < D; e += blockDim.x) {
    float o = sm.vpart[e];
#pragma unroll
    for (int w2 = 1; w2 < NWV; ++w2) o += sm.vpart[w2 * D + e];
    out[e] = o;
  }
  if (tid == 0) {
    if (a.tau) a.tau[bh] = (float)tau;
    if (a.support_count) a.support_count[bh] = nsup;
    if (a.psum) a.psum[bh] = (float)ps;
  }
}

template <int DT, int D, int AK, int CAP>
__global__ __launch_bounds__(kTauThreads) void tau_v_kernel(DecodeArgs a) {
  __shared__ TauSmem<CAP> sm;
  tau_v_block<DT, D, AK, CAP>(a, blockIdx.y, blockIdx.x, sm);
}

// The balanced gather's grid: as many blocks as can be resident at once
// (blocks per compute unit from the runtime's occupancy query for this
// instance), so that no block waits for a second round; at most `cap`.
template <auto Kernel>  // one cached query per kernel instance
static int resident_grid(int cus, int cap) {
  static const int per_cu = [] {
    int n = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Kernel, kDecThreads, 0) == hipSuccess ? n : 0;
  }();
  return per_cu > 0 ? (per_cu * cus < cap ? per_cu * cus : cap) : cap;
}


template <int DT, int D>
static hipError_t decode_dispatch(const DecodeArgs& a, int slots, int bal_blocks, int cus, hipStream_t s) {
  const dim3 g1(slots, a.batch * a.n_kv_heads), b1(kDecThreads);
  const bool mfma = DT == EKV_BF16;
  const bool lvl = a.max_items > kTauFewItems;  // some unit may have that many items
  if (mfma && bal_blocks > 0) {
#define EKV_BAL1(GG, LV)                                                                          \
  hipLaunchKernelGGL((gather_mfma_kernel<D, GG, 4, true, LV>),                                    \
                     dim3(resident_grid<gather_mfma_kernel<D, GG, 4, true, LV>>(cus, bal_blocks)), b1, 0, s, a, 0)
#define EKV_BAL(GG) \
  if (lvl) EKV_BAL1(GG, true); else EKV_BAL1(GG, false)
    switch (a.group) {
      case 1: EKV_BAL(1); break;
      case 2: EKV_BAL(2); break;
      case 4: EKV_BAL(4); break;
      default: EKV_BAL(8); break;
    }
#undef EKV_BAL
#undef EKV_BAL1
  } else if (mfma) {
#define EKV_G(GG)                                                                                  \
  if (lvl) hipLaunchKernelGGL((gather_mfma_kernel<D, GG, 4, false, true>), g1, b1, 0, s, a, slots); \
  else hipLaunchKernelGGL((gather_mfma_kernel<D, GG, 4, false, false>), g1, b1, 0, s, a, slots)
    switch (a.group) {
      case 1: EKV_G(1); break;
      case 2: EKV_G(2); break;
      case 4: EKV_G(4); break;
      default: EKV_G(8); break;
    }
#undef EKV_G
  } else {
    switch (a.group) {
      case 1: hipLaunchKernelGGL((gather_valu_kernel<DT, D, 1>), g1, b1, 0, s, a, slots); break;
      case 2: hipLaunchKernelGGL((gather_valu_kernel<DT, D, 2>), g1, b1, 0, s, a, slots); break;
      case 4: hipLaunchKernelGGL((gather_valu_kernel<DT, D, 4>), g1, b1, 0, s, a, slots); break;
      case 8: hipLaunchKernelGGL((gather_valu_kernel<DT, D, 8>), g1, b1, 0, s, a, slots); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2(a.n_q_heads, a.batch), b2(kTauThreads);
  if (a.alpha == 2.0f) hipLaunchKernelGGL((tau_v_kernel<DT, D, 0, kLdsCands>), g2, b2, 0, s, a);
  else if (a.alpha == 1.5f) hipLaunchKernelGGL((tau_v_kernel<DT, D, 1, kLdsCands>), g2, b2, 0, s, a);
  // other alpha (supports of hundreds of tokens, thousands of candidates):
  // the larger list when every (sequence, query head) block has a compute
  // unit of its own, where it costs no occupancy (it costs about 2 us per
  // block in the weights and output phases, which the smaller supports of
  // alpha 1.5 and 2 do not win back)
  else if ((long long)a.batch * a.n_q_heads <= cus)
    hipLaunchKernelGGL((tau_v_kernel<DT, D, 2, kLdsCandsBig>), g2, b2, 0, s, a);
  else hipLaunchKernelGGL((tau_v_kernel<DT, D, 2, kLdsCands>), g2, b2, 0, s, a);
  return hipGetLastError();
}

// Gather grid: (slots, units).  A unit has at most `items` 64-token items
// (the largest possible selection); on the matrix-core path items are
// grouped into super-items of four (more loads in flight per block).  slots
// is chosen so the grid holds about `target_blocks` blocks, and never
// exceeds the work.  With 64 to 512 units on the matrix-core path the
// `target_blocks` blocks instead share all units' super-items evenly (the
// balanced assignment above): selections differ in size between units, and
// a fixed number of blocks per unit would wait for the largest.
hipError_t launch_decode(const DecodeArgs& a, int target_blocks, hipStream_t s) {
  const long long pages = a.sel ? (a.cap < a.max_pages ? a.cap : a.max_pages) : a.max_pages;
  const long long items = (pages * a.page_size + kItemTokens - 1) / kItemTokens;
  const bool mfma = a.kv_dtype == EKV_BF16;
  const int sub = mfma ? 4 : 1;
  const long long supers = (items + sub - 1) / sub;
  const int units = a.batch * a.n_kv_heads;
  long long slots = (target_blocks + units - 1) / units;
  if (slots > supers) slots = supers;
  if (slots < 1) slots = 1;
  if (slots > 65535) slots = 65535;
  const int bal = mfma && units >= 64 && units <= 512 ? target_blocks : 0;
  const int cus = target_blocks / 4;  // target_blocks: four per compute unit
  if (a.kv_dtype == EKV_BF16)
    return a.head_dim == 128 ? decode_dispatch<EKV_BF16, 128>(a, (int)slots, bal, cus, s)
                             : decode_dispatch<EKV_BF16, 64>(a, (int)slots, bal, cus, s);
  return a.head_dim == 128 ? decode_dispatch<EKV_F32, 128>(a, (int)slots, 0, cus, s)
                           : decode_dispatch<EKV_F32, 64>(a, (int)slots, 0, cus, s);
}

// ---------------------------------------------------------------------------
// Softmax attention decode, the comparison the EntmaxKV summary draws
// (sec. 1 and 3): z = scale q.k over the same page list (selected pages, or
// the whole cache), p = softmax(z) renormalised over that set, o = sum p v.
// Flash-decode split over the page list: block (slot, unit) scores its
// super-items on the matrix cores (as the gather does, coefficient scale q),
// keeps a running maximum M and sum l of exp(z - M) per head, stages the
// super-item's V rows in LDS and accumulates sum exp(z - M) v; a combine
// kernel merges the blocks' (M, l, acc) per head in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kSmxSub = 2;  // items (of 64 tokens) per softmax super-item

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void softmax_part_kernel(DecodeArgs a, int slots, float* part) {
  constexpr int SUB = kSmxSub;
  constexpr int KB = D / 32;
  constexpr int CH = D / 8;                   // 16-byte chunks per V row
  constexpr int QT = kDecThreads / (4 * CH);  // token groups of the accumulation
  constexpr int TT = SUB * kItemTokens;       // tokens per super-item
  static_assert(4 * CH * QT == kDecThreads, "thread layout");
  __shared__ u32x4_t s_a[KB][kWave];
  __shared__ float s_max[SUB][4][4];
  __shared__ float s_sum[4][4];
  __shared__ float s_e[4][TT];
  // the V tile; after the last tile it holds the token groups' sums
  __shared__ uint4 s_v[TT][CH];
  static_assert(sizeof(float) * QT * 4 * D <= sizeof(uint4) * TT * CH, "accumulator alias");
  float (*s_acc)[4][D] = reinterpret_cast<float (*)[4][D]>(&s_v[0][0]);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int u = blockIdx.y, Hkv = a.n_kv_heads, P = a.page_size;
  const int b = u / Hkv, g = u - b * Hkv;
  const int r = 16 * w + col;  // this lane's token within an item
  // accumulation layout: thread = (token group tq, head ha, 16-byte chunk ca)
  const int ca = tid % CH, ha = (tid / CH) % 4, tq = tid / (4 * CH);

  const float* qg = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * D;
  LimbChunks<KB> lc;
  limb_fetch<KB, G>(lc, [&](int h, int k0, float* v) {
    const float4* qv = reinterpret_cast<const float4*>(qg + (size_t)h * D + k0);
    const float4 q0 = qv[0], q1 = qv[1];
    v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w; v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  });
  UnitCtx ctx;
  TokenRef tr[SUB];
  resolve_refs<SUB>(a, u, b, blockIdx.x * SUB, r, true, &ctx, tr);
  const float sc = a.scale;
  limb_build<KB, G>(s_a, lc, [sc](int, float qv) { return qv * sc; });
  __syncthreads();

  // running maximum of head grp (score lanes) and of head ha (accumulating
  // threads): the same recurrence over the same values, so equal per head
  float Mg = -INFINITY, M = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const int n_super = (ctx.n_items + SUB - 1) / SUB;
  for (int sj = blockIdx.x; sj < n_super; sj += slots) {
    if (sj != (int)blockIdx.x) resolve_refs<SUB>(a, u, b, sj * SUB, r, false, &ctx, tr);
    // K and V rows of the lane's tokens: 4 x 16 bytes each per item
    u32x4_t bv[SUB][KB];
    uint4 vv[SUB][KB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      if (tr[s].phys >= 0) {
        const size_t rowi = (((size_t)tr[s].phys * a.hkv_mem + (g >> a.kv_shift)) * P + tr[s].slot) * D + 8 * grp;
        const uint16_t* krow = reinterpret_cast<const uint16_t*>(a.k) + rowi;
        const uint16_t* vrow = reinterpret_cast<const uint16_t*>(a.v) + rowi;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bv[s][kb] = *reinterpret_cast<const u32x4_t*>(krow + 32 * kb);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) vv[s][kb] = tr[s].valid ? ldg16(vrow + 32 * kb) : make_uint4(0u, 0u, 0u, 0u);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          bv[s][kb] = u32x4_t{0u, 0u, 0u, 0u};
          vv[s][kb] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    float z[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) c = mfma_bf16(s_a[kb][lane], bv[s][kb], c);
      z[s] = tr[s].valid && grp < G ? (c[0] + c[1]) + c[2] : -INFINITY;
      const float m = group_reduce<16>(z[s], [](float x, float y) { return fmaxf(x, y); });
      if (col == 0) s_max[s][w][grp] = m;
      // V chunk kb of this lane's token covers columns 8 grp + 32 kb .. + 8
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s_v[s * kItemTokens + r][grp + 4 * kb] = vv[s][kb];
    }
    __syncthreads();
    auto new_max = [&](int h, float mold) {
      float mm = mold;
#pragma unroll
      for (int s = 0; s < SUB; ++s)
        mm = fmaxf(mm, fmaxf(fmaxf(s_max[s][0][h], s_max[s][1][h]), fmaxf(s_max[s][2][h], s_max[s][3][h])));
      return mm;
    };
    const float mg = new_max(grp, Mg);
    float esum = 0.f;
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      const float e = (grp < G && mg > -INFINITY) ? __expf(z[s] - mg) : 0.f;
      esum += e;
      s_e[grp][s * kItemTokens + r] = e;
    }
    Mg = mg;
    esum = group_reduce<16>(esum, [](float x, float y) { return x + y; });
    if (col == 0) s_sum[w][grp] = esum;
    __syncthreads();
    // head ha: rescale the running sums to the new maximum, add this tile
    const float mn = new_max(ha, M);
    const float cs = M > -INFINITY ? __expf(M - mn) : 0.f;
    l = l * cs + ((s_sum[0][ha] + s_sum[1][ha]) + (s_sum[2][ha] + s_sum[3][ha]));
    M = mn;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= cs;
    if (ha < G) {
      for (int tok = tq; tok < TT; tok += QT) {
        const float e = s_e[ha][tok];
        float f[8];
        Elem<EKV_BF16>::unpack(s_v[tok][ca], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(e, f[j], acc[j]);
      }
    }
    __syncthreads();  // s_max, s_e, s_v and s_sum are rewritten next
  }
  // combine the token groups; write this block's (M, l, acc) per head
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) s_acc[tq][ha][ca * 8 + j] = acc[j];
  __syncthreads();
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int h = i / D, d = i - h * D;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < QT; ++t) sum += s_acc[t][h][d];
    const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + h;
    part[(bh * slots + blockIdx.x) * (D + 2) + 2 + d] = sum;
  }
  if (tq == 0 && ca == 0 && ha < G) {
    const size_t bh = (size_t)b * a.n_q_heads + (size_t)g * G + ha;
    float* pp = part + (bh * slots + blockIdx.x) * (D + 2);
    pp[0] = M;
    pp[1] = l;
  }
}

// One block per (sequence, query head): o = sum_i e^{M_i - M} acc_i / L,
// L = sum_i e^{M_i - M} l_i, lse = M + log L.  The blocks' maxima and sums
// are read in one round; then thread (column d, slot group sg) sums its
// slots sixteen loads at a time, and the groups are added in order.
constexpr int kSmxCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kSmxCombineThreads) void softmax_combine_kernel(DecodeArgs a, int slots,
                                                                             const float* part, float* lse) {
  constexpr int NG = kSmxCombineThreads / D;
  __shared__ float s_c[kSmxMaxSlots];
  __shared__ float s_o[NG][D];
  __shared__ float red[16];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = tid % D, sg = tid / D;
  const size_t bh = (size_t)b * a.n_q_heads + h;
  const float* pp = part + bh * slots * (D + 2);
  const bool has = tid < slots;
  const float mi = has ? pp[(size_t)tid * (D + 2)] : -INFINITY;
  const float li = has ? pp[(size_t)tid * (D + 2) + 1] : 0.f;
  const float M = block_max(mi, red);
  const float c = (M > -INFINITY && mi > -INFINITY) ? __expf(mi - M) : 0.f;
  if (has) s_c[tid] = c;
  const float L = block_sum(c * li, red);  // block_sum's barriers also publish s_c
  float o = 0.f;
  for (int i0 = sg; i0 < slots; i0 += 16 * NG) {
    float v[16], w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * NG;
      v[u] = i < slots ? pp[(size_t)i * (D + 2) + 2 + d] : 0.f;
      w[u] = i < slots ? s_c[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) o = fmaf(w[u], v[u], o);
  }
  s_o[sg][d] = o;
  __syncthreads();
  if (sg == 0) {
    float t = s_o[0][d];
#pragma unroll
    for (int j = 1; j < NG; ++j) t += s_o[j][d];
    a.out[bh * D + d] = L > 0.f ? t / L : 0.f;
    if (d == 0 && lse) lse[bh] = L > 0.f ? M + logf(L) : -INFINITY;
  }
}

hipError_t launch_softmax(const DecodeArgs& a, int target_blocks, float* part, int max_slots, float* lse,
                          hipStream_t s) {
  const long long pages = a.sel ? (a.cap < a.max_pages ? a.cap : a.max_pages) : a.max_pages;
  const long long items = (pages * a.page_size + kItemTokens - 1) / kItemTokens;
  const long long supers = (items + kSmxSub - 1) / kSmxSub;
  const int units = a.batch * a.n_kv_heads;
  long long slots = (target_blocks + units - 1) / units;
  if (slots > supers) slots = supers;
  if (slots > max_slots) slots = max_slots;
  if (slots < 1) slots = 1;
  const dim3 g1((unsigned)slots, units), b1(kDecThreads);
#define EKV_SMX(DD, GG) hipLaunchKernelGGL((softmax_part_kernel<DD, GG>), g1, b1, 0, s, a, (int)slots, part)
  if (a.head_dim == 128) {
    if (a.group == 1) EKV_SMX(128, 1); else if (a.group == 2) EKV_SMX(128, 2); else EKV_SMX(128, 4);
  } else {
    if (a.group == 1) EKV_SMX(64, 1); else if (a.group == 2) EKV_SMX(64, 2); else EKV_SMX(64, 4);
  }
#undef EKV_SMX
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2(a.n_q_heads, a.batch);
  static_assert(kSmxMaxSlots <= kSmxCombineThreads, "one block maximum per combine thread");
  if (a.head_dim == 128)
    hipLaunchKernelGGL((softmax_combine_kernel<128>), g2, dim3(kSmxCombineThreads), 0, s, a, (int)slots, part, lse);
  else
    hipLaunchKernelGGL((softmax_combine_kernel<64>), g2, dim3(kSmxCombineThreads), 0, s, a, (int)slots, part, lse);
  return hipGetLastError();
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
