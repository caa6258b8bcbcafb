// extern "C" entry points: host-side validation, workspace carving and
// launches.  Nothing here allocates device memory; every argument problem is
// reported before the first HIP call.
#include <math.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "ekv_kernels.h"

// Fixed device scratch of ekv_entmax_decode_noalloc: every device the
// library runs on holds one copy, for the life of the process.  Host code
// never uses the name as an address: the per-device address comes from
// hipGetSymbolAddress (static_scratch below).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

ekv_status fail(ekv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ekv_status check_cache(const ekv_cache* c) {
  if (!c) return fail(EKV_ERR_INVALID_ARG, "cache is NULL");
  if (c->n_phys_pages <= 0) return fail(EKV_ERR_INVALID_ARG, "n_phys_pages must be > 0");
  if (c->n_kv_heads <= 0) return fail(EKV_ERR_INVALID_ARG, "n_kv_heads must be > 0");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(EKV_ERR_INVALID_ARG, "head_dim must be 64 or 128");
  const int P = c->page_size;
  if (P < 1 || P > 1024 || (P & (P - 1)) != 0)
    return fail(EKV_ERR_INVALID_ARG, "page_size must be a power of two in [1, 1024]");
  if (c->kv_dtype != EKV_F32 && c->kv_dtype != EKV_BF16) return fail(EKV_ERR_INVALID_ARG, "kv_dtype must be EKV_F32 or EKV_BF16");
  if (!c->k || !c->v) return fail(EKV_ERR_INVALID_ARG, "cache k/v pointer is NULL");
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->k_box) || !aligned16(c->k_moments))
    return fail(EKV_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
  const double elems = (double)c->n_phys_pages * c->n_kv_heads * P * c->head_dim;
  if (elems >= 9.0e18) return fail(EKV_ERR_INVALID_ARG, "cache too large");
  return EKV_OK;
}

ekv_status check_seqs(const ekv_cache* c, const ekv_seqs* s) {
  if (!s) return fail(EKV_ERR_INVALID_ARG, "seqs is NULL");
  if (s->batch <= 0) return fail(EKV_ERR_INVALID_ARG, "batch must be > 0");
  if (s->max_pages <= 0) return fail(EKV_ERR_INVALID_ARG, "max_pages must be > 0");
  if (!s->page_table || !s->seq_lens) return fail(EKV_ERR_INVALID_ARG, "page_table/seq_lens is NULL");
  if ((long long)s->max_pages * c->page_size > 0x7fffffffLL)
    return fail(EKV_ERR_INVALID_ARG, "max_pages * page_size must fit in int32");
  if ((long long)s->batch * c->n_kv_heads > ekv::kMaxUnits)
    return fail(EKV_ERR_UNSUPPORTED, "batch * n_kv_heads above 4096");
  return EKV_OK;
}

ekv_status check_heads(const ekv_cache* c, int32_t n_q_heads, int* group) {
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
    return fail(EKV_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(EKV_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8");
  *group = G;
  return EKV_OK;
}

// Pages of the longest list a decode with capacity `cap` reads (cap <= 0:
// the whole cache).
int list_pages(const ekv_seqs* s, int32_t cap) { return cap > 0 && cap < s->max_pages ? cap : s->max_pages; }

// Workspace layout for decodes of lists of up to item_pages pages; a call
// that uses no per-item region (selection, scoring, softmax decode) needs
// only the part before them.
ekv_status check_ws(const ekv_cache* c, const ekv_seqs* s, int32_t n_q_heads, void* ws, size_t ws_bytes,
                    int item_pages, bool items, ekv::Layout* L) {
  *L = ekv::make_layout(s->batch, c->n_kv_heads, n_q_heads, s->max_pages, c->page_size, c->head_dim, item_pages);
  if (!ws) return fail(EKV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(ws)) return fail(EKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const size_t need = items ? L->total : L->item_cnt;
  if (ws_bytes < need)
    return fail(EKV_ERR_WORKSPACE, "workspace holds " + std::to_string(ws_bytes) + " bytes, needs " +
                                       std::to_string(need) +
                                       (items ? " (size it with this call's cap, or 0 for full-cache decodes)" : ""));
  return EKV_OK;
}

template <typename T> T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

ekv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return EKV_OK;
  return fail(EKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// The same arguments seen as one selection unit per (sequence, query head):
// group 1, unit head h reads the cache records of KV head h / G.
template <typename Args> Args per_query_head_view(const Args& a) {
  Args u = a;
  int shift = 0;
  while ((1 << shift) < a.group) ++shift;
  u.n_kv_heads = a.n_q_heads;
  u.group = 1;
  u.kv_shift = shift;
  return u;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

ekv_status static_scratch(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(EKV_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return EKV_OK;
}

}  // namespace

extern "C" {

size_t ekv_workspace_size(const ekv_cache* cache, const ekv_seqs* seqs, int32_t n_q_heads, int32_t cap) {
  int G = 0;
  if (check_cache(cache) != EKV_OK || check_seqs(cache, seqs) != EKV_OK ||
      check_heads(cache, n_q_heads, &G) != EKV_OK)
    return 0;
  return ekv::make_layout(seqs->batch, cache->n_kv_heads, n_q_heads, seqs->max_pages, cache->page_size,
                          cache->head_dim, list_pages(seqs, cap)).total;
}

ekv_status ekv_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || ws_bytes == 0) return fail(EKV_ERR_WORKSPACE, "workspace is NULL or empty");
  if (!aligned16(workspace) || ws_bytes % 16 != 0)
    return fail(EKV_ERR_WORKSPACE, "workspace must be 16-byte aligned with a size that is a multiple of 16");
  return hip_status(ekv::launch_fill_zero(workspace, ws_bytes, (hipStream_t)stream), "workspace init");
}

ekv_status ekv_append_kv(const ekv_cache* cache, const ekv_seqs* seqs, const void* k_new, const void* v_new,
                         int32_t n_new, void* workspace, size_t ws_bytes, void* stream) {
  ekv_status st;
  if ((st = check_cache(cache)) != EKV_OK) return st;
  if ((st = check_seqs(cache, seqs)) != EKV_OK) return st;
  if (n_new < 0) return fail(EKV_ERR_INVALID_ARG, "n_new must be >= 0");
  if (n_new > 0 && (!k_new || !v_new)) return fail(EKV_ERR_INVALID_ARG, "k_new/v_new is NULL");
  if (n_new > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(EKV_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  if ((long long)n_new > (long long)seqs->max_pages * cache->page_size)
    return fail(EKV_ERR_INVALID_ARG, "n_new exceeds max_pages * page_size");
  // append only touches the status word at the start of the workspace
  if (!workspace || ws_bytes < 256 || !aligned16(workspace))
    return fail(EKV_ERR_WORKSPACE, "workspace is NULL, unaligned or smaller than 256 bytes");
  if (n_new == 0) return EKV_OK;
  ekv::AppendArgs a{};
  a.batch = seqs->batch; a.n_kv_heads = cache->n_kv_heads; a.page_size = cache->page_size;
  a.head_dim = cache->head_dim; a.kv_dtype = cache->kv_dtype; a.max_pages = seqs->max_pages;
  a.n_phys = cache->n_phys_pages; a.n_new = n_new;
  a.page_table = seqs->page_table; a.seq_lens = seqs->seq_lens;
  a.k = cache->k; a.v = cache->v; a.k_box = cache->k_box; a.k_moments = cache->k_moments;
  a.k_new = k_new; a.v_new = v_new;
  a.status = at<uint32_t>(workspace, 0);
  return hip_status(ekv::launch_append(a, (hipStream_t)stream), "append_kv launch");
}

static ekv_status prepare_select(const ekv_cache* cache, const ekv_seqs* seqs, const float* q, int32_t n_q_heads,
                                 const ekv_select_params* p, void* workspace, size_t ws_bytes,
                                 ekv::SelectArgs* a, ekv::Layout* L) {
  ekv_status st;
  int G = 0;
  if ((st = check_cache(cache)) != EKV_OK) return st;
  if ((st = check_seqs(cache, seqs)) != EKV_OK) return st;
  if ((st = check_heads(cache, n_q_heads, &G)) != EKV_OK) return st;
  if (!q || !aligned16(q)) return fail(EKV_ERR_INVALID_ARG, "q is NULL or not 16-byte aligned");
  if (!p) return fail(EKV_ERR_INVALID_ARG, "params is NULL");
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return fail(EKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (p->policy == EKV_SELECT_BBOX_TOPK) {
    if (!cache->k_box) return fail(EKV_ERR_INVALID_ARG, "bounding-box selection needs cache->k_box");
    if (p->top_k < 1) return fail(EKV_ERR_INVALID_ARG, "top_k must be >= 1");
    if (seqs->max_pages > 65535) return fail(EKV_ERR_UNSUPPORTED, "top-k selection supports up to 65535 pages per sequence");
  } else if (p->policy == EKV_SELECT_GAUSS) {
    if (!cache->k_moments) return fail(EKV_ERR_INVALID_ARG, "Gaussian selection needs cache->k_moments");
    if (!(p->alpha >= 1.1f && p->alpha <= 2.0f))
      return fail(EKV_ERR_UNSUPPORTED, "Gaussian selection supports alpha in [1.1, 2]");
    if (!(p->delta >= 0.f) || !isfinite(p->delta)) return fail(EKV_ERR_INVALID_ARG, "delta must be finite and >= 0");
    if (p->min_pages < 1) return fail(EKV_ERR_INVALID_ARG, "min_pages must be >= 1");
    if (p->min_pages > 1 && seqs->max_pages > 65535)
      return fail(EKV_ERR_UNSUPPORTED, "min_pages > 1 supports up to 65535 pages per sequence");
  } else {
    return fail(EKV_ERR_INVALID_ARG, "unknown selection policy");
  }
  if (!(p->alpha > 1.f) || !isfinite(p->alpha)) return fail(EKV_ERR_INVALID_ARG, "alpha must be finite and > 1");
  if (p->per_head != 0 && p->per_head != 1) return fail(EKV_ERR_INVALID_ARG, "per_head must be 0 or 1");
  if (p->per_head && (long long)seqs->batch * n_q_heads > ekv::kMaxUnits)
    return fail(EKV_ERR_UNSUPPORTED, "per-query-head selection needs batch * n_q_heads <= 4096");
  if ((st = check_ws(cache, seqs, n_q_heads, workspace, ws_bytes, 1, false, L)) != EKV_OK) return st;
  *a = ekv::SelectArgs{};
  a->batch = seqs->batch; a->n_kv_heads = cache->n_kv_heads; a->n_q_heads = n_q_heads; a->group = G;
  a->hkv_mem = cache->n_kv_heads; a->kv_shift = 0; a->per_head_scores = 0;
  a->page_size = cache->page_size; a->head_dim = cache->head_dim; a->kv_dtype = cache->kv_dtype;
  a->max_pages = seqs->max_pages; a->n_phys = cache->n_phys_pages;
  a->page_table = seqs->page_table; a->seq_lens = seqs->seq_lens;
  a->k_box = cache->k_box; a->k_moments = cache->k_moments; a->q = q;
  a->policy = p->policy; a->top_k = p->top_k; a->min_pages = p->min_pages;
  a->alpha = p->alpha; a->scale = p->scale; a->delta = p->delta;
  a->scores = at<float>(workspace, L->scores);
  a->score_stride = ekv::score_stride(seqs->max_pages);
  a->musd = at<float2>(workspace, L->musd);
  a->ehat = at<float>(workspace, L->ehat);
  a->stats_out = nullptr;
  a->tau_hat = at<double>(workspace, L->tau_hat);
  a->keep_bits = at<uint64_t>(workspace, L->keep_bits);
  a->keep_words = ekv::keep_words(a->max_pages);
  a->done = at<uint32_t>(workspace, L->sel_done);
  a->status = at<uint32_t>(workspace, L->status);
  return EKV_OK;
}

ekv_status ekv_select_pages(const ekv_cache* cache, const ekv_seqs* seqs, const float* q, int32_t n_q_heads,
                            const ekv_select_params* params, int32_t* sel, int32_t* sel_count, int32_t cap,
                            float* tau_hat, void* workspace, size_t ws_bytes, void* stream) {
  ekv::SelectArgs a;
  ekv::Layout L;
  ekv_status st = prepare_select(cache, seqs, q, n_q_heads, params, workspace, ws_bytes, &a, &L);
  if (st != EKV_OK) return st;
  if (!sel || !sel_count) return fail(EKV_ERR_INVALID_ARG, "sel/sel_count is NULL");
  if (cap < 1) return fail(EKV_ERR_INVALID_ARG, "cap must be >= 1");
  if (params->policy == EKV_SELECT_BBOX_TOPK && cap < params->top_k)
    return fail(EKV_ERR_CAPACITY, "cap must be >= top_k");
  if (params->policy == EKV_SELECT_GAUSS && cap < seqs->max_pages)
    return fail(EKV_ERR_CAPACITY, "Gaussian selection needs cap >= max_pages");
  a.sel = sel; a.sel_count = sel_count; a.cap = cap; a.tau_hat_out = tau_hat;
  hipStream_t s = (hipStream_t)stream;
  // Scoring reads each page record once per KV head in both modes; per
  // query head, the bound is written per head and the top-k, threshold
  // estimate and keep test run on (sequence, query head) units.
  const bool per_head = params->per_head && a.group > 1;
  if (!per_head) {  // room for the scoring blocks' top-k candidate lists; the launchers decide whether to use them
    a.cand = at<uint64_t>(workspace, L.cand);
    a.cand_cut = at<uint32_t>(workspace, L.cand_cut);
  }
  const ekv::SelectArgs u = per_head ? per_query_head_view(a) : a;
  if (params->policy == EKV_SELECT_BBOX_TOPK) {
    a.per_head_scores = per_head;
    if ((st = hip_status(ekv::launch_score_bbox(a, s), "score_bbox launch")) != EKV_OK) return st;
    return hip_status(ekv::launch_topk(u, s), "topk launch");
  }
  if ((st = hip_status(ekv::launch_score_gauss(a, s), "score_gauss launch")) != EKV_OK) return st;
  if ((st = hip_status(ekv::launch_tau_hat(u, s), "tau_hat launch")) != EKV_OK) return st;
  if (params->min_pages > 1) return hip_status(ekv::launch_gauss_floor(u, s), "gauss_floor launch");
  return EKV_OK;
}

ekv_status ekv_score_pages(const ekv_cache* cache, const ekv_seqs* seqs, const float* q, int32_t n_q_heads,
                           const ekv_select_params* params, float* scores, void* workspace, size_t ws_bytes,
                           void* stream) {
  ekv::SelectArgs a;
  ekv::Layout L;
  ekv_status st = prepare_select(cache, seqs, q, n_q_heads, params, workspace, ws_bytes, &a, &L);
  if (st != EKV_OK) return st;
  if (!scores || !aligned16(scores)) return fail(EKV_ERR_INVALID_ARG, "scores is NULL or not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (params->policy == EKV_SELECT_BBOX_TOPK) {
    a.scores = scores;
    a.score_stride = seqs->max_pages;
    a.per_head_scores = params->per_head && a.group > 1;
    return hip_status(ekv::launch_score_bbox(a, s), "score_bbox launch");
  }
  a.stats_out = reinterpret_cast<float4*>(scores);
  return hip_status(ekv::launch_score_gauss(a, s), "score_gauss launch");
}

// Validation and argument packing shared by the decode entry points (the
// workspace-dependent fields are filled in by the caller).
ekv_status prepare_decode(const ekv_cache* cache, const ekv_seqs* seqs, const float* q, int32_t n_q_heads,
                          float alpha, float scale, const int32_t* sel, const int32_t* sel_count, int32_t cap,
                          int32_t sel_heads, float* out, ekv::DecodeArgs* a) {
  ekv_status st;
  int G = 0;
  if ((st = check_cache(cache)) != EKV_OK) return st;
  if ((st = check_seqs(cache, seqs)) != EKV_OK) return st;
  if ((st = check_heads(cache, n_q_heads, &G)) != EKV_OK) return st;
  if (!q || !aligned16(q)) return fail(EKV_ERR_INVALID_ARG, "q is NULL or not 16-byte aligned");
  if (!out || !aligned16(out)) return fail(EKV_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  if (!(alpha > 1.f) || !isfinite(alpha)) return fail(EKV_ERR_INVALID_ARG, "alpha must be finite and > 1");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(EKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (sel && (!sel_count || cap < 1)) return fail(EKV_ERR_INVALID_ARG, "sel needs sel_count and cap >= 1");
  if (sel && sel_heads != cache->n_kv_heads && sel_heads != n_q_heads)
    return fail(EKV_ERR_INVALID_ARG, "sel_heads must be n_kv_heads or n_q_heads");
  const bool per_head = sel && sel_heads == n_q_heads && G > 1;
  if (per_head && (long long)seqs->batch * n_q_heads > ekv::kMaxUnits)
    return fail(EKV_ERR_UNSUPPORTED, "per-query-head page lists need batch * n_q_heads <= 4096");
  *a = ekv::DecodeArgs{};
  a->batch = seqs->batch; a->n_kv_heads = cache->n_kv_heads; a->n_q_heads = n_q_heads; a->group = G;
  a->hkv_mem = cache->n_kv_heads; a->kv_shift = 0; a->sel_shift = 0;
  a->page_size = cache->page_size; a->head_dim = cache->head_dim; a->kv_dtype = cache->kv_dtype;
  a->max_pages = seqs->max_pages; a->n_phys = cache->n_phys_pages;
  a->page_table = seqs->page_table; a->seq_lens = seqs->seq_lens;
  a->k = cache->k; a->v = cache->v; a->q = q; a->alpha = alpha; a->scale = scale;
  a->sel = sel; a->sel_count = sel_count; a->cap = sel ? cap : 0;
  a->out = out;
  if (per_head) *a = per_query_head_view(*a);
  return EKV_OK;
}

// The optional outputs of an entmax decode.
ekv_status decode_outputs(ekv::DecodeArgs* a, float* tau, int32_t* support_count, float* psum, int32_t* support_idx,
                          float* support_p, int32_t support_cap) {
  if ((support_idx || support_p) && support_cap < 1)
    return fail(EKV_ERR_INVALID_ARG, "support_idx/support_p need support_cap >= 1");
  a->tau = tau; a->support_count = support_count; a->psum = psum;
  a->support_idx = support_idx; a->support_p = support_p; a->support_cap = support_cap;
  return EKV_OK;
}

// The per-item regions of layout L inside the buffer at `base`.
void decode_regions(ekv::DecodeArgs* a, void* base, const ekv::Layout& L) {
  a->max_items = (int)L.max_items;
  a->item_cnt = at<int32_t>(base, L.item_cnt);
  a->item_max = at<float>(base, L.item_max);
  a->item_lb = at<float>(base, L.item_lb);
  a->item_lvl = at<uint32_t>(base, L.item_lvl);
  a->cand_x = at<float>(base, L.cand_x);
  a->cand_t = at<int32_t>(base, L.cand_t);
  a->cand_r = at<int32_t>(base, L.cand_r);
  a->ovf_x = at<float>(base, L.ovf_x);
  a->ovf_t = at<int32_t>(base, L.ovf_t);
  a->ovf_r = at<int32_t>(base, L.ovf_r);
}

ekv_status ekv_entmax_decode(const ekv_cache* cache, const ekv_seqs* seqs, const float* q, int32_t n_q_heads,
                             float alpha, float scale, const int32_t* sel, const int32_t* sel_count, int32_t cap,
                             int32_t sel_heads, float* out, float* tau, int32_t* support_count, float* psum,
                             int32_t* support_idx, float* support_p, int32_t support_cap, void* workspace,
                             size_t ws_bytes, void* stream) {
  ekv::DecodeArgs a;
  ekv::Layout L;
  ekv_status st = prepare_decode(cache, seqs, q, n_q_heads, alpha, scale, sel, sel_count, cap, sel_heads, out, &a);
  if (st != EKV_OK) return st;
  if ((st = decode_outputs(&a, tau, support_count, psum, support_idx, support_p, support_cap)) != EKV_OK) return st;
  if ((st = check_ws(cache, seqs, n_q_heads, workspace, ws_bytes, list_pages(seqs, sel ? cap : 0), true, &L)) !=
      EKV_OK)
    return st;
  a.status = at<uint32_t>(workspace, L.status);
  decode_regions(&a, workspace, L);
  // about 4 gather blocks per compute unit (one resident wave of blocks)
  return hip_status(ekv::launch_decode(a, 4 * device_cus(), (hipStream_t)stream), "entmax_decode launch");
}

ekv_status ekv_entmax_decode_noalloc(const ekv_cache* cache, const ekv_seqs* seqs, const float* q,
                                     int32_t n_q_heads, float alpha, float scale, const int32_t* sel,
                                     const int32_t* sel_count, int32_t cap, int32_t sel_heads, float* out, float* tau,
                                     int32_t* support_count, float* psum, int32_t* support_idx, float* support_p,
                                     int32_t support_cap, uint32_t* dev_status, void* stream) {
  ekv::DecodeArgs a;
  ekv_status st = prepare_decode(cache, seqs, q, n_q_heads, alpha, scale, sel, sel_count, cap, sel_heads, out, &a);
  if (st != EKV_OK) return st;
  if ((st = decode_outputs(&a, tau, support_count, psum, support_idx, support_p, support_cap)) != EKV_OK) return st;
  const ekv::Layout L = ekv::make_decode_layout(seqs->batch, n_q_heads, cache->page_size,
                                                list_pages(seqs, sel ? cap : 0));
  if (L.total > kStaticScratchBytes)
    return fail(EKV_ERR_WORKSPACE, "entmax_decode_noalloc: this call needs " + std::to_string(L.total) +
                                       " bytes of scratch, above its fixed " + std::to_string(kStaticScratchBytes) +
                                       " (fewer query heads or sequences, or a smaller cap)");
  void* base = nullptr;
  if ((st = static_scratch(&base)) != EKV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dev_status) {
    a.status = dev_status;
  } else {
    // the status word of the scratch, cleared for this call (no report)
    a.status = at<uint32_t>(base, L.status);
    if ((st = hip_status(ekv::launch_fill_zero(a.status, 16, s), "scratch status clear")) != EKV_OK) return st;
  }
  decode_regions(&a, base, L);
  return hip_status(ekv::launch_decode(a, 4 * device_cus(), s), "entmax_decode_noalloc launch");
}

ekv_status ekv_softmax_decode(const ekv_cache* cache, const ekv_seqs* seqs, const float* q, int32_t n_q_heads,
                              float scale, const int32_t* sel, const int32_t* sel_count, int32_t cap,
                              int32_t sel_heads, float* out, float* lse, void* workspace, size_t ws_bytes,
                              void* stream) {
  ekv::DecodeArgs a;
  ekv::Layout L;
  ekv_status st = prepare_decode(cache, seqs, q, n_q_heads, 2.0f, scale, sel, sel_count, cap, sel_heads, out, &a);
  if (st != EKV_OK) return st;
  if ((st = check_ws(cache, seqs, n_q_heads, workspace, ws_bytes, 1, false, &L)) != EKV_OK) return st;
  a.status = at<uint32_t>(workspace, L.status);
  if (cache->kv_dtype != EKV_BF16) return fail(EKV_ERR_UNSUPPORTED, "softmax decode needs bf16 keys/values");
  if (a.group == 8) {
    // the kernels hold four heads per unit: split each query group in two
    // halves, each reading its KV head's rows and page list
    a.n_kv_heads *= 2;
    a.group = 4;
    a.kv_shift += 1;
    if (a.sel) a.sel_shift = 1;
  }
  float* part = at<float>(workspace, L.smx_part);
  return hip_status(ekv::launch_softmax(a, 4 * device_cus(), part, ekv::kSmxMaxSlots, lse, (hipStream_t)stream),
                    "softmax_decode launch");
}

ekv_status ekv_read_device_status(void* workspace, size_t ws_bytes, int32_t* host_flags, void* stream) {
  if (!workspace || ws_bytes < 256) return fail(EKV_ERR_WORKSPACE, "workspace is NULL or too small");
  if (!host_flags) return fail(EKV_ERR_INVALID_ARG, "host_flags is NULL");
  hipStream_t s = (hipStream_t)stream;
  uint32_t v = 0;
  // ordered after the stream's earlier work; the word is cleared by a fill
  // kernel on the same stream, then the stream (only) is waited for
  hipError_t e = hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = ekv::launch_fill_zero(workspace, 16, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "read device status");
  *host_flags = (int32_t)v;
  return EKV_OK;
}

ekv_status ekv_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!src || !aligned16(src) || bytes % 16 != 0)
    return fail(EKV_ERR_INVALID_ARG, "src must be a 16-byte aligned buffer of a multiple of 16 bytes");
  if (!sink) return fail(EKV_ERR_INVALID_ARG, "sink is NULL");
  if (blocks > 65535) return fail(EKV_ERR_INVALID_ARG, "blocks must be <= 65535");
  const int nb = blocks > 0 ? blocks : 8 * device_cus();
  return hip_status(ekv::launch_stream_read(src, bytes, sink, nb, (hipStream_t)stream), "stream_read launch");
}

const char* ekv_status_string(int32_t status) {
  switch (status) {
    case EKV_OK: return "ok";
    case EKV_ERR_INVALID_ARG: return "invalid argument";
    case EKV_ERR_UNSUPPORTED: return "unsupported";
    case EKV_ERR_WORKSPACE: return "workspace missing or too small";
    case EKV_ERR_CAPACITY: return "selection capacity too small";
    case EKV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* ekv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
