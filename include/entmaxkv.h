/*
 * entmaxkv.h - C ABI of the EntmaxKV support-aware paged sparse
 * alpha-entmax decode step for AMD Instinct MI355X (gfx950).
 *
 * The method ("EntmaxKV: Support-Aware Decoding for Entmax Attention",
 * arXiv 2605.21649; gist.science technical summary sections 2.A-2.C, the
 * authors' abstract) decodes one token over a paged KV cache in four steps:
 *   1. score every page from lightweight per-page metadata (a coordinate-wise
 *      k_min/k_max bounding box, or Gaussian first/second moments) before any
 *      key or value is loaded                              (summary sec. 2.A)
 *   2. choose candidate pages: fixed-budget top-k on the box bound, or the
 *      Gaussian-aware selector that estimates the global entmax threshold
 *      tau_hat and keeps pages whose estimated maximum exceeds tau_hat-Delta
 *                                                          (summary sec. 2.B)
 *   3./4. load only those pages and run exact alpha-entmax attention over
 *      them                                                (summary sec. 2.C)
 * with p_j = [(alpha-1) z_j - tau]_+^(1/(alpha-1)), z_j = scale q.k_j,
 * sum p = 1, output sum_j p_j v_j.  When the chosen pages contain the entmax
 * support the output equals the full-cache output (summary sec. 3).
 *
 * Conventions shared by every call:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     never allocates and never frees.  Scratch memory is the caller-owned
 *     workspace (see ekv_workspace_size / ekv_workspace_init).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns; no call synchronises,
 *     except ekv_read_device_status.
 *   - Every call validates its arguments on the host and returns a negative
 *     ekv_status before enqueueing anything if they are invalid; nothing is
 *     launched in that case.  ekv_last_error() then returns a message.
 *   - Conditions only the device can see (a page-table entry outside
 *     [0, n_phys_pages), a sequence longer than max_pages*page_size) set bits
 *     of a status word in the workspace; the offending page is skipped.  Read
 *     it with ekv_read_device_status on the stream of the calls.
 *   - Calls that share one workspace must be ordered (same stream or
 *     explicit dependencies); concurrent calls on one workspace race.
 *   - No exception crosses this boundary.
 */
#ifndef ENTMAXKV_H
#define ENTMAXKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EKV_OK = 0,
  EKV_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or value   */
  EKV_ERR_UNSUPPORTED = -2, /* valid request outside what is implemented    */
  EKV_ERR_WORKSPACE = -3,   /* workspace null or smaller than required      */
  EKV_ERR_CAPACITY = -4,    /* selection capacity smaller than required     */
  EKV_ERR_HIP = -5          /* a HIP launch or copy returned an error       */
} ekv_status;

typedef enum { EKV_F32 = 0, EKV_BF16 = 1 } ekv_dtype;

typedef enum {
  EKV_SELECT_BBOX_TOPK = 0, /* top-k pages by the bounding-box upper bound  */
  EKV_SELECT_GAUSS = 1      /* Gaussian-aware threshold selector           */
} ekv_policy;

/* Device status bits (ekv_read_device_status). */
#define EKV_DEV_BAD_PAGE 0x1    /* page-table entry out of [0, n_phys_pages) */
#define EKV_DEV_BAD_LENGTH 0x2  /* seq_len < 0 or > max_pages * page_size    */
#define EKV_DEV_OVERFLOW 0x4    /* an internal list hit its capacity         */

/*
 * The paged cache and its per-page metadata (summary sec. 2.A: the cache is
 * split into pages; per page the coordinate-wise minimum and maximum key and
 * the first and second moments of the keys are stored).
 *   k, v       [n_phys_pages][n_kv_heads][page_size][head_dim], kv_dtype
 *   k_box      [n_phys_pages][n_kv_heads][2][head_dim], kv_dtype:
 *              [..][0][i] = min over the page's tokens of k_i, [..][1][i] = max
 *              (min/max of stored values are exact in the storage type)
 *   k_moments  [n_phys_pages][n_kv_heads][2][head_dim], float32:
 *              [..][0][i] = mean of k_i over the page's tokens,
 *              [..][1][i] = sum of squared deviations from that mean (so the
 *              population variance is this / n_p), maintained by Welford's
 *              update in token order
 * k_box or k_moments may be NULL when that selector is not used.
 * Supported: head_dim in {64, 128}; page_size a power of two in [1, 1024];
 * kv_dtype EKV_F32 or EKV_BF16; n_kv_heads >= 1.  All pointers 16-byte
 * aligned.
 */
typedef struct {
  int32_t n_phys_pages;
  int32_t n_kv_heads;
  int32_t page_size;
  int32_t head_dim;
  int32_t kv_dtype; /* ekv_dtype */
  int32_t reserved;
  void* k;
  void* v;
  void* k_box;
  float* k_moments;
} ekv_cache;

/*
 * The batch of sequences.
 *   page_table [batch][max_pages] int32: logical page -> physical page.
 *              Entries for pages at or beyond a sequence's length are unused.
 *   seq_lens   [batch] int32: current token count of each sequence.
 * Page allocation belongs to the caller: it writes page-table entries before
 * appending into a page.  The library never writes either array.
 */
typedef struct {
  int32_t batch;
  int32_t max_pages;
  const int32_t* page_table;
  const int32_t* seq_lens;
} ekv_seqs;

/*
 * Selection parameters (summary sec. 2.B).
 *   policy     ekv_policy
 *   top_k      pages kept per (sequence, KV head) by EKV_SELECT_BBOX_TOPK
 *              (all pages when top_k >= the sequence's page count)
 *   alpha      entmax alpha; EKV_SELECT_GAUSS supports alpha in [1.1, 2]
 *              (closed-form expectations at 1.5 and 2; otherwise truncated
 *              normal moments tabulated by quadrature on each call and
 *              interpolated)
 *   top_k      also applies per query head when per_head = 1
 *   scale      score scale, normally 1/sqrt(head_dim)
 *   delta      EKV_SELECT_GAUSS safety margin, in the scaled score domain
 *              x = (alpha-1) scale q.k where the threshold lives
 *   per_head   0: one page set per (sequence, KV head), shared by the KV
 *              head's query-head group (the group-level rule below);
 *              1: one page set per (sequence, query head), each head scored
 *              and selected on its own.  The summary does not say how
 *              grouped-query heads share a selection; both are offered.
 *   min_pages  EKV_SELECT_GAUSS: the fewest pages kept per selection unit
 *              (>= 1; entmax over an empty set is undefined).  When the keep
 *              rule keeps fewer than min(min_pages, n_b) pages, the unit keeps
 *              the min(min_pages, n_b) pages of largest margin
 *              max_h (e_hat - tau_hat) instead, lower page id first on equal
 *              margins.  Values above 1 need max_pages <= 65535.  Not used by
 *              EKV_SELECT_BBOX_TOPK, which always keeps min(top_k, n_b) pages.
 */
typedef struct {
  int32_t policy;
  int32_t top_k;
  float alpha;
  float scale;
  float delta;
  int32_t per_head;
  int32_t min_pages;
} ekv_select_params;

/*
 * Workspace bytes for the calls on this cache/batch shape with n_q_heads
 * query heads.  Returns 0 if the shape is invalid.
 *   cap  the largest page-list capacity of the sparse ekv_entmax_decode
 *        calls the workspace will serve; its per-item candidate regions
 *        (four bytes per token of a list, six arrays per query head) are
 *        sized for lists of min(cap, max_pages) pages.  cap <= 0 sizes them
 *        for the whole cache, which a full-cache decode (sel == NULL) needs.
 * Selection, scoring and softmax decode use only the part before those
 * regions, which does not depend on cap.  Every call checks ws_bytes against
 * what it needs and returns EKV_ERR_WORKSPACE when it is short.
 */
size_t ekv_workspace_size(const ekv_cache* cache, const ekv_seqs* seqs, int32_t n_q_heads, int32_t cap);

/*
 * Prepare a fresh workspace (clears its control words with a fill kernel on
 * `stream`).  Required once after allocation; the calls keep it consistent
 * afterwards.  Call again after any call that failed on the device.
 */
ekv_status ekv_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/*
 * Append n_new tokens to every sequence (the cache grows by one token per
 * decode step, summary sec. 1): token i of sequence b goes to logical
 * position seq_lens[b] + i, i.e. page (seq_lens[b]+i)/page_size, slot
 * (seq_lens[b]+i) % page_size.  The page's metadata is re-initialised when
 * the token starts the page and updated otherwise (k_min/k_max by min/max,
 * moments by Welford's update in token order), so appending tokens one call
 * at a time and appending them in one call give bit-identical metadata.
 *   k_new, v_new  [batch][n_new][n_kv_heads][head_dim], kv_dtype, 16-byte
 *                 aligned
 * seq_lens holds the lengths BEFORE the append and is not modified; the
 * caller advances it.  Needs seq_lens[b] + n_new <= max_pages * page_size
 * and page-table entries for every touched page.
 */
ekv_status ekv_append_kv(const ekv_cache* cache, const ekv_seqs* seqs, const void* k_new,
                         const void* v_new, int32_t n_new, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * Score pages and select candidates for every (sequence, KV head); the
 * selection is shared by the KV head's query-head group.  With
 * params->per_head = 1 every query head gets its own selection: the rules
 * below then apply with a group of one head (its own bound, its own
 * threshold estimate), and sel/sel_count have n_q_heads rows per sequence.
 *   q          [batch][n_q_heads][head_dim] float32, 16-byte aligned;
 *              n_q_heads = G * n_kv_heads with G in {1, 2, 4, 8}
 *   sel        [batch][H][cap] int32: ascending logical page ids, with
 *              H = n_kv_heads (shared) or n_q_heads (per_head = 1)
 *   sel_count  [batch][H] int32: number of valid entries in sel
 *   tau_hat    optional [batch][n_q_heads] float32 (EKV_SELECT_GAUSS only):
 *              the estimated threshold per query head
 *   workspace  at least the cap-independent part (ekv_workspace_size)
 * BBOX_TOPK: page score = max over the group's heads of
 *   scale * sum_i max(q_i k_min_i, q_i k_max_i), the tightest upper bound
 *   the box gives on q.k (summary sec. 2.A); keeps the min(top_k, n_b)
 *   highest, lower page id first on equal scores.  Needs cap >= top_k
 *   (else EKV_ERR_CAPACITY) and max_pages <= 65535 (else
 *   EKV_ERR_UNSUPPORTED).
 * GAUSS: per query head, page scores are modelled as Gaussian with mean
 *   (alpha-1) scale q.mu and variance ((alpha-1) scale)^2 sum_i q_i^2 var_i;
 *   tau_hat solves sum_p n_p E[(Y_p - t)_+^(1/(alpha-1))] = 1; a page is kept
 *   when, for some head of the group, mean + sd sqrt(2 ln n_p) - tau_hat >
 *   -delta; at least one page is always kept.  Needs cap >= max_pages (else
 *   EKV_ERR_CAPACITY).
 */
ekv_status ekv_select_pages(const ekv_cache* cache, const ekv_seqs* seqs, const float* q,
                            int32_t n_q_heads, const ekv_select_params* params, int32_t* sel,
                            int32_t* sel_count, int32_t cap, float* tau_hat, void* workspace,
                            size_t ws_bytes, void* stream);

/*
 * Exact alpha-entmax decode (summary sec. 2.C) over the selected pages, or
 * over the whole cache when sel == NULL (full-cache baseline).
 *   q          [batch][n_q_heads][head_dim] float32
 *   alpha      > 1 (exact threshold for 1.5 and 2, Newton-converged otherwise)
 *   sel, sel_count, cap  as produced by ekv_select_pages (sel_count entries
 *              are clamped to [0, cap] and to the sequence's page count)
 *   sel_heads  rows of sel per sequence: n_kv_heads (query head h reads the
 *              list of KV head h / G) or n_q_heads (query head h reads its
 *              own list, from per_head selection); any other value is
 *              EKV_ERR_INVALID_ARG when sel != NULL, ignored otherwise
 *   out        [batch][n_q_heads][head_dim] float32, 16-byte aligned:
 *              sum_j p_j v_j
 *   tau        optional [batch][n_q_heads] float32: the threshold (x domain)
 *   support_count optional [batch][n_q_heads] int32: tokens with p_j > 0
 *   psum       optional [batch][n_q_heads] float32: sum_j p_j
 *   support_idx optional [batch][n_q_heads][support_cap] int32: ascending
 *              logical token ids of the support (first support_cap of them)
 *   support_p  optional [batch][n_q_heads][support_cap] float32: their
 *              weights p_j, in the same order (needs support_cap >= 1)
 * Scores are accumulated in float32; the threshold is finalised in float64.
 */
ekv_status ekv_entmax_decode(const ekv_cache* cache, const ekv_seqs* seqs, const float* q,
                             int32_t n_q_heads, float alpha, float scale, const int32_t* sel,
                             const int32_t* sel_count, int32_t cap, int32_t sel_heads, float* out, float* tau,
                             int32_t* support_count, float* psum, int32_t* support_idx,
                             float* support_p, int32_t support_cap, void* workspace, size_t ws_bytes,
                             void* stream);

/*
 * ekv_entmax_decode without a workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, kernels and results as
 * ekv_entmax_decode, except:
 *   - scratch: a fixed 64 MiB device array inside the library, one per
 *     device, held from the library's load until the process ends.  Its
 *     per-item regions take 6 * 64 * 4 + 16 = 1552 bytes per (sequence, query
 *     head, 64-token item of the longest list): a call whose lists (cap pages,
 *     or the whole cache when sel == NULL) need more returns
 *     EKV_ERR_WORKSPACE before launching anything.  The call allocates
 *     nothing.
 *   - dev_status: optional device uint32; the EKV_DEV_* bits of this call are
 *     OR-ed into it (the caller clears it).  With NULL they are not reported.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents: calls that overlap on one device (other streams, other
 * threads) race and must be ordered by the caller.
 */
ekv_status ekv_entmax_decode_noalloc(const ekv_cache* cache, const ekv_seqs* seqs, const float* q,
                                     int32_t n_q_heads, float alpha, float scale, const int32_t* sel,
                                     const int32_t* sel_count, int32_t cap, int32_t sel_heads, float* out,
                                     float* tau, int32_t* support_count, float* psum, int32_t* support_idx,
                                     float* support_p, int32_t support_cap, uint32_t* dev_status, void* stream);

/*
 * Softmax attention decode over the same page list, the baseline the
 * EntmaxKV summary compares against (sec. 1 and 3: softmax gives every
 * token a positive weight, so a dropped page always leaves some error):
 * z_j = scale q.k_j over the selected pages' tokens (sel != NULL) or the
 * whole cache (sel == NULL), p = softmax(z) over that set, out = sum_j p_j v_j.
 *   lse   optional [batch][n_q_heads] float32: log sum_j exp(z_j) over the
 *         set (-inf when it is empty); the full-cache mass outside a kept
 *         set J is 1 - exp(lse_J - lse_full)
 * Other arguments as for ekv_entmax_decode.  Needs bf16 K/V (else
 * EKV_ERR_UNSUPPORTED).  Accumulates in float32 with a running maximum per
 * block, merged in a fixed order.
 */
ekv_status ekv_softmax_decode(const ekv_cache* cache, const ekv_seqs* seqs, const float* q,
                              int32_t n_q_heads, float scale, const int32_t* sel,
                              const int32_t* sel_count, int32_t cap, int32_t sel_heads, float* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * Page scores only (diagnostics and parity checks).
 *   BBOX_TOPK: scores [batch][H][max_pages] float32, the page score used by
 *              the selector (-inf for pages past the sequence end); H as in
 *              ekv_select_pages.
 *   GAUSS:     scores [batch][n_q_heads][max_pages][4] float32:
 *              (mean_Y, sd_Y, estimated max, n_p) per page.
 */
ekv_status ekv_score_pages(const ekv_cache* cache, const ekv_seqs* seqs, const float* q,
                           int32_t n_q_heads, const ekv_select_params* params, float* scores,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Copy the device status word (EKV_DEV_* bits) to *host_flags and clear it,
 * in order after the work already enqueued on `stream`.  Synchronous: waits
 * for `stream` (only) before returning.  Work on other streams that shares
 * the workspace must be ordered before it by the caller.
 */
ekv_status ekv_read_device_status(void* workspace, size_t ws_bytes, int32_t* host_flags, void* stream);

/*
 * Measurement helper, not part of the decode path: one plain streaming read
 * of `bytes` (a multiple of 16) from the 16-byte aligned device buffer src,
 * with `blocks` blocks of 256 threads (<= 0: eight per compute unit), on
 * `stream`.  Timing it after the caches are evicted gives the read-stream
 * ceiling the decode kernels are compared with at the same size.  sink:
 * one device uint32 the kernel may set (its value is meaningless).
 */
ekv_status ekv_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/* Static description of a status code. */
const char* ekv_status_string(int32_t status);

/* Message describing the most recent failure on the calling thread. */
const char* ekv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAXKV_H */
