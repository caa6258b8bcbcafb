// Kernel argument blocks and launchers of the EntmaxKV HIP library.
#pragma once

#include "ekv_common.h"

namespace ekv {

// Limits the kernels are compiled for (checked on the host before launch).
constexpr int kMaxGroup = 8;         // query heads per KV head
constexpr int kMaxUnits = 4096;      // batch * n_kv_heads
constexpr int kLdsCands = 4096;      // candidates kept in LDS by the threshold solve

struct AppendArgs {
  int batch, n_kv_heads, page_size, head_dim, kv_dtype, max_pages, n_phys, n_new;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* k;
  void* v;
  void* k_box;
  float* k_moments;
  const void* k_new;
  const void* v_new;
  uint32_t* status;
};

// n_kv_heads and group describe the selection units: a unit is (sequence,
// KV head) with `group` query heads, or, in per-query-head mode, (sequence,
// query head) with group 1.  Cache records of unit head g live at KV head
// g >> kv_shift of the cache's hkv_mem heads.
struct SelectArgs {
  int batch, n_kv_heads, n_q_heads, group, page_size, head_dim, kv_dtype, max_pages, n_phys;
  int hkv_mem, kv_shift;
  int per_head_scores;  // bbox scoring: one score row per query head instead of the group maximum
  const int32_t* page_table;
  const int32_t* seq_lens;
  const void* k_box;
  const float* k_moments;
  const float* q;
  int policy, top_k, min_pages;
  float alpha, scale, delta;
  int32_t* sel;
  int32_t* sel_count;
  int cap;
  float* tau_hat_out;  // optional
  float* scores;       // bbox page scores [B*Hkv][score_stride]
  int score_stride;
  float2* musd;        // Gaussian page score (mean_Y, sd_Y) [B*Hq*max_pages]
  float* ehat;         // estimated page maximum [B*Hq*max_pages]
  float4* stats_out;   // optional (mean_Y, sd_Y, e_hat, n_p) copy for diagnostics
  double* tau_hat;     // [B*Hq]
  uint64_t* keep_bits; // [B*Hq][keep_words] keep decisions of each query head (bit p: page p)
  int keep_words;
  uint64_t* cand;      // [B*Hkv][cand_lists][kCandPerList] top-k candidate lists (NULL: none)
  uint32_t* cand_cut;  // [B*Hkv][cand_lists]
  int cand_lists;      // candidate lists per unit written by the scoring; 0: top-k reads every score
  uint32_t* done;      // [B*Hkv] arrival counters, zero between calls
  uint32_t* status;
};

struct DecodeArgs {
  int batch, n_kv_heads, n_q_heads, group, page_size, head_dim, kv_dtype, max_pages, n_phys;
  int hkv_mem, kv_shift;  // as in SelectArgs
  int sel_shift;          // unit u reads page-list row u >> sel_shift (two units per list row when a
                          // query group is split in halves)
  const int32_t* page_table;
  const int32_t* seq_lens;
  const void* k;
  const void* v;
  const float* q;
  float alpha, scale;
  const int32_t* sel;  // NULL: every page of every sequence
  const int32_t* sel_count;
  int cap;
  float* out;
  float* tau;            // optional
  int32_t* support_count;  // optional
  float* psum;           // optional
  int32_t* support_idx;  // optional
  float* support_p;      // optional
  int support_cap;
  int max_items;  // per (sequence, query head)
  int32_t* item_cnt;
  float* item_max;
  float* item_lb;
  uint32_t* item_lvl;
  float* cand_x;
  int32_t* cand_t;
  int32_t* cand_r;
  float* ovf_x;
  int32_t* ovf_t;
  int32_t* ovf_r;
  uint32_t* status;
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_score_bbox(const SelectArgs& a, hipStream_t s);
hipError_t launch_topk(const SelectArgs& a, hipStream_t s);
hipError_t launch_score_gauss(const SelectArgs& a, hipStream_t s);
hipError_t launch_tau_hat(const SelectArgs& a, hipStream_t s);
hipError_t launch_gauss_floor(const SelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int target_blocks, hipStream_t s);
// softmax decode over the same page list; `part` holds max_slots * (D + 2)
// floats per query head
hipError_t launch_softmax(const DecodeArgs& a, int target_blocks, float* part, int max_slots, float* lse,
                          hipStream_t s);

}  // namespace ekv
