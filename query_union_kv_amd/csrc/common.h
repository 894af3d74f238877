// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pw.h"

// ---- debug build (-DPW_DEBUG) ------------------------------------------------------------
// PW_DCHECK(cond) counts, in a device counter of its translation unit, every lane at which
// an index or ring invariant does not hold (no trap: the kernels still clamp and skip as in
// the release build, so a violation never faults).  pw_debug_violations() (api.cpp) reads
// and clears the counters of every translation unit.  Release builds compile it away.
#ifdef PW_DEBUG
#define PW_DEBUG_COUNTER_DEFINE(name)                                                   \
  static __device__ unsigned int pw_dbg_count;                                        \
  unsigned long long name() {                                                          \
    unsigned int v = 0, z = 0;                                                         \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(pw_dbg_count), sizeof(v)) != hipSuccess)    \
      return ~0ull;                                                                    \
    if (hipMemcpyToSymbol(HIP_SYMBOL(pw_dbg_count), &z, sizeof(z)) != hipSuccess)      \
      return ~0ull;                                                                    \
    return v;                                                                          \
  }
#define PW_DCHECK(cond)                                      \
  do {                                                       \
    if (!(cond)) atomicAdd(&pw_dbg_count, 1u);                \
  } while (0)
#else
#define PW_DEBUG_COUNTER_DEFINE(name)
#define PW_DCHECK(cond) \
  do {                  \
  } while (0)
#endif

namespace pw {

#ifdef PW_DEBUG
// per-translation-unit readers of the debug counters (read and clear; ~0 on a HIP error)
unsigned long long debug_count_attn();
unsigned long long debug_count_prep();
unsigned long long debug_count_pageunion();
#endif

// Records a formatted error message for pw_last_error() and returns `status`.
pw_status fail(pw_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Turns the result of the last launch into a status.
pw_status check_launch(const char* what);

// ---- launchers (validated arguments only) --------------------------------------------
pw_status launch_append_kv(const void* k_new, const void* v_new, int n_tok, int hkv, int d,
                           int64_t stride_tok, int first_token, void* k_cache, void* v_cache,
                           int kv_dtype, float* k_scale, float* v_scale, int page_size,
                           int n_pages, int64_t stride_head, int64_t stride_page,
                           hipStream_t stream);

pw_status launch_page_bitsets(const int32_t* topk, int n_rows, int hkv, int k, int n_pages,
                              uint64_t* bits, int32_t* bad_id_count, hipStream_t stream);

pw_status launch_group(const uint64_t* bits, int nq, int hkv, int n_pages, int window,
                       int max_group, int n_groups, int32_t* group_qids, int32_t* group_size,
                       hipStream_t stream);

pw_status launch_union_tables(const uint64_t* bits, int n_rows, int hkv, int n_pages,
                              const int32_t* group_rows, const int32_t* group_size, int n_groups,
                              int group_width, int32_t* union_off, int32_t* union_pages,
                              uint8_t* union_qmask, int64_t capacity, hipStream_t stream);

// Fused bitsets + grouping + union tables (windows <= 64, n_pages <= 1024), and the
// work order of pw_schedule_items when item_order is not NULL.
bool prepare_fusable(int n_pages, int window);
pw_status launch_prepare(const int32_t* topk, int nq, int hkv, int k, int n_pages, int window,
                         int max_group, int n_groups, uint64_t* bits, int32_t* bad_id_count,
                         int32_t* group_qids, int32_t* group_size, int32_t* union_off,
                         int32_t* union_pages, uint8_t* union_qmask, int64_t capacity,
                         int32_t* item_order, int halves, hipStream_t stream);

// Member order of 5..8-member groups for 4-member row tiles, with member-mask bits to match.
pw_status launch_arrange(const uint64_t* bits, int nq, int hkv, int n_pages, int n_groups,
                         int max_group, int32_t* group_qids, const int32_t* group_size,
                         const int32_t* union_off, uint8_t* union_qmask, int64_t capacity,
                         hipStream_t stream);

// Exclusive prefix sum in place: off[1..n] hold counts; afterwards off[i] = sum of the
// first i counts (off[0] = 0).  One workgroup.
pw_status launch_scan(int32_t* off, int n, hipStream_t stream);
// Largest-first work order of n items (the work order of pw_schedule_items).
pw_status launch_schedule(const int32_t* union_off, int n, int32_t* order, hipStream_t stream);

// Page-major work items of the direct KV-page union, and the lse merge of its partials.
size_t page_workspace_bytes(int nq, int hkv, int n_pages);
pw_status launch_page_tables(const uint64_t* bits, int nq, int hkv, int n_pages, int k_max,
                             int chunk, void* workspace, int32_t* item_off, int32_t* item_kvh,
                             int32_t* item_page, int32_t* item_qids, int32_t* item_size,
                             int32_t* item_slot, int64_t item_capacity, hipStream_t stream);
pw_status launch_page_merge(const uint64_t* bits, int nq, int hkv, int g0, int g1, int G, int d,
                            int n_pages, int k_max, const void* part_o, const float* part_lse,
                            void* out, float* lse, hipStream_t stream);

struct AttnArgs {
  const void* q;
  int nq, hq, hkv, d;
  const void* k_cache;
  const void* v_cache;
  int kv_dtype;
  const float* k_scale;
  const float* v_scale;
  int page_size, n_pages;
  int64_t stride_head, stride_page;
  const int32_t* q_pos;
  int kv_len;
  float sm_scale;
  const int32_t* group_qids;
  const int32_t* group_size;
  int n_groups, max_group, shared_table;
  const int32_t* union_off;
  const int32_t* union_pages;
  const uint8_t* union_qmask;
  int64_t capacity;
  void* out;
  float* lse;
  // Page-major items (all NULL otherwise): item i runs for KV head item_kvh[i] over the
  // one page union_pages[i]; the items [*item_lo_dev, *item_hi_dev) run (n_groups bounds
  // their count); member j's row goes to partial row out_slot[i * max_group + j] * G +
  // (h - g*G).
  // > 1: the table of every item is cut into n_split consecutive slices, one workgroup
  // each; row (q, h) of slice s goes to partial row ((q*hkv + g)*n_split + s)*G + (h - g*G)
  // of out/lse (merged afterwards by launch_page_merge with bits == NULL).
  int n_split = 1;
  const int32_t* item_kvh = nullptr;
  const int32_t* item_lo_dev = nullptr;
  const int32_t* item_hi_dev = nullptr;
  const int32_t* out_slot = nullptr;
  // Work order (NULL: item order): position r of the launch runs item item_order[r]
  // (only with n_split == 1 and no page-major items).
  const int32_t* item_order = nullptr;
};

pw_status launch_sparse_prefill(const AttnArgs& a, hipStream_t stream);

// Largest (max_group * hq/hkv) one work item of pw_sparse_prefill supports.
int max_rows_per_item(int d, int kv_dtype);

}  // namespace pw
