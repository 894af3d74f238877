// C ABI of the query-union sparse-prefill library: host-side validation of every
// scalar argument, then the kernel launches.  Declarations and argument meaning are
// in include/pw.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>

#include "common.h"

#define PW_VERSION "0.1.0"

namespace pw {
namespace {
thread_local char g_err[512] = "";
}

pw_status fail(pw_status status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

pw_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PW_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PW_OK;
}

}  // namespace pw

using pw::fail;

extern "C" {

const char* pw_version(void) { return PW_VERSION; }

int64_t pw_debug_violations(void) {
#ifdef PW_DEBUG
  const unsigned long long a = pw::debug_count_attn(), b = pw::debug_count_prep(),
                           c = pw::debug_count_pageunion();
  if (a == ~0ull || b == ~0ull || c == ~0ull) return -1;
  return (int64_t)(a + b + c);
#else
  return -2;
#endif
}

const char* pw_last_error(void) { return pw::g_err; }

int pw_words(int n_pages) { return n_pages < 0 ? -1 : (n_pages + 63) / 64; }

int pw_num_groups(int nq, int window, int max_group) {
  if (nq < 0 || window < 1 || max_group < 1) return -1;
  const int full = nq / window, rest = nq % window;
  const int64_t total = (int64_t)full * ((window + max_group - 1) / max_group) +
                        (rest + max_group - 1) / max_group;
  return total > INT32_MAX ? -1 : (int)total;
}

int64_t pw_union_capacity(int n_tables, int group_width, int k_max, int n_pages) {
  if (n_tables < 0 || group_width < 1 || k_max < 0 || n_pages < 1) return -1;
  const int64_t per = std::min<int64_t>(n_pages, (int64_t)group_width * k_max);
  return (int64_t)n_tables * per;
}

pw_status pw_append_kv(const void* k_new, const void* v_new, int n_tok, int hkv, int d,
                       int64_t stride_tok, int first_token, void* k_cache, void* v_cache,
                       int kv_dtype, float* k_scale, float* v_scale, int page_size, int n_pages,
                       int64_t stride_head, int64_t stride_page, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (n_tok < 0 || hkv < 1 || first_token < 0 || page_size < 1 || n_pages < 1)
    return fail(PW_ERR_ARG, "pw_append_kv: bad sizes n_tok=%d hkv=%d first_token=%d page_size=%d n_pages=%d",
                n_tok, hkv, first_token, page_size, n_pages);
  if (d < 8 || d > 1024 || d % 8)
    return fail(PW_ERR_UNSUPPORTED, "pw_append_kv: d=%d (a multiple of 8 in 8..1024)", d);
  if (hkv > 65535) return fail(PW_ERR_UNSUPPORTED, "pw_append_kv: hkv=%d > 65535", hkv);
  if ((int64_t)n_pages * page_size >= INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_append_kv: n_pages*page_size must stay below 2^31");
  if (kv_dtype != PW_KV_BF16 && kv_dtype != PW_KV_FP8_E4M3)
    return fail(PW_ERR_UNSUPPORTED, "pw_append_kv: kv_dtype=%d", kv_dtype);
  if (stride_tok < (int64_t)hkv * d || stride_tok % 8)
    return fail(PW_ERR_ARG, "pw_append_kv: stride_tok=%lld must be >= hkv*d and a multiple of 8",
                (long long)stride_tok);
  const int esz = kv_dtype == PW_KV_FP8_E4M3 ? 1 : 2;
  if (stride_page < (int64_t)page_size * d || stride_head < 0)
    return fail(PW_ERR_ARG, "pw_append_kv: stride_page=%lld < page_size*d or stride_head < 0",
                (long long)stride_page);
  if ((stride_page * esz) % 16 || (stride_head * esz) % 16)
    return fail(PW_ERR_ARG, "pw_append_kv: strides must be multiples of 16 bytes");
  if (n_tok == 0) return PW_OK;
  if ((int64_t)first_token + n_tok - 1 >= (int64_t)n_pages * page_size)
    return fail(PW_ERR_CAPACITY, "pw_append_kv: tokens %d..%lld do not fit %d pages of %d",
                first_token, (long long)first_token + n_tok - 1, n_pages, page_size);
  if (!k_new || !v_new || !k_cache || !v_cache)
    return fail(PW_ERR_ARG, "pw_append_kv: null required pointer");
  if (kv_dtype == PW_KV_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(PW_ERR_ARG, "pw_append_kv: fp8 KV needs k_scale and v_scale");
  if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16)
    return fail(PW_ERR_ARG, "pw_append_kv: inputs and caches must be 16-byte aligned");
  return pw::launch_append_kv(k_new, v_new, n_tok, hkv, d, stride_tok, first_token, k_cache,
                              v_cache, kv_dtype, k_scale, v_scale, page_size, n_pages, stride_head,
                              stride_page, stream);
}

pw_status pw_page_bitsets(const int32_t* topk, int n_rows, int hkv, int k, int n_pages,
                          uint64_t* bits, int32_t* bad_id_count, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (n_rows < 0 || hkv < 1 || k < 1 || n_pages < 1)
    return fail(PW_ERR_ARG, "pw_page_bitsets: bad sizes n_rows=%d hkv=%d k=%d n_pages=%d", n_rows,
                hkv, k, n_pages);
  if (k > 4096) return fail(PW_ERR_UNSUPPORTED, "pw_page_bitsets: k=%d > 4096", k);
  if (n_pages > 65536)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_bitsets: n_pages=%d > 65536", n_pages);
  if ((int64_t)n_rows * hkv > INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_bitsets: n_rows*hkv too large");
  if (n_rows > 0 && (!topk || !bits)) return fail(PW_ERR_ARG, "pw_page_bitsets: null topk/bits");
  return pw::launch_page_bitsets(topk, n_rows, hkv, k, n_pages, bits, bad_id_count, stream);
}

pw_status pw_group(const uint64_t* bits, int nq, int hkv, int n_pages, int window, int max_group,
                   int32_t* group_qids, int32_t* group_size, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (nq < 0 || hkv < 1 || n_pages < 1)
    return fail(PW_ERR_ARG, "pw_group: bad sizes nq=%d hkv=%d n_pages=%d", nq, hkv, n_pages);
  if (max_group < 1 || max_group > 8)
    return fail(PW_ERR_UNSUPPORTED, "pw_group: max_group=%d not in 1..8", max_group);
  if (window < 1 || window > 1024)
    return fail(PW_ERR_UNSUPPORTED, "pw_group: window=%d not in 1..1024", window);
  if (window % max_group)
    return fail(PW_ERR_ARG, "pw_group: window=%d is not a multiple of max_group=%d", window,
                max_group);
  if (n_pages > 4096) return fail(PW_ERR_UNSUPPORTED, "pw_group: n_pages=%d > 4096", n_pages);
  const int n_groups = pw_num_groups(nq, window, max_group);
  if (n_groups < 0 || (int64_t)n_groups * hkv * max_group > INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_group: too many groups");
  if (nq > 0 && (!bits || !group_qids || !group_size))
    return fail(PW_ERR_ARG, "pw_group: null pointer argument");
  return pw::launch_group(bits, nq, hkv, n_pages, window, max_group, n_groups, group_qids,
                          group_size, stream);
}

pw_status pw_arrange_groups(const uint64_t* bits, int nq, int hkv, int n_pages, int hq,
                            int n_groups, int max_group, int32_t* group_qids,
                            const int32_t* group_size, const int32_t* union_off,
                            uint8_t* union_qmask, int64_t capacity, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (nq < 0 || hkv < 1 || hq < 1 || n_pages < 1 || n_groups < 0 || capacity < 0)
    return fail(PW_ERR_ARG, "pw_arrange_groups: bad sizes nq=%d hkv=%d hq=%d n_pages=%d n_groups=%d",
                nq, hkv, hq, n_pages, n_groups);
  if (hq % hkv) return fail(PW_ERR_ARG, "pw_arrange_groups: hq=%d not a multiple of hkv=%d", hq, hkv);
  if (max_group < 1 || max_group > 8)
    return fail(PW_ERR_UNSUPPORTED, "pw_arrange_groups: max_group=%d not in 1..8", max_group);
  if (n_pages > 65536) return fail(PW_ERR_UNSUPPORTED, "pw_arrange_groups: n_pages=%d > 65536", n_pages);
  // row tiles hold 16 query-head rows: only 4-member tiles (hq/hkv = 4) with groups of more
  // than one tile have a choice to make
  if (hq / hkv != 4 || max_group <= 4 || nq == 0 || n_groups == 0) return PW_OK;
  if (!bits || !group_qids || !group_size || !union_off)
    return fail(PW_ERR_ARG, "pw_arrange_groups: null required pointer");
  return pw::launch_arrange(bits, nq, hkv, n_pages, n_groups, max_group, group_qids, group_size,
                            union_off, union_qmask, capacity, stream);
}

pw_status pw_union_tables(const uint64_t* bits, int n_rows, int hkv, int n_pages,
                          const int32_t* group_rows, const int32_t* group_size, int n_groups,
                          int group_width, int k_max, int32_t* union_off, int32_t* union_pages,
                          uint8_t* union_qmask, int64_t capacity, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (n_rows < 0 || hkv < 1 || n_pages < 1 || n_groups < 0 || k_max < 0)
    return fail(PW_ERR_ARG, "pw_union_tables: bad sizes n_rows=%d hkv=%d n_pages=%d n_groups=%d k_max=%d",
                n_rows, hkv, n_pages, n_groups, k_max);
  if (group_width < 1 || group_width > 64)
    return fail(PW_ERR_UNSUPPORTED, "pw_union_tables: group_width=%d not in 1..64", group_width);
  if (union_qmask && group_width > 8)
    return fail(PW_ERR_UNSUPPORTED, "pw_union_tables: member masks need group_width <= 8 (got %d)",
                group_width);
  if (n_pages > 65536)
    return fail(PW_ERR_UNSUPPORTED, "pw_union_tables: n_pages=%d > 65536", n_pages);
  const int64_t n_tables = (int64_t)hkv * n_groups;
  if (n_tables >= INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_union_tables: too many tables");
  const int64_t need = pw_union_capacity((int)n_tables, group_width, k_max, n_pages);
  if (capacity < need)
    return fail(PW_ERR_CAPACITY, "pw_union_tables: capacity %lld < required %lld",
                (long long)capacity, (long long)need);
  if (capacity > INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_union_tables: capacity %lld exceeds int32 offsets",
                (long long)capacity);
  if (!union_off) return fail(PW_ERR_ARG, "pw_union_tables: null union_off");
  if (group_rows == nullptr && (int64_t)n_groups * group_width < n_rows)
    return fail(PW_ERR_ARG, "pw_union_tables: consecutive groups need n_groups*group_width >= n_rows");
  if (n_tables > 0 && (!bits || (need > 0 && !union_pages)))
    return fail(PW_ERR_ARG, "pw_union_tables: null pointer argument");
  return pw::launch_union_tables(bits, n_rows, hkv, n_pages, group_rows, group_size, n_groups,
                                 group_width, union_off, union_pages, union_qmask, capacity,
                                 stream);
}

namespace {

// pw_prepare and pw_prepare_halves: halves = 1 lists the union of each half of every group
// (tables 2j, 2j + 1 of group j, width max_group / 2) instead of the group's.
pw_status prepare_common(const char* fn, const int32_t* topk, int nq, int hkv, int k, int n_pages,
                         int window, int max_group, uint64_t* bits, int32_t* bad_id_count,
                         int32_t* group_qids, int32_t* group_size, int32_t* union_off,
                         int32_t* union_pages, uint8_t* union_qmask, int64_t capacity,
                         int32_t* item_order, int halves, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (nq < 0 || hkv < 1 || k < 1 || n_pages < 1)
    return fail(PW_ERR_ARG, "%s: bad sizes nq=%d hkv=%d k=%d n_pages=%d", fn, nq, hkv, k, n_pages);
  if (k > 4096) return fail(PW_ERR_UNSUPPORTED, "%s: k=%d > 4096", fn, k);
  if (max_group < 1 || max_group > 8)
    return fail(PW_ERR_UNSUPPORTED, "%s: max_group=%d not in 1..8", fn, max_group);
  if (halves && max_group % 2)
    return fail(PW_ERR_ARG, "%s: max_group=%d is odd (two halves need an even width)", fn, max_group);
  if (window < 1 || window > 1024)
    return fail(PW_ERR_UNSUPPORTED, "%s: window=%d not in 1..1024", fn, window);
  if (window % max_group)
    return fail(PW_ERR_ARG, "%s: window=%d is not a multiple of max_group=%d", fn, window, max_group);
  if (n_pages > 4096) return fail(PW_ERR_UNSUPPORTED, "%s: n_pages=%d > 4096", fn, n_pages);
  const int n_groups = pw_num_groups(nq, window, max_group);
  if (n_groups < 0 || (int64_t)n_groups * hkv * max_group > INT32_MAX / 2)
    return fail(PW_ERR_UNSUPPORTED, "%s: too many groups", fn);
  const int n_tables = hkv * n_groups * (halves ? 2 : 1);
  const int width = halves ? max_group / 2 : max_group;
  const int64_t need = pw_union_capacity(n_tables, width, k, n_pages);
  if (capacity < need)
    return fail(PW_ERR_CAPACITY, "%s: capacity %lld < required %lld", fn, (long long)capacity,
                (long long)need);
  if (capacity > INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "%s: capacity %lld exceeds int32 offsets", fn, (long long)capacity);
  if (!union_off) return fail(PW_ERR_ARG, "%s: null union_off", fn);
  if (nq > 0 && (!topk || !bits || !group_qids || !group_size || !union_pages || !union_qmask))
    return fail(PW_ERR_ARG, "%s: null pointer argument", fn);
  if (pw::prepare_fusable(n_pages, window))
    return pw::launch_prepare(topk, nq, hkv, k, n_pages, window, max_group, n_groups, bits,
                              bad_id_count, group_qids, group_size, union_off, union_pages,
                              union_qmask, capacity, item_order, halves, stream);
  pw_status st = pw::launch_page_bitsets(topk, nq, hkv, k, n_pages, bits, bad_id_count, stream);
  if (st == PW_OK)
    st = pw::launch_group(bits, nq, hkv, n_pages, window, max_group, n_groups, group_qids,
                          group_size, stream);
  if (st == PW_OK)   // halves: the member lists as [hkv][2 n_groups][mg/2], absent members -1
    st = pw::launch_union_tables(bits, nq, hkv, n_pages, group_qids, halves ? nullptr : group_size,
                                 halves ? 2 * n_groups : n_groups, width, union_off, union_pages,
                                 union_qmask, capacity, stream);
  if (st == PW_OK && item_order) st = pw::launch_schedule(union_off, n_tables, item_order, stream);
  return st;
}

}  // namespace

pw_status pw_prepare(const int32_t* topk, int nq, int hkv, int k, int n_pages, int window,
                     int max_group, uint64_t* bits, int32_t* bad_id_count, int32_t* group_qids,
                     int32_t* group_size, int32_t* union_off, int32_t* union_pages,
                     uint8_t* union_qmask, int64_t capacity, int32_t* item_order,
                     hipStream_t stream) {
  return prepare_common("pw_prepare", topk, nq, hkv, k, n_pages, window, max_group, bits,
                        bad_id_count, group_qids, group_size, union_off, union_pages, union_qmask,
                        capacity, item_order, 0, stream);
}

pw_status pw_prepare_halves(const int32_t* topk, int nq, int hkv, int k, int n_pages, int window,
                            int max_group, uint64_t* bits, int32_t* bad_id_count,
                            int32_t* group_qids, int32_t* group_size, int32_t* union_off,
                            int32_t* union_pages, uint8_t* union_qmask, int64_t capacity,
                            int32_t* item_order, hipStream_t stream) {
  return prepare_common("pw_prepare_halves", topk, nq, hkv, k, n_pages, window, max_group, bits,
                        bad_id_count, group_qids, group_size, union_off, union_pages, union_qmask,
                        capacity, item_order, 1, stream);
}

int64_t pw_page_items_capacity(int nq, int hkv, int k_max, int n_pages, int chunk) {
  if (nq < 0 || hkv < 1 || k_max < 1 || n_pages < 1 || chunk < 1) return -1;
  const int64_t edges = (int64_t)nq * hkv * std::min(k_max, n_pages);
  const int64_t n_gp = (int64_t)hkv * n_pages;
  return std::min(edges, (edges + n_gp * (chunk - 1) + chunk - 1) / chunk);
}

size_t pw_page_workspace_bytes(int nq, int hkv, int n_pages) {
  if (nq < 0 || hkv < 1 || n_pages < 1) return 0;
  return pw::page_workspace_bytes(nq, hkv, n_pages);
}

pw_status pw_page_tables(const uint64_t* bits, int nq, int hkv, int n_pages, int k_max, int chunk,
                         void* workspace, size_t workspace_bytes, int32_t* item_off,
                         int32_t* item_kvh, int32_t* item_page, int32_t* item_qids,
                         int32_t* item_size, int32_t* item_slot, int64_t item_capacity,
                         hipStream_t stream) {
  pw::g_err[0] = 0;
  if (nq < 0 || hkv < 1 || n_pages < 1 || k_max < 1)
    return fail(PW_ERR_ARG, "pw_page_tables: bad sizes nq=%d hkv=%d n_pages=%d k_max=%d", nq, hkv,
                n_pages, k_max);
  if (chunk < 1 || chunk > 64) return fail(PW_ERR_UNSUPPORTED, "pw_page_tables: chunk=%d not in 1..64", chunk);
  if (n_pages > 65536) return fail(PW_ERR_UNSUPPORTED, "pw_page_tables: n_pages=%d > 65536", n_pages);
  if (hkv > 65535 || nq > 64 * 65535)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_tables: hkv=%d or nq=%d too large", hkv, nq);
  if ((int64_t)nq * hkv * k_max >= INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_tables: nq*hkv*k_max must stay below 2^31");
  const int64_t need = pw_page_items_capacity(nq, hkv, k_max, n_pages, chunk);
  if (item_capacity < need)
    return fail(PW_ERR_CAPACITY, "pw_page_tables: item_capacity %lld < %lld", (long long)item_capacity,
                (long long)need);
  if (workspace_bytes < pw::page_workspace_bytes(nq, hkv, n_pages))
    return fail(PW_ERR_CAPACITY, "pw_page_tables: workspace_bytes %zu < %zu", workspace_bytes,
                pw::page_workspace_bytes(nq, hkv, n_pages));
  if (!item_off) return fail(PW_ERR_ARG, "pw_page_tables: null item_off");
  if (nq > 0 && (!bits || !workspace || !item_kvh || !item_page || !item_qids || !item_size || !item_slot))
    return fail(PW_ERR_ARG, "pw_page_tables: null required pointer");
  if ((uintptr_t)workspace % 8) return fail(PW_ERR_ARG, "pw_page_tables: workspace must be 8-byte aligned");
  return pw::launch_page_tables(bits, nq, hkv, n_pages, k_max, chunk, workspace, item_off, item_kvh,
                                item_page, item_qids, item_size, item_slot, item_capacity, stream);
}

pw_status pw_page_union_prefill(const void* q, int nq, int hq, int hkv, int d, const void* k_cache,
                                const void* v_cache, int kv_dtype, const float* k_scale,
                                const float* v_scale, int page_size, int n_pages,
                                int64_t stride_head, int64_t stride_page, const int32_t* q_pos,
                                int kv_len, float sm_scale, const uint64_t* bits, int k_max,
                                int chunk, const int32_t* item_off, const int32_t* item_kvh,
                                const int32_t* item_page, const int32_t* item_qids,
                                const int32_t* item_size, const int32_t* item_slot,
                                int64_t item_capacity, void* partial_o, float* partial_lse,
                                void* out, float* lse, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (nq < 0 || hq < 1 || hkv < 1 || n_pages < 1 || kv_len < 0 || k_max < 1 || item_capacity < 0)
    return fail(PW_ERR_ARG, "pw_page_union_prefill: bad sizes nq=%d hq=%d hkv=%d n_pages=%d k_max=%d",
                nq, hq, hkv, n_pages, k_max);
  if (hq % hkv) return fail(PW_ERR_ARG, "pw_page_union_prefill: hq=%d not a multiple of hkv=%d", hq, hkv);
  const int G = hq / hkv;
  if (d != 64 && d != 128) return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: d=%d (64 or 128)", d);
  if (page_size != 64 && page_size != 128)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: page_size=%d (64 or 128)", page_size);
  if (kv_dtype != PW_KV_BF16 && kv_dtype != PW_KV_FP8_E4M3)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: kv_dtype=%d", kv_dtype);
  if (chunk < 1 || chunk > 64 || (int64_t)G * chunk > pw::max_rows_per_item(d, kv_dtype))
    return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: chunk=%d (1..64, (hq/hkv)*chunk <= %d)",
                chunk, pw::max_rows_per_item(d, kv_dtype));
  if ((int64_t)k_max * G > 16384)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: k_max*(hq/hkv)=%lld > 16384",
                (long long)k_max * G);
  if ((int64_t)nq * hkv * k_max >= INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: nq*hkv*k_max must stay below 2^31");
  if (item_capacity >= INT32_MAX / 8)
    return fail(PW_ERR_UNSUPPORTED, "pw_page_union_prefill: item_capacity too large");
  const int esz = kv_dtype == PW_KV_FP8_E4M3 ? 1 : 2;
  if (stride_page < (int64_t)page_size * d || stride_head < 0)
    return fail(PW_ERR_ARG, "pw_page_union_prefill: stride_page < page_size*d or stride_head < 0");
  if ((stride_page * esz) % 16 || (stride_head * esz) % 16)
    return fail(PW_ERR_ARG, "pw_page_union_prefill: strides must be multiples of 16 bytes");
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out | (uintptr_t)partial_o) % 16)
    return fail(PW_ERR_ARG, "pw_page_union_prefill: q, caches, partial_o and out must be 16-byte aligned");
  if (!(sm_scale > 0.f)) return fail(PW_ERR_ARG, "pw_page_union_prefill: sm_scale must be positive");
  if (nq == 0) return PW_OK;
  if (!q || !k_cache || !v_cache || !q_pos || !bits || !item_off || !item_kvh || !item_page ||
      !item_qids || !item_size || !item_slot || !partial_o || !partial_lse || !out)
    return fail(PW_ERR_ARG, "pw_page_union_prefill: null required pointer");
  if (kv_dtype == PW_KV_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(PW_ERR_ARG, "pw_page_union_prefill: fp8 KV needs k_scale and v_scale");
  // KV heads run in batches of a few heads, so that a batch's partial rows (written by the
  // attention, read back by the merge) are mostly still in the 256 MB last-level cache.
  // When one head's partials alone exceed that, batching gains nothing: all heads at once.
  const int64_t part_per_head = (int64_t)nq * k_max * G * (d * 2 + 4);
  int hb = (int)std::min<int64_t>(hkv, (320ll << 20) / std::max<int64_t>(part_per_head, 1));
  if (hb < 2) hb = hkv;
  if (const char* e = getenv("PW_PAGE_HEAD_BATCH")) {
    const int v = atoi(e);
    if (v >= 1) hb = std::min(v, hkv);
  }
  for (int g0 = 0; g0 < hkv; g0 += hb) {
    const int g1 = std::min(hkv, g0 + hb);
    const int64_t cap = std::min<int64_t>(item_capacity,
                                          pw_page_items_capacity(nq, g1 - g0, k_max, n_pages, chunk));
    if (cap > 0) {
      pw::AttnArgs a{q, nq, hq, hkv, d, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_size,
                     n_pages, stride_head, stride_page, q_pos, kv_len, sm_scale, item_qids,
                     item_size, (int)cap, chunk, 0, nullptr, item_page, nullptr,
                     item_capacity, partial_o, partial_lse};
      a.item_kvh = item_kvh;
      a.item_lo_dev = item_off + (int64_t)g0 * n_pages;
      a.item_hi_dev = item_off + (int64_t)g1 * n_pages;
      a.out_slot = item_slot;
      const pw_status st = pw::launch_sparse_prefill(a, stream);
      if (st != PW_OK) return st;
    }
    const pw_status st = pw::launch_page_merge(bits, nq, hkv, g0, g1, G, d, n_pages, k_max,
                                               partial_o, partial_lse, out, lse, stream);
    if (st != PW_OK) return st;
  }
  return PW_OK;
}

// Host validation shared by the entry points that run the union attention kernel.
static pw_status check_sparse_prefill(const pw::AttnArgs& a, const char* who) {
  if (a.nq < 0 || a.hq < 1 || a.hkv < 1 || a.n_pages < 1 || a.n_groups < 0 || a.kv_len < 0 ||
      a.capacity < 0)
    return fail(PW_ERR_ARG, "%s: bad sizes nq=%d hq=%d hkv=%d n_pages=%d n_groups=%d kv_len=%d", who,
                a.nq, a.hq, a.hkv, a.n_pages, a.n_groups, a.kv_len);
  if (a.hq % a.hkv) return fail(PW_ERR_ARG, "%s: hq=%d not a multiple of hkv=%d", who, a.hq, a.hkv);
  // the kernel packs page + 1 into 24 bits of a lane register
  if (a.n_pages > (1 << 24) - 2) return fail(PW_ERR_UNSUPPORTED, "%s: n_pages=%d > 2^24 - 2", who, a.n_pages);
  if (a.d != 64 && a.d != 128) return fail(PW_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", who, a.d);
  if (a.page_size != 64 && a.page_size != 128)
    return fail(PW_ERR_UNSUPPORTED, "%s: page_size=%d (64 or 128)", who, a.page_size);
  if (a.kv_dtype != PW_KV_BF16 && a.kv_dtype != PW_KV_FP8_E4M3)
    return fail(PW_ERR_UNSUPPORTED, "%s: kv_dtype=%d", who, a.kv_dtype);
  // Member masks and explicit groups hold up to 8 members; consecutive groups over tables
  // without member masks (every member uses every page) may be wider.
  const bool wide_ok = a.group_qids == nullptr && a.union_qmask == nullptr;
  if (a.max_group < 1 || a.max_group > (wide_ok ? 256 : 8))
    return fail(PW_ERR_UNSUPPORTED, "%s: max_group=%d not in 1..%d", who, a.max_group,
                wide_ok ? 256 : 8);
  const int G = a.hq / a.hkv;
  const int max_rows = wide_ok ? pw::max_rows_per_item(a.d, a.kv_dtype) : 64;
  if ((int64_t)G * a.max_group > max_rows)
    return fail(PW_ERR_UNSUPPORTED, "%s: (hq/hkv)*max_group=%d > %d", who, G * a.max_group, max_rows);
  if (a.shared_table != 0 && a.shared_table != 1)
    return fail(PW_ERR_ARG, "%s: shared_table=%d (0 or 1)", who, a.shared_table);
  const int esz = a.kv_dtype == PW_KV_FP8_E4M3 ? 1 : 2;
  if (a.stride_page < (int64_t)a.page_size * a.d || a.stride_head < 0)
    return fail(PW_ERR_ARG, "%s: stride_page=%lld < page_size*d or stride_head < 0", who,
                (long long)a.stride_page);
  if ((a.stride_page * esz) % 16 || (a.stride_head * esz) % 16)
    return fail(PW_ERR_ARG, "%s: strides must be multiples of 16 bytes", who);
  if (((uintptr_t)a.q | (uintptr_t)a.k_cache | (uintptr_t)a.v_cache | (uintptr_t)a.out) % 16)
    return fail(PW_ERR_ARG, "%s: q, caches and out must be 16-byte aligned", who);
  if (!a.group_qids && a.n_groups * (int64_t)a.max_group < a.nq)
    return fail(PW_ERR_ARG, "%s: consecutive groups need n_groups*max_group >= nq", who);
  if ((int64_t)a.hkv * a.n_groups >= INT32_MAX / 8)
    return fail(PW_ERR_UNSUPPORTED, "%s: too many work items", who);
  if (!(a.sm_scale > 0.f) || a.sm_scale != a.sm_scale)
    return fail(PW_ERR_ARG, "%s: sm_scale must be positive", who);
  if (a.nq > 0 && a.n_groups > 0) {
    if (!a.q || !a.k_cache || !a.v_cache || !a.q_pos || !a.union_off || !a.out)
      return fail(PW_ERR_ARG, "%s: null required pointer", who);
    if (a.group_qids && !a.group_size)
      return fail(PW_ERR_ARG, "%s: group_size is required with group_qids", who);
    if (a.kv_dtype == PW_KV_FP8_E4M3 && (!a.k_scale || !a.v_scale))
      return fail(PW_ERR_ARG, "%s: fp8 KV needs k_scale and v_scale", who);
    if (a.capacity > 0 && !a.union_pages) return fail(PW_ERR_ARG, "%s: null union_pages", who);
  }
  return PW_OK;
}

pw_status pw_shared_table_prefill(const void* q, int nq, int hq, int hkv, int d,
                                  const void* k_cache, const void* v_cache, int kv_dtype,
                                  const float* k_scale, const float* v_scale, int page_size,
                                  int n_pages, int64_t stride_head, int64_t stride_page,
                                  const int32_t* q_pos, int kv_len, float sm_scale, int max_group,
                                  const int32_t* union_off, const int32_t* union_pages,
                                  int64_t capacity, int n_split, void* partial_o,
                                  float* partial_lse, void* out, float* lse, hipStream_t stream) {
  pw::g_err[0] = 0;
  if (n_split < 1 || n_split > 64)
    return fail(PW_ERR_UNSUPPORTED, "pw_shared_table_prefill: n_split=%d not in 1..64", n_split);
  if (max_group < 1) return fail(PW_ERR_ARG, "pw_shared_table_prefill: max_group=%d", max_group);
  const int n_groups = nq > 0 ? (nq + max_group - 1) / max_group : 0;
  if (n_split == 1)
    return pw_sparse_prefill(q, nq, hq, hkv, d, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                             page_size, n_pages, stride_head, stride_page, q_pos, kv_len, sm_scale,
                             nullptr, nullptr, n_groups, max_group, 1, union_off, union_pages,
                             nullptr, capacity, nullptr, out, lse, stream);
  if (hkv < 1 || hq < 1 || hq % hkv)
    return fail(PW_ERR_ARG, "pw_shared_table_prefill: hq=%d hkv=%d", hq, hkv);
  const int G = hq / hkv;
  if ((int64_t)n_split * G > 16384)
    return fail(PW_ERR_UNSUPPORTED, "pw_shared_table_prefill: n_split*(hq/hkv) > 16384");
  if ((int64_t)nq * hkv * n_split >= INT32_MAX)
    return fail(PW_ERR_UNSUPPORTED, "pw_shared_table_prefill: nq*hkv*n_split must stay below 2^31");
  if ((int64_t)hkv * n_groups * n_split >= INT32_MAX / 8)
    return fail(PW_ERR_UNSUPPORTED, "pw_shared_table_prefill: too many work items");
  if (nq > 0 && (!partial_o || !partial_lse))
    return fail(PW_ERR_ARG, "pw_shared_table_prefill: n_split > 1 needs partial_o and partial_lse");
  if ((uintptr_t)partial_o % 16)
    return fail(PW_ERR_ARG, "pw_shared_table_prefill: partial_o must be 16-byte aligned");
  // the attention's own validation (wide consecutive groups over shared tables), writing
  // the slice partials; then the lse merge into out / lse
  pw::AttnArgs a{q, nq, hq, hkv, d, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_size,
                 n_pages, stride_head, stride_page, q_pos, kv_len, sm_scale, nullptr, nullptr,
                 n_groups, max_group, 1, union_off, union_pages, nullptr, capacity, partial_o,
                 partial_lse};
  a.n_split = n_split;
  const pw_status st = check_sparse_prefill(a, "pw_shared_table_prefill");
  if (st != PW_OK || nq == 0) return st;
  if (!out) return fail(PW_ERR_ARG, "pw_shared_table_prefill: null out");
  if ((uintptr_t)out % 16) return fail(PW_ERR_ARG, "pw_shared_table_prefill: out must be 16-byte aligned");
  const pw_status st2 = pw::launch_sparse_prefill(a, stream);
  if (st2 != PW_OK) return st2;
  return pw::launch_page_merge(nullptr, nq, hkv, 0, hkv, G, d, n_pages, n_split, partial_o,
                               partial_lse, out, lse, stream);
}

pw_status pw_sparse_prefill(const void* q, int nq, int hq, int hkv, int d, const void* k_cache,
                            const void* v_cache, int kv_dtype, const float* k_scale,
                            const float* v_scale, int page_size, int n_pages, int64_t stride_head,
                            int64_t stride_page, const int32_t* q_pos, int kv_len, float sm_scale,
                            const int32_t* group_qids, const int32_t* group_size, int n_groups,
                            int max_group, int shared_table, const int32_t* union_off,
                            const int32_t* union_pages, const uint8_t* union_qmask,
                            int64_t capacity, const int32_t* item_order, void* out, float* lse,
                            hipStream_t stream) {
  pw::g_err[0] = 0;
  pw::AttnArgs a{q, nq, hq, hkv, d, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_size,
                 n_pages, stride_head, stride_page, q_pos, kv_len, sm_scale, group_qids, group_size,
                 n_groups, max_group, shared_table, union_off, union_pages, union_qmask, capacity,
                 out, lse};
  a.item_order = item_order;
  const pw_status st = check_sparse_prefill(a, "pw_sparse_prefill");
  if (st != PW_OK || nq == 0 || n_groups == 0) return st;
  if (item_order && shared_table)
    return fail(PW_ERR_ARG, "pw_sparse_prefill: item_order needs shared_table = 0");
  return pw::launch_sparse_prefill(a, stream);
}

pw_status pw_schedule_items(const int32_t* union_off, int n_items, int32_t* item_order,
                            hipStream_t stream) {
  pw::g_err[0] = 0;
  if (n_items < 0) return fail(PW_ERR_ARG, "pw_schedule_items: n_items=%d", n_items);
  if (n_items == 0) return PW_OK;
  if (!union_off || !item_order) return fail(PW_ERR_ARG, "pw_schedule_items: null pointer");
  return pw::launch_schedule(union_off, n_items, item_order, stream);
}

}  // extern "C"
