/* pw.h - query-union sparse-attention prefill on AMD Instinct MI355X (gfx950).
 *
 * Sparse prefill in which every query keeps its own TopK set of KV-cache
 * pages (its support), queries are grouped by selected-page affinity, each
 * group's page union is read once, and causal online-softmax attention runs
 * for every query over exactly its own pages, each output row written to the
 * query's original ID ("PageWeaver: KV-Guided Query Unions for Sparse
 * Attention", abstract and Figs. 1-3; "CompactAttention: Accelerating Chunked
 * Prefill with Block-Union KV Selection", summary "Approach").
 *
 * Conventions for every entry point
 *  - C ABI.  Arrays are row-major, sizes are int32 unless noted, and every
 *    array argument is a DEVICE pointer unless noted.
 *  - The caller allocates and frees every buffer.  The library keeps no device
 *    state between calls, never allocates device memory and never
 *    synchronises: each call validates its scalar arguments on the host,
 *    enqueues its kernels on `stream` (NULL = the null stream) and returns.
 *  - On any non-OK status nothing has been enqueued and outputs are untouched;
 *    pw_last_error() returns a thread-local message explaining why.
 *  - Support content rules (shared by every step): page IDs < 0 are empty
 *    slots, duplicate IDs collapse (a support is a set), IDs >= n_pages are
 *    ignored and counted (pw_page_bitsets).  A page wholly after a query's
 *    position is legal; its keys are causally masked.
 *  - Thread safety: calls are independent; the library has no global state
 *    other than the per-thread error text.
 */
#ifndef PW_H_
#define PW_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int pw_status;
#define PW_OK 0
#define PW_ERR_ARG (-1)         /* bad size, null pointer or inconsistent arguments   */
#define PW_ERR_UNSUPPORTED (-2) /* valid request outside what the kernels implement   */
#define PW_ERR_CAPACITY (-3)    /* an output buffer is smaller than its required size */
#define PW_ERR_HIP (-4)         /* a HIP launch or runtime call failed                */

/* KV cache element types. */
#define PW_KV_BF16 0     /* bfloat16                                                       */
#define PW_KV_FP8_E4M3 1 /* OCP fp8 E4M3 ("e4m3fn": bias 7, max 448, no inf) with an fp32
                            scale per (KV head, page) for K and for V; value = code*scale. */

/* ---- host helpers (no device work) ------------------------------------------------ */

/* Version string of the library. */
const char* pw_version(void);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* pw_last_error(void);

/* Debug builds (libpw_debug.so, compiled with -DPW_DEBUG): the kernels count every lane at
 * which an index or LDS-ring invariant does not hold (table offsets inside capacity and
 * ascending, listed pages valid, a tile's loads inside its ring stage, listed members
 * queries of the chunk, output rows in range, union entries within capacity, page-major
 * items within their bound), without trapping; this returns the count since the last call
 * and clears it (synchronous; -1 on a HIP error).  Release builds return -2.            */
int64_t pw_debug_violations(void);

/* 64-bit words per page bitset row: ceil(n_pages / 64). */
int pw_words(int n_pages);

/* Groups per KV head produced by pw_group: each window of `window`
 * consecutive query IDs yields ceil(len / max_group) groups.  -1 on bad args. */
int pw_num_groups(int nq, int window, int max_group);

/* Minimum `capacity` (entries) of union_pages / union_qmask for pw_union_tables:
 * n_tables * min(n_pages, group_width * k_max), where k_max bounds every row's
 * support size.  -1 on bad args. */
int64_t pw_union_capacity(int n_tables, int group_width, int k_max, int n_pages);

/* ---- (0) chunk K/V append ---------------------------------------------------------------
 * PageWeaver abstract (FP8 KV throughout, chunked prefill) and CompactAttention
 * "Approach" (attention in place over the paged, KV-head-major cache): the chunk's
 * keys and values enter the cache before it is attended.  Token t = first_token + i
 * goes to page t / page_size, slot t % page_size, of every KV head.
 *   bf16 cache: the bits are copied.
 *   fp8 cache, for K and V separately and every touched (KV head, page):
 *     a = max |x| over the chunk's tokens on the page;
 *     a page the chunk starts part way into (its earlier slots hold earlier tokens)
 *     keeps its scale when a/448 does not exceed it, else takes a/448 and has its
 *     earlier slots re-encoded from code * old scale; any other touched page takes
 *     a/448, or 1 when a == 0.  Codes are e4m3fn(clamp(x / scale, -448, 448)) with
 *     the correctly rounded fp32 quotient and round-to-nearest-even.
 *   Slots after the chunk's last token on its last page are zeroed, so that every
 *   slot of a page that attention reads holds a finite value.
 * Pages other than the touched ones are not accessed.
 *
 * k_new, v_new  bf16, token i of KV head g at element i*stride_tok + g*d, the d
 *               elements contiguous (e.g. slices of a fused QKV projection output)
 * k_cache, v_cache, page_size, n_pages, stride_head, stride_page: as in
 *               pw_sparse_prefill (elements of kv_dtype)
 * k_scale, v_scale  fp32 [hkv][n_pages], read and written (fp8 only, else NULL)
 * Non-finite inputs give unspecified codes (no fault).  Calls that overlap in time
 * on the same pages race.
 * Limits: n_tok >= 0, first_token >= 0, the chunk's last page < n_pages,
 *   n_pages * page_size < 2^31, 8 <= d <= 1024 with d % 8 == 0, stride_tok >= hkv*d
 *   and a multiple of 8, strides in bytes multiples of 16, pointers 16-byte aligned. */
pw_status pw_append_kv(const void* k_new, const void* v_new, int n_tok, int hkv, int d,
                       int64_t stride_tok, int first_token, void* k_cache, void* v_cache,
                       int kv_dtype, float* k_scale, float* v_scale, int page_size, int n_pages,
                       int64_t stride_head, int64_t stride_page, hipStream_t stream);

/* ---- (1) page bitsets -------------------------------------------------------------
 * PageWeaver Fig. 1: fixed TopK pages per query guide the regrouping.  Row r of
 * KV head g becomes a bitset with bit p set iff page p is in the support, built
 * by wavefront ballots (one 64-page word per ballot).
 *
 * topk          int32 [n_rows][hkv][k]         page IDs, -1 = empty slot
 * bits          uint64 [hkv][n_rows][pw_words(n_pages)]   output, bit p in word p/64
 * bad_id_count  int32 [1] or NULL: incremented once per ID >= n_pages (caller zeroes it)
 * Limits: n_rows >= 0, hkv >= 1, 1 <= k <= 4096, 1 <= n_pages <= 65536.            */
pw_status pw_page_bitsets(const int32_t* topk, int n_rows, int hkv, int k, int n_pages,
                          uint64_t* bits, int32_t* bad_id_count, hipStream_t stream);

/* ---- (2) bounded affinity grouping --------------------------------------------------
 * PageWeaver abstract and Figs. 1-2: a bounded GPU search over selected-page
 * affinity produces query IDs; original IDs keep support, position and output
 * address.  Rule: per KV head, disjoint windows of `window` consecutive query
 * IDs are grouped independently; the seed is the lowest ungrouped ID; the group
 * repeatedly takes the ungrouped candidate with the largest overlap
 * popcount(bits[c] & U) with its current union U (ties -> lower ID; zero
 * overlap still joins) until it has max_group members or the window is empty.
 *
 * bits        uint64 [hkv][nq][pw_words(n_pages)]  (from pw_page_bitsets)
 * group_qids  int32 [hkv][G][max_group] output, G = pw_num_groups(nq, window, max_group);
 *             members in pick order, -1 padded.  Groups are ordered by window,
 *             then creation.
 * group_size  int32 [hkv][G] output, 1..max_group.
 * Limits: 1 <= max_group <= 8, window % max_group == 0, window <= 1024,
 *         n_pages <= 4096.                                                          */
pw_status pw_group(const uint64_t* bits, int nq, int hkv, int n_pages, int window,
                   int max_group, int32_t* group_qids, int32_t* group_size, hipStream_t stream);

/* ---- (2b) members arranged for row tiles --------------------------------------------------
 * QUILT summary, "Cascaded Sharing": after the pages shared by a whole group, reuse is
 * sought inside smaller subgroups.  The attention skips work per row tile of 16 query-head
 * rows, i.e. per subgroup of 16/(hq/hkv) members, so the subgroups that matter are the
 * tiles: a page selected only inside one tile costs that tile alone.  For hq/hkv = 4 and
 * groups of 5..8 members (two tiles), this reorders each group's members so that the split
 * into [first 4 | rest] - the first tile holding the group's seed - has the smallest
 * |union of tile 1| + |union of tile 2|, ties to the first split in lexicographic order of
 * the seed's three partners' positions; each tile keeps its members' relative order.
 * The member-mask bits of the group's union entries are permuted to match, so the tables
 * stay consistent and the attention result is unchanged (bit for bit).  Other GQA ratios
 * and smaller groups: no-op.
 * bits, group_qids, group_size: as for pw_group (groups updated in place); union_off,
 * union_qmask, capacity: the tables pw_union_tables / pw_prepare wrote for these groups
 * (union_qmask updated in place; NULL: none).
 * Limits: 1 <= max_group <= 8, n_pages <= 65536.                                            */
pw_status pw_arrange_groups(const uint64_t* bits, int nq, int hkv, int n_pages, int hq,
                            int n_groups, int max_group, int32_t* group_qids,
                            const int32_t* group_size, const int32_t* union_off,
                            uint8_t* union_qmask, int64_t capacity, hipStream_t stream);

/* ---- (3) union tables -----------------------------------------------------------------
 * PageWeaver Fig. 2 (a group's union is visited once, members keep their own
 * pages) and CompactAttention "Approach" (Q-block and intra-group head unions
 * give a per-KV-group block table).  For every table e = g * n_groups + j the
 * union of the member rows' bitsets is listed in ascending page order, built by
 * popcount, prefix sum and compaction.
 *
 * bits         uint64 [hkv][n_rows][pw_words(n_pages)]
 * group_rows   int32 [hkv][n_groups][group_width]: row indices (-1 padded); member j
 *              of a table is group_rows[..][j].  NULL: consecutive groups, member j of
 *              table g * n_groups + i is row i * group_width + j (rows >= n_rows absent),
 *              the original-order groups of PageWeaver Fig. 2 (then n_groups * group_width
 *              >= n_rows is required)
 * group_size   int32 [hkv][n_groups] or NULL (then every table has group_width members)
 * union_off    int32 [hkv*n_groups + 1] output: exclusive prefix sum of union sizes
 * union_pages  int32 [capacity] output: pages of table e at [union_off[e], union_off[e+1])
 * union_qmask  uint8 [capacity] output or NULL: bit j set iff member j selected the page;
 *              requires group_width <= 8
 * capacity     entries available; must be >= pw_union_capacity(hkv*n_groups,
 *              group_width, k_max, n_pages).  Entries past capacity are never
 *              written (defensive clamp if k_max understated the supports).
 * Limits: 1 <= group_width <= 64, n_pages <= 65536.                                  */
pw_status pw_union_tables(const uint64_t* bits, int n_rows, int hkv, int n_pages,
                          const int32_t* group_rows, const int32_t* group_size, int n_groups,
                          int group_width, int k_max, int32_t* union_off, int32_t* union_pages,
                          uint8_t* union_qmask, int64_t capacity, hipStream_t stream);

/* ---- (1)+(2)+(3) fused ------------------------------------------------------------------
 * Exactly pw_page_bitsets(topk) followed by pw_group(bits) and
 * pw_union_tables(bits, group_rows = group_qids, group_size, group_width = max_group,
 * k_max = k, union_qmask): the same outputs, bit for bit, in fewer launches.  For
 * window <= 64 and n_pages <= 1024 one workgroup per (window, KV head) builds the
 * window's bitsets, groups it and sizes its unions (then a prefix sum and the union
 * listing follow); other shapes run the three steps.  Arguments and limits as in the
 * three calls; union_qmask is required; capacity >= pw_union_capacity(hkv*G,
 * max_group, k, n_pages) with G = pw_num_groups(nq, window, max_group).
 * item_order   int32 [hkv*G] output or NULL: when given, also the work order of
 *              pw_schedule_items(union_off, hkv*G, item_order), computed in the union
 *              listing's launch (the same values as the separate call).               */
pw_status pw_prepare(const int32_t* topk, int nq, int hkv, int k, int n_pages, int window,
                     int max_group, uint64_t* bits, int32_t* bad_id_count, int32_t* group_qids,
                     int32_t* group_size, int32_t* union_off, int32_t* union_pages,
                     uint8_t* union_qmask, int64_t capacity, int32_t* item_order,
                     hipStream_t stream);

/* The same for groups run as two halves (QUILT summary, "Cascaded Sharing": the subgroup
 * level of the sharing cascade): bitsets and groups exactly as pw_prepare, then the union
 * tables of each group's two halves instead of the group's - exactly
 * pw_union_tables(bits, group_rows = group_qids viewed as [hkv][2G][max_group/2],
 * group_size = NULL, n_groups = 2G, group_width = max_group/2, k_max = k, union_qmask):
 * table 2j + h lists the union of members [h*max_group/2, (h+1)*max_group/2) of group j
 * in pick order (absent members are -1 and skipped), with their member masks.  Run the
 * attention on these tables with group_qids viewed the same way, n_groups = 2G and
 * max_group/2 members per table.  max_group must be even; capacity >=
 * pw_union_capacity(2*hkv*G, max_group/2, k, n_pages); item_order, when given, has 2*hkv*G
 * entries (pw_schedule_items over the half tables).  Same fused launches as pw_prepare
 * for window <= 64 and n_pages <= 1024.                                                */
pw_status pw_prepare_halves(const int32_t* topk, int nq, int hkv, int k, int n_pages, int window,
                            int max_group, uint64_t* bits, int32_t* bad_id_count,
                            int32_t* group_qids, int32_t* group_size, int32_t* union_off,
                            int32_t* union_pages, uint8_t* union_qmask, int64_t capacity,
                            int32_t* item_order, hipStream_t stream);

/* ---- (4) ID-aware union attention -----------------------------------------------------
 * PageWeaver abstract, Fig. 1 and Fig. 3: each group's union pages are staged
 * on chip once; for every member the same lanes compute QK, the masked online
 * softmax and PV, keeping the member's state and writing its rows to its
 * original ID, with no reordered Q and no cross-page partial outputs.
 * CompactAttention "Approach": attention runs in place over the paged cache in
 * KV-head-major layout.
 *
 * Work item (g, j) = KV head g, group j: rows (member m, head h) for the
 * members m of the group and h in [g*G, (g+1)*G), G = hq / hkv.  For every union
 * page P of the item's table and every token t = P*page_size + s of it, key t
 * is used by member m iff m selected P (union_qmask bit, or always when
 * union_qmask is NULL), t <= q_pos[m] and t < kv_len.  Output
 *   out[m][h][:] = sum_t softmax_t(sm_scale * q[m][h] . K[g][t]) V[g][t]
 * rounded to bf16 (0 when no key is used), lse[m][h] = natural-log sum-exp
 * of the scaled scores (-inf when no key is used).
 *
 * q           bf16 [nq][hq][d]
 * k_cache     [hkv][*][page_size][d] element type kv_dtype; page P of head g at
 * v_cache       byte offset (g*stride_head + P*stride_page) * elem_size, the d
 *             elements of a token contiguous, tokens of a page contiguous
 * k_scale     fp32 [hkv][n_pages] (fp8 only, else NULL); same for v_scale
 * q_pos       int32 [nq] absolute position of each query
 * group_qids  int32 [hkv][n_groups][max_group] (-1 padded) or NULL: then group j
 *             is the consecutive IDs [j*max_group, min((j+1)*max_group, nq))
 * group_size  int32 [hkv][n_groups] (required iff group_qids != NULL)
 * shared_table 0: item (g, j) uses table g*n_groups + j;
 *             1: every item of KV head g uses table g (a per-KV-group block table)
 * union_off / union_pages / union_qmask: tables as written by pw_union_tables
 *             (union_qmask NULL = every member uses every page of its table)
 * capacity    entries in union_pages (reads are clamped to it)
 * item_order  int32 [hkv*n_groups] or NULL: the order the work items are started in,
 *             position r running item item_order[r] (see pw_schedule_items); must be a
 *             permutation of 0 .. hkv*n_groups-1 (entries out of range are skipped).  It
 *             changes no output bit.  Requires shared_table = 0.
 * out         bf16 [nq][hq][d]; each row written exactly once if it belongs to
 *             a group; rows of queries in no group are left untouched
 * lse         fp32 [nq][hq] or NULL
 * Precondition on the cache contents: every K and V slot of every page in a work
 * item's table - the slots at and past kv_len included - holds a finite value, with
 * scaled scores inside the fp32 range.  Keys a row does not use get probability 0,
 * but they still pass through the MFMAs of its 16-row tile, so a NaN or infinity
 * there (in a page only another member selected, or past the cache end) would reach
 * rows whose result does not depend on it; with finite contents such slots change no
 * bit of those rows.  pw_append_kv writes zeros into the slots after a chunk's last
 * token, so a cache filled by it meets the precondition.
 * Limits: d in {64, 128}; page_size in {64, 128}; hq % hkv == 0; 1 <= n_pages <= 2^24 - 2;
 *   with group_qids or union_qmask: 1 <= max_group <= 8 and G * max_group <= 64;
 *   with neither (consecutive groups, every member uses every page of its table -
 *   the dense form over a shared per-KV-group table): max_group <= 256 and
 *   G * max_group <= 256 rows (bf16, d=128), 128 (fp8 d=128, bf16 d=64), 64 (fp8 d=64).  */
pw_status pw_sparse_prefill(const void* q, int nq, int hq, int hkv, int d,
                            const void* k_cache, const void* v_cache, int kv_dtype,
                            const float* k_scale, const float* v_scale, int page_size,
                            int n_pages, int64_t stride_head, int64_t stride_page,
                            const int32_t* q_pos, int kv_len, float sm_scale,
                            const int32_t* group_qids, const int32_t* group_size, int n_groups,
                            int max_group, int shared_table, const int32_t* union_off,
                            const int32_t* union_pages, const uint8_t* union_qmask,
                            int64_t capacity, const int32_t* item_order, void* out, float* lse,
                            hipStream_t stream);

/* ---- (4a) work order for (4) ---------------------------------------------------------------
 * Not from the source pages: a scheduling aid for pw_sparse_prefill on this GPU.  Its
 * work items run in 8 consecutive ranges of ceil(n_items / 8) positions, one range per
 * XCD, started in position order; items differ in union size (the 64K fp8 Top16 workload:
 * 61 .. 113 pages), and when the large ones come last they set the end of the launch.
 * item_order lists every range's items by union size (union_off[e+1] - union_off[e]),
 * largest first, ties by lower item index; a range longer than 8192 keeps item order.
 *
 * union_off   int32 [n_items + 1] (from pw_union_tables / pw_prepare)
 * item_order  int32 [n_items] output, a permutation of 0 .. n_items-1
 * Limits: n_items >= 0.                                                                     */
pw_status pw_schedule_items(const int32_t* union_off, int n_items, int32_t* item_order,
                            hipStream_t stream);

/* ---- (4b) shared block tables with the table split across workgroups ---------------------
 * CompactAttention "Approach": with one block table per KV group (shared_table = 1 of
 * pw_sparse_prefill, consecutive groups, every member using every page of the table) the
 * work is dense paged attention, and a chunk has few query-head rows per KV group (a
 * 1024-query chunk: 256 work items of 128 rows), too few to fill the chip.  Here table g
 * is cut into n_split consecutive slices, one workgroup each, and the slices' partial
 * results - normalised rows and their lse, in partial row ((q*hkv + g)*n_split + s)*G +
 * (h - g*G) - are merged by lse into out / lse.  The result is the attention of
 * pw_sparse_prefill(shared_table = 1, group_qids = NULL, union_qmask = NULL).
 * Arguments as in pw_sparse_prefill; max_group as there (consecutive groups of
 * max_group queries, ceil(nq / max_group) groups).  n_split = 1 is pw_sparse_prefill
 * itself (partial buffers unused).
 * partial_o    workspace bf16 [nq*hq*n_split][d]
 * partial_lse  workspace fp32 [nq*hq*n_split]
 * Limits: as pw_sparse_prefill's wide form; 1 <= n_split <= 64.                           */
pw_status pw_shared_table_prefill(const void* q, int nq, int hq, int hkv, int d,
                                  const void* k_cache, const void* v_cache, int kv_dtype,
                                  const float* k_scale, const float* v_scale, int page_size,
                                  int n_pages, int64_t stride_head, int64_t stride_page,
                                  const int32_t* q_pos, int kv_len, float sm_scale, int max_group,
                                  const int32_t* union_off, const int32_t* union_pages,
                                  int64_t capacity, int n_split, void* partial_o,
                                  float* partial_lse, void* out, float* lse, hipStream_t stream);

/* ---- (4c) pw_shared_table_prefill allocating nothing -----------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Exactly pw_shared_table_prefill (the
 * same kernels, the same result bit for bit), but the slice partials live in a device array
 * that the library owns: pw_noalloc_scratch_bytes() = 32 MiB on each device the call runs
 * on (the current device, which must be the stream's), held until the process ends and
 * looked up once per device.  Arguments as pw_shared_table_prefill without partial_o and
 * partial_lse.  PW_ERR_CAPACITY, with nothing enqueued, when the partials - nq*hq*n_split
 * bf16 rows of d (rounded up to 256 bytes) plus nq*hq*n_split fp32 - exceed the array;
 * n_split = 1 uses none of it.  Every call on a device shares its array: calls that
 * overlap in time on one GPU race.  Nothing in it needs clearing (each call writes every
 * partial row before merging it).                                                        */
size_t pw_noalloc_scratch_bytes(void);
pw_status pw_shared_table_prefill_noalloc(const void* q, int nq, int hq, int hkv, int d,
                                          const void* k_cache, const void* v_cache, int kv_dtype,
                                          const float* k_scale, const float* v_scale, int page_size,
                                          int n_pages, int64_t stride_head, int64_t stride_page,
                                          const int32_t* q_pos, int kv_len, float sm_scale,
                                          int max_group, const int32_t* union_off,
                                          const int32_t* union_pages, int64_t capacity, int n_split,
                                          void* out, float* lse, hipStream_t stream);

/* ---- (5) direct KV-page union (page-major execution) -----------------------------------
 * PageWeaver abstract: the page-major alternative to query unions visits every
 * (KV head, page) once for all queries that selected it, and pays for it with
 * per-page partial results that must be reduced.  Work item = (KV head g, page P,
 * up to `chunk` consecutive queries of P's ascending list of selecting queries).
 * Every member's partial result - the causal softmax over P's usable keys,
 * normalised, with its lse - goes to slot (q*hkv + g)*k_max + rank, rank = the
 * position of P among the ascending pages of S(q, g); each row's partials are then
 * merged by their lse.  The result is the same attention as pw_sparse_prefill over
 * the same supports.
 *
 * Upper bound on the items pw_page_tables writes: min(E, ceil((E + hkv*n_pages*(chunk-1))
 * / chunk)) with E = nq*hkv*min(k_max, n_pages).  -1 on bad args.                      */
int64_t pw_page_items_capacity(int nq, int hkv, int k_max, int n_pages, int chunk);

/* Bytes of workspace pw_page_tables needs: the per-page query columns
 * (hkv*n_pages*ceil(nq/64) uint64) and a per-row rank table (hkv*nq*pw_words(n_pages)
 * int32).  0 on bad args.                                                                */
size_t pw_page_workspace_bytes(int nq, int hkv, int n_pages);

/* Page-major work items from support bitsets.
 * bits        uint64 [hkv][nq][pw_words(n_pages)] (from pw_page_bitsets)
 * k_max       bounds every support size (the TopK width); partial slots use it
 * workspace   device buffer of workspace_bytes >= pw_page_workspace_bytes(), 8-byte aligned
 * item_off    int32 [hkv*n_pages + 1] output: exclusive prefix sum of items per (g, P),
 *             KV-head-major; item_off[hkv*n_pages] = number of items N
 * item_kvh, item_page, item_size  int32 [item_capacity] outputs (first N written)
 * item_qids, item_slot  int32 [item_capacity][chunk] outputs: members (ascending IDs)
 *             and their partial slots, -1 padded
 * Limits: 1 <= chunk <= 64, n_pages <= 65536, nq*hkv*k_max < 2^31,
 *   item_capacity >= pw_page_items_capacity(...).                                        */
pw_status pw_page_tables(const uint64_t* bits, int nq, int hkv, int n_pages, int k_max, int chunk,
                         void* workspace, size_t workspace_bytes, int32_t* item_off,
                         int32_t* item_kvh, int32_t* item_page, int32_t* item_qids,
                         int32_t* item_size, int32_t* item_slot, int64_t item_capacity,
                         hipStream_t stream);

/* Attention through page-major items, then the lse merge.  Arguments q .. sm_scale,
 * out and lse as in pw_sparse_prefill (every row of out/lse is written); bits, k_max,
 * chunk and the item arrays as given to / written by pw_page_tables.
 * partial_o    workspace bf16 [nq*hkv*k_max*(hq/hkv)][d]: normalised partial rows
 * partial_lse  workspace fp32 [nq*hkv*k_max*(hq/hkv)]
 * Limits: d in {64, 128}; page_size in {64, 128}; 1 <= chunk <= 64 and
 *   (hq/hkv)*chunk <= 256 rows (bf16, d=128), 128 (fp8 d=128, bf16 d=64), 64 (fp8 d=64);
 *   k_max*(hq/hkv) <= 16384.                                                              */
pw_status pw_page_union_prefill(const void* q, int nq, int hq, int hkv, int d, const void* k_cache,
                                const void* v_cache, int kv_dtype, const float* k_scale,
                                const float* v_scale, int page_size, int n_pages,
                                int64_t stride_head, int64_t stride_page, const int32_t* q_pos,
                                int kv_len, float sm_scale, const uint64_t* bits, int k_max,
                                int chunk, const int32_t* item_off, const int32_t* item_kvh,
                                const int32_t* item_page, const int32_t* item_qids,
                                const int32_t* item_size, const int32_t* item_slot,
                                int64_t item_capacity, void* partial_o, float* partial_lse,
                                void* out, float* lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PW_H_ */
