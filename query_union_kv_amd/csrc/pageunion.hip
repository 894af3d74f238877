// Direct KV-page union on gfx950: page-major work items and the lse merge.
//
// Method: "PageWeaver: KV-Guided Query Unions for Sparse Attention" (abstract):
// besides query unions, the page-major alternative visits every (KV head, page)
// once for all the queries that selected it, at the price of per-page partial
// results that must be reduced.  Here each work item is (KV head g, page P, up
// to `chunk` consecutive queries of P's ascending query list); the union
// attention kernel runs it as a one-page table and writes every member's
// normalised partial row and its lse to the slot (query, g, rank of P in the
// query's support); k_page_merge then combines each row's partials.
//
//   k_page_transpose  64x64 bit tiles of the support bitsets transposed by 64
//                     wavefront ballots into per-page query columns
//   k_page_count      items per (g, P) = ceil(|column| / chunk)
//   k_row_prefix      per-row popcount prefix, for the rank of a page in a support
//   (prefix sum)      item offsets
//   k_page_members    one wave per item: its KV head, page, member IDs, size, slots
//   k_page_merge      lse-weighted sum of each row's partials
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace pw {

PW_DEBUG_COUNTER_DEFINE(debug_count_pageunion)

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x - v;
}

// grid (words, qwords, hkv), one wave: lane i holds word w of query 64*qb + i; ballot j
// collects bit j of every lane, i.e. the 64 queries' flags for page 64*w + j.
__global__ __launch_bounds__(64) void k_page_transpose(const uint64_t* __restrict__ bits, int nq,
                                                       int words, int n_pages, int qwords,
                                                       uint64_t* __restrict__ cols) {
  const int lane = threadIdx.x;
  const int w = blockIdx.x, qb = blockIdx.y, g = blockIdx.z;
  const int q = qb * kWave + lane;
  const uint64_t row = q < nq ? bits[((int64_t)g * nq + q) * words + w] : 0ull;
  uint64_t mine = 0;
#pragma unroll
  for (int j = 0; j < kWave; ++j) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(((row >> j) & 1ull) != 0);
    if (lane == j) mine = m;
  }
  const int page = w * kWave + lane;
  if (page < n_pages) cols[((int64_t)g * n_pages + page) * qwords + qb] = mine;
}

// One wave per (g, P): number of queries in the column -> item count at item_off[gp + 1].
__global__ __launch_bounds__(256) void k_page_count(const uint64_t* __restrict__ cols, int n_gp,
                                                    int qwords, int chunk,
                                                    int32_t* __restrict__ item_off) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gp = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gp >= n_gp) return;
  int c = 0;
  for (int w = lane; w < qwords; w += kWave) c += __popcll(cols[(int64_t)gp * qwords + w]);
  c = wave_sum(c);
  if (lane == 0) item_off[gp + 1] = (c + chunk - 1) / chunk;
}

// Rank table: pre[g][q][w] = number of support pages of (q, g) in words 0..w-1, so that
// the rank of page P in S(q, g) is pre[g][q][P/64] + popcount(word P/64 below P).
__global__ __launch_bounds__(256) void k_row_prefix(const uint64_t* __restrict__ bits, int rows,
                                                    int words, int32_t* __restrict__ pre) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  int c = 0;
  for (int w = 0; w < words; ++w) {
    pre[(int64_t)r * words + w] = c;
    c += __popcll(bits[(int64_t)r * words + w]);
  }
}

// Position of the n-th set bit (0-based) of x; x has more than n set bits.
__device__ __forceinline__ int nth_set_bit(uint64_t x, int n) {
  int pos = 0;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const uint64_t lo = x & ((1ull << s) - 1ull);
    const int c = __popcll(lo);
    if (n >= c) {
      n -= c;
      x >>= s;
      pos += s;
    } else {
      x = lo;
    }
  }
  return pos;
}

// One wave per work item (grid: an upper bound; waves past the device item count exit).
// The item's column (g, P) is found by binary search over item_off; lane m takes entry
// e = (it - item_off[gp]) * chunk + m of the column: the word holding it comes from a
// binary search over the lanes' inclusive popcount prefix, the query from the word's
// set bits.  Slot = (q * hkv + g) * k_max + rank (rank >= k_max: slot -1; k_max bounds
// every support size, so this does not happen for bitsets of k_max-wide TopK rows).
__global__ __launch_bounds__(256) void k_page_members(
    const uint64_t* __restrict__ bits, const uint64_t* __restrict__ cols,
    const int32_t* __restrict__ pre, int nq, int hkv, int words, int n_pages, int qwords,
    int chunk, int k_max, const int32_t* __restrict__ item_off, int64_t item_capacity,
    int32_t* __restrict__ item_kvh, int32_t* __restrict__ item_page,
    int32_t* __restrict__ item_qids, int32_t* __restrict__ item_size,
    int32_t* __restrict__ item_slot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n_gp = hkv * n_pages;
  const int it = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int n_items = item_off[n_gp];
  PW_DCHECK(it != 0 || n_items <= item_capacity);   // the host's item bound held
  if (it >= n_items || it >= item_capacity) return;
  int lo = 0, hi = n_gp;            // last gp with item_off[gp] <= it
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (item_off[mid] <= it) lo = mid; else hi = mid;
  }
  const int gp = lo;
  const int g = gp / n_pages, page = gp - g * n_pages;
  const int e0 = (it - item_off[gp]) * chunk;
  const int pw = page >> 6;
  const uint64_t below = (1ull << (page & 63)) - 1ull;
  int base = 0;
  for (int w0 = 0; w0 < qwords; w0 += kWave) {
    const uint64_t cw = w0 + lane < qwords ? cols[(int64_t)gp * qwords + w0 + lane] : 0ull;
    const int c = __popcll(cw);
    const int incl = wave_excl_scan(c, lane) + c;
    const int tot = __shfl(incl, kWave - 1, kWave);
    for (int m0 = 0; m0 < chunk; m0 += kWave) {
      const int m = m0 + lane;
      const int e = e0 + m - base;                       // entry index inside this block
      const bool mine = m < chunk && e >= 0 && e < tot;
      int wl = 0, wh = kWave - 1;                        // number of lanes with incl <= e
      for (int s = 0; s < 6; ++s) {
        const int mid = (wl + wh + 1) >> 1;
        const int im = __shfl(incl, mid > 0 ? mid - 1 : 0, kWave);
        if (mid == 0 || im <= e) wl = mid; else wh = mid - 1;
      }
      const int w = wl;
      const uint64_t word = __shfl(cw, w, kWave);
      const int before = __shfl(incl, w, kWave) - __popcll(word);
      if (mine) {
        const int q = (w0 + w) * kWave + nth_set_bit(word, e - before);
        const int64_t row = (int64_t)g * nq + q;
        const int rank = pre[row * words + pw] + __popcll(bits[row * words + pw] & below);
        item_qids[(int64_t)it * chunk + m] = q;
        item_slot[(int64_t)it * chunk + m] = rank < k_max ? (q * hkv + g) * k_max + rank : -1;
      }
    }
    base += tot;
  }
  const int size = min(chunk, base - e0);
  for (int m = size + lane; m < chunk; m += kWave) {
    item_qids[(int64_t)it * chunk + m] = -1;
    item_slot[(int64_t)it * chunk + m] = -1;
  }
  if (lane == 0) {
    item_kvh[it] = g;
    item_page[it] = page;
    item_size[it] = size;
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ void k_fill_i32(int32_t* __restrict__ p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// One wave per (query, KV head).  Row (q, h) has partials at slots
// (q * hkv + g) * k_max + r, r < min(|S(q, g)|, k_max) (r < k_max when bits is NULL);
// partial row = slot * G + (h - gG).
//   lse = log sum_r exp(lse_r),  out = sum_r exp(lse_r - lse) * o_r
// Rows without usable keys (every lse_r = -inf, or no partials) get 0 and -inf.
// Dynamic LDS: k_max * G floats per wave (the weights).
template <int D>
__global__ __launch_bounds__(64) void k_page_merge(
    const uint64_t* __restrict__ bits, int nq, int hkv, int g0, int hb, int G, int words, int k_max,
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float wts[];
  const int lane = threadIdx.x;
  const int qg = blockIdx.x;                   // KV heads g0 .. g0 + hb - 1
  const int q = qg / hb, g = g0 + (qg - q * hb);
  if (q >= nq) return;
  int n = k_max;            // bits == NULL: every one of the k_max slots holds a partial
  if (bits) {
    const uint64_t* row = bits + ((int64_t)g * nq + q) * words;
    n = 0;
    for (int w = lane; w < words; w += kWave) n += __popcll(row[w]);
    n = min(wave_sum(n), k_max);
  }
  const int64_t slot0 = ((int64_t)q * hkv + g) * k_max;
  const int hq = hkv * G;
  for (int i = lane; i < n * G; i += kWave) wts[i] = part_lse[slot0 * G + i];
  __syncthreads();
  // each lane owns head columns h = lane, lane + 64, ... of the weights: their lse, then
  // their weights in place (no other lane touches them)
  for (int h = lane; h < G; h += kWave) {
    float row_lse = -INFINITY;
    float m = -INFINITY;
    for (int r = 0; r < n; ++r) m = fmaxf(m, wts[r * G + h]);
    if (m != -INFINITY) {
      float s = 0.f;
      for (int r = 0; r < n; ++r) s += __expf(wts[r * G + h] - m);
      row_lse = m + __logf(s);
    }
    for (int r = 0; r < n; ++r)
      wts[r * G + h] = row_lse == -INFINITY ? 0.f : __expf(wts[r * G + h] - row_lse);
    if (lse) lse[(int64_t)q * hq + g * G + h] = row_lse;
  }
  __syncthreads();
  constexpr int kC = D / 8;   // 8-element chunks per head row
  for (int c = lane; c < G * kC; c += kWave) {
    const int hl = c / kC, e0 = (c - hl * kC) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* src = part_o + (slot0 * G + hl) * D + e0;
    // every partial row below n was written (a page without usable keys has o = 0 and
    // weight 0), so the loads need no guard; batches of 8 keep them all in flight
    for (int r0 = 0; r0 < n; r0 += 8) {
      bf16x8 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r0 + i < n) v[i] = *reinterpret_cast<const bf16x8*>(src + (int64_t)(r0 + i) * G * D);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (r0 + i >= n) break;
        const float w = wts[(r0 + i) * G + hl];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += w * (float)v[i][k];
      }
    }
    bf16x8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (__bf16)acc[k];
    *reinterpret_cast<bf16x8*>(out + ((int64_t)q * hq + g * G + hl) * D + e0) = o;
  }
}

}  // namespace

size_t page_workspace_bytes(int nq, int hkv, int n_pages) {
  const int64_t qwords = (nq + 63) / 64, words = (n_pages + 63) / 64;
  const int64_t cols = (int64_t)hkv * n_pages * qwords * 8;
  return (size_t)(cols + (int64_t)hkv * nq * words * 4);
}

pw_status launch_page_tables(const uint64_t* bits, int nq, int hkv, int n_pages, int k_max,
                             int chunk, void* workspace, int32_t* item_off, int32_t* item_kvh,
                             int32_t* item_page, int32_t* item_qids, int32_t* item_size,
                             int32_t* item_slot, int64_t item_capacity, hipStream_t stream) {
  const int words = (n_pages + 63) / 64;
  const int qwords = (nq + 63) / 64;
  const int n_gp = hkv * n_pages;
  uint64_t* cols = (uint64_t*)workspace;
  int32_t* pre = (int32_t*)((char*)workspace + (size_t)n_gp * qwords * 8);
  if (nq > 0) {
    hipLaunchKernelGGL(k_page_transpose, dim3(words, qwords, hkv), dim3(64), 0, stream, bits, nq,
                       words, n_pages, qwords, cols);
    hipLaunchKernelGGL(k_page_count, dim3((n_gp + 3) / 4), dim3(256), 0, stream, cols, n_gp,
                       qwords, chunk, item_off);
    hipLaunchKernelGGL(k_row_prefix, dim3((hkv * nq + 255) / 256), dim3(256), 0, stream, bits,
                       hkv * nq, words, pre);
  } else {
    hipLaunchKernelGGL(k_fill_i32, dim3((n_gp + 255) / 256), dim3(256), 0, stream, item_off + 1,
                       n_gp, 0);
  }
  pw_status st = launch_scan(item_off, n_gp, stream);
  if (st != PW_OK || nq == 0 || item_capacity == 0) return st;
  hipLaunchKernelGGL(k_page_members, dim3((unsigned)((item_capacity + 3) / 4)), dim3(256), 0, stream,
                     bits, cols, pre, nq, hkv, words, n_pages, qwords, chunk, k_max, item_off,
                     item_capacity, item_kvh, item_page, item_qids, item_size, item_slot);
  return check_launch("pw_page_tables");
}

pw_status launch_page_merge(const uint64_t* bits, int nq, int hkv, int g0, int g1, int G, int d,
                            int n_pages, int k_max, const void* part_o, const float* part_lse,
                            void* out, float* lse, hipStream_t stream) {
  const int words = (n_pages + 63) / 64;
  const size_t lds = (size_t)k_max * G * sizeof(float);
  const int hb = g1 - g0;
  const dim3 grid((unsigned)((int64_t)nq * hb));
  if (d == 128)
    hipLaunchKernelGGL(k_page_merge<128>, grid, dim3(64), lds, stream, bits, nq, hkv, g0, hb, G,
                       words, k_max, (const uint16_t*)part_o, part_lse, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL(k_page_merge<64>, grid, dim3(64), lds, stream, bits, nq, hkv, g0, hb, G,
                       words, k_max, (const uint16_t*)part_o, part_lse, (uint16_t*)out, lse);
  return check_launch("pw_page_union_prefill (merge)");
}

}  // namespace pw
