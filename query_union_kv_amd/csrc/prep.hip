// Preparation kernels for query-union execution on gfx950 (wave64):
//   page bitsets   -- wavefront ballots over LDS page flags
//   grouping       -- bounded greedy affinity search, one workgroup per (KV head, window)
//   union tables   -- OR + popcount, prefix sum, compaction into ascending page lists
//
// Method: "PageWeaver: KV-Guided Query Unions for Sparse Attention" (abstract,
// Figs. 1-2): fixed TopK pages per query, a bounded GPU search over
// selected-page affinity that returns query IDs, and per-group page unions
// whose members keep their own supports.  "CompactAttention" (summary,
// "Approach"): unions across Q-blocks and heads of a KV group give one block
// table per KV group; the union kernels build both.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace pw {

PW_DEBUG_COUNTER_DEFINE(debug_count_prep)

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, kWave));
  return v;
}
// Exclusive prefix sum across the wave (lane order).
__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x - v;
}
// Makes this wave's earlier LDS writes visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------------------
// (1) page bitsets.  Each wave owns an LDS flag array of `words*64` bytes, one byte per
// page.  For a row, lanes holding valid IDs set their page's flag; then for every 64-page
// word the wave reads 64 consecutive flags (lane l <-> page 64w + l) and one ballot is the
// word.  Flags are cleared as they are read, so the array is zero again for the next row.
// Duplicate IDs write the same flag; negative IDs are skipped; IDs >= n_pages are counted.
// MAXW > 0 bounds the word count at compile time, so every flag read of a row is issued
// before the first ballot waits on it; MAXW == 0 is the general loop.
template <int MAXW>
__global__ void k_page_bitsets(const int32_t* __restrict__ topk, int n_rows, int hkv, int k,
                               int n_pages, int words, uint64_t* __restrict__ bits,
                               int32_t* __restrict__ bad_id_count) {
  extern __shared__ uint8_t flags_all[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int waves = blockDim.x / kWave;
  uint8_t* flags = flags_all + (size_t)wave * words * kWave;
  for (int i = lane * 16; i < words * kWave; i += kWave * 16)
    *reinterpret_cast<uint4*>(flags + i) = make_uint4(0, 0, 0, 0);
  wave_lds_sync();

  const int64_t total = (int64_t)n_rows * hkv;
  int bad = 0;
  for (int64_t item = (int64_t)blockIdx.x * waves + wave; item < total;
       item += (int64_t)gridDim.x * waves) {
    const int g = (int)(item / n_rows);
    const int r = (int)(item - (int64_t)g * n_rows);
    const int32_t* ids = topk + ((int64_t)r * hkv + g) * k;
    for (int j = lane; j < k; j += kWave) {
      const int id = ids[j];
      if (id >= n_pages) ++bad;
      else if (id >= 0) flags[id] = 1;
    }
    wave_lds_sync();
    uint64_t* dst = bits + item * words;   // item = g * n_rows + r
    if constexpr (MAXW > 0) {
      uint8_t f[MAXW];
#pragma unroll
      for (int w = 0; w < MAXW; ++w) f[w] = w < words ? flags[w * kWave + lane] : 0;
      uint64_t mine = 0;
#pragma unroll
      for (int w = 0; w < MAXW; ++w) {
        const uint64_t word = __ballot(f[w] != 0);
        if (lane == w) mine = word;
      }
#pragma unroll
      for (int w = 0; w < MAXW; ++w)
        if (w < words) flags[w * kWave + lane] = 0;
      if (lane < words) dst[lane] = mine;
    } else {
      uint64_t mine = 0;
      for (int w = 0; w < words; ++w) {
        const bool f = flags[w * kWave + lane] != 0;
        const uint64_t word = __ballot(f);
        flags[w * kWave + lane] = 0;
        if (lane == (w & (kWave - 1))) mine = word;
        if ((w & (kWave - 1)) == kWave - 1 || w == words - 1) {
          const int base = w & ~(kWave - 1);
          if (lane <= w - base) dst[base + lane] = mine;
        }
      }
    }
    wave_lds_sync();
  }
  bad = wave_sum(bad);
  if (bad_id_count != nullptr && lane == 0 && bad > 0) atomicAdd(bad_id_count, bad);
}

// ---------------------------------------------------------------------------------------
// (2) bounded greedy affinity grouping.  One workgroup per (window, KV head); thread c is
// candidate query start + c and keeps its bitset in registers (MAXW words).  The group
// union U lives in LDS.  Every pick is a workgroup argmax over the key
// (overlap << 11) | (2047 - c), so equal overlaps resolve to the lower query ID.
template <int MAXW>
__global__ void k_group(const uint64_t* __restrict__ bits, int nq, int words, int window,
                        int max_group, int n_groups, int32_t* __restrict__ group_qids,
                        int32_t* __restrict__ group_size) {
  __shared__ uint64_t U[MAXW];
  __shared__ int red[16];
  const int g = blockIdx.y;
  const int start = blockIdx.x * window;
  const int len = min(window, nq - start);
  const int c = threadIdx.x;
  const int lane = c & (kWave - 1), wave = c / kWave;
  const int nwaves = blockDim.x / kWave;
  const bool valid = c < len;

  uint64_t mine[MAXW];
  const uint64_t* row = bits + ((int64_t)g * nq + start + c) * words;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) mine[w] = (valid && w < words) ? row[w] : 0ull;

  auto block_max = [&](int v) -> int {
    v = wave_max(v);
    if (nwaves > 1) {
      if (lane == 0) red[wave] = v;
      __syncthreads();
      int r = red[0];
      for (int i = 1; i < nwaves; ++i) r = max(r, red[i]);
      __syncthreads();
      v = r;
    }
    return v;
  };

  bool is_free = valid;
  int remaining = len;
  int gi = 0;
  const int64_t gbase = (int64_t)g * n_groups + (int64_t)blockIdx.x * (window / max_group);
  while (remaining > 0) {
    // seed: the lowest ungrouped ID (max of 2047 - c over free lanes)
    const int seed = 2047 - block_max(is_free ? 2047 - c : -1);
    if (c == seed) {
      is_free = false;
#pragma unroll
      for (int w = 0; w < MAXW; ++w) if (w < words) U[w] = mine[w];
    }
    __syncthreads();
    int members[8];
    members[0] = seed;
    int cnt = 1;
    --remaining;
    while (cnt < max_group && remaining > 0) {
      int score = 0;
#pragma unroll
      for (int w = 0; w < MAXW; ++w)
        if (w < words) score += __popcll(mine[w] & U[w]);
      const int best = block_max(is_free ? ((score << 11) | (2047 - c)) : -1);
      const int pick = 2047 - (best & 2047);
      __syncthreads();                       // every lane has read U before it changes
      if (c == pick) {
        is_free = false;
#pragma unroll
        for (int w = 0; w < MAXW; ++w) if (w < words) U[w] |= mine[w];
      }
      __syncthreads();
#pragma unroll
      for (int j = 1; j < 8; ++j) if (j == cnt) members[j] = pick;
      ++cnt;
      --remaining;
    }
    if (c < max_group) {
      int v = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) if (j == c && j < cnt) v = start + members[j];
      group_qids[(gbase + gi) * max_group + c] = v;
    }
    if (c == 0) group_size[gbase + gi] = cnt;
    ++gi;
  }
}

// Wave-wide maximum by DPP: row_shr 1/2/4/8 gives every 16-lane row its maximum in
// lane 15, row_bcast 15/31 folds the rows into lane 63, which is read back.
__device__ __forceinline__ int wave_max_dpp(int v) {
  constexpr int kLow = -2147483647 - 1;
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// Same search for windows of at most 64 candidates: one wave per (window, KV head), the
// group union U held in scalar registers (wave-uniform), candidates' bitsets in their
// lanes, the free set as a 64-bit lane mask, and the argmax key (overlap << 6 | 63 - c)
// reduced with DPP.  No LDS and no barriers on the pick chain.
template <int MAXW>
__global__ __launch_bounds__(64) void k_group_wave(const uint64_t* __restrict__ bits, int nq,
                                                   int words, int window, int max_group,
                                                   int n_groups, int32_t* __restrict__ group_qids,
                                                   int32_t* __restrict__ group_size) {
  const int g = blockIdx.y;
  const int start = blockIdx.x * window;
  const int len = min(window, nq - start);
  const int c = threadIdx.x;
  const bool valid = c < len;
  uint32_t lo[MAXW], hi[MAXW];
  const uint64_t* row = bits + ((int64_t)g * nq + start + c) * words;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    const uint64_t x = (valid && w < words) ? row[w] : 0ull;
    lo[w] = (uint32_t)x;
    hi[w] = (uint32_t)(x >> 32);
  }
  uint64_t free_mask = __ballot(valid);
  const int64_t gbase = (int64_t)g * n_groups + (int64_t)blockIdx.x * (window / max_group);
  int gi = 0;
  while (free_mask) {
    const int seed = __builtin_ctzll(free_mask);           // lowest ungrouped ID
    free_mask &= free_mask - 1;
    uint32_t ulo[MAXW], uhi[MAXW];
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      ulo[w] = __builtin_amdgcn_readlane(lo[w], seed);
      uhi[w] = __builtin_amdgcn_readlane(hi[w], seed);
    }
    int members[8];
    members[0] = seed;
    int cnt = 1;
    while (cnt < max_group && free_mask) {
      int score = 0;   // words past `words` are zero in every lane: no bound checks needed
#pragma unroll
      for (int w = 0; w < MAXW; ++w)
        score += __builtin_popcount(lo[w] & ulo[w]) + __builtin_popcount(hi[w] & uhi[w]);
      const bool is_free = (free_mask >> c) & 1ull;
      const int best = wave_max_dpp(is_free ? ((score << 6) | (63 - c)) : -1);
      const int pick = 63 - (best & 63);
      free_mask &= ~(1ull << pick);
#pragma unroll
      for (int w = 0; w < MAXW; ++w) {
        ulo[w] |= __builtin_amdgcn_readlane(lo[w], pick);
        uhi[w] |= __builtin_amdgcn_readlane(hi[w], pick);
      }
#pragma unroll
      for (int j = 1; j < 8; ++j) if (j == cnt) members[j] = pick;
      ++cnt;
    }
    if (c < max_group) {
      int v = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) if (j == c && j < cnt) v = start + members[j];
      group_qids[(gbase + gi) * max_group + c] = v;
    }
    if (c == 0) group_size[gbase + gi] = cnt;
    ++gi;
  }
}

// ---------------------------------------------------------------------------------------
// Fused preparation for windows of at most 64 queries and at most 1024 pages: one
// workgroup per (window, KV head) builds the window's bitsets, runs the bounded greedy
// grouping and writes every group's union size, so only the prefix sum and the union
// listing remain.  Results are identical to the three separate steps.
//  * bitsets: the window's rows live in LDS (64 x 1024 bits); every valid ID sets its bit
//    with an LDS atomic OR, and the rows are copied out to `bits`;
//  * grouping: wave v scores words [2v, 2v+2) of every candidate (lane = candidate) and the
//    partial overlaps are summed through LDS, so the pick chain is split over up to eight
//    waves; the argmax key and the union U follow the single-wave search exactly.
//    (Measured on the 64K fp8 Top16 tables: one wave per window took 7 us longer and two
//    waves 11 us longer than four; eight match four there and gain 3 us where a window
//    spans four words.)
//  * with `halves` set, each group's two halves - members [0, mg/2) and [mg/2, mg) in pick
//    order - get a table each (tables 2j and 2j + 1 for group j): the union of the first
//    half is U as it stood when the half was complete, the second half's union is
//    accumulated from its own members.
constexpr int kFusedWordsPerWave = 2;
constexpr int kFusedMaxWaves = 16 / kFusedWordsPerWave;   // 1024 pages
static_assert(kFusedMaxWaves == 8, "the partial scores are summed as a tree of eight");

__global__ __launch_bounds__(64 * kFusedMaxWaves) void k_prepare(
    const int32_t* __restrict__ topk, int nq, int hkv, int k, int n_pages, int words, int window,
    int max_group, int n_groups, uint64_t* __restrict__ bits, int32_t* __restrict__ bad_id_count,
    int32_t* __restrict__ group_qids, int32_t* __restrict__ group_size,
    int32_t* __restrict__ union_count, int halves) {
  __shared__ uint32_t rows[64][33];                    // +1 dword per row against bank conflicts
  // per-candidate partial scores of the (up to 8) waves, wave-major so that the writes
  // and the reads (stride 64 dwords) are free of bank conflicts; two buffers, alternating
  // per pick, so one barrier per pick suffices
  __shared__ int part[2][kFusedMaxWaves][64];
  __shared__ int usz_acc[128];  // union size of each of the window's (<= 64) groups or halves
  const int g = blockIdx.y;
  const int start = blockIdx.x * window;
  const int len = min(window, nq - start);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;

  for (int i = tid; i < 64 * 33; i += blockDim.x) (&rows[0][0])[i] = 0u;
  __syncthreads();
  int bad = 0;
  for (int idx = tid; idx < len * k; idx += blockDim.x) {
    const int c = idx / k;
    const int id = topk[((int64_t)(start + c) * hkv + g) * k + (idx - c * k)];
    if (id >= n_pages) ++bad;
    else if (id >= 0) atomicOr(&rows[c][id >> 5], 1u << (id & 31));
  }
  bad = wave_sum(bad);
  if (bad_id_count != nullptr && lane == 0 && bad > 0) atomicAdd(bad_id_count, bad);
  __syncthreads();
  for (int idx = tid; idx < len * words; idx += blockDim.x) {
    const int c = idx / words;
    const int w = idx - c * words;
    bits[((int64_t)g * nq + start + c) * words + w] =
        (uint64_t)rows[c][2 * w] | ((uint64_t)rows[c][2 * w + 1] << 32);
  }

  // this wave's slice of the candidates' bitsets (zero past `words` and past `len`)
  uint32_t lo[kFusedWordsPerWave], hi[kFusedWordsPerWave];
#pragma unroll
  for (int i = 0; i < kFusedWordsPerWave; ++i) {
    const int w = wave * kFusedWordsPerWave + i;
    const bool ok = lane < len && w < words;
    lo[i] = ok ? rows[lane][2 * w] : 0u;
    hi[i] = ok ? rows[lane][2 * w + 1] : 0u;
  }
  uint64_t free_mask = __ballot(lane < len);
  const int64_t gbase = (int64_t)g * n_groups + (int64_t)blockIdx.x * (window / max_group);
  int gi = 0;
  int pb = 0;   // partial-score buffer of the next pick
  if (nwaves > 1)
    for (int i = tid; i < 2 * 64 * kFusedMaxWaves; i += blockDim.x) (&part[0][0][0])[i] = 0;
  for (int i = tid; i < 128; i += blockDim.x) usz_acc[i] = 0;
  const int half_w = halves ? max_group / 2 : max_group;   // members in the first half
  __syncthreads();
  while (free_mask) {
    const int seed = __builtin_ctzll(free_mask);
    free_mask &= free_mask - 1;
    uint32_t ulo[kFusedWordsPerWave], uhi[kFusedWordsPerWave];
#pragma unroll
    for (int i = 0; i < kFusedWordsPerWave; ++i) {
      ulo[i] = __builtin_amdgcn_readlane(lo[i], seed);
      uhi[i] = __builtin_amdgcn_readlane(hi[i], seed);
    }
    // halves: the first half's union (U until the half is complete) and the second's
    uint32_t h0lo[kFusedWordsPerWave] = {}, h0hi[kFusedWordsPerWave] = {};
    uint32_t h1lo[kFusedWordsPerWave] = {}, h1hi[kFusedWordsPerWave] = {};
    int members[8];
    members[0] = seed;
    int cnt = 1;
    while (cnt < max_group && free_mask) {
      if (cnt == half_w) {   // (uniform) the first half is complete
#pragma unroll
        for (int i = 0; i < kFusedWordsPerWave; ++i) {
          h0lo[i] = ulo[i];
          h0hi[i] = uhi[i];
        }
      }
      int partial = 0;
#pragma unroll
      for (int i = 0; i < kFusedWordsPerWave; ++i)
        partial += __builtin_popcount(lo[i] & ulo[i]) + __builtin_popcount(hi[i] & uhi[i]);
      int score = partial;
      if (nwaves > 1) {
        // a wave rewrites buffer pb only two picks later, after every wave has passed the
        // barrier of the pick in between (and so has read this pick's partials)
        part[pb][wave][lane] = partial;
        __syncthreads();
        int ps[kFusedMaxWaves];
#pragma unroll
        for (int v = 0; v < kFusedMaxWaves; ++v) ps[v] = part[pb][v][lane];   // unused slots stay 0
        score = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
        pb ^= 1;
      }
      const bool is_free = (free_mask >> lane) & 1ull;
      const int best = wave_max_dpp(is_free ? ((score << 6) | (63 - lane)) : -1);
      const int pick = 63 - (best & 63);
      free_mask &= ~(1ull << pick);
#pragma unroll
      for (int i = 0; i < kFusedWordsPerWave; ++i) {
        const uint32_t plo = __builtin_amdgcn_readlane(lo[i], pick);
        const uint32_t phi = __builtin_amdgcn_readlane(hi[i], pick);
        ulo[i] |= plo;
        uhi[i] |= phi;
        if (cnt >= half_w) {   // (uniform) a member of the second half
          h1lo[i] |= plo;
          h1hi[i] |= phi;
        }
      }
#pragma unroll
      for (int j = 1; j < 8; ++j) if (j == cnt) members[j] = pick;
      ++cnt;
    }
    // union sizes: popcount over every wave's words, summed by LDS atomics (read after the
    // loop, so no barrier per group)
    if (halves) {
      if (cnt <= half_w) {   // (uniform) no second half: the first half's union is U
#pragma unroll
        for (int i = 0; i < kFusedWordsPerWave; ++i) {
          h0lo[i] = ulo[i];
          h0hi[i] = uhi[i];
        }
      }
      int s0 = 0, s1 = 0;
#pragma unroll
      for (int i = 0; i < kFusedWordsPerWave; ++i) {
        s0 += __builtin_popcount(h0lo[i]) + __builtin_popcount(h0hi[i]);
        s1 += __builtin_popcount(h1lo[i]) + __builtin_popcount(h1hi[i]);
      }
      if (lane == 0) {
        atomicAdd(&usz_acc[2 * gi], s0);
        atomicAdd(&usz_acc[2 * gi + 1], s1);
      }
    } else {
      int usz = 0;
#pragma unroll
      for (int i = 0; i < kFusedWordsPerWave; ++i) usz += __builtin_popcount(ulo[i]) + __builtin_popcount(uhi[i]);
      if (lane == 0) atomicAdd(&usz_acc[gi], usz);
    }
    if (wave == 0) {
      if (lane < max_group) {
        int v = -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) if (j == lane && j < cnt) v = start + members[j];
        group_qids[(gbase + gi) * max_group + lane] = v;
      }
      if (lane == 0) group_size[gbase + gi] = cnt;
    }
    ++gi;
  }
  __syncthreads();   // (every wave made the same picks, so all arrive here)
  if (halves) {
    if (tid < 2 * gi) union_count[2 * gbase + tid + 1] = usz_acc[tid];
  } else if (tid < gi) {
    union_count[gbase + tid + 1] = usz_acc[tid];
  }
}

// ---------------------------------------------------------------------------------------
// (2b) members arranged for row tiles (QUILT's cascaded sharing at row-tile granularity).
// One wave per group of 5..8 members (4 members per 16-row tile).  A split is the three
// positions {a < b < c} in 1..n-1 that join position 0 in the first tile; its cost is
// |union of tile 1| + |union of tile 2|.  Lanes hold 64 bitset words of all members at a
// time and every split's cost is summed over them.  The cheapest split, first in
// lexicographic order on ties, orders the members (each tile keeps their relative order),
// and the group's member-mask bits are permuted to match: new bit j = old bit order[j].
__global__ __launch_bounds__(256) void k_arrange(const uint64_t* __restrict__ bits, int nq, int words,
                                                 int n_tables, int n_groups, int max_group,
                                                 int32_t* __restrict__ group_qids,
                                                 const int32_t* __restrict__ group_size,
                                                 const int32_t* __restrict__ union_off,
                                                 uint8_t* __restrict__ union_qmask,
                                                 int64_t capacity) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (e >= n_tables) return;
  const int g = e / n_groups;
  const int n = min(max(group_size[e], 0), max_group);
  if (n <= 4 || n > 8) return;
  int32_t* qids = group_qids + (int64_t)e * max_group;
  int mem[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mem[i] = i < n ? qids[i] : 0;
  // lanes hold 64 of the bitset words at a time; every split's cost is summed over the
  // lanes.  Splits are indexed by their rank among all 35 triples of 1..7 in lexicographic
  // order (a static index, so costs stay in registers); those with c > n-1 do not exist.
  const int m = n - 1;
  int costs[35];
#pragma unroll
  for (int i = 0; i < 35; ++i) costs[i] = 0;
  for (int w0 = 0; w0 < words; w0 += kWave) {
    const int w = w0 + lane;
    uint64_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      x[i] = (i < n && w < words) ? bits[((int64_t)g * nq + mem[i]) * words + w] : 0ull;
    int r = 0;
#pragma unroll
    for (int a = 1; a <= 7; ++a)
#pragma unroll
      for (int b = a + 1; b <= 7; ++b)
#pragma unroll
        for (int c = b + 1; c <= 7; ++c, ++r) {
          if (c > m) continue;
          const int mask = 1 | (1 << a) | (1 << b) | (1 << c);
          uint64_t ua = 0, ub = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if ((mask >> i) & 1) ua |= x[i];
            else ub |= x[i];              // positions >= n hold zeros
          }
          costs[r] += wave_sum(__popcll(ua) + __popcll(ub));
        }
  }
  int best_cost = 0x7fffffff, bmask = 0;
  {
    int r = 0;
#pragma unroll
    for (int a = 1; a <= 7; ++a)
#pragma unroll
      for (int b = a + 1; b <= 7; ++b)
#pragma unroll
        for (int c = b + 1; c <= 7; ++c, ++r)
          if (c <= m && costs[r] < best_cost) {
            best_cost = costs[r];
            bmask = 1 | (1 << a) | (1 << b) | (1 << c);
          }
  }
  // new position j holds old position order(j) = (perm >> 4j) & 15: the first tile's
  // positions ascending, then the rest ascending
  uint32_t perm = 0;
  int k = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < n && ((bmask >> i) & 1)) { perm |= (uint32_t)i << (4 * k); ++k; }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < n && !((bmask >> i) & 1)) { perm |= (uint32_t)i << (4 * k); ++k; }
  const int src = lane < 8 ? (int)((perm >> (4 * lane)) & 15u) : 0;
  int newq = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) if (i == src) newq = mem[i];
  if (lane < n) qids[lane] = newq;
  if (union_qmask) {
    const int64_t b0 = min<int64_t>(max(union_off[e], 0), capacity);
    const int64_t b1 = min<int64_t>(union_off[e + 1], capacity);
    for (int64_t x = b0 + lane; x < b1; x += kWave) {
      const uint32_t old = union_qmask[x];
      uint32_t nw = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < n) nw |= ((old >> ((perm >> (4 * j)) & 15u)) & 1u) << j;
      union_qmask[x] = (uint8_t)nw;
    }
  }
}

// ---------------------------------------------------------------------------------------
// (3) union tables.  Table e = g * n_groups + j; one wave per table.
__device__ __forceinline__ int member_count(const int32_t* group_size, int e, int group_width) {
  return group_size ? min(max(group_size[e], 0), group_width) : group_width;
}

// Row of member j of table e: group_rows[e][j], or with group_rows NULL the consecutive
// rows of the KV head's group e % n_groups, (e % n_groups) * group_width + j.
__device__ __forceinline__ int member_row(const int32_t* group_rows, int e, int n_groups,
                                          int group_width, int j) {
  return group_rows ? group_rows[(int64_t)e * group_width + j] : (e % n_groups) * group_width + j;
}

__global__ void k_union_count(const uint64_t* __restrict__ bits, int n_rows, int words,
                              const int32_t* __restrict__ group_rows,
                              const int32_t* __restrict__ group_size, int n_groups, int n_tables,
                              int group_width, int32_t* __restrict__ union_off) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (e >= n_tables) return;
  const int g = e / n_groups;
  const int sz = member_count(group_size, e, group_width);
  int cnt = 0;
  for (int w = lane; w < words; w += kWave) {
    uint64_t u = 0;
    for (int j = 0; j < sz; ++j) {
      const int r = member_row(group_rows, e, n_groups, group_width, j);
      if (r >= 0 && r < n_rows) u |= bits[((int64_t)g * n_rows + r) * words + w];
    }
    cnt += __popcll(u);
  }
  cnt = wave_sum(cnt);
  if (lane == 0) union_off[e + 1] = cnt;
}

// In-place inclusive scan of union_off[1 .. n] by one workgroup of 1024 threads (four
// consecutive entries per thread per 4096-entry chunk), so that union_off becomes the
// exclusive prefix sum of the table sizes.
__global__ void k_union_scan(int32_t* __restrict__ union_off, int n) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  if (t == 0) {
    carry_s = 0;
    union_off[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < n; base += 4096) {
    const int i0 = base + 4 * t;
    int v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = i0 + q < n ? union_off[i0 + q + 1] : 0;
#pragma unroll
    for (int q = 1; q < 4; ++q) v[q] += v[q - 1];
    const int ex = wave_excl_scan(v[3], lane);
    if (lane == kWave - 1) wsum[wave] = ex + v[3];
    __syncthreads();
    int before = carry_s;
    for (int k = 0; k < wave; ++k) before += wsum[k];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i0 + q < n) union_off[i0 + q + 1] = before + ex + v[q];
    __syncthreads();
    if (t == 1023) carry_s = before + ex + v[3];
    __syncthreads();
  }
}

// Work order for the union attention: the n items are cut into 8 consecutive ranges of
// per = ceil(n / 8) (the ranges the attention hands to the 8 XCDs) and each range is
// listed by union size, largest first, ties by lower item index: the ascending order of
// the keys (-size, index).  One workgroup per range runs a bitonic network.  Ranges of
// up to 1024 items hold one 32-bit key per thread and exchange partners with lane
// shuffles (distance < 64) or through LDS (distance >= 64); longer ranges, up to
// kScheduleCap, sort 64-bit keys in LDS; a range longer than that keeps item order.
// `key` is LDS for schedule_lds_bytes(per) bytes; the workgroup has at least
// min(1024, N) threads, N = per rounded up to a power of two >= 64, and every thread of
// it calls this (the ranges' sorts hold barriers).
constexpr int kScheduleCap = 8192;
__device__ void schedule_range(const int32_t* __restrict__ union_off, int n, int per, int range,
                               int32_t* __restrict__ order, uint64_t* key) {
  const int lo = range * per;
  const int m = min(n, lo + per) - lo;
  if (m <= 0) return;
  const int t = threadIdx.x;
  if (m > kScheduleCap) {
    for (int i = t; i < m; i += blockDim.x) order[lo + i] = lo + i;
    return;
  }
  int N = 64;
  while (N < m) N <<= 1;
  auto size_of = [&](int i) { return max(union_off[lo + i + 1] - union_off[lo + i], 0); };
  // (a range holding a union of 2^19 pages or more takes the 64-bit keys below)
  if (N <= 1024 && !__syncthreads_or(t < m && size_of(t) > 0x7FFFF)) {
    // key = (2^19 - 1 - size) << 13 | local index; padding sorts last
    uint32_t* k32 = reinterpret_cast<uint32_t*>(key);
    uint32_t v = 0xFFFFFFFFu;
    if (t < m) v = ((uint32_t)(0x7FFFF - size_of(t)) << 13) | (uint32_t)t;
    for (int k = 2; k <= N; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint32_t o;
        if (j >= 64) {
          if (t < N) k32[t] = v;
          __syncthreads();
          o = t < N ? k32[t ^ j] : v;
          __syncthreads();
        } else {
          o = (uint32_t)__shfl_xor((int)v, j, 64);
        }
        const bool up = (t & k) == 0, lower = (t & j) == 0;
        v = lower == up ? min(v, o) : max(v, o);
      }
    if (t < m) order[lo + t] = lo + (int)(v & 0x1FFFu);
    return;
  }
  for (int i = t; i < N; i += blockDim.x) {
    uint64_t k = ~0ull;   // padding sorts last
    if (i < m) k = ((uint64_t)(uint32_t)(INT32_MAX - size_of(i)) << 32) | (uint32_t)(lo + i);
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < N / 2; i += blockDim.x) {
        const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));   // pair (a, a + j)
        const bool up = (a & k) == 0;
        const uint64_t ka = key[a], kb = key[a + j];
        if ((ka > kb) == up) {
          key[a] = kb;
          key[a + j] = ka;
        }
      }
      __syncthreads();
    }
  for (int i = t; i < m; i += blockDim.x) order[lo + i] = (int32_t)(uint32_t)key[i];
}

__host__ __device__ constexpr int schedule_keys(int per) {
  int N = 64;
  while (N < per) N <<= 1;
  return N;
}
__host__ __device__ constexpr int schedule_threads(int per) {
  return schedule_keys(per) < 1024 ? schedule_keys(per) : 1024;
}
// LDS for any range of m <= per items: 8 N(m) bytes while m <= kScheduleCap (a shorter
// last range may sort where the others keep item order)
__host__ __device__ constexpr int schedule_lds_bytes(int per) {
  return 8 * schedule_keys(per < kScheduleCap ? per : kScheduleCap);
}

__global__ __launch_bounds__(1024) void k_schedule(const int32_t* __restrict__ union_off, int n,
                                                   int per, int32_t* __restrict__ order) {
  extern __shared__ uint64_t sched_key[];
  schedule_range(union_off, n, per, blockIdx.x, order, sched_key);
}

// Lane l of a wave covers pages [64*w + 16*s, +16) of a 1024-page chunk, w = l / 4 and
// s = l % 4 within the chunk, so that no lane lists more than 16 pages however closely
// a union clusters (a whole 64-page word per lane left the wave waiting on lanes with
// 40 and more pages of one community).  Lanes go in page order, so one exclusive scan
// of the lane counts places every page.
template <bool QMASK>
__device__ void emit_table(const uint64_t* __restrict__ bits, int n_rows, int words,
                           const int32_t* __restrict__ group_rows,
                           const int32_t* __restrict__ group_size, int n_groups, int n_tables,
                           int group_width, const int32_t* __restrict__ union_off,
                           int32_t* __restrict__ union_pages, uint8_t* __restrict__ union_qmask,
                           int64_t capacity, int e, int lane) {
  if (e >= n_tables) return;
  const int g = e / n_groups;
  const int sz = member_count(group_size, e, group_width);
  int r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r[j] = j < sz ? member_row(group_rows, e, n_groups, group_width, j) : -1;
    if (r[j] >= n_rows) r[j] = -1;   // (negative: no member)
  }
  const int sh = 16 * (lane & 3);
  int64_t pos = union_off[e];
  PW_DCHECK(lane != 0 || (pos >= 0 && pos <= union_off[e + 1]));   // prefix sums ascend
  for (int w0 = 0; w0 < words; w0 += kWave / 4) {
    const int w = w0 + (lane >> 2);
    uint32_t mw[8];
    uint32_t u = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mw[j] = 0u;
      if (w < words && r[j] >= 0)
        mw[j] = (uint32_t)(bits[((int64_t)g * n_rows + r[j]) * words + w] >> sh) & 0xFFFFu;
      u |= mw[j];
    }
    if (!QMASK)   // (member masks need at most 8 members; plain tables take up to 64)
      for (int j = 8; j < sz; ++j) {
        const int rj = member_row(group_rows, e, n_groups, group_width, j);
        if (w < words && rj >= 0 && rj < n_rows)
          u |= (uint32_t)(bits[((int64_t)g * n_rows + rj) * words + w] >> sh) & 0xFFFFu;
      }
    const int pc = __popc(u);
    int64_t p = pos + wave_excl_scan(pc, lane);
    const int chunk_total = wave_sum(pc);
    const int base = w * 64 + sh;
    while (u) {
      const int b = __ffs(u) - 1;
      u &= u - 1;
      PW_DCHECK(p < capacity);   // (the host's capacity bound held for this table)
      if (p < capacity) {
        union_pages[p] = base + b;
        if (QMASK) {
          int qm = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) qm |= (int)((mw[j] >> b) & 1u) << j;
          union_qmask[p] = (uint8_t)qm;
        }
      }
      ++p;
    }
    pos += chunk_total;
  }
}


template <bool QMASK>
__global__ void k_union_emit(const uint64_t* __restrict__ bits, int n_rows, int words,
                             const int32_t* __restrict__ group_rows,
                             const int32_t* __restrict__ group_size, int n_groups, int n_tables,
                             int group_width, const int32_t* __restrict__ union_off,
                             int32_t* __restrict__ union_pages, uint8_t* __restrict__ union_qmask,
                             int64_t capacity) {
  emit_table<QMASK>(bits, n_rows, words, group_rows, group_size, n_groups, n_tables, group_width,
                    union_off, union_pages, union_qmask, capacity,
                    blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave, threadIdx.x & (kWave - 1));
}

// The union listing and the work order in one launch (both only read the prefix sums):
// workgroups 0..7 sort the 8 ranges, the others list blockDim / 64 tables each.
__global__ __launch_bounds__(1024) void k_union_emit_schedule(
    const uint64_t* __restrict__ bits, int n_rows, int words, const int32_t* __restrict__ group_rows,
    const int32_t* __restrict__ group_size, int n_groups, int n_tables, int group_width,
    const int32_t* __restrict__ union_off, int32_t* __restrict__ union_pages,
    uint8_t* __restrict__ union_qmask, int64_t capacity, int per, int32_t* __restrict__ order) {
  extern __shared__ uint64_t sched_key[];
  if (blockIdx.x < 8) {   // (uniform over the workgroup: its barriers are all reached)
    schedule_range(union_off, n_tables, per, blockIdx.x, order, sched_key);
    return;
  }
  emit_table<true>(bits, n_rows, words, group_rows, group_size, n_groups, n_tables, group_width,
                   union_off, union_pages, union_qmask, capacity,
                   (blockIdx.x - 8) * (blockDim.x / kWave) + threadIdx.x / kWave,
                   threadIdx.x & (kWave - 1));
}

}  // namespace

// ---------------------------------------------------------------------------------------
pw_status launch_arrange(const uint64_t* bits, int nq, int hkv, int n_pages, int n_groups,
                         int max_group, int32_t* group_qids, const int32_t* group_size,
                         const int32_t* union_off, uint8_t* union_qmask, int64_t capacity,
                         hipStream_t stream) {
  const int n_tables = hkv * n_groups;
  if (n_tables == 0) return PW_OK;
  hipLaunchKernelGGL(k_arrange, dim3((n_tables + 3) / 4), dim3(256), 0, stream, bits, nq,
                     (n_pages + 63) / 64, n_tables, n_groups, max_group, group_qids, group_size,
                     union_off, union_qmask, capacity);
  return check_launch("pw_arrange_groups");
}

pw_status launch_schedule(const int32_t* union_off, int n, int32_t* order, hipStream_t stream) {
  if (n <= 0) return PW_OK;
  const int per = (n + 7) / 8;
  hipLaunchKernelGGL(k_schedule, dim3(8), dim3(schedule_threads(per)), schedule_lds_bytes(per),
                     stream, union_off, n, per, order);
  return check_launch("schedule_items");
}

pw_status launch_scan(int32_t* off, int n, hipStream_t stream) {
  hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(1024), 0, stream, off, n);
  return check_launch("prefix sum");
}

pw_status launch_page_bitsets(const int32_t* topk, int n_rows, int hkv, int k, int n_pages,
                              uint64_t* bits, int32_t* bad_id_count, hipStream_t stream) {
  const int words = (n_pages + 63) / 64;
  const int64_t total = (int64_t)n_rows * hkv;
  if (total == 0) return PW_OK;
  const int per_wave = words * kWave;
  const int waves = std::max(1, std::min(4, 65536 / per_wave));
  const int64_t want = (total + waves - 1) / waves;
  const int blocks = (int)std::min<int64_t>(want, 1024);
  const size_t lds = (size_t)waves * per_wave;
  if (words <= 4)
    hipLaunchKernelGGL(k_page_bitsets<4>, dim3(blocks), dim3(waves * kWave), lds, stream, topk,
                       n_rows, hkv, k, n_pages, words, bits, bad_id_count);
  else if (words <= 16)
    hipLaunchKernelGGL(k_page_bitsets<16>, dim3(blocks), dim3(waves * kWave), lds, stream, topk,
                       n_rows, hkv, k, n_pages, words, bits, bad_id_count);
  else
    hipLaunchKernelGGL(k_page_bitsets<0>, dim3(blocks), dim3(waves * kWave), lds, stream, topk,
                       n_rows, hkv, k, n_pages, words, bits, bad_id_count);
  return check_launch("page_bitsets");
}

pw_status launch_group(const uint64_t* bits, int nq, int hkv, int n_pages, int window,
                       int max_group, int n_groups, int32_t* group_qids, int32_t* group_size,
                       hipStream_t stream) {
  if (nq == 0) return PW_OK;
  const int words = (n_pages + 63) / 64;
  const int n_windows = (nq + window - 1) / window;
  if (window <= 64) {
    dim3 grid(n_windows, hkv), block(64);
#define PW_GROUPW_CASE(W)                                                                    \
    if (words <= W) {                                                                        \
      hipLaunchKernelGGL(k_group_wave<W>, grid, block, 0, stream, bits, nq, words, window,  \
                         max_group, n_groups, group_qids, group_size);                       \
      return check_launch("group");                                                          \
    }
    PW_GROUPW_CASE(1)
    PW_GROUPW_CASE(2)
    PW_GROUPW_CASE(4)
    PW_GROUPW_CASE(8)
    PW_GROUPW_CASE(16)   // beyond 16 words the union no longer fits in scalar registers
#undef PW_GROUPW_CASE
  }
  const int threads = ((std::min(window, nq) + kWave - 1) / kWave) * kWave;
  dim3 grid(n_windows, hkv), block(threads);
#define PW_GROUP_CASE(W)                                                                     \
  if (words <= W) {                                                                          \
    hipLaunchKernelGGL(k_group<W>, grid, block, 0, stream, bits, nq, words, window, max_group, \
                       n_groups, group_qids, group_size);                                    \
    return check_launch("group");                                                            \
  }
  PW_GROUP_CASE(1)
  PW_GROUP_CASE(2)
  PW_GROUP_CASE(4)
  PW_GROUP_CASE(8)
  PW_GROUP_CASE(16)
  PW_GROUP_CASE(32)
  PW_GROUP_CASE(64)
#undef PW_GROUP_CASE
  return fail(PW_ERR_UNSUPPORTED, "pw_group: n_pages=%d needs %d words > 64", n_pages, words);
}

bool prepare_fusable(int n_pages, int window) { return n_pages <= 1024 && window <= 64; }

pw_status launch_prepare(const int32_t* topk, int nq, int hkv, int k, int n_pages, int window,
                         int max_group, int n_groups, uint64_t* bits, int32_t* bad_id_count,
                         int32_t* group_qids, int32_t* group_size, int32_t* union_off,
                         int32_t* union_pages, uint8_t* union_qmask, int64_t capacity,
                         int32_t* item_order, int halves, hipStream_t stream) {
  const int words = (n_pages + 63) / 64;
  // halves: table 2j + h is half h of group j, members [h mg/2, (h + 1) mg/2) of its list,
  // read through the member lists viewed as [hkv][2 n_groups][mg/2] (absent members are -1)
  const int n_tables = hkv * n_groups * (halves ? 2 : 1);
  const int32_t* t_rows = group_qids;
  const int32_t* t_size = halves ? nullptr : group_size;
  const int t_groups = halves ? 2 * n_groups : n_groups;
  const int t_width = halves ? max_group / 2 : max_group;
  if (nq > 0) {
    const int nwaves = (words + kFusedWordsPerWave - 1) / kFusedWordsPerWave;
    dim3 grid((nq + window - 1) / window, hkv), block(nwaves * kWave);
    hipLaunchKernelGGL(k_prepare, grid, block, 0, stream, topk, nq, hkv, k, n_pages, words, window,
                       max_group, n_groups, bits, bad_id_count, group_qids, group_size, union_off,
                       halves);
    pw_status st = check_launch("prepare");
    if (st != PW_OK) return st;
  }
  hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(1024), 0, stream, union_off, n_tables);
  pw_status st = check_launch("union_scan");
  if (st != PW_OK || n_tables == 0) return st;
  if (item_order) {
    const int per = (n_tables + 7) / 8;
    const int threads = schedule_threads(per);
    const int wpb = threads / kWave;
    hipLaunchKernelGGL(k_union_emit_schedule, dim3(8 + (n_tables + wpb - 1) / wpb), dim3(threads),
                       schedule_lds_bytes(per), stream, bits, nq, words, t_rows, t_size, t_groups,
                       n_tables, t_width, union_off, union_pages, union_qmask, capacity, per,
                       item_order);
    return check_launch("union_emit_schedule");
  }
  const int wpb = 4;
  const int blocks = (n_tables + wpb - 1) / wpb;
  hipLaunchKernelGGL(k_union_emit<true>, dim3(blocks), dim3(wpb * kWave), 0, stream, bits, nq,
                     words, t_rows, t_size, t_groups, n_tables, t_width, union_off, union_pages,
                     union_qmask, capacity);
  return check_launch("union_emit");
}

pw_status launch_union_tables(const uint64_t* bits, int n_rows, int hkv, int n_pages,
                              const int32_t* group_rows, const int32_t* group_size, int n_groups,
                              int group_width, int32_t* union_off, int32_t* union_pages,
                              uint8_t* union_qmask, int64_t capacity, hipStream_t stream) {
  const int words = (n_pages + 63) / 64;
  const int n_tables = hkv * n_groups;
  if (n_tables == 0) {   // only union_off[0] = 0
    hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(1024), 0, stream, union_off, 0);
    return check_launch("union_scan");
  }
  const int wpb = 4;
  const int blocks = (n_tables + wpb - 1) / wpb;
  hipLaunchKernelGGL(k_union_count, dim3(blocks), dim3(wpb * kWave), 0, stream, bits, n_rows,
                     words, group_rows, group_size, n_groups, n_tables, group_width, union_off);
  pw_status st = check_launch("union_count");
  if (st != PW_OK) return st;
  hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(1024), 0, stream, union_off, n_tables);
  st = check_launch("union_scan");
  if (st != PW_OK) return st;
  if (union_qmask)
    hipLaunchKernelGGL(k_union_emit<true>, dim3(blocks), dim3(wpb * kWave), 0, stream, bits,
                       n_rows, words, group_rows, group_size, n_groups, n_tables, group_width,
                       union_off, union_pages, union_qmask, capacity);
  else
    hipLaunchKernelGGL(k_union_emit<false>, dim3(blocks), dim3(wpb * kWave), 0, stream, bits,
                       n_rows, words, group_rows, group_size, n_groups, n_tables, group_width,
                       union_off, union_pages, union_qmask, capacity);
  return check_launch("union_emit");
}

}  // namespace pw
