// ID-aware union attention for gfx950 (CDNA4, wave64; MFMA 16x16x32 bf16 and, for fp8 K,
// 16x16x128 fp8).
//
// Method: "PageWeaver: KV-Guided Query Unions for Sparse Attention" (abstract,
// Fig. 1, Fig. 3): a group's union pages are staged on chip once and the same
// lanes compute QK, the masked online softmax and PV for every member, keeping
// the member's state and writing its rows to its original ID, with no
// reordered Q and no cross-page partial outputs; subgroups that did not select
// a page skip its math but still honour the staging buffers' lifetime.
// "CompactAttention" (summary, "Approach"): attention reads the paged cache in
// place, KV-head-major, including one shared block table per KV group.
//
// Work item = (KV head g, group j); its rows are (member m, head h) pairs,
// row r = m * G + (h - g*G).  A workgroup of NW waves owns one item; wave w
// holds MT row tiles of 16 rows (rows 16*(w*MT + mt) + 0..15), so every K/V
// fragment read and converted from LDS feeds MT MFMA row tiles.
//
// Every union page is cut into 32-token tiles, streamed into an ST-deep LDS
// ring by direct global->LDS loads (global_load_lds_dwordx4, issued from
// inline assembly so that the only waits on them are the explicit vmcnt waits
// below).  Per tile:
//   * S^T[key][row] = K . Q^T on MFMA: keys are the MFMA rows, so each lane
//     ends with one query row and 8 of its keys and row statistics stay in
//     the lane;
//   * support mask (the member selected the page) + causal mask, online
//     softmax in the log2 domain; the reference used for the exponentials
//     is set on a row's first used tile and raised only when a lane's share
//     of a tile's row sum of P = 2^(score - reference) passes 2^30, so the
//     accumulators are rescaled rarely (exact either way: numerator and
//     denominator share the reference);
//   * O^T[d][row] += V^T . P^T on MFMA, V^T read from LDS with the CDNA4
//     transposing loads (ds_read_b64_tr_b8 / _b16).
// fp8 (OCP e4m3fn) K codes feed the fp8 MFMA as stored (d = 128: each Q row split
// exactly into two e4m3 parts) or convert exactly to bf16 (d = 64); V codes convert
// exactly to bf16.  The K page scale folds into the score scale and the V page scale
// into P (the row sum uses unscaled P).
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace pw {

PW_DEBUG_COUNTER_DEFINE(debug_count_attn)

namespace {

constexpr int kWave = 64;
constexpr int kTK = 32;               // tokens per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The reference used for the exponentials is raised only when a lane's share of a tile's
// row sum of P (P = 2^(score - reference)) exceeds 2^30 (the tile's row sum then 2^32 at
// most): well inside fp32/bf16 range, and bf16/fp32 precision is relative, so nothing is
// lost while P stays below it.
constexpr float kRescaleShare = 0x1p30f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
#define PW_LDS __attribute__((address_space(3)))
#define PW_CONST __attribute__((address_space(4)))

struct Params {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* q_pos;
  const int32_t* group_qids;
  const int32_t* group_size;
  const int32_t* union_off;
  const int32_t* union_pages;
  const uint8_t* union_qmask;
  uint16_t* out;
  float* lse;
  const int32_t* item_kvh;      // page-major items (else NULL): KV head of each item
  const int32_t* item_lo_dev;   // page-major items: run items [*item_lo_dev, *item_hi_dev)
  const int32_t* item_hi_dev;   //   (n_items bounds their count)
  const int32_t* out_slot;      // page-major items: partial slot per (item, member)
  int64_t stride_head_b;   // bytes
  int64_t stride_page_b;   // bytes
  int64_t capacity;
  int nq, hq, hkv, G;
  int page_size, n_pages, kv_len;
  int n_groups, max_group, shared_table;
  int n_split;             // > 1: each item's table is cut into n_split slices (partials)
  int n_items, items_per_xcd;
  const int32_t* item_order;    // NULL or a permutation: position r runs item item_order[r]
  float score_scale;       // sm_scale * log2(e)
};

// XOR swizzle of the 16-byte chunks of one LDS token row.  Chosen so that the K
// operand reads and the transposing V reads fall on distinct banks.  Measured on gfx950
// (64 banks of 4 bytes): a 16-byte read serves the wave in four phases of 16 lanes that
// start at lane 8 (lanes 8..23, 24..39, 40..55, 56..63 with 0..7); an 8-byte transposing
// read in two phases of 32 lanes.  For 256-byte rows (bf16, d = 128) a phase then holds
// the K rows of two neighbouring row groups, and chunk bit 0 taken from key bit 2 (not
// bit 4) keeps them apart: no bank conflicts on either read, against 4 conflict cycles
// per K read before.
template <int CHUNKS>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CHUNKS >= 16) {
    return (((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3)) & (CHUNKS - 1);
  } else {
    return (((r >> 1) & 1) | (((r >> 3) & 1) << 1) | ((((r >> 2) ^ (r >> 4)) & 1) << 2)) & (CHUNKS - 1);
  }
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Direct global -> LDS copies of 16 bytes per lane, N loads sharing one M0 (the LDS
// address; declared clobbered, so the compiler restores whatever it keeps there).  Load k
// reads sbase + voff[k] + k*STRIDE (sbase wave-uniform, voff per lane) and lands at LDS
// m0 + k*STRIDE + 16*l for lane l: the instruction offset applies to both addresses
// (measured).  The offset field holds < 4096.  An s_nop gives the one wait state an M0
// write needs before an LDS-DMA load reads it (the compiler keeps the same distance for
// its own M0 writes; a load that reads M0 may be followed by an M0 write at once).
template <int N, int STRIDE>
__device__ __forceinline__ void dma16_group(const uint32_t* voff, const void* sbase, uint32_t m0) {
  static_assert((N == 1 || N == 2 || N == 4) && (N - 1) * STRIDE < 4096, "offset field");
  if constexpr (N == 1) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2"
        :
        : "v"(voff[0]), "s"(m0), "s"(sbase)
        : "memory", "m0");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %3\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:%4"
        :
        : "v"(voff[0]), "v"(voff[1]), "s"(m0), "s"(sbase), "n"(STRIDE)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %5\n\t"
        "global_load_lds_dwordx4 %1, %5 offset:%6\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:%7\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:%8"
        :
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(m0), "s"(sbase), "n"(STRIDE),
          "n"(2 * STRIDE), "n"(3 * STRIDE)
        : "memory", "m0");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until the loads of at most `newer` tiles (K loads each) are still in flight.
template <int K, int MAXN>
__device__ __forceinline__ void wait_tiles(int newer) {
  if constexpr (MAXN == 0) {
    wait_vmcnt<0>();
  } else {
    if (newer >= MAXN) wait_vmcnt<K * MAXN>();
    else wait_tiles<K, MAXN - 1>(newer);
  }
}

template <int D, bool FP8, int MT, int NW, int ST>
struct Cfg {
  static constexpr int kEsz = FP8 ? 1 : 2;
  static constexpr int kRowBytes = D * kEsz;              // one token row of K or V
  static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
  static constexpr int kTensorBytes = kTK * kRowBytes;    // K or V tile
  static constexpr int kStageBytes = 2 * kTensorBytes;
  static constexpr int kThreads = NW * kWave;
  static constexpr int kDmaPerTensor = kTensorBytes / (16 * kThreads);  // per lane
  static_assert(kDmaPerTensor >= 1, "every wave issues at least one load per tensor");
  static constexpr int kDmaPerTile = 2 * kDmaPerTensor;
  // a tensor's loads go out in groups of kDmaGroup sharing one M0: load k of a group sits
  // k * NW KiB above the group's first in both memories, within the 4 KiB offset field
  static constexpr int kDmaGroup = (kDmaPerTensor % 4 == 0 && 4 * NW <= 4)   ? 4
                                   : (kDmaPerTensor % 2 == 0 && 2 * NW <= 4) ? 2
                                                                             : 1;
  static constexpr int kDc = D / 32;                       // MFMA k-steps over d
  static constexpr int kDt = D / 16;                       // 16-wide d tiles of O
  static_assert(kTensorBytes % (16 * kThreads) == 0, "tile must split evenly into DMA slots");
  static_assert(kDmaPerTile * (ST - 2) < 64, "vmcnt range");
  static_assert(ST >= 2 && ST <= 4, "2..4 stages");
  // Waves per SIMD the tile ring's LDS admits (160 KiB per CU, 4 SIMDs).  Where it admits
  // three, the kernel is built for three (<= 168 VGPRs) and streams its K fragments
  // instead of holding a whole tile's; elsewhere two waves with the K tile held in
  // registers are faster.  One-row-tile items whose ring admits ten waves per CU (two
  // SIMDs can then hold three) are still held, but built for three waves (the 2K-query
  // GQA bf16 chunk: attention -2 %, a few registers spilled outside the tile loop).
  static constexpr int kLdsWaves = (160 * 1024 / (ST * kStageBytes)) * NW / 4;
  static constexpr bool kStreamK = kLdsWaves >= 3;
  static constexpr int kWavesPerSimd =
      kStreamK || (MT == 1 && (160 * 1024 / (ST * kStageBytes)) * NW >= 10) ? 3 : 2;
  // fp8 K with d = 128: S^T = K . Q^T on the fp8 MFMA (16x16x128), K straight from LDS
  static constexpr bool kF8Mma = FP8 && D == 128;
};

template <int D, bool FP8, int MT, int NW, int ST>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(Cfg<D, FP8, MT, NW, ST>::kWavesPerSimd))) void k_attn(Params p) {
  using C = Cfg<D, FP8, MT, NW, ST>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[ST * C::kStageBytes];

  // XCD-aware work order: workgroup b runs on XCD b % 8; each XCD gets a contiguous
  // range of positions (KV-head-major items), so one XCD's L2 serves neighbouring groups
  // of the same KV head.  Workgroups are dispatched in order, so a work order that lists
  // each range's largest unions first (pw_schedule_items) leaves the short items for the
  // end, where they fill the gaps instead of extending the tail.
  const int b = blockIdx.x;
  int n_items = p.n_items, per_xcd = p.items_per_xcd, item0 = 0;
  if (p.item_lo_dev) {   // page-major: the grid is an upper bound of the device count
    item0 = *p.item_lo_dev;
    n_items = min(n_items, *p.item_hi_dev - item0);
    per_xcd = (n_items + 7) >> 3;
    if ((b >> 3) >= per_xcd) return;
  }
  const int item_rel = (b & 7) * per_xcd + (b >> 3);
  if (item_rel >= n_items) return;
  const int item_s = p.item_order ? p.item_order[item_rel] : item0 + item_rel;
  if (item_s < 0 || item_s >= item0 + n_items) return;   // (a damaged work order)
  // table slices: item_s = item * n_split + slice (consecutive slices share an XCD's L2)
  const int slice = p.n_split > 1 ? item_s % p.n_split : 0;
  const int item = p.n_split > 1 ? item_s / p.n_split : item_s;
  const int g = p.item_kvh ? p.item_kvh[item] : item / p.n_groups;
  const int j = item - g * p.n_groups;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform per wave
  const int li = lane & 15;      // MFMA row/col index inside a 16-lane group
  const int lq = lane >> 4;      // 16-lane group 0..3

  // ---- members and this lane's query rows -------------------------------------------
  int gsize;
  const int32_t* qids = nullptr;
  if (p.group_qids) {
    gsize = min(max(p.group_size[item], 0), p.max_group);
    qids = p.group_qids + (int64_t)item * p.max_group;
  } else {
    gsize = min(p.max_group, p.nq - j * p.max_group);
  }
  // query ID (-1: none), query head and partial slot of this lane's row in row tile m;
  // computed again in the epilogue rather than kept live through the tile loop
  auto row_info = [&](int m, int& id, int& hq_row, int& slot) {
    const int row = 16 * (wave * MT + m) + li;
    const int member = row / p.G;
    hq_row = g * p.G + (row - member * p.G);
    id = -1;
    if (member < gsize) id = qids ? qids[member] : j * p.max_group + member;
    PW_DCHECK(member >= gsize || id < p.nq);   // a listed member is a query of the chunk
    if (id >= p.nq) id = -1;
    slot = -1;
    if (p.out_slot && id >= 0) {
      slot = p.out_slot[(int64_t)item * p.max_group + member];
      if (slot < 0) id = -1;
    }
  };
  int row_lim[MT], my_bit[MT], mt_members[MT], mt_lim[MT];
  bf16x8 qf[C::kF8Mma ? 1 : MT][C::kDc];
  i32x8 qh[C::kF8Mma ? MT : 1], ql[C::kF8Mma ? MT : 1];
  float qs[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row0 = 16 * (wave * MT + m);
    const int member = (row0 + li) / p.G;
    int id, hh, slot;
    row_info(m, id, hh, slot);
    const int qpos = id >= 0 ? p.q_pos[id] : -1;
    row_lim[m] = min(qpos, p.kv_len - 1);          // last usable token of this row
    int mm = 0;
    if (p.union_qmask) {            // member-mask bit per member (max_group <= 8)
      my_bit[m] = id >= 0 ? (1 << member) : 0;
      for (int r = row0; r < row0 + 16; ++r) {
        const int mb = r / p.G;
        if (mb < gsize) mm |= 1 << mb;
      }
    } else {                        // every member uses every page: one shared bit
      my_bit[m] = id >= 0 ? 1 : 0;
      mm = row0 / p.G < gsize ? 1 : 0;
    }
    mt_members[m] = __builtin_amdgcn_readfirstlane(mm);   // same in every lane
    int lim = row_lim[m];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) lim = max(lim, __shfl_xor(lim, o, kWave));
    mt_lim[m] = __builtin_amdgcn_readfirstlane(lim);      // same in every lane
    qs[m] = 1.f;
    if constexpr (C::kF8Mma) {
      // Q^T fragments for the fp8 MFMA: the row is scaled by 2^e (its largest magnitude
      // lands in [128, 256)) and split into hi = e4m3(q 2^e) and lo = e4m3(q 2^e - hi).
      // hi + lo equals q 2^e exactly for every element above 2^-10 of the row maximum (a
      // bf16 significand is 8 bits, an e4m3 one 4), and 2^-e is undone in the score
      // scale.  Lane group lq holds d = 16lq .. +16 (bytes 0..15) and 64 + 16lq .. +16
      // (bytes 16..31), the same slots as the K operand.
      float x[32];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          i32x4 v = i32x4{0, 0, 0, 0};
          if (id >= 0)
            v = *reinterpret_cast<const i32x4*>(p.q + ((int64_t)id * p.hq + hh) * D + 64 * h + 16 * lq + 8 * w);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x[16 * h + 8 * w + 2 * k] = __builtin_bit_cast(float, (int)((uint32_t)v[k] << 16));
            x[16 * h + 8 * w + 2 * k + 1] = __builtin_bit_cast(float, (int)((uint32_t)v[k] & 0xFFFF0000u));
          }
        }
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(x[k]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      int ex = 0;
      if (mx > 0.f && mx <= 3.0e38f) (void)frexpf(mx, &ex);   // mx = f 2^ex, f in [0.5, 1)
      const int e = mx > 0.f && mx <= 3.0e38f ? 8 - ex : 0;
      qs[m] = __builtin_amdgcn_ldexpf(1.f, -e);
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float y[4], r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = __builtin_amdgcn_ldexpf(x[4 * w + k], e);
        int hw = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], hw, true);
        const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
        const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
        r[0] = y[0] - d0[0];
        r[1] = y[1] - d0[1];
        r[2] = y[2] - d1[0];
        r[3] = y[3] - d1[1];
        int lw = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
        lw = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lw, true);
        qh[m][w] = hw;
        ql[m][w] = lw;
      }
    } else {
      // Q^T fragments (B operand of S^T = K . Q^T): row li, d = 32c + 8lq .. +8
#pragma unroll
      for (int c = 0; c < C::kDc; ++c) {
        if (id >= 0) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(p.q + ((int64_t)id * p.hq + hh) * D +
                                                           32 * c + 8 * lq);
          qf[m][c] = __builtin_bit_cast(bf16x8, v);
        } else {
          qf[m][c] = bf16x8{};
        }
      }
    }
  }

  // ---- table of this item -----------------------------------------------------------
  const int table = p.shared_table ? g : item;
  int64_t e_begin = item, e_end = item + 1;   // page-major items: one page each
  if (p.union_off) {
    e_begin = p.union_off[table];
    e_end = p.union_off[table + 1];
  }
  PW_DCHECK(lane != 0 || (e_begin >= 0 && e_begin <= e_end && e_end <= p.capacity));
  e_begin = min<int64_t>(max<int64_t>(e_begin, 0), p.capacity);
  e_end = min<int64_t>(e_end, p.capacity);
  if (p.n_split > 1) {   // this item's slice of the table
    const int64_t per = (max<int64_t>(e_end - e_begin, 0) + p.n_split - 1) / p.n_split;
    e_begin = min<int64_t>(e_begin + per * slice, e_end);
    e_end = min<int64_t>(e_begin + per, e_end);
  }
  const int tpp_shift = p.page_size == 128 ? 2 : 1;          // log2(tiles per page)
  const int n_tiles = (int)max<int64_t>(e_end - e_begin, 0) << tpp_shift;

  const uint8_t* kbase = p.k_cache + (int64_t)g * p.stride_head_b;
  const uint8_t* vbase = p.v_cache + (int64_t)g * p.stride_head_b;
  // metadata through the scalar cache (constant address space): uniform per tile
  const PW_CONST int32_t* cpages = (const PW_CONST int32_t*)p.union_pages;

  // per-lane byte offsets of this lane's DMA slots inside one K (or V) tile
  uint32_t dma_off[C::kDmaPerTensor];
#pragma unroll
  for (int i = 0; i < C::kDmaPerTensor; ++i) {
    const int slot = (i * NW + wave) * kWave + lane;
    const int r = slot / C::kChunks;
    const int pc = slot - r * C::kChunks;
    // less the in-group offset that the load instruction adds back
    dma_off[i] = r * C::kRowBytes + ((pc ^ swz<C::kChunks>(r)) << 4) - (i % C::kDmaGroup) * NW * 1024;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(PW_LDS void*)lds;
  const PW_LDS uint8_t* lds_p = (const PW_LDS uint8_t*)lds;

  // per-lane LDS read offsets inside one stage (the stage base is an immediate)
  // (fp8 MFMA: two whole 16-byte chunks per key block, d = 16lq .. +16 and 64 + 16lq .. +16)
  int k_off[2][C::kF8Mma ? 2 : C::kDc];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = 8 * (li >> 2) + 4 * kb + (li & 3);   // MFMA row li of key block kb
    if constexpr (C::kF8Mma) {
#pragma unroll
      for (int h = 0; h < 2; ++h) k_off[kb][h] = key * C::kRowBytes + (((lq + 4 * h) ^ swz<C::kChunks>(key)) << 4);
    } else {
#pragma unroll
      for (int c = 0; c < C::kDc; ++c) {
        const int byte = (32 * c + 8 * lq) * C::kEsz;
        k_off[kb][c] = key * C::kRowBytes + (((byte >> 4) ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
      }
    }
  }
  constexpr int kVr = FP8 ? C::kDt : 2 * C::kDt;
  int v_off[kVr];
#pragma unroll
  for (int dt = 0; dt < C::kDt; ++dt) {
    if constexpr (FP8) {
      // ds_read_b64_tr_b8: output byte e of lane li = V[8*lq + e][16*dt + li] when source
      // lane li reads key 8*lq + (li >> 1), columns 16*dt + 8*(li & 1) .. +8
      const int key = 8 * lq + (li >> 1);
      const int byte = 16 * dt + 8 * (li & 1);
      v_off[dt] = C::kTensorBytes + key * C::kRowBytes + (((byte >> 4) ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
    } else {
      // ds_read_b64_tr_b16: output element e of lane li = V[key0 + e][16*dt + li] when
      // source lane li reads key key0 + (li >> 2), columns 16*dt + 4*(li & 3) .. +4
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key = 8 * lq + 4 * hf + (li >> 2);
        const int byte = (16 * dt + 4 * (li & 3)) * 2;
        v_off[2 * dt + hf] = C::kTensorBytes + key * C::kRowBytes + (((byte >> 4) ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
      }
    }
  }

  auto page_of = [&](int t) -> int {
    const int pg = cpages[e_begin + (t >> tpp_shift)];
    return (pg >= 0 && pg < p.n_pages) ? pg : -1;
  };

  // Per-page metadata, one table entry per lane: entries md_base .. md_base + 63 of the
  // item's table (relative to e_begin), refilled when the tile loop passes them (every
  // 64 pages).  A tile reads its page's values with v_readlane instead of scalar loads:
  // the K/V scales sit at random addresses, and their latency stalled every tile.
  int md_base = 0, md_pq = 0;   // (page + 1) | member mask << 24 (page + 1 = 0: invalid)
  float md_sc = 0.f, md_lvs = 0.f, md_ivs = 1.f;      // score scale * ks, log2 vs, 1 / vs
  auto refill = [&](int base) {
    md_base = base;
    int pg = -1, qm = 0;
    float ks = 1.f, vs = 1.f;
    if (p.item_kvh) {
      // page-major items hold one page: every lane takes it through the scalar cache,
      // whose round trip is shorter than a vector load's on these two-tile items
      if (e_begin < e_end) {   // (an empty table reads nothing)
        pg = cpages[e_begin];
        pg = (pg >= 0 && pg < p.n_pages) ? pg : -1;
      }
      qm = 0xFF;
      if constexpr (FP8) {
        if (pg >= 0) {
          ks = ((const PW_CONST float*)p.k_scale)[(int64_t)g * p.n_pages + pg];
          vs = ((const PW_CONST float*)p.v_scale)[(int64_t)g * p.n_pages + pg];
        }
      }
    } else {
      const int64_t e = e_begin + base + lane;
      if (e < e_end) {
        pg = p.union_pages[e];
        pg = (pg >= 0 && pg < p.n_pages) ? pg : -1;
        qm = p.union_qmask ? (int)p.union_qmask[e] : 0xFF;
      }
      if constexpr (FP8) {
        if (pg >= 0) {
          ks = p.k_scale[(int64_t)g * p.n_pages + pg];
          vs = p.v_scale[(int64_t)g * p.n_pages + pg];
        }
      }
    }
    md_pq = (pg + 1) | (qm << 24);   // n_pages <= 2^24 - 2 (checked on the host)
    md_sc = p.score_scale * ks;                        // log2-domain score scale
    md_lvs = FP8 ? __builtin_amdgcn_logf(vs) : 0.f;    // log2 of the V page scale
    // 1 / vs only scales the row sums, so the hardware reciprocal (1 ulp) is ample
    md_ivs = FP8 ? __builtin_amdgcn_rcpf(vs) : 1.f;
  };
  auto lane_i = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
  auto lane_f = [](float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  };

  // Every tile issues the same number of loads (an invalid page reads page 0 and is
  // never computed), so the vmcnt waits below are exact.
  // off_known: the byte offset of the tile's page when the caller has it already (from the
  // load of the page's first tile; kNoPage: look it up).  Returns the page's byte offset.
  constexpr int64_t kNoPage = -1;
  auto issue = [&](int t, auto stage_c, int64_t off_known) -> int64_t {
    constexpr int SS = decltype(stage_c)::value;
    const int ent = t >> tpp_shift;
    int64_t pg_off;
    if (off_known != kNoPage) {
      pg_off = off_known;
    } else if (ent - md_base < kWave) {   // held by the lanes (the loop never looks back)
      const int pg = (lane_i(md_pq, ent - md_base) & 0xFFFFFF) - 1;
      pg_off = (int64_t)__builtin_amdgcn_readfirstlane(max(pg, 0)) * p.stride_page_b;
    } else {                       // a page past the held entries: the scalar table
      pg_off = (int64_t)max(page_of(t), 0) * p.stride_page_b;
    }
    const int64_t off = pg_off + (int64_t)(t & ((1 << tpp_shift) - 1)) * C::kTensorBytes;
    // the tile's loads land inside its stage of the ring
    PW_DCHECK(lane != 0 || (t >= 0 && t < n_tiles && SS >= 0 && SS < ST &&
                            ((C::kDmaPerTensor - 1) * NW + wave + 1) * kWave * 16 <= C::kTensorBytes));
    const uint8_t* kt = kbase + off;
    const uint8_t* vt = vbase + off;
    constexpr int GN = C::kDmaGroup;
#pragma unroll
    for (int i = 0; i < C::kDmaPerTensor; i += GN)
      dma16_group<GN, NW * 1024>(dma_off + i, kt, lds_base + SS * C::kStageBytes + (i * NW + wave) * (kWave * 16));
#pragma unroll
    for (int i = 0; i < C::kDmaPerTensor; i += GN)
      dma16_group<GN, NW * 1024>(dma_off + i, vt,
                                 lds_base + SS * C::kStageBytes + C::kTensorBytes + (i * NW + wave) * (kWave * 16));
    return pg_off;
  };

  // ---- running state ------------------------------------------------------------------
  f32x4 o[MT][C::kDt];
  // m_ref: the row's reference, +inf while it has none (so that log2 vs - m_ref is -inf and
  // every P of the row is 0 until the reference is set); thr: rescale threshold of the
  // row-sum share (below)
  float m_ref[MT], l_run[MT], thr[MT];
  int mt_min[MT];   // smallest usable last token over the valid rows of a row tile
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int dt = 0; dt < C::kDt; ++dt) o[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[m] = INFINITY;
    l_run[m] = 0.f;
    thr[m] = -INFINITY;
    int lim = my_bit[m] != 0 ? row_lim[m] : 0x7fffffff;   // my_bit != 0: the row has a query
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) lim = min(lim, __shfl_xor(lim, sh, kWave));
    mt_min[m] = __builtin_amdgcn_readfirstlane(lim);
  }

  refill(0);
  asm volatile("" ::"v"(md_pq), "v"(md_sc), "v"(md_lvs), "v"(md_ivs));
  // Make every earlier global load complete here, before the first direct-to-LDS load is
  // issued: the compiler does not see those loads, so a wait it placed later for its own
  // loads would also wait for the whole ring.
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if constexpr (C::kF8Mma) {
      // (dword by dword: the host pass checks the constraint against its own registers)
#pragma unroll
      for (int w = 0; w < 8; ++w) asm volatile("" ::"v"(qh[m][w]), "v"(ql[m][w]));
      asm volatile("" ::"v"(qs[m]));
    } else {
#pragma unroll
      for (int c = 0; c < C::kDc; ++c) asm volatile("" ::"v"(__builtin_bit_cast(i32x4, qf[m][c])));
    }
    asm volatile("" ::"v"(row_lim[m]), "v"(my_bit[m]));
  }

  // ---- one tile: S^T = K Q^T, masked online softmax, O^T += V^T P^T --------------------
  // what a tile needs of its page: shared by the tiles of one page
  struct PageCtx {
    int pg, qm, abits;        // page (-1: invalid), member mask, bit m: row tile m selects it
    int tok_base;             // the page's first token
    float sc, lvs, inv_vs;    // score scale * ks, log2 vs, 1 / vs
    // per selecting row tile m (bit m of abits): the row's score scale, the bias of the
    // fast-path exponent (log2 vs - reference, or -inf for a row that did not select the page
    // or has no reference yet; kept current when a rescale moves the reference), and the
    // lanes whose row selected the page
    float scm[MT], bias[MT];
    uint64_t selm[MT];
  };
  auto page_ctx = [&](int t) {
    const int ent = t >> tpp_shift;
    if (ent - md_base >= kWave) refill(ent & ~(kWave - 1));   // every 64 pages (uniform)
    const int l = ent - md_base;
    const int pq = lane_i(md_pq, l);
    PageCtx c;
    c.pg = (pq & 0xFFFFFF) - 1;
    c.tok_base = c.pg * p.page_size;
    PW_DCHECK(lane != 0 || (c.pg >= 0 && l >= 0 && l < kWave));   // a listed page, held by the lanes
    c.qm = (int)((uint32_t)pq >> 24);
    // (adds and shifts only: x != 0 as (x + 2^n - 1) >> n for x < 2^n, which the compiler
    // does not turn into compares, so that the mask stays in a scalar register)
    int ab = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) ab |= (int)(((uint32_t)(c.qm & mt_members[m]) + 0xFFu) >> 8) << m;
    c.abits = ab & -(int)((((uint32_t)pq & 0xFFFFFFu) + 0xFFFFFFu) >> 24);   // (none for an invalid page)
    c.sc = lane_f(md_sc, l);
    c.lvs = lane_f(md_lvs, l);
    c.inv_vs = lane_f(md_ivs, l);
    // (the values of a row tile that does not select the page are never read)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if ((c.abits >> m) & 1) {   // uniform
        const bool sel = (c.qm & my_bit[m]) != 0;
        c.scm[m] = C::kF8Mma ? c.sc * qs[m] : c.sc;   // fp8 MFMA: undo the row's 2^e
        c.bias[m] = sel ? c.lvs - m_ref[m] : -INFINITY;   // (-inf too while m_ref = +inf)
        c.selm[m] = __builtin_amdgcn_ballot_w64(sel);
      }
    }
    return c;
  };

  auto compute = [&](int t, auto stage_c, PageCtx& pc) {
    constexpr int SS = decltype(stage_c)::value;
    const int qm = pc.qm;
    const int tok0 = pc.tok_base + (t & ((1 << tpp_shift) - 1)) * kTK;
    // bit m: row tile m selects the page and reaches into the tile.  Uniform; in the held
    // forms built with integer operations only (tok0 <= mt_lim iff the sign bit of
    // mt_lim - tok0 is clear; both are token indices below 2^30), so that it stays in a
    // scalar register (compares leave it in a lane mask that is copied through a vector
    // register; the streamed forms, at their register limit, spill less with compares)
    int act_bits = 0;
    bool act_b[MT];
    if constexpr (C::kStreamK) {
      bool any = false;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        act_b[m] = ((pc.abits >> m) & 1) != 0 && tok0 <= mt_lim[m];
        any |= act_b[m];
      }
      if (!any) return;
    } else {
      int reach = 0;
#pragma unroll
      for (int m = 0; m < MT; ++m) reach |= (int)((~(uint32_t)(mt_lim[m] - tok0)) >> 31) << m;
      act_bits = pc.abits & reach;
      if (act_bits == 0) return;
    }
    auto act = [&](int m) { return C::kStreamK ? act_b[m] : ((act_bits >> m) & 1) != 0; };
    const float sc = pc.sc;
    const float lvs = pc.lvs;
    const float inv_vs = pc.inv_vs;
    const PW_LDS uint8_t* st = lds_p + SS * C::kStageBytes;

    // K fragments (A operand of S^T = K . Q^T), shared by every row tile.  Held form:
    // the whole tile's fragments are read first, then each row tile's MFMAs run.
    // Streamed form: each fragment is read, converted and fed to every active row
    // tile's MFMAs, then dropped (same products, same accumulation order).  With the fp8
    // MFMA a key block's fragment is its 32 e4m3 bytes per lane, used as stored, and one
    // key block costs two MFMAs per row tile (Q's hi and lo parts).
    auto kfrag8 = [&](int kb) -> i32x8 {
      const i32x4 a = *reinterpret_cast<const PW_LDS i32x4*>(st + k_off[kb][0]);
      const i32x4 b = *reinterpret_cast<const PW_LDS i32x4*>(st + k_off[kb][C::kF8Mma ? 1 : 0]);
      return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };
    auto kfrag = [&](int kb, int c) -> bf16x8 {
      if constexpr (FP8) {
        return fp8x8_to_bf16(*reinterpret_cast<const PW_LDS i32x2*>(st + k_off[kb][c]));
      } else {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const PW_LDS i32x4*>(st + k_off[kb][c]));
      }
    };
    bf16x8 ka[C::kStreamK || C::kF8Mma ? 1 : 2][C::kStreamK || C::kF8Mma ? 1 : C::kDc];
    i32x8 ka8[C::kF8Mma && !C::kStreamK ? 2 : 1];
    f32x4 s2all[C::kStreamK ? MT : 1][2];
    if constexpr (C::kStreamK) {
      auto qk_tiles = [&](auto act_c) {
        constexpr int ACT = decltype(act_c)::value;   // bit m: row tile m active
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) s2all[m][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (C::kF8Mma) {   // every hi product before the lo ones that depend on it
            const i32x8 kf = kfrag8(kb);
#pragma unroll
            for (int m = 0; m < MT; ++m)
              if (((ACT >> m) & 1) != 0)
                s2all[m][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qh[m], s2all[m][kb], 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int m = 0; m < MT; ++m)
              if (((ACT >> m) & 1) != 0)
                s2all[m][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, ql[m], s2all[m][kb], 0, 0, 0, 0, 0, 0);
          } else {
#pragma unroll
            for (int c = 0; c < C::kDc; ++c) {
              const bf16x8 kf = kfrag(kb, c);
#pragma unroll
              for (int m = 0; m < MT; ++m)
                if (((ACT >> m) & 1) != 0)
                  s2all[m][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[m][c], s2all[m][kb], 0, 0, 0);
            }
          }
        }
      };
      static_assert(MT <= 2, "row tiles per wave");
      if constexpr (MT == 1) {
        qk_tiles(std::integral_constant<int, 1>{});
      } else {
        if (act(0) && act(1)) qk_tiles(std::integral_constant<int, 3>{});
        else if (act(0)) qk_tiles(std::integral_constant<int, 1>{});
        else qk_tiles(std::integral_constant<int, 2>{});
      }
    } else if constexpr (C::kF8Mma) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ka8[kb] = kfrag8(kb);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < C::kDc; ++c) ka[kb][c] = kfrag(kb, c);
    }

    // V^T fragments (A operand of O^T += V^T . P^T): lane li = d column 16*dt + li, k-slots
    // e = tile keys 8*lq + e.  One-wave items read and convert them here, ahead of the
    // softmax, so that the LDS latency and the conversions overlap the QK MFMAs; the
    // three-wave forms (no registers to spare) read each right before its MFMAs.
    constexpr bool kEarlyV = !C::kStreamK;
    auto vfrag = [&](int dt) -> bf16x8 {
      if constexpr (FP8) {
        return fp8x8_to_bf16(__builtin_amdgcn_ds_read_tr8_b64_v2i32((PW_LDS i32x2*)(st + v_off[dt])));
      } else {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PW_LDS bf16x4*)(st + v_off[2 * dt]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PW_LDS bf16x4*)(st + v_off[2 * dt + 1]));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    // (held form: the reads are issued here and the fp8 codes converted right before the PV
    // MFMAs, after one wait for every LDS read, instead of one wait per fragment)
    bf16x8 va[kEarlyV ? C::kDt : 1];
    i32x2 va8[kEarlyV && FP8 ? C::kDt : 1];
    if constexpr (kEarlyV) {
#pragma unroll
      for (int dt = 0; dt < C::kDt; ++dt) {
        if constexpr (FP8) va8[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PW_LDS i32x2*)(st + v_off[dt]));
        else va[dt] = vfrag(dt);
      }
    }

    bf16x8 pf[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (!kEarlyV) pf[m] = bf16x8{};   // (this form's PV runs every row tile)
      if (!act(m)) continue;
      f32x4 s2[2];
      if constexpr (C::kF8Mma && !C::kStreamK) {   // both key blocks' hi products, then lo
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s2[kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka8[kb], qh[m], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s2[kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka8[kb], ql[m], s2[kb], 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (C::kStreamK) {
          s2[kb] = s2all[m][kb];
        } else if constexpr (!C::kF8Mma) {   // (the held fp8 form computed S above)
          // one-row-tile waves (two of them share an item's ring) raise their priority
          // while they issue MFMAs, so that a wave entering its MFMA block goes ahead of
          // one in its softmax and the two drift into alternating phases (C2 attention
          // 0.143 -> 0.137 ms; the two-row-tile forms gain nothing from it)
          if constexpr (MT == 1) if (kb == 0) __builtin_amdgcn_s_setprio(1);
          s2[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < C::kDc; ++c)
            s2[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][c], qf[m][c], s2[kb], 0, 0, 0);
          if constexpr (MT == 1) if (kb == 1) __builtin_amdgcn_s_setprio(0);
        }
      }
      // lane holds row li of tile m and tile keys 8*lq + 4*kb + ii
      const float scm = pc.scm[m];
      const bool tile_full = tok0 + kTK - 1 <= mt_min[m];          // uniform
      // scores in the log2 domain; keys after a row's last usable token -> -inf.  A tile
      // wholly before every row's limit (the common case) needs no causal compare.
      auto scores = [&](float bias, float* x, auto masked_c, int lim) {
        // key tok0 + 8lq + 4kb + ii is past the row's limit iff 4kb + ii > rel
        const int rel = decltype(masked_c)::value ? lim - tok0 - 8 * lq : 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            float v = __builtin_fmaf(s2[kb][ii], scm, bias);
            if constexpr (decltype(masked_c)::value)
              if (4 * kb + ii > rel) v = -INFINITY;
            x[4 * kb + ii] = v;
          }
      };
      // fast path: P = exp2(s*sc - reference + log2 vs) with the current reference
      float pv[8];
      const float bias0 = pc.bias[m];
      // the lanes whose row reaches into the tile (all in a full tile; tile_full is tested
      // once, so the compiler keeps it a scalar compare rather than a lane mask)
      uint64_t reach_rows = ~uint64_t(0);
      if (tile_full) {
        scores(bias0, pv, std::false_type{}, 0);
      } else {
        scores(bias0, pv, std::true_type{}, row_lim[m]);
        reach_rows = __builtin_amdgcn_ballot_w64(tok0 <= row_lim[m]);
      }
      // P is rounded to bf16 for the PV MFMA, and the row sum adds up exactly those rounded
      // values: numerator and denominator then carry the same weights, so a row whose
      // softmax is dominated by one key gets that key's value without the rounding of its
      // weight (which would otherwise reach 2^-9 of |V|).  This lane's share of the row
      // sum (its 8 of the tile's 32 keys) comes from four bf16 dot products with ones; the
      // four lanes of a row are added up once, in the epilogue.
      auto round_sum = [&](const float* x, bf16x8& pb) {
#pragma unroll
        for (int k = 0; k < 8; ++k) pb[k] = (__bf16)x[k];
        const bf16x2 one{(__bf16)1.0f, (__bf16)1.0f};
        float s01 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0], pb[1]}, one, 0.f, false);
        float s45 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[4], pb[5]}, one, 0.f, false);
        s01 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2], pb[3]}, one, s01, false);
        s45 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[6], pb[7]}, one, s45, false);
        return s01 + s45;
      };
#pragma unroll
      for (int k = 0; k < 8; ++k) pv[k] = __builtin_amdgcn_exp2f(pv[k]);
      float lsum = round_sum(pv, pf[m]);
      // The reference must be set (first used tile of a row) or raised (a lane's share of a
      // row sum passed 2^30, or overflowed): rare, wave-uniform slow path.  The decision is
      // made per row - lanes li, li+16, li+32 and li+48 hold row li - so that every key of
      // a row is exponentiated against the same reference.
      // A lane needs it when its row selected the page and reaches into the tile, and its
      // share of the row sum is above thr (-inf while the row has no reference, else 2^30;
      // the row sum is never negative, so this is "no reference yet, or above 2^30").
      const uint64_t nb = __builtin_amdgcn_ballot_w64(!(lsum * inv_vs <= thr[m])) & pc.selm[m] & reach_rows;
      if (nb) {
        const bool sel = (qm & my_bit[m]) != 0;
        const uint32_t rows = (uint32_t)(nb | (nb >> 16) | (nb >> 32) | (nb >> 48)) & 0xFFFFu;
        const bool need = (rows >> li) & 1u;
        float raw[8];
        // (its own copy of the limit, so that the compiler does not share these compares
        // with the fast path's and hoist them out of its masked branch)
        int lim = row_lim[m];
        asm volatile("" : "+v"(lim));
        scores(sel ? 0.f : -INFINITY, raw, std::true_type{}, lim);
        float mloc = -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k) mloc = fmaxf(mloc, raw[k]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const bool has_ref = m_ref[m] != INFINITY;
        float m_new = need ? (has_ref ? fmaxf(mloc, m_ref[m]) : mloc) : m_ref[m];
        if (m_new == -INFINITY) m_new = INFINITY;   // (no finite score: still no reference)
        const float alpha = has_ref ? __builtin_amdgcn_exp2f(m_ref[m] - m_new) : 0.f;
        l_run[m] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::kDt; ++dt) o[m][dt] *= alpha;
        m_ref[m] = m_new;
        thr[m] = m_new == INFINITY ? -INFINITY : kRescaleShare;
        pc.bias[m] = sel ? lvs - m_new : -INFINITY;   // (the page's next tile)
        // only the rows that moved their reference recompute P: every other row keeps its
        // fast-path values, so a row's arithmetic never depends on its tile-mates
        if (need) {
#pragma unroll
          for (int k = 0; k < 8; ++k) pv[k] = __builtin_amdgcn_exp2f(raw[k] + pc.bias[m]);
          lsum = round_sum(pv, pf[m]);
        }
      }
      l_run[m] += lsum * inv_vs;
    }

    // O^T[d][row] += V^T . P^T.  With the fragments already in registers, each row tile's
    // MFMAs form one block behind one uniform branch, and an inactive row tile (P = 0)
    // skips its block; otherwise every row tile runs (its P is 0 when inactive).
    if constexpr (kEarlyV) {
      // every fragment passes through one empty asm statement, so that the compiler waits
      // once for all of them instead of before each conversion or MFMA
      static_assert(C::kDt == 8 || C::kDt == 4, "d = 128 or 64");
      if constexpr (FP8) {
        if constexpr (C::kDt == 8)
          asm volatile("" : "+v"(va8[0]), "+v"(va8[1]), "+v"(va8[2]), "+v"(va8[3]), "+v"(va8[4]), "+v"(va8[5]),
                       "+v"(va8[6]), "+v"(va8[7]));
        else
          asm volatile("" : "+v"(va8[0]), "+v"(va8[1]), "+v"(va8[2]), "+v"(va8[3]));
#pragma unroll
        for (int dt = 0; dt < C::kDt; ++dt) va[dt] = fp8x8_to_bf16(va8[dt]);
      } else {
        i32x4 vr[C::kDt];
#pragma unroll
        for (int dt = 0; dt < C::kDt; ++dt) vr[dt] = __builtin_bit_cast(i32x4, va[dt]);
        if constexpr (C::kDt == 8)
          asm volatile("" : "+v"(vr[0]), "+v"(vr[1]), "+v"(vr[2]), "+v"(vr[3]), "+v"(vr[4]), "+v"(vr[5]),
                       "+v"(vr[6]), "+v"(vr[7]));
        else
          asm volatile("" : "+v"(vr[0]), "+v"(vr[1]), "+v"(vr[2]), "+v"(vr[3]));
#pragma unroll
        for (int dt = 0; dt < C::kDt; ++dt) va[dt] = __builtin_bit_cast(bf16x8, vr[dt]);
      }
      if constexpr (MT == 1) __builtin_amdgcn_s_setprio(1);   // (see the QK block above)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (MT > 1 && !act(m)) continue;
#pragma unroll
        for (int dt = 0; dt < C::kDt; ++dt)
          o[m][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pf[m], o[m][dt], 0, 0, 0);
      }
      if constexpr (MT == 1) __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int dt = 0; dt < C::kDt; ++dt) {
        const bf16x8 a = vfrag(dt);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          o[m][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[m], o[m][dt], 0, 0, 0);
      }
    }
  };

  // ---- pipeline: tile t lives in stage t % ST; the loop is unrolled by ST so that every
  // stage offset is a compile-time immediate ------------------------------------------------
  // (next_known: the caller knows that tile t + ST - 1 exists; off_next: its page's byte
  // offset, or kNoPage; returns the page offset of the load issued, kNoPage if none)
  auto step = [&](int t, auto stage_c, PageCtx& pc, int64_t off_next, bool next_known = false) {
    constexpr int SS = decltype(stage_c)::value;
    wait_tiles<C::kDmaPerTile, ST - 2>(min(n_tiles - 1 - t, ST - 2));   // tile t has landed
    if constexpr (NW > 1) __builtin_amdgcn_s_barrier();                 // ... for every wave
    int64_t off = kNoPage;
    if (next_known || t + ST - 1 < n_tiles)
      off = issue(t + ST - 1, std::integral_constant<int, (SS + ST - 1) % ST>{}, off_next);
    compute(t, stage_c, pc);
    return off;
  };
  // Several waves over a four-stage ring step by pairs of tiles: tiles t, t + 1 have landed
  // for every wave and every wave is done with t - 2, t - 1, whose stages then take t + 2 and
  // t + 3.  One barrier per two tiles instead of one per tile, two tiles of prefetch instead
  // of three (the 128K block-union chunk: 0.744 -> 0.731 ms).
  constexpr bool kPairs = ST == 4 && NW > 1;
  auto pair = [&](int t, auto sa, auto sb, auto sc, auto sd) {
    wait_vmcnt<0>();                   // this wave's loads of t, t + 1 (nothing newer yet)
    __builtin_amdgcn_s_barrier();      // ... and every other wave's
    if (t + 2 < n_tiles) issue(t + 2, sc, kNoPage);
    if (t + 3 < n_tiles) issue(t + 3, sd, kNoPage);
    {
      PageCtx c = page_ctx(t);
      compute(t, sa, c);
    }
    if (t + 1 < n_tiles) {   // (its page values read after tile t's rescale, if any)
      PageCtx c = page_ctx(t + 1);
      compute(t + 1, sb, c);
    }
  };
  int64_t page_off = kNoPage;   // (two-stage ring) byte offset of the next pair's page
  if (0 < n_tiles) page_off = issue(0, std::integral_constant<int, 0>{}, kNoPage);
  if constexpr (ST > 2) if (1 < n_tiles) issue(1, std::integral_constant<int, 1>{}, kNoPage);
  if constexpr (ST > 3 && !kPairs) if (2 < n_tiles) issue(2, std::integral_constant<int, 2>{}, kNoPage);
  if constexpr (kPairs) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    for (int t0 = 0; t0 < n_tiles; t0 += 4) {
      pair(t0, S0{}, S1{}, S2{}, S3{});
      if (t0 + 2 < n_tiles) pair(t0 + 2, S2{}, S3{}, S0{}, S1{});
    }
  } else if constexpr (ST == 2) {
    // a page holds 2 or 4 tiles (n_tiles is even) and t0 is even, so tile t0 + 1 exists and
    // shares t0's page: its values are read once, and its load needs no page lookup
    for (int t0 = 0; t0 < n_tiles; t0 += 2) {
      PageCtx pc = page_ctx(t0);   // (a rescale in tile t0 updates its bias for t0 + 1)
      step(t0, std::integral_constant<int, 0>{}, pc, page_off, true);
      page_off = step(t0 + 1, std::integral_constant<int, 1>{}, pc, kNoPage);
    }
  } else {
    for (int t0 = 0; t0 < n_tiles; t0 += ST) {
      // (each tile's page values are read after the previous tile's rescale, if any)
      {
        PageCtx c = page_ctx(t0);
        step(t0, std::integral_constant<int, 0>{}, c, kNoPage);
      }
      if (t0 + 1 < n_tiles) {
        PageCtx c = page_ctx(t0 + 1);
        step(t0 + 1, std::integral_constant<int, 1>{}, c, kNoPage);
      }
      if constexpr (ST > 2)
        if (t0 + 2 < n_tiles) {
          PageCtx c = page_ctx(t0 + 2);
          step(t0 + 2, std::integral_constant<int, 2>{}, c, kNoPage);
        }
      if constexpr (ST > 3)
        if (t0 + 3 < n_tiles) {
          PageCtx c = page_ctx(t0 + 3);
          step(t0 + 3, std::integral_constant<int, 3>{}, c, kNoPage);
        }
    }
  }
  wait_vmcnt<0>();

  // ---- epilogue: rows to their original IDs ------------------------------------------
#pragma unroll
  for (int m = 0; m < MT; ++m) {   // the row sums: add the four lanes' shares of each row
    l_run[m] += __shfl_xor(l_run[m], 16, kWave);
    l_run[m] += __shfl_xor(l_run[m], 32, kWave);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int id, hh, slot;
    row_info(m, id, hh, slot);
    if (id < 0) continue;
    const float inv = l_run[m] > 0.f ? 1.0f / l_run[m] : 0.f;
    int64_t orow = (int64_t)id * p.hq + hh;
    if (p.out_slot)          // page-major partial slot
      orow = (int64_t)slot * p.G + (hh - g * p.G);
    else if (p.n_split > 1)  // table-slice partial: slot (q, g, slice)
      orow = (((int64_t)id * p.hkv + g) * p.n_split + slice) * p.G + (hh - g * p.G);
    PW_DCHECK(orow >= 0 && (p.out_slot != nullptr || orow < (int64_t)p.nq * p.hq * max(p.n_split, 1)));
    uint16_t* dst = p.out + orow * D;
#pragma unroll
    for (int dt = 0; dt < C::kDt; ++dt) {
      const bf16x4 v{(__bf16)(o[m][dt][0] * inv), (__bf16)(o[m][dt][1] * inv),
                     (__bf16)(o[m][dt][2] * inv), (__bf16)(o[m][dt][3] * inv)};
      *reinterpret_cast<bf16x4*>(dst + 16 * dt + 4 * lq) = v;
    }
    if (p.lse && lq == 0)
      p.lse[orow] = l_run[m] > 0.f ? (m_ref[m] + __log2f(l_run[m])) * kLn2 : -INFINITY;
  }
}

template <int D, bool FP8, int MT, int NW, int ST>
pw_status launch_t(const Params& p, hipStream_t stream) {
  const int grid = 8 * p.items_per_xcd;
  hipLaunchKernelGGL((k_attn<D, FP8, MT, NW, ST>), dim3(grid), dim3(NW * kWave), 0, stream, p);
  return check_launch("sparse_prefill");
}

// Row tiling: <= 16 rows -> one wave, one row tile; <= 32 -> one wave, two row tiles;
// <= 64 -> two waves of two row tiles.
// Depth of the LDS tile ring.  The ring's LDS is what limits resident waves, and more
// resident waves beat deeper prefetch: one-wave items use 2 stages (fp8 d=128: 16 KiB,
// ten items per CU); items of 2 waves use 2 (3 for page-major items), wider items 4.
// PW_ATTN_STAGES (2, 3 or 4) overrides it for tuning.
template <int D, bool FP8, int MT, int NW>
pw_status launch_nw(const Params& p, hipStream_t stream) {
  static const int env_st = [] {
    const char* e = getenv("PW_ATTN_STAGES");
    const int v = e ? atoi(e) : 0;
    return (v >= 2 && v <= 4) ? v : 0;
  }();
  // two-wave items: 2 stages for tables of many pages (the two tiles of a page then share
  // its values), 3 for page-major items (one page each, nothing to share)
  const int st = env_st ? env_st : (NW == 1 ? 2 : (NW == 2 ? (p.item_kvh ? 3 : 2) : 4));
  if (st == 2) return launch_t<D, FP8, MT, NW, 2>(p, stream);
  if (st == 3) return launch_t<D, FP8, MT, NW, 3>(p, stream);
  return launch_t<D, FP8, MT, NW, 4>(p, stream);
}

// Rows per work item: <= 16 -> one wave, one row tile; <= 32 -> one wave, two row tiles,
// or two waves of one row tile where the one-wave form's ring leaves less than two waves
// per SIMD (bf16, d = 128: 32 KiB per item, five items per CU); more -> 2, 4 or 8 waves
// of two row tiles sharing the LDS ring (the wide forms serve shared per-KV-group tables,
// where every extra row reuses the staged tile).  The two-wave form of a 32-row item
// computes its two row tiles in parallel over the same staged tiles: on the 2K-query GQA
// bf16 chunk 0.180 -> 0.152 ms; where LDS admits two one-wave items per SIMD (fp8) it is
// slower (64K fp8 Top16: 0.313 -> 0.334 ms).  Outputs are identical either way.
template <int D, bool FP8>
pw_status launch_d(const Params& p, int rows, hipStream_t stream) {
  constexpr int kSlots = kTK * D * (FP8 ? 1 : 2) / 1024;    // 1 KiB load slots per tensor
  constexpr bool kSplit32 = Cfg<D, FP8, 2, 1, 2>::kLdsWaves < 2;
  if (rows <= 16) return launch_nw<D, FP8, 1, 1>(p, stream);
  if (rows <= 32) return kSplit32 ? launch_nw<D, FP8, 1, 2>(p, stream) : launch_nw<D, FP8, 2, 1>(p, stream);
  if (rows <= 64) return launch_nw<D, FP8, 2, 2>(p, stream);
  if constexpr (kSlots >= 4) if (rows <= 128) return launch_nw<D, FP8, 2, 4>(p, stream);
  if constexpr (kSlots >= 8) if (rows <= 256) return launch_nw<D, FP8, 2, 8>(p, stream);
  return fail(PW_ERR_UNSUPPORTED, "pw_sparse_prefill: %d rows per work item", rows);
}

}  // namespace

int max_rows_per_item(int d, int kv_dtype) {
  const int slots = kTK * d * (kv_dtype == PW_KV_FP8_E4M3 ? 1 : 2) / 1024;
  return 32 * std::min(8, std::max(2, slots));
}

pw_status launch_sparse_prefill(const AttnArgs& a, hipStream_t stream) {
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_cache = static_cast<const uint8_t*>(a.k_cache);
  p.v_cache = static_cast<const uint8_t*>(a.v_cache);
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.q_pos = a.q_pos;
  p.group_qids = a.group_qids;
  p.group_size = a.group_size;
  p.union_off = a.union_off;
  p.union_pages = a.union_pages;
  p.union_qmask = a.union_qmask;
  p.out = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.item_kvh = a.item_kvh;
  p.item_lo_dev = a.item_lo_dev;
  p.item_hi_dev = a.item_hi_dev;
  p.out_slot = a.out_slot;
  p.item_order = a.n_split == 1 && !a.item_kvh ? a.item_order : nullptr;
  const int esz = a.kv_dtype == PW_KV_FP8_E4M3 ? 1 : 2;
  p.stride_head_b = a.stride_head * esz;
  p.stride_page_b = a.stride_page * esz;
  p.capacity = a.capacity;
  p.nq = a.nq;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.page_size = a.page_size;
  p.n_pages = a.n_pages;
  p.kv_len = a.kv_len;
  p.n_groups = a.n_groups;
  p.max_group = a.max_group;
  p.shared_table = a.shared_table;
  p.n_split = a.n_split;
  p.n_items = a.item_kvh ? a.n_groups : a.hkv * a.n_groups * a.n_split;   // page-major: capacity
  p.items_per_xcd = (p.n_items + 7) / 8;
  p.score_scale = a.sm_scale * kLog2e;
  if (p.n_items == 0) return PW_OK;
  const int rows = a.max_group * p.G;
  const bool fp8 = a.kv_dtype == PW_KV_FP8_E4M3;
  if (a.d == 128) return fp8 ? launch_d<128, true>(p, rows, stream) : launch_d<128, false>(p, rows, stream);
  if (a.d == 64) return fp8 ? launch_d<64, true>(p, rows, stream) : launch_d<64, false>(p, rows, stream);
  return fail(PW_ERR_UNSUPPORTED, "pw_sparse_prefill: d=%d", a.d);
}

}  // namespace pw
