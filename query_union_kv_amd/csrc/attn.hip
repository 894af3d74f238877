// ID-aware union attention for gfx950 (CDNA4, wave64, MFMA 16x16x32 bf16).
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
// Work item = (KV head g, group j).  Its rows are (member m, head h) pairs,
// row r = m * G + (h - g*G); wave w of the workgroup owns rows 16w .. 16w+15.
// Every union page is cut into 64-token tiles.  Per tile:
//   * all waves stage K and V (64 x D each) into one of two LDS buffers
//     (global -> registers -> LDS, prefetching the next tile while computing);
//   * S^T[key][row] = K . Q^T on MFMA (keys are the MFMA rows, so each lane
//     ends with one query row and 16 of its keys, and row statistics stay in
//     the lane);
//   * support mask (member selected the page) + causal mask, online softmax in
//     the log2 domain;
//   * O^T[d][row] += V^T . P^T on MFMA, V^T read from LDS with the CDNA4
//     transposing loads (ds_read_b64_tr_b8 / _b16).
// fp8 (OCP e4m3fn) codes are converted exactly to bf16; the K page scale folds
// into the score scale and the V page scale into P (the row sum uses unscaled P).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace pw {
namespace {

constexpr int kWave = 64;
constexpr int kTile = 64;          // tokens per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define PW_LDS __attribute__((address_space(3)))

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
  int64_t stride_head_b;   // bytes
  int64_t stride_page_b;   // bytes
  int64_t capacity;
  int nq, hq, hkv, G;
  int page_size, n_pages, kv_len;
  int n_groups, max_group, shared_table;
  int n_items, items_per_xcd;
  float score_scale;       // sm_scale * log2(e)
};

// XOR swizzle of 16-byte chunks inside an LDS row; keeps the MFMA operand reads and
// the transposing V reads spread over distinct banks.
template <int CHUNKS>
__device__ __forceinline__ int swz(int row) {
  const int f = ((row >> 1) & 1) | ((((row >> 2) ^ (row >> 4)) & 1) << 1) | (((row >> 3) & 1) << 2) |
                (((row >> 0) & 1) << 3);
  return f & (CHUNKS - 1);
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int D, bool FP8, int NW>
struct Cfg {
  static constexpr int kEsz = FP8 ? 1 : 2;
  static constexpr int kRowBytes = D * kEsz;               // one token row of K or V
  static constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr int kTensorBytes = kTile * kRowBytes;   // K or V tile
  static constexpr int kStageBytes = 2 * kTensorBytes;
  static constexpr int kThreads = NW * kWave;
  static constexpr int kTotalChunks = 2 * kTile * kChunks;  // K and V of one tile
  static constexpr int kChunksPerThread = (kTotalChunks + kThreads - 1) / kThreads;
  static constexpr bool kRagged = kTotalChunks % kThreads != 0;
  static constexpr int kDc = D / 32;                        // MFMA k-steps over d
  static constexpr int kDt = D / 16;                        // 16-wide d tiles of O
};

template <int D, bool FP8, int NW>
__global__ __launch_bounds__(NW * kWave) void k_attn(Params p) {
  using C = Cfg<D, FP8, NW>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::kStageBytes];

  // XCD-aware work order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // range of items (KV-head-major), so one XCD's L2 serves neighbouring groups of the
  // same KV head.
  const int b = blockIdx.x;
  const int item = (b & 7) * p.items_per_xcd + (b >> 3);
  if (item >= p.n_items) return;
  const int g = item / p.n_groups;
  const int j = item - g * p.n_groups;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int li = lane & 15;      // MFMA row/col index inside a 16-lane group
  const int lq = lane >> 4;      // 16-lane group 0..3

  // ---- members and this lane's query row ------------------------------------------
  int gsize;
  const int32_t* qids = nullptr;
  if (p.group_qids) {
    gsize = min(max(p.group_size[item], 0), p.max_group);
    qids = p.group_qids + (int64_t)item * p.max_group;
  } else {
    gsize = min(p.max_group, p.nq - j * p.max_group);
  }
  const int row = wave * 16 + li;
  const int member = row / p.G;
  const int h = g * p.G + (row - member * p.G);
  int qid = -1;
  if (member < gsize) qid = qids ? qids[member] : j * p.max_group + member;
  if (qid >= p.nq) qid = -1;
  const bool row_valid = qid >= 0;
  const int qpos = row_valid ? p.q_pos[qid] : -1;
  const int row_lim = min(qpos, p.kv_len - 1);   // last usable token of this row

  // members owned by this wave (bit m) and the wave's last usable token
  int wave_members = 0;
  for (int r = wave * 16; r < wave * 16 + 16; ++r) {
    const int m = r / p.G;
    if (m < gsize) wave_members |= 1 << m;
  }
  int wave_lim = row_lim;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) wave_lim = max(wave_lim, __shfl_xor(wave_lim, o, kWave));

  // ---- Q^T fragments (B operand of S^T = K . Q^T): row li, d = 32c + 8lq .. +8 ------
  bf16x8 qf[C::kDc];
#pragma unroll
  for (int c = 0; c < C::kDc; ++c) {
    if (row_valid) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(p.q + ((int64_t)qid * p.hq + h) * D + 32 * c + 8 * lq);
      qf[c] = __builtin_bit_cast(bf16x8, v);
    } else {
      qf[c] = bf16x8{};
    }
  }

  // ---- table of this item -----------------------------------------------------------
  const int table = p.shared_table ? g : item;
  const int64_t e_begin = min<int64_t>(max(p.union_off[table], 0), p.capacity);
  const int64_t e_end = min<int64_t>(p.union_off[table + 1], p.capacity);
  const int tpp = p.page_size / kTile;                       // tiles per page
  const int n_tiles = (int)max<int64_t>(e_end - e_begin, 0) * tpp;

  const uint8_t* kbase = p.k_cache + (int64_t)g * p.stride_head_b;
  const uint8_t* vbase = p.v_cache + (int64_t)g * p.stride_head_b;

  // per-tile metadata, uniform over the workgroup
  struct Meta { int page, sub, qm; float ks, vs; };
  auto meta_of = [&](int t) -> Meta {
    Meta m;
    const int64_t e = e_begin + t / tpp;
    m.sub = t - (t / tpp) * tpp;
    m.page = p.union_pages[e];
    m.qm = p.union_qmask ? p.union_qmask[e] : 0xFF;
    if (m.page < 0 || m.page >= p.n_pages) { m.page = -1; m.qm = 0; }
    m.ks = 1.0f;
    m.vs = 1.0f;
    if (FP8 && m.page >= 0) {
      m.ks = p.k_scale[(int64_t)g * p.n_pages + m.page];
      m.vs = p.v_scale[(int64_t)g * p.n_pages + m.page];
    }
    return m;
  };

  // ---- staging: global -> registers -> LDS ------------------------------------------
  i32x4 stage_regs[C::kChunksPerThread];
  auto load_tile = [&](const Meta& m) {
    if (m.page < 0) return;
    const int64_t off = (int64_t)m.page * p.stride_page_b + (int64_t)m.sub * kTile * C::kRowBytes;
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int cid = tid + i * C::kThreads;                 // 0 .. kTotalChunks-1
      if (C::kRagged && cid >= C::kTotalChunks) break;
      const int tensor = cid / (kTile * C::kChunks);
      const int rem = cid - tensor * (kTile * C::kChunks);
      const uint8_t* src = (tensor ? vbase : kbase) + off + (int64_t)rem * 16;
      stage_regs[i] = *reinterpret_cast<const i32x4*>(src);
    }
  };
  auto store_tile = [&](int stage, const Meta& m) {
    if (m.page < 0) return;
    uint8_t* dst = lds + stage * C::kStageBytes;
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int cid = tid + i * C::kThreads;
      if (C::kRagged && cid >= C::kTotalChunks) break;
      const int tensor = cid / (kTile * C::kChunks);
      const int rem = cid - tensor * (kTile * C::kChunks);
      const int r = rem / C::kChunks;
      const int ch = rem - r * C::kChunks;
      *reinterpret_cast<i32x4*>(dst + tensor * C::kTensorBytes + r * C::kRowBytes +
                                ((ch ^ swz<C::kChunks>(r)) << 4)) = stage_regs[i];
    }
  };

  // ---- running state ------------------------------------------------------------------
  f32x4 o[C::kDt];
#pragma unroll
  for (int t = 0; t < C::kDt; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int my_bit = row_valid ? (1 << member) : 0;

  Meta cur = n_tiles > 0 ? meta_of(0) : Meta{-1, 0, 0, 1.f, 1.f};
  if (n_tiles > 0) {
    load_tile(cur);
    store_tile(0, cur);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    Meta nxt{-1, 0, 0, 1.f, 1.f};
    if (t + 1 < n_tiles) {
      nxt = meta_of(t + 1);
      load_tile(nxt);
    }
    const int tok0 = cur.page * p.page_size + cur.sub * kTile;
    const bool wave_active = cur.page >= 0 && (cur.qm & wave_members) != 0 && tok0 <= wave_lim;
    if (wave_active) {
      const uint8_t* kt = lds + stage * C::kStageBytes;
      const uint8_t* vt = kt + C::kTensorBytes;
      // S^T blocks: MFMA row i of key block kb holds key pi(kb, i)
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int key = 32 * (kb >> 1) + 8 * (li >> 2) + 4 * (kb & 1) + (li & 3);
        const uint8_t* krow = kt + key * C::kRowBytes;
#pragma unroll
        for (int c = 0; c < C::kDc; ++c) {
          const int byte = (32 * c + 8 * lq) * C::kEsz;
          const int ch = byte >> 4;
          const uint8_t* src = krow + ((ch ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
          bf16x8 a;
          if constexpr (FP8) {
            a = fp8x8_to_bf16(*reinterpret_cast<const i32x2*>(src));
          } else {
            a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(src));
          }
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], s[kb], 0, 0, 0);
        }
      }
      // lane holds row li and keys 32*(kb>>1) + 8*lq + 4*(kb&1) + ii
      const bool sel = (cur.qm & my_bit) != 0;
      const float sc = p.score_scale * cur.ks;
      const bool full = tok0 + kTile - 1 <= row_lim;
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int key = 32 * (kb >> 1) + 8 * lq + 4 * (kb & 1) + ii;
          const bool ok = sel && (full || tok0 + key <= row_lim);
          const float v = ok ? s[kb][ii] * sc : -INFINITY;
          s[kb][ii] = v;
          mloc = fmaxf(mloc, v);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float e = __builtin_amdgcn_exp2f(s[kb][ii] - m_use);
          s[kb][ii] = e;
          lsum += e;
        }
      lsum += __shfl_xor(lsum, 16, kWave);
      lsum += __shfl_xor(lsum, 32, kWave);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < C::kDt; ++dt) o[dt] *= alpha;
      // P^T operand (B): chunk c2 covers keys 32*c2 + 8*lq + 0..7 = blocks 2c2 (0..3), 2c2+1 (4..7)
      bf16x8 pf[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          pf[c2][ii] = (__bf16)(s[2 * c2][ii] * cur.vs);
          pf[c2][4 + ii] = (__bf16)(s[2 * c2 + 1][ii] * cur.vs);
        }
      }
      // O^T[d][row] += V^T . P^T ; A operand lane li = d column, keys 32*c2 + 8*lq + 0..7
#pragma unroll
      for (int dt = 0; dt < C::kDt; ++dt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          bf16x8 a;
          if constexpr (FP8) {
            // byte e of output lane li = V[key0 + e][16*dt + li]; source lane li reads
            // key0 + (li >> 1), columns 16*dt + 8*(li & 1) .. +8
            const int key = 32 * c2 + 8 * lq + (li >> 1);
            const int byte = 16 * dt + 8 * (li & 1);
            const uint8_t* src = vt + key * C::kRowBytes + (((byte >> 4) ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
            const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PW_LDS i32x2*)(src));
            a = fp8x8_to_bf16(raw);
          } else {
            // element e of output lane li = V[key0 + e][16*dt + li]; source lane li reads
            // key0 + (li >> 2), columns 16*dt + 4*(li & 3) .. +4
            bf16x4 lo, hi;
            {
              const int key = 32 * c2 + 8 * lq + (li >> 2);
              const int byte = (16 * dt + 4 * (li & 3)) * 2;
              const uint8_t* src = vt + key * C::kRowBytes + (((byte >> 4) ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
              lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PW_LDS bf16x4*)(src));
            }
            {
              const int key = 32 * c2 + 8 * lq + 4 + (li >> 2);
              const int byte = (16 * dt + 4 * (li & 3)) * 2;
              const uint8_t* src = vt + key * C::kRowBytes + (((byte >> 4) ^ swz<C::kChunks>(key)) << 4) + (byte & 15);
              hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PW_LDS bf16x4*)(src));
            }
            a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[c2], o[dt], 0, 0, 0);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile(stage ^ 1, nxt);
    __syncthreads();
    cur = nxt;
  }

  // ---- epilogue: rows to their original IDs ------------------------------------------
  if (row_valid) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    uint16_t* dst = p.out + ((int64_t)qid * p.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < C::kDt; ++dt) {
      const bf16x4 v{(__bf16)(o[dt][0] * inv), (__bf16)(o[dt][1] * inv), (__bf16)(o[dt][2] * inv),
                     (__bf16)(o[dt][3] * inv)};
      *reinterpret_cast<bf16x4*>(dst + 16 * dt + 4 * lq) = v;
    }
    if (p.lse && lq == 0)
      p.lse[(int64_t)qid * p.hq + h] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, bool FP8, int NW>
pw_status launch_t(const Params& p, hipStream_t stream) {
  const int grid = 8 * p.items_per_xcd;
  hipLaunchKernelGGL((k_attn<D, FP8, NW>), dim3(grid), dim3(NW * kWave), 0, stream, p);
  return check_launch("sparse_prefill");
}

template <int D, bool FP8>
pw_status launch_d(const Params& p, int nw, hipStream_t stream) {
  switch (nw) {
    case 1: return launch_t<D, FP8, 1>(p, stream);
    case 2: return launch_t<D, FP8, 2>(p, stream);
    case 3: return launch_t<D, FP8, 3>(p, stream);
    case 4: return launch_t<D, FP8, 4>(p, stream);
  }
  return fail(PW_ERR_UNSUPPORTED, "pw_sparse_prefill: %d waves", nw);
}

}  // namespace

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
  p.n_items = a.hkv * a.n_groups;
  p.items_per_xcd = (p.n_items + 7) / 8;
  p.score_scale = a.sm_scale * kLog2e;
  if (p.n_items == 0) return PW_OK;
  const int rows = a.max_group * p.G;
  const int nw = (rows + 15) / 16;
  const bool fp8 = a.kv_dtype == PW_KV_FP8_E4M3;
  if (a.d == 128) return fp8 ? launch_d<128, true>(p, nw, stream) : launch_d<128, false>(p, nw, stream);
  if (a.d == 64) return fp8 ? launch_d<64, true>(p, nw, stream) : launch_d<64, false>(p, nw, stream);
  return fail(PW_ERR_UNSUPPORTED, "pw_sparse_prefill: d=%d", a.d);
}

}  // namespace pw
