// Chunk K/V append into the paged cache, with per-(KV head, page) fp8 e4m3fn
// quantisation (PageWeaver abstract: FP8 KV throughout; CompactAttention
// "Approach": the paged cache is KV-head-major and attention reads it in place).
//
// One workgroup per (touched page, KV head, tensor).  The page's new tokens are
// loaded into registers (every load in flight at once), a block max over them
// decides the page scale, and the codes are written from the registers; the
// page's earlier slots are re-encoded only when its scale grows, and slots after
// the chunk's last token are zeroed.  The kernel is HBM-bound:
// 2 bytes read and 1 (fp8) or 2 (bf16) bytes written per element.
//
// Scale rule per touched (head, page): a = max |x| over the chunk's tokens on the
// page; a page the chunk starts part way into keeps its scale when a/448 does not
// exceed it, else takes a/448 (earlier slots re-encoded from code * old scale);
// any other page takes a/448, or 1 when a == 0.  Every code is the nearest e4m3fn
// value to the correctly rounded fp32 quotient x / scale, ties to even (computed by
// a reciprocal product wherever that provably gives the same code).

#include <hip/hip_runtime.h>

#include "common.h"

namespace pw {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t stride_tok;       // elements between consecutive tokens of k_new / v_new
  int d, ps, n_pages;
  int first_token, last_token, first_page;
  uint8_t* k_cache;
  uint8_t* v_cache;
  float* k_scale;
  float* v_scale;
  int64_t stride_head_b, stride_page_b;   // bytes
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Codes of e4m3fn(clamp(RN(x / s), -448, 448)) for two values, as two bytes.
//
// v_cvt_pk_fp8_f32 rounds fp32 to OCP e4m3fn to nearest, ties to even, and maps
// (448, 449] to 448 (measured on every fp32 magnitude up to 449, both signs), so
// code(v) = e4m3fn(clamp(v)) is monotone in v there.  With r = RN(1/s) and s a normal
// number well inside the exponent range, q = RN(x * r) is within 3 units of 2^-24 of
// RN(x / s) (relative), so RN(x / s) - clamped to 448 when q is - lies between
// q * (1 - 2^-21) and q * (1 + 2^-21) even after those products round: when the two
// ends get the same code, so does RN(x / s).  Only otherwise (a value within a few
// ulps of a rounding boundary, or an exact tie) is the correctly rounded quotient
// computed.  fast == false always divides.
constexpr float kDown = 1.0f - 0x1p-21f;
constexpr float kUp = 1.0f + 0x1p-21f;

__device__ __forceinline__ uint32_t quant2(float x0, float x1, float s, float r, bool fast) {
  if (fast) {
    const float q0 = __builtin_amdgcn_fmed3f(x0 * r, -448.0f, 448.0f);
    const float q1 = __builtin_amdgcn_fmed3f(x1 * r, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0 * kDown, q1 * kDown, 0, false);
    const int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q0 * kUp, q1 * kUp, 0, false);
    if (((lo ^ hi) & 0xFFFF) == 0) return (uint32_t)lo & 0xFFFFu;
  }
  const float q0 = __builtin_amdgcn_fmed3f(__fdiv_rn(x0, s), -448.0f, 448.0f);
  const float q1 = __builtin_amdgcn_fmed3f(__fdiv_rn(x1, s), -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[w]);
  return r;
}

// blockIdx.x: page - first_page, blockIdx.y: KV head, blockIdx.z: 0 = K, 1 = V.
// Work unit: 8 consecutive elements of one token (16 bytes of bf16 input); thread t
// owns units t + 256 i.  With UPT > 0 a page has at most 256 * UPT units and each
// thread keeps its units in registers, all loads in flight at once; UPT == 0 is
// the general form for larger pages (two passes, the second served from L2).
template <bool FP8, int UPT>
__global__ __launch_bounds__(kThreads) void k_append(AppendParams p) {
  __shared__ float red[kWaves];
  const int page = p.first_page + (int)blockIdx.x;
  const int g = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const uint16_t* src = (is_v ? p.v_new : p.k_new) + (int64_t)g * p.d;
  uint8_t* dst = (is_v ? p.v_cache : p.k_cache) + g * p.stride_head_b + page * p.stride_page_b;
  const int base = page * p.ps;
  const int s0 = max(p.first_token - base, 0);            // first slot the chunk writes
  const int s1 = min(p.last_token - base, p.ps - 1) + 1;  // one past its last slot
  const int cpr = p.d >> 3;                               // units per token
  const int u_end = p.ps * cpr;
  const int u_new0 = s0 * cpr, u_new1 = s1 * cpr;
  auto src_unit = [&](int u) -> uint4 {
    const int s = u / cpr, c = (u - s * cpr) << 3;
    return *(const uint4*)(src + (int64_t)(base + s - p.first_token) * p.stride_tok + c);
  };
  auto is_new = [&](int u) { return u >= u_new0 && u < u_new1; };

  if constexpr (!FP8) {
    if constexpr (UPT > 0) {
      uint4 v[UPT];
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int u = threadIdx.x + i * kThreads;
        v[i] = is_new(u) ? src_unit(u) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int u = threadIdx.x + i * kThreads;
        if (u >= u_new0 && u < u_end) *(uint4*)(dst + (int64_t)u * 16) = v[i];
      }
    } else {
      for (int u = u_new0 + threadIdx.x; u < u_end; u += kThreads) {
        const uint4 v = u < u_new1 ? src_unit(u) : make_uint4(0, 0, 0, 0);
        *(uint4*)(dst + (int64_t)u * 16) = v;
      }
    }
    return;
  } else {
    float* scale = (is_v ? p.v_scale : p.k_scale) + (int64_t)g * p.n_pages + page;
    const float s_old = s0 > 0 ? *scale : 0.f;   // read before the barrier in block_max
    auto unit_max = [](const uint4& v) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
      return m;
    };
    auto encode_unit = [](const uint4& v, float s, float r, bool fast) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t pair = quant2(bf16_lo(w[i]), bf16_hi(w[i]), s, r, fast);
        o[i >> 1] |= pair << (16 * (i & 1));
      }
      return make_uint2(o[0], o[1]);
    };
    [[maybe_unused]] uint4 v[UPT > 0 ? UPT : 1];
    float amax = 0.f;
    if constexpr (UPT > 0) {
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int u = threadIdx.x + i * kThreads;
        v[i] = is_new(u) ? src_unit(u) : make_uint4(0, 0, 0, 0);   // zeros: |0| leaves the max
      }
#pragma unroll
      for (int i = 0; i < UPT; ++i) amax = fmaxf(amax, unit_max(v[i]));
    } else {
      for (int u = u_new0 + threadIdx.x; u < u_new1; u += kThreads) amax = fmaxf(amax, unit_max(src_unit(u)));
    }
    amax = block_max(amax, red);
    float s_new = __fdiv_rn(amax, 448.0f);
    bool grow = false;
    if (s0 > 0) {
      grow = s_new > s_old;
      if (!grow) s_new = s_old;
    } else if (amax == 0.f) {
      s_new = 1.f;
    }
    const float r_new = __fdiv_rn(1.0f, s_new);
    const bool fast = s_new >= 0x1p-100f && s_new <= 0x1p100f;
    if (grow) {   // a mid-page chunk raised the scale: re-encode the page's earlier slots
      for (int u = threadIdx.x; u < u_new0; u += kThreads) {
        const uint2 c = *(const uint2*)(dst + (int64_t)u * 8);
        const uint32_t cw[2] = {c.x, c.y};
        uint32_t o[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[h], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[h], true);
          const float x[4] = {lo[0], lo[1], hi[0], hi[1]};
          o[h] = quant2(x[0] * s_old, x[1] * s_old, s_new, r_new, fast) |
                 (quant2(x[2] * s_old, x[3] * s_old, s_new, r_new, fast) << 16);
        }
        *(uint2*)(dst + (int64_t)u * 8) = make_uint2(o[0], o[1]);
      }
    }
    if constexpr (UPT > 0) {
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int u = threadIdx.x + i * kThreads;
        // slots past the chunk hold zeros in v[i], which encode to code 0
        if (u >= u_new0 && u < u_end) *(uint2*)(dst + (int64_t)u * 8) = encode_unit(v[i], s_new, r_new, fast);
      }
    } else {
      for (int u = u_new0 + threadIdx.x; u < u_end; u += kThreads)
        *(uint2*)(dst + (int64_t)u * 8) =
            u < u_new1 ? encode_unit(src_unit(u), s_new, r_new, fast) : make_uint2(0, 0);
    }
    if (threadIdx.x == 0) *scale = s_new;
  }
}

}  // namespace

pw_status launch_append_kv(const void* k_new, const void* v_new, int n_tok, int hkv, int d,
                           int64_t stride_tok, int first_token, void* k_cache, void* v_cache,
                           int kv_dtype, float* k_scale, float* v_scale, int page_size,
                           int n_pages, int64_t stride_head, int64_t stride_page,
                           hipStream_t stream) {
  if (n_tok == 0) return PW_OK;
  const int esize = kv_dtype == PW_KV_FP8_E4M3 ? 1 : 2;
  AppendParams p;
  p.k_new = (const uint16_t*)k_new;
  p.v_new = (const uint16_t*)v_new;
  p.stride_tok = stride_tok;
  p.d = d;
  p.ps = page_size;
  p.n_pages = n_pages;
  p.first_token = first_token;
  p.last_token = first_token + n_tok - 1;
  p.first_page = first_token / page_size;
  p.k_cache = (uint8_t*)k_cache;
  p.v_cache = (uint8_t*)v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.stride_head_b = stride_head * esize;
  p.stride_page_b = stride_page * esize;
  const dim3 grid(p.last_token / page_size - p.first_page + 1, hkv, 2);
  const int units = page_size * (d / 8);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, p); };
  if (esize == 1) {
    if (units <= kThreads * 4) go(k_append<true, 4>);
    else if (units <= kThreads * 8) go(k_append<true, 8>);
    else go(k_append<true, 0>);
  } else {
    if (units <= kThreads * 4) go(k_append<false, 4>);
    else if (units <= kThreads * 8) go(k_append<false, 8>);
    else go(k_append<false, 0>);
  }
  return check_launch("pw_append_kv");
}

}  // namespace pw
