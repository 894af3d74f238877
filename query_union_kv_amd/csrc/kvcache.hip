// Chunk K/V append into the paged cache, with per-(KV head, page) fp8 e4m3fn
// quantisation (PageWeaver abstract: FP8 KV throughout; CompactAttention
// "Approach": the paged cache is KV-head-major and attention reads it in place).
//
// One workgroup per (touched page, KV head, tensor).  The page's new tokens are
// read once to find their largest magnitude (a block max), the page scale is
// decided, and a second pass - served from L2, the page was just read - writes
// the codes; the page's earlier slots are re-encoded only when its scale grows,
// and slots after the chunk's last token are zeroed.  The kernel is HBM-bound:
// 2 bytes read and 1 (fp8) or 2 (bf16) bytes written per element.
//
// Scale rule per touched (head, page): a = max |x| over the chunk's tokens on the
// page; a page the chunk starts part way into keeps its scale when a/448 does not
// exceed it, else takes a/448 (earlier slots re-encoded from code * old scale);
// any other page takes a/448, or 1 when a == 0.  Every quotient is the correctly
// rounded fp32 division and every code the nearest e4m3fn value, ties to even.

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

// Nearest OCP e4m3fn code of a finite fp32 value with |q| <= 448, ties to the even
// code.  Normal range (|q| >= 2^-6): keep 3 of the 23 mantissa bits with
// round-to-nearest-even on the 20 dropped bits; a carry out of the mantissa moves
// into the exponent field, which is the correctly rounded result.  Subnormal
// range: the value in units of 2^-9 (exact scaling), rounded to an integer
// 0..8 by the hardware's round-to-nearest-even; 8 is the smallest normal's code.
__device__ __forceinline__ uint32_t e4m3_rne(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(q);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t e = (ua >> 23) - 120u;             // rebias 127 -> 7
    const uint32_t m = ua & 0x7FFFFFu;
    const uint32_t r = m >> 20, rem = m & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (r & 1u));
    mag = (e << 3) + r + up;
  }
  return sign | mag;
}

__device__ __forceinline__ uint32_t quant(float x, float s) {
  const float q = fminf(fmaxf(__fdiv_rn(x, s), -448.0f), 448.0f);
  return e4m3_rne(q);
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
// Work unit: 8 consecutive elements of one token (16 bytes of bf16 input).
template <bool FP8>
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

  if constexpr (!FP8) {
    for (int u = u_new0 + threadIdx.x; u < u_end; u += kThreads) {
      const uint4 v = u < u_new1 ? src_unit(u) : make_uint4(0, 0, 0, 0);
      *(uint4*)(dst + (int64_t)u * 16) = v;
    }
    return;
  } else {
    float* scale = (is_v ? p.v_scale : p.k_scale) + (int64_t)g * p.n_pages + page;
    const float s_old = s0 > 0 ? *scale : 0.f;   // read before the barrier in block_max
    float amax = 0.f;
    for (int u = u_new0 + threadIdx.x; u < u_new1; u += kThreads) {
      const uint4 v = src_unit(u);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
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
    if (grow) {
      for (int u = threadIdx.x; u < u_new0; u += kThreads) {
        const uint2 c = *(const uint2*)(dst + (int64_t)u * 8);
        const uint32_t cw[2] = {c.x, c.y};
        uint32_t o[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[h], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[h], true);
          const float x[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int i = 0; i < 4; ++i) o[h] |= quant(x[i] * s_old, s_new) << (8 * i);
        }
        *(uint2*)(dst + (int64_t)u * 8) = make_uint2(o[0], o[1]);
      }
    }
    for (int u = u_new0 + threadIdx.x; u < u_end; u += kThreads) {
      uint32_t o[2] = {0, 0};
      if (u < u_new1) {
        const uint4 v = src_unit(u);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t pair = quant(bf16_lo(w[i]), s_new) | (quant(bf16_hi(w[i]), s_new) << 8);
          o[i >> 1] |= pair << (16 * (i & 1));
        }
      }
      *(uint2*)(dst + (int64_t)u * 8) = make_uint2(o[0], o[1]);
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
  if (esize == 1)
    hipLaunchKernelGGL(k_append<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_append<false>, grid, dim3(kThreads), 0, stream, p);
  return check_launch("pw_append_kv");
}

}  // namespace pw
