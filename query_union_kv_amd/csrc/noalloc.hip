// An entry point that allocates nothing: pw_shared_table_prefill with its slice partials
// in a file-scope device array owned by the library (one per device, held until the
// process ends), for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per device
constexpr int kMaxDevices = 64;

// In host code this name is a host-side stand-in, not a device address: only the address
// returned by hipGetSymbolAddress (per device) is passed to kernels.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up once per device with that device current.
pw_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return pw::fail(PW_ERR_HIP, "pw_shared_table_prefill_noalloc: hipGetDevice: %s (device %d)",
                    hipGetErrorString(e), dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return pw::fail(PW_ERR_HIP, "pw_shared_table_prefill_noalloc: hipGetSymbolAddress: %s",
                      hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PW_OK;
}

}  // namespace

extern "C" {

size_t pw_noalloc_scratch_bytes(void) { return kScratchBytes; }

pw_status pw_shared_table_prefill_noalloc(const void* q, int nq, int hq, int hkv, int d,
                                          const void* k_cache, const void* v_cache, int kv_dtype,
                                          const float* k_scale, const float* v_scale, int page_size,
                                          int n_pages, int64_t stride_head, int64_t stride_page,
                                          const int32_t* q_pos, int kv_len, float sm_scale,
                                          int max_group, const int32_t* union_off,
                                          const int32_t* union_pages, int64_t capacity, int n_split,
                                          void* out, float* lse, hipStream_t stream) {
  void* part_o = nullptr;
  float* part_lse = nullptr;
  if (n_split > 1 && nq > 0 && hq > 0 && d > 0) {
    // partial rows (q, g, slice, h): bf16 rows of d, then their fp32 lse, 256-byte aligned
    const int64_t rows = (int64_t)nq * hq * n_split;
    const int64_t o_bytes = (rows * d * 2 + 255) / 256 * 256;
    const int64_t need = o_bytes + rows * 4;
    if (need > (int64_t)kScratchBytes)
      return pw::fail(PW_ERR_CAPACITY,
                      "pw_shared_table_prefill_noalloc: partials need %lld bytes (nq*hq*n_split = %lld "
                      "rows) > the %zu-byte scratch array",
                      (long long)need, (long long)rows, kScratchBytes);
    void* base = nullptr;
    const pw_status st = scratch_address(&base);
    if (st != PW_OK) return st;
    part_o = base;
    part_lse = reinterpret_cast<float*>(static_cast<uint8_t*>(base) + o_bytes);
  }
  return pw_shared_table_prefill(q, nq, hq, hkv, d, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                 page_size, n_pages, stride_head, stride_page, q_pos, kv_len,
                                 sm_scale, max_group, union_off, union_pages, capacity, n_split,
                                 part_o, part_lse, out, lse, stream);
}

}  // extern "C"
