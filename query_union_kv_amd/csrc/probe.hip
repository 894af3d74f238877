// Read-bandwidth probes for the benchmark (libpw_probe.so; not part of the method).
//
// The union attention reads every group's union pages once, but the same pages are read
// by many groups, and those re-reads are served by the caches (the 4 MB L2 of each XCD,
// the 256 MB last-level cache) rather than by HBM.  These kernels measure what each level
// delivers to the compute units for plain streaming reads, so that the attention's
// logical read rate can be put against a measured peak of the level that serves it:
//   mode 0  vector loads (global_load_dwordx4), eight 16-byte loads in flight per lane;
//   mode 1  direct global -> LDS loads (global_load_lds_dwordx4, the attention's load
//           path), twelve to sixteen 1 KiB wave loads in flight per wave.
// Workgroup b reads `seg` contiguous bytes at offset (b * seg) mod bytes: with a buffer of
// a few MiB every XCD re-reads the same lines from its L2; with 128 MiB the lines come
// from the last-level cache once it is warm; with several GiB they come from HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_read_vec(const uint4* __restrict__ buf, int64_t n16,
                                                       int64_t seg16, uint32_t* __restrict__ sink) {
  const int64_t base = ((int64_t)blockIdx.x * seg16) % n16;
  const uint4* p = buf + base;
  uint32_t acc = 0;
  // seg16 is a multiple of 8 * kThreads (checked on the host): no partial steps
  for (int64_t i = threadIdx.x; i < seg16; i += 8 * kThreads) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[i + k * kThreads];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // a store the compiler cannot rule out keeps the loads live
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Twelve to sixteen direct-to-LDS loads per wave in flight: each wave owns 16 KiB of LDS, load k of a
// group lands at its slot k (1 KiB: 16 bytes per lane).  The LDS contents are never read.
__global__ __launch_bounds__(kThreads) void k_read_lds(const uint8_t* __restrict__ buf, int64_t bytes,
                                                       int64_t seg, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * 16 * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * seg) % bytes;
  const uint8_t* p = buf + base;
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(lds + wave * 16384);
  // a wave's step covers 16 KiB; the 4 waves of the workgroup interleave by 16 KiB
  for (int64_t off = (int64_t)wave * 16384; off < seg; off += 4 * 16384) {
    const uint8_t* s = p + off;
    const uint32_t v0 = (uint32_t)lane * 16;
    asm volatile(
        "s_waitcnt vmcnt(12)\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:2048\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:3072\n\t"
        :
        : "v"(v0), "s"(m0), "s"(s)
        : "memory", "m0");
    asm volatile(
        "s_waitcnt vmcnt(12)\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:2048\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:3072\n\t"
        :
        : "v"(v0), "s"(m0 + 4096), "s"(s + 4096)
        : "memory", "m0");
    asm volatile(
        "s_waitcnt vmcnt(12)\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:2048\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:3072\n\t"
        :
        : "v"(v0), "s"(m0 + 8192), "s"(s + 8192)
        : "memory", "m0");
    asm volatile(
        "s_waitcnt vmcnt(12)\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:2048\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:3072\n\t"
        :
        : "v"(v0), "s"(m0 + 12288), "s"(s + 12288)
        : "memory", "m0");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (threadIdx.x == 0) sink[blockIdx.x] = 1u;
}

}  // namespace

extern "C" {

// Reads n_blocks * seg bytes of buf (bytes long) with workgroup b at offset
// (b * seg) % bytes; sink receives one word per workgroup.  Returns 0, or -1 on bad
// arguments (nothing launched): bytes % seg != 0, seg not a multiple of 32 KiB (mode 0)
// or 64 KiB (mode 1), misaligned buf, or mode not 0/1; -4 if the launch failed.
int pwp_read(const void* buf, int64_t bytes, int64_t seg, int n_blocks, int mode, uint32_t* sink,
             hipStream_t stream) {
  if (!buf || !sink || bytes <= 0 || seg <= 0 || n_blocks <= 0 || bytes % seg) return -1;
  if ((uintptr_t)buf % 16) return -1;
  if (mode == 0) {
    if (seg % (16 * 8 * kThreads)) return -1;
    hipLaunchKernelGGL(k_read_vec, dim3(n_blocks), dim3(kThreads), 0, stream, (const uint4*)buf,
                       bytes / 16, seg / 16, sink);
  } else if (mode == 1) {
    if (seg % (4 * 16384)) return -1;
    hipLaunchKernelGGL(k_read_lds, dim3(n_blocks), dim3(kThreads), 0, stream, (const uint8_t*)buf,
                       bytes, seg, sink);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
