// probe.hip -- measured ceilings that the hot-path kernels are reported
// against beside the published peaks: a plain coalesced streaming read (the
// HBM ceiling of the matvec kernels) and a loop of independent int8 MFMAs
// (the matrix-core ceiling of the GEMM kernels).  Neither computes anything
// of the method; each keeps its work alive through a checksum that is stored
// only if it takes one impossible value.
#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// One non-temporal 16-byte load per lane and many workgroups: of the read
// shapes measured on 35.65 MB (1..4 chunks per lane, 1024..8192 workgroups,
// plain or non-temporal loads) this one streamed fastest.
constexpr int kReadUnroll = 1;     // 16-byte chunks per lane, all loaded before use
constexpr uint32_t kNever = 0x9E3779B9u;

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                         uint32_t *sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x;
  u32x4 v[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const int64_t i = base + 256 * u;
    v[u] = __builtin_nontemporal_load(p + (i < n16 ? i : n16 - 1));
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == kNever) sink[0] = acc;
}

// Four independent accumulating chains per wave; operands change every round
// so no MFMA can be hoisted or merged.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int32_t iters, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, 3 * lane + 1, 5, 7};
  const i32x4 b = {11, lane ^ 5, 13, 17};
  i32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) {
      i32x4 ac = a;
      ac.y ^= c;
      acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ac, b, acc[c], 0, 0, 0);
    }
    a.x += 1;
  }
  uint32_t s = 0;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= (uint32_t)acc[c][r];
  if (s == kNever) sink[0] = s;
}

}  // namespace

hipError_t launch_probe_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t grid = (n16 + 256 * kReadUnroll - 1) / (256 * kReadUnroll);
  hipLaunchKernelGGL(probe_read_kernel, dim3((uint32_t)grid), dim3(256), 0, s,
                     static_cast<const u32x4 *>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int32_t iters, uint32_t *sink, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(kProbeWorkgroups), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace q8
