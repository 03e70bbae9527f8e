// debug.hip -- the LDS poisoning aid of the race tests.  A kernel that reads
// LDS before writing it, or before the barrier that publishes another wave's
// writes, computes from whatever the LDS held, usually the leftovers of an
// identical earlier launch, which hides the bug.  debug_poison_lds_kernel
// fills the LDS of every compute unit with a chosen pattern first; running a
// kernel after different patterns and comparing its outputs then exposes
// such reads.  debug_read_lds_kernel checks that the fill reaches later
// launches (LDS is not cleared between workgroups).  Nothing here is on the
// product path.
#include "launch.h"

namespace q8 {
namespace {

// Every lane stores `pattern` into all kDebugLdsDwords of its workgroup's
// LDS.  Five such workgroups fill a compute unit's 160 KB and the grid gives
// every compute unit several of them; the stores are volatile so none is
// dropped as dead.
__global__ __launch_bounds__(256) void debug_poison_lds_kernel(uint32_t pattern) {
  __shared__ uint32_t lds[kDebugLdsDwords];
  volatile uint32_t *v = lds;
  for (int i = threadIdx.x; i < kDebugLdsDwords; i += 256) v[i] = pattern;
}

// Each workgroup copies the kDebugLdsDwords of LDS it was given, unwritten,
// to its slice of `seen` (volatile loads, so the reads happen).
__global__ __launch_bounds__(256) void debug_read_lds_kernel(uint32_t *seen) {
  __shared__ uint32_t lds[kDebugLdsDwords];
  volatile uint32_t *v = lds;
  for (int i = threadIdx.x; i < kDebugLdsDwords; i += 256)
    seen[(int64_t)blockIdx.x * kDebugLdsDwords + i] = v[i];
}

}  // namespace

hipError_t launch_debug_poison_lds(uint32_t pattern, hipStream_t s) {
  hipLaunchKernelGGL(debug_poison_lds_kernel, dim3(kDebugPoisonWorkgroups), dim3(256), 0, s,
                     pattern);
  return hipGetLastError();
}

hipError_t launch_debug_read_lds(uint32_t *seen, int32_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(debug_read_lds_kernel, dim3((uint32_t)workgroups), dim3(256), 0, s, seen);
  return hipGetLastError();
}

}  // namespace q8
