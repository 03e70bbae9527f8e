// q8_device.h -- device-side helpers shared by the gfx950 kernels of this
// library (block layout constants, binary16 decode, dword-aligned loads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

constexpr int kBlockElems = 32;  // values per Q8_0 block
constexpr int kBlockBytes = 34;  // binary16 scale + 32 int8 quants
constexpr int kPairBytes = 68;   // two consecutive blocks = 17 dwords
constexpr int kPairDwords = 17;

// 16-byte vector of dwords that only promises 4-byte alignment: gfx950 global
// loads/stores accept dword-aligned dwordx4 accesses.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// Load the 17 dwords of a block pair (68 bytes, dword aligned).
__device__ __forceinline__ void load_pair(const uint8_t *p, uint32_t (&d)[kPairDwords]) {
  const u32x4_a4 *v = reinterpret_cast<const u32x4_a4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4_a4 t = v[i];
    d[4 * i + 0] = t.x;
    d[4 * i + 1] = t.y;
    d[4 * i + 2] = t.z;
    d[4 * i + 3] = t.w;
  }
  d[16] = reinterpret_cast<const uint32_t *>(p)[16];
}

// Exact int32 dot products of the two blocks of a pair, w against x, both in
// raw pair layout: dword 0 = [dA lo, dA hi, qA0, qA1], dwords 1..7 = qA2..29,
// dword 8 = [qA30, qA31, dB lo, dB hi], dwords 9..16 = qB0..31.  The scale
// bytes are masked out of x so they contribute nothing.
__device__ __forceinline__ void pair_dots(const uint32_t (&w)[kPairDwords],
                                          const uint32_t (&x)[kPairDwords],
                                          int &sA, int &sB) {
  int a = __builtin_amdgcn_sdot4(w[0], x[0] & 0xFFFF0000u, 0, false);
#pragma unroll
  for (int i = 1; i < 8; ++i) a = __builtin_amdgcn_sdot4(w[i], x[i], a, false);
  a = __builtin_amdgcn_sdot4(w[8], x[8] & 0x0000FFFFu, a, false);
  int b = __builtin_amdgcn_sdot4(w[9], x[9], 0, false);
#pragma unroll
  for (int i = 10; i < 17; ++i) b = __builtin_amdgcn_sdot4(w[i], x[i], b, false);
  sA = a;
  sB = b;
}

}  // namespace q8
