// quantize.hip -- activation quantizer: fp32 rows -> Q8_0 blocks.
//
// Block rule (ds4-learning "Part 3: 模型架构", section 2, the row quantizer
// listing, applied per 32 values with a binary16 scale):
//   amax = max|x_i|, d32 = amax / 127, q_i = roundf(x_i / d32), d = fp16(d32).
// Both divisions are IEEE fp32 (hipcc's default correctly rounded divide),
// roundf rounds halves away from zero, the fp16 conversion rounds to nearest
// even and keeps subnormals (gfx950 denormal mode is left at "preserve").
// Zero blocks, non-finite blocks and scales that overflow binary16 follow the
// conventions stated in q8_0.h.
//
// The kernel is bound by HBM traffic (4 bytes read and 1.0625 bytes written
// per value).
#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

// Quantizes 32 values; returns the binary16 scale bits and the quants packed
// little-endian into 8 dwords.
__device__ __forceinline__ uint32_t quantize_block32(const float (&v)[32], uint32_t (&qd)[8]) {
  bool finite = true;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    finite = finite && __builtin_isfinite(v[i]);
    float a = fabsf(v[i]);
    amax = a > amax ? a : amax;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) qd[j] = 0;
  if (!finite) return 0x7E00u;
  if (!(amax > 0.0f)) return 0u;
  const float d = amax / 127.0f;
  if (!(d > 0.0f)) return 0u;  // d32 underflowed: zero block
  const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)d);
  if ((h & 0x7FFFu) == 0x7C00u) return 0x7E00u;  // scale does not fit binary16
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float r = v[i] / d;
    float qr = roundf(r);
    qr = fminf(fmaxf(qr, -127.0f), 127.0f);
    qd[i / 4] |= ((uint32_t)(int)qr & 0xFFu) << (8 * (i % 4));
  }
  return h;
}

// Needs x 16-byte aligned, x_q 4-byte aligned and an even block count.  16
// lanes per block pair, one float4 each (a wave reads 1 KB of contiguous x per
// load).
// A workgroup quantizes U * 16 consecutive pairs: 16 lanes per pair, U pairs
// per lane group, all U float4 loads issued before any math so every lane
// keeps U * 16 bytes in flight.  Both streams are touched once, so the loads
// and stores are non-temporal: on the 2048 x 32768 input (340 MB moved) that
// took 68-71 us to 60-63 us on one box, where a plain device copy of as many
// bytes runs at about 5.3 TB/s.
template <int U>
__global__ __launch_bounds__(256) void quantize_pair_kernel(const float *__restrict__ x,
                                                            uint8_t *__restrict__ xq,
                                                            int64_t total_pairs,
                                                            int64_t pairs_per_row,
                                                            int64_t in_dim) {
  const int sub = (int)(threadIdx.x & 15);     // 0..7 block A, 8..15 block B
  const int64_t first = (int64_t)blockIdx.x * (16 * U) + (threadIdx.x >> 4);
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t pair_raw = first + 16 * u;
    const int64_t pair = pair_raw < total_pairs ? pair_raw : total_pairs - 1;
    const int64_t row = pair / pairs_per_row;
    const int64_t p = pair - row * pairs_per_row;
    const f32x4 t =
        __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + row * in_dim + p * 64 + sub * 4));
    v[u] = make_float4(t.x, t.y, t.z, t.w);
  }
  // The workgroup's 16 U pairs are consecutive bytes of x_q: they are
  // gathered in LDS and written with one coalesced dword per lane and store
  // (256 contiguous bytes per wave instruction) instead of one 64-byte run
  // per pair and store.  On the prefill_b input the fastest launch went from
  // 55.2 to 52.9 us (rocprofv3, one box).  Pairs past the end are quantized
  // (their loads re-read the last pair) but not stored.
  constexpr int NP = 16 * U;
  __shared__ uint32_t stage[NP * kPairDwords];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int lp = (int)(threadIdx.x >> 4) + 16 * u;  // pair within the workgroup
    const PairWords pw = quantize_pair16(v[u], sub);  // every lane takes part (DPP)
    stage[lp * kPairDwords + sub + 1] = pw.hi;
    if (sub == 0) stage[lp * kPairDwords] = pw.lo;
  }
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * NP;
  const int64_t valid = min((int64_t)NP, total_pairs - p0) * kPairDwords;  // dwords to store
  uint32_t *dst = reinterpret_cast<uint32_t *>(xq + p0 * kPairBytes);
#pragma unroll
  for (int k = 0; k < (NP * kPairDwords + 255) / 256; ++k) {
    const int d = 256 * k + (int)threadIdx.x;
    if (d < valid) __builtin_nontemporal_store(stage[d], dst + d);
  }
}

__global__ __launch_bounds__(256) void quantize_block_kernel(const float *__restrict__ x,
                                                             uint8_t *__restrict__ xq,
                                                             int64_t total_blocks,
                                                             int64_t blocks_per_row,
                                                             int64_t in_dim) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total_blocks) return;
  const int64_t row = g / blocks_per_row;
  const int64_t b = g - row * blocks_per_row;
  const float *src = x + row * in_dim + b * kBlockElems;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = src[i];
  uint32_t qd[8];
  const uint32_t h = quantize_block32(v, qd);
  uint16_t *dst = reinterpret_cast<uint16_t *>(xq + g * kBlockBytes);
  dst[0] = (uint16_t)h;
#pragma unroll
  for (int j = 0; j < 16; ++j) dst[1 + j] = (uint16_t)(qd[j / 2] >> (16 * (j % 2)));
}

}  // namespace

hipError_t launch_quantize(void *x_q, const float *x, int64_t n_tok, int64_t in_dim, bool fast,
                           hipStream_t s) {
  const int64_t nb = in_dim / kBlockElems;
  if (fast) {
    const int64_t ppr = nb / 2;
    const int64_t total = n_tok * ppr;
    // Four pairs per lane group once there are enough pairs for the chip.
    if (total >= (int64_t)4 * 16 * 1024) {
      const int64_t grid = (total + 63) / 64;
      hipLaunchKernelGGL(quantize_pair_kernel<4>, dim3((uint32_t)grid), dim3(256), 0, s, x,
                         static_cast<uint8_t *>(x_q), total, ppr, in_dim);
    } else {
      const int64_t grid = (total + 15) / 16;
      hipLaunchKernelGGL(quantize_pair_kernel<1>, dim3((uint32_t)grid), dim3(256), 0, s, x,
                         static_cast<uint8_t *>(x_q), total, ppr, in_dim);
    }
  } else {
    const int64_t total = n_tok * nb;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(quantize_block_kernel, dim3((uint32_t)grid), dim3(256), 0, s, x,
                       static_cast<uint8_t *>(x_q), total, nb, in_dim);
  }
  return hipGetLastError();
}

}  // namespace q8
