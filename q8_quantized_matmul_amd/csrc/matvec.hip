// matvec.hip -- weight-streaming Q8_0 kernels for few tokens per weight row:
// decode (n_tok = 1), small batches, and the grouped expert matmul whose
// experts each see a handful of tokens.
//
// The operation is the pages' Q8_0 matvec y = x @ W with both operands in
// Q8_0 ("Part 6: 代码走读", trace 3; "Part 3: 模型架构", section 2, item 4).
// Each output needs in_dim/32 block dots S_b (exact int32 from packed int8
// dot4 instructions), each scaled by the exact fp32 product d_w * d_x and
// summed in fp32.
//
// Design for gfx950 (HBM-bound: ~2 int ops per weight byte):
//   * A lane owns one block PAIR (68 bytes = 17 dwords, dword aligned when the
//     row has an even block count), so a wave streams 64 consecutive pairs =
//     4352 contiguous bytes per load round with dwordx4 loads; weights are
//     read exactly once.
//   * The x_q row is in the same pair layout, so the lane dots its weight
//     dwords against the x dwords at the same offsets, with the x scale bytes
//     masked to zero; no repacking of the 2-byte-misaligned first block.
//   * Rows shorter than 64 pairs share a wave (64/P rows per wave); longer
//     rows are split into 64-pair chunks over up to 4 waves of the workgroup
//     and reduced through LDS.  Lane partial sums are reduced with xor
//     shuffles in a fixed order, so results are deterministic.
//   * Each workgroup loads all of its weight rows before touching x, so every
//     wave has RG * CPW * 272 bytes in flight per lane group.
#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

struct MatvecArgs {
  float *out;
  int32_t *blocksums;
  const uint8_t *w;                 // dense weights
  const uint8_t *const *expert_w;   // grouped: device table of expert bases
  const uint8_t *x_q;
  const int32_t *counts;            // grouped: pairs per expert
  const int32_t *offsets;           // grouped: first list slot per expert
  const int32_t *pairs;             // grouped: expert-major pair list
  int64_t out_dim;
  int64_t n_items;                  // dense: n_tok
  int64_t row_bytes;                // (in_dim / 32) * 34
  int64_t nb;                       // in_dim / 32
  int32_t n_used;                   // grouped
  int32_t x_rows;                   // grouped: 0 = row per token, 1 = row per pair
};

template <int LPR, int WPR, int CPW, int RG, bool GROUPED, bool STORE_S>
__global__ __launch_bounds__(256) void matvec_kernel(const MatvecArgs a) {
  constexpr int RPW = 64 / LPR;                   // rows per wave row-group
  constexpr int ROWS_PER_SLOT = RG * RPW;
  constexpr int TILE_ROWS = (4 / WPR) * ROWS_PER_SLOT;
  __shared__ float red[4][RG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = wave / WPR;
  const int part = wave % WPR;

  const uint8_t *w = a.w;
  const int32_t *items = nullptr;
  int64_t n_items = a.n_items;
  if constexpr (GROUPED) {
    const int e = blockIdx.y;
    n_items = a.counts[e];
    if (n_items == 0) return;  // uniform across the workgroup
    w = a.expert_w[e];
    items = a.pairs + a.offsets[e];
  }

  const int64_t row0 = (int64_t)blockIdx.x * TILE_ROWS + slot * ROWS_PER_SLOT + lane / LPR;
  int64_t pair_of[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
    pair_of[c] = (LPR < 64) ? (int64_t)(lane % LPR) : (int64_t)(c * WPR + part) * 64 + lane;

  uint32_t wr[RG][CPW][kPairDwords];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int64_t row = row0 + g * RPW;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (row < a.out_dim) {
        load_pair(w + row * a.row_bytes + pair_of[c] * kPairBytes, wr[g][c]);
      } else {
#pragma unroll
        for (int i = 0; i < kPairDwords; ++i) wr[g][c][i] = 0;
      }
    }
  }

  for (int64_t it = 0; it < n_items; ++it) {
    int64_t xrow = it, orow = it;
    if constexpr (GROUPED) {
      const int64_t pr = items[it];
      orow = pr;
      xrow = a.x_rows ? pr : pr / a.n_used;
    }
    float acc[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      uint32_t xr[kPairDwords];
      load_pair(a.x_q + xrow * a.row_bytes + pair_of[c] * kPairBytes, xr);
      const float dxA = f16_bits_to_f32(xr[0]);
      const float dxB = f16_bits_to_f32(xr[8] >> 16);
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        int sA, sB;
        pair_dots(wr[g][c], xr, sA, sB);
        const float scA = f16_bits_to_f32(wr[g][c][0]) * dxA;
        const float scB = f16_bits_to_f32(wr[g][c][8] >> 16) * dxB;
        acc[g] += scA * (float)sA;
        acc[g] += scB * (float)sB;
        if constexpr (STORE_S) {
          const int64_t row = row0 + g * RPW;
          if (row < a.out_dim) {
            int32_t *bs = a.blocksums + (orow * a.out_dim + row) * a.nb + 2 * pair_of[c];
            bs[0] = sA;
            bs[1] = sB;
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) acc[g] += __shfl_xor(acc[g], m, 64);
    }
    if constexpr (WPR > 1) {
      if (lane == 0) {
#pragma unroll
        for (int g = 0; g < RG; ++g) red[wave][g] = acc[g];
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          float v = red[wave][g];
#pragma unroll
          for (int p = 1; p < WPR; ++p) v += red[wave + p][g];
          acc[g] = v;
        }
      }
      __syncthreads();
    }
    if (part == 0 && (lane % LPR) == 0) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int64_t row = row0 + g * RPW;
        if (row < a.out_dim) a.out[orow * a.out_dim + row] = acc[g];
      }
    }
  }
}

// ---- generic fallback: one wave per (token, row), lanes stride over blocks.
// Works for any block count and 2-byte aligned operands.
template <bool STORE_S>
__device__ __forceinline__ void generic_row_dot(float *out, int32_t *bs, const uint8_t *wrow,
                                                const uint8_t *xrow, int64_t nb) {
  const int lane = threadIdx.x & 63;
  float acc = 0.0f;
  for (int64_t b = lane; b < nb; b += 64) {
    const uint16_t *wb = reinterpret_cast<const uint16_t *>(wrow + b * kBlockBytes);
    const uint16_t *xb = reinterpret_cast<const uint16_t *>(xrow + b * kBlockBytes);
    int s = 0;
#pragma unroll
    for (int j = 1; j < 17; ++j) {
      const uint32_t wu = wb[j], xu = xb[j];
      s += (int)(int8_t)(wu & 0xFF) * (int)(int8_t)(xu & 0xFF);
      s += (int)(int8_t)(wu >> 8) * (int)(int8_t)(xu >> 8);
    }
    acc += (f16_bits_to_f32(wb[0]) * f16_bits_to_f32(xb[0])) * (float)s;
    if constexpr (STORE_S) bs[b] = s;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (lane == 0) *out = acc;
}

template <bool STORE_S>
__global__ __launch_bounds__(256) void generic_kernel(float *__restrict__ out,
                                                      int32_t *__restrict__ blocksums,
                                                      const uint8_t *__restrict__ w,
                                                      const uint8_t *__restrict__ xq,
                                                      int64_t out_dim, int64_t n_tok,
                                                      int64_t nb) {
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= out_dim * n_tok) return;  // uniform per wave
  const int64_t t = job / out_dim;
  const int64_t o = job - t * out_dim;
  generic_row_dot<STORE_S>(out + job, STORE_S ? blocksums + job * nb : nullptr,
                           w + o * nb * kBlockBytes, xq + t * nb * kBlockBytes, nb);
}

// Grouped fallback: one wave per (pair, row); pairs with an invalid expert id
// are skipped (their rows are filled with NaN by the routing kernel).
template <bool STORE_S>
__global__ __launch_bounds__(256) void generic_grouped_kernel(
    float *__restrict__ out, int32_t *__restrict__ blocksums,
    const uint8_t *const *__restrict__ expert_w, int32_t n_expert,
    const int32_t *__restrict__ selected, int32_t n_used, const uint8_t *__restrict__ xq,
    int32_t x_rows, int64_t out_dim, int64_t n_pairs, int64_t nb) {
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= out_dim * n_pairs) return;
  const int64_t pr = job / out_dim;
  const int64_t o = job - pr * out_dim;
  const int32_t e = selected[pr];
  if (e < 0 || e >= n_expert) return;
  const int64_t xrow = x_rows ? pr : pr / n_used;
  generic_row_dot<STORE_S>(out + job, STORE_S ? blocksums + job * nb : nullptr,
                           expert_w[e] + o * nb * kBlockBytes, xq + xrow * nb * kBlockBytes, nb);
}

typedef void (*MatvecFn)(const MatvecArgs);

template <int LPR, int WPR, int CPW, bool GROUPED, bool STORE_S>
MatvecFn pick_rg(int rg) {
  if constexpr (CPW == 1) {
    if (rg >= 4) return matvec_kernel<LPR, WPR, CPW, 4, GROUPED, STORE_S>;
  }
  if constexpr (CPW <= 2) {
    if (rg >= 2) return matvec_kernel<LPR, WPR, CPW, 2, GROUPED, STORE_S>;
  }
  return matvec_kernel<LPR, WPR, CPW, 1, GROUPED, STORE_S>;
}

template <bool GROUPED, bool STORE_S>
MatvecFn pick_kernel(const MatvecShape &sh, int rg) {
  switch (sh.lanes_per_row) {
    case 1: return pick_rg<1, 1, 1, GROUPED, STORE_S>(rg);
    case 2: return pick_rg<2, 1, 1, GROUPED, STORE_S>(rg);
    case 4: return pick_rg<4, 1, 1, GROUPED, STORE_S>(rg);
    case 8: return pick_rg<8, 1, 1, GROUPED, STORE_S>(rg);
    case 16: return pick_rg<16, 1, 1, GROUPED, STORE_S>(rg);
    case 32: return pick_rg<32, 1, 1, GROUPED, STORE_S>(rg);
    default: break;
  }
  const int key = sh.waves_per_row * 10 + sh.chunks_per_wave;
  switch (key) {
    case 11: return pick_rg<64, 1, 1, GROUPED, STORE_S>(rg);
    case 13: return pick_rg<64, 1, 3, GROUPED, STORE_S>(rg);
    case 21: return pick_rg<64, 2, 1, GROUPED, STORE_S>(rg);
    case 22: return pick_rg<64, 2, 2, GROUPED, STORE_S>(rg);
    case 41: return pick_rg<64, 4, 1, GROUPED, STORE_S>(rg);
    case 42: return pick_rg<64, 4, 2, GROUPED, STORE_S>(rg);
    case 43: return pick_rg<64, 4, 3, GROUPED, STORE_S>(rg);
    case 44: return pick_rg<64, 4, 4, GROUPED, STORE_S>(rg);
    default: return nullptr;
  }
}

int max_rg(const MatvecShape &sh) { return sh.chunks_per_wave == 1 ? 4 : (sh.chunks_per_wave == 2 ? 2 : 1); }

int64_t tile_rows(const MatvecShape &sh, int rg) {
  return (int64_t)(4 / sh.waves_per_row) * rg * (64 / sh.lanes_per_row);
}

// Fewest rows per workgroup that still leaves >= 1024 workgroups (4 per CU);
// small matrices get single-row-group tiles so all 256 CUs take part.
int choose_rg(const MatvecShape &sh, int64_t rows, int64_t experts) {
  int rg = max_rg(sh);
  while (rg > 1) {
    const int64_t tiles = (rows + tile_rows(sh, rg) - 1) / tile_rows(sh, rg);
    if (tiles * experts >= 1024) break;
    rg /= 2;
  }
  return rg;
}

}  // namespace

bool matvec_shape(int64_t in_dim, MatvecShape *shape) {
  if (in_dim <= 0 || in_dim % 64 != 0) return false;  // need whole block pairs
  const int64_t P = in_dim / 64;
  MatvecShape sh{};
  if (P < 64) {
    if ((P & (P - 1)) != 0) return false;  // lanes of a row must tile a wave
    sh = {(int)P, 1, 1};
  } else {
    if (P % 64 != 0) return false;
    const int64_t C = P / 64;
    int wpr = (C % 4 == 0) ? 4 : (C % 2 == 0 ? 2 : 1);
    const int64_t cpw = C / wpr;
    if (cpw > 4 || (wpr < 4 && cpw > 3) || (wpr == 2 && cpw > 2)) return false;
    sh = {64, wpr, (int)cpw};
  }
  if (shape) *shape = sh;
  return true;
}

hipError_t launch_matvec(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                         int64_t out_dim, const void *x_q, int64_t n_tok, hipStream_t s) {
  MatvecShape sh;
  if (!matvec_shape(in_dim, &sh)) return hipErrorInvalidValue;
  const int rg = choose_rg(sh, out_dim, 1);
  MatvecFn fn = blocksums ? pick_kernel<false, true>(sh, rg) : pick_kernel<false, false>(sh, rg);
  if (!fn) return hipErrorInvalidValue;
  MatvecArgs a{};
  a.out = out;
  a.blocksums = blocksums;
  a.w = static_cast<const uint8_t *>(w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.out_dim = out_dim;
  a.n_items = n_tok;
  a.nb = in_dim / kBlockElems;
  a.row_bytes = a.nb * kBlockBytes;
  const int64_t tiles = (out_dim + tile_rows(sh, rg) - 1) / tile_rows(sh, rg);
  hipLaunchKernelGGL(fn, dim3((uint32_t)tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_matvec_grouped(float *out, int32_t *blocksums, const void *const *expert_w,
                                 int32_t n_expert, int64_t in_dim, int64_t out_dim,
                                 const void *x_q, int32_t x_rows, int32_t n_used,
                                 const int32_t *counts, const int32_t *offsets,
                                 const int32_t *pairs, hipStream_t s) {
  MatvecShape sh;
  if (!matvec_shape(in_dim, &sh)) return hipErrorInvalidValue;
  const int rg = choose_rg(sh, out_dim, n_expert);
  MatvecFn fn = blocksums ? pick_kernel<true, true>(sh, rg) : pick_kernel<true, false>(sh, rg);
  if (!fn) return hipErrorInvalidValue;
  MatvecArgs a{};
  a.out = out;
  a.blocksums = blocksums;
  a.expert_w = reinterpret_cast<const uint8_t *const *>(expert_w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.counts = counts;
  a.offsets = offsets;
  a.pairs = pairs;
  a.out_dim = out_dim;
  a.nb = in_dim / kBlockElems;
  a.row_bytes = a.nb * kBlockBytes;
  a.n_used = n_used;
  a.x_rows = x_rows;
  const int64_t tiles = (out_dim + tile_rows(sh, rg) - 1) / tile_rows(sh, rg);
  hipLaunchKernelGGL(fn, dim3((uint32_t)tiles, (uint32_t)n_expert), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_generic_grouped(float *out, int32_t *blocksums, const void *const *expert_w,
                                  int32_t n_expert, int64_t in_dim, int64_t out_dim,
                                  const int32_t *selected, int32_t n_used, const void *x_q,
                                  int32_t x_rows, int64_t n_tok, hipStream_t s) {
  const int64_t n_pairs = n_tok * n_used;
  const int64_t grid = (out_dim * n_pairs + 3) / 4;
  const int64_t nb = in_dim / kBlockElems;
  const uint8_t *const *ew = reinterpret_cast<const uint8_t *const *>(expert_w);
  const uint8_t *xq = static_cast<const uint8_t *>(x_q);
  if (blocksums) {
    hipLaunchKernelGGL(generic_grouped_kernel<true>, dim3((uint32_t)grid), dim3(256), 0, s, out,
                       blocksums, ew, n_expert, selected, n_used, xq, x_rows, out_dim, n_pairs, nb);
  } else {
    hipLaunchKernelGGL(generic_grouped_kernel<false>, dim3((uint32_t)grid), dim3(256), 0, s, out,
                       blocksums, ew, n_expert, selected, n_used, xq, x_rows, out_dim, n_pairs, nb);
  }
  return hipGetLastError();
}

hipError_t launch_generic(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                          int64_t out_dim, const void *x_q, int64_t n_tok, hipStream_t s) {
  const int64_t jobs = out_dim * n_tok;
  const int64_t grid = (jobs + 3) / 4;
  const int64_t nb = in_dim / kBlockElems;
  if (blocksums) {
    hipLaunchKernelGGL(generic_kernel<true>, dim3((uint32_t)grid), dim3(256), 0, s, out,
                       blocksums, static_cast<const uint8_t *>(w),
                       static_cast<const uint8_t *>(x_q), out_dim, n_tok, nb);
  } else {
    hipLaunchKernelGGL(generic_kernel<false>, dim3((uint32_t)grid), dim3(256), 0, s, out,
                       blocksums, static_cast<const uint8_t *>(w),
                       static_cast<const uint8_t *>(x_q), out_dim, n_tok, nb);
  }
  return hipGetLastError();
}

}  // namespace q8
