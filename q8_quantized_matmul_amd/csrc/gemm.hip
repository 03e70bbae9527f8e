// gemm.hip -- Q8_0 x Q8_0 GEMM on gfx950 matrix cores for many tokens
// (prefill, and any call with n_tok >= 16).
//
// Same arithmetic as the matvec ("Part 6: 代码走读", trace 3): per output
// (t, o) and 32-value block b, an exact int32 block dot S_b times the exact
// fp32 scale product d_w * d_x, summed in fp32.  The pages run this on
// matrix units only from 16 tokens up ("Part 6: GPU 加速", C3 NAX paragraph)
// and accept a different fp32 reduction order for batched GEMMs than for
// decode ("Part 6: GPU 加速", section 4m); this kernel is deterministic but not
// bitwise equal to the matvec.
//
// gfx950 mapping:
//   * One K-step of v_mfma_i32_32x32x32_i8 is exactly one Q8_0 block, so every
//     MFMA result is a 32x32 tile of exact S_b (rows = output features o,
//     columns = tokens t).
//   * The per-element scale d_w[o] * d_x[t] of that block is the outer product
//     of two binary16 vectors: one v_mfma_f32_32x32x8_f16 with only K-slot 0
//     populated yields it exactly in fp32, in the same accumulator layout.
//     The VALU then does 2 ops per element and block (int->float, fma).
//   * Workgroup = 4 waves in a 2x2 grid, each wave TI x TJ tiles of 32x32.
//     A K-stage of KB blocks stages qs of 64*TI weight rows and 64*TJ token
//     rows into LDS as aligned 16-byte chunks (row stride KB*32+16 bytes, so
//     ds_read_b128 rows fall on distinct banks) and the binary16 scales in
//     separate arrays.  Global loads fetch whole block pairs (68 bytes) per
//     lane; the misaligned first block of a pair is realigned in registers.
//     The next stage's global loads are issued before the current stage's
//     MFMAs (register prefetch).
//   * Split-K over grid.z writes fp32 partials to caller workspace; a second
//     kernel sums them in split order (deterministic, no atomics).
#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

struct GemmArgs {
  float *out;        // final output, or the split partials
  int32_t *blocksums;
  const uint8_t *w;
  const uint8_t *x_q;
  int64_t out_dim;
  int64_t n_tok;
  int64_t nb;
  int64_t row_bytes;
  int64_t blocks_per_split;
};

template <int TI, int TJ, int KB, bool STORE_S>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs a) {
  constexpr int BO = 64 * TI;         // output rows per workgroup
  constexpr int BT = 64 * TJ;         // tokens per workgroup
  constexpr int ROWB = KB * 32 + 16;  // LDS bytes per row (padded)
  constexpr int PPR = KB / 2;         // block pairs per row per stage
  constexpr int NPAIR_W = BO * PPR;
  constexpr int NPAIR = NPAIR_W + BT * PPR;
  constexpr int PPT = (NPAIR + 255) / 256;
  static_assert(KB % 2 == 0, "stage must hold whole block pairs");

  __shared__ __attribute__((aligned(16))) uint8_t qsW[BO * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t qsX[BT * ROWB];
  __shared__ uint16_t scW[KB][BO];
  __shared__ uint16_t scX[KB][BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t o_tile = (int64_t)blockIdx.x * BO;
  const int64_t t_tile = (int64_t)blockIdx.y * BT;
  const int64_t b_begin = (int64_t)blockIdx.z * a.blocks_per_split;
  const int64_t b_end = min(b_begin + a.blocks_per_split, a.nb);
  const int o_w = (wave & 1) * 32 * TI;   // wave's first row inside the tile
  const int t_w = (wave >> 1) * 32 * TJ;  // wave's first token inside the tile

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint32_t pre[PPT][kPairDwords];

  auto gload = [&](int64_t b0) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int j = tid + 256 * p;
      if (j < NPAIR) {
        const bool isw = j < NPAIR_W;
        const int jj = isw ? j : j - NPAIR_W;
        const int row = jj / PPR;
        const int pr = jj % PPR;
        const int64_t grow = (isw ? o_tile : t_tile) + row;
        const int64_t lim = isw ? a.out_dim : a.n_tok;
        const int64_t blk = b0 + 2 * pr;
        if (grow < lim && blk < b_end) {
          load_pair((isw ? a.w : a.x_q) + grow * a.row_bytes + blk * kBlockBytes, pre[p]);
        } else {
#pragma unroll
          for (int i = 0; i < kPairDwords; ++i) pre[p][i] = 0;
        }
      }
    }
  };

  auto lstore = [&]() {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int j = tid + 256 * p;
      if (j < NPAIR) {
        const bool isw = j < NPAIR_W;
        const int jj = isw ? j : j - NPAIR_W;
        const int row = jj / PPR;
        const int pr = jj % PPR;
        uint8_t *qs = (isw ? qsW : qsX) + row * ROWB + pr * 64;
        const uint32_t *d = pre[p];
        i32x4 a0 = {(int)__builtin_amdgcn_alignbyte(d[1], d[0], 2),
                    (int)__builtin_amdgcn_alignbyte(d[2], d[1], 2),
                    (int)__builtin_amdgcn_alignbyte(d[3], d[2], 2),
                    (int)__builtin_amdgcn_alignbyte(d[4], d[3], 2)};
        i32x4 a1 = {(int)__builtin_amdgcn_alignbyte(d[5], d[4], 2),
                    (int)__builtin_amdgcn_alignbyte(d[6], d[5], 2),
                    (int)__builtin_amdgcn_alignbyte(d[7], d[6], 2),
                    (int)__builtin_amdgcn_alignbyte(d[8], d[7], 2)};
        i32x4 b0 = {(int)d[9], (int)d[10], (int)d[11], (int)d[12]};
        i32x4 b1 = {(int)d[13], (int)d[14], (int)d[15], (int)d[16]};
        reinterpret_cast<i32x4 *>(qs)[0] = a0;
        reinterpret_cast<i32x4 *>(qs)[1] = a1;
        reinterpret_cast<i32x4 *>(qs)[2] = b0;
        reinterpret_cast<i32x4 *>(qs)[3] = b1;
        if (isw) {
          scW[2 * pr][row] = (uint16_t)(d[0] & 0xFFFFu);
          scW[2 * pr + 1][row] = (uint16_t)(d[8] >> 16);
        } else {
          scX[2 * pr][row] = (uint16_t)(d[0] & 0xFFFFu);
          scX[2 * pr + 1][row] = (uint16_t)(d[8] >> 16);
        }
      }
    }
  };

  const int lrow = lane & 31;          // row/column of the 32x32 operand this lane feeds
  const int khalf = (lane >> 5) * 16;  // which 16 bytes of the block's 32 quants
  const i32x16 izero = {};
  const f32x16 fzero = {};

  gload(b_begin);
  for (int64_t b0 = b_begin; b0 < b_end; b0 += KB) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (b0 + KB < b_end) gload(b0 + KB);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (b0 + kb < b_end) {
        i32x4 A[TI], B[TJ];
        f16x4 SA[TI], SB[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int r = o_w + 32 * i + lrow;
          A[i] = *reinterpret_cast<const i32x4 *>(qsW + r * ROWB + kb * 32 + khalf);
          const uint16_t s = lane < 32 ? scW[kb][r] : (uint16_t)0;
          SA[i] = f16x4{__builtin_bit_cast(_Float16, s), (_Float16)0, (_Float16)0, (_Float16)0};
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int r = t_w + 32 * j + lrow;
          B[j] = *reinterpret_cast<const i32x4 *>(qsX + r * ROWB + kb * 32 + khalf);
          const uint16_t s = lane < 32 ? scX[kb][r] : (uint16_t)0;
          SB[j] = f16x4{__builtin_bit_cast(_Float16, s), (_Float16)0, (_Float16)0, (_Float16)0};
        }
#pragma unroll
        for (int i = 0; i < TI; ++i) {
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const i32x16 S = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], izero, 0, 0, 0);
            const f32x16 C = __builtin_amdgcn_mfma_f32_32x32x8f16(SA[i], SB[j], fzero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf((float)S[r], C[r], acc[i][j][r]);
            if constexpr (STORE_S) {
              const int64_t t = t_tile + t_w + 32 * j + lrow;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int64_t o = o_tile + o_w + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (t < a.n_tok && o < a.out_dim)
                  a.blocksums[(t * a.out_dim + o) * a.nb + b0 + kb] = S[r];
              }
            }
          }
        }
      }
    }
  }

  // Accumulator layout of a 32x32 MFMA tile: lane l holds column l%32 and
  // rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
  float *dst = a.out + (int64_t)blockIdx.z * a.n_tok * a.out_dim;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t t = t_tile + t_w + 32 * j + lrow;
      if (t < a.n_tok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t o = o_tile + o_w + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (o < a.out_dim) dst[t * a.out_dim + o] = acc[i][j][r];
        }
      }
    }
  }
}

// out[i] = sum over splits s = 0..n_split-1 (in order) of partials[s][i].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(float *__restrict__ out,
                                                            const float *__restrict__ part,
                                                            int64_t n, int n_split) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = part[i];
  for (int s = 1; s < n_split; ++s) v += part[(int64_t)s * n + i];
  out[i] = v;
}

constexpr int kStageBlocks = 4;

}  // namespace

bool gemm_supported(int64_t in_dim) { return in_dim > 0 && in_dim % 64 == 0; }

static int gemm_tj(int64_t n_tok) { return n_tok <= 64 ? 1 : 2; }

int gemm_auto_split(int64_t in_dim, int64_t out_dim, int64_t n_tok) {
  const int64_t nb = in_dim / kBlockElems;
  const int tj = gemm_tj(n_tok);
  const int64_t tiles = ((out_dim + 127) / 128) * ((n_tok + 64 * tj - 1) / (64 * tj));
  int64_t split = (512 + tiles - 1) / tiles;           // aim for >= 512 workgroups
  split = std::max<int64_t>(split, (nb + 127) / 128);  // fp32 chains of <= 128 blocks
  split = std::min<int64_t>(split, nb / (2 * kStageBlocks));
  split = std::min<int64_t>(split, 16);
  return (int)std::max<int64_t>(split, 1);
}

size_t gemm_workspace_bytes(int64_t out_dim, int64_t n_tok, int split) {
  return split > 1 ? (size_t)split * (size_t)out_dim * (size_t)n_tok * sizeof(float) : 0;
}

hipError_t launch_gemm(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                       int64_t out_dim, const void *x_q, int64_t n_tok, int split,
                       float *partials, hipStream_t s) {
  const int64_t nb = in_dim / kBlockElems;
  int64_t bps = (nb + split - 1) / split;
  bps = (bps + kStageBlocks - 1) / kStageBlocks * kStageBlocks;
  const int64_t n_split = (nb + bps - 1) / bps;
  GemmArgs a{};
  a.out = n_split > 1 ? partials : out;
  a.blocksums = blocksums;
  a.w = static_cast<const uint8_t *>(w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.out_dim = out_dim;
  a.n_tok = n_tok;
  a.nb = nb;
  a.row_bytes = nb * kBlockBytes;
  a.blocks_per_split = bps;
  const int tj = gemm_tj(n_tok);
  const dim3 grid((uint32_t)((out_dim + 127) / 128), (uint32_t)((n_tok + 64 * tj - 1) / (64 * tj)),
                  (uint32_t)n_split);
  if (tj == 1) {
    if (blocksums) hipLaunchKernelGGL((gemm_kernel<2, 1, kStageBlocks, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<2, 1, kStageBlocks, false>), grid, dim3(256), 0, s, a);
  } else {
    if (blocksums) hipLaunchKernelGGL((gemm_kernel<2, 2, kStageBlocks, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<2, 2, kStageBlocks, false>), grid, dim3(256), 0, s, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_split == 1) return err;
  const int64_t n = n_tok * out_dim;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, out,
                     partials, n, (int)n_split);
  return hipGetLastError();
}

}  // namespace q8
