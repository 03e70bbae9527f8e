// skinny.hip -- Q8_0 matmul for up to 64 tokens on the matrix cores, with
// the weights streamed once from HBM straight into MFMA registers (the plan
// uses it from 20 tokens).
//
// The method is the same as everywhere (ds4-learning "Part 6: 代码走读",
// trace 3: out[t][o] = sum over blocks of d_w * d_x * S_b); this kernel
// covers the regime between the weight-streaming matvec and the LDS-tiled
// GEMM, as the pages' backends keep dedicated kernels and a split-K path for
// narrow batches ("Part 6: GPU 加速", sections 4c and 4s).  Tokens are the
// MFMA's M dimension (one or two 32-token tiles), output rows its N dimension
// (32 per wave).
//
//   * One v_mfma_i32_32x32x32_i8 per (token tile, block) gives the exact
//     S_b of the 32x32 tile; one v_mfma_f32_32x32x8_f16 with only K slot 0
//     populated gives the matching d_w * d_x outer product, exactly; the
//     epilogue is acc += float(S_b) * scale.
//   * A lane reads the block pair (68 bytes) of its row: the 20 bytes around
//     its half of block 2p (re-aligned by 2 bytes), its half of block 2p + 1,
//     and the dword holding block 2p + 1's scale.  Token rows are read the
//     same way from x_q (L2-resident).  Everything is dword aligned.
//   * The 4 waves of a workgroup take interleaved block pairs of the
//     workgroup's K range and are summed through LDS in wave order; K ranges
//     of different workgroups (split-K) go to partials that the ordered
//     reduce kernel sums.  Every sum has a fixed order: results are
//     deterministic.
#include <algorithm>

#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

typedef uint32_t u32x4_a4s __attribute__((ext_vector_type(4), aligned(4)));

struct SkinnyArgs {
  float *out;            // [n_tok][out_dim], or partials [n_split][n_tok][out_dim]
  const uint8_t *w;      // [out_dim][row_bytes]
  const uint8_t *x_q;    // [n_tok][row_bytes]
  int64_t out_dim;
  int64_t n_tok;
  int64_t row_bytes;
  int32_t n_pairs;       // block pairs per row
  int32_t pairs_per_split;
};

// The 10 dwords one lane needs of a block pair at p (dword aligned): F = the
// 5 dwords holding its half of block 2p (2-byte offset), G = its half of
// block 2p + 1, d8 = the dword holding block 2p + 1's scale.
struct PairPart {
  uint32_t F[5];
  uint32_t G[4];
  uint32_t d8;
};

__device__ __forceinline__ void load_part(const uint8_t *pair, int h, PairPart &r) {
  const u32x4_a4s f = *reinterpret_cast<const u32x4_a4s *>(pair + 16 * h);
  const u32x4_a4s g = *reinterpret_cast<const u32x4_a4s *>(pair + 36 + 16 * h);
  r.F[0] = f.x;
  r.F[1] = f.y;
  r.F[2] = f.z;
  r.F[3] = f.w;
  r.F[4] = *reinterpret_cast<const uint32_t *>(pair + 16 * h + 16);
  r.G[0] = g.x;
  r.G[1] = g.y;
  r.G[2] = g.z;
  r.G[3] = g.w;
  r.d8 = *reinterpret_cast<const uint32_t *>(pair + 32);
}

// MFMA operand (16 quant bytes) of block 2p + blk and its scale bits (only
// for half 0 of a live slot; half 1 feeds the zero K slots of the scale
// MFMA, and a zero scale on both sides makes a slot add exactly nothing).
__device__ __forceinline__ i32x4 part_operand(const PairPart &r, int blk, bool keep, uint32_t &sc) {
  if (blk == 0) {
    sc = keep ? (r.F[0] & 0xFFFFu) : 0u;
    return i32x4{(int)__builtin_amdgcn_alignbyte(r.F[1], r.F[0], 2),
                 (int)__builtin_amdgcn_alignbyte(r.F[2], r.F[1], 2),
                 (int)__builtin_amdgcn_alignbyte(r.F[3], r.F[2], 2),
                 (int)__builtin_amdgcn_alignbyte(r.F[4], r.F[3], 2)};
  }
  sc = keep ? (r.d8 >> 16) : 0u;
  return i32x4{(int)r.G[0], (int)r.G[1], (int)r.G[2], (int)r.G[3]};
}

// MT token tiles of 32.  Grid: x = 32-row output tiles, y = K splits.
template <int MT>
__global__ __launch_bounds__(256) void skinny_kernel(const SkinnyArgs a) {
  __shared__ float red[4][MT][16][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int64_t o = (int64_t)blockIdx.x * 32 + n;
  const int64_t lo = o < a.out_dim ? o : a.out_dim - 1;  // rows past the end re-read the last
  const uint8_t *wrow = a.w + lo * a.row_bytes;
  const uint8_t *xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = 32 * m + n;
    xrow[m] = a.x_q + (t < a.n_tok ? t : a.n_tok - 1) * a.row_bytes;
  }
  const int p_begin = blockIdx.y * a.pairs_per_split;
  const int p_end = min(p_begin + a.pairs_per_split, a.n_pairs);
  // This wave's pairs: p_begin + wave, + 4, ... (count uniform per wave).
  const int n_mine = p_begin + wave < p_end ? (p_end - p_begin - wave + 3) / 4 : 0;

  float acc[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;

  const i32x16 izero = {};
  const f32x16 fzero = {};
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

  // The wave's pairs go in batches of NB: all loads of a batch are issued
  // before its math, so one memory latency covers NB pairs.  Slots past the
  // wave's last pair re-load that pair (same addresses) and run with zero
  // scales, so every batch issues the same loads and the same math (a
  // conditional use would let the compiler sink the loads into it).
  constexpr int NB = 4;
  for (int i0 = 0; i0 < n_mine; i0 += NB) {
    PairPart wp[NB], xp[NB][MT];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p_begin + wave + 4 * min(i0 + j, n_mine - 1);
      load_part(wrow + (int64_t)p * 68, h, wp[j]);
#pragma unroll
      for (int m = 0; m < MT; ++m) load_part(xrow[m] + (int64_t)p * 68, h, xp[j][m]);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool keep = h == 0 && i0 + j < n_mine;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        uint32_t sw;
        const i32x4 B = part_operand(wp[j], blk, keep, sw);
        const f16x4 SB = __builtin_bit_cast(f16x4, u32x2{sw, 0u});
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          uint32_t sx;
          const i32x4 A = part_operand(xp[j][m], blk, keep, sx);
          const f16x4 SA = __builtin_bit_cast(f16x4, u32x2{sx, 0u});
          const i32x16 S = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, izero, 0, 0, 0);
          const f32x16 C = __builtin_amdgcn_mfma_f32_32x32x8f16(SA, SB, fzero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][r] = fmaf((float)S[r], C[r], acc[m][r]);
        }
      }
    }
  }

  // Sum the four waves in wave order; wave w finishes values r = 4w .. 4w+3.
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][m][r][lane] = acc[m][r];
  __syncthreads();
  float *dst = a.out + (int64_t)blockIdx.y * a.n_tok * a.out_dim;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 4 * wave + k;
      const float v = ((red[0][m][r][lane] + red[1][m][r][lane]) + red[2][m][r][lane]) +
                      red[3][m][r][lane];
      // Element r of a lane: token 32 m + 8 (r / 4) + 4 h + r % 4, column n.
      const int64_t t = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
      if (t < a.n_tok && o < a.out_dim) dst[t * a.out_dim + o] = v;
    }
  }
}

}  // namespace

bool skinny_supported(int64_t in_dim, int64_t n_tok) {
  return in_dim > 0 && in_dim % 64 == 0 && n_tok >= 1 && n_tok <= kSkinnyMaxTokens;
}

// Splits: enough workgroups for the chip (about 256), at least one pair per
// wave, at most 16.
int skinny_auto_split(int64_t in_dim, int64_t out_dim) {
  const int64_t tiles = (out_dim + 31) / 32;
  const int64_t pairs = in_dim / 64;
  int64_t split = (256 + tiles - 1) / tiles;
  split = std::min<int64_t>(split, std::max<int64_t>(pairs / 4, 1));
  split = std::min<int64_t>(split, 16);
  return (int)std::max<int64_t>(split, 1);
}

size_t skinny_workspace_bytes(int64_t out_dim, int64_t n_tok, int split) {
  return split > 1 ? (size_t)split * (size_t)out_dim * (size_t)n_tok * sizeof(float) : 0;
}

hipError_t launch_skinny(float *out, const void *w, int64_t in_dim, int64_t out_dim,
                         const void *x_q, int64_t n_tok, int split, float *partials,
                         hipStream_t s) {
  SkinnyArgs a{};
  a.n_pairs = (int32_t)(in_dim / 64);
  const int pps = (a.n_pairs + split - 1) / split;
  const int n_split = (a.n_pairs + pps - 1) / pps;
  a.out = n_split > 1 ? partials : out;
  a.w = static_cast<const uint8_t *>(w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.out_dim = out_dim;
  a.n_tok = n_tok;
  a.row_bytes = (in_dim / 32) * 34;
  a.pairs_per_split = pps;
  const dim3 grid((uint32_t)((out_dim + 31) / 32), (uint32_t)n_split);
  if (n_tok > 32) hipLaunchKernelGGL(skinny_kernel<2>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(skinny_kernel<1>, grid, dim3(256), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_split == 1) return err;
  return launch_splitk_reduce(out, partials, n_tok * out_dim, n_split, s);
}

}  // namespace q8
