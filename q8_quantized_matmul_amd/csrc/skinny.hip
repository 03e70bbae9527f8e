// skinny.hip -- Q8_0 matmul for up to 64 tokens on the matrix cores (the
// plan uses it from 16 tokens), a 32-row output tile per workgroup.
//
// The method is the same as everywhere (ds4-learning "Part 6: 代码走读",
// trace 3: out[t][o] = sum over blocks of d_w * d_x * S_b); this kernel
// covers the regime between the weight-streaming matvec and the LDS-tiled
// GEMM, as the pages' backends keep dedicated kernels and a split-K path for
// narrow batches ("Part 6: GPU 加速", sections 4c and 4s).  Tokens are the
// MFMA's M dimension (one or two 32-token tiles), output rows its N dimension.
//
//   * The workgroup's K range goes through LDS in stages of 4 block pairs
//     (272 bytes of every token and weight row), double-buffered, filled by
//     direct global->LDS copies in which consecutive lanes read consecutive
//     bytes of a row (16-byte copies where rows are whole 16-byte chunks,
//     dword copies otherwise).  Reading the MFMA operand layout straight from
//     memory instead (each lane its own row) left the kernel bound by
//     address processing, 1.2-2x slower depending on the split.
//   * Wave w takes pair w of each stage.  One v_mfma_i32_32x32x32_i8 per
//     (token tile, block) gives the exact S_b of the 32x32 tile; one
//     v_mfma_f32_32x32x8_f16 with only K slot 0 populated gives the matching
//     d_w * d_x outer product, exactly; the epilogue is acc += float(S_b) * scale.
//   * The 4 waves are summed through LDS in wave order; K ranges of different
//     workgroups (split-K) go to partials that the ordered reduce kernel sums.
//     Every sum has a fixed order: results are deterministic.
#include <algorithm>

#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

struct SkinnyArgs {
  float *out;            // [n_tok][out_dim], or partials [n_split][n_tok][out_dim]
  int32_t *blocksums;    // debug: S_b [n_tok][out_dim][2 * n_pairs], or null
  const uint8_t *w;      // [out_dim][row_bytes]
  const uint8_t *x_q;    // [n_tok][row_bytes]
  int64_t out_dim;
  int64_t n_tok;
  int64_t row_bytes;
  int32_t n_pairs;       // block pairs per row
  int32_t pairs_per_split;
};

// A stage holds kStagePairs block pairs (one per wave) of every row of the
// workgroup: 32 * MT token rows, then 32 weight rows, 272 bytes each.
constexpr int kStagePairs = 4;
constexpr int kStageRowBytes = kStagePairs * kPairBytes;  // 272
constexpr int kStageRowDwords = kStageRowBytes / 4;       // 68
constexpr int kCopyPeriod = 17;                           // 17 copies of 64 dwords = 16 rows
static_assert(kCopyPeriod * 64 == 16 * kStageRowDwords, "copy pattern period");

template <int MT>
struct SkinnyStage {
  static constexpr int XROWS = 32 * MT;
  static constexpr int ROWS = XROWS + 32;
  static constexpr int BYTES = ROWS * kStageRowBytes;
};

// One block of the wave's pair: operands from the staged rows, then per
// token tile one int8 MFMA (S_b) and one scale MFMA (d_x * d_w), added as
// acc += float(S_b) * scale.  STORE_S (debug) also writes S_b of block `blk`
// for output column `o`.
template <int B, int MT, bool STORE_S>
__device__ __forceinline__ void skinny_block(const uint8_t *const (&xrow)[MT], const uint8_t *wrow,
                                             int h, float (&acc)[MT][16], const SkinnyArgs &a,
                                             int64_t blk, int64_t o) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const i32x16 izero = {};
  const f32x16 fzero = {};
  T4Raw rw;
  t4_read<B>(wrow, h, rw);
  uint32_t sw;
  const i32x4 Bop = t4_prep<B>(rw, h, sw);
  const f16x4 SB = __builtin_bit_cast(f16x4, u32x2{sw, 0u});
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    T4Raw rx;
    t4_read<B>(xrow[m], h, rx);
    uint32_t sx;
    const i32x4 Aop = t4_prep<B>(rx, h, sx);
    const f16x4 SA = __builtin_bit_cast(f16x4, u32x2{sx, 0u});
    const i32x16 S = __builtin_amdgcn_mfma_i32_32x32x32_i8(Aop, Bop, izero, 0, 0, 0);
    const f32x16 C = __builtin_amdgcn_mfma_f32_32x32x8f16(SA, SB, fzero, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = fmaf((float)S[r], C[r], acc[m][r]);
    if constexpr (STORE_S) {
      // Element r: token 32 m + 8 (r / 4) + 4 h + r % 4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
        if (t < a.n_tok && o < a.out_dim) a.blocksums[(t * a.out_dim + o) * 2 * a.n_pairs + blk] = S[r];
      }
    }
  }
}

// Stage copies, dword granularity (any in_dim % 64 == 0): waves 0 .. MT-1
// move token rows 32 w + r, waves 2 and 3 weight rows o_tile + 16 (w - 2) + r
// (stage rows XROWS + 16 (w - 2) + r).  Lane l of copy k moves flat dword
// 64 k + l of a group of 16 rows.  Each group of 16 rows is read through a
// buffer resource based at that group's first row plus the stage's byte
// offset, whose range ends at the end of the wave's last valid row, and the
// lane's whole offset is its 32-bit voffset: the hardware range check covers
// voffset only (not the scalar offset), so everything a copy adds to the base
// has to be in voffset or in the base.  Rows past the matrix, and the bytes
// past the end of the last valid row (a short last stage), then lie outside
// the range and read as zero; what lands in LDS for them feeds only outputs
// that are not stored, or pairs past the split that no wave multiplies.
template <int MT>
struct DwordCopies {
  static constexpr int XROWS = 32 * MT;
  const uint8_t *gbase = nullptr;
  int64_t valid_bytes = 0;  // bytes of the wave's valid rows, from gbase
  uint32_t off[kCopyPeriod];
  int grp_rows = 0, first = 0, p_begin;
  int64_t rows16;

  __device__ __forceinline__ DwordCopies(const SkinnyArgs &a, int wave, int lane, int64_t o_tile,
                                         int pb)
      : p_begin(pb) {
    int64_t valid = 0;
    if (wave < MT) {
      grp_rows = 32;
      first = 32 * wave;
      gbase = a.x_q + (int64_t)first * a.row_bytes;
      valid = a.n_tok - first;
    } else if (wave >= 2) {
      grp_rows = 16;
      first = XROWS + 16 * (wave - 2);
      const int64_t o0 = o_tile + 16 * (wave - 2);
      gbase = a.w + o0 * a.row_bytes;
      valid = a.out_dim - o0;
    }
    valid = valid < 0 ? 0 : (valid > grp_rows ? grp_rows : valid);
    valid_bytes = valid * a.row_bytes;
#pragma unroll
    for (int k = 0; k < kCopyPeriod; ++k) {
      const int f = 64 * k + lane;
      const int r = f / kStageRowDwords;
      off[k] = (uint32_t)(r * (int)a.row_bytes + 4 * (f - r * kStageRowDwords));
    }
    rows16 = 16 * a.row_bytes;
  }

  __device__ __forceinline__ void issue(uint8_t *stage, int s) const {
    if (grp_rows == 0) return;
    const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(stage + first * kStageRowBytes);
    const int64_t sb = (int64_t)(p_begin + s * kStagePairs) * kPairBytes;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (g == 1 && grp_rows == 16) break;
      // Group g: rows 16 g .. 16 g + 15 of the wave, from byte sb of each row.
      const int64_t start = sb + g * rows16;
      const int64_t left = valid_bytes - start;
      const rsrc_t rsrc = make_rsrc(gbase + start, (uint32_t)(left > 0 ? left : 0));
#pragma unroll
      for (int k = 0; k < kCopyPeriod; ++k) {
        buffer_load_lds_raw(rsrc,
                            reinterpret_cast<__attribute__((address_space(3))) uint32_t *>(
                                (uintptr_t)(lds + 256 * (k + kCopyPeriod * g))),
                            4, (int)off[k], 0, 0, 0);
      }
    }
  }
};

// Stage copies, 16-byte granularity (in_dim % 256 == 0, so every row and
// every stage is whole 16-byte chunks, and 16-byte-aligned operands): the
// stage's ROWS * 17 chunks, x rows then weight rows, go out as 64-chunk wave
// copies, copy i taken by wave i % 4.  Rows past the matrix re-read its last
// row (their outputs are not stored).
template <int MT>
struct ChunkCopies {
  static constexpr int XROWS = 32 * MT;
  static constexpr int CHUNKS = (XROWS + 32) * (kStageRowBytes / 16);
  static constexpr int INSTS = (CHUNKS + 63) / 64;
  static constexpr int PER_WAVE = (INSTS + 3) / 4;
  const uint8_t *src[PER_WAVE];
  int wave, lane, p_begin;

  __device__ __forceinline__ ChunkCopies(const SkinnyArgs &a, int w, int l, int64_t o_tile, int pb)
      : wave(w), lane(l), p_begin(pb) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int c = min(64 * (wave + 4 * j) + lane, CHUNKS - 1);
      const int row = c / (kStageRowBytes / 16);
      const int part = c - row * (kStageRowBytes / 16);
      const int64_t g = row < XROWS ? min<int64_t>(row, a.n_tok - 1)
                                    : min<int64_t>(o_tile + row - XROWS, a.out_dim - 1);
      src[j] = (row < XROWS ? a.x_q : a.w) + g * a.row_bytes + 16 * part;
    }
  }

  __device__ __forceinline__ void issue(uint8_t *stage, int s) const {
    const int64_t sb = (int64_t)(p_begin + s * kStagePairs) * kPairBytes;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int inst = wave + 4 * j;
      if (inst < INSTS && 64 * inst + lane < CHUNKS)
        __builtin_amdgcn_global_load_lds(src[j] + sb, stage + 1024 * inst, 16, 0, 0);
    }
  }
};

// MT token tiles of 32.  Grid: x = 32-row output tiles, y = K splits.
template <int MT, class COPY, bool STORE_S>
__global__ __launch_bounds__(256) void skinny_kernel(const SkinnyArgs a) {
  using St = SkinnyStage<MT>;
  __shared__ __attribute__((aligned(16))) uint8_t ring[2 * St::BYTES];
  static_assert(4 * MT * 16 * 64 * sizeof(float) <= sizeof(ring), "reduction fits the ring");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31;
  const int h = lane >> 5;
  const int64_t o_tile = (int64_t)blockIdx.x * 32;
  const int p_begin = blockIdx.y * a.pairs_per_split;
  const int p_end = min(p_begin + a.pairs_per_split, a.n_pairs);
  const int nstages = (p_end - p_begin + kStagePairs - 1) / kStagePairs;

  COPY copies(a, wave, lane, o_tile, p_begin);
  auto issue = [&](int st, int buf) { copies.issue(ring + buf * St::BYTES, st); };

  float acc[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;

  issue(0, 0);
  for (int s = 0; s < nstages; ++s) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of stage s have landed
    __syncthreads();                // ... and every wave's; buffer (s+1)&1 is free
    if (s + 1 < nstages) issue(s + 1, (s + 1) & 1);
    // Wave w takes pair w of the stage (blocks 2w, 2w+1), which starts 68 w
    // bytes into each staged row: in the 136-byte slice w / 2, at block 0 or 2.
    const int pair = p_begin + s * kStagePairs + wave;
    if (pair < p_end) {
      const uint8_t *st = ring + (s & 1) * St::BYTES + 136 * (wave >> 1);
      const uint8_t *xrow[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) xrow[m] = st + (32 * m + lrow) * kStageRowBytes;
      const uint8_t *wrow = st + (St::XROWS + lrow) * kStageRowBytes;
      const int64_t blk = 2 * (int64_t)pair;  // the pair's first block
      const int64_t o = o_tile + lrow;
      if (wave & 1) {
        skinny_block<2, MT, STORE_S>(xrow, wrow, h, acc, a, blk, o);
        skinny_block<3, MT, STORE_S>(xrow, wrow, h, acc, a, blk + 1, o);
      } else {
        skinny_block<0, MT, STORE_S>(xrow, wrow, h, acc, a, blk, o);
        skinny_block<1, MT, STORE_S>(xrow, wrow, h, acc, a, blk + 1, o);
      }
    }
  }

  // Sum the four waves in wave order; wave w finishes values r = 4w .. 4w+3.
  __syncthreads();  // every wave is done with the ring
  float(*red)[MT][16][64] = reinterpret_cast<float(*)[MT][16][64]>(ring);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][m][r][lane] = acc[m][r];
  __syncthreads();
  const int64_t o = o_tile + lrow;
  float *dst = a.out + (int64_t)blockIdx.y * a.n_tok * a.out_dim;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 4 * wave + k;
      const float v = ((red[0][m][r][lane] + red[1][m][r][lane]) + red[2][m][r][lane]) +
                      red[3][m][r][lane];
      // Element r of a lane: token 32 m + 8 (r / 4) + 4 h + r % 4, column lrow.
      const int64_t t = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
      if (t < a.n_tok && o < a.out_dim) dst[t * a.out_dim + o] = v;
    }
  }
}

// Every variant explicitly instantiated: without this the host side of the
// front end dropped two of them (the host stubs were referenced but never
// emitted).
template __global__ void skinny_kernel<1, ChunkCopies<1>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<2, ChunkCopies<2>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<1, ChunkCopies<1>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<2, ChunkCopies<2>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<1, DwordCopies<1>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<2, DwordCopies<2>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<1, DwordCopies<1>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<2, DwordCopies<2>, true>(const SkinnyArgs);

template <int MT, bool STORE_S>
void launch_skinny_variant(bool wide, dim3 grid, const SkinnyArgs &a, hipStream_t s) {
  if (wide) {
    auto k = skinny_kernel<MT, ChunkCopies<MT>, STORE_S>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
  } else {
    auto k = skinny_kernel<MT, DwordCopies<MT>, STORE_S>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
  }
}

}  // namespace

bool skinny_supported(int64_t in_dim, int64_t n_tok) {
  return in_dim > 0 && in_dim % 64 == 0 && (in_dim / 32) * kBlockBytes <= (1 << 24) && n_tok >= 1 &&
         n_tok <= kSkinnyMaxTokens;
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

hipError_t launch_skinny(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                         int64_t out_dim, const void *x_q, int64_t n_tok, int split,
                         float *partials, hipStream_t s) {
  SkinnyArgs a{};
  a.blocksums = blocksums;
  a.n_pairs = (int32_t)(in_dim / 64);
  // Splits are whole stages (the last one may be short).
  const int pps = (((a.n_pairs + split - 1) / split + kStagePairs - 1) / kStagePairs) * kStagePairs;
  const int n_split = (a.n_pairs + pps - 1) / pps;
  a.out = n_split > 1 ? partials : out;
  a.w = static_cast<const uint8_t *>(w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.out_dim = out_dim;
  a.n_tok = n_tok;
  a.row_bytes = (in_dim / 32) * 34;
  a.pairs_per_split = pps;
  const dim3 grid((uint32_t)((out_dim + 31) / 32), (uint32_t)n_split);
  // 16-byte copies need whole 16-byte chunks: rows of 8k blocks, 16-aligned bases.
  const bool wide = in_dim % 256 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(x_q) & 15) == 0;
  const bool two = n_tok > 32;
  if (blocksums) {
    if (two) launch_skinny_variant<2, true>(wide, grid, a, s);
    else launch_skinny_variant<1, true>(wide, grid, a, s);
  } else {
    if (two) launch_skinny_variant<2, false>(wide, grid, a, s);
    else launch_skinny_variant<1, false>(wide, grid, a, s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_split == 1) return err;
  return launch_splitk_reduce(out, partials, n_tok * out_dim, n_split, s);
}

}  // namespace q8
