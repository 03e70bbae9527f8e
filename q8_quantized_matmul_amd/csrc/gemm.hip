// gemm.hip -- Q8_0 x Q8_0 GEMM on gfx950 matrix cores for many tokens
// (prefill, and any call with more than 64 tokens; 12..64 go to the skinny
// kernel).
//
// Same arithmetic as the matvec ("Part 6: 代码走读", trace 3): per output
// (t, o) and 32-value block b, an exact int32 block dot S_b times the exact
// fp32 scale product d_w * d_x, summed in fp32.  The pages move batched
// Q8_0 matmuls onto matrix units ("Part 6: GPU 加速", C3 NAX paragraph) and
// accept a different fp32 reduction order for batched GEMMs than for decode
// ("Part 6: GPU 加速", section 4m); this kernel is deterministic but not
// bitwise equal to the matvec.
//
// gfx950 mapping:
//   * One K-step of v_mfma_i32_32x32x32_i8 is exactly one Q8_0 block, so every
//     MFMA result is a 32x32 tile of exact S_b (rows = output features o,
//     columns = tokens t).
//   * The per-element scale d_w[o] * d_x[t] of that block is the outer product
//     of two binary16 vectors: one v_mfma_f32_32x32x8_f16 with only K-slot 0
//     populated yields it exactly in fp32, in the same accumulator layout.
//     The VALU then does 2 ops per element and block (int->float, fma); the
//     four-tile kernel moves the int->float conversion onto the matrix core
//     as well (a biased int8 accumulator and an exact f16-MFMA unbias) and
//     keeps one fma.
//   * Workgroup = 4 waves in a 2x2 grid, each wave TI x TJ tiles of 32x32.
//     A K-stage of KB blocks stages qs of 64*TI weight rows and 64*TJ token
//     rows into LDS as aligned 16-byte chunks (row stride KB*32+16 bytes, so
//     ds_read_b128 rows fall on distinct banks) and the binary16 scales in
//     separate arrays.  Global loads fetch whole block pairs (68 bytes) per
//     lane; the misaligned first block of a pair is realigned in registers.
//     The next stage's global loads are issued before the current stage's
//     MFMAs (register prefetch).
//   * The whole-tile shapes of both prefill workloads take gemm_t4_kernel
//     (four 32x32 tiles per wave, direct-to-LDS copies, further down); the
//     kernels here take the rest.
//   * Split-K writes fp32 partials to caller workspace; a second kernel sums
//     them in split order (deterministic, no atomics).
#include <utility>

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
  int32_t tiles_o;   // output-row tiles
  int32_t tiles_t;   // token tiles
  int32_t n_split;
};

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.  The
// linear workgroup id is renumbered so that each XCD receives a contiguous run
// of tiles, and runs are laid out as bands of kGroupO output-row tiles by all
// token tiles, split-major: the workgroups sharing an XCD then share weight
// and activation panels in its L2.
constexpr int kXcds = 8;
constexpr int kGroupO = 8;

__device__ __forceinline__ void tile_of(const GemmArgs &a, int &to, int &tt, int &ts) {
  const int n = a.tiles_o * a.tiles_t * a.n_split;
  const int lin = blockIdx.x;
  int l = lin;
  if (n % kXcds == 0) l = (lin % kXcds) * (n / kXcds) + lin / kXcds;
  const int per_split = a.tiles_o * a.tiles_t;
  ts = l / per_split;
  const int r = l - ts * per_split;
  const int band = r / (kGroupO * a.tiles_t);
  const int o0 = band * kGroupO;
  const int width = min(kGroupO, a.tiles_o - o0);
  const int w = r - band * kGroupO * a.tiles_t;
  to = o0 + w % width;
  tt = w / width;
}

template <int TI, int TJ, int KB, bool STORE_S>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs a) {
  constexpr int BO = 64 * TI;         // output rows per workgroup
  constexpr int BT = 64 * TJ;         // tokens per workgroup
  constexpr int ROWB = KB * 32 + 16;  // LDS bytes per row (padded)
  constexpr int PPR = KB / 2;         // block pairs per row per stage
  constexpr int NPAIR_W = BO * PPR;
  constexpr int NPAIR = NPAIR_W + BT * PPR;
  constexpr int PPT = (NPAIR + 255) / 256;
  constexpr int NT = TI * TJ;         // MFMA tiles per wave
  static_assert(KB % 2 == 0, "stage must hold whole block pairs");
  constexpr bool FULL = NPAIR % 256 == 0;  // every lane loads PPT pairs

  __shared__ __attribute__((aligned(16))) uint8_t qsW[BO * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t qsX[BT * ROWB];
  __shared__ uint16_t scW[KB][BO];
  __shared__ uint16_t scX[KB][BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int to, tt, ts;
  tile_of(a, to, tt, ts);
  const int64_t o_tile = (int64_t)to * BO;
  const int64_t t_tile = (int64_t)tt * BT;
  const int64_t b_begin = (int64_t)ts * a.blocks_per_split;
  const int64_t b_end = min(b_begin + a.blocks_per_split, a.nb);
  const int o_w = (wave & 1) * 32 * TI;   // wave's first row inside the tile
  const int t_w = (wave >> 1) * 32 * TJ;  // wave's first token inside the tile

  // Load descriptors: each lane fetches PPT block pairs per stage.  Rows past
  // the matrix are clamped to its last row (their outputs are never stored);
  // pairs past the K range re-read the last valid pair with zeroed scales.
  const uint8_t *src[PPT];
  uint8_t *dst_qs[PPT];
  uint16_t *dst_sc[PPT];
  int sc_ld[PPT];
  int blk_off[PPT];  // first block of the lane's pair inside a stage
#pragma unroll
  for (int p = 0; p < PPT; ++p) {
    const int j = min(tid + 256 * p, NPAIR - 1);
    const bool isw = j < NPAIR_W;
    const int jj = isw ? j : j - NPAIR_W;
    const int row = jj / PPR;
    const int pr = jj % PPR;
    const int64_t grow = min((isw ? o_tile : t_tile) + row, (isw ? a.out_dim : a.n_tok) - 1);
    src[p] = (isw ? a.w : a.x_q) + grow * a.row_bytes;
    dst_qs[p] = (isw ? qsW : qsX) + row * ROWB + pr * 64;
    dst_sc[p] = (isw ? &scW[2 * pr][row] : &scX[2 * pr][row]);
    sc_ld[p] = isw ? BO : BT;
    blk_off[p] = 2 * pr;
  }

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
      if (!FULL && tid + 256 * p >= NPAIR) continue;
      const int64_t blk = b0 + blk_off[p];
      const bool kvalid = blk < b_end;
      load_pair(src[p] + (kvalid ? blk : b_end - 2) * kBlockBytes, pre[p]);
      if (!kvalid) {
        pre[p][0] &= 0xFFFF0000u;  // scale of the pair's first block
        pre[p][8] &= 0x0000FFFFu;  // scale of the pair's second block
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      if (!FULL && tid + 256 * p >= NPAIR) continue;
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
      i32x4 *q = reinterpret_cast<i32x4 *>(dst_qs[p]);
      q[0] = a0;
      q[1] = a1;
      q[2] = b0;
      q[3] = b1;
      dst_sc[p][0] = (uint16_t)(d[0] & 0xFFFFu);
      dst_sc[p][sc_ld[p]] = (uint16_t)(d[8] >> 16);
    }
  };

  const int lrow = lane & 31;          // row/column of the 32x32 operand this lane feeds
  const int khalf = (lane >> 5) * 16;  // which 16 bytes of the block's 32 quants
  const i32x16 izero = {};
  const f32x16 fzero = {};

  // Scale tile of a block: every lane feeds the binary16 scale of its row
  // (column) into K-slot 0 of its half, so the f16 MFMA returns
  // 2 * d_w[o] * d_x[t] exactly; the final store multiplies by 0.5.
  auto tile_mfma = [&](int kb, int t, i32x16 &S, f32x16 &C) {
    const int i = t / TJ, j = t % TJ;
    const int ro = o_w + 32 * i + lrow;
    const int rt = t_w + 32 * j + lrow;
    const i32x4 A = *reinterpret_cast<const i32x4 *>(qsW + ro * ROWB + kb * 32 + khalf);
    const i32x4 B = *reinterpret_cast<const i32x4 *>(qsX + rt * ROWB + kb * 32 + khalf);
    const f16x4 SA = {__builtin_bit_cast(_Float16, scW[kb][ro]), (_Float16)0, (_Float16)0, (_Float16)0};
    const f16x4 SB = {__builtin_bit_cast(_Float16, scX[kb][rt]), (_Float16)0, (_Float16)0, (_Float16)0};
    S = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, izero, 0, 0, 0);
    C = __builtin_amdgcn_mfma_f32_32x32x8f16(SA, SB, fzero, 0, 0, 0);
  };

  gload(b_begin);
  for (int64_t b0 = b_begin; b0 < b_end; b0 += KB) {
    __syncthreads();
    lstore();
    __syncthreads();
    gload(b0 + KB);  // past the end: clamped, in-bounds, unused
    // Software pipeline over (block, tile): the MFMAs of the next tile are
    // issued before the int->float + fma epilogue of the current one.  Blocks
    // past the K range carry zero scales, so every stage runs all KB blocks.
    i32x16 S[2];
    f32x16 C[2];
    tile_mfma(0, 0, S[0], C[0]);
#pragma unroll
    for (int step = 0; step < KB * NT; ++step) {
      const int kb = step / NT, t = step % NT;
      if (step + 1 < KB * NT) tile_mfma((step + 1) / NT, (step + 1) % NT, S[(step + 1) & 1], C[(step + 1) & 1]);
      const int i = t / TJ, j = t % TJ;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[i][j][r] = fmaf((float)S[step & 1][r], C[step & 1][r], acc[i][j][r]);
      if constexpr (STORE_S) {
        const int64_t tt = t_tile + t_w + 32 * j + lrow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t o = o_tile + o_w + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (tt < a.n_tok && o < a.out_dim && b0 + kb < b_end)
            a.blocksums[(tt * a.out_dim + o) * a.nb + b0 + kb] = S[step & 1][r];
        }
      }
    }
  }

  // Accumulator layout of a 32x32 MFMA tile: lane l holds column l%32 and
  // rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.  The 0.5 undoes the doubled
  // scale tile (exact).
  float *dst = a.out + (int64_t)ts * a.n_tok * a.out_dim;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t t = t_tile + t_w + 32 * j + lrow;
      if (t < a.n_tok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t o = o_tile + o_w + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (o < a.out_dim) dst[t * a.out_dim + o] = 0.5f * acc[i][j][r];
        }
      }
    }
  }
}

// ---- Direct-to-LDS variant (in_dim % 256 == 0, n_tok > 64) -------------
// A stage is 8 blocks = 272 bytes of every row = 17 aligned 16-byte chunks.
// global_load_lds_dwordx4 copies 64 consecutive chunks per wave instruction
// straight into LDS (no VGPR staging, no repack), rows kept contiguous, so
// each instruction reads ~1 KB of contiguous rows.  Two stages ring in LDS:
// the copies of stage s+1 are in flight while stage s is multiplied, with one
// barrier per stage.  An MFMA operand (16 quant bytes at 34*kb + 2 + 16*h in
// the row) spans at most two chunks: two aligned ds_read_b128 and, for even
// blocks, four v_alignbyte realign it.  Workgroup = 8 waves on a 128x128
// tile, each wave 32 output rows x 64 tokens (two 32x32 MFMA tiles).
namespace lds {
constexpr int BO = 128;
constexpr int BT = 128;
constexpr int ROWS = BO + BT;
constexpr int KB = 8;
constexpr int RB = KB * kBlockBytes;    // 272
constexpr int CPR = RB / 16;            // 17
constexpr int REGION_W = BO * RB;       // weight rows first, then token rows
constexpr int STAGE = ROWS * RB;        // 69632 bytes
constexpr int INSTS = ROWS * CPR / 64;  // 68 wave loads per stage
constexpr int WAVES = 8;
constexpr int LPW = (INSTS + WAVES - 1) / WAVES;
static_assert(ROWS * CPR % 64 == 0 && (BO * CPR) % 64 == 0, "whole wave loads per region");
}  // namespace lds

// Raw LDS data of one operand of block KBI: the 16-byte chunk holding the
// first quant byte of half h and the chunk after it.  The block's binary16
// scale sits two bytes before its quants, i.e. inside chunk 0 for every block
// but the last of a stage, whose scale is read separately.
struct RawOperand {
  i32x4 c0, c1;
  uint32_t scale7;  // only for the last block of a stage
};

template <int KBI>
__device__ __forceinline__ RawOperand read_operand(const uint8_t *row, int h) {
  constexpr int O = KBI * kBlockBytes + 2;  // quant offset for h = 0
  constexpr int M = O % 16;
  const uint8_t *p = row + (O - M) + 16 * h;
  RawOperand r;
  r.c0 = *reinterpret_cast<const i32x4 *>(p);
  if constexpr (M != 0) r.c1 = *reinterpret_cast<const i32x4 *>(p + 16);
  if constexpr (M < 2) r.scale7 = *reinterpret_cast<const uint16_t *>(row + KBI * kBlockBytes);
  return r;
}

// 16 quant bytes of the operand realigned for the MFMA, and its scale bits for
// half 0 (zero for half 1).
template <int KBI>
__device__ __forceinline__ i32x4 prepare_operand(const RawOperand &r, int h, uint32_t &scale) {
  constexpr int O = KBI * kBlockBytes + 2;
  constexpr int M = O % 16;
  const uint32_t d0[4] = {(uint32_t)r.c0.x, (uint32_t)r.c0.y, (uint32_t)r.c0.z, (uint32_t)r.c0.w};
  if constexpr (M >= 2) {
    constexpr int SB = M - 2;  // byte of the scale inside chunk 0 (even)
    scale = h ? 0u : (d0[SB / 4] >> (8 * (SB % 4))) & 0xFFFFu;
  } else {
    scale = h ? 0u : r.scale7;
  }
  if constexpr (M == 0) {
    return r.c0;
  } else {
    const uint32_t d[8] = {d0[0], d0[1], d0[2], d0[3],
                           (uint32_t)r.c1.x, (uint32_t)r.c1.y, (uint32_t)r.c1.z, (uint32_t)r.c1.w};
    constexpr int K = M / 4;
    if constexpr (M % 4 == 0) {
      return i32x4{(int)d[K], (int)d[K + 1], (int)d[K + 2], (int)d[K + 3]};
    } else {
      return i32x4{(int)__builtin_amdgcn_alignbyte(d[K + 1], d[K], 2),
                   (int)__builtin_amdgcn_alignbyte(d[K + 2], d[K + 1], 2),
                   (int)__builtin_amdgcn_alignbyte(d[K + 3], d[K + 2], 2),
                   (int)__builtin_amdgcn_alignbyte(d[K + 4], d[K + 3], 2)};
    }
  }
}

template <bool STORE_S>
__global__ __launch_bounds__(512, 1) void gemm_lds_kernel(const GemmArgs a) {
  using namespace lds;
  __shared__ __attribute__((aligned(16))) uint8_t ring[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int to, tt, ts;
  tile_of(a, to, tt, ts);
  const int64_t o_tile = (int64_t)to * BO;
  const int64_t t_tile = (int64_t)tt * BT;
  const int64_t b_begin = (int64_t)ts * a.blocks_per_split;
  const int64_t b_end = min(b_begin + a.blocks_per_split, a.nb);
  const int nstages = (int)((b_end - b_begin) / KB);  // splits are whole stages

  // Copy descriptors: wave load i moves chunks [64*local, 64*local + 64) of the
  // weight (local < 34) or token region.  Rows past the matrix are clamped to
  // its last row; their outputs are never stored.
  const uint8_t *src[LPW];
  uint32_t dst[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int inst = min(wave + WAVES * i, INSTS - 1);
    const bool isw = inst < INSTS / 2;
    const int local = isw ? inst : inst - INSTS / 2;
    const int c = local * 64 + lane;
    const int row = c / CPR;
    const int part = c - row * CPR;
    const int64_t grow = min((isw ? o_tile : t_tile) + row, (isw ? a.out_dim : a.n_tok) - 1);
    src[i] = (isw ? a.w : a.x_q) + grow * a.row_bytes + part * 16;
    dst[i] = (isw ? 0u : (uint32_t)REGION_W) + (uint32_t)local * 1024u;
  }
  auto issue = [&](int64_t b0, int buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      if (wave + WAVES * i < INSTS)  // uniform per wave
        __builtin_amdgcn_global_load_lds(src[i] + b0 * kBlockBytes, ring + buf * STAGE + dst[i], 16, 0, 0);
    }
  };

  const int wo = wave & 3;   // 32 output rows each
  const int wt = wave >> 2;  // 64 tokens each
  const int lrow = lane & 31;
  const int h = lane >> 5;
  const i32x16 izero = {};
  const f32x16 fzero = {};
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  // Results of one block's MFMAs (two token tiles), consumed one block later.
  struct BlockOut {
    i32x16 S[2];
    f32x16 C[2];
  };
  auto epilogue = [&](const BlockOut &o, int64_t b) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = fmaf((float)o.S[j][r], o.C[j][r], acc[j][r]);
      if constexpr (STORE_S) {
        const int64_t t = t_tile + 64 * wt + 32 * j + lrow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t oo = o_tile + 32 * wo + 8 * (r >> 2) + 4 * h + (r & 3);
          if (b >= 0 && t < a.n_tok && oo < a.out_dim) a.blocksums[(t * a.out_dim + oo) * a.nb + b] = o.S[j][r];
        }
      }
    }
  };

  // `prev` starts as zero tiles (its epilogue adds exactly 0), so every step
  // runs the same straight-line code.
  BlockOut prev;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    prev.S[j] = izero;
    prev.C[j] = fzero;
  }
  int64_t prev_b = -1;  // block of `prev`, -1 before the first block
  issue(b_begin, 0);
  for (int s = 0; s < nstages; ++s) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of stage s have landed
    __syncthreads();                // ... and every wave's; buffer (s+1)&1 is free
    if (s + 1 < nstages) issue(b_begin + (int64_t)(s + 1) * KB, (s + 1) & 1);
    const uint8_t *st = ring + (s & 1) * STAGE;
    const uint8_t *arow = st + (32 * wo + lrow) * RB;
    const uint8_t *brow0 = st + REGION_W + (64 * wt + lrow) * RB;
    const uint8_t *brow1 = brow0 + 32 * RB;
    const int64_t b0 = b_begin + (int64_t)s * KB;

    // Per block, four groups kept in this order: realignment of this block's
    // operands (read one block earlier), LDS reads of the next block's
    // operands, the MFMAs of this block, and the int->float/fma epilogue of
    // the previous block.  The previous
    // block's MFMA results and the next block's LDS data thus have a whole
    // group of work to arrive.  The scale tile comes from an f16 MFMA whose
    // K-slot 0 holds the binary16 scales (half 1 feeds zeros), giving
    // d_w * d_x exactly in the accumulator layout of the int8 tile.
    RawOperand ra = read_operand<0>(arow, h);
    RawOperand rb0 = read_operand<0>(brow0, h);
    RawOperand rb1 = read_operand<0>(brow1, h);
    [&]<int... KBI>(std::integer_sequence<int, KBI...>) {
      (([&] {
         uint32_t sa, sb0, sb1;
         const i32x4 A = prepare_operand<KBI>(ra, h, sa);
         const i32x4 B0 = prepare_operand<KBI>(rb0, h, sb0);
         const i32x4 B1 = prepare_operand<KBI>(rb1, h, sb1);
         __builtin_amdgcn_sched_barrier(0);
         if constexpr (KBI + 1 < KB) {
           ra = read_operand<KBI + 1>(arow, h);
           rb0 = read_operand<KBI + 1>(brow0, h);
           rb1 = read_operand<KBI + 1>(brow1, h);
         }
         __builtin_amdgcn_sched_barrier(0);
         BlockOut cur;
         const f16x4 SA = __builtin_bit_cast(f16x4, u32x2{sa, 0u});
         cur.S[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B0, izero, 0, 0, 0);
         cur.C[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(SA, __builtin_bit_cast(f16x4, u32x2{sb0, 0u}), fzero, 0, 0, 0);
         cur.S[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B1, izero, 0, 0, 0);
         cur.C[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(SA, __builtin_bit_cast(f16x4, u32x2{sb1, 0u}), fzero, 0, 0, 0);
         epilogue(prev, prev_b);
         // Interleave: each MFMA of this block followed by 16 epilogue VALU ops.
#pragma unroll
         for (int g = 0; g < 4; ++g) {
           __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
           __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // 16 VALU
         }
         __builtin_amdgcn_sched_barrier(0);
         prev = cur;
         prev_b = b0 + KBI;
       }()), ...);
    }(std::make_integer_sequence<int, KB>{});
  }
  epilogue(prev, prev_b);

  float *dstp = a.out + (int64_t)ts * a.n_tok * a.out_dim;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t t = t_tile + 64 * wt + 32 * j + lrow;
    if (t < a.n_tok) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t o = o_tile + 32 * wo + 8 * (r >> 2) + 4 * h + (r & 3);
        if (o < a.out_dim) dstp[t * a.out_dim + o] = acc[j][r];
      }
    }
  }
}

// ---- Four-tile kernel: 128 x 128 workgroup tiles, 4 waves of 64 x 64.
//
// Each wave owns four independent 32x32 MFMA tiles, so the scale epilogue of
// one tile (one fma per output and block; the int32 -> fp32 conversion runs
// on the matrix core, see below) overlaps the matrix-core work of the next,
// and two workgroups per CU give each SIMD two such waves.
//
// Stages of 4 blocks: a row's 4 blocks are a 136-byte slice (dwords d0..d33),
// staged as nine 16-byte slots at a 144-byte LDS pitch -- slice dwords 0..3,
// 4..7, ..., 28..31 and 30..33 -- so (128 token rows + 128 weight rows) x 144
// bytes = 36 KB per stage, two stages per workgroup.  The stage is filled by
// 16-byte direct-to-LDS loads: lane l of copy instruction k moves slot
// (64k + l) % 9 of row (64k + l) / 9 of its wave's 64-row region, so nine
// instructions cover the wave's rows.  The copies of the next stage are
// spread over the current one (three after each of its first three blocks)
// rather than issued together after the barrier.
//
// Operands: K permuted the same way on both sides so that each is one
// aligned 16-byte LDS read plus a v_bfi patch (perm_read / perm_prep in
// q8_device.h, which states the permutation).  (An earlier version realigned
// 24-byte windows with four v_alignbyte per operand, from 8-byte reads that
// conflicted on every other row; this one takes 1 instead of 4 VALU
// operations per operand and tile-block.)
//
// The MFMA's A operand is the token tile and B the weight tile, so a lane's
// column of the result is an output column and the stores coalesce.  Only
// whole tiles: out_dim and n_tok multiples of 128, in_dim of 128.  Its debug
// instantiation writes every block's S_b as well.
namespace t4 {
constexpr int BO = 128;
constexpr int BT = 128;
constexpr int KB = 4;
constexpr int RB = 144;
constexpr int CH = RB / 16;
constexpr int STAGE = (BO + BT) * RB;
constexpr int WAVE_BYTES = 64 * RB;
constexpr int NCOPY = 64 * CH / 64;
}  // namespace t4

template <bool STORE_S>
__global__ __launch_bounds__(256, 2) void gemm_t4_kernel(const GemmArgs a) {
  using namespace t4;
  __shared__ __attribute__((aligned(16))) uint8_t ring[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int to, tt, ts;
  tile_of(a, to, tt, ts);
  const int64_t o_tile = (int64_t)to * BO;
  const int64_t t_tile = (int64_t)tt * BT;
  const int64_t b_begin = (int64_t)ts * a.blocks_per_split;
  const int64_t b_end = min(b_begin + a.blocks_per_split, a.nb);
  const int nstages = (int)((b_end - b_begin) / KB);

  // Copies as in the four-tile kernel: waves 0, 1 token rows, 2, 3 weight
  // rows; lane l of copy k moves slot (64k + l) % 9 of row (64k + l) / 9.
  uint32_t off[NCOPY];
#pragma unroll
  for (int k = 0; k < NCOPY; ++k) {
    const int f = 64 * k + lane;
    const int r = f / CH;
    const int j = f - r * CH;
    off[k] = (uint32_t)(r * (int)a.row_bytes + (j < CH - 1 ? 16 * j : KB * kBlockBytes - 16));
  }
  const uint8_t *copy_base = wave < 2 ? a.x_q + (t_tile + 64 * wave) * a.row_bytes
                                      : a.w + (o_tile + 64 * (wave - 2)) * a.row_bytes;
  const rsrc_t rsrc = make_rsrc(copy_base, (uint32_t)(64 * a.row_bytes));
  auto issue = [&](int64_t b0, int buf) {
    const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(ring + buf * STAGE + wave * WAVE_BYTES);
    const int sb = (int)(b0 * kBlockBytes);
#pragma unroll
    for (int k = 0; k < NCOPY; ++k) {
      buffer_load_lds_raw(rsrc,
                          reinterpret_cast<__attribute__((address_space(3))) uint32_t *>(
                              (uintptr_t)(lds + 1024 * k)),
                          16, (int)off[k], sb, 0, 0);
    }
  };

  const int wt = wave & 1;
  const int wo = wave >> 1;
  const int lrow = lane & 31;
  const int h = lane >> 5;
  const f32x16 fzero = {};
  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;

  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const i32x16 ibias = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                        0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                        0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
  const f16x4 unbias_a = h ? f16x4{0, 0, 0, 0} : f16x4{(_Float16)-3072.0f, 0, 0, 0};
  const f16x4 unbias_b = h ? f16x4{0, 0, 0, 0} : f16x4{(_Float16)4096.0f, 0, 0, 0};
  const PermLane pl(h);

  struct TileOut {
    f32x16 S;
    f32x16 C;
  };
  TileOut slot[2];
  slot[1].S = fzero;
  slot[1].C = fzero;
  auto epilogue = [&]<int Q>(const TileOut &o) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[Q][r] = fmaf(o.S[r], o.C[r], acc[Q][r]);
  };

  using Raw = PermRaw;
  auto read_raw = [&]<int B>(const uint8_t *row, Raw &r) { perm_read<B>(row, h, r); };
  auto prep = [&]<int B>(const Raw &r, uint32_t &scale) -> i32x4 { return perm_prep<B>(r, pl, scale); };

  issue(b_begin, 0);
  for (int s = 0; s < nstages; ++s) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of stage s have landed
    __syncthreads();                // ... and every wave's; buffer (s+1)&1 is free
    const uint8_t *st = ring + (s & 1) * STAGE;
    const uint8_t *arow0 = st + (64 * wt + lrow) * RB;
    const uint8_t *arow1 = arow0 + 32 * RB;
    const uint8_t *brow0 = st + (BT + 64 * wo + lrow) * RB;
    const uint8_t *brow1 = brow0 + 32 * RB;
    const int64_t stage_b0 = b_begin + (int64_t)s * KB;
    // The next stage's copies go out three at a time after blocks 0..2.  On
    // the last stage they re-read this stage into the idle buffer (in
    // bounds, never read) instead of branching: a branch in the middle of
    // the pipelined block sequence made the compiler spill.
    const uint32_t next_lds =
        (uint32_t)reinterpret_cast<uintptr_t>(ring + ((s + 1) & 1) * STAGE + wave * WAVE_BYTES);
    const int next_sb = (int)((b_begin + (int64_t)(s + 1 < nstages ? s + 1 : s) * KB) * kBlockBytes);

    Raw xa0, xa1, xb0, xb1;
    read_raw.template operator()<0>(arow0, xa0);
    read_raw.template operator()<0>(arow1, xa1);
    read_raw.template operator()<0>(brow0, xb0);
    read_raw.template operator()<0>(brow1, xb1);
    [&]<int... B>(std::integer_sequence<int, B...>) {
      (([&] {
         const int64_t blk = stage_b0 + B;
         uint32_t sa0, sa1, sb0, sb1;
         const i32x4 A0 = prep.template operator()<B>(xa0, sa0);
         const i32x4 A1 = prep.template operator()<B>(xa1, sa1);
         const i32x4 B0 = prep.template operator()<B>(xb0, sb0);
         const i32x4 B1 = prep.template operator()<B>(xb1, sb1);
         __builtin_amdgcn_sched_barrier(0);
         if constexpr (B + 1 < KB) {
           read_raw.template operator()<B + 1>(arow0, xa0);
           read_raw.template operator()<B + 1>(arow1, xa1);
           read_raw.template operator()<B + 1>(brow0, xb0);
           read_raw.template operator()<B + 1>(brow1, xb1);
         }
         __builtin_amdgcn_sched_barrier(0);
         const f16x4 SA[2] = {__builtin_bit_cast(f16x4, u32x2{sa0, 0u}),
                              __builtin_bit_cast(f16x4, u32x2{sa1, 0u})};
         const f16x4 SB[2] = {__builtin_bit_cast(f16x4, u32x2{sb0, 0u}),
                              __builtin_bit_cast(f16x4, u32x2{sb1, 0u})};
         const i32x4 AA[2] = {A0, A1};
         const i32x4 BB[2] = {B0, B1};
         [&]<int... Q>(std::integer_sequence<int, Q...>) {
           (([&] {
              TileOut &cur = slot[Q & 1];
              const TileOut &prev = slot[(Q + 1) & 1];
              __builtin_amdgcn_s_setprio(1);
              const i32x16 biased =
                  __builtin_amdgcn_mfma_i32_32x32x32_i8(AA[Q >> 1], BB[Q & 1], ibias, 0, 0, 0);
              cur.C = __builtin_amdgcn_mfma_f32_32x32x8f16(SA[Q >> 1], SB[Q & 1], fzero, 0, 0, 0);
              cur.S = __builtin_amdgcn_mfma_f32_32x32x8f16(unbias_a, unbias_b,
                                                          __builtin_bit_cast(f32x16, biased), 0, 0, 0);
              if constexpr (STORE_S) {
                const int64_t o = o_tile + 64 * wo + 32 * (Q & 1) + lrow;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int64_t t = t_tile + 64 * wt + 32 * (Q >> 1) + 8 * (r >> 2) + 4 * h + (r & 3);
                  a.blocksums[(t * a.out_dim + o) * a.nb + blk] = (int32_t)cur.S[r];
                }
              }
              epilogue.template operator()<(Q + 3) & 3>(prev);
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
              __builtin_amdgcn_s_setprio(0);
              __builtin_amdgcn_sched_barrier(0);
            }()), ...);
         }(std::make_integer_sequence<int, 4>{});
         if constexpr (B < 3) {
#pragma unroll
           for (int kk = 0; kk < 3; ++kk) {
             const int k = 3 * B + kk;
             buffer_load_lds_raw(rsrc,
                                 reinterpret_cast<__attribute__((address_space(3))) uint32_t *>(
                                     (uintptr_t)(next_lds + 1024 * k)),
                                 16, (int)off[k], next_sb, 0, 0);
           }
         }
         __builtin_amdgcn_sched_barrier(0);
       }()), ...);
    }(std::make_integer_sequence<int, KB>{});
  }
  epilogue.template operator()<3>(slot[1]);
  __builtin_amdgcn_s_waitcnt(0);  // the last stage's copies land before the workgroup ends

  float *dstp = a.out + (int64_t)ts * a.n_tok * a.out_dim;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t o = o_tile + 64 * wo + 32 * (q & 1) + lrow;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t_tile + 64 * wt + 32 * (q >> 1) + 8 * (r >> 2) + 4 * h + (r & 3);
      dstp[t * a.out_dim + o] = acc[q][r];
    }
  }
}

// out[i] = sum over splits s = 0..n_split-1 (in order) of partials[s][i].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(float *__restrict__ out,
                                                            const float *__restrict__ part,
                                                            int64_t n, int n_split) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // Partials 0, 1, ... summed in that order; eight loads are issued before
  // their adds (past the last split they re-read the last one, unused).
  float v = 0.0f;
  for (int s0 = 0; s0 < n_split; s0 += 8) {
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = part[(int64_t)min(s0 + k, n_split - 1) * n + i];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < n_split) v = s0 + k == 0 ? p[k] : v + p[k];
  }
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
  // Aim for >= 256 workgroups, >= 512 from 256 tokens.  Forced splits, graph
  // replays on one box: at 256 / 512 tokens 16384 -> 4096 69.6 -> 60.4 us
  // (4 -> 8 splits), 16384 -> 2048 at 512 66.5 -> 56.8 (4 -> 8), 32768 ->
  // 1024 at 512 65.2 -> 57.2 (8 -> 16), 4096 -> 8192 at 256 40.8 -> 39.0
  // (2 -> 4) and at 512 59.7 -> 61.3 (1 -> 2); below 256 tokens 256
  // workgroups measured best or even (16384 -> 4096 at 65: 43.5 us with 8
  // splits, 49.7 with 16).
  const int64_t want = n_tok >= 256 ? 512 : 256;
  int64_t split = (want + tiles - 1) / tiles;
  split = std::max<int64_t>(split, (nb + 127) / 128);  // fp32 chains of <= 128 blocks
  split = std::min<int64_t>(split, nb / (2 * kStageBlocks));
  split = std::min<int64_t>(split, 16);
  return (int)std::max<int64_t>(split, 1);
}

// Partials [split][n_tok][out_dim] after the workspace's counter bytes (which
// this kernel leaves untouched, so the skinny kernel's counters stay zero).
size_t gemm_workspace_bytes(int64_t out_dim, int64_t n_tok, int split) {
  return split > 1 ? kWsCounterBytes + (size_t)split * (size_t)out_dim * (size_t)n_tok * sizeof(float)
                   : 0;
}

static bool use_lds_kernel(int64_t nb, int64_t n_tok) { return nb % lds::KB == 0 && n_tok > 64; }

// The four-tile kernel takes whole 128 x 128 tiles and 4-block stages.
// Its copies address a wave's 64 rows with 32-bit buffer offsets, so rows
// are limited to 2^24 bytes.
static bool use_t4_kernel(int64_t nb, int64_t out_dim, int64_t n_tok) {
  return nb % t4::KB == 0 && out_dim % t4::BO == 0 && n_tok % t4::BT == 0 &&
         nb * kBlockBytes <= (int64_t{1} << 24);
}

hipError_t launch_gemm(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                       int64_t out_dim, const void *x_q, int64_t n_tok, int split,
                       void *workspace, hipStream_t s) {
  const int64_t nb = in_dim / kBlockElems;
  float *partials =
      workspace ? reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + kWsCounterBytes)
                : nullptr;
  // The direct-to-LDS kernels copy 16-byte chunks; they take operands whose
  // bases are 16-byte aligned (torch allocations are), the register-staged
  // kernel the rest (it needs 4 bytes).
  const bool a16 = ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(x_q)) & 15) == 0;
  const bool four = a16 && use_t4_kernel(nb, out_dim, n_tok);
  const bool direct = a16 && !four && use_lds_kernel(nb, n_tok);
  const int stage = four ? t4::KB : (direct ? lds::KB : kStageBlocks);
  int64_t bps = (nb + split - 1) / split;
  bps = (bps + stage - 1) / stage * stage;
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
  a.n_split = (int32_t)n_split;
  if (four) {
    a.tiles_o = (int32_t)(out_dim / t4::BO);
    a.tiles_t = (int32_t)(n_tok / t4::BT);
    const dim3 grid((uint32_t)a.tiles_o * (uint32_t)a.tiles_t * (uint32_t)n_split);
    if (blocksums) hipLaunchKernelGGL(gemm_t4_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gemm_t4_kernel<false>, grid, dim3(256), 0, s, a);
  } else if (direct) {
    a.tiles_o = (int32_t)((out_dim + lds::BO - 1) / lds::BO);
    a.tiles_t = (int32_t)((n_tok + lds::BT - 1) / lds::BT);
    const dim3 grid((uint32_t)a.tiles_o * (uint32_t)a.tiles_t * (uint32_t)n_split);
    if (blocksums) hipLaunchKernelGGL(gemm_lds_kernel<true>, grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL(gemm_lds_kernel<false>, grid, dim3(512), 0, s, a);
  } else {
    const int tj = gemm_tj(n_tok);
    a.tiles_o = (int32_t)((out_dim + 127) / 128);
    a.tiles_t = (int32_t)((n_tok + 64 * tj - 1) / (64 * tj));
    const dim3 grid((uint32_t)a.tiles_o * (uint32_t)a.tiles_t * (uint32_t)n_split);
    if (tj == 1) {
      if (blocksums) hipLaunchKernelGGL((gemm_kernel<2, 1, kStageBlocks, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gemm_kernel<2, 1, kStageBlocks, false>), grid, dim3(256), 0, s, a);
    } else {
      if (blocksums) hipLaunchKernelGGL((gemm_kernel<2, 2, kStageBlocks, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gemm_kernel<2, 2, kStageBlocks, false>), grid, dim3(256), 0, s, a);
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_split == 1) return err;
  return launch_splitk_reduce(out, partials, n_tok * out_dim, (int)n_split, s);
}

hipError_t launch_splitk_reduce(float *out, const float *partials, int64_t n, int n_split,
                                hipStream_t s) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, out,
                     partials, n, n_split);
  return hipGetLastError();
}

}  // namespace q8
