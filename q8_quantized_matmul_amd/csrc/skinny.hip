// skinny.hip -- Q8_0 matmul for up to 256 tokens on the matrix cores (the
// plan uses it from 12 to 64 tokens, from 2 for rows the matvec cannot take,
// and up to 256 for moderate shapes, skinny_many_tokens), a 32-row output
// tile per workgroup.
//
// The method is the same as everywhere (ds4-learning "Part 6: 代码走读",
// trace 3: out[t][o] = sum over blocks of d_w * d_x * S_b); this kernel
// covers the regime between the weight-streaming matvec and the LDS-tiled
// GEMM, as the pages' backends keep dedicated kernels and a split-K path for
// narrow batches ("Part 6: GPU 加速", sections 4c and 4s).  Tokens are the
// MFMA's M dimension (one or two 32-token tiles), output rows its N dimension.
//
//   * The workgroup's K range is cut into steps of 2 block pairs (a 136-byte
//     slice of every row).  Eight waves, two per SIMD: wave w takes token
//     tile m = w / KQ and steps w % KQ, w % KQ + KQ, ... (KQ = 8 / MT waves
//     per token tile), and streams them through a private LDS region with
//     its own direct global->LDS copies of the 32 token rows of its tile and
//     the 32 weight rows, staged at a 144-byte pitch with K permuted for
//     aligned 16-byte operand reads (as in the tiled GEMM; q8_device.h
//     perm_read).  Consecutive lanes copy consecutive bytes of a row: 16-byte
//     copies where rows are whole 16-byte chunks, dword copies otherwise.  A
//     wave waits for its own copies only: the K loop has no workgroup
//     barrier, so the waves overlap one another's loads and matrix work.
//   * Per block, one v_mfma_i32_32x32x32_i8 gives the exact S_b of the 32x32
//     tile (converted to fp32 on the matrix core, as in the tiled GEMM) and
//     one v_mfma_f32_32x32x8_f16 with only K slot 0 populated the matching
//     d_w * d_x outer product, exactly; the epilogue is
//     acc += float(S_b) * scale.
//   * The waves of a token tile are summed through LDS in wave order.  With split-K,
//     each workgroup leaves its sums in caller workspace and the last
//     workgroup of an output tile to arrive adds them in split order.  Every
//     sum has a fixed order: results are deterministic.
//   * From 33 tokens with 64 to 128 output tiles, the two token tiles go to
//     separate workgroups (grid z) instead of a K split (skinny_token_split),
//     and with fewer tiles too for rows of up to 64 pairs, beside their K
//     split (skinny_tile_rows);
//     above 64 tokens (up to 256) every token tile does, with one split or,
//     for long rows, two (partials and counters per row and token tile).
#include <algorithm>
#include <utility>

#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

struct SkinnyArgs {
  float *out;            // [n_tok][out_dim]
  float *partials;       // split-K: [n_split][tiles][MT][16][64 lanes], else null
  uint32_t *arrivals;    // split-K: one arrival counter per output tile, else null
  int32_t *blocksums;    // debug: S_b [n_tok][out_dim][2 * n_pairs], or null
  const uint8_t *w;      // [out_dim][row_bytes]
  const uint8_t *x_q;    // [n_tok][row_bytes]
  int64_t out_dim;
  int64_t n_tok;
  int64_t row_bytes;
  int32_t n_pairs;       // block pairs per row
  int32_t pairs_per_split;
};

constexpr int kWaves = 8;
constexpr int kStepPairs = 2;                          // pairs of a row per step
constexpr int kSliceBytes = kStepPairs * kPairBytes;   // 136 bytes of a row per step
constexpr int kPitch = kPermPitch;                     // 144 LDS bytes per staged row
constexpr int kPitchDwords = kPitch / 4;               // 36
constexpr int kGroupCopies = 9;                        // dword copies of 16 staged rows
static_assert(kGroupCopies * 64 == 16 * kPitchDwords, "copy pattern period");

// One wave's staged step: the 32 token rows of its tile, then the 32 weight
// rows, 144 LDS bytes each.
constexpr int kStepRows = 64;
constexpr int kStepBytes = kStepRows * kPitch;  // 9216

// Byte of a row's slice that 16-byte slot j (0..8) of its staged row holds:
// slots 0..7 the first 128 bytes, slot 8 bytes 120..135.
__device__ __forceinline__ int slot_byte(int j) { return j < kPermSlots - 1 ? 16 * j : kSliceBytes - 16; }

// s_waitcnt on the vector-memory counter alone (expcnt and lgkmcnt left at
// their maxima): at most N of this wave's vector memory operations remain.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "the counter holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Step copies, dword granularity (any in_dim % 64 == 0): the step's rows in
// groups of 16 (token rows 32 m + 16 g for g = 0, 1, then weight rows
// o_tile + 16 (g - 2)), 9 copies per group: lane l of copy k moves staged
// dword 64 k + l of the group (row r = that / 36 at LDS byte 4 (that % 36):
// slice dwords 0..31, then 30..33).  Each group is read through a buffer
// resource based at its first row plus the step's byte offset in the row,
// whose range ends at the end of the group's last valid row, and the lane's
// whole offset is its 32-bit voffset: the hardware range check covers
// voffset only (not the scalar offset), so everything a copy adds to the
// base has to be in voffset or in the base.  Rows past the matrix, and the
// bytes past the end of the last valid row (an odd pair count's last step),
// then lie outside the range and read as zero; what lands in LDS for them
// feeds only outputs that are not stored, or a pair past the split that
// runs with zero scales.
template <int R>
struct DwordCopies {
  static constexpr int NBUF = R;
  static constexpr int GROUPS = kStepRows / 16;
  static constexpr int PER_STEP = GROUPS * kGroupCopies;  // this wave's copies per step
  const uint8_t *base[GROUPS];
  int64_t valid_bytes[GROUPS];  // bytes of the group's valid rows, from base
  uint32_t off[kGroupCopies];

  __device__ __forceinline__ DwordCopies(const SkinnyArgs &a, int lane, int m, int64_t o_tile) {
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      int64_t valid;
      if (g < 2) {
        base[g] = a.x_q + (int64_t)(32 * m + 16 * g) * a.row_bytes;
        valid = a.n_tok - (32 * m + 16 * g);
      } else {
        const int64_t o0 = o_tile + 16 * (g - 2);
        base[g] = a.w + o0 * a.row_bytes;
        valid = a.out_dim - o0;
      }
      valid = valid < 0 ? 0 : (valid > 16 ? 16 : valid);
      valid_bytes[g] = valid * a.row_bytes;
    }
#pragma unroll
    for (int k = 0; k < kGroupCopies; ++k) {
      const int f = 64 * k + lane;
      const int r = f / kPitchDwords;
      const int d = f - r * kPitchDwords;
      off[k] = (uint32_t)(r * (int)a.row_bytes + (d < 32 ? 4 * d : kSliceBytes - 16 + 4 * (d - 32)));
    }
  }

  // Copies of the step whose first pair is pair0 into the staged rows at lds.
  __device__ __forceinline__ void issue(uint8_t *lds_step, int pair0) const {
    const int64_t start = (int64_t)pair0 * kPairBytes;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      const int64_t left = valid_bytes[g] - start;
      const rsrc_t rsrc = make_rsrc(base[g] + start, (uint32_t)(left > 0 ? left : 0));
      const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(lds_step + 16 * g * kPitch);
#pragma unroll
      for (int k = 0; k < kGroupCopies; ++k) {
        buffer_load_lds_raw(rsrc,
                            reinterpret_cast<__attribute__((address_space(3))) uint32_t *>(
                                (uintptr_t)(lds + 256 * k)),
                            4, (int)off[k], 0, 0, 0);
      }
    }
  }
};

// Step copies, 16-byte granularity (in_dim % 256 == 0 and 16-byte-aligned
// operands, so every step starts on an 8-byte boundary of a row): the step's
// 64 * 9 slots (row, then slot) go out as 9 copies of 64.  Rows past the
// matrix re-read its last row (their outputs are not stored).
template <int R>
struct ChunkCopies {
  static constexpr int NBUF = R;
  static constexpr int PER_STEP = kStepRows * kPermSlots / 64;  // this wave's copies per step
  static_assert(PER_STEP * 64 == kStepRows * kPermSlots, "whole copies");
  const uint8_t *src[PER_STEP];  // row base + slot byte

  __device__ __forceinline__ ChunkCopies(const SkinnyArgs &a, int lane, int m, int64_t o_tile) {
#pragma unroll
    for (int k = 0; k < PER_STEP; ++k) {
      const int c = 64 * k + lane;
      const int row = c / kPermSlots;
      const int slot = c - row * kPermSlots;
      const uint8_t *rowp = row < 32 ? a.x_q + min<int64_t>(32 * m + row, a.n_tok - 1) * a.row_bytes
                                     : a.w + min<int64_t>(o_tile + row - 32, a.out_dim - 1) * a.row_bytes;
      src[k] = rowp + slot_byte(slot);
    }
  }

  __device__ __forceinline__ void issue(uint8_t *lds_step, int pair0) const {
    const int64_t start = (int64_t)pair0 * kPairBytes;
#pragma unroll
    for (int k = 0; k < PER_STEP; ++k)
      __builtin_amdgcn_global_load_lds(
          src[k] + start,
          reinterpret_cast<__attribute__((address_space(3))) void *>((uintptr_t)(lds_step + 1024 * k)),
          16, 0, 0);
  }
};

// Wait until this wave's oldest in-flight step has landed, with `behind`
// later steps (PW copies each) still allowed in flight (behind < NBUF).
template <int PW, int NBUF>
__device__ __forceinline__ void wait_steps(int behind) {
  static_assert(NBUF == 1 || NBUF == 2, "one or two steps in flight");
  if constexpr (NBUF == 2) {
    if (behind > 0) {
      wait_vmcnt<PW>();
      return;
    }
  }
  wait_vmcnt<0>();
}

// The four blocks of one staged step.  Per block: the int8 MFMA accumulates
// S_b onto the constant 0x4B400000 (1.5 * 2^23 as fp32 bits; |S_b| < 2^22,
// so the int32 sum read as fp32 is exactly 1.5 * 2^23 + S_b), an f16 MFMA
// adds the exact product (-3072) * 4096 = -1.5 * 2^23 in K slot 0 (so the
// tile holds float(S_b) exactly, converted on the matrix core), and another
// gives the d_x * d_w outer product; the VALU is left with one fma per
// output: acc += float(S_b) * scale, in block order.  The next block's
// operands are read before this block's matrix work.  Blocks of a pair at or
// past `pair_end` (an odd pair count's last step) run with zero scales.
// STORE_S (debug) also writes S_b of the valid blocks for output column o,
// tokens of tile m.
template <bool STORE_S>
__device__ __forceinline__ void skinny_step(const uint8_t *st, int lrow, int h, const PermLane &pl,
                                            float (&acc)[16], const SkinnyArgs &a, int pair0,
                                            int pair_end, int m, int64_t o) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const f32x16 fzero = {};
  const i32x16 ibias = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                        0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                        0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
  const f16x4 unbias_a = h ? f16x4{0, 0, 0, 0} : f16x4{(_Float16)-3072.0f, 0, 0, 0};
  const f16x4 unbias_b = h ? f16x4{0, 0, 0, 0} : f16x4{(_Float16)4096.0f, 0, 0, 0};
  const uint8_t *xrow = st + lrow * kPitch;
  const uint8_t *wrow = st + (32 + lrow) * kPitch;
  const bool second = pair0 + 1 < pair_end;  // blocks 2, 3 are a valid pair

  PermRaw rw[2], rx[2];
  perm_read<0>(wrow, h, rw[0]);
  perm_read<0>(xrow, h, rx[0]);
  [&]<int... B>(std::integer_sequence<int, B...>) {
    (([&] {
       constexpr int cur = B & 1, nxt = cur ^ 1;
       uint32_t sw, sx;
       const i32x4 W = perm_prep<B>(rw[cur], pl, sw);
       const i32x4 X = perm_prep<B>(rx[cur], pl, sx);
       if constexpr (B + 1 < 4) {
         perm_read<B + 1>(wrow, h, rw[nxt]);
         perm_read<B + 1>(xrow, h, rx[nxt]);
       }
       if constexpr (B >= 2) {
         if (!second) sw = sx = 0u;
       }
       const i32x16 biased = __builtin_amdgcn_mfma_i32_32x32x32_i8(X, W, ibias, 0, 0, 0);
       const f32x16 S = __builtin_amdgcn_mfma_f32_32x32x8f16(unbias_a, unbias_b,
                                                            __builtin_bit_cast(f32x16, biased), 0, 0, 0);
       const f32x16 C = __builtin_amdgcn_mfma_f32_32x32x8f16(
           __builtin_bit_cast(f16x4, u32x2{sx, 0u}), __builtin_bit_cast(f16x4, u32x2{sw, 0u}),
           fzero, 0, 0, 0);
#pragma unroll
       for (int r = 0; r < 16; ++r) acc[r] = fmaf(S[r], C[r], acc[r]);
       if constexpr (STORE_S) {
         // Element r: token 32 m + 8 (r / 4) + 4 h + r % 4.
         const int64_t blk = 2 * (int64_t)pair0 + B;
         if (B < 2 || second) {
#pragma unroll
           for (int r = 0; r < 16; ++r) {
             const int64_t t = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
             if (t < a.n_tok && o < a.out_dim)
               a.blocksums[(t * a.out_dim + o) * 2 * a.n_pairs + blk] = (int32_t)S[r];
           }
         }
       }
     }()), ...);
  }(std::make_integer_sequence<int, 4>{});
}

// MT token tiles of 32.  Grid: x = 32-row output tiles, y = K splits, z =
// groups of MT token tiles taken by separate workgroups: the workgroup at z
// reads and writes the token rows from 32 MT z on.
template <int MT, class COPY, bool STORE_S>
__global__ __launch_bounds__(512) void skinny_kernel(const SkinnyArgs a0) {
  SkinnyArgs a = a0;
  if (blockIdx.z > 0) {
    const int64_t t0 = 32 * MT * (int64_t)blockIdx.z;
    a.x_q += t0 * a.row_bytes;
    a.out += t0 * a.out_dim;
    if (a.blocksums) a.blocksums += t0 * a.out_dim * 2 * a.n_pairs;
    a.n_tok -= t0;
  }
  constexpr int NBUF = COPY::NBUF;
  constexpr int KQ = kWaves / MT;  // waves per token tile
  constexpr int PER = 2 * MT;      // values of the workgroup's tile set a wave finishes
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves * NBUF * kStepBytes];
  __shared__ uint32_t arrived_before;
  static_assert(kWaves * 16 * 64 * sizeof(float) <= sizeof(ring), "reduction fits the ring");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = wave / KQ;   // token tile
  const int kq = wave % KQ;  // first step of this wave
  const int lrow = lane & 31;
  const int h = lane >> 5;
  const PermLane pl(h);
  const int64_t o_tile = (int64_t)blockIdx.x * 32;
  const int64_t o = o_tile + lrow;
  const int p_begin = blockIdx.y * a.pairs_per_split;
  const int p_end = min(p_begin + a.pairs_per_split, a.n_pairs);
  const int nsteps = (p_end - p_begin + kStepPairs - 1) / kStepPairs;
  const int mine = nsteps > kq ? (nsteps - kq + KQ - 1) / KQ : 0;  // steps of this wave

  COPY copies(a, lane, m, o_tile);
  uint8_t *const region = ring + wave * NBUF * kStepBytes;
  auto pair_of = [&](int i) { return p_begin + kStepPairs * (kq + KQ * i); };

  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  // Step i of this wave lives in buffer i % NBUF of its region; the next
  // step goes out as soon as the buffer it reuses has been read.
  int issued = 0;
  for (; issued < NBUF && issued < mine; ++issued)
    copies.issue(region + issued * kStepBytes, pair_of(issued));
  for (int i = 0; i < mine; ++i) {
    wait_steps<COPY::PER_STEP, NBUF>(issued - i - 1);
    const uint8_t *st = region + (NBUF == 2 ? (i & 1) : 0) * kStepBytes;
    skinny_step<STORE_S>(st, lrow, h, pl, acc, a, pair_of(i), p_end, m, o);
    if (issued < mine) {
      // Every read of buffer i % NBUF has been consumed by the MFMAs above.
      copies.issue(region + (issued % NBUF) * kStepBytes, pair_of(issued));
      ++issued;
    }
  }

  // Sum the KQ waves of each token tile in wave order; wave w finishes
  // values v = PER w .. PER w + PER - 1 of the workgroup (tile v / 16,
  // element v % 16).
  __syncthreads();  // every wave is done with its region (no copy is in flight)
  float(*red)[16][64] = reinterpret_cast<float(*)[16][64]>(ring);
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  float v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int val = PER * wave + k;
    const int tm = val >> 4, r = val & 15;
    float sum = red[KQ * tm][r][lane];
#pragma unroll
    for (int j = 1; j < KQ; ++j) sum += red[KQ * tm + j][r][lane];
    v[k] = sum;
  }

  if (gridDim.y > 1) {
    // Split-K: every workgroup of an output tile leaves its sums in the
    // partials (one coalesced slot per value), then counts itself in.  The
    // last to arrive adds the tile's partials in split order, 0 first, as the
    // ordered reduce would, stores the result and re-arms the counter for the
    // next call.  Nobody waits for anybody.
    //
    // Coherence without cache-wide fences: the partials are stored and
    // loaded with device-scope (agent) atomic accesses, which the L2 of every
    // XCD treats as coherent, and every wave waits for its stores to complete
    // before the barrier that precedes the arrival.  A fence at device scope
    // would write back and invalidate the whole L2 of the XCD in every
    // workgroup instead.
    // Output tiles: (32-row tile, 32-token tile) pairs of a grid with token
    // tiles in z, else 32-row tiles.
    const int64_t tiles = (int64_t)gridDim.x * gridDim.z;
    const int64_t tile = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
    constexpr int VALS = MT * 16 * 64;  // floats per workgroup
    const int64_t slot = (int64_t)(PER * wave) * 64 + lane;
    const int64_t mine_off = ((int64_t)blockIdx.y * tiles + tile) * VALS + slot;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      __hip_atomic_store(a.partials + mine_off + k * 64, v[k], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();  // this wave's partials are visible at device scope
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // ... and every wave's
    asm volatile("" ::: "memory");
    if (threadIdx.x == 0)
      arrived_before = __hip_atomic_fetch_add(a.arrivals + tile, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived_before != gridDim.y - 1) return;  // uniform: one LDS value
    float sum[PER];
    const int64_t first = tile * VALS + slot;
    for (int s0 = 0; s0 < (int)gridDim.y; s0 += 4) {
      float p[4][PER];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sp = min(s0 + j, (int)gridDim.y - 1);  // past the last split: re-read, unused
#pragma unroll
        for (int k = 0; k < PER; ++k)
          p[j][k] = sp == (int)blockIdx.y
                        ? v[k]
                        : __hip_atomic_load(a.partials + first + sp * tiles * VALS + k * 64,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < PER; ++k)
          if (s0 + j < (int)gridDim.y) sum[k] = s0 + j == 0 ? p[j][k] : sum[k] + p[j][k];
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(a.arrivals + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = sum[k];
  }

#pragma unroll
  for (int k = 0; k < PER; ++k) {
    // Value v = PER w + k: tile m = v / 16, element r = v % 16 of a lane:
    // token 32 m + 8 (r / 4) + 4 h + r % 4, column lrow.
    const int val = PER * wave + k;
    const int tm = val >> 4, r = val & 15;
    const int64_t t = 32 * tm + 8 * (r >> 2) + 4 * h + (r & 3);
    if (t < a.n_tok && o < a.out_dim) a.out[t * a.out_dim + o] = v[k];
  }
}

// Every variant explicitly instantiated: without this the host side of the
// front end dropped some of them (the host stubs were referenced but never
// emitted).
template __global__ void skinny_kernel<1, ChunkCopies<1>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<1, ChunkCopies<2>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<2, ChunkCopies<1>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<2, ChunkCopies<2>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<1, DwordCopies<1>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<1, DwordCopies<2>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<2, DwordCopies<1>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<2, DwordCopies<2>, false>(const SkinnyArgs);
template __global__ void skinny_kernel<1, ChunkCopies<1>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<1, ChunkCopies<2>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<2, ChunkCopies<1>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<2, ChunkCopies<2>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<1, DwordCopies<1>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<1, DwordCopies<2>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<2, DwordCopies<1>, true>(const SkinnyArgs);
template __global__ void skinny_kernel<2, DwordCopies<2>, true>(const SkinnyArgs);

template <int MT, int R, bool STORE_S>
void launch_skinny_copies(bool wide, dim3 grid, const SkinnyArgs &a, hipStream_t s) {
  if (wide) {
    auto k = skinny_kernel<MT, ChunkCopies<R>, STORE_S>;
    hipLaunchKernelGGL(k, grid, dim3(64 * kWaves), 0, s, a);
  } else {
    auto k = skinny_kernel<MT, DwordCopies<R>, STORE_S>;
    hipLaunchKernelGGL(k, grid, dim3(64 * kWaves), 0, s, a);
  }
}

// Two steps in flight per wave when a wave has more than one step.
template <bool STORE_S>
void launch_skinny_variant(int mt, bool two_steps, bool wide, dim3 grid, const SkinnyArgs &a,
                           hipStream_t s) {
  if (mt == 2) {
    if (two_steps) launch_skinny_copies<2, 2, STORE_S>(wide, grid, a, s);
    else launch_skinny_copies<2, 1, STORE_S>(wide, grid, a, s);
  } else {
    if (two_steps) launch_skinny_copies<1, 2, STORE_S>(wide, grid, a, s);
    else launch_skinny_copies<1, 1, STORE_S>(wide, grid, a, s);
  }
}

int skinny_mt(int64_t n_tok) { return n_tok > 32 ? 2 : 1; }

}  // namespace

bool skinny_supported(int64_t in_dim, int64_t n_tok) {
  return in_dim > 0 && in_dim % 64 == 0 && (in_dim / 32) * kBlockBytes <= (1 << 24) && n_tok >= 1 &&
         n_tok <= kSkinnyWideMaxTokens;
}

// Above 64 tokens, graph replays on one box (tiled GEMM with its own split
// -> this kernel, one workgroup per (32-row tile, 32-token tile), one split):
// 4096 -> 2048 at 65 / 128 / 256 tokens 19.0 / 18.6 / 21.6 -> 8.4 / 9.0 /
// 15.9 us, 2048 -> 4096 18.0 / 18.9 / 21.5 -> 9.8 / 10.5 / 18.4, 4096 -> 1024
// 14.1 / 13.5 / 17.9 -> 7.7 / 7.9 / 8.7, 7168 -> 2048 20.4 / 19.7 / 24.2 ->
// 11.3 / 12.0 / 22.0.  The GEMM stays ahead where every token tile would
// re-read many weights (1024 -> 32768: 24.2 against 37.1 us at 65 tokens)
// and where long rows leave too few workgroups without a K split (32768 ->
// 1024: 37.4 against 43.6 us); at 512 tokens 4096 -> 2048 is even (28.9 /
// 29.3 us).  Hence rows of at most 128 block pairs and at most 128 row
// tiles, with one split (a K split measured slower on them, or even).  Long
// rows with few row tiles take two splits up to 128 tokens (partials per row
// and token tile): 32768 -> 1024 at 65 / 128 tokens 39.2 / 37.1 -> 26.6 /
// 29.5 us (4 and 8 splits slower; at 256 tokens the GEMM, 38.8 against
// 48.8 us); with more row tiles (16384 -> 2048, -> 4096) the GEMM leads.
bool skinny_many_tokens(int64_t in_dim, int64_t out_dim, int64_t n_tok) {
  if (n_tok <= kSkinnyMaxTokens || n_tok > kSkinnyWideMaxTokens) return false;
  const int64_t pairs = in_dim / 64, tiles = (out_dim + 31) / 32;
  if (pairs <= 128 && tiles <= 128) return true;
  return n_tok <= 128 && pairs >= 256 && tiles <= 32;
}

// Token tiles in separate workgroups: from 33 tokens, with 64 to 128 output
// tiles of 32 rows, one split and a workgroup per (row tile, token tile)
// instead of one per row tile with both token tiles (and, below 128 tiles,
// a K split with its in-launch completion).  Every weight row is then read
// by two workgroups.  Graph replays at 64 tokens, one box: 4096 -> 2048
// 8.63 -> 7.97 us (against split 4), 2048 -> 4096 8.14 -> 6.15 us (against
// 128 workgroups); 7168 -> 2048 the same (11.1 us); with 32 tiles (4096 ->
// 1024: 7.5 -> 7.65 us) too few workgroups remain, and with 1024 tiles
// (1024 -> 32768 at 40 tokens: 20.7 -> 25.8 us) the second read of the
// weights costs more than it saves.
//
// Below 64 row tiles, rows of up to 64 block pairs split their token tiles
// the same way and keep their K split (graph replays, one box, both tiles in
// one workgroup -> one per workgroup): 4096 -> 1024 at 64 tokens 7.59 ->
// 6.63 us, 4096 -> 512 at 48 7.25 -> 5.80, 4096 -> 256 at 64 6.65 -> 5.53,
// 1024 -> 520 at 40 4.93 -> 3.72; with the eight splits of longer rows it
// was slower (8192 -> 1024 at 48: 9.6 -> 12.3 us, 32768 -> 1024 at 64:
// 19.1 -> 22.9).
static bool skinny_tile_rows(int64_t in_dim, int64_t out_dim, int64_t n_tok) {
  const int64_t tiles = (out_dim + 31) / 32;
  return n_tok > 32 && n_tok <= kSkinnyMaxTokens && tiles <= 128 &&
         (tiles >= 64 || in_dim / 64 <= 64);
}
static bool skinny_token_split(int64_t out_dim, int64_t n_tok) {
  const int64_t tiles = (out_dim + 31) / 32;
  return n_tok > 32 && tiles >= 64 && tiles <= 128;
}

// Splits.  The split-K completion (partials out, an arrival counter, the
// last arrival's sum) puts about 1.5 us of serial memory round trips on the
// critical path, so a split has to buy more than that: with 128 or more
// tiles half the chip is already busy and one split is fastest; below that,
// enough workgroups for the chip (about 256), at least 16 block pairs per
// split (a full step for each of the eight waves), at most 16 splits; none
// where the token tiles go to separate workgroups.
int skinny_auto_split(int64_t in_dim, int64_t out_dim, int64_t n_tok) {
  if (n_tok > kSkinnyMaxTokens) return in_dim / 64 > 128 ? 2 : 1;
  if (skinny_token_split(out_dim, n_tok)) return 1;
  const int64_t tiles = (out_dim + 31) / 32;
  const int64_t pairs = in_dim / 64;
  if (tiles >= 128) return 1;
  int64_t split = (256 + tiles - 1) / tiles;
  split = std::min<int64_t>(split, std::max<int64_t>(pairs / (kStepPairs * kWaves), 1));
  split = std::min<int64_t>(split, 16);
  return (int)std::max<int64_t>(split, 1);
}

// Workspace of a split-K launch: the arrival counters (zero between calls)
// in the first kWsCounterBytes, then the partials, MT * 4 KiB per workgroup.
// (4 KiB per 32-token tile and workgroup: with token tiles in workgroups of
// their own one each, else MT each -- the same bytes.)
size_t skinny_workspace_bytes(int64_t out_dim, int64_t n_tok, int split) {
  if (split <= 1) return 0;
  const int64_t tiles = (out_dim + 31) / 32;
  return kWsCounterBytes + (size_t)split * (size_t)tiles * (size_t)((n_tok + 31) / 32) * 4096;
}

// One arrival counter per output tile: per 32-row tile, and per token tile
// too where those have workgroups of their own.
bool skinny_split_ok(int64_t in_dim, int64_t out_dim, int64_t n_tok, int split) {
  const bool own = n_tok > kSkinnyMaxTokens || skinny_tile_rows(in_dim, out_dim, n_tok);
  const int64_t tiles = (out_dim + 31) / 32 * (own ? (n_tok + 31) / 32 : 1);
  return split <= 1 || tiles <= (int64_t)(kWsCounterBytes / 4);
}

hipError_t launch_skinny(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                         int64_t out_dim, const void *x_q, int64_t n_tok, int split,
                         void *workspace, hipStream_t s) {
  SkinnyArgs a{};
  a.out = out;
  a.blocksums = blocksums;
  a.n_pairs = (int32_t)(in_dim / 64);
  // Splits are whole steps (the last one may be short).
  const int pps = ((a.n_pairs + split - 1) / split + kStepPairs - 1) / kStepPairs * kStepPairs;
  const int n_split = (a.n_pairs + pps - 1) / pps;
  if (n_split > 1) {
    a.arrivals = static_cast<uint32_t *>(workspace);
    a.partials = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + kWsCounterBytes);
  }
  a.w = static_cast<const uint8_t *>(w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.out_dim = out_dim;
  a.n_tok = n_tok;
  a.row_bytes = (in_dim / 32) * 34;
  a.pairs_per_split = pps;
  const bool tsplit = n_tok > kSkinnyMaxTokens || skinny_tile_rows(in_dim, out_dim, n_tok);
  // Above kSkinnyMaxTokens with one split, two token tiles per workgroup
  // where that still leaves >= 192 workgroups (row tiles x 32-token tiles >=
  // 384): the weights are read half as often.  Graph replays, one box, one
  // tile -> two per workgroup: 2048 -> 4096 at 65 / 128 / 256 tokens 10.0 /
  // 10.5 / 18.6 -> 8.7 / 9.0 / 15.6 us, 4096 -> 2048 at 192 / 256 14.9 /
  // 15.7 -> 13.0 / 13.5, 8192 -> 2048 at 256 24.3 -> 23.0; with fewer tiles
  // slower (4096 -> 2048 at 128: 9.0 -> 12.6, 4096 -> 1024: 8.0 -> 11.8).
  const int64_t rtiles = (out_dim + 31) / 32, ttiles = (n_tok + 31) / 32;
  const int tz = n_tok > kSkinnyMaxTokens && n_split == 1 && rtiles * ttiles >= 384 ? 2 : 1;
  const dim3 grid((uint32_t)rtiles, (uint32_t)n_split,
                  tsplit ? (uint32_t)((ttiles + tz - 1) / tz) : 1u);
  // 16-byte copies need rows of 8k blocks and 16-aligned bases.
  const bool wide = in_dim % 256 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(x_q) & 15) == 0;
  const int mt = tsplit ? tz : skinny_mt(n_tok);
  const bool two_steps = pps > kStepPairs * (kWaves / mt);
  if (blocksums) launch_skinny_variant<true>(mt, two_steps, wide, grid, a, s);
  else launch_skinny_variant<false>(mt, two_steps, wide, grid, a, s);
  return hipGetLastError();
}

}  // namespace q8
