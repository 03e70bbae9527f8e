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
//     and reduced through LDS.  Lane partial sums are reduced with DPP adds
//     in a fixed order (group_sum), so results are deterministic.
//   * Each workgroup issues all of its weight loads before it needs x, so a
//     lane has RG * CPW pairs (68 bytes each) in flight.  x comes from LDS:
//     staged there by direct copies (StagedX: grouped launches and two or
//     more tokens), or quantized there from fp32 by the workgroup itself
//     (LdsX: the list launch); single-token launches read it per wave from
//     global memory (GlobalX), rows of 64 or more pairs as coalesced chunks
//     issued ahead of the weights.
#include <algorithm>
#include <type_traits>

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
  const uint8_t *const *expert_w2;  // paired: second table (up projections)
  float clamp;                      // paired: SwiGLU limit, <= 0 for none
};

// SwiGLU of one output ("Part 3: 模型架构", section 4): the optional 2-bit
// path limits (gate from above, up to +-clamp; NaN passes), then
// silu(g) * u with silu(g) = g / (1 + exp(-g)).
__device__ __forceinline__ float swiglu_one(float g, float u, float clamp) {
  if (clamp > 0.0f) {
    if (g > clamp) g = clamp;
    if (u > clamp) u = clamp;
    if (u < -clamp) u = -clamp;
  }
  return (g / (1.0f + expf(-g))) * u;
}

// Where a workgroup reads its x_q rows from.
//
// GlobalX: the caller's x_q in device memory (L2-resident after first touch).
struct GlobalX {
  const uint8_t *x_q;
  int64_t row_bytes;
  __device__ __forceinline__ void prefetch() {}
  __device__ __forceinline__ void publish() {}
  __device__ __forceinline__ void advance(int64_t) {}
  __device__ __forceinline__ void load(int64_t, int64_t xrow, int64_t pair,
                                       uint32_t (&d)[kPairDwords]) const {
    load_pair(x_q + xrow * row_bytes + pair * kPairBytes, d);
  }
};

// The same x source for the single-token matvec kernel, whose body loads
// item 0's x pairs before the weights (attn_q_b separate matvec 7.78 -> 7.65
// us on one box).  The list kernel keeps GlobalX, which loads early only in
// rows of 64 or more pairs (coalesced chunk loads, decode5 15.3 -> 14.4 us):
// there lane-strided early loads of the short rows cost decode5 15.0 -> 16.1 us.
struct GlobalXFirst : GlobalX {};

// StagedX: the x_q rows of the workgroup's items, XT at a time, copied into
// LDS by direct global->LDS dword copies (64 consecutive dwords per wave
// instruction; wave w copies the rows w, w+4, ...).  The copies of the first
// XT rows are issued before the weight loads, so their latency hides under
// the weight stream, and every wave then reads its pairs from LDS instead of
// issuing per-item global loads.  With more than XT items two buffers
// alternate: the next XT rows are copied while the current ones are used.
// ROW_DW = dwords of one x_q row; rows sit at a stride rounded up to 64
// dwords, the lanes past a row's end re-read its last dword into the padding.
template <int ROW_DW, int XT>
struct StagedX {
  static constexpr bool kStaged = true;  // weights, if coalesced, use one region per wave
  static constexpr int STRIDE = (ROW_DW + 63) / 64 * 64;
  static constexpr int NI = STRIDE / 64;
  static constexpr int BUF = XT * STRIDE;  // dwords per buffer
  uint32_t *lds;             // 2 * BUF dwords
  const uint8_t *x_q;
  int64_t row_bytes;
  const int32_t *items;      // grouped: pair ids; null: item i is x row i
  int64_t n_items;
  uint32_t n_used;
  int32_t x_rows;
  int64_t base = 0;          // first item of the rows being read
  int cur = 0;               // buffer holding them

  // Issue the copies of items [first, first + XT) into buffer `buf`.
  __device__ __forceinline__ void stage(int64_t first, int buf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int rows = (int)min((int64_t)XT, n_items - first);
    uint32_t *dst = lds + buf * BUF;
    for (int t = wave; t < rows; t += 4) {
      int64_t xrow = first + t;
      if (items) {
        const uint32_t pr = (uint32_t)items[first + t];
        xrow = x_rows ? pr : pr / n_used;
      }
      const uint8_t *src = x_q + xrow * row_bytes;
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int d = min(64 * k + lane, ROW_DW - 1);
        __builtin_amdgcn_global_load_lds(src + 4 * d, dst + t * STRIDE + 64 * k, 4, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void prefetch() { stage(0, 0); }
  // Wait for this wave's copies (and the weights) and then every wave's;
  // then start the next rows, if any, into the other buffer.
  __device__ __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (base + XT < n_items) stage(base + XT, cur ^ 1);
  }
  // Called at the top of item `it` (uniform across the workgroup).  The
  // barrier inside publish() also means every wave is done with the rows
  // before, so their buffer can take the rows after next.
  __device__ __forceinline__ void advance(int64_t it) {
    if (it - base == XT) {
      base = it;
      cur ^= 1;
      publish();
    }
  }
  __device__ __forceinline__ void load(int64_t it, int64_t, int64_t pair,
                                       uint32_t (&d)[kPairDwords]) const {
    const uint32_t *b = lds + cur * BUF + (int)(it - base) * STRIDE + (int)pair * kPairDwords;
#pragma unroll
    for (int i = 0; i < kPairDwords; ++i) d[i] = b[i];
  }
};

// x rows per staging buffer: as many as fit in about 20 KB of LDS, 1 to 16;
// with SMALL (the grouped kernels, which also stage their weights through
// 17 KB of LDS) about 8.5 KB, so that four workgroups fit a CU.
template <int LPR, int WPR, int CPW, bool SMALL = false>
struct StagedShape {
  static constexpr int ROW_DW = kPairDwords * (LPR < 64 ? LPR : 64 * WPR * CPW);
  static constexpr int STRIDE = (ROW_DW + 63) / 64 * 64;
  static constexpr int XT_RAW = (SMALL ? 8704 : 20480) / (4 * STRIDE);
  static constexpr int XT = XT_RAW < 1 ? 1 : (XT_RAW > 16 ? 16 : XT_RAW);
  using X = StagedX<ROW_DW, XT>;
};

// LdsX: fp32 activation rows quantized by the workgroup itself into LDS, so a
// decode projection needs no separate quantizer launch.  Up to kFusePairs
// pairs (n_tok * in_dim <= 4096 values) are quantized in one pass, 4 lanes per
// pair.  The fp32 loads are issued before the weight loads (prefetch) and
// consumed after them (publish), so the quantization hides under the weight
// stream.  One workgroup per item (the writer) also stores the rows to
// global x_q.
constexpr int kFusePairs = 64;  // 256 threads / 4 lanes per pair

struct LdsX {
  uint32_t *lds;          // kFusePairs * 17 dwords
  const float *x;         // fp32 [n_tok][in_dim]
  uint8_t *x_q_out;       // written when non-null (writer workgroup only)
  int log2_ppr;           // pairs per row = 1 << log2_ppr (a power of two here)
  int n_pairs;            // n_tok << log2_ppr, 1 ..= kFusePairs
  int64_t in_dim;
  float4 v[4];

  // Every thread loads (pairs past the end re-read the last pair), so the
  // number of loads in flight is the same on every path and the wait before
  // publish leaves the weight loads outstanding.
  __device__ __forceinline__ void prefetch() {
    const int j = threadIdx.x & 3;
    const int p = min((int)(threadIdx.x >> 2), n_pairs - 1);
    const int row = p >> log2_ppr;
    const int pp = p - (row << log2_ppr);
    const float4 *src = reinterpret_cast<const float4 *>(x + row * in_dim + pp * 64 + j * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = src[k];
  }
  __device__ __forceinline__ void publish() {
    const int j = threadIdx.x & 3;
    const int p = threadIdx.x >> 2;
    uint32_t out[5];
    quantize_pair4(v, j, out);
    if (p < n_pairs) {
      const int first = pair4_first(j), count = pair4_count(j);
      uint32_t *l = lds + p * kPairDwords + first;
#pragma unroll
      for (int k = 0; k < 5; ++k)
        if (k < count) l[k] = out[k];
      if (x_q_out) {
        uint32_t *g = reinterpret_cast<uint32_t *>(x_q_out + p * kPairBytes) + first;
#pragma unroll
        for (int k = 0; k < 5; ++k)
          if (k < count) g[k] = out[k];
      }
    }
    __syncthreads();
  }
  __device__ __forceinline__ void advance(int64_t) {}
  __device__ __forceinline__ void load(int64_t, int64_t xrow, int64_t pair,
                                       uint32_t (&d)[kPairDwords]) const {
    const uint32_t *b = lds + (((int)xrow << log2_ppr) + (int)pair) * kPairDwords;
#pragma unroll
    for (int i = 0; i < kPairDwords; ++i) d[i] = b[i];
  }
};

// LdsXWave: the one-item fused kernel when x has at most 16 pairs, which is
// one wave's share of the quantizer: every wave quantizes the whole row into
// its own 16-pair quarter of the buffer (lds points there), so no workgroup
// barrier stands between the x loads and the dots.  The x_q copy is written
// by wave 0 of the writer workgroup (x_q_out is null on the other waves).
struct LdsXWave : LdsX {
  __device__ __forceinline__ void prefetch() {
    const int lane = threadIdx.x & 63;
    const int j = lane & 3;
    const int p = min(lane >> 2, n_pairs - 1);
    const int row = p >> log2_ppr;
    const int pp = p - (row << log2_ppr);
    const float4 *src = reinterpret_cast<const float4 *>(x + row * in_dim + pp * 64 + j * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = src[k];
  }
  __device__ __forceinline__ void publish() {
    const int lane = threadIdx.x & 63;
    const int j = lane & 3;
    const int p = lane >> 2;
    uint32_t out[5];
    quantize_pair4(v, j, out);
    if (p < n_pairs) {
      const int first = pair4_first(j), count = pair4_count(j);
      uint32_t *l = lds + p * kPairDwords + first;
#pragma unroll
      for (int k = 0; k < 5; ++k)
        if (k < count) l[k] = out[k];
      if (x_q_out) {
        uint32_t *g = reinterpret_cast<uint32_t *>(x_q_out + p * kPairBytes) + first;
#pragma unroll
        for (int k = 0; k < 5; ++k)
          if (k < count) g[k] = out[k];
      }
    }
    // LDS operations of one wave run in order: the wave's own reads of its
    // quarter follow these writes without a workgroup barrier.
    __builtin_amdgcn_wave_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
};
constexpr int kWaveXPairs = 16;

// Coalesced weight staging (COAL bodies): a wave's 64 pairs are 4352 bytes =
// 1088 dwords; at most two such regions per wave, four waves.
constexpr int kCoalDwords = 64 * kPairDwords;
constexpr int kCoalRegions = 2;
constexpr int kCoalLdsDwords = 4 * kCoalRegions * kCoalDwords;
// Bodies that stage their weights this way: rows of at least four pairs, so
// that the matrix ends on a 16-byte boundary of every region (a 16-byte load
// is then wholly inside or wholly past it), and at most two (row group, chunk)
// regions per wave.  The list kernel's two-row-group body of 32768-wide rows
// (four chunks per wave) also takes it, its chunks passing through the two
// regions in turn: 8.6 -> 8.2 us for that row as a one-item list, where the
// same body in the single-token kernel gained nothing.
constexpr bool coal_body(int lpr, int rg, int cpw) { return rg * cpw <= kCoalRegions && lpr >= 4; }
constexpr bool coal_list_body(int lpr, int wpr, int rg, int cpw) {
  return coal_body(lpr, rg, cpw) || (lpr == 64 && wpr == 4 && cpw == 2 && rg == 2);
}

// One wave's 64-pair chunk (4352 contiguous bytes) from coalesced registers
// to the pair layout: lane l holds the chunk's 16-byte pieces l, l + 64,
// l + 128, l + 192 and its dword 1024 + l; they are written to the wave's LDS
// region `reg` (kCoalDwords dwords) in byte order, and lane l reads back pair
// l at dword 17 l.  LDS operations of one wave run in order; the fences keep
// the compiler from moving them past each other or past the region's next use.
__device__ __forceinline__ void coal_to_pair(uint32_t *reg, const u32x4_a4 (&piece)[4],
                                             uint32_t tail, int lane,
                                             uint32_t (&d)[kPairDwords]) {
  u32x4_a4 *dst = reinterpret_cast<u32x4_a4 *>(reg);
#pragma unroll
  for (int k = 0; k < 4; ++k) dst[64 * k + lane] = piece[k];
  reg[1024 + lane] = tail;
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int i = 0; i < kPairDwords; ++i) d[i] = reg[kPairDwords * lane + i];
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One workgroup tile of the matvec: TILE_ROWS weight rows against n_items x
// rows.  `tile` is the tile index within the matrix; `w` and `items` the
// (possibly per-expert) weights and item list.
// PAIR: two weight matrices of the same shape (w and w2, the gate and up
// projections) against the same x rows; the stored output is their SwiGLU.
//
// COAL: the weight rows come in through whole coalesced 16-byte non-temporal
// loads, passed through a per-wave LDS region from which each lane reads its
// pair, instead of per-lane 68-byte pair loads (wst: kCoalDwords dwords per
// region, (RG * CPW) regions per wave).  Single-token bodies of rows of 64 or
// more pairs also pass item 0's x chunks through the wave's first region
// (without COAL, wst holds one region per wave for that).
template <int LPR, int WPR, int CPW, int RG, bool GROUPED, bool STORE_S, class XS,
          bool PAIR = false, bool COAL = false>
__device__ __forceinline__ void matvec_body(const MatvecArgs &a, int64_t tile, const uint8_t *w,
                                            const int32_t *items, int64_t n_items, XS &xs,
                                            const uint8_t *w2 = nullptr, uint32_t *wst = nullptr) {
  constexpr int RPW = 64 / LPR;                   // rows per wave row-group
  constexpr int ROWS_PER_SLOT = RG * RPW;
  constexpr int TILE_ROWS = (4 / WPR) * ROWS_PER_SLOT;
  constexpr int NM = PAIR ? 2 : 1;                // weight matrices
  __shared__ float red[4][NM][RG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = wave / WPR;
  const int part = wave % WPR;

  const int64_t row0 = tile * TILE_ROWS + slot * ROWS_PER_SLOT + lane / LPR;
  int64_t pair_of[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
    pair_of[c] = (LPR < 64) ? (int64_t)(lane % LPR) : (int64_t)(c * WPR + part) * 64 + lane;

  // A global x row is otherwise loaded only once the weights have landed:
  // item 0's pairs are loaded first here, so their latency overlaps the
  // weight stream, with GlobalXFirst (the single-token matvec kernel) and
  // for the list kernel's rows of 64 or more pairs.  In those rows a wave's x
  // pairs are one contiguous chunk: they come in through coalesced 16-byte
  // loads (8 cache lines per instruction instead of 34 for lane-strided pair
  // loads), turned into the pair layout through LDS once the weight loads
  // are issued.  Callers launch with at least one item, and pair_of stays
  // inside the row.
  constexpr bool XPRE =
      (std::is_same_v<XS, GlobalXFirst> || (std::is_same_v<XS, GlobalX> && LPR == 64 && COAL)) &&
      !GROUPED && CPW <= 2;
  constexpr bool XCOAL = XPRE && LPR == 64;
  uint32_t xpre[CPW][kPairDwords];
  u32x4_a4 xpiece[XCOAL ? CPW : 1][4];
  uint32_t xtail[XCOAL ? CPW : 1];
  if constexpr (XCOAL) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint8_t *src = xs.x_q + (int64_t)(c * WPR + part) * 64 * kPairBytes;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        xpiece[c][k] = *reinterpret_cast<const u32x4_a4 *>(src + 16 * (64 * k + lane));
      xtail[c] = *reinterpret_cast<const uint32_t *>(src + 4096 + 4 * lane);
    }
  } else if constexpr (XPRE) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) xs.load(0, 0, pair_of[c], xpre[c]);
  }
  auto x_from_pieces = [&]() {
    if constexpr (XCOAL) {
      const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
      uint32_t *reg = wst + wave_u * (COAL ? kCoalRegions : 1) * kCoalDwords;
#pragma unroll
      for (int c = 0; c < CPW; ++c) coal_to_pair(reg, xpiece[c], xtail[c], lane, xpre[c]);
    }
  };
  // Every lane issues the same loads (rows past the end re-read the last row,
  // whose results are never stored), so the wait for the prefetched x rows
  // can leave the weight loads in flight.
  xs.prefetch();
  uint32_t wr[NM][RG][CPW][kPairDwords];
  if constexpr (COAL) {
    static_assert(GROUPED || requires { XS::kStaged; } || (!PAIR && coal_list_body(LPR, WPR, RG, CPW)),
                  "coalesced weight staging");
    // A wave's 64 pairs of one (matrix, row group, chunk) are 4352 contiguous
    // bytes: RPW whole rows, or one 64-pair chunk of a row.  Lane l loads
    // 16-byte chunks l, l + 64, l + 128, l + 192 and then dword 1024 + l, so
    // every lane issues the same five loads.  Loads of a region that reaches
    // past the last row are clamped to the matrix's last bytes: what they
    // bring feeds only outputs that are not stored, and nothing is read
    // outside the matrix.  The loads go to registers (not direct to LDS) and
    // nothing branches between them and the earlier x loads, so waiting for x
    // does not wait for the weights.  The chunks pass through the wave's
    // NREG regions in turn (one per wave where the x rows are staged in LDS
    // too); a region is rewritten only after the
    // wave's reads of it.  The grouped kernels' weight bases come from the
    // device table, so their loads go through global pointers explicitly.
    constexpr int NREG = (GROUPED || requires { XS::kStaged; }) ? 1 : kCoalRegions;
    const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t rb0 = tile * TILE_ROWS + (wave_u / WPR) * ROWS_PER_SLOT;
    uint32_t *mine = wst + wave_u * (NREG * kCoalDwords);
    u32x4_a4 ch[NM][RG][CPW][4];
    uint32_t tail[NM][RG][CPW];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint8_t *wm = m == 0 ? w : w2;
      const uint8_t *wend = wm + a.out_dim * a.row_bytes;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          const int64_t chunk0 = LPR < 64 ? 0 : (int64_t)(c * WPR + (wave_u % WPR)) * 64;
          const uint8_t *src = wm + (rb0 + g * RPW) * a.row_bytes + chunk0 * kPairBytes;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint8_t *q = src + 16 * (64 * k + lane);
            q = q < wend - 16 ? q : wend - 16;
            if constexpr (GROUPED)
              ch[m][g][c][k] = __builtin_nontemporal_load((global_u32x4_a4 *)q);
            else
              ch[m][g][c][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4 *>(q));
          }
          const uint8_t *q = src + 4096 + 4 * lane;
          q = q < wend - 4 ? q : wend - 4;
          if constexpr (GROUPED)
            tail[m][g][c] = __builtin_nontemporal_load((global_u32 *)q);
          else
            tail[m][g][c] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(q));
        }
      }
    }
    xs.publish();
    x_from_pieces();
    // Through this wave's LDS regions: write the region back in byte order,
    // then lane l reads its pair at byte 68 l.  LDS operations of one wave
    // run in order, so no barrier is needed; the fences keep the compiler
    // from moving a region's next writes above its reads.
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          uint32_t *reg = mine + (((m * RG + g) * CPW + c) % NREG) * kCoalDwords;
          u32x4_a4 *dst = reinterpret_cast<u32x4_a4 *>(reg);
#pragma unroll
          for (int k = 0; k < 4; ++k) dst[64 * k + lane] = ch[m][g][c][k];
          reg[1024 + lane] = tail[m][g][c];
          __builtin_amdgcn_wave_barrier();
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
          for (int i = 0; i < kPairDwords; ++i) wr[m][g][c][i] = reg[kPairDwords * lane + i];
        }
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int64_t row = row0 + g * RPW;
      const int64_t lrow = row < a.out_dim ? row : a.out_dim - 1;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        if constexpr (GROUPED) {
          load_pair_global(w + lrow * a.row_bytes + pair_of[c] * kPairBytes, wr[0][g][c]);
          if constexpr (PAIR)
            load_pair_global(w2 + lrow * a.row_bytes + pair_of[c] * kPairBytes, wr[NM - 1][g][c]);
        } else {
          load_pair(w + lrow * a.row_bytes + pair_of[c] * kPairBytes, wr[0][g][c]);
        }
      }
    }
    xs.publish();
    x_from_pieces();
  }

  for (int64_t it = 0; it < n_items; ++it) {
    xs.advance(it);
    int64_t xrow = it, orow = it;
    if constexpr (GROUPED) {
      const int64_t pr = items[it];
      orow = pr;
      xrow = a.x_rows ? pr : pr / a.n_used;
    }
    float acc[NM][RG];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int g = 0; g < RG; ++g) acc[m][g] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      uint32_t xr[kPairDwords];
      if constexpr (XPRE) {
        if (it == 0) {
#pragma unroll
          for (int i = 0; i < kPairDwords; ++i) xr[i] = xpre[c][i];
        } else {
          xs.load(it, xrow, pair_of[c], xr);
        }
      } else {
        xs.load(it, xrow, pair_of[c], xr);
      }
      const float dxA = f16_bits_to_f32(xr[0]);
      const float dxB = f16_bits_to_f32(xr[8] >> 16);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          int sA, sB;
          pair_dots(wr[m][g][c], xr, sA, sB);
          const float scA = f16_bits_to_f32(wr[m][g][c][0]) * dxA;
          const float scB = f16_bits_to_f32(wr[m][g][c][8] >> 16) * dxB;
          acc[m][g] += scA * (float)sA;
          acc[m][g] += scB * (float)sB;
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
    }
    // Grouped bodies with four sums per lane (RG row groups x NM matrices)
    // of 32- or 64-lane rows reduce them together, in a fixed order: two
    // transposing steps across the quad (lane i ^ 1, then i ^ 2; each lane
    // keeps half of its values and adds its partner's copy of them), so lane
    // i ends with sum j = 2 (i & 1) + ((i >> 1) & 1) of its quad; then the
    // row (DPP rotations by 4 and 8) and the other 16-lane row (and for 64-lane
    // rows the other half) by LDS-crossbar permutes.  About 15 instructions
    // for the four sums against 24 dependent DPP adds one sum at a time:
    // moe gate projection 351-353 -> 334-339 us on one box.
    constexpr bool QUAD = GROUPED && WPR == 1 && RG * NM == 4 && (LPR == 32 || LPR == 64);
    if constexpr (QUAD) {
      float v[4];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int g = 0; g < RG; ++g) v[m * RG + g] = acc[m][g];
      const bool b0 = lane & 1, b1 = (lane >> 1) & 1;
      const float r0 = (b0 ? v[2] : v[0]) + dpp_f32<kDppXor1>(b0 ? v[0] : v[2]);
      const float r1 = (b0 ? v[3] : v[1]) + dpp_f32<kDppXor1>(b0 ? v[1] : v[3]);
      float t = (b1 ? r1 : r0) + dpp_f32<kDppXor2>(b1 ? r0 : r1);
      t += dpp_f32<kDppRowRor4>(t);
      t += dpp_f32<kDppRowRor8>(t);
      t += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (lane ^ 16), __builtin_bit_cast(int, t)));
      if constexpr (LPR == 64)
        t += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (lane ^ 32), __builtin_bit_cast(int, t)));
      // Lane q < 4 of each row holds sum j = 2 (q & 1) + (q >> 1); a pair
      // body's gate sums (j = g) sit in lanes 0 and 2, each with its up sum
      // (j = RG + g) in the next lane.
      const int q = lane & (LPR - 1);
      const float up = PAIR ? dpp_f32<kDppXor1>(t) : 0.0f;
      if (q < 4 && (!PAIR || (q & 1) == 0)) {
        const int j = 2 * (q & 1) + (q >> 1);
        const int64_t row = row0 + j * RPW;
        float val = t;
        if constexpr (PAIR) val = swiglu_one(t, up, a.clamp);
        if (row < a.out_dim) a.out[orow * a.out_dim + row] = val;
      }
      continue;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        acc[m][g] = group_sum<LPR>(acc[m][g]);
      }
    }
    if constexpr (WPR > 1) {
      if (group_sum_lane<64>(lane)) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int g = 0; g < RG; ++g) red[wave][m][g] = acc[m][g];
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            float v = red[wave][m][g];
#pragma unroll
            for (int p = 1; p < WPR; ++p) v += red[wave + p][m][g];
            acc[m][g] = v;
          }
        }
      }
      __syncthreads();
    }
    if (part == 0 && group_sum_lane<LPR>(lane)) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int64_t row = row0 + g * RPW;
        float v = acc[0][g];
        if constexpr (PAIR) v = swiglu_one(acc[0][g], acc[NM - 1][g], a.clamp);
        if (row < a.out_dim) a.out[orow * a.out_dim + row] = v;
      }
    }
  }
}

// STAGED: x rows staged in LDS (StagedX); otherwise read from global memory
// by every wave (GlobalX), which is cheaper for a single token row.
template <int LPR, int WPR, int CPW, int RG, bool GROUPED, bool STORE_S, bool STAGED>
__global__ __launch_bounds__(256) void matvec_kernel(const MatvecArgs a) {
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
  if constexpr (STAGED) {
    // Grouped launches stage their weights coalesced too, through one LDS
    // region per wave, beside a smaller x buffer (four workgroups per CU):
    // moe gate projection 335 -> 305 us, down 328 -> 302 us against per-lane
    // pair loads (one box).  Plain staged launches (2..11 tokens) do so for
    // 32768-wide rows, whose x buffer holds one row either way: 32768 -> 1024
    // at 2 / 4 / 8 tokens 13.4 / 17.5 / 25.6 -> 12.6 / 16.5 / 24.7 us; at
    // in_dim 1024 and 4096 it measured slower from four tokens on.
    constexpr bool GCOAL = LPR >= 4 && (GROUPED || (LPR == 64 && WPR == 4 && CPW == 2));
    using SX = typename StagedShape<LPR, WPR, CPW, GROUPED && GCOAL>::X;
    __shared__ __attribute__((aligned(16))) uint32_t xbuf[2 * SX::BUF];
    SX xs{xbuf, a.x_q, a.row_bytes, items, n_items, (uint32_t)a.n_used, a.x_rows};
    if constexpr (GCOAL) {
      __shared__ __attribute__((aligned(16))) uint32_t wst[4 * kCoalDwords];
      matvec_body<LPR, WPR, CPW, RG, GROUPED, STORE_S, SX, false, true>(a, blockIdx.x, w, items,
                                                                       n_items, xs, nullptr, wst);
    } else {
      matvec_body<LPR, WPR, CPW, RG, GROUPED, STORE_S>(a, blockIdx.x, w, items, n_items, xs);
    }
  } else if constexpr (!GROUPED && coal_body(LPR, RG, CPW)) {
    __shared__ __attribute__((aligned(16))) uint32_t wst[kCoalLdsDwords];
    GlobalXFirst xs{{a.x_q, a.row_bytes}};
    matvec_body<LPR, WPR, CPW, RG, GROUPED, STORE_S, GlobalXFirst, false, true>(
        a, blockIdx.x, w, items, n_items, xs, nullptr, wst);
  } else {
    // one LDS region per wave for the x chunks of rows of 64 or more pairs
    __shared__ __attribute__((aligned(16))) uint32_t xst[LPR == 64 ? 4 * kCoalDwords : 1];
    GlobalXFirst xs{{a.x_q, a.row_bytes}};
    matvec_body<LPR, WPR, CPW, RG, GROUPED, STORE_S>(a, blockIdx.x, w, items, n_items, xs,
                                                     nullptr, xst);
  }
}

// Grouped gate+up pair with the SwiGLU epilogue (one x load feeds both
// matrices; the mid row is written once).
template <int LPR, int WPR, int CPW, int RG>
__global__ __launch_bounds__(256) void matvec_pair_kernel(const MatvecArgs a) {
  const int e = blockIdx.y;
  const int64_t n_items = a.counts[e];
  if (n_items == 0) return;  // uniform across the workgroup
  constexpr bool GCOAL = LPR >= 4;  // weights staged coalesced, as in the grouped kernel
  using SX = typename StagedShape<LPR, WPR, CPW, GCOAL>::X;
  __shared__ __attribute__((aligned(16))) uint32_t xbuf[2 * SX::BUF];
  const int32_t *items = a.pairs + a.offsets[e];
  SX xs{xbuf, a.x_q, a.row_bytes, items, n_items, (uint32_t)a.n_used, a.x_rows};
  if constexpr (GCOAL) {
    __shared__ __attribute__((aligned(16))) uint32_t wst[4 * kCoalDwords];
    matvec_body<LPR, WPR, CPW, RG, true, false, SX, true, true>(a, blockIdx.x, a.expert_w[e], items,
                                                                n_items, xs, a.expert_w2[e], wst);
  } else {
    matvec_body<LPR, WPR, CPW, RG, true, false, SX, true>(a, blockIdx.x, a.expert_w[e], items,
                                                          n_items, xs, a.expert_w2[e]);
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

template <int LPR, int WPR, int CPW, bool GROUPED, bool STORE_S, bool STAGED>
MatvecFn pick_rg_x(int rg) {
  if constexpr (CPW == 1 || (CPW == 2 && WPR == 4)) {
    if (rg >= 4) return matvec_kernel<LPR, WPR, CPW, 4, GROUPED, STORE_S, STAGED>;
  }
  if constexpr (CPW <= 2) {
    if (rg >= 2) return matvec_kernel<LPR, WPR, CPW, 2, GROUPED, STORE_S, STAGED>;
  }
  return matvec_kernel<LPR, WPR, CPW, 1, GROUPED, STORE_S, STAGED>;
}

// Grouped launches always stage their x rows; plain ones stage them from two
// tokens up (the `staged` argument).
template <int LPR, int WPR, int CPW, bool GROUPED, bool STORE_S>
MatvecFn pick_rg(int rg, bool staged) {
  if constexpr (GROUPED) {
    return pick_rg_x<LPR, WPR, CPW, true, STORE_S, true>(rg);
  } else {
    return staged ? pick_rg_x<LPR, WPR, CPW, false, STORE_S, true>(rg)
                  : pick_rg_x<LPR, WPR, CPW, false, STORE_S, false>(rg);
  }
}

template <bool GROUPED, bool STORE_S>
MatvecFn pick_kernel(const MatvecShape &sh, int rg, bool staged) {
  switch (sh.lanes_per_row) {
    case 1: return pick_rg<1, 1, 1, GROUPED, STORE_S>(rg, staged);
    case 2: return pick_rg<2, 1, 1, GROUPED, STORE_S>(rg, staged);
    case 4: return pick_rg<4, 1, 1, GROUPED, STORE_S>(rg, staged);
    case 8: return pick_rg<8, 1, 1, GROUPED, STORE_S>(rg, staged);
    case 16: return pick_rg<16, 1, 1, GROUPED, STORE_S>(rg, staged);
    case 32: return pick_rg<32, 1, 1, GROUPED, STORE_S>(rg, staged);
    default: break;
  }
  const int key = sh.waves_per_row * 10 + sh.chunks_per_wave;
  switch (key) {
    case 11: return pick_rg<64, 1, 1, GROUPED, STORE_S>(rg, staged);
    case 13: return pick_rg<64, 1, 3, GROUPED, STORE_S>(rg, staged);
    case 21: return pick_rg<64, 2, 1, GROUPED, STORE_S>(rg, staged);
    case 22: return pick_rg<64, 2, 2, GROUPED, STORE_S>(rg, staged);
    case 41: return pick_rg<64, 4, 1, GROUPED, STORE_S>(rg, staged);
    case 42: return pick_rg<64, 4, 2, GROUPED, STORE_S>(rg, staged);
    case 43: return pick_rg<64, 4, 3, GROUPED, STORE_S>(rg, staged);
    case 44: return pick_rg<64, 4, 4, GROUPED, STORE_S>(rg, staged);
    default: return nullptr;
  }
}

int max_rg(const MatvecShape &sh) {
  if (sh.chunks_per_wave == 1 || (sh.chunks_per_wave == 2 && sh.waves_per_row == 4)) return 4;
  return sh.chunks_per_wave == 2 ? 2 : 1;
}

int64_t tile_rows(const MatvecShape &sh, int rg) {
  return (int64_t)(4 / sh.waves_per_row) * rg * (64 / sh.lanes_per_row);
}

// Fewest rows per workgroup that still leaves >= 1024 workgroups (4 per CU);
// small matrices get single-row-group tiles so all 256 CUs take part.  Rows
// of 8 chunks (in_dim 32768) are the exception: there each workgroup reads
// the whole x_q row (as many bytes as one weight row), so row groups that
// share it win as long as 256 workgroups remain.
int choose_rg(const MatvecShape &sh, int64_t rows, int64_t experts) {
  const bool wide = sh.waves_per_row * sh.chunks_per_wave >= 8;
  const int64_t want = wide ? 256 : 1024;
  int rg = max_rg(sh);
  while (rg > 1) {
    const int64_t tiles = (rows + tile_rows(sh, rg) - 1) / tile_rows(sh, rg);
    if (tiles * experts >= want) break;
    rg /= 2;
  }
  return rg;
}

// ---- multi-matrix launch: independent small-batch projections in one grid.
//
// Workgroups are numbered across the items in order; item i owns tiles
// [first_tile_i, first_tile_{i+1}).  Each item runs the matvec body of its own
// row shape with one or two row groups per wave slot.  Items that carry fp32 rows
// quantize them in the workgroup (LdsX: rows of up to 64 pairs = 4096 values,
// shape codes 0..6, at most kFusePairs pairs over all tokens); the others read x_q from memory.  The per-output
// arithmetic and its order are those of the single-matrix kernel, so each item's
// result is bit-identical to a separate quantize + matvec call.
struct ListItemDev {
  float *out;
  const uint8_t *w;
  const float *x;      // non-null: quantize these fp32 rows in the workgroup
  uint8_t *x_q;        // x set: written by the item's first workgroup if non-null; else read
  int64_t out_dim;
  int64_t nb;          // in_dim / 32
  int32_t shape;       // row-shape code (shape_code)
  int32_t rg;          // row groups per wave slot (1 or 2)
  int32_t first_tile;  // first workgroup of the item
  int32_t pad;
};

struct ListArgs {
  ListItemDev item[kListMax];
  int32_t n_items;
  int32_t n_tok;
};

template <int LPR, int WPR, int CPW, int RG, class XS>
__device__ __forceinline__ void list_tile(const MatvecArgs &m, int64_t tile, XS &xs,
                                          uint32_t *wst) {
  if constexpr (coal_list_body(LPR, WPR, RG, CPW))
    matvec_body<LPR, WPR, CPW, RG, false, false, XS, false, true>(m, tile, m.w, nullptr,
                                                                  m.n_items, xs, nullptr, wst);
  else
    matvec_body<LPR, WPR, CPW, RG, false, false>(m, tile, m.w, nullptr, m.n_items, xs);
}

// Row shapes with one 64-pair chunk per wave, and 32768-wide rows (four
// waves of two chunks), take one or two row groups per wave slot; the other
// two-chunk shapes take one.
template <int LPR, int WPR, int CPW, class XS>
__device__ __forceinline__ void list_tile_rg(int rg, const MatvecArgs &m, int64_t tile, XS &xs,
                                             uint32_t *wst) {
  if constexpr (CPW == 1 || (CPW == 2 && WPR == 4)) {
    if (rg == 2) {
      list_tile<LPR, WPR, CPW, 2>(m, tile, xs, wst);
      return;
    }
  }
  list_tile<LPR, WPR, CPW, 1>(m, tile, xs, wst);
}

template <bool FUSED, class XS>
__device__ __forceinline__ void list_dispatch(int code, int rg, const MatvecArgs &m, int64_t tile,
                                              XS &xs, uint32_t *wst) {
  switch (code) {
    case 0: list_tile_rg<1, 1, 1>(rg, m, tile, xs, wst); break;
    case 1: list_tile_rg<2, 1, 1>(rg, m, tile, xs, wst); break;
    case 2: list_tile_rg<4, 1, 1>(rg, m, tile, xs, wst); break;
    case 3: list_tile_rg<8, 1, 1>(rg, m, tile, xs, wst); break;
    case 4: list_tile_rg<16, 1, 1>(rg, m, tile, xs, wst); break;
    case 5: list_tile_rg<32, 1, 1>(rg, m, tile, xs, wst); break;
    case 6: list_tile_rg<64, 1, 1>(rg, m, tile, xs, wst); break;
    default: break;
  }
  if constexpr (!FUSED) {
    switch (code) {
      case 7: list_tile_rg<64, 2, 1>(rg, m, tile, xs, wst); break;
      case 8: list_tile_rg<64, 2, 2>(rg, m, tile, xs, wst); break;
      case 9: list_tile_rg<64, 4, 1>(rg, m, tile, xs, wst); break;
      case 10: list_tile_rg<64, 4, 2>(rg, m, tile, xs, wst); break;
      default: break;
    }
  }
}

// Held to 128 VGPRs, four waves per SIMD, as many as its LDS allows: the
// two-row-group body of 32768-wide rows would otherwise take 146 and cost
// every item of the launch a wave (decode5 from x_q 11.0 -> 10.75 us with it).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void matvec_list_kernel(
    const ListArgs a) {
  __shared__ uint32_t xbuf[kFusePairs * kPairDwords];
  __shared__ __attribute__((aligned(16))) uint32_t wst[kCoalLdsDwords];
  // The item of this workgroup: the last one whose first tile is at or below
  // blockIdx.x.  The first tiles of all slots are read at once (no loop
  // carried load), and item 0 is fetched beside them, so a one-item launch
  // waits for a single round of argument loads.
  ListItemDev it = a.item[0];
  if (a.n_items > 1) {
    int i = 0;
#pragma unroll
    for (int j = 1; j < kListMax; ++j)
      if (j < a.n_items && (int)blockIdx.x >= a.item[j].first_tile) i = j;
    if (i) it = a.item[i];
  }
  MatvecArgs m{};
  m.out = it.out;
  m.w = it.w;
  m.x_q = it.x_q;
  m.out_dim = it.out_dim;
  m.n_items = a.n_tok;
  m.nb = it.nb;
  m.row_bytes = it.nb * kBlockBytes;
  const int64_t tile = (int64_t)blockIdx.x - it.first_tile;
  if (it.x) {
    LdsX xs;
    xs.lds = xbuf;
    xs.x = it.x;
    xs.x_q_out = tile == 0 ? it.x_q : nullptr;
    xs.log2_ppr = __builtin_ctzll((uint64_t)(it.nb / 2));
    xs.n_pairs = a.n_tok << xs.log2_ppr;
    xs.in_dim = it.nb * kBlockElems;
    list_dispatch<true>(it.shape, it.rg, m, tile, xs, wst);
  } else {
    GlobalX xs{it.x_q, m.row_bytes};
    list_dispatch<false>(it.shape, it.rg, m, tile, xs, wst);
  }
}

// A one-item list with fp32 rows: the same body as the list kernel's fused
// items (so the same outputs, bit for bit), in a kernel of its own with a
// plain argument block and only that body's code.  Against the list kernel
// this saves ~0.25 us per launch on the attn_q_b shape.
// WAVEX: at most kWaveXPairs pairs of x, quantized by every wave (LdsXWave).
template <int LPR, int RG, bool WAVEX>
__global__ __launch_bounds__(256) void matvec_fused_kernel(const MatvecArgs m, const float *x,
                                                           uint8_t *x_q_out) {
  static_assert(4 * kWaveXPairs <= kFusePairs, "four wave quarters fit the x buffer");
  __shared__ uint32_t xbuf[kFusePairs * kPairDwords];
  __shared__ __attribute__((aligned(16))) uint32_t wst[kCoalLdsDwords];
  std::conditional_t<WAVEX, LdsXWave, LdsX> xs;
  const int wave = (int)(threadIdx.x >> 6);
  xs.lds = WAVEX ? xbuf + wave * (kWaveXPairs * kPairDwords) : xbuf;
  xs.x = x;
  xs.x_q_out = blockIdx.x == 0 && (!WAVEX || wave == 0) ? x_q_out : nullptr;
  xs.log2_ppr = __builtin_ctzll((uint64_t)(m.nb / 2));
  xs.n_pairs = (int)(m.n_items << xs.log2_ppr);
  xs.in_dim = m.nb * kBlockElems;
  list_tile<LPR, 1, 1, RG>(m, blockIdx.x, xs, wst);
}

typedef void (*FusedFn)(const MatvecArgs, const float *, uint8_t *);

template <int LPR, bool WAVEX>
FusedFn pick_fused_rg(int rg) {
  return rg == 2 ? matvec_fused_kernel<LPR, 2, WAVEX> : matvec_fused_kernel<LPR, 1, WAVEX>;
}

template <bool WAVEX>
FusedFn pick_fused_shape(int code, int rg) {
  switch (code) {
    case 0: return pick_fused_rg<1, WAVEX>(rg);
    case 1: return pick_fused_rg<2, WAVEX>(rg);
    case 2: return pick_fused_rg<4, WAVEX>(rg);
    case 3: return pick_fused_rg<8, WAVEX>(rg);
    case 4: return pick_fused_rg<16, WAVEX>(rg);
    case 5: return pick_fused_rg<32, WAVEX>(rg);
    case 6: return pick_fused_rg<64, WAVEX>(rg);
    default: return nullptr;
  }
}

FusedFn pick_fused(int code, int rg, int64_t n_pairs) {
  return n_pairs <= kWaveXPairs ? pick_fused_shape<true>(code, rg)
                                : pick_fused_shape<false>(code, rg);
}

// Shape code of a matvec row shape, -1 when the list kernel has no body for
// it: rows of 3 or 4 chunks per wave (in_dim 12288, 49152, 65536) need about
// twice the registers and would halve the occupancy of every item in the grid.
int shape_code(const MatvecShape &sh) {
  switch (sh.lanes_per_row) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    case 16: return 4;
    case 32: return 5;
    default: break;
  }
  switch (sh.waves_per_row * 10 + sh.chunks_per_wave) {
    case 11: return 6;
    case 21: return 7;
    case 22: return 8;
    case 41: return 9;
    case 42: return 10;
    default: return -1;
  }
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
  int rg = choose_rg(sh, out_dim, 1);
  const bool staged = n_tok >= 2;
  // Single-token launches with rows of >= 4 pairs stage their weights through
  // coalesced loads (at most two 64-pair regions per wave): cap the row groups
  // to fit (in_dim 32768: one row group instead of four).
  if (!staged && sh.lanes_per_row >= 4)
    while (rg > 1 && rg * sh.chunks_per_wave > 2) rg /= 2;
  MatvecFn fn = blocksums ? pick_kernel<false, true>(sh, rg, staged)
                          : pick_kernel<false, false>(sh, rg, staged);
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
  MatvecFn fn = blocksums ? pick_kernel<true, true>(sh, rg, true) : pick_kernel<true, false>(sh, rg, true);
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

typedef void (*PairFn)(const MatvecArgs);

template <int LPR, int WPR, int CPW>
PairFn pick_pair_rg(int rg) {
  if (rg >= 2) return matvec_pair_kernel<LPR, WPR, CPW, 2>;
  return matvec_pair_kernel<LPR, WPR, CPW, 1>;
}

// Paired (gate, up) rows hold twice the weight registers, so shapes with more
// than one chunk per wave, or more than two row groups, are not offered.
PairFn pick_pair_kernel(const MatvecShape &sh, int rg) {
  switch (sh.lanes_per_row) {
    case 1: return pick_pair_rg<1, 1, 1>(rg);
    case 2: return pick_pair_rg<2, 1, 1>(rg);
    case 4: return pick_pair_rg<4, 1, 1>(rg);
    case 8: return pick_pair_rg<8, 1, 1>(rg);
    case 16: return pick_pair_rg<16, 1, 1>(rg);
    case 32: return pick_pair_rg<32, 1, 1>(rg);
    default: break;
  }
  switch (sh.waves_per_row * 10 + sh.chunks_per_wave) {
    case 11: return pick_pair_rg<64, 1, 1>(rg);
    case 21: return pick_pair_rg<64, 2, 1>(rg);
    case 41: return pick_pair_rg<64, 4, 1>(rg);
    default: return nullptr;
  }
}

bool matvec_pair_ok(int64_t in_dim) {
  MatvecShape sh;
  return matvec_shape(in_dim, &sh) && pick_pair_kernel(sh, 1) != nullptr;
}

hipError_t launch_matvec_grouped_pair(float *out, const void *const *gate_w,
                                      const void *const *up_w, int32_t n_expert, int64_t in_dim,
                                      int64_t out_dim, const void *x_q, int32_t n_used,
                                      const int32_t *counts, const int32_t *offsets,
                                      const int32_t *pairs, float clamp, hipStream_t s) {
  MatvecShape sh;
  if (!matvec_shape(in_dim, &sh)) return hipErrorInvalidValue;
  const int rg = std::min(choose_rg(sh, out_dim, n_expert), 2);
  PairFn fn = pick_pair_kernel(sh, rg);
  if (!fn) return hipErrorInvalidValue;
  MatvecArgs a{};
  a.out = out;
  a.expert_w = reinterpret_cast<const uint8_t *const *>(gate_w);
  a.expert_w2 = reinterpret_cast<const uint8_t *const *>(up_w);
  a.x_q = static_cast<const uint8_t *>(x_q);
  a.counts = counts;
  a.offsets = offsets;
  a.pairs = pairs;
  a.out_dim = out_dim;
  a.nb = in_dim / kBlockElems;
  a.row_bytes = a.nb * kBlockBytes;
  a.n_used = n_used;
  a.x_rows = 0;
  a.clamp = clamp;
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

bool list_item_ok(int64_t in_dim) {
  MatvecShape sh;
  return matvec_shape(in_dim, &sh) && shape_code(sh) >= 0;
}

bool list_item_fusable(int64_t in_dim, int64_t n_tok) {
  MatvecShape sh;
  if (!matvec_shape(in_dim, &sh)) return false;
  const int code = shape_code(sh);
  return code >= 0 && code <= 6 && n_tok * (in_dim / 64) <= kFusePairs;
}

hipError_t launch_matvec_list(const ListItem *items, int n_items, int64_t n_tok, hipStream_t s) {
  if (n_items < 1 || n_items > kListMax) return hipErrorInvalidValue;
  ListArgs a{};
  int64_t tiles = 0;
  for (int i = 0; i < n_items; ++i) {
    const ListItem &src = items[i];
    MatvecShape sh;
    if (!matvec_shape(src.in_dim, &sh)) return hipErrorInvalidValue;
    const int code = shape_code(sh);
    if (code < 0 || (src.x && !list_item_fusable(src.in_dim, n_tok))) return hipErrorInvalidValue;
    ListItemDev &d = a.item[i];
    d.out = src.out;
    d.w = static_cast<const uint8_t *>(src.w);
    d.x = src.x;
    d.x_q = static_cast<uint8_t *>(src.x_q);
    d.out_dim = src.out_dim;
    d.nb = src.in_dim / kBlockElems;
    // Two row groups per wave slot where the item alone still fills 1024
    // workgroups (256 for 32768-wide rows): fewer, fuller workgroups stay
    // resident in one round, and a 32768-wide x row is read once per two
    // weight rows instead of once per row (decode5 from x_q 11.0 -> 10.75 us).
    // Items quantized in the launch take two from 256 rows on: every
    // workgroup reads the whole fp32 row, so fuller workgroups halve those
    // reads (router + shared gate/up 7.87 -> 7.42 us; decode5 unchanged).
    const bool two = sh.chunks_per_wave == 1 || (sh.chunks_per_wave == 2 && sh.waves_per_row == 4);
    const bool fused_two = src.x && sh.chunks_per_wave == 1 && src.out_dim >= 256;
    const int rg = (two && (fused_two || choose_rg(sh, src.out_dim, 1) >= 2)) ? 2 : 1;
    d.shape = code;
    d.rg = rg;
    d.first_tile = (int32_t)tiles;
    tiles += (src.out_dim + tile_rows(sh, rg) - 1) / tile_rows(sh, rg);
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
  }
  a.n_items = n_items;
  a.n_tok = (int32_t)n_tok;
  if (n_items == 1 && a.item[0].x) {
    const ListItemDev &d = a.item[0];
    FusedFn fn = pick_fused(d.shape, d.rg, n_tok * (d.nb / 2));
    if (!fn) return hipErrorInvalidValue;
    MatvecArgs m{};
    m.out = d.out;
    m.w = d.w;
    m.x_q = d.x_q;
    m.out_dim = d.out_dim;
    m.n_items = n_tok;
    m.nb = d.nb;
    m.row_bytes = d.nb * kBlockBytes;
    hipLaunchKernelGGL(fn, dim3((uint32_t)tiles), dim3(256), 0, s, m, d.x, d.x_q);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(matvec_list_kernel, dim3((uint32_t)tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace q8
