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

// The same through a pointer taken as global memory explicitly.  For bases
// read from a device table (the grouped kernels' expert weights) the compiler
// would otherwise emit flat loads, which also count on the LDS/scalar wait
// counter.  Only the grouped kernels use it: elsewhere the pointers are kernel
// arguments, already known to be global.
typedef __attribute__((address_space(1))) const u32x4_a4 global_u32x4_a4;
typedef __attribute__((address_space(1))) const uint32_t global_u32;
__device__ __forceinline__ void load_pair_global(const uint8_t *p, uint32_t (&d)[kPairDwords]) {
  global_u32x4_a4 *v = (global_u32x4_a4 *)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4_a4 t = v[i];
    d[4 * i + 0] = t.x;
    d[4 * i + 1] = t.y;
    d[4 * i + 2] = t.z;
    d[4 * i + 3] = t.w;
  }
  d[16] = ((global_u32 *)p)[16];
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

// ---- Q8_0 activation quantization of one block pair by 16 lanes.
//
// Block rule ("Part 3: 模型架构", section 2, the row quantizer, applied per 32
// values with a binary16 scale): amax = max|x_i|, d32 = amax / 127 (IEEE fp32
// division), q_i = roundf(x_i / d32) clamped to +-127, stored scale
// binary16(d32) rounded to nearest even with subnormals kept.  A zero block
// (amax == 0 or d32 == 0) is all zero; a non-finite value in the block, or a
// d32 that overflows binary16, gives scale 0x7E00 and zero quants.
//
// The quotient x/d32 is formed as x * (1/d32), with 1/d32 an IEEE division
// done once per block.  That product is within 3 * 2^-24 * 127.5 < 2.3e-5 of
// the IEEE quotient, so whenever it lies at least kTieMargin from every
// half-integer, both round to the same integer -- and, not being a tie,
// round-to-nearest-even of the product gives it.  A lane holding a value
// inside the margin (rare), or a block whose d32 is subnormal (1/d32 may
// overflow), recomputes all its quotients as IEEE divisions rounded half away
// from zero, so the quants are exactly roundf(x / d32).
constexpr float kTieMargin = 6.103515625e-05f;  // 2^-14

// q[i] = clamp(roundf(v[i] / d), -127, 127).
template <int N>
__device__ __forceinline__ void quant_values(const float (&v)[N], float d, float inv, bool exact,
                                             int (&q)[N]) {
  float r[N];
  bool near = exact;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float p = v[i] * inv;
    r[i] = __builtin_rintf(p);
    near = near || fabsf(p - r[i]) > 0.5f - kTieMargin;
  }
  if (near) {  // rare: IEEE quotients
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = roundf(v[i] / d);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) q[i] = (int)__builtin_amdgcn_fmed3f(r[i], -127.0f, 127.0f);
}

__device__ __forceinline__ uint32_t pack4(int q0, int q1, int q2, int q3) {
  return ((uint32_t)q0 & 0xFFu) | (((uint32_t)q1 & 0xFFu) << 8) | (((uint32_t)q2 & 0xFFu) << 16) |
         ((uint32_t)q3 << 24);
}

// The dwords one lane stores of a quantized pair (17 dwords, see pair_dots for
// the layout): lane `sub` stores `hi` at dword sub + 1, lane 0 also `lo` at
// dword 0.
struct PairWords {
  uint32_t hi;
  uint32_t lo;
};

// Cross-lane moves inside a 16-lane DPP row (the 16-lane groups below are
// row aligned): kDppXor1 / kDppXor2 read lane i^1 / i^2 (quad permutes),
// kDppHalfMirror reads lane 7-i of the same 8-lane half row, kDppNext reads
// lane i+1 (row shift left by one).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowRor4 = 0x124;  // the 16-lane row rotated by 4 lanes
constexpr int kDppRowRor8 = 0x128;  // ... and by 8 lanes
constexpr int kDppNext = 0x101;
constexpr int kDppMirror = 0x140;    // lane 15-i of the same 16-lane row
constexpr int kDppBcast15 = 0x142;   // lane 15 of the previous row
constexpr int kDppBcast31 = 0x143;   // lane 31, to rows 2 and 3

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}

// Sum over aligned groups of N lanes (N a power of two <= 64) with DPP adds:
// a butterfly over lanes within 16-lane rows, then row broadcasts.  Every
// level adds two equal-size partial sums, so the result has the same value
// as a xor-shuffle butterfly.  For N <= 16 every lane of a group holds the
// sum; for N = 32 the lanes 16..31 of the group; for N = 64 the lanes
// 48..63 (group_sum_lane gives one of them).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f32<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f32<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<kDppMirror>(v);
  if constexpr (N >= 32) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), kDppBcast15, 0xA, 0xF, false));
  }
  if constexpr (N >= 64) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), kDppBcast31, 0xC, 0xF, false));
  }
  return v;
}
template <int N>
__device__ __forceinline__ bool group_sum_lane(int lane) {
  return N <= 16 ? (lane % N) == 0 : (lane % N) == N - 1;
}

// Lanes 16j..16j+15 of the wave hold one pair of 64 values, lane sub = lane &
// 15 holding values 4*sub..4*sub+3 in v (lanes 0..7 block A, 8..15 block B).
// Every lane of the wave must call this (it exchanges values inside its
// 16-lane group).
__device__ __forceinline__ PairWords quantize_pair16(float4 v, int sub) {
  // Non-finite values count as +inf so one max-reduction also flags them.
  // The max over the 8 lanes of a block: quads first, then the mirrored quad.
  auto mag = [](float t) { return __builtin_isfinite(t) ? fabsf(t) : __builtin_huge_valf(); };
  float amax = fmaxf(fmaxf(mag(v.x), mag(v.y)), fmaxf(mag(v.z), mag(v.w)));
  amax = fmaxf(amax, dpp_f32<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f32<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_f32<kDppHalfMirror>(amax));

  uint32_t bits = 0, qd = 0;
  if (!__builtin_isfinite(amax)) {
    bits = 0x7E00u;
  } else if (amax > 0.0f) {
    const float d = amax / 127.0f;
    if (d > 0.0f) {
      bits = __builtin_bit_cast(uint16_t, (_Float16)d);
      if ((bits & 0x7FFFu) == 0x7C00u) {
        bits = 0x7E00u;  // scale does not fit binary16
      } else {
        const bool exact = d < 1.17549435e-38f;  // subnormal d32: 1/d32 may overflow
        const float inv = 1.0f / d;
        const float vals[4] = {v.x, v.y, v.z, v.w};
        int q[4];
        quant_values(vals, d, inv, exact, q);
        qd = pack4(q[0], q[1], q[2], q[3]);
      }
    }
  }

  // Pair dwords: [dA | qA0..1] [qA2..29 in 7 dwords] [qA30..31 | dB] [qB 8 dwords].
  // Lane g < 8 forms dword g+1 from its own quants and lane g+1's; lane 0 also
  // forms dword 0; lanes 8..15 form dwords 9..16.
  const uint32_t next = dpp_u32<kDppNext>(qd);     // lane sub+1's quants
  const uint32_t bitsB = dpp_u32<kDppNext>(bits);  // at lane 7: lane 8's (block B) scale
  PairWords r;
  if (sub < 7) {
    r.hi = (qd >> 16) | (next << 16);
  } else if (sub == 7) {
    r.hi = (qd >> 16) | (bitsB << 16);
  } else {
    r.hi = qd;
  }
  r.lo = bits | (qd << 16);
  return r;
}

// The same block rule with 4 lanes per pair, for quantizing a whole row of up
// to 4096 values in one pass of a 256-thread workgroup.  Lanes 4i..4i+3 hold
// one pair; lane j = lane & 3 holds values 16j..16j+15 in v[0..3] (j = 0, 1
// block A, j = 2, 3 block B).  Every lane of the wave must call this.
// Lane j stores out[0 .. pair4_count(j)) at dwords pair4_first(j) onward:
// lane 0 dwords 0..4, lane 1 dwords 5..8, lane 2 dwords 9..12, lane 3 13..16.
__device__ __forceinline__ int pair4_first(int j) { return j == 0 ? 0 : 1 + 4 * j; }
__device__ __forceinline__ int pair4_count(int j) { return j == 0 ? 5 : 4; }

__device__ __forceinline__ void quantize_pair4(const float4 (&v)[4], int j, uint32_t (&out)[5]) {
  auto mag = [](float t) { return __builtin_isfinite(t) ? fabsf(t) : __builtin_huge_valf(); };
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    amax = fmaxf(amax, fmaxf(fmaxf(mag(v[k].x), mag(v[k].y)), fmaxf(mag(v[k].z), mag(v[k].w))));
  amax = fmaxf(amax, dpp_f32<kDppXor1>(amax));  // the other half of the block

  uint32_t bits = 0, qd[4] = {0, 0, 0, 0};
  if (!__builtin_isfinite(amax)) {
    bits = 0x7E00u;
  } else if (amax > 0.0f) {
    const float d = amax / 127.0f;
    if (d > 0.0f) {
      bits = __builtin_bit_cast(uint16_t, (_Float16)d);
      if ((bits & 0x7FFFu) == 0x7C00u) {
        bits = 0x7E00u;  // scale does not fit binary16
      } else {
        const bool exact = d < 1.17549435e-38f;  // subnormal d32: 1/d32 may overflow
        const float inv = 1.0f / d;
        float vals[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vals[4 * k] = v[k].x;
          vals[4 * k + 1] = v[k].y;
          vals[4 * k + 2] = v[k].z;
          vals[4 * k + 3] = v[k].w;
        }
        int q[16];
        quant_values(vals, d, inv, exact, q);
#pragma unroll
        for (int k = 0; k < 4; ++k) qd[k] = pack4(q[4 * k], q[4 * k + 1], q[4 * k + 2], q[4 * k + 3]);
      }
    }
  }

  // Block A's quants start 2 bytes into the pair, so lanes 0 and 1 shift their
  // bytes by two: lane 0 borrows lane 1's first two quants, lane 1 lane 2's
  // (block B's) scale.  Block B's quants are dword aligned.
  const uint32_t nxt = dpp_u32<kDppNext>(qd[0]);  // at lane 0: qA16, qA17 in the low half
  const uint32_t bitsB = dpp_u32<kDppNext>(bits); // at lane 1: block B's scale
  if (j == 0) {
    out[0] = bits | (qd[0] << 16);
#pragma unroll
    for (int k = 1; k < 4; ++k) out[k] = (qd[k - 1] >> 16) | (qd[k] << 16);
    out[4] = (qd[3] >> 16) | (nxt << 16);
  } else if (j == 1) {
#pragma unroll
    for (int k = 0; k < 3; ++k) out[k] = (qd[k] >> 16) | (qd[k + 1] << 16);
    out[3] = (qd[3] >> 16) | (bitsB << 16);
    out[4] = 0;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = qd[k];
    out[4] = 0;
  }
}

// Staged rows of the matrix-core kernels: a row's 4 blocks (a 136-byte
// slice, dwords d0..d33) as nine 16-byte slots at a 144-byte LDS pitch --
// slice dwords 0..3, 4..7, ..., 28..31 and 30..33.
//
// A block dot sums qw_k * qx_k over k, so any permutation of k applied to
// both operands gives the same S_b.  With the slice's pairs d0..d16 and
// e0..e16 = d17..d33, a pair being
//   [sA | qA0 qA1] [qA2 .. qA29] [qA30 qA31 | sB] [qB0 .. qB31],
// the two 16-byte halves of each block's operand are
//   block 0: {bfi(d0, d8), d1, d2, d3}   | {d4, d5, d6, d7}     slots 0 | 1
//   block 1: {d16, d9, d10, d11}         | {d12, d13, d14, d15} slots 2 | 3
//   block 2: {e7, bfi(e0, e8), e1, e2}   | {e3, e4, e5, e6}     slots 4 | 5
//   block 3: {e11, e12, e9, e10}         | {e13, e14, e15, e16} slots 6 | 8
// where bfi(a, b) takes a's high half (the block's first two quants) and b's
// low half (its last two).  So every operand is one aligned 16-byte LDS read
// (consecutive rows sit 9 slots apart, which keeps those reads free of bank
// conflicts) plus, for half 0, one or two dwords of the next slot patched in
// with v_bfi; half 1 reads the same patch address and keeps its own dwords.
// The scales come out of the same reads: block 0's in d0's low half, block
// 1's in d8's high half, block 2's in e0's low half, block 3's in e8's high
// half.
constexpr int kPermPitch = 144;  // LDS bytes per staged 4-block row
constexpr int kPermSlots = kPermPitch / 16;

// Raw operand of block B: the half's 16-byte slot and the patch dwords from
// the slot after half 0's.
struct PermRaw {
  i32x4 v;
  uint32_t p0, p1;
};

template <int B>
__device__ __forceinline__ void perm_read(const uint8_t *row, int h, PermRaw &r) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  constexpr int S0 = B == 0 ? 0 : B == 1 ? 2 : B == 2 ? 4 : 6;  // half 0's slot
  constexpr int S1 = B == 3 ? 8 : S0 + 1;                        // half 1's slot
  constexpr int SP = B == 3 ? 7 : S0 + 2;                        // patch slot
  r.v = *reinterpret_cast<const i32x4 *>(row + 16 * (h ? S1 : S0));
  if constexpr (B < 2) {
    r.p0 = *reinterpret_cast<const uint32_t *>(row + 16 * SP);
  } else {
    const u32x2 pp = *reinterpret_cast<const u32x2 *>(row + 16 * SP);
    r.p0 = pp.x;
    r.p1 = pp.y;
  }
}

// Per-lane constants of perm_prep: bfi masks (bits taken from the slot
// dword, the rest from the patch) and the byte selects of the scale.
struct PermLane {
  uint32_t keep_hi;  // the high half on half 0, everything on half 1
  uint32_t keep_h1;  // nothing on half 0, everything on half 1
  uint32_t sel_lo;   // scale bytes 0, 1 on half 0 (zero on half 1)
  uint32_t sel_hi;   // scale bytes 2, 3 on half 0 (zero on half 1)
  __device__ __forceinline__ explicit PermLane(int h)
      : keep_hi(h ? 0xFFFFFFFFu : 0xFFFF0000u),
        keep_h1(h ? 0xFFFFFFFFu : 0u),
        sel_lo(h ? 0x0C0C0C0Cu : 0x0C0C0100u),
        sel_hi(h ? 0x0C0C0C0Cu : 0x0C0C0302u) {}
};

__device__ __forceinline__ uint32_t perm_bfi(uint32_t keep, uint32_t x, uint32_t y) {
  return (x & keep) | (y & ~keep);
}

// The operand of block B in the permuted order, and the scale bits for half
// 0 (zero for half 1, which feeds the unused K slots of the scale MFMA).
template <int B>
__device__ __forceinline__ i32x4 perm_prep(const PermRaw &r, const PermLane &pl, uint32_t &scale) {
  uint32_t v0 = (uint32_t)r.v.x, v1 = (uint32_t)r.v.y;
  if constexpr (B == 0) {           // {bfi(d0, d8), d1, d2, d3}
    scale = __builtin_amdgcn_perm(0u, v0, pl.sel_lo);
    v0 = perm_bfi(pl.keep_hi, v0, r.p0);
  } else if constexpr (B == 1) {    // {d16, d9, d10, d11}
    scale = __builtin_amdgcn_perm(0u, v0, pl.sel_hi);
    v0 = perm_bfi(pl.keep_h1, v0, r.p0);
  } else if constexpr (B == 2) {    // {e7, bfi(e0, e8), e1, e2}
    scale = __builtin_amdgcn_perm(0u, v1, pl.sel_lo);
    v1 = perm_bfi(pl.keep_hi, v1, r.p1);
    v0 = perm_bfi(pl.keep_h1, v0, r.p0);
  } else {                          // {e11, e12, e9, e10}
    scale = __builtin_amdgcn_perm(0u, v1, pl.sel_hi);
    v0 = perm_bfi(pl.keep_h1, v0, r.p0);
    v1 = perm_bfi(pl.keep_h1, v1, r.p1);
  }
  return i32x4{(int)v0, (int)v1, r.v.z, r.v.w};
}

// Direct global->LDS dword copy through a buffer resource: a 32-bit lane
// offset and a scalar offset, so the copy needs no 64-bit address per lane.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ void buffer_load_lds_raw(rsrc_t rsrc, __attribute__((address_space(3))) uint32_t *lds,
                                    int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer resource over [base, base + bytes): stride 0, 32-bit dword format.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return rsrc_t{(int32_t)(uint32_t)b, (int32_t)(uint32_t)(b >> 32) & 0xFFFF, (int32_t)bytes,
                0x00020000};
}

}  // namespace q8
