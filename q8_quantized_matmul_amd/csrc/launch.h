// launch.h -- internal host-side launchers, one per kernel family.  Each
// returns hipSuccess or the launch error; argument checks happen in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// quantize.hip
hipError_t launch_quantize(void *x_q, const float *x, int64_t n_tok, int64_t in_dim,
                           bool fast, hipStream_t s);

// matvec.hip: weight-streaming kernels for few tokens per weight row.
struct MatvecShape {
  int lanes_per_row;   // pairs handled by the lanes of one row (<= 64)
  int waves_per_row;   // waves cooperating on one row (split over chunks)
  int chunks_per_wave; // 64-pair chunks per wave (1 when lanes_per_row < 64)
};
bool matvec_shape(int64_t in_dim, MatvecShape *shape);
hipError_t launch_matvec(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                         int64_t out_dim, const void *x_q, int64_t n_tok, hipStream_t s);
hipError_t launch_generic(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                          int64_t out_dim, const void *x_q, int64_t n_tok, hipStream_t s);
hipError_t launch_matvec_grouped(float *out, int32_t *blocksums, const void *const *expert_w,
                                 int32_t n_expert, int64_t in_dim, int64_t out_dim,
                                 const void *x_q, int32_t x_rows, int32_t n_used,
                                 const int32_t *counts, const int32_t *offsets,
                                 const int32_t *pairs, hipStream_t s);
hipError_t launch_generic_grouped(float *out, int32_t *blocksums, const void *const *expert_w,
                                  int32_t n_expert, int64_t in_dim, int64_t out_dim,
                                  const int32_t *selected, int32_t n_used, const void *x_q,
                                  int32_t x_rows, int64_t n_tok, hipStream_t s);

// Multi-matrix small-batch launch (one grid over up to kListMax projections).
constexpr int kListMax = 16;
struct ListItem {
  float *out;
  const void *w;
  const float *x;   // non-null: quantized inside the launch (list_item_fusable)
  void *x_q;        // read when x is null; written when x is set and x_q non-null
  int64_t in_dim;
  int64_t out_dim;
};
bool list_item_ok(int64_t in_dim);
bool list_item_fusable(int64_t in_dim, int64_t n_tok);
hipError_t launch_matvec_list(const ListItem *items, int n_items, int64_t n_tok, hipStream_t s);

bool matvec_pair_ok(int64_t in_dim);
hipError_t launch_matvec_grouped_pair(float *out, const void *const *gate_w,
                                      const void *const *up_w, int32_t n_expert, int64_t in_dim,
                                      int64_t out_dim, const void *x_q, int32_t n_used,
                                      const int32_t *counts, const int32_t *offsets,
                                      const int32_t *pairs, float clamp, hipStream_t s);

// moe.hip
struct MoeLayout {
  int64_t counts, offsets, pairs;  // int32 element offsets inside the workspace
  int64_t total_ints;
};
MoeLayout moe_layout(int64_t n_tok, int32_t n_used, int32_t n_expert);
hipError_t launch_moe_route(const int32_t *selected, int64_t n_tok, int32_t n_used,
                            int32_t n_expert, int32_t *ws, float *nan_rows, int64_t nan_dim,
                            hipStream_t s, int32_t *invalid_out);
// Routing tables of q8_0_moe_grouped_noalloc: a static device array of this
// many bytes; moe_static_scratch gives its address on the current device.
constexpr size_t kMoeStaticScratchBytes = size_t{1} << 20;
constexpr int kMaxDevicesStatic = 64;
hipError_t moe_static_scratch(int32_t **ptr);
// The routed expert FFN: buffers already validated, intermediates placed.
struct MoeFfn {
  float *out;
  const void *const *gate_w, *const *up_w, *const *down_w;
  int32_t n_expert, n_used;
  int64_t d_model, d_ff, n_tok;
  const int32_t *selected;
  const float *weights;
  const void *x_q;
  float clamp;
  float *mid;   // [n_tok*n_used][d_ff]
  void *mid_q;  // [n_tok*n_used][d_ff/32] blocks
  float *y;     // [n_tok*n_used][d_model]
};
hipError_t launch_moe_ffn(const MoeFfn &f, int32_t *ws, hipStream_t s);
hipError_t launch_moe(float *out, int32_t *blocksums, const void *const *expert_w,
                      int32_t n_expert, int64_t in_dim, int64_t out_dim,
                      const int32_t *selected, int32_t n_used, const void *x_q,
                      int32_t x_rows, int64_t n_tok, int32_t *workspace, bool fast,
                      hipStream_t s, int32_t *invalid_out = nullptr);

// Caller workspace of q8_0_matmul split-K plans: arrival counters of the
// skinny kernel's in-launch reduction (zero between calls) in the first
// kWsCounterBytes, partial sums after them.
constexpr size_t kWsCounterBytes = 4096;

// skinny.hip: matrix-core matmul, token and weight rows staged in LDS.  Up to
// kSkinnyMaxTokens tokens a workgroup may hold both token tiles and split-K
// is reduced inside the launch; up to kSkinnyWideMaxTokens every 32-token
// tile has workgroups of its own and there is one split.
constexpr int64_t kSkinnyMaxTokens = 64;
constexpr int64_t kSkinnyWideMaxTokens = 256;
bool skinny_supported(int64_t in_dim, int64_t n_tok);
// Shapes for which the plan prefers the skinny kernel to the tiled GEMM from
// kSkinnyMaxTokens + 1 to kSkinnyWideMaxTokens tokens.
bool skinny_many_tokens(int64_t in_dim, int64_t out_dim, int64_t n_tok);
int skinny_auto_split(int64_t in_dim, int64_t out_dim, int64_t n_tok);
// A split needs one counter per 32-row output tile.
bool skinny_split_ok(int64_t in_dim, int64_t out_dim, int64_t n_tok, int split);
size_t skinny_workspace_bytes(int64_t out_dim, int64_t n_tok, int split);
hipError_t launch_skinny(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                         int64_t out_dim, const void *x_q, int64_t n_tok, int split,
                         void *workspace, hipStream_t s);

// gemm.hip: int8 MFMA GEMM with per-block scales.
bool gemm_supported(int64_t in_dim);
int gemm_auto_split(int64_t in_dim, int64_t out_dim, int64_t n_tok);
size_t gemm_workspace_bytes(int64_t out_dim, int64_t n_tok, int split);
hipError_t launch_gemm(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                       int64_t out_dim, const void *x_q, int64_t n_tok, int split,
                       void *workspace, hipStream_t s);
// out[i] = sum over s = 0..n_split-1, in order, of partials[s * n + i].
hipError_t launch_splitk_reduce(float *out, const float *partials, int64_t n, int n_split,
                                hipStream_t s);

// probe.hip: measured ceilings (a streaming read, an empty launch, int8 MFMA loops).
constexpr int kProbeWorkgroups = 512;  // 2 per CU, 4 waves each
constexpr int kProbeChains = 4;        // independent MFMA chains per wave
hipError_t launch_probe_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_launch(int32_t workgroups, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_mfma(int32_t iters, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_mix(int32_t iters, int32_t mix, uint32_t *sink, hipStream_t s);
// debug.hip: LDS poisoning for the race tests: kDebugLdsDwords of LDS per workgroup (five
// workgroups fill a compute unit's 160 KB), four rounds of them per compute unit.
constexpr int kDebugLdsDwords = 8192;
constexpr int kDebugPoisonWorkgroups = 256 * 5 * 4;
hipError_t launch_debug_poison_lds(uint32_t pattern, hipStream_t s);
hipError_t launch_debug_read_lds(uint32_t *seen, int32_t workgroups, hipStream_t s);

}  // namespace q8
