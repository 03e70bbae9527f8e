/*
 * q8_0.h -- C ABI of the Q8_0 quantized matmul library for AMD MI355X (gfx950).
 *
 * The operation is the ds4 engine's Q8_0 matmul/matvec and its Q8_0 expert
 * matmuls, as described on the ds4-learning pages:
 *   - "Part 6: 代码走读", trace 3 (GPU matmul 与 matvec): Q8_0 weights times
 *     Q8_0 activations, arguments (out, weights, in_dim, out_dim, x, n_tok),
 *     in_dim must be a multiple of the 32-value Q8_0 block.
 *   - "Part 3: 模型架构", section 2: the per-block quantization rule
 *     (amax, scale = amax/127, q = roundf(x/scale)) and y = x @ W.
 *   - "Part 6: 代码走读", trace 5 (GPU MoE): per-token selected expert lists
 *     drive one expert matmul per (token, slot).
 *   - "Part 6: GPU 加速", section 1 (ds4_gpu.h): backend types never appear in
 *     the interface, the caller owns every buffer, work is enqueued
 *     asynchronously and the caller synchronizes before reading results.
 *
 * Q8_0 block: 32 values in 34 bytes -- a little-endian binary16 scale d
 * followed by 32 int8 quants q; value_i = d * q_i.  A matrix [rows][k] is
 * stored as rows * (k/32) consecutive blocks, row-major (row r, block b at
 * byte offset (r * (k/32) + b) * 34).
 *
 * Conventions for every call below:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates and frees nothing.  Inputs are read-only.
 *   - Calls only enqueue work on `stream` (0 = the null stream) and return;
 *     the caller synchronizes the stream before reading outputs.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and returned as a negative Q8_0_E* code; nothing is written then.
 *   - n_tok == 0 or out_dim == 0 is a successful no-op.
 *   - Pointers must be at least 2-byte aligned (Q8_0_EALIGN otherwise); the
 *     fast kernels need 4-byte alignment (16-byte for fp32 inputs and for the
 *     direct-to-LDS GEMM kernels) and fall back to a generic kernel when it is
 *     missing.  The floor is 2 bytes, not 16, because Q8_0 rows are multiples
 *     of 34 bytes: a slice starting at an odd block is only 2-byte aligned,
 *     and such zero-copy views of a weight file are valid operands.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Calls on different streams touching disjoint outputs are independent.
 */
#ifndef Q8_0_H
#define Q8_0_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

#define Q8_0_BLOCK_ELEMS 32
#define Q8_0_BLOCK_BYTES 34

enum {
    Q8_0_OK = 0,
    Q8_0_EINVAL = -1,     /* bad size, null pointer, bad mode */
    Q8_0_EALIGN = -2,     /* pointer alignment below 2 bytes */
    Q8_0_ELAUNCH = -3,    /* the HIP runtime rejected a kernel launch */
    Q8_0_EWORKSPACE = -4, /* workspace missing or smaller than required */
    Q8_0_ENODEV = -5      /* no usable gfx950 device for the stream */
};

/* Kernel variants (for q8_0_matmul_debug; 0 lets the library choose). */
enum {
    Q8_0_KERNEL_AUTO = 0,
    Q8_0_KERNEL_GENERIC = 1, /* one block per lane, any shape           */
    Q8_0_KERNEL_MATVEC = 2,  /* weight-streaming matvec, small n_tok     */
    Q8_0_KERNEL_MFMA = 3,    /* int8 MFMA GEMM, large n_tok              */
    Q8_0_KERNEL_SKINNY = 4   /* int8 MFMA, rows staged in LDS, n_tok <= 256 */
};

/* Quantize activations to Q8_0 ("Part 3: 模型架构", section 2 rule, per
 * 32-value block with a binary16 scale).
 *   x   : fp32 [n_tok][in_dim], row-major.
 *   x_q : n_tok * (in_dim/32) * 34 bytes, written.
 * Per block: amax = max|x_i|; d32 = amax/127 (IEEE fp32 division);
 * q_i = roundf(x_i / d32) (IEEE division, halves away from zero) clamped to
 * [-127, 127]; stored scale = binary16(d32), round to nearest even.  A block
 * with amax == 0 (or d32 == 0) is all zeros.  A block holding a NaN or an
 * infinity, or whose d32 does not fit binary16 (d32 >= 65520), is stored with
 * scale 0x7E00 (NaN) and zero quants, so every output that uses it is NaN.
 * (Such values are only seen by the device after the call has returned, so
 * they are reported in the data rather than by a return code.)
 * Errors: in_dim % 32 != 0, negative sizes, null pointers -> Q8_0_EINVAL. */
int q8_0_quantize_act(void *x_q, const float *x, int64_t n_tok, int64_t in_dim,
                      hipStream_t stream);

/* Workspace bytes q8_0_matmul would use for its fastest plan on this shape
 * (split-K partial sums); 0 when the plan needs none. */
size_t q8_0_matmul_workspace_bytes(int64_t in_dim, int64_t out_dim, int64_t n_tok);

/* Q8_0 matmul ("Part 6: 代码走读", trace 3: ds4_gpu_matmul_q8_0_tensor):
 *   out[t][o] = sum_b fp32(d_w[o][b]) * fp32(d_x[t][b]) * S_b[t][o],
 *   S_b[t][o] = sum_{i<32} qw[o][b][i] * qx[t][b][i]  (exact int32).
 *   out : fp32 [n_tok][out_dim], written.
 *   w   : Q8_0 [out_dim][in_dim/32] blocks.
 *   x_q : Q8_0 [n_tok][in_dim/32] blocks (e.g. from q8_0_quantize_act).
 *   workspace / workspace_bytes : optional caller scratch (device memory,
 *     16-byte aligned) for split-K plans; with less than
 *     q8_0_matmul_workspace_bytes() the library picks a plan that fits (same
 *     results up to fp32 summation order).  Zero-fill it once before its
 *     first use and keep it for later calls: its first 4096 bytes hold the
 *     arrival counters of the in-launch split-K reduction, which every call
 *     leaves at zero again (the partial sums after them need no
 *     initialization).  Calls that share a workspace must not overlap in time
 *     (issue them on one stream).
 *     These two arguments are an addition to the pages' matmul signature: the
 *     library allocates nothing ("Part 6: GPU 加速", summary: no allocation on
 *     the hot path), so a split-K plan needs its partials from the caller;
 *     NULL / 0 is always valid.
 * The fp32 result is within 1e-5 * sum_b |d_w d_x S_b| + 1e-6 of the exact
 * value; S_b itself is exact.  Errors: in_dim % 32 != 0 or in_dim == 0 with
 * out_dim > 0, negative sizes, null pointers -> Q8_0_EINVAL. */
int q8_0_matmul(float *out, const void *w, int64_t in_dim, int64_t out_dim,
                const void *x_q, int64_t n_tok, void *workspace,
                size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes q8_0_moe_grouped needs (routing tables and lists).  The
 * size depends on the routing shape only (not on in_dim or out_dim): the
 * workspace holds the per-expert counts, offsets and the pair list. */
size_t q8_0_moe_workspace_bytes(int64_t n_tok, int32_t n_used, int32_t n_expert);

/* Grouped expert matmul ("Part 6: 代码走读", trace 5: the gate/up and down
 * expert projections of ds4_gpu_routed_moe_one_tensor, one weight set per call).
 *   expert_w : DEVICE array of n_expert device pointers; expert e's weights are
 *              Q8_0 [out_dim][in_dim/32] blocks at expert_w[e].  The table
 *              lives on the device (like the pages' expert table, "Part 6: GPU
 *              加速", section 4a) so a call copies nothing from the host and
 *              can be captured in a HIP graph; build it once per weight set.
 *   selected : device int32 [n_tok][n_used], token -> expert ids (slot order).
 *   x_q      : Q8_0 rows; x_rows == 0: one row per token (gate/up input),
 *              x_rows == 1: one row per (token, slot) pair, row t*n_used + j
 *              (down input).
 *   out      : fp32 [n_tok][n_used][out_dim], written:
 *              out[t][j] = matmul(W_{selected[t][j]}, x row).
 * Routing happens on the GPU (no host round trip): counts, offsets and a
 * stable expert-major pair list are built in `workspace`, then each touched
 * expert's weights are streamed once for all of its pairs.  Duplicate ids in
 * a row are computed independently.  An id outside [0, n_expert) cannot be
 * seen on the host: its pair's output row is set to NaN and the int32 at byte
 * offset 0 of `workspace` holds, once the stream reaches the end of the call,
 * the number of such pairs.
 * Errors: bad sizes/mode/null pointers -> Q8_0_EINVAL; workspace smaller than
 * q8_0_moe_workspace_bytes() -> Q8_0_EWORKSPACE. */
int q8_0_moe_grouped(float *out, const void *const *expert_w, int32_t n_expert,
                     int64_t in_dim, int64_t out_dim, const int32_t *selected,
                     int32_t n_used, const void *x_q, int32_t x_rows,
                     int64_t n_tok, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the grouped
 * expert matmul of q8_0_moe_grouped without the workspace argument.  The
 * routing tables go to a static device array inside the library instead, of
 * Q8_0_MOE_STATIC_SCRATCH_BYTES bytes, which each GPU the library runs on
 * holds until the process ends.  Arguments, results and errors are those of
 * q8_0_moe_grouped (same kernels, bit-identical outputs), except:
 *   n_invalid : optional device int32; when not NULL it receives, once the
 *               stream reaches the end of the call, the number of pairs whose
 *               expert id lies outside [0, n_expert) (their rows are NaN).
 *   A routing shape with q8_0_moe_workspace_bytes(n_tok, n_used, n_expert)
 *   above Q8_0_MOE_STATIC_SCRATCH_BYTES (about 260,000 (token, slot) pairs
 *   at 256 experts) -> Q8_0_EWORKSPACE, nothing enqueued.
 * The call allocates nothing.  Every call on one GPU shares that GPU's array
 * (the routing writes every word it later reads, so no clearing is needed):
 * calls that overlap on one GPU, e.g. on two streams at once, race and give
 * undefined results; serialize them. */
#define Q8_0_MOE_STATIC_SCRATCH_BYTES (1u << 20)
int q8_0_moe_grouped_noalloc(float *out, const void *const *expert_w, int32_t n_expert,
                             int64_t in_dim, int64_t out_dim, const int32_t *selected,
                             int32_t n_used, const void *x_q, int32_t x_rows, int64_t n_tok,
                             int32_t *n_invalid, hipStream_t stream);

/* Arguments of q8_0_moe_ffn. */
typedef struct q8_0_moe_ffn_args {
    float *out;                  /* fp32 [n_tok][d_model], written                  */
    const void *const *gate_w;   /* DEVICE table of n_expert device pointers; expert
                                    e's gate projection, Q8_0 [d_ff][d_model/32]     */
    const void *const *up_w;     /* DEVICE table: up projections, [d_ff][d_model/32] */
    const void *const *down_w;   /* DEVICE table: down projections, [d_model][d_ff/32] */
    int32_t n_expert;
    int32_t n_used;              /* experts per token                               */
    int64_t d_model;             /* expert input and output width                   */
    int64_t d_ff;                /* expert hidden width                             */
    int64_t n_tok;
    const int32_t *selected;     /* device int32 [n_tok][n_used]: expert ids         */
    const float *weights;        /* device fp32 [n_tok][n_used]: routing weights     */
    const void *x_q;             /* device Q8_0 [n_tok][d_model/32]                  */
    float clamp;                 /* SwiGLU limit (10 in the pages' 2-bit path); <= 0
                                    or NaN: no clamp                                */
    float *mid;                  /* optional fp32 [n_tok*n_used][d_ff] (NULL: kept in
                                    the workspace)                                   */
    void *mid_q;                 /* optional Q8_0 [n_tok*n_used][d_ff/32] (NULL: idem) */
    float *y;                    /* optional fp32 [n_tok*n_used][d_model], each pair's
                                    down output (NULL: idem)                         */
} q8_0_moe_ffn_args;

/* Workspace bytes q8_0_moe_ffn needs: routing tables plus room for mid, mid_q
 * and y (used only for those the caller does not supply). */
size_t q8_0_moe_ffn_workspace_bytes(int64_t n_tok, int32_t n_used, int32_t n_expert,
                                    int64_t d_model, int64_t d_ff);

/* The routed expert FFN ("Part 6: 代码走读", trace 5,
 * ds4_gpu_routed_moe_one_tensor: gate+up projections of the selected experts,
 * SwiGLU, down projections, weighted sum; "Part 3: 模型架构", section 4, the
 * SwiGLU activation and its clamp).  For token t and slot j, e = selected[t][j]:
 *   gate = W_gate[e] x_t, up = W_up[e] x_t          (Q8_0 matmuls as q8_0_matmul)
 *   mid  = silu(gate) * up, silu(g) = g / (1 + exp(-g)), after the optional
 *          limits (gate from above, up to +-clamp)  (fp32)
 *   mid_q = q8_0_quantize_act(mid)                  (the pair's Q8_0 row)
 *   y    = W_down[e] mid_q                          (as q8_0_matmul)
 *   out[t] = sum_j weights[t][j] * y[t][j], in slot order, one fp32 fma per slot.
 * Gate and up of a pair are computed in one pass over both matrices.  Each
 * touched expert's three matrices are streamed once for all of its pairs.
 * Ids outside [0, n_expert): the pair's y row is NaN (so is the token's out
 * row), its mid and mid_q rows are unspecified, and the int32 at byte 0 of the
 * workspace counts such pairs once the stream reaches the end of the call.
 * Shapes: d_model one of 64 * 2^k up to 4096, or 8192 or 16384 (the paired
 * gate+up kernel); d_ff any in_dim the weight-streaming matvec takes (a
 * multiple of 64: 64 * 2^k below 4096, or a multiple of 4096 up to 65536
 * with 1-3 chunks of 4096 per wave); other shapes give Q8_0_EINVAL.
 * Errors: bad sizes or null pointers -> Q8_0_EINVAL; workspace smaller than
 * q8_0_moe_ffn_workspace_bytes() -> Q8_0_EWORKSPACE. */
int q8_0_moe_ffn(const q8_0_moe_ffn_args *args, void *workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* One projection of q8_0_matmul_list. */
typedef struct q8_0_matmul_item {
    float *out;        /* fp32 [n_tok][out_dim], written                      */
    const void *w;     /* Q8_0 [out_dim][in_dim/32] blocks                     */
    const float *x;    /* fp32 [n_tok][in_dim] to quantize first, or NULL      */
    void *x_q;         /* Q8_0 [n_tok][in_dim/32]: read when x is NULL; when x
                          is set it receives the quantized rows, and may be
                          NULL if the item is quantized inside the launch (see
                          below)                                               */
    int64_t in_dim;
    int64_t out_dim;
} q8_0_matmul_item;

#define Q8_0_LIST_MAX 16

/* Several independent projections that read the same number of tokens, in as
 * few launches as possible ("Part 6: GPU 加速", section 4n, the exact decode
 * fusions: adjacent small dispatches are merged -- e.g. the router with the
 * shared expert's gate/up, or the q_a/kv pair -- and the merged kernel must
 * give bit-identical results; section 4m: per-token launch overhead of
 * serial decode).
 *   items   : HOST array of n_items descriptors (1 <= n_items <= 16), read
 *             during the call only.
 *   n_tok   : tokens of every item.
 * For each item: if x is set, x_q_i = q8_0_quantize_act(x); then
 * out = q8_0_matmul(w, x_q_i) with no workspace.  Every output and every
 * x_q byte is bit-identical to those separate calls.
 * Items on the weight-streaming path (n_tok < 12) share one launch.  An item
 * with x set whose in_dim is one of 64, 128, ..., 4096 with n_tok * in_dim <=
 * 4096 (and x 16-byte, x_q 4-byte aligned) is quantized inside that launch,
 * so a list of such decode projections is a single kernel launch; x_q may
 * then be NULL.  Other items with x set are quantized by a launch of their
 * own first and need x_q.  Items off the weight-streaming path run as
 * q8_0_matmul would.
 * Several items may share one x (and one x_q, which they then all write with
 * the same bytes).  Otherwise no item may write memory another item reads.
 * Errors: n_items outside [1, 16], any item invalid as for q8_0_matmul, or
 * x set with x_q NULL on an item that is not quantized inside the launch
 * -> Q8_0_EINVAL (nothing is enqueued). */
int q8_0_matmul_list(const q8_0_matmul_item *items, int32_t n_items, int64_t n_tok,
                     hipStream_t stream);

/* Test hook: q8_0_matmul with a forced kernel variant and split-K count
 * (0 = automatic) that also writes every block's exact integer dot S_b into
 * blocksums (device int32 [n_tok][out_dim][in_dim/32]) when it is not NULL.
 * The kernel that runs is the one the same call without blocksums would run
 * (its debug instantiation), so the S_b checked are those of the timed path.
 * Errors as q8_0_matmul, plus Q8_0_EINVAL when the forced variant cannot run
 * this shape (also a skinny split-K over more than 1024 output tiles: tiles
 * of 32 rows, and of 32 rows x 32 tokens above 64 tokens), and Q8_0_EWORKSPACE when a forced split needs more workspace than
 * q8_0_matmul_debug_workspace_bytes() reports for it. */
int q8_0_matmul_debug(float *out, int32_t *blocksums, const void *w,
                      int64_t in_dim, int64_t out_dim, const void *x_q,
                      int64_t n_tok, void *workspace, size_t workspace_bytes,
                      int32_t variant, int32_t split_k, hipStream_t stream);

/* Test hook: q8_0_moe_grouped that also writes each pair's block sums into
 * blocksums (device int32 [n_tok*n_used][out_dim][in_dim/32]). */
int q8_0_moe_grouped_debug(float *out, int32_t *blocksums,
                           const void *const *expert_w, int32_t n_expert,
                           int64_t in_dim, int64_t out_dim,
                           const int32_t *selected, int32_t n_used,
                           const void *x_q, int32_t x_rows, int64_t n_tok,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Host-only: workspace bytes q8_0_matmul_debug needs for this shape with the
 * forced variant and split-K count (as there; 0 = automatic), under the same
 * zero-fill rule as q8_0_matmul's workspace.  0 when that plan needs none or
 * cannot run this shape. */
size_t q8_0_matmul_debug_workspace_bytes(int64_t in_dim, int64_t out_dim, int64_t n_tok,
                                         int32_t variant, int32_t split_k);

/* Host-only: the kernel variant and split-K count q8_0_matmul would use for
 * this shape and workspace, assuming suitably aligned pointers.  Touches no
 * device.  Returns Q8_0_OK or Q8_0_EINVAL for an invalid shape. */
int q8_0_matmul_plan(int64_t in_dim, int64_t out_dim, int64_t n_tok,
                     size_t workspace_bytes, int32_t *variant, int32_t *split_k);

/* Measurement probe (the measured ceiling that the weight-streaming kernels
 * are reported against beside the 8 TB/s peak; decode is bound by reading
 * the weights, "Part 3: 模型架构", section 4): a plain coalesced read of
 * `bytes` bytes at `buf`, 64 bytes in flight per lane.
 *   buf  : device memory, 16-byte aligned; read only.
 *   bytes: a positive multiple of 16.
 *   sink : device uint32; written only if the loaded data hash to one fixed
 *          value, which keeps the loads from being optimized away.
 * Errors: bad size or alignment, null pointers -> Q8_0_EINVAL. */
int q8_0_probe_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Measurement probe (the fixed cost of a launch, part of the decode ceiling:
 * a token's work is a chain of short dispatches, "Part 6: GPU 加速",
 * section 4n): an empty kernel of `workgroups` workgroups of 256 lanes that
 * exits at once.  sink: device uint32, never written.
 * Errors: workgroups outside [1, 65536], null sink -> Q8_0_EINVAL. */
int q8_0_probe_launch(int32_t workgroups, uint32_t *sink, hipStream_t stream);

/* Measurement probe (the matrix-core ceiling that the int8 GEMM kernels are
 * reported against beside the 5 POPS peak): 512 workgroups of 4 waves, each
 * wave `iters` rounds of 4 independent v_mfma_i32_32x32x32_i8, i.e.
 * 512 * 4 * 4 * 65536 * iters integer operations.  sink as above.
 * Errors: iters < 1, null sink -> Q8_0_EINVAL. */
int q8_0_probe_mfma_i8(int32_t iters, uint32_t *sink, hipStream_t stream);

/* Measurement probe (the ceiling of the prefill GEMM's own formulation):
 * the GEMM's per-tile-block instruction mix on registers only, no memory
 * traffic, in the same grid and with the same int8 work per round as
 * q8_0_probe_mfma_i8 (so the rates compare directly):
 *   mix 0: the int8 MFMA alone;
 *   mix 1: per 32x32 tile and block, the biased int8 MFMA, the f16 MFMA of
 *          the scale outer product, the f16 MFMA that removes the bias, and
 *          16 fp32 fmas (the four-tile kernel's tile step);
 *   mix 2: the int8 MFMA and the scale MFMA, with the int->float
 *          conversion as 16 VALU converts before the 16 fmas.
 * sink as above.  Errors: iters < 1, mix outside 0..2, null sink ->
 * Q8_0_EINVAL. */
int q8_0_probe_mfma_mix(int32_t iters, int32_t mix, uint32_t *sink, hipStream_t stream);

/* Debug aid of the race tests (a kernel that reads LDS it has not written,
 * or reads it before the barrier that publishes it, computes from whatever
 * the LDS held; the pages record such bugs -- a barrier of too narrow a scope,
 * "Part 6: GPU 加速", section 4n, and threadgroup memory allocated too small,
 * caught by a debug layer, section 4p): fills the whole LDS of every compute
 * unit with `pattern`, so that the next launch on `stream` starts with every
 * LDS byte holding it.  Running a kernel after two different patterns and
 * comparing its outputs bit for bit shows whether it reads unwritten LDS.
 * Stream-ordered; allocates nothing.  Errors: no device -> Q8_0_ENODEV. */
int q8_0_debug_poison_lds(uint32_t pattern, hipStream_t stream);

/* LDS dwords each workgroup of q8_0_debug_read_lds copies out. */
#define Q8_0_DEBUG_LDS_DWORDS 8192

/* The check that q8_0_debug_poison_lds reaches later launches: `workgroups`
 * workgroups each copy the Q8_0_DEBUG_LDS_DWORDS dwords of LDS they were
 * given, without writing them first, to seen[w * Q8_0_DEBUG_LDS_DWORDS ...].
 *   seen      : device uint32, workgroups * Q8_0_DEBUG_LDS_DWORDS, written.
 *   workgroups: 1 .. 4096.
 * Errors: null or unaligned seen, workgroups out of range -> Q8_0_EINVAL. */
int q8_0_debug_read_lds(uint32_t *seen, int32_t workgroups, hipStream_t stream);

/* Static description of a status code. */
const char *q8_0_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q8_0_H */
