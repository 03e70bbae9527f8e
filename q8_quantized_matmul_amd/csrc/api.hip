// api.hip -- the C ABI of include/q8_0.h: host-side argument checks, kernel
// selection and launches on the caller's stream.  Nothing here allocates
// device memory; every buffer, including scratch, belongs to the caller, except
// the routing tables of q8_0_moe_grouped_noalloc, which live in a static
// device array of the library (moe.hip).
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "launch.h"
#include "q8_0.h"

static_assert(Q8_0_MOE_STATIC_SCRATCH_BYTES == q8::kMoeStaticScratchBytes,
              "header and library agree on the static routing scratch");
static_assert(Q8_0_DEBUG_LDS_DWORDS == q8::kDebugLdsDwords,
              "header and library agree on the LDS read-back size");

namespace {

// Regimes by token count (measured on 4096->2048, 2048->4096, 4096->1024,
// 4096->512 and 1024->32768, graph-replayed calls): the weight-streaming
// matvec below 12 tokens, the skinny matrix-core kernel (one launch, split-K
// inside it) from 12 to 64 and, for shapes skinny_many_tokens accepts, up to
// 256; the LDS-tiled GEMM above.  Rows the matvec
// cannot take (pair counts that are neither a power of two below 64 nor a
// multiple of 64, e.g. in_dim 1536 or 7168) go to the skinny kernel from two
// tokens: the generic kernel's cost grows by 3-4 us per token there.
constexpr int64_t kSkinnyMinTokens = 12;
// The shared list launch takes the matvec items, so below the skinny regime.
constexpr int64_t kListMaxTokens = kSkinnyMinTokens - 1;
constexpr int32_t kMaxExperts = 8192;
constexpr int kMaxDevices = 64;

// 1 = gfx950, -1 = other architecture, 0 = not looked at yet.
std::atomic<int> g_device_ok[kMaxDevices];

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q8_0_ENODEV;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q8_0_ENODEV;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? Q8_0_OK : Q8_0_ENODEV;
}

int status_of(hipError_t e) { return e == hipSuccess ? Q8_0_OK : Q8_0_ELAUNCH; }

// Plan for q8_0_matmul: which kernel, how many K splits.
struct Plan {
  int32_t variant;
  int32_t split;
};

bool matvec_ok(int64_t in_dim) { return q8::matvec_shape(in_dim, nullptr); }

Plan make_plan(int64_t in_dim, int64_t out_dim, int64_t n_tok, size_t ws_bytes, bool fast_align) {
  Plan p{Q8_0_KERNEL_GENERIC, 1};
  if (!fast_align) return p;
  const bool skinny_regime =
      (n_tok <= q8::kSkinnyMaxTokens && (n_tok >= kSkinnyMinTokens || (n_tok >= 2 && !matvec_ok(in_dim)))) ||
      q8::skinny_many_tokens(in_dim, out_dim, n_tok);
  if (skinny_regime && q8::skinny_supported(in_dim, n_tok)) {
    p.variant = Q8_0_KERNEL_SKINNY;
    int split = q8::skinny_split_ok(in_dim, out_dim, n_tok, 2) ? q8::skinny_auto_split(in_dim, out_dim, n_tok) : 1;
    while (split > 1 && q8::skinny_workspace_bytes(out_dim, n_tok, split) > ws_bytes) --split;
    p.split = split;
  } else if (n_tok > q8::kSkinnyMaxTokens && q8::gemm_supported(in_dim)) {
    p.variant = Q8_0_KERNEL_MFMA;
    int split = q8::gemm_auto_split(in_dim, out_dim, n_tok);
    while (split > 1 && q8::gemm_workspace_bytes(out_dim, n_tok, split) > ws_bytes) --split;
    p.split = split;
  } else if (matvec_ok(in_dim)) {
    p.variant = Q8_0_KERNEL_MATVEC;
  }
  return p;
}

// The plan for a forced variant and split-K count (0 = automatic).
int forced_plan(int64_t in_dim, int64_t out_dim, int64_t n_tok, size_t ws_bytes, bool fast_align,
                int32_t variant, int32_t split_k, Plan *out) {
  if (split_k < 0 || variant < 0 || variant > Q8_0_KERNEL_SKINNY) return Q8_0_EINVAL;
  Plan p = make_plan(in_dim, out_dim, n_tok, ws_bytes, fast_align);
  if (variant != Q8_0_KERNEL_AUTO) {
    if (variant != Q8_0_KERNEL_GENERIC && !fast_align) return Q8_0_EINVAL;
    if (variant == Q8_0_KERNEL_MATVEC && !matvec_ok(in_dim)) return Q8_0_EINVAL;
    if (variant == Q8_0_KERNEL_MFMA && !q8::gemm_supported(in_dim)) return Q8_0_EINVAL;
    if (variant == Q8_0_KERNEL_SKINNY && !q8::skinny_supported(in_dim, n_tok)) return Q8_0_EINVAL;
    if (variant != p.variant) p.split = 1;
    p.variant = variant;
  }
  if (split_k > 0) {
    if (p.variant != Q8_0_KERNEL_MFMA && p.variant != Q8_0_KERNEL_SKINNY && split_k != 1)
      return Q8_0_EINVAL;
    p.split = split_k;
  }
  if (p.variant == Q8_0_KERNEL_SKINNY && !q8::skinny_split_ok(in_dim, out_dim, n_tok, p.split)) return Q8_0_EINVAL;
  *out = p;
  return Q8_0_OK;
}

size_t plan_workspace_bytes(const Plan &p, int64_t out_dim, int64_t n_tok) {
  if (p.variant == Q8_0_KERNEL_SKINNY) return q8::skinny_workspace_bytes(out_dim, n_tok, p.split);
  if (p.variant == Q8_0_KERNEL_MFMA) return q8::gemm_workspace_bytes(out_dim, n_tok, p.split);
  return 0;
}

int validate_matmul(const float *out, const void *w, int64_t in_dim, int64_t out_dim,
                    const void *x_q, int64_t n_tok) {
  if (in_dim < 0 || out_dim < 0 || n_tok < 0) return Q8_0_EINVAL;
  if (in_dim % Q8_0_BLOCK_ELEMS != 0) return Q8_0_EINVAL;
  if (n_tok == 0 || out_dim == 0) return Q8_0_OK;
  if (in_dim == 0) return Q8_0_EINVAL;
  if (!out || !w || !x_q) return Q8_0_EINVAL;
  if (!aligned(out, 4) || !aligned(w, 2) || !aligned(x_q, 2)) return Q8_0_EALIGN;
  return Q8_0_OK;
}

int run_matmul(float *out, int32_t *blocksums, const void *w, int64_t in_dim, int64_t out_dim,
               const void *x_q, int64_t n_tok, void *workspace, size_t workspace_bytes,
               int32_t variant, int32_t split_k, hipStream_t stream) {
  int st = validate_matmul(out, w, in_dim, out_dim, x_q, n_tok);
  if (st != Q8_0_OK || n_tok == 0 || out_dim == 0) return st;
  if (workspace == nullptr) workspace_bytes = 0;
  if (workspace && !aligned(workspace, 16)) return Q8_0_EALIGN;
  const bool fast_align = aligned(w, 4) && aligned(x_q, 4);
  Plan p;
  if ((st = forced_plan(in_dim, out_dim, n_tok, workspace_bytes, fast_align, variant, split_k, &p)) !=
      Q8_0_OK)
    return st;
  if (plan_workspace_bytes(p, out_dim, n_tok) > workspace_bytes) return Q8_0_EWORKSPACE;
  if ((st = check_device()) != Q8_0_OK) return st;
  switch (p.variant) {
    case Q8_0_KERNEL_MFMA:
      return status_of(q8::launch_gemm(out, blocksums, w, in_dim, out_dim, x_q, n_tok, p.split,
                                       workspace, stream));
    case Q8_0_KERNEL_SKINNY:
      return status_of(q8::launch_skinny(out, blocksums, w, in_dim, out_dim, x_q, n_tok, p.split,
                                         workspace, stream));
    case Q8_0_KERNEL_MATVEC:
      return status_of(q8::launch_matvec(out, blocksums, w, in_dim, out_dim, x_q, n_tok, stream));
    default:
      return status_of(q8::launch_generic(out, blocksums, w, in_dim, out_dim, x_q, n_tok, stream));
  }
}

// Checks of the grouped call's arguments other than the workspace.  Returns
// Q8_0_OK with *empty set when there is nothing to do.
int validate_moe(const float *out, const void *const *expert_w, int32_t n_expert, int64_t in_dim,
                 int64_t out_dim, const int32_t *selected, int32_t n_used, const void *x_q,
                 int32_t x_rows, int64_t n_tok, bool *empty) {
  *empty = true;
  if (n_expert < 1 || n_expert > kMaxExperts || n_used < 1 || n_tok < 0 || in_dim < 0 ||
      out_dim < 0 || (x_rows != 0 && x_rows != 1) || in_dim % Q8_0_BLOCK_ELEMS != 0)
    return Q8_0_EINVAL;
  if (n_tok * (int64_t)n_used > INT32_MAX) return Q8_0_EINVAL;
  if (n_tok == 0 || out_dim == 0) return Q8_0_OK;
  if (in_dim == 0) return Q8_0_EINVAL;
  if (!out || !expert_w || !selected || !x_q) return Q8_0_EINVAL;
  if (!aligned(out, 4) || !aligned(selected, 4) || !aligned(expert_w, 8) || !aligned(x_q, 2))
    return Q8_0_EALIGN;
  *empty = false;
  return Q8_0_OK;
}

int launch_moe_checked(float *out, int32_t *blocksums, const void *const *expert_w,
                       int32_t n_expert, int64_t in_dim, int64_t out_dim,
                       const int32_t *selected, int32_t n_used, const void *x_q, int32_t x_rows,
                       int64_t n_tok, int32_t *ws, int32_t *invalid_out, hipStream_t stream) {
  // Expert matrices are only known on the device; the fast kernel needs the
  // x rows and every expert base dword aligned, which torch allocations and
  // even-block-count row slices satisfy.  x_q alignment is checked here.
  const bool fast = aligned(x_q, 4) && matvec_ok(in_dim);
  return status_of(q8::launch_moe(out, blocksums, expert_w, n_expert, in_dim, out_dim, selected,
                                  n_used, x_q, x_rows, n_tok, ws, fast, stream, invalid_out));
}

int run_moe(float *out, int32_t *blocksums, const void *const *expert_w, int32_t n_expert,
            int64_t in_dim, int64_t out_dim, const int32_t *selected, int32_t n_used,
            const void *x_q, int32_t x_rows, int64_t n_tok, void *workspace,
            size_t workspace_bytes, hipStream_t stream) {
  bool empty = true;
  int st = validate_moe(out, expert_w, n_expert, in_dim, out_dim, selected, n_used, x_q, x_rows,
                        n_tok, &empty);
  if (st != Q8_0_OK || empty) return st;
  if (!workspace || workspace_bytes < q8_0_moe_workspace_bytes(n_tok, n_used, n_expert))
    return Q8_0_EWORKSPACE;
  if (!aligned(workspace, 16)) return Q8_0_EALIGN;
  if ((st = check_device()) != Q8_0_OK) return st;
  return launch_moe_checked(out, blocksums, expert_w, n_expert, in_dim, out_dim, selected, n_used,
                            x_q, x_rows, n_tok, static_cast<int32_t *>(workspace), nullptr,
                            stream);
}

// q8_0_moe_grouped_noalloc: the routing tables live in the library's static
// device array (moe.hip) instead of caller workspace.
int run_moe_noalloc(float *out, const void *const *expert_w, int32_t n_expert, int64_t in_dim,
                    int64_t out_dim, const int32_t *selected, int32_t n_used, const void *x_q,
                    int32_t x_rows, int64_t n_tok, int32_t *n_invalid, hipStream_t stream) {
  bool empty = true;
  int st = validate_moe(out, expert_w, n_expert, in_dim, out_dim, selected, n_used, x_q, x_rows,
                        n_tok, &empty);
  if (st != Q8_0_OK || empty) return st;
  if (n_invalid && !aligned(n_invalid, 4)) return Q8_0_EALIGN;
  if (q8_0_moe_workspace_bytes(n_tok, n_used, n_expert) > Q8_0_MOE_STATIC_SCRATCH_BYTES)
    return Q8_0_EWORKSPACE;
  if ((st = check_device()) != Q8_0_OK) return st;
  int32_t *scratch = nullptr;
  if (q8::moe_static_scratch(&scratch) != hipSuccess || !scratch) return Q8_0_ENODEV;
  return launch_moe_checked(out, nullptr, expert_w, n_expert, in_dim, out_dim, selected, n_used,
                            x_q, x_rows, n_tok, scratch, n_invalid, stream);
}

// Byte layout of the q8_0_moe_ffn workspace: routing ints, then mid, mid_q
// and y, each 256-byte aligned.
struct FfnLayout {
  size_t route, mid, mid_q, y, total;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

FfnLayout ffn_layout(int64_t n_tok, int32_t n_used, int32_t n_expert, int64_t d_model,
                     int64_t d_ff) {
  FfnLayout L{};
  const int64_t pairs = n_tok * n_used;
  L.route = 0;
  L.mid = align256(q8_0_moe_workspace_bytes(n_tok, n_used, n_expert));
  L.mid_q = L.mid + align256((size_t)(pairs * d_ff) * sizeof(float));
  L.y = L.mid_q + align256((size_t)(pairs * (d_ff / Q8_0_BLOCK_ELEMS) * Q8_0_BLOCK_BYTES));
  L.total = L.y + align256((size_t)(pairs * d_model) * sizeof(float));
  return L;
}

int run_moe_ffn(const q8_0_moe_ffn_args *a, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (!a) return Q8_0_EINVAL;
  if (a->n_expert < 1 || a->n_expert > kMaxExperts || a->n_used < 1 || a->n_tok < 0 ||
      a->d_model <= 0 || a->d_ff <= 0)
    return Q8_0_EINVAL;
  if (a->n_tok * (int64_t)a->n_used > INT32_MAX) return Q8_0_EINVAL;
  if (!q8::matvec_pair_ok(a->d_model) || !matvec_ok(a->d_ff)) return Q8_0_EINVAL;
  if (a->n_tok == 0) return Q8_0_OK;
  if (!a->out || !a->gate_w || !a->up_w || !a->down_w || !a->selected || !a->weights || !a->x_q)
    return Q8_0_EINVAL;
  if (!aligned(a->out, 4) || !aligned(a->gate_w, 8) || !aligned(a->up_w, 8) ||
      !aligned(a->down_w, 8) || !aligned(a->selected, 4) || !aligned(a->weights, 4) ||
      !aligned(a->x_q, 4) || (a->mid && !aligned(a->mid, 16)) ||
      (a->mid_q && !aligned(a->mid_q, 4)) || (a->y && !aligned(a->y, 4)))
    return Q8_0_EALIGN;
  const FfnLayout L = ffn_layout(a->n_tok, a->n_used, a->n_expert, a->d_model, a->d_ff);
  if (!workspace || workspace_bytes < L.total) return Q8_0_EWORKSPACE;
  if (!aligned(workspace, 256)) return Q8_0_EALIGN;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  q8::MoeFfn f{};
  f.out = a->out;
  f.gate_w = a->gate_w;
  f.up_w = a->up_w;
  f.down_w = a->down_w;
  f.n_expert = a->n_expert;
  f.n_used = a->n_used;
  f.d_model = a->d_model;
  f.d_ff = a->d_ff;
  f.n_tok = a->n_tok;
  f.selected = a->selected;
  f.weights = a->weights;
  f.x_q = a->x_q;
  f.clamp = a->clamp;
  f.mid = a->mid ? a->mid : reinterpret_cast<float *>(ws + L.mid);
  f.mid_q = a->mid_q ? a->mid_q : static_cast<void *>(ws + L.mid_q);
  f.y = a->y ? a->y : reinterpret_cast<float *>(ws + L.y);
  return status_of(q8::launch_moe_ffn(f, reinterpret_cast<int32_t *>(ws), stream));
}

// How q8_0_matmul_list runs one item.
struct ListPlan {
  bool active;      // out_dim > 0: the item produces output
  bool prequant;    // x is quantized into x_q by a launch of its own first
  bool in_list;     // the matvec runs inside the shared list launch
  bool fused;       // ... and quantizes x inside that launch
};

int plan_list_item(const q8_0_matmul_item &it, int64_t n_tok, ListPlan *lp) {
  *lp = ListPlan{};
  if (it.in_dim < 0 || it.out_dim < 0 || it.in_dim % Q8_0_BLOCK_ELEMS != 0) return Q8_0_EINVAL;
  if (it.in_dim == 0 && it.out_dim > 0) return Q8_0_EINVAL;
  if (it.out_dim > 0 && (!it.out || !it.w || (!it.x && !it.x_q))) return Q8_0_EINVAL;
  if ((it.out && !aligned(it.out, 4)) || (it.w && !aligned(it.w, 2)) ||
      (it.x_q && !aligned(it.x_q, 2)) || (it.x && !aligned(it.x, 4)))
    return Q8_0_EALIGN;
  if (it.in_dim == 0) return Q8_0_OK;  // nothing to quantize or multiply
  lp->active = it.out_dim > 0;
  if (!lp->active) {  // no output: only the requested x_q, if any
    lp->prequant = it.x && it.x_q;
    return Q8_0_OK;
  }
  const bool w4 = aligned(it.w, 4);
  if (it.x && w4 && aligned(it.x, 16) && (!it.x_q || aligned(it.x_q, 4))) {
    const Plan p = make_plan(it.in_dim, it.out_dim, n_tok, 0, true);
    lp->fused = p.variant == Q8_0_KERNEL_MATVEC && q8::list_item_ok(it.in_dim) &&
                q8::list_item_fusable(it.in_dim, n_tok);
  }
  if (lp->fused) {
    lp->in_list = true;
    return Q8_0_OK;
  }
  if (it.x) {
    if (!it.x_q) return Q8_0_EINVAL;
    lp->prequant = true;
  }
  const Plan p = make_plan(it.in_dim, it.out_dim, n_tok, 0, w4 && aligned(it.x_q, 4));
  lp->in_list = p.variant == Q8_0_KERNEL_MATVEC && q8::list_item_ok(it.in_dim) &&
                n_tok <= kListMaxTokens;
  return Q8_0_OK;
}

int run_list(const q8_0_matmul_item *items, int32_t n_items, int64_t n_tok, hipStream_t stream) {
  if (!items || n_items < 1 || n_items > Q8_0_LIST_MAX || n_tok < 0) return Q8_0_EINVAL;
  ListPlan lp[Q8_0_LIST_MAX];
  bool work = false;
  for (int32_t i = 0; i < n_items; ++i) {
    const int st = plan_list_item(items[i], n_tok, &lp[i]);
    if (st != Q8_0_OK) return st;
    work = work || lp[i].active || lp[i].prequant;
  }
  if (n_tok == 0 || !work) return Q8_0_OK;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  for (int32_t i = 0; i < n_items; ++i) {
    if (!lp[i].prequant) continue;
    if ((st = q8_0_quantize_act(items[i].x_q, items[i].x, n_tok, items[i].in_dim, stream)) != Q8_0_OK)
      return st;
  }
  q8::ListItem batch[Q8_0_LIST_MAX];
  int n_batch = 0;
  for (int32_t i = 0; i < n_items; ++i) {
    if (!lp[i].in_list) continue;
    const q8_0_matmul_item &it = items[i];
    batch[n_batch++] = q8::ListItem{it.out, it.w, lp[i].fused ? it.x : nullptr, it.x_q, it.in_dim,
                                    it.out_dim};
  }
  if (n_batch > 0 && (st = status_of(q8::launch_matvec_list(batch, n_batch, n_tok, stream))) != Q8_0_OK)
    return st;
  for (int32_t i = 0; i < n_items; ++i) {
    if (!lp[i].active || lp[i].in_list) continue;
    const q8_0_matmul_item &it = items[i];
    st = run_matmul(it.out, nullptr, it.w, it.in_dim, it.out_dim, it.x_q, n_tok, nullptr, 0,
                    Q8_0_KERNEL_AUTO, 0, stream);
    if (st != Q8_0_OK) return st;
  }
  return Q8_0_OK;
}

}  // namespace

extern "C" {

int q8_0_quantize_act(void *x_q, const float *x, int64_t n_tok, int64_t in_dim,
                      hipStream_t stream) {
  if (n_tok < 0 || in_dim < 0 || in_dim % Q8_0_BLOCK_ELEMS != 0) return Q8_0_EINVAL;
  if (n_tok == 0 || in_dim == 0) return Q8_0_OK;
  if (!x_q || !x) return Q8_0_EINVAL;
  if (!aligned(x, 4) || !aligned(x_q, 2)) return Q8_0_EALIGN;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  const bool fast = aligned(x, 16) && aligned(x_q, 4) && (in_dim / Q8_0_BLOCK_ELEMS) % 2 == 0;
  return status_of(q8::launch_quantize(x_q, x, n_tok, in_dim, fast, stream));
}

size_t q8_0_matmul_workspace_bytes(int64_t in_dim, int64_t out_dim, int64_t n_tok) {
  return q8_0_matmul_debug_workspace_bytes(in_dim, out_dim, n_tok, Q8_0_KERNEL_AUTO, 0);
}

size_t q8_0_matmul_debug_workspace_bytes(int64_t in_dim, int64_t out_dim, int64_t n_tok,
                                         int32_t variant, int32_t split_k) {
  if (in_dim <= 0 || out_dim <= 0 || n_tok <= 0 || in_dim % Q8_0_BLOCK_ELEMS != 0) return 0;
  Plan p;
  if (forced_plan(in_dim, out_dim, n_tok, SIZE_MAX, true, variant, split_k, &p) != Q8_0_OK) return 0;
  return plan_workspace_bytes(p, out_dim, n_tok);
}

int q8_0_matmul(float *out, const void *w, int64_t in_dim, int64_t out_dim, const void *x_q,
                int64_t n_tok, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_matmul(out, nullptr, w, in_dim, out_dim, x_q, n_tok, workspace, workspace_bytes,
                    Q8_0_KERNEL_AUTO, 0, stream);
}

int q8_0_matmul_debug(float *out, int32_t *blocksums, const void *w, int64_t in_dim,
                      int64_t out_dim, const void *x_q, int64_t n_tok, void *workspace,
                      size_t workspace_bytes, int32_t variant, int32_t split_k,
                      hipStream_t stream) {
  if (blocksums && !aligned(blocksums, 4)) return Q8_0_EALIGN;
  return run_matmul(out, blocksums, w, in_dim, out_dim, x_q, n_tok, workspace, workspace_bytes,
                    variant, split_k, stream);
}

int q8_0_matmul_plan(int64_t in_dim, int64_t out_dim, int64_t n_tok, size_t workspace_bytes,
                     int32_t *variant, int32_t *split_k) {
  if (in_dim < 0 || out_dim < 0 || n_tok < 0 || in_dim % Q8_0_BLOCK_ELEMS != 0)
    return Q8_0_EINVAL;
  Plan p = make_plan(in_dim, out_dim, n_tok, workspace_bytes, true);
  if (variant) *variant = p.variant;
  if (split_k) *split_k = p.split;
  return Q8_0_OK;
}

size_t q8_0_moe_workspace_bytes(int64_t n_tok, int32_t n_used, int32_t n_expert) {
  if (n_tok < 0 || n_used < 1 || n_expert < 1) return 0;
  const q8::MoeLayout L = q8::moe_layout(n_tok, n_used, n_expert);
  return (size_t)((L.total_ints * (int64_t)sizeof(int32_t) + 255) / 256 * 256);
}

int q8_0_moe_grouped(float *out, const void *const *expert_w, int32_t n_expert, int64_t in_dim,
                     int64_t out_dim, const int32_t *selected, int32_t n_used, const void *x_q,
                     int32_t x_rows, int64_t n_tok, void *workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return run_moe(out, nullptr, expert_w, n_expert, in_dim, out_dim, selected, n_used, x_q, x_rows,
                 n_tok, workspace, workspace_bytes, stream);
}

int q8_0_moe_grouped_noalloc(float *out, const void *const *expert_w, int32_t n_expert,
                             int64_t in_dim, int64_t out_dim, const int32_t *selected,
                             int32_t n_used, const void *x_q, int32_t x_rows, int64_t n_tok,
                             int32_t *n_invalid, hipStream_t stream) {
  return run_moe_noalloc(out, expert_w, n_expert, in_dim, out_dim, selected, n_used, x_q, x_rows,
                         n_tok, n_invalid, stream);
}

int q8_0_moe_grouped_debug(float *out, int32_t *blocksums, const void *const *expert_w,
                           int32_t n_expert, int64_t in_dim, int64_t out_dim,
                           const int32_t *selected, int32_t n_used, const void *x_q,
                           int32_t x_rows, int64_t n_tok, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (blocksums && !aligned(blocksums, 4)) return Q8_0_EALIGN;
  return run_moe(out, blocksums, expert_w, n_expert, in_dim, out_dim, selected, n_used, x_q,
                 x_rows, n_tok, workspace, workspace_bytes, stream);
}

size_t q8_0_moe_ffn_workspace_bytes(int64_t n_tok, int32_t n_used, int32_t n_expert,
                                    int64_t d_model, int64_t d_ff) {
  if (n_tok < 0 || n_used < 1 || n_expert < 1 || d_model <= 0 || d_ff <= 0) return 0;
  return ffn_layout(n_tok, n_used, n_expert, d_model, d_ff).total;
}

int q8_0_moe_ffn(const q8_0_moe_ffn_args *args, void *workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return run_moe_ffn(args, workspace, workspace_bytes, stream);
}

int q8_0_matmul_list(const q8_0_matmul_item *items, int32_t n_items, int64_t n_tok,
                     hipStream_t stream) {
  return run_list(items, n_items, n_tok, stream);
}

int q8_0_probe_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || bytes > (size_t)INT64_MAX)
    return Q8_0_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return Q8_0_EINVAL;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  return status_of(q8::launch_probe_read(buf, (int64_t)bytes, sink, stream));
}

int q8_0_probe_launch(int32_t workgroups, uint32_t *sink, hipStream_t stream) {
  if (workgroups < 1 || workgroups > 65536 || !sink || !aligned(sink, 4)) return Q8_0_EINVAL;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  return status_of(q8::launch_probe_launch(workgroups, sink, stream));
}

int q8_0_probe_mfma_i8(int32_t iters, uint32_t *sink, hipStream_t stream) {
  if (iters < 1 || !sink || !aligned(sink, 4)) return Q8_0_EINVAL;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  return status_of(q8::launch_probe_mfma(iters, sink, stream));
}

int q8_0_probe_mfma_mix(int32_t iters, int32_t mix, uint32_t *sink, hipStream_t stream) {
  if (iters < 1 || mix < 0 || mix > 2 || !sink || !aligned(sink, 4)) return Q8_0_EINVAL;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  return status_of(q8::launch_probe_mix(iters, mix, sink, stream));
}

int q8_0_debug_poison_lds(uint32_t pattern, hipStream_t stream) {
  int st = check_device();
  if (st != Q8_0_OK) return st;
  return status_of(q8::launch_debug_poison_lds(pattern, stream));
}

int q8_0_debug_read_lds(uint32_t *seen, int32_t workgroups, hipStream_t stream) {
  if (!seen || !aligned(seen, 4) || workgroups < 1 || workgroups > 4096) return Q8_0_EINVAL;
  int st = check_device();
  if (st != Q8_0_OK) return st;
  return status_of(q8::launch_debug_read_lds(seen, workgroups, stream));
}

const char *q8_0_strerror(int status) {
  switch (status) {
    case Q8_0_OK: return "ok";
    case Q8_0_EINVAL: return "invalid argument (size, mode or null pointer)";
    case Q8_0_EALIGN: return "pointer alignment too small";
    case Q8_0_ELAUNCH: return "kernel launch failed";
    case Q8_0_EWORKSPACE: return "workspace missing or too small";
    case Q8_0_ENODEV: return "no gfx950 device current";
    default: return "unknown status";
  }
}

}  // extern "C"
