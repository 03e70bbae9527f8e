// moe.hip -- routing preparation for the grouped expert matmul.
//
// The pages' routed-MoE call takes, per token, the list of selected experts
// ("Part 6: 代码走读", trace 5, ds4_gpu_routed_moe_one_tensor) and runs each
// expert's projection for its tokens.  To stream every touched expert's
// weights once, the (token, slot) pairs are regrouped expert-major on the GPU
// with no host round trip:
//   counts[e]   pairs routed to expert e
//   offsets[e]  exclusive prefix sum of counts (offsets[n_expert] = valid pairs)
//   pairs[...]  pair ids t*n_used + j, grouped by expert, ascending within an
//               expert (a stable counting sort, so the order is deterministic)
// Pairs whose id is outside [0, n_expert) are counted in workspace[0] and
// their output rows are filled with NaN.
//
// One workgroup of 1024 lanes does it: LDS atomics count (integer, so the
// result is order independent), in-wave scans and the 16 wave totals build
// the offsets, and each 1024-pair chunk is scattered with in-wave ranks from
// ballots (lanes sharing an expert id are found bit by bit) and waves taking
// their turn in index order.  The ids are read from memory once, in the
// counting pass, and kept in LDS.
#include <mutex>

#include "launch.h"
#include "q8_device.h"

namespace q8 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kHeaderInts = 16;
constexpr int kKeyChunk = 4096;  // expert ids staged in LDS per scatter pass

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const int32_t *__restrict__ selected, int64_t n_pairs, int32_t n_expert, int32_t key_bits,
    int32_t *__restrict__ ws, int64_t off_counts, int64_t off_offsets, int64_t off_pairs,
    float *__restrict__ out, int64_t out_dim, int32_t *__restrict__ invalid_out) {
  extern __shared__ int32_t lds[];
  int32_t *running = lds;                  // [n_expert]
  int32_t *keys = lds + n_expert;          // [kKeyChunk]
  int32_t *wave_sum = keys + kKeyChunk;    // [kRouteWaves]
  int32_t *slot_base = wave_sum + kRouteWaves;  // [kRouteWaves][64]
  __shared__ int32_t invalid;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < n_expert; e += kRouteThreads) running[e] = 0;
  if (tid == 0) invalid = 0;
  __syncthreads();

  // Count; the first chunk of ids stays in LDS for the scatter.
  for (int64_t i = tid; i < n_pairs; i += kRouteThreads) {
    const int32_t e = selected[i];
    if (i < kKeyChunk) keys[i] = e;
    if (e >= 0 && e < n_expert) atomicAdd(&running[e], 1);
    else atomicAdd(&invalid, 1);
  }
  __syncthreads();

  // counts and exclusive offsets; each lane owns a contiguous run of experts.
  const int32_t per = (n_expert + kRouteThreads - 1) / kRouteThreads;
  const int32_t e0 = min(tid * per, n_expert);
  const int32_t e1 = min(e0 + per, n_expert);
  int32_t local = 0;
  for (int32_t e = e0; e < e1; ++e) local += running[e];
  const int32_t incl = wave_inclusive_scan(local, lane);
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int32_t base = incl - local, total = 0;
  for (int w = 0; w < kRouteWaves; ++w) {
    const int32_t t = wave_sum[w];
    if (w < wave) base += t;
    total += t;
  }
  for (int32_t e = e0; e < e1; ++e) {
    const int32_t c = running[e];
    ws[off_counts + e] = c;
    ws[off_offsets + e] = base;
    running[e] = base;  // becomes the next free slot of expert e
    base += c;
  }
  if (tid == 0) {
    ws[off_offsets + n_expert] = total;
    ws[0] = invalid;
    if (invalid_out) *invalid_out = invalid;
  }
  __syncthreads();

  // Stable scatter, 1024 pairs at a time: each wave ranks its lanes among
  // those sharing an expert id, then the waves take slots in index order.
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t chunk = 0; chunk < n_pairs; chunk += kRouteThreads) {
    if (chunk > 0 && chunk % kKeyChunk == 0) {
      // Stage the next kKeyChunk ids (the barrier ending the previous chunk
      // has retired every read of the old ones).
      const int len = (int)min<int64_t>(kKeyChunk, n_pairs - chunk);
      for (int j = tid; j < len; j += kRouteThreads) keys[j] = selected[chunk + j];
      __syncthreads();
    }
    const int64_t i = chunk + tid;
    const int32_t e = i < n_pairs ? keys[i % kKeyChunk] : -1;
    const bool valid = e >= 0 && e < n_expert;
    const uint32_t key = valid ? (uint32_t)e : (uint32_t)n_expert;
    uint64_t peers = __ballot(1);
    for (int bit = 0; bit < key_bits; ++bit) {
      const bool set = (key >> bit) & 1u;
      const uint64_t b = __ballot(set);
      peers &= set ? b : ~b;
    }
    const int rank = __popcll(peers & below);
    const int leader = __ffsll((unsigned long long)peers) - 1;
    for (int w = 0; w < kRouteWaves; ++w) {
      if (wave == w && valid && rank == 0) {
        slot_base[w * 64 + lane] = running[e];
        running[e] += __popcll(peers);
      }
      __syncthreads();
    }
    if (valid) ws[off_pairs + slot_base[wave * 64 + leader] + rank] = (int32_t)i;
    __syncthreads();
  }

  // Rows of pairs with an invalid expert id become NaN (error path only).
  if (invalid > 0) {
    for (int64_t i = 0; i < n_pairs; ++i) {
      const int32_t e = selected[i];
      if (e < 0 || e >= n_expert) {
        for (int64_t o = tid; o < out_dim; o += kRouteThreads)
          out[i * out_dim + o] = __builtin_nanf("");
      }
    }
  }
}

}  // namespace

MoeLayout moe_layout(int64_t n_tok, int32_t n_used, int32_t n_expert) {
  MoeLayout L;
  L.counts = kHeaderInts;
  L.offsets = L.counts + n_expert;
  L.pairs = L.offsets + n_expert + 1;
  L.total_ints = L.pairs + n_tok * n_used;
  return L;
}

size_t moe_route_lds_bytes(int32_t n_expert) {
  return sizeof(int32_t) * ((size_t)n_expert + kKeyChunk + kRouteWaves + kRouteWaves * 64);
}

hipError_t launch_moe_route(const int32_t *selected, int64_t n_tok, int32_t n_used,
                            int32_t n_expert, int32_t *ws, float *nan_rows, int64_t nan_dim,
                            hipStream_t s, int32_t *invalid_out) {
  const MoeLayout L = moe_layout(n_tok, n_used, n_expert);
  const int64_t n_pairs = n_tok * n_used;
  int key_bits = 1;
  while ((1ll << key_bits) <= (int64_t)n_expert) ++key_bits;  // n_expert itself is the sentinel
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), moe_route_lds_bytes(n_expert),
                     s, selected, n_pairs, n_expert, key_bits, ws, L.counts, L.offsets, L.pairs,
                     nan_rows, nan_dim, invalid_out);
  return hipGetLastError();
}

hipError_t launch_moe(float *out, int32_t *blocksums, const void *const *expert_w,
                      int32_t n_expert, int64_t in_dim, int64_t out_dim,
                      const int32_t *selected, int32_t n_used, const void *x_q, int32_t x_rows,
                      int64_t n_tok, int32_t *ws, bool fast, hipStream_t s,
                      int32_t *invalid_out) {
  const MoeLayout L = moe_layout(n_tok, n_used, n_expert);
  hipError_t err =
      launch_moe_route(selected, n_tok, n_used, n_expert, ws, out, out_dim, s, invalid_out);
  if (err != hipSuccess) return err;
  if (fast) {
    return launch_matvec_grouped(out, blocksums, expert_w, n_expert, in_dim, out_dim, x_q, x_rows,
                                 n_used, ws + L.counts, ws + L.offsets, ws + L.pairs, s);
  }
  return launch_generic_grouped(out, blocksums, expert_w, n_expert, in_dim, out_dim, selected,
                                n_used, x_q, x_rows, n_tok, s);
}

// ---- Routing tables without caller workspace.
//
// For callers that cannot allocate device memory, q8_0_moe_grouped_noalloc
// keeps the routing tables (the same layout as the caller workspace of
// q8_0_moe_grouped) in this file-scope device array.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code the
// array's name is only a host-side stand-in for the symbol, never a device
// address: the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is passed to
// kernels.  Every call on one GPU shares the array; the routing kernel writes
// every word a call reads before reading it, so nothing needs clearing, and
// calls that overlap on one GPU (different streams) race on it.
static __device__ __align__(256) int32_t scratch[kMoeStaticScratchBytes / sizeof(int32_t)];

hipError_t moe_static_scratch(int32_t **ptr) {
  static std::mutex mu;
  static int32_t *per_device[kMaxDevicesStatic] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevicesStatic) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = static_cast<int32_t *>(p);
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

namespace {

// out[t][o] = sum over j = 0..n_used-1 (in that order) of
// weights[t][j] * y[t*n_used + j][o], one fma per slot: the routed MoE's
// weighted combine ("Part 6: 代码走读", trace 5, step 4), deterministic.
__global__ __launch_bounds__(256) void moe_combine_kernel(float *__restrict__ out,
                                                          const float *__restrict__ y,
                                                          const float *__restrict__ weights,
                                                          int64_t n_tok, int32_t n_used,
                                                          int64_t dim) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_tok * dim) return;
  const int64_t t = i / dim;
  const int64_t o = i - t * dim;
  const float *yt = y + t * n_used * dim + o;
  const float *wt = weights + t * n_used;
  float acc = 0.0f;
  for (int32_t j = 0; j < n_used; ++j) acc = fmaf(wt[j], yt[(int64_t)j * dim], acc);
  out[i] = acc;
}

}  // namespace

hipError_t launch_moe_ffn(const MoeFfn &f, int32_t *ws, hipStream_t s) {
  const MoeLayout L = moe_layout(f.n_tok, f.n_used, f.n_expert);
  const int64_t n_pairs = f.n_tok * f.n_used;
  // 1. Routing; the down outputs of pairs with an invalid id are set to NaN.
  hipError_t err =
      launch_moe_route(f.selected, f.n_tok, f.n_used, f.n_expert, ws, f.y, f.d_model, s, nullptr);
  if (err != hipSuccess) return err;
  // 2. gate and up of every pair in one pass, SwiGLU into mid.
  err = launch_matvec_grouped_pair(f.mid, f.gate_w, f.up_w, f.n_expert, f.d_model, f.d_ff, f.x_q,
                                   f.n_used, ws + L.counts, ws + L.offsets, ws + L.pairs, f.clamp, s);
  if (err != hipSuccess) return err;
  // 3. mid -> Q8_0 rows, one per pair.
  err = launch_quantize(f.mid_q, f.mid, n_pairs, f.d_ff, true, s);
  if (err != hipSuccess) return err;
  // 4. down projection of every pair.
  err = launch_matvec_grouped(f.y, nullptr, f.down_w, f.n_expert, f.d_ff, f.d_model, f.mid_q, 1,
                              f.n_used, ws + L.counts, ws + L.offsets, ws + L.pairs, s);
  if (err != hipSuccess) return err;
  // 5. weighted combine per token.
  const int64_t n = f.n_tok * f.d_model;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, f.out,
                     f.y, f.weights, f.n_tok, f.n_used, f.d_model);
  return hipGetLastError();
}

}  // namespace q8
