// C-ABI entry points: host-side argument checks, workspace carving, kernel enqueue.
// Every check runs before anything is enqueued; no call allocates or synchronizes.
#include <atomic>
#include <limits>
#include <mutex>

#include "mx_internal.hpp"

namespace mx {

static constexpr size_t WS_ALIGN = 256;

static size_t align_up(size_t v) { return (v + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

MoeWorkspace moe_workspace_carve(void* base, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  MoeWorkspace w{};
  const size_t F = (size_t)(T * k);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? static_cast<char*>(base) + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.ctl = reinterpret_cast<int32_t*>(take(MX_WORKSPACE_CTL_BYTES));
  w.ids = reinterpret_cast<int32_t*>(take(F * 4));
  w.gates = reinterpret_cast<float*>(take(F * 4));
  w.counts = reinterpret_cast<int32_t*>(take((size_t)E * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  w.sorted_slots = reinterpret_cast<int32_t*>(take(F * 4));
  w.active = reinterpret_cast<int32_t*>(take((size_t)E * 4));
  w.num_active = reinterpret_cast<int32_t*>(take(8));
  w.h = reinterpret_cast<uint16_t*>(take(F * (size_t)I * 2));
  w.dpart = reinterpret_cast<float*>(take(F * (size_t)H * 4));
  w.bytes = off;
  return w;
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static constexpr int64_t INT_LIM = std::numeric_limits<int32_t>::max();

static int check_moe_sizes(int64_t T, int64_t E, int64_t k) {
  if (T < 1 || T > MX_MAX_TOKENS) return MX_ERR_SHAPE;
  if (E < 1 || E > MX_MAX_EXPERTS) return MX_ERR_SHAPE;
  if (k < 1 || k > MX_MAX_TOPK || k > E) return MX_ERR_SHAPE;
  return MX_OK;
}

// The gate_up GEMM (reduction length H) stages the weight scales 1024 K values (four
// 256-value segments) at a time, so H must be a multiple of 1024; the down GEMM (reduction
// length I) takes any multiple of 256, e.g. I = 256 for one tensor-parallel eighth of an
// expert of 2048.
static int check_expert_dims(int64_t H, int64_t I) {
  if (H < 1024 || I < 256 || H % 1024 != 0 || I % 256 != 0 || H > 65536 || I > 65536) return MX_ERR_SHAPE;
  return MX_OK;
}

// ------------------------------------------------------------------ static scratch

// The scratch of moe_mxfp4_forward_noalloc, for callers that cannot allocate: one array
// per GPU (each device that loads the library holds its own copy until the process ends).
// Host code never uses this name as an address: it is a host-side stand-in for the device
// symbol.  noalloc_scratch() looks the array's device address up once per device, with
// hipGetSymbolAddress, and every later use goes through that address.
static __device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;

// Zeroes `words` int32 words (the workspace control words the expert GEMMs count in).
__global__ void __launch_bounds__(256) zero_words_kernel(int32_t* __restrict__ p, int words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0;
}

// The current device's scratch address.  On a device's first call it also enqueues, on
// `stream`, a kernel that zeroes the control words at the array's start (the array is
// zero when the code object loads, and every forward leaves them zero; this makes the
// first call independent of that).  A kernel rather than a memset, so that a first call
// under graph capture records an ordinary kernel node.
static int noalloc_scratch(void** out, hipStream_t stream) {
  static std::mutex mu;
  static void* addr[NOALLOC_MAX_DEVICES];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return MX_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MX_ERR_HIP;
    const int words = MX_WORKSPACE_CTL_BYTES / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream, static_cast<int32_t*>(p),
                       words);
    if (hipGetLastError() != hipSuccess) return MX_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return MX_OK;
}

static bool sort_view_ok(const int32_t* counts, const int32_t* offsets, const int32_t* sorted_slots,
                         const int32_t* active, const int32_t* num_active) {
  return counts && offsets && sorted_slots && active && num_active;
}

static bool sort_view_aligned(const int32_t* counts, const int32_t* offsets, const int32_t* sorted_slots,
                              const int32_t* active, const int32_t* num_active) {
  return aligned(counts, 4) && aligned(offsets, 4) && aligned(sorted_slots, 4) && aligned(active, 4) &&
         aligned(num_active, 4);
}

}  // namespace mx

using namespace mx;

extern "C" {

int mx_version(void) { return 100; }

const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case MX_ERR_ALIGN: return "a pointer is not aligned as required";
    case MX_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MX_ERR_HIP: return "the HIP runtime reported an error while enqueueing";
    case MX_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
    default: return "unknown status";
  }
}

int mx_linear(const uint16_t* x, const uint8_t* w_codes, const uint8_t* w_scales, uint16_t* y, int64_t T, int64_t K,
              int64_t N, void* stream) {
  if (!x || !w_codes || !w_scales || !y) return MX_ERR_NULL;
  if (T < 1 || N < 1 || K < 32 || K % 32 != 0) return MX_ERR_SHAPE;
  if (T > INT_LIM || K > INT_LIM || N > INT_LIM || T * K > (int64_t)1 << 40 || N * K > (int64_t)1 << 42)
    return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w_codes, 16) || !aligned(y, 8)) return MX_ERR_ALIGN;
  if (K % 256 == 0 && !aligned(w_scales, 8)) return MX_ERR_ALIGN;  // 8-byte scale loads
  return launch_mx_linear(x, w_codes, w_scales, y, (int)T, (int)K, (int)N, static_cast<hipStream_t>(stream));
}

int mx_linear_a8(const uint16_t* x, const uint8_t* w_codes, const uint8_t* w_scales, uint16_t* y, int64_t T,
                 int64_t K, int64_t N, void* stream) {
  if (!x || !w_codes || !w_scales || !y) return MX_ERR_NULL;
  if (T < 1 || N < 1 || K < 32 || K % 32 != 0) return MX_ERR_SHAPE;
  if (T > INT_LIM || K > INT_LIM || N > INT_LIM || T * K > (int64_t)1 << 40 || N * K > (int64_t)1 << 42)
    return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w_codes, 16) || !aligned(y, 8)) return MX_ERR_ALIGN;
  if (K % 256 == 0 && !aligned(w_scales, 8)) return MX_ERR_ALIGN;  // 8-byte scale loads
  return launch_mx_linear_a8(x, w_codes, w_scales, y, (int)T, (int)K, (int)N, static_cast<hipStream_t>(stream));
}

int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (rows < 1 || K < 32 || K % 32 != 0 || rows * (K / 32) > ((int64_t)1 << 38)) return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 8)) return MX_ERR_ALIGN;
  return launch_mxfp8_quantize(x, rows, K, codes, scales, static_cast<hipStream_t>(stream));
}

int mxfp4_dequantize(const uint8_t* w_codes, const uint8_t* w_scales, int64_t rows, int64_t K, uint16_t* out,
                     void* stream) {
  if (!w_codes || !w_scales || !out) return MX_ERR_NULL;
  if (rows < 1 || K < 32 || K % 32 != 0 || rows * (K / 32) > ((int64_t)1 << 38)) return MX_ERR_SHAPE;
  if (!aligned(w_codes, 16) || !aligned(out, 16)) return MX_ERR_ALIGN;
  return launch_dequant(w_codes, w_scales, rows, K, out, static_cast<hipStream_t>(stream));
}

int moe_route_topk(const float* logits, int64_t T, int64_t E, int64_t top_k, int32_t* ids, float* gates,
                   void* stream) {
  if (!logits || !ids || !gates) return MX_ERR_NULL;
  const int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK) return st;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(gates, 4)) return MX_ERR_ALIGN;
  return launch_route(logits, (int)T, (int)E, (int)top_k, 0, ids, gates, static_cast<hipStream_t>(stream));
}

int moe_sort_by_expert(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_slots, int32_t* active, int32_t* num_active, void* stream) {
  if (!ids || !counts || !offsets || !sorted_slots || !active || !num_active) return MX_ERR_NULL;
  const int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK) return st;
  if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_slots, 4) ||
      !aligned(active, 4) || !aligned(num_active, 4))
    return MX_ERR_ALIGN;
  return launch_sort(ids, (int)T, (int)top_k, (int)E, counts, offsets, sorted_slots, active, num_active,
                     static_cast<hipStream_t>(stream));
}

int moe_route_sort(const float* logits, int64_t T, int64_t E, int64_t top_k, int32_t* ids, float* gates,
                   int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* active, int32_t* num_active,
                   void* stream) {
  if (!logits || !ids || !gates || !counts || !offsets || !sorted_slots || !active || !num_active) return MX_ERR_NULL;
  const int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK) return st;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(gates, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(sorted_slots, 4) || !aligned(active, 4) || !aligned(num_active, 4))
    return MX_ERR_ALIGN;
  return launch_route_sort(logits, (int)T, (int)E, (int)top_k, 0, ids, gates, counts, offsets, sorted_slots, active,
                           num_active, static_cast<hipStream_t>(stream));
}

int moe_gate_up_swiglu(const uint16_t* x, const uint8_t* w_gate_up, const uint8_t* s_gate_up, const int32_t* counts,
                       const int32_t* offsets, const int32_t* sorted_slots, const int32_t* active,
                       const int32_t* num_active, uint16_t* h, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_gate_up || !s_gate_up || !h || !sort_view_ok(counts, offsets, sorted_slots, active, num_active))
    return MX_ERR_NULL;
  int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK || (st = check_expert_dims(H, I)) != MX_OK) return st;
  if (!aligned(x, 16) || !aligned(w_gate_up, 16) || !aligned(s_gate_up, 16) || !aligned(h, 8) ||
      !sort_view_aligned(counts, offsets, sorted_slots, active, num_active))
    return MX_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return MX_ERR_WORKSPACE;
  const MoeWorkspace ws = moe_workspace_carve(workspace, T, H, I, E, top_k);
  if (workspace_bytes < ws.bytes) return MX_ERR_WORKSPACE;
  const SortView sv{counts, offsets, sorted_slots, active, num_active};
  return launch_gate_up(x, w_gate_up, s_gate_up, sv, h, ws.ctl, (int)T, (int)H, (int)I, (int)E, (int)top_k, false,
                        static_cast<hipStream_t>(stream));
}

int moe_gate_up_swiglu_from_ids(const uint16_t* x, const int32_t* ids, const uint8_t* w_gate_up,
                                const uint8_t* s_gate_up, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                                int32_t* active, int32_t* num_active, uint16_t* h, int64_t T, int64_t H, int64_t I,
                                int64_t E, int64_t top_k, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !ids || !w_gate_up || !s_gate_up || !h || !sort_view_ok(counts, offsets, sorted_slots, active, num_active))
    return MX_ERR_NULL;
  int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK || (st = check_expert_dims(H, I)) != MX_OK) return st;
  if (!gate_up_sorted_fits((int)T, (int)E, (int)top_k, (int)H, (int)I)) return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(ids, 4) || !aligned(w_gate_up, 16) || !aligned(s_gate_up, 16) || !aligned(h, 8) ||
      !sort_view_aligned(counts, offsets, sorted_slots, active, num_active))
    return MX_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return MX_ERR_WORKSPACE;
  const MoeWorkspace ws = moe_workspace_carve(workspace, T, H, I, E, top_k);
  if (workspace_bytes < ws.bytes) return MX_ERR_WORKSPACE;
  return launch_gate_up_sorted(x, ids, w_gate_up, s_gate_up, h, counts, offsets, sorted_slots, active, num_active,
                               ws.ctl, (int)T, (int)H, (int)I, (int)E, (int)top_k, false,
                               static_cast<hipStream_t>(stream));
}

int moe_down_combine(const uint16_t* h, const float* gates, const uint8_t* w_down, const uint8_t* s_down,
                     const int32_t* counts, const int32_t* offsets, const int32_t* sorted_slots, const int32_t* active,
                     const int32_t* num_active, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || !gates || !w_down || !s_down || !y || !sort_view_ok(counts, offsets, sorted_slots, active, num_active))
    return MX_ERR_NULL;
  int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK || (st = check_expert_dims(H, I)) != MX_OK) return st;
  if (!aligned(h, 16) || !aligned(gates, 4) || !aligned(w_down, 16) || !aligned(s_down, 16) || !aligned(y, 8) ||
      !sort_view_aligned(counts, offsets, sorted_slots, active, num_active))
    return MX_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return MX_ERR_WORKSPACE;
  const MoeWorkspace ws = moe_workspace_carve(workspace, T, H, I, E, top_k);
  if (workspace_bytes < ws.bytes) return MX_ERR_WORKSPACE;
  const SortView sv{counts, offsets, sorted_slots, active, num_active};
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool combined = false;
  if ((st = launch_down(h, gates, w_down, s_down, sv, ws.dpart, y, &combined, ws.ctl, (int)T, (int)H, (int)I, (int)E,
                        (int)top_k, false, s)) != MX_OK)
    return st;
  return combined ? MX_OK : launch_combine(ws.dpart, gates, y, (int)T, (int)H, (int)top_k, s);
}

int moe_expert_gemms_from_ids(const uint16_t* x, const int32_t* ids, const uint8_t* w_gate_up,
                              const uint8_t* s_gate_up, const uint8_t* w_down, const uint8_t* s_down, uint16_t* h,
                              int h_prefilled, float* d, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !ids || !w_gate_up || !s_gate_up || !w_down || !s_down || !h || !d) return MX_ERR_NULL;
  int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK || (st = check_expert_dims(H, I)) != MX_OK) return st;
  if (!experts_sorted_fits((int)T, (int)E, (int)top_k, (int)H, (int)I)) return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(ids, 4) || !aligned(w_gate_up, 16) || !aligned(s_gate_up, 16) ||
      !aligned(w_down, 16) || !aligned(s_down, 16) || !aligned(h, 16) || !aligned(d, 16))
    return MX_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return MX_ERR_WORKSPACE;
  const MoeWorkspace ws = moe_workspace_carve(workspace, T, H, I, E, top_k);
  if (workspace_bytes < ws.bytes) return MX_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!h_prefilled && (st = launch_fill_ones(h, (size_t)(T * top_k * I * 2), s)) != MX_OK) return st;
  return launch_experts_sorted(x, ids, w_gate_up, s_gate_up, w_down, s_down, h, d, ws.ctl, (int)T, (int)H, (int)I,
                               (int)E, (int)top_k, false, s);
}

int moe_combine(const float* d, const float* gates, uint16_t* y, int64_t T, int64_t H, int64_t top_k, void* stream) {
  if (!d || !gates || !y) return MX_ERR_NULL;
  if (T < 1 || T > MX_MAX_TOKENS || top_k < 1 || top_k > MX_MAX_TOPK || H < 4 || H > 65536 || H % 4 != 0)
    return MX_ERR_SHAPE;
  if (!aligned(d, 16) || !aligned(gates, 4) || !aligned(y, 8)) return MX_ERR_ALIGN;
  return launch_combine(d, gates, y, (int)T, (int)H, (int)top_k, static_cast<hipStream_t>(stream));
}

size_t moe_mxfp4_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k) {
  if (T < 1 || H < 1 || I < 1 || E < 1 || top_k < 1) return 0;
  return moe_workspace_carve(nullptr, T, H, I, E, top_k).bytes;
}

// The layer over E routed experts (top_k of them per token) and ns shared experts after them;
// act8: MXFP8 activations for both expert GEMMs.
// The checks of the layer forward's arguments other than the workspace.
static int moe_forward_args(const uint16_t* x, const float* router_logits, int64_t top_k, int64_t ns,
                            const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                            const uint8_t* s_down, const uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E) {
  if (!x || !router_logits || !w_gate_up || !s_gate_up || !w_down || !s_down || !y) return MX_ERR_NULL;
  int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK) return st;
  if (ns < 0 || E + ns > MX_MAX_EXPERTS || top_k + ns > MX_MAX_TOPK) return MX_ERR_SHAPE;
  if ((st = check_expert_dims(H, I)) != MX_OK) return st;
  if (!aligned(x, 16) || !aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(s_gate_up, 16) ||
      !aligned(s_down, 16) || !aligned(y, 8) || !aligned(router_logits, 4))
    return MX_ERR_ALIGN;
  return MX_OK;
}

static int moe_forward_impl(const uint16_t* x, const float* router_logits, int64_t top_k, int64_t ns,
                            const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                            const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                            void* workspace, size_t workspace_bytes, bool act8, void* stream) {
  int st = moe_forward_args(x, router_logits, top_k, ns, w_gate_up, s_gate_up, w_down, s_down, y, T, H, I, E);
  if (st != MX_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return MX_ERR_WORKSPACE;
  // every slot, routed and shared, is one row of the expert GEMMs
  const MoeWorkspace ws = moe_workspace_carve(workspace, T, H, I, E + ns, top_k + ns);
  if (workspace_bytes < ws.bytes) return MX_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int t = (int)T, h = (int)H, i = (int)I, e = (int)E, k = (int)top_k, n = (int)ns;
  const SortView sv{ws.counts, ws.offsets, ws.sorted_slots, ws.active, ws.num_active};
  if (n == 0 && experts_sorted_fits(t, e, k, h, i) && experts_sorted_pays(t, e, k, i)) {
    // the routing launch (which also fills h with 0xFFFF), one launch for both expert
    // GEMMs, then the combine
    if ((st = launch_route(router_logits, t, e, k, 0, ws.ids, ws.gates, s, ws.h, (size_t)t * k * i * 2)) != MX_OK)
      return st;
    if ((st = launch_experts_sorted(x, ws.ids, w_gate_up, s_gate_up, w_down, s_down, ws.h, ws.dpart, ws.ctl, t, h, i, e,
                                    k, act8, s)) != MX_OK)
      return st;
    return launch_combine(ws.dpart, ws.gates, y, t, h, k, s);
  } else if (n == 0 && gate_up_routed_fits(t, e, k, h, i)) {
    // small T: gate_up routes and sorts in every workgroup and writes the sort for down
    if ((st = launch_gate_up_routed(x, router_logits, w_gate_up, s_gate_up, ws.h, ws.counts, ws.offsets,
                                    ws.sorted_slots, ws.active, ws.num_active, ws.gates, t, h, i, e, k, act8, s)) !=
        MX_OK)
      return st;
  } else if (n == 0 && gate_up_sorted_fits(t, e, k, h, i)) {
    // up to 32 tokens: the routing launch, then gate_up sorts the slots in every workgroup
    if ((st = launch_route(router_logits, t, e, k, 0, ws.ids, ws.gates, s)) != MX_OK) return st;
    if ((st = launch_gate_up_sorted(x, ws.ids, w_gate_up, s_gate_up, ws.h, ws.counts, ws.offsets, ws.sorted_slots,
                                    ws.active, ws.num_active, ws.ctl, t, h, i, e, k, act8, s)) != MX_OK)
      return st;
  } else if (t > 16 && t <= EXPERTS_MAX_T && experts_fits(h, i) && experts_sorted_pays(t, e + n, k + n, i)) {
    // shared experts, or more than 256 slots: the route and sort launches (the route launch
    // also fills h with 0xFFFF), one launch for both expert GEMMs, then the combine
    if ((st = launch_route_sort(router_logits, t, e, k, n, ws.ids, ws.gates, ws.counts, ws.offsets, ws.sorted_slots,
                                ws.active, ws.num_active, s, ws.h, (size_t)t * (k + n) * i * 2)) != MX_OK)
      return st;
    if ((st = launch_experts(x, sv, w_gate_up, s_gate_up, w_down, s_down, ws.h, ws.dpart, ws.ctl, h, i, k + n, act8,
                             s)) != MX_OK)
      return st;
    return launch_combine(ws.dpart, ws.gates, y, t, h, k + n, s);
  } else {
    if ((st = launch_route_sort(router_logits, t, e, k, n, ws.ids, ws.gates, ws.counts, ws.offsets, ws.sorted_slots,
                                ws.active, ws.num_active, s)) != MX_OK)
      return st;
    if ((st = launch_gate_up(x, w_gate_up, s_gate_up, sv, ws.h, ws.ctl, t, h, i, e + n, k + n, act8, s)) != MX_OK)
      return st;
  }
  bool combined = false;
  if ((st = launch_down(ws.h, ws.gates, w_down, s_down, sv, ws.dpart, y, &combined, ws.ctl, t, h, i, e + n, k + n,
                        act8, s)) != MX_OK)
    return st;
  return combined ? MX_OK : launch_combine(ws.dpart, ws.gates, y, t, h, k + n, s);
}

int moe_mxfp4_forward(const uint16_t* x, const float* router_logits, int64_t top_k, const uint8_t* w_gate_up,
                      const uint8_t* s_gate_up, const uint8_t* w_down, const uint8_t* s_down, uint16_t* y, int64_t T,
                      int64_t H, int64_t I, int64_t E, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_impl(x, router_logits, top_k, 0, w_gate_up, s_gate_up, w_down, s_down, y, T, H, I, E, workspace,
                          workspace_bytes, false, stream);
}

int moe_mxfp4_forward_noalloc(const uint16_t* x, const float* router_logits, int64_t top_k, const uint8_t* w_gate_up,
                              const uint8_t* s_gate_up, const uint8_t* w_down, const uint8_t* s_down, uint16_t* y,
                              int64_t T, int64_t H, int64_t I, int64_t E, void* stream) {
  int st = moe_forward_args(x, router_logits, top_k, 0, w_gate_up, s_gate_up, w_down, s_down, y, T, H, I, E);
  if (st != MX_OK) return st;
  const size_t need = moe_workspace_carve(nullptr, T, H, I, E, top_k).bytes;
  if (need > (size_t)MX_NOALLOC_SCRATCH_BYTES) return MX_ERR_SCRATCH;
  void* ws = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = noalloc_scratch(&ws, s)) != MX_OK) return st;
  return moe_forward_impl(x, router_logits, top_k, 0, w_gate_up, s_gate_up, w_down, s_down, y, T, H, I, E, ws,
                          (size_t)MX_NOALLOC_SCRATCH_BYTES, false, stream);
}

int moe_mxfp4_forward_shared(const uint16_t* x, const float* router_logits, int64_t top_k, int64_t n_shared,
                             const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                             const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_impl(x, router_logits, top_k, n_shared, w_gate_up, s_gate_up, w_down, s_down, y, T, H, I, E,
                          workspace, workspace_bytes, false, stream);
}

int moe_mxfp4_forward_a8(const uint16_t* x, const float* router_logits, int64_t top_k, int64_t n_shared,
                         const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                         const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_impl(x, router_logits, top_k, n_shared, w_gate_up, s_gate_up, w_down, s_down, y, T, H, I, E,
                          workspace, workspace_bytes, true, stream);
}

int moe_mxfp4_forward_persistent(const uint16_t* x, const float* router_logits, int64_t top_k,
                                 const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                                 const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !router_logits || !w_gate_up || !s_gate_up || !w_down || !s_down || !y) return MX_ERR_NULL;
  int st = check_moe_sizes(T, E, top_k);
  if (st != MX_OK) return st;
  if ((st = check_expert_dims(H, I)) != MX_OK) return st;
  if (!fused_layer_fits((int)T, (int)E, (int)top_k, (int)H, (int)I)) return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(s_gate_up, 16) ||
      !aligned(s_down, 16) || !aligned(y, 8) || !aligned(router_logits, 4))
    return MX_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return MX_ERR_WORKSPACE;
  const MoeWorkspace ws = moe_workspace_carve(workspace, T, H, I, E, top_k);
  if (workspace_bytes < ws.bytes) return MX_ERR_WORKSPACE;
  return launch_moe_fused(x, router_logits, w_gate_up, s_gate_up, w_down, s_down, ws.h, ws.dpart, y, ws.ctl, (int)T,
                          (int)H, (int)I, (int)E, (int)top_k, static_cast<hipStream_t>(stream));
}

}  // extern "C"
