// Router top-k with a softmax over the selected logits, and the token->expert counting sort.
//
// Routing: one wavefront per token (moe_route.hpp).
//
// Sort: each expert receives a few token rows ("Zyphra Inference Wave 2", Kernel Results);
// grouping the routed slots by expert lets each expert's weights be read once for up to 16
// of its rows (one MFMA row tile).  The order is fixed (experts ascending, slot ascending), so the result is
// bit-exact and independent of thread timing.
//
// For up to 16 tokens the layer forward runs both in one single-workgroup launch
// (moe_route_sort_kernel); beyond that, and for the stage entry points, one kernel each.
#include "moe_route.hpp"

namespace mx {

// Slot j < k + ns of a token: the j-th routed expert and its gate for j < k, else the shared
// expert E + j - k with gate 1 (a model's always-active experts follow its routed ones).
__device__ __forceinline__ int slot_expert(int j, int k, int E, int routed) { return j < k ? routed : E + j - k; }
__device__ __forceinline__ float slot_gate(int j, int k, float routed) { return j < k ? routed : 1.0f; }

// One wavefront per token.  Workgroups past the routing ones fill `fill` (n16 16-byte units)
// with all ones: the h rows of a launch whose down items read them while gate_up writes them
// start out as 0xFFFF (the expert launch's "not yet written" pattern).
template <int PER>
__global__ void __launch_bounds__(256) moe_route_kernel(const float* __restrict__ logits, int T, int E, int k, int ns,
                                                        int32_t* __restrict__ ids, float* __restrict__ gates,
                                                        u32x4* __restrict__ fill, int64_t n16) {
  const int route_wgs = (T + 3) / 4;
  if ((int)blockIdx.x >= route_wgs) {
    const int64_t stride = (int64_t)(gridDim.x - route_wgs) * 256;
    for (int64_t i = (int64_t)(blockIdx.x - route_wgs) * 256 + threadIdx.x; i < n16; i += stride)
      fill[i] = u32x4{~0u, ~0u, ~0u, ~0u};
    return;
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[PER];
  route_load<PER>(logits + (size_t)t * E, E, lane, v);
  int e;
  float g;
  route_select<PER>(v, E, k, lane, e, g);
  const int kk = k + ns;
  if (lane < kk) {
    ids[(size_t)t * kk + lane] = slot_expert(lane, k, E, e);
    gates[(size_t)t * kk + lane] = slot_gate(lane, k, g);
  }
}

int launch_route(const float* logits, int T, int E, int k, int ns, int32_t* ids, float* gates, hipStream_t stream,
                 void* fill, size_t fill_bytes) {
  const int64_t n16 = fill ? (int64_t)(fill_bytes / 16) : 0;
  const int64_t fill_wgs = (n16 + 1023) / 1024 < 256 ? (n16 + 1023) / 1024 : 256;  // 4 stores per thread up to 4 MB
  const dim3 grid((unsigned)((T + 3) / 4 + fill_wgs)), block(256);
  u32x4* f = static_cast<u32x4*>(fill);
  switch (route_per(E)) {
    case 4: hipLaunchKernelGGL(moe_route_kernel<4>, grid, block, 0, stream, logits, T, E, k, ns, ids, gates, f, n16); break;
    case 8: hipLaunchKernelGGL(moe_route_kernel<8>, grid, block, 0, stream, logits, T, E, k, ns, ids, gates, f, n16); break;
    default:
      hipLaunchKernelGGL(moe_route_kernel<16>, grid, block, 0, stream, logits, T, E, k, ns, ids, gates, f, n16);
      break;
  }
  return hip_status(hipGetLastError());
}

// All ones over n16 16-byte units (the single expert launch's "not yet written" h, when no
// routing launch fills it).
__global__ void __launch_bounds__(256) mx_fill_ones_kernel(u32x4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = u32x4{~0u, ~0u, ~0u, ~0u};
}

int launch_fill_ones(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return MX_OK;
  const int64_t wgs = (n16 + 1023) / 1024 < 1024 ? (n16 + 1023) / 1024 : 1024;
  hipLaunchKernelGGL(mx_fill_ones_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, static_cast<u32x4*>(p), n16);
  return hip_status(hipGetLastError());
}

// ------------------------------------------------------------------ sort

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WORDS = MX_MAX_EXPERTS * (MX_MAX_TOKENS / 32);  // one bit per (expert, token)

// LDS of the sort: a token mask per expert, each expert's offset and the scan's wave sums.
struct SortShared {
  uint32_t bits[SORT_WORDS];
  int32_t off[MX_MAX_EXPERTS];
  int32_t wave_sum[SORT_THREADS / 64];
  int32_t wave_max[SORT_THREADS / 64];
  uint64_t wave_cls[SORT_THREADS / 64];
};

// Row class of an active expert: 3 for 8 or more routed rows, 2 for 4-7, 1 for 2-3, 0 for 1.
// The active list runs heaviest class first, so the expert GEMMs deal and claim the items
// with the most rows (the longest, since each stages its rows' activations) before the
// lightest, and the last items claimed are short.
__device__ __forceinline__ int row_class(int c) { return c >= 8 ? 3 : c >= 4 ? 2 : c >= 2 ? 1 : 0; }

// Counting sort from the token masks (bits must hold every routed (expert, token) pair).
// A slot (t, j) routed to expert e sets bit t of expert e's mask; because a token's k
// experts are distinct, the rank of the slot among expert e's slots is the number of set
// bits below t, which fixes a stable order without any ordering of atomics.  Counts and
// offsets come from one packed block-wide scan, the active list's positions (row class
// descending, then expert id) from a second one over four 16-bit class counters, and the
// largest count from a block maximum.  `ids` is read for the scatter
// (global or LDS).  Must be called by all SORT_THREADS threads.
__device__ __forceinline__ void sort_from_bits(SortShared& sh, const int32_t* ids, int T, int k, int E,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ sorted_slots, int32_t* __restrict__ active,
                                               int32_t* __restrict__ num_active) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = (T + 31) >> 5;
  const int F = T * k;
  // per-expert count and active flag, packed as count | flag << 16 (count <= T < 2^16)
  const int e = tid;
  int cnt = 0;
  if (e < E)
    for (int w = 0; w < words; ++w) cnt += __popc(sh.bits[e * words + w]);
  const int packed = cnt | ((cnt > 0) ? (1 << 16) : 0);
  // block-wide exclusive scan of `packed` over e = 0..E-1 (E <= 1024 = blockDim)
  int incl = packed;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh.wave_sum[wave] = incl;
  // per-class active flags, one 16-bit field per class (at most 1024 experts per class)
  const uint64_t cpk = (cnt > 0) ? (1ull << (16 * row_class(cnt))) : 0ull;
  uint64_t cincl = cpk;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(cincl, off);
    if (lane >= off) cincl += o;
  }
  if (lane == 63) sh.wave_cls[wave] = cincl;
  int most = cnt;  // largest count, over the wavefront
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) most = max(most, __shfl_xor(most, off));
  if (lane == 0) sh.wave_max[wave] = most;
  __syncthreads();
  if (wave == 0) {
    int wv = (lane < SORT_THREADS / 64) ? sh.wave_sum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(wv, off);
      if (lane >= off) wv += o;
    }
    if (lane < SORT_THREADS / 64) sh.wave_sum[lane] = wv;  // inclusive over waves
  } else if (wave == 1) {
    uint64_t cv = (lane < SORT_THREADS / 64) ? sh.wave_cls[lane] : 0ull;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t o = __shfl_up(cv, off);
      if (lane >= off) cv += o;
    }
    if (lane < SORT_THREADS / 64) sh.wave_cls[lane] = cv;  // inclusive over waves
  }
  __syncthreads();
  const int excl = incl - packed + (wave > 0 ? sh.wave_sum[wave - 1] : 0);
  const int off_e = excl & 0xFFFF;
  const uint64_t cexcl = cincl - cpk + (wave > 0 ? sh.wave_cls[wave - 1] : 0ull);
  const uint64_t ctot = sh.wave_cls[SORT_THREADS / 64 - 1];
  if (e < E) {
    sh.off[e] = off_e;
    counts[e] = cnt;
    offsets[e] = off_e;
    if (cnt > 0) {
      // heavier classes first: the totals of the classes above, then this class's rank
      const int c = row_class(cnt);
      int pos = (int)((cexcl >> (16 * c)) & 0xFFFFu);
      for (int d = c + 1; d < 4; ++d) pos += (int)((ctot >> (16 * d)) & 0xFFFFu);
      active[pos] = e;
    }
  }
  const int total = sh.wave_sum[SORT_THREADS / 64 - 1];
  const int n_act = total >> 16;
  if (e < E && e >= n_act) active[e] = -1;
  if (tid == 0) {
    offsets[E] = total & 0xFFFF;
    num_active[0] = n_act;
    int m = 0;
    for (int w = 0; w < SORT_THREADS / 64; ++w) m = max(m, sh.wave_max[w]);
    num_active[1] = m;
  }
  __syncthreads();
  for (int f = tid; f < F; f += SORT_THREADS) {
    const int ee = ids[f];
    if (ee < 0 || ee >= E) continue;
    const int t = f / k;
    const uint32_t* b = sh.bits + ee * words;
    int rank = __popc(b[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(b[w]);
    sorted_slots[sh.off[ee] + rank] = f;
  }
}

// Single workgroup: the token masks from the routed ids, then the counting sort.
__global__ void __launch_bounds__(SORT_THREADS) moe_sort_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                                int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_slots,
                                                                int32_t* __restrict__ active,
                                                                int32_t* __restrict__ num_active) {
  __shared__ SortShared sh;
  const int tid = threadIdx.x;
  const int words = (T + 31) >> 5;
  const int F = T * k;
  for (int i = tid; i < E * words; i += SORT_THREADS) sh.bits[i] = 0u;
  __syncthreads();
  for (int f = tid; f < F; f += SORT_THREADS) {
    const int e = ids[f];
    const int t = f / k;
    if (e >= 0 && e < E) atomicOr(&sh.bits[e * words + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  sort_from_bits(sh, ids, T, k, E, counts, offsets, sorted_slots, active, num_active);
}

int launch_sort(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                int32_t* active, int32_t* num_active, hipStream_t stream) {
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(SORT_THREADS), 0, stream, ids, T, k, E, counts, offsets,
                     sorted_slots, active, num_active);
  return hip_status(hipGetLastError());
}

// ------------------------------------------------------------------ route + sort, one launch

// Single workgroup of SORT_THREADS: wave w routes tokens w, w + 16, ... (loading the next
// token's logits before routing the current one), writing ids and gates (the ns shared
// slots after the k routed ones) and setting the token masks directly; the ids stay in LDS
// for the sort over the E + ns experts.
template <int PER>
__global__ void __launch_bounds__(SORT_THREADS) moe_route_sort_kernel(
    const float* __restrict__ logits, int T, int E, int k, int ns, int32_t* __restrict__ ids, float* __restrict__ gates,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active) {
  __shared__ SortShared sh;
  __shared__ int32_t s_ids[MX_MAX_TOKENS * MX_MAX_TOPK];
  constexpr int NW = SORT_THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = (T + 31) >> 5;
  const int kk = k + ns;
  float v[PER], vn[PER];
  route_load<PER>(logits + (size_t)min(wave, T - 1) * E, E, lane, v);
  for (int i = tid; i < (E + ns) * words; i += SORT_THREADS) sh.bits[i] = 0u;
  __syncthreads();
  for (int t = wave; t < T; t += NW) {
    // unconditional (the last row again past the end), so the waits stay exact
    route_load<PER>(logits + (size_t)min(t + NW, T - 1) * E, E, lane, vn);
    int e;
    float g;
    route_select<PER>(v, E, k, lane, e, g);
    if (lane < kk) {
      const int ee = slot_expert(lane, k, E, e);
      ids[(size_t)t * kk + lane] = ee;
      gates[(size_t)t * kk + lane] = slot_gate(lane, k, g);
      s_ids[t * kk + lane] = ee;
      atomicOr(&sh.bits[ee * words + (t >> 5)], 1u << (t & 31));
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = vn[i];
  }
  __syncthreads();
  sort_from_bits(sh, s_ids, T, kk, E + ns, counts, offsets, sorted_slots, active, num_active);
}

// Up to this many tokens (one per wavefront of the workgroup) route and sort run as one
// launch; beyond it the single workgroup's routing would take longer than the routing
// kernel spread over T / 4 workgroups plus a separate sort launch.
constexpr int ROUTE_SORT_FUSED_MAX_T = SORT_THREADS / 64;

int launch_route_sort(const float* logits, int T, int E, int k, int ns, int32_t* ids, float* gates, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_slots, int32_t* active, int32_t* num_active,
                      hipStream_t stream, void* fill, size_t fill_bytes) {
  if (fill && T <= ROUTE_SORT_FUSED_MAX_T) return MX_ERR_SHAPE;  // the single-workgroup launch does not fill
  if (T > ROUTE_SORT_FUSED_MAX_T) {
    const int st = launch_route(logits, T, E, k, ns, ids, gates, stream, fill, fill_bytes);
    if (st != MX_OK) return st;
    return launch_sort(ids, T, k + ns, E + ns, counts, offsets, sorted_slots, active, num_active, stream);
  }
  const dim3 grid(1), block(SORT_THREADS);
  switch (route_per(E)) {
    case 4:
      hipLaunchKernelGGL(moe_route_sort_kernel<4>, grid, block, 0, stream, logits, T, E, k, ns, ids, gates, counts,
                         offsets, sorted_slots, active, num_active);
      break;
    case 8:
      hipLaunchKernelGGL(moe_route_sort_kernel<8>, grid, block, 0, stream, logits, T, E, k, ns, ids, gates, counts,
                         offsets, sorted_slots, active, num_active);
      break;
    default:
      hipLaunchKernelGGL(moe_route_sort_kernel<16>, grid, block, 0, stream, logits, T, E, k, ns, ids, gates, counts,
                         offsets, sorted_slots, active, num_active);
      break;
  }
  return hip_status(hipGetLastError());
}

}  // namespace mx
