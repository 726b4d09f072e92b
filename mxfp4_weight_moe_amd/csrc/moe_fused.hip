// The whole MoE layer in one launch for small T: routing, sort, gate_up + SwiGLU, down and
// the gate-weighted combine.  Also, at the end of this file, the layer forward's gate_up
// launches for T <= 16, which does the routing and sort of this launch in each workgroup and
// leaves down and the combine to their own launches, and for 16 < T <= 32, which sorts the
// routed slots in each workgroup.
//
// At small T a layer streams only tens of microseconds of weights, and each kernel
// boundary (the GPU draining one kernel and starting the next) costs microseconds.  The
// Lithos page ("Specialization unlocks engine performance", 1. Megakernels) and the AMD
// megakernel blog ("What Drives the Speedup", 1. Megakernels) remove such boundaries with
// persistent kernels whose workgroups hand data to one another through memory and
// synchronize only where data is shared.  Here:
//
//   routing  every workgroup routes all T tokens and sorts the slots itself, into LDS
//            (T <= 16: a few microseconds, and the same result everywhere).
//   gate_up  the workgroups stream the gate_up items (moe_policies.hpp) and write h with
//            device-coherent stores; each then adds its item count to a device counter,
//            and the one that completes the count raises a ready flag, replicated on 64
//            lines so that the polls of the workgroups spread over the memory channels.
//   down     each wavefront requests its first weights, then waits for its replica of the
//            flag before loading h.  The down outputs are written with device-coherent
//            stores.
//   combine  each workgroup adds one to the counter of every column quad it finished; the
//            one that completes a quad (one item per active expert) has all of that quad's
//            down outputs and combines those columns for every token, j ascending, exactly
//            as the combine kernel of the multi-launch path does.
//
// No cache-wide write-back or invalidate is used: the data handed between workgroups
// moves with sc1 accesses, and a wavefront's own stores are complete (s_waitcnt vmcnt(0))
// before it publishes a count.  The last workgroup to finish (an exit counter) resets the
// counters, so every call leaves the workspace control words zero, as it found them.
//
// The waits assume every workgroup of the grid is resident at once (the grid is sized to
// the device's occupancy for this kernel).  A wait that would outlast any layer by far
// gives up and raises the error word instead of hanging.
#include "moe_policies.hpp"
#include "moe_route.hpp"

namespace mx {

constexpr int FUSED_MAX_SLOTS = 128;  // T * k
constexpr int FUSED_XCHUNK = GU_XCHUNK;
static_assert(MX_FUSED_MAX_TOKENS <= 32, "a token mask per expert is one 32-bit word");
static_assert(MX_FUSED_MAX_TOKENS <= 16, "one row group (16 rows) per expert");

// The workgroup's routing and sort (LDS).  Active experts are numbered a = 0.. in
// ascending expert order.
struct FusedSort {
  int32_t act[FUSED_MAX_SLOTS];    // expert id of active expert a
  int32_t cnt[FUSED_MAX_SLOTS];    // its routed rows
  int32_t off[FUSED_MAX_SLOTS];    // its first sorted position
  int32_t slots[FUSED_MAX_SLOTS];  // flat slot at each sorted position
  float gates[FUSED_MAX_SLOTS];    // gate of each flat slot t * k + j
  int32_t na;                      // active experts
  int32_t wave_sum[WG_WAVES];
  int32_t ndone;                   // column quads this workgroup completed
  int32_t last;                    // this workgroup finished last
  int32_t h_ready;                 // the workgroup's poller saw every h row written
};
__shared__ FusedSort fsort;

struct LdsSort {
  __device__ __forceinline__ int num_active() const { return __builtin_amdgcn_readfirstlane(fsort.na); }
  __device__ __forceinline__ int expert(int a) const { return __builtin_amdgcn_readfirstlane(fsort.act[a]); }
  __device__ __forceinline__ int count(int a) const { return __builtin_amdgcn_readfirstlane(fsort.cnt[a]); }
  __device__ __forceinline__ int offset(int a) const { return __builtin_amdgcn_readfirstlane(fsort.off[a]); }
  __device__ __forceinline__ int slot(int i) const { return __builtin_amdgcn_readfirstlane(fsort.slots[i]); }
  __device__ __forceinline__ int count_lane(int a) const { return fsort.cnt[a]; }
};

// Routing and counting sort of one workgroup into fsort; `tmp` is scratch LDS of at least
// 9 KB (token masks, per-expert offsets, routed ids).  Wave w routes tokens w, w + 4, ...;
// a slot (t, j) routed to expert e sets bit t of e's mask, and since a token's k experts
// are distinct, the slot's rank among e's slots is the number of mask bits below t.
// Counts, offsets and active positions come from one scan over the experts, 4 per thread.
template <int PER>
__device__ __forceinline__ void fused_route_sort(const float* __restrict__ logits, int T, int E, int k,
                                                 uint8_t* __restrict__ tmp) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(tmp);             // [E]
  int32_t* eoff = reinterpret_cast<int32_t*>(tmp + 4096);        // [E]
  int32_t* sids = reinterpret_cast<int32_t*>(tmp + 8192);        // [T * k]
  static_assert(MX_MAX_EXPERTS * 4 <= 4096 && FUSED_MAX_SLOTS * 4 <= 1024, "scratch layout");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float v[PER], vn[PER];
  route_load<PER>(logits + (size_t)min(wave, T - 1) * E, E, lane, v);
  for (int i = tid; i < E; i += WG_WAVES * 64) bits[i] = 0u;
  __syncthreads();
  for (int t = wave; t < T; t += WG_WAVES) {
    // the next token of this wave (unconditional: the last row again past the end)
    route_load<PER>(logits + (size_t)min(t + WG_WAVES, T - 1) * E, E, lane, vn);
    int e;
    float g;
    route_select<PER>(v, E, k, lane, e, g);
    if (lane < k) {
      sids[t * k + lane] = e;
      fsort.gates[t * k + lane] = g;
      atomicOr(&bits[e], 1u << t);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = vn[i];
  }
  __syncthreads();
  // exclusive scan of (count | active << 16) over the experts
  int c[4], packed[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    c[q] = (e < E) ? __popc(bits[e]) : 0;
    packed[q] = c[q] | (c[q] > 0 ? (1 << 16) : 0);
    sum += packed[q];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) fsort.wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w = 0; w < wave; ++w) run += fsort.wave_sum[w];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < E) {
      eoff[e] = run & 0xFFFF;
      if (c[q] > 0) {
        const int a = run >> 16;
        fsort.act[a] = e;
        fsort.cnt[a] = c[q];
        fsort.off[a] = run & 0xFFFF;
      }
    }
    run += packed[q];
  }
  if (tid == WG_WAVES * 64 - 1) fsort.na = run >> 16;
  __syncthreads();
  for (int f = tid; f < T * k; f += WG_WAVES * 64) {
    const int e = sids[f];
    const int t = f / k;
    fsort.slots[eoff[e] + __popc(bits[e] & ((1u << t) - 1u))] = f;
  }
  __syncthreads();
}

// Items of workgroup wg among n dealt round-robin over g workgroups.
__device__ __forceinline__ int items_of(int wg, int g, int n) { return wg < n ? (n - 1 - wg) / g + 1 : 0; }

template <int PER, int NSG, int NSD>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, const uint8_t* __restrict__ wgu,
    const uint8_t* __restrict__ sgu, const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd, uint16_t* hbuf,
    float* dpart, uint16_t* __restrict__ y, int32_t* ctl, int T, int H, int I, int E, int k) {
  __shared__ __attribute__((aligned(16))) uint8_t xbufs[2 * FUSED_XCHUNK];
  __shared__ __attribute__((aligned(16))) uint8_t slabs[WG_WAVES][SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sslabs[WG_WAVES][ScaleRun4::slab_bytes<2>()];
  __shared__ uint32_t xctr[2];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wg = blockIdx.x, n_wg = gridDim.x;
  if (tid < 2) xctr[tid] = 0u;
  fused_route_sort<PER>(logits, T, E, k, xbufs);
  const LdsSort meta;
  const int na = meta.num_active();
  // items dealt round-robin (T <= 16: one row group per expert, no extra groups)
  StaticUnits units;

  // ---------------------------------------------------------------- gate_up + SwiGLU
  using PG = GateUpPolicy<NSG, LdsSort, FUSED_XCHUNK, true>;
  const int n_gu = na * (I / (PG::TILE * WG_WAVES));
  {
    PG p;
    p.xrowsegs = XGeom<FUSED_XCHUNK>::ROWSEGS;
    p.nseg = H / SEG_K;
    p.nquad = I / (PG::TILE * WG_WAVES);
    p.na = na;
    p.n_items = n_gu;
    p.xact = x;
    p.wgu = wgu;
    p.sgu = sgu;
    p.h = hbuf;
    p.H = H;
    p.I = I;
    p.k = k;
    p.kinv = ((1u << 24) + (uint32_t)k - 1u) / (uint32_t)k;
    p.e_codes = (size_t)2 * I * (H / 2);
    p.e_scales = (size_t)2 * I * (H / 32);
    stream_items<PG, GU_SPS>(p, units, xbufs, xctr, slabs[wave], sslabs[wave], wave, lane);
  }
  // Publish: this workgroup's h stores are complete; add its item count.  The workgroup
  // whose count completes the total raises every replica of the ready flag.
  wait_own_stores();
  __syncthreads();
  if (tid == 0) {
    const int mine = items_of(wg, n_wg, n_gu);
    if (mine > 0) {
      const int old = __hip_atomic_fetch_add(&ctl[CTL_GU_DONE], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + mine == n_gu)
        for (int r = 0; r < CTL_READY_REPLICAS; ++r)
          __hip_atomic_store(&ctl[CTL_READY0 + r * CTL_READY_STRIDE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    xctr[0] = 0u;  // fresh chunk hand-off for the down items
    xctr[1] = 0u;
    fsort.h_ready = 0;
  }
  __syncthreads();

  // ---------------------------------------------------------------- down
  using PD = DownPolicy<NSD, LdsSort, FUSED_XCHUNK, true>;
  const int nquad_dn = H / (PD::TILE * WG_WAVES);
  const int n_dn = na * nquad_dn;
  {
    PD p;
    p.xrowsegs = XGeom<FUSED_XCHUNK>::ROWSEGS;
    p.nseg = I / SEG_K;
    p.nquad = nquad_dn;
    p.na = na;
    p.n_items = n_dn;
    p.xact = hbuf;
    p.wd = wd;
    p.sd = sd;
    p.dpart = dpart;
    p.H = H;
    p.I = I;
    p.e_codes = (size_t)H * (I / 2);
    p.e_scales = (size_t)H * (I / 32);
    p.ready = ctl + CTL_READY0 + (wg % CTL_READY_REPLICAS) * CTL_READY_STRIDE;
    p.err = ctl + CTL_ERR;
    p.flag = (lds_i32*)&fsort.h_ready;
    p.ready_target = 1;
    p.wave = wave;
    stream_items<PD, DN_SPS>(p, units, xbufs, xctr, slabs[wave], sslabs[wave], wave, lane);
  }
  wait_own_stores();
  __syncthreads();

  // ---------------------------------------------------------------- combine
  // Wave 0 counts this workgroup's items per column quad, 64 items per round; a quad is
  // complete when its count reaches na (one item per active expert, all valid for T <= 16).
  int32_t* done = reinterpret_cast<int32_t*>(xbufs);  // quads completed here (<= nquad_dn)
  if (wave == 0) {
    int nd = 0;
    for (int base = wg; base < n_dn; base += 64 * n_wg) {
      const int it = base + lane * n_wg;
      bool fin = false;
      int q = 0;
      if (it < n_dn) {
        q = it % nquad_dn;
        fin = __hip_atomic_fetch_add(&ctl[CTL_QUAD0 + q], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == na - 1;
      }
      const uint64_t m = __ballot(fin);
      if (fin) done[nd + __popcll(m & ((1ull << lane) - 1ull))] = q;
      nd += __popcll(m);
    }
    if (lane == 0) fsort.ndone = nd;
  }
  __syncthreads();
  constexpr int QV = PD::TILE * WG_WAVES / 4;  // 4-column groups per quad
  const int nd = fsort.ndone;
  for (int d = 0; d < nd; ++d) {
    const int c0 = done[d] * (QV * 4);
    for (int i = tid; i < T * QV; i += WG_WAVES * 64) {
      const int t = i / QV;
      const int n = c0 + (i - t * QV) * 4;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      // slots in batches of 8: all loads of a batch in flight at once, then the sum, j ascending
      for (int j0 = 0; j0 < k; j0 += 8) {
        u32x4 dv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          dv[jj] = ld16_coherent(dpart + (size_t)(t * k + min(j0 + jj, k - 1)) * H + n);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          if (j0 + jj < k) {
            const float g = fsort.gates[t * k + j0 + jj];
            acc += f32x4{g * __uint_as_float(dv[jj][0]), g * __uint_as_float(dv[jj][1]),
                         g * __uint_as_float(dv[jj][2]), g * __uint_as_float(dv[jj][3])};
          }
        }
      }
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
      *reinterpret_cast<u32x2*>(y + (size_t)t * H + n) = u32x2{lo, hi};
    }
  }

  // ---------------------------------------------------------------- exit
  // Every workgroup's counter updates precede its exit count; the last one resets them.
  __syncthreads();
  if (tid == 0)
    fsort.last = __hip_atomic_fetch_add(&ctl[CTL_EXIT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_wg - 1;
  __syncthreads();
  if (fsort.last) {
    for (int i = tid; i < nquad_dn; i += WG_WAVES * 64)
      __hip_atomic_store(&ctl[CTL_QUAD0 + i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < CTL_READY_REPLICAS)
      __hip_atomic_store(&ctl[CTL_READY0 + tid * CTL_READY_STRIDE], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(&ctl[CTL_GU_DONE], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctl[CTL_EXIT], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ gate_up with its own routing

// The layer forward's gate_up launch for small T.  Every workgroup routes all T tokens and
// sorts the slots into LDS itself (fused_route_sort, as the persistent layer does), so no
// route + sort launch precedes it and the item metadata comes from LDS instead of a chain of
// dependent loads.  Workgroup 0 also writes what the down launch needs to the workspace: the
// counts and offsets of all E experts, the sorted slots, the gates, the active list and
// {active experts, largest count}.  Its active list is in ascending expert order, not row
// class order; the down launch accepts any order, since its items and outputs are indexed
// by expert and sorted position.  h is identical to that of the stage entry points
// (moe_route_sort, then moe_gate_up_swiglu): the same rows at the same sorted positions.
// Nothing waits on another workgroup.
struct SortOut {
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slots;
  int32_t* active;
  int32_t* num_active;
};

template <int PER, int NS, int SPS, bool A8>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_gate_up_routed_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, const uint8_t* __restrict__ wgu,
    const uint8_t* __restrict__ sgu, uint16_t* __restrict__ h, SortOut out, float* __restrict__ gates, int T, int H,
    int I, int E, int k) {
  __shared__ __attribute__((aligned(16))) uint8_t xbufs[2 * GU_XCHUNK];
  __shared__ __attribute__((aligned(16))) uint8_t slabs[WG_WAVES][SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sslabs[WG_WAVES][ScaleRun4::slab_bytes<NS>()];
  __shared__ uint32_t xctr[2];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (tid < 2) xctr[tid] = 0u;
  fused_route_sort<PER>(logits, T, E, k, xbufs);
  const LdsSort meta;
  const int na = meta.num_active();
  if (blockIdx.x == 0) {
    // the token masks and expert offsets are still in the routing scratch (xbufs)
    const uint32_t* bits = reinterpret_cast<const uint32_t*>(xbufs);
    const int32_t* eoff = reinterpret_cast<const int32_t*>(xbufs + 4096);
    for (int e = tid; e < E; e += WG_WAVES * 64) {
      out.counts[e] = __popc(bits[e]);
      out.offsets[e] = eoff[e];
    }
    for (int i = tid; i < T * k; i += WG_WAVES * 64) {
      out.sorted_slots[i] = fsort.slots[i];
      gates[i] = fsort.gates[i];
    }
    for (int a = tid; a < na; a += WG_WAVES * 64) out.active[a] = fsort.act[a];
    if (wave == 0) {
      int m = 0;
      for (int a = lane; a < na; a += 64) m = max(m, fsort.cnt[a]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
      if (lane == 0) {
        out.offsets[E] = T * k;
        out.num_active[0] = na;
        out.num_active[1] = m;
      }
    }
  }
  __syncthreads();  // the routing scratch has been read; the stream reuses xbufs
  using PG = GateUpPolicy<NS, LdsSort, GU_XCHUNK, false, A8>;
  PG p;
  p.xrowsegs = XGeom<GU_XCHUNK>::ROWSEGS;
  p.calign = SPS;
  p.nseg = H / SEG_K;
  p.nquad = I / (PG::TILE * WG_WAVES);
  p.na = na;
  p.n_items = na * p.nquad;  // T <= 16: one row group per expert
  p.xact = x;
  p.wgu = wgu;
  p.sgu = sgu;
  p.h = h;
  p.H = H;
  p.I = I;
  p.k = k;
  p.kinv = ((1u << 24) + (uint32_t)k - 1u) / (uint32_t)k;
  p.e_codes = (size_t)2 * I * (H / 2);
  p.e_scales = (size_t)2 * I * (H / 32);
  StaticUnits units;
  stream_items<PG, SPS>(p, units, xbufs, xctr, slabs[wave], sslabs[wave], wave, lane);
}

template <class K>
static int routed_occupancy(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, WG_WAVES * 64, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

// Tiles and grid as the gate_up launch chooses them: half-width tiles when full-width items
// would leave resident slots idle and twice the items still fit in one round, and then
// 4-segment steps while the items are fewer than the slots.
// A8: MXFP8 activations (the deeper ring's registers are not available there)
template <int PER, bool A8>
static int launch_routed_per(const uint16_t* x, const float* logits, const uint8_t* wgu, const uint8_t* sgu,
                             uint16_t* h, const SortOut& out, float* gates, int T, int H, int I, int E, int k,
                             hipStream_t stream) {
  static const int occ2 = routed_occupancy(moe_gate_up_routed_kernel<PER, 2, GU_SPS, A8>);
  static const int occ1 = routed_occupancy(moe_gate_up_routed_kernel<PER, 1, GU_SPS, A8>);
  const int64_t na_max = (int64_t)T * k < E ? (int64_t)T * k : E;
  const int64_t items_full = na_max * (I / (SUB_ROWS * WG_WAVES));
  const int64_t cus = device_cu_count();
  const dim3 block(WG_WAVES * 64);
  if (2 * items_full > cus * occ1) {
    const dim3 grid((unsigned)(items_full < cus * occ2 ? items_full : cus * occ2));
    hipLaunchKernelGGL((moe_gate_up_routed_kernel<PER, 2, GU_SPS, A8>), grid, block, 0, stream, x, logits, wgu, sgu,
                       h, out, gates, T, H, I, E, k);
    return hip_status(hipGetLastError());
  }
  const dim3 grid((unsigned)(2 * items_full));
  if constexpr (!A8) {
    if (H % (SEG_K * GU_SPS_DEEP) == 0 && 2 * items_full < cus * occ1) {
      hipLaunchKernelGGL((moe_gate_up_routed_kernel<PER, 1, GU_SPS_DEEP, A8>), grid, block, 0, stream, x, logits, wgu,
                         sgu, h, out, gates, T, H, I, E, k);
      return hip_status(hipGetLastError());
    }
  }
  hipLaunchKernelGGL((moe_gate_up_routed_kernel<PER, 1, GU_SPS, A8>), grid, block, 0, stream, x, logits, wgu, sgu, h,
                     out, gates, T, H, I, E, k);
  return hip_status(hipGetLastError());
}

// ------------------------------------------------------------------ gate_up with its own sort

// For 16 < T <= 32 the forward launches the routing alone (moe_route_kernel writes the ids
// and gates), and every gate_up workgroup sorts the T k slots into LDS itself, replacing
// the sort launch and the chain of dependent metadata loads at each item.  (Routing in
// every workgroup, as the T <= 16 launch does, costs more than a launch at 32 tokens: each
// wave would route 8 tokens one after another.)  The sort is the sort kernel's: counts and
// offsets in expert order, slots stable by flat slot, the active list by row class
// (heaviest first) and then expert id (-1 after the last); workgroup 0 writes it for the
// down launch, equal to moe_sort_by_expert's on the same ids.
constexpr int SORTED_MAX_T = 32;        // one 32-bit token mask per expert
constexpr int SORTED_MAX_SLOTS = 256;   // T * k

struct WgSort {
  int32_t act[SORTED_MAX_SLOTS];      // expert of active expert a
  int32_t cnt_off[SORTED_MAX_SLOTS];  // its count | its first sorted position << 16
  int32_t slots[SORTED_MAX_SLOTS];    // flat slot at each sorted position
  int32_t na;                         // active experts
  int32_t max_rows;                   // largest count
  int32_t wave_sum[WG_WAVES];
  int32_t wave_max[WG_WAVES];
  uint64_t wave_cls[WG_WAVES];
};
typedef __attribute__((address_space(3))) WgSort lds_wgsort;

struct LdsSortW {
  lds_wgsort* s;
  __device__ __forceinline__ int num_active() const { return __builtin_amdgcn_readfirstlane(s->na); }
  __device__ __forceinline__ int max_rows() const { return __builtin_amdgcn_readfirstlane(s->max_rows); }
  __device__ __forceinline__ int expert(int a) const { return __builtin_amdgcn_readfirstlane(s->act[a]); }
  __device__ __forceinline__ int count(int a) const { return __builtin_amdgcn_readfirstlane(s->cnt_off[a] & 0xFFFF); }
  __device__ __forceinline__ int offset(int a) const { return __builtin_amdgcn_readfirstlane(s->cnt_off[a] >> 16); }
  __device__ __forceinline__ int slot(int i) const { return __builtin_amdgcn_readfirstlane(s->slots[i]); }
  __device__ __forceinline__ int count_lane(int a) const { return s->cnt_off[a] & 0xFFFF; }
};

// Row class as the sort kernel ranks it: 3 for 8 or more rows, 2 for 4-7, 1 for 2-3, 0 for 1.
__device__ __forceinline__ int wg_row_class(int c) { return c >= 8 ? 3 : c >= 4 ? 2 : c >= 2 ? 1 : 0; }

// Inclusive scan over the workgroup's threads (4 wavefronts) of a per-thread value, with
// the wavefront totals in `ws`; returns the exclusive prefix and the total.
template <class V, class WS>
__device__ __forceinline__ V wg_exclusive_scan(V v, WS ws, V& total, int lane, int wave) {
  V incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const V o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) ws[wave] = incl;
  __syncthreads();
  V before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < WG_WAVES; ++w) {
    if (w < wave) before += ws[w];
    total += ws[w];
  }
  return incl - v + before;
}

// The workgroup's sort of the T * k routed slots (ids: [T, k], T <= 32, E <= 1024) into
// *ws, with `tmp` as 8 KB of scratch (token masks and expert offsets).  Each thread takes
// 4 consecutive experts.  Must be called by all threads.
__device__ __forceinline__ void wg_sort_slots(const int32_t* __restrict__ ids, int T, int E, int k, lds_wgsort* ws,
                                              uint8_t* __restrict__ tmp) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(tmp);       // [E] token masks
  int32_t* eoff = reinterpret_cast<int32_t*>(tmp + 4096);  // [E] first sorted position
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int F = T * k;
  for (int i = tid; i < E; i += WG_WAVES * 64) bits[i] = 0u;
  __syncthreads();
  const int my_e = (tid < F) ? ids[tid] : -1;  // F <= 256 = one slot per thread
  if (my_e >= 0 && my_e < E) atomicOr(&bits[my_e], 1u << (tid / k));
  __syncthreads();
  int c[4];
  int packed = 0, most = 0;
  uint64_t cls = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    c[q] = (e < E) ? __popc(bits[e]) : 0;
    packed += c[q] | (c[q] > 0 ? (1 << 16) : 0);
    if (c[q] > 0) cls += 1ull << (16 * wg_row_class(c[q]));
    most = max(most, c[q]);
  }
  int ptot;
  int run = wg_exclusive_scan(packed, ws->wave_sum, ptot, lane, wave);
  uint64_t ctot;
  uint64_t crun = wg_exclusive_scan(cls, ws->wave_cls, ctot, lane, wave);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) most = max(most, __shfl_xor(most, off));
  if (lane == 0) ws->wave_max[wave] = most;
  // the active list: heavier classes first (the totals of the classes above), then by id
  int base[4];
#pragma unroll
  for (int cl = 0; cl < 4; ++cl) {
    base[cl] = 0;
    for (int d = cl + 1; d < 4; ++d) base[cl] += (int)((ctot >> (16 * d)) & 0xFFFFu);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < E) {
      eoff[e] = run & 0xFFFF;
      if (c[q] > 0) {
        const int cl = wg_row_class(c[q]);
        const int a = base[cl] + (int)((crun >> (16 * cl)) & 0xFFFFu);
        ws->act[a] = e;
        ws->cnt_off[a] = c[q] | ((run & 0xFFFF) << 16);
        crun += 1ull << (16 * cl);
      }
    }
    run += c[q] | (c[q] > 0 ? (1 << 16) : 0);
  }
  __syncthreads();
  if (tid == 0) {
    ws->na = ptot >> 16;
    int m = 0;
    for (int w = 0; w < WG_WAVES; ++w) m = max(m, ws->wave_max[w]);
    ws->max_rows = m;
  }
  if (my_e >= 0 && my_e < E) {
    const int t = tid / k;
    ws->slots[eoff[my_e] + __popc(bits[my_e] & ((1u << t) - 1u))] = tid;
  }
  __syncthreads();
}

template <int NS, int SPS, bool A8>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_gate_up_sorted_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const uint8_t* __restrict__ wgu,
    const uint8_t* __restrict__ sgu, uint16_t* __restrict__ h, SortOut out, int T, int H, int I, int E, int k,
    int32_t* claim) {
  __shared__ __attribute__((aligned(16))) uint8_t xbufs[2 * GU_XCHUNK];
  __shared__ __attribute__((aligned(16))) uint8_t slabs[WG_WAVES][SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sslabs[WG_WAVES][ScaleRun4::slab_bytes<NS>()];
  __shared__ uint32_t xctr[2];
  __shared__ int32_t cq[4];
  __shared__ WgSort wsort;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (tid < 2) xctr[tid] = 0u;
  lds_wgsort* ws = (lds_wgsort*)&wsort;
  wg_sort_slots(ids, T, E, k, ws, xbufs);
  const LdsSortW meta{ws};
  const int na = meta.num_active();
  if (blockIdx.x == 0) {
    // the token masks and expert offsets are still in the sort scratch (xbufs)
    const uint32_t* bits = reinterpret_cast<const uint32_t*>(xbufs);
    const int32_t* eoff = reinterpret_cast<const int32_t*>(xbufs + 4096);
    for (int e = tid; e < E; e += WG_WAVES * 64) {
      out.counts[e] = __popc(bits[e]);
      out.offsets[e] = eoff[e];
    }
    for (int i = tid; i < T * k; i += WG_WAVES * 64) out.sorted_slots[i] = ws->slots[i];
    for (int a = tid; a < E; a += WG_WAVES * 64) out.active[a] = a < na ? ws->act[a] : -1;
    if (tid == 0) {
      out.offsets[E] = T * k;
      out.num_active[0] = na;
      out.num_active[1] = ws->max_rows;
    }
  }
  __syncthreads();  // the sort scratch has been read; the stream reuses xbufs
  using PG = GateUpPolicy<NS, LdsSortW, GU_XCHUNK, false, A8>;
  PG p;
  p.m = meta;
  p.xrowsegs = XGeom<GU_XCHUNK>::ROWSEGS;
  p.calign = SPS;
  p.nseg = H / SEG_K;
  p.nquad = I / (PG::TILE * WG_WAVES);
  p.na = na;
  p.n_items = ((meta.max_rows() + 15) >> 4) * na * p.nquad;  // row-group levels that exist
  p.xact = x;
  p.wgu = wgu;
  p.sgu = sgu;
  p.h = h;
  p.H = H;
  p.I = I;
  p.k = k;
  p.kinv = ((1u << 24) + (uint32_t)k - 1u) / (uint32_t)k;
  p.e_codes = (size_t)2 * I * (H / 2);
  p.e_scales = (size_t)2 * I * (H / 32);
  ClaimedUnits seq{claim, (lds_i32*)cq, na * p.nquad, 0, false};
  stream_items<PG, SPS>(p, seq, xbufs, xctr, slabs[wave], sslabs[wave], wave, lane);
  seq.finish();
}

template <bool A8>
static int launch_sorted_run(const uint16_t* x, const int32_t* ids, const uint8_t* wgu, const uint8_t* sgu,
                             uint16_t* h, const SortOut& out, int32_t* claim, int T, int H, int I, int E, int k,
                             hipStream_t stream) {
  static const int occ2 = routed_occupancy(moe_gate_up_sorted_kernel<2, GU_SPS, A8>);
  static const int occ1 = routed_occupancy(moe_gate_up_sorted_kernel<1, GU_SPS, A8>);
  const int64_t na_max = (int64_t)T * k < E ? (int64_t)T * k : E;
  const int64_t items_full = ((T + 15) / 16) * na_max * (I / (SUB_ROWS * WG_WAVES));
  const int64_t cus = device_cu_count();
  const dim3 block(WG_WAVES * 64);
  if (2 * items_full > cus * occ1) {
    const dim3 grid((unsigned)(items_full < cus * occ2 ? items_full : cus * occ2));
    hipLaunchKernelGGL((moe_gate_up_sorted_kernel<2, GU_SPS, A8>), grid, block, 0, stream, x, ids, wgu, sgu, h, out,
                       T, H, I, E, k, claim);
  } else {
    const dim3 grid((unsigned)(2 * items_full));
    hipLaunchKernelGGL((moe_gate_up_sorted_kernel<1, GU_SPS, A8>), grid, block, 0, stream, x, ids, wgu, sgu, h, out,
                       T, H, I, E, k, claim);
  }
  return hip_status(hipGetLastError());
}

bool gate_up_sorted_fits(int T, int E, int k, int H, int I) {
  return T <= SORTED_MAX_T && T * k <= SORTED_MAX_SLOTS && E <= 1024 && H % (SEG_K * GU_SPS) == 0 &&
         H % (SEG_K * SRUN) == 0 && I % (SUB_ROWS * WG_WAVES) == 0;
}

int launch_gate_up_sorted(const uint16_t* x, const int32_t* ids, const uint8_t* wgu, const uint8_t* sgu, uint16_t* h,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* active,
                          int32_t* num_active, int32_t* ctl, int T, int H, int I, int E, int k, bool act8,
                          hipStream_t stream) {
  if (!gate_up_sorted_fits(T, E, k, H, I)) return MX_ERR_SHAPE;
  const SortOut out{counts, offsets, sorted_slots, active, num_active};
  if (act8) return launch_sorted_run<true>(x, ids, wgu, sgu, h, out, ctl + CTL_CLAIM_GU, T, H, I, E, k, stream);
  return launch_sorted_run<false>(x, ids, wgu, sgu, h, out, ctl + CTL_CLAIM_GU, T, H, I, E, k, stream);
}

// ------------------------------------------------------------------ gate_up and down in one launch

// Up to 32 tokens, wherever the gate_up items can be 3 or more per resident workgroup (from 6
// tokens at top-8), the forward runs both expert GEMMs in one launch, so that down's items
// fill the end of gate_up's: a workgroup whose gate_up claims run out starts on down items
// at once, instead of idling until the slowest workgroup of a gate_up launch finishes (13 us
// of idle per workgroup on average at 32 tokens, Zipf routing) and then paying a launch
// boundary and down's start-up.  The pages' own step ("Zyphra Inference Wave 2", Kernel
// Results) fused both GEMMs into one kernel body and spilled registers; here the two phases
// share the launch, not the body: each workgroup streams its gate_up items to the end
// (stream_items), then its down items, through the same LDS.
//
// Hand-off of h without flags: h is filled with 0xFFFF before the launch (by the routing
// launch; the kernel boundary leaves no older copy of it in any cache), gate_up writes each
// element once with device-coherent stores, and a down wave that loads an 0xFFFF (not yet
// written, or a NaN with that bit pattern) waits until every workgroup has finished its
// gate_up phase and loads again, coherently (xchunk_settle).  Items are
// taken in the same expert order in both phases, so down reaches an expert long after its
// gate_up items finished and the wait is practically never taken; a per-item flag written
// by gate_up was measured instead and cost 3-40 us at 32 tokens (stores and atomics from
// many workgroups into a few cache lines queue behind one another).
//
// Workgroups wait for one another only in that rare case, and only for workgroups of the
// launch to finish their gate_up items, which need nothing from anyone: the grid is sized to
// what the device holds at once at this kernel's occupancy, so every workgroup runs.  A wait
// that outlasts SPIN_LIMIT polls sets the error word and goes on.  The last workgroup to
// exit resets the counters, so the control words are zero again after the launch.
// The down phase runs at gate_up's occupancy (2 workgroups per CU, not down's 3), so its
// waves keep two steps of 2 segments in flight instead of one; the registers are there (205).
// Measured: T = 32 Zipf 380.4 -> 379.7 us per layer, uniform T = 32 587.6 -> 585.6.
constexpr int DN_SPS_DEEP = 4;
static_assert(SRUN % DN_SPS_DEEP == 0, "scale runs end on steps");

template <int NS, class Meta, class SR, bool A8>
struct DownAfterGateUp : DownPolicy<NS, Meta, GU_XCHUNK, false, SR, A8, false> {
  static constexpr bool SENTINEL = true;
  // (ready: workgroups past their gate_up items; ready_target: the grid; err: the error word)
  __device__ __forceinline__ void wait_all_written() const {
    for (uint32_t n = 0;; ++n) {
      const int v =
          __builtin_amdgcn_readfirstlane(__hip_atomic_load(this->ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (v >= this->ready_target) break;
      if (n == SPIN_LIMIT) {
        __hip_atomic_store(this->err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
};

// LDS of the single expert launch (besides the sort it may hold)
struct ExpertsLds {
  uint8_t* xbufs;    // 2 * GU_XCHUNK
  uint8_t* slabs;    // WG_WAVES * SLAB_BYTES
  uint8_t* sslabs;   // WG_WAVES * ScaleRun4::slab_bytes<2>()
  uint32_t* xctr;    // 2
  int32_t* cq;       // 4
  int32_t* last;     // 1
};

// Both phases and the exit, for the sort in `meta` (the workgroup's own in LDS, or the sort
// launches' in global memory); A8: MXFP8 activations (x and h quantized as they are staged).
template <bool A8, class Meta>
__device__ __forceinline__ void experts_phases(const Meta& meta, const ExpertsLds& L, const uint16_t* __restrict__ x,
                                               const uint8_t* __restrict__ wgu, const uint8_t* __restrict__ sgu,
                                               const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd,
                                               uint16_t* h, float* __restrict__ dpart, int32_t* ctl, int H, int I,
                                               int k) {
  constexpr int SSLAB = ScaleRun4::slab_bytes<2>();
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int na = meta.num_active();
  const int levels = (meta.max_rows() + 15) >> 4;  // row-group levels that exist

  // ---------------------------------------------------------------- gate_up + SwiGLU
  {
    using PG = GateUpPolicy<2, Meta, GU_XCHUNK, true, A8>;
    PG p;
    p.m = meta;
    p.xrowsegs = XGeom<GU_XCHUNK>::ROWSEGS;
    p.calign = GU_SPS;
    p.nseg = H / SEG_K;
    p.nquad = I / (PG::TILE * WG_WAVES);
    p.na = na;
    p.n_items = levels * na * p.nquad;
    p.xact = x;
    p.wgu = wgu;
    p.sgu = sgu;
    p.h = h;
    p.H = H;
    p.I = I;
    p.k = k;
    p.kinv = ((1u << 24) + (uint32_t)k - 1u) / (uint32_t)k;
    p.e_codes = (size_t)2 * I * (H / 2);
    p.e_scales = (size_t)2 * I * (H / 32);
    ClaimedUnits seq{ctl + CTL_CLAIM_GU, (lds_i32*)L.cq, na * p.nquad, 0, false};
    stream_items<PG, GU_SPS>(p, seq, L.xbufs, L.xctr, L.slabs + wave * SLAB_BYTES, L.sslabs + wave * SSLAB, wave,
                             lane);
    seq.finish();
  }
  // this workgroup's h stores are complete; count it, and start a fresh chunk hand-off
  wait_own_stores();
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_fetch_add(&ctl[CTL_GU_DONE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    L.xctr[0] = 0u;
    L.xctr[1] = 0u;
  }
  __syncthreads();

  // ---------------------------------------------------------------- down
  {
    using PD = DownAfterGateUp<2, Meta, ScaleRun4, A8>;
    constexpr int SPS = A8 ? DN_SPS : DN_SPS_DEEP;  // the MXFP8 phase has no registers for the deeper ring
    PD p;
    p.m = meta;
    p.xrowsegs = XGeom<GU_XCHUNK>::ROWSEGS;
    p.calign = SPS;
    p.nseg = I / SEG_K;
    p.nquad = H / (PD::TILE * WG_WAVES);
    p.na = na;
    p.n_items = levels * na * p.nquad;
    p.xact = h;
    p.wd = wd;
    p.sd = sd;
    p.dpart = dpart;
    p.H = H;
    p.I = I;
    p.e_codes = (size_t)H * (I / 2);
    p.e_scales = (size_t)H * (I / 32);
    p.ready = ctl + CTL_GU_DONE;
    p.ready_target = (int)gridDim.x;
    p.err = ctl + CTL_ERR;
    p.flag = nullptr;
    p.wave = wave;
    ClaimedUnits seq{ctl + CTL_CLAIM_DN, (lds_i32*)L.cq, na * p.nquad, 0, false};
    stream_items<PD, SPS>(p, seq, L.xbufs, L.xctr, L.slabs + wave * SLAB_BYTES, L.sslabs + wave * SSLAB, wave,
                                  lane);
    seq.finish();
  }

  // ---------------------------------------------------------------- exit
  __syncthreads();
  if (tid == 0)
    *L.last = __hip_atomic_fetch_add(&ctl[CTL_EXIT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (int)gridDim.x - 1;
  __syncthreads();
  if (*L.last && tid == 0) {
    __hip_atomic_store(&ctl[CTL_GU_DONE], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctl[CTL_EXIT], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

#define MX_EXPERTS_LDS                                                                   \
  __shared__ __attribute__((aligned(16))) uint8_t xbufs[2 * GU_XCHUNK];                   \
  __shared__ __attribute__((aligned(16))) uint8_t slabs[WG_WAVES * SLAB_BYTES];           \
  __shared__ __attribute__((aligned(16))) uint8_t sslabs[WG_WAVES * ScaleRun4::slab_bytes<2>()]; \
  __shared__ uint32_t xctr[2];                                                            \
  __shared__ int32_t cq[4];                                                               \
  __shared__ int32_t last;                                                                \
  const ExpertsLds lds{xbufs, slabs, sslabs, xctr, cq, &last};                            \
  if (threadIdx.x < 2) xctr[threadIdx.x] = 0u

// T <= 32: every workgroup sorts the routed ids itself.
template <bool A8>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_experts_sorted_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const uint8_t* __restrict__ wgu,
    const uint8_t* __restrict__ sgu, const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd, uint16_t* h,
    float* __restrict__ dpart, int32_t* ctl, int T, int H, int I, int E, int k) {
  MX_EXPERTS_LDS;
  __shared__ WgSort wsort;
  lds_wgsort* ws = (lds_wgsort*)&wsort;
  wg_sort_slots(ids, T, E, k, ws, xbufs);  // ends with a barrier: xbufs is free again
  experts_phases<A8>(LdsSortW{ws}, lds, x, wgu, sgu, wd, sd, h, dpart, ctl, H, I, k);
}

// Any T: the sort launches' result in global memory.
template <bool A8>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_experts_kernel(
    const uint16_t* __restrict__ x, SortView sv, const uint8_t* __restrict__ wgu, const uint8_t* __restrict__ sgu,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd, uint16_t* h, float* __restrict__ dpart,
    int32_t* ctl, int H, int I, int k) {
  MX_EXPERTS_LDS;
  __syncthreads();
  experts_phases<A8>(GlobalSort{sv}, lds, x, wgu, sgu, wd, sd, h, dpart, ctl, H, I, k);
}
#undef MX_EXPERTS_LDS

// The sort fits one workgroup and I and H take 4-segment scale runs and 4- and 2-segment
// steps.  The launch is correct for any number of items (workgroups without any pass
// through); whether it pays is experts_sorted_pays.
bool experts_sorted_fits(int T, int E, int k, int H, int I) {
  return gate_up_sorted_fits(T, E, k, H, I) && I % (SEG_K * SRUN) == 0 && I % (SEG_K * DN_SPS_DEEP) == 0 &&
         H % (2 * SUB_ROWS * WG_WAVES) == 0;
}

// The single launch pays once the gate_up items are at least 3 per resident workgroup
// (512 on MI355X) when every slot routes to its own expert.  With fewer, every expert's
// gate_up items finish in the last round, so down waits for the whole gate_up phase while
// the early workgroups' down weight loads take bandwidth from gate_up's last items:
// measured against the separate launches, T = 2 75.7 -> 82.1 and T = 4 125.2 -> 154.8 us per
// layer (1 and 2 items per workgroup), but T = 8 220.3 -> 217.4 and T = 16 392.1 -> 387.4.
constexpr int64_t EXPERTS_MIN_ITEMS = 3 * 512;
bool experts_sorted_pays(int T, int E, int k, int I) {
  const int64_t na_max = (int64_t)T * k < E ? (int64_t)T * k : E;
  return na_max * (I / (SUB_ROWS * WG_WAVES)) >= EXPERTS_MIN_ITEMS;
}

template <bool A8>
static int launch_experts_sorted_run(const uint16_t* x, const int32_t* ids, const uint8_t* wgu, const uint8_t* sgu,
                                     const uint8_t* wd, const uint8_t* sd, uint16_t* h, float* dpart, int32_t* ctl,
                                     int T, int H, int I, int E, int k, hipStream_t stream) {
  static const int occ = routed_occupancy(moe_experts_sorted_kernel<A8>);
  const dim3 grid((unsigned)(device_cu_count() * occ)), block(WG_WAVES * 64);
  hipLaunchKernelGGL(moe_experts_sorted_kernel<A8>, grid, block, 0, stream, x, ids, wgu, sgu, wd, sd, h, dpart, ctl, T,
                     H, I, E, k);
  return hip_status(hipGetLastError());
}

int launch_experts_sorted(const uint16_t* x, const int32_t* ids, const uint8_t* wgu, const uint8_t* sgu,
                          const uint8_t* wd, const uint8_t* sd, uint16_t* h, float* dpart, int32_t* ctl, int T, int H,
                          int I, int E, int k, bool act8, hipStream_t stream) {
  if (!experts_sorted_fits(T, E, k, H, I)) return MX_ERR_SHAPE;
  if (act8) return launch_experts_sorted_run<true>(x, ids, wgu, sgu, wd, sd, h, dpart, ctl, T, H, I, E, k, stream);
  return launch_experts_sorted_run<false>(x, ids, wgu, sgu, wd, sd, h, dpart, ctl, T, H, I, E, k, stream);
}

bool experts_fits(int H, int I) {
  return H % (SEG_K * GU_SPS) == 0 && H % (SEG_K * SRUN) == 0 && I % (SEG_K * SRUN) == 0 &&
         I % (SEG_K * DN_SPS_DEEP) == 0 && H % (2 * SUB_ROWS * WG_WAVES) == 0;
}

template <bool A8>
static int launch_experts_run(const uint16_t* x, const SortView& sv, const uint8_t* wgu, const uint8_t* sgu,
                              const uint8_t* wd, const uint8_t* sd, uint16_t* h, float* dpart, int32_t* ctl, int H,
                              int I, int k, hipStream_t stream) {
  static const int occ = routed_occupancy(moe_experts_kernel<A8>);
  const dim3 grid((unsigned)(device_cu_count() * occ)), block(WG_WAVES * 64);
  hipLaunchKernelGGL(moe_experts_kernel<A8>, grid, block, 0, stream, x, sv, wgu, sgu, wd, sd, h, dpart, ctl, H, I, k);
  return hip_status(hipGetLastError());
}

int launch_experts(const uint16_t* x, const SortView& sv, const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd,
                   const uint8_t* sd, uint16_t* h, float* dpart, int32_t* ctl, int H, int I, int k, bool act8,
                   hipStream_t stream) {
  if (!experts_fits(H, I)) return MX_ERR_SHAPE;
  if (act8) return launch_experts_run<true>(x, sv, wgu, sgu, wd, sd, h, dpart, ctl, H, I, k, stream);
  return launch_experts_run<false>(x, sv, wgu, sgu, wd, sd, h, dpart, ctl, H, I, k, stream);
}

// Measured against the route + sort launch followed by gate_up (graph replay, 4 layers):
// T = 1 50.0 -> 46.7 us per layer, T = 2 81.4 -> 77.9, T = 4 132.0 -> 127.8, T = 8 226.8 ->
// 223.1, T = 16 392.4 -> 391.2.
bool gate_up_routed_fits(int T, int E, int k, int H, int I) {
  (void)E;
  return T <= MX_FUSED_MAX_TOKENS && T * k <= FUSED_MAX_SLOTS && H % (SEG_K * GU_SPS) == 0 &&
         H % (SEG_K * SRUN) == 0 && I % (SUB_ROWS * WG_WAVES) == 0;
}

int launch_gate_up_routed(const uint16_t* x, const float* logits, const uint8_t* wgu, const uint8_t* sgu, uint16_t* h,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* active,
                          int32_t* num_active, float* gates, int T, int H, int I, int E, int k, bool act8,
                          hipStream_t stream) {
  if (!gate_up_routed_fits(T, E, k, H, I)) return MX_ERR_SHAPE;
  const SortOut out{counts, offsets, sorted_slots, active, num_active};
  if (act8) {
    switch (route_per(E)) {
      case 4: return launch_routed_per<4, true>(x, logits, wgu, sgu, h, out, gates, T, H, I, E, k, stream);
      case 8: return launch_routed_per<8, true>(x, logits, wgu, sgu, h, out, gates, T, H, I, E, k, stream);
      default: return launch_routed_per<16, true>(x, logits, wgu, sgu, h, out, gates, T, H, I, E, k, stream);
    }
  }
  switch (route_per(E)) {
    case 4: return launch_routed_per<4, false>(x, logits, wgu, sgu, h, out, gates, T, H, I, E, k, stream);
    case 8: return launch_routed_per<8, false>(x, logits, wgu, sgu, h, out, gates, T, H, I, E, k, stream);
    default: return launch_routed_per<16, false>(x, logits, wgu, sgu, h, out, gates, T, H, I, E, k, stream);
  }
}

// ------------------------------------------------------------------ launcher

template <int PER, int NSG, int NSD>
static int fused_launch_one(const uint16_t* x, const float* logits, const uint8_t* wgu, const uint8_t* sgu,
                            const uint8_t* wd, const uint8_t* sd, uint16_t* hbuf, float* dpart, uint16_t* y,
                            int32_t* ctl, int T, int H, int I, int E, int k, int64_t items, hipStream_t stream) {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_fused_kernel<PER, NSG, NSD>, WG_WAVES * 64, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t cap = (int64_t)device_cu_count() * occ;
  const int grid = (int)(items < cap ? items : cap);
  hipLaunchKernelGGL((moe_fused_kernel<PER, NSG, NSD>), dim3(grid), dim3(WG_WAVES * 64), 0, stream, x, logits, wgu,
                     sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k);
  return hip_status(hipGetLastError());
}

template <int PER>
static int fused_launch_per(bool gu_half, bool dn_half, const uint16_t* x, const float* logits, const uint8_t* wgu,
                            const uint8_t* sgu, const uint8_t* wd, const uint8_t* sd, uint16_t* hbuf, float* dpart,
                            uint16_t* y, int32_t* ctl, int T, int H, int I, int E, int k, int64_t items,
                            hipStream_t stream) {
  if (gu_half)
    return dn_half ? fused_launch_one<PER, 1, 1>(x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k, items, stream)
                   : fused_launch_one<PER, 1, 2>(x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k, items, stream);
  return dn_half ? fused_launch_one<PER, 2, 1>(x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k, items, stream)
                 : fused_launch_one<PER, 2, 2>(x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k, items, stream);
}

bool fused_layer_fits(int T, int E, int k, int H, int I) {
  (void)E;
  return T <= MX_FUSED_MAX_TOKENS && T * k <= FUSED_MAX_SLOTS && H % (SEG_K * GU_SPS) == 0 &&
         H % (SEG_K * SRUN) == 0 && I % (SEG_K * DN_SPS) == 0 && I % (SEG_K * SRUN) == 0 &&
         I % (SUB_ROWS * WG_WAVES) == 0 && H % (2 * SUB_ROWS * WG_WAVES) == 0 && H / (SUB_ROWS * WG_WAVES) <= CTL_MAX_QUADS;
}

int launch_moe_fused(const uint16_t* x, const float* logits, const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd,
                     const uint8_t* sd, uint16_t* hbuf, float* dpart, uint16_t* y, int32_t* ctl, int T, int H, int I,
                     int E, int k, hipStream_t stream) {
  if (!fused_layer_fits(T, E, k, H, I)) return MX_ERR_SHAPE;
  // Half-width tiles when full-width ones would leave the device's workgroup slots idle
  // (two resident workgroups per CU): the same rule as the multi-launch path.
  const int64_t na_max = (int64_t)T * k < E ? (int64_t)T * k : E;
  const int64_t slots = (int64_t)device_cu_count() * 2;
  const int64_t gu_full = na_max * (I / (SUB_ROWS * WG_WAVES));
  const int64_t dn_full = na_max * (H / (2 * SUB_ROWS * WG_WAVES));
  const bool gu_half = 2 * gu_full <= slots, dn_half = 2 * dn_full <= slots;
  const int64_t gu_items = gu_half ? 2 * gu_full : gu_full, dn_items = dn_half ? 2 * dn_full : dn_full;
  const int64_t items = gu_items > dn_items ? gu_items : dn_items;
  switch (route_per(E)) {
    case 4:
      return fused_launch_per<4>(gu_half, dn_half, x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k,
                                 items, stream);
    case 8:
      return fused_launch_per<8>(gu_half, dn_half, x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k,
                                 items, stream);
    default:
      return fused_launch_per<16>(gu_half, dn_half, x, logits, wgu, sgu, wd, sd, hbuf, dpart, y, ctl, T, H, I, E, k,
                                  items, stream);
  }
}

}  // namespace mx
