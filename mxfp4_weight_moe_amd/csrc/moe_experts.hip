// The two expert GEMM kernels of the MXFP4 MoE layer (work lists and epilogues in
// moe_policies.hpp) and the combine, for launches that follow the sort kernels.
//
// "Zyphra Inference Wave 2", Kernel Results: a kernel fusing both stages spilled registers
// and ran slower, and an atomic-add combine was slower for the MX formats.  So: two GEMM
// kernels with fused epilogues, no float atomics.
//
//   combine: y[t,:] = bf16(sum_j fl32(gate[t,j] * d[t*k + j,:])), j ascending.
//            A kernel of its own, except at the smallest T (moe_down_kernel's FUSE variant,
//            at most two items per workgroup): there every workgroup's items are dealt
//            statically and each expert has one row group, so a workgroup can count, once
//            its own items are done, the items finished per column quad; the one that
//            completes a quad combines its columns.
//
// A persistent grid of workgroups sized to the device streams the items back to back
// (mx_stream.hpp): extra row groups and three first-group items per workgroup dealt
// statically, the rest claimed from a device counter in the workspace as workgroups become
// free, so that workgroups finish together however unevenly the items' row counts and the
// workgroups' memory speeds fall.  The
// number of active experts is read on the device, so there is no host readback.
#include "moe_policies.hpp"

namespace mx {

// A8: MXFP8 activations (x for gate_up, h for down) and the scaled MFMA
template <int NS, bool A8 = false>
using GateUpPlain = GateUpPolicy<NS, GlobalSort, GU_XCHUNK, false, A8>;
template <int NS, class SR, bool A8 = false, bool FUSE = false>
using DownPlain = DownPolicy<NS, GlobalSort, DN_XCHUNK, false, SR, A8, FUSE>;

// ------------------------------------------------------------------ kernels

// SPS: segments per weight step (GU_SPS, or GU_SPS_DEEP for half-width launches with fewer
// items than resident workgroup slots)
template <int NS, int SPS, bool A8>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_gate_up_kernel(const uint16_t* __restrict__ x,
                                                                    const uint8_t* __restrict__ wgu,
                                                                    const uint8_t* __restrict__ sgu, SortView sv,
                                                                    uint16_t* __restrict__ h, int H, int I, int k,
                                                                    int32_t* claim) {
  using P = GateUpPlain<NS, A8>;
  __shared__ __attribute__((aligned(16))) uint8_t xbufs[2 * P::XCHUNK];
  __shared__ __attribute__((aligned(16))) uint8_t slabs[WG_WAVES][SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sslabs[WG_WAVES][P::Scales::template slab_bytes<NS>()];
  __shared__ uint32_t xctr[2];
  __shared__ int32_t cq[4];
  if (threadIdx.x < 2) xctr[threadIdx.x] = 0u;
  __syncthreads();
  // wave index as a scalar, so every per-item quantity derived from it stays uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  P p;
  p.xrowsegs = XGeom<P::XCHUNK>::ROWSEGS;
  p.calign = SPS;
  p.m.sv = sv;
  p.nseg = H / SEG_K;
  p.nquad = I / (P::TILE * WG_WAVES);
  p.na = p.m.num_active();
  p.n_items = ((p.m.max_rows() + 15) >> 4) * p.na * p.nquad;  // row-group levels that exist
  ClaimedUnits seq{claim, (lds_i32*)cq, p.na * p.nquad, 0, false};
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
  stream_items<P, SPS>(p, seq, xbufs, xctr, slabs[wave], sslabs[wave], wave, lane);
  seq.finish();
}

// The combine of the column quads this workgroup completes (FUSE launches).  Its items are
// it = blockIdx.x + m * gridDim.x (no claims, one row group per expert), the down outputs
// were written with device-coherent stores, and each wave's stores have completed
// (vmcnt(0)) before the count.  A quad is complete when its count reaches na; the workgroup
// that completes it resets the counter (nothing else touches it in this launch) and sums
// the quad's columns for every token, j ascending, as moe_combine_kernel does.
template <int TILE>
__device__ __forceinline__ void combine_own_quads(int na, int nquad, int32_t* qctr, const float* __restrict__ gates,
                                                  const float* dpart, uint16_t* __restrict__ y, int T, int k, int H,
                                                  int32_t* done, uint32_t* ndone, int wave, int lane) {
  wait_own_stores();
  __syncthreads();
  const int n_first = na * nquad;
  if (wave == 0) {
    int nd = 0;
    for (int base = (int)blockIdx.x; base < n_first; base += 64 * (int)gridDim.x) {
      const int it = base + lane * (int)gridDim.x;
      bool fin = false;
      int q = 0;
      if (it < n_first) {
        q = it % nquad;
        fin = __hip_atomic_fetch_add(&qctr[q], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == na - 1;
        if (fin) __hip_atomic_store(&qctr[q], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const uint64_t m = __ballot(fin);
      if (fin) done[nd + __popcll(m & ((1ull << lane) - 1ull))] = q;
      nd += __popcll(m);
    }
    if (lane == 0) *ndone = (uint32_t)nd;
  }
  __syncthreads();
  constexpr int QV = TILE * WG_WAVES / 4;  // 4-column groups per quad
  const int nd = (int)*ndone;
  const int tid = wave * 64 + lane;
  for (int d = 0; d < nd; ++d) {
    const int c0 = done[d] * (QV * 4);
    for (int i = tid; i < T * QV; i += WG_WAVES * 64) {
      const int t = i / QV;
      const int n = c0 + (i - t * QV) * 4;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += 8) {  // 8 loads in flight, then the sum, j ascending
        u32x4 dv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) dv[jj] = ld16_coherent(dpart + (size_t)(t * k + min(j0 + jj, k - 1)) * H + n);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          if (j0 + jj < k) {
            const float g = gates[t * k + j0 + jj];
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
}

// SR, SPS: scale run and weight step (ScaleRun4, DN_SPS when I % 1024 == 0, else 1 and 1).
// FUSE: the launch also combines (small T; the launcher checks that no item is claimed).
template <int NS, class SR, int SPS, bool A8, bool FUSE>
__global__ void __launch_bounds__(WG_WAVES * 64) moe_down_kernel(const uint16_t* __restrict__ h,
                                                                 const uint8_t* __restrict__ wd,
                                                                 const uint8_t* __restrict__ sd, SortView sv,
                                                                 float* __restrict__ dpart, int H, int I,
                                                                 int32_t* ctl, const float* __restrict__ gates,
                                                                 uint16_t* __restrict__ y, int T, int k) {
  using P = DownPlain<NS, SR, A8, FUSE>;
  __shared__ __attribute__((aligned(16))) uint8_t xbufs[2 * P::XCHUNK];
  __shared__ __attribute__((aligned(16))) uint8_t slabs[WG_WAVES][SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sslabs[WG_WAVES][P::Scales::template slab_bytes<NS>()];
  __shared__ uint32_t xctr[2];
  __shared__ int32_t cq[4];
  if (threadIdx.x < 2) xctr[threadIdx.x] = 0u;
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  P p;
  p.xrowsegs = XGeom<P::XCHUNK>::ROWSEGS;
  p.m.sv = sv;
  p.nseg = I / SEG_K;
  p.nquad = H / (P::TILE * WG_WAVES);
  p.na = p.m.num_active();
  p.n_items = ((p.m.max_rows() + 15) >> 4) * p.na * p.nquad;  // row-group levels that exist
  ClaimedUnits seq{ctl + CTL_CLAIM_DN, (lds_i32*)cq, p.na * p.nquad, 0, false};
  p.xact = h;
  p.wd = wd;
  p.sd = sd;
  p.dpart = dpart;
  p.H = H;
  p.I = I;
  p.e_codes = (size_t)H * (I / 2);
  p.e_scales = (size_t)H * (I / 32);
  stream_items<P, SPS>(p, seq, xbufs, xctr, slabs[wave], sslabs[wave], wave, lane);
  if constexpr (FUSE)
    combine_own_quads<P::TILE>(p.na, p.nquad, ctl + CTL_QUAD0, gates, dpart, y, T, k, H,
                               reinterpret_cast<int32_t*>(xbufs), &xctr[0], wave, lane);
  seq.finish();
}

// One thread per (token, 4 consecutive outputs): fp32 sum of the gate-weighted slots, j ascending.
// The slots are loaded 8 at a time, all in flight together, and then summed in order, so a
// thread's loads do not wait for one another (one round trip per 8 slots, not per slot).
__global__ void __launch_bounds__(256) moe_combine_kernel(const float* __restrict__ dpart, const float* __restrict__ gates,
                                                          uint16_t* __restrict__ y, int T, int H, int k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_t = H / 4;
  if (i >= (int64_t)T * per_t) return;
  const int64_t t = i / per_t, n = (i - t * per_t) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 d[8];
    float g[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = min(j0 + jj, k - 1);  // past k: the last slot again, not summed
      d[jj] = *reinterpret_cast<const f32x4*>(dpart + (size_t)(t * k + j) * H + n);
      g[jj] = gates[t * k + j];
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (j0 + jj < k) acc += f32x4{g[jj] * d[jj][0], g[jj] * d[jj][1], g[jj] * d[jj][2], g[jj] * d[jj][3]};
  }
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
  *reinterpret_cast<u32x2*>(y + t * H + n) = u32x2{lo, hi};
}

// ------------------------------------------------------------------ launchers

template <class K>
static int resident_wgs_per_cu(K kernel, int block) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

// Persistent grid: all workgroups resident at once, and no more than there are items.
static int expert_grid(int64_t max_items, int wgs_per_cu) {
  const int64_t cap = (int64_t)device_cu_count() * wgs_per_cu;
  return (int)(max_items < cap ? max_items : cap);
}

static int64_t max_active(int T, int E, int k) { return (int64_t)T * k < E ? (int64_t)T * k : E; }
static int row_groups(int T) { return (T + 15) / 16; }

// Full-width tiles unless they would leave resident workgroup slots idle (few active
// experts and row groups, i.e. small T) and half-width tiles, twice the items, still fit in
// one round of the slots: then half-width tiles, twice the waves.  second_round: also
// half-width tiles when the full-width items need more than one round of the slots but
// less than two, where the second round would be run by a fraction of the workgroups while
// the others idle (down at T = 2 and 3: 1.15 and 1.7 rounds, 77.4 -> 76.6 and 105.1 ->
// 102.8 us per layer; from 2.2 rounds at T = 4 on, and at T = 1, half-width was slower).
// (The kernels are template arguments, so each pair caches its own occupancy: kernels of
// one signature share a type.)
template <auto K2, auto K1>
static bool use_half_tiles(int64_t items_full, int& grid, bool second_round = false) {
  static const int occ2 = resident_wgs_per_cu(K2, WG_WAVES * 64);
  static const int occ1 = resident_wgs_per_cu(K1, WG_WAVES * 64);
  const int64_t slots2 = (int64_t)device_cu_count() * occ2;
  const bool half = 2 * items_full <= (int64_t)device_cu_count() * occ1 ||
                    (second_round && items_full > slots2 && items_full < 2 * slots2);
  grid = half ? expert_grid(2 * items_full, occ1) : expert_grid(items_full, occ2);
  return half;
}

template <bool A8, int SPS>
static int launch_gate_up_sps(const uint16_t* x, const uint8_t* wgu, const uint8_t* sgu, const SortView& sv,
                              uint16_t* h, int32_t* ctl, int T, int H, int I, int E, int k, bool half, int grid,
                              hipStream_t stream) {
  if (half)
    hipLaunchKernelGGL((moe_gate_up_kernel<1, SPS, A8>), dim3(grid), dim3(WG_WAVES * 64), 0, stream, x, wgu, sgu, sv,
                       h, H, I, k, ctl + CTL_CLAIM_GU);
  else
    hipLaunchKernelGGL((moe_gate_up_kernel<2, SPS, A8>), dim3(grid), dim3(WG_WAVES * 64), 0, stream, x, wgu, sgu, sv,
                       h, H, I, k, ctl + CTL_CLAIM_GU);
  return hip_status(hipGetLastError());
}

template <bool A8>
static int launch_gate_up_run(const uint16_t* x, const uint8_t* wgu, const uint8_t* sgu, const SortView& sv,
                              uint16_t* h, int32_t* ctl, int T, int H, int I, int E, int k, hipStream_t stream) {
  const int gmax = row_groups(T);
  const int64_t items_full = (int64_t)gmax * max_active(T, E, k) * (I / (GateUpPlain<2>::TILE * WG_WAVES));
  int grid = 0;
  const bool half =
      use_half_tiles<moe_gate_up_kernel<2, GU_SPS, A8>, moe_gate_up_kernel<1, GU_SPS, A8>>(items_full, grid);
  static const int occ = resident_wgs_per_cu(moe_gate_up_kernel<2, GU_SPS, A8>, WG_WAVES * 64);
  const int64_t items = half ? 2 * items_full : items_full;
  if constexpr (!A8) {  // the MXFP8 kernel's registers leave no room for the deeper ring
    if (half && H % (SEG_K * GU_SPS_DEEP) == 0 && items < (int64_t)device_cu_count() * occ)
      return launch_gate_up_sps<A8, GU_SPS_DEEP>(x, wgu, sgu, sv, h, ctl, T, H, I, E, k, half, grid, stream);
  }
  return launch_gate_up_sps<A8, GU_SPS>(x, wgu, sgu, sv, h, ctl, T, H, I, E, k, half, grid, stream);
}

int launch_gate_up(const uint16_t* x, const uint8_t* wgu, const uint8_t* sgu, const SortView& sv, uint16_t* h,
                   int32_t* ctl, int T, int H, int I, int E, int k, bool act8, hipStream_t stream) {
  if (H % (SEG_K * GU_SPS) != 0 || H % (SEG_K * SRUN) != 0 || I % (SUB_ROWS * WG_WAVES) != 0) return MX_ERR_SHAPE;
  if (act8) return launch_gate_up_run<true>(x, wgu, sgu, sv, h, ctl, T, H, I, E, k, stream);
  return launch_gate_up_run<false>(x, wgu, sgu, sv, h, ctl, T, H, I, E, k, stream);
}

// The combine goes into the down launch when every expert has one row group (T <= 16) and
// no workgroup can get more than two items (min(T k, E) experts times the column quads):
// then nothing is claimed, and the last workgroups' combine replaces a launch that costs
// more.  With more items per workgroup the combine at the end of the last ones costs more
// than the launch it saves (measured: slower at T = 8, and at T = 4 for I = 256).
constexpr int FUSE_MAX_ITEMS = 2;
static_assert(FUSE_MAX_ITEMS <= DYNAMIC_MIN, "a fused launch claims nothing");
static bool fuse_combine(int T, int E, int k, int nquad, int grid) {
  return T <= 16 && nquad <= CTL_MAX_QUADS && max_active(T, E, k) * nquad <= (int64_t)FUSE_MAX_ITEMS * grid;
}

template <int NS, class SR, int SPS, bool A8>
static void launch_down_tiles(bool fuse, int grid, const uint16_t* h, const uint8_t* wd, const uint8_t* sd,
                              const SortView& sv, float* dpart, int32_t* ctl, const float* gates, uint16_t* y, int T,
                              int H, int I, int k, hipStream_t stream) {
  if (fuse)
    hipLaunchKernelGGL((moe_down_kernel<NS, SR, SPS, A8, true>), dim3(grid), dim3(WG_WAVES * 64), 0, stream, h, wd, sd,
                       sv, dpart, H, I, ctl, gates, y, T, k);
  else
    hipLaunchKernelGGL((moe_down_kernel<NS, SR, SPS, A8, false>), dim3(grid), dim3(WG_WAVES * 64), 0, stream, h, wd,
                       sd, sv, dpart, H, I, ctl, gates, y, T, k);
}

// Wide tiles (4 subtiles, 64 output columns per wave) for reductions of one 256-value
// segment per scale run (I not a multiple of 1024, e.g. one tensor-parallel eighth of an
// expert): such an item is a single step, so its fixed costs (item metadata, the activation
// hand-off, the epilogue) outweigh its weight bytes, and the wider tile halves the items.
// The launch runs 2 workgroups per CU instead of 3, and half the items balance less
// evenly, so wide tiles pay only when the workgroups get at least WIDE_MIN_ITEMS items
// (host bound: min(T k, E) active experts).  Measured on the TP8 share: down 43.1 ->
// 37.9 us at T = 32, but 19.3 -> 20.7 us at T = 4 (under 2 items per workgroup).
constexpr int WIDE_MIN_ITEMS = 4;

template <class SR, int SPS, bool A8>
static int launch_down_run(const uint16_t* h, const float* gates, const uint8_t* wd, const uint8_t* sd,
                           const SortView& sv, float* dpart, uint16_t* y, bool& combined, int32_t* ctl, int T, int H,
                           int I, int E, int k, hipStream_t stream) {
  const int gmax = row_groups(T);
  const int64_t items_full = (int64_t)gmax * max_active(T, E, k) * (H / (DownPlain<2, SR>::TILE * WG_WAVES));
  int grid = 0;
  if constexpr (SR::SRUN == 1 && !A8) {
    if (H % (DownPlain<4, SR>::TILE * WG_WAVES) == 0) {
      static const int occ4 = resident_wgs_per_cu(moe_down_kernel<4, SR, SPS, A8, false>, WG_WAVES * 64);
      if (items_full / 2 >= (int64_t)WIDE_MIN_ITEMS * device_cu_count() * occ4) {
        grid = expert_grid(items_full / 2, occ4);
        const int nquad = H / (DownPlain<4, SR>::TILE * WG_WAVES);
        combined = fuse_combine(T, E, k, nquad, grid);
        launch_down_tiles<4, SR, SPS, A8>(combined, grid, h, wd, sd, sv, dpart, ctl, gates, y, T, H, I, k, stream);
        return hip_status(hipGetLastError());
      }
    }
  }
  if (use_half_tiles<moe_down_kernel<2, SR, SPS, A8, false>, moe_down_kernel<1, SR, SPS, A8, false>>(items_full,
                                                                                                    grid, true)) {
    const int nquad = H / (DownPlain<1, SR>::TILE * WG_WAVES);
    combined = fuse_combine(T, E, k, nquad, grid);
    launch_down_tiles<1, SR, SPS, A8>(combined, grid, h, wd, sd, sv, dpart, ctl, gates, y, T, H, I, k, stream);
  } else {
    const int nquad = H / (DownPlain<2, SR>::TILE * WG_WAVES);
    combined = fuse_combine(T, E, k, nquad, grid);
    launch_down_tiles<2, SR, SPS, A8>(combined, grid, h, wd, sd, sv, dpart, ctl, gates, y, T, H, I, k, stream);
  }
  return hip_status(hipGetLastError());
}

template <bool A8>
static int launch_down_mode(const uint16_t* h, const float* gates, const uint8_t* wd, const uint8_t* sd,
                            const SortView& sv, float* dpart, uint16_t* y, bool& combined, int32_t* ctl, int T, int H,
                            int I, int E, int k, hipStream_t stream) {
  // down's reduction length is I: 4-segment scale runs and 2-segment steps when I % 1024 == 0,
  // one-segment runs and steps for any other multiple of 256
  if (I % (SEG_K * SRUN) == 0 && I % (SEG_K * DN_SPS) == 0)
    return launch_down_run<ScaleRun4, DN_SPS, A8>(h, gates, wd, sd, sv, dpart, y, combined, ctl, T, H, I, E, k,
                                                  stream);
  if (I % SEG_K == 0)
    return launch_down_run<ScaleRun<1>, 1, A8>(h, gates, wd, sd, sv, dpart, y, combined, ctl, T, H, I, E, k, stream);
  return MX_ERR_SHAPE;
}

int launch_down(const uint16_t* h, const float* gates, const uint8_t* wd, const uint8_t* sd, const SortView& sv,
                float* dpart, uint16_t* y, bool* combined, int32_t* ctl, int T, int H, int I, int E, int k, bool act8,
                hipStream_t stream) {
  *combined = false;
  if (H % (2 * SUB_ROWS * WG_WAVES) != 0) return MX_ERR_SHAPE;
  if (act8) return launch_down_mode<true>(h, gates, wd, sd, sv, dpart, y, *combined, ctl, T, H, I, E, k, stream);
  return launch_down_mode<false>(h, gates, wd, sd, sv, dpart, y, *combined, ctl, T, H, I, E, k, stream);
}

int launch_combine(const float* dpart, const float* gates, uint16_t* y, int T, int H, int k, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H / 4);
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dpart, gates, y, T,
                     H, k);
  return hip_status(hipGetLastError());
}

}  // namespace mx
