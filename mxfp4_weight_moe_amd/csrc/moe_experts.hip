// The two expert GEMMs of the MXFP4 MoE layer and the combine.
//
// "Zyphra Inference Wave 2", section "Quantization": an MXFP4 expert runs two expert
// GEMMs and combines the results, and a decode step reads only the routed experts; Kernel
// Results: a kernel fusing both stages spilled registers and ran slower, and an atomic-add
// combine was slower for the MX formats.  So: two GEMM kernels with fused epilogues, no
// float atomics.
//
//   gate_up: work item = (active expert, 16 intermediate columns).  One wavefront streams
//            the 16 gate rows and the matching 16 up rows of that expert over all H, for
//            every token row routed to the expert, then applies SwiGLU and rounds h to
//            bf16.  h rows are stored in sorted-slot order, contiguous per expert.
//   down:    work item = (active expert, 32 output columns); multiplies the expert's h rows
//            by W_down and stores gate-weighted fp32 partial outputs per flat slot.
//   combine: y[t,:] = bf16(sum_j partial[t*k + j,:]) with j ascending.
//
// Both GEMM kernels are persistent: a grid sized to the device loops over the work list,
// whose length (number of active experts) is read on the device, so no host readback.
#include "mx_device.hpp"
#include "mx_internal.hpp"

namespace mx {

struct ExpertList {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted_slots;
  const int32_t* active;
  const int32_t* num_active;
};

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ------------------------------------------------------------------ gate_up + SwiGLU

template <int W, int MT>
__device__ __forceinline__ void gate_up_pass(const uint16_t* __restrict__ x, const uint8_t* __restrict__ wexp,
                                             const uint8_t* __restrict__ sexp, const ExpertList& el,
                                             uint16_t* __restrict__ h, int H, int I, int k, int p, int row0, int R,
                                             int mp, uint8_t* slab, f32x4* red, int wave, int lane) {
  constexpr int NS = 2;
  constexpr int D = (MT == 1) ? 3 : 2;
  StreamLanes<NS, MT> L;
  lanes_init_lds(L, lane);
  const size_t kb = (size_t)H >> 1, ks = (size_t)H >> 5;
  const int n0 = p * SUB_ROWS;
  for (int q = 0; q < 2; ++q) {
    const int r = n0 + (lane >> 3) + 8 * q;
    L.w[0][q] = wexp + (size_t)r * kb + (lane & 7) * 16;        // gate rows
    L.w[1][q] = wexp + (size_t)(I + r) * kb + (lane & 7) * 16;  // up rows
  }
  L.s[0] = sexp + (size_t)(n0 + (lane & 15)) * ks;
  L.s[1] = sexp + (size_t)(I + n0 + (lane & 15)) * ks;
  for (int mt = 0; mt < MT; ++mt) {
    const int rr = mp + mt * 16 + (lane & 15);
    if (rr < R) {
      const int t = el.sorted_slots[row0 + rr] / k;
      L.x[mt] = x + (size_t)t * H + 32 * (lane >> 4);
    } else {
      L.x[mt] = nullptr;
    }
  }
  const int nseg = H / SEG_K;
  const int sg0 = nseg * wave / W, sg1 = nseg * (wave + 1) / W;
  f32x4 acc[MT][NS];
  acc_zero(acc);
  stream_segments<NS, MT, D>(L, sg0, sg1, 0, slab, acc, lane);
  wg_reduce<NS, MT, W>(acc, red, wave, lane);
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int rr = mp + mt * 16 + (lane & 15);
      if (rr >= R) continue;
      uint32_t o[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint16_t a = f32_to_bf16_rne(silu_mul(acc[mt][0][2 * j], acc[mt][1][2 * j]));
        const uint16_t b = f32_to_bf16_rne(silu_mul(acc[mt][0][2 * j + 1], acc[mt][1][2 * j + 1]));
        o[j] = (uint32_t)a | ((uint32_t)b << 16);
      }
      *reinterpret_cast<u32x2*>(h + (size_t)(row0 + rr) * I + n0 + 4 * (lane >> 4)) = u32x2{o[0], o[1]};
    }
  }
}

template <int W>
__global__ void __launch_bounds__(W * 64) moe_gate_up_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ wgu,
                                                             const uint8_t* __restrict__ sgu, ExpertList el,
                                                             uint16_t* __restrict__ h, int H, int I, int k) {
  __shared__ __attribute__((aligned(16))) uint8_t slabs[W][2 * SLAB_BYTES];
  __shared__ f32x4 red[(W > 1) ? W * 2 * 2 * 64 : 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int npair = I / SUB_ROWS;
  const int items = *el.num_active * npair;
  const size_t e_codes = (size_t)2 * I * (H / 2), e_scales = (size_t)2 * I * (H / 32);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int a = it / npair, p = it - a * npair;
    const int e = el.active[a];
    const int row0 = el.offsets[e], R = el.counts[e];
    const uint8_t* wexp = wgu + (size_t)e * e_codes;
    const uint8_t* sexp = sgu + (size_t)e * e_scales;
    for (int mp = 0; mp < R; mp += 32) {
      if (R - mp > 16)
        gate_up_pass<W, 2>(x, wexp, sexp, el, h, H, I, k, p, row0, R, mp, slabs[wave], red, wave, lane);
      else
        gate_up_pass<W, 1>(x, wexp, sexp, el, h, H, I, k, p, row0, R, mp, slabs[wave], red, wave, lane);
    }
  }
}

// ------------------------------------------------------------------ down + gate weighting

template <int W, int MT>
__device__ __forceinline__ void down_pass(const uint16_t* __restrict__ h, const uint8_t* __restrict__ wexp,
                                          const uint8_t* __restrict__ sexp, const ExpertList& el,
                                          const float* __restrict__ gates, float* __restrict__ dpart, int H, int I,
                                          int q32, int row0, int R, int mp, uint8_t* slab, f32x4* red, int wave,
                                          int lane) {
  constexpr int NS = 2;
  constexpr int D = (MT == 1) ? 3 : 2;
  StreamLanes<NS, MT> L;
  lanes_init_lds(L, lane);
  const size_t kb = (size_t)I >> 1, ks = (size_t)I >> 5;
  const int n0 = q32 * 32;
  for (int i = 0; i < NS; ++i) {
    for (int q = 0; q < 2; ++q) L.w[i][q] = wexp + (size_t)(n0 + 16 * i + (lane >> 3) + 8 * q) * kb + (lane & 7) * 16;
    L.s[i] = sexp + (size_t)(n0 + 16 * i + (lane & 15)) * ks;
  }
  for (int mt = 0; mt < MT; ++mt) {
    const int rr = mp + mt * 16 + (lane & 15);
    L.x[mt] = (rr < R) ? h + (size_t)(row0 + rr) * I + 32 * (lane >> 4) : nullptr;
  }
  const int nseg = I / SEG_K;
  const int sg0 = nseg * wave / W, sg1 = nseg * (wave + 1) / W;
  f32x4 acc[MT][NS];
  acc_zero(acc);
  stream_segments<NS, MT, D>(L, sg0, sg1, 0, slab, acc, lane);
  wg_reduce<NS, MT, W>(acc, red, wave, lane);
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int rr = mp + mt * 16 + (lane & 15);
      if (rr >= R) continue;
      const int f = el.sorted_slots[row0 + rr];
      const float g = gates[f];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        f32x4 v = acc[mt][i];
        v = f32x4{g * v[0], g * v[1], g * v[2], g * v[3]};
        *reinterpret_cast<f32x4*>(dpart + (size_t)f * H + n0 + 16 * i + 4 * (lane >> 4)) = v;
      }
    }
  }
}

template <int W>
__global__ void __launch_bounds__(W * 64) moe_down_kernel(const uint16_t* __restrict__ h, const uint8_t* __restrict__ wd,
                                                          const uint8_t* __restrict__ sd, ExpertList el,
                                                          const float* __restrict__ gates, float* __restrict__ dpart,
                                                          int H, int I) {
  __shared__ __attribute__((aligned(16))) uint8_t slabs[W][2 * SLAB_BYTES];
  __shared__ f32x4 red[(W > 1) ? W * 2 * 2 * 64 : 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ntile = H / 32;
  const int items = *el.num_active * ntile;
  const size_t e_codes = (size_t)H * (I / 2), e_scales = (size_t)H * (I / 32);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int a = it / ntile, q32 = it - a * ntile;
    const int e = el.active[a];
    const int row0 = el.offsets[e], R = el.counts[e];
    const uint8_t* wexp = wd + (size_t)e * e_codes;
    const uint8_t* sexp = sd + (size_t)e * e_scales;
    for (int mp = 0; mp < R; mp += 32) {
      if (R - mp > 16)
        down_pass<W, 2>(h, wexp, sexp, el, gates, dpart, H, I, q32, row0, R, mp, slabs[wave], red, wave, lane);
      else
        down_pass<W, 1>(h, wexp, sexp, el, gates, dpart, H, I, q32, row0, R, mp, slabs[wave], red, wave, lane);
    }
  }
}

// ------------------------------------------------------------------ combine

// One thread per (token, 4 consecutive outputs): fp32 sum over the k slots, j ascending.
__global__ void __launch_bounds__(256) moe_combine_kernel(const float* __restrict__ dpart, uint16_t* __restrict__ y, int T,
                                                          int H, int k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_t = H / 4;
  if (i >= (int64_t)T * per_t) return;
  const int64_t t = i / per_t, n = (i - t * per_t) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) acc += *reinterpret_cast<const f32x4*>(dpart + (size_t)(t * k + j) * H + n);
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
  *reinterpret_cast<u32x2*>(y + t * H + n) = u32x2{lo, hi};
}

// ------------------------------------------------------------------ launchers

static ExpertList expert_list(const MoeWorkspace& ws) {
  return ExpertList{ws.counts, ws.offsets, ws.sorted_slots, ws.active, ws.num_active};
}

// Persistent grid: enough workgroups to cover every possible item when few experts can be
// active, otherwise a fixed number of workgroups per compute unit.
static int persistent_grid(int64_t max_items, int wgs_per_cu) {
  const int64_t cap = (int64_t)device_cu_count() * wgs_per_cu;
  return (int)(max_items < cap ? max_items : cap);
}

int launch_gate_up(const uint16_t* x, const uint8_t* wgu, const uint8_t* sgu, const MoeWorkspace& ws, int T, int H,
                   int I, int E, int k, hipStream_t stream) {
  const int64_t max_active = (int64_t)T * k < E ? (int64_t)T * k : E;
  const int grid = persistent_grid(max_active * (I / SUB_ROWS), 8);
  hipLaunchKernelGGL((moe_gate_up_kernel<1>), dim3(grid), dim3(64), 0, stream, x, wgu, sgu, expert_list(ws), ws.h, H, I,
                     k);
  return hip_status(hipGetLastError());
}

int launch_down(const uint8_t* wd, const uint8_t* sd, const MoeWorkspace& ws, int T, int H, int I, int E, int k,
                hipStream_t stream) {
  const int64_t max_active = (int64_t)T * k < E ? (int64_t)T * k : E;
  const int grid = persistent_grid(max_active * (H / 32), 8);
  hipLaunchKernelGGL((moe_down_kernel<1>), dim3(grid), dim3(64), 0, stream, ws.h, wd, sd, expert_list(ws), ws.gates,
                     ws.dpart, H, I);
  return hip_status(hipGetLastError());
}

int launch_combine(const MoeWorkspace& ws, uint16_t* y, int T, int H, int k, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H / 4);
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, ws.dpart, y, T, H, k);
  return hip_status(hipGetLastError());
}

}  // namespace mx
