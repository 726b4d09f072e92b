// HBM reference kernels: a streaming read and a copy over one buffer, the yardsticks the
// expert-weight stream is measured against.  "Zyphra Inference Wave 2" (footnote 6 to its
// roofline discussion) measures MI355X's HBM with a plain copy kernel and reaches 6.07 of
// the nominal 8 TB/s; these kernels give the same figure on the box a benchmark runs on.
//
// Both walk the buffer grid-stride in 16-byte pieces with nontemporal accesses, as the
// expert GEMMs read their weights, each thread keeping several pieces in flight.  The read
// kernel folds what it loads into an XOR (kept in registers, reduced across the wave and
// XORed into four device words with vector atomics), so its loads are live and its result
// can be checked bit for bit.
#include "mx_device.hpp"
#include "mx_internal.hpp"

namespace mx {

constexpr int HBM_BLOCK = 256;
// Shapes measured on MI355X (4 GiB, medians of 15): the read reaches 6.9 TB/s with one
// contiguous chunk per workgroup, 8 pieces in flight per thread and 4 workgroups per CU
// (grid-stride reads peaked at 6.0); the copy reaches 4.8 TB/s grid-stride with 8 in
// flight and 8 workgroups per CU, about what hipMemcpy gives (4.9).
constexpr int HBM_READ_UNROLL = 8;
constexpr int HBM_READ_WGS_PER_CU = 4;
constexpr int HBM_COPY_UNROLL = 8;
constexpr int HBM_COPY_WGS_PER_CU = 8;

// Workgroup b reads pieces [b * per, min((b + 1) * per, n16)); per is a multiple of 256
// pieces (4 KB), so chunks start on cache lines.
__global__ void __launch_bounds__(HBM_BLOCK) hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16, int64_t per,
                                                             uint32_t* __restrict__ xor_out) {
  const int64_t b = (int64_t)blockIdx.x * per;
  const int64_t e = b + per < n16 ? b + per : n16;
  int64_t i = b + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (HBM_READ_UNROLL - 1) * HBM_BLOCK < e; i += HBM_READ_UNROLL * HBM_BLOCK) {
    u32x4 v[HBM_READ_UNROLL];
#pragma unroll
    for (int u = 0; u < HBM_READ_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * HBM_BLOCK);
#pragma unroll
    for (int u = 0; u < HBM_READ_UNROLL; ++u) acc ^= v[u];
  }
  for (; i < e; i += HBM_BLOCK) acc ^= __builtin_nontemporal_load(src + i);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t a = acc[c];
    for (int off = 32; off > 0; off >>= 1) a ^= (uint32_t)__shfl_xor((int)a, off, 64);
    acc[c] = a;
  }
  // XOR with zero changes nothing, so a wave whose fold is zero skips its atomic: a buffer
  // of repeated words (the benchmark's) then adds no atomics to the timed read.
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (acc[c] != 0u) atomicXor(xor_out + c, acc[c]);
  }
}

__global__ void __launch_bounds__(HBM_BLOCK) hbm_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                             int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * HBM_BLOCK;
  int64_t i = (int64_t)blockIdx.x * HBM_BLOCK + threadIdx.x;
  for (; i + (HBM_COPY_UNROLL - 1) * stride < n16; i += HBM_COPY_UNROLL * stride) {
    u32x4 v[HBM_COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < HBM_COPY_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < HBM_COPY_UNROLL; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

static int hbm_grid(int64_t n16, int wgs_per_cu, int64_t pieces_per_wg) {
  const int64_t want = (int64_t)device_cu_count() * wgs_per_cu;
  const int64_t need = (n16 + pieces_per_wg - 1) / pieces_per_wg;
  return (int)(need < want ? need : want);
}

}  // namespace mx

using namespace mx;

extern "C" {

int mx_hbm_read(const void* src, size_t bytes, uint32_t* xor_out, void* stream) {
  if (!src || !xor_out) return MX_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 46)) return MX_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(xor_out, 4)) return MX_ERR_ALIGN;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int grid = hbm_grid(n16, HBM_READ_WGS_PER_CU, (int64_t)HBM_BLOCK * HBM_READ_UNROLL);
  const int64_t per = ((n16 + grid - 1) / grid + HBM_BLOCK - 1) / HBM_BLOCK * HBM_BLOCK;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(HBM_BLOCK), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), n16, per, xor_out);
  return hip_status(hipGetLastError());
}

int mx_hbm_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return MX_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 46)) return MX_ERR_SHAPE;
  if (!aligned(dst, 16) || !aligned(src, 16)) return MX_ERR_ALIGN;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int grid = hbm_grid(n16, HBM_COPY_WGS_PER_CU, (int64_t)HBM_BLOCK * HBM_COPY_UNROLL);
  hipLaunchKernelGGL(hbm_copy_kernel, dim3(grid), dim3(HBM_BLOCK), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n16);
  return hip_status(hipGetLastError());
}

}  // extern "C"
