// Router top-k with a softmax over the selected logits, and the token->expert counting sort.
//
// Routing: the pages benchmark top-8 routing over 256 and 384 experts ("Zyphra Inference
// Wave 2", Figure 10) and profile "top-k expert routing" as its own phase (AMD megakernel
// blog, section "4. Data Locality").  The gate definition (softmax over the k selected
// logits) and the tie rule (lower expert id first) are this library's reading.
//
// Sort: each expert receives a few token rows ("Zyphra Inference Wave 2", Kernel Results);
// grouping the routed slots by expert lets each expert's weights be read once for all of
// its rows.  The order is fixed (experts ascending, slot ascending), so the result is
// bit-exact and independent of thread timing.
#include "mx_device.hpp"
#include "mx_internal.hpp"

namespace mx {

constexpr int ROUTE_MAX_PER_LANE = MX_MAX_EXPERTS / 64;  // logits held per lane

// (value, id) ordering of the router: larger value first, then lower id.
__device__ __forceinline__ bool route_better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

// One wavefront per token.
__global__ void __launch_bounds__(256) moe_route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  const int per = (E + 63) >> 6;
  float v[ROUTE_MAX_PER_LANE];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
    const int e = lane + 64 * i;
    if (i < per && e < E) {
      v[i] = l[e];
    } else {
      v[i] = 0.f;
      taken |= 1u << i;
    }
  }
  float my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_huge_valf();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
      if (i < per && !((taken >> i) & 1u)) {
        const int e = lane + 64 * i;
        if (route_better(v[i], e, bv, be)) {
          bv = v[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (route_better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float m = __shfl(my_v, 0);
  const float ex = (lane < k) ? expf(my_v - m) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    gates[(size_t)t * k + lane] = ex / sum;
  }
}

int launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* gates, hipStream_t stream) {
  hipLaunchKernelGGL(moe_route_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, ids, gates);
  return hip_status(hipGetLastError());
}

// ------------------------------------------------------------------ sort

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WORDS = MX_MAX_EXPERTS * (MX_MAX_TOKENS / 32);  // one bit per (expert, token)

// Single workgroup.  A slot (t, j) routed to expert e sets bit t of expert e's token mask;
// because a token's k experts are distinct, the rank of the slot among expert e's slots is
// the number of set bits below t, which fixes a stable order without any ordering of
// atomics.  Counts and the active list come from one packed block-wide scan.
__global__ void __launch_bounds__(SORT_THREADS) moe_sort_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                                int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_slots,
                                                                int32_t* __restrict__ active,
                                                                int32_t* __restrict__ num_active) {
  __shared__ uint32_t bits[SORT_WORDS];
  __shared__ int32_t s_off[MX_MAX_EXPERTS];
  __shared__ int32_t s_wave[SORT_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = (T + 31) >> 5;
  const int F = T * k;
  for (int i = tid; i < E * words; i += SORT_THREADS) bits[i] = 0u;
  __syncthreads();
  for (int f = tid; f < F; f += SORT_THREADS) {
    const int e = ids[f];
    const int t = f / k;
    if (e >= 0 && e < E) atomicOr(&bits[e * words + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  // per-expert count and active flag, packed as count | flag << 16 (count <= T < 2^16)
  const int e = tid;
  int cnt = 0;
  if (e < E)
    for (int w = 0; w < words; ++w) cnt += __popc(bits[e * words + w]);
  const int packed = cnt | ((cnt > 0) ? (1 << 16) : 0);
  // block-wide exclusive scan of `packed` over e = 0..E-1 (E <= 1024 = blockDim)
  int incl = packed;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int wv = (lane < SORT_THREADS / 64) ? s_wave[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(wv, off);
      if (lane >= off) wv += o;
    }
    if (lane < SORT_THREADS / 64) s_wave[lane] = wv;  // inclusive over waves
  }
  __syncthreads();
  const int excl = incl - packed + (wave > 0 ? s_wave[wave - 1] : 0);
  const int off_e = excl & 0xFFFF;
  const int act_pos = excl >> 16;
  if (e < E) {
    s_off[e] = off_e;
    counts[e] = cnt;
    offsets[e] = off_e;
    if (cnt > 0) active[act_pos] = e;
  }
  const int total = s_wave[SORT_THREADS / 64 - 1];
  const int n_act = total >> 16;
  if (e < E && e >= n_act) active[e] = -1;
  if (tid == 0) {
    offsets[E] = total & 0xFFFF;
    *num_active = n_act;
  }
  __syncthreads();
  for (int f = tid; f < F; f += SORT_THREADS) {
    const int ee = ids[f];
    if (ee < 0 || ee >= E) continue;
    const int t = f / k;
    const uint32_t* b = bits + ee * words;
    int rank = __popc(b[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(b[w]);
    sorted_slots[s_off[ee] + rank] = f;
  }
}

int launch_sort(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                int32_t* active, int32_t* num_active, hipStream_t stream) {
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(SORT_THREADS), 0, stream, ids, T, k, E, counts, offsets,
                     sorted_slots, active, num_active);
  return hip_status(hipGetLastError());
}

}  // namespace mx
