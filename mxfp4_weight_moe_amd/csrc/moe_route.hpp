// Device helpers of the router: top-k of one token by one wavefront, with a softmax over the
// selected logits.
//
// The pages benchmark top-8 routing over 256 and 384 experts ("Zyphra Inference Wave 2",
// Figure 10) and profile "top-k expert routing" as its own phase (AMD megakernel blog,
// section "4. Data Locality").  The gate definition (softmax over the k selected logits)
// and the tie rule (lower expert id first) are this library's reading.
#pragma once
#include "mx_device.hpp"
#include "mx_internal.hpp"

namespace mx {

// Order-preserving unsigned key of a float (larger float, larger key); -0 is first
// normalised to +0 so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t route_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float route_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// a = max(a, a of the lane that DPP control CTRL selects); lanes of rows outside ROW_MASK
// receive 0 and keep a.  (Valid keys are never 0: route_key maps every finite value, -0 and
// +0 included, above it; 0 marks an empty or already taken entry.)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void max32_dpp(uint32_t& a) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, ROW_MASK, 0xF, false);
  a = o > a ? o : a;
}

// Sum over each row of 16 lanes (every lane of the row gets it).
template <int CTRL>
__device__ __forceinline__ float row_add_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_BCAST15 = 0x142;  // lane 15 of each row to the next row
constexpr int DPP_ROW_BCAST31 = 0x143;  // lane 31 to rows 2 and 3

// Maximum over the wavefront, returned uniform: within each row of 16 lanes by four
// exchanges, then rows 0+1 into row 1 and 2+3 into row 3, then row 1 into row 3.
__device__ __forceinline__ uint32_t wave_max32(uint32_t a) {
  max32_dpp<DPP_QUAD_XOR1, 0xF>(a);
  max32_dpp<DPP_QUAD_XOR2, 0xF>(a);
  max32_dpp<DPP_ROW_HALF_MIRROR, 0xF>(a);
  max32_dpp<DPP_ROW_MIRROR, 0xF>(a);
  max32_dpp<DPP_ROW_BCAST15, 0xA>(a);
  max32_dpp<DPP_ROW_BCAST31, 0xC>(a);
  return (uint32_t)__builtin_amdgcn_readlane((int)a, 63);
}

// One token's logits, lane l holding logits l, l + 64, ... (PER per lane, E <= 64 PER).
// The loads are unconditional (indices past E re-read logit E-1, never used) so that they
// are all in flight at once: the logits are not cache-resident after the weight stream.
template <int PER>
__device__ __forceinline__ void route_load(const float* __restrict__ l, int E, int lane, float (&v)[PER]) {
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = l[min(lane + 64 * i, E - 1)];
}

// Top-k of one token by one wavefront, from its loaded logits.  Each of the k rounds takes
// the wave's largest untaken value key (one 32-bit maximum per lane, then over the
// wavefront with DPP exchanges); its winner is the lowest expert id holding that key, which
// is the lowest lane of the first slot i whose ballot of key == maximum is not empty (ids
// lane + 64 i: a lower slot always has the lower id), and its key becomes 0 (taken).  So a
// larger value wins and equal values go to the lower expert id.  Lane j < k returns the
// j-th winner (slots in descending logit order) and its softmax gate over the k winners.
template <int PER>
__device__ __forceinline__ void route_select(const float (&v)[PER], int E, int k, int lane, int& my_e,
                                             float& my_gate) {
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = (lane + 64 * i < E) ? route_key(v[i]) : 0u;
  uint32_t my_key = 0u;
  my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t b = key[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) b = key[i] > b ? key[i] : b;
    const uint32_t w = wave_max32(b);
    int wi = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint64_t m = __ballot(key[i] == w);
      if (m) {
        wi = 64 * i + (int)__builtin_ctzll(m);
        break;
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = (wi == lane + 64 * i) ? 0u : key[i];
    if (lane == j) {
      my_key = w;
      my_e = wi;
    }
  }
  // softmax over the k winners, relative to the largest (slot 0)
  const float m = route_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
  const float ex = (lane < k) ? expf(route_value(my_key) - m) : 0.f;
  float s = row_add_step<DPP_QUAD_XOR1>(ex);
  s = row_add_step<DPP_QUAD_XOR2>(s);
  s = row_add_step<DPP_ROW_HALF_MIRROR>(s);
  s = row_add_step<DPP_ROW_MIRROR>(s);
  const float sum = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 0)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 16))) +
                    (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 32)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 48)));
  my_gate = ex / sum;
}

// Logits per lane for E experts: 4, 8 or 16 (E <= MX_MAX_EXPERTS = 1024).
static_assert(MX_MAX_EXPERTS <= 64 * 16, "at most 16 logits per lane");
inline int route_per(int E) { return E <= 256 ? 4 : (E <= 512 ? 8 : 16); }

}  // namespace mx
