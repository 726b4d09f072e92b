// Work lists and epilogues of the two expert GEMMs, as policies for stream_items().
//
// "Zyphra Inference Wave 2", section "Quantization": an MXFP4 expert runs two expert
// GEMMs and combines the results, and a decode step reads only the routed experts.
//
//   gate_up: item = (row group of an active expert, 4 tiles of intermediate columns).
//            Each of the 4 wavefronts of a workgroup streams the gate rows and the matching
//            up rows of its tile (16 + 16, or 8 + 8 for half-width tiles) over all H, then
//            applies SwiGLU and rounds h to bf16.  h rows are stored in sorted-slot order.
//   down:    item = (row group of an active expert, 4 tiles of 32 output columns, or 16
//            for half-width tiles); stores the fp32 down outputs per flat slot.
//
// A row group is up to 16 of the expert's routed rows (one MFMA m-tile); experts with more
// rows have several groups.  Items are numbered group-major, then expert, then column
// tile quad: it = (g * na + a) * nquad + quad, so the first na * nquad items are the first
// row groups of every active expert (all valid) and the rest are the extra groups of
// experts with more than 16 rows (valid only where the expert has that many rows).
//
// Two parameters adapt the policies to where they run:
//   Meta  where the sort outputs come from: GlobalSort (written by an earlier launch, read
//         through the scalar data path) or a per-workgroup copy in LDS (the single-launch
//         layer, which sorts in every workgroup).
//   COH   whether h and the down outputs are handed to other workgroups of the same launch.
//         Then they are written and read with device-coherent accesses (the sc1 bit: the
//         store is visible device-wide once it completes, the load misses any cache that
//         is not coherent device-wide), so no cache-wide write-back or invalidate is needed.
#pragma once
#include "mx_internal.hpp"
#include "mx_stream.hpp"

namespace mx {

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Item metadata written by an earlier launch is read through the scalar data path: the
// kernels never write it, and scalar loads do not queue behind the wave's in-flight vector
// loads, so setting up the next item does not drain the weight stream.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;

__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) { return ((cint_ptr)p)[i]; }

// Sort outputs in global memory (an earlier launch wrote them).
struct GlobalSort {
  SortView sv;
  __device__ __forceinline__ int num_active() const { return ld_uniform(sv.num_active, 0); }
  __device__ __forceinline__ int max_rows() const { return ld_uniform(sv.num_active, 1); }
  __device__ __forceinline__ int expert(int a) const { return ld_uniform(sv.active, a); }
  __device__ __forceinline__ int count(int a) const { return ld_uniform(sv.counts, expert(a)); }
  __device__ __forceinline__ int offset(int a) const { return ld_uniform(sv.offsets, expert(a)); }
  __device__ __forceinline__ int slot(int i) const { return ld_uniform(sv.sorted_slots, i); }
  // the rows of active expert a for a per-lane a (vector loads)
  __device__ __forceinline__ int count_lane(int a) const { return sv.counts[sv.active[a]]; }
};

// Bounded wait for a device-wide counter to reach `target`.  One wavefront of the
// workgroup polls (polls of every wavefront on one address queue behind each other and
// behind the counter's own updates) and raises the LDS flag; the others wait on the flag.
// A wait that outlasts SPIN_LIMIT polls (far longer than any layer) raises *err and
// returns, so a kernel never waits forever.
constexpr uint32_t SPIN_LIMIT = 1u << 18;

__device__ __forceinline__ void wait_counter(int32_t* ctr, int target, int32_t* err, lds_i32* flag, int wave) {
  if (wave == 0) {
    for (uint32_t n = 0;; ++n) {
      const int v =
          __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (v >= target) break;
      if (n == SPIN_LIMIT) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    __hip_atomic_store((int32_t*)flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    while (__hip_atomic_load((int32_t*)flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(2);
  }
  __asm__ volatile("" ::: "memory");
}

// Flat slot of row `j` (< 16) of a group of `rows` rows starting at sorted position `base`,
// as a per-lane value for lane row j = lane & 15 (-1 past the group).
template <class Meta>
__device__ __forceinline__ int group_slot(const Meta& m, int base, int rows, int lane) {
  const int j = lane & 15;
  int v = -1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < rows) {
      const int s = m.slot(base + r);
      v = (j == r) ? s : v;
    }
  }
  return v;
}

// This wave's stores (and loads) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_own_stores() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Segments per weight step: an item's segments (H / 256 for gate_up, I / 256 for down)
// must be a multiple of these, which the launchers check.  Activation chunks are a
// multiple of both, so they end on steps of either kernel.
constexpr int GU_SPS = 2;  // gate_up: 28 segments per item at H = 7168
constexpr int DN_SPS = 2;  // down: 8 segments per item at I = 2048
constexpr int CHUNK_ALIGN = GU_SPS > DN_SPS ? GU_SPS : DN_SPS;
// A half-width gate_up launch with fewer items than resident workgroup slots (bf16
// activations) takes steps of 4 segments: each workgroup streams one item, a half-width step
// is only 4 KB per wave, and the launch's bytes in flight, not the memory system, set its
// rate.  LDS holds gate_up to 2 workgroups per CU, so the twice-deeper ring's registers cost
// no occupancy.  Measured on the TP8 share at T = 4: gate_up 23.3 -> 19.4 us.  Full-width
// launches keep 2-segment steps (8 KB per wave): at T = 1 with a shared expert (288 items)
// the deeper ring was 4.5% slower.
constexpr int GU_SPS_DEEP = 4;
static_assert(CHUNK_ALIGN % GU_SPS == 0 && CHUNK_ALIGN % DN_SPS == 0, "chunks must end on steps");
// Activation chunk buffers: gate_up keeps 2 workgroups per CU with 32 KB chunks; down's
// items are short (I / 256 segments) and run 3 workgroups per CU with 16 KB chunks.
constexpr int GU_XCHUNK = 32768;
constexpr int DN_XCHUNK = 16384;
static_assert(SUB_ROWS * CHUNK_ALIGN <= XGeom<GU_XCHUNK>::ROWSEGS && SUB_ROWS * CHUNK_ALIGN <= XGeom<DN_XCHUNK>::ROWSEGS,
              "a chunk must hold one step of a full row group");
static_assert(SUB_ROWS * GU_SPS_DEEP <= XGeom<GU_XCHUNK>::ROWSEGS, "a gate_up chunk must hold one deep step of 16 rows");

struct ItemIndex {
  int a, quad, g;
};

__device__ __forceinline__ ItemIndex item_decode(int it, int nquad, int na) {
  ItemIndex r;
  const int q = it / nquad;
  r.quad = it - q * nquad;
  r.g = q / na;
  r.a = q - r.g * na;
  return r;
}

// Fields shared by both expert GEMMs: the work list over (row group, expert, tile quad).
template <class Meta>
struct ExpertItems {
  Meta m;
  int nseg, n_items, nquad, na;
  static constexpr bool SENTINEL = false;  // activations are complete when the launch starts
  int xrowsegs;  // row-segments per activation chunk
  int calign = CHUNK_ALIGN;  // chunk lengths are multiples of this (the launch's weight step)

  __device__ __forceinline__ int first_groups() const { return na * nquad; }
  // whether item `it` (per lane) exists: its row group starts below the expert's count
  __device__ __forceinline__ bool valid_lane(int it) const {
    const ItemIndex ix = item_decode(it, nquad, na);
    return ix.g * 16 < m.count_lane(ix.a);
  }
  __device__ __forceinline__ ItemInfo info(int it) const {
    const ItemIndex ix = item_decode(it, nquad, na);
    ItemInfo f;
    f.e = m.expert(ix.a);
    f.rows = min(16, m.count(ix.a) - ix.g * 16);
    f.row0 = m.offset(ix.a) + ix.g * 16;
    f.tile0 = ix.quad * WG_WAVES;
    f.cs = chunk_segments(f.rows, nseg, calign, xrowsegs);
    return f;
  }
  // nothing to wait for unless a policy says otherwise
  __device__ __forceinline__ void wait_inputs() const {}
};

// ------------------------------------------------------------------ gate_up + SwiGLU

// NS = 2: a wave's tile is 16 intermediate columns: subtile 0 = their 16 gate rows,
//         subtile 1 = the 16 matching up rows.
// NS = 1: a wave's tile is 8 intermediate columns: one subtile of their 8 gate rows
//         (rows 0-7) and the 8 matching up rows (rows 8-15).  The MFMA result rows 8-15 sit
//         in lanes 32-63, so one lane swap brings each up value beside its gate value.
// Half-width tiles double the waves streaming a launch with few items (small T).
template <int NS_, class Meta, int XCHUNK_, bool COH, bool A8 = false>
struct GateUpPolicy : ExpertItems<Meta> {
  static constexpr int NS = NS_;
  static constexpr int XCHUNK = XCHUNK_;
  static constexpr bool ACT8 = A8;  // x quantized to MXFP8 as it is staged
  typedef ScaleRun4 Scales;  // H % 1024 == 0
  static constexpr int TILE = NS == 2 ? SUB_ROWS : SUB_ROWS / 2;  // intermediate columns per wave
  struct EpiState {
    int hrow;  // h row of the group's first row
    int rows;  // valid rows in the group
    int n0;    // first intermediate column of this wave's tile
  };
  const uint16_t* xact;  // x [T, H]
  const uint8_t* wgu;
  const uint8_t* sgu;
  uint16_t* h;
  int H, I, k;
  uint32_t kinv;  // ceil(2^24 / k)
  size_t e_codes, e_scales;

  __device__ __forceinline__ u32x4 xload(const uint16_t* p) const { return ld16(p); }
  // token = slot / k as (slot * ceil(2^24 / k)) >> 24, exact for slot < 8192 and k <= 32
  static_assert(MX_MAX_TOKENS * MX_MAX_TOPK <= 8192 && MX_MAX_TOPK <= 32, "reciprocal range");
  __device__ __forceinline__ int x_row_offset(const ItemInfo& f, int m) const {
    const uint32_t slot = (uint32_t)this->m.slot(f.row0 + m);
    return (int)(((uint64_t)slot * kinv) >> 24) * H;
  }
  // weight row of row r (0..15) of subtile i of this wave's tile
  __device__ __forceinline__ int wrow(const ItemInfo& f, int wave, int i, int r) const {
    const int n0 = (f.tile0 + wave) * TILE;
    if (NS == 2) return (i ? I : 0) + n0 + r;
    return (r < 8) ? n0 + r : I + n0 + r - 8;
  }
  __device__ __forceinline__ void w_setup(const ItemInfo& f, int wave, WCursor<NS, Scales>& c, int lane) const {
    const uint8_t* we = wgu + (size_t)f.e * e_codes;
    const size_t kb = (size_t)H >> 1;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        c.w[i][q] = we + (size_t)wrow(f, wave, i, (lane >> 3) + 8 * q) * kb + (lane & 7) * 16;
  }
  __device__ __forceinline__ const uint8_t* scale_row(const ItemInfo& f, int wave, int i, int r) const {
    return sgu + (size_t)f.e * e_scales + (size_t)wrow(f, wave, i, r) * (H >> 5);
  }
  __device__ __forceinline__ void c_setup(const ItemInfo& f, int wave, EpiState& s, int) const {
    s.hrow = f.row0;
    s.rows = f.rows;
    s.n0 = (f.tile0 + wave) * TILE;
  }
  // MFMA result: lane l holds rows 4 (l >> 4) + 0..3 of the tile for token row l & 15.
  __device__ __forceinline__ void epilogue(const EpiState& s, const f32x4 (&acc)[NS], int lane) const {
    const int r = lane & 15;
    float g[4], u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] = acc[0][i];
      if constexpr (NS == 2) {
        u[i] = acc[1][i];
      } else {
        const uint32_t b = __float_as_uint(acc[0][i]);
        u[i] = __uint_as_float(__builtin_amdgcn_permlane32_swap(b, b, false, false)[1]);  // lane l <- lane l + 32
      }
    }
    if (r >= s.rows || (NS == 1 && lane >= 32)) return;
    uint32_t o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint16_t a = f32_to_bf16_rne(silu_mul(g[2 * j], u[2 * j]));
      const uint16_t b = f32_to_bf16_rne(silu_mul(g[2 * j + 1], u[2 * j + 1]));
      o[j] = (uint32_t)a | ((uint32_t)b << 16);
    }
    uint16_t* dst = h + (size_t)(s.hrow + r) * I + s.n0 + 4 * (lane >> 4);
    if (COH)
      st8_coherent(dst, (uint64_t)o[0] | ((uint64_t)o[1] << 32));
    else
      *reinterpret_cast<u32x2*>(dst) = u32x2{o[0], o[1]};
  }
};

// ------------------------------------------------------------------ down

// A wave's tile is NS x 16 output columns (subtile i = columns n0 + 16 i ... + 15).  The
// scale run is 4 segments when I % 1024 == 0, else 1 (I a multiple of 256, e.g. one
// tensor-parallel eighth of an expert).  DCOH: the down outputs are written with
// device-coherent stores (other workgroups of the launch combine them).
template <int NS_, class Meta, int XCHUNK_, bool COH, class SR = ScaleRun4, bool A8 = false, bool DCOH = COH>
struct DownPolicy : ExpertItems<Meta> {
  static constexpr int NS = NS_;
  static constexpr int XCHUNK = XCHUNK_;
  static constexpr bool ACT8 = A8;  // h quantized to MXFP8 as it is staged
  typedef SR Scales;
  static constexpr int TILE = NS * SUB_ROWS;  // output columns per wave
  struct EpiState {
    int slot;  // flat slot of this lane's row, -1 if the row is past the group
    int n0;    // first output column of this wave's tile
  };
  const uint16_t* xact;  // h [T*k, I], rows in sorted order
  const uint8_t* wd;
  const uint8_t* sd;
  float* dpart;
  int H, I;
  size_t e_codes, e_scales;
  // COH: h is produced by other workgroups of the launch; the first activation load of the
  // workgroup waits until *ready reaches ready_target (`flag`: zeroed LDS word for the wait)
  int32_t* ready;
  int32_t* err;
  lds_i32* flag;
  int ready_target;
  int wave;

  __device__ __forceinline__ u32x4 xload(const uint16_t* p) const {
    if (COH) return ld16_coherent(p);
    return ld16(p);
  }
  __device__ __forceinline__ void wait_inputs() const {
    if (COH) wait_counter(ready, ready_target, err, flag, wave);
  }
  __device__ __forceinline__ int x_row_offset(const ItemInfo& f, int m) const { return (f.row0 + m) * I; }
  __device__ __forceinline__ void w_setup(const ItemInfo& f, int wave, WCursor<NS, Scales>& c, int lane) const {
    const uint8_t* we = wd + (size_t)f.e * e_codes;
    const size_t kb = (size_t)I >> 1;
    const int n0 = (f.tile0 + wave) * TILE;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) c.w[i][q] = we + (size_t)(n0 + 16 * i + (lane >> 3) + 8 * q) * kb + (lane & 7) * 16;
  }
  __device__ __forceinline__ const uint8_t* scale_row(const ItemInfo& f, int wave, int i, int r) const {
    const int n = (f.tile0 + wave) * TILE + SUB_ROWS * i + r;
    return sd + (size_t)f.e * e_scales + (size_t)n * (I >> 5);
  }
  __device__ __forceinline__ void c_setup(const ItemInfo& f, int wave, EpiState& s, int lane) const {
    s.slot = group_slot(this->m, f.row0, f.rows, lane);
    s.n0 = (f.tile0 + wave) * TILE;
  }
  __device__ __forceinline__ void epilogue(const EpiState& s, const f32x4 (&acc)[NS], int lane) const {
    if (s.slot < 0) return;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float* dst = dpart + (size_t)s.slot * H + s.n0 + 16 * i + 4 * (lane >> 4);
      if (DCOH) {
        st8_coherent(dst, (uint64_t)__float_as_uint(acc[i][0]) | ((uint64_t)__float_as_uint(acc[i][1]) << 32));
        st8_coherent(dst + 2, (uint64_t)__float_as_uint(acc[i][2]) | ((uint64_t)__float_as_uint(acc[i][3]) << 32));
      } else {
        *reinterpret_cast<f32x4*>(dst) = acc[i];
      }
    }
  }
};

}  // namespace mx
