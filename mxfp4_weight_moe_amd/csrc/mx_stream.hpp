// Continuous weight streaming for the expert GEMMs.
//
// A wavefront owns a strided subset of the work items (item it = wave_id + j * n_waves).
// Each item is `nseg` segments of 256 K values over NS weight subtiles of 16 rows.  The
// wave walks the concatenated segment sequence of all its items with two register rings:
//   - weights (+ scales) for segment g + DW are issued after segment g is consumed;
//   - activations for segment g + DX are issued just before them, DX < DW.
// Loads retire in issue order, so waiting for the activations of segment g also covers
// its weights (issued earlier) and leaves the later weight loads in flight.  The rings
// run across item boundaries: there is no pipeline drain between items, only the
// epilogue of the finished item.
//
// Activation rows are handled 16 at a time (one MFMA m-tile).  An expert with more than
// 16 routed rows yields one item per group of 16 rows.  Activations are read with raw
// buffer loads; lanes of rows past the end of a group use an out-of-range offset, so the
// load returns zeros without touching memory and without a branch around it.
//
// Every step issues the same loads whatever the state (an exhausted cursor re-reads its
// last segment), so the compiler's wait counts are exact: each step waits only for the
// segment it consumes.
#pragma once
#include "mx_device.hpp"

namespace mx {

template <int NS>
struct WRing {
  u32x4 w[NS][2];
  u32x2 s[NS];
};

struct XRing {
  u32x4 x[8];
};

template <int NS>
struct WCursor {
  int it;   // current item (>= n_items: exhausted)
  int seg;  // next segment to load
  const uint8_t* w[NS][2];
  const uint8_t* s[NS];
};

struct XCursor {
  int it;
  int seg;
  int xoff;  // byte offset of this lane's activation row (+ 32 * (lane >> 4) values); X_NONE if none
};

constexpr int X_NONE = 0x7F000000;  // beyond any activation buffer this library addresses (<= 1 GiB)

// Raw buffer resource over `bytes` bytes at `base` (stride 0, 32-bit offsets, bounds-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int NS>
__device__ __forceinline__ void wring_load(WRing<NS>& r, const WCursor<NS>& c) {
  const size_t wo = (size_t)c.seg * SEG_BYTES;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    r.w[i][0] = ld_stream16(c.w[i][0] + wo);
    r.w[i][1] = ld_stream16(c.w[i][1] + wo);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) r.s[i] = ld8(c.s[i] + (size_t)c.seg * SEG_SCALES);
}

__device__ __forceinline__ void xring_load(XRing& r, const XCursor& c, __amdgpu_buffer_rsrc_t xr) {
  const int o = c.xoff + c.seg * SEG_K * 2;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r.x[h * 4 + q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, o + h * 256 + q * 16, 0, 0));
}

// Consume one segment: LDS transpose of the codes, decode, MFMA into acc[NS].
template <int NS>
__device__ __forceinline__ void segment_compute(const WRing<NS>& wr, const XRing& xr, uint8_t* __restrict__ slab,
                                                const uint32_t (&lds_wr)[2], const uint32_t (&lds_rd)[2],
                                                uint32_t sshift, f32x4 (&acc)[NS]) {
  u32x4 wc[NS][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    *reinterpret_cast<u32x4*>(slab + i * SLAB_BYTES + lds_wr[0]) = wr.w[i][0];
    *reinterpret_cast<u32x4*>(slab + i * SLAB_BYTES + lds_wr[1]) = wr.w[i][1];
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    wc[i][0] = *reinterpret_cast<const u32x4*>(slab + i * SLAB_BYTES + lds_rd[0]);
    wc[i][1] = *reinterpret_cast<const u32x4*>(slab + i * SLAB_BYTES + lds_rd[1]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float sc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) sc[i] = e8m0_scale_operand((wr.s[i][h] >> sshift) & 0xFFu);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 xb = as_bf16x8(xr.x[h * 4 + c]);
#pragma unroll
      for (int i = 0; i < NS; ++i) acc[i] = mfma_bf16(decode8(wc[i][h][c], sc[i]), xb, acc[i]);
    }
  }
}

// Drive the rings over the wave's items.  Policy P provides:
//   static constexpr int NS;   int nseg;   int n_items;
//   bool valid(int it)                           -- item has rows to compute
//   void w_setup(int it, WCursor<NS>&, lane)     -- weight/scale row pointers, segment 0
//   void x_setup(int it, XCursor&, lane)         -- activation byte offset (X_NONE: no row)
//   __amdgpu_buffer_rsrc_t xrsrc                 -- the activation buffer
//   void c_setup(int it, EpiState&, lane)        -- epilogue state (may issue loads)
//   void epilogue(const EpiState&, const f32x4 (&acc)[NS], lane)
template <class P, int DW, int DX>
__device__ __forceinline__ void stream_items(P& p, int wave_id, int n_waves, uint8_t* __restrict__ slab, int lane) {
  constexpr int NS = P::NS;
  static_assert(DX < DW, "activations must be issued after the weights of the same segment");
  static_assert(DW % DX == 0, "ring depths must nest");
  uint32_t lds_wr[2], lds_rd[2];
  for (int q = 0; q < 2; ++q) lds_wr[q] = slab_off((uint32_t)(lane >> 3) + 8u * q, (uint32_t)(lane & 7));
  for (int h = 0; h < 2; ++h) lds_rd[h] = slab_off((uint32_t)(lane & 15), (uint32_t)(lane >> 4) + 4u * h);
  const uint32_t sshift = 8u * (uint32_t)(lane >> 4);

  auto next_valid = [&](int it) {
    while (it < p.n_items && !p.valid(it)) it += n_waves;
    return it;
  };
  const int first = next_valid(wave_id);
  if (first >= p.n_items) return;

  WCursor<NS> cw;
  XCursor cx;
  typename P::EpiState es;
  cw.it = first;
  cw.seg = 0;
  p.w_setup(first, cw, lane);
  cx.it = first;
  cx.seg = 0;
  p.x_setup(first, cx, lane);
  int cit = first, cseg = 0;
  p.c_setup(first, es, lane);

  // Advance a cursor by one segment; once past its last item it stays on its last
  // segment, so the loads it keeps issuing read valid memory.
  auto advance_w = [&]() {
    if (cw.seg + 1 < p.nseg) {
      ++cw.seg;
    } else {
      const int nx = next_valid(cw.it + n_waves);
      if (nx < p.n_items) {
        cw.it = nx;
        cw.seg = 0;
        p.w_setup(nx, cw, lane);
      }
    }
  };
  auto advance_x = [&]() {
    if (cx.seg + 1 < p.nseg) {
      ++cx.seg;
    } else {
      const int nx = next_valid(cx.it + n_waves);
      if (nx < p.n_items) {
        cx.it = nx;
        cx.seg = 0;
        p.x_setup(nx, cx, lane);
      }
    }
  };

  WRing<NS> rw[DW];
  XRing rx[DX];
#pragma unroll
  for (int d = 0; d < DX; ++d)
#pragma unroll
    for (int v = 0; v < 8; ++v) rx[d].x[v] = u32x4{0u, 0u, 0u, 0u};
  // prologue: weights DW segments ahead, then activations DX segments ahead
#pragma unroll
  for (int d = 0; d < DW; ++d) {
    wring_load(rw[d], cw);
    advance_w();
  }
#pragma unroll
  for (int d = 0; d < DX; ++d) {
    xring_load(rx[d], cx, p.xrsrc);
    advance_x();
  }

  f32x4 acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  while (cit < p.n_items) {
#pragma unroll
    for (int u = 0; u < DW; ++u) {
      if (cit < p.n_items) {
        segment_compute<NS>(rw[u], rx[u % DX], slab, lds_wr, lds_rd, sshift, acc);
        if (++cseg == p.nseg) {
          p.epilogue(es, acc, lane);
#pragma unroll
          for (int i = 0; i < NS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          cit = next_valid(cit + n_waves);
          cseg = 0;
          if (cit < p.n_items) p.c_setup(cit, es, lane);
        }
      }
      xring_load(rx[u % DX], cx, p.xrsrc);
      advance_x();
      wring_load(rw[u], cw);
      advance_w();
    }
  }
}

}  // namespace mx
