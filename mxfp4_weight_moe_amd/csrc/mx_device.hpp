// Device-side building blocks for streaming MXFP4 weights through bf16 MFMA on gfx950.
//
// Format (Zyphra Inference Wave 2, section "Quantization."): blocks of 32 E2M1 4-bit
// values share one E8M0 power-of-two scale, 4.25 bits per value.  Layout taken by this
// library: a weight matrix with `rows` output features and reduction length K is stored
// row-major as codes [rows][K/2] (two codes per byte, element 2i in the low nibble) and
// scales [rows][K/32] (one byte per 32 consecutive K values of one row).
//
// Streaming scheme (one wavefront):
//   * A "segment" is 256 K values of a row: 128 code bytes (8 MX blocks) + 8 scale bytes.
//   * Codes are loaded as 16-byte nontemporal loads, 8 rows x 128 contiguous bytes per
//     instruction, so every instruction moves whole 128-byte lines.
//   * The 16x128-byte subtile is transposed through a wave-private LDS slab (XOR-swizzled
//     16-byte chunks, conflict-free on both sides) into the MFMA operand layout: lane l
//     holds row (l & 15), MX blocks (l >> 4) and (l >> 4) + 4.
//   * Each dword of codes (8 values) becomes 8 bf16 with v_cvt_scalef32_pk_bf16_fp4, whose
//     scale operand is an fp32 whose exponent field is the E8M0 byte (so 0x00 -> 2^-127,
//     0xFF -> NaN, exactly the E8M0 meaning).  Products with bf16 activations are exact
//     and v_mfma_f32_16x16x32_bf16 accumulates them in fp32.
//   * The 32 K values an MFMA consumes are a permutation of the segment shared by both
//     operands: MFMA lane group g = l >> 4 at step (h, c) carries K offsets
//     32 * (g + 4h) + 8c + [0, 8) of the segment.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int SEG_K = 256;       // K values per segment
constexpr int SEG_BYTES = 128;   // code bytes per row per segment
constexpr int SEG_SCALES = 8;    // scale bytes per row per segment
constexpr int SUB_ROWS = 16;     // rows per MFMA subtile
constexpr int SLAB_BYTES = SUB_ROWS * SEG_BYTES;  // LDS bytes per subtile transpose slab

// ------------------------------------------------------------------ scalar helpers

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN; overflow rounds to Inf.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Device-coherent 8- and 16-byte accesses (agent-scope relaxed atomics compile to plain
// loads and stores with the sc1 bit).
__device__ __forceinline__ void st8_coherent(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld8_coherent(const void* p) {
  return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 ld16_coherent(const void* p) {
  const uint64_t a = ld8_coherent(p);
  const uint64_t b = ld8_coherent(static_cast<const uint8_t*>(p) + 8);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// The conversion instruction reads the E8M0 scale from the exponent field of an fp32.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// 8 E2M1 codes (one dword, element 0 in the low nibble) -> 8 bf16 = code value * 2^(s-127).
__device__ __forceinline__ bf16x8 decode8(uint32_t codes, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  bf16x4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld_stream16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// ------------------------------------------------------------------ the streaming core

// Per-lane addressing of one wavefront over NS weight subtiles (16 rows each) and MT
// activation m-tiles (16 rows each).  Pointers are set up once per work item.
template <int NS, int MT>
struct StreamLanes {
  const uint8_t* w[NS][2];  // code bytes: row (l>>3) + 8q, byte (l&7)*16, segment 0
  const uint8_t* s[NS];     // scale bytes: row (l&15), segment 0
  const uint16_t* x[MT];    // activation row of column (l&15), element 32*(l>>4); null = zero row
  uint32_t lds_wr[2];       // slab byte offsets written by this lane (q = 0, 1)
  uint32_t lds_rd[2];       // slab byte offsets read by this lane (h = 0, 1)
  uint32_t sshift;          // bit offset of this lane's block within a scale dword
};

// Slab byte offset of (row r, 16-byte block b): rows of 128 B, blocks XOR-swizzled by row.
__device__ __forceinline__ uint32_t slab_off(uint32_t r, uint32_t b) { return r * SEG_BYTES + ((b ^ (r & 7u)) << 4); }

template <int NS, int MT>
__device__ __forceinline__ void lanes_init_lds(StreamLanes<NS, MT>& L, int lane) {
  for (int q = 0; q < 2; ++q) L.lds_wr[q] = slab_off((uint32_t)(lane >> 3) + 8u * q, (uint32_t)(lane & 7));
  for (int h = 0; h < 2; ++h) L.lds_rd[h] = slab_off((uint32_t)(lane & 15), (uint32_t)(lane >> 4) + 4u * h);
  L.sshift = 8u * (uint32_t)(lane >> 4);
}

// One pipeline stage: everything one segment needs, loaded ahead of use.
template <int NS, int MT>
struct Stage {
  u32x4 w[NS][2];
  u32x2 s[NS];
  u32x4 x[MT][8];
};

template <int NS, int MT>
__device__ __forceinline__ void stage_zero_x(Stage<NS, MT>& st) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 8; ++v) st.x[mt][v] = u32x4{0u, 0u, 0u, 0u};
}

// Activation pieces (8 values each) of half h of a segment: piece c of a lane in group g.
// bf16 activations: the lane's row pointer is x + t * K + 32 * g, and pieces 0-3 are block
// g + 4h.  A8 (MXFP8 activations for the scaled MFMA): the row pointer is
// x + t * K + 32 * (g >> 1) + 16 * (g & 1); pieces 0, 1 are half (g & 1) of block 4h + (g >> 1)
// and pieces 2, 3 the same half of block 4h + 2 + (g >> 1).
template <bool A8>
__device__ __forceinline__ int x_piece_off(int h, int c) {
  return A8 ? h * 128 + (c >> 1) * 64 + (c & 1) * 8 : h * 128 + c * 8;
}
template <bool A8>
__device__ __forceinline__ int x_piece_block(int g, int h, int c) {
  return A8 ? 4 * h + 2 * (c >> 1) + (g >> 1) : g + 4 * h;
}

typedef __attribute__((address_space(3))) const uint16_t* lds_cu16_ptr;
typedef __attribute__((address_space(3))) const u32x4* lds_cu32x4_ptr;

// Load segment `sg` (a full segment: all 8 blocks of the 256 K values exist).  XL: the
// activation rows L.x point into LDS (staged there by the caller), read with LDS loads.
template <int NS, int MT, bool A8 = false, bool XL = false>
__device__ __forceinline__ void stage_load(Stage<NS, MT>& st, const StreamLanes<NS, MT>& L, int sg) {
  const size_t wo = (size_t)sg * SEG_BYTES;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    st.w[i][0] = ld_stream16(L.w[i][0] + wo);
    st.w[i][1] = ld_stream16(L.w[i][1] + wo);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) st.s[i] = ld8(L.s[i] + (size_t)sg * SEG_SCALES);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (L.x[mt]) {
      if constexpr (XL) {
        const lds_cu16_ptr xp = (lds_cu16_ptr)L.x[mt] + sg * SEG_K;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c = 0; c < 4; ++c) st.x[mt][h * 4 + c] = *(lds_cu32x4_ptr)(xp + x_piece_off<A8>(h, c));
      } else {
        const uint16_t* xp = L.x[mt] + (size_t)sg * SEG_K;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c = 0; c < 4; ++c) st.x[mt][h * 4 + c] = ld16(xp + x_piece_off<A8>(h, c));
      }
    }
  }
}

// Load a final partial segment with `nb` (< 8) valid MX blocks; missing blocks read as
// zero codes and zero activations, so they add nothing.
template <int NS, int MT, bool A8 = false>
__device__ __forceinline__ void stage_load_tail(Stage<NS, MT>& st, const StreamLanes<NS, MT>& L, int sg, int nb,
                                                int lane) {
  const size_t wo = (size_t)sg * SEG_BYTES;
  const bool wok = (lane & 7) < nb;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    st.w[i][0] = wok ? ld_stream16(L.w[i][0] + wo) : u32x4{0u, 0u, 0u, 0u};
    st.w[i][1] = wok ? ld_stream16(L.w[i][1] + wo) : u32x4{0u, 0u, 0u, 0u};
  }
  const int b0 = lane >> 4;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const uint8_t* sp = L.s[i] + (size_t)sg * SEG_SCALES;
    // only bytes b0 and b0 + 4 of the 8 are used by this lane
    uint32_t lo = (b0 < nb) ? (uint32_t)sp[b0] << (8 * b0) : 0x7Fu << (8 * b0);
    uint32_t hi = (b0 + 4 < nb) ? (uint32_t)sp[b0 + 4] << (8 * b0) : 0x7Fu << (8 * b0);
    st.s[i] = u32x2{lo, hi};
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t* xp = L.x[mt] + (size_t)sg * SEG_K;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = (L.x[mt] != nullptr) && (x_piece_block<A8>(b0, h, c) < nb);
        st.x[mt][h * 4 + c] = ok ? ld16(xp + x_piece_off<A8>(h, c)) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

// Consume one stage: transpose codes through the wave's LDS slabs, decode, MFMA.
template <int NS, int MT>
__device__ __forceinline__ void stage_compute(const Stage<NS, MT>& st, const StreamLanes<NS, MT>& L,
                                              uint8_t* __restrict__ slab, f32x4 (&acc)[MT][NS]) {
  u32x4 wc[NS][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    *reinterpret_cast<u32x4*>(slab + i * SLAB_BYTES + L.lds_wr[0]) = st.w[i][0];
    *reinterpret_cast<u32x4*>(slab + i * SLAB_BYTES + L.lds_wr[1]) = st.w[i][1];
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    wc[i][0] = *reinterpret_cast<const u32x4*>(slab + i * SLAB_BYTES + L.lds_rd[0]);
    wc[i][1] = *reinterpret_cast<const u32x4*>(slab + i * SLAB_BYTES + L.lds_rd[1]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float sc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) sc[i] = e8m0_scale_operand((st.s[i][h] >> L.sshift) & 0xFFu);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bf16x8 wb = decode8(wc[i][h][c], sc[i]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][i] = mfma_bf16(wb, as_bf16x8(st.x[mt][h * 4 + c]), acc[mt][i]);
      }
    }
  }
}

template <int NS, int MT>
__device__ void stage_compute_a8(const Stage<NS, MT>& st, const StreamLanes<NS, MT>& L, uint8_t* __restrict__ slab,
                                 f32x4 (&acc)[MT][NS], int lane);  // mx_act8.hpp

template <int NS, int MT, bool A8>
__device__ __forceinline__ void stage_consume(const Stage<NS, MT>& st, const StreamLanes<NS, MT>& L,
                                              uint8_t* __restrict__ slab, f32x4 (&acc)[MT][NS], int lane) {
  if constexpr (A8)
    stage_compute_a8(st, L, slab, acc, lane);
  else
    stage_compute(st, L, slab, acc);
}

// Stream segments [sg0, sg1) (+ an optional partial tail segment with nb_tail blocks at
// index sg1, not with XL) into acc with a D-deep register pipeline.  XL: the activation
// rows are in LDS.
template <int NS, int MT, int D, bool A8 = false, bool XL = false>
__device__ __forceinline__ void stream_segments(const StreamLanes<NS, MT>& L, int sg0, int sg1, int nb_tail,
                                                uint8_t* __restrict__ slab, f32x4 (&acc)[MT][NS], int lane) {
  Stage<NS, MT> st[D];
#pragma unroll
  for (int d = 0; d < D; ++d) stage_zero_x(st[d]);
  const int n = sg1 - sg0;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < n) stage_load<NS, MT, A8, XL>(st[d], L, sg0 + d);
  for (int b = 0; b < n; b += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (b + d < n) {
        stage_consume<NS, MT, A8>(st[d], L, slab, acc, lane);
        if (b + d + D < n) stage_load<NS, MT, A8, XL>(st[d], L, sg0 + b + d + D);
      }
    }
  }
  if (!XL && nb_tail > 0) {
    stage_load_tail<NS, MT, A8>(st[0], L, sg1, nb_tail, lane);
    stage_consume<NS, MT, A8>(st[0], L, slab, acc, lane);
  }
}

template <int NS, int MT>
__device__ __forceinline__ void acc_zero(f32x4 (&acc)[MT][NS]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Wave-local sum of acc over the W waves of a workgroup, through LDS (fixed order, so
// the result does not depend on timing).  `red` holds W * MT * NS * 64 f32x4.  Every
// wave calls it; afterwards wave 0's acc holds the total.
template <int NS, int MT, int W>
__device__ __forceinline__ void wg_reduce(f32x4 (&acc)[MT][NS], f32x4* red, int wave, int lane) {
  if (W == 1) return;
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < NS; ++i) red[((wave * MT + mt) * NS + i) * 64 + lane] = acc[mt][i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        f32x4 a = red[((0 * MT + mt) * NS + i) * 64 + lane];
        for (int w = 1; w < W; ++w) a += red[((w * MT + mt) * NS + i) * 64 + lane];
        acc[mt][i] = a;
      }
  }
  __syncthreads();
}

}  // namespace mx
