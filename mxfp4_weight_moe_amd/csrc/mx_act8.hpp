// MXFP8 activations for the scaled MFMA of gfx950.
//
// The AMD megakernel blog ("Bringing Ultra-Fast, Interactive LLM Inference to AMD Instinct
// MI355X GPUs", section "3. Low-Precision Data Types") feeds MXFP4 weights to the matrix
// instructions with MXFP8 activations; the Zyphra page ("Zyphra Inference Wave 2",
// Appendix B) names the scaled f8f6f4 MFMA as the full-rate FP8/FP4 path.  Here the
// activations are quantized on the fly, block by block, and the weights' E2M1 codes and
// E8M0 scales go to v_mfma_scale_f32_16x16x128_f8f6f4 as they are: no decode on the VALU.
//
// Quantization (OCP MX, E4M3 elements): per block of 32 consecutive K values of one row,
// scale = 2^(floor(log2 amax) - 8), clamped at 2^-127, and each value / scale rounded to the
// nearest E4M3 value (ties to even), saturating at +-448.  A block with an Inf or NaN gets
// scale 0xFF and codes 0x7F.  v_cvt_scalef32_pk_fp8_bf16 divides by the E8M0 scale held in an
// fp32's exponent field and rounds to nearest even, but returns NaN past 448, so inputs are
// first clamped to 448 * scale (exact in bf16).  Since floor(log2 amax) is the bf16 exponent
// field, the whole rule is integer work on the bf16 bits.
//
// Operand layout of the 16x16x128 MFMA (16 output rows x 16 tokens, K = 4 blocks of 32):
//   A = weights (E2M1, format 4): lane group g = l >> 4 holds K block g, 32 values, in the
//       low 4 of its 8 operand registers, with that block's scale;
//   B = activations (E4M3, format 0): lane group g holds 16 values of block g >> 1 (half
//       g & 1) in registers 0-3 and the same half of block 2 + (g >> 1) in registers 4-7,
//       and supplies the scale of block g.
// Within a 32-value block the hardware sums products in groups of 8 and drops the bits of
// each product that lie more than about 14 binades below the largest product of its group;
// the result is therefore not exact (the error is at most about 7 * 2^-14 of the sum of the
// group's |products|).
#pragma once
#include "mx_device.hpp"

namespace mx {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short s16x2;

// Running per-half maxima of |x| over bf16 pairs (bit patterns of non-negative bf16 order
// like the values; Inf and NaN sort above every finite value).
__device__ __forceinline__ uint32_t absmax_pk(uint32_t m, uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                __builtin_bit_cast(u16x2, d & 0x7FFF7FFFu)));
}
__device__ __forceinline__ uint32_t absmax_fold(uint32_t m) { return max(m & 0xFFFFu, m >> 16); }
__device__ __forceinline__ uint32_t absmax8(const u32x4& v) {
  uint32_t m = absmax_pk(absmax_pk(v[0] & 0x7FFF7FFFu, v[1]), v[2]);
  return absmax_fold(absmax_pk(m, v[3]));
}

// E8M0 scale byte of a block from the bit pattern of its largest |x|.
__device__ __forceinline__ uint32_t act8_scale(uint32_t amax) {
  if (amax >= 0x7F80u) return 0xFFu;
  const uint32_t ef = amax >> 7;  // bf16 exponent field = floor(log2 amax) + 127 for normal amax
  return ef > 8u ? ef - 8u : 0u;
}

// 8 bf16 values (ascending in memory) -> 8 E4M3 codes (ascending bytes) at scale byte sb.
__device__ __forceinline__ u32x2 act8_codes8(const u32x4& v, uint32_t sb) {
  const uint32_t lim = ((sb + 8u) << 7) | 0x60u;  // bf16 bits of 448 * 2^(sb - 127), sb <= 246
  const u16x2 lim2 = {(unsigned short)lim, (unsigned short)lim};
  const float sc = __uint_as_float(sb << 23);
  uint32_t out[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t d[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t a = v[2 * j + q];
      const u16x2 m = __builtin_elementwise_min(__builtin_bit_cast(u16x2, a & 0x7FFF7FFFu), lim2);
      d[q] = __builtin_bit_cast(uint32_t, m) | (a & 0x80008000u);
    }
    s16x2 c = {0, 0};
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, d[0]), sc, false);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, d[1]), sc, true);
    out[j] = __builtin_bit_cast(uint32_t, c);
  }
  if (sb == 0xFFu) return u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
  return u32x2{out[0], out[1]};
}

// One 8-value piece of a block whose 4 pieces sit in 4 consecutive lanes (lane & 3 = piece,
// all 4 lanes active): the block's scale byte (sb) and this piece's 8 codes.
__device__ __forceinline__ u32x2 act8_quant_quad(const u32x4& v, uint32_t& sb) {
  uint32_t m = absmax8(v);
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  sb = act8_scale(m);
  return act8_codes8(v, sb);
}

// acc += W (E2M1 block per lane group, scale ws) x X (E4M3, scale xs), K = 128.
__device__ __forceinline__ f32x4 mfma_scale_a8(const u32x4& w, const u32x4& xlo, const u32x4& xhi, f32x4 c, int ws,
                                               int xs) {
  const i32x8 a = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  const i32x8 b = {(int)xlo[0], (int)xlo[1], (int)xlo[2], (int)xlo[3],
                   (int)xhi[0], (int)xhi[1], (int)xhi[2], (int)xhi[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, ws, 0, xs);
}

// ------------------------------------------------------------------ dense layer

// One segment with activations quantized in the lane: each lane holds its two half-blocks,
// finds their block maxima with the lane holding the other halves (lane l ^ 16), and takes
// the scale of block g from lane group g (groups 1 and 2 swap theirs).
template <int NS, int MT>
__device__ void stage_compute_a8(const Stage<NS, MT>& st, const StreamLanes<NS, MT>& L,
                                                 uint8_t* __restrict__ slab, f32x4 (&acc)[MT][NS], int lane) {
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
  const int g = lane >> 4;
  const int src = (g == 1) ? lane + 16 : (g == 2) ? lane - 16 : lane;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int ws[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) ws[i] = (int)((st.s[i][h] >> L.sshift) & 0xFFu);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4* p = &st.x[mt][h * 4];
      uint32_t mlo = max(absmax8(p[0]), absmax8(p[1]));
      uint32_t mhi = max(absmax8(p[2]), absmax8(p[3]));
      mlo = max(mlo, (uint32_t)__builtin_amdgcn_ds_swizzle((int)mlo, 0x401F));  // lane ^ 16
      mhi = max(mhi, (uint32_t)__builtin_amdgcn_ds_swizzle((int)mhi, 0x401F));
      const uint32_t slo = act8_scale(mlo), shi = act8_scale(mhi);
      const u32x2 c0 = act8_codes8(p[0], slo), c1 = act8_codes8(p[1], slo);
      const u32x2 c2 = act8_codes8(p[2], shi), c3 = act8_codes8(p[3], shi);
      const uint32_t recv = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)((g == 1) ? shi : slo));
      const int xs = (int)((g == 0) ? slo : (g == 3) ? shi : recv);
      const u32x4 xlo = {c0[0], c0[1], c1[0], c1[1]}, xhi = {c2[0], c2[1], c3[0], c3[1]};
#pragma unroll
      for (int i = 0; i < NS; ++i) acc[mt][i] = mfma_scale_a8(wc[i][h], xlo, xhi, acc[mt][i], ws[i], xs);
    }
  }
}

}  // namespace mx
