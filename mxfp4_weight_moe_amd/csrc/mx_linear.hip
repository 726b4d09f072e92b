// Dense MXFP4 linear layer (y = x W^T, W in MXFP4, x and y bf16, fp32 accumulation) and
// the standalone MXFP4 -> bf16 decode.
//
// The dense layer is the MXFP4 projection the AMD megakernel blog applies to attention
// projections and the LM head ("Bringing Ultra-Fast, Interactive LLM Inference to AMD
// Instinct MI355X GPUs", section "3. Low-Precision Data Types").  Two activation modes:
// bf16 (decode to bf16, bf16 MFMA), and MXFP8 as in that blog (activations quantized in the
// lanes, scaled MFMA; mx_act8.hpp).
//
// Work split: one workgroup per 16 output rows of W; its W waves split the K segments and
// sum their partial tiles through LDS in a fixed order.  Activation rows are processed in
// passes of up to 32 (two MFMA m-tiles).  One or two tokens with few output rows take a
// path of their own (one row per wave, below).
#include "mx_act8.hpp"
#include "mx_device.hpp"
#include "mx_internal.hpp"

namespace mx {

// DEEP: a 4-deep load pipeline for one m-tile (every segment of a wave in flight when the
// K split gives it at most 4), where the kernel's registers allow it; else 3 (one m-tile) or
// 2 (two m-tiles).  XL: x is the workgroup's LDS copy of the activations (same layout).
template <int W, int MT, bool SBYTE, bool A8, bool DEEP = false, bool XL = false>
__device__ __forceinline__ void dense_pass(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                           const uint8_t* __restrict__ s, uint16_t* __restrict__ y, int T, int K,
                                           int N, int n0, int mp, uint8_t* slab, f32x4* red, int wave, int lane) {
  constexpr int NS = 1;
  constexpr int D = (MT == 1) ? (DEEP ? 4 : 3) : 2;
  StreamLanes<NS, MT> L;
  lanes_init_lds(L, lane);
  const int kb = K >> 1, ks = K >> 5;
  for (int q = 0; q < 2; ++q) {
    const int r = min(n0 + (lane >> 3) + 8 * q, N - 1);
    L.w[0][q] = w + (size_t)r * kb + (lane & 7) * 16;
  }
  L.s[0] = s + (size_t)min(n0 + (lane & 15), N - 1) * ks;
  for (int mt = 0; mt < MT; ++mt) {
    const int t = mp + mt * 16 + (lane & 15);
    const int xo = A8 ? 32 * (lane >> 5) + 16 * ((lane >> 4) & 1) : 32 * (lane >> 4);
    L.x[mt] = (t < T) ? x + (size_t)t * K + xo : nullptr;
  }
  const int nseg = K / SEG_K;
  const int nb_tail = (K % SEG_K) / 32;
  const int sg0 = (int)((long)nseg * wave / W), sg1 = (int)((long)nseg * (wave + 1) / W);
  f32x4 acc[MT][NS];
  acc_zero(acc);
  if (SBYTE) {
    // Scale rows are not 8-byte aligned: every segment goes through the per-byte path.
    Stage<NS, MT> st;
    stage_zero_x(st);
    for (int sg = sg0; sg < sg1; ++sg) {
      stage_load_tail<NS, MT, A8>(st, L, sg, 8, lane);
      stage_consume<NS, MT, A8>(st, L, slab, acc, lane);
    }
    if (wave == W - 1 && nb_tail > 0) {
      stage_load_tail<NS, MT, A8>(st, L, nseg, nb_tail, lane);
      stage_consume<NS, MT, A8>(st, L, slab, acc, lane);
    }
  } else {
    stream_segments<NS, MT, D, A8, XL>(L, sg0, sg1, (wave == W - 1) ? nb_tail : 0, slab, acc, lane);
  }
  wg_reduce<NS, MT, W>(acc, red, wave, lane);
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = mp + mt * 16 + (lane & 15);
      if (t >= T) continue;
      const int n = n0 + 4 * (lane >> 4);
      uint16_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_rne(acc[mt][0][j]);
      uint16_t* yp = y + (size_t)t * N + n;
      if (n + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<u32x2*>(yp) = u32x2{(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
      } else {
        for (int j = 0; j < 4; ++j)
          if (n + j < N) yp[j] = o[j];
      }
    }
  }
}

// ONE_TILE: T <= 16, a single pass of one m-tile; the kernel then holds only that pass, whose
// registers leave room (with bf16 activations) for the 4-deep pipeline.
// XL (one tile, K % 256 == 0, T * K <= DENSE_XL_MAX): the workgroup first copies x into LDS
// (dynamic shared memory of T * K bf16) with full-width 16-byte loads, and the waves read
// their MFMA activation fragments from there.  Read from global memory, each fragment load
// has only T of every 16 lanes active, so at T = 4 the activation loads were 8 of the 11
// load instructions per segment and a fifth of the call's time.
constexpr int DENSE_XL_MAX = 32768;  // activation values staged in LDS (64 KB)
template <int W, bool SBYTE, bool A8, bool ONE_TILE, bool XL = false>
__global__ void __launch_bounds__(W * 64) mx_linear_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                           const uint8_t* __restrict__ s, uint16_t* __restrict__ y,
                                                           int T, int K, int N) {
  __shared__ __attribute__((aligned(16))) uint8_t slabs[W][SLAB_BYTES];
  __shared__ f32x4 red[(W > 1) ? W * 2 * 64 : 1];
  extern __shared__ u32x4 xdyn[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * SUB_ROWS;
  if constexpr (XL) {
    static_assert(ONE_TILE && !SBYTE, "LDS activations: one tile, whole segments");
    // 8 loads of a thread in flight at once, then their stores; no branches (a piece past
    // the end is the last piece again, stored with the same value)
    const int n16 = T * K / 8, nt = W * 64, t = threadIdx.x;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int i0 = t; i0 < n16; i0 += 8 * nt) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = xv[min(i0 + u * nt, n16 - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) xdyn[min(i0 + u * nt, n16 - 1)] = v[u];
    }
    __syncthreads();
    dense_pass<W, 1, SBYTE, A8, !A8, true>(reinterpret_cast<const uint16_t*>(xdyn), w, s, y, T, K, N, n0, 0,
                                           slabs[wave], red, wave, lane);
  } else if constexpr (ONE_TILE) {
    dense_pass<W, 1, SBYTE, A8, !A8>(x, w, s, y, T, K, N, n0, 0, slabs[wave], red, wave, lane);
  } else {
    for (int mp = 0; mp < T; mp += 32) {
      if (T - mp > 16)
        dense_pass<W, 2, SBYTE, A8>(x, w, s, y, T, K, N, n0, mp, slabs[wave], red, wave, lane);
      else
        dense_pass<W, 1, SBYTE, A8>(x, w, s, y, T, K, N, n0, mp, slabs[wave], red, wave, lane);
    }
  }
}

// ------------------------------------------------------------------ one row per wave (T <= 2)

// For one or two tokens and few output rows the MFMA tiles of 16 rows leave most CUs idle
// (2048 rows are 128 tiles for 256 CUs), and a call is about one memory round trip:
// measured on MI355X inside a HIP graph, a plain read of 2.2 MB takes 3.4 us spread over
// 137 workgroups and 2.1 us over 546.  Here a workgroup of 4 waves owns 4 output rows, one
// per wave, and each lane one MX block of its row at a time (16 code bytes, one scale
// byte): the codes are decoded straight to fp32 with the scaled conversion
// (v_cvt_scalef32_pk_f32_fp4, the E8M0 byte in the operand's exponent field, so 0xFF gives
// NaN), the products x * w are exact in fp32 (at most 8 + 2 significant bits), each lane
// sums its blocks in ascending K with fused multiply-adds (one rounding per term, as the
// plain sum of exact products), and the 64 lane sums are added in a fixed butterfly order.
// The activations (T * K <= 16384 values) are staged in LDS once per workgroup: read by
// every wave from global memory instead, the same few KB were requested by all 2048 waves
// of the 1-token layer and the call took 4.1 us; staged, 3.1 us (the MFMA path: 3.75 us).
constexpr int ROWS_WG = 4;
constexpr int ROWS_MAX_T = 2;
constexpr int ROWS_MAX_TK = 16384;  // activations staged in LDS: T * K bf16 values
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

template <int TT>
__global__ void __launch_bounds__(ROWS_WG * 64) mx_linear_rows_kernel(const uint16_t* __restrict__ x,
                                                                      const uint8_t* __restrict__ w,
                                                                      const uint8_t* __restrict__ s,
                                                                      uint16_t* __restrict__ y, int T, int K, int N) {
  __shared__ u32x4 xs[ROWS_MAX_TK / 8];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * ROWS_WG + (threadIdx.x >> 6);
  const int n = min(row, N - 1);  // rows past N compute row N - 1 again and store nothing
  const int nb = K >> 5;
  const uint8_t* wr = w + (size_t)n * (K >> 1);
  const uint8_t* sr = s + (size_t)n * nb;
  for (int i = threadIdx.x; i < T * K / 8; i += ROWS_WG * 64) xs[i] = ld16(x + (size_t)i * 8);
  __syncthreads();
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  // blocks lane, lane + 64, ...: four at a time, their loads issued before any use
  for (int b0 = 0; b0 < nb; b0 += 4 * 64) {
    u32x4 c[4];
    uint32_t sb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = min(b0 + u * 64 + lane, nb - 1);  // past the row's end: its last block, not summed
      c[u] = ld_stream16(wr + (size_t)b * 16);
      sb[u] = sr[b];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + u * 64 + lane;
      if (b >= nb) continue;
      const float sc = e8m0_scale_operand(sb[u]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // code dword q: K values 8q .. 8q + 7 of the block
        // byte p: values 8q + 2p (low nibble) and 8q + 2p + 1
        const f32x2 wv[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u][q], sc, 0),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u][q], sc, 1),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u][q], sc, 2),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u][q], sc, 3)};
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const u32x4 xw = xs[(min(t, T - 1) * K + b * 32) / 8 + q];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            acc[t] = __builtin_fmaf(bf16_lo(xw[p]), wv[p][0], acc[t]);
            acc[t] = __builtin_fmaf(bf16_hi(xw[p]), wv[p][1], acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float v = acc[t];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
    acc[t] = v;
  }
  if (row < N && lane < TT && lane < T) {
    float v = acc[0];
#pragma unroll
    for (int t = 1; t < TT; ++t) v = (lane == t) ? acc[t] : v;
    y[(size_t)lane * N + n] = f32_to_bf16_rne(v);
  }
}

template <bool A8>
static int launch_dense(const uint16_t* x, const uint8_t* w, const uint8_t* s, uint16_t* y, int T, int K, int N,
                        hipStream_t stream) {
  const int items = (N + SUB_ROWS - 1) / SUB_ROWS;
  if constexpr (!A8) {
    // one or two tokens and fewer 16-row tiles than two per CU: one row per wave
    if (T <= ROWS_MAX_T && T * K <= ROWS_MAX_TK && items < 2 * device_cu_count()) {
      const dim3 grid((unsigned)((N + ROWS_WG - 1) / ROWS_WG)), block(ROWS_WG * 64);
      if (T == 1)
        hipLaunchKernelGGL((mx_linear_rows_kernel<1>), grid, block, 0, stream, x, w, s, y, T, K, N);
      else
        hipLaunchKernelGGL((mx_linear_rows_kernel<2>), grid, block, 0, stream, x, w, s, y, T, K, N);
      return hip_status(hipGetLastError());
    }
  }
  const int nseg = K / SEG_K;
  // Up to 8 waves split K; with MXFP8 activations at most 4, whose registers then fit
  // without spilling (8 waves of 64 lanes leave each lane half the register file).
  constexpr int WMAX = A8 ? 4 : 8;
  int W = 1;
  while (W < WMAX && 2 * W <= nseg && items * W < 2048) W *= 2;
  const bool sbyte = (K % SEG_K) != 0;
  const bool xl = T <= 16 && !sbyte && T * K <= DENSE_XL_MAX;
  const unsigned xl_bytes = xl ? (unsigned)(T * K * 2) : 0u;
  dim3 grid(items), block(W * 64);
#define MXL1(WW, SB, OT, XX) \
  hipLaunchKernelGGL((mx_linear_kernel<WW, SB, A8, OT, XX>), grid, block, xl_bytes, stream, x, w, s, y, T, K, N)
#define MXL(WW, SB)                           \
  do {                                        \
    if (T <= 16 && !(SB) && xl)               \
      MXL1(WW, false, true, true);            \
    else if (T <= 16)                         \
      MXL1(WW, SB, true, false);              \
    else                                      \
      MXL1(WW, SB, false, false);             \
  } while (0)
  if (sbyte) {
    switch (W) {
      case 1: MXL(1, true); break;
      case 2: MXL(2, true); break;
      case 4: MXL(4, true); break;
      default:
        if constexpr (WMAX == 8) MXL(8, true);
        break;
    }
  } else {
    switch (W) {
      case 1: MXL(1, false); break;
      case 2: MXL(2, false); break;
      case 4: MXL(4, false); break;
      default:
        if constexpr (WMAX == 8) MXL(8, false);
        break;
    }
  }
#undef MXL
#undef MXL1
  return hip_status(hipGetLastError());
}

int launch_mx_linear(const uint16_t* x, const uint8_t* w, const uint8_t* s, uint16_t* y, int T, int K, int N,
                     hipStream_t stream) {
  return launch_dense<false>(x, w, s, y, T, K, N, stream);
}

int launch_mx_linear_a8(const uint16_t* x, const uint8_t* w, const uint8_t* s, uint16_t* y, int T, int K, int N,
                        hipStream_t stream) {
  return launch_dense<true>(x, w, s, y, T, K, N, stream);
}

// ------------------------------------------------------------------ MXFP8 quantization

// One thread per 8-value piece; the 4 pieces of a block are 4 consecutive threads (rows are
// contiguous and K % 32 == 0, so piece p belongs to block p / 4 of the flattened tensor).
__global__ void __launch_bounds__(256) mxfp8_quantize_kernel(const uint16_t* __restrict__ x, int64_t npieces,
                                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = p < npieces;  // npieces % 4 == 0: a block's 4 threads are all in or all out
  const u32x4 v = ok ? ld16(x + p * 8) : u32x4{0u, 0u, 0u, 0u};
  uint32_t sb;
  const u32x2 c = act8_quant_quad(v, sb);
  if (ok) {
    *reinterpret_cast<u32x2*>(codes + p * 8) = c;
    if ((p & 3) == 0) scales[p >> 2] = (uint8_t)sb;
  }
}

int launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                          hipStream_t stream) {
  const int64_t npieces = rows * (K / 8);
  const int64_t grid = (npieces + 255) / 256;
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, npieces, codes, scales);
  return hip_status(hipGetLastError());
}

// ------------------------------------------------------------------ decode

// One thread per MX block: 16 code bytes + 1 scale byte -> 32 bf16 (64 bytes).
__global__ void __launch_bounds__(256) mxfp4_dequant_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ s,
                                                            int64_t nblocks, uint16_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4 codes = ld16(w + b * 16);
  const float sc = e8m0_scale_operand(s[b]);
  u32x4* o = reinterpret_cast<u32x4*>(out + b * 32);
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = __builtin_bit_cast(u32x4, decode8(codes[c], sc));
}

int launch_dequant(const uint8_t* w, const uint8_t* s, int64_t rows, int64_t K, uint16_t* out, hipStream_t stream) {
  const int64_t nblocks = rows * (K / 32);  // blocks are contiguous in both tensors
  const int64_t grid = (nblocks + 255) / 256;
  hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, s, nblocks, out);
  return hip_status(hipGetLastError());
}

}  // namespace mx
