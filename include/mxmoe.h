/*
 * mxmoe -- MXFP4 weight-streaming MoE expert layer and dense MXFP4 linear layer for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (sources):
 *   - MXFP4 ("Zyphra Inference Wave 2", section "Quantization."; the Open Compute
 *     Project MX specification it names): blocks of 32 E2M1 4-bit values share one
 *     E8M0 power-of-two scale; 4.25 bits per value.  E2M1 code c: sign = bit 3,
 *     magnitude {0, 0.5, 1, 1.5, 2, 3, 4, 6}[c & 7].  E8M0 byte s: 2^(s-127), 0xFF = NaN.
 *   - The MoE step ("Zyphra Inference Wave 2", sections "Speculative decoding." and
 *     "Quantization"): a step of T tokens (requests x speculative positions) reads each
 *     routed expert's weights once and applies them to every token routed to it; an
 *     MXFP4 expert runs two expert GEMMs and a combine.
 *   - Expert shapes of the pages' fused-MoE benchmarks (same page, Figure 10):
 *     H = 7168, E = 256 or 384, top-k = 8.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers owned by the caller, unless stated otherwise.  The
 *     library never allocates, never frees, never synchronizes, and keeps no state
 *     between calls.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream); buffers must stay alive until that work completes.
 *   - Tensors are dense row-major.  bf16 values are passed as their 16-bit patterns.
 *   - MXFP4 weight layout: a matrix with R output rows and reduction length K is
 *     codes [R][K/2] uint8 (element 2i in the low nibble of byte i) plus
 *     scales [R][K/32] uint8 (one E8M0 byte per 32 consecutive K values of one row).
 *   - Code and activation base pointers must be 16-byte aligned; scale pointers 8-byte
 *     aligned for mx_linear and 16-byte aligned for the MoE calls.
 *   - Return value: MX_OK (0) or a negative MX_ERR_* code.  All argument checks run on
 *     the host before anything is enqueued; a failed check enqueues nothing.  Device
 *     data (NaN, Inf) is not checked: NaN scales and NaN activations propagate.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef MX_API
#define MX_API __attribute__((visibility("default")))
#endif

enum mx_status {
  MX_OK = 0,
  MX_ERR_NULL = -1,      /* a required pointer is NULL */
  MX_ERR_SHAPE = -2,     /* a size is out of range or not a required multiple */
  MX_ERR_ALIGN = -3,     /* a pointer is not aligned as required */
  MX_ERR_WORKSPACE = -4, /* workspace missing or smaller than moe_mxfp4_workspace_size */
  MX_ERR_HIP = -5,       /* the HIP runtime reported an error while enqueueing */
  MX_ERR_SCRATCH = -6    /* moe_mxfp4_forward_noalloc: the call needs more than its static scratch */
};

/* Limits checked by every call. */
#define MX_MAX_TOKENS 256     /* T for the MoE calls */
#define MX_MAX_EXPERTS 1024   /* E */
#define MX_MAX_TOPK 32        /* top_k */

/* Library version (major * 10000 + minor * 100 + patch). */
MX_API int mx_version(void);

/* Static description of a status code; never NULL. */
MX_API const char* mx_status_string(int status);

/*
 * Dense MXFP4 linear layer: y[t,n] = bf16_rne( sum_k x[t,k] * w[n,k] ), products exact,
 * fp32 accumulation.  The MXFP4 projection the AMD megakernel blog ("Bringing Ultra-Fast,
 * Interactive LLM Inference to AMD Instinct MI355X GPUs", section "3. Low-Precision Data
 * Types") applies to attention projections and the LM head, here with bf16 activations;
 * decode reads every weight on every pass, so a call's weight bytes set a floor on its
 * time (same section).
 *   x       bf16 [T, K]
 *   w_codes uint8 [N, K/2], w_scales uint8 [N, K/32]
 *   y       bf16 [T, N]   (written)
 *   T >= 1, N >= 1, K >= 32 and K % 32 == 0.
 */
MX_API int mx_linear(const uint16_t* x, const uint8_t* w_codes, const uint8_t* w_scales, uint16_t* y, int64_t T,
              int64_t K, int64_t N, void* stream);

/*
 * MXFP8 activations (the AMD megakernel blog, "Bringing Ultra-Fast, Interactive LLM
 * Inference to AMD Instinct MI355X GPUs", section "3. Low-Precision Data Types": MXFP4
 * weights fed to the matrix instructions with MXFP8 activations).  The OCP MX format with
 * E4M3 elements (bias 7, largest 448, S.1111.111 = NaN): per block of 32 consecutive K
 * values of a row, the E8M0 scale is 2^(floor(log2 amax) - 8) clamped at 2^-127, and each
 * value divided by it is rounded to the nearest E4M3 value (ties to even), saturating at
 * +-448.  An all-zero block gets scale byte 0; a block with an Inf or NaN gets scale 0xFF
 * and codes 0x7F.
 *
 * mxfp8_quantize: the quantizer alone (bit-exact).
 *   x      bf16 [rows, K] (16-byte aligned), codes uint8 [rows, K] (8-byte aligned, written),
 *   scales uint8 [rows, K/32] (written).  rows >= 1, K >= 32, K % 32 == 0.
 */
MX_API int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Dense MXFP4 linear layer with MXFP8 activations: y[t,n] = bf16_rne( sum_k q(x)[t,k] w[n,k] ),
 * q(x) as mxfp8_quantize gives it (quantized inside the kernel; nothing is written back).
 * The products go to gfx950's scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) with the
 * weights' E2M1 codes and E8M0 scales as stored, accumulating in fp32.  That instruction does
 * not sum exactly: within groups of 8 products it drops bits more than about 14 binades
 * below the group's largest product, so |y - exact| stays below about 2^-10 of
 * sum_k |q(x) w| plus the bf16 rounding.  Arguments as for mx_linear.
 */
MX_API int mx_linear_a8(const uint16_t* x, const uint8_t* w_codes, const uint8_t* w_scales, uint16_t* y, int64_t T,
                        int64_t K, int64_t N, void* stream);

/*
 * Decode MXFP4 to bf16: out[r,k] = E2M1(code) * 2^(s-127), exact (NaN for s = 0xFF;
 * +-Inf where the value exceeds the bf16 range, i.e. only for s >= 253).
 *   w_codes uint8 [rows, K/2], w_scales uint8 [rows, K/32], out bf16 [rows, K].
 *   rows >= 1, K >= 32, K % 32 == 0.
 */
MX_API int mxfp4_dequantize(const uint8_t* w_codes, const uint8_t* w_scales, int64_t rows, int64_t K, uint16_t* out,
                     void* stream);

/*
 * Top-k routing with a softmax over the selected logits ("Zyphra Inference Wave 2",
 * Figure 10: top-8 routing over 256 and 384 experts; the AMD megakernel blog, section
 * "4. Data Locality", profiles top-k expert routing as a phase of its own).  The pages fix
 * neither tie order nor gate normalisation; the plainest reading is taken: for each token
 * t, the k largest logits[t,:] (ties go to the lower expert id), in descending-logit order;
 * gates[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) in fp32 (a softmax over the k
 * selected logits).
 *   logits fp32 [T, E] (must be finite), ids int32 [T, top_k], gates fp32 [T, top_k].
 *   1 <= T <= MX_MAX_TOKENS, 1 <= top_k <= min(E, MX_MAX_TOPK), E <= MX_MAX_EXPERTS.
 */
MX_API int moe_route_topk(const float* logits, int64_t T, int64_t E, int64_t top_k, int32_t* ids, float* gates,
                   void* stream);

/*
 * Counting sort of the T*top_k flat slots f = t*top_k + j by expert id ids[f]: experts
 * ascending, f ascending within an expert (bit-exact, deterministic).  "Zyphra Inference
 * Wave 2" (sections "Speculative decoding." and "Quantization") has a step read each
 * routed expert's weights once for all tokens routed to it; grouping the slots by expert
 * is what lets the expert GEMMs do that.  The stable order is the plainest reading.
 *   ids          int32 [T, top_k]; each row must hold top_k DISTINCT ids in [0, E)
 *                (as moe_route_topk produces); other ids are skipped.
 *   counts       int32 [E]       slots per expert
 *   offsets      int32 [E + 1]   exclusive prefix sum of counts
 *   sorted_slots int32 [T*top_k] flat slots in sorted order
 *   active       int32 [E]       experts with counts > 0, by row class descending (class 3:
 *                                counts >= 8; 2: 4-7; 1: 2-3; 0: 1), then by expert id
 *                                ascending; -1 after the last.  The expert GEMMs take their
 *                                work in this order, so the items with the most rows go first
 *   num_active   int32 [2]       the number of active experts, then the largest count
 *                                (the expert GEMMs use it to bound their row groups)
 */
MX_API int moe_sort_by_expert(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_slots, int32_t* active, int32_t* num_active,
                       void* stream);

/*
 * moe_route_topk followed by moe_sort_by_expert of its ids: one launch for T <= 16, two
 * beyond.  moe_mxfp4_forward runs it as its first stage beyond 32 tokens (and with shared
 * experts).  Up to 32 tokens it routes alone and its expert launch sorts where
 * moe_expert_gemms_from_ids pays; otherwise, up to 16 tokens its gate_up launch routes and
 * sorts in every workgroup, and from 17 to 32 it routes alone and gate_up sorts
 * (moe_gate_up_swiglu_from_ids).
 * That internal sort has the same counts, offsets and sorted slots, but keeps its active
 * list in ascending expert order and leaves the entries past the last one unwritten (its
 * down launch accepts any order).  Arguments, outputs and limits as for those two calls.
 */
MX_API int moe_route_sort(const float* logits, int64_t T, int64_t E, int64_t top_k, int32_t* ids, float* gates,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* active,
                          int32_t* num_active, void* stream);

/*
 * Stage hook: the gate_up GEMM with its SwiGLU epilogue, for every routed slot, from a
 * moe_sort_by_expert result (counts, offsets, sorted_slots, active, num_active).  For the
 * slot f = sorted_slots[p] routed to expert e (offsets[e] <= p < offsets[e+1]) of token
 * t = f / top_k:  h[p, n] = bf16_rne( silu(g_n) * u_n ) with g, u as in moe_mxfp4_forward.
 *   h  bf16 [T*top_k, I] (written; rows in sorted-slot order).  Other arguments and limits
 *   as for moe_mxfp4_forward, including the workspace, whose control words the call uses
 *   (to deal out its work) and leaves zero.  Each routed expert's gate_up weights are read
 *   once per 16 rows routed to it.
 */
MX_API int moe_gate_up_swiglu(const uint16_t* x, const uint8_t* w_gate_up, const uint8_t* s_gate_up,
                              const int32_t* counts, const int32_t* offsets, const int32_t* sorted_slots,
                              const int32_t* active, const int32_t* num_active, uint16_t* h, int64_t T, int64_t H,
                              int64_t I, int64_t E, int64_t top_k, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Stage hook: gate_up with SwiGLU straight from the routed ids (moe_route_topk's output),
 * sorting the slots inside the launch: every workgroup sorts the T*top_k slots itself, and
 * the launch also writes the sort (counts, offsets, sorted_slots, active, num_active), equal
 * to moe_sort_by_expert's on the same ids.  moe_mxfp4_forward runs it for 16 < T <= 32
 * without shared experts where moe_expert_gemms_from_ids does not apply (MXFP8 activations,
 * I % 1024 != 0, or too few items), in place of the sort launch: a token's routed expert GEMMs read
 * each routed expert's weights once ("Zyphra Inference Wave 2", section "Quantization"),
 * and a launch boundary costs microseconds at this size (the AMD megakernel blog, "What
 * Drives the Speedup", 1. Megakernels).
 *   ids     int32 [T, top_k], each in [0, E)
 *   outputs h as for moe_gate_up_swiglu (identical values), and the sort arrays as for
 *           moe_sort_by_expert (written).
 *   T <= 32, T*top_k <= 256, E <= 1024 (MX_ERR_SHAPE otherwise); other arguments, limits
 *   and the workspace as for moe_gate_up_swiglu.
 */
MX_API int moe_gate_up_swiglu_from_ids(const uint16_t* x, const int32_t* ids, const uint8_t* w_gate_up,
                                       const uint8_t* s_gate_up, int32_t* counts, int32_t* offsets,
                                       int32_t* sorted_slots, int32_t* active, int32_t* num_active, uint16_t* h,
                                       int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Stage hook: both expert GEMMs in one launch, straight from the routed ids, as
 * moe_mxfp4_forward runs them without shared experts for T <= 32 whenever the gate_up items
 * can be 3 or more per resident workgroup (min(T*top_k, E) * I / 64 >= 1536; from 6 tokens
 * at top-8 and I = 2048): every workgroup sorts
 * the T*top_k slots itself, streams its share of the gate_up items and then its share of the
 * down items, so that down work fills the end of the gate_up work ("Zyphra Inference Wave 2",
 * Kernel Results, for the two GEMMs of an MXFP4 expert; the AMD megakernel blog, "What Drives
 * the Speedup", 1. Megakernels, for removing the boundary between dependent kernels).
 *   ids  int32 [T, top_k], each row top_k distinct ids in [0, E) (moe_route_topk's output)
 *   h    bf16 [T*top_k, I] (written): h as moe_gate_up_swiglu writes it (identical values;
 *        rows in sorted-slot order).  It is also the hand-off between the two GEMMs: the
 *        down items recognise rows that gate_up has not written yet by the pattern 0xFFFF
 *        in every element (a NaN that SwiGLU produces only from NaN inputs; if it does, the
 *        launch only waits longer), so h must hold 0xFFFF throughout when the launch starts.
 *   h_prefilled  0: the call first fills h with 0xFFFF (one more launch, as moe_mxfp4_forward
 *        does inside its routing launch); 1: the caller has done so on this stream.  With 1
 *        and any other content in h the results are undefined.
 *   d    fp32 [T*top_k, H] (written): d[t*top_k + j, n] = sum_i h[p(t,j), i] * Wd[e][n, i]
 *        (fp32), the slot's down output before its gate; moe_combine makes y from it.
 * The launch's workgroups may wait for one another: a down item that finds an unwritten h
 * row waits until every workgroup has finished its gate_up items.  The grid is sized to what
 * the device holds at once, so all of them run; a wait that outlasts any layer by far gives
 * up, leaves d undefined and sets the int32 at byte offset 8 of the workspace to 1 (sticky,
 * as for moe_mxfp4_forward_persistent).  T <= 32, T*top_k <= 256, E <= 1024 and
 * I % 1024 == 0 (MX_ERR_SHAPE otherwise); with fewer items than that bound the results are
 * the same, only slower than separate launches.  Other arguments, limits and the workspace
 * as for moe_gate_up_swiglu.
 */
MX_API int moe_expert_gemms_from_ids(const uint16_t* x, const int32_t* ids, const uint8_t* w_gate_up,
                                     const uint8_t* s_gate_up, const uint8_t* w_down, const uint8_t* s_down,
                                     uint16_t* h, int h_prefilled, float* d, int64_t T, int64_t H, int64_t I,
                                     int64_t E, int64_t top_k, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Stage hook: the gate-weighted combine, y[t, n] = bf16_rne( sum_j gates[t, j] * d[t*top_k + j, n] )
 * in fp32, j ascending (the last step of moe_mxfp4_forward; "Zyphra Inference Wave 2",
 * section "Quantization": the routed experts' outputs are combined with their router weights).
 *   d      fp32 [T*top_k, H]   gates  fp32 [T, top_k]   y  bf16 [T, H] (written)
 *   1 <= T <= MX_MAX_TOKENS, 1 <= top_k <= MX_MAX_TOPK, 4 <= H <= 65536, H % 4 == 0.
 */
MX_API int moe_combine(const float* d, const float* gates, uint16_t* y, int64_t T, int64_t H, int64_t top_k,
                       void* stream);

/*
 * Stage hook: the down GEMM with the gate-weighted combine, from gate_up's h and the sort
 * result:  y[t, n] = bf16_rne( sum_j gates[t, j] * sum_i h[p(t,j), i] * Wd[e][n, i] ), where
 * p(t, j) is the sorted position of slot t*top_k + j.  Uses `workspace` (at least
 * moe_mxfp4_workspace_size bytes, 256-byte aligned, control words zero) as scratch.
 */
MX_API int moe_down_combine(const uint16_t* h, const float* gates, const uint8_t* w_down, const uint8_t* s_down,
                            const int32_t* counts, const int32_t* offsets, const int32_t* sorted_slots,
                            const int32_t* active, const int32_t* num_active, uint16_t* y, int64_t T, int64_t H,
                            int64_t I, int64_t E, int64_t top_k, void* workspace, size_t workspace_bytes,
                            void* stream);

/* The first MX_WORKSPACE_CTL_BYTES bytes of a MoE workspace are control words: counters
 * through which the workgroups of a launch deal out their work.  They must be zero before
 * the workspace is first used, and every call leaves them zero again. */
#define MX_WORKSPACE_CTL_BYTES 57344

/* Bytes of device workspace moe_mxfp4_forward needs for these sizes. */
MX_API size_t moe_mxfp4_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k);

/*
 * MoE expert layer with MXFP4 weights and SwiGLU experts:
 *   route:   ids, gates = moe_route_topk(router_logits, top_k)
 *   gate_up: for slot (t, j) with expert e = ids[t,j]:
 *              g_n = sum_c x[t,c] Wgu[e][n,c],  u_n = sum_c x[t,c] Wgu[e][I+n,c]    (fp32)
 *              h_n = bf16_rne( silu(g_n) * u_n ),  silu(g) = g / (1 + exp(-g))    n < I
 *   down:    d_n = sum_i h_i Wd[e][n,i]                                          (fp32)
 *   combine: y[t,n] = bf16_rne( sum_j gates[t,j] * d_{t,j,n} )                    (fp32)
 * Each routed expert's weights are read from HBM once per 16 tokens routed to it (once per
 * call for T <= 16, where no expert has more than 16 rows); experts no token routes to are
 * not read.  Up to 32 tokens (from 17 with shared experts), where the gate_up items can be
 * 3 or more per resident workgroup (min(T * slots per token, experts) * I / 64 >= 1536 with
 * I % 1024 == 0; from 6 tokens at top-8), both expert GEMMs run in one launch whose
 * workgroups may wait for one another (moe_expert_gemms_from_ids).  Such a wait is bounded: if one ever gave up, y is
 * undefined and the int32 at byte offset 8 of the workspace reads 1 (sticky, as for
 * moe_mxfp4_forward_persistent).
 *   x             bf16 [T, H]
 *   router_logits fp32 [T, E] (finite)
 *   w_gate_up     uint8 [E, 2I, H/2]  (rows [0, I) gate, rows [I, 2I) up)
 *   s_gate_up     uint8 [E, 2I, H/32]
 *   w_down        uint8 [E, H, I/2]
 *   s_down        uint8 [E, H, I/32]
 *   y             bf16 [T, H]   (written)
 *   workspace     device buffer of at least moe_mxfp4_workspace_size(T, H, I, E, top_k)
 *                 bytes, 256-byte aligned.  Its first MX_WORKSPACE_CTL_BYTES must be zero
 *                 before its first use (every call leaves them zero); the rest needs no
 *                 initialization and is overwritten.  Calls that share a workspace must
 *                 not overlap in time (two streams need two workspaces).
 *   1 <= T <= MX_MAX_TOKENS; 1 <= top_k <= min(E, MX_MAX_TOPK); E <= MX_MAX_EXPERTS;
 *   1024 <= H <= 65536 and H % 1024 == 0 (the gate_up GEMM stages its scales 1024 K
 *   values at a time); 256 <= I <= 65536 and I % 256 == 0 (the down GEMM streams 256 K
 *   values per segment; I = 256 is one tensor-parallel eighth of an expert of 2048).
 *   MX_ERR_SHAPE otherwise.
 */
MX_API int moe_mxfp4_forward(const uint16_t* x, const float* router_logits, int64_t top_k, const uint8_t* w_gate_up,
                      const uint8_t* s_gate_up, const uint8_t* w_down, const uint8_t* s_down, uint16_t* y,
                      int64_t T, int64_t H, int64_t I, int64_t E, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation: moe_mxfp4_forward without a workspace
 * argument.  Its scratch (the sort, h and the fp32 down outputs, as in the workspace) is a
 * static device array of MX_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends; the call allocates nothing.  Results are bit for bit those of
 * moe_mxfp4_forward.  Arguments and limits as for moe_mxfp4_forward, and:
 *   - MX_ERR_SCRATCH when moe_mxfp4_workspace_size(T, H, I, E, top_k) exceeds
 *     MX_NOALLOC_SCRATCH_BYTES (it holds T = 128 tokens, top-8, H = 7168, I = 2048,
 *     E = 384; not T * top_k much beyond 1024 slots at H = 7168);
 *   - every call on one GPU shares that GPU's array: calls that overlap in time on one
 *     GPU (two streams, or two host threads) race and give undefined results;
 *   - the first call on a GPU also enqueues, on `stream`, a kernel that zeroes the
 *     array's control words.
 */
#define MX_NOALLOC_SCRATCH_BYTES (40 << 20)
MX_API int moe_mxfp4_forward_noalloc(const uint16_t* x, const float* router_logits, int64_t top_k,
                                     const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                                     const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                                     void* stream);

/*
 * The MoE layer with shared experts: every token reads its top_k routed experts (of E,
 * chosen from router_logits [T, E]) and the n_shared shared experts, whose outputs add to
 * the gate-weighted routed ones with weight 1 ("Zyphra Inference Wave 2", section
 * "Quantization": a token uses its top-K routed experts plus the layer's shared experts;
 * GLM-5.3 has 8 routed and 1 shared of 257).
 *   y[t,n] = bf16_rne( sum_{j<top_k} gates[t,j] d_{t,j,n} + sum_{s<n_shared} d^S_{t,s,n} )
 * summed in fp32 with j ascending and then s ascending; d^S is expert E + s's SwiGLU output.
 * The weight tensors hold E + n_shared experts: [E + n_shared, 2I, H/2] etc., the shared
 * ones last.  The workspace must hold moe_mxfp4_workspace_size(T, H, I, E + n_shared,
 * top_k + n_shared) bytes.  0 <= n_shared; E + n_shared <= MX_MAX_EXPERTS;
 * top_k + n_shared <= MX_MAX_TOPK; other arguments as for moe_mxfp4_forward.
 */
MX_API int moe_mxfp4_forward_shared(const uint16_t* x, const float* router_logits, int64_t top_k, int64_t n_shared,
                                    const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                                    const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The MoE layer (with n_shared shared experts, as moe_mxfp4_forward_shared) with MXFP8
 * activations: x is quantized (as mxfp8_quantize) before the gate_up GEMM and the bf16 h
 * before the down GEMM, inside the GEMM kernels as they stage them; both GEMMs run on the
 * scaled MFMA as mx_linear_a8 does ("Zyphra Inference Wave 2", section "Quantization": an
 * MXFP4 expert quantizes the activations, runs the two expert GEMMs and combines the
 * results).  Routing, sort, SwiGLU with its bf16 rounding, and the fp32 combine are those
 * of moe_mxfp4_forward.  Arguments, workspace and limits as for moe_mxfp4_forward_shared.
 */
MX_API int moe_mxfp4_forward_a8(const uint16_t* x, const float* router_logits, int64_t top_k, int64_t n_shared,
                                const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                                const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same layer as moe_mxfp4_forward, as ONE persistent launch (the megakernels of the
 * Lithos page, "Specialization unlocks engine performance", and of the AMD megakernel
 * blog, "What Drives the Speedup": workgroups hand data to one another through memory
 * instead of kernel boundaries).  Every workgroup routes and sorts all tokens itself; the
 * gate_up and down phases hand h over through device counters in the workspace, and the
 * workgroup that completes a column tile's down outputs combines it.  Results are bit-for-
 * bit those of moe_mxfp4_forward.  Arguments as for moe_mxfp4_forward, plus:
 *   - T <= 16 and T * top_k <= 128 (MX_ERR_SHAPE otherwise);
 *   - no other work may occupy the GPU's compute units while it runs: its workgroups
 *     wait for one another.  A wait that outlasts any layer by far gives up, leaving y
 *     undefined and the int32 word at byte offset 8 of the workspace set to 1 (sticky;
 *     the caller clears it).
 * On MI355X it is not faster than moe_mxfp4_forward: kernel boundaries inside a HIP graph
 * cost about a microsecond, and its in-kernel hand-offs cost as much.
 */
MX_API int moe_mxfp4_forward_persistent(const uint16_t* x, const float* router_logits, int64_t top_k,
                                        const uint8_t* w_gate_up, const uint8_t* s_gate_up, const uint8_t* w_down,
                                        const uint8_t* s_down, uint16_t* y, int64_t T, int64_t H, int64_t I,
                                        int64_t E, void* workspace, size_t workspace_bytes, void* stream);

/*
 * HBM reference kernels (measurement utilities, not steps of the layer).  "Zyphra
 * Inference Wave 2" (footnote 6 of its roofline discussion) measures MI355X's HBM with a
 * plain copy kernel, 6.07 of the nominal 8 TB/s; these give the same kind of yardstick on
 * the GPU at hand.  Both stream the buffer once in 16-byte nontemporal pieces over the
 * whole device.
 *
 * mx_hbm_read: reads `bytes` bytes at src and XORs them into xor_out: word c (c < 4)
 *   receives the XOR of 32-bit word c of every 16-byte piece.  xor_out is 4 uint32 device
 *   words that the CALLER zeroes before the call (the kernel XORs into them).
 * mx_hbm_copy: copies `bytes` bytes from src to dst (the ranges must not overlap).
 *   bytes >= 16 and bytes % 16 == 0; src and dst 16-byte aligned, xor_out 4-byte aligned.
 */
MX_API int mx_hbm_read(const void* src, size_t bytes, uint32_t* xor_out, void* stream);
MX_API int mx_hbm_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
