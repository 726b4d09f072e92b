// Host-side internals shared by the C-ABI translation units (not part of the public API).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mxmoe.h"

namespace mx {

// Control words at the start of the workspace (int32 indices), zero between calls: the
// expert GEMMs' claim counters and the single-launch layer's counters and flags.  Words
// that many workgroups update sit on lines of their own, 512 bytes apart, so that their
// traffic spreads over memory channels instead of queueing on one.
constexpr int CTL_GU_DONE = 0;      // single launch: gate_up items whose h rows are written
constexpr int CTL_EXIT = 1;         // single launch: workgroups that have finished
constexpr int CTL_ERR = 2;          // single launch: set to 1 by a wait that gave up (sticky)
constexpr int CTL_CLAIM_GU = 256;   // gate_up claim classes (16 x 128 words)
constexpr int CTL_CLAIM_DN = 2304;  // down claim classes (16 x 128 words)
constexpr int CTL_QUAD0 = 4352;     // single launch: per down column quad, items finished
constexpr int CTL_MAX_QUADS = 1024;
// Replicas of the single launch's "every h row written" flag, one 512-byte line apart.
constexpr int CTL_READY0 = 6144;
constexpr int CTL_READY_REPLICAS = 64;
constexpr int CTL_READY_STRIDE = 128;
static_assert(CTL_CLAIM_DN - CTL_CLAIM_GU >= 16 * 128 && CTL_QUAD0 - CTL_CLAIM_DN >= 16 * 128, "claim classes");
static_assert(CTL_QUAD0 + CTL_MAX_QUADS <= CTL_READY0, "control block layout");
static_assert((CTL_READY0 + CTL_READY_REPLICAS * CTL_READY_STRIDE) * 4 == MX_WORKSPACE_CTL_BYTES, "control block size");

// Largest T the single-launch layer takes.
constexpr int MX_FUSED_MAX_TOKENS = 16;

// Layout of the moe_mxfp4_forward workspace, carved in this order, 256-byte aligned.
struct MoeWorkspace {
  int32_t* ctl;           // [MX_WORKSPACE_CTL_BYTES / 4] control words
  int32_t* ids;           // [T*k]
  float* gates;           // [T*k]
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* sorted_slots;  // [T*k]
  int32_t* active;        // [E]
  int32_t* num_active;    // [2]: active experts, largest count
  uint16_t* h;            // [T*k, I] bf16, rows in sorted-slot order
  float* dpart;           // [T*k, H] fp32 down outputs, rows by flat slot
  size_t bytes;
};

MoeWorkspace moe_workspace_carve(void* base, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k);

// The outputs of the token->expert sort, as the expert GEMM kernels read them.
struct SortView {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted_slots;
  const int32_t* active;
  const int32_t* num_active;
};

inline int hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_cu_count();

// Kernel launchers (enqueue only; arguments already validated).
int launch_mx_linear(const uint16_t* x, const uint8_t* w, const uint8_t* s, uint16_t* y, int T, int K, int N,
                     hipStream_t stream);
int launch_dequant(const uint8_t* w, const uint8_t* s, int64_t rows, int64_t K, uint16_t* out, hipStream_t stream);
// MXFP8 activations: the dense layer with x quantized in the lanes, and the quantizer alone
int launch_mx_linear_a8(const uint16_t* x, const uint8_t* w, const uint8_t* s, uint16_t* y, int T, int K, int N,
                        hipStream_t stream);
int launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                          hipStream_t stream);
// ns: shared experts E .. E + ns - 1, routed by every token with gate 1 after its k routed
// slots (ids and gates are [T, k + ns]; the sort then runs over E + ns experts)
// fill: optionally, fill_bytes (a multiple of 16) of device memory set to all ones in the same launch
int launch_route(const float* logits, int T, int E, int k, int ns, int32_t* ids, float* gates, hipStream_t stream,
                 void* fill = nullptr, size_t fill_bytes = 0);
// bytes (a multiple of 16) of device memory set to all ones
int launch_fill_ones(void* p, size_t bytes, hipStream_t stream);
int launch_sort(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                int32_t* active, int32_t* num_active, hipStream_t stream);
// route + sort: one single-workgroup launch up to 16 tokens, the route and sort launches
// beyond (fill: as launch_route's, beyond 16 tokens only)
int launch_route_sort(const float* logits, int T, int E, int k, int ns, int32_t* ids, float* gates, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_slots, int32_t* active, int32_t* num_active,
                      hipStream_t stream, void* fill = nullptr, size_t fill_bytes = 0);
// ctl: the workspace's control words (the expert GEMMs claim their units there);
// act8: MXFP8 activations (x, resp. h, quantized as they are staged) and the scaled MFMA
int launch_gate_up(const uint16_t* x, const uint8_t* wgu, const uint8_t* sgu, const SortView& sv, uint16_t* h,
                   int32_t* ctl, int T, int H, int I, int E, int k, bool act8, hipStream_t stream);
// *combined is set when the down launch also wrote y (small T); otherwise the caller
// launches the combine
int launch_down(const uint16_t* h, const float* gates, const uint8_t* wd, const uint8_t* sd, const SortView& sv,
                float* dpart, uint16_t* y, bool* combined, int32_t* ctl, int T, int H, int I, int E, int k, bool act8,
                hipStream_t stream);
int launch_combine(const float* dpart, const float* gates, uint16_t* y, int T, int H, int k, hipStream_t stream);
// gate_up for 16 < T <= 32: sorts the routed ids (moe_route_kernel's output) in every
// workgroup and writes the sort for a down launch (the stage entry point, and the forward
// with MXFP8 activations or where the single expert launch below does not apply).
bool gate_up_sorted_fits(int T, int E, int k, int H, int I);
int launch_gate_up_sorted(const uint16_t* x, const int32_t* ids, const uint8_t* wgu, const uint8_t* sgu, uint16_t* h,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* active,
                          int32_t* num_active, int32_t* ctl, int T, int H, int I, int E, int k, bool act8,
                          hipStream_t stream);
// Both expert GEMMs in one launch (bf16 activations, T <= 32): every workgroup sorts the
// routed ids, streams its gate_up items, then its down items.  h must hold 0xFFFF in every
// element when it starts (launch_route's fill); the combine follows.  The forward uses it
// where experts_sorted_pays.
bool experts_sorted_fits(int T, int E, int k, int H, int I);
bool experts_sorted_pays(int T, int E, int k, int I);
// The same launch from a sort in global memory (moe_sort_by_expert's outputs).  The forward
// uses it up to EXPERTS_MAX_T tokens: beyond, the down phase at gate_up's occupancy (2
// workgroups per CU instead of 3) costs more than the ends of the launches it saves
// (measured with the route and sort launches before it: T = 64 816.5 us per layer either
// way, T = 128 with E = 384 1,330.5 -> 1,340.6; shared expert at T = 32 405.6 -> 398.4).
constexpr int EXPERTS_MAX_T = 32;
bool experts_fits(int H, int I);
int launch_experts(const uint16_t* x, const SortView& sv, const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd,
                   const uint8_t* sd, uint16_t* h, float* dpart, int32_t* ctl, int H, int I, int k, bool act8,
                   hipStream_t stream);
int launch_experts_sorted(const uint16_t* x, const int32_t* ids, const uint8_t* wgu, const uint8_t* sgu,
                          const uint8_t* wd, const uint8_t* sd, uint16_t* h, float* dpart, int32_t* ctl, int T, int H,
                          int I, int E, int k, bool act8, hipStream_t stream);
// The forward's gate_up for small T with the routing and sort done in every workgroup (no
// route + sort launch before it); it also writes the sort outputs and gates for the down
// launch.  gate_up_routed_fits says when it applies (no shared experts); act8: MXFP8
// activations, as launch_gate_up.
bool gate_up_routed_fits(int T, int E, int k, int H, int I);
int launch_gate_up_routed(const uint16_t* x, const float* logits, const uint8_t* wgu, const uint8_t* sgu, uint16_t* h,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* active,
                          int32_t* num_active, float* gates, int T, int H, int I, int E, int k, bool act8,
                          hipStream_t stream);
// The whole layer as one persistent launch (small T); fused_layer_fits says when it applies.
bool fused_layer_fits(int T, int E, int k, int H, int I);
int launch_moe_fused(const uint16_t* x, const float* logits, const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd,
                     const uint8_t* sd, uint16_t* hbuf, float* dpart, uint16_t* y, int32_t* ctl, int T, int H, int I,
                     int E, int k, hipStream_t stream);

}  // namespace mx
