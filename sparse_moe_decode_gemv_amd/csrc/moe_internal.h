// Internal launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Optional per-kernel timing for the measurement entry point: the i-th
// kernel a call launches records start[i] when it starts executing and
// stop[i] when it ends (hipExtLaunchKernel); kernels past n launch plainly.
struct KernelTimer {
  hipEvent_t* start;
  hipEvent_t* stop;
  int n;     // event pairs available
  int used;  // kernels launched so far
};

inline bool timer_slot(KernelTimer* tm, hipEvent_t* a, hipEvent_t* b) {
  if (!tm) return false;
  const int i = tm->used++;
  if (i >= tm->n) return false;
  *a = tm->start[i];
  *b = tm->stop[i];
  return true;
}

}  // namespace moe

// Launch K (parenthesised when it has template arguments) plainly, or with
// the timer's next event pair.
#define MOE_LAUNCH(TM, K, G, B, LDS, S, ...)                                    \
  do {                                                                          \
    hipEvent_t moe_e0_ = nullptr, moe_e1_ = nullptr;                            \
    if (::moe::timer_slot((TM), &moe_e0_, &moe_e1_))                             \
      hipExtLaunchKernelGGL(K, G, B, LDS, S, moe_e0_, moe_e1_, 0u, __VA_ARGS__); \
    else                                                                        \
      hipLaunchKernelGGL(K, G, B, LDS, S, __VA_ARGS__);                          \
  } while (0)

namespace moe {

// Lane mapping of a row-streaming GEMV over MXFP4 rows of `nblk` 32-element
// blocks: `lanes` lanes share a row and each handles `bpl` blocks strided by
// `lanes`, so one wave covers 64/lanes rows per load instruction.
struct RowMap {
  int lanes;
  int bpl;
};

// gate/up rows (reduction over H): a half wave (32 lanes) per matrix.
inline RowMap gateup_map(int H) {
  int nb = H / 32, g = 32;
  while (nb % g) g >>= 1;
  return {g, nb / g};
}
constexpr int kMaxBplGateUp = 8;
constexpr int kMaxFfn = 8192;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxTokens = 64;

// ---- T = 1 path ------------------------------------------------------------

struct LayerT1 {
  int H, E, k, F, S;
  int Fs;  // shared expert's FFN width (equal to F unless act_sh is set)
  // inputs
  const uint16_t* x;         // bf16 [H]: layer input, or h when gamma != null
  const uint16_t* gamma;     // RMSNorm gain (stack) or null
  float eps;
  const uint16_t* residual;  // bf16 [H] or null
  uint16_t* out;             // bf16 [H]
  uint16_t* trace;           // optional copy of out
  // weights
  const uint16_t* router_w;
  const uint8_t *g_codes, *g_scales, *u_codes, *u_scales, *d_codes, *d_scales;
  const uint8_t *sg_codes, *sg_scales, *su_codes, *su_scales, *sd_codes, *sd_scales;
  // workspace
  float* logits;       // [E]
  int32_t* idx;        // [k]
  float* wts;          // [k]
  uint16_t* act_hl;    // bf16 [2][k + S][F]: gated activations split as
                       // leading part + remainder (routed slots, then shared)
  uint16_t* act_sh;    // shared expert of another width (Fs != F): its own
                       // bf16 [2][Fs], and act_hl holds the k routed slots only
  float* part_sh;      // [H]: the shared expert's down rows (Fs != F)
  float* part;         // [k + S][H]: weighted down-projection rows per slot
  // down kernels' combine: add part_in[row] after the slots, or write the
  // unrounded sum to part_out[row] instead of the output (Fs != F passes)
  const float* part_in;
  float* part_out;
  uint32_t* counters;  // per row chunk, zero between calls (workspace head)
  uint16_t* xn;        // [H] normalised input (stack)
  // optional user outputs
  float* logits_out;
  int32_t* idx_out;
  float* w_out;
  KernelTimer* timer;  // host-side, measurement entry point only (else null)
};

// K1a router, K2 top-k when idx is null and gate/up (shared expert first
// when with_shared; fp32 activations into act, or split bf16 into L.act_hl
// when act is null), K3 down of every slot (the shared expert last) +
// combine; launch_topk_t1 is the stand-alone top-k of the router entry point.
hipError_t launch_router_t1(const LayerT1& L, hipStream_t s);
hipError_t launch_topk_t1(const LayerT1& L, hipStream_t s);
hipError_t launch_gateup_t1(const LayerT1& L, const uint16_t* x, const int32_t* idx,
                            float* act, bool with_shared, hipStream_t s);
hipError_t launch_down_combine_t1(const LayerT1& L, hipStream_t s);
// The whole single-token layer: router, gate/up with the selection, down +
// combine.
hipError_t launch_layer_t1(LayerT1& L, hipStream_t s);

// ---- 2 <= T <= 64 path ------------------------------------------------------

struct LayerTB {
  int T, H, E, k, F, S;
  int KS;                     // router K splits (H % (128 KS) == 0)
  // inputs
  const uint16_t* x;          // bf16 [T][H] MoE input
  const uint16_t* residual;   // bf16 [T][H] or null
  uint16_t* out;              // bf16 [T][H]
  uint16_t* trace;            // optional copy of out
  // weights
  const uint16_t* router_w;
  const uint8_t *g_codes, *g_scales, *u_codes, *u_scales, *d_codes, *d_scales;
  const uint8_t *sg_codes, *sg_scales, *su_codes, *su_scales, *sd_codes, *sd_scales;
  // workspace
  float* part;                // [KS][T][E] partial router logits
  int32_t* idx;               // [T][k]
  float* wts;                 // [T][k]
  int32_t* ginfo;             // [0]: number of groups (active experts + shared);
                              // [1], [2]: passes of the routed groups, of all groups
  int32_t* g_expert;          // [E + 1] expert of each group (E: the shared expert)
  int32_t* g_start;           // [E + 1] first sorted position of the group
  int32_t* g_count;           // [E + 1] pairs in the group
  int32_t* order;             // [T k + T] pair id at each sorted position
  int32_t* pos_of;            // [T k] sorted position of pair t k + j
  // the groups cut into passes of at most 16 pairs, in group order (pass p
  // of group g holds its pairs 16 p .. 16 p + 15); null: not written
  int32_t* pass_group;        // [passes] group of each pass
  int32_t* pass_n0;           // [passes] first pair of the pass within its group
  uint16_t* act_hi;           // [T k + T][F] bf16 leading part of silu(g) u
  uint16_t* act_lo;           // [T k + T][F] bf16 remainder
  float* y;                   // [T k + T][H] expert outputs per sorted pair
  // shared expert of another width (Fs != F): its activations get planes of
  // their own, [T][Fs] (else null), and its gate/up and down run as passes
  // of their own
  uint16_t *act_sh_hi, *act_sh_lo;
  int Fs;
  // groups one grouped gate/up or down launch covers: 0 every group, 1 the
  // routed ones (the shared group, last when present, is left out), 2 the
  // shared group alone; act_hi/act_lo row r holds sorted position pos0 + r
  int gmode, pos0;
  // optional user outputs
  float* logits_out;          // [T][E]
  int32_t* idx_out;           // [T][k]
  float* w_out;               // [T][k]
  int32_t* offsets_out;       // [E + 1] grouping offsets
  int32_t* pairs_out;         // [T k] pair ids sorted by expert
  KernelTimer* timer;         // host-side, measurement entry point only (else null)
};

// Router K splits for hidden size H: the largest KS <= 16 with H % (128 KS) == 0.
inline int router_splits(int H) {
  int ks = 16;
  while (ks > 1 && H % (128 * ks)) --ks;
  return ks;
}

hipError_t launch_router_tb(const LayerTB& L, hipStream_t s);
hipError_t launch_topk_tb(const LayerTB& L, hipStream_t s);
hipError_t launch_group_tb(const LayerTB& L, hipStream_t s);
hipError_t launch_gateup_tb(const LayerTB& L, hipStream_t s);
hipError_t launch_down_tb(const LayerTB& L, hipStream_t s);
hipError_t launch_combine_tb(const LayerTB& L, hipStream_t s);
hipError_t launch_rmsnorm_tb(const uint16_t* h, const uint16_t* gamma, float eps, int T, int H,
                             uint16_t* xn, hipStream_t s);

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace moe
