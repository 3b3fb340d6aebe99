/*
 * moe.h - C ABI of libmoe_decode.so, an MI355X (gfx950) implementation of
 * the memory-bound decode step of a sparse Mixture-of-Experts layer.
 *
 * The step follows the Kimi K3 decode pages: each token picks 16 of 896
 * routed experts (page "英伟达用1.2万行CuTe DSL Megakernel，如何优化Kimi K3？",
 * section "一个工程师、1.2万行代码、AI辅助开发"; tmtpost page, section "现象"),
 * expert weights are MXFP4 (tmtpost page, section "现象"), a shared expert is
 * always active beside the routed ones (page "AI手搓1.2万行代码榨干GB300!…",
 * section 02; smzdm page, section "四步改造"), and the layer ends with the
 * residual add (smzdm page, section "慢的根源").  The fast path is limited to
 * small batches (up to 64 tokens), as the pages' latency path is (page
 * "AI手搓1.2万行代码榨干GB300!…", section 03).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers named in a struct or argument are DEVICE pointers unless
 *    the comment says "host".  The caller owns every buffer; the library
 *    never allocates, frees or synchronises and keeps no global state.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *    Calls are safe to capture into a HIP graph: no host read-back, no
 *    allocation, no memset nodes.
 *  - Every argument is validated on the host before anything is enqueued;
 *    on error nothing is enqueued and a negative moe_status is returned.
 *    Kernel faults surface at the caller's next synchronisation.
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - MXFP4 matrix M[R][C] (OCP Microscaling v1.0: E2M1 elements, one E8M0
 *    scale 2^(b-127) per 32 consecutive elements of a row, b = 0xFF is NaN):
 *      codes  uint8 [R][C/2]  element 2i in bits 3:0 of byte i, 2i+1 in 7:4
 *      scales uint8 [R][C/32]
 *    codes must be 16-byte aligned, scales 4-byte aligned (kernels read
 *    scales as aligned 32-bit words; rows are a multiple of 4 bytes long
 *    for every accepted shape).  The reduction dimension is the row:
 *    C = H for gate/up, C = F for down.
 *  - Workspace: `ws` is a 16-byte aligned device buffer of at least
 *    moe_workspace_size() bytes.  Its first MOE_WS_COUNTER_BYTES bytes are
 *    reserved for counters and must be zero before the first call
 *    (moe_workspace_init() zero-fills the whole buffer); calls leave them at
 *    zero.  The rest is scratch that each call writes before it reads it, so
 *    one workspace serves any number of calls on one stream.  Calls that
 *    overlap in time (different streams) need different workspaces.
 *  - Results depend on the inputs only: a call repeated on the same inputs
 *    (eager or replayed from a graph) gives identical bits.  Sums run in a
 *    fixed order and no floating-point atomics are used.
 *  - Expert indices read from device memory (topk_idx arguments, or the
 *    router's own output) are clamped to [0, E) before addressing weights;
 *    an out-of-range index gives unspecified values for that slot, never an
 *    out-of-bounds access.
 *
 * Limits (MOE_ERR_UNSUPPORTED beyond them)
 *    0 <= T <= 64 tokens (T = 0 is a no-op returning MOE_OK)
 *    H % 256 == 0, 256 <= H <= 8192, and (H/256)/gcd(H/256, 4) <= 8
 *      (every multiple of 256 up to 2048, and e.g. 3072, 4096, 7168, 8192)
 *    F % 128 == 0, 128 <= F <= 8192
 *    1 <= k <= min(E, 32), 1 <= E <= 1024
 *    n_shared in {0, 1}; with a shared expert, shared_ffn % 128 == 0 and
 *      128 <= shared_ffn <= 8192 (it may differ from ffn at any T)
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_WS_COUNTER_BYTES 256
#define MOE_MAX_LAYER_KERNELS 8    /* kernels one moe_decode_layer call launches, at most */
#define MOE_STREAM_SINK_WORDS 4096 /* uint32 words moe_stream_read may write to `sink` */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20) /* scratch of moe_decode_layer_noalloc, per GPU */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad value, aliasing */
  MOE_ERR_UNSUPPORTED = -2, /* well-formed but outside the limits above */
  MOE_ERR_WORKSPACE = -3,   /* ws null or smaller than moe_workspace_size() */
  MOE_ERR_HIP = -4          /* a HIP launch failed */
} moe_status;

typedef struct {
  int32_t hidden;     /* H */
  int32_t n_experts;  /* E, routed experts */
  int32_t top_k;      /* k, routed experts used per token */
  int32_t ffn;        /* F, width of each routed expert */
  int32_t n_shared;   /* S in {0, 1} */
  int32_t shared_ffn; /* Fs, the shared expert's FFN width (when S = 1) */
} moe_shape;

typedef struct {
  const uint8_t* codes;  /* [R][C/2], 16-byte aligned */
  const uint8_t* scales; /* [R][C/32], 4-byte aligned */
} moe_mx_mat;

typedef struct {
  const uint16_t* router_w; /* bf16 [E][H], 16-byte aligned */
  moe_mx_mat gate;          /* routed, expert-major [E][F][H] */
  moe_mx_mat up;            /* routed, expert-major [E][F][H] */
  moe_mx_mat down;          /* routed, expert-major [E][H][F] */
  moe_mx_mat s_gate;        /* shared [Fs][H]; ignored when n_shared == 0 */
  moe_mx_mat s_up;          /* shared [Fs][H] */
  moe_mx_mat s_down;        /* shared [H][Fs] */
} moe_layer_weights;

/* Workspace bytes needed for calls with up to `max_tokens` tokens.
 * Returns MOE_OK and writes *bytes (host pointer). */
int moe_workspace_size(const moe_shape* shape, int32_t max_tokens, size_t* bytes);

/* Zero-fill a workspace (a fill kernel, not a memset node). */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Router GEMV and top-k selection.
 *   l[t][e] = sum_h x[t][h] * Wr[e][h]  (fp32 accumulation of exact bf16
 *   products); the k largest logits per token ordered by (logit desc,
 *   expert index asc), -0 treated as +0; weights = softmax over those k.
 * x        bf16 [T][H], 16-byte aligned
 * router_w bf16 [E][H], 16-byte aligned
 * topk_idx int32 [T][k] out;  topk_w fp32 [T][k] out (sums to 1 per token)
 * logits   fp32 [T][E] out, may be NULL */
int moe_router_topk(const moe_shape* shape, const uint16_t* x, const uint16_t* router_w,
                    int32_t n_tokens, int32_t* topk_idx, float* topk_w, float* logits,
                    void* ws, size_t ws_bytes, void* stream);

/* Gate/up projections of the selected experts with SiLU gating:
 *   act[t][j][f] = silu(G_e x_t)[f] * (U_e x_t)[f],  e = topk_idx[t][j]
 * computed in fp32 from the MXFP4 weights (dequantised in the dot product).
 * topk_idx int32 [T][k] (device; clamped to [0, E) before addressing),
 * act fp32 [T][k][F] out.  T must be 0 or 1 (T > 1: MOE_ERR_UNSUPPORTED;
 * the batched layer runs its own grouped gate/up).
 * This is the layer's dominant HBM stream, exported for measurement. */
int moe_expert_gateup(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                      const int32_t* topk_idx, int32_t n_tokens, float* act,
                      void* ws, size_t ws_bytes, void* stream);

/* One MoE decode layer:
 *   out[t] = residual[t] + sum_j topk_w[t][j] * y_{idx[t][j]}(x_t) + y_shared(x_t)
 *   y_e(x) = D_e (silu(G_e x) * (U_e x)), shared expert weight 1
 * rounded once to bf16 (nearest even).  T = 1 runs the single-token kernels;
 * 2 <= T <= 64 groups the (token, slot) pairs by expert and runs grouped
 * MFMA kernels (gate/up streams a selected expert's weights once per 32 of
 * its tokens; down requests them once per 16, and those passes run side by
 * side on one XCD, so the repeats are mostly served by its L2).
 * x        bf16 [T][H]
 * residual bf16 [T][H] or NULL (no residual); may equal x
 * out      bf16 [T][H]; may equal residual, must not overlap x otherwise
 * topk_idx_out int32 [T][k] / topk_w_out fp32 [T][k]: optional copies */
int moe_decode_layer(const moe_shape* shape, const moe_layer_weights* w, const uint16_t* x,
                     const uint16_t* residual, uint16_t* out, int32_t n_tokens,
                     int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_decode_layer for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same validation, kernels and results, with no workspace argument.
 * Its scratch is a library-owned device array of MOE_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per GPU, held until the process ends; nothing is allocated or
 * freed by any call.  Shapes whose workspace (moe_workspace_size for
 * n_tokens) exceeds that size return MOE_ERR_UNSUPPORTED: every
 * single-token shape fits, and the K3-sized layer fits up to 24
 * tokens.  Every call on a GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams, or host threads) race and give
 * undefined results; serialise them.  The first call on each device looks
 * up the array's address and clears its counter head with a fill kernel on
 * `stream`; make that first call outside graph capture (later calls may be
 * captured).  Other arguments as for moe_decode_layer. */
int moe_decode_layer_noalloc(const moe_shape* shape, const moe_layer_weights* w,
                             const uint16_t* x, const uint16_t* residual, uint16_t* out,
                             int32_t n_tokens, int32_t* topk_idx_out, float* topk_w_out,
                             void* stream);

/* Measurement variant of moe_decode_layer: the same validation, kernels and
 * results, but kernel i of the call is launched with hipExtLaunchKernel so
 * that HIP records when it starts and ends executing on the GPU (the pages
 * count kernels per decoder layer and the gaps between them: page
 * "AI手搓1.2万行代码榨干GB300!…", section 02).
 * events      host array of 2 * max_kernels hipEvent_t handles created by
 *             the caller with timing enabled: kernel i records events[2i]
 *             at its start and events[2i+1] at its end; kernels past
 *             max_kernels (0 <= max_kernels <= MOE_MAX_LAYER_KERNELS)
 *             launch untimed
 * n_kernels   host int32 out: number of kernels the call launched (3 for
 *             one token, 6 for 2..64 tokens; one and two more when the
 *             shared expert's width differs from the routed experts')
 * The events are recorded eagerly, so the call is not meant for graph
 * capture; read them after synchronising the stream. */
int moe_decode_layer_timed(const moe_shape* shape, const moe_layer_weights* w,
                           const uint16_t* x, const uint16_t* residual, uint16_t* out,
                           int32_t n_tokens, int32_t* topk_idx_out, float* topk_w_out,
                           void* ws, size_t ws_bytes, void* stream, void* const* events,
                           int32_t max_kernels, int32_t* n_kernels);

/* Measurement helper: one plain streaming read of `bytes` bytes at `buf`
 * (16-byte aligned, bytes a multiple of 16) with 16-byte nontemporal loads
 * over the whole chip, the rate a weight stream can reach on this GPU.
 * sink: device uint32 [MOE_STREAM_SINK_WORDS]; each workgroup stores the xor
 * of the words it read (contents otherwise meaningless). */
int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* A stack of decode layers run back to back.  Per layer l:
 *   xn = bf16(h * gamma_l / sqrt(mean(h^2) + eps));  h = bf16(h + MoE_l(xn))
 * layers  host array [n_layers] of weight sets (read during the call only)
 * gammas  host array [n_layers] of device bf16 [H] pointers
 * hidden  bf16 [T][H], input h_0 and output h_L (updated in place)
 * topk_idx_out  int32 [n_layers][T][k] or NULL
 * hidden_trace  bf16 [n_layers][T][H] or NULL: h after each layer */
int moe_decode_stack(const moe_shape* shape, const moe_layer_weights* layers,
                     const uint16_t* const* gammas, float eps, int32_t n_layers,
                     uint16_t* hidden, int32_t n_tokens, int32_t* topk_idx_out,
                     uint16_t* hidden_trace, void* ws, size_t ws_bytes, void* stream);

/* Token grouping used by the batched path: a stable counting sort of the
 * T*k (token, slot) pairs by expert.
 *   topk_idx int32 [T][k] (device); values are clamped to [0, E)
 *   offsets int32 [E+1] out: pairs of expert e are pairs[offsets[e]..offsets[e+1])
 *   pairs   int32 [T*k] out: t*k + j, increasing within each expert
 * 0 <= T <= 64, 1 <= k <= min(E, 32), E <= 1024; ws as from
 * moe_workspace_size for any shape with these E, k and at least T tokens. */
int moe_group_by_expert(const int32_t* topk_idx, int32_t n_tokens, int32_t top_k,
                        int32_t n_experts, int32_t* offsets, int32_t* pairs,
                        void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
