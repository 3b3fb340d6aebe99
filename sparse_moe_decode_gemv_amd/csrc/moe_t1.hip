// Single-token (batch 1) decode layer: three kernels per layer, one stream.
//
//  K1a router GEMV over all E rows (one wave per row, every load of the row
//      in flight at once).
//  K2  top-k + softmax (radix select) in every workgroup, then gate/up GEMVs
//      with fused MXFP4 dequant and SiLU gating -> fp32 activations: first
//      the shared expert's rows, then those of the k selected experts.  The
//      shared expert does not depend on routing (the pages run it beside the
//      selected experts: page "AI手搓1.2万行代码榨干GB300!…", section 02;
//      smzdm page, section "四步改造"), so every wave requests its shared
//      rows before the selection and the selection latency is spent under
//      shared-expert bytes.
//  K3  down GEMVs of the k selected experts and of the shared expert,
//      router-weighted combine (shared weight 1) and residual add -> bf16.
//      One workgroup per CU owns a slab of output rows, each wave streams
//      two slots' rows of the slab, and the slots are summed in LDS in a
//      fixed order (deterministic, no floating-point atomics).
//
// Decode is bound by streaming weights from HBM (page "英伟达用1.2万行CuTe DSL
// Megakernel…", section "解码优化为何比训练优化更难"; tmtpost page, section
// "为什么是解码"), so every kernel reads each weight byte once with 16-byte
// nontemporal loads, keeps the activation vector in registers, and decodes
// MXFP4 in registers right before the dot product.
//
// Data passes between kernels only through stream order: no workgroup reads
// what another workgroup of the same launch wrote, so no cross-CU fences or
// flags are needed (the ordering bug the pages report came from activation
// loads moved above a wait: page "英伟达用1.2万行CuTe DSL Megakernel…",
// section "写在最后"; page "AI手搓1.2万行代码榨干GB300!…", section 03).
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxH = 8192;
constexpr int kMaxChunks = kMaxH / 8;          // 16-byte chunks of a bf16 row
constexpr int kChunksPerLane = kMaxChunks / kBlock;

// v if keep, else zero (component-wise select: no stack copies).
__device__ __forceinline__ uint4 keep_or_zero(bool keep, uint4 v) {
  uint4 r;
  r.x = keep ? v.x : 0u;
  r.y = keep ? v.y : 0u;
  r.z = keep ? v.z : 0u;
  r.w = keep ? v.w : 0u;
  return r;
}

// Index of the calling wave in its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// -------------------------------------------------------------------------
// Activation staging: bf16 x -> LDS as bf16 pairs, optionally RMSNorm'ed,
// zero-padded to kMaxChunks chunks.  Every workgroup computes the identical
// vector (fixed reduction order).  All global loads of a thread are issued
// before the first LDS write.
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                        float eps, int H, uint32_t* x_lds, float* red,
                        uint16_t* __restrict__ xn_out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint4* x16 = reinterpret_cast<const uint4*>(x);
  const uint4* g16 = reinterpret_cast<const uint4*>(gamma);
  uint4* l16 = reinterpret_cast<uint4*>(x_lds);
  const int nch = H / 8;
  uint4 v[kChunksPerLane], g[kChunksPerLane];
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = tid + i * kBlock;
    const int cc = c < nch ? c : nch - 1;
    v[i] = x16[cc];
    if (gamma) g[i] = g16[cc];
  }
  if (!gamma) {
#pragma unroll
    for (int i = 0; i < kChunksPerLane; ++i) {
      const int c = tid + i * kBlock;
      l16[c] = keep_or_zero(c < nch, v[i]);
    }
    __syncthreads();
    return;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = tid + i * kBlock;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    float part = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = bf16_to_f32(w[d] & 0xFFFFu), b = bf16_to_f32(w[d] >> 16);
      part = __builtin_fmaf(a, a, part);
      part = __builtin_fmaf(b, b, part);
    }
    ss += c < nch ? part : 0.f;
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = tid + i * kBlock;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = bf16_to_f32(w[d] & 0xFFFFu) * inv * bf16_to_f32(gw[d] & 0xFFFFu);
      const float b = bf16_to_f32(w[d] >> 16) * inv * bf16_to_f32(gw[d] >> 16);
      o[d] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    }
    const uint4 ov = {o[0], o[1], o[2], o[3]};
    l16[c] = keep_or_zero(c < nch, ov);
    if (xn_out && c < nch) reinterpret_cast<uint4*>(xn_out)[c] = ov;
  }
  __syncthreads();
}

// x staging for the gate/up rows, in two halves so that other loads can be
// issued between them: stage_x_load issues the global loads, stage_x_store
// writes LDS (zero padding included) and ends with a barrier.
//
// Layout: 16-byte chunk c of x (block b = c / 4 of 32 elements, quarter
// q = c % 4) is stored at x_chunk_pos(b, q).  A gate/up lane reads the four
// quarters of its blocks b = col + lanes * i; in the natural order the 32
// lanes of a half wave would read at a 64-byte stride, four lanes to a bank
// group.  Here, for one (i, q), consecutive lanes read consecutive chunks.
// The map permutes each group of 128 chunks, so the padded LDS range
// (kMaxChunks, a multiple of 128) maps onto itself.
__device__ __forceinline__ int x_chunk_pos(int b, int q) {
  return (((b >> 5) << 2) + q) * 32 + (b & 31);
}
struct XStage {
  uint4 v[kChunksPerLane];
};
__device__ __forceinline__ void stage_x_load(const uint16_t* __restrict__ x, int H, XStage& st) {
  const uint4* x16 = reinterpret_cast<const uint4*>(x);
  const int nch = H / 8;
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = threadIdx.x + i * kBlock;
    st.v[i] = x16[c < nch ? c : nch - 1];
  }
}
__device__ __forceinline__ void stage_x_store(const XStage& st, int H, uint32_t* x_lds) {
  uint4* l16 = reinterpret_cast<uint4*>(x_lds);
  const int nch = H / 8;
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = threadIdx.x + i * kBlock;
    l16[x_chunk_pos(c >> 2, c & 3)] = keep_or_zero(c < nch, st.v[i]);
  }
  __syncthreads();
}
static_assert(kMaxChunks % 128 == 0, "the chunk map permutes whole groups of 128");

// -------------------------------------------------------------------------
// Router rows: one wave per row; the row's 16-byte chunks are strided over
// the lanes and every chunk is requested before the first dot product (and
// before x is staged).  The loads always cover kMaxChunks chunks so that no
// load is conditional: chunks past the row end load the row's last chunk
// again (in bounds) and meet the zero padding of x in LDS.
struct RouterRow {
  uint4 v[kMaxChunks / kWave];
};
__device__ __forceinline__ void router_row_load(const LayerT1& L, int e, RouterRow& R) {
  const int lane = threadIdx.x & 63;
  const int nch = L.H / 8;
  const uint8_t* row = reinterpret_cast<const uint8_t*>(L.router_w + (size_t)e * L.H);
#pragma unroll
  for (int i = 0; i < kMaxChunks / kWave; ++i) {
    const int c = i * kWave + lane;
    R.v[i] = ld_stream16(row + (size_t)(c < nch ? c : nch - 1) * 16);
  }
}
__device__ __forceinline__ void router_row_finish(const LayerT1& L, int e, const RouterRow& R,
                                                  const uint32_t* x_lds) {
  const int lane = threadIdx.x & 63;
  const uint4* xl = reinterpret_cast<const uint4*>(x_lds);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks / kWave; ++i) {
    const uint4 xv = xl[i * kWave + lane];
    a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(R.v[i].x), as_bf16x2(xv.x), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(R.v[i].y), as_bf16x2(xv.y), a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(R.v[i].z), as_bf16x2(xv.z), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(R.v[i].w), as_bf16x2(xv.w), a1, false);
  }
  const float s = group_sum_last(a0 + a1, kWave);
  if (lane == kWave - 1) {
    L.logits[e] = s;
    if (L.logits_out) L.logits_out[e] = s;
  }
}

// -------------------------------------------------------------------------
// Gate/up row pairs.  Lanes 0..31 stream gate rows, lanes 32..63 the up rows
// with the same index; `lanes` lanes per row (8, 16 or 32), BPL blocks per
// lane, 32/lanes rows per half wave.  A task is one such group of row pairs.
// Tasks 0 .. ns-1 belong to the shared expert (no routing needed, so they
// can be requested before the selection is known), tasks ns .. are the
// routed slots in order.  x comes from LDS, so the registers hold only
// weights in flight: every wave keeps two tasks' loads outstanding.
struct GateUpJob {
  const uint8_t *g_codes, *g_scales, *u_codes, *u_scales;      // routed [E][F][H]
  const uint8_t *sg_codes, *sg_scales, *su_codes, *su_scales;  // shared [F][H]
  const int32_t* e_lds;  // expert of each routed slot, in LDS
  int H, F, k;
  int ns;                // shared tasks (0 without a shared expert)
  float* act;            // [k + 1][F]: routed slots, then the shared expert
};

// LANES > 0 fixes the lanes per row at compile time: the block offsets of a
// row then fold into the load instructions' immediate offsets.
template <int BPL, int LANES = 0>
struct GateUp {
  int half, rig, col, lanes, rph, tps;
  // this lane's matrices (gate for lanes 0..31, up for 32..63), routed and
  // shared: chosen once, so that a task only selects between the two
  const uint8_t *rc, *rs, *shc, *shs;

  __device__ void init(const GateUpJob& J, int lanes_) {
    const int lane = threadIdx.x & 63;
    lanes = LANES ? LANES : lanes_;
    half = lane >> 5;
    rig = (lane & 31) / lanes;
    col = (lane & 31) % lanes;
    rph = 32 / lanes;
    tps = J.F / rph;
    rc = half ? J.u_codes : J.g_codes;
    rs = half ? J.u_scales : J.g_scales;
    shc = half ? J.su_codes : J.sg_codes;
    shs = half ? J.su_scales : J.sg_scales;
  }
  // act row (slot; k for the shared expert) and matrix row of task t
  __device__ __forceinline__ void locate(const GateUpJob& J, int t, bool& sh, int& slot,
                                         int& j) const {
    sh = t < J.ns;
    const int tr = sh ? t : t - J.ns;
    const int s = sh ? 0 : tr / tps;
    slot = sh ? J.k : s;
    j = (tr - s * tps) * rph + rig;
  }
  __device__ __forceinline__ void load(const GateUpJob& J, int t, uint4 (&c)[BPL],
                                       uint32_t (&sc)[BPL]) const {
    bool sh;
    int slot, j;
    locate(J, t, sh, slot, j);
    // selects, not branches: the loads stay unconditional
    const int e = J.e_lds[sh ? 0 : slot];
    const size_t row = (size_t)(sh ? 0 : e) * J.F + j;
    const uint8_t* cb = (sh ? shc : rc) + row * (size_t)(J.H / 2);
    const uint8_t* sb = (sh ? shs : rs) + row * (size_t)(J.H / 32);
    if (LANES) {
      // lane base once, constant strides: immediate offsets on the loads
      const u32x4* cp = reinterpret_cast<const u32x4*>(cb) + col;
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(sb) + (col >> 2);
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const u32x4 t = __builtin_nontemporal_load(cp + LANES * i);
        c[i] = make_uint4(t.x, t.y, t.z, t.w);
        sc[i] = __builtin_nontemporal_load(sp + (LANES / 4) * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const int b = col + lanes * i;
        c[i] = ld_stream16(cb + (size_t)b * 16);
        sc[i] = ld_stream_word_of(sb, b);
      }
    }
  }
  __device__ __forceinline__ void finish(const GateUpJob& J, const uint32_t* x_lds, int t,
                                         const uint4 (&c)[BPL], const uint32_t (&sc)[BPL]) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const uint4* xl = reinterpret_cast<const uint4*>(x_lds);
      const int b = col + lanes * i;
      uint32_t xv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = xl[x_chunk_pos(b, q)];
        xv[4 * q + 0] = v.x;
        xv[4 * q + 1] = v.y;
        xv[4 * q + 2] = v.z;
        xv[4 * q + 3] = v.w;
      }
      // rows are 4-byte multiples and lanes % 4 == 0: block b's byte is b & 3
      const float scale = e8m0_to_f32(byte_of(sc[i], (col + lanes * i) & 3));
      acc = __builtin_fmaf(block_dot_bf16(c[i], xv), scale, acc);
      // keep the x reads of later blocks from being hoisted (register use)
      __builtin_amdgcn_sched_barrier(0);
    }
    if (LANES) acc = group_sum_last_c<LANES ? LANES : 32>(acc);
    else acc = group_sum_last(acc, lanes);
    const float up = __shfl_xor(acc, 32, kWave);
    if (half == 0 && col == lanes - 1) {
      bool sh;
      int slot, j;
      locate(J, t, sh, slot, j);
      J.act[(size_t)slot * J.F + j] = silu(acc) * up;
    }
  }
};

// Tasks first, first + stride, ... below ntask; the first task's weights are
// already in (ca, sa) (requested by the caller ahead of the x staging).  Task
// i + 1 is requested before task i is reduced.  The loop runs an exact trip
// count and the last one or two tasks are peeled, so no load sits under a
// branch that rejoins: at such a join the compiler's wait counts assume the
// path without the load and would wait for the newer loads as well.
template <int BPL, int LANES>
__device__ void gateup_tasks(const GateUp<BPL, LANES>& g, const GateUpJob& J, const uint32_t* x_lds,
                             int ntask, int first, int stride, uint4 (&ca)[BPL],
                             uint32_t (&sa)[BPL]) {
  if (first >= ntask) return;
  const int n = (ntask - first + stride - 1) / stride;
  uint4 cb[BPL];
  uint32_t sb[BPL];
  int t = first, i = 0;
  for (; i + 2 < n; i += 2, t += 2 * stride) {
    g.load(J, t + stride, cb, sb);
    g.finish(J, x_lds, t, ca, sa);
    g.load(J, t + 2 * stride, ca, sa);
    g.finish(J, x_lds, t + stride, cb, sb);
  }
  if (n - i == 2) {
    g.load(J, t + stride, cb, sb);
    g.finish(J, x_lds, t, ca, sa);
    g.finish(J, x_lds, t + stride, cb, sb);
  } else {
    g.finish(J, x_lds, t, ca, sa);
  }
}

// -------------------------------------------------------------------------
// Down rows of one matrix D[H][F] against fp32 activations held in
// registers; `lanes` lanes per row, BPL blocks per lane, 64/lanes rows per
// load instruction.
// LANES > 0 fixes the lane count at compile time (shifts and a constant
// reduction width); LANES = 0 takes it at run time.
template <int BPL, int LANES = 0>
struct DownLanes {
  int rig, col, lanes, rpw;
  float ar[BPL][32];

  __device__ void init_map(int lanes_) {
    const int lane = threadIdx.x & 63;
    lanes = LANES ? LANES : lanes_;
    rig = lane / lanes;
    col = lane % lanes;
    rpw = kWave / lanes;
  }
  __device__ __forceinline__ float reduce(float v) const {
    if (LANES) return group_sum_last_c<LANES ? LANES : 64>(v);
    return group_sum_last(v, lanes);
  }
  // Pins the activations: the wait for their loads happens here, not
  // inside a later loop (an empty asm that claims to modify the registers).
  __device__ __forceinline__ void settle_act() {
#pragma unroll
    for (int i = 0; i < BPL; ++i)
#pragma unroll
      for (int q = 0; q < 32; ++q) asm volatile("" : "+v"(ar[i][q]));
  }
  __device__ void load_act(const float* a) {
    const float4* a16 = reinterpret_cast<const float4*>(a);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = col + lanes * i;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = a16[b * 8 + q];
        ar[i][4 * q + 0] = v.x;
        ar[i][4 * q + 1] = v.y;
        ar[i][4 * q + 2] = v.z;
        ar[i][4 * q + 3] = v.w;
      }
    }
  }
  // Rows row0 .. row0 + rpw - 1 (row0 uniform across the wave; this lane's
  // row is row0 + rig).  Addresses are a wave-uniform base plus a 32-bit
  // lane offset, which keeps one scalar base per load instead of a 64-bit
  // vector address (many rows are in flight at once).
  __device__ __forceinline__ void load_row(const uint8_t* codes, const uint8_t* scales, int F,
                                           int row0, uint4 (&c)[BPL], uint32_t (&sc)[BPL]) const {
    const uint8_t* cb = codes + (size_t)row0 * (F / 2);
    const uint8_t* sb = scales + (size_t)row0 * (F / 32);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const uint32_t b = (uint32_t)(col + lanes * i);
      c[i] = ld_stream16(cb + ((uint32_t)rig * (uint32_t)(F / 2) + b * 16u));
      sc[i] = ld_stream_word_of(sb + (uint32_t)rig * (uint32_t)(F / 32), (int)b);
    }
  }
  // The same rows of one matrix given as buffer descriptors (codes, scales):
  // the row offset goes in a scalar register, the lane offset in one vector
  // register shared by every row.
  __device__ __forceinline__ void load_row_buf(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                               int F, int row0, uint4 (&c)[BPL],
                                               uint32_t (&sc)[BPL]) const {
    const uint32_t soc = (uint32_t)row0 * (uint32_t)(F / 2);
    const uint32_t sos = (uint32_t)row0 * (uint32_t)(F / 32);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const uint32_t b = (uint32_t)(col + lanes * i);
      c[i] = buf_ld16(rc, (uint32_t)rig * (uint32_t)(F / 2) + b * 16u, soc);
      sc[i] = buf_ld4(rs, ((uint32_t)rig * (uint32_t)(F / 32) + b) & ~3u, sos);
    }
  }
  __device__ __forceinline__ float dot(const uint4 (&c)[BPL], const uint32_t (&sc)[BPL]) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < BPL; ++i)
      acc = __builtin_fmaf(block_dot_f32(c[i], ar[i]),
                           e8m0_to_f32(byte_of(sc[i], (col + lanes * i) & 3)), acc);
    return acc;
  }
};

// -------------------------------------------------------------------------
// K1a: router rows.  Each wave requests its first row before x is staged
// (RMSNorm'ed for the stack; workgroup 0 also stores the normalised x for
// the next kernel), so that the weight stream starts at once.
__global__ __launch_bounds__(kBlock) void k1_router(LayerT1 L) {
  __shared__ __align__(16) uint32_t x_lds[kMaxH / 2];
  __shared__ float red[kWaves];
  const int wid = wave_id();
  const int gw = blockIdx.x * kWaves + wid, nw = gridDim.x * kWaves;
  RouterRow R;
  router_row_load(L, gw < L.E ? gw : L.E - 1, R);
  stage_x(L.x, L.gamma, L.eps, L.H, x_lds, red, (L.gamma && blockIdx.x == 0) ? L.xn : nullptr);
  if (gw < L.E) router_row_finish(L, gw, R, x_lds);
  for (int e = gw + nw; e < L.E; e += nw) {
    router_row_load(L, e, R);
    router_row_finish(L, e, R, x_lds);
  }
}

// K1b (router-only entry point): top-k + softmax of the logits, one workgroup.
__global__ __launch_bounds__(kBlock) void k1_topk(LayerT1 L) {
  __shared__ TopkLds tk;
  float lg[kTopkPerThread];
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) {
    const int e = threadIdx.x * kTopkPerThread + i;
    lg[i] = L.logits[e < L.E ? e : L.E - 1];
  }
  topk_softmax_block(lg, L.E, L.k, tk, L.idx, L.wts, L.idx_out, L.w_out);
}

// Two waves per SIMD for the gate/up kernel: three (at most 168 registers)
// measured no faster, and the selection then covers fewer shared tasks.
constexpr int kK2WavesPerSimd = 2;

// K2: gate/up of the shared expert and of the k selected experts.  With
// idx == null the experts are selected here: every workgroup runs the same
// top-k on the router logits (deterministic, identical in every workgroup)
// and workgroup 0 publishes the indices and weights for K3 and the caller.
// With a shared expert (PRE) a wave whose first task is a shared one
// requests it before the selection, so the selection latency is spent under
// shared-expert bytes.
template <int BPLH, int LANES, bool PRE>
__global__ __launch_bounds__(kBlock, kK2WavesPerSimd) void k2_gateup(LayerT1 L, const uint16_t* __restrict__ x,
                                                    const int32_t* __restrict__ idx,
                                                    float* __restrict__ act, int gu_lanes, int ns) {
  __shared__ __align__(16) uint32_t x_lds[kMaxH / 2];
  __shared__ int32_t e_lds[kMaxTopK];
  __shared__ float w_lds[kMaxTopK];
  __shared__ TopkLds tk;
  const int wid = wave_id();
  const GateUpJob J{L.g_codes,  L.g_scales,  L.u_codes,  L.u_scales, L.sg_codes, L.sg_scales,
                    L.su_codes, L.su_scales, e_lds,      L.H,        L.F,        L.k,
                    ns,         act};
  GateUp<BPLH, LANES> g;
  g.init(J, gu_lanes);
  const int first = blockIdx.x * kWaves + wid, ntask = ns + L.k * g.tps;
  // Request order matters: loads complete in order for the wait counter, so
  // the selection's inputs go first and the shared weights last; waiting
  // for the logits then leaves the shared weights in flight.
  float lg[kTopkPerThread];
  int32_t e_in = 0;
  if (idx) {
    e_in = idx[threadIdx.x < L.k ? threadIdx.x : 0];
  } else {
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) {
      const int e = threadIdx.x * kTopkPerThread + i;
      lg[i] = L.logits[e < L.E ? e : L.E - 1];
    }
  }
  XStage xs;
  stage_x_load(x, L.H, xs);
  uint4 ca[BPLH];
  uint32_t sa[BPLH];
  const bool early = PRE && first < ns;  // wave-uniform
  if (early) g.load(J, first, ca, sa);
  if (idx) {
    if (threadIdx.x < L.k)
      e_lds[threadIdx.x] = e_in < 0 ? 0 : (e_in >= L.E ? L.E - 1 : e_in);  // never address outside
    __syncthreads();
  } else {
    topk_softmax_block(lg, L.E, L.k, tk, e_lds, w_lds, nullptr, nullptr);
    __syncthreads();
  }
  if (!early) g.load(J, first < ntask ? first : ntask - 1, ca, sa);
  stage_x_store(xs, L.H, x_lds);
  if (!idx && blockIdx.x == 0 && threadIdx.x < L.k) {
    const int e = e_lds[threadIdx.x];
    const float w = w_lds[threadIdx.x];
    L.idx[threadIdx.x] = e;
    L.wts[threadIdx.x] = w;
    if (L.idx_out) L.idx_out[threadIdx.x] = e;
    if (L.w_out) L.w_out[threadIdx.x] = w;
  }
  gateup_tasks(g, J, x_lds, ntask, first, gridDim.x * kWaves, ca, sa);
}

// K3: one workgroup per row slab of `gpb` row groups, one slab per CU.  With
// nw waves, wave w streams the slab's rows of two routed slots at once, w
// and w + nw (then w + 2 nw and w + 3 nw, ...), with the activations of
// both slots in registers.  Rows go in bursts of kK3Burst row groups per
// slot, double-buffered: the next burst is requested before the current one
// is reduced, so every wave keeps one to two bursts in flight.  A wave left
// with a single slot streams that slot alone.  The shared expert (weight 1)
// is split by rows instead: wave w takes its share of the slab's rows.  Its
// rows and activations need no routing, so they are requested first, while
// the expert ids are still in flight, and reduced once the first routed
// burst has been requested.  Each row result is added to the wave's own LDS
// partial; the partials are then summed in wave order and the residual is
// added.  (F = 4096 keeps one routed slot per pass: its two blocks per lane
// double the activation registers.)
constexpr int kK3MaxWaves = 8;  // 2 waves per SIMD: up to 256 registers
constexpr int kK3MaxRows = 64;
constexpr int kK3Burst = 4;
constexpr int kK3ShRows = 4;     // shared row groups requested up front per wave

template <int BPLF, int LANES>
struct DownBurst {
  uint4 ca[kK3Burst][BPLF], cb[kK3Burst][BPLF];
  uint32_t xa[kK3Burst][BPLF], xb[kK3Burst][BPLF];
};

// Where a slot's down rows come from: buffer descriptors of its matrix, its
// combine weight and its activations.
struct DownSlot {
  __amdgpu_buffer_rsrc_t rc, rs;
  float w;
  const float* act;
};
// Routed slot s (< k).  e_v / w_v hold the routed experts and weights one
// per lane (lane i: slot i), loaded once by the caller, so that every slot
// reads them with a lane read instead of a memory round trip of its own.
__device__ __forceinline__ DownSlot routed_slot(const LayerT1& L, int s, int e_v, float w_v) {
  const size_t mat_c = (size_t)L.H * (L.F / 2), mat_s = (size_t)L.H * (L.F / 32);
  const int e0 = __builtin_amdgcn_readlane(e_v, s);
  const int e = e0 < 0 ? 0 : (e0 >= L.E ? L.E - 1 : e0);  // never address outside
  DownSlot d;
  d.rc = buf_rsrc(L.d_codes + e * mat_c, (uint32_t)mat_c);
  d.rs = buf_rsrc(L.d_scales + e * mat_s, (uint32_t)mat_s);
  d.w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_v), s));
  d.act = L.act + (size_t)s * L.F;
  return d;
}
// The shared expert; without one the descriptors are empty (reads give 0)
// and the activations point at slot 0 (in bounds, unused).
__device__ __forceinline__ DownSlot shared_slot(const LayerT1& L) {
  const size_t mat_c = (size_t)L.H * (L.F / 2), mat_s = (size_t)L.H * (L.F / 32);
  DownSlot d;
  d.rc = buf_rsrc(L.S ? L.sd_codes : nullptr, L.S ? (uint32_t)mat_c : 0u);
  d.rs = buf_rsrc(L.S ? L.sd_scales : nullptr, L.S ? (uint32_t)mat_s : 0u);
  d.w = 1.f;
  d.act = L.act + (L.S ? (size_t)L.k * L.F : 0);
  return d;
}

// One wave's pass over the slab for one or two routed slots (TWO),
// accumulating into its LDS partial row `red`; `between` runs once the
// first bursts and the activations have been requested.  DEPTH bursts are
// in flight while one is reduced.  Every request is unconditional: a load
// under a branch that rejoins makes the compiler wait for the newer loads
// as well.  Bursts past the slab end are issued against an empty
// descriptor: they return zeros without a memory access (a scalar select,
// so the lane offsets stay loop-invariant registers).
template <int BPLF, int LANES, bool TWO, int DEPTH, typename Between>
__device__ __forceinline__ void down_pass(const LayerT1& L, const DownSlot& A, const DownSlot& B,
                                          DownLanes<BPLF, LANES>& dA, DownLanes<BPLF, LANES>& dB,
                                          int gbase, int ng, float* red, Between between) {
  constexpr int NB = kK3Burst;
  const int nb = (ng + NB - 1) / NB;
  const __amdgpu_buffer_rsrc_t none = buf_rsrc(nullptr, 0u);
  auto load_burst = [&](int i, DownBurst<BPLF, LANES>& P) {
    const bool skip = i >= nb;
    const auto rca = skip ? none : A.rc, rsa = skip ? none : A.rs;
    const auto rcb = skip ? none : B.rc, rsb = skip ? none : B.rs;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int g = i * NB + j;
      const int row0 = (gbase + (g < ng ? g : ng - 1)) * dA.rpw;
      dA.load_row_buf(rca, rsa, L.F, row0, P.ca[j], P.xa[j]);
      if (TWO) dB.load_row_buf(rcb, rsb, L.F, row0, P.cb[j], P.xb[j]);
    }
  };
  auto use_burst = [&](int i, const DownBurst<BPLF, LANES>& P) {
    const int g0 = i * NB;
    float v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // one row of one slot at a time: unpacking more at once costs registers
      v[j] = A.w * dA.dot(P.ca[j], P.xa[j]);
      __builtin_amdgcn_sched_barrier(0);
      if (TWO) v[j] = __builtin_fmaf(B.w, dB.dot(P.cb[j], P.xb[j]), v[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = dA.reduce(v[j]);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (g0 + j < ng && dA.col == dA.lanes - 1) red[(g0 + j) * dA.rpw + dA.rig] += v[j];
  };
  // Activations first: the loop is then entered, as it is re-entered, with
  // exactly the weight bursts outstanding, and the compiler's wait counts
  // in the loop need not cover a younger activation load.
  dA.load_act(A.act);
  if (TWO) dB.load_act(B.act);
  DownBurst<BPLF, LANES> P, Q;
  load_burst(0, P);
  if constexpr (DEPTH == 3) {
    DownBurst<BPLF, LANES> R;
    load_burst(1, Q);
    // Wait for the activations now, with two bursts in flight: entering the
    // loop with them still outstanding would put 64 loads in flight at its
    // first request, past what the wait counter tracks, and every later
    // wait in the loop would be too deep.
    dA.settle_act();
    if (TWO) dB.settle_act();
    between();
    for (int i = 0; i < nb; i += 3) {
      load_burst(i + 2, R);
      __builtin_amdgcn_sched_barrier(0);
      use_burst(i, P);
      if (i + 1 >= nb) break;
      load_burst(i + 3, P);
      __builtin_amdgcn_sched_barrier(0);
      use_burst(i + 1, Q);
      if (i + 2 >= nb) break;
      load_burst(i + 4, Q);
      __builtin_amdgcn_sched_barrier(0);
      use_burst(i + 2, R);
    }
  } else {
    between();
    for (int i = 0; i < nb; i += 2) {
      load_burst(i + 1, Q);
      __builtin_amdgcn_sched_barrier(0);
      use_burst(i, P);
      if (i + 1 >= nb) break;
      load_burst(i + 2, P);
      __builtin_amdgcn_sched_barrier(0);
      use_burst(i + 1, Q);
    }
  }
}

template <int BPLF, int LANES>
__global__ __launch_bounds__(kK3MaxWaves * kWave) void k3_down_combine(LayerT1 L, int dn_lanes,
                                                                       int gpb) {
  __shared__ float red[kK3MaxWaves][kK3MaxRows];
  constexpr bool PAIRS = BPLF == 1;
  const int wid = wave_id(), lane = threadIdx.x & 63;
  const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  // routed experts and weights, lane i holding slot i (k <= 32 < 64); these
  // go first so that waiting for them leaves the later requests in flight
  const int e_v = L.idx[lane < L.k ? lane : 0];
  const float w_v = L.wts[lane < L.k ? lane : 0];
  DownLanes<BPLF, LANES> dA, dB, dS;
  dA.init_map(dn_lanes);
  dB.init_map(dn_lanes);
  dS.init_map(dn_lanes);
  const int ngroups = L.H / dA.rpw;
  const int gbase = blockIdx.x * gpb;
  const int ng = ngroups - gbase < gpb ? ngroups - gbase : gpb;  // groups of this slab
  const int R = ng * dA.rpw;
  // each wave zeroes and later accumulates only its own partial row: no
  // barrier needed before the first accumulation
  for (int t = lane; t < R; t += kWave) red[wid][t] = 0.f;
  // residual of this thread's output row, requested now so that the final
  // combine waits on nothing but LDS.  A raw 32-bit buffer read: without a
  // residual the descriptor is empty and the read gives 0, with no branch.
  const int trow = gbase * dA.rpw + (threadIdx.x < R ? threadIdx.x : 0);
  const uint32_t res_word = buf_ld4(buf_rsrc(L.residual, L.residual ? (uint32_t)L.H * 2u : 0u),
                                    ((uint32_t)trow * 2u) & ~3u, 0u);
  // this wave's share of the shared expert's row groups: [sh0, sh1)
  const int sh0 = L.S ? wid * ng / nw : 0, sh1 = L.S ? (wid + 1) * ng / nw : 0;
  const DownSlot SH = shared_slot(L);
  uint4 shc[kK3ShRows][BPLF];
  uint32_t shs[kK3ShRows][BPLF];
#pragma unroll
  for (int j = 0; j < kK3ShRows; ++j) {
    const int g = sh0 + j < sh1 ? sh0 + j : (sh1 > sh0 ? sh1 - 1 : 0);
    dS.load_row_buf(SH.rc, SH.rs, L.F, (gbase + g) * dS.rpw, shc[j], shs[j]);
  }
  dS.load_act(SH.act);
  auto shared_rows = [&]() {
#pragma unroll
    for (int j = 0; j < kK3ShRows; ++j) {
      float v = dS.dot(shc[j], shs[j]);
      __builtin_amdgcn_sched_barrier(0);
      v = dS.reduce(v);
      if (sh0 + j < sh1 && dS.col == dS.lanes - 1) red[wid][(sh0 + j) * dS.rpw + dS.rig] += v;
    }
  };

  const int step = PAIRS ? 2 * nw : nw;
  auto routed = [&](int s0, auto between) {
    const int sb = s0 + nw;
    const DownSlot A = routed_slot(L, s0, e_v, w_v);
    // three bursts in flight where the registers allow it (one block per lane)
    constexpr int DEPTH = BPLF == 1 ? 3 : 2;
    if (PAIRS && sb < L.k) {
      const DownSlot B = routed_slot(L, sb, e_v, w_v);
      down_pass<BPLF, LANES, PAIRS, DEPTH>(L, A, B, dA, dB, gbase, ng, red[wid], between);
    } else {
      down_pass<BPLF, LANES, false, DEPTH>(L, A, A, dA, dB, gbase, ng, red[wid], between);
    }
  };
  // The first pass is not part of the loop: inside it the shared rows would
  // be loop-invariant, and the compiler would reduce them (and wait for
  // them) before the first routed burst is requested.
  if (wid < L.k) {
    routed(wid, [&]() {
      __builtin_amdgcn_sched_barrier(0);
      shared_rows();
    });
  } else {
    shared_rows();  // a wave without routed slots
  }
  for (int s0 = wid + step; s0 < L.k; s0 += step) routed(s0, []() {});
  // shared row groups past the ones requested up front (only when the slab
  // has more than kK3ShRows groups per wave)
  for (int g = sh0 + kK3ShRows; g < sh1; ++g) {
    uint4 c[BPLF];
    uint32_t x[BPLF];
    dS.load_row_buf(SH.rc, SH.rs, L.F, (gbase + g) * dS.rpw, c, x);
    const float v = dS.reduce(dS.dot(c, x));
    if (dS.col == dS.lanes - 1) red[wid][g * dS.rpw + dS.rig] += v;
  }
  __syncthreads();
  if ((int)threadIdx.x < R) {  // R <= kK3MaxRows <= the workgroup size
    float tot = 0.f;
    for (int v = 0; v < nw; ++v) tot += red[v][threadIdx.x];
    const float res = bf16_to_f32((res_word >> (16 * (trow & 1))) & 0xFFFFu);
    const uint16_t o = f32_to_bf16(tot + res);
    L.out[trow] = o;
    if (L.trace) L.trace[trow] = o;
  }
}

// K3, activations in LDS (one block per lane, F a multiple of 32 x lanes,
// and every slot's activations within kK3LdsActBytes).  The workgroup first
// copies the activations of all slots into LDS; then the work is a list of
// bursts, (slot, kK3Burst row groups of the slab), the shared expert's
// first, dealt round robin to kK3LdsWaves waves.  A wave keeps three bursts
// in flight and reads the slot's activations from LDS once per burst, so it
// needs few registers: four waves per SIMD.  Requests past the end of a
// wave's list go to an empty descriptor (zeros, no memory traffic).  Row
// results go to the wave's LDS partial row; partials are summed in wave
// order with the residual, as in the register variant.
constexpr int kK3LdsWaves = 16;
constexpr int kK3LdsActBytes = 144 * 1024;
static_assert(kK3LdsActBytes % (16 * kK3LdsWaves * kWave) == 0, "whole staging rounds");

template <int LANES>
struct LdsBurst {
  uint4 c[kK3Burst];
  uint32_t x[kK3Burst];
  int as, c0;  // activation slot and first row group (wave-uniform)
  float w;     // combine weight
};

template <int LANES>
__global__ __launch_bounds__(kK3LdsWaves * kWave) void k3_down_lds(LayerT1 L, int gpb) {
  extern __shared__ __align__(16) float k3_smem[];
  float* act_lds = k3_smem;                                        // [slots][8][F/32][4]
  float* red = k3_smem + (size_t)(L.k + (L.S ? 1 : 0)) * L.F;   // [waves][kK3MaxRows]
  constexpr int NB = kK3Burst;
  // one block per lane: F = 32 LANES, and a row group (64 / LANES rows) is
  // always 1 KB of codes and 64 bytes of scales
  constexpr uint32_t kGroupCodes = 1024, kGroupScales = 64;
  const int wid = wave_id(), lane = threadIdx.x & 63;
  const int nslots = L.k + (L.S ? 1 : 0);
  // routed experts and weights, lane i holding slot i (k <= 32 < 64)
  const int e_v = L.idx[lane < L.k ? lane : 0];
  const float w_v = L.wts[lane < L.k ? lane : 0];
  DownLanes<1, LANES> d;
  d.init_map(LANES);
  const int ngroups = L.H / d.rpw;
  const int gbase = blockIdx.x * gpb;
  const int ng = ngroups - gbase < gpb ? ngroups - gbase : gpb;  // groups of this slab
  const int R = ng * d.rpw;
  float* red_w = red + wid * kK3MaxRows;
  for (int t = lane; t < R; t += kWave) red_w[t] = 0.f;
  const int trow = gbase * d.rpw + (threadIdx.x < R ? threadIdx.x : 0);
  const uint32_t res_word = buf_ld4(buf_rsrc(L.residual, L.residual ? (uint32_t)L.H * 2u : 0u),
                                    ((uint32_t)trow * 2u) & ~3u, 0u);
  // activations -> LDS: float4 j of a slot (elements 4j..4j+3, block j/8,
  // chunk j%8) goes to position (j%8) * nbk + j/8, so that a chunk read of
  // consecutive blocks by consecutive lanes touches consecutive addresses
  const int nbk = L.F / 32, f4_per_slot = L.F / 4, f4_total = nslots * f4_per_slot;
  // one staging round covers kK3LdsActBytes (the launcher's bound)
  constexpr int kStage = kK3LdsActBytes / 16 / (kK3LdsWaves * kWave);
  f32x4 st[kStage];  // native vectors: an array of HIP's float4 struct lands in scratch
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int j = u * (int)blockDim.x + (int)threadIdx.x;
    st[u] = reinterpret_cast<const f32x4*>(L.act)[j < f4_total ? j : f4_total - 1];
  }

  // this wave's bursts: b = wid, wid + nw, ...; burst b covers list slot
  // p = b / nch (0: the shared expert when present) and chunk b % nch
  const int nch = (ng + NB - 1) / NB, nbt = nslots * nch;
  constexpr int nw = kK3LdsWaves;
  // b / nch as a multiply and shift (scalar divisions are long sequences):
  // exact for b < 2^16 / 64 with nch <= 64 (here b < 33 * 16, nch <= 16)
  const int inv_nch = (65536 + nch - 1) / nch;
  const size_t mat_c = (size_t)L.H * (L.F / 2), mat_s = (size_t)L.H * (L.F / 32);
  // lane offsets within a row group (loop-invariant vector registers)
  const uint32_t voc = (uint32_t)d.rig * (uint32_t)(L.F / 2) + (uint32_t)d.col * 16u;
  const uint32_t vos = ((uint32_t)d.rig * (uint32_t)(L.F / 32) + (uint32_t)d.col) & ~3u;
  // Burst i of this wave: slot, weight and row groups are computed once,
  // here, and travel with the buffer.  The matrix base and the size are
  // selected as scalars and one descriptor is built from them (selecting
  // whole descriptors compiles to branches).  Row groups past the slab end
  // read the next rows of the matrix, or zeros past its end; their results
  // are dropped.
  auto load_burst = [&](int i, LdsBurst<LANES>& P) {
    const int b = wid + i * nw;
    const int bb = b < nbt ? b : nbt - 1;
    const int p = (bb * inv_nch) >> 16;
    const bool sh = L.S && p == 0;
    const int s = sh ? 0 : p - (L.S ? 1 : 0);  // routed slot
    const int e0 = __builtin_amdgcn_readlane(e_v, s);
    const int e = sh ? 0 : (e0 < 0 ? 0 : (e0 >= L.E ? L.E - 1 : e0));  // never address outside
    P.as = sh ? L.k : s;
    P.w = sh ? 1.f : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_v), s));
    P.c0 = (bb - p * nch) * NB;
    const bool live = b < nbt;
    const auto rc = buf_rsrc((sh ? L.sd_codes : L.d_codes) + (size_t)e * mat_c,
                             live ? (uint32_t)mat_c : 0u);
    const auto rs = buf_rsrc((sh ? L.sd_scales : L.d_scales) + (size_t)e * mat_s,
                             live ? (uint32_t)mat_s : 0u);
    const uint32_t g0 = (uint32_t)(gbase + P.c0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      P.c[j] = buf_ld16(rc, voc + j * kGroupCodes, g0 * kGroupCodes);
      P.x[j] = buf_ld4(rs, vos + j * kGroupScales, g0 * kGroupScales);
    }
  };
  auto use_burst = [&](int i, const LdsBurst<LANES>& P) {
    const bool live = wid + i * nw < nbt;
    // this lane's 32 activations of the slot, chunk by chunk
    const f32x4* a4 = reinterpret_cast<const f32x4*>(act_lds) + (size_t)P.as * f4_per_slot + d.col;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 v = a4[q * nbk];
      d.ar[0][4 * q + 0] = v.x;
      d.ar[0][4 * q + 1] = v.y;
      d.ar[0][4 * q + 2] = v.z;
      d.ar[0][4 * q + 3] = v.w;
    }
    float v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint4 c1[1] = {P.c[j]};
      const uint32_t x1[1] = {P.x[j]};
      v[j] = P.w * d.dot(c1, x1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = d.reduce(v[j]);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (live && P.c0 + j < ng && d.col == d.lanes - 1) red_w[(P.c0 + j) * d.rpw + d.rig] += v[j];
  };

  LdsBurst<LANES> P, Q, Rb;
  load_burst(0, P);
  load_burst(1, Q);
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int j = u * (int)blockDim.x + (int)threadIdx.x;
    if (j < f4_total) {
      const int sl = j / f4_per_slot, jj = j - sl * f4_per_slot;
      reinterpret_cast<f32x4*>(act_lds)[sl * f4_per_slot + (jj & 7) * nbk + (jj >> 3)] = st[u];
    }
  }
  __syncthreads();  // activations in LDS
  const int nb = (nbt - wid + nw - 1) / nw;  // bursts of this wave
  for (int i = 0; i < nb; i += 3) {
    load_burst(i + 2, Rb);
    __builtin_amdgcn_sched_barrier(0);
    use_burst(i, P);
    if (i + 1 >= nb) break;
    load_burst(i + 3, P);
    __builtin_amdgcn_sched_barrier(0);
    use_burst(i + 1, Q);
    if (i + 2 >= nb) break;
    load_burst(i + 4, Q);
    __builtin_amdgcn_sched_barrier(0);
    use_burst(i + 2, Rb);
  }
  __syncthreads();
  if ((int)threadIdx.x < R) {  // R <= kK3MaxRows <= the workgroup size
    float tot = 0.f;
    for (int v = 0; v < nw; ++v) tot += red[v * kK3MaxRows + threadIdx.x];
    const float res = bf16_to_f32((res_word >> (16 * (trow & 1))) & 0xFFFFu);
    const uint16_t o = f32_to_bf16(tot + res);
    L.out[trow] = o;
    if (L.trace) L.trace[trow] = o;
  }
}

// ---------------------------------------------------------------- dispatch
constexpr int kK2WavesPerCU = 4 * kK2WavesPerSimd;
constexpr int kNumCU = 256;

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

template <int B>
hipError_t k2_launch(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                     int n_gu, int lanes, int ns, bool pre, hipStream_t s) {
#define K2(LN, P) \
  hipLaunchKernelGGL((k2_gateup<B, LN, P>), dim3(n_gu), dim3(kBlock), 0, s, L, x, idx, act, lanes, ns)
  if (lanes == 32) {  // the common case (H a multiple of 1024): offsets fold
    if (pre) K2(32, true);
    else K2(32, false);
  } else {
    if (pre) K2(0, true);
    else K2(0, false);
  }
#undef K2
  return hipPeekAtLastError();
}

// More than 64 KB of dynamic LDS needs the function's limit raised first
// (set on every launch: cheap, and correct on whichever device is current).
template <int LN>
hipError_t k3_lds_launch(const LayerT1& L, int gpb, int nblk, size_t lds, hipStream_t s) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k3_down_lds<LN>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k3_down_lds<LN>), dim3(nblk), dim3(kK3LdsWaves * kWave), lds, s, L, gpb);
  return hipPeekAtLastError();
}

}  // namespace

hipError_t launch_router_t1(const LayerT1& L, hipStream_t s) {
  hipLaunchKernelGGL(k1_router, dim3(ceil_div(L.E, kWaves)), dim3(kBlock), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_topk_t1(const LayerT1& L, hipStream_t s) {
  hipLaunchKernelGGL(k1_topk, dim3(1), dim3(kBlock), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_gateup_t1(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                            bool with_shared, hipStream_t s) {
  const RowMap gm = gateup_map(L.H);
  const int tps = L.F / (32 / gm.lanes);  // tasks per expert
  const int ns = (with_shared && L.S) ? tps : 0;
  const int tasks = ns + L.k * tps;
  const int cap = kNumCU * kK2WavesPerCU / kWaves;
  int n_gu = ceil_div(tasks, kWaves * 4) < cap ? ceil_div(tasks, kWaves * 4) : cap;
  // with a shared expert every wave starts on a shared task (tps is a
  // multiple of kWaves for every accepted F), requested before the selection
  const bool pre = ns > 0;
  if (pre && n_gu * kWaves > ns) n_gu = ns / kWaves;
  switch (gm.bpl) {
    case 1: return k2_launch<1>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 2: return k2_launch<2>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 3: return k2_launch<3>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 4: return k2_launch<4>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 5: return k2_launch<5>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 6: return k2_launch<6>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 7: return k2_launch<7>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
    case 8: return k2_launch<8>(L, x, idx, act, n_gu, gm.lanes, ns, pre, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_combine_t1(const LayerT1& L, hipStream_t s) {
  const RowMap dm = down_map(L.F);
  const int ngroups = L.H / (kWave / dm.lanes);
  const int gpb = ceil_div(ngroups, kNumCU);  // one slab per CU
  const int nblk = ceil_div(ngroups, gpb);
  if (gpb * (kWave / dm.lanes) > kK3MaxRows) return hipErrorInvalidValue;
  // one expert's down matrix is addressed through a 32-bit buffer descriptor
  if ((size_t)L.H * (size_t)(L.F / 2) > 0x7FFFFFFFu) return hipErrorInvalidValue;
  const size_t act_bytes = (size_t)(L.k + (L.S ? 1 : 0)) * L.F * sizeof(float);
  if (dm.bpl == 1 && act_bytes <= (size_t)kK3LdsActBytes) {
    const size_t lds = act_bytes + (size_t)kK3LdsWaves * kK3MaxRows * sizeof(float);
    switch (dm.lanes) {
      case 64: return k3_lds_launch<64>(L, gpb, nblk, lds, s);
      case 32: return k3_lds_launch<32>(L, gpb, nblk, lds, s);
      case 16: return k3_lds_launch<16>(L, gpb, nblk, lds, s);
      case 8: return k3_lds_launch<8>(L, gpb, nblk, lds, s);
      case 4: return k3_lds_launch<4>(L, gpb, nblk, lds, s);
    }
    return hipErrorInvalidValue;
  }
  const int per_wave = dm.bpl == 1 ? 2 : 1;  // routed slots streamed together
  int nw = ceil_div(L.k, per_wave);
  if (nw > kK3MaxWaves) nw = kK3MaxWaves;
  if (nw * kWave < gpb * (kWave / dm.lanes)) nw = ceil_div(gpb * (kWave / dm.lanes), kWave);
  const dim3 g(nblk), b(nw * kWave);
#define K3(BP, LN) hipLaunchKernelGGL((k3_down_combine<BP, LN>), g, b, 0, s, L, dm.lanes, gpb)
  if (dm.bpl == 2) K3(2, 64);
  else if (dm.lanes == 64) K3(1, 64);
  else if (dm.lanes == 32) K3(1, 32);
  else if (dm.lanes == 16) K3(1, 16);
  else if (dm.lanes == 8) K3(1, 8);
  else if (dm.lanes == 4) K3(1, 4);
  else return hipErrorInvalidValue;
#undef K3
  return hipPeekAtLastError();
}

// ------------------------------------------------------------------ utils
namespace {
__global__ void zero_fill_kernel(uint32_t* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t g = (n + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(g > 4096 ? 4096 : g)), dim3(256), 0, s,
                     (uint32_t*)p, n);
  return hipPeekAtLastError();
}

}  // namespace moe
