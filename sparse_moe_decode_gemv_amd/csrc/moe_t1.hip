// Single-token (batch 1) decode layer: three kernels per layer, one stream.
//
//  K1a router GEMV over all E rows (one wave per row, every load of the row
//      in flight at once).
//  K2  top-k + softmax (one wave per workgroup) in every workgroup, then gate/up GEMVs
//      with fused MXFP4 dequant and SiLU gating -> gated activations (fp32
//      for the gate/up entry point; in the layer, two bf16 parts for K3):
//      first the shared expert's rows, then those of the k selected experts.  The
//      shared expert does not depend on routing (the pages run it beside the
//      selected experts: page "AI手搓1.2万行代码榨干GB300!…", section 02;
//      smzdm page, section "四步改造"), so every wave requests its shared
//      rows before the selection and the selection latency is spent under
//      shared-expert bytes.
//  K3  down GEMVs of the k selected experts and of the shared expert,
//      router-weighted combine (shared weight 1) and residual add -> bf16.
//      The gated activations arrive split into two bf16 parts (leading part
//      + remainder), so the products run on v_mfma_f32_4x4x4_16b_bf16 with
//      about 16 significant bits of the activation, and the vector ALU only
//      decodes MXFP4.  When every slot's activations fit in LDS, one
//      workgroup per CU owns a slab of output rows for every slot and sums
//      the slots in LDS in a fixed order (deterministic, no floating-point
//      atomics); otherwise a workgroup owns one slot's rows of one chunk and
//      the chunk's last workgroup combines (see k3_down).
//
// Decode is bound by streaming weights from HBM (page "英伟达用1.2万行CuTe DSL
// Megakernel…", section "解码优化为何比训练优化更难"; tmtpost page, section
// "为什么是解码"), so every kernel reads each weight byte once with 16-byte
// nontemporal loads and decodes MXFP4 in registers right before use.
//
// Between kernels data passes through stream order.  Inside a launch only
// k3_down's chunk combine crosses workgroups, through agent-scope atomic
// accesses and a counter (the ordering bug the pages report came from
// activation loads moved above a wait: page "英伟达用1.2万行CuTe DSL
// Megakernel…", section "写在最后"; page "AI手搓1.2万行代码榨干GB300!…",
// section 03).
#include "moe.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kK3SlabW = 8;  // waves per workgroup of the slab down kernel (two per SIMD)
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
// vector (fixed reduction order).  In two halves: stage_x_request issues the
// loads of x and gamma (no branch: a null gamma reads through an empty
// descriptor, which returns zeros without a memory access), stage_x_finish
// waits for them and writes LDS.  The router requests x before its weight
// rows, so that the norm is computed while the rows stream in; with the x
// and gamma loads behind the rows, or a gamma load under a branch (which
// the compiler sank past the wait for the rows), each layer of the stack
// paid about 1.2 us more in this kernel.
struct XNorm {
  uint4 v[kChunksPerLane], g[kChunksPerLane];
};
__device__ __forceinline__ void stage_x_request(const uint16_t* x, const uint16_t* gamma, int H, XNorm& X) {
  const int tid = threadIdx.x;
  const int nch = H / 8;
  const auto rx = buf_rsrc(x, 2u * (uint32_t)H), rg = buf_rsrc(gamma, gamma ? 2u * (uint32_t)H : 0u);
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = tid + i * kBlock;
    const uint32_t off = 16u * (uint32_t)(c < nch ? c : nch - 1);
    X.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
    X.g[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, (int)off, 0, 0));
  }
}
__device__ __forceinline__ void stage_x_finish(const XNorm& X, bool norm, float eps, int H, uint32_t* x_lds,
                                               float* red, uint16_t* __restrict__ xn_out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint4* l16 = reinterpret_cast<uint4*>(x_lds);
  const int nch = H / 8;
  if (!norm) {
#pragma unroll
    for (int i = 0; i < kChunksPerLane; ++i) {
      const int c = tid + i * kBlock;
      l16[c] = keep_or_zero(c < nch, X.v[i]);
    }
    __syncthreads();
    return;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = tid + i * kBlock;
    const uint32_t w[4] = {X.v[i].x, X.v[i].y, X.v[i].z, X.v[i].w};
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
    const uint32_t w[4] = {X.v[i].x, X.v[i].y, X.v[i].z, X.v[i].w};
    const uint32_t gw[4] = {X.g[i].x, X.g[i].y, X.g[i].z, X.g[i].w};
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
// Every workgroup copies the same x at the same moment; each starts at its
// own chunk (a rotation of the order), so that the workgroups of an XCD do
// not all ask one L2 channel for the same lines.  Chunk slots past the end
// of x hold the zero padding at their own positions.
__device__ __forceinline__ int x_stage_chunk(int i, int nch) {
  const int c = threadIdx.x + i * kBlock;
  if (c >= nch) return c;
  const int r = c + (int)(((unsigned)blockIdx.x * 8u * 8u) % (unsigned)nch);
  return r >= nch ? r - nch : r;
}
__device__ __forceinline__ void stage_x_load(const uint16_t* __restrict__ x, int H, XStage& st) {
  const uint4* x16 = reinterpret_cast<const uint4*>(x);
  const int nch = H / 8;
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = x_stage_chunk(i, nch);
    st.v[i] = x16[c < nch ? c : nch - 1];
  }
}
__device__ __forceinline__ void stage_x_store(const XStage& st, int H, uint32_t* x_lds) {
  uint4* l16 = reinterpret_cast<uint4*>(x_lds);
  const int nch = H / 8;
#pragma unroll
  for (int i = 0; i < kChunksPerLane; ++i) {
    const int c = x_stage_chunk(i, nch);
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
  float* act;            // fp32 [k + 1][F]: routed slots, then the shared expert
  uint16_t* act_hl;      // or bf16 [2][nslot][F]: leading parts, then remainders
  int nslot;
  uint16_t* act_sh;      // shared expert of width Fs != F: bf16 [2][Fs] (else null)
  int Fs;
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
    if (LANES == 32) {
      // lane base once, constant strides: immediate offsets on the loads.
      // The row's 8 BPL scale dwords come in one or two loads (lane col:
      // dwords col and col + 32, clamped to the row); finish() fetches each
      // block's dword from its lane with ds_bpermute.
      const u32x4* cp = reinterpret_cast<const u32x4*>(cb) + col;
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(sb);
      constexpr int ND = 8 * BPL;  // scale dwords of a row
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const u32x4 t = __builtin_nontemporal_load(cp + LANES * i);
        c[i] = make_uint4(t.x, t.y, t.z, t.w);
      }
      sc[0] = __builtin_nontemporal_load(sw + (col < ND ? col : ND - 1));
      if (BPL > 4) sc[1] = __builtin_nontemporal_load(sw + (col + 32 < ND ? col + 32 : ND - 1));
#pragma unroll
      for (int i = (BPL > 4 ? 2 : 1); i < BPL; ++i) sc[i] = 0u;
    } else if (LANES) {
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
                                         const uint4 (&c)[BPL], const uint32_t (&sc_in)[BPL]) const {
    uint32_t sc[BPL];
    if (LANES == 32) {  // block col + 32 i's dword (col / 4 + 8 i) from the lane holding it
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < BPL; ++i)
        sc[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane & 32) + (((col >> 2) + 8 * i) & 31)),
                                                       (int)sc_in[i < 4 ? 0 : 1]);
    } else {
#pragma unroll
      for (int i = 0; i < BPL; ++i) sc[i] = sc_in[i];
    }
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
    // Every lane stores; only a row's owner (the last lane of its gate group)
    // has an offset inside the buffer, the others' stores are dropped by the
    // range check.  No branch, so the wait counts of the task loop stay exact.
    bool sh;
    int slot, j;
    locate(J, t, sh, slot, j);
    const bool own = half == 0 && col == lanes - 1;
    const float a = silu(acc) * up;
    if (J.act_hl) {  // a = hi + lo to about 16 significant bits
      const uint16_t hi = f32_to_bf16(a);
      const float d = a - bf16_to_f32(hi);
      const uint16_t lo = f32_to_bf16(d == d ? d : 0.f);
      // the shared expert has its own two planes when its width differs
      const bool sep = sh && J.act_sh;  // wave-uniform
      const uint32_t plane = sep ? (uint32_t)J.Fs : (uint32_t)J.nslot * (uint32_t)J.F;
      const auto r = buf_rsrc(sep ? J.act_sh : J.act_hl, 4u * plane);
      const uint32_t o = own ? 2u * (uint32_t)(sep ? j : slot * J.F + j) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b16(hi, r, (int)o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(lo, r, (int)(own ? o + 2u * plane : o), 0, 0);
    } else {
      const auto r = buf_rsrc(J.act, 4u * (uint32_t)(J.k + 1) * (uint32_t)J.F);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r,
                                            (int)(own ? 4u * (uint32_t)(slot * J.F + j) : 0xFFFFFFF0u), 0, 0);
    }
  }
};

// A wave's task list: first + i * stride for i < n1, then first2 + (i - n1)
// * stride2 up to n tasks in all.
struct TaskSeq {
  int first, stride, n1, first2, stride2, n;
  __device__ __forceinline__ int at(int i) const {
    return i < n1 ? first + i * stride : first2 + (i - n1) * stride2;
  }
};

// The tasks of q in order; the first task's weights are already in (ca, sa)
// (requested by the caller ahead of the x staging).  Task i + 1 is requested
// before task i is reduced.  The loop runs an exact trip count and the last
// one or two tasks are peeled, so no load sits under a branch that rejoins:
// at such a join the compiler's wait counts assume the path without the load
// and would wait for the newer loads as well.
template <int BPL, int LANES>
__device__ void gateup_tasks(const GateUp<BPL, LANES>& g, const GateUpJob& J, const uint32_t* x_lds,
                             const TaskSeq& q, uint4 (&ca)[BPL], uint32_t (&sa)[BPL]) {
  const int n = q.n;
  if (n <= 0) return;
  uint4 cb[BPL];
  uint32_t sb[BPL];
  int i = 0;
  for (; i + 2 < n; i += 2) {
    g.load(J, q.at(i + 1), cb, sb);
    g.finish(J, x_lds, q.at(i), ca, sa);
    g.load(J, q.at(i + 2), ca, sa);
    g.finish(J, x_lds, q.at(i + 1), cb, sb);
  }
  if (n - i == 2) {
    g.load(J, q.at(i + 1), cb, sb);
    g.finish(J, x_lds, q.at(i), ca, sa);
    g.finish(J, x_lds, q.at(i + 1), cb, sb);
  } else {
    g.finish(J, x_lds, q.at(i), ca, sa);
  }
}

// -------------------------------------------------------------------------
// K1a: router rows.  Each thread requests its x (and gamma) chunks, then
// each wave its first row, all before x is staged (RMSNorm'ed for the
// stack; workgroup 0 also stores the normalised x for the next kernel):
// the weight stream starts at once and the staging waits for x only.
__global__ __launch_bounds__(kBlock) void k1_router(LayerT1 L) {
  __shared__ __align__(16) uint32_t x_lds[kMaxH / 2];
  __shared__ float red[kWaves];
  const int wid = wave_id();
  const int gw = blockIdx.x * kWaves + wid, nw = gridDim.x * kWaves;
  XNorm X;
  stage_x_request(L.x, L.gamma, L.H, X);
  __builtin_amdgcn_sched_barrier(0);
  RouterRow R;
  router_row_load(L, gw < L.E ? gw : L.E - 1, R);
  __builtin_amdgcn_sched_barrier(0);
  stage_x_finish(X, L.gamma != nullptr, L.eps, L.H, x_lds, red, (L.gamma && blockIdx.x == 0) ? L.xn : nullptr);
  if (gw < L.E) router_row_finish(L, gw, R, x_lds);
  for (int e = gw + nw; e < L.E; e += nw) {
    router_row_load(L, e, R);
    router_row_finish(L, e, R, x_lds);
  }
}

// Lane l of a wave: router logits 16 l .. 16 l + 15 (four 16-byte loads),
// then as order-preserving keys (experts past E are absent: key 0).
__device__ __forceinline__ void load_logits16(const float* logits, int E, f32x4 (&v)[4]) {
  const int lane = threadIdx.x & 63;
  const auto rl = buf_rsrc(logits, 4u * (uint32_t)E);  // E = 0: zeros, no access
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, 64 * lane + 16 * q, 0, 0));
}
__device__ __forceinline__ void logit_keys16(const f32x4 (&v)[4], int E, uint32_t (&key)[16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) key[4 * q + c] = 16 * lane + 4 * q + c < E ? f32_order_key(v[q][c]) : 0u;
}

// K1b (router-only entry point): top-k + softmax of the logits, one workgroup.
__global__ __launch_bounds__(kBlock) void k1_topk(LayerT1 L) {
  __shared__ TopkLds tk;
  if (wave_id() == 0) {
    f32x4 lv[4];
    uint32_t key[16];
    load_logits16(L.logits, L.E, lv);
    logit_keys16(lv, L.E, key);
    if (!topk_softmax_wave(key, L.E, L.k, tk, L.idx, L.wts, L.idx_out, L.w_out))
      topk_softmax_wave_rounds(key, L.E, L.k, L.idx, L.wts, L.idx_out, L.w_out);  // many ties
  }
}

// Two waves per SIMD for the gate/up kernel: three (at most 168 registers)
// measured no faster, and the selection then covers fewer shared tasks.
constexpr int kK2WavesPerSimd = 2;
constexpr int kK2OldRounds = 3;  // task rounds given to the older workgroups only (2: +0.5 us, 4..6: no better)

// K2: gate/up of the shared expert and of the k selected experts.  With
// idx == null the experts are selected here: every workgroup runs the same
// top-k on the router logits (deterministic, identical in every workgroup)
// and workgroup 0 publishes the indices and weights for K3 and the caller.
// With a shared expert (PRE) the workgroups whose waves all start on a
// shared task (the first ns / 4) request it before the selection, so the
// selection latency is spent under shared-expert bytes; the others (when
// the expert is narrower than the grid has waves) request their first task
// after it.  The two kinds are separate code paths chosen per workgroup, so
// neither has a load under a branch that rejoins.
struct K2Lds {
  uint32_t x[kMaxH / 2];
  int32_t e[kMaxTopK];
  float w[kMaxTopK];
  TopkLds tk;
};

template <int BPLH, int LANES, bool EARLY>
__device__ __forceinline__ void k2_body(const LayerT1& L, const uint16_t* __restrict__ x,
                                        const int32_t* __restrict__ idx, float* __restrict__ act,
                                        int gu_lanes, int ns, K2Lds& sm) {
  uint32_t* x_lds = sm.x;
  int32_t* e_lds = sm.e;
  float* w_lds = sm.w;
  TopkLds& tk = sm.tk;
  const int wid = wave_id();
  const GateUpJob J{L.g_codes,  L.g_scales,  L.u_codes,  L.u_scales, L.sg_codes, L.sg_scales,
                    L.su_codes, L.su_scales, e_lds,      L.H,        L.F,        L.k,
                    ns,         act,        act ? nullptr : L.act_hl,
                    L.k + (L.S && !L.act_sh ? 1 : 0), act ? nullptr : L.act_sh, L.Fs};
  GateUp<BPLH, LANES> g;
  g.init(J, gu_lanes);
  const int first = blockIdx.x * kWaves + wid, ntask = ns + L.k * g.tps;
  // Request order matters: loads complete in order for the wait counter, so
  // the selection's inputs go first and the shared weights last; waiting
  // for the logits then leaves the shared weights in flight.  Wave 0 makes
  // the selection alone (no barrier inside it).
  // (both requested unconditionally, the unneeded ones through an empty
  // descriptor, so that every path has the same loads in flight; only wave 0
  // reads the logits)
  f32x4 lv[4];
  const int32_t e_in = (int32_t)buf_ld4(buf_rsrc(idx, idx ? 4u * (uint32_t)L.k : 0u),
                                        4u * (threadIdx.x < L.k ? threadIdx.x : 0u), 0u);
  load_logits16(L.logits, (idx || wid != 0) ? 0 : L.E, lv);
  XStage xs;
  stage_x_load(x, L.H, xs);
  uint4 ca[BPLH];
  uint32_t sa[BPLH];
  constexpr bool early = EARLY;  // every wave of this workgroup starts on a shared task
  if (early) g.load(J, first, ca, sa);
  if (idx) {
    if (threadIdx.x < L.k)
      e_lds[threadIdx.x] = e_in < 0 ? 0 : (e_in >= L.E ? L.E - 1 : e_in);  // never address outside
    __syncthreads();
  } else {
    if (wid == 0) {
      uint32_t key[16];
      logit_keys16(lv, L.E, key);
      if (!topk_softmax_wave(key, L.E, L.k, tk, e_lds, w_lds, nullptr, nullptr))
        topk_softmax_wave_rounds(key, L.E, L.k, e_lds, w_lds, nullptr, nullptr);  // many ties
    }
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
  // Rounds of one task per wave, except that the last kK2OldRounds rounds
  // go to the older half of the workgroups (launched first: on each CU the
  // older workgroup's waves are served first and would otherwise finish
  // early, leaving the younger ones streaming with half the loads in flight).
  const int nw = gridDim.x * kWaves, rounds = ntask / nw;
  TaskSeq q{first, nw, 0, 0, nw / 2, 0};
  if (rounds >= 8) {
    const int split = (rounds - kK2OldRounds) * nw;
    q.n1 = rounds - kK2OldRounds;
    q.first2 = split + first;
    q.n = q.n1 + (first < nw / 2 && q.first2 < ntask ? (ntask - q.first2 + nw / 2 - 1) / (nw / 2) : 0);
  } else {
    q.n1 = q.n = first < ntask ? (ntask - first + nw - 1) / nw : 0;
  }
  gateup_tasks(g, J, x_lds, q, ca, sa);
}

template <int BPLH, int LANES, bool PRE>
__global__ __launch_bounds__(kBlock, kK2WavesPerSimd) void k2_gateup(LayerT1 L, const uint16_t* __restrict__ x,
                                                    const int32_t* __restrict__ idx,
                                                    float* __restrict__ act, int gu_lanes, int ns) {
  __shared__ __align__(16) K2Lds sm;
  if (PRE && (int)blockIdx.x < ns / kWaves)  // workgroup-uniform
    k2_body<BPLH, LANES, true>(L, x, idx, act, gu_lanes, ns, sm);
  else
    k2_body<BPLH, LANES, false>(L, x, idx, act, gu_lanes, ns, sm);
}

// K3: down projection of every slot on the matrix cores, router-weighted
// combine with the shared expert (weight 1) and residual add -> bf16.
//
// Workgroup (slot s, chunk c): the chunk is a run of row groups of the
// slot's down matrix D[H][F], and the workgroup's waves are kqn slices of
// the reduction index (NI load instructions each) times nsn row streams.
// One load instruction reads 64 / CPR rows, 16 CPR contiguous bytes of each
// (four rows x 256 bytes when F >= 512: whole cache lines), one MXFP4 block
// per lane.  The lanes are laid out as v_mfma_f32_4x4x4_16b_bf16 wants them:
// lane 4 b + i holds A_b[i][.] (row i of block b, b = one lane's block) and
// B_b[.][i] (column i), so the loaded blocks are A operands as they stand.
// Block b's B operand is the matching stretch of the slot's activation:
// column 0 its leading bf16 part, column 1 the remainder (together about 16
// significant bits), columns 2 and 3 zero.  A wave holds its slice of B for
// the whole launch; the vector ALU only decodes codes to exact bf16 (scale
// folded in), the matrix cores multiply, and each row's total is the sum of
// its accumulator over the lanes of its blocks.  Every wave keeps three row
// groups' loads in flight.  Slice sums meet in LDS, added in slice order.
//
// The combine crosses workgroups: the nslots workgroups of a chunk store
// their weighted rows with agent-scope atomic stores (coherent across the
// L2s) and then count themselves on the chunk's counter with one
// acquire-release increment per workgroup, which orders the rows before the
// count.  The workgroup that counts last (its increment acquires every
// earlier one) reads every slot's rows with agent-scope atomic loads, sums
// them in slot order (deterministic: no floating-point atomics), adds the
// residual, stores bf16 and clears the counter for the next call.
constexpr int kK3W = 8;                       // waves per workgroup (two per SIMD)
// row groups in flight per wave, within 256 registers (two waves per SIMD)
constexpr int k3_depth(int ni) { return ni == 4 ? 4 : 6; }
constexpr int kK3RedFloats = 8192;            // LDS slice sums [kqn][chunk rows]
constexpr int kK3MaxChunks = MOE_WS_COUNTER_BYTES / 4;

typedef __attribute__((ext_vector_type(4))) short s16x4;  // four bf16: a 4x4x4 operand

template <int NI>
struct DownGroup {
  uint4 c[NI];      // per instruction: this lane's MXFP4 block (16 code bytes)
  uint32_t sc[NI];  // per instruction: the row's scale dword holding the block's byte
};

__device__ __forceinline__ s16x4 pack_bf16x4(bf16x2 lo, bf16x2 hi) {
  const uint2 v = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  return __builtin_bit_cast(s16x4, v);
}
__device__ __forceinline__ s16x4 dwords_bf16x4(uint32_t a, uint32_t b) {
  const uint2 v = make_uint2(a, b);
  return __builtin_bit_cast(s16x4, v);
}
__device__ __forceinline__ f32x4 mfma4(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ld_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// One row group on the matrix cores.  Lane 4 b + i4 holds, for each of the
// NI instructions, block cc of row 4 rho + i4 (codes and scale dword) and
// the matching B fragments (bv: 32 bf16 of the activation, column i4).
// Returns the row quad's four row sums, valid in the quad's last lane.
template <int CPR, int NI>
__device__ __forceinline__ f32x4 down_group_rows(const DownGroup<NI>& P, const u32x4 (&bv)[NI][4], int cc) {
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const float scl = e8m0_to_f32(byte_of(P.sc[t], cc & 3));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t cw = dword_of(P.c[t], u);
      const s16x4 x0 = pack_bf16x4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scl, 0),
                                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scl, 1));
      const s16x4 x1 = pack_bf16x4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scl, 2),
                                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scl, 3));
      a0 = mfma4(x0, dwords_bf16x4(bv[t][u][0], bv[t][u][1]), a0);
      a1 = mfma4(x1, dwords_bf16x4(bv[t][u][2], bv[t][u][3]), a1);
    }
  }
  // row 4 rho + r: accumulator r summed over the row quad's lanes
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = group_sum_last_c<4 * CPR>(a0[r] + a1[r]);
  return v;
}

template <int CPR, int NI, int D, int W>
__global__ __launch_bounds__(W * kWave) void k3_down(LayerT1 L, int nchunk,
                                                                                    int kqn, int nsn) {
  constexpr int RPI = 64 / CPR;  // rows of a row group
  constexpr int GW = 4 * CPR;    // lanes of one row quad
  __shared__ __align__(16) float red[kK3RedFloats];
  __shared__ int last;
  const int wid = wave_id(), lane = threadIdx.x & 63;
  const int b = lane >> 2, i4 = lane & 3;       // MFMA block; row (A) and column (B) in it
  const int rho = b / CPR, cc = b - rho * CPR;  // row quad, block within the instruction
  const int nslots = L.k + (L.S ? 1 : 0);
  const int s = blockIdx.x / nchunk, c = blockIdx.x - s * nchunk;  // slot, chunk
  const int kq = wid % kqn, st = wid / kqn;                        // slice, row stream
  const int nrg = L.H / RPI, nb = L.F / 32;
  const int cg0 = c * nrg / nchunk, cg1 = (c + 1) * nrg / nchunk;  // the chunk's row groups
  const int crows = (cg1 - cg0) * RPI;
  const int g0 = cg0 + (cg1 - cg0) * st / nsn, g1 = cg0 + (cg1 - cg0) * (st + 1) / nsn;
  const int n = g1 - g0;  // row groups of this wave
  // the slot: routed (expert idx[s], weight wts[s]) or, s == k, the shared one
  const bool sh = s >= L.k;
  const int e0 = sh ? 0 : L.idx[s];
  const int e = sh ? 0 : (e0 < 0 ? 0 : (e0 >= L.E ? L.E - 1 : e0));  // never address outside
  const float w = sh ? 1.f : L.wts[s];
  const uint32_t F2 = (uint32_t)L.F / 2, F32 = (uint32_t)L.F / 32;
  const uint32_t mat_c = (uint32_t)L.H * F2, mat_s = (uint32_t)L.H * F32;
  const uint8_t* cb = (sh ? L.sd_codes : L.d_codes) + (size_t)e * mat_c;
  const uint8_t* sb = (sh ? L.sd_scales : L.d_scales) + (size_t)e * mat_s;
  const uint32_t row_in = 4u * (uint32_t)rho + (uint32_t)i4;  // this lane's row in a group (A)
  // instruction t reads block (kq NI + t) CPR + cc of each row; blocks past
  // the row (F / 32 not a multiple of CPR) re-read the row's last block and
  // meet a zero B operand; instructions wholly past it are not issued
  // (empty descriptor)
  uint32_t voc[NI], vos[NI], voa[NI];
  bool ilive[NI];
  {
    const uint32_t arow = (uint32_t)((i4 == 1 ? nslots + s : s) * L.F);
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const int gb = (kq * NI + t) * CPR + cc;
      const int gbc = gb < nb ? gb : nb - 1;
      ilive[t] = (kq * NI + t) * CPR < nb;
      voc[t] = row_in * F2 + 16u * (uint32_t)gbc;
      vos[t] = row_in * F32 + 4u * (uint32_t)(gbc >> 2);
      voa[t] = (gb < nb && i4 < 2) ? 2u * (arow + 32u * (uint32_t)gb) : 0xFFFFFF00u;
    }
  }
  // B operand: the block's 32 activation elements (column i4), or zeros
  u32x4 bv[NI][4];
  {
    const auto ra = buf_rsrc(L.act_hl, 4u * (uint32_t)nslots * (uint32_t)L.F);  // [2][nslots][F] bf16
#pragma unroll
    for (int t = 0; t < NI; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        bv[t][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ra, (int)(voa[t] + 16u * u), 0, kBufNT));
  }
  auto load_group = [&](int i, DownGroup<NI>& P) {
    const bool live = i < n;
    const uint32_t g = (uint32_t)__builtin_amdgcn_readfirstlane(g0 + (live ? i : 0));
    const uint32_t soc = g * RPI * F2, sos = g * RPI * F32;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const bool lv = live && ilive[t];
      P.c[t] = buf_ld16(buf_rsrc(cb, lv ? mat_c : 0u), voc[t], soc);
      P.sc[t] = buf_ld4(buf_rsrc(sb, lv ? mat_s : 0u), vos[t], sos);
    }
  };
  auto use_group = [&](int i, const DownGroup<NI>& P) {
    const f32x4 v = down_group_rows<CPR, NI>(P, bv, cc);
    if ((lane & (GW - 1)) == GW - 1)
      *reinterpret_cast<f32x4*>(&red[kq * crows + (g0 + i - cg0) * RPI + 4 * rho]) = v;
  };
  // issue order is wait order: activation, then groups 0 .. D-2 (pinned).
  // The activation is waited for here, with those groups in flight, so that
  // the loop is entered as it is re-entered: with D - 1 groups pending
  DownGroup<NI> ring[D];
#pragma unroll
  for (int k = 0; k < D - 1; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    load_group(k, ring[k]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NI; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(bv[t][u]));
  // whole rounds of D groups (group i + k + D - 1 requested before group
  // i + k is used), then the last D - 1 at most
  int i = 0;
  for (; i + D <= n; i += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      load_group(i + k + D - 1, ring[(k + D - 1) % D]);
      __builtin_amdgcn_sched_barrier(0);
      use_group(i + k, ring[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < D - 1; ++k)
    if (i + k < n) use_group(i + k, ring[k]);
  __syncthreads();

  // the slot's weighted rows of the chunk (slices in order), published
  float* part = L.part + (size_t)s * L.H + (size_t)cg0 * RPI;
  for (int r = (int)threadIdx.x; r < crows; r += (int)blockDim.x) {
    float v = 0.f;
    for (int kk = 0; kk < kqn; ++kk) v += red[kk * crows + r];
    st_agent(part + r, w * v);
  }
  // Every wave's stores happen before thread 0's increment (barrier); the
  // increment releases them at agent scope and, in the last workgroup,
  // acquires the other workgroups' rows, which the barrier then hands on
  // to every thread of the workgroup.  Each wave also waits for its own
  // stores before the barrier, so they have reached the coherent level
  // whatever order the memory path keeps between waves.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&L.counters[c], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(nslots - 1);
  __syncthreads();
  if (!last) return;
  // last of the chunk: every slot's rows, summed in slot order (all requested
  // at once; indices past the last slot repeat it and are masked)
  const float* p0 = L.part + (size_t)cg0 * RPI;
  for (int r = (int)threadIdx.x; r < crows; r += (int)blockDim.x) {
    float pv[kMaxTopK + 1];
#pragma unroll
    for (int u = 0; u <= kMaxTopK; ++u) pv[u] = ld_agent(p0 + (size_t)(u < nslots ? u : nslots - 1) * L.H + r);
    float tot = 0.f;
#pragma unroll
    for (int u = 0; u <= kMaxTopK; ++u) tot += u < nslots ? pv[u] : 0.f;
    const int row = cg0 * RPI + r;
    if (L.part_in) tot += L.part_in[row];
    if (L.part_out) {
      L.part_out[row] = tot;
      continue;
    }
    if (L.residual) tot += bf16_to_f32(L.residual[row]);
    const uint16_t o = f32_to_bf16(tot);
    L.out[row] = o;
    if (L.trace) L.trace[row] = o;
  }
  if (threadIdx.x == 0) __hip_atomic_store(&L.counters[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K3 when the split activations of every slot fit in LDS (F <= 2048 with
// these tiles): workgroup = a slab of gpb row groups for every slot, so the
// slots are combined inside the workgroup and no workgroup waits for
// another.  The activations ([2][nslots][F] bf16) are copied to LDS with
// direct loads issued before the first weight requests (waiting for them
// then leaves the weights in flight).  A wave's tasks are consecutive
// (slot, row group) pairs in slot-major order, so it reads its B operand
// from LDS only when its slot changes.  The weighted row sums of every slot
// meet in LDS and are added in slot order, with the residual.
constexpr int kK3SlabD = 4;                  // row groups in flight per wave
constexpr size_t kK3SlabLds = 156 * 1024;    // LDS budget: activations + row sums

// SC1 (F = 512 NI exactly, 16 blocks per instruction): one scale dword per
// lane and group, lane 4b+i holding dword b of row i's scales; the dword
// with block 16t + b's byte is then fetched from lane 4(4t + b/4) + i by
// ds_bpermute, one vector-memory instruction per group instead of NI.
//
// ONE: every workgroup owns one row group (narrow experts), so every task is
// another slot; the waves then take tasks wid, wid + W, ... (measured: the
// TP-16 slice 17.32 against 17.67 us per layer).  Otherwise a wave takes a
// block of consecutive tasks, so that a slot's row groups share its B
// operand (the strided order ran 2.3 us slower at FFN 2048).
template <int CPR, int NI, bool SC1, bool ONE>
__global__ __launch_bounds__(kK3SlabW * kWave) void k3_slab(LayerT1 L, int gpb) {
  constexpr int RPI = 64 / CPR, GW = 4 * CPR, D = kK3SlabD, W = kK3SlabW;
  extern __shared__ __align__(16) uint8_t k3_smem[];
  const int wid = wave_id(), lane = threadIdx.x & 63;
  const int b = lane >> 2, i4 = lane & 3;       // MFMA block; row (A) and column (B) in it
  const int rho = b / CPR, cc = b - rho * CPR;  // row quad, block within the instruction
  const int nslots = L.k + (L.S ? 1 : 0);
  const int nrg = L.H / RPI, nb = L.F / 32;
  const int gb0 = blockIdx.x * gpb;
  const int G = ONE ? 1 : (gpb < nrg - gb0 ? gpb : nrg - gb0);  // row groups of this workgroup
  const int srows = G * RPI;
  const int ntask = nslots * G;
  constexpr int TS = ONE ? W : 1;  // task stride of a wave
  const int w0 = ONE ? wid : ntask * wid / W;
  const int n = ONE ? (ntask > wid ? (ntask - wid + W - 1) / W : 0) : ntask * (wid + 1) / W - w0;
  const uint32_t abytes = 4u * (uint32_t)nslots * (uint32_t)L.F;
  const uint32_t akb = (abytes + 1023u) / 1024u;  // 1 KB copies
  float* red = reinterpret_cast<float*>(k3_smem + 1024u * akb);  // [nslots][srows]

  // activations -> LDS, one KB per wave instruction (past the end: zeros)
  {
    const auto ra = buf_rsrc(L.act_hl, abytes);
    for (uint32_t kb = (uint32_t)wid; kb < akb; kb += W)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, k3_smem + 1024u * kb, 16, 16 * lane, 1024 * kb, 0, 0);
  }
  const uint32_t F2 = (uint32_t)L.F / 2, F32 = (uint32_t)L.F / 32;
  const uint32_t mat_c = (uint32_t)L.H * F2, mat_s = (uint32_t)L.H * F32;
  const uint32_t row_in = 4u * (uint32_t)rho + (uint32_t)i4;
  uint32_t voc[NI], vos[NI];
  bool ilive[NI];
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int gb = t * CPR + cc;
    const int gbc = gb < nb ? gb : nb - 1;
    ilive[t] = t * CPR < nb;
    voc[t] = row_in * F2 + 16u * (uint32_t)gbc;
    vos[t] = row_in * F32 + 4u * (uint32_t)(gbc >> 2);
  }
  const uint32_t vos1 = row_in * F32 + 4u * (uint32_t)b;  // SC1: dword b of the row
  // task i of the wave: t = w0 + TS i, slot t / G, row group gb0 + t % G
  auto load_group = [&](int i, DownGroup<NI>& P) {
    const bool live = i < n;
    const int t = w0 + TS * (live ? i : 0);
    const int sl = __builtin_amdgcn_readfirstlane(t / G);
    const uint32_t g = (uint32_t)(gb0 + (t - sl * G));
    const bool sh = sl >= L.k;
    const int e0 = sh ? 0 : ld_uniform(L.idx + sl);  // scalar load: no vector wait
    const int e = e0 < 0 ? 0 : (e0 >= L.E ? L.E - 1 : e0);  // never address outside
    const uint8_t* cb = (sh ? L.sd_codes : L.d_codes) + (size_t)e * mat_c;
    const uint8_t* sb = (sh ? L.sd_scales : L.d_scales) + (size_t)e * mat_s;
    const uint32_t soc = g * RPI * F2, sos = g * RPI * F32;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const bool lv = live && ilive[u];
      P.c[u] = buf_ld16(buf_rsrc(cb, lv ? mat_c : 0u), voc[u], soc);
      if (!SC1) P.sc[u] = buf_ld4(buf_rsrc(sb, lv ? mat_s : 0u), vos[u], sos);
      else if (u > 0) P.sc[u] = 0u;
    }
    if (SC1) P.sc[0] = buf_ld4(buf_rsrc(sb, live ? mat_s : 0u), vos1, sos);
  };
  DownGroup<NI> ring[D];
#pragma unroll
  for (int k = 0; k < D - 1; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    load_group(k, ring[k]);
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // activations in LDS (the compiler waits for the copies only)

  // B operand of slot sl from LDS: 32 activation elements per block, column
  // i4 (0: leading parts, 1: remainders, 2 and 3: zeros)
  u32x4 bv[NI][4];
  int bslot = -1;
  auto load_b = [&](int sl) {
    const uint16_t* ar = reinterpret_cast<const uint16_t*>(k3_smem) + (size_t)(i4 == 1 ? nslots + sl : sl) * L.F;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const int gb = t * CPR + cc;
      const bool on = i4 < 2 && gb < nb;
      const u32x4* src = reinterpret_cast<const u32x4*>(ar + 32 * (on ? gb : 0));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 v = src[u];
        const u32x4 z = {0u, 0u, 0u, 0u};
        bv[t][u] = on ? v : z;
      }
    }
  };
  auto use_group = [&](int i, const DownGroup<NI>& P) {
    const int t = w0 + TS * i;
    const int sl = __builtin_amdgcn_readfirstlane(t / G);
    if (sl != bslot) {
      load_b(sl);
      bslot = sl;
    }
    const float ws = sl >= L.k ? 1.f : ld_uniform(L.wts + sl);
    f32x4 v;
    if (SC1) {
      DownGroup<NI> Q = P;
#pragma unroll
      for (int t = 0; t < NI; ++t)
        Q.sc[t] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * t + 4 * (b >> 2) + i4), (int)P.sc[0]);
      v = down_group_rows<CPR, NI>(Q, bv, cc);
    } else {
      v = down_group_rows<CPR, NI>(P, bv, cc);
    }
    if ((lane & (GW - 1)) == GW - 1) {
      const f32x4 o = {ws * v[0], ws * v[1], ws * v[2], ws * v[3]};
      *reinterpret_cast<f32x4*>(&red[sl * srows + (t - sl * G) * RPI + 4 * rho]) = o;
    }
  };
  bslot = __builtin_amdgcn_readfirstlane(w0 / G);
  load_b(bslot);
  int i = 0;
  for (; i + D <= n; i += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      load_group(i + k + D - 1, ring[(k + D - 1) % D]);
      __builtin_amdgcn_sched_barrier(0);
      use_group(i + k, ring[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < D - 1; ++k)
    if (i + k < n) use_group(i + k, ring[k]);
  __syncthreads();

  // slots summed in order (then a separately computed shared expert), residual added
  for (int r = (int)threadIdx.x; r < srows; r += (int)blockDim.x) {
    float tot = 0.f;
    for (int q = 0; q < nslots; ++q) tot += red[q * srows + r];
    const int row = gb0 * RPI + r;
    if (L.part_in) tot += L.part_in[row];
    if (L.part_out) {
      L.part_out[row] = tot;
      continue;
    }
    if (L.residual) tot += bf16_to_f32(L.residual[row]);
    const uint16_t o = f32_to_bf16(tot);
    L.out[row] = o;
    if (L.trace) L.trace[row] = o;
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
  MOE_LAUNCH(L.timer, (k2_gateup<B, LN, P>), dim3(n_gu), dim3(kBlock), 0, s, L, x, idx, act, lanes, ns)
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
template <int CPR, int NI, bool SC1, bool ONE>
hipError_t k3_slab_launch1(const LayerT1& L, int gpb, int nblk, size_t lds, hipStream_t s) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k3_slab<CPR, NI, SC1, ONE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  MOE_LAUNCH(L.timer, (k3_slab<CPR, NI, SC1, ONE>), dim3(nblk), dim3(kK3SlabW * kWave), lds, s, L, gpb);
  return hipPeekAtLastError();
}
template <int CPR, int NI, bool SC1 = false>
hipError_t k3_slab_launch(const LayerT1& L, int gpb, int nblk, size_t lds, hipStream_t s) {
  return gpb == 1 ? k3_slab_launch1<CPR, NI, SC1, true>(L, gpb, nblk, lds, s)
                  : k3_slab_launch1<CPR, NI, SC1, false>(L, gpb, nblk, lds, s);
}

}  // namespace

hipError_t launch_router_t1(const LayerT1& L, hipStream_t s) {
  MOE_LAUNCH(L.timer, k1_router, dim3(ceil_div(L.E, kWaves)), dim3(kBlock), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_topk_t1(const LayerT1& L, hipStream_t s) {
  MOE_LAUNCH(L.timer, k1_topk, dim3(1), dim3(kBlock), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_gateup_t1(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                            bool with_shared, hipStream_t s) {
  const RowMap gm = gateup_map(L.H);
  const int tps = L.F / (32 / gm.lanes);  // tasks per expert
  const int ns = (with_shared && L.S) ? L.Fs / (32 / gm.lanes) : 0;  // the shared expert's
  const int tasks = ns + L.k * tps;
  const int cap = kNumCU * kK2WavesPerCU / kWaves;
  // about four tasks per wave where there are enough, else one per wave on
  // as many workgroups as the chip holds (narrow experts: latency-bound)
  int n_gu = ceil_div(tasks, kWaves * 4);
  if (n_gu < cap) n_gu = ceil_div(tasks, kWaves) < cap ? ceil_div(tasks, kWaves) : cap;
  if (n_gu > cap) n_gu = cap;
  // with a shared expert the first ns / kWaves workgroups start on shared
  // tasks (tps is a multiple of kWaves for every accepted F), requested
  // before the selection
  const bool pre = ns > 0;
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

namespace {

// How the down projection + combine runs for a layer's shape.
struct DownPlan {
  bool ok, slab;
  int cpr, ni, ni1, nb;
  int gpb, nblk;       // slab kernel: row groups per workgroup, workgroups
  size_t lds;          // slab kernel: dynamic LDS bytes
  int kqn, nsn, nchunk;  // split kernel
};

DownPlan plan_down(const LayerT1& L) {
  DownPlan P{};
  const int nslots = L.k + (L.S ? 1 : 0);
  const int nb = L.F / 32;
  P.nb = nb;
  if (L.F % 128 || L.H % 64 || nslots < 1) return P;
  // one expert's down matrix is addressed through 32-bit buffer offsets
  if ((size_t)L.H * (size_t)(L.F / 2) > 0x7FFFFFFFu) return P;
  const int cpr = nb <= 4 ? 4 : (nb <= 8 ? 8 : 16);  // blocks per row per instruction
  const int ninst = ceil_div(nb, cpr);               // instructions per row
  P.cpr = cpr;
  P.ni = ninst >= 4 ? 4 : (ninst >= 2 ? 2 : 1);
  P.kqn = ceil_div(ninst, P.ni);
  {  // every slot in one workgroup when the activations fit in LDS
    P.ni1 = ninst <= 1 ? 1 : (ninst <= 2 ? 2 : 4);
    const int rpi = 64 / cpr, nrg = L.H / rpi;
    int gpb = ceil_div(nrg, kNumCU);  // about one workgroup per CU
    // narrow experts: when a one-group slab needs little LDS, several
    // workgroups fit on a CU, so use about two per CU (TP-16 slice: 448
    // workgroups instead of 224, 18.8 -> 18.5 us per layer)
    if (1024 * (size_t)ceil_div(4L * nslots * L.F, 1024) + 4 * (size_t)nslots * rpi <= 40 * 1024)
      gpb = ceil_div(nrg, 2 * kNumCU);
    P.gpb = gpb;
    P.nblk = ceil_div(nrg, gpb);
    P.lds = 1024 * (size_t)ceil_div(4L * nslots * L.F, 1024) + 4 * (size_t)nslots * gpb * rpi;
    if (ninst <= 4 && P.lds <= kK3SlabLds) {
      P.ok = P.slab = true;
      return P;
    }
  }
  if (P.kqn > kK3W) return P;
  P.nsn = kK3W / P.kqn;
  const int rpi = 64 / cpr, nrg = L.H / rpi;
  // about one workgroup per CU, within the counters and the LDS slice sums
  int nchunk = kNumCU / nslots;
  if (nchunk < 1) nchunk = 1;
  const int cap = nrg < kK3MaxChunks ? nrg : kK3MaxChunks;
  if (nchunk > cap) nchunk = cap;
  while (P.kqn * ceil_div(nrg, nchunk) * rpi > kK3RedFloats && nchunk < cap) ++nchunk;
  if (P.kqn * ceil_div(nrg, nchunk) * rpi > kK3RedFloats) return P;
  P.nchunk = nchunk;
  P.ok = true;
  return P;
}

hipError_t launch_down(const LayerT1& L, const DownPlan& P, hipStream_t s) {
  if (!P.ok) return hipErrorInvalidValue;
  if (P.slab) {
    const int gpb = P.gpb, nblk = P.nblk;
    const size_t lds = P.lds;
    if (P.cpr == 4) return k3_slab_launch<4, 1>(L, gpb, nblk, lds, s);
    if (P.cpr == 8) return k3_slab_launch<8, 1>(L, gpb, nblk, lds, s);
    if (P.ni1 == 1) return k3_slab_launch<16, 1>(L, gpb, nblk, lds, s);
    if (P.ni1 == 2)
      return P.nb == 32 ? k3_slab_launch<16, 2, true>(L, gpb, nblk, lds, s)
                        : k3_slab_launch<16, 2>(L, gpb, nblk, lds, s);
    return P.nb == 64 ? k3_slab_launch<16, 4, true>(L, gpb, nblk, lds, s)
                      : k3_slab_launch<16, 4>(L, gpb, nblk, lds, s);
  }
  const int nslots = L.k + (L.S ? 1 : 0);
  const int nchunk = P.nchunk, kqn = P.kqn, nsn = P.nsn;
  const dim3 g(nslots * nchunk), b(kqn * nsn * kWave);
#define K3(C, N) MOE_LAUNCH(L.timer, (k3_down<C, N, k3_depth(N), kK3W>), g, b, 0, s, L, nchunk, kqn, nsn)
  if (P.cpr == 4) K3(4, 1);
  else if (P.cpr == 8) K3(8, 1);
  else if (P.ni == 1) K3(16, 1);
  else if (P.ni == 2) K3(16, 2);
  else K3(16, 4);
#undef K3
  return hipPeekAtLastError();
}

}  // namespace

hipError_t launch_down_combine_t1(const LayerT1& L, hipStream_t s) {
  return launch_down(L, plan_down(L), s);
}

hipError_t launch_layer_t1(LayerT1& L, hipStream_t s) {
  if (L.S && L.act_sh) {
    // shared expert of another width: its down projection is a pass of its
    // own (one slot, FFN Fs) into part_sh, which the routed pass adds where
    // the shared slot's rows would have been added (after the routed slots)
    LayerT1 Ls = L;
    Ls.k = 0;
    Ls.F = L.Fs;
    Ls.act_hl = L.act_sh;
    Ls.act_sh = nullptr;
    Ls.part_out = L.part_sh;
    Ls.residual = nullptr;
    Ls.out = nullptr;
    Ls.trace = nullptr;
    LayerT1 Lr = L;
    Lr.S = 0;
    Lr.part_in = L.part_sh;
    const DownPlan Ps = plan_down(Ls), Pr = plan_down(Lr);
    if (!Ps.ok || !Pr.ok) return hipErrorInvalidValue;
    hipError_t e = launch_router_t1(L, s);
    if (e != hipSuccess) return e;
    e = launch_gateup_t1(L, L.gamma ? L.xn : L.x, nullptr, nullptr, true, s);
    if (e != hipSuccess) return e;
    e = launch_down(Ls, Ps, s);
    if (e != hipSuccess) return e;
    return launch_down(Lr, Pr, s);
  }
  const DownPlan P = plan_down(L);
  if (!P.ok) return hipErrorInvalidValue;
  hipError_t e = launch_router_t1(L, s);
  if (e != hipSuccess) return e;
  e = launch_gateup_t1(L, L.gamma ? L.xn : L.x, nullptr, nullptr, true, s);
  if (e != hipSuccess) return e;
  return launch_down(L, P, s);
}

// ------------------------------------------------------------------ utils
namespace {
__global__ void zero_fill_kernel(uint32_t* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}
}  // namespace

namespace {
// Plain streaming read of a buffer: every thread keeps kStreamUnroll
// 16-byte nontemporal loads in flight, a wave's loads of one round cover
// 1 KB of contiguous bytes, and each workgroup stores one xor of what it
// read (so that no load is dead).
constexpr int kStreamUnroll = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  const size_t stride = (size_t)gridDim.x * 256 * kStreamUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * 256 * kStreamUnroll + threadIdx.x; base < n16; base += stride) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = ld_stream16(reinterpret_cast<const uint8_t*>(p + (i < n16 ? i : n16 - 1)));
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}
}  // namespace

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t per = (size_t)256 * kStreamUnroll;
  const size_t want = (n16 + per - 1) / per;
  const unsigned g = (unsigned)(want < MOE_STREAM_SINK_WORDS ? want : MOE_STREAM_SINK_WORDS);
  hipLaunchKernelGGL(stream_read_kernel, dim3(g), dim3(256), 0, s, reinterpret_cast<const uint4*>(p),
                     n16, sink);
  return hipPeekAtLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t g = (n + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(g > 4096 ? 4096 : g)), dim3(256), 0, s,
                     (uint32_t*)p, n);
  return hipPeekAtLastError();
}

}  // namespace moe
