// Single-token (batch 1) decode layer: four kernels per layer, one stream.
//
//  K1a router GEMV over all E rows (one wave per row, every load of the row
//      in flight at once).  Spare workgroups stream the shared expert's
//      gate/up rows: the shared expert does not depend on routing (the pages
//      run it beside the selected experts: page "AI手搓1.2万行代码榨干GB300!…",
//      section 02; smzdm page, section "四步改造").
//  K1b top-k + softmax in workgroup 0 (radix select); the other workgroups run
//      the shared expert's down projection, so the selection latency is
//      spent under shared-expert bytes.
//  K2  gate/up GEMVs of the k selected experts with fused MXFP4 dequant and
//      SiLU gating -> fp32 activations.
//  K3  down GEMVs of the selected experts, router-weighted combine with the
//      shared output (weight 1) and residual add -> bf16.  One 16-wave
//      workgroup per CU owns a slab of output rows, wave w streams slot w's
//      rows of the slab, and the slots are summed in LDS in a fixed order
//      (deterministic, no floating-point atomics).
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

// -------------------------------------------------------------------------
// Router rows: one wave per row; the row's 16-byte chunks are strided over
// the lanes and every chunk is requested before the first dot product.  The
// loop always covers kMaxChunks chunks so that no load is conditional:
// chunks past the row end load the row's last chunk again (in bounds) and
// meet the zero padding of x in LDS.
__device__ void router_rows(const LayerT1& L, const uint32_t* x_lds, int gw, int nw) {
  const int lane = threadIdx.x & 63;
  const int nch = L.H / 8;
  const uint4* xl = reinterpret_cast<const uint4*>(x_lds);
  for (int e = gw; e < L.E; e += nw) {
    const uint8_t* row = reinterpret_cast<const uint8_t*>(L.router_w + (size_t)e * L.H);
    uint4 v[kMaxChunks / kWave];
#pragma unroll
    for (int i = 0; i < kMaxChunks / kWave; ++i) {
      const int c = i * kWave + lane;
      v[i] = ld_stream16(row + (size_t)(c < nch ? c : nch - 1) * 16);
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks / kWave; ++i) {
      const uint4 xv = xl[i * kWave + lane];
      a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].x), as_bf16x2(xv.x), a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].y), as_bf16x2(xv.y), a1, false);
      a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].z), as_bf16x2(xv.z), a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].w), as_bf16x2(xv.w), a1, false);
    }
    const float s = group_sum_last(a0 + a1, kWave);
    if (lane == kWave - 1) {
      L.logits[e] = s;
      if (L.logits_out) L.logits_out[e] = s;
    }
  }
}

// -------------------------------------------------------------------------
// Gate/up row pairs.  Lanes 0..31 stream gate rows, lanes 32..63 the up rows
// with the same index; `lanes` lanes per row (8, 16 or 32), BPL blocks per
// lane, 32/lanes rows per half wave.  A task is one such group of row pairs.
// x comes from LDS, so the registers hold only weights in flight: every
// wave keeps two tasks' loads outstanding (static double buffer).
struct GateUpJob {
  const uint8_t *g_codes, *g_scales, *u_codes, *u_scales;
  const int32_t* e_lds;  // expert of each slot, in LDS (null: expert 0)
  int H, F;
  float* act;            // [slots][F]
};

template <int BPL>
struct GateUp {
  int half, rig, col, lanes, rph, tps;

  __device__ void init(int lanes_, int F) {
    const int lane = threadIdx.x & 63;
    lanes = lanes_;
    half = lane >> 5;
    rig = (lane & 31) / lanes;
    col = (lane & 31) % lanes;
    rph = 32 / lanes;
    tps = F / rph;
  }
  __device__ __forceinline__ void load(const GateUpJob& J, int t, uint4 (&c)[BPL],
                                       uint32_t (&sc)[BPL]) const {
    const int s = t / tps;
    const int j = (t - s * tps) * rph + rig;
    const int e = J.e_lds ? J.e_lds[s] : 0;
    const size_t row = (size_t)e * J.F + j;
    const uint8_t* cb = (half ? J.u_codes : J.g_codes) + row * (size_t)(J.H / 2);
    const uint8_t* sb = (half ? J.u_scales : J.g_scales) + row * (size_t)(J.H / 32);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = col + lanes * i;
      c[i] = ld_stream16(cb + (size_t)b * 16);
      sc[i] = ld_stream8(sb + b);
    }
  }
  __device__ __forceinline__ void finish(const GateUpJob& J, const uint32_t* x_lds, int t,
                                         const uint4 (&c)[BPL], const uint32_t (&sc)[BPL]) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const uint4* xl = reinterpret_cast<const uint4*>(x_lds) + (col + lanes * i) * 4;
      uint32_t xv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = xl[q];
        xv[4 * q + 0] = v.x;
        xv[4 * q + 1] = v.y;
        xv[4 * q + 2] = v.z;
        xv[4 * q + 3] = v.w;
      }
      acc = __builtin_fmaf(block_dot_bf16(c[i], xv), e8m0_to_f32(sc[i]), acc);
    }
    acc = group_sum_last(acc, lanes);
    const float up = __shfl_xor(acc, 32, kWave);
    if (half == 0 && col == lanes - 1) {
      const int s = t / tps;
      const int j = (t - s * tps) * rph + rig;
      J.act[(size_t)s * J.F + j] = silu(acc) * up;
    }
  }
};

template <int BPL>
__device__ void gateup_tasks(const GateUp<BPL>& g, const GateUpJob& J, const uint32_t* x_lds,
                             int ntask, int first, int stride) {
  uint4 ca[BPL], cb[BPL];
  uint32_t sa[BPL], sb[BPL];
  int t = first;
  if (t < ntask) g.load(J, t, ca, sa);
  while (t < ntask) {
    const int t1 = t + stride;
    if (t1 < ntask) g.load(J, t1, cb, sb);
    g.finish(J, x_lds, t, ca, sa);
    if (t1 >= ntask) break;
    const int t2 = t1 + stride;
    if (t2 < ntask) g.load(J, t2, ca, sa);
    g.finish(J, x_lds, t1, cb, sb);
    t = t2;
  }
}

// -------------------------------------------------------------------------
// Down rows of one matrix D[H][F] against fp32 activations held in
// registers; `lanes` lanes per row, BPL blocks per lane, 64/lanes rows per
// load instruction.
template <int BPL>
struct DownLanes {
  int rig, col, lanes, rpw;
  float ar[BPL][32];

  __device__ void init_map(int lanes_) {
    const int lane = threadIdx.x & 63;
    lanes = lanes_;
    rig = lane / lanes;
    col = lane % lanes;
    rpw = kWave / lanes;
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
  __device__ __forceinline__ void load_row(const uint8_t* codes, const uint8_t* scales, int F,
                                           int row, uint4 (&c)[BPL], uint32_t (&sc)[BPL]) const {
    const uint8_t* cb = codes + (size_t)row * (F / 2);
    const uint8_t* sb = scales + (size_t)row * (F / 32);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = col + lanes * i;
      c[i] = ld_stream16(cb + (size_t)b * 16);
      sc[i] = ld_stream8(sb + b);
    }
  }
  __device__ __forceinline__ float dot(const uint4 (&c)[BPL], const uint32_t (&sc)[BPL]) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < BPL; ++i)
      acc = __builtin_fmaf(block_dot_f32(c[i], ar[i]), e8m0_to_f32(sc[i]), acc);
    return acc;
  }
};

// -------------------------------------------------------------------------
// K1a: router rows (+ shared gate/up in the workgroups past n_router).
template <int BPLH>
__global__ __launch_bounds__(kBlock) void k1_router(LayerT1 L, int n_router, int gu_lanes) {
  __shared__ __align__(16) uint32_t x_lds[kMaxH / 2];
  __shared__ float red[kWaves];
  const int wid = wave_id();
  stage_x(L.x, L.gamma, L.eps, L.H, x_lds, red,
          (L.gamma && blockIdx.x == 0) ? L.xn : nullptr);
  if ((int)blockIdx.x < n_router) {
    router_rows(L, x_lds, blockIdx.x * kWaves + wid, n_router * kWaves);
    return;
  }
  GateUp<BPLH> g;
  g.init(gu_lanes, L.F);
  const GateUpJob J{L.sg_codes, L.sg_scales, L.su_codes, L.su_scales, nullptr, L.H, L.F,
                    L.act + (size_t)L.k * L.F};
  gateup_tasks(g, J, x_lds, g.tps, (blockIdx.x - n_router) * kWaves + wid,
               (gridDim.x - n_router) * kWaves);
}

// K1b: top-k + softmax in workgroup 0; shared down rows -> y_shared in the
// others, kRowsK1b row groups per wave with all loads in flight.
constexpr int kRowsK1b = 8;
template <int BPLF>
__global__ __launch_bounds__(kBlock) void k1_topk(LayerT1 L, int dn_lanes) {
  __shared__ TopkLds tk;
  if (blockIdx.x == 0) {
    float lg[kTopkPerThread];
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) {
      const int e = threadIdx.x * kTopkPerThread + i;
      lg[i] = L.logits[e < L.E ? e : L.E - 1];
    }
    topk_softmax_block(lg, L.E, L.k, tk, L.idx, L.wts, L.idx_out, L.w_out);
    return;
  }
  const int wid = wave_id();
  DownLanes<BPLF> d;
  d.init_map(dn_lanes);
  d.load_act(L.act + (size_t)L.k * L.F);
  const int ngroups = L.H / d.rpw;
  const int g0 = ((blockIdx.x - 1) * kWaves + wid) * kRowsK1b;
  uint4 c[kRowsK1b][BPLF];
  uint32_t sc[kRowsK1b][BPLF];
#pragma unroll
  for (int j = 0; j < kRowsK1b; ++j) {
    const int g = g0 + j < ngroups ? g0 + j : ngroups - 1;
    d.load_row(L.sd_codes, L.sd_scales, L.F, g * d.rpw + d.rig, c[j], sc[j]);
  }
  float v[kRowsK1b];
#pragma unroll
  for (int j = 0; j < kRowsK1b; ++j) v[j] = d.dot(c[j], sc[j]);
#pragma unroll
  for (int j = 0; j < kRowsK1b; ++j) v[j] = group_sum_last(v[j], d.lanes);
#pragma unroll
  for (int j = 0; j < kRowsK1b; ++j)
    if (g0 + j < ngroups && d.col == d.lanes - 1) L.y_shared[(g0 + j) * d.rpw + d.rig] = v[j];
}

// K2: routed gate/up of the k selected experts.
template <int BPLH>
__global__ __launch_bounds__(kBlock) void k2_gateup(LayerT1 L, const uint16_t* __restrict__ x,
                                                    const int32_t* __restrict__ idx,
                                                    float* __restrict__ act, int gu_lanes) {
  __shared__ __align__(16) uint32_t x_lds[kMaxH / 2];
  __shared__ int32_t e_lds[kMaxTopK];
  const int wid = wave_id();
  if (threadIdx.x < L.k) {
    const int e = idx[threadIdx.x];
    e_lds[threadIdx.x] = e < 0 ? 0 : (e >= L.E ? L.E - 1 : e);  // never address outside
  }
  stage_x(x, nullptr, 0.f, L.H, x_lds, nullptr, nullptr);
  GateUp<BPLH> g;
  g.init(gu_lanes, L.F);
  const GateUpJob J{L.g_codes, L.g_scales, L.u_codes, L.u_scales, e_lds, L.H, L.F, act};
  gateup_tasks(g, J, x_lds, L.k * g.tps, blockIdx.x * kWaves + wid, gridDim.x * kWaves);
}

// K3: one workgroup of kK3Waves waves per row slab of `gpb` row groups.  Wave
// w streams the slab's rows of slots w, w + kK3Waves, ... (activations of the
// slot held in registers) and adds each weighted row result to its own LDS
// partial; the waves' partials are then added in wave order together with
// the shared output and the residual.
constexpr int kK3Waves = 8;
constexpr int kK3Block = kK3Waves * kWave;
constexpr int kK3MaxRows = 64;
constexpr int kK3SlabsPerCU = 2;
template <int BPLF>
__global__ __launch_bounds__(kK3Block) void k3_down_combine(LayerT1 L, int dn_lanes, int gpb) {
  __shared__ float red[kK3Waves][kK3MaxRows];
  __shared__ int32_t e_lds[kMaxTopK];
  __shared__ float w_lds[kMaxTopK];
  constexpr int NB = 8 / BPLF;  // row groups per burst of loads
  const int wid = wave_id(), lane = threadIdx.x & 63;
  DownLanes<BPLF> d;
  d.init_map(dn_lanes);
  const int ngroups = L.H / d.rpw;
  const int gbase = blockIdx.x * gpb;
  const int ng = ngroups - gbase < gpb ? ngroups - gbase : gpb;  // groups of this slab
  const int R = ng * d.rpw;
  for (int t = lane; t < R; t += kWave) red[wid][t] = 0.f;
  if (threadIdx.x < L.k) {
    const int e = L.idx[threadIdx.x];
    e_lds[threadIdx.x] = e < 0 ? 0 : (e >= L.E ? L.E - 1 : e);
    w_lds[threadIdx.x] = L.wts[threadIdx.x];
  }
  __syncthreads();

  for (int s = wid; s < L.k; s += kK3Waves) {
    const int e = e_lds[s];
    const float w = w_lds[s];
    const uint8_t* codes = L.d_codes + (size_t)e * L.H * (L.F / 2);
    const uint8_t* scales = L.d_scales + (size_t)e * L.H * (L.F / 32);
    d.load_act(L.act + (size_t)s * L.F);
    for (int g0 = 0; g0 < ng; g0 += NB) {
      uint4 c[NB][BPLF];
      uint32_t sc[NB][BPLF];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int g = g0 + j < ng ? g0 + j : ng - 1;
        d.load_row(codes, scales, L.F, (gbase + g) * d.rpw + d.rig, c[j], sc[j]);
      }
      float v[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) v[j] = d.dot(c[j], sc[j]);
#pragma unroll
      for (int j = 0; j < NB; ++j) v[j] = group_sum_last(v[j], d.lanes);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (g0 + j < ng && d.col == d.lanes - 1) red[wid][(g0 + j) * d.rpw + d.rig] += w * v[j];
    }
  }
  __syncthreads();
  const int nwk = L.k < kK3Waves ? L.k : kK3Waves;
  for (int t = threadIdx.x; t < R; t += kK3Block) {
    float tot = 0.f;
    for (int v = 0; v < nwk; ++v) tot += red[v][t];
    const int row = gbase * d.rpw + t;
    if (L.S) tot += L.y_shared[row];
    if (L.residual) tot += bf16_to_f32(L.residual[row]);
    const uint16_t o = f32_to_bf16(tot);
    L.out[row] = o;
    if (L.trace) L.trace[row] = o;
  }
}

// ---------------------------------------------------------------- dispatch
constexpr int kK2WavesPerCU = 8;
constexpr int kNumCU = 256;

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

template <int B>
hipError_t k1a_launch(const LayerT1& L, int n_router, int n_shared, int lanes, hipStream_t s) {
  hipLaunchKernelGGL(k1_router<B>, dim3(n_router + n_shared), dim3(kBlock), 0, s, L, n_router,
                     lanes);
  return hipPeekAtLastError();
}

template <int B>
hipError_t k2_launch(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                     int n_gu, int lanes, hipStream_t s) {
  hipLaunchKernelGGL(k2_gateup<B>, dim3(n_gu), dim3(kBlock), 0, s, L, x, idx, act, lanes);
  return hipPeekAtLastError();
}

}  // namespace

hipError_t launch_router_t1(const LayerT1& L, bool with_shared, hipStream_t s) {
  const RowMap gm = gateup_map(L.H);
  const int n_router = ceil_div(L.E, kWaves);
  int n_shared = 0;
  if (with_shared && L.S) {
    const int tasks = L.F / (32 / gm.lanes);
    n_shared = ceil_div(tasks, kWaves * 2);  // about two row pairs per wave
  }
  switch (gm.bpl) {
    case 1: return k1a_launch<1>(L, n_router, n_shared, gm.lanes, s);
    case 2: return k1a_launch<2>(L, n_router, n_shared, gm.lanes, s);
    case 3: return k1a_launch<3>(L, n_router, n_shared, gm.lanes, s);
    case 4: return k1a_launch<4>(L, n_router, n_shared, gm.lanes, s);
    case 5: return k1a_launch<5>(L, n_router, n_shared, gm.lanes, s);
    case 6: return k1a_launch<6>(L, n_router, n_shared, gm.lanes, s);
    case 7: return k1a_launch<7>(L, n_router, n_shared, gm.lanes, s);
    case 8: return k1a_launch<8>(L, n_router, n_shared, gm.lanes, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk_t1(const LayerT1& L, bool with_shared, hipStream_t s) {
  const RowMap dm = down_map(L.F);
  int n_sd = 0;
  if (with_shared && L.S) n_sd = ceil_div(L.H / (kWave / dm.lanes), kWaves * kRowsK1b);
  if (dm.bpl == 1)
    hipLaunchKernelGGL(k1_topk<1>, dim3(1 + n_sd), dim3(kBlock), 0, s, L, dm.lanes);
  else if (dm.bpl == 2)
    hipLaunchKernelGGL(k1_topk<2>, dim3(1 + n_sd), dim3(kBlock), 0, s, L, dm.lanes);
  else
    return hipErrorInvalidValue;
  return hipPeekAtLastError();
}

hipError_t launch_gateup_t1(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                            hipStream_t s) {
  const RowMap gm = gateup_map(L.H);
  const int tasks = L.k * (L.F / (32 / gm.lanes));
  const int cap = kNumCU * kK2WavesPerCU / kWaves;
  const int n_gu = ceil_div(tasks, kWaves * 4) < cap ? ceil_div(tasks, kWaves * 4) : cap;
  switch (gm.bpl) {
    case 1: return k2_launch<1>(L, x, idx, act, n_gu, gm.lanes, s);
    case 2: return k2_launch<2>(L, x, idx, act, n_gu, gm.lanes, s);
    case 3: return k2_launch<3>(L, x, idx, act, n_gu, gm.lanes, s);
    case 4: return k2_launch<4>(L, x, idx, act, n_gu, gm.lanes, s);
    case 5: return k2_launch<5>(L, x, idx, act, n_gu, gm.lanes, s);
    case 6: return k2_launch<6>(L, x, idx, act, n_gu, gm.lanes, s);
    case 7: return k2_launch<7>(L, x, idx, act, n_gu, gm.lanes, s);
    case 8: return k2_launch<8>(L, x, idx, act, n_gu, gm.lanes, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_combine_t1(const LayerT1& L, hipStream_t s) {
  const RowMap dm = down_map(L.F);
  const int ngroups = L.H / (kWave / dm.lanes);
  const int gpb = ceil_div(ngroups, kNumCU * kK3SlabsPerCU);
  const int nblk = ceil_div(ngroups, gpb);
  if (gpb * (kWave / dm.lanes) > kK3MaxRows) return hipErrorInvalidValue;
  if (dm.bpl == 1)
    hipLaunchKernelGGL(k3_down_combine<1>, dim3(nblk), dim3(kK3Block), 0, s, L, dm.lanes, gpb);
  else if (dm.bpl == 2)
    hipLaunchKernelGGL(k3_down_combine<2>, dim3(nblk), dim3(kK3Block), 0, s, L, dm.lanes, gpb);
  else
    return hipErrorInvalidValue;
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
