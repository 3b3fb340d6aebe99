// Single-token (batch 1) decode layer: three kernels per layer.
//
//  K1  router GEMV over all E rows, then top-k + softmax in the last
//      workgroup to finish (completion ticket).  Spare workgroups stream the
//      shared expert's gate/up rows meanwhile: the shared expert does not
//      depend on routing, so it fills the routing bubble (the pages run it on
//      a side stream beside the selected experts: page "AI手搓1.2万行代码榨干
//      GB300!…", section 02; smzdm page, section "四步改造").
//  K2  gate/up GEMVs of the k selected experts with fused MXFP4 dequant and
//      SiLU gating -> fp32 activations; spare workgroups run the shared
//      expert's down projection.
//  K3  down GEMVs of the selected experts, router-weighted combine, shared
//      output and residual add -> bf16.  Each workgroup owns a slab of output
//      rows and reduces its experts in a fixed order (deterministic, no
//      floating-point atomics).
//
// Decode is bound by streaming weights from HBM (page "英伟达用1.2万行CuTe DSL
// Megakernel…", section "解码优化为何比训练优化更难"; tmtpost page, section
// "为什么是解码"), so every kernel reads each weight byte once with 16-byte
// loads, keeps the activation vector in registers or LDS, and decodes MXFP4
// in registers right before the dot product.
//
// Cross-workgroup hand-off (K1's ticket) publishes only values written by
// this launch and reads them after an agent-scope acquire; only static
// weights are ever read ahead of a synchronisation point (the ordering bug
// the pages report came from activation loads moved above a wait: page
// "英伟达用1.2万行CuTe DSL Megakernel…", section "写在最后"; page "AI手搓1.2万行
// 代码榨干GB300!…", section 03).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxH = 8192;

// -------------------------------------------------------------------------
// Activation staging: bf16 x -> LDS as bf16 pairs, optionally RMSNorm'ed.
// Every workgroup computes the identical vector (fixed reduction order).
__device__ void stage_x(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                        float eps, int H, uint32_t* x_lds, float* red,
                        uint16_t* __restrict__ xn_out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint4* x16 = reinterpret_cast<const uint4*>(x);
  uint4* l16 = reinterpret_cast<uint4*>(x_lds);
  const int nch = H / 8;
  if (!gamma) {
    for (int c = tid; c < nch; c += kBlock) l16[c] = x16[c];
    __syncthreads();
    return;
  }
  float ss = 0.f;
  for (int c = tid; c < nch; c += kBlock) {
    const uint4 v = x16[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = bf16_to_f32(w[d] & 0xFFFFu), b = bf16_to_f32(w[d] >> 16);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  const uint4* g16 = reinterpret_cast<const uint4*>(gamma);
  for (int c = tid; c < nch; c += kBlock) {
    const uint4 v = x16[c], g = g16[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = bf16_to_f32(w[d] & 0xFFFFu) * inv * bf16_to_f32(gw[d] & 0xFFFFu);
      const float b = bf16_to_f32(w[d] >> 16) * inv * bf16_to_f32(gw[d] >> 16);
      o[d] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    }
    const uint4 ov = {o[0], o[1], o[2], o[3]};
    l16[c] = ov;
    if (xn_out) reinterpret_cast<uint4*>(xn_out)[c] = ov;
  }
  __syncthreads();
}

// -------------------------------------------------------------------------
// Router rows: one wave per row, 16-byte chunks strided over the lanes.
__device__ void router_rows(const LayerT1& L, const uint32_t* x_lds, int gw, int nw) {
  const int lane = threadIdx.x & 63;
  const int nch = L.H / 8;
  const uint4* xl = reinterpret_cast<const uint4*>(x_lds);
  for (int e = gw; e < L.E; e += nw) {
    const uint4* row = reinterpret_cast<const uint4*>(L.router_w + (size_t)e * L.H);
    float a0 = 0.f, a1 = 0.f;
    for (int base = 0; base < nch; base += 8 * kWave) {
      uint4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = base + i * kWave + lane;
        if (c < nch) v[i] = row[c];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = base + i * kWave + lane;
        if (c < nch) {
          const uint4 xv = xl[c];
          a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].x), as_bf16x2(xv.x), a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].y), as_bf16x2(xv.y), a1, false);
          a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].z), as_bf16x2(xv.z), a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[i].w), as_bf16x2(xv.w), a1, false);
        }
      }
    }
    const float s = wave_sum(a0 + a1);
    if (lane == 0) {
      L.logits[e] = s;
      if (L.logits_out) L.logits_out[e] = s;
    }
  }
}

// Top-k + softmax by one wave.  Keys are (order key of the logit, ~index),
// so the unsigned maximum is the largest logit with the lowest index.
__device__ void topk_softmax_wave(const LayerT1& L) {
  const int lane = threadIdx.x & 63;
  constexpr int kPer = kMaxExperts / kWave;
  uint64_t keys[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = i * kWave + lane;
    keys[i] = 0ull;
    if (e < L.E)
      keys[i] = ((uint64_t)f32_order_key(L.logits[e]) << 32) | (uint64_t)(~(uint32_t)e);
  }
  uint64_t mine = 0ull;
  for (int r = 0; r < L.k; ++r) {
    uint64_t m = keys[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) m = keys[i] > m ? keys[i] : m;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t o = __shfl_xor(m, off, kWave);
      m = o > m ? o : m;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) keys[i] = keys[i] == m ? 0ull : keys[i];
    if (lane == r) mine = m;
  }
  const bool act = lane < L.k;
  const float l = act ? f32_from_order_key((uint32_t)(mine >> 32)) : 0.f;
  const float lmax = __shfl(l, 0, kWave);
  const float ex = act ? expf(l - lmax) : 0.f;
  const float sum = wave_sum(ex);
  if (act) {
    const int e = (int)(~(uint32_t)(mine & 0xFFFFFFFFull));
    const float w = ex / sum;
    L.idx[lane] = e;
    L.wts[lane] = w;
    if (L.idx_out) L.idx_out[lane] = e;
    if (L.w_out) L.w_out[lane] = w;
  }
}

// -------------------------------------------------------------------------
// Gate/up row pairs.  Lanes 0..31 stream gate rows, lanes 32..63 the up rows
// with the same index; `map.lanes` lanes per row, BPL blocks per lane.  x for
// the lane's blocks stays in registers for the whole loop.
template <int BPL>
struct GateUpLanes {
  int half, rig, col, lanes, rph;
  uint32_t xr[BPL][16];

  __device__ void init(const uint32_t* xsrc, int lanes_) {
    const int lane = threadIdx.x & 63;
    lanes = lanes_;
    half = lane >> 5;
    rig = (lane & 31) / lanes;
    col = (lane & 31) % lanes;
    rph = 32 / lanes;
    const uint4* x16 = reinterpret_cast<const uint4*>(xsrc);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = col + lanes * i;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = x16[b * 4 + q];
        xr[i][4 * q + 0] = v.x;
        xr[i][4 * q + 1] = v.y;
        xr[i][4 * q + 2] = v.z;
        xr[i][4 * q + 3] = v.w;
      }
    }
  }
};

struct GateUpJob {
  const uint8_t *g_codes, *g_scales, *u_codes, *u_scales;
  const int32_t* idx;  // expert of each slot (null: expert 0 for every slot)
  int E, H, F;
  float* act;          // [slots][F]
};

template <int BPL>
__device__ __forceinline__ void gateup_load(const GateUpLanes<BPL>& g, const GateUpJob& J,
                                            int slot, int j, uint4 (&c)[BPL],
                                            uint32_t (&sc)[BPL]) {
  int e = J.idx ? J.idx[slot] : 0;
  e = e < 0 ? 0 : (e >= J.E ? J.E - 1 : e);  // never address outside the weights
  const size_t row = (size_t)e * J.F + j;
  const uint8_t* cb = (g.half ? J.u_codes : J.g_codes) + row * (size_t)(J.H / 2);
  const uint8_t* sb = (g.half ? J.u_scales : J.g_scales) + row * (size_t)(J.H / 32);
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = g.col + g.lanes * i;
    c[i] = *reinterpret_cast<const uint4*>(cb + (size_t)b * 16);
    sc[i] = sb[b];
  }
}

template <int BPL>
__device__ void gateup_tasks(GateUpLanes<BPL>& g, const GateUpJob& J, int nslots, int first,
                             int stride) {
  const int tps = J.F / g.rph;  // tasks per slot
  const int ntask = nslots * tps;
  if (first >= ntask) return;
  uint4 c[BPL];
  uint32_t sc[BPL];
  {
    const int s = first / tps;
    gateup_load(g, J, s, (first - s * tps) * g.rph + g.rig, c, sc);
  }
  for (int t = first; t < ntask; t += stride) {
    const int s = t / tps;
    const int j = (t - s * tps) * g.rph + g.rig;
    uint4 cn[BPL];
    uint32_t scn[BPL];
    const int tn = t + stride;
    if (tn < ntask) {
      const int sn = tn / tps;
      gateup_load(g, J, sn, (tn - sn * tps) * g.rph + g.rig, cn, scn);
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < BPL; ++i)
      acc = __builtin_fmaf(block_dot_bf16(c[i], g.xr[i]), e8m0_to_f32(sc[i]), acc);
    acc = group_sum(acc, g.lanes);
    const float up = __shfl_xor(acc, 32, kWave);
    if (g.half == 0 && g.col == 0) J.act[(size_t)s * J.F + j] = silu(acc) * up;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      c[i] = cn[i];
      sc[i] = scn[i];
    }
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
      c[i] = *reinterpret_cast<const uint4*>(cb + (size_t)b * 16);
      sc[i] = sb[b];
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
// K1: router + top-k (+ shared gate/up in the blocks past n_router).
template <int BPLH>
__global__ __launch_bounds__(kBlock) void k1_router_topk(LayerT1 L, int n_router,
                                                         int gu_lanes) {
  __shared__ __align__(16) uint32_t x_lds[kMaxH / 2];
  __shared__ float red[kWaves];
  __shared__ int last_flag;
  const int wid = threadIdx.x >> 6;
  const bool router_block = (int)blockIdx.x < n_router;
  stage_x(L.x, L.gamma, L.eps, L.H, x_lds, red,
          (L.gamma && blockIdx.x == 0) ? L.xn : nullptr);

  if (!router_block) {
    GateUpLanes<BPLH> g;
    g.init(x_lds, gu_lanes);
    GateUpJob J{L.sg_codes, L.sg_scales, L.su_codes, L.su_scales, nullptr, 1, L.H, L.F,
                L.act + (size_t)L.k * L.F};
    const int nw = (gridDim.x - n_router) * kWaves;
    gateup_tasks(g, J, 1, (blockIdx.x - n_router) * kWaves + wid, nw);
    return;
  }

  router_rows(L, x_lds, blockIdx.x * kWaves + wid, n_router * kWaves);
  // publish this block's logits, then take a completion ticket
  fence_release_agent();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(L.ticket, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == (unsigned)n_router - 1u);
  }
  __syncthreads();
  if (!last_flag) return;
  fence_acquire_agent();
  if (wid == 0) {
    topk_softmax_wave(L);
    if (threadIdx.x == 0)
      __hip_atomic_store(L.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// K2: routed gate/up (+ shared down in the blocks past n_gu).
template <int BPLH, int BPLF>
__global__ __launch_bounds__(kBlock) void k2_gateup(LayerT1 L, const uint16_t* __restrict__ x,
                                                    const int32_t* __restrict__ idx,
                                                    float* __restrict__ act, int n_gu,
                                                    int gu_lanes, int dn_lanes) {
  const int wid = threadIdx.x >> 6;
  if ((int)blockIdx.x < n_gu) {
    GateUpLanes<BPLH> g;
    g.init(reinterpret_cast<const uint32_t*>(x), gu_lanes);
    GateUpJob J{L.g_codes, L.g_scales, L.u_codes, L.u_scales, idx, L.E, L.H, L.F, act};
    gateup_tasks(g, J, L.k, blockIdx.x * kWaves + wid, n_gu * kWaves);
    return;
  }
  // shared expert down projection: y_shared[r] = D_s[r] . act_shared
  DownLanes<BPLF> d;
  d.init_map(dn_lanes);
  d.load_act(L.act + (size_t)L.k * L.F);
  const int ngroups = L.H / d.rpw;
  const int nw = (gridDim.x - n_gu) * kWaves;
  for (int rg = (blockIdx.x - n_gu) * kWaves + wid; rg < ngroups; rg += nw) {
    const int row = rg * d.rpw + d.rig;
    uint4 c[BPLF];
    uint32_t sc[BPLF];
    d.load_row(L.sd_codes, L.sd_scales, L.F, row, c, sc);
    const float v = group_sum(d.dot(c, sc), d.lanes);
    if (d.col == 0) L.y_shared[row] = v;
  }
}

// K3: routed down + weighted combine + shared + residual, one slab of rows
// per workgroup; waves take slots w, w + kWaves, ...
constexpr int kMaxGroups = 16;
template <int BPLF>
__global__ __launch_bounds__(kBlock) void k3_down_combine(LayerT1 L, int dn_lanes, int ngroups) {
  __shared__ float red[kWaves][kMaxGroups * kWave];
  const int wid = threadIdx.x >> 6;
  DownLanes<BPLF> d;
  d.init_map(dn_lanes);
  const int R = ngroups * d.rpw;
  const int r0 = blockIdx.x * R;
  float acc[kMaxGroups];
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) acc[g] = 0.f;

  for (int s = wid; s < L.k; s += kWaves) {
    int e = L.idx[s];
    e = e < 0 ? 0 : (e >= L.E ? L.E - 1 : e);
    const float w = L.wts[s];
    d.load_act(L.act + (size_t)s * L.F);
    const uint8_t* codes = L.d_codes + (size_t)e * L.H * (L.F / 2);
    const uint8_t* scales = L.d_scales + (size_t)e * L.H * (L.F / 32);
#pragma unroll
    for (int g0 = 0; g0 < kMaxGroups; g0 += 8) {
      if (g0 >= ngroups) break;
      uint4 c[8][BPLF];
      uint32_t sc[8][BPLF];
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g0 + g < ngroups) d.load_row(codes, scales, L.F, r0 + (g0 + g) * d.rpw + d.rig, c[g], sc[g]);
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g0 + g < ngroups) acc[g0 + g] = __builtin_fmaf(w, d.dot(c[g], sc[g]), acc[g0 + g]);
    }
  }
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) {
    if (g < ngroups) {
      const float v = group_sum(acc[g], d.lanes);
      if (d.col == 0) red[wid][g * d.rpw + d.rig] = v;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < R; t += kBlock) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += red[w][t];
    const int row = r0 + t;
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

template <int BPLH>
hipError_t k1_launch(const LayerT1& L, int n_router, int n_shared, int lanes, hipStream_t s) {
  hipLaunchKernelGGL(k1_router_topk<BPLH>, dim3(n_router + n_shared), dim3(kBlock), 0, s, L,
                     n_router, lanes);
  return hipPeekAtLastError();
}

template <int BPLH, int BPLF>
hipError_t k2_launch(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                     int n_gu, int n_sd, int gl, int dl, hipStream_t s) {
  hipLaunchKernelGGL((k2_gateup<BPLH, BPLF>), dim3(n_gu + n_sd), dim3(kBlock), 0, s, L, x, idx,
                     act, n_gu, gl, dl);
  return hipPeekAtLastError();
}

template <int BPLF>
hipError_t k3_launch(const LayerT1& L, int nblk, int lanes, int ngroups, hipStream_t s) {
  hipLaunchKernelGGL(k3_down_combine<BPLF>, dim3(nblk), dim3(kBlock), 0, s, L, lanes, ngroups);
  return hipPeekAtLastError();
}

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

}  // namespace

hipError_t launch_router_topk_t1(const LayerT1& L, bool with_shared, hipStream_t s) {
  const RowMap gm = gateup_map(L.H);
  const int n_router = ceil_div(L.E, kWaves);
  int n_shared = 0;
  if (with_shared && L.S) {
    const int tasks = L.F / (32 / gm.lanes);
    n_shared = ceil_div(tasks, kWaves * 4);  // about four row pairs per wave
  }
  switch (gm.bpl) {
    case 1: return k1_launch<1>(L, n_router, n_shared, gm.lanes, s);
    case 2: return k1_launch<2>(L, n_router, n_shared, gm.lanes, s);
    case 3: return k1_launch<3>(L, n_router, n_shared, gm.lanes, s);
    case 4: return k1_launch<4>(L, n_router, n_shared, gm.lanes, s);
    case 5: return k1_launch<5>(L, n_router, n_shared, gm.lanes, s);
    case 6: return k1_launch<6>(L, n_router, n_shared, gm.lanes, s);
    case 7: return k1_launch<7>(L, n_router, n_shared, gm.lanes, s);
    case 8: return k1_launch<8>(L, n_router, n_shared, gm.lanes, s);
  }
  return hipErrorInvalidValue;
}

template <int BPLH>
static hipError_t k2_dispatch_f(const LayerT1& L, const uint16_t* x, const int32_t* idx,
                                float* act, int n_gu, int n_sd, int gl, const RowMap& dm,
                                hipStream_t s) {
  switch (dm.bpl) {
    case 1: return k2_launch<BPLH, 1>(L, x, idx, act, n_gu, n_sd, gl, dm.lanes, s);
    case 2: return k2_launch<BPLH, 2>(L, x, idx, act, n_gu, n_sd, gl, dm.lanes, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gateup_t1(const LayerT1& L, const uint16_t* x, const int32_t* idx, float* act,
                            bool with_shared_down, hipStream_t s) {
  const RowMap gm = gateup_map(L.H), dm = down_map(L.F);
  const int tasks = L.k * (L.F / (32 / gm.lanes));
  const int n_gu = ceil_div(tasks, kWaves * 4) < kNumCU * kK2WavesPerCU / kWaves
                       ? ceil_div(tasks, kWaves * 4)
                       : kNumCU * kK2WavesPerCU / kWaves;
  const int n_sd = (with_shared_down && L.S) ? ceil_div(L.H / (kWave / dm.lanes), kWaves * 8) : 0;
  switch (gm.bpl) {
    case 1: return k2_dispatch_f<1>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 2: return k2_dispatch_f<2>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 3: return k2_dispatch_f<3>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 4: return k2_dispatch_f<4>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 5: return k2_dispatch_f<5>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 6: return k2_dispatch_f<6>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 7: return k2_dispatch_f<7>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
    case 8: return k2_dispatch_f<8>(L, x, idx, act, n_gu, n_sd, gm.lanes, dm, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_combine_t1(const LayerT1& L, hipStream_t s) {
  const RowMap dm = down_map(L.F);
  const int rpw = kWave / dm.lanes;
  // rows per workgroup: a power of two (divides H), aiming at >= 512 blocks
  int ngroups = kMaxGroups;
  while (ngroups > 1 && L.H / (ngroups * rpw) < 448) ngroups >>= 1;
  const int nblk = L.H / (ngroups * rpw);
  switch (dm.bpl) {
    case 1: return k3_launch<1>(L, nblk, dm.lanes, ngroups, s);
    case 2: return k3_launch<2>(L, nblk, dm.lanes, ngroups, s);
  }
  return hipErrorInvalidValue;
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
