// Batched decode layer (2 <= T <= 64 tokens): six kernels on one stream
// (eight when the shared expert's FFN width differs from the routed
// experts': its group then runs its own gate/up and down launches).
//
//  router   logits of all T tokens as bf16 MFMA tiles (16 experts x 16
//           tokens per fragment), the reduction dimension split KS ways;
//           partial sums go to the workspace.
//  topk     one workgroup per token: adds the KS partials in a fixed order,
//           stages the logits in LDS, then one wave runs the top-k +
//           softmax shared with the single-token path.
//  group    one workgroup: a 64-bit token mask per expert gives each
//           (token, slot) pair its stable rank inside its expert, hence a
//           counting sort of the pairs by expert (pairs of an expert ordered
//           by token), and the list of active experts; the shared expert is
//           appended as one more group holding every token.
//  gateup   grouped GEMM per (group, 16-row tile): A = 16 gate rows and 16 up
//           rows, MXFP4 decoded to exact bf16 in registers; B = the group's
//           token activations (bf16), one or two 16-token tiles per pass over
//           the weights; fp32 accumulation; SiLU gating in the epilogue.
//           The gated activation a is stored as two bf16 parts,
//           a_hi = bf16(a) and a_lo = bf16(a - a_hi), so that the down GEMM
//           keeps ~16 significant bits of a on bf16 MFMA.
//  down     grouped GEMM per (group, 16-row tile of the hidden size) over
//           a_hi and a_lo -> fp32 expert outputs per sorted pair; at FFN
//           2048 each wave runs its units as one chunk stream
//           (kb_down_flat; kb_down_w8 for batches of at most 8 tokens).
//  combine  per token: residual + sum_j w_j y_j (slot order) + y_shared ->
//           bf16; fixed order, no floating-point atomics.
//
// At batch 64 the selected experts are shared by several tokens (skewed
// routing puts up to ~30 tokens on one expert, and the shared expert sees
// all of them), so gate/up and down are real contractions and run on MFMA
// (the pages' size-specialised kernels for larger batches: smzdm page,
// section "四步改造"; the pages' fast path stops at 64 tokens: page "AI手搓
// 1.2万行代码榨干GB300!…", section 03).  Weight bytes still dominate, so the
// grouped kernels keep consecutive waves on consecutive row tiles of one
// expert, request each chunk two chunks ahead with 16-byte buffer loads,
// request a tile's scales once per work item (chunk by chunk, the weight
// stream evicted the scale lines between uses), and keep the count of
// requests per chunk low (no staging requests for token rows past the
// group).  The operand layout covers 64 bytes of each of 16 rows per wave
// instruction (the next request completes the line through L2); where LDS
// allows (one-tile gate/up passes, the down kernel at up to 8 tokens) the
// weights are requested instead as 4 rows x 256 bytes, nontemporal, and
// moved to the operand layout through a wave-private LDS tile.
//
// MFMA v_mfma_f32_16x16x32_bf16 fragments (lane l = 16 q + r): A holds
// A[r][8q .. 8q+7], B holds B[8q .. 8q+7][r], the result C[4q .. 4q+3][r].
// The reduction index is permuted consistently in A and B: for a 128-wide
// step, lane group q owns MXFP4 block q of the step (one 16-byte load) and
// MFMA s of the step takes elements 8s .. 8s+7 of that block.
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_topk.h"

#include <type_traits>

namespace moe {
namespace {


constexpr int kBlk = 256;
constexpr int kWv = kBlk / kWave;
constexpr int kGroupBlock = 1024;
constexpr int kTileRows = 16;
constexpr int kMaxRouterSplits = 16;

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Inclusive scan over a workgroup of kGroupBlock threads (16 waves).  The
// wave totals are read back all at once and masked, rather than in a loop of
// wid dependent LDS reads (the last wave's 15 reads were most of a scan).
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  constexpr int NW = kGroupBlock / kWave;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == kWave - 1) wsum[wid] = inc;
  __syncthreads();
  uint32_t before = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) before += w < wid ? wsum[w] : 0u;
  __syncthreads();
  return before + inc;
}

// ---------------------------------------------------------------- router
// One wave per (16-expert tile, K split); KS splits of H, each a multiple of
// 128, walked 128 elements (four MFMA steps) at a time with all loads of the
// step issued first.  Tokens past T and experts past E read in-bounds
// neighbours whose results are dropped.
__global__ __launch_bounds__(kBlk) void kb_router(LayerTB L, int n_et) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15;
  const int w = blockIdx.x * kWv + wave_id();
  const int et = w % n_et, ks = w / n_et;
  if (ks >= L.KS) return;
  const int Kc = L.H / L.KS;
  const int k0 = ks * Kc;
  const int NT = (L.T + 15) / 16;
  const int erow = et * kTileRows + r < L.E ? et * kTileRows + r : L.E - 1;
  const uint8_t* arow = reinterpret_cast<const uint8_t*>(L.router_w + (size_t)erow * L.H);
  const uint8_t* brow[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = nt * 16 + r < L.T ? nt * 16 + r : L.T - 1;
    brow[nt] = reinterpret_cast<const uint8_t*>(L.x + (size_t)t * L.H);
  }
  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = k0; kk < k0 + Kc; kk += 128) {
    uint4 a[4], b[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = ld_stream16(arow + (size_t)(kk + 32 * s + 8 * q) * 2);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (nt < NT) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          b[nt][s] = *reinterpret_cast<const uint4*>(brow[nt] + (size_t)(kk + 32 * s + 8 * q) * 2);
      }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (nt < NT) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[nt] = mfma16(as_bf16x8(a[s]), as_bf16x8(b[nt][s]), acc[nt]);
      }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = nt * 16 + r;
    if (nt < NT && t < L.T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = et * kTileRows + 4 * q + i;
        if (e < L.E) L.part[((size_t)ks * L.T + t) * L.E + e] = acc[nt][i];
      }
    }
  }
}

// ---------------------------------------------------------------- top-k
// V4 (E % 4 == 0): thread t requests experts 4 t .. 4 t + 3 of every split
// as one 16-byte load (a wave's request is 1 KB contiguous), and wave 0 reads
// its lanes' 16 logits back as four 16-byte LDS reads.  Scalar loads at a
// 16-byte lane stride cost a vector-memory instruction per expert and split,
// and 16 scalar LDS reads at a 64-byte lane stride conflict on the banks.
template <bool V4>
__global__ __launch_bounds__(kTopkBlock) void kb_topk(LayerTB L) {
  static_assert(kTopkPerThread == 4, "a thread's four logits are one 16-byte piece");
  __shared__ TopkLds tk;
  __shared__ __align__(16) float lg_lds[kMaxExperts];
  const int t = blockIdx.x;
  // all partial loads first (split index clamped, extra splits ignored), then
  // the sums in split order
  float v[kMaxRouterSplits][kTopkPerThread];
  const int e0 = threadIdx.x * kTopkPerThread;
  if constexpr (V4) {
    const int eb = e0 + 4 <= L.E ? e0 : L.E - 4;  // in bounds; threads past E are ignored
#pragma unroll
    for (int ks = 0; ks < kMaxRouterSplits; ++ks) {
      const int kc = ks < L.KS ? ks : L.KS - 1;
      const float4 f = *reinterpret_cast<const float4*>(L.part + ((size_t)kc * L.T + t) * L.E + eb);
      v[ks][0] = f.x;
      v[ks][1] = f.y;
      v[ks][2] = f.z;
      v[ks][3] = f.w;
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < kMaxRouterSplits; ++ks) {
      const int kc = ks < L.KS ? ks : L.KS - 1;
#pragma unroll
      for (int i = 0; i < kTopkPerThread; ++i) {
        const int e = e0 + i;
        v[ks][i] = L.part[((size_t)kc * L.T + t) * L.E + (e < L.E ? e : L.E - 1)];
      }
    }
  }
  float lg[kTopkPerThread];
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) {
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < kMaxRouterSplits; ++ks) s += ks < L.KS ? v[ks][i] : 0.f;
    lg[i] = s;
    const int e = e0 + i;
    if (L.logits_out && e < L.E) L.logits_out[(size_t)t * L.E + e] = s;
  }
  // the selection by one wave (as for a single token): logits through LDS,
  // lane l taking experts 16 l .. 16 l + 15; no barrier inside
  *reinterpret_cast<float4*>(&lg_lds[e0]) = make_float4(lg[0], lg[1], lg[2], lg[3]);
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    uint32_t key[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(&lg_lds[16 * lane + 4 * j]);
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // a mask, not a branch, so the reads stay 16 bytes wide
        const int e = 16 * lane + 4 * j + i;
        key[4 * j + i] = f32_order_key(fv[i]) & (0u - (uint32_t)(e < L.E));
      }
    }
    const size_t o = (size_t)t * L.k;
    int32_t* io = L.idx_out ? L.idx_out + o : nullptr;
    float* wo = L.w_out ? L.w_out + o : nullptr;
    if (!topk_softmax_wave(key, L.E, L.k, tk, L.idx + o, L.wts + o, io, wo))
      topk_softmax_wave_rounds(key, L.E, L.k, L.idx + o, L.wts + o, io, wo);  // many ties
  }
}

// ---------------------------------------------------------------- group
// Stable counting sort of the T k pairs by expert.  Each token's k experts
// are distinct (top-k output), so the rank of pair (t, j) among the pairs of
// expert e is the number of tokens below t that chose e: a popcount of the
// expert's token mask.  (For caller-supplied indices that repeat an expert
// within a token the grouping is unspecified, but every position stays in
// bounds.)
__global__ __launch_bounds__(kGroupBlock) void kb_group(LayerTB L) {
  constexpr int PPT = (kMaxTokens * kMaxTopK + kGroupBlock - 1) / kGroupBlock;  // pairs per thread
  __shared__ uint32_t s_mask[kMaxExperts][2];
  __shared__ int s_off[kMaxExperts];
  __shared__ __align__(16) uint32_t s_wsum[kGroupBlock / kWave];
  const int tid = threadIdx.x;
  const int P = L.T * L.k;
  s_mask[tid][0] = 0u;
  s_mask[tid][1] = 0u;
  // this thread's pairs tid, tid + kGroupBlock, ...: their experts stay in
  // registers for the placement below
  int pe[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int p = tid + j * kGroupBlock;
    const int e = p < P ? L.idx[p] : 0;
    pe[j] = e < 0 ? 0 : (e >= L.E ? L.E - 1 : e);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int p = tid + j * kGroupBlock;
    if (p < P) {
      const int t = p / L.k;
      atomicOr(&s_mask[pe[j]][t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  const int cnt = tid < L.E ? __popc(s_mask[tid][0]) + __popc(s_mask[tid][1]) : 0;
  const int act = cnt > 0 ? 1 : 0;
  const int npass = (cnt + 15) / 16;  // passes of at most 16 pairs
  // pair offsets (<= 2048) and active-group counts (<= 1024) in one scan
  const uint32_t oa = block_incl_scan((uint32_t)cnt | ((uint32_t)act << 16), s_wsum);
  const int off_incl = (int)(oa & 0xFFFFu), act_incl = (int)(oa >> 16);
  const int pass_incl = (int)block_incl_scan((uint32_t)npass, s_wsum);
  const int off = off_incl - cnt;
  s_off[tid] = off;
  if (act) {
    const int a = act_incl - 1;
    L.g_expert[a] = tid;
    L.g_start[a] = off;
    L.g_count[a] = cnt;
    if (L.pass_group)
      for (int q = 0; q < npass; ++q) {
        L.pass_group[pass_incl - npass + q] = a;
        L.pass_n0[pass_incl - npass + q] = 16 * q;
      }
  }
  if (L.offsets_out && tid < L.E) L.offsets_out[tid] = off;
  if (tid == kGroupBlock - 1) {
    const int nact = act_incl;
    L.ginfo[0] = nact + L.S;
    if (L.S) {
      L.g_expert[nact] = L.E;
      L.g_start[nact] = P;
      L.g_count[nact] = L.T;
    }
    if (L.pass_group) {
      const int nps = L.S ? (L.T + 15) / 16 : 0;  // the shared group's passes
      for (int q = 0; q < nps; ++q) {
        L.pass_group[pass_incl + q] = nact;
        L.pass_n0[pass_incl + q] = 16 * q;
      }
      L.ginfo[1] = pass_incl;
      L.ginfo[2] = pass_incl + nps;
    }
    if (L.offsets_out) L.offsets_out[L.E] = off_incl;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int p = tid + j * kGroupBlock;
    if (p < P) {
      const int e = pe[j];
      const int t = p / L.k;
      const uint32_t m0 = s_mask[e][0], m1 = s_mask[e][1];
      const int below = t < 32 ? __popc(m0 & ((1u << t) - 1u))
                               : __popc(m0) + __popc(m1 & ((1u << (t - 32)) - 1u));
      int pos = s_off[e] + below;
      pos = pos < P ? pos : P - 1;
      L.order[pos] = p;
      L.pos_of[p] = pos;
      if (L.pairs_out) L.pairs_out[pos] = p;
    }
  }
  if (L.S)
    for (int t = tid; t < L.T; t += kGroupBlock) L.order[P + t] = P + t;
}

// Groups [g0, g1) that a grouped gate/up or down launch covers (gmode).
__device__ __forceinline__ void group_range(const LayerTB& L, int& g0, int& g1) {
  const int ng = ld_uniform(L.ginfo);  // grouping tables: scalar loads
  g0 = L.gmode == 2 ? ng - 1 : 0;
  g1 = L.gmode == 1 ? ng - L.S : ng;
}

// Passes [v0, v1) that a down launch covers (gmode, as group_range).
__device__ __forceinline__ void pass_range(const LayerTB& L, int& v0, int& v1) {
  const int nr = ld_uniform(L.ginfo + 1), na = ld_uniform(L.ginfo + 2);
  v0 = L.gmode == 2 ? nr : 0;
  v1 = L.gmode == 1 ? nr : na;
}

// Rows of the activation planes a launch reads: every pair, the routed
// pairs alone (their own planes when the shared expert has its own width),
// or the shared pairs alone (rows pos0 ..).
__device__ __forceinline__ uint32_t act_rows(const LayerTB& L) {
  const int P = L.T * L.k;
  return (uint32_t)((L.gmode == 1 ? P : P + L.S * L.T) - L.pos0);
}

// Token of a sorted pair id: routed pairs are t k + j, shared pairs P + t.
__device__ __forceinline__ int token_of(const LayerTB& L, int pid) {
  const int P = L.T * L.k;
  int t = pid < P ? pid / L.k : pid - P;
  return t < 0 ? 0 : (t >= L.T ? L.T - 1 : t);
}

// ---------------------------------------------------------------- gate/up
// Workgroup items (group, 4 consecutive 16-row tiles) in group-major order, so
// the workgroups running together read consecutive rows of one expert.  The
// four waves share the group's tokens: per K chunk of KC elements the
// workgroup stages up to 32 tokens' activations in LDS (two 16-token MFMA
// tiles; rows padded by 16 bytes so that the 16 lanes of a ds_read_b128 phase
// hit distinct banks), double buffered; each wave streams its own 16 gate and
// 16 up rows in registers (two statically named register sets) and multiplies
// each decoded weight fragment into both tiles.  A group of m tokens thus
// streams its weights ceil(m / 32) times (with skewed routing the hot experts
// hold 17..32 tokens; only the shared expert's group, which holds every
// token, exceeds 32 at batch 64).  When a pass holds 16 tokens or fewer the
// second tile is neither staged (empty descriptor) nor multiplied (a
// workgroup-uniform branch around products only).
//
// Pipeline of chunk c (one barrier per chunk): products of chunk c, then
// the requests for chunk c + 2 (token activations into staging registers,
// then weights into the set chunk c used), then chunk c + 1's activations,
// requested one chunk earlier, go to LDS.  Scheduling fences keep the
// requests in this order (the wait counter completes them in order).  Every wait is thus for requests
// a whole chunk old, never for the ones just issued.  Requests past the
// last chunk re-read the last one (in bounds, unused), so that no load sits
// under a branch.
template <int KC>
struct TokLds {
  uint4 b[2][16][KC / 8 + 1];
};
template <int KC>
struct TokLds2 {  // two 16-token tiles per buffer
  uint4 b[2][32][KC / 8 + 1];
};

template <int KC>
struct GuRegs {
  uint4 ag[KC / 128], au[KC / 128];
  uint32_t sg, su;  // scale dwords (see ld_tile), when not preloaded
};
// A tile's scale dwords for every chunk (NCH fixed at compile time): entry c
// is what ld_tile would request for chunk c.  Requested once per work item.
template <int NCH>
struct TileScales {
  uint32_t g[NCH > 0 ? NCH : 1], u[NCH > 0 ? NCH : 1];
};

// A wave's 16-row MXFP4 weight tile: codes [16][rowc bytes] and scales
// [16][rows bytes] from wave-uniform bases (lane r reads row r).  Both are
// read with the default cache policy, not the nontemporal one: a request
// covers 64 bytes of each row, so every 128-byte code line is completed by
// the next request, and a chunk needs only 16 scale bytes of each row, so a
// tile's scale lines serve all its chunks.  Nontemporal requests fetched
// such lines from HBM again (measured: batch-64 layer 3.0 ms with both
// nontemporal, 2.43 ms with cached scales, 2.26 ms with both cached).  Every
// request uses a per-lane offset fixed for the whole tile plus the chunk's
// position as a scalar offset, so no address register is rebuilt (or
// overwritten by a load) inside the chunk loop.  A request past the last
// chunk goes through an empty descriptor: the instruction is issued (so the
// wait counts stay exact) but touches no memory.
struct Tile {
  const uint8_t *c, *s;
  uint32_t rowc, rows;
};
__device__ __forceinline__ Tile make_tile(const uint8_t* codes, const uint8_t* scales, size_t row0,
                                          int K) {
  // the first row is wave-uniform: keep the bases in scalar registers
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row0);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(row0 >> 32));
  const size_t r0 = ((size_t)hi << 32) | lo;
  return {codes + r0 * (size_t)(K / 2), scales + r0 * (size_t)(K / 32), (uint32_t)K / 2, (uint32_t)K / 32};
}

// Scales: the chunk's KC / 32 scale bytes of row r are KC / 128 dwords;
// lane (q, r) requests dword q of them (one request per matrix and chunk,
// rather than one byte request per block), and the byte of block
// 4 kk + q is later taken from lane (kk, r) with ds_bpermute (scale_of).
template <int KC>
__device__ __forceinline__ void ld_codes(uint4 (&a)[KC / 128], const Tile& T, uint32_t voc, int c, int nch) {
  const bool live = c < nch;
  const uint32_t cc = (uint32_t)(live ? c : nch - 1);
  const auto rc = buf_rsrc(T.c, live ? 16u * T.rowc : 0u);
  const uint32_t soc = cc * (KC / 2);
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) {  // block cc * KC / 32 + 4 kk + q of row r
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(voc + 64u * kk), (int)soc, 0);
    a[kk] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}
template <int KC>
__device__ __forceinline__ void ld_tile(uint4 (&a)[KC / 128], uint32_t& sd, const Tile& T, uint32_t voc,
                                        uint32_t vos, int c, int nch) {
  ld_codes<KC>(a, T, voc, c, nch);
  const bool live = c < nch;
  const uint32_t cc = (uint32_t)(live ? c : nch - 1);
  const auto rs = buf_rsrc(T.s, live ? 16u * T.rows : 0u);
  sd = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)vos, (int)(cc * (KC / 32)), 0);
}
// Every chunk's scale dword of a tile at once (the same requests ld_tile
// makes chunk by chunk).  A tile's scale bytes (16 rows x H / 32) span a few
// dozen lines that each serve several chunks; requested a chunk at a time,
// the weight stream evicted them from L2 between uses, and the gate/up
// kernel fetched each scale line about 2.6 times (counted at batch 64).
template <int KC, int NCH>
__device__ __forceinline__ void ld_scales(uint32_t (&sd)[NCH], const Tile& T, uint32_t vos) {
  const auto rs = buf_rsrc(T.s, 16u * T.rows);
#pragma unroll
  for (int c = 0; c < NCH; ++c) sd[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)vos, c * (KC / 32), 0);
}
// Per-lane scale offsets of a tile: codes of block q, scale dword q (the
// last dword for lanes past the chunk's dwords).
template <int KC>
__device__ __forceinline__ void tile_offsets(const Tile& T, int q, int r, uint32_t& voc, uint32_t& vos) {
  constexpr int ND = KC / 128;
  voc = (uint32_t)r * T.rowc + 16u * (uint32_t)q;
  vos = (uint32_t)r * T.rows + 4u * (uint32_t)(q < ND ? q : ND - 1);
}
// E8M0 scale of block 4 kk + q of lane (q, r)'s row, from lane (kk, r)'s dword.
__device__ __forceinline__ float scale_of(uint32_t sd, int kk, int q, int r) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * kk + r), (int)sd);
  return e8m0_to_f32(byte_of(w, q));
}

// Token-activation staging: a chunk of a token row (PER x 16 16-byte pieces)
// is staged by 16 threads, thread j taking pieces j, j + 16, ..., so that
// each request covers 256 contiguous bytes of the row (one descriptor over
// the whole array, the row and piece as a fixed per-thread offset, the
// chunk as a scalar offset).
template <int PER>
struct Stage {
  u32x4 v[PER];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 256u * i), (int)soff, 0));
  }
  __device__ __forceinline__ void store(uint4* dst) const {  // dst: the thread's first piece
    u32x4* p = reinterpret_cast<u32x4*>(dst);
#pragma unroll
    for (int i = 0; i < PER; ++i) p[16 * i] = v[i];
  }
};

// PRE: the scales were requested for the whole tile (ld_scales): codes only.
template <int KC, bool PRE>
__device__ __forceinline__ void gu_load_a(GuRegs<KC>& R, const Tile& G, const Tile& U, uint32_t voc,
                                          uint32_t vos, int c, int nch) {
  if (PRE) {
    ld_codes<KC>(R.ag, G, voc, c, nch);
    ld_codes<KC>(R.au, U, voc, c, nch);
  } else {
    ld_tile<KC>(R.ag, R.sg, G, voc, vos, c, nch);
    ld_tile<KC>(R.au, R.su, U, voc, vos, c, nch);
  }
}

// Wide requests (one-tile gate/up passes at 512-element chunks): a wave
// instruction reads 4 rows x 256 bytes of the tile (lane l: row 4 kk + l / 16,
// bytes 16 (l % 16) of the chunk), nontemporal, instead of the operand
// layout's 16 rows x 64 bytes.  A streaming probe of the two shapes reads
// 7.0 against 6.3 TB/s.  to_operand then moves the chunk to the operand
// layout through a wave-private LDS tile of 16 x 16 pieces of 16 bytes
// (piece b of row R stored at R * 16 + (b ^ R): the row-wise stores and the
// column-wise loads both hit distinct banks), so that lane (q, r) holds
// bytes 64 kk + 16 q of row r, as ld_codes would have loaded them.
template <int KC>
__device__ __forceinline__ void ld_codes_wide(uint4 (&a)[KC / 128], const Tile& T, int c, int nch) {
  static_assert(KC == 512, "a chunk is 256 bytes of each of the 16 rows");
  const int lane = threadIdx.x & 63;
  const bool live = c < nch;
  const uint32_t cc = (uint32_t)(live ? c : nch - 1);
  const auto rc = buf_rsrc(T.c, live ? 16u * T.rowc : 0u);
  const uint32_t vo = (uint32_t)(lane >> 4) * T.rowc + 16u * (uint32_t)(lane & 15);
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(vo + 4u * kk * T.rowc), (int)(cc * (KC / 2)), kBufNT);
    a[kk] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}
constexpr int kWideTile = 256;  // uint4 per wave and matrix
// (The loads read other lanes' stores: a wavefront-scope fence keeps every
// store before every load.  The next chunk's stores come after the barrier
// that ends the chunk, which already orders them after these loads.)
template <int KC>
__device__ __forceinline__ void to_operand(uint4 (&a)[KC / 128], uint4* slot) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15;
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) {
    const int row = 4 * kk + q;  // stored: piece r of row 4 kk + q
    slot[row * 16 + (r ^ row)] = a[kk];
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) a[kk] = slot[r * 16 + ((4 * kk + q) ^ r)];
}

// Products of one chunk: token tile 0 (LDS rows 0..15) always, tile 1 (rows
// 16..31) when `two` (workgroup-uniform), from the same decoded fragments.
template <int KC>
__device__ __forceinline__ void gu_mma(const GuRegs<KC>& R, uint32_t sg, uint32_t su,
                                       const uint4 (*bt)[KC / 8 + 1], int q, int r, bool two,
                                       f32x4 (&cg)[2], f32x4 (&cu)[2]) {
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) {
    const float fg = scale_of(sg, kk, q, r), fu = scale_of(su, kk, q, r);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 ag = fp4x8_to_bf16(dword_of(R.ag[kk], s), fg);
      const bf16x8 au = fp4x8_to_bf16(dword_of(R.au[kk], s), fu);
      const bf16x8 b0 = as_bf16x8(bt[r][kk * 16 + 4 * q + s]);
      cg[0] = mfma16(ag, b0, cg[0]);
      cu[0] = mfma16(au, b0, cu[0]);
      if (two) {
        const bf16x8 b1 = as_bf16x8(bt[16 + r][kk * 16 + 4 * q + s]);
        cg[1] = mfma16(ag, b1, cg[1]);
        cu[1] = mfma16(au, b1, cu[1]);
      }
    }
  }
}

// NCH > 0: the chunk count (H / KC) fixed at compile time; the chunk loop
// is then unrolled whole, so that the wait counts carry no loop back-edge
// merge (with one, the compiler's waits become conservative and every chunk
// waits for the requests just issued).
// One pass of an item over the weights: tokens n0 .. n0 + 15 (TWO: n0 + 31)
// of the group.  The one-tile and two-tile passes are separate code paths,
// chosen per pass, so neither carries the other's requests.  With NCH > 0
// the scales come from TS (requested once per item), else chunk by chunk.
// WIDE: weights through ld_codes_wide and the wave's LDS tiles wt (gate)
// and wt + kWideTile (up); NCH > 0 and one token tile only.
template <int KC, int NCH, bool TWO, bool WIDE, class Lds>
__device__ __forceinline__ void gu_pass(const LayerTB& L, Lds& S, const Tile& G, const Tile& U,
                                        const TileScales<NCH>& TS, uint32_t voc, uint32_t vos, int start,
                                        int m, int n0, int rq, uint4* wt) {
  static_assert(!WIDE || (NCH > 0 && !TWO), "wide requests: scales preloaded, one token tile");
  constexpr bool PRE = NCH > 0;
  constexpr int PER = KC / 128;  // staged uint4 per thread per chunk and tile
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15, wid = wave_id();
  const int nch = NCH ? NCH : L.H / KC;
  const int sc = tid >> 4, sj = tid & 15;  // staging: token rows sc (and 16 + sc), first piece (stride 16)
  const auto rx = buf_rsrc(L.x, (uint32_t)L.T * (uint32_t)L.H * 2u), rx0 = buf_rsrc(L.x, 0u);
  const int cs0 = n0 + sc < m ? n0 + sc : m - 1, cs1 = n0 + 16 + sc < m ? n0 + 16 + sc : m - 1;
  const uint32_t xv0 = (uint32_t)token_of(L, L.order[start + cs0]) * (uint32_t)L.H * 2u + 16u * (uint32_t)sj;
  const uint32_t xv1 = TWO ? (uint32_t)token_of(L, L.order[start + cs1]) * (uint32_t)L.H * 2u + 16u * (uint32_t)sj : 0u;
  auto xso = [&](int c) { return (uint32_t)(c < nch ? c : nch - 1) * (uint32_t)(KC * 2); };
  // this wave stages rows 4 wid .. 4 wid + 3 of each tile; past the group's
  // tokens it requests nothing (empty descriptor: zeros, whose products are
  // dropped)
  const auto rw0 = 4 * wid < m - n0 ? rx : rx0, rw1 = 16 + 4 * wid < m - n0 ? rx : rx0;
  f32x4 cg[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  f32x4 cu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  auto load_w = [&](GuRegs<KC>& A, int c) {
    if constexpr (WIDE) {
      ld_codes_wide<KC>(A.ag, G, c, nch);
      ld_codes_wide<KC>(A.au, U, c, nch);
    } else {
      gu_load_a<KC, PRE>(A, G, U, voc, vos, c, nch);
    }
  };
  GuRegs<KC> A0, A1;
  Stage<PER> xa0, xa1, xb0, xb1;
  xa0.load(rw0, xv0, xso(0));
  if (TWO) xa1.load(rw1, xv1, xso(0));
  __builtin_amdgcn_sched_barrier(0);
  load_w(A0, 0);
  __builtin_amdgcn_sched_barrier(0);
  xb0.load(rw0, xv0, xso(1));
  if (TWO) xb1.load(rw1, xv1, xso(1));
  __builtin_amdgcn_sched_barrier(0);
  load_w(A1, 1);
  __builtin_amdgcn_sched_barrier(0);
  xa0.store(&S.b[0][sc][sj]);
  if (TWO) xa1.store(&S.b[0][16 + sc][sj]);
  __syncthreads();
  // chunk c: weights in Ac, activations in LDS buffer bu; chunk c + 1's
  // weights and activations (xs) in flight; xl takes chunk c + 2's
  auto step = [&](int c, GuRegs<KC>& Ac, Stage<PER>& xl0, Stage<PER>& xl1, const Stage<PER>& xs0,
                  const Stage<PER>& xs1, const uint4 (*bu)[KC / 8 + 1], uint4 (*bs)[KC / 8 + 1]) {
    if constexpr (WIDE) {
      to_operand<KC>(Ac.ag, wt);
      to_operand<KC>(Ac.au, wt + kWideTile);
    }
    if constexpr (PRE)
      gu_mma<KC>(Ac, TS.g[c], TS.u[c], bu, q, r, TWO, cg, cu);
    else
      gu_mma<KC>(Ac, Ac.sg, Ac.su, bu, q, r, TWO, cg, cu);
    if (!NCH || c + 2 < nch) {
      xl0.load(rw0, xv0, xso(c + 2));
      if (TWO) xl1.load(rw1, xv1, xso(c + 2));
      __builtin_amdgcn_sched_barrier(0);
      load_w(Ac, c + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!NCH || c + 1 < nch) {
      xs0.store(&bs[sc][sj]);
      if (TWO) xs1.store(&bs[16 + sc][sj]);
    }
    __syncthreads();
  };
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; c += 2) {
      step(c, A0, xa0, xa1, xb0, xb1, S.b[0], S.b[1]);
      if (c + 1 < NCH) step(c + 1, A1, xb0, xb1, xa0, xa1, S.b[1], S.b[0]);
    }
  } else {
    for (int c = 0; c < nch; c += 2) {
      step(c, A0, xa0, xa1, xb0, xb1, S.b[0], S.b[1]);
      if (c + 1 >= nch) break;
      step(c + 1, A1, xb0, xb1, xa0, xa1, S.b[1], S.b[0]);
    }
  }
#pragma unroll
  for (int t = 0; t < (TWO ? 2 : 1); ++t) {
    if (n0 + 16 * t + r < m) {
      const size_t o = (size_t)(start + n0 + 16 * t + r - L.pos0) * L.F + (rq * kWv + wid) * kTileRows + 4 * q;
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = silu(cg[t][i]) * cu[t][i];
        hi[i] = f32_to_bf16(a);
        lo[i] = f32_to_bf16(a - bf16_to_f32(hi[i]));
      }
      uint2 vh, vl;
      vh.x = (uint32_t)hi[0] | ((uint32_t)hi[1] << 16);
      vh.y = (uint32_t)hi[2] | ((uint32_t)hi[3] << 16);
      vl.x = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
      vl.y = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
      *reinterpret_cast<uint2*>(L.act_hi + o) = vh;
      *reinterpret_cast<uint2*>(L.act_lo + o) = vl;
    }
  }
}

// One-tile passes request their weights wide (ld_codes_wide).  In the
// one-tile kernel (batches of at most 16 tokens) the wave tiles take 32 KB
// more LDS, so two workgroups per CU instead of three.
constexpr bool kGuWide = true;

// MAXT: token tiles per pass (1 when no group can exceed 16 tokens: T <= 16,
// which keeps the smaller LDS and one more workgroup per CU).
template <int KC, int NCH, int MAXT>
__global__ __launch_bounds__(kBlk) void kb_gateup(LayerTB L) {
  using Lds = typename std::conditional<MAXT == 2, TokLds2<KC>, TokLds<KC>>::type;
  constexpr bool WIDE = kGuWide && NCH > 0 && KC == 512;  // one-tile passes
  __shared__ Lds S;
  // per wave: the gate and up tiles of the wide requests.  With two token
  // tiles they take the second tile's staging rows, which one-tile passes
  // leave unused (16 rows of 65 pieces in each buffer: two waves' tiles).
  __shared__ uint4 wtile[WIDE && MAXT == 1 ? kWv : 1][2 * kWideTile];
  const int lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15, wid = wave_id();
  int g0, g1;
  group_range(L, g0, g1);
  const int quads = L.F / (kTileRows * kWv);
  const int nitems = (g1 - g0) * quads;
  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    const int gi = it / quads, rq = it - gi * quads, g = g0 + gi;
    const int e = ld_uniform(L.g_expert + g), start = ld_uniform(L.g_start + g), m = ld_uniform(L.g_count + g);
    const bool sh = e >= L.E;
    const size_t row0 = (sh ? 0 : (size_t)e * L.F) + (size_t)(rq * kWv + wid) * kTileRows;
    const Tile G = make_tile(sh ? L.sg_codes : L.g_codes, sh ? L.sg_scales : L.g_scales, row0, L.H);
    const Tile U = make_tile(sh ? L.su_codes : L.u_codes, sh ? L.su_scales : L.u_scales, row0, L.H);
    uint32_t voc, vos;
    tile_offsets<KC>(G, q, r, voc, vos);
    uint4* const wt = !WIDE ? nullptr
                      : MAXT == 1 ? wtile[wid]
                                  : &S.b[wid >> 1][16][0] + (wid & 1) * (2 * kWideTile);
    TileScales<NCH> TS;
    if constexpr (NCH > 0) {
      ld_scales<KC, NCH>(TS.g, G, vos);
      ld_scales<KC, NCH>(TS.u, U, vos);
    }
    for (int n0 = 0; n0 < m; n0 += 16 * MAXT) {
      if (MAXT == 2 && m - n0 > 16)  // workgroup-uniform
        gu_pass<KC, NCH, true, false>(L, S, G, U, TS, voc, vos, start, m, n0, rq, nullptr);
      else
        gu_pass<KC, NCH, false, WIDE>(L, S, G, U, TS, voc, vos, start, m, n0, rq, wt);
    }
  }
}

// ---------------------------------------------------------------- down
// Workgroup items (group, kDnWaves consecutive 16-row tiles of the hidden
// size); per K chunk the workgroup stages the 16 pairs' a_hi and a_lo in LDS
// (double buffered) and each wave streams its 16 down rows, pipelined as in
// the gate/up kernel (waits only for requests a chunk old).
constexpr int kDnWaves = 8;
constexpr int kDnBlock = kDnWaves * kWave;

template <int KC>
struct DnRegs {
  uint4 a[KC / 128];
  uint32_t sc;  // scale dword (see ld_tile)
};

template <int KC>
__device__ __forceinline__ void dn_load_a(DnRegs<KC>& R, const Tile& D, uint32_t voc, uint32_t vos, int c,
                                          int nch) {
  ld_tile<KC>(R.a, R.sc, D, voc, vos, c, nch);
}

// The scale dword of block group kk comes from lane (kk, r)'s sd (chunk by
// chunk, see ld_tile) or, with a unit's scales in one quad per lane (QUAD:
// lane (c, r) holds dwords 4c .. 4c + 3 of row r), from lane (c, r)'s
// element kk.
template <int KC, bool QUAD = false>
__device__ __forceinline__ void dn_mma(const DnRegs<KC>& R, const uint4 (*bh)[KC / 8 + 1],
                                       const uint4 (*bl)[KC / 8 + 1], int q, int r, f32x4& acc,
                                       const u32x4* quad = nullptr, int c = 0) {
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) {
    const float f = QUAD ? e8m0_to_f32(byte_of((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * c + r), (int)(*quad)[kk]), q))
                         : scale_of(R.sc, kk, q, r);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 av = fp4x8_to_bf16(dword_of(R.a[kk], s), f);
      acc = mfma16(av, as_bf16x8(bh[r][kk * 16 + 4 * q + s]), acc);
      acc = mfma16(av, as_bf16x8(bl[r][kk * 16 + 4 * q + s]), acc);
    }
  }
}

// The general down kernel (any FFN width that is a multiple of KC; FFN 2048
// runs kb_down_flat below).
template <int KC>
__global__ __launch_bounds__(kDnBlock) void kb_down(LayerTB L) {
  __shared__ TokLds<KC> Sh, Sl;
  constexpr int PER = KC / 128;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15, wid = wave_id();
  int g0, g1;
  group_range(L, g0, g1);
  const int slabs = L.H / (kTileRows * kDnWaves);
  const int nitems = (g1 - g0) * slabs;
  const int nch = L.F / KC;
  const bool st_lo = wid >= kDnWaves / 2;  // staging: waves 0..3 stage a_hi, 4..7 a_lo
  const int sc = (tid & 255) >> 4, sj = tid & 15;  // token row, first piece (stride 16)
  // staged pairs: a_hi (waves 0..3) or a_lo (waves 4..7), [rows][F] bf16
  const uint32_t nrows = act_rows(L);
  const auto ra = buf_rsrc(st_lo ? L.act_lo : L.act_hi, nrows * (uint32_t)L.F * 2u);
  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    const int gi = it / slabs, sb = it - gi * slabs, g = g0 + gi;
    const int e = ld_uniform(L.g_expert + g), start = ld_uniform(L.g_start + g), m = ld_uniform(L.g_count + g);
    const bool sh = e >= L.E;
    const int rt = sb * kDnWaves + wid;
    const size_t row0 = (sh ? 0 : (size_t)e * L.H) + (size_t)rt * kTileRows;
    const Tile D = make_tile(sh ? L.sd_codes : L.d_codes, sh ? L.sd_scales : L.d_scales, row0, L.F);
    uint32_t voc, vos;
    tile_offsets<KC>(D, q, r, voc, vos);
    for (int n0 = 0; n0 < m; n0 += 16) {
      const int cs = n0 + sc < m ? n0 + sc : m - 1;
      const uint32_t xvo = (uint32_t)(start + cs - L.pos0) * (uint32_t)L.F * 2u + 16u * (uint32_t)sj;
      auto xso = [&](int c) { return (uint32_t)(c < nch ? c : nch - 1) * (uint32_t)(KC * 2); };
      uint4 (*sbuf0)[KC / 8 + 1] = st_lo ? Sl.b[0] : Sh.b[0];
      uint4 (*sbuf1)[KC / 8 + 1] = st_lo ? Sl.b[1] : Sh.b[1];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      DnRegs<KC> A0, A1;
      Stage<PER> xa, xb;
      xa.load(ra, xvo, xso(0));
      __builtin_amdgcn_sched_barrier(0);
      dn_load_a<KC>(A0, D, voc, vos, 0, nch);
      __builtin_amdgcn_sched_barrier(0);
      xb.load(ra, xvo, xso(1));
      __builtin_amdgcn_sched_barrier(0);
      dn_load_a<KC>(A1, D, voc, vos, 1, nch);
      __builtin_amdgcn_sched_barrier(0);
      xa.store(&sbuf0[sc][sj]);
      __syncthreads();
      auto step = [&](int c, DnRegs<KC>& Ac, Stage<PER>& xl, const Stage<PER>& xs, int bu,
                      uint4 (*bs)[KC / 8 + 1]) {
        dn_mma<KC>(Ac, Sh.b[bu], Sl.b[bu], q, r, acc);
        xl.load(ra, xvo, xso(c + 2));
        __builtin_amdgcn_sched_barrier(0);
        dn_load_a<KC>(Ac, D, voc, vos, c + 2, nch);
        __builtin_amdgcn_sched_barrier(0);
        xs.store(&bs[sc][sj]);
        __syncthreads();
      };
      for (int c = 0; c < nch; c += 2) {
        step(c, A0, xa, xb, 0, sbuf1);
        if (c + 1 >= nch) break;
        step(c + 1, A1, xb, xa, 1, sbuf0);
      }
      if (n0 + r < m) {
        float4 v;
        v.x = acc[0];
        v.y = acc[1];
        v.z = acc[2];
        v.w = acc[3];
        *reinterpret_cast<float4*>(L.y + (size_t)(start + n0 + r) * L.H + rt * kTileRows + 4 * q) = v;
      }
    }
  }
}

// The down kernel for an even, compile-time chunk count (FFN 2048: four
// chunks of 512).  A unit is (pass, slab of 8 row tiles): a pass is at most
// 16 pairs of one group (the grouping kernel lists the passes in group
// order), and units are dealt out pass-major, so the passes of a group that
// holds more than 16 pairs reach the same slab `slabs` units apart -- on
// the same XCD when slabs is a multiple of 8 (hidden 7168: 56), and at about
// the same time -- and read its weights through one L2.  (With the passes of
// a slab run one after another by one workgroup, the weights were fetched
// again for each pass.)  PASSES = false (at most 16 tokens, so every group
// is one pass) walks the groups directly.  A wave's work is the sequence of
// its units, and it runs that sequence as one stream of chunks: the last two
// chunks of a unit request the next unit's first two, so a unit starts with
// its weights already in flight instead of a cold pipeline (with four
// chunks per unit, that start was most of a unit's time).  Past the last
// unit the requests go through empty descriptors and the output store
// through a range check, so that no request sits under a branch.
//
// A unit's scales (16 rows x F / 32 bytes) are requested once, with its
// first chunk: lane (c, r) takes the 16 bytes of row r that chunk c uses.
// Requested chunk by chunk, the scale lines were evicted between a unit's
// chunks and fetched again (about 1.4 times their bytes at batch 64).
template <int KC, int NCH, bool PASSES>
__global__ __launch_bounds__(kDnBlock) void kb_down_flat(LayerTB L) {
  static_assert(NCH >= 2 && NCH % 2 == 0, "units alternate register sets by chunk parity");
  static_assert(NCH == 4 && KC == 512, "a unit's scales are one 16-byte piece per lane (q, r)");
  __shared__ TokLds<KC> Sh, Sl;
  constexpr int PER = KC / 128;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15, wid = wave_id();
  int v0, v1;
  if (PASSES) pass_range(L, v0, v1);
  else group_range(L, v0, v1);
  const int slabs = L.H / (kTileRows * kDnWaves);
  const int nitems = (v1 - v0) * slabs;
  // staging: waves 0..3 stage a_hi, 4..7 a_lo (a wave-uniform choice, so the
  // descriptor stays in scalar registers)
  const bool st_lo = wid >= kDnWaves / 2;
  const int sc = (tid & 255) >> 4, sj = tid & 15;  // token row, first piece (stride 16)
  const uint32_t npairs = (uint32_t)(L.T * L.k + L.S * L.T);
  const uint32_t nrows = act_rows(L);
  const uint16_t* abase = st_lo ? L.act_lo : L.act_hi;
  const auto ra = buf_rsrc(abase, nrows * (uint32_t)L.F * 2u), ra0 = buf_rsrc(abase, 0u);
  const auto ry = buf_rsrc(L.y, npairs * (uint32_t)L.H * 4u);
  uint4 (*sbuf[2])[KC / 8 + 1] = {st_lo ? Sl.b[0] : Sh.b[0], st_lo ? Sl.b[1] : Sh.b[1]};

  struct Unit {
    Tile D;
    uint32_t voc, xvo;
    int pair0, m, n0, rt;
    bool live;
  };
  auto unit_at = [&](int it) {
    Unit u;
    u.live = it < nitems;
    const int itc = u.live ? it : nitems - 1;
    const int vi = itc / slabs, sb = itc - vi * slabs, v = v0 + vi;
    const int g = PASSES ? ld_uniform(L.pass_group + v) : v, n0 = PASSES ? ld_uniform(L.pass_n0 + v) : 0;
    const int e = ld_uniform(L.g_expert + g), start = ld_uniform(L.g_start + g), m = ld_uniform(L.g_count + g);
    const bool sh = e >= L.E;
    u.rt = sb * kDnWaves + wid;
    const size_t row0 = (sh ? 0 : (size_t)e * L.H) + (size_t)u.rt * kTileRows;
    u.D = make_tile(sh ? L.sd_codes : L.d_codes, sh ? L.sd_scales : L.d_scales, row0, L.F);
    u.voc = (uint32_t)r * u.D.rowc + 16u * (uint32_t)q;  // codes of block q of row r (scales: below)
    const int cs = n0 + sc < m ? n0 + sc : m - 1;
    u.xvo = (uint32_t)(start + cs - L.pos0) * (uint32_t)L.F * 2u + 16u * (uint32_t)sj;
    u.pair0 = start + n0;
    u.m = m;
    u.n0 = n0;
    return u;
  };
  // a wave stages rows 4 (wid & 3) .. + 3 of the unit's 16; when they are all
  // past the unit's pairs it requests nothing (empty descriptor: zeros)
  const int srow0 = 4 * (wid & 3);
  auto load_chunk = [&](const Unit& u, int c, DnRegs<KC>& A, Stage<PER>& X, u32x4& Q) {
    X.load(u.live && srow0 < u.m - u.n0 ? ra : ra0, u.xvo, (uint32_t)c * (uint32_t)(KC * 2));
    __builtin_amdgcn_sched_barrier(0);
    ld_codes<KC>(A.a, u.D, u.voc, u.live ? c : NCH, NCH);
    if (c == 0)  // the unit's scales: bytes 16 q .. 16 q + 15 of row r
      Q = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(u.D.s, u.live ? 16u * u.D.rows : 0u),
                                                (int)(r * u.D.rows + 16u * (uint32_t)q), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  int it = blockIdx.x;
  if (it >= nitems) return;
  Unit cur = unit_at(it);
  DnRegs<KC> A0, A1;
  Stage<PER> xa, xb;
  u32x4 qc, qn;  // this unit's scales, the next unit's
  load_chunk(cur, 0, A0, xa, qc);
  load_chunk(cur, 1, A1, xb, qc);
  xa.store(&sbuf[0][sc][sj]);
  __syncthreads();
  for (;;) {
    const Unit nxt = unit_at(it + (int)gridDim.x);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      DnRegs<KC>& Ac = (c & 1) ? A1 : A0;
      Stage<PER>& xl = (c & 1) ? xb : xa;
      const Stage<PER>& xs = (c & 1) ? xa : xb;
      dn_mma<KC, true>(Ac, Sh.b[c & 1], Sl.b[c & 1], q, r, acc, &qc, c);
      if (c + 2 < NCH) load_chunk(cur, c + 2, Ac, xl, qc);
      else load_chunk(nxt, c + 2 - NCH, Ac, xl, qn);
      xs.store(&sbuf[(c + 1) & 1][sc][sj]);
      __syncthreads();
    }
    // rows of valid pairs only (the store's range check drops the others)
    const bool ok = cur.n0 + r < cur.m;
    const uint32_t yo = ok ? 4u * ((uint32_t)(cur.pair0 + r) * (uint32_t)L.H + (uint32_t)(cur.rt * kTileRows + 4 * q))
                           : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ry, (int)yo, 0, 0);
    if (!nxt.live) break;
    it += (int)gridDim.x;
    cur = nxt;
    qc = qn;  // waits for the next unit's first chunk, which its first products need anyway
  }
}

// The FFN-2048 down kernel for batches of at most 8 tokens (no group holds
// more than 8 pairs, so a unit is a whole group): kb_down_flat's units and
// chunk stream, with
//  - 8 staged pair rows instead of 16 (16 KB of LDS per part instead of 33),
//    pieces swizzled instead of padded (piece p of row R at p ^ R), and
//  - the weights requested wide (ld_codes_wide: 4 rows x 256 B per wave
//    instruction, nontemporal) and moved to the operand layout through a
//    4 KB LDS tile per wave (to_operand), which the freed LDS holds.
// Operand columns 8..15 read the rows of columns 0..7 again (an LDS
// broadcast); their results are not stored.
template <int KC>
struct TokLdsSw8 {
  uint4 b[2][8][KC / 8];
};
template <int KC>
__device__ __forceinline__ void dn_mma_w8(const DnRegs<KC>& R, const uint4 (*bh)[KC / 8],
                                          const uint4 (*bl)[KC / 8], int q, int r, f32x4& acc,
                                          const u32x4& quad, int c) {
  const int r8 = r & 7;
#pragma unroll
  for (int kk = 0; kk < KC / 128; ++kk) {
    const float f = e8m0_to_f32(byte_of((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * c + r), (int)quad[kk]), q));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 av = fp4x8_to_bf16(dword_of(R.a[kk], s), f);
      acc = mfma16(av, as_bf16x8(bh[r8][kk * 16 + ((4 * q + s) ^ r8)]), acc);
      acc = mfma16(av, as_bf16x8(bl[r8][kk * 16 + ((4 * q + s) ^ r8)]), acc);
    }
  }
}
// A thread's two staged pieces of one pair row (32 threads a row, pieces
// j and j + 32).
struct Stage8 {
  u32x4 v[2];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 512u * i), (int)soff, 0));
  }
  __device__ __forceinline__ void store(uint4* dst) const {  // dst: the thread's first piece
    u32x4* p = reinterpret_cast<u32x4*>(dst);
#pragma unroll
    for (int i = 0; i < 2; ++i) p[32 * i] = v[i];
  }
};

template <int KC, int NCH>
__global__ __launch_bounds__(kDnBlock) void kb_down_w8(LayerTB L) {
  static_assert(NCH == 4 && KC == 512, "a unit's scales are one 16-byte piece per lane (q, r)");
  __shared__ TokLdsSw8<KC> Sh, Sl;
  __shared__ uint4 dtile[kDnWaves][kWideTile];  // the waves' wide-request tiles
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15, wid = wave_id();
  int v0, v1;
  group_range(L, v0, v1);
  const int slabs = L.H / (kTileRows * kDnWaves);
  const int nitems = (v1 - v0) * slabs;
  // staging: waves 0..3 stage a_hi, 4..7 a_lo; thread row sc (0..7), pieces sj, sj + 32
  const bool st_lo = wid >= kDnWaves / 2;
  const int sc = (tid & 255) >> 5, sj = tid & 31;
  const uint32_t npairs = (uint32_t)(L.T * L.k + L.S * L.T);
  const uint32_t nrows = act_rows(L);
  const uint16_t* abase = st_lo ? L.act_lo : L.act_hi;
  const auto ra = buf_rsrc(abase, nrows * (uint32_t)L.F * 2u), ra0 = buf_rsrc(abase, 0u);
  const auto ry = buf_rsrc(L.y, npairs * (uint32_t)L.H * 4u);
  uint4 (*sbuf[2])[KC / 8] = {st_lo ? Sl.b[0] : Sh.b[0], st_lo ? Sl.b[1] : Sh.b[1]};
  uint4* const tile = dtile[wid];

  struct Unit {
    Tile D;
    uint32_t xvo;
    int pair0, m, rt;
    bool live;
  };
  auto unit_at = [&](int it) {
    Unit u;
    u.live = it < nitems;
    const int itc = u.live ? it : nitems - 1;
    const int vi = itc / slabs, sb = itc - vi * slabs, g = v0 + vi;
    const int e = ld_uniform(L.g_expert + g), start = ld_uniform(L.g_start + g), m = ld_uniform(L.g_count + g);
    const bool sh = e >= L.E;
    u.rt = sb * kDnWaves + wid;
    const size_t row0 = (sh ? 0 : (size_t)e * L.H) + (size_t)u.rt * kTileRows;
    u.D = make_tile(sh ? L.sd_codes : L.d_codes, sh ? L.sd_scales : L.d_scales, row0, L.F);
    const int cs = sc < m ? sc : m - 1;
    u.xvo = (uint32_t)(start + cs - L.pos0) * (uint32_t)L.F * 2u + 16u * (uint32_t)sj;
    u.pair0 = start;
    u.m = m;
    return u;
  };
  // a wave stages rows 2 (wid & 3) and 2 (wid & 3) + 1; when both are past
  // the group's pairs it requests nothing (empty descriptor: zeros)
  const int srow0 = 2 * (wid & 3);
  auto load_chunk = [&](const Unit& u, int c, DnRegs<KC>& A, Stage8& X, u32x4& Q) {
    X.load(u.live && srow0 < u.m ? ra : ra0, u.xvo, (uint32_t)c * (uint32_t)(KC * 2));
    __builtin_amdgcn_sched_barrier(0);
    ld_codes_wide<KC>(A.a, u.D, u.live ? c : NCH, NCH);
    if (c == 0)  // the unit's scales: bytes 16 q .. 16 q + 15 of row r
      Q = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(u.D.s, u.live ? 16u * u.D.rows : 0u),
                                                (int)(r * u.D.rows + 16u * (uint32_t)q), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  int it = blockIdx.x;
  if (it >= nitems) return;
  Unit cur = unit_at(it);
  DnRegs<KC> A0, A1;
  Stage8 xa, xb;
  u32x4 qc, qn;  // this unit's scales, the next unit's
  load_chunk(cur, 0, A0, xa, qc);
  load_chunk(cur, 1, A1, xb, qc);
  xa.store(&sbuf[0][sc][sj ^ sc]);
  __syncthreads();
  for (;;) {
    const Unit nxt = unit_at(it + (int)gridDim.x);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      DnRegs<KC>& Ac = (c & 1) ? A1 : A0;
      Stage8& xl = (c & 1) ? xb : xa;
      const Stage8& xs = (c & 1) ? xa : xb;
      to_operand<KC>(Ac.a, tile);  // the chunk's closing barrier orders its loads before the next stores
      dn_mma_w8<KC>(Ac, Sh.b[c & 1], Sl.b[c & 1], q, r, acc, qc, c);
      if (c + 2 < NCH) load_chunk(cur, c + 2, Ac, xl, qc);
      else load_chunk(nxt, c + 2 - NCH, Ac, xl, qn);
      xs.store(&sbuf[(c + 1) & 1][sc][sj ^ sc]);
      __syncthreads();
    }
    // columns of valid pairs only (the store's range check drops the others)
    const bool ok = r < 8 && r < cur.m;
    const uint32_t yo = ok ? 4u * ((uint32_t)(cur.pair0 + r) * (uint32_t)L.H + (uint32_t)(cur.rt * kTileRows + 4 * q))
                           : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ry, (int)yo, 0, 0);
    if (!nxt.live) break;
    it += (int)gridDim.x;
    cur = nxt;
    qc = qn;  // waits for the next unit's first chunk, which its first products need anyway
  }
}

// ---------------------------------------------------------------- combine
// Workgroup (token t, chunk of 8 kBlk hidden elements); each thread adds its
// 8 elements over the slots in order, then the shared output and the
// residual, and rounds once to bf16.
//
// KB > 0 (k == KB): every slot's rows, the shared row and the residual are
// requested before the first addition, so a thread waits for one memory
// round trip; the shared row and the residual come through descriptors that
// are empty when absent.  KB == 0 (any k): whole batches of kCombineBatch
// slots request their rows together, the remaining slots go one at a time.
// The additions are in the same order either way.
template <int KB>
__global__ __launch_bounds__(kBlk) void kb_combine(LayerTB L) {
  const int t = blockIdx.x;
  const int h0 = (blockIdx.y * kBlk + threadIdx.x) * 8;
  if (h0 >= L.H) return;
  const int P = L.T * L.k;
  const int npos = P + L.S * L.T;
  const size_t o = (size_t)t * L.H + h0;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // the token's weights and pair positions are workgroup-uniform (scalar loads)
  const float* wt = L.wts + (size_t)t * L.k;
  const int32_t* pt = L.pos_of + (size_t)t * L.k;
  auto row_of = [&](int j) {
    int pos = ld_uniform(pt + j);
    pos = pos < 0 ? 0 : (pos >= npos ? npos - 1 : pos);
    return reinterpret_cast<const float4*>(L.y + (size_t)pos * L.H + h0);
  };
  auto add = [&](float w, const float4& a, const float4& b) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w, v[i], acc[i]);
  };
  auto add_shared = [&](const float4& a, const float4& b) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  };
  auto add_residual = [&](const uint4& rv) {
    const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      acc[2 * d] += bf16_to_f32(rw[d] & 0xFFFFu);
      acc[2 * d + 1] += bf16_to_f32(rw[d] >> 16);
    }
  };
  if constexpr (KB > 0) {
    float4 ya[KB], yb[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const float4* yp = row_of(u);
      ya[u] = yp[0];
      yb[u] = yp[1];
    }
    const uint32_t so = 4u * (uint32_t)((size_t)(P + t) * L.H + h0);
    const auto rs = buf_rsrc(L.y, L.S ? 4u * (uint32_t)npos * (uint32_t)L.H : 0u);
    const auto rr = buf_rsrc(L.residual, L.residual ? 2u * (uint32_t)L.T * (uint32_t)L.H : 0u);
    const uint4 sa = buf_ld16(rs, so, 0u), sb = buf_ld16(rs, so + 16u, 0u);
    const uint4 rv = buf_ld16(rr, 2u * (uint32_t)o, 0u);
    __builtin_amdgcn_sched_barrier(0);  // every request above issued before the first addition
#pragma unroll
    for (int u = 0; u < KB; ++u) add(ld_uniform(wt + u), ya[u], yb[u]);
    if (L.S) add_shared(__builtin_bit_cast(float4, sa), __builtin_bit_cast(float4, sb));
    if (L.residual) add_residual(rv);
  } else {
    constexpr int kCombineBatch = 8;
    int j0 = 0;
    for (; j0 + kCombineBatch <= L.k; j0 += kCombineBatch) {
      float4 ya[kCombineBatch], yb[kCombineBatch];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const float4* yp = row_of(j0 + u);
        ya[u] = yp[0];
        yb[u] = yp[1];
      }
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) add(ld_uniform(wt + j0 + u), ya[u], yb[u]);
    }
    for (int j = j0; j < L.k; ++j) {
      const float4* yp = row_of(j);
      add(ld_uniform(wt + j), yp[0], yp[1]);
    }
    if (L.S) {
      const float4* yp = reinterpret_cast<const float4*>(L.y + (size_t)(P + t) * L.H + h0);
      add_shared(yp[0], yp[1]);
    }
    if (L.residual) add_residual(*reinterpret_cast<const uint4*>(L.residual + o));
  }
  uint32_t ow[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    ow[d] = (uint32_t)f32_to_bf16(acc[2 * d]) | ((uint32_t)f32_to_bf16(acc[2 * d + 1]) << 16);
  const uint4 ov = {ow[0], ow[1], ow[2], ow[3]};
  *reinterpret_cast<uint4*>(L.out + o) = ov;
  if (L.trace) *reinterpret_cast<uint4*>(L.trace + o) = ov;
}

// ---------------------------------------------------------------- rmsnorm
// xn[t] = bf16(h[t] * gamma / sqrt(mean(h[t]^2) + eps)), one workgroup per
// token, the same reduction order as the single-token prologue.
constexpr int kMaxChunksPerThread = 8192 / 8 / kBlk;
__global__ __launch_bounds__(kBlk) void kb_rmsnorm(const uint16_t* __restrict__ h,
                                                   const uint16_t* __restrict__ gamma, float eps,
                                                   int H, uint16_t* __restrict__ xn) {
  __shared__ float red[kWv];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const uint4* x16 = reinterpret_cast<const uint4*>(h + (size_t)t * H);
  const uint4* g16 = reinterpret_cast<const uint4*>(gamma);
  const int nch = H / 8;
  uint4 v[kMaxChunksPerThread], g[kMaxChunksPerThread];
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = tid + i * kBlk;
    const int cc = c < nch ? c : nch - 1;
    v[i] = x16[cc];
    g[i] = g16[cc];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = tid + i * kBlk;
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
  if (lane == 0) red[wave_id()] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWv; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  uint4* o16 = reinterpret_cast<uint4*>(xn + (size_t)t * H);
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = tid + i * kBlk;
    if (c < nch) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
      uint32_t ov[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float a = bf16_to_f32(w[d] & 0xFFFFu) * inv * bf16_to_f32(gw[d] & 0xFFFFu);
        const float b = bf16_to_f32(w[d] >> 16) * inv * bf16_to_f32(gw[d] >> 16);
        ov[d] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
      }
      const uint4 o = {ov[0], ov[1], ov[2], ov[3]};
      o16[c] = o;
    }
  }
}

// Grouped gate/up workgroups per CU (every one resident at once).  Two token
// tiles per pass: 512-element chunks fit two (180 registers, 66.5 KB LDS),
// 256-element chunks three (147 registers, 33 KB).  One tile (T <= 16):
// three with 512-element chunks (137 registers, 33 KB), four with 256 (109).
constexpr int kGroupedBlocksPerCU[2] = {4, 3};     // 256-element chunks, by tiles - 1
constexpr int kGroupedBlocksPerCU512[2] = {kGuWide ? 2 : 3, 2};  // 512-element chunks
constexpr int kDownBlocksPerCU = 2;
constexpr int kNumCUs = 256;

}  // namespace

hipError_t launch_router_tb(const LayerTB& L, hipStream_t s) {
  const int n_et = (L.E + kTileRows - 1) / kTileRows;
  const int nw = n_et * L.KS;
  MOE_LAUNCH(L.timer, kb_router, dim3((nw + kWv - 1) / kWv), dim3(kBlk), 0, s, L, n_et);
  return hipPeekAtLastError();
}

hipError_t launch_topk_tb(const LayerTB& L, hipStream_t s) {
  if (L.E % 4 == 0)
    MOE_LAUNCH(L.timer, kb_topk<true>, dim3(L.T), dim3(kTopkBlock), 0, s, L);
  else
    MOE_LAUNCH(L.timer, kb_topk<false>, dim3(L.T), dim3(kTopkBlock), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_group_tb(const LayerTB& L, hipStream_t s) {
  MOE_LAUNCH(L.timer, kb_group, dim3(1), dim3(kGroupBlock), 0, s, L);
  return hipPeekAtLastError();
}

template <int MAXT>
hipError_t launch_gateup_tiles(const LayerTB& L, hipStream_t s) {
  // H % 256 == 0 always; 512-element chunks where they divide H
  // every workgroup resident at once (items are dealt out round-robin)
  const dim3 g512(kNumCUs * kGroupedBlocksPerCU512[MAXT - 1]);
  if (L.H == 7168)
    MOE_LAUNCH(L.timer, (kb_gateup<512, 14, MAXT>), g512, dim3(kBlk), 0, s, L);
  else if (L.H == 8192)
    MOE_LAUNCH(L.timer, (kb_gateup<512, 16, MAXT>), g512, dim3(kBlk), 0, s, L);
  else if (L.H % 512 == 0)
    MOE_LAUNCH(L.timer, (kb_gateup<512, 0, MAXT>), g512, dim3(kBlk), 0, s, L);
  else
    MOE_LAUNCH(L.timer, (kb_gateup<256, 0, MAXT>), dim3(kNumCUs * kGroupedBlocksPerCU[MAXT - 1]), dim3(kBlk), 0, s,
               L);
  return hipPeekAtLastError();
}

hipError_t launch_gateup_tb(const LayerTB& L, hipStream_t s) {
  // a group holds at most T tokens (each token picks an expert once)
  return L.T > 16 ? launch_gateup_tiles<2>(L, s) : launch_gateup_tiles<1>(L, s);
}

hipError_t launch_down_tb(const LayerTB& L, hipStream_t s) {
  const dim3 grid(kNumCUs * kDownBlocksPerCU);
  // a group holds at most T pairs: more than one pass only when T > 16
  if (L.F == 2048 && L.T <= 8)
    MOE_LAUNCH(L.timer, (kb_down_w8<512, 4>), grid, dim3(kDnBlock), 0, s, L);
  else if (L.F == 2048 && L.T > 16)
    MOE_LAUNCH(L.timer, (kb_down_flat<512, 4, true>), grid, dim3(kDnBlock), 0, s, L);
  else if (L.F == 2048)
    MOE_LAUNCH(L.timer, (kb_down_flat<512, 4, false>), grid, dim3(kDnBlock), 0, s, L);
  else if (L.F % 512 == 0)
    MOE_LAUNCH(L.timer, kb_down<512>, grid, dim3(kDnBlock), 0, s, L);
  else if (L.F % 256 == 0)
    MOE_LAUNCH(L.timer, kb_down<256>, grid, dim3(kDnBlock), 0, s, L);
  else
    MOE_LAUNCH(L.timer, kb_down<128>, grid, dim3(kDnBlock), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_combine_tb(const LayerTB& L, hipStream_t s) {
  const int chunks = (L.H + 8 * kBlk - 1) / (8 * kBlk);
  if (L.k == 16)
    MOE_LAUNCH(L.timer, kb_combine<16>, dim3(L.T, chunks), dim3(kBlk), 0, s, L);
  else
    MOE_LAUNCH(L.timer, kb_combine<0>, dim3(L.T, chunks), dim3(kBlk), 0, s, L);
  return hipPeekAtLastError();
}

hipError_t launch_rmsnorm_tb(const uint16_t* h, const uint16_t* gamma, float eps, int T, int H,
                             uint16_t* xn, hipStream_t s) {
  hipLaunchKernelGGL(kb_rmsnorm, dim3(T), dim3(kBlk), 0, s, h, gamma, eps, H, xn);
  return hipPeekAtLastError();
}

}  // namespace moe
