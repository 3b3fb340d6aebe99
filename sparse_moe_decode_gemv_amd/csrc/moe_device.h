// Device-side helpers of the gfx950 MoE decode kernels.
//
// MXFP4 blocks (OCP Microscaling v1.0) are 16 code bytes (32 E2M1 elements,
// element 2i in the low nibble of byte i) sharing one E8M0 scale byte.  The
// hot loops turn code bytes into exact bf16 or fp32 element pairs with the
// CDNA4 conversion instructions and fold the power-of-two block scale in
// once per block, in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kWave = 64;

// Streaming loads of static weights: each weight byte is read once per call,
// so the loads carry the nontemporal hint and do not displace cached
// activations.
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint32_t ld_stream8(const uint8_t* p) {
  return __builtin_nontemporal_load(p);
}
// The 32-bit word that holds byte b of a 4-byte aligned row (the caller
// extracts the byte with byte_of(w, b & 3)).  Used for scale bytes that stay
// in flight across a loop iteration: a byte load's result gets a
// zero-extension that the compiler may place before the loop's back edge,
// which waits for the load there.
__device__ __forceinline__ uint32_t ld_stream_word_of(const uint8_t* row, int b) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row) + (b >> 2));
}
// Raw buffer access: a descriptor (base, size in bytes) held in scalar
// registers, a per-lane 32-bit offset and a wave-uniform scalar offset.
// Used where many rows are in flight at once: every row then needs one
// scalar offset instead of a 64-bit vector address.  Reads at or past
// `bytes` return zero.
constexpr int kBufDataFormat = 0x00020000;  // descriptor word 3 for raw dword data (gfx9)
constexpr int kBufNT = 2;                   // cache policy: nontemporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufDataFormat);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kBufNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kBufNT);
}
// A wave-uniform read of data no kernel of the launch writes, through the
// scalar data cache (a scalar load: it waits on lgkmcnt, not on the vector
// memory counter that tracks the weight stream).
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int byte) {
  return __builtin_amdgcn_ubfe(w, 8 * byte, 8);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 byte -> fp32 2^(b-127) (exact; denormal for b = 0); 0xFF is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  const float s = __builtin_amdgcn_ldexpf(1.0f, (int)b - 127);
  return b == 0xFFu ? __uint_as_float(0x7FC00000u) : s;
}

// bf16 pair view of a dword (element 2i in the low half).
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) {
  return __builtin_bit_cast(bf16x2, v);
}

// Dot product of one 32-element MXFP4 block (4 code dwords, scale not
// applied) with 32 bf16 activations (16 dwords, pairs in element order).
__device__ __forceinline__ float block_dot_bf16(const uint4 c, const uint32_t* xv) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 0);
    bf16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 1);
    bf16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 2);
    bf16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 3);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(w0, as_bf16x2(xv[4 * d + 0]), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(w1, as_bf16x2(xv[4 * d + 1]), a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(w2, as_bf16x2(xv[4 * d + 2]), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(w3, as_bf16x2(xv[4 * d + 3]), a1, false);
  }
  return a0 + a1;
}

// Dot product of one 32-element MXFP4 block with 32 fp32 activations.
__device__ __forceinline__ float block_dot_f32(const uint4 c, const float* av) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 0);
    const f32x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 1);
    const f32x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 2);
    const f32x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 3);
    const float* a = av + 8 * d;
    a0 = __builtin_fmaf(w0.x, a[0], a0);
    a1 = __builtin_fmaf(w0.y, a[1], a1);
    a0 = __builtin_fmaf(w1.x, a[2], a0);
    a1 = __builtin_fmaf(w1.y, a[3], a1);
    a0 = __builtin_fmaf(w2.x, a[4], a0);
    a1 = __builtin_fmaf(w2.y, a[5], a1);
    a0 = __builtin_fmaf(w3.x, a[6], a0);
    a1 = __builtin_fmaf(w3.y, a[7], a1);
  }
  return a0 + a1;
}

// Sum over aligned groups of `width` lanes (width a power of two, 4..64) by
// DPP: butterflies inside quads, half rows and rows of 16 lanes, then row
// broadcasts across rows.  The group's total is valid in the group's last
// lane (lane % width == width - 1); other lanes hold partial sums.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_term(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float group_sum_last(float v, int width) {
  v += dpp_term<0xB1, 0xF>(v);                  // quad_perm 1,0,3,2
  v += dpp_term<0x4E, 0xF>(v);                  // quad_perm 2,3,0,1
  if (width >= 8) v += dpp_term<0x141, 0xF>(v);   // row_half_mirror
  if (width >= 16) v += dpp_term<0x140, 0xF>(v);  // row_mirror
  if (width >= 32) v += dpp_term<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  if (width >= 64) v += dpp_term<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// group_sum_last for a width known at compile time.
template <int W>
__device__ __forceinline__ float group_sum_last_c(float v) {
  static_assert(W >= 4 && W <= 64 && (W & (W - 1)) == 0, "group width");
  v += dpp_term<0xB1, 0xF>(v);
  v += dpp_term<0x4E, 0xF>(v);
  if (W >= 8) v += dpp_term<0x141, 0xF>(v);
  if (W >= 16) v += dpp_term<0x140, 0xF>(v);
  if (W >= 32) v += dpp_term<0x142, 0xA>(v);
  if (W >= 64) v += dpp_term<0x143, 0xC>(v);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Maximum over the 64 lanes, returned uniformly: DPP butterflies inside each
// row of 16 lanes, then the four row results are read out and combined.
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false)); // row_half_mirror
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false)); // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return umax32(umax32(r0, r1), umax32(r2, r3));
}

// Inclusive prefix sum over the 64 lanes (DPP row shifts, then row
// broadcasts across rows).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_term_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_term_u32<0x111, 0xF>(v);  // row_shr:1
  v += dpp_term_u32<0x112, 0xF>(v);  // row_shr:2
  v += dpp_term_u32<0x114, 0xF>(v);  // row_shr:4
  v += dpp_term_u32<0x118, 0xF>(v);  // row_shr:8
  v += dpp_term_u32<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_term_u32<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Order-preserving 32-bit key of an fp32 value (-0 folded onto +0), so that
// unsigned comparison of keys orders the values.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---- v_mfma_f32_16x16x32_bf16 fragments ------------------------------------
// Lane l = 16 q + r holds A[r][8q .. 8q+7] and B[8q .. 8q+7][r]; the result
// lane holds C[4q .. 4q+3][r].  The reduction index may be permuted freely as
// long as A and B use the same permutation.

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight MXFP4 elements (one code dword, element order) times the block
// scale, as exact bf16 values.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  const bf16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int s) {
  return s == 0 ? v.x : (s == 1 ? v.y : (s == 2 ? v.z : v.w));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace moe
