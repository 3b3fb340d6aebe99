// Device filler for synthetic MXFP4 expert bytes.
//
// Implements the same counter-based stream as moe_inputs/__init__.py: word i
// of the stream keyed by K is the (i+1)-th SplitMix64 output for seed K
// (Steele, Lea and Flood, OOPSLA 2014; finaliser constants from Vigna's public
// splitmix64.c).  Code bytes are the little-endian bytes of the words; scale
// byte j is lo + floor(hi32(word_j) * count / 2^32).  Input generation only:
// nothing here belongs to the decode computation.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t sm64(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void fill_codes_kernel(uint64_t* __restrict__ dst, uint64_t key,
                                  uint64_t word_start, uint64_t n_words) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += stride)
    dst[i] = sm64(key, word_start + i);
}

__global__ void fill_scales_kernel(uint8_t* __restrict__ dst, uint64_t key,
                                   uint64_t start, uint64_t n, int lo, int count) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const uint64_t hi = sm64(key, start + i) >> 32;
    dst[i] = (uint8_t)(lo + (int)((hi * (uint64_t)count) >> 32));
  }
}

unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : (g ? g : 1));
}

}  // namespace

extern "C" int moe_inputs_fill_codes(void* dst, uint64_t key, uint64_t word_start,
                                     uint64_t n_words, void* stream) {
  if (n_words == 0) return 0;
  if (!dst || ((uintptr_t)dst & 7)) return -1;
  hipLaunchKernelGGL(fill_codes_kernel, dim3(grid_for(n_words)), dim3(256), 0,
                     (hipStream_t)stream, (uint64_t*)dst, key, word_start, n_words);
  return hipPeekAtLastError() == hipSuccess ? 0 : -4;
}

extern "C" int moe_inputs_fill_scales(void* dst, uint64_t key, uint64_t start,
                                      uint64_t n, int lo, int count, void* stream) {
  if (n == 0) return 0;
  if (!dst || count <= 0 || lo < 0 || lo + count > 256) return -1;
  hipLaunchKernelGGL(fill_scales_kernel, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream, (uint8_t*)dst, key, start, n, lo, count);
  return hipPeekAtLastError() == hipSuccess ? 0 : -4;
}
