// Device-side helpers shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 raw bits <-> float.  bf16 -> float is exact (a 16-bit shift).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}
// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// Two floats -> packed bf16 pair (lo = a, hi = b), round to nearest even
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Inclusive scan of a 64-bit value over the 64 lanes of a wave.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive block-wide scan of a 64-bit value (blockDim.x a multiple of 64,
// at most 1024 threads).  `tmp` must hold 17 uint64 in LDS.  Returns the
// exclusive prefix; *total receives the block sum.  Contains barriers.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t x, uint64_t* tmp,
                                                        uint64_t* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  uint64_t inc = wave_incl_scan_u64(x);
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint64_t v = lane < nw ? tmp[lane] : 0;
    uint64_t vi = wave_incl_scan_u64(v);
    if (lane < nw) tmp[lane] = vi - v;   // exclusive prefix of wave totals
    if (lane == nw - 1) tmp[16] = vi;
  }
  __syncthreads();
  uint64_t res = tmp[wid] + inc - x;
  *total = tmp[16];
  __syncthreads();
  return res;
}

}  // namespace tsa
