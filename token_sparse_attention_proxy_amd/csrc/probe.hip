// Sustained bf16 MFMA throughput probe (include/tsa_probe.h).
//
// A register-only loop of v_mfma_f32_32x32x16_bf16 with two waves per SIMD
// and four independent accumulator chains: the shape the attention kernel's
// MFMA stream has, without its LDS, VALU and memory work.  The operands are
// either constant or random bf16 words; the rate differs because the chip's
// clock depends on how much the datapath toggles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;            // 8 waves: two per SIMD
constexpr int kMfmaPerIter = 16;
constexpr double kFlopPerMfma = 2.0 * 32 * 32 * 16;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Two bf16 values with random sign and mantissa and exponent 125..128
// (magnitudes in [0.25, 2)), from the 32 bits of h.
__device__ __forceinline__ uint32_t random_pair(uint32_t h) {
  const uint32_t lo = (h & 0x807fu) | ((125u + ((h >> 7) & 3u)) << 7);
  const uint32_t g = h >> 16;
  const uint32_t hi = (g & 0x807fu) | ((125u + ((g >> 7) & 3u)) << 7);
  return lo | (hi << 16);
}

template <bool RANDOM>
__global__ __launch_bounds__(kThreads, 1) void mfma_probe(float* __restrict__ sink, int iters) {
  // 96 KB of LDS, never touched: one workgroup per compute unit.
  __shared__ float reserve[24 * 1024];
  if (iters < 0) reserve[threadIdx.x] = 0.f;
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 wa, wb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t s = tid * 64u + uint32_t(i * 8 + e);
      wa[e] = RANDOM ? random_pair(mix32(s)) : 0x3f803f80u;                 // 1.0
      wb[e] = RANDOM ? random_pair(mix32(s ^ 0x9e3779b9u)) : 0x3f003f00u;   // 0.5
    }
    a[i] = __builtin_bit_cast(bf16x8, wa);
    b[i] = __builtin_bit_cast(bf16x8, wb);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < kMfmaPerIter; ++m)
      acc[m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % 8], b[(3 * m + (m >> 3)) % 8],
                                                           acc[m % 4], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += acc[c][e];
  sink[tid] = r;
}

int grid_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // namespace

extern "C" size_t tsa_probe_sink_bytes(void) {
  return size_t(grid_blocks()) * kThreads * sizeof(float);
}

extern "C" int tsa_probe_mfma_bf16(int random_operands, int iters, void* sink, size_t sink_bytes,
                                   double* flops, void* stream) {
  if (!sink || !flops || iters < 1) return 1;
  const int blocks = grid_blocks();
  if (blocks < 1 || sink_bytes < size_t(blocks) * kThreads * sizeof(float)) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (random_operands)
    mfma_probe<true><<<blocks, kThreads, 0, st>>>(static_cast<float*>(sink), iters);
  else
    mfma_probe<false><<<blocks, kThreads, 0, st>>>(static_cast<float*>(sink), iters);
  if (hipGetLastError() != hipSuccess) return 4;
  *flops = double(blocks) * (kThreads / 64) * double(iters) * kMfmaPerIter * kFlopPerMfma;
  return 0;
}
