// Proxy scoring: "Dynamic Token Coverage", scoring (gist.science summary of
// Token Sparse Attention, section 2).  The last w queries of each head attend
// causally to all keys; each softmax row is summed column-wise and divided by
// w to give per-token importance s[b,h,j].
//
// An exact softmax needs every row's max and normaliser before any column
// sum can be formed, so the work is two streaming passes over K plus a small
// merge; no L x w buffer is ever held:
//   pass 1  per (key chunk, head): per-row (max, sum of exp) over the chunk
//   merge   per proxy row: global max and 1/Z, chunk partials combined in fp64
//   pass 2  per (key chunk, head): s_j = (1/w) sum_r exp2(x_rj - M_r) / Z_r
// Logits are kept in exp2 units: x = <q, k> * log2(e)/sqrt(d).  Both passes
// evaluate x with the same code, so pass 2 sees exactly the values pass 1
// reduced.  All reductions run in a fixed order: the result is deterministic.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

constexpr int kThreads = kScoreChunk;   // one key per thread
constexpr int kRowTile = 16;            // proxy rows staged in LDS at a time

// Load one key row into registers as fp32.
template <typename T, int D>
__device__ __forceinline__ void load_row(const T* __restrict__ src, float (&r)[D]) {
#pragma unroll
  for (int i = 0; i < D; ++i) r[i] = Elem<T>::load(src, i);
}

template <int D>
__device__ __forceinline__ float dot_scaled(const float (&k)[D], const float* __restrict__ q,
                                            float c) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) acc = fmaf(q[i], k[i], acc);
  return acc * c;
}

// Stage proxy rows [r0, r0+n) of head (b,h) into LDS as fp32.
template <typename T, int D>
__device__ __forceinline__ void stage_q(const T* __restrict__ qh, int L, int w, int r0, int n,
                                        float* __restrict__ qs) {
  for (int e = threadIdx.x; e < n * D; e += kThreads) {
    const int ri = r0 + e / D;
    qs[e] = Elem<T>::load(qh, int64_t(L - w + ri) * D + (e % D));
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void score_pass1(const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        float2* __restrict__ part, int Hq, int Hkv,
                                                        int L, int w, int n_chunk, float c) {
  __shared__ float qs[kRowTile * D];
  __shared__ float red[2][kRowTile][kThreads / 64];
  const int chunk = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / (Hq / Hkv);
  const int j = chunk * kScoreChunk + threadIdx.x;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const T* qh = q + (int64_t(b) * Hq + h) * int64_t(L) * D;
  const T* kg = k + (int64_t(b) * Hkv + g) * int64_t(L) * D;
  float kr[D];
  if (j < L) load_row<T, D>(kg + int64_t(j) * D, kr);
  else {
#pragma unroll
    for (int i = 0; i < D; ++i) kr[i] = 0.f;
  }
  for (int r0 = 0; r0 < w; r0 += kRowTile) {
    const int n = min(kRowTile, w - r0);
    __syncthreads();
    stage_q<T, D>(qh, L, w, r0, n, qs);
    __syncthreads();
    for (int ri = 0; ri < n; ++ri) {
      const int r = L - w + r0 + ri;
      const bool vis = j <= r;   // causal proxy row; also excludes j >= L
      const float x = vis ? dot_scaled<D>(kr, qs + ri * D, c) : -INFINITY;
      const float m = wave_max(x);
      const float e = vis ? exp2f(x - m) : 0.f;
      const float z = wave_sum(e);
      if (lane == 0) {
        red[0][ri][wid] = m;
        red[1][ri][wid] = z;
      }
    }
    __syncthreads();
    if (threadIdx.x < n) {
      const int ri = threadIdx.x;
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < kThreads / 64; ++i) m = fmaxf(m, red[0][ri][i]);
      float z = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < kThreads / 64; ++i)
          if (red[0][ri][i] != -INFINITY) z += red[1][ri][i] * exp2f(red[0][ri][i] - m);
      }
      part[((int64_t(bh) * w) + r0 + ri) * n_chunk + chunk] = make_float2(m, z);
    }
  }
}

// One thread per proxy row: combine chunk partials (sums in fp64).
__global__ void score_merge(const float2* __restrict__ part, float2* __restrict__ rowstat,
                            int64_t rows, int n_chunk) {
  const int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const float2* p = part + r * n_chunk;
  float m = -INFINITY;
  for (int i = 0; i < n_chunk; ++i) m = fmaxf(m, p[i].x);
  double z = 0.0;
  for (int i = 0; i < n_chunk; ++i)
    if (p[i].x != -INFINITY) z += double(p[i].y) * exp2(double(p[i].x) - double(m));
  rowstat[r] = make_float2(m, float(1.0 / z));
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void score_pass2(const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        const float2* __restrict__ rowstat,
                                                        float* __restrict__ s, int Hq, int Hkv,
                                                        int L, int w, float c) {
  __shared__ float qs[kRowTile * D];
  __shared__ float2 st[kRowTile];
  const int chunk = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / (Hq / Hkv);
  const int j = chunk * kScoreChunk + threadIdx.x;
  const T* qh = q + (int64_t(b) * Hq + h) * int64_t(L) * D;
  const T* kg = k + (int64_t(b) * Hkv + g) * int64_t(L) * D;
  float kr[D];
  if (j < L) load_row<T, D>(kg + int64_t(j) * D, kr);
  else {
#pragma unroll
    for (int i = 0; i < D; ++i) kr[i] = 0.f;
  }
  float acc = 0.f;
  for (int r0 = 0; r0 < w; r0 += kRowTile) {
    const int n = min(kRowTile, w - r0);
    __syncthreads();
    stage_q<T, D>(qh, L, w, r0, n, qs);
    if (threadIdx.x < n) st[threadIdx.x] = rowstat[int64_t(bh) * w + r0 + threadIdx.x];
    __syncthreads();
    for (int ri = 0; ri < n; ++ri) {
      const int r = L - w + r0 + ri;
      if (j <= r) {
        const float x = dot_scaled<D>(kr, qs + ri * D, c);
        acc += exp2f(x - st[ri].x) * st[ri].y;
      }
    }
  }
  if (j < L) s[int64_t(bh) * L + j] = acc / float(w);
}

template <typename T, int D>
hipError_t run(const Shape& sh, const void* q, const void* k, float* scores, char* ws,
               hipStream_t st) {
  const StepWs lay = step_ws_layout(sh);
  float2* part = reinterpret_cast<float2*>(ws + lay.part);
  float2* rowstat = reinterpret_cast<float2*>(ws + lay.rowstat);
  const float c = kLog2e / sqrtf(float(D));
  const int nc = sh.n_chunk();
  dim3 grid(nc, sh.B * sh.Hq);
  score_pass1<T, D><<<grid, kThreads, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                               part, sh.Hq, sh.Hkv, sh.L, sh.w, nc, c);
  const int64_t rows = int64_t(sh.B) * sh.Hq * sh.w;
  score_merge<<<unsigned((rows + 255) / 256), 256, 0, st>>>(part, rowstat, rows, nc);
  score_pass2<T, D><<<grid, kThreads, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                               rowstat, scores, sh.Hq, sh.Hkv, sh.L, sh.w, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const Shape& sh, const void* q, const void* k, float* scores, char* ws,
                        hipStream_t st) {
  if (sh.dtype == TSA_BF16)
    return sh.d == 128 ? run<uint16_t, 128>(sh, q, k, scores, ws, st)
                       : run<uint16_t, 64>(sh, q, k, scores, ws, st);
  return sh.d == 128 ? run<float, 128>(sh, q, k, scores, ws, st)
                     : run<float, 64>(sh, q, k, scores, ws, st);
}

}  // namespace tsa
