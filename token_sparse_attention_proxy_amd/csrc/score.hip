// Proxy scoring: "Dynamic Token Coverage", scoring (gist.science summary of
// Token Sparse Attention, section 2).  The last w queries of each head attend
// causally to all keys; each softmax row is summed column-wise and divided by
// w to give per-token importance s[b,h,j].
//
// An exact softmax needs every row's max and normaliser before any column
// sum can be formed, so the work is two streaming passes over K plus a small
// merge; no L x w buffer is ever held:
//   pass 1  per (key chunk, KV head): per-row (max, sum of exp) over the chunk
//   merge   per proxy row: global max and 1/Z, chunk partials combined in fp64
//   pass 2  per (key chunk, KV head): s_j = (1/w) sum_r exp2(x_rj - M_r) / Z_r
// Logits are kept in exp2 units: x = <q, k> * log2(e)/sqrt(d).  Every
// reduction runs in a fixed order, so the result is deterministic.
//
// bf16 path (gfx950 MFMA): each 128-key chunk of a KV head is staged in LDS
// and serves the proxy rows of a group of its query heads (all G of them when
// their rows fit the eight waves), as 32-row tiles (a head's rows are padded
// to whole tiles); a workgroup walks a group of consecutive chunks with the
// next chunk's K loaded while the current one is computed.
// Pass 1 computes S^T = K Q^T (v_mfma_f32_32x32x16_bf16) so each lane owns a
// proxy row and keeps an online (max, sum); pass 2 computes S = Q K^T so each
// lane owns a key column and sums the 16 rows it holds, then the two lane
// halves, then the row tiles of the head (through LDS, in tile order).  The Q
// fragments and the LDS K reads are identical in the two orientations.
// f32 path: plain fp32 VALU kernels (one key per thread).
//
// causal = 0 (alternative reading): every proxy row sees all L keys.
#include <type_traits>

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
                                                        int L, int w, int n_chunk, float c,
                                                        int causal) {
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
      const bool vis = causal ? j <= r : j < L;   // j <= r also excludes j >= L
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

// One wave per proxy row: combine the chunk partials.  Lane i takes chunks
// i, i+64, ...; the row max is a wave max, the sum is accumulated in fp64 per
// lane and then reduced over the lanes in a fixed butterfly order, so the
// result is deterministic.  The grid also zeroes the words of two ranges
// (n0, n1 may be 0): in the whole op, the counters that the budget and the
// selection start from.
constexpr int kMergeWaves = 4;
__global__ __launch_bounds__(64 * kMergeWaves) void score_merge(const float2* __restrict__ part,
                                                                float2* __restrict__ rowstat,
                                                                int64_t rows, int n_chunk,
                                                                uint32_t* __restrict__ z0,
                                                                int64_t n0,
                                                                uint32_t* __restrict__ z1,
                                                                int64_t n1) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n0 + n1; i += stride) {
    if (i < n0) z0[i] = 0u;
    else z1[i - n0] = 0u;
  }
  const int64_t r = int64_t(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;                   // whole wave exits together
  const float2* p = part + r * n_chunk;
  float m = -INFINITY;
  for (int i = lane; i < n_chunk; i += 64) m = fmaxf(m, p[i].x);
  m = wave_max(m);
  double z = 0.0;
  for (int i = lane; i < n_chunk; i += 64)
    if (p[i].x != -INFINITY) z += double(p[i].y) * exp2(double(p[i].x) - double(m));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
  if (lane == 0) rowstat[r] = make_float2(m, float(1.0 / z));
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void score_pass2(const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        const float2* __restrict__ rowstat,
                                                        float* __restrict__ s, int Hq, int Hkv,
                                                        int L, int w, float c, int causal) {
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
      if (causal ? j <= r : j < L) {
        const float x = dot_scaled<D>(kr, qs + ri * D, c);
        acc += exp2f(x - st[ri].x) * st[ri].y;
      }
    }
  }
  if (j < L) s[int64_t(bh) * L + j] = acc / float(w);
}

// ---------------------------------------------------------------- bf16 MFMA
constexpr int kMWaves = 8;
constexpr int kMThreads = 64 * kMWaves;  // 8 waves: one proxy row tile each at the usual shapes
constexpr int kMPad = 8;                 // bf16 padding per K row in LDS
constexpr int kMTarget = 512;            // workgroups per pass the chunk grouping aims at

// Query heads of one KV head that a workgroup scores together: all of them
// when their proxy-row tiles fit the waves, else as many whole heads as fit
// (at least one).  Each 128-key chunk of K is then staged once per group.
int score_heads_per_group(int G, int w) {
  const int rt = (w + 31) / 32;
  if (G * rt <= kMWaves) return G;
  return rt >= kMWaves ? 1 : kMWaves / rt;
}

// One 128-key chunk of K as 16-byte pieces spread over the workgroup (rows past L read as 0).
template <int D>
struct KChunk {
  static constexpr int kCPR = D / 8;                        // pieces per row
  static constexpr int kN = kScoreChunk * kCPR / kMThreads;  // pieces per thread
  u32x4 r[kN];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ kg, int L, int j0) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int ch = threadIdx.x + kMThreads * i;
      const int row = ch / kCPR, col = ch % kCPR;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (j0 + row < L) z = *reinterpret_cast<const u32x4*>(kg + int64_t(j0 + row) * D + col * 8);
      r[i] = z;
    }
  }
  __device__ __forceinline__ void store(uint16_t (*ks)[D + kMPad]) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int ch = threadIdx.x + kMThreads * i;
      *reinterpret_cast<u32x4*>(&ks[ch / kCPR][(ch % kCPR) * 8]) = r[i];
    }
  }
};

// Q fragments of one 32-row proxy tile: lane holds q[row l%32][16t + 8*(l/32) .. +8];
// rows past w are zero.
template <int D>
__device__ __forceinline__ void load_q_tile(const uint16_t* __restrict__ qh, int L, int w, int r0,
                                            bf16x8 (&qf)[D / 16]) {
  const int lane = threadIdx.x & 63;
  const int r = r0 + (lane & 31), half = lane >> 5;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (r < w) z = *reinterpret_cast<const u32x4*>(qh + int64_t(L - w + r) * D + 16 * t + 8 * half);
    qf[t] = __builtin_bit_cast(bf16x8, z);
  }
}

__device__ __forceinline__ float xhalf_max(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float xhalf_other(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const int lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? sw[1] : sw[0]);
}

// Both passes: one workgroup per (group of cpg consecutive 128-key chunks, KV
// head, group of hpg of its query heads).  It walks its chunks with K
// double-buffered in LDS (the next chunk is loaded into registers while the
// current one is computed), and the proxy row tiles of its heads ("units",
// ceil(w/32) per head) are spread over the waves.  When there are no more
// units than waves, each wave keeps its unit's Q fragments in registers for
// the whole walk.  The arithmetic per (chunk, unit) is the same as one chunk
// on its own, so the result depends neither on cpg nor on hpg.

// Pass 1: per proxy row and chunk, (max, sum of exp2(x - max)) over the chunk's visible keys.
template <int D>
__global__ __launch_bounds__(kMThreads) void score_mfma_rowstats(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, float2* __restrict__ part,
    int Hq, int Hkv, int L, int w, int n_chunk, int cpg, int hpg, float c, int causal) {
  constexpr int KS = D / 16;
  __shared__ uint16_t ks[2][kScoreChunk][D + kMPad];
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv, RT = (w + 31) / 32;
  const int h0 = g * G + int(blockIdx.z) * hpg;            // first query head of this workgroup
  const int units = min(hpg, g * G + G - h0) * RT;
  const int ch0 = int(blockIdx.x) * cpg, ch1 = min(ch0 + cpg, n_chunk);
  if (ch0 >= ch1) return;                   // whole workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, half = lane >> 5;
  const uint16_t* kg = k + (int64_t(b) * Hkv + g) * L * D;
  const bool own = units <= kMWaves;
  bf16x8 qf[KS];
  if (own && wave < units)
    load_q_tile<D>(q + int64_t(b * Hq + h0 + wave / RT) * L * D, L, w, 32 * (wave % RT), qf);
  KChunk<D> kc;
  kc.load(kg, L, ch0 * kScoreChunk);
  kc.store(ks[0]);
  __syncthreads();
  const f32x16 zero = {};
  for (int ch = ch0; ch < ch1; ++ch) {
    const int buf = (ch - ch0) & 1;
    if (ch + 1 < ch1) kc.load(kg, L, (ch + 1) * kScoreChunk);
    const int j0 = ch * kScoreChunk;
    // keys of this chunk that some proxy row cannot see (causal), or keys past
    // L (either reading): masking needed
    const bool edge = causal ? j0 + kScoreChunk - 1 > L - w : j0 + kScoreChunk > L;
    for (int unit = wave; unit < units; unit += kMWaves) {
      const int h = h0 + unit / RT, r0 = 32 * (unit % RT);
      const int bh = b * Hq + h;
      if (!own) load_q_tile<D>(q + int64_t(bh) * L * D, L, w, r0, qf);
      const int r = r0 + l32;                 // this lane's proxy row
      const int pos = L - w + r;              // its sequence position
      // One loop for the chunks that need no mask and one for the edge
      // chunks, so the interior loop carries no compare or select.
      auto walk = [&](auto edge_c) {
        constexpr bool EDGE = decltype(edge_c)::value;
        float m = -INFINITY, z = 0.f;
        // Not unrolled: the rolled loop keeps the register count low enough
        // for two workgroups per CU.
#pragma unroll 1
        for (int kt = 0; kt < kScoreChunk / 32; ++kt) {
          f32x16 acc;
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ks[buf][32 * kt + l32][16 * t + 8 * half]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], t == 0 ? zero : acc, 0, 0, 0);
          }
          // Raw logits; c > 0, so the max of the scaled logits is the scaled max.
          if constexpr (EDGE) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = j0 + 32 * kt + 8 * (e >> 2) + 4 * half + (e & 3);
              if (key > (causal ? pos : L - 1) || r >= w) acc[e] = -INFINITY;
            }
          }
          float tm = acc[0];
#pragma unroll
          for (int e = 1; e < 16; ++e) tm = fmaxf(tm, acc[e]);
          const float mn = fmaxf(m, tm * c);
          if (mn == -INFINITY) continue;      // nothing visible yet for this lane
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f(fmaf(acc[e], c, -mn));
          z = z * __builtin_amdgcn_exp2f(m - mn) + sum;
          m = mn;
        }
        return make_float2(m, z);
      };
      const float2 mz = edge ? walk(std::true_type{}) : walk(std::false_type{});
      const float m = mz.x, z = mz.y;
      // combine the two lane halves, which saw different keys of the same row
      const float mo = xhalf_other(m), zo = xhalf_other(z);
      const float M = fmaxf(m, mo);
      float Z = 0.f;
      if (M != -INFINITY) {
        if (m != -INFINITY) Z += z * __builtin_amdgcn_exp2f(m - M);
        if (mo != -INFINITY) Z += zo * __builtin_amdgcn_exp2f(mo - M);
      }
      if (half == 0 && r < w) part[((int64_t(bh) * w) + r) * n_chunk + ch] = make_float2(M, Z);
    }
    if (ch + 1 < ch1) kc.store(ks[buf ^ 1]);
    __syncthreads();
  }
}

// Pass 2: column sums of the normalised proxy rows, per head, divided by w.
// Registers are capped for four waves per SIMD (two workgroups per CU when
// their LDS fits): 4% faster at 128K than one workgroup per CU, same bits.
template <int D>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(4))) void score_mfma_colsum(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float2* __restrict__ rowstat, float* __restrict__ s, int Hq, int Hkv, int L, int w,
    int n_chunk, int cpg, int hpg, float c, int causal) {
  constexpr int KS = D / 16;
  extern __shared__ float colsum[];       // [2][units][kScoreChunk]
  __shared__ uint16_t ks[2][kScoreChunk][D + kMPad];
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv, RT = (w + 31) / 32;
  const int h0 = g * G + int(blockIdx.z) * hpg;            // first query head of this workgroup
  const int nh = min(hpg, g * G + G - h0);                   // its query heads
  const int units = nh * RT;
  const int ch0 = int(blockIdx.x) * cpg, ch1 = min(ch0 + cpg, n_chunk);
  if (ch0 >= ch1) return;                   // whole workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, half = lane >> 5;
  const uint16_t* kg = k + (int64_t(b) * Hkv + g) * L * D;
  const bool own = units <= kMWaves;
  // Q fragments and the statistics of the 16 rows this lane holds in the
  // accumulator, for one unit
  bf16x8 qf[KS];
  float mrow[16], izrow[16];
  int pos0 = 0;              // sequence position of row 0 of the current unit
  auto load_unit = [&](int unit) {
    const int bh = b * Hq + h0 + unit / RT, r0 = 32 * (unit % RT);
    load_q_tile<D>(q + int64_t(bh) * L * D, L, w, r0, qf);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rr = r0 + 8 * (v >> 2) + 4 * half + (v & 3);
      float2 st = make_float2(0.f, 0.f);
      if (rr < w) st = rowstat[int64_t(bh) * w + rr];
      mrow[v] = st.x;
      izrow[v] = st.y;                    // 0 for padding rows: they add nothing
    }
    pos0 = L - w + r0;
  };
  if (own && wave < units) load_unit(wave);
  KChunk<D> kc;
  kc.load(kg, L, ch0 * kScoreChunk);
  kc.store(ks[0]);
  __syncthreads();
  const f32x16 zero = {};
  for (int ch = ch0; ch < ch1; ++ch) {
    const int buf = (ch - ch0) & 1;
    float* cs_buf = colsum + buf * units * kScoreChunk;
    if (ch + 1 < ch1) kc.load(kg, L, (ch + 1) * kScoreChunk);
    const int j0 = ch * kScoreChunk;
    // causal: keys of this chunk that some proxy row cannot see.  Keys past L
    // never reach s, so the non-causal reading needs no mask here.
    const bool edge = causal && j0 + kScoreChunk - 1 > L - w;
    for (int unit = wave; unit < units; unit += kMWaves) {
      if (!own) load_unit(unit);
      // One loop for the chunks that need no mask and one for the edge
      // chunks, so the interior loop carries no compare or select.
      auto walk = [&](auto edge_c) {
        constexpr bool EDGE = decltype(edge_c)::value;
        // Not unrolled: the rolled loop keeps the register count low enough
        // for two workgroups per CU.
#pragma unroll 1
        for (int kt = 0; kt < kScoreChunk / 32; ++kt) {
          f32x16 acc;
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&ks[buf][32 * kt + l32][16 * t + 8 * half]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t], bk, t == 0 ? zero : acc, 0, 0, 0);
          }
          if constexpr (EDGE) {
            const int key = j0 + 32 * kt + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (key > pos0 + 8 * (v >> 2) + 4 * half + (v & 3)) acc[v] = -INFINITY;
          }
          // two independent sums of the rows this lane holds, added at the end
          float cs0 = 0.f, cs1 = 0.f;
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            cs0 = fmaf(__builtin_amdgcn_exp2f(fmaf(acc[v], c, -mrow[v])), izrow[v], cs0);
            cs1 = fmaf(__builtin_amdgcn_exp2f(fmaf(acc[v + 1], c, -mrow[v + 1])), izrow[v + 1], cs1);
          }
          float csum = cs0 + cs1;
          csum += xhalf_other(csum);
          if (half == 0) cs_buf[unit * kScoreChunk + 32 * kt + l32] = csum;
        }
      };
      if (edge) walk(std::true_type{});
      else walk(std::false_type{});
    }
    if (ch + 1 < ch1) kc.store(ks[buf ^ 1]);
    __syncthreads();
    // s = (sum over the head's row tiles, in tile order) / w
    for (int i = threadIdx.x; i < nh * kScoreChunk; i += kMThreads) {
      const int hl = i / kScoreChunk, kk = i % kScoreChunk;
      const int j = j0 + kk;
      if (j >= L) continue;
      float acc = 0.f;
      for (int rt = 0; rt < RT; ++rt) acc += cs_buf[(hl * RT + rt) * kScoreChunk + kk];
      s[(int64_t(b) * Hq + h0 + hl) * L + j] = acc / float(w);
    }
  }
}

template <typename T, int D>
hipError_t run(const Shape& sh, const void* q, const void* k, float* scores, char* ws,
               hipStream_t st, const StepClear& z) {
  const StepWs lay = step_ws_layout(sh);
  float2* part = reinterpret_cast<float2*>(ws + lay.part);
  float2* rowstat = reinterpret_cast<float2*>(ws + lay.rowstat);
  const float c = kLog2e / sqrtf(float(D));
  const int nc = sh.n_chunk();
  const int64_t rows = int64_t(sh.B) * sh.Hq * sh.w;
  if constexpr (std::is_same<T, uint16_t>::value) {
    const int heads_kv = sh.B * sh.Hkv;
    const int hpg = score_heads_per_group(sh.G(), sh.w);
    const int ngroups = (sh.G() + hpg - 1) / hpg;
    const int cpg = max(1, (nc * heads_kv * ngroups + kMTarget - 1) / kMTarget);   // chunks per workgroup
    const dim3 grid((nc + cpg - 1) / cpg, heads_kv, ngroups);
    const int units = hpg * ((sh.w + 31) / 32);
    const size_t colsum_bytes = sizeof(float) * 2 * size_t(units) * kScoreChunk;
    score_mfma_rowstats<D><<<grid, kMThreads, 0, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), part, sh.Hq, sh.Hkv,
        sh.L, sh.w, nc, cpg, hpg, c, int(sh.causal_proxy()));
    score_merge<<<unsigned((rows + kMergeWaves - 1) / kMergeWaves), 64 * kMergeWaves, 0, st>>>(
        part, rowstat, rows, nc, z.p0, z.n0, z.p1, z.n1);
    score_mfma_colsum<D><<<grid, kMThreads, colsum_bytes, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), rowstat, scores, sh.Hq,
        sh.Hkv, sh.L, sh.w, nc, cpg, hpg, c, int(sh.causal_proxy()));
  } else {
    const dim3 grid(nc, sh.B * sh.Hq);
    score_pass1<T, D><<<grid, kThreads, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                 part, sh.Hq, sh.Hkv, sh.L, sh.w, nc, c,
                                                 int(sh.causal_proxy()));
    score_merge<<<unsigned((rows + kMergeWaves - 1) / kMergeWaves), 64 * kMergeWaves, 0, st>>>(
        part, rowstat, rows, nc, z.p0, z.n0, z.p1, z.n1);
    score_pass2<T, D><<<grid, kThreads, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                 rowstat, scores, sh.Hq, sh.Hkv, sh.L, sh.w, c,
                                                 int(sh.causal_proxy()));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const Shape& sh, const void* q, const void* k, float* scores, char* ws,
                        hipStream_t st, const StepClear* clear) {
  const StepClear z = clear ? *clear : StepClear{nullptr, 0, nullptr, 0};
  if (sh.dtype == TSA_BF16)
    return sh.d == 128 ? run<uint16_t, 128>(sh, q, k, scores, ws, st, z)
                       : run<uint16_t, 64>(sh, q, k, scores, ws, st, z);
  return sh.d == 128 ? run<float, 128>(sh, q, k, scores, ws, st, z)
                     : run<float, 64>(sh, q, k, scores, ws, st, z);
}

}  // namespace tsa
