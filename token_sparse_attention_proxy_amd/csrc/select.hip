// Per-head selection: "Dynamic Token Coverage", per-head selection
// (gist.science summary of Token Sparse Attention, section 2).  With the
// global budget K fixed, each head independently keeps its own top-K tokens
// by its own scores.  Order: score descending, then index ascending, so the
// chosen set is unique.  The set is written in ascending index order (which
// keeps the causal order of the compressed sequence), with the inverse map.
//
// Scores are non-negative floats, so their bit patterns order like the
// values; NaN and negative values rank as 0.  One workgroup per head:
//   1. radix descent (11/11/10-bit digits) finds T, the K-th largest key;
//   2. with c_gt = #{key > T} and need = K - c_gt, token j is kept when
//      key_j > T, or key_j == T and fewer than `need` T-valued tokens
//      precede it; one block scan per 4096 tokens (four contiguous tokens
//      per thread) of the packed (greater, equal) counts gives every kept
//      token its output slot.
// Both phases walk the scores four contiguous tokens per thread per step,
// with the next step's loads issued before the current step's work.
// Only integer operations are involved: results are bit-exact and
// deterministic.
//
// Kept window (alternative reading): the last `keep` positions are always
// in the set; the radix selection then runs over the first L - keep tokens
// with K - keep slots, and the window fills slots K - keep .. K - 1.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kBuckets = 2048;
constexpr int kPer = 4;                 // contiguous tokens per thread per step (a multiple of 4)
constexpr int kStep = kThreads * kPer;

__device__ __forceinline__ uint32_t score_key(float x) {
  return (x > 0.0f) ? __float_as_uint(x) : 0u;   // NaN, -0, negatives -> 0
}

// Keys of tokens j0 .. j0 + kPer - 1 (0 past nc); one 16-byte load when aligned.
__device__ __forceinline__ void load_keys(const float* __restrict__ sh, int j0, int nc, bool vec,
                                          uint32_t (&u)[kPer]) {
  if (vec && j0 + kPer <= nc) {
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sh + j0 + 4 * v);
#pragma unroll
      for (int q = 0; q < 4; ++q) u[4 * v + q] = score_key(x[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPer; ++q) u[q] = j0 + q < nc ? score_key(sh[j0 + q]) : 0u;
  }
}

__global__ __launch_bounds__(kThreads) void select_topk(const float* __restrict__ s,
                                                        const int32_t* __restrict__ budget,
                                                        int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ rank, int Hq,
                                                        int L, int bud_b, int bud_h, int keep) {
  __shared__ uint32_t hist[kBuckets];
  __shared__ uint64_t scan_tmp[17];
  __shared__ int dsel;
  __shared__ uint32_t sh_above;
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int t = threadIdx.x;
  const int K = min(max(budget[b * bud_b + h * bud_h], 0), L);
  const int nc = L - keep;                      // candidates: tokens before the kept window
  const int Kc = max(K - keep, 0);              // slots filled by selection
  const float* sh = s + int64_t(bh) * L;
  int32_t* ih = idx + int64_t(bh) * L;
  int32_t* rh = rank + int64_t(bh) * L;
  const bool vec = (L % kPer) == 0 && (reinterpret_cast<uintptr_t>(s) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(rank) % 16) == 0;   // rows start 16-byte aligned

  // ---- 1. the K-th largest key T
  uint32_t prefix = 0, above = 0;
  const int widths[3] = {11, 11, 10};
  int lo = 32;
  for (int lev = 0; lev < 3; ++lev) {
    const int width = widths[lev];
    const int hi = lo;
    lo -= width;
    for (int i = t; i < kBuckets; i += kThreads) hist[i] = 0;
    if (t == 0) dsel = -1;
    __syncthreads();
    uint32_t u[kPer], un[kPer];
    load_keys(sh, kPer * t, nc, vec, u);
    for (int base = 0; base < nc; base += kStep) {
      load_keys(sh, base + kStep + kPer * t, nc, vec, un);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint32_t top = hi >= 32 ? 0u : (u[q] >> hi);
        if (base + kPer * t + q < nc && top == prefix)
          atomicAdd(&hist[(u[q] >> lo) & ((1u << width) - 1u)], 1u);
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) u[q] = un[q];
    }
    __syncthreads();
    // Thread t owns digits dA = 2047-2t and dB = dA-1 (descending order).
    const int dA = kBuckets - 1 - 2 * t, dB = dA - 1;
    const uint32_t cA = hist[dA], cB = hist[dB];
    uint64_t tot;
    const uint64_t excl = block_excl_scan_u64(uint64_t(cA) + cB, scan_tmp, &tot);
    // largest digit whose cumulative count from the top reaches K
    if (uint64_t(above) + excl + cA >= uint64_t(Kc)) atomicMax(&dsel, dA);
    else if (uint64_t(above) + excl + cA + cB >= uint64_t(Kc)) atomicMax(&dsel, dB);
    __syncthreads();
    const int d = dsel < 0 ? 0 : dsel;
    if (t == ((kBuckets - 1 - d) >> 1)) sh_above = above + uint32_t(excl) + ((d == dB) ? cA : 0u);
    __syncthreads();
    above = sh_above;
    prefix = (prefix << width) | uint32_t(d);
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need = uint32_t(Kc) - above;  // T-valued tokens to keep, lowest indices first

  // ---- 2. ascending compaction
  uint32_t carry_gt = 0, carry_eq = 0;
  uint32_t u[kPer], un[kPer];
  load_keys(sh, kPer * t, nc, vec, u);
  for (int base = 0; base < nc; base += kStep) {
    const int j0 = base + kPer * t;
    load_keys(sh, j0 + kStep, nc, vec, un);
    uint32_t gt[kPer], eq[kPer], ngt = 0, neq = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const bool in = j0 + q < nc;
      gt[q] = in && u[q] > T;
      eq[q] = in && u[q] == T;
      ngt += gt[q];
      neq += eq[q];
    }
    uint64_t tot;
    const uint64_t ex = block_excl_scan_u64((uint64_t(ngt) << 32) | neq, scan_tmp, &tot);
    uint32_t gt_before = carry_gt + uint32_t(ex >> 32);
    uint32_t eq_before = carry_eq + uint32_t(ex & 0xffffffffu);
    int32_t rk[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const bool kept = gt[q] || (eq[q] && eq_before < need);
      const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
      if (kept && j0 + q < nc) ih[pos] = j0 + q;
      rk[q] = kept ? int32_t(pos) : -1;
      gt_before += gt[q];
      eq_before += eq[q];
    }
    if (vec && j0 + kPer <= nc) {
#pragma unroll
      for (int v = 0; v < kPer / 4; ++v)
        *reinterpret_cast<int4*>(rh + j0 + 4 * v) = make_int4(rk[4 * v], rk[4 * v + 1], rk[4 * v + 2], rk[4 * v + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (j0 + q < nc) rh[j0 + q] = rk[q];
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) u[q] = un[q];
    carry_gt += uint32_t(tot >> 32);
    carry_eq += uint32_t(tot & 0xffffffffu);
  }
  // the kept window, in order after the selected candidates
  for (int j = nc + t; j < L; j += kThreads) {
    const int pos = Kc + (j - nc);
    ih[pos] = j;
    rh[j] = pos;
  }
  for (int i = Kc + keep + t; i < L; i += kThreads) ih[i] = -1;
}

}  // namespace

hipError_t launch_select(const Shape& sh, const float* scores, const int32_t* budget,
                         int32_t* idx, int32_t* rank, char* ws, hipStream_t st) {
  (void)ws;
  select_topk<<<sh.B * sh.Hq, kThreads, 0, st>>>(scores, budget, idx, rank, sh.Hq, sh.L,
                                                 sh.bud_b(), sh.bud_h(), sh.keep());
  return hipGetLastError();
}

}  // namespace tsa
