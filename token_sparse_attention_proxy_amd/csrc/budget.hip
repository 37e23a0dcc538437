// Global budget: "Dynamic Token Coverage", budget allocation (gist.science
// summary of Token Sparse Attention, section 2).  Tokens are ordered by
// ascending importance and the low tail is pruned while the pruned mass
// stays within tau; the result is one budget shared by every head of the
// sequence.
//
// Importance of token j is the head-mean of the per-head scores.  It is
// counted exactly: sigma_j = sum_h floor(clip(s,0,1) * 2^50) is a 64-bit
// integer, so every sum below is exact and independent of reduction order.
// With C(p) the sum of the p smallest sigma and thr = floor(Hq*tau*2^50):
//   P = max{p in [0, L-1] : C(p) <= thr},  budget = L - P   (tau = 0: L).
//
// The cut is found without sorting: a most-significant-digit radix descent
// over the sigma values keeps (count, mass) histograms and at each level
// moves into the first digit bucket where the running mass exceeds thr.  It
// stops when that bucket holds one value or all bits are fixed; all values
// left in the bucket are then equal, and P follows in closed form.
//
// Alternative readings: with per-head budgets each (b, h) is a row of its
// own (sigma = that head's quantised scores, thr = floor(tau*2^50)); with a
// kept window only the first L - w tokens are candidates and
// P = max{p in [0, min(L - w, L - 1)] : C(p) <= thr}.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

constexpr int kSigmaThreads = 256;
constexpr int kCutThreads = 1024;
constexpr int kDigitBits = 11;
constexpr int kBuckets = 1 << kDigitBits;
constexpr int kPer = 4;                      // sigma values per thread per step of the cut
constexpr int kStep = kCutThreads * kPer;

// sigma[j0 .. j0 + kPer) (0 past nc); two 16-byte loads when aligned.
__device__ __forceinline__ void load_vals(const uint64_t* __restrict__ sg, int j0, int nc, bool vec,
                                          uint64_t (&v)[kPer]) {
  if (vec && j0 + kPer <= nc) {
#pragma unroll
    for (int q = 0; q < kPer; q += 2) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(sg + j0 + q);
      v[q] = uint64_t(x[0]) | (uint64_t(x[1]) << 32);
      v[q + 1] = uint64_t(x[2]) | (uint64_t(x[3]) << 32);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPer; ++q) v[q] = j0 + q < nc ? sg[j0 + q] : 0;
  }
}

__device__ __forceinline__ uint64_t quantise(float x) {
  // fmaxf/fminf return the non-NaN operand, so NaN counts as 0.
  x = fminf(fmaxf(x, 0.0f), 1.0f);
  return uint64_t(double(x) * 1125899906842624.0);   // * 2^50, exact; truncation = floor
}

__global__ void clear_u64(uint64_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// sigma[r,j] = sum over the hpr query heads of budget row r, in head order,
// of the quantised score, for the nc candidate tokens j < nc.
__global__ __launch_bounds__(kSigmaThreads) void budget_sigma(const float* __restrict__ s,
                                                              uint64_t* __restrict__ sigma,
                                                              uint64_t* __restrict__ sigmax,
                                                              int hpr, int L, int nc) {
  __shared__ uint64_t red[kSigmaThreads / 64];
  const int b = blockIdx.y;
  const int j = blockIdx.x * kSigmaThreads + threadIdx.x;
  uint64_t acc = 0;
  if (j < nc) {
    const float* sb = s + int64_t(b) * hpr * L + j;
    for (int h = 0; h < hpr; ++h) acc += quantise(sb[int64_t(h) * L]);
    sigma[int64_t(b) * L + j] = acc;
  }
  // block max, then one integer atomic per block
  uint64_t m = acc;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t y = __shfl_xor(m, o, 64);
    m = y > m ? y : m;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t mm = 0;
    for (int i = 0; i < kSigmaThreads / 64; ++i) mm = red[i] > mm ? red[i] : mm;
    atomicMax(reinterpret_cast<unsigned long long*>(sigmax + b), (unsigned long long)mm);
  }
}

// One workgroup per budget row: radix descent for the coverage cut over the
// nc candidates; P is at most pmax.
__global__ __launch_bounds__(kCutThreads) void budget_cut(const uint64_t* __restrict__ sigma,
                                                          const uint64_t* __restrict__ sigmax,
                                                          int32_t* __restrict__ budget, int L,
                                                          int nc, int pmax, uint64_t thr) {
  __shared__ uint32_t cnt[kBuckets];
  __shared__ uint64_t mass[kBuckets];
  __shared__ uint64_t scan_tmp[17];
  __shared__ int first_cross;
  __shared__ uint64_t sh_below_mass, sh_bucket_mass;
  __shared__ uint32_t sh_below_cnt, sh_bucket_cnt;

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const uint64_t* sg = sigma + int64_t(b) * L;
  const bool vec = (L % 2) == 0 && (reinterpret_cast<uintptr_t>(sigma) % 16) == 0;   // 16-byte rows
  const uint64_t maxv = sigmax[b];
  int lo = maxv ? 64 - __clzll((long long)maxv) : 1;   // bits above `lo` are zero for all values
  uint64_t prefix = 0;          // value of bits [lo + width, 64) shared by the candidates
  uint64_t mass_below = 0;      // exact mass of all values below the candidate range
  uint64_t cnt_below = 0;
  uint64_t n_eq = 0, T = 0;
  bool crossed = true;

  while (true) {
    const int width = lo < kDigitBits ? lo : kDigitBits;
    lo -= width;
    const int hi = lo + width;
    for (int i = t; i < kBuckets; i += kCutThreads) {
      cnt[i] = 0;
      mass[i] = 0;
    }
    if (t == 0) first_cross = kBuckets;
    __syncthreads();
    // Four values per thread per step, the next step's loads issued first.
    uint64_t v[kPer], vn[kPer];
    load_vals(sg, kPer * t, nc, vec, v);
    for (int base = 0; base < nc; base += kStep) {
      load_vals(sg, base + kStep + kPer * t, nc, vec, vn);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const uint64_t top = hi >= 64 ? 0 : (v[q] >> hi);
        if (base + kPer * t + q < nc && top == prefix) {
          const int dgt = int((v[q] >> lo) & uint64_t(kBuckets - 1));
          atomicAdd(&cnt[dgt], 1u);
          atomicAdd(reinterpret_cast<unsigned long long*>(&mass[dgt]), (unsigned long long)v[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) v[q] = vn[q];
    }
    __syncthreads();
    // Each thread owns two consecutive buckets; exclusive scan of their masses.
    const int d0 = 2 * t;
    const uint64_t m0 = mass[d0], m1 = mass[d0 + 1];
    uint64_t total;
    const uint64_t excl = block_excl_scan_u64(m0 + m1, scan_tmp, &total);
    const uint64_t room = thr - mass_below;       // mass_below <= thr holds throughout
    if (excl + m0 > room) atomicMin(&first_cross, d0);
    else if (excl + m0 + m1 > room) atomicMin(&first_cross, d0 + 1);
    __syncthreads();
    const int dstar = first_cross;
    if (dstar == kBuckets) {          // the whole candidate range stays within the threshold
      crossed = false;
      break;
    }
    // Mass of the buckets below d*: the owner of d* knows its prefix.
    if (t == (dstar >> 1)) {
      sh_below_mass = excl + ((dstar & 1) ? m0 : 0);
      sh_bucket_mass = (dstar & 1) ? m1 : m0;
    }
    // Count below d*: a second scan over the counts.
    const uint64_t c01 = uint64_t(cnt[d0]) + cnt[d0 + 1];
    uint64_t ctot;
    const uint64_t cex = block_excl_scan_u64(c01, scan_tmp, &ctot);
    if (t == (dstar >> 1)) {
      sh_below_cnt = uint32_t(cex + ((dstar & 1) ? cnt[d0] : 0));
      sh_bucket_cnt = cnt[dstar];
    }
    __syncthreads();
    mass_below += sh_below_mass;
    cnt_below += sh_below_cnt;
    n_eq = sh_bucket_cnt;
    const uint64_t bucket_mass = sh_bucket_mass;
    prefix = (prefix << width) | uint64_t(dstar);
    __syncthreads();
    if (n_eq == 1 || lo == 0) {
      T = bucket_mass / n_eq;         // all values left in the bucket are equal
      break;
    }
  }
  if (t == 0) {
    uint64_t P;
    if (!crossed) {
      P = uint64_t(pmax);
    } else {
      const uint64_t m = (thr - mass_below) / T;
      P = cnt_below + (m < n_eq - 1 ? m : n_eq - 1);
      if (P > uint64_t(pmax)) P = uint64_t(pmax);
    }
    budget[b] = int32_t(uint64_t(L) - P);
  }
}

__global__ void budget_fill(int32_t* __restrict__ budget, int rows, int L) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < rows) budget[i] = L;
}

}  // namespace

hipError_t launch_budget(const Shape& sh, const float* scores, int32_t* budget, char* ws,
                         hipStream_t st) {
  const int rows = sh.bud_rows();
  if (sh.tau == 0.0f) {   // tau = 0 prunes nothing
    budget_fill<<<(rows + 255) / 256, 256, 0, st>>>(budget, rows, sh.L);
    return hipGetLastError();
  }
  const StepWs lay = step_ws_layout(sh);
  uint64_t* sigma = reinterpret_cast<uint64_t*>(ws + lay.sigma);
  uint64_t* sigmax = reinterpret_cast<uint64_t*>(ws + lay.sigmax);
  const int hpr = sh.per_head() ? 1 : sh.Hq;     // query heads per budget row
  const int nc = sh.L - sh.keep();                // pruning candidates
  const int pmax = nc < sh.L - 1 ? nc : sh.L - 1;
  // floor(hpr * tau * 2^50): tau has a 24-bit significand and hpr <= 2^12, so
  // the product is exact in double.
  const double x = double(hpr) * double(sh.tau) * 1125899906842624.0;
  const uint64_t thr = uint64_t(x);
  clear_u64<<<(rows + 255) / 256, 256, 0, st>>>(sigmax, rows);
  if (nc > 0)
    budget_sigma<<<dim3((nc + kSigmaThreads - 1) / kSigmaThreads, rows), kSigmaThreads, 0, st>>>(
        scores, sigma, sigmax, hpr, sh.L, nc);
  budget_cut<<<rows, kCutThreads, 0, st>>>(sigma, sigmax, budget, sh.L, nc, pmax, thr);
  return hipGetLastError();
}

}  // namespace tsa
