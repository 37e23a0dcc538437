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
// The cut is found without sorting, over the whole GPU:
//   1. sigma pass (many workgroups): sigma_j, and a histogram of (count,
//      exact mass) over 4096 log-scale buckets of sigma (bit length and the
//      six bits after the leading one: monotonic in sigma), merged into a
//      global histogram with integer atomics;
//   2. extract pass (many workgroups): every workgroup scans the histogram
//      in ascending order to the first bucket where the running mass
//      exceeds thr (the same integer scan everywhere), and copies that
//      bucket's values into a candidate list (order free: only the multiset
//      matters below);
//   3. cut, in the same launch, by the last workgroup of each budget row to
//      finish its extraction (a counter taken after a device-scope fence
//      tells it that every candidate is written; no workgroup waits): every
//      value below the bucket is pruned; inside it, a most-significant-digit
//      radix descent over the candidates (in LDS when they fit) moves into
//      the first digit bucket whose running mass exceeds what is left of
//      thr, and stops when that bucket holds one value or all bits are
//      fixed; all values left are then equal and P follows in closed form.
//
// Alternative readings: with per-head budgets each (b, h) is a row of its
// own (sigma = that head's quantised scores, thr = floor(tau*2^50)); with a
// kept window only the first L - w tokens are candidates and
// P = max{p in [0, min(L - w, L - 1)] : C(p) <= thr}.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

constexpr int kThreads = 256;                // sigma pass
constexpr int kPer = 4;                      // sigma pass: tokens per thread (one 16-byte load per head)
constexpr int kSigChunk = kThreads * kPer;   // tokens per sigma workgroup
constexpr int kCutThreads = 1024;            // extract and cut
constexpr int kExPer = 2;                    // extract pass: tokens per thread (one 16-byte load)
constexpr int kExChunk = kCutThreads * kExPer;   // tokens per extract workgroup
constexpr int kLogBuckets = kBudgetLogBuckets;   // 4096: 6 bits of bit length, 6 after the leading one
constexpr int kDigitBits = 11;
constexpr int kBuckets = 1 << kDigitBits;
constexpr int kCandLds = 12288;              // candidates held in LDS by the cut (96 KiB)
// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt 0 only (expcnt 7
// and lgkmcnt 15 do not wait): every vector memory operation of the wave,
// stores included, has completed.
constexpr int kWaitVmem = 0x0f70;

__device__ __forceinline__ uint64_t quantise(float x) {
  // fmaxf/fminf return the non-NaN operand, so NaN counts as 0.
  x = fminf(fmaxf(x, 0.0f), 1.0f);
  return uint64_t(double(x) * 1125899906842624.0);   // * 2^50, exact; truncation = floor
}

// Log-scale bucket of v: (bit length) * 64 + the six bits after the leading
// one (the low bits, zero-padded, when v has fewer than seven bits).  Equal
// values share a bucket and a larger value never gets a smaller bucket.
__device__ __forceinline__ int log_bucket(uint64_t v) {
  if (v == 0) return 0;
  const int e = 64 - __clzll((long long)v);           // 1 .. 64
  const uint32_t m = e >= 7 ? uint32_t(v >> (e - 7)) & 63u : uint32_t(v << (7 - e)) & 63u;
  return (min(e, 63) << 6) | int(m);
}

__global__ void clear_words(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// sigma[r,j] = sum over the hpr query heads of budget row r of the quantised
// score (exact integers, so the order does not matter), for the nc candidate
// tokens j < nc; and the row's log-bucket histogram of sigma (count, mass),
// gathered in LDS per workgroup and merged into the row's histogram with
// integer atomics.
__global__ __launch_bounds__(kThreads) void budget_sigma(const float* __restrict__ s,
                                                         uint64_t* __restrict__ sigma,
                                                         uint32_t* __restrict__ hcnt,
                                                         uint64_t* __restrict__ hmass, int hpr,
                                                         int L, int nc) {
  __shared__ uint32_t lc[kLogBuckets];
  __shared__ uint64_t lm[kLogBuckets];
  const int r = blockIdx.y;
  const int t = threadIdx.x;
  for (int i = t; i < kLogBuckets; i += kThreads) {
    lc[i] = 0u;
    lm[i] = 0u;
  }
  const int j = int(blockIdx.x) * kSigChunk + kPer * t;
  const float* sr = s + int64_t(r) * hpr * L;
  const bool vec = (L % kPer) == 0 && (reinterpret_cast<uintptr_t>(s) % 16) == 0;
  uint64_t acc[kPer] = {0, 0, 0, 0};
  if (vec && j + kPer <= nc) {
#pragma unroll 8
    for (int h = 0; h < hpr; ++h) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sr + int64_t(h) * L + j);
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] += quantise(x[q]);
    }
  } else {
    for (int h = 0; h < hpr; ++h)
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (j + q < nc) acc[q] += quantise(sr[int64_t(h) * L + j + q]);
  }
  __syncthreads();                        // the LDS histogram is clear
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (j + q < nc) {
      sigma[int64_t(r) * L + j + q] = acc[q];
      const int bk = log_bucket(acc[q]);
      atomicAdd(&lc[bk], 1u);
      atomicAdd(reinterpret_cast<unsigned long long*>(&lm[bk]), (unsigned long long)acc[q]);
    }
  }
  __syncthreads();
  uint32_t* gc = hcnt + int64_t(r) * kLogBuckets;
  uint64_t* gm = hmass + int64_t(r) * kLogBuckets;
  for (int i = t; i < kLogBuckets; i += kThreads) {
    if (lc[i]) {
      atomicAdd(&gc[i], lc[i]);
      atomicAdd(reinterpret_cast<unsigned long long*>(&gm[i]), (unsigned long long)lm[i]);
    }
  }
}

// Ascending scan of the log histogram: the first bucket whose running mass
// exceeds thr, with the count and mass of all buckets below it
// (crossed = 0: the whole candidate mass stays within thr).  The same in
// every workgroup; contains barriers.
struct Cross {
  uint64_t mass_below, cnt_below;
  int bucket, crossed;
};
template <int NT>
__device__ __forceinline__ Cross find_cross(const uint32_t* __restrict__ hc,
                                            const uint64_t* __restrict__ hm, uint64_t thr,
                                            uint64_t* tmp, uint64_t* sh) {
  constexpr int kLogPerThread = kLogBuckets / NT;
  const int t = threadIdx.x;
  const int d0 = kLogPerThread * t;              // this thread's buckets, ascending
  uint64_t m[kLogPerThread];
  uint64_t msum = 0, csum = 0;
#pragma unroll
  for (int i = 0; i < kLogPerThread; ++i) {
    m[i] = hm[d0 + i];
    msum += m[i];
    csum += hc[d0 + i];
  }
  if (t == 0) sh[0] = kLogBuckets;
  uint64_t tot;
  const uint64_t mex = block_excl_scan_u64(msum, tmp, &tot);
  const uint64_t cex = block_excl_scan_u64(csum, tmp, &tot);
  uint64_t run = mex;
  int found = -1;
#pragma unroll
  for (int i = 0; i < kLogPerThread; ++i) {
    if (found < 0 && run + m[i] > thr) found = d0 + i;
    run += m[i];
  }
  if (found >= 0) atomicMin(reinterpret_cast<unsigned long long*>(&sh[0]), (unsigned long long)found);
  __syncthreads();
  Cross c;
  c.bucket = int(sh[0]);
  c.crossed = c.bucket < kLogBuckets;
  if (c.crossed && t == c.bucket / kLogPerThread) {
    uint64_t mb = mex, cb = cex;
#pragma unroll
    for (int i = 0; i < kLogPerThread; ++i)
      if (d0 + i < c.bucket) {
        mb += m[i];
        cb += hc[d0 + i];
      }
    sh[1] = mb;
    sh[2] = cb;
  }
  __syncthreads();
  c.mass_below = c.crossed ? sh[1] : 0;
  c.cnt_below = c.crossed ? sh[2] : 0;
  __syncthreads();
  return c;
}

// The values of the crossing bucket, appended to cand[r] by every workgroup
// of row r (ncand[r] counts them; one atomic per workgroup reserves its
// slots), then the exact cut inside the bucket by the last workgroup of the
// row to finish: done[r] counts finished workgroups.  Each workgroup's
// candidate stores are made visible device-wide before its count (release),
// and the last workgroup's reads come after its count (acquire), so it sees
// every candidate.  No workgroup waits for another.
__global__ __launch_bounds__(kCutThreads) void budget_extract_cut(
    const uint64_t* __restrict__ sigma, const uint32_t* __restrict__ hcnt,
    const uint64_t* __restrict__ hmass, uint64_t* __restrict__ cand_g,
    uint32_t* __restrict__ ncand, uint32_t* __restrict__ done, int32_t* __restrict__ budget,
    int L, int nc, int pmax, uint64_t thr) {
  __shared__ uint64_t cand_s[kCandLds];
  __shared__ uint32_t cnt[kBuckets];
  __shared__ uint64_t mass[kBuckets];
  __shared__ uint64_t scan_tmp[17];
  __shared__ uint64_t sh[3];
  __shared__ uint32_t base_s;
  __shared__ int last_s;
  __shared__ int first_cross;
  __shared__ uint64_t sh_below_mass, sh_bucket_mass;
  __shared__ uint32_t sh_below_cnt, sh_bucket_cnt;

  const int r = blockIdx.y;
  const int t = threadIdx.x;
  const int j0 = int(blockIdx.x) * kExChunk + kExPer * t;
  const uint64_t* sg = sigma + int64_t(r) * L;
  uint64_t v[kExPer];
#pragma unroll
  for (int q = 0; q < kExPer; ++q) v[q] = j0 + q < nc ? sg[j0 + q] : 0;   // in flight during the scan
  const Cross c = find_cross<kCutThreads>(hcnt + int64_t(r) * kLogBuckets,
                                          hmass + int64_t(r) * kLogBuckets, thr, scan_tmp, sh);
  uint64_t* cand_row = cand_g + int64_t(r) * L;
  if (c.crossed) {                                 // uniform over the workgroup
    uint32_t nhit = 0;
#pragma unroll
    for (int q = 0; q < kExPer; ++q) {
      const int j = j0 + q;
      const bool hit = j < nc && log_bucket(v[q]) == c.bucket;
      nhit += hit;
      if (!hit) v[q] = ~uint64_t(0);             // marks a miss (no sigma reaches 2^64 - 1)
    }
    uint64_t total;
    const uint64_t off = block_excl_scan_u64(nhit, scan_tmp, &total);
    if (total > 0) {                               // uniform
      if (t == 0) base_s = atomicAdd(&ncand[r], uint32_t(total));
      __syncthreads();
      uint64_t* cr = cand_row + base_s + off;
      uint32_t k = 0;
#pragma unroll
      for (int q = 0; q < kExPer; ++q)
        if (v[q] != ~uint64_t(0)) cr[k++] = v[q];
    }
  }
  // Every wave waits until its candidate stores have reached the L2; after
  // the barrier, thread 0's release increment writes the L2 back before the
  // count is taken, so every candidate of the workgroup is visible device-wide
  // by then.  The workgroup that takes the last count invalidates its caches
  // (acquire) before reading: one write-back per workgroup, one invalidation
  // per row.
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  __syncthreads();
  if (t == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(&done[r], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == gridDim.x - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    last_s = last;
  }
  __syncthreads();
  if (!last_s) return;                   // whole workgroup

  if (!c.crossed) {                      // the whole candidate mass stays within thr
    if (t == 0) budget[r] = L - pmax;
    return;
  }
  const uint64_t mass_out = c.mass_below;   // pruned: every value below the bucket
  const uint64_t cnt_out = c.cnt_below;
  const int n = int(__hip_atomic_load(&ncand[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const uint64_t* cand = cand_row;
  if (n <= kCandLds) {
    for (int i = t; i < n; i += kCutThreads) cand_s[i] = cand[i];
    cand = cand_s;                      // generic pointer to LDS from here on
  }
  __syncthreads();
  // Every candidate shares the bit length e and the top seven bits.
  const int e = c.bucket >> 6;
  int lo = e > 7 ? e - 7 : 0;           // bits below the shared prefix
  const uint64_t room = thr - mass_out;
  uint64_t prefix = n > 0 ? (cand[0] >> lo) : 0;
  uint64_t mass_below = 0, cnt_below = 0;   // within the bucket
  uint64_t n_eq = uint64_t(n), T = n > 0 ? cand[0] : 1;
  while (lo > 0) {
    const int width = lo < kDigitBits ? lo : kDigitBits;
    lo -= width;
    const int hi = lo + width;
    for (int i = t; i < kBuckets; i += kCutThreads) {
      cnt[i] = 0;
      mass[i] = 0;
    }
    if (t == 0) first_cross = kBuckets;
    __syncthreads();
    for (int i = t; i < n; i += kCutThreads) {
      const uint64_t v = cand[i];
      if ((v >> hi) == prefix) {
        const int dgt = int((v >> lo) & uint64_t(kBuckets - 1));
        atomicAdd(&cnt[dgt], 1u);
        atomicAdd(reinterpret_cast<unsigned long long*>(&mass[dgt]), (unsigned long long)v);
      }
    }
    __syncthreads();
    // Each thread owns two consecutive buckets; exclusive scan of their masses.
    const int d0 = 2 * t;
    const uint64_t m0 = mass[d0], m1 = mass[d0 + 1];
    uint64_t total;
    const uint64_t excl = block_excl_scan_u64(m0 + m1, scan_tmp, &total);
    const uint64_t left = room - mass_below;       // mass_below <= room holds throughout
    if (excl + m0 > left) atomicMin(&first_cross, d0);
    else if (excl + m0 + m1 > left) atomicMin(&first_cross, d0 + 1);
    __syncthreads();
    const int dstar = first_cross;    // exists: the bucket's total mass exceeds room
    if (t == (dstar >> 1)) {
      sh_below_mass = excl + ((dstar & 1) ? m0 : 0);
      sh_bucket_mass = (dstar & 1) ? m1 : m0;
    }
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
      T = bucket_mass / n_eq;         // all values left in the digit bucket are equal
      break;
    }
  }
  if (t == 0) {
    // T > 0: a crossing bucket has positive mass
    const uint64_t m = (room - mass_below) / T;
    uint64_t P = cnt_out + cnt_below + (m < n_eq - 1 ? m : n_eq - 1);
    if (P > uint64_t(pmax)) P = uint64_t(pmax);
    budget[r] = int32_t(uint64_t(L) - P);
  }
}

__global__ void budget_fill(int32_t* __restrict__ budget, int rows, int L) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < rows) budget[i] = L;
}

}  // namespace

int64_t budget_clear_words(const Shape& sh) {
  const StepWs lay = step_ws_layout(sh);
  return int64_t(lay.bud_ncand + sizeof(uint32_t) * 2 * size_t(sh.bud_rows()) - lay.bud_hcnt) /
         int64_t(sizeof(uint32_t));
}

hipError_t launch_budget(const Shape& sh, const float* scores, int32_t* budget, char* ws,
                         hipStream_t st, bool cleared) {
  const int rows = sh.bud_rows();
  if (sh.tau == 0.0f) {   // tau = 0 prunes nothing
    budget_fill<<<(rows + 255) / 256, 256, 0, st>>>(budget, rows, sh.L);
    return hipGetLastError();
  }
  const StepWs lay = step_ws_layout(sh);
  uint64_t* sigma = reinterpret_cast<uint64_t*>(ws + lay.sigma);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + lay.bud_cand);
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(ws + lay.bud_hcnt);
  uint64_t* hmass = reinterpret_cast<uint64_t*>(ws + lay.bud_hmass);
  uint32_t* ncand = reinterpret_cast<uint32_t*>(ws + lay.bud_ncand);
  uint32_t* done = ncand + rows;
  const int hpr = sh.per_head() ? 1 : sh.Hq;     // query heads per budget row
  const int nc = sh.L - sh.keep();                // pruning candidates
  const int pmax = nc < sh.L - 1 ? nc : sh.L - 1;
  // floor(hpr * tau * 2^50): tau has a 24-bit significand and hpr <= 2^12, so
  // the product is exact in double.
  const double x = double(hpr) * double(sh.tau) * 1125899906842624.0;
  const uint64_t thr = uint64_t(x);
  if (!cleared) {
    // the count and mass histograms, the candidate and the finished-workgroup
    // counters are contiguous words
    const int64_t words = budget_clear_words(sh);
    clear_words<<<unsigned((words + 255) / 256), 256, 0, st>>>(hcnt, words);
  }
  budget_sigma<<<dim3((max(nc, 1) + kSigChunk - 1) / kSigChunk, rows), kThreads, 0, st>>>(
      scores, sigma, hcnt, hmass, hpr, sh.L, nc);
  budget_extract_cut<<<dim3((max(nc, 1) + kExChunk - 1) / kExChunk, rows), kCutThreads, 0, st>>>(
      sigma, hcnt, hmass, cand, ncand, done, budget, sh.L, nc, pmax, thr);
  return hipGetLastError();
}

}  // namespace tsa
