// Per-head selection: "Dynamic Token Coverage", per-head selection
// (gist.science summary of Token Sparse Attention, section 2).  With the
// global budget K fixed, each head independently keeps its own top-K tokens
// by its own scores.  Order: score descending, then index ascending, so the
// chosen set is unique.  The set is written in ascending index order (which
// keeps the causal order of the compressed sequence), with the inverse map.
//
// Scores are non-negative floats, so their bit patterns order like the
// values; NaN and negative values rank as 0.  The tokens of every head are
// split into chunks, one workgroup each, so the whole GPU works on the
// selection:
//   1. three histogram passes (11/11/10-bit digits of the key, most
//      significant first) find T, the K-th largest key.  Each pass adds its
//      chunk's LDS histogram to the head's global histogram with integer
//      atomics; every workgroup of the next pass reads that histogram and
//      picks the digit itself (the same integer scan in every workgroup), so
//      no pass waits on another inside a launch;
//   2. the last histogram pass also records, per chunk, the number of keys
//      above the 22-bit prefix and the suffix sums S[b] = #{keys on the
//      prefix with last digit >= b}, so that once the last digit d is known
//      (T = prefix:d) the chunk holds #{key > T} = above + S[d+1] and
//      #{key == T} = S[d] - S[d+1] keys;
//   3. the compaction pass picks d itself (the same scan in every
//      workgroup); with need = K - #{key > T}, token j is kept when
//      key_j > T, or key_j == T and fewer than `need` T-valued tokens precede
//      it.  A workgroup starts from the counts of the chunks before it and
//      runs a block scan per 1024 tokens of packed (greater, equal) counts,
//      which gives every kept token its output slot.
// Only integer operations are involved: results are bit-exact, deterministic
// and independent of the chunking.
//
// Kept window (alternative reading): the last `keep` positions are always
// in the set; the selection then runs over the first L - keep tokens with
// K - keep slots, and the window fills slots K - keep .. K - 1.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

constexpr int kThreads = 256;
constexpr int kBuckets = kSelectBuckets;
constexpr int kPer = 4;                         // contiguous tokens per thread per step
constexpr int kStep = kThreads * kPer;          // tokens per block step
constexpr int kDigitsPerThread = kBuckets / kThreads;
constexpr int kWidth[3] = {11, 11, 10};
constexpr int kLo[3] = {21, 10, 0};             // lowest key bit of each level's digit
constexpr int kTargetBlocks = 1024;             // workgroups per pass the chunking aims at
constexpr int kLastBins = 1 << kWidth[2];       // digits of the last level
static_assert(kSelectTabStride == kLastBins + 2, "per-chunk table: S[0..1024] and the count above");

__device__ __forceinline__ uint32_t score_key(float x) {
  return (x > 0.0f) ? __float_as_uint(x) : 0u;   // NaN, -0, negatives -> 0
}

// Keys of tokens j0 .. j0 + kPer - 1 (0 at or past j1); one 16-byte load when aligned.
__device__ __forceinline__ void load_keys(const float* __restrict__ sh, int j0, int j1, bool vec,
                                          uint32_t (&u)[kPer]) {
  if (vec && j0 + kPer <= j1) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(sh + j0);
#pragma unroll
    for (int q = 0; q < kPer; ++q) u[q] = score_key(x[q]);
  } else {
#pragma unroll
    for (int q = 0; q < kPer; ++q) u[q] = j0 + q < j1 ? score_key(sh[j0 + q]) : 0u;
  }
}

struct Head {
  int bh, K, nc, Kc;
  int j0, j1;                       // this workgroup's chunk of the candidates
  const float* s;
  bool vec;
};

__device__ __forceinline__ Head head_of(const float* __restrict__ s, const int32_t* __restrict__ budget,
                                        int Hq, int L, int bud_b, int bud_h, int keep, int chunk) {
  Head hd;
  hd.bh = blockIdx.y;
  const int b = hd.bh / Hq, h = hd.bh % Hq;
  hd.K = min(max(budget[b * bud_b + h * bud_h], 0), L);
  hd.nc = L - keep;                         // candidates: tokens before the kept window
  hd.Kc = max(hd.K - keep, 0);              // slots filled by selection
  hd.j0 = int(blockIdx.x) * chunk;
  hd.j1 = min(hd.j0 + chunk, hd.nc);
  hd.s = s + int64_t(hd.bh) * L;
  hd.vec = (L % kPer) == 0 && (reinterpret_cast<uintptr_t>(s) % 16) == 0;   // rows 16-byte aligned
  return hd;
}

// Digit pick of one level (every workgroup computes the same): the largest
// digit d whose count from the top, added to `above` (tokens above the
// current range), reaches Kc; `above` becomes above + #{digits > d}.  With
// no such digit (not reachable for Kc <= candidates) d = 0.  Contains
// barriers; `tmp` holds 17 uint64 of LDS and `sel` two ints.
__device__ __forceinline__ void pick_digit(const uint32_t* __restrict__ hist, uint32_t Kc,
                                           uint32_t& d_out, uint32_t& above, uint64_t* tmp,
                                           int* sel) {
  const int t = threadIdx.x;
  const int dhi = kBuckets - 1 - kDigitsPerThread * t;   // this thread's digits, descending
  uint32_t c[kDigitsPerThread];
  uint64_t local = 0;
#pragma unroll
  for (int i = 0; i < kDigitsPerThread; ++i) {
    c[i] = hist[dhi - i];
    local += c[i];
  }
  if (t == 0) sel[0] = -1;
  uint64_t total;
  const uint64_t excl = block_excl_scan_u64(local, tmp, &total);   // barriers inside
  uint64_t run = uint64_t(above) + excl;
  int found = -1;
#pragma unroll
  for (int i = 0; i < kDigitsPerThread; ++i) {
    if (found < 0 && run + c[i] >= uint64_t(Kc)) found = dhi - i;
    run += c[i];
  }
  if (found >= 0) atomicMax(&sel[0], found);
  __syncthreads();
  const int d = sel[0] < 0 ? 0 : sel[0];
  if (t == (kBuckets - 1 - d) / kDigitsPerThread) {     // the owner of d: tokens above it
    uint64_t r = uint64_t(above) + excl;
#pragma unroll
    for (int i = 0; i < kDigitsPerThread; ++i)
      if (i < dhi - d) r += c[i];
    sel[1] = int(uint32_t(r));
  }
  __syncthreads();
  d_out = uint32_t(d);
  above = uint32_t(sel[1]);
  __syncthreads();
}

__global__ void sel_clear(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// One histogram level.  hist: [3][heads][kBuckets]; state: [3][heads][2]
// holds (prefix, above) after the pick of each level.
// The last level also writes the chunk's table for the compaction:
// tab[(head * nch + chunk) * kSelectTabStride + b] = S[b] for b <= 1024
// (S[1024] = 0), and entry 1025 = #{keys whose 22-bit prefix is above the
// picked one}.
template <int LEVEL>
__global__ __launch_bounds__(kThreads) void sel_level(const float* __restrict__ s,
                                                      const int32_t* __restrict__ budget,
                                                      uint32_t* __restrict__ hist,
                                                      uint32_t* __restrict__ state,
                                                      uint32_t* __restrict__ tab, int heads,
                                                      int Hq, int L, int bud_b, int bud_h,
                                                      int keep, int chunk, int nch) {
  __shared__ uint32_t lh[kBuckets];
  __shared__ uint64_t tmp[17];
  __shared__ int sel[2];
  const Head hd = head_of(s, budget, Hq, L, bud_b, bud_h, keep, chunk);
  const int t = threadIdx.x;
  uint32_t u[kPer], un[kPer];
  load_keys(hd.s, hd.j0 + kPer * t, hd.j1, hd.vec, u);   // in flight during the pick
  uint32_t prefix = 0, above = 0;
  if constexpr (LEVEL == 0) {
    if (blockIdx.x == 0) {                 // the later levels' histograms of this head
      for (int i = t; i < 2 * kBuckets; i += kThreads) {
        const int lv = 1 + i / kBuckets;
        hist[(int64_t(lv) * heads + hd.bh) * kBuckets + i % kBuckets] = 0u;
      }
    }
  }
  if constexpr (LEVEL >= 1) {
    if (LEVEL >= 2) {
      prefix = state[(int64_t(LEVEL - 2) * heads + hd.bh) * 2];
      above = state[(int64_t(LEVEL - 2) * heads + hd.bh) * 2 + 1];
    }
    uint32_t d;
    pick_digit(hist + (int64_t(LEVEL - 1) * heads + hd.bh) * kBuckets, uint32_t(hd.Kc), d, above,
               tmp, sel);
    prefix = (prefix << kWidth[LEVEL - 1]) | d;
    if (blockIdx.x == 0 && t == 0) {
      state[(int64_t(LEVEL - 1) * heads + hd.bh) * 2] = prefix;
      state[(int64_t(LEVEL - 1) * heads + hd.bh) * 2 + 1] = above;
    }
  }
  if (hd.j0 >= hd.j1) return;                       // whole workgroup
  constexpr int lo = kLo[LEVEL], hi = lo + kWidth[LEVEL];
  for (int i = t; i < kBuckets; i += kThreads) lh[i] = 0u;
  __syncthreads();
  uint32_t nabove = 0;                              // last level: keys above the prefix
  for (int base = hd.j0; base < hd.j1; base += kStep) {
    load_keys(hd.s, base + kStep + kPer * t, hd.j1, hd.vec, un);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const uint32_t top = hi >= 32 ? 0u : (u[q] >> hi);
      const bool in = base + kPer * t + q < hd.j1;
      if (in && top == prefix) atomicAdd(&lh[(u[q] >> lo) & ((1u << kWidth[LEVEL]) - 1u)], 1u);
      if constexpr (LEVEL == 2) nabove += in && top > prefix;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) u[q] = un[q];
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t(LEVEL) * heads + hd.bh) * kBuckets;
  for (int i = t; i < kBuckets; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
  if constexpr (LEVEL == 2) {
    // suffix sums of the chunk's last-digit histogram: thread t owns digits
    // 4t .. 4t + 3; S[b] = (keys on the prefix) - (those with digit < b)
    static_assert(kLastBins == kThreads * 4, "four digits per thread");
    uint32_t c[4];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = lh[4 * t + i];
      mine += c[i];
    }
    uint64_t tot;
    const uint64_t ex = block_excl_scan_u64((uint64_t(nabove) << 32) | mine, tmp, &tot);
    const uint32_t on_prefix = uint32_t(tot & 0xffffffffu);
    uint32_t below = uint32_t(ex & 0xffffffffu);
    uint32_t* tb = tab + (int64_t(hd.bh) * nch + blockIdx.x) * kSelectTabStride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tb[4 * t + i] = on_prefix - below;
      below += c[i];
    }
    if (t == 0) {
      tb[kLastBins] = 0u;
      tb[kLastBins + 1] = uint32_t(tot >> 32);
    }
  }
}

// Zeroes row j0 + 4 * l + q of o (vpr 16-byte vectors per row) for every
// lane l whose bit is set in the wave-uniform mask m: 64 / vpr rows per store
// instruction, lanes split as (row of the instruction, vector of the row).
__device__ __forceinline__ void zero_masked_rows(u32x4* __restrict__ o, int64_t hrow, int j0, int q,
                                                 uint64_t m, int vpr) {
  const int lane = threadIdx.x & 63;
  const int per = 64 / vpr, sub = lane / vpr, vec = lane % vpr;
  while (m) {
    int row = -1;                                  // this lane's token among the next `per`
    for (int i = 0; i < per; ++i) {
      const int bit = m ? __builtin_ctzll(m) : -1;
      m &= m - 1;
      if (i == sub) row = bit;
    }
    if (row >= 0)
      __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                  o + (hrow + j0 + 4 * row + q) * vpr + vec);
  }
}

// Picks the last digit (so T is known), then the ascending compaction of
// each chunk, then the kept window and the -1 fill, split over the
// workgroups by position.  Grid x covers ceil(L / chunk).  With zo set (the
// whole op), the rows of zo [B,Hq,L,vpr*16 bytes] of the candidates left out
// are zeroed as they are found, the decompression's zero part.
__global__ __launch_bounds__(kThreads) void sel_compact(const float* __restrict__ s,
                                                        const int32_t* __restrict__ budget,
                                                        const uint32_t* __restrict__ hist,
                                                        const uint32_t* __restrict__ state,
                                                        const uint32_t* __restrict__ tab,
                                                        int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ rank,
                                                        u32x4* __restrict__ zo, int vpr, int heads,
                                                        int Hq, int L, int bud_b, int bud_h,
                                                        int keep, int chunk, int nch) {
  __shared__ uint64_t tmp[17];
  __shared__ int sel[2];
  const Head hd = head_of(s, budget, Hq, L, bud_b, bud_h, keep, chunk);
  const int t = threadIdx.x;
  int32_t* ih = idx + int64_t(hd.bh) * L;
  int32_t* rh = rank + int64_t(hd.bh) * L;
  if (hd.j0 < hd.j1) {
    uint32_t u[kPer], un[kPer];
    load_keys(hd.s, hd.j0 + kPer * t, hd.j1, hd.vec, u);   // in flight during the pick
    const uint32_t prefix = state[(int64_t(1) * heads + hd.bh) * 2];
    uint32_t above = state[(int64_t(1) * heads + hd.bh) * 2 + 1];
    uint32_t d;
    pick_digit(hist + (int64_t(2) * heads + hd.bh) * kBuckets, uint32_t(hd.Kc), d, above, tmp,
               sel);
    // Kc = 0 keeps no candidate: a threshold above every key (keys are at
    // most 0x7f800000), with nothing above or equal to it in any chunk.
    const bool none = hd.Kc == 0;
    const uint32_t T = none ? 0xffffffffu : (prefix << kWidth[2]) | d;
    if (none) above = 0;
    const uint32_t need = uint32_t(hd.Kc) - above;   // T-valued tokens to keep, lowest first
    // Tokens above / equal to T in the chunks before this one, from the
    // tables of the last histogram pass (d < 1024 whenever Kc > 0), summed
    // by the first wave.
    if (t < 64) {
      uint64_t before = 0;
      if (!none) {
        for (int c = t; c < int(blockIdx.x); c += 64) {
          const uint32_t* tb = tab + (int64_t(hd.bh) * nch + c) * kSelectTabStride;
          const int dc = min(int(d), kLastBins);    // reads stay inside the chunk's table
          const uint32_t s_d = tb[dc], s_d1 = tb[min(dc + 1, kLastBins)];
          before += (uint64_t(tb[kLastBins + 1] + s_d1) << 32) | (s_d - s_d1);
        }
      }
      before = wave_incl_scan_u64(before);
      if (t == 63) tmp[16] = before;
    }
    __syncthreads();
    uint32_t carry_gt = uint32_t(tmp[16] >> 32), carry_eq = uint32_t(tmp[16] & 0xffffffffu);
    __syncthreads();                               // tmp is reused by the scans below
    const bool vrank = hd.vec && (reinterpret_cast<uintptr_t>(rank) % 16) == 0;
    for (int base = hd.j0; base < hd.j1; base += kStep) {
      const int j0 = base + kPer * t;
      load_keys(hd.s, j0 + kStep, hd.j1, hd.vec, un);
      uint32_t gt[kPer], eq[kPer], ngt = 0, neq = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const bool in = j0 + q < hd.j1;
        gt[q] = in && u[q] > T;
        eq[q] = in && u[q] == T;
        ngt += gt[q];
        neq += eq[q];
      }
      uint64_t tot;
      const uint64_t ex = block_excl_scan_u64((uint64_t(ngt) << 32) | neq, tmp, &tot);
      uint32_t gt_before = carry_gt + uint32_t(ex >> 32);
      uint32_t eq_before = carry_eq + uint32_t(ex & 0xffffffffu);
      int32_t rk[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const bool kept = gt[q] || (eq[q] && eq_before < need);
        const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
        if (kept) ih[pos] = j0 + q;
        rk[q] = kept ? int32_t(pos) : -1;
        gt_before += gt[q];
        eq_before += eq[q];
      }
      if (vrank && j0 + kPer <= hd.j1) {
        *reinterpret_cast<int4*>(rh + j0) = make_int4(rk[0], rk[1], rk[2], rk[3]);
      } else {
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          if (j0 + q < hd.j1) rh[j0 + q] = rk[q];
      }
      if (zo) {                                    // uniform over the grid
        const int jw = base + kPer * 64 * (t >> 6);   // first token of this wave's step
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          zero_masked_rows(zo, int64_t(hd.bh) * L, jw, q,
                           __ballot(j0 + q < hd.j1 && rk[q] < 0), vpr);
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) u[q] = un[q];
      carry_gt += uint32_t(tot >> 32);
      carry_eq += uint32_t(tot & 0xffffffffu);
    }
  }
  // positions p0 .. p1 of this workgroup: the kept window (tokens nc .. L-1
  // fill slots Kc ..), then -1 from slot Kc + keep on
  const int p0 = int(blockIdx.x) * chunk, p1 = min(p0 + chunk, L);
  for (int j = max(p0, hd.nc) + t; j < p1; j += kThreads) {
    const int pos = hd.Kc + (j - hd.nc);
    ih[pos] = j;
    rh[j] = pos;
  }
  for (int i = max(p0, hd.Kc + keep) + t; i < p1; i += kThreads) ih[i] = -1;
}

}  // namespace

SelectPlan select_plan(const Shape& sh) {
  SelectPlan p;
  const int heads = sh.B * sh.Hq;
  const int nc = sh.L - sh.keep();
  // chunks of whole block steps, about kTargetBlocks workgroups over all heads
  const int per_head = max(1, kTargetBlocks / heads);
  int chunk = (max(nc, 1) + per_head - 1) / per_head;
  chunk = max(kStep, (chunk + kStep - 1) / kStep * kStep);
  p.chunk = chunk;
  p.nch = max(1, (nc + chunk - 1) / chunk);
  p.ngrid = max(p.nch, (sh.L + chunk - 1) / chunk);
  return p;
}

hipError_t launch_select(const Shape& sh, const float* scores, const int32_t* budget,
                         int32_t* idx, int32_t* rank, char* ws, hipStream_t st, bool cleared,
                         void* zero_o) {
  const StepWs lay = step_ws_layout(sh);
  const SelectPlan p = select_plan(sh);
  const int heads = sh.B * sh.Hq;
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + lay.sel_hist);
  uint32_t* state = reinterpret_cast<uint32_t*>(ws + lay.sel_state);
  uint32_t* tab = reinterpret_cast<uint32_t*>(ws + lay.sel_tab);
  if (!cleared) {
    const int64_t nh = int64_t(heads) * kBuckets;   // level 0; level 0's pass clears the others
    sel_clear<<<unsigned((nh + 255) / 256), 256, 0, st>>>(hist, nh);
  }
  const dim3 grid(p.nch, heads);
  const int bb = sh.bud_b(), bhh = sh.bud_h(), keep = sh.keep();
  sel_level<0><<<grid, kThreads, 0, st>>>(scores, budget, hist, state, tab, heads, sh.Hq, sh.L,
                                          bb, bhh, keep, p.chunk, p.nch);
  sel_level<1><<<grid, kThreads, 0, st>>>(scores, budget, hist, state, tab, heads, sh.Hq, sh.L,
                                          bb, bhh, keep, p.chunk, p.nch);
  sel_level<2><<<grid, kThreads, 0, st>>>(scores, budget, hist, state, tab, heads, sh.Hq, sh.L,
                                          bb, bhh, keep, p.chunk, p.nch);
  sel_compact<<<dim3(p.ngrid, heads), kThreads, 0, st>>>(
      scores, budget, hist, state, tab, idx, rank, static_cast<u32x4*>(zero_o),
      int(sh.row_bytes() / 16), heads, sh.Hq, sh.L, bb, bhh, keep, p.chunk, p.nch);
  return hipGetLastError();
}

}  // namespace tsa
