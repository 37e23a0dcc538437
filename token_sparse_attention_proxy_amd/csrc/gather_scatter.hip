// Compression and decompression: "Core architecture", stages 1 and 2
// (gist.science summary of Token Sparse Attention, section 2).
//
// gather:  for i < K_b, qc[b,h,i] = Q[b,h,idx_i]; kc/vc[b,h,i] = K/V[b,g(h),idx_i]
// scatter: for every j < L, o[b,h,j] = rank_j >= 0 ? oc[b,h,rank_j] : 0
//
// Both are pure byte movement: rows are copied as 16-byte vectors, one row
// per group of lanes, with streaming (non-temporal) stores: the outputs are
// not read again by these kernels.  The scatter is destination-driven, so each output
// row is written exactly once (copied or zero-filled) and coalesced.
//
// zero_unselected: o[b,h,j] = 0 for every j with rank_j < 0.  It is the part
// of decompression left when the attention kernel itself writes the
// selected rows to their sequence positions.
//
// gather by rank (K and V only, the whole op): source-driven, each K/V row of
// a KV head is read once and written to every query head of the group that
// selected it, at its slot rank[b,h,j]: the same bytes as the gather, with
// the shared source rows read once instead of once per query head.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

constexpr int kThreads = 256;
// Rows per block, measured at the 128K shape: the gather of Q, K and V, the
// scatter and the source-driven K/V gather run best with 32 (the latter 2.4%
// faster than 64, 4% than 128), the index-driven K/V gather with 128.
constexpr int kRowsGatherQKV = 32;
constexpr int kRowsGatherKV = 128;
constexpr int kRowsScatter = 32;
constexpr int kZeroWaveRows = 256;     // zero fill: rows per wave
constexpr int kRowsByRank = 32;

// VPR: 16-byte vectors per row (row bytes / 16).  One block copies compact
// rows [i0, i0 + RPB) for all G query heads of one KV group, head
// after head: the heads of a group select nearly the same tokens, so their
// K/V source rows are read from HBM once and then hit in cache.  WQ = false
// gathers K and V only (the whole op reads Q through the index set).
template <int VPR, bool WQ, int RPB = WQ ? kRowsGatherQKV : kRowsGatherKV>
__global__ __launch_bounds__(kThreads) void gather_rows(
    const u32x4* __restrict__ q, const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ budget, u32x4* __restrict__ qc,
    u32x4* __restrict__ kc, u32x4* __restrict__ vc, int Hq, int Hkv, int L, int bud_b,
    int bud_h) {
  constexpr int kRowsPerPass = kThreads / VPR;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int i0 = blockIdx.x * RPB;
  const int sub = threadIdx.x / VPR, vec = threadIdx.x % VPR;
  const int64_t grow = (int64_t(b) * Hkv + g) * L;        // first row of (b,g)
  for (int hl = 0; hl < G; ++hl) {
    const int h = g * G + hl;
    const int n = min(max(budget[b * bud_b + h * bud_h], 0), L);
    if (i0 >= n) continue;
    const int i1 = min(i0 + RPB, n);
    const int64_t hrow = (int64_t(b) * Hq + h) * L;   // first row of (b,h)
    constexpr int R = RPB / kRowsPerPass;             // rows per thread, all loads first
    int src[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = i0 + sub + r * kRowsPerPass;
      src[r] = i < i1 ? idx[hrow + i] : -1;
    }
    u32x4 aq[R], ak[R], av[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const bool ok = src[r] >= 0 && src[r] < L;
      if constexpr (WQ) aq[r] = ok ? q[(hrow + src[r]) * VPR + vec] : z;
      ak[r] = ok ? k[(grow + src[r]) * VPR + vec] : z;
      av[r] = ok ? v[(grow + src[r]) * VPR + vec] : z;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = i0 + sub + r * kRowsPerPass;
      if (i < i1) {
        const int64_t dst = (hrow + i) * VPR + vec;
        if constexpr (WQ) __builtin_nontemporal_store(aq[r], qc + dst);
        __builtin_nontemporal_store(ak[r], kc + dst);
        __builtin_nontemporal_store(av[r], vc + dst);
      }
    }
  }
}

// One block takes source rows [j0, j0 + kRowsByRank) of one KV head (b, g):
// every load (K, V and the G rank entries of each row) is issued before the
// first store.
template <int VPR>
__global__ __launch_bounds__(kThreads) void gather_kv_by_rank(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int32_t* __restrict__ rank,
    u32x4* __restrict__ kc, u32x4* __restrict__ vc, int Hq, int Hkv, int L, int nc) {
  constexpr int kRowsPerPass = kThreads / VPR;
  constexpr int R = kRowsByRank / kRowsPerPass;     // rows per thread
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int j0 = blockIdx.x * kRowsByRank;
  const int sub = threadIdx.x / VPR, vec = threadIdx.x % VPR;
  const int64_t grow = (int64_t(b) * Hkv + g) * L;        // first row of (b,g)
  const int64_t hrow0 = (int64_t(b) * Hq + int64_t(g) * G) * L;   // first row of head (b, gG)
  u32x4 ak[R], av[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = j0 + sub + r * kRowsPerPass;
    const u32x4 z = {0u, 0u, 0u, 0u};
    ak[r] = j < nc ? k[(grow + j) * VPR + vec] : z;
    av[r] = j < nc ? v[(grow + j) * VPR + vec] : z;
  }
  for (int hl = 0; hl < G; ++hl) {
    const int64_t hrow = hrow0 + int64_t(hl) * L;
    int slot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = j0 + sub + r * kRowsPerPass;
      slot[r] = j < nc ? rank[hrow + j] : -1;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (slot[r] >= 0 && slot[r] < L) {
        const int64_t dst = (hrow + slot[r]) * VPR + vec;
        __builtin_nontemporal_store(ak[r], kc + dst);
        __builtin_nontemporal_store(av[r], vc + dst);
      }
    }
  }
}

template <int VPR>
__global__ __launch_bounds__(kThreads) void scatter_rows(const u32x4* __restrict__ oc,
                                                         const int32_t* __restrict__ rank,
                                                         u32x4* __restrict__ o, int L) {
  constexpr int kRowsPerPass = kThreads / VPR;
  constexpr int kIter = (kRowsScatter + kRowsPerPass - 1) / kRowsPerPass;
  const int bh = blockIdx.y;
  const int j0 = blockIdx.x * kRowsScatter;
  const int sub = threadIdx.x / VPR, vec = threadIdx.x % VPR;
  const int64_t hrow = int64_t(bh) * L;
  // rank entries, then the rows they select, then the stores: each phase's
  // loads overlap instead of every store waiting on its own two loads
  int r[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int j = j0 + sub + i * kRowsPerPass;
    r[i] = (j < L && sub + i * kRowsPerPass < kRowsScatter) ? rank[hrow + j] : -1;
  }
  u32x4 val[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    val[i] = u32x4{0u, 0u, 0u, 0u};
    if (r[i] >= 0 && r[i] < L) val[i] = oc[(hrow + r[i]) * VPR + vec];
  }
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int j = j0 + sub + i * kRowsPerPass;
    if (j < L && sub + i * kRowsPerPass < kRowsScatter)
      __builtin_nontemporal_store(val[i], o + (hrow + j) * VPR + vec);
  }
}

// Each wave takes kZeroWaveRows consecutive rows of one head in groups of
// 64: one coalesced load of the group's rank entries, a ballot of the
// unselected rows, and zero stores of 64 / VPR such rows per instruction.
// Most rows are selected, so most groups store nothing.
template <int VPR>
__global__ __launch_bounds__(kThreads) void zero_rows(const int32_t* __restrict__ rank,
                                                      u32x4* __restrict__ o, int L) {
  constexpr int kGroups = kZeroWaveRows / 64;
  constexpr int kRowsPerStore = 64 / VPR;
  static_assert(kGroups * 64 == kZeroWaveRows && kRowsPerStore * VPR == 64, "zero-fill shape");
  const int bh = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / VPR, vec = lane % VPR;
  const int64_t hrow = int64_t(bh) * L;
  const int jw = (int(blockIdx.x) * (kThreads / 64) + wave) * kZeroWaveRows;
  int r[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int j = jw + 64 * g + lane;
    r[g] = j < L ? rank[hrow + j] : 0;
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    uint64_t m = __ballot(r[g] < 0);         // wave-uniform: unselected rows of the group
    while (m) {
      int row = -1;                            // this lane's row among the next kRowsPerStore
#pragma unroll
      for (int t = 0; t < kRowsPerStore; ++t) {
        const int bit = m ? __builtin_ctzll(m) : -1;
        m &= m - 1;
        if (t == sub) row = bit;
      }
      if (row >= 0)
        __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, o + (hrow + jw + 64 * g + row) * VPR + vec);
    }
  }
}

template <int VPR>
hipError_t zero_vpr(const Shape& sh, const int32_t* rank, void* o, hipStream_t st) {
  constexpr int rows_per_block = kZeroWaveRows * (kThreads / 64);
  dim3 grid((sh.L + rows_per_block - 1) / rows_per_block, sh.B * sh.Hq);
  zero_rows<VPR><<<grid, kThreads, 0, st>>>(rank, static_cast<u32x4*>(o), sh.L);
  return hipGetLastError();
}

template <int VPR>
hipError_t gather_vpr(const Shape& sh, const void* q, const void* k, const void* v,
                      const int32_t* idx, const int32_t* budget, void* qc, void* kc, void* vc,
                      hipStream_t st) {
  const int rpb = qc ? kRowsGatherQKV : kRowsGatherKV;
  dim3 grid((sh.L + rpb - 1) / rpb, sh.B * sh.Hkv);
  auto kern = qc ? gather_rows<VPR, true> : gather_rows<VPR, false>;
  kern<<<grid, kThreads, 0, st>>>(
      static_cast<const u32x4*>(q), static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
      idx, budget, static_cast<u32x4*>(qc), static_cast<u32x4*>(kc), static_cast<u32x4*>(vc),
      sh.Hq, sh.Hkv, sh.L, sh.bud_b(), sh.bud_h());
  return hipGetLastError();
}

template <int VPR>
hipError_t gather_by_rank_vpr(const Shape& sh, const void* k, const void* v, const int32_t* rank,
                              void* kc, void* vc, hipStream_t st) {
  dim3 grid((sh.L + kRowsByRank - 1) / kRowsByRank, sh.B * sh.Hkv);
  gather_kv_by_rank<VPR><<<grid, kThreads, 0, st>>>(
      static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), rank, static_cast<u32x4*>(kc),
      static_cast<u32x4*>(vc), sh.Hq, sh.Hkv, sh.L, sh.L);
  return hipGetLastError();
}

template <int VPR>
hipError_t scatter_vpr(const Shape& sh, const void* oc, const int32_t* rank, void* o,
                       hipStream_t st) {
  dim3 grid((sh.L + kRowsScatter - 1) / kRowsScatter, sh.B * sh.Hq);
  scatter_rows<VPR><<<grid, kThreads, 0, st>>>(static_cast<const u32x4*>(oc), rank,
                                                static_cast<u32x4*>(o), sh.L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const Shape& sh, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* budget, void* qc, void* kc, void* vc,
                         hipStream_t st) {
  switch (sh.row_bytes() / 16) {
    case 8: return gather_vpr<8>(sh, q, k, v, idx, budget, qc, kc, vc, st);
    case 16: return gather_vpr<16>(sh, q, k, v, idx, budget, qc, kc, vc, st);
    case 32: return gather_vpr<32>(sh, q, k, v, idx, budget, qc, kc, vc, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_kv_by_rank(const Shape& sh, const void* k, const void* v,
                                    const int32_t* rank, void* kc, void* vc, hipStream_t st) {
  switch (sh.row_bytes() / 16) {
    case 8: return gather_by_rank_vpr<8>(sh, k, v, rank, kc, vc, st);
    case 16: return gather_by_rank_vpr<16>(sh, k, v, rank, kc, vc, st);
    case 32: return gather_by_rank_vpr<32>(sh, k, v, rank, kc, vc, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_zero_unselected(const Shape& sh, const int32_t* rank, void* o, hipStream_t st) {
  switch (sh.row_bytes() / 16) {
    case 8: return zero_vpr<8>(sh, rank, o, st);
    case 16: return zero_vpr<16>(sh, rank, o, st);
    case 32: return zero_vpr<32>(sh, rank, o, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scatter(const Shape& sh, const void* oc, const int32_t* rank, void* o,
                          hipStream_t st) {
  switch (sh.row_bytes() / 16) {
    case 8: return scatter_vpr<8>(sh, oc, rank, o, st);
    case 16: return scatter_vpr<16>(sh, oc, rank, o, st);
    case 32: return scatter_vpr<32>(sh, oc, rank, o, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tsa
