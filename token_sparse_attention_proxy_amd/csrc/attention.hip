// Causal attention on dense tensors: the attention over the compressed
// Q, K, V of Token Sparse Attention (gist.science summary, section 2, "Core
// architecture": the compressed tensors stay dense and contiguous, so an
// ordinary dense attention kernel runs on them), and, with the GQA head map,
// the dense baseline over the full sequence.
//
//   o[i] = sum_{j<=i} softmax_j(<q_i, k_j>/sqrt(d)) v_j,   i < n
//
// bf16 path (gfx950 MFMA, wave64):
//   * a workgroup owns 256 query rows of one head (8 waves x 32 rows, two
//     waves per SIMD) and walks 64-key tiles of K and V through four LDS
//     buffers: two tiles are computed per barrier while the next two are
//     staged;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the A operand is 32 keys
//     read from LDS, the B operand is the wave's 32 query rows kept in
//     registers, so every lane owns one query row;
//   * keys are read into the MFMA rows in a fixed permutation (bits 2 and 3
//     of the row index swapped) so that the S^T accumulator, converted to
//     bf16, is directly the B operand of O^T = V^T P^T;
//   * V is transposed in registers while staged, so LDS holds V^T and the
//     A operand of the PV product is one 16-byte LDS read per lane;
//   * Q is scaled by c = log2(e)/sqrt(d) once, when the wave loads it, and
//     rounded to bf16, so S^T comes out of the MFMA in log2 units;
//   * softmax with a fixed per-row reference: p = exp2(S - m) where m is the
//     row max over the first key tile.  Every later S^T chain starts from
//     an accumulator holding -m, so the subtraction costs nothing, and the
//     loop needs no running max, no cross-lane reduction and no rescaling
//     of O, which stays in accumulator registers touched only by MFMA: one
//     exp2, half a bf16 pack and one fp32 add (the row sum) per score.
//     (Row sums as bf16 dot2 against (1, 1) would take half the
//     instructions, but v_dot2 does not overlap MFMA issue on gfx950 the
//     way plain fp32 VALU does.)
//     Softmax is invariant to the reference, so the result equals the usual
//     one up to rounding.
//     A row sum above 2^64 (a later logit far above the first tile's max)
//     makes the workgroup recompute with the exact row max as reference, so
//     nothing can overflow;
//   * P rounded to bf16 for the PV product, fp32 row sums of the unrounded
//     P, fp32 output accumulators, final division and round-to-nearest-even
//     to bf16;
//   * loads and stores go through buffer resources sized to the n valid
//     rows: out-of-range rows read as 0 and are never written, without
//     branches;
//   * only each wave's diagonal tile is masked; tiles above it are skipped;
//   * query blocks are issued heaviest first (the causal triangle), across
//     groups of 8 KV heads, each KV head's query heads on one XCD;
//   * block-sparse composition (BS): a caller's bit mask over (64-row query
//     block, 64-key block) pairs of the compressed sequence says which key
//     tiles each query block sees (its diagonal block always).  A workgroup
//     stages only the tiles some of its four query blocks see, and each wave
//     computes only the tiles its own query block sees.
// f32 path: a plain fp32 VALU kernel (one query row per thread).
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {
namespace {

// ---------------------------------------------------------------- bf16 MFMA
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup: 32 per wave
constexpr int kBN = 64;           // keys per tile
constexpr int kKPad = 8;          // bf16 elements of padding per K row in LDS
constexpr int kVPad = 8;          // bf16 elements of padding per V^T row in LDS
constexpr int kXcds = 8;          // workgroups go round-robin to the 8 XCDs in dispatch order
// A row sum above 2^64 means some exponent relative to the reference max
// may have overflowed or lost range: the workgroup then recomputes with the
// exact row max as reference.
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64

// MFMA row i of a 32-key subtile holds key perm32(i): bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int i) {
  return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Buffer resource over `bytes` bytes from `p`: loads past the end return 0,
// stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, int(bytes), 0x00020000);
}

// max / sum of x[l] and x[l ^ 32] in every lane l.
__device__ __forceinline__ float max_halves(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D, int NBUF>
struct AttnSmem {
  uint16_t k[NBUF][kBN][D + kKPad];
  uint16_t vt[NBUF][D][kBN + kVPad];
};

// Key index held in element e of the S^T accumulator of a 32-key subtile, for a lane in `half`.
__device__ __forceinline__ int acc_key(int e, int half) {
  return 16 * (e >> 3) + 8 * half + 4 * ((e >> 2) & 1) + (e & 3);
}

// IDX = false: q, k, v, o are dense per-head tensors and row i is row i.
// IDX = true: compact row i of head (b,h) is sequence row idx[b,h,i]; Q, K, V
// are read and O is written through the index set (compression, attention
// and decompression of the selected rows in one pass).
// BS = true: bmask is the block mask, [B*Hq][NB][NW] uint32 with NB = ceil(L/64)
// and NW = ceil(NB/32); bit kb % 32 of word [qb][kb / 32] set = query block qb
// sees key block kb.
// QO = true (with IDX = false): K and V are the compact per-head tensors, and
// only Q is read and O written through the index set, so the key walk is the
// compact one and neither a compact Q nor a compact O is needed.
template <int D, bool IDX, bool BS, bool QO>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ budget,
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ bmask,
    uint16_t* __restrict__ o, int Hq, int Hk, int kv_group, int L, int bud_b, int bud_h,
    float c) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KCH = kBN * D / 8 / kThreads;          // 16-byte K chunks per thread
  constexpr int VPAIRS = (kBN / 4) * (D / 8);          // (4-key group, 8-d chunk) pairs
  constexpr int DT = D / 32;                           // 32-wide d tiles of O^T
  constexpr int KS = D / 16;                           // k-steps of S^T
  constexpr int NSUB = kBN / 32;                       // 32-key subtiles
  static_assert(KCH >= 1 && VPAIRS <= kThreads, "tile shape");
  // Four tile buffers: the main walks compute two tiles per barrier while
  // the next two are staged; the exact-max rescans use two of them.
  __shared__ AttnSmem<D, 4> sm;
  __shared__ int idx_s[IDX ? 4 : 1][kBN];     // sequence rows of upcoming key tiles (slot = tile % 4)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, half = lane >> 5;
  // Dispatch order: heads in groups of 8 KV heads (8 * kv_group query
  // heads); within a group, the heaviest query blocks of all its heads
  // first, so each group ends on light blocks and no long block starts near
  // the end.  Workgroups go to the XCDs round-robin, so linear position
  // mod 8 picks the XCD: every query head of one KV head lands on the same
  // XCD and its L2 serves that head's K and V alone.
  const int nqb = (L + kBM - 1) / kBM;
  const int lin = int(blockIdx.x) + int(blockIdx.y) * nqb;
  const int G8 = kXcds * kv_group;
  const int grp = lin / (G8 * nqb);
  const int hg = min(G8, int(gridDim.y) - grp * G8);
  const int rem = lin - grp * G8 * nqb;
  const int bh = grp * G8 + (hg == G8 ? (rem % kXcds) * kv_group + (rem / kXcds) % kv_group : rem % hg);
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / kv_group;
  const int n = budget ? min(max(budget[b * bud_b + h * bud_h], 0), L) : L;
  const int q0 = (nqb - 1 - rem / hg) * kBM;
  if (q0 >= n) return;

  // Rows past the valid range read as 0 and are never written.  Indexed
  // reads address the full sequence; compact rows >= n map to row L.
  constexpr bool QIDX = IDX || QO;           // Q and O through the index set
  const uint32_t qo_bytes = uint32_t(QIDX ? L : n) * D * 2;
  const uint32_t kv_bytes = uint32_t(IDX ? L : n) * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + int64_t(bh) * L * D, qo_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + (int64_t(b) * Hk + hk) * L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + (int64_t(b) * Hk + hk) * L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + int64_t(bh) * L * D, qo_bytes);
  const int wr0 = q0 + 32 * wave;            // first query row of this wave
  const int qrow = wr0 + l32;                // the row this lane owns
  const int wdiag = wr0 / kBN;               // tile holding this wave's diagonal

  const int32_t* __restrict__ idx_h = QIDX ? idx + int64_t(bh) * L : nullptr;
  const int qsrc = QIDX ? (qrow < n ? idx_h[qrow] : L) : qrow;   // sequence row of this lane's query

  // Q^T as the B operand: lane holds q[qrow][16t + 8*half .. +8].
  bf16x8 qf[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t)
    qf[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                           rq, (qsrc * D + 16 * t + 8 * half) * 2, 0, 0));

  // Q^T pre-scaled by c = log2(e)/sqrt(d) and rounded to bf16, so the S^T
  // accumulators are logits in log2 units.
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    u32x4 w = __builtin_bit_cast(u32x4, qf[t]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pack_bf16x2(__uint_as_float(w[e] << 16) * c, __uint_as_float(w[e] & 0xffff0000u) * c);
    qf[t] = __builtin_bit_cast(bf16x8, w);
  }
  const int kv_end = min(q0 + kBM, n);
  const int ntiles = (kv_end + kBN - 1) / kBN;

  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int vkg = tid % (kBN / 4), vdc = tid / (kBN / 4);   // (key group, d chunk) of this thread

  // Indexed staging.  The sequence rows of key tile t are fetched from HBM
  // (one per thread of wave 0) well before they are needed, published to
  // LDS slot t % 4 before a barrier, and read into this thread's row
  // registers before the K/V loads of tile t are issued (the paired main
  // walk: see there; the per-tile rescan: fetched at the top of iteration
  // t-4, published at t-3, read in t-2, loaded at the top of t-1).  The K/V
  // loads then wait on nothing, and no index work sits before a barrier.
  int krs[KCH], vrs[4];      // sequence rows of the K and V rows this thread stages next
  auto fetch_idx = [&](int tile) {
    const int key = tile * kBN + tid;
    return (IDX && tid < kBN && key < n) ? idx_h[key] : L;
  };
  auto put_idx = [&](int tile, int val) {
    if (IDX && tid < kBN) idx_s[tile & 3][tid] = val;
  };
  auto read_rows = [&](int tile) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int row = (tid + kThreads * i) / (D / 8);
      krs[i] = IDX ? idx_s[tile & 3][row] : tile * kBN + row;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) vrs[r] = IDX ? idx_s[tile & 3][4 * vkg + r] : tile * kBN + 4 * vkg + r;
  };
  auto load_tile = [&](int tile) {
    if (!IDX) read_rows(tile);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int col = (tid + kThreads * i) % (D / 8);
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (krs[i] * D + col * 8) * 2, 0, 0);
    }
    if (tid < VPAIRS) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = __builtin_amdgcn_raw_buffer_load_b128(rv, (vrs[r] * D + vdc * 8) * 2, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / (D / 8), col = ch % (D / 8);
      *reinterpret_cast<u32x4*>(&sm.k[buf][row][col * 8]) = kreg[i];
    }
    if (tid < VPAIRS) {
      // 4 keys x 8 d  ->  8 rows of V^T, 4 keys each
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a0 = vreg[0][p], a1 = vreg[1][p], a2 = vreg[2][p], a3 = vreg[3][p];
        u32x2 lo, hi;
        lo.x = (a0 & 0xffffu) | (a1 << 16);
        lo.y = (a2 & 0xffffu) | (a3 << 16);
        hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
        hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&sm.vt[buf][8 * vdc + 2 * p][4 * vkg]) = lo;
        *reinterpret_cast<u32x2*>(&sm.vt[buf][8 * vdc + 2 * p + 1][4 * vkg]) = hi;
      }
    }
  };
  int held = L;               // index entry fetched for the ring, published next iteration
  auto begin_walk = [&]() {
    if (IDX) {
      const int i0 = fetch_idx(0), i1 = fetch_idx(1), i2 = fetch_idx(2);
      held = fetch_idx(3);
      put_idx(0, i0);
      put_idx(1, i1);
      __syncthreads();
      read_rows(0);
      load_tile(0);
      read_rows(1);
      __syncthreads();                 // slot 0 is free again
      put_idx(2, i2);
    } else {
      load_tile(0);
    }
    store_tile(0);
    __syncthreads();
  };


  const int krow = perm32(l32);
  const f32x16 zero = {};

  // S^T = K Q^T for the tile in `buf`: two independent accumulator chains.
  auto qk = [&](int buf, f32x16 (&sacc)[NSUB], const f32x16& init) {
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[buf][32 * sb + krow][16 * t + 8 * half]);
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], t == 0 ? init : sacc[sb], 0, 0, 0);
      }
  };
  auto mask = [&](int key0, f32x16 (&sacc)[NSUB]) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key0 + 32 * sb + acc_key(e, half) > qrow) sacc[sb][e] = -INFINITY;
  };
  auto tile_max = [&](const f32x16 (&sacc)[NSUB]) {
    float m = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, sacc[sb][e]);
    return max_halves(m);
  };

  f32x16 oacc[DT];
  float m_ref = 0.f;      // exp2 reference of this lane's row
  f32x16 bias = zero;     // -m_ref in every element: the S^T chains start from it
  auto set_ref = [&](float m) {
    m_ref = m;
#pragma unroll
    for (int e = 0; e < 16; ++e) bias[e] = -m;
  };
  // This lane's share of the row sum, as four independent partial sums kept
  // across the whole key walk (pair p of a subtile adds into lsum[p % 4]).
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
  auto clear_sum = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum[i] = 0.f;
  };
  auto row_sum = [&]() { return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]); };

  // P = exp2(S - m_ref) (biased: S^T already holds -m_ref from its chain start),
  // rounded to bf16; fp32 row sums of P (four partial sums), then O^T += V^T P^T.
  auto pv = [&](int buf, const f32x16 (&sacc)[NSUB], bool biased) {
    const float mneg = biased ? 0.f : -m_ref;
    bf16x8 pb[NSUB * 2];
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[sb][8 * tt + 2 * e2] + mneg);
          const float p1 = __builtin_amdgcn_exp2f(sacc[sb][8 * tt + 2 * e2 + 1] + mneg);
          pk[e2] = pack_bf16x2(p0, p1);
          lsum[e2] += p0 + p1;
        }
        pb[2 * sb + tt] = __builtin_bit_cast(bf16x8, pk);
      }
#pragma unroll
    for (int kk = 0; kk < NSUB * 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][32 * dt + l32][16 * kk + 8 * half]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], oacc[dt], 0, 0, 0);
      }
  };

  // The same tile as qk + pv (same operations in the same accumulation
  // orders, so the same bits) for tiles below the diagonal, written as one
  // software pipeline in program order: LDS operand reads run PF ahead of
  // their MFMA, the S^T chain of subtile q+1 carries the exp/convert/row-sum
  // work of subtile q, and the PV MFMAs of the first subtiles carry that of
  // the last.
  auto hot = [&](int buf) {
    constexpr int NQK = NSUB * KS;            // S^T MFMAs, chain after chain
    constexpr int NPV = 2 * NSUB * DT;        // O^T MFMAs, kk-major
    constexpr int NR = NQK + NPV;             // operand reads, in MFMA order
    constexpr int PF = 3;
    constexpr int LAST = NSUB - 1;
    constexpr int LAST_SLOT = 2 * LAST * DT;  // PV MFMAs that can carry the last subtile's softmax
    constexpr int LPP = (8 + LAST_SLOT - 1) / LAST_SLOT;   // its pairs per carrying MFMA
    static_assert(LAST >= 1 && 8 % KS == 0, "pipeline shape");
    const uint16_t* kbase = &sm.k[buf][krow][8 * half];
    const uint16_t* vbase = &sm.vt[buf][l32][8 * half];
    auto rd = [&](int r) {
      if (r < NQK)
        return *reinterpret_cast<const bf16x8*>(kbase + 32 * (r / KS) * (D + kKPad) + 16 * (r % KS));
      const int j = r - NQK;
      return *reinterpret_cast<const bf16x8*>(vbase + 32 * (j % DT) * (kBN + kVPad) + 16 * (j / DT));
    };
    f32x16 sacc[NSUB];
    u32x4 pk[2 * NSUB];
    auto softmax_pair = [&](int sb, int p) {  // elements 2p, 2p+1 of subtile sb
      const float p0 = __builtin_amdgcn_exp2f(sacc[sb][2 * p]);
      const float p1 = __builtin_amdgcn_exp2f(sacc[sb][2 * p + 1]);
      pk[2 * sb + p / 4][p % 4] = pack_bf16x2(p0, p1);
      lsum[p % 4] += p0 + p1;
    };
    bf16x8 ring[PF + 1];
#pragma unroll
    for (int r = 0; r < PF; ++r) ring[r] = rd(r);
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      if (m + PF < NR) ring[(m + PF) % (PF + 1)] = rd(m + PF);
      const bf16x8 a = ring[m % (PF + 1)];
      if (m < NQK) {
        const int sb = m / KS, t = m % KS;
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], t == 0 ? bias : sacc[sb], 0, 0, 0);
        if (sb >= 1) {                        // softmax of subtile sb-1, 8/KS pairs per MFMA
#pragma unroll
          for (int p = t * (8 / KS); p < (t + 1) * (8 / KS); ++p) softmax_pair(sb - 1, p);
        }
      } else {
        const int j = m - NQK, kk = j / DT, dt = j % DT;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pk[kk]),
                                                           oacc[dt], 0, 0, 0);
        if (j < LAST_SLOT) {
#pragma unroll
          for (int p = j * LPP; p < (j + 1) * LPP && p < 8; ++p) softmax_pair(LAST, p);
        }
      }
    }
    // Pin the operand reads PF MFMAs ahead, whatever the surrounding code,
    // and spread the tile's 32 exps evenly from a quarter chain after the
    // first S^T chain ends (its accumulator is then ready), so the row-sum
    // and pack work fills the gaps between them.  The indexed walk runs
    // fastest with them one MFMA later (measured: about 1%).
    constexpr int EXP_PER = 16 / KS;          // exps per MFMA, the rate of the chain that carries them
    constexpr int EXP_FIRST = KS + KS / 4 + (IDX ? 1 : 0);
    constexpr int EXP_SLOTS = 32 / EXP_PER;
    static_assert(EXP_FIRST + EXP_SLOTS <= NR, "exp slots");
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + PF < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i >= EXP_FIRST && i < EXP_FIRST + EXP_SLOTS) __builtin_amdgcn_sched_group_barrier(0x400, EXP_PER, 0);
    }
  };

  // Block mask of this head (BS only).  The workgroup's query blocks are
  // qb0 .. qb0 + QB - 1; each wave's query block is its diagonal tile.  The
  // walk keeps a cursor on one 32-tile word of the mask: the four rows' words
  // of the current word are in registers and those of the next word are
  // prefetched.  When the cursor steps onto a word, the tiles of that word
  // the workgroup needs and those this wave uses are folded into two
  // wave-uniform bit sets, so finding the next tile and whether a wave uses
  // it is a few scalar operations; only a run of empty words costs a wait.  Mask words
  // are read with buffer (vector-memory) loads, which never share a wait
  // counter with the LDS operand reads of the MFMA loop.
  constexpr int QB = kBM / kBN;
  const int NB = (L + kBN - 1) / kBN, NW = (NB + 31) >> 5;
  const __amdgpu_buffer_rsrc_t rmask =
      make_rsrc(BS ? bmask + int64_t(bh) * NB * NW : bmask, BS ? uint32_t(NB * NW) * 4 : 0u);
  const int qb0 = q0 / kBN;
  const int wsel = wdiag - qb0;          // this wave's row among the QB (0 .. QB-1)
  int wd_cur = 0;                        // word under the cursor
  uint32_t rw_cur[QB], rw_nxt[QB];       // row words of word wd_cur and wd_cur + 1
  uint32_t u_cur = 0, w_cur = 0;         // of word wd_cur: tiles needed, tiles this wave's row sees
  auto load_word = [&](int wd, uint32_t (&rw)[QB]) {   // rows past NB read as 0 (outside the buffer)
    const bool in = wd < NW;
#pragma unroll
    for (int i = 0; i < QB; ++i)
      rw[i] = uint32_t(__builtin_amdgcn_raw_buffer_load_b32(rmask, ((qb0 + i) * NW + (in ? wd : 0)) * 4, 0, 0));
    if (!in) {
#pragma unroll
      for (int i = 0; i < QB; ++i) rw[i] = 0u;
    }
  };
  // Tiles of word wd the workgroup needs: mask bits of its rows below qb0,
  // every tile in [qb0, ntiles) (diagonal blocks), nothing at or past ntiles.
  auto needed_bits = [&](int wd, const uint32_t (&rw)[QB]) {
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < QB; ++i) u |= rw[i];
    const int lo = wd << 5;
    const int a = min(max(qb0 - lo, 0), 32), e = min(max(ntiles - lo, 0), 32);
    const uint32_t below_e = e >= 32 ? ~0u : ((1u << e) - 1u);
    const uint32_t from_a = a >= 32 ? 0u : (~0u << a);
    u = (u & ~from_a) | from_a;          // tiles >= qb0 are always needed
    return __builtin_amdgcn_readfirstlane(u & below_e);
  };
  auto set_word = [&]() {                // fold the cursor's row words into u_cur, w_cur
    u_cur = needed_bits(wd_cur, rw_cur);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < QB; ++i) w = (i == wsel) ? rw_cur[i] : w;
    w_cur = __builtin_amdgcn_readfirstlane(w);
  };
  auto next_from = [&](int p) {          // first needed tile >= p; moves the cursor to it
    if ((p >> 5) == wd_cur) {
      const uint32_t u = u_cur & (~0u << (p & 31));
      if (u) return (wd_cur << 5) + __builtin_ctz(u);
      p = (wd_cur + 1) << 5;
    }
    if ((p >> 5) == wd_cur + 1 && p < ntiles) {   // step onto the prefetched word
      ++wd_cur;
#pragma unroll
      for (int i = 0; i < QB; ++i) rw_cur[i] = rw_nxt[i];
      load_word(wd_cur + 1, rw_nxt);
      set_word();
      const uint32_t u = u_cur & (~0u << (p & 31));
      if (u) return (wd_cur << 5) + __builtin_ctz(u);
      p = (wd_cur + 1) << 5;
    }
    while (p < ntiles) {                 // a run of empty words: load as we go
      wd_cur = p >> 5;
      load_word(wd_cur, rw_cur);
      load_word(wd_cur + 1, rw_nxt);
      set_word();
      const uint32_t u = u_cur & (~0u << (p & 31));
      if (u) return (wd_cur << 5) + __builtin_ctz(u);
      p = (wd_cur + 1) << 5;
    }
    return ntiles;
  };
  auto wave_uses = [&](int t) {          // needs the cursor on t's word
    if (t > wdiag) return false;
    if (t == wdiag || !BS) return true;
    if (wdiag >= NB) return false;       // a wave past the last row
    return ((w_cur >> (t & 31)) & 1u) != 0;
  };
  auto begin_bs = [&]() {                // cursor on word 0; returns the first tile
    wd_cur = 0;
    load_word(0, rw_cur);
    load_word(1, rw_nxt);
    set_word();
    return next_from(0);
  };

  // attempt 0: reference = max of the first key tile; attempt 1 (rare): exact row max.
  for (int attempt = 0; attempt < 2; ++attempt) {
    if constexpr (BS) {
      // Walk only the tiles the workgroup needs, in order.  The next tiles,
      // and whether this wave uses them, are looked up ahead, so no mask
      // read sits in front of a tile's work.  (The exact-max rescan walks
      // one tile per barrier through two buffers.)
      if (attempt == 1) {
        float m = -INFINITY;
        int cur = begin_bs(), buf = 0;
        bool use_cur = wave_uses(cur);
        int nxt = next_from(cur + 1);
        bool use_nxt = nxt < ntiles && wave_uses(nxt);
        load_tile(cur);
        store_tile(0);
        __syncthreads();
        while (true) {
          const int nxt2 = nxt < ntiles ? next_from(nxt + 1) : ntiles;   // before the K/V loads
          const bool use_nxt2 = nxt2 < ntiles && wave_uses(nxt2);
          if (nxt < ntiles) load_tile(nxt);
          if (use_cur) {
            f32x16 sacc[NSUB];
            qk(buf, sacc, zero);
            if (cur == wdiag) mask(cur * kBN, sacc);
            m = fmaxf(m, tile_max(sacc));
          }
          if (nxt < ntiles) store_tile(buf ^ 1);
          __syncthreads();
          if (nxt >= ntiles) break;
          cur = nxt;
          nxt = nxt2;
          use_cur = use_nxt;
          use_nxt = use_nxt2;
          buf ^= 1;
        }
        set_ref(m);
      }
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i] = zero;
      clear_sum();
      bool have_ref = attempt == 1;      // the first tile a wave uses sets its reference
      auto bs_compute = [&](int tile, bool use, int buf) {
        if (!use) return;
        if (tile < wdiag && have_ref) {
          hot(buf);
        } else {
          f32x16 sacc[NSUB];
          qk(buf, sacc, have_ref ? bias : zero);
          if (tile == wdiag) mask(tile * kBN, sacc);
          if (!have_ref) set_ref(tile_max(sacc));
          pv(buf, sacc, have_ref);
        }
        have_ref = true;
      };
      // The needed tiles c0 < c1 < c2 < c3 (ntiles when exhausted), with
      // whether this wave uses each: c0 and c1 sit in buffers s and s+1 and
      // are computed while c2 and c3 are staged into s+2 and s+3; one
      // barrier per pair.
      int c0 = begin_bs();
      bool u0 = wave_uses(c0);
      int c1 = c0 < ntiles ? next_from(c0 + 1) : ntiles;
      bool u1 = c1 < ntiles && wave_uses(c1);
      int c2 = c1 < ntiles ? next_from(c1 + 1) : ntiles;
      bool u2 = c2 < ntiles && wave_uses(c2);
      int c3 = c2 < ntiles ? next_from(c2 + 1) : ntiles;
      bool u3 = c3 < ntiles && wave_uses(c3);
      load_tile(c0);
      store_tile(0);
      if (c1 < ntiles) {
        load_tile(c1);
        store_tile(1);
      }
      __syncthreads();
      int sb0 = 0;
      while (true) {
        if (c2 < ntiles) load_tile(c2);
        bs_compute(c0, u0, sb0);
        if (c2 < ntiles) store_tile((sb0 + 2) & 3);
        if (c3 < ntiles) load_tile(c3);
        if (c1 < ntiles) bs_compute(c1, u1, (sb0 + 1) & 3);
        // The walk's look-ahead runs while this pair's last MFMAs drain, not
        // in front of the next pair's work.
        const int c4 = c3 < ntiles ? next_from(c3 + 1) : ntiles;
        const bool u4 = c4 < ntiles && wave_uses(c4);
        const int c5 = c4 < ntiles ? next_from(c4 + 1) : ntiles;
        const bool u5 = c5 < ntiles && wave_uses(c5);
        if (c3 < ntiles) store_tile((sb0 + 3) & 3);
        __syncthreads();
        if (c2 >= ntiles) break;
        c0 = c2;
        u0 = u2;
        c1 = c3;
        u1 = u3;
        c2 = c4;
        u2 = u4;
        c3 = c5;
        u3 = u5;
        sb0 = (sb0 + 2) & 3;
      }
      const bool bad = !(sum_halves(row_sum()) <= kSumLimit);
      if (!__syncthreads_or(bad)) break;
      continue;
    }
    if (attempt == 1) {
      float m = -INFINITY;
      begin_walk();
      for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile & 1;
        put_idx(tile + 3, held);
        held = fetch_idx(tile + 4);               // before the K/V loads: never waits on them
        if (tile + 1 < ntiles) load_tile(tile + 1);
        if (IDX) read_rows(tile + 2);
        if (tile <= wdiag) {
          f32x16 sacc[NSUB];
          qk(buf, sacc, zero);
          if (tile == wdiag) mask(tile * kBN, sacc);
          m = fmaxf(m, tile_max(sacc));
        }
        if (tile + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
      }
      set_ref(m);
    }
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = zero;
    clear_sum();
    auto compute = [&](int tile, int buf) {
      if (tile < wdiag && tile > 0) {
        hot(buf);                       // no mask, no reductions
      } else if (tile <= wdiag) {
        const bool ref_tile = tile == 0 && attempt == 0;
        f32x16 sacc[NSUB];
        qk(buf, sacc, ref_tile ? zero : bias);
        if (tile == wdiag) mask(tile * kBN, sacc);
        if (ref_tile) set_ref(tile_max(sacc));
        pv(buf, sacc, !ref_tile);
      }
    };
    // Tiles t and t+1 sit in buffers t%4 and (t+1)%4; tiles t+2 and t+3
    // are staged into the other two while they are computed, and one
    // barrier per pair publishes them and frees t and t+1.
    // Indexed: the sequence rows of tile u are fetched from HBM (wave 0)
    // in the pair two before the one that loads u, published to LDS slot
    // u % 4 in the pair before it, and read into the row registers half a
    // pair before the load.
    int held0 = L, held1 = L;
    if constexpr (IDX) {
      const int i0 = fetch_idx(0), i1 = fetch_idx(1), i2 = fetch_idx(2), i3 = fetch_idx(3);
      const int i4 = fetch_idx(4);
      held0 = fetch_idx(5);
      held1 = fetch_idx(6);
      put_idx(0, i0);
      put_idx(1, i1);
      put_idx(2, i2);
      put_idx(3, i3);
      __syncthreads();
      read_rows(0);
      load_tile(0);
      store_tile(0);
      if (1 < ntiles) {
        read_rows(1);
        load_tile(1);
        store_tile(1);
      }
      read_rows(2);
      __syncthreads();                 // slot 0 is free again
      put_idx(4, i4);
    } else {
      load_tile(0);
      store_tile(0);
      if (1 < ntiles) {
        load_tile(1);
        store_tile(1);
      }
    }
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
      put_idx(t + 5, held0);
      put_idx(t + 6, held1);
      held0 = fetch_idx(t + 7);        // before the K/V loads: never waits on them
      held1 = fetch_idx(t + 8);
      if (t + 2 < ntiles) load_tile(t + 2);
      if (IDX) read_rows(t + 3);
      compute(t, t & 3);
      if (t + 2 < ntiles) store_tile((t + 2) & 3);
      if (t + 1 < ntiles) {
        if (t + 3 < ntiles) load_tile(t + 3);
        if (IDX) read_rows(t + 4);
        compute(t + 1, (t + 1) & 3);
        if (t + 3 < ntiles) store_tile((t + 3) & 3);
      }
      __syncthreads();
    }
    const bool bad = !(sum_halves(row_sum()) <= kSumLimit);
    if (!__syncthreads_or(bad)) break;
  }

  // epilogue: O = O^T / l; lane holds d = 32dt + 8g + 4*half + {0..3} of its row.
  const float inv = 1.0f / sum_halves(row_sum());
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk;
      pk.x = pack_bf16x2(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
      pk.y = pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(pk, ro, (qsrc * D + 32 * dt + 8 * g + 4 * half) * 2, 0, 0);
    }
}

// ---------------------------------------------------------------- f32 VALU
constexpr int kF32Rows = 64;    // query rows per workgroup (one per thread)
constexpr int kF32Keys = 32;    // keys per LDS tile

template <int D, bool IDX, bool BS, bool QO>
__global__ __launch_bounds__(kF32Rows) void attn_fwd_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ budget, const int32_t* __restrict__ idx,
    const uint32_t* __restrict__ bmask, float* __restrict__ o, int Hq, int Hk, int kv_group,
    int L, int bud_b, int bud_h, float c) {
  static_assert(kF32Rows == 64 && 64 % kF32Keys == 0, "block mask granularity");
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  __shared__ int rows_s[kF32Keys];
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / kv_group;
  const int n = budget ? min(max(budget[b * bud_b + h * bud_h], 0), L) : L;
  const int nqb = (L + kF32Rows - 1) / kF32Rows;
  const int q0 = (nqb - 1 - int(blockIdx.x)) * kF32Rows;
  if (q0 >= n) return;
  const int i = q0 + threadIdx.x;
  const int64_t qbase = int64_t(bh) * L * D;
  const int64_t kvbase = (int64_t(b) * Hk + hk) * L * D;
  const int32_t* __restrict__ idx_h = (IDX || QO) ? idx + int64_t(bh) * L : nullptr;
  // sequence row of this query; -1 past the budget (or for an index outside [0, L))
  int qsrc = i < n ? ((IDX || QO) ? idx_h[i] : i) : -1;
  if (qsrc >= L) qsrc = -1;
  float qr[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = qsrc >= 0 ? q[qbase + int64_t(qsrc) * D + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = min(q0 + kF32Rows, n);
  const int NB = (L + 63) / 64, NW = (NB + 31) >> 5, qb = q0 / 64;
  const uint32_t* __restrict__ bm_row = BS ? bmask + (int64_t(bh) * NB + qb) * NW : nullptr;
  for (int key0 = 0; key0 < kv_end; key0 += kF32Keys) {
    const int kb = key0 / 64;
    if (BS && kb != qb && !((bm_row[kb >> 5] >> (kb & 31)) & 1u)) continue;   // block-uniform
    __syncthreads();
    if (threadIdx.x < kF32Keys) {
      const int key = key0 + threadIdx.x;
      const int src = key < n ? (IDX ? idx_h[key] : key) : -1;
      rows_s[threadIdx.x] = src < L ? src : -1;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Keys * D; e += kF32Rows) {
      const int r = e / D, col = e % D;
      const int src = rows_s[r];
      ks[r][col] = src >= 0 ? k[kvbase + int64_t(src) * D + col] : 0.f;
      vs[r][col] = src >= 0 ? v[kvbase + int64_t(src) * D + col] : 0.f;
    }
    __syncthreads();
    float x[kF32Keys];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qr[e], ks[r][e], dot);
      x[r] = (key0 + r <= i) ? dot * c : -INFINITY;
      mt = fmaxf(mt, x[r]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      const float p = exp2f(x[r] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vs[r][e], acc[e]);
    }
    m = m_new;
  }
  if (qsrc >= 0) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) o[qbase + int64_t(qsrc) * D + e] = acc[e] * inv;
  }
}

template <int D, bool IDX, bool BS, bool QO>
hipError_t run_bf16(const Shape& sh, const void* q, const void* k, const void* v,
                    const int32_t* budget, const int32_t* idx, const uint32_t* bmask,
                    int kv_group, void* o, hipStream_t st) {
  const float c = kLog2e / sqrtf(float(D));
  dim3 grid((sh.L + kBM - 1) / kBM, sh.B * sh.Hq);
  attn_fwd_bf16<D, IDX, BS, QO><<<grid, kThreads, 0, st>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), budget, idx, bmask, static_cast<uint16_t*>(o), sh.Hq,
      sh.Hq / kv_group, kv_group, sh.L, sh.bud_b(), sh.bud_h(), c);
  return hipGetLastError();
}

template <int D, bool IDX, bool BS, bool QO>
hipError_t run_f32(const Shape& sh, const void* q, const void* k, const void* v,
                   const int32_t* budget, const int32_t* idx, const uint32_t* bmask, int kv_group,
                   void* o, hipStream_t st) {
  const float c = kLog2e / sqrtf(float(D));
  dim3 grid((sh.L + kF32Rows - 1) / kF32Rows, sh.B * sh.Hq);
  attn_fwd_f32<D, IDX, BS, QO><<<grid, kF32Rows, 0, st>>>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      budget, idx, bmask, static_cast<float*>(o), sh.Hq, sh.Hq / kv_group, kv_group, sh.L,
      sh.bud_b(), sh.bud_h(), c);
  return hipGetLastError();
}

template <bool IDX, bool BS, bool QO = false>
hipError_t run(const Shape& sh, const void* q, const void* k, const void* v,
               const int32_t* budget, const int32_t* idx, const uint32_t* bmask, int kv_group,
               void* o, hipStream_t st) {
  if (sh.dtype == TSA_BF16)
    return sh.d == 128 ? run_bf16<128, IDX, BS, QO>(sh, q, k, v, budget, idx, bmask, kv_group, o, st)
                       : run_bf16<64, IDX, BS, QO>(sh, q, k, v, budget, idx, bmask, kv_group, o, st);
  return sh.d == 128 ? run_f32<128, IDX, BS, QO>(sh, q, k, v, budget, idx, bmask, kv_group, o, st)
                     : run_f32<64, IDX, BS, QO>(sh, q, k, v, budget, idx, bmask, kv_group, o, st);
}

}  // namespace

hipError_t launch_attention(const Shape& sh, const void* q, const void* k, const void* v,
                            const int32_t* budget, const int32_t* idx, int kv_group, void* o,
                            hipStream_t st, const uint32_t* bmask) {
  if (bmask) {
    if (idx) return hipErrorInvalidValue;     // block-sparse runs on the compact tensors
    return run<false, true>(sh, q, k, v, budget, nullptr, bmask, kv_group, o, st);
  }
  return idx ? run<true, false>(sh, q, k, v, budget, idx, nullptr, kv_group, o, st)
             : run<false, false>(sh, q, k, v, budget, nullptr, nullptr, kv_group, o, st);
}

hipError_t launch_attention_qo(const Shape& sh, const void* q, const void* kc, const void* vc,
                               const int32_t* budget, const int32_t* idx, void* o,
                               hipStream_t st) {
  return run<false, false, true>(sh, q, kc, vc, budget, idx, nullptr, 1, o, st);
}

}  // namespace tsa
