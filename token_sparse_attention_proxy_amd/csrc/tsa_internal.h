// Internal declarations shared by the HIP translation units of libtsa.so.
// Not installed; the public interface is include/tsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa.h"

namespace tsa {

// ---------------------------------------------------------------- constants
constexpr int kScoreFracBits = 50;     // budget masses are counted in units of 2^-50
constexpr int kScoreChunk = 128;       // keys per proxy-scoring workgroup
constexpr int kMaxScoreTiles = 92;    // 32-row proxy tiles per query head (bf16 scoring LDS)
constexpr int kMaxHq = 4096;           // keeps the budget's integer masses below 2^63
constexpr int64_t kMaxL = int64_t(1) << 22;   // per-head tensors stay below 2^31 bytes
constexpr int kMaxHeads = 65535;       // B*Hq: grid y of the per-head launches
constexpr int kForwardFusedMaxL = 32768;   // tsa_forward takes the fused kernels up to this L

// ---------------------------------------------------------------- shapes
struct Shape {
  int B, Hq, Hkv, L, d, w;
  float tau;
  int dtype;          // TSA_F32 / TSA_BF16
  int flags;          // TSA_FLAG_* bits
  int G() const { return Hq / Hkv; }
  bool causal_proxy() const { return !(flags & TSA_FLAG_NONCAUSAL_PROXY); }
  bool per_head() const { return (flags & TSA_FLAG_PER_HEAD_BUDGET) != 0; }
  int keep() const { return (flags & TSA_FLAG_KEEP_WINDOW) ? w : 0; }
  // Budget of head (b, h) is budget[b * bud_b() + h * bud_h()].
  int bud_b() const { return per_head() ? Hq : 1; }
  int bud_h() const { return per_head() ? 1 : 0; }
  int bud_rows() const { return per_head() ? B * Hq : B; }
  int eb() const { return dtype == TSA_BF16 ? 2 : 4; }
  int64_t row_bytes() const { return int64_t(d) * eb(); }
  int n_chunk() const { return (L + kScoreChunk - 1) / kScoreChunk; }
};

constexpr int kBudgetLogBuckets = 4096;   // log-scale buckets of the budget's first pass
constexpr int kSelectBuckets = 2048;      // digit buckets of the selection's histogram passes
constexpr int kSelectTabStride = 1026;    // words per chunk table of the selection's last pass

// Chunking of the selection: each head's candidates in `nch` chunks of
// `chunk` tokens (one workgroup each); the compaction grid covers L in
// `ngrid` chunks.
struct SelectPlan {
  int chunk, nch, ngrid;
};
SelectPlan select_plan(const Shape& s);

// Step-scratch layout (offsets in bytes from the workspace base, 256-aligned).
// R = budget rows (B, or B*Hq with per-head budgets).
struct StepWs {
  size_t part;        // float2 [B*Hq*w*n_chunk]: per-chunk (max, sum) of each proxy row
  size_t rowstat;     // float2 [B*Hq*w]: (max in exp2 units, 1/Z) of each proxy row
  size_t sigma;       // uint64 [R*L]: quantised masses (head-summed if R = B)
  size_t bud_cand;    // uint64 [R*L]: values of each row's crossing bucket
  size_t bud_hcnt;    // uint32 [R*4096]: log-bucket counts   } cleared together:
  size_t bud_hmass;   // uint64 [R*4096]: log-bucket masses   } contiguous, in
  size_t bud_ncand;   // uint32 [2R]: candidates, finished    } this order
                      //   extract workgroups per row        }
  size_t sel_hist;    // uint32 [3*B*Hq*2048]: selection histograms, one per digit level
  size_t sel_state;   // uint32 [3*B*Hq*2]: (prefix, count above) after each level's pick
  size_t sel_tab;     // uint32 [B*Hq*nch*1026]: per chunk, suffix sums of the last digit and
                      //   the count above the 22-bit prefix
  size_t total;
};
StepWs step_ws_layout(const Shape& s);

// Forward-scratch layout: step scratch first, then the intermediates.
struct FwdWs {
  StepWs step;
  size_t scores;      // float [B*Hq*L]
  size_t rank;        // int32 [B*Hq*L]
  size_t fused_total; // end of rank: all the fused forward needs
  size_t kc, vc;      // dtype [B*Hq*L*d] each: compact K and V of every head
  size_t total;
};
FwdWs fwd_ws_layout(const Shape& s);

// Words the budget and the selection need zeroed before they start: the
// whole op has its scoring pass clear them (score_merge), so those steps
// launch no clear kernels of their own.
struct StepClear {
  uint32_t* p0;
  int64_t n0;
  uint32_t* p1;
  int64_t n1;
};
int64_t budget_clear_words(const Shape& s);   // from bud_hcnt on
StepClear step_clear(const Shape& s, char* ws);

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() after enqueueing its kernels on `st`.
hipError_t launch_score(const Shape& s, const void* q, const void* k, float* scores,
                        char* ws, hipStream_t st, const StepClear* clear = nullptr);
// cleared = true: the histograms and counters the step starts from are
// already zero (the whole op clears them in its scoring pass, clear_steps).
hipError_t launch_budget(const Shape& s, const float* scores, int32_t* budget, char* ws,
                         hipStream_t st, bool cleared = false);
// zero_o != nullptr: the compaction also zeroes the rows of zero_o ([B,Hq,L,d])
// of the candidates it leaves out (launch_zero_unselected's work, when no
// kept window is in force: the window's rows are always selected).
hipError_t launch_select(const Shape& s, const float* scores, const int32_t* budget,
                         int32_t* idx, int32_t* rank, char* ws, hipStream_t st,
                         bool cleared = false, void* zero_o = nullptr);
// qc == nullptr: K and V only.
hipError_t launch_gather(const Shape& s, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* budget, void* qc, void* kc,
                         void* vc, hipStream_t st);
// idx == nullptr: q, k, v, o hold rows 0..n-1 of each head (dense or
// compact).  Otherwise they are full-length sequence tensors and compact
// row i of head (b,h) is sequence row idx[b,h,i]; only those rows of o are
// written.
// bmask != nullptr: block-sparse attention on compact tensors (idx must be
// nullptr); see attn_fwd_bf16 for the mask layout.
hipError_t launch_attention(const Shape& s, const void* q, const void* k, const void* v,
                            const int32_t* budget, const int32_t* idx, int kv_group, void* o,
                            hipStream_t st, const uint32_t* bmask = nullptr);
// K and V compact (kc, vc as launch_gather writes them), Q read and O written
// through the index set: only the selected rows of o are written.
hipError_t launch_attention_qo(const Shape& s, const void* q, const void* kc, const void* vc,
                               const int32_t* budget, const int32_t* idx, void* o,
                               hipStream_t st);
// K and V only, source-driven through the rank map: kc/vc[b,h,rank[b,h,j]] = K/V[b,g(h),j]
// for every j with rank >= 0 (the same bytes as launch_gather with qc == nullptr).
hipError_t launch_gather_kv_by_rank(const Shape& s, const void* k, const void* v,
                                    const int32_t* rank, void* kc, void* vc, hipStream_t st);
hipError_t launch_zero_unselected(const Shape& s, const int32_t* rank, void* o, hipStream_t st);
hipError_t launch_scatter(const Shape& s, const void* oc, const int32_t* rank, void* o,
                          hipStream_t st);

}  // namespace tsa
