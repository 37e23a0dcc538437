// C ABI of libtsa.so: validation, workspace carving and launch sequencing.
// Kernels live in the other translation units; see tsa_internal.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "tsa_internal.h"

namespace {

thread_local std::string g_last_error;

tsa_status fail(tsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tsa_status fail(tsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tsa_status ok() {
  g_last_error.clear();
  return TSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Shape checks shared by every entry point.
tsa_status check_problem(const tsa_problem* p, tsa::Shape* out) {
  if (!p) return fail(TSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->L < 1 || p->d < 1 || p->w < 1)
    return fail(TSA_ERR_INVALID_ARG, "dimensions must be >= 1 (B=%d Hq=%d Hkv=%d L=%d d=%d w=%d)",
                p->B, p->Hq, p->Hkv, p->L, p->d, p->w);
  if (p->Hq % p->Hkv != 0)
    return fail(TSA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->w > p->L) return fail(TSA_ERR_INVALID_ARG, "w=%d exceeds L=%d", p->w, p->L);
  if (p->Hq > tsa::kMaxHq) return fail(TSA_ERR_INVALID_ARG, "Hq=%d exceeds %d", p->Hq, tsa::kMaxHq);
  if (int64_t(p->L) > tsa::kMaxL) return fail(TSA_ERR_INVALID_ARG, "L=%d exceeds 2^22", p->L);
  // Several launches put the (sequence, head) pair in grid y, whose limit is 65535.
  if (int64_t(p->B) * p->Hq > tsa::kMaxHeads)
    return fail(TSA_ERR_UNSUPPORTED, "B*Hq=%lld exceeds %d", (long long)(int64_t(p->B) * p->Hq),
                tsa::kMaxHeads);
  if (std::isnan(p->tau) || !(p->tau >= 0.0f) || !(p->tau < 1.0f))
    return fail(TSA_ERR_INVALID_ARG, "tau=%g is outside [0, 1)", double(p->tau));
  if (p->flags & ~(TSA_FLAG_NONCAUSAL_PROXY | TSA_FLAG_PER_HEAD_BUDGET | TSA_FLAG_KEEP_WINDOW))
    return fail(TSA_ERR_UNSUPPORTED, "unknown flag bits 0x%x", unsigned(p->flags));
  if (p->dtype != TSA_F32 && p->dtype != TSA_BF16)
    return fail(TSA_ERR_UNSUPPORTED, "dtype %d is not supported (TSA_F32=0, TSA_BF16=1)", p->dtype);
  if (p->d != 64 && p->d != 128)
    return fail(TSA_ERR_UNSUPPORTED, "head dim d=%d is not supported (64 or 128)", p->d);
  if (p->dtype == TSA_BF16 && (p->w + 31) / 32 > tsa::kMaxScoreTiles)
    return fail(TSA_ERR_UNSUPPORTED, "ceil(w/32) = %d proxy-row tiles per head exceeds %d (w <= %d)",
                (p->w + 31) / 32, tsa::kMaxScoreTiles, 32 * tsa::kMaxScoreTiles);
  *out = tsa::Shape{p->B, p->Hq, p->Hkv, p->L, p->d, p->w, p->tau, p->dtype, p->flags};
  return TSA_OK;
}

tsa_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(TSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(TSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return TSA_OK;
}

tsa_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(TSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
  if (need > 0 && (!ws || !aligned256(ws)))
    return fail(TSA_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  return TSA_OK;
}

// Host-forceable launch failure, for testing error propagation without a GPU fault.
bool fault_injected() {
  const char* e = std::getenv("TSA_FAULT_INJECT");
  return e && std::strcmp(e, "launch") == 0;
}

tsa_status launched(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(TSA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
  return ok();
}

tsa_status injected(const char* what) {
  return fail(TSA_ERR_HIP, "%s: injected launch failure (TSA_FAULT_INJECT)", what);
}

// ---------------------------------------------------------------- no-allocation scratch
// Library-owned scratch of tsa_forward_fused_noalloc: one copy of this array
// lives on every GPU the library runs on, for the life of the process.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in for the symbol); each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
constexpr size_t kNoAllocBytes = size_t(TSA_NOALLOC_SCRATCH_BYTES);
static_assert(kNoAllocBytes % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // per device, filled on first use

// Device address of this device's scratch array (resolved once per device).
tsa_status scratch_for(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TSA_ERR_UNSUPPORTED, "device %d is beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t err = hipGetDevice(&cur);
    if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
    void* ptr = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    if (err != hipSuccess || !ptr)
      return fail(TSA_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(err));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TSA_OK;
}

// The device a stream belongs to (the current device for the null stream).
tsa_status stream_device(hipStream_t st, int* dev) {
  hipError_t err = st ? hipStreamGetDevice(st, dev) : hipGetDevice(dev);
  if (err != hipSuccess) return fail(TSA_ERR_HIP, "stream device: %s", hipGetErrorString(err));
  return TSA_OK;
}

tsa_status run_forward_fused(const tsa::Shape& sh, const void* q, const void* k, const void* v,
                             void* o, int32_t* budget, int32_t* idx, char* base, hipStream_t st,
                             const char* what);

#define TSA_TRY(expr)                 \
  do {                                \
    tsa_status st_ = (expr);          \
    if (st_ != TSA_OK) return st_;    \
  } while (0)

}  // namespace

namespace tsa {

StepWs step_ws_layout(const Shape& s) {
  StepWs w{};
  size_t off = 0;
  w.part = off;
  off = align256(off + sizeof(float) * 2 * size_t(s.B) * s.Hq * s.w * s.n_chunk());
  w.rowstat = off;
  off = align256(off + sizeof(float) * 2 * size_t(s.B) * s.Hq * s.w);
  const size_t rows = size_t(s.bud_rows());
  w.sigma = off;
  off = align256(off + sizeof(uint64_t) * rows * s.L);
  w.bud_cand = off;
  off = align256(off + sizeof(uint64_t) * rows * s.L);
  w.bud_hcnt = off;                      // hcnt, hmass, ncand: contiguous (cleared together)
  off = align256(off + sizeof(uint32_t) * rows * kBudgetLogBuckets);
  w.bud_hmass = off;
  off = align256(off + sizeof(uint64_t) * rows * kBudgetLogBuckets);
  w.bud_ncand = off;
  off = align256(off + sizeof(uint32_t) * 2 * rows);
  const size_t heads = size_t(s.B) * s.Hq;
  w.sel_hist = off;
  off = align256(off + sizeof(uint32_t) * 3 * heads * kSelectBuckets);
  w.sel_state = off;
  off = align256(off + sizeof(uint32_t) * 3 * heads * 2);
  w.sel_tab = off;
  off = align256(off + sizeof(uint32_t) * heads * size_t(select_plan(s).nch) * kSelectTabStride);
  w.total = off;
  return w;
}

StepClear step_clear(const Shape& s, char* ws) {
  const StepWs w = step_ws_layout(s);
  StepClear c;
  c.p0 = reinterpret_cast<uint32_t*>(ws + w.bud_hcnt);
  c.n0 = budget_clear_words(s);
  c.p1 = reinterpret_cast<uint32_t*>(ws + w.sel_hist);   // the first level's histograms
  c.n1 = int64_t(s.B) * s.Hq * kSelectBuckets;
  return c;
}

FwdWs fwd_ws_layout(const Shape& s) {
  FwdWs f{};
  f.step = step_ws_layout(s);
  size_t off = f.step.total;
  const size_t heads = size_t(s.B) * s.Hq;
  f.scores = off;
  off = align256(off + sizeof(float) * heads * s.L);
  f.rank = off;
  off = align256(off + sizeof(int32_t) * heads * s.L);
  f.fused_total = off;
  const size_t tens = heads * size_t(s.L) * size_t(s.row_bytes());
  f.kc = off;
  off = align256(off + tens);
  f.vc = off;
  off = align256(off + tens);
  f.total = off;
  return f;
}

}  // namespace tsa

extern "C" {

const char* tsa_status_string(tsa_status st) {
  // A C caller may pass any int.  In C++ a value outside the enumerators'
  // range is undefined once loaded as the enum type, so read the bits as int.
  static_assert(sizeof(tsa_status) == sizeof(int), "tsa_status is int-sized");
  int v;
  std::memcpy(&v, &st, sizeof(v));
  switch (v) {
    case TSA_OK: return "TSA_OK";
    case TSA_ERR_INVALID_ARG: return "TSA_ERR_INVALID_ARG";
    case TSA_ERR_UNSUPPORTED: return "TSA_ERR_UNSUPPORTED";
    case TSA_ERR_WORKSPACE: return "TSA_ERR_WORKSPACE";
    case TSA_ERR_HIP: return "TSA_ERR_HIP";
  }
  return "TSA_ERR_UNKNOWN";
}

const char* tsa_last_error(void) { return g_last_error.c_str(); }

const char* tsa_version(void) { return "tsa 0.1 gfx950"; }

size_t tsa_workspace_bytes(const tsa_problem* prob) {
  tsa::Shape s;
  if (check_problem(prob, &s) != TSA_OK) return 0;
  return tsa::step_ws_layout(s).total;
}

size_t tsa_forward_workspace_bytes(const tsa_problem* prob) {
  tsa::Shape s;
  if (check_problem(prob, &s) != TSA_OK) return 0;
  return tsa::fwd_ws_layout(s).total;
}

size_t tsa_fused_workspace_bytes(const tsa_problem* prob) {
  tsa::Shape s;
  if (check_problem(prob, &s) != TSA_OK) return 0;
  return tsa::fwd_ws_layout(s).fused_total;
}

tsa_status tsa_score(const tsa_problem* prob, const void* q, const void* k, float* s, void* ws,
                     size_t ws_bytes, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(s, "s"));
  TSA_TRY(check_ws(ws, ws_bytes, tsa::step_ws_layout(sh).total));
  if (fault_injected()) return injected("tsa_score");
  return launched(tsa::launch_score(sh, q, k, s, static_cast<char*>(ws), hipStream_t(stream)),
                  "tsa_score");
}

tsa_status tsa_budget(const tsa_problem* prob, const float* s, int32_t* budget, void* ws,
                      size_t ws_bytes, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(s, "s"));
  TSA_TRY(check_ptr(budget, "budget"));
  TSA_TRY(check_ws(ws, ws_bytes, tsa::step_ws_layout(sh).total));
  if (fault_injected()) return injected("tsa_budget");
  return launched(tsa::launch_budget(sh, s, budget, static_cast<char*>(ws), hipStream_t(stream)),
                  "tsa_budget");
}

tsa_status tsa_select(const tsa_problem* prob, const float* s, const int32_t* budget, int32_t* idx,
                      int32_t* rank, void* ws, size_t ws_bytes, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(s, "s"));
  TSA_TRY(check_ptr(budget, "budget"));
  TSA_TRY(check_ptr(idx, "idx"));
  TSA_TRY(check_ptr(rank, "rank"));
  TSA_TRY(check_ws(ws, ws_bytes, tsa::step_ws_layout(sh).total));
  if (fault_injected()) return injected("tsa_select");
  return launched(
      tsa::launch_select(sh, s, budget, idx, rank, static_cast<char*>(ws), hipStream_t(stream)),
      "tsa_select");
}

tsa_status tsa_gather(const tsa_problem* prob, const void* q, const void* k, const void* v,
                      const int32_t* idx, const int32_t* budget, void* qc, void* kc, void* vc,
                      void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(idx, "idx"));
  TSA_TRY(check_ptr(budget, "budget"));
  if (qc) TSA_TRY(check_ptr(qc, "qc"));   // NULL: K and V only
  TSA_TRY(check_ptr(kc, "kc"));
  TSA_TRY(check_ptr(vc, "vc"));
  if (fault_injected()) return injected("tsa_gather");
  return launched(tsa::launch_gather(sh, q, k, v, idx, budget, qc, kc, vc, hipStream_t(stream)),
                  "tsa_gather");
}

tsa_status tsa_gather_kv(const tsa_problem* prob, const void* k, const void* v,
                         const int32_t* rank, void* kc, void* vc, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(rank, "rank"));
  TSA_TRY(check_ptr(kc, "kc"));
  TSA_TRY(check_ptr(vc, "vc"));
  if (fault_injected()) return injected("tsa_gather_kv");
  return launched(tsa::launch_gather_kv_by_rank(sh, k, v, rank, kc, vc, hipStream_t(stream)),
                  "tsa_gather_kv");
}

tsa_status tsa_attention(const tsa_problem* prob, const void* q, const void* k, const void* v,
                         const int32_t* budget, int32_t kv_group, void* o, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(o, "o"));
  if (budget && !aligned16(budget)) return fail(TSA_ERR_INVALID_ARG, "budget is not 16-byte aligned");
  if (kv_group < 1 || sh.Hq % kv_group != 0)
    return fail(TSA_ERR_INVALID_ARG, "kv_group=%d must be >= 1 and divide Hq=%d", kv_group, sh.Hq);
  if (fault_injected()) return injected("tsa_attention");
  return launched(
      tsa::launch_attention(sh, q, k, v, budget, nullptr, kv_group, o, hipStream_t(stream)),
      "tsa_attention");
}

size_t tsa_block_mask_words(const tsa_problem* prob) {
  tsa::Shape s;
  if (check_problem(prob, &s) != TSA_OK) return 0;
  const size_t nb = (size_t(s.L) + 63) / 64, nw = (nb + 31) / 32;
  return size_t(s.B) * s.Hq * nb * nw;
}

tsa_status tsa_attention_block_sparse(const tsa_problem* prob, const void* q, const void* k,
                                      const void* v, const int32_t* budget, int32_t kv_group,
                                      const uint32_t* block_mask, void* o, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(o, "o"));
  TSA_TRY(check_ptr(block_mask, "block_mask"));
  if (budget && !aligned16(budget)) return fail(TSA_ERR_INVALID_ARG, "budget is not 16-byte aligned");
  if (kv_group < 1 || sh.Hq % kv_group != 0)
    return fail(TSA_ERR_INVALID_ARG, "kv_group=%d must be >= 1 and divide Hq=%d", kv_group, sh.Hq);
  if (fault_injected()) return injected("tsa_attention_block_sparse");
  return launched(tsa::launch_attention(sh, q, k, v, budget, nullptr, kv_group, o,
                                        hipStream_t(stream), block_mask),
                  "tsa_attention_block_sparse");
}

tsa_status tsa_scatter(const tsa_problem* prob, const void* oc, const int32_t* rank, void* o,
                       void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(oc, "oc"));
  TSA_TRY(check_ptr(rank, "rank"));
  TSA_TRY(check_ptr(o, "o"));
  if (fault_injected()) return injected("tsa_scatter");
  return launched(tsa::launch_scatter(sh, oc, rank, o, hipStream_t(stream)), "tsa_scatter");
}

tsa_status tsa_forward(const tsa_problem* prob, const void* q, const void* k, const void* v, void* o,
                       int32_t* budget, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(o, "o"));
  TSA_TRY(check_ptr(budget, "budget"));
  TSA_TRY(check_ptr(idx, "idx"));
  const tsa::FwdWs f = tsa::fwd_ws_layout(sh);
  TSA_TRY(check_ws(ws, ws_bytes, f.total));
  if (fault_injected()) return injected("tsa_forward");
  char* base = static_cast<char*>(ws);
  hipStream_t st = hipStream_t(stream);
  // Up to 32K tokens the attention reading K and V through the index set
  // (the fused path) is faster than writing the compact copies and reading
  // them back; the bits are the same.
  if (sh.L <= tsa::kForwardFusedMaxL)
    return run_forward_fused(sh, q, k, v, o, budget, idx, base, st, "tsa_forward");
  float* scores = reinterpret_cast<float*>(base + f.scores);
  int32_t* rank = reinterpret_cast<int32_t*>(base + f.rank);
  void* kc = base + f.kc;
  void* vc = base + f.vc;
  hipError_t err;
  // the scoring pass zeroes what the budget and the selection start from
  const tsa::StepClear clr = tsa::step_clear(sh, base);
  if ((err = tsa::launch_score(sh, q, k, scores, base, st, &clr)) != hipSuccess)
    return launched(err, "tsa_forward/score");
  if ((err = tsa::launch_budget(sh, scores, budget, base, st, true)) != hipSuccess)
    return launched(err, "tsa_forward/budget");
  // the selection's compaction also zeroes the rows of o it leaves out
  if ((err = tsa::launch_select(sh, scores, budget, idx, rank, base, st, true, o)) != hipSuccess)
    return launched(err, "tsa_forward/select");
  // Compression of K and V (each source row read once, written to every head
  // that selected it); the attention reads Q and writes O through the index
  // set: with the zeroed rows, the same bits as gather, attention on the
  // compact Q, K, V and scatter.
  if ((err = tsa::launch_gather_kv_by_rank(sh, k, v, rank, kc, vc, st)) != hipSuccess)
    return launched(err, "tsa_forward/gather");
  if ((err = tsa::launch_attention_qo(sh, q, kc, vc, budget, idx, o, st)) != hipSuccess)
    return launched(err, "tsa_forward/attention");
  return ok();
}

tsa_status tsa_attention_indexed(const tsa_problem* prob, const void* q, const void* k,
                                 const void* v, const int32_t* idx, const int32_t* budget, void* o,
                                 void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(idx, "idx"));
  TSA_TRY(check_ptr(budget, "budget"));
  TSA_TRY(check_ptr(o, "o"));
  if (fault_injected()) return injected("tsa_attention_indexed");
  return launched(tsa::launch_attention(sh, q, k, v, budget, idx, sh.Hq / sh.Hkv, o,
                                        hipStream_t(stream)),
                  "tsa_attention_indexed");
}

tsa_status tsa_attention_qo_indexed(const tsa_problem* prob, const void* q, const void* kc,
                                    const void* vc, const int32_t* idx, const int32_t* budget,
                                    void* o, void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(kc, "kc"));
  TSA_TRY(check_ptr(vc, "vc"));
  TSA_TRY(check_ptr(idx, "idx"));
  TSA_TRY(check_ptr(budget, "budget"));
  TSA_TRY(check_ptr(o, "o"));
  if (fault_injected()) return injected("tsa_attention_qo_indexed");
  return launched(tsa::launch_attention_qo(sh, q, kc, vc, budget, idx, o, hipStream_t(stream)),
                  "tsa_attention_qo_indexed");
}

tsa_status tsa_zero_unselected(const tsa_problem* prob, const int32_t* rank, void* o,
                               void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_problem(prob, &sh));
  TSA_TRY(check_ptr(rank, "rank"));
  TSA_TRY(check_ptr(o, "o"));
  if (fault_injected()) return injected("tsa_zero_unselected");
  return launched(tsa::launch_zero_unselected(sh, rank, o, hipStream_t(stream)),
                  "tsa_zero_unselected");
}

}  // extern "C"

namespace {

// The kernels of the fused whole op, with their scratch at `base` (the
// layout of tsa::fwd_ws_layout up to fused_total).
tsa_status run_forward_fused(const tsa::Shape& sh, const void* q, const void* k, const void* v,
                             void* o, int32_t* budget, int32_t* idx, char* base, hipStream_t st,
                             const char* what) {
  const tsa::FwdWs f = tsa::fwd_ws_layout(sh);
  float* scores = reinterpret_cast<float*>(base + f.scores);
  int32_t* rank = reinterpret_cast<int32_t*>(base + f.rank);
  hipError_t err;
  const tsa::StepClear clr = tsa::step_clear(sh, base);
  if ((err = tsa::launch_score(sh, q, k, scores, base, st, &clr)) != hipSuccess)
    return launched(err, what);
  if ((err = tsa::launch_budget(sh, scores, budget, base, st, true)) != hipSuccess)
    return launched(err, what);
  // the selection's compaction also zeroes the rows of o it leaves out
  if ((err = tsa::launch_select(sh, scores, budget, idx, rank, base, st, true, o)) != hipSuccess)
    return launched(err, what);
  if ((err = tsa::launch_attention(sh, q, k, v, budget, idx, sh.Hq / sh.Hkv, o, st)) != hipSuccess)
    return launched(err, what);
  return ok();
}

tsa_status check_forward_args(const tsa_problem* prob, const void* q, const void* k,
                              const void* v, const void* o, const int32_t* budget,
                              const int32_t* idx, tsa::Shape* sh) {
  TSA_TRY(check_problem(prob, sh));
  TSA_TRY(check_ptr(q, "q"));
  TSA_TRY(check_ptr(k, "k"));
  TSA_TRY(check_ptr(v, "v"));
  TSA_TRY(check_ptr(o, "o"));
  TSA_TRY(check_ptr(budget, "budget"));
  TSA_TRY(check_ptr(idx, "idx"));
  return TSA_OK;
}

}  // namespace

extern "C" {

tsa_status tsa_forward_fused(const tsa_problem* prob, const void* q, const void* k, const void* v,
                             void* o, int32_t* budget, int32_t* idx, void* ws, size_t ws_bytes,
                             void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_forward_args(prob, q, k, v, o, budget, idx, &sh));
  TSA_TRY(check_ws(ws, ws_bytes, tsa::fwd_ws_layout(sh).fused_total));
  if (fault_injected()) return injected("tsa_forward_fused");
  return run_forward_fused(sh, q, k, v, o, budget, idx, static_cast<char*>(ws),
                           hipStream_t(stream), "tsa_forward_fused");
}

tsa_status tsa_forward_fused_noalloc(const tsa_problem* prob, const void* q, const void* k,
                                     const void* v, void* o, int32_t* budget, int32_t* idx,
                                     void* stream) {
  tsa::Shape sh;
  TSA_TRY(check_forward_args(prob, q, k, v, o, budget, idx, &sh));
  const size_t need = tsa::fwd_ws_layout(sh).fused_total;
  if (need > kNoAllocBytes)
    return fail(TSA_ERR_UNSUPPORTED,
                "this problem needs %zu bytes of scratch; the no-allocation entry point holds "
                "%zu (use tsa_forward_fused with a workspace)", need, kNoAllocBytes);
  if (fault_injected()) return injected("tsa_forward_fused_noalloc");
  hipStream_t st = hipStream_t(stream);
  int dev = 0;
  TSA_TRY(stream_device(st, &dev));
  void* base = nullptr;
  TSA_TRY(scratch_for(dev, &base));
  return run_forward_fused(sh, q, k, v, o, budget, idx, static_cast<char*>(base), st,
                           "tsa_forward_fused_noalloc");
}

}  // extern "C"
