/*
 * tsa.h - C ABI of the Token Sparse Attention prefill library (libtsa.so).
 *
 * Method: "Token Sparse Attention: Efficient Long-Context Inference with
 * Interleaved Token Selection" (Jo, Kang, Song, Kim, 2026).  The method
 * detail is in the gist.science summary, section 2 "Methodology":
 *   - "Core architecture", stage 1 (compression): per attention head a set
 *     S_h of token indices is chosen from importance scores, and Q, K, V are
 *     gathered into dense, contiguous tensors of reduced length L' << L;
 *     selection is independent per head.
 *   - "Core architecture", stage 2 (decompression): the L' x d output is
 *     scattered back into a zero-initialised L x d tensor at the head's
 *     indices; unselected positions are zero.
 *   - "Dynamic Token Coverage": importance comes from a light proxy attention
 *     map of recent queries against all keys, summed column-wise; tokens are
 *     sorted by ascending importance and the tail is pruned while the pruned
 *     mass stays within a coverage threshold tau, which fixes one global
 *     budget; then every head takes its own top-k.
 *
 * Conventions shared by every entry point:
 *   - Memory: every tensor pointer is DEVICE memory allocated and owned by the
 *     caller.  The library never allocates, frees or synchronises the host;
 *     all work is enqueued on `stream` (a hipStream_t; NULL = null stream)
 *     and the call returns once it is enqueued.
 *   - Layout: row-major contiguous.  Q is [B,Hq,L,d], K and V are
 *     [B,Hkv,L,d], in `dtype` (TSA_F32 = float, TSA_BF16 = bfloat16).  Tensor
 *     pointers must be 16-byte aligned.  Offsets are 64-bit.
 *   - GQA: query head h uses KV head h / (Hq/Hkv).
 *   - Budget: the per-sequence budget K_b stays on the device ([B] int32).
 *     Compact per-head buffers have capacity L rows; kernels read K_b, so no
 *     host read-back happens anywhere and the sequence is graph-capturable.
 *   - Validation is synchronous and happens before anything is enqueued.
 *     TSA_ERR_INVALID_ARG: a null problem or tensor pointer, a misaligned
 *     tensor pointer, any dimension < 1, Hq % Hkv != 0, w > L, Hq > 4096,
 *     L > 2^22, tau outside [0, 1) or NaN, a bad kv_group.
 *     TSA_ERR_UNSUPPORTED: d not in {64, 128}, an unknown dtype, B*Hq > 65535
 *     (sequence-head pairs), or (bf16) w > 2944 (92 proxy-row tiles of 32 rows
 *     per head).
 *     TSA_ERR_WORKSPACE: ws_bytes below what the *_workspace_bytes query
 *     returns, or a null / misaligned (256 B) workspace.
 *     TSA_ERR_HIP: a launch failed; tsa_last_error() holds the detail.
 *   - Threading: no global mutable state except the thread-local error text
 *     and the per-device scratch address table of tsa_forward_fused_noalloc
 *     (filled once per device, under a lock); concurrent calls on different
 *     streams with different buffers are safe.
 */
#ifndef TSA_H_
#define TSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tsa_status {
  TSA_OK = 0,
  TSA_ERR_INVALID_ARG = 1,
  TSA_ERR_UNSUPPORTED = 2,
  TSA_ERR_WORKSPACE = 3,
  TSA_ERR_HIP = 4
} tsa_status;

typedef enum tsa_dtype { TSA_F32 = 0, TSA_BF16 = 1 } tsa_dtype;

/* Alternative readings of the method, as bits of tsa_problem.flags (0 = the
 * main reading).  The pages leave these points open ("Dynamic Token
 * Coverage", scoring and budget bullets); each bit switches one of them.
 *   TSA_FLAG_NONCAUSAL_PROXY  every proxy row sees all L keys (main reading:
 *                             row r sees keys j <= r).
 *   TSA_FLAG_PER_HEAD_BUDGET  each head cuts its own importance curve
 *                             against tau, so budgets differ per head: every
 *                             `budget` argument is then [B,Hq] int32 instead
 *                             of [B] (main reading: one budget per sequence
 *                             from the head-mean importance).
 *   TSA_FLAG_KEEP_WINDOW      the w proxy positions L-w..L-1 are never
 *                             pruned: only tokens before them are pruning
 *                             candidates, and every head keeps the window
 *                             plus its top (K - w) candidates (K >= w). */
enum {
  TSA_FLAG_NONCAUSAL_PROXY = 1,
  TSA_FLAG_PER_HEAD_BUDGET = 2,
  TSA_FLAG_KEEP_WINDOW = 4
};

/* Problem shape.  w: number of proxy (most recent) queries; tau: coverage
 * threshold in [0, 1).  dtype: a tsa_dtype value.  flags: TSA_FLAG_* bits
 * (0 for the main reading). */
typedef struct tsa_problem {
  int32_t B, Hq, Hkv, L, d, w;
  float tau;
  int32_t dtype;
  int32_t flags;
} tsa_problem;

/* "Budget" below means budget[b] for the main reading and budget[b,h] under
 * TSA_FLAG_PER_HEAD_BUDGET; K_b (or K_bh) is that value. */

/* Human-readable name of a status code (static storage); "TSA_ERR_UNKNOWN"
 * for a value that is not a tsa_status. */
const char* tsa_status_string(tsa_status st);

/* Detail text of the last failing call on this thread ("" if none). */
const char* tsa_last_error(void);

/* Library version string, e.g. "tsa 0.1 gfx950". */
const char* tsa_version(void);

/* Scratch bytes needed by tsa_score, tsa_budget and tsa_select (one buffer
 * serves all three; it need not be cleared).  0 on an invalid problem. */
size_t tsa_workspace_bytes(const tsa_problem* prob);

/* Scratch bytes needed by tsa_forward: the step scratch plus the
 * intermediate scores, rank map and the compact per-head K and V. */
size_t tsa_forward_workspace_bytes(const tsa_problem* prob);

/* Scratch bytes needed by tsa_forward_fused: the step scratch plus the
 * intermediate scores and rank map (no compact tensors). */
size_t tsa_fused_workspace_bytes(const tsa_problem* prob);

/* Proxy scoring ("Dynamic Token Coverage", scoring).  For every query head h
 * and proxy row r in [L-w, L): logits x_rj = <Q[b,h,r], K[b,g(h),j]>/sqrt(d)
 * over the causally visible keys j <= r, one softmax per row, and
 *   s[b,h,j] = (1/w) * sum_r p_rj        (each head's row sums to 1).
 * q: [B,Hq,L,d] (only the last w rows are read); k: [B,Hkv,L,d];
 * s: [B,Hq,L] float32 output.  Deterministic (fixed reduction order). */
tsa_status tsa_score(const tsa_problem* prob, const void* q, const void* k, float* s,
                     void* ws, size_t ws_bytes, void* stream);

/* Global budget ("Dynamic Token Coverage", budget allocation).  Per batch
 * element: sigma_j = sum_h floor(clip(s[b,h,j],0,1) * 2^50) (exact integers),
 * C(p) = sum of the p smallest sigma_j, P = max{p in [0,L-1] :
 * C(p) <= Hq*tau*2^50} (P = 0 when tau = 0), budget[b] = L - P.  This is the
 * head-mean pruned mass compared with tau, counted exactly in units of
 * 2^-50.  Scores whose per-head sums exceed 1 + 2^-10 (not produced by
 * tsa_score) give an unspecified but in-range budget.
 * s: [B,Hq,L] float32; budget: [B] int32 output. */
tsa_status tsa_budget(const tsa_problem* prob, const float* s, int32_t* budget,
                      void* ws, size_t ws_bytes, void* stream);

/* Per-head top-K ("Dynamic Token Coverage", per-head selection), K = budget[b].
 * Tokens are ranked by (s descending, index ascending); NaN and negative
 * scores rank as 0.  idx[b,h,0..K) receives the chosen indices in ascending
 * order and idx[b,h,K..L) = -1; rank[b,h,j] = position of j in that list,
 * or -1.  s: [B,Hq,L] float32; budget: [B] int32 (device, 1..L);
 * idx, rank: [B,Hq,L] int32 outputs. */
tsa_status tsa_select(const tsa_problem* prob, const float* s, const int32_t* budget,
                      int32_t* idx, int32_t* rank, void* ws, size_t ws_bytes, void* stream);

/* Compression ("Core architecture", stage 1).  For i < K_b:
 *   qc[b,h,i] = Q[b,h,idx_i], kc[b,h,i] = K[b,g(h),idx_i], vc[b,h,i] = V[b,g(h),idx_i].
 * Rows i >= K_b of qc/kc/vc are not written.  q: [B,Hq,L,d]; k, v:
 * [B,Hkv,L,d]; idx: [B,Hq,L] int32 (first K_b entries in [0,L));
 * qc, kc, vc: [B,Hq,L,d] outputs.  Bit-exact copies.  qc may be NULL: then
 * only kc and vc are written (the input of tsa_attention_qo_indexed). */
tsa_status tsa_gather(const tsa_problem* prob, const void* q, const void* k, const void* v,
                      const int32_t* idx, const int32_t* budget, void* qc, void* kc, void* vc,
                      void* stream);

/* Compression of K and V only ("Core architecture", stage 1), source-driven:
 * every K/V row of a KV head is read once and written to each of its query
 * heads that selected it,
 *   kc[b,h,rank[b,h,j]] = K[b,g(h),j], vc[b,h,rank[b,h,j]] = V[b,g(h),j]
 * for every j with rank[b,h,j] >= 0.  With rank as tsa_select writes it, this
 * is tsa_gather with qc = NULL, bit for bit; tsa_forward runs it.  k, v:
 * [B,Hkv,L,d]; rank: [B,Hq,L] int32 (values in [-1, L)); kc, vc: [B,Hq,L,d]
 * outputs (rows at or past K_b are not written). */
tsa_status tsa_gather_kv(const tsa_problem* prob, const void* k, const void* v,
                         const int32_t* rank, void* kc, void* vc, void* stream);

/* Causal attention on dense tensors (the compressed tensors, or the
 * uncompressed ones for the dense baseline).  For i < n:
 *   o[b,h,i] = sum_{j<=i} softmax_j(<q[b,h,i], k[b,h/kv_group,j]>/sqrt(d)) v[b,h/kv_group,j]
 * with n = budget[b] (device) or n = L when budget is NULL.  kv_group = 1 for
 * the compact per-head K/V (k, v: [B,Hq,L,d]); kv_group = Hq/Hkv for the
 * dense GQA layout (k, v: [B,Hkv,L,d]).  Rows i >= n of o are not written.
 * bf16: bf16 MFMA products, fp32 accumulation and softmax, output rounded
 * to nearest even; f32: fp32 throughout. */
tsa_status tsa_attention(const tsa_problem* prob, const void* q, const void* k, const void* v,
                         const int32_t* budget, int32_t kv_group, void* o, void* stream);

/* Words of the block mask taken by tsa_attention_block_sparse:
 * B * Hq * NB * NW with NB = ceil(L/64), NW = ceil(NB/32).  0 on an invalid
 * problem. */
size_t tsa_block_mask_words(const tsa_problem* prob);

/* Block-sparse attention on the compressed tensors: the composition with
 * sparse attention kernels that the pages name (section 3 "Key
 * contributions", compatibility item; section 4, combination with
 * FlexPrefill).  The sparse pattern itself comes from the caller.  As
 * tsa_attention, except that key j is visible to row i only when j <= i and
 * either i and j lie in the same block of 64 rows, or the mask marks the
 * (i / 64, j / 64) block pair visible:
 *   block_mask[((b*Hq + h)*NB + qb)*NW + kb/32] bit (kb % 32) == 1.
 * Diagonal blocks are always visible (so every row keeps at least itself);
 * bits at or above the diagonal are ignored.  Masked tiles are neither
 * loaded nor computed.  block_mask: device uint32, tsa_block_mask_words
 * words.  Results equal tsa_attention when every bit is set. */
tsa_status tsa_attention_block_sparse(const tsa_problem* prob, const void* q, const void* k,
                                      const void* v, const int32_t* budget, int32_t kv_group,
                                      const uint32_t* block_mask, void* o, void* stream);

/* Decompression ("Core architecture", stage 2).  For every j < L:
 *   o[b,h,j] = rank[b,h,j] >= 0 ? oc[b,h,rank[b,h,j]] : +0.0
 * Each output row is written exactly once.  oc: [B,Hq,L,d]; rank: [B,Hq,L]
 * int32 (values in [-1, L)); o: [B,Hq,L,d] output. */
tsa_status tsa_scatter(const tsa_problem* prob, const void* oc, const int32_t* rank, void* o,
                       void* stream);

/* The whole op: score -> budget -> select -> gather -> attention -> scatter,
 * run as tsa_score -> tsa_budget -> tsa_select -> tsa_gather of K and V ->
 * tsa_zero_unselected -> tsa_attention_qo_indexed, which gives the same bits
 * without materialising the compact Q and O (the zeroing of the unselected
 * rows is done by the selection's last pass, as it finds them, rather than
 * by a launch of its own).  For L <= 32768 it runs the
 * kernels of tsa_forward_fused instead (the attention reads K and V through
 * the index set, faster at those lengths), with the same bits again.
 * o: [B,Hq,L,d] output (unselected rows exactly zero); budget: [B] int32
 * output; idx: [B,Hq,L] int32 output (as tsa_select).  ws must hold
 * tsa_forward_workspace_bytes(prob) bytes. */
tsa_status tsa_forward(const tsa_problem* prob, const void* q, const void* k, const void* v,
                       void* o, int32_t* budget, int32_t* idx, void* ws, size_t ws_bytes,
                       void* stream);

/* Compression, attention and decompression of the selected rows in one
 * kernel ("Core architecture", stages 1 and 2, with the dense attention on
 * the compressed tensors between them).  For i < K_b, with t = idx[b,h,i]:
 *   o[b,h,t] = sum_{j<=i} softmax_j(<Q[b,h,t], K[b,g(h),idx_j]>/sqrt(d)) V[b,g(h),idx_j]
 * which is tsa_gather -> tsa_attention(kv_group=1) -> tsa_scatter on the
 * selected rows, bit for bit.  q, o: [B,Hq,L,d]; k, v: [B,Hkv,L,d];
 * idx: [B,Hq,L] int32 whose first K_b entries are ascending rows in [0,L)
 * (as tsa_select writes them); budget: [B] int32 (device).  Only the
 * selected rows of o are written; the other rows are left as they are. */
tsa_status tsa_attention_indexed(const tsa_problem* prob, const void* q, const void* k,
                                 const void* v, const int32_t* idx, const int32_t* budget, void* o,
                                 void* stream);

/* Attention of the selected queries over the compressed keys, with Q read and
 * O written through the index set ("Core architecture", stage 1 attention
 * and the copy part of stage 2).  For i < K_b, with t = idx[b,h,i]:
 *   o[b,h,t] = sum_{j<=i} softmax_j(<Q[b,h,t], kc[b,h,j]>/sqrt(d)) vc[b,h,j]
 * which is tsa_attention(qc, kc, vc, kv_group=1) -> tsa_scatter on the
 * selected rows, bit for bit, without the compact Q and O.  q, o:
 * [B,Hq,L,d]; kc, vc: [B,Hq,L,d] as tsa_gather writes them (first K_b rows
 * valid); idx: [B,Hq,L] int32 as tsa_select writes it; budget: [B] int32
 * (device), or [B,Hq] under TSA_FLAG_PER_HEAD_BUDGET.  Only the selected
 * rows of o are written; the other rows are left as they are. */
tsa_status tsa_attention_qo_indexed(const tsa_problem* prob, const void* q, const void* kc,
                                    const void* vc, const int32_t* idx, const int32_t* budget,
                                    void* o, void* stream);

/* Decompression when the attention writes the selected rows itself (the
 * whole op and the fused path; "Core architecture", stage 2, the zero part): o[b,h,j] = +0.0 for every j with rank[b,h,j] < 0; other rows are
 * left as they are.  rank: [B,Hq,L] int32 (as tsa_select writes it);
 * o: [B,Hq,L,d]. */
tsa_status tsa_zero_unselected(const tsa_problem* prob, const int32_t* rank, void* o, void* stream);

/* The whole op with the fused kernel: score -> budget -> select ->
 * tsa_zero_unselected -> tsa_attention_indexed (the zeroing again done by
 * the selection's last pass).  Same arguments and the
 * same results, bit for bit, as tsa_forward, without the compact K and V
 * (the attention reads them through the index set): ws must hold
 * tsa_fused_workspace_bytes(prob) bytes. */
tsa_status tsa_forward_fused(const tsa_problem* prob, const void* q, const void* k, const void* v,
                             void* o, int32_t* budget, int32_t* idx, void* ws, size_t ws_bytes,
                             void* stream);

/* Bytes of the library-owned scratch of tsa_forward_fused_noalloc: one copy
 * per GPU the library runs on, held until the process ends. */
#define TSA_NOALLOC_SCRATCH_BYTES (128u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * op, arguments and results (bit for bit) as tsa_forward_fused, with the
 * scratch taken from a static device array of TSA_NOALLOC_SCRATCH_BYTES
 * instead of a caller workspace.  Nothing is allocated: no hipMalloc,
 * hipFree or allocating library call.  The caller still passes every input
 * and output.
 *   - TSA_ERR_UNSUPPORTED when the problem's scratch
 *     (tsa_fused_workspace_bytes) exceeds TSA_NOALLOC_SCRATCH_BYTES;
 *     about 55 MiB at B=1, Hq=32, L=128K, w=64.
 *   - The scratch is resolved on the stream's device (the current device for
 *     the null stream) on its first call there; make that first call outside
 *     graph capture.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (the kernels clear what must start at zero).  Calls
 *     that overlap on one GPU (different streams or threads, no ordering
 *     between them) race on it and give undefined results. */
tsa_status tsa_forward_fused_noalloc(const tsa_problem* prob, const void* q, const void* k,
                                     const void* v, void* o, int32_t* budget, int32_t* idx,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H_ */
