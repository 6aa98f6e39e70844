/*
 * sap.h -- document-masked causal attention for one sequence-parallel rank,
 * on AMD Instinct MI355X (gfx950). C ABI of libsap.so.
 *
 * What is computed. Several documents are packed into one sequence; a token
 * attends to itself and to earlier tokens of its own document only (HSAP
 * summary page, gptget.net/papers/2606.30460, original abstract: causal
 * attention on packed sequences without cross-contamination). Masks are
 * defined on global token positions, so they stay right after the sequence
 * is sharded (AutoSP page, gist.science/zh/paper/2604.27089, section 2.A,
 * index recomputation). A rank holds some query rows and, per call, some
 * key/value rows -- one ring step's chunks (SP blog page,
 * bmjup.com/post/14448.html, core principles: ring of KV chunks) or, for a
 * head-sharded rank, the whole sequence (same page, comparison table: head
 * split with all-to-all). Each call returns partial O plus log-sum-exp; the
 * partials merge exactly into full attention (same page, FAQ Q1:
 * computation-equivalent to one device).
 *
 * For query row r (global position i) and key row c (global position j):
 *     allowed(r, c)  <=>  ds(i) <= j <= i,   ds(i) = first position of i's document
 *     O[r,h]   = sum_c softmax_c(scale * q[r,h].k[c,g]) v[c,g]   over allowed c
 *     LSE[h,r] = ln sum_c exp(scale * q[r,h].k[c,g])              (natural log)
 *     g = h / (Hq / Hkv)  (contiguous GQA groups)
 * A row with no allowed key in a call has O = 0 and LSE = -inf exactly.
 *
 * Conventions shared by every entry point:
 *  - Device tensors are plain device pointers. Layouts: q, dout bf16
 *    [rows][Hq][D] with row stride q_row_stride elements; k, v bf16
 *    [rows][Hkv][D] with row stride kv_row_stride elements; the head stride is
 *    D and D is contiguous. o, dq fp32 [Tq][Hq][D] dense; lse fp32 [Hq][Tq]
 *    dense; dk, dv fp32 [Tkv][Hkv][D] dense. Tq / Tkv are the plan's local
 *    row counts (one past the last local row of its segments).
 *  - Pointers must be 16-byte aligned, row strides multiples of 8 elements.
 *  - The caller owns every tensor, stream and workspace. The library
 *    allocates device memory only in sap_plan_upload (freed by
 *    sap_plan_free); compute calls allocate nothing.
 *  - Compute calls are asynchronous on the given hipStream_t (NULL = the
 *    null stream) and never synchronise the host.
 *  - Every argument is checked on the host before anything is launched; on
 *    error nothing is launched and sap_last_error() describes the problem.
 *    Launch failures return SAP_ERR_HIP. No C++ exception crosses the ABI.
 *  - Plans are immutable after creation and may be shared by calls on any
 *    stream; sap_plan_free requires that no call using the plan is in flight.
 */
#ifndef SAP_H
#define SAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAP_OK = 0,
  SAP_ERR_INVALID_ARG = 1,  /* bad pointer, size, segment table, stride ... */
  SAP_ERR_UNSUPPORTED = 2,  /* valid but not compiled (head_dim, tile shape) or too large for one dispatch */
  SAP_ERR_NO_MEMORY = 3,    /* host or device allocation failed */
  SAP_ERR_HIP = 4,          /* a HIP runtime call or launch failed */
  SAP_ERR_STATE = 5         /* e.g. a compute call on a plan not uploaded */
} sap_status;

/* Global positions [global_start, global_end) of the packed sequence map to
 * local buffer rows local_start, local_start + 1, ... */
typedef struct {
  int32_t global_start;
  int32_t global_end;
  int32_t local_start;
} sap_segment;

enum { SAP_TILE_FULL = 0, SAP_TILE_DIAGONAL = 1, SAP_TILE_PARTIAL = 2 };

typedef struct sap_plan_s *sap_plan_t;

typedef struct {
  int64_t n_tiles;               /* listed (non-empty) tile pairs */
  int64_t n_full, n_diagonal, n_partial;
  int64_t useful_pairs_per_head; /* allowed (query, key) pairs in this call */
  int32_t n_q_tiles, n_kv_tiles;
  int32_t n_touched_q_tiles;     /* Q tiles with at least one listed pair */
  int32_t n_touched_kv_tiles;    /* KV tiles with at least one listed pair */
  int32_t tq, tkv;               /* local row counts */
  int32_t block_m, block_n;
  int32_t uploaded;              /* 1 after sap_plan_upload */
} sap_plan_stats;

/*
 * sap_plan -- the sequence-aware schedule of one call (host only).
 * The one-device form of the HSAP summary page's method section: the
 * schedule for incomplete tensors and irregular attention is generated ahead
 * of the run. It lists every (Q tile, KV tile) pair that holds at least one
 * allowed pair, with its mask class:
 *   Q tiles: runs of block_m local rows from each Q segment's local_start
 *   (the last run of a segment may be shorter), numbered over the segments in
 *   local-row order; KV tiles likewise with block_n.
 *   For a Q tile with positions [a, b] and a KV tile [c, e]:
 *     EMPTY (omitted) <=> c > b or e < ds(a);
 *     FULL <=> e <= a and c >= ds(b);  DIAGONAL <=> not FULL and c >= ds(b);
 *     PARTIAL otherwise.
 *   Listed in q_tile then kv_tile ascending order.
 * cu_seqlens: host int32 [n_docs + 1], cu[0] = 0, non-decreasing (empty
 *   documents allowed), cu[n_docs] = total length < 2^31.
 * q_segs / kv_segs: host arrays; each segment inside [0, total), global
 *   ranges pairwise disjoint and local ranges pairwise disjoint within a
 *   table. n_kv_segs may be 0 (an empty call).
 * block_m, block_n: one of 16, 32, 64, 128, 256. Compute calls accept only
 *   the shapes they are compiled for: forward 128 x 64 or 256 x 64
 *   (block_m x block_n; 256-row tiles let the 8 waves of a workgroup share
 *   each K/V tile when the GQA group size is odd), backward 64 x 128; merge
 *   accepts any plan.
 * out: receives the plan; release with sap_plan_free.
 * Errors: SAP_ERR_INVALID_ARG, SAP_ERR_NO_MEMORY.
 */
sap_status sap_plan(const int32_t *cu_seqlens, int32_t n_docs,
                    const sap_segment *q_segs, int32_t n_q_segs,
                    const sap_segment *kv_segs, int32_t n_kv_segs,
                    int32_t block_m, int32_t block_n, sap_plan_t *out);

/* Copies the plan's device tables to the current HIP device (hipMalloc +
 * copy on hip_stream, then waits for the copy). Needed once before any
 * compute call. Errors: SAP_ERR_INVALID_ARG, SAP_ERR_NO_MEMORY, SAP_ERR_HIP. */
sap_status sap_plan_upload(sap_plan_t plan, void *hip_stream);

/* Summary counts of a plan. */
sap_status sap_plan_info(sap_plan_t plan, sap_plan_stats *out);

/* Host copy of the tile list in canonical order; cap = capacity of each
 * output array (must be >= n_tiles). Any output pointer may be NULL. */
sap_status sap_plan_tiles(sap_plan_t plan, int32_t *q_tile, int32_t *kv_tile,
                          uint8_t *cls, int64_t cap);

/* Host copy of the touched Q tiles (ascending) and, per Q tile, its
 * (local_start, n_rows, global_start) triple into q_tiles_desc[3*n_q_tiles]. */
sap_status sap_plan_q_tiles(sap_plan_t plan, int32_t *touched, int32_t cap_touched,
                            int32_t *q_tiles_desc, int32_t cap_desc);

/* Frees host and device memory of a plan. NULL is ignored. */
void sap_plan_free(sap_plan_t plan);

/*
 * sap_balance -- document-aware assignment of query chunks to ranks (host
 * only). Uneven document lengths leave some GPUs idle (SP blog page,
 * bmjup.com/post/14448.html, future trends and challenges); the HSAP summary
 * page (gptget.net/papers/2606.30460, technical contributions) balances the
 * devices by scheduling. The sequence is cut into chunks of chunk_rows
 * consecutive positions; chunk c's work is its allowed (query, key) pairs
 * per head, the sum over its positions i of i - ds(i) + 1. Every rank gets
 * n_chunks / n_ranks chunks (equal token counts); chunks are taken heaviest
 * first (ties: lower chunk index) and each goes to the rank with the least
 * work so far among those with room (ties: lower rank). A rank then holds
 * its chunks in ascending position order: its Q segment table, and the KV
 * rows it contributes to the other ranks.
 * cu_seqlens: as for sap_plan. The total length must be a positive multiple
 *   of chunk_rows * n_ranks.
 * owner: host int32 [n_chunks] (n_chunks = total / chunk_rows), receives the
 *   rank of every chunk; cap_owner = its capacity.
 * rank_work: host int64 [n_ranks] or NULL, receives each rank's work.
 * O(n_chunks log n_chunks + n_docs). Errors: SAP_ERR_INVALID_ARG,
 *   SAP_ERR_NO_MEMORY (nothing written on error).
 */
sap_status sap_balance(const int32_t *cu_seqlens, int32_t n_docs, int32_t n_ranks, int32_t chunk_rows,
                       int32_t *owner, int64_t cap_owner, int64_t *rank_work);

/*
 * sap_attn_fwd -- partial attention of the plan's Q rows against this call's
 * KV rows (one ring step, or the whole sequence for a head-sharded rank).
 * For every listed tile pair it takes S = q k^T on bf16 matrix cores (fp32
 * accumulate), masks by class, runs an online softmax in fp32 and
 * accumulates P v. Writes o [Tq][Hq][D] and lse [Hq][Tq] for exactly the
 * rows of touched Q tiles (rows of a touched tile with no allowed key get
 * O = 0, LSE = -inf); all other rows are left untouched.
 * q, k, v: bf16 device pointers to local row 0 of each buffer.
 * hq % hkv == 0; d in {64, 128}; scale > 0 (usually 1/sqrt(d)).
 * Plan tile shape must be 128 x 64 or 256 x 64 (same results). Deterministic
 * (no atomics).
 */
sap_status sap_attn_fwd(sap_plan_t plan, const void *q, const void *k, const void *v,
                        int64_t q_row_stride, int64_t kv_row_stride,
                        int32_t hq, int32_t hkv, int32_t d, float scale,
                        float *o, float *lse, void *hip_stream);

/*
 * sap_attn_fwd_merge -- sap_attn_fwd with the ring step's merge folded into
 * the kernel epilogue: this call's partial (O_b, L_b) over the plan's KV rows
 * is merged into the running result o_acc [Tq][Hq][D] / lse_acc [Hq][Tq]
 * (fp32 device, in place) exactly as sap_lse_merge does,
 *   L = ln(e^La + e^Lb);  O = e^(La-L) O_a + e^(Lb-L) O_b,
 * for the rows of touched Q tiles that have at least one allowed key in this
 * call; every other row keeps its running values. Same tile shapes
 * (128 x 64 or 256 x 64), arguments and checks as sap_attn_fwd. A ring rank calls sap_attn_fwd for
 * its first step and sap_attn_fwd_merge for each later step: no partial
 * buffers, no separate merge pass. Deterministic (no atomics).
 */
sap_status sap_attn_fwd_merge(sap_plan_t plan, const void *q, const void *k, const void *v,
                              int64_t q_row_stride, int64_t kv_row_stride,
                              int32_t hq, int32_t hkv, int32_t d, float scale,
                              float *o_acc, float *lse_acc, void *hip_stream);

/*
 * sap_lse_merge -- exact merge of a partial result into a running one
 * (SP blog page, bmjup.com/post/14448.html, FAQ Q1: sequence parallelism is
 * computation-equivalent to one device, so the ring's partial results must
 * combine into exactly the full-sequence attention; the log-sum-exp merge is
 * that combination):
 *   L = ln(e^La + e^Lb);  O = e^(La-L) O_a + e^(Lb-L) O_b
 * (a side with L = -inf contributes nothing -- its O is not read into the
 * result, so it may hold anything, even NaN; both -inf leaves O = 0,
 * L = -inf). In place on o_acc / lse_acc. With a plan, only the rows of its
 * touched Q tiles are read and written -- the rest are unchanged, which is
 * exact since the partial holds no keys for them; with plan == NULL all tq
 * rows are merged. tq must equal the plan's Tq when a plan is given.
 * Bound by HBM traffic: (12 D + 16) bytes per (row, head).
 */
sap_status sap_lse_merge(sap_plan_t plan, float *o_acc, float *lse_acc,
                         const float *o_part, const float *lse_part,
                         int32_t tq, int32_t hq, int32_t d, void *hip_stream);

/*
 * The backward (recompute form). Only O and LSE are kept from the forward;
 * the probabilities are recomputed from them instead of being stored -- the
 * attention-level echo of the AutoSP page (gist.science/zh/paper/2604.27089)
 * section 2.B, which keeps attention's saved state and recomputes the large
 * intermediates. The gradients are those of the mask and forward above
 * (HSAP summary page, gptget.net/papers/2606.30460, original abstract; AutoSP
 * page section 2.A step 4: masks on global positions), and the per-step
 * calls of a ring add up to the full-sequence gradient (SP blog page,
 * bmjup.com/post/14448.html, FAQ Q1: computation-equivalent to one device).
 *
 * sap_attn_bwd_workspace -- device workspace bytes of the backward calls:
 * fp32 row terms D_r = dO_r . O_r ([hq][Tq], omitted when hq == 0) followed
 * by the fp32 partial dK / dV sums of the plan's split KV tiles (the planner
 * splits a KV tile whose partner Q tiles are many into chunks handled by
 * separate workgroups; their partial sums are added up in a fixed order).
 * sap_attn_bwd needs sap_attn_bwd_workspace(plan, hq, hkv, d) bytes;
 * sap_attn_bwd_accumulate needs sap_attn_bwd_workspace(plan, 0, hkv, d),
 * which is 0 when the plan splits nothing. Returns 0 for invalid arguments.
 */
size_t sap_attn_bwd_workspace(sap_plan_t plan, int32_t hq, int32_t hkv, int32_t d);

/*
 * sap_attn_bwd -- recompute-based backward of this call's share (AutoSP page,
 * gist.science/zh/paper/2604.27089, section 2.B: recompute rather than store):
 *   P = exp(scale q k^T - LSE_final) on allowed pairs, D_r = dO_r . O_final_r,
 *   dV += P^T dO;  dS = P o (dO v^T - D);  dQ += scale dS k;  dK += scale dS^T q.
 * o / lse_final are the merged forward results over *all* KV rows, so the
 * sum of per-step calls is the full gradient. dq, dk, dv are ACCUMULATED
 * (+=, fp32); the caller zeroes them once. No atomics: dK/dV come from a
 * KV-major pass and dQ from a Q-major pass, each owning its output rows (a
 * split KV tile's chunks write workspace slots that one pass adds in a fixed
 * order), so the result is deterministic: the same inputs give the same
 * bits. workspace: device, 16-byte aligned, >= sap_attn_bwd_workspace(plan,
 * hq, hkv, d) bytes; its contents on entry do not matter. Calls sharing one
 * workspace must not overlap. q, k, v, dout bf16 and o fp32 as in the
 * conventions above; lse_final fp32 [Hq][Tq]; hq % hkv == 0, d in {64, 128};
 * scale > 0 and finite. Plan tile shape must be 64 x 128 (block_m x block_n).
 * Every argument of both passes (row terms, then dK/dV and dQ) is checked
 * before anything is launched. Errors: SAP_ERR_INVALID_ARG (NULL or
 * misaligned pointer, bad stride, workspace too small), SAP_ERR_UNSUPPORTED
 * (head dim, tile shape, or a plan too large for one dispatch's grid),
 * SAP_ERR_STATE (plan not uploaded to this device), SAP_ERR_HIP (launch).
 */
sap_status sap_attn_bwd(sap_plan_t plan, const void *q, const void *k, const void *v,
                        const float *o, const float *lse_final, const void *dout,
                        int64_t q_row_stride, int64_t kv_row_stride,
                        int32_t hq, int32_t hkv, int32_t d, float scale,
                        float *dq, float *dk, float *dv,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * sap_attn_bwd_rowterm -- the backward's row terms D_r = dO_r . O_r (O the
 * final merged forward output) for the rows of the plan's touched Q tiles,
 * into delta fp32 [Hq][Tq] (device; other rows untouched). HBM-bound.
 * Part of the recompute backward (AutoSP page, gist.science/zh/paper/2604.27089,
 * section 2.B): D_r replaces the stored probabilities' row sums of P dP.
 * Because it uses the final O, a ring rank computes it once, with the plan of
 * its own chunk (which touches every local row), and reuses it for every
 * step's sap_attn_bwd_accumulate -- so the steps add up to the one-device
 * gradient (SP blog page, bmjup.com/post/14448.html, FAQ Q1).
 * o: fp32 device [Tq][Hq][D]; dout: bf16 device, row stride q_row_stride;
 * hq > 0, d in {64, 128}. Plan tile shape 64 x 128. Errors:
 * SAP_ERR_INVALID_ARG (NULL or misaligned pointer, bad stride),
 * SAP_ERR_UNSUPPORTED (shape, or a plan too large for one dispatch),
 * SAP_ERR_STATE (plan not uploaded), SAP_ERR_HIP (launch failure).
 */
sap_status sap_attn_bwd_rowterm(sap_plan_t plan, const float *o, const void *dout,
                                int64_t q_row_stride, int32_t hq, int32_t d,
                                float *delta, void *hip_stream);

/*
 * sap_attn_bwd_accumulate -- sap_attn_bwd without the row-term pass (the
 * recompute backward of the AutoSP page, gist.science/zh/paper/2604.27089,
 * section 2.B, for one ring step: its dQ, dK, dV add into the running
 * gradients, which sum over the steps to the one-device gradient, SP blog
 * page, bmjup.com/post/14448.html, FAQ Q1). The caller passes delta fp32
 * [Hq][Tq] from sap_attn_bwd_rowterm (it must hold the rows of this plan's
 * touched Q tiles). Same outputs, layouts and accumulation rules as
 * sap_attn_bwd; equals sap_attn_bwd_dkdv followed by sap_attn_bwd_dq.
 * workspace: device, 16-byte aligned, >= sap_attn_bwd_workspace(plan, 0, hkv,
 * d) bytes (may be NULL when that is 0); calls sharing one workspace must not
 * overlap. Plan tile shape 64 x 128. Errors as sap_attn_bwd.
 */
sap_status sap_attn_bwd_accumulate(sap_plan_t plan, const void *q, const void *k, const void *v,
                                   const float *lse_final, const float *delta, const void *dout,
                                   int64_t q_row_stride, int64_t kv_row_stride,
                                   int32_t hq, int32_t hkv, int32_t d, float scale,
                                   float *dq, float *dk, float *dv,
                                   void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * sap_attn_bwd_dkdv -- the key-side half of sap_attn_bwd_accumulate: the
 * KV-major pass (per KV tile, over its partner Q tiles) that adds
 *   dV += P^T dO,  dK += scale dS^T q
 * into dk, dv (fp32 device [Tkv][Hkv][D], accumulated), then adds the
 * workspace slots of split KV tiles in a fixed order. A ring rank returns
 * dK / dV to the chunks' owners, so computing them first lets that transfer
 * overlap the dQ pass (the SP blog page's compute / communication overlap,
 * bmjup.com/post/14448.html, core principles); the maths is that of the
 * recompute backward (AutoSP page, gist.science/zh/paper/2604.27089,
 * section 2.B). Arguments as sap_attn_bwd_accumulate without dq; workspace
 * >= sap_attn_bwd_workspace(plan, 0, hkv, d) bytes. Deterministic.
 */
sap_status sap_attn_bwd_dkdv(sap_plan_t plan, const void *q, const void *k, const void *v,
                             const float *lse_final, const float *delta, const void *dout,
                             int64_t q_row_stride, int64_t kv_row_stride,
                             int32_t hq, int32_t hkv, int32_t d, float scale,
                             float *dk, float *dv, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * sap_attn_bwd_dq -- the query-side half of sap_attn_bwd_accumulate: the
 * Q-major pass (per Q tile, over its partner KV tiles) that recomputes
 * S and dP and adds dQ += scale dS k into dq (fp32 device [Tq][Hq][D],
 * accumulated). Same recompute backward (AutoSP page,
 * gist.science/zh/paper/2604.27089, section 2.B). Needs no workspace.
 * Arguments as sap_attn_bwd_accumulate without dk, dv, workspace.
 * Deterministic (each workgroup owns its dQ rows).
 */
sap_status sap_attn_bwd_dq(sap_plan_t plan, const void *q, const void *k, const void *v,
                           const float *lse_final, const float *delta, const void *dout,
                           int64_t q_row_stride, int64_t kv_row_stride,
                           int32_t hq, int32_t hkv, int32_t d, float scale,
                           float *dq, void *hip_stream);

/*
 * sap_attn_bwd_noalloc -- sap_attn_bwd for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving or
 * training loops, harnesses that forbid hipMalloc. It takes no workspace:
 * the row terms and the split-tile partial sums go to a fixed device scratch
 * array inside the library (SAP_BWD_NOALLOC_MAX_BYTES per GPU, reserved
 * when the library is loaded and held until the process ends). The call
 * allocates nothing -- no hipMalloc, hipFree or allocating library routine;
 * its first call on a device looks the array's address up once
 * (hipGetSymbolAddress) with that device current.
 * Arguments, outputs and accumulation rules are those of sap_attn_bwd (same
 * kernels, same bits). A plan whose sap_attn_bwd_workspace(plan, hq, hkv, d)
 * exceeds SAP_BWD_NOALLOC_MAX_BYTES is refused with SAP_ERR_UNSUPPORTED
 * before anything is launched (use sap_attn_bwd with a workspace); the 64 MiB
 * cover e.g. a 64K-token five-head training shard (1.2 MiB) or a 512K-token
 * four-head Ulysses shard (8 MiB), not a 32-head 128K zigzag rank (134 MiB).
 * Every call on one GPU shares that GPU's scratch and it keeps the last
 * call's contents: nothing needs clearing (each call writes every word it
 * reads before reading it), but calls that overlap on one GPU -- on
 * different streams, or from different threads -- race on it and must be
 * serialised by the caller.
 */
#define SAP_BWD_NOALLOC_MAX_BYTES (64u << 20)
sap_status sap_attn_bwd_noalloc(sap_plan_t plan, const void *q, const void *k, const void *v,
                                const float *o, const float *lse_final, const void *dout,
                                int64_t q_row_stride, int64_t kv_row_stride,
                                int32_t hq, int32_t hkv, int32_t d, float scale,
                                float *dq, float *dk, float *dv, void *hip_stream);

/* Message of the last failed call on this thread ("" if none). */
const char *sap_last_error(void);

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t sap_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAP_H */
