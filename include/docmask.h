/*
 * docmask.h - C ABI of libdocmask.so: document-masked (intra-document causal)
 * attention over a packed variable-length sequence, as one context-parallel
 * rank computes it, on AMD Instinct MI355X (gfx950).
 *
 * Definitions come from public pages on context parallelism:
 *  - "FlashCP: Load-Balanced Communication-Efficient Context Parallelism for
 *    LLM Training", section 2.1 and Figure 1(a): documents are packed into one
 *    sequence and a query attends only to keys of its own document that are
 *    not after it (the diagonal is included, as the shard workload
 *    W = (2p + s + 1) s / 2 of section 3.1 counts it).  Section 2.2: a CP
 *    worker holds several query chunks (2 x CP chunking) and sees the KV of
 *    other workers.
 *  - "LLM Context Parallel in Production": document boundaries travel as
 *    cumulative-length arrays; results over separate KV blocks are combined
 *    with the row maximum and exponential sum (online softmax); kernels skip
 *    blocks with no valid pair and the effective block count is logged.
 *
 * Conventions shared by every call
 *  - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16).
 *  - Q, O, dO: [Tq][Hq][D] row-major, where the Tq local query rows are the
 *    chunks concatenated in list order.  K, V: [Tkv][Hkv][D] with
 *    Tkv = kv_hi - kv_lo; row r holds global position kv_lo + r.
 *  - LSE: float [Hq][Tq], natural log of the sum of exp(score).
 *  - cu_seqlens: device int32 [n_docs + 1], cu[0] = 0, non-decreasing; the
 *    documents cover every global position a call touches.
 *  - GQA: query head h reads KV head h / (Hq / Hkv).
 *  - A query row with no allowed key in [kv_lo, kv_hi) gets O = 0 and
 *    LSE = -inf.
 *  - Every pointer argument named *_dev or a tensor is device memory owned by
 *    the caller; chunk arrays are host memory read during the call.  The
 *    attention, merge, scheduler and exchange calls allocate nothing and
 *    keep no state between calls (everything a call needs lives in its
 *    arguments and the caller's workspace); they are re-entrant.  The only
 *    process-wide state is the opt-in kernel timer below (its event pool and
 *    totals).  Calls on one stream run in order; calls that share a
 *    workspace must not overlap.
 *  - Work is enqueued on `stream` (0 = the null stream).  The return value
 *    reports argument validation (checked on the host before anything is
 *    enqueued) and launch errors; device-side input errors (malformed
 *    cu_seqlens) are recorded in the workspace and read back with
 *    docmask_check_errors.
 *  - Tensor pointers must be 16-byte aligned; D must be 64 or 128;
 *    Hq % Hkv == 0; chunks must be disjoint, in ascending position order,
 *    and at most DOCMASK_MAX_CHUNKS; softmax_scale must be finite and
 *    positive (scale 0 would turn masked scores into NaN, a negative one
 *    would reverse the softmax reference), else DOCMASK_EINVAL.
 */
#ifndef DOCMASK_H
#define DOCMASK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DOCMASK_MAX_CHUNKS 256

/* Global query positions [g_start, g_start + len) held by this rank. */
typedef struct {
  int32_t g_start;
  int32_t len;
} docmask_chunk;

typedef enum {
  DOCMASK_OK = 0,
  DOCMASK_EINVAL = -1,        /* bad argument (null pointer, shape, chunk list, alignment) */
  DOCMASK_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. D not in {64, 128}) */
  DOCMASK_EWORKSPACE = -3,    /* workspace missing or smaller than docmask_workspace_size */
  DOCMASK_EHIP = -4,          /* a HIP launch failed */
  DOCMASK_EDEVICE_INPUT = -5, /* reported by docmask_check_errors: malformed cu_seqlens */
  DOCMASK_ESCRATCH = -6       /* docmask_attn_fwd_noalloc: problem exceeds its static scratch */
} docmask_status;

/* Operations a workspace is sized for. */
enum { DOCMASK_OP_FWD = 1, DOCMASK_OP_BWD = 2 };

/* Flags of docmask_attn_bwd. */
enum {
  /* Add this call's dQ share into dq instead of overwriting it: for split-KV
   * backward, where each call holds one KV block and the caller sums the
   * shares (dK and dV of each block are exact per call). */
  DOCMASK_ACCUMULATE_DQ = 1,
  /* The workspace already holds Delta = rowsum(dO * O) from an earlier call
   * with the same o, d_o, chunks and heads (e.g. the previous KV block of a
   * split-KV backward): skip recomputing it.  Delta sits at a fixed place in
   * the workspace that depends only on Hq and the chunk rows, so the earlier
   * call may have held a KV range of any length (the workspace must still be
   * large enough for every call that uses it). */
  DOCMASK_DELTA_READY = 2
};

/* Workspace bytes docmask_attn_fwd (op = DOCMASK_OP_FWD) or docmask_attn_bwd
 * (op = DOCMASK_OP_BWD) needs for this problem.  Returns 0 if the arguments
 * are invalid. */
size_t docmask_workspace_size(int op, int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks,
                              int32_t kv_lo, int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d);

/* Tile scheduler (block skipping; production guide "Causal Attention Creates
 * Rank Load Imbalance"; FlashCP section 3.2 for the need list).
 * Q tiles of bq rows are anchored at each chunk start and never cross a chunk;
 * KV tiles of bk keys are anchored at kv_lo; last tiles may be ragged.  A tile
 * pair is SKIP if it holds no allowed pair, FULL if every pair is allowed,
 * PARTIAL otherwise.  Outputs (device, int32 unless noted; any may be NULL):
 *   qtile_desc  [n_qtiles][4]  {kt_lo, kt_full_lo, kt_full_hi, kt_hi}: the
 *               non-skipped KV tiles [kt_lo, kt_hi) and the FULL ones inside;
 *               no FULL tile -> kt_full_lo = kt_full_hi = kt_hi; none at all
 *               -> all four 0.
 *   kvtile_desc [n_kvtiles][4] {qt_lo, qt_full_lo, qt_full_hi, qt_hi} over the
 *               global Q-tile index, same encoding.
 *   need        [n_chunks][2]  key positions [lo, hi) the chunk's rows may
 *               attend ((0, 0) if none): the chunk's KV need list.
 *   lpt_q       [n_qtiles]     Q tiles by descending non-skipped KV tile
 *               count, ties by ascending index.
 *   lpt_kv      [n_kvtiles]    KV tiles likewise.
 *   counters    int64 [4]      {non-skipped pairs, FULL, PARTIAL, allowed
 *               (row, key) pairs per head}.
 * n_qtiles = sum over chunks of ceil(len / bq); n_kvtiles =
 * ceil((kv_hi - kv_lo) / bk).  Workspace: docmask_schedule_workspace_size. */
size_t docmask_schedule_workspace_size(const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                                       int32_t kv_hi, int32_t bq, int32_t bk);
int docmask_schedule(const int32_t* cu_seqlens_dev, int32_t n_docs, const docmask_chunk* chunks,
                     int32_t n_chunks, int32_t kv_lo, int32_t kv_hi, int32_t bq, int32_t bk,
                     int32_t* qtile_desc, int32_t* kvtile_desc, int32_t* need, int32_t* lpt_q,
                     int32_t* lpt_kv, int64_t* counters, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Forward: O (bf16 [Tq][Hq][D]) and LSE (float [Hq][Tq]) of
 *   O_ih = sum_j softmax_j(scale * q_ih . k_j,h/G) v_j,h/G
 * over the allowed keys j in [kv_lo, kv_hi) (FlashCP section 2.1).  A call
 * whose KV range is one block of the sequence yields the partial result that
 * lse_merge combines. */
int docmask_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                     int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                     int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, kernels and
 * arguments as docmask_attn_fwd, with the workspace replaced by a static
 * device array of DOCMASK_NOALLOC_SCRATCH_BYTES inside the library (one per
 * GPU, held until the process ends; enough for about three million query
 * rows).  A problem whose docmask_workspace_size(DOCMASK_OP_FWD, ...)
 * exceeds it returns DOCMASK_ESCRATCH before anything is enqueued.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the caller still owns q, k, v, cu_seqlens, o and lse.  Every call on one
 * GPU shares that GPU's array: calls that may overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller.  Device
 * input errors are recorded in the array's first word; this entry point has
 * no error read-back of its own (use docmask_attn_fwd with a workspace and
 * docmask_check_errors to diagnose malformed cu_seqlens). */
#define DOCMASK_NOALLOC_SCRATCH_BYTES (4u << 20)
int docmask_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                             int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                             int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* o,
                             float* lse, hipStream_t stream);

/* Forward with O written as float32 [Tq][Hq][D] (otherwise identical to
 * docmask_attn_fwd, same workspace): partial results for lse_merge_f32, so
 * that a row's value is rounded to bf16 once, after the merge, instead of
 * once per partial and again after it. */
int docmask_attn_fwd_f32out(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                            int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                            int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d, float softmax_scale, float* o,
                            float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward: exact gradients of <dO, O> (FlashCP Figure 6 "Attention BWD";
 * the pages do not write it out, so this is the plain calculus):
 *   P = exp(S - LSE), Delta = rowsum(dO * O), dV = P^T dO,
 *   dS = P * (dO V^T - Delta), dQ = scale dS K, dK = scale dS^T Q,
 * summing dK and dV over the query heads of each KV group.  o and lse are the
 * forward's outputs over the full KV extent of the rows (the merged values
 * for split-KV).  Outputs are float32: dq [Tq][Hq][D], dk and dv
 * [Tkv][Hkv][D].  dq is overwritten unless flags has DOCMASK_ACCUMULATE_DQ;
 * Delta is recomputed unless flags has DOCMASK_DELTA_READY.  Precision: the
 * products run on bf16 matrix cores (P and dS rounded to bf16), except the
 * pairs among each document's first 32 positions -- the rows with the fewest
 * keys, whose P and dS are the largest -- which are computed in float32, with
 * their rows' Delta taken from the float32 P and dP rather than from the bf16
 * o when all their keys lie in [kv_lo, kv_hi). */
int docmask_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* d_o, const int32_t* cu_seqlens_dev, int32_t n_docs,
                     const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo, int32_t kv_hi,
                     int32_t hq, int32_t hkv, int32_t d, float softmax_scale, float* dq, float* dk,
                     float* dv, int flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Online-softmax merge of partial results over disjoint KV ranges (production
 * guide, "Core Principle: Split Q, Circulate KV"): per row and head,
 *   m = max_p LSE_p, LSE = m + ln sum_p exp(LSE_p - m),
 *   O = sum_p exp(LSE_p - LSE) O_p;  all partials empty -> (0, -inf).
 * o_parts: bf16 [n_parts][rows][hq][d]; lse_parts: float [n_parts][hq][rows];
 * o_out: bf16 [rows][hq][d]; lse_out: float [hq][rows].  n_parts >= 1.  Math
 * in float32.  Outputs must not alias inputs. */
int lse_merge(const void* o_parts, const float* lse_parts, int32_t n_parts, int32_t rows, int32_t hq,
              int32_t d, void* o_out, float* lse_out, hipStream_t stream);

/* lse_merge over float32 partials o_parts [n_parts][rows][hq][d] (from
 * docmask_attn_fwd_f32out); same rule, arguments and bf16 outputs. */
int lse_merge_f32(const float* o_parts, const float* lse_parts, int32_t n_parts, int32_t rows, int32_t hq,
                  int32_t d, void* o_out, float* lse_out, hipStream_t stream);

/* Waits for `stream`, then reports device-side input errors recorded in a
 * workspace by the last call that used it: DOCMASK_OK or
 * DOCMASK_EDEVICE_INPUT (cu_seqlens not starting at 0, decreasing, or not
 * covering the positions used).  After such an error the attention kernels
 * of that call wrote nothing. */
int docmask_check_errors(const void* workspace, hipStream_t stream);

/* float32 -> bf16 (round to nearest even) copy of n elements, for callers
 * that want bf16 gradients. */
int docmask_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t stream);

const char* docmask_strerror(int status);

/* ------------------------------------------------------------------------
 * KV exchange of sharding-aware context parallelism (FlashCP section 3.2,
 * "Dynamic Sharding-aware Communication", and Eq. 5): a worker sends only the
 * KV rows of its document shards that are not the last shard of their
 * document (a document kept whole on one worker is its own last shard),
 * compacted into one continuous buffer with no per-document padding; the
 * collective itself is the caller's.  A receiving worker places the rows its
 * chunks need, and its own rows, at their global positions in the KV range
 * [kv_lo, kv_hi) the attention entry points take.  Shards are the
 * intersections of a worker's chunks with documents.
 *
 * Row maps are host arrays: rows [src, src + len) of a source go to rows
 * [dst, dst + len) of a destination.
 */
typedef struct {
  int32_t src;
  int32_t dst;
  int32_t len;
} docmask_rowmap;

/* Copies rows by a map list: dst[m.dst + t] = src[m.src + t] for every map m
 * and t < m.len, for one tensor (src_v = dst_v = NULL) or two (K and V, same
 * maps); a map with src = -1 writes len zero rows at dst instead.  Rows are
 * row_bytes long (a positive multiple of 16; Hkv * D * 2 for bf16 KV).  Maps
 * must be sorted by dst and disjoint there, with len >= 0, src >= -1 and
 * every row inside [0, src_rows) and [0, dst_rows); any number of maps (one
 * launch per 128).  zero_gaps != 0 also zeroes every destination row that no
 * map covers, so that the whole of [0, dst_rows) is written; otherwise those
 * rows are left untouched.  Source and destination must not overlap; tensor
 * pointers 16-byte aligned; source pointers are checked only when a map
 * copies, and a call that writes nothing (dst_rows = 0, or no map and no
 * zeroing) checks no pointer.  Bandwidth bound: copied rows are read once and
 * every written row is written once. */
int docmask_copy_rows(const void* src_k, const void* src_v, int64_t src_rows, void* dst_k, void* dst_v,
                      int64_t dst_rows, int64_t row_bytes, const docmask_rowmap* maps, int32_t n_maps,
                      int zero_gaps, hipStream_t stream);

/* Sharding planner, host only: FlashCP's heuristic (Algorithm 1, section
 * 3.4) over documents of the given lengths (packed in this order) for
 * n_workers CP workers and a target workload ratio R = max / mean >= 1.
 * Documents stay whole (Whole-Doc sharding, section 3.3) and are cut only to
 * equalise token counts (Eq. 2), head first; while the ratio exceeds R the
 * longest remaining document switches to Per-Doc sharding (pieces i and
 * 2N-1-i of 2N, section 2.3).  Shard workload W = (2p + s + 1) s / 2
 * (section 3.1).  The pages leave two steps open; this library reads them
 * as: a worker above its token target gives back its most recently added
 * shards, and each goes to the least-loaded worker below its target, as
 * much of its head as that worker lacks, the rest onward (ties always to the
 * lowest worker index).
 * Outputs: chunks = every worker's chunk list (global positions, ascending,
 * adjacent shards joined) concatenated in worker order, worker_n_chunks[j]
 * entries for worker j; per_doc (capacity n_docs, may be NULL) = ids of the
 * Per-Doc documents, ascending, *n_per_doc of them; *ratio = the plan's
 * workload ratio.  chunks = NULL only reports the counts; max_chunks below
 * their sum is DOCMASK_EINVAL. */
int docmask_plan_shards(const int32_t* doc_lengths, int32_t n_docs, int32_t n_workers, double target_ratio,
                        docmask_chunk* chunks, int32_t max_chunks, int32_t* worker_n_chunks, int32_t* per_doc,
                        int32_t* n_per_doc, double* ratio);

/* Send side, host only.  For one worker's chunk list (ascending, disjoint,
 * inside the sequence) and host cu_seqlens, the maps from its local KV rows
 * (chunks concatenated) to the packed send buffer, in local order, coalesced
 * where rows are contiguous in both; *send_rows = rows sent (the worker's
 * term of Eq. 5's maximum).  maps = NULL only reports *n_maps and
 * *send_rows; otherwise max_maps < *n_maps is DOCMASK_EINVAL. */
int docmask_exchange_send_maps(const int32_t* cu_seqlens, int32_t n_docs, const docmask_chunk* chunks,
                               int32_t n_chunks, docmask_rowmap* maps, int32_t max_maps, int32_t* n_maps,
                               int64_t* send_rows);

/* Receive side, host only.  all_chunks holds every worker's chunk list in
 * worker order (worker k's rank_n_chunks[k] entries); together they must
 * cover [0, cu_seqlens[n_docs]) exactly once (each token on one worker).  The
 * gathered buffer holds worker k's packed rows at rows [k * slot_rows, ...);
 * slot_rows must be at least every worker's send_rows.  For worker `rank`:
 * *kv_lo, *kv_hi = the KV range its chunks need (the document start of each
 * chunk's first row up to the chunk end; 0, 0 without rows); `remote` = maps
 * from the gathered buffer to rows of [kv_lo, kv_hi) (position - kv_lo),
 * covering exactly the other workers' sent rows inside the need intervals,
 * plus zero runs (src = -1), sorted by dst; `local` = maps from the worker's
 * local KV rows to the same destination (one per non-empty chunk).  Copying
 * `remote` and `local` (no zero_gaps) writes every row an allowed pair can
 * reach, and zeros over the other rows of each 128-row block (counted from
 * kv_lo) that holds such a row: the attention entry points read KV in whole
 * tiles of at most 128 rows from kv_lo, so the rest of [kv_lo, kv_hi) is
 * never read and stays untouched.  NULL map arrays only report counts;
 * capacities below the counts are DOCMASK_EINVAL. */
int docmask_exchange_recv_maps(const int32_t* cu_seqlens, int32_t n_docs, const docmask_chunk* all_chunks,
                               const int32_t* rank_n_chunks, int32_t n_ranks, int32_t rank, int64_t slot_rows,
                               int32_t* kv_lo, int32_t* kv_hi, docmask_rowmap* remote, int32_t max_remote,
                               int32_t* n_remote, docmask_rowmap* local, int32_t max_local, int32_t* n_local);

/* Kernel timing (instrumentation; defines no attention operation).
 * While enabled, every kernel launch of the library is bracketed by two HIP
 * events recorded on the launch stream, and their elapsed times are summed
 * per kernel class.  No work is skipped or reordered; the only cost is the
 * event records.  docmask_timing_enable(1) clears the totals and starts
 * recording, docmask_timing_enable(0) stops it.  docmask_timing_read waits
 * for every recorded pair, then returns the summed milliseconds and launch
 * count of one class since the last enable; DOCMASK_EINVAL for an unknown
 * class or null output, DOCMASK_EHIP if an event query failed.  The
 * schedule class covers the whole tile-scheduler build of one call (its five
 * small kernels).  Process-wide, thread-safe; the event pool lives until the
 * process ends. */
enum {
  DOCMASK_KERNEL_SCHEDULE = 0,
  DOCMASK_KERNEL_FWD = 1,
  DOCMASK_KERNEL_DELTA = 2,     /* never launched: Delta is formed inside the dQ kernel */
  DOCMASK_KERNEL_DKDV = 3,
  DOCMASK_KERNEL_DQ = 4,
  DOCMASK_KERNEL_MERGE = 5,
  DOCMASK_KERNEL_CONVERT = 6,
  DOCMASK_KERNEL_COPY = 7,      /* docmask_copy_rows */
  DOCMASK_KERNEL_HEAD = 8,      /* the backward's fp32 pass over pairs at document starts */
  DOCMASK_N_KERNEL_CLASSES = 9
};
int docmask_timing_enable(int enable);
int docmask_timing_read(int kernel_class, double* total_ms, int64_t* launches);
const char* docmask_kernel_class_name(int kernel_class);

/* Matrix-core rate probe (instrumentation; defines no attention operation).
 * Measures what the matrix cores sustain on given bf16 data: n_workgroups
 * workgroups of 4 waves (at most two resident per compute unit) each run `iters`
 * iterations of back-to-back bf16 MFMAs on operands held in registers, with no
 * other memory traffic.  shape 32: 16 v_mfma_f32_32x32x16_bf16 per iteration
 * (the dK/dV kernel's instruction) into accumulator k mod 4; shape 16: 32
 * v_mfma_f32_16x16x32_bf16 (the forward's and the dQ kernel's) into
 * accumulator k mod 8; the same 2^19 products per wave and iteration.  Lane
 * gl (global thread index) loads its 8 A and 8 B operand registers once, 8
 * bf16 values each, from `operands` (device, n_operands values, 16-byte
 * aligned): A slot j at (128 gl + 8 j) mod n_operands, B slot j at (128 gl +
 * 64 + 8 j) mod n_operands; MFMA k of an iteration multiplies A slot k mod 8
 * by B slot 3k mod 8.  Operand layouts: 32 x 16 A, lane l holds row l mod 32,
 * columns 8 (l / 32) .. +8, and 16 x 32 B, column l mod 32, rows 8 (l / 32)
 * .. +8 (shape 32); 16 x 32 A, row l mod 16, columns 8 (l / 16) .. +8, and
 * 32 x 16 B, column l mod 16, rows 8 (l / 16) .. +8 (shape 16).  Each lane
 * writes the sum of its accumulator elements to out[gl] (device float, 256
 * n_workgroups entries).  Work per call: 32768 * 16 * iters * 4 *
 * n_workgroups flop.  Asynchronous on `stream`; DOCMASK_EINVAL for null or
 * misaligned pointers, n_operands < 128 or not a multiple of 8, n_workgroups
 * < 1, iters < 0, a shape other than 32 or 16. */
int docmask_mfma_probe(const void* operands, int64_t n_operands, int32_t n_workgroups, int32_t iters, int32_t shape,
                       float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DOCMASK_H */
