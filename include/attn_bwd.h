/*
 * attn_bwd.h -- attention backward (dQ, dK, dV) on AMD Instinct MI355X (gfx950).
 *
 * Two forms of the same backward pass over variable-length TND batches with
 * grouped-query attention:
 *
 *   dense    -- page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section:
 *               Y = Softmax(Mask(Q K^T * scale)) V with Q = [query, queryRope] and
 *               K = [key, keyRope] concatenated on the head dimension;
 *               dV = P^T dY, dQ = dS K * scale, dqRope = dS kRope * scale,
 *               dK = dS^T Q * scale, dkRope = dS^T qRope * scale.
 *   selected -- page "NsaSelectedAttentionGrad" (README), formula section: every
 *               query token and KV head gathers selectedBlockCount blocks of
 *               selectedBlockSize key/value rows through topkIndices
 *               (selectedKey = Gather(key, topkIndices[i])), then the same backward.
 *
 * dS is the softmax Jacobian applied to dP = dY V^T:  dS = P * (dP - rowsum(dY * O)),
 * where rowsum(dY * O) equals rowsum(P * dP) because O = P V (no dropout; keep_prob
 * is 1, the only value the dense page's constraints allow).
 *
 * Calling convention (both pages describe a two-phase call: a workspace-size query
 * that validates the parameters, then an execute call on a stream with a caller-
 * allocated workspace):
 *   1. attn_bwd_workspace_size(&problem, &bytes)   -- host only, validates.
 *   2. allocate `bytes` of device memory (any alignment >= 256 B).
 *   3. attn_bwd_dense_varlen(...) or attn_bwd_selected(...) on a HIP stream.
 * The problem struct is passed again at execute time; the library keeps no state
 * between calls other than a small pinned host staging ring for schedule tables.
 *
 * Layouts (all device tensors contiguous, row-major, TND = [tokens, heads, dim],
 * the rows of every sequence packed back to back with no padding):
 *   query [T1, N1, d_qk]     query_rope [T1, N1, d_rope]     dq / dq_rope likewise
 *   key   [T2, N2, d_qk]     key_rope   [T2, N2, d_rope]     dk / dk_rope likewise
 *   value [T2, N2, d_v]      out, dy    [T1, N1, d_v]        dv [T2, N2, d_v]
 *   softmax_max, softmax_sum [T1, N1, 8] float32 -- the row maximum m of the
 *       scaled, masked scores and l = sum_j exp(s_j - m); lane 0 is read.
 *   topk_indices [T1, N2, block_count] int32 -- block ids inside the token's own
 *       sequence: id selects KV rows cu_seqlens_kv[b] + id*block_size + [0, block_size).
 * Query head h uses KV head h / (N1 / N2).
 *
 * Ownership: the caller owns every device buffer, including the workspace.  The
 * library allocates no device memory.  Outputs are fully overwritten (KV rows that
 * no query attends receive 0).  Work is enqueued on `hip_stream` (NULL = default
 * stream) and returns before it completes; inputs, outputs and workspace must stay
 * valid until the stream reaches that point.  The small per-call tables (sequence
 * offsets, work lists) pass through a ring of four pinned host slots per device: the
 * first call on a device, and a call whose tables outgrow its slot, allocate pinned
 * host memory (held until the process ends); a call waits on the host only when the
 * slot it takes still serves a call four calls back that the GPU has not reached.
 *
 * Errors: every check runs before anything is enqueued; on failure nothing is
 * enqueued and no output is touched.  Out-of-range topk ids are caller errors: the
 * kernels skip such entries and raise a device-side flag that the next call on the
 * same workspace does not read (see attn_bwd_check_index_flag).
 *
 * Determinism: with deterministic = 1 the outputs are bitwise identical for
 * identical inputs, problem and device.  Both pages say the default is
 * non-deterministic and determinism can be enabled; every path behind this
 * interface is deterministic in both modes except the indexer's dK with
 * `dkdv_atomic` = 1 (see below).
 */
#ifndef ATTN_BWD_H_
#define ATTN_BWD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULLPTR = 1,      /* a required pointer is NULL                        */
  ATTN_ERR_INVALID = 2,      /* a shape / value constraint of the pages is broken */
  ATTN_ERR_UNSUPPORTED = 3,  /* valid per the pages but not built here            */
  ATTN_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than the query returned */
  ATTN_ERR_HIP = 5           /* a HIP runtime call failed                         */
} attn_status_t;

typedef enum { ATTN_BF16 = 0, ATTN_FP16 = 1, ATTN_FP32 = 2 } attn_dtype_t;
typedef enum { ATTN_OP_DENSE = 0, ATTN_OP_SELECTED = 1, ATTN_OP_SELECTED_FWD = 2, ATTN_OP_INDEXER = 3 } attn_op_t;
typedef enum { ATTN_LAYOUT_TND = 0, ATTN_LAYOUT_BSND = 1 } attn_layout_t;

typedef struct {
  int32_t op;                     /* attn_op_t                                              */
  int32_t dtype;                  /* dense: ATTN_BF16 or ATTN_FP32; selected (backward and
                                     forward): ATTN_BF16 or ATTN_FP16                         */
  int32_t batch;                  /* B >= 1                                                 */
  int32_t layout;                 /* attn_layout_t.  TND: sequences of their own lengths,
                                     given by cu_seqlens_q / cu_seqlens_kv.  BSND (selected
                                     backward and forward only; the dense page takes TND):
                                     [B, S, N, D] with every sequence seq_len_q queries and
                                     seq_len_kv keys long -- the same memory as TND with equal
                                     lengths; the cu_seqlens pointers must be NULL.          */
  const int64_t* cu_seqlens_q;    /* TND: HOST [B+1]: 0, then running sums of query lengths;
                                     a length may be 0 (dense constraints allow S = 0)     */
  const int64_t* cu_seqlens_kv;   /* TND: HOST [B+1]: same for key/value lengths           */
  int64_t seq_len_q, seq_len_kv;  /* BSND: S of query and of key / value (0 for TND)        */
  int32_t n1, n2;                 /* query / KV heads, n1 % n2 == 0                         */
  int32_t d_qk;                   /* head dim of query / key (the non-rope part)            */
  int32_t d_rope;                 /* dense: head dim of queryRope / keyRope (0 = none);
                                     selected: must be 0                                    */
  int32_t d_v;                    /* head dim of value / out / dy                           */
  double scale;                   /* scaleValue: the factor written 1/sqrt(d) on the pages  */
  int32_t causal;                 /* dense: 1 = key j visible to query i iff j <= i + off
                                     (positions within the sequence; off from mask_align);
                                     selected: 0                                            */
  int32_t mask_align;             /* dense, causal or band: 0 = off 0 (first query aligned with
                                     the first key), 1 = off S2_b - S1_b (last query aligned
                                     with the last key); the same when the lengths are equal */
  int32_t band;                   /* dense: 1 = window mask: key j visible to query i iff
                                     i + off - pre_tokens <= j <= i + off + next_tokens
                                     (excludes causal).  The dense page names sparse modes with
                                     preTokens / nextTokens; their definitions are not on it,
                                     this is the reading taken.  Rows that see no key get
                                     zero gradients.                                         */
  int64_t pre_tokens, next_tokens;/* band only (0 otherwise); |value| <= 2^30, pre + next >= 0 */
  int32_t block_size;             /* selected: selectedBlockSize (<= 128, multiple of 16)  */
  int32_t block_count;            /* selected: selectedBlockCount (1..128, count*size < 8192)*/
  int32_t deterministic;          /* 1 = bitwise reproducible                               */
  int32_t dkdv_atomic;            /* indexer: 1 = scatter dK with fp32 atomics from the
                                     query-major pass (non-deterministic, smaller workspace);
                                     0 = sum each key row's shares in a fixed order through an
                                     inverted index (faster: on the 8K / topK 2048 workload
                                     the whole call takes about half the time).  Ignored (treated as 0) when
                                     deterministic = 1.  Selected and selected-forward: reserved,
                                     1 with deterministic = 0 returns ATTN_ERR_UNSUPPORTED.
                                     Dense: must be 0.                                        */
  int32_t dense_dq_mode;          /* dense bf16 only (0 for every other problem): how dQ is
                                     formed.  1 = the KV-major pass stores dS (bf16, 8 KiB per
                                     64 x 64 (query tile, key tile) block and query head, in the
                                     workspace) and dQ = scale * dS K is a plain product;
                                     2 = dQ is recomputed query-major (S and dP formed again, no
                                     dS storage); 0 = automatic: 1 while the dS storage is at
                                     most 8 GiB, else 2.  Both give results within the same
                                     tolerance and are deterministic.                          */
  int32_t sel_window_tokens;      /* selected only (0 for dense): the backward runs over windows
                                     of at most this many consecutive query tokens, one after
                                     the other, so that the per-block dQ shares of one window
                                     (block_count * n1 * d_qk bf16 per token) fit the workspace;
                                     0 = automatic: the largest windows whose shares take at most
                                     64 GiB.  A smaller value shrinks the workspace (and costs
                                     time: each window reloads every block and carries its fp32
                                     dK / dV sums).  Any value gives results within the same
                                     tolerance; deterministic.                                  */
} attn_bwd_problem_t;

/* Validate `p` and return the workspace size in bytes for its execute call.
 * Host only; touches no device.  Returns ATTN_OK, ATTN_ERR_NULLPTR (p, bytes or a
 * cu_seqlens array is NULL), ATTN_ERR_INVALID or ATTN_ERR_UNSUPPORTED. */
attn_status_t attn_bwd_workspace_size(const attn_bwd_problem_t* p, uint64_t* bytes);

/* Dense varlen backward (page "aclnnFlashAttentionUnpaddingScoreGradV3").
 * p->op must be ATTN_OP_DENSE.  Tensors are in p->dtype (bf16 or fp32) except the
 * float32 statistics.  q_rope / k_rope / dq_rope / dk_rope must be NULL iff
 * p->d_rope == 0.  `out` is the forward output O (used for rowsum(dY * O)). */
attn_status_t attn_bwd_dense_varlen(const attn_bwd_problem_t* p,
                                    const void* q, const void* q_rope,
                                    const void* k, const void* k_rope,
                                    const void* v, const void* out, const void* dy,
                                    const float* softmax_max, const float* softmax_sum,
                                    void* dq, void* dq_rope, void* dk, void* dk_rope, void* dv,
                                    void* workspace, uint64_t workspace_bytes,
                                    void* hip_stream);

/* Size of the fixed device scratch array behind attn_bwd_dense_varlen_noalloc (64 MiB). */
#define ATTN_BWD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* attn_bwd_dense_varlen without a workspace, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, layouts and results are those of attn_bwd_dense_varlen; the workspace is a
 * fixed array of ATTN_BWD_NOALLOC_SCRATCH_BYTES in the library's device code, one per GPU,
 * held from the library's load until the process ends.  The call allocates nothing: no
 * hipMalloc / hipFree / pinned host memory and no events (the per-kernel timing of
 * attn_bwd_profiling does not see it); its schedule tables are copied from pageable host
 * memory with hipMemcpyAsync on `hip_stream`.  With dense_dq_mode = 0 it picks the stored-dS
 * mode when that plan fits the array, else the recompute mode.
 * Returns ATTN_ERR_WORKSPACE (nothing enqueued) when the problem needs more than the array
 * (the workspace-size query gives the need); the other codes as attn_bwd_dense_varlen.
 * Every call on one GPU uses the same array: calls that overlap on one GPU (other streams,
 * other host threads) race and give wrong results; calls ordered on one stream are safe. */
attn_status_t attn_bwd_dense_varlen_noalloc(const attn_bwd_problem_t* p,
                                            const void* q, const void* q_rope,
                                            const void* k, const void* k_rope,
                                            const void* v, const void* out, const void* dy,
                                            const float* softmax_max, const float* softmax_sum,
                                            void* dq, void* dq_rope, void* dk, void* dk_rope, void* dv,
                                            void* hip_stream);

/* Selected (NSA) backward (page "NsaSelectedAttentionGrad").  p->op must be
 * ATTN_OP_SELECTED, p->dtype ATTN_BF16 or ATTN_FP16 (all tensors but the float32 statistics
 * and the int32 ids in that type).  The page lists attentionOut as optional: with out == NULL
 * the row term rowsum(P * dP) is formed by an extra query-major pass over the gathered key and
 * value rows (P from the passed statistics, dP = dY V^T) instead of rowsum(dY * O); the
 * gradients are the same up to rounding. */
attn_status_t attn_bwd_selected(const attn_bwd_problem_t* p,
                                const void* q, const void* k, const void* v,
                                const void* out, const void* dy,
                                const float* softmax_max, const float* softmax_sum,
                                const int32_t* topk_indices,
                                void* dq, void* dk, void* dv,
                                void* workspace, uint64_t workspace_bytes,
                                void* hip_stream);

/* Selected (NSA) forward, the producer of the backward's attentionOut, softmaxMax and
 * softmaxSum (page "NsaSelectedAttentionGrad", parameter table: the forward's output and
 * intermediate outputs).  For every query token and KV head its G query heads attend to the
 * rows that topk_indices gathers (Gather(key, ids), Gather(value, ids), formula section):
 *   s = scale * Q K^T,  m = max s,  l = sum exp(s - m),  out = sum exp(s - m) V / l,
 * softmax_max = m and softmax_sum = l, each written to all 8 lanes of [T1, N1, 8] float32.
 * p->op must be ATTN_OP_SELECTED_FWD with the constraints of the selected backward;
 * attn_bwd_workspace_size(p) gives its (small) workspace: the sequence tables and the index
 * flag.  q [T1, N1, d_qk], k [T2, N2, d_qk], v [T2, N2, d_v], out [T1, N1, d_v] in p->dtype
 * (bf16 or fp16).  A repeated id counts twice; an out-of-range id is skipped and raises the
 * flag (attn_bwd_check_index_flag with this workspace).  A row whose ids are all out of
 * range gets out = 0, m = -inf, l = 0. */
attn_status_t attn_fwd_selected(const attn_bwd_problem_t* p,
                                const void* q, const void* k, const void* v,
                                const int32_t* topk_indices,
                                void* out, float* softmax_max, float* softmax_sum,
                                void* workspace, uint64_t workspace_bytes,
                                void* hip_stream);

/* Diagnostic: build only the inverted index of a selected problem (the first stage of
 * attn_bwd_selected) and copy it out, so that it can be checked entry by entry.
 * Keys are (KV head, block) pairs numbered kvh * NB + (blocks of the earlier sequences) + id,
 * NB = the total number of blocks over all sequences (S2_b / block_size summed).
 *   offsets [N2 * NB + 1]   key k's list is lists[offsets[k] .. offsets[k + 1])
 *   lists   [T1 * N2 * block_count]  entries t * block_count + slot, ascending within a key;
 *                           only offsets[N2 * NB] of them are written (out-of-range ids are left
 *                           out and raise the flag)
 *   order   [N2 * NB]       the keys in the order the KV-major pass takes them: by length
 *                           class, then by key.  With t_0 = the longest list's length and
 *                           t_(k+1) = floor(4 t_k / 5), the class is the least k < 31 with
 *                           length > t_(k+1), else 31; class 0 first (identity order above
 *                           8192 keys)
 * All three are device buffers owned by the caller; `workspace` as for attn_bwd_selected.
 * Asynchronous on `hip_stream`; p->op must be ATTN_OP_SELECTED. */
attn_status_t attn_bwd_selected_index(const attn_bwd_problem_t* p, const int32_t* topk_indices,
                                      int32_t* offsets, int32_t* lists, int32_t* order,
                                      void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* Lightning-indexer backward (page "aclnnLightningIndexerGrad", formula section):
 *   S = ReLU(Q . Gather(K, Indices)),  Y = dy * Weights,  dW = Reduce(S * dy),
 *   dQ = ReluGrad(Y, S) . Gather(K, Indices),  dK = ScatterAdd(ReluGrad(Y, S) . Q, Indices).
 * The page's shape table is lost in its text; the readings taken: for query token t, key
 * head n2 and the G = n1 / n2 query heads h of n2 (h / G = n2),
 *   S[t, h, k] = max(0, sum_d Q[t, h, d] K[idx, n2, d])  with idx = cu_kv[b] + indices[t, n2, k],
 *   Y[t, h, k] = dy[t, n2, k] * weights[t, h],  ReluGrad(Y, S) = Y where S > 0, else 0,
 *   dW[t, h] = sum_k S[t, h, k] dy[t, n2, k]; no scale factor.
 * p->op = ATTN_OP_INDEXER, p->dtype = ATTN_BF16, d_qk = D = 128, d_v = 0, block_size = 1,
 * block_count = topK (1 .. 128K, and every sequence with queries has at least topK keys),
 * G <= 64, B <= 1024, layout TND or BSND.  Tensors (bf16): q [T1, n1, 128], k [T2, n2, 128],
 * weights [T1, n1], dy [T1, n2, topK]; indices int32 [T1, n2, topK] (key positions inside
 * the token's sequence; a repeated index counts twice; an out-of-range one contributes
 * nothing and raises the flag of attn_bwd_check_index_flag); outputs dq [T1, n1, 128],
 * dk [T2, n2, 128], dweights [T1, n1].  dK: by default each (token, key head, slot)'s share
 * of dK is kept (rounded to bf16) and the shares of a key row are added in fp32 in ascending
 * (token, slot) order through an inverted index, over windows of query tokens whose shares
 * take at most 8 GiB (sel_window_tokens caps the window further) -- deterministic whatever
 * `deterministic` says;
 * dkdv_atomic = 1 with deterministic = 0 scatters the shares with fp32 atomics instead.
 * dQ and dW have one writer per row in every mode. */
attn_status_t attn_bwd_indexer(const attn_bwd_problem_t* p,
                               const void* q, const void* k, const void* weights, const void* dy,
                               const int32_t* indices,
                               void* dq, void* dk, void* dweights,
                               void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* Read (synchronously, on `hip_stream`) the device flag that a selected call raises
 * when it meets a topk id outside [0, S2_b / block_size).  Writes 1 to *raised when
 * the flag is set, 0 otherwise.  `workspace` is the one passed to that call. */
attn_status_t attn_bwd_check_index_flag(const attn_bwd_problem_t* p, const void* workspace,
                                        int32_t* raised, void* hip_stream);

/* Per-kernel timing, a measurement aid (off by default).  While enabled, every kernel
 * the library launches is bracketed by two HIP events on the caller's stream; no
 * synchronisation is added to the launches.  attn_bwd_profile_read synchronises on the
 * recorded events, folds them into per-kernel totals, and returns entry `index`
 * (0-based, in first-seen order): the kernel's name (static storage), total elapsed
 * milliseconds and number of launches; ATTN_ERR_INVALID when `index` is past the last
 * entry.  attn_bwd_profile_reset clears the totals.  Not thread-safe with respect to
 * concurrent calls that launch work. */
attn_status_t attn_bwd_profiling(int32_t enable);
attn_status_t attn_bwd_profile_reset(void);
attn_status_t attn_bwd_profile_read(int32_t index, const char** name, double* total_ms, int64_t* launches);

/* Short English text for a status code (static storage). */
const char* attn_bwd_status_string(attn_status_t s);

/* Library version, "major.minor.patch" (static storage). */
const char* attn_bwd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H_ */
