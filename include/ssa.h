/*
 * ssa.h - C ABI of the SSA dual-stream block-sparse attention (forward and
 * backward) for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the method is described on the pages on SSA,
 * "Sparse Sparse Attention"):
 *   - "SSA: Achieving Sparser Attention by Aligning Full and Sparse Attention
 *     Outputs in Feature Space" (xugj520.cn), section "Practical
 *     Implementation of SSA": the sequence is cut into blocks, each block is
 *     mean-pooled, the query is scored against the earlier block
 *     representations, the top-k blocks are kept and attention runs over
 *     their tokens only;
 *   - same page, "SSA's Dual-Stream Training Mechanism" and "Bidirectional
 *     Attention Alignment": a full and a sparse attention stream per layer,
 *     compared by the sparsity loss ||a_full - sg[a_sparse]|| and the
 *     commitment loss ||a_sparse - sg[a_full]||;
 *   - "Technische Samenvatting: SSA (Sparse Sparse Attention)"
 *     (gist.science), "2. Methodologie": the counterpart output per layer and
 *     the dropped attention mass delta(t).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, on the device: Q [B,Hq,Nq,D],
 *     K and V [B,Hkv,Nk,D], outputs [B,Hq,Nq,D]. Query i sits at key
 *     position Nk - Nq + i. Prefill has Nq == Nk; decode has Nq == 1.
 *   - Element type: SSA_BF16 (bfloat16) or SSA_F32 for Q, K, V and the two
 *     attention outputs. delta, lse, pooled vectors and losses are float32.
 *   - Supported (else SSA_ERR_UNSUPPORTED): D in {64, 128}; block_size 64,
 *     or 16 with SSA_BF16; Nk a multiple of 64 with at most 4096 blocks;
 *     Nq in {Nk, 1}; Hq <= 256; Hq/Hkv <= 16.
 *   - Ownership: the caller owns every buffer; the library never allocates
 *     device or host memory. Scratch memory is the caller's workspace of
 *     ssa_workspace_bytes() bytes (ssa_bwd_workspace_bytes() for the
 *     backward; device memory, 256-byte aligned). The one exception is
 *     ssa_align_loss_noalloc, whose 8 KiB of partial sums are a static
 *     device array of the library (one per GPU, loaded with the library).
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream). Every call only enqueues kernels on it and returns without
 *     synchronising. Calls are reentrant; calls that share a workspace must
 *     be ordered on one stream.
 *   - Errors: all validation happens on the host before any launch; a
 *     failing call enqueues nothing (except SSA_ERR_HIP, reported from the
 *     launch itself). No call aborts or throws. ssa_last_error_message()
 *     gives the thread's last error text. Non-finite inputs give unspecified
 *     outputs (they are not checked).
 */
#ifndef SSA_H
#define SSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSA_OK = 0,
  SSA_ERR_INVALID_ARG = 1,  /* null pointer, inconsistent shape or head map,
                               budget below the forced blocks, sizes <= 0 */
  SSA_ERR_UNSUPPORTED = 2,  /* a valid problem outside the supported set */
  SSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than needed */
  SSA_ERR_HIP = 4           /* a HIP runtime error while launching */
} ssa_status;

typedef enum { SSA_F32 = 0, SSA_BF16 = 1 } ssa_dtype;

/* Block selection granularity (ssa_problem.selection).
 *   SSA_SELECT_PER_HEAD : one list per (b, q head, query block)
 *   SSA_SELECT_GROUP    : one list per (b, kv head, query block), given to
 *                         every q head of that GQA group; a key block's group
 *                         score is the sum of its q heads' scores (float64,
 *                         q heads in ascending index order). The pages select
 *                         per query ("Practical Implementation of SSA"); the
 *                         group reading lets a GQA group share one list.
 *   SSA_SELECT_TOKEN    : one list per (b, q head, query row): each row
 *                         scores its own query vector (as float32) against
 *                         the pooled key blocks, the page's q Mean(K)^T for
 *                         a single query; candidates and forced blocks are
 *                         those of the block holding the row. idx is then
 *                         [B,Hq,Nq,budget] and cnt [B,Hq,Nq]; budget <= 64.
 *                         In decode (Nq == 1) it is SSA_SELECT_PER_HEAD. */
typedef enum {
  SSA_SELECT_PER_HEAD = 0,
  SSA_SELECT_GROUP = 1,
  SSA_SELECT_TOKEN = 2
} ssa_selection;

/* One attention problem (one layer's attention of one batch).
 *   B, Hq, Hkv : batch, query heads, key/value heads (Hq % Hkv == 0)
 *   Nq, Nk     : query rows and key positions per head
 *   D          : head dimension
 *   block_size : tokens per key block and query rows per query block
 *   budget     : selected key blocks per row, forced blocks included
 *   n_sink     : leading blocks always kept ("sink")
 *   n_local    : blocks ending at the query's own block always kept ("local")
 *   scale      : attention logit scale; 0 means 1/sqrt(D)
 *   dtype      : ssa_dtype of Q, K, V and the attention outputs
 *   head_map   : host array [Hq] giving the kv head of each q head, or NULL
 *                for h / (Hq/Hkv); every kv head must receive exactly Hq/Hkv
 *                q heads. Read during the call only.
 *   selection  : ssa_selection; SSA_SELECT_PER_HEAD (0) unless set */
typedef struct {
  int32_t B, Hq, Hkv, Nq, Nk, D, block_size, budget, n_sink, n_local;
  float scale;
  int32_t dtype;
  const int32_t* head_map;
  int32_t selection;
} ssa_problem;

/* Device workspace bytes needed by every forward call below for problem p
 * (the largest of their needs, so one workspace serves them all; the
 * backward has its own query). Returns 0 when p is invalid or unsupported.
 * Besides intermediates (pooled blocks, V transposed) the workspace holds
 * the bf16 prefill's work-queue counters, which ssa_attn_fwd resets itself:
 * no part of the workspace needs clearing by the caller. */
size_t ssa_workspace_bytes(const ssa_problem* p);

/* Block mean-pool ("Practical Implementation of SSA": mean pooling of each
 * block). x is [B, H, N, D] of p->dtype on the device (N = p->Nk);
 * pooled is [B, H, N/block_size, D] float32: per block and d, the float64
 * sum of the block's tokens in ascending order, divided by block_size,
 * rounded once to float32. Used by decode callers to keep the pooled-key
 * table of a KV cache; H is the head count of x. */
ssa_status ssa_pool_blocks(const ssa_problem* p, const void* x, int32_t H,
                           float* pooled, void* stream);

/* Block selection ("Practical Implementation of SSA": similarity with every
 * earlier block representation, top-k most relevant blocks).
 *   q        : [B,Hq,Nq,D] device, p->dtype
 *   k        : [B,Hkv,Nk,D] device, p->dtype; may be NULL when k_pooled is
 *              given
 *   k_pooled : [B,Hkv,Nk/block_size,D] float32 device from ssa_pool_blocks,
 *              or NULL to pool k here
 *   idx      : out [B,Hq,nQB,budget] int32, nQB = Nq/block_size (prefill) or
 *              1 (decode); the selected key blocks of each (b, h, query
 *              block) in ascending order, padded with -1. With
 *              SSA_SELECT_TOKEN (prefill) one list per query row:
 *              [B,Hq,Nq,budget]
 *   cnt      : out [B,Hq,nQB] int32 ([B,Hq,Nq] per token), the number of
 *              valid idx entries
 * The query block's representation is its mean-pooled Q (decode, and every
 * row with SSA_SELECT_TOKEN: the query itself, as float32). Scores are float64 dot products of the float32 pooled vectors,
 * summed over d in ascending order, unscaled. With p->selection ==
 * SSA_SELECT_GROUP every q head of a GQA group receives the group's list,
 * ranked by the float64 sum of the heads' scores (ascending q head order). Forced blocks (the first
 * n_sink blocks and the n_local blocks ending at the query's own block) are
 * always kept; the remaining budget goes to the best-scoring causal blocks,
 * exact ties to the lower block index; when no more candidates than free
 * slots remain every causal block is kept. */
ssa_status ssa_select_blocks(const ssa_problem* p, const void* q, const void* k,
                             const float* k_pooled, int32_t* idx, int32_t* cnt,
                             void* ws, size_t ws_bytes, void* stream);

/* Dual-stream attention forward ("SSA's Dual-Stream Training Mechanism":
 * full stream over every causal key; "Practical Implementation of SSA":
 * sparse stream over the tokens of the selected blocks; "2. Methodologie":
 * the counterpart output and the dropped mass).
 *   q, k, v  : device inputs as above; idx, cnt from ssa_select_blocks
 *              (laid out for p->selection; with SSA_SELECT_TOKEN each row's
 *              list must be ascending, as ssa_select_blocks writes it)
 *   h_full   : out [B,Hq,Nq,D] p->dtype: softmax(scale q k^T) v over keys
 *              j <= position of the query; NULL selects sparse-only mode
 *              (only the selected blocks are read)
 *   h_sparse : out [B,Hq,Nq,D] p->dtype: the same with the softmax taken
 *              over the causal keys of the selected blocks only (required)
 *   delta    : out [B,Hq,Nq] float32 or NULL: full-softmax mass on causal
 *              keys outside the selected blocks (must be NULL when h_full is)
 *   lse      : out [2,B,Hq,Nq] float32 or NULL: natural-log log-sum-exp of
 *              the scaled logits of the full (plane 0) and sparse (plane 1)
 *              streams; plane 0 is left untouched in sparse-only mode
 * The float32 accumulators are rounded once to the output type. */
ssa_status ssa_attn_fwd(const ssa_problem* p, const void* q, const void* k,
                        const void* v, const int32_t* idx, const int32_t* cnt,
                        void* h_full, void* h_sparse, float* delta, float* lse,
                        void* ws, size_t ws_bytes, void* stream);

/* Alignment losses ("Bidirectional Attention Alignment"), read as mean
 * squared errors over all B*Hq*Nq*D elements.
 *   h_full, h_sparse : device inputs [B,Hq,Nq,D] p->dtype
 *   loss             : out device float32[2] = {L_sparsity, L_commitment};
 *                      both forward values are mean((h_full - h_sparse)^2),
 *                      reduced deterministically from float64 partials
 *   grad_full        : out [B,Hq,Nq,D] p->dtype or NULL:
 *                      dL_sparsity/dh_full = 2 (h_full - h_sparse) / n
 *   grad_sparse      : out [B,Hq,Nq,D] p->dtype or NULL:
 *                      dL_commitment/dh_sparse = 2 (h_sparse - h_full) / n
 * (the stop-gradient side of each loss receives no gradient). */
ssa_status ssa_align_loss(const ssa_problem* p, const void* h_full,
                          const void* h_sparse, float* loss, void* grad_full,
                          void* grad_sparse, void* ws, size_t ws_bytes,
                          void* stream);

/* ssa_align_loss for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, results and arguments without the workspace. The
 * float64 partial sums live in a static device array of the library, 8 KiB
 * on each GPU that loads it (1024 partials, enough for any problem size),
 * held until the process ends; its address is looked up on the first call
 * on each device. Nothing is allocated and nothing needs clearing (every
 * partial is written before it is read). Calls on one GPU share that array:
 * calls that may overlap on one GPU (on different streams, or from different
 * threads) race and must be serialised by the caller.
 * Errors: as ssa_align_loss; SSA_ERR_HIP if the stream's device cannot be
 * found, SSA_ERR_UNSUPPORTED for a device index of 64 or more. */
ssa_status ssa_align_loss_noalloc(const ssa_problem* p, const void* h_full,
                                  const void* h_sparse, float* loss,
                                  void* grad_full, void* grad_sparse,
                                  void* stream);

/* Device workspace bytes needed by ssa_attn_bwd for problem p: per-row
 * statistics (16 bytes per query row) and, for SSA_BF16, the selection bits
 * of the dK/dV walk (2 bytes per q head, 128-key tile and 32-row step; 32
 * more with SSA_SELECT_TOKEN, the row masks of the four 32-key blocks),
 * a float32 copy of dQ (the full-stream pass hands its partial sums to the
 * sparse-stream pass), float32 copies of dK and dV for each head group of
 * the full-stream pass (one group, or up to Hq/Hkv when there are fewer than
 * 4096 pairs of 128-key tile and kv head) and Hq/Hkv float32 copies of dK
 * and dV (one per q head of a group for the sparse pass). Returns 0 when p
 * is invalid, unsupported or a decode problem. */
size_t ssa_bwd_workspace_bytes(const ssa_problem* p);

/* Backward pass of both attention streams ("Bidirectional Attention
 * Alignment": the stop-gradient sends the sparsity loss's gradient to
 * h_full only and the commitment loss's to h_sparse only; "2. Methodologie":
 * the auxiliary output is not passed to later layers). The caller adds the
 * task-loss gradient of the primary stream and alpha times the alignment
 * seeds of ssa_align_loss into one upstream gradient per stream; this call
 * returns the gradients of sum(d_full * h_full) + sum(d_sparse * h_sparse)
 * with the block selection held fixed (top-k passes no gradient):
 *   dV = P_f^T d_full + P_s^T d_sparse,
 *   dS = P_f * (d_full V^T - rowsum(d_full * h_full))
 *      + P_s * (d_sparse V^T - rowsum(d_sparse * h_sparse)),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * with P_f, P_s recomputed from the forward's log-sum-exp.
 *   q, k, v      : the forward's inputs; idx, cnt its selection
 *   h_full       : [B,Hq,Nq,D] p->dtype, the forward's output (needed when
 *                  d_full is given)
 *   h_sparse     : [B,Hq,Nq,D] p->dtype (needed when d_sparse is given)
 *   lse          : [2,B,Hq,Nq] float32 from ssa_attn_fwd (plane 0 read when
 *                  d_full is given, plane 1 when d_sparse is)
 *   d_full       : [B,Hq,Nq,D] p->dtype, dL/dh_full, or NULL for zero
 *   d_sparse     : [B,Hq,Nq,D] p->dtype, dL/dh_sparse, or NULL for zero;
 *                  not both NULL. With d_full NULL only the selected blocks
 *                  are visited.
 *   dq           : out [B,Hq,Nq,D] p->dtype
 *   dk, dv       : out [B,Hkv,Nk,D] p->dtype, each kv head summed over its
 *                  q heads (deterministic: no atomics)
 *   ws, ws_bytes : at least ssa_bwd_workspace_bytes(p) bytes
 * Prefill problems only (Nq == Nk; decode gives SSA_ERR_UNSUPPORTED).
 * With SSA_SELECT_TOKEN each row's own list selects its sparse keys.
 * float32 accumulation; P and dS enter the bf16 products rounded to bf16;
 * outputs are rounded once. */
ssa_status ssa_attn_bwd(const ssa_problem* p, const void* q, const void* k,
                        const void* v, const int32_t* idx, const int32_t* cnt,
                        const void* h_full, const void* h_sparse,
                        const float* lse, const void* d_full,
                        const void* d_sparse, void* dq, void* dk, void* dv,
                        void* ws, size_t ws_bytes, void* stream);

/* Measurement hook, for callers that time the attention kernel of a prefill
 * call on its own (a benchmark's roofline): while set, every bf16 prefill
 * ssa_attn_fwd records `start` on its stream immediately before launching
 * the attention kernel and `stop` immediately after it, so that the pair
 * brackets that one kernel and not the V transpose launched before it.
 *   start, stop : hipEvent_t handles (passed as void*), created and owned by
 *                 the caller, both non-NULL; NULL, NULL clears the hook
 * The setting is process-wide and not synchronised: set it from the thread
 * that issues the calls, with no call in flight on another thread. Decode and
 * float32 calls ignore it. Errors: SSA_ERR_INVALID_ARG when exactly one of
 * the two is NULL (the previous setting is kept). */
ssa_status ssa_set_attn_timing_events(void* start, void* stop);

/* Static text of a status code. */
const char* ssa_status_string(ssa_status s);

/* Text of the calling thread's last error (empty if none). */
const char* ssa_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H */
