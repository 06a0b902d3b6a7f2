/*
 * spava.h -- C ABI of the approximate-attention prefill library (gfx950).
 *
 * The library computes one transformer layer's prefill attention the way
 * "Spava / APB-V: Accelerating Long-Video Understanding via
 * Sequence-Parallelism-aware Approximate Attention" describes it, with all
 * virtual hosts' context blocks on one GPU:
 *
 *   token rows  = [ anchor (la) | block 0 (L) | ... | block V-1 (L) | query (n_q) ]
 *                 (Figure 2 caption: B_a, B^(h), B_qr)
 *   1. spava_score_topk      score every key of every block by the query
 *                            block's attention and keep the top lp per block
 *                            and KV head (Figure 5 caption; review "What
 *                            carries the argument"; ledger axiom on ArgTop_lp)
 *      spava_score_topk_context  the same with the block's own tokens as the
 *                            scorers (review, Referee Report, major comment
 *                            1); spava_kv_overlap compares two selections
 *   2. spava_gather_passing  copy the kept K,V rows into passing blocks
 *                            (Figure 2 caption: blocks compressed, then passed)
 *   3. spava_attn_fwd        anchor and context tokens attend over anchor +
 *                            earlier hosts' passing blocks + own block
 *                            (review "Core claim"; Referee Report, Eq. (4));
 *                            query tokens produce one partial per key group in
 *                            the same pass (Figure 3 caption: fused context
 *                            and query forward)
 *   4. spava_lse_merge       merge the query partials through their
 *                            log-sum-exp (ledger axiom: Eq. 5, Appendix A)
 *
 * Conventions shared by every call
 *   - Pointers named q, k, v, kp, vp, o, lse, o_part, lse_part, scores, idx
 *     and ws are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises; every call only enqueues work on
 *     `stream` (a hipStream_t; NULL = the null stream) and returns.
 *   - Tensors are row-major in the layouts stated below and must be 16-byte
 *     aligned.  Outputs are always dense; q, k and v follow the plan's
 *     strides (dense when they are 0).
 *   - Return value: SPAVA_OK or an error code.  Argument checks run on the
 *     host before anything is enqueued; on an error nothing is enqueued and
 *     spava_last_error() (per thread) describes it.  A launch failure
 *     returns SPAVA_ELAUNCH.
 *   - Identical inputs give bitwise-identical outputs (no atomics on values).
 *   - Q and K are taken after any positional encoding; none is applied.
 *   - Query head a uses KV head a / (n_q_heads / n_kv_heads).
 */
#ifndef SPAVA_H
#define SPAVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPAVA_VERSION 200

#define SPAVA_OK 0
#define SPAVA_EINVAL 1        /* null pointer, bad size, misaligned pointer   */
#define SPAVA_EUNSUPPORTED 2  /* head_dim other than 64/128, unknown dtype    */
#define SPAVA_EWORKSPACE 3    /* workspace smaller than the *_ws_bytes size    */
#define SPAVA_ELAUNCH 4       /* a kernel launch failed                        */

#define SPAVA_BF16 0          /* bfloat16 inputs, float32 arithmetic           */
#define SPAVA_F32 1           /* float32 inputs, float32 arithmetic            */

#define SPAVA_PHASE_ALL 0     /* spava_attn_fwd_phase: every row               */
#define SPAVA_PHASE_LOCAL 1   /* rows that read no passing block               */
#define SPAVA_PHASE_PASSING 2 /* context rows of hosts 1..V-1                  */

/*
 * One layer's sequence split (Figure 2 caption) and head geometry.
 *   n_anchor   la  >= 0   anchor tokens (first la rows)
 *   n_hosts    V   >= 1   virtual hosts (context blocks)
 *   host_len   L   >= 1   tokens per context block
 *   n_query    n_q >= 0   query-block tokens (last n_q rows)
 *   n_q_heads, n_kv_heads  Hq % Hkv == 0
 *   head_dim   d   64 or 128
 *   lp             passing length, 0 <= lp <= L
 *   dtype          SPAVA_BF16 or SPAVA_F32 (element type of q,k,v,kp,vp,o)
 *   scale          softmax scale; 0 means 1/sqrt(d)
 *   q_stride_tok, q_stride_head    element strides of q between tokens and
 *   kv_stride_tok, kv_stride_head  between heads (k and v share theirs);
 *                  channels are contiguous.  0 means the dense layout
 *                  (Hq*d, d and Hkv*d, d), so a zero-initialised plan tail
 *                  keeps the dense tensors below.  Each stride must be a
 *                  multiple of 16 bytes / element size (rows stay 16-byte
 *                  aligned), and each token stride at least d (a token's
 *                  channels end before the next token's start) and below
 *                  2^24 bytes; a packed QKV projection output [N][Hq+2Hkv][d]
 *                  is q = qkv, k = qkv + Hq*d, v = qkv + (Hq+Hkv)*d with
 *                  token strides (Hq+2Hkv)*d and head strides d.
 * N = la + V*L + n_q rows in total; N * max(Hq, Hkv) * d must be < 2^31, and
 * so must the element extent of q and of k/v under their strides.  The
 * outputs (o, kp, vp, partials) are always dense.
 */
typedef struct spava_plan {
  int32_t n_anchor;
  int32_t n_hosts;
  int32_t host_len;
  int32_t n_query;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t lp;
  int32_t dtype;
  float scale;
  int64_t q_stride_tok;
  int64_t q_stride_head;
  int64_t kv_stride_tok;
  int64_t kv_stride_head;
} spava_plan;

/* SPAVA_VERSION of the built library. */
int spava_version(void);

/* Text of the last error raised on the calling thread ("" if none). */
const char* spava_last_error(void);

/* Host-only check of a plan; returns SPAVA_OK or the code a call would. */
int spava_plan_check(const spava_plan* plan);

/*
 * Workspace bytes spava_score_topk needs for the query rows' softmax
 * normalisers over each block, rounded up to 256: float32 plans keep one
 * log-sum-exp per row, float32 [V][Hkv][n_q*G]; bf16 plans keep a (max, sum)
 * pair per row and key chunk of the block, float32 [C][V][Hkv][n_q*G][2]
 * with C = ceil(L/512) for L <= 8192 (chunks of 512 keys), else
 * C = ceil(T / ceil(T/16)) with T = ceil(L/64) (at most 16 chunks).  Then,
 * from the next 256-byte boundary, room for float32 [V][Hkv][L] scores (used
 * when the caller passes scores = NULL; a caller that passes scores may
 * provide a workspace without it).
 */
size_t spava_score_topk_ws_bytes(const spava_plan* plan);

/*
 * Step 1: block scores and top-lp selection.
 * Scoring rule (Figure 5 caption: query logits Q_qr K^(h)T rank block h): for
 * block h and KV head g,
 *     scores[h][g][j] = sum over query tokens i and query heads a of group g
 *                       of softmax_j( q[la+V*L+i][a] . k[la+h*L+j][g] * scale )
 * with the softmax over the L keys of block h only.  Selection (ledger axiom:
 * ArgTop_lp): the lp indices first in the order (score descending, index
 * ascending), written in ascending order.
 *   q       [N][Hq][d]      dtype (plan strides)
 *   k       [N][Hkv][d]     dtype (plan strides)
 *   scores  [V][Hkv][L]     float32, written (also useful as a diagnostic);
 *                           may be NULL: the scores then live in ws
 *   idx     [V][Hkv][lp]    int32 block-local key indices, written
 *   ws      >= spava_score_topk_ws_bytes(plan) bytes of scratch
 * With n_q == 0 every score is 0 and idx = 0..lp-1.
 */
int spava_score_topk(const spava_plan* plan, const void* q, const void* k,
                     float* scores, int32_t* idx, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * Step 1 for callers that cannot allocate (code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it): the
 * same scores and selection as spava_score_topk, bit for bit, with the
 * workspace taken from a static device array of SPAVA_NOALLOC_SCRATCH_BYTES
 * inside the library instead of a caller buffer.  Calls no hipMalloc,
 * hipFree or allocating library routine.
 *   q, k, scores, idx   as spava_score_topk (scores may be NULL: the scores
 *                       then live in the static scratch too)
 * Errors as spava_score_topk; SPAVA_EWORKSPACE when the plan needs more than
 * SPAVA_NOALLOC_SCRATCH_BYTES (the size spava_score_topk_ws_bytes reports,
 * less the scores' room when scores is not NULL), checked on the host before
 * anything is enqueued.  Each GPU holds one copy of the array (64 MiB) from
 * the first call on it until the process ends.  Every call on one GPU shares
 * that copy: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  Nothing in the scratch needs
 * to start at zero (every byte read is written earlier in the same call).
 */
#define SPAVA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int spava_score_topk_noalloc(const spava_plan* plan, const void* q,
                             const void* k, float* scores, int32_t* idx,
                             void* stream);

/*
 * Workspace bytes spava_score_topk_context needs: as spava_score_topk_ws_bytes
 * with the block's L tokens as the scoring rows, float32 [V][Hkv][L*G] for
 * float32 plans and float32 [V][Hkv][L*G][2] (one key chunk) for bf16 plans;
 * bf16 plans
 * add (from the next 256-byte boundary) float32 [Z][V][Hkv][L] column sums of
 * Z = G * ceil(L / S) row splits, S = max(1024, 32 * ceil(ceil(L/8) / 32))
 * tokens each, when Z > 1.
 */
size_t spava_score_topk_context_ws_bytes(const spava_plan* plan);

/*
 * Context-driven selection: the alternative the APB-V review's Referee
 * Report (major comment 1) asks to compare against -- a block's own tokens,
 * not the query block, decide which of its keys are passed on.  For block h
 * and KV head g,
 *     scores[h][g][j] = sum over block tokens t >= j and query heads a of
 *                       group g of softmax_{j' <= t}( q[la+h*L+t][a] .
 *                       k[la+h*L+j'][g] * scale )
 * i.e. every token attends causally over its own block (diagonal included)
 * and the probabilities it gives each key are summed.  Selection, layouts,
 * alignment and errors as spava_score_topk; ws >=
 * spava_score_topk_context_ws_bytes(plan).  L * (n_q_heads / n_kv_heads)
 * must be below 2^31.  Costs about one causal attention pass per block
 * (two MFMA passes over its L x L logits), against the L x n_q logits of the
 * query-driven rule.
 */
int spava_score_topk_context(const spava_plan* plan, const void* q,
                             const void* k, float* scores, int32_t* idx,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Overlap of two selections (APB-V review, "What would settle it": how many
 * of the query-selected keys the context-driven rule also selects).
 *   idx_a, idx_b  [n_lists][lp] int32, each list strictly ascending (as
 *                 spava_score_topk and spava_score_topk_context write them)
 *   counts        [n_lists] int32, written: |a_i intersect b_i|, or -1 for
 *                 a list pair where either list is not strictly ascending
 * n_lists = V * Hkv for the outputs of the two selectors.  Pointers are
 * device pointers, 4-byte aligned; n_lists * lp must be below 2^31.
 */
int spava_kv_overlap(int32_t n_lists, int32_t lp, const int32_t* idx_a,
                     const int32_t* idx_b, int32_t* counts, void* stream);

/*
 * Step 2: passing blocks (Figure 2 caption).
 *   kp[g][h][t][:] = k[la + h*L + idx[h][g][t]][g][:]
 *   vp[g][h][t][:] = v[la + h*L + idx[h][g][t]][g][:]
 *   k, v    [N][Hkv][d]        dtype
 *   idx     [V][Hkv][lp]       int32, each in [0, L) (not checked on device;
 *                              an out-of-range index is clamped into the block)
 *   kp, vp  [Hkv][V][lp][d]    dtype, written
 * kp/vp may be reused once the stream has passed spava_attn_fwd (the pages
 * discard passing blocks right after attention).
 */
int spava_gather_passing(const spava_plan* plan, const void* k, const void* v,
                         const int32_t* idx, void* kp, void* vp, void* stream);

/*
 * Step 3: fused approximate attention forward (Figure 3 caption; review
 * "Core claim"; Referee Report, Eq. (4) key list [K_a, K_p, K^(h)]).
 *   anchor token t < la:           keys 0..t                       (causal)
 *   context token t of host h:     keys anchor, kp/vp[g][0..h-1],
 *                                  own block rows <= t              (causal)
 *   query partial 0:               keys anchor, query rows <= t     (causal)
 *   query partial h+1:             keys of block h                  (all)
 * Softmax with the plan's scale; LSE is the natural log of the sum of
 * exp(scaled logits).
 *   q [N][Hq][d]; k, v [N][Hkv][d]; kp, vp [Hkv][V][lp][d]      dtype
 *   o         [N][Hq][d]          dtype; rows [0, la+V*L) written
 *   lse       [Hq][N]             float32; columns [0, la+V*L) written
 *   o_part    [V+1][n_q][Hq][d]   float32, written (may be NULL if n_q == 0)
 *   lse_part  [V+1][Hq][n_q]      float32, written (may be NULL if n_q == 0)
 * No workspace: K and V tiles are read straight from k, v, kp, vp.
 * Dense causal attention is the plan {la=0, V=1, L=N, n_q=0, lp=0}
 * (one host degrades to standard attention).
 */
int spava_attn_fwd(const spava_plan* plan, const void* q, const void* k,
                   const void* v, const void* kp, const void* vp, void* o,
                   float* lse, float* o_part, float* lse_part, void* stream);

/*
 * Step 3 in two phases, for the ordering of the Spava page's Figure 5 (the
 * query block's attention over block h comes first and its Q_qr K^(h)T is
 * reused to score block h).  Arguments, layouts and results as
 * spava_attn_fwd; the union of the two phases writes exactly what one
 * spava_attn_fwd call writes, bit for bit.
 *   SPAVA_PHASE_LOCAL    anchor rows, context rows of host 0 and the query
 *                        partials o_part/lse_part (no passing block is read:
 *                        kp, vp may be NULL).
 *   SPAVA_PHASE_PASSING  context rows of hosts 1..V-1 (o_part, lse_part are
 *                        not touched and may be NULL).
 *   SPAVA_PHASE_ALL      the same as spava_attn_fwd.
 * The order of calls is then: spava_attn_fwd_phase(LOCAL) ->
 * spava_score_topk_from_partials -> spava_gather_passing ->
 * spava_attn_fwd_phase(PASSING) -> spava_lse_merge.
 */
int spava_attn_fwd_phase(const spava_plan* plan, int32_t phase, const void* q,
                         const void* k, const void* v, const void* kp,
                         const void* vp, void* o, float* lse, float* o_part,
                         float* lse_part, void* stream);

/*
 * Step 1 after spava_attn_fwd_phase(LOCAL): the same scores and selection as
 * spava_score_topk, with each query row's softmax normaliser over block h
 * taken from the query partial over block h (lse_part[h+1], natural log)
 * instead of a separate pass (Figure 5 caption: Q_qr K^(h)T serves both the
 * query partial and the scoring).  No workspace.
 *   lse_part  [V+1][Hq][n_q] float32 as spava_attn_fwd_phase(LOCAL) wrote it
 *             (may be NULL when n_q == 0)
 * Other arguments, layouts, alignment and errors as spava_score_topk.
 */
int spava_score_topk_from_partials(const spava_plan* plan, const void* q,
                                   const void* k, const float* lse_part,
                                   float* scores, int32_t* idx, void* stream);

/*
 * Step 4: log-sum-exp merge of partial attention results (ledger axiom,
 * Eq. 5 / Appendix A).  For row r, head a:
 *     m   = max_p lse_part[p][a][r]
 *     w_p = exp(lse_part[p][a][r] - m)
 *     o[r*o_row_stride + a*head_dim + c] = sum_p w_p o_part[p][r][a][c] / sum_p w_p
 *     lse[a*lse_head_stride + r]          = m + log(sum_p w_p)
 * If every partial has lse = -inf the row gets o = 0 and lse = -inf.
 *   o_part    [n_parts][n_rows][n_heads][head_dim]  float32
 *   lse_part  [n_parts][n_heads][n_rows]            float32
 *   o         out_dtype (SPAVA_BF16 or SPAVA_F32), strided as above
 *   lse       float32, strided as above
 * For the query rows of spava_attn_fwd: n_parts = V+1, n_rows = n_q,
 * o = o + (la+V*L)*Hq*d with o_row_stride = Hq*d, lse = lse + (la+V*L) with
 * lse_head_stride = N.
 */
int spava_lse_merge(int32_t n_parts, int32_t n_rows, int32_t n_heads,
                    int32_t head_dim, const float* o_part, const float* lse_part,
                    void* o, int64_t o_row_stride, float* lse,
                    int64_t lse_head_stride, int32_t out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPAVA_H */
