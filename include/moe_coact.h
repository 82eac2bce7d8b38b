/*
 * moe_coact.h -- C ABI of the co-activation-aware MoE token dispatch engine
 * (HIP, gfx950).
 *
 * The engine takes top-k router output of one MoE layer and
 *   1. counts expert co-activation (per-expert counts, E x E pair counts,
 *      Ochiai similarity, next-layer transition counts),
 *   2. builds a deduplicated dispatch plan for a given expert -> rank
 *      placement (one send row per token and destination rank),
 *   3. permutes token rows into rank-contiguous send buffers,
 *   4. combines the returned rows back to token order with the gate weights,
 *   5. predicts each token's next-layer rank and orders tokens by it (token
 *      shuffling),
 *   6. lays the received rows out per expert on the destination side,
 *   7. runs the backward mirror (scaled scatter, gate gradients),
 *   8. keeps moving averages of the statistics and plans a co-activation
 *      placement from them.
 * The ranks of the expert-parallel group are logical: each (source rank,
 * destination rank) block of the send buffer stands for one all-to-all
 * message.
 *
 * Sources (page title, section):
 *   [EC] "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead
 *        with Correlated Placement and Token Shuffling", abstract.
 *   [CB] "Cobalt: Leveraging Expert Co-activation for Efficient Distributed
 *        MoE Training", Key Observation and Problem Formulation.
 *   [CE] "Training Communication-Efficient Mixture-of-Experts Language Models
 *        with Layer Re-Configuration", footnote 3 (hidden-state dispatch,
 *        routed-probability dispatch, hidden-state combine).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  Every buffer is
 *     owned by the caller; the library allocates nothing and keeps no state
 *     between calls, so calls on different streams may run concurrently as
 *     long as their buffers differ.  The one exception is
 *     moe_dispatch_plan_noalloc, whose scratch is a fixed device array
 *     shared by all its calls on a device (see there).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns without synchronising.
 *   - The return value is a moe_status.  A negative status other than
 *     MOE_ERR_HIP means the arguments were rejected on the host and NOTHING
 *     was enqueued.  MOE_ERR_HIP means the HIP runtime reported an error
 *     right after one of the call's kernel launches (hipGetLastError, which
 *     also returns an error an earlier HIP call on this thread left behind);
 *     kernels of the call launched before it may still run.
 *   - Errors that depend on device data set bits (MOE_DERR_*) in *d_err with
 *     an atomic OR.  d_err is an int32 device word that the caller zeroes;
 *     it may be NULL (then such errors go unreported).  When a bit is set the
 *     outputs are unspecified, except as stated per bit, but no kernel reads
 *     or writes outside the buffers described here.
 *   - Index arrays are int32; T*k must stay below 2^31.
 *   - The row-moving calls (moe_permute, moe_gather, moe_shuffle_dispatch,
 *     moe_combine, moe_permute_scaled, moe_row_dot) run many blocks at once,
 *     so an output that shares bytes with an input would be read after other
 *     blocks overwrote it: they return MOE_ERR_SHAPE, launching nothing,
 *     when an output's extent (rows times row bytes) overlaps an input's.
 */
#ifndef MOE_COACT_H
#define MOE_COACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,      /* a required pointer is NULL                      */
  MOE_ERR_SHAPE = -2,     /* a size is out of range (limits below)           */
  MOE_ERR_DTYPE = -3,     /* unknown dtype code                              */
  MOE_ERR_ALIGN = -4,     /* row size or pointer alignment not supported     */
  MOE_ERR_WORKSPACE = -5, /* workspace smaller than the size query returns   */
  MOE_ERR_HIP = -6        /* a kernel launch failed                          */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Device-side error bits OR-ed into *d_err. */
#define MOE_DERR_EXPERT_RANGE 1  /* a top-k id is outside [0, E): that slot is skipped   */
#define MOE_DERR_EXPERT_DUP 2    /* a token lists one expert twice                       */
#define MOE_DERR_RANK_RANGE 4    /* a placement entry is outside [0, G): slot skipped    */
#define MOE_DERR_CAPACITY 8      /* plan: more rows than row_capacity (counters stay
                                    valid; rows >= capacity are not written)             */
#define MOE_DERR_SRC_OFFSETS 16  /* src_offsets not nondecreasing from 0 to T            */
#define MOE_DERR_ROW_RANGE 32    /* permute/combine: a row index >= the buffer's rows    */
#define MOE_DERR_SYNC 64         /* shuffle: blocks waiting on each other gave up after
                                    their bound (outputs unspecified)                    */

/* Limits checked on the host.  Besides these, the row-moving calls
   (moe_permute, moe_gather, moe_shuffle_dispatch, moe_combine,
   moe_permute_scaled, moe_row_dot) return MOE_ERR_SHAPE, launching nothing,
   when one launch would need 2^32 or more work-items (the dispatch packet
   counts them in 32 bits): roughly when rows times 16-byte row vectors
   reach 2^32, i.e. inputs of several tens of GB. */
#define MOE_MAX_K 8      /* experts per token           */
#define MOE_MAX_E 256    /* experts per layer           */
#define MOE_MAX_G 64     /* logical ranks in the group  */

/* Human-readable name of a status code (static string, host). */
const char* moe_status_string(int status);

/* ------------------------------------------------------------------------
 * moe_coact_stats -- co-activation statistics of one layer.
 *
 * [CB] Key Observation: the set of tokens that activate each expert, and the
 * Ochiai similarity |A n B| / sqrt(|A| |B|) of two experts' token sets.
 * [EC] abstract: expert pairs selected together within a layer, and the
 * experts a token picks at one layer predicting those it picks at the next.
 *
 *   topk          [T*k]   int32, row-major [T][k]: the experts D_t of token t
 *   topk_next     [T*k_next] int32 or NULL: the same tokens' experts at the
 *                         next layer (E_next experts); needed for transition
 *   expert_count  [E]     int32 out: |A_e|, tokens that selected e
 *   pair_count    [E*E]   int32 out or NULL: C[i*E+j] = |A_i n A_j|, full
 *                         symmetric, diagonal = expert_count
 *   ochiai        [E*E]   float out or NULL (needs pair_count):
 *                         C[i][j] / sqrt(n_i * n_j) evaluated in double and
 *                         rounded once to float; 0 where n_i * n_j == 0
 *   transition    [E*E_next] int32 out or NULL (needs topk_next):
 *                         X[i*E_next+j] = #{t : i in D_t, j in D'_t}
 *   ws, ws_bytes  workspace of at least
 *                 moe_coact_stats_workspace_size(T, E, pair_count != NULL,
 *                 transition != NULL ? E_next : 0) bytes, 16-byte aligned:
 *                 per-split partial counts (at most 128 splits of the tokens)
 * Limits: 1 <= k, k_next <= 8; 1 <= E, E_next <= 256; T >= 0.
 * d_err bits: EXPERT_RANGE (slot skipped), EXPERT_DUP (the repeat is skipped).
 * Integer outputs are exact and independent of scheduling; every output
 * element is written.
 * ---------------------------------------------------------------------- */
int moe_coact_stats_workspace_size(int64_t T, int E, int pairs, int E_next,
                                   size_t* ws_bytes /* host */);
int moe_coact_stats(const int32_t* topk, int64_t T, int k, int E,
                    const int32_t* topk_next, int k_next, int E_next,
                    int32_t* expert_count, int32_t* pair_count, float* ochiai,
                    int32_t* transition, int32_t* d_err, void* ws, size_t ws_bytes,
                    void* stream);

/* ------------------------------------------------------------------------
 * moe_dispatch_plan -- deduplicated dispatch plan.
 *
 * [EC] abstract: deduplicated dispatch -- a token reaches a given GPU at
 * most one time, however many of its experts live there.
 * [CB] Problem Formulation: tokens t with selected experts D_t, source rank
 * s_t, node N(r) of rank r, cross-node volume
 * V = sum_t |{N(r_t^e) : e in D_t} minus {N(s_t)}|; with one replica per
 * expert, r_t^e = expert_rank[e].
 *
 * R_t = {expert_rank[e] : e in D_t}.  One send row per (t, r in R_t).  Rows
 * are ordered by (source rank s, destination rank r, token t ascending), so
 * block (s, r) = rows [send_offsets[s*G+r], send_offsets[s*G+r+1]) is the
 * message from s to r.  Source ranks hold contiguous token ranges:
 * s_t = the s with src_offsets[s] <= t < src_offsets[s+1].
 *
 *   topk          [T*k] int32: experts of each token
 *   gates         [T*k] float or NULL: gate weight of each slot
 *   expert_rank   [E]   int32: the placement p(e)
 *   G             logical ranks (1..64); ranks_per_node divides G;
 *                 node(r) = r / ranks_per_node
 *   src_offsets   [G+1] int32 or NULL (NULL = equal shards, T % G == 0)
 *   row_capacity  rows available in row_token / row_weight;
 *                 T * min(k, G) always suffices
 *   send_counts   [G*G]   int32 out: S[s*G+r]
 *   send_offsets  [G*G+1] int32 out: exclusive prefix of S; last = N
 *   row_token     [row_capacity] int32 out: token of each row
 *   row_weight    [row_capacity] float out or NULL: the token's gate mass on
 *                 the row's rank, a float running sum over ascending slot j
 *                 (0 if gates is NULL)
 *   token_rows    [T*k] int32 out: rows of token t by ascending rank, then -1
 *   slot_row      [T*k] int32 out or NULL: row carrying slot (t, j)
 *   counters      [8] int64 out: N, T*k, local_rows (r == s_t),
 *                 local_assign (slots with p(e) == s_t), node_rows
 *                 (sum_t distinct destination nodes), V, max rows received
 *                 by one rank, 0
 *   ws, ws_bytes  workspace of at least moe_dispatch_plan_workspace_size()
 *                 bytes, 16-byte aligned
 * d_err bits: EXPERT_RANGE, EXPERT_DUP, RANK_RANGE, CAPACITY, SRC_OFFSETS.
 * ---------------------------------------------------------------------- */
int moe_dispatch_plan_workspace_size(int64_t T, int G, size_t* ws_bytes /* host */);
int moe_dispatch_plan(const int32_t* topk, const float* gates, int64_t T, int k, int E,
                      const int32_t* expert_rank, int G, int ranks_per_node,
                      const int32_t* src_offsets, int64_t row_capacity,
                      int32_t* send_counts, int32_t* send_offsets, int32_t* row_token,
                      float* row_weight, int32_t* token_rows, int32_t* slot_row,
                      int64_t* counters, int32_t* d_err, void* ws, size_t ws_bytes,
                      void* stream);

/* ------------------------------------------------------------------------
 * moe_dispatch_plan_noalloc -- moe_dispatch_plan without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, outputs and d_err bits as moe_dispatch_plan minus ws and
 * ws_bytes; the results are identical.  The per-tile scratch lives in a
 * device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends; the call allocates nothing and
 * calls no allocating routine.  Its address is looked up once per device on
 * the first call there, so the calling thread's current device must be the
 * stream's device.  Every call on one device shares that device's array:
 * calls whose work overlaps on one device (other streams, other threads)
 * race and give wrong plans.
 * Returns MOE_ERR_WORKSPACE (nothing enqueued) when
 * moe_dispatch_plan_workspace_size(T, G) exceeds MOE_NOALLOC_SCRATCH_BYTES
 * (e.g. T above about 3.9 million tokens at G = 64), and MOE_ERR_HIP when
 * the device or the array's address cannot be obtained.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_dispatch_plan_noalloc(const int32_t* topk, const float* gates, int64_t T, int k, int E,
                              const int32_t* expert_rank, int G, int ranks_per_node,
                              const int32_t* src_offsets, int64_t row_capacity,
                              int32_t* send_counts, int32_t* send_offsets, int32_t* row_token,
                              float* row_weight, int32_t* token_rows, int32_t* slot_row,
                              int64_t* counters, int32_t* d_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_dispatch_plan_gathered -- the plan of a shuffled batch.
 *
 * [EC] abstract: tokens are shuffled toward the rank forecast for their
 * next-layer experts, and the next layer's dispatch starts from there.  This
 * is moe_dispatch_plan on the routing in the shuffled order -- position p
 * holds token perm[p], i.e. topk'[p] = topk[perm[p]], gates'[p] =
 * gates[perm[p]] -- and writes that gathered routing out as well, so the
 * routing needs no separate move.  Every plan output is indexed by position,
 * exactly as moe_dispatch_plan(topk', gates', ...) would give it.
 *
 *   topk, gates     [T*k] in the original token order (gates may be NULL)
 *   perm            [T] int32: the token at each position (moe_shuffle_predict's
 *                   perm); entries outside [0, T) set ROW_RANGE and that
 *                   position plans no rows (its topk_out row is -1)
 *   topk_out        [T*k] int32 out: topk'; gates_out [T*k] float out: gates'
 *                   (required when gates is given); neither may alias its input
 *   everything else as for moe_dispatch_plan (src_offsets by position, e.g.
 *   the shuffle's shard_offsets; same workspace size).
 * d_err bits: as moe_dispatch_plan, plus ROW_RANGE for perm.
 * ---------------------------------------------------------------------- */
int moe_dispatch_plan_gathered(const int32_t* topk, const float* gates, const int32_t* perm,
                               int64_t T, int k, int E, const int32_t* expert_rank, int G,
                               int ranks_per_node, const int32_t* src_offsets,
                               int64_t row_capacity, int32_t* send_counts,
                               int32_t* send_offsets, int32_t* row_token, float* row_weight,
                               int32_t* token_rows, int32_t* slot_row, int64_t* counters,
                               int32_t* topk_out, float* gates_out, int32_t* d_err, void* ws,
                               size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute -- row scatter into send buffers (the dispatched hidden
 * states of [CE] footnote 3; also the token shuffle of [EC] abstract).
 *
 *   out[dest[t*width + q]] = x[t]   for t < T, q < width, dest >= 0
 * Rows are copied bit for bit, so any element type works.
 *   x          [T * row_bytes] bytes
 *   dest       [T*width] int32: destination rows (-1 = none), e.g. a plan's
 *              token_rows (width = k) or a shuffle's dest_pos (width = 1)
 *   out        [out_rows * row_bytes] bytes; rows nobody targets are untouched
 *   n_valid    int32 device word or NULL: when set, only tokens
 *              t < min(T, *n_valid) are moved (e.g. a plan's row count, read
 *              on the device so the host need not wait for it)
 * row_bytes must be a positive multiple of 4 and x, out 4-byte aligned; rows
 * that are multiples of 16 bytes with 16-byte aligned buffers take the wide
 * path.  width in 1..8.
 * d_err bits: ROW_RANGE (dest >= out_rows; that copy is skipped).
 * ---------------------------------------------------------------------- */
int moe_permute(const void* x, int64_t T, int64_t row_bytes, const int32_t* dest, int width,
                void* out, int64_t out_rows, const int32_t* n_valid, int32_t* d_err,
                void* stream);

/* ------------------------------------------------------------------------
 * moe_shuffle_dispatch -- the token shuffle's move and the next layer's
 * dispatch in one pass ([EC] abstract: tokens are shuffled to the rank
 * predicted to hold their next-layer experts and dispatched from there):
 *   x_out[p] = x[perm[p]]
 *   send[token_rows[p*k + q]] = x[perm[p]]   for q < k, entry >= 0
 * i.e. the shuffle's move (moe_gather(x, perm)) followed by
 * moe_permute(x_out, token_rows), reading each row once.  token_rows is the
 * next layer's plan over the shuffled order (moe_dispatch_plan on the
 * shuffled routing with the shuffle's shard_offsets).
 *   x          [T * row_bytes] bytes
 *   perm       [T] int32: the token at each shuffled position
 *              (moe_shuffle_predict's perm)
 *   token_rows [T*k] int32, by shuffled position
 *   x_out      [T * row_bytes] bytes, send [send_rows * row_bytes] bytes
 * Same row-size and alignment rules as moe_permute; k in 1..8.
 * d_err bits: ROW_RANGE (a perm entry outside [0, T) -- that position is
 * skipped -- or a send row >= send_rows -- that copy is skipped).
 * ---------------------------------------------------------------------- */
int moe_shuffle_dispatch(const void* x, int64_t T, int64_t row_bytes, const int32_t* perm,
                         const int32_t* token_rows, int k, void* x_out, void* send,
                         int64_t send_rows, int32_t* d_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_gather -- row gather, the destination-ordered form of moe_permute for
 * maps in which every output row has one source: the token shuffle of [EC]
 * abstract (out = x[perm]) and the expansion of received rows into expert
 * rows (out[i] = send[erow_src[i]], see moe_expert_plan).
 *
 *   out[i] = x[src[i]]   for i < n_rows (and i < *n_valid when given), src >= 0
 * Rows are copied bit for bit.
 *   x          [x_rows * row_bytes] bytes
 *   src        [n_rows] int32: source row of each output row (-1 = leave the
 *              output row untouched)
 *   out        [n_rows * row_bytes] bytes
 *   n_valid    int32 device word or NULL, as for moe_permute
 * Same row-size and alignment rules as moe_permute; n_rows, x_rows < 2^31.
 * d_err bits: ROW_RANGE (src >= x_rows; that row is skipped).
 * ---------------------------------------------------------------------- */
int moe_gather(const void* x, int64_t x_rows, int64_t row_bytes, const int32_t* src,
               int64_t n_rows, void* out, const int32_t* n_valid, int32_t* d_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_combine -- weighted combine back to token order (the hidden-state
 * combine of [CE] footnote 3 over the deduplicated rows of [EC] abstract).
 *
 *   y[t] = sum_{q : rows[t*k+q] >= 0} a(rows[t*k+q]) * z[rows[t*k+q]]
 * with a = row_weight (NULL: a = 1, for expert sides that applied the gates
 * themselves).  Summed in float in ascending q, rounded once to y_dtype
 * (bf16: round to nearest even).
 *   z        [z_rows * H] of z_dtype (MOE_F32 or MOE_BF16)
 *   rows     [T*k] int32, e.g. a plan's token_rows
 *   y        [T * H] of y_dtype
 *   n_valid  int32 device word or NULL: when set, only outputs
 *            t < min(T, *n_valid) are written (the rest are untouched)
 * H * sizeof(z_dtype) and H * sizeof(y_dtype) must be multiples of 16 bytes,
 * z and y 16-byte aligned.  k in 1..8.
 * d_err bits: ROW_RANGE (row >= z_rows; that term is skipped).
 * ---------------------------------------------------------------------- */
int moe_combine(const void* z, int z_dtype, int64_t z_rows, int64_t H, const int32_t* rows,
                int k, const float* row_weight, int64_t T, void* y, int y_dtype,
                const int32_t* n_valid, int32_t* d_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_shuffle_predict -- token shuffling ([EC] abstract: tokens reordered by
 * the rank forecast for their next-layer experts).
 *
 * score_t[r] = sum_{i in D_t} sum_{j : expert_rank_next[j] == r} X[i][j]
 * (64-bit integer sums of the transition counts), pred_t = the highest
 * scoring rank, the lowest rank on ties.  Tokens are then ordered by pred,
 * stably (ascending t within a rank).
 *
 *   topk              [T*k] int32: this layer's experts
 *   transition        [E*E_next] int32: X, e.g. from moe_coact_stats
 *   expert_rank_next  [E_next] int32: next-layer placement
 *   pred_rank         [T] int32 out
 *   dest_pos          [T] int32 out: new position of token t
 *   perm              [T] int32 out or NULL: token at new position q
 *   shard_offsets     [G+1] int32 out: first position of each rank's tokens
 *                     (usable as the next plan's src_offsets)
 *   ws, ws_bytes      workspace of moe_shuffle_predict_workspace_size() bytes,
 *                     256-byte aligned
 * Limits: 1 <= k <= 8, 1 <= E, E_next <= 256, 1 <= G <= 64.
 * d_err bits: EXPERT_RANGE, RANK_RANGE (entries skipped).
 * ---------------------------------------------------------------------- */
int moe_shuffle_predict_workspace_size(int64_t T, int E, int G, size_t* ws_bytes /* host */);
int moe_shuffle_predict(const int32_t* topk, int64_t T, int k, int E, const int32_t* transition,
                        int E_next, const int32_t* expert_rank_next, int G, int32_t* pred_rank,
                        int32_t* dest_pos, int32_t* perm, int32_t* shard_offsets,
                        int32_t* d_err, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_shuffle_balanced -- token shuffling with equal shards: every rank
 * receives exactly T/G tokens (T % G == 0), as the reduce-scatter that
 * carries the shuffle hands each rank a fixed share ([EC] abstract).
 * Tokens in order take their highest-scoring rank (the scores of
 * moe_shuffle_predict, lower rank on ties) that still has room.  Arguments,
 * outputs and workspace rules as for moe_shuffle_predict, with
 * moe_shuffle_balanced_workspace_size(); pred_rank receives the assigned
 * rank and shard_offsets = [0, T/G, 2T/G, ..., T].
 * ---------------------------------------------------------------------- */
int moe_shuffle_balanced_workspace_size(int64_t T, int E, int G, size_t* ws_bytes /* host */);
int moe_shuffle_balanced(const int32_t* topk, int64_t T, int k, int E, const int32_t* transition,
                         int E_next, const int32_t* expert_rank_next, int G, int32_t* pred_rank,
                         int32_t* dest_pos, int32_t* perm, int32_t* shard_offsets,
                         int32_t* d_err, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_plan -- destination-side layout for the expert computation.
 *
 * Every assignment (t, j) -- expert e = D_t[j] on rank r = expert_rank[e] --
 * gets one expert row; rows are ordered by (r, e, t), so each rank's
 * received tokens expand into one contiguous block per local expert
 * (ascending expert id), the layout a grouped expert GEMM consumes
 * ("Training Communication-Efficient Mixture-of-Experts Language Models with
 * Layer Re-Configuration": alltoall dispatch, grouped GEMM; footnote 3: the
 * routed probabilities travel with the rows).
 *
 *   topk, gates, T, k, E, expert_rank, G   as for moe_dispatch_plan
 *   slot_row      [T*k] int32: the dispatch plan's row of each slot
 *   send_rows     rows of row_dest (the send buffer's capacity)
 *   erow          [T*k] int32 out: expert row of each slot (-1 if skipped)
 *   expert_first  [E] int32 out: first expert row of expert e
 *   expert_count  [E] int32 out: rows of expert e
 *   rank_offsets  [G+1] int32 out: first expert row of each rank
 *   erow_weight   [T*k] float out or NULL: the gate carried by each expert row
 *   erow_slot     [T*k] int32 out or NULL: t*k + j of each expert row
 *   erow_src      [T*k] int32 out or NULL: the send row each expert row is
 *                 expanded from (slot_row of its slot; -1 if out of range)
 *   row_dest      [send_rows*k] int32 out: for send row (t, r), the expert
 *                 rows of t's slots on r in ascending slot order, then -1
 *                 (all -1 for rows no slot maps to)
 *   ws, ws_bytes  workspace of moe_expert_plan_workspace_size() bytes
 * With these, moe_gather(send, send_rows, row_bytes, erow_src, T*k, ...)
 * (or, equivalently, moe_permute(send, send_rows, row_bytes, row_dest, k,
 * ...)) expands the received rows into expert rows, and moe_combine(expert_out,
 * ..., row_dest, k, erow_weight, send_rows, reply, ...) forms each (t, r)
 * reply row sum_{j on r} w_tj * expert_out[erow(t, j)]; the final
 * moe_combine of the replies is then unweighted.
 * d_err bits: EXPERT_RANGE, EXPERT_DUP, RANK_RANGE, ROW_RANGE (slot_row
 * outside [0, send_rows)).
 * ---------------------------------------------------------------------- */
int moe_expert_plan_workspace_size(int64_t T, int E, size_t* ws_bytes /* host */);
int moe_expert_plan(const int32_t* topk, const float* gates, int64_t T, int k, int E,
                    const int32_t* expert_rank, int G, const int32_t* slot_row, int64_t send_rows,
                    int32_t* erow, int32_t* expert_first, int32_t* expert_count,
                    int32_t* rank_offsets, float* erow_weight, int32_t* erow_slot,
                    int32_t* erow_src, int32_t* row_dest, int32_t* d_err, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward mirror.  The all-to-alls run again in the backward pass with the
 * data flowing back ([EC] abstract; [CE] footnote 3: inverse all-to-alls of
 * the dispatch, routed-probability dispatch and combine).  For the weighted
 * combine y_t = sum_q a(row_q) z[row_q]:
 *   dL/dz[row] = a(row) * dL/dy_t          -> moe_permute_scaled
 *   dL/dw_tj   = <dL/dy_t, z[slot_row(t,j)]> -> moe_row_dot
 * and the adjoint of moe_permute is the unweighted moe_combine.
 *
 * moe_permute_scaled:  out[dest[t*width+q]] = scale[dest] * x[t] for every
 *   dest >= 0, the product formed in fp32 and rounded once to out_dtype.
 *   x [T*H] of x_dtype; dest [T*width] int32; scale [out_rows] float (indexed
 *   by the destination row); out [out_rows*H] of out_dtype (untargeted rows
 *   untouched); n_valid as for moe_permute.  H*sizeof must be a multiple of
 *   16 bytes for both types (8 elements when a bf16 side is involved),
 *   buffers 16-byte aligned.  d_err bits: ROW_RANGE.
 * moe_row_dot:  out[t*width+q] = <a[t], b[rows[t*width+q]]> summed in fp32
 *   in a fixed order (0 where the row is < 0).  a [T*H], b [b_rows*H],
 *   out [T*width] float.  Same row-size rules.  d_err bits: ROW_RANGE.
 * ---------------------------------------------------------------------- */
int moe_permute_scaled(const void* x, int x_dtype, int64_t T, int64_t H, const int32_t* dest,
                       int width, const float* scale, void* out, int out_dtype, int64_t out_rows,
                       const int32_t* n_valid, int32_t* d_err, void* stream);
int moe_row_dot(const void* a, int a_dtype, int64_t T, int64_t H, const void* b, int b_dtype,
                int64_t b_rows, const int32_t* rows, int width, float* out,
                const int32_t* n_valid, int32_t* d_err, void* stream);

/* ------------------------------------------------------------------------
 * Statistics over steps and placement ("Cobalt: Leveraging Expert
 * Co-activation for Efficient Distributed MoE Training", Stage 1: the layout
 * is re-planned periodically from moving averages of co-selection counts
 * and expert loads; [EC] abstract: experts often selected together go on
 * the same GPU).
 *
 * moe_ema_update:  state[i] = beta * state[i] + (1 - beta) * x[i] for
 *   i < n, each product and the sum rounded to float separately.  state
 *   [n] float (device, in/out), x [n] int32 (device), 0 <= beta <= 1.
 * moe_place_experts (HOST pointers, runs on the host, synchronous):
 *   coact [E*E] float (co-selection weights, diagonal ignored), load [E]
 *   float, eps >= 0, expert_rank [E] int32 out.  Every rank receives E/G
 *   experts (E % G == 0).  Ranks are filled one at a time, in order; each
 *   step adds the unplaced expert most co-selected with the rank's experts
 *   so far (ties: larger total co-activation, then lower id), preferring
 *   experts that keep the rank's load within (1 + eps) * sum(load) / G.
 *   Double-precision sums in ascending expert order.
 * ---------------------------------------------------------------------- */
int moe_ema_update(float* state, const int32_t* x, int64_t n, float beta, void* stream);
int moe_place_experts(const float* coact /* host */, const float* load /* host */, int E, int G,
                      double eps, int32_t* expert_rank /* host */);

#ifdef __cplusplus
}
#endif

#endif /* MOE_COACT_H */
