/*
 * longspark.h -- C ABI of the LongSpark fixed-cost drafting path on MI355X.
 *
 * Source: the paper page "LongSpark: Efficient speculative decoding with a
 * fixed-cost parallel drafter" (arXiv 2609.37029).  One decoding round
 * (Fig. 2): (a) the target verifies the drafted block; (b) fixed-size views
 * of the target's state are kept -- a recent KV window and a global context
 * summary; (c) the drafter attends over those views to propose the next
 * block, at a cost that does not depend on the prefix length.  The summary is
 * initialised over the whole prefix at prefill and then updated with only the
 * newly retained rows, at most B+1 per round (Fig. 3).
 *
 * The pages print no formula for the summary.  This library implements S
 * slots per KV head: slot j pools retained rows p = 0..t (t = newest) with
 * weight w_jp = exp(u_j . k_p / sqrt(d)) * lambda_j^(t-p) (0^0 = 1); its key
 * is sum w k / sum w and its value sum w v / sum w.  The state is kept as an
 * online-softmax triple per slot: a_jp = u_j.k_p/sqrt(d) + (t-p) ln lambda_j,
 * m = max_p a_jp, l = sum_p exp(a_jp - m), n = sum_p exp(a_jp - m) [k_p ; v_p].
 *
 * Conventions for every entry point
 *   - All array pointers are DEVICE memory owned by the caller.  The library
 *     never allocates, frees or keeps a pointer after a call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and never synchronises with the host.
 *   - Arrays are dense row-major in the shapes given below.  "dtype" arrays
 *     hold IEEE float32 (LS_F32) or bfloat16 (LS_BF16) per `ls_dims.dtype`.
 *   - Errors that the host can see (NULL pointer, bad size, unsupported
 *     shape or dtype, workspace too small, misaligned pointer) are returned
 *     BEFORE anything is launched.  LS_ERR_HIP means a launch failed.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Calls that share one workspace or one state must not overlap (same
 *     stream, or ordered with events).
 *
 * Supported shapes: Hq % Hkv == 0; 1 <= B <= 47; 1 <= V <= 2^20;
 *   C*(B+1) <= 65535; W >= 0 with B+1 <= W when W > 0; S >= 0;
 *   C*Hkv*S <= 2^30.
 *   LS_F32 : d in {16, 32, 64, 128}, S <= 256 (any number of query rows
 *            B*Hq/Hkv per KV head).
 *   LS_BF16: d == 128, S in {0, 64, 128}, W % 32 == 0, B*Hq/Hkv <= 64.
 * W = 0 switches the window view off and S = 0 the summary view (the view
 * ablations of Table 5, cost side): the drafter then attends to the other
 * views and the block, and the switched-off view's state arrays may be NULL
 * (ring_k, ring_v, ring_pos when W = 0; sum_m, sum_l, sum_n, slot_k, slot_v,
 * u, log_lambda when S = 0).
 * Pointers to dtype arrays, ring_pos and sum_n must be 16-byte aligned.
 * The values of the window and of the slots are kept in key tiles of 32
 * (per tile: [d][32]) so that the drafter's P.V product reads contiguous
 * keys per dimension and each 32-key tile is one contiguous block.
 * With d = 128 the keys of the window and of the slots are kept in tiles of
 * 32 keys too, in the order in which the drafter's 16x16x32 MFMA reads its
 * A operand: key k = 8a + 4b + r (a < 4, b < 2, r < 4) and dimension
 * e = 32s + 8g + i (s < 4, g < 4, i < 8) of a tile sit at element
 * ((((b*4 + s)*4 + g)*16 + 4a + r)*8 + i of the tile's 32*128 elements.
 * Other d keep keys row-major.  The state is the library's own: callers
 * allocate it, move it as a whole and never read it element by element.
 */
#ifndef LONGSPARK_H
#define LONGSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ls_dtype { LS_F32 = 0, LS_BF16 = 1 } ls_dtype;

typedef enum ls_status {
  LS_OK = 0,
  LS_ERR_NULL = 1,      /* a required pointer is NULL                        */
  LS_ERR_SHAPE = 2,     /* a size is out of range or not supported           */
  LS_ERR_DTYPE = 3,     /* dtype is neither LS_F32 nor LS_BF16               */
  LS_ERR_WORKSPACE = 4, /* workspace missing or smaller than required        */
  LS_ERR_ALIGN = 5,     /* a pointer lacks the required 16-byte alignment    */
  LS_ERR_HIP = 6,       /* the HIP runtime reported an error at launch       */
  LS_ERR_SCRATCH = 7    /* too large for ls_verify_greedy_noalloc's static
                           scratch (see there)                              */
} ls_status;

/* A hipStream_t; NULL selects the default stream. */
typedef void* ls_stream;

/* Sizes shared by every call. */
typedef struct ls_dims {
  int32_t C;     /* concurrent sequences                                  */
  int32_t Hq;    /* query heads of the drafter's attention                */
  int32_t Hkv;   /* KV heads (GQA: query head hq reads KV head hq/(Hq/Hkv)) */
  int32_t d;     /* head dimension                                        */
  int32_t W;     /* rows of the recent-KV ring window                     */
  int32_t S;     /* summary slots per KV head                             */
  int32_t B;     /* drafted block length; B+1 positions are verified      */
  int32_t V;     /* vocabulary size                                       */
  int32_t dtype; /* ls_dtype of every "dtype" array                       */
} ls_dims;

/* The drafter's fixed-size context state (Fig. 2 (b)) plus parameters.
 * Its size is independent of the prefix length. */
typedef struct ls_state {
  void* ring_k;             /* [C, Hkv, W, d] dtype: window keys (32-key
                               tiles in MFMA operand order when d = 128)    */
  void* ring_v;             /* dtype window values in key tiles of 32:
                               [C, Hkv, W/32, d, 32] ([C, Hkv, d, W] when
                               W % 32 != 0)                                 */
  int32_t* ring_pos;        /* [C, W] absolute position held, -1 = empty     */
  int32_t* seq_len;         /* [C] retained rows per sequence                */
  float* sum_m;             /* [C, Hkv, S] running max m (natural log units) */
  float* sum_l;             /* [C, Hkv, S] denominator l                     */
  float* sum_n;             /* [C, Hkv, S, 2d] numerator n: keys | values;
                               bf16 states keep each 32-slot tile in MFMA
                               accumulator order: entry e = 32t + 8g + 4b + r
                               of slot s at float ((t*4+g)*64 + 32b + s)*4 + r */
  void* slot_k;             /* [C, Hkv, S, d] dtype: n[:d] / l (32-key
                               tiles in MFMA operand order when d = 128)    */
  void* slot_v;             /* dtype n[d:] / l in key tiles of 32:
                               [C, Hkv, S/32, d, 32] ([C, Hkv, d, S] when
                               S % 32 != 0)                                 */
  const void* u;            /* [Hkv, S, d] dtype: slot queries               */
  const float* log_lambda;  /* [S] ln(lambda_j); -INFINITY for lambda_j = 0  */
  int32_t* err_flag;        /* [1] sticky device error word, 0 = no error    */
  void* workspace;          /* scratch, see ls_workspace_bytes               */
  size_t workspace_bytes;
} ls_state;

/* Bytes of workspace that every call below needs for prefixes of up to
 * `max_L0` rows.  The workspace is scratch that each call overwrites before
 * reading (split partials); it needs no initialisation and carries nothing
 * from one call to the next.  Returns 0 if `dims` is invalid. */
size_t ls_workspace_bytes(const ls_dims* dims, int32_t max_L0);

/* Prefill view (Fig. 3: the summary is initialised over the full prefix).
 *   k_prefix, v_prefix: [C, prefix_rows_stride, Hkv, d] dtype, token-major
 *     (the serving KV-cache layout); rows 0..L0-1 of each sequence are read.
 *   L0 >= 1, prefix_rows_stride >= L0.
 * Writes sum_m, sum_l, sum_n, slot_k, slot_v over all L0 rows (t = L0-1);
 * the ring gets rows max(0, L0-W)..L0-1 at slot p mod W with ring_pos = p,
 * other ring slots get zero rows and position -1; seq_len = L0; err_flag = 0.
 * Cost O(L0): the only call that reads the prefix. */
ls_status ls_summary_init(const ls_dims* dims, const ls_state* state, const void* k_prefix,
                          const void* v_prefix, int32_t L0, int64_t prefix_rows_stride,
                          ls_stream stream);

/* Greedy verification (Fig. 2 (a); Table 3, T = 0).
 *   logits:     [C, B+1, V] dtype, the target's scores at the B+1 verified
 *               positions (last committed token, drafts 1..B); no NaN.
 *   draft:      [C, B] int32 drafted tokens.
 *   target_tok: [C, B+1] int32 out, g_i = argmax_v logits[c,i,v], lowest
 *               index on ties (+0 and -0 compare equal).
 *   tau:        [C] int32 out, M+1 where M is the longest prefix with
 *               draft[c,i] == g_i; tau is in [1, B+1].
 *   workspace:  as sized by ls_workspace_bytes (any max_L0). */
ls_status ls_verify_greedy(const ls_dims* dims, const void* logits, const int32_t* draft,
                           int32_t* target_tok, int32_t* tau, void* workspace,
                           size_t workspace_bytes, ls_stream stream);

/* Per-round update (Fig. 2 (b), Fig. 3: only the newly retained rows).
 *   k_new, v_new: [C, B+1, Hkv, d] dtype, KV rows of the verified positions.
 *   tau: [C] int32 in DEVICE memory (e.g. from ls_verify_greedy): rows
 *        0..tau[c]-1 are retained.  Values outside [1, B+1] are clamped into
 *        it and set bit 0 of *err_flag.
 * Appends the rows to the ring at slot (L+i) mod W (ring_pos = L+i), shifts
 * every slot's m by tau*ln(lambda_j), merges the new rows into (m, l, n),
 * rewrites slot_k/slot_v and sets seq_len += tau.  O(tau*S*d) work per
 * (sequence, KV head); the prefix is never read. */
ls_status ls_append_accepted(const ls_dims* dims, const ls_state* state, const void* k_new,
                             const void* v_new, const int32_t* tau, ls_stream stream);

/* Greedy verification followed by the per-round update (Fig. 2 (a) then
 * (b): the target verifies the drafted block, the accepted rows extend the
 * views).  The same results, bit for bit, as ls_verify_greedy (into
 * target_tok and tau) then ls_append_accepted with that tau, in one launch
 * fewer: the update derives tau itself from the verification's partial
 * argmax keys, so the verification's finishing launch is not needed.
 *   logits, draft, target_tok, tau: as in ls_verify_greedy (tau is written,
 *        in [1, B+1]); the keys go to state->workspace.
 *   k_new, v_new: as in ls_append_accepted.
 * f32 shapes run the two entry points' launches. */
ls_status ls_verify_append(const ls_dims* dims, const ls_state* state, const void* logits,
                           const int32_t* draft, int32_t* target_tok, int32_t* tau,
                           const void* k_new, const void* v_new, ls_stream stream);

/* ls_verify_greedy without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * ls_verify_greedy, minus the workspace; it allocates nothing.
 * Its C*(B+1)*ceil(V/8192) partial argmax keys live in a static 512 KiB
 * device array that the library holds on each GPU it runs on until the
 * process ends: at most 65536 keys (e.g. C*(B+1) <= 3449 at V = 151936).
 * Larger calls return LS_ERR_SCRATCH before anything is launched.  Every
 * call on one GPU shares that array: calls that overlap on one GPU
 * (different streams without ordering) race; calls ordered on one stream
 * are safe (each writes every key it reads, nothing carries over).
 * LS_ERR_HIP if the array's device address cannot be obtained. */
ls_status ls_verify_greedy_noalloc(const ls_dims* dims, const void* logits, const int32_t* draft,
                                   int32_t* target_tok, int32_t* tau, ls_stream stream);

/* One whole drafting round (Fig. 2: (a) the target verifies the drafted
 * block, (b) the accepted rows extend the views, (c) the drafter attends
 * over the views): ls_verify_append followed by ls_draft_attention, in two
 * launches instead of three.  The update and the draft attention share one
 * launch; the draft sees the window as updated (the tau new rows in place of
 * the ones they replace) and the merged slots.
 *   logits, draft, target_tok, tau, k_new, v_new: as in ls_verify_append.
 *   q, k_blk, v_blk, out: as in ls_draft_attention (the next block's
 *       queries and block rows; out is the attention output).
 * The state, target_tok and tau are bit for bit those of the two calls; out
 * equals theirs up to the order in which the softmax visits the keys (the
 * new window rows and the slots are attended as chunks of their own, and
 * the probabilities enter P.V rounded to bf16 against the running maximum).
 * The state's workspace also holds per-(sequence, KV head, 32-slot tile)
 * arrival counters that the key pass zeroes and the update leaves at zero
 * (no carry-over between calls).  Shapes other than bf16, d = 128, S in {64, 128}, B + 1 <= 32,
 * W a positive multiple of 32 and at most 64 query rows B*Hq/Hkv per KV
 * head run the two calls' launches.  Equal to ls_verify_keys followed by
 * ls_update_draft on the same stream. */
ls_status ls_verify_append_draft(const ls_dims* dims, const ls_state* state, const void* logits,
                                 const int32_t* draft, int32_t* target_tok, int32_t* tau,
                                 const void* k_new, const void* v_new, const void* q,
                                 const void* k_blk, const void* v_blk, void* out,
                                 ls_stream stream);

/* The two launches of ls_verify_append_draft as calls of their own, for a
 * caller that wants to place other work between them.
 * ls_verify_keys: the verification's pass over the logits (Fig. 2 (a)): the
 *   per-chunk argmax keys of the C*(B+1) rows go to the state's workspace,
 *   together with the lengths seq_len as they stand (the update appends at
 *   those lengths) and zeroed arrival counters.  Reads logits only; changes
 *   no state.  LS_ERR_NULL if logits is null.
 * ls_update_draft: the rest of the round (Fig. 2 (a) acceptance, (b), (c))
 *   from what the last ls_verify_keys on this state's workspace left there:
 *   target_tok, tau, the update and the draft attention, as
 *   ls_verify_append_draft.  Arguments as there, minus logits.  A second
 *   call without a new key pass appends the same accepted rows at the same
 *   lengths again (the ring rows and lengths come out the same, the summary
 *   merges them once more); the results are unspecified if no key pass ran
 *   on the workspace since it was allocated. */
ls_status ls_verify_keys(const ls_dims* dims, const ls_state* state, const void* logits,
                         ls_stream stream);
ls_status ls_update_draft(const ls_dims* dims, const ls_state* state, const int32_t* draft,
                          int32_t* target_tok, int32_t* tau, const void* k_new, const void* v_new,
                          const void* q, const void* k_blk, const void* v_blk, void* out,
                          ls_stream stream);

/* Drafter block attention (Fig. 2 (c)).
 *   q:            [C, B, Hq, d] dtype, block queries.
 *   k_blk, v_blk: [C, B, Hkv, d] dtype, block keys/values.
 *   out:          [C, B, Hq, d] dtype.
 * out = softmax(q k^T / sqrt(d)) v over the occupied ring rows, the S slots
 * and the B block rows of the query's KV head; bidirectional (no mask).
 * Reads W + S + B rows per KV head whatever the prefix length. */
ls_status ls_draft_attention(const ls_dims* dims, const ls_state* state, const void* q,
                             const void* k_blk, const void* v_blk, void* out, ls_stream stream);

/* Drafter proposal at T = 0 (Fig. 1 caption: drafting time counts the
 * proposal and sampling of the drafted tokens; Table 3: greedy decoding).
 *   logits:    [C, B, V] dtype, the drafter's scores at the B block
 *              positions; no NaN.
 *   draft_tok: [C, B] int32 out, argmax over V of each row, lowest index on
 *              ties (+0 and -0 compare equal).
 *   workspace: as sized by ls_workspace_bytes (any max_L0).
 * The same chunked reduction as ls_verify_greedy, over the C*B rows. */
ls_status ls_draft_argmax(const ls_dims* dims, const void* logits, int32_t* draft_tok,
                          void* workspace, size_t workspace_bytes, ls_stream stream);

/* Boundary state view (Fig. 2 (b): a state taken from the target at the
 * accepted boundary): the newest committed position of each sequence.
 *   hidden:   [C, B+1, H] dtype, the target's states at the B+1 verified
 *             positions (caller's buffer, read only).
 *   H:        state width in elements, H >= 1.
 *   tau:      [C] int32 in DEVICE memory (e.g. from ls_verify_greedy); a
 *             value outside [1, B+1] is clamped and, if err_flag is not NULL,
 *             sets bit 0 of *err_flag.
 *   out:      [C, H] dtype out: row tau[c]-1 of sequence c, bit for bit.
 *   err_flag: int32 in device memory, or NULL. */
ls_status ls_gather_boundary(const ls_dims* dims, const void* hidden, int32_t H,
                             const int32_t* tau, void* out, int32_t* err_flag, ls_stream stream);

/* Target-side verification attention of one layer (Fig. 2 (a): the target
 * verifies the proposed block, attending over its whole context) -- the
 * per-round cost that grows with the prefix, which the drafter's fixed-size
 * views avoid.
 *   k_cache, v_cache: [C, rows_stride, Hkv, d] dtype, token-major; rows
 *               0..L[c]-1 are the context and rows L[c]..L[c]+B hold the B+1
 *               verified positions of sequence c (read only).
 *   L:          [C] int32 in DEVICE memory, context rows per sequence; a value
 *               outside [0, max_rows - B - 1] is clamped and, if err_flag is
 *               not NULL, sets bit 0 of *err_flag.
 *   max_rows:   host bound on L[c] + B + 1, with B + 1 <= max_rows <=
 *               rows_stride (sizes the grid and the workspace).
 *   q:          [C, B+1, Hq, d] dtype queries of the verified positions.
 *   out:        [C, B+1, Hq, d] dtype: query i of head hq attends to rows
 *               0..L[c]+i of KV head hq/(Hq/Hkv), scale 1/sqrt(d).
 *   workspace:  at least ls_workspace_bytes(dims, max_rows - B - 1) bytes.
 *   LS_BF16 needs (B+1)*Hq/Hkv <= 128.  Cost O(L): every context row is read. */
ls_status ls_verify_attention(const ls_dims* dims, const void* k_cache, const void* v_cache,
                              int64_t rows_stride, const int32_t* L, int32_t max_rows,
                              const void* q, void* out, void* workspace, size_t workspace_bytes,
                              int32_t* err_flag, ls_stream stream);

/* Sampled verification of a drafted block (Table 1: accepted lengths with
 * sampling at temperature 1; Table 3 is the greedy case, ls_verify_greedy).
 * The pages do not print the rule; this is the textbook speculative-sampling
 * rule.  p_j = softmax(target row j / T), q_j = softmax(drafter row j / T);
 * draft j is accepted when u_accept[c, j] * q_j(d) < p_j(d); at the first
 * rejection the token is drawn from max(0, p_j - q_j) (from p_j when that
 * residual is zero everywhere, i.e. p_j == q_j and the drafted token had
 * p = q = 0), after B acceptances from p_B, as the smallest k whose running
 * sum exceeds u_sample[c] times the total (inverse CDF over the vocabulary
 * in index order).
 *   target_logits: [C, B+1, V] dtype; draft_logits: [C, B, V] dtype; no NaN.
 *   draft:         [C, B] int32 drafted tokens (each in [0, V)).
 *   temperature:   T > 0 (host value).
 *   u_accept:      [C, B] float32 uniforms in [0, 1) (device).
 *   u_sample:      [C] float32 uniforms in [0, 1) (device).
 *   tokens:        [C, B+1] int32 out: the tau[c] emitted tokens, then -1.
 *   tau:           [C] int32 out, in [1, B+1].
 *   workspace:     as sized by ls_workspace_bytes (any max_L0).
 * Probabilities are formed in fp32 (base-2 exponentials of x log2(e) / T). */
ls_status ls_verify_sampling(const ls_dims* dims, const void* target_logits,
                             const void* draft_logits, const int32_t* draft, float temperature,
                             const float* u_accept, const float* u_sample, int32_t* tokens,
                             int32_t* tau, void* workspace, size_t workspace_bytes,
                             ls_stream stream);

/* Static description of a status code (any integer: unknown values give
 * "unknown status"). */
const char* ls_status_string(int32_t status);

/* Library ABI version (major * 100 + minor). */
int32_t ls_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LONGSPARK_H */
