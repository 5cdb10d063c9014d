/*
 * specverify.h - C ABI of libspecverify, the verify step of speculative
 * sampling on AMD Instinct MI355X (gfx950).
 *
 * Sources (the pages, cited by title and section):
 *   [A] "Speculative Decoding: Cách LLM Sinh Văn Bản Nhanh Gấp 2–3 Lần" (anhtu.dev)
 *   [B] "投机解码：让大模型「猜」着跑的数学魔术" (blog.oscine.io)
 *   [C] "5.3 Medusa, EAGLE và MTP" (infra-guide-du8.pages.dev)
 *   [D] "Спекулятивное декодирование: ускорение инференса LLM на 20–50%" (glukhov.org)
 *
 * Conventions shared by every entry point:
 *  - Array arguments are DEVICE pointers owned by the caller; the library
 *    never frees or retains them.  Layouts are row-major and contiguous with
 *    the vocabulary innermost: logits_p [B][K+1][V], logits_q [B][K][V],
 *    draft_tokens / u_accept [B][K], u_resample / out_n_accepted [B],
 *    out_tokens [B][K+1].
 *  - Logit element type: SPECV_F32 (float) or SPECV_BF16 (bfloat16 bits).
 *    Pointers must be aligned to their element size; 16-byte alignment with
 *    V*element_size a multiple of 16 selects the vectorised sweep, anything
 *    else a scalar sweep with the same results.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    nothing synchronises: results are valid once the caller synchronises.
 *    Argument checks happen on the host before any HIP call; a non-zero
 *    return means nothing was enqueued (SPECV_E_HIP: a launch failed).
 *  - No allocation: the caller passes a workspace of at least
 *    spec_verify_workspace_size() bytes (256-byte aligned).  Concurrent calls
 *    must use distinct workspaces.  Inputs are read-only; outputs are fully
 *    overwritten.
 *  - Logits must be finite or -inf with at least one finite value per row
 *    (NaN gives unspecified tokens, never an out-of-bounds access).  A draft
 *    id outside [0, V) fails its acceptance test and sets flag bit 2.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPECV_F32 = 0, SPECV_BF16 = 1 } specv_dtype_t;

#define SPECV_OK            0
#define SPECV_E_NULL       -1   /* a required pointer is NULL */
#define SPECV_E_SHAPE      -2   /* B < 1, K < 1, K > SPECV_MAX_K, V < 1, or sizes overflow */
#define SPECV_E_DTYPE      -3   /* dtype is not a specv_dtype_t */
#define SPECV_E_TEMP       -4   /* T is NaN, infinite, negative, or so small that 1/T overflows */
#define SPECV_E_WORKSPACE  -5   /* workspace NULL, misaligned, or smaller than required */
#define SPECV_E_ALIGN      -6   /* a logits pointer is not aligned to its element size */
#define SPECV_E_HIP        -7   /* a kernel launch failed */
#define SPECV_E_SCRATCH    -8   /* spec_verify_noalloc: the shape needs more than SPECV_NOALLOC_SCRATCH bytes */

#define SPECV_MAX_K        32   /* one 64-lane wave runs the acceptance scan */
#define SPECV_MAX_TREE     64   /* token-tree nodes: one per lane of a wave */
#define SPECV_MAX_NGRAM    16   /* largest n-gram the prompt-lookup proposer matches */
#define SPECV_NOALLOC_SCRATCH (32u << 20)  /* bytes of spec_verify_noalloc's static scratch per device */

/* Flag bits of out_flags.  SPECV_FLAG_FP64 reports which path drew the
 * token, not what was drawn: on batches of at most 128 sequences, where one
 * sequence's draw is shared by several workgroups, a workgroup that still
 * cannot see another's published sums after a short bounded wait hands the
 * draw to the fp64 path, so in principle this bit may differ between two
 * identical calls.  The tokens, the counts and the other bits never do (the
 * fp64 path draws the same token wherever the fast one is certified).  Rows
 * of at most 2048 tokens take one launch that draws every token in fp64
 * (see spec_short_max_seqs): there the bit is set on every sequence. */
#define SPECV_FLAG_FP64      1  /* the draw was made by the fp64 path: the fp32 draw could not certify its token */
#define SPECV_FLAG_ZW_ZERO   2  /* residual mass was zero after rounding; drew from p_n instead */
#define SPECV_FLAG_BAD_DRAFT 4  /* an evaluated draft id was outside [0, V) and was rejected */

/*
 * Bytes of workspace spec_verify needs for this shape.  Returns 0 when the
 * shape or dtype is invalid.  T selects the mode: greedy (T == 0) needs less.
 */
size_t spec_verify_workspace_size(int B, int K, int V, int dtype, float T);

/*
 * spec_verify - one verify step for B sequences of K draft tokens.
 *
 * Sampling mode (T > 0).  With p_k = softmax(logits_p[b][k] / T) and
 * q_k = softmax(logits_q[b][k] / T) ([A] "Toán học của sự miễn phí";
 * [B] "拒绝采样"; [D] "Математическая гарантия"), draft token x_k =
 * draft_tokens[b][k] is accepted iff u_accept[b][k] < min(1, p_k(x_k)/q_k(x_k))
 * ([B] "验收标准的精确数学", equation alpha(x)), scanning k = 0, 1, ... and
 * stopping at the first rejection n ([B] "多 Token 验证：左到右，遇错即停").
 * At n < K the emitted token is drawn from max(0, p_n - q_n)/Z ([B]
 * "拒绝之后怎么办？——残差分布", equations p_resid and Z; [D] equation r(x));
 * at n == K it is drawn from p_K (the bonus token: [A] third rule of the
 * acceptance procedure; [B] "多 Token 验证", fourth step).  The draw is an
 * inverse CDF: the smallest token v, in ascending id order, whose running
 * weight sum exceeds u_resample[b] times the total.
 *
 * Greedy mode (T == 0).  a_k = first index of the maximum of logits_p[b][k];
 * accept while a_k == x_k; emit a_n ([C] section 9.1 greedy matching;
 * [D] "Механизм «черновик — проверка»", longest matching prefix).
 * logits_q, u_accept and u_resample are not read and may be NULL.
 *
 * Outputs: out_tokens[b] = x_0..x_{n-1}, the drawn token, then -1 padding;
 * out_n_accepted[b] = n in [0, K] ([B] "多 Token 验证": one to k+1 tokens).
 *
 * Rows past a sequence's first rejection are never needed.  When the logit
 * rows total at least 256 MiB (B*(2K+1)*V*element_size; B*(K+1)*V*... in
 * greedy mode), the rows are read in rounds of positions 0, 1-2 and 3-K, and
 * a round skips the sequences that rejected in an earlier one; smaller
 * inputs are read in one sweep.  The environment variable
 * SPECV_ROUNDS_MIN_BYTES, read once per process, replaces that threshold (0:
 * always rounds).  Both ways give identical outputs.  spec_verify_ex and
 * spec_verify_ragged_ex with out_logz always read every row.
 *
 * logits_p      [B][K+1][V] target logits (dtype)
 * logits_q      [B][K][V]   draft logits (dtype); may be NULL iff T == 0
 * draft_tokens  [B][K] int32
 * u_accept      [B][K] float in (0,1); may be NULL iff T == 0
 * u_resample    [B]    float in (0,1); may be NULL iff T == 0
 * T             temperature: 0 = greedy, else finite and > 0
 * B, K, V       1 <= K <= SPECV_MAX_K, B >= 1, V >= 1
 * out_tokens    [B][K+1] int32 (written)
 * out_n_accepted[B] int32 (written)
 * dtype         SPECV_F32 or SPECV_BF16
 * workspace     device scratch of workspace_bytes >= spec_verify_workspace_size()
 * stream        hipStream_t (as void*); NULL = null stream
 * Returns SPECV_OK or a negative SPECV_E_* code.
 */
int spec_verify(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_noalloc - spec_verify for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace, the same kernels and
 * results.  Its scratch is a static device array of SPECV_NOALLOC_SCRATCH
 * bytes that the library holds on each device it runs on until the process
 * ends; its address is looked up on the first call on a device.  Shapes
 * whose workspace (spec_verify_workspace_size) exceeds it return
 * SPECV_E_SCRATCH with nothing enqueued; the five workloads of this library's
 * tests need at most about 16 MB.  It calls no allocator.  Every call on one
 * device shares that scratch: calls that may overlap on one device (other
 * streams, other threads) race and must be serialised by the caller.  Each
 * call resets what it needs inside its own kernels, so no clearing is
 * required between calls.
 */
int spec_verify_noalloc(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                        const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                        int32_t* out_tokens, int32_t* out_n_accepted, int dtype, void* stream);

/*
 * spec_verify_ex - spec_verify plus diagnostics for tests and benchmarks.
 *
 * out_logz    [B][2K+1] float or NULL: natural-log normalisers
 *             log sum_v exp(logit/T), K+1 target rows then K draft rows
 *             (sampling mode only; untouched when T == 0).
 * out_flags   [B] int32 or NULL: SPECV_FLAG_* bits per sequence.
 * ev_sweep_begin, ev_sweep_end
 *             hipEvent_t (as void*) or NULL: when both are given they are
 *             recorded with the first and the last row-sweep dispatch of the
 *             call, so a caller can time the row sweep alone.
 */
int spec_verify_ex(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                   const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                   int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream,
                   float* out_logz, int32_t* out_flags, void* ev_sweep_begin, void* ev_sweep_end);

/* spec_verify_ex with every row-sweep launch of the call timed on its own,
 * for a benchmark's per-kernel roofline.  ev_begin[i] and ev_end[i]
 * (hipEvent_t handles, as void*) are recorded with the start and the end of
 * the call's i-th sweep launch (one launch when every row is swept at once,
 * up to three when the rows are read in rounds); launches from n_events on
 * are not timed, and the acceptance launches between rounds lie outside every
 * pair.  *n_sweeps (host memory, or NULL) receives the number of sweep
 * launches.  Returns what spec_verify_ex returns, or SPECV_E_SHAPE for
 * n_events < 0 and SPECV_E_NULL when n_events > 0 and an event array is NULL. */
int spec_verify_sweep_timed(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                            const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                            int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream,
                            float* out_logz, int32_t* out_flags, void* const* ev_begin, void* const* ev_end,
                            int n_events, int* n_sweeps);

/*
 * spec_verify_ragged - spec_verify with a draft count per sequence, and
 * optional per-position acceptance counters.
 *
 * num_drafts     [B] int32 (device): sequence b uses its first K_b drafts,
 *                0 <= K_b <= K (values outside are clamped), as when the
 *                draft length is adapted per sequence ([B] "最优猜测长度 k：
 *                贪心还是保守？", adaptive k).  Layouts stay those of
 *                spec_verify, padded to K: target rows past K_b, draft rows,
 *                drafts and accept uniforms past K_b - 1 are not read.  A
 *                sequence that accepts all K_b drafts takes its bonus token
 *                from target row K_b.  out_tokens keeps K+1 entries per
 *                sequence, -1 after the emitted token.
 * position_stats [2K] uint64 (device) or NULL: counters this call adds to
 *                (the caller zeroes them once): position_stats[k] counts the
 *                sequences whose draft k was tested (k <= n and k < K_b),
 *                position_stats[K + k] those whose draft k was accepted
 *                (k < n).  Acceptance by draft position is what [D] "Когда
 *                процент принятия падает" and "Мониторинг в производстве"
 *                watch.  Calls adding to the same counters must not overlap.
 * All other arguments, the workspace size and the return codes are those of
 * spec_verify; num_drafts may not be NULL.
 */
int spec_verify_ragged(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                       const int32_t* num_drafts, const float* u_accept, const float* u_resample, float T,
                       int B, int K, int V, int32_t* out_tokens, int32_t* out_n_accepted,
                       uint64_t* position_stats, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * spec_verify_ragged_ex - spec_verify_ragged plus the diagnostics of
 * spec_verify_ex: out_logz [B][2K+1] float or NULL (natural-log normalisers,
 * K+1 target rows then K draft rows; the rows a sequence does not use, past
 * its K_b, are not written; untouched when T == 0) and out_flags [B] int32
 * or NULL (SPECV_FLAG_* bits).
 */
int spec_verify_ragged_ex(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                          const int32_t* num_drafts, const float* u_accept, const float* u_resample, float T,
                          int B, int K, int V, int32_t* out_tokens, int32_t* out_n_accepted,
                          uint64_t* position_stats, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream, float* out_logz, int32_t* out_flags);

/*
 * Token trees ([A] "Token tree: kiểm nhiều nhánh đoán cùng lúc"; [C] sections
 * 3.1, 3.2, 8 and 9.1).  A tree of N nodes (1 <= N <= SPECV_MAX_TREE) is
 * parents [N] int32 with parents[0] == -1 (node 0, the root, holds the last
 * committed token) and parents[v] < v, plus a token per node; row v of the
 * logits scores the token after node v.  A node whose parent is not in
 * [0, v) sees only itself, has depth 0 and is never accepted.
 *
 * spec_verify_tree_greedy - greedy verification of B trees.  Node v is
 * accepted when its parent is and its token is the first arg-max of its
 * parent's row; the round's output is the path from the root to the deepest
 * accepted node d (the lowest index among equally deep ones), then the
 * first arg-max of row d ([A]: the deepest accepted branch is the output;
 * [C] 9.1: greedy matching, which is exact for T = 0).
 *   logits         [B][N][V] target logits (dtype), aligned to the element size
 *   tree_tokens    [B][N] int32; parents [B][N] int32
 *   out_tokens     [B][N] int32: the path's tokens after the root, the bonus
 *                  token, then -1
 *   out_path       [B][N] int32 or NULL: node indices of the path (root
 *                  first), then -1 (which nodes' cache entries to keep)
 *   out_n_accepted [B] int32: accepted drafts = depth of d
 *   workspace      spec_verify_tree_workspace_size() bytes, 256-byte aligned
 * Returns the SPECV_* codes of spec_verify; nothing synchronises.
 */
size_t spec_verify_tree_workspace_size(int B, int N, int V, int dtype);

int spec_verify_tree_greedy(const void* logits, const int32_t* tree_tokens, const int32_t* parents, int B, int N,
                            int V, int32_t* out_tokens, int32_t* out_path, int32_t* out_n_accepted, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_tree_mask - the tree attention mask and depth position ids of B trees
 * ([C] 3.1: a node sees the shared prefix and its own ancestors only; 3.2:
 * its position id is its depth; 8: worked example).
 *   parents   [B][N] int32 (device)
 *   out_mask  [B][N][N] uint8 or NULL: out_mask[b][i][j] = 1 when node i may
 *             attend to node j (j is i or an ancestor of i), else 0
 *   out_depth [B][N] int32 or NULL: depth of every node (root 0)
 * At least one output must be given.  Needs no workspace.
 */
int spec_tree_mask(const int32_t* parents, int B, int N, uint8_t* out_mask, int32_t* out_depth, void* stream);

/*
 * spec_ngram_propose - n-gram (prompt-lookup) drafts from the token history
 * of B sequences ([D] "Спекулятивное декодирование на n-граммах": when the
 * latest tokens repeat an earlier n-gram, propose what followed it, with an
 * n-gram size and a minimum number of hits; [A]: Prompt Lookup, drafts taken
 * from the context).  For sizes n = n_max down to n_min, an occurrence of the
 * history's last n tokens ends at e (1 <= e <= L - 1: a token follows it);
 * the largest n with at least min_hits occurrences wins, and the draft is
 * the K tokens after its latest occurrence, cut at the end of the history.
 *   history   [B][L_max] int32 (device), row b valid for its first lengths[b]
 *   lengths   [B] int32 (device), clamped to [0, L_max]
 *   n_min, n_max   1 <= n_min <= n_max <= SPECV_MAX_NGRAM
 *   min_hits  >= 1;  K  1 <= K <= SPECV_MAX_K
 *   out_draft [B][K] int32: the draft, then -1;  out_count [B] int32: its length (0: none)
 * Returns SPECV_OK, SPECV_E_NULL or SPECV_E_SHAPE (any size out of range);
 * needs no workspace; nothing synchronises.
 */
int spec_ngram_propose(const int32_t* history, const int32_t* lengths, int B, int L_max, int n_min, int n_max,
                       int min_hits, int K, int32_t* out_draft, int32_t* out_count, void* stream);

/*
 * spec_rounds_min_bytes - the input size from which the verify calls read
 * logit rows in rounds and skip the rows past each sequence's first
 * rejection (and token trees the rows below a rejected node): checking
 * stops there ([B] "多 Token 验证：左到右，遇错即停").  Smaller inputs take one
 * sweep of every row, whose fewer launches cost less than the rows they would
 * skip.  The default is 256 MiB of logit rows, or SPECV_ROUNDS_MIN_BYTES from
 * the environment at the first use.  bytes >= 0 sets the threshold for the
 * process and returns the previous one; a negative (or non-finite) value only
 * returns it.  Both ways give the same outputs.
 */
double spec_rounds_min_bytes(double bytes);

/*
 * spec_short_max_seqs - the largest batch whose sampling calls on rows of at
 * most 2048 tokens take the one-launch path (one workgroup per sequence does
 * every step: normalisers, acceptance test of u_k < min(1, p_k(x_k) /
 * q_k(x_k)) ([B] "验收标准的精确数学") and the residual or bonus draw in fp64
 * ([B] "拒绝之后怎么办？——残差分布")); larger batches take the general path
 * (row sweep, per-sequence fast draw, fp64 draw for what it cannot
 * certify).  The default is no limit (INT_MAX), or SPECV_SHORT_MAX_SEQS from
 * the environment at the first use.  n >= 0 sets the limit for the process
 * (0: the general path always) and returns the previous one; a negative value
 * only returns it.  Both paths compute the same method; their fp32
 * normalisers round differently, so a count (and then the token) can differ
 * only where an acceptance test is a near-tie, and SPECV_FLAG_FP64 differs
 * (see there).  Thread-safe; a call already under way keeps the path it took.
 */
int spec_short_max_seqs(int n);

/*
 * The n-gram map: spec_ngram_propose's proposals kept up to date in a hash
 * table per sequence instead of rescanning the history on every call ([D]
 * "Спекулятивное декодирование на n-граммах": the map variants key a hash
 * table by the current n-gram and keep what followed it, for a lookup in
 * place of the linear scan).  A table holds, for every n-gram of the sizes in
 * use that a token follows, its count and its latest end; a call adds the
 * n-grams whose following token is new and looks up the current suffix, so
 * its cost follows the tokens added, not the history's length.
 *
 * spec_ngram_map_bytes - device bytes of B tables of `capacity` slots each
 * (16 bytes a slot, plus 16 per table); 0 unless 1 <= B and capacity is a
 * power of two in [SPECV_NGRAM_MAP_MIN_SLOTS, SPECV_NGRAM_MAP_MAX_SLOTS].  A
 * table stays correct while it holds at most about half as many distinct
 * n-grams as slots (n_max - n_min + 1 per token of history, at most).
 */
#define SPECV_NGRAM_MAP_MIN_SLOTS 64
#define SPECV_NGRAM_MAP_MAX_SLOTS (1 << 28)
#define SPECV_NGRAM_MAP_FULL      1   /* out_status: an insert found no free slot; the table is too small */
size_t spec_ngram_map_bytes(int B, int capacity);

/*
 * spec_ngram_map_update - add each sequence's new tokens to its table and
 * propose drafts from it.  For sequence b with previous length len_old[b] and
 * length now len_new[b] (both clamped to [0, L_max], len_old to at most
 * len_new): when len_old[b] is 0 its table is cleared and built from the
 * whole history; otherwise the n-grams of sizes n_min..n_max ending at
 * positions len_old[b] .. len_new[b] - 1 (those whose following token arrived
 * since the previous call) are added.  Then the draft is what
 * spec_ngram_propose returns for the history h[0..len_new[b]) with the same
 * n_min, n_max, min_hits and K, unless two different n-grams of one history
 * share a 64-bit key (probability about N^2 / 2^65 for N n-grams).
 *   tables    spec_ngram_map_bytes(B, capacity) bytes of device memory, 16-byte
 *             aligned, owned by the caller and kept between calls; its
 *             contents are valid only for the same capacity, n_min and n_max,
 *             and only when len_old[b] is the len_new[b] of the previous call
 *             (or 0)
 *   history, L_max, n_min, n_max, min_hits, K, out_draft, out_count: as for
 *             spec_ngram_propose
 *   len_old, len_new  [B] int32 (device)
 *   out_status [B] int32 or NULL: 0, or SPECV_NGRAM_MAP_FULL when the table
 *             has overflowed (since it was last built): then no draft is
 *             proposed (count 0) until a call with len_old[b] == 0 rebuilds it
 * Returns SPECV_OK, SPECV_E_NULL, SPECV_E_SHAPE (a size out of range, or
 * spec_ngram_map_bytes(B, capacity) == 0), SPECV_E_ALIGN (tables) or
 * SPECV_E_HIP; needs no workspace; nothing synchronises.  Calls on one table
 * must not overlap.
 */
int spec_ngram_map_update(void* tables, int capacity, const int32_t* history, const int32_t* len_old,
                          const int32_t* len_new, int B, int L_max, int n_min, int n_max, int min_hits, int K,
                          int32_t* out_draft, int32_t* out_count, int32_t* out_status, void* stream);

/* Device-side input validation, a debugging aid.  While it is on, every
 * spec_verify* call (spec_verify, _ex, _noalloc, _ragged, _ragged_ex) first
 * runs one more pass over the inputs it uses and adds what it finds to
 * counters kept on the current device, in this order:
 *   SPECV_DBG_CALLS             calls validated
 *   SPECV_DBG_BAD_DRAFT_IDS     draft ids outside [0, V) at positions 0 .. K_b - 1
 *   SPECV_DBG_BAD_U_ACCEPT      accept uniforms outside (0, 1) (NaN included), same positions
 *   SPECV_DBG_BAD_U_RESAMPLE    resample uniforms outside (0, 1)
 *   SPECV_DBG_NAN_LOGITS        NaN logits in the rows the call reads
 *   SPECV_DBG_INF_LOGITS        +inf logits in those rows
 *   SPECV_DBG_ROWS_NO_FINITE    rows among them without a finite logit
 * (the uniforms are counted in sampling mode only; the rows a call reads are
 * target rows 0 .. K_b and draft rows 0 .. K_b - 1 of each sequence).  The
 * verify step still runs on such inputs, with unspecified tokens and never an
 * out-of-bounds access.  The pass reads every used logit once more, so it is
 * for debugging, not for timing.  The environment variable SPECV_DEBUG=1,
 * read at the first call, turns validation on; spec_debug_enable overrides it.
 * The counters are per-device state of the library: calls on one device that
 * overlap in time add to the same counters. */
#define SPECV_DEBUG_COUNTERS      7
#define SPECV_DBG_CALLS           0
#define SPECV_DBG_BAD_DRAFT_IDS   1
#define SPECV_DBG_BAD_U_ACCEPT    2
#define SPECV_DBG_BAD_U_RESAMPLE  3
#define SPECV_DBG_NAN_LOGITS      4
#define SPECV_DBG_INF_LOGITS      5
#define SPECV_DBG_ROWS_NO_FINITE  6

/* Turn validation on (on != 0) or off for later calls; returns the previous
 * setting (0 or 1). */
int spec_debug_enable(int on);

/* Copy the current device's first n counters (1 <= n <= SPECV_DEBUG_COUNTERS)
 * to host memory `out`, after the device's work so far has finished (it
 * synchronises the device).  Returns SPECV_OK, SPECV_E_NULL, SPECV_E_SHAPE (n
 * out of range) or SPECV_E_HIP. */
int spec_debug_counters(unsigned long long* out, int n);

/* Zero the current device's counters (synchronising the device).  Returns
 * SPECV_OK or SPECV_E_HIP. */
int spec_debug_reset(void);

/* Static description of a return code. */
const char* spec_verify_strerror(int code);

/* Library version string, e.g. "libspecverify 0.1 gfx950". */
const char* spec_verify_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
