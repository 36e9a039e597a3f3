/*
 * treedraft.h -- C ABI of the MI355X (gfx950) verify-side path of budget-aware
 * tree speculative decoding over block-diffusion drafts.
 *
 * The method (BASTION: "Bastion: Budget-Aware Speculative Decoding with
 * Tree-structured Block Diffusion Drafting", technical summary, "Methodik")
 * turns the drafter's per-position marginals q_k into a prefix-closed draft
 * tree, sizes the tree with an online budget controller, and has the target
 * verify the whole tree in one parallel pass.  The five calls below are the
 * steps of one verify step:
 *
 *   td_draft_topk        log-softmax normaliser and top-K of every position
 *   td_build_tree        best-first tree with the S(N) stop
 *   td_tree_mask         bit-packed ancestor-or-self masks
 *   td_tree_verify_attn  tree attention against context KV + tree KV
 *   td_accept            greedy acceptance walk and bonus token
 *
 * Conventions shared by every call
 *  - Every array pointer is DEVICE memory owned by the caller, unless a
 *    comment says otherwise.  The library allocates nothing and keeps no
 *    state besides a thread-local error string.
 *  - Launch plans (slices per logit row, key chunks per context) are sized
 *    for the 256 compute units of the MI355X (gfx950); they stay correct on
 *    a part with another count, only less well balanced.
 *  - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *    NULL = the default stream).  TD_OK means "validated and enqueued".
 *    Tree sizes (n_nodes) stay on the device: no call waits for the host.
 *  - Validation runs first; on any status other than TD_OK nothing was
 *    enqueued and td_last_error() describes the problem.
 *  - All arrays are C-contiguous in the layouts stated per call.
 *  - bf16 is IEEE binary32 truncated to its upper 16 bits (bfloat16).
 *  - Calls are reentrant; concurrent calls on different streams are safe as
 *    long as they do not share output or workspace buffers.
 */
#ifndef TREEDRAFT_H
#define TREEDRAFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TD_ABI_VERSION 2

/* Compiled capacities. */
#define TD_MAX_TOPK 32        /* K */
#define TD_MAX_BLOCK 32       /* drafter block positions B */
#define TD_MAX_NODES 255      /* n_max: draft nodes per tree (root excluded) */
#define TD_MAX_VOCAB 262144   /* token ids must fit in 18 bits */
#define TD_MAX_BATCH 4096

typedef enum {
    TD_OK = 0,
    TD_EINVAL = 1,        /* null pointer, bad size, misaligned buffer, too small workspace */
    TD_ECAPACITY = 2,     /* a size above the compiled capacities */
    TD_EUNSUPPORTED = 3,  /* dtype / head_dim combination not built */
    TD_EHIP = 4,          /* the HIP runtime reported an error */
    TD_ESYNC = 5          /* td_workspace_status: a cross-workgroup hand-off gave up */
} td_status;

typedef enum { TD_F32 = 0, TD_BF16 = 1 } td_dtype;

int td_abi_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *td_last_error(void);

/* ------------------------------------------------------------------------
 * td_draft_topk -- stage (a).
 * The path score of a tree node is the product of the drafter's marginals
 * q_k along its path (Methodik §1, path scoring).  For every (sequence b,
 * block position k) this computes, over the FULL vocabulary:
 *   lse[b][k]        = log sum_v exp(l[b][k][v])                 (float64)
 *   topk_id[b][k][j] = the j-th largest logit's token id; ties go to the
 *                      smaller id; j = 0..K-1                     (int32)
 *   topk_logq[b][k][j] = l[b][k][topk_id] - lse[b][k] = log q_k    (float64)
 * Inputs:
 *   logits      [batch][block][*] with row (b,k) starting at element
 *               (b*block + k) * pos_stride; vocab entries per row are used.
 *               dtype TD_F32 or TD_BF16.  The base pointer must be aligned
 *               to the element size (rows aligned to 16 bytes stream fastest).
 *   1 <= K <= min(TD_MAX_TOPK, vocab); 1 <= block <= TD_MAX_BLOCK.
 * Workspace: at least td_draft_topk_workspace(batch, block, vocab, K) bytes
 *   of device memory, 16-byte aligned.  It must be ZERO-FILLED before its
 *   first use and again whenever batch, block, vocab or K change (it holds
 *   the workgroups' call epochs, which tag the partial results they hand
 *   over); every call leaves it ready for the next call of the same shape.
 *   Calls that overlap in time must not share a workspace.  A broken
 *   hand-off is reported by td_workspace_status (lse of the row is NaN).
 */
size_t td_draft_topk_workspace(int32_t batch, int32_t block, int32_t vocab, int32_t K);
td_status td_draft_topk(const void *logits, td_dtype dtype, int32_t batch, int32_t block,
                        int32_t vocab, int64_t pos_stride, int32_t K, int32_t *topk_id,
                        double *topk_logq, double *lse, void *workspace,
                        size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * td_workspace_status -- did a call that used this workspace give up waiting?
 * The top-K kernel and the verify step's first kernel hand partial results
 * from workgroup to workgroup through the workspace (epoch-tagged words).  A
 * waiter polls a bounded number of times; if the words never arrive (the
 * workspace was not zero-filled after a shape change, two overlapping calls
 * shared it, or the GPU started the waiting workgroups before the ones they
 * wait for and those could not run) it gives up instead of hanging:
 *   - a row merger writes lse = NaN for its row (its ids and log q are then
 *     meaningless), and
 *   - a tree builder writes n_nodes = -1 for its sequence (its tree entries
 *     are then meaningless; the verify step's attention then writes no
 *     row and its acceptance reports A = 0 with the root's target token),
 * and each sets a bit in a status word at the start of the workspace.
 * This call waits for `stream`, reads that word and clears it: TD_OK if no
 * call gave up since the last check, TD_ESYNC otherwise (td_last_error()
 * names the failed hand-offs).  It synchronises the stream; a serving loop
 * calls it when it reads results back.  workspace: a workspace of
 * td_draft_topk or td_verify_step (not of td_tree_verify_attn).
 */
td_status td_workspace_status(void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * td_build_tree -- stage (b).
 * Best-first construction of the prefix-closed draft tree (Methodik §2):
 * starting from the root (the last verified token, depth 0, rho = 1), the
 * valid candidate with the largest path score rho is added until the budget
 * is used.  The children of a node at depth d are the top-K tokens of
 * position d+1, with log rho(child) = log rho(node) + log q_{d+1}(token).
 * Candidates are ordered by log rho descending, then depth ascending, then
 * token id ascending, then parent index ascending (a total order).
 * With use_stop != 0 the online budget controller (Methodik §3) inserts the
 * next candidate only while the estimated speedup rises:
 *   A_hat(n) = ahat0 + sum_{i=1..n} rho(i),
 *   C(n)     = cost_a + cost_b*n + cost_c*max(0, n - cost_knee),
 *   S(n)     = A_hat(n) * l_ar / C(n),
 * stopping before node n+1 when S(n+1) <= S(n).  Otherwise exactly
 * min(n_max, available candidates) nodes are inserted.  log rho, A_hat and S
 * are accumulated in float64.
 * Selective verification (the FlexDraft page, Methodik §3, Flex-Decoding:
 * branches of low cumulative draft confidence are pruned; a node's
 * cumulative confidence is its path score rho): when min_logrho < 0 no
 * node with log rho < min_logrho is inserted (0, positive or -INFINITY:
 * no threshold, so a zero-filled argument block prunes nothing); since the
 * best candidate bounds
 * all others, growth stops at the first best candidate below it.  branch
 * (1..K; other values mean K) caps the children per node at the ranks
 * 0..branch-1 of the next position; branch = 1 drafts the single top-1
 * branch of the sequential mode (see td_flex_budget).
 * Inputs:  topk_id [batch][block][K], topk_logq [batch][block][K] as written
 *          by td_draft_topk (ids in [0, TD_MAX_VOCAB); the kernel uses the
 *          low 18 bits of each id); root_token [batch] or NULL (then -1 is
 *          stored).
 * Outputs (index 0 = root; nodes in insertion order, parent index < child):
 *   n_nodes     [batch]           number of draft nodes N (root excluded)
 *   node_token  [batch][n_max+1]  token id (-1 beyond N)
 *   node_parent [batch][n_max+1]  parent index (-1 for the root and beyond N)
 *   node_depth  [batch][n_max+1]  depth (-1 beyond N)
 *   node_logrho [batch][n_max+1]  log rho (0 for the root and beyond N)
 *   ahat        [batch]           A_hat(N)                     (may be NULL)
 *   speedup     [batch]           S(N)                         (may be NULL)
 * 0 <= n_max <= TD_MAX_NODES.
 */
td_status td_build_tree(const int32_t *topk_id, const double *topk_logq, int32_t batch,
                        int32_t block, int32_t K, int32_t n_max, int32_t use_stop, double cost_a,
                        double cost_b, double cost_c, int32_t cost_knee, double l_ar,
                        double ahat0, int32_t branch, double min_logrho,
                        const int32_t *root_token, int32_t *n_nodes,
                        int32_t *node_token, int32_t *node_parent, int32_t *node_depth,
                        double *node_logrho, double *ahat, double *speedup, void *stream);

/* ------------------------------------------------------------------------
 * td_flex_budget -- the batch-size switch of the FlexDraft page (Methodik §3,
 * Flex-Decoding, dynamic switching): small batches verify the whole tree,
 * large ones a single branch drafted from the verified prefix.  Host
 * function (no GPU work): for a step of `batch` sequences, writes *branch =
 * K and *n_max_out = n_max when switch_batch <= 0 or batch < switch_batch,
 * else *branch = 1 and *n_max_out = min(n_max, block).  Pass both to
 * td_build_tree / td_step_args.  Either pointer may be NULL.
 */
void td_flex_budget(int32_t batch, int32_t switch_batch, int32_t K, int32_t n_max, int32_t block,
                    int32_t *branch, int32_t *n_max_out);

/* ------------------------------------------------------------------------
 * td_fit_cost -- the tachometer's fit (Methodik §3, latency modelling: a
 * roofline model of the verification latency, calibrated on observed
 * runtimes).  Host function; every pointer is HOST memory.  Fits
 *   C(N) = a + b N + c max(0, N - knee)
 * to count >= 3 measured pairs (n[i] draft nodes, t[i] verification time)
 * by least squares: every integer knee in [knee_min, knee_max] is tried and
 * the smallest residual sum of squares wins (equal sums: the smaller knee;
 * a knee at or past every n[i] fits c = 0).  Writes a, b, c, knee and, if
 * rss is not NULL, the residual sum.  For td_build_tree's stop, pass the
 * coefficients as they are with l_ar = a (the one-token step), or divided
 * by a with l_ar = 1.
 */
td_status td_fit_cost(const double *n, const double *t, int32_t count, int32_t knee_min,
                      int32_t knee_max, double *a, double *b, double *c, int32_t *knee,
                      double *rss);

/* ------------------------------------------------------------------------
 * td_tree_mask -- stage (b').
 * The draft tree is prefix-closed (Methodik §1, marginal independence: the
 * per-position candidates combine freely into a prefix tree), and the target
 * verifies all its nodes in one parallel pass (Problemstellung), so each
 * node's query may see exactly the tokens of its own prefix: the context and
 * the tree nodes on its root path.  This call writes that set as a bit-packed
 * ancestor-or-self mask of every tree row: bit j of row i is set iff node j
 * lies on the root path of node i (i included).  Row i = row(parent(i)) |
 * (1 << i).
 * Inputs:  node_parent [batch][nq_max], n_nodes [batch] (nq_max = n_max+1).
 * Output:  mask [batch][nq_max][words], words = (nq_max + 63) / 64; bit j of
 *          a row is bit (j % 64) of word j / 64.  Rows beyond n_nodes are 0.
 */
td_status td_tree_mask(const int32_t *node_parent, const int32_t *n_nodes, int32_t batch,
                       int32_t nq_max, uint64_t *mask, void *stream);

/* ------------------------------------------------------------------------
 * td_tree_verify_attn -- stage (c).
 * The target verifies the whole tree in one parallel pass (Methodik; tree
 * verification).  For sequence b, query head h and tree row i <= n_nodes[b]:
 *   out[b][i][h] = sum_j softmax_j(scale * q[b][i][h] . k_j) v_j
 * over the admitted keys j: all context keys of b, plus the tree keys whose
 * bit is set in mask row (b, i).  KV head of query head h is h / (hq/hkv).
 * Rows i > n_nodes[b] of out are not written (their contents are left as
 * they were): only the tree's rows are verified.
 * Inputs:
 *   q        [batch][nq_max][hq][head_dim]
 *   k_ctx, v_ctx [total_ctx][hkv][head_dim]; sequence b owns the region of
 *            rows ctx_offsets[b] .. ctx_offsets[b+1]-1 (ctx_offsets int64
 *            [batch+1], device, non-decreasing, ctx_offsets[0] = 0,
 *            ctx_offsets[batch] = total_ctx).  Its context is the whole
 *            region when ctx_lengths is NULL, else the region's first
 *            ctx_lengths[b] rows (int64 [batch], device; values are clamped
 *            to [0, region size]); the rest of a region is room for tokens
 *            that td_kv_commit appends.  max_ctx is not used.
 *   k_tree, v_tree [batch][nq_max][hkv][head_dim]
 *   mask     as written by td_tree_mask; n_nodes [batch].
 *   dtype TD_BF16 or TD_F32 (all of q/k/v/out); head_dim 64 or 128.
 *   Accumulation is float32; out has the input dtype.
 * Workspace: td_tree_verify_attn_workspace(...) bytes, 16-byte aligned
 *   (per-chunk partial results; no state is kept between calls).  Calls
 *   that overlap in time must not share a workspace.
 */
size_t td_tree_verify_attn_workspace(int32_t batch, int32_t nq_max, int32_t hq, int32_t hkv,
                                     int32_t head_dim, int64_t total_ctx, int64_t max_ctx);
td_status td_tree_verify_attn(const void *q, const void *k_ctx, const void *v_ctx,
                              const int64_t *ctx_offsets, const int64_t *ctx_lengths,
                              int64_t total_ctx, int64_t max_ctx,
                              const void *k_tree, const void *v_tree, const uint64_t *mask,
                              const int32_t *n_nodes, int32_t batch, int32_t nq_max, int32_t hq,
                              int32_t hkv, int32_t head_dim, float scale, td_dtype dtype,
                              void *out, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * td_accept -- stage (d).
 * Greedy verification at temperature 0 (Experimental results: greedy
 * decoding): from the root, step to the child whose token equals the
 * target's greedy token at the current node, while one exists.  The number
 * of steps is the accepted length A; the target's token at the last
 * accepted node is the bonus token (the correct token at the first
 * rejection point).
 * Inputs:  node_token, node_parent [batch][n_max+1], n_nodes [batch] as
 *          written by td_build_tree (siblings carry distinct tokens);
 *          target_token [batch][n_max+1]: the target's greedy token at every
 *          node 0..n_nodes[b].
 * Outputs: accept_len [batch]; accept_path [batch][block+1]: node indices,
 *          root first, -1 padded; bonus_token [batch].
 */
td_status td_accept(const int32_t *node_token, const int32_t *node_parent, const int32_t *n_nodes,
                    const int32_t *target_token, int32_t batch, int32_t n_max, int32_t block,
                    int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token,
                    void *stream);

/* ------------------------------------------------------------------------
 * td_kv_commit -- after stage (d): the accepted prefix becomes context.
 * The target verified every tree node in one pass and decoding continues
 * from the accepted prefix (Problemstellung); the keys and values that pass
 * computed for the prefix's tokens are kept rather than recomputed (the
 * FlexDraft page, Methodik §3, decoupled execution: the verification's KV
 * cache is reused).  For sequence b with accepted length A = accept_len[b]
 * and path p_0 = 0 (the root), p_1 .. p_A = accept_path[b][0..A]: the tree
 * rows p_0 .. p_A of k_tree / v_tree (every KV head) are copied, in that
 * order, to rows ctx_offsets[b] + L_b, ... of k_cache / v_cache, where
 * L_b = ctx_lengths[b]; then ctx_lengths[b] += A + 1 and next_root[b] =
 * bonus_token[b] (the bonus token is the next step's root).  Rows that
 * would pass the end of b's region (ctx_offsets[b+1]) are not written and
 * ctx_lengths[b] stops at the region's size; a region with room for
 * block + 1 more rows never overflows.
 * Inputs:  k_tree, v_tree [batch][nq_max][hkv][head_dim] (the tree rows
 *          given to td_tree_verify_attn); accept_len [batch], accept_path
 *          [batch][block+1], bonus_token [batch] as written by td_accept
 *          (path entries outside [0, nq_max) end the copy).
 * In/out:  k_cache, v_cache [total][hkv][head_dim] (the context arrays of
 *          td_tree_verify_attn; same dtype as the tree rows); ctx_lengths
 *          [batch] int64.  ctx_offsets [batch+1] as for the attention.
 * Output:  next_root [batch] (may be NULL).
 * dtype TD_BF16 or TD_F32; head_dim 64 or 128; 16-byte aligned arrays.
 */
td_status td_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accept_len,
                       const int32_t *accept_path, const int32_t *bonus_token, int32_t batch,
                       int32_t nq_max, int32_t block, int32_t hkv, int32_t head_dim,
                       td_dtype dtype, void *k_cache, void *v_cache, const int64_t *ctx_offsets,
                       int64_t *ctx_lengths, int32_t *next_root, void *stream);

/* ------------------------------------------------------------------------
 * The verification pass, one layer (a stand-in for the target model; the
 * pages fix no model).  The target scores every tree node in one parallel
 * pass (Problemstellung) and acceptance compares its greedy token at each
 * node (Experimentelle Ergebnisse: temperature 0).  These two calls give a
 * one-layer target over the tree, with weights the caller provides:
 *   td_tree_qkv        inputs of td_tree_verify_attn from the tree tokens;
 *   td_lm_head_argmax  target_token of td_accept from the attention output.
 * Readings: node i's input is the embedding row of its token; Q, K, V are
 * linear projections of it; the query and key heads get rotary position
 * embedding (rotate-half: dims j and j + D/2 of a head turn by the angle
 * pos * rope_base^(-2j/D)) at position pos = L_b + depth(i), L_b the
 * context length (tree siblings share a position); the attention output of
 * all query heads (hidden = hq * head_dim) is the final hidden state; the
 * greedy token is its argmax over the LM head (ties: smaller id).
 * All matrices are bf16, rows contiguous, 16-byte aligned; products
 * accumulate in float32; hidden must be a multiple of 128.  The workspace
 * (td_verify_layer_workspace bytes, 16-byte aligned) holds partial sums
 * only and needs no initialisation; one buffer serves both calls.
 */
size_t td_verify_layer_workspace(int32_t batch, int32_t nq_max, int32_t hq, int32_t hkv,
                                 int32_t head_dim, int32_t vocab);

/* td_tree_qkv
 * Inputs:  embed [vocab][hidden]; w_qkv [(hq + 2 hkv) head_dim][hidden]
 *          (output rows: the hq query heads, then hkv key heads, then hkv
 *          value heads, head_dim each); node_token, node_depth
 *          [batch][nq_max] and n_nodes [batch] as written by td_build_tree
 *          (the root's token must be set: pass root_token there; a token
 *          outside [0, vocab) reads embedding row 0); ctx_offsets /
 *          ctx_lengths as for td_tree_verify_attn (they give L_b).
 * Outputs: q [batch][nq_max][hq][head_dim], k_tree, v_tree
 *          [batch][nq_max][hkv][head_dim] (bf16); rows past n_nodes[b] are
 *          zero.  rope_base > 1 (Qwen3: 1e6).
 */
td_status td_tree_qkv(const void *embed, const void *w_qkv, const int32_t *node_token,
                      const int32_t *node_depth, const int32_t *n_nodes,
                      const int64_t *ctx_offsets, const int64_t *ctx_lengths, int32_t batch,
                      int32_t nq_max, int32_t vocab, int32_t hq, int32_t hkv, int32_t head_dim,
                      double rope_base, void *q, void *k_tree, void *v_tree, void *workspace,
                      size_t workspace_bytes, void *stream);

/* td_lm_head_argmax
 * Inputs:  hidden_rows [batch][nq_max][hq * head_dim] (the attention
 *          output: td_tree_verify_attn's out); w_lm [vocab][hq * head_dim];
 *          n_nodes [batch].
 * Output:  target_token [batch][nq_max]: the argmax over the vocabulary of
 *          the row's logits (float32 accumulation; equal values go to the
 *          smaller id), -1 past n_nodes[b].  The logits never reach memory.
 */
td_status td_lm_head_argmax(const void *hidden_rows, const void *w_lm, const int32_t *n_nodes,
                            int32_t batch, int32_t nq_max, int32_t hq, int32_t head_dim,
                            int32_t vocab, int32_t *target_token, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * td_verify_step -- the whole verify step, stages (a) to (d), in three
 * kernels instead of the five calls' seven: (1) top-K of every position,
 * then, by the last position of each sequence to finish, that sequence's
 * tree and mask rows; (2) the split-KV context attention; (3) the partial
 * merge with the tree keys, and the acceptance walk.  A call of both stages
 * with bf16 attention at head dim 128, topk <= 8, short contexts (key
 * chunks of 128 keys in at most about 512 work items: up to about 8192
 * context tokens in all at 8 KV heads) and at most 256 top-K workgroups
 * runs (2) inside (1), as extra workgroups that wait only for their
 * sequence's tree size: two kernels.  Every result equals
 * what the five calls above produce on the same inputs, into the same
 * output arrays (the fields below use their names, layouts and rules).
 * nq_max = n_max + 1.  target_token [batch][n_max+1] is an input: the
 * target's greedy token at every node of the tree this step builds.
 * Workspace: td_verify_step_workspace(args) bytes (a function of the shape
 * fields and attn_dtype), 16-byte aligned,
 * ZERO-FILLED before its first use and again whenever the shape fields
 * (batch, block, vocab, topk, n_max, hq, hkv, head_dim, total_ctx) change;
 * every call leaves it ready for the next call of the same shape.  Calls
 * that overlap in time must not share a workspace.  A broken hand-off is
 * reported by td_workspace_status (see there for the sentinels).
 * With commit != 0 the step also performs td_kv_commit (inside its last kernel,
 * after each sequence's acceptance walk): ctx_lengths must then be set, and
 * k_ctx / v_ctx are written (rows past each context) as k_cache / v_cache.
 * stages selects the kernels a call enqueues: TD_STEP_DRAFT (kernel 1: top-K,
 * tree, mask), TD_STEP_VERIFY (kernels 2 and 3: attention and acceptance),
 * or 0 for both.  A serving loop builds the tree with TD_STEP_DRAFT, runs the
 * target model over the tree's tokens to obtain q, k_tree, v_tree and the
 * target tokens, then calls TD_STEP_VERIFY with the same argument block and
 * workspace; a TD_STEP_VERIFY call reads the tree arrays and mask rows that
 * the earlier TD_STEP_DRAFT call wrote.  Only the fields of the selected
 * stages are checked.
 */
enum { TD_STEP_DRAFT = 1, TD_STEP_VERIFY = 2 };
typedef struct {
    /* stage (a) */
    const void *logits;
    td_dtype logits_dtype;
    int32_t batch, block, vocab;
    int64_t pos_stride;
    int32_t topk;
    /* stage (b) */
    int32_t n_max, use_stop;
    double cost_a, cost_b, cost_c;
    int32_t cost_knee;
    double l_ar, ahat0;
    const int32_t *root_token; /* may be NULL */
    int32_t branch;            /* children per node (1..topk; other values: topk) */
    double min_logrho;         /* selective verification threshold if < 0 (0: off) */
    /* stage (c) */
    const void *q, *k_ctx, *v_ctx;
    const int64_t *ctx_offsets;
    int64_t *ctx_lengths; /* [batch] or NULL (NULL: whole regions, no commit) */
    int64_t total_ctx, max_ctx;
    const void *k_tree, *v_tree;
    int32_t hq, hkv, head_dim;
    float scale;
    td_dtype attn_dtype;
    /* stage (d) */
    const int32_t *target_token;
    /* after (d): KV commit of the accepted path (td_kv_commit) */
    int32_t commit;       /* nonzero: commit; needs ctx_lengths */
    int32_t *next_root;   /* [batch] or NULL: the bonus tokens, as next roots */
    /* outputs */
    int32_t *topk_id;
    double *topk_logq, *lse;
    int32_t *n_nodes, *node_token, *node_parent, *node_depth;
    double *node_logrho, *ahat, *speedup; /* ahat, speedup may be NULL */
    uint64_t *mask;
    void *out;
    int32_t *accept_len, *accept_path, *bonus_token;
    int32_t stages; /* TD_STEP_DRAFT | TD_STEP_VERIFY; 0 means both */
} td_step_args;

/* sizeof(td_step_args), for bindings that lay the struct out themselves */
size_t td_step_args_bytes(void);
size_t td_verify_step_workspace(const td_step_args *args);
td_status td_verify_step(const td_step_args *args, void *workspace, size_t workspace_bytes,
                         void *stream);

/* ------------------------------------------------------------------------
 * td_verify_step_events -- td_verify_step with timing events attached to its
 * kernels (a measurement aid): start_event (a hipEvent_t, or NULL) is
 * recorded when the call's first kernel begins executing and stop_event
 * (hipEvent_t or NULL) when its last kernel has finished, from the kernels'
 * own dispatch timestamps, so hipEventElapsedTime(start, stop) is the
 * execution time of the call's kernels (for one kernel, its duration as a
 * kernel-trace profiler reports it; for several, from the first one's start
 * to the last one's end) without the launch gaps before them.  The events
 * must have been created by the caller (with timing enabled) on the
 * stream's device.  Not for use under stream capture.  Same arguments,
 * results and statuses as td_verify_step otherwise.
 */
td_status td_verify_step_events(const td_step_args *args, void *workspace, size_t workspace_bytes,
                                void *stream, void *start_event, void *stop_event);

/* ------------------------------------------------------------------------
 * td_verify_step_kernels -- the number of kernels td_verify_step enqueues
 * for args (a measurement aid, like the two calls below): 1 for
 * TD_STEP_DRAFT, 2 for TD_STEP_VERIFY, and for both stages 3, or 2 when the
 * context split runs inside the first kernel (see td_verify_step).  0 when
 * the shape fields are invalid.  Reads only the host-side fields.
 */
int32_t td_verify_step_kernels(const td_step_args *args);

/* ------------------------------------------------------------------------
 * td_verify_step_kernel_events -- td_verify_step_events for a range of the
 * call's kernels (0-based, in launch order): start_event is recorded when
 * kernel first_kernel begins and stop_event when kernel last_kernel ends,
 * while the whole step runs as usual.  TD_EINVAL (nothing enqueued) when
 * 0 <= first_kernel <= last_kernel < td_verify_step_kernels(args) fails.
 */
td_status td_verify_step_kernel_events(const td_step_args *args, void *workspace,
                                       size_t workspace_bytes, void *stream, int32_t first_kernel,
                                       int32_t last_kernel, void *start_event, void *stop_event);

/* ------------------------------------------------------------------------
 * td_verify_step_noalloc -- td_verify_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same kernels and results, with the workspace
 * in a static device array of the library (64 MiB per GPU, held by each GPU
 * the library runs on until the process ends) instead of a caller buffer.
 * The caller still passes every input and output through args.  The call
 * allocates nothing; on its first call on a device it looks up that
 * device's copy of the array.  Each call clears the array's hand-off words
 * itself (one small fill kernel ahead of the step's kernels, when the draft
 * stage is selected), so shape changes between calls need no caller action.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give wrong results; a
 * draft-only call and its verify-only call may be split as in
 * td_verify_step.  Hand-off failures show only as the sentinels described
 * at td_workspace_status (lse NaN, n_nodes -1).
 * Returns TD_ECAPACITY when td_verify_step_workspace(args) exceeds 64 MiB
 * (one sequence of 4096 context tokens with a 64-node budget at 32/8 heads
 * of 128 needs 36 MiB; 64 sequences of 8k-token contexts need more: use
 * td_verify_step there), otherwise the statuses of td_verify_step.
 */
td_status td_verify_step_noalloc(const td_step_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TREEDRAFT_H */
