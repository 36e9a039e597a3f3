/*
 * CPU oracle for the verify-side path of budget-aware tree speculative
 * decoding (BASTION: "Bastion: Budget-Aware Speculative Decoding with
 * Tree-structured Block Diffusion Drafting", technical summary, "Methodik"
 * sections 1-3 and "Experimentelle Ergebnisse").
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the path computes.  It is used by the test-suite, by the
 * smoke check and by the benchmark's CPU-baseline leg, and by nothing else.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Arithmetic is float64 throughout; inputs in bfloat16 or float32 are widened
 * exactly.  Loops run in the order the definitions read; no blocking, no
 * reordering, no fast-math.  Independent outputs (one logit row, one
 * sequence's tree, one attention row of one head) may be computed by
 * different OpenMP threads; each output's own arithmetic runs in the same
 * order whatever the thread count, so results do not depend on it.
 *
 * Readings of points the pages leave open (listed again in the design notes):
 *  - the branching universe at depth d+1 is the top-K of q_{d+1} (K is a
 *    parameter; the pages build the tree from the per-position marginals);
 *  - ties between candidates are broken by (depth asc, token asc, parent
 *    index asc) after log path score desc; top-K ties go to the smaller id;
 *  - the root counts in A_hat with weight ahat0 (1 by default: the root is
 *    the bonus token every verify step yields), N counts draft nodes only;
 *  - a node is inserted only while S strictly rises: S(n+1) > S(n);
 *  - tree attention: every tree row sees the whole context and exactly its
 *    ancestor-or-self set of tree nodes; rows beyond the tree are zero;
 *  - the target token at depth B uses position B's marginal.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads used by the functions below (1 without OpenMP); returns the count
 * in effect. */
int or_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

enum { OR_OK = 0, OR_EINVAL = 1, OR_EDISAGREE = 5 };

/* Exact widening of one stored logit / attention element to float64.
 * dtype 0: IEEE float32.  dtype 1: bfloat16 (upper half of a float32). */
static double widen(const void *base, int dtype, int64_t idx)
{
    if (dtype == 0)
        return (double)((const float *)base)[idx];
    uint32_t u = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Stage (a): log-softmax normaliser and top-K of every drafter position.   */
/* Path score rho needs q_k(x) (Methodik §1, "Pfad-Bewertung"): here          */
/* log q_k(v) = l_kv - lse_k with lse_k = log sum_v exp(l_kv).               */
/* ------------------------------------------------------------------------ */

typedef struct {
    double value;
    int32_t id;
} or_cand;

/* Order for top-K selection: larger raw logit first, then smaller id. */
static int cmp_cand(const void *pa, const void *pb)
{
    const or_cand *a = (const or_cand *)pa, *b = (const or_cand *)pb;
    if (a->value > b->value) return -1;
    if (a->value < b->value) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

int or_draft_topk(const void *logits, int dtype, int batch, int block, int vocab,
                  int64_t pos_stride, int K, int32_t *topk_id, double *topk_logq,
                  double *lse_out)
{
    if (!logits || batch < 0 || block <= 0 || vocab <= 0 || K <= 0 || K > vocab ||
        pos_stride < vocab || (dtype != 0 && dtype != 1))
        return OR_EINVAL;
    int status = OR_OK;
#pragma omp parallel
    {
    or_cand *all = (or_cand *)malloc(sizeof(or_cand) * (size_t)vocab);
    if (!all) {
#pragma omp atomic write
        status = OR_EINVAL;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < (int64_t)batch * block; ++r) {
        if (!all) continue;
        int b = (int)(r / block), k = (int)(r % block);
        {
            int64_t row = ((int64_t)b * block + k) * pos_stride;
            /* max, then the sum of exp(l - max) in token order */
            double m = -INFINITY;
            for (int v = 0; v < vocab; ++v) {
                double x = widen(logits, dtype, row + v);
                if (x > m) m = x;
            }
            double s = 0.0;
            for (int v = 0; v < vocab; ++v)
                s += exp(widen(logits, dtype, row + v) - m);
            double lse = m + log(s);
            /* full sort of the vocabulary, then the first K */
            for (int v = 0; v < vocab; ++v) {
                all[v].value = widen(logits, dtype, row + v);
                all[v].id = v;
            }
            qsort(all, (size_t)vocab, sizeof(or_cand), cmp_cand);
            int64_t o = ((int64_t)b * block + k) * K;
            for (int j = 0; j < K; ++j) {
                topk_id[o + j] = all[j].id;
                if (topk_logq) topk_logq[o + j] = all[j].value - lse;
            }
            if (lse_out) lse_out[(int64_t)b * block + k] = lse;
        }
    }
    free(all);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Stage (b): best-first construction of the prefix-closed tree and the     */
/* adaptive stop.  Methodik §2: A_hat(T) = sum_{i in T} rho(i); repeatedly   */
/* add the valid node of largest rho.  Methodik §3: stop when               */
/* S(N) = A_hat(T_N) L_AR / C(N) starts to fall.                            */
/*                                                                          */
/* Candidates are kept in a flat list with ALL children of every inserted   */
/* node; each step scans the whole list for the best one.                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    double logrho;
    int32_t depth, token, parent;
} or_node;

/* 1 if a is preferred to b: larger log rho, then smaller depth, then smaller
 * token id, then smaller parent index. */
static int better(const or_node *a, const or_node *b)
{
    if (a->logrho != b->logrho) return a->logrho > b->logrho;
    if (a->depth != b->depth) return a->depth < b->depth;
    if (a->token != b->token) return a->token < b->token;
    return a->parent < b->parent;
}

static double cost_model(int n, double ca, double cb, double cc, int knee)
{
    double over = n - knee > 0 ? (double)(n - knee) : 0.0;
    return ca + cb * (double)n + cc * over;
}

int or_build_tree(const int32_t *topk_id, const double *topk_logq, int batch, int block, int K,
                  int n_max, int use_stop, double ca, double cb, double cc, int knee,
                  double l_ar, double ahat0, const int32_t *root_token, int32_t *n_nodes,
                  int32_t *node_token, int32_t *node_parent, int32_t *node_depth,
                  double *node_logrho, double *ahat_out, double *speedup_out,
                  double *s_curve /* optional [batch][n_max+1]: S(n) of T_n, NAN beyond */,
                  int branch /* children per node: ranks 0..branch-1 (<= 0 or > K: K) */,
                  double min_logrho /* selective verification: no node below this log rho
                                       (a threshold when < 0; 0 or more: none) */)
{
    if (!topk_id || !topk_logq || batch < 0 || block <= 0 || K <= 0 || n_max < 0)
        return OR_EINVAL;
    /* Selective verification (FlexDraft page, "Methodik" 3, Flex-Decoding): a
     * candidate's cumulative draft confidence is its path score rho; branches
     * below the threshold are pruned, and since every remaining candidate
     * scores at most the best one, growth stops at the first best candidate
     * below it.  Dynamic switching runs large batches on a single branch:
     * branch = 1 keeps only each position's top-1 token. */
    int nb = (branch <= 0 || branch > K) ? K : branch;
    int cap = K * (n_max + 1) + 1;
    int W = n_max + 1;
    int status = OR_OK;
#pragma omp parallel
    {
    or_node *front = (or_node *)malloc(sizeof(or_node) * (size_t)cap);
    if (!front) {
#pragma omp atomic write
        status = OR_EINVAL;
    }
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        if (!front) continue;
        int32_t *tok = node_token + (int64_t)b * W;
        int32_t *par = node_parent + (int64_t)b * W;
        int32_t *dep = node_depth + (int64_t)b * W;
        double *lr = node_logrho + (int64_t)b * W;
        for (int i = 0; i < W; ++i) { tok[i] = -1; par[i] = -1; dep[i] = -1; lr[i] = 0.0; }
        tok[0] = root_token ? root_token[b] : -1;
        dep[0] = 0;
        lr[0] = 0.0; /* rho(root) = empty product = 1 */
        if (s_curve)
            for (int i = 0; i < W; ++i) s_curve[(int64_t)b * W + i] = NAN;

        const int32_t *ids = topk_id + (int64_t)b * block * K;
        const double *lq = topk_logq + (int64_t)b * block * K;

        int nf = 0;
        for (int j = 0; j < nb; ++j) { /* children of the root use q_1 */
            front[nf].logrho = lq[j];
            front[nf].depth = 1;
            front[nf].token = ids[j];
            front[nf].parent = 0;
            ++nf;
        }
        int n = 0;
        double ahat = ahat0;
        double s_now = ahat * l_ar / cost_model(0, ca, cb, cc, knee);
        if (s_curve) s_curve[(int64_t)b * W] = s_now;
        while (n < n_max && nf > 0) {
            int best = 0;
            for (int f = 1; f < nf; ++f)
                if (better(&front[f], &front[best])) best = f;
            or_node nd = front[best];
            if (min_logrho < 0.0 && nd.logrho < min_logrho)
                break; /* the best candidate is below the confidence threshold */
            double ahat_next = ahat + exp(nd.logrho);
            double s_next = ahat_next * l_ar / cost_model(n + 1, ca, cb, cc, knee);
            if (use_stop && !(s_next > s_now))
                break; /* S would not rise: the tree is T_n */
            ++n;
            tok[n] = nd.token;
            par[n] = nd.parent;
            dep[n] = nd.depth;
            lr[n] = nd.logrho;
            ahat = ahat_next;
            s_now = s_next;
            if (s_curve) s_curve[(int64_t)b * W + n] = s_now;
            front[best] = front[nf - 1];
            --nf;
            if (nd.depth < block) { /* children at depth d+1 use q_{d+1} */
                for (int j = 0; j < nb; ++j) {
                    front[nf].logrho = nd.logrho + lq[(int64_t)nd.depth * K + j];
                    front[nf].depth = nd.depth + 1;
                    front[nf].token = ids[(int64_t)nd.depth * K + j];
                    front[nf].parent = n;
                    ++nf;
                }
            }
        }
        n_nodes[b] = n;
        if (ahat_out) ahat_out[b] = ahat;
        if (speedup_out) speedup_out[b] = s_now;
    }
    free(front);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Stage (b'): ancestor-or-self mask of every tree row, as explicit sets    */
/* (a node's set is its parent's set plus itself), packed into 64-bit words. */
/* ------------------------------------------------------------------------ */

int or_tree_mask(const int32_t *node_parent, const int32_t *n_nodes, int batch, int nq_max,
                 uint64_t *mask)
{
    if (!node_parent || !n_nodes || !mask || batch < 0 || nq_max <= 0) return OR_EINVAL;
    int words = (nq_max + 63) / 64;
    unsigned char *set = (unsigned char *)malloc((size_t)nq_max * (size_t)nq_max);
    if (!set) return OR_EINVAL;
    for (int b = 0; b < batch; ++b) {
        const int32_t *par = node_parent + (int64_t)b * nq_max;
        int rows = n_nodes[b] + 1;
        if (rows > nq_max) { free(set); return OR_EINVAL; }
        memset(set, 0, (size_t)nq_max * (size_t)nq_max);
        for (int i = 0; i < rows; ++i) {
            if (i > 0) {
                int p = par[i];
                if (p < 0 || p >= i) { free(set); return OR_EINVAL; }
                for (int j = 0; j < nq_max; ++j) set[(size_t)i * nq_max + j] = set[(size_t)p * nq_max + j];
            }
            set[(size_t)i * nq_max + i] = 1;
        }
        for (int i = 0; i < nq_max; ++i)
            for (int w = 0; w < words; ++w) {
                uint64_t x = 0;
                for (int t = 0; t < 64; ++t) {
                    int j = w * 64 + t;
                    if (j < nq_max && set[(size_t)i * nq_max + j]) x |= (uint64_t)1 << t;
                }
                mask[((int64_t)b * nq_max + i) * words + w] = x;
            }
    }
    free(set);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Stage (c): tree verification attention.  For sequence b, query head h and */
/* tree row i <= N: the admitted keys are the whole context of b and the     */
/* tree nodes set in row i of the mask; softmax(scale q.k) weighs their      */
/* values.  KV head of query head h is h / (hq / hkv).                       */
/* ------------------------------------------------------------------------ */

/* ctx_lengths (optional): sequence b's context is the first ctx_lengths[b]
 * rows of its region ctx_offsets[b] .. ctx_offsets[b+1]-1 (the rest of the
 * region is room for later tokens); NULL: the whole region. */
static int64_t ctx_len(const int64_t *ctx_offsets, const int64_t *ctx_lengths, int b)
{
    int64_t region = ctx_offsets[b + 1] - ctx_offsets[b];
    if (!ctx_lengths) return region;
    return ctx_lengths[b] < region ? ctx_lengths[b] : region;
}

int or_tree_attn(const void *q, const void *k_ctx, const void *v_ctx, const int64_t *ctx_offsets,
                 const int64_t *ctx_lengths, const void *k_tree, const void *v_tree,
                 const uint64_t *mask, const int32_t *n_nodes, int batch, int nq_max, int hq,
                 int hkv, int d, double scale, int dtype, double *out, int32_t b_begin,
                 int32_t b_end,
                 int32_t row_limit /* rows > row_limit are skipped (left zero); <0: all */)
{
    if (!q || !k_ctx || !v_ctx || !ctx_offsets || !k_tree || !v_tree || !mask || !n_nodes ||
        !out || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || b_begin < 0 ||
        b_end > batch || b_begin > b_end)
        return OR_EINVAL;
    int words = (nq_max + 63) / 64;
    int group = hq / hkv;
    int64_t maxlen = 0;
    for (int b = b_begin; b < b_end; ++b)
        if (ctx_len(ctx_offsets, ctx_lengths, b) > maxlen) maxlen = ctx_len(ctx_offsets, ctx_lengths, b);
    int status = OR_OK;
#pragma omp parallel
    {
    double *sc = (double *)malloc(sizeof(double) * (size_t)(maxlen + nq_max));
    if (!sc) {
#pragma omp atomic write
        status = OR_EINVAL;
    }
    /* one (sequence, row, head) output per iteration */
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < (int64_t)(b_end - b_begin) * nq_max * hq; ++t) {
        if (!sc) continue;
        int b = b_begin + (int)(t / ((int64_t)nq_max * hq));
        int i = (int)((t / hq) % nq_max);
        int h = (int)(t % hq);
        int64_t c0 = ctx_offsets[b], L = ctx_len(ctx_offsets, ctx_lengths, b);
        int rows = n_nodes[b] + 1;
        {
            {
                double *o = out + (((int64_t)(b - b_begin) * nq_max + i) * hq + h) * d;
                for (int e = 0; e < d; ++e) o[e] = 0.0;
                if (i >= rows || (row_limit >= 0 && i > row_limit)) continue;
                int g = h / group;
                int64_t qoff = (((int64_t)b * nq_max + i) * hq + h) * d;
                const uint64_t *mrow = mask + ((int64_t)b * nq_max + i) * words;
                /* scores: context keys first, then admitted tree keys */
                double m = -INFINITY;
                for (int64_t j = 0; j < L; ++j) {
                    int64_t koff = ((c0 + j) * hkv + g) * d;
                    double s = 0.0;
                    for (int e = 0; e < d; ++e)
                        s += widen(q, dtype, qoff + e) * widen(k_ctx, dtype, koff + e);
                    sc[j] = s * scale;
                    if (sc[j] > m) m = sc[j];
                }
                for (int j = 0; j < nq_max; ++j) {
                    sc[L + j] = -INFINITY;
                    if (!((mrow[j / 64] >> (j % 64)) & 1u)) continue;
                    int64_t koff = (((int64_t)b * nq_max + j) * hkv + g) * d;
                    double s = 0.0;
                    for (int e = 0; e < d; ++e)
                        s += widen(q, dtype, qoff + e) * widen(k_tree, dtype, koff + e);
                    sc[L + j] = s * scale;
                    if (sc[L + j] > m) m = sc[L + j];
                }
                double den = 0.0;
                for (int64_t j = 0; j < L + nq_max; ++j) {
                    sc[j] = (sc[j] == -INFINITY) ? 0.0 : exp(sc[j] - m);
                    den += sc[j];
                }
                for (int64_t j = 0; j < L; ++j) {
                    double p = sc[j] / den;
                    int64_t voff = ((c0 + j) * hkv + g) * d;
                    for (int e = 0; e < d; ++e) o[e] += p * widen(v_ctx, dtype, voff + e);
                }
                for (int j = 0; j < nq_max; ++j) {
                    if (sc[L + j] == 0.0) continue;
                    double p = sc[L + j] / den;
                    int64_t voff = (((int64_t)b * nq_max + j) * hkv + g) * d;
                    for (int e = 0; e < d; ++e) o[e] += p * widen(v_tree, dtype, voff + e);
                }
            }
        }
    }
    free(sc);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Stage (d): greedy acceptance (temperature 0, "Experimentelle             */
/* Ergebnisse").  A draft node is accepted iff every node on its root path   */
/* carries the target's greedy token at its parent.  The accepted nodes form */
/* a chain from the root; its length is A and the target's token at its end  */
/* is the bonus token.  Computed twice, by the per-node predicate and by the */
/* root-to-leaf walk, which must agree.                                     */
/* ------------------------------------------------------------------------ */

int or_accept(const int32_t *node_token, const int32_t *node_parent, const int32_t *n_nodes,
              const int32_t *target_token, int batch, int n_max, int block, int32_t *accept_len,
              int32_t *accept_path, int32_t *bonus_token)
{
    if (!node_token || !node_parent || !n_nodes || !target_token || batch < 0 || n_max < 0 ||
        block <= 0)
        return OR_EINVAL;
    int W = n_max + 1;
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)W);
    int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)W);
    if (!acc || !depth) { free(acc); free(depth); return OR_EINVAL; }
    int status = OR_OK;
    for (int b = 0; b < batch; ++b) {
        const int32_t *tok = node_token + (int64_t)b * W;
        const int32_t *par = node_parent + (int64_t)b * W;
        const int32_t *tgt = target_token + (int64_t)b * W;
        int rows = n_nodes[b] + 1;
        /* 1) predicate: accepted(i) = accepted(parent) and token(i) == target(parent) */
        acc[0] = 1;
        depth[0] = 0;
        int best = 0;
        for (int i = 1; i < rows; ++i) {
            int p = par[i];
            depth[i] = depth[p] + 1;
            acc[i] = acc[p] && tok[i] == tgt[p];
            if (acc[i] && depth[i] > depth[best]) best = i;
        }
        int A1 = depth[best];
        /* 2) walk: from the root, step to the child carrying the target token */
        int u = 0, A2 = 0;
        int32_t *path = accept_path + (int64_t)b * (block + 1);
        for (int t = 0; t <= block; ++t) path[t] = -1;
        path[0] = 0;
        for (;;) {
            int next = -1;
            for (int c = 1; c < rows; ++c)
                if (par[c] == u && tok[c] == tgt[u]) { next = c; break; }
            if (next < 0) break;
            u = next;
            ++A2;
            if (A2 <= block) path[A2] = u;
        }
        if (A1 != A2 || u != best) status = OR_EDISAGREE;
        accept_len[b] = A2;
        bonus_token[b] = tgt[u];
    }
    free(acc);
    free(depth);
    return status;
}

/* ------------------------------------------------------------------------ */
/* After verification: the accepted path becomes context.  The target has  */
/* verified the tree in one pass and decoding continues from the accepted   */
/* prefix ("Problemstellung"); its keys and values, computed in that pass,  */
/* are kept (the KV cache of the verification is reused, as the FlexDraft   */
/* page's decoupled execution does).  For sequence b with accepted length A  */
/* and path p_0 = root, p_1 .. p_A: tree rows p_0 .. p_A are appended, in    */
/* that order, after the L_b context rows of b's region; L_b grows by A+1;  */
/* the bonus token is the next step's root.  Rows that would not fit in the */
/* region are not written and L_b stops at the region's end.               */
/* ------------------------------------------------------------------------ */

int or_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accept_len,
                 const int32_t *accept_path, const int32_t *bonus_token, int batch, int nq_max,
                 int block, int hkv, int d, int dtype, void *k_cache, void *v_cache,
                 const int64_t *ctx_offsets, int64_t *ctx_lengths, int32_t *next_root)
{
    if (!k_tree || !v_tree || !accept_len || !accept_path || !k_cache || !v_cache ||
        !ctx_offsets || !ctx_lengths || batch < 0 || nq_max <= 0 || block <= 0 || hkv <= 0 ||
        d <= 0 || (dtype != 0 && dtype != 1))
        return OR_EINVAL;
    size_t esz = dtype == 0 ? 4 : 2;
    size_t row_bytes = (size_t)hkv * (size_t)d * esz; /* one token: every KV head */
    for (int b = 0; b < batch; ++b) {
        int A = accept_len[b];
        if (A < 0 || A > block) return OR_EINVAL;
        int64_t region = ctx_offsets[b + 1] - ctx_offsets[b];
        int64_t L = ctx_lengths[b];
        if (L < 0 || L > region) return OR_EINVAL;
        for (int j = 0; j <= A; ++j) {
            int node = accept_path[(int64_t)b * (block + 1) + j];
            if (node < 0 || node >= nq_max) return OR_EINVAL;
            if (L >= region) break; /* the region is full */
            int64_t dst = ctx_offsets[b] + L;
            int64_t src = (int64_t)b * nq_max + node;
            memcpy((char *)k_cache + (size_t)dst * row_bytes,
                   (const char *)k_tree + (size_t)src * row_bytes, row_bytes);
            memcpy((char *)v_cache + (size_t)dst * row_bytes,
                   (const char *)v_tree + (size_t)src * row_bytes, row_bytes);
            L = L + 1;
        }
        ctx_lengths[b] = L;
        if (next_root) next_root[b] = bonus_token ? bonus_token[b] : -1;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Dynamic switching by batch size (FlexDraft page, "Methodik" 3): below    */
/* switch_batch sequences a step verifies the full tree (branch K, budget   */
/* n_max); at or above it, a single branch (branch 1, at most block nodes). */
/* switch_batch <= 0 never switches.                                        */
/* ------------------------------------------------------------------------ */
void or_flex_budget(int batch, int switch_batch, int K, int n_max, int block, int *branch_out,
                    int *n_max_out)
{
    if (switch_batch > 0 && batch >= switch_batch) {
        *branch_out = 1;
        *n_max_out = n_max < block ? n_max : block;
    } else {
        *branch_out = K;
        *n_max_out = n_max;
    }
}

/* ------------------------------------------------------------------------ */
/* A one-layer stand-in for the target's verification pass over the tree   */
/* (the target scores every tree node in one parallel pass, "Problem-       */
/* stellung"; its greedy token at each node is what acceptance compares,    */
/* "Experimentelle Ergebnisse": temperature 0).  The pages fix no model; the */
/* readings here: a node's input is the embedding row of its token; Q, K, V */
/* are linear projections of it; rotary position embedding (rotate-half,    */
/* inverse frequencies base^(-2j/D)) at the node's sequence position, which */
/* is the context length plus its depth (tree siblings share a position);   */
/* the attention output row (all query heads, hq * D = hidden) is the final */
/* hidden state, and the target's greedy token is the argmax over the       */
/* vocabulary of its product with the LM head (ties: smaller id).           */
/* ------------------------------------------------------------------------ */

/* element k of bf16 row r of a [rows][cols] table */
static double bf(const void *t, int64_t cols, int64_t r, int64_t k)
{
    return widen(t, 1, r * cols + k);
}

int or_tree_qkv(const void *embed, const void *w_qkv, const int32_t *node_token,
                const int32_t *node_depth, const int32_t *n_nodes, const int64_t *ctx_offsets,
                const int64_t *ctx_lengths, int batch, int nq_max, int hidden, int vocab, int hq,
                int hkv, int d, double rope_base, double *q, double *k, double *v)
{
    if (!embed || !w_qkv || !node_token || !node_depth || !n_nodes || !ctx_offsets || !q || !k ||
        !v || batch < 0 || nq_max <= 0 || hidden <= 0 || vocab <= 0 || hq <= 0 || hkv <= 0 ||
        d <= 0 || d % 2)
        return OR_EINVAL;
    int nout = (hq + 2 * hkv) * d;
#pragma omp parallel
    {
    double *y = (double *)malloc(sizeof(double) * (size_t)nout);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < (int64_t)batch * nq_max; ++t) {
        int b = (int)(t / nq_max), i = (int)(t % nq_max);
        double *qo = q + t * hq * d, *ko = k + t * hkv * d, *vo = v + t * hkv * d;
        for (int e = 0; e < hq * d; ++e) qo[e] = 0.0;
        for (int e = 0; e < hkv * d; ++e) { ko[e] = 0.0; vo[e] = 0.0; }
        if (!y || i > n_nodes[b]) continue;
        int tok = node_token[t];
        if (tok < 0 || tok >= vocab) tok = 0; /* no token: row 0 of the table */
        /* projection: y[n] = sum_k x[k] w[n][k], in k order */
        for (int n = 0; n < nout; ++n) {
            double acc = 0.0;
            for (int kk = 0; kk < hidden; ++kk)
                acc += bf(embed, hidden, tok, kk) * bf(w_qkv, hidden, n, kk);
            y[n] = acc;
        }
        /* rotary position embedding of the query and key heads */
        int64_t len = ctx_offsets[b + 1] - ctx_offsets[b];
        if (ctx_lengths && ctx_lengths[b] < len) len = ctx_lengths[b] < 0 ? 0 : ctx_lengths[b];
        int depth = node_depth[t] < 0 ? 0 : node_depth[t];
        double pos = (double)(len + depth);
        for (int h = 0; h < hq + hkv; ++h) {
            double *x = y + (int64_t)h * d;
            for (int j = 0; j < d / 2; ++j) {
                double ang = pos * pow(rope_base, -2.0 * j / d);
                double c = cos(ang), s = sin(ang);
                double x1 = x[j], x2 = x[j + d / 2];
                x[j] = x1 * c - x2 * s;
                x[j + d / 2] = x2 * c + x1 * s;
            }
        }
        for (int e = 0; e < hq * d; ++e) qo[e] = y[e];
        for (int e = 0; e < hkv * d; ++e) {
            ko[e] = y[hq * d + e];
            vo[e] = y[(hq + hkv) * d + e];
        }
    }
    free(y);
    }
    return OR_OK;
}

int or_lm_head_argmax(const void *rows, const void *w_lm, const int32_t *n_nodes, int batch,
                      int nq_max, int hidden, int vocab, int32_t *target, double *best,
                      double *second)
{
    if (!rows || !w_lm || !n_nodes || !target || batch < 0 || nq_max <= 0 || hidden <= 0 ||
        vocab <= 0)
        return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < (int64_t)batch * nq_max; ++t) {
        int b = (int)(t / nq_max), i = (int)(t % nq_max);
        target[t] = -1;
        if (best) best[t] = NAN;
        if (second) second[t] = NAN;
        if (i > n_nodes[b]) continue;
        double m1 = -INFINITY, m2 = -INFINITY;
        int arg = -1;
        for (int n = 0; n < vocab; ++n) {
            double acc = 0.0;
            for (int kk = 0; kk < hidden; ++kk)
                acc += bf(rows, hidden, t, kk) * bf(w_lm, hidden, n, kk);
            if (acc > m1) { /* strictly larger: the smaller id keeps a tie */
                m2 = m1;
                m1 = acc;
                arg = n;
            } else if (acc > m2) {
                m2 = acc;
            }
        }
        target[t] = arg;
        if (best) best[t] = m1;
        if (second) second[t] = m2;
    }
    return OR_OK;
}
