/* Sanitizer driver for the CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Built together with oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitizers.py: it calls
 * every oracle entry point on small seeded inputs, including the edge cases
 * the pins exercise (ragged vocabularies, K = vocab, a budget of 0, an empty
 * context, a commit at the end of its region, rows past a tree), and checks
 * each call's status and a few invariants of its outputs.  Any out-of-bounds
 * access, use of freed memory or undefined behaviour aborts the run.
 * Prints "sanitize driver ok" and exits 0 when every call passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int or_set_threads(int n);
int or_draft_topk(const void *logits, int dtype, int batch, int block, int vocab,
                  int64_t pos_stride, int K, int32_t *topk_id, double *topk_logq,
                  double *lse_out);
int or_build_tree(const int32_t *topk_id, const double *topk_logq, int batch, int block, int K,
                  int n_max, int use_stop, double ca, double cb, double cc, int knee,
                  double l_ar, double ahat0, const int32_t *root_token, int32_t *n_nodes,
                  int32_t *node_token, int32_t *node_parent, int32_t *node_depth,
                  double *node_logrho, double *ahat_out, double *speedup_out, double *s_curve,
                  int branch, double min_logrho);
int or_tree_mask(const int32_t *node_parent, const int32_t *n_nodes, int batch, int nq_max,
                 uint64_t *mask);
int or_tree_attn(const void *q, const void *k_ctx, const void *v_ctx, const int64_t *ctx_offsets,
                 const int64_t *ctx_lengths, const void *k_tree, const void *v_tree,
                 const uint64_t *mask, const int32_t *n_nodes, int batch, int nq_max, int hq,
                 int hkv, int d, double scale, int dtype, double *out, int32_t b_begin,
                 int32_t b_end, int32_t row_limit);
int or_accept(const int32_t *node_token, const int32_t *node_parent, const int32_t *n_nodes,
              const int32_t *target_token, int batch, int n_max, int block, int32_t *accept_len,
              int32_t *accept_path, int32_t *bonus_token);
int or_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accept_len,
                 const int32_t *accept_path, const int32_t *bonus_token, int batch, int nq_max,
                 int block, int hkv, int d, int dtype, void *k_cache, void *v_cache,
                 const int64_t *ctx_offsets, int64_t *ctx_lengths, int32_t *next_root);
void or_flex_budget(int batch, int switch_batch, int K, int n_max, int block, int *branch_out,
                    int *n_max_out);
int or_tree_qkv(const void *embed, const void *w_qkv, const int32_t *node_token,
                const int32_t *node_depth, const int32_t *n_nodes, const int64_t *ctx_offsets,
                const int64_t *ctx_lengths, int batch, int nq_max, int hidden, int vocab, int hq,
                int hkv, int d, double rope_base, double *q, double *k, double *v);
int or_lm_head_argmax(const void *rows, const void *w_lm, const int32_t *n_nodes, int batch,
                      int nq_max, int hidden, int vocab, int32_t *target, double *best,
                      double *second);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

/* xorshift64*: uniform in [0, 1) */
static double urand(void)
{
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static float frand(void) { return (float)(4.0 * urand() - 2.0); }

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n)
{
    void *p = calloc(n ? n : 1, 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int g_fail = 0;
#define CHECK(cond, what)                                                    \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "check failed: %s (%s:%d)\n", what, __FILE__, __LINE__); \
            g_fail = 1;                                                      \
        }                                                                    \
    } while (0)

/* One pass over the whole path at the given sizes. */
static void run_case(int batch, int block, int vocab, int K, int n_max, int use_stop, int branch,
                     double min_logrho, const int64_t *ctx_len, int room)
{
    const int nq = n_max + 1;
    const int hq = 4, hkv = 2, d = 8, hidden = hq * d;
    const int64_t rows = (int64_t)batch * block;

    /* (a) top-K on float32 logits with a ragged row stride */
    const int64_t stride = vocab + 3;
    float *logits = xmalloc(sizeof(float) * (size_t)(rows * stride));
    for (int64_t i = 0; i < rows * stride; ++i) logits[i] = frand();
    int32_t *tid = xmalloc(sizeof(int32_t) * (size_t)(rows * K));
    double *tlq = xmalloc(sizeof(double) * (size_t)(rows * K));
    double *lse = xmalloc(sizeof(double) * (size_t)rows);
    CHECK(or_draft_topk(logits, 0, batch, block, vocab, stride, K, tid, tlq, lse) == 0, "topk");
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 1; j < K; ++j) CHECK(tlq[r * K + j] <= tlq[r * K + j - 1], "topk order");

    /* (b) tree, (b') mask */
    int32_t root[64];
    for (int b = 0; b < batch; ++b) root[b] = b % vocab;
    int32_t *nn = xmalloc(sizeof(int32_t) * (size_t)batch);
    int32_t *tok = xmalloc(sizeof(int32_t) * (size_t)(batch * nq));
    int32_t *par = xmalloc(sizeof(int32_t) * (size_t)(batch * nq));
    int32_t *dep = xmalloc(sizeof(int32_t) * (size_t)(batch * nq));
    double *lr = xmalloc(sizeof(double) * (size_t)(batch * nq));
    double *ah = xmalloc(sizeof(double) * (size_t)batch);
    double *sp = xmalloc(sizeof(double) * (size_t)batch);
    double *sc = xmalloc(sizeof(double) * (size_t)(batch * nq));
    CHECK(or_build_tree(tid, tlq, batch, block, K, n_max, use_stop, 1.0, 0.005, 0.03, 32, 1.0, 1.0,
                        root, nn, tok, par, dep, lr, ah, sp, sc, branch, min_logrho) == 0, "tree");
    for (int b = 0; b < batch; ++b) {
        CHECK(nn[b] >= 0 && nn[b] <= n_max, "tree size");
        for (int i = 1; i <= nn[b]; ++i)
            CHECK(par[b * nq + i] >= 0 && par[b * nq + i] < i, "parent before child");
    }
    const int words = (nq + 63) / 64;
    uint64_t *mask = xmalloc(sizeof(uint64_t) * (size_t)(batch * nq * words));
    CHECK(or_tree_mask(par, nn, batch, nq, mask) == 0, "mask");
    for (int b = 0; b < batch; ++b)
        for (int i = 0; i <= nn[b]; ++i)
            CHECK((mask[((int64_t)b * nq + i) * words + i / 64] >> (i % 64)) & 1u, "mask self");

    /* f4: Q/K/V of the tree tokens and the LM-head targets (bf16 tables) */
    int64_t *off = xmalloc(sizeof(int64_t) * (size_t)(batch + 1));
    int64_t *lens = xmalloc(sizeof(int64_t) * (size_t)batch);
    off[0] = 0;
    for (int b = 0; b < batch; ++b) {
        lens[b] = ctx_len[b];
        off[b + 1] = off[b] + ctx_len[b] + room;
    }
    const int64_t total = off[batch];
    uint16_t *embed = xmalloc(sizeof(uint16_t) * (size_t)vocab * hidden);
    uint16_t *wqkv = xmalloc(sizeof(uint16_t) * (size_t)(hq + 2 * hkv) * d * hidden);
    uint16_t *wlm = xmalloc(sizeof(uint16_t) * (size_t)vocab * hidden);
    for (int64_t i = 0; i < (int64_t)vocab * hidden; ++i) embed[i] = to_bf16(frand());
    for (int64_t i = 0; i < (int64_t)(hq + 2 * hkv) * d * hidden; ++i) wqkv[i] = to_bf16(frand());
    for (int64_t i = 0; i < (int64_t)vocab * hidden; ++i) wlm[i] = to_bf16(frand());
    for (int b = 0; b < batch; ++b) tok[b * nq] = root[b];
    double *qd = xmalloc(sizeof(double) * (size_t)(batch * nq * hq * d));
    double *kd = xmalloc(sizeof(double) * (size_t)(batch * nq * hkv * d));
    double *vd = xmalloc(sizeof(double) * (size_t)(batch * nq * hkv * d));
    CHECK(or_tree_qkv(embed, wqkv, tok, dep, nn, off, lens, batch, nq, hidden, vocab, hq, hkv, d,
                      1e6, qd, kd, vd) == 0, "qkv");

    /* (c) attention over float32 copies, contexts given by lengths */
    float *q = xmalloc(sizeof(float) * (size_t)(batch * nq * hq * d));
    float *kt = xmalloc(sizeof(float) * (size_t)(batch * nq * hkv * d));
    float *vt = xmalloc(sizeof(float) * (size_t)(batch * nq * hkv * d));
    for (int64_t i = 0; i < (int64_t)batch * nq * hq * d; ++i) q[i] = (float)(qd[i] * 0.1);
    for (int64_t i = 0; i < (int64_t)batch * nq * hkv * d; ++i) {
        kt[i] = (float)(kd[i] * 0.1);
        vt[i] = (float)vd[i];
    }
    float *kc = xmalloc(sizeof(float) * (size_t)((total + 1) * hkv * d));
    float *vc = xmalloc(sizeof(float) * (size_t)((total + 1) * hkv * d));
    for (int64_t i = 0; i < total * hkv * d; ++i) {
        kc[i] = frand();
        vc[i] = frand();
    }
    double *out = xmalloc(sizeof(double) * (size_t)(batch * nq * hq * d));
    CHECK(or_tree_attn(q, kc, vc, off, lens, kt, vt, mask, nn, batch, nq, hq, hkv, d,
                       1.0 / sqrt((double)d), 0, out, 0, batch, -1) == 0, "attention");
    for (int64_t i = 0; i < (int64_t)batch * nq * hq * d; ++i) CHECK(isfinite(out[i]), "finite");

    uint16_t *hid = xmalloc(sizeof(uint16_t) * (size_t)(batch * nq * hidden));
    for (int64_t i = 0; i < (int64_t)batch * nq * hidden; ++i) hid[i] = to_bf16((float)out[i]);
    int32_t *target = xmalloc(sizeof(int32_t) * (size_t)(batch * nq));
    double *best = xmalloc(sizeof(double) * (size_t)(batch * nq));
    double *second = xmalloc(sizeof(double) * (size_t)(batch * nq));
    CHECK(or_lm_head_argmax(hid, wlm, nn, batch, nq, hidden, vocab, target, best, second) == 0,
          "lm head");

    /* (d) acceptance, then f1 commit (one row of room: commits stop at the region end) */
    int32_t *alen = xmalloc(sizeof(int32_t) * (size_t)batch);
    int32_t *path = xmalloc(sizeof(int32_t) * (size_t)(batch * (block + 1)));
    int32_t *bonus = xmalloc(sizeof(int32_t) * (size_t)batch);
    /* half the rows follow the tree (deep acceptances), half take the LM head */
    for (int b = 0; b < batch; ++b)
        for (int i = 0; i <= nn[b]; ++i) {
            int child = -1;
            for (int c = 1; c <= nn[b]; ++c)
                if (par[b * nq + c] == i) { child = c; break; }
            if (b % 2 == 0 && child > 0) target[b * nq + i] = tok[b * nq + child];
        }
    CHECK(or_accept(tok, par, nn, target, batch, n_max, block, alen, path, bonus) == 0, "accept");
    for (int b = 0; b < batch; ++b) CHECK(alen[b] >= 0 && alen[b] <= block, "accept length");
    int32_t *next = xmalloc(sizeof(int32_t) * (size_t)batch);
    CHECK(or_kv_commit(kt, vt, alen, path, bonus, batch, nq, block, hkv, d, 0, kc, vc, off, lens,
                       next) == 0, "commit");
    for (int b = 0; b < batch; ++b) {
        CHECK(lens[b] <= off[b + 1] - off[b], "commit within its region");
        CHECK(next[b] == bonus[b], "bonus is the next root");
    }

    int br = 0, nm = 0;
    or_flex_budget(batch, 4, K, n_max, block, &br, &nm);
    CHECK(br >= 1 && nm >= 0 && nm <= n_max, "flex budget");

    free(logits); free(tid); free(tlq); free(lse); free(nn); free(tok); free(par); free(dep);
    free(lr); free(ah); free(sp); free(sc); free(mask); free(off); free(lens); free(embed);
    free(wqkv); free(wlm); free(qd); free(kd); free(vd); free(q); free(kt); free(vt); free(kc);
    free(vc); free(out); free(hid); free(target); free(best); free(second); free(alen);
    free(path); free(bonus); free(next);
}

int main(void)
{
    or_set_threads(2);
    const int64_t ctx_a[4] = {37, 0, 5, 64};
    const int64_t ctx_b[2] = {0, 0};
    run_case(4, 8, 101, 4, 16, 1, 0, 0.0, ctx_a, 1);      /* S(N) stop, ragged contexts */
    run_case(4, 8, 101, 4, 16, 0, 0, 0.0, ctx_a, 9);      /* fixed N */
    run_case(2, 4, 33, 33, 40, 0, 2, -3.0, ctx_b, 0);     /* K = vocab, branch cap, threshold,
                                                             empty contexts without room */
    run_case(1, 16, 257, 8, 0, 1, 0, 0.0, ctx_a, 2);      /* a budget of 0 */
    run_case(3, 5, 70, 3, 130, 0, 0, 0.0, ctx_a, 17);     /* mask rows of three words */
    if (g_fail) return 1;
    printf("sanitize driver ok\n");
    return 0;
}
