// Launchers shared between translation units (internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tree_core.h"
#include "treedraft.h"

namespace td {

struct TreeParams;
struct TreeOut;

// The top-K and verify-step workspaces start with a 16-byte status header:
// word 0 collects kStatus* bits, set by a waiter that gave up on a hand-off.
constexpr size_t kStatusBytes = 16;
constexpr uint32_t kStatusMerge = 1u;  // a row merger gave up (lse NaN)
constexpr uint32_t kStatusTree = 2u;   // a tree builder gave up (n_nodes -1)
constexpr uint32_t kStatusSplit = 4u;  // a context-split workgroup gave up waiting for its tree size

// children per node of the tree builders: branch in 1..K, else K
inline int tree_branch(int branch, int K) { return branch >= 1 && branch <= K ? branch : K; }

// top-K workspace bytes (status header, per-workgroup epoch-tagged partials,
// row records)
size_t topk_workspace_bytes(int batch, int block, int vocab, int K);

// The verify step's first kernel: top-K of every position, then each
// sequence's tree and mask rows (TreeOut::mask must be set).
void launch_topk_tree(const void *logits, td_dtype dtype, int batch, int block, int vocab,
                      int64_t pos_stride, int K, void *ws, int32_t *topk_id, double *topk_logq,
                      double *lse, const TreeParams &tp, const TreeOut &to, hipStream_t st);

// Context-attention inputs of the verify step's fused first kernel (bf16,
// head dim 128); ws is the attention part of the step workspace.
struct SplitInputs {
    const void *q, *k_ctx, *v_ctx;
    const int64_t *off, *lens;
    int64_t total_ctx;
    int nq_max, hq, hkv;
    float scale;
    void *ws;
};
// Whether the verify step runs its context split inside the first kernel.
bool step_fuses_split(int batch, int block, int vocab, int K, int nq_max, int hq, int hkv, int head_dim,
                      int64_t total_ctx, td_dtype attn_dtype);
// The first kernel with the context split (TreeOut::ready must be set).
void launch_topk_tree_split(const void *logits, td_dtype dtype, int batch, int block, int vocab,
                            int64_t pos_stride, int K, void *ws, int32_t *topk_id, double *topk_logq,
                            double *lse, const TreeParams &tp, const TreeOut &to, const SplitInputs &si,
                            hipStream_t st);

// Tree attention; with accept_* set, the combine kernel also runs the
// acceptance walk of every sequence.
// With commit set, the acceptance workgroup of each sequence then appends the
// accepted path's K/V to the context (cm).
struct AcceptArgs {
    const int32_t *node_token, *node_parent, *target_token;
    int n_max, block;
    int32_t *accept_len, *accept_path, *bonus_token;
    int commit;
    CommitArgs cm;
    uint64_t *ready;  // [batch] tree-size words of the fused first kernel, cleared here (or null)
};
size_t attn_workspace_bytes(int batch, int nq_max, int hq, int hkv, int head_dim,
                            int64_t total_ctx, td_dtype dtype, bool fused_plan = false);
void launch_attention(const void *q, const void *k_ctx, const void *v_ctx, const int64_t *off,
                      const int64_t *lens, int64_t total_ctx, const void *k_tree, const void *v_tree,
                      const uint64_t *mask, const int32_t *n_nodes, int batch, int nq_max, int hq,
                      int hkv, int head_dim, float scale, td_dtype dtype, void *ws, void *out,
                      const AcceptArgs *acc, hipStream_t st, bool split = true);

// Argument checks shared by the per-stage entry points and the fused step
// (they record td_last_error text and return the status).
td_status check_topk_args(const void *logits, td_dtype dtype, int32_t batch, int32_t block,
                          int32_t vocab, int64_t pos_stride, int32_t K, const int32_t *topk_id,
                          const double *topk_logq, const double *lse);
td_status check_tree_args(const int32_t *topk_id, const double *topk_logq, int32_t batch,
                          int32_t block, int32_t K, int32_t n_max, const int32_t *n_nodes,
                          const int32_t *node_token, const int32_t *node_parent,
                          const int32_t *node_depth, const double *node_logrho);
td_status check_attn_args(const void *q, const void *k_ctx, const void *v_ctx,
                          const int64_t *ctx_offsets, int64_t total_ctx, int64_t max_ctx,
                          const void *k_tree, const void *v_tree, const uint64_t *mask,
                          const int32_t *n_nodes, int32_t batch, int32_t nq_max, int32_t hq,
                          int32_t hkv, int32_t head_dim, td_dtype dtype, const void *out);
td_status check_accept_args(const int32_t *node_token, const int32_t *node_parent,
                            const int32_t *n_nodes, const int32_t *target_token, int32_t batch,
                            int32_t n_max, int32_t block, const int32_t *accept_len,
                            const int32_t *accept_path, const int32_t *bonus_token);

}  // namespace td
