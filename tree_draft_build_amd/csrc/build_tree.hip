// Stand-alone kernels of stage (b) best-first tree construction with the
// online budget stop, stage (b') bit-packed ancestor masks and stage (d)
// greedy acceptance; the device cores live in tree_core.h.

#include "step_launch.h"
#include "tree_core.h"

namespace td {
namespace {

// One wavefront per sequence: load the top-K tables into LDS, build.
template <int SLOTS>
__global__ __launch_bounds__(kWave) void build_tree_kernel(const int32_t *__restrict__ topk_id,
                                                           const double *__restrict__ topk_logq,
                                                           TreeParams P, TreeOut o) {
    __shared__ TreeLds t;
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int root_tok = P.root_token ? P.root_token[b] : -1;
    const int BK = P.block * P.K;
    for (int e = lane; e < BK; e += kWave) {
        t.ids[e] = static_cast<int>(static_cast<uint32_t>(topk_id[static_cast<int64_t>(b) * BK + e]) & kTokenMask);
        t.lq[e] = topk_logq[static_cast<int64_t>(b) * BK + e];
    }
    wave_lds_sync();
    build_tree_wave<SLOTS>(t, P, o, b, lane, root_tok);
}

// One thread per (sequence, row): walk the parent chain and set the bits.
__global__ __launch_bounds__(256) void tree_mask_kernel(const int32_t *__restrict__ node_parent,
                                                        const int32_t *__restrict__ n_nodes,
                                                        int batch, int nq_max,
                                                        uint64_t *__restrict__ mask) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= static_cast<int64_t>(batch) * nq_max) return;
    const int b = static_cast<int>(t / nq_max);
    const int i = static_cast<int>(t % nq_max);
    const int words = (nq_max + 63) / 64;
    uint64_t w[4] = {0, 0, 0, 0};
    if (i <= n_nodes[b]) {
        const int32_t *par = node_parent + static_cast<int64_t>(b) * nq_max;
        int u = i;
        // at most nq_max steps: a well-formed tree reaches the root sooner
        for (int step = 0; step < nq_max; ++step) {
            const uint64_t bit = 1ull << (u & 63);
            const int q = u >> 6;
            w[0] |= q == 0 ? bit : 0;
            w[1] |= q == 1 ? bit : 0;
            w[2] |= q == 2 ? bit : 0;
            w[3] |= q == 3 ? bit : 0;
            if (u == 0) break;
            const int p = par[u];
            if (p < 0 || p >= u) break;  // malformed parent: stop
            u = p;
        }
    }
    uint64_t *row = mask + t * words;
    for (int k = 0; k < words; ++k) row[k] = k == 0 ? w[0] : k == 1 ? w[1] : k == 2 ? w[2] : w[3];
}

// One wavefront per sequence.
__global__ __launch_bounds__(kWave) void accept_kernel(
    const int32_t *__restrict__ node_token, const int32_t *__restrict__ node_parent,
    const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ target_token, int n_max,
    int block, int32_t *__restrict__ accept_len, int32_t *__restrict__ accept_path,
    int32_t *__restrict__ bonus_token) {
    accept_wave(node_token, node_parent, n_nodes, target_token, n_max, block, accept_len,
                accept_path, bonus_token, blockIdx.x, threadIdx.x);
}

}  // namespace
}  // namespace td

using namespace td;

td_status td::check_tree_args(const int32_t *topk_id, const double *topk_logq, int32_t batch,
                             int32_t block, int32_t K, int32_t n_max, const int32_t *n_nodes,
                             const int32_t *node_token, const int32_t *node_parent,
                             const int32_t *node_depth, const double *node_logrho) {
    if (!topk_id || !topk_logq || !n_nodes || !node_token || !node_parent || !node_depth ||
        !node_logrho)
        return fail(TD_EINVAL, "build_tree: null pointer argument");
    if (batch <= 0 || block <= 0 || K <= 0 || n_max < 0)
        return fail(TD_EINVAL, "build_tree: batch, block, K must be positive, n_max >= 0");
    if (K > TD_MAX_TOPK || block > TD_MAX_BLOCK || n_max > TD_MAX_NODES || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "build_tree: K, block, n_max or batch above capacity");
    if (!aligned8(topk_logq) || !aligned8(node_logrho))
        return fail(TD_EINVAL, "build_tree: misaligned float64 array");
    return TD_OK;
}

extern "C" td_status td_build_tree(const int32_t *topk_id, const double *topk_logq, int32_t batch,
                                   int32_t block, int32_t K, int32_t n_max, int32_t use_stop,
                                   double cost_a, double cost_b, double cost_c, int32_t cost_knee,
                                   double l_ar, double ahat0, int32_t branch, double min_logrho,
                                   const int32_t *root_token,
                                   int32_t *n_nodes, int32_t *node_token, int32_t *node_parent,
                                   int32_t *node_depth, double *node_logrho, double *ahat,
                                   double *speedup, void *stream) {
    clear_error();
    const td_status chk = check_tree_args(topk_id, topk_logq, batch, block, K, n_max, n_nodes,
                                          node_token, node_parent, node_depth, node_logrho);
    if (chk != TD_OK) return chk;
    TreeParams P{block, K, n_max, use_stop, cost_a, cost_b, cost_c, cost_knee, l_ar, ahat0,
                 root_token, tree_branch(branch, K), min_logrho};
    TreeOut o{n_nodes, node_token, node_parent, node_depth, node_logrho, ahat, speedup, nullptr};
    hipStream_t st = as_stream(stream);
    switch (tree_slots(n_max)) {  // frontier: 1 + 2 n_max entries over 64 lanes
    case 1: hipLaunchKernelGGL(build_tree_kernel<1>, dim3(batch), dim3(kWave), 0, st, topk_id, topk_logq, P, o); break;
    case 2: hipLaunchKernelGGL(build_tree_kernel<2>, dim3(batch), dim3(kWave), 0, st, topk_id, topk_logq, P, o); break;
    case 4: hipLaunchKernelGGL(build_tree_kernel<4>, dim3(batch), dim3(kWave), 0, st, topk_id, topk_logq, P, o); break;
    default: hipLaunchKernelGGL(build_tree_kernel<8>, dim3(batch), dim3(kWave), 0, st, topk_id, topk_logq, P, o); break;
    }
    return check_launch("td_build_tree");
}

extern "C" td_status td_tree_mask(const int32_t *node_parent, const int32_t *n_nodes, int32_t batch,
                                  int32_t nq_max, uint64_t *mask, void *stream) {
    clear_error();
    if (!node_parent || !n_nodes || !mask) return fail(TD_EINVAL, "td_tree_mask: null pointer");
    if (batch <= 0 || nq_max <= 0) return fail(TD_EINVAL, "td_tree_mask: sizes must be positive");
    if (nq_max > TD_MAX_NODES + 1 || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "td_tree_mask: nq_max or batch above capacity");
    if (!aligned8(mask)) return fail(TD_EINVAL, "td_tree_mask: mask must be 8-byte aligned");
    const int64_t threads = static_cast<int64_t>(batch) * nq_max;
    hipLaunchKernelGGL(tree_mask_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, as_stream(stream), node_parent, n_nodes, batch, nq_max, mask);
    return check_launch("td_tree_mask");
}

td_status td::check_accept_args(const int32_t *node_token, const int32_t *node_parent,
                               const int32_t *n_nodes, const int32_t *target_token, int32_t batch,
                               int32_t n_max, int32_t block, const int32_t *accept_len,
                               const int32_t *accept_path, const int32_t *bonus_token) {
    if (!node_token || !node_parent || !n_nodes || !target_token || !accept_len || !accept_path ||
        !bonus_token)
        return fail(TD_EINVAL, "accept: null pointer argument");
    if (batch <= 0 || n_max < 0 || block <= 0)
        return fail(TD_EINVAL, "accept: batch and block must be positive, n_max >= 0");
    if (n_max > TD_MAX_NODES || block > TD_MAX_BLOCK || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "accept: n_max, block or batch above capacity");
    return TD_OK;
}

extern "C" td_status td_accept(const int32_t *node_token, const int32_t *node_parent,
                               const int32_t *n_nodes, const int32_t *target_token, int32_t batch,
                               int32_t n_max, int32_t block, int32_t *accept_len,
                               int32_t *accept_path, int32_t *bonus_token, void *stream) {
    clear_error();
    const td_status chk = check_accept_args(node_token, node_parent, n_nodes, target_token, batch,
                                            n_max, block, accept_len, accept_path, bonus_token);
    if (chk != TD_OK) return chk;
    hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(kWave), 0, as_stream(stream), node_token,
                       node_parent, n_nodes, target_token, n_max, block, accept_len, accept_path,
                       bonus_token);
    return check_launch("td_accept");
}

extern "C" void td_flex_budget(int32_t batch, int32_t switch_batch, int32_t K, int32_t n_max,
                               int32_t block, int32_t *branch, int32_t *n_max_out) {
    const bool single = switch_batch > 0 && batch >= switch_batch;
    if (branch) *branch = single ? 1 : K;
    if (n_max_out) *n_max_out = single ? (n_max < block ? n_max : block) : n_max;
}
