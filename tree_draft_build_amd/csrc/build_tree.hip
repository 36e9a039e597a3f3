// Stage (b): best-first construction of the prefix-closed draft tree with the
// online budget stop; stage (b'): bit-packed ancestor masks; stage (d): the
// greedy acceptance walk.
//
// BASTION, "Methodik" §2: the tree grows by repeatedly adding the valid
// candidate of largest path score rho; §3: growth stops when the estimated
// speedup S(N) = A_hat(T_N) L_AR / C(N) stops rising.
//
// build_tree: one wavefront per sequence.  The frontier is spread over the 64
// lanes (entry e lives in slot e/64 of lane e%64).  Children are pushed
// lazily: inserting the node (parent p, rank j, depth d) pushes only
//   - its next sibling (p, rank j+1), and
//   - its first child (rank 0 at depth d+1).
// Every other candidate c has a predecessor that precedes it in the order
// (the previous sibling, whose score is >= c's, or the parent, whose score is
// >= c's at smaller depth), and c is pushed when that predecessor is
// inserted, so the frontier maximum is always the global maximum over all
// valid candidates and at most 1 + 2 N entries are ever live.
// The order is (log rho desc, depth asc, token asc, parent index asc); the
// last three keys are packed into one 32-bit word compared ascending:
//   depth << 26 | token << 8 | parent.

#include "td_internal.h"

namespace td {
namespace {

constexpr uint32_t kEmptyKey = 0xffffffffu;

__device__ __forceinline__ uint32_t pack_key(int depth, int token, int parent) {
    return (static_cast<uint32_t>(depth) << 26) | (static_cast<uint32_t>(token) << 8) |
           static_cast<uint32_t>(parent);
}

// a precedes b
__device__ __forceinline__ bool precedes(double la, uint32_t ka, double lb, uint32_t kb) {
    return la > lb || (la == lb && ka < kb);
}

__device__ __forceinline__ double cost_model(int n, double a, double b, double c, int knee) {
#pragma clang fp contract(off)
    double over = n - knee > 0 ? static_cast<double>(n - knee) : 0.0;
    return a + b * static_cast<double>(n) + c * over;
}

template <int SLOTS>
__global__ __launch_bounds__(kWave) void build_tree_kernel(
    const int32_t *__restrict__ topk_id, const double *__restrict__ topk_logq, int block, int K,
    int n_max, int use_stop, double ca, double cb, double cc, int knee, double l_ar, double ahat0,
    const int32_t *__restrict__ root_token, int32_t *__restrict__ n_nodes,
    int32_t *__restrict__ node_token, int32_t *__restrict__ node_parent,
    int32_t *__restrict__ node_depth, double *__restrict__ node_logrho, double *__restrict__ ahat_out,
    double *__restrict__ speedup_out) {
#pragma clang fp contract(off)
    __shared__ int s_ids[TD_MAX_BLOCK * TD_MAX_TOPK];
    __shared__ double s_lq[TD_MAX_BLOCK * TD_MAX_TOPK];
    __shared__ int s_tok[TD_MAX_NODES + 1];
    __shared__ int s_par[TD_MAX_NODES + 1];
    __shared__ int s_dep[TD_MAX_NODES + 1];
    __shared__ double s_lr[TD_MAX_NODES + 1];

    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int BK = block * K;
    for (int e = lane; e < BK; e += kWave) {
        s_ids[e] = topk_id[static_cast<int64_t>(b) * BK + e];
        s_lq[e] = topk_logq[static_cast<int64_t>(b) * BK + e];
    }
    __syncthreads();

    // frontier slots of this lane
    double f_lr[SLOTS];
    uint32_t f_key[SLOTS];
    int f_rank[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        f_lr[s] = -INFINITY;
        f_key[s] = kEmptyKey;
        f_rank[s] = 0;
    }
    // entry 0: the best child of the root (rank 0 of position 1)
    if (lane == 0) {
        f_lr[0] = s_lq[0];
        f_key[0] = pack_key(1, s_ids[0], 0);
        f_rank[0] = 0;
    }
    int count = 1;  // entries ever pushed (uniform across lanes)

    int n = 0;
    double ahat = ahat0;
    double s_now = ahat * l_ar / cost_model(0, ca, cb, cc, knee);
    if (lane == 0) {
        s_tok[0] = root_token ? root_token[b] : -1;
        s_par[0] = -1;
        s_dep[0] = 0;
        s_lr[0] = 0.0;
    }

    while (n < n_max) {
        // lane-local best slot
        double bl = f_lr[0];
        uint32_t bk = f_key[0];
#pragma unroll
        for (int s = 1; s < SLOTS; ++s)
            if (precedes(f_lr[s], f_key[s], bl, bk)) {
                bl = f_lr[s];
                bk = f_key[s];
            }
        // wave-wide best
        double wl = bl;
        uint32_t wk = bk;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            double ol = __shfl_xor(wl, o, kWave);
            uint32_t ok = __shfl_xor(wk, o, kWave);
            if (precedes(ol, ok, wl, wk)) {
                wl = ol;
                wk = ok;
            }
        }
        if (wk == kEmptyKey) break;  // no valid candidate left

        const double ahat_next = ahat + exp(wl);
        const double s_next = ahat_next * l_ar / cost_model(n + 1, ca, cb, cc, knee);
        if (use_stop && !(s_next > s_now)) break;

        // the owner lane removes the entry and publishes its rank
        const bool owner = (bk == wk) && (bl == wl);
        int my_rank = 0;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
            if (owner && f_key[s] == wk) {
                my_rank = f_rank[s];
                f_lr[s] = -INFINITY;
                f_key[s] = kEmptyKey;
            }
        const unsigned long long ob = __ballot(owner);
        const int owner_lane = __ffsll(static_cast<long long>(ob)) - 1;
        const int rank = __shfl(my_rank, owner_lane, kWave);

        const int depth = static_cast<int>(wk >> 26);
        const int token = static_cast<int>((wk >> 8) & 0x3ffffu);
        const int parent = static_cast<int>(wk & 0xffu);
        ++n;
        if (lane == 0) {
            s_tok[n] = token;
            s_par[n] = parent;
            s_dep[n] = depth;
            s_lr[n] = wl;
        }
        __syncthreads();  // s_lr[parent] is read by every lane below
        ahat = ahat_next;
        s_now = s_next;

        // lazy pushes: next sibling, then first child
        if (rank + 1 < K) {
            const int e = count++;
            const int j = (depth - 1) * K + rank + 1;
            const double plr = parent == 0 ? 0.0 : s_lr[parent];
            if (lane == (e & (kWave - 1))) {
#pragma unroll
                for (int s = 0; s < SLOTS; ++s)
                    if (s == (e >> 6)) {
                        f_lr[s] = plr + s_lq[j];
                        f_key[s] = pack_key(depth, s_ids[j], parent);
                        f_rank[s] = rank + 1;
                    }
            }
        }
        if (depth < block) {
            const int e = count++;
            const int j = depth * K;
            if (lane == (e & (kWave - 1))) {
#pragma unroll
                for (int s = 0; s < SLOTS; ++s)
                    if (s == (e >> 6)) {
                        f_lr[s] = wl + s_lq[j];
                        f_key[s] = pack_key(depth + 1, s_ids[j], n);
                        f_rank[s] = 0;
                    }
            }
        }
    }
    __syncthreads();

    const int W = n_max + 1;
    const int64_t base = static_cast<int64_t>(b) * W;
    for (int i = lane; i < W; i += kWave) {
        const bool in = i <= n;
        node_token[base + i] = in ? s_tok[i] : -1;
        node_parent[base + i] = in ? s_par[i] : -1;
        node_depth[base + i] = in ? s_dep[i] : -1;
        node_logrho[base + i] = in ? s_lr[i] : 0.0;
    }
    if (lane == 0) {
        n_nodes[b] = n;
        if (ahat_out) ahat_out[b] = ahat;
        if (speedup_out) speedup_out[b] = s_now;
    }
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

// One wavefront per sequence: from the root, step to the child carrying the
// target's greedy token while one exists.
__global__ __launch_bounds__(kWave) void accept_kernel(
    const int32_t *__restrict__ node_token, const int32_t *__restrict__ node_parent,
    const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ target_token, int n_max,
    int block, int32_t *__restrict__ accept_len, int32_t *__restrict__ accept_path,
    int32_t *__restrict__ bonus_token) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int W = n_max + 1;
    const int64_t base = static_cast<int64_t>(b) * W;
    const int n = min(n_nodes[b], n_max);
    int32_t *path = accept_path + static_cast<int64_t>(b) * (block + 1);
    for (int t = lane; t <= block; t += kWave) path[t] = t == 0 ? 0 : -1;
    int u = 0;
    int A = 0;
    // the tree has depth <= block, so at most block steps
    for (int step = 0; step < block; ++step) {
        const int want = target_token[base + u];
        int next = 0x7fffffff;
        for (int c0 = 1; c0 <= n; c0 += kWave) {
            const int c = c0 + lane;
            const bool hit = c <= n && node_parent[base + c] == u && node_token[base + c] == want;
            const unsigned long long m = __ballot(hit);
            if (m) {
                next = c0 + __ffsll(static_cast<long long>(m)) - 1;
                break;
            }
        }
        if (next == 0x7fffffff) break;
        u = next;
        ++A;
        if (lane == 0) path[A] = u;
    }
    if (lane == 0) {
        accept_len[b] = A;
        bonus_token[b] = target_token[base + u];
    }
}

}  // namespace
}  // namespace td

using namespace td;

extern "C" td_status td_build_tree(const int32_t *topk_id, const double *topk_logq, int32_t batch,
                                   int32_t block, int32_t K, int32_t n_max, int32_t use_stop,
                                   double cost_a, double cost_b, double cost_c, int32_t cost_knee,
                                   double l_ar, double ahat0, const int32_t *root_token,
                                   int32_t *n_nodes, int32_t *node_token, int32_t *node_parent,
                                   int32_t *node_depth, double *node_logrho, double *ahat,
                                   double *speedup, void *stream) {
    clear_error();
    if (!topk_id || !topk_logq || !n_nodes || !node_token || !node_parent || !node_depth ||
        !node_logrho)
        return fail(TD_EINVAL, "td_build_tree: null pointer argument");
    if (batch <= 0 || block <= 0 || K <= 0 || n_max < 0)
        return fail(TD_EINVAL, "td_build_tree: batch, block, K must be positive, n_max >= 0");
    if (K > TD_MAX_TOPK || block > TD_MAX_BLOCK || n_max > TD_MAX_NODES || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "td_build_tree: K, block, n_max or batch above capacity");
    if (!aligned8(topk_logq) || !aligned8(node_logrho))
        return fail(TD_EINVAL, "td_build_tree: misaligned float64 array");
    // frontier capacity: 1 + 2 n_max entries over 64 lanes
    const int need = 1 + 2 * n_max;
    hipStream_t st = as_stream(stream);
#define TD_LAUNCH_TREE(SL)                                                                       \
    hipLaunchKernelGGL((build_tree_kernel<SL>), dim3(batch), dim3(kWave), 0, st, topk_id,       \
                       topk_logq, block, K, n_max, use_stop, cost_a, cost_b, cost_c, cost_knee, \
                       l_ar, ahat0, root_token, n_nodes, node_token, node_parent, node_depth,   \
                       node_logrho, ahat, speedup)
    if (need <= 64)
        TD_LAUNCH_TREE(1);
    else if (need <= 128)
        TD_LAUNCH_TREE(2);
    else if (need <= 256)
        TD_LAUNCH_TREE(4);
    else
        TD_LAUNCH_TREE(8);
#undef TD_LAUNCH_TREE
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

extern "C" td_status td_accept(const int32_t *node_token, const int32_t *node_parent,
                               const int32_t *n_nodes, const int32_t *target_token, int32_t batch,
                               int32_t n_max, int32_t block, int32_t *accept_len,
                               int32_t *accept_path, int32_t *bonus_token, void *stream) {
    clear_error();
    if (!node_token || !node_parent || !n_nodes || !target_token || !accept_len || !accept_path ||
        !bonus_token)
        return fail(TD_EINVAL, "td_accept: null pointer argument");
    if (batch <= 0 || n_max < 0 || block <= 0)
        return fail(TD_EINVAL, "td_accept: batch and block must be positive, n_max >= 0");
    if (n_max > TD_MAX_NODES || block > TD_MAX_BLOCK || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "td_accept: n_max, block or batch above capacity");
    hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(kWave), 0, as_stream(stream), node_token,
                       node_parent, n_nodes, target_token, n_max, block, accept_len, accept_path,
                       bonus_token);
    return check_launch("td_accept");
}
