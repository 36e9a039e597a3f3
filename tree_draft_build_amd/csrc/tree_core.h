// Device cores of stage (b) best-first tree construction with the online
// budget stop, stage (b') ancestor masks and stage (d) greedy acceptance,
// shared by the stand-alone kernels and the fused verify step.
//
// BASTION, "Methodik" §2: the tree grows by repeatedly adding the valid
// candidate of largest path score rho; §3: growth stops when the estimated
// speedup S(N) = A_hat(T_N) L_AR / C(N) stops rising.
//
// One wavefront builds one sequence's tree.  The frontier is spread over the
// 64 lanes (entry e lives in slot e/64 of lane e%64).  Children are pushed
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
#pragma once

#include "td_internal.h"

namespace td {

constexpr uint32_t kEmptyKey = 0xffffffffu;
// Token ids fit in 18 bits (TD_MAX_VOCAB = 2^18); the frontier key packs them
// so, and the builders mask the ids they load with this before packing.
constexpr uint32_t kTokenMask = 0x3ffffu;
constexpr float kLog2e = 1.4426950408889634f;  // log2(e): exponentials are taken in base 2

// LDS ordering inside one wavefront: LDS operations of a wave complete in
// issue order; this keeps the compiler from moving them and waits for them.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), other counters untouched
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t pack_key(int depth, int token, int parent) {
    return (static_cast<uint32_t>(depth) << 26) | (static_cast<uint32_t>(token) << 8) |
           static_cast<uint32_t>(parent);
}

// lane `src` (wave-uniform) of a double
__device__ __forceinline__ double read_lane_d(double x, int src) {
    const uint64_t u = __double_as_longlong(x);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), src);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), src);
    return __longlong_as_double(static_cast<long long>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32)));
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

struct TreeParams {
    int block, K, n_max, use_stop;
    double ca, cb, cc;
    int knee;
    double l_ar, ahat0;
    const int32_t *root_token;  // may be null
    int branch;                 // children per node, 1..K (ranks 0..branch-1)
    double min_logrho;          // selective verification: no node below this (< 0; else off)
};

struct TreeOut {
    int32_t *n_nodes, *node_token, *node_parent, *node_depth;
    double *node_logrho, *ahat, *speedup;  // ahat / speedup may be null
    uint64_t *mask;                        // null: no mask rows
    // Non-null in the verify step's fused first kernel: word b receives
    // (1 << 32) | n of sequence b as soon as its tree size n is final, for
    // the context-split workgroups of the same launch; the step's last
    // kernel clears it again.
    uint64_t *ready;
};

// LDS of one tree build: the top-K tables and the inserted nodes
struct TreeLds {
    int ids[TD_MAX_BLOCK * TD_MAX_TOPK];
    double lq[TD_MAX_BLOCK * TD_MAX_TOPK];
    int tok[TD_MAX_NODES + 1];
    int par[TD_MAX_NODES + 1];
    int dep[TD_MAX_NODES + 1];
    double lr[TD_MAX_NODES + 1];
};

// Frontier slots per lane for a budget of n_max nodes: 1 + 2 (n_max - 1)
// entries (each insertion but the last pushes at most two).
__host__ __device__ inline int tree_slots(int n_max) {
    const int need = 1 + 2 * (n_max > 1 ? n_max - 1 : 0);
    return need <= 64 ? 1 : need <= 128 ? 2 : need <= 256 ? 4 : 8;
}

// Build sequence b's tree with one wavefront from the tables in t.ids/t.lq
// (already in LDS, ordered by (position, rank)).  Writes every output array
// of sequence b, and its mask rows when o.mask is set.  root_tok is the
// token of node 0 (the caller loads it early; it is needed only at the end).
// PREFILLED: the other waves of the workgroup have written every entry and
// mask row past the root as if beyond the tree (prefill_tree_outputs) and
// meet this wave at a workgroup barrier before the tree's own entries are
// written; only entries 0..n are written here then.
template <int SLOTS, bool PREFILLED, bool STOP>
__device__ __forceinline__ void build_tree_wave_t(TreeLds &t, const TreeParams &P, const TreeOut &o, int b,
                                                  int lane, int root_tok) {
#pragma clang fp contract(off)
    const int K = P.K;
    constexpr bool stop = STOP;
    // Frontier slots of this lane: log rho, order key, rank among the
    // siblings and the parent's log rho (the next sibling's score is the
    // parent's plus its table entry).  Nothing the selection loop reads is
    // in LDS except the read-only top-K tables.
    double f_lr[SLOTS], f_plr[SLOTS];
    uint32_t f_key[SLOTS];
    int f_rank[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        f_lr[s] = -INFINITY;
        f_plr[s] = 0.0;
        f_key[s] = kEmptyKey;
        f_rank[s] = 0;
    }
    // entry 0: the best child of the root (rank 0 of position 1)
    if (lane == 0) {
        f_lr[0] = t.lq[0];
        f_key[0] = pack_key(1, t.ids[0], 0);
    }
    int count = 1;  // entries ever pushed (uniform across lanes)

    int n = 0;
    double ahat = P.ahat0;
    double s_now = ahat * P.l_ar / cost_model(0, P.ca, P.cb, P.cc, P.knee);
    if (lane == 0) {
        t.par[0] = -1;
        t.dep[0] = 0;
        t.lr[0] = 0.0;
    }
    // Inserted node i's record (token, parent, depth, log rho) stays in lane
    // i % 64, slot i / 64, until the loop ends: no LDS store inside the loop,
    // so its table reads never queue behind one.
    int r_tok[SLOTS], r_par[SLOTS], r_dep[SLOTS];
    double r_lr[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        r_tok[s] = 0;
        r_par[s] = -1;
        r_dep[s] = 0;
        r_lr[s] = 0.0;
    }

    while (n < P.n_max) {
        // counters are wave-uniform: say so, keeping the loop's control scalar
        n = __builtin_amdgcn_readfirstlane(n);
        count = __builtin_amdgcn_readfirstlane(count);
        // lane-local best slot
        double bl = f_lr[0];
        uint32_t bk = f_key[0];
        int bs = 0;
#pragma unroll
        for (int s = 1; s < SLOTS; ++s)
            if (precedes(f_lr[s], f_key[s], bl, bk)) {
                bl = f_lr[s];
                bk = f_key[s];
                bs = s;
            }
        // The stop rule for this lane's own best entry: A_hat and S with it
        // inserted (rho = exp(log rho)), computed beside the selection below,
        // whose winner's values are then taken from its lane.
        double ah_mine = 0.0, s_mine = 0.0;
        if constexpr (STOP) {
            ah_mine = ahat + exp(bl);
            s_mine = ah_mine * P.l_ar / cost_model(n + 1, P.ca, P.cb, P.cc, P.knee);
        }
        double wl;
        uint32_t wk;
        {
            // wave-wide largest log rho (register butterfly on the score
            // alone), then the lanes that hold it: one in general, several
            // only for equal scores, when the smallest key among them wins
            double m = bl;
            m = fmax(m, xchg_d<0>(m));
            m = fmax(m, xchg_d<1>(m));
            m = fmax(m, xchg_d<2>(m));
            m = fmax(m, xchg_d<3>(m));
            m = fmax(m, xchg_d<4>(m));
            m = fmax(m, xchg_d<5>(m));
            wl = read_lane_d(m, 0);
            const bool at = bl == wl;
            const unsigned long long hold = __ballot(at);
            uint32_t kk = at ? bk : kEmptyKey;
            if (__popcll(hold) > 1) {
                kk = min(kk, xchg<0>(kk));
                kk = min(kk, xchg<1>(kk));
                kk = min(kk, xchg<2>(kk));
                kk = min(kk, xchg<3>(kk));
                kk = min(kk, xchg<4>(kk));
                kk = min(kk, xchg<5>(kk));
            }
            wk = kk;
            // the first holding lane has the winner's key in either case
            wk = __builtin_amdgcn_readlane(wk, __ffsll(static_cast<long long>(hold)) - 1);
        }
        // every lane holds the winner: make that explicit (scalar registers),
        // so that the loop's exits and counters are uniform
        wl = read_lane_d(wl, 0);
        wk = __builtin_amdgcn_readfirstlane(wk);
        if (wk == kEmptyKey) break;  // no valid candidate left
        // selective verification: every remaining candidate scores at most
        // the best one, so the first one below the threshold ends the tree
        if (P.min_logrho < 0.0 && wl < P.min_logrho) break;

        // the owner lane (its best slot bs holds the entry) hands over the
        // entry's rank, parent score and rho
        const bool owner = (bk == wk) && (bl == wl);
        int my_rank = f_rank[0];
        double my_plr = f_plr[0];
#pragma unroll
        for (int s = 1; s < SLOTS; ++s)
            if (bs == s) {
                my_rank = f_rank[s];
                my_plr = f_plr[s];
            }
        const unsigned long long ob = __ballot(owner);
        const int owner_lane = __ffsll(static_cast<long long>(ob)) - 1;
        const int rank = __builtin_amdgcn_readlane(my_rank, owner_lane);
        const double plr = read_lane_d(my_plr, owner_lane);

        if constexpr (STOP) {
            const double s_next = read_lane_d(s_mine, owner_lane);
            if (!(s_next > s_now)) break;
            ahat = read_lane_d(ah_mine, owner_lane);
            s_now = s_next;
        }
        // remove the entry
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
            if (owner && bs == s) {
                f_lr[s] = -INFINITY;
                f_key[s] = kEmptyKey;
            }

        const int depth = static_cast<int>(wk >> 26);
        const int token = static_cast<int>((wk >> 8) & 0x3ffffu);
        const int parent = static_cast<int>(wk & 0xffu);
        ++n;
        {
            const int rs = n >> 6;  // uniform
            const bool mine = lane == (n & (kWave - 1));
#pragma unroll
            for (int s = 0; s < SLOTS; ++s)
                if (s == rs) {
                    r_tok[s] = mine ? token : r_tok[s];
                    r_par[s] = mine ? parent : r_par[s];
                    r_dep[s] = mine ? depth : r_dep[s];
                    r_lr[s] = mine ? wl : r_lr[s];
                }
        }

        // Lazy pushes: next sibling, then first child (none after the last
        // node).  Entry e goes to lane e % 64, slot e / 64: the slot is
        // chosen by a uniform branch, the lane by a select.
        if (n == P.n_max) break;
        auto put = [&](int e, double lr, uint32_t key, int rnk, double plr_) __attribute__((always_inline)) {
            const int se = e >> 6;
            const bool mine = lane == (e & (kWave - 1));
#pragma unroll
            for (int s = 0; s < SLOTS; ++s)
                if (s == se) {
                    f_lr[s] = mine ? lr : f_lr[s];
                    f_key[s] = mine ? key : f_key[s];
                    f_rank[s] = mine ? rnk : f_rank[s];
                    f_plr[s] = mine ? plr_ : f_plr[s];
                }
        };
        // both table entries are read at once (an unused one reads entry 0)
        const bool sib = rank + 1 < P.branch;
        const bool kid = depth < P.block;
        const int j_sib = sib ? (depth - 1) * K + rank + 1 : 0;
        const int j_kid = kid ? depth * K : 0;
        const double lq_sib = t.lq[j_sib], lq_kid = t.lq[j_kid];
        const int id_sib = t.ids[j_sib], id_kid = t.ids[j_kid];
        if (sib) put(count++, plr + lq_sib, pack_key(depth, id_sib, parent), rank + 1, plr);
        if (kid) put(count++, wl + lq_kid, pack_key(depth + 1, id_kid, n), 0, wl);
    }
    // the records of nodes 1..n to LDS (node 0's were written above)
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        const int i = s * kWave + lane;
        if (i >= 1 && i <= n) {
            t.tok[i] = r_tok[s];
            t.par[i] = r_par[s];
            t.dep[i] = r_dep[s];
            t.lr[i] = r_lr[s];
        }
    }
    if (o.ready && lane == 0)  // one 8-byte word: the size is never seen without its flag
        __hip_atomic_store(o.ready + b, (uint64_t{1} << 32) | static_cast<uint32_t>(n), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    wave_lds_sync();
    if (!stop) {  // A_hat(n) and S(n) of the tree built (sum in any order: float64)
        double part = 0.0;
        for (int i = 1 + lane; i <= n; i += kWave) part += exp(t.lr[i]);
        ahat = P.ahat0 + wave_sum(part);
        s_now = ahat * P.l_ar / cost_model(n, P.ca, P.cb, P.cc, P.knee);
    }
    if constexpr (PREFILLED) __syncthreads();  // the prefill stores have landed

    const int W = P.n_max + 1;
    const int64_t base = static_cast<int64_t>(b) * W;
    const int lim = PREFILLED ? n + 1 : W;  // entries written here
    for (int i = lane; i < lim; i += kWave) {
        const bool in = i <= n;
        o.node_token[base + i] = !in ? -1 : i == 0 ? root_tok : t.tok[i];
        o.node_parent[base + i] = in ? t.par[i] : -1;
        o.node_depth[base + i] = in ? t.dep[i] : -1;
        o.node_logrho[base + i] = in ? t.lr[i] : 0.0;
    }
    if (o.mask) {
        // ancestor-or-self rows from the parents in LDS (depth <= block steps)
        const int words = (W + 63) / 64;
        for (int i = lane; i < lim; i += kWave) {
            uint64_t w[4] = {0, 0, 0, 0};
            if (i <= n) {
                int u = i;
                for (int step = 0; step <= P.block; ++step) {
                    const uint64_t bit = 1ull << (u & 63);
                    const int qw = u >> 6;
                    w[0] |= qw == 0 ? bit : 0;
                    w[1] |= qw == 1 ? bit : 0;
                    w[2] |= qw == 2 ? bit : 0;
                    w[3] |= qw == 3 ? bit : 0;
                    if (u == 0) break;
                    u = t.par[u];
                }
            }
            uint64_t *row = o.mask + (base + i) * words;
            for (int k = 0; k < words; ++k) row[k] = k == 0 ? w[0] : k == 1 ? w[1] : k == 2 ? w[2] : w[3];
        }
    }
    if (lane == 0) {
        o.n_nodes[b] = n;
        if (o.ahat) o.ahat[b] = ahat;
        if (o.speedup) o.speedup[b] = s_now;
    }
}

// Build sequence b's tree (see build_tree_wave_t), with or without the
// S(N) stop.
template <int SLOTS, bool PREFILLED = false>
__device__ __forceinline__ void build_tree_wave(TreeLds &t, const TreeParams &P, const TreeOut &o, int b, int lane,
                                                int root_tok) {
    if (P.use_stop != 0)
        build_tree_wave_t<SLOTS, PREFILLED, true>(t, P, o, b, lane, root_tok);
    else
        build_tree_wave_t<SLOTS, PREFILLED, false>(t, P, o, b, lane, root_tok);
}

// The outputs of sequence b past the root as if beyond the tree (token,
// parent and depth -1, log rho 0, zero mask rows), by threads t0, t0 +
// nthreads, ...; the tree builder then writes entries 0..n over them.
__device__ __forceinline__ void prefill_tree_outputs(const TreeParams &P, const TreeOut &o, int b, int t0,
                                                     int nthreads) {
    const int W = P.n_max + 1;
    const int64_t base = static_cast<int64_t>(b) * W;
    for (int i = 1 + t0; i < W; i += nthreads) {
        o.node_token[base + i] = -1;
        o.node_parent[base + i] = -1;
        o.node_depth[base + i] = -1;
        o.node_logrho[base + i] = 0.0;
    }
    if (o.mask) {
        const int words = (W + 63) / 64;
        uint64_t *m = o.mask + (base + 1) * words;
        for (int k = t0; k < (W - 1) * words; k += nthreads) m[k] = 0;
    }
}

// Greedy acceptance of sequence b with one wavefront: from the root, step to
// the child carrying the target's greedy token while one exists.  With
// lds_path / lds_acc set, the path (root first) and (A, bonus) are also left
// in LDS for the workgroup.
__device__ __forceinline__ void accept_wave(const int32_t *__restrict__ node_token,
                                            const int32_t *__restrict__ node_parent,
                                            const int32_t *__restrict__ n_nodes,
                                            const int32_t *__restrict__ target_token, int n_max,
                                            int block, int32_t *__restrict__ accept_len,
                                            int32_t *__restrict__ accept_path,
                                            int32_t *__restrict__ bonus_token, int b, int lane,
                                            int *lds_path = nullptr, int *lds_acc = nullptr) {
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
        if (lane == 0) {
            path[A] = u;
            if (lds_path) lds_path[A] = u;
        }
    }
    if (lane == 0) {
        const int bonus = target_token[base + u];
        accept_len[b] = A;
        bonus_token[b] = bonus;
        if (lds_path) lds_path[0] = 0;
        if (lds_acc) {
            lds_acc[0] = A;
            lds_acc[1] = bonus;
        }
    }
}

// KV commit of the accepted path (the verified prefix becomes context; the
// verification's keys and values are kept): for sequence b, tree rows
// path[0..A] (root first) are copied, every KV head at once, after the L
// context rows of b's region ctx_offsets[b] .. ctx_offsets[b+1]-1; rows that
// would pass the region's end are dropped.  One token's keys of every KV
// head are row16 16-byte vectors.
struct CommitArgs {
    const uint4 *k_tree, *v_tree;  // [batch][nq_max][row16]
    uint4 *k_cache, *v_cache;      // [total][row16]
    const int64_t *ctx_offsets;    // [batch + 1]
    int64_t *ctx_lengths;          // [batch], advanced by the rows written
    int32_t *next_root;            // [batch] or null: the bonus token
    int nq_max, row16;
};

// The context length of b, clamped to its region (read before any thread
// of the committing workgroup may advance it).
__device__ __forceinline__ int64_t commit_length(const CommitArgs &c, int b) {
    const int64_t region = c.ctx_offsets[b + 1] - c.ctx_offsets[b];
    const int64_t L = c.ctx_lengths[b];
    return L < 0 ? 0 : (L > region ? region : L);
}

// Threads t, t + nthreads, ... of one workgroup copy the rows; path[0..A]
// are valid tree rows (< nq_max); L from commit_length.
__device__ __forceinline__ void commit_seq(const CommitArgs &c, int b, const int *path, int A,
                                           int bonus, int64_t L, int t, int nthreads) {
    const int64_t base = c.ctx_offsets[b];
    const int64_t room = c.ctx_offsets[b + 1] - base - L;
    const int rows = static_cast<int>(A + 1 < room ? A + 1 : room);
    for (int e = t; e < rows * c.row16; e += nthreads) {
        const int j = e / c.row16;
        const int v = e - j * c.row16;
        const int64_t src = (static_cast<int64_t>(b) * c.nq_max + path[j]) * c.row16 + v;
        const int64_t dst = (base + L + j) * c.row16 + v;
        c.k_cache[dst] = c.k_tree[src];
        c.v_cache[dst] = c.v_tree[src];
    }
    if (t == 0) {
        c.ctx_lengths[b] = L + (rows > 0 ? rows : 0);
        if (c.next_root) c.next_root[b] = bonus;
    }
}

}  // namespace td
