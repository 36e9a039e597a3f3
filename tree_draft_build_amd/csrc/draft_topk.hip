// Stage (a): per-position log-softmax normaliser and top-K over the full
// vocabulary (BASTION, "Methodik" §1: path scores are products of the
// drafter's per-position marginals q_k, so every q_k of a candidate is needed).
//
// One kernel, grid (splits, rows).  Each workgroup streams one contiguous
// slice of one vocabulary row with 16-byte loads (up to 4 per thread in
// flight), keeping per lane a running max m and a float64 sum s of
// exp(x - m), and a sorted register list of candidate keys.
//
// Candidates are 64-bit order keys, ord(logit) << 32 | ~id, so one unsigned
// compare orders them by larger logit, then smaller id, and every
// compare-exchange is branch-free.
//
// Exact pre-filter: after its first batch of loads each wave cuts its lanes
// into KM >= K groups, takes every group's maximum and keeps tau = the
// smallest of them.  Those KM maxima are distinct elements >= tau, so the
// slice's K-th largest element is >= tau and no element below tau can be in
// the top K: only elements >= tau enter a lane's list.
//
// Selection: each wave compacts its lanes' surviving candidates into LDS and
// ranks them by counting (a key's rank = number of keys that beat it; keys
// are distinct), so its K best land in their slots in one parallel pass;
// wave 0 then ranks the 4 waves' winners.  Should a wave hold more than
// kWaveCap candidates (rows of many equal logits), a K-round tournament over
// its lane lists (wave-wide key max per round) takes over.  The
// workgroup publishes its (m, s, K keys) with agent-scope atomic stores and
// counts in; the last workgroup of the row bounds the row's K-th key from
// below by the K-th best partial head, ranks the partial keys above that
// bound the same way, writes lse = M + log(sum_s s_s exp(m_s - M))
// (float64), the ids and log q = l - lse, and resets the row's counter.

#include <algorithm>

#include "step_launch.h"
#include "td_internal.h"
#include "tree_core.h"

namespace td {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBatch = 4;  // 16-byte vectors per thread in flight
constexpr int kCandCap = 512;  // candidates ranked in LDS by counting
constexpr int kWaveCap = kCandCap / kTopkWaves;  // per wave
constexpr float kLog2e = 1.4426950408889634f;

// Order key: larger key = larger logit, then smaller id.  -0 becomes +0 first
// so that the two zeros tie and the id decides.  0 is the empty key.
__device__ __forceinline__ uint64_t cand_key(float v, int id) {
    uint32_t u = __float_as_uint(v + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(id));
}
__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t u = static_cast<uint32_t>(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int key_id(uint64_t k) {
    return static_cast<int>(~static_cast<uint32_t>(k));
}

template <int L>
__device__ __forceinline__ uint64_t xchg_k(uint64_t k) {
    return static_cast<uint64_t>(xchg<L>(static_cast<uint32_t>(k))) |
           (static_cast<uint64_t>(xchg<L>(static_cast<uint32_t>(k >> 32))) << 32);
}
__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    k = kmax(k, xchg_k<0>(k));
    k = kmax(k, xchg_k<1>(k));
    k = kmax(k, xchg_k<2>(k));
    k = kmax(k, xchg_k<3>(k));
    k = kmax(k, xchg_k<4>(k));
    k = kmax(k, xchg_k<5>(k));
    return k;
}

// max over aligned groups of 64/G lanes, then min over the G groups
template <int G>
__device__ __forceinline__ float group_max_min(float v) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32, "group count");
    constexpr int kMaxLevels = G == 4 ? 4 : G == 8 ? 3 : G == 16 ? 2 : 1;
    if constexpr (kMaxLevels > 0) v = fmaxf(v, xchg_f<0>(v));
    if constexpr (kMaxLevels > 1) v = fmaxf(v, xchg_f<1>(v));
    if constexpr (kMaxLevels > 2) v = fmaxf(v, xchg_f<2>(v));
    if constexpr (kMaxLevels > 3) v = fmaxf(v, xchg_f<3>(v));
    if constexpr (kMaxLevels <= 1) v = fminf(v, xchg_f<1>(v));
    if constexpr (kMaxLevels <= 2) v = fminf(v, xchg_f<2>(v));
    if constexpr (kMaxLevels <= 3) v = fminf(v, xchg_f<3>(v));
    v = fminf(v, xchg_f<4>(v));
    v = fminf(v, xchg_f<5>(v));
    return v;
}

// Sorted (descending) list of a lane's best KM keys; 0 marks an empty slot.
template <int KM>
struct KeyList {
    uint64_t k[KM];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int j = 0; j < KM; ++j) k[j] = 0;
    }
    // insert x keeping the order; the last key falls off
    __device__ __forceinline__ void insert(uint64_t x) {
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            const bool sw = x > k[j];
            const uint64_t t = sw ? k[j] : x;
            k[j] = sw ? x : k[j];
            x = t;
        }
    }
    __device__ __forceinline__ void pop_if(bool p) {
#pragma unroll
        for (int j = 0; j + 1 < KM; ++j) k[j] = p ? k[j + 1] : k[j];
        k[KM - 1] = p ? 0 : k[KM - 1];
    }
};

// K-round tournament over the wave's lane lists; win[] is the same in every
// lane afterwards (0 where fewer than K candidates exist).
template <int KM, int KW>
__device__ __forceinline__ void wave_select(KeyList<KW> &l, int K, uint64_t (&win)[KM]) {
#pragma unroll
    for (int r = 0; r < KM; ++r) {
        win[r] = 0;
        if (r < K) {
            const uint64_t best = wave_max_key(l.k[0]);
            win[r] = best;
            l.pop_if(best != 0 && l.k[0] == best);
        }
    }
}

// Workspace layout: for R rows, P = rows * splits partials and B sequences
//   uint32 count[R + B] | double s[P] | float m[P] | uint64 key[P][K]
// (each 16-byte aligned; the B sequence counters serve the fused step).
// count[] must be zero before the first call and is zero again after every
// call.
struct TopkWs {
    unsigned int *count;
    double *s;
    float *m;
    uint64_t *key;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

inline size_t topk_ws_bytes(int64_t rows, int64_t parts, int K) {
    return align16(rows * 4 + rows * 4) + align16(parts * 8) + align16(parts * 4) +
           align16(parts * K * 8);
}

__host__ __device__ inline TopkWs topk_ws(void *base, int64_t rows, int64_t parts, int K) {
    char *p = static_cast<char *>(base);
    TopkWs w;
    w.count = reinterpret_cast<unsigned int *>(p);
    p += align16(rows * 4 + rows * 4);  // row counters, then (up to rows) sequence counters
    w.s = reinterpret_cast<double *>(p);
    p += align16(parts * 8);
    w.m = reinterpret_cast<float *>(p);
    p += align16(parts * 4);
    w.key = reinterpret_cast<uint64_t *>(p);
    (void)K;
    return w;
}

// Cross-workgroup hand-off through the workspace: agent-scope relaxed
// atomic stores and loads (coherent without L2 write-back/invalidate).
template <typename V>
__device__ __forceinline__ void publish(V *p, V x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V fetch(const V *p) {
    return __hip_atomic_load(const_cast<V *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Elements per 16-byte vector.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void unpack(const u32x4 &w, float (&x)[8]) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
        x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
    __device__ __forceinline__ static float scalar(const uint16_t *p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void unpack(const u32x4 &w, float (&x)[4]) {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
    __device__ __forceinline__ static float scalar(const float *p) { return *p; }
};

// Lane state: running max m, float64 sum s of exp(x - m), candidate list.
template <int KM>
struct LaneAcc {
    float m;
    double s;
    KeyList<KM> top;

    template <int N>
    __device__ __forceinline__ void add_exp(const float (&x)[N]) {
        float vmax = x[0];
#pragma unroll
        for (int j = 1; j < N; ++j) vmax = fmaxf(vmax, x[j]);
        if (vmax > m) {  // rescale the running sum to the new max
            s *= static_cast<double>(__builtin_amdgcn_exp2f((m - vmax) * kLog2e));
            m = vmax;
        }
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < N; ++j) ls += __builtin_amdgcn_exp2f((x[j] - m) * kLog2e);
        s += static_cast<double>(ls);
    }
    // candidates: every element >= tau (the list keeps the lane's best KM).
    // One insertion per loop trip over the lane's pending elements, so the
    // wave pays for max-over-lanes insertions rather than for every element.
    template <int N>
    __device__ __forceinline__ void add_cand(const float (&x)[N], int base_id, float tau) {
        uint32_t pend = 0;
#pragma unroll
        for (int j = 0; j < N; ++j) pend |= (x[j] >= tau ? 1u : 0u) << j;
        while (pend) {
            const int j = __builtin_ctz(pend);
            pend &= pend - 1;
            float xj = x[0];
#pragma unroll
            for (int q = 1; q < N; ++q) xj = (q == j) ? x[q] : xj;
            top.insert(cand_key(xj, base_id + j));
        }
    }
};

// Exact top-K of C distinct nonzero keys buf[0..C) (in LDS) by counting: the
// key beaten by exactly r others is the (r+1)-th best.  out[0..K) must hold 0
// beforehand (slots stay 0 when C < K).
// Same, for a buffer that may hold empty (0) slots, which are skipped.
__device__ __forceinline__ void rank_select_nz(const uint64_t *buf, int C, int K, uint64_t *out,
                                               int tid, int nthreads) {
    for (int e = tid; e < C; e += nthreads) {
        const uint64_t mine = buf[e];
        if (mine == 0) continue;
        int rank = 0;
        for (int u = 0; u < C; ++u) rank += buf[u] > mine;
        if (rank < K) out[rank] = mine;
    }
}

__device__ __forceinline__ void rank_select(const uint64_t *buf, int C, int K, uint64_t *out,
                                            int tid, int nthreads) {
    for (int e = tid; e < C; e += nthreads) {
        const uint64_t mine = buf[e];
        int rank = 0;
        int u = 0;
        for (; u + 4 <= C; u += 4)
            rank += (buf[u] > mine) + (buf[u + 1] > mine) + (buf[u + 2] > mine) + (buf[u + 3] > mine);
        for (; u < C; ++u) rank += buf[u] > mine;
        if (rank < K) out[rank] = mine;
    }
}

// FUSE: the verify step's first kernel.  The row outputs are then written
// with agent-scope atomic stores, and the last row of each sequence to finish
// builds that sequence's tree (and mask rows) from them in wave 0.
template <typename T, int KM, bool FUSE, int SLOTS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const T *__restrict__ logits,
                                                            int vocab, int64_t pos_stride,
                                                            int slice, int splits, int K, void *ws,
                                                            int64_t parts,
                                                            int32_t *__restrict__ topk_id,
                                                            double *__restrict__ topk_logq,
                                                            double *__restrict__ lse_out,
                                                            TreeParams tp, TreeOut to) {
    constexpr int N = Vec<T>::N;
    const int sp = blockIdx.x;
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int lo = sp * slice;
    const int hi = min(vocab, lo + slice);
    const T *rowp = logits + static_cast<int64_t>(row) * pos_stride;

    __shared__ int sm_wcnt[kTopkWaves];
    __shared__ float sm_m[kTopkWaves];
    __shared__ double sm_s[kTopkWaves];
    __shared__ uint64_t sm_cand[kCandCap];
    __shared__ uint64_t sm_wave[kTopkWaves][KM];
    __shared__ uint64_t sm_win[KM];
    __shared__ uint64_t sm_head[64];
    __shared__ uint64_t sm_tau_key;
    __shared__ int sm_cnt;
    __shared__ int sm_last;

    LaneAcc<KM> acc;
    acc.m = -INFINITY;
    acc.s = 0.0;
    acc.top.init();

    // scalar head up to the first 16-byte boundary (rows need only element
    // alignment), full 16-byte vectors, then a scalar tail
    const int head = static_cast<int>(
        ((16 - (reinterpret_cast<uintptr_t>(rowp + lo) & 15)) & 15) / sizeof(T));
    const int vlo = min(hi, lo + head);
    const int nvec = (hi - vlo) / N;
    const int tail0 = vlo + nvec * N;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + vlo);

    // ---- first batch: loads in flight, exp sums, then the pre-filter ----
    float hx[1] = {-INFINITY};
    const bool has_head = tid < vlo - lo;
    const int head_id = lo + tid;
    if (has_head) hx[0] = Vec<T>::scalar(rowp + head_id);
    u32x4 w[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int i = tid + u * kTopkThreads;
        if (i < nvec) w[u] = __builtin_nontemporal_load(vp + i);
    }
    float lmax = has_head ? hx[0] : -INFINITY;
    if (has_head) acc.add_exp(hx);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int i = tid + u * kTopkThreads;
        if (i < nvec) {
            float x[N];
            Vec<T>::unpack(w[u], x);
            acc.add_exp(x);
#pragma unroll
            for (int j = 0; j < N; ++j) lmax = fmaxf(lmax, x[j]);
        }
    }
    // Pre-filter bound: cut the wave into KM groups of 64/KM lanes; tau = the
    // smallest of the groups' maxima.  The KM group maxima are KM >= K
    // distinct elements >= tau, so the slice's K-th largest is >= tau.
    const float tau = group_max_min<KM>(lmax);
    if (has_head) acc.add_cand(hx, head_id, tau);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int i = tid + u * kTopkThreads;
        if (i < nvec) {
            float x[N];
            Vec<T>::unpack(w[u], x);
            acc.add_cand(x, vlo + i * N, tau);
        }
    }
    // ---- remaining batches ----
    for (int i0 = tid + kBatch * kTopkThreads; i0 < nvec; i0 += kBatch * kTopkThreads) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * kTopkThreads;
            if (i < nvec) w[u] = __builtin_nontemporal_load(vp + i);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * kTopkThreads;
            if (i < nvec) {
                float x[N];
                Vec<T>::unpack(w[u], x);
                acc.add_exp(x);
                acc.add_cand(x, vlo + i * N, tau);
            }
        }
    }
    for (int e = tail0 + tid; e < hi; e += kTopkThreads) {
        float x[1] = {Vec<T>::scalar(rowp + e)};
        acc.add_exp(x);
        acc.add_cand(x, e, tau);
    }

    // ---- workgroup partial: (m, s) and the top K of the lanes' lists ----
    const float wm = wave_max(acc.m);
    const double contrib =
        (acc.m == -INFINITY) ? 0.0
                             : acc.s * static_cast<double>(__builtin_amdgcn_exp2f((acc.m - wm) * kLog2e));
    const double ws_sum = wave_sum(contrib);
    // per wave: compact the lanes' candidates into LDS and rank them
    int n_l = 0;
#pragma unroll
    for (int j = 0; j < KM; ++j) n_l += acc.top.k[j] != 0;
    uint64_t *wcand = &sm_cand[wave * kWaveCap];
    if (lane == 0) sm_wcnt[wave] = 0;
    if (lane < KM) sm_wave[wave][lane] = 0;
    __builtin_amdgcn_wave_barrier();
    const int off = atomicAdd(&sm_wcnt[wave], n_l);
    __builtin_amdgcn_wave_barrier();
    const int Cw = sm_wcnt[wave];  // same for every lane of the wave
    if (Cw <= kWaveCap) {
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < n_l) wcand[off + j] = acc.top.k[j];
        __builtin_amdgcn_wave_barrier();
        rank_select(wcand, Cw, K, sm_wave[wave], lane, kWave);
    } else {
        // many equal logits: a K-round tournament over the lane lists
        uint64_t win[KM];
        wave_select<KM, KM>(acc.top, K, win);
        if (lane == 0)
#pragma unroll
            for (int j = 0; j < KM; ++j) sm_wave[wave][j] = win[j];
    }
    if (lane == 0) {
        sm_m[wave] = wm;
        sm_s[wave] = ws_sum;
    }
    __syncthreads();
    // the 4 waves' winners (distinct keys) ranked the same way
    if (tid < KM) sm_win[tid] = 0;
    __syncthreads();
    if (wave == 0) {
        uint64_t *all = &sm_wave[0][0];
        rank_select_nz(all, kTopkWaves * KM, K, sm_win, lane, kWave);
    }
    __syncthreads();

    const int64_t rows = gridDim.y;
    TopkWs ws_ = topk_ws(ws, rows, parts, K);
    const int64_t part = static_cast<int64_t>(row) * splits + sp;
    // publish with agent-scope atomic stores (coherent across the chip's L2
    // caches by themselves); each wave waits for its own stores, then one
    // thread counts in
    if (tid < K) publish(&ws_.key[part * K + tid], sm_win[tid]);
    if (tid == 0) {
        float M = sm_m[0];
#pragma unroll
        for (int q = 1; q < kTopkWaves; ++q) M = fmaxf(M, sm_m[q]);
        double S = 0.0;
#pragma unroll
        for (int q = 0; q < kTopkWaves; ++q)
            if (sm_m[q] != -INFINITY)
                S += sm_s[q] * static_cast<double>(__builtin_amdgcn_exp2f((sm_m[q] - M) * kLog2e));
        publish(&ws_.m[part], M);
        publish(&ws_.s[part], S);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        sm_last = __hip_atomic_fetch_add(&ws_.count[row], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == static_cast<unsigned>(splits - 1);
    __syncthreads();
    if (!sm_last) return;

    // ---- last workgroup of the row: merge the row's partials ----
    // tau_key = K-th best of the partials' heads bounds the row's K-th best
    // from below; only keys >= tau_key can be in the row's top K.
    const int PK = splits * K;
    if (tid < splits) sm_head[tid] = fetch(&ws_.key[(static_cast<int64_t>(row) * splits + tid) * K]);
    if (tid == 0) {
        sm_cnt = 0;
        sm_tau_key = 0;
    }
    if (tid < KM) sm_win[tid] = 0;
    __syncthreads();
    if (tid < splits && splits >= K) {
        const uint64_t h = sm_head[tid];
        int rank = 0;
        for (int u = 0; u < splits; ++u) rank += sm_head[u] > h;
        if (rank == K - 1) sm_tau_key = h;
    }
    __syncthreads();
    const uint64_t tau_key = sm_tau_key;
    for (int e = tid; e < PK; e += kTopkThreads) {
        const uint64_t k = fetch(&ws_.key[static_cast<int64_t>(row) * PK + e]);
        if (k != 0 && k >= tau_key) {
            const int o = atomicAdd(&sm_cnt, 1);
            if (o < kCandCap) sm_cand[o] = k;
        }
    }
    __syncthreads();
    const int C2 = sm_cnt;
    if (C2 <= kCandCap) {
        rank_select(sm_cand, C2, K, sm_win, tid, kTopkThreads);
    } else if (wave == 0) {
        // many equal logits: tournament over the partial lists
        KeyList<KM> t;
        t.init();
        if (lane < splits)
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (j < K) t.k[j] = fetch(&ws_.key[(static_cast<int64_t>(row) * splits + lane) * K + j]);
        uint64_t win[KM];
        wave_select<KM, KM>(t, K, win);
        if (lane == 0)
#pragma unroll
            for (int j = 0; j < KM; ++j) sm_win[j] = win[j];
    }
    __syncthreads();
    if (wave != 0) return;
    float m = -INFINITY;
    double ssum = 0.0;
    if (lane < splits) {
        const int64_t pt = static_cast<int64_t>(row) * splits + lane;
        m = fetch(&ws_.m[pt]);
        ssum = fetch(&ws_.s[pt]);
    }
    const float M = wave_max(m);
    const double c = (m == -INFINITY) ? 0.0 : ssum * exp(static_cast<double>(m) - static_cast<double>(M));
    const double S = wave_sum(c);
    const double lse = static_cast<double>(M) + log(S);
    if (lane < K) {
        const uint64_t k = sm_win[lane];
        const int32_t id = key_id(k);
        const double lq = static_cast<double>(key_value(k)) - lse;
        if constexpr (FUSE) {
            publish(&topk_id[static_cast<int64_t>(row) * K + lane], id);
            publish(&topk_logq[static_cast<int64_t>(row) * K + lane], lq);
        } else {
            topk_id[static_cast<int64_t>(row) * K + lane] = id;
            topk_logq[static_cast<int64_t>(row) * K + lane] = lq;
        }
    }
    if (lane == 0) {
        lse_out[row] = lse;
        ws_.count[row] = 0u;  // ready for the next call
    }
    if constexpr (FUSE) {
        // sequence completion: the last of its rows builds the tree
        __shared__ TreeLds tl;
        const int b = row / tp.block;
        unsigned int *seq_count = ws_.count + rows;
        __builtin_amdgcn_s_waitcnt(0);  // this row's outputs are complete
        int last = 0;
        if (lane == 0)
            last = __hip_atomic_fetch_add(&seq_count[b], 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) ==
                   static_cast<unsigned>(tp.block - 1);
        last = __builtin_amdgcn_readfirstlane(last);
        if (!last) return;
        const int BK = tp.block * K;
        for (int e = lane; e < BK; e += kWave) {
            tl.ids[e] = fetch(&topk_id[static_cast<int64_t>(b) * BK + e]);
            tl.lq[e] = fetch(&topk_logq[static_cast<int64_t>(b) * BK + e]);
        }
        wave_lds_sync();
        build_tree_wave<SLOTS>(tl, tp, to, b, lane);
        if (lane == 0) seq_count[b] = 0u;
    }
}

// Split plan: enough workgroups to cover the chip, at least kMinSlice
// elements per workgroup, at most one partial per lane of the merge wave.
constexpr int kTargetWgs = 1024;
constexpr int kMinSlice = 4096;

struct TopkPlan {
    int splits;
    int slice;
};

inline TopkPlan topk_plan(int64_t rows, int vocab) {
    int64_t want = (kTargetWgs + rows - 1) / rows;
    int64_t cap = (vocab + kMinSlice - 1) / kMinSlice;
    int splits = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>({want, cap, 64})));
    int slice = (vocab + splits - 1) / splits;
    slice = (slice + 7) & ~7;  // 16-byte aligned slices for both element types
    splits = (vocab + slice - 1) / slice;
    return {splits, slice};
}

template <typename T, int KM, bool FUSE, int SLOTS>
void launch_topk(const void *logits, int rows, int vocab, int64_t pos_stride, int K,
                 const TopkPlan &pl, void *ws, int32_t *topk_id, double *topk_logq, double *lse,
                 const TreeParams &tp, const TreeOut &to, hipStream_t st) {
    const int64_t parts = static_cast<int64_t>(rows) * pl.splits;
    hipLaunchKernelGGL((topk_kernel<T, KM, FUSE, SLOTS>), dim3(pl.splits, rows), dim3(kTopkThreads),
                       0, st, static_cast<const T *>(logits), vocab, pos_stride, pl.slice, pl.splits,
                       K, ws, parts, topk_id, topk_logq, lse, tp, to);
}

template <typename T, bool FUSE, int SLOTS>
void launch_topk_k(const void *logits, int rows, int vocab, int64_t pos_stride, int K,
                   const TopkPlan &pl, void *ws, int32_t *topk_id, double *topk_logq, double *lse,
                   const TreeParams &tp, const TreeOut &to, hipStream_t st) {
    if (K <= 4)
        launch_topk<T, 4, FUSE, SLOTS>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id, topk_logq,
                                       lse, tp, to, st);
    else if (K <= 8)
        launch_topk<T, 8, FUSE, SLOTS>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id, topk_logq,
                                       lse, tp, to, st);
    else if (K <= 16)
        launch_topk<T, 16, FUSE, SLOTS>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id,
                                        topk_logq, lse, tp, to, st);
    else
        launch_topk<T, 32, FUSE, SLOTS>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id,
                                        topk_logq, lse, tp, to, st);
}

template <bool FUSE, int SLOTS>
void launch_topk_dt(const void *logits, td_dtype dtype, int rows, int vocab, int64_t pos_stride,
                    int K, void *ws, int32_t *topk_id, double *topk_logq, double *lse,
                    const TreeParams &tp, const TreeOut &to, hipStream_t st) {
    const TopkPlan pl = topk_plan(rows, vocab);
    if (dtype == TD_BF16)
        launch_topk_k<uint16_t, FUSE, SLOTS>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id,
                                             topk_logq, lse, tp, to, st);
    else
        launch_topk_k<float, FUSE, SLOTS>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id,
                                          topk_logq, lse, tp, to, st);
}

}  // namespace

size_t topk_workspace_bytes(int batch, int block, int vocab, int K) {
    const int64_t rows = static_cast<int64_t>(batch) * block;
    const TopkPlan pl = topk_plan(rows, vocab);
    return topk_ws_bytes(rows, rows * pl.splits, K);
}

void launch_topk_tree(const void *logits, td_dtype dtype, int batch, int block, int vocab,
                      int64_t pos_stride, int K, void *ws, int32_t *topk_id, double *topk_logq,
                      double *lse, const TreeParams &tp, const TreeOut &to, hipStream_t st) {
    const int rows = batch * block;
    switch (tree_slots(tp.n_max)) {
    case 1:
        launch_topk_dt<true, 1>(logits, dtype, rows, vocab, pos_stride, K, ws, topk_id, topk_logq,
                                lse, tp, to, st);
        break;
    case 2:
        launch_topk_dt<true, 2>(logits, dtype, rows, vocab, pos_stride, K, ws, topk_id, topk_logq,
                                lse, tp, to, st);
        break;
    case 4:
        launch_topk_dt<true, 4>(logits, dtype, rows, vocab, pos_stride, K, ws, topk_id, topk_logq,
                                lse, tp, to, st);
        break;
    default:
        launch_topk_dt<true, 8>(logits, dtype, rows, vocab, pos_stride, K, ws, topk_id, topk_logq,
                                lse, tp, to, st);
        break;
    }
}

}  // namespace td

using namespace td;

extern "C" size_t td_draft_topk_workspace(int32_t batch, int32_t block, int32_t vocab, int32_t K) {
    if (batch <= 0 || block <= 0 || vocab <= 0 || K <= 0) return 0;
    return topk_workspace_bytes(batch, block, vocab, K);
}

td_status td::check_topk_args(const void *logits, td_dtype dtype, int32_t batch, int32_t block,
                             int32_t vocab, int64_t pos_stride, int32_t K, const int32_t *topk_id,
                             const double *topk_logq, const double *lse) {
    if (!logits || !topk_id || !topk_logq || !lse)
        return fail(TD_EINVAL, "draft_topk: null pointer argument");
    if (batch <= 0 || block <= 0 || vocab <= 0 || K <= 0)
        return fail(TD_EINVAL, "draft_topk: batch, block, vocab and K must be positive");
    if (K > vocab) return fail(TD_EINVAL, "draft_topk: K exceeds the vocabulary");
    if (K > TD_MAX_TOPK) return fail(TD_ECAPACITY, "draft_topk: K above TD_MAX_TOPK");
    if (block > TD_MAX_BLOCK) return fail(TD_ECAPACITY, "draft_topk: block above TD_MAX_BLOCK");
    if (batch > TD_MAX_BATCH) return fail(TD_ECAPACITY, "draft_topk: batch above TD_MAX_BATCH");
    if (vocab > TD_MAX_VOCAB) return fail(TD_ECAPACITY, "draft_topk: vocab above TD_MAX_VOCAB");
    if (dtype != TD_F32 && dtype != TD_BF16)
        return fail(TD_EUNSUPPORTED, "draft_topk: dtype must be TD_F32 or TD_BF16");
    if (pos_stride < vocab) return fail(TD_EINVAL, "draft_topk: pos_stride < vocab");
    const int esz = dtype == TD_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(logits) % esz) != 0)
        return fail(TD_EINVAL, "draft_topk: logits must be aligned to the element size");
    if (!aligned8(topk_logq) || !aligned8(lse))
        return fail(TD_EINVAL, "draft_topk: misaligned float64 output");
    return TD_OK;
}

extern "C" td_status td_draft_topk(const void *logits, td_dtype dtype, int32_t batch, int32_t block,
                                   int32_t vocab, int64_t pos_stride, int32_t K, int32_t *topk_id,
                                   double *topk_logq, double *lse, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    clear_error();
    const td_status st =
        check_topk_args(logits, dtype, batch, block, vocab, pos_stride, K, topk_id, topk_logq, lse);
    if (st != TD_OK) return st;
    if (!workspace || !aligned16(workspace))
        return fail(TD_EINVAL, "td_draft_topk: null or misaligned workspace");
    if (workspace_bytes < td_draft_topk_workspace(batch, block, vocab, K))
        return fail(TD_EINVAL, "td_draft_topk: workspace too small");
    const TreeParams tp{};
    const TreeOut to{};
    launch_topk_dt<false, 1>(logits, dtype, batch * block, vocab, pos_stride, K, workspace, topk_id,
                             topk_logq, lse, tp, to, as_stream(stream));
    return check_launch("td_draft_topk");
}
