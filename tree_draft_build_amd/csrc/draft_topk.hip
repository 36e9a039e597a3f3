// Stage (a): per-position log-softmax normaliser and top-K over the full
// vocabulary (BASTION, "Methodik" §1: path scores are products of the
// drafter's per-position marginals q_k, so every q_k of a candidate is needed).
//
// One kernel, grid (splits, rows).  Each workgroup streams one contiguous
// slice of one vocabulary row with 16-byte loads (two batches of four per
// thread in flight), keeping per lane a reference max m and a float64 sum s
// of exp(x - m).  On whole batches the reference moves only when the batch
// maximum passes it by more than 2^8 (one ballot per batch), and the
// batch's 32 terms are summed pairwise in fp32 before they reach s.
//
// Candidates are 64-bit order keys, ord(logit) << 32 | ~id, so one unsigned
// compare orders them by larger logit, then smaller id.
//
// Exact pre-filter: after its first batch of loads each wave cuts its lanes
// into KM >= K groups, takes every group's maximum and keeps tau = the
// smallest of them.  Those KM maxima are distinct elements >= tau, so the
// slice's K-th largest element is >= tau and no element below tau can be in
// the top K.  The bound is raised the same way from the lanes' running
// maxima as the stream goes on, and shared among the waves through LDS.
//
// Candidates: the elements >= tau are appended to the wave's LDS region,
// one ballot per element position and one store per candidate (a batch
// whose lanes all stay below tau costs one ballot).  Selection: the waves'
// bounds are pooled (their maximum still bounds the workgroup's K-th
// largest from below), each wave packs its region's keys at or above that
// bound, and every thread holding a key ranks it by counting the keys that
// beat it (keys are distinct), so the K best land in their slots in one
// parallel pass.  Should a region overflow (rows of many equal or ascending
// logits), the workgroup selects again from its slice with sorted per-lane
// lists of the best KM keys above the pooled bound.  The
// workgroup publishes its (m, s, K keys) as epoch-tagged words; the row's
// highest slice waits for every tag, bounds the row's K-th key from below by
// the K-th best partial head, ranks the partial keys above that bound the
// same way, and writes lse = M + log(sum_s s_s exp(m_s - M)) (float64), the
// ids and log q = l - lse.

#include <algorithm>
#include <type_traits>

#include "attn_split.h"
#include "step_launch.h"
#include "td_internal.h"
#include "tree_core.h"

namespace td {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBatch = 4;  // 16-byte vectors per thread in flight
constexpr int kCandCap = 1024;  // candidates held in LDS (kWaveCap per wave)
// Words of a row's partials held by the merger: splits * (2K + 3) with
// splits <= min(64, 1024 / K) is at most 2240 for every K <= 32.
constexpr int kMergeWords = 2304;
constexpr int kWaveCap = kCandCap / kTopkWaves;  // per wave
static_assert(kWaveCap % 8 == 0 && kWaveCap >= 32, "regions hold whole groups of 8 keys");
constexpr float kLazyTop = 8.f;  // log2 slack of the fast path's reference maximum

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

// Workspace layout for R rows of `splits` partials each (zero-filled once,
// and again whenever the problem's shape changes):
//   uint32 status[4]                bit kStatusMerge / kStatusTree is set when
//          a row merger / tree builder gave up waiting for a hand-off (read
//          and cleared by td_workspace_status)
//   uint64 part[R][splits][2K + 4]  per workgroup: its epoch (word 0), then
//          the tagged words of its partial: key j low/high halves (1 + 2j,
//          2 + 2j), log2 max (2K + 1), float64 sum (2K + 2, 2K + 3)
//   uint64 rowrec[R][3K]            tagged row results for the fused tree
//          build: id j (j), log q j low/high halves (K + 2j, K + 2j + 1)
// Each workgroup reads only its own epoch word and advances it when done,
// so every epoch of a workspace counts the calls made with it.  A tagged
// word carries 32 data bits under a 32-bit tag (the epoch plus one) and is
// written and read as one 8-byte atomic, so a reader takes a word only once
// the word of this call has landed.
struct TopkWs {
    uint32_t *status;
    uint64_t *part;
    uint64_t *rowrec;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }
__host__ __device__ inline int part_words(int K) { return 2 * K + 3; }  // data words

inline size_t topk_ws_bytes(int64_t rows, int64_t parts, int K) {
    return kStatusBytes + align16(parts * (part_words(K) + 1) * 8) + align16(rows * 3 * K * 8);
}

__host__ __device__ inline TopkWs topk_ws(void *base, int64_t rows, int64_t parts, int K) {
    char *p = static_cast<char *>(base);
    TopkWs w;
    w.status = reinterpret_cast<uint32_t *>(p);
    p += kStatusBytes;
    w.part = reinterpret_cast<uint64_t *>(p);
    p += align16(parts * (part_words(K) + 1) * 8);
    w.rowrec = reinterpret_cast<uint64_t *>(p);
    (void)rows;
    return w;
}

// Agent-scope relaxed atomics: coherent across the chip's L2 caches by
// themselves (no cache write-back or invalidate).
template <typename V>
__device__ __forceinline__ V fetch(const V *p) {
    return __hip_atomic_load(const_cast<V *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void publish(V *p, V x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_word(uint64_t *p, uint32_t data, uint32_t tag) {
    publish(p, (static_cast<uint64_t>(tag) << 32) | data);
}

// Polls of words whose writers have not landed them yet, per get_words call.
// Every awaited word comes from a workgroup of lower index in the same
// launch, which the dispatcher normally starts before the waiting one, so
// the wait is a few microseconds.  The bound guards against a broken
// protocol (a workspace not re-zeroed after a shape change, or workgroups
// started out of index order while the waiting ones fill the chip): the
// waiter then gives up, its outputs carry the documented sentinels (lse NaN,
// n_nodes -1) and it sets its bit in the workspace status word.
constexpr int kSpinLimit = 1 << 16;

__device__ __forceinline__ void raise_status(uint32_t *status, uint32_t bit) {
    __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads n <= NW tagged words p[idx[u]] (all loads in flight at once) into
// out[u]; returns false if some word never carried the tag.  Every poll
// re-reads all words still missing at once, so a late writer costs one
// round trip after it lands, not one per word.
template <int NW>
__device__ __forceinline__ bool get_words(const uint64_t *p, const int (&idx)[NW], int n,
                                          uint32_t tag, uint32_t (&out)[NW]) {
    uint64_t v[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u)
        if (u < n) v[u] = fetch(p + idx[u]);
    auto tagged = [&](int u) { return u >= n || static_cast<uint32_t>(v[u] >> 32) == tag; };
    for (int spins = 0; spins < kSpinLimit; ++spins) {
        bool all = true;
#pragma unroll
        for (int u = 0; u < NW; ++u) all = all && tagged(u);
        if (all) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < NW; ++u)
            if (!tagged(u)) v[u] = fetch(p + idx[u]);
    }
    bool ok = true;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        ok = ok && tagged(u);
        out[u] = u < n ? static_cast<uint32_t>(v[u]) : 0;
    }
    return ok;
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

// Lane state: reference max m (and ml = m log2 e) and the float64 sum s of
// 2^(x log2 e - ml) = exp(x - m).
struct LaneAcc {
    float m, ml;
    double s;

    __device__ __forceinline__ void init() {
        m = -INFINITY;
        ml = -INFINITY;
        s = 0.0;
    }
    template <int N>
    __device__ __forceinline__ static float vmax(const float (&x)[N]) {
        float v = x[0];
#pragma unroll
        for (int j = 1; j < N; ++j) v = fmaxf(v, x[j]);
        return v;
    }
    template <int N>
    __device__ __forceinline__ void add_exp(const float (&x)[N], float vm) {
        if (vm > m) {  // rescale the running sum to the new max
            const float nl = vm * kLog2e;
            s *= static_cast<double>(__builtin_amdgcn_exp2f(ml - nl));
            m = vm;
            ml = nl;
        }
        if (m != -INFINITY) {  // elements of -inf add nothing
            float ls = 0.f;
#pragma unroll
            for (int j = 0; j < N; ++j) ls += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -ml));
            s += static_cast<double>(ls);
        }
    }
    // A batch of NB full vectors with maximum bm, on the fast path: the
    // reference maximum moves only when the batch passes it by more than
    // 2^kLazyTop (one ballot per batch), so exponent arguments stay <= 8 and
    // fp32 keeps them to a few ulp; the batch's terms are summed pairwise
    // in fp32 and added to the float64 sum once.  With ml = -inf the batch
    // holds only -inf elements (a finite one moves the reference), and an
    // offset of 0 maps them to exp2(-inf) = 0.
    template <int NB, int N>
    __device__ __forceinline__ void add_batch(const float (&x)[NB][N], float bm) {
        const float bl = bm * kLog2e;
        if (__ballot(bl > ml + kLazyTop)) {
            if (bl > ml + kLazyTop) {
                s *= static_cast<double>(__builtin_amdgcn_exp2f(ml - bl));
                m = bm;
                ml = bl;
            }
        }
        const float off = ml == -INFINITY ? 0.f : -ml;
        float e[NB * N];
#pragma unroll
        for (int u = 0; u < NB; ++u)
#pragma unroll
            for (int j = 0; j < N; ++j) e[u * N + j] = __builtin_amdgcn_exp2f(fmaf(x[u][j], kLog2e, off));
#pragma unroll
        for (int w = 1; w < NB * N; w *= 2)
#pragma unroll
            for (int j = 0; j + w < NB * N; j += 2 * w) e[j] += e[j + w];
        s += static_cast<double>(e[0]);
    }
};

// Number of keys in buf[0..n8) that beat x: buf is 16-byte aligned LDS, n8 a
// multiple of 8, and every lane of the wave reads the same addresses
// (broadcast loads, no bank conflicts).
__device__ __forceinline__ int count_above_lds(const uint64_t *buf, int n8, uint64_t x) {
    const u64x2 *b = reinterpret_cast<const u64x2 *>(buf);
    int r = 0;
    for (int u = 0; u < n8 / 2; u += 4) {
        const u64x2 a = b[u], c = b[u + 1], d = b[u + 2], e = b[u + 3];
        r += (a.x > x) + (a.y > x) + (c.x > x) + (c.y > x) + (d.x > x) + (d.y > x) + (e.x > x) + (e.y > x);
    }
    return r;
}

// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ int lane_rank(uint64_t m) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

__device__ __forceinline__ uint64_t readlane64(uint64_t x, int j) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), j);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), j);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Exclusive prefix sum over the wave's lanes of v in [0, 2^BITS), and the
// wave's total, from one ballot per bit.
template <int BITS>
__device__ __forceinline__ int wave_prefix(int v, int lane, int &total) {
    const uint64_t below = (1ull << lane) - 1;
    int off = 0;
    total = 0;
#pragma unroll
    for (int bit = 0; bit < BITS; ++bit) {
        const uint64_t m = __ballot((v >> bit) & 1);
        off += __popcll(m & below) << bit;
        total += __popcll(m) << bit;
    }
    return off;
}

// kBatch vectors per thread; indices past the slice repeat its last vector
// (same cache lines), so every load is issued and the loads in flight can
// be counted exactly.  Requires last >= 0.
template <typename T>
__device__ __forceinline__ void load_batch(u32x4 (&w)[kBatch], const u32x4 *vp, int i0, int last) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) w[u] = __builtin_nontemporal_load(vp + min(i0 + u * kTopkThreads, last));
}

// Hand-off protocol (no writer ever waits for its own stores, and no word is
// contended): every workgroup reads its epoch with its first loads in
// flight and leaves its partial as tagged words; the row's last slice
// (highest workgroup index of the row) merges the row, polling the other
// partials until they carry this call's tag.
//
// FUSE: the verify step's first kernel.  The row mergers also leave their
// row's results as tagged words, and the merger of each sequence's last row
// gathers them and builds that sequence's tree (and mask rows) in wave 0.
// The workgroup's LDS (the verify step's fused first kernel overlays it with
// the context split's key buffer).
struct NoTree {};
template <int KM, bool FUSE>
struct TopkLds {
    float m[kTopkWaves];
    double s[kTopkWaves];
    alignas(16) uint64_t cand[kCandCap];
    float tau[kTopkWaves];
    bool over[kTopkWaves];
    alignas(16) uint64_t wtop[kTopkWaves * TD_MAX_TOPK];
    alignas(16) float live[kTopkWaves];
    alignas(16) uint64_t heads[kWave];
    int cnt[kTopkWaves];
    uint64_t win[KM];
    uint32_t part[kMergeWords];
    uint32_t epoch;
    int fail;
    double lse;
    std::conditional_t<FUSE, TreeLds, NoTree> tl;
};

// Workgroup (slice sp, logit row `row`) of a launch over `rows` rows.
template <typename T, int KM, bool FUSE, int SLOTS>
__device__ __forceinline__ void topk_body(const T *__restrict__ logits, int vocab, int64_t pos_stride,
                                          int slice, int splits, int K, void *ws,
                                          int32_t *__restrict__ topk_id,
                                          double *__restrict__ topk_logq,
                                          double *__restrict__ lse_out, const TreeParams &tp,
                                          const TreeOut &to, int sp, int row, int rows,
                                          TopkLds<KM, FUSE> &L) {
    constexpr int N = Vec<T>::N;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int lo = sp * slice;
    const int hi = min(vocab, lo + slice);
    const T *rowp = logits + static_cast<int64_t>(row) * pos_stride;
    const TopkWs W = topk_ws(ws, rows, static_cast<int64_t>(rows) * splits, K);
    const int PW = part_words(K);

    float(&sm_m)[kTopkWaves] = L.m;
    double(&sm_s)[kTopkWaves] = L.s;
    uint64_t(&sm_cand)[kCandCap] = L.cand;
    float(&sm_tau)[kTopkWaves] = L.tau;
    bool(&sm_over)[kTopkWaves] = L.over;
    uint64_t(&sm_wtop)[kTopkWaves * TD_MAX_TOPK] = L.wtop;
    float(&sm_live)[kTopkWaves] = L.live;
    static_assert(kTopkWaves == 4, "the live bounds are read as one 16-byte vector");
    uint64_t(&sm_heads)[kWave] = L.heads;
    int(&sm_cnt)[kTopkWaves] = L.cnt;
    uint64_t(&sm_win)[KM] = L.win;
    uint32_t(&sm_part)[kMergeWords] = L.part;
    uint32_t &sm_epoch = L.epoch;
    int &sm_fail = L.fail;

    LaneAcc acc;
    acc.init();
    // This wave's candidate region: the keys of the elements that reached the
    // wave's bound when they were seen, appended in any order.  wn counts
    // every append (wave-uniform); keys past kWaveCap are not stored, and the
    // slice is then selected again on the exact path after the stream.
    uint64_t *const wcand = &sm_cand[wave * kWaveCap];
    int wn = 0;
    bool wover = false;  // some append found the region full (wave-uniform)

    // scalar head up to the first 16-byte boundary (rows need only element
    // alignment), full 16-byte vectors, then a scalar tail
    const int head = static_cast<int>(
        ((16 - (reinterpret_cast<uintptr_t>(rowp + lo) & 15)) & 15) / sizeof(T));
    const int vlo = min(hi, lo + head);
    const int nvec = (hi - vlo) / N;
    const int tail0 = vlo + nvec * N;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + vlo);
    constexpr int kStep = kBatch * kTopkThreads;

    // ---- the head element, the first two batches, then the row ticket ----
    // (loads complete in issue order: every thread loads the head element,
    // lanes past the head an element of the row that is not used, so that
    // waiting for it never waits for the batches)
    const bool has_head = tid < vlo - lo;
    const int head_id = lo + tid;
    const float hraw = Vec<T>::scalar(rowp + (has_head ? head_id : min(lo, vocab - 1)));
    // The batches' loads are issued unconditionally too: a slice without a
    // whole vector reads the 16-byte block holding an element of the row
    // (memory of the row's page), whose values are not used.
    const T *blk = rowp + min(lo, vocab - 1);
    blk -= (reinterpret_cast<uintptr_t>(blk) & 15) / sizeof(T);  // pointer arithmetic: stays global
    const u32x4 *vld = nvec > 0 ? vp : reinterpret_cast<const u32x4 *>(blk);
    const int last = max(nvec - 1, 0);
    u32x4 wa[kBatch], wb[kBatch];
    load_batch<T>(wa, vld, tid, last);
    load_batch<T>(wb, vld, tid + kStep, last);
    // the waves' live bounds start at -inf for everyone before anyone reads them
    if (tid < kTopkWaves) sm_live[tid] = -INFINITY;
    __syncthreads();
    const bool merger = sp == splits - 1;
    int root_tok = -1;  // the tree builder's root token, wanted only at its end
    if constexpr (FUSE) {
        if (merger && row % tp.block == tp.block - 1 && tp.root_token) root_tok = tp.root_token[row / tp.block];
    }
    const int PS = PW + 1;  // words per workgroup slot
    uint64_t *slot = W.part + (static_cast<int64_t>(row) * splits + sp) * PS;
    // the epoch is the slot word's low half (the high half stays zero); every
    // thread reads it (one request per wave), which keeps the load counts exact
    const uint32_t r_ep = fetch(reinterpret_cast<const uint32_t *>(slot));

    float tau = -INFINITY;
    // Appends the elements of x (ids base_id ..) that reach the bound, in
    // lanes where `live`: a wave-uniform call.  Each lane marks its pending
    // elements, then every trip of the loop appends each lane's lowest
    // pending one (one ballot, one LDS store per candidate); the trips are
    // as many as the most candidates a lane has in x.  vm bounds x from above.
    auto cand_vec = [&](const auto &x, float vm, int base_id, bool live) {
        constexpr int n = sizeof(x) / sizeof(float);
        if (!__ballot(live && vm >= tau)) return;
        uint32_t pend = 0;
#pragma unroll
        for (int j = 0; j < n; ++j) pend |= (live && x[j] >= tau ? 1u : 0u) << j;
        for (;;) {
            const uint64_t m = __ballot(pend != 0);
            if (!m) break;
            if (pend) {
                const int j = __builtin_ctz(pend);
                pend &= pend - 1;
                float xj = x[0];
#pragma unroll
                for (int q = 1; q < n; ++q) xj = q == j ? x[q] : xj;
                const int pos = wn + lane_rank(m);
                if (pos < kWaveCap) wcand[pos] = cand_key(xj, base_id + j);
            }
            wn += __popcll(m);
            wover = wover || wn > kWaveCap;
        }
    };
    // Keeps the K best keys of the region (ranked by counting; keys are
    // distinct) and raises the bound to the value of the K-th: every element
    // at or above the bound was appended, so that is the K-th largest the
    // wave has seen, and elements equal to it still pass the bound (a
    // smaller id beats it).  After an overflow the stored keys are a subset
    // and their K-th is still a valid bound.
    uint64_t *const wtop = &sm_wtop[wave * TD_MAX_TOPK];
    auto compact = [&]() {
        const int n = min(wn, kWaveCap);
        const int n8 = (n + 7) & ~7;
        if (lane < 8 && n + lane < n8) wcand[n + lane] = 0;
        wave_lds_sync();
        for (int e = lane; e < n; e += kWave) {
            const uint64_t mine = wcand[e];
            const int r = count_above_lds(wcand, n8, mine);
            if (r < K) wtop[r] = mine;
        }
        wave_lds_sync();
        if (lane < K && lane < n) wcand[lane] = wtop[lane];
        wave_lds_sync();
        if (n >= K) tau = fmaxf(tau, key_value(wcand[K - 1]));
        wn = min(n, K);
    };

    // ---- batch 0: exp sums, then the pre-filter bound ----
    float hx[1] = {has_head ? hraw : -INFINITY};
    float lmax = hx[0];
    if (has_head) acc.add_exp(hx, hx[0]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int i = tid + u * kTopkThreads;
        if (i < nvec) {
            float x[N];
            Vec<T>::unpack(wa[u], x);
            const float vm = LaneAcc::vmax(x);
            acc.add_exp(x, vm);
            lmax = fmaxf(lmax, vm);
        }
    }
    // Pre-filter bound: cut the wave into KM groups of 64/KM lanes; tau = the
    // smallest of the groups' maxima.  The KM group maxima are KM >= K
    // distinct elements >= tau, so the slice's K-th largest is >= tau.
    tau = group_max_min<KM>(lmax);
    cand_vec(hx, hx[0], head_id, has_head);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int i = tid + u * kTopkThreads;
        float x[N];
        Vec<T>::unpack(wa[u], x);
        cand_vec(x, LaneAcc::vmax(x), vlo + i * N, i < nvec);
    }
    // (a slice of a few batches gains nothing from a tighter bound)
    if (wn > 2 * K && nvec > 4 * kStep) compact();

    // ---- remaining batches, the next batch's loads in flight ----
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~(kWave - 1));  // wave-uniform
    // a batch that ends past the slice in some lane of the wave
    auto process = [&](const u32x4 (&w)[kBatch], int i0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * kTopkThreads;
            float x[N];
            Vec<T>::unpack(w[u], x);
            const float vm = LaneAcc::vmax(x);
            if (i < nvec) acc.add_exp(x, vm);
            cand_vec(x, vm, vlo + i * N, i < nvec);
        }
    };
    // Fast path for a batch whose vectors are all inside the slice for every
    // lane of the wave (a wave-uniform test): no per-vector range checks, the
    // batch-level sum, and candidates looked at only when some lane's batch
    // maximum reaches the bound.
    auto process_full = [&](const u32x4 (&w)[kBatch], int i0) {
        float x[kBatch][N];
        float vm[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            Vec<T>::unpack(w[u], x[u]);
            vm[u] = LaneAcc::vmax(x[u]);
        }
        static_assert(kBatch == 4, "batch maximum over four vectors");
        const float bm = fmaxf(fmaxf(vm[0], vm[1]), fmaxf(vm[2], vm[3]));
        acc.add_batch(x, bm);
        if (__ballot(bm >= tau)) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) cand_vec(x[u], vm[u], vlo + (i0 + u * kTopkThreads) * N, true);
        }
    };
    // every lane's last vector of the batch starting at k is inside the slice
    auto full_batch = [&](int k) { return wbase + (kWave - 1) + k + (kBatch - 1) * kTopkThreads < nvec; };
    // The bound is tightened by compacting the region once it holds more
    // than 2K keys.  Each wave's bound also bounds the workgroup's K-th
    // largest, so the waves share them through LDS (a stale value is still a
    // valid bound): every wave filters with the best of the four.
    auto tighten = [&]() {
        if (wn > 2 * K) compact();
        if (lane == 0) sm_live[wave] = tau;
        const u32x4 lv = *reinterpret_cast<const u32x4 *>(sm_live);
        tau = fmaxf(tau, fmaxf(fmaxf(__uint_as_float(lv.x), __uint_as_float(lv.y)),
                               fmaxf(__uint_as_float(lv.z), __uint_as_float(lv.w))));
    };
    // Batch k sits in wb for odd k / kStep, wa for even; each buffer is
    // refilled with the batch two ahead as soon as it has been processed
    // (unconditionally: past the slice the loads repeat its last vector).
    // The bound is tightened once per two batches.
    if (wbase + kStep < nvec) {
        load_batch<T>(wa, vld, tid + 2 * kStep, last);
        for (int k = kStep;;) {
            if (full_batch(k)) process_full(wb, tid + k);
            else process(wb, tid + k);
            load_batch<T>(wb, vld, tid + k + 2 * kStep, last);
            k += kStep;
            if (wbase + k >= nvec) break;
            if (full_batch(k)) process_full(wa, tid + k);
            else process(wa, tid + k);
            load_batch<T>(wa, vld, tid + k + 2 * kStep, last);
            tighten();
            k += kStep;
            if (wbase + k >= nvec) break;
        }
    }
    {  // the scalar tail: fewer than N elements, one per thread
        const int e = tail0 + tid;
        const bool in = e < hi;
        float xt[1] = {-INFINITY};
        if (in) {
            xt[0] = Vec<T>::scalar(rowp + e);
            acc.add_exp(xt, xt[0]);
        }
        cand_vec(xt, xt[0], e, in);
    }

    // ---- workgroup partial: (log2 max, sum) and the top K of the candidates ----
    const float wml = wave_max(acc.ml);
    const double contrib =
        (acc.m == -INFINITY) ? 0.0 : acc.s * static_cast<double>(__builtin_amdgcn_exp2f(acc.ml - wml));
    const double ws_sum = wave_sum(contrib);
    if (lane == 0) {
        sm_m[wave] = wml;
        sm_s[wave] = ws_sum;
        sm_tau[wave] = tau;
        sm_over[wave] = wover;
    }
    if (tid == 0) {
        sm_epoch = r_ep;
        sm_fail = 0;
    }
    if (tid < KM) sm_win[tid] = 0;
    __syncthreads();
    // Each wave's bound is at most the workgroup's K-th largest element, so
    // their maximum is one too: only candidates at or above it compete.
    float tau_wg = sm_tau[0];
    bool over = sm_over[0];
#pragma unroll
    for (int q = 1; q < kTopkWaves; ++q) {
        tau_wg = fmaxf(tau_wg, sm_tau[q]);
        over = over || sm_over[q];
    }
    int Cw = 0;
    if (!over) {
        // keep the region's keys at or above the bound, packed at its start
        // (a trip writes only slots it has read)
        for (int e0 = 0; e0 < wn; e0 += kWave) {
            const int e = e0 + lane;
            const uint64_t k = e < wn ? wcand[e] : 0;
            const bool keep = k != 0 && key_value(k) >= tau_wg;
            const uint64_t m = __ballot(keep);
            wave_lds_sync();
            if (keep) wcand[Cw + lane_rank(m)] = k;
            Cw += __popcll(m);
        }
    } else {
        // A region overflowed (rows of many equal or ascending logits): every
        // wave selects again from its share of the slice with a sorted list
        // of its best KM keys per lane, keeping only elements >= tau_wg.
        KeyList<KM> top;
        top.init();
        auto insert_vec = [&](const auto &x, int base_id, bool live) {
            constexpr int n = sizeof(x) / sizeof(float);
#pragma unroll
            for (int j = 0; j < n; ++j)
                if (live && x[j] >= tau_wg) top.insert(cand_key(x[j], base_id + j));
        };
        insert_vec(hx, head_id, has_head);
        for (int i = tid; i < nvec; i += kTopkThreads) {
            float x[N];
            Vec<T>::unpack(vp[i], x);
            insert_vec(x, vlo + i * N, true);
        }
        {
            const int e = tail0 + tid;
            float xt[1] = {-INFINITY};
            if (e < hi) xt[0] = Vec<T>::scalar(rowp + e);
            insert_vec(xt, e, e < hi);
        }
        int n_l = 0;
#pragma unroll
        for (int j = 0; j < KM; ++j) n_l += top.k[j] != 0;
        constexpr int kCountBits = KM <= 4 ? 3 : KM <= 8 ? 4 : KM <= 16 ? 5 : 6;
        const int off = wave_prefix<kCountBits>(n_l, lane, Cw);
        if (Cw <= kWaveCap) {
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (j < n_l) wcand[off + j] = top.k[j];
        } else {
            // the wave's K best by a K-round tournament
            uint64_t win[KM];
            wave_select<KM, KM>(top, K, win);
            if (lane == 0)
#pragma unroll
                for (int j = 0; j < KM; ++j) wcand[j] = win[j];
            Cw = KM;
        }
    }
    // pad the region to a multiple of 8 keys with empty (0) keys
    const int C8 = (Cw + 7) & ~7;
    if (lane < 8 && Cw + lane < C8) wcand[Cw + lane] = 0;
    if (lane == 0) sm_cnt[wave] = C8;
    __syncthreads();
    // Rank the union by counting: the thread holding a key counts the keys
    // that beat it (keys are distinct), reading every region with broadcast
    // LDS loads, and a key beaten by r < K others is the (r+1)-th best.
    {
        int nreg[kTopkWaves];
        int Ct = 0;
#pragma unroll
        for (int q = 0; q < kTopkWaves; ++q) {
            nreg[q] = sm_cnt[q];
            Ct += nreg[q];
        }
        for (int e = tid; e < Ct; e += kTopkThreads) {
            int q = 0, i = e;
#pragma unroll
            for (int r = 0; r + 1 < kTopkWaves; ++r)
                if (q == r && i >= nreg[r]) {
                    i -= nreg[r];
                    q = r + 1;
                }
            const uint64_t mine = sm_cand[q * kWaveCap + i];
            int rank = 0;
#pragma unroll
            for (int r = 0; r < kTopkWaves; ++r) rank += count_above_lds(&sm_cand[r * kWaveCap], nreg[r], mine);
            if (mine != 0 && rank < K) sm_win[rank] = mine;
        }
    }
    __syncthreads();

    // ---- this workgroup's partial: tagged words, or the merger's own LDS ----
    const uint32_t tag = sm_epoch + 1u;
    uint64_t *mypart = slot + 1;
    uint32_t *ownp = &sm_part[sp * PW];
    if (tid < 2 * K) {
        const uint64_t k = sm_win[tid >> 1];
        const uint32_t v = static_cast<uint32_t>((tid & 1) ? (k >> 32) : k);
        if (merger) ownp[tid] = v;
        else put_word(mypart + tid, v, tag);
    } else if (tid == 2 * K) {
        float M = sm_m[0];
#pragma unroll
        for (int q = 1; q < kTopkWaves; ++q) M = fmaxf(M, sm_m[q]);
        double S = 0.0;
#pragma unroll
        for (int q = 0; q < kTopkWaves; ++q)
            if (sm_m[q] != -INFINITY)
                S += sm_s[q] * static_cast<double>(__builtin_amdgcn_exp2f(sm_m[q] - M));
        const uint64_t sb = static_cast<uint64_t>(__double_as_longlong(S));
        if (merger) {
            ownp[2 * K] = __float_as_uint(M);
            ownp[2 * K + 1] = static_cast<uint32_t>(sb);
            ownp[2 * K + 2] = static_cast<uint32_t>(sb >> 32);
        } else {
            put_word(mypart + 2 * K, __float_as_uint(M), tag);
            put_word(mypart + 2 * K + 1, static_cast<uint32_t>(sb), tag);
            put_word(mypart + 2 * K + 2, static_cast<uint32_t>(sb >> 32), tag);
        }
    }
    if (tid == 0) publish(slot, static_cast<uint64_t>(tag));  // the next call's epoch
    if (!merger) return;

    // ---- the row merger: gather every partial of the row ----
    // (the merger's own words, split splits - 1, are the last PW and in LDS)
    const uint64_t *rp = W.part + static_cast<int64_t>(row) * splits * PS;
    const int nw = (splits - 1) * PW;
    for (int w0 = 0; w0 < nw; w0 += 4 * kTopkThreads) {
        int idx[4];
        uint32_t val[4];
        int n = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int w = w0 + tid + u * kTopkThreads;
            idx[u] = (w / PW) * PS + 1 + w % PW;  // data word w % PW of slot w / PW
            if (w < nw) n = u + 1;
        }
        if (n > 0 && !get_words(rp, idx, n, tag, val)) sm_fail = 1;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (u < n) sm_part[w0 + tid + u * kTopkThreads] = val[u];
    }
    __syncthreads();

    // ---- wave 1: the row's normaliser, while wave 0 selects the row's top K ----
    double &sm_lse = L.lse;
    if (wave == 1) {
        float ml = -INFINITY;
        double ssum = 0.0;
        if (lane < splits) {
            const uint32_t *w = &sm_part[lane * PW + 2 * K];
            ml = __uint_as_float(w[0]);
            ssum = __longlong_as_double(static_cast<long long>(
                static_cast<uint64_t>(w[1]) | (static_cast<uint64_t>(w[2]) << 32)));
        }
        const float M = wave_max(ml);
        const double c = (ml == -INFINITY) ? 0.0
                                           : ssum * static_cast<double>(__builtin_amdgcn_exp2f(ml - M));
        const double S = wave_sum(c);
        constexpr double kLn2 = 0.6931471805599453;
        const double lse = sm_fail ? NAN : static_cast<double>(M) * kLn2 + log(S);
        if (lane == 0) {
            sm_lse = lse;
            lse_out[row] = lse;
            if (sm_fail) raise_status(W.status, kStatusMerge);
        }
    }

    // ---- the row's top K from the partials (wave 0, broadcast LDS counts) ----
    if (wave == 0) {
        auto part_key = [&](int s, int j) -> uint64_t {
            const uint32_t *w = &sm_part[s * PW + 2 * j];
            return static_cast<uint64_t>(w[0]) | (static_cast<uint64_t>(w[1]) << 32);
        };
        // tau_key = K-th best of the partials' heads bounds the row's K-th
        // best from below; only keys >= tau_key can be in the row's top K.
        const uint64_t hd = lane < splits ? part_key(lane, 0) : 0;
        sm_heads[lane] = hd;  // splits <= 64; zeros pad to a multiple of 8
        wave_lds_sync();
        uint64_t tau_key = 0;
        if (splits >= K) {
            const int rank = count_above_lds(sm_heads, (splits + 7) & ~7, hd);
            const uint64_t at = __ballot(lane < splits && rank == K - 1);
            if (at) tau_key = readlane64(hd, __ffsll(static_cast<long long>(at)) - 1);
        }
        const uint64_t below = (1ull << lane) - 1;
        // lane e of a trip reads key e % KM of partial e / KM (KM >= K)
        const int PK = splits * KM;
        int C2 = 0;
        for (int e0 = 0; e0 < PK; e0 += kWave) {
            const int e = e0 + lane;
            const uint64_t k = (e < PK && e % KM < K) ? part_key(e / KM, e % KM) : 0;
            const bool take = k != 0 && k >= tau_key;
            const uint64_t m = __ballot(take);
            const int o = C2 + __popcll(m & below);
            if (take && o < kCandCap) sm_cand[o] = k;
            C2 += __popcll(m);
        }
        if (lane < KM) sm_win[lane] = 0;
        if (C2 <= kCandCap) {
            const int C8 = (C2 + 7) & ~7;
            for (int p = C2 + lane; p < C8; p += kWave) sm_cand[p] = 0;
            wave_lds_sync();
            for (int e = lane; e < C2; e += kWave) {
                const uint64_t mine = sm_cand[e];
                const int rank = count_above_lds(sm_cand, C8, mine);
                if (rank < K) sm_win[rank] = mine;
            }
        } else {
            // many equal logits: tournament over the partial lists
            KeyList<KM> t;
            t.init();
            if (lane < splits)
#pragma unroll
                for (int j = 0; j < KM; ++j)
                    if (j < K) t.k[j] = part_key(lane, j);
            uint64_t win[KM];
            wave_select<KM, KM>(t, K, win);
            if (lane == 0)
#pragma unroll
                for (int j = 0; j < KM; ++j) sm_win[j] = win[j];
        }
    }  // wave 0
    __syncthreads();  // every wave is still resident here
    if (wave != 0) {
        if constexpr (FUSE) {
            if (row % tp.block == tp.block - 1) {
                // the sequence's tree builder: while wave 0 builds, the other
                // waves write the entries past the root as beyond the tree
                prefill_tree_outputs(tp, to, row / tp.block, tid - kWave, kTopkThreads - kWave);
                __builtin_amdgcn_s_waitcnt(0);  // acknowledged before wave 0 writes the tree
                __syncthreads();
            }
        }
        return;
    }

    // ---- the row's outputs (wave 0) ----
    const double lse = sm_lse;
    int32_t id = -1;
    double lq = 0.0;
    if (lane < K) {
        const uint64_t k = sm_win[lane];
        id = key_id(k);
        lq = static_cast<double>(key_value(k)) - lse;
        topk_id[static_cast<int64_t>(row) * K + lane] = id;
        topk_logq[static_cast<int64_t>(row) * K + lane] = lq;
    }
    if constexpr (FUSE) {
        // leave the row's results for the sequence's tree builder (the merger
        // of the sequence's last row, which keeps its own row in LDS)
        TreeLds &tl = L.tl;
        const uint32_t stag = tag;  // every slot of a workspace holds the same epoch
        const int b = row / tp.block;
        const int rl = row - b * tp.block;
        if (rl != tp.block - 1) {
            uint64_t *rr = W.rowrec + static_cast<int64_t>(row) * 3 * K;
            if (lane < K) {
                const uint64_t qb = static_cast<uint64_t>(__double_as_longlong(lq));
                put_word(rr + lane, static_cast<uint32_t>(id), stag);
                put_word(rr + K + 2 * lane, static_cast<uint32_t>(qb), stag);
                put_word(rr + K + 2 * lane + 1, static_cast<uint32_t>(qb >> 32), stag);
            }
            return;
        }
        if (lane < K) {
            tl.ids[rl * K + lane] = id;
            tl.lq[rl * K + lane] = lq;
        }

        // the sequence's tree builder: gather the other rows, build the tree
        const int BK = (tp.block - 1) * K;
        const uint64_t *sr = W.rowrec + static_cast<int64_t>(b) * tp.block * 3 * K;
        bool ok = true;
        // two entries per lane and trip: id, log q low and high words each
        for (int e0 = lane; e0 < BK; e0 += 2 * kWave) {
            int idx[6];
            uint32_t v[6];
            int n = 0;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = e0 + u * kWave;
                const int r = e / K, j = e % K;
                idx[3 * u] = r * 3 * K + j;
                idx[3 * u + 1] = r * 3 * K + K + 2 * j;
                idx[3 * u + 2] = r * 3 * K + K + 2 * j + 1;
                if (e < BK) n = 3 * (u + 1);
            }
            ok = get_words(sr, idx, n, stag, v) && ok;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = e0 + u * kWave;
                if (e < BK) {
                    // ids are < 2^18 (TD_MAX_VOCAB); the mask keeps a word that
                    // never arrived from steering the builder's table indexing
                    tl.ids[e] = static_cast<int>(v[3 * u] & kTokenMask);
                    tl.lq[e] = __longlong_as_double(static_cast<long long>(
                        static_cast<uint64_t>(v[3 * u + 1]) | (static_cast<uint64_t>(v[3 * u + 2]) << 32)));
                }
            }
        }
        wave_lds_sync();
        build_tree_wave<SLOTS, true>(tl, tp, to, b, lane, root_tok);
        if (lane == 0 && !ok) {
            to.n_nodes[b] = -1;
            raise_status(W.status, kStatusTree);
        }
    }
}

template <typename T, int KM, bool FUSE, int SLOTS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const T *__restrict__ logits,
                                                            int vocab, int64_t pos_stride,
                                                            int slice, int splits, int K, void *ws,
                                                            int32_t *__restrict__ topk_id,
                                                            double *__restrict__ topk_logq,
                                                            double *__restrict__ lse_out,
                                                            TreeParams tp, TreeOut to) {
    __shared__ TopkLds<KM, FUSE> lds;
    topk_body<T, KM, FUSE, SLOTS>(logits, vocab, pos_stride, slice, splits, K, ws, topk_id, topk_logq,
                                  lse_out, tp, to, blockIdx.x, blockIdx.y, gridDim.y, lds);
}

// ---------------------------------------------------------------------------
// The verify step's first kernel with the context split folded in: one
// launch fewer, and the split's loads and first row groups run while the
// draft is still being selected.  Workgroups 0 .. topk_wgs - 1 are the top-K
// and tree workgroups (slice sp of row r at index r * splits + sp, the order
// of the two-dimensional launch, so every hand-off still waits only on
// lower indices); the others are split work items, which wait only for the
// tree builders' size words.  The two roles share the LDS, so two
// workgroups fit a compute unit.
// ---------------------------------------------------------------------------
template <int KM, int D>
union DraftSplitLds {
    TopkLds<KM, true> t;
    FusedSplitLds<D> s;
};

template <typename T, int KM, int SLOTS, int D>
__global__ __launch_bounds__(kTopkThreads) void topk_split_kernel(
    const T *__restrict__ logits, int vocab, int64_t pos_stride, int slice, int splits, int rows, int K,
    void *ws, int32_t *__restrict__ topk_id, double *__restrict__ topk_logq, double *__restrict__ lse_out,
    TreeParams tp, TreeOut to, int topk_wgs, SplitArgs sa) {
    static_assert(kTopkThreads == kAttnThreads, "one workgroup size for both roles");
    __shared__ DraftSplitLds<KM, D> lds;
    const int wg = blockIdx.x;
    if (wg < topk_wgs) {
        topk_body<T, KM, true, SLOTS>(logits, vocab, pos_stride, slice, splits, K, ws, topk_id, topk_logq,
                                      lse_out, tp, to, wg % splits, wg / splits, rows, lds.t);
        return;
    }
    fused_split<D>(sa, wg - topk_wgs, lds.s);
}

// Split plan.  When every row can be cut into slices of at most kOneRound
// elements with one workgroup per compute unit, do that: the loads of a
// slice then all go out at once and no compute unit serves two slices (the
// latency-bound case of a few rows).  Otherwise enough workgroups to cover
// the chip a few times over, at least kMinSlice elements per workgroup, and
// at most one partial per lane of the merge wave.
constexpr int kCUs = 256;  // compute units of the gfx950 parts
constexpr int kOneRound = 2 * kBatch * kTopkThreads * 8;  // two batches of bf16 vectors
constexpr int kTargetWgs = 1024;
constexpr int kMinSlice = 8192;

struct TopkPlan {
    int splits;
    int slice;
};

inline TopkPlan topk_plan(int64_t rows, int vocab, int K) {
    const int64_t most = std::min<int64_t>(64, 1024 / K);
    const int64_t per_cu = kCUs / std::max<int64_t>(1, rows);
    int64_t want;
    if (per_cu >= 1 && (vocab + per_cu - 1) / per_cu <= kOneRound) {
        want = per_cu;
    } else {
        const int64_t cover = (kTargetWgs + rows - 1) / rows;
        const int64_t cap = (vocab + kMinSlice - 1) / kMinSlice;
        want = std::min(cover, cap);
    }
    int splits = static_cast<int>(std::max<int64_t>(1, std::min(want, most)));
    int slice = (vocab + splits - 1) / splits;
    slice = (slice + 7) & ~7;  // 16-byte aligned slices for both element types
    splits = (vocab + slice - 1) / slice;
    return {splits, slice};
}

template <typename T, int KM, bool FUSE, int SLOTS>
void launch_topk(const void *logits, int rows, int vocab, int64_t pos_stride, int K,
                 const TopkPlan &pl, void *ws, int32_t *topk_id, double *topk_logq, double *lse,
                 const TreeParams &tp, const TreeOut &to, hipStream_t st) {
    TD_LAUNCH((topk_kernel<T, KM, FUSE, SLOTS>), dim3(pl.splits, rows), dim3(kTopkThreads),
                       0, st, static_cast<const T *>(logits), vocab, pos_stride, pl.slice, pl.splits,
                       K, ws, topk_id, topk_logq, lse, tp, to);
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
    const TopkPlan pl = topk_plan(rows, vocab, K);
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
    const TopkPlan pl = topk_plan(rows, vocab, K);
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

// The fused first kernel serves steps whose split chunks fit its one buffer
// (short contexts: one chunk of at most kFusedKeys keys per work item) and
// whose top-K takes at most one workgroup per compute unit, with bf16
// attention at head dim 128 and K <= 8; the others keep the split kernel.
bool step_fuses_split(int batch, int block, int vocab, int K, int nq_max, int hq, int hkv, int head_dim,
                      int64_t total_ctx, td_dtype attn_dtype) {
    if (attn_dtype != TD_BF16 || head_dim != 128 || K > 8) return false;
    const int64_t rows = static_cast<int64_t>(batch) * block;
    const TopkPlan tk = topk_plan(rows, vocab, K);
    if (rows * tk.splits > kCUs) return false;
    const AttnPlan pl = attn_plan(batch, nq_max, hq, hkv, total_ctx, Sub<uint16_t>::CH, kFusedItems);
    return pl.chunk == kFusedKeys && pl.items <= kFusedItems + static_cast<int64_t>(batch) * hkv;
}

void launch_topk_tree_split(const void *logits, td_dtype dtype, int batch, int block, int vocab,
                            int64_t pos_stride, int K, void *ws, int32_t *topk_id, double *topk_logq,
                            double *lse, const TreeParams &tp, const TreeOut &to, const SplitInputs &si,
                            hipStream_t st) {
    const int rows = batch * block;
    const TopkPlan tk = topk_plan(rows, vocab, K);
    const AttnPlan pl = attn_plan(batch, si.nq_max, si.hq, si.hkv, si.total_ctx, Sub<uint16_t>::CH, kFusedItems);
    SplitArgs sa;
    sa.q = static_cast<const uint16_t *>(si.q);
    sa.k_ctx = static_cast<const uint16_t *>(si.k_ctx);
    sa.v_ctx = static_cast<const uint16_t *>(si.v_ctx);
    sa.ctx_offsets = si.off;
    sa.ctx_lengths = si.lens;
    sa.ready = to.ready;
    sa.status = static_cast<uint32_t *>(ws);
    sa.all_rows = tp.use_stop == 0;
    sa.batch = batch;
    sa.nq_max = si.nq_max;
    sa.hq = si.hq;
    sa.hkv = si.hkv;
    sa.group = pl.group;
    sa.n_rg = pl.n_rg;
    sa.chunk = pl.chunk;
    sa.scale2 = si.scale * kLog2e;
    sa.ws = static_cast<float *>(si.ws);
    sa.prow_total = split_prow_total(pl, si.hkv);
    sa.seqinfo = split_seqinfo(si.ws, pl, si.hkv, 128, partial_o_bytes(true));
    const int topk_wgs = rows * tk.splits;
    const dim3 grid(static_cast<unsigned>(topk_wgs + pl.items));
#define TD_FUSED(TT, KMM, SL)                                                                      \
    TD_LAUNCH((topk_split_kernel<TT, KMM, SL, 128>), grid, dim3(kTopkThreads), 0, st,             \
              static_cast<const TT *>(logits), vocab, pos_stride, tk.slice, tk.splits, rows, K, ws, \
              topk_id, topk_logq, lse, tp, to, topk_wgs, sa)
#define TD_FUSED_SL(TT, KMM)                                                                       \
    switch (tree_slots(tp.n_max)) {                                                                \
    case 1: TD_FUSED(TT, KMM, 1); break;                                                           \
    case 2: TD_FUSED(TT, KMM, 2); break;                                                           \
    case 4: TD_FUSED(TT, KMM, 4); break;                                                           \
    default: TD_FUSED(TT, KMM, 8); break;                                                          \
    }
    if (dtype == TD_BF16) {
        if (K <= 4) { TD_FUSED_SL(uint16_t, 4) } else { TD_FUSED_SL(uint16_t, 8) }
    } else {
        if (K <= 4) { TD_FUSED_SL(float, 4) } else { TD_FUSED_SL(float, 8) }
    }
#undef TD_FUSED_SL
#undef TD_FUSED
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
