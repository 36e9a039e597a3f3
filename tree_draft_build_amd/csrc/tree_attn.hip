// Stage (c): tree verification attention (BASTION: the target scores every
// node of the draft tree in one parallel pass; a node may only see the
// context and its own root path).
//
// For sequence b, query head h (KV head g = h / G, G = hq / hkv) and tree row
// i <= n_nodes[b], the admitted keys are the whole context of b plus the
// tree nodes on the root path of i.  The context part is dense and carries
// almost all bytes and flops; the tree part is sparse (at most depth+1 keys
// per row).  The G heads of a KV group times the tree rows form the M
// dimension (row r = i * G + hh), cut into row groups of 16.  Two kernels:
//
//  split            split-KV over the context (attn_split_bf16 streams keys
//                   straight into LDS and reads V transposed from there;
//                   attn_split_f32 stages through registers).  Work item =
//                   (key chunk of one sequence, KV head); a sequence with an
//                   empty context still gets one chunk with no keys.  The
//                   chunk's first loads are issued before the tree size and
//                   the queries arrive, and each next sub-chunk's loads fly
//                   during the compute.  A wave owns up to OWN row groups
//                   (queries and O^T accumulators in registers; bf16 at
//                   D = 128 runs one-group code for trees of up to 4 row
//                   groups, and 3 or, when the grid is throughput-bound, 5
//                   for larger ones) and shares each K and V
//                   fragment it reads from LDS among them; row
//                   blocks of 4 OWN row groups are processed in turn; a block
//                   of fewer than 4 row groups splits the keys of each
//                   sub-chunk over the waves, which merge through LDS.
//                   Softmax is online in base 2.  One (m, l, O) partial per
//                   tree row and chunk is stored.
//  attn_tree_combine one wave per output row of the trees (the rows of all
//                   trees are numbered through a prefix sum of the tree
//                   sizes, and the waves take them in turn):
//                   merges the chunk partials (every load in flight at
//                   once), adds the ancestor-masked tree keys (sparse: one
//                   dot product per set mask bit) and writes the normalised
//                   row; rows past a tree are not written.
//
// MFMA 16x16x32 bf16 operand layout (wave64): A (16 x 32): lane l holds row
// l % 16, k = 8 (l / 16) .. +7; B (32 x 16): lane l holds column l % 16, the
// same k; C (16 x 16): lane l holds column l % 16, rows 4 (l / 16) .. +3.
// The f32 variant uses MFMA 16x16x4 (A/B: lane l holds k = l / 16).
// Keys inside a 32-key tile are taken by the PV product in the order the S^T
// product leaves them in registers: lane slot t of lane group h is key
// 4h + t (t < 4) or 16 + 4h + t - 4 (t >= 4); the contraction is invariant
// under that permutation.

#include <algorithm>
#include <type_traits>

#include "step_launch.h"
#include "td_internal.h"
#include "tree_core.h"

#include "attn_split.h"

namespace td {
namespace {

// ---------------------------------------------------------------------------
// attn_tree_combine: lane j owns dims D/8 (j / 8) .. +D/8-1 of a row.  R = 1
// (rows with many chunk partials): one row per wave, lane j takes chunks
// c = j % 8 (mod 8), all partial loads of the row in flight at once, and the
// chunk groups are summed by the register butterfly levels 0..2 (within 8
// lanes).  R = 8 (rows with few partials): eight rows per wave, lane group
// j % 8 takes row j % 8 and all its chunks.  Tree keys: each lane dots its
// dims, and lane ^ 8, ^ 16, ^ 32 exchanges sum the 8 dim slices of the row.
// ---------------------------------------------------------------------------
constexpr int kCombineRows = kAttnThreads / kWave;  // waves per workgroup
// The rows of the trees, (sequence b, KV head g, row r = tree row i * G +
// head) with r < G (n_b + 1), are numbered b-major through the prefix sums
// of hq (n_b + 1) (each workgroup computes them in LDS from the tree sizes),
// and wave w takes the R rows R w .., then R (w + W) .., ... of the W waves
// in the grid.  The grid has one wave per R row slots of the capacity, at
// most about twice the waves the chip holds at the combine's register use
// (3 per SIMD).
constexpr int64_t kCombineWaves = 256 * 4 * 3 * 2;
inline int combine_blocks(int64_t slots, int R) {
    const int64_t waves = (slots + R - 1) / R;
    return static_cast<int>(std::max<int64_t>(
        1, std::min<int64_t>((waves + kCombineRows - 1) / kCombineRows, kCombineWaves / kCombineRows)));
}
// Rows per combine wave: eight when the sequences average few chunks.
inline int combine_rows_per_wave(int64_t n_chunks, int batch) { return n_chunks <= 12LL * batch ? 8 : 1; }

// N consecutive elements (16-byte aligned) widened to float.
template <typename T, int N>
__device__ __forceinline__ void load_slice(const T *p, float (&x)[N]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k8 = 0; k8 < N / 8; ++k8) {
            const u32x4 w = reinterpret_cast<const u32x4 *>(p)[k8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * k8 + 2 * e] = bf16_lo(w[e]);
                x[8 * k8 + 2 * e + 1] = bf16_hi(w[e]);
            }
        }
    } else {
#pragma unroll
        for (int k4 = 0; k4 < N / 4; ++k4) {
            const f32x4 w = reinterpret_cast<const f32x4 *>(p)[k4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * k4 + e] = w[e];
        }
    }
}

// The same slice as raw 16-byte words (loads in flight, no use yet), and
// their widening to float.
template <typename T, int N> constexpr int raw_words() { return N * static_cast<int>(sizeof(T)) / 16; }
template <typename T, int N>
__device__ __forceinline__ void load_raw(const T *p, u32x4 (&w)[raw_words<T, N>()]) {
#pragma unroll
    for (int k = 0; k < raw_words<T, N>(); ++k) w[k] = reinterpret_cast<const u32x4 *>(p)[k];
}
template <typename T, int N>
__device__ __forceinline__ void widen(const u32x4 (&w)[raw_words<T, N>()], float (&x)[N]) {
#pragma unroll
    for (int k = 0; k < raw_words<T, N>(); ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (sizeof(T) == 2) {
                x[8 * k + 2 * e] = bf16_lo(w[k][e]);
                x[8 * k + 2 * e + 1] = bf16_hi(w[k][e]);
            } else {
                x[4 * k + e] = __uint_as_float(w[k][e]);
            }
        }
    }
}

// ACC: the grid carries one more workgroup per sequence, whose wave 0 runs
// the acceptance walk (the verify step's last kernel).
template <typename T, int D, bool ACC, int R>
__global__ __launch_bounds__(kAttnThreads) void attn_tree_combine(
    const T *__restrict__ q, const int2 *__restrict__ seqinfo, const T *__restrict__ k_tree,
    const T *__restrict__ v_tree, const uint64_t *__restrict__ mask,
    const int32_t *__restrict__ n_nodes, int batch, int nq_max, int hq, int hkv, int group, int n_rg,
    int chunk, float scale2, const float *__restrict__ ws, int64_t prow_total, T *__restrict__ out,
    int n_blocks, int nch_max, AcceptArgs accept) {
    constexpr int kSlice = D / 8;  // dims per lane group
    const int rows_per_bg = group * nq_max;
    if constexpr (ACC) {
        if (static_cast<int>(blockIdx.x) >= n_blocks) {
            const int bs = static_cast<int>(blockIdx.x) - n_blocks;
            if (accept.ready && threadIdx.x == 0)  // the next fused first kernel waits for a new size
                __hip_atomic_store(accept.ready + bs, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __shared__ int s_path[TD_MAX_BLOCK + 1];
            __shared__ int s_acc[2];  // accepted length, bonus token
            if (threadIdx.x < kWave)
                accept_wave(accept.node_token, accept.node_parent, n_nodes, accept.target_token,
                            accept.n_max, accept.block, accept.accept_len, accept.accept_path,
                            accept.bonus_token, bs, threadIdx.x, s_path, s_acc);
            if (accept.commit) {  // the accepted path becomes context (uniform branch)
                __shared__ int64_t s_len;
                if (threadIdx.x == 0) s_len = commit_length(accept.cm, bs);
                __syncthreads();
                commit_seq(accept.cm, bs, s_path, s_acc[0], s_acc[1], s_len, threadIdx.x,
                           kAttnThreads);
            }
            return;
        }
    }
    static_assert(R == 1 || R == 8, "one or eight rows per wave");
    constexpr int kCG = 8 / R;  // chunk groups per row
    const int lane = threadIdx.x & 63;
    const int slice = lane >> 3;
    const int cg = R == 1 ? (lane & 7) : 0;
    // one sequence: its record is loaded with the tree size, one round trip
    // before the partials rather than two
    int2 si0 = int2{0, 0};
    int nn0 = 0;
    if (batch == 1) {
        nn0 = n_nodes[0];
        si0 = seqinfo[0];
    }
    // row (b, g, r) of this lane (of its lane group when R = 8); `store`:
    // a real row (a lane group past the last row repeats one, unstored)
    auto combine_row = [&](int b, int g, int r, bool store, auto one_seq) __attribute__((always_inline)) {
        constexpr bool kOne = decltype(one_seq)::value;
        const int i = r / group;
        const int h = g * group + r % group;
        T *orow = out + ((static_cast<int64_t>(b) * nq_max + i) * hq + h) * D + slice * kSlice;
        // Everything this row needs that does not depend on other loads goes out
        // first: the query slice, the mask row and the root's key and value
        // (the root is on every row's path).
        const T *qrow = q + ((static_cast<int64_t>(b) * nq_max + i) * hq + h) * D + slice * kSlice;
        const int64_t kv0 = (static_cast<int64_t>(b) * nq_max * hkv + g) * D + slice * kSlice;
        float qv[kSlice], k0v[kSlice], v0v[kSlice];
        load_slice<T, kSlice>(qrow, qv);
        load_slice<T, kSlice>(k_tree + kv0, k0v);
        load_slice<T, kSlice>(v_tree + kv0, v0v);
        const int words = (nq_max + 63) / 64;
        const uint64_t *mrow = mask + (static_cast<int64_t>(b) * nq_max + i) * words;
        uint64_t mw[4];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) mw[wd] = wd < words ? mrow[wd] : 0;

        // first chunk and chunk count of sequence b (left by the split kernel).
        // One sequence: its chunks start at 0 and number at most nch_max
        // (known on the host), so the partials' loads go out with the record
        // and the chunks past its count are dropped below.
        const int2 si = kOne ? si0 : seqinfo[b];
        const int nch = si.y;
        const int64_t cb = kOne ? 0 : si.x;
        const int nch_l = kOne ? nch_max : nch;
        const int rg = r / kRowsPerGroup;
        const int rr = r % kRowsPerGroup;
        const float *wm = ws;
        const float *wl = ws + prow_total;
        using PO = typename PartialO<T>::type;
        const PO *wo = reinterpret_cast<const PO *>(ws + 2 * prow_total);

        // context partials: lane group cg takes chunks cg, cg + 8, ...; up to
        // kCB of them per trip with all their loads in flight, merged online
        constexpr int kCB = 4;
        float M = -INFINITY;
        float Lsum = 0.f;
        float acc[kSlice];
#pragma unroll
        for (int k = 0; k < kSlice; ++k) acc[k] = 0.f;
        for (int c0 = 0; c0 < nch_l; c0 += kCG * kCB) {
            float mv[kCB], lv[kCB];
            float ov[kCB][kSlice];
#pragma unroll
            for (int u = 0; u < kCB; ++u) {
                const int cc = min(c0 + cg + kCG * u, nch_l - 1);  // in range; repeats are dropped below
                const int64_t pr = prow_index(cb + cc, g, rg, rr, hkv, n_rg);
                mv[u] = wm[pr];
                lv[u] = wl[pr];
                load_slice<PO, kSlice>(&wo[pr * D + slice * kSlice], ov[u]);
            }
            // Branch-free on purpose: every loaded value is used, so the
            // compiler keeps all of a trip's loads in flight together instead of
            // sinking the O loads behind the m loads.  Repeated, empty and (one
            // sequence) never-written chunks are selected away, not weighted by
            // 0: a slot past the sequence's chunks may hold anything.
            float mb = M;
#pragma unroll
            for (int u = 0; u < kCB; ++u) mb = fmaxf(mb, c0 + cg + kCG * u < nch ? mv[u] : -INFINITY);
            const float base = mb == -INFINITY ? 0.f : mb;
            const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - base);
            Lsum *= fo;
#pragma unroll
            for (int k = 0; k < kSlice; ++k) acc[k] *= fo;
#pragma unroll
            for (int u = 0; u < kCB; ++u) {
                const bool use = c0 + cg + kCG * u < nch && mv[u] != -INFINITY;
                const float f = use ? __builtin_amdgcn_exp2f(mv[u] - base) : 0.f;
                Lsum += use ? f * lv[u] : 0.f;
#pragma unroll
                for (int k = 0; k < kSlice; ++k) acc[k] += use ? f * ov[u][k] : 0.f;
            }
            M = mb;
        }
        // merge the 8 chunk groups (levels 0..2 of the lane exchanges)
        if constexpr (R == 1) {
            float Mg = M;
            Mg = fmaxf(Mg, xchg_f<0>(Mg));
            Mg = fmaxf(Mg, xchg_f<1>(Mg));
            Mg = fmaxf(Mg, xchg_f<2>(Mg));
            const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mg);
            Lsum *= f;
            Lsum += xchg_f<0>(Lsum);
            Lsum += xchg_f<1>(Lsum);
            Lsum += xchg_f<2>(Lsum);
#pragma unroll
            for (int k = 0; k < kSlice; ++k) {
                acc[k] *= f;
                acc[k] += xchg_f<0>(acc[k]);
                acc[k] += xchg_f<1>(acc[k]);
                acc[k] += xchg_f<2>(acc[k]);
            }
            M = Mg;
        }

        // tree keys on the root path of i (mask row), one dot product per bit;
        // the root's key and value are already in registers
        auto add_key = [&](const float (&kk)[kSlice], const float (&vv)[kSlice]) {
            float dot = 0.f;
#pragma unroll
            for (int k = 0; k < kSlice; ++k) dot += qv[k] * kk[k];
            dot += xor8_f(dot);
            dot += xchg_f<4>(dot);
            dot += xchg_f<5>(dot);
            const float sc = dot * scale2;
            const float Mn = fmaxf(M, sc);
            const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
            const float fn = __builtin_amdgcn_exp2f(sc - Mn);
            Lsum = Lsum * fo + fn;
#pragma unroll
            for (int k = 0; k < kSlice; ++k) acc[k] = acc[k] * fo + vv[k] * fn;
            M = Mn;
        };
        if (mw[0] & 1ull) add_key(k0v, v0v);
        mw[0] &= ~1ull;
        // the other keys kTB at a time, all their loads in flight before the
        // first is used (bits in increasing order, as a one-by-one walk)
        constexpr int kTB = sizeof(T) == 2 ? 4 : 2;
        constexpr int kRW = raw_words<T, kSlice>();
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            uint64_t bits = mw[wd];
            while (bits) {
                bool have[kTB];
                u32x4 kr[kTB][kRW], vr[kTB][kRW];
#pragma unroll
                for (int u = 0; u < kTB; ++u) {
                    const int j = wd * 64 + __ffsll(static_cast<long long>(bits)) - 1;
                    have[u] = bits != 0 && j < nq_max;  // bits beyond the tree rows are ignored
                    bits &= bits - 1;
                    if (have[u]) {
                        const int64_t kv =
                            ((static_cast<int64_t>(b) * nq_max + j) * hkv + g) * D + slice * kSlice;
                        load_raw<T, kSlice>(k_tree + kv, kr[u]);
                        load_raw<T, kSlice>(v_tree + kv, vr[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < kTB; ++u) {
                    if (have[u]) {
                        float kk[kSlice], vv[kSlice];
                        widen<T, kSlice>(kr[u], kk);
                        widen<T, kSlice>(vr[u], vv);
                        add_key(kk, vv);
                    }
                }
            }
        }
        if (cg == 0 && store) {
            const float inv = 1.f / Lsum;
#pragma unroll
            for (int k = 0; k < kSlice; ++k) orow[k] = from_f32<T>(acc[k] * inv);
        }
    };
    // prefix sums of the rows of the trees, per sequence: pre[b] = rows of
    // sequences < b (each thread sums a run of sequences, then the runs are
    // scanned in LDS)
    __shared__ uint32_t pre[TD_MAX_BATCH + 1];
    __shared__ uint32_t runs[kAttnThreads];
    const uint32_t sub = R == 1 ? 0u : static_cast<uint32_t>(lane & 7);
    const uint32_t step = static_cast<uint32_t>(n_blocks) * kCombineRows * R;
    const uint32_t first = (blockIdx.x * kCombineRows + (threadIdx.x >> 6)) * R;
    if (batch == 1) {  // one sequence: no sums to share
        // the root's rows (node 0 of every head) need no tree size: their
        // loads go out before it arrives; a tree build that gave up
        // (n_nodes < 0) has no rows, so nothing is stored then
        const uint32_t roots = static_cast<uint32_t>(hq);
        for (uint32_t t0 = first; t0 < roots; t0 += step) {
            const uint32_t t = min(t0 + sub, roots - 1);
            combine_row(0, static_cast<int>(t / group), static_cast<int>(t % group),
                        t0 + sub < roots && nn0 >= 0, std::true_type{});
        }
        if (nn0 <= 0) return;
        // then nodes 1 .. n: row r = group i + head offset of KV head g
        const uint32_t n1 = static_cast<uint32_t>(min(nn0, nq_max - 1));
        const uint32_t rows_g = static_cast<uint32_t>(group) * n1;
        const uint32_t total = static_cast<uint32_t>(hkv) * rows_g;
        for (uint32_t t0 = first; t0 < total; t0 += step) {
            const uint32_t t = min(t0 + sub, total - 1);
            const uint32_t g = t / rows_g;
            combine_row(0, static_cast<int>(g), group + static_cast<int>(t - g * rows_g), t0 + sub < total,
                        std::true_type{});
        }
        return;
    }
    {
        const int per = (batch + kAttnThreads - 1) / kAttnThreads;
        const int b0 = threadIdx.x * per;
        const int b1 = min(batch, b0 + per);
        uint32_t sum = 0;
        for (int b = b0; b < b1; ++b) {
            const int n = min(n_nodes[b], nq_max - 1);
            pre[b] = sum;
            sum += n >= 0 ? static_cast<uint32_t>(hq) * (n + 1) : 0u;
        }
        runs[threadIdx.x] = sum;
        __syncthreads();
        if (threadIdx.x < kWave) {  // exclusive scan of the 256 runs: 4 per lane, then the lanes
            static_assert(kAttnThreads == 4 * kWave, "four runs per lane");
            const int l = threadIdx.x;
            const uint32_t r0 = runs[4 * l], r1 = runs[4 * l + 1], r2 = runs[4 * l + 2],
                           r3 = runs[4 * l + 3];
            const uint32_t own = r0 + r1 + r2 + r3;
            uint32_t inc = own;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const uint32_t o = __shfl_up(inc, d, kWave);
                inc += l >= d ? o : 0u;
            }
            const uint32_t ex = inc - own;
            runs[4 * l] = ex;
            runs[4 * l + 1] = ex + r0;
            runs[4 * l + 2] = ex + r0 + r1;
            runs[4 * l + 3] = ex + r0 + r1 + r2;
            if (l == kWave - 1) pre[batch] = inc;
        }
        __syncthreads();
        const uint32_t add = runs[threadIdx.x];
        for (int b = b0; b < b1; ++b) pre[b] += add;
        __syncthreads();
    }
    const uint32_t total = pre[batch];
    for (uint32_t t0 = first; t0 < total; t0 += step) {
        const uint32_t t = min(t0 + sub, total - 1);
        // the sequence of row t: the last b with pre[b] <= t (binary search)
        int lo = 0, hi = batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo;
        const uint32_t rest = t - pre[b];
        const uint32_t rows_g = static_cast<uint32_t>(group) * (min(n_nodes[b], nq_max - 1) + 1);
        const uint32_t g = rest / rows_g;
        combine_row(b, static_cast<int>(g), static_cast<int>(rest - g * rows_g), t0 + sub < total,
                    std::false_type{});
    }
}

template <typename T, int D>
void launch_attn(const void *q, const void *k_ctx, const void *v_ctx, const int64_t *off,
                 const int64_t *lens, const void *k_tree, const void *v_tree, const uint64_t *mask,
                 const int32_t *n_nodes, int batch, int nq_max, int hq, int hkv, float scale,
                 const AttnPlan &pl, void *ws, void *out, const AcceptArgs *acc, hipStream_t st,
                 bool split) {
    const float scale2 = scale * kLog2e;
    const int64_t prow_total = split_prow_total(pl, hkv);
    int2 *seqinfo = split_seqinfo(ws, pl, hkv, D, sizeof(T));
#define TD_SPLIT(OWN)                                                                          \
    TD_LAUNCH((attn_split_f32<D, OWN>), dim3(static_cast<unsigned>(pl.n_chunks * hkv)), \
                       dim3(kAttnThreads), 0, st, static_cast<const float *>(q),                \
                       static_cast<const float *>(k_ctx), static_cast<const float *>(v_ctx), off, lens, \
                       n_nodes, batch, nq_max, hq, hkv, pl.group, pl.n_rg, pl.chunk, scale2,    \
                       static_cast<float *>(ws), prow_total, seqinfo)
#define TD_SPLIT_BF2(SUB, OWN, OWN2)                                                           \
    TD_LAUNCH((attn_split_bf16<D, OWN, OWN2, SUB>), dim3(static_cast<unsigned>(pl.n_chunks * hkv)), \
                       dim3(kAttnThreads), 0, st, static_cast<const uint16_t *>(q),             \
                       static_cast<const uint16_t *>(k_ctx), static_cast<const uint16_t *>(v_ctx), \
                       off, lens, n_nodes, batch, nq_max, hq, hkv, pl.group, pl.n_rg, pl.chunk,   \
                       scale2, static_cast<float *>(ws), prow_total, seqinfo)
    const bool ring4 = pl.chunk >= kRingChunk;
#define TD_SPLIT_BF_2(OWN, OWN2)                                                               \
    do {                                                                                       \
        if (ring4) TD_SPLIT_BF2(64, OWN, OWN2);                                                \
        else TD_SPLIT_BF2(128, OWN, OWN2);                                                     \
    } while (0)
#define TD_SPLIT_BF(OWN) TD_SPLIT_BF_2(OWN, OWN)
    const int own = std::min(pl.own, max_own<T, D>());
    if (!split) {
        // the split ran inside the step's first kernel
    } else if constexpr (max_own<T, D>() == 5) {
        switch (own) {
        case 1: TD_SPLIT_BF(1); break;
        case 2: TD_SPLIT_BF(2); break;
        case 3: TD_SPLIT_BF(3); break;
        case 4: TD_SPLIT_BF(4); break;
        default: TD_SPLIT_BF(5); break;
        }
    } else if constexpr (max_own<T, D>() == 3) {
        switch (own) {
        case 1: TD_SPLIT_BF(1); break;
        case 2: TD_SPLIT_BF(2); break;
        default:
            // trees of up to 4 row groups take the one-group code; larger
            // ones 5 per wave when the chip has several work items per
            // compute unit (one pass over the keys up to 20 row groups),
            // else 3 (a latency-bound step: the lighter code)
            if (pl.own > 3 && pl.items > 2 * kAttnCUs) TD_SPLIT_BF_2(1, 5);
            else TD_SPLIT_BF_2(1, 3);
            break;
        }
    } else {
        if (own <= 1) TD_SPLIT(1);
        else TD_SPLIT(2);
    }
#undef TD_SPLIT
#undef TD_SPLIT_BF
#undef TD_SPLIT_BF_2
#undef TD_SPLIT_BF2
    const int rpw = combine_rows_per_wave(pl.n_chunks, batch);
    // one sequence: at most n_chunks - 1 chunks (the plan adds one per sequence)
    const int nch_max = batch == 1 ? static_cast<int>(std::max<int64_t>(1, pl.n_chunks - 1)) : 0;
    const int blocks = combine_blocks(static_cast<int64_t>(batch) * hkv * pl.group * nq_max, rpw);
#define TD_COMBINE(ACC, NB, ARGS)                                                                \
    if (rpw == 8) TD_COMBINE_R(ACC, 8, NB, ARGS);                                                \
    else TD_COMBINE_R(ACC, 1, NB, ARGS)
#define TD_COMBINE_R(ACC, RR, NB, ARGS)                                                          \
    TD_LAUNCH((attn_tree_combine<T, D, ACC, RR>), dim3(static_cast<unsigned>(NB)),               \
                       dim3(kAttnThreads), 0, st, static_cast<const T *>(q), seqinfo,             \
                       static_cast<const T *>(k_tree), static_cast<const T *>(v_tree), mask,      \
                       n_nodes, batch, nq_max, hq, hkv, pl.group, pl.n_rg, pl.chunk, scale2,      \
                       static_cast<const float *>(ws), prow_total, static_cast<T *>(out), blocks, \
                       nch_max, ARGS)
    if (acc) {
        TD_COMBINE(true, blocks + batch, *acc);
    } else {
        TD_COMBINE(false, blocks, AcceptArgs{});
    }
#undef TD_COMBINE
#undef TD_COMBINE_R
}

inline int sub_chunk(td_dtype dt) { return dt == TD_BF16 ? Sub<uint16_t>::CH : Sub<float>::CH; }

inline size_t attn_ws_size(const AttnPlan &pl, int batch, int hkv, int D, td_dtype dtype) {
    return split_partial_bytes(pl, hkv, D, partial_o_bytes(dtype == TD_BF16)) + static_cast<size_t>(batch) * 8;
}

}  // namespace

size_t attn_workspace_bytes(int batch, int nq_max, int hq, int hkv, int head_dim,
                            int64_t total_ctx, td_dtype dtype, bool fused_plan) {
    const AttnPlan pl = attn_plan(batch, nq_max, hq, hkv, total_ctx, sub_chunk(dtype),
                                  fused_plan ? kFusedItems : kAttnItems);
    return std::max<size_t>(16, attn_ws_size(pl, batch, hkv, head_dim, dtype));
}

void launch_attention(const void *q, const void *k_ctx, const void *v_ctx, const int64_t *off,
                      const int64_t *lens, int64_t total_ctx, const void *k_tree, const void *v_tree,
                      const uint64_t *mask, const int32_t *n_nodes, int batch, int nq_max, int hq,
                      int hkv, int head_dim, float scale, td_dtype dtype, void *ws, void *out,
                      const AcceptArgs *acc, hipStream_t st, bool split) {
    // without the split, the partials are the fused first kernel's (its plan)
    const AttnPlan pl = attn_plan(batch, nq_max, hq, hkv, total_ctx, sub_chunk(dtype),
                                  split ? kAttnItems : kFusedItems);
    const bool bf = dtype == TD_BF16;
#define TD_ATTN(T, DD)                                                                          \
    launch_attn<T, DD>(q, k_ctx, v_ctx, off, lens, k_tree, v_tree, mask, n_nodes, batch, nq_max, hq, \
                       hkv, scale, pl, ws, out, acc, st, split)
    if (bf && head_dim == 128)
        TD_ATTN(uint16_t, 128);
    else if (bf)
        TD_ATTN(uint16_t, 64);
    else if (head_dim == 128)
        TD_ATTN(float, 128);
    else
        TD_ATTN(float, 64);
#undef TD_ATTN
}

}  // namespace td

using namespace td;

extern "C" size_t td_tree_verify_attn_workspace(int32_t batch, int32_t nq_max, int32_t hq,
                                                int32_t hkv, int32_t head_dim, int64_t total_ctx,
                                                int64_t max_ctx) {
    (void)max_ctx;
    if (batch <= 0 || nq_max <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || head_dim <= 0 ||
        total_ctx < 0)
        return 0;
    // the larger of the two dtypes' plans, so one size serves both
    return std::max(attn_workspace_bytes(batch, nq_max, hq, hkv, head_dim, total_ctx, TD_BF16),
                    attn_workspace_bytes(batch, nq_max, hq, hkv, head_dim, total_ctx, TD_F32));
}

td_status td::check_attn_args(const void *q, const void *k_ctx, const void *v_ctx,
                             const int64_t *ctx_offsets, int64_t total_ctx, int64_t max_ctx,
                             const void *k_tree, const void *v_tree, const uint64_t *mask,
                             const int32_t *n_nodes, int32_t batch, int32_t nq_max, int32_t hq,
                             int32_t hkv, int32_t head_dim, td_dtype dtype, const void *out) {
    if (!q || !k_tree || !v_tree || !ctx_offsets || !mask || !n_nodes || !out)
        return fail(TD_EINVAL, "tree_verify_attn: null pointer argument");
    if (total_ctx > 0 && (!k_ctx || !v_ctx))
        return fail(TD_EINVAL, "tree_verify_attn: null context K/V with total_ctx > 0");
    if (batch <= 0 || nq_max <= 0 || hq <= 0 || hkv <= 0 || total_ctx < 0 || max_ctx < 0)
        return fail(TD_EINVAL, "tree_verify_attn: sizes must be positive");
    if (hq % hkv != 0) return fail(TD_EINVAL, "tree_verify_attn: hq must be a multiple of hkv");
    if (nq_max > TD_MAX_NODES + 1 || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "tree_verify_attn: nq_max or batch above capacity");
    if (dtype != TD_F32 && dtype != TD_BF16)
        return fail(TD_EUNSUPPORTED, "tree_verify_attn: dtype must be TD_F32 or TD_BF16");
    if (head_dim != 64 && head_dim != 128)
        return fail(TD_EUNSUPPORTED, "tree_verify_attn: head_dim must be 64 or 128");
    if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
        (k_ctx && !aligned16(k_ctx)) || (v_ctx && !aligned16(v_ctx)) || !aligned8(mask) ||
        !aligned8(ctx_offsets))
        return fail(TD_EINVAL, "tree_verify_attn: buffers must be 16-byte aligned");
    const AttnPlan pl = attn_plan(batch, nq_max, hq, hkv, total_ctx, sub_chunk(dtype));
    if (pl.items > 0x7fffffffLL || static_cast<int64_t>(batch) * hkv * pl.n_rg * 4 > 0x7fffffffLL)
        return fail(TD_ECAPACITY, "tree_verify_attn: grid too large");
    return TD_OK;
}

extern "C" td_status td_tree_verify_attn(const void *q, const void *k_ctx, const void *v_ctx,
                                         const int64_t *ctx_offsets, const int64_t *ctx_lengths,
                                         int64_t total_ctx,
                                         int64_t max_ctx, const void *k_tree, const void *v_tree,
                                         const uint64_t *mask, const int32_t *n_nodes,
                                         int32_t batch, int32_t nq_max, int32_t hq, int32_t hkv,
                                         int32_t head_dim, float scale, td_dtype dtype, void *out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    const td_status chk = check_attn_args(q, k_ctx, v_ctx, ctx_offsets, total_ctx, max_ctx, k_tree,
                                          v_tree, mask, n_nodes, batch, nq_max, hq, hkv, head_dim,
                                          dtype, out);
    if (chk != TD_OK) return chk;
    if (ctx_lengths && !aligned8(ctx_lengths))
        return fail(TD_EINVAL, "td_tree_verify_attn: misaligned ctx_lengths");
    if (!workspace || !aligned16(workspace))
        return fail(TD_EINVAL, "td_tree_verify_attn: null or misaligned workspace");
    if (workspace_bytes <
        td_tree_verify_attn_workspace(batch, nq_max, hq, hkv, head_dim, total_ctx, max_ctx))
        return fail(TD_EINVAL, "td_tree_verify_attn: workspace too small");
    launch_attention(q, k_ctx, v_ctx, ctx_offsets, ctx_lengths, total_ctx, k_tree, v_tree, mask, n_nodes, batch,
                     nq_max, hq, hkv, head_dim, scale, dtype, workspace, out, nullptr,
                     as_stream(stream));
    return check_launch("td_tree_verify_attn");
}
