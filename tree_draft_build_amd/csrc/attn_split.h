// Device code of the split-KV context attention (attn_split_bf16,
// attn_split_f32) and its plan, shared by the attention launcher and by the
// verify step's fused first kernel.  The operation, operand layouts and key
// order are described at the top of tree_attn.hip.
#pragma once

#include <algorithm>
#include <type_traits>

#include "step_launch.h"
#include "td_internal.h"
#include "tree_core.h"

namespace td {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kAttnThreads = 256;
constexpr int kAttnCUs = 256;  // compute units of the gfx950 parts
constexpr int kAttnWaves = 4;
constexpr int kRowsPerGroup = 16;
constexpr int kKeyTile = 32;
// Row groups a wave may own: its query fragments and O^T accumulators live
// in registers (about 54 per row group at D = 128, 30 at D = 64).
template <typename T, int D>
constexpr int max_own() {
    return sizeof(T) == 4 ? 2 : (D == 128 ? 3 : 5);
}

template <typename T> struct Sub;
template <> struct Sub<uint16_t> { static constexpr int CH = 128; };
template <> struct Sub<float> { static constexpr int CH = 64; };

// ---------------------------------------------------------------------------
// split plan (host and device agree on it)
// ---------------------------------------------------------------------------
struct AttnPlan {
    int group;         // G = hq / hkv
    int n_rg;          // row groups of 16 per (b, g) at nq_max rows
    int own;           // row groups per wave and row block (block = 4 own), uncapped
    int chunk;         // keys per work item (a multiple of the sub-chunk)
    int64_t n_chunks;  // upper bound of sum_b ceil(L_b / chunk)
    int64_t items;     // n_chunks * hkv split work items
};

// Split work items the chunk length aims at: about one workgroup per compute
// unit, so that each streams one long chunk (every workgroup start and end
// drains its ring once) and few partials are written.
constexpr int64_t kAttnItems = 256;
// The verify step's fused first kernel (the split beside one top-K workgroup
// per compute unit, two workgroups per unit) keeps 128-key chunks up to
// about this many work items.
constexpr int64_t kFusedItems = 512;

inline AttnPlan attn_plan(int batch, int nq_max, int hq, int hkv, int64_t total_ctx, int CH,
                          int64_t aim = kAttnItems) {
    AttnPlan p;
    p.group = hq / hkv;
    p.n_rg = (p.group * nq_max + kRowsPerGroup - 1) / kRowsPerGroup;
    // one row block holds 4 own row groups: as many as the registers allow,
    // so that a chunk's keys stream once for every tree row where they can
    p.own = std::max(1, (p.n_rg + kAttnWaves - 1) / kAttnWaves);
    // about `aim` work items over the context; longer chunks keep the
    // partial traffic small when the context is long
    const int64_t work = std::max<int64_t>(1, total_ctx) * hkv;
    int chunk = CH;
    while (chunk < 32 * CH && work / chunk > aim) chunk *= 2;
    p.chunk = chunk;
    p.n_chunks = (total_ctx + chunk - 1) / chunk + batch;
    p.items = static_cast<int64_t>(hkv) * p.n_chunks;
    return p;
}

// Workspace: partial rows [n_chunks][hkv][n_rg][16]: m (float32), then l,
// then O[D]; row r of a (chunk, KV head) lives at prow_index(...); then one
// record per sequence (its first chunk index and chunk count), written by
// the split kernel and read by the combine kernel, which so never reads the
// context lengths (a fused KV commit may advance them in the same kernel).
__device__ __forceinline__ int64_t prow_index(int64_t c, int g, int rg, int row, int hkv, int n_rg) {
    return ((c * hkv + g) * n_rg + rg) * kRowsPerGroup + row;
}

// Locate chunk c of the ragged concatenation: sequence b and its key range.
// Sequence b owns max(1, ceil(L_b / chunk)) chunks (an empty context has one
// chunk with no keys, so the tree keys are still attended).
__device__ __forceinline__ int64_t chunks_of(int64_t L, int chunk) {
    return L > 0 ? (L + chunk - 1) / chunk : 1;
}

// Context length of sequence s: its region off[s] .. off[s+1]-1, or the
// first lens[s] rows of it when lengths are given (clamped to the region).
__device__ __forceinline__ int64_t seq_len(const int64_t *__restrict__ off,
                                           const int64_t *__restrict__ lens, int s) {
    const int64_t region = off[s + 1] - off[s];
    return lens ? std::max<int64_t>(0, std::min<int64_t>(lens[s], region)) : region;
}

// Inclusive sum over lanes 0..i of the wave, in lane i: row shifts within
// each row of 16 lanes, then the rows' totals broadcast onwards (lanes with
// no source add 0).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// A value of lane j of the wave as a 64-bit scalar.
__device__ __forceinline__ int64_t readlane64(int64_t v, int j) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), j));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), j));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Locate the chunk of work item c: sequence b, its key range, its first
// chunk index and its chunk count; c is replaced by the chunk's index in
// sequence order (the index of its partial rows).  A wave-uniform call.
//
// Up to 64 sequences, the items take the chunks longest first: every full
// chunk (sequence order), then the sequences' last, shorter chunks by
// decreasing length (ties: lower sequence first).  Workgroups start in about
// item order, so the short chunks fill the gaps at the end of the grid
// instead of a long chunk starting last.  Lane j holds sequence j; inclusive
// scans of the chunk counts over the lanes place an item, and a tail's rank
// is counted over the other lanes.
//
// More sequences: items in sequence order; lane j takes sequence s0 + j of
// each group of 64 (all lanes' loads in flight at once) and a scan of the
// chunk counts finds the sequence whose chunks cover c.  (A group's chunk
// count fits 32 bits: a chunk holds at least 128 keys of the K buffer.)
__device__ __forceinline__ bool find_chunk(const int64_t *__restrict__ off,
                                           const int64_t *__restrict__ lens, int batch, int chunk,
                                           int64_t &c, int &b, int64_t &k0, int64_t &k1,
                                           int64_t &cbase, int &nch) {
    if (batch == 1) {  // one sequence: uniform loads (scalar cache), no scan
        const int64_t L = seq_len(off, lens, 0);
        const int64_t n = chunks_of(L, chunk);
        if (c >= n) return false;
        b = 0;
        cbase = 0;
        k0 = c * chunk;
        k1 = std::min<int64_t>(L, k0 + chunk);
        nch = static_cast<int>(n);
        return true;
    }
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    if (batch <= kWave) {
        const bool in = lane < batch;
        const int64_t L = in ? seq_len(off, lens, lane) : 0;
        const uint32_t n = in ? static_cast<uint32_t>(chunks_of(L, chunk)) : 0u;
        // the last chunk's length (0 for an empty context), and the full chunks
        const uint32_t tlen = in ? static_cast<uint32_t>(L - static_cast<int64_t>(n - 1u) * chunk) : 0u;
        const uint32_t f = in ? (tlen == static_cast<uint32_t>(chunk) ? n : n - 1u) : 0u;
        const uint32_t tail = n - f;  // 1: the last chunk is short (or has no keys)
        const uint32_t n_incl = wave_incl_sum(n);
        const uint32_t f_incl = wave_incl_sum(f);
        // the grid is sized for an upper bound of the chunk count
        if (c >= static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(n_incl, kWave - 1))))
            return false;
        const int64_t full = static_cast<uint32_t>(__builtin_amdgcn_readlane(f_incl, kWave - 1));
        int j;
        int64_t local;  // the chunk's index within its sequence
        if (c < full) {
            const uint64_t hit = __ballot(in && c < static_cast<int64_t>(f_incl));
            j = __ffsll(static_cast<long long>(hit)) - 1;  // uniform
            local = c - (static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(f_incl, j))) -
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(f, j)));
        } else {
            const int64_t t = c - full;
            uint32_t rank = 0;
            for (int s = 0; s < batch; ++s) {
                const uint32_t ts = static_cast<uint32_t>(__builtin_amdgcn_readlane(tail, s));
                const uint32_t ls = static_cast<uint32_t>(__builtin_amdgcn_readlane(tlen, s));
                rank += (ts != 0u && (ls > tlen || (ls == tlen && s < lane))) ? 1u : 0u;
            }
            const uint64_t hit = __ballot(in && tail != 0u && static_cast<int64_t>(rank) == t);
            if (!hit) return false;
            j = __ffsll(static_cast<long long>(hit)) - 1;
            local = static_cast<uint32_t>(__builtin_amdgcn_readlane(f, j));
        }
        const uint32_t nj = static_cast<uint32_t>(__builtin_amdgcn_readlane(n, j));
        const int64_t Lj = readlane64(L, j);
        b = j;
        cbase = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(n_incl, j))) - nj;
        c = cbase + local;
        k0 = local * chunk;
        k1 = std::min<int64_t>(Lj, k0 + chunk);
        nch = static_cast<int>(nj);
        return true;
    }
    int64_t acc = 0;
    for (int s0 = 0; s0 < batch; s0 += kWave) {
        const int s = s0 + lane;
        const bool in = s < batch;
        const int64_t L = in ? seq_len(off, lens, s) : 0;
        const uint32_t n = in ? static_cast<uint32_t>(chunks_of(L, chunk)) : 0u;
        const uint32_t inc = wave_incl_sum(n);
        const uint64_t hit = __ballot(in && c < acc + static_cast<int64_t>(inc));
        if (hit) {
            const int j = __ffsll(static_cast<long long>(hit)) - 1;  // uniform
            const uint32_t incj = __builtin_amdgcn_readlane(inc, j);
            const uint32_t nj = __builtin_amdgcn_readlane(n, j);
            const int64_t Lj = readlane64(L, j);
            b = s0 + j;
            cbase = acc + static_cast<int64_t>(incj) - static_cast<int64_t>(nj);
            k0 = (c - cbase) * chunk;
            k1 = std::min<int64_t>(Lj, k0 + chunk);
            nch = static_cast<int>(nj);
            return true;
        }
        acc += static_cast<int64_t>(__builtin_amdgcn_readlane(inc, kWave - 1));
    }
    return false;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Partial rows of the split (m, l, then O[D] per row, in three regions):
// m and l in float32; O in bf16 for bf16 attention (half the bytes the
// combine reads back; its rounding is far below the output's own bf16
// rounding) and in float32 for float32 attention.
template <typename T> struct PartialO;
template <> struct PartialO<uint16_t> { using type = uint16_t; };
template <> struct PartialO<float> { using type = float; };
__host__ __device__ constexpr int partial_o_bytes(bool bf16) { return bf16 ? 2 : 4; }
// four consecutive O values of a partial row
__device__ __forceinline__ void put_o4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }
__device__ __forceinline__ void put_o4(uint16_t *p, f32x4 v) {
    *reinterpret_cast<u32x2 *>(p) =
        u32x2{static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
              static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16)};
}

__device__ __forceinline__ int slot_key(int h4, int t) { return t < 4 ? 4 * h4 + t : 12 + 4 * h4 + t; }

// ---------------------------------------------------------------------------
// attn_split_f32 / attn_split_bf16: one key chunk of one KV head
// ---------------------------------------------------------------------------

// float32 split kernel: K and V key-major in LDS, one sub-chunk at a time.
template <typename T, int D> struct Lds;
template <int D> struct Lds<float, D> {
    static constexpr int CH = Sub<float>::CH;
    static constexpr int KP = D + 4;
    static constexpr int VP = D + 4;    // sV key-major for f32
    static constexpr int bytes_kv = (CH * KP + CH * VP) * 4;
};

template <typename T, int D>
constexpr int split_lds_bytes() {
    constexpr int kv = Lds<T, D>::bytes_kv;
    constexpr int mg = kAttnWaves * kRowsPerGroup * (D + 2) * 4;
    return kv > mg ? kv : mg;
}

// Per row group state of a wave: running max, lane-partial sum, O^T tiles.
template <int D>
struct RowState {
    float m;
    float l;
    f32x4 o[D / 16];
    __device__ __forceinline__ void init() {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
};

template <int D>
__device__ __forceinline__ void tile_f32(const float *sK, const float *sV, const float (&qa)[D / 4],
                                         int kt, int valid, float scale2, int lane, RowState<D> &st) {
    using L = Lds<float, D>;
    const int col = lane & 15;
    const int h4 = lane >> 4;
    f32x4 s[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const float *krow = sK + (kt * kKeyTile + 16 * hf + col) * L::KP + h4 * (D / 4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k4 = 0; k4 < D / 16; ++k4) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(krow + 4 * k4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qa[4 * k4 + e], acc, 0, 0, 0);
        }
        s[hf] = acc;
    }
    float sc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float v = (t < 4 ? s[0][t] : s[1][t - 4]) * scale2;
        sc[t] = kt * kKeyTile + slot_key(h4, t) < valid ? v : -INFINITY;
    }
    float tmax = sc[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) tmax = fmaxf(tmax, sc[t]);
    tmax = fmaxf(tmax, xchg_f<4>(tmax));
    tmax = fmaxf(tmax, xchg_f<5>(tmax));
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        p[t] = __builtin_amdgcn_exp2f(sc[t] - m_new);
        ps += p[t];
    }
    st.l = st.l * alpha + ps;
    st.m = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 acc = st.o[dt] * alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float a = sV[(kt * kKeyTile + slot_key(h4, t)) * L::VP + 16 * dt + col];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[t], acc, 0, 0, 0);
        }
        st.o[dt] = acc;
    }
}

// Global -> register staging of one sub-chunk (keys clamped into range).
template <typename T, int D> struct Stage;

template <int D> struct Stage<float, D> {
    using L = Lds<float, D>;
    static constexpr int kPieces = L::CH * D / 4 / kAttnThreads;
    u32x4 k[kPieces];
    u32x4 v[kPieces];

    __device__ __forceinline__ void load(const float *kbase, const float *vbase, int64_t kstride,
                                         int valid, int tid) {
#pragma unroll
        for (int r = 0; r < kPieces; ++r) {
            const int p = tid + kAttnThreads * r;
            const int key = min(p / (D / 4), valid - 1);
            k[r] = *reinterpret_cast<const u32x4 *>(kbase + key * kstride + (p % (D / 4)) * 4);
            v[r] = *reinterpret_cast<const u32x4 *>(vbase + key * kstride + (p % (D / 4)) * 4);
        }
    }
    __device__ __forceinline__ void store(float *sK, float *sV, int tid) const {
#pragma unroll
        for (int r = 0; r < kPieces; ++r) {
            const int p = tid + kAttnThreads * r;
            const int off = (p / (D / 4)) * L::KP + (p % (D / 4)) * 4;
            *reinterpret_cast<u32x4 *>(sK + off) = k[r];
            *reinterpret_cast<u32x4 *>(sV + off) = v[r];
        }
    }
};

// The float32 split kernel (see attn_split_bf16 for the bf16 one): each
// sub-chunk is staged through registers into LDS while the previous one is
// computed on.
template <int D, int OWN>
__global__ __launch_bounds__(kAttnThreads) void attn_split_f32(
    const float *__restrict__ q, const float *__restrict__ k_ctx, const float *__restrict__ v_ctx,
    const int64_t *__restrict__ ctx_offsets, const int64_t *__restrict__ ctx_lengths,
    const int32_t *__restrict__ n_nodes, int batch, int nq_max, int hq, int hkv, int group, int n_rg,
    int chunk, float scale2, float *__restrict__ ws, int64_t prow_total, int2 *__restrict__ seqinfo) {
    using T = float;
    using L = Lds<T, D>;
    constexpr int CH = L::CH;
    __shared__ __attribute__((aligned(16))) char lds[split_lds_bytes<T, D>()];
    T *sK = reinterpret_cast<T *>(lds);
    T *sV = sK + CH * L::KP;

    int64_t c = blockIdx.x / hkv;  // the work item, then its chunk
    const int g = static_cast<int>(blockIdx.x % hkv);
    int b, nch;
    int64_t k0, k1, cbase;
    if (!find_chunk(ctx_offsets, ctx_lengths, batch, chunk, c, b, k0, k1, cbase, nch)) return;
    if (k0 == 0 && g == 0 && threadIdx.x == 0)
        seqinfo[b] = int2{static_cast<int>(cbase), nch};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;
    const int h4 = lane >> 4;

    // the KV stream goes first: its loads fly while the tree size and the
    // queries arrive
    const int64_t ctx0 = ctx_offsets[b];
    const int64_t kstride = static_cast<int64_t>(hkv) * D;
    const T *kbase = k_ctx + (ctx0 * hkv + g) * D;
    const T *vbase = v_ctx + (ctx0 * hkv + g) * D;
    const int n_sub = static_cast<int>((k1 - k0 + CH - 1) / CH);
    Stage<T, D> stage;
    if (n_sub > 0) {
        const int valid0 = static_cast<int>(std::min<int64_t>(CH, k1 - k0));
        stage.load(kbase + k0 * kstride, vbase + k0 * kstride, kstride, valid0, tid);
    }
    const int rows_b = group * min(__builtin_amdgcn_readfirstlane(n_nodes[b]) + 1, nq_max);
    const int n_rg_b = (rows_b + kRowsPerGroup - 1) / kRowsPerGroup;
    const T *qb = q + static_cast<int64_t>(b) * nq_max * hq * D;

    // row blocks of at most 4 OWN row groups, balanced
    constexpr int kBlock = kAttnWaves * OWN;
    const int n_blk = (n_rg_b + kBlock - 1) / kBlock;
    const int per_blk = n_blk > 0 ? (n_rg_b + n_blk - 1) / n_blk : 1;
    for (int rb0 = 0; rb0 < n_rg_b; rb0 += per_blk) {
        const int nrg = min(per_blk, n_rg_b - rb0);
        // wave -> (row groups, key tiles) assignment
        //   nrg >= 4: wave w owns row groups w and w + 4 of the block, all keys
        //   nrg <  4: p2 = 1, 2 or 4 row slots; waves share a row group's keys
        const int p2 = nrg >= 4 ? 4 : (nrg == 1 ? 1 : (nrg == 2 ? 2 : 4));
        const int kt_step = kAttnWaves / p2;
        const int kt_first = wave / p2;
        constexpr int kMaxOwn = OWN;
        int own_rg[kMaxOwn];
        int n_own = 0;
#pragma unroll
        for (int j = 0; j < kMaxOwn; ++j) {
            const int rl = (nrg >= 4) ? wave + kAttnWaves * j : (j == 0 ? wave % p2 : nrg);
            own_rg[j] = rl;
            n_own += rl < nrg ? 1 : 0;
        }
        const bool split_mode = nrg < 4;

        // queries of the owned row groups (B operand layout); rows past the
        // tree read row 0 of the group and are never published
        RowState<D> st[kMaxOwn];
        float qf[kMaxOwn][D / 4];
#pragma unroll
        for (int j = 0; j < kMaxOwn; ++j) {
            st[j].init();
            const int r = (rb0 + own_rg[j]) * kRowsPerGroup + col;
            const bool ok = j < n_own && r < rows_b;
            const int qi = ok ? r / group : 0;
            const int qh = g * group + (ok ? r % group : 0);
            const T *qrow = qb + (static_cast<int64_t>(qi) * hq + qh) * D;
#pragma unroll
            for (int k4 = 0; k4 < D / 16; ++k4) {
                f32x4 w = *reinterpret_cast<const f32x4 *>(qrow + h4 * (D / 4) + 4 * k4);
#pragma unroll
                for (int e = 0; e < 4; ++e) qf[j][4 * k4 + e] = w[e];
            }
        }
        if (rb0 > 0 && n_sub > 0) {  // another row block: stream the chunk again
            const int valid0 = static_cast<int>(std::min<int64_t>(CH, k1 - k0));
            stage.load(kbase + k0 * kstride, vbase + k0 * kstride, kstride, valid0, tid);
        }
        for (int sc = 0; sc < n_sub; ++sc) {
            const int64_t s0 = k0 + static_cast<int64_t>(sc) * CH;
            const int valid = static_cast<int>(std::min<int64_t>(CH, k1 - s0));
            stage.store(sK, sV, tid);
            __syncthreads();
            if (sc + 1 < n_sub) {  // next sub-chunk's loads fly during the compute
                const int64_t s1 = s0 + CH;
                const int valid1 = static_cast<int>(std::min<int64_t>(CH, k1 - s1));
                stage.load(kbase + s1 * kstride, vbase + s1 * kstride, kstride, valid1, tid);
            }
            const int ntiles = (valid + kKeyTile - 1) / kKeyTile;
            for (int kt = split_mode ? kt_first : 0; kt < ntiles; kt += split_mode ? kt_step : 1) {
#pragma unroll
                for (int j = 0; j < kMaxOwn; ++j)
                    if (j < n_own) tile_f32<D>(sK, sV, qf[j], kt, valid, scale2, lane, st[j]);
            }
            __syncthreads();
        }

        // row sums over the four lane groups
#pragma unroll
        for (int j = 0; j < kMaxOwn; ++j) {
            st[j].l += xchg_f<4>(st[j].l);
            st[j].l += xchg_f<5>(st[j].l);
        }

        float *wm = ws;
        float *wl = ws + prow_total;
        float *wo = ws + 2 * prow_total;
        if (!split_mode || kt_step == 1) {
            // each owned row group is complete in this wave: store its rows
#pragma unroll
            for (int j = 0; j < kMaxOwn; ++j) {
                if (j >= n_own) break;
                const int rg = rb0 + own_rg[j];
                if (rg * kRowsPerGroup + col >= rows_b) continue;
                const int64_t pr = prow_index(c, g, rg, col, hkv, n_rg);
                if (h4 == 0) {
                    wm[pr] = st[j].m;
                    wl[pr] = st[j].l;
                }
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    *reinterpret_cast<f32x4 *>(&wo[pr * D + 16 * dt + 4 * h4]) = st[j].o[dt];
            }
        } else {
            // split mode: kt_step waves per row group merge through LDS
            float *mw = reinterpret_cast<float *>(lds);        // [4][16]
            float *lw = mw + kAttnWaves * kRowsPerGroup;       // [4][16]
            float *ow = lw + kAttnWaves * kRowsPerGroup;       // [4][16][D]
            if (n_own > 0) {
                if (h4 == 0) {
                    mw[wave * kRowsPerGroup + col] = st[0].m;
                    lw[wave * kRowsPerGroup + col] = st[0].l;
                }
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    *reinterpret_cast<f32x4 *>(&ow[(wave * kRowsPerGroup + col) * D + 16 * dt + 4 * h4]) =
                        st[0].o[dt];
            }
            __syncthreads();
            // 16 threads per (row slot, row), each a D/16 slice; slot s merges
            // waves s, s + p2, ...
            constexpr int kPer = D / 16;
            for (int idx = tid; idx < p2 * kRowsPerGroup * 16; idx += kAttnThreads) {
                const int sl = idx / (kRowsPerGroup * 16);
                const int r = (idx / 16) % kRowsPerGroup;
                if (sl >= nrg || (rb0 + sl) * kRowsPerGroup + r >= rows_b) continue;
                const int ds = (idx % 16) * kPer;
                float M = -INFINITY;
                for (int v = sl; v < kAttnWaves; v += p2) M = fmaxf(M, mw[v * kRowsPerGroup + r]);
                float Ls = 0.f;
                float acc[kPer];
#pragma unroll
                for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
                for (int v = sl; v < kAttnWaves; v += p2) {
                    const float mv = mw[v * kRowsPerGroup + r];
                    const float f = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
                    Ls += f * lw[v * kRowsPerGroup + r];
#pragma unroll
                    for (int k = 0; k < kPer; ++k) acc[k] += f * ow[(v * kRowsPerGroup + r) * D + ds + k];
                }
                const int64_t pr = prow_index(c, g, rb0 + sl, r, hkv, n_rg);
                if ((idx % 16) == 0) {
                    wm[pr] = M;
                    wl[pr] = Ls;
                }
#pragma unroll
                for (int k = 0; k < kPer; k += 4)
                    *reinterpret_cast<f32x4 *>(&wo[pr * D + ds + k]) =
                        f32x4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]};
            }
            __syncthreads();  // LDS is reused by the next row block
        }
    }
}

// ---------------------------------------------------------------------------
// attn_split_bf16: the bf16 split kernel.  Sub-chunks of SUB keys stream
// straight from HBM into a ring of LDS buffers (global_load_lds, 16 bytes per
// lane) while one buffer is computed on, and no register holds staged data:
// two buffers of 128 keys (chunks of up to 512 keys: fewer, larger steps), or
// five of 64 keys (longer chunks: four sub-chunks, 128 KB, in flight per
// compute unit during the compute).  K and V sit key-major in LDS with no
// padding; the 16-byte pieces of a row are permuted instead, so that the
// reads below fall in distinct banks:
//   K: piece p of key row r sits at piece p ^ kswz(r).  S^T = K Q^T reads 16
//     consecutive key rows at one piece (A operand): 16 distinct pieces;
//   V: 32-byte segment s of key row r sits at segment s ^ vswz(r).
//     O^T += V^T P^T needs V transposed, which ds_read_b64_tr_b16 delivers.
//     Within a group of 16 lanes it hands lane i, as element j, element i % 4
//     of the 4 elements at the address of lane 4 j + i / 4, so lane m of
//     group G addresses 4 head dims of key 4 G + m / 4: lane i then holds head
//     dim i of keys 4 G .. 4 G + 3 (and, from a second read, of keys 16 + 4 G
//     ..), the order in which S^T leaves P in registers.  The 8 keys of a half
//     wave read one segment each, in 8 distinct segments.
// Both swizzles repeat every 16 rows, so a lane's offsets inside a row are
// the same for every tile and half tile, and the direct loads only choose
// which global piece each lane's slot receives.
// ---------------------------------------------------------------------------
// buffers of the ring for a sub-chunk of SUB keys
template <int SUB> constexpr int ring_of() { return SUB == 64 ? 5 : 2; }
constexpr int kRingChunk = 1024;  // chunks of at least this many keys take 64-key sub-chunks

template <int D> __host__ __device__ constexpr int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __host__ __device__ constexpr int vswz(int r) { return D == 128 ? (r & 7) : ((r >> 1) & 3); }
// LDS slots (16-byte pieces) of one K or V region: whole rounds of 16-byte
// loads of the workgroup, so every wave issues the same, compile-time number
// of direct loads (the compiler can then wait for an earlier load without
// waiting for them).
template <int SUB, int D> constexpr int region_slots() {
    static_assert(D == 64 || D == 128, "head dims of the bf16 split kernel");
    static_assert(SUB * (D / 8) % kAttnThreads == 0, "whole rounds of direct loads");
    return SUB * (D / 8);
}
template <int SUB, int D> constexpr int sub_k_elems() { return region_slots<SUB, D>() * 8; }
template <int SUB, int D> constexpr int sub_elems() { return 2 * region_slots<SUB, D>() * 8; }
// direct-load instructions each wave issues per sub-chunk (K and V)
template <int SUB, int D> constexpr int sub_loads() { return 2 * region_slots<SUB, D>() / kAttnThreads; }

// Wait until at most N of this wave's vector-memory loads are outstanding
// (the N most recent); LDS and export counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned u2_t __attribute__((ext_vector_type(2)));

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds + 16 l (lds must be the same for the whole wave).
__device__ __forceinline__ void lds_dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void *)p));
}

// Enqueue the direct loads of one sub-chunk's K (V = false) or V rows: the
// lane of LDS slot `slot` (row slot / P, permuted piece slot % P) loads the
// global piece that belongs there; rows at or past `valid` repeat key
// valid - 1 and are masked later.
template <int SUB, int D, bool V>
__device__ __forceinline__ void issue_rows(const uint16_t *gbase, int ks32, int valid, uint16_t *lds,
                                           int wave, int lane) {
    constexpr int P = D / 8;
    constexpr int kRounds = region_slots<SUB, D>() / kAttnThreads;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const int slot0 = (r * kAttnWaves + wave) * kWave;  // first slot of this wave (uniform)
        const int slot = slot0 + lane;
        const int row = slot / P;
        const int pp = slot % P;
        const int piece = V ? ((((pp >> 1) ^ vswz<D>(row)) << 1) | (pp & 1)) : (pp ^ kswz<D>(row));
        lds_dma16(gbase + min(row, valid - 1) * ks32 + 8 * piece, lds + 8 * slot0);
    }
}

// K fragments of one 32-key tile (the A operand of S^T = K Q^T: lane l
// reads key 16 hf + l % 16 of the tile, dims 8 (l / 16) + 32 ks ..), all
// reads in flight before one wait.  Issued from assembly: the compiler's
// schedule of the plain loads waits for each read before issuing the next.
template <int D>
__device__ __forceinline__ void read_k(const uint16_t *sK, int kt, int lane, bf16x8 (&fk)[2][D / 32]) {
    constexpr int P = D / 8;
    const int col = lane & 15;
    const int h4 = lane >> 4;
    // Row kt 32 + 16 hf + col has swizzle sw = kswz(col) in both halves, and
    // piece h4 + 4 ks of it sits at (h4 ^ (sw & 3)) + 4 (ks ^ (sw >> 2)): the
    // address of ks is x ^ (64 ks) for the ks = 0 address x (the ring is
    // 256-byte aligned and rows are 128 or 256 bytes, so bits 6 and 7 of
    // the row base are zero).  Temporaries t0 / t1 hold the others in turn,
    // each rewritten only after another pair of reads has been issued.
    const int sw = kswz<D>(col);
    const uint32_t x = (lds_addr(sK) + (kt * kKeyTile + col) * P * 16 + 16 * (h4 ^ (sw & 3))) |
                       static_cast<uint32_t>((sw >> 2) << 6);
    u32x4 t[2 * (D / 32)];
    uint32_t t0, t1;
    if constexpr (D == 128) {
        asm volatile(
            "v_xor_b32 %8, 64, %10\n"
            "v_xor_b32 %9, 0x80, %10\n"
            "ds_read_b128 %0, %10\n"
            "ds_read_b128 %4, %10 offset:4096\n"
            "ds_read_b128 %1, %8\n"
            "ds_read_b128 %5, %8 offset:4096\n"
            "ds_read_b128 %2, %9\n"
            "ds_read_b128 %6, %9 offset:4096\n"
            "v_xor_b32 %8, 0xc0, %10\n"
            "ds_read_b128 %3, %8\n"
            "ds_read_b128 %7, %8 offset:4096\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
              "=&v"(t[6]), "=&v"(t[7]), "=&v"(t0), "=&v"(t1)
            : "v"(x));
    } else {
        asm volatile(
            "v_xor_b32 %4, 64, %6\n"
            "ds_read_b128 %0, %6\n"
            "ds_read_b128 %2, %6 offset:2048\n"
            "ds_read_b128 %1, %4\n"
            "ds_read_b128 %3, %4 offset:2048\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t0), "=&v"(t1)
            : "v"(x));
    }
    (void)t1;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) fk[hf][ks] = __builtin_bit_cast(bf16x8, t[hf * (D / 32) + ks]);
}

// V^T fragments of one 32-key tile, all reads in flight before one wait.
// The LDS reads are issued from assembly: the compiler's own transposing-read
// builtin makes it wait for the other buffer's loads first.
template <int D>
__device__ __forceinline__ void read_vt(const uint16_t *sV, int kt, int lane, bf16x8 (&fv)[D / 16]) {
    constexpr int P = D / 8;
    const int G = lane >> 4;
    const int m = lane & 15;
    // key row kt 32 + 4 G + m / 4 (and 16 further, same swizzle), dims
    // 16 s + 4 (m % 4) .. of segment s, which sits at segment s ^ w: the
    // address of segment s is x ^ (32 s) for the s = 0 address x (bits 5..7
    // of the row base are zero).  Temporaries t0 / t1 hold the others in turn,
    // each rewritten only after another pair of reads has been issued.
    const int r0 = kt * kKeyTile + 4 * G + (m >> 2);
    const int w = vswz<D>(r0);
    const uint32_t x = (lds_addr(sV) + r0 * P * 16 + 8 * (m & 3)) | static_cast<uint32_t>(w << 5);
    u2_t t[2 * (D / 16)];
    uint32_t t0, t1;
    if constexpr (D == 128) {
        asm volatile(
            "v_xor_b32 %16, 32, %18\n"
            "v_xor_b32 %17, 64, %18\n"
            "ds_read_b64_tr_b16 %0, %18\n"
            "ds_read_b64_tr_b16 %1, %18 offset:4096\n"
            "ds_read_b64_tr_b16 %2, %16\n"
            "ds_read_b64_tr_b16 %3, %16 offset:4096\n"
            "ds_read_b64_tr_b16 %4, %17\n"
            "ds_read_b64_tr_b16 %5, %17 offset:4096\n"
            "v_xor_b32 %16, 0x60, %18\n"
            "ds_read_b64_tr_b16 %6, %16\n"
            "ds_read_b64_tr_b16 %7, %16 offset:4096\n"
            "v_xor_b32 %17, 0x80, %18\n"
            "ds_read_b64_tr_b16 %8, %17\n"
            "ds_read_b64_tr_b16 %9, %17 offset:4096\n"
            "v_xor_b32 %16, 0xa0, %18\n"
            "ds_read_b64_tr_b16 %10, %16\n"
            "ds_read_b64_tr_b16 %11, %16 offset:4096\n"
            "v_xor_b32 %17, 0xc0, %18\n"
            "ds_read_b64_tr_b16 %12, %17\n"
            "ds_read_b64_tr_b16 %13, %17 offset:4096\n"
            "v_xor_b32 %16, 0xe0, %18\n"
            "ds_read_b64_tr_b16 %14, %16\n"
            "ds_read_b64_tr_b16 %15, %16 offset:4096\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
              "=&v"(t[6]), "=&v"(t[7]), "=&v"(t[8]), "=&v"(t[9]), "=&v"(t[10]), "=&v"(t[11]),
              "=&v"(t[12]), "=&v"(t[13]), "=&v"(t[14]), "=&v"(t[15]), "=&v"(t0), "=&v"(t1)
            : "v"(x));
    } else {
        asm volatile(
            "v_xor_b32 %8, 32, %10\n"
            "v_xor_b32 %9, 64, %10\n"
            "ds_read_b64_tr_b16 %0, %10\n"
            "ds_read_b64_tr_b16 %1, %10 offset:2048\n"
            "ds_read_b64_tr_b16 %2, %8\n"
            "ds_read_b64_tr_b16 %3, %8 offset:2048\n"
            "ds_read_b64_tr_b16 %4, %9\n"
            "ds_read_b64_tr_b16 %5, %9 offset:2048\n"
            "v_xor_b32 %8, 0x60, %10\n"
            "ds_read_b64_tr_b16 %6, %8\n"
            "ds_read_b64_tr_b16 %7, %8 offset:2048\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
              "=&v"(t[6]), "=&v"(t[7]), "=&v"(t0), "=&v"(t1)
            : "v"(x));
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        fv[dt] = __builtin_bit_cast(bf16x8, u32x4{t[2 * dt].x, t[2 * dt].y, t[2 * dt + 1].x, t[2 * dt + 1].y});
}

// Headroom of the lazy running maximum (base 2): a row's reference maximum
// moves only when one of its scores passes it by more than this, so every
// probability stays below 2^kLazyMax (exact in float32 and bf16) and the
// accumulators are rescaled on few tiles.  Any reference value gives the
// same softmax; the partials carry theirs to the combine.
constexpr float kLazyMax = 8.f;

// One 32-key tile for the OWN row groups a wave owns (all of them computed:
// a row group past the tree has zero queries and is never stored): S^T =
// K Q^T (K rows read from LDS once for all), then, in one straight block,
// P = exp2(S scale2 - m) and O^T += V^T P^T (V^T fragments read once), so
// the matrix core works on one row group while the vector unit makes the
// next one's probabilities.  Keys at or past `valid` are masked.
template <int D, int OWN>
__device__ __forceinline__ void tile_dma(const uint16_t *sK, const uint16_t *sV,
                                         const bf16x8 (&qf)[OWN][D / 32], int kt, int valid,
                                         float scale2, int lane, RowState<D> (&st)[OWN]) {
    const int h4 = lane >> 4;
    float sc[OWN][8];
    {
        bf16x8 fk[2][D / 32];
        read_k<D>(sK, kt, lane, fk);
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[hf][ks], qf[j][ks], a, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < 4; ++t) sc[j][4 * hf + t] = a[t];
            }
    }
    if (kt * kKeyTile + kKeyTile > valid) {
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                sc[j][t] = kt * kKeyTile + slot_key(h4, t) < valid ? sc[j][t] : -INFINITY;
    }
    // does any score of this lane pass its row's reference by the headroom?
    float lmax[OWN];
    bool over = false;
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
        float x = sc[j][0];
#pragma unroll
        for (int t = 1; t < 8; ++t) x = fmaxf(x, sc[j][t]);
        lmax[j] = x;
        over = over || x * scale2 > st[j].m + kLazyMax;
    }
    if (__builtin_amdgcn_ballot_w64(over)) {  // the first tile, then rarely
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            float tmax = fmaxf(lmax[j], xchg_f<4>(lmax[j]));
            tmax = fmaxf(tmax, xchg_f<5>(tmax));
            const float m_new = fmaxf(st[j].m, tmax * scale2);
            const float alpha = __builtin_amdgcn_exp2f(st[j].m - m_new);
            st[j].l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) st[j].o[dt] *= alpha;
            st[j].m = m_new;
        }
    }
    bf16x8 fv[D / 16];
    read_vt<D>(sV, kt, lane, fv);
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
        bf16x8 pf;
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[j][t], scale2, -st[j].m));
            ps += p;
            pf[t] = static_cast<__bf16>(p);  // round to nearest even
        }
        st[j].l += ps;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            st[j].o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fv[dt], pf, st[j].o[dt], 0, 0, 0);
    }
}

// OWN2 > OWN: a tree of more than 4 OWN row groups is processed with OWN2
// per wave instead (one pass over the keys where OWN would need several);
// smaller trees keep the lighter OWN code.
template <int D, int OWN, int OWN2, int SUB>
__global__ __launch_bounds__(kAttnThreads) void attn_split_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_ctx,
    const uint16_t *__restrict__ v_ctx, const int64_t *__restrict__ ctx_offsets,
    const int64_t *__restrict__ ctx_lengths, const int32_t *__restrict__ n_nodes, int batch,
    int nq_max, int hq, int hkv, int group, int n_rg, int chunk, float scale2,
    float *__restrict__ ws, int64_t prow_total, int2 *__restrict__ seqinfo) {
    // kRing buffers, each K then V of one sub-chunk; the merge scratch of
    // split mode reuses the ring once no load is in flight
    constexpr int kSubB = SUB;
    constexpr int kRing = ring_of<SUB>();
    constexpr int kSubElems = sub_elems<SUB, D>();
    __shared__ __attribute__((aligned(256))) uint16_t sring[kRing * kSubElems];
    uint16_t *const sbuf0 = sring;
    constexpr int kVOff = sub_k_elems<SUB, D>();  // the V region follows the K region
    constexpr int kLoads = sub_loads<SUB, D>();
    static_assert((kRing - 2) * kLoads < 64, "the loads of the sub-chunks in flight fit the wait counter");
    auto ring = [&](int sc) { return sring + (sc % kRing) * kSubElems; };

    int64_t c = blockIdx.x / hkv;  // the work item, then its chunk
    const int g = static_cast<int>(blockIdx.x % hkv);
    int b, nch;
    int64_t k0, k1, cbase;
    if (!find_chunk(ctx_offsets, ctx_lengths, batch, chunk, c, b, k0, k1, cbase, nch)) return;
    if (k0 == 0 && g == 0 && threadIdx.x == 0)
        seqinfo[b] = int2{static_cast<int>(cbase), nch};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int h4 = lane >> 4;

    // the KV stream goes first: its loads fly while the tree size and the
    // queries arrive
    const int64_t ctx0 = ctx_offsets[b];
    const int64_t kstride = static_cast<int64_t>(hkv) * D;
    const uint16_t *kbase = k_ctx + (ctx0 * hkv + g) * D;
    const uint16_t *vbase = v_ctx + (ctx0 * hkv + g) * D;
    const int n_sub = static_cast<int>((k1 - k0 + kSubB - 1) / kSubB);
    // sub-chunk sc: keys k0 + sc kSubB .., `valid` of them
#define TD_SUB_VALID(sc) \
    static_cast<int>(std::min<int64_t>(kSubB, k1 - k0 - static_cast<int64_t>(sc) * kSubB))
// (a chunk without keys loads copies of the first queries instead: every
// workgroup issues its first sub-chunk's loads unconditionally)
#define TD_ISSUE(sc, buf)                                                                      \
    {                                                                                          \
        const int64_t s0_ = (k0 + static_cast<int64_t>(sc) * kSubB) * kstride;               \
        const int v_ = TD_SUB_VALID(sc);                                                       \
        issue_rows<SUB, D, false>(v_ > 0 ? kbase + s0_ : q, static_cast<int>(kstride),         \
                                      v_ > 0 ? v_ : 1, buf, wave, lane);                       \
        issue_rows<SUB, D, true>(v_ > 0 ? vbase + s0_ : q, static_cast<int>(kstride),          \
                                      v_ > 0 ? v_ : 1, buf + kVOff, wave, lane);               \
    }
    // in flight while the first loads are issued; read as uniform (else the
    // compiler may run the key loops' control on the vector unit)
    const int nn_b = __builtin_amdgcn_readfirstlane(n_nodes[b]);
    const uint16_t *qb = q + static_cast<int64_t>(b) * nq_max * hq * D;
    // Row group 0 (tree rows of the root onwards) always has work: its
    // queries load now rather than after the tree size arrives.
    bf16x8 q0[D / 32];
    {
        const int qi = min(col / group, nq_max - 1);
        const uint16_t *qrow = qb + (static_cast<int64_t>(qi) * hq + g * group + col % group) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            q0[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + 32 * ks + 8 * h4));
    }
    // the ring's first kRing - 1 sub-chunks (sub-chunk 0 even without keys)
    TD_ISSUE(0, ring(0));
#pragma unroll
    for (int p = 1; p + 1 < kRing; ++p)
        if (n_sub > p) TD_ISSUE(p, ring(p));
    const int rows_b = group * min(nn_b + 1, nq_max);
    const int n_rg_b = (rows_b + kRowsPerGroup - 1) / kRowsPerGroup;
    if (n_rg_b <= 0) {  // no row at all (a tree build that gave up): drain the loads above
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    auto row_blocks = [&](auto own_tag) __attribute__((always_inline)) {
        constexpr int OWNX = decltype(own_tag)::value;
        // row blocks of at most 4 OWNX row groups, balanced
        constexpr int kBlock = kAttnWaves * OWNX;
        const int n_blk = (n_rg_b + kBlock - 1) / kBlock;
        const int per_blk = n_blk > 0 ? (n_rg_b + n_blk - 1) / n_blk : 1;
        for (int rb0 = 0; rb0 < n_rg_b; rb0 += per_blk) {
            if (rb0 > 0 && n_sub > 0) {  // another row block: stream the chunk again
#pragma unroll
                for (int p = 0; p + 1 < kRing; ++p)
                    if (n_sub > p) TD_ISSUE(p, ring(p));
            }
            const int nrg = min(per_blk, n_rg_b - rb0);
            // wave -> (row groups, key tiles) assignment
            //   nrg >= 4: wave w owns row groups w, w + 4, ... of the block, all keys
            //   nrg <  4: p2 = 1, 2 or 4 row slots; waves share a row group's keys
            const int p2 = nrg >= 4 ? 4 : (nrg == 1 ? 1 : (nrg == 2 ? 2 : 4));
            const int kt_step = kAttnWaves / p2;
            const int kt_first = wave / p2;
            int own_rg[OWNX];
            int n_own = 0;
#pragma unroll
            for (int j = 0; j < OWNX; ++j) {
                const int rl = (nrg >= 4) ? wave + kAttnWaves * j : (j == 0 ? wave % p2 : nrg);
                own_rg[j] = rl;
                n_own += rl < nrg ? 1 : 0;
            }
            const bool split_mode = nrg < 4;

            // queries of the owned row groups (B operand layout); rows past the
            // tree read row 0 of the group and are never published
            RowState<D> st[OWNX];
            bf16x8 qf[OWNX][D / 32];
#pragma unroll
            for (int j = 0; j < OWNX; ++j) {
                st[j].init();
                if (rb0 + own_rg[j] == 0) {  // already loaded
#pragma unroll
                    for (int ks = 0; ks < D / 32; ++ks) qf[j][ks] = q0[ks];
                    continue;
                }
                if (j >= n_own) {  // no row group: never read
#pragma unroll
                    for (int ks = 0; ks < D / 32; ++ks) qf[j][ks] = bf16x8{};
                    continue;
                }
                const int r = (rb0 + own_rg[j]) * kRowsPerGroup + col;
                const bool ok = j < n_own && r < rows_b;
                const int qi = ok ? r / group : 0;
                const int qh = g * group + (ok ? r % group : 0);
                const uint16_t *qrow = qb + (static_cast<int64_t>(qi) * hq + qh) * D;
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
                    qf[j][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + 32 * ks + 8 * h4));
            }
            // The queries arrive behind the ring's first direct loads; waiting
            // for all of them here (they land together) settles the queries
            // once, so no wait inside the loop below is held up by them.
            __builtin_amdgcn_s_waitcnt(0);

#define TD_COMPUTE(buf, sc)                                                                    \
        {                                                                                          \
            const int valid = TD_SUB_VALID(sc);                                                    \
            const int ntiles = (valid + kKeyTile - 1) / kKeyTile;                                  \
            for (int kt = split_mode ? kt_first : 0; kt < ntiles; kt += split_mode ? kt_step : 1) { \
                tile_dma<D, OWNX>(buf, buf + kVOff, qf, kt, valid, scale2, lane, st);               \
            }                                                                                      \
        }
            // sub-chunk sc sits in buffer sc % kRing; the kRing - 2 after it
            // stay in flight while it is waited for, and sub-chunk
            // sc + kRing - 1 goes into the buffer sub-chunk sc - 1 used
            for (int sc = 0; sc < n_sub; ++sc) {
                const int ahead = min(kRing - 2, n_sub - 1 - sc);  // sub-chunks issued after sc
                if (kRing > 4 && ahead >= 3) wait_vm<(kRing > 4 ? 3 : 0) * kLoads>();
                else if (ahead >= 2) wait_vm<2 * kLoads>();
                else if (ahead == 1) wait_vm<kLoads>();
                else wait_vm<0>();
                __syncthreads();  // everyone's loads of sc have landed; buffer sc - 1 is free
                if (sc + kRing - 1 < n_sub) TD_ISSUE(sc + kRing - 1, ring(sc + kRing - 1));
                uint16_t *const cur = ring(sc);
                TD_COMPUTE(cur, sc);
            }
#undef TD_COMPUTE
            __builtin_amdgcn_s_waitcnt(0);  // also a sub-chunk 0 without keys
            __syncthreads();  // every wave is done with every buffer

            // row sums over the four lane groups
#pragma unroll
            for (int j = 0; j < OWNX; ++j) {
                st[j].l += xchg_f<4>(st[j].l);
                st[j].l += xchg_f<5>(st[j].l);
            }

            float *wm = ws;
            float *wl = ws + prow_total;
            uint16_t *wo = reinterpret_cast<uint16_t *>(ws + 2 * prow_total);
            if (!split_mode || kt_step == 1) {
                // each owned row group is complete in this wave: store its rows
#pragma unroll
                for (int j = 0; j < OWNX; ++j) {
                    if (j >= n_own) break;
                    const int rg = rb0 + own_rg[j];
                    if (rg * kRowsPerGroup + col >= rows_b) continue;
                    const int64_t pr = prow_index(c, g, rg, col, hkv, n_rg);
                    if (h4 == 0) {
                        wm[pr] = st[j].m;
                        wl[pr] = st[j].l;
                    }
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt)
                        put_o4(&wo[pr * D + 16 * dt + 4 * h4], st[j].o[dt]);
                }
            } else {
                // split mode: kt_step waves per row group merge through LDS
                constexpr int kMP = D + 4;
                static_assert((2 * kAttnWaves * kRowsPerGroup + kAttnWaves * kRowsPerGroup * kMP) * 4 <=
                                  kRing * kSubElems * 2,
                              "the merge area fits the ring");
                float *mw = reinterpret_cast<float *>(sbuf0);      // [4][16]
                float *lw = mw + kAttnWaves * kRowsPerGroup;       // [4][16]
                float *ow = lw + kAttnWaves * kRowsPerGroup;       // [4][16][kMP]
                // rows padded by 4 floats: the 16 rows of one 16-byte store land
                // in distinct banks
                if (n_own > 0) {
                    if (h4 == 0) {
                        mw[wave * kRowsPerGroup + col] = st[0].m;
                        lw[wave * kRowsPerGroup + col] = st[0].l;
                    }
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt)
                        *reinterpret_cast<f32x4 *>(&ow[(wave * kRowsPerGroup + col) * kMP + 16 * dt + 4 * h4]) =
                            st[0].o[dt];
                }
                __syncthreads();
                // 16 threads per (row slot, row), each a D/16 slice; slot s merges
                // waves s, s + p2, ...
                constexpr int kPer = D / 16;
                for (int idx = tid; idx < p2 * kRowsPerGroup * 16; idx += kAttnThreads) {
                    const int sl = idx / (kRowsPerGroup * 16);
                    const int r = (idx / 16) % kRowsPerGroup;
                    if (sl >= nrg || (rb0 + sl) * kRowsPerGroup + r >= rows_b) continue;
                    const int ds = (idx % 16) * kPer;
                    float M = -INFINITY;
                    for (int v = sl; v < kAttnWaves; v += p2) M = fmaxf(M, mw[v * kRowsPerGroup + r]);
                    float Ls = 0.f;
                    float acc[kPer];
#pragma unroll
                    for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
                    for (int v = sl; v < kAttnWaves; v += p2) {
                        const float mv = mw[v * kRowsPerGroup + r];
                        const float f = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
                        Ls += f * lw[v * kRowsPerGroup + r];
#pragma unroll
                        for (int k = 0; k < kPer; ++k) acc[k] += f * ow[(v * kRowsPerGroup + r) * kMP + ds + k];
                    }
                    const int64_t pr = prow_index(c, g, rb0 + sl, r, hkv, n_rg);
                    if ((idx % 16) == 0) {
                        wm[pr] = M;
                        wl[pr] = Ls;
                    }
#pragma unroll
                    for (int k = 0; k < kPer; k += 4)
                        put_o4(&wo[pr * D + ds + k], f32x4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]});
                }
                __syncthreads();  // LDS is reused by the next row block
            }
        }
    };
    if (OWN2 > OWN && n_rg_b > kAttnWaves * OWN)
        row_blocks(std::integral_constant<int, OWN2>{});
    else
        row_blocks(std::integral_constant<int, OWN>{});
#undef TD_ISSUE
#undef TD_SUB_VALID
}

// Partial rows of a plan (the split kernel's output): m and l (float32), then
// O[D] (o_bytes each) per row; the per-sequence chunk records follow them.
inline int64_t split_prow_total(const AttnPlan &pl, int hkv) {
    return pl.n_chunks * hkv * pl.n_rg * kRowsPerGroup;
}
inline size_t split_partial_bytes(const AttnPlan &pl, int hkv, int D, int o_bytes) {
    return static_cast<size_t>(split_prow_total(pl, hkv)) * (8 + static_cast<size_t>(D) * o_bytes);
}
inline int2 *split_seqinfo(void *ws, const AttnPlan &pl, int hkv, int D, int o_bytes) {
    return reinterpret_cast<int2 *>(static_cast<char *>(ws) + split_partial_bytes(pl, hkv, D, o_bytes));
}

// ---------------------------------------------------------------------------
// The context split as part of the verify step's first kernel, for plans
// whose chunks hold at most one sub-chunk of kFusedKeys keys.  Such a
// workgroup runs beside the draft workgroups of the same launch: it loads
// its chunk into one LDS buffer and the queries of row group `wave` (every
// query row exists in memory, whatever the tree size), computes that row
// group over the whole chunk, stores the root's rows (tree row 0 is in every
// tree), and only then waits for the sequence's tree size, which the tree
// builder publishes as one tagged word.  The other rows inside the tree are
// stored after it; a larger tree continues with row groups
// wave + 4, wave + 8, ... from the same buffer (their queries loaded one
// group ahead).  A tree of fixed size (no S(N) stop) fills every row, so
// there the workgroup computes all row groups at once and never waits.  The
// partials and chunk records are those of attn_split_bf16.
// ---------------------------------------------------------------------------
constexpr int kFusedKeys = Sub<uint16_t>::CH;

struct SplitArgs {
    const uint16_t *q, *k_ctx, *v_ctx;
    const int64_t *ctx_offsets, *ctx_lengths;
    const uint64_t *ready;  // [batch] tagged tree sizes: (1 << 32) | n
    uint32_t *status;       // kStatusSplit is raised here when the wait gives up
    int all_rows;           // nonzero: every query row, without waiting (fixed-size trees)
    int batch, nq_max, hq, hkv, group, n_rg, chunk;
    float scale2;
    float *ws;
    int64_t prow_total;
    int2 *seqinfo;
};

template <int D>
struct FusedSplitLds {
    alignas(256) uint16_t buf[sub_elems<kFusedKeys, D>()];
    int nn;  // the tree size, from wave 0 to the others
};

// Polls of the tree-size word before giving up (each one a memory round
// trip plus a short sleep; the builder finishes within tens of microseconds).
constexpr int kReadySpins = 1 << 16;
constexpr int kNoTree = -0x40000000;  // the wait gave up

template <int D>
__device__ __forceinline__ void fused_split(const SplitArgs &a, int64_t item, FusedSplitLds<D> &L) {
    constexpr int kVOff = sub_k_elems<kFusedKeys, D>();
    int64_t c = item / a.hkv;  // the work item, then its chunk
    const int g = static_cast<int>(item % a.hkv);
    int b, nch;
    int64_t k0, k1, cbase;
    if (!find_chunk(a.ctx_offsets, a.ctx_lengths, a.batch, a.chunk, c, b, k0, k1, cbase, nch)) return;
    if (k0 == 0 && g == 0 && threadIdx.x == 0) a.seqinfo[b] = int2{static_cast<int>(cbase), nch};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int h4 = lane >> 4;
    const int valid = static_cast<int>(k1 - k0);  // 0 .. kFusedKeys
    const int kstride = a.hkv * D;
    {
        // (a chunk without keys loads copies of the first query row instead)
        const int64_t at = ((a.ctx_offsets[b] + k0) * a.hkv + g) * D;
        issue_rows<kFusedKeys, D, false>(valid > 0 ? a.k_ctx + at : a.q, kstride, valid > 0 ? valid : 1,
                                         L.buf, wave, lane);
        issue_rows<kFusedKeys, D, true>(valid > 0 ? a.v_ctx + at : a.q, kstride, valid > 0 ? valid : 1,
                                        L.buf + kVOff, wave, lane);
    }
    // queries of row group rg in the B operand layout (rows past the
    // nq_max query rows read the last one; they are never stored)
    const uint16_t *qb = a.q + static_cast<int64_t>(b) * a.nq_max * a.hq * D;
    auto load_q = [&](int rg, bf16x8 (&qf)[1][D / 32]) __attribute__((always_inline)) {
        const int r = rg * kRowsPerGroup + col;
        const int qi = min(r / a.group, a.nq_max - 1);
        const uint16_t *qrow = qb + (static_cast<int64_t>(qi) * a.hq + g * a.group + r % a.group) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            qf[0][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + 32 * ks + 8 * h4));
    };
    const int ntiles = (valid + kKeyTile - 1) / kKeyTile;
    float *wm = a.ws;
    float *wl = a.ws + a.prow_total;
    uint16_t *wo = reinterpret_cast<uint16_t *>(a.ws + 2 * a.prow_total);
    // one row group (queries qf) over the whole chunk
    auto run = [&](const bf16x8 (&qf)[1][D / 32]) __attribute__((always_inline)) {
        RowState<D> st[1];
        st[0].init();
        for (int kt = 0; kt < ntiles; ++kt) tile_dma<D, 1>(L.buf, L.buf + kVOff, qf, kt, valid, a.scale2, lane, st);
        st[0].l += xchg_f<4>(st[0].l);
        st[0].l += xchg_f<5>(st[0].l);
        return st[0];
    };
    // rows lo .. hi - 1 of row group rg
    auto put = [&](int rg, const RowState<D> &st, int lo, int hi) __attribute__((always_inline)) {
        const int r = rg * kRowsPerGroup + col;
        if (r < lo || r >= hi) return;
        const int64_t pr = prow_index(c, g, rg, col, a.hkv, a.n_rg);
        if (h4 == 0) {
            wm[pr] = st.m;
            wl[pr] = st.l;
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            put_o4(&wo[pr * D + 16 * dt + 4 * h4], st.o[dt]);
    };

    bf16x8 qf[1][D / 32], qn[1][D / 32];
    load_q(wave, qf);
    load_q(wave + kAttnWaves, qn);  // the group after it, should the tree be that large
    wait_vm<0>();
    __syncthreads();  // every wave's part of the chunk is in LDS
    if (a.all_rows) {
        // A tree of fixed size fills all nq_max rows (unless its candidates
        // run out; rows past it are never read): every row group now, while
        // the tree is being built, and no wait for its size.
        const int rows_all = a.group * a.nq_max;
        for (int rg = wave; rg < a.n_rg; rg += kAttnWaves) {
            if (rg > wave) {
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) qf[0][ks] = qn[0][ks];
                if (rg + kAttnWaves < a.n_rg) load_q(rg + kAttnWaves, qn);
            }
            put(rg, run(qf), 0, rows_all);
        }
        return;
    }
    RowState<D> st0;
    st0.init();
    if (wave < a.n_rg) {
        st0 = run(qf);
        put(wave, st0, 0, a.group);  // the root's rows are in every tree: stored now
    }

    // the tree size (wave 0 polls; the others wait at the barrier)
    if (wave == 0) {
        const uint64_t *rw = a.ready + b;
        uint64_t w = __hip_atomic_load(const_cast<uint64_t *>(rw), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int spins = 0; (w >> 32) == 0 && spins < kReadySpins; ++spins) {
            __builtin_amdgcn_s_sleep(2);
            w = __hip_atomic_load(const_cast<uint64_t *>(rw), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) {
            L.nn = (w >> 32) != 0 ? static_cast<int>(static_cast<uint32_t>(w)) : kNoTree;
            if ((w >> 32) == 0) __hip_atomic_fetch_or(a.status, kStatusSplit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    const int nn = __builtin_amdgcn_readfirstlane(L.nn);
    if (nn == kNoTree) return;
    const int rows_b = a.group * min(nn + 1, a.nq_max);  // 0 when the build gave up (nn = -1)
    const int n_rg_b = (rows_b + kRowsPerGroup - 1) / kRowsPerGroup;
    if (wave < n_rg_b) put(wave, st0, a.group, rows_b);
    for (int rg = wave + kAttnWaves; rg < n_rg_b; rg += kAttnWaves) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) qf[0][ks] = qn[0][ks];
        if (rg + kAttnWaves < n_rg_b) load_q(rg + kAttnWaves, qn);
        put(rg, run(qf), 0, rows_b);
    }
}

}  // namespace
}  // namespace td
