// Stage (c): tree verification attention (BASTION: the target scores every
// node of the draft tree in one parallel pass; a node may only see the
// context and its own root path).
//
// For sequence b, query head h (KV head g = h / G, G = hq / hkv) and tree row
// i <= n_nodes[b], the admitted keys are the whole context of b plus the
// tree nodes on the root path of i.  The context part is dense and carries
// almost all bytes and flops; the tree part is sparse (at most depth+1 keys
// per row).  Two kernels:
//
//  attn_ctx_split   split-KV over the context.  Work item = (KV head g, row
//                   group of 16 query rows, context chunk).  The G heads of a
//                   group times the tree rows form the M dimension (row
//                   r = i * G + hh).  Each of the 4 waves takes 32-key tiles
//                   of the chunk; per tile
//                      S^T (32 keys x 16 rows) = K Q^T   2 x (D/32) MFMA 16x16x32
//                      online softmax in base 2 on S^T
//                      O^T (D x 16 rows) += V^T P^T      D/16 MFMA 16x16x32
//                   K comes straight from HBM in the MFMA A layout (16-byte
//                   loads, head_dim contiguous); V is staged in LDS and read
//                   key-strided for the A operand of the second product.  The
//                   4 waves then merge through LDS and one (m, l, O) partial
//                   per row is written.
//  attn_tree_combine one workgroup per (b, g, row group): merges the
//                   context partials, adds the ancestor-masked tree keys
//                   (sparse: one dot product per set mask bit) and writes
//                   the normalised output; rows beyond the tree are zeroed.
//
// MFMA 16x16x32 bf16 operand layout (wave64): A (16 x 32): lane l holds row
// l % 16, k = 8 (l / 16) .. +7; B (32 x 16): lane l holds column l % 16, the
// same k; C (16 x 16): lane l holds column l % 16, rows 4 (l / 16) .. +3.
// The f32 variant uses MFMA 16x16x4 (A/B: lane l holds k = l / 16).

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = 4;
constexpr int kRowsPerGroup = 16;
constexpr int kKeyTile = 32;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// split plan (host and device agree on it)
// ---------------------------------------------------------------------------
struct AttnPlan {
    int group;     // G = hq / hkv
    int n_rg;      // row groups of 16 per (b, g)
    int chunk;     // keys per work item (multiple of kAttnWaves * kKeyTile)
    int64_t n_chunks;  // upper bound of sum_b ceil(L_b / chunk)
    int64_t items;     // hkv * n_rg * n_chunks
};

inline AttnPlan attn_plan(int batch, int nq_max, int hq, int hkv, int64_t total_ctx) {
    AttnPlan p;
    p.group = hq / hkv;
    p.n_rg = (p.group * nq_max + kRowsPerGroup - 1) / kRowsPerGroup;
    // aim at ~1024 work items over the whole context
    const int64_t work = std::max<int64_t>(1, total_ctx) * hkv;
    int chunk = kAttnWaves * kKeyTile;
    while (chunk < 4096 && work / chunk > 1024) chunk *= 2;
    p.chunk = chunk;
    p.n_chunks = (total_ctx + chunk - 1) / chunk + batch;
    p.items = static_cast<int64_t>(hkv) * p.n_rg * p.n_chunks;
    return p;
}

inline size_t attn_ws_bytes(const AttnPlan &p, int D) {
    const int64_t rows = p.items * kRowsPerGroup;
    return static_cast<size_t>(rows) * (2 + D) * sizeof(float);
}

struct AttnWs {
    float *m;  // [items][16]
    float *l;  // [items][16]
    float *o;  // [items][16][D]
};

__host__ __device__ inline AttnWs attn_ws(void *base, int64_t items, int D) {
    AttnWs w;
    w.m = static_cast<float *>(base);
    w.l = w.m + items * kRowsPerGroup;
    w.o = w.l + items * kRowsPerGroup;
    return w;
}

// Locate chunk c of the ragged concatenation: sequence b and its key range.
// Returns false if c lies beyond the last sequence's chunks.
__device__ __forceinline__ bool find_chunk(const int64_t *__restrict__ off, int batch, int chunk,
                                           int64_t c, int &b, int64_t &k0, int64_t &k1) {
    int64_t acc = 0;
    for (int s = 0; s < batch; ++s) {
        const int64_t L = off[s + 1] - off[s];
        const int64_t n = (L + chunk - 1) / chunk;
        if (c < acc + n) {
            b = s;
            k0 = (c - acc) * chunk;
            k1 = std::min<int64_t>(L, k0 + chunk);
            return true;
        }
        acc += n;
    }
    return false;
}

// first global chunk index of sequence b
__device__ __forceinline__ int64_t chunk_base(const int64_t *__restrict__ off, int b, int chunk) {
    int64_t acc = 0;
    for (int s = 0; s < b; ++s) acc += (off[s + 1] - off[s] + chunk - 1) / chunk;
    return acc;
}

// ---------------------------------------------------------------------------
// dtype-specific fragments
// ---------------------------------------------------------------------------
template <typename T, int D> struct Frag;

// bf16: MFMA 16x16x32.  A lane's k-slice for step s is d = 32 s + 8 (l/16) .. +7.
template <int D> struct Frag<uint16_t, D> {
    static constexpr int kSteps = D / 32;
    typedef bf16x8 QK;  // one operand register group per step

    __device__ __forceinline__ static QK load8(const uint16_t *p) {
        u32x4 w = *reinterpret_cast<const u32x4 *>(p);
        return __builtin_bit_cast(bf16x8, w);
    }
    __device__ __forceinline__ static QK zero() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }
    // operand for step s of the row/key `ptr` points at (head_dim contiguous)
    __device__ __forceinline__ static QK qk_operand(const uint16_t *row, int s, int lane) {
        return load8(row + 32 * s + 8 * (lane >> 4));
    }
    __device__ __forceinline__ static f32x4 mma_qk(QK a, QK b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // P^T operand: lane (row, h) holds its 8 probabilities in slot order
    // t<4 -> key 4h+t, t>=4 -> key 16+4h+t-4.
    __device__ __forceinline__ static QK p_operand(const float (&p)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = static_cast<uint32_t>(f32_to_bf16(p[2 * k])) |
                   (static_cast<uint32_t>(f32_to_bf16(p[2 * k + 1])) << 16);
        return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }
    // V^T operand for d-tile dt from the key-major LDS tile (pitch in elements).
    __device__ __forceinline__ static QK v_operand(const uint16_t *sv, int pitch, int dt, int lane) {
        const int d = 16 * dt + (lane & 15);
        const int h = lane >> 4;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t0 = 2 * k, t1 = 2 * k + 1;
            const int k0 = t0 < 4 ? 4 * h + t0 : 16 + 4 * h + (t0 - 4);
            const int k1 = t1 < 4 ? 4 * h + t1 : 16 + 4 * h + (t1 - 4);
            w[k] = static_cast<uint32_t>(sv[k0 * pitch + d]) |
                   (static_cast<uint32_t>(sv[k1 * pitch + d]) << 16);
        }
        return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }
    __device__ __forceinline__ static f32x4 mma_pv(QK a, QK b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static float to_f32(uint16_t x) {
        return __uint_as_float(static_cast<uint32_t>(x) << 16);
    }
    __device__ __forceinline__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};

// f32: MFMA 16x16x4.  A lane holds head_dim run d = h*(D/4) .. +D/4-1 and uses
// element s of it at step s; the contraction covers every d exactly once.
template <int D> struct Frag<float, D> {
    static constexpr int kSteps = D / 4;
    struct QK {
        float v[D / 4];
    };
    __device__ __forceinline__ static QK qk_all(const float *row, int lane) {
        QK q;
        const float *p = row + (lane >> 4) * (D / 4);
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
            u32x4 w = *reinterpret_cast<const u32x4 *>(p + 4 * k);
            q.v[4 * k + 0] = __uint_as_float(w.x);
            q.v[4 * k + 1] = __uint_as_float(w.y);
            q.v[4 * k + 2] = __uint_as_float(w.z);
            q.v[4 * k + 3] = __uint_as_float(w.w);
        }
        return q;
    }
    __device__ __forceinline__ static QK zero() {
        QK q;
#pragma unroll
        for (int k = 0; k < D / 4; ++k) q.v[k] = 0.f;
        return q;
    }
    __device__ __forceinline__ static float to_f32(float x) { return x; }
    __device__ __forceinline__ static float from_f32(float x) { return x; }
};

// ---------------------------------------------------------------------------
// attn_ctx_split
// ---------------------------------------------------------------------------

// LDS: per wave a V tile of 32 keys (pitch D + 8 elements); after the key
// loop the same memory holds the per-wave (m, l, O) for the merge.
template <typename T, int D>
constexpr int ctx_lds_bytes() {
    constexpr int vt = kAttnWaves * kKeyTile * (D + 8) * static_cast<int>(sizeof(T));
    constexpr int mg = kAttnWaves * kRowsPerGroup * (D + 2) * 4;
    return vt > mg ? vt : mg;
}

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_ctx_split(
    const T *__restrict__ q, const T *__restrict__ k_ctx, const T *__restrict__ v_ctx,
    const int64_t *__restrict__ ctx_offsets, const int32_t *__restrict__ n_nodes, int batch,
    int nq_max, int hq, int hkv, int group, int n_rg, int chunk, int64_t n_chunks, float scale2,
    void *ws, int64_t items) {
    using F = Frag<T, D>;
    constexpr int kPitch = D + 8;
    __shared__ __attribute__((aligned(16))) char lds[ctx_lds_bytes<T, D>()];

    const int64_t item = blockIdx.x;
    const int rg = static_cast<int>(item % n_rg);
    const int g = static_cast<int>((item / n_rg) % hkv);
    const int64_t c = item / (static_cast<int64_t>(n_rg) * hkv);
    int b;
    int64_t k0, k1;
    if (!find_chunk(ctx_offsets, batch, chunk, c, b, k0, k1)) return;
    // rows of this sequence; n_nodes beyond nq_max - 1 is clamped (bad input)
    const int rows_b = group * min(n_nodes[b] + 1, nq_max);
    if (rg * kRowsPerGroup >= rows_b) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;  // this lane's query row within the group (C/B layout)
    const int h4 = lane >> 4;

    // query row of this lane
    const int r = rg * kRowsPerGroup + col;
    const bool row_ok = r < rows_b;
    const int qi = row_ok ? r / group : 0;
    const int qh = g * group + (row_ok ? r % group : 0);
    const T *qrow = q + ((static_cast<int64_t>(b) * nq_max + qi) * hq + qh) * D;

    const int64_t ctx0 = ctx_offsets[b];
    const int64_t kstride = static_cast<int64_t>(hkv) * D;  // elements between keys
    const T *kbase = k_ctx + (ctx0 * hkv + g) * D;
    const T *vbase = v_ctx + (ctx0 * hkv + g) * D;
    T *sv = reinterpret_cast<T *>(lds) + wave * kKeyTile * kPitch;

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nkeys = k1 - k0;
    const int ntiles = static_cast<int>((nkeys + kKeyTile - 1) / kKeyTile);

    if constexpr (sizeof(T) == 2) {
        typename F::QK qf[F::kSteps];
#pragma unroll
        for (int s = 0; s < F::kSteps; ++s) qf[s] = row_ok ? F::qk_operand(qrow, s, lane) : F::zero();

        for (int t = wave; t < ntiles; t += kAttnWaves) {
            const int64_t t0 = k0 + static_cast<int64_t>(t) * kKeyTile;
            const int valid = static_cast<int>(std::min<int64_t>(kKeyTile, k1 - t0));
            // K operands for both 16-key halves (key index clamped in range)
            typename F::QK kf[2][F::kSteps];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int kk = std::min(16 * hf + col, valid - 1);
                const T *krow = kbase + (t0 + kk) * kstride;
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s) kf[hf][s] = F::qk_operand(krow, s, lane);
            }
            // V tile -> LDS (key-major), 16-byte pieces, clamped keys
            constexpr int kPieces = kKeyTile * D / 8;
#pragma unroll
            for (int p0 = 0; p0 < kPieces; p0 += 64) {
                const int p = p0 + lane;
                const int key = p / (D / 8);
                const int db = p % (D / 8);
                const int kk = std::min(key, valid - 1);
                u32x4 w = *reinterpret_cast<const u32x4 *>(vbase + (t0 + kk) * kstride + db * 8);
                *reinterpret_cast<u32x4 *>(sv + key * kPitch + db * 8) = w;
            }
            // S^T = K Q^T
            f32x4 st[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s) acc = F::mma_qk(kf[hf][s], qf[s], acc);
                st[hf] = acc;
            }
            // this lane's 8 scores in slot order; keys beyond the chunk -> -inf
            float sc[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const int key = tt < 4 ? 4 * h4 + tt : 16 + 4 * h4 + (tt - 4);
                const float v = (tt < 4 ? st[0][tt] : st[1][tt - 4]) * scale2;
                sc[tt] = key < valid ? v : -INFINITY;
            }
            float tmax = sc[0];
#pragma unroll
            for (int tt = 1; tt < 8; ++tt) tmax = fmaxf(tmax, sc[tt]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float p[8];
            float ps = 0.f;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                p[tt] = __builtin_amdgcn_exp2f(sc[tt] - m_new);
                ps += p[tt];
            }
            l_run = l_run * alpha + ps;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            const typename F::QK pf = F::p_operand(p);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                o[dt] = F::mma_pv(F::v_operand(sv, kPitch, dt, lane), pf, o[dt]);
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        // f32 inputs: MFMA 16x16x4
        const typename F::QK qa = row_ok ? F::qk_all(qrow, lane) : F::zero();
        for (int t = wave; t < ntiles; t += kAttnWaves) {
            const int64_t t0 = k0 + static_cast<int64_t>(t) * kKeyTile;
            const int valid = static_cast<int>(std::min<int64_t>(kKeyTile, k1 - t0));
            f32x4 st[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int kk = std::min(16 * hf + col, valid - 1);
                const typename F::QK ka = F::qk_all(kbase + (t0 + kk) * kstride, lane);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.v[s], qa.v[s], acc, 0, 0, 0);
                st[hf] = acc;
            }
            constexpr int kPieces = kKeyTile * D / 4;
#pragma unroll
            for (int p0 = 0; p0 < kPieces; p0 += 64) {
                const int pp = p0 + lane;
                const int key = pp / (D / 4);
                const int db = pp % (D / 4);
                const int kk = std::min(key, valid - 1);
                u32x4 w = *reinterpret_cast<const u32x4 *>(vbase + (t0 + kk) * kstride + db * 4);
                *reinterpret_cast<u32x4 *>(sv + key * kPitch + db * 4) = w;
            }
            float sc[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const int key = tt < 4 ? 4 * h4 + tt : 16 + 4 * h4 + (tt - 4);
                const float v = (tt < 4 ? st[0][tt] : st[1][tt - 4]) * scale2;
                sc[tt] = key < valid ? v : -INFINITY;
            }
            float tmax = sc[0];
#pragma unroll
            for (int tt = 1; tt < 8; ++tt) tmax = fmaxf(tmax, sc[tt]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float p[8];
            float ps = 0.f;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                p[tt] = __builtin_amdgcn_exp2f(sc[tt] - m_new);
                ps += p[tt];
            }
            l_run = l_run * alpha + ps;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            // O^T += V^T P^T, 8 steps of 4 keys; step u uses key
            // u<4 -> 4h+u, u>=4 -> 16+4h+u-4 (this lane's p[u])
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const int d = 16 * dt + col;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int key = u < 4 ? 4 * h4 + u : 16 + 4 * h4 + (u - 4);
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sv[key * kPitch + d], p[u], o[dt],
                                                                 0, 0, 0);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }

    // l: sum of the four key-slices of this row
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);

    // ---- merge the 4 waves through LDS ----
    __syncthreads();  // V tiles are dead
    float *sm = reinterpret_cast<float *>(lds);
    float *mw = sm;                                          // [4][16]
    float *lw = mw + kAttnWaves * kRowsPerGroup;             // [4][16]
    float *ow = lw + kAttnWaves * kRowsPerGroup;             // [4][16][D]
    if (h4 == 0) {
        mw[wave * kRowsPerGroup + col] = m_run;
        lw[wave * kRowsPerGroup + col] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            ow[(wave * kRowsPerGroup + col) * D + 16 * dt + 4 * h4 + k] = o[dt][k];
    __syncthreads();

    AttnWs w = attn_ws(ws, items, D);
    const int row = tid >> 4;           // 0..15
    const int dsub = (tid & 15) * (D / 16);
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kAttnWaves; ++wv) M = fmaxf(M, mw[wv * kRowsPerGroup + row]);
    float L = 0.f;
    float acc[D / 16];
#pragma unroll
    for (int k = 0; k < D / 16; ++k) acc[k] = 0.f;
#pragma unroll
    for (int wv = 0; wv < kAttnWaves; ++wv) {
        const float mv = mw[wv * kRowsPerGroup + row];
        const float f = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        L += f * lw[wv * kRowsPerGroup + row];
#pragma unroll
        for (int k = 0; k < D / 16; ++k) acc[k] += f * ow[(wv * kRowsPerGroup + row) * D + dsub + k];
    }
    const int64_t prow = item * kRowsPerGroup + row;
    if ((tid & 15) == 0) {
        w.m[prow] = M;
        w.l[prow] = L;
    }
#pragma unroll
    for (int k = 0; k < D / 16; ++k) w.o[prow * D + dsub + k] = acc[k];
}

// ---------------------------------------------------------------------------
// attn_tree_combine
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_tree_combine(
    const T *__restrict__ q, const int64_t *__restrict__ ctx_offsets, const T *__restrict__ k_tree,
    const T *__restrict__ v_tree, const uint64_t *__restrict__ mask,
    const int32_t *__restrict__ n_nodes, int batch, int nq_max, int hq, int hkv, int group,
    int n_rg, int chunk, float scale2, const void *ws, int64_t items, T *__restrict__ out) {
    using F = Frag<T, D>;
    constexpr int kPer = D / 16;  // output dims per thread
    const int rg = blockIdx.x % n_rg;
    const int g = (blockIdx.x / n_rg) % hkv;
    const int b = blockIdx.x / (n_rg * hkv);
    const int tid = threadIdx.x;
    const int row = tid >> 4;
    const int dsub = (tid & 15) * kPer;
    const int r = rg * kRowsPerGroup + row;
    const int i = r / group;
    const int hh = r % group;
    if (i >= nq_max) return;
    const int h = g * group + hh;
    T *orow = out + ((static_cast<int64_t>(b) * nq_max + i) * hq + h) * D + dsub;
    const int n = min(n_nodes[b], nq_max - 1);
    if (i > n) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) orow[k] = F::from_f32(0.f);
        return;
    }

    // context partials of this row
    AttnWs w = attn_ws(const_cast<void *>(ws), items, D);
    const int64_t L = ctx_offsets[b + 1] - ctx_offsets[b];
    const int64_t nch = (L + chunk - 1) / chunk;
    const int64_t cb = chunk_base(ctx_offsets, b, chunk);
    float M = -INFINITY, Lsum = 0.f;
    float acc[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
    for (int64_t c = cb; c < cb + nch; ++c) {
        const int64_t item = (c * hkv + g) * n_rg + rg;
        const int64_t prow = item * kRowsPerGroup + row;
        const float mc = w.m[prow];
        const float Mn = fmaxf(M, mc);
        const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        const float fn = __builtin_amdgcn_exp2f(mc - Mn);
        Lsum = Lsum * fo + w.l[prow] * fn;
#pragma unroll
        for (int k = 0; k < kPer; ++k) acc[k] = acc[k] * fo + w.o[prow * D + dsub + k] * fn;
        M = Mn;
    }

    // tree keys on the root path of i (mask row), one dot product per bit
    const T *qrow = q + ((static_cast<int64_t>(b) * nq_max + i) * hq + h) * D + dsub;
    float qv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) qv[k] = F::to_f32(qrow[k]);
    const int words = (nq_max + 63) / 64;
    const uint64_t *mrow = mask + (static_cast<int64_t>(b) * nq_max + i) * words;
    for (int wd = 0; wd < words; ++wd) {
        uint64_t bits = mrow[wd];
        while (bits) {
            const int j = wd * 64 + __ffsll(static_cast<long long>(bits)) - 1;
            bits &= bits - 1;
            if (j >= nq_max) break;  // bits beyond the tree rows are ignored
            const int64_t kv = ((static_cast<int64_t>(b) * nq_max + j) * hkv + g) * D + dsub;
            float dot = 0.f;
#pragma unroll
            for (int k = 0; k < kPer; ++k) dot += qv[k] * F::to_f32(k_tree[kv + k]);
            // reduce over the 16 threads of this row
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            dot += __shfl_xor(dot, 4, 64);
            dot += __shfl_xor(dot, 8, 64);
            const float s = dot * scale2;
            const float Mn = fmaxf(M, s);
            const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
            const float fn = __builtin_amdgcn_exp2f(s - Mn);
            Lsum = Lsum * fo + fn;
#pragma unroll
            for (int k = 0; k < kPer; ++k) acc[k] = acc[k] * fo + F::to_f32(v_tree[kv + k]) * fn;
            M = Mn;
        }
    }
    const float inv = 1.f / Lsum;
#pragma unroll
    for (int k = 0; k < kPer; ++k) orow[k] = F::from_f32(acc[k] * inv);
}

template <typename T, int D>
void launch_attn(const void *q, const void *k_ctx, const void *v_ctx, const int64_t *off,
                 const void *k_tree, const void *v_tree, const uint64_t *mask,
                 const int32_t *n_nodes, int batch, int nq_max, int hq, int hkv, float scale,
                 const AttnPlan &pl, void *ws, void *out, hipStream_t st) {
    const float scale2 = scale * kLog2e;
    if (pl.items > 0)
        hipLaunchKernelGGL((attn_ctx_split<T, D>), dim3(static_cast<unsigned>(pl.items)),
                           dim3(kAttnThreads), 0, st, static_cast<const T *>(q),
                           static_cast<const T *>(k_ctx), static_cast<const T *>(v_ctx), off, n_nodes,
                           batch, nq_max, hq, hkv, pl.group, pl.n_rg, pl.chunk, pl.n_chunks, scale2,
                           ws, pl.items);
    hipLaunchKernelGGL((attn_tree_combine<T, D>),
                       dim3(static_cast<unsigned>(batch * hkv * pl.n_rg)), dim3(kAttnThreads), 0,
                       st, static_cast<const T *>(q), off, static_cast<const T *>(k_tree),
                       static_cast<const T *>(v_tree), mask, n_nodes, batch, nq_max, hq, hkv,
                       pl.group, pl.n_rg, pl.chunk, scale2, ws, pl.items, static_cast<T *>(out));
}

}  // namespace
}  // namespace td

using namespace td;

extern "C" size_t td_tree_verify_attn_workspace(int32_t batch, int32_t nq_max, int32_t hq,
                                                int32_t hkv, int32_t head_dim, int64_t total_ctx,
                                                int64_t max_ctx) {
    (void)max_ctx;
    if (batch <= 0 || nq_max <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || head_dim <= 0 ||
        total_ctx < 0)
        return 0;
    AttnPlan pl = attn_plan(batch, nq_max, hq, hkv, total_ctx);
    return std::max<size_t>(16, attn_ws_bytes(pl, head_dim));
}

extern "C" td_status td_tree_verify_attn(const void *q, const void *k_ctx, const void *v_ctx,
                                         const int64_t *ctx_offsets, int64_t total_ctx,
                                         int64_t max_ctx, const void *k_tree, const void *v_tree,
                                         const uint64_t *mask, const int32_t *n_nodes,
                                         int32_t batch, int32_t nq_max, int32_t hq, int32_t hkv,
                                         int32_t head_dim, float scale, td_dtype dtype, void *out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (!q || !k_tree || !v_tree || !ctx_offsets || !mask || !n_nodes || !out || !workspace)
        return fail(TD_EINVAL, "td_tree_verify_attn: null pointer argument");
    if (total_ctx > 0 && (!k_ctx || !v_ctx))
        return fail(TD_EINVAL, "td_tree_verify_attn: null context K/V with total_ctx > 0");
    if (batch <= 0 || nq_max <= 0 || hq <= 0 || hkv <= 0 || total_ctx < 0 || max_ctx < 0)
        return fail(TD_EINVAL, "td_tree_verify_attn: sizes must be positive");
    if (hq % hkv != 0) return fail(TD_EINVAL, "td_tree_verify_attn: hq must be a multiple of hkv");
    if (nq_max > TD_MAX_NODES + 1 || batch > TD_MAX_BATCH)
        return fail(TD_ECAPACITY, "td_tree_verify_attn: nq_max or batch above capacity");
    if (dtype != TD_F32 && dtype != TD_BF16)
        return fail(TD_EUNSUPPORTED, "td_tree_verify_attn: dtype must be TD_F32 or TD_BF16");
    if (head_dim != 64 && head_dim != 128)
        return fail(TD_EUNSUPPORTED, "td_tree_verify_attn: head_dim must be 64 or 128");
    if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
        !aligned16(workspace) || (k_ctx && !aligned16(k_ctx)) || (v_ctx && !aligned16(v_ctx)) ||
        !aligned8(mask) || !aligned8(ctx_offsets))
        return fail(TD_EINVAL, "td_tree_verify_attn: buffers must be 16-byte aligned");
    if (workspace_bytes <
        td_tree_verify_attn_workspace(batch, nq_max, hq, hkv, head_dim, total_ctx, max_ctx))
        return fail(TD_EINVAL, "td_tree_verify_attn: workspace too small");
    AttnPlan pl = attn_plan(batch, nq_max, hq, hkv, total_ctx);
    if (pl.items > 0x7fffffffLL || static_cast<int64_t>(batch) * hkv * pl.n_rg > 0x7fffffffLL)
        return fail(TD_ECAPACITY, "td_tree_verify_attn: grid too large");
    if (total_ctx == 0) pl.items = 0;
    hipStream_t st = as_stream(stream);
    const bool bf = dtype == TD_BF16;
#define TD_ATTN(T, DD)                                                                          \
    launch_attn<T, DD>(q, k_ctx, v_ctx, ctx_offsets, k_tree, v_tree, mask, n_nodes, batch,     \
                       nq_max, hq, hkv, scale, pl, workspace, out, st)
    if (bf && head_dim == 128)
        TD_ATTN(uint16_t, 128);
    else if (bf)
        TD_ATTN(uint16_t, 64);
    else if (head_dim == 128)
        TD_ATTN(float, 128);
    else
        TD_ATTN(float, 64);
#undef TD_ATTN
    return check_launch("td_tree_verify_attn");
}
