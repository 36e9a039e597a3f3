// A one-layer stand-in for the target's verification pass over the draft
// tree (BASTION: the target scores every tree node in one parallel pass;
// acceptance compares its greedy token at each node, temperature 0):
//
//   td_tree_qkv        the tree tokens' embedding rows times the Q/K/V
//                      projection, rotary position embedding at position
//                      (context length + depth), bf16 q / k_tree / v_tree in
//                      the layouts td_tree_verify_attn reads;
//   td_lm_head_argmax  the argmax over the vocabulary of each tree row's
//                      hidden state (the attention output of all query
//                      heads) times the LM head: the target's greedy token.
//
// Both products have few rows (the tree rows of a step) against a long
// weight matrix, so they stream the weights from HBM once.  One kernel,
// gemm_rows, computes C[m][n] = sum_k A[m][k] W[n][k] (both operands
// k-contiguous bf16, float32 accumulation, v_mfma_f32_16x16x32_bf16):
//  - a workgroup (4 waves) owns 128 columns and up to 80 rows (RM row
//    groups of 16); a wave owns 32 columns (two 16-column blocks) of every
//    row group;
//  - the A rows (gathered by token id for the embedding) go through LDS in
//    chunks of 128 k, two buffers, with direct global-to-LDS loads; each row
//    of a chunk is padded by one 16-byte piece so the 16 rows of a fragment
//    read fall in distinct banks;
//  - each wave streams its own W columns into registers one chunk ahead
//    (W is read exactly once per row tile);
//  - the epilogue either stores float32 partial sums of one k slice (the
//    projection, split over k so that a 6144-column product fills the chip)
//    or keeps, per row, the best (value, column) of the tile (the LM head:
//    the logits never reach memory).
// Two small kernels finish: the projection's k slices summed in a fixed
// order, rotated and rounded to bf16; the LM head's tile winners reduced to
// one token per row (ties to the smaller id).

#include <algorithm>
#include <climits>

#include "step_launch.h"
#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGT = 256;                 // threads per workgroup
constexpr int kGW = kGT / kWave;         // waves
constexpr int kCB = 2;                   // 16-column blocks per wave
constexpr int kBN = kGW * kCB * 16;      // columns per workgroup
constexpr int kKC = 128;                 // k per LDS chunk
constexpr int kPc = kKC / 8 + 1;         // 16-byte pieces per LDS row (one pad)
constexpr int kMaxRM = 5;                // row groups of 16 per workgroup

template <int RM> constexpr int a_rounds() { return (16 * RM * kPc + kGT - 1) / kGT; }

__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}

// A compiler barrier: no memory operation is moved across it (the hardware
// is not affected).
__device__ __forceinline__ void pin_order() { asm volatile("" ::: "memory"); }

// Wait until at most N of this wave's vector-memory loads are outstanding
// (the N most recent); LDS and export counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void *)p));
}

// The A operand: problem row m is row index[m] of base (index null: row m);
// an index outside [0, n_rows) reads row 0.
struct RowsA {
    const uint16_t *base;
    int64_t ld;
    const int32_t *index;
    int n_rows;
};

__device__ __forceinline__ const uint16_t *row_ptr(const RowsA &a, int m) {
    int r = a.index ? a.index[m] : m;
    if (r < 0 || r >= a.n_rows) r = 0;
    return a.base + static_cast<int64_t>(r) * a.ld;
}

// A fragments of one 32-k step for RM row groups (lane l: row 16 rb + l%16,
// k 8 (l/16) ..), all reads in flight before one wait.  Issued from
// assembly: the compiler would otherwise wait for the other buffer's direct
// loads before every LDS read.
template <int RM>
__device__ __forceinline__ void read_a(uint32_t addr, bf16x8 (&af)[RM]) {
    constexpr int S = 16 * kPc * 16;  // bytes between row groups
    u32x4 t[RM];
    if constexpr (RM == 1) {
        asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=&v"(t[0]) : "v"(addr));
    } else if constexpr (RM == 2) {
        asm volatile("ds_read_b128 %0, %2\n ds_read_b128 %1, %2 offset:%3\n s_waitcnt lgkmcnt(0)"
                     : "=&v"(t[0]), "=&v"(t[1]) : "v"(addr), "i"(S));
    } else if constexpr (RM == 3) {
        asm volatile("ds_read_b128 %0, %3\n ds_read_b128 %1, %3 offset:%4\n"
                     " ds_read_b128 %2, %3 offset:%5\n s_waitcnt lgkmcnt(0)"
                     : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]) : "v"(addr), "i"(S), "i"(2 * S));
    } else if constexpr (RM == 4) {
        asm volatile("ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:%5\n"
                     " ds_read_b128 %2, %4 offset:%6\n ds_read_b128 %3, %4 offset:%7\n"
                     " s_waitcnt lgkmcnt(0)"
                     : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
                     : "v"(addr), "i"(S), "i"(2 * S), "i"(3 * S));
    } else {
        static_assert(RM == 5, "row groups");
        asm volatile("ds_read_b128 %0, %5\n ds_read_b128 %1, %5 offset:%6\n"
                     " ds_read_b128 %2, %5 offset:%7\n ds_read_b128 %3, %5 offset:%8\n"
                     " ds_read_b128 %4, %5 offset:%9\n s_waitcnt lgkmcnt(0)"
                     : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4])
                     : "v"(addr), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S));
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) af[r] = __builtin_bit_cast(bf16x8, t[r]);
}

// MODE 0: float32 partial sums of k slice z = blockIdx.y into
//         part[(z * M + m) * N + n];
// MODE 1: per row m, the best (value, column) of this workgroup's columns
//         into best[m * col_tiles + column tile] (value bits, column).
// Requires K_slice a multiple of kKC and 16-byte aligned rows.
// Workgroup order: the chip hands consecutive workgroups to its 8 XCDs in
// turn, each XCD with its own L2.  The row tiles of one column tile read the
// same weight columns, so they are given ids that differ by multiples of 8
// (one XCD, one L2): ids run over (group of 8 column tiles, row tile, column
// tile within the group).
constexpr int kXcds = 8;
struct TileId {
    int col, row;
};
__device__ __forceinline__ TileId tile_of(int id, int row_tiles, int col_tiles) {
    const int per_group = kXcds * row_tiles;
    const int g = id / per_group;
    const int rest = id - g * per_group;
    const int first = g * kXcds;
    const int width = min(kXcds, col_tiles - first);  // the last group may be narrower
    return {first + rest % width, rest / width};
}

template <int RM, int MODE>
__global__ __launch_bounds__(kGT) void gemm_rows(RowsA a, const uint16_t *w, int M,
                                                 int N, int K, int k_slice, int row_tiles,
                                                 int col_tiles, float *__restrict__ part,
                                                 int2 *__restrict__ best) {
    constexpr int BM = 16 * RM;
    constexpr int R = a_rounds<RM>();
    __shared__ __attribute__((aligned(16))) uint16_t sa0[R * kGT * 8];
    __shared__ __attribute__((aligned(16))) uint16_t sa1[R * kGT * 8];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const TileId tl = tile_of(blockIdx.x, row_tiles, col_tiles);
    const int m0 = tl.row * BM;
    const int k0 = blockIdx.y * k_slice;
    const int n_chunks = k_slice / kKC;

    // direct loads of the A rows: slot s = r 256 + tid holds (row s / kPc,
    // piece s % kPc); pad pieces and rows past M load copies
    const uint16_t *src[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * kGT + tid;
        const int row = min(s / kPc, BM - 1);
        const int piece = min(s % kPc, kPc - 2);
        src[r] = row_ptr(a, min(m0 + row, M - 1)) + k0 + 8 * piece;
    }
    auto issue = [&](int c, uint16_t *buf) {
#pragma unroll
        for (int r = 0; r < R; ++r) dma16(src[r] + c * kKC, buf + 8 * ((r * kGW + wave) * kWave));
    };

    // this wave's W columns (clamped; columns past N are dropped later)
    const int col0 = tl.col * kBN + wave * (kCB * 16) + (lane & 15);
    const uint16_t *wrow[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
        wrow[cb] = w + static_cast<int64_t>(min(col0 + 16 * cb, N - 1)) * K + k0 + 8 * (lane >> 4);
    auto load_w = [&](int c, u32x4 (&dst)[4][kCB]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb)
                dst[ks][cb] = *reinterpret_cast<const u32x4 *>(wrow[cb] + c * kKC + ks * 32);
    };

    f32x4 acc[RM][kCB];
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) acc[r][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t a_off = ((lane & 15) * kPc + (lane >> 4)) * 16;  // bytes, row group 0
    auto compute = [&](const uint16_t *buf, const u32x4 (&wb)[4][kCB]) {
        const uint32_t base = lds_addr(buf) + a_off;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 af[RM];
            read_a<RM>(base + ks * 64, af);
#pragma unroll
            for (int r = 0; r < RM; ++r)
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb)
                    acc[r][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[r], __builtin_bit_cast(bf16x8, wb[ks][cb]), acc[r][cb], 0, 0, 0);
        }
    };

    // Chunk c: A rows in LDS buffer c % 2 (one chunk ahead: the rows are
    // few and stay in L2), this wave's W columns in register buffer c % 3
    // (two chunks ahead: W streams from HBM, and its loads in flight set the
    // rate).  Issue order: A(0) W(0) A(1) W(1) W(2), then after chunk c
    // A(c + 2) W(c + 3); so when chunk c is waited for, the loads issued
    // after its last one are exactly W(c + 1), A(c + 1) and W(c + 2): R
    // direct A loads and 2 kWL W loads.  Every load is issued (chunks past
    // the last repeat the last one), so that count never changes and the
    // compiler's own waits for the W registers stay exact too.
    u32x4 w0[4][kCB], w1[4][kCB], w2[4][kCB];
    constexpr int kWL = 4 * kCB;  // W loads per chunk and lane
    const int last = n_chunks - 1;
    issue(0, sa0);
    pin_order();
    load_w(0, w0);
    pin_order();
    issue(min(1, last), sa1);
    pin_order();
    load_w(min(1, last), w1);
    load_w(min(2, last), w2);
    // The barriers below are plain s_barrier: a __syncthreads() fence would
    // wait for every load in flight (the direct LDS loads share the vector
    // memory counter), W prefetches included.  The waits they need are
    // explicit: each wave waits for its own direct loads of a chunk before
    // the barrier that publishes it, and the A fragment reads wait for their
    // data before the barrier that frees their buffer.
    // The wait counts assume the program order of the loads: compiler
    // barriers (pin_order) keep every load between the same waits and
    // barriers, and the A loads of a chunk before the W loads that follow
    // (w is not declared __restrict__: loads through a restricted read-only
    // pointer count as invariant, and a compiler barrier would not hold them).
    auto arrive = [&](int) __attribute__((always_inline)) {
        pin_order();
        wait_vm<kWL + R + kWL>();
        __builtin_amdgcn_s_barrier();  // everyone's A rows of chunk c have landed
        pin_order();
    };
    auto refill = [&](int c, uint16_t *buf, u32x4 (&wb)[4][kCB]) __attribute__((always_inline)) {
        pin_order();
        __builtin_amdgcn_s_barrier();  // everyone is done with chunk c's A buffer
        pin_order();
        issue(min(c + 2, last), buf);
        pin_order();
        load_w(min(c + 3, last), wb);
        pin_order();
    };
    auto step = [&](int c, u32x4 (&wb)[4][kCB]) __attribute__((always_inline)) {
        uint16_t *const buf = (c & 1) ? sa1 : sa0;
        arrive(c);
        compute(buf, wb);
        refill(c, buf, wb);
    };
    // The first three chunks run before the loop, so that the loop is
    // entered in the state it repeats (the compiler's own waits for the W
    // registers are then exact instead of a full wait per trip).
    step(0, w0);
    if (n_chunks > 1) step(1, w1);
    if (n_chunks > 2) step(2, w2);
    for (int c = 3; c < n_chunks; c += 3) {
        step(c, w0);
        if (c + 1 >= n_chunks) break;
        step(c + 1, w1);
        if (c + 2 >= n_chunks) break;
        step(c + 2, w2);
    }
    __builtin_amdgcn_s_waitcnt(0);

    // C fragment: lane l holds column l % 16, rows 4 (l / 16) + i
    if constexpr (MODE == 0) {
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) {
                const int n = col0 + 16 * cb;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * r + 4 * (lane >> 4) + i;
                    if (m < M && n < N)
                        part[(static_cast<int64_t>(blockIdx.y) * M + m) * N + n] = acc[r][cb][i];
                }
            }
    } else {
        __shared__ float s_val[kGW][BM];
        __shared__ int s_col[kGW][BM];
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = -INFINITY;
                int col = INT_MAX;
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb) {  // increasing columns: ties keep the first
                    const int n = col0 + 16 * cb;
                    const float x = acc[r][cb][i];
                    if (n < N && x > v) {
                        v = x;
                        col = n;
                    }
                }
                // the 16 lanes of a row share rows 4 (l / 16) + i: levels 0..3
#define TD_ARGMAX_LEVEL(L)                                                    \
                {                                                             \
                    const float ov = xchg_f<L>(v);                            \
                    const int oc = xchg_i<L>(col);                            \
                    if (ov > v || (ov == v && oc < col)) {                    \
                        v = ov;                                               \
                        col = oc;                                             \
                    }                                                         \
                }
                TD_ARGMAX_LEVEL(0)
                TD_ARGMAX_LEVEL(1)
                TD_ARGMAX_LEVEL(2)
                TD_ARGMAX_LEVEL(3)
#undef TD_ARGMAX_LEVEL
                if ((lane & 15) == 0) {
                    const int row = 16 * r + 4 * (lane >> 4) + i;
                    s_val[wave][row] = v;
                    s_col[wave][row] = col;
                }
            }
        __syncthreads();
        if (tid < BM && m0 + tid < M) {
            float v = s_val[0][tid];
            int col = s_col[0][tid];
#pragma unroll
            for (int q = 1; q < kGW; ++q) {  // waves own increasing columns
                if (s_val[q][tid] > v) {
                    v = s_val[q][tid];
                    col = s_col[q][tid];
                }
            }
            best[static_cast<int64_t>(m0 + tid) * col_tiles + tl.col] = int2{__float_as_int(v), col};
        }
    }
}

// Context length of sequence b (whole region, or the given length clamped).
__device__ __forceinline__ int64_t ctx_len_of(const int64_t *off, const int64_t *lens, int b) {
    const int64_t region = off[b + 1] - off[b];
    if (!lens) return region;
    const int64_t L = lens[b];
    return L < 0 ? 0 : (L > region ? region : L);
}

// Workgroup (m, y): problem row m = b nq + i, pairs 256 y .. 256 y + 255 of
// it, one per thread (all of a thread's loads in flight at once): the k
// slices summed in order,
// rotary embedding of the query and key heads at position L_b + depth(i)
// (rotate-half pairs (j, j + D/2), frequency base^(-2j/D), angle and its
// sine and cosine in float64), rounded to bf16; rows past the tree: zeros.
__global__ __launch_bounds__(256) void qkv_finish(const float *__restrict__ part, int splits,
                                                  int M, int N, const int32_t *__restrict__ depth,
                                                  const int32_t *__restrict__ n_nodes,
                                                  const int64_t *__restrict__ off,
                                                  const int64_t *__restrict__ lens, int nq, int hq,
                                                  int hkv, int D, double rope_base,
                                                  uint16_t *__restrict__ q,
                                                  uint16_t *__restrict__ k,
                                                  uint16_t *__restrict__ v) {
    const int m = blockIdx.x;
    const int b = m / nq;
    const int i = m - b * nq;
    const int e = blockIdx.y * blockDim.x + threadIdx.x;
    const bool in_tree = i <= n_nodes[b];
    const int dep = depth[m] < 0 ? 0 : depth[m];
    const double pos = static_cast<double>(ctx_len_of(off, lens, b) + dep);
    const int half = D / 2;
    const int pairs = (hq + 2 * hkv) * half;
    // the rotation of pair j is the same for every head of the row
    __shared__ float s_cos[64], s_sin[64];
    if (threadIdx.x < half) {
        const double ang = pos * exp2(-2.0 * threadIdx.x / D * log2(rope_base));
        double sn, cs;
        sincos(ang, &sn, &cs);
        s_cos[threadIdx.x] = static_cast<float>(cs);
        s_sin[threadIdx.x] = static_cast<float>(sn);
    }
    __syncthreads();
    if (e < pairs) {
        const int h = e / half;
        const int j = e - h * half;
        const int n1 = h * D + j;
        float x1 = 0.f, x2 = 0.f;
        for (int z = 0; z < splits; ++z) {
            const float *p = part + (static_cast<int64_t>(z) * M + m) * N;
            x1 += p[n1];
            x2 += p[n1 + half];
        }
        float y1 = x1, y2 = x2;
        if (h < hq + hkv) {
            const float cf = s_cos[j], sf = s_sin[j];
            y1 = x1 * cf - x2 * sf;
            y2 = x2 * cf + x1 * sf;
        }
        if (!in_tree) y1 = y2 = 0.f;
        uint16_t *dst;
        if (h < hq)
            dst = q + (static_cast<int64_t>(m) * hq + h) * D;
        else if (h < hq + hkv)
            dst = k + (static_cast<int64_t>(m) * hkv + (h - hq)) * D;
        else
            dst = v + (static_cast<int64_t>(m) * hkv + (h - hq - hkv)) * D;
        dst[j] = f32_to_bf16(y1);
        dst[j + half] = f32_to_bf16(y2);
    }
}

// One wave per problem row: the best of its column tiles (larger value,
// then smaller column); -1 for rows past the tree.
__global__ __launch_bounds__(256) void argmax_finish(const int2 *__restrict__ best, int n_tiles,
                                                     int M, int nq,
                                                     const int32_t *__restrict__ n_nodes,
                                                     int32_t *__restrict__ target) {
    const int m = blockIdx.x * (256 / kWave) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= M) return;
    float v = -INFINITY;
    int col = INT_MAX;
    for (int t = lane; t < n_tiles; t += kWave) {
        const int2 p = best[static_cast<int64_t>(m) * n_tiles + t];
        const float x = __int_as_float(p.x);
        if (x > v || (x == v && p.y < col)) {
            v = x;
            col = p.y;
        }
    }
#define TD_ARGMAX_LEVEL(L)                                        \
    {                                                             \
        const float ov = xchg_f<L>(v);                            \
        const int oc = xchg_i<L>(col);                            \
        if (ov > v || (ov == v && oc < col)) {                    \
            v = ov;                                               \
            col = oc;                                             \
        }                                                         \
    }
    TD_ARGMAX_LEVEL(0)
    TD_ARGMAX_LEVEL(1)
    TD_ARGMAX_LEVEL(2)
    TD_ARGMAX_LEVEL(3)
    TD_ARGMAX_LEVEL(4)
    TD_ARGMAX_LEVEL(5)
#undef TD_ARGMAX_LEVEL
    if (lane == 0) {
        const int b = m / nq;
        target[m] = (m - b * nq) <= n_nodes[b] ? col : -1;
    }
}

// Row groups per workgroup for M rows, and the row tiles.
inline int rows_rm(int M) { return std::min(kMaxRM, (M + 15) / 16); }
inline int row_tiles(int M) { return (M + 16 * rows_rm(M) - 1) / (16 * rows_rm(M)); }
inline int col_tiles(int N) { return (N + kBN - 1) / kBN; }

// k slices of the projection: the most (a power of two dividing the chunk
// count) that keep the grid at or under 512 workgroups.
inline int qkv_splits(int M, int N, int K) {
    const int chunks = K / kKC;
    const int tiles = col_tiles(N) * row_tiles(M);
    int s = 1;
    while (s * 2 <= chunks && chunks % (s * 2) == 0 && tiles * s * 2 <= 512) s *= 2;
    return s;
}

template <int MODE>
void launch_gemm(const RowsA &a, const uint16_t *w, int M, int N, int K, int splits, float *part,
                 int2 *best, hipStream_t st) {
    const int rt = row_tiles(M), ct = col_tiles(N);
    const dim3 grid(rt * ct, splits);
    const int k_slice = K / splits;
#define TD_GEMM(RM) \
    TD_LAUNCH((gemm_rows<RM, MODE>), grid, dim3(kGT), 0, st, a, w, M, N, K, k_slice, rt, ct, part, best)
    switch (rows_rm(M)) {
    case 1: TD_GEMM(1); break;
    case 2: TD_GEMM(2); break;
    case 3: TD_GEMM(3); break;
    case 4: TD_GEMM(4); break;
    default: TD_GEMM(5); break;
    }
#undef TD_GEMM
}

size_t qkv_ws(int M, int N, int K) {
    return static_cast<size_t>(qkv_splits(M, N, K)) * M * N * sizeof(float);
}
size_t lm_ws(int M, int vocab) { return static_cast<size_t>(M) * col_tiles(vocab) * sizeof(int2); }

}  // namespace
}  // namespace td

using namespace td;

extern "C" size_t td_verify_layer_workspace(int32_t batch, int32_t nq_max, int32_t hq, int32_t hkv,
                                            int32_t head_dim, int32_t vocab) {
    if (batch <= 0 || nq_max <= 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || vocab <= 0) return 0;
    const int M = batch * nq_max;
    const int H = hq * head_dim;
    const int N = (hq + 2 * hkv) * head_dim;
    if (H % kKC) return 0;
    return std::max<size_t>(16, std::max(qkv_ws(M, N, H), lm_ws(M, vocab)));
}

namespace {
td_status check_layer(const char *who, int32_t batch, int32_t nq_max, int32_t hq, int32_t hkv,
                      int32_t head_dim, int32_t vocab, void *workspace, size_t workspace_bytes,
                      size_t need) {
    if (batch <= 0 || nq_max <= 0 || hq <= 0 || hkv <= 0 || vocab <= 0)
        return fail(TD_EINVAL, "verify layer: sizes must be positive");
    if (hq % hkv) return fail(TD_EINVAL, "verify layer: hq must be a multiple of hkv");
    if (head_dim != 64 && head_dim != 128)
        return fail(TD_EUNSUPPORTED, "verify layer: head_dim must be 64 or 128");
    if ((hq * head_dim) % kKC)
        return fail(TD_EUNSUPPORTED, "verify layer: hidden = hq * head_dim must be a multiple of 128");
    if (batch > TD_MAX_BATCH || nq_max > TD_MAX_NODES + 1)
        return fail(TD_ECAPACITY, "verify layer: batch or nq_max above capacity");
    if (static_cast<int64_t>(batch) * nq_max * std::max(vocab, (hq + 2 * hkv) * head_dim) >
        (int64_t(1) << 40))
        return fail(TD_ECAPACITY, "verify layer: problem too large");
    if (!workspace || !aligned16(workspace))
        return fail(TD_EINVAL, "verify layer: null or misaligned workspace");
    if (workspace_bytes < need) {
        set_error("%s: workspace too small", who);
        return TD_EINVAL;
    }
    return TD_OK;
}
}  // namespace

extern "C" td_status td_tree_qkv(const void *embed, const void *w_qkv, const int32_t *node_token,
                                 const int32_t *node_depth, const int32_t *n_nodes,
                                 const int64_t *ctx_offsets, const int64_t *ctx_lengths,
                                 int32_t batch, int32_t nq_max, int32_t vocab, int32_t hq,
                                 int32_t hkv, int32_t head_dim, double rope_base, void *q,
                                 void *k_tree, void *v_tree, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    clear_error();
    if (!embed || !w_qkv || !node_token || !node_depth || !n_nodes || !ctx_offsets || !q ||
        !k_tree || !v_tree)
        return fail(TD_EINVAL, "td_tree_qkv: null pointer argument");
    td_status st = check_layer("td_tree_qkv", batch, nq_max, hq, hkv, head_dim, vocab, workspace,
                               workspace_bytes,
                               qkv_ws(batch * nq_max, (hq + 2 * hkv) * head_dim, hq * head_dim));
    if (st != TD_OK) return st;
    if (!aligned16(embed) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k_tree) ||
        !aligned16(v_tree) || !aligned8(ctx_offsets) || (ctx_lengths && !aligned8(ctx_lengths)))
        return fail(TD_EINVAL, "td_tree_qkv: misaligned array");
    if (!(rope_base > 1.0)) return fail(TD_EINVAL, "td_tree_qkv: rope_base must exceed 1");
    const int M = batch * nq_max;
    const int H = hq * head_dim;
    const int N = (hq + 2 * hkv) * head_dim;
    const int splits = qkv_splits(M, N, H);
    hipStream_t s = as_stream(stream);
    float *part = static_cast<float *>(workspace);
    const RowsA a{static_cast<const uint16_t *>(embed), H, node_token, vocab};
    launch_gemm<0>(a, static_cast<const uint16_t *>(w_qkv), M, N, H, splits, part, nullptr, s);
    const int pairs = (hq + 2 * hkv) * head_dim / 2;
    TD_LAUNCH(qkv_finish, dim3(M, (pairs + 255) / 256), dim3(256), 0, s, part, splits, M, N, node_depth, n_nodes,
              ctx_offsets, ctx_lengths, nq_max, hq, hkv, head_dim, rope_base,
              static_cast<uint16_t *>(q), static_cast<uint16_t *>(k_tree),
              static_cast<uint16_t *>(v_tree));
    return check_launch("td_tree_qkv");
}

extern "C" td_status td_lm_head_argmax(const void *hidden_rows, const void *w_lm,
                                       const int32_t *n_nodes, int32_t batch, int32_t nq_max,
                                       int32_t hq, int32_t head_dim, int32_t vocab,
                                       int32_t *target_token, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    clear_error();
    if (!hidden_rows || !w_lm || !n_nodes || !target_token)
        return fail(TD_EINVAL, "td_lm_head_argmax: null pointer argument");
    td_status st = check_layer("td_lm_head_argmax", batch, nq_max, hq, hq, head_dim, vocab,
                               workspace, workspace_bytes, lm_ws(batch * nq_max, vocab));
    if (st != TD_OK) return st;
    if (!aligned16(hidden_rows) || !aligned16(w_lm))
        return fail(TD_EINVAL, "td_lm_head_argmax: misaligned array");
    const int M = batch * nq_max;
    const int H = hq * head_dim;
    hipStream_t s = as_stream(stream);
    int2 *best = static_cast<int2 *>(workspace);
    const RowsA a{static_cast<const uint16_t *>(hidden_rows), H, nullptr, M};
    launch_gemm<1>(a, static_cast<const uint16_t *>(w_lm), M, vocab, H, 1, nullptr, best, s);
    const int tiles = col_tiles(vocab);
    TD_LAUNCH(argmax_finish, dim3((M + 3) / 4), dim3(256), 0, s, best, tiles, M, nq_max, n_nodes,
              target_token);
    return check_launch("td_lm_head_argmax");
}
