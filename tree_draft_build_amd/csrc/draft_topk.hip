// Stage (a): per-position log-softmax normaliser and top-K over the full
// vocabulary (BASTION, "Methodik" §1: path scores are products of the
// drafter's per-position marginals q_k, so every q_k of a candidate is needed).
//
// Two kernels:
//   topk_partial  grid (splits, rows): each workgroup streams one contiguous
//                 slice of one vocabulary row with 16-byte loads, keeping a
//                 running max / float64 sum of exp per lane and a sorted
//                 register top-K per lane; the workgroup then merges its 256
//                 lanes into one (max, sum, top-K) partial.
//   topk_merge    grid (rows): one wavefront per row merges the row's
//                 partials: lse = M + log(sum_s s_s exp(m_s - M)) in float64,
//                 and a K-round tournament over the sorted partial lists.
// Order of candidates everywhere: larger logit first, then smaller token id.

#include <algorithm>

#include "td_internal.h"

namespace td {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

// (v, id) precedes (w, jd) in the selection order.
__device__ __forceinline__ bool before(float v, int id, float w, int jd) {
    return v > w || (v == w && id < jd);
}

// Sorted (descending) list of the KM best (value, id) pairs seen by a lane.
template <int KM>
struct LaneTop {
    float v[KM];
    int id[KM];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            v[j] = -INFINITY;
            id[j] = 0x7fffffff;
        }
    }
    // Insert (x, i) keeping the list sorted; the last entry falls off.
    __device__ __forceinline__ void insert(float x, int i) {
        float cv = x;
        int ci = i;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            bool sw = before(cv, ci, v[j], id[j]);
            float tv = sw ? v[j] : cv;
            int ti = sw ? id[j] : ci;
            v[j] = sw ? cv : v[j];
            id[j] = sw ? ci : id[j];
            cv = tv;
            ci = ti;
        }
    }
    // Remove the head (the list shifts up by one).
    __device__ __forceinline__ void pop_if(bool p) {
#pragma unroll
        for (int j = 0; j + 1 < KM; ++j) {
            v[j] = p ? v[j + 1] : v[j];
            id[j] = p ? id[j + 1] : id[j];
        }
        v[KM - 1] = p ? -INFINITY : v[KM - 1];
        id[KM - 1] = p ? 0x7fffffff : id[KM - 1];
    }
};

// Wave-wide best (value, id) of the lanes' heads.
__device__ __forceinline__ void wave_best(float &v, int &id) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float w = __shfl_xor(v, o, kWave);
        int jd = __shfl_xor(id, o, kWave);
        if (before(w, jd, v, id)) {
            v = w;
            id = jd;
        }
    }
}

// Workspace layout: for P = rows * splits partials
//   double s[P] | float m[P] | float v[P][K] | int id[P][K]   (each 16-byte aligned)
struct TopkWs {
    double *s;
    float *m;
    float *v;
    int *id;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

inline size_t topk_ws_bytes(int64_t parts, int K) {
    return align16(parts * 8) + align16(parts * 4) + align16(parts * K * 4) + align16(parts * K * 4);
}

__host__ __device__ inline TopkWs topk_ws(void *base, int64_t parts, int K) {
    char *p = static_cast<char *>(base);
    TopkWs w;
    w.s = reinterpret_cast<double *>(p);
    p += align16(parts * 8);
    w.m = reinterpret_cast<float *>(p);
    p += align16(parts * 4);
    w.v = reinterpret_cast<float *>(p);
    p += align16(parts * K * 4);
    w.id = reinterpret_cast<int *>(p);
    return w;
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

// Lane state: running max m, float64 sum s of exp(x - m), and the top list.
template <int KM>
struct LaneAcc {
    float m;
    double s;
    LaneTop<KM> top;

    template <int N>
    __device__ __forceinline__ void add(const float (&x)[N], int base_id) {
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
        if (vmax > top.v[KM - 1]) {
#pragma unroll
            for (int j = 0; j < N; ++j)
                if (x[j] > top.v[KM - 1]) top.insert(x[j], base_id + j);
        }
    }
};

template <typename T, int KM>
__global__ __launch_bounds__(kTopkThreads) void topk_partial(const T *__restrict__ logits,
                                                             int vocab, int64_t pos_stride,
                                                             int slice, int splits, int K,
                                                             void *ws, int64_t parts) {
    constexpr int N = Vec<T>::N;
    const int sp = blockIdx.x;
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int lo = sp * slice;
    const int hi = min(vocab, lo + slice);
    const T *rowp = logits + static_cast<int64_t>(row) * pos_stride;

    LaneAcc<KM> acc;
    acc.m = -INFINITY;
    acc.s = 0.0;
    acc.top.init();

    // scalar head up to the first 16-byte boundary (rows need only element
    // alignment), then full 16-byte vectors, then a scalar tail
    const int head = static_cast<int>(
        ((16 - (reinterpret_cast<uintptr_t>(rowp + lo) & 15)) & 15) / sizeof(T));
    const int vlo = min(hi, lo + head);
    if (tid < vlo - lo) {
        float x[1] = {Vec<T>::scalar(rowp + lo + tid)};
        acc.add(x, lo + tid);
    }
    const int nvec = (hi - vlo) / N;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + vlo);
    int i = tid;
    for (; i + 3 * kTopkThreads < nvec; i += 4 * kTopkThreads) {
        u32x4 w0 = __builtin_nontemporal_load(vp + i);
        u32x4 w1 = __builtin_nontemporal_load(vp + i + kTopkThreads);
        u32x4 w2 = __builtin_nontemporal_load(vp + i + 2 * kTopkThreads);
        u32x4 w3 = __builtin_nontemporal_load(vp + i + 3 * kTopkThreads);
        float x[N];
        Vec<T>::unpack(w0, x); acc.add(x, vlo + i * N);
        Vec<T>::unpack(w1, x); acc.add(x, vlo + (i + kTopkThreads) * N);
        Vec<T>::unpack(w2, x); acc.add(x, vlo + (i + 2 * kTopkThreads) * N);
        Vec<T>::unpack(w3, x); acc.add(x, vlo + (i + 3 * kTopkThreads) * N);
    }
    for (; i < nvec; i += kTopkThreads) {
        u32x4 w0 = __builtin_nontemporal_load(vp + i);
        float x[N];
        Vec<T>::unpack(w0, x);
        acc.add(x, vlo + i * N);
    }
    // ragged tail, one element per lane
    for (int e = vlo + nvec * N + tid; e < hi; e += kTopkThreads) {
        float x[1] = {Vec<T>::scalar(rowp + e)};
        acc.add(x, e);
    }

    // ---- workgroup reduction ----
    __shared__ float sm_m[kTopkWaves];
    __shared__ double sm_s[kTopkWaves];
    __shared__ float sm_v[kTopkWaves][TD_MAX_TOPK];
    __shared__ int sm_id[kTopkWaves][TD_MAX_TOPK];

    float wm = wave_max(acc.m);
    double contrib = (acc.m == -INFINITY)
                         ? 0.0
                         : acc.s * static_cast<double>(__builtin_amdgcn_exp2f((acc.m - wm) * kLog2e));
    double ws_sum = wave_sum(contrib);

    // K-round tournament over the 64 lanes' sorted lists
    for (int j = 0; j < K; ++j) {
        float bv = acc.top.v[0];
        int bi = acc.top.id[0];
        wave_best(bv, bi);
        if (lane == 0) {
            sm_v[wave][j] = bv;
            sm_id[wave][j] = bi;
        }
        acc.top.pop_if(acc.top.id[0] == bi && acc.top.v[0] == bv);
    }
    if (lane == 0) {
        sm_m[wave] = wm;
        sm_s[wave] = ws_sum;
    }
    __syncthreads();

    if (wave == 0) {
        // lanes 0..3 take the four wave lists, the rest stay empty
        LaneTop<KM> t;
        t.init();
        float m = -INFINITY;
        double s = 0.0;
        if (lane < kTopkWaves) {
            for (int j = 0; j < K; ++j) t.insert(sm_v[lane][j], sm_id[lane][j]);
            m = sm_m[lane];
            s = sm_s[lane];
        }
        float M = wave_max(m);
        double c = (m == -INFINITY) ? 0.0
                                    : s * static_cast<double>(__builtin_amdgcn_exp2f((m - M) * kLog2e));
        double S = wave_sum(c);
        TopkWs w = topk_ws(ws, parts, K);
        const int64_t part = static_cast<int64_t>(row) * splits + sp;
        float myv = -INFINITY;
        int myid = 0x7fffffff;
        for (int j = 0; j < K; ++j) {
            float bv = t.v[0];
            int bi = t.id[0];
            wave_best(bv, bi);
            if (lane == j) {
                myv = bv;
                myid = bi;
            }
            t.pop_if(t.id[0] == bi && t.v[0] == bv);
        }
        if (lane < K) {
            w.v[part * K + lane] = myv;
            w.id[part * K + lane] = myid;
        }
        if (lane == 0) {
            w.m[part] = M;
            w.s[part] = S;
        }
    }
}

template <int KM>
__global__ __launch_bounds__(kWave) void topk_merge(const void *ws, int64_t parts, int splits,
                                                    int K, int32_t *__restrict__ topk_id,
                                                    double *__restrict__ topk_logq,
                                                    double *__restrict__ lse_out) {
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    TopkWs w = topk_ws(const_cast<void *>(ws), parts, K);
    LaneTop<KM> t;
    t.init();
    float m = -INFINITY;
    double s = 0.0;
    if (lane < splits) {
        const int64_t part = static_cast<int64_t>(row) * splits + lane;
        for (int j = 0; j < K; ++j) t.insert(w.v[part * K + j], w.id[part * K + j]);
        m = w.m[part];
        s = w.s[part];
    }
    float M = wave_max(m);
    double c = (m == -INFINITY) ? 0.0 : s * exp(static_cast<double>(m) - static_cast<double>(M));
    double S = wave_sum(c);
    const double lse = static_cast<double>(M) + log(S);
    float myv = -INFINITY;
    int myid = 0;
    for (int j = 0; j < K; ++j) {
        float bv = t.v[0];
        int bi = t.id[0];
        wave_best(bv, bi);
        if (lane == j) {
            myv = bv;
            myid = bi;
        }
        t.pop_if(t.id[0] == bi && t.v[0] == bv);
    }
    if (lane < K) {
        topk_id[static_cast<int64_t>(row) * K + lane] = myid;
        topk_logq[static_cast<int64_t>(row) * K + lane] = static_cast<double>(myv) - lse;
    }
    if (lane == 0) lse_out[row] = lse;
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

template <typename T, int KM>
void launch_topk(const void *logits, int rows, int vocab, int64_t pos_stride, int K,
                 const TopkPlan &pl, void *ws, int32_t *topk_id, double *topk_logq, double *lse,
                 hipStream_t st) {
    const int64_t parts = static_cast<int64_t>(rows) * pl.splits;
    hipLaunchKernelGGL((topk_partial<T, KM>), dim3(pl.splits, rows), dim3(kTopkThreads), 0, st,
                       static_cast<const T *>(logits), vocab, pos_stride, pl.slice, pl.splits, K,
                       ws, parts);
    hipLaunchKernelGGL((topk_merge<KM>), dim3(rows), dim3(kWave), 0, st, ws, parts, pl.splits, K,
                       topk_id, topk_logq, lse);
}

template <typename T>
void launch_topk_k(const void *logits, int rows, int vocab, int64_t pos_stride, int K,
                   const TopkPlan &pl, void *ws, int32_t *topk_id, double *topk_logq, double *lse,
                   hipStream_t st) {
    if (K <= 4)
        launch_topk<T, 4>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id, topk_logq, lse, st);
    else if (K <= 8)
        launch_topk<T, 8>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id, topk_logq, lse, st);
    else if (K <= 16)
        launch_topk<T, 16>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id, topk_logq, lse, st);
    else
        launch_topk<T, 32>(logits, rows, vocab, pos_stride, K, pl, ws, topk_id, topk_logq, lse, st);
}

}  // namespace
}  // namespace td

using namespace td;

extern "C" size_t td_draft_topk_workspace(int32_t batch, int32_t block, int32_t vocab, int32_t K) {
    if (batch <= 0 || block <= 0 || vocab <= 0 || K <= 0) return 0;
    const int64_t rows = static_cast<int64_t>(batch) * block;
    TopkPlan pl = topk_plan(rows, vocab);
    return topk_ws_bytes(rows * pl.splits, K);
}

extern "C" td_status td_draft_topk(const void *logits, td_dtype dtype, int32_t batch, int32_t block,
                                   int32_t vocab, int64_t pos_stride, int32_t K, int32_t *topk_id,
                                   double *topk_logq, double *lse, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    clear_error();
    if (!logits || !topk_id || !topk_logq || !lse || !workspace)
        return fail(TD_EINVAL, "td_draft_topk: null pointer argument");
    if (batch <= 0 || block <= 0 || vocab <= 0 || K <= 0)
        return fail(TD_EINVAL, "td_draft_topk: batch, block, vocab and K must be positive");
    if (K > vocab) return fail(TD_EINVAL, "td_draft_topk: K exceeds the vocabulary");
    if (K > TD_MAX_TOPK) return fail(TD_ECAPACITY, "td_draft_topk: K above TD_MAX_TOPK");
    if (block > TD_MAX_BLOCK) return fail(TD_ECAPACITY, "td_draft_topk: block above TD_MAX_BLOCK");
    if (batch > TD_MAX_BATCH) return fail(TD_ECAPACITY, "td_draft_topk: batch above TD_MAX_BATCH");
    if (vocab > TD_MAX_VOCAB) return fail(TD_ECAPACITY, "td_draft_topk: vocab above TD_MAX_VOCAB");
    if (dtype != TD_F32 && dtype != TD_BF16)
        return fail(TD_EUNSUPPORTED, "td_draft_topk: dtype must be TD_F32 or TD_BF16");
    if (pos_stride < vocab) return fail(TD_EINVAL, "td_draft_topk: pos_stride < vocab");
    const int esz = dtype == TD_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(logits) % esz) != 0)
        return fail(TD_EINVAL, "td_draft_topk: logits must be aligned to the element size");
    if (!aligned16(workspace) || !aligned8(topk_logq) || !aligned8(lse))
        return fail(TD_EINVAL, "td_draft_topk: misaligned workspace or output");
    if (workspace_bytes < td_draft_topk_workspace(batch, block, vocab, K))
        return fail(TD_EINVAL, "td_draft_topk: workspace too small");
    const int rows = batch * block;
    TopkPlan pl = topk_plan(rows, vocab);
    hipStream_t st = as_stream(stream);
    if (dtype == TD_BF16)
        launch_topk_k<uint16_t>(logits, rows, vocab, pos_stride, K, pl, workspace, topk_id,
                                topk_logq, lse, st);
    else
        launch_topk_k<float>(logits, rows, vocab, pos_stride, K, pl, workspace, topk_id, topk_logq,
                             lse, st);
    return check_launch("td_draft_topk");
}
