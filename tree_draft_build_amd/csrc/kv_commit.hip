// After acceptance: the accepted prefix becomes context.  The target has
// verified the tree in one pass and decoding continues from the accepted
// prefix (BASTION, "Problemstellung"); the keys and values of the prefix's
// tokens, computed in that pass, are kept (the FlexDraft page, "Methodik"
// §3, decoupled execution: the verification's KV cache is reused).  The
// device core (commit_seq) is shared with the verify step's last kernel.

#include "step_launch.h"
#include "tree_core.h"

namespace td {
namespace {

// One workgroup per sequence: the path into LDS (up to its first entry
// outside the tree rows), then every thread copies 16-byte vectors.
__global__ __launch_bounds__(256) void kv_commit_kernel(const int32_t *__restrict__ accept_len,
                                                        const int32_t *__restrict__ accept_path,
                                                        const int32_t *__restrict__ bonus_token,
                                                        int block, CommitArgs c) {
    __shared__ int s_path[TD_MAX_BLOCK + 1];
    __shared__ int s_rows;
    __shared__ int64_t s_len;
    const int b = blockIdx.x;
    if (threadIdx.x == 0) {
        int A = accept_len[b];
        A = A < 0 ? 0 : (A > block ? block : A);
        int rows = 0;
        const int32_t *p = accept_path + static_cast<int64_t>(b) * (block + 1);
        for (int j = 0; j <= A; ++j) {
            const int node = p[j];
            if (node < 0 || node >= c.nq_max) break;
            s_path[j] = node;
            rows = j + 1;
        }
        s_rows = rows;
        s_len = commit_length(c, b);
    }
    __syncthreads();
    const int bonus = bonus_token ? bonus_token[b] : -1;
    commit_seq(c, b, s_path, s_rows - 1, bonus, s_len, threadIdx.x, blockDim.x);
}

}  // namespace
}  // namespace td

using namespace td;

extern "C" td_status td_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accept_len,
                                  const int32_t *accept_path, const int32_t *bonus_token,
                                  int32_t batch, int32_t nq_max, int32_t block, int32_t hkv,
                                  int32_t head_dim, td_dtype dtype, void *k_cache, void *v_cache,
                                  const int64_t *ctx_offsets, int64_t *ctx_lengths,
                                  int32_t *next_root, void *stream) {
    clear_error();
    if (!k_tree || !v_tree || !accept_len || !accept_path || !bonus_token || !k_cache ||
        !v_cache || !ctx_offsets || !ctx_lengths)
        return fail(TD_EINVAL, "td_kv_commit: null pointer argument");
    if (batch <= 0 || nq_max <= 0 || block <= 0 || hkv <= 0)
        return fail(TD_EINVAL, "td_kv_commit: sizes must be positive");
    if (batch > TD_MAX_BATCH || nq_max > TD_MAX_NODES + 1 || block > TD_MAX_BLOCK)
        return fail(TD_ECAPACITY, "td_kv_commit: batch, nq_max or block above capacity");
    if (dtype != TD_F32 && dtype != TD_BF16)
        return fail(TD_EUNSUPPORTED, "td_kv_commit: dtype must be TD_F32 or TD_BF16");
    if (head_dim != 64 && head_dim != 128)
        return fail(TD_EUNSUPPORTED, "td_kv_commit: head_dim must be 64 or 128");
    if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned8(ctx_offsets) || !aligned8(ctx_lengths))
        return fail(TD_EINVAL, "td_kv_commit: misaligned array");
    const int esz = dtype == TD_F32 ? 4 : 2;
    const CommitArgs c{static_cast<const uint4 *>(k_tree), static_cast<const uint4 *>(v_tree),
                       static_cast<uint4 *>(k_cache), static_cast<uint4 *>(v_cache), ctx_offsets,
                       ctx_lengths, next_root, nq_max, hkv * head_dim * esz / 16};
    hipLaunchKernelGGL(kv_commit_kernel, dim3(batch), dim3(256), 0, as_stream(stream), accept_len,
                       accept_path, bonus_token, block, c);
    return check_launch("td_kv_commit");
}
