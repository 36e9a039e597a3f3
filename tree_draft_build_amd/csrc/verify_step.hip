// td_verify_step: the verify step of budget-aware tree speculative decoding
// (BASTION, "Methodik" §1-§3) as three kernels, or two.  Kernel boundaries cost a few
// microseconds each on this GPU, which at batch 1 is as much as the stages'
// own memory time, so the step fuses what the five stage calls keep apart:
//   1. top-K of every position; the last position of each sequence to finish
//      builds the sequence's tree and mask rows in the same kernel;
//   2. split-KV context attention;
//   3. partial merge with the ancestor-masked tree keys, plus the acceptance
//      walk of every sequence.
// For short contexts (chunks of at most 128 keys) and a top-K of at most one
// workgroup per compute unit, kernel 2's work items join kernel 1 as extra
// workgroups: they load their keys and compute while the draft is selected,
// and wait only for their sequence's tree size.
// The device code is the stage calls' own.

#include <algorithm>
#include <mutex>

#include "step_launch.h"
#include "td_internal.h"
#include "tree_core.h"

using namespace td;

namespace {

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The workspace: the top-K part (status word, hand-off words), the tree-size
// words of the fused first kernel (one per sequence), then the attention
// partials.
size_t ready_offset(const td_step_args *a) {
    return topk_workspace_bytes(a->batch, a->block, a->vocab, a->topk);
}
size_t topk_part(const td_step_args *a) {
    return round_up(ready_offset(a) + static_cast<size_t>(a->batch) * 8, 256);
}

bool fuses_split(const td_step_args *a) {
    return step_fuses_split(a->batch, a->block, a->vocab, a->topk, a->n_max + 1, a->hq, a->hkv,
                            a->head_dim, a->total_ctx, a->attn_dtype);
}

}  // namespace

extern "C" size_t td_step_args_bytes(void) { return sizeof(td_step_args); }

extern "C" size_t td_verify_step_workspace(const td_step_args *a) {
    if (!a || a->batch <= 0 || a->block <= 0 || a->vocab <= 0 || a->topk <= 0 || a->n_max < 0 ||
        a->hq <= 0 || a->hkv <= 0 || a->hq % a->hkv || a->total_ctx < 0)
        return 0;
    const int nq_max = a->n_max + 1;
    // the attention partials of the step's own dtype (either's, should the
    // field hold neither: validation then rejects the call anyway)
    const bool known = a->attn_dtype == TD_BF16 || a->attn_dtype == TD_F32;
    const size_t attn = known ? attn_workspace_bytes(a->batch, nq_max, a->hq, a->hkv, a->head_dim,
                                                     a->total_ctx, a->attn_dtype)
                              : std::max(attn_workspace_bytes(a->batch, nq_max, a->hq, a->hkv,
                                                              a->head_dim, a->total_ctx, TD_BF16),
                                         attn_workspace_bytes(a->batch, nq_max, a->hq, a->hkv,
                                                              a->head_dim, a->total_ctx, TD_F32));
    // a call of both stages may run the split in the first kernel, with that
    // kernel's plan (128-key chunks): room for either plan's partials
    const size_t fused = fuses_split(a) ? attn_workspace_bytes(a->batch, nq_max, a->hq, a->hkv, a->head_dim,
                                                               a->total_ctx, a->attn_dtype, true)
                                        : 0;
    return topk_part(a) + std::max(attn, fused);
}

namespace {

// Validation of the argument block (no workspace): records the message and
// returns the status; enqueues nothing.
td_status check_step(const td_step_args *a) {
    if (!a) return fail(TD_EINVAL, "td_verify_step: null args");
    const int stages = a->stages == 0 ? (TD_STEP_DRAFT | TD_STEP_VERIFY) : a->stages;
    if (stages & ~(TD_STEP_DRAFT | TD_STEP_VERIFY))
        return fail(TD_EINVAL, "td_verify_step: stages must be a mask of TD_STEP_DRAFT, TD_STEP_VERIFY");
    const bool draft = stages & TD_STEP_DRAFT;
    const bool verify = stages & TD_STEP_VERIFY;
    td_status st = TD_OK;
    if (draft) {
        st = check_topk_args(a->logits, a->logits_dtype, a->batch, a->block, a->vocab,
                             a->pos_stride, a->topk, a->topk_id, a->topk_logq, a->lse);
        if (st != TD_OK) return st;
        st = check_tree_args(a->topk_id, a->topk_logq, a->batch, a->block, a->topk, a->n_max,
                             a->n_nodes, a->node_token, a->node_parent, a->node_depth,
                             a->node_logrho);
        if (st != TD_OK) return st;
    }
    const int nq_max = a->n_max + 1;
    if (verify) {
        if (a->n_max < 0 || a->n_max > TD_MAX_NODES)
            return fail(TD_ECAPACITY, "td_verify_step: n_max out of range");
        st = check_attn_args(a->q, a->k_ctx, a->v_ctx, a->ctx_offsets, a->total_ctx, a->max_ctx,
                             a->k_tree, a->v_tree, a->mask, a->n_nodes, a->batch, nq_max, a->hq,
                             a->hkv, a->head_dim, a->attn_dtype, a->out);
        if (st != TD_OK) return st;
        st = check_accept_args(a->node_token, a->node_parent, a->n_nodes, a->target_token,
                               a->batch, a->n_max, a->block, a->accept_len, a->accept_path,
                               a->bonus_token);
        if (st != TD_OK) return st;
    }
    if (!a->mask || !aligned8(a->mask)) return fail(TD_EINVAL, "td_verify_step: mask must be set");
    if (a->ctx_lengths && !aligned8(a->ctx_lengths))
        return fail(TD_EINVAL, "td_verify_step: misaligned ctx_lengths");
    if (verify && a->commit) {
        if (!a->ctx_lengths)
            return fail(TD_EINVAL, "td_verify_step: commit needs ctx_lengths");
        if (!a->k_ctx || !a->v_ctx)
            return fail(TD_EINVAL, "td_verify_step: commit needs the context arrays");
    }
    return TD_OK;
}

// Enqueue the selected stages (arguments already checked).
td_status launch_step(const td_step_args *a, void *workspace, void *stream) {
    const int stages = a->stages == 0 ? (TD_STEP_DRAFT | TD_STEP_VERIFY) : a->stages;
    const bool draft = stages & TD_STEP_DRAFT;
    const bool verify = stages & TD_STEP_VERIFY;
    const int nq_max = a->n_max + 1;
    hipStream_t s = as_stream(stream);
    char *ws = static_cast<char *>(workspace);
    uint64_t *ready = reinterpret_cast<uint64_t *>(ws + ready_offset(a));
    // both stages in one call: the context split may join the first kernel
    const bool fuse = draft && verify && fuses_split(a);
    if (draft) {
        const TreeParams tp{a->block, a->topk, a->n_max, a->use_stop, a->cost_a, a->cost_b,
                            a->cost_c, a->cost_knee, a->l_ar, a->ahat0, a->root_token,
                            tree_branch(a->branch, a->topk), a->min_logrho};
        const TreeOut to{a->n_nodes, a->node_token, a->node_parent, a->node_depth,
                         a->node_logrho, a->ahat, a->speedup, a->mask, fuse ? ready : nullptr};
        if (fuse) {
            const SplitInputs si{a->q, a->k_ctx, a->v_ctx, a->ctx_offsets, a->ctx_lengths, a->total_ctx,
                                 nq_max, a->hq, a->hkv, a->scale, ws + topk_part(a)};
            launch_topk_tree_split(a->logits, a->logits_dtype, a->batch, a->block, a->vocab,
                                   a->pos_stride, a->topk, ws, a->topk_id, a->topk_logq, a->lse, tp,
                                   to, si, s);
        } else {
            launch_topk_tree(a->logits, a->logits_dtype, a->batch, a->block, a->vocab, a->pos_stride,
                             a->topk, ws, a->topk_id, a->topk_logq, a->lse, tp, to, s);
        }
    }
    if (verify) {
        AcceptArgs acc{a->node_token, a->node_parent, a->target_token, a->n_max, a->block,
                       a->accept_len, a->accept_path, a->bonus_token, a->commit != 0, CommitArgs{}};
        if (a->commit) {
            const int esz = a->attn_dtype == TD_F32 ? 4 : 2;
            acc.cm = CommitArgs{static_cast<const uint4 *>(a->k_tree),
                                static_cast<const uint4 *>(a->v_tree),
                                static_cast<uint4 *>(const_cast<void *>(a->k_ctx)),
                                static_cast<uint4 *>(const_cast<void *>(a->v_ctx)),
                                a->ctx_offsets, a->ctx_lengths, a->next_root, nq_max,
                                a->hkv * a->head_dim * esz / 16};
        }
        acc.ready = ready;
        launch_attention(a->q, a->k_ctx, a->v_ctx, a->ctx_offsets, a->ctx_lengths, a->total_ctx, a->k_tree,
                         a->v_tree, a->mask, a->n_nodes, a->batch, nq_max, a->hq, a->hkv,
                         a->head_dim, a->scale, a->attn_dtype, ws + topk_part(a), a->out, &acc, s,
                         !fuse);
    }
    return check_launch("td_verify_step");
}

}  // namespace

extern "C" td_status td_verify_step(const td_step_args *a, void *workspace, size_t workspace_bytes,
                                    void *stream) {
    clear_error();
    const td_status st = check_step(a);
    if (st != TD_OK) return st;
    if (!workspace || !aligned16(workspace))
        return fail(TD_EINVAL, "td_verify_step: null or misaligned workspace");
    const size_t need = td_verify_step_workspace(a);
    if (need == 0)
        return fail(TD_EINVAL, "td_verify_step: invalid shape fields (batch, block, vocab, topk, "
                               "n_max, hq, hkv, total_ctx)");
    if (workspace_bytes < need) return fail(TD_EINVAL, "td_verify_step: workspace too small");
    return launch_step(a, workspace, stream);
}

extern "C" int32_t td_verify_step_kernels(const td_step_args *a) {
    if (!a || td_verify_step_workspace(a) == 0) return 0;
    const int stages = a->stages == 0 ? (TD_STEP_DRAFT | TD_STEP_VERIFY) : a->stages;
    if (stages & ~(TD_STEP_DRAFT | TD_STEP_VERIFY)) return 0;
    const bool draft = stages & TD_STEP_DRAFT;
    const bool verify = stages & TD_STEP_VERIFY;
    if (draft && verify && fuses_split(a)) return 2;
    return (draft ? 1 : 0) + (verify ? 2 : 0);
}

extern "C" td_status td_verify_step_events(const td_step_args *a, void *workspace,
                                           size_t workspace_bytes, void *stream, void *start_event,
                                           void *stop_event) {
    t_launch_events = {static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event), 0,
                       0x7fffffff, 0};
    const td_status st = td_verify_step(a, workspace, workspace_bytes, stream);
    t_launch_events = {};
    return st;
}

extern "C" td_status td_verify_step_kernel_events(const td_step_args *a, void *workspace,
                                                  size_t workspace_bytes, void *stream,
                                                  int32_t first_kernel, int32_t last_kernel,
                                                  void *start_event, void *stop_event) {
    clear_error();
    const int n = td_verify_step_kernels(a);
    if (n > 0 && (first_kernel < 0 || last_kernel < first_kernel || last_kernel >= n))
        return fail(TD_EINVAL, "td_verify_step_kernel_events: kernel range outside the call's kernels");
    t_launch_events = {static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event),
                       first_kernel, last_kernel, 0};
    const td_status st = td_verify_step(a, workspace, workspace_bytes, stream);
    t_launch_events = {};
    return st;
}

// ---------------------------------------------------------------------------
// td_verify_step_noalloc: the same kernels with the workspace in a static
// device array instead of a caller buffer, for callers that cannot allocate.
// Each GPU the library runs on holds its own copy of the array until the
// process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on its first call.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch address of the current device (looked up once per device).
td_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_error("td_verify_step_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
        return TD_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(TD_ECAPACITY, "td_verify_step_noalloc: device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("td_verify_step_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
            return TD_EHIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TD_OK;
}

// Zero n bytes (a multiple of 16, 16-byte aligned) with ordinary vector
// stores: the top-K hand-off words of the previous call must not be seen.
__global__ __launch_bounds__(256) void zero_fill(uint4 *__restrict__ p, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

extern "C" td_status td_verify_step_noalloc(const td_step_args *a, void *stream) {
    clear_error();
    td_status st = check_step(a);
    if (st != TD_OK) return st;
    const size_t need = td_verify_step_workspace(a);
    if (need == 0) return fail(TD_EINVAL, "td_verify_step_noalloc: invalid shape fields");
    if (need > kScratchBytes)
        return fail(TD_ECAPACITY, "td_verify_step_noalloc: the problem needs more than the 64 MiB "
                                  "scratch; use td_verify_step with a workspace");
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != TD_OK) return st;
    const int stages = a->stages == 0 ? (TD_STEP_DRAFT | TD_STEP_VERIFY) : a->stages;
    if (stages & TD_STEP_DRAFT) {
        // every call starts from cleared hand-off words (the array keeps the
        // last call's contents, possibly of another shape); the attention
        // partials need no clearing
        const int64_t n16 = static_cast<int64_t>(topk_part(a) / 16);
        const unsigned blocks = static_cast<unsigned>(std::min<int64_t>(1024, (n16 + 255) / 256));
        hipLaunchKernelGGL(zero_fill, dim3(blocks), dim3(256), 0, as_stream(stream),
                           static_cast<uint4 *>(ws), n16);
    }
    return launch_step(a, ws, stream);
}
