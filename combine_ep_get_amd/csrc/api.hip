// C ABI of libepget (declared in include/ep_get.h): argument validation,
// workspace sizing and kernel launches.  Nothing here allocates, frees or
// synchronises, except ep_read_status, which exists to synchronise.
//
// Limits are those of "DeepEP V2 ElasticBuffer 架构深度分析" (the
// kNumMaxRanks / kNumMaxExperts / kNumMaxExpertsPerRank block); argument
// checks before launch play the role of the host asserts that the pages'
// runtime uses ("DeepEP Symmetric Memory 全面架构分析" §7.3, §9.1).
#include <limits.h>

#include <atomic>
#include <mutex>

#include "../../include/ep_get.h"
#include "ep_internal.h"
#include "hier_internal.h"

namespace {

using epget::WsLayout;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Checks every field that does not depend on S.
int check_shape(const ep_problem *p) {
    if (!p) return EP_ERR_INVALID_ARG;
    if (p->reserved != 0) return EP_ERR_INVALID_ARG;
    if (p->num_tokens < 0) return EP_ERR_INVALID_ARG;
    if (p->hidden < 8 || p->hidden % 8 != 0 || p->hidden > EP_MAX_HIDDEN) return EP_ERR_INVALID_ARG;
    if (p->num_experts < 1 || p->num_experts > EP_MAX_EXPERTS) return EP_ERR_INVALID_ARG;
    if (p->num_ranks < 1 || p->num_ranks > EP_MAX_RANKS) return EP_ERR_INVALID_ARG;
    if (p->num_experts % p->num_ranks != 0) return EP_ERR_INVALID_ARG;
    if (p->num_experts / p->num_ranks > EP_MAX_EXPERTS_PER_RANK) return EP_ERR_INVALID_ARG;
    if (p->num_groups < 1 || p->num_ranks % p->num_groups != 0) return EP_ERR_INVALID_ARG;
    if (p->num_topk < 1 || p->num_topk > EP_MAX_TOPK) return EP_ERR_INVALID_ARG;
    if (p->expert_alignment < 1) return EP_ERR_INVALID_ARG;
    const int64_t entries = static_cast<int64_t>(p->num_tokens) * p->num_topk;
    const int64_t pad = static_cast<int64_t>(p->num_experts) * p->expert_alignment;
    // index arithmetic in the kernels overshoots the last entry or token by
    // less than a tile (at most 16384) before it is clamped or tested
    if (entries + pad > INT32_MAX - (1 << 16)) return EP_ERR_INVALID_ARG;
    // the chunk table is read through raw buffer loads with 32-bit byte
    // offsets, and an offset past the table (0xFFFFFFFC) must stay out of
    // range for predicated loads: fewer than 2^30 table entries
    const WsLayout w = epget::ws_layout(p->num_tokens, p->num_topk, p->num_experts, p->num_ranks,
                                        p->num_groups);
    if (w.nchunks * w.pitch >= (int64_t{1} << 30)) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

int check_problem(const ep_problem *p) {
    const int rc = check_shape(p);
    if (rc != EP_OK) return rc;
    if (p->rank_stride_rows < 1) return EP_ERR_INVALID_ARG;
    if (p->rank_stride_rows * p->num_ranks > INT32_MAX) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

epget::CopyParams copy_params(const ep_problem *p) {
    epget::CopyParams c;
    c.T = p->num_tokens;
    c.H = p->hidden;
    c.K = p->num_topk;
    c.nvec = p->hidden / 8;
    c.vpt = 1;
    c.num_rows = p->rank_stride_rows * p->num_ranks;
    return c;
}

// Validates the layout call's arguments and fills lp.
int layout_params(const ep_problem *p, const int32_t *topk_idx, int32_t *expert_count,
                  int32_t *expert_offset, int32_t *rank_row_count, int32_t *rank_token_count,
                  int32_t *group_token_count, uint8_t *is_token_in_rank, int32_t *token_slot,
                  int64_t *cumulative_expert_recv, void *workspace, size_t workspace_bytes,
                  epget::LayoutParams *out) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    const bool has_tokens = p->num_tokens > 0;
    if (!expert_count || !expert_offset || !rank_row_count || !rank_token_count || !workspace)
        return EP_ERR_INVALID_ARG;
    if (has_tokens && (!topk_idx || !is_token_in_rank || !token_slot)) return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(expert_count, 4) || !aligned(expert_offset, 4) ||
        !aligned(rank_row_count, 4) || !aligned(rank_token_count, 4) ||
        !aligned(group_token_count, 4) || !aligned(token_slot, 4) ||
        !aligned(cumulative_expert_recv, 8) || !aligned(workspace, 256))
        return EP_ERR_INVALID_ARG;
    const WsLayout w = epget::ws_layout(p->num_tokens, p->num_topk, p->num_experts,
                                        p->num_ranks, p->num_groups);
    if (workspace_bytes < static_cast<size_t>(w.bytes)) return EP_ERR_INVALID_ARG;

    epget::LayoutParams &lp = *out;
    lp.topk_idx = topk_idx;
    lp.T = p->num_tokens;
    lp.K = p->num_topk;
    lp.E = p->num_experts;
    lp.R = p->num_ranks;
    lp.G = p->num_groups;
    lp.A = p->expert_alignment;
    lp.L = p->num_experts / p->num_ranks;
    lp.ranks_per_group = p->num_ranks / p->num_groups;
    lp.div_L = epget::FastDiv::make(static_cast<uint32_t>(lp.L));
    lp.S = static_cast<int32_t>(p->rank_stride_rows);
    lp.chunk_tokens = w.chunk_tokens;
    lp.nchunks = static_cast<int32_t>(w.nchunks);
    lp.ncols = w.ncols;
    lp.pitch = w.pitch;
    int nbits = 0;
    while ((1 << nbits) < p->num_experts) ++nbits;
    lp.nbits = nbits;
    lp.expert_count = expert_count;
    lp.expert_offset = expert_offset;
    lp.rank_row_count = rank_row_count;
    lp.rank_token_count = rank_token_count;
    lp.group_token_count = group_token_count;
    lp.is_token_in_rank = is_token_in_rank;
    lp.token_slot = token_slot;
    lp.cumulative = cumulative_expert_recv;
    char *ws = static_cast<char *>(workspace);
    lp.status = reinterpret_cast<int32_t *>(ws);
    lp.totals = reinterpret_cast<int32_t *>(ws + w.totals_off);
    lp.table = reinterpret_cast<int32_t *>(ws + w.table_off);
    lp.count_t = reinterpret_cast<int32_t *>(ws + w.count_t_off);
    lp.excl_t = reinterpret_cast<int32_t *>(ws + w.excl_t_off);
    return EP_OK;
}

// Validates the bf16 dispatch call's pointers and fills a.
int dispatch_args(const uint16_t *x, const float *topk_weights, const int32_t *token_slot,
                  uint16_t *recv_x, int32_t *recv_src_token, float *recv_weight,
                  epget::DispatchArgs *out) {
    if (!x || !token_slot || !recv_x) return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(token_slot, 4) ||
        !aligned(topk_weights, 4) || !aligned(recv_src_token, 4) || !aligned(recv_weight, 4))
        return EP_ERR_INVALID_ARG;
    epget::DispatchArgs a = {};
    a.x = x;
    a.w = topk_weights;
    a.slot = token_slot;
    a.recv = recv_x;
    a.recv_src = recv_src_token;
    a.recv_w = recv_weight;
    *out = a;
    return EP_OK;
}

// Validates the FP8 dispatch call's arguments (H % 128 == 0, scale strides,
// pointers) and fills c and a.  With no tokens only the sizes are checked.
int dispatch_fp8_args(const ep_problem *p, const uint8_t *x_fp8, const float *x_sf,
                      const float *topk_weights, const int32_t *token_slot, uint8_t *recv_x_fp8,
                      float *recv_sf, int64_t sf_token_stride, int64_t sf_hidden_stride,
                      int32_t *recv_src_token, float *recv_weight, epget::CopyParams *c,
                      epget::DispatchArgs *out) {
    if (p->hidden % 128 != 0 || sf_token_stride < 1 || sf_hidden_stride < 1)
        return EP_ERR_INVALID_ARG;
    const int64_t nsf = p->hidden / 128;
    const int64_t rows = p->rank_stride_rows * p->num_ranks;
    // the largest scale index must be addressable
    if ((rows - 1) > (INT64_MAX - (nsf - 1) * sf_hidden_stride) / sf_token_stride)
        return EP_ERR_INVALID_ARG;
    *c = copy_params(p);
    c->nvec = p->hidden / 16;
    *out = epget::DispatchArgs{};
    if (p->num_tokens == 0) return EP_OK;
    if (!x_fp8 || !x_sf || !token_slot || !recv_x_fp8 || !recv_sf) return EP_ERR_INVALID_ARG;
    if (!aligned(x_fp8, 16) || !aligned(recv_x_fp8, 16) || !aligned(x_sf, 4) ||
        !aligned(recv_sf, 4) || !aligned(token_slot, 4) || !aligned(topk_weights, 4) ||
        !aligned(recv_src_token, 4) || !aligned(recv_weight, 4))
        return EP_ERR_INVALID_ARG;
    epget::DispatchArgs a = {};
    a.x = x_fp8;
    a.w = topk_weights;
    a.slot = token_slot;
    a.recv = recv_x_fp8;
    a.recv_src = recv_src_token;
    a.recv_w = recv_weight;
    a.x_sf = x_sf;
    a.recv_sf = recv_sf;
    a.sf_ts = sf_token_stride;
    a.sf_hs = sf_hidden_stride;
    a.nsf = static_cast<int32_t>(nsf);
    // token-major rows padded to whole 128-byte lines are written whole
    const bool whole_lines = sf_hidden_stride == 1 && sf_token_stride > nsf && sf_token_stride % 32 == 0 &&
                             sf_token_stride - nsf < 32;
    a.sf_row = static_cast<int32_t>(whole_lines ? sf_token_stride : nsf);
    *out = a;
    return EP_OK;
}

}  // namespace

extern "C" {

size_t ep_workspace_bytes(const ep_problem *p) {
    if (check_shape(p) != EP_OK) return 0;
    const WsLayout w = epget::ws_layout(p->num_tokens, p->num_topk, p->num_experts,
                                        p->num_ranks, p->num_groups);
    return static_cast<size_t>(w.bytes);
}

int64_t ep_rank_stride_hint(const ep_problem *p) {
    if (check_shape(p) != EP_OK) return -1;
    const int64_t L = p->num_experts / p->num_ranks;
    const int64_t per_token = p->num_topk < L ? p->num_topk : L;
    const int64_t s = p->num_tokens * per_token + L * (p->expert_alignment - 1);
    return s > 0 ? s : 1;
}

int ep_get_layout(const ep_problem *p, const int32_t *topk_idx, int32_t *expert_count,
                  int32_t *expert_offset, int32_t *rank_row_count, int32_t *rank_token_count,
                  int32_t *group_token_count, uint8_t *is_token_in_rank, int32_t *token_slot,
                  int64_t *cumulative_expert_recv, void *workspace, size_t workspace_bytes,
                  void *stream) {
    epget::LayoutParams lp;
    const int rc = layout_params(p, topk_idx, expert_count, expert_offset, rank_row_count,
                                 rank_token_count, group_token_count, is_token_in_rank, token_slot,
                                 cumulative_expert_recv, workspace, workspace_bytes, &lp);
    if (rc != EP_OK) return rc;
    return hip_rc(epget::launch_layout(lp, static_cast<hipStream_t>(stream)));
}

int ep_dispatch(const ep_problem *p, const uint16_t *x, const float *topk_weights,
                const int32_t *token_slot, uint16_t *recv_x, int32_t *recv_src_token,
                float *recv_weight, void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    if (p->num_tokens == 0) return EP_OK;
    epget::DispatchArgs a;
    rc = dispatch_args(x, topk_weights, token_slot, recv_x, recv_src_token, recv_weight, &a);
    if (rc != EP_OK) return rc;
    return hip_rc(epget::launch_dispatch(copy_params(p), a, static_cast<hipStream_t>(stream)));
}

int ep_layout_dispatch(const ep_problem *p, const int32_t *topk_idx, int32_t *expert_count,
                       int32_t *expert_offset, int32_t *rank_row_count, int32_t *rank_token_count,
                       int32_t *group_token_count, uint8_t *is_token_in_rank, int32_t *token_slot,
                       int64_t *cumulative_expert_recv, void *workspace, size_t workspace_bytes,
                       const uint16_t *x, const float *topk_weights, uint16_t *recv_x,
                       int32_t *recv_src_token, float *recv_weight, void *stream) {
    epget::LayoutParams lp;
    int rc = layout_params(p, topk_idx, expert_count, expert_offset, rank_row_count, rank_token_count,
                           group_token_count, is_token_in_rank, token_slot, cumulative_expert_recv,
                           workspace, workspace_bytes, &lp);
    if (rc != EP_OK) return rc;
    epget::DispatchArgs a = {};
    if (p->num_tokens > 0) {
        rc = dispatch_args(x, topk_weights, token_slot, recv_x, recv_src_token, recv_weight, &a);
        if (rc != EP_OK) return rc;
    }
    return hip_rc(epget::launch_layout_dispatch(lp, copy_params(p), a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Scratch of ep_layout_dispatch_noalloc: the layout workspace (column totals
// and chunk tables) of one call, in the library's own device memory so that
// the call allocates nothing.  Each device holds its own copy for the life of
// the process.  In host code `scratch` is only a stand-in for the symbol:
// kernels get the device address that hipGetSymbolAddress returns, never
// the array's name.
static __device__ __align__(256) unsigned char scratch[EP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.  The stream must belong to the
// current device, since the kernels run there.
int device_scratch(hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return EP_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = 0;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return EP_ERR_HIP;
        if (sdev != dev) return EP_ERR_INVALID_ARG;
    }
    void *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return EP_ERR_HIP;
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout_dispatch_noalloc(const ep_problem *p, const int32_t *topk_idx, int32_t *expert_count,
                               int32_t *expert_offset, int32_t *rank_row_count,
                               int32_t *rank_token_count, int32_t *group_token_count,
                               uint8_t *is_token_in_rank, int32_t *token_slot,
                               int64_t *cumulative_expert_recv, int32_t *status, const uint16_t *x,
                               const float *topk_weights, uint16_t *recv_x, int32_t *recv_src_token,
                               float *recv_weight, void *stream) {
    // sizes first, so that a problem too large for the scratch is refused
    // before any device call
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    const WsLayout w = epget::ws_layout(p->num_tokens, p->num_topk, p->num_experts,
                                        p->num_ranks, p->num_groups);
    if (w.bytes > static_cast<int64_t>(EP_NOALLOC_SCRATCH_BYTES)) return EP_ERR_SCRATCH_LIMIT;
    if (!status || !aligned(status, 4)) return EP_ERR_INVALID_ARG;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if ((rc = device_scratch(st, &ws)) != EP_OK) return rc;
    epget::LayoutParams lp;
    rc = layout_params(p, topk_idx, expert_count, expert_offset, rank_row_count, rank_token_count,
                       group_token_count, is_token_in_rank, token_slot, cumulative_expert_recv, ws,
                       EP_NOALLOC_SCRATCH_BYTES, &lp);
    if (rc != EP_OK) return rc;
    lp.status = status;  // the caller's word, not the scratch's first bytes
    epget::DispatchArgs a = {};
    if (p->num_tokens > 0) {
        rc = dispatch_args(x, topk_weights, token_slot, recv_x, recv_src_token, recv_weight, &a);
        if (rc != EP_OK) return rc;
    }
    return hip_rc(epget::launch_layout_dispatch(lp, copy_params(p), a, st));
}

int ep_quantize_fp8(const ep_problem *p, const uint16_t *x, uint8_t *x_fp8, float *x_sf,
                    void *stream) {
    int rc = check_shape(p);
    if (rc != EP_OK) return rc;
    if (p->hidden % 128 != 0) return EP_ERR_INVALID_ARG;
    if (p->num_tokens == 0) return EP_OK;
    if (!x || !x_fp8 || !x_sf) return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(x_fp8, 16) || !aligned(x_sf, 4)) return EP_ERR_INVALID_ARG;
    return hip_rc(epget::launch_quantize_fp8(p->num_tokens, p->hidden, x, x_fp8, x_sf,
                                             static_cast<hipStream_t>(stream)));
}

int ep_dispatch_fp8(const ep_problem *p, const uint8_t *x_fp8, const float *x_sf,
                    const float *topk_weights, const int32_t *token_slot, uint8_t *recv_x_fp8,
                    float *recv_sf, int64_t sf_token_stride, int64_t sf_hidden_stride,
                    int32_t *recv_src_token, float *recv_weight, void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    epget::CopyParams c;
    epget::DispatchArgs a;
    rc = dispatch_fp8_args(p, x_fp8, x_sf, topk_weights, token_slot, recv_x_fp8, recv_sf,
                           sf_token_stride, sf_hidden_stride, recv_src_token, recv_weight, &c, &a);
    if (rc != EP_OK || p->num_tokens == 0) return rc;
    return hip_rc(epget::launch_dispatch(c, a, static_cast<hipStream_t>(stream)));
}

int ep_layout_dispatch_fp8(const ep_problem *p, const int32_t *topk_idx, int32_t *expert_count,
                           int32_t *expert_offset, int32_t *rank_row_count, int32_t *rank_token_count,
                           int32_t *group_token_count, uint8_t *is_token_in_rank, int32_t *token_slot,
                           int64_t *cumulative_expert_recv, void *workspace, size_t workspace_bytes,
                           const uint8_t *x_fp8, const float *x_sf, const float *topk_weights,
                           uint8_t *recv_x_fp8, float *recv_sf, int64_t sf_token_stride,
                           int64_t sf_hidden_stride, int32_t *recv_src_token, float *recv_weight,
                           void *stream) {
    epget::LayoutParams lp;
    int rc = layout_params(p, topk_idx, expert_count, expert_offset, rank_row_count, rank_token_count,
                           group_token_count, is_token_in_rank, token_slot, cumulative_expert_recv,
                           workspace, workspace_bytes, &lp);
    if (rc != EP_OK) return rc;
    epget::CopyParams c;
    epget::DispatchArgs a;
    rc = dispatch_fp8_args(p, x_fp8, x_sf, topk_weights, token_slot, recv_x_fp8, recv_sf,
                           sf_token_stride, sf_hidden_stride, recv_src_token, recv_weight, &c, &a);
    if (rc != EP_OK) return rc;
    return hip_rc(epget::launch_layout_dispatch(lp, c, a, static_cast<hipStream_t>(stream)));
}

int ep_combine(const ep_problem *p, const uint16_t *y, const int32_t *token_slot,
               const float *topk_weights, uint16_t *out, void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    if (p->num_tokens == 0) return EP_OK;
    if (!y || !token_slot || !out) return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(token_slot, 4) ||
        !aligned(topk_weights, 4))
        return EP_ERR_INVALID_ARG;
    return hip_rc(epget::launch_combine(copy_params(p), y, token_slot, topk_weights, out,
                                        static_cast<hipStream_t>(stream)));
}

int ep_combine_topk_weights(const ep_problem *p, const float *recv_weight,
                            const int32_t *token_slot, float *combined_topk_weights,
                            void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    if (p->num_tokens == 0) return EP_OK;
    if (!recv_weight || !token_slot || !combined_topk_weights) return EP_ERR_INVALID_ARG;
    if (!aligned(recv_weight, 4) || !aligned(token_slot, 4) || !aligned(combined_topk_weights, 4))
        return EP_ERR_INVALID_ARG;
    return hip_rc(epget::launch_combine_weights(copy_params(p), recv_weight, token_slot,
                                                combined_topk_weights,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int check_groups(const ep_problem *p, int64_t SG) {
    if (SG < 1 || SG * p->num_groups > INT32_MAX) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

epget::HierParams hier_params(const ep_problem *p, int64_t SG) {
    epget::HierParams h;
    h.G = p->num_groups;
    h.ranks_per_group = p->num_ranks / p->num_groups;
    h.S = static_cast<int32_t>(p->rank_stride_rows);
    h.SG = static_cast<int32_t>(SG);
    h.group_rows = SG * p->num_groups;
    return h;
}

}  // namespace

extern "C" {

int ep_get_group_layout(const ep_problem *p, const uint8_t *is_token_in_rank,
                        int64_t group_stride_rows, int32_t *group_slot, int32_t *status,
                        void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    if ((rc = check_groups(p, group_stride_rows)) != EP_OK) return rc;
    if (!aligned(status, 4)) return EP_ERR_INVALID_ARG;
    if (p->num_tokens == 0) return EP_OK;
    if (!is_token_in_rank || !group_slot || !aligned(group_slot, 4)) return EP_ERR_INVALID_ARG;
    return hip_rc(epget::launch_group_layout(p->num_tokens, p->num_ranks,
                                             hier_params(p, group_stride_rows), is_token_in_rank,
                                             group_slot, status, static_cast<hipStream_t>(stream)));
}

int ep_dispatch_hier(const ep_problem *p, const uint16_t *x, const float *topk_weights,
                     const int32_t *token_slot, const int32_t *group_slot,
                     int64_t group_stride_rows, uint16_t *group_buf, uint16_t *recv_x,
                     int32_t *recv_src_token, float *recv_weight, void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    if ((rc = check_groups(p, group_stride_rows)) != EP_OK) return rc;
    if (p->num_tokens == 0) return EP_OK;
    if (!x || !token_slot || !group_slot || !group_buf || !recv_x) return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(group_buf, 16) || !aligned(recv_x, 16) ||
        !aligned(token_slot, 4) || !aligned(group_slot, 4) || !aligned(topk_weights, 4) ||
        !aligned(recv_src_token, 4) || !aligned(recv_weight, 4))
        return EP_ERR_INVALID_ARG;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const epget::HierParams h = hier_params(p, group_stride_rows);
    // stage 1: each token once to every group it reaches
    hipError_t err = epget::launch_group_dispatch(copy_params(p), h, x, group_slot, group_buf, st);
    if (err != hipSuccess) return EP_ERR_HIP;
    // stage 2: group rows to the entries' rows
    epget::DispatchArgs a2 = {};
    a2.w = topk_weights;
    a2.slot = token_slot;
    a2.recv = recv_x;
    a2.recv_src = recv_src_token;
    a2.recv_w = recv_weight;
    return hip_rc(epget::launch_expand(copy_params(p), h, a2, group_slot, group_buf, st));
}

int ep_combine_hier(const ep_problem *p, const uint16_t *y, const int32_t *token_slot,
                    const float *topk_weights, const int32_t *group_slot,
                    int64_t group_stride_rows, uint16_t *group_buf, uint16_t *out, void *stream) {
    int rc = check_problem(p);
    if (rc != EP_OK) return rc;
    if ((rc = check_groups(p, group_stride_rows)) != EP_OK) return rc;
    if (p->num_tokens == 0) return EP_OK;
    if (!y || !token_slot || !group_slot || !group_buf || !out) return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(group_buf, 16) || !aligned(out, 16) ||
        !aligned(token_slot, 4) || !aligned(group_slot, 4) || !aligned(topk_weights, 4))
        return EP_ERR_INVALID_ARG;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const epget::HierParams h = hier_params(p, group_stride_rows);
    // stage 1: per-(token, group) partials, rounded to bf16 in the group rows
    hipError_t err = epget::launch_combine_partial(copy_params(p), h, y, token_slot, topk_weights,
                                                   group_slot, group_buf, st);
    if (err != hipSuccess) return EP_ERR_HIP;
    // stage 2: sum of the token's group rows
    return hip_rc(epget::launch_combine_groups(copy_params(p), h, group_buf, group_slot, out, st));
}

int ep_read_status(const void *workspace, void *stream) {
    if (!workspace || !aligned(workspace, 4)) return EP_ERR_INVALID_ARG;
    int32_t v = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&v, workspace, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess)
        return EP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return EP_ERR_HIP;
    return v;
}

const char *ep_error_string(int code) {
    switch (code) {
        case EP_OK: return "ok";
        case EP_ERR_INVALID_ARG: return "invalid argument";
        case EP_ERR_HIP: return "HIP runtime error";
        case EP_ERR_CAPACITY: return "rank slice capacity exceeded";
        case EP_ERR_BAD_EXPERT: return "expert id out of range";
        case EP_ERR_SCRATCH_LIMIT:
            return "problem needs more layout scratch than the library's static buffer holds";
        default: return "unknown error";
    }
}

}  // extern "C"
