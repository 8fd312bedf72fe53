/*
 * ep_get.h — C ABI of libepget: MoE token layout, dispatch and combine for
 * one source rank on one MI355X (gfx950), with the R destination ranks held
 * as fixed-stride slices of one receive buffer.
 *
 * Pages cited (by title):
 *   [SYM] "DeepEP Symmetric Memory 全面架构分析"
 *         (DeepEP symmetric memory: full architecture analysis)
 *   [V2]  "DeepEP V2 ElasticBuffer 架构深度分析"
 *         (DeepEP V2 ElasticBuffer architecture in depth; no section headings,
 *         its code blocks are cited by what they show)
 *   [V1]  "第 3 章 V1：Buffer 初始化与通信域建立"
 *         (chapter 3, V1 buffer initialisation and communicator set-up)
 *
 * Conventions for every entry point:
 *   - All pointers named "device" point to device memory the caller owns
 *     (allocated e.g. by PyTorch); the library allocates and frees nothing
 *     and keeps no state between calls.  Every array must hold at least the
 *     elements its stated shape implies: the kernels index it by the
 *     problem's sizes and cannot see its length.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  The hot
 *     calls (ep_get_layout, ep_dispatch, ep_combine) only enqueue kernels:
 *     they never synchronise, so their results are ready when the stream
 *     reaches that point.
 *   - Return value: EP_OK, or a negative EP_ERR_* code.  Argument problems
 *     are found on the host before anything is enqueued (EP_ERR_INVALID_ARG);
 *     a failed launch gives EP_ERR_HIP.  Problems only the device can see (an
 *     expert id out of range, a slice overflow) are written to a status word
 *     in the workspace that ep_read_status returns.  This is the C form of
 *     the host asserts and the exception with line info that [SYM] §7.3 and
 *     [V2] (pp_send/pp_recv block) show.
 *
 * Notation, following the dispatch launch arguments of [SYM] §6.1:
 *   T num_tokens, H hidden, E num_experts, K num_topk, R num_ranks
 *   (scale-up ranks), G num_groups, A expert_alignment, S rank_stride_rows,
 *   L = E / R local experts per rank, rank(e) = e / L,
 *   group(r) = r / (R / G).
 *
 * Receive buffer: slice r occupies rows [r*S, (r+1)*S) of an [R*S, H] bf16
 * array — the same byte offset in every rank's symmetric buffer, as [SYM]
 * §5.1 maps one symmetric offset to each peer.  Inside slice r the experts of
 * rank r own consecutive segments in local-expert order; expert e's segment
 * starts at row expert_offset[e] (aligned to A) and holds its rows in
 * ascending source token, then ascending top-k position.
 */
#ifndef EP_GET_H
#define EP_GET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_OK 0
#define EP_ERR_INVALID_ARG (-1) /* bad sizes, limits, NULL or misaligned pointer, small workspace */
#define EP_ERR_HIP (-2)         /* a HIP runtime call or kernel launch failed */
#define EP_ERR_CAPACITY (-3)    /* some rank needs more than S rows (device-detected) */
#define EP_ERR_BAD_EXPERT (-4)  /* an id outside [0,E) other than -1 (device-detected) */
#define EP_ERR_SCRATCH_LIMIT (-5) /* the problem needs more than EP_NOALLOC_SCRATCH_BYTES of
                                     layout scratch (ep_layout_dispatch_noalloc only) */

/* Size of the static device buffer behind ep_layout_dispatch_noalloc. */
#define EP_NOALLOC_SCRATCH_BYTES (8u << 20)

/* Limits of [V2] (kNumMaxRanks, kNumMaxExperts, kNumMaxExpertsPerRank)
 * and this library's own top-k and hidden-size limits (a row of H bf16
 * must fit the launch grid: 2^24 channels is a 32 MiB row). */
#define EP_MAX_RANKS 1024
#define EP_MAX_EXPERTS 2048
#define EP_MAX_EXPERTS_PER_RANK 256
#define EP_MAX_TOPK 32
#define EP_MAX_HIDDEN (1 << 24)

/* Problem description shared by all calls.  Valid when:
 *   T >= 0; H >= 8 and H % 8 == 0 (rows are whole 16-byte vectors);
 *   1 <= E <= 2048; 1 <= R <= 1024; E % R == 0; E / R <= 256;
 *   1 <= G and R % G == 0; 1 <= K <= 32; A >= 1;
 *   S >= 1; R * S <= INT32_MAX (slots are int32);
 *   T * K + E * A <= INT32_MAX - 65536 (entry and token indices stay int32
 *   with room for the kernels' tiles to run past the end before clamping);
 *   ceil(T / floor(1024 / K)) * round_up(E + R + G + 1, 64) < 2^30 (the
 *   layout's table of per-chunk counts is addressed with 32-bit byte
 *   offsets; this binds only past about 2.6e8 entries at E = 2048,
 *   R = G = 1024, and never at E <= 256 with R <= 64). */
typedef struct ep_problem {
    int32_t num_tokens;       /* T: tokens of this source rank */
    int32_t hidden;           /* H: bf16 elements per row, a multiple of 8, <= EP_MAX_HIDDEN */
    int32_t num_experts;      /* E */
    int32_t num_topk;         /* K */
    int32_t num_ranks;        /* R: destination ranks (slices) */
    int32_t num_groups;       /* G: scale-out groups, 1 unless hierarchical */
    int32_t expert_alignment; /* A: segment starts are multiples of A ([SYM] §6.1) */
    int32_t reserved;         /* must be 0 */
    int64_t rank_stride_rows; /* S: rows per rank slice, the same for every rank */
} ep_problem;

/* Bytes of device workspace ep_get_layout needs for this problem (chunk
 * count tables and the status word), or 0 if the problem is invalid.  The
 * workspace must be 256-byte aligned; its contents need no initialisation. */
size_t ep_workspace_bytes(const ep_problem *problem);

/* Worst-case rows one source rank can put in one slice, ignoring
 * problem->rank_stride_rows: T * min(K, L) + L * (A - 1).  The analogue of
 * sizing the buffer from num_max_tokens_per_rank ([SYM] §9.1, §9.5
 * get_buffer_size_hint).  Returns -1 if the problem is otherwise invalid. */
int64_t ep_rank_stride_hint(const ep_problem *problem);

/* Routing layout: the counts, prefix sums and per-entry destination slots
 * that [SYM] §6.1 passes to the dispatch kernel (per-scale-up-rank and
 * per-expert prefix sums, unaligned per-expert counts, dst_buffer_slot_idx)
 * and that [SYM] §7.3 reads back per rank and per local expert.
 *
 * Input:
 *   topk_idx [T,K] int32 device, row-major; -1 marks an empty entry.
 * Outputs (device, caller-allocated, fully overwritten):
 *   expert_count      [E] int32  rows routed to each expert (the unaligned
 *                                per-expert receive count)
 *   expert_offset     [E] int32  first row of expert e's segment inside slice
 *                                rank(e): sum over lower local experts of the
 *                                same rank of align_up(expert_count, A)
 *   rank_row_count    [R] int32  expanded rows per rank (sum of its experts'
 *                                counts; all of them sum to the number of
 *                                valid entries)
 *   rank_token_count  [R] int32  tokens with at least one entry on the rank
 *   group_token_count [G] int32  tokens with at least one entry in the group
 *                                ([V1] §3.2 groups ranks by eight); may be NULL
 *   is_token_in_rank  [T,R] uint8 1 if token t has an entry on rank r, else 0
 *   token_slot        [T,K] int32 destination row of entry (t,j) in the
 *                                [R*S,H] receive buffer: rank(e)*S +
 *                                expert_offset[e] + (number of earlier entries,
 *                                token-major, naming the same expert); -1 for
 *                                empty or invalid ids and for rows at or past
 *                                S inside their slice.  This is the handle
 *                                ep_dispatch and ep_combine take ([SYM] §9.2).
 *                                Reusing it for later dispatch/combine calls
 *                                without a new layout is the cached mode of
 *                                [SYM] §6.1 (cached_mode).
 *   cumulative_expert_recv [E] int64, or NULL: expert_count is added to it
 *                                (the cumulative per-expert receive
 *                                statistics of [SYM] §6.1); the caller
 *                                zeroes it once.  8-byte aligned.
 *   workspace         ep_workspace_bytes(problem) bytes, device.
 * Device-detected errors (read with ep_read_status): an id outside [0,E)
 * other than -1 gives EP_ERR_BAD_EXPERT and is treated as empty; a rank whose
 * aligned rows exceed S gives EP_ERR_CAPACITY and its excess rows get slot -1.
 * The bad-id error is reported in preference to the capacity error.  Each
 * call overwrites the status. */
int ep_get_layout(const ep_problem *problem, const int32_t *topk_idx,
                  int32_t *expert_count, int32_t *expert_offset,
                  int32_t *rank_row_count, int32_t *rank_token_count,
                  int32_t *group_token_count, uint8_t *is_token_in_rank,
                  int32_t *token_slot, int64_t *cumulative_expert_recv,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Dispatch: recv_x[token_slot[t,j], :] = x[t, :] (bit copy), plus
 * recv_src_token[slot] = t and recv_weight[slot] = topk_weights[t,j] — the
 * hidden row, source token index and top-k weight that the received token
 * record of [V2] (TokenLayout block) carries; [SYM] §6.1 lists x,
 * topk_weights and dst_buffer_slot_idx among the dispatch arguments.
 *
 *   x              [T,H] bf16 (raw uint16) device, 16-byte aligned
 *   topk_weights   [T,K] fp32 device, or NULL (every weight is 1)
 *   token_slot     [T,K] int32 device, from ep_get_layout
 *   recv_x         [R*S,H] bf16 device, 16-byte aligned
 *   recv_src_token [R*S] int32 device, or NULL (not written)
 *   recv_weight    [R*S] fp32 device, or NULL (not written)
 * Slots outside [0, R*S) are skipped.  Rows that no slot names (alignment
 * padding, unused capacity) are left untouched. */
int ep_dispatch(const ep_problem *problem, const uint16_t *x,
                const float *topk_weights, const int32_t *token_slot,
                uint16_t *recv_x, int32_t *recv_src_token, float *recv_weight,
                void *stream);

/* Layout then dispatch in one call: the effect of ep_get_layout followed by
 * ep_dispatch on the same stream, with the arguments, outputs, errors and
 * status of both.  [SYM] §6.1 feeds the layout's prefix sums and slots
 * straight into the dispatch launch; here, when the batch is small enough
 * for four layout chunks of 1024 entries (T*K <= 4096 after rounding to
 * whole tokens: decode-sized batches; three chunks when R > 64), both run
 * as a single kernel in which every dispatching workgroup derives its own
 * token's slots, which saves a launch on the latency-bound path.  Batches of
 * up to 128 chunks with expert_alignment 1 run the count pass and then one
 * kernel that finishes the layout while each dispatching workgroup derives
 * its token's slots from per-chunk counts (two launches instead of three);
 * other batches run the two calls' kernels.
 * token_slot is written as ep_get_layout writes it. */
int ep_layout_dispatch(const ep_problem *problem, const int32_t *topk_idx,
                       int32_t *expert_count, int32_t *expert_offset,
                       int32_t *rank_row_count, int32_t *rank_token_count,
                       int32_t *group_token_count, uint8_t *is_token_in_rank,
                       int32_t *token_slot, int64_t *cumulative_expert_recv,
                       void *workspace, size_t workspace_bytes,
                       const uint16_t *x, const float *topk_weights,
                       uint16_t *recv_x, int32_t *recv_src_token,
                       float *recv_weight, void *stream);

/* ep_layout_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The layout's scratch lives in a static
 * device array of EP_NOALLOC_SCRATCH_BYTES (8 MiB) inside the library, one
 * copy per device, held until the process ends; the call itself allocates
 * and frees nothing.  The status word goes to the caller's `status` (one
 * int32, device, 4-byte aligned; read it with ep_read_status(status,
 * stream)); every other argument, output, error and status is that of
 * ep_layout_dispatch, and the results are identical.
 *
 * Limits: a problem whose workspace (ep_workspace_bytes) exceeds
 * EP_NOALLOC_SCRATCH_BYTES is refused with EP_ERR_SCRATCH_LIMIT before
 * anything is enqueued.  That covers, e.g., 128 chunks of 1024 entries at
 * the largest E, R and G, and over two million entries at E = 256, R = 16.
 * The scratch of the current device is used, and the stream must belong to
 * that device (else EP_ERR_INVALID_ARG).  Every call on a device shares that
 * device's scratch: calls that overlap on one device (on different streams,
 * or from different host threads without ordering) race and give wrong
 * results.  Calls in order on one stream are safe; the scratch keeps the
 * last call's contents, and each call rewrites what it reads, so nothing
 * needs clearing between calls. */
int ep_layout_dispatch_noalloc(const ep_problem *problem, const int32_t *topk_idx,
                               int32_t *expert_count, int32_t *expert_offset,
                               int32_t *rank_row_count, int32_t *rank_token_count,
                               int32_t *group_token_count, uint8_t *is_token_in_rank,
                               int32_t *token_slot, int64_t *cumulative_expert_recv,
                               int32_t *status, const uint16_t *x, const float *topk_weights,
                               uint16_t *recv_x, int32_t *recv_src_token, float *recv_weight,
                               void *stream);

/* Combine: out[t,h] = bf16(sum_{j<K} w[t,j] * y[token_slot[t,j], h]), with an
 * fp32 accumulator folded in ascending j by fused multiply-add and one
 * round-to-nearest-even to bf16 — the top-k-weighted reduction that [SYM]
 * §9.2's combine(x, handle, topk_weights) performs back into token order.
 *
 *   y            [R*S,H] bf16 device (expert outputs in the receive layout),
 *                16-byte aligned
 *   token_slot   [T,K] int32 device, from ep_get_layout
 *   topk_weights [T,K] fp32 device, or NULL (unit weights)
 *   out          [T,H] bf16 device, 16-byte aligned
 * Slots outside [0, R*S) contribute nothing; a token with no valid slot
 * gets zeros. */
int ep_combine(const ep_problem *problem, const uint16_t *y,
               const int32_t *token_slot, const float *topk_weights,
               uint16_t *out, void *stream);

/* FP8 (e4m3) quantisation of token rows for FP8 dispatch: one fp32 scale per
 * token and block of 128 channels, sf = amax / 448, codes = the nearest e4m3
 * value (OCP "fn": bias 7, 3 mantissa bits, largest 448; ties to even,
 * larger magnitudes saturate) of x * (448 / amax), all in fp32; an all-zero
 * block gets sf = 0 and zero codes.  The pages show FP8 dispatch with scale
 * factors ([SYM] §6.1 sf arguments, §9.2 use_fp8_dispatch) but not the
 * quantisation rule; this is the reading taken.  Requires H % 128 == 0.
 *
 *   x      [T,H] bf16 device, 16-byte aligned
 *   x_fp8  [T,H] uint8 device (e4m3 codes), 16-byte aligned
 *   x_sf   [T,H/128] fp32 device, token-major */
int ep_quantize_fp8(const ep_problem *problem, const uint16_t *x, uint8_t *x_fp8,
                    float *x_sf, void *stream);

/* FP8 dispatch: as ep_dispatch, with rows of H e4m3 bytes and each row's
 * H/128 scale factors ([SYM] §6.1: sf, sf_token_stride, sf_hidden_stride).
 * The scale of received row r and channel block b goes to
 * recv_sf[r * sf_token_stride + b * sf_hidden_stride]: token-major is
 * (H/128, 1); the TMA-aligned column-major layout of [V2] (elastic.py block)
 * is (1, R*S rounded up to the alignment).  recv_sf must hold
 * (R*S-1)*sf_token_stride + (H/128-1)*sf_hidden_stride + 1 floats.
 * Requires H % 128 == 0 and strides >= 1.
 * Token-major rows padded to whole 128-byte lines (sf_hidden_stride 1,
 * sf_token_stride = H/128 rounded up to a multiple of 32, larger than H/128)
 * are written whole: entries H/128 .. sf_token_stride-1 of every received
 * row except the last row of recv_sf (R*S-1) are set to 0.  With recv_sf
 * 128-byte aligned, no line of the scales is then written in parts by
 * different workgroups, which is the faster layout for large batches.
 *
 *   x_fp8        [T,H] uint8 device, 16-byte aligned
 *   x_sf         [T,H/128] fp32 device, token-major
 *   topk_weights [T,K] fp32 device, or NULL (every weight is 1)
 *   token_slot   [T,K] int32 device, from ep_get_layout
 *   recv_x_fp8   [R*S,H] uint8 device, 16-byte aligned
 *   recv_sf      fp32 device, see above
 *   recv_src_token, recv_weight: as in ep_dispatch (may be NULL) */
int ep_dispatch_fp8(const ep_problem *problem, const uint8_t *x_fp8, const float *x_sf,
                    const float *topk_weights, const int32_t *token_slot,
                    uint8_t *recv_x_fp8, float *recv_sf, int64_t sf_token_stride,
                    int64_t sf_hidden_stride, int32_t *recv_src_token, float *recv_weight,
                    void *stream);

/* FP8 layout then dispatch in one call: ep_get_layout followed by
 * ep_dispatch_fp8, with the arguments, outputs, errors and status of both;
 * one kernel up to four layout chunks, as for ep_layout_dispatch
 * (decode-sized batches, where [SYM] §9.2's use_fp8_dispatch matters most
 * for latency). */
int ep_layout_dispatch_fp8(const ep_problem *problem, const int32_t *topk_idx,
                           int32_t *expert_count, int32_t *expert_offset,
                           int32_t *rank_row_count, int32_t *rank_token_count,
                           int32_t *group_token_count, uint8_t *is_token_in_rank,
                           int32_t *token_slot, int64_t *cumulative_expert_recv,
                           void *workspace, size_t workspace_bytes,
                           const uint8_t *x_fp8, const float *x_sf, const float *topk_weights,
                           uint8_t *recv_x_fp8, float *recv_sf, int64_t sf_token_stride,
                           int64_t sf_hidden_stride, int32_t *recv_src_token,
                           float *recv_weight, void *stream);

/* Two-level (hierarchical) path for G > 1 scale-out groups of R/G ranks:
 * "DeepEP V2 ElasticBuffer 架构深度分析" (hybrid dispatch selected when there
 * is more than one scale-out rank; logical topology block) and [V1] §3.2
 * (ranks grouped by eight) show a dispatch that sends each token once to
 * every group it needs and expands it inside the group.  Here the group
 * stage goes through a group buffer of G slices of SG rows ([G*SG, H] bf16):
 * a token's row in group g is group_slot[t,g] = g*SG + (number of earlier
 * tokens reaching group g), or -1 if it does not reach g (or would sit at or
 * past SG).  The group of entry (t,j) is (token_slot[t,j] / S) / (R/G).
 * Requires SG >= 1 and G*SG <= INT32_MAX.
 *
 * ep_get_group_layout: group_slot [T,G] int32 from is_token_in_rank [T,R]
 *   (an output of ep_get_layout).  SG = T never drops a token.  status: NULL,
 *   or one int32 on the device, 4-byte aligned (typically the layout's
 *   workspace, whose first word is the status ep_read_status returns): when
 *   some group is reached by more than SG tokens, it is lowered to
 *   EP_ERR_CAPACITY unless it already holds a lower code (EP_ERR_BAD_EXPERT
 *   stays); it is never raised or cleared, so a standalone word must be set
 *   to EP_OK first.
 * ep_dispatch_hier: x -> group_buf (one row per token and group), then each
 *   entry's row is copied from its group's row into recv_x; recv_src_token
 *   and recv_weight as in ep_dispatch.  recv_x ends up identical to
 *   ep_dispatch's when no group row was dropped.  An entry whose group row
 *   was dropped (group_slot -1 for its group although the token has an entry
 *   there) gets recv_src_token -1 and recv_weight 0, and its row of recv_x is
 *   not written; ep_combine_hier leaves such entries out.
 * ep_combine_hier: per (token, group) the partial sum over the token's
 *   entries in that group, folded in fp32 with FMA in ascending j and rounded
 *   to bf16 into the group row (the value that would cross the scale-out
 *   link); then out[t] = bf16(sum of its group rows), fp32 accumulate.
 *   group_buf is overwritten. */
int ep_get_group_layout(const ep_problem *problem, const uint8_t *is_token_in_rank,
                        int64_t group_stride_rows, int32_t *group_slot, int32_t *status,
                        void *stream);
int ep_dispatch_hier(const ep_problem *problem, const uint16_t *x, const float *topk_weights,
                     const int32_t *token_slot, const int32_t *group_slot,
                     int64_t group_stride_rows, uint16_t *group_buf, uint16_t *recv_x,
                     int32_t *recv_src_token, float *recv_weight, void *stream);
int ep_combine_hier(const ep_problem *problem, const uint16_t *y, const int32_t *token_slot,
                    const float *topk_weights, const int32_t *group_slot,
                    int64_t group_stride_rows, uint16_t *group_buf, uint16_t *out,
                    void *stream);

/* Combined top-k weights: combined_topk_weights[t,j] = recv_weight[token_slot[t,j]]
 * (0 for slots outside [0, R*S)) — the per-row weights that travelled with
 * the dispatched rows, gathered back into token order, as combine returns
 * combined_topk_weights beside combined_x in [SYM] §9.2.  After ep_dispatch
 * with weights it reproduces topk_weights exactly.
 *
 *   recv_weight           [R*S] fp32 device (ep_dispatch's recv_weight)
 *   token_slot            [T,K] int32 device
 *   combined_topk_weights [T,K] fp32 device, written */
int ep_combine_topk_weights(const ep_problem *problem, const float *recv_weight,
                            const int32_t *token_slot, float *combined_topk_weights,
                            void *stream);

/* Synchronises `stream`, then returns the status word the last
 * ep_get_layout on that workspace wrote (EP_OK, EP_ERR_BAD_EXPERT or
 * EP_ERR_CAPACITY), or EP_ERR_HIP / EP_ERR_INVALID_ARG if it cannot read it. */
int ep_read_status(const void *workspace, void *stream);

/* Static, human-readable name of an EP_* code. */
const char *ep_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* EP_GET_H */
