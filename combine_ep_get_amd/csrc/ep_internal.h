// Internal declarations shared by the HIP translation units of libepget.
// Not part of the public ABI (that is include/ep_get.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epget {

// Entries (token, top-k pairs) per layout chunk.  One wave walks a chunk in
// 64-entry steps when it assigns slots, and the count tables hold one row per
// chunk, so this trades slot-walk latency against scan-table size.
constexpr int kChunkEntries = 1024;
// Largest batch (T * K entries) that the one-call layout and dispatch runs
// as a single kernel, every dispatching workgroup taking the whole batch's
// histogram: a few chunks.
constexpr int kFusedMaxEntries = 4 * kChunkEntries;

// Workspace layout, all offsets in bytes from the workspace base:
//   [0, 256)                  status word (int32) + padding
//   [256, 256 + pitch*4)      column totals of the chunk table
//   [table_off, ...)          chunk table: nchunks rows x pitch int32
//   [count_t_off, ...)        E x nchunks int32: per-chunk expert counts,
//                             expert-major (one-call layout and dispatch)
//   [excl_t_off, ...)         E x nchunks int32: per-chunk counts of the
//                             lower experts of the same rank, expert-major
// Columns of the chunk table: E experts | R ranks | G groups | 1 bad-id count.
struct WsLayout {
    int64_t nchunks;      // >= 1
    int32_t chunk_tokens; // tokens per chunk
    int32_t ncols;        // E + R + G + 1
    int32_t pitch;        // ncols rounded up to a multiple of 64
    int64_t totals_off;
    int64_t table_off;
    int64_t count_t_off, excl_t_off;
    int64_t bytes;
};

WsLayout ws_layout(int32_t T, int32_t K, int32_t E, int32_t R, int32_t G);

// Division by a runtime divisor d <= 1024 of dividends n < 2^22 as a
// multiply-high with m = ceil(2^32 / d); exact on that whole range (checked
// exhaustively), and a handful of instructions instead of the generic
// reciprocal-and-correct sequence.
struct FastDiv {
    uint64_t m;
    static FastDiv make(uint32_t d) { return FastDiv{((1ull << 32) + d - 1) / d}; }
    __device__ __forceinline__ uint32_t operator()(uint32_t n) const {
        return static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> 32);
    }
};

struct LayoutParams {
    const int32_t *topk_idx;
    int32_t T, K, E, R, G, A, L, ranks_per_group;
    FastDiv div_L;
    int32_t S;
    int32_t chunk_tokens, nchunks, ncols, pitch, nbits;
    int32_t *expert_count, *expert_offset, *rank_row_count, *rank_token_count;
    int32_t *group_token_count;  // may be null
    uint8_t *is_token_in_rank;
    int32_t *token_slot;
    int64_t *cumulative;  // may be null
    int32_t *status, *totals, *table;
    // expert-major per-chunk counts and in-rank exclusive prefixes; the count
    // pass fills them only when non-null (the one-call multi-chunk path)
    int32_t *count_t, *excl_t;
};

struct CopyParams {
    int32_t T, H, K;
    int32_t nvec;      // 16-byte vectors per row (H / 8 for bf16, H / 16 for fp8)
    int32_t vpt;       // vectors per thread (<= kMaxVpt)
    int64_t num_rows;  // R * S
};

// Pointers of one dispatch.  Rows are moved as 16-byte vectors whatever
// their element type; x_sf / recv_sf are the optional per-row scale factors
// (nsf per row; element (row, b) of recv_sf at row * sf_ts + b * sf_hs).
// sf_row entries are written per received row: nsf, or the whole padded row
// (its entries past nsf as 0) when the rows are padded to whole 128-byte
// lines; the last row of recv_sf never takes the padding.
struct DispatchArgs {
    const void *x;
    const float *w;
    const int32_t *slot;
    void *recv;
    int32_t *recv_src;
    float *recv_w;
    const float *x_sf;
    float *recv_sf;
    int64_t sf_ts, sf_hs;
    int32_t nsf, sf_row;
};

constexpr int kCopyThreads = 128;      // dispatch workgroup size
constexpr int kFusedThreads = 256;     // workgroup of the single-kernel layout + dispatch
constexpr int kMaxVpt = 8;            // dispatch vectors per thread
constexpr int kCombineMaxThreads = 1024;

hipError_t launch_layout(const LayoutParams &p, hipStream_t stream);
hipError_t launch_dispatch(const CopyParams &c, const DispatchArgs &a, hipStream_t stream);
// launch_layout then launch_dispatch, as one kernel when the batch is one
// layout chunk.
hipError_t launch_layout_dispatch(const LayoutParams &p, const CopyParams &c, const DispatchArgs &a,
                                  hipStream_t stream);
hipError_t launch_quantize_fp8(int32_t T, int32_t H, const uint16_t *x, uint8_t *q, float *sf,
                               hipStream_t stream);
hipError_t launch_combine(const CopyParams &c, const uint16_t *y, const int32_t *slot,
                          const float *w, uint16_t *out, hipStream_t stream);
hipError_t launch_combine_weights(const CopyParams &c, const float *recv_w, const int32_t *slot,
                                  float *combined_w, hipStream_t stream);

// Grid shape for the row kernels with workgroups of `threads`: (tokens,
// column splits) and vectors per thread, chosen so that small batches still
// spread over about `want` workgroups.
constexpr int kCopyWorkgroups = 2048;   // 8 per CU
constexpr int kFusedWorkgroups = 1024;  // the single-kernel layout + dispatch
void copy_grid(int32_t T, int32_t nvec, int32_t threads, int32_t *splits, int32_t *vpt,
               int32_t want = kCopyWorkgroups);
// Grid of the combine: (tokens, row pieces) and threads per workgroup (one
// 16-byte column vector per thread).
void combine_grid(int32_t T, int32_t nvec, int32_t *splits, int32_t *threads);

}  // namespace epget
