// Routing layout kernels for gfx950 (wave64).
//
// Computes, for one source rank, the per-expert / per-rank / per-group counts,
// the token-to-rank map, the aligned within-slice expert offsets and the
// destination slot of every (token, top-k) entry — the quantities that the
// dispatch launch of "DeepEP Symmetric Memory 全面架构分析" §6.1 receives
// (per-rank and per-expert prefix sums, unaligned per-expert counts,
// expert_alignment, dst_buffer_slot_idx) and that its §7.3 reads back.
//
// Slot order is deterministic: inside each expert segment rows are in
// ascending token, then ascending top-k position.  No atomic decides an
// order; LDS atomics only form counts, and positions come from a two-pass
// scan plus a wave64 ballot match inside each 64-entry step.
//
// Multi-chunk path (three launches):
//   1. count: one workgroup per chunk of entries builds an LDS histogram of
//      [experts | ranks | groups | bad ids] and writes one table row;
//   2. scan:  per 64-column tile, 16 waves split the chunk rows, sum them,
//      combine partial sums in LDS and rewrite the table in place as
//      exclusive per-chunk bases; column totals go to the count outputs;
//   3. slot:  one wave per chunk derives the expert offsets from the totals
//      (wave scan), seeds an LDS cursor per expert with offset + chunk base
//      and walks the chunk in 64-entry steps.
// Single-chunk path (one launch): the same steps inside one workgroup, with
// the histogram itself as the totals.
#include "../../include/ep_get.h"
#include "ep_internal.h"

namespace epget {
namespace {

__device__ __forceinline__ bool valid_id(int32_t e, int32_t E) {
    return static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
}

__device__ __forceinline__ int32_t align_up(int32_t v, int32_t a) { return (v + a - 1) / a * a; }

// Chunk histogram into LDS.  Called by the whole workgroup; ends with a
// barrier.  s_hist: pitch ints; s_idx: the chunk's ids (loaded here).
// Also writes the chunk's rows of is_token_in_rank.
__device__ void chunk_histogram(const LayoutParams &p, int t0, int t1, int *s_hist, int *s_idx) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n = (t1 - t0) * p.K;
    for (int i = tid; i < p.ncols; i += nt) s_hist[i] = 0;
    const int32_t *src = p.topk_idx + static_cast<int64_t>(t0) * p.K;
    for (int i = tid; i < n; i += nt) s_idx[i] = src[i];
    __syncthreads();

    const int bad_col = p.E + p.R + p.G;
    for (int i = tid; i < n; i += nt) {
        const int e = s_idx[i];
        if (e == -1) continue;
        atomicAdd(&s_hist[valid_id(e, p.E) ? e : bad_col], 1);
    }
    // token-to-rank map (one byte per (token, rank)) and unique tokens per rank
    const int nr = (t1 - t0) * p.R;
    uint8_t *map = p.is_token_in_rank + static_cast<int64_t>(t0) * p.R;
    for (int i = tid; i < nr; i += nt) {
        const int tl = i / p.R, r = i - tl * p.R;
        const int *ids = s_idx + tl * p.K;
        int in = 0;
        for (int j = 0; j < p.K; ++j) {
            const int e = ids[j];
            in |= valid_id(e, p.E) && e / p.L == r;
        }
        map[i] = static_cast<uint8_t>(in);
        if (in) atomicAdd(&s_hist[p.E + r], 1);
    }
    // unique tokens per group
    const int ng = (t1 - t0) * p.G;
    for (int i = tid; i < ng; i += nt) {
        const int tl = i / p.G, g = i - tl * p.G;
        const int *ids = s_idx + tl * p.K;
        int in = 0;
        for (int j = 0; j < p.K; ++j) {
            const int e = ids[j];
            in |= valid_id(e, p.E) && (e / p.L) / p.ranks_per_group == g;
        }
        if (in) atomicAdd(&s_hist[p.E + p.R + g], 1);
    }
    __syncthreads();
}

// Exclusive scans over all experts of the aligned and raw counts, by one
// wave: each lane sums a contiguous run of experts, a shuffle scan combines
// the lanes.  s_aln / s_raw get E+1 entries (the last one is the total).
__device__ void wave_scan_counts(const LayoutParams &p, const int32_t *counts, int *s_aln, int *s_raw) {
    const int lane = __lane_id();
    const int per = (p.E + 63) / 64;
    const int e0 = min(p.E, lane * per), e1 = min(p.E, e0 + per);
    int sa = 0, sr = 0;
    for (int e = e0; e < e1; ++e) {
        const int c = counts[e];
        sa += align_up(c, p.A);
        sr += c;
    }
    int ia = sa, ir = sr;
    for (int d = 1; d < 64; d <<= 1) {
        const int ta = __shfl_up(ia, d, 64), tr = __shfl_up(ir, d, 64);
        if (lane >= d) { ia += ta; ir += tr; }
    }
    int ea = ia - sa, er = ir - sr;
    for (int e = e0; e < e1; ++e) {
        const int c = counts[e];
        s_aln[e] = ea;
        s_raw[e] = er;
        ea += align_up(c, p.A);
        er += c;
    }
    if (lane == 63) { s_aln[p.E] = ia; s_raw[p.E] = ir; }
}

// Per-rank results from the scans (rank_row_count, capacity check).  Called by
// `nt` threads with index `tid`; returns nonzero if any of this thread's ranks
// overflows its slice.
__device__ int finish_ranks(const LayoutParams &p, const int *s_aln, const int *s_raw, int tid, int nt) {
    int over = 0;
    for (int r = tid; r < p.R; r += nt) {
        const int lo = r * p.L, hi = lo + p.L;
        p.rank_row_count[r] = s_raw[hi] - s_raw[lo];
        over |= (s_aln[hi] - s_aln[lo]) > p.S;
    }
    return over;
}

__device__ __forceinline__ int32_t status_code(int bad, int over) {
    return bad ? EP_ERR_BAD_EXPERT : (over ? EP_ERR_CAPACITY : EP_OK);
}

// Slot assignment for entries [t0*K, t1*K) by one wave, in 64-entry steps.
// s_cur[e] holds the next free row of expert e inside its slice; s_idx holds
// the chunk's ids.  Within a step, lanes naming the same expert are found by
// matching the id bit by bit with ballots; each takes the cursor plus the
// number of matching lanes below it, and the lowest of them advances the
// cursor.  One wave's LDS accesses complete in issue order, so every lane
// reads the cursor before the update lands.
__device__ void wave_assign_slots(const LayoutParams &p, int t0, int t1, int *s_cur, const int *s_idx) {
    const int lane = __lane_id();
    const int64_t first = static_cast<int64_t>(t0) * p.K;
    const int n = (t1 - t0) * p.K;
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        const bool act = i < n;
        const int e = act ? s_idx[i] : -1;
        const bool ok = act && valid_id(e, p.E);
        uint64_t same = __ballot(ok);
        for (int b = 0; b < p.nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t set = __ballot(ok && bit);
            same &= bit ? set : ~set;
        }
        const uint64_t below = same & lanes_below;
        int cur = 0;
        if (ok) cur = s_cur[e];
        if (ok && below == 0) s_cur[e] = cur + __popcll(same);
        if (act) {
            int slot = -1;
            if (ok) {
                const int pos = cur + __popcll(below);
                if (pos < p.S) slot = (e / p.L) * p.S + pos;
            }
            p.token_slot[first + i] = slot;
        }
    }
}

__global__ __launch_bounds__(256) void layout_count_kernel(LayoutParams p) {
    extern __shared__ int smem[];
    int *s_hist = smem;
    int *s_idx = smem + p.pitch;
    const int c = blockIdx.x;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    chunk_histogram(p, t0, t1, s_hist, s_idx);
    int32_t *row = p.table + static_cast<int64_t>(c) * p.pitch;
    for (int i = threadIdx.x; i < p.ncols; i += blockDim.x) row[i] = s_hist[i];
}

constexpr int kScanWaves = 16;

__global__ __launch_bounds__(64 * kScanWaves) void layout_scan_kernel(LayoutParams p) {
    __shared__ int s_part[kScanWaves][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;
    const int per = (p.nchunks + kScanWaves - 1) / kScanWaves;
    const int c0 = min(p.nchunks, w * per), c1 = min(p.nchunks, c0 + per);
    const bool live = col < p.ncols;
    int sum = 0;
    if (live) {
#pragma unroll 8
        for (int c = c0; c < c1; ++c) sum += p.table[static_cast<int64_t>(c) * p.pitch + col];
    }
    s_part[w][lane] = sum;
    __syncthreads();
    int base = 0, total = 0;
    for (int i = 0; i < kScanWaves; ++i) {
        const int v = s_part[i][lane];
        base += i < w ? v : 0;
        total += v;
    }
    if (!live) return;
    int run = base;
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
        int32_t *q = p.table + static_cast<int64_t>(c) * p.pitch + col;
        const int v = *q;
        *q = run;
        run += v;
    }
    if (w == 0) {
        p.totals[col] = total;
        if (col < p.E) {
            p.expert_count[col] = total;
        } else if (col < p.E + p.R) {
            p.rank_token_count[col - p.E] = total;
        } else if (col < p.E + p.R + p.G) {
            if (p.group_token_count) p.group_token_count[col - p.E - p.R] = total;
        }
    }
}

__global__ __launch_bounds__(64) void layout_slot_kernel(LayoutParams p) {
    extern __shared__ int smem[];
    int *s_aln = smem;
    int *s_raw = s_aln + (p.E + 1);
    int *s_cur = s_raw + (p.E + 1);
    int *s_idx = s_cur + p.E;
    const int lane = threadIdx.x;
    const int c = blockIdx.x;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    const int n = (t1 - t0) * p.K;
    const int32_t *src = p.topk_idx + static_cast<int64_t>(t0) * p.K;
    for (int i = lane; i < n; i += 64) s_idx[i] = src[i];
    wave_scan_counts(p, p.expert_count, s_aln, s_raw);
    __syncthreads();
    const int32_t *chunk_base = p.table + static_cast<int64_t>(c) * p.pitch;
    for (int e = lane; e < p.E; e += 64) {
        const int off = s_aln[e] - s_aln[(e / p.L) * p.L];
        s_cur[e] = off + chunk_base[e];
        if (c == 0) p.expert_offset[e] = off;
    }
    if (c == 0) {
        const int over = finish_ranks(p, s_aln, s_raw, lane, 64);
        const bool any_over = __ballot(over) != 0;
        if (lane == 0) *p.status = status_code(p.totals[p.E + p.R + p.G] > 0, any_over);
    }
    __syncthreads();
    wave_assign_slots(p, t0, t1, s_cur, s_idx);
}

__global__ __launch_bounds__(256) void layout_single_kernel(LayoutParams p) {
    extern __shared__ int smem[];
    __shared__ int s_over;
    const int idx_cap = kChunkEntries + 64;
    int *s_hist = smem;
    int *s_idx = s_hist + p.pitch;
    int *s_aln = s_idx + idx_cap;
    int *s_raw = s_aln + (p.E + 1);
    int *s_cur = s_raw + (p.E + 1);
    const int tid = threadIdx.x, nt = blockDim.x;
    if (tid == 0) s_over = 0;
    chunk_histogram(p, 0, p.T, s_hist, s_idx);
    for (int i = tid; i < p.E + p.R + p.G; i += nt) {
        const int v = s_hist[i];
        if (i < p.E) {
            p.expert_count[i] = v;
        } else if (i < p.E + p.R) {
            p.rank_token_count[i - p.E] = v;
        } else if (p.group_token_count) {
            p.group_token_count[i - p.E - p.R] = v;
        }
    }
    if (tid < 64) wave_scan_counts(p, s_hist, s_aln, s_raw);
    __syncthreads();
    for (int e = tid; e < p.E; e += nt) {
        const int off = s_aln[e] - s_aln[(e / p.L) * p.L];
        s_cur[e] = off;
        p.expert_offset[e] = off;
    }
    if (finish_ranks(p, s_aln, s_raw, tid, nt)) atomicOr(&s_over, 1);
    __syncthreads();
    if (tid == 0) *p.status = status_code(s_hist[p.E + p.R + p.G] > 0, s_over);
    if (tid < 64) wave_assign_slots(p, 0, p.T, s_cur, s_idx);
}

}  // namespace

WsLayout ws_layout(int32_t T, int32_t K, int32_t E, int32_t R, int32_t G) {
    WsLayout w;
    w.chunk_tokens = kChunkEntries / K > 0 ? kChunkEntries / K : 1;
    const int64_t n = (static_cast<int64_t>(T) + w.chunk_tokens - 1) / w.chunk_tokens;
    w.nchunks = n > 0 ? n : 1;
    w.ncols = E + R + G + 1;
    w.pitch = (w.ncols + 63) / 64 * 64;
    w.totals_off = 256;
    w.table_off = w.totals_off + (static_cast<int64_t>(w.pitch) * 4 + 255) / 256 * 256;
    w.bytes = w.table_off + w.nchunks * w.pitch * 4;
    return w;
}

hipError_t launch_layout(const LayoutParams &p, hipStream_t stream) {
    if (p.nchunks == 1) {
        const size_t lds = sizeof(int) * (p.pitch + (kChunkEntries + 64) + 2 * (p.E + 1) + p.E);
        layout_single_kernel<<<1, 256, lds, stream>>>(p);
        return hipGetLastError();
    }
    const size_t lds_count = sizeof(int) * (p.pitch + p.chunk_tokens * p.K);
    layout_count_kernel<<<p.nchunks, 256, lds_count, stream>>>(p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    layout_scan_kernel<<<p.pitch / 64, 64 * kScanWaves, 0, stream>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds_slot = sizeof(int) * (2 * (p.E + 1) + p.E + p.chunk_tokens * p.K);
    layout_slot_kernel<<<p.nchunks, 64, lds_slot, stream>>>(p);
    return hipGetLastError();
}

}  // namespace epget
