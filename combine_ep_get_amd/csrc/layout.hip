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
//   3. assign: one workgroup per chunk derives the expert offsets from the
//      totals (wave scan), splits the chunk over its four waves with per-wave
//      expert histograms, seeds one LDS cursor per (wave, expert) with
//      offset + chunk base + earlier waves' counts, and each wave walks its
//      part in 64-entry steps.
// Single-chunk path (one launch): the same steps inside one workgroup, with
// the histogram itself as the totals.
// Every global read a step needs is issued as one batch of independent loads
// (indices clamped into range, selects instead of branches), so each step
// costs about one memory round trip.
#include "../../include/ep_get.h"
#include "ep_internal.h"

namespace epget {
namespace {

constexpr int kThreads = 256;                           // count and assign kernels
constexpr int kWaves = kThreads / 64;
constexpr int kIdsPerThread = kChunkEntries / kThreads;  // ids each thread loads
constexpr int kMaxExpertsPerThread = EP_MAX_EXPERTS / kThreads;
constexpr int kScanWaves = 16;
constexpr int kScanPerWave = 8;                         // chunk rows per wave per round

__device__ __forceinline__ bool valid_id(int32_t e, int32_t E) {
    return static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
}

__device__ __forceinline__ int32_t align_up(int32_t v, int32_t a) { return (v + a - 1) / a * a; }

// Raw buffer view of an int32 array of n elements.  A load at an index the
// caller marks invalid reads 0 through the hardware range check of the buffer
// descriptor, so predicated loads need no branch (a select on a loaded value
// would be turned back into a branch around the load).
struct I32Buffer {
    static constexpr int32_t kFlags = 0x00020000;  // gfx9 raw buffer, 32-bit data
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ I32Buffer(const int32_t *base, uint32_t n)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(base), 0, n * 4u, kFlags)) {}
    __device__ int32_t load(uint32_t i, bool valid) const {
        return __builtin_amdgcn_raw_buffer_load_b32(rsrc, valid ? i * 4u : 0xFFFFFFFCu, 0, 0);
    }
};

// Loads the n (<= kChunkEntries) ids at src into s_idx.  Every thread issues
// its kIdsPerThread loads back to back (indices clamped into range, so no
// load sits behind a branch); only the LDS stores are predicated.
__device__ __forceinline__ void load_ids(const int32_t *src, int n, int *s_idx) {
    if (n <= 0) return;
    int v[kIdsPerThread];
#pragma unroll
    for (int k = 0; k < kIdsPerThread; ++k) v[k] = src[min(static_cast<int>(threadIdx.x) + k * kThreads, n - 1)];
#pragma unroll
    for (int k = 0; k < kIdsPerThread; ++k) {
        const int i = threadIdx.x + k * kThreads;
        if (i < n) s_idx[i] = v[k];
    }
}

// Entries per wave when a chunk of n entries is split over the kWaves waves
// (a multiple of 64, so every wave but the last walks whole 64-entry steps).
__device__ __forceinline__ int wave_span(int n) { return (n + kWaves * 64 - 1) / (kWaves * 64) * 64; }

// Entries in LDS are packed after the first pass: (rank << 12) | expert for a
// valid id (expert < 4096, rank < 1024), -1 for an empty or invalid one.
constexpr int kRankShift = 12;
constexpr int kExpertMask = (1 << kRankShift) - 1;

// Histogram of a chunk (raw ids in s_idx, packed in place) into s_hist
// columns [experts | ranks | groups | bad ids], the chunk's rows of
// is_token_in_rank, and (if s_wave is not null) per-wave expert histograms
// for the slot walk.  Contains barriers: call from the whole workgroup.
__device__ void chunk_histogram(const LayoutParams &p, int t0, int t1, int *s_idx,
                                int *s_hist, int *s_wave) {
    const int tid = threadIdx.x;
    const int n = (t1 - t0) * p.K;
    const int span = wave_span(n);
    const int bad_col = p.E + p.R + p.G;
    for (int i = tid; i < n; i += kThreads) {
        const int e = s_idx[i];
        if (e == -1) continue;
        if (!valid_id(e, p.E)) {
            atomicAdd(&s_hist[bad_col], 1);
            s_idx[i] = -1;
            continue;
        }
        atomicAdd(&s_hist[e], 1);
        if (s_wave) atomicAdd(&s_wave[(i / span) * p.E + e], 1);
        s_idx[i] = static_cast<int>(p.div_L(e) << kRankShift) | e;
    }
    __syncthreads();
    // token-to-rank map (one byte per (token, rank)) and unique tokens per rank
    const int nr = (t1 - t0) * p.R;
    uint8_t *map = p.is_token_in_rank + static_cast<int64_t>(t0) * p.R;
    for (int i = tid; i < nr; i += kThreads) {
        const int tl = p.div_R(i), r = i - tl * p.R;
        const int *ids = s_idx + tl * p.K;
        int in = 0;
        for (int j = 0; j < p.K; ++j) in |= (ids[j] >> kRankShift) == r;
        map[i] = static_cast<uint8_t>(in);
        if (in) atomicAdd(&s_hist[p.E + r], 1);
    }
    // unique tokens per group: ranks [g*rpg, (g+1)*rpg)
    const int ng = (t1 - t0) * p.G;
    for (int i = tid; i < ng; i += kThreads) {
        const int tl = p.div_G(i), g = i - tl * p.G;
        const int lo = g * p.ranks_per_group, hi = lo + p.ranks_per_group;
        const int *ids = s_idx + tl * p.K;
        int in = 0;
        for (int j = 0; j < p.K; ++j) {
            const int r = ids[j] >> kRankShift;
            in |= r >= lo && r < hi;
        }
        if (in) atomicAdd(&s_hist[p.E + p.R + g], 1);
    }
}

// Exclusive scans over all experts of the aligned and raw counts, by one
// wave: each lane sums a contiguous run of experts, a shuffle scan combines
// the lanes.  s_aln and s_raw get E+1 entries (the last one is the total).
// `counts` may be the same array as s_raw (each lane reads its run before it
// overwrites it).
__device__ void wave_scan_counts(const LayoutParams &p, const int *counts, int *s_aln, int *s_raw) {
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

// Per-rank results from the scans: rank_row_count and the capacity check.
// Returns nonzero if one of this thread's ranks overflows its slice.
__device__ int finish_ranks(const LayoutParams &p, const int *s_aln, const int *s_raw) {
    int over = 0;
    for (int r = threadIdx.x; r < p.R; r += kThreads) {
        const int lo = r * p.L, hi = lo + p.L;
        p.rank_row_count[r] = s_raw[hi] - s_raw[lo];
        over |= (s_aln[hi] - s_aln[lo]) > p.S;
    }
    return over;
}

__device__ __forceinline__ int32_t status_code(int bad, int over) {
    return bad ? EP_ERR_BAD_EXPERT : (over ? EP_ERR_CAPACITY : EP_OK);
}

// Slot assignment by one wave for entries [i0, i1) of the chunk (packed
// entries in s_idx, global entry index first + i), in 64-entry steps.  s_cur[e] holds
// the next free row of expert e inside its slice.  Within a step, lanes naming
// the same expert are found by matching the id bit by bit with ballots; each
// takes the cursor plus the number of matching lanes below it, and the lowest
// of them advances the cursor.  One wave's LDS accesses complete in issue
// order, so every lane reads the cursor before the update lands.
__device__ void wave_assign_slots(const LayoutParams &p, int64_t first, int i0, int i1,
                                  int *s_cur, const int *s_idx) {
    const int lane = __lane_id();
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    for (int base = i0; base < i1; base += 64) {
        const int i = base + lane;
        const bool act = i < i1;
        const int v = act ? s_idx[i] : -1;
        const bool ok = v >= 0;
        const int e = v & kExpertMask;
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
                if (pos < p.S) slot = (v >> kRankShift) * p.S + pos;
            }
            p.token_slot[first + i] = slot;
        }
    }
}

// Multi-chunk pass 1: one workgroup per chunk writes its histogram row.
__global__ __launch_bounds__(kThreads) void layout_count_kernel(LayoutParams p) {
    extern __shared__ int smem[];
    int *s_idx = smem;
    int *s_hist = smem + kChunkEntries;
    const int c = blockIdx.x;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    load_ids(p.topk_idx + static_cast<int64_t>(t0) * p.K, (t1 - t0) * p.K, s_idx);
    for (int i = threadIdx.x; i < p.ncols; i += kThreads) s_hist[i] = 0;
    __syncthreads();
    chunk_histogram(p, t0, t1, s_idx, s_hist, nullptr);
    __syncthreads();
    int32_t *row = p.table + static_cast<int64_t>(c) * p.pitch;
    for (int i = threadIdx.x; i < p.ncols; i += kThreads) row[i] = s_hist[i];
}

// Multi-chunk pass 2: per 64-column tile, rewrite the table in place as
// exclusive per-chunk bases and write the column totals.  Rounds of
// kScanWaves * kScanPerWave chunk rows; each wave keeps its rows in registers
// so one round costs one load round trip.
__global__ __launch_bounds__(64 * kScanWaves) void layout_scan_kernel(LayoutParams p) {
    __shared__ int s_part[kScanWaves][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;  // < pitch, so loads stay inside the row
    const bool live = col < p.ncols;
    const I32Buffer table(p.table, static_cast<uint32_t>(p.nchunks) * p.pitch);
    int carry = 0;
    for (int cb = 0; cb < p.nchunks; cb += kScanWaves * kScanPerWave) {
        const int c0 = cb + w * kScanPerWave;
        int v[kScanPerWave];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kScanPerWave; ++k) {
            const int c = c0 + k;
            v[k] = table.load(static_cast<uint32_t>(c) * p.pitch + col, live && c < p.nchunks);
            sum += v[k];
        }
        s_part[w][lane] = sum;
        __syncthreads();
        int run = carry, round_total = 0;
        for (int i = 0; i < kScanWaves; ++i) {
            const int x = s_part[i][lane];
            run += i < w ? x : 0;
            round_total += x;
        }
#pragma unroll
        for (int k = 0; k < kScanPerWave; ++k) {
            if (live && c0 + k < p.nchunks) p.table[static_cast<int64_t>(c0 + k) * p.pitch + col] = run;
            run += v[k];
        }
        carry += round_total;
        __syncthreads();
    }
    if (w == 0 && live) {
        p.totals[col] = carry;
        if (col < p.E) {
            p.expert_count[col] = carry;
        } else if (col < p.E + p.R) {
            p.rank_token_count[col - p.E] = carry;
        } else if (col < p.E + p.R + p.G) {
            if (p.group_token_count) p.group_token_count[col - p.E - p.R] = carry;
        }
    }
}

// Slot assignment for one chunk by four waves.  kFused: the whole batch is
// one chunk and this kernel also builds the histogram and writes the counts;
// otherwise the counts and the chunk's bases come from passes 1 and 2.
// Workgroup 0 writes expert_offset, rank_row_count and the status word.
//
// LDS: s_idx [kChunkEntries] | s_hist [pitch] (fused only) | s_raw [E+1]
// (not fused; fused uses s_hist) | s_aln [E+1] | s_wave [kWaves][E].
template <bool kFused>
__global__ __launch_bounds__(kThreads) void layout_assign_kernel(LayoutParams p) {
    extern __shared__ int smem[];
    __shared__ int s_over;
    int *s_idx = smem;
    int *s_hist = s_idx + kChunkEntries;
    int *s_raw = s_hist;  // fused: the histogram's expert columns become the raw scan
    int *s_aln = s_raw + (kFused ? p.pitch : p.E + 1);
    int *s_wave = s_aln + (p.E + 1);
    const int tid = threadIdx.x, w = tid >> 6;
    const int c = blockIdx.x;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    const int n = (t1 - t0) * p.K;
    const int64_t first = static_cast<int64_t>(t0) * p.K;

    // 1. ids, (unfused) counts and this chunk's bases; clear the histograms
    load_ids(p.topk_idx + first, n, s_idx);
    int base[kMaxExpertsPerThread];
    if (!kFused) {
        const int32_t *row = p.table + static_cast<int64_t>(c) * p.pitch;
        int cnt[kMaxExpertsPerThread];
#pragma unroll
        for (int k = 0; k < kMaxExpertsPerThread; ++k) {
            const int e = min(tid + k * kThreads, p.E - 1);
            cnt[k] = p.expert_count[e];
            base[k] = row[e];
        }
#pragma unroll
        for (int k = 0; k < kMaxExpertsPerThread; ++k) {
            const int e = tid + k * kThreads;
            if (e < p.E) s_raw[e] = cnt[k];
        }
    } else {
#pragma unroll
        for (int k = 0; k < kMaxExpertsPerThread; ++k) base[k] = 0;
        for (int i = tid; i < p.ncols; i += kThreads) s_hist[i] = 0;
    }
    for (int i = tid; i < kWaves * p.E; i += kThreads) s_wave[i] = 0;
    if (tid == 0) s_over = 0;
    __syncthreads();

    // 2. histograms (fused: all columns; always: per-wave expert counts)
    if (kFused) {
        chunk_histogram(p, t0, t1, s_idx, s_hist, s_wave);
    } else {
        const int span = wave_span(n);
        for (int i = tid; i < n; i += kThreads) {
            const int e = s_idx[i];
            if (valid_id(e, p.E)) {
                atomicAdd(&s_wave[(i / span) * p.E + e], 1);
                s_idx[i] = static_cast<int>(p.div_L(e) << kRankShift) | e;
            } else {
                s_idx[i] = -1;
            }
        }
    }
    __syncthreads();
    if (kFused) {
        for (int i = tid; i < p.E + p.R + p.G; i += kThreads) {
            const int v = s_hist[i];
            if (i < p.E) {
                p.expert_count[i] = v;
            } else if (i < p.E + p.R) {
                p.rank_token_count[i - p.E] = v;
            } else if (p.group_token_count) {
                p.group_token_count[i - p.E - p.R] = v;
            }
        }
        __syncthreads();  // s_hist's expert part becomes s_raw below
    }
    const int bad = kFused ? s_hist[p.E + p.R + p.G] : p.totals[p.E + p.R + p.G];
    if (tid < 64) wave_scan_counts(p, s_raw, s_aln, s_raw);
    __syncthreads();

    // 3. cursors: offset + chunk base, then per-wave bases inside the chunk
#pragma unroll
    for (int k = 0; k < kMaxExpertsPerThread; ++k) {
        const int e = tid + k * kThreads;
        if (e < p.E) {
            const int off = s_aln[e] - s_aln[p.div_L(e) * p.L];
            int b = off + base[k];
            for (int ww = 0; ww < kWaves; ++ww) {
                const int h = s_wave[ww * p.E + e];
                s_wave[ww * p.E + e] = b;
                b += h;
            }
            if (c == 0) p.expert_offset[e] = off;
        }
    }
    if (c == 0 && finish_ranks(p, s_aln, s_raw)) atomicOr(&s_over, 1);
    __syncthreads();
    if (c == 0 && tid == 0) *p.status = status_code(bad > 0, s_over);

    // 4. each wave walks its part of the chunk
    const int span = wave_span(n);
    wave_assign_slots(p, first, min(n, w * span), min(n, (w + 1) * span), s_wave + w * p.E, s_idx);
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
    const size_t lds_assign_tail = sizeof(int) * ((p.E + 1) + kWaves * p.E);
    if (p.nchunks == 1) {
        const size_t lds = sizeof(int) * (kChunkEntries + p.pitch) + lds_assign_tail;
        layout_assign_kernel<true><<<1, kThreads, lds, stream>>>(p);
        return hipGetLastError();
    }
    const size_t lds_count = sizeof(int) * (kChunkEntries + p.pitch);
    layout_count_kernel<<<p.nchunks, kThreads, lds_count, stream>>>(p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    layout_scan_kernel<<<p.pitch / 64, 64 * kScanWaves, 0, stream>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds = sizeof(int) * (kChunkEntries + (p.E + 1)) + lds_assign_tail;
    layout_assign_kernel<false><<<p.nchunks, kThreads, lds, stream>>>(p);
    return hipGetLastError();
}

}  // namespace epget
