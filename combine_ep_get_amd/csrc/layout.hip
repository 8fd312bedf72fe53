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
// Entries are processed in chunks of kChunkEntries.
// Multi-chunk path (two or three launches):
//   1. count:  one workgroup per chunk builds an LDS histogram of
//      [experts | ranks | groups | bad ids], writes the chunk's rows of
//      is_token_in_rank and one row of the chunk table;
//   2. scan:   per 64-column tile, 16 waves split the chunk rows, keep them in
//      registers, combine partial sums in LDS and rewrite the table in place
//      as exclusive per-chunk bases; column totals go to the count outputs;
//   3. assign: one workgroup of W waves per chunk derives the expert offsets
//      from the totals (a workgroup scan built on DPP wave scans), counts each wave's share of the
//      chunk per expert, seeds one LDS cursor per (wave, expert) with offset +
//      chunk base + earlier waves' counts, and each wave walks its share in
//      64-entry steps.  W is 16 when E <= 512, so a full chunk is one step
//      per wave.  When the table is small (chunks x experts per thread <=
//      kMaxTableSum) each assign workgroup sums the table rows it needs
//      itself and pass 2 is skipped.
// Single-chunk path (one launch, batches of up to kChunkEntries entries): the
// assign workgroup also builds the histogram and writes the counts, and a
// second workgroup writes the token-to-rank map and unique-token counts.
// Layout and dispatch in one launch (batches of up to kFusedMaxEntries
// entries): two workgroups write the layout outputs while every dispatching
// workgroup derives its own token's slots from LDS histograms of the batch
// (layout_dispatch_kernel).
// Up to kMaxCallChunks chunks with A = 1: the count pass, then one launch
// that does the same from expert-major per-chunk counts
// (dispatch_chunks_kernel).
//
// Every global read a step needs is issued as one batch of independent loads
// (indices clamped into range, a buffer load's range check where a predicate
// is needed), so each step costs about one memory round trip.
#include <algorithm>

#include "../../include/ep_get.h"
#include "device_common.h"

namespace epget {
namespace {

constexpr int kCountThreads = 256;
constexpr int kScanWaves = 16;
constexpr int kScanPerWave = 8;  // chunk rows per wave per round

// Entries in LDS are packed after the entry pass: (rank << 12) | expert for a
// valid id (expert < 4096, rank < 1024), -1 for an empty or invalid one.
constexpr int kRankShift = 12;
constexpr int kExpertMask = (1 << kRankShift) - 1;

__device__ __forceinline__ bool valid_id(int32_t e, int32_t E) {
    return static_cast<uint32_t>(e) < static_cast<uint32_t>(E);
}

// Round v up to a multiple of a; a mask when a is a power of two (the usual
// alignment), a division otherwise.
__device__ __forceinline__ int32_t align_up(int32_t v, int32_t a) {
    return (a & (a - 1)) == 0 ? (v + a - 1) & ~(a - 1) : (v + a - 1) / a * a;
}

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
// its loads back to back (indices clamped into range, so no load sits behind
// a branch); only the LDS stores are predicated.
template <int NT>
__device__ __forceinline__ void load_ids(const int32_t *src, int n, int *s_idx) {
    constexpr int kPer = kChunkEntries / NT;
    if (n <= 0) return;
    int v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = src[min(static_cast<int>(threadIdx.x) + k * NT, n - 1)];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + k * NT;
        if (i < n) s_idx[i] = v[k];
    }
}

// Entries per wave when n entries are split over W waves (a multiple of 64,
// so every wave but the last walks whole 64-entry steps).
__device__ __forceinline__ int wave_span(int n, int W) { return (n + W * 64 - 1) / (W * 64) * 64; }

// Entry pass over the chunk's raw ids in s_idx: counts experts and bad ids
// into s_hist (if not null), each wave's share per expert into s_wave[w*E+e]
// (if not null), and packs every entry in place.
template <int NT>
__device__ void entry_pass(const LayoutParams &p, int n, int W, int *s_idx, int *s_hist, int *s_wave) {
    const int span = wave_span(n, W);
    const int bad_col = p.E + p.R + p.G;
    for (int i = threadIdx.x; i < n; i += NT) {
        const int e = s_idx[i];
        if (!valid_id(e, p.E)) {
            if (e != -1 && s_hist) atomicAdd(&s_hist[bad_col], 1);
            s_idx[i] = -1;
            continue;
        }
        if (s_hist) atomicAdd(&s_hist[e], 1);
        if (s_wave) atomicAdd(&s_wave[(i / span) * p.E + e], 1);
        s_idx[i] = static_cast<int>(p.div_L(e) << kRankShift) | e;
    }
}

// One token's row of is_token_in_rank from the bit mask of its ranks
// (R <= 64): whole 8-byte words where the row allows, bytes otherwise.
__device__ __forceinline__ void write_map_row(uint8_t *row, int R, uint64_t mask) {
    int r = 0;
    if ((reinterpret_cast<uintptr_t>(row) & 7) == 0) {
        for (; r + 8 <= R; r += 8) {
            uint64_t bytes = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) bytes |= ((mask >> (r + b)) & 1ull) << (8 * b);
            *reinterpret_cast<uint64_t *>(row + r) = bytes;
        }
    }
    for (; r < R; ++r) row[r] = static_cast<uint8_t>((mask >> r) & 1);
}

// Token pass over packed entries: the chunk's rows of is_token_in_rank and
// unique tokens per rank and per group (added into s_hist).  With R <= 64 a
// thread takes a whole token as a bit mask of its ranks, and per-rank /
// per-group totals are popcounts of wave ballots; otherwise one thread per
// (token, rank) and (token, group) pair.
template <int NT>
__device__ void token_pass(const LayoutParams &p, int t0, int t1, const int *s_idx, int *s_hist) {
    const int ntok = t1 - t0;
    uint8_t *map = p.is_token_in_rank + static_cast<int64_t>(t0) * p.R;
    if (p.R <= 64) {
        const int lane = __lane_id();
        const int rpg = p.ranks_per_group;
        const uint64_t group_bits = rpg >= 64 ? ~0ull : (1ull << rpg) - 1ull;
        for (int base = 0; base < ntok; base += NT) {
            const int tl = base + threadIdx.x;
            const bool act = tl < ntok;
            uint64_t mask = 0;
            if (act) {
                const int *ids = s_idx + tl * p.K;
                if ((p.K & 3) == 0) {  // 16-byte LDS reads of four entries
                    for (int j = 0; j < p.K; j += 4) {
                        const int4 q = *reinterpret_cast<const int4 *>(ids + j);
                        mask |= (q.x >= 0 ? 1ull << (q.x >> kRankShift) : 0ull) |
                                (q.y >= 0 ? 1ull << (q.y >> kRankShift) : 0ull) |
                                (q.z >= 0 ? 1ull << (q.z >> kRankShift) : 0ull) |
                                (q.w >= 0 ? 1ull << (q.w >> kRankShift) : 0ull);
                    }
                } else {
                    for (int j = 0; j < p.K; ++j) {
                        const int v = ids[j];
                        if (v >= 0) mask |= 1ull << (v >> kRankShift);
                    }
                }
                write_map_row(map + static_cast<int64_t>(tl) * p.R, p.R, mask);
            }
            // lane r collects rank r's count, lane g group g's; one LDS
            // atomic per wave and column instead of one per ballot
            int rank_cnt = 0, group_cnt = 0;
            for (int r = 0; r < p.R; ++r) {
                const int cnt = __popcll(__ballot(act && ((mask >> r) & 1)));
                rank_cnt = lane == r ? cnt : rank_cnt;
            }
            for (int g = 0; g < p.G; ++g) {
                const bool in = act && ((mask >> (g * rpg)) & group_bits) != 0;
                const int cnt = __popcll(__ballot(in));
                group_cnt = lane == g ? cnt : group_cnt;
            }
            if (lane < p.R && rank_cnt) atomicAdd(&s_hist[p.E + lane], rank_cnt);
            if (lane < p.G && group_cnt) atomicAdd(&s_hist[p.E + p.R + lane], group_cnt);
        }
        return;
    }
    // R > 64.  Map rows: the chunk's rows (one run of ntok * R bytes) are
    // cleared with 16-byte stores, then each entry sets its rank's byte
    // (entries of a token that share a rank write the same 1).  The clearing
    // stores are waited for before the barrier, so no 1 can be overtaken by
    // the 0 it replaces.
    const int nbytes = ntok * p.R;
    const int head = min(static_cast<int>((16 - (reinterpret_cast<uintptr_t>(map) & 15)) & 15), nbytes);
    const int nunits = (nbytes - head) >> 4;
    const int tail0 = head + (nunits << 4);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int u = threadIdx.x; u < nunits; u += NT) *reinterpret_cast<u32x4 *>(map + head + (u << 4)) = zero;
    for (int i = threadIdx.x; i < head + (nbytes - tail0); i += NT) map[i < head ? i : tail0 + (i - head)] = 0;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // An entry also counts its token for its rank (its group) when no
    // earlier entry of the token has that rank (group).
    const int nent = ntok * p.K;
    for (int i = threadIdx.x; i < nent; i += NT) {
        const int v = s_idx[i];
        if (v < 0) continue;
        const int tl = i / p.K, j = i - tl * p.K;
        const int *ids = s_idx + (i - j);
        const int r = v >> kRankShift;
        const int g = r / p.ranks_per_group;
        map[static_cast<int64_t>(tl) * p.R + r] = 1;
        bool first_r = true, first_g = true;
        for (int jj = 0; jj < j; ++jj) {
            const int u = ids[jj];
            if (u < 0) continue;
            const int ru = u >> kRankShift;
            first_r &= ru != r;
            first_g &= ru / p.ranks_per_group != g;
        }
        if (first_r) atomicAdd(&s_hist[p.E + r], 1);
        if (first_g) atomicAdd(&s_hist[p.E + p.R + g], 1);
    }
}

// Exclusive scans over all experts of the aligned and raw counts by the
// whole workgroup: thread t sums the ept = ceil(E / NT) <= EPT experts
// [t*ept, (t+1)*ept), a DPP wave scan combines the threads of a wave, and the
// wave totals go through LDS.  s_aln and s_raw get E+1 entries (the last one
// is the total).  `counts` may be the same LDS array as s_raw: every thread
// reads its experts before the barrier that precedes the writes.  Contains
// barriers: call from the whole workgroup.  block_scan_counts below picks the
// instantiation.
template <int NT, int EPT>
__device__ void block_scan_counts_n(const LayoutParams &p, const int *counts, int *s_aln,
                                    int *s_raw, int *s_wsum) {
    constexpr int kWavesPerBlock = NT / 64;
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    const int ept = (p.E + NT - 1) / NT;
    const int e0 = threadIdx.x * ept;
    int ca[EPT], cr[EPT];
    int sa = 0, sr = 0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) cr[k] = k < ept && e0 + k < p.E ? counts[e0 + k] : 0;
    // A is uniform: branch once instead of selecting per expert (the
    // generic division would otherwise run for every count)
    if (p.A == 1) {
#pragma unroll
        for (int k = 0; k < EPT; ++k) ca[k] = cr[k];
    } else {
#pragma unroll
        for (int k = 0; k < EPT; ++k) ca[k] = align_up(cr[k], p.A);
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        sa += ca[k];
        sr += cr[k];
    }
    const int ia = wave_inclusive_sum(sa), ir = wave_inclusive_sum(sr);
    if (lane == 63) {
        s_wsum[w] = ia;
        s_wsum[kWavesPerBlock + w] = ir;
    }
    __syncthreads();
    int pa = 0, pr = 0, ta = 0, tr = 0;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) {
        const int a = s_wsum[i], r = s_wsum[kWavesPerBlock + i];
        pa += i < w ? a : 0;
        pr += i < w ? r : 0;
        ta += a;
        tr += r;
    }
    int ea = pa + ia - sa, er = pr + ir - sr;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        if (k < ept && e0 + k < p.E) {
            s_aln[e0 + k] = ea;
            s_raw[e0 + k] = er;
        }
        ea += ca[k];
        er += cr[k];
    }
    if (threadIdx.x == 0) {
        s_aln[p.E] = ta;
        s_raw[p.E] = tr;
    }
}

// block_scan_counts_n with two experts per thread when that covers E (up to
// 256 experts on 128 threads), else with EPT, so that the common case's
// loops carry no idle iterations: the EPT = 16 form took 1.0 µs of a
// dispatching workgroup's slot derivation at E = 256.  E is the same for the
// whole workgroup, so every thread takes the same branch to the same
// barriers.
template <int NT, int EPT>
__device__ __forceinline__ void block_scan_counts(const LayoutParams &p, const int *counts, int *s_aln,
                                                  int *s_raw, int *s_wsum) {
    if constexpr (EPT > 2) {
        if (p.E <= 2 * NT) return block_scan_counts_n<NT, 2>(p, counts, s_aln, s_raw, s_wsum);
    }
    block_scan_counts_n<NT, EPT>(p, counts, s_aln, s_raw, s_wsum);
}

// Per-rank results from the scans: rank_row_count and the capacity check.
// Returns nonzero if one of this thread's ranks overflows its slice.
template <int NT>
__device__ int finish_ranks(const LayoutParams &p, const int *s_aln, const int *s_raw) {
    int over = 0;
    for (int r = threadIdx.x; r < p.R; r += NT) {
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
// entries in s_idx, global entry index first + i), in 64-entry steps.  The
// wave's cursor for expert e is s_cur[e]: the next free row of e inside its
// slice.  Within a step, lanes naming the same expert are found by
// matching the id bit by bit with ballots; each takes the cursor plus the
// number of matching lanes below it, and the lowest of them advances the
// cursor.  One wave's LDS accesses complete in issue order, so every lane
// reads the cursor before the update lands.
__device__ __forceinline__ void wave_assign_slots(const LayoutParams &p, int64_t first, int i0,
                                                  int i1, int *s_cur, const int *s_idx) {
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

constexpr int kCountEPT = (EP_MAX_EXPERTS + kCountThreads - 1) / kCountThreads;

// Multi-chunk pass 1: the chunk's histogram row.  For the one-call layout
// and dispatch (p.count_t set) it also writes, expert-major, the chunk's
// count of each expert and the chunk's count of the lower experts of the
// same rank (an exclusive scan of the histogram restarted at each rank's
// first expert); there each chunk has two workgroups side by side, so that
// the token pass (the rank map and unique tokens) no longer precedes the
// expert counts the next launch waits for: workgroups [0, nchunks) count
// experts and bad ids, [nchunks, 2 nchunks) map tokens, each writing its
// own columns of the row (1024-8192 tokens: the layout-and-dispatch phase
// 0.75-1.1 µs shorter).  Otherwise one workgroup per chunk does both.
// LDS: s_idx [kChunkEntries] | s_hist [pitch] | s_raw [E+1] | s_aln [E+1].
__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(LayoutParams p) {
    extern __shared__ __align__(16) int smem[];
    __shared__ int s_wsum[2 * kCountThreads / 64];
    int *s_idx = smem;
    int *s_hist = smem + kChunkEntries;
    const bool split = p.count_t != nullptr;
    const int c = split ? static_cast<int>(blockIdx.x) % p.nchunks : blockIdx.x;
    const bool experts = !split || static_cast<int>(blockIdx.x) < p.nchunks;
    const bool tokens = !split || static_cast<int>(blockIdx.x) >= p.nchunks;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    const int n = (t1 - t0) * p.K;
    load_ids<kCountThreads>(p.topk_idx + static_cast<int64_t>(t0) * p.K, n, s_idx);
    for (int i = threadIdx.x; i < p.ncols; i += kCountThreads) s_hist[i] = 0;
    __syncthreads();
    // packs every entry (rank next to id); counts experts only in the expert role
    entry_pass<kCountThreads>(p, n, 1, s_idx, experts ? s_hist : nullptr, nullptr);
    __syncthreads();
    if (tokens) {
        token_pass<kCountThreads>(p, t0, t1, s_idx, s_hist);
        __syncthreads();
    }
    int32_t *row = p.table + static_cast<int64_t>(c) * p.pitch;
    const int bad_col = p.E + p.R + p.G;
    for (int i = threadIdx.x; i < p.ncols; i += kCountThreads) {
        const bool expert_col = i < p.E || i == bad_col;
        if (expert_col ? experts : tokens) row[i] = s_hist[i];
    }
    if (split && experts) {
        int *s_raw = s_hist + p.pitch;
        int *s_aln = s_raw + (p.E + 1);
        block_scan_counts<kCountThreads, kCountEPT>(p, s_hist, s_aln, s_raw, s_wsum);
        __syncthreads();
        for (int e = threadIdx.x; e < p.E; e += kCountThreads) {
            const int64_t at = static_cast<int64_t>(e) * p.nchunks + c;
            p.count_t[at] = s_hist[e];
            p.excl_t[at] = s_raw[e] - s_raw[static_cast<int>(p.div_L(e)) * p.L];
        }
    }
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

// How the assign kernel gets each expert's total and its chunk's base.
enum AssignMode {
    kFusedChunk = 0,   // one chunk: this kernel builds the histogram itself
    kSumTable = 1,     // sums the count table's rows (after pass 1 only)
    kScannedTable = 2  // reads the bases and totals pass 2 wrote
};

// What a fused-chunk workgroup computes: everything, or one of two halves
// that two workgroups run side by side (the per-token half: the token-to-rank
// map and unique tokens per rank and group; the per-expert half: counts,
// offsets, rank rows and the status).
enum LayoutPart { kLayoutAll = 0, kLayoutExperts = 1, kLayoutTokens = 2 };

// Experts each thread of a W-wave assign workgroup scans.
template <int W>
constexpr int assign_experts_per_thread() {
    return ((W >= 16 ? 512 : (W >= 8 ? 1024 : EP_MAX_EXPERTS)) + 64 * W - 1) / (64 * W);
}

// Slot assignment for chunk c by a workgroup of W waves.  Workgroup 0
// writes expert_offset, rank_row_count and the status word (and, unless
// pass 2 ran, the per-expert / per-rank / per-group counts).  Without kWalk
// everything but the slots is computed (a fused dispatch derives those per
// token instead).  For a one-chunk batch kPart lets two workgroups share the
// work: the per-expert half (which keeps the walk) and the per-token half.
//
// LDS: s_idx [kChunkEntries] | fused: s_hist [pitch], whose expert columns
// later hold the raw scan; otherwise s_raw [E+1] | s_aln [E+1] | s_wave [W*E]
// (s_wave only with kWalk).
template <int W, int kMode, bool kWalk, int kPart = kLayoutAll>
__device__ void assign_chunk(const LayoutParams &p, int c) {
    constexpr bool kFused = kMode == kFusedChunk;
    constexpr int NT = 64 * W;
    constexpr int kEPT = assign_experts_per_thread<W>();
    extern __shared__ __align__(16) int smem[];
    __shared__ int s_over;
    __shared__ int s_wsum[2 * W];
    int *s_idx = smem;
    int *s_hist = s_idx + kChunkEntries;
    int *s_raw = s_hist;
    int *s_aln = s_raw + (kFused ? p.pitch : p.E + 1);
    int *s_wave = s_aln + (p.E + 1);
    const int tid = threadIdx.x, w = tid >> 6;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    const int n = (t1 - t0) * p.K;
    const int64_t first = static_cast<int64_t>(t0) * p.K;

    // 1. ids, (unfused) counts and this chunk's bases; clear the histograms
    load_ids<NT>(p.topk_idx + first, n, s_idx);
    int base[kEPT];
    int bad = 0;
    if (kMode == kScannedTable) {
        const int32_t *row = p.table + static_cast<int64_t>(c) * p.pitch;
        int cnt[kEPT];
#pragma unroll
        for (int k = 0; k < kEPT; ++k) {
            const int e = min(tid + k * NT, p.E - 1);
            cnt[k] = p.expert_count[e];
            base[k] = row[e];
        }
#pragma unroll
        for (int k = 0; k < kEPT; ++k) {
            const int e = tid + k * NT;
            if (e < p.E) {
                s_raw[e] = cnt[k];
                if (c == 0 && p.cumulative) p.cumulative[e] += cnt[k];
            }
        }
        bad = p.totals[p.E + p.R + p.G];
    } else if (kMode == kSumTable) {
        // Column e of the table: its total over all chunks and its sum over
        // the chunks before this one, kSumBatch rows per load batch (buffer
        // loads return 0 past the last row).
        constexpr int kSumBatch = 32;
        const I32Buffer table(p.table, static_cast<uint32_t>(p.nchunks) * p.pitch);
#pragma unroll
        for (int k = 0; k < kEPT; ++k) {
            const int e = tid + k * NT;
            int tot = 0, pre = 0;
            for (int c0 = 0; c0 < p.nchunks; c0 += kSumBatch) {
                int v[kSumBatch];
#pragma unroll
                for (int q = 0; q < kSumBatch; ++q)
                    v[q] = table.load(static_cast<uint32_t>(c0 + q) * p.pitch + e,
                                      e < p.E && c0 + q < p.nchunks);
#pragma unroll
                for (int q = 0; q < kSumBatch; ++q) {
                    tot += v[q];
                    pre += c0 + q < c ? v[q] : 0;
                }
            }
            base[k] = pre;
            if (e < p.E) {
                s_raw[e] = tot;
                if (c == 0) {
                    p.expert_count[e] = tot;
                    if (p.cumulative) p.cumulative[e] += tot;
                }
            }
        }
        // rank, group and bad-id columns: workgroup 0 writes their totals,
        // and every workgroup needs the bad-id total for the status
        for (int col = p.E + tid; col < p.ncols; col += NT) {
            if (c != 0 && col != p.ncols - 1) continue;
            int tot = 0;
            for (int c0 = 0; c0 < p.nchunks; c0 += kSumBatch) {
                int v[kSumBatch];
#pragma unroll
                for (int q = 0; q < kSumBatch; ++q)
                    v[q] = table.load(static_cast<uint32_t>(c0 + q) * p.pitch + col, c0 + q < p.nchunks);
#pragma unroll
                for (int q = 0; q < kSumBatch; ++q) tot += v[q];
            }
            if (col == p.ncols - 1) {
                s_over = tot;  // bad-id total, read back below
            } else if (col < p.E + p.R) {
                p.rank_token_count[col - p.E] = tot;
            } else if (p.group_token_count) {
                p.group_token_count[col - p.E - p.R] = tot;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < kEPT; ++k) base[k] = 0;
        for (int i = tid; i < p.ncols; i += NT) s_hist[i] = 0;
    }
    if (kWalk)
        for (int i = tid; i < W * p.E; i += NT) s_wave[i] = 0;
    if (kMode != kSumTable && tid == 0) s_over = 0;
    __syncthreads();
    if (kMode == kSumTable) {
        bad = s_over;
        __syncthreads();  // s_over is reused as the capacity flag
        if (tid == 0) s_over = 0;
    }

    // 2. per-wave expert counts (and, fused, the whole histogram)
    static_assert(kPart == kLayoutAll || kFused, "split layouts are fused-chunk only");
    static_assert(!(kWalk && kPart == kLayoutTokens), "the slot walk belongs to the per-expert half");
    constexpr bool kExperts = kPart != kLayoutTokens, kTokens = kPart != kLayoutExperts;
    entry_pass<NT>(p, n, W, s_idx, kFused && kExperts ? s_hist : nullptr, kWalk ? s_wave : nullptr);
    __syncthreads();
    if (kFused) {
        if (kTokens) token_pass<NT>(p, t0, t1, s_idx, s_hist);
        __syncthreads();
        for (int i = tid; i < p.E + p.R + p.G; i += NT) {
            const int v = s_hist[i];
            if (i < p.E) {
                if (kExperts) {
                    p.expert_count[i] = v;
                    if (p.cumulative) p.cumulative[i] += v;
                }
            } else if (!kTokens) {
                continue;
            } else if (i < p.E + p.R) {
                p.rank_token_count[i - p.E] = v;
            } else if (p.group_token_count) {
                p.group_token_count[i - p.E - p.R] = v;
            }
        }
        if (!kExperts) return;  // the whole workgroup, after its last barrier
        __syncthreads();  // s_hist's expert columns become s_raw below
    }
    if (kFused) bad = s_hist[p.E + p.R + p.G];
    block_scan_counts<NT, kEPT>(p, s_raw, s_aln, s_raw, s_wsum);
    __syncthreads();

    // 3. cursors: offset + chunk base, then each wave's base inside the chunk
#pragma unroll
    for (int k = 0; k < kEPT; ++k) {
        const int e = tid + k * NT;
        if (e < p.E) {
            const int off = s_aln[e] - s_aln[p.div_L(e) * p.L];
            if (kWalk) {
                int h[W];
#pragma unroll
                for (int ww = 0; ww < W; ++ww) h[ww] = s_wave[ww * p.E + e];
                int b = off + base[k];
#pragma unroll
                for (int ww = 0; ww < W; ++ww) {
                    s_wave[ww * p.E + e] = b;
                    b += h[ww];
                }
            }
            if (c == 0) p.expert_offset[e] = off;
        }
    }
    if (c == 0 && finish_ranks<NT>(p, s_aln, s_raw)) atomicOr(&s_over, 1);
    __syncthreads();
    if (c == 0 && tid == 0) *p.status = status_code(bad > 0, s_over);

    // 4. each wave walks its share of the chunk
    if (kWalk) {
        const int span = wave_span(n, W);
        wave_assign_slots(p, first, min(n, w * span), min(n, (w + 1) * span), s_wave + w * p.E, s_idx);
    }
}

template <int W, int kMode>
__global__ __launch_bounds__(64 * W) void layout_assign_kernel(LayoutParams p) {
    assign_chunk<W, kMode, true>(p, blockIdx.x);
}

// A one-chunk batch on two workgroups: workgroup 0 takes the per-expert half
// and the slot walk, workgroup 1 the per-token half (token-to-rank map and
// unique tokens per rank and group), which then leaves the critical path.
template <int W>
__global__ __launch_bounds__(64 * W) void layout_one_chunk_kernel(LayoutParams p) {
    if (blockIdx.x == 0)
        assign_chunk<W, kFusedChunk, true, kLayoutExperts>(p, 0);
    else
        assign_chunk<W, kFusedChunk, false, kLayoutTokens>(p, 0);
}

// Largest table sum (rows x experts per thread) the assign kernel does itself
// instead of running pass 2.
constexpr int kMaxTableSum = 64;

template <int W>
hipError_t launch_assign(const LayoutParams &p, hipStream_t stream) {
    const size_t tail = sizeof(int) * ((p.E + 1) + static_cast<size_t>(W) * p.E);
    constexpr int kEPT = assign_experts_per_thread<W>();
    if (p.nchunks == 1) {
        const size_t lds = sizeof(int) * (kChunkEntries + p.pitch) + tail;
        layout_one_chunk_kernel<W><<<2, 64 * W, lds, stream>>>(p);
        return hipGetLastError();
    }
    const size_t lds_count = sizeof(int) * (kChunkEntries + p.pitch + 2 * (p.E + 1));
    layout_count_kernel<<<p.nchunks, kCountThreads, lds_count, stream>>>(p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds = sizeof(int) * (kChunkEntries + (p.E + 1)) + tail;
    if (static_cast<int64_t>(p.nchunks) * kEPT <= kMaxTableSum) {
        layout_assign_kernel<W, kSumTable><<<p.nchunks, 64 * W, lds, stream>>>(p);
        return hipGetLastError();
    }
    layout_scan_kernel<<<p.pitch / 64, 64 * kScanWaves, 0, stream>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    layout_assign_kernel<W, kScannedTable><<<p.nchunks, 64 * W, lds, stream>>>(p);
    return hipGetLastError();
}

// Slots of token t's K entries when the whole batch has at most kMaxEntries
// (a multiple of NT, at most kFusedMaxEntries) entries, found by one
// workgroup of NT threads without the slot walk.  Entry (t, j) with expert e lands at row
//   expert_offset[e] + #{entries before (t, j) naming e}
// of its rank's slice, which is the slot the walk assigns.  The workgroup
// builds two LDS histograms of the batch, one over all entries and one over
// the entries of tokens before t, and scans the first into the aligned
// offsets; the count of earlier entries is the second histogram plus the
// earlier duplicates of e inside the token.  Returns slot j in lane j of
// every wave (j < K), as slot_of reads it.  lds holds 3 * E + 2 ints,
// s_wsum 2 * NT / 64.  Contains barriers.
template <int NT, int kMaxEntries>
__device__ __forceinline__ int32_t token_slots_one_chunk(const LayoutParams &p, int t, int *lds, int *s_wsum) {
    constexpr int kPer = kMaxEntries / NT;
    constexpr int kEPT = (EP_MAX_EXPERTS + NT - 1) / NT;
    const int n = p.T * p.K;
    const int tid = threadIdx.x, lane = __lane_id();
    int *s_all = lds;                   // E + 1: counts, then their exclusive scan
    int *s_aln = s_all + (p.E + 1);     // E + 1: exclusive scan of aligned counts
    int *s_before = s_aln + (p.E + 1);  // E: counts over tokens before t
    const int32_t *trow = p.topk_idx + static_cast<int64_t>(t) * p.K;
    const int lane_id = trow[min(lane, p.K - 1)];
    int ids[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) ids[k] = p.topk_idx[min(tid + k * NT, n - 1)];
    for (int i = tid; i < p.E; i += NT) {
        s_all[i] = 0;
        s_before[i] = 0;
    }
    __syncthreads();
    const int first = t * p.K;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * NT;
        if (i < n && valid_id(ids[k], p.E)) {
            atomicAdd(&s_all[ids[k]], 1);
            if (i < first) atomicAdd(&s_before[ids[k]], 1);
        }
    }
    __syncthreads();
    block_scan_counts<NT, kEPT>(p, s_all, s_aln, s_all, s_wsum);
    __syncthreads();
    const int j = min(lane, p.K - 1);
    int dup = 0;
    for (int jj = 0; jj < p.K; ++jj)
        dup += (jj < j && __builtin_amdgcn_readlane(lane_id, jj) == lane_id) ? 1 : 0;
    if (!valid_id(lane_id, p.E)) return -1;
    const int rank = static_cast<int>(p.div_L(lane_id));
    const int pos = s_aln[lane_id] - s_aln[rank * p.L] + s_before[lane_id] + dup;
    return pos < p.S ? rank * p.S + pos : -1;
}

// The layout outputs of a batch of at most kFusedMaxEntries entries except
// the slots, by one workgroup of NT threads that takes the batch chunk by
// chunk through LDS: with kExperts the per-expert half (counts, aligned
// offsets, rows per rank, status), with kTokens the per-token half (token-to-
// rank map, unique tokens per rank and group).  LDS: s_idx [kChunkEntries] |
// s_hist [pitch] | s_aln [E+1].  Contains barriers.
template <int NT, bool kExperts, bool kTokens>
__device__ void fused_layout(const LayoutParams &p, int *lds) {
    constexpr int kEPT = (EP_MAX_EXPERTS + NT - 1) / NT;
    __shared__ int s_wsum[2 * NT / 64];
    __shared__ int s_over;
    int *s_idx = lds;
    int *s_hist = s_idx + kChunkEntries;
    int *s_aln = s_hist + p.pitch;
    const int tid = threadIdx.x;
    for (int i = tid; i < p.ncols; i += NT) s_hist[i] = 0;
    if (tid == 0) s_over = 0;
    for (int c = 0; c < p.nchunks; ++c) {
        const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
        const int n = (t1 - t0) * p.K;
        __syncthreads();  // the previous chunk is done with s_idx
        load_ids<NT>(p.topk_idx + static_cast<int64_t>(t0) * p.K, n, s_idx);
        __syncthreads();
        entry_pass<NT>(p, n, 1, s_idx, kExperts ? s_hist : nullptr, nullptr);
        if (kTokens) {
            __syncthreads();
            token_pass<NT>(p, t0, t1, s_idx, s_hist);
        }
    }
    __syncthreads();
    if (kTokens) {
        for (int i = tid; i < p.R + p.G; i += NT) {
            const int v = s_hist[p.E + i];
            if (i < p.R)
                p.rank_token_count[i] = v;
            else if (p.group_token_count)
                p.group_token_count[i - p.R] = v;
        }
    }
    if (!kExperts) return;  // the whole workgroup, after its last barrier
    for (int e = tid; e < p.E; e += NT) {
        p.expert_count[e] = s_hist[e];
        if (p.cumulative) p.cumulative[e] += s_hist[e];
    }
    const int bad = s_hist[p.E + p.R + p.G];
    __syncthreads();  // the counts above are read before the scan rewrites them
    block_scan_counts<NT, kEPT>(p, s_hist, s_aln, s_hist, s_wsum);
    __syncthreads();
    for (int e = tid; e < p.E; e += NT)
        p.expert_offset[e] = s_aln[e] - s_aln[static_cast<int>(p.div_L(e)) * p.L];
    if (finish_ranks<NT>(p, s_aln, s_hist)) atomicOr(&s_over, 1);
    __syncthreads();
    if (tid == 0) *p.status = status_code(bad > 0, s_over);
}

// Layout and dispatch in one launch for a batch of at most kMaxEntries
// entries (one chunk, or up to kFusedMaxEntries), on a (T, splits + 1)
// grid.  Workgroups (0, 0) and (1, 0), dispatched first, compute and write
// the layout except the slots: the per-expert half (counts, offsets, rank
// rows, status) and the per-token half (token-to-rank map, unique tokens per
// rank and group), over one chunk in LDS or chunk by chunk; the rest of row
// y = 0 has nothing to do.  Workgroup
// (t, y > 0) finds the slots of token t itself, writes them to token_slot if
// y == 1, and dispatches column run y - 1 of the token's row.  Token t's
// workgroups have the linear ids, and so the XCDs, that dispatch_kernel
// gives them, which the combine's grid shares: rows a small batch leaves in
// an XCD's L2 are read back there.
// The operands of a dispatching workgroup's first loads (the ids, the row,
// the batch sizes) also come as leading scalar arguments, which arrive
// preloaded in SGPRs; the structures' other fields load while those loads
// are in flight.
template <int VPT, int kMaxEntries>
__global__ __launch_bounds__(kFusedThreads) void layout_dispatch_kernel(
    const int32_t *topk_idx, const void *x, int32_t T, int32_t K, int32_t E, int32_t nvec, LayoutParams p,
    CopyParams c, DispatchArgs a) {
    p.topk_idx = topk_idx;
    p.T = c.T = T;
    p.K = c.K = K;
    p.E = E;
    c.nvec = nvec;
    a.x = x;
    extern __shared__ __align__(16) int smem[];
    __shared__ int s_wsum[2 * kFusedThreads / 64];
    if (blockIdx.y == 0) {
        // the layout, split over workgroups (0, 0) and (1, 0) when there are two
        if constexpr (kMaxEntries == kChunkEntries) {
            constexpr int W = kFusedThreads / 64;
            if (gridDim.x == 1)
                assign_chunk<W, kFusedChunk, false, kLayoutAll>(p, 0);
            else if (blockIdx.x == 0)
                assign_chunk<W, kFusedChunk, false, kLayoutExperts>(p, 0);
            else if (blockIdx.x == 1)
                assign_chunk<W, kFusedChunk, false, kLayoutTokens>(p, 0);
        } else {
            if (gridDim.x == 1)
                fused_layout<kFusedThreads, true, true>(p, smem);
            else if (blockIdx.x == 0)
                fused_layout<kFusedThreads, true, false>(p, smem);
            else if (blockIdx.x == 1)
                fused_layout<kFusedThreads, false, true>(p, smem);
        }
        return;
    }
    const int t = blockIdx.x;
    const int v0 = (blockIdx.y - 1) * (kFusedThreads * VPT) + threadIdx.x;
    u32x4 buf[VPT];
    load_token_row<VPT, kFusedThreads>(c, a, t, v0, buf);
    const int32_t lane_slot = token_slots_one_chunk<kFusedThreads, kMaxEntries>(p, t, smem, s_wsum);
    const bool meta = blockIdx.y == 1;
    if (meta && static_cast<int>(threadIdx.x) < p.K)
        p.token_slot[static_cast<int64_t>(t) * p.K + threadIdx.x] = lane_slot;
    store_token_rows<VPT, kFusedThreads, true>(c, a, t, v0, meta, lane_slot, buf);
}

// Workgroups that lead the 1-D grid of the multi-chunk one-call kernel:
// the first takes the layout outputs, the others have nothing to do.  Eight
// keep the copy workgroups on the XCDs (linear id modulo 8) that the
// combine's grid gives the same tokens.  A (T, splits + 1) grid with the
// layout in row 0 left T - 1 workgroups idle, all dispatched ahead of the
// copies: 16383 of them at 16384 tokens, where the 1-D grid took the step
// from 772 to 769 µs.  (The decode-sized kernel keeps its 2-D grid, which
// measured 0.3 µs faster on a 128-token step.)
constexpr int kLeadWorkgroups = 8;

// Token and column run of copy workgroup `b` (b >= kLeadWorkgroups) of a
// grid of kLeadWorkgroups + T * splits workgroups.
__device__ __forceinline__ void copy_role(int b, int T, int *t, int *run) {
    const int i = b - kLeadWorkgroups;
    *run = i / T;
    *t = i - *run * T;
}

// Largest chunk count of the two-launch one-call path: a wave reads the
// per-chunk counts with one lane per chunk, in CR <= kMaxChunkRounds rounds
// of 64 chunks.
constexpr int kMaxChunkRounds = 2;
constexpr int kMaxCallChunks = 64 * kMaxChunkRounds;

// Slots of token t's K entries in chunk c of a multi-chunk batch (A = 1),
// found by one workgroup of NT threads from the count pass's expert-major
// arrays instead of a slot walk.  Entry (t, j) with expert e lands at row
//   sum over chunks of (lower experts of e's rank)     -- expert_offset[e]
//   + sum over chunks before c of (e)                  -- earlier chunks
//   + #{entries of chunk c before (t, j) naming e}
// of its rank's slice, which is the row the walk assigns.  The third term is
// an LDS histogram of the chunk's entries before token t plus the earlier
// duplicates of e inside the token.  The per-chunk sums take CR rounds of
// 64 chunks (one lane per chunk).  Returns slot j in lane j of every wave.
// lds holds E ints.  Contains barriers.
template <int NT, int CR, bool kEarlySums, class IssueRow>
__device__ int32_t token_slots_in_chunk(const LayoutParams &p, int t, int c, int *s_before, int *s_part,
                                        IssueRow issue_row) {
    constexpr int kPer = kChunkEntries / NT;
    constexpr int kWaves = NT / 64;
    constexpr int kRound = 4;  // top-k positions per wave and round
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int t0 = c * p.chunk_tokens, t1 = min(p.T, t0 + p.chunk_tokens);
    const int n = (t1 - t0) * p.K;
    const int32_t *cid = p.topk_idx + static_cast<int64_t>(t0) * p.K;
    // the caller's loads of the token's row go first, or right behind the
    // token's ids when the sums are loaded early (which need those ids)
    if constexpr (!kEarlySums) issue_row();
    const int lane_id = cid[(t - t0) * p.K + min(lane, p.K - 1)];
    if constexpr (kEarlySums) {
        issue_row();
        __builtin_amdgcn_sched_barrier(0);  // keep the row loads ahead of the sums
    }
    // the per-chunk sums of top-k positions j0 + q * kWaves: lane l reads
    // chunks l, l + 64, ...
    const I32Buffer cnt_t(p.count_t, static_cast<uint32_t>(p.E) * p.nchunks);
    const I32Buffer exc_t(p.excl_t, static_cast<uint32_t>(p.E) * p.nchunks);
    auto load_sums = [&](int j0, int (&part)[kRound]) {
#pragma unroll
        for (int q = 0; q < kRound; ++q) {
            const int j = j0 + q * kWaves;
            const int e = __builtin_amdgcn_readlane(lane_id, min(j, p.K - 1));
            const bool live = j < p.K && valid_id(e, p.E);
            const uint32_t row = static_cast<uint32_t>(live ? e : 0) * p.nchunks;
            part[q] = 0;
#pragma unroll
            for (int r = 0; r < CR; ++r) {
                const int cc = lane + 64 * r;
                const bool ok = live && cc < p.nchunks;
                part[q] += exc_t.load(row + cc, ok) + cnt_t.load(row + cc, ok && cc < c);
            }
        }
    };
    auto reduce_sums = [&](int j0, const int (&part)[kRound]) {
#pragma unroll
        for (int q = 0; q < kRound; ++q) {
            const int j = j0 + q * kWaves;
            if (j < p.K) {
                const int sum = wave_inclusive_sum(part[q]);
                if (lane == 63) s_part[j] = sum;
            }
        }
    };
    // with kEarlySums the first round's sums are loaded as soon as the
    // token's ids are in, so that they travel with the row and the chunk's
    // ids (more registers live at once); otherwise after the histogram
    int part[kRound];
    if constexpr (kEarlySums) load_sums(w, part);
    int ids[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) ids[k] = cid[min(tid + k * NT, n - 1)];
    for (int i = tid; i < p.E; i += NT) s_before[i] = 0;
    __syncthreads();
    const int before = (t - t0) * p.K;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        if (tid + k * NT < before && valid_id(ids[k], p.E)) atomicAdd(&s_before[ids[k]], 1);
    int j0 = w;
    if constexpr (kEarlySums) {
        reduce_sums(j0, part);
        j0 += kWaves * kRound;
    }
    for (; j0 < p.K; j0 += kWaves * kRound) {
        load_sums(j0, part);
        reduce_sums(j0, part);
    }
    __syncthreads();
    const int j = min(lane, p.K - 1);
    int dup = 0;
    for (int jj = 0; jj < p.K; ++jj)
        dup += (jj < j && __builtin_amdgcn_readlane(lane_id, jj) == lane_id) ? 1 : 0;
    if (!valid_id(lane_id, p.E)) return -1;
    const int pos = s_part[j] + s_before[lane_id] + dup;
    return pos < p.S ? static_cast<int>(p.div_L(lane_id)) * p.S + pos : -1;
}

// The layout outputs of a multi-chunk batch from the count pass's table, by
// one workgroup of NT threads: totals of every column, per-expert counts and
// aligned offsets, unique tokens per rank and group, rows per rank and the
// status.  LDS: s_raw [E+1] | s_aln [E+1].  Contains barriers.
template <int NT>
__device__ void finish_layout_from_table(const LayoutParams &p, int *lds) {
    constexpr int kEPT = (EP_MAX_EXPERTS + NT - 1) / NT;
    constexpr int kBatch = 16;
    __shared__ int s_wsum[2 * NT / 64];
    __shared__ int s_bad, s_over;
    int *s_raw = lds;
    int *s_aln = s_raw + (p.E + 1);
    const int tid = threadIdx.x;
    const I32Buffer table(p.table, static_cast<uint32_t>(p.nchunks) * p.pitch);
    if (tid == 0) s_over = 0;
    // every column has one owner; the last one (bad ids) sets s_bad
    for (int col = tid; col < p.ncols; col += NT) {
        int tot = 0;
        for (int c0 = 0; c0 < p.nchunks; c0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                v[q] = table.load(static_cast<uint32_t>(c0 + q) * p.pitch + col, c0 + q < p.nchunks);
#pragma unroll
            for (int q = 0; q < kBatch; ++q) tot += v[q];
        }
        if (col < p.E) {
            s_raw[col] = tot;
            p.expert_count[col] = tot;
            if (p.cumulative) p.cumulative[col] += tot;
        } else if (col < p.E + p.R) {
            p.rank_token_count[col - p.E] = tot;
        } else if (col < p.E + p.R + p.G) {
            if (p.group_token_count) p.group_token_count[col - p.E - p.R] = tot;
        } else {
            s_bad = tot;
        }
    }
    __syncthreads();
    block_scan_counts<NT, kEPT>(p, s_raw, s_aln, s_raw, s_wsum);
    __syncthreads();
    for (int e = tid; e < p.E; e += NT) p.expert_offset[e] = s_aln[e] - s_aln[static_cast<int>(p.div_L(e)) * p.L];
    if (finish_ranks<NT>(p, s_aln, s_raw)) atomicOr(&s_over, 1);
    __syncthreads();
    if (tid == 0) *p.status = status_code(s_bad > 0, s_over);
}

// Layout and dispatch of a multi-chunk batch (A = 1, at most kMaxCallChunks
// chunks) in the launch after the count pass, on a 1-D grid of
// kLeadWorkgroups + T * splits workgroups: workgroup 0 writes the layout
// outputs from the table, and copy workgroup (t, run) derives token t's
// slots, writes them if run == 0, and dispatches column run `run` of its
// row.
template <int VPT, int CR>
__global__ __launch_bounds__(kCopyThreads) void dispatch_chunks_kernel(LayoutParams p, CopyParams c,
                                                                       DispatchArgs a) {
    extern __shared__ __align__(16) int smem[];
    __shared__ int s_part[EP_MAX_TOPK];
    const int b = blockIdx.x;
    if (b < kLeadWorkgroups) {
        if (b == 0) finish_layout_from_table<kCopyThreads>(p, smem);
        return;
    }
    int t, run;
    copy_role(b, p.T, &t, &run);
    const int v0 = run * (kCopyThreads * VPT) + threadIdx.x;
    u32x4 buf[VPT];
    // early sums pay when the kernel still fits 64 VGPRs (16 workgroups per
    // CU) or when a batch of more than 64 chunks needs several rounds of
    // resident workgroups anyway
    constexpr bool kEarlySums = CR > 1 || VPT <= 4;
    const int32_t lane_slot = token_slots_in_chunk<kCopyThreads, CR, kEarlySums>(
        p, t, t / p.chunk_tokens, smem, s_part, [&] { load_token_row<VPT>(c, a, t, v0, buf); });
    const bool meta = run == 0;
    if (meta && static_cast<int>(threadIdx.x) < p.K)
        p.token_slot[static_cast<int64_t>(t) * p.K + threadIdx.x] = lane_slot;
    store_token_rows<VPT, kCopyThreads, false, true>(c, a, t, v0, meta, lane_slot, buf);
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
    const int64_t tr = (static_cast<int64_t>(E) * w.nchunks * 4 + 255) / 256 * 256;
    w.count_t_off = w.table_off + (w.nchunks * w.pitch * 4 + 255) / 256 * 256;
    w.excl_t_off = w.count_t_off + tr;
    w.bytes = w.excl_t_off + tr;
    return w;
}

hipError_t launch_layout(const LayoutParams &lp, hipStream_t stream) {
    LayoutParams p = lp;
    p.count_t = p.excl_t = nullptr;  // only the one-call path reads them
    // Walking waves per chunk: as many as the per-(wave, expert) cursors
    // allow within 64 KB of LDS.
    if (p.E <= 512) return launch_assign<16>(p, stream);
    if (p.E <= 1024) return launch_assign<8>(p, stream);
    return launch_assign<4>(p, stream);
}

hipError_t launch_layout_dispatch(const LayoutParams &p, const CopyParams &c, const DispatchArgs &a,
                                  hipStream_t stream) {
    // the single-kernel form has larger workgroups: its slot derivation is
    // on the critical path, and 256 threads share it faster than 128
    // Past 64 ranks one workgroup builds the rank map of the single-kernel
    // form chunk by chunk, and at four chunks that outlasts the dispatch: the
    // count pass plus one kernel took 25.2 µs against 32.7 µs (T = 512,
    // E = 1024, R = 128), while at two or three chunks the single kernel
    // stays ahead (16.4 against 26.8 µs at T = 200, R = 256).
    const bool one_chunk = p.T > 0 && static_cast<int64_t>(p.T) * p.K <= kFusedMaxEntries &&
                           (p.nchunks <= 3 || p.R <= 64);
    // The single kernel aims at half the copy kernels' workgroups: each of
    // them builds the batch's histograms, and at 512 tokens 1024 workgroups
    // took the step from 29.9 to 26.7 µs against 2048 (at 128 tokens a row
    // has only four workgroups' worth of vectors either way).
    int32_t splits, vpt;
    copy_grid(c.T, c.nvec, one_chunk ? kFusedThreads : kCopyThreads, &splits, &vpt,
              one_chunk ? kFusedWorkgroups : kCopyWorkgroups);
    CopyParams cp = c;
    cp.vpt = vpt;
    if (!one_chunk && p.T > 0 && p.nchunks <= kMaxCallChunks && p.A == 1) {
        const int64_t blocks = kLeadWorkgroups + static_cast<int64_t>(c.T) * splits;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        const dim3 grid(static_cast<uint32_t>(blocks));
        // count pass (with the expert-major arrays), then one launch that
        // finishes the layout and dispatches, each workgroup deriving its
        // token's slots
        const size_t lds_count = sizeof(int) * (kChunkEntries + p.pitch + 2 * (p.E + 1));
        // two workgroups per chunk: expert counts and the token pass side by side
        layout_count_kernel<<<2 * p.nchunks, kCountThreads, lds_count, stream>>>(p);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const size_t lds = sizeof(int) * 2 * (p.E + 1);
        static_assert(kMaxChunkRounds == 2, "the launch instantiates one and two rounds");
        const bool two_rounds = p.nchunks > 64;
        switch (vpt) {
#define EP_DISPATCH_CHUNKS_CASE(V)                                                         \
    case V:                                                                                \
        if (two_rounds)                                                                    \
            dispatch_chunks_kernel<V, 2><<<grid, kCopyThreads, lds, stream>>>(p, cp, a);   \
        else                                                                               \
            dispatch_chunks_kernel<V, 1><<<grid, kCopyThreads, lds, stream>>>(p, cp, a);   \
        break;
            EP_DISPATCH_CHUNKS_CASE(1)
            EP_DISPATCH_CHUNKS_CASE(2)
            EP_DISPATCH_CHUNKS_CASE(3)
            EP_DISPATCH_CHUNKS_CASE(4)
            EP_DISPATCH_CHUNKS_CASE(5)
            EP_DISPATCH_CHUNKS_CASE(6)
            EP_DISPATCH_CHUNKS_CASE(7)
            EP_DISPATCH_CHUNKS_CASE(8)
#undef EP_DISPATCH_CHUNKS_CASE
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (!one_chunk) {
        const hipError_t err = launch_layout(p, stream);
        if (err != hipSuccess || p.T == 0) return err;
        return launch_dispatch(c, a, stream);
    }
    const dim3 grid(c.T, splits + 1);
    // LDS: the larger of the layout workgroup's (ids, histogram, aligned
    // scan) and a dispatch workgroup's (two histograms and a scan)
    const size_t lds = sizeof(int) * std::max<size_t>(kChunkEntries + p.pitch + p.E + 1,
                                                      3 * static_cast<size_t>(p.E) + 2);
    switch (vpt) {
#define EP_LAYOUT_DISPATCH_CASE(V)                                                                   \
    case V:                                                                                          \
        if (p.nchunks == 1)                                                                          \
            layout_dispatch_kernel<V, kChunkEntries><<<grid, kFusedThreads, lds, stream>>>(         \
                p.topk_idx, a.x, p.T, p.K, p.E, cp.nvec, p, cp, a);                                 \
        else                                                                                         \
            layout_dispatch_kernel<V, kFusedMaxEntries><<<grid, kFusedThreads, lds, stream>>>(      \
                p.topk_idx, a.x, p.T, p.K, p.E, cp.nvec, p, cp, a);                                 \
        break;
        EP_LAYOUT_DISPATCH_CASE(1)
        EP_LAYOUT_DISPATCH_CASE(2)
        EP_LAYOUT_DISPATCH_CASE(3)
        EP_LAYOUT_DISPATCH_CASE(4)
        EP_LAYOUT_DISPATCH_CASE(5)
        EP_LAYOUT_DISPATCH_CASE(6)
        EP_LAYOUT_DISPATCH_CASE(7)
        EP_LAYOUT_DISPATCH_CASE(8)
#undef EP_LAYOUT_DISPATCH_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace epget
