// Two-level (hierarchical) path for gfx950: group slots, the group stage of
// dispatch and combine, and the expansion inside a group.
//
// "DeepEP V2 ElasticBuffer 架构深度分析" (hybrid dispatch; logical topology
// block) and "第 3 章 V1：Buffer 初始化与通信域建立" §3.2 (ranks grouped by
// eight) send a token once to every scale-out group it reaches and expand
// it inside the group.  The group stage needs, per group, the row of each
// such token in the group buffer: a stable compaction of the tokens whose
// is_token_in_rank bytes are nonzero on any of the group's ranks, capped at
// the group's SG rows.  The combine mirrors it: per (token, group) the
// partial sum of the token's entries in the group, rounded to bf16 (what
// would cross the scale-out link), then the sum of the group rows.
#include "../../include/ep_get.h"
#include "device_common.h"
#include "hier_internal.h"

namespace epget {
namespace {

// Group slots of a batch of up to 4096 tokens.  One workgroup of NT threads
// per group takes the tokens in passes of NT * kGroupTpt.  In a pass, thread
// i first reads the rank bytes of tokens i, i + NT, i + 2 NT, ...
// (neighbouring lanes read neighbouring rows) and leaves a 0/1 flag per
// token in LDS; it then owns kGroupTpt consecutive flags, counts them, and a
// workgroup scan (DPP inside waves, wave totals through LDS) gives each
// thread its first position; the slots are written back in the first order,
// so the stores of a wave also cover neighbouring rows.  The launch picks the
// smallest NT whose pass holds the batch, so the batch is one pass and pays
// its load latency once.
constexpr int kGroupTpt = 16;  // flags per thread in the scan

// kWords: the group's rank bytes are read four at a time (ranks per group a
// multiple of 4 and the map 4-byte aligned, so every word is aligned).
template <bool kWords, int NT>
__global__ __launch_bounds__(NT) void group_layout_kernel(int32_t T, int32_t R, HierParams h,
                                                          const uint8_t *__restrict__ map,
                                                          int32_t *__restrict__ group_slot,
                                                          int32_t *__restrict__ status) {
    constexpr int kPass = NT * kGroupTpt;
    __shared__ __align__(16) uint8_t s_flag[kPass];
    __shared__ int s_first[NT];
    __shared__ uint32_t s_bits[NT];
    __shared__ int s_wsum[NT / 64];
    const int g = blockIdx.x;
    const int i = threadIdx.x, lane = __lane_id(), w = i >> 6;
    const int r0 = g * h.ranks_per_group;
    int carry = 0;
    for (int base = 0; base < T; base += kPass) {
        uint32_t in[kGroupTpt];
#pragma unroll
        for (int k = 0; k < kGroupTpt; ++k) in[k] = 0;
        // rank by rank (word by word), so the loads of all the tokens issue
        // together; a k whose NT tokens all lie past T loads nothing
        for (int r = 0; r < h.ranks_per_group; r += kWords ? 4 : 1) {
#pragma unroll
            for (int k = 0; k < kGroupTpt; ++k) {
                if (base + k * NT >= T) break;
                const int t = min(base + i + k * NT, T - 1);
                const uint8_t *b = map + static_cast<int64_t>(t) * R + r0 + r;
                in[k] |= kWords ? *reinterpret_cast<const uint32_t *>(b) : *b;
            }
        }
#pragma unroll
        for (int k = 0; k < kGroupTpt; ++k) s_flag[i + k * NT] = (base + i + k * NT < T && in[k]) ? 1 : 0;
        __syncthreads();
        // flags base + i*kGroupTpt ... as bits: byte b of a word is bit 8b
        const u32x4 f = *reinterpret_cast<const u32x4 *>(s_flag + i * kGroupTpt);
        uint32_t bits = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t v = f[q];
            bits |= ((v & 1u) | ((v >> 7) & 2u) | ((v >> 14) & 4u) | ((v >> 21) & 8u)) << (4 * q);
        }
        const int n = __popc(bits);
        const int incl = wave_inclusive_sum(n);
        if (lane == 63) s_wsum[w] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int q = 0; q < NT / 64; ++q) {
            const int v = s_wsum[q];
            before += q < w ? v : 0;
            total += v;
        }
        s_first[i] = carry + before + incl - n;
        s_bits[i] = bits;
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < kGroupTpt; ++k) {
            if (base + k * NT >= T) break;
            const int e = i + k * NT;  // token base + e, owned by thread e / kGroupTpt
            const int t = base + e;
            if (t < T) {
                const uint32_t ob = s_bits[e / kGroupTpt];
                const int b = e % kGroupTpt;
                const int pos = s_first[e / kGroupTpt] + __popc(ob & ((1u << b) - 1u));
                group_slot[static_cast<int64_t>(t) * h.G + g] =
                    ((ob >> b) & 1u) && pos < h.SG ? g * h.SG + pos : -1;
            }
        }
        carry += total;
        __syncthreads();  // LDS is rewritten by the next pass
    }
    // more tokens reach the group than it has rows: lower the status to the
    // capacity error, keeping a lower (bad-id) code already there
    if (status && i == 0 && carry > h.SG) atomicMin(status, EP_ERR_CAPACITY);
}

// Group slots of a batch of more than 4096 tokens: tiles of kTileTokens
// tokens, one workgroup per (tile, group), all running at once.  A
// workgroup finds how many tokens of the earlier tiles reach its group, then
// places its own tile as one pass of group_layout_kernel does (two flags per
// thread).  Two ways to find the earlier tiles' count:
//   - kPrefixed: three launches.  group_tile_count_kernel writes each
//     (tile, group) count into the group slot of the tile's first token,
//     group_tile_scan_kernel turns those counts into exclusive prefixes in
//     place, and each placing workgroup reads its own tile's prefix before
//     it overwrites the tile; no workgroup reads a slot another one writes.
//   - otherwise one launch, in which each workgroup recounts the earlier
//     tiles (reading their rank bytes again, four tokens per thread in
//     flight, together with its own tile's).  The recount grows with the
//     square of the batch: the last tile's workgroup reads nearly the whole
//     map.
// A single workgroup per group walking the batch pass after pass paid the
// map's load latency on one CU at every pass.
constexpr int kTileThreads = 1024;
constexpr int kTileTpt = 2;
constexpr int kRecountTpt = 4;
constexpr int kTileTokens = kTileThreads * kTileTpt;

// Smallest tile count that takes the three launches.  Measured (µs, R = 16,
// G = 2): recount 6.2 at 4 tiles, 9.5 at 8, 30.2 at 32; three launches
// 8.2-8.8 at any size up to 64 tiles (and at R = 1024, G = 128, 32768
// tokens: 84 against 418).
constexpr int kPrefixMinTiles = 7;

// Whether token t reaches group g, for the kTileTpt tokens base + i + k *
// kTileThreads of a tile (tokens past T give 0).
template <bool kWords>
__device__ __forceinline__ void tile_flags(int32_t T, int32_t R, const HierParams &h, const uint8_t *map, int g,
                                           int base, uint32_t (&in)[kTileTpt]) {
    const int i = threadIdx.x, r0 = g * h.ranks_per_group;
#pragma unroll
    for (int k = 0; k < kTileTpt; ++k) in[k] = 0;
    for (int r = 0; r < h.ranks_per_group; r += kWords ? 4 : 1) {
#pragma unroll
        for (int k = 0; k < kTileTpt; ++k) {
            const int t = min(base + i + k * kTileThreads, T - 1);
            const uint8_t *b = map + static_cast<int64_t>(t) * R + r0 + r;
            in[k] |= kWords ? *reinterpret_cast<const uint32_t *>(b) : *b;
        }
    }
#pragma unroll
    for (int k = 0; k < kTileTpt; ++k) in[k] = (base + i + k * kTileThreads < T && in[k]) ? 1u : 0u;
}

// Pass 1 of the three-launch form: tokens of tile blockIdx.x reaching group
// blockIdx.y, written to group_slot[first token of the tile, g].
template <bool kWords>
__global__ __launch_bounds__(kTileThreads) void group_tile_count_kernel(int32_t T, int32_t R, HierParams h,
                                                                        const uint8_t *__restrict__ map,
                                                                        int32_t *__restrict__ group_slot) {
    __shared__ int s_wsum[kTileThreads / 64];
    const int c = blockIdx.x, g = blockIdx.y;
    const int i = threadIdx.x, lane = __lane_id(), w = i >> 6;
    const int base = c * kTileTokens;
    uint32_t in[kTileTpt];
    tile_flags<kWords>(T, R, h, map, g, base, in);
    int n = 0;
#pragma unroll
    for (int k = 0; k < kTileTpt; ++k) n += static_cast<int>(in[k]);
    const int incl = wave_inclusive_sum(n);
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    if (i == 0) {
        int total = 0;
#pragma unroll
        for (int q = 0; q < kTileThreads / 64; ++q) total += s_wsum[q];
        group_slot[static_cast<int64_t>(base) * h.G + g] = total;
    }
}

// Pass 2: for group blockIdx.x, the tile counts left by pass 1 (in the slot
// of each tile's first token) become exclusive prefixes, in place, 1024
// tiles at a time.  (Pass 3's last tile reports an overflow.)
__global__ __launch_bounds__(kTileThreads) void group_tile_scan_kernel(int32_t ntiles, HierParams h,
                                                                       int32_t *__restrict__ group_slot) {
    __shared__ int s_wsum[kTileThreads / 64];
    const int g = blockIdx.x;
    const int i = threadIdx.x, lane = __lane_id(), w = i >> 6;
    int carry = 0;
    for (int c0 = 0; c0 < ntiles; c0 += kTileThreads) {
        const int c = c0 + i;
        int32_t *at = group_slot + (static_cast<int64_t>(min(c, ntiles - 1)) * kTileTokens) * h.G + g;
        const int v = c < ntiles ? *at : 0;
        const int incl = wave_inclusive_sum(v);
        if (lane == 63) s_wsum[w] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int q = 0; q < kTileThreads / 64; ++q) {
            const int s = s_wsum[q];
            before += q < w ? s : 0;
            total += s;
        }
        if (c < ntiles) *at = carry + before + incl - v;
        carry += total;
        __syncthreads();  // s_wsum is rewritten by the next round
    }
}

template <bool kWords, bool kPrefixed>
__global__ __launch_bounds__(kTileThreads) void group_tiles_kernel(int32_t T, int32_t R, HierParams h,
                                                                   const uint8_t *__restrict__ map,
                                                                   int32_t *__restrict__ group_slot,
                                                                   int32_t *__restrict__ status) {
    __shared__ uint8_t s_flag[kTileTokens];
    __shared__ int s_first[kTileThreads];
    __shared__ uint32_t s_bits[kTileThreads];
    __shared__ int s_wsum[kTileThreads / 64];
    __shared__ int s_prefix;
    const int c = blockIdx.x, g = blockIdx.y;
    const int i = threadIdx.x, lane = __lane_id(), w = i >> 6;
    const int r0 = g * h.ranks_per_group;
    const int base = c * kTileTokens;
    // the prefix the scan left in the slot of the tile's first token, read
    // before any thread of this workgroup overwrites it
    if (kPrefixed && i == 0) s_prefix = group_slot[static_cast<int64_t>(base) * h.G + g];
    // the tile's own rank bytes first, so that their loads are in flight
    // with the recount's
    uint32_t in_tile[kTileTpt];
    tile_flags<kWords>(T, R, h, map, g, base, in_tile);
    // 1. tokens before the tile that reach the group, kRecountTpt per thread
    // in flight (without a prefix)
    int cnt = 0;
    for (int t0 = i; !kPrefixed && t0 < base; t0 += kRecountTpt * kTileThreads) {
        uint32_t in[kRecountTpt];
#pragma unroll
        for (int k = 0; k < kRecountTpt; ++k) in[k] = 0;
        for (int r = 0; r < h.ranks_per_group; r += kWords ? 4 : 1) {
#pragma unroll
            for (int k = 0; k < kRecountTpt; ++k) {
                if (t0 - i + k * kTileThreads >= base) break;
                const int t = min(t0 + k * kTileThreads, base - 1);
                const uint8_t *b = map + static_cast<int64_t>(t) * R + r0 + r;
                in[k] |= kWords ? *reinterpret_cast<const uint32_t *>(b) : *b;
            }
        }
#pragma unroll
        for (int k = 0; k < kRecountTpt; ++k) cnt += (t0 + k * kTileThreads < base && in[k]) ? 1 : 0;
    }
    const int cnt_incl = wave_inclusive_sum(cnt);
    if (lane == 63) s_wsum[w] = cnt_incl;
    // 2. the tile: flags in token order, kTileTpt consecutive flags per thread
#pragma unroll
    for (int k = 0; k < kTileTpt; ++k) s_flag[i + k * kTileThreads] = static_cast<uint8_t>(in_tile[k]);
    __syncthreads();
    int carry = 0;
    if (kPrefixed) {
        carry = s_prefix;
    } else {
#pragma unroll
        for (int q = 0; q < kTileThreads / 64; ++q) carry += s_wsum[q];
    }
    __syncthreads();
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < kTileTpt; ++q) bits |= static_cast<uint32_t>(s_flag[i * kTileTpt + q]) << q;
    const int n = __popc(bits);
    const int incl = wave_inclusive_sum(n);
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int q = 0; q < kTileThreads / 64; ++q) before += q < w ? s_wsum[q] : 0;
    s_first[i] = carry + before + incl - n;
    s_bits[i] = bits;
    // the last thread's count runs to the end of the tile: past SG, the
    // group overflows (as in group_layout_kernel)
    if (status && i == kTileThreads - 1 && carry + before + incl > h.SG) atomicMin(status, EP_ERR_CAPACITY);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTileTpt; ++k) {
        const int e = i + k * kTileThreads;  // token base + e, owned by thread e / kTileTpt
        const int t = base + e;
        if (t < T) {
            const uint32_t ob = s_bits[e / kTileTpt];
            const int b = e % kTileTpt;
            const int pos = s_first[e / kTileTpt] + __popc(ob & ((1u << b) - 1u));
            group_slot[static_cast<int64_t>(t) * h.G + g] =
                ((ob >> b) & 1u) && pos < h.SG ? g * h.SG + pos : -1;
        }
    }
}

template <bool kWords>
void launch_group_layout_nt(int32_t T, int32_t R, const HierParams &h, const uint8_t *map, int32_t *group_slot,
                            int32_t *status, hipStream_t stream) {
    if (T <= 64 * kGroupTpt) {
        group_layout_kernel<kWords, 64><<<h.G, 64, 0, stream>>>(T, R, h, map, group_slot, status);
    } else if (T <= 256 * kGroupTpt) {
        group_layout_kernel<kWords, 256><<<h.G, 256, 0, stream>>>(T, R, h, map, group_slot, status);
    } else {
        const int ntiles = (T + kTileTokens - 1) / kTileTokens;
        const dim3 grid(ntiles, h.G);
        if (ntiles >= kPrefixMinTiles) {
            group_tile_count_kernel<kWords><<<grid, kTileThreads, 0, stream>>>(T, R, h, map, group_slot);
            group_tile_scan_kernel<<<h.G, kTileThreads, 0, stream>>>(ntiles, h, group_slot);
            group_tiles_kernel<kWords, true><<<grid, kTileThreads, 0, stream>>>(T, R, h, map, group_slot, status);
        } else {
            group_tiles_kernel<kWords, false><<<grid, kTileThreads, 0, stream>>>(T, R, h, map, group_slot, status);
        }
    }
}

// Group of a valid entry slot in the two-level path: rank = slot / S,
// group = rank / (R / G).
struct GroupOf {
    int32_t S, ranks_per_group, g;
    __device__ bool operator()(int32_t s) const { return (s / S) / ranks_per_group == g; }
};

// Calls f(g, gs) for each group g, in ascending order, whose slot
// gs = gsrow[g] is a group row (0 <= gs < G*SG).  With few groups (kWide
// false) the slots are read one by one through the scalar cache.  With many,
// lane l of a wave reads the slot of group g0 + l and a ballot marks the
// valid ones, so a token costs one load per 64 groups and one step per group
// it reaches, whatever G is; the mask is wave-uniform, and every lane of the
// wave must take part.  The two forms are separate instantiations: the wide
// one holds more registers, which the few-group kernels cannot spare.
constexpr int kNarrowGroups = 8;  // the largest G that takes the scalar walk

template <bool kWide, class F>
__device__ __forceinline__ void for_each_group_row(const HierParams &h, const int32_t *gsrow, F &&f) {
    if constexpr (!kWide) {
        for (int g = 0; g < h.G; ++g) {
            const int32_t gs = gsrow[g];
            if (gs >= 0 && gs < h.group_rows) f(g, gs);
        }
    } else {
        const int lane = __lane_id();
        for (int g0 = 0; g0 < h.G; g0 += 64) {
            const int32_t gs_l = gsrow[min(g0 + lane, h.G - 1)];
            uint64_t m = __ballot(g0 + lane < h.G && gs_l >= 0 && gs_l < h.group_rows);
            while (m) {
                const int b = __builtin_ctzll(m);
                m &= m - 1;
                f(g0 + b, __builtin_amdgcn_readlane(gs_l, b));
            }
        }
    }
}

// Whether a batch's group rows are too many for the 256 MB last-level cache
// to hold them between two stages: the estimate is min(G, K) rows per token.
// Past 192 MiB the stages that write group rows (the dispatch's first, the
// combine's partials) store them with the non-temporal hint; below it
// plainly, so that the next stage finds them in the cache.  Two-level steps
// (H = 7168, G = 2; µs, plain → non-temporal, group rows by the estimate):
//   T = 4096, R = 8 (117 MB)     278.4 → 287.5
//   T = 6144, R = 16 (176 MB)    418.7 → 422.0
//   T = 9000, R = 16 (258 MB)    632.9 → 610.6
//   T = 12000, R = 16 (344 MB)   860.2 → 811.4
//   T = 16384, R = 16 (470 MB)  1171.5 → 1106.7
// and the 8192-token Zipf batch with 8 KB rows (134 MB) 301.3 → 309.6.
constexpr int64_t kGroupStreamBytes = int64_t(192) << 20;

bool stream_group_rows(const CopyParams &c, const HierParams &h) {
    const int64_t per_token = h.G < c.K ? h.G : c.K;
    return static_cast<int64_t>(c.T) * per_token * c.nvec * 16 > kGroupStreamBytes;
}

// Two-level dispatch, stage 1: token t's row, loaded once, to its row in
// every group it reaches (kStream: with the non-temporal hint).
template <int VPT, bool kWide, bool kStream>
__global__ __launch_bounds__(kCopyThreads) void group_dispatch_kernel(CopyParams c, HierParams h,
                                                                      const uint16_t *__restrict__ x,
                                                                      const int32_t *__restrict__ group_slot,
                                                                      uint16_t *__restrict__ group_buf) {
    const int t = blockIdx.x;
    const int v0 = blockIdx.y * (kCopyThreads * VPT) + threadIdx.x;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x) + static_cast<int64_t>(t) * c.nvec;
    u32x4 buf[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) buf[v] = __builtin_nontemporal_load(src + min(v0 + v * kCopyThreads, c.nvec - 1));
    u32x4 *rows = reinterpret_cast<u32x4 *>(group_buf);
    for_each_group_row<kWide>(h, group_slot + static_cast<int64_t>(t) * h.G, [&](int, int32_t gs) {
        u32x4 *dst = rows + static_cast<int64_t>(gs) * c.nvec;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int col = v0 + v * kCopyThreads;
            if (col >= c.nvec) continue;
            if constexpr (kStream)
                __builtin_nontemporal_store(buf[v], dst + col);
            else
                dst[col] = buf[v];
        }
        if (VPT >= kRowWaitMinVpt) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    });
}

// Two-level combine, stage 1: for each group the token reaches, the partial
// sum over the token's entries in that group, rounded to bf16 into the
// group buffer row group_slot[t,g].  With K <= KG the K rows are loaded once
// and each group folds its own entries from registers (ascending j, as in
// gather_fold); gathering per group instead kept half as many loads in
// flight and loaded row 0 for the other groups' entries: 18 µs slower on a
// 4096-token step with four groups, 22 µs on 16384 tokens with two.
// kStream stores the partials with the non-temporal hint.
template <int KG, bool kWide, bool kStream>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_partial_kernel(
    CopyParams c, HierParams h, const uint16_t *__restrict__ y, const int32_t *__restrict__ slot,
    const float *__restrict__ w, const int32_t *__restrict__ group_slot,
    uint16_t *__restrict__ group_buf) {
    const int t = blockIdx.x;
    const int32_t *srow = slot + static_cast<int64_t>(t) * c.K;
    const float *wrow = w ? w + static_cast<int64_t>(t) * c.K : nullptr;
    const int col = blockIdx.y * blockDim.x + threadIdx.x;
    const int colc = min(col, c.nvec - 1);
    const int32_t *gsrow = group_slot + static_cast<int64_t>(t) * h.G;
    u32x4 *rows = reinterpret_cast<u32x4 *>(group_buf);
    auto store_partial = [&](int32_t gs, const float (&acc)[8]) {
        if (col >= c.nvec) return;
        u32x4 *dst = rows + static_cast<int64_t>(gs) * c.nvec + col;
        if constexpr (kStream)
            __builtin_nontemporal_store(pack_row(acc), dst);
        else
            *dst = pack_row(acc);
    };
    if (c.K <= KG) {
        // all K rows in flight once, then folded group by group from registers
        u32x4 in[KG];
        int32_t grp[KG];
        float wj[KG];
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
            const int j = min(jj, c.K - 1);
            const int32_t s = srow[j];
            const bool ok = jj < c.K && slot_ok(s, c.num_rows);
            grp[jj] = ok ? (s / h.S) / h.ranks_per_group : -1;
            wj[jj] = wrow ? wrow[j] : 1.0f;
            const int64_t row = ok ? s : 0;
            in[jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(y + row * c.H) + colc);
        }
        for_each_group_row<kWide>(h, gsrow, [&](int g, int32_t gs) {
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
            for (int jj = 0; jj < KG; ++jj) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = __builtin_fmaf(wj[jj], bf16_lo(in[jj][q]), acc[2 * q]);
                    const float hi = __builtin_fmaf(wj[jj], bf16_hi(in[jj][q]), acc[2 * q + 1]);
                    acc[2 * q] = grp[jj] == g ? lo : acc[2 * q];
                    acc[2 * q + 1] = grp[jj] == g ? hi : acc[2 * q + 1];
                }
            }
            store_partial(gs, acc);
        });
        return;
    }
    for_each_group_row<kWide>(h, gsrow, [&](int g, int32_t gs) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        gather_fold<KG>(c, y, srow, wrow, colc, GroupOf{h.S, h.ranks_per_group, g}, acc);
        store_partial(gs, acc);
    });
}

// Two-level combine, stage 2: out[t] = the sum of token t's group rows in
// ascending g, fp32 accumulate, one rounding to bf16.  Rows are gathered KG
// at a time, all in flight; a position without a valid row loads row 0 (in
// bounds) and discards it by a select, as gather_fold does.  With few groups
// every group is a position; with many (kWide) only the valid rows are,
// found 64 groups at a time by a ballot.
template <int KG, bool kWide>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_groups_kernel(
    CopyParams c, HierParams h, const uint16_t *__restrict__ group_buf, const int32_t *__restrict__ group_slot,
    uint16_t *__restrict__ out) {
    const int t = blockIdx.x;
    const int col = blockIdx.y * blockDim.x + threadIdx.x;
    const int colc = min(col, c.nvec - 1);
    const int32_t *gsrow = group_slot + static_cast<int64_t>(t) * h.G;
    const u32x4 *rows = reinterpret_cast<const u32x4 *>(group_buf);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    auto fold = [&](const u32x4 (&in)[KG], const bool (&ok)[KG]) {
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = __builtin_fmaf(1.0f, bf16_lo(in[jj][q]), acc[2 * q]);
                const float hi = __builtin_fmaf(1.0f, bf16_hi(in[jj][q]), acc[2 * q + 1]);
                acc[2 * q] = ok[jj] ? lo : acc[2 * q];
                acc[2 * q + 1] = ok[jj] ? hi : acc[2 * q + 1];
            }
        }
    };
    if constexpr (!kWide) {
        for (int g0 = 0; g0 < h.G; g0 += KG) {
            u32x4 in[KG];
            bool ok[KG];
#pragma unroll
            for (int jj = 0; jj < KG; ++jj) {
                const int32_t gs = gsrow[min(g0 + jj, h.G - 1)];
                ok[jj] = g0 + jj < h.G && gs >= 0 && gs < h.group_rows;
                const int64_t row = ok[jj] ? gs : 0;
                in[jj] = __builtin_nontemporal_load(rows + row * c.nvec + colc);
            }
            fold(in, ok);
        }
    } else {
        const int lane = __lane_id();
        for (int g0 = 0; g0 < h.G; g0 += 64) {
            const int32_t gs_l = gsrow[min(g0 + lane, h.G - 1)];
            uint64_t m = __ballot(g0 + lane < h.G && gs_l >= 0 && gs_l < h.group_rows);
            while (m) {
                u32x4 in[KG];
                bool ok[KG];
#pragma unroll
                for (int jj = 0; jj < KG; ++jj) {
                    ok[jj] = m != 0;
                    const int b = ok[jj] ? __builtin_ctzll(m) : 0;
                    m &= m - 1;
                    const int64_t row = ok[jj] ? __builtin_amdgcn_readlane(gs_l, b) : 0;
                    in[jj] = __builtin_nontemporal_load(rows + row * c.nvec + colc);
                }
                fold(in, ok);
            }
        }
    }
    if (col < c.nvec)
        __builtin_nontemporal_store(pack_row(acc), reinterpret_cast<u32x4 *>(out + static_cast<int64_t>(t) * c.H) + col);
}

// Two-level dispatch, stage 2: each group row of the token goes to the
// entries of that group (with the entry's source index and weight; an entry
// whose group row was dropped for capacity gets source -1 and weight 0, and
// its row is not written).  With
// few groups each (token, group) has workgroups of its own (blockIdx.z = g),
// so a token's groups are expanded side by side rather than one after the
// other: on a 16384-token step with two groups the dispatch took 10 µs less
// and, from the order in which the rows then arrive, the combine after it
// up to 10 µs less on 4096 tokens with four groups.
template <int VPT, bool kWide>
__global__ __launch_bounds__(kCopyThreads) void expand_kernel(CopyParams c, HierParams h,
                                                              DispatchArgs a,
                                                              const int32_t *__restrict__ group_slot,
                                                              const uint16_t *__restrict__ group_buf) {
    const int t = blockIdx.x;
    u32x4 *recv = static_cast<u32x4 *>(a.recv);
    const int v0 = blockIdx.y * (kCopyThreads * VPT) + threadIdx.x;
    const int32_t lane_slot = a.slot[static_cast<int64_t>(t) * c.K + min(static_cast<int>(__lane_id()), c.K - 1)];
    if (blockIdx.y == 0 && blockIdx.z == 0 && static_cast<int>(threadIdx.x) < c.K) {
        const int j = threadIdx.x;  // lane j of wave 0
        if (slot_ok(lane_slot, c.num_rows)) {
            const int g = (lane_slot / h.S) / h.ranks_per_group;
            const int32_t gs = group_slot[static_cast<int64_t>(t) * h.G + g];
            const bool kept = gs >= 0 && gs < h.group_rows;
            if (a.recv_src) a.recv_src[lane_slot] = kept ? t : -1;
            if (a.recv_w)
                a.recv_w[lane_slot] = !kept ? 0.0f : a.w ? a.w[static_cast<int64_t>(t) * c.K + j] : 1.0f;
        }
    }
    auto body = [&](int g, int32_t gs) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(group_buf) + static_cast<int64_t>(gs) * c.nvec;
        u32x4 buf[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) buf[v] = src[min(v0 + v * kCopyThreads, c.nvec - 1)];
        const GroupOf in_group{h.S, h.ranks_per_group, g};
        for (int j = 0; j < c.K; ++j) {
            const int32_t s = slot_of(lane_slot, j);
            if (!slot_ok(s, c.num_rows) || !in_group(s)) continue;
            u32x4 *dst = recv + static_cast<int64_t>(s) * c.nvec;
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int col = v0 + v * kCopyThreads;
                if (col < c.nvec) dst[col] = buf[v];
            }
        }
    };
    if constexpr (!kWide) {
        const int g = blockIdx.z;
        const int32_t gs = group_slot[static_cast<int64_t>(t) * h.G + g];
        if (gs >= 0 && gs < h.group_rows) body(g, gs);
    } else {
        for_each_group_row<kWide>(h, group_slot + static_cast<int64_t>(t) * h.G, body);
    }
}

}  // namespace

hipError_t launch_group_layout(int32_t T, int32_t R, const HierParams &h, const uint8_t *map,
                               int32_t *group_slot, int32_t *status, hipStream_t stream) {
    if (h.ranks_per_group % 4 == 0 && reinterpret_cast<uintptr_t>(map) % 4 == 0)
        launch_group_layout_nt<true>(T, R, h, map, group_slot, status, stream);
    else
        launch_group_layout_nt<false>(T, R, h, map, group_slot, status, stream);
    return hipGetLastError();
}

hipError_t launch_expand(const CopyParams &c, const HierParams &h, const DispatchArgs &a,
                         const int32_t *group_slot, const uint16_t *group_buf, hipStream_t stream) {
    int32_t splits, vpt;
    copy_grid(c.T, c.nvec, kCopyThreads, &splits, &vpt);
    CopyParams p = c;
    p.vpt = vpt;
    dim3 grid(c.T, splits, h.G > kNarrowGroups ? 1 : h.G);
    switch (vpt) {
#define EP_EXPAND_CASE(V)                                                                    \
    case V:                                                                                  \
        if (h.G > kNarrowGroups)                                                             \
            expand_kernel<V, true><<<grid, kCopyThreads, 0, stream>>>(p, h, a, group_slot, group_buf); \
        else                                                                                 \
            expand_kernel<V, false><<<grid, kCopyThreads, 0, stream>>>(p, h, a, group_slot, group_buf); \
        break;
        EP_EXPAND_CASE(1)
        EP_EXPAND_CASE(2)
        EP_EXPAND_CASE(3)
        EP_EXPAND_CASE(4)
        EP_EXPAND_CASE(5)
        EP_EXPAND_CASE(6)
        EP_EXPAND_CASE(7)
        EP_EXPAND_CASE(8)
#undef EP_EXPAND_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_group_dispatch(const CopyParams &c, const HierParams &h, const uint16_t *x,
                                 const int32_t *group_slot, uint16_t *group_buf, hipStream_t stream) {
    int32_t splits, vpt;
    copy_grid(c.T, c.nvec, kCopyThreads, &splits, &vpt);
    CopyParams p = c;
    p.vpt = vpt;
    dim3 grid(c.T, splits);
    const bool stream_rows = stream_group_rows(c, h);
    switch (vpt) {
#define EP_GROUP_DISPATCH_KERNEL(V, W) \
    (stream_rows ? group_dispatch_kernel<V, W, true> : group_dispatch_kernel<V, W, false>)
#define EP_GROUP_DISPATCH_CASE(V)                                                                          \
    case V:                                                                                                \
        if (h.G > kNarrowGroups)                                                                           \
            EP_GROUP_DISPATCH_KERNEL(V, true)<<<grid, kCopyThreads, 0, stream>>>(p, h, x, group_slot, group_buf); \
        else                                                                                               \
            EP_GROUP_DISPATCH_KERNEL(V, false)<<<grid, kCopyThreads, 0, stream>>>(p, h, x, group_slot, group_buf); \
        break;
        EP_GROUP_DISPATCH_CASE(1)
        EP_GROUP_DISPATCH_CASE(2)
        EP_GROUP_DISPATCH_CASE(3)
        EP_GROUP_DISPATCH_CASE(4)
        EP_GROUP_DISPATCH_CASE(5)
        EP_GROUP_DISPATCH_CASE(6)
        EP_GROUP_DISPATCH_CASE(7)
        EP_GROUP_DISPATCH_CASE(8)
#undef EP_GROUP_DISPATCH_CASE
#undef EP_GROUP_DISPATCH_KERNEL
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine_groups(const CopyParams &c, const HierParams &h, const uint16_t *group_buf,
                                 const int32_t *group_slot, uint16_t *out, hipStream_t stream) {
    int32_t splits, threads;
    combine_grid(c.T, c.nvec, &splits, &threads);
    dim3 grid(c.T, splits);
    // rows in flight per round: all G positions with few groups; with many,
    // the valid rows, of which a token has at most min(G, K)
    const bool wide = h.G > kNarrowGroups;
    const int n = wide ? (h.G < c.K ? h.G : c.K) : h.G;
#define EP_COMBINE_GROUPS(KG)                                                                          \
    do {                                                                                               \
        if (wide)                                                                                      \
            combine_groups_kernel<KG, true><<<grid, threads, 0, stream>>>(c, h, group_buf, group_slot, out); \
        else                                                                                           \
            combine_groups_kernel<KG, false><<<grid, threads, 0, stream>>>(c, h, group_buf, group_slot, out); \
    } while (0)
    if (n <= 2)
        EP_COMBINE_GROUPS(2);
    else if (n <= 4)
        EP_COMBINE_GROUPS(4);
    else
        EP_COMBINE_GROUPS(8);
#undef EP_COMBINE_GROUPS
    return hipGetLastError();
}

hipError_t launch_combine_partial(const CopyParams &c, const HierParams &h, const uint16_t *y,
                                  const int32_t *slot, const float *w, const int32_t *group_slot,
                                  uint16_t *group_buf, hipStream_t stream) {
    int32_t splits, threads;
    combine_grid(c.T, c.nvec, &splits, &threads);
    dim3 grid(c.T, splits);
    const bool wide = h.G > kNarrowGroups;
    const bool stream_rows = stream_group_rows(c, h);
#define EP_COMBINE_PARTIAL(KG, W)                                                                \
    (stream_rows ? combine_partial_kernel<KG, W, true> : combine_partial_kernel<KG, W, false>)<<< \
        grid, threads, 0, stream>>>(c, h, y, slot, w, group_slot, group_buf)
    if (c.K <= 4 && wide)
        EP_COMBINE_PARTIAL(4, true);
    else if (c.K <= 4)
        EP_COMBINE_PARTIAL(4, false);
    else if (wide)
        EP_COMBINE_PARTIAL(8, true);
    else
        EP_COMBINE_PARTIAL(8, false);
#undef EP_COMBINE_PARTIAL
    return hipGetLastError();
}

}  // namespace epget
