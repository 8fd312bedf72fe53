// Group slots of the two-level path for gfx950.
//
// "DeepEP V2 ElasticBuffer 架构深度分析" (hybrid dispatch; logical topology
// block) and "第 3 章 V1：Buffer 初始化与通信域建立" §3.2 (ranks grouped by
// eight) send a token once to every scale-out group it reaches.  The group stage needs, per group, the
// row of each such token in the group buffer: a stable compaction of the
// tokens whose is_token_in_rank bytes are nonzero on any of the group's
// ranks, capped at the group's SG rows.
#include "../../include/ep_get.h"
#include "device_common.h"

namespace epget {
namespace {

// One workgroup of NT threads per group takes the tokens in passes of
// NT * kGroupTpt.  In a pass, thread i first reads the rank bytes of tokens
// i, i + NT, i + 2 NT, ... (neighbouring lanes read neighbouring rows) and
// leaves a 0/1 flag per token in LDS; it then owns kGroupTpt consecutive
// flags, counts them, and a workgroup scan (DPP inside waves, wave totals
// through LDS) gives each thread its first position; the slots are written
// back in the first order, so the stores of a wave also cover neighbouring
// rows.  The launch picks the smallest NT whose pass holds the batch (up to
// 16384 tokens), so a batch pays its load latency once.
constexpr int kGroupTpt = 16;  // flags per thread in the scan

// kWords: the group's rank bytes are read four at a time (ranks per group a
// multiple of 4 and the map 4-byte aligned, so every word is aligned).
template <bool kWords, int NT>
__global__ __launch_bounds__(NT) void group_layout_kernel(int32_t T, int32_t R, HierParams h,
                                                          const uint8_t *__restrict__ map,
                                                          int32_t *__restrict__ group_slot) {
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
}

template <bool kWords>
void launch_group_layout_nt(int32_t T, int32_t R, const HierParams &h, const uint8_t *map, int32_t *group_slot,
                            hipStream_t stream) {
    if (T <= 64 * kGroupTpt)
        group_layout_kernel<kWords, 64><<<h.G, 64, 0, stream>>>(T, R, h, map, group_slot);
    else if (T <= 256 * kGroupTpt)
        group_layout_kernel<kWords, 256><<<h.G, 256, 0, stream>>>(T, R, h, map, group_slot);
    else
        group_layout_kernel<kWords, 1024><<<h.G, 1024, 0, stream>>>(T, R, h, map, group_slot);
}

}  // namespace

hipError_t launch_group_layout(int32_t T, int32_t R, const HierParams &h, const uint8_t *map,
                               int32_t *group_slot, hipStream_t stream) {
    if (h.ranks_per_group % 4 == 0 && reinterpret_cast<uintptr_t>(map) % 4 == 0)
        launch_group_layout_nt<true>(T, R, h, map, group_slot, stream);
    else
        launch_group_layout_nt<false>(T, R, h, map, group_slot, stream);
    return hipGetLastError();
}

}  // namespace epget
