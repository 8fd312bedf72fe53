// Device helpers shared by the kernels of libepget: wave64 prefix sums, the
// 16-byte row copy of dispatch, and the gather-and-fold of combine with its
// bf16 packing.  Internal header.
#pragma once

#include "ep_internal.h"

namespace epget {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool slot_ok(int32_t s, int64_t num_rows) {
    return s >= 0 && s < num_rows;
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP moves: shifts
// by 1, 2, 4, 8 inside each row of 16 lanes, then the broadcasts of lane 15
// into rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes whose source is
// outside the row read 0 (bound control) and the broadcasts write 0 to the
// rows their mask leaves out, so every step is one add with a DPP operand.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
    return v;
}

// Dispatch of one token by one workgroup of NT threads, which owns the
// 16-byte column vectors v0 + v * NT (v < VPT) of the row.
// Rows are moved as 16-byte vectors whatever their element type (bf16, or
// e4m3 codes with per-row scale factors).
//
// load_token_row: the thread's vectors of x[t].  Loads are unconditional
// (the column is clamped into the row) so they issue back to back; x is read
// once, so they carry the non-temporal hint (measured about 1 µs faster on a
// 4096-token step).
template <int VPT, int NT = kCopyThreads>
__device__ __forceinline__ void load_token_row(const CopyParams &c, const DispatchArgs &a, int t, int v0,
                                               u32x4 (&buf)[VPT]) {
    const u32x4 *src = static_cast<const u32x4 *>(a.x) + static_cast<int64_t>(t) * c.nvec;
#pragma unroll
    for (int v = 0; v < VPT; ++v) buf[v] = __builtin_nontemporal_load(src + min(v0 + v * NT, c.nvec - 1));
}

// Slot j of the token, held by lane j of every wave (j < K <= 32): a
// readlane puts it in a scalar register, so walking the K rows waits on no
// memory (the slots are loaded once, with the row, before any store).
__device__ __forceinline__ int32_t slot_of(int32_t lane_slot, int j) {
    return __builtin_amdgcn_readlane(lane_slot, j);
}

// From this many vectors per thread on, a workgroup waits for one row's
// stores to complete before it issues the next row's.
constexpr int kRowWaitMinVpt = 4;

// s_waitcnt with vmcnt = 0 and the other counters at their maximum (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// store_token_rows: the vectors to the K destination rows (a row outside
// [0, num_rows) is skipped); with `meta`, also each received row's source
// token and weight and its scale factors.  lane_slot as for slot_of.  The
// weight is loaded where it is written, and its wait holds back what
// follows: with kMetaLast the source and weight go after the rows, otherwise
// before them (measured: after the rows, the 16384-token one-call step took
// 769 µs against 772; before them, the 128-token decode step 8.7 µs against
// 9.1).  Scale factors always go after the rows.
// kStream stores the rows with the non-temporal hint, for batches whose rows
// all fit in the caches: plain stores leave them dirty in L2, and the
// write-back at the end of the kernel then delays its completion (a
// 128-token decode step took 9.3 µs with plain stores and 8.7-8.9 µs with
// streaming ones, while a 16384-token step lost 5 %: there the rows leave L2
// during the kernel anyway, and streaming stores reach HBM more slowly).
template <int VPT, int NT = kCopyThreads, bool kStream = false, bool kMetaLast = false>
__device__ __forceinline__ void store_token_rows(const CopyParams &c, const DispatchArgs &a, int t, int v0,
                                                 bool meta, int32_t lane_slot, const u32x4 (&buf)[VPT]) {
    // lane j of wave 0 writes entry j's source and weight (j < K)
    const bool meta_lane = meta && static_cast<int>(threadIdx.x) < c.K && slot_ok(lane_slot, c.num_rows);
    auto write_meta = [&] {
        const int j = threadIdx.x;
        if (a.recv_src) a.recv_src[lane_slot] = t;
        if (a.recv_w) a.recv_w[lane_slot] = a.w ? a.w[static_cast<int64_t>(t) * c.K + j] : 1.0f;
    };
    if (!kMetaLast && meta_lane) write_meta();
    u32x4 *recv = static_cast<u32x4 *>(a.recv);
    for (int j = 0; j < c.K; ++j) {
        const int32_t s = slot_of(lane_slot, j);
        if (!slot_ok(s, c.num_rows)) continue;
        u32x4 *dst = recv + static_cast<int64_t>(s) * c.nvec;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int col = v0 + v * NT;
            if (col < c.nvec) {
                if (kStream)
                    __builtin_nontemporal_store(buf[v], dst + col);
                else
                    dst[col] = buf[v];
            }
        }
        if (VPT >= kRowWaitMinVpt) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    if (kMetaLast && meta_lane) write_meta();
    // per-row scale factors, one thread per block of channels, after the
    // rows so that their loads do not hold the rows' stores back.  Padded
    // rows are written whole (sf_row entries, the padding as 0).  A line
    // shared by neighbouring slots, whose workgroups on different XCDs each
    // write part of it, made the 16384-token FP8 dispatch take 242 µs; with
    // whole lines it takes 225 µs (217 µs without scales).
    if (meta && a.x_sf) {
        for (int b = threadIdx.x; b < a.sf_row; b += NT) {
            const bool pad = b >= a.nsf;
            const float v = pad ? 0.0f : a.x_sf[static_cast<int64_t>(t) * a.nsf + b];
            for (int j = 0; j < c.K; ++j) {
                const int32_t s = slot_of(lane_slot, j);
                if (slot_ok(s, c.num_rows) && !(pad && s == c.num_rows - 1))
                    a.recv_sf[s * a.sf_ts + b * a.sf_hs] = v;
            }
        }
    }
}

// The two bf16 values packed in a 32-bit word, as fp32 (low half, high half).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Two fp32 values rounded to bf16 (nearest even) and packed, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Folds the top-k rows of one token at 16-byte column colc into acc, in
// ascending j with fp32 FMA, for the entries whose slot is valid and passes
// keep(slot).  KG entries are gathered per round, all KG loads in flight; an
// entry that does not count loads row 0 instead (always in bounds) and is
// discarded by a select, so no load sits behind a branch.  The rows are read
// once, so the loads carry the non-temporal hint.
template <int KG, class Keep>
__device__ __forceinline__ void gather_fold(const CopyParams &c, const uint16_t *__restrict__ y,
                                            const int32_t *srow, const float *wrow, int colc,
                                            Keep keep, float acc[8]) {
    for (int j0 = 0; j0 < c.K; j0 += KG) {
        u32x4 in[KG];
        bool ok[KG];
        float wj[KG];
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
            const int j = min(j0 + jj, c.K - 1);
            const int32_t s = srow[j];
            ok[jj] = j0 + jj < c.K && slot_ok(s, c.num_rows) && keep(s);
            wj[jj] = wrow ? wrow[j] : 1.0f;
            const int64_t row = ok[jj] ? s : 0;
            in[jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(y + row * c.H) + colc);
        }
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = __builtin_fmaf(wj[jj], bf16_lo(in[jj][q]), acc[2 * q]);
                const float hi = __builtin_fmaf(wj[jj], bf16_hi(in[jj][q]), acc[2 * q + 1]);
                acc[2 * q] = ok[jj] ? lo : acc[2 * q];
                acc[2 * q + 1] = ok[jj] ? hi : acc[2 * q + 1];
            }
        }
    }
}

// Eight fp32 accumulators as one 16-byte vector of bf16.
__device__ __forceinline__ u32x4 pack_row(const float acc[8]) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    return o;
}

}  // namespace
}  // namespace epget
