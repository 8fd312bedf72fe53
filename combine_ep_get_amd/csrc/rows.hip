// Row kernels for gfx950: dispatch scatter and weighted combine.
//
// Both are pure HBM streaming.  A workgroup owns one token and a contiguous
// run of 16-byte column vectors of its row; the token's K destination slots
// and weights are workgroup-uniform, so they live in scalar registers.
//
// dispatch ("DeepEP Symmetric Memory 全面架构分析" §6.1 dispatch arguments;
// the received record of "DeepEP V2 ElasticBuffer 架构深度分析", TokenLayout
// block): each thread loads its vectors of x[t] once and stores them to all
// K destination rows — one read, K writes per vector (the row copy itself is
// in device_common.h, shared with the one-launch layout and dispatch).
//
// combine (same first page, §9.2 combine(x, handle, topk_weights)): each
// thread gathers the K rows' vectors for one column position (K loads in
// flight), folds them into eight fp32 accumulators in ascending j with fused
// multiply-add, and rounds once to bf16 (round-to-nearest-even, the
// hardware's packed bf16 conversion).
#include "../../include/ep_get.h"
#include "device_common.h"

namespace epget {
namespace {

// One workgroup of NT threads per (token, run of columns): each thread loads
// its VPT vectors of x[t] once and stores them to all K destination rows;
// the workgroup with blockIdx.y == 0 also writes the rows' metadata.
template <int VPT, int NT>
__global__ __launch_bounds__(NT) void dispatch_kernel(CopyParams c, DispatchArgs a) {
    const int t = blockIdx.x;
    const int v0 = blockIdx.y * (NT * VPT) + threadIdx.x;
    const int32_t lane_slot = a.slot[static_cast<int64_t>(t) * c.K + min(static_cast<int>(__lane_id()), c.K - 1)];
    u32x4 buf[VPT];
    load_token_row<VPT, NT>(c, a, t, v0, buf);
    store_token_rows<VPT, NT>(c, a, t, v0, blockIdx.y == 0, lane_slot, buf);
}

// e4m3 (OCP "fn": bias 7, 3 mantissa bits, largest finite 448, no
// infinities) code of v: nearest value with ties to even, magnitudes above
// 448 saturate, NaN gives 0x7F.  Below 2^-6 the grid is the subnormal step
// 2^-9; above, the mantissa is rounded at 2^(e-3) for v in [2^e, 2^(e+1)).
// Scaling by powers of two is exact and rintf rounds half to even.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a != a) return 0x7Fu;
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | static_cast<uint32_t>(rintf(a * 512.0f));
    int e = static_cast<int>((u >> 23) & 0xFFu) - 127;
    int m = static_cast<int>(rintf(ldexpf(a, 3 - e)));  // 8..16
    if (m == 16) {
        m = 8;
        e += 1;
    }
    return sign | static_cast<uint32_t>(((e + 7) << 3) | (m - 8));
}

// Per-token, per-128-channel e4m3 quantisation: 8 lanes hold a block of 128
// channels (16 bf16 each: two 16-byte loads, one 16-byte store of codes).
// With H a multiple of 128 the blocks of all tokens tile x in order: block p
// (token p / (H/128), block p % (H/128)) starts at element 128 p and owns
// scale p, so the grid walks the flat block index and a workgroup of
// kQuantThreads covers 16 * kQuantThreads consecutive channels of x, with no
// idle lanes at the row ends.
constexpr int kQuantThreads = 256;
constexpr int kQuantLanesPerBlock = 8;
constexpr int kQuantBlocksPerGroup = kQuantThreads / kQuantLanesPerBlock;

__global__ __launch_bounds__(kQuantThreads) void quantize_fp8_kernel(int64_t nblocks, const uint16_t *__restrict__ x,
                                                                     uint8_t *__restrict__ q,
                                                                     float *__restrict__ sf) {
    const int lane = threadIdx.x % kQuantLanesPerBlock;
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * kQuantBlocksPerGroup + threadIdx.x / kQuantLanesPerBlock;
    const bool live = blk < nblocks;
    const int64_t off = (live ? blk : nblocks - 1) * 128 + lane * 16;
    const u32x4 in0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + off));
    const u32x4 in1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + off) + 1);
    float f[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_lo(in0[k]);
        f[2 * k + 1] = bf16_hi(in0[k]);
        f[8 + 2 * k] = bf16_lo(in1[k]);
        f[8 + 2 * k + 1] = bf16_hi(in1[k]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(f[k]));
#pragma unroll
    for (int d = 1; d < kQuantLanesPerBlock; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kQuantLanesPerBlock));
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        f[k] *= inv;
        nan |= f[k] != f[k];
    }
    u32x4 codes;
    if (!nan) {
        // gfx950's packed conversion to OCP e4m3 rounds to nearest even; the
        // clamp gives the saturation at +-448 (a scaled value can exceed 448
        // by an ulp of fp32)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float c[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] = fminf(fmaxf(f[4 * w + k], -448.0f), 448.0f);
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], word, true);
            codes[w] = static_cast<uint32_t>(word);
        }
    } else {
        // a NaN (a NaN input, or inf times a zero scale) takes the explicit
        // encoder, which maps it to 0x7F
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) word |= f32_to_e4m3(f[4 * w + k]) << (8 * k);
            codes[w] = word;
        }
    }
    if (live) {
        *reinterpret_cast<u32x4 *>(q + off) = codes;
        if (lane == 0) sf[blk] = amax / 448.0f;
    }
}


struct KeepAll {
    __device__ bool operator()(int32_t) const { return true; }
};

// One thread per 16-byte column vector: a workgroup covers a whole row (or a
// contiguous piece of it for small batches), so each thread makes exactly
// one pass.  The gathered rows are read with the non-temporal hint (without
// it the combine after a dispatch takes half as long again), and the output
// row is stored with it too: a plain store was 4 µs faster on the 4096-token
// step but 50 µs slower on the 16384-token one and 13 µs slower with FP8
// dispatch, as the dirty output lines then have to leave the last-level
// cache during the next step.
//
// Its arguments are scalars only, all within the 14 dwords that arrive
// preloaded in SGPRs, and the workgroup width is one of them (blockDim
// would be a load of its own): no wave waits for a kernel-argument load
// before its first loads, which took about 0.2-0.3 µs off the 128- and
// 256-token steps.
template <int KG>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(
    const uint16_t *__restrict__ y, const int32_t *__restrict__ slot, const float *__restrict__ w,
    uint16_t *__restrict__ out, int32_t H, int32_t K, int32_t nvec, int32_t threads, int64_t num_rows) {
    const CopyParams c{0, H, K, nvec, 0, num_rows};
    const int t = blockIdx.x;
    const int32_t *srow = slot + static_cast<int64_t>(t) * c.K;
    const float *wrow = w ? w + static_cast<int64_t>(t) * c.K : nullptr;
    const int col = blockIdx.y * threads + threadIdx.x;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    gather_fold<KG>(c, y, srow, wrow, min(col, c.nvec - 1), KeepAll{}, acc);
    if (col < c.nvec)
        __builtin_nontemporal_store(pack_row(acc), reinterpret_cast<u32x4 *>(out + static_cast<int64_t>(t) * c.H) + col);
}

// Rows of fewer than kNarrowVectors 16-byte vectors (under 1 KB): one
// thread per (entry, vector) for the dispatch and one per (token, vector)
// for the combine, so that a workgroup spans several tokens instead of
// leaving most of its lanes idle (at 16-byte rows a token-per-workgroup
// dispatch kept one lane of 128 busy).  A batch too small to fill the chip
// this way keeps the per-token kernels, which spread it over more
// workgroups: the 128-token, 256-wide combine took 4.0 µs packed against
// 3.0 µs per token.  The combine packs rows of up to 16 vectors from 16384
// threads on; wider ones, which already fill half a wave, only from 2^20.
constexpr int kNarrowVectors = 64;
constexpr int kNarrowThreads = 256;

bool narrow_dispatch(const CopyParams &c) {
    return c.nvec < kNarrowVectors && static_cast<int64_t>(c.T) * c.K * c.nvec >= 65536;
}

bool narrow_combine(const CopyParams &c) {
    const int64_t n = static_cast<int64_t>(c.T) * c.nvec;
    return c.nvec < kNarrowVectors && ((c.nvec <= 16 && n >= 16384) || n >= (int64_t{1} << 20));
}

__global__ __launch_bounds__(kNarrowThreads) void dispatch_narrow_kernel(CopyParams c, DispatchArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kNarrowThreads + threadIdx.x;
    if (gid >= static_cast<int64_t>(c.T) * c.K * c.nvec) return;
    const int64_t e = gid / c.nvec;  // entry (t, j) = t * K + j
    const int v = static_cast<int>(gid - e * c.nvec);
    const int t = static_cast<int>(e / c.K);
    const int32_t s = a.slot[e];
    if (!slot_ok(s, c.num_rows)) return;
    // x[t] is read by its K entries, so its loads stay cached
    const u32x4 *src = static_cast<const u32x4 *>(a.x) + static_cast<int64_t>(t) * c.nvec;
    static_cast<u32x4 *>(a.recv)[static_cast<int64_t>(s) * c.nvec + v] = src[v];
    if (v == 0) {
        if (a.recv_src) a.recv_src[s] = t;
        if (a.recv_w) a.recv_w[s] = a.w ? a.w[e] : 1.0f;
    }
    if (a.x_sf) {
        // nsf <= nvec, so entry b < nsf is thread v = b's; the padding of a
        // padded row (b >= nsf) takes further rounds
        for (int b = v; b < a.sf_row; b += c.nvec) {
            const bool pad = b >= a.nsf;
            if (!(pad && s == c.num_rows - 1))
                a.recv_sf[s * a.sf_ts + b * a.sf_hs] = pad ? 0.0f : a.x_sf[static_cast<int64_t>(t) * a.nsf + b];
        }
    }
}

template <int KG>
__global__ __launch_bounds__(kNarrowThreads) void combine_narrow_kernel(
    CopyParams c, const uint16_t *__restrict__ y, const int32_t *__restrict__ slot,
    const float *__restrict__ w, uint16_t *__restrict__ out) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kNarrowThreads + threadIdx.x;
    const int64_t total = static_cast<int64_t>(c.T) * c.nvec;
    const int64_t gc = gid < total ? gid : total - 1;
    const int t = static_cast<int>(gc / c.nvec);
    const int col = static_cast<int>(gc - static_cast<int64_t>(t) * c.nvec);
    const int32_t *srow = slot + static_cast<int64_t>(t) * c.K;
    const float *wrow = w ? w + static_cast<int64_t>(t) * c.K : nullptr;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    gather_fold<KG>(c, y, srow, wrow, col, KeepAll{}, acc);
    if (gid < total)
        __builtin_nontemporal_store(pack_row(acc), reinterpret_cast<u32x4 *>(out + static_cast<int64_t>(t) * c.H) + col);
}

// combined_topk_weights: one thread per (token, top-k) entry.
__global__ __launch_bounds__(256) void combine_weights_kernel(CopyParams c, const float *__restrict__ recv_w,
                                                              const int32_t *__restrict__ slot,
                                                              float *__restrict__ combined_w) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<int64_t>(c.T) * c.K) return;
    const int32_t s = slot[i];
    combined_w[i] = slot_ok(s, c.num_rows) ? recv_w[s] : 0.0f;
}

}  // namespace

void copy_grid(int32_t T, int32_t nvec, int32_t threads, int32_t *splits, int32_t *vpt, int32_t want) {
    // Aim for at least `want` workgroups so that decode-sized batches still
    // cover the chip; large batches get one workgroup per token and several
    // vectors per thread.
    const int64_t want_blocks = want;
    int64_t need = T >= want_blocks ? 1 : (want_blocks + (T > 0 ? T : 1) - 1) / (T > 0 ? T : 1);
    int64_t v = (nvec + threads * need - 1) / (threads * need);
    if (v < 1) v = 1;
    if (v > kMaxVpt) v = kMaxVpt;
    *vpt = static_cast<int32_t>(v);
    *splits = static_cast<int32_t>((nvec + threads * v - 1) / (threads * v));
}

void combine_grid(int32_t T, int32_t nvec, int32_t *splits, int32_t *threads) {
    // One thread per column vector.  A workgroup takes a whole row when the
    // batch alone gives enough workgroups; otherwise rows are cut into
    // pieces of at least one wave so that about 2048 workgroups run.
    const int64_t want_blocks = 2048;
    const int64_t t = T > 0 ? T : 1;
    int64_t pieces = t >= want_blocks ? 1 : (want_blocks + t - 1) / t;
    int64_t n = (nvec + pieces - 1) / pieces;
    n = (n + 63) / 64 * 64;
    if (n > kCombineMaxThreads) n = kCombineMaxThreads;
    if (n < 64) n = 64;
    *threads = static_cast<int32_t>(n);
    *splits = static_cast<int32_t>((nvec + n - 1) / n);
}

hipError_t launch_dispatch(const CopyParams &c, const DispatchArgs &a, hipStream_t stream) {
    if (narrow_dispatch(c)) {
        const int64_t n = static_cast<int64_t>(c.T) * c.K * c.nvec;
        const int64_t blocks = (n + kNarrowThreads - 1) / kNarrowThreads;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        dispatch_narrow_kernel<<<static_cast<uint32_t>(blocks), kNarrowThreads, 0, stream>>>(c, a);
        return hipGetLastError();
    }
    // batches so small that rows split into one-vector pieces take the
    // wider workgroups of the single-kernel layout + dispatch (decode-sized
    // dispatch 0.4 µs faster; at two or more vectors per thread they were
    // slower)
    int32_t splits, vpt;
    copy_grid(c.T, c.nvec, kCopyThreads, &splits, &vpt);
    const bool wide = vpt == 1;
    if (wide) copy_grid(c.T, c.nvec, kFusedThreads, &splits, &vpt);
    CopyParams p = c;
    p.vpt = vpt;
    dim3 grid(c.T, splits);
    switch (vpt) {
#define EP_DISPATCH_CASE(V)                                                             \
    case V:                                                                             \
        if (wide)                                                                       \
            dispatch_kernel<V, kFusedThreads><<<grid, kFusedThreads, 0, stream>>>(p, a); \
        else                                                                            \
            dispatch_kernel<V, kCopyThreads><<<grid, kCopyThreads, 0, stream>>>(p, a);  \
        break;
        EP_DISPATCH_CASE(1)
        EP_DISPATCH_CASE(2)
        EP_DISPATCH_CASE(3)
        EP_DISPATCH_CASE(4)
        EP_DISPATCH_CASE(5)
        EP_DISPATCH_CASE(6)
        EP_DISPATCH_CASE(7)
        EP_DISPATCH_CASE(8)
#undef EP_DISPATCH_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(int32_t T, int32_t H, const uint16_t *x, uint8_t *q, float *sf,
                               hipStream_t stream) {
    const int64_t nblocks = static_cast<int64_t>(T) * (H / 128);
    const int64_t groups = (nblocks + kQuantBlocksPerGroup - 1) / kQuantBlocksPerGroup;
    if (groups > INT32_MAX) return hipErrorInvalidValue;
    quantize_fp8_kernel<<<static_cast<uint32_t>(groups), kQuantThreads, 0, stream>>>(nblocks, x, q, sf);
    return hipGetLastError();
}

hipError_t launch_combine(const CopyParams &c, const uint16_t *y, const int32_t *slot,
                          const float *w, uint16_t *out, hipStream_t stream) {
    if (narrow_combine(c)) {
        const int64_t n = static_cast<int64_t>(c.T) * c.nvec;
        const int64_t blocks = (n + kNarrowThreads - 1) / kNarrowThreads;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        const uint32_t g = static_cast<uint32_t>(blocks);
        if (c.K <= 1)
            combine_narrow_kernel<1><<<g, kNarrowThreads, 0, stream>>>(c, y, slot, w, out);
        else if (c.K <= 2)
            combine_narrow_kernel<2><<<g, kNarrowThreads, 0, stream>>>(c, y, slot, w, out);
        else if (c.K <= 4)
            combine_narrow_kernel<4><<<g, kNarrowThreads, 0, stream>>>(c, y, slot, w, out);
        else
            combine_narrow_kernel<8><<<g, kNarrowThreads, 0, stream>>>(c, y, slot, w, out);
        return hipGetLastError();
    }
    int32_t splits, threads;
    combine_grid(c.T, c.nvec, &splits, &threads);
    dim3 grid(c.T, splits);
    if (c.K <= 1) {
        combine_kernel<1><<<grid, threads, 0, stream>>>(y, slot, w, out, c.H, c.K, c.nvec, threads, c.num_rows);
    } else if (c.K <= 2) {
        combine_kernel<2><<<grid, threads, 0, stream>>>(y, slot, w, out, c.H, c.K, c.nvec, threads, c.num_rows);
    } else if (c.K <= 4) {
        combine_kernel<4><<<grid, threads, 0, stream>>>(y, slot, w, out, c.H, c.K, c.nvec, threads, c.num_rows);
    } else {
        combine_kernel<8><<<grid, threads, 0, stream>>>(y, slot, w, out, c.H, c.K, c.nvec, threads, c.num_rows);
    }
    return hipGetLastError();
}

hipError_t launch_combine_weights(const CopyParams &c, const float *recv_w, const int32_t *slot,
                                  float *combined_w, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(c.T) * c.K;
    combine_weights_kernel<<<(n + 255) / 256, 256, 0, stream>>>(c, recv_w, slot, combined_w);
    return hipGetLastError();
}

}  // namespace epget
