// Bandwidth probes for gfx950: a streaming read, a streaming write and a
// copy of a large buffer, in the access shapes the row kernels use (16-byte
// vectors, neighbouring lanes on neighbouring vectors, four vectors per
// thread in flight), and the combine's and the dispatch's read : write mixes
// (k planes folded into one, one plane stored to k) without their routing.
// They measure the practical HBM ceilings that the dispatch and combine
// kernels are compared with; they are not part of the dispatch/combine path
// and live in their own library, libepprobe.so.
//
// The sizing of copies against bandwidth follows the traffic model that
// "DeepEP V2 ElasticBuffer 架构深度分析" (get_theoretical_num_sms block)
// applies to its own kernels: data movement is the cost.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPer = 4;  // vectors per thread
constexpr int64_t kTile = static_cast<int64_t>(kThreads) * kPer;

// Reads n vectors; the xor of what a thread read is stored only if it equals
// `magic` (never, for the caller's data), so the loads cannot be dropped.
template <bool kNonTemporal>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *__restrict__ src, int64_t n,
                                                        uint32_t magic, uint32_t *__restrict__ sink) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile + threadIdx.x;
    u32x4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i = base + k * kThreads;
        const u32x4 *p = src + (i < n ? i : n - 1);
        v[k] = kNonTemporal ? __builtin_nontemporal_load(p) : *p;
    }
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    if (x == magic) sink[0] = x;
}

template <bool kNonTemporal>
__global__ __launch_bounds__(kThreads) void write_kernel(u32x4 *__restrict__ dst, int64_t n, uint32_t value) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile + threadIdx.x;
    const u32x4 v = {value, value ^ 1u, value ^ 2u, value ^ 3u};
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i = base + k * kThreads;
        if (i < n) {
            if (kNonTemporal)
                __builtin_nontemporal_store(v, dst + i);
            else
                dst[i] = v;
        }
    }
}

// Non-temporal loads and plain stores, as the dispatch kernels move rows.
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                        int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile + threadIdx.x;
    u32x4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i = base + k * kThreads;
        v[k] = __builtin_nontemporal_load(src + (i < n ? i : n - 1));
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i = base + k * kThreads;
        if (i < n) dst[i] = v[k];
    }
}

// The combine's data movement without its routing: each thread reads the
// same vector of k planes of n vectors (non-temporal), folds them and
// stores one vector (non-temporal), k : 1 reads to writes.
__global__ __launch_bounds__(kThreads) void gather_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                          int64_t n, int k) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= n) return;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int p = 0; p < k; p += 8) {
        u32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = __builtin_nontemporal_load(src + static_cast<int64_t>(min(p + q, k - 1)) * n + i);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (p + q < k) acc ^= v[q];
    }
    __builtin_nontemporal_store(acc, dst + i);
}

// The dispatch's data movement without its routing: each thread reads one
// vector (non-temporal) and stores it to k planes (plain stores), 1 : k.
__global__ __launch_bounds__(kThreads) void scatter_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                           int64_t n, int k) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= n) return;
    const u32x4 v = __builtin_nontemporal_load(src + i);
    for (int p = 0; p < k; ++p) dst[static_cast<int64_t>(p) * n + i] = v;
}

// One workgroup that does nothing: back to back, the launch-to-launch floor
// of a stream, against which latency-bound steps of a few kernels are read.
__global__ __launch_bounds__(64) void empty_kernel() {}

// Grid for n vectors; 0 if the size is not usable (n < 1 or too many tiles).
uint32_t grid_for(int64_t bytes) {
    if (bytes < 16 || bytes % 16 != 0) return 0;
    const int64_t tiles = (bytes / 16 + kTile - 1) / kTile;
    return tiles > 0x7FFFFFFF ? 0 : static_cast<uint32_t>(tiles);
}

}  // namespace

extern "C" {

// Each returns 0, -1 for a bad size or pointer (bytes must be a positive
// multiple of 16; pointers 16-byte aligned, device memory), or -2 for a
// failed launch.  They only enqueue on `stream`.
int ep_probe_read(const void *src, int64_t bytes, int nontemporal, void *sink, void *stream) {
    const uint32_t g = grid_for(bytes);
    if (!g || !src || !sink || reinterpret_cast<uintptr_t>(src) % 16) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n = bytes / 16;
    if (nontemporal)
        read_kernel<true><<<g, kThreads, 0, st>>>(static_cast<const u32x4 *>(src), n, 0x9E3779B9u,
                                                  static_cast<uint32_t *>(sink));
    else
        read_kernel<false><<<g, kThreads, 0, st>>>(static_cast<const u32x4 *>(src), n, 0x9E3779B9u,
                                                   static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ep_probe_write(void *dst, int64_t bytes, int nontemporal, void *stream) {
    const uint32_t g = grid_for(bytes);
    if (!g || !dst || reinterpret_cast<uintptr_t>(dst) % 16) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n = bytes / 16;
    if (nontemporal)
        write_kernel<true><<<g, kThreads, 0, st>>>(static_cast<u32x4 *>(dst), n, 0x5A5A5A5Au);
    else
        write_kernel<false><<<g, kThreads, 0, st>>>(static_cast<u32x4 *>(dst), n, 0x5A5A5A5Au);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ep_probe_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    const uint32_t g = grid_for(bytes);
    if (!g || !src || !dst || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return -1;
    copy_kernel<<<g, kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4 *>(src),
                                                                        static_cast<u32x4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ep_probe_empty(void *stream) {
    empty_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>();
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Gather: src holds k planes of `bytes` (k * bytes in all), dst one plane.
// Scatter: src holds one plane of `bytes`, dst k planes.  1 <= k <= 64.
int ep_probe_gather(const void *src, void *dst, int64_t bytes, int k, void *stream) {
    if (bytes < 16 || bytes % 16 || k < 1 || k > 64 || !src || !dst ||
        reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return -1;
    const int64_t n = bytes / 16, g = (n + kThreads - 1) / kThreads;
    if (g > 0x7FFFFFFF) return -1;
    gather_kernel<<<static_cast<uint32_t>(g), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n, k);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ep_probe_scatter(const void *src, void *dst, int64_t bytes, int k, void *stream) {
    if (bytes < 16 || bytes % 16 || k < 1 || k > 64 || !src || !dst ||
        reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return -1;
    const int64_t n = bytes / 16, g = (n + kThreads - 1) / kThreads;
    if (g > 0x7FFFFFFF) return -1;
    scatter_kernel<<<static_cast<uint32_t>(g), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n, k);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
