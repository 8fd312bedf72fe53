// Bandwidth probes for gfx950: a streaming read, a streaming write and a
// copy of a large buffer, in the access shapes the row kernels use (16-byte
// vectors, neighbouring lanes on neighbouring vectors, four vectors per
// thread in flight), and the combine's and the dispatch's read : write mixes
// (8 planes folded into one, one plane stored to 8) without their routing,
// in several workgroup shapes each.
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

// The combine's data movement without its routing: each thread reads V
// vectors of each of k = 8 planes of n vectors (non-temporal), folds the
// planes and stores V vectors (non-temporal), 8 : 1 reads to writes.
template <int V, int NT>
__global__ __launch_bounds__(NT) void gather_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                    int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * NT * V + threadIdx.x;
    u32x4 v[8][V];
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int64_t i = base + q * NT;
            v[p][q] = __builtin_nontemporal_load(src + p * n + (i < n ? i : n - 1));
        }
#pragma unroll
    for (int q = 0; q < V; ++q) {
        u32x4 acc = v[0][q];
#pragma unroll
        for (int p = 1; p < 8; ++p) acc ^= v[p][q];
        const int64_t i = base + q * NT;
        if (i < n) __builtin_nontemporal_store(acc, dst + i);
    }
}

// The dispatch's data movement without its routing: each thread reads V
// vectors (non-temporal) and stores them to each of k = 8 planes (plain
// stores), 1 : 8, with or without a wait for each plane's stores.
template <int V, int NT, bool kWait>
__global__ __launch_bounds__(NT) void scatter_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                     int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * NT * V + threadIdx.x;
    u32x4 v[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        const int64_t i = base + q * NT;
        v[q] = __builtin_nontemporal_load(src + (i < n ? i : n - 1));
    }
    for (int p = 0; p < 8; ++p) {
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int64_t i = base + q * NT;
            if (i < n) dst[p * n + i] = v[q];
        }
        if (kWait) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
}

// The shapes measured: (vectors per thread, threads per workgroup[, wait]).
struct MixShape {
    int v, nt, wait;
};
constexpr MixShape kGatherShapes[] = {{1, 256, 0}, {2, 256, 0}, {4, 256, 0}, {1, 896, 0}, {2, 448, 0}, {1, 1024, 0}};
constexpr MixShape kScatterShapes[] = {{1, 256, 0}, {2, 256, 1}, {4, 256, 0}, {4, 256, 1},
                                       {7, 128, 0}, {7, 128, 1}, {8, 128, 1}};

template <int V, int NT>
void launch_gather(const u32x4 *s, u32x4 *d, int64_t n, hipStream_t st) {
    gather_kernel<V, NT><<<static_cast<uint32_t>((n + NT * V - 1) / (NT * V)), NT, 0, st>>>(s, d, n);
}

template <int V, int NT, bool W>
void launch_scatter(const u32x4 *s, u32x4 *d, int64_t n, hipStream_t st) {
    scatter_kernel<V, NT, W><<<static_cast<uint32_t>((n + NT * V - 1) / (NT * V)), NT, 0, st>>>(s, d, n);
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

// Number of gather and scatter shapes; shape i is described by
// ep_probe_mix_shape (vectors per thread, threads, wait flag).
int ep_probe_mix_shapes(int scatter) {
    return scatter ? static_cast<int>(sizeof kScatterShapes / sizeof kScatterShapes[0])
                   : static_cast<int>(sizeof kGatherShapes / sizeof kGatherShapes[0]);
}

int ep_probe_mix_shape(int scatter, int i, int *vectors, int *threads, int *wait) {
    if (i < 0 || i >= ep_probe_mix_shapes(scatter)) return -1;
    const MixShape m = scatter ? kScatterShapes[i] : kGatherShapes[i];
    *vectors = m.v;
    *threads = m.nt;
    *wait = m.wait;
    return 0;
}

// Gather (scatter == 0): src holds 8 planes of `bytes` (8 * bytes in all),
// dst one plane.  Scatter: src holds one plane of `bytes`, dst 8 planes.
// `shape` picks the workgroup shape.
int ep_probe_mix(int scatter, int shape, const void *src, void *dst, int64_t bytes, void *stream) {
    if (bytes < 16 || bytes % 16 || !src || !dst || reinterpret_cast<uintptr_t>(src) % 16 ||
        reinterpret_cast<uintptr_t>(dst) % 16 || bytes / 16 > (int64_t{1} << 36))
        return -1;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    u32x4 *d = static_cast<u32x4 *>(dst);
    const int64_t n = bytes / 16;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (!scatter) {
        switch (shape) {
            case 0: launch_gather<1, 256>(s, d, n, st); break;
            case 1: launch_gather<2, 256>(s, d, n, st); break;
            case 2: launch_gather<4, 256>(s, d, n, st); break;
            case 3: launch_gather<1, 896>(s, d, n, st); break;
            case 4: launch_gather<2, 448>(s, d, n, st); break;
            case 5: launch_gather<1, 1024>(s, d, n, st); break;
            default: return -1;
        }
    } else {
        switch (shape) {
            case 0: launch_scatter<1, 256, false>(s, d, n, st); break;
            case 1: launch_scatter<2, 256, true>(s, d, n, st); break;
            case 2: launch_scatter<4, 256, false>(s, d, n, st); break;
            case 3: launch_scatter<4, 256, true>(s, d, n, st); break;
            case 4: launch_scatter<7, 128, false>(s, d, n, st); break;
            case 5: launch_scatter<7, 128, true>(s, d, n, st); break;
            case 6: launch_scatter<8, 128, true>(s, d, n, st); break;
            default: return -1;
        }
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
