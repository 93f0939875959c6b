// read_probe.hip -- the device's streaming-read ceiling, for the benchmark.
//
// Not part of the library's interface (it is built into its own shared
// object, libbsa_probe.so): the benchmark reports its kernels' bandwidth both
// against the published HBM peak and against what a plain streaming read
// reaches on the same device.  Every thread reads 16-byte chunks with a
// grid-stride loop, kUnroll loads in flight, and folds them with XOR; the
// result is stored only when it matches a value it never takes in practice,
// so the loads stay but nothing is written.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                        u32x4* sink) {
    const size_t tid = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = tid;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= p[i];
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[tid] = acc;
}

// Nontemporal loads; CONTIG: workgroup b reads [b*share, (b+1)*share) with a
// block-stride loop instead of the grid-stride walk.
template <bool CONTIG>
__global__ __launch_bounds__(kThreads) void read_nt_kernel(const u32x4* __restrict__ p, size_t n16,
                                                           u32x4* sink) {
    const size_t tid = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    size_t begin, end, stride;
    if (CONTIG) {
        const size_t share = (n16 + gridDim.x - 1) / gridDim.x;
        begin = static_cast<size_t>(blockIdx.x) * share;
        end = begin + share < n16 ? begin + share : n16;
        begin += threadIdx.x;
        stride = kThreads;
    } else {
        begin = tid;
        end = n16;
        stride = static_cast<size_t>(gridDim.x) * kThreads;
    }
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = begin;
    for (; i + (kUnroll - 1) * stride < end; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < end; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[tid] = acc;
}

// Scattered 16 KiB chunks, the decode's pattern (a 32-token tile is 8 KiB of
// K and 8 KiB of V from a page anywhere in the pools): wave v of the grid
// reads chunks v, v + W, v + 2W, ... (W waves), each as 16 one-KiB wave
// loads (16 bytes per lane, nontemporal), two chunks in flight, with chunk c
// taken from position (c * P) mod the chunk count for a prime P above any
// chunk count used, which makes the map a permutation.
constexpr int kChunk16 = 1024;  // 16-byte elements per 16 KiB chunk
__global__ __launch_bounds__(kThreads) void read_chunks_kernel(const u32x4* __restrict__ p, size_t n16,
                                                               u32x4* sink) {
    const size_t tid = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const size_t wave = tid >> 6;
    const size_t nwaves = static_cast<size_t>(gridDim.x) * (kThreads / 64);
    const size_t nchunks = n16 / kChunk16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t c = wave; c < nchunks; c += 2 * nwaves) {
        u32x4 v[2][16];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const size_t cc = c + u * nwaves;
            const size_t chunk = (cc * 2654435761ull) % nchunks;
            const u32x4* q = p + chunk * kChunk16 + lane;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[u][j] = (cc < nchunks) ? __builtin_nontemporal_load(q + j * 64) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc ^= v[u][j];
    }
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[tid] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the device buffer `buf` with
// `workgroups` workgroups of 256 threads on `stream`, in access mode `mode`
// (0: grid-stride plain loads, 1: grid-stride nontemporal, 2: contiguous
// share per workgroup, 3: scattered 16 KiB chunks, which needs `bytes` to be
// a multiple of 16 KiB, and fewer than 2^31 chunks).  `sink`: device memory of at least workgroups * 256 *
// 16 bytes (normally left untouched).  Returns 0, or -1 for a bad argument,
// -2 for a failed launch.
extern "C" __attribute__((visibility("default"))) int bsa_probe_read_mode(const void* buf, size_t bytes,
                                                                          void* sink, int workgroups,
                                                                          int mode, hipStream_t stream) {
    if (!buf || !sink || workgroups < 1 || bytes % 16 != 0 || mode < 0 || mode > 3) return -1;
    const size_t nchunks = bytes / (16 * kChunk16);
    if (mode == 3 && (bytes % (16 * kChunk16) != 0 || nchunks == 0 || nchunks >= (size_t{1} << 31)))
        return -1;
    const u32x4* p = static_cast<const u32x4*>(buf);
    u32x4* k = static_cast<u32x4*>(sink);
    if (mode == 0)
        hipLaunchKernelGGL(read_kernel, dim3(workgroups), dim3(kThreads), 0, stream, p, bytes / 16, k);
    else if (mode == 1)
        hipLaunchKernelGGL(read_nt_kernel<false>, dim3(workgroups), dim3(kThreads), 0, stream, p, bytes / 16, k);
    else if (mode == 2)
        hipLaunchKernelGGL(read_nt_kernel<true>, dim3(workgroups), dim3(kThreads), 0, stream, p, bytes / 16, k);
    else
        hipLaunchKernelGGL(read_chunks_kernel, dim3(workgroups), dim3(kThreads), 0, stream, p, bytes / 16, k);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Mode 0 of the above.
extern "C" __attribute__((visibility("default"))) int bsa_probe_read(const void* buf, size_t bytes,
                                                                     void* sink, int workgroups,
                                                                     hipStream_t stream) {
    return bsa_probe_read_mode(buf, bytes, sink, workgroups, 0, stream);
}
