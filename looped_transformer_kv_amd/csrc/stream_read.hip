// stream_read.hip -- a plain streaming read of a device buffer: the achievable HBM read bandwidth
// on the same run, against which the decode kernels' latent bandwidth is also reported.
//
// Every 16-byte word is read exactly once with coalesced 16-byte loads (U per thread in flight,
// grid-stride over whole tiles, then a guarded tail); each workgroup stores the XOR of the 32-bit
// words it read in its own sink slot (no atomics: one contended address would serialise the
// workgroups' end), which keeps the loads live and lets a test check that every byte was read.
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                               size_t n, uint32_t *sink) {
    __shared__ uint32_t red[kThreads / 64];
    constexpr size_t tile = (size_t)kThreads * kUnroll;
    const size_t full = n / tile;
    uint32_t acc = 0;
    for (size_t t = blockIdx.x; t < full; t += gridDim.x) {
        const uint4 *base = p + t * tile + threadIdx.x;
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = base[(size_t)u * kThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (size_t j = full * tile + (size_t)blockIdx.x * kThreads + threadIdx.x; j < n;
         j += (size_t)gridDim.x * kThreads) {
        const uint4 v = p[j];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // wave-level XOR, then the workgroup's waves through LDS, one plain store per workgroup
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < kThreads / 64; ++w) x ^= red[w];
        sink[blockIdx.x] = x;
    }
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    const size_t n = bytes / 16;
    const size_t tiles = (n + (size_t)kThreads * kUnroll - 1) / ((size_t)kThreads * kUnroll);
    // two workgroups per CU; never more than the sink's kStreamReadSlots entries
    const unsigned blocks =
        (unsigned)(tiles < kStreamReadSlots ? (tiles ? tiles : 1) : kStreamReadSlots);
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, st,
                       static_cast<const uint4 *>(buf), n, sink);
    return hipGetLastError();
}

}  // namespace lla
