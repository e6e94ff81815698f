// Streaming-read bandwidth probe: reads a buffer once with 16-byte
// non-temporal loads, the access the expert kernels use, and folds the
// words into one value per workgroup so that no load is dead.  It measures
// the HBM read rate this device actually reaches, which the benchmark
// reports beside the vendor peak.
#include "device.h"

namespace mq {

constexpr int kStreamUnroll = 8;

// grid: any number of workgroups of 256 threads; every byte below
// n16 * 16 is read once.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* buf, int64_t n16, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
        uint4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld_stream16(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = ld_stream16(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[4];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace mq
