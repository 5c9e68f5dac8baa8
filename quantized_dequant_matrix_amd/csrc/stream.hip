// A plain streaming read of device memory: the measured ceiling that the
// GEMV kernels' effective bandwidth is compared with.  Every 16-byte word of
// the buffer is loaded once: each wave reads a contiguous 4 KB chunk per
// round (four 16-byte loads per lane, each instruction 1 KB contiguous),
// chunks dealt to the waves round-robin, the words past the last whole chunk
// by single loads.  Each workgroup stores the XOR of the 32-bit words it
// read, so that no load can be dropped.  Of the read patterns measured on
// MI355X (grid-stride with 4, 8 or 16 loads in flight per lane, wave chunks
// of 4, 8 or 16 KB, a contiguous slab per workgroup, loads straight into
// LDS), 4 KB wave chunks were the fastest or within 1% of it at 50 MB,
// 117 MB and 1.5 GB.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kLoadsPerLane = 4;
constexpr int64_t kChunkWords = static_cast<int64_t>(kWave) * kLoadsPerLane;  // 16-byte words per wave round

__global__ __launch_bounds__(kBlockThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                    uint32_t* __restrict__ out) {
    __shared__ uint32_t part[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    const int64_t nfull = n16 / kChunkWords;
    uint32_t acc = 0;
    for (int64_t c = wave; c < nfull; c += nwaves) {
        const uint4* q = p + c * kChunkWords + lane;
        uint4 v[kLoadsPerLane];
#pragma unroll
        for (int u = 0; u < kLoadsPerLane; ++u) v[u] = q[u * kWave];
#pragma unroll
        for (int u = 0; u < kLoadsPerLane; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the words past the last whole chunk (fewer than one chunk)
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x;
    if (nfull * kChunkWords + t < n16) {
        const uint4 a = p[nfull * kChunkWords + t];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
    if (lane == 0) part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < kWavesPerBlock; ++w) x ^= part[w];
        out[blockIdx.x] = x;  // one plain store per workgroup: no shared word, no atomics
    }
}

}  // namespace

hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* out, int workgroups, hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kBlockThreads), 0, stream,
                       static_cast<const uint4*>(p), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace qmv
