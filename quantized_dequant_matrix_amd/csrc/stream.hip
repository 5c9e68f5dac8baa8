// A plain streaming read of device memory: the measured ceiling that the
// GEMV kernels' effective bandwidth is compared with.  Every 16-byte word of
// the buffer is loaded once with coalesced 16-byte loads (each wave reads
// 1 KB contiguous per load instruction, four loads in flight per lane), and
// each workgroup stores the XOR of the 32-bit words it read, so that no load
// can be dropped.  Weights of a decode step are read the same way, once, from HBM.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

__global__ __launch_bounds__(kBlockThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                    uint32_t* __restrict__ out) {
    __shared__ uint32_t part[kWavesPerBlock];
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlockThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kWavesPerBlock; ++w) t ^= part[w];
        out[blockIdx.x] = t;  // one plain store per workgroup: no shared word, no atomics
    }
}

}  // namespace

hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* out, int workgroups, hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kBlockThreads), 0, stream,
                       static_cast<const uint4*>(p), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace qmv
