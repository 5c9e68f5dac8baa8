// Two-stage top-k over float32 logits, with the soft-cap applied to the
// selected values ["Gemma 4 M4 Max kernel roadmap", K1: logit soft-capping;
// K2 step 6: on-GPU top-k reduction; "Metal kernel capability table",
// section 6: f32_topk_partial, a partial pass then a fan-in].
//
// Order: larger value first, equal values -> lower index first, NaN after
// every number.  Each (value, index) pair is packed into one 64-bit key whose
// unsigned order is exactly that order:
//   high 32 bits: the float's bits mapped to an increasing unsigned code
//                 (NaN -> 0, -0 -> +0), low 32 bits: 0xFFFFFFFF - index.
// Keys are unique, so round r of a selection is simply "the largest key below
// the key chosen in round r-1": no per-element bookkeeping is needed.
//
// Stage 1: one workgroup per 4096-entry chunk keeps its keys in registers and
//          emits its k best (fewer than k valid entries leave zero keys).
// Stage 2: one workgroup per activation row selects the k best candidates
//          and writes indices and soft-capped values.
#include <stdint.h>

#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kChunk = 4096;
constexpr int kPerThread = kChunk / kBlockThreads;  // 16

__device__ __forceinline__ uint64_t order_key(float v, uint32_t idx) {
    uint32_t code;
    if (v != v) {
        code = 0u;
    } else {
        if (v == 0.0f) v = 0.0f;  // -0 ranks with +0
        const uint32_t b = __float_as_uint(v);
        code = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    return (static_cast<uint64_t>(code) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
        v = umax64(v, (static_cast<uint64_t>(hi) << 32) | lo);
    }
    return v;
}

// Block-wide maximum; every thread gets the result.
__device__ __forceinline__ uint64_t block_max64(uint64_t v, uint64_t* red) {
    v = wave_max64(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
    __syncthreads();
    uint64_t r = red[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) r = umax64(r, red[i]);
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kBlockThreads)
void topk_chunk_kernel(const float* __restrict__ y, int64_t N, int k, int nchunks,
                       uint64_t* __restrict__ cand) {
    __shared__ uint64_t red[kWavesPerBlock];
    const int m = blockIdx.y;
    const int c = blockIdx.x;
    const float* ym = y + static_cast<int64_t>(m) * N;
    uint64_t key[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int64_t idx = static_cast<int64_t>(c) * kChunk + i * kBlockThreads + threadIdx.x;
        key[i] = idx < N ? order_key(ym[idx], static_cast<uint32_t>(idx)) : 0ull;
    }
    uint64_t* out = cand + (static_cast<int64_t>(m) * nchunks + c) * k;
    uint64_t bound = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
            if (key[i] < bound) best = umax64(best, key[i]);
        best = block_max64(best, red);
        if (threadIdx.x == 0) out[r] = best;
        bound = best;
    }
}

__global__ __launch_bounds__(kBlockThreads)
void topk_merge_kernel(const float* __restrict__ y, int64_t N, int k, int nchunks, float softcap,
                       const uint64_t* __restrict__ cand, float* __restrict__ top_val,
                       int32_t* __restrict__ top_idx) {
    __shared__ uint64_t red[kWavesPerBlock];
    const int m = blockIdx.x;
    const int64_t ncand = static_cast<int64_t>(nchunks) * k;
    const uint64_t* cm = cand + static_cast<int64_t>(m) * ncand;
    uint64_t bound = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0ull;
        for (int64_t i = threadIdx.x; i < ncand; i += kBlockThreads) {
            const uint64_t v = cm[i];
            if (v < bound) best = umax64(best, v);
        }
        best = block_max64(best, red);
        if (threadIdx.x == 0) {
            // k <= N guarantees a real key every round; a zero key would mean
            // "nothing left" and is never dereferenced.
            const uint32_t idx = 0xFFFFFFFFu - static_cast<uint32_t>(best);
            const bool real = best != 0ull && idx < static_cast<uint64_t>(N);
            const float v = real ? y[static_cast<int64_t>(m) * N + idx] : __builtin_nanf("");
            top_idx[static_cast<int64_t>(m) * k + r] = real ? static_cast<int32_t>(idx) : -1;
            top_val[static_cast<int64_t>(m) * k + r] = softcap * tanhf(v / softcap);
        }
        bound = best;
    }
}

int chunks_of(int64_t N) { return static_cast<int>((N + kChunk - 1) / kChunk); }

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t topk_ws_bytes(int64_t N, int64_t M, int k) {
    const size_t ybytes = align256(static_cast<size_t>(N) * static_cast<size_t>(M) * sizeof(float));
    const size_t cbytes = static_cast<size_t>(M) * chunks_of(N) * static_cast<size_t>(k) * sizeof(uint64_t);
    return ybytes + align256(cbytes);
}

hipError_t launch_topk(const float* y, float* top_val, int32_t* top_idx, int64_t N, int64_t M, int k,
                       float softcap, void* ws, hipStream_t stream) {
    const int nchunks = chunks_of(N);
    uint64_t* cand = reinterpret_cast<uint64_t*>(
        static_cast<char*>(ws) + align256(static_cast<size_t>(N) * static_cast<size_t>(M) * sizeof(float)));
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(nchunks, static_cast<unsigned>(M)), dim3(kBlockThreads), 0,
                       stream, y, N, k, nchunks, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<unsigned>(M)), dim3(kBlockThreads), 0, stream,
                       y, N, k, nchunks, softcap, cand, top_val, top_idx);
    return hipGetLastError();
}

}  // namespace qmv
