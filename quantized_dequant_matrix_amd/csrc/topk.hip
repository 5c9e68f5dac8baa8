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
// A real key is never 0 (index < 2^31), so 0 means "nothing".  Keys are
// unique, so round r of a selection is "the largest key below the key chosen
// in round r-1": no per-element bookkeeping is needed.
//
// Stage 1: every wave owns a 1024-entry chunk (16 keys per lane, in
//          registers) and emits its k best; each round is a lane-local scan
//          plus a DPP wave reduction, with no workgroup barrier.
// Stage 2: one 1024-thread workgroup per activation row: each wave selects
//          the k best of its share of the candidates, then one wave selects
//          the k best of those and writes indices and soft-capped values.
#include <stdint.h>

#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kChunk = 1024;                  // entries per wave in stage 1
constexpr int kPerLane = kChunk / kWave;      // 16
constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMergeRegs = 8;                 // candidates a lane keeps in registers in stage 2

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

// Lanes the DPP pattern does not write keep 0, the identity of the max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, ROW_MASK, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, ROW_MASK, 0xF, false));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Maximum over the 64 lanes, returned to every lane.  Inclusive prefix
// maxima within each row of 16 lanes (row_shr 1, 2, 4, 8), then row 0's
// maximum into row 1 and row 2's into row 3 (row_bcast 15), then row 1's into
// rows 2-3 (row_bcast 31): lane 63 ends with the maximum of all lanes.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
    v = umax64(v, dpp64<0x111, 0xF>(v));
    v = umax64(v, dpp64<0x112, 0xF>(v));
    v = umax64(v, dpp64<0x114, 0xF>(v));
    v = umax64(v, dpp64<0x118, 0xF>(v));
    v = umax64(v, dpp64<0x142, 0xA>(v));
    v = umax64(v, dpp64<0x143, 0xC>(v));
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// k rounds over NK keys per lane held in registers; lane r writes the
// round-r winner to out[r] (r < k).
template <int NK>
__device__ __forceinline__ void wave_select(const uint64_t (&key)[NK], int k, uint64_t* out) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t bound = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < NK; ++i)
            if (key[i] < bound) best = umax64(best, key[i]);
        best = wave_max64(best);
        if (lane == (r & (kWave - 1))) out[r] = best;
        bound = best;
    }
}

__global__ __launch_bounds__(kBlockThreads)
void topk_chunk_kernel(const float* __restrict__ y, int64_t N, int k, int nwchunks,
                       uint64_t* __restrict__ cand) {
    const int m = blockIdx.y;
    const int c = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;  // this wave's chunk
    if (c >= nwchunks) return;                                        // whole wave leaves together
    const int lane = threadIdx.x & (kWave - 1);
    const float* ym = y + static_cast<int64_t>(m) * N;
    uint64_t key[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int64_t idx = static_cast<int64_t>(c) * kChunk + i * kWave + lane;
        key[i] = idx < N ? order_key(ym[idx], static_cast<uint32_t>(idx)) : 0ull;
    }
    wave_select(key, k, cand + (static_cast<int64_t>(m) * nwchunks + c) * k);
}

__global__ __launch_bounds__(kMergeThreads)
void topk_merge_kernel(const float* __restrict__ y, int64_t N, int k, int nwchunks, float softcap,
                       const uint64_t* __restrict__ cand, float* __restrict__ top_val,
                       int32_t* __restrict__ top_idx) {
    __shared__ uint64_t stage[kMergeWaves * 64];
    const int m = blockIdx.x;
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t ncand = static_cast<int64_t>(nwchunks) * k;
    const uint64_t* cm = cand + static_cast<int64_t>(m) * ncand;
    // wave w owns candidates [lo, hi)
    const int64_t per = (ncand + kMergeWaves - 1) / kMergeWaves;
    const int64_t lo = w * per;
    const int64_t hi = (lo + per < ncand) ? lo + per : ncand;
    if (per <= static_cast<int64_t>(kWave) * kMergeRegs) {
        uint64_t key[kMergeRegs];
#pragma unroll
        for (int i = 0; i < kMergeRegs; ++i) {
            const int64_t j = lo + i * kWave + lane;
            key[i] = j < hi ? cm[j] : 0ull;
        }
        wave_select(key, k, stage + w * 64);
    } else {
        // very large N: scan this wave's share from memory every round
        uint64_t bound = ~0ull;
        for (int r = 0; r < k; ++r) {
            uint64_t best = 0ull;
            for (int64_t j = lo + lane; j < hi; j += kWave) {
                const uint64_t v = cm[j];
                if (v < bound) best = umax64(best, v);
            }
            best = wave_max64(best);
            if (lane == r) stage[w * 64 + r] = best;
            bound = best;
        }
    }
    __syncthreads();
    if (w == 0) {
        // k <= 64 winners per wave, 16 waves: 16 keys per lane
        uint64_t key[kMergeWaves];
#pragma unroll
        for (int i = 0; i < kMergeWaves; ++i) key[i] = lane < k ? stage[i * 64 + lane] : 0ull;
        uint64_t bound = ~0ull;
        for (int r = 0; r < k; ++r) {
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < kMergeWaves; ++i)
                if (key[i] < bound) best = umax64(best, key[i]);
            best = wave_max64(best);
            if (lane == 0) {
                // k <= N guarantees a real key every round; a zero key would
                // mean "nothing left" and is never dereferenced.
                const uint32_t idx = 0xFFFFFFFFu - static_cast<uint32_t>(best);
                const bool real = best != 0ull && idx < static_cast<uint64_t>(N);
                const float v = real ? y[static_cast<int64_t>(m) * N + idx] : __builtin_nanf("");
                top_idx[static_cast<int64_t>(m) * k + r] = real ? static_cast<int32_t>(idx) : -1;
                top_val[static_cast<int64_t>(m) * k + r] = softcap * tanhf(v / softcap);
            }
            bound = best;
        }
    }
}

int64_t wave_chunks_of(int64_t N) { return (N + kChunk - 1) / kChunk; }

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t topk_ws_bytes(int64_t N, int64_t M, int k) {
    const size_t ybytes = align256(static_cast<size_t>(N) * static_cast<size_t>(M) * sizeof(float));
    const size_t cbytes =
        static_cast<size_t>(M) * static_cast<size_t>(wave_chunks_of(N)) * static_cast<size_t>(k) * sizeof(uint64_t);
    return ybytes + align256(cbytes);
}

hipError_t launch_topk(const float* y, float* top_val, int32_t* top_idx, int64_t N, int64_t M, int k,
                       float softcap, void* ws, hipStream_t stream) {
    const int nwchunks = static_cast<int>(wave_chunks_of(N));
    uint64_t* cand = reinterpret_cast<uint64_t*>(
        static_cast<char*>(ws) + align256(static_cast<size_t>(N) * static_cast<size_t>(M) * sizeof(float)));
    const unsigned blocks = static_cast<unsigned>((nwchunks + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(blocks, static_cast<unsigned>(M)), dim3(kBlockThreads), 0, stream,
                       y, N, k, nwchunks, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<unsigned>(M)), dim3(kMergeThreads), 0, stream,
                       y, N, k, nwchunks, softcap, cand, top_val, top_idx);
    return hipGetLastError();
}

}  // namespace qmv
