// Q4_0 weights x Q8-quantized activations ["Metal kernel capability table",
// section 1: q4_matvec_v4 (Q4_0 x Q8 int8 + scales); section 2: quantize_q8;
// "Gemma 4 M4 Max kernel roadmap", K3: batched Q4_0 matrix-matrix kernels].
//
// Step 1 (quantize_q8_kernel): every 32-element block of x gets
//   d = max|x| / 127 (IEEE float32 division), q = clamp(round(x / d), +-127)
// (round half away from zero; an all-zero block gives d = 0, q = 0).
// Step 2 (qmm_dot_kernel): exact int32 block sums
//   isum = sum_j (q_w - 8) * q_x
// with v_dot4_i32_i8, then y += isum * d_w * d_x in float32.  The weight
// codes enter the dot products as 16 (q_w - 8) in a signed byte, so the dot
// gives 16 isum exactly (|16 isum| <= 32*128*127) and the shift back is exact.
#include <utility>

#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kQxStride = kUnitElems + 16;  // bytes of one unit's codes in LDS (+16 B pad)

__global__ __launch_bounds__(kBlockThreads)
void quantize_q8_kernel(const float* __restrict__ x, int8_t* __restrict__ q, float* __restrict__ d,
                        int64_t total) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlockThreads;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x; e - threadIdx.x < total;
         e += stride) {
        const bool ok = e < total;  // total % 32 == 0: whole 32-lane groups agree
        const float v = ok ? x[e] : 0.0f;
        float a = fabsf(v);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
        const float db = a / 127.0f;
        int qv = 0;
        if (a != 0.0f) {
            float t = roundf(v / db);
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            qv = static_cast<int>(t);
        }
        if (ok) {
            q[e] = static_cast<int8_t>(qv);
            if ((threadIdx.x & 31) == 0) d[e >> 5] = db;
        }
    }
}

// Lane (segment s, index u) of a wave handles units u, u + L, ..., u + (C-1) L
// of one row per pass; a wave holds S segments (one row each).  G = C * L.
template <bool WRITE_ISUM>
__global__ __launch_bounds__(kBlockThreads)
void qmm_dot_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ qx,
                    const float* __restrict__ dx, float* __restrict__ y, int32_t* __restrict__ isum,
                    int N, int G, int C, int L, int S, int npasses, int m0) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int m = m0 + blockIdx.y;
    const int64_t K = static_cast<int64_t>(G) * kUnitElems;
    const int nb = G * 8;
    unsigned char* qs = lds;                                                   // G * kQxStride bytes
    float* ds = reinterpret_cast<float*>(lds + static_cast<size_t>(G) * kQxStride);  // nb floats

    // stage this row's activation codes and scales
    const int8_t* qxm = qx + m * K;
    for (int i = threadIdx.x; i < G * 16; i += kBlockThreads) {
        const uint4 v = reinterpret_cast<const uint4*>(qxm)[i];
        *reinterpret_cast<uint4*>(qs + (i >> 4) * kQxStride + (i & 15) * 16) = v;
    }
    // the block-sum export passes no scales (dx == nullptr) and never reads ds
    if constexpr (!WRITE_ISUM) {
        for (int i = threadIdx.x; i < nb; i += kBlockThreads) ds[i] = dx[static_cast<int64_t>(m) * nb + i];
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int seg = lane / L;
    const int u0 = lane - seg * L;
    const bool active = seg < S;
    const int64_t row_bytes = static_cast<int64_t>(G) * 144;
    const int wave_stride = gridDim.x * kWavesPerBlock;

    for (int pass = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; pass < npasses; pass += wave_stride) {
        const int row = pass * S + seg;
        const bool ok = active && row < N;
        float acc = 0.0f;
        for (int c = 0; c < C; ++c) {
            const int u = u0 + c * L;
            uint32_t U[36];
            if (ok) {
                const uint4* src = reinterpret_cast<const uint4*>(W + row * row_bytes + u * 144);
#pragma unroll
                for (int t = 0; t < 9; ++t) {
                    const uint4 v = src[t];
                    U[4 * t] = v.x; U[4 * t + 1] = v.y; U[4 * t + 2] = v.z; U[4 * t + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int t = 0; t < 36; ++t) U[t] = 0x88888888u;
            }
            int ux = u * kQxStride;
            asm volatile("" : "+v"(ux));
            const uint4* xq = reinterpret_cast<const uint4*>(qs + ux);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int b0 = 18 * k;
                const uint32_t dbits = ((b0 & 3) == 2) ? (U[b0 >> 2] >> 16) : (U[b0 >> 2] & 0xffffu);
                const int qb = b0 + 2;
                const uint4 xa = xq[2 * k];      // elements 0..15 of block k
                const uint4 xb = xq[2 * k + 1];  // elements 16..31
                const uint32_t xlo[4] = {xa.x, xa.y, xa.z, xa.w};
                const uint32_t xhi[4] = {xb.x, xb.y, xb.z, xb.w};
                int s16 = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t raw = ((qb & 3) == 0) ? U[(qb >> 2) + t]
                                                         : shift16(U[(qb >> 2) + t + 1], U[(qb >> 2) + t]);
                    const uint32_t v = raw ^ 0x88888888u;
                    const uint32_t hi = v & 0xF0F0F0F0u;
                    const uint32_t lo = (v << 4) & 0xF0F0F0F0u;
                    s16 = __builtin_amdgcn_sdot4(static_cast<int>(lo), static_cast<int>(xlo[t]), s16, false);
                    s16 = __builtin_amdgcn_sdot4(static_cast<int>(hi), static_cast<int>(xhi[t]), s16, false);
                }
                const int blk = u * 8 + k;
                if constexpr (WRITE_ISUM) {
                    if (ok) isum[(static_cast<int64_t>(m) * N + row) * nb + blk] = s16 >> 4;
                } else {
                    const float scale = half_bits_to_float(dbits) * 0.0625f * ds[blk];
                    acc = fmaf(static_cast<float>(s16), scale, acc);
                }
            }
        }
        if constexpr (!WRITE_ISUM) {
            acc = segment_sum(acc, u0, L);
            if (ok && u0 == 0) y[static_cast<int64_t>(m) * N + row] = acc;
        }
    }
}

// Any K % 32 == 0: one wave per (row, activation row) pair, lanes over the
// blocks of the row; Q4_0 blocks read with 16-bit loads, codes from global.
template <bool WRITE_ISUM>
__global__ __launch_bounds__(kBlockThreads)
void qmm_generic_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ qx,
                        const float* __restrict__ dx, float* __restrict__ y, int32_t* __restrict__ isum,
                        int64_t N, int64_t K, int64_t M) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nb = K / 32;
    const int64_t row_bytes = nb * 18;
    const int64_t wave_stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    for (int64_t p = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; p < N * M;
         p += wave_stride) {
        const int64_t row = p % N;
        const int64_t m = p / N;
        float acc = 0.0f;
        for (int64_t b = lane; b < nb; b += kWave) {
            const uint16_t* blk = reinterpret_cast<const uint16_t*>(W + row * row_bytes + 18 * b);
            const uint32_t* xq = reinterpret_cast<const uint32_t*>(qx + m * K + 32 * b);
            int s16 = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t raw = static_cast<uint32_t>(blk[1 + 2 * t]) |
                                     (static_cast<uint32_t>(blk[2 + 2 * t]) << 16);
                const uint32_t v = raw ^ 0x88888888u;
                const uint32_t hi = v & 0xF0F0F0F0u;
                const uint32_t lo = (v << 4) & 0xF0F0F0F0u;
                s16 = __builtin_amdgcn_sdot4(static_cast<int>(lo), static_cast<int>(xq[t]), s16, false);
                s16 = __builtin_amdgcn_sdot4(static_cast<int>(hi), static_cast<int>(xq[4 + t]), s16, false);
            }
            if constexpr (WRITE_ISUM) {
                isum[(m * N + row) * nb + b] = s16 >> 4;
            } else {
                acc = fmaf(static_cast<float>(s16), half_bits_to_float(blk[0]) * 0.0625f * dx[m * nb + b], acc);
            }
        }
        if constexpr (!WRITE_ISUM) {
            acc = wave_sum(acc);
            if (lane == 0) y[m * N + row] = acc;
        }
    }
}

// Units per lane C and lanes per segment L = G / C: the split of a row that
// keeps the most lanes of a wave busy (ties: fewer units per lane).
void plan_segments(int G, int* C, int* L, int* S) {
    int bestC = G, bestL = 1, best_active = 0;
    for (int c = 1; c <= G; ++c) {
        if (G % c) continue;
        const int l = G / c;
        if (l > kWave) continue;
        const int active = (kWave / l) * l;
        if (active > best_active) { best_active = active; bestC = c; bestL = l; }
    }
    *C = bestC;
    *L = bestL;
    *S = kWave / bestL;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t qmm_ws_bytes(int64_t K, int64_t M) {
    return align256(static_cast<size_t>(M) * static_cast<size_t>(K)) +
           align256(static_cast<size_t>(M) * static_cast<size_t>(K / 32) * sizeof(float));
}

hipError_t launch_quantize_q8(const float* x, int8_t* q, float* d, int64_t K, int64_t M, hipStream_t stream) {
    const int64_t total = K * M;
    int64_t blocks = (total + kBlockThreads - 1) / kBlockThreads;
    const int64_t cap = static_cast<int64_t>(device_cus()) * 64;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(quantize_q8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0, stream,
                       x, q, d, total);
    return hipGetLastError();
}

// Largest K whose activation codes and scales fit one workgroup's LDS.
constexpr int64_t kDotMaxG = 200;

hipError_t launch_qmm(const void* W, const int8_t* qx, const float* dx, float* y, int32_t* isum,
                      int64_t N64, int64_t K, int64_t M, hipStream_t stream) {
    if (K % kUnitElems != 0 || K / kUnitElems > kDotMaxG) {
        int64_t blocks = (N64 * M + kWavesPerBlock - 1) / kWavesPerBlock;
        const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
        if (blocks > cap) blocks = cap;
        if (isum) {
            hipLaunchKernelGGL((qmm_generic_kernel<true>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads),
                               0, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N64, K, M);
        } else {
            hipLaunchKernelGGL((qmm_generic_kernel<false>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads),
                               0, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N64, K, M);
        }
        return hipGetLastError();
    }
    const int N = static_cast<int>(N64);
    const int G = static_cast<int>(K / kUnitElems);
    int C, L, S;
    plan_segments(G, &C, &L, &S);
    const int npasses = (N + S - 1) / S;
    const int max_blocks = device_cus() * 4;
    int blocks = (npasses + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    const size_t lds = static_cast<size_t>(G) * kQxStride + static_cast<size_t>(G) * 8 * sizeof(float);
    for (int64_t m0 = 0; m0 < M; m0 += 65535) {
        const int64_t mc = (M - m0 < 65535) ? (M - m0) : 65535;
        if (isum) {
            hipLaunchKernelGGL((qmm_dot_kernel<true>), dim3(blocks, static_cast<unsigned>(mc)), dim3(kBlockThreads),
                               lds, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N, G, C, L, S,
                               npasses, static_cast<int>(m0));
        } else {
            hipLaunchKernelGGL((qmm_dot_kernel<false>), dim3(blocks, static_cast<unsigned>(mc)), dim3(kBlockThreads),
                               lds, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N, G, C, L, S,
                               npasses, static_cast<int>(m0));
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmv
