// Q4_0 weights x Q8-quantized activations ["Metal kernel capability table",
// section 1: q4_matvec_v4 (Q4_0 x Q8 int8 + scales); section 2: quantize_q8;
// "Gemma 4 M4 Max kernel roadmap", K3: batched Q4_0 matrix-matrix kernels].
//
// Step 1 (quantize_q8_kernel): every 32-element block of x gets
//   d = max|x| / 127 (IEEE float32 division), q = clamp(round(x / d), +-127)
// (round half away from zero; an all-zero block gives d = 0, q = 0).
// Step 2: exact int32 block sums
//   isum = sum_j (q_w - 8) * q_x
// then y += isum * d_w * d_x in float32.  The weight codes enter the integer
// products as 16 (q_w - 8) in a signed byte, so the sums are 16 isum exactly
// (|16 isum| <= 32*128*127) and the shift back is exact.
//   M == 1: qmm_dot_kernel, v_dot4_i32_i8 per lane (an HBM-bound GEMV).
//   M >= 2: the work is a dense int8 contraction: one v_mfma_i32_16x16x32_i8
//           covers exactly one block (K = 32) of a 16 x 16 tile of (m, n), so
//           every block sum stays exact and gets its own scale in the float
//           epilogue.  qmm_wide_kernel takes the large tilings (M = 512 class),
//           qmm_mfma_kernel the narrow ones (M = 16 class) and the block-sum
//           export.
#include <utility>

#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kQxStride = kUnitElems + 16;  // bytes of one unit's codes in LDS (+16 B pad)

// Layout of the quantized activations for the MFMA kernel ("fragment
// layout"), with Mt = ceil(M / 16) tiles of 16 rows and nb = K / 32 blocks:
//   codes  [Mt][nb / 2][64 lanes][16 B]: lane l = i + 16 g holds, for row
//          16 t + i, bytes 0..7 = block 2c and bytes 8..15 = block 2c + 1,
//          each as x[4g .. 4g+3] followed by x[16+4g .. 16+4g+3] -- the same
//          elements as code bytes 4g .. 4g+3 of a Q4_0 block (low nibbles,
//          then high nibbles), so one code dword of the weights pairs with
//          one 8-byte operand of the activations;
//   scales [Mt][nb][16] float: d_x of row 16 t + i for block b.
// Rows M .. 16 Mt - 1 are quantized as zeros.
struct FragLayout {
    int64_t nb;
    __device__ __forceinline__ int64_t code_dword(int64_t m, int64_t b, int t) const {
        const int64_t mt = m >> 4, i = m & 15;
        const int g = t & 3, half = t >> 2;  // t: which 4 elements of the block (4t .. 4t+3)
        return (((mt * (nb >> 1) + (b >> 1)) * kWave + i + 16 * g) * 16 + (b & 1) * 8 + half * 4) >> 2;
    }
    __device__ __forceinline__ int64_t scale_index(int64_t m, int64_t b) const {
        return ((m >> 4) * nb + b) * 16 + (m & 15);
    }
};

// The scale d_x of a block as three bfloat16 terms, d_x = h + m + l exactly
// (each a truncation of what is left: 8 + 8 + 8 significant bits cover the
// 24 of a float32; only parts below the bfloat16 range, under 2^-133, are
// lost).  The wide MFMA kernel forms the products d_w * d_x with a
// bfloat16 MFMA from these terms.  Returned as the 16-byte operand pair
// (h, m, l, h | m, l, 0, 0): k-half 0 and k-half 1 of that MFMA's A operand.
__device__ __forceinline__ uint4 bf16_split3(float v) {
    const uint32_t h = __float_as_uint(v) & 0xffff0000u;
    const float r1 = v - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r1) & 0xffff0000u;
    const uint32_t l = __float_as_uint(r1 - __uint_as_float(m)) & 0xffff0000u;
    return make_uint4((h >> 16) | m, (l >> 16) | h, (m >> 16) | l, 0u);
}

// Layouts of the quantized activations in the workspace.
//   kLayoutRows:  codes [M][K], scales float [M][K/32] (M == 1, the export).
//   kLayoutFrag:  the fragment layout above (narrow MFMA tiling).
//   kLayoutSplit: (wide MFMA tiling) tiles of 32 rows, Mt = Mrows / 32:
//                 codes [Mt][K/32][64 lanes][16 B], lane l = i + 32 h holding
//                 elements 16 h .. 16 h + 15 of row 32 t + i; scales as
//                 bf16_split3 operands, uint4 [Mt][K/32][32] (row 32 t + i).
//                 One wave's operand of a block is 1 KB contiguous.
// Rows M .. Mrows - 1 are quantized as zeros.
enum QLayout : int { kLayoutRows = 0, kLayoutFrag = 1, kLayoutSplit = 2 };

// One 8-lane group per 32-element block, 4 elements per lane.
template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads)
void quantize_q8_kernel(const float* __restrict__ x, int8_t* __restrict__ q, float* __restrict__ d,
                        int64_t K, int64_t M, int64_t Mrows, bool vec_x, bool vec_q) {
    static_assert(LAYOUT == kLayoutRows || LAYOUT == kLayoutFrag, "kLayoutSplit: quantize_q8_tiles_kernel");
    const int64_t nb = K / 32;
    const int64_t total = Mrows * nb;  // blocks, padding rows included
    const int t = threadIdx.x & 7;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (kBlockThreads / 8);
    // the loop bound is taken per wave so that shuffles see whole groups
    for (int64_t wave_first = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + (threadIdx.x & ~(kWave - 1))) / 8;
         wave_first < total; wave_first += stride) {
        const int64_t blk = wave_first + (threadIdx.x & (kWave - 1)) / 8;
        const bool ok = blk < total;
        const int64_t m = ok ? blk / nb : 0;
        const int64_t b = ok ? blk - m * nb : 0;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ok && m < M) {
            const float* src = x + m * K + 32 * b + 4 * t;
            if (vec_x) {
                const float4 f = *reinterpret_cast<const float4*>(src);
                v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = src[e];
            }
        }
        float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 8));
        const float db = a / 127.0f;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int qv = 0;
            if (a != 0.0f) {
                float r = roundf(v[e] / db);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                qv = static_cast<int>(r);
            }
            packed |= (static_cast<uint32_t>(qv) & 0xffu) << (8 * e);
        }
        if (ok) {
            if constexpr (LAYOUT == kLayoutFrag) {
                const FragLayout L{nb};
                reinterpret_cast<uint32_t*>(q)[L.code_dword(m, b, t)] = packed;
                if (t == 0) d[L.scale_index(m, b)] = db;
            } else {
                int8_t* dst = q + m * K + 32 * b + 4 * t;
                if (vec_q) {
                    *reinterpret_cast<uint32_t*>(dst) = packed;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = static_cast<int8_t>(packed >> (8 * e));
                }
                if (t == 0) d[m * nb + b] = db;
            }
        }
    }
}

// kLayoutSplit: one wave per (32-row tile, block); lane l = i + 32 h
// quantizes elements 16 h .. 16 h + 15 of row 32 t + i (the block's amax
// joins the two halves with one exchange) and writes its 16 code bytes where
// the wide kernel's lane l reads them: each wave writes 1 KB contiguous.
// The arithmetic is quantize_q8_kernel's, element for element.
__global__ __launch_bounds__(kBlockThreads)
void quantize_q8_tiles_kernel(const float* __restrict__ x, int8_t* __restrict__ q, uint4* __restrict__ ds,
                              int64_t K, int64_t M, int64_t Mrows, bool vec_x) {
    const int64_t nb = K / 32;
    const int64_t items = (Mrows / 32) * nb;
    const int lane = threadIdx.x & (kWave - 1);
    const int i = lane & 31, h = lane >> 5;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    for (int64_t it = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; it < items;
         it += stride) {
        const int64_t mt = it / nb, b = it - mt * nb;
        const int64_t m = mt * 32 + i;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = 0.0f;
        if (m < M) {
            const float* src = x + m * K + 32 * b + 16 * h;
            if (vec_x) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 f = reinterpret_cast<const float4*>(src)[c];
                    v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = src[e];
            }
        }
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(v[e]));
        a = fmaxf(a, __shfl_xor(a, 32, kWave));
        const float db = a / 127.0f;
        uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            int qv = 0;
            if (a != 0.0f) {
                float r = roundf(v[e] / db);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                qv = static_cast<int>(r);
            }
            packed[e / 4] |= (static_cast<uint32_t>(qv) & 0xffu) << (8 * (e % 4));
        }
        reinterpret_cast<uint4*>(q)[it * kWave + lane] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        if (h == 0) ds[it * 32 + i] = bf16_split3(db);
    }
}

// Lane (segment s, index u) of a wave handles units u, u + L, ..., u + (C-1) L
// of one row per pass; a wave holds S segments (one row each).  G = C * L.
template <bool WRITE_ISUM>
__global__ __launch_bounds__(kBlockThreads)
void qmm_dot_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ qx,
                    const float* __restrict__ dx, float* __restrict__ y, int32_t* __restrict__ isum,
                    int N, int G, int C, int L, int S, int npasses, int m0, int isn0, int isn1) {
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
    // the block-sum mode reads no scales
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
                    if (ok && row >= isn0 && row < isn1)
                        isum[(static_cast<int64_t>(m) * (isn1 - isn0) + (row - isn0)) * nb + blk] = s16 >> 4;
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
                        int64_t N, int64_t K, int64_t M, int64_t isn0, int64_t isn1) {
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
                if (row >= isn0 && row < isn1) isum[(m * (isn1 - isn0) + (row - isn0)) * nb + b] = s16 >> 4;
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

// Units per lane C and lanes per segment L = G / C: the smallest C (so the
// most waves) that keeps at least 54 of a wave's 64 lanes busy, else the
// split with the most busy lanes.
void plan_segments(int G, int* C, int* L, int* S) {
    int bestC = G, bestL = 1, best_active = 0;
    for (int c = 1; c <= G; ++c) {
        if (G % c) continue;
        const int l = G / c;
        if (l > kWave) continue;
        const int active = (kWave / l) * l;
        if (active >= 54) { bestC = c; bestL = l; break; }
        if (active > best_active) { best_active = active; bestC = c; bestL = l; }
    }
    *C = bestC;
    *L = bestL;
    *S = kWave / bestL;
}

// ------------------------------------------------------------ MFMA kernel
// Tiles of (m, n) per workgroup: TM = 16 MW WM activation rows by TN = 16 NW
// WN weight rows; four waves in a WM x WN x WK grid, each wave owning MW x NW
// 16 x 16 sub-tiles (WK > 1: the waves split the blocks of a tile and their
// partial sums are added in LDS, in wave order).  A workgroup covers blocks
// [ks kb, (ks + 1) kb) of K; with several K splits it writes partial sums
// that qmm_reduce_kernel adds in split order.
//
// Weights: the workgroup copies TN rows x KC blocks (raw GGUF bytes) into
// LDS per chunk, 16-byte coalesced, prefetching the next chunk into
// registers while it computes on this one.  Operand of lane (j = l % 16,
// g = l / 16) for weight row j: code dword g of the block, split into the
// low and the high nibbles as 16 (q - 8) signed bytes.  Activations come
// from the fragment layout written by quantize_q8_kernel<true>.
//
// v_mfma_i32_16x16x32_i8: A 16 x 32 (lane l: row l % 16, 8 bytes of k-group
// l / 16), B 32 x 16 (lane l: column l % 16, same k-group), D 16 x 16 int32
// (lane l: column l % 16, rows 4 (l / 16) .. +3).  The eight k values of a
// k-group are the same eight block elements in A and in B, so the product
// is the block's integer sum whatever order the hardware adds them in.
typedef int v4i __attribute__((ext_vector_type(4)));

enum QmmMode : int { kModeY = 0, kModePartial = 1, kModeISum = 2 };

__device__ __forceinline__ uint64_t q4_codes_to_s8(uint32_t c) {
    const uint32_t lo = ((c << 4) ^ 0x88888880u) & 0xF0F0F0F0u;  // elements 4g .. 4g+3
    const uint32_t hi = (c ^ 0x88888888u) & 0xF0F0F0F0u;         // elements 16+4g .. 16+4g+3
    return static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
}

template <int MW, int NW, int WM, int WN, int WK, int KC, int MODE>
__global__ __launch_bounds__(kBlockThreads)
void qmm_mfma_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ xa,
                     const float* __restrict__ xd, float* __restrict__ out, int32_t* __restrict__ isum,
                     int N, int64_t M, int nb, int64_t tm0, int64_t tiles_m, int tiles_n, int kb_per,
                     int64_t nwg, int isn0, int isn1) {
    constexpr int TN = 16 * NW * WN;
    constexpr int RB = KC * 18;       // bytes of one weight row per chunk
    constexpr int RS = RB + 16;       // LDS row stride: rows 4 banks apart (mod 64)
    constexpr int PR = RB / 16;       // 16-byte pieces per row
    constexpr int LPT = TN * PR / kBlockThreads;
    static_assert(KC % 8 == 0 && TN * PR == LPT * kBlockThreads, "the weight chunk must split evenly");
    static_assert(WM * WN * WK == kWavesPerBlock, "four waves per workgroup");
    __shared__ __align__(16) uint32_t wt[TN * RS / 4];

    // Consecutive workgroup ids are dealt round-robin to the 8 XCDs; give
    // each XCD a contiguous run of tiles (same weight rows, all m-tiles) so
    // that its L2 serves the weight reuse.
    int64_t lin = blockIdx.x;
    if (nwg % 8 == 0) lin = (lin % 8) * (nwg / 8) + lin / 8;
    const int64_t tm = tm0 + lin % tiles_m;
    lin /= tiles_m;
    const int tn = static_cast<int>(lin % tiles_n);
    const int ks = static_cast<int>(lin / tiles_n);
    const int kb0 = ks * kb_per;
    const int kb1 = min(nb, kb0 + kb_per);
    const int n0 = tn * TN;
    const int64_t row_bytes = static_cast<int64_t>(nb) * 18;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int wk = w % WK;
    const int wn = (w / WK) % WN;
    const int wm = w / (WK * WN);
    const int li = lane & 15;
    const int lg = lane >> 4;

    uint32_t pre[LPT * 4];
    auto fetch = [&](int c0) {
        const int valid = min(KC, kb1 - c0) * 18;  // a multiple of 144
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const int p = t * kBlockThreads + static_cast<int>(threadIdx.x);
            const int r = p / PR;
            const int q = p - r * PR;
            const int row = min(n0 + r, N - 1);             // rows past N: any valid row
            const int off = (q * 16 < valid) ? q * 16 : 0;  // blocks past the split: any valid piece
            const uint4 v = *reinterpret_cast<const uint4*>(W + row * row_bytes + static_cast<int64_t>(c0) * 18 + off);
            pre[4 * t + 0] = v.x;
            pre[4 * t + 1] = v.y;
            pre[4 * t + 2] = v.z;
            pre[4 * t + 3] = v.w;
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const int p = t * kBlockThreads + static_cast<int>(threadIdx.x);
            const int r = p / PR;
            const int q = p - r * PR;
            *reinterpret_cast<uint4*>(wt + r * (RS / 4) + q * 4) =
                make_uint4(pre[4 * t], pre[4 * t + 1], pre[4 * t + 2], pre[4 * t + 3]);
        }
    };

    float acc[MW][NW][4];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][ni][r] = 0.0f;

    fetch(kb0);
    for (int c0 = kb0; c0 < kb1; c0 += KC) {
        __syncthreads();  // every wave is done with the previous chunk
        stash();
        __syncthreads();
        if (c0 + KC < kb1) fetch(c0 + KC);
        const int npair = min(KC, kb1 - c0) >> 1;
        struct AFrag {
            uint64_t e[MW], o[MW];
            float xe[MW][4], xo[MW][4];
        };
        // activations of block pair cp of this chunk (blocks b, b + 1)
        auto load_a = [&](int cp, AFrag& A) {
            const int64_t b = c0 + 2 * cp;
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
                const int64_t mt = tm * (MW * WM) + wm * MW + mi;  // 16-row tile
                const uint4 v = *reinterpret_cast<const uint4*>(xa + ((mt * (nb >> 1) + (b >> 1)) * kWave + lane) * 16);
                A.e[mi] = static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32);
                A.o[mi] = static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32);
                if constexpr (MODE != kModeISum) {
                    const float4 de = *reinterpret_cast<const float4*>(xd + (mt * nb + b) * 16 + 4 * lg);
                    const float4 dq = *reinterpret_cast<const float4*>(xd + (mt * nb + b + 1) * 16 + 4 * lg);
                    A.xe[mi][0] = de.x; A.xe[mi][1] = de.y; A.xe[mi][2] = de.z; A.xe[mi][3] = de.w;
                    A.xo[mi][0] = dq.x; A.xo[mi][1] = dq.y; A.xo[mi][2] = dq.z; A.xo[mi][3] = dq.w;
                }
            }
        };
        auto mul_pair = [&](int cp, const AFrag& A) {
            const int64_t b = c0 + 2 * cp;
            uint64_t be[NW], bo[NW];
            float se[NW], so[NW];
#pragma unroll
            for (int ni = 0; ni < NW; ++ni) {
                const uint32_t* rowp = wt + ((wn * NW + ni) * 16 + li) * (RS / 4) + 9 * cp;
                // block b: codes at bytes 2 + 4g .. 5 + 4g of the pair (2 mod 4)
                const uint32_t ce = __builtin_amdgcn_alignbyte(rowp[lg + 1], rowp[lg], 2);
                // block b + 1: codes at bytes 20 + 4g .. (aligned)
                const uint32_t co = rowp[5 + lg];
                be[ni] = q4_codes_to_s8(ce);
                bo[ni] = q4_codes_to_s8(co);
                if constexpr (MODE != kModeISum) {
                    se[ni] = half_bits_to_float(rowp[0] & 0xffffu) * 0.0625f;  // d of block b / 16
                    so[ni] = half_bits_to_float(rowp[4] >> 16) * 0.0625f;      // d of block b + 1 / 16
                }
            }
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
#pragma unroll
                for (int ni = 0; ni < NW; ++ni) {
                    const v4i zero = {0, 0, 0, 0};
                    const v4i De = __builtin_amdgcn_mfma_i32_16x16x32_i8(static_cast<long>(A.e[mi]),
                                                                          static_cast<long>(be[ni]), zero, 0, 0, 0);
                    const v4i Do = __builtin_amdgcn_mfma_i32_16x16x32_i8(static_cast<long>(A.o[mi]),
                                                                          static_cast<long>(bo[ni]), zero, 0, 0, 0);
                    if constexpr (MODE == kModeISum) {
                        const int n = n0 + (wn * NW + ni) * 16 + li;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int64_t m = (tm * (MW * WM) + wm * MW + mi) * 16 + 4 * lg + r;
                            if (m < M && n >= isn0 && n < isn1) {
                                int32_t* dst = isum + (m * (isn1 - isn0) + (n - isn0)) * nb + b;
                                dst[0] = De[r] >> 4;
                                dst[1] = Do[r] >> 4;
                            }
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            acc[mi][ni][r] = fmaf(static_cast<float>(De[r]), se[ni] * A.xe[mi][r], acc[mi][ni][r]);
                            acc[mi][ni][r] = fmaf(static_cast<float>(Do[r]), so[ni] * A.xo[mi][r], acc[mi][ni][r]);
                        }
                    }
                }
            }
        };
        // This wave's pairs are wk, wk + WK, ...  The activations of the next
        // one are requested before the current one is multiplied; the loads
        // are unconditional (past the last pair they re-read the last pair)
        // so that no branch merges the waits.
        if (wk < npair) {
            AFrag A0, A1;
            int cp = wk;
            load_a(cp, A0);
            while (true) {
                load_a(min(cp + WK, npair - 1), A1);
                mul_pair(cp, A0);
                cp += WK;
                if (cp >= npair) break;
                load_a(min(cp + WK, npair - 1), A0);
                mul_pair(cp, A1);
                cp += WK;
                if (cp >= npair) break;
            }
        }
    }
    if constexpr (MODE != kModeISum) {
        if constexpr (WK > 1) {
            constexpr int NV = MW * NW * 4;
            static_assert((WK - 1) * WM * WN * NV * kWave <= TN * RS / 4, "reduction fits the weight tile");
            __syncthreads();  // the weight tile is free
            float* red = reinterpret_cast<float*>(wt);
            const int slot = wm * WN + wn;
            if (wk > 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    red[(((wk - 1) * WM * WN + slot) * NV + v) * kWave + lane] = acc[v / (NW * 4)][(v / 4) % NW][v % 4];
            }
            __syncthreads();
            if (wk == 0) {
                for (int j = 1; j < WK; ++j) {
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        acc[v / (NW * 4)][(v / 4) % NW][v % 4] += red[(((j - 1) * WM * WN + slot) * NV + v) * kWave + lane];
                }
            }
        }
        if (wk == 0) {
            float* o = out + static_cast<int64_t>(ks) * M * N;
#pragma unroll
            for (int mi = 0; mi < MW; ++mi)
#pragma unroll
                for (int ni = 0; ni < NW; ++ni) {
                    const int n = n0 + (wn * NW + ni) * 16 + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t m = (tm * (MW * WM) + wm * MW + mi) * 16 + 4 * lg + r;
                        if (m < M && n < N) o[m * N + n] = acc[mi][ni][r];
                    }
                }
        }
    }
}

// The wide tiling (M = 512 class): 64 x 64 outputs per workgroup, four waves
// as 2 (halves of the 64 activation rows) x 2 (even and odd blocks of each
// chunk), each wave a 32 x 64 tile = two 32 x 32 MFMA tiles.
//
// v_mfma_i32_32x32x32_i8 covers exactly one block: A 32 x 32 (lane l: row
// l % 32, elements 16 (l / 32) .. + 15 of the block), B 32 x 32 (lane l:
// column l % 32, the same 16 elements), D 32 x 32 int32 (lane l: column
// l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4 for i < 16).  A and B take the
// same element at the same byte of the same lane half, so D is the block's
// integer sum whatever order the hardware adds in.
//   * Activations: the tile-major layout (kLayoutSplit), a wave's operand of
//     a block is one coalesced 1 KB load, from global memory, three of the
//     wave's blocks ahead.
//   * Weights: 64 rows x 16 blocks per chunk, fetched one chunk ahead into
//     registers (whole block pairs, eight lanes per row), decoded
//     once per workgroup into LDS planes [block][half][row][16 B] of
//     16 (q - 8) signed bytes (half 0: low nibbles = elements 0 .. 15, half
//     1: high nibbles = elements 16 .. 31), so the integer sums are 16 isum.
//   * Scales: the product d_w * d_x / 16 of every (row, column) of a block
//     comes from one v_mfma_f32_32x32x8_bf16 (the same D layout) over the
//     exact bfloat16 terms of both scales: A = (h, m, l, h | m, l, 0, 0) of
//     d_x (bf16_split3), B = (H, H, H, L | L, L, 0, 0) of d_w / 16 = H + L
//     (11 significant bits: 8 + 3), so the six products h H + m H + l H +
//     h L + m L + l L are exact and summed in float32.  The epilogue is then
//     one convert and one FMA per output and block: acc += float(D) * S.
// The two waves of a row half add their sums in LDS at the end, even blocks
// first.  MODE kModeISum stores the block sums D / 16 of rows n in
// [isn0, isn1) instead (isum [M][isn1 - isn0][nb]), with every other step
// unchanged.
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short s4 __attribute__((ext_vector_type(4)));

// Which tiles and which chunks of 16 blocks each workgroup of a wide launch
// takes.  Items 0 .. whole - 1 are whole 64 x 64 tiles; items whole ..
// whole + parts - 1 share the remaining tiles' chunks, item j taking the
// units [j units / parts, (j + 1) units / parts) of the unit sequence (tile
// whole + u / nch, chunk u % nch), at most two tiles each, and write their
// sums to partial slots that qmm_wide_fixup_kernel adds in chunk order.  A
// CU holds workgroups i, i + 256 and i + 512 (three resident per CU), so with
// whole = 2 * 256 every CU gets two whole tiles and one share of the rest:
// even work instead of three tiles on some CUs and two on others.  Within
// each kind, consecutive items are dealt to the 8 XCDs so that each XCD gets
// a contiguous run (the same weight rows for all m-tiles).
struct WideSchedule {
    int64_t tm0;      // first m-tile of the launch
    int64_t tiles_m;  // m-tiles in the launch (tile t: m-tile t % tiles_m, n-tile t / tiles_m)
    int nch;          // chunks of 16 blocks per tile
    int whole;        // whole-tile items
    int parts;        // chunk-share items (0: none)
    int64_t units;    // (tiles - whole) * nch
};

// Item i of n consecutive items of one kind -> its rank in that kind, such
// that XCD i % 8 (where consecutive workgroups land) gets ranks
// (i % 8) n / 8 .. (i % 8 + 1) n / 8 - 1.
__device__ inline int64_t xcd_run(int64_t i, int64_t n) { return n % 8 == 0 ? (i % 8) * (n / 8) + i / 8 : i; }
// First unit of share j.
__device__ inline int64_t share_start(int64_t j, const WideSchedule& S) { return j * S.units / S.parts; }

template <int MODE>
__global__ __launch_bounds__(kBlockThreads)
void qmm_wide_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ xq, const uint4* __restrict__ xs,
                     float* __restrict__ out, float* __restrict__ part, int32_t* __restrict__ isum, int N, int64_t M,
                     int nb, WideSchedule S, int isn0, int isn1) {
    static_assert(MODE == kModeY || MODE == kModeISum, "y or block sums");
    constexpr int TM = 64, TN = 64, KC = 16;
    // LDS planes, [block j][half g] each TN rows of 16 (or 8) bytes.  The
    // stride of a block's plane pair is odd in 16-byte (8-byte) units, so
    // that the eight lanes that stash the eight block pairs of one row, and
    // the rows next to them, write to different banks.
    constexpr int kQStride = 2 * TN + 1;  // uint4 per block j
    constexpr int kSStride = 2 * TN + 1;  // uint2 per block j
    static_assert(kWavesPerBlock == 4 && KC == 16, "two block pairs of 32 rows per thread");
    __shared__ __align__(16) uint4 bq[KC * kQStride];   // decoded codes, 32.3 KB
    __shared__ __align__(16) uint2 bsc[KC * kSStride];  // scale operands, 16.1 KB

    const int64_t row_bytes = static_cast<int64_t>(nb) * 18;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int wm = w & 1;      // activation rows 32 wm .. 32 wm + 31 of the tile
    const int wk = w >> 1;     // blocks wk, wk + 2, ... of each chunk
    const int li = lane & 31;  // A row / B column of the lane
    const int lg = lane >> 5;  // k half of the lane
    const int fp = threadIdx.x & 7;
    const int fr = threadIdx.x >> 3;

    // this workgroup's segments: (tile, first chunk, end chunk, partial slot)
    const int64_t item = blockIdx.x;
    int64_t seg_tile[2];
    int seg_cb[2], seg_ce[2], nseg;
    int64_t share = -1;
    if (item < S.whole) {
        seg_tile[0] = xcd_run(item, S.whole);
        seg_cb[0] = 0;
        seg_ce[0] = S.nch;
        nseg = 1;
    } else {
        share = xcd_run(item - S.whole, S.parts);
        const int64_t u0 = share_start(share, S), u1 = share_start(share + 1, S);
        nseg = 0;
        // a share is shorter than a tile (the plan splits fewer than 256
        // tiles over 256 shares), so it meets at most two of them
        for (int64_t u = u0; u < u1 && nseg < 2;) {
            const int64_t r = u / S.nch;  // remaining tile
            const int64_t ue = ((r + 1) * S.nch < u1) ? (r + 1) * S.nch : u1;
            seg_tile[nseg] = S.whole + r;
            seg_cb[nseg] = static_cast<int>(u - r * S.nch);
            seg_ce[nseg] = static_cast<int>(ue - r * S.nch);
            ++nseg;
            u = ue;
        }
    }

    // (unrolled: as a loop the two passes held 60 more VGPRs live)
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
        if (sg >= nseg) break;
        const int64_t tile = seg_tile[sg];
        const int64_t tm = S.tm0 + tile % S.tiles_m;
        const int n0 = static_cast<int>(tile / S.tiles_m) * TN;
        const int kb0 = seg_cb[sg] * KC;
        const int kb1 = min(nb, seg_ce[sg] * KC);

        // Weight chunk (64 rows x 16 blocks): thread t fetches block pair
        // fp = t % 8 (36 bytes, 4-byte aligned) of rows fr = t / 8 and
        // fr + 32, so that eight consecutive lanes read a row's 288 bytes.  A
        // last chunk of 8 blocks reads (unused) pairs 0 .. 3 again; rows past
        // N read row N - 1.
        const uint8_t* frow0 = W + static_cast<int64_t>(min(n0 + fr, N - 1)) * row_bytes;
        const uint8_t* frow1 = W + static_cast<int64_t>(min(n0 + fr + 32, N - 1)) * row_bytes;
        uint32_t raw[2][9];
        auto fetch = [&](int c0) {
            const int b0 = c0 + 2 * fp;
            const int64_t off = static_cast<int64_t>(b0 < kb1 ? b0 : c0) * 18;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint8_t* src = (h ? frow1 : frow0) + off;
                const u32x4_a4 a = *reinterpret_cast<const u32x4_a4*>(src);
                const u32x4_a4 b = *reinterpret_cast<const u32x4_a4*>(src + 16);
                raw[h][0] = a.x; raw[h][1] = a.y; raw[h][2] = a.z; raw[h][3] = a.w;
                raw[h][4] = b.x; raw[h][5] = b.y; raw[h][6] = b.z; raw[h][7] = b.w;
                raw[h][8] = *reinterpret_cast<const uint32_t*>(src + 32);
            }
        };
        auto stash = [&]() {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = fr + 32 * h;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int j = 2 * fp + e;
                    uint32_t dbits, code[4];
                    if (e == 0) {  // first block of the pair: d at bytes 0-1, codes 2 bytes in
                        dbits = raw[h][0] & 0xffffu;
#pragma unroll
                        for (int g = 0; g < 4; ++g) code[g] = __builtin_amdgcn_alignbyte(raw[h][g + 1], raw[h][g], 2);
                    } else {  // second: d at bytes 18-19, codes at 20 .. 35 (aligned)
                        dbits = raw[h][4] >> 16;
#pragma unroll
                        for (int g = 0; g < 4; ++g) code[g] = raw[h][5 + g];
                    }
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        lo[g] = ((code[g] << 4) ^ 0x88888880u) & 0xF0F0F0F0u;  // elements 4g .. 4g + 3
                        hi[g] = (code[g] ^ 0x88888888u) & 0xF0F0F0F0u;         // elements 16 + 4g .. 16 + 4g + 3
                    }
                    bq[j * kQStride + row] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                    bq[j * kQStride + TN + row] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                    // d_w / 16 = H + L exactly (11 significant bits)
                    const float d16 = half_bits_to_float(dbits) * 0.0625f;
                    const uint32_t H = __float_as_uint(d16) & 0xffff0000u;
                    const uint32_t L = __float_as_uint(d16 - __uint_as_float(H)) & 0xffff0000u;
                    bsc[j * kSStride + row] = make_uint2((H >> 16) | H, (H >> 16) | L);
                    bsc[j * kSStride + TN + row] = make_uint2((L >> 16) | L, 0u);
                }
            }
        };

        // activation operands of block b (tile-major layout: 1 KB of codes and
        // 512 B of scale terms per 32-row tile and block)
        const int64_t at = tm * 2 + wm;  // 32-row tile
        const uint4* arow = reinterpret_cast<const uint4*>(xq) + at * nb * kWave + lane;
        const uint4* srow = xs + at * nb * 32 + li;
        struct AOp {
            v4i q;
            uint2 s;
        };
        auto load_a = [&](int64_t b, AOp& A) {
            A.q = __builtin_bit_cast(v4i, arow[b * kWave]);
            const uint2* sp = reinterpret_cast<const uint2*>(srow + b * 32);
            A.s = sp[lg];
        };

        float acc[2][16];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

        auto mul_block = [&](int j, const AOp& A, int64_t b) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const v4i bw = __builtin_bit_cast(v4i, bq[j * kQStride + lg * TN + 32 * t + li]);
                const v16i zi = {};
                const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A.q, bw, zi, 0, 0, 0);
                if constexpr (MODE == kModeISum) {
                    const int n = n0 + 32 * t + li;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t m = tm * TM + 32 * wm + 8 * (r / 4) + 4 * lg + (r % 4);
                        if (m < M && n >= isn0 && n < isn1)
                            isum[(m * (isn1 - isn0) + (n - isn0)) * nb + b] = D[r] >> 4;
                    }
                } else {
                    const uint2 ws = bsc[j * kSStride + lg * TN + 32 * t + li];
                    const v16f zf = {};
                    const v16f Sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s4, A.s),
                                                                             __builtin_bit_cast(s4, ws), zf, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[t][r] = fmaf(static_cast<float>(D[r]), Sc[r], acc[t][r]);
                }
            }
        };

        // This wave's blocks of the segment are b = kb0 + wk, + 2, ... (the
        // segment has an even block count).  Their activation operands stream
        // through a ring of four register sets, three blocks ahead of the
        // multiplies and across chunk boundaries; the loads are unconditional
        // (past the wave's last block they read it again).  A chunk gives
        // every wave 8 blocks (4 in a last half chunk), so the ring is back at
        // slot 0 at every chunk start.
        const int64_t blast = kb1 - 2 + wk;
        auto ahead = [&](int64_t b) { return b < blast ? b : blast; };
        AOp A0, A1, A2, A3;
        load_a(ahead(kb0 + wk), A0);
        load_a(ahead(kb0 + wk + 2), A1);
        load_a(ahead(kb0 + wk + 4), A2);
        fetch(kb0);
        for (int c0 = kb0; c0 < kb1; c0 += KC) {
            __syncthreads();  // every wave is done with the previous chunk (or segment)
            stash();
            __syncthreads();
            if (c0 + KC < kb1) fetch(c0 + KC);
            const int nblk = min(KC, kb1 - c0);  // 16, or 8 for a last half chunk
            for (int j = wk; j < nblk; j += 8) {
                const int64_t b = c0 + j;
                load_a(ahead(b + 6), A3);
                mul_block(j, A0, b);
                load_a(ahead(b + 8), A0);
                mul_block(j + 2, A1, b + 2);
                load_a(ahead(b + 10), A1);
                mul_block(j + 4, A2, b + 4);
                load_a(ahead(b + 12), A2);
                mul_block(j + 6, A3, b + 6);
            }
        }
        if constexpr (MODE == kModeY) {
            __syncthreads();  // the LDS planes are free
            float* red = reinterpret_cast<float*>(bq);
            if (wk == 1) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[((wm * 2 + t) * 16 + r) * kWave + lane] = acc[t][r];
            }
            __syncthreads();
            if (wk == 0) {
                // a whole tile goes to y; a share of a tile to its partial
                // slot [share][segment][64 rows][64 columns]
                float* slot = share >= 0 ? part + (share * 2 + sg) * (TM * TN) : nullptr;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int nl = 32 * t + li;
                    const int n = n0 + nl;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float v = acc[t][r] + red[((wm * 2 + t) * 16 + r) * kWave + lane];
                        const int ml = 32 * wm + 8 * (r / 4) + 4 * lg + (r % 4);
                        const int64_t m = tm * TM + ml;
                        if (slot) {
                            slot[ml * TN + nl] = v;
                        } else if (m < M && n < N) {
                            out[m * N + n] = v;
                        }
                    }
                }
            }
        }
    }
}

// y of the tiles that the chunk-share items split: the partial sums of each
// tile added in chunk order (so in share order).  Four workgroups per tile,
// one float4 of the tile per thread and share; the share bookkeeping is per
// workgroup.
__global__ __launch_bounds__(kBlockThreads)
void qmm_wide_fixup_kernel(const float* __restrict__ part, float* __restrict__ y, int N, int64_t M, WideSchedule S) {
    constexpr int TM = 64, TN = 64, kParts = TM * TN / 4 / kBlockThreads;
    static_assert(kParts == 4, "four workgroups per tile");
    const int64_t r = blockIdx.x / kParts;  // remaining tile
    const int quarter = blockIdx.x % kParts;
    const int64_t tile = S.whole + r;
    const int64_t tm = S.tm0 + tile % S.tiles_m;
    const int n0 = static_cast<int>(tile / S.tiles_m) * TN;
    const int64_t u0 = r * S.nch, u1 = (r + 1) * S.nch;
    // shares j0 .. j1 hold the tile's units u0 .. u1 - 1, in chunk order: the
    // share holding unit u is the last j with j units / parts <= u, that is
    // ((u + 1) parts - 1) / units; only j0 may have begun on the tile before
    const int64_t j0 = ((u0 + 1) * S.parts - 1) / S.units;
    const int64_t j1 = (u1 * S.parts - 1) / S.units;
    const int f4 = quarter * kBlockThreads + static_cast<int>(threadIdx.x);  // float4 of the tile
    const int first_seg = share_start(j0, S) < u0 ? 1 : 0;
    float4 v = reinterpret_cast<const float4*>(part + (j0 * 2 + first_seg) * (TM * TN))[f4];
    for (int64_t q = j0 + 1; q <= j1; ++q) {
        const float4 p = reinterpret_cast<const float4*>(part + q * 2 * (TM * TN))[f4];
        v.x += p.x;
        v.y += p.y;
        v.z += p.z;
        v.w += p.w;
    }
    const int e = 4 * f4;
    const int64_t m = tm * TM + e / TN;
    const int n = n0 + e % TN;
    const float o[4] = {v.x, v.y, v.z, v.w};
    if (m < M) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (n + c < N) y[m * N + n + c] = o[c];
    }
}

// ------------------------------------------------ float32 activations
// Q4_0 weights times float32 activations for small M (2 .. 32 rows: the
// fixed-eight verifier and the 32-row prefill tile of ["Gemma 4 M4 Max
// kernel roadmap", K3 prefill path and K5 advanced candidates]), reading the
// weights once for all rows.  The activations are not quantized: each
// 32-element block of a row is scaled by a power of two s = 2^e so that its
// largest magnitude lies in [2^14, 2^15), and split into two float16 terms,
// hi = f16(x / s) and lo = f16(x / s - hi).  (q - 8) is exact in float16, so
// two v_mfma_f32_16x16x32_f16 per block (hi, then lo into the same
// accumulator) give sum (q - 8) (hi + lo) with exact products and float32
// sums; |x / s - hi - lo| <= 2^-22 |x / s| for all but float16-subnormal
// terms, which lie 2^-24 below the block maximum.  The epilogue is
// y += D * (d_w * s) with d_w the block's float16 scale.

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Layout of the split activations, Mt = tiles of 16 rows, nb = K / 32:
//   hl [Mt][nb][64 lanes][32 B]: lane l = i + 16 g holds, for row 16 t + i,
//      hi then lo of x[4g .. 4g+3] and x[16+4g .. 16+4g+3] of block b (the
//      elements of code dword g of a Q4_0 block: low nibbles, then high);
//   sx [Mt][nb][16] float: s of row 16 t + i, block b.
// Rows M .. 16 Mt - 1 hold zeros (s = 1).
__global__ __launch_bounds__(kBlockThreads)
void split_f16_kernel(const float* __restrict__ x, uint8_t* __restrict__ hl, float* __restrict__ sx, int64_t K,
                      int64_t M, int64_t Mrows, bool vec_x) {
    const int64_t nb = K / 32;
    const int64_t total = Mrows * nb;
    const int t = threadIdx.x & 7;  // elements 4 t .. 4 t + 3 of the block
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (kBlockThreads / 8);
    for (int64_t wave_first = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + (threadIdx.x & ~(kWave - 1))) / 8;
         wave_first < total; wave_first += stride) {
        const int64_t blk = wave_first + (threadIdx.x & (kWave - 1)) / 8;
        const bool ok = blk < total;
        const int64_t m = ok ? blk / nb : 0;
        const int64_t b = ok ? blk - m * nb : 0;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ok && m < M) {
            const float* src = x + m * K + 32 * b + 4 * t;
            if (vec_x) {
                const float4 f = *reinterpret_cast<const float4*>(src);
                v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = src[e];
            }
        }
        float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 8));
        // s = 2^e with a / s in [2^14, 2^15); zero or non-finite blocks keep s = 1
        const int e = (a > 0.0f && a <= 3.4028234663852886e38f) ? ilogbf(a) - 14 : 0;
        h2 hi[2], lo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float x0 = ldexpf(v[2 * h], -e), x1 = ldexpf(v[2 * h + 1], -e);
            const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
            hi[h] = h2{h0, h1};
            lo[h] = h2{static_cast<_Float16>(x0 - static_cast<float>(h0)),
                       static_cast<_Float16>(x1 - static_cast<float>(h1))};
        }
        if (ok) {
            const int64_t mt = m >> 4, i = m & 15;
            const int g = (t & 3), half = t >> 2;  // elements 4t..: low nibbles (t < 4) or high (t >= 4)
            uint8_t* dst = hl + (((mt * nb + b) * kWave + i + 16 * g) * 32) + half * 8;
            *reinterpret_cast<uint2*>(dst) = make_uint2(__builtin_bit_cast(uint32_t, hi[0]), __builtin_bit_cast(uint32_t, hi[1]));
            *reinterpret_cast<uint2*>(dst + 16) = make_uint2(__builtin_bit_cast(uint32_t, lo[0]), __builtin_bit_cast(uint32_t, lo[1]));
            if (t == 0) sx[(mt * nb + b) * 16 + i] = ldexpf(1.0f, e);
        }
    }
}

// Code dword c of a Q4_0 block (code bytes 4g .. 4g+3) as the eight float16
// values (q - 8) in the element order of the split layout.
__device__ __forceinline__ h8 q4_codes_to_h8(uint32_t c) {
    const uint32_t p01 = __builtin_amdgcn_perm(0u, c, 0x0c010c00u);  // byte 0 -> bits 0..7, byte 1 -> 16..23
    const uint32_t p23 = __builtin_amdgcn_perm(0u, c, 0x0c030c02u);  // bytes 2, 3 likewise
    constexpr uint32_t kNib = 0x000F000Fu, kMagic = 0x64006400u;    // float16 1024 + n
    const h2 off = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const h2 a = __builtin_bit_cast(h2, (p01 & kNib) | kMagic) - off;         // elements 4g, 4g+1
    const h2 b = __builtin_bit_cast(h2, (p23 & kNib) | kMagic) - off;         // 4g+2, 4g+3
    const h2 c2 = __builtin_bit_cast(h2, ((p01 >> 4) & kNib) | kMagic) - off;  // 16+4g, 16+4g+1
    const h2 d = __builtin_bit_cast(h2, ((p23 >> 4) & kNib) | kMagic) - off;   // 16+4g+2, 16+4g+3
    return h8{a[0], a[1], b[0], b[1], c2[0], c2[1], d[0], d[1]};
}

// 16 MW rows of m x 16 NW weight rows per workgroup: every wave multiplies
// all of them, the four waves split each chunk's block pairs, their sums are
// added in LDS in wave order, and K may be split across workgroups
// (PARTIAL: write split ks of the partial sums).  The weight chunk is staged
// as raw GGUF bytes (16 NW rows x KC blocks) with 16-byte loads, the next
// chunk prefetched into registers.  The activation loads are the costly
// traffic here (32 bytes per lane per block and m-tile from the caches), so
// each is used for NW weight tiles.
template <int MW, int NW, int KC, bool PARTIAL>
__global__ __launch_bounds__(kBlockThreads)
void qmm_f16_kernel(const uint8_t* __restrict__ W, const uint8_t* __restrict__ hl, const float* __restrict__ sx,
                    float* __restrict__ out, int N, int64_t M, int nb, int64_t tm0, int64_t tiles_m, int tiles_n,
                    int kb_per, int64_t nwg) {
    constexpr int TN = 16 * NW;
    constexpr int WK = kWavesPerBlock;
    constexpr int RB = KC * 18;
    constexpr int RS = RB + 16;  // LDS row stride: rows 4 banks apart (mod 64)
    constexpr int PR = RB / 16;
    constexpr int LPT = TN * PR / kBlockThreads;
    static_assert(KC % 8 == 0 && TN * PR == LPT * kBlockThreads, "the weight chunk must split evenly");
    constexpr int NV = MW * NW * 4;
    static_assert((WK - 1) * NV * kWave <= TN * RS / 4, "the reduction fits the weight tile");
    __shared__ __align__(16) uint32_t wt[TN * RS / 4];

    int64_t lin = blockIdx.x;
    if (nwg % 8 == 0) lin = (lin % 8) * (nwg / 8) + lin / 8;
    const int64_t tm = tm0 + lin % tiles_m;
    lin /= tiles_m;
    const int tn = static_cast<int>(lin % tiles_n);
    const int ks = static_cast<int>(lin / tiles_n);
    const int kb0 = ks * kb_per;
    const int kb1 = min(nb, kb0 + kb_per);
    const int n0 = tn * TN;
    const int64_t row_bytes = static_cast<int64_t>(nb) * 18;

    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15;
    const int lg = lane >> 4;

    uint32_t pre[LPT * 4];
    auto fetch = [&](int c0) {
        const int valid = min(KC, kb1 - c0) * 18;  // a multiple of 144
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const int p = t * kBlockThreads + static_cast<int>(threadIdx.x);
            const int r = p / PR;
            const int q = p - r * PR;
            const int row = min(n0 + r, N - 1);             // rows past N: any valid row
            const int off = (q * 16 < valid) ? q * 16 : 0;  // blocks past the split: any valid piece
            const uint4 v = *reinterpret_cast<const uint4*>(W + row * row_bytes + static_cast<int64_t>(c0) * 18 + off);
            pre[4 * t + 0] = v.x;
            pre[4 * t + 1] = v.y;
            pre[4 * t + 2] = v.z;
            pre[4 * t + 3] = v.w;
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const int p = t * kBlockThreads + static_cast<int>(threadIdx.x);
            const int r = p / PR;
            const int q = p - r * PR;
            *reinterpret_cast<uint4*>(wt + r * (RS / 4) + q * 4) =
                make_uint4(pre[4 * t], pre[4 * t + 1], pre[4 * t + 2], pre[4 * t + 3]);
        }
    };

    float acc[MW][NW][4];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][ni][r] = 0.0f;

    struct AFrag {
        h8 h[MW][2], l[MW][2];  // hi / lo of blocks b, b + 1
        float s[MW][2][4];      // their scales, rows 4 lg .. 4 lg + 3
    };

    fetch(kb0);
    for (int c0 = kb0; c0 < kb1; c0 += KC) {
        __syncthreads();  // every wave is done with the previous chunk
        stash();
        __syncthreads();
        if (c0 + KC < kb1) fetch(c0 + KC);
        const int npair = min(KC, kb1 - c0) >> 1;
        // Rows past M are zero in the split layout (scale 1).  Lanes of such
        // rows all read the tile's first zero row: one address, no extra
        // traffic, and no branch around the loads.
        auto load_a = [&](int cp, AFrag& A) {
            const int64_t b = c0 + 2 * cp;
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
                const int64_t mt = tm * MW + mi;
                const int64_t live = M - mt * 16;  // real rows of this tile (may exceed 16)
                const int ai = (live < 16 && li > live) ? static_cast<int>(live) : li;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint4* src = reinterpret_cast<const uint4*>(hl + ((mt * nb + b + j) * kWave + ai + 16 * lg) * 32);
                    A.h[mi][j] = __builtin_bit_cast(h8, src[0]);
                    A.l[mi][j] = __builtin_bit_cast(h8, src[1]);
                    const float4 sv = *reinterpret_cast<const float4*>(sx + (mt * nb + b + j) * 16 + 4 * lg);
                    A.s[mi][j][0] = sv.x; A.s[mi][j][1] = sv.y; A.s[mi][j][2] = sv.z; A.s[mi][j][3] = sv.w;
                }
            }
        };
        auto mul_pair = [&](int cp, const AFrag& A) {
#pragma unroll
            for (int ni = 0; ni < NW; ++ni) {
                const uint32_t* rowp = wt + (ni * 16 + li) * (RS / 4) + 9 * cp;
                h8 bw[2];
                float dw[2];
                bw[0] = q4_codes_to_h8(__builtin_amdgcn_alignbyte(rowp[lg + 1], rowp[lg], 2));  // block b: codes 2 mod 4
                bw[1] = q4_codes_to_h8(rowp[5 + lg]);                                         // block b + 1: aligned
                dw[0] = half_bits_to_float(rowp[0] & 0xffffu);
                dw[1] = half_bits_to_float(rowp[4] >> 16);
#pragma unroll
                for (int mi = 0; mi < MW; ++mi) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                        v4f D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[mi][j], bw[j], zero, 0, 0, 0);
                        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.l[mi][j], bw[j], D, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[mi][ni][r] = fmaf(D[r], dw[j] * A.s[mi][j][r], acc[mi][ni][r]);
                    }
                }
            }
        };
        // the activations of the next pair are requested before the current
        // pair is multiplied, with unconditional loads
        if (wk < npair) {
            AFrag A0, A1;
            int cp = wk;
            load_a(cp, A0);
            while (true) {
                load_a(min(cp + WK, npair - 1), A1);
                mul_pair(cp, A0);
                cp += WK;
                if (cp >= npair) break;
                load_a(min(cp + WK, npair - 1), A0);
                mul_pair(cp, A1);
                cp += WK;
                if (cp >= npair) break;
            }
        }
    }
    __syncthreads();  // the weight tile is free
    float* red = reinterpret_cast<float*>(wt);
    if (wk > 0) {
#pragma unroll
        for (int v = 0; v < NV; ++v) red[((wk - 1) * NV + v) * kWave + lane] = acc[v / (NW * 4)][(v / 4) % NW][v % 4];
    }
    __syncthreads();
    if (wk == 0) {
        for (int j = 1; j < WK; ++j) {
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[v / (NW * 4)][(v / 4) % NW][v % 4] += red[((j - 1) * NV + v) * kWave + lane];
        }
        float* o = out + (PARTIAL ? static_cast<int64_t>(ks) * M * N : 0);
#pragma unroll
        for (int ni = 0; ni < NW; ++ni) {
            const int n = n0 + ni * 16 + li;
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = (tm * MW + mi) * 16 + 4 * lg + r;
                    if (m < M && n < N) o[m * N + n] = acc[mi][ni][r];
                }
            }
        }
    }
}

// y = sum over K splits of the partial sums, in split order.
__global__ __launch_bounds__(kBlockThreads)
void qmm_reduce_kernel(const float* __restrict__ P, float* __restrict__ y, int ks, int64_t MN) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlockThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x; i < MN; i += stride) {
        float s = P[i];
        for (int k = 1; k < ks; ++k) s += P[k * MN + i];
        y[i] = s;
    }
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest K whose activation codes and scales fit one workgroup's LDS in
// qmm_dot_kernel.
constexpr int64_t kDotMaxG = 200;

// The two MFMA tilings: wide (64 x 64 per workgroup, qmm_wide_kernel) and
// narrow (16 x 32 per workgroup: each wave two 16 x 16 tiles sharing one
// activation load, the four waves splitting K, chunks of 64 blocks).
#define QMM_NARROW 1, 2, 1, 1, 4, 64
constexpr int kWideTM = 64, kWideTN = 64, kNarrowTM = 16, kNarrowTN = 32;

enum QmmPath : int { kPathDot = 0, kPathGeneric = 1, kPathWide = 2, kPathNarrow = 3 };

// Everything about a call that depends only on (N, K, M): kernels, tiles,
// K splits and the workspace parts, so that the workspace size and the
// launches always agree.
struct QmmPlan {
    int path = kPathGeneric;
    int64_t tiles_m = 0;
    int tiles_n = 0, ks = 1, kb = 0;
    int64_t xrows = 0;  // activation rows in the workspace (padded to the tile height)
    int whole = 0, parts = 0;  // the wide tiling's item split (wide_schedule)
    size_t q_bytes = 0, d_bytes = 0, p_bytes = 0;
};

// The wide tiling's workgroups are resident three per CU (48.4 KB of LDS
// each), and a CU receives workgroups i, i + C and i + 2C of a grid of at
// most 3C.  With C < T < 3C tiles and T % C != 0, a grid of one workgroup
// per tile leaves some CUs a tile more than others; instead the last
// T - floor(T / C) C tiles are cut into C equal shares of chunks.  The split
// is planned for C = 256 (the MI355X count) so that workspace sizes do not
// depend on the device; a device with another count runs one workgroup per
// tile.
constexpr int kWideCUs = 256;

void wide_schedule(int64_t tiles, int64_t nch, int* whole, int* parts) {
    const int64_t per = tiles / kWideCUs;
    // (the shares are never empty: at least one chunk each)
    if (tiles > kWideCUs && tiles < 3 * kWideCUs && (tiles % kWideCUs) * nch >= kWideCUs) {
        *whole = static_cast<int>(per * kWideCUs);
        *parts = kWideCUs;
    } else {
        *whole = static_cast<int>(tiles);
        *parts = 0;
    }
}

QmmPlan plan_qmm(int64_t N, int64_t K, int64_t M) {
    QmmPlan p;
    const int64_t nb = K / 32;
    const bool units = K % kUnitElems == 0;
    if (M == 1 || !units) {
        p.path = (units && K / kUnitElems <= kDotMaxG) ? kPathDot : kPathGeneric;
        p.xrows = M;
    } else if (ceil_div(M, kWideTM) * ceil_div(N, kWideTN) >= 512) {
        p.path = kPathWide;
        p.tiles_m = ceil_div(M, kWideTM);
        p.tiles_n = static_cast<int>(ceil_div(N, kWideTN));
        p.ks = 1;
        p.kb = static_cast<int>(nb);
        p.xrows = p.tiles_m * kWideTM;
        if (p.tiles_m * p.tiles_n < (int64_t{1} << 30)) wide_schedule(p.tiles_m * p.tiles_n, ceil_div(nb, 16), &p.whole, &p.parts);
    } else {
        p.path = kPathNarrow;
        p.tiles_m = ceil_div(M, kNarrowTM);
        p.tiles_n = static_cast<int>(ceil_div(N, kNarrowTN));
        const int64_t tiles = p.tiles_m * p.tiles_n;
        // about 1024 workgroups: enough to stream the weights from every CU,
        // few enough to be resident at once (4 per CU); a workgroup that
        // signalled the others through memory would need a cache writeback
        // per workgroup, so the splits are added by a second kernel
        int64_t ks = 1024 / tiles;
        ks = ks < nb / 8 ? ks : nb / 8;
        ks = ks > 1 ? ks : 1;
        const int64_t kb = ceil_div(ceil_div(nb, ks), 8) * 8;
        p.kb = static_cast<int>(kb);
        p.ks = static_cast<int>(ceil_div(nb, kb));
        p.xrows = p.tiles_m * kNarrowTM;
    }
    p.q_bytes = align256(static_cast<size_t>(p.xrows) * static_cast<size_t>(K));
    // scales: float32, or the wide tiling's 16-byte bf16 operand pairs
    const size_t dsize = p.path == kPathWide ? sizeof(uint4) : sizeof(float);
    p.d_bytes = align256(static_cast<size_t>(p.xrows) * static_cast<size_t>(nb) * dsize);
    p.p_bytes = p.ks > 1 ? align256(static_cast<size_t>(p.ks) * static_cast<size_t>(M) * static_cast<size_t>(N) *
                                    sizeof(float))
                         : 0;
    // the wide tiling's partial slots: two 64 x 64 float32 tiles per share
    if (p.parts > 0) p.p_bytes = static_cast<size_t>(p.parts) * 2 * kWideTM * kWideTN * sizeof(float);
    return p;
}

template <int LAYOUT>
hipError_t launch_quantize(const float* x, int8_t* q, float* d, int64_t K, int64_t M, int64_t Mrows,
                           hipStream_t stream) {
    if constexpr (LAYOUT == kLayoutSplit) {
        const int64_t items = (Mrows / 32) * (K / 32);
        int64_t blocks = ceil_div(items, kWavesPerBlock);
        const int64_t cap = static_cast<int64_t>(device_cus()) * 16;
        if (blocks > cap) blocks = cap;
        const bool vec_x = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
        hipLaunchKernelGGL(quantize_q8_tiles_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0,
                           stream, x, q, reinterpret_cast<uint4*>(d), K, M, Mrows, vec_x);
    } else {
        const int64_t groups = Mrows * (K / 32);
        int64_t blocks = ceil_div(groups * 8, kBlockThreads);
        const int64_t cap = static_cast<int64_t>(device_cus()) * 64;
        if (blocks > cap) blocks = cap;
        const bool vec_x = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
        const bool vec_q = (reinterpret_cast<uintptr_t>(q) & 3) == 0;
        hipLaunchKernelGGL((quantize_q8_kernel<LAYOUT>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0,
                           stream, x, q, d, K, M, Mrows, vec_x, vec_q);
    }
    return hipGetLastError();
}

template <int MW, int NW, int WM, int WN, int WK, int KC, int MODE>
hipError_t launch_mfma(const QmmPlan& p, const void* W, const int8_t* xa, const float* xd, float* out,
                       int32_t* isum, int64_t isn0, int64_t isn1, int64_t N, int64_t K, int64_t M,
                       hipStream_t stream) {
    // slices of m-tiles keep the grid within 2^30 workgroups
    const int64_t per_mt = static_cast<int64_t>(p.tiles_n) * p.ks;
    int64_t mt_slice = (int64_t{1} << 30) / per_mt;
    mt_slice = mt_slice < p.tiles_m ? mt_slice : p.tiles_m;
    for (int64_t tm0 = 0; tm0 < p.tiles_m; tm0 += mt_slice) {
        const int64_t tms = (p.tiles_m - tm0 < mt_slice) ? p.tiles_m - tm0 : mt_slice;
        const int64_t nwg = tms * per_mt;
        hipLaunchKernelGGL((qmm_mfma_kernel<MW, NW, WM, WN, WK, KC, MODE>), dim3(static_cast<unsigned>(nwg)),
                           dim3(kBlockThreads), 0, stream, static_cast<const uint8_t*>(W), xa, xd, out, isum,
                           static_cast<int>(N), M, static_cast<int>(K / 32), tm0, tms, p.tiles_n, p.kb, nwg,
                           static_cast<int>(isn0), static_cast<int>(isn1));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The wide path: qmm_wide_kernel over all tiles, in slices of m-tiles that
// keep the grid within 2^30 workgroups; with a chunk-share split (one slice),
// qmm_wide_fixup_kernel then writes the split tiles' y.
template <int MODE>
hipError_t launch_wide(const QmmPlan& p, const void* W, const int8_t* xa, const float* xd, float* y, float* part,
                       int32_t* isum, int64_t isn0, int64_t isn1, int64_t N, int64_t K, int64_t M,
                       hipStream_t stream) {
    int64_t mt_slice = (int64_t{1} << 30) / p.tiles_n;
    mt_slice = mt_slice < p.tiles_m ? mt_slice : p.tiles_m;
    const int64_t nb = K / 32;
    const bool split = p.parts > 0 && device_cus() == kWideCUs;
    for (int64_t tm0 = 0; tm0 < p.tiles_m; tm0 += mt_slice) {
        const int64_t tms = (p.tiles_m - tm0 < mt_slice) ? p.tiles_m - tm0 : mt_slice;
        const int64_t tiles = tms * p.tiles_n;
        WideSchedule S;
        S.tm0 = tm0;
        S.tiles_m = tms;
        S.nch = static_cast<int>(ceil_div(nb, 16));
        S.whole = split ? p.whole : static_cast<int>(tiles);
        S.parts = split ? p.parts : 0;
        S.units = (tiles - S.whole) * S.nch;
        const int64_t nwg = static_cast<int64_t>(S.whole) + S.parts;
        hipLaunchKernelGGL((qmm_wide_kernel<MODE>), dim3(static_cast<unsigned>(nwg)), dim3(kBlockThreads), 0,
                           stream, static_cast<const uint8_t*>(W), xa, reinterpret_cast<const uint4*>(xd), y, part,
                           isum, static_cast<int>(N), M, static_cast<int>(nb), S, static_cast<int>(isn0),
                           static_cast<int>(isn1));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (MODE == kModeY && S.parts > 0) {
            hipLaunchKernelGGL(qmm_wide_fixup_kernel, dim3(static_cast<unsigned>(4 * (tiles - S.whole))),
                               dim3(kBlockThreads), 0, stream, part, y, static_cast<int>(N), M, S);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Plan of qmm_q4_0_f32act for (N, K, M): M == 1 or K % 256 != 0 take the
// float32 matrix-vector kernels row by row (no workspace); otherwise the
// split activations, the float16 MFMA kernel (16 or 32 rows per tile) and,
// when K is split across workgroups, the ordered reduction.
struct F32ActPlan {
    bool mfma = false;
    int mw = 1, nw = 2;  // 16-row tiles of m per workgroup, of n per wave
    int64_t tiles_m = 0;
    int tiles_n = 0, ks = 1, kb = 0;
    int64_t xrows = 0;
    size_t hl_bytes = 0, s_bytes = 0, p_bytes = 0;
};

F32ActPlan plan_f32act(int64_t N, int64_t K, int64_t M) {
    F32ActPlan p;
    const int64_t nb = K / 32;
    if (M == 1 || K % kUnitElems != 0) return p;
    p.mfma = true;
    // one 16-row m-tile with two n-tiles per wave, or two m-tiles with four:
    // more n-tiles per wave share each activation load
    p.mw = M > 16 ? 2 : 1;
    p.nw = M > 16 ? 4 : 2;
    p.tiles_m = ceil_div(M, 16 * p.mw);
    p.tiles_n = static_cast<int>(ceil_div(N, 16 * p.nw));
    const int64_t tiles = p.tiles_m * p.tiles_n;
    // about 1024 workgroups, as for the narrow int8 tiling
    int64_t ks = 1024 / tiles;
    ks = ks < nb / 8 ? ks : nb / 8;
    ks = ks > 1 ? ks : 1;
    const int64_t kb = ceil_div(ceil_div(nb, ks), 8) * 8;
    p.kb = static_cast<int>(kb);
    p.ks = static_cast<int>(ceil_div(nb, kb));
    p.xrows = p.tiles_m * 16 * p.mw;
    p.hl_bytes = align256(static_cast<size_t>(p.xrows) * static_cast<size_t>(K) * 4);
    p.s_bytes = align256(static_cast<size_t>(p.xrows) * static_cast<size_t>(nb) * sizeof(float));
    p.p_bytes = p.ks > 1 ? align256(static_cast<size_t>(p.ks) * static_cast<size_t>(M) * static_cast<size_t>(N) *
                                    sizeof(float))
                         : 0;
    return p;
}

template <int MW, int NW, int KC, bool PARTIAL>
hipError_t launch_f16(const F32ActPlan& p, const void* W, const uint8_t* hl, const float* sx, float* out, int64_t N,
                      int64_t K, int64_t M, hipStream_t stream) {
    const int64_t per_mt = static_cast<int64_t>(p.tiles_n) * p.ks;
    int64_t mt_slice = (int64_t{1} << 30) / per_mt;
    mt_slice = mt_slice < p.tiles_m ? mt_slice : p.tiles_m;
    for (int64_t tm0 = 0; tm0 < p.tiles_m; tm0 += mt_slice) {
        const int64_t tms = (p.tiles_m - tm0 < mt_slice) ? p.tiles_m - tm0 : mt_slice;
        const int64_t nwg = tms * per_mt;
        hipLaunchKernelGGL((qmm_f16_kernel<MW, NW, KC, PARTIAL>), dim3(static_cast<unsigned>(nwg)), dim3(kBlockThreads),
                           0, stream, static_cast<const uint8_t*>(W), hl, sx, out, static_cast<int>(N), M,
                           static_cast<int>(K / 32), tm0, tms, p.tiles_n, p.kb, nwg);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The M == 1 and K % 256 != 0 paths (row-major activation codes).
hipError_t launch_dot(const QmmPlan& p, const void* W, const int8_t* qx, const float* dx, float* y, int32_t* isum,
                      int64_t isn0, int64_t isn1, int64_t N64, int64_t K, int64_t M, hipStream_t stream) {
    if (p.path == kPathGeneric) {
        int64_t blocks = (N64 * M + kWavesPerBlock - 1) / kWavesPerBlock;
        const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
        if (blocks > cap) blocks = cap;
        if (isum) {
            hipLaunchKernelGGL((qmm_generic_kernel<true>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads),
                               0, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N64, K, M, isn0, isn1);
        } else {
            hipLaunchKernelGGL((qmm_generic_kernel<false>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads),
                               0, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N64, K, M, isn0, isn1);
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
                               npasses, static_cast<int>(m0), static_cast<int>(isn0), static_cast<int>(isn1));
        } else {
            hipLaunchKernelGGL((qmm_dot_kernel<false>), dim3(blocks, static_cast<unsigned>(mc)), dim3(kBlockThreads),
                               lds, stream, static_cast<const uint8_t*>(W), qx, dx, y, isum, N, G, C, L, S,
                               npasses, static_cast<int>(m0), static_cast<int>(isn0), static_cast<int>(isn1));
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t qmm_ws_bytes(int64_t N, int64_t K, int64_t M) {
    const QmmPlan p = plan_qmm(N, K, M);
    return p.q_bytes + p.d_bytes + p.p_bytes;
}

hipError_t launch_quantize_q8(const float* x, int8_t* q, float* d, int64_t K, int64_t M, hipStream_t stream) {
    return launch_quantize<kLayoutRows>(x, q, d, K, M, M, stream);
}

hipError_t launch_qmm_q8act(const void* W, const float* x, float* y, int32_t* isum, int64_t isn0, int64_t isn1,
                            int64_t N, int64_t K, int64_t M, void* ws, hipStream_t stream) {
    const QmmPlan p = plan_qmm(N, K, M);
    int8_t* q = static_cast<int8_t*>(ws);
    float* d = reinterpret_cast<float*>(static_cast<char*>(ws) + p.q_bytes);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.q_bytes + p.d_bytes);
    const bool mfma = p.path == kPathWide || p.path == kPathNarrow;
    hipError_t e = p.path == kPathWide     ? launch_quantize<kLayoutSplit>(x, q, d, K, M, p.xrows, stream)
                   : p.path == kPathNarrow ? launch_quantize<kLayoutFrag>(x, q, d, K, M, p.xrows, stream)
                                           : launch_quantize<kLayoutRows>(x, q, d, K, M, M, stream);
    if (e != hipSuccess) return e;
    if (!mfma) return launch_dot(p, W, q, d, isum ? nullptr : y, isum, isn0, isn1, N, K, M, stream);
    if (p.path == kPathWide) {
        return isum ? launch_wide<kModeISum>(p, W, q, d, nullptr, part, isum, isn0, isn1, N, K, M, stream)
                    : launch_wide<kModeY>(p, W, q, d, y, part, nullptr, 0, 0, N, K, M, stream);
    }
    // the narrow tiling: the block-sum mode runs the same grid, K splits included
    if (isum) return launch_mfma<QMM_NARROW, kModeISum>(p, W, q, d, nullptr, isum, isn0, isn1, N, K, M, stream);
    if (p.ks == 1) return launch_mfma<QMM_NARROW, kModeY>(p, W, q, d, y, nullptr, 0, 0, N, K, M, stream);
    e = launch_mfma<QMM_NARROW, kModePartial>(p, W, q, d, part, nullptr, 0, 0, N, K, M, stream);
    if (e != hipSuccess) return e;
    const int64_t MN = M * N;
    int64_t blocks = ceil_div(MN, kBlockThreads);
    const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(qmm_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0, stream,
                       part, y, p.ks, MN);
    return hipGetLastError();
}

size_t qmm_f32act_ws_bytes(int64_t N, int64_t K, int64_t M) {
    const F32ActPlan p = plan_f32act(N, K, M);
    const size_t b = p.hl_bytes + p.s_bytes + p.p_bytes;
    return b > 256 ? b : 256;
}

hipError_t launch_qmm_f32act(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, void* ws,
                             hipStream_t stream) {
    const F32ActPlan p = plan_f32act(N, K, M);
    if (!p.mfma) {
        for (int64_t m = 0; m < M; ++m) {
            const hipError_t e = launch_gemv(0, W, nullptr, x + m * K, nullptr, y + m * N, N, K, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    uint8_t* hl = static_cast<uint8_t*>(ws);
    float* sx = reinterpret_cast<float*>(static_cast<char*>(ws) + p.hl_bytes);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.hl_bytes + p.s_bytes);
    {
        const int64_t groups = p.xrows * (K / 32);
        int64_t blocks = ceil_div(groups * 8, kBlockThreads);
        const int64_t cap = static_cast<int64_t>(device_cus()) * 64;
        if (blocks > cap) blocks = cap;
        const bool vec_x = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
        hipLaunchKernelGGL(split_f16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0, stream, x,
                           hl, sx, K, M, p.xrows, vec_x);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e;
    // weight chunks: 32 rows x 64 blocks or 64 rows x 32 blocks (37 KB of LDS)
    if (p.ks == 1) {
        e = p.mw == 2 ? launch_f16<2, 4, 32, false>(p, W, hl, sx, y, N, K, M, stream)
                      : launch_f16<1, 2, 64, false>(p, W, hl, sx, y, N, K, M, stream);
        return e;
    }
    e = p.mw == 2 ? launch_f16<2, 4, 32, true>(p, W, hl, sx, part, N, K, M, stream)
                  : launch_f16<1, 2, 64, true>(p, W, hl, sx, part, N, K, M, stream);
    if (e != hipSuccess) return e;
    const int64_t MN = M * N;
    int64_t blocks = ceil_div(MN, kBlockThreads);
    const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(qmm_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0, stream, part,
                       y, p.ks, MN);
    return hipGetLastError();
}

}  // namespace qmv
