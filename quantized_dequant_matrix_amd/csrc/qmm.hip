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

// One 8-lane group per 32-element block, 4 elements per lane.  FRAG: write
// the fragment layout (rows padded to a multiple of 16), else row-major
// codes [M][K] and scales [M][K/32].
template <bool FRAG>
__global__ __launch_bounds__(kBlockThreads)
void quantize_q8_kernel(const float* __restrict__ x, int8_t* __restrict__ q, float* __restrict__ d,
                        int64_t K, int64_t M, int64_t Mrows, bool vec_x, bool vec_q) {
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
            if constexpr (FRAG) {
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

// The wide tiling (M = 512 class), with the weight codes decoded once per
// workgroup.  A 64 x 64 tile per workgroup, 32 x 32 per wave (2 x 2 MFMA tiles
// of 16 x 16).  Per chunk of KC = 16 blocks:
//   * weights: a thread owns 4 whole blocks (72 bytes) of one of the 64 rows,
//     fetched with 8-byte loads one chunk ahead, decoded in registers to
//     16 (q - 8) signed bytes and d / 16, and stored in LDS in the MFMA
//     operand layout: block j, k-group g, row r at
//     bq[j * kBlockStride + g * kGroupStride + 2 r] (8 bytes).  The group
//     stride puts a wave's four k-group reads on bank halves two by two, the
//     block stride puts the four quarter-row writers of a wave on disjoint
//     banks;
//   * activations: read from the fragment layout in global memory (the
//     whole [M, K] set stays in the caches), one block pair ahead of the
//     multiplies, with unconditional loads so that no branch merges the
//     waits (the pair after the last one re-reads the last pair).
//
// MODE kModeISum replaces the float epilogue by a store of the exact block
// sums of the rows n in [isn0, isn1) (isum [M][isn1 - isn0][nb]); every other
// step -- the grid, the weight stash and decode, the operand layouts and the
// MFMAs -- is the one that computes y.
template <int KC, int MODE>
__global__ __launch_bounds__(kBlockThreads)
void qmm_wide_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ xa, const float* __restrict__ xd,
                     float* __restrict__ out, int32_t* __restrict__ isum, int N, int64_t M, int nb, int64_t tm0,
                     int64_t tiles_m, int tiles_n, int64_t nwg, int isn0, int isn1) {
    static_assert(MODE == kModeY || MODE == kModeISum, "y or block sums");
    constexpr int MW = 2, NW = 2, WM = 2, WN = 2;
    constexpr int TN = 16 * NW * WN;           // 64 weight rows
    constexpr int kGroupStride = 2 * TN + 32;  // dwords: k-groups 32 banks apart
    constexpr int kBlockStride = 4 * kGroupStride + 4;
    static_assert(TN * 4 == kBlockThreads, "a thread owns one quarter of a row's chunk");
    static_assert(KC == 16, "four quarters of four blocks per row");
    static_assert(WM * WN == kWavesPerBlock, "four waves per workgroup");
    __shared__ __align__(16) uint32_t bq[KC * kBlockStride];
    __shared__ float bs[KC * TN];

    // Each XCD gets a contiguous run of tiles (same weight rows, all m-tiles).
    int64_t lin = blockIdx.x;
    if (nwg % 8 == 0) lin = (lin % 8) * (nwg / 8) + lin / 8;
    const int64_t tm = tm0 + lin % tiles_m;
    const int tn = static_cast<int>(lin / tiles_m);
    const int n0 = tn * TN;
    const int64_t row_bytes = static_cast<int64_t>(nb) * 18;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int wn = w % WN;
    const int wm = w / WN;
    const int li = lane & 15;
    const int lg = lane >> 4;

    // Weight chunk: thread -> row fr, quarter fq = blocks 4 fq .. 4 fq + 3.
    // nb is a multiple of 8, so a quarter is either whole or past the end;
    // quarters past the end (and rows past N) read valid bytes that are never
    // used.  Rows are 16-byte aligned (nb * 18 = 144 * (nb / 8)).
    const int fr = threadIdx.x >> 2;
    const int fq = threadIdx.x & 3;
    const uint8_t* frow = W + static_cast<int64_t>(min(n0 + fr, N - 1)) * row_bytes;
    uint2 raw[9];
    auto fetch = [&](int c0) {
        const int b0 = c0 + 4 * fq;
        const int64_t off = (b0 < nb) ? static_cast<int64_t>(b0) * 18 : 0;
        const uint2* src = reinterpret_cast<const uint2*>(frow + off);
#pragma unroll
        for (int i = 0; i < 9; ++i) raw[i] = src[i];
    };
    auto stash = [&]() {
        uint32_t dw[18];
#pragma unroll
        for (int i = 0; i < 9; ++i) {
            dw[2 * i] = raw[i].x;
            dw[2 * i + 1] = raw[i].y;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int blk = 4 * fq + j;
            uint32_t dbits, code[4];
            if ((j & 1) == 0) {  // block starts on a dword: codes 2 bytes in
                const int q0 = (18 * j) / 4;
                dbits = dw[q0] & 0xffffu;
#pragma unroll
                for (int g = 0; g < 4; ++g) code[g] = __builtin_amdgcn_alignbyte(dw[q0 + g + 1], dw[q0 + g], 2);
            } else {  // block starts 2 bytes into a dword: codes aligned
                const int q0 = (18 * j - 2) / 4;
                dbits = dw[q0] >> 16;
#pragma unroll
                for (int g = 0; g < 4; ++g) code[g] = dw[q0 + 1 + g];
            }
            uint32_t* dst = bq + blk * kBlockStride + 2 * fr;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint64_t v = q4_codes_to_s8(code[g]);
                *reinterpret_cast<uint2*>(dst + g * kGroupStride) =
                    make_uint2(static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32));
            }
            bs[blk * TN + fr] = half_bits_to_float(dbits) * 0.0625f;
        }
    };

    struct AFrag {
        uint64_t e[MW], o[MW];      // codes of blocks b, b + 1
        float xe[MW][4], xo[MW][4];  // their scales, rows 4 lg .. 4 lg + 3
    };
    auto load_a = [&](int64_t b, AFrag& A) {
#pragma unroll
        for (int mi = 0; mi < MW; ++mi) {
            const int64_t mt = tm * (MW * WM) + wm * MW + mi;
            const uint4 v = *reinterpret_cast<const uint4*>(xa + ((mt * (nb >> 1) + (b >> 1)) * kWave + lane) * 16);
            A.e[mi] = static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32);
            A.o[mi] = static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32);
            const float4 de = *reinterpret_cast<const float4*>(xd + (mt * nb + b) * 16 + 4 * lg);
            const float4 dq = *reinterpret_cast<const float4*>(xd + (mt * nb + b + 1) * 16 + 4 * lg);
            A.xe[mi][0] = de.x; A.xe[mi][1] = de.y; A.xe[mi][2] = de.z; A.xe[mi][3] = de.w;
            A.xo[mi][0] = dq.x; A.xo[mi][1] = dq.y; A.xo[mi][2] = dq.z; A.xo[mi][3] = dq.w;
        }
    };

    float acc[MW][NW][4];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ni = 0; ni < NW; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][ni][r] = 0.0f;

    // block pair jp of the chunk in LDS (blocks b, b + 1 of the row), activations from A
    auto mul_pair = [&](int jp, const AFrag& A, int64_t b) {
        const int je = 2 * jp, jo = 2 * jp + 1;
#pragma unroll
        for (int ni = 0; ni < NW; ++ni) {
            const int r = (wn * NW + ni) * 16 + li;
            const uint2 be2 = *reinterpret_cast<const uint2*>(bq + je * kBlockStride + lg * kGroupStride + 2 * r);
            const uint2 bo2 = *reinterpret_cast<const uint2*>(bq + jo * kBlockStride + lg * kGroupStride + 2 * r);
            const float se = bs[je * TN + r];
            const float so = bs[jo * TN + r];
            const uint64_t be = static_cast<uint64_t>(be2.x) | (static_cast<uint64_t>(be2.y) << 32);
            const uint64_t bo = static_cast<uint64_t>(bo2.x) | (static_cast<uint64_t>(bo2.y) << 32);
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
                const v4i zero = {0, 0, 0, 0};
                const v4i De = __builtin_amdgcn_mfma_i32_16x16x32_i8(static_cast<long>(A.e[mi]), static_cast<long>(be),
                                                                      zero, 0, 0, 0);
                const v4i Do = __builtin_amdgcn_mfma_i32_16x16x32_i8(static_cast<long>(A.o[mi]), static_cast<long>(bo),
                                                                      zero, 0, 0, 0);
                if constexpr (MODE == kModeISum) {
                    const int n = n0 + r;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t m = (tm * (MW * WM) + wm * MW + mi) * 16 + 4 * lg + q;
                        if (m < M && n >= isn0 && n < isn1) {
                            int32_t* dst = isum + (m * (isn1 - isn0) + (n - isn0)) * nb + b;
                            dst[0] = De[q] >> 4;
                            dst[1] = Do[q] >> 4;
                        }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[mi][ni][q] = fmaf(static_cast<float>(De[q]), se * A.xe[mi][q], acc[mi][ni][q]);
                        acc[mi][ni][q] = fmaf(static_cast<float>(Do[q]), so * A.xo[mi][q], acc[mi][ni][q]);
                    }
                }
            }
        }
    };

    AFrag A0, A1;
    load_a(0, A0);
    fetch(0);
    for (int c0 = 0; c0 < nb; c0 += KC) {
        __syncthreads();  // every wave is done with the previous chunk
        stash();
        __syncthreads();
        if (c0 + KC < nb) fetch(c0 + KC);
        const int npair = min(KC, nb - c0) >> 1;  // 4 or 8: even
        for (int jp = 0; jp < npair; jp += 2) {
            load_a(c0 + 2 * jp + 2, A1);
            mul_pair(jp, A0, c0 + 2 * jp);
            const int64_t nxt = c0 + 2 * jp + 4;
            load_a(nxt < nb ? nxt : nb - 2, A0);
            mul_pair(jp + 1, A1, c0 + 2 * jp + 2);
        }
    }
    if constexpr (MODE == kModeY) {
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int ni = 0; ni < NW; ++ni) {
                const int n = n0 + (wn * NW + ni) * 16 + li;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t m = (tm * (MW * WM) + wm * MW + mi) * 16 + 4 * lg + q;
                    if (m < M && n < N) out[m * N + n] = acc[mi][ni][q];
                }
            }
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

// The two MFMA tilings: wide (64 x 64 per workgroup, 32 x 32 per wave) and
// narrow (16 x 16 per workgroup, the four waves splitting K).
#define QMM_WIDE 2, 2, 2, 2, 1, 32
#define QMM_NARROW 1, 1, 1, 1, 4, 128
constexpr int kWideTM = 64, kWideTN = 64, kNarrowTM = 16, kNarrowTN = 16;

enum QmmPath : int { kPathDot = 0, kPathGeneric = 1, kPathWide = 2, kPathNarrow = 3 };

// Everything about a call that depends only on (N, K, M): kernels, tiles,
// K splits and the workspace parts, so that the workspace size and the
// launches always agree.
struct QmmPlan {
    int path = kPathGeneric;
    int64_t tiles_m = 0;
    int tiles_n = 0, ks = 1, kb = 0;
    int64_t xrows = 0;  // activation rows in the workspace (padded to the tile height)
    size_t q_bytes = 0, d_bytes = 0, p_bytes = 0;
};

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
    p.d_bytes = align256(static_cast<size_t>(p.xrows) * static_cast<size_t>(nb) * sizeof(float));
    p.p_bytes = p.ks > 1 ? align256(static_cast<size_t>(p.ks) * static_cast<size_t>(M) * static_cast<size_t>(N) *
                                    sizeof(float))
                         : 0;
    return p;
}

template <bool FRAG>
hipError_t launch_quantize(const float* x, int8_t* q, float* d, int64_t K, int64_t M, int64_t Mrows,
                           hipStream_t stream) {
    const int64_t groups = Mrows * (K / 32);
    int64_t blocks = ceil_div(groups * 8, kBlockThreads);
    const int64_t cap = static_cast<int64_t>(device_cus()) * 64;
    if (blocks > cap) blocks = cap;
    const bool vec_x = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    const bool vec_q = (reinterpret_cast<uintptr_t>(q) & 3) == 0;
    hipLaunchKernelGGL((quantize_q8_kernel<FRAG>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0,
                       stream, x, q, d, K, M, Mrows, vec_x, vec_q);
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
// keep the grid within 2^30 workgroups.
template <int MODE>
hipError_t launch_wide(const QmmPlan& p, const void* W, const int8_t* xa, const float* xd, float* y,
                       int32_t* isum, int64_t isn0, int64_t isn1, int64_t N, int64_t K, int64_t M,
                       hipStream_t stream) {
    int64_t mt_slice = (int64_t{1} << 30) / p.tiles_n;
    mt_slice = mt_slice < p.tiles_m ? mt_slice : p.tiles_m;
    for (int64_t tm0 = 0; tm0 < p.tiles_m; tm0 += mt_slice) {
        const int64_t tms = (p.tiles_m - tm0 < mt_slice) ? p.tiles_m - tm0 : mt_slice;
        const int64_t nwg = tms * p.tiles_n;
        hipLaunchKernelGGL((qmm_wide_kernel<16, MODE>), dim3(static_cast<unsigned>(nwg)), dim3(kBlockThreads), 0,
                           stream, static_cast<const uint8_t*>(W), xa, xd, y, isum, static_cast<int>(N), M,
                           static_cast<int>(K / 32), tm0, tms, p.tiles_n, nwg, static_cast<int>(isn0),
                           static_cast<int>(isn1));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
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
    return launch_quantize<false>(x, q, d, K, M, M, stream);
}

hipError_t launch_qmm_q8act(const void* W, const float* x, float* y, int32_t* isum, int64_t isn0, int64_t isn1,
                            int64_t N, int64_t K, int64_t M, void* ws, hipStream_t stream) {
    const QmmPlan p = plan_qmm(N, K, M);
    int8_t* q = static_cast<int8_t*>(ws);
    float* d = reinterpret_cast<float*>(static_cast<char*>(ws) + p.q_bytes);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.q_bytes + p.d_bytes);
    const bool mfma = p.path == kPathWide || p.path == kPathNarrow;
    hipError_t e = mfma ? launch_quantize<true>(x, q, d, K, M, p.xrows, stream)
                        : launch_quantize<false>(x, q, d, K, M, M, stream);
    if (e != hipSuccess) return e;
    if (!mfma) return launch_dot(p, W, q, d, isum ? nullptr : y, isum, isn0, isn1, N, K, M, stream);
    if (p.path == kPathWide) {
        return isum ? launch_wide<kModeISum>(p, W, q, d, nullptr, isum, isn0, isn1, N, K, M, stream)
                    : launch_wide<kModeY>(p, W, q, d, y, nullptr, 0, 0, N, K, M, stream);
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
