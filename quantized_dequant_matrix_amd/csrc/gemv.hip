// Fused-dequant matrix-vector kernels for Q4_0, Q8_0, Q4_K and Q6_K weights
// with float32 activations and float32 accumulation, and the gated GELU pair.
//
// What is computed: y[n] = sum_k w[n][k] x[k] with w decoded from the block
// formats on the fly ["Gemma 4 M4 Max kernel roadmap", K2 step 1: direct
// Q4_0 matrix-vector with fused dequantization and F32 accumulation; step 5:
// gated GELU FFN projection pair; "Metal kernel capability table", section 1
// (q4_f32_matvec, q4k_matvec, q6k_matvec) and section 4 (q4k_ffn_gate_up:
// both matrices in one dispatch)].
//
// The pages' Metal kernels give each SIMD group four or eight rows with
// threadgroup staging.  On gfx950 the layout is chosen for wave64 and HBM
// instead:
//   * A lane owns one 256-weight "unit" (8 blocks, 144 B or 272 B) of a row,
//     streamed with 16-byte loads; every block sits at a compile-time byte
//     offset inside the unit, so no per-lane realignment logic is needed.
//   * The L = K/256 lanes that own the units of one row form a segment; a
//     wave holds S = 64/L segments (3 rows at K = 5376, 4 at K = 4096), so
//     every load instruction moves whole rows and nearly all lanes work.
//   * The activation vector is staged once per workgroup in LDS, padded per
//     unit so that the lanes of a segment hit different banks; each lane
//     reuses the 32 values of a block for R rows.
//   * Each row's partial sums are reduced across its segment with cross-lane
//     shuffles.
// Codes are turned into exact signed values before multiplying:
//   Q4_0: (q - 8) * 16 as a signed byte, from (b ^ 0x88) & 0xF0, then one
//         byte-select convert per weight; the factor 16 is folded into d.
//   Q8_0: the signed code byte is converted directly.
//   Q4_K: w = fma(d*scale, q, -dmin*min) per weight, exact up to one rounding.
//   Q6_K: 4 (q - 32) as a signed byte, built from the nibble and the two high
//         bits with shifts and one mask-merge per 4 weights, then one
//         byte-select convert per weight; each 16-weight partial sum is
//         scaled by d*scale (exact) and the row sum by 1/4 (exact).
// So every product carries at most the rounding of float32 arithmetic on
// the exact weight, and the float32 sums stay within 1e-5 * sum|w x|.
#include <utility>

#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
        (fn(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- Q4_0
// Block k (0..7) of a 144-byte unit U[36]: fp16 d at byte 18k, codes at
// bytes 18k+2 .. 18k+17.  Returns d * sum_j 16 (q_j - 8) x_j (16x the block's
// contribution; the caller scales the row sum by 1/16, exactly).
template <int k>
__device__ __forceinline__ float q4_0_block_dot(const uint32_t* U, const float* xk) {
    constexpr int b0 = 18 * k;
    constexpr int dwd = b0 >> 2;
    const uint32_t dbits = ((b0 & 3) == 2) ? (U[dwd] >> 16) : (U[dwd] & 0xffffu);
    const float d = half_bits_to_float(dbits);  // the factor 1/16 is applied once per row
    constexpr int qb = b0 + 2;
    uint32_t qs[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if constexpr ((qb & 3) == 0) {
            qs[t] = U[(qb >> 2) + t];
        } else {
            qs[t] = shift16(U[(qb >> 2) + t + 1], U[(qb >> 2) + t]);
        }
    }
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // 16 (q - 8) as signed bytes: flip the code's top bit, keep the
        // nibble in the high half of each byte (one bitop3 each on gfx950)
        const uint32_t hi = (qs[t] ^ 0x88888888u) & 0xF0F0F0F0u;          // elements 16+4t+i
        const uint32_t lo = ((qs[t] << 4) ^ 0x88888880u) & 0xF0F0F0F0u;   // elements 4t+i
        s0 = fmaf(sbyte<0>(lo), xk[4 * t + 0], s0);
        s1 = fmaf(sbyte<1>(lo), xk[4 * t + 1], s1);
        s0 = fmaf(sbyte<2>(lo), xk[4 * t + 2], s0);
        s1 = fmaf(sbyte<3>(lo), xk[4 * t + 3], s1);
        s0 = fmaf(sbyte<0>(hi), xk[16 + 4 * t + 0], s0);
        s1 = fmaf(sbyte<1>(hi), xk[16 + 4 * t + 1], s1);
        s0 = fmaf(sbyte<2>(hi), xk[16 + 4 * t + 2], s0);
        s1 = fmaf(sbyte<3>(hi), xk[16 + 4 * t + 3], s1);
    }
    return d * (s0 + s1);
}

// ---------------------------------------------------------------- Q8_0
// Block k (0..7) of a 272-byte unit U[68]: fp16 d at byte 34k, int8 codes at
// bytes 34k+2 .. 34k+33 (read in place with byte selects).
template <int k>
__device__ __forceinline__ float q8_0_block_dot(const uint32_t* U, const float* xk) {
    constexpr int b0 = 34 * k;
    constexpr int dwd = b0 >> 2;
    const uint32_t dbits = ((b0 & 3) == 2) ? (U[dwd] >> 16) : (U[dwd] & 0xffffu);
    const float d = half_bits_to_float(dbits);
    float s[2] = {0.f, 0.f};
    static_for<32>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int pos = b0 + 2 + e;
        s[e & 1] = fmaf(sbyte<pos & 3>(U[pos >> 2]), xk[e], s[e & 1]);
    });
    return d * (s[0] + s[1]);
}

// ---------------------------------------------------------------- Q4_K
// Sub-block j (0..7) of a 144-byte super-block U[36]: d, dmin in dword 0,
// 6-bit scales/mins in bytes 4..15, codes of sub-blocks 2c, 2c+1 in the low
// and high nibbles of bytes 16+32c .. 16+32c+31.
template <int j>
__device__ __forceinline__ float q4_k_sub_dot(const uint32_t* U, const float* xk) {
    auto P = [&](int i) -> uint32_t { return (U[1 + (i >> 2)] >> (8 * (i & 3))) & 0xffu; };
    uint32_t sc, mn;
    if constexpr (j < 4) {
        sc = P(j) & 63u;
        mn = P(j + 4) & 63u;
    } else {
        sc = (P(j + 4) & 15u) | ((P(j - 4) >> 6) << 4);
        mn = (P(j + 4) >> 4) | ((P(j) >> 6) << 4);
    }
    const float a = half_bits_to_float(U[0] & 0xffffu) * static_cast<float>(sc);  // exact
    const float nb = -(half_bits_to_float(U[0] >> 16) * static_cast<float>(mn));  // exact
    constexpr int c = j >> 1;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t raw = U[4 + 8 * c + t];
        const uint32_t q = (j & 1) ? ((raw >> 4) & 0x0F0F0F0Fu) : (raw & 0x0F0F0F0Fu);
        s0 = fmaf(fmaf(a, ubyte<0>(q), nb), xk[4 * t + 0], s0);
        s1 = fmaf(fmaf(a, ubyte<1>(q), nb), xk[4 * t + 1], s1);
        s0 = fmaf(fmaf(a, ubyte<2>(q), nb), xk[4 * t + 2], s0);
        s1 = fmaf(fmaf(a, ubyte<3>(q), nb), xk[4 * t + 3], s1);
    }
    return s0 + s1;
}

// ---------------------------------------------------------------- Q6_K
// Block k (0..7) of a realigned Q6_K super-block U[54]: the 32 weights
// 32k .. 32k+31, i.e. half h = k/4, group g = k%4.  ql in dwords 0..31, qh
// in 32..47, int8 scales in 48..51, fp16 d in U[53].  Element
// 128h + 32g + l takes the low (g < 2) or high (g >= 2) nibble of ql byte
// 64h + 32(g%2) + l and bits 2g, 2g+1 of qh byte 32h + l.  The byte
//   ((nibble << 2) | (high bits << 6)) ^ 0x80
// is 4 (q - 32) as a signed byte.  Returns 4x the block's contribution.
template <int k>
__device__ __forceinline__ float q6_k_block_dot(const uint32_t* U, const float* xk) {
    constexpr int h = k >> 2;
    constexpr int g = k & 3;
    const float d = half_bits_to_float(U[53]);
    float s[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t L = U[16 * h + 8 * (g & 1) + t];
        const uint32_t H = U[32 + 8 * h + t];
        const uint32_t nib = (g < 2) ? (L << 2) : (L >> 2);                 // nibble -> bits 2..5
        const uint32_t hb = (g == 0) ? (H << 6) : (g == 1) ? (H << 4) : (g == 2) ? (H << 2) : H;  // -> bits 6, 7
        const uint32_t b = ((nib & 0x3C3C3C3Cu) | (hb & 0xC0C0C0C0u)) ^ 0x80808080u;
        float* sp = s[t >> 2];
        sp[0] = fmaf(sbyte<0>(b), xk[4 * t + 0], sp[0]);
        sp[1] = fmaf(sbyte<1>(b), xk[4 * t + 1], sp[1]);
        sp[0] = fmaf(sbyte<2>(b), xk[4 * t + 2], sp[0]);
        sp[1] = fmaf(sbyte<3>(b), xk[4 * t + 3], sp[1]);
    }
    // sub-blocks 8h + 2g and 8h + 2g + 1: scale bytes 2g, 2g+1 (mod 4) of
    // dword 48 + 2h + g/2
    const uint32_t scw = U[48 + 2 * h + (g >> 1)];
    const float a0 = d * sbyte<(2 * g) & 3>(scw);        // exact
    const float a1 = d * sbyte<((2 * g) & 3) + 1>(scw);  // exact
    return fmaf(a1, s[1][0] + s[1][1], a0 * (s[0][0] + s[0][1]));
}

// Q6_K words as loaded -- U[0..51] = super-block bytes [sh, sh + 208),
// U[52] = the 16-bit rest (bytes 208-209 if sh = 0, bytes 0-1 if sh = 2) --
// become the super-block's own dwords 0..51 and d in U[53].  One v_perm_b32
// per dword with a per-lane selector: bytes 4-7 of {U[i], U[i-1]} (U[i]
// itself) when sh = 0, bytes 2-5 when sh = 2.
__device__ __forceinline__ void q6_k_realign(uint32_t* U, uint32_t sh) {
    const uint32_t sel = sh ? 0x05040302u : 0x07060504u;
    U[53] = sh ? (U[51] >> 16) : U[52];
#pragma unroll
    for (int i = 51; i > 0; --i) U[i] = __builtin_amdgcn_perm(U[i], U[i - 1], sel);
    U[0] = __builtin_amdgcn_perm(U[0], U[52] << 16, sel);
}

template <int F, int k>
__device__ __forceinline__ float unit_block_dot(const uint32_t* U, const float* xk) {
    if constexpr (F == kQ4_0) return q4_0_block_dot<k>(U, xk);
    else if constexpr (F == kQ8_0) return q8_0_block_dot<k>(U, xk);
    else if constexpr (F == kQ4_K) return q4_k_sub_dot<k>(U, xk);
    else return q6_k_block_dot<k>(U, xk);
}

// Factor that turns a row's sum of unit_block_dot results into y.
template <int F>
constexpr float kRowScale = (F == kQ4_0) ? 0.0625f : (F == kQ6_K ? 0.25f : 1.0f);

// Stage x[0..K) into LDS as G padded unit slices.  Each thread issues a batch
// of loads before the matching LDS writes (indices past the end are clamped
// to the last element, which is then written twice with the same value), so a
// workgroup waits for a couple of memory round trips, not one per element.
constexpr int kMaxUnits = 63;
__device__ __forceinline__ void stage_x(float* xs, const float* __restrict__ x, int G) {
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        constexpr int kPer = 4;  // 16-byte loads in flight per thread
        const int n4 = G * (kUnitElems / 4);
        for (int base = 0; base < n4; base += kPer * kBlockThreads) {
            float4 v[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = min(base + j * kBlockThreads + static_cast<int>(threadIdx.x), n4 - 1);
                v[j] = reinterpret_cast<const float4*>(x)[i];
            }
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = min(base + j * kBlockThreads + static_cast<int>(threadIdx.x), n4 - 1);
                *reinterpret_cast<float4*>(xs + (i >> 6) * kXsStride + (i & 63) * 4) = v[j];
            }
        }
    } else {
        // unaligned x: 4 scalar loads in flight per thread (few registers:
        // the weights of the first pass are already in flight)
        const int n = G * kUnitElems;
        for (int base = 0; base < n; base += 4 * kBlockThreads) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = x[min(base + j * kBlockThreads + static_cast<int>(threadIdx.x), n - 1)];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = min(base + j * kBlockThreads + static_cast<int>(threadIdx.x), n - 1);
                xs[(i >> 8) * kXsStride + (i & 255)] = v[j];
            }
        }
    }
}

// ------------------------------------------------------------ unit kernel
// K % 256 == 0 and G = K/256 <= 63.  Lane (segment s, unit u) of a wave
// handles unit u of R consecutive rows per pass; a pass covers S*R rows.
// PAIR: the same rows of two matrices (gate, up), output gelu(g) * u.
template <int F, int R, bool PAIR>
__global__ __launch_bounds__(kBlockThreads)
void gemv_unit_kernel(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                      const float* __restrict__ x, float* __restrict__ y,
                      int N, int G, int S, int npasses) {
    constexpr int VEC = UnitInfo<F>::kVec;
    constexpr int UB = UnitInfo<F>::kBytes;
    constexpr int NM = PAIR ? 2 : 1;
    extern __shared__ float xs[];

    const int lane = threadIdx.x & (kWave - 1);
    const int L = G;
    const int seg = lane / L;
    const int u = lane - seg * L;
    const bool active = seg < S;
    const int64_t row_bytes = static_cast<int64_t>(G) * UB;
    const int wave_stride = gridDim.x * kWavesPerBlock;
    int pass = blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);

    constexpr bool kQ6 = (F == kQ6_K);
    uint32_t U[NM * R][VEC * 4 + (kQ6 ? 2 : 0)];
    uint32_t sh[NM * R];  // Q6_K: byte offset of the super-block past its dword (0 or 2)
    auto load = [&](int p) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // Rows past the end (and lanes outside every segment) load the
            // last row again: valid memory, results never stored.
            int row = (p * S + seg) * R + r;
            row = row < N ? row : N - 1;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const uint8_t* base = (m == 0 ? W0 : W1) + row * row_bytes + u * UB;
                if constexpr (kQ6) {
                    // W is 16-byte aligned and super-blocks are 210 B, so a
                    // super-block starts 0 or 2 (= sh) bytes past a dword.
                    // Its bytes [sh, sh + 208) are 13 dword-aligned 16-byte
                    // pieces; the two bytes left over ([208, 210) when sh = 0,
                    // [0, 2) when sh = 2) come in one 16-bit load.  Every
                    // load stays inside the super-block.
                    const uint32_t o = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(base) & 2);
                    sh[m * R + r] = o;
                    const u32x4_a4* src = reinterpret_cast<const u32x4_a4*>(base + o);
#pragma unroll
                    for (int t = 0; t < VEC; ++t) {
                        const u32x4_a4 v = src[t];
                        U[m * R + r][4 * t + 0] = v.x;
                        U[m * R + r][4 * t + 1] = v.y;
                        U[m * R + r][4 * t + 2] = v.z;
                        U[m * R + r][4 * t + 3] = v.w;
                    }
                    U[m * R + r][52] = *reinterpret_cast<const uint16_t*>(base + (o ? 0 : 208));
                } else {
                    const uint4* src = reinterpret_cast<const uint4*>(base);
#pragma unroll
                    for (int t = 0; t < VEC; ++t) {
                        const uint4 v = src[t];
                        U[m * R + r][4 * t + 0] = v.x;
                        U[m * R + r][4 * t + 1] = v.y;
                        U[m * R + r][4 * t + 2] = v.z;
                        U[m * R + r][4 * t + 3] = v.w;
                    }
                }
            }
        }
    };

    // Start the weight stream before staging the activations.
    if (pass < npasses) load(pass);
    stage_x(xs, x, G);
    __syncthreads();

    while (pass < npasses) {
        // Re-derive the LDS pointer each pass so that the compiler does not
        // hoist the whole 1 KB activation slice into registers for the
        // lifetime of the loop (that would cap occupancy at one wave/SIMD).
        int xoff = u * kXsStride;
        asm volatile("" : "+v"(xoff));
        const float* xw = xs + xoff;
        float acc[NM * R];
#pragma unroll
        for (int i = 0; i < NM * R; ++i) acc[i] = 0.f;
        if constexpr (kQ6) {
#pragma unroll
            for (int i = 0; i < NM * R; ++i) q6_k_realign(U[i], sh[i]);
        }
        static_for<8>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            float xk[32];
            const float4* xv = reinterpret_cast<const float4*>(xw + 32 * k);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float4 v = xv[t];
                xk[4 * t + 0] = v.x;
                xk[4 * t + 1] = v.y;
                xk[4 * t + 2] = v.z;
                xk[4 * t + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < NM * R; ++i) {
                acc[i] += unit_block_dot<F, k>(U[i], xk);
                // Materialize the sum here: otherwise the compiler sinks the
                // work of later rows past earlier reductions and keeps every
                // block's activations live in registers.
                asm volatile("" : "+v"(acc[i]));
            }
        });
        const int row0 = (pass * S + seg) * R;
        constexpr float kScale = kRowScale<F>;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float v0 = segment_sum(acc[r], u, L) * kScale;
            if constexpr (PAIR) {
                float v1 = segment_sum(acc[R + r], u, L) * kScale;
                if (active && u == 0 && row0 + r < N) y[row0 + r] = gelu_tanh(v0) * v1;
            } else {
                if (active && u == 0 && row0 + r < N) y[row0 + r] = v0;
            }
        }
        pass += wave_stride;
        if (pass < npasses) load(pass);
    }
}

// --------------------------------------------------------- generic kernel
// Any K % 32 == 0 (K % 256 == 0 for Q4_K and Q6_K).  One wave per row, lanes
// stride over the row's blocks, activations read from global memory.  Rows
// need not be 16-byte aligned; Q4_0 / Q8_0 / Q6_K blocks are read with
// 16-bit loads.
template <int F>
__device__ __forceinline__ float generic_block_dot(const uint8_t* __restrict__ row, int64_t b,
                                                   const float* __restrict__ x) {
    if constexpr (F == kQ4_0) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row + 18 * b);
        const float d = half_bits_to_float(p[0]);
        const float* xb = x + 32 * b;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const uint32_t two = p[1 + h];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int byte = (two >> (8 * i)) & 0xff;
                s = fmaf(static_cast<float>((byte & 15) - 8), xb[2 * h + i], s);
                s = fmaf(static_cast<float>((byte >> 4) - 8), xb[16 + 2 * h + i], s);
            }
        }
        return d * s;
    } else if constexpr (F == kQ8_0) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row + 34 * b);
        const float d = half_bits_to_float(p[0]);
        const float* xb = x + 32 * b;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            const uint32_t two = p[1 + h];
            s = fmaf(static_cast<float>(static_cast<int8_t>(two & 0xff)), xb[2 * h], s);
            s = fmaf(static_cast<float>(static_cast<int8_t>(two >> 8)), xb[2 * h + 1], s);
        }
        return d * s;
    } else if constexpr (F == kQ6_K) {
        // 2-byte aligned super-block: 16-bit loads
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row + 210 * b);
        uint32_t U[54];
#pragma unroll
        for (int i = 0; i < 52; ++i) U[i] = static_cast<uint32_t>(p[2 * i]) | (static_cast<uint32_t>(p[2 * i + 1]) << 16);
        U[53] = p[104];
        const float* xb = x + 256 * b;
        float s = 0.f;
        static_for<8>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            s += q6_k_block_dot<k>(U, xb + 32 * k);
        });
        return 0.25f * s;
    } else {
        const uint4* src = reinterpret_cast<const uint4*>(row + 144 * b);
        uint32_t U[36];
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const uint4 v = src[t];
            U[4 * t] = v.x; U[4 * t + 1] = v.y; U[4 * t + 2] = v.z; U[4 * t + 3] = v.w;
        }
        const float* xb = x + 256 * b;
        float s = 0.f;
        static_for<8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            s += q4_k_sub_dot<j>(U, xb + 32 * j);
        });
        return s;
    }
}

template <int F, bool PAIR>
__global__ __launch_bounds__(kBlockThreads)
void gemv_generic_kernel(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                         const float* __restrict__ x, float* __restrict__ y,
                         int N, int64_t nblocks, int64_t row_bytes) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_stride = gridDim.x * kWavesPerBlock;
    for (int row = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < N; row += wave_stride) {
        float a0 = 0.f, a1 = 0.f;
        for (int64_t b = lane; b < nblocks; b += kWave) {
            a0 += generic_block_dot<F>(W0 + row * row_bytes, b, x);
            if constexpr (PAIR) a1 += generic_block_dot<F>(W1 + row * row_bytes, b, x);
        }
        a0 = wave_sum(a0);
        if constexpr (PAIR) a1 = wave_sum(a1);
        if (lane == 0) {
            if constexpr (PAIR) y[row] = gelu_tanh(a0) * a1;
            else y[row] = a0;
        }
    }
}

template <int F, int R, bool PAIR>
hipError_t launch_unit(const void* W0, const void* W1, const float* x, float* y, int N, int G,
                       hipStream_t stream) {
    const int S = kWave / G;
    const int rows_per_pass = S * R;
    const int npasses = (N + rows_per_pass - 1) / rows_per_pass;
    // At most as many workgroups as are resident at once (4 per CU at
    // <= 128 VGPRs); longer matrices take several passes per wave.  One
    // matrix at a time runs best with 3 per CU: a wave's first loads then
    // share the memory system with fewer others and arrive sooner.
    const int max_blocks = device_cus() * (PAIR ? 4 : 3);
    int blocks = (npasses + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    const size_t lds = static_cast<size_t>(G) * kXsStride * sizeof(float);
    hipLaunchKernelGGL((gemv_unit_kernel<F, R, PAIR>), dim3(blocks), dim3(kBlockThreads), lds, stream,
                       static_cast<const uint8_t*>(W0), static_cast<const uint8_t*>(W1), x, y,
                       N, G, S, npasses);
    return hipGetLastError();
}

template <int F, bool PAIR>
hipError_t launch_generic(const void* W0, const void* W1, const float* x, float* y, int N, int64_t K,
                          hipStream_t stream) {
    const int64_t per = (F == kQ4_K || F == kQ6_K) ? 256 : 32;
    const int64_t bytes = (F == kQ4_0) ? 18 : (F == kQ8_0 ? 34 : (F == kQ4_K ? 144 : 210));
    const int64_t nb = K / per;
    const int max_blocks = device_cus() * 8;
    int blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL((gemv_generic_kernel<F, PAIR>), dim3(blocks), dim3(kBlockThreads), 0, stream,
                       static_cast<const uint8_t*>(W0), static_cast<const uint8_t*>(W1), x, y,
                       N, nb, nb * bytes);
    return hipGetLastError();
}

}  // namespace

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Largest K the unit kernels take: the padded activation slices must fit in
// 64 KiB of LDS per workgroup (63 units = 65,520 B).
constexpr int64_t kUnitMaxG = kMaxUnits;

hipError_t launch_gemv(int fmt, const void* W, const void* W_up, const float* x, float* y,
                       int64_t N64, int64_t K, hipStream_t stream) {
    const int N = static_cast<int>(N64);
    const bool unit = (K % kUnitElems == 0) && (K / kUnitElems <= kUnitMaxG);
    const int G = static_cast<int>(K / kUnitElems);
    if (W_up != nullptr) {
        return unit ? launch_unit<kQ4_0, 1, true>(W, W_up, x, y, N, G, stream)
                    : launch_generic<kQ4_0, true>(W, W_up, x, y, N, K, stream);
    }
    switch (fmt) {
    case kQ4_0:
        return unit ? launch_unit<kQ4_0, 1, false>(W, nullptr, x, y, N, G, stream)
                    : launch_generic<kQ4_0, false>(W, nullptr, x, y, N, K, stream);
    case kQ8_0:
        return unit ? launch_unit<kQ8_0, 1, false>(W, nullptr, x, y, N, G, stream)
                    : launch_generic<kQ8_0, false>(W, nullptr, x, y, N, K, stream);
    case kQ4_K:
        return unit ? launch_unit<kQ4_K, 1, false>(W, nullptr, x, y, N, G, stream)
                    : launch_generic<kQ4_K, false>(W, nullptr, x, y, N, K, stream);
    default:
        return unit ? launch_unit<kQ6_K, 1, false>(W, nullptr, x, y, N, G, stream)
                    : launch_generic<kQ6_K, false>(W, nullptr, x, y, N, K, stream);
    }
}

}  // namespace qmv
