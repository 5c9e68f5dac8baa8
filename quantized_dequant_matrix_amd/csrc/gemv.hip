// Fused-dequant matrix-vector kernels for Q4_0, Q8_0, Q4_K, Q6_K and MXFP4
// weights with float32 activations and float32 accumulation, and the gated
// GELU pair.
//
// What is computed: y[n] = sum_k w[n][k] x[k] with w decoded from the block
// formats on the fly ["Gemma 4 M4 Max kernel roadmap", K2 step 1: a Q4_0
// matrix-vector product whose dot product decodes the blocks itself and sums
// in float32; step 5: the FFN's gate and up projections; "Metal kernel
// capability table", section 1
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
//   MXFP4: gfx950's packed FP4 conversion (v_cvt_scalef32_pk_f32_fp4) turns
//         one code byte into its two float32 values (exact) -- one op per
//         two weights -- then one FMA per weight; each 32-weight sum is
//         multiplied by its E8M0 scale 2^(e - 127) (exact, power of two).
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
        uint32_t q = (j & 1) ? ((raw >> 4) & 0x0F0F0F0Fu) : (raw & 0x0F0F0F0Fu);
        // Keep the nibble mask opaque: otherwise the compiler folds it into
        // each byte's shift and extracts bytes 1 and 2 with a bit-field
        // extract plus a byte-0 convert, instead of one v_cvt_f32_ubyteN
        // per weight (13% more VALU work, about 5% of the launch).
        asm("" : "+v"(q));
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

// ---------------------------------------------------------------- MXFP4
// Block k (0..7) of an MXFP4 unit U[34]: code dwords 4k .. 4k+3 (element 2i
// in the low and 2i+1 in the high nibble of code byte i), E8M0 scale bytes
// in U[32], U[33].  The conversion runs at scale 1.0 (exponent 127, i.e.
// 2^0); the block's own scale multiplies the block sum.
typedef float v2f_t __attribute__((ext_vector_type(2)));

// E8M0 exponent byte -> float32 2^(e - 127): e = 0 is 2^-127 (a float32
// subnormal), e = 255 is NaN.
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
    const uint32_t bits = (e == 0) ? 0x00400000u : (e == 255 ? 0x7FC00000u : (e << 23));
    return __builtin_bit_cast(float, bits);
}

template <int k>
__device__ __forceinline__ float mxfp4_block_dot(const uint32_t* U, const float* xk) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t c = U[4 * k + t];
        const v2f_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
        const v2f_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
        const v2f_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
        const v2f_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
        s0 = fmaf(p0[0], xk[8 * t + 0], s0);
        s1 = fmaf(p0[1], xk[8 * t + 1], s1);
        s0 = fmaf(p1[0], xk[8 * t + 2], s0);
        s1 = fmaf(p1[1], xk[8 * t + 3], s1);
        s0 = fmaf(p2[0], xk[8 * t + 4], s0);
        s1 = fmaf(p2[1], xk[8 * t + 5], s1);
        s0 = fmaf(p3[0], xk[8 * t + 6], s0);
        s1 = fmaf(p3[1], xk[8 * t + 7], s1);
    }
    const uint32_t e = (U[32 + (k >> 2)] >> (8 * (k & 3))) & 0xffu;
    return (s0 + s1) * e8m0_to_float(e);
}

template <int F, int k>
__device__ __forceinline__ float unit_block_dot(const uint32_t* U, const float* xk) {
    if constexpr (F == kQ4_0) return q4_0_block_dot<k>(U, xk);
    else if constexpr (F == kQ8_0) return q8_0_block_dot<k>(U, xk);
    else if constexpr (F == kQ4_K) return q4_k_sub_dot<k>(U, xk);
    else if constexpr (F == kQ6_K) return q6_k_block_dot<k>(U, xk);
    else return mxfp4_block_dot<k>(U, xk);
}

// Factor that turns a row's sum of unit_block_dot results into y.
template <int F>
constexpr float kRowScale = (F == kQ4_0) ? 0.0625f : (F == kQ6_K ? 0.25f : 1.0f);

// Stage the activations into LDS as G padded unit slices: x[0..K), or, for
// the down projection of a gated FFN (GIN), gelu(x[k]) * xu[k] formed here
// in float32.  Each thread issues a batch of loads before the matching LDS
// writes (indices past the end are clamped to the last element, which is
// then written twice with the same value), so a workgroup waits for a couple
// of memory round trips, not one per element.
constexpr int kMaxUnits = 63;

template <bool GIN>
__device__ __forceinline__ float staged_value(float a, float b) {
    if constexpr (GIN) return gelu_tanh(a) * b;
    else return a;
}

// NT: the workgroup's thread count (every thread of the workgroup calls this).
template <bool GIN>
__device__ __forceinline__ void stage_x(float* xs, const float* __restrict__ x, const float* __restrict__ xu, int G,
                                        const int NT) {
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | (GIN ? reinterpret_cast<uintptr_t>(xu) : 0)) & 15) == 0;
    if (vec) {
        constexpr int kPer = GIN ? 2 : 4;  // 16-byte loads in flight per thread (per input)
        const int n4 = G * (kUnitElems / 4);
        for (int base = 0; base < n4; base += kPer * NT) {
            float4 v[kPer], w[GIN ? kPer : 1];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = min(base + j * NT + static_cast<int>(threadIdx.x), n4 - 1);
                v[j] = reinterpret_cast<const float4*>(x)[i];
                if constexpr (GIN) w[j] = reinterpret_cast<const float4*>(xu)[i];
            }
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = min(base + j * NT + static_cast<int>(threadIdx.x), n4 - 1);
                if constexpr (GIN) {
                    v[j].x = staged_value<true>(v[j].x, w[j].x);
                    v[j].y = staged_value<true>(v[j].y, w[j].y);
                    v[j].z = staged_value<true>(v[j].z, w[j].z);
                    v[j].w = staged_value<true>(v[j].w, w[j].w);
                }
                *reinterpret_cast<float4*>(xs + (i >> 6) * kXsStride + (i & 63) * 4) = v[j];
            }
        }
    } else {
        // unaligned activations: 4 scalar loads in flight per thread and
        // input (few registers: the weights of the first pass are already
        // in flight)
        const int n = G * kUnitElems;
        for (int base = 0; base < n; base += 4 * NT) {
            float v[4], w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = min(base + j * NT + static_cast<int>(threadIdx.x), n - 1);
                v[j] = x[i];
                w[j] = GIN ? xu[i] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = min(base + j * NT + static_cast<int>(threadIdx.x), n - 1);
                xs[(i >> 8) * kXsStride + (i & 255)] = staged_value<GIN>(v[j], w[j]);
            }
        }
    }
}

// One lane's 256-weight unit at base: UnitInfo<F>::kVec 16-byte loads into
// U (and, for Q6_K, the 16-bit rest into U[52] and the super-block's offset
// past its dword into sh; q6_k_realign then puts the words in place).
// sbase: MXFP4 only, the unit's 8 scale bytes in the scale plane.
template <int F>
__device__ __forceinline__ void load_unit(uint32_t* U, uint32_t& sh, const uint8_t* base,
                                          const uint8_t* sbase = nullptr) {
    constexpr int VEC = UnitInfo<F>::kVec;
    if constexpr (F == kQ6_K) {
        // W is 16-byte aligned and super-blocks are 210 B, so a super-block
        // starts 0 or 2 (= sh) bytes past a dword.  Its bytes [sh, sh + 208)
        // are 13 dword-aligned 16-byte pieces; the two bytes left over
        // ([208, 210) when sh = 0, [0, 2) when sh = 2) come in one 16-bit
        // load.  Every load stays inside the super-block.
        const uint32_t o = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(base) & 2);
        sh = o;
        const u32x4_a4* src = reinterpret_cast<const u32x4_a4*>(base + o);
#pragma unroll
        for (int t = 0; t < VEC; ++t) {
            const u32x4_a4 v = src[t];
            U[4 * t + 0] = v.x;
            U[4 * t + 1] = v.y;
            U[4 * t + 2] = v.z;
            U[4 * t + 3] = v.w;
        }
        U[52] = *reinterpret_cast<const uint16_t*>(base + (o ? 0 : 208));
    } else {
        sh = 0;
        const uint4* src = reinterpret_cast<const uint4*>(base);
#pragma unroll
        for (int t = 0; t < VEC; ++t) {
            const uint4 v = src[t];
            U[4 * t + 0] = v.x;
            U[4 * t + 1] = v.y;
            U[4 * t + 2] = v.z;
            U[4 * t + 3] = v.w;
        }
        if constexpr (F == kMXFP4) {
            const uint2 sc = *reinterpret_cast<const uint2*>(sbase);
            U[32] = sc.x;
            U[33] = sc.y;
        }
    }
}

template <int F>
constexpr int kUnitWords = UnitInfo<F>::kVec * 4 + ((F == kQ6_K || F == kMXFP4) ? 2 : 0);

// Bytes of a unit's scales in a separate scale plane (MXFP4), else 0.
template <int F>
constexpr int kUnitScaleBytes = (F == kMXFP4) ? 8 : 0;

// acc[i] = the sum over unit i's 256 weights of (decoded weight) * x, for NR
// units held in U that share the activation slice xw (LDS), times the
// format's 1/kRowScale.
template <int F, int NR, int UW>
__device__ __forceinline__ void dot_units(uint32_t (&U)[NR][UW], const uint32_t (&sh)[NR],
                                          const float* xw, float (&acc)[NR]) {
    static_assert(UW >= kUnitWords<F>, "unit words");
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = 0.f;
    if constexpr (F == kQ6_K) {
#pragma unroll
        for (int i = 0; i < NR; ++i) q6_k_realign(U[i], sh[i]);
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
        for (int i = 0; i < NR; ++i) {
            acc[i] += unit_block_dot<F, k>(U[i], xk);
            // Materialize the sum here: otherwise the compiler sinks the
            // work of later units past earlier reductions and keeps every
            // block's activations live in registers.
            asm volatile("" : "+v"(acc[i]));
        }
    });
}

// ------------------------------------------------------------ unit kernel
// K % 256 == 0 and G = K/256 <= 63.  Lane (segment s, unit u) of a wave
// handles unit u of R consecutive rows per pass; a pass covers S*R rows.
// PAIR: the same rows of two matrices (gate, up), output gelu(g) * u.
//
// Occupancy the compiler schedules for: 5 waves per SIMD for one Q4_0
// matrix (its schedule at 72 VGPRs runs about 3% faster than the one at the
// default budget), the default elsewhere (the pair would spill, and Q8_0
// runs slower).
template <int F, bool PAIR, bool GIN>
constexpr int kUnitWavesPerSimd = (F == kQ4_0 && !PAIR && !GIN) ? 5 : 0;

template <int F, int R, bool PAIR, bool GIN>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(kUnitWavesPerSimd<F, PAIR, GIN>)))
void gemv_unit_kernel(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                      const float* __restrict__ x, const float* __restrict__ xu, float* __restrict__ y,
                      int N, int G, int S, int npasses) {
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

    uint32_t U[NM * R][kUnitWords<F>];
    uint32_t sh[NM * R];  // Q6_K: byte offset of the super-block past its dword (0 or 2)
    auto load = [&](int p) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // Rows past the end (and lanes outside every segment) load the
            // last row again: valid memory, results never stored.
            int row = (p * S + seg) * R + r;
            row = row < N ? row : N - 1;
            if constexpr (F == kMXFP4) {
                // W0: code plane, W1: scale plane
                load_unit<F>(U[r], sh[r], W0 + row * row_bytes + u * UB,
                             W1 + static_cast<int64_t>(row) * G * kUnitScaleBytes<F> + u * kUnitScaleBytes<F>);
            } else {
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    load_unit<F>(U[m * R + r], sh[m * R + r], (m == 0 ? W0 : W1) + row * row_bytes + u * UB);
            }
        }
    };

    // Loads complete in issue order for the wait counter, so whichever of the
    // activation staging and the first pass's weights is requested second
    // waits for the other too.  Staging first lets the decode start as the
    // weights arrive; requesting the weights first starts the stream ~1 us
    // earlier.  Measured (event-timed, warm, alternating builds): staging
    // first was 3-10% faster for Q4_K, Q6_K and MXFP4, but 1.5% slower for
    // the Q4_0 benchmark step and 0.5-1.5% slower for Q8_0.
    constexpr bool kStageFirst = F == kQ4_K || F == kQ6_K || F == kMXFP4;
    if (!kStageFirst && pass < npasses) load(pass);
    stage_x<GIN>(xs, x, xu, G, kBlockThreads);
    if (kStageFirst && pass < npasses) load(pass);
    __syncthreads();

    while (pass < npasses) {
        // Re-derive the LDS pointer each pass so that the compiler does not
        // hoist the whole 1 KB activation slice into registers for the
        // lifetime of the loop (that would cap occupancy at one wave/SIMD).
        int xoff = u * kXsStride;
        asm volatile("" : "+v"(xoff));
        const float* xw = xs + xoff;
        float acc[NM * R];
        dot_units<F, NM * R>(U, sh, xw, acc);
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

// ------------------------------------------------------- three-matrix kernel
// Three matrices that share x and K (G = K/256 <= 63 units) in one launch:
// the attention input projections of a Q4_K_M model, Q and K rows in format
// FA and V rows in format FB.  The passes of the three matrices form one
// index space (V's first: its units are the largest, so the launch ends on
// the cheaper ones); a wave takes passes like the unit kernel and decodes
// with the format of the pass's matrix (a wave-uniform branch).
template <int FA, int FB>
__global__ __launch_bounds__(kBlockThreads)
void gemv_qkv_kernel(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Wk, const uint8_t* __restrict__ Wv,
                     const float* __restrict__ x, float* __restrict__ yq, float* __restrict__ yk,
                     float* __restrict__ yv, int Nq, int Nk, int Nv, int G, int S, int Pv, int Pq, int Pk) {
    constexpr int UWMAX = kUnitWords<FA> > kUnitWords<FB> ? kUnitWords<FA> : kUnitWords<FB>;
    extern __shared__ float xs[];
    const int lane = threadIdx.x & (kWave - 1);
    const int seg = lane / G;
    const int u = lane - seg * G;
    const bool active = seg < S;
    const int64_t rbA = static_cast<int64_t>(G) * UnitInfo<FA>::kBytes;
    const int64_t rbB = static_cast<int64_t>(G) * UnitInfo<FB>::kBytes;
    const int npasses = Pv + Pq + Pk;
    const int wave_stride = gridDim.x * kWavesPerBlock;
    int pass = blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);

    uint32_t U[1][UWMAX];
    uint32_t sh[1];
    auto load = [&](int p) {
        if (p < Pv) {
            int row = p * S + seg;
            row = row < Nv ? row : Nv - 1;
            load_unit<FB>(U[0], sh[0], Wv + row * rbB + u * UnitInfo<FB>::kBytes);
        } else {
            const bool isq = p < Pv + Pq;
            const int n = isq ? Nq : Nk;
            int row = (p - (isq ? Pv : Pv + Pq)) * S + seg;
            row = row < n ? row : n - 1;
            load_unit<FA>(U[0], sh[0], (isq ? Wq : Wk) + row * rbA + u * UnitInfo<FA>::kBytes);
        }
    };

    // activations first, as in the unit kernel's Q4_K / Q6_K launches (4% faster)
    stage_x<false>(xs, x, nullptr, G, kBlockThreads);
    if (pass < npasses) load(pass);
    __syncthreads();

    while (pass < npasses) {
        int xoff = u * kXsStride;
        asm volatile("" : "+v"(xoff));
        const float* xw = xs + xoff;
        float acc[1];
        float* yo;
        int n, row;
        float scale;
        if (pass < Pv) {
            dot_units<FB, 1>(U, sh, xw, acc);
            yo = yv;
            n = Nv;
            row = pass * S + seg;
            scale = kRowScale<FB>;
        } else {
            dot_units<FA, 1>(U, sh, xw, acc);
            const bool isq = pass < Pv + Pq;
            yo = isq ? yq : yk;
            n = isq ? Nq : Nk;
            row = (pass - (isq ? Pv : Pv + Pq)) * S + seg;
            scale = kRowScale<FA>;
        }
        const float v = segment_sum(acc[0], u, G) * scale;
        if (active && u == 0 && row < n) yo[row] = v;
        pass += wave_stride;
        if (pass < npasses) load(pass);
    }
}

// ----------------------------------------------------------- split kernel
// K % 256 == 0 and G = K/256 > 63: rows longer than a wave has lanes for one
// unit each (the FFN down projection, K = 21504, has G = 84).  Each row is
// cut into KS slices of Gs units; a "slot" is S rows x one slice, one unit
// per lane, exactly like a pass of the unit kernel on a short row.
//   * A workgroup stages all of x once (up to 160 KB of LDS) and owns a
//     contiguous range of row groups (S rows each); the ranges differ by at
//     most one group, so every CU streams the same number of bytes.
//   * Its waves take the range's slots in turn (slot = group * KS + slice)
//     with no barrier between slots; each wave requests its next slot's
//     weights as soon as the current ones are decoded.
//   * Slice sums go to LDS.  After one barrier per chunk of CH groups, the
//     KS slice sums of each row are added in slice order, so the result does
//     not depend on timing.
constexpr int kSplitThreads = 1024;

template <int F, bool GIN>
__global__ __launch_bounds__(kSplitThreads)
void gemv_split_kernel(const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, const float* __restrict__ x,
                       const float* __restrict__ xu, float* __restrict__ y, int N, int G, int KS, int Gs, int S,
                       int NG, int CH) {
    constexpr int UB = UnitInfo<F>::kBytes;
    extern __shared__ float xs[];
    float* red = xs + G * kXsStride;  // [CH][S][KS] slice sums of the current chunk

    const int nwaves = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int seg = lane / Gs;
    const int uu = lane - seg * Gs;
    const int64_t row_bytes = static_cast<int64_t>(G) * UB;

    // this workgroup's row groups [g0, g1)
    const int base = NG / static_cast<int>(gridDim.x);
    const int rem = NG - base * static_cast<int>(gridDim.x);
    const int b = blockIdx.x;
    const int g0 = b * base + (b < rem ? b : rem);
    const int g1 = g0 + base + (b < rem ? 1 : 0);

    uint32_t U[1][kUnitWords<F>];
    uint32_t sh[1];
    // slot index within the chunk starting at group c0 -> (row, unit)
    auto load = [&](int c0, int slot) {
        const int g = c0 + slot / KS;
        const int u = (slot % KS) * Gs + uu;
        const int uc = u < G ? u : G - 1;  // lanes past the last unit load a valid one, summed as 0
        int row = g * S + seg;
        row = row < N ? row : N - 1;  // rows past the end load the last row; never stored
        load_unit<F>(U[0], sh[0], W + row * row_bytes + uc * UB,
                     Ws + (static_cast<int64_t>(row) * G + uc) * kUnitScaleBytes<F>);
    };

    int c0 = g0;
    int cn = min(CH, g1 - c0);
    int slot = wave;
    // The activations are staged before the first slot's weights are
    // requested, so that the staging's wait (loads complete in issue order for
    // the wait counter) does not include the weights and the decode starts as
    // they arrive: 2-5% faster for every format at the down shape.
    bool have = false;  // U holds the weights of (c0, slot)
    stage_x<GIN>(xs, x, xu, G, blockDim.x);
    if (slot < cn * KS) {
        load(c0, slot);
        have = true;
    }
    __syncthreads();

    while (c0 < g1) {
        const int cn_next_c0 = c0 + cn;
        const int cn_next = min(CH, g1 - cn_next_c0);
        // a wave with no slot in the previous chunk has not loaded yet
        if (!have && slot < cn * KS) load(c0, slot);
        while (slot < cn * KS) {
            const int kq = slot % KS;
            const int u = kq * Gs + uu;
            const bool live = seg < S && u < G;
            int xoff = (u < G ? u : G - 1) * kXsStride;
            asm volatile("" : "+v"(xoff));
            float acc[1];
            dot_units<F, 1>(U, sh, xs + xoff, acc);
            const int gl = slot / KS;
            // The weights of this slot are consumed: request the next slot's
            // (in this chunk or, past its end, in the next one).
            const int next = slot + nwaves;
            have = true;
            if (next < cn * KS) load(c0, next);
            else if (wave < cn_next * KS) load(cn_next_c0, wave);
            else have = false;
            const float v = segment_sum(live ? acc[0] : 0.f, uu, Gs);
            if (seg < S && uu == 0) red[(gl * S + seg) * KS + kq] = v;
            slot = next;
        }
        __syncthreads();
        for (int r = threadIdx.x; r < cn * S; r += blockDim.x) {
            const int row = c0 * S + r;
            const float* part = red + r * KS;
            float t = part[0];
            for (int q = 1; q < KS; ++q) t += part[q];
            if (row < N) y[row] = t * kRowScale<F>;
        }
        __syncthreads();  // the sums are read before the next chunk rewrites them
        c0 = cn_next_c0;
        cn = cn_next;
        slot = wave;
    }
}

// --------------------------------------------------------- generic kernel
// Activations of the generic kernel: x[i], or gelu(x[i]) * xu[i] for the
// gated down projection (formed per use, float32).
template <bool GIN>
struct ActIn {
    const float* __restrict__ x;
    const float* __restrict__ xu;
    __device__ __forceinline__ float operator()(int64_t i) const {
        if constexpr (GIN) return gelu_tanh(x[i]) * xu[i];
        else return x[i];
    }
};

// srow: MXFP4 only, the row's scale bytes (one per block).
template <int F, bool GIN>
__device__ __forceinline__ float generic_block_dot(const uint8_t* __restrict__ row, int64_t b, ActIn<GIN> xa,
                                                   const uint8_t* __restrict__ srow) {
    if constexpr (F == kMXFP4) {
        const uint4 c = reinterpret_cast<const uint4*>(row)[b];
        uint32_t U[34];
        U[0] = c.x; U[1] = c.y; U[2] = c.z; U[3] = c.w;
        U[32] = srow[b];
        float xk[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) xk[i] = xa(32 * b + i);
        return mxfp4_block_dot<0>(U, xk);
    } else if constexpr (F == kQ4_0) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row + 18 * b);
        const float d = half_bits_to_float(p[0]);
        const int64_t xb = 32 * b;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const uint32_t two = p[1 + h];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int byte = (two >> (8 * i)) & 0xff;
                s = fmaf(static_cast<float>((byte & 15) - 8), xa(xb + 2 * h + i), s);
                s = fmaf(static_cast<float>((byte >> 4) - 8), xa(xb + 16 + 2 * h + i), s);
            }
        }
        return d * s;
    } else if constexpr (F == kQ8_0) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row + 34 * b);
        const float d = half_bits_to_float(p[0]);
        const int64_t xb = 32 * b;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            const uint32_t two = p[1 + h];
            s = fmaf(static_cast<float>(static_cast<int8_t>(two & 0xff)), xa(xb + 2 * h), s);
            s = fmaf(static_cast<float>(static_cast<int8_t>(two >> 8)), xa(xb + 2 * h + 1), s);
        }
        return d * s;
    } else {
        // Q4_K (16-byte aligned super-blocks) or Q6_K (2-byte aligned, read
        // with 16-bit loads) decoded by the unit kernels' block functions
        uint32_t U[54];
        if constexpr (F == kQ4_K) {
            const uint4* src = reinterpret_cast<const uint4*>(row + 144 * b);
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                const uint4 v = src[t];
                U[4 * t] = v.x; U[4 * t + 1] = v.y; U[4 * t + 2] = v.z; U[4 * t + 3] = v.w;
            }
        } else {
            const uint16_t* p = reinterpret_cast<const uint16_t*>(row + 210 * b);
#pragma unroll
            for (int i = 0; i < 52; ++i)
                U[i] = static_cast<uint32_t>(p[2 * i]) | (static_cast<uint32_t>(p[2 * i + 1]) << 16);
            U[53] = p[104];
        }
        float s = 0.f;
        static_for<8>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            float xk[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) xk[i] = xa(256 * b + 32 * k + i);
            if constexpr (F == kQ4_K) s += q4_k_sub_dot<k>(U, xk);
            else s += q6_k_block_dot<k>(U, xk);
            asm volatile("" : "+v"(s));  // one block's activations live at a time
        });
        return s * kRowScale<F>;
    }
}

// Any K % 32 == 0 (K % 256 == 0 for Q4_K and Q6_K).  One wave per row, lanes
// stride over the row's blocks, activations read from global memory.  Rows
// need not be 16-byte aligned; Q4_0 / Q8_0 / Q6_K blocks are read with
// 16-bit loads.
template <int F, bool PAIR, bool GIN>
__global__ __launch_bounds__(kBlockThreads)
void gemv_generic_kernel(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                         const float* __restrict__ x, const float* __restrict__ xu, float* __restrict__ y,
                         int N, int64_t nblocks, int64_t row_bytes) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_stride = gridDim.x * kWavesPerBlock;
    const ActIn<GIN> xa{x, xu};
    for (int row = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < N; row += wave_stride) {
        float a0 = 0.f, a1 = 0.f;
        // MXFP4: W1 is the scale plane, one byte per block
        const uint8_t* srow = (F == kMXFP4) ? W1 + row * nblocks : nullptr;
        for (int64_t b = lane; b < nblocks; b += kWave) {
            a0 += generic_block_dot<F, GIN>(W0 + row * row_bytes, b, xa, srow);
            if constexpr (PAIR) a1 += generic_block_dot<F, GIN>(W1 + row * row_bytes, b, xa, nullptr);
        }
        a0 = wave_sum(a0);
        if constexpr (PAIR) a1 = wave_sum(a1);
        if (lane == 0) {
            if constexpr (PAIR) y[row] = gelu_tanh(a0) * a1;
            else y[row] = a0;
        }
    }
}

template <int F, int R, bool PAIR, bool GIN>
hipError_t launch_unit(const void* W0, const void* W1, const float* x, const float* xu, float* y, int N, int G,
                       hipStream_t stream) {
    const int S = kWave / G;
    const int rows_per_pass = S * R;
    const int npasses = (N + rows_per_pass - 1) / rows_per_pass;
    // One matrix at a time runs best with 3 workgroups per CU, all resident
    // at once, its waves taking several passes each: a wave's first loads
    // then share the memory system with fewer others and arrive sooner.  The
    // pair (4 resident per CU at its 123 VGPRs) and Q6_K, whose passes carry
    // the most bytes (18 and 13.4 KB per wave), run best with one pass per
    // wave and workgroups replacing each other as they finish (1792 at the
    // gate shape), up to 8 per CU before waves loop.
    const int max_blocks = device_cus() * ((PAIR || F == kQ6_K) ? 8 : 3);
    int blocks = (npasses + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    const size_t lds = static_cast<size_t>(G) * kXsStride * sizeof(float);
    hipLaunchKernelGGL((gemv_unit_kernel<F, R, PAIR, GIN>), dim3(blocks), dim3(kBlockThreads), lds, stream,
                       static_cast<const uint8_t*>(W0), static_cast<const uint8_t*>(W1), x, xu, y,
                       N, G, S, npasses);
    return hipGetLastError();
}

// Slicing of a long row for gemv_split_kernel: KS slices of Gs units, S rows
// per slot, NG row groups over `blocks` workgroups of `threads`, CH groups
// per chunk of slice sums in LDS.
struct SplitPlan {
    int KS, Gs, S, NG, CH, blocks, threads;
    size_t lds;
};

// Picks the slice count that keeps the most lanes on real units (ties: fewer
// slices).  False if x does not fit in LDS.
bool plan_split(int G, int N, SplitPlan* p) {
    int best = 0;
    double best_eff = -1.0;
    for (int ks = 2; ks <= 16; ++ks) {
        const int gs = (G + ks - 1) / ks;
        if (gs > kWave) continue;
        const int s = kWave / gs;
        const double eff = static_cast<double>(s) * G / (static_cast<double>(kWave) * ks);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = ks;
        }
    }
    if (best == 0) return false;
    p->KS = best;
    p->Gs = (G + best - 1) / best;
    p->S = kWave / p->Gs;
    p->NG = (N + p->S - 1) / p->S;
    const size_t max_lds = static_cast<size_t>(device_max_lds());
    const size_t x_bytes = static_cast<size_t>(G) * kXsStride * sizeof(float);
    const size_t group_bytes = static_cast<size_t>(p->S) * p->KS * sizeof(float);
    if (x_bytes + group_bytes > max_lds) return false;
    // Two workgroups of 8 waves per CU when both fit in LDS with a chunk of
    // at least 8 groups each, else one of 16 waves.
    const int per_cu = (2 * (x_bytes + 8 * group_bytes) <= max_lds) ? 2 : 1;
    p->threads = kSplitThreads / per_cu;
    const int max_blocks = device_cus() * per_cu;
    p->blocks = p->NG < max_blocks ? p->NG : max_blocks;
    const int per_block = (p->NG + p->blocks - 1) / p->blocks;
    const size_t room = (max_lds / per_cu - x_bytes) / group_bytes;
    p->CH = static_cast<int>(room < static_cast<size_t>(per_block) ? room : static_cast<size_t>(per_block));
    if (p->CH > 1024) p->CH = 1024;
    p->lds = x_bytes + static_cast<size_t>(p->CH) * group_bytes;
    return true;
}

template <int F, bool GIN>
hipError_t launch_split(const void* W, const void* Ws, const float* x, const float* xu, float* y, int N, int G,
                        const SplitPlan& p, hipStream_t stream) {
    hipLaunchKernelGGL((gemv_split_kernel<F, GIN>), dim3(p.blocks), dim3(p.threads), p.lds, stream,
                       static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(Ws), x, xu, y, N, G, p.KS, p.Gs,
                       p.S, p.NG, p.CH);
    return hipGetLastError();
}

template <int F, bool PAIR, bool GIN>
hipError_t launch_generic(const void* W0, const void* W1, const float* x, const float* xu, float* y, int N,
                          int64_t K, hipStream_t stream) {
    const int64_t per = (F == kQ4_K || F == kQ6_K) ? 256 : 32;
    const int64_t bytes = (F == kQ4_0) ? 18 : (F == kQ8_0 ? 34 : (F == kQ4_K ? 144 : (F == kQ6_K ? 210 : 16)));
    const int64_t nb = K / per;
    const int max_blocks = device_cus() * 8;
    int blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL((gemv_generic_kernel<F, PAIR, GIN>), dim3(blocks), dim3(kBlockThreads), 0, stream,
                       static_cast<const uint8_t*>(W0), static_cast<const uint8_t*>(W1), x, xu, y,
                       N, nb, nb * bytes);
    return hipGetLastError();
}

// One format, plain or gated input: unit kernel, split kernel or generic.
// Ws: the scale plane (MXFP4), else nullptr.
template <int F, bool GIN>
hipError_t launch_one(const void* W, const float* x, const float* xu, float* y, int N, int64_t K,
                      hipStream_t stream, const void* Ws = nullptr) {
    if (K % kUnitElems == 0) {
        const int G = static_cast<int>(K / kUnitElems);
        if (G <= kMaxUnits) return launch_unit<F, 1, false, GIN>(W, Ws, x, xu, y, N, G, stream);
        SplitPlan p;
        if (plan_split(G, N, &p)) return launch_split<F, GIN>(W, Ws, x, xu, y, N, G, p, stream);
    }
    return launch_generic<F, false, GIN>(W, Ws, x, xu, y, N, K, stream);
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

int device_max_lds() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n <= 0)
            n = 65536;
        cached[dev] = n;
    }
    return cached[dev];
}

hipError_t launch_gemv(int fmt, const void* W, const void* W_up, const float* x, const float* x_up, float* y,
                       int64_t N64, int64_t K, hipStream_t stream) {
    const int N = static_cast<int>(N64);
    if (W_up != nullptr) {
        // the gated pair: gate and up rows of the same shape in one launch
        const bool unit = (K % kUnitElems == 0) && (K / kUnitElems <= kMaxUnits);
        return unit ? launch_unit<kQ4_0, 1, true, false>(W, W_up, x, nullptr, y, N, static_cast<int>(K / kUnitElems),
                                                        stream)
                    : launch_generic<kQ4_0, true, false>(W, W_up, x, nullptr, y, N, K, stream);
    }
    if (x_up != nullptr) {
        switch (fmt) {
        case kQ4_0: return launch_one<kQ4_0, true>(W, x, x_up, y, N, K, stream);
        case kQ4_K: return launch_one<kQ4_K, true>(W, x, x_up, y, N, K, stream);
        default: return launch_one<kQ6_K, true>(W, x, x_up, y, N, K, stream);
        }
    }
    switch (fmt) {
    case kQ4_0: return launch_one<kQ4_0, false>(W, x, nullptr, y, N, K, stream);
    case kQ8_0: return launch_one<kQ8_0, false>(W, x, nullptr, y, N, K, stream);
    case kQ4_K: return launch_one<kQ4_K, false>(W, x, nullptr, y, N, K, stream);
    default: return launch_one<kQ6_K, false>(W, x, nullptr, y, N, K, stream);
    }
}

hipError_t launch_gemv_mxfp4(const void* codes, const void* scales, const float* x, float* y, int64_t N, int64_t K,
                             hipStream_t stream) {
    return launch_one<kMXFP4, false>(codes, x, nullptr, y, static_cast<int>(N), K, stream, scales);
}

hipError_t launch_qkv(const void* Wq, const void* Wk, const void* Wv, const float* x, float* yq, float* yk, float* yv,
                      int64_t Nq, int64_t Nk, int64_t Nv, int64_t K, hipStream_t stream) {
    const int G = static_cast<int>(K / kUnitElems);
    if (G > kMaxUnits) {
        // long rows: one split-kernel launch per matrix
        hipError_t e = launch_one<kQ4_K, false>(Wq, x, nullptr, yq, static_cast<int>(Nq), K, stream);
        if (e == hipSuccess) e = launch_one<kQ4_K, false>(Wk, x, nullptr, yk, static_cast<int>(Nk), K, stream);
        if (e == hipSuccess) e = launch_one<kQ6_K, false>(Wv, x, nullptr, yv, static_cast<int>(Nv), K, stream);
        return e;
    }
    const int S = kWave / G;
    const int Pq = static_cast<int>((Nq + S - 1) / S);
    const int Pk = static_cast<int>((Nk + S - 1) / S);
    const int Pv = static_cast<int>((Nv + S - 1) / S);
    const int npasses = Pq + Pk + Pv;
    const int max_blocks = device_cus() * 3;
    int blocks = (npasses + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    const size_t lds = static_cast<size_t>(G) * kXsStride * sizeof(float);
    hipLaunchKernelGGL((gemv_qkv_kernel<kQ4_K, kQ6_K>), dim3(blocks), dim3(kBlockThreads), lds, stream,
                       static_cast<const uint8_t*>(Wq), static_cast<const uint8_t*>(Wk),
                       static_cast<const uint8_t*>(Wv), x, yq, yk, yv, static_cast<int>(Nq), static_cast<int>(Nk),
                       static_cast<int>(Nv), G, S, Pv, Pq, Pk);
    return hipGetLastError();
}

}  // namespace qmv
