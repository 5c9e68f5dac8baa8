// Device-side helpers shared by the libqmv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;          // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlockThreads / kWave;

// A "unit" is the smallest run of whole blocks that starts and ends on a
// 16-byte boundary: 8 Q4_0 blocks (144 B), 8 Q8_0 blocks (272 B) or one Q4_K
// super-block (144 B); and, as the one exception, one Q6_K super-block
// (210 B, 2-byte aligned).  Each covers 256 weights.  With K % 256 == 0 every row,
// and every unit in it, is 16-byte aligned, so a lane can stream a unit with
// plain 16-byte loads and find each block at a compile-time byte offset.
constexpr int kUnitElems = 256;
// The activation slice of one unit is stored in LDS with 4 floats of padding
// so that lanes holding consecutive units start on different LDS banks.
constexpr int kXsStride = kUnitElems + 4;

enum Format : int { kQ4_0 = 0, kQ8_0 = 1, kQ4_K = 2, kQ6_K = 3, kMXFP4 = 4 };

template <int F> struct UnitInfo;
template <> struct UnitInfo<kQ4_0> { static constexpr int kBytes = 144; static constexpr int kVec = 9; };
template <> struct UnitInfo<kQ8_0> { static constexpr int kBytes = 272; static constexpr int kVec = 17; };
template <> struct UnitInfo<kQ4_K> { static constexpr int kBytes = 144; static constexpr int kVec = 9; };
// A Q6_K super-block (210 B) starts on a 2-byte boundary only: its lane reads
// the 13 dword-aligned 16-byte pieces from the dword at or before its start
// and two 16-bit words at its end, then realigns (see gemv.hip).
template <> struct UnitInfo<kQ6_K> { static constexpr int kBytes = 210; static constexpr int kVec = 13; };

// MXFP4 keeps codes and scales in two planes: a unit is 8 blocks, i.e. 128
// code bytes (kBytes, kVec below) plus 8 scale bytes from the scale plane.
template <> struct UnitInfo<kMXFP4> { static constexpr int kBytes = 128; static constexpr int kVec = 8; };

// 16-byte vector with 4-byte alignment: one global_load_dwordx4 from an
// address that is only dword aligned.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// Signed byte i of a dword, converted to float (one SDWA convert on gfx950).
template <int I>
__device__ __forceinline__ float sbyte(uint32_t v) {
    return static_cast<float>(static_cast<int8_t>(v >> (8 * I)));
}

// Unsigned byte i of a dword, converted to float (v_cvt_f32_ubyteI).
template <int I>
__device__ __forceinline__ float ubyte(uint32_t v) {
    return static_cast<float>(static_cast<uint8_t>(v >> (8 * I)));
}

// Bytes [2, 6) of the 8-byte little-endian pair (lo, hi).
__device__ __forceinline__ uint32_t shift16(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// Sum of v over the L consecutive lanes [slot_base, slot_base + L) of a
// wave; the total lands in the first lane of the segment (u == 0), where u
// is the lane's index inside its segment.  Works for any 1 <= L <= 64.
__device__ __forceinline__ float segment_sum(float v, int u, int L) {
    for (int o = 1; o < L; o <<= 1) {
        float t = __shfl_down(v, o, kWave);
        if (u + o < L) v += t;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// GELU, tanh form: v/2 (1 + tanh z), z = sqrt(2/pi) (v + 0.044715 v^3).
// Evaluated as v / (1 + e^(-2z)), the same function (1 + tanh z =
// 2 / (1 + e^(-2z))) without the cancellation of 1 + tanh z near z << 0,
// with e^(-2z) = 2^(-2z log2 e) from v_exp_f32 and the quotient from
// v_rcp_f32: a few instructions instead of a tanhf call.  Error: a few ulp
// of the result, plus the exponent argument's rounding, which matters only
// where the result is below e^-1 |v| 2^-24.  e^(-2z) overflowing to +inf
// gives -0 for v << 0, and underflowing to 0 gives v: never NaN.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    const float inner = c * (v + 0.044715f * v * v * v);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * inner);  // -2 log2(e) z
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace qmv
