/*
 * oracle.c -- plain CPU reference ("oracle") for fused-dequant quantized
 * matrix-vector products.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: it is used by tests/, by __graft_entry__.smoke() and by the
 * cpu_baseline leg of bench.py, and by nothing else.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Everything here is the plain definition of what the hot path computes,
 * written out in float64 with naive loops in index order.  No blocking, no
 * fusion, no reordering.  The only exceptions, each marked where it occurs,
 * are the steps whose precision the method itself fixes at float32 (the
 * activation quantizer) so that integer codes are decided in the same
 * precision on both sides.
 *
 * Sources ("the pages"):
 *   [roadmap]  "Gemma 4 M4 Max kernel roadmap" (gem, docs/research)
 *   [captable] "Metal kernel capability table (Phase B ground truth)" (larql)
 * Block formats are the GGUF Q4_0 / Q8_0 / Q4_K layouts that both pages load
 * (roadmap K0: strict GGUF loader; captable section 1: 18 B Q4_0, 34 B Q8_0,
 * 144 B Q4_K blocks).  Where the pages leave a detail open, the reading
 * adopted is stated at the function that depends on it ("Reading: ...").
 *
 * Parity status of each function is stated in its comment ("pinned by ...").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_Q4_0 0
#define ORACLE_Q8_0 1
#define ORACLE_Q4_K 2
#define ORACLE_Q6_K 3

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 -> double.                                        */
/* Definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.*/
/* e == 0: subnormal, value = f * 2^-24; e == 31: inf (f == 0) or NaN.  */
/* Pinned by tests against numpy's float16 conversion for all 65536    */
/* bit patterns.                                                       */
/* ------------------------------------------------------------------ */
double oracle_fp16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Bytes per row of K weights, or -1 if K is not a whole number of blocks. */
int64_t oracle_row_bytes(int fmt, int64_t K) {
    switch (fmt) {
    case ORACLE_Q4_0: return (K % 32) ? -1 : (K / 32) * 18;
    case ORACLE_Q8_0: return (K % 32) ? -1 : (K / 32) * 34;
    case ORACLE_Q4_K: return (K % 256) ? -1 : (K / 256) * 144;
    case ORACLE_Q6_K: return (K % 256) ? -1 : (K / 256) * 210;
    default: return -1;
    }
}

/* ------------------------------------------------------------------ */
/* Q4_0 block (18 B, 32 weights): fp16 d, then 16 bytes of 4-bit codes. */
/* w = (q - 8) * d.                                                     */
/* Reading (nibble order, GGUF): byte j of the code area holds element */
/* j in its low nibble and element j+16 in its high nibble.            */
/* [roadmap K1: Q4_0 dequantization; captable section 1, 18 B Q4_0]    */
/* Pinned by hand-built blocks (q=8 -> 0, q=0 -> -8d, q=15 -> 7d,      */
/* element order) in tests/test_oracle_formats.py.                     */
/* ------------------------------------------------------------------ */
static void dequant_q4_0_block(const uint8_t* b, double* w) {
    double d = oracle_fp16_to_f64(rd16(b));
    for (int j = 0; j < 16; ++j) {
        int lo = b[2 + j] & 0x0f;
        int hi = b[2 + j] >> 4;
        w[j] = (double)(lo - 8) * d;
        w[j + 16] = (double)(hi - 8) * d;
    }
}

/* Q8_0 block (34 B, 32 weights): fp16 d then 32 signed bytes; w = q * d. */
/* Reading: interleaved layout (scale inside the block), as in GGUF.     */
/* [roadmap K1: Q8_0 dequantization; roadmap K2 step 6: Q8_0 tied      */
/* embedding/output projection]                                         */
static void dequant_q8_0_block(const uint8_t* b, double* w) {
    double d = oracle_fp16_to_f64(rd16(b));
    for (int j = 0; j < 32; ++j) w[j] = (double)(int8_t)b[2 + j] * d;
}

/* Q4_K super-block (144 B, 256 weights) [captable section 1, q4k_matvec]:
 *   bytes 0-1 d (fp16), 2-3 dmin (fp16), 4-15 twelve bytes holding eight
 *   6-bit sub-block scales and eight 6-bit sub-block mins, 16-143 codes.
 * Reading (GGUF packing):
 *   j < 4 : scale_j = P[j] & 63,                    min_j = P[j+4] & 63
 *   j >= 4: scale_j = (P[j+4] & 15) | (P[j-4] >> 6) << 4,
 *           min_j   = (P[j+4] >> 4) | (P[j]   >> 6) << 4
 *   sub-blocks 2c and 2c+1 (c = 0..3) take the low and the high nibbles of
 *   code bytes 32c .. 32c+31.
 *   w = d * scale_j * q - dmin * min_j.
 * Pinned by a bit-placement pack/unpack round trip and hand-built
 * single-scale / single-min super-blocks in tests/test_oracle_formats.py. */
void oracle_q4_k_scale_min(const uint8_t* P, int j, int* sc, int* mn) {
    if (j < 4) {
        *sc = P[j] & 63;
        *mn = P[j + 4] & 63;
    } else {
        *sc = (P[j + 4] & 15) | ((P[j - 4] >> 6) << 4);
        *mn = (P[j + 4] >> 4) | ((P[j] >> 6) << 4);
    }
}

static void dequant_q4_k_block(const uint8_t* b, double* w) {
    double d = oracle_fp16_to_f64(rd16(b));
    double dmin = oracle_fp16_to_f64(rd16(b + 2));
    const uint8_t* P = b + 4;
    const uint8_t* qs = b + 16;
    for (int j = 0; j < 8; ++j) {
        int sc, mn;
        oracle_q4_k_scale_min(P, j, &sc, &mn);
        int c = j / 2;
        for (int l = 0; l < 32; ++l) {
            uint8_t byte = qs[32 * c + l];
            int q = (j % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
            w[32 * j + l] = d * (double)sc * (double)q - dmin * (double)mn;
        }
    }
}

/* Q6_K super-block (210 B, 256 weights) [captable section 1, q6k_matvec:
 * "Q6_K 210B planar"; the format of the V and down projections in the
 * pages' Q4_K_M mix, captable section 2 q4k_q6k_qkv_proj]:
 *   bytes 0-127 ql (low 4 bits of the codes), 128-191 qh (high 2 bits),
 *   192-207 sixteen signed 8-bit sub-block scales, 208-209 d (fp16).
 * Reading (the pages give the size and the word "planar" only; the GGUF
 * super-block is what their loaders read):
 *   element e = 128h + 32g + l (h < 2, g < 4, l < 32) takes
 *     the low nibble (g = 0, 1) or the high nibble (g = 2, 3) of
 *     ql[64h + 32(g mod 2) + l], and bits 2g, 2g+1 of qh[32h + l] as its
 *     two high bits;  q = nibble + 16 * high bits, in 0..63;
 *   w_e = d * scale[e / 16] * (q - 32).
 * Pinned by hand-built super-blocks (q = 32 -> 0, 0 -> -32 d s,
 * 63 -> 31 d s, signed scales -128 and 127, every element placed alone) in
 * tests/test_oracle_formats.py. */
static void dequant_q6_k_block(const uint8_t* b, double* w) {
    const uint8_t* ql = b;
    const uint8_t* qh = b + 128;
    const int8_t* sc = (const int8_t*)(b + 192);
    double d = oracle_fp16_to_f64(rd16(b + 208));
    for (int e = 0; e < 256; ++e) {
        int h = e / 128, g = (e % 128) / 32, l = e % 32;
        uint8_t lowbyte = ql[64 * h + 32 * (g % 2) + l];
        int nib = (g < 2) ? (lowbyte & 0x0f) : (lowbyte >> 4);
        int high = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = nib + 16 * high;
        w[e] = d * (double)sc[e / 16] * (double)(q - 32);
    }
}

/* ------------------------------------------------------------------ */
/* MXFP4 [captable section 1: mxfp4_matvec, 16 code bytes per 32     */
/* weights, E8M0 scales outside the blocks; roadmap K5: a next weight   */
/* layout that decodes with packed hardware conversions].  Two planes: */
/*   codes  [N][K/32][16 B]: 32 four-bit E2M1 elements per block,       */
/*   scales [N][K/32] bytes: one E8M0 exponent per block.               */
/* Reading (the pages give the sizes and the word "ext" only):          */
/*   element 2i of a block is the low nibble of code byte i, element     */
/*   2i+1 its high nibble (the consecutive-pair order of MX checkpoints  */
/*   stored as separate block and scale tensors);                       */
/*   E2M1 (OCP Microscaling formats): sign bit, 2 exponent bits with     */
/*   bias 1, 1 mantissa bit; exponent 0 is subnormal (m * 2^-1), no      */
/*   infinities or NaNs;                                                 */
/*   E8M0: 2^(e - 127), e = 255 is NaN;                                  */
/*   w = E2M1(code) * E8M0(scale).                                       */
/* Pinned in tests/test_oracle_mxfp4.py: E8M0 against torch's           */
/* float8_e8m0fnu for all 256 bytes, E2M1 against a generic minifloat   */
/* decoder that is itself checked on numpy's float16 and torch's        */
/* float8_e4m3fn, element order and plane layout on hand-built blocks.  */
/* ------------------------------------------------------------------ */
double oracle_e2m1_to_f64(int code) {
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v = (e == 0) ? ldexp((double)m, -1) : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return sign ? -v : v;
}

double oracle_e8m0_to_f64(int e) {
    return (e == 255) ? NAN : ldexp(1.0, e - 127);
}

int64_t oracle_mxfp4_plane_bytes(int64_t K, int64_t* scale_bytes) {
    if (K % 32) return -1;
    if (scale_bytes) *scale_bytes = K / 32;
    return (K / 32) * 16;
}

/* One row: codes row (K/2 bytes), scales row (K/32 bytes). */
int oracle_dequant_mxfp4_row(const uint8_t* codes, const uint8_t* scales, int64_t K, double* w) {
    if (K % 32) return -1;
    for (int64_t b = 0; b < K / 32; ++b) {
        double s = oracle_e8m0_to_f64(scales[b]);
        for (int i = 0; i < 16; ++i) {
            uint8_t byte = codes[16 * b + i];
            w[32 * b + 2 * i] = oracle_e2m1_to_f64(byte & 0x0f) * s;
            w[32 * b + 2 * i + 1] = oracle_e2m1_to_f64(byte >> 4) * s;
        }
    }
    return 0;
}

/* y[m][i] = sum_k w[r_i][k] x[m][k], S = sum |w x|, as oracle_qmv, for an
 * MXFP4 matrix given as its two planes. */
int oracle_qmv_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                     const float* x, int64_t M, const int64_t* rows, int64_t nrows,
                     double* y, double* S) {
    if (K % 32) return -1;
    if (rows == NULL) nrows = N;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        if (r < 0 || r >= N) return -2;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            if (!w) continue;
            int64_t r = rows ? rows[i] : i;
            oracle_dequant_mxfp4_row(codes + r * (K / 2), scales + r * (K / 32), K, w);
            for (int64_t m = 0; m < M; ++m) {
                const float* xm = x + m * K;
                double acc = 0.0, sabs = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = w[k] * (double)xm[k];
                    acc += p;
                    sabs += fabs(p);
                }
                y[m * nrows + i] = acc;
                if (S) S[m * nrows + i] = sabs;
            }
        }
        free(w);
    }
    return bad ? -3 : 0;
}

/* Dequantize one row of K weights to float64.  Returns 0, or -1 on a bad
 * format / K. */
int oracle_dequant_row(int fmt, const uint8_t* row, int64_t K, double* w) {
    if (oracle_row_bytes(fmt, K) < 0) return -1;
    if (fmt == ORACLE_Q4_0) {
        for (int64_t b = 0; b < K / 32; ++b) dequant_q4_0_block(row + 18 * b, w + 32 * b);
    } else if (fmt == ORACLE_Q8_0) {
        for (int64_t b = 0; b < K / 32; ++b) dequant_q8_0_block(row + 34 * b, w + 32 * b);
    } else if (fmt == ORACLE_Q4_K) {
        for (int64_t b = 0; b < K / 256; ++b) dequant_q4_k_block(row + 144 * b, w + 256 * b);
    } else {
        for (int64_t b = 0; b < K / 256; ++b) dequant_q6_k_block(row + 210 * b, w + 256 * b);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Matrix-vector product with fused dequantization, float64.           */
/*   y[m][i] = sum_k w[r_i][k] * x[m][k]      (naive, k ascending)      */
/*   S[m][i] = sum_k |w[r_i][k] * x[m][k]|    (scale of the tolerance)  */
/* for the selected rows r_i (rows == NULL: all N rows in order).      */
/* Output layout: [M][nrows].                                          */
/* [roadmap K1: matrix-vector; roadmap K2 step 1: the Q4_0 product    */
/* that decodes blocks inside the dot product, float32 sums]           */
/* Pinned by exact rational brute force (K = 32, 64), e_i columns and  */
/* linearity in tests/test_oracle_qmv.py.                              */
/* ------------------------------------------------------------------ */
int oracle_qmv(int fmt, const uint8_t* W, int64_t N, int64_t K,
               const float* x, int64_t M,
               const int64_t* rows, int64_t nrows,
               double* y, double* S) {
    int64_t rb = oracle_row_bytes(fmt, K);
    if (rb < 0) return -1;
    if (rows == NULL) nrows = N;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        if (r < 0 || r >= N) return -2;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            if (!w) continue;
            int64_t r = rows ? rows[i] : i;
            oracle_dequant_row(fmt, W + r * rb, K, w);
            for (int64_t m = 0; m < M; ++m) {
                const float* xm = x + m * K;
                double acc = 0.0, sabs = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = w[k] * (double)xm[k];
                    acc += p;
                    sabs += fabs(p);
                }
                y[m * nrows + i] = acc;
                if (S) S[m * nrows + i] = sabs;
            }
        }
        free(w);
    }
    return bad ? -3 : 0;
}

/* ------------------------------------------------------------------ */
/* GELU, tanh form, float64:                                           */
/*   gelu(v) = v/2 * (1 + tanh(sqrt(2/pi) * (v + 0.044715 v^3)))        */
/* Reading: "GELU-gated FFN" [roadmap K1, K2 step 5] is the tanh form  */
/* used for Gemma [captable section 4, geglu_gelu_tanh].  For |v| so    */
/* large that v^3 overflows, tanh saturates to +-1 and the result is v  */
/* or 0, never NaN.                                                    */
/* Pinned by special values and the erf form within 1e-3 in tests.      */
/* ------------------------------------------------------------------ */
double oracle_gelu_tanh(double v) {
    const double c = sqrt(2.0 / M_PI);
    double inner = c * (v + 0.044715 * v * v * v);
    /* tanh(+-inf) = +-1, so an overflowing cube still gives v or -0. */
    return 0.5 * v * (1.0 + tanh(inner));
}

/* Gated pair: h = gelu(g) * u   [roadmap K2 step 5: the FFN's gate and up projections] */
void oracle_geglu(const double* g, const double* u, int64_t n, double* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = oracle_gelu_tanh(g[i]) * u[i];
}

/* ------------------------------------------------------------------ */
/* Down projection of a gated FFN with the GELU gate applied to its     */
/* input [captable section 4: q4k_geglu_gelu_tanh_down and              */
/* q6k_geglu_gelu_tanh_down take the gate and up activations and fold   */
/* the GELU-tanh product into the down matrix-vector; roadmap K2 step 5: */
/* the gated GELU FFN]:                                                 */
/*   h[m][k] = gelu(g[m][k]) * u[m][k]             (float64)            */
/*   y[m][i] = sum_k w[r_i][k] * h[m][k]           (naive, k ascending) */
/*   S[m][i] = sum_k |w[r_i][k] * h[m][k]|                              */
/*   E[m][i] = sum_k |w[r_i][k]| |u[m][k]| (|g[m][k]| + |gelu(g[m][k])|) */
/* E scales the error a float32 evaluation of h may add (the tolerance  */
/* rule in __init__.py).                                                */
/* Pinned in tests/test_oracle_geglu_down.py by gates of +-64 (gelu     */
/* exactly 64 or -0 in float64, so y = 64 W u exactly or 0), u = 0, and */
/* the agreement of S and E with qmv's S at those gates.                */
/* ------------------------------------------------------------------ */
int oracle_qmv_geglu_down(int fmt, const uint8_t* W, int64_t N, int64_t K,
                          const float* g, const float* u, int64_t M,
                          const int64_t* rows, int64_t nrows,
                          double* y, double* S, double* E) {
    int64_t rb = oracle_row_bytes(fmt, K);
    if (rb < 0) return -1;
    if (rows == NULL) nrows = N;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        if (r < 0 || r >= N) return -2;
    }
    double* h = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* e = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!h || !e) { free(h); free(e); return -3; }
    for (int64_t t = 0; t < M * K; ++t) {
        double gl = oracle_gelu_tanh((double)g[t]);
        h[t] = gl * (double)u[t];
        e[t] = fabs((double)u[t]) * (fabs((double)g[t]) + fabs(gl));
    }
    int bad = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            if (!w) continue;
            int64_t r = rows ? rows[i] : i;
            oracle_dequant_row(fmt, W + r * rb, K, w);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0, sabs = 0.0, eabs = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = w[k] * h[m * K + k];
                    acc += p;
                    sabs += fabs(p);
                    eabs += fabs(w[k]) * e[m * K + k];
                }
                y[m * nrows + i] = acc;
                if (S) S[m * nrows + i] = sabs;
                if (E) E[m * nrows + i] = eabs;
            }
        }
        free(w);
    }
    free(h);
    free(e);
    return bad ? -3 : 0;
}

/* Logit soft-cap z = cap * tanh(y / cap), float64.                     */
/* [roadmap K1: logit soft-capping]; cap = 30 for the logit workload.   */
void oracle_softcap(const double* y, int64_t n, double cap, double* z) {
    for (int64_t i = 0; i < n; ++i) z[i] = cap * tanh(y[i] / cap);
}

/* ------------------------------------------------------------------ */
/* Activation quantization to Q8 per 32-element block.                 */
/* [captable section 2: quantize_q8, f32 -> int8 + per-32 scales;      */
/* captable section 1: q4_matvec_v4 takes Q8 int8 + scales]            */
/* Reading (the pages name the step only): all in float32 because the   */
/* codes are integers decided by float arithmetic and both sides must   */
/* decide them in the same precision:                                  */
/*   amax = max |x|;  d = amax / 127 (IEEE division);                   */
/*   q = clamp(round_half_away_from_zero(x / d), -127, 127);           */
/*   amax == 0  ->  d = 0, q = 0.                                       */
/* K must be a multiple of 32 (no partial tail block: the captable's    */
/* finding F6 is a tail-scale defect of exactly this step).            */
/* Pinned by tie and degenerate blocks in tests/test_oracle_q8.py.      */
/* ------------------------------------------------------------------ */
int oracle_quantize_q8(const float* x, int64_t M, int64_t K, int8_t* q, float* d) {
    if (K % 32) return -1;
    int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + m * K + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float db = amax / 127.0f;
            d[m * nb + b] = db;
            for (int i = 0; i < 32; ++i) {
                int8_t v = 0;
                if (amax != 0.0f) {
                    float t = roundf(xb[i] / db);
                    if (t > 127.0f) t = 127.0f;
                    if (t < -127.0f) t = -127.0f;
                    v = (int8_t)t;
                }
                q[m * K + 32 * b + i] = v;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Integer block dot products of Q4_0 weights with Q8 activations.     */
/*   isum[m][i][b] = sum_{j<32} (q_w[r_i][32b+j] - 8) * q_x[m][32b+j]    */
/* accumulated in int64 and checked to fit int32 (returns -4 if not).   */
/* [captable section 1: q4_matvec_v4, Q4_0 x Q8 int8 + scales]         */
/* Output layout [M][nrows][K/32].                                     */
/* Pinned by an integer-valued case with unit scales in tests.          */
/* ------------------------------------------------------------------ */
int oracle_q4_0_q8_blocksums(const uint8_t* W, int64_t N, int64_t K,
                             const int8_t* qx, int64_t M,
                             const int64_t* rows, int64_t nrows, int32_t* isum) {
    if (K % 32) return -1;
    int64_t nb = K / 32, rb = nb * 18;
    if (rows == NULL) nrows = N;
    int overflow = 0;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        if (r < 0 || r >= N) return -2;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = W + r * rb + 18 * b;
            int qw[32];
            for (int j = 0; j < 16; ++j) {
                qw[j] = (blk[2 + j] & 0x0f) - 8;
                qw[j + 16] = (blk[2 + j] >> 4) - 8;
            }
            for (int64_t m = 0; m < M; ++m) {
                int64_t s = 0;
                for (int j = 0; j < 32; ++j) s += (int64_t)qw[j] * (int64_t)qx[m * K + 32 * b + j];
                if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
                isum[(m * nrows + i) * nb + b] = (int32_t)s;
            }
        }
    }
    return overflow ? -4 : 0;
}

/* y[m][i] = sum_b isum * d_w * d_x  (float64), with
 * S[m][i] = sum_b |d_w * d_x| * sum_j |(q_w - 8) * q_x|.
 * [captable section 1: q4_matvec_v4 scales the int block sums by both
 * block scales]  Needs the quantized activations (oracle_quantize_q8).  */
int oracle_qmm_q4_0_q8(const uint8_t* W, int64_t N, int64_t K,
                       const int8_t* qx, const float* dx, int64_t M,
                       const int64_t* rows, int64_t nrows, double* y, double* S) {
    if (K % 32) return -1;
    int64_t nb = K / 32, rb = nb * 18;
    if (rows == NULL) nrows = N;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        if (r < 0 || r >= N) return -2;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* blk = W + r * rb + 18 * b;
                double dw = oracle_fp16_to_f64(rd16(blk));
                double dxb = (double)dx[m * nb + b];
                int64_t s = 0, sa = 0;
                for (int j = 0; j < 16; ++j) {
                    int lo = (blk[2 + j] & 0x0f) - 8;
                    int hi = (blk[2 + j] >> 4) - 8;
                    int64_t p0 = (int64_t)lo * qx[m * K + 32 * b + j];
                    int64_t p1 = (int64_t)hi * qx[m * K + 32 * b + j + 16];
                    s += p0 + p1;
                    sa += llabs(p0) + llabs(p1);
                }
                acc += (double)s * dw * dxb;
                sabs += fabs(dw * dxb) * (double)sa;
            }
            y[m * nrows + i] = acc;
            if (S) S[m * nrows + i] = sabs;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Top-k by full sort.                                                  */
/* [roadmap K4: top_k = 0 means an exhaustive sort of all logits; the   */
/* bounded heap there is an optimisation of the same selection]         */
/* Reading (order): value descending, equal values -> lower index       */
/* first, NaN after every number (NaNs among themselves by index).      */
/* Merge sort of indices: stable and independent of qsort's order.      */
/* Pinned against a brute-force selection in tests/test_oracle_special.py. */
/* ------------------------------------------------------------------ */
static int before(const double* v, int32_t a, int32_t b) {
    /* strict "a ranks before b" */
    double va = v[a], vb = v[b];
    int na = isnan(va), nb = isnan(vb);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb;  /* a is a number, b is NaN */
    }
    if (va > vb) return 1;
    if (va < vb) return 0;
    return a < b;
}

static void msort(const double* v, int32_t* idx, int32_t* tmp, int64_t n) {
    if (n < 2) return;
    int64_t h = n / 2;
    msort(v, idx, tmp, h);
    msort(v, idx + h, tmp, n - h);
    int64_t i = 0, j = h, o = 0;
    while (i < h && j < n) {
        if (before(v, idx[j], idx[i])) tmp[o++] = idx[j++];
        else tmp[o++] = idx[i++];
    }
    while (i < h) tmp[o++] = idx[i++];
    while (j < n) tmp[o++] = idx[j++];
    memcpy(idx, tmp, sizeof(int32_t) * (size_t)n);
}

int oracle_topk(const double* y, int64_t n, int32_t k, int32_t* out_idx) {
    if (n < 1 || k < 1 || k > n || n > INT32_MAX) return -1;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!idx || !tmp) { free(idx); free(tmp); return -3; }
    for (int64_t i = 0; i < n; ++i) idx[i] = (int32_t)i;
    msort(y, idx, tmp, n);
    memcpy(out_idx, idx, sizeof(int32_t) * (size_t)k);
    free(idx);
    free(tmp);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Token selection from the k selected pairs (values z[0..k) sorted,
 * largest first; idx the matching vocabulary indices), [roadmap K5: top-k40
 * and top-p tokens selected on the device after the tied projection].
 * Reading: softmax over the k soft-capped values at temperature T, the
 * nucleus is the smallest prefix whose probability reaches top_p, and the
 * token is drawn by inverse CDF within the nucleus from the caller's uniform
 * u in [0, 1).  NaN values weigh 0; if every weight is 0 the first pair is
 * taken.  cum[0..k) receives the prefix sums of the weights (float64), so a
 * caller can see how far u and top_p lie from a decision boundary.
 * Pinned by tests/test_oracle_sample.py (hand-computed two- and three-way
 * cases, k = 1, top_p = 1, flat weights, NaN weights). */
int oracle_sample_topp(const double* z, const int32_t* idx, int32_t k, double T, double top_p, double u,
                       int32_t* token, int32_t* nucleus, double* cum) {
    if (k < 1 || !(T > 0.0) || !(top_p > 0.0) || !(top_p <= 1.0)) return 1;
    double s = 0.0;
    for (int32_t i = 0; i < k; ++i) {
        const double w = (isnan(z[i]) || isnan(z[0])) ? 0.0 : exp((z[i] - z[0]) / T);
        s += w;
        cum[i] = s;
    }
    int32_t n = 1, j = 0;
    if (s > 0.0) {
        n = k;
        for (int32_t i = 0; i < k; ++i) {
            if (cum[i] >= top_p * s) { n = i + 1; break; }
        }
        const double target = u * cum[n - 1];
        j = n - 1;
        for (int32_t i = 0; i < n; ++i) {
            if (cum[i] > target) { j = i; break; }
        }
    }
    *token = idx[j];
    *nucleus = n;
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the OpenMP loops (timing the oracle single-threaded). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
