/*
 * qmv.h -- C ABI of libqmv.so: matrix-vector (and small matrix-matrix)
 * products over block-quantized weights with the dequantization fused into
 * the dot product, for AMD Instinct MI355X (gfx950).
 *
 * Sources ("the pages"):
 *   [roadmap]  "Gemma 4 M4 Max kernel roadmap" (gem, docs/research)
 *   [captable] "Metal kernel capability table (Phase B ground truth)" (larql)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every buffer pointer is a DEVICE pointer owned by the caller.  The
 *   library allocates nothing, copies nothing between host and device and
 *   never synchronizes; buffers may be reused across calls (the persistent
 *   buffer path, [roadmap K2: persistent/no-copy buffers; K4: arenas
 *   allocated once, no tensor-sized allocation during generation]).
 *   Weights and activations are only read.  Outputs and workspaces must not
 *   overlap any input.
 * Weights W.  N rows, row-major, each row K weights stored as K/32 blocks
 *   (Q4_0, Q8_0) or K/256 super-blocks (Q4_K, Q6_K) in the GGUF byte layout:
 *     Q4_0 (18 B / 32 weights): fp16 d, 16 bytes of codes; byte j holds
 *          element j (low nibble) and element j+16 (high nibble);
 *          w = (q - 8) * d.
 *     Q8_0 (34 B / 32 weights): fp16 d, 32 int8 codes; w = q * d.
 *     Q4_K (144 B / 256 weights): fp16 d, fp16 dmin, 12 bytes packing eight
 *          6-bit sub-block scales and eight 6-bit mins, 128 code bytes;
 *          w = d * scale_j * q - dmin * min_j for sub-block j.
 *     Q6_K (210 B / 256 weights): 128 bytes of low nibbles ql, 64 bytes of
 *          high 2-bit pairs qh, 16 int8 sub-block scales, fp16 d; element
 *          128h + 32g + l (h < 2, g < 4, l < 32) has the low (g < 2) or
 *          high (g >= 2) nibble of ql[64h + 32(g % 2) + l] and bits 2g, 2g+1
 *          of qh[32h + l]; w = d * scale[e / 16] * (q - 32).
 *   [captable section 1: 18 B Q4_0, 144 B Q4_K, 210 B Q6_K; roadmap K1:
 *   Q4_0 and Q8_0 dequantization]
 * Activations x: float32 [M][K] row-major.  Outputs y: float32 [M][N].
 * Accumulation is float32 [roadmap K2 step 1: F32 accumulation].
 * Stream.  Work is enqueued on `stream` (0 = the null stream) and runs
 *   asynchronously; QMV_OK means "enqueued".  Calls are reentrant when they
 *   do not share output or workspace buffers.
 * Errors.  All arguments are checked on the host before anything is
 *   enqueued; on any error nothing is launched and the call returns the
 *   status below [captable section 9: dimensions are validated when a
 *   call is made rather than taken for granted, and no path may skip part
 *   of the work without an error; captable findings F6, F13 and F17 are the
 *   defects this rules out]:
 *     QMV_ERR_NULL       a required pointer is NULL
 *     QMV_ERR_SHAPE      N, M < 1; M > 65535; K < 32 or K % 32 != 0 (K % 256
 *                        != 0 for Q4_K, Q6_K); a size or a byte count overflows int64, or
 *                        N >= 2^31
 *     QMV_ERR_ALIGN      W or a workspace is not 16-byte aligned, or an f32
 *                        / int32 buffer is not 4-byte aligned
 *     QMV_ERR_WORKSPACE  workspace smaller than the *_ws_bytes() size
 *     QMV_ERR_ARG        other argument out of range (k, softcap)
 *     QMV_ERR_LAUNCH     the HIP runtime rejected a launch
 *   There is no ceiling on K.  Any N is accepted (row tails are masked).
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMV_OK = 0,
    QMV_ERR_NULL = 1,
    QMV_ERR_SHAPE = 2,
    QMV_ERR_ALIGN = 3,
    QMV_ERR_WORKSPACE = 4,
    QMV_ERR_LAUNCH = 5,
    QMV_ERR_ARG = 6
} qmv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* qmv_status_str(int status);

/* y[m][n] = sum_k w[n][k] * x[m][k], Q4_0 weights.
 * [roadmap K2 step 1: the Q4_0 matrix-vector product that decodes blocks
 *  inside the dot product and sums in float32; captable section 1:
 *  q4_f32_matvec, Q4_0 weights times float32 activations]
 * M > 1 is M independent matrix-vector products. */
int qmv_q4_0(const void* W, const float* x, float* y,
             int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* As qmv_q4_0 for Q8_0 weights.
 * [roadmap K1: Q8_0 dequantization, matrix-vector; K2 step 6: Q8_0
 *  embedding/output projection] */
int qmv_q8_0(const void* W, const float* x, float* y,
             int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* As qmv_q4_0 for Q4_K weights (K % 256 == 0).
 * [captable section 1: q4k_matvec, Q4_K 144 B x f32] */
int qmv_q4_k(const void* W, const float* x, float* y,
             int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* As qmv_q4_0 for Q6_K weights (K % 256 == 0).  W must be 16-byte aligned
 * like every weight buffer; the 210-byte super-blocks inside it are read at
 * their 2-byte alignment.
 * [captable section 1: q6k_matvec, Q6_K 210 B planar x f32] */
int qmv_q6_k(const void* W, const float* x, float* y,
             int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* As qmv_q4_0 for MXFP4 weights held in two planes:
 *   W_codes  [N][K/32][16 B]: 32 E2M1 elements per block, element 2i in the
 *            low and 2i+1 in the high nibble of byte i (E2M1: sign, two
 *            exponent bits with bias 1, one mantissa bit; values
 *            +-{0, 0.5, 1, 1.5, 2, 3, 4, 6});
 *   W_scales [N][K/32]: one E8M0 byte e per block, scale 2^(e - 127)
 *            (e = 255 is NaN and makes the row's output NaN);
 *   w = E2M1(code) * 2^(e - 127).  K % 32 == 0; both planes 16-byte
 *   aligned.  The codes are converted with gfx950's packed FP4 conversion.
 * [captable section 1: mxfp4_matvec, 16 code bytes per 32 weights with the
 *  E8M0 scales held outside the blocks; roadmap K5: the next weight layout
 *  should decode with the hardware's packed conversions] */
int qmv_mxfp4(const void* W_codes, const void* W_scales, const float* x, float* y,
              int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* Gated GELU projection pair: h[m][n] = gelu(g) * u with g = W_gate x[m],
 * u = W_up x[m], both Q4_0 [N][K], gelu the tanh form
 * v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).  Both matrices are read
 * in one launch.
 * [roadmap K1: GELU-gated FFN; K2 step 5: the FFN's gate and up projections;
 *  captable section 4: q4k_ffn_gate_up (two matrices, one dispatch) and
 *  geglu_gelu_tanh] */
int qmv_q4_0_geglu(const void* W_gate, const void* W_up, const float* x, float* h,
                   int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* Down projection of a gated FFN with the GELU gate folded into its input:
 *   y[m][n] = sum_k w[n][k] * h[m][k],  h[m][k] = gelu(g[m][k]) * u[m][k],
 * gelu the tanh form above, h formed in float32 while the activations are
 * staged (never written to memory).  g and u: float32 [M][K], the gate and
 * up projections' outputs; W_down: [N][K] in the format of the name
 * (K % 256 == 0 for Q4_K and Q6_K).  Long rows (K > 16128, e.g. the
 * 21504-wide FFN down projection) split K across the waves of a workgroup
 * and add the slices in a fixed order.
 * [captable section 4: q4k_geglu_gelu_tanh_down, q6k_geglu_gelu_tanh_down
 *  (GELU-tanh product fused into the down projection); roadmap K2 step 5:
 *  gated GELU FFN] */
int qmv_q4_0_geglu_down(const void* W_down, const float* g, const float* u, float* y,
                        int64_t N, int64_t K, int64_t M, hipStream_t stream);
int qmv_q4_k_geglu_down(const void* W_down, const float* g, const float* u, float* y,
                        int64_t N, int64_t K, int64_t M, hipStream_t stream);
int qmv_q6_k_geglu_down(const void* W_down, const float* g, const float* u, float* y,
                        int64_t N, int64_t K, int64_t M, hipStream_t stream);

/* The attention input projections of a Q4_K_M model in one launch:
 *   q[m] = Wq x[m], k[m] = Wk x[m] (Q4_K, [Nq][K] and [Nk][K]),
 *   v[m] = Wv x[m] (Q6_K, [Nv][K]),
 * outputs float32 [M][Nq], [M][Nk], [M][Nv].  K % 256 == 0.  Each output
 * row is the same product qmv_q4_k / qmv_q6_k form for that row.
 * Rows longer than 16128 weights take one launch per matrix.
 * [captable section 2: q4k_q6k_qkv_proj, Q and K in Q4_K with V in Q6_K in one
 *  dispatch, and the route that selects it for the (Q4_K, Q4_K, Q6_K) mix;
 *  finding F2: a QKV route must honour V's own format] */
int qmv_q4_k_q6_k_qkv(const void* Wq, const void* Wk, const void* Wv, const float* x,
                      float* q, float* k, float* v, int64_t Nq, int64_t Nk, int64_t Nv,
                      int64_t K, int64_t M, hipStream_t stream);

/* Q4_0 weights times Q8-quantized activations, y float32 [M][N].
 * Step 1 quantizes each 32-element block of x (float32 arithmetic):
 *   amax = max|x|, d_x = amax / 127 (IEEE division),
 *   q = clamp(round_half_away_from_zero(x / d_x), -127, 127),
 *   amax == 0 -> d_x = 0 and q = 0;
 * the int8 codes and scales go to the workspace.  Step 2 forms the exact
 * int32 block sums isum = sum_j (q_w - 8) * q_x with integer dot products
 * (v_dot4 for M == 1, int8 MFMA for M >= 2) and accumulates
 * y += isum * d_w * d_x in float32.
 * Activations must be finite.
 * [captable section 1: q4_matvec_v4, Q4_0 x Q8 int8 + scales; section 2:
 *  quantize_q8; roadmap K3: batched Q4_0 matrix-matrix kernels for prefill]
 * ws: device buffer of at least qmm_q4_0_q8act_ws_bytes(N, K, M) bytes,
 * 16-byte aligned, contents overwritten.  It holds the int8 codes and
 * scales of x (rows padded to the kernel's tile height) and, when the
 * contraction splits K across workgroups (small M, or the last tiles of a
 * large grid shared out in K chunks so that every CU gets the same work),
 * the float32 partial sums.  The size depends on (N, K, M) only; 0 means an
 * invalid shape. */
size_t qmm_q4_0_q8act_ws_bytes(int64_t N, int64_t K, int64_t M);
int qmm_q4_0_q8act(const void* W, const float* x, float* y,
                   int64_t N, int64_t K, int64_t M,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Q4_0 weights times float32 activations for a few rows at once (small M:
 * the fixed-eight verifier batch and the 32-row prefill tile), reading the
 * weights once for all rows.  y float32 [M][N] = sum_k w[n][k] x[m][k], to
 * the same float32 accuracy as qmv_q4_0; the activations are NOT quantized.
 * Method: every 32-element block of a row is scaled by a power of two s
 * (its largest magnitude into [2^14, 2^15)) and split into two float16
 * terms hi + lo (hi = f16(x / s), lo = f16(x / s - hi)); the block products
 * (q - 8) * hi and (q - 8) * lo are formed by float16 MFMA with float32
 * sums and rescaled by d_w * s in float32.  M == 1 and K % 256 != 0 run the
 * float32 matrix-vector kernels row by row instead.
 * Activations must be finite.
 * [roadmap K3: batched Q4_0 matrix-matrix kernels, the 64 x 32 prefill MMA;
 *  K5: the fixed-eight Q4_0 verifier; batches below eight used the
 *  matrix-vector kernel there]
 * ws: device buffer of at least qmm_q4_0_f32act_ws_bytes(N, K, M) bytes,
 * 16-byte aligned, contents overwritten.  It holds the split activations
 * and scales (rows padded to the tile height) and, when K is split across
 * workgroups, the float32 partial sums.  The size depends on (N, K, M)
 * only; 0 means an invalid shape. */
size_t qmm_q4_0_f32act_ws_bytes(int64_t N, int64_t K, int64_t M);
int qmm_q4_0_f32act(const void* W, const float* x, float* y,
                    int64_t N, int64_t K, int64_t M,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Logit projection over a Q8_0 tied embedding, soft-cap and top-k.
 *   y[m][n] = sum_k w[n][k] x[m][k]                (float32)
 *   z = softcap * tanh(y / softcap)
 *   top_idx[m][0..k) = indices of the k largest y[m][.], largest first,
 *     equal values -> lower index first, NaN after all numbers;
 *   top_val[m][i] = z[m][top_idx[m][i]].
 * Ranking uses y: the cap is strictly increasing, so it selects the same
 * set, and ranking after the cap would let float32 saturation near the cap
 * decide it.  1 <= k <= min(N, 64); softcap finite and > 0.
 * [roadmap K1: logit soft-capping; K2 step 6: Q8_0 output projection and
 *  on-GPU top-k reduction; captable section 6: f32_topk_partial, a
 *  two-phase partial/fan-in top-k]
 * ws: device buffer of at least logits_topk_ws_bytes(N, M, k) bytes,
 * 16-byte aligned, contents overwritten (it holds y). */
size_t logits_topk_ws_bytes(int64_t N, int64_t M, int32_t k);
int logits_topk(const void* W_q8_0, const float* x, float* top_val, int32_t* top_idx,
                int64_t N, int64_t K, int64_t M, int32_t k, float softcap,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* logits_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results, with the workspace taken from
 * a fixed device array inside the library instead of a caller's buffer.
 * The array holds QMV_STATIC_SCRATCH_BYTES (8 MiB); each GPU that runs the
 * library has its own copy, kept until the process ends.  A call needs
 * logits_topk_ws_bytes(N, M, k) <= QMV_STATIC_SCRATCH_BYTES (a 262,144-entry
 * vocabulary: up to 7 rows at k = 10, 5 at k = 64), else it returns
 * QMV_ERR_WORKSPACE and launches nothing; QMV_ERR_LAUNCH also if the runtime
 * cannot give the array's address.  No call allocates or frees memory.
 * Every call on one GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (on different streams, or from different host threads)
 * race and must be ordered by the caller.  Nothing in the array needs to
 * start at zero (each call writes every byte it reads), and it keeps the last
 * call's logits until the next call. */
#define QMV_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
int logits_topk_noalloc(const void* W_q8_0, const float* x, float* top_val, int32_t* top_idx,
                        int64_t N, int64_t K, int64_t M, int32_t k, float softcap, hipStream_t stream);

/* Token selection on the device after the logit projection: logits_topk,
 * then one draw per row from the k selected pairs.
 *   w_i = exp((top_val[m][i] - top_val[m][0]) / temperature), i < k
 *         (NaN values weigh 0);
 *   nucleus[m] = the smallest n >= 1 with w_0 + ... + w_{n-1} >= top_p * (w_0 + ... + w_{k-1});
 *   token[m] = top_idx[m][j] for the first j < n with
 *         w_0 + ... + w_j > u[m] * (w_0 + ... + w_{n-1})   (j = n - 1 if none);
 * all in float32, the prefix sums in one fixed order, so the draw is a
 * deterministic function of u.  u: device float32 [M], each in [0, 1), from
 * the caller's generator.  temperature > 0 and finite, 0 < top_p <= 1.
 * top_val / top_idx receive the k pairs as in logits_topk.
 * [roadmap K5: top-k40 / top-p tokens selected on the device after the tied
 *  output projection, with a (value, token) frontier]
 * ws: as logits_topk (logits_topk_ws_bytes(N, M, k) bytes). */
int logits_sample(const void* W_q8_0, const float* x, const float* u, int32_t* token, int32_t* nucleus,
                  float* top_val, int32_t* top_idx, int64_t N, int64_t K, int64_t M, int32_t k, float softcap,
                  float temperature, float top_p, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- diagnostics: expose intermediate results of the paths above so
 * that tests can check them bit for bit ---- */

/* Step 1 of qmm_q4_0_q8act alone: q int8 [M][K], d float32 [M][K/32]. */
int qmvdbg_quantize_q8(const float* x, int8_t* q, float* d,
                       int64_t K, int64_t M, hipStream_t stream);

/* The integer block sums of qmm_q4_0_q8act, from the launches that
 * qmm_q4_0_q8act(W, x, y, N, K, M, ws, ws_bytes) makes: the same
 * quantization of x into ws, the same kernel (v_dot4 for M == 1, the narrow
 * or the wide int8 MFMA tiling for M >= 2, chosen by (N, K, M) alone) on the
 * same grid, with the float epilogue y += isum * d_w * d_x replaced by a
 * store of the exact block sums of the rows n0 <= n < n1:
 *   isum[m][n - n0][b] = sum_{j < 32} (q_w[n][32 b + j] - 8) * q_x[m][32 b + j]
 * (int32 [M][n1 - n0][K/32]).  y is not written.  0 <= n0 < n1 <= N, else
 * QMV_ERR_ARG; other arguments and errors as qmm_q4_0_q8act.
 * [captable section 1: q4_matvec_v4, Q4_0 x Q8 int8 block dot products;
 *  roadmap K3: batched Q4_0 matrix-matrix prefill] */
int qmvdbg_qmm_q4_0_q8act_blocksums(const void* W, const float* x, int32_t* isum,
                                    int64_t N, int64_t K, int64_t M, int64_t n0, int64_t n1,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* The top-k stages of logits_topk on a given float32 vector y [M][N]:
 * same ordering rule, values returned as softcap * tanh(y / softcap). */
int qmvdbg_topk_f32(const float* y, float* top_val, int32_t* top_idx,
                    int64_t N, int64_t M, int32_t k, float softcap,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* The draw of logits_sample alone, on given sorted pairs top_val / top_idx
 * [M][k] (k <= 64). */
int qmvdbg_sample_f32(const float* top_val, const int32_t* top_idx, const float* u,
                      int32_t* token, int32_t* nucleus, int64_t M, int32_t k,
                      float temperature, float top_p, hipStream_t stream);

/* A plain streaming read, the measured ceiling for the kernels above: reads
 * the `bytes` bytes at p (a multiple of 16, p 16-byte aligned) once with
 * coalesced 16-byte loads (each wave a contiguous 4 KB chunk per round), on
 * a grid of `workgroups` 256-thread workgroups.
 * out[w], w < workgroups, receives the XOR of the 32-bit words that
 * workgroup w read (0 if none), so the XOR of out[0 .. workgroups) is the
 * XOR of the whole buffer.  out must hold `workgroups` words.
 * Errors: NULL pointers -> QMV_ERR_NULL; bytes < 16 or not a multiple of
 * 16 -> QMV_ERR_SHAPE; workgroups outside [1, 65536] -> QMV_ERR_ARG;
 * misaligned p or out -> QMV_ERR_ALIGN.
 * [roadmap K5: the tied output projection is judged against the
 *  sustainable memory-streaming rate, which this read measures on MI355X] */
int qmvdbg_stream_read(const void* p, int64_t bytes, uint32_t* out, int32_t workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
