// C ABI of libqmv.so: argument checking and dispatch.  Every check runs on
// the host before anything is enqueued; on any error nothing is launched.
// The checks follow the dispatcher contract the "Metal kernel capability
// table" (section 9) asks for: every dimension is validated when the call
// is made rather than taken for granted, no path drops part of the work
// unannounced, and cutting an input short without an error counts as a bug
// (findings F6, F13, F17 there).
#include "../../include/qmv.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "qmv_internal.h"

static_assert(qmv::kStaticScratchBytes == QMV_STATIC_SCRATCH_BYTES, "one size for the static workspace");

namespace {

constexpr int64_t kMaxN = (int64_t{1} << 31) - 1;
// Activation rows: the matrix-vector entry points launch once per row, so a
// bound keeps a mistaken M from queueing an unbounded number of launches.
constexpr int64_t kMaxM = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// a * b without int64 overflow (a, b >= 0)
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Shape rules common to every weight matrix: N rows of K weights, M rows of
// activations.  elems is the weights per block (32, or 256 for Q4_K) and
// bytes the bytes per block.
int check_shape(int64_t N, int64_t K, int64_t M, int64_t elems, int64_t bytes) {
    if (N < 1 || M < 1 || K < 32 || M > kMaxM) return QMV_ERR_SHAPE;
    if (K % 32 != 0 || K % elems != 0) return QMV_ERR_SHAPE;
    if (N > kMaxN || K > kMaxN) return QMV_ERR_SHAPE;
    int64_t t;
    if (!mul_ok(N, (K / elems) * bytes, &t)) return QMV_ERR_SHAPE;  // weight bytes
    if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t)) return QMV_ERR_SHAPE;  // activation bytes
    if (!mul_ok(M, N, &t) || !mul_ok(t, 8, &t)) return QMV_ERR_SHAPE;  // output / candidate bytes
    return QMV_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? QMV_OK : QMV_ERR_LAUNCH; }

// W_up: second matrix of the gated pair.  x_up: up activations of the gated
// input (y = W (gelu(x) * x_up)).  At most one of them is given.
int gemv(int fmt, const void* W, const void* W_up, const float* x, const float* x_up, float* y, int64_t N,
         int64_t K, int64_t M, hipStream_t stream) {
    if (!W || !x || !y) return QMV_ERR_NULL;
    const int64_t elems = (fmt >= 2) ? 256 : 32;
    const int64_t bytes = (fmt == 0) ? 18 : (fmt == 1 ? 34 : (fmt == 2 ? 144 : 210));
    int rc = check_shape(N, K, M, elems, bytes);
    if (rc) return rc;
    if (!aligned(W, 16) || (W_up && !aligned(W_up, 16)) || !aligned(x, 4) || (x_up && !aligned(x_up, 4)) ||
        !aligned(y, 4))
        return QMV_ERR_ALIGN;
    for (int64_t m = 0; m < M; ++m) {
        rc = launched(qmv::launch_gemv(fmt, W, W_up, x + m * K, x_up ? x_up + m * K : nullptr, y + m * N, N, K,
                                       stream));
        if (rc) return rc;
    }
    return QMV_OK;
}

}  // namespace

extern "C" {

const char* qmv_status_str(int status) {
    switch (status) {
    case QMV_OK: return "ok";
    case QMV_ERR_NULL: return "null pointer";
    case QMV_ERR_SHAPE: return "invalid shape (N >= 1; 1 <= M <= 65535; K >= 32, K % 32 == 0, K % 256 == 0 for Q4_K and Q6_K; no overflow)";
    case QMV_ERR_ALIGN: return "misaligned buffer (W and workspace 16 B, float/int32 buffers 4 B)";
    case QMV_ERR_WORKSPACE: return "workspace too small";
    case QMV_ERR_LAUNCH: return "kernel launch failed";
    case QMV_ERR_ARG: return "argument out of range";
    default: return "unknown status";
    }
}

int qmv_q4_0(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, hipStream_t stream) {
    return gemv(0, W, nullptr, x, nullptr, y, N, K, M, stream);
}

int qmv_q8_0(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, hipStream_t stream) {
    return gemv(1, W, nullptr, x, nullptr, y, N, K, M, stream);
}

int qmv_q4_k(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, hipStream_t stream) {
    return gemv(2, W, nullptr, x, nullptr, y, N, K, M, stream);
}

int qmv_q6_k(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, hipStream_t stream) {
    return gemv(3, W, nullptr, x, nullptr, y, N, K, M, stream);
}

int qmv_mxfp4(const void* W_codes, const void* W_scales, const float* x, float* y, int64_t N, int64_t K, int64_t M,
              hipStream_t stream) {
    if (!W_codes || !W_scales || !x || !y) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 17);  // 16 code bytes + 1 scale byte per block
    if (rc) return rc;
    if (!aligned(W_codes, 16) || !aligned(W_scales, 16) || !aligned(x, 4) || !aligned(y, 4)) return QMV_ERR_ALIGN;
    for (int64_t m = 0; m < M; ++m) {
        rc = launched(qmv::launch_gemv_mxfp4(W_codes, W_scales, x + m * K, y + m * N, N, K, stream));
        if (rc) return rc;
    }
    return QMV_OK;
}

int qmv_q4_0_geglu(const void* W_gate, const void* W_up, const float* x, float* h, int64_t N, int64_t K,
                   int64_t M, hipStream_t stream) {
    if (!W_up) return QMV_ERR_NULL;
    return gemv(0, W_gate, W_up, x, nullptr, h, N, K, M, stream);
}

int qmv_q4_0_geglu_down(const void* W_down, const float* g, const float* u, float* y, int64_t N, int64_t K, int64_t M,
                        hipStream_t stream) {
    if (!u) return QMV_ERR_NULL;
    return gemv(0, W_down, nullptr, g, u, y, N, K, M, stream);
}

int qmv_q4_k_geglu_down(const void* W_down, const float* g, const float* u, float* y, int64_t N, int64_t K, int64_t M,
                        hipStream_t stream) {
    if (!u) return QMV_ERR_NULL;
    return gemv(2, W_down, nullptr, g, u, y, N, K, M, stream);
}

int qmv_q6_k_geglu_down(const void* W_down, const float* g, const float* u, float* y, int64_t N, int64_t K, int64_t M,
                        hipStream_t stream) {
    if (!u) return QMV_ERR_NULL;
    return gemv(3, W_down, nullptr, g, u, y, N, K, M, stream);
}

int qmv_q4_k_q6_k_qkv(const void* Wq, const void* Wk, const void* Wv, const float* x, float* q, float* k, float* v,
                      int64_t Nq, int64_t Nk, int64_t Nv, int64_t K, int64_t M, hipStream_t stream) {
    if (!Wq || !Wk || !Wv || !x || !q || !k || !v) return QMV_ERR_NULL;
    int rc = check_shape(Nq, K, M, 256, 144);
    if (!rc) rc = check_shape(Nk, K, M, 256, 144);
    if (!rc) rc = check_shape(Nv, K, M, 256, 210);
    if (rc) return rc;
    if (!aligned(Wq, 16) || !aligned(Wk, 16) || !aligned(Wv, 16) || !aligned(x, 4) || !aligned(q, 4) ||
        !aligned(k, 4) || !aligned(v, 4))
        return QMV_ERR_ALIGN;
    for (int64_t m = 0; m < M; ++m) {
        rc = launched(qmv::launch_qkv(Wq, Wk, Wv, x + m * K, q + m * Nq, k + m * Nk, v + m * Nv, Nq, Nk, Nv, K,
                                      stream));
        if (rc) return rc;
    }
    return QMV_OK;
}

size_t qmm_q4_0_q8act_ws_bytes(int64_t N, int64_t K, int64_t M) {
    if (check_shape(N, K, M, 32, 18) != QMV_OK) return 0;
    return qmv::qmm_ws_bytes(N, K, M);
}

int qmm_q4_0_q8act(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
    if (!W || !x || !y || !ws) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 18);
    if (rc) return rc;
    if (!aligned(W, 16) || !aligned(x, 4) || !aligned(y, 4) || !aligned(ws, 16)) return QMV_ERR_ALIGN;
    if (ws_bytes < qmm_q4_0_q8act_ws_bytes(N, K, M)) return QMV_ERR_WORKSPACE;
    return launched(qmv::launch_qmm_q8act(W, x, y, nullptr, 0, 0, N, K, M, ws, stream));
}

size_t qmm_q4_0_f32act_ws_bytes(int64_t N, int64_t K, int64_t M) {
    if (check_shape(N, K, M, 32, 18) != QMV_OK) return 0;
    return qmv::qmm_f32act_ws_bytes(N, K, M);
}

int qmm_q4_0_f32act(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
    if (!W || !x || !y || !ws) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 18);
    if (rc) return rc;
    if (!aligned(W, 16) || !aligned(x, 4) || !aligned(y, 4) || !aligned(ws, 16)) return QMV_ERR_ALIGN;
    if (ws_bytes < qmm_q4_0_f32act_ws_bytes(N, K, M)) return QMV_ERR_WORKSPACE;
    return launched(qmv::launch_qmm_f32act(W, x, y, N, K, M, ws, stream));
}

size_t logits_topk_ws_bytes(int64_t N, int64_t M, int32_t k) {
    if (N < 1 || M < 1 || k < 1 || N > kMaxN) return 0;
    int64_t t;
    if (!mul_ok(M, N, &t) || !mul_ok(t, 8 * static_cast<int64_t>(k), &t)) return 0;
    return qmv::topk_ws_bytes(N, M, k);
}

// k, the cap and the outputs of a top-k call; then the workspace it needs
static int check_topk_params(int64_t N, int64_t M, int32_t k, float softcap, const float* top_val,
                             const int32_t* top_idx) {
    if (!top_val || !top_idx) return QMV_ERR_NULL;
    if (M > 65535) return QMV_ERR_SHAPE;
    if (k < 1 || k > 64 || k > N) return QMV_ERR_ARG;
    if (!(softcap > 0.0f) || !(softcap <= 3.4028234663852886e38f)) return QMV_ERR_ARG;
    if (!aligned(top_val, 4) || !aligned(top_idx, 4)) return QMV_ERR_ALIGN;
    if (logits_topk_ws_bytes(N, M, k) == 0) return QMV_ERR_SHAPE;
    return QMV_OK;
}

static int check_topk_args(int64_t N, int64_t M, int32_t k, float softcap, const float* top_val,
                           const int32_t* top_idx, void* ws, size_t ws_bytes) {
    if (!ws) return QMV_ERR_NULL;
    const int rc = check_topk_params(N, M, k, softcap, top_val, top_idx);
    if (rc) return rc;
    if (!aligned(ws, 16)) return QMV_ERR_ALIGN;
    if (ws_bytes < logits_topk_ws_bytes(N, M, k)) return QMV_ERR_WORKSPACE;
    return QMV_OK;
}

int logits_topk(const void* W_q8_0, const float* x, float* top_val, int32_t* top_idx, int64_t N, int64_t K,
                int64_t M, int32_t k, float softcap, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!W_q8_0 || !x) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 34);
    if (rc) return rc;
    rc = check_topk_args(N, M, k, softcap, top_val, top_idx, ws, ws_bytes);
    if (rc) return rc;
    if (!aligned(W_q8_0, 16) || !aligned(x, 4)) return QMV_ERR_ALIGN;
    float* y = static_cast<float*>(ws);
    for (int64_t m = 0; m < M; ++m) {
        rc = launched(qmv::launch_gemv(1, W_q8_0, nullptr, x + m * K, nullptr, y + m * N, N, K, stream));
        if (rc) return rc;
    }
    return launched(qmv::launch_topk(y, top_val, top_idx, N, M, k, softcap, ws, stream));
}

int logits_topk_noalloc(const void* W_q8_0, const float* x, float* top_val, int32_t* top_idx, int64_t N, int64_t K,
                        int64_t M, int32_t k, float softcap, hipStream_t stream) {
    // every check (the static workspace's size included) comes before the
    // runtime is asked for the workspace's address
    if (!W_q8_0 || !x) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 34);
    if (rc) return rc;
    rc = check_topk_params(N, M, k, softcap, top_val, top_idx);
    if (rc) return rc;
    if (logits_topk_ws_bytes(N, M, k) > qmv::kStaticScratchBytes) return QMV_ERR_WORKSPACE;
    if (!aligned(W_q8_0, 16) || !aligned(x, 4)) return QMV_ERR_ALIGN;
    void* ws = qmv::static_scratch();
    if (!ws) return QMV_ERR_LAUNCH;
    return logits_topk(W_q8_0, x, top_val, top_idx, N, K, M, k, softcap, ws, qmv::kStaticScratchBytes, stream);
}

static int check_sample_args(const float* u, const int32_t* token, const int32_t* nucleus, float temperature,
                             float top_p) {
    if (!u || !token || !nucleus) return QMV_ERR_NULL;
    if (!(temperature > 0.0f) || !(temperature <= 3.4028234663852886e38f)) return QMV_ERR_ARG;
    if (!(top_p > 0.0f) || !(top_p <= 1.0f)) return QMV_ERR_ARG;
    if (!aligned(u, 4) || !aligned(token, 4) || !aligned(nucleus, 4)) return QMV_ERR_ALIGN;
    return QMV_OK;
}

int logits_sample(const void* W_q8_0, const float* x, const float* u, int32_t* token, int32_t* nucleus,
                  float* top_val, int32_t* top_idx, int64_t N, int64_t K, int64_t M, int32_t k, float softcap,
                  float temperature, float top_p, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!W_q8_0 || !x) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 34);
    if (rc) return rc;
    rc = check_topk_args(N, M, k, softcap, top_val, top_idx, ws, ws_bytes);
    if (rc) return rc;
    rc = check_sample_args(u, token, nucleus, temperature, top_p);
    if (rc) return rc;
    if (!aligned(W_q8_0, 16) || !aligned(x, 4)) return QMV_ERR_ALIGN;
    float* y = static_cast<float*>(ws);
    for (int64_t m = 0; m < M; ++m) {
        rc = launched(qmv::launch_gemv(1, W_q8_0, nullptr, x + m * K, nullptr, y + m * N, N, K, stream));
        if (rc) return rc;
    }
    // the selection kernel makes the draw too where it can (one launch fewer)
    qmv::TopPDraw draw;
    draw.u = u;
    draw.token = token;
    draw.nucleus = nucleus;
    draw.temperature = temperature;
    draw.top_p = top_p;
    bool drawn = false;
    rc = launched(qmv::launch_topk(y, top_val, top_idx, N, M, k, softcap, ws, stream, draw, &drawn));
    if (rc || drawn) return rc;
    return launched(qmv::launch_sample(top_val, top_idx, u, token, nucleus, M, k, temperature, top_p, stream));
}

int qmvdbg_quantize_q8(const float* x, int8_t* q, float* d, int64_t K, int64_t M, hipStream_t stream) {
    if (!x || !q || !d) return QMV_ERR_NULL;
    if (K < 32 || K % 32 != 0 || M < 1 || K > kMaxN) return QMV_ERR_SHAPE;
    int64_t t;
    if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t)) return QMV_ERR_SHAPE;
    if (!aligned(x, 4) || !aligned(d, 4)) return QMV_ERR_ALIGN;
    return launched(qmv::launch_quantize_q8(x, q, d, K, M, stream));
}

int qmvdbg_qmm_q4_0_q8act_blocksums(const void* W, const float* x, int32_t* isum, int64_t N, int64_t K, int64_t M,
                                    int64_t n0, int64_t n1, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!W || !x || !isum || !ws) return QMV_ERR_NULL;
    int rc = check_shape(N, K, M, 32, 18);
    if (rc) return rc;
    if (n0 < 0 || n1 <= n0 || n1 > N) return QMV_ERR_ARG;
    int64_t t;
    if (!mul_ok(M, n1 - n0, &t) || !mul_ok(t, (K / 32) * 4, &t)) return QMV_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(x, 4) || !aligned(isum, 4) || !aligned(ws, 16)) return QMV_ERR_ALIGN;
    if (ws_bytes < qmm_q4_0_q8act_ws_bytes(N, K, M)) return QMV_ERR_WORKSPACE;
    return launched(qmv::launch_qmm_q8act(W, x, nullptr, isum, n0, n1, N, K, M, ws, stream));
}

int qmvdbg_topk_f32(const float* y, float* top_val, int32_t* top_idx, int64_t N, int64_t M, int32_t k,
                    float softcap, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!y) return QMV_ERR_NULL;
    if (N < 1 || M < 1 || N > kMaxN) return QMV_ERR_SHAPE;
    int rc = check_topk_args(N, M, k, softcap, top_val, top_idx, ws, ws_bytes);
    if (rc) return rc;
    if (!aligned(y, 4)) return QMV_ERR_ALIGN;
    return launched(qmv::launch_topk(y, top_val, top_idx, N, M, k, softcap, ws, stream));
}

int qmvdbg_sample_f32(const float* top_val, const int32_t* top_idx, const float* u, int32_t* token, int32_t* nucleus,
                      int64_t M, int32_t k, float temperature, float top_p, hipStream_t stream) {
    if (!top_val || !top_idx) return QMV_ERR_NULL;
    if (M < 1 || M > 65535) return QMV_ERR_SHAPE;
    if (k < 1 || k > 64) return QMV_ERR_ARG;
    int rc = check_sample_args(u, token, nucleus, temperature, top_p);
    if (rc) return rc;
    if (!aligned(top_val, 4) || !aligned(top_idx, 4)) return QMV_ERR_ALIGN;
    return launched(qmv::launch_sample(top_val, top_idx, u, token, nucleus, M, k, temperature, top_p, stream));
}

int qmvdbg_stream_read(const void* p, int64_t bytes, uint32_t* out, int32_t workgroups, hipStream_t stream) {
    if (!p || !out) return QMV_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0) return QMV_ERR_SHAPE;
    if (workgroups < 1 || workgroups > 65536) return QMV_ERR_ARG;
    if (!aligned(p, 16) || !aligned(out, 4)) return QMV_ERR_ALIGN;
    return launched(qmv::launch_stream_read(p, bytes, out, workgroups, stream));
}

}  // extern "C"
