// Drives the C ABI's host-side argument checking (qmv_api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers
// replaced by stubs that record their arguments and launch nothing.  Built and
// run by tests/test_native_sanitizers.py (host code only, no GPU).
// Exit status 0: every call returned the expected status and every accepted
// call reached its launcher with the expected shape.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "qmv.h"
#include "qmv_internal.h"

namespace {
int64_t g_calls = 0, g_N = -1, g_K = -1;
void rec(int64_t N, int64_t K) { ++g_calls; g_N = N; g_K = K; }
}  // namespace

namespace qmv {
int device_cus() { return 256; }
int device_max_lds() { return 163840; }
hipError_t launch_gemv(int, const void*, const void*, const float*, const float*, float*, int64_t N, int64_t K,
                       hipStream_t) { rec(N, K); return hipSuccess; }
hipError_t launch_gemv_mxfp4(const void*, const void*, const float*, float*, int64_t N, int64_t K, hipStream_t) {
    rec(N, K); return hipSuccess; }
hipError_t launch_qkv(const void*, const void*, const void*, const float*, float*, float*, float*, int64_t Nq,
                      int64_t, int64_t, int64_t K, hipStream_t) { rec(Nq, K); return hipSuccess; }
size_t topk_ws_bytes(int64_t N, int64_t M, int k) { return static_cast<size_t>(N * M * 4 + M * k * 8 * 64); }
hipError_t launch_topk(const float*, float*, int32_t*, int64_t N, int64_t, int, float, void*, hipStream_t,
                       const TopPDraw&, bool* drawn) {
    if (drawn) *drawn = false;  // so that logits_sample also reaches launch_sample
    rec(N, 0); return hipSuccess; }
void* static_scratch() { alignas(256) static unsigned char buf[4096]; return buf; }
hipError_t launch_sample(const float*, const int32_t*, const float*, int32_t*, int32_t*, int64_t M, int k, float,
                         float, hipStream_t) { rec(M, k); return hipSuccess; }
size_t qmm_ws_bytes(int64_t N, int64_t K, int64_t M) { return static_cast<size_t>(M * K * 2 + N * M * 4 + 256); }
hipError_t launch_quantize_q8(const float*, int8_t*, float*, int64_t K, int64_t M, hipStream_t) {
    rec(M, K); return hipSuccess; }
hipError_t launch_qmm_q8act(const void*, const float*, float*, int32_t*, int64_t, int64_t, int64_t N, int64_t K,
                            int64_t, void*, hipStream_t) { rec(N, K); return hipSuccess; }
size_t qmm_f32act_ws_bytes(int64_t N, int64_t K, int64_t M) { return static_cast<size_t>(M * K * 4 + N * M * 4 + 256); }
hipError_t launch_qmm_f32act(const void*, const float*, float*, int64_t N, int64_t K, int64_t, void*, hipStream_t) {
    rec(N, K); return hipSuccess; }
hipError_t launch_stream_read(const void*, int64_t bytes, uint32_t*, int workgroups, hipStream_t) {
    rec(bytes, workgroups); return hipSuccess; }
}  // namespace qmv

static int failures = 0;
#define EXPECT(expr, want) do { const int got_ = (expr); if (got_ != (want)) { \
    std::fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #expr, got_, (want)); ++failures; } } while (0)

int main() {
    alignas(16) static unsigned char W[4096], W2[4096], W3[4096], ws[1 << 16];
    alignas(16) static float x[4096], y[4096], u[4096];
    alignas(16) static int32_t idx[4096];
    const hipStream_t s = nullptr;
    const int64_t big = INT64_MAX / 2;

    // accepted shapes reach the launcher once per activation row
    g_calls = 0;
    EXPECT(qmv_q4_0(W, x, y, 8, 256, 3, s), QMV_OK);
    if (g_calls != 3 || g_N != 8 || g_K != 256) { std::fprintf(stderr, "gemv launches\n"); ++failures; }
    EXPECT(qmv_q8_0(W, x, y, 8, 96, 1, s), QMV_OK);
    EXPECT(qmv_q4_k(W, x, y, 8, 512, 1, s), QMV_OK);
    EXPECT(qmv_q6_k(W, x, y, 8, 512, 1, s), QMV_OK);
    EXPECT(qmv_mxfp4(W, W2, x, y, 8, 96, 1, s), QMV_OK);
    EXPECT(qmv_q4_0_geglu(W, W2, x, y, 8, 256, 2, s), QMV_OK);
    EXPECT(qmv_q6_k_geglu_down(W, x, u, y, 8, 512, 1, s), QMV_OK);
    EXPECT(qmv_q4_k_q6_k_qkv(W, W2, W3, x, y, y + 64, y + 128, 8, 4, 4, 512, 1, s), QMV_OK);

    // shapes, including products that overflow int64
    const int64_t Ns[] = {0, -1, 1, INT32_MAX, (int64_t{1} << 31), big};
    const int64_t Kq[] = {0, 16, 31, 33, 256, 288, (int64_t{1} << 40), big};
    const int64_t Ms[] = {0, -3, 1, (int64_t{1} << 41), big};
    for (int64_t N : Ns) for (int64_t K : Kq) for (int64_t M : Ms) {
        (void)qmv_q4_0(W, x, y, N, K, M, s);
        (void)qmv_q6_k(W, x, y, N, K, M, s);
        (void)qmv_mxfp4(W, W2, x, y, N, K, M, s);
        (void)qmv_q4_k_q6_k_qkv(W, W2, W3, x, y, y, y, N, N, N, K, M, s);
        (void)qmm_q4_0_q8act_ws_bytes(N, K, M);
        (void)qmm_q4_0_f32act_ws_bytes(N, K, M);
        (void)logits_topk_ws_bytes(N, M, 10);
        (void)logits_topk_ws_bytes(N, M, 64);
    }
    EXPECT(qmv_q4_0(W, x, y, 8, 1 << 21, int64_t{1} << 41, s), QMV_ERR_SHAPE);
    EXPECT(qmv_q4_0(W, x, y, 1, 256, 65536, s), QMV_ERR_SHAPE);  // activation rows are bounded
    g_calls = 0;
    EXPECT(qmv_q8_0(W, x, y, 1, 32, 65535, s), QMV_OK);
    if (g_calls != 65535) { std::fprintf(stderr, "row launches %lld\n", static_cast<long long>(g_calls)); ++failures; }
    EXPECT(qmv_q4_0(W, x, y, int64_t{1} << 31, 256, 1, s), QMV_ERR_SHAPE);
    EXPECT(qmv_q6_k(W, x, y, 8, 288, 1, s), QMV_ERR_SHAPE);
    EXPECT(qmv_mxfp4(W, W2, x, y, 8, 48, 1, s), QMV_ERR_SHAPE);
    EXPECT(qmv_mxfp4(W, W2 + 8, x, y, 8, 64, 1, s), QMV_ERR_ALIGN);
    EXPECT(qmv_q4_k_q6_k_qkv(W, W2, W3, x, y, y, y, 8, 0, 4, 512, 1, s), QMV_ERR_SHAPE);
    if (logits_topk_ws_bytes(big, big, 64) != 0) { std::fprintf(stderr, "ws overflow not caught\n"); ++failures; }

    // workspaces
    const size_t need = qmm_q4_0_q8act_ws_bytes(64, 256, 4);
    EXPECT(qmm_q4_0_q8act(W, x, y, 64, 256, 4, ws, need, s), QMV_OK);
    EXPECT(qmm_q4_0_q8act(W, x, y, 64, 256, 4, ws, need - 1, s), QMV_ERR_WORKSPACE);
    g_calls = 0;
    EXPECT(logits_topk_noalloc(W, x, y, idx, 100, 64, 2, 10, 30.0f, s), QMV_OK);
    if (g_calls != 3 || g_N != 100) { std::fprintf(stderr, "noalloc top-k launches\n"); ++failures; }
    EXPECT(logits_topk_noalloc(W, x, y, idx, 262144, 64, 8, 10, 30.0f, s), QMV_ERR_WORKSPACE);
    EXPECT(logits_topk_noalloc(W, x, y, idx, big, 64, 8, 10, 30.0f, s), QMV_ERR_SHAPE);
    EXPECT(logits_topk_noalloc(W, x, y, idx, 100, 64, 1, 0, 30.0f, s), QMV_ERR_ARG);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, idx, 64, 256, 4, 8, 24, ws, need, s), QMV_OK);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, idx, 64, 256, 4, 8, 24, ws, need - 1, s), QMV_ERR_WORKSPACE);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, idx, 64, 256, 4, 8, 8, ws, need, s), QMV_ERR_ARG);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, idx, 64, 256, 4, -1, 8, ws, need, s), QMV_ERR_ARG);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, idx, 64, 256, 4, 0, 65, ws, need, s), QMV_ERR_ARG);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, nullptr, 64, 256, 4, 0, 8, ws, need, s), QMV_ERR_NULL);
    EXPECT(qmvdbg_qmm_q4_0_q8act_blocksums(W, x, idx, 64, 256, 4, 0, 8, ws + 8, need, s), QMV_ERR_ALIGN);
    const size_t needf = qmm_q4_0_f32act_ws_bytes(64, 256, 4);
    EXPECT(qmm_q4_0_f32act(W, x, y, 64, 256, 4, ws, needf, s), QMV_OK);
    const size_t needt = logits_topk_ws_bytes(100, 2, 10);
    EXPECT(logits_topk(W, x, y, idx, 100, 256, 2, 10, 30.0f, ws, needt, s), QMV_OK);
    EXPECT(logits_topk(W, x, y, idx, 100, 256, 2, 65, 30.0f, ws, needt, s), QMV_ERR_ARG);
    EXPECT(logits_topk(W, x, y, idx, 100, 256, 2, 10, -1.0f, ws, needt, s), QMV_ERR_ARG);
    EXPECT(logits_sample(W, x, u, idx, idx + 8, y, idx + 16, 100, 256, 2, 10, 30.0f, 0.7f, 0.9f, ws, needt, s),
           QMV_OK);
    EXPECT(qmvdbg_sample_f32(y, idx, u, idx + 8, idx + 16, 2, 10, 0.7f, 0.9f, s), QMV_OK);
    EXPECT(qmvdbg_quantize_q8(x, reinterpret_cast<int8_t*>(ws), y, 256, 2, s), QMV_OK);
    g_calls = 0;
    EXPECT(qmvdbg_stream_read(W, 4096, reinterpret_cast<uint32_t*>(idx), 7, s), QMV_OK);
    if (g_calls != 1 || g_N != 4096 || g_K != 7) { std::fprintf(stderr, "stream read launch\n"); ++failures; }
    EXPECT(qmvdbg_stream_read(W, big & ~int64_t{15}, reinterpret_cast<uint32_t*>(idx), 1, s), QMV_OK);
    EXPECT(qmvdbg_stream_read(W, 4096, reinterpret_cast<uint32_t*>(idx), 0, s), QMV_ERR_ARG);
    EXPECT(qmvdbg_stream_read(W, 4095, reinterpret_cast<uint32_t*>(idx), 0, s), QMV_ERR_SHAPE);
    for (int st = -1; st < 9; ++st) (void)qmv_status_str(st);

    if (failures) { std::fprintf(stderr, "%d failures\n", failures); return 1; }
    std::printf("api host driver: ok\n");
    return 0;
}
