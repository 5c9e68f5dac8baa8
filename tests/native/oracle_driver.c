/* Runs every oracle function once on small, exactly sized buffers, so that
 * AddressSanitizer sees any access past them and UndefinedBehaviorSanitizer
 * any undefined arithmetic.  Built and run by tests/test_native_sanitizers.py.
 * Exit status 0: every call returned its success code. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_fp16_to_f64(uint16_t h);
int64_t oracle_row_bytes(int fmt, int64_t K);
int oracle_dequant_row(int fmt, const uint8_t* row, int64_t K, double* w);
int oracle_qmv(int fmt, const uint8_t* W, int64_t N, int64_t K, const float* x, int64_t M,
               const int64_t* rows, int64_t nrows, double* y, double* S);
int oracle_qmv_geglu_down(int fmt, const uint8_t* W, int64_t N, int64_t K, const float* g, const float* u,
                          int64_t M, const int64_t* rows, int64_t nrows, double* y, double* S, double* E);
int oracle_dequant_mxfp4_row(const uint8_t* codes, const uint8_t* scales, int64_t K, double* w);
int oracle_qmv_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, const float* x, int64_t M,
                     const int64_t* rows, int64_t nrows, double* y, double* S);
void oracle_geglu(const double* g, const double* u, int64_t n, double* h);
void oracle_softcap(const double* y, int64_t n, double cap, double* z);
int oracle_quantize_q8(const float* x, int64_t M, int64_t K, int8_t* q, float* d);
int oracle_q4_0_q8_blocksums(const uint8_t* W, int64_t N, int64_t K, const int8_t* qx, int64_t M,
                             const int64_t* rows, int64_t nrows, int32_t* isum);
int oracle_qmm_q4_0_q8(const uint8_t* W, int64_t N, int64_t K, const int8_t* qx, const float* dx, int64_t M,
                       const int64_t* rows, int64_t nrows, double* y, double* S);
int oracle_topk(const double* y, int64_t n, int32_t k, int32_t* out_idx);
int oracle_sample_topp(const double* z, const int32_t* idx, int32_t k, double T, double top_p, double u,
                       int32_t* token, int32_t* nucleus, double* cum);

static unsigned rnd(void) {
    static unsigned s = 12345u;
    s = s * 1103515245u + 12345u;
    return s >> 8;
}

static void* must(void* p) {
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

#define CHECK(expr) do { int rc_ = (expr); if (rc_ != 0) { fprintf(stderr, "%s -> %d\n", #expr, rc_); return 1; } } while (0)

int main(void) {
    const int64_t N = 5, M = 2;
    const int64_t Ks[5] = {96, 96, 512, 512, 96};  /* per format: Q4_0, Q8_0, Q4_K, Q6_K; MXFP4 last */
    for (int fmt = 0; fmt < 4; ++fmt) {
        const int64_t K = Ks[fmt];
        const int64_t rb = oracle_row_bytes(fmt, K);
        if (rb <= 0) { fprintf(stderr, "row bytes %d\n", fmt); return 1; }
        uint8_t* W = must(malloc((size_t)(N * rb)));
        for (int64_t i = 0; i < N * rb; ++i) W[i] = (uint8_t)rnd();
        /* fp16 scales: keep them finite (exponent field below 31) */
        float* x = must(malloc(sizeof(float) * (size_t)(M * K)));
        float* u = must(malloc(sizeof(float) * (size_t)(M * K)));
        for (int64_t i = 0; i < M * K; ++i) { x[i] = (float)((int)(rnd() % 2001) - 1000) / 250.0f; u[i] = x[i] * 0.5f; }
        double* w = must(malloc(sizeof(double) * (size_t)K));
        double* y = must(malloc(sizeof(double) * (size_t)(M * N)));
        double* S = must(malloc(sizeof(double) * (size_t)(M * N)));
        double* E = must(malloc(sizeof(double) * (size_t)(M * N)));
        const int64_t rows[3] = {4, 0, 2};
        CHECK(oracle_dequant_row(fmt, W + (N - 1) * rb, K, w));
        CHECK(oracle_qmv(fmt, W, N, K, x, M, NULL, 0, y, S));
        CHECK(oracle_qmv(fmt, W, N, K, x, M, rows, 3, y, S));
        CHECK(oracle_qmv_geglu_down(fmt, W, N, K, x, u, M, NULL, 0, y, S, E));
        if (oracle_qmv(fmt, W, N, K + 1, x, M, NULL, 0, y, S) == 0) { fprintf(stderr, "bad K accepted\n"); return 1; }
        free(W); free(x); free(u); free(w); free(y); free(S); free(E);
    }
    {
        const int64_t K = Ks[4];
        uint8_t* codes = must(malloc((size_t)(N * K / 2)));
        uint8_t* scales = must(malloc((size_t)(N * K / 32)));
        for (int64_t i = 0; i < N * K / 2; ++i) codes[i] = (uint8_t)rnd();
        for (int64_t i = 0; i < N * K / 32; ++i) scales[i] = (uint8_t)rnd();
        float* x = must(malloc(sizeof(float) * (size_t)(M * K)));
        for (int64_t i = 0; i < M * K; ++i) x[i] = (float)(i % 7) - 3.0f;
        double* w = must(malloc(sizeof(double) * (size_t)K));
        double* y = must(malloc(sizeof(double) * (size_t)(M * N)));
        double* S = must(malloc(sizeof(double) * (size_t)(M * N)));
        CHECK(oracle_dequant_mxfp4_row(codes + (N - 1) * K / 2, scales + (N - 1) * K / 32, K, w));
        CHECK(oracle_qmv_mxfp4(codes, scales, N, K, x, M, NULL, 0, y, S));
        free(codes); free(scales); free(x); free(w); free(y); free(S);
    }
    {
        const int64_t K = 64;
        float* x = must(malloc(sizeof(float) * (size_t)(M * K)));
        for (int64_t i = 0; i < M * K; ++i) x[i] = (float)((int)(rnd() % 301) - 150) / 7.0f;
        x[5] = 0.0f;
        int8_t* q = must(malloc((size_t)(M * K)));
        float* d = must(malloc(sizeof(float) * (size_t)(M * K / 32)));
        CHECK(oracle_quantize_q8(x, M, K, q, d));
        const int64_t rb = oracle_row_bytes(0, K);
        uint8_t* W = must(malloc((size_t)(N * rb)));
        for (int64_t i = 0; i < N * rb; ++i) W[i] = (uint8_t)rnd();
        int32_t* isum = must(malloc(sizeof(int32_t) * (size_t)(M * N * K / 32)));
        double* y = must(malloc(sizeof(double) * (size_t)(M * N)));
        double* S = must(malloc(sizeof(double) * (size_t)(M * N)));
        CHECK(oracle_q4_0_q8_blocksums(W, N, K, q, M, NULL, 0, isum));
        CHECK(oracle_qmm_q4_0_q8(W, N, K, q, d, M, NULL, 0, y, S));
        free(x); free(q); free(d); free(W); free(isum); free(y); free(S);
    }
    {
        const int64_t n = 100;
        double* v = must(malloc(sizeof(double) * (size_t)n));
        double* z = must(malloc(sizeof(double) * (size_t)n));
        double* h = must(malloc(sizeof(double) * (size_t)n));
        for (int64_t i = 0; i < n; ++i) v[i] = (double)((int)(rnd() % 21) - 10);
        int32_t idx[64];
        CHECK(oracle_topk(v, n, 64, idx));
        CHECK(oracle_topk(v, n, (int32_t)n > 64 ? 1 : 1, idx));
        oracle_softcap(v, n, 30.0, z);
        oracle_geglu(v, z, n, h);
        double cum[64];
        int32_t tok, nuc;
        CHECK(oracle_sample_topp(z, idx, 64, 0.7, 0.9, 0.5, &tok, &nuc, cum));
        free(v); free(z); free(h);
    }
    for (int b = 0; b < 65536; b += 97) (void)oracle_fp16_to_f64((uint16_t)b);
    printf("oracle driver: ok\n");
    return 0;
}
