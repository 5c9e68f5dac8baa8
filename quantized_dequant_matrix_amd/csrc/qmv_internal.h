// Host-side internal interface between the C ABI (qmv_api.cpp) and the
// kernel translation units.  Arguments reaching these functions have already
// been validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qmv {

// Compute units of the current device (cached per device id).
int device_cus();

// Largest dynamic LDS per workgroup of the current device (cached).
int device_max_lds();

// One matrix-vector product (one activation row).  fmt: 0 Q4_0, 1 Q8_0,
// 2 Q4_K, 3 Q6_K.  W_up != nullptr selects the gated pair (Q4_0 only):
// y = gelu(W x) * (W_up x).  x_up != nullptr selects the gated input
// (Q4_0, Q4_K, Q6_K): y = W (gelu(x) * x_up).
hipError_t launch_gemv(int fmt, const void* W, const void* W_up, const float* x, const float* x_up, float* y,
                       int64_t N, int64_t K, hipStream_t stream);

// MXFP4: code plane [N][K/32][16 B] and scale plane [N][K/32] (E8M0).
hipError_t launch_gemv_mxfp4(const void* codes, const void* scales, const float* x, float* y, int64_t N, int64_t K,
                             hipStream_t stream);

// Q and K (Q4_K) and V (Q6_K) rows of one activation row in one launch
// (K % 256 == 0; rows longer than 63 units take one launch per matrix).
hipError_t launch_qkv(const void* Wq, const void* Wk, const void* Wv, const float* x, float* yq, float* yk, float* yv,
                      int64_t Nq, int64_t Nk, int64_t Nv, int64_t K, hipStream_t stream);

// A top-p draw from the k selected pairs of each row: the caller's uniform
// numbers u[M], the drawn token and nucleus size per row.  token == nullptr:
// no draw.
struct TopPDraw {
    const float* u = nullptr;
    int32_t* token = nullptr;
    int32_t* nucleus = nullptr;
    float temperature = 1.0f;
    float top_p = 1.0f;
};

// Top-k over y[M][N] (float32), candidates in ws.  With draw.token set, the
// selection kernel also makes the draw when its path allows (*drawn = true);
// otherwise launch_sample must follow.
size_t topk_ws_bytes(int64_t N, int64_t M, int k);
hipError_t launch_topk(const float* y, float* top_val, int32_t* top_idx, int64_t N, int64_t M,
                       int k, float softcap, void* ws, hipStream_t stream, const TopPDraw& draw = TopPDraw{},
                       bool* drawn = nullptr);

// The workspace of logits_topk_noalloc: a device array of this many bytes,
// one per GPU, never allocated or freed by a call.  static_scratch() gives
// the current device's copy (its address is looked up once per device), or
// nullptr if the runtime cannot name it.
constexpr size_t kStaticScratchBytes = size_t{8} << 20;
void* static_scratch();

// One token per row from the k selected pairs (top-p with temperature, the
// caller's uniform numbers u[M]).
hipError_t launch_sample(const float* top_val, const int32_t* top_idx, const float* u, int32_t* token,
                         int32_t* nucleus, int64_t M, int k, float temperature, float top_p, hipStream_t stream);

// Q4_0 x Q8 activations.  The workspace layout (and its size) depends on
// (N, K, M) only.
size_t qmm_ws_bytes(int64_t N, int64_t K, int64_t M);
// Row-major codes [M][K] and scales [M][K/32] (step 1 alone).
hipError_t launch_quantize_q8(const float* x, int8_t* q, float* d, int64_t K, int64_t M,
                              hipStream_t stream);
// Both steps: quantize x into ws, then y = the scaled block sums.  With
// isum != nullptr the same plan, kernels and grids run with the float
// epilogue replaced by a store of the int32 block sums of rows [isn0, isn1):
// isum [M][isn1 - isn0][K/32]; y is not written.
hipError_t launch_qmm_q8act(const void* W, const float* x, float* y, int32_t* isum, int64_t isn0, int64_t isn1,
                            int64_t N, int64_t K, int64_t M, void* ws, hipStream_t stream);

// Q4_0 x float32 activations (small M).  The workspace layout (and size)
// depends on (N, K, M) only.
size_t qmm_f32act_ws_bytes(int64_t N, int64_t K, int64_t M);
hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* out, int workgroups, hipStream_t stream);
hipError_t launch_qmm_f32act(const void* W, const float* x, float* y, int64_t N, int64_t K, int64_t M,
                             void* ws, hipStream_t stream);

}  // namespace qmv
