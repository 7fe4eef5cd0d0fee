// capi.cpp -- the exported C ABI of libfp8bs (declared in include/fp8bs.h).
//
// Each entry point validates its arguments completely before anything is
// enqueued, then calls one launcher on the caller's stream.  The only state
// kept is a per-device record of whether the device is gfx950 and how many
// compute units it has, filled on the first call that reaches a device.
#include "../../include/fp8bs.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    std::once_flag once;
    bool supported = false;
    int num_cus = 0;
};
DeviceInfo g_devices[kMaxDevices];

fp8bs_status check_device(int* num_cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8BS_ERR_HIP;
    DeviceInfo& d = g_devices[dev];
    std::call_once(d.once, [&] {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
        d.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.num_cus = prop.multiProcessorCount;
    });
    if (!d.supported) return FP8BS_ERR_UNSUPPORTED;
    *num_cus = d.num_cus;
    return FP8BS_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool mult128(int64_t v) { return v >= 0 && v % 128 == 0; }

// Pointer must be non-NULL (unless the tensor is empty) and aligned.
fp8bs_status check_ptr(const void* p, bool empty, size_t align) {
    if (empty) return FP8BS_OK;
    if (!p) return FP8BS_ERR_NULL;
    if (!aligned(p, align)) return FP8BS_ERR_ALIGN;
    return FP8BS_OK;
}

#define FP8BS_TRY(expr)                      \
    do {                                     \
        fp8bs_status st_ = (expr);           \
        if (st_ != FP8BS_OK) return st_;     \
    } while (0)

fp8bs_status launched(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_HIP; }

}  // namespace

extern "C" {

int fp8bs_version(void) { return 200; }

const char* fp8bs_status_string(fp8bs_status status) {
    switch (status) {
        case FP8BS_OK: return "ok";
        case FP8BS_ERR_NULL: return "null pointer";
        case FP8BS_ERR_SHAPE: return "invalid shape (negative, or not a multiple of 128)";
        case FP8BS_ERR_ALIGN: return "misaligned pointer";
        case FP8BS_ERR_DTYPE: return "unknown output dtype";
        case FP8BS_ERR_WORKSPACE: return "workspace too small";
        case FP8BS_ERR_HIP: return "HIP runtime error";
        case FP8BS_ERR_UNSUPPORTED: return "unsupported device (gfx950 required)";
    }
    return "unknown status";
}

fp8bs_status fp8_quantize_rowtile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                  fp8bs_stream_t stream) {
    if (M < 0 || !mult128(K)) return FP8BS_ERR_SHAPE;
    const bool empty = (M == 0 || K == 0);
    FP8BS_TRY(check_ptr(x, empty, 16));
    FP8BS_TRY(check_ptr(q, empty, 16));
    FP8BS_TRY(check_ptr(s, empty, 4));
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_quant_rowtile(x, M, K, q, s, stream));
}

fp8bs_status fp8_quantize_block(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* q_t,
                                float* s, fp8bs_stream_t stream) {
    if (!mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    const bool empty = (N == 0 || K == 0);
    FP8BS_TRY(check_ptr(w, empty, 16));
    FP8BS_TRY(check_ptr(q, empty, 16));
    FP8BS_TRY(check_ptr(s, empty, 4));
    if (q_t && !aligned(q_t, 16)) return FP8BS_ERR_ALIGN;
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_quant_block(w, N, K, q, q_t, s, stream));
}

fp8bs_status fp8_quantize_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt,
                                     float* st, fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(C)) return FP8BS_ERR_SHAPE;
    const bool empty = (M == 0 || C == 0);
    FP8BS_TRY(check_ptr(x, empty, 16));
    FP8BS_TRY(check_ptr(qt, empty, 16));
    FP8BS_TRY(check_ptr(st, empty, 4));
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_quant_transposed(x, M, C, qt, st, stream));
}

fp8bs_status fp8_quantize_dual(const uint16_t* x, int64_t M, int64_t C, uint8_t* q, float* s,
                               uint8_t* qt, float* st, fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(C)) return FP8BS_ERR_SHAPE;
    const bool empty = (M == 0 || C == 0);
    FP8BS_TRY(check_ptr(x, empty, 16));
    FP8BS_TRY(check_ptr(q, empty, 16));
    FP8BS_TRY(check_ptr(s, empty, 4));
    FP8BS_TRY(check_ptr(qt, empty, 16));
    FP8BS_TRY(check_ptr(st, empty, 4));
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_quant_dual(x, M, C, q, s, qt, st, stream));
}

static fp8bs_status gemm_common(fp8bs::ScaleMode mode, const uint8_t* A, const float* sA,
                                const uint8_t* B, const float* sB, void* C, int yt, int64_t I,
                                int64_t J, int64_t Kc, void* workspace, size_t workspace_bytes,
                                fp8bs_stream_t stream) {
    if (yt != FP8BS_OUT_F32 && yt != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
    const bool out_empty = (I == 0 || J == 0);
    const bool in_empty = out_empty || Kc == 0;
    FP8BS_TRY(check_ptr(A, in_empty, 16));
    FP8BS_TRY(check_ptr(sA, in_empty, 4));
    FP8BS_TRY(check_ptr(B, in_empty, 16));
    FP8BS_TRY(check_ptr(sB, in_empty, 4));
    FP8BS_TRY(check_ptr(C, out_empty, 16));
    if (workspace && !aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
    if (out_empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    if (workspace && workspace_bytes > 0 &&
        workspace_bytes < fp8bs::gemm_workspace_bytes(mode, I, J, Kc, cus))
        return FP8BS_ERR_WORKSPACE;
    if (!workspace) workspace_bytes = 0;
    return launched(fp8bs::launch_gemm(mode, A, sA, B, sB, C, yt == FP8BS_OUT_BF16, I, J, Kc,
                                       workspace, workspace_bytes, cus, stream));
}

fp8bs_status fp8_gemm_fprop(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, fp8bs_out_dtype yt, int64_t M, int64_t N, int64_t K,
                            fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    return gemm_common(fp8bs::kScaleBlock, xq, xs, wq, ws, y, (int)yt, M, N, K, nullptr, 0, stream);
}

fp8bs_status fp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                            const float* ws, void* dx, fp8bs_out_dtype dxt, int64_t M, int64_t N,
                            int64_t K, fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    // TN form: rows of dY (contraction N) against rows of W^T ([K, N]).
    return gemm_common(fp8bs::kScaleBlockT, dyq, dys, wq_t, ws, dx, (int)dxt, M, K, N, nullptr, 0,
                       stream);
}

fp8bs_status fp8_gemm_dgrad_quantized(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                                      const float* ws, uint16_t* dx, uint8_t* dxq, float* dxs,
                                      int64_t M, int64_t N, int64_t K, fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    const bool out_empty = (M == 0 || K == 0);
    const bool in_empty = out_empty || N == 0;
    FP8BS_TRY(check_ptr(dyq, in_empty, 16));
    FP8BS_TRY(check_ptr(dys, in_empty, 4));
    FP8BS_TRY(check_ptr(wq_t, in_empty, 16));
    FP8BS_TRY(check_ptr(ws, in_empty, 4));
    FP8BS_TRY(check_ptr(dxq, out_empty, 16));
    FP8BS_TRY(check_ptr(dxs, out_empty, 4));
    if (dx && !aligned(dx, 16)) return FP8BS_ERR_ALIGN;
    if (out_empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    // TN form, as fp8_gemm_dgrad: rows of dY against rows of W^T, contraction N.
    return launched(fp8bs::launch_gemm_quantized(fp8bs::kScaleBlockT, dyq, dys, wq_t, ws, dx, dxq,
                                                 dxs, M, K, N, stream));
}

fp8bs_status fp8_gemm_wgrad(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                            const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    // TN form: rows of dY^T ([N, M]) against rows of X^T ([K, M]), contraction M.
    return gemm_common(fp8bs::kScaleRow, dytq, dyts, xtq, xts, dw, FP8BS_OUT_F32, N, K, M,
                       workspace, workspace_bytes, stream);
}

size_t fp8_gemm_wgrad_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return 0;
    int cus = 0;
    if (check_device(&cus) != FP8BS_OK) return 0;
    return fp8bs::gemm_workspace_bytes(fp8bs::kScaleRow, N, K, M, cus);
}

fp8bs_status bf16_gemm_tn(const uint16_t* a, const uint16_t* b, void* c, fp8bs_out_dtype ct,
                          int64_t I, int64_t J, int64_t K, fp8bs_stream_t stream) {
    if (I < 0 || !mult128(J) || !mult128(K)) return FP8BS_ERR_SHAPE;
    if ((int)ct != FP8BS_OUT_F32 && (int)ct != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
    const bool out_empty = (I == 0 || J == 0);
    const bool in_empty = out_empty || K == 0;
    FP8BS_TRY(check_ptr(a, in_empty, 16));
    FP8BS_TRY(check_ptr(b, in_empty, 16));
    FP8BS_TRY(check_ptr(c, out_empty, 16));
    if (out_empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_gemm_bf16(a, b, c, ct == FP8BS_OUT_BF16, I, J, K, stream));
}

fp8bs_status fp8_encode_e4m3(const float* x, int64_t n, uint8_t* q, fp8bs_stream_t stream) {
    if (n < 0) return FP8BS_ERR_SHAPE;
    FP8BS_TRY(check_ptr(x, n == 0, 16));
    FP8BS_TRY(check_ptr(q, n == 0, 16));
    if (n == 0) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_encode_e4m3(x, n, q, stream));
}

fp8bs_status fp8bs_mfma_rate(float* out, int64_t blocks, int iters, float v,
                             fp8bs_stream_t stream) {
    if (blocks < 0 || blocks > INT32_MAX || iters < 0) return FP8BS_ERR_SHAPE;
    FP8BS_TRY(check_ptr(out, blocks == 0, 16));
    if (blocks == 0) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_mfma_rate(out, blocks, iters, v, stream));
}

}  // extern "C"
