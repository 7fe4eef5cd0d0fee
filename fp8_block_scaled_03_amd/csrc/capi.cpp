// capi.cpp -- the exported C ABI of libfp8bs (declared in include/fp8bs.h).
//
// Each entry point validates its arguments completely before anything is
// enqueued, then calls one launcher on the caller's stream.  The only state
// kept is a per-device record of whether the device is gfx950 and how many
// compute units it has, filled by the first call on a device whose
// properties query succeeds.
#include "../../include/fp8bs.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace {

constexpr int kMaxDevices = 64;

// Per device: 0 = not yet known, 1 = gfx950, 2 = another device.  Written
// once the properties query has succeeded; a failed query is reported as
// FP8BS_ERR_HIP and asked again on the next call.
struct DeviceInfo {
    std::atomic<int> state{0};
    std::atomic<int> num_cus{0};
};
DeviceInfo g_devices[kMaxDevices];
std::mutex g_device_mutex;

fp8bs_status check_device(int* num_cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8BS_ERR_HIP;
    DeviceInfo& d = g_devices[dev];
    int state = d.state.load(std::memory_order_acquire);
    if (state == 0) {
        std::lock_guard<std::mutex> lock(g_device_mutex);
        state = d.state.load(std::memory_order_acquire);
        if (state == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BS_ERR_HIP;
            d.num_cus.store(prop.multiProcessorCount, std::memory_order_relaxed);
            state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
            d.state.store(state, std::memory_order_release);
        }
    }
    if (state != 1) return FP8BS_ERR_UNSUPPORTED;
    *num_cus = d.num_cus.load(std::memory_order_relaxed);
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

// A launch refused for its size (more work-items along a grid dimension than
// one dispatch holds; nothing was enqueued) is a shape error; any other
// failure is the runtime's.
fp8bs_status launched(hipError_t e) {
    if (e == hipSuccess) return FP8BS_OK;
    return e == hipErrorInvalidConfiguration ? FP8BS_ERR_SHAPE : FP8BS_ERR_HIP;
}

// The integer a caller passed for an enum parameter.  A C caller may pass any
// int there; in C++ an enum object holding a value outside its enumerators'
// range may not be read as the enum, so the value is read through its object
// representation instead.
template <typename E>
int enum_value(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

}  // namespace

extern "C" {

int fp8bs_version(void) { return 300; }

const char* fp8bs_status_string(fp8bs_status status) {
    switch (enum_value(status)) {
        case FP8BS_OK: return "ok";
        case FP8BS_ERR_NULL: return "null pointer";
        case FP8BS_ERR_SHAPE: return "invalid shape (negative, or not a multiple of 128)";
        case FP8BS_ERR_ALIGN: return "misaligned pointer";
        case FP8BS_ERR_DTYPE: return "unknown output dtype";
        case FP8BS_ERR_WORKSPACE: return "workspace too small";
        case FP8BS_ERR_HIP: return "HIP runtime error";
        case FP8BS_ERR_UNSUPPORTED: return "unsupported device (gfx950 required)";
        case FP8BS_ERR_VALUE: return "scalar argument out of range";
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

static fp8bs_status check_block_job(const fp8bs_block_job& j) {
    if (!mult128(j.N) || !mult128(j.K)) return FP8BS_ERR_SHAPE;
    const bool empty = (j.N == 0 || j.K == 0);
    FP8BS_TRY(check_ptr(j.w, empty, 16));
    FP8BS_TRY(check_ptr(j.q, empty, 16));
    FP8BS_TRY(check_ptr(j.s, empty, 4));
    if (j.q_t && !aligned(j.q_t, 16)) return FP8BS_ERR_ALIGN;
    return FP8BS_OK;
}

fp8bs_status fp8_quantize_block_many(const fp8bs_block_job* jobs, int count,
                                     fp8bs_stream_t stream) {
    if (count < 0) return FP8BS_ERR_SHAPE;
    if (count > 0 && !jobs) return FP8BS_ERR_NULL;
    bool any = false;
    for (int i = 0; i < count; ++i) {
        FP8BS_TRY(check_block_job(jobs[i]));
        any = any || (jobs[i].N > 0 && jobs[i].K > 0);
    }
    if (!any) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    fp8bs::BlockJobs batch{};
    for (int i = 0; i <= count; ++i) {
        if (i == count || batch.count == fp8bs::kMaxBlockJobs) {
            if (batch.count > 0) {
                const fp8bs_status st = launched(fp8bs::launch_quant_block_many(batch, stream));
                if (st != FP8BS_OK) return st;
            }
            batch = fp8bs::BlockJobs{};
            if (i == count) break;
        }
        const fp8bs_block_job& j = jobs[i];
        if (j.N == 0 || j.K == 0) continue;
        const int c = batch.count++;
        batch.job[c] = fp8bs::BlockJob{j.w, j.N, j.K, j.q, j.q_t, j.s};
        batch.first[c + 1] = batch.first[c] + (j.N / 128) * (j.K / 128);
    }
    return FP8BS_OK;
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

fp8bs_status fp8_swiglu_quantize_dual(const uint16_t* gate_up, int64_t M, int64_t F, uint8_t* q,
                                      float* s, uint8_t* qt, float* st, uint16_t* h,
                                      fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(F)) return FP8BS_ERR_SHAPE;
    const bool empty = (M == 0 || F == 0);
    FP8BS_TRY(check_ptr(gate_up, empty, 16));
    FP8BS_TRY(check_ptr(q, empty, 16));
    FP8BS_TRY(check_ptr(s, empty, 4));
    FP8BS_TRY(check_ptr(qt, empty, 16));
    FP8BS_TRY(check_ptr(st, empty, 4));
    if (h && !aligned(h, 16)) return FP8BS_ERR_ALIGN;
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_swiglu_dual(gate_up, M, F, q, s, qt, st, h, stream));
}

fp8bs_status fp8_rmsnorm_quantize_dual(const uint16_t* x, const uint16_t* gamma, float eps,
                                       int64_t M, int64_t C, uint8_t* q, float* s, uint8_t* qt,
                                       float* st, float* rstd, uint16_t* y,
                                       fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(C)) return FP8BS_ERR_SHAPE;
    if (!(eps >= 0.0f) || !(eps <= 3.4e38f)) return FP8BS_ERR_VALUE;
    const bool empty = (M == 0 || C == 0);
    FP8BS_TRY(check_ptr(x, empty, 16));
    FP8BS_TRY(check_ptr(gamma, empty, 16));
    FP8BS_TRY(check_ptr(q, empty, 16));
    FP8BS_TRY(check_ptr(s, empty, 4));
    FP8BS_TRY(check_ptr(qt, empty, 16));
    FP8BS_TRY(check_ptr(st, empty, 4));
    FP8BS_TRY(check_ptr(rstd, empty, 4));
    if (y && !aligned(y, 16)) return FP8BS_ERR_ALIGN;
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_rmsnorm_dual(x, gamma, eps, M, C, q, s, qt, st, rstd, y, stream));
}

fp8bs_status fp8_swiglu_backward_quantize_dual(const uint16_t* dh, const uint16_t* gate_up,
                                               int64_t M, int64_t F, uint8_t* q, float* s,
                                               uint8_t* qt, float* st, uint16_t* dgate_up,
                                               fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(F)) return FP8BS_ERR_SHAPE;
    const bool empty = (M == 0 || F == 0);
    FP8BS_TRY(check_ptr(dh, empty, 16));
    FP8BS_TRY(check_ptr(gate_up, empty, 16));
    FP8BS_TRY(check_ptr(q, empty, 16));
    FP8BS_TRY(check_ptr(s, empty, 4));
    FP8BS_TRY(check_ptr(qt, empty, 16));
    FP8BS_TRY(check_ptr(st, empty, 4));
    if (dgate_up && !aligned(dgate_up, 16)) return FP8BS_ERR_ALIGN;
    if (empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_swiglu_bwd_dual(dh, gate_up, M, F, q, s, qt, st, dgate_up, stream));
}

static fp8bs_status gemm_common(fp8bs::ScaleMode mode, const uint8_t* A, const float* sA,
                                const uint8_t* B, const float* sB, void* C, int yt, int64_t I,
                                int64_t J, int64_t Kc, void* workspace, size_t workspace_bytes,
                                fp8bs_stream_t stream, bool mfma8 = false) {
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
    const size_t need = mfma8 ? fp8bs::gemm_mfma8_workspace_bytes(mode, I, J, Kc, cus)
                              : fp8bs::gemm_workspace_bytes(mode, I, J, Kc, cus);
    if (workspace && workspace_bytes > 0 && workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
    if (!workspace) workspace_bytes = 0;
    if (mfma8)
        return launched(fp8bs::launch_gemm_mfma8(mode, A, sA, B, sB, C, yt == FP8BS_OUT_BF16, I,
                                                 J, Kc, workspace, workspace_bytes, cus, stream));
    return launched(fp8bs::launch_gemm(mode, A, sA, B, sB, C, yt == FP8BS_OUT_BF16, I, J, Kc,
                                       workspace, workspace_bytes, cus, stream));
}

fp8bs_status fp8_gemm_fprop(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, fp8bs_out_dtype yt, int64_t M, int64_t N, int64_t K,
                            fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    return gemm_common(fp8bs::kScaleBlock, xq, xs, wq, ws, y, enum_value(yt), M, N, K, nullptr, 0,
                       stream);
}

fp8bs_status fp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                            const float* ws, void* dx, fp8bs_out_dtype dxt, int64_t M, int64_t N,
                            int64_t K, fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    // TN form: rows of dY (contraction N) against rows of W^T ([K, N]).
    return gemm_common(fp8bs::kScaleBlockT, dyq, dys, wq_t, ws, dx, enum_value(dxt), M, K, N,
                       nullptr, 0, stream);
}

fp8bs_status fp8_gemm_fprop_mfma8(const uint8_t* xq, const float* xs, const uint8_t* wq,
                                  const float* ws, void* y, fp8bs_out_dtype yt, int64_t M,
                                  int64_t N, int64_t K, fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    return gemm_common(fp8bs::kScaleBlock, xq, xs, wq, ws, y, enum_value(yt), M, N, K, nullptr, 0,
                       stream, true);
}

fp8bs_status fp8_gemm_dgrad_mfma8(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                                  const float* ws, void* dx, fp8bs_out_dtype dxt, int64_t M,
                                  int64_t N, int64_t K, fp8bs_stream_t stream) {
    if (M < 0 || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    return gemm_common(fp8bs::kScaleBlockT, dyq, dys, wq_t, ws, dx, enum_value(dxt), M, K, N,
                       nullptr, 0, stream, true);
}

fp8bs_status fp8_gemm_wgrad_mfma8(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                  const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                                  void* workspace, size_t workspace_bytes, fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    return gemm_common(fp8bs::kScaleRow, dytq, dyts, xtq, xts, dw, FP8BS_OUT_F32, N, K, M,
                       workspace, workspace_bytes, stream, true);
}

size_t fp8_gemm_wgrad_mfma8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return 0;
    int cus = 0;
    if (check_device(&cus) != FP8BS_OK) return 0;
    return fp8bs::gemm_mfma8_workspace_bytes(fp8bs::kScaleRow, N, K, M, cus);
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

fp8bs_status fp8_gemm_wgrad_noalloc(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                    const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                                    fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    const bool out_empty = (N == 0 || K == 0);
    const bool in_empty = out_empty || M == 0;
    FP8BS_TRY(check_ptr(dytq, in_empty, 16));
    FP8BS_TRY(check_ptr(dyts, in_empty, 4));
    FP8BS_TRY(check_ptr(xtq, in_empty, 16));
    FP8BS_TRY(check_ptr(xts, in_empty, 4));
    FP8BS_TRY(check_ptr(dw, out_empty, 16));
    if (out_empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    bool too_big = false;
    const hipError_t e =
        fp8bs::launch_wgrad_noalloc(dytq, dyts, xtq, xts, dw, M, N, K, cus, stream, &too_big);
    if (too_big) return FP8BS_ERR_WORKSPACE;
    return launched(e);
}

size_t fp8_gemm_wgrad_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return 0;
    int cus = 0;
    if (check_device(&cus) != FP8BS_OK) return 0;
    return fp8bs::gemm_workspace_bytes(fp8bs::kScaleRow, N, K, M, cus);
}

fp8bs_status fp8_gemm_wgrad_accumulate(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                       const float* xts, float* dw, int64_t M, int64_t N,
                                       int64_t K, void* workspace, size_t workspace_bytes,
                                       fp8bs_stream_t stream) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return FP8BS_ERR_SHAPE;
    const bool out_empty = (N == 0 || K == 0);
    const bool in_empty = out_empty || M == 0;
    FP8BS_TRY(check_ptr(dytq, in_empty, 16));
    FP8BS_TRY(check_ptr(dyts, in_empty, 4));
    FP8BS_TRY(check_ptr(xtq, in_empty, 16));
    FP8BS_TRY(check_ptr(xts, in_empty, 4));
    FP8BS_TRY(check_ptr(dw, out_empty, 16));
    if (workspace && !aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
    if (out_empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    if (workspace && workspace_bytes > 0 &&
        workspace_bytes < fp8bs::wgrad_accumulate_workspace_bytes(N, K, M, cus))
        return FP8BS_ERR_WORKSPACE;
    if (!workspace) workspace_bytes = 0;
    // TN form, as fp8_gemm_wgrad.
    return launched(fp8bs::launch_wgrad_accumulate(dytq, dyts, xtq, xts, dw, N, K, M, workspace,
                                                   workspace_bytes, cus, stream));
}

size_t fp8_gemm_wgrad_accumulate_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!mult128(M) || !mult128(N) || !mult128(K)) return 0;
    int cus = 0;
    if (check_device(&cus) != FP8BS_OK) return 0;
    return fp8bs::wgrad_accumulate_workspace_bytes(N, K, M, cus);
}

fp8bs_status bf16_gemm_tn(const uint16_t* a, const uint16_t* b, void* c, fp8bs_out_dtype ct,
                          int64_t I, int64_t J, int64_t K, fp8bs_stream_t stream) {
    if (I < 0 || !mult128(J) || !mult128(K)) return FP8BS_ERR_SHAPE;
    const int cv = enum_value(ct);
    if (cv != FP8BS_OUT_F32 && cv != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
    const bool out_empty = (I == 0 || J == 0);
    const bool in_empty = out_empty || K == 0;
    FP8BS_TRY(check_ptr(a, in_empty, 16));
    FP8BS_TRY(check_ptr(b, in_empty, 16));
    FP8BS_TRY(check_ptr(c, out_empty, 16));
    if (out_empty) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_gemm_bf16(a, b, c, cv == FP8BS_OUT_BF16, I, J, K, cus, stream));
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

fp8bs_status fp8bs_hbm_rate(const uint16_t* x, int64_t n, uint8_t* y0, uint8_t* y1,
                            fp8bs_stream_t stream) {
    if (n < 0) return FP8BS_ERR_SHAPE;
    FP8BS_TRY(check_ptr(x, n == 0, 16));
    FP8BS_TRY(check_ptr(y0, n == 0, 16));
    if (y1 && !aligned(y1, 16)) return FP8BS_ERR_ALIGN;
    if (n == 0) return FP8BS_OK;
    int cus;
    FP8BS_TRY(check_device(&cus));
    return launched(fp8bs::launch_hbm_rate(x, n, y0, y1, stream));
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
