// internal.h -- launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace fp8bs {

// A grid dimension covers at most 2^32 - 1 work-items (the HSA dispatch
// packet's grid size is a 32-bit count of work-items, not of workgroups).
constexpr uint64_t kMaxGridItems = 0xFFFFFFFFull;

// A one-dimensional grid of `blocks` workgroups.  A count past what a dim3
// holds saturates, so that launch() rejects it instead of a truncated grid
// running part of the work.
inline dim3 grid1d(int64_t blocks) {
    return dim3(blocks > (int64_t)kMaxGridItems ? (unsigned)kMaxGridItems : (unsigned)blocks);
}

// Launch kernel k on stream with the given arguments (converted to the
// kernel's parameter types) and return the status of this launch alone:
// hipLaunchKernel reports its own failure directly, so an error left behind
// by an earlier, unrelated HIP call on this thread is never returned (nor
// cleared) here.  A grid with more than kMaxGridItems work-items along a
// dimension is refused with hipErrorInvalidConfiguration before anything is
// enqueued.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    if ((uint64_t)grid.x * block.x > kMaxGridItems || (uint64_t)grid.y * block.y > kMaxGridItems ||
        (uint64_t)grid.z * block.z > kMaxGridItems)
        return hipErrorInvalidConfiguration;
    std::tuple<KArgs...> values(args...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, stream);
        },
        values);
}

// How the B operand's scale for (row j, contraction block kb) is found.
enum ScaleMode : int {
    kScaleBlock = 0,    // sB[(j/128) * nkb + kb]          weights, forward
    kScaleBlockT = 1,   // sB[kb * (J/128) + j/128]        weights read transposed, dgrad
    kScaleRow = 2       // sB[j * nkb + kb]                token-axis tiles, wgrad
};

hipError_t launch_quant_rowtile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                hipStream_t stream);
hipError_t launch_quant_block(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* q_t,
                              float* s, hipStream_t stream);
// Up to kMaxBlockJobs weights quantized by one launch (passed by value as a
// kernel argument); first[j] is the first workgroup of job j, first[count]
// the total.
constexpr int kMaxBlockJobs = 16;
struct BlockJob {
    const uint16_t* w;
    int64_t N, K;
    uint8_t* q;
    uint8_t* q_t;
    float* s;
};
struct BlockJobs {
    int count;
    int64_t first[kMaxBlockJobs + 1];
    BlockJob job[kMaxBlockJobs];
};
hipError_t launch_quant_block_many(const BlockJobs& jobs, hipStream_t stream);
hipError_t launch_quant_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt, float* st,
                                   hipStream_t stream);
hipError_t launch_quant_dual(const uint16_t* x, int64_t M, int64_t C, uint8_t* q, float* s,
                             uint8_t* qt, float* st, hipStream_t stream);
hipError_t launch_swiglu_dual(const uint16_t* gu, int64_t M, int64_t F, uint8_t* q, float* s,
                              uint8_t* qt, float* st, uint16_t* h, hipStream_t stream);
hipError_t launch_rmsnorm_dual(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                               int64_t C, uint8_t* q, float* s, uint8_t* qt, float* st,
                               float* rstd, uint16_t* y, hipStream_t stream);
hipError_t launch_swiglu_bwd_dual(const uint16_t* dh, const uint16_t* gu, int64_t M, int64_t F,
                                  uint8_t* q, float* s, uint8_t* qt, float* st, uint16_t* dgu,
                                  hipStream_t stream);
hipError_t launch_encode_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream);

// C[I, J] = sum_kb sA(i,kb) sB(j,kb) sum_{k in kb} dec(A[i][k]) dec(B[j][k]);
// A [I, Kc], B [J, Kc] codes, contraction contiguous.  out_bf16 selects the
// output dtype.  workspace (nullable) enables a split of the contraction.
hipError_t launch_gemm(ScaleMode mode, const uint8_t* A, const float* sA, const uint8_t* B,
                       const float* sB, void* C, bool out_bf16, int64_t I, int64_t J, int64_t Kc,
                       void* workspace, size_t workspace_bytes, int num_cus, hipStream_t stream);

size_t gemm_workspace_bytes(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus);

// Contraction split of the 256x256-tile kernels for this shape: `pieces`
// launches along grid y, piece 0 over blocks [0, p0), the others nps blocks
// each (split_begin / split_end); pieces == 1 when allow_split is false or a
// split does not pay.
struct GemmSplit {
    int pieces;
    int p0;
    int nps;
};
GemmSplit big_tile_split(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus,
                         bool allow_split);
// out[e] = ((out[e] + ws[0][e]) + ws[1][e]) + ..., `slices` FP32 slices of n
// elements (n a multiple of 4) after out.
hipError_t launch_splitk_reduce(const float* ws, float* out, int64_t n, int slices,
                               hipStream_t stream);

// As launch_gemm, with each block's sum P formed by gfx950's FP8 MFMA
// (v_mfma_f32_16x16x128_f8f6f4) instead of exactly: always the 256x256 tile;
// a row-scaled (kScaleRow, FP32) launch splits when workspace_bytes covers
// gemm_mfma8_workspace_bytes.
size_t gemm_mfma8_workspace_bytes(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus);
hipError_t launch_gemm_mfma8(ScaleMode mode, const uint8_t* A, const float* sA, const uint8_t* B,
                             const float* sB, void* C, bool out_bf16, int64_t I, int64_t J,
                             int64_t Kc, void* workspace, size_t workspace_bytes, int num_cus,
                             hipStream_t stream);

// C[I, J] += the kScaleRow launch_gemm result (FP32), C holding FP32 values on
// entry.  The split plan needs wgrad_accumulate_workspace_bytes (every piece,
// the first included, in the workspace); with less, the call does not split.
size_t wgrad_accumulate_workspace_bytes(int64_t I, int64_t J, int64_t Kc, int num_cus);
hipError_t launch_wgrad_accumulate(const uint8_t* A, const float* sA, const uint8_t* B,
                                   const float* sB, float* C, int64_t I, int64_t J, int64_t Kc,
                                   void* workspace, size_t workspace_bytes, int num_cus,
                                   hipStream_t stream);

// As launch_gemm with BF16 output (C, nullable), plus the output quantized in
// 1x128 row tiles: codes Cq [I, J], scales Cs [I, J/128].  Modes kScaleBlock
// and kScaleBlockT; 256x256 kernel, no split.
hipError_t launch_gemm_quantized(ScaleMode mode, const uint8_t* A, const float* sA,
                                 const uint8_t* B, const float* sB, uint16_t* C, uint8_t* Cq,
                                 float* Cs, int64_t I, int64_t J, int64_t Kc, hipStream_t stream);

// wgrad exactly as launch_gemm(kScaleRow, ...) with a workspace of
// gemm_workspace_bytes, the workspace being a static device array of
// noalloc_scratch_bytes() (noalloc.hip).  Shapes needing more set *too_big
// and launch nothing.
size_t noalloc_scratch_bytes();
hipError_t launch_wgrad_noalloc(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                                int num_cus, hipStream_t stream, bool* too_big);

// C[I, J] = A B^T with A [I, K], B [J, K] BF16 (unquantized comparator).
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, bool out_bf16,
                            int64_t I, int64_t J, int64_t K, int num_cus, hipStream_t stream);

// Diagnostic: y0[i] = high byte of x[i], y1[i] (if y1) = low byte (hbm_rate_kernel).
hipError_t launch_hbm_rate(const uint16_t* x, int64_t n, uint8_t* y0, uint8_t* y1,
                           hipStream_t stream);

// Diagnostic: blocks x 256 threads of MFMA-only work (see mfma_rate_kernel).
hipError_t launch_mfma_rate(float* out, int64_t blocks, int iters, float v, hipStream_t stream);

}  // namespace fp8bs
