// internal.h -- launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8bs {

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
hipError_t launch_quant_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt, float* st,
                                   hipStream_t stream);
hipError_t launch_quant_dual(const uint16_t* x, int64_t M, int64_t C, uint8_t* q, float* s,
                             uint8_t* qt, float* st, hipStream_t stream);
hipError_t launch_encode_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream);

// C[I, J] = sum_kb sA(i,kb) sB(j,kb) sum_{k in kb} dec(A[i][k]) dec(B[j][k]);
// A [I, Kc], B [J, Kc] codes, contraction contiguous.  out_bf16 selects the
// output dtype.  workspace (nullable) enables a split of the contraction.
hipError_t launch_gemm(ScaleMode mode, const uint8_t* A, const float* sA, const uint8_t* B,
                       const float* sB, void* C, bool out_bf16, int64_t I, int64_t J, int64_t Kc,
                       void* workspace, size_t workspace_bytes, int num_cus, hipStream_t stream);

size_t gemm_workspace_bytes(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus);

// As launch_gemm with BF16 output (C, nullable), plus the output quantized in
// 1x128 row tiles: codes Cq [I, J], scales Cs [I, J/128].  Modes kScaleBlock
// and kScaleBlockT; 256x256 kernel, no split.
hipError_t launch_gemm_quantized(ScaleMode mode, const uint8_t* A, const float* sA,
                                 const uint8_t* B, const float* sB, uint16_t* C, uint8_t* Cq,
                                 float* Cs, int64_t I, int64_t J, int64_t Kc, hipStream_t stream);

// C[I, J] = A B^T with A [I, K], B [J, K] BF16 (unquantized comparator).
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, bool out_bf16,
                            int64_t I, int64_t J, int64_t K, hipStream_t stream);

// Diagnostic: blocks x 256 threads of MFMA-only work (see mfma_rate_kernel).
hipError_t launch_mfma_rate(float* out, int64_t blocks, int iters, float v, hipStream_t stream);

}  // namespace fp8bs
