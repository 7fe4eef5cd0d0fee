// gemm.hip -- block-scaled FP8 GEMM core for gfx950 (fprop, dgrad, wgrad).
//
// Puro-2B technical report, section 2 "FP8": the main linear layers' matmuls
// run in FP8 on block-quantized operands, with accumulation kept in FP32.
// Every GEMM here has the "TN" form
//     C[i][j] = sum_kb sA(i,kb) * sB(j,kb) * P(i,j,kb),
//     P(i,j,kb) = sum_{k in block kb} dec(A[i][k]) * dec(B[j][k]),
// with A [I, Kc] and B [J, Kc] holding E4M3 codes, contraction contiguous.
//
// Accumulation precision.  gfx950's FP8 MFMA instructions add their products
// in groups of eight consecutive K with a fixed-point window of about 13-14
// bits below the group's largest product (smaller products are truncated
// toward zero); on N(0,1)-like tiles that is a relative error of ~1.5e-5 per
// block sum, far from FP32.  Every E4M3 value is exact in FP16, and the FP16
// MFMA accumulates its products at FP32 precision, so the codes are widened
// to FP16 in registers (v_cvt_scalef32_pk_f16_fp8, scale 1) and contracted
// with v_mfma_f32_16x16x32_f16: four chained instructions give P for one
// 128-wide block in FP32, which is folded into the FP32 accumulator with one
// FMA per output element (acc += P * sA*sB).
//
// Workgroup tile 128 (i) x 128 (j) x 128 (k), four waves in a 2x2 grid, each
// wave a 64x64 patch of 4x4 MFMA tiles.  FP8 tiles are staged in LDS (double
// buffered, 16-byte chunks XOR-swizzled by row so the fragment reads are
// bank-conflict free); the next block's global loads are issued before the
// current block's MFMAs.  The MFMA operands are swapped (B tile as the first
// source) so that each lane owns four consecutive output columns of one row
// and stores them as one vector.
#include "device_common.h"
#include "internal.h"

namespace fp8bs {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Eight E4M3 codes (two dwords) -> eight FP16 values, exactly.
__device__ __forceinline__ v8h widen8(uint32_t lo, uint32_t hi) {
    v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kBK + ((chunk ^ (row & 7)) << 4);
}

template <int MODE, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemm_bs_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ C, int64_t I, int64_t J, int64_t Kc,
    int tiles_j) {
    __shared__ __align__(16) uint8_t As[2][kBM * kBK];
    __shared__ __align__(16) uint8_t Bs[2][kBN * kBK];
    __shared__ float sAs[2][kBM];
    __shared__ float sBs[2][kBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave & 1, wj = wave >> 1;
    const int ti = blockIdx.x / tiles_j, tj = blockIdx.x % tiles_j;
    const int64_t i0 = (int64_t)ti * kBM, j0 = (int64_t)tj * kBN;
    const int nkb = (int)(Kc / kBK);
    const int64_t jb_count = J / kBN;

    // global -> register staging (4 chunks of A and 4 of B per thread)
    uint4 ra[4], rb[4];
    float rsa = 0.f, rsb = 0.f;
    const uint8_t* a_rows[4];
    const uint8_t* b_rows[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int id = q * kThreads + tid;
        int row = id >> 3, c = id & 7;
        int64_t gi = min(i0 + row, I - 1);
        a_rows[q] = A + gi * Kc + c * 16;
        b_rows[q] = B + (j0 + row) * Kc + c * 16;
    }
    const float* sa_ptr = sA + min(i0 + (tid & 127), I - 1) * nkb;

    auto load_global = [&](int kb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ra[q] = *reinterpret_cast<const uint4*>(a_rows[q] + (int64_t)kb * kBK);
            rb[q] = *reinterpret_cast<const uint4*>(b_rows[q] + (int64_t)kb * kBK);
        }
        if (tid < 128) {
            rsa = sa_ptr[kb];
        } else {
            if (MODE == kScaleRow)
                rsb = sB[(j0 + (tid - 128)) * nkb + kb];
            else if (MODE == kScaleBlock)
                rsb = sB[(int64_t)tj * nkb + kb];
            else
                rsb = sB[(int64_t)kb * jb_count + tj];
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int id = q * kThreads + tid;
            int row = id >> 3, c = id & 7;
            *reinterpret_cast<uint4*>(&As[buf][swz(row, c)]) = ra[q];
            *reinterpret_cast<uint4*>(&Bs[buf][swz(row, c)]) = rb[q];
        }
        if (tid < 128)
            sAs[buf][tid] = rsa;
        else
            sBs[buf][tid - 128] = rsb;
    };

    v4f acc[4][4];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[it][jt] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int g = lane >> 4;

    if (nkb > 0) {
        load_global(0);
        store_lds(0);
        __syncthreads();
    }
    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nkb) load_global(kb + 1);

        // raw codes: lane (r16, g) holds bytes [32g, 32g+32) of row r16 of a 16-row subtile
        uint4 a_lo[4], a_hi[4], b_lo[4], b_hi[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            int row = wi * 64 + it * 16 + r16;
            a_lo[it] = *reinterpret_cast<const uint4*>(&As[buf][swz(row, 2 * g)]);
            a_hi[it] = *reinterpret_cast<const uint4*>(&As[buf][swz(row, 2 * g + 1)]);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            int row = wj * 64 + jt * 16 + r16;
            b_lo[jt] = *reinterpret_cast<const uint4*>(&Bs[buf][swz(row, 2 * g)]);
            b_hi[jt] = *reinterpret_cast<const uint4*>(&Bs[buf][swz(row, 2 * g + 1)]);
        }
        // FP16 fragments: chunk c (0..3) of a lane is bytes [8c, 8c+8) of its 32 bytes;
        // A and B use the same byte -> K assignment, so each 4-MFMA chain sums the
        // whole 128-wide block.
        v8h af[4][4], bfr[4][4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            af[it][0] = widen8(a_lo[it].x, a_lo[it].y);
            af[it][1] = widen8(a_lo[it].z, a_lo[it].w);
            af[it][2] = widen8(a_hi[it].x, a_hi[it].y);
            af[it][3] = widen8(a_hi[it].z, a_hi[it].w);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            bfr[jt][0] = widen8(b_lo[jt].x, b_lo[jt].y);
            bfr[jt][1] = widen8(b_lo[jt].z, b_lo[jt].w);
            bfr[jt][2] = widen8(b_hi[jt].x, b_hi[jt].y);
            bfr[jt][3] = widen8(b_hi[jt].z, b_hi[jt].w);
        }
        float sa[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) sa[it] = sAs[buf][wi * 64 + it * 16 + r16];
        if (MODE != kScaleRow) {
            const float sb = sBs[buf][0];
#pragma unroll
            for (int it = 0; it < 4; ++it) sa[it] = sa[it] * sb;
        }
        float sbv[4][4];
        if (MODE == kScaleRow) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int v = 0; v < 4; ++v) sbv[jt][v] = sBs[buf][wj * 64 + jt * 16 + 4 * g + v];
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                // D[j][i] with j = 4g+v (rows of the B subtile), i = r16 (rows of the A subtile)
                v4f p = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfr[jt][c], af[it][c], p, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float c = (MODE == kScaleRow) ? sa[it] * sbv[jt][v] : sa[it];
                    acc[it][jt][v] = __builtin_fmaf(p[v], c, acc[it][jt][v]);
                }
            }
        }
        if (kb + 1 < nkb) store_lds(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane owns C[i][j .. j+3]
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        int64_t i = i0 + wi * 64 + it * 16 + r16;
        if (i >= I) continue;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            int64_t j = j0 + wj * 64 + jt * 16 + 4 * g;
            if (OUT_BF16) {
                uint16_t* Cb = reinterpret_cast<uint16_t*>(C);
                uint2 pk;
                pk.x = f32_to_bf16_rne(acc[it][jt][0]) | (f32_to_bf16_rne(acc[it][jt][1]) << 16);
                pk.y = f32_to_bf16_rne(acc[it][jt][2]) | (f32_to_bf16_rne(acc[it][jt][3]) << 16);
                *reinterpret_cast<uint2*>(Cb + i * J + j) = pk;
            } else {
                float* Cf = reinterpret_cast<float*>(C);
                *reinterpret_cast<float4*>(Cf + i * J + j) =
                    make_float4(acc[it][jt][0], acc[it][jt][1], acc[it][jt][2], acc[it][jt][3]);
            }
        }
    }
}

template <int MODE, bool BF16>
static hipError_t launch_t(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                           void* C, int64_t I, int64_t J, int64_t Kc, hipStream_t stream) {
    int64_t tiles_i = (I + kBM - 1) / kBM;
    int64_t tiles_j = J / kBN;
    int64_t blocks = tiles_i * tiles_j;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_bs_fp8_kernel<MODE, BF16>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, A, sA, B, sB, C, I, J, Kc, (int)tiles_j);
    return hipGetLastError();
}

size_t gemm_workspace_bytes(ScaleMode, int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemm(ScaleMode mode, const uint8_t* A, const float* sA, const uint8_t* B,
                       const float* sB, void* C, bool out_bf16, int64_t I, int64_t J, int64_t Kc,
                       void*, size_t, int, hipStream_t stream) {
    switch (mode) {
        case kScaleBlock:
            return out_bf16 ? launch_t<kScaleBlock, true>(A, sA, B, sB, C, I, J, Kc, stream)
                            : launch_t<kScaleBlock, false>(A, sA, B, sB, C, I, J, Kc, stream);
        case kScaleBlockT:
            return out_bf16 ? launch_t<kScaleBlockT, true>(A, sA, B, sB, C, I, J, Kc, stream)
                            : launch_t<kScaleBlockT, false>(A, sA, B, sB, C, I, J, Kc, stream);
        case kScaleRow:
            return out_bf16 ? launch_t<kScaleRow, true>(A, sA, B, sB, C, I, J, Kc, stream)
                            : launch_t<kScaleRow, false>(A, sA, B, sB, C, I, J, Kc, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fp8bs
