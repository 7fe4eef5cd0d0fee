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
// to FP16 (v_cvt_scalef32_pk_f16_fp8, scale 1) and contracted with
// v_mfma_f32_16x16x32_f16: four chained instructions give P for one 128-wide
// block in FP32, which is folded into the FP32 accumulator with one FMA per
// output element (acc += P * sA*sB).
//
// Workgroup tile 128 (i) x 128 (j) x 128 (k), four waves in a 2x2 grid, each
// wave a 64x64 patch of 4x4 MFMA tiles; two workgroups share a CU.  Each
// thread loads its share of the next block's FP8 codes into registers while
// the current block is contracted; the codes are widened to FP16 once, as
// they are stored to LDS (16-byte chunks XOR-swizzled by row so the fragment
// reads are bank-conflict free).  The MFMA operands are swapped (B tile as
// the first source) so that each lane owns four consecutive output columns of
// one row and stores them as one vector.
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
constexpr int kTileBytes = kBM * kBK;       // one FP8 operand tile: 16 KB

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of 16-byte chunk c (0..7, K = 16c .. 16c+15) of tile row r.  The
// chunk index is XORed with bits 1..3 of the row, so that the 16 lanes served
// together by a 16-byte LDS read (16 consecutive rows, one logical chunk)
// cover all 64 banks exactly once.
__device__ __forceinline__ int lds_off(int row, int c) {
    return row * kBK + ((c ^ ((row >> 1) & 7)) << 4);
}

// vmcnt(0): this wave's global loads (including those into LDS) have landed.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int MODE, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void gemm_bs_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ C, int64_t I, int64_t J, int64_t Kc,
    int tiles_j) {
    __shared__ __align__(16) uint8_t As[2][kTileBytes];
    __shared__ __align__(16) uint8_t Bs[2][kTileBytes];
    __shared__ __align__(16) float sAs[2][kBM];
    __shared__ __align__(16) float sBs[2][kBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave & 1, wj = wave >> 1;
    const int ti = blockIdx.x / tiles_j, tj = blockIdx.x % tiles_j;
    const int64_t i0 = (int64_t)ti * kBM, j0 = (int64_t)tj * kBN;
    const int nkb = (int)(Kc / kBK);
    const int64_t jb_count = J / kBN;

    // Direct global -> LDS loads: wave w fills 1 KB pieces 4w .. 4w+3 of each
    // tile (8 rows each).  Lane l lands at LDS slot l of its piece, i.e. row
    // 8*piece + l/8, physical chunk l%8, so it fetches the logical chunk that
    // the swizzle puts there.
    const uint8_t* a_src[4];
    const uint8_t* b_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int row = 8 * (4 * wave + j) + (lane >> 3);
        int c = (lane & 7) ^ ((row >> 1) & 7);
        a_src[j] = A + min(i0 + row, I - 1) * Kc + c * 16;
        b_src[j] = B + (j0 + row) * Kc + c * 16;
    }
    // Scales: waves 0/1 load the A-row scales of rows 64w + lane, waves 2/3 the
    // B scales (per row for wgrad, one block scale otherwise).
    const float* s_src;
    if (wave < 2) {
        s_src = sA + min(i0 + 64 * wave + lane, I - 1) * nkb;
    } else if (MODE == kScaleRow) {
        s_src = sB + (j0 + 64 * (wave - 2) + lane) * nkb;
    } else if (MODE == kScaleBlock) {
        s_src = sB + (int64_t)tj * nkb;
    } else {
        s_src = sB + tj;            // + kb * jb_count below
    }

    auto issue_loads = [&](int kb, int buf) {
        const int64_t koff = (int64_t)kb * kBK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_global_load_lds(a_src[j] + koff,
                                             (lds_void*)(&As[buf][(4 * wave + j) * 1024]), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(b_src[j] + koff,
                                             (lds_void*)(&Bs[buf][(4 * wave + j) * 1024]), 16, 0, 0);
        }
        const float* sp = (MODE == kScaleBlockT && wave >= 2) ? s_src + (int64_t)kb * jb_count
                                                               : s_src + kb;
        float* sdst = (wave < 2) ? &sAs[buf][64 * wave] : &sBs[buf][64 * (wave - 2)];
        __builtin_amdgcn_global_load_lds(sp, (lds_void*)sdst, 4, 0, 0);
    };

    v4f acc[4][4];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[it][jt] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int g = lane >> 4;

    if (nkb > 0) issue_loads(0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        wait_global_loads();
        __syncthreads();          // block kb is in LDS; everyone is done with buf^1
        if (kb + 1 < nkb) issue_loads(kb + 1, buf ^ 1);

        const uint8_t* At = As[buf];
        const uint8_t* Bt = Bs[buf];
        v4f p[4][4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) p[it][jt] = v4f{0.f, 0.f, 0.f, 0.f};
        // Lane (r16, g) holds bytes [32g, 32g+32) of its row of each 16-row
        // subtile, read as two 16-byte halves h.  MFMA chunk c = 2h + e takes
        // bytes [8c, 8c+8) of them for A and B alike, so the 4-instruction chain
        // covers every K of the block once.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 ar[4], br[4];
#pragma unroll
            for (int it = 0; it < 4; ++it)
                ar[it] = *reinterpret_cast<const uint4*>(At + lds_off(wi * 64 + it * 16 + r16, 2 * g + h));
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                br[jt] = *reinterpret_cast<const uint4*>(Bt + lds_off(wj * 64 + jt * 16 + r16, 2 * g + h));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                v8h af[4], bf[4];
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    af[it] = e ? widen8(ar[it].z, ar[it].w) : widen8(ar[it].x, ar[it].y);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
                    bf[jt] = e ? widen8(br[jt].z, br[jt].w) : widen8(br[jt].x, br[jt].y);
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt)
                        // D[j][i]: j = 4g+v (rows of the B subtile), i = r16 (rows of the A subtile)
                        p[it][jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[jt], af[it], p[it][jt],
                                                                            0, 0, 0);
            }
        }
        // fold: acc += P * sA(i) * sB(j)
        float sa[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) sa[it] = sAs[buf][wi * 64 + it * 16 + r16];
        if (MODE != kScaleRow) {
            const float sb = sBs[buf][0];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const float cs = sa[it] * sb;
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[it][jt][v] = __builtin_fmaf(p[it][jt][v], cs, acc[it][jt][v]);
            }
        } else {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const float4 sb = *reinterpret_cast<const float4*>(&sBs[buf][wj * 64 + jt * 16 + 4 * g]);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    acc[it][jt][0] = __builtin_fmaf(p[it][jt][0], sa[it] * sb.x, acc[it][jt][0]);
                    acc[it][jt][1] = __builtin_fmaf(p[it][jt][1], sa[it] * sb.y, acc[it][jt][1]);
                    acc[it][jt][2] = __builtin_fmaf(p[it][jt][2], sa[it] * sb.z, acc[it][jt][2]);
                    acc[it][jt][3] = __builtin_fmaf(p[it][jt][3], sa[it] * sb.w, acc[it][jt][3]);
                }
            }
        }
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
