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
// Two kernels share that arithmetic:
//   gemm_bs_fp8_kernel      workgroup tile 128 (i) x 128 (j) x 128 (k), four
//                           waves of 64x64, two workgroups per CU; used for
//                           wgrad (two per-row scales per fold) and for grids
//                           too small to give every CU a 256x256 tile; can
//                           split the contraction (FP32 slices in a caller
//                           workspace, summed in a fixed order).
//   gemm_bs_fp8_big_kernel  256 x 256 x 128, eight waves of 64x128, one
//                           workgroup per CU; fprop and dgrad.  Each wave
//                           widens its A fragments once per block and keeps
//                           them in registers while B fragments stream.
// Both stage the FP8 tiles of the next block in LDS with direct global->LDS
// loads (double buffered, 16-byte chunks XOR-swizzled by row so the fragment
// reads are bank-conflict free) while the current block is contracted, and
// hand out output tiles in an XCD-aware grouped order (gemm_common.h).  The
// MFMA operands are swapped (B fragment as the first source) so that each
// lane owns four consecutive output columns of one row and stores them as one
// vector.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"

namespace fp8bs {

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

template <int MODE, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void gemm_bs_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ C, int64_t I, int64_t J, int64_t Kc,
    int tiles_i, int tiles_j, int nps) {
    __shared__ __align__(16) uint8_t As[2][kTileBytes];
    __shared__ __align__(16) uint8_t Bs[2][kTileBytes];
    __shared__ __align__(16) float sAs[2][kBM];
    __shared__ __align__(16) float sBs[2][kBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave & 1, wj = wave >> 1;
    int ti, tj;
    tile_coords(blockIdx.x, tiles_i, tiles_j, &ti, &tj);
    const int64_t i0 = (int64_t)ti * kBM, j0 = (int64_t)tj * kBN;
    const int nkb_all = (int)(Kc / kBK);
    const int kb0 = blockIdx.y * nps;                 // split s: blocks [s*nps, (s+1)*nps)
    const int nkb = min(nkb_all, kb0 + nps) - kb0;
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
        s_src = sA + min(i0 + 64 * wave + lane, I - 1) * nkb_all;
    } else if (MODE == kScaleRow) {
        s_src = sB + (j0 + 64 * (wave - 2) + lane) * nkb_all;
    } else if (MODE == kScaleBlock) {
        s_src = sB + (int64_t)tj * nkb_all;
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

    if (nkb > 0) issue_loads(kb0, 0);
    for (int k = 0; k < nkb; ++k) {
        const int buf = k & 1;
        wait_global_loads();
        __syncthreads();          // this block is in LDS; everyone is done with buf^1
        if (k + 1 < nkb) issue_loads(kb0 + k + 1, buf ^ 1);

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
                pk.x = pack_bf16x2(acc[it][jt][0], acc[it][jt][1]);
                pk.y = pack_bf16x2(acc[it][jt][2], acc[it][jt][3]);
                *reinterpret_cast<uint2*>(Cb + i * J + j) = pk;
            } else {
                float* Cf = reinterpret_cast<float*>(C) + (int64_t)blockIdx.y * I * J;
                *reinterpret_cast<float4*>(Cf + i * J + j) =
                    make_float4(acc[it][jt][0], acc[it][jt][1], acc[it][jt][2], acc[it][jt][3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large-tile kernel: workgroup tile 256 (i) x 256 (j) x 128 (k), eight waves
// in a 4 (i) x 2 (j) grid, each wave a 64 x 128 patch.  A wave widens its 64
// A rows to FP16 once per block and keeps them in registers (64 VGPRs), then
// streams its eight 16-row B subtiles: per subtile it widens one 8-code chunk
// at a time and runs the 4-instruction MFMA chain for its four A subtiles, so
// 192 widenings feed 128 MFMAs (1.5 per MFMA, against 2 in the small kernel).
// Tiles are ordered for the L2s: each XCD (the hardware deals workgroups to
// the eight XCDs round-robin) gets a contiguous chunk of the tile order, and
// the order walks groups of four tile rows column by column, so the tiles an
// XCD runs together share A and B rows.  gridDim.y splits the contraction:
// split s sums blocks [s*nps, (s+1)*nps) into its own FP32 slice of C.
// ---------------------------------------------------------------------------
constexpr int kBigM = 256;
constexpr int kBigN = 256;
constexpr int kBigThreads = 512;
constexpr int kBigTile = kBigM * kBK;      // one FP8 operand tile: 32 KB
// QOUT: the epilogue also quantizes the BF16 output in 1x128 row tiles (the
// rule of quant_rowtile_kernel) and stores codes Cq [I, J] and scales
// Cs [I, J/128]; C (BF16) may then be null.  A wave's 128 output columns of a
// row are exactly one such tile, held by the four lanes r16 + 16g.
template <int MODE, bool OUT_BF16, bool QOUT = false>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_bs_fp8_big_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ C, int64_t I, int64_t J, int64_t Kc,
    int tiles_i, int tiles_j, int nps, uint8_t* __restrict__ Cq = nullptr,
    float* __restrict__ Cs = nullptr) {
    __shared__ __align__(16) uint8_t As[2][kBigTile];
    __shared__ __align__(16) uint8_t Bs[2][kBigTile];
    __shared__ __align__(16) float sAs[2][kBigM];
    __shared__ __align__(16) float sBs[2][kBigN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave & 3, wj = wave >> 2;
    int ti, tj;
    tile_coords(blockIdx.x, tiles_i, tiles_j, &ti, &tj);
    const int64_t i0 = (int64_t)ti * kBigM, j0 = (int64_t)tj * kBigN;
    const int nkb_all = (int)(Kc / kBK);
    const int kb0 = blockIdx.y * nps;
    const int kb1 = min(nkb_all, kb0 + nps);
    const int nkb = kb1 - kb0;
    const int nkb_row = nkb_all;                  // scale row stride (blocks per row)
    const int64_t jb_count = J / kBN;             // 128-wide column blocks of B

    // Direct global -> LDS loads.  Waves 0..3 fill the 32 KB A and B tiles
    // (wave w: 1 KB pieces 8w .. 8w+7, 8 rows each; lane l lands at row
    // 8*piece + l/8, physical chunk l%8 of the swizzle); waves 4..7, which
    // share SIMDs with them, only load scales and go straight on to their
    // MFMAs after each barrier.  For this lane, piece 8w + j is row
    // prow + 8j with swizzled chunk pc (j even) or pc ^ 4 (j odd).
    const int prow = 64 * (wave & 3) + (lane >> 3);
    const int pc = (lane & 7) ^ ((prow >> 1) & 7);
    // Scales: waves 0..3 load the A-row scales of rows 64w + lane, waves 4..7
    // the B scales of rows 64(w-4) + lane (per row, or their column block's).
    const float* s_src;
    int64_t s_step;                               // stride per contraction block
    if (wave < 4) {
        s_src = sA + min(i0 + 64 * wave + lane, I - 1) * nkb_row;
        s_step = 1;
    } else {
        int64_t jr = min(j0 + 64 * (wave - 4) + lane, J - 1);
        if (MODE == kScaleRow) {
            s_src = sB + jr * nkb_row;
            s_step = 1;
        } else if (MODE == kScaleBlock) {
            s_src = sB + (jr / kBN) * nkb_row;
            s_step = 1;
        } else {
            s_src = sB + jr / kBN;
            s_step = jb_count;
        }
    }

    auto issue_loads = [&](int kb, int buf) {
        const int64_t koff = (int64_t)kb * kBK;
        if (wave < 4) {
            // Recomputed per call (the empty asm hides the loop invariance):
            // sixteen precomputed 64-bit addresses would cost 32 registers.
            int pr = prow, pcc = pc;
            asm volatile("" : "+v"(pr), "+v"(pcc));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = pr + 8 * j;
                const int c = (j & 1) ? (pcc ^ 4) : pcc;
                __builtin_amdgcn_global_load_lds(A + min(i0 + row, I - 1) * Kc + koff + c * 16,
                                                 (lds_void*)(&As[buf][(8 * wave + j) * 1024]), 16,
                                                 0, 0);
                __builtin_amdgcn_global_load_lds(B + min(j0 + row, J - 1) * Kc + koff + c * 16,
                                                 (lds_void*)(&Bs[buf][(8 * wave + j) * 1024]), 16,
                                                 0, 0);
            }
        }
        float* sdst = (wave < 4) ? &sAs[buf][64 * wave] : &sBs[buf][64 * (wave - 4)];
        __builtin_amdgcn_global_load_lds(s_src + kb * s_step, (lds_void*)sdst, 4, 0, 0);
    };

    v4f acc[4][8];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int js = 0; js < 8; ++js) acc[it][js] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int g = lane >> 4;

    if (nkb > 0) issue_loads(kb0, 0);
    for (int k = 0; k < nkb; ++k) {
        const int buf = k & 1;
        wait_global_loads();
        __syncthreads();
        if (k + 1 < nkb) issue_loads(kb0 + k + 1, buf ^ 1);

        const uint8_t* At = As[buf];
        const uint8_t* Bt = Bs[buf];
        // This wave's A rows for the whole block, widened once: af[it][c] is
        // MFMA chunk c (bytes [8c, 8c+8) of the lane's 32) of subtile it.
        v8h af[4][4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = wi * 64 + it * 16 + r16;
            uint4 lo = *reinterpret_cast<const uint4*>(At + lds_off(row, 2 * g));
            uint4 hi = *reinterpret_cast<const uint4*>(At + lds_off(row, 2 * g + 1));
            af[it][0] = widen8(lo.x, lo.y);
            af[it][1] = widen8(lo.z, lo.w);
            af[it][2] = widen8(hi.x, hi.y);
            af[it][3] = widen8(hi.z, hi.w);
        }
        float sa[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) sa[it] = sAs[buf][wi * 64 + it * 16 + r16];
        if (MODE != kScaleRow) {
            const float sb = sBs[buf][128 * wj];      // the wave's 128 columns share one block scale
#pragma unroll
            for (int it = 0; it < 4; ++it) sa[it] = sa[it] * sb;
        }
#pragma unroll
        for (int js = 0; js < 8; ++js) {
            const int row = wj * 128 + js * 16 + r16;
            uint4 lo = *reinterpret_cast<const uint4*>(Bt + lds_off(row, 2 * g));
            uint4 hi = *reinterpret_cast<const uint4*>(Bt + lds_off(row, 2 * g + 1));
            v4f p[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) p[it] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w0 = c == 0 ? lo.x : c == 1 ? lo.z : c == 2 ? hi.x : hi.z;
                const uint32_t w1 = c == 0 ? lo.y : c == 1 ? lo.w : c == 2 ? hi.y : hi.w;
                const v8h bf = widen8(w0, w1);
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    p[it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[it][c], p[it], 0, 0, 0);
            }
            if (MODE != kScaleRow) {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[it][js][v] = __builtin_fmaf(p[it][v], sa[it], acc[it][js][v]);
            } else {
                const float4 sb =
                    *reinterpret_cast<const float4*>(&sBs[buf][wj * 128 + js * 16 + 4 * g]);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    acc[it][js][0] = __builtin_fmaf(p[it][0], sa[it] * sb.x, acc[it][js][0]);
                    acc[it][js][1] = __builtin_fmaf(p[it][1], sa[it] * sb.y, acc[it][js][1]);
                    acc[it][js][2] = __builtin_fmaf(p[it][2], sa[it] * sb.z, acc[it][js][2]);
                    acc[it][js][3] = __builtin_fmaf(p[it][3], sa[it] * sb.w, acc[it][js][3]);
                }
            }
        }
    }

    // epilogue: lane owns C[i][j .. j+3]; split s writes its own FP32 slice
    if constexpr (OUT_BF16) __syncthreads();   // every wave done with the LDS tiles
    if (j0 + 128 * wj >= J) return;
    if constexpr (QOUT) {
        const int64_t jt = j0 + 128 * wj;                  // first column of the row tiles
        uint8_t* stage = (wave < 4 ? &As[0][0] : &Bs[0][0]) + (wave & 3) * 16384;
        // Scales of the row tiles from the BF16-rounded values.
        float inv[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            uint32_t m = 0;
#pragma unroll
            for (int js = 0; js < 8; ++js) {
                m = absmax_pair(m, pack_bf16x2(acc[it][js][0], acc[it][js][1]));
                m = absmax_pair(m, pack_bf16x2(acc[it][js][2], acc[it][js][3]));
            }
            m = absmax_fold(m);
            m = max(m, (uint32_t)__shfl_xor((int)m, 16));
            m = max(m, (uint32_t)__shfl_xor((int)m, 32));
            const TileScale ts = tile_scale(m, &g_scale_tables);
            inv[it] = ts.inv;
            const int64_t i = i0 + wi * 64 + it * 16 + r16;
            if (g == 0 && i < I) Cs[i * (J / kTile) + jt / kTile] = ts.s;
        }
        // The BF16 copy, when asked for, then the codes: each restaged through
        // LDS and stored as whole rows (16-byte chunks XOR-swizzled by row).
        if (C) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int row = it * 16 + r16;
#pragma unroll
                for (int js = 0; js < 8; ++js) {
                    const int b = js * 32 + g * 8;
                    const int phys = (((b >> 4) ^ (row & 15)) << 4) | (b & 15);
                    *reinterpret_cast<uint2*>(stage + row * 256 + phys) =
                        make_uint2(pack_bf16x2(acc[it][js][0], acc[it][js][1]),
                                   pack_bf16x2(acc[it][js][2], acc[it][js][3]));
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): the wave's LDS writes
            __builtin_amdgcn_wave_barrier();
            uint16_t* Cb = reinterpret_cast<uint16_t*>(C);
#pragma unroll
            for (int pass = 0; pass < 16; ++pass) {
                const int row = pass * 4 + (lane >> 4);
                const int c = lane & 15;
                const uint4 w =
                    *reinterpret_cast<const uint4*>(stage + row * 256 + ((c ^ (row & 15)) << 4));
                const int64_t i = i0 + wi * 64 + row;
                if (i < I) *reinterpret_cast<uint4*>(Cb + i * J + jt + c * 8) = w;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = it * 16 + r16;
#pragma unroll
            for (int js = 0; js < 8; ++js) {
                const uint32_t p0 = pack_bf16x2(acc[it][js][0], acc[it][js][1]);
                const uint32_t p1 = pack_bf16x2(acc[it][js][2], acc[it][js][3]);
                *reinterpret_cast<uint32_t*>(stage + row * 128 + ((js ^ (row & 7)) << 4) + 4 * g) =
                    cvt4_e4m3(bf16_lo(p0) * inv[it], bf16_hi(p0) * inv[it], bf16_lo(p1) * inv[it],
                              bf16_hi(p1) * inv[it]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
            const int row = pass * 8 + (lane >> 3);
            const int c = lane & 7;                            // 16-byte chunk of the 128 codes
            const uint4 w =
                *reinterpret_cast<const uint4*>(stage + row * 128 + ((c ^ (row & 7)) << 4));
            const int64_t i = i0 + wi * 64 + row;
            if (i < I) *reinterpret_cast<uint4*>(Cq + i * J + jt + c * 16) = w;
        }
        return;
    }
    if constexpr (OUT_BF16) {
        // Restage the wave's 64x128 BF16 patch through LDS (the tiles are no
        // longer needed) so that it leaves as whole 256-byte rows in 16-byte
        // stores; 16-byte chunks are XOR-swizzled by row.
        uint8_t* stage = (wave < 4 ? &As[0][0] : &Bs[0][0]) + (wave & 3) * 16384;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = it * 16 + r16;
#pragma unroll
            for (int js = 0; js < 8; ++js) {
                const int b = js * 32 + g * 8;                 // byte offset in the row
                const int phys = (((b >> 4) ^ (row & 15)) << 4) | (b & 15);
                *reinterpret_cast<uint2*>(stage + row * 256 + phys) =
                    make_uint2(pack_bf16x2(acc[it][js][0], acc[it][js][1]),
                               pack_bf16x2(acc[it][js][2], acc[it][js][3]));
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): the wave's LDS writes
        __builtin_amdgcn_wave_barrier();
        uint16_t* Cb = reinterpret_cast<uint16_t*>(C);
#pragma unroll
        for (int pass = 0; pass < 16; ++pass) {
            const int row = pass * 4 + (lane >> 4);
            const int c = lane & 15;                           // 16-byte chunk of the row
            const uint4 w =
                *reinterpret_cast<const uint4*>(stage + row * 256 + ((c ^ (row & 15)) << 4));
            const int64_t i = i0 + wi * 64 + row;
            if (i < I) *reinterpret_cast<uint4*>(Cb + i * J + j0 + wj * 128 + c * 8) = w;
        }
        return;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int64_t i = i0 + wi * 64 + it * 16 + r16;
        if (i >= I) continue;
#pragma unroll
        for (int js = 0; js < 8; ++js) {
            const int64_t j = j0 + wj * 128 + js * 16 + 4 * g;
            if (OUT_BF16) {
                uint16_t* Cb = reinterpret_cast<uint16_t*>(C);
                uint2 pk;
                pk.x = pack_bf16x2(acc[it][js][0], acc[it][js][1]);
                pk.y = pack_bf16x2(acc[it][js][2], acc[it][js][3]);
                *reinterpret_cast<uint2*>(Cb + i * J + j) = pk;
            } else {
                float* Cf = reinterpret_cast<float*>(C) + (int64_t)blockIdx.y * I * J;
                *reinterpret_cast<float4*>(Cf + i * J + j) =
                    make_float4(acc[it][js][0], acc[it][js][1], acc[it][js][2], acc[it][js][3]);
            }
        }
    }
}

// Sum of the split slices, in split order: out[e] = sum_s ws[s][e] (fixed order,
// so the result does not depend on timing).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float4* __restrict__ ws,
                                                            float4* __restrict__ out, int64_t n4,
                                                            int splits) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    float4 a = ws[e];
    for (int s = 1; s < splits; ++s) {
        const float4 b = ws[(int64_t)s * n4 + e];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    out[e] = a;
}

template <int MODE, bool BF16>
static hipError_t launch_small(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                               void* C, int64_t I, int64_t J, int64_t Kc, int splits, int nps,
                               hipStream_t stream) {
    int64_t tiles_i = (I + kBM - 1) / kBM;
    int64_t tiles_j = J / kBN;
    int64_t blocks = tiles_i * tiles_j;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_bs_fp8_kernel<MODE, BF16>), dim3((unsigned)blocks, splits),
                       dim3(kThreads), 0, stream, A, sA, B, sB, C, I, J, Kc, (int)tiles_i,
                       (int)tiles_j, nps);
    return hipGetLastError();
}

template <int MODE, bool BF16>
static hipError_t launch_big(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                             void* C, int64_t I, int64_t J, int64_t Kc, int splits, int nps,
                             hipStream_t stream) {
    int tiles_i = (int)((I + kBigM - 1) / kBigM);
    int tiles_j = (int)((J + kBigN - 1) / kBigN);
    hipLaunchKernelGGL((gemm_bs_fp8_big_kernel<MODE, BF16>), dim3(tiles_i * tiles_j, splits),
                       dim3(kBigThreads), 0, stream, A, sA, B, sB, C, I, J, Kc, tiles_i, tiles_j,
                       nps);
    return hipGetLastError();
}

// Launch plan for one GEMM: which kernel, and how many contraction splits.
struct Plan {
    bool big;
    int splits;
    int nps;     // contraction blocks per split
};

// FP8BS_GEMM_KERNEL=small|big forces one kernel (a testing aid; the default
// "auto" picks the large tile when it yields at least one tile per CU).  Read
// on every call so a test can switch it between calls.
static int kernel_override() {
    const char* e = getenv("FP8BS_GEMM_KERNEL");
    if (!e) return 0;
    if (!strcmp(e, "small")) return 1;
    if (!strcmp(e, "big")) return 2;
    return 0;
}

static Plan plan_gemm(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus,
                      bool allow_split) {
    Plan p{false, 1, (int)(Kc / kBK)};
    const int64_t nkb = Kc / kBK;
    const int cus = num_cus > 0 ? num_cus : 256;
    const int force = kernel_override();
    if (nkb == 0) return p;
    const int64_t big_tiles = ((I + kBigM - 1) / kBigM) * ((J + kBigN - 1) / kBigN);
    const int64_t small_tiles = ((I + kBM - 1) / kBM) * (J / kBN);
    // fprop/dgrad: the 256x256 tile once it gives every CU a tile.  wgrad: the
    // 256x256 tile (with a split of the contraction) while its tiles alone
    // cannot fill the CUs; past that, the 128x128 tile, which needs no split
    // and so moves no FP32 partials through HBM (measured in the full step).
    if (force == 2) p.big = true;
    else if (force == 1) p.big = false;
    else p.big = I >= kBigM && (mode == kScaleRow ? big_tiles < cus : big_tiles >= cus);
    // Split the contraction (FP32 output only, with a caller workspace) into
    // s = 1, 2, 4, ... parts, taking the s that minimizes (full waves of
    // resident workgroups) x (contraction blocks per workgroup); ties go to
    // the smaller s, whose reduction pass is cheaper.
    if (mode == kScaleRow && allow_split) {
        const int64_t tiles = p.big ? big_tiles : small_tiles;
        const int64_t slots = p.big ? cus : 2 * cus;           // workgroups resident at once
        int best = 1;
        int64_t best_cost = -1;
        for (int s = 1; s <= 16 && nkb / s >= 4; s *= 2) {
            const int64_t cost = ((tiles * s + slots - 1) / slots) * ((nkb + s - 1) / s);
            if (best_cost < 0 || cost < best_cost) {
                best_cost = cost;
                best = s;
            }
        }
        if (best > 1) {
            p.nps = (int)((nkb + best - 1) / best);
            p.splits = (int)((nkb + p.nps - 1) / p.nps);
        }
    }
    return p;
}

size_t gemm_workspace_bytes(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus) {
    Plan p = plan_gemm(mode, I, J, Kc, num_cus, true);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)I * (size_t)J * sizeof(float);
}

template <int MODE>
static hipError_t launch_mode(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                              void* C, bool out_bf16, int64_t I, int64_t J, int64_t Kc,
                              void* workspace, size_t workspace_bytes, int num_cus,
                              hipStream_t stream) {
    const size_t need = gemm_workspace_bytes((ScaleMode)MODE, I, J, Kc, num_cus);
    const bool can_split = !out_bf16 && workspace && need > 0 && workspace_bytes >= need;
    Plan p = plan_gemm((ScaleMode)MODE, I, J, Kc, num_cus, can_split);
    if (p.splits <= 1) {
        if (p.big)
            return out_bf16 ? launch_big<MODE, true>(A, sA, B, sB, C, I, J, Kc, 1, p.nps, stream)
                            : launch_big<MODE, false>(A, sA, B, sB, C, I, J, Kc, 1, p.nps, stream);
        return out_bf16 ? launch_small<MODE, true>(A, sA, B, sB, C, I, J, Kc, 1, p.nps, stream)
                        : launch_small<MODE, false>(A, sA, B, sB, C, I, J, Kc, 1, p.nps, stream);
    }
    hipError_t e = p.big ? launch_big<MODE, false>(A, sA, B, sB, workspace, I, J, Kc, p.splits,
                                                   p.nps, stream)
                         : launch_small<MODE, false>(A, sA, B, sB, workspace, I, J, Kc, p.splits,
                                                     p.nps, stream);
    if (e != hipSuccess) return e;
    const int64_t n4 = I * J / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<const float4*>(workspace),
                       reinterpret_cast<float4*>(C), n4, p.splits);
    return hipGetLastError();
}

hipError_t launch_gemm_quantized(ScaleMode mode, const uint8_t* A, const float* sA,
                                 const uint8_t* B, const float* sB, uint16_t* C, uint8_t* Cq,
                                 float* Cs, int64_t I, int64_t J, int64_t Kc, hipStream_t stream) {
    const int tiles_i = (int)((I + kBigM - 1) / kBigM);
    const int tiles_j = (int)((J + kBigN - 1) / kBigN);
    const int nkb = (int)(Kc / kBK);
    if (tiles_i == 0 || tiles_j == 0) return hipSuccess;
    if (mode == kScaleBlockT)
        hipLaunchKernelGGL((gemm_bs_fp8_big_kernel<kScaleBlockT, true, true>),
                           dim3(tiles_i * tiles_j, 1), dim3(kBigThreads), 0, stream, A, sA, B, sB,
                           (void*)C, I, J, Kc, tiles_i, tiles_j, nkb, Cq, Cs);
    else if (mode == kScaleBlock)
        hipLaunchKernelGGL((gemm_bs_fp8_big_kernel<kScaleBlock, true, true>),
                           dim3(tiles_i * tiles_j, 1), dim3(kBigThreads), 0, stream, A, sA, B, sB,
                           (void*)C, I, J, Kc, tiles_i, tiles_j, nkb, Cq, Cs);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemm(ScaleMode mode, const uint8_t* A, const float* sA, const uint8_t* B,
                       const float* sB, void* C, bool out_bf16, int64_t I, int64_t J, int64_t Kc,
                       void* workspace, size_t workspace_bytes, int num_cus, hipStream_t stream) {
    switch (mode) {
        case kScaleBlock:
            return launch_mode<kScaleBlock>(A, sA, B, sB, C, out_bf16, I, J, Kc, workspace,
                                            workspace_bytes, num_cus, stream);
        case kScaleBlockT:
            return launch_mode<kScaleBlockT>(A, sA, B, sB, C, out_bf16, I, J, Kc, workspace,
                                             workspace_bytes, num_cus, stream);
        case kScaleRow:
            return launch_mode<kScaleRow>(A, sA, B, sB, C, out_bf16, I, J, Kc, workspace,
                                          workspace_bytes, num_cus, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fp8bs
