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
// block in FP32, which is folded into the FP32 accumulator: acc += P * sA*sB,
// one FMA per output element where sA*sB is one product per row and block
// (fprop, dgrad), a multiply (sA*sB, formed before the MFMAs) and an FMA
// where both scales vary along the tile (wgrad).
//
// Two kernels share that arithmetic:
//   gemm_bs_fp8_kernel      workgroup tile 128 (i) x 128 (j) x 128 (k), four
//                           waves of 64x64, two workgroups per CU; both FP8
//                           tiles staged in LDS by direct global->LDS loads
//                           (double buffered, 16-byte chunks XOR-swizzled by
//                           row) and widened by every wave that reads them.
//                           Used for wgrad without a split workspace when the
//                           256x256 tiles alone fill the CUs, and for grids
//                           too small to give every CU a 256x256 tile.
//   gemm_bs_fp8_big_kernel  256 x 256 x 128, eight waves of 32x256, one
//                           workgroup per CU; fprop, dgrad (also with the
//                           quantizing epilogue) and wgrad.  B is
//                           widened once per block into an FP16 LDS tile, A
//                           goes straight to registers.
// Both can split the contraction (FP32 slices in a caller workspace, summed
// in a fixed order) and hand out output tiles in an XCD-aware grouped order
// (gemm_common.h).  The MFMA operands are swapped (B fragment as the first
// source) so that each lane owns four consecutive output columns of one row
// and stores them as one vector.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <type_traits>
#include <vector>

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

template <int MODE, bool OUT_BF16, bool ACC = false>
__global__ __launch_bounds__(kThreads, 2) void gemm_bs_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ C, int64_t I, int64_t J, int64_t Kc,
    int tiles_i, int tiles_j, int p0, int nps, float* __restrict__ Wsp) {
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
    // only the row-scaled (wgrad) mode is ever split
    const int kb0 = MODE == kScaleRow ? split_begin(blockIdx.y, p0, nps) : 0;
    const int nkb = MODE == kScaleRow ? split_end(blockIdx.y, p0, nps, nkb_all) - kb0 : nkb_all;
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
        int c = (lane & 7) ^ lds_swz_fp8(row);
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
            for (int it = 0; it < 4; ++it) {
                const int row = wi * 64 + it * 16 + r16;
                ar[it] = *reinterpret_cast<const uint4*>(At + lds_off(row, 2 * g + h, lds_swz_fp8(row)));
            }
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int row = wj * 64 + jt * 16 + r16;
                br[jt] = *reinterpret_cast<const uint4*>(Bt + lds_off(row, 2 * g + h, lds_swz_fp8(row)));
            }
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
                float* Cf = MODE == kScaleRow ? split_out(blockIdx.y, C, Wsp, I, J)
                                              : reinterpret_cast<float*>(C);
                if constexpr (ACC) {
                    v4f* dst = reinterpret_cast<v4f*>(Cf + i * J + j);
                    *dst = *dst + acc[it][jt];
                } else {
                    *reinterpret_cast<float4*>(Cf + i * J + j) = make_float4(
                        acc[it][jt][0], acc[it][jt][1], acc[it][jt][2], acc[it][jt][3]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large-tile kernel: workgroup tile 256 (i) x 256 (j) x 128 (k), eight waves,
// wave w owning the 32 x 256 output patch of rows 32w .. 32w+31.
//   B: the 256 x 128 codes of a block are widened ONCE, cooperatively (lane l
//      of wave w takes 64 codes of row 32w + l%32), and stored in LDS as FP16
//      (64 KB, double buffered); every wave reads its B fragments from there.
//   A: a wave's 32 rows are its own, so they go straight from global memory
//      to registers and are widened once per block.
// 64 widenings feed a wave's 128 MFMAs per block (0.5 per MFMA; 1.5 when every
// wave widens the B fragments it reads from an FP8 tile), so the VALU work
// (widening and the scale fold) stays well below the MFMA time.
// Per block: the next block's B codes are requested at the top; after the
// fourth of eight MFMA groups they are widened and stored into the other FP16
// buffer in one burst, and the next block's A codes are requested.  Each MFMA
// group's B fragments are read from LDS one group ahead.  In the block-scaled
// modes each group's partial sums are folded one group late, while the next
// group's MFMAs run.  The epilogue works in two 128-column halves; in the
// block-scaled modes the first leaves during the last block, once its columns
// are final.
// The FP16 B tile is stored in fragment order: the 16 bytes that lane l reads
// for MFMA chunk c of B subtile js sit at ((4 js + c) * 64 + l) * 16, so every
// fragment read is one contiguous 1 KB block (gfx950's LDS serves those
// without bank conflicts whatever the lane-to-chunk pattern; the row-major
// FP16 tile with row-swizzled chunks it replaced measured bank conflicts on a
// third of the LDS cycles).  A thread widening row R, codes
// [8q, 8q+8), writes them where lane (R % 16) + 16 (q / 4) finds them for
// chunk q % 4 of subtile R / 16; eight consecutive lanes always write eight
// different rows mod 8, which keeps those stores conflict-free as well.
// The contraction order inside a block is permuted alike for A and B: lane
// (r16, g) supplies codes [32g + 8c, 32g + 8c + 8) of its row to MFMA chunk c,
// so one 32-byte global load per row gives a lane its four chunks.
// Tiles are ordered for the L2s (tile_coords); gridDim.y splits the
// contraction (split_begin / split_end / split_out).
// QOUT: the epilogue also quantizes the BF16 output in 1x128 row tiles (the
// rule of quant_rowtile_kernel) and stores codes Cq [I, J] and scales
// Cs [I, J/128]; C (BF16) may then be null.  A wave's 256 output columns of a
// row are two such tiles, each held by the four lanes r16 + 16g.
// ---------------------------------------------------------------------------
constexpr int kBigM = 256;
constexpr int kBigN = 256;
constexpr int kBigThreads = 512;
constexpr int kF16Tile = 256 * 256;        // FP16 B tile: 256 rows x 256 bytes

__device__ __forceinline__ int f16_frag_off(int row, int q) {
    return (((row >> 4) * 4 + (q & 3)) * 64 + (q >> 2) * 16 + (row & 15)) * 16;
}

template <int MODE, bool OUT_BF16, bool QOUT = false, bool ACC = false>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_bs_fp8_big_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ C, int64_t I, int64_t J, int64_t Kc,
    int tiles_i, int tiles_j, int p0, int nps, float* __restrict__ Wsp,
    uint8_t* __restrict__ Cq, float* __restrict__ Cs) {
    __shared__ __align__(16) uint8_t Bh[2][kF16Tile];
    __shared__ __align__(16) float sBs[2][MODE == kScaleRow ? kBigN : 4];   // per-row B scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    int ti, tj;
    tile_coords(blockIdx.x, tiles_i, tiles_j, &ti, &tj);
    const int64_t i0 = (int64_t)ti * kBigM, j0 = (int64_t)tj * kBigN;
    const int nkb_all = (int)(Kc / kBK);
    // Only the row-scaled (wgrad) mode is ever split; the others sum all
    // blocks.  The quantizing epilogue's instantiation takes its block range
    // from the launch arguments too (p0 = the block count): the compiler then
    // waits for a block's A codes once, ahead of the barrier, instead of in
    // steps among the widenings, and that measured 10% faster for it (and no
    // faster for the plain instantiations).
    constexpr bool kRangeArgs = MODE == kScaleRow || QOUT;
    const int kb0 = kRangeArgs ? split_begin(blockIdx.y, p0, nps) : 0;
    const int nkb = kRangeArgs ? split_end(blockIdx.y, p0, nps, nkb_all) - kb0 : nkb_all;
    const int64_t jb_count = J / kBN;

    // A: rows 32w + 16it + r16 (clamped; rows past I are never stored), the
    // lane's 32 bytes [32g, 32g+32) of each block.
    const uint8_t* a_src[2];
    const float* sa_src[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int64_t row = min(i0 + 32 * wave + 16 * it + r16, I - 1);
        a_src[it] = A + row * Kc + 32 * g;
        sa_src[it] = sA + row * nkb_all;
    }
    // B: lane l of wave w widens bytes [64h, 64h+64) of row 32w + l%32
    // (h = l/32).
    const int brow = 32 * wave + (lane & 31);
    const int bh = lane >> 5;
    const int64_t bj = min(j0 + brow, J - 1);
    const uint8_t* b_src = B + bj * Kc + 64 * bh;
    const float* sbr_src = MODE == kScaleRow ? sB + bj * nkb_all : sB;   // scale row of B row brow
    const int64_t jb0 = j0 / kBN;
    const int64_t jb1 = min(jb0 + 1, jb_count - 1);

    uint4 an[2][2];           // next block's A codes
    uint4 bn[4];              // next block's B codes
    float san[2], sbn0 = 0.f, sbn1 = 0.f, sbrn = 0.f;
    auto load_a = [&](int kb) {
        const int64_t koff = (int64_t)kb * kBK;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            an[it][0] = *reinterpret_cast<const uint4*>(a_src[it] + koff);
            an[it][1] = *reinterpret_cast<const uint4*>(a_src[it] + koff + 16);
            san[it] = sa_src[it][kb];
        }
        if (MODE == kScaleBlock) {
            sbn0 = sB[jb0 * nkb_all + kb];
            sbn1 = sB[jb1 * nkb_all + kb];
        } else if (MODE == kScaleBlockT) {
            sbn0 = sB[(int64_t)kb * jb_count + jb0];
            sbn1 = sB[(int64_t)kb * jb_count + jb1];
        }
    };
    auto load_b = [&](int kb) {
        const int64_t koff = (int64_t)kb * kBK;
#pragma unroll
        for (int q = 0; q < 4; ++q) bn[q] = *reinterpret_cast<const uint4*>(b_src + koff + 16 * q);
        if (MODE == kScaleRow) sbrn = sbr_src[kb];
    };
    // Widen and store codes [16p, 16p+16) of the lane's 64 (two chunks).
    // The opaque register dependence (an asm statement stays between the
    // LDS reads around it) keeps the compiler from hoisting the widening,
    // and with it the wait for these loads, towards the top of the block,
    // where the codes are still in flight.
    auto store_b = [&](int buf, int p) {
        uint8_t* dst = Bh[buf];
        uint4 w = bn[p];
        asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
        *reinterpret_cast<v8h*>(dst + f16_frag_off(brow, 8 * bh + 2 * p)) = widen8(w.x, w.y);
        *reinterpret_cast<v8h*>(dst + f16_frag_off(brow, 8 * bh + 2 * p + 1)) = widen8(w.z, w.w);
        if (MODE == kScaleRow && p == 0) sBs[buf][brow] = sbrn;   // both halves of the row write it
    };

    // B subtiles per MFMA group: two, so a group is four independent chains
    // of four MFMAs (two A subtiles x two B subtiles), in every mode.
    constexpr int JJ = 2;
    v4f acc[2][16];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int js = 0; js < 16; ++js) acc[it][js] = v4f{0.f, 0.f, 0.f, 0.f};

    if (nkb > 0) {
        load_b(kb0);
        load_a(kb0);
#pragma unroll
        for (int part = 0; part < 4; ++part) store_b(0, part);
    }
    // Output half h (columns j0 + 128h .. +127, i.e. B subtiles 8h .. 8h+7)
    // of the tile: lane owns C[i][j .. j+3]; split s writes its own FP32
    // slice.  Half 0 is final after the fourth MFMA group of the last block;
    // in the block-scaled modes it leaves then, while the second half is
    // computed.  BF16 outputs (and the
    // codes of the quantizing epilogue) are restaged through this wave's 8 KB
    // of Bh[lbuf ^ 1], which nothing reads or writes during the last block
    // (lbuf: the buffer the last block reads), so that they leave as whole
    // rows in 16-byte stores.
    const bool j_full = j0 + kBigN <= J;             // else only the first 128 columns exist
    // The row-scaled (FP32) instantiation has no registers for the early half.
    constexpr bool kEarlyHalf = MODE != kScaleRow;
    constexpr bool kLagFold = MODE != kScaleRow && !QOUT;
    auto out_half = [&](auto h_tag, int lbuf) __attribute__((always_inline)) {
        constexpr int h = decltype(h_tag)::value;
        if (h == 1 && !j_full) return;
        const int64_t jh = j0 + 128 * h;             // first column of the half
        uint8_t* stage = &Bh[lbuf ^ 1][0] + wave * 8192;
        // BF16 half rows (256 bytes, 16-byte chunks XOR-swizzled by row).
        auto store_bf16 = [&](uint16_t* Cb) __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int row = 16 * it + r16;
#pragma unroll
                for (int jq = 0; jq < 8; ++jq) {
                    const int js = 8 * h + jq;
                    const int b = jq * 32 + g * 8;         // byte offset in the half row
                    const int phys = (((b >> 4) ^ (row & 15)) << 4) | (b & 15);
                    *reinterpret_cast<uint2*>(stage + row * 256 + phys) =
                        make_uint2(pack_bf16x2(acc[it][js][0], acc[it][js][1]),
                                   pack_bf16x2(acc[it][js][2], acc[it][js][3]));
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): the wave's LDS writes
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int pass = 0; pass < 8; ++pass) {
                const int row = 4 * pass + (lane >> 4);
                const int c = lane & 15;                   // 16-byte chunk of the half row
                const uint4 w =
                    *reinterpret_cast<const uint4*>(stage + row * 256 + ((c ^ (row & 15)) << 4));
                const int64_t i = i0 + 32 * wave + row;
                if (i < I) *reinterpret_cast<uint4*>(Cb + i * J + jh + c * 8) = w;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        };
        if constexpr (QOUT) {
            // Scale of the row tile (columns jh .. jh+127) from the
            // BF16-rounded values, then the BF16 copy if asked for, then the
            // codes (32 rows x 128 bytes, chunks XOR-swizzled by row).
            float inv[2];
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                uint32_t m = 0;
#pragma unroll
                for (int jq = 0; jq < 8; ++jq) {
                    const int js = 8 * h + jq;
                    m = absmax_pair(m, pack_bf16x2(acc[it][js][0], acc[it][js][1]));
                    m = absmax_pair(m, pack_bf16x2(acc[it][js][2], acc[it][js][3]));
                }
                m = absmax_fold(m);
                m = max(m, (uint32_t)__shfl_xor((int)m, 16));
                m = max(m, (uint32_t)__shfl_xor((int)m, 32));
                const TileScale ts = tile_scale(m, &g_scale_tables);
                inv[it] = ts.inv;
                const int64_t i = i0 + 32 * wave + 16 * it + r16;
                if (g == 0 && i < I) Cs[i * jb_count + jb0 + h] = ts.s;
            }
            if (C) store_bf16(reinterpret_cast<uint16_t*>(C));
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int row = 16 * it + r16;
#pragma unroll
                for (int jq = 0; jq < 8; ++jq) {
                    const int js = 8 * h + jq;
                    const uint32_t p0 = pack_bf16x2(acc[it][js][0], acc[it][js][1]);
                    const uint32_t p1 = pack_bf16x2(acc[it][js][2], acc[it][js][3]);
                    *reinterpret_cast<uint32_t*>(stage + row * 128 + ((jq ^ (row & 7)) << 4) + 4 * g) =
                        cvt4_e4m3(bf16_lo(p0) * inv[it], bf16_hi(p0) * inv[it], bf16_lo(p1) * inv[it],
                                  bf16_hi(p1) * inv[it]);
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {
                const int row = 8 * pass + (lane >> 3);
                const int c = lane & 7;                    // 16-byte chunk of the 128 codes
                const uint4 w =
                    *reinterpret_cast<const uint4*>(stage + row * 128 + ((c ^ (row & 7)) << 4));
                const int64_t i = i0 + 32 * wave + row;
                if (i < I) *reinterpret_cast<uint4*>(Cq + i * J + jh + c * 16) = w;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        } else if constexpr (OUT_BF16) {
            store_bf16(reinterpret_cast<uint16_t*>(C));
        } else {
            float* Cf = MODE == kScaleRow ? split_out(blockIdx.y, C, Wsp, I, J)
                                          : reinterpret_cast<float*>(C);
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int64_t i = i0 + 32 * wave + 16 * it + r16;
                if (i >= I) continue;
#pragma unroll
                for (int jq = 0; jq < 8; ++jq) {
                    const int js = 8 * h + jq;
                    if constexpr (ACC) {
                        v4f* dst = reinterpret_cast<v4f*>(Cf + i * J + jh + 16 * jq + 4 * g);
                        *dst = *dst + acc[it][js];
                    } else {
                        *reinterpret_cast<float4*>(Cf + i * J + jh + 16 * jq + 4 * g) =
                            make_float4(acc[it][js][0], acc[it][js][1], acc[it][js][2],
                                        acc[it][js][3]);
                    }
                }
            }
        }
    };

    // One block; MORE: the next block is loaded and staged during this one.
    // The last block runs as its own copy, so the loop body has no branch.
    auto run_block = [&](int k, auto more_tag) __attribute__((always_inline)) {
        constexpr bool more = decltype(more_tag)::value;
        const int buf = k & 1;
        __syncthreads();          // B of this block is in Bh[buf]; all waves are done with Bh[buf^1]
        v8h af[2][4];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            af[it][0] = widen8(an[it][0].x, an[it][0].y);
            af[it][1] = widen8(an[it][0].z, an[it][0].w);
            af[it][2] = widen8(an[it][1].x, an[it][1].y);
            af[it][3] = widen8(an[it][1].z, an[it][1].w);
        }
        float cs0[2], cs1[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            cs0[it] = san[it] * sbn0;         // kScaleRow: unused
            cs1[it] = san[it] * sbn1;
        }
        float sa[2] = {san[0], san[1]};
        if constexpr (more) load_b(kb0 + k + 1);      // widened in the middle of this block
        const uint8_t* Bt = Bh[buf];
        // MFMA step t = 4 jp + c reads B fragments (subtiles JJ jp + jj, chunk
        // c), kAhead steps ahead, so the MFMAs in between cover the LDS
        // latency (two steps ahead costs more in registers than it gains).
        constexpr int kAhead = 1;
        constexpr int kSets = kAhead + 1;
        auto frag = [&](int t, int jj) {
            return *reinterpret_cast<const v8h*>(
                Bt + ((4 * (JJ * (t >> 2) + jj) + (t & 3)) * 64 + lane) * 16);
        };
        v8h bq[kSets][JJ];
#pragma unroll
        for (int t = 0; t < kAhead; ++t)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) bq[t][jj] = frag(t, jj);
        // Fold one MFMA group's partials (B subtiles JJ jq .. JJ jq + JJ - 1) into acc.
        // Row-scaled mode: the scale products sA(i) sB(j) of one MFMA group's
        // outputs, one per element since both scales vary along the tile,
        // formed before the group's MFMAs.  They do not wait for the MFMA
        // results, so the multiplies issue while the matrix core works and
        // only the FMA of the fold waits (3.6% faster over a layer's four
        // wgrad shapes than multiplying the partials after the MFMAs).
        v4f csr[JJ][2];
        auto scale_products = [&](int jq) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const float4 sb =
                    *reinterpret_cast<const float4*>(&sBs[buf][16 * (JJ * jq + jj) + 4 * g]);
#pragma unroll
                for (int it = 0; it < 2; ++it)
                    csr[jj][it] = v4f{sa[it] * sb.x, sa[it] * sb.y, sa[it] * sb.z, sa[it] * sb.w};
            }
        };
        auto fold = [&](v4f (&q)[JJ][2], int jq) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const int js = JJ * jq + jj;
                if (MODE != kScaleRow) {
#pragma unroll
                    for (int it = 0; it < 2; ++it) {
                        const float cs = js < 8 ? cs0[it] : cs1[it];
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[it][js][v] = __builtin_fmaf(q[jj][it][v], cs, acc[it][js][v]);
                    }
                } else {
#pragma unroll
                    for (int it = 0; it < 2; ++it)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[it][js][v] =
                                __builtin_fmaf(q[jj][it][v], csr[jj][it][v], acc[it][js][v]);
                }
            }
        };
        // kLagFold: group jp's partials are folded while group jp + 1's MFMAs
        // run, so the FMAs fill the matrix core's issue gaps instead of waiting
        // for the group's last MFMA.  That needs a second set of partials (16
        // registers).  The quantizing epilogue has no room for them; the
        // row-scaled mode fits them only by spilling two values outside the
        // loop and measured no faster with them, so both fold each group
        // right after it.
        v4f pl[JJ][2];
#pragma unroll
        for (int jp = 0; jp < 16 / JJ; ++jp) {
            if constexpr (MODE == kScaleRow) scale_products(jp);
            v4f p[JJ][2];
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj)
#pragma unroll
                for (int it = 0; it < 2; ++it) p[jj][it] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int t = 4 * jp + c;
                if (t + kAhead < 64 / JJ) {
#pragma unroll
                    for (int jj = 0; jj < JJ; ++jj) bq[(t + kAhead) % kSets][jj] = frag(t + kAhead, jj);
                }
#pragma unroll
                for (int jj = 0; jj < JJ; ++jj)
#pragma unroll
                    for (int it = 0; it < 2; ++it)
                        // D[j][i]: j = 4g+v (rows of the B subtile), i = r16 (rows of the A subtile)
                        p[jj][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bq[t % kSets][jj], af[it][c],
                                                                            p[jj][it], 0, 0, 0);
            }
            if constexpr (kLagFold) {
                if (jp > 0) fold(pl, jp - 1);
#pragma unroll
                for (int jj = 0; jj < JJ; ++jj)
#pragma unroll
                    for (int it = 0; it < 2; ++it) pl[jj][it] = p[jj][it];
            } else {
                fold(p, jp);
            }
            if constexpr (more) {
                if (jp == 3) {
#pragma unroll
                    for (int part = 0; part < 4; ++part) store_b(buf ^ 1, part);   // B of the next block, widened once
                    load_a(kb0 + k + 1);      // its A codes, in flight until the next block
                }
            } else if constexpr (kEarlyHalf) {
                // columns 0..127 (groups 0..3) are final once group 3 is folded
                if (jp == (kLagFold ? 4 : 3)) out_half(std::integral_constant<int, 0>{}, buf);
            }
        }
        if constexpr (kLagFold) fold(pl, 16 / JJ - 1);
    };
    for (int k = 0; k + 1 < nkb; ++k) run_block(k, std::true_type{});
    if (nkb > 0) run_block(nkb - 1, std::false_type{});
    const int lbuf = nkb > 0 ? (nkb - 1) & 1 : 0;
    if (!kEarlyHalf || nkb == 0) out_half(std::integral_constant<int, 0>{}, lbuf);
    out_half(std::integral_constant<int, 1>{}, lbuf);
}

// Sum of the split pieces, in piece order: out[e] = (((out[e] + ws[0][e]) +
// ws[1][e]) + ...), where out already holds piece 0 (fixed order, so the
// result does not depend on timing).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float4* __restrict__ ws,
                                                            float4* __restrict__ out, int64_t n4,
                                                            int slices) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    float4 a = out[e];
    for (int s = 0; s < slices; ++s) {
        const float4 b = ws[(int64_t)s * n4 + e];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    out[e] = a;
}

// The accumulating form: every piece is in the workspace (piece y in slice
// y); their sum, in piece order, is added to out once:
// out[e] = out[e] + (((ws[0][e] + ws[1][e]) + ...)), so the result equals the
// plain call's result added to out.
__global__ __launch_bounds__(256) void splitk_reduce_acc_kernel(const float4* __restrict__ ws,
                                                                float4* __restrict__ out,
                                                                int64_t n4, int slices) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    float4 a = ws[e];
    for (int s = 1; s < slices; ++s) {
        const float4 b = ws[(int64_t)s * n4 + e];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    const float4 o = out[e];
    out[e] = make_float4(o.x + a.x, o.y + a.y, o.z + a.z, o.w + a.w);
}

template <int MODE, bool BF16, bool ACC = false>
static hipError_t launch_small(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                               void* C, int64_t I, int64_t J, int64_t Kc, int pieces, int p0,
                               int nps, float* Wsp, hipStream_t stream) {
    int64_t tiles_i = (I + kBM - 1) / kBM;
    int64_t tiles_j = J / kBN;
    int64_t blocks = tiles_i * tiles_j;
    if (blocks == 0) return hipSuccess;
    return launch(gemm_bs_fp8_kernel<MODE, BF16, ACC>, dim3(grid1d(blocks).x, pieces), dim3(kThreads),
                  stream, A, sA, B, sB, C, I, J, Kc, (int)tiles_i, (int)tiles_j, p0, nps, Wsp);
}

template <int MODE, bool BF16, bool ACC = false>
static hipError_t launch_big(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                             void* C, int64_t I, int64_t J, int64_t Kc, int pieces, int p0,
                             int nps, float* Wsp, hipStream_t stream) {
    int tiles_i = (int)((I + kBigM - 1) / kBigM);
    int tiles_j = (int)((J + kBigN - 1) / kBigN);
    return launch(gemm_bs_fp8_big_kernel<MODE, BF16, false, ACC>, dim3(tiles_i * tiles_j, pieces),
                  dim3(kBigThreads), stream, A, sA, B, sB, C, I, J, Kc, tiles_i, tiles_j, p0, nps,
                  Wsp, (uint8_t*)nullptr, (float*)nullptr);
}

// Launch plan for one GEMM: which kernel, and how its contraction is split
// (split_begin / split_end: piece 0 has p0 blocks, the others nps, the last
// clipped).
struct Plan {
    bool big;
    int pieces;    // 1: no split
    int p0;
    int nps;
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

// Time at which the last workgroup of a split launch finishes, in units of
// one contraction block: the dispatcher hands workgroups out in launch order
// (every tile's piece 0, then every tile's piece 1, ...) to the first of
// `slots` resident places to come free, and a workgroup takes its block
// count plus a fixed per-workgroup cost (prologue, first loads, epilogue),
// taken here as three blocks.
static int64_t split_makespan(int64_t tiles, int64_t slots, int64_t nkb, int pieces, int p0,
                              int nps) {
    constexpr int64_t kFixed = 3;
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
    for (int64_t i = 0; i < slots; ++i) free_at.push(0);
    int64_t end = 0;
    for (int y = 0; y < pieces; ++y) {
        const int64_t b0 = y == 0 ? 0 : p0 + (int64_t)(y - 1) * nps;
        const int64_t b1 = std::min<int64_t>(nkb, y == 0 ? p0 : p0 + (int64_t)y * nps);
        const int64_t len = b1 - b0 + kFixed;
        for (int64_t t = 0; t < tiles; ++t) {
            const int64_t start = free_at.top();
            free_at.pop();
            free_at.push(start + len);
            end = std::max(end, start + len);
        }
    }
    return end;
}

static Plan plan_gemm_uncached(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int cus,
                               bool allow_split, int force) {
    const int64_t nkb = Kc / kBK;
    Plan p{false, 1, (int)nkb, (int)nkb};
    if (nkb == 0) return p;
    const int64_t big_tiles = ((I + kBigM - 1) / kBigM) * ((J + kBigN - 1) / kBigN);
    const int64_t small_tiles = ((I + kBM - 1) / kBM) * (J / kBN);
    // fprop/dgrad: the 256x256 tile once it gives every CU a tile.  wgrad: the
    // 256x256 tile whenever the contraction may be split (a caller workspace)
    // or its tiles alone cannot fill the CUs; otherwise the 128x128 tile,
    // whose two workgroups per CU balance the grid without a split.
    if (force == 2) p.big = true;
    else if (force == 1) p.big = false;
    else p.big = I >= kBigM && (mode == kScaleRow ? (allow_split || big_tiles < cus)
                                                   : big_tiles >= cus);
    if (mode != kScaleRow || !allow_split) return p;
    // Split the contraction (FP32 output with a caller workspace) when that
    // shortens the launch: candidates are equal pieces (2 .. 8 of them, at
    // least 4 blocks each) and two unequal pieces, the longer first; the one
    // with the earliest simulated finish wins, ties going to fewer pieces
    // (each piece after the first costs an FP32 slice written and read back).
    const int64_t tiles = p.big ? big_tiles : small_tiles;
    const int64_t slots = p.big ? cus : 2 * (int64_t)cus;     // workgroups resident at once
    if (tiles >= 4 * slots || tiles * 8 > (int64_t)1 << 20) return p;
    int64_t best = split_makespan(tiles, slots, nkb, 1, (int)nkb, (int)nkb);
    auto consider = [&](int pieces, int p0, int nps) {
        const int64_t t = split_makespan(tiles, slots, nkb, pieces, p0, nps);
        if (t < best || (t == best && pieces < p.pieces)) {
            best = t;
            p.pieces = pieces;
            p.p0 = p0;
            p.nps = nps;
        }
    };
    for (int s = 2; s <= 8 && nkb / s >= 4; ++s) {
        const int nps = (int)((nkb + s - 1) / s);
        consider((int)((nkb - nps + nps - 1) / nps) + 1, nps, nps);
    }
    const int step = (int)std::max<int64_t>(1, nkb / 32);
    for (int64_t p0 = (nkb + 1) / 2 + step; p0 <= nkb - 4; p0 += step)
        consider(2, (int)p0, (int)(nkb - p0));
    return p;
}

// Plans depend only on the shape, the device's CU count and the options, so
// each is simulated once per process.
static Plan plan_gemm(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus,
                      bool allow_split, int force = -1) {
    const int cus = num_cus > 0 ? num_cus : 256;
    if (force < 0) force = kernel_override();
    static std::mutex mu;
    static std::map<std::tuple<int, int64_t, int64_t, int64_t, int, bool, int>, Plan> cache;
    const auto key = std::make_tuple((int)mode, I, J, Kc, cus, allow_split, force);
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    const Plan p = plan_gemm_uncached(mode, I, J, Kc, cus, allow_split, force);
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() > 4096) cache.clear();
    cache.emplace(key, p);
    return p;
}

hipError_t launch_splitk_reduce(const float* ws, float* out, int64_t n, int slices,
                               hipStream_t stream) {
    const int64_t n4 = n / 4;
    if (n4 == 0 || slices <= 0) return hipSuccess;
    return launch(splitk_reduce_kernel, grid1d((n4 + 255) / 256), dim3(256), stream,
                  reinterpret_cast<const float4*>(ws), reinterpret_cast<float4*>(out), n4,
                  slices);
}

GemmSplit big_tile_split(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus,
                         bool allow_split) {
    const Plan p = plan_gemm(mode, I, J, Kc, num_cus, allow_split, 2);
    return GemmSplit{p.pieces, p.p0, p.nps};
}

size_t gemm_workspace_bytes(ScaleMode mode, int64_t I, int64_t J, int64_t Kc, int num_cus) {
    Plan p = plan_gemm(mode, I, J, Kc, num_cus, true);
    if (p.pieces <= 1) return 0;
    return (size_t)(p.pieces - 1) * (size_t)I * (size_t)J * sizeof(float);
}

template <int MODE>
static hipError_t launch_mode(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                              void* C, bool out_bf16, int64_t I, int64_t J, int64_t Kc,
                              void* workspace, size_t workspace_bytes, int num_cus,
                              hipStream_t stream) {
    const size_t need = gemm_workspace_bytes((ScaleMode)MODE, I, J, Kc, num_cus);
    const bool can_split = !out_bf16 && workspace && need > 0 && workspace_bytes >= need;
    Plan p = plan_gemm((ScaleMode)MODE, I, J, Kc, num_cus, can_split);
    float* Wsp = p.pieces > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
    hipError_t e;
    if (out_bf16)
        e = p.big ? launch_big<MODE, true>(A, sA, B, sB, C, I, J, Kc, 1, p.p0, p.nps, nullptr, stream)
                  : launch_small<MODE, true>(A, sA, B, sB, C, I, J, Kc, 1, p.p0, p.nps, nullptr,
                                             stream);
    else
        e = p.big ? launch_big<MODE, false>(A, sA, B, sB, C, I, J, Kc, p.pieces, p.p0, p.nps, Wsp,
                                            stream)
                  : launch_small<MODE, false>(A, sA, B, sB, C, I, J, Kc, p.pieces, p.p0, p.nps,
                                              Wsp, stream);
    if (e != hipSuccess || p.pieces <= 1) return e;
    const int64_t n4 = I * J / 4;
    return launch(splitk_reduce_kernel, grid1d((n4 + 255) / 256), dim3(256), stream,
                  reinterpret_cast<const float4*>(Wsp), reinterpret_cast<float4*>(C), n4,
                  p.pieces - 1);
}

size_t wgrad_accumulate_workspace_bytes(int64_t I, int64_t J, int64_t Kc, int num_cus) {
    const size_t need = gemm_workspace_bytes(kScaleRow, I, J, Kc, num_cus);
    return need ? need + (size_t)I * (size_t)J * sizeof(float) : 0;
}

// C += the row-scaled GEMM.  Unsplit, the epilogue adds the result to C.
// Split, every piece goes to the workspace (piece 0 in slice 0, which is the
// kernels' output pointer for that launch) and the reduction adds their sum
// to C; the pieces, the plan and the order of the sum are those of the plain
// call, so C ends as C + (the plain call's result) bit for bit.
hipError_t launch_wgrad_accumulate(const uint8_t* A, const float* sA, const uint8_t* B,
                                   const float* sB, float* C, int64_t I, int64_t J, int64_t Kc,
                                   void* workspace, size_t workspace_bytes, int num_cus,
                                   hipStream_t stream) {
    const size_t need = wgrad_accumulate_workspace_bytes(I, J, Kc, num_cus);
    const bool can_split = workspace && need > 0 && workspace_bytes >= need;
    Plan p = plan_gemm(kScaleRow, I, J, Kc, num_cus, can_split);
    if (p.pieces <= 1)
        return p.big ? launch_big<kScaleRow, false, true>(A, sA, B, sB, C, I, J, Kc, 1, p.p0, p.nps,
                                                          nullptr, stream)
                     : launch_small<kScaleRow, false, true>(A, sA, B, sB, C, I, J, Kc, 1, p.p0,
                                                            p.nps, nullptr, stream);
    float* S = reinterpret_cast<float*>(workspace);
    hipError_t e =
        p.big ? launch_big<kScaleRow, false>(A, sA, B, sB, S, I, J, Kc, p.pieces, p.p0, p.nps,
                                             S + I * J, stream)
              : launch_small<kScaleRow, false>(A, sA, B, sB, S, I, J, Kc, p.pieces, p.p0, p.nps,
                                               S + I * J, stream);
    if (e != hipSuccess) return e;
    const int64_t n4 = I * J / 4;
    return launch(splitk_reduce_acc_kernel, grid1d((n4 + 255) / 256), dim3(256), stream,
                  reinterpret_cast<const float4*>(S), reinterpret_cast<float4*>(C), n4, p.pieces);
}

hipError_t launch_gemm_quantized(ScaleMode mode, const uint8_t* A, const float* sA,
                                 const uint8_t* B, const float* sB, uint16_t* C, uint8_t* Cq,
                                 float* Cs, int64_t I, int64_t J, int64_t Kc, hipStream_t stream) {
    const int tiles_i = (int)((I + kBigM - 1) / kBigM);
    const int tiles_j = (int)((J + kBigN - 1) / kBigN);
    const int nkb = (int)(Kc / kBK);
    if (tiles_i == 0 || tiles_j == 0) return hipSuccess;
    if (mode == kScaleBlockT)
        return launch(gemm_bs_fp8_big_kernel<kScaleBlockT, true, true>, dim3(tiles_i * tiles_j, 1),
                      dim3(kBigThreads), stream, A, sA, B, sB, (void*)C, I, J, Kc, tiles_i,
                      tiles_j, nkb, nkb, (float*)nullptr, Cq, Cs);
    if (mode == kScaleBlock)
        return launch(gemm_bs_fp8_big_kernel<kScaleBlock, true, true>, dim3(tiles_i * tiles_j, 1),
                      dim3(kBigThreads), stream, A, sA, B, sB, (void*)C, I, J, Kc, tiles_i,
                      tiles_j, nkb, nkb, (float*)nullptr, Cq, Cs);
    return hipErrorInvalidValue;
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

// Attainable FP16 MFMA rate on this device: every wave issues iters x 16
// rounds of eight independent v_mfma_f32_16x16x32_f16 chains and touches
// memory only to store its result, so the kernel's time is the matrix cores'
// own, at the clock they hold under MFMA load.  (The compiler adds about 56
// accumulator-register moves per 128 MFMAs at the loop edge; they run on the
// VALU beside the other waves' MFMAs.)  With every operand element equal to
// v, each output element of a chain grows by 32 v^2 per instruction, and each
// thread stores the sum of its 32 accumulator elements: 16384 v^2 iters.
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* __restrict__ out, int iters,
                                                        float v) {
    const _Float16 h = (_Float16)v;
    const v8h a = {h, h, h, h, h, h, h, h};
    v4f acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, acc[j], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

hipError_t launch_mfma_rate(float* out, int64_t blocks, int iters, float v, hipStream_t stream) {
    if (blocks == 0) return hipSuccess;
    return launch(mfma_rate_kernel, grid1d(blocks), dim3(256), stream, out, iters, v);
}

}  // namespace fp8bs
