// gemm_bf16.hip -- unquantized BF16 GEMM for gfx950: the comparator of the
// FP8 path.
//
// The Puro-2B technical report (lkr-homepage blog, section 2 "FP8") measures
// its FP8 training against BF16 training of the same model; this kernel is
// the BF16 side of that comparison at the linear layers' shapes:
//     C[i][j] = sum_k A[i][k] * B[j][k],   A [I, K], B [J, K] BF16,
// contraction contiguous ("TN"), products accumulated in FP32 by the MFMA.
//
// Workgroup tile 256 (i) x 256 (j) x 64 (k); eight waves in a 4x2 grid, each
// a 64x128 patch of 4x8 MFMA tiles; BF16 tiles (256 rows of 128 bytes, 32 KB
// per operand) double-buffered in LDS through direct global->LDS loads;
// v_mfma_f32_16x16x32_bf16 accumulates straight into the FP32 accumulators
// (nothing to widen, no per-block scale fold).  This wave's A fragments for
// the 64-wide step are read once and kept in registers; B fragments stream.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"

namespace fp8bs {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kB16M = 256;
constexpr int kB16N = 256;
constexpr int kB16K = 64;                       // BF16 values per 128-byte tile row
constexpr int kB16Threads = 512;
constexpr int kB16Tile = kB16M * kRowBytes;     // one operand tile: 32 KB

template <bool OUT_BF16>
__global__ __launch_bounds__(kB16Threads, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C,
    int64_t I, int64_t J, int64_t K, int tiles_i, int tiles_j) {
    __shared__ __align__(16) uint8_t As[2][kB16Tile];
    __shared__ __align__(16) uint8_t Bs[2][kB16Tile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave & 3, wj = wave >> 2;
    int ti, tj;
    tile_coords(blockIdx.x, tiles_i, tiles_j, &ti, &tj);
    const int64_t i0 = (int64_t)ti * kB16M, j0 = (int64_t)tj * kB16N;
    const int nks = (int)(K / kB16K);
    const int64_t row_bytes = K * 2;

    // Direct global -> LDS loads.  Waves 0..3 fill both 32 KB tiles (wave w:
    // 1 KB pieces 8w .. 8w+7, 8 rows each; lane l lands at row 8*piece + l/8,
    // physical chunk l%8, and fetches the logical chunk the swizzle puts
    // there); waves 4..7 go straight on to their MFMAs after each barrier.
    // Rows past the end of A or B are clamped to the last row (never stored).
    const uint8_t* a_bytes = reinterpret_cast<const uint8_t*>(A);
    const uint8_t* b_bytes = reinterpret_cast<const uint8_t*>(B);
    const int prow = 64 * (wave & 3) + (lane >> 3);
    const int pc = (lane & 7) ^ lds_swz_bf16(prow);
    auto issue_loads = [&](int ks, int buf) {
        if (wave >= 4) return;
        const int64_t koff = (int64_t)ks * kRowBytes;
        int pr = prow, pcc = pc;
        asm volatile("" : "+v"(pr), "+v"(pcc));       // keep the address math per call
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = pr + 8 * j;
            const int c = (j & 1) ? (pcc ^ 4) : pcc;    // row + 8j flips bit 2 of the swizzle for odd j
            __builtin_amdgcn_global_load_lds(a_bytes + min(i0 + row, I - 1) * row_bytes + koff + c * 16,
                                             (lds_void*)(&As[buf][(8 * wave + j) * 1024]), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(b_bytes + min(j0 + row, J - 1) * row_bytes + koff + c * 16,
                                             (lds_void*)(&Bs[buf][(8 * wave + j) * 1024]), 16, 0, 0);
        }
    };

    v4f acc[4][8];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int js = 0; js < 8; ++js) acc[it][js] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int g = lane >> 4;

    if (nks > 0) issue_loads(0, 0);
    for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        wait_global_loads();
        __syncthreads();

        const uint8_t* At = As[buf];
        const uint8_t* Bt = Bs[buf];
        // MFMA chunk c covers K = 32c .. 32c+31 of the step; lane (r16, g)
        // supplies K = 32c + 8g .. +7 of its row: 16-byte chunk 4c + g.
        // Every fragment of the step is read before the next step's direct
        // loads are issued: the compiler waits for all outstanding direct
        // loads before an LDS read (it cannot tell the two buffers apart),
        // so reads issued after them would wait for the next step's data.
        v8bf af[4][2], bfr[8][2];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = wi * 64 + it * 16 + r16;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                af[it][c] =
                    *reinterpret_cast<const v8bf*>(At + lds_off(row, 4 * c + g, lds_swz_bf16(row)));
        }
#pragma unroll
        for (int js = 0; js < 8; ++js) {
            const int row = wj * 128 + js * 16 + r16;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                bfr[js][c] =
                    *reinterpret_cast<const v8bf*>(Bt + lds_off(row, 4 * c + g, lds_swz_bf16(row)));
        }
        if (ks + 1 < nks) issue_loads(ks + 1, buf ^ 1);
#pragma unroll
        for (int js = 0; js < 8; ++js) {
            const v8bf* bf = bfr[js];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    // D[j][i]: j = 4g+v (rows of the B subtile), i = r16 (rows of the A subtile)
                    acc[it][js] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[c], af[it][c],
                                                                          acc[it][js], 0, 0, 0);
        }
    }

    // epilogue: lane owns C[i][j .. j+3]
    if constexpr (OUT_BF16) __syncthreads();         // every wave done with the LDS tiles
    if (j0 + 128 * wj >= J) return;
    if constexpr (OUT_BF16) {
        // Restage the wave's 64x128 BF16 patch through LDS so that it leaves
        // as whole 256-byte rows in 16-byte stores (chunks XOR-swizzled by row).
        uint8_t* stage = (wave < 4 ? &As[0][0] : &Bs[0][0]) + (wave & 3) * 16384;
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
        __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): the wave's LDS writes
        __builtin_amdgcn_wave_barrier();
        uint16_t* Cb = reinterpret_cast<uint16_t*>(C);
#pragma unroll
        for (int pass = 0; pass < 16; ++pass) {
            const int row = pass * 4 + (lane >> 4);
            const int c = lane & 15;
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
                uint2 pk;
                pk.x = pack_bf16x2(acc[it][js][0], acc[it][js][1]);
                pk.y = pack_bf16x2(acc[it][js][2], acc[it][js][3]);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + i * J + j) = pk;
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(C) + i * J + j) =
                    make_float4(acc[it][js][0], acc[it][js][1], acc[it][js][2], acc[it][js][3]);
            }
        }
    }
}

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, bool out_bf16,
                            int64_t I, int64_t J, int64_t K, hipStream_t stream) {
    const int64_t tiles_i = (I + kB16M - 1) / kB16M;
    const int64_t tiles_j = (J + kB16N - 1) / kB16N;
    const int64_t blocks = tiles_i * tiles_j;
    if (blocks == 0) return hipSuccess;
    if (out_bf16)
        return launch(gemm_bf16_kernel<true>, grid1d(blocks), dim3(kB16Threads), stream, A,
                      B, C, I, J, K, (int)tiles_i, (int)tiles_j);
    return launch(gemm_bf16_kernel<false>, grid1d(blocks), dim3(kB16Threads), stream, A, B,
                  C, I, J, K, (int)tiles_i, (int)tiles_j);
}

}  // namespace fp8bs
