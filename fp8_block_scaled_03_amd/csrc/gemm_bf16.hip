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
// (nothing to widen, no per-block scale fold).  A step's A and B fragments
// are read into registers before the next step's loads are issued.  Grids
// whose 256 x 256 tiles would leave half the CUs idle (weight-gradient
// shapes, whose outputs are small) run 128 x 128 tiles of four waves.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"

namespace fp8bs {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kB16K = 64;                       // BF16 values per 128-byte tile row

// T x T output tiles (T = 256 or 128) of 2 T / 64 waves in a (T/64) x 2 grid,
// each wave a 64 x T/2 patch of 4 x T/32 MFMA tiles.  T = 128 (four waves,
// two workgroups per CU) serves grids that the 256 x 256 tiles leave
// partly idle.
template <int T, bool OUT_BF16>
__global__ __launch_bounds__(2 * T, T == 256 ? 1 : 2) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C,
    int64_t I, int64_t J, int64_t K, int tiles_i, int tiles_j) {
    constexpr int WI = T / 64;                  // waves along i; also the loading waves
    constexpr int JS = T / 32;                  // B subtiles per wave
    constexpr int kTile = T * kRowBytes;        // one operand tile
    __shared__ __align__(16) uint8_t As[2][kTile];
    __shared__ __align__(16) uint8_t Bs[2][kTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave % WI, wj = wave / WI;
    int ti, tj;
    tile_coords(blockIdx.x, tiles_i, tiles_j, &ti, &tj);
    const int64_t i0 = (int64_t)ti * T, j0 = (int64_t)tj * T;
    const int nks = (int)(K / kB16K);
    const int64_t row_bytes = K * 2;

    // Direct global -> LDS loads.  Waves 0 .. WI-1 fill both tiles (wave w:
    // 1 KB pieces 8w .. 8w+7, 8 rows each; lane l lands at row 8*piece + l/8,
    // physical chunk l%8, and fetches the logical chunk the swizzle puts
    // there); the other waves go straight on to their MFMAs after each barrier.
    // Rows past the end of A or B are clamped to the last row (never stored).
    const uint8_t* a_bytes = reinterpret_cast<const uint8_t*>(A);
    const uint8_t* b_bytes = reinterpret_cast<const uint8_t*>(B);
    const int prow = 64 * wave + (lane >> 3);
    const int pc = (lane & 7) ^ lds_swz_bf16(prow);
    auto issue_loads = [&](int ks, int buf) {
        if (wave >= WI) return;
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

    v4f acc[4][JS];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int js = 0; js < JS; ++js) acc[it][js] = v4f{0.f, 0.f, 0.f, 0.f};

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
        v8bf af[4][2], bfr[JS][2];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = wi * 64 + it * 16 + r16;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                af[it][c] =
                    *reinterpret_cast<const v8bf*>(At + lds_off(row, 4 * c + g, lds_swz_bf16(row)));
        }
#pragma unroll
        for (int js = 0; js < JS; ++js) {
            const int row = wj * (T / 2) + js * 16 + r16;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                bfr[js][c] =
                    *reinterpret_cast<const v8bf*>(Bt + lds_off(row, 4 * c + g, lds_swz_bf16(row)));
        }
        if (ks + 1 < nks) issue_loads(ks + 1, buf ^ 1);
#pragma unroll
        for (int js = 0; js < JS; ++js) {
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
    if (j0 + (T / 2) * wj >= J) return;
    if constexpr (OUT_BF16) {
        // Restage the wave's 64 x T/2 BF16 patch through LDS so that it leaves
        // as whole T-byte rows in 16-byte stores (chunks XOR-swizzled by row).
        constexpr int CH = T / 16;                       // 16-byte chunks per staged row
        uint8_t* stage = (wave < 4 ? &As[0][0] : &Bs[0][0]) + (wave & 3) * (64 * T);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = it * 16 + r16;
#pragma unroll
            for (int js = 0; js < JS; ++js) {
                const int b = js * 32 + g * 8;
                const int phys = (((b >> 4) ^ (row & (CH - 1))) << 4) | (b & 15);
                *reinterpret_cast<uint2*>(stage + row * T + phys) =
                    make_uint2(pack_bf16x2(acc[it][js][0], acc[it][js][1]),
                               pack_bf16x2(acc[it][js][2], acc[it][js][3]));
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): the wave's LDS writes
        __builtin_amdgcn_wave_barrier();
        uint16_t* Cb = reinterpret_cast<uint16_t*>(C);
#pragma unroll
        for (int pass = 0; pass < CH; ++pass) {
            const int row = pass * (64 / CH) + lane / CH;
            const int c = lane % CH;
            const uint4 w =
                *reinterpret_cast<const uint4*>(stage + row * T + ((c ^ (row & (CH - 1))) << 4));
            const int64_t i = i0 + wi * 64 + row;
            if (i < I) *reinterpret_cast<uint4*>(Cb + i * J + j0 + wj * (T / 2) + c * 8) = w;
        }
        return;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int64_t i = i0 + wi * 64 + it * 16 + r16;
        if (i >= I) continue;
#pragma unroll
        for (int js = 0; js < JS; ++js) {
            const int64_t j = j0 + wj * (T / 2) + js * 16 + 4 * g;
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

template <int T>
static hipError_t launch_bf16_tiles(const uint16_t* A, const uint16_t* B, void* C, bool out_bf16,
                                    int64_t I, int64_t J, int64_t K, hipStream_t stream) {
    const int64_t tiles_i = (I + T - 1) / T;
    const int64_t tiles_j = (J + T - 1) / T;
    const int64_t blocks = tiles_i * tiles_j;
    if (blocks == 0) return hipSuccess;
    if (out_bf16)
        return launch(gemm_bf16_kernel<T, true>, grid1d(blocks), dim3(2 * T), stream, A, B, C, I,
                      J, K, (int)tiles_i, (int)tiles_j);
    return launch(gemm_bf16_kernel<T, false>, grid1d(blocks), dim3(2 * T), stream, A, B, C, I, J,
                  K, (int)tiles_i, (int)tiles_j);
}

// The 256 x 256 tile once it gives more than half the CUs a tile; below that
// the 128 x 128 tile (four times the workgroups, two per CU), which is the
// slower of the two per CU: at 2048 x 2048 outputs (64 large tiles) it took
// 27% less time, at 4096 x 2048 (128) 10% less, and at 2048 x 6144 (192) 55%
// more, with a 16,384-long contraction.
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, bool out_bf16,
                            int64_t I, int64_t J, int64_t K, int num_cus, hipStream_t stream) {
    const int64_t big_tiles = ((I + 255) / 256) * ((J + 255) / 256);
    if (2 * big_tiles > (num_cus > 0 ? num_cus : 256))
        return launch_bf16_tiles<256>(A, B, C, out_bf16, I, J, K, stream);
    return launch_bf16_tiles<128>(A, B, C, out_bf16, I, J, K, stream);
}

}  // namespace fp8bs
