// quantize.hip -- tile quantizers BF16 -> E4M3 codes + FP32 scales (gfx950).
//
// Puro-2B technical report, section 2 "FP8": the FP8 matmul operands use
// DeepSeek-V3-style fine-grained quantization -- 1x128 tiles for activations
// and gradients, 128x128 blocks for weights, one FP32 scale per tile.
//
// The kernels are HBM-bound (read 2 B and write 1 B per element per output
// axis, plus 4 B of scale per tile): row tiles, weight blocks, and token-axis
// tiles with or without the row tiles of the same read.  Loads are 16-byte vectors covering whole 128-byte lines,
// the amax is reduced across the lanes that share a tile, and the codes are
// produced by the packed FP32 -> E4M3 conversion instruction.  The per-tile
// divisions are table lookups (see tile_scale in device_common.h).
#include "device_common.h"
#include "internal.h"

namespace fp8bs {

// ---------------------------------------------------------------------------
// Row tiles.  The tensor [M, K] with K % 128 == 0 is a flat sequence of
// M*K/128 tiles of 128 consecutive elements, and s is the flat sequence of
// their scales, so the kernel is one-dimensional.  Eight lanes share a tile:
// lane l of the group holds elements [8l, 8l+8) and [64+8l, 64+8l+8), so each
// load instruction of a wave covers eight whole 128-byte lines.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 2;
constexpr int kRowTilesPerBlock = kRowThreads / 8 * kRowUnroll;   // 64

__global__ __launch_bounds__(kRowThreads) void quant_rowtile_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, float* __restrict__ s, int64_t ntiles) {
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int sub = threadIdx.x & 7;
    const int64_t base = (int64_t)blockIdx.x * kRowTilesPerBlock + (threadIdx.x >> 3);
    uint4 v[kRowUnroll][2];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
        int64_t t = base + u * (kRowThreads / 8);
        if (t < ntiles) {
            v[u][0] = load_stream16(x + t * 16 + sub);
            v[u][1] = load_stream16(x + t * 16 + 8 + sub);
        } else {
            v[u][0] = make_uint4(0, 0, 0, 0);
            v[u][1] = make_uint4(0, 0, 0, 0);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
        int64_t t = base + u * (kRowThreads / 8);
        uint32_t m = absmax_u4(absmax_u4(0u, v[u][0]), v[u][1]);
        m = absmax_fold(m);
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2));
        m = max(m, (uint32_t)__shfl_xor((int)m, 4));
        TileScale ts = tile_scale(m, &tab);
        if (t < ntiles) {
            q[t * 16 + sub] = quant8(v[u][0], ts.inv);
            q[t * 16 + 8 + sub] = quant8(v[u][1], ts.inv);
            if (sub == 0) s[t] = ts.s;
        }
    }
}

hipError_t launch_quant_rowtile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                hipStream_t stream) {
    int64_t ntiles = M * (K / kTile);
    if (ntiles == 0) return hipSuccess;
    int64_t blocks = (ntiles + kRowTilesPerBlock - 1) / kRowTilesPerBlock;
    hipLaunchKernelGGL(quant_rowtile_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q), s, ntiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight blocks.  One workgroup per 128x128 block: each thread loads 8 chunks
// of 8 BF16 (16 threads per 256-byte row), the block amax is reduced across
// the wave and then across the 4 waves through LDS.  With q_t the codes also
// go through an LDS tile and leave transposed, 16 bytes per store.
// ---------------------------------------------------------------------------
constexpr int kBlkThreads = 256;
constexpr int kBlkLdsStride = kTile + 4;   // bytes per code row in LDS

__global__ __launch_bounds__(kBlkThreads) void quant_block_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ q,
    uint8_t* __restrict__ q_t, float* __restrict__ s) {
    __shared__ uint32_t red[kBlkThreads / 64];
    __shared__ __align__(16) uint8_t codes[kTile * kBlkLdsStride];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int tid = threadIdx.x;
    const int64_t kb_count = K / kTile;
    const int64_t bi = blockIdx.x / kb_count, bj = blockIdx.x % kb_count;
    const int64_t n0 = bi * kTile, k0 = bj * kTile;

    uint4 v[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int c = i * kBlkThreads + tid;
        int row = c >> 4, cc = c & 15;
        v[i] = load_stream16(w + (n0 + row) * K + k0 + cc * 8);
        m = absmax_u4(m, v[i]);
    }
    m = absmax_fold(m);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    TileScale ts = tile_scale(m, &tab);
    if (tid == 0) s[bi * kb_count + bj] = ts.s;

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int c = i * kBlkThreads + tid;
        int row = c >> 4, cc = c & 15;
        uint2 code = quant8(v[i], ts.inv);
        *reinterpret_cast<uint2*>(q + (n0 + row) * K + k0 + cc * 8) = code;
        if (q_t) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kBlkLdsStride + cc * 8);
            dst[0] = code.x;
            dst[1] = code.y;
        }
    }
    if (!q_t) return;
    __syncthreads();
    // Thread -> 16 (n) x 4 (k) sub-block: read 16 dwords (rows n..n+15, bytes
    // k..k+3), transpose 4x4 byte groups, write 4 rows of q_t, 16 bytes each.
    const int nn = (tid & 7) * 16;
    const int kk = (tid >> 3) * 4;
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        d[i] = *reinterpret_cast<const uint32_t*>(codes + (nn + i) * kBlkLdsStride + kk);
    uint32_t out[4][4];   // out[k'][g] holds n = nn+4g .. nn+4g+3 of row kk+k'
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t a0 = d[4 * g + 0], a1 = d[4 * g + 1], a2 = d[4 * g + 2], a3 = d[4 * g + 3];
        // byte k' of a_i -> byte i of out[k']
        uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.b0 a1.b0 a0.b1 a1.b1
        uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
        uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.b2 a1.b2 a0.b3 a1.b3
        uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
        out[0][g] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
        out[1][g] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
        out[2][g] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
        out[3][g] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
#pragma unroll
    for (int kp = 0; kp < 4; ++kp)
        *reinterpret_cast<uint4*>(q_t + (k0 + kk + kp) * N + n0 + nn) =
            make_uint4(out[kp][0], out[kp][1], out[kp][2], out[kp][3]);
}

hipError_t launch_quant_block(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* q_t,
                              float* s, hipStream_t stream) {
    int64_t blocks = (N / kTile) * (K / kTile);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_block_kernel, dim3((unsigned)blocks), dim3(kBlkThreads), 0, stream, w,
                       N, K, q, q_t, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token-axis tiles, alone or with the row tiles from the same read.  One
// workgroup per 128 tokens x 128 channels: each channel column of the tile is
// one token-axis tile and each token row one row tile (1x128 along channels),
// so with ROWS the workgroup reads the BF16 tile once and writes both code
// sets and both scale sets (fp8_quantize_dual); without, only the token-axis
// ones (fp8_quantize_transposed).
//   512 threads: the 38 KB LDS tile allows four workgroups per CU, and with
//   eight waves each that is eight waves per SIMD to cover the loads' latency.
//   Rows: thread t holds chunk t%16 (8 channels) of rows 32q + t/16, q = 0..3;
//     the 16 lanes of a row reduce its amax with four lane swaps.
//   Columns: the tile is copied to LDS with token r stored at physical row
//     8*(r%16) + r/16 and a 72-dword row stride, so that the 64 lanes of a
//     column read below address 64 different dword banks (dword address
//     mod 64 is 8g + p mod 64) and each 16-lane row write is one contiguous
//     256-byte row; thread
//     (pair p, group g) then reads channels 2p, 2p+1 of tokens 16g .. 16g+15
//     and reduces each channel over the 8 groups.
// ---------------------------------------------------------------------------
constexpr int kDualThreads = 512;
constexpr int kDualStrideDw = 72;                    // dwords per LDS token row

__device__ __forceinline__ int dual_row(int r) { return ((r & 15) << 3) + (r >> 4); }

template <bool ROWS>
__global__ __launch_bounds__(kDualThreads) void quant_dual_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t C, uint8_t* __restrict__ q,
    float* __restrict__ s, uint8_t* __restrict__ qt, float* __restrict__ st) {
    __shared__ __align__(16) uint32_t tile[kTile * kDualStrideDw];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int tid = threadIdx.x;
    const int64_t cblocks = C / kTile;
    const int64_t mb = blockIdx.x / cblocks, cb = blockIdx.x % cblocks;
    const int64_t m0 = mb * kTile, c0 = cb * kTile;
    const int chunk = tid & 15;                         // 8 channels: 8*chunk .. +7
    const int rsub = tid >> 4;                          // rows rsub + 32q

    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = load_stream16(x + (m0 + 32 * i + rsub) * C + c0 + chunk * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + rsub;
        *reinterpret_cast<uint4*>(tile + dual_row(r) * kDualStrideDw + chunk * 4) = v[i];
    }

    __syncthreads();              // scale tables in LDS

    // Row tiles.
#pragma unroll
    for (int i = 0; i < 4 && ROWS; ++i) {
        uint32_t m = absmax_fold(absmax_u4(0u, v[i]));
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2));
        m = max(m, (uint32_t)__shfl_xor((int)m, 4));
        m = max(m, (uint32_t)__shfl_xor((int)m, 8));
        const TileScale ts = tile_scale(m, &tab);
        const int64_t row = m0 + 32 * i + rsub;
        *reinterpret_cast<uint2*>(q + row * C + c0 + chunk * 8) = quant8(v[i], ts.inv);
        if (chunk == 0) s[row * cblocks + cb] = ts.s;
    }
    __syncthreads();

    // Token-axis tiles.
    const int g = tid & 7;
    const int64_t mbn = M / kTile;
    {
        const int p = tid >> 3;                         // channel pair: 2p, 2p+1
        uint32_t d[16];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            d[i] = tile[dual_row(16 * g + i) * kDualStrideDw + p];
            m = absmax_pair(m, d[i]);
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
            uint32_t other = (uint32_t)__shfl_xor((int)m, o);
            m = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                                                  __builtin_bit_cast(ushort2_t, m),
                                                  __builtin_bit_cast(ushort2_t, other)));
        }
        const TileScale t0 = tile_scale(m & 0xFFFFu, &tab);
        const TileScale t1 = tile_scale(m >> 16, &tab);
        uint32_t w0[4], w1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = d[4 * j], b = d[4 * j + 1], c = d[4 * j + 2], e = d[4 * j + 3];
            w0[j] = cvt4_e4m3(bf16_lo(a) * t0.inv, bf16_lo(b) * t0.inv, bf16_lo(c) * t0.inv,
                              bf16_lo(e) * t0.inv);
            w1[j] = cvt4_e4m3(bf16_hi(a) * t1.inv, bf16_hi(b) * t1.inv, bf16_hi(c) * t1.inv,
                              bf16_hi(e) * t1.inv);
        }
        const int64_t ch = c0 + 2 * p;
        *reinterpret_cast<uint4*>(qt + ch * M + m0 + g * 16) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        *reinterpret_cast<uint4*>(qt + (ch + 1) * M + m0 + g * 16) =
            make_uint4(w1[0], w1[1], w1[2], w1[3]);
        if (g == 0) {
            st[ch * mbn + mb] = t0.s;
            st[(ch + 1) * mbn + mb] = t1.s;
        }
    }
}

hipError_t launch_quant_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt, float* st,
                                   hipStream_t stream) {
    int64_t blocks = (M / kTile) * (C / kTile);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_dual_kernel<false>, dim3((unsigned)blocks), dim3(kDualThreads), 0,
                       stream, x, M, C, (uint8_t*)nullptr, (float*)nullptr, qt, st);
    return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t M, int64_t C, uint8_t* q, float* s,
                             uint8_t* qt, float* st, hipStream_t stream) {
    int64_t blocks = (M / kTile) * (C / kTile);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_dual_kernel<true>, dim3((unsigned)blocks), dim3(kDualThreads), 0, stream,
                       x, M, C, q, s, qt, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Diagnostic: clamp + convert, elementwise (4 values per thread).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void encode_e4m3_kernel(const float* __restrict__ x, int64_t n,
                                                          uint8_t* __restrict__ q) {
    int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        float4 v = *reinterpret_cast<const float4*>(x + i);
        *reinterpret_cast<uint32_t*>(q + i) =
            cvt4_e4m3(clamp_e4m3(v.x), clamp_e4m3(v.y), clamp_e4m3(v.z), clamp_e4m3(v.w));
    } else {
        for (int64_t j = i; j < n; ++j)
            q[j] = (uint8_t)(cvt4_e4m3(clamp_e4m3(x[j]), 0.f, 0.f, 0.f) & 0xFFu);
    }
}

hipError_t launch_encode_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 1023) / 1024;
    hipLaunchKernelGGL(encode_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, q);
    return hipGetLastError();
}

}  // namespace fp8bs
