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
#include <algorithm>

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
    return launch(quant_rowtile_kernel, grid1d(blocks), dim3(kRowThreads), stream,
                  reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q), s, ntiles);
}

// ---------------------------------------------------------------------------
// Weight blocks.  One workgroup per 128x128 block.  Thread t loads the 16-byte
// chunk c = t % 16 (8 BF16) of the four consecutive rows 4 (t / 16) + j and,
// in a second pass, of the rows 64 further on: each load instruction of a wave
// covers four whole 256-byte rows.  The block amax is reduced across the wave
// and then across the 4 waves through LDS.  The codes go out row-major as they
// are (8 bytes per thread and row, whole 128-byte rows per instruction), and,
// for q_t, each 4 rows x 4 columns of a thread are transposed in registers (4
// byte permutes per 4 dwords) into four dwords, each holding 4 consecutive
// rows n of one column k.  Those go to an LDS tile laid out as q_t[k][n] with
// the 16-byte chunks of row k XOR-swizzled by (k / 8) % 8: a dword store of a
// wave then touches 32 banks twice at most, and the 16-byte reads that feed
// the q_t stores (eight lanes per 128-byte row of q_t) are conflict-free.
// ---------------------------------------------------------------------------
constexpr int kBlkThreads = 256;

// Dword index in the transposed LDS tile of (k, n/4).
__device__ __forceinline__ int blk_t_dword(int k, int n4) {
    return k * 32 + (n4 ^ (((k >> 3) & 7) << 2));
}

// 4x4 byte transpose: byte j of a_i -> byte i of out[j].
__device__ __forceinline__ void transpose4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                             uint32_t out[4]) {
    const uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.b0 a1.b0 a0.b1 a1.b1
    const uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.b2 a1.b2 a0.b3 a1.b3
    const uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Block `blk` (row-major over the N/128 x K/128 blocks) of one weight; the
// caller provides the LDS and loads the scale tables.
__device__ __forceinline__ void block_tile(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                           uint8_t* __restrict__ q, uint8_t* __restrict__ q_t,
                                           float* __restrict__ s, int64_t blk, uint32_t* red,
                                           uint32_t* tile_t, const ScaleTables& tab) {
    const int tid = threadIdx.x;
    const int64_t kb_count = K / kTile;
    const int64_t bi = blk / kb_count, bj = blk % kb_count;
    const int64_t n0 = bi * kTile, k0 = bj * kTile;
    const int cc = tid & 15;              // 16-byte chunk of the row: columns 8cc .. 8cc+7
    const int rg = tid >> 4;              // rows 4rg .. 4rg+3 (+64 in the second pass)

    uint4 v[2][4];
    uint32_t m = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 64 * h + 4 * rg + j;
            v[h][j] = load_stream16(w + (n0 + row) * K + k0 + cc * 8);
            m = absmax_u4(m, v[h][j]);
        }
    m = absmax_fold(m);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const TileScale ts = tile_scale(m, &tab);
    if (tid == 0) s[bi * kb_count + bj] = ts.s;   // (tile_scale reads tab, published by the barrier above)

#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint2 code[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 64 * h + 4 * rg + j;
            code[j] = quant8(v[h][j], ts.inv);
            *reinterpret_cast<uint2*>(q + (n0 + row) * K + k0 + cc * 8) = code[j];
        }
        if (q_t) {
            const int n4 = 16 * h + rg;   // rows 4 n4 .. 4 n4 + 3
            uint32_t t0[4], t1[4];
            transpose4x4(code[0].x, code[1].x, code[2].x, code[3].x, t0);   // columns 8cc .. +3
            transpose4x4(code[0].y, code[1].y, code[2].y, code[3].y, t1);   // columns 8cc+4 .. +7
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                tile_t[blk_t_dword(8 * cc + kk, n4)] = t0[kk];
                tile_t[blk_t_dword(8 * cc + 4 + kk, n4)] = t1[kk];
            }
        }
    }
    if (!q_t) return;
    __syncthreads();
    // Row k of q_t's block, 16 rows n per lane: eight lanes per 128-byte row.
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int k = 32 * p + (tid >> 3);
        const int ch = tid & 7;                        // n = 16 ch .. 16 ch + 15
        const uint4 d = *reinterpret_cast<const uint4*>(&tile_t[blk_t_dword(k, 4 * ch)]);
        *reinterpret_cast<uint4*>(q_t + (k0 + k) * N + n0 + 16 * ch) = d;
    }
}

__global__ __launch_bounds__(kBlkThreads) void quant_block_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ q,
    uint8_t* __restrict__ q_t, float* __restrict__ s) {
    __shared__ uint32_t red[kBlkThreads / 64];
    __shared__ __align__(16) uint32_t tile_t[kTile * kTile / 4];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    block_tile(w, N, K, q, q_t, s, blockIdx.x, red, tile_t, tab);
}

// Several weights in one launch: workgroup b quantizes block b - first[j] of
// job j, first[j] <= b < first[j + 1].  One launch of all the blocks fills the
// CUs where a weight alone (256 to 1536 blocks) leaves many idle or in a
// ragged last round.
__global__ __launch_bounds__(kBlkThreads) void quant_block_many_kernel(BlockJobs jobs) {
    __shared__ uint32_t red[kBlkThreads / 64];
    __shared__ __align__(16) uint32_t tile_t[kTile * kTile / 4];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int64_t b = blockIdx.x;
    int j = 0;
    while (j + 1 < jobs.count && b >= jobs.first[j + 1]) ++j;
    const BlockJob& job = jobs.job[j];
    block_tile(job.w, job.N, job.K, job.q, job.q_t, job.s, b - jobs.first[j], red, tile_t, tab);
}

hipError_t launch_quant_block(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* q_t,
                              float* s, hipStream_t stream) {
    int64_t blocks = (N / kTile) * (K / kTile);
    if (blocks == 0) return hipSuccess;
    return launch(quant_block_kernel, grid1d(blocks), dim3(kBlkThreads), stream, w, N, K,
                  q, q_t, s);
}

hipError_t launch_quant_block_many(const BlockJobs& jobs, hipStream_t stream) {
    const int64_t blocks = jobs.first[jobs.count];
    if (blocks == 0) return hipSuccess;
    return launch(quant_block_many_kernel, grid1d(blocks), dim3(kBlkThreads), stream, jobs);
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

// Where a thread's BF16 values come from: 8 consecutive channels (col ..
// col+7) of token row `row`, the thread's i-th row of the tile (i = 0..3).
// DualPlain reads them from X [M, C].
struct DualPlain {
    const uint16_t* __restrict__ x;
    int64_t C;
    __device__ __forceinline__ uint4 operator()(int, int64_t row, int64_t col) const {
        return load_stream16(x + row * C + col);
    }
};

// Gates below kLowGate.  There 1 + e^g is 1 in FP32, so sigmoid(g) equals
// e^g and 1 - sigmoid(g) equals 1 to FP32 precision.  Further down, e^-g
// overflows FP32 (g < -88.7) and 1 / (1 + e^-g) is an FP32 denormal
// (g < -87.3), while the products that contain sigmoid(g) can still be normal
// BF16 values (BF16 reaches down to 2^-133, and |u| up to 2^128).  So below
// kLowGate those products are formed from logarithms (exp_product).
constexpr float kLowGate = -64.0f;

// log2|x| for finite x != 0, FP32 denormals included (scaled by 2^64 first).
__device__ __forceinline__ float log2_abs(float x) {
    const float a = fabsf(x);
    return a < 1.17549435e-38f ? __log2f(a * 18446744073709551616.0f) - 64.0f : __log2f(a);
}

// x y z e^g for g < kLowGate, with any finite x, y, z:
// sign(x y z) 2^L, L = log2|x| + log2|y| + log2|z| + g log2(e).  The integer
// part of L is applied by ldexp (a single rounding, into the denormals when
// the result is that small), the fraction by the hardware exponential.  L's
// rounding (an absolute error near 2^-15 at g = -300) makes the relative
// error near 2^-15, far inside BF16's 2^-9 rounding step.
__device__ __forceinline__ float exp_product(float g, float x, float y, float z) {
    const uint32_t sign =
        (__float_as_uint(x) ^ __float_as_uint(y) ^ __float_as_uint(z)) & 0x80000000u;
    if (x == 0.0f || y == 0.0f || z == 0.0f) return __uint_as_float(sign);
    // Below 2^-300 the result is zero in FP32; the floor keeps the exponent an int.
    const float l =
        fmaxf(log2_abs(x) + log2_abs(y) + log2_abs(z) + g * 1.44269504f, -300.0f);
    const float n = floorf(l);
    const float r = ldexpf(__builtin_amdgcn_exp2f(l - n), (int)n);
    return __uint_as_float(__float_as_uint(r) | sign);
}

// SwiGLU of the MLP, formed on the way in: h = silu(g) * u, silu(g) =
// g / (1 + e^-g), in FP32 and rounded to BF16 (ties to even), with the gate g
// in columns 0..F-1 of the gate/up projection's output [M, 2F] and the up
// value u in columns F..2F-1.  The exponential and the reciprocal are the
// hardware approximations (relative error near 2^-20 for the gates of real
// activations), far inside BF16's 2^-9 rounding step; below kLowGate,
// h = g u e^g by exp_product.  H itself is stored only when h is given.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    if (g < kLowGate) return exp_product(g, g, u, 1.0f);
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}
struct DualSwiglu {
    const uint16_t* __restrict__ gu;
    int64_t F;
    uint16_t* __restrict__ h;
    __device__ __forceinline__ uint4 operator()(int, int64_t row, int64_t col) const {
        const uint16_t* p = gu + row * 2 * F + col;
        const uint4 g = load_stream16(p), u = load_stream16(p + F);
        uint4 r;
        r.x = pack_bf16x2(swiglu_f32(bf16_lo(g.x), bf16_lo(u.x)), swiglu_f32(bf16_hi(g.x), bf16_hi(u.x)));
        r.y = pack_bf16x2(swiglu_f32(bf16_lo(g.y), bf16_lo(u.y)), swiglu_f32(bf16_hi(g.y), bf16_hi(u.y)));
        r.z = pack_bf16x2(swiglu_f32(bf16_lo(g.z), bf16_lo(u.z)), swiglu_f32(bf16_hi(g.z), bf16_hi(u.z)));
        r.w = pack_bf16x2(swiglu_f32(bf16_lo(g.w), bf16_lo(u.w)), swiglu_f32(bf16_hi(g.w), bf16_hi(u.w)));
        if (h) *reinterpret_cast<uint4*>(h + row * F + col) = r;
        return r;
    }
};

// SwiGLU backward, formed on the way in: for column f of H, the gate half of
// the gate/up gradient [M, 2F] is d_gate = dh * u * silu'(g), silu'(g) =
// s (1 + g (1 - s)) with s = 1 / (1 + e^-g), and the up half (column F + f)
// is d_up = dh * silu(g) = dh * g * s, each rounded to BF16.  1 - s is taken
// as e^-g * s for g >= 0 (no cancellation as s nears 1) and as 1 - s below
// (where s < 1/2).  Below kLowGate, s = e^g and 1 - s = 1, so d_gate =
// dh u (1 + g) e^g and d_up = dh g e^g, both by exp_product.  Above it the
// products are formed in FP32 in the order written, each rounding once; where
// dh * u overflows FP32 (the gradient itself need not, silu'(g) being as
// small as 1e-26 there), d_gate comes from logarithms too.  One workgroup
// quantizes the gate tile and then the up tile of the same tokens and
// columns f: the first pass keeps the thread's dh and g in registers for the
// second, so each input is read once.  The BF16 gradient is stored only when
// dgu is given.
__device__ __forceinline__ float swiglu_bwd_gate_f32(float d, float g, float u) {
    if (g < kLowGate) return exp_product(g, d, u, 1.0f + g);
    const float e = __expf(-g);
    const float sg = __builtin_amdgcn_rcpf(1.0f + e);
    const float om = g >= 0.0f ? e * sg : 1.0f - sg;
    const float ds = sg * (1.0f + g * om);
    const float du = d * u;
    if (!(fabsf(du) <= 3.40282347e38f)) return exp_product(0.0f, d, u, ds);
    return du * ds;
}
__device__ __forceinline__ float swiglu_bwd_up_f32(float d, float g) {
    if (g < kLowGate) return exp_product(g, d, g, 1.0f);
    return d * (g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)));
}
struct SwigluBwdRegs {
    uint4 d[4], g[4];
};
struct DualSwigluBwdGate {
    const uint16_t* __restrict__ dh;
    const uint16_t* __restrict__ gu;
    int64_t F;
    uint16_t* __restrict__ dgu;
    SwigluBwdRegs* keep;
    __device__ __forceinline__ uint4 operator()(int i, int64_t row, int64_t f) const {
        const uint4 d = load_stream16(dh + row * F + f);
        const uint4 g = load_stream16(gu + row * 2 * F + f);
        const uint4 u = load_stream16(gu + row * 2 * F + F + f);
        keep->d[i] = d;
        keep->g[i] = g;
        uint4 r;
        r.x = pack_bf16x2(swiglu_bwd_gate_f32(bf16_lo(d.x), bf16_lo(g.x), bf16_lo(u.x)),
                          swiglu_bwd_gate_f32(bf16_hi(d.x), bf16_hi(g.x), bf16_hi(u.x)));
        r.y = pack_bf16x2(swiglu_bwd_gate_f32(bf16_lo(d.y), bf16_lo(g.y), bf16_lo(u.y)),
                          swiglu_bwd_gate_f32(bf16_hi(d.y), bf16_hi(g.y), bf16_hi(u.y)));
        r.z = pack_bf16x2(swiglu_bwd_gate_f32(bf16_lo(d.z), bf16_lo(g.z), bf16_lo(u.z)),
                          swiglu_bwd_gate_f32(bf16_hi(d.z), bf16_hi(g.z), bf16_hi(u.z)));
        r.w = pack_bf16x2(swiglu_bwd_gate_f32(bf16_lo(d.w), bf16_lo(g.w), bf16_lo(u.w)),
                          swiglu_bwd_gate_f32(bf16_hi(d.w), bf16_hi(g.w), bf16_hi(u.w)));
        if (dgu) *reinterpret_cast<uint4*>(dgu + row * 2 * F + f) = r;
        return r;
    }
};
struct DualSwigluBwdUp {
    int64_t F;
    uint16_t* __restrict__ dgu;
    const SwigluBwdRegs* keep;
    __device__ __forceinline__ uint4 operator()(int i, int64_t row, int64_t col) const {
        const uint4 d = keep->d[i], g = keep->g[i];
        uint4 r;
        r.x = pack_bf16x2(swiglu_bwd_up_f32(bf16_lo(d.x), bf16_lo(g.x)),
                          swiglu_bwd_up_f32(bf16_hi(d.x), bf16_hi(g.x)));
        r.y = pack_bf16x2(swiglu_bwd_up_f32(bf16_lo(d.y), bf16_lo(g.y)),
                          swiglu_bwd_up_f32(bf16_hi(d.y), bf16_hi(g.y)));
        r.z = pack_bf16x2(swiglu_bwd_up_f32(bf16_lo(d.z), bf16_lo(g.z)),
                          swiglu_bwd_up_f32(bf16_hi(d.z), bf16_hi(g.z)));
        r.w = pack_bf16x2(swiglu_bwd_up_f32(bf16_lo(d.w), bf16_lo(g.w)),
                          swiglu_bwd_up_f32(bf16_hi(d.w), bf16_hi(g.w)));
        if (dgu) *reinterpret_cast<uint4*>(dgu + row * 2 * F + col) = r;
        return r;
    }
};

// One 128 x 128 tile (token block mb, channel block cb of C channels): its
// row tiles and token-axis tiles.  `tile` is the workgroup's LDS tile and
// `tab` its scale tables (loaded by the caller; the first barrier below
// publishes them).
// RMSNorm, formed on the way in: y = x * r * gamma in FP32, rounded to
// BF16, with r = 1/sqrt(mean(x^2) + eps) of the token row, computed for every
// row beforehand (rmsnorm_rstd_kernel).  y itself is stored only when given.
struct DualRmsNorm {
    const uint16_t* __restrict__ x;
    int64_t C;
    const uint16_t* __restrict__ gamma;
    const float* __restrict__ rstd;
    uint16_t* __restrict__ y;
    __device__ __forceinline__ uint4 operator()(int, int64_t row, int64_t col) const {
        const uint4 v = load_stream16(x + row * C + col);
        const uint4 w = *reinterpret_cast<const uint4*>(gamma + col);
        const float r = rstd[row];
        uint4 o;
        o.x = pack_bf16x2(bf16_lo(v.x) * r * bf16_lo(w.x), bf16_hi(v.x) * r * bf16_hi(w.x));
        o.y = pack_bf16x2(bf16_lo(v.y) * r * bf16_lo(w.y), bf16_hi(v.y) * r * bf16_hi(w.y));
        o.z = pack_bf16x2(bf16_lo(v.z) * r * bf16_lo(w.z), bf16_hi(v.z) * r * bf16_hi(w.z));
        o.w = pack_bf16x2(bf16_lo(v.w) * r * bf16_lo(w.w), bf16_hi(v.w) * r * bf16_hi(w.w));
        if (y) *reinterpret_cast<uint4*>(y + row * C + col) = o;
        return o;
    }
};

template <bool ROWS, class Src>
__device__ __forceinline__ void dual_tile(const Src& src, int64_t M, int64_t C, int64_t mb,
                                          int64_t cb, uint32_t* __restrict__ tile,
                                          const ScaleTables& tab, uint8_t* __restrict__ q,
                                          float* __restrict__ s, uint8_t* __restrict__ qt,
                                          float* __restrict__ st) {
    const int tid = threadIdx.x;
    const int64_t cblocks = C / kTile;
    const int64_t m0 = mb * kTile, c0 = cb * kTile;
    const int chunk = tid & 15;                         // 8 channels: 8*chunk .. +7
    const int rsub = tid >> 4;                          // rows rsub + 32q

    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = src(i, m0 + 32 * i + rsub, c0 + chunk * 8);
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

template <bool ROWS>
__global__ __launch_bounds__(kDualThreads) void quant_dual_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t C, uint8_t* __restrict__ q,
    float* __restrict__ s, uint8_t* __restrict__ qt, float* __restrict__ st) {
    __shared__ __align__(16) uint32_t tile[kTile * kDualStrideDw];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int64_t cblocks = C / kTile;
    dual_tile<ROWS>(DualPlain{x, C}, M, C, blockIdx.x / cblocks, blockIdx.x % cblocks, tile, tab,
                    q, s, qt, st);
}

__global__ __launch_bounds__(kDualThreads) void swiglu_dual_kernel(
    const uint16_t* __restrict__ gu, int64_t M, int64_t F, uint8_t* __restrict__ q,
    float* __restrict__ s, uint8_t* __restrict__ qt, float* __restrict__ st,
    uint16_t* __restrict__ h) {
    __shared__ __align__(16) uint32_t tile[kTile * kDualStrideDw];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int64_t fblocks = F / kTile;
    dual_tile<true>(DualSwiglu{gu, F, h}, M, F, blockIdx.x / fblocks, blockIdx.x % fblocks, tile,
                    tab, q, s, qt, st);
}

__global__ __launch_bounds__(kDualThreads) void swiglu_bwd_dual_kernel(
    const uint16_t* __restrict__ dh, const uint16_t* __restrict__ gu, int64_t M, int64_t F,
    uint8_t* __restrict__ q, float* __restrict__ s, uint8_t* __restrict__ qt,
    float* __restrict__ st, uint16_t* __restrict__ dgu) {
    __shared__ __align__(16) uint32_t tile[kTile * kDualStrideDw];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int64_t fblocks = F / kTile;
    const int64_t mb = blockIdx.x / fblocks, fb = blockIdx.x % fblocks;
    SwigluBwdRegs keep;
    dual_tile<true>(DualSwigluBwdGate{dh, gu, F, dgu, &keep}, M, 2 * F, mb, fb, tile, tab, q, s,
                    qt, st);
    __syncthreads();              // every thread is done with the LDS tile of the gate pass
    // The kept values pass through an empty asm statement after the barrier,
    // so the up pass's arithmetic is not hoisted into the gate pass (where
    // its results would hold registers across the whole pass).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        asm volatile("" : "+v"(keep.d[i].x), "+v"(keep.d[i].y), "+v"(keep.d[i].z), "+v"(keep.d[i].w));
        asm volatile("" : "+v"(keep.g[i].x), "+v"(keep.g[i].y), "+v"(keep.g[i].z), "+v"(keep.g[i].w));
    }
    dual_tile<true>(DualSwigluBwdUp{F, dgu, &keep}, M, 2 * F, mb, fblocks + fb, tile, tab, q, s,
                    qt, st);
}

// r = 1/sqrt(mean(x^2) + eps) per token row: one wave per row, each lane
// summing the squares of its 16-byte pieces (columns 8l, 8l + 512, ...) in
// FP32, then a butterfly over the wave; correctly rounded square root and
// division.  Four rows per 256-thread workgroup.
constexpr int64_t kRstdMaxBlocks = 1 << 20;   // 4M rows per pass of the grid

__global__ __launch_bounds__(256) void rmsnorm_rstd_kernel(const uint16_t* __restrict__ x,
                                                           int64_t M, int64_t C, float eps,
                                                           float* __restrict__ rstd) {
    const int lane = threadIdx.x & 63;
    // One wave per row; the grid is capped (kRstdMaxBlocks), so a wave may
    // take several rows, gridDim.x * 4 apart.
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < M;
         row += (int64_t)gridDim.x * 4) {
        const uint16_t* xr = x + row * C;
        float ss = 0.f;
        for (int64_t c = 8 * lane; c < C; c += 512) {
            const uint4 v = load_stream16(xr + c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = bf16_lo(w[j]), b = bf16_hi(w[j]);
                ss = __builtin_fmaf(a, a, ss);
                ss = __builtin_fmaf(b, b, ss);
            }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);   // the same sum in every lane
        float r = 1.0f / sqrtf(ss / (float)C + eps);
        // The sum of squares left FP32's range: it overflowed (|x| above
        // about 1e19), or the squares underflowed (every |x| below about
        // 2^-50) while eps is too small to dominate them.  Such a row is
        // summed again as x 2^-k, k the exponent of its largest |x|, and
        // r = 2^-k / sqrt(mean((x 2^-k)^2) + eps 2^-2k).
        if (!(ss <= 3.0e38f) || (ss < 0x1p-100f && eps < 0x1p-60f)) {
            float amax = 0.f;
            for (int64_t c = 8 * lane; c < C; c += 512) {
                const uint4 v = load_stream16(xr + c);
                amax = fmaxf(amax, __uint_as_float(absmax_fold(absmax_u4(0u, v)) << 16));
            }
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            if (amax > 0.f) {
                int k;
                frexpf(amax, &k);                       // amax = m 2^k, m in [1/2, 1)
                float s2 = 0.f;
                for (int64_t c = 8 * lane; c < C; c += 512) {
                    const uint4 v = load_stream16(xr + c);
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float a = ldexpf(bf16_lo(w[j]), -k), b = ldexpf(bf16_hi(w[j]), -k);
                        s2 = __builtin_fmaf(a, a, s2);
                        s2 = __builtin_fmaf(b, b, s2);
                    }
                }
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) s2 += __shfl_xor(s2, o);
                int ke = 0;
                if (eps > 0.f) frexpf(eps, &ke);
                // eps 2^-2k above 2^100 dominates the mean (at most 1) beyond FP32 precision
                r = (eps > 0.f && ke - 2 * k > 100)
                        ? 1.0f / sqrtf(eps)
                        : ldexpf(1.0f / sqrtf(s2 / (float)C + ldexpf(eps, -2 * k)), -k);
            }
        }
        if (lane == 0) rstd[row] = r;
    }
}

__global__ __launch_bounds__(kDualThreads) void rmsnorm_dual_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
    const float* __restrict__ rstd, int64_t M, int64_t C, uint8_t* __restrict__ q,
    float* __restrict__ s, uint8_t* __restrict__ qt, float* __restrict__ st,
    uint16_t* __restrict__ y) {
    __shared__ __align__(16) uint32_t tile[kTile * kDualStrideDw];
    __shared__ ScaleTables tab;
    load_scale_tables(&tab);
    const int64_t cblocks = C / kTile;
    dual_tile<true>(DualRmsNorm{x, C, gamma, rstd, y}, M, C, blockIdx.x / cblocks,
                    blockIdx.x % cblocks, tile, tab, q, s, qt, st);
}

hipError_t launch_rmsnorm_dual(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                               int64_t C, uint8_t* q, float* s, uint8_t* qt, float* st,
                               float* rstd, uint16_t* y, hipStream_t stream) {
    if (M == 0 || C == 0) return hipSuccess;
    // The dual kernel's grid is checked first, so that a refused call
    // enqueues nothing.
    const int64_t tiles = (M / kTile) * (C / kTile);
    if ((uint64_t)tiles * kDualThreads > kMaxGridItems) return hipErrorInvalidConfiguration;
    const int64_t rstd_blocks = std::min<int64_t>((M + 3) / 4, kRstdMaxBlocks);
    hipError_t e = launch(rmsnorm_rstd_kernel, grid1d(rstd_blocks), dim3(256), stream, x, M, C, eps,
                          rstd);
    if (e != hipSuccess) return e;
    return launch(rmsnorm_dual_kernel, grid1d(tiles), dim3(kDualThreads), stream, x, gamma,
                  (const float*)rstd, M, C, q, s, qt, st, y);
}

hipError_t launch_swiglu_bwd_dual(const uint16_t* dh, const uint16_t* gu, int64_t M, int64_t F,
                                  uint8_t* q, float* s, uint8_t* qt, float* st, uint16_t* dgu,
                                  hipStream_t stream) {
    int64_t blocks = (M / kTile) * (F / kTile);
    if (blocks == 0) return hipSuccess;
    return launch(swiglu_bwd_dual_kernel, grid1d(blocks), dim3(kDualThreads), stream, dh,
                  gu, M, F, q, s, qt, st, dgu);
}

hipError_t launch_swiglu_dual(const uint16_t* gu, int64_t M, int64_t F, uint8_t* q, float* s,
                              uint8_t* qt, float* st, uint16_t* h, hipStream_t stream) {
    int64_t blocks = (M / kTile) * (F / kTile);
    if (blocks == 0) return hipSuccess;
    return launch(swiglu_dual_kernel, grid1d(blocks), dim3(kDualThreads), stream, gu, M, F,
                  q, s, qt, st, h);
}

hipError_t launch_quant_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt, float* st,
                                   hipStream_t stream) {
    int64_t blocks = (M / kTile) * (C / kTile);
    if (blocks == 0) return hipSuccess;
    return launch(quant_dual_kernel<false>, grid1d(blocks), dim3(kDualThreads), stream, x,
                  M, C, (uint8_t*)nullptr, (float*)nullptr, qt, st);
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t M, int64_t C, uint8_t* q, float* s,
                             uint8_t* qt, float* st, hipStream_t stream) {
    int64_t blocks = (M / kTile) * (C / kTile);
    if (blocks == 0) return hipSuccess;
    return launch(quant_dual_kernel<true>, grid1d(blocks), dim3(kDualThreads), stream, x, M,
                  C, q, s, qt, st);
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
    return launch(encode_e4m3_kernel, grid1d(blocks), dim3(256), stream, x, n, q);
}

// ---------------------------------------------------------------------------
// Diagnostic: the quantizers' memory traffic without their arithmetic.  Each
// thread reads 16 BF16 values (32 bytes, non-temporal) and writes their 16
// high bytes to y0 and, when y1 is given, their 16 low bytes to y1: 2 bytes
// read and 1 or 2 bytes written per element, in 16-byte accesses, the
// streaming pattern of the row-tile / token-axis quantizers (one code array)
// and of the dual-axis quantizer (two).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hbm_rate_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                       uint8_t* __restrict__ y0,
                                                       uint8_t* __restrict__ y1) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (i + 16 <= n) {
        const uint4 a = load_stream16(x + i);
        const uint4 b = load_stream16(x + i + 8);
        // bytes 1, 3, 5, 7 of each 8-byte half: the high bytes of four values
        auto hi4 = [](uint32_t u, uint32_t v) { return __builtin_amdgcn_perm(v, u, 0x07050301u); };
        auto lo4 = [](uint32_t u, uint32_t v) { return __builtin_amdgcn_perm(v, u, 0x06040200u); };
        *reinterpret_cast<uint4*>(y0 + i) =
            make_uint4(hi4(a.x, a.y), hi4(a.z, a.w), hi4(b.x, b.y), hi4(b.z, b.w));
        if (y1)
            *reinterpret_cast<uint4*>(y1 + i) =
                make_uint4(lo4(a.x, a.y), lo4(a.z, a.w), lo4(b.x, b.y), lo4(b.z, b.w));
    } else {
        for (int64_t j = i; j < n; ++j) {
            y0[j] = (uint8_t)(x[j] >> 8);
            if (y1) y1[j] = (uint8_t)(x[j] & 0xFFu);
        }
    }
}

hipError_t launch_hbm_rate(const uint16_t* x, int64_t n, uint8_t* y0, uint8_t* y1,
                           hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int64_t blocks = (n + 4095) / 4096;
    return launch(hbm_rate_kernel, grid1d(blocks), dim3(256), stream, x, n, y0, y1);
}

}  // namespace fp8bs
