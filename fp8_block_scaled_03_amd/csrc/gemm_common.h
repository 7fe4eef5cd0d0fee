// gemm_common.h -- pieces shared by the GEMM kernels: LDS tile layout, the
// wait for direct global->LDS loads, and the workgroup -> output tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef float v4f __attribute__((ext_vector_type(4)));

// LDS tiles hold rows of 128 bytes (128 FP8 codes, or 64 BF16 values).
constexpr int kRowBytes = 128;

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of 16-byte chunk c (0..7, K = 16c .. 16c+15) of tile row r.  The
// chunk index is XORed with bits 1..3 of the row, so that the 16 lanes served
// together by a 16-byte LDS read (16 consecutive rows, one logical chunk)
// cover all 64 banks exactly once.
__device__ __forceinline__ int lds_off(int row, int c) {
    return row * kRowBytes + ((c ^ ((row >> 1) & 7)) << 4);
}

// vmcnt(0): this wave's global loads (including those into LDS) have landed.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Output tile of workgroup bid.  Tiles are handed out in groups of
// kGroupRows tile rows (column-major inside a group) so that workgroups in
// flight share operand panels; when the tile count is a multiple of 8, the
// workgroups the dispatcher sends to one XCD (bid % 8) get one contiguous run
// of that order, so the sharing happens inside one XCD's L2.
constexpr int kGroupRows = 4;

__device__ __forceinline__ void tile_coords(int bid, int tiles_i, int tiles_j, int* ti, int* tj) {
    const int T = tiles_i * tiles_j;
    int t = bid;
    if ((T & 7) == 0) t = (bid & 7) * (T >> 3) + (bid >> 3);      // contiguous chunk per XCD
    const int per_group = kGroupRows * tiles_j;
    const int grp = t / per_group;
    const int rows = min(kGroupRows, tiles_i - grp * kGroupRows);
    const int r = t - grp * per_group;
    *ti = grp * kGroupRows + r % rows;
    *tj = r / rows;
}

// Contraction split of a FP32-output GEMM: piece 0 sums blocks [0, p0) and
// writes the output itself; piece y >= 1 sums blocks [p0 + (y-1) nps,
// p0 + y nps) (the last one clipped to the contraction) into FP32 slice y-1
// of the workspace Wsp.  splitk_reduce_kernel then adds the slices to the
// output in piece order.  An unsplit launch has p0 = the block count.
__device__ __forceinline__ int split_begin(int y, int p0, int nps) {
    return y == 0 ? 0 : p0 + (y - 1) * nps;
}
__device__ __forceinline__ int split_end(int y, int p0, int nps, int nkb_all) {
    return min(nkb_all, y == 0 ? p0 : p0 + y * nps);
}
__device__ __forceinline__ float* split_out(int y, void* C, float* Wsp, int64_t I, int64_t J) {
    return y == 0 ? reinterpret_cast<float*>(C) : Wsp + (int64_t)(y - 1) * I * J;
}

}  // namespace fp8bs
