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

// Row r's 16-byte chunk c (0..7, K = 16c .. 16c+15) is stored at physical
// chunk c ^ swz(r).  A fragment read takes one logical chunk per lane group
// g = lane / 16 from 16 consecutive rows (lanes r16 = lane % 16).  Which row
// swizzle keeps those reads free of LDS bank conflicts depends on the chunks
// the four lane groups read; both swizzles below were chosen by rocprofv3's
// LDS bank-conflict counter (conflict cycles over LDS-active cycles):
//   lds_swz_fp8   rows' bits 0..2, bit 3 flipping the lowest: for reads in
//                 which group g takes chunks 2g and 2g+1 (the FP8 tiles of
//                 the FP8-MFMA and the 128x128 kernels): 0-5%, against
//                 46-49% with lds_swz_bf16;
//   lds_swz_bf16  rows' bits 1..3: for reads in which group g takes chunk g
//                 or 4+g (the BF16 comparator's tiles): 3%, against 50% with
//                 lds_swz_fp8.
__device__ __forceinline__ int lds_swz_fp8(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_swz_bf16(int row) { return (row >> 1) & 7; }

// Byte offset of 16-byte chunk c of tile row `row` under row swizzle swz.
__device__ __forceinline__ int lds_off(int row, int c, int swz) {
    return row * kRowBytes + ((c ^ swz) << 4);
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
