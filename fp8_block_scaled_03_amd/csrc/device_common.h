// device_common.h -- device helpers shared by the libfp8bs HIP kernels (gfx950 only).
//
// E4M3 here is OCP E4M3FN, the format gfx950's FP8 conversion and MFMA
// instructions use.  The tile rule (Puro-2B technical report, section 2
// "FP8", after DeepSeek-V3's fine-grained quantization): a = max(amax, 2^-100),
// s = a/448, inv = 448/a (both correctly rounded), code = RNE(clamp(x*inv)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxFloor = 0x1p-100f;
constexpr int kTile = 128;

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: marked non-temporal).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Two BF16 values packed in a dword -> FP32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Running max of |x| over packed BF16 pairs, as 15-bit magnitudes.  For finite
// values the magnitude bit pattern orders like the value, so this is exact.
__device__ __forceinline__ uint32_t absmax_pair(uint32_t m, uint32_t pair) {
    ushort2_t a = __builtin_bit_cast(ushort2_t, m);
    ushort2_t b = __builtin_bit_cast(ushort2_t, pair & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
__device__ __forceinline__ uint32_t absmax_fold(uint32_t m) { return max(m & 0xFFFFu, m >> 16); }

// amax (15-bit BF16 magnitude) -> (scale, inverse scale), both correctly rounded.
struct TileScale {
    float s;
    float inv;
};
__device__ __forceinline__ TileScale tile_scale(uint32_t amax_bits) {
    float amax = __uint_as_float(amax_bits << 16);
    float a = fmaxf(amax, kAmaxFloor);
    TileScale t;
    t.s = __fdiv_rn(a, kE4M3Max);
    t.inv = __fdiv_rn(kE4M3Max, a);
    return t;
}

__device__ __forceinline__ float clamp_e4m3(float p) {
    return __builtin_amdgcn_fmed3f(p, -kE4M3Max, kE4M3Max);
}

// Four FP32 values (already within +-448) -> four E4M3 codes, byte i = value i.
// v_cvt_pk_fp8_f32 rounds to nearest even and keeps the sign of zero.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// Eight BF16 values (a uint4) times inv -> eight codes (a uint2).
__device__ __forceinline__ uint2 quant8(uint4 v, float inv) {
    uint2 r;
    r.x = cvt4_e4m3(clamp_e4m3(bf16_lo(v.x) * inv), clamp_e4m3(bf16_hi(v.x) * inv),
                    clamp_e4m3(bf16_lo(v.y) * inv), clamp_e4m3(bf16_hi(v.y) * inv));
    r.y = cvt4_e4m3(clamp_e4m3(bf16_lo(v.z) * inv), clamp_e4m3(bf16_hi(v.z) * inv),
                    clamp_e4m3(bf16_lo(v.w) * inv), clamp_e4m3(bf16_hi(v.w) * inv));
    return r;
}

__device__ __forceinline__ uint32_t absmax_u4(uint32_t m, uint4 v) {
    m = absmax_pair(m, v.x);
    m = absmax_pair(m, v.y);
    m = absmax_pair(m, v.z);
    m = absmax_pair(m, v.w);
    return m;
}

// FP32 -> BF16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace fp8bs
