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
//
// a = max(amax, 2^-100) is a BF16 value: a = m * 2^(E-127) with m = 1 + k/128,
// k = the 7 mantissa bits, E the biased exponent (the floor 2^-100 is k = 0,
// E = 27, and lifts BF16 subnormals to it).  Scaling by a power of two commutes
// with rounding while results stay normal, which they do here (2^-109 < a/448
// and 448/a < 2^109), so
//     fl32(448 / a) = fl32(448 / m) * 2^(127-E),   fl32(a / 448) = fl32(m / 448) * 2^(E-127),
// and both divisions reduce to a lookup in 128-entry tables of correctly
// rounded quotients (computed by the compiler) plus an exact ldexp.
struct TileScale {
    float s;
    float inv;
};

struct ScaleTables {
    float inv[128];    // fl32(448 / m_k)
    float s[128];      // fl32(m_k / 448)
};

constexpr ScaleTables make_scale_tables() {
    ScaleTables t{};
    for (int k = 0; k < 128; ++k) {
        const float m = 1.0f + static_cast<float>(k) / 128.0f;     // exact
        t.inv[k] = kE4M3Max / m;
        t.s[k] = m / kE4M3Max;
    }
    return t;
}

__device__ const ScaleTables g_scale_tables = make_scale_tables();

constexpr uint32_t kFloorBits = 27u << 7;     // 2^-100 as a BF16 magnitude

// Copy the tables into LDS (call with every thread, then synchronize).
__device__ __forceinline__ void load_scale_tables(ScaleTables* dst) {
    const int t = threadIdx.x;
    if (t < 128) {
        dst->inv[t] = g_scale_tables.inv[t];
        dst->s[t] = g_scale_tables.s[t];
    }
}

__device__ __forceinline__ TileScale tile_scale(uint32_t amax_bits, const ScaleTables* tab) {
    const uint32_t b = max(amax_bits, kFloorBits);
    const int k = (int)(b & 0x7Fu);
    const int e = (int)(b >> 7) - 127;
    TileScale t;
    t.s = __builtin_ldexpf(tab->s[k], e);
    t.inv = __builtin_ldexpf(tab->inv[k], -e);
    return t;
}

__device__ __forceinline__ float clamp_e4m3(float p) {
    return __builtin_amdgcn_fmed3f(p, -kE4M3Max, kE4M3Max);
}

// Four FP32 values -> four E4M3 codes, byte i = value i.  v_cvt_pk_fp8_f32
// rounds to nearest even, keeps the sign of zero, returns 0x7E/0xFE for
// magnitudes up to 464 and NaN above.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// Eight BF16 values (a uint4) times inv -> eight codes (a uint2).  No clamp to
// +-448 is needed: |x| <= a gives |fl32(x * fl32(448/a))| <= 448 (1 + 2^-23) <
// 464, which the conversion maps to +-448 exactly as clamping first would.
__device__ __forceinline__ uint2 quant8(uint4 v, float inv) {
    uint2 r;
    r.x = cvt4_e4m3(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
    r.y = cvt4_e4m3(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
    return r;
}

__device__ __forceinline__ uint32_t absmax_u4(uint32_t m, uint4 v) {
    m = absmax_pair(m, v.x);
    m = absmax_pair(m, v.y);
    m = absmax_pair(m, v.z);
    m = absmax_pair(m, v.w);
    return m;
}

// Two FP32 values -> two BF16 (low half = a), round to nearest, ties to even:
// one v_cvt_pk_bf16_f32 (the conversion honours the default rounding mode).
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{a, b}, v2bf_t));
}

}  // namespace fp8bs
