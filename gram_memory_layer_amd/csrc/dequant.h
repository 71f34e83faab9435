// fp8 e4m3fn value times an e8m0 power-of-two scale, rounded to bf16
// ("Module engram" docs, stage 2 and regen_table: each value is widened to
// fp32, multiplied by the scale of its 32-wide block, and the product is
// rounded to bf16).
//
// The e4m3 code is decoded by bit manipulation (exact in fp32: 1 sign,
// 4 exponent bits with bias 7, 3 fraction bits, exponent field 0 subnormal,
// S.1111.111 NaN); the scale code c becomes the fp32 2^(c-127) (c = 0 is the
// fp32 subnormal 2^-127, c = 255 is NaN).  Their product is one IEEE fp32
// multiply -- exact except where it leaves the fp32 range -- and the result is
// rounded to bf16 nearest-even.  Built with fp32 denormals preserved.
#pragma once

#include "internal.h"

namespace engram {

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 0xFu;
    const uint32_t m = c & 7u;
    float v;
    if (e == 0) {
        v = (float)m * 0x1p-9f;                       // subnormal: m/8 * 2^-6
    } else {
        v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    }
    v = __uint_as_float(__float_as_uint(v) | sign);
    if (e == 0xFu && m == 7u) v = __uint_as_float(0x7FC00000u);
    return v;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
    if (c == 0xFFu) return __uint_as_float(0x7FC00000u);
    if (c == 0u) return __uint_as_float(0x00400000u);  // 2^-127
    return __uint_as_float(c << 23);
}

// 8 consecutive e4m3 codes (little-endian in lo, hi) with one scale -> 8 bf16
// packed two per uint32.
__device__ __forceinline__ void dequant8(uint32_t lo, uint32_t hi, float scale, uint32_t out[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t word = (i < 2) ? lo : hi;
        const uint32_t c0 = (word >> (16 * (i & 1))) & 0xFFu;
        const uint32_t c1 = (word >> (16 * (i & 1) + 8)) & 0xFFu;
        const uint32_t b0 = f32_to_bf16(e4m3_to_f32(c0) * scale);
        const uint32_t b1 = f32_to_bf16(e4m3_to_f32(c1) * scale);
        out[i] = b0 | (b1 << 16);
    }
}

}  // namespace engram
