// Device encoders shared by the kernels that write new K/V rows into the
// pool: the cache-write kernels and the decode kernels' fused write.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// 16-bit source element -> float32 (exact).
template <int SRC>
__device__ __forceinline__ float widen(uint32_t bits16) {
    if constexpr (SRC == PA_BF16) {
        return __uint_as_float(bits16 << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    }
}

// float32 -> OCP e4m3 code: round to nearest, ties to even; magnitudes at or
// beyond 448 saturate to 448; NaN keeps its sign and becomes 0x7F / 0xFF.
__device__ __forceinline__ uint32_t e4m3_from_float(float y) {
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a != a) return sign | 0x7Fu;
    if (!(a < 448.0f)) return sign | 0x7Eu;
    if (a < 0.015625f) {
        // Subnormal range: multiples of 2^-9.  a * 512 is exact and < 8;
        // rintf rounds half to even.  8 (= 2^-6) becomes the smallest normal.
        return sign | (uint32_t)rintf(a * 512.0f);
    }
    // Normal range [2^-6, 448): keep 3 of the 23 mantissa bits, rounding the
    // dropped 20 bits to nearest even; a carry bumps the exponent correctly.
    uint32_t ab = __float_as_uint(a);
    ab += 0x7FFFFu + ((ab >> 20) & 1u);
    const uint32_t e = (ab >> 23) - 127u + 7u;   // 1 .. 15
    const uint32_t m = (ab >> 20) & 7u;
    return sign | (e << 3) | m;
}

// 16 bytes of a pool row holding the new token: `src` points at the source
// elements (16-bit, SRC) that land in them -- 8 for a 16-bit pool (a bit
// copy), 16 for an fp8 pool (each divided by `scale` in IEEE fp32 and
// encoded as e4m3).
template <int SRC, int KVT>
__device__ __forceinline__ uint4 encode_chunk16(const uint16_t* src, float scale) {
    if constexpr (KVT != PA_FP8_E4M3) {
        return *reinterpret_cast<const uint4*>(src);
    } else {
        const uint4 lo = *reinterpret_cast<const uint4*>(src);
        const uint4 hi = *reinterpret_cast<const uint4*>(src + 8);
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t h = (w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            packed[e >> 2] |= e4m3_from_float(__fdiv_rn(widen<SRC>(h), scale)) << ((e & 3) * 8);
        }
        return make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
}

}  // namespace pa
