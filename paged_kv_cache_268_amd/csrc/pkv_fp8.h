// pkv_fp8.h -- OCP E4M3 encoding on the device, shared by the 8-bit append
// and the block quantiser.  Internal; the public ABI is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kE4M3Max = 448.0f;   // largest finite E4M3 value (S.1111.110)

// fp32 -> E4M3 code: round to nearest, ties to even; magnitudes from 448 on
// (infinity included) saturate to 448; NaN gives the NaN code.
//   normal range (|y| >= 2^-6): keep the top 3 fraction bits of the fp32
//   value, rounding on the 20 dropped bits, and rebias the exponent (127 -> 7);
//   subnormal range: the value is a multiple of 2^-9, so round |y| * 2^9 to an
//   integer (8 rounds up into the smallest normal, which is code 8).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
    uint32_t u = __builtin_bit_cast(uint32_t, y);
    const uint32_t sign = (u >> 24) & 0x80u;
    u &= 0x7FFFFFFFu;
    if (u > 0x7F800000u) return 0x7Fu;                        // NaN
    if (u >= 0x43E00000u) return sign | 0x7Eu;                // |y| >= 448
    if (u < 0x3C800000u) {                                    // |y| < 2^-6
        const float m = __builtin_rintf(__builtin_bit_cast(float, u) * 512.0f);
        return sign | (uint32_t)m;
    }
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    const uint32_t code = (r >> 20) - ((127u - 7u) << 3);
    return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Block quantiser: items[i] = (source block, destination block, used rows).
struct QuantArgs {
    const void* src_k;           // [*][Hkv][bs][D] of 16-bit values
    const void* src_v;
    uint8_t* dst_k;              // [*][Hkv][bs][D] E4M3 codes
    uint8_t* dst_v;
    float* k_scale;              // [*][Hkv]
    float* v_scale;
    const int32_t* items;        // device [n][3]
    int32_t n;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t head_dim;
    int32_t src_bf16;
};

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream);

}  // namespace pkv
