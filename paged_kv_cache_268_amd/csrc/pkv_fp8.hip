// pkv_fp8.hip -- 16-bit K/V blocks -> OCP E4M3 blocks with one fp32 scale per
// (block, kv head), for the 8-bit cache (reduced-precision storage of cached
// K/V, "LLM+Agent 全栈推理底座" 5.2).
//
// One 256-thread workgroup per (item, kv head) handles K and then V: the
// largest magnitude over the block's first `used` rows, scale = amax / 448
// (1 when every value is 0), each value divided by the scale in fp32 and
// rounded to the nearest code; rows from `used` on are written as code 0.
// Threads own 8 consecutive values (one 16-byte load, one 8-byte store).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_fp8.h"

namespace pkv {

constexpr int kQThreads = 256;

__device__ __forceinline__ float widen16(uint32_t h, bool bf16) {
    if (bf16) return __builtin_bit_cast(float, h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ void quantize_tile(const uint16_t* src, uint8_t* dst, float* scale_out, int used_vec,
                                              int nvec, bool bf16, float* s_red) {
    float amax = 0.f;
    for (int i = threadIdx.x; i < used_vec; i += kQThreads) {
        const uint4 w = reinterpret_cast<const uint4*>(src)[i];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax = fmaxf(amax, fabsf(widen16(ws[e] & 0xFFFFu, bf16)));
            amax = fmaxf(amax, fabsf(widen16(ws[e] >> 16, bf16)));
        }
    }
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
    __syncthreads();
    float m = s_red[0];
#pragma unroll
    for (int w = 1; w < kQThreads / 64; ++w) m = fmaxf(m, s_red[w]);
    const float scale = m > 0.f ? m / kE4M3Max : 1.f;
    if (threadIdx.x == 0) *scale_out = scale;
    for (int i = threadIdx.x; i < nvec; i += kQThreads) {
        uint2 o = make_uint2(0, 0);
        if (i < used_vec) {
            const uint4 w = reinterpret_cast<const uint4*>(src)[i];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
            uint32_t b[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                b[2 * e] = f32_to_e4m3(widen16(ws[e] & 0xFFFFu, bf16) / scale);
                b[2 * e + 1] = f32_to_e4m3(widen16(ws[e] >> 16, bf16) / scale);
            }
            o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
            o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        }
        reinterpret_cast<uint2*>(dst)[i] = o;
    }
    __syncthreads();     // s_red is reused by the next tile
}

__global__ void __launch_bounds__(kQThreads) kv_quantize_fp8_kernel(QuantArgs a) {
    __shared__ float s_red[kQThreads / 64];
    const int Hkv = a.num_kv_heads, bs = a.block_size, D = a.head_dim;
    const int item = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
    const int32_t sb = a.items[3 * (int64_t)item], db = a.items[3 * (int64_t)item + 1];
    const int used = min(max(a.items[3 * (int64_t)item + 2], 0), bs);
    const int64_t tile = ((int64_t)sb * Hkv + g) * bs * D;
    const int64_t dtile = ((int64_t)db * Hkv + g) * bs * D;
    const int nvec = bs * D / 8, used_vec = used * D / 8;
    const bool bf16 = a.src_bf16 != 0;
    quantize_tile(reinterpret_cast<const uint16_t*>(a.src_k) + tile, a.dst_k + dtile, a.k_scale + (int64_t)db * Hkv + g,
                  used_vec, nvec, bf16, s_red);
    quantize_tile(reinterpret_cast<const uint16_t*>(a.src_v) + tile, a.dst_v + dtile, a.v_scale + (int64_t)db * Hkv + g,
                  used_vec, nvec, bf16, s_red);
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream) {
    if (a.n == 0) return hipSuccess;
    const int64_t grid = (int64_t)a.n * a.num_kv_heads;
    if (a.n < 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_quantize_fp8_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
