// pkv_fp8.hip -- 16-bit K/V blocks -> OCP E4M3 blocks with one fp32 scale per
// (block, kv head), for the 8-bit cache (reduced-precision storage of cached
// K/V, "从零开始构建LLM推理引擎：模型执行器深度解析" 5.2, KV缓存管理技巧).
//
// One wave per (item, kv head), four per workgroup: the largest magnitude over
// the block's first `used` rows of K and of V, scale = amax / 448 (1 when every
// value is 0), each value divided by its scale in fp32 and rounded to the
// nearest code; rows from `used` on are written as code 0 (and never read).
// Lane l owns 16-byte vectors l, l + 64, ... of the (block, kv head) tile of
// K and of V (8 values each, VPL per lane): every load is issued before any
// arithmetic, both maxima are wave reductions (no LDS, no barrier), and the
// codes are encoded from registers into 8-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_fp8.h"

namespace pkv {

constexpr int kQWaves = 4;
constexpr int kQThreads = kQWaves * 64;

__device__ __forceinline__ float widen16(uint32_t h, bool bf16) {
    if (bf16) return __builtin_bit_cast(float, h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float vec_amax(uint4 w, bool bf16, float amax) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(widen16(ws[e] & 0xFFFFu, bf16)));
        amax = fmaxf(amax, fabsf(widen16(ws[e] >> 16, bf16)));
    }
    return amax;
}

__device__ __forceinline__ uint2 vec_encode(uint4 w, bool bf16, float scale) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        b[2 * e] = f32_to_e4m3(widen16(ws[e] & 0xFFFFu, bf16) / scale);
        b[2 * e + 1] = f32_to_e4m3(widen16(ws[e] >> 16, bf16) / scale);
    }
    return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

__device__ __forceinline__ float wave_max(float x) {
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// VPL = (block_size * head_dim / 8) / 64 vectors per lane per tile.
template <int VPL>
__global__ void __launch_bounds__(kQThreads) kv_quantize_fp8_kernel(QuantArgs a) {
    const int lane = threadIdx.x & 63;
    const int Hkv = a.num_kv_heads, bs = a.block_size, D = a.head_dim;
    const int64_t pair = (int64_t)blockIdx.x * kQWaves + (threadIdx.x >> 6);
    if (pair >= (int64_t)a.n * Hkv) return;
    const int64_t item = pair / Hkv;
    const int g = (int)(pair % Hkv);
    const int32_t sb = a.items[3 * item], db = a.items[3 * item + 1];
    const int used = min(max(a.items[3 * item + 2], 0), bs);
    const int used_vec = used * (D / 8);
    const int64_t tile = ((int64_t)sb * Hkv + g) * bs * D / 8;      // in 16-byte vectors
    const int64_t dtile = ((int64_t)db * Hkv + g) * bs * D / 8;     // in 8-byte code words
    const uint4* sk = reinterpret_cast<const uint4*>(a.src_k) + tile;
    const uint4* sv = reinterpret_cast<const uint4*>(a.src_v) + tile;
    const bool bf16 = a.src_bf16 != 0;

    uint4 vk[VPL], vv[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int i = lane + 64 * j;
        vk[j] = i < used_vec ? sk[i] : make_uint4(0, 0, 0, 0);
        vv[j] = i < used_vec ? sv[i] : make_uint4(0, 0, 0, 0);
    }
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        ak = vec_amax(vk[j], bf16, ak);
        av = vec_amax(vv[j], bf16, av);
    }
    ak = wave_max(ak);
    av = wave_max(av);
    const float sck = ak > 0.f ? ak / kE4M3Max : 1.f;
    const float scv = av > 0.f ? av / kE4M3Max : 1.f;
    if (lane == 0) {
        a.k_scale[(int64_t)db * Hkv + g] = sck;
        a.v_scale[(int64_t)db * Hkv + g] = scv;
    }
    uint2* dk = reinterpret_cast<uint2*>(a.dst_k) + dtile;
    uint2* dv = reinterpret_cast<uint2*>(a.dst_v) + dtile;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int i = lane + 64 * j;
        dk[i] = i < used_vec ? vec_encode(vk[j], bf16, sck) : make_uint2(0, 0);
        dv[i] = i < used_vec ? vec_encode(vv[j], bf16, scv) : make_uint2(0, 0);
    }
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream) {
    if (a.n == 0) return hipSuccess;
    if (a.n < 0) return hipErrorInvalidValue;
    const int64_t pairs = (int64_t)a.n * a.num_kv_heads;
    const int64_t grid = (pairs + kQWaves - 1) / kQWaves;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t vecs = (int64_t)a.block_size * a.head_dim / 8;   // per (block, kv head) tile
    switch (vecs) {
        case 128: hipLaunchKernelGGL(kv_quantize_fp8_kernel<2>, dim3((unsigned)grid), dim3(kQThreads), 0, stream, a); break;
        case 256: hipLaunchKernelGGL(kv_quantize_fp8_kernel<4>, dim3((unsigned)grid), dim3(kQThreads), 0, stream, a); break;
        case 512: hipLaunchKernelGGL(kv_quantize_fp8_kernel<8>, dim3((unsigned)grid), dim3(kQThreads), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
