// pkv_tier.hip -- block moves between the GPU block pool and the pinned host
// tier ("LLM+Agent 全栈推理底座" 4.2, TieredBlockManager: blocks past a
// sequence's GPU window go to pinned CPU memory and are copied back when the
// sequence is needed again).
//
// One launch moves a whole batch of blocks: workgroup i copies block
// pairs[i].src of the source tier to block pairs[i].dst of the destination
// tier, K and V.  A block is one contiguous [Hkv][bs][D] piece of either pool,
// so each thread streams 16-byte pieces: all of its loads (K and V) are issued
// before its stores, which keeps many host-link transactions in flight per
// workgroup.  The same kernel serves both directions: the host tier is
// addressed through its device-mapped pointer (the GPU's loads or stores
// cross the host link).  For an 8-bit pool the block's per-kv-head K and V
// scales move with its codes.  The copy is bit-exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_tier.h"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;     // 16-byte pieces per thread per pass, for K and for V each

__global__ void __launch_bounds__(kCopyThreads) kv_tier_copy_kernel(TierCopyArgs a) {
    __shared__ int32_t s_pair[2];
    if (threadIdx.x < 2) s_pair[threadIdx.x] = a.pairs[2 * (int64_t)blockIdx.x + threadIdx.x];
    __syncthreads();
    if ((int)threadIdx.x < a.scales_per_block) {
        const int64_t so = (int64_t)s_pair[0] * a.scales_per_block + threadIdx.x;
        const int64_t dof = (int64_t)s_pair[1] * a.scales_per_block + threadIdx.x;
        a.ks_dst[dof] = a.ks_src[so];
        a.vs_dst[dof] = a.vs_src[so];
    }
    const int64_t src = (int64_t)s_pair[0] * a.vec_per_block;
    const int64_t dst = (int64_t)s_pair[1] * a.vec_per_block;
    for (int base = 0; base < a.vec_per_block; base += kCopyThreads * kCopyUnroll) {
        uint4 kx[kCopyUnroll], vx[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int i = base + u * kCopyThreads + (int)threadIdx.x;
            if (i < a.vec_per_block) {
                kx[u] = a.k_src[src + i];
                vx[u] = a.v_src[src + i];
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int i = base + u * kCopyThreads + (int)threadIdx.x;
            if (i < a.vec_per_block) {
                a.k_dst[dst + i] = kx[u];
                a.v_dst[dst + i] = vx[u];
            }
        }
    }
}

hipError_t launch_tier_copy(const TierCopyArgs& a, hipStream_t stream) {
    if (a.n == 0) return hipSuccess;
    if (a.n < 0 || a.vec_per_block <= 0 || a.scales_per_block < 0 || a.scales_per_block > kCopyThreads ||
        (a.scales_per_block > 0 && (!a.ks_src || !a.vs_src || !a.ks_dst || !a.vs_dst)))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_tier_copy_kernel, dim3((unsigned)a.n), dim3(kCopyThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
