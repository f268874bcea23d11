// pkv_tier.h -- internal interface of the block-move kernel between the GPU
// block pool and the pinned host tier.  Not installed; the public ABI is
// include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Block moves between the GPU pool and the host tier (either direction).
struct TierCopyArgs {
    const uint4* k_src;          // base of the source tier's K blocks ([blocks][Hkv][bs][D])
    const uint4* v_src;
    uint4* k_dst;                // base of the destination tier's K blocks
    uint4* v_dst;
    const int32_t* pairs;        // device-readable (pinned host) [n][2]: source block, destination block
    // 8-bit pools: the K and V scales of each block ([blocks][Hkv] fp32 in both tiers) move with
    // its codes; null for 16-bit pools.
    const float* ks_src;
    const float* vs_src;
    float* ks_dst;
    float* vs_dst;
    int32_t n;
    int32_t vec_per_block;       // 16-byte pieces per block (Hkv * bs * D * element bytes / 16)
    int32_t scales_per_block;    // Hkv when the scales move, else 0
};

hipError_t launch_tier_copy(const TierCopyArgs& a, hipStream_t stream);

}  // namespace pkv
