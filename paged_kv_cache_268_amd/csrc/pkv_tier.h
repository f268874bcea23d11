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
    int32_t n;
    int32_t vec_per_block;       // 16-byte pieces per block (Hkv * bs * D * 2 / 16)
};

hipError_t launch_tier_copy(const TierCopyArgs& a, hipStream_t stream);

}  // namespace pkv
