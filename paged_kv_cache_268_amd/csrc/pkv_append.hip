// pkv_append.hip -- write one new token's K/V per sequence into its slot.
//
// The host has already reserved the slots (free-list pops, copy-on-write
// decisions); each work item arrives as (seq, slot, table_pos, new_block,
// cow_src, cow_ntok, new_len).  One 64-thread workgroup per (item, kv head):
//   1. copy-on-write: rows [0, cow_ntok) of (cow_src, g) -> (new_block, g), K and V;
//   2. the new row k_new[i][g][:] / v_new[i][g][:] -> slot's row of kv head g;
//   3. (kv head 0 only) block_tables[seq][table_pos] = new_block if one was
//      taken, context_lens[seq] = new_len.
// Rows are moved with 16-byte loads and stores; the copy is bit-exact.
// The slot of token t is table[t / block_size] * block_size + t % block_size
// ("架构解构：推理引擎的四层抽象", PagedAttention section: logical->physical block
// table; "LLM+Agent 全栈推理底座" 4.2: blocks taken from a free list on demand).
//
// Step 1 runs as its own launch before steps 2-3 whenever some item copies:
// a block one item copies from may be the tail that another item of the same
// call writes into (its last other holder), so every copy must finish first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"

namespace pkv {

template <bool COPY_PHASE>
__global__ void __launch_bounds__(64) kv_append_kernel(AppendArgs a) {
    const int i = blockIdx.x / a.num_kv_heads;
    const int g = blockIdx.x % a.num_kv_heads;
    const AppendItem it = a.items[i];
    const int D = a.head_dim, bs = a.block_size, Hkv = a.num_kv_heads;
    const int vec_per_row = D / 8;                 // uint4 per row
    uint4* kc = reinterpret_cast<uint4*>(a.k_cache);
    uint4* vc = reinterpret_cast<uint4*>(a.v_cache);

    if constexpr (COPY_PHASE) {
        if (it.cow_src >= 0) {
            const int64_t src = ((int64_t)it.cow_src * Hkv + g) * bs * vec_per_row;
            const int64_t dst = ((int64_t)it.new_block * Hkv + g) * bs * vec_per_row;
            for (int x = threadIdx.x; x < it.cow_ntok * vec_per_row; x += 64) {
                kc[dst + x] = kc[src + x];
                vc[dst + x] = vc[src + x];
            }
        }
        return;
    }
    const int blk = it.slot / bs, off = it.slot % bs;
    const int64_t row = (((int64_t)blk * Hkv + g) * bs + off) * vec_per_row;
    const int64_t srow = ((int64_t)i * Hkv + g) * vec_per_row;
    const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
    const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
    for (int x = threadIdx.x; x < vec_per_row; x += 64) {
        kc[row + x] = kn[srow + x];
        vc[row + x] = vn[srow + x];
    }
    if (g == 0 && threadIdx.x == 0) {
        if (it.new_block >= 0) a.block_tables[(int64_t)it.seq * a.table_stride + it.tpos] = it.new_block;
        a.context_lens[it.seq] = it.new_len;
    }
}

hipError_t launch_append(const AppendArgs& a, bool any_copy, hipStream_t stream) {
    if (a.n == 0) return hipSuccess;
    const dim3 grid((unsigned)(a.n * a.num_kv_heads));
    if (any_copy) {
        hipLaunchKernelGGL(kv_append_kernel<true>, grid, dim3(64), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kv_append_kernel<false>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
