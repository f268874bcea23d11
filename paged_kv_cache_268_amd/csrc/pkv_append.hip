// pkv_append.hip -- write one new token's K/V per sequence into its slot.
//
// The host has already reserved the slots (free-list pops, copy-on-write
// decisions); each work item is (seq, slot, table_pos, new_block, cow_src,
// cow_ntok, new_len).  Up to 160 items travel in the kernel arguments;
// larger batches, and the copy-on-write phase, read them from pinned host
// memory.  One 256-thread workgroup per item:
//   1. copy-on-write: rows [0, cow_ntok) of (cow_src, g) -> (new_block, g) for
//      every kv head g, K and V;
//   2. the new rows k_new[i][g][:] / v_new[i][g][:] -> the slot's row of every
//      kv head g;
//   3. block_tables[seq][table_pos] = new_block if one was taken,
//      context_lens[seq] = new_len.
// Rows are moved with 16-byte loads and stores; the copy is bit-exact.
// The slot of token t is table[t / block_size] * block_size + t % block_size
// ("架构解构：推理引擎的四层抽象", PagedAttention section: logical->physical block
// table; "LLM+Agent 全栈推理底座" 4.2: blocks taken from a free list on demand).
//
// 8-bit (E4M3) pools: the new bf16 rows are divided by their block's scale
// and rounded to the nearest code; a row that starts a new block (slot at
// offset 0 of a block this call took) uses, and records as that block's
// scales, the pool's default scales of its kv head; copy-on-write also copies
// the source block's scales.
//
// Step 1 runs as its own launch before steps 2-3 whenever some item copies:
// a block one item copies from may be the tail that another item of the same
// call writes into (its last other holder), so every copy must finish first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_append.h"
#include "pkv_fp8.h"

namespace pkv {

// Copy-on-write phase: rows [0, cow_ntok) of every kv head, (cow_src, g) ->
// (new_block, g), K and V, for the items that need it.
__global__ void __launch_bounds__(256) kv_append_cow_kernel(AppendArgs a) {
    __shared__ AppendItem s_it;
    if (threadIdx.x == 0) s_it = a.items[blockIdx.x];
    __syncthreads();
    const AppendItem it = s_it;
    if (it.cow_src < 0) return;
    const int bs = a.block_size, Hkv = a.num_kv_heads;
    const int vec_per_row = a.kv8 ? a.head_dim / 16 : a.head_dim / 8;   // uint4 per row
    uint4* kc = reinterpret_cast<uint4*>(a.k_cache);
    uint4* vc = reinterpret_cast<uint4*>(a.v_cache);
    if (a.kv8 && (int)threadIdx.x < Hkv) {
        a.k_scale[(int64_t)it.new_block * Hkv + threadIdx.x] = a.k_scale[(int64_t)it.cow_src * Hkv + threadIdx.x];
        a.v_scale[(int64_t)it.new_block * Hkv + threadIdx.x] = a.v_scale[(int64_t)it.cow_src * Hkv + threadIdx.x];
    }
    const int per_head = it.cow_ntok * vec_per_row;
    for (int x = threadIdx.x; x < Hkv * per_head; x += blockDim.x) {
        const int g = x / per_head, r = x % per_head;
        const int64_t src = ((int64_t)it.cow_src * Hkv + g) * bs * vec_per_row + r;
        const int64_t dst = ((int64_t)it.new_block * Hkv + g) * bs * vec_per_row + r;
        kc[dst] = kc[src];
        vc[dst] = vc[src];
    }
}

// Write phase: one 256-thread workgroup per item moves 16-byte pieces of the
// new K/V row of every kv head into the slot, then updates the tables.
// 8-bit pool: 8 bf16 values of the new row per thread -> 8 codes.  use_init:
// the block was opened in this call, so its scales are the defaults (another
// workgroup of the same call may not have recorded them yet); record: this
// row opens the block and records them.
__device__ __forceinline__ void append_row_fp8(const AppendArgs& a, int i, int blk, int off, bool use_init,
                                               bool record) {
    const int bs = a.block_size, Hkv = a.num_kv_heads, per_row = a.head_dim / 8;
    const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
    const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
    uint2* kc = reinterpret_cast<uint2*>(a.k_cache);
    uint2* vc = reinterpret_cast<uint2*>(a.v_cache);
    for (int x = threadIdx.x; x < Hkv * per_row; x += blockDim.x) {
        const int g = x / per_row, r = x % per_row;
        const int64_t bg = (int64_t)blk * Hkv + g;
        const float ks = use_init ? a.k_init[g] : a.k_scale[bg];
        const float vs = use_init ? a.v_init[g] : a.v_scale[bg];
        const int64_t src = ((int64_t)i * Hkv + g) * per_row + r;
        const int64_t row = (bg * bs + off) * per_row + r;
        const uint4 w[2] = {kn[src], vn[src]};
        const float sc[2] = {ks, vs};
        uint2 o[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t ws[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
            uint32_t b[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                b[2 * e] = f32_to_e4m3(__builtin_bit_cast(float, ws[e] << 16) / sc[t]);
                b[2 * e + 1] = f32_to_e4m3(__builtin_bit_cast(float, ws[e] & 0xFFFF0000u) / sc[t]);
            }
            o[t] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
        }
        kc[row] = o[0];
        vc[row] = o[1];
    }
    if (record && (int)threadIdx.x < Hkv) {
        a.k_scale[(int64_t)blk * Hkv + threadIdx.x] = a.k_init[threadIdx.x];
        a.v_scale[(int64_t)blk * Hkv + threadIdx.x] = a.v_init[threadIdx.x];
    }
}

// 16-bit pool: the new row of every kv head, 16-byte pieces, bit-exact.
__device__ __forceinline__ void append_row16(const AppendArgs& a, int i, int blk, int off) {
    const int bs = a.block_size, Hkv = a.num_kv_heads, vec_per_row = a.head_dim / 8;
    uint4* kc = reinterpret_cast<uint4*>(a.k_cache);
    uint4* vc = reinterpret_cast<uint4*>(a.v_cache);
    const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
    const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
    for (int x = threadIdx.x; x < Hkv * vec_per_row; x += blockDim.x) {
        const int g = x / vec_per_row, r = x % vec_per_row;
        const int64_t row = (((int64_t)blk * Hkv + g) * bs + off) * vec_per_row + r;
        const int64_t src = ((int64_t)i * Hkv + g) * vec_per_row + r;
        kc[row] = kn[src];
        vc[row] = vn[src];
    }
}

__device__ __forceinline__ void append_item(const AppendArgs& a, int i, int seq, int slot, int new_block,
                                            int new_len) {
    const int bs = a.block_size;
    if (a.kv8) {
        const bool fresh = new_block >= 0 && slot % bs == 0;
        append_row_fp8(a, i, slot / bs, slot % bs, fresh, fresh);
    } else {
        append_row16(a, i, slot / bs, slot % bs);
    }
    if (threadIdx.x == 0) {
        if (new_block >= 0) a.block_tables[(int64_t)seq * a.table_stride + (new_len - 1) / bs] = new_block;
        a.context_lens[seq] = new_len;
    }
}

__global__ void __launch_bounds__(256) kv_append_kernel_args(AppendArgs a, ArgItems items) {
    const ArgItem it = items.it[blockIdx.x];
    append_item(a, blockIdx.x, it.seq, it.slot, it.new_block, it.new_len);
}

__global__ void __launch_bounds__(256) kv_append_kernel_host(AppendArgs a) {
    __shared__ AppendItem s_it;
    if (threadIdx.x == 0) s_it = a.items[blockIdx.x];   // host memory: read once
    __syncthreads();
    append_item(a, blockIdx.x, s_it.seq, s_it.slot, s_it.new_block, s_it.new_len);
}

// Multi-token append: one workgroup per token (row i of k_new / v_new).  Only
// a sequence's last token of the call writes its length; a token that opened
// or copied a block publishes the table entry.
__global__ void __launch_bounds__(256) kv_append_tokens_kernel(AppendArgs a, const TokenItem* tokens) {
    __shared__ TokenItem s_t;
    if (threadIdx.x == 0) s_t = tokens[blockIdx.x];     // host memory: read once
    __syncthreads();
    const TokenItem t = s_t;
    const int bs = a.block_size, blk = t.slot / bs, off = t.slot % bs;
    if (a.kv8) {
        const bool fresh = (t.flags & kTokFresh) != 0;
        append_row_fp8(a, blockIdx.x, blk, off, fresh, fresh && off == 0);
    } else {
        append_row16(a, blockIdx.x, blk, off);
    }
    if (threadIdx.x == 0) {
        if (t.flags & kTokTable) a.block_tables[(int64_t)t.seq * a.table_stride + t.tpos] = blk;
        if (t.flags & kTokLast) a.context_lens[t.seq] = t.tpos * bs + off + 1;
    }
}

hipError_t launch_append_tokens(const AppendArgs& a, int32_t n_tokens, const TokenItem* tokens, bool any_copy,
                                hipStream_t stream) {
    if (any_copy && a.n > 0) {
        hipLaunchKernelGGL(kv_append_cow_kernel, dim3((unsigned)a.n), dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (n_tokens > 0) hipLaunchKernelGGL(kv_append_tokens_kernel, dim3((unsigned)n_tokens), dim3(256), 0, stream, a, tokens);
    return hipGetLastError();
}

hipError_t launch_append_cow(const AppendArgs& a, hipStream_t stream) {
    if (a.n == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_append_cow_kernel, dim3((unsigned)a.n), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, bool any_copy, const ArgItems* inl, hipStream_t stream) {
    if (a.n == 0) return hipSuccess;
    const dim3 grid((unsigned)a.n);
    if (any_copy) {
        hipLaunchKernelGGL(kv_append_cow_kernel, grid, dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (inl && a.n <= kArgItems)
        hipLaunchKernelGGL(kv_append_kernel_args, grid, dim3(256), 0, stream, a, *inl);
    else
        hipLaunchKernelGGL(kv_append_kernel_host, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
