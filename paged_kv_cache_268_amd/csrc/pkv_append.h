// pkv_append.h -- internal interface of the K/V append kernels.  Not
// installed; the public ABI is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// One append item, as staged by the host (7 int32).
struct AppendItem {
    int32_t seq, slot, tpos, new_block, cow_src, cow_ntok, new_len;
};

// Items small enough to travel in the kernel arguments (no host-memory read
// on the device): 16 bytes each, up to kArgItems of them.
struct ArgItem {
    int32_t seq, slot, new_block, new_len;     // table_pos = (new_len - 1) / block_size
};
constexpr int kArgItems = 160;
struct ArgItems {
    ArgItem it[kArgItems];
};

struct AppendArgs {
    const AppendItem* items;     // device-readable (pinned host) [n]
    const void* k_new;           // [n][Hkv][D]
    const void* v_new;
    void* k_cache;               // [NB][Hkv][bs][D]
    void* v_cache;
    int32_t* block_tables;       // [max_seqs][table_stride]
    int32_t* context_lens;       // [max_seqs]
    int32_t n;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t table_stride;
    // 8-bit (E4M3) pools: new rows (bf16) are quantised with their block's
    // scale; a block started by this call takes the default scales.
    int32_t kv8;
    float* k_scale;              // [num_blocks][Hkv]
    float* v_scale;
    const float* k_init;         // [Hkv] default scales of new blocks
    const float* v_init;
};

// One token of a multi-token append (kv_append_tokens).
struct TokenItem {
    int32_t seq, slot, tpos, flags;
};
constexpr int32_t kTokLast = 1;        // last token of its sequence in this call: write the length
constexpr int32_t kTokFresh = 2;       // its block was opened (not copied) in this call: default 8-bit scales
constexpr int32_t kTokTable = 4;       // publish block_tables[seq][tpos] = slot / block_size

// items_in_args: a.n <= kArgItems and `inl` holds the items (copy-on-write
// still reads a.items, in the separate copy launch).
hipError_t launch_append(const AppendArgs& a, bool any_copy, const ArgItems* inl, hipStream_t stream);
// Only the copy-on-write phase of an append (items in a.items): the fused
// append + decode writes the rows itself.
hipError_t launch_append_cow(const AppendArgs& a, hipStream_t stream);
// Multi-token append: copy-on-write of a.n items of a.items (those with
// cow_src >= 0) first, then one workgroup per token of `tokens`.
hipError_t launch_append_tokens(const AppendArgs& a, int32_t n_tokens, const TokenItem* tokens, bool any_copy,
                                hipStream_t stream);

}  // namespace pkv
