// pkv_prefill.h -- internal interface of the chunked-prefill attention kernel.
// Not installed; the public ABI is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// A workgroup of kPrefillWaves waves covers kPrefillRows (chunk query, q head)
// rows of one kv head (32 per wave): kPrefillRows / G consecutive chunk
// queries times the G q heads of the group.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = 32 * kPrefillWaves;
constexpr int kPrefillMaxSeqs = 4096;
constexpr int kPrefillSortSeqs = 128;   // up to this many sequences, longest contexts are scheduled first

// Chunk queries per workgroup for a kv group of G q heads (0 when G is too large).
inline int prefill_query_tile(int group) { return group >= 1 && group <= kPrefillRows ? kPrefillRows / group : 0; }

struct PrefillArgs {
    const void* q;                   // [total_q][Hq][D]
    const void* k_cache;             // [NB][Hkv][bs][D]
    const void* v_cache;
    const int32_t* block_tables;     // row s at block_tables + s * table_stride
    const int32_t* context_lens;     // [B]: tokens in the cache, the chunk included
    const int32_t* cu_q;             // [B + 1]: chunk rows of sequence s are cu_q[s] .. cu_q[s+1]-1
    void* out;                       // [total_q][Hq][D]
    float* lse;                      // [total_q][Hq], natural log, nullable
    float scale;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t table_stride;
    int32_t total_q;
    int32_t max_context_len;
    int32_t out_dtype;               // kOut* of pkv_kernels.h
    int32_t query_tile;              // chunk queries per workgroup: prefill_query_tile(Hq / Hkv)
    int32_t grid_tiles;              // query tiles the grid covers (>= sum over s of ceil(m_s / query_tile))
};

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, bool bf16, hipStream_t stream);

}  // namespace pkv
