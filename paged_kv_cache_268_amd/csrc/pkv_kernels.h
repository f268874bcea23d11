// pkv_kernels.h -- internal interface between the host library and the HIP
// kernels of libpkv.so.  Not installed; the public ABI is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kNumXcds = 8;      // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kOutF32 = 0, kOutF16 = 1, kOutBF16 = 2;

constexpr int kMaxSeqs = 4096;   // sequences per decode call (prefix of tile counts kept in LDS)
constexpr int kTileTokens = 16;  // tokens per tile of the split

// K/V storage and query type of a decode call.
// FP8_BF16Q: OCP E4M3 K/V with scales, bf16 q; FP8_BF16Q_PAIR: the same with two
// adjacent kv heads per wave (even kv head counts).
enum class KvKind { F16, BF16, FP8_BF16Q, FP8_BF16Q_PAIR };

struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;    // [num_blocks][Hkv] scales of 8-bit K (null for 16-bit K/V)
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    void* out;
    float* lse;              // natural log, nullable
    int32_t* ws_hdr;         // [2 + B + 1]: T, C, prefix of padded tiles (x Hkv) over sequences
    float* ws_out;           // [rows][GC][D] normalised segment outputs, GC = q heads of a wave's kv heads
    float* ws_lse;           // [rows][GC], log2 domain; segment k of pair p = (s, head group) in row c + p
    float scale;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t table_stride;
    int32_t fixed_chunk;     // tiles per chunk (partition_size / 16); 0 = balanced split
    int32_t num_waves;       // waves in the grid (multiple of 4)
    int32_t seg_rows;        // rows of ws_out / ws_lse
    int32_t max_context_len;
    int32_t out_dtype;       // kOut*
    int32_t heads_per_wave;  // kv heads a wave takes per tile: 1, or 2 for FP8_BF16Q_PAIR
    int32_t pair_halves;     // fixed partitions of >= 2 tiles: two waves per chunk (split_pair_lds_bytes of LDS)
    // Fused append (paged_decode_append_split_kernel only): the new rows
    // [n_items][Hkv][D] and the tables and lengths the kernel updates.
    const void* k_new;
    const void* v_new;
    int32_t* tables_out;     // = block_tables
    int32_t* lens_out;       // = context_lens
    int32_t n_items;
};

// One appended token of a fused append + decode, 8 bytes: the sequence (low
// 12 bits) and its new length (high 20 bits) in one word, and the block the
// call opened or copied into (-1: none).  The new row's slot is not carried:
// the kernel stores the row into the block of the tile that holds it, which
// it finds as it reads that tile.  Travels in the kernel arguments.
struct FuseItem {
    uint32_t seq_len;
    int32_t new_block;
    __host__ __device__ int seq() const { return (int)(seq_len & 0xFFFu); }
    __host__ __device__ int new_len() const { return (int)(seq_len >> 12); }
};
constexpr int kFuseItems = 320;
constexpr int kFuseMaxLen = (1 << 20) - 1;   // largest new length an item holds
static_assert(kMaxSeqs <= 4096, "a sequence index fits the item's 12 bits");
struct FuseItems {
    FuseItem it[kFuseItems];
};

struct MergeArgs {
    const int32_t* context_lens;
    const int32_t* ws_hdr;
    const float* ws_out;
    const float* ws_lse;
    void* out;
    float* lse;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t fixed_chunk;
    int32_t max_seg;         // upper bound of segments per (sequence, kv head) (launch shape only)
    int32_t seg_rows;        // rows of ws_out / ws_lse
    int32_t max_context_len;
    int32_t out_dtype;
    int32_t heads_per_wave;  // as the split kernel's: a kv head g sits in list group g / heads_per_wave
};


// start / stop: null, or events that take the split dispatch's own start and
// end timestamps (hipExtLaunchKernel; no marker packets join the stream).
// Dynamic LDS a split launch with pair_halves needs (the softmax state exchange).
inline size_t split_pair_lds_bytes(int head_dim) { return (size_t)2 * 2 * (4 * (head_dim / 16) + 2) * 64 * sizeof(float); }

hipError_t launch_split(const DecodeArgs& a, int head_dim, int block_size, int group_pad, KvKind kind,
                        hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// The split kernel with the append of a.n_items new tokens (16-bit K/V, one
// kv head per wave): lengths and tables come from the items for the appended
// sequences, the new rows from k_new / v_new, and the kernel writes the rows,
// lengths and table entries that kv_append would have written.
hipError_t launch_split_append(const DecodeArgs& a, const FuseItems& items, int head_dim, int block_size, int group_pad,
                               KvKind kind, hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Resident waves per CU of the split kernel instance (occupancy query).
hipError_t split_waves_per_cu(int head_dim, int block_size, int group_pad, KvKind kind, int* waves_per_cu);
hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream);

}  // namespace pkv
