/*
 * pkv.h -- C ABI of libpkv.so: paged-KV attention decode on AMD Instinct
 * MI355X (gfx950).
 *
 * The setting (sources are the three web pages this library follows):
 *   - KV cache split into fixed-size blocks, allocated on demand
 *     ("LLM+Agent 全栈推理底座：Triton 算子优化・语义级缓存・分布式调度", 2.1 paged KV
 *     cache; 4.2 BlockManager: ceil(n / block_size) blocks, popped from a free list);
 *   - a per-sequence logical->physical block table kept by the host runtime and
 *     dereferenced inside the attention kernel, blocks not contiguous in memory
 *     ("架构解构：推理引擎的四层抽象", PagedAttention section, and the runtime
 *     layer's KV-cache lifecycle with metadata updates between kernel launches);
 *   - scaled dot-product attention with scale 1/sqrt(d) and a stable softmax
 *     ("从零开始构建LLM推理引擎：模型执行器深度解析", 3.1);
 *   - fp32 accumulation of 16-bit inputs ("LLM+Agent 全栈推理底座", 4.1);
 *   - tiled attention with an online softmax that never writes scores to HBM,
 *     modified to address the paged layout indirectly
 *     ("架构解构：推理引擎的四层抽象", FlashAttention integration section).
 *
 * Conventions for every call:
 *   - Device buffers are allocated and owned by the caller; the library only
 *     borrows them for the duration of the work it enqueues.  No call
 *     allocates device memory.  A pool owns host memory only (its metadata
 *     and a small pinned staging ring).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without waiting for it.  Argument checks are
 *     synchronous: on a non-zero status nothing was enqueued and, for pool
 *     calls, the pool is unchanged.
 *   - Status: 0 (PKV_OK) or a negative PKV_E* code; pkv_last_error() returns
 *     a message for the calling thread's most recent failure.  No call throws.
 *   - Device-side contents (table entries, context lengths) are trusted by
 *     the decode kernels; kv_validate_tables() checks them on the host.
 *   - Calls on one pool are not thread-safe; distinct pools are independent.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pkv_stream_t;   /* the same type as hipStream_t */
typedef struct ihipEvent_t* pkv_event_t;     /* the same type as hipEvent_t */

enum {
    PKV_OK = 0,
    PKV_EINVAL = -1,        /* bad argument, unknown sequence, inconsistent sizes */
    PKV_ENOMEM = -2,        /* block pool (or sequence slots) exhausted */
    PKV_EUNSUPPORTED = -3,  /* valid but not built: head_dim, block_size, dtype, group size */
    PKV_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
    PKV_EWORKSPACE = -5     /* workspace missing or smaller than paged_attn_workspace_bytes() */
};

/* PKV_FP8_E4M3: OCP 8-bit float E4M3 (1 sign, 4 exponent bits, bias 7, 3
 * fraction bits, no infinities, S.1111.111 = NaN), one byte per value. */
enum { PKV_F16 = 0, PKV_BF16 = 1, PKV_F32 = 2, PKV_FP8_E4M3 = 3 };

/* Message for the calling thread's last failed call ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------
 * Block pool: host bookkeeping of fixed-size KV blocks
 * ("LLM+Agent 全栈推理底座" 4.2 BlockManager; "架构解构：推理引擎的四层抽象"
 * PagedAttention section: the block table lives in the host runtime).
 *
 * Device layout the pool describes (all C-contiguous, caller-allocated):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim] of kv_dtype
 *   block_tables     : int32 [max_seqs][max_blocks_per_seq]; row = sequence id;
 *                      entries past ceil(len / block_size) are -1
 *   context_lens     : int32 [max_seqs]
 * ------------------------------------------------------------------------ */
typedef struct pkv_pool_desc {
    int32_t num_blocks;          /* physical blocks in k_cache / v_cache (>= 1) */
    int32_t block_size;          /* tokens per block: 16 or 32 */
    int32_t num_kv_heads;        /* >= 1 */
    int32_t head_dim;            /* 64 or 128 */
    int32_t kv_dtype;            /* PKV_F16, PKV_BF16, or PKV_FP8_E4M3 (then set scales, below) */
    int32_t max_seqs;            /* rows of block_tables / context_lens (>= 1) */
    int32_t max_blocks_per_seq;  /* columns of block_tables (>= 1) */
} pkv_pool_desc;

typedef struct pkv_pool pkv_pool;

/* Create a pool over caller-owned k_cache / v_cache.  alloc_order (host,
 * nullable, num_blocks entries) must be a permutation of [0, num_blocks):
 * blocks are handed out as alloc_order[0], alloc_order[1], ... (the free list
 * is alloc_order reversed and allocation pops its last element, as the page's
 * BlockManager does).  NULL means 0, 1, 2, ...  *out receives the handle. */
int kv_block_pool_create(const pkv_pool_desc* desc, void* k_cache, void* v_cache,
                         const int32_t* alloc_order, pkv_pool** out);

/* Release the pool's host memory.  Waits for pending kv_append staging. NULL ok. */
void kv_block_pool_destroy(pkv_pool* pool);

/* New empty sequence (length 0); its id is the lowest free row. PKV_ENOMEM if none. */
int kv_seq_add(pkv_pool* pool, int32_t* seq_id_out);

/* Register a sequence whose `len` tokens already sit in the listed physical
 * blocks (host array of n_blocks ids, n_blocks == ceil(len / block_size), no
 * repeats).  Blocks not yet held are taken off the free list; blocks already
 * held by other sequences become shared (reference count + 1).  Host only: call
 * kv_write_tables() to publish the change to the device tables. */
int kv_seq_import(pkv_pool* pool, int32_t len, const int32_t* block_ids, int32_t n_blocks,
                  int32_t* seq_id_out);

/* New sequence sharing all of src's blocks (prefix reuse); host only. */
int kv_seq_fork(pkv_pool* pool, int32_t src_seq, int32_t* seq_id_out);

/* Drop the sequence: each of its blocks loses one reference, in logical
 * order; blocks left with none return to the free list (the next allocation
 * reuses the last one released).  Host only. */
int kv_seq_free(pkv_pool* pool, int32_t seq_id);

/* Host view of one sequence: its length and up to `cap` block-list entries
 * (a GPU block id b >= 0, or -2 - c for host-tier block c). */
int kv_seq_info(const pkv_pool* pool, int32_t seq_id, int32_t* len_out,
                int32_t* block_ids_out, int32_t cap, int32_t* n_blocks_out);

/* Free blocks, live sequences, reference count of one block (block < 0: skip). */
int kv_pool_stats(const pkv_pool* pool, int32_t* num_free_out, int32_t* num_seqs_out,
                  int32_t block, int32_t* refcount_out);

/* Host-only allocation step of kv_append: for the n listed sequences (host
 * array, no repeats), reserve the slot of each one's next token.  A sequence
 * at t tokens takes a new block when t % block_size == 0; if instead its
 * partly filled tail block is shared, it takes a new block and the t %
 * block_size used slots are to be copied (copy-on-write).  All or nothing:
 * PKV_ENOMEM (pool) or PKV_EINVAL (max_blocks_per_seq reached, unknown or
 * repeated id) leave the pool unchanged.  items_out (host, nullable) receives
 * n rows of 7 int32: seq, slot (= block * block_size + t % block_size),
 * table_pos (= t / block_size), new_block (-1: none), cow_src (-1: none),
 * cow_ntok, new_len. */
int kv_reserve(pkv_pool* pool, int32_t n, const int32_t* seq_ids, int32_t* items_out);

/* Append one token to each of n sequences: kv_reserve, then on `stream`
 * copy-on-write any shared tail block, write k_new[i] / v_new[i] into the
 * reserved slot of every kv head, and update the device block_tables and
 * context_lens rows of those sequences.
 *   seq_ids      : host int32 [n]
 *   k_new, v_new : device [n][num_kv_heads][head_dim] of kv_dtype
 *   block_tables : device int32 [max_seqs][max_blocks_per_seq]
 *   context_lens : device int32 [max_seqs]
 * The tables must have been published with kv_write_tables() after any
 * import / fork / free.  The per-call metadata travels through a pinned host
 * ring; a call waits only if the ring slot it reuses is still in flight. */
int kv_append(pkv_pool* pool, int32_t n, const int32_t* seq_ids,
              const void* k_new, const void* v_new,
              int32_t* block_tables, int32_t* context_lens, pkv_stream_t stream);

/* 8-bit pools (kv_dtype PKV_FP8_E4M3; k_cache / v_cache hold one E4M3 code per
 * value): the device scales of every (block, kv head), k_scale / v_scale
 * float [num_blocks][num_kv_heads], and the default scales of new blocks,
 * k_init / v_init float [num_kv_heads] (device, caller-owned, borrowed).
 * kv_append on such a pool takes bf16 k_new / v_new, divides each value by
 * its block's scale (fp32) and stores the nearest code (ties to even,
 * saturating at +-448); a row that starts a block this call took first
 * records k_init / v_init as that block's scales; copy-on-write copies the
 * scales with the codes.  Required before kv_append on an 8-bit pool. */
int kv_block_pool_set_fp8_scales(pkv_pool* pool, float* k_scale, float* v_scale,
                                 const float* k_init, const float* v_init);

/* Quantise 16-bit K/V blocks into an 8-bit cache, on `stream`.  items: device
 * int32 [n][3] = (source block, destination block, used rows).  For each item
 * and kv head g, separately for K and V: amax = max |x| over the first `used`
 * rows of the source (block, g) tile; scale = amax / 448 (fp32; 1 when amax is
 * 0) goes to k_scale (v_scale)[destination][g]; every used value becomes the
 * E4M3 code nearest to x / scale (fp32 division; ties to even; saturating);
 * rows from `used` on become code 0.
 *   src_k, src_v : device [*][num_kv_heads][block_size][head_dim] of src_dtype (F16 / BF16)
 *   dst_k, dst_v : device uint8 [*][num_kv_heads][block_size][head_dim]
 *   k_scale, v_scale : device float [*][num_kv_heads]
 * Destination blocks must be distinct. */
int kv_quantize_fp8(int32_t n, const int32_t* items, const void* src_k, const void* src_v,
                    int32_t src_dtype, void* dst_k, void* dst_v, float* k_scale, float* v_scale,
                    int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                    pkv_stream_t stream);

/* Append counts[i] tokens to each of the n listed sequences (a prefill chunk):
 * the same as appending them one at a time, each sequence's tokens in a row,
 * sequences in list order (so the same blocks, slots and copy-on-write), in
 * one call on `stream`.  All or nothing (PKV_ENOMEM, PKV_EINVAL as kv_append;
 * counts may be 0).
 *   seq_ids, counts : host int32 [n]
 *   k_new, v_new    : device [sum(counts)][num_kv_heads][head_dim] of kv_dtype
 *                     (bf16 for 8-bit pools), rows of seq_ids[0] first
 *   block_tables, context_lens : device, as for kv_append
 * The per-token metadata travels through a pinned host ring; a call waits
 * only if the ring slot it reuses is still in flight. */
int kv_append_tokens(pkv_pool* pool, int32_t n, const int32_t* seq_ids, const int32_t* counts,
                     const void* k_new, const void* v_new, int32_t* block_tables,
                     int32_t* context_lens, pkv_stream_t stream);

/* Publish the whole host view to the device tables (-1 past each length,
 * length 0 for free rows and for sequences parked in the host tier), ordered
 * on `stream`. */
int kv_write_tables(pkv_pool* pool, int32_t* block_tables, int32_t* context_lens,
                    pkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Host tier ("LLM+Agent 全栈推理底座" 4.2, TieredBlockManager: a sequence keeps
 * its most recent gpu_window blocks in GPU memory; the colder blocks before
 * them move to pinned host memory and are copied back when the sequence is
 * needed again).
 *
 * Host layout (caller-allocated pinned memory, e.g. hipHostMalloc; the pool
 * borrows it until destroyed):
 *   k_host, v_host : [num_host_blocks][num_kv_heads][block_size][head_dim] of kv_dtype
 * Host blocks come from their own free list, handed out 0, 1, 2, ... and
 * reused last-released-first.  Moving a block gives the moving sequence a
 * private copy in the other tier; the old block loses one reference and is
 * freed when none are left, so a block another sequence still holds stays
 * where it is.  A sequence holding any host block is parked: kv_append and
 * kv_reserve reject it (PKV_EINVAL) and kv_write_tables publishes it with
 * length 0 until kv_seq_restore brings it back.  Block moves are one batched
 * copy kernel per call on `stream` (GPU loads / stores across the host link);
 * later work that reuses a freed block, or reads the host buffers from the
 * CPU, must be ordered after it (same stream or synchronised).
 * ------------------------------------------------------------------------ */

/* Give the pool a host tier of num_host_blocks blocks.  k_host / v_host must
 * be pinned, device-mapped host memory (PKV_EINVAL otherwise), 16-byte
 * aligned, of the layout above.  Once per pool. */
int kv_block_pool_attach_host_tier(pkv_pool* pool, int32_t num_host_blocks, void* k_host,
                                   void* v_host);

/* The host tier of an 8-bit pool (kv_dtype PKV_FP8_E4M3): as above, with the
 * codes in k_host / v_host (uint8 [num_host_blocks][num_kv_heads][block_size]
 * [head_dim]) and each host block's scales in k_scale_host / v_scale_host
 * (float [num_host_blocks][num_kv_heads], pinned, device-mapped, 4-byte
 * aligned): a block's K and V scales move with its codes, both ways.  The
 * pool's device scales (kv_block_pool_set_fp8_scales) must be set before
 * kv_seq_offload / kv_seq_restore.  At most 256 kv heads.
 * kv_block_pool_attach_host_tier refuses an 8-bit pool, and this call a
 * 16-bit one. */
int kv_block_pool_attach_host_tier_fp8(pkv_pool* pool, int32_t num_host_blocks, void* k_host, void* v_host,
                                       float* k_scale_host, float* v_scale_host);

/* For each of the n listed sequences (host array, no repeats) holding more
 * than gpu_window blocks (gpu_window >= 1), move every GPU block before its
 * last gpu_window blocks to a new host block, in sequence order then logical
 * order.  All or nothing: PKV_ENOMEM if the host tier has too few free
 * blocks, PKV_EINVAL for a bad id or window; nothing changes then. */
int kv_seq_offload(pkv_pool* pool, int32_t n, const int32_t* seq_ids, int32_t gpu_window,
                   pkv_stream_t stream);

/* Copy every host block of the n listed sequences back into new GPU blocks
 * (taken from the GPU free list in sequence order, then logical order) and
 * un-park them.  All or nothing: PKV_ENOMEM if the GPU pool has too few free
 * blocks.  Host bookkeeping only changes the device tables through a later
 * kv_write_tables(). */
int kv_seq_restore(pkv_pool* pool, int32_t n, const int32_t* seq_ids, pkv_stream_t stream);

/* Free host blocks, and the reference count of host block `block` (< 0: skip). */
int kv_host_tier_stats(const pkv_pool* pool, int32_t* num_free_out, int32_t block,
                       int32_t* refcount_out);

/* Debug: check host copies of device tables (block_tables [n_seqs][table_stride],
 * context_lens [n_seqs]): every entry a context reaches is in [0, num_blocks)
 * and ceil(len / block_size) <= table_width.  Returns PKV_OK or PKV_EINVAL with
 * the first offending (seq, entry) in the message. */
int kv_validate_tables(int32_t n_seqs, const int32_t* block_tables, int32_t table_stride,
                       int32_t table_width, const int32_t* context_lens,
                       int32_t num_blocks, int32_t block_size);

/* ------------------------------------------------------------------------
 * Decode attention: one query token per sequence over its whole paged context.
 *
 *   q            : device [num_seqs][num_q_heads][head_dim], q_dtype
 *   k_cache,
 *   v_cache      : device [num_blocks][num_kv_heads][block_size][head_dim], kv_dtype
 *   block_tables : device int32, row s at block_tables + s * table_stride
 *   context_lens : device int32 [num_seqs], each in [0, max_context_len]
 *   out          : device [num_seqs][num_q_heads][head_dim], out_dtype; 16-byte
 *                  aligned for PKV_F32, 8-byte aligned for 16-bit outputs
 *   lse          : device float [num_seqs][num_q_heads] or NULL: natural-log
 *                  sum of exp(scores); -inf for an empty context; 4-byte aligned
 * q, k_cache and v_cache are 16-byte aligned; tables and lengths 4-byte.  A
 * misaligned pointer is refused with PKV_EINVAL before anything is enqueued.
 *
 * For q head h the kv head is h / (num_q_heads / num_kv_heads) (contiguous
 * GQA groups).  out[s][h] = sum_t softmax_t(scale * q[s][h] . K[t]) V[t] over
 * t < context_lens[s], with K[t] / V[t] read at block
 * block_tables[s][t / block_size], slot t % block_size.  An empty context
 * gives out = 0.  Scores, softmax and sums are fp32.
 *
 * Split.  All (sequence, kv head, 16-token tile) triples form one list,
 * sequence-major, cut into chunks of C tiles; the grid's waves take the chunks
 * in turn.  (With 8-bit K/V and an even kv head count a wave takes two
 * adjacent kv heads of each tile: the list then runs over (sequence, kv head
 * pair, tile), and both heads of a pair share the pair's segments.)  Balanced mode (partition_size 0): C = max(4, ceil(tiles / waves)),
 * so every wave gets the same share whatever the lengths.  Fixed mode
 * (partition_size P > 0): C = P / 16 and each (sequence, kv head) is padded to
 * whole chunks, so a chunk is exactly the partition [p P, min((p + 1) P, len)).
 * A chunk's part inside one (sequence, kv head) is a segment: its normalised
 * output and lse go to the workspace, and a merge kernel combines the segments
 * of each (sequence, q head) by their lse.  A (sequence, kv head) covered by
 * one segment is written directly.
 * ------------------------------------------------------------------------ */
typedef struct pkv_attn_desc {
    int32_t num_seqs;            /* at most 4096 per call */
    int32_t num_q_heads;
    int32_t num_kv_heads;        /* divides num_q_heads; group size 1..8 */
    int32_t head_dim;            /* 64 or 128 */
    int32_t block_size;          /* 16 or 32 */
    int32_t num_blocks;          /* for documentation and validation only */
    int32_t table_stride;        /* int32 elements between block-table rows */
    int32_t max_context_len;     /* host upper bound of context_lens[] (sizes grid and workspace) */
    int32_t partition_size;      /* 0 = balanced split; else a multiple of block_size (fixed partitions) */
    int32_t q_dtype;             /* PKV_F16 / PKV_BF16: equal to kv_dtype, or PKV_BF16 with 8-bit K/V */
    int32_t kv_dtype;            /* PKV_F16 / PKV_BF16, or PKV_FP8_E4M3 (decode through the _fp8 calls) */
    int32_t out_dtype;           /* PKV_F32, or the same as q_dtype */
    int32_t num_waves;           /* waves in the grid; 0 = every wave that fits the device at once */
} pkv_attn_desc;

/* Partition size of the descriptor's split (0 = balanced), or a negative status. */
int32_t paged_attn_partition_size(const pkv_attn_desc* desc);

/* Waves the decode grid will have (resolves num_waves = 0 with an occupancy
 * query on the current device), or a negative status. */
int32_t paged_attn_grid_waves(const pkv_attn_desc* desc);

/* Kernel launches paged_attn_decode / paged_attn_decode_fp8 makes for the
 * descriptor: 1 when no (sequence, kv head) can span more than one segment
 * (the split kernel writes every output itself), else 2 (split kernel, then
 * merge kernel), or a negative status. */
int32_t paged_attn_decode_launches(const pkv_attn_desc* desc);

/* Bytes of device workspace paged_attn_decode needs (0 on a bad descriptor).
 * With num_waves = 0 the size depends on the current device (the grid is
 * sized by an occupancy query).  Layout, each part 256-byte aligned, with
 * GC = (num_q_heads / num_kv_heads) * HW q heads per row (HW = 2 for an
 * 8-bit cache with an even kv head count, else 1), pairs = num_seqs *
 * num_kv_heads / HW, and rows = pairs + (fixed: pairs * ceil(max_context_len
 * / P); balanced: the grid's waves):
 *   int32 hdr[3 + num_seqs]   (tiles, chunk size, tile prefix [num_seqs + 1])
 *   float seg_out[rows][GC][head_dim]   (normalised segment outputs)
 *   float seg_lse[rows][GC]             (log2-domain lse)
 * Segment k of pair p (sequence s, kv heads p % (num_kv_heads / HW) * HW ..)
 * sits in row (its chunk index) + p, the chunk index being the one
 * paged_attn_plan's slot k counts from. */
size_t paged_attn_workspace_bytes(const pkv_attn_desc* desc);

/* The whole decode: the split pass, then (if a (sequence, kv head) may span
 * several segments) the merge pass, both on `stream`.  workspace: device,
 * 256-byte aligned, workspace_bytes >= paged_attn_workspace_bytes(desc); its
 * contents on entry do not matter.  Calls sharing one workspace must be
 * ordered (same stream or synchronised). */
int paged_attn_decode(const pkv_attn_desc* desc, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* paged_attn_decode for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode, with the workspace taken from a static scratch array that the
 * library holds on every GPU it runs on (32 MiB per GPU, kept until the process
 * ends) instead of a caller buffer.  Arguments as for paged_attn_decode; the
 * caller still owns q, the caches, the tables, out and lse.  The call makes no
 * device allocation.  A descriptor whose workspace (paged_attn_workspace_bytes)
 * exceeds the scratch is refused with PKV_EWORKSPACE before anything is
 * enqueued.  Every call on one GPU uses that GPU's one scratch, which keeps the
 * last call's contents: calls that overlap on one GPU (different streams or
 * threads, unsynchronised) race and give undefined results; order them.  The
 * scratch's address is looked up on the first call on each device. */
int paged_attn_decode_noalloc(const pkv_attn_desc* desc, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, void* out, float* lse,
                              pkv_stream_t stream);

/* The two passes on their own (paged_attn_decode == partials then merge; the
 * partials can be exchanged between them, e.g. for a context-parallel split). */
int paged_attn_decode_partials(const pkv_attn_desc* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, pkv_stream_t stream);
int paged_attn_merge(const pkv_attn_desc* desc, const int32_t* context_lens, void* out,
                     float* lse, const void* workspace, size_t workspace_bytes,
                     pkv_stream_t stream);

/* One decode step in one launch (two when the split leaves segments to
 * merge): kv_append(pool, n, seq_ids, k_new, v_new, block_tables,
 * context_lens, stream) followed by paged_attn_decode(desc, q, the pool's
 * k_cache and v_cache, block_tables, context_lens, scale, out, lse, workspace,
 * workspace_bytes, stream), with the append folded into the split kernel: the
 * kernel takes the appended sequences' lengths and new table entries from the
 * call and their new K/V rows from k_new / v_new, and stores what kv_append
 * stores (rows, lengths, table entries).  Pool state, caches, tables, lengths,
 * out and lse afterwards are bit for bit those of the two calls: the new token
 * attends to itself, as a causal mask lets a query attend to its own position
 * ("从零开始构建LLM推理引擎：模型执行器深度解析" 3.1; the KV cache update is part of
 * executing a batch there, 5.1; metadata is updated between launches,
 * "架构解构：推理引擎的四层抽象", PagedAttention section).
 *   16-bit pools only (8-bit pools: PKV_EUNSUPPORTED); the descriptor's kv
 *   dtype, head_dim, block_size, num_kv_heads must be the pool's and
 *   table_stride its max_blocks_per_seq; every listed sequence must be listed
 *   once, below desc->num_seqs, with room in its table and no blocks in the
 *   host tier, and its new length at most desc->max_context_len (PKV_EINVAL,
 *   nothing enqueued and the pool unchanged).
 *   Up to PKV_FUSE_MAX_ITEMS appended sequences travel in the kernel arguments
 *   (with max_context_len below 2^20); more go through kv_append and the plain
 *   decode (same results).  Sequences whose
 *   tail block is shared get their copy-on-write copy in a launch before.
 *   start / stop: both NULL, or timing events that the split dispatch stamps
 *   as in paged_attn_decode_partials_timed (the merge is not timed). */
enum { PKV_FUSE_MAX_ITEMS = 320 };
int kv_append_decode(pkv_pool* pool, int32_t n, const int32_t* seq_ids, const void* k_new,
                     const void* v_new, int32_t* block_tables, int32_t* context_lens,
                     const pkv_attn_desc* desc, const void* q, float scale, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, pkv_event_t start, pkv_event_t stop,
                     pkv_stream_t stream);

/* paged_attn_decode_partials (16-bit K/V: k_scale = v_scale = NULL) or
 * paged_attn_decode_partials_fp8 (8-bit K/V: the scales as there), with the
 * split kernel's duration taken by two events: start and stop (hipEvent_t,
 * created by the caller with timing enabled, on the stream's device) receive
 * the start and end timestamps of the split kernel's own dispatch
 * (hipExtLaunchKernel), so no marker packets are added to the stream and
 * timed launches run back to back as untimed ones do;
 * hipEventElapsedTime(start, stop) is then the kernel's duration.  Both events
 * must be non-NULL (PKV_EINVAL).  Everything else, including the outputs and
 * the workspace, is as for the untimed calls. */
int paged_attn_decode_partials_timed(const pkv_attn_desc* desc, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     float scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, pkv_event_t start, pkv_event_t stop,
                                     pkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Decode over an 8-bit K/V cache (kv_dtype PKV_FP8_E4M3, q_dtype PKV_BF16).
 * Reduced-precision storage of cached K/V ("从零开始构建LLM推理引擎：模型执行器深度解析"
 * 5.2, KV缓存管理技巧: historical KV kept at reduced precision) in the OCP E4M3 format with one fp32
 * scale per (block, kv head):
 *   k_cache, v_cache : device uint8 [num_blocks][num_kv_heads][block_size][head_dim]
 *   k_scale, v_scale : device float [num_blocks][num_kv_heads]
 * A K (V) code c in block b, kv head g stands for e4m3(c) * k_scale[b][g]
 * (v_scale[b][g]); everything else is paged_attn_decode: scores, softmax and
 * sums in fp32, same split, same workspace, same outputs.  The 16-bit entry
 * points reject an 8-bit descriptor (PKV_EINVAL) and these reject a 16-bit one.
 * ------------------------------------------------------------------------ */
int paged_attn_decode_fp8(const pkv_attn_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const float* k_scale, const float* v_scale,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          pkv_stream_t stream);
int paged_attn_decode_partials_fp8(const pkv_attn_desc* desc, const void* q, const void* k_cache,
                                   const void* v_cache, const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   float scale, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, pkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Chunked prefill attention ("架构解构：推理引擎的四层抽象", FlashAttention
 * section: tiled attention with an online softmax over K/V reached through
 * the block table).  Many query tokens per sequence, causal.
 *
 *   q            : device [total_q][num_q_heads][head_dim], q_dtype
 *   k_cache,
 *   v_cache      : device [num_blocks][num_kv_heads][block_size][head_dim], kv_dtype (= q_dtype)
 *   block_tables : device int32, row s at block_tables + s * table_stride
 *   context_lens : device int32 [num_seqs]: tokens of sequence s in the cache,
 *                  this chunk's included (its K/V must already be written)
 *   cu_seqlens_q : device int32 [num_seqs + 1], non-decreasing from 0 to total_q:
 *                  rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of q and out are
 *                  sequence s's chunk, m_s of them, m_s <= context_lens[s]
 *   out          : device [total_q][num_q_heads][head_dim], out_dtype
 *   lse          : device float [total_q][num_q_heads] or NULL (natural log)
 * Chunk row i of sequence s sits at position context_lens[s] - m_s + i and
 * attends to the tokens at positions 0 .. that position: out = softmax(scale *
 * q . K) V over them, fp32 accumulation.  No workspace; asynchronous on
 * `stream`.  A row whose position would be negative (m_s > context_lens[s],
 * outside the contract) gets out = 0, lse = -inf.
 * ------------------------------------------------------------------------ */
typedef struct pkv_prefill_desc {
    int32_t num_seqs;            /* at most 4096 per call */
    int32_t num_q_heads;
    int32_t num_kv_heads;        /* divides num_q_heads */
    int32_t head_dim;            /* 64 or 128 */
    int32_t block_size;          /* 16 or 32 */
    int32_t num_blocks;          /* for documentation and validation only */
    int32_t table_stride;        /* int32 elements between block-table rows */
    int32_t total_q;             /* rows of q / out (= cu_seqlens_q[num_seqs]) */
    int32_t max_context_len;     /* host upper bound of context_lens[] */
    int32_t q_dtype;             /* PKV_F16 / PKV_BF16 */
    int32_t kv_dtype;            /* equal to q_dtype */
    int32_t out_dtype;           /* PKV_F32 or q_dtype */
} pkv_prefill_desc;

int paged_attn_prefill(const pkv_prefill_desc* desc, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* cu_seqlens_q, float scale,
                       void* out, float* lse, pkv_stream_t stream);

/* Measurement: read the first floor(bytes / 16384) * 16384 bytes of buf (device,
 * 16-byte aligned) once with 16-byte vector loads, each wave taking contiguous
 * 16 KiB pieces in turn, workgroups x 256 threads, non-temporal loads if
 * nontemporal != 0 -- the rate HBM delivers to plain streaming reads, the
 * ceiling for the decode kernels' K/V reads.  sink: device uint32
 * [workgroups * 256], written only in the (practically never) case that a
 * thread's XOR of its loaded words equals 0x9E3779B9.  Asynchronous on `stream`. */
int pkv_read_probe(const void* buf, size_t bytes, int32_t workgroups, int32_t nontemporal, uint32_t* sink,
                   pkv_stream_t stream);

/* Debug: the segments of the split for host context lengths, in (seq, kv
 * head, slot) order, as rows of 5 int32: seq, kv_head, slot, tok_lo, tok_hi.
 * Writes min(count, cap) rows to items_out (nullable) and the count to *n_out.
 * With num_waves = 0 in balanced mode this queries the current device. */
int paged_attn_plan(const pkv_attn_desc* desc, const int32_t* context_lens_host,
                    int32_t* items_out, int64_t cap, int64_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
