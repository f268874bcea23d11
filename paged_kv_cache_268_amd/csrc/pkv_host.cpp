// pkv_host.cpp -- host side of libpkv.so: the C ABI of include/pkv.h.
//
// Block pool bookkeeping follows the page's BlockManager ("LLM+Agent 全栈推理底座",
// 4.2): fixed-size blocks, ceil(n / block_size) blocks per sequence, blocks
// taken by popping the end of a free list.  The device pool is fixed, so an
// empty free list is an error (PKV_ENOMEM), never growth.  The block table is
// kept here on the host and published to the device between kernel launches
// ("架构解构：推理引擎的四层抽象", PagedAttention section and runtime layer).
// Shared blocks (prefix reuse, "LLM+Agent 全栈推理底座" 2.2 / 4.4) carry a
// reference count and are copied before a write (copy-on-write).
// The host tier ("LLM+Agent 全栈推理底座" 4.2, TieredBlockManager) keeps a
// sequence's last gpu_window blocks on the GPU and moves the ones before them
// to caller-owned pinned host memory, copied back when the sequence is needed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pkv.h"
#include "pkv_append.h"
#include "pkv_fp8.h"
#include "pkv_noalloc.h"
#include "pkv_probe.h"
#include "pkv_kernels.h"
#include "pkv_prefill.h"
#include "pkv_tier.h"

static_assert(pkv::kFuseItems == PKV_FUSE_MAX_ITEMS, "the fused kernel carries the documented number of items");

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int fail_hip(hipError_t e, const char* what) {
    return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kRing = 8;   // pinned staging slots for kv_append metadata
constexpr int kCopyRing = 4;   // pinned staging slots for host-tier block moves

// A block list entry: a GPU block id b >= 0, or host block c written -2 - c.
inline bool is_host(int32_t e) { return e <= -2; }
inline int32_t host_id(int32_t e) { return -2 - e; }
inline int32_t host_entry(int32_t c) { return -2 - c; }

}  // namespace

struct pkv_pool {
    pkv_pool_desc d{};
    void* k_cache = nullptr;
    void* v_cache = nullptr;
    // 8-bit pools: per-(block, kv head) scales and the default scales of new blocks (device).
    float* k_scale = nullptr;
    float* v_scale = nullptr;
    const float* k_init = nullptr;
    const float* v_init = nullptr;

    // Free list: a stack (allocation pops the back).  Removing a block from
    // the middle (kv_seq_import) leaves a tombstone (-1) so the order of the
    // rest is kept; pos[b] is b's index in the stack or -1.
    std::vector<int32_t> stack;
    std::vector<int32_t> pos;
    int32_t num_free = 0;

    std::vector<int32_t> ref;                    // holders per block
    std::vector<std::vector<int32_t>> blocks;    // per sequence row
    std::vector<int32_t> len;
    std::vector<uint8_t> live;
    int32_t num_live = 0;

    struct Slot {
        pkv::AppendItem* host = nullptr;
        hipEvent_t ev = nullptr;
        bool pending = false;
    };
    Slot ring[kRing];
    int next = 0;
    bool ring_ready = false;
    std::vector<pkv::AppendItem> stage;          // kv_append items before they go to the kernel

    int32_t* tab_host = nullptr;                 // staging for kv_write_tables
    hipEvent_t tab_ev = nullptr;
    bool tab_pending = false;

    // Host tier: caller-owned pinned buffers, their device-mapped addresses,
    // a LIFO free list of host blocks and a reference count per host block.
    int32_t num_host = 0;
    void* k_host_dev = nullptr;
    void* v_host_dev = nullptr;
    float* ks_host_dev = nullptr;                // 8-bit pools: host-tier scales [num_host][Hkv]
    float* vs_host_dev = nullptr;
    std::vector<int32_t> host_stack;
    std::vector<int32_t> host_ref;
    std::vector<int32_t> nhost;                  // host blocks held, per sequence row (> 0: parked)
    struct CopySlot {
        int32_t* pairs = nullptr;                // pinned, device-readable [cap][2]
        int64_t cap = 0;
        hipEvent_t ev = nullptr;
        bool pending = false;
    };
    CopySlot copy_ring[kCopyRing];
    int copy_next = 0;
    struct TokSlot {                             // kv_append_tokens staging (pinned, device-readable)
        uint8_t* buf = nullptr;
        size_t cap = 0;
        hipEvent_t ev = nullptr;
        bool pending = false;
    };
    TokSlot tok_ring[kCopyRing];
    int tok_next = 0;

    int32_t pop_free() {
        while (!stack.empty() && stack.back() < 0) stack.pop_back();
        const int32_t b = stack.back();
        stack.pop_back();
        pos[b] = -1;
        --num_free;
        return b;
    }
    void push_free(int32_t b) {
        pos[b] = (int32_t)stack.size();
        stack.push_back(b);
        ++num_free;
    }
    void remove_free(int32_t b) {
        stack[pos[b]] = -1;
        pos[b] = -1;
        --num_free;
        if (stack.size() > 64 && (size_t)num_free * 2 < stack.size()) compact();
    }
    void compact() {
        std::vector<int32_t> s;
        s.reserve(num_free);
        for (int32_t b : stack)
            if (b >= 0) {
                pos[b] = (int32_t)s.size();
                s.push_back(b);
            }
        stack.swap(s);
    }
    int32_t new_row() const {
        for (int32_t i = 0; i < d.max_seqs; ++i)
            if (!live[i]) return i;
        return -1;
    }
    bool valid_seq(int32_t s) const { return s >= 0 && s < d.max_seqs && live[s]; }

    // Drop one holder of a block-list entry; a block with none left is freed in its tier.
    void unref(int32_t e) {
        if (is_host(e)) {
            const int32_t c = host_id(e);
            if (--host_ref[c] == 0) host_stack.push_back(c);
        } else if (--ref[e] == 0) {
            push_free(e);
        }
    }
    void addref(int32_t e) {
        if (is_host(e)) ++host_ref[host_id(e)];
        else ++ref[e];
    }
};

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

// --------------------------------------------------------------------------
// Pool
// --------------------------------------------------------------------------

int kv_block_pool_create(const pkv_pool_desc* desc, void* k_cache, void* v_cache,
                         const int32_t* alloc_order, pkv_pool** out) {
    if (!desc || !out) return fail(PKV_EINVAL, "kv_block_pool_create: null desc or out");
    const pkv_pool_desc& d = *desc;
    if (d.num_blocks < 1 || d.num_kv_heads < 1 || d.max_seqs < 1 || d.max_blocks_per_seq < 1)
        return fail(PKV_EINVAL, "kv_block_pool_create: sizes must be positive");
    if (d.block_size != 16 && d.block_size != 32)
        return fail(PKV_EUNSUPPORTED, "block_size %d (16 or 32)", d.block_size);
    if (d.head_dim != 64 && d.head_dim != 128)
        return fail(PKV_EUNSUPPORTED, "head_dim %d (64 or 128)", d.head_dim);
    if (d.kv_dtype != PKV_F16 && d.kv_dtype != PKV_BF16 && d.kv_dtype != PKV_FP8_E4M3)
        return fail(PKV_EUNSUPPORTED, "kv_dtype %d (PKV_F16, PKV_BF16 or PKV_FP8_E4M3)", d.kv_dtype);
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
        return fail(PKV_EINVAL, "k_cache / v_cache must be 16-byte aligned");
    std::vector<uint8_t> seen(d.num_blocks, 0);
    if (alloc_order) {
        for (int32_t i = 0; i < d.num_blocks; ++i) {
            const int32_t b = alloc_order[i];
            if (b < 0 || b >= d.num_blocks || seen[b])
                return fail(PKV_EINVAL, "alloc_order is not a permutation (entry %d = %d)", i, b);
            seen[b] = 1;
        }
    }
    pkv_pool* p = new pkv_pool;
    p->d = d;
    p->k_cache = k_cache;
    p->v_cache = v_cache;
    p->stack.resize(d.num_blocks);
    p->pos.resize(d.num_blocks);
    for (int32_t i = 0; i < d.num_blocks; ++i) {
        const int32_t b = alloc_order ? alloc_order[d.num_blocks - 1 - i] : d.num_blocks - 1 - i;
        p->stack[i] = b;
        p->pos[b] = i;
    }
    p->num_free = d.num_blocks;
    p->ref.assign(d.num_blocks, 0);
    p->blocks.assign(d.max_seqs, {});
    p->len.assign(d.max_seqs, 0);
    p->live.assign(d.max_seqs, 0);
    p->nhost.assign(d.max_seqs, 0);
    *out = p;
    return PKV_OK;
}

void kv_block_pool_destroy(pkv_pool* p) {
    if (!p) return;
    for (auto& s : p->ring) {
        if (s.pending) (void)hipEventSynchronize(s.ev);
        if (s.ev) (void)hipEventDestroy(s.ev);
        if (s.host) (void)hipHostFree(s.host);
    }
    for (auto& c : p->copy_ring) {
        if (c.pending) (void)hipEventSynchronize(c.ev);
        if (c.ev) (void)hipEventDestroy(c.ev);
        if (c.pairs) (void)hipHostFree(c.pairs);
    }
    for (auto& t : p->tok_ring) {
        if (t.pending) (void)hipEventSynchronize(t.ev);
        if (t.ev) (void)hipEventDestroy(t.ev);
        if (t.buf) (void)hipHostFree(t.buf);
    }
    if (p->tab_pending) (void)hipEventSynchronize(p->tab_ev);
    if (p->tab_ev) (void)hipEventDestroy(p->tab_ev);
    if (p->tab_host) (void)hipHostFree(p->tab_host);
    delete p;
}

int kv_seq_add(pkv_pool* p, int32_t* seq_id_out) {
    if (!p || !seq_id_out) return fail(PKV_EINVAL, "kv_seq_add: null argument");
    const int32_t s = p->new_row();
    if (s < 0) return fail(PKV_ENOMEM, "kv_seq_add: all %d sequence rows in use", p->d.max_seqs);
    p->live[s] = 1;
    p->blocks[s].clear();
    p->len[s] = 0;
    p->nhost[s] = 0;
    ++p->num_live;
    *seq_id_out = s;
    return PKV_OK;
}

int kv_seq_import(pkv_pool* p, int32_t len, const int32_t* block_ids, int32_t n_blocks,
                  int32_t* seq_id_out) {
    if (!p || !seq_id_out || (n_blocks > 0 && !block_ids)) return fail(PKV_EINVAL, "kv_seq_import: null argument");
    const int32_t bs = p->d.block_size;
    if (len < 0 || n_blocks != ceil_div(len, bs))
        return fail(PKV_EINVAL, "kv_seq_import: %d blocks for %d tokens (need %lld)", n_blocks, len,
                    (long long)ceil_div(len, bs));
    if (n_blocks > p->d.max_blocks_per_seq)
        return fail(PKV_EINVAL, "kv_seq_import: %d blocks > max_blocks_per_seq %d", n_blocks, p->d.max_blocks_per_seq);
    std::vector<int32_t> ids(block_ids, block_ids + n_blocks);
    std::vector<int32_t> sorted = ids;
    std::sort(sorted.begin(), sorted.end());
    for (size_t i = 0; i < sorted.size(); ++i) {
        if (sorted[i] < 0 || sorted[i] >= p->d.num_blocks)
            return fail(PKV_EINVAL, "kv_seq_import: block id %d out of range", sorted[i]);
        if (i && sorted[i] == sorted[i - 1]) return fail(PKV_EINVAL, "kv_seq_import: block %d repeated", sorted[i]);
    }
    const int32_t s = p->new_row();
    if (s < 0) return fail(PKV_ENOMEM, "kv_seq_import: all %d sequence rows in use", p->d.max_seqs);
    for (int32_t b : ids) {
        if (p->ref[b] == 0) p->remove_free(b);
        ++p->ref[b];
    }
    p->live[s] = 1;
    p->blocks[s] = ids;
    p->len[s] = len;
    p->nhost[s] = 0;
    ++p->num_live;
    *seq_id_out = s;
    return PKV_OK;
}

int kv_seq_fork(pkv_pool* p, int32_t src, int32_t* seq_id_out) {
    if (!p || !seq_id_out) return fail(PKV_EINVAL, "kv_seq_fork: null argument");
    if (!p->valid_seq(src)) return fail(PKV_EINVAL, "kv_seq_fork: unknown sequence %d", src);
    const int32_t s = p->new_row();
    if (s < 0) return fail(PKV_ENOMEM, "kv_seq_fork: all %d sequence rows in use", p->d.max_seqs);
    for (int32_t b : p->blocks[src]) p->addref(b);
    p->live[s] = 1;
    p->blocks[s] = p->blocks[src];
    p->len[s] = p->len[src];
    p->nhost[s] = p->nhost[src];
    ++p->num_live;
    *seq_id_out = s;
    return PKV_OK;
}

int kv_seq_free(pkv_pool* p, int32_t s) {
    if (!p) return fail(PKV_EINVAL, "kv_seq_free: null pool");
    if (!p->valid_seq(s)) return fail(PKV_EINVAL, "kv_seq_free: unknown sequence %d", s);
    for (int32_t b : p->blocks[s]) p->unref(b);
    p->blocks[s].clear();
    p->len[s] = 0;
    p->nhost[s] = 0;
    p->live[s] = 0;
    --p->num_live;
    return PKV_OK;
}

int kv_seq_info(const pkv_pool* p, int32_t s, int32_t* len_out, int32_t* block_ids_out, int32_t cap,
                int32_t* n_blocks_out) {
    if (!p) return fail(PKV_EINVAL, "kv_seq_info: null pool");
    if (!p->valid_seq(s)) return fail(PKV_EINVAL, "kv_seq_info: unknown sequence %d", s);
    const auto& b = p->blocks[s];
    if (len_out) *len_out = p->len[s];
    if (n_blocks_out) *n_blocks_out = (int32_t)b.size();
    if (block_ids_out)
        for (int32_t i = 0; i < cap && i < (int32_t)b.size(); ++i) block_ids_out[i] = b[i];
    return PKV_OK;
}

int kv_pool_stats(const pkv_pool* p, int32_t* num_free_out, int32_t* num_seqs_out, int32_t block,
                  int32_t* refcount_out) {
    if (!p) return fail(PKV_EINVAL, "kv_pool_stats: null pool");
    if (num_free_out) *num_free_out = p->num_free;
    if (num_seqs_out) *num_seqs_out = p->num_live;
    if (block >= 0) {
        if (block >= p->d.num_blocks) return fail(PKV_EINVAL, "kv_pool_stats: block %d out of range", block);
        if (refcount_out) *refcount_out = p->ref[block];
    }
    return PKV_OK;
}

// The slot of sequence s's next token (capacity checked by the caller): a new
// block when its length is a multiple of block_size, else a copy of a shared,
// partly filled tail (copy-on-write), else the tail itself.
static pkv::AppendItem take_slot(pkv_pool* p, int32_t s) {
    const int32_t bs = p->d.block_size;
    auto& blk = p->blocks[s];
    const int32_t t = p->len[s];
    const int32_t tpos = t / bs, off = t % bs;
    pkv::AppendItem it{s, 0, tpos, -1, -1, 0, t + 1};
    if (off == 0) {
        it.new_block = p->pop_free();
        p->ref[it.new_block] = 1;
        blk.push_back(it.new_block);
    } else if (p->ref[blk.back()] > 1) {
        it.new_block = p->pop_free();
        p->ref[it.new_block] = 1;
        it.cow_src = blk.back();
        it.cow_ntok = off;
        --p->ref[it.cow_src];
        blk.back() = it.new_block;
    }
    it.slot = blk[tpos] * bs + off;
    p->len[s] = t + 1;
    return it;
}

// Blocks that copy-on-write takes in one call, given the shared (reference
// count > 1), partly filled tail block of every listed sequence that writes
// into its tail.  Sequences copy in list order while the tail still has
// another holder, and each copy drops one reference, so k listed holders of a
// tail held r times take min(k, r - 1) copies: when every holder is listed,
// the last one writes in place.
static int64_t cow_blocks(const pkv_pool* p, std::vector<int32_t>& tails) {
    std::sort(tails.begin(), tails.end());
    int64_t n = 0;
    for (size_t i = 0; i < tails.size();) {
        size_t j = i;
        while (j < tails.size() && tails[j] == tails[i]) ++j;
        n += std::min<int64_t>((int64_t)(j - i), (int64_t)p->ref[tails[i]] - 1);
        i = j;
    }
    return n;
}

static int reserve_impl(pkv_pool* p, int32_t n, const int32_t* seq_ids, pkv::AppendItem* items, bool* any_copy) {
    if (n < 0 || (n > 0 && !seq_ids)) return fail(PKV_EINVAL, "kv_reserve: bad n or seq_ids");
    const int32_t bs = p->d.block_size;
    std::vector<uint8_t> mark(p->d.max_seqs, 0);
    std::vector<int32_t> shared_tails;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        if (!p->valid_seq(s)) return fail(PKV_EINVAL, "kv_reserve: unknown sequence %d", s);
        if (mark[s]) return fail(PKV_EINVAL, "kv_reserve: sequence %d listed twice", s);
        if (p->nhost[s]) return fail(PKV_EINVAL, "kv_reserve: sequence %d has blocks in the host tier (restore it first)", s);
        mark[s] = 1;
        const int32_t t = p->len[s];
        if (t % bs == 0) {
            if (t / bs >= p->d.max_blocks_per_seq)
                return fail(PKV_EINVAL, "kv_reserve: sequence %d is full (%d blocks)", s, p->d.max_blocks_per_seq);
            ++need;
        } else if (p->ref[p->blocks[s].back()] > 1) {
            shared_tails.push_back(p->blocks[s].back());
        }
    }
    need += cow_blocks(p, shared_tails);
    if (need > p->num_free)
        return fail(PKV_ENOMEM, "kv_reserve: need %lld blocks, %d free", (long long)need, p->num_free);
    bool copy = false;
    for (int32_t i = 0; i < n; ++i) {
        const pkv::AppendItem it = take_slot(p, seq_ids[i]);
        copy |= it.cow_src >= 0;
        if (items) items[i] = it;
    }
    if (any_copy) *any_copy = copy;
    return PKV_OK;
}

int kv_reserve(pkv_pool* p, int32_t n, const int32_t* seq_ids, int32_t* items_out) {
    if (!p) return fail(PKV_EINVAL, "kv_reserve: null pool");
    static_assert(sizeof(pkv::AppendItem) == 7 * sizeof(int32_t), "item layout");
    return reserve_impl(p, n, seq_ids, reinterpret_cast<pkv::AppendItem*>(items_out), nullptr);
}

static int ensure_ring(pkv_pool* p) {
    if (p->ring_ready) return PKV_OK;
    for (auto& s : p->ring) {
        hipError_t e = hipHostMalloc((void**)&s.host, sizeof(pkv::AppendItem) * (size_t)p->d.max_seqs,
                                     hipHostMallocCoherent | hipHostMallocMapped);
        if (e != hipSuccess) return fail_hip(e, "hipHostMalloc (append staging)");
        e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
        if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
    }
    p->ring_ready = true;
    return PKV_OK;
}

int kv_block_pool_set_fp8_scales(pkv_pool* p, float* k_scale, float* v_scale, const float* k_init,
                                 const float* v_init) {
    if (!p) return fail(PKV_EINVAL, "kv_block_pool_set_fp8_scales: null pool");
    if (p->d.kv_dtype != PKV_FP8_E4M3) return fail(PKV_EINVAL, "kv_block_pool_set_fp8_scales: not an 8-bit pool");
    if (!k_scale || !v_scale || !k_init || !v_init || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
        !aligned(k_init, 4) || !aligned(v_init, 4))
        return fail(PKV_EINVAL, "kv_block_pool_set_fp8_scales: null or misaligned pointer");
    p->k_scale = k_scale;
    p->v_scale = v_scale;
    p->k_init = k_init;
    p->v_init = v_init;
    return PKV_OK;
}

int kv_append(pkv_pool* p, int32_t n, const int32_t* seq_ids, const void* k_new, const void* v_new,
              int32_t* block_tables, int32_t* context_lens, pkv_stream_t stream) {
    if (!p) return fail(PKV_EINVAL, "kv_append: null pool");
    if (n == 0) return PKV_OK;
    const bool kv8 = p->d.kv_dtype == PKV_FP8_E4M3;
    if (kv8 && !p->k_scale) return fail(PKV_EINVAL, "kv_append: 8-bit pool without scales (kv_block_pool_set_fp8_scales)");
    if (!k_new || !v_new || !block_tables || !context_lens || !p->k_cache || !p->v_cache)
        return fail(PKV_EINVAL, "kv_append: null device pointer");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return fail(PKV_EINVAL, "kv_append: k_new / v_new must be 16-byte aligned");
    if (n < 0 || n > p->d.max_seqs) return fail(PKV_EINVAL, "kv_append: n = %d", n);
    // Up to kArgItems items without copy-on-write travel in the kernel
    // arguments: nothing on the device reads host memory and the call needs no
    // staging slot (and no event to guard one).  Otherwise the items go through
    // the pinned ring.
    int rc = ensure_ring(p);
    if (rc) return rc;
    auto& slot = p->ring[p->next];
    const bool small = n <= pkv::kArgItems;
    if (!small && slot.pending) {
        hipError_t e = hipEventSynchronize(slot.ev);
        if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize (append staging)");
        slot.pending = false;
    }
    if (p->stage.size() < (size_t)n) p->stage.resize((size_t)p->d.max_seqs);
    pkv::AppendItem* items = small ? p->stage.data() : slot.host;
    bool any_copy = false;
    rc = reserve_impl(p, n, seq_ids, items, &any_copy);
    if (rc) return rc;
    const bool staged = !small || any_copy;   // the device reads the items from the ring slot
    if (staged && small) {
        if (slot.pending) {
            hipError_t e = hipEventSynchronize(slot.ev);
            if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize (append staging; pool state now ahead of the device)");
            slot.pending = false;
        }
        std::memcpy(slot.host, items, sizeof(pkv::AppendItem) * (size_t)n);
        items = slot.host;
    }
    pkv::AppendArgs a{};
    a.items = staged ? slot.host : nullptr;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = p->k_cache;
    a.v_cache = p->v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.n = n;
    a.num_kv_heads = p->d.num_kv_heads;
    a.head_dim = p->d.head_dim;
    a.block_size = p->d.block_size;
    a.table_stride = p->d.max_blocks_per_seq;
    a.kv8 = kv8 ? 1 : 0;
    a.k_scale = p->k_scale;
    a.v_scale = p->v_scale;
    a.k_init = p->k_init;
    a.v_init = p->v_init;
    pkv::ArgItems inl;
    if (small)
        for (int32_t i = 0; i < n; ++i) inl.it[i] = {items[i].seq, items[i].slot, items[i].new_block, items[i].new_len};
    hipError_t e = pkv::launch_append(a, any_copy, small ? &inl : nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "kv_append launch (pool state now ahead of the device)");
    if (staged) {
        e = hipEventRecord(slot.ev, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
        slot.pending = true;
        p->next = (p->next + 1) % kRing;
    }
    return PKV_OK;
}

int kv_append_tokens(pkv_pool* p, int32_t n, const int32_t* seq_ids, const int32_t* counts, const void* k_new,
                     const void* v_new, int32_t* block_tables, int32_t* context_lens, pkv_stream_t stream) {
    if (!p) return fail(PKV_EINVAL, "kv_append_tokens: null pool");
    if (n < 0 || n > p->d.max_seqs || (n > 0 && (!seq_ids || !counts)))
        return fail(PKV_EINVAL, "kv_append_tokens: bad n, seq_ids or counts");
    const bool kv8 = p->d.kv_dtype == PKV_FP8_E4M3;
    if (kv8 && !p->k_scale) return fail(PKV_EINVAL, "kv_append_tokens: 8-bit pool without scales (kv_block_pool_set_fp8_scales)");
    const int32_t bs = p->d.block_size;
    std::vector<uint8_t> mark(p->d.max_seqs, 0);
    std::vector<int32_t> shared_tails;
    int64_t need = 0, total = 0, cows = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i], c = counts[i];
        if (!p->valid_seq(s)) return fail(PKV_EINVAL, "kv_append_tokens: unknown sequence %d", s);
        if (mark[s]) return fail(PKV_EINVAL, "kv_append_tokens: sequence %d listed twice", s);
        mark[s] = 1;
        if (p->nhost[s]) return fail(PKV_EINVAL, "kv_append_tokens: sequence %d has blocks in the host tier", s);
        if (c < 0) return fail(PKV_EINVAL, "kv_append_tokens: count %d", c);
        if (c == 0) continue;
        const int64_t t = p->len[s];
        if (ceil_div(t + c, bs) > p->d.max_blocks_per_seq)
            return fail(PKV_EINVAL, "kv_append_tokens: sequence %d would exceed %d blocks", s, p->d.max_blocks_per_seq);
        need += ceil_div(t + c, bs) - ceil_div(t, bs);
        if (t % bs && p->ref[p->blocks[s].back()] > 1) {
            shared_tails.push_back(p->blocks[s].back());
            ++cows;                              // upper bound: sizes the staging buffer
        }
        total += c;
    }
    need += cow_blocks(p, shared_tails);
    if (need > p->num_free)
        return fail(PKV_ENOMEM, "kv_append_tokens: need %lld blocks, %d free", (long long)need, p->num_free);
    if (total == 0) return PKV_OK;
    if (total > 0x7FFFFFFF) return fail(PKV_EINVAL, "kv_append_tokens: too many tokens");
    if (!k_new || !v_new || !block_tables || !context_lens || !p->k_cache || !p->v_cache)
        return fail(PKV_EINVAL, "kv_append_tokens: null device pointer");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return fail(PKV_EINVAL, "kv_append_tokens: k_new / v_new must be 16-byte aligned");
    // Staging: tokens, then copy-on-write items, in one pinned buffer of a small ring.
    const size_t tok_bytes = sizeof(pkv::TokenItem) * (size_t)total;
    const size_t cow_off = (tok_bytes + 255) / 256 * 256;
    const size_t bytes = cow_off + sizeof(pkv::AppendItem) * (size_t)std::max<int64_t>(cows, 1);
    auto& sl = p->tok_ring[p->tok_next];
    if (!sl.ev) {
        hipError_t e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
        if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags (token staging)");
    }
    if (sl.pending) {
        hipError_t e = hipEventSynchronize(sl.ev);
        if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize (token staging)");
        sl.pending = false;
    }
    if (sl.cap < bytes) {
        if (sl.buf) (void)hipHostFree(sl.buf);
        sl.buf = nullptr;
        sl.cap = 0;
        const size_t cap = std::max<size_t>(bytes, 65536);
        hipError_t e = hipHostMalloc((void**)&sl.buf, cap, hipHostMallocCoherent | hipHostMallocMapped);
        if (e != hipSuccess) return fail_hip(e, "hipHostMalloc (token staging)");
        sl.cap = cap;
    }
    auto* tok = reinterpret_cast<pkv::TokenItem*>(sl.buf);
    auto* cow = reinterpret_cast<pkv::AppendItem*>(sl.buf + cow_off);
    int64_t k = 0, nc = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i], c = counts[i];
        int32_t fresh_block = -1;                // block this sequence opened (not copied) in this call
        for (int32_t j = 0; j < c; ++j) {
            const pkv::AppendItem it = take_slot(p, s);
            int32_t flags = 0;
            if (j == c - 1) flags |= pkv::kTokLast;
            if (it.new_block >= 0) {
                flags |= pkv::kTokTable;
                fresh_block = it.cow_src >= 0 ? -1 : it.new_block;
            }
            if (it.cow_src >= 0) cow[nc++] = it;
            if (fresh_block >= 0 && it.slot / bs == fresh_block) flags |= pkv::kTokFresh;
            tok[k++] = pkv::TokenItem{s, it.slot, it.tpos, flags};
        }
    }
    pkv::AppendArgs a{};
    a.items = cow;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = p->k_cache;
    a.v_cache = p->v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.n = (int32_t)nc;
    a.num_kv_heads = p->d.num_kv_heads;
    a.head_dim = p->d.head_dim;
    a.block_size = bs;
    a.table_stride = p->d.max_blocks_per_seq;
    a.kv8 = kv8 ? 1 : 0;
    a.k_scale = p->k_scale;
    a.v_scale = p->v_scale;
    a.k_init = p->k_init;
    a.v_init = p->v_init;
    hipError_t e = pkv::launch_append_tokens(a, (int32_t)total, tok, nc > 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "kv_append_tokens launch (pool state now ahead of the device)");
    e = hipEventRecord(sl.ev, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
    sl.pending = true;
    p->tok_next = (p->tok_next + 1) % kCopyRing;
    return PKV_OK;
}

int kv_write_tables(pkv_pool* p, int32_t* block_tables, int32_t* context_lens, pkv_stream_t stream) {
    if (!p || !block_tables || !context_lens) return fail(PKV_EINVAL, "kv_write_tables: null argument");
    const size_t W = p->d.max_blocks_per_seq, S = p->d.max_seqs;
    if (!p->tab_host) {
        hipError_t e = hipHostMalloc((void**)&p->tab_host, sizeof(int32_t) * S * (W + 1), hipHostMallocDefault);
        if (e != hipSuccess) return fail_hip(e, "hipHostMalloc (table staging)");
        e = hipEventCreateWithFlags(&p->tab_ev, hipEventDisableTiming);
        if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
    }
    if (p->tab_pending) {
        hipError_t e = hipEventSynchronize(p->tab_ev);
        if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize (table staging)");
        p->tab_pending = false;
    }
    int32_t* tab = p->tab_host;
    int32_t* lens = p->tab_host + S * W;
    for (size_t s = 0; s < S; ++s) {
        const auto& b = p->blocks[s];
        const bool parked = p->nhost[s] > 0;     // not attendable until restored
        for (size_t j = 0; j < W; ++j) tab[s * W + j] = !parked && j < b.size() ? b[j] : -1;
        lens[s] = parked ? 0 : p->len[s];
    }
    hipError_t e = hipMemcpyAsync(block_tables, tab, sizeof(int32_t) * S * W, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(context_lens, lens, sizeof(int32_t) * S, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e == hipSuccess) e = hipEventRecord(p->tab_ev, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "kv_write_tables copy");
    p->tab_pending = true;
    return PKV_OK;
}

// --------------------------------------------------------------------------
// Host tier
// --------------------------------------------------------------------------

// Device-mapped address of pinned host memory, or null (pageable memory is refused).
static void* mapped(void* h) {
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, h) != hipSuccess || at.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return d;
}

static int attach_tier(pkv_pool* p, int32_t num_host_blocks, void* k_host, void* v_host, float* ks_host,
                       float* vs_host, const char* who) {
    if (p->num_host) return fail(PKV_EINVAL, "%s: the pool already has a host tier", who);
    if (num_host_blocks < 1) return fail(PKV_EINVAL, "%s: %d host blocks", who, num_host_blocks);
    if (!aligned(k_host, 16) || !aligned(v_host, 16))
        return fail(PKV_EINVAL, "%s: host buffers must be 16-byte aligned", who);
    if (ks_host && (!aligned(ks_host, 4) || !aligned(vs_host, 4)))
        return fail(PKV_EINVAL, "%s: host scale arrays must be 4-byte aligned", who);
    // Only pinned host memory (hipHostMalloc) is reachable from a kernel; a
    // pageable buffer is refused here, before any copy could touch it.
    void* kd = mapped(k_host);
    void* vd = mapped(v_host);
    void* ksd = ks_host ? mapped(ks_host) : nullptr;
    void* vsd = vs_host ? mapped(vs_host) : nullptr;
    if (!kd || !vd || (ks_host && (!ksd || !vsd)))
        return fail(PKV_EINVAL, "%s: host buffers are not pinned, device-mapped host memory "
                                "(allocate them with hipHostMalloc)", who);
    p->num_host = num_host_blocks;
    p->k_host_dev = kd;
    p->v_host_dev = vd;
    p->ks_host_dev = static_cast<float*>(ksd);
    p->vs_host_dev = static_cast<float*>(vsd);
    p->host_stack.resize(num_host_blocks);
    for (int32_t i = 0; i < num_host_blocks; ++i) p->host_stack[i] = num_host_blocks - 1 - i;   // pops 0, 1, ...
    p->host_ref.assign(num_host_blocks, 0);
    return PKV_OK;
}

int kv_block_pool_attach_host_tier(pkv_pool* p, int32_t num_host_blocks, void* k_host, void* v_host) {
    if (!p || !k_host || !v_host) return fail(PKV_EINVAL, "kv_block_pool_attach_host_tier: null argument");
    if (p->d.kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_EINVAL, "kv_block_pool_attach_host_tier: an 8-bit pool's host tier also holds the block "
                                "scales (kv_block_pool_attach_host_tier_fp8)");
    return attach_tier(p, num_host_blocks, k_host, v_host, nullptr, nullptr, "kv_block_pool_attach_host_tier");
}

int kv_block_pool_attach_host_tier_fp8(pkv_pool* p, int32_t num_host_blocks, void* k_host, void* v_host,
                                       float* k_scale_host, float* v_scale_host) {
    const char* who = "kv_block_pool_attach_host_tier_fp8";
    if (!p || !k_host || !v_host || !k_scale_host || !v_scale_host) return fail(PKV_EINVAL, "%s: null argument", who);
    if (p->d.kv_dtype != PKV_FP8_E4M3) return fail(PKV_EINVAL, "%s: not an 8-bit pool", who);
    if (p->d.num_kv_heads > 256)
        return fail(PKV_EUNSUPPORTED, "%s: %d kv heads (the block-move kernel carries at most 256 scales per block)",
                    who, p->d.num_kv_heads);
    return attach_tier(p, num_host_blocks, k_host, v_host, k_scale_host, v_scale_host, who);
}

int kv_host_tier_stats(const pkv_pool* p, int32_t* num_free_out, int32_t block, int32_t* refcount_out) {
    if (!p) return fail(PKV_EINVAL, "kv_host_tier_stats: null pool");
    if (!p->num_host) return fail(PKV_EINVAL, "kv_host_tier_stats: the pool has no host tier");
    if (num_free_out) *num_free_out = (int32_t)p->host_stack.size();
    if (block >= 0) {
        if (block >= p->num_host) return fail(PKV_EINVAL, "kv_host_tier_stats: host block %d out of range", block);
        if (refcount_out) *refcount_out = p->host_ref[block];
    }
    return PKV_OK;
}

// A staging slot for n (source, destination) pairs, waiting for the slot's
// previous launch if it is still in flight and growing it if it is too small.
static int copy_slot(pkv_pool* p, int64_t n, pkv_pool::CopySlot** out) {
    auto& c = p->copy_ring[p->copy_next];
    if (!c.ev) {
        hipError_t e = hipEventCreateWithFlags(&c.ev, hipEventDisableTiming);
        if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags (block-move staging)");
    }
    if (c.pending) {
        hipError_t e = hipEventSynchronize(c.ev);
        if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize (block-move staging)");
        c.pending = false;
    }
    if (c.cap < n) {
        if (c.pairs) (void)hipHostFree(c.pairs);
        c.pairs = nullptr;
        c.cap = 0;
        const int64_t cap = std::max<int64_t>(n, 1024);
        hipError_t e = hipHostMalloc((void**)&c.pairs, sizeof(int32_t) * 2 * (size_t)cap,
                                     hipHostMallocCoherent | hipHostMallocMapped);
        if (e != hipSuccess) return fail_hip(e, "hipHostMalloc (block-move staging)");
        c.cap = cap;
    }
    *out = &c;
    return PKV_OK;
}

static int check_ids(const pkv_pool* p, int32_t n, const int32_t* seq_ids, const char* who) {
    if (n < 0 || (n > 0 && !seq_ids)) return fail(PKV_EINVAL, "%s: bad n or seq_ids", who);
    std::vector<uint8_t> mark(p->d.max_seqs, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        if (!p->valid_seq(s)) return fail(PKV_EINVAL, "%s: unknown sequence %d", who, s);
        if (mark[s]) return fail(PKV_EINVAL, "%s: sequence %d listed twice", who, s);
        mark[s] = 1;
    }
    return PKV_OK;
}

static int launch_moves(pkv_pool* p, pkv_pool::CopySlot* c, int64_t n, bool to_host, hipStream_t stream) {
    if (n == 0) return PKV_OK;
    pkv::TierCopyArgs a{};
    const void* dev_k = p->k_cache;
    const void* dev_v = p->v_cache;
    a.k_src = static_cast<const uint4*>(to_host ? dev_k : p->k_host_dev);
    a.v_src = static_cast<const uint4*>(to_host ? dev_v : p->v_host_dev);
    a.k_dst = static_cast<uint4*>(to_host ? p->k_host_dev : p->k_cache);
    a.v_dst = static_cast<uint4*>(to_host ? p->v_host_dev : p->v_cache);
    a.pairs = c->pairs;
    a.n = (int32_t)n;
    const bool kv8 = p->d.kv_dtype == PKV_FP8_E4M3;
    a.vec_per_block = (int32_t)((int64_t)p->d.num_kv_heads * p->d.block_size * p->d.head_dim * (kv8 ? 1 : 2) / 16);
    if (kv8) {
        a.ks_src = to_host ? p->k_scale : p->ks_host_dev;
        a.vs_src = to_host ? p->v_scale : p->vs_host_dev;
        a.ks_dst = to_host ? p->ks_host_dev : p->k_scale;
        a.vs_dst = to_host ? p->vs_host_dev : p->v_scale;
        a.scales_per_block = p->d.num_kv_heads;
    }
    hipError_t e = pkv::launch_tier_copy(a, stream);
    if (e != hipSuccess) return fail_hip(e, "block-move launch (pool state now ahead of the device)");
    e = hipEventRecord(c->ev, stream);
    if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
    c->pending = true;
    p->copy_next = (p->copy_next + 1) % kCopyRing;
    return PKV_OK;
}

int kv_seq_offload(pkv_pool* p, int32_t n, const int32_t* seq_ids, int32_t gpu_window, pkv_stream_t stream) {
    if (!p) return fail(PKV_EINVAL, "kv_seq_offload: null pool");
    if (!p->num_host) return fail(PKV_EINVAL, "kv_seq_offload: the pool has no host tier");
    if (gpu_window < 1) return fail(PKV_EINVAL, "kv_seq_offload: gpu_window %d (must be >= 1)", gpu_window);
    if (!p->k_cache || !p->v_cache) return fail(PKV_EINVAL, "kv_seq_offload: the pool has no device caches");
    if (p->d.kv_dtype == PKV_FP8_E4M3 && !p->k_scale)
        return fail(PKV_EINVAL, "kv_seq_offload: 8-bit pool without scales (kv_block_pool_set_fp8_scales)");
    int rc = check_ids(p, n, seq_ids, "kv_seq_offload");
    if (rc) return rc;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        const auto& b = p->blocks[seq_ids[i]];
        const int64_t cold = (int64_t)b.size() > gpu_window ? (int64_t)b.size() - gpu_window : 0;
        for (int64_t j = 0; j < cold; ++j) need += is_host(b[j]) ? 0 : 1;
    }
    if (need > (int64_t)p->host_stack.size())
        return fail(PKV_ENOMEM, "kv_seq_offload: need %lld host blocks, %zu free", (long long)need, p->host_stack.size());
    pkv_pool::CopySlot* c = nullptr;
    if (need) {
        rc = copy_slot(p, need, &c);
        if (rc) return rc;
    }
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        auto& b = p->blocks[s];
        const int64_t cold = (int64_t)b.size() > gpu_window ? (int64_t)b.size() - gpu_window : 0;
        for (int64_t j = 0; j < cold; ++j) {
            const int32_t g = b[j];
            if (is_host(g)) continue;
            const int32_t h = p->host_stack.back();
            p->host_stack.pop_back();
            p->host_ref[h] = 1;
            c->pairs[2 * k] = g;
            c->pairs[2 * k + 1] = h;
            ++k;
            b[j] = host_entry(h);
            ++p->nhost[s];
            p->unref(g);
        }
    }
    return launch_moves(p, c, k, true, (hipStream_t)stream);
}

int kv_seq_restore(pkv_pool* p, int32_t n, const int32_t* seq_ids, pkv_stream_t stream) {
    if (!p) return fail(PKV_EINVAL, "kv_seq_restore: null pool");
    if (!p->num_host) return fail(PKV_EINVAL, "kv_seq_restore: the pool has no host tier");
    if (!p->k_cache || !p->v_cache) return fail(PKV_EINVAL, "kv_seq_restore: the pool has no device caches");
    if (p->d.kv_dtype == PKV_FP8_E4M3 && !p->k_scale)
        return fail(PKV_EINVAL, "kv_seq_restore: 8-bit pool without scales (kv_block_pool_set_fp8_scales)");
    int rc = check_ids(p, n, seq_ids, "kv_seq_restore");
    if (rc) return rc;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) need += p->nhost[seq_ids[i]];
    if (need > p->num_free)
        return fail(PKV_ENOMEM, "kv_seq_restore: need %lld blocks, %d free", (long long)need, p->num_free);
    pkv_pool::CopySlot* c = nullptr;
    if (need) {
        rc = copy_slot(p, need, &c);
        if (rc) return rc;
    }
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        if (!p->nhost[s]) continue;
        for (auto& e : p->blocks[s]) {
            if (!is_host(e)) continue;
            const int32_t g = p->pop_free();
            p->ref[g] = 1;
            c->pairs[2 * k] = host_id(e);
            c->pairs[2 * k + 1] = g;
            ++k;
            p->unref(e);
            e = g;
        }
        p->nhost[s] = 0;
    }
    return launch_moves(p, c, k, false, (hipStream_t)stream);
}

int kv_quantize_fp8(int32_t n, const int32_t* items, const void* src_k, const void* src_v, int32_t src_dtype,
                    void* dst_k, void* dst_v, float* k_scale, float* v_scale, int32_t num_kv_heads,
                    int32_t block_size, int32_t head_dim, pkv_stream_t stream) {
    if (n < 0) return fail(PKV_EINVAL, "kv_quantize_fp8: n = %d", n);
    if (n == 0) return PKV_OK;
    if (!items || !src_k || !src_v || !dst_k || !dst_v || !k_scale || !v_scale)
        return fail(PKV_EINVAL, "kv_quantize_fp8: null pointer");
    if (src_dtype != PKV_F16 && src_dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "kv_quantize_fp8: src_dtype %d", src_dtype);
    if (num_kv_heads < 1 || (block_size != 16 && block_size != 32) || (head_dim != 64 && head_dim != 128))
        return fail(PKV_EUNSUPPORTED, "kv_quantize_fp8: shape (Hkv %d, block %d, head_dim %d)", num_kv_heads, block_size,
                    head_dim);
    if (!aligned(items, 4) || !aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 8) || !aligned(dst_v, 8) ||
        !aligned(k_scale, 4) || !aligned(v_scale, 4))
        return fail(PKV_EINVAL, "kv_quantize_fp8: misaligned pointer");
    pkv::QuantArgs a{};
    a.src_k = src_k;
    a.src_v = src_v;
    a.dst_k = static_cast<uint8_t*>(dst_k);
    a.dst_v = static_cast<uint8_t*>(dst_v);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.items = items;
    a.n = n;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.head_dim = head_dim;
    a.src_bf16 = src_dtype == PKV_BF16;
    hipError_t e = pkv::launch_quantize_fp8(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "kv_quantize_fp8 launch");
    return PKV_OK;
}

int kv_validate_tables(int32_t n_seqs, const int32_t* block_tables, int32_t table_stride, int32_t table_width,
                       const int32_t* context_lens, int32_t num_blocks, int32_t block_size) {
    if (n_seqs < 0 || (n_seqs > 0 && (!block_tables || !context_lens)) || block_size <= 0 ||
        table_width > table_stride)
        return fail(PKV_EINVAL, "kv_validate_tables: bad arguments");
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int32_t c = context_lens[s];
        if (c < 0) return fail(PKV_EINVAL, "kv_validate_tables: sequence %d has length %d", s, c);
        const int64_t nb = ceil_div(c, block_size);
        if (nb > table_width)
            return fail(PKV_EINVAL, "kv_validate_tables: sequence %d needs %lld blocks > width %d", s,
                        (long long)nb, table_width);
        for (int64_t j = 0; j < nb; ++j) {
            const int32_t b = block_tables[(int64_t)s * table_stride + j];
            if (b < 0 || b >= num_blocks)
                return fail(PKV_EINVAL, "kv_validate_tables: sequence %d entry %lld = %d out of [0, %d)", s,
                            (long long)j, b, num_blocks);
        }
    }
    return PKV_OK;
}

}  // extern "C"

// --------------------------------------------------------------------------
// Decode
// --------------------------------------------------------------------------

namespace {

constexpr int32_t kTile = pkv::kTileTokens;
constexpr int32_t kMinChunk = 4;            // must equal the kernel's balanced-split minimum

struct Plan {
    int32_t part_size = 0;                  // 0 = balanced split
    int32_t fixed_chunk = 0;                // part_size / 16
    int32_t max_seg = 0;                    // upper bound of segments per (sequence, kv head)
    int32_t seg_rows = 0;                   // workspace rows (after size_workspace)
    int32_t num_waves = 0;                  // resolved grid size (0 until resolved)
    int32_t group_pad = 0;
    int32_t heads_per_wave = 1;             // kv heads one wave takes per tile (2: 8-bit K/V, even Hkv)
    pkv::KvKind kind = pkv::KvKind::F16;
    int32_t out_kind = pkv::kOutF32;
    size_t hdr_bytes = 0, out_bytes = 0, ws_bytes = 0;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

int resolve(const pkv_attn_desc* d, Plan* pl) {
    if (!d) return fail(PKV_EINVAL, "null descriptor");
    if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_context_len < 0 || d->num_waves < 0)
        return fail(PKV_EINVAL, "descriptor: bad sizes");
    if (d->num_seqs > pkv::kMaxSeqs) return fail(PKV_EUNSUPPORTED, "num_seqs %d > %d", d->num_seqs, pkv::kMaxSeqs);
    if (d->num_q_heads % d->num_kv_heads)
        return fail(PKV_EINVAL, "num_q_heads %d not a multiple of num_kv_heads %d", d->num_q_heads, d->num_kv_heads);
    const int G = d->num_q_heads / d->num_kv_heads;
    if (G > 8) return fail(PKV_EUNSUPPORTED, "q heads per kv head = %d (at most 8)", G);
    if (d->head_dim != 64 && d->head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (64 or 128)", d->head_dim);
    if (d->block_size != 16 && d->block_size != 32)
        return fail(PKV_EUNSUPPORTED, "block_size %d (16 or 32)", d->block_size);
    if (d->kv_dtype == PKV_FP8_E4M3) {
        if (d->q_dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "8-bit K/V needs a bf16 query");
    } else {
        if (d->kv_dtype != PKV_F16 && d->kv_dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "kv_dtype %d", d->kv_dtype);
        if (d->q_dtype != d->kv_dtype) return fail(PKV_EUNSUPPORTED, "q_dtype must equal kv_dtype");
    }
    if (d->out_dtype == PKV_F32)
        pl->out_kind = pkv::kOutF32;
    else if (d->out_dtype == d->q_dtype)
        pl->out_kind = d->q_dtype == PKV_BF16 ? pkv::kOutBF16 : pkv::kOutF16;
    else
        return fail(PKV_EUNSUPPORTED, "out_dtype must be PKV_F32 or equal q_dtype");
    if (d->num_blocks < 0) return fail(PKV_EINVAL, "num_blocks %d", d->num_blocks);
    const int64_t need_w = ceil_div(d->max_context_len, d->block_size);
    if (d->table_stride < need_w)
        return fail(PKV_EINVAL, "table_stride %d < ceil(max_context_len / block_size) = %lld", d->table_stride,
                    (long long)need_w);
    const int32_t P = d->partition_size;
    if (P < 0 || (P > 0 && P % d->block_size))
        return fail(PKV_EINVAL, "partition_size %d must be 0 or a multiple of block_size %d", P, d->block_size);
    pl->part_size = P;
    pl->fixed_chunk = P / kTile;
    const int64_t max_tiles = ceil_div(d->max_context_len, kTile);
    if (P > 0) {
        pl->max_seg = (int32_t)std::max<int64_t>(1, ceil_div(d->max_context_len, P));
    } else {
        pl->max_seg = (int32_t)(ceil_div(max_tiles, kMinChunk) + 1);
    }
    // Flattened tile indices are int32 on the device.
    const int64_t per_seq = P > 0 ? (int64_t)pl->max_seg * pl->fixed_chunk : max_tiles;
    if ((int64_t)d->num_seqs * d->num_kv_heads * per_seq >= (int64_t)1 << 30)
        return fail(PKV_EUNSUPPORTED, "too many tiles in one call (num_seqs x kv heads x tiles >= 2^30)");
    // 8-bit K/V with an even kv head count: a wave takes two adjacent kv heads
    // of each tile (4 KiB contiguous per tile at D = 128 instead of 2 KiB).
    const bool pair = d->kv_dtype == PKV_FP8_E4M3 && d->num_kv_heads % 2 == 0;
    pl->heads_per_wave = pair ? 2 : 1;
    const int cols = G * pl->heads_per_wave;  // MFMA B-operand columns in use
    pl->group_pad = cols <= 1 ? 1 : cols <= 2 ? 2 : cols <= 4 ? 4 : cols <= 8 ? 8 : 16;
    pl->kind = d->kv_dtype == PKV_FP8_E4M3 ? (pair ? pkv::KvKind::FP8_BF16Q_PAIR : pkv::KvKind::FP8_BF16Q)
             : d->kv_dtype == PKV_BF16    ? pkv::KvKind::BF16
                                          : pkv::KvKind::F16;
    return PKV_OK;
}

// Workspace layout for a resolved split (num_waves known): a segment k of
// the pair p = (sequence, head group) is written to row (its chunk index) + p.
// Balanced mode has at most num_waves chunks (C >= ceil(T / num_waves)),
// fixed mode at most max_seg per pair; so rows = that bound + pairs.
int size_workspace(const pkv_attn_desc* d, Plan* pl) {
    const int64_t pairs = (int64_t)d->num_seqs * (d->num_kv_heads / pl->heads_per_wave);
    const int64_t chunks = pl->fixed_chunk > 0 ? pairs * pl->max_seg : (int64_t)pl->num_waves;
    const int64_t rows = std::max<int64_t>(chunks + pairs, 1);
    if (rows >= ((int64_t)1 << 31)) return fail(PKV_EUNSUPPORTED, "workspace rows %lld exceed int32", (long long)rows);
    const int64_t cols = (int64_t)(d->num_q_heads / d->num_kv_heads) * pl->heads_per_wave;   // q heads per row
    pl->seg_rows = (int32_t)rows;
    pl->hdr_bytes = up256(sizeof(int32_t) * (3 + (size_t)d->num_seqs));
    pl->out_bytes = up256((size_t)rows * cols * d->head_dim * sizeof(float));
    pl->ws_bytes = pl->hdr_bytes + pl->out_bytes + up256((size_t)rows * cols * sizeof(float));
    return PKV_OK;
}

// Waves in the grid: the descriptor's value (rounded up to whole workgroups),
// else every wave that fits the current device at once.  A fixed split never
// gets more waves than it has chunks.
int resolve_waves(const pkv_attn_desc* d, Plan* pl) {
    int64_t nw = d->num_waves;
    if (nw == 0) {
        // Occupancy and CU count per (instance, device), looked up once.  The
        // values are properties of the device and the code object, so threads
        // that race here store the same numbers; the entries are atomics so
        // that concurrent calls (on distinct pools or workspaces) are safe.
        static std::atomic<int> cache[2][2][5][4][64];   // [D][bs][gp][kv kind][device] -> waves per CU
        static std::atomic<int> cus[64];
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
        if (dev < 0 || dev >= 64) return fail(PKV_EUNSUPPORTED, "device index %d", dev);
        const int di = d->head_dim == 128 ? 1 : 0, bi = d->block_size == 32 ? 1 : 0;
        const int gi = pl->group_pad == 1 ? 0 : pl->group_pad == 2 ? 1 : pl->group_pad == 4 ? 2
                     : pl->group_pad == 8 ? 3 : 4;
        std::atomic<int>& slot = cache[di][bi][gi][(int)pl->kind][dev];
        int wpc = slot.load(std::memory_order_relaxed);
        if (wpc == 0) {
            e = pkv::split_waves_per_cu(d->head_dim, d->block_size, pl->group_pad, pl->kind, &wpc);
            if (e != hipSuccess) return fail_hip(e, "occupancy query");
            slot.store(wpc, std::memory_order_relaxed);
        }
        int ncu = cus[dev].load(std::memory_order_relaxed);
        if (ncu == 0) {
            e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute");
            cus[dev].store(ncu, std::memory_order_relaxed);
        }
        nw = (int64_t)std::max(wpc, 4) * ncu;
    }
    if (pl->fixed_chunk > 0) {
        const int64_t chunks = (int64_t)d->num_seqs * (d->num_kv_heads / pl->heads_per_wave) * pl->max_seg;
        nw = std::min(nw, std::max<int64_t>(chunks, 1));
    }
    nw = std::min<int64_t>((nw + 3) / 4 * 4, (int64_t)1 << 28);
    pl->num_waves = (int32_t)nw;
    return PKV_OK;
}

// The split the kernel makes, replayed on the host for given lengths: calls
// f(seq, kv_head, slot, tok_lo, tok_hi) for every segment in order.  The list
// holds (sequence, head group, tile), a group being the heads_per_wave kv heads
// one wave takes together; every head of a group starts at the group's tile.
template <class F>
int enumerate_segments(const pkv_attn_desc* d, const Plan& pl, const int32_t* ctx_host, F&& f) {
    const int B = d->num_seqs, Hkv = d->num_kv_heads, hw = pl.heads_per_wave;
    std::vector<int64_t> pre(B + 1, 0);
    std::vector<int32_t> nt(B), pt(B);
    for (int s = 0; s < B; ++s) {
        const int32_t n = std::min(std::max(ctx_host[s], 0), d->max_context_len);
        nt[s] = (int32_t)ceil_div(n, kTile);
        pt[s] = pl.fixed_chunk > 0 ? (int32_t)(ceil_div(nt[s], pl.fixed_chunk) * pl.fixed_chunk) : nt[s];
        pre[s + 1] = pre[s] + (int64_t)pt[s] * (Hkv / hw);
    }
    const int64_t T = pre[B];
    const int64_t C = pl.fixed_chunk > 0 ? pl.fixed_chunk : std::max<int64_t>(kMinChunk, ceil_div(T, pl.num_waves));
    for (int s = 0; s < B; ++s) {
        for (int g = 0; g < Hkv && nt[s] > 0; ++g) {
            const int64_t first = pre[s] + (int64_t)(g / hw) * pt[s];
            const int64_t c0 = first / C, c1 = (first + nt[s] - 1) / C;
            for (int64_t ch = c0; ch <= c1; ++ch) {
                const int64_t j0 = std::max<int64_t>(ch * C - first, 0);
                const int64_t j1 = std::min<int64_t>((ch + 1) * C - first, nt[s]);
                const int32_t tlo = (int32_t)(j0 * kTile);
                const int32_t thi = (int32_t)std::min<int64_t>(j1 * kTile, std::min(ctx_host[s], d->max_context_len));
                f(s, g, (int32_t)(ch - c0), tlo, thi);
            }
        }
    }
    return PKV_OK;
}

// Decode pointers.  Outputs: the kernels store rows of fp32 out with 16-byte
// vector stores and 16-bit out with 4-byte stores, so out must be 16-byte
// (fp32) or 8-byte (16-bit) aligned; lse (nullable) 4-byte aligned.
int check_ptrs(const Plan& pl, const void* q, const void* k, const void* v, const int32_t* tables,
               const int32_t* lens, const void* out, const float* lse, const void* ws, size_t ws_bytes,
               bool need_inputs) {
    if (need_inputs) {
        if (!q || !k || !v || !tables || !lens) return fail(PKV_EINVAL, "null input pointer");
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(tables, 4) || !aligned(lens, 4))
            return fail(PKV_EINVAL, "q, k_cache, v_cache must be 16-byte aligned");
    }
    if (!out) return fail(PKV_EINVAL, "null out");
    if (!aligned(out, pl.out_kind == pkv::kOutF32 ? 16 : 8))
        return fail(PKV_EINVAL, "out must be %d-byte aligned", pl.out_kind == pkv::kOutF32 ? 16 : 8);
    if (lse && !aligned(lse, 4)) return fail(PKV_EINVAL, "lse must be 4-byte aligned");
    if (!ws || ws_bytes < pl.ws_bytes)
        return fail(PKV_EWORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, pl.ws_bytes);
    if (!aligned(ws, 256)) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
    return PKV_OK;
}

}  // namespace

extern "C" {

int32_t paged_attn_partition_size(const pkv_attn_desc* d) {
    Plan pl;
    int rc = resolve(d, &pl);
    return rc ? rc : pl.part_size;
}

int32_t paged_attn_grid_waves(const pkv_attn_desc* d) {
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    rc = resolve_waves(d, &pl);
    return rc ? rc : pl.num_waves;
}

int32_t paged_attn_decode_launches(const pkv_attn_desc* d) {
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    if (pl.fixed_chunk == 0 && (rc = resolve_waves(d, &pl))) return rc;
    if ((rc = size_workspace(d, &pl))) return rc;
    return pl.max_seg <= 1 ? 1 : 2;
}

size_t paged_attn_workspace_bytes(const pkv_attn_desc* d) {
    Plan pl;
    if (resolve(d, &pl)) return 0;
    // Only the balanced split's size depends on the grid.
    if (pl.fixed_chunk == 0 && resolve_waves(d, &pl)) return 0;
    if (size_workspace(d, &pl)) return 0;
    return pl.ws_bytes;
}

// Kernel arguments of a split launch for a resolved, checked plan.
static pkv::DecodeArgs decode_args(const pkv_attn_desc* d, const Plan& pl, const void* q, const void* k_cache,
                                   const void* v_cache, const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                                   float* lse, void* workspace) {
    char* ws = reinterpret_cast<char*>(workspace);
    pkv::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.lse = lse;
    a.ws_hdr = reinterpret_cast<int32_t*>(ws);
    a.ws_out = reinterpret_cast<float*>(ws + pl.hdr_bytes);
    a.ws_lse = reinterpret_cast<float*>(ws + pl.hdr_bytes + pl.out_bytes);
    a.scale = scale;
    a.num_seqs = d->num_seqs;
    a.num_q_heads = d->num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.table_stride = d->table_stride;
    a.fixed_chunk = pl.fixed_chunk;
    a.num_waves = pl.num_waves;
    a.seg_rows = pl.seg_rows;
    a.max_context_len = d->max_context_len;
    a.out_dtype = pl.out_kind;
    a.heads_per_wave = pl.heads_per_wave;
    a.pair_halves = pl.fixed_chunk >= 2 ? 1 : 0;   // fixed partitions: two waves per chunk
    return a;
}

static int partials_impl(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, pkv_stream_t stream, bool fp8_call, pkv_event_t start = nullptr,
                         pkv_event_t stop = nullptr) {
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    const bool kv8 = pl.kind == pkv::KvKind::FP8_BF16Q || pl.kind == pkv::KvKind::FP8_BF16Q_PAIR;
    if (kv8 != fp8_call)
        return fail(PKV_EINVAL, kv8 ? "kv_dtype PKV_FP8_E4M3 goes through the _fp8 entry points (they take the scales)"
                                    : "the _fp8 entry points need kv_dtype PKV_FP8_E4M3");
    if (kv8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
        return fail(PKV_EINVAL, "8-bit K/V: null or misaligned k_scale / v_scale");
    if (d->num_seqs == 0) return PKV_OK;
    rc = resolve_waves(d, &pl);
    if (rc) return rc;
    rc = size_workspace(d, &pl);
    if (rc) return rc;
    rc = check_ptrs(pl, q, k_cache, v_cache, block_tables, context_lens, out, lse, workspace, workspace_bytes, true);
    if (rc) return rc;
    const pkv::DecodeArgs a = decode_args(d, pl, q, k_cache, v_cache, kv8 ? k_scale : nullptr, kv8 ? v_scale : nullptr,
                                          block_tables, context_lens, scale, out, lse, workspace);
    hipError_t e = pkv::launch_split(a, d->head_dim, d->block_size, pl.group_pad, pl.kind, (hipStream_t)stream,
                                     (hipEvent_t)start, (hipEvent_t)stop);
    if (e != hipSuccess) return fail_hip(e, "split kernel launch");
    return PKV_OK;
}

int paged_attn_decode_partials_timed(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                     const int32_t* context_lens, float scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, pkv_event_t start, pkv_event_t stop,
                                     pkv_stream_t stream) {
    if (!d) return fail(PKV_EINVAL, "null descriptor");
    if (!start || !stop) return fail(PKV_EINVAL, "paged_attn_decode_partials_timed: null start or stop event");
    return partials_impl(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, out, lse,
                         workspace, workspace_bytes, stream, d->kv_dtype == PKV_FP8_E4M3, start, stop);
}

int paged_attn_decode_partials(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
    return partials_impl(d, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, scale, out, lse,
                         workspace, workspace_bytes, stream, false);
}

int paged_attn_decode_partials_fp8(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                                   const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, pkv_stream_t stream) {
    return partials_impl(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, out, lse,
                         workspace, workspace_bytes, stream, true);
}

int paged_attn_merge(const pkv_attn_desc* d, const int32_t* context_lens, void* out, float* lse,
                     const void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    if (d->num_seqs == 0 || pl.max_seg <= 1) return PKV_OK;
    if (!context_lens || !aligned(context_lens, 4)) return fail(PKV_EINVAL, "null context_lens");
    rc = resolve_waves(d, &pl);
    if (rc) return rc;
    rc = size_workspace(d, &pl);
    if (rc) return rc;
    rc = check_ptrs(pl, nullptr, nullptr, nullptr, nullptr, nullptr, out, lse, workspace, workspace_bytes, false);
    if (rc) return rc;
    const char* ws = reinterpret_cast<const char*>(workspace);
    pkv::MergeArgs a{};
    a.context_lens = context_lens;
    a.ws_hdr = reinterpret_cast<const int32_t*>(ws);
    a.ws_out = reinterpret_cast<const float*>(ws + pl.hdr_bytes);
    a.ws_lse = reinterpret_cast<const float*>(ws + pl.hdr_bytes + pl.out_bytes);
    a.out = out;
    a.lse = lse;
    a.num_seqs = d->num_seqs;
    a.num_q_heads = d->num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.fixed_chunk = pl.fixed_chunk;
    a.max_seg = pl.max_seg;
    a.seg_rows = pl.seg_rows;
    a.max_context_len = d->max_context_len;
    a.out_dtype = pl.out_kind;
    a.heads_per_wave = pl.heads_per_wave;
    hipError_t e = pkv::launch_merge(a, d->head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "merge kernel launch");
    return PKV_OK;
}

int kv_append_decode(pkv_pool* p, int32_t n, const int32_t* seq_ids, const void* k_new, const void* v_new,
                     int32_t* block_tables, int32_t* context_lens, const pkv_attn_desc* d, const void* q, float scale,
                     void* out, float* lse, void* workspace, size_t workspace_bytes, pkv_event_t start,
                     pkv_event_t stop, pkv_stream_t stream) {
    if (!p || !d) return fail(PKV_EINVAL, "kv_append_decode: null pool or descriptor");
    if (p->d.kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_EUNSUPPORTED, "kv_append_decode: 8-bit pools append with kv_append and decode with "
                                      "paged_attn_decode_fp8");
    if (d->kv_dtype != p->d.kv_dtype || d->head_dim != p->d.head_dim || d->block_size != p->d.block_size ||
        d->num_kv_heads != p->d.num_kv_heads || d->table_stride != p->d.max_blocks_per_seq)
        return fail(PKV_EINVAL, "kv_append_decode: the descriptor's kv dtype, head_dim, block_size, num_kv_heads and "
                                "table_stride must be the pool's");
    if (n < 0 || n > p->d.max_seqs || (n > 0 && !seq_ids)) return fail(PKV_EINVAL, "kv_append_decode: bad n or seq_ids");
    if (n > 0 && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)))
        return fail(PKV_EINVAL, "kv_append_decode: k_new / v_new null or not 16-byte aligned");
    if ((start == nullptr) != (stop == nullptr))
        return fail(PKV_EINVAL, "kv_append_decode: give both timing events or neither");
    if (d->num_seqs > p->d.max_seqs) return fail(PKV_EINVAL, "kv_append_decode: num_seqs beyond the pool's rows");
    std::vector<uint8_t> listed(p->d.max_seqs, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        if (!p->valid_seq(s)) return fail(PKV_EINVAL, "kv_append_decode: unknown sequence %d", s);
        // The append's own refusals (kv_reserve), checked here too so that they
        // come before anything is set up.
        if (listed[s]) return fail(PKV_EINVAL, "kv_append_decode: sequence %d listed twice", s);
        listed[s] = 1;
        if (p->nhost[s])
            return fail(PKV_EINVAL, "kv_append_decode: sequence %d has blocks in the host tier (restore it first)", s);
        if (p->len[s] % p->d.block_size == 0 && p->len[s] / p->d.block_size >= p->d.max_blocks_per_seq)
            return fail(PKV_EINVAL, "kv_append_decode: sequence %d is full (%d blocks)", s, p->d.max_blocks_per_seq);
        if (s >= d->num_seqs)
            return fail(PKV_EINVAL, "kv_append_decode: sequence %d is not among the %d decoded rows", s, d->num_seqs);
        if ((int64_t)p->len[s] + 1 > d->max_context_len)
            return fail(PKV_EINVAL, "kv_append_decode: sequence %d would exceed max_context_len %d", s,
                        d->max_context_len);
    }
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    if (d->num_seqs == 0) return PKV_OK;
    rc = resolve_waves(d, &pl);
    if (rc) return rc;
    rc = size_workspace(d, &pl);
    if (rc) return rc;
    rc = check_ptrs(pl, q, p->k_cache, p->v_cache, block_tables, context_lens, out, lse, workspace, workspace_bytes,
                    true);
    if (rc) return rc;
    if (n > pkv::kFuseItems || d->max_context_len > pkv::kFuseMaxLen) {
        // More items than the kernel arguments carry, or lengths beyond what an
        // item holds: the same work as two calls.
        rc = kv_append(p, n, seq_ids, k_new, v_new, block_tables, context_lens, stream);
        if (rc) return rc;
        rc = start ? paged_attn_decode_partials_timed(d, q, p->k_cache, p->v_cache, nullptr, nullptr, block_tables,
                                                      context_lens, scale, out, lse, workspace, workspace_bytes, start,
                                                      stop, stream)
                   : paged_attn_decode_partials(d, q, p->k_cache, p->v_cache, block_tables, context_lens, scale, out,
                                                lse, workspace, workspace_bytes, stream);
        if (rc) return rc;
        return paged_attn_merge(d, context_lens, out, lse, workspace, workspace_bytes, stream);
    }
    rc = ensure_ring(p);
    if (rc) return rc;
    if (p->stage.size() < (size_t)n) p->stage.resize((size_t)p->d.max_seqs);
    bool any_copy = false;
    rc = reserve_impl(p, n, seq_ids, p->stage.data(), &any_copy);
    if (rc) return rc;
    pkv::AppendArgs aa{};
    aa.k_cache = p->k_cache;
    aa.v_cache = p->v_cache;
    aa.block_tables = block_tables;
    aa.context_lens = context_lens;
    aa.n = n;
    aa.num_kv_heads = p->d.num_kv_heads;
    aa.head_dim = p->d.head_dim;
    aa.block_size = p->d.block_size;
    aa.table_stride = p->d.max_blocks_per_seq;
    if (any_copy) {
        // A copied tail must hold its rows before the decode reads the copy:
        // the copy-on-write phase runs first, from the pinned ring.
        auto& slot = p->ring[p->next];
        if (slot.pending) {
            hipError_t e = hipEventSynchronize(slot.ev);
            if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize (append staging; pool state now ahead of the device)");
            slot.pending = false;
        }
        std::memcpy(slot.host, p->stage.data(), sizeof(pkv::AppendItem) * (size_t)n);
        aa.items = slot.host;
        hipError_t e = pkv::launch_append_cow(aa, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "copy-on-write launch (pool state now ahead of the device)");
        e = hipEventRecord(slot.ev, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
        slot.pending = true;
        p->next = (p->next + 1) % kRing;
    }
    pkv::FuseItems fi;
    for (int32_t i = 0; i < n; ++i) {
        const pkv::AppendItem& it = p->stage[(size_t)i];
        fi.it[i] = {(uint32_t)it.seq | ((uint32_t)it.new_len << 12), it.new_block};
    }
    pkv::DecodeArgs a = decode_args(d, pl, q, p->k_cache, p->v_cache, nullptr, nullptr, block_tables, context_lens,
                                    scale, out, lse, workspace);
    a.k_new = k_new;
    a.v_new = v_new;
    a.tables_out = block_tables;
    a.lens_out = context_lens;
    a.n_items = n;
    hipError_t e = pkv::launch_split_append(a, fi, d->head_dim, d->block_size, pl.group_pad, pl.kind,
                                            (hipStream_t)stream, (hipEvent_t)start, (hipEvent_t)stop);
    if (e != hipSuccess) return fail_hip(e, "fused append + split launch (pool state now ahead of the device)");
    return paged_attn_merge(d, context_lens, out, lse, workspace, workspace_bytes, stream);
}

int paged_attn_decode(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
    int rc = paged_attn_decode_partials(d, q, k_cache, v_cache, block_tables, context_lens, scale, out, lse,
                                        workspace, workspace_bytes, stream);
    if (rc) return rc;
    return paged_attn_merge(d, context_lens, out, lse, workspace, workspace_bytes, stream);
}

int paged_attn_decode_noalloc(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                              float* lse, pkv_stream_t stream) {
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    if (d->num_seqs == 0) return PKV_OK;
    rc = resolve_waves(d, &pl);
    if (rc) return rc;
    rc = size_workspace(d, &pl);
    if (rc) return rc;
    if (pl.ws_bytes > pkv::kScratchBytes)
        return fail(PKV_EWORKSPACE,
                    "paged_attn_decode_noalloc: this split needs %zu bytes of workspace, the static scratch holds "
                    "%zu (use paged_attn_decode with a caller workspace)",
                    pl.ws_bytes, pkv::kScratchBytes);
    void* ws = nullptr;
    size_t cap = 0;
    hipError_t e = pkv::static_scratch(&ws, &cap);
    if (e != hipSuccess) return fail_hip(e, "paged_attn_decode_noalloc: static scratch address");
    return paged_attn_decode(d, q, k_cache, v_cache, block_tables, context_lens, scale, out, lse, ws, cap, stream);
}

int paged_attn_decode_fp8(const pkv_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, pkv_stream_t stream) {
    int rc = paged_attn_decode_partials_fp8(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                                            scale, out, lse, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return paged_attn_merge(d, context_lens, out, lse, workspace, workspace_bytes, stream);
}

int paged_attn_prefill(const pkv_prefill_desc* d, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_seqlens_q,
                       float scale, void* out, float* lse, pkv_stream_t stream) {
    if (!d) return fail(PKV_EINVAL, "paged_attn_prefill: null descriptor");
    if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->total_q < 0 || d->max_context_len < 0)
        return fail(PKV_EINVAL, "paged_attn_prefill: bad sizes");
    if (d->num_seqs > pkv::kPrefillMaxSeqs)
        return fail(PKV_EUNSUPPORTED, "paged_attn_prefill: num_seqs %d > %d", d->num_seqs, pkv::kPrefillMaxSeqs);
    if (d->num_q_heads % d->num_kv_heads)
        return fail(PKV_EINVAL, "num_q_heads %d not a multiple of num_kv_heads %d", d->num_q_heads, d->num_kv_heads);
    if (d->head_dim != 64 && d->head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d (64 or 128)", d->head_dim);
    if (d->block_size != 16 && d->block_size != 32)
        return fail(PKV_EUNSUPPORTED, "block_size %d (16 or 32)", d->block_size);
    if ((d->q_dtype != PKV_F16 && d->q_dtype != PKV_BF16) || d->kv_dtype != d->q_dtype)
        return fail(PKV_EUNSUPPORTED, "paged_attn_prefill: q_dtype %d / kv_dtype %d (both PKV_F16 or both PKV_BF16)",
                    d->q_dtype, d->kv_dtype);
    int out_kind;
    if (d->out_dtype == PKV_F32)
        out_kind = pkv::kOutF32;
    else if (d->out_dtype == d->q_dtype)
        out_kind = d->q_dtype == PKV_BF16 ? pkv::kOutBF16 : pkv::kOutF16;
    else
        return fail(PKV_EUNSUPPORTED, "out_dtype must be PKV_F32 or equal q_dtype");
    const int64_t need_w = ceil_div(d->max_context_len, d->block_size);
    if (d->table_stride < need_w)
        return fail(PKV_EINVAL, "table_stride %d < ceil(max_context_len / block_size) = %lld", d->table_stride,
                    (long long)need_w);
    if (d->num_seqs == 0 || d->total_q == 0) return PKV_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !cu_seqlens_q || !out)
        return fail(PKV_EINVAL, "paged_attn_prefill: null pointer");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
        !aligned(context_lens, 4) || !aligned(cu_seqlens_q, 4) || !aligned(out, out_kind == pkv::kOutF32 ? 16 : 8) ||
        (lse && !aligned(lse, 4)))
        return fail(PKV_EINVAL, "paged_attn_prefill: misaligned pointer (q, caches 16 bytes; out 16 (fp32) or 8)");
    // A workgroup takes Qt = 256 / G chunk queries of one kv head's G q heads.
    // Query tiles: sum over s of ceil(m_s / Qt) <= total_q / Qt + num_seqs.
    const int32_t qtile = pkv::prefill_query_tile(d->num_q_heads / d->num_kv_heads);
    if (qtile == 0)
        return fail(PKV_EUNSUPPORTED, "paged_attn_prefill: group of %d q heads per kv head (at most %d)",
                    d->num_q_heads / d->num_kv_heads, pkv::kPrefillRows);
    const int64_t tiles = ceil_div(d->total_q, qtile) + d->num_seqs;
    if (tiles * d->num_kv_heads > 0x7FFFFFFF) return fail(PKV_EUNSUPPORTED, "paged_attn_prefill: grid too large");
    pkv::PrefillArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.cu_q = cu_seqlens_q;
    a.out = out;
    a.lse = lse;
    a.scale = scale;
    a.num_seqs = d->num_seqs;
    a.num_q_heads = d->num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.table_stride = d->table_stride;
    a.total_q = d->total_q;
    a.max_context_len = d->max_context_len;
    a.out_dtype = out_kind;
    a.query_tile = qtile;
    a.grid_tiles = (int32_t)tiles;
    hipError_t e = pkv::launch_prefill(a, d->head_dim, d->block_size, d->q_dtype == PKV_BF16, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "prefill kernel launch");
    return PKV_OK;
}

int pkv_read_probe(const void* buf, size_t bytes, int32_t workgroups, int32_t nontemporal, uint32_t* sink,
                   pkv_stream_t stream) {
    const size_t slice = (size_t)pkv::read_probe_slice_bytes();
    if (!buf || !aligned(buf, 16) || !sink || !aligned(sink, 4))
        return fail(PKV_EINVAL, "pkv_read_probe: buf (16-byte aligned) and sink (4-byte aligned) are required");
    if (bytes < slice) return fail(PKV_EINVAL, "pkv_read_probe: %zu bytes, at least %zu needed", bytes, slice);
    if (workgroups < 1 || workgroups > (1 << 20)) return fail(PKV_EINVAL, "pkv_read_probe: workgroups %d", workgroups);
    hipError_t e = pkv::launch_read_probe(buf, (int64_t)bytes, workgroups, nontemporal != 0, sink, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "read probe launch");
    return PKV_OK;
}

int paged_attn_plan(const pkv_attn_desc* d, const int32_t* context_lens_host, int32_t* items_out, int64_t cap,
                    int64_t* n_out) {
    Plan pl;
    int rc = resolve(d, &pl);
    if (rc) return rc;
    if (!n_out || (d->num_seqs > 0 && !context_lens_host)) return fail(PKV_EINVAL, "paged_attn_plan: null argument");
    for (int32_t s = 0; s < d->num_seqs; ++s)
        if (context_lens_host[s] < 0 || context_lens_host[s] > d->max_context_len)
            return fail(PKV_EINVAL, "paged_attn_plan: context_lens[%d] = %d outside [0, %d]", s, context_lens_host[s],
                        d->max_context_len);
    rc = resolve_waves(d, &pl);
    if (rc) return rc;
    int64_t n = 0;
    enumerate_segments(d, pl, context_lens_host, [&](int32_t s, int32_t g, int32_t k, int32_t lo, int32_t hi) {
        if (items_out && n < cap) {
            int32_t* r = items_out + n * 5;
            r[0] = s;
            r[1] = g;
            r[2] = k;
            r[3] = lo;
            r[4] = hi;
        }
        ++n;
    });
    *n_out = n;
    return PKV_OK;
}

}  // extern "C"
