// pkv_decode.hip -- paged-KV attention decode kernels for gfx950 (CDNA4).
//
// What is computed: for each sequence s and q head h, attention of the one
// query row q[s][h] over the sequence's whole cached context, whose K/V rows
// sit in fixed-size physical blocks found through the per-sequence block
// table and addressed indirectly inside the kernel ("架构解构：推理引擎的四层抽象",
// PagedAttention section).  Scores are q.k scaled by 1/sqrt(d), softmax is the
// stable form ("从零开始构建LLM推理引擎：模型执行器深度解析", 3.1), all sums are fp32
// ("LLM+Agent 全栈推理底座", 4.1), and the softmax runs online over tiles so no
// score ever reaches HBM ("架构解构：推理引擎的四层抽象", FlashAttention
// integration section).
//
// Work decomposition.  A persistent grid of 256-thread workgroups (4 wave64),
// as many as fit the device at once.  Every (sequence s, kv head g, 16-token
// tile j) is one entry of a flattened, sequence-major list; the list is cut
// into chunks of C tiles and wave w of the NW waves takes chunks w, w + NW,
// ...  With C = ceil(T / NW) (balanced mode) every wave gets the same number
// of tiles whatever the context lengths; with C = P / 16 and each (s, g)
// padded to whole chunks (fixed mode) a chunk is one partition of P tokens.
// A 16-token tile of one (block, kv head) is 16*D*2 bytes contiguous and
// never crosses a block (block_size is 16 or 32).
//
// QK on the matrix core.  The G q heads of the kv group form the B operand of
// v_mfma_f32_16x16x32 (32 d x 16 heads, heads >= G zero) and stay in
// registers, so every K row is read once per kv head, not once per q head.
// The A operand is 16 K rows x 32 d: lane l loads 16 bytes of one row, so one
// wave load instruction reads 64 contiguous bytes of each of the 16 rows.
// D/32 MFMAs give the 16x16 score tile.  A-operand row m holds token
// (m >> 2) + 4 (m & 3) of the tile, so lane l of the result holds the scores
// of tokens l/16 + 4i (i = 0..3) for head l%16.
// Softmax: one running reference max per head; it moves only when a tile's
// max exceeds it by more than TAU (log2 units), so the accumulator rescale is
// a rare event and every weight stays <= 2^TAU.  Rows past the context get
// weight 0 by selection and their V is zeroed before use, so stale or NaN
// data in unused slots never reaches a sum.
// PV on the matrix core as well, with no data movement between the two: a V
// row is loaded by 16 lanes (D/16 values each, so a wave load instruction
// reads 4 whole rows, contiguous), and lane l's four loads of a tile hold
// tokens l/16 + 4i for d in [D/16 (l%16), D/16 (l%16 + 1)) -- for each of its
// D/16 values e, exactly the A operand of v_mfma_f32_16x16x16 (16 d rows x 16
// tokens), while the score layout above is exactly its B operand (16 tokens x
// 16 heads).  The weights go in as two 16-bit halves (hi + lo, about 16
// significant bits), so PV is 2 D/16 small MFMAs per tile instead of a long
// run of vector FMAs.
// End of a segment (the part of a chunk inside one (s, g)): lane l holds
// D/4 consecutive output values of head l%16 and the result is either the
// final output (the segment covers all of (s, g)) or a normalised partial
// plus its log2-domain lse in the workspace for the merge kernel.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"



namespace pkv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;
constexpr float kTau = 8.0f;           // lazy-rescale threshold (log2 units)
constexpr int kMinChunk = 4;           // balanced split: at least 4 tiles (64 tokens) per chunk
constexpr int kMergeWidePairs = 1024;  // merge: a workgroup per pair up to this many pairs...
constexpr int kMergeWideSegments = 32; // ...or for fixed partitions with more slots than this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <bool BF16> struct MfmaType { using vec = f16x8; };
template <> struct MfmaType<true> { using vec = bf16x8; };

// C += A(16x32) * B(32x16), fp32 accumulate (v_mfma_f32_16x16x32_{bf16,f16}).
template <bool BF16>
__device__ __forceinline__ floatx4 mfma_16x16x32(typename MfmaType<BF16>::vec a, typename MfmaType<BF16>::vec b,
                                                 floatx4 c) {
    if constexpr (BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Cross-row helpers (gfx950 v_permlane{16,32}_swap with both operands = x):
// permlane16_swap yields x[l & ~16] and x[l | 16], permlane32_swap yields
// x[l % 32] and x[32 + l % 32]; combining the pair reduces across lanes
// l ^ 16 (resp. l ^ 32) with no LDS round trip.
__device__ __forceinline__ float xsum16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xmax16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float xmax32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
template <bool C, class T, class F> struct Pick { using type = T; };
template <class T, class F> struct Pick<false, T, F> { using type = F; };

typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two OCP E4M3 codes (bytes 0-1 of w, or bytes 2-3 with HI) -> one word of
// packed bf16, exact (v_cvt_scalef32_pk_bf16_fp8, scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Four OCP E4M3 codes (bytes of w, low byte first) -> two words of packed
// bf16 (codes 0-1, codes 2-3), exact: v_cvt_scalef32_pk_bf16_fp8 with scale 1
// (every E4M3 value has at most 4 significant bits; checked on all 256 codes).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// C += A(16x16) * B(16x16), fp32 accumulate (v_mfma_f32_16x16x16_{bf16,f16});
// a and b: four packed 16-bit values, the lane's k = 4 (l/16) .. 4 (l/16) + 3.
template <bool BF16>
__device__ __forceinline__ floatx4 mfma_16x16x16(uint2 a, uint2 b, floatx4 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Two floats -> their 16-bit roundings (hi, packed) and the roundings of what
// is left (lo, packed): x = hi + lo to within 2^-18 |x| (bf16) or 2^-22 |x|
// (f16, x in the normal range).
template <bool BF16>
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    if constexpr (BF16) {
        const bf16x2 h = {(__bf16)x0, (__bf16)x1};
        const bf16x2 l = {(__bf16)(x0 - (float)h.x), (__bf16)(x1 - (float)h.y)};
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, l);
    } else {
        const f16x2 h = {(_Float16)x0, (_Float16)x1};
        const f16x2 l = {(_Float16)(x0 - (float)h.x), (_Float16)(x1 - (float)h.y)};
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, l);
    }
}

// K/V tile loads.  Every K/V byte is read once per launch, so the loads are
// non-temporal: the lines are not kept in the caches for reuse, which on
// this access pattern (random 2-4 KiB pieces of the pool) measured about 10 %
// faster for the 16-bit kernel than plain loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_once16(const void* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}
// A lane's piece of one V row: NW 32-bit words.
template <int NW> struct VPiece { uint32_t w[NW]; };
template <int NW, bool ONCE>
__device__ __forceinline__ VPiece<NW> load_piece(const void* p) {
    VPiece<NW> v;
    if constexpr (NW == 4) {
        const uint4 t = ONCE ? load_once16(p) : *reinterpret_cast<const uint4*>(p);
        v.w[0] = t.x; v.w[1] = t.y; v.w[2] = t.z; v.w[3] = t.w;
    } else if constexpr (NW == 2) {
        const u32x2 t = ONCE ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                             : *reinterpret_cast<const u32x2*>(p);
        v.w[0] = t[0]; v.w[1] = t[1];
    } else {
        v.w[0] = ONCE ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p))
                      : *reinterpret_cast<const uint32_t*>(p);
    }
    return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))   // NaN stays NaN
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, int out_dtype) {
    if (out_dtype == kOutF32) {
        reinterpret_cast<float*>(out)[idx] = v;
    } else if (out_dtype == kOutBF16) {
        reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
    } else {
        reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
    }
}

// Workgroup id -> logical workgroup id.  The hardware hands workgroup i to
// XCD i % 8; this makes consecutive logical ids land on one XCD (and so share
// its L2).  Consecutive logical workgroups take consecutive chunks of the
// flattened tile list, so sequences next to each other in the batch (a
// shared-prefix group) are read through the same L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    const int per = n / kNumXcds;
    if (i < per * kNumXcds) return (i % kNumXcds) * per + i / kNumXcds;
    return i;
}

// Context length of sequence s as the kernels use it (clamped to
// [0, max_context_len]); tiles of one kv head of it (16 tokens each), and the
// same count padded to whole chunks when the chunk size is fixed.
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int s) {
    return min(max(a.context_lens[s], 0), a.max_context_len);
}
__device__ __forceinline__ int len_tiles(int n) { return (n + kTile - 1) / kTile; }
__device__ __forceinline__ int padded_tiles(int nt, int fixed_chunk) {
    return fixed_chunk > 0 ? (nt + fixed_chunk - 1) / fixed_chunk * fixed_chunk : nt;
}

// The split.  A wave takes HW kv heads of each tile: HW = 2 for 8-bit K/V
// with an even kv head count (the two heads' (block, kv head) pieces are
// adjacent, so a tile's K and V reads are 4 KiB contiguous at D = 128 instead
// of 2 KiB), else 1.  All (sequence s, head group q, tile j) are laid out in
// one list, sequence-major: the tiles of kv head g start at first(s, g) =
// pre[s] + (g / HW) * pt_s, pre[s] = (Hkv / HW) * sum_{s' < s} pt_s'.  With
// HW = 2 the B operand holds both heads' q groups (2G columns), the two K
// tiles go through it in two MFMA chains and each lane keeps the scores of
// its own column's head; PV runs one chain per head with the other head's
// columns' weights zero.  The list is cut into chunks of C tiles;
// wave w of the NW waves in the grid takes chunks w, w + NW, ...  Balanced
// mode (partition_size 0): pt_s = tiles of s, C = max(kMinChunk, ceil(T / NW))
// so every wave gets an equal share whatever the lengths.  Fixed mode:
// C = partition_size / 16 and pt_s is padded to a multiple of C, so a chunk
// is exactly one partition [pC*16, min((p+1)C*16, len)) of one (s, g).
// A chunk's part inside one (s, g) is a segment; it writes its normalised
// output and log2-domain lse to slot k = c - first(s, g) / C, or the final
// output directly when it covers all of (s, g).
// Waves per SIMD: the 16-bit instances take what the compiler gives (two
// fit, <= 256 registers); the 8-bit one-head instances are held to 168 so
// three fit, which measured about 5 % faster (half the bytes per tile, so
// more waves keep as many bytes in flight); the 8-bit two-head instances
// (a whole 4 KiB K or V tile per wave) run two per SIMD.
// FUSE: the same split with the append of the step's new tokens folded in
// (16-bit K/V, one kv head per wave; see paged_decode_append_split_kernel).
template <int D, int BS, int GP, bool BF16, bool KV8, int HW, bool FUSE>
__device__ __forceinline__ void split_body(const DecodeArgs& a, const FuseItem* fit) {
    constexpr int KS = D / 32;            // MFMA k-steps per tile
    constexpr int KL = KV8 ? D / 64 : KS; // K load instructions per tile (16 bytes per lane each)
    constexpr int EPL = D / 16;           // V: values per lane of a row (16 lanes per row)
    constexpr int NW = EPL * (KV8 ? 1 : 2) / 4;   // V: 32-bit words per lane of a row
    constexpr int NI = 4;                 // V: load instructions per tile (4 rows each)
    static_assert(GP <= 16, "kv group of at most 16 q heads");
    static_assert(!KV8 || BF16, "8-bit K/V pair with a bf16 query");
    static_assert(NW == 1 || NW == 2 || NW == 4, "V piece of 4, 8 or 16 bytes");
    static_assert(HW == 1 || HW == 2, "one or two kv heads per wave");
    static_assert(!FUSE || (!KV8 && HW == 1), "fused append: 16-bit K/V, one kv head per wave");
    using MfmaIn = typename MfmaType<BF16>::vec;
    using VLoad = VPiece<NW>;
    constexpr int DEPTH = 2;              // tiles in flight per wave
    static_assert(128 % DEPTH == 0, "a window of 128 positions holds whole pipeline steps");
    // f16 weights go to PV times 2^7 (<= 2^15 with TAU = 8), clear of the f16
    // subnormal range; the output divides it out.
    constexpr float kPScale = BF16 ? 1.f : 128.f;

    __shared__ int s_pre[kMaxSeqs + 1];
    __shared__ int s_len[kMaxSeqs];       // clamped context lengths, read once per workgroup
    __shared__ int s_wsum[kWaves];
    // Fused append: item index of each sequence (kNoItem: not appended).
    constexpr uint16_t kNoItem = 0xFFFF;
    static_assert(kFuseItems < kNoItem, "item index fits 16 bits");
    __shared__ uint16_t s_item[FUSE ? kMaxSeqs : 1];
    __shared__ FuseItem s_fit[FUSE ? kFuseItems : 1];   // the items, read from the kernel arguments once
    // Paired halves (a.pair_halves): softmax state exchange, 2 buffers x 2
    // wave pairs x (4 EPL + 2) floats x 64 lanes, dynamic LDS of the launch.
    extern __shared__ __align__(16) float xch[];

    const int lane = threadIdx.x & 63;
    // Wave index as a uniform (scalar) value, so loops stay scalar.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int B = a.num_seqs, Hkv = a.num_kv_heads;
    const int HG = Hkv / HW;              // list entries per (sequence, tile): kv heads taken HW at a time

    // The first kThreads context lengths are loaded before anything waits, so
    // their latency overlaps the fused append's reading of its items.
    const int len0 = (int)threadIdx.x < B ? a.context_lens[threadIdx.x] : 0;
    if constexpr (FUSE) {
        // An appended sequence's length is its item's new length: another
        // workgroup of this launch may be storing that length (and the new
        // block's table entry) while this one reads them.
        for (int s = threadIdx.x; s < B; s += kThreads) s_item[s] = kNoItem;
        for (int i = threadIdx.x; i < a.n_items; i += kThreads) s_fit[i] = fit[i];
        __syncthreads();
        for (int i = threadIdx.x; i < a.n_items; i += kThreads) s_item[s_fit[i].seq()] = (uint16_t)i;
        __syncthreads();
    }
    auto len_of = [&](int s) -> int {
        if constexpr (FUSE) {
            const int ii = s_item[s];
            if (ii != kNoItem) return min(max(s_fit[ii].new_len(), 0), a.max_context_len);
        }
        return min(max(s < kThreads ? len0 : a.context_lens[s], 0), a.max_context_len);
    };

    // ---- prefix of padded tiles over sequences (every workgroup, in LDS) ----
    int running = 0;
    for (int base = 0; base < B; base += kThreads) {
        const int s = base + (int)threadIdx.x;
        const int n = s < B ? len_of(s) : 0;
        if (s < B) s_len[s] = n;
        const int v = padded_tiles(len_tiles(n), a.fixed_chunk);
        int x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_wsum[wave] = x;
        __syncthreads();
        int woff = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            woff += w < wave ? s_wsum[w] : 0;
            tot += s_wsum[w];
        }
        if (s < B) s_pre[s] = (running + woff + x - v) * HG;
        running += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) s_pre[B] = running * HG;
    __syncthreads();
    const int T = s_pre[B];
    const int C = a.fixed_chunk > 0 ? a.fixed_chunk : max(kMinChunk, (T + a.num_waves - 1) / a.num_waves);
    const int NC = (T + C - 1) / C;

    const int lwg = xcd_remap(blockIdx.x, gridDim.x);
    if (lwg == 0) {
        // Publish the split for the merge kernel, and write the output of
        // every empty context (no chunk covers it): zeros, lse = -inf.
        for (int i = threadIdx.x; i <= B; i += kThreads) a.ws_hdr[2 + i] = s_pre[i];
        if (threadIdx.x == 0) { a.ws_hdr[0] = T; a.ws_hdr[1] = C; }
        if constexpr (FUSE) {
            // What kv_append writes besides the rows: the new lengths and the
            // table entries of blocks the call opened or copied into.
            for (int i = threadIdx.x; i < a.n_items; i += kThreads) {
                const FuseItem it = s_fit[i];
                a.lens_out[it.seq()] = it.new_len();
                if (it.new_block >= 0)
                    a.tables_out[(int64_t)it.seq() * a.table_stride + (it.new_len() - 1) / BS] = it.new_block;
            }
        }
        for (int s = 0; s < B; ++s) {
            if (s_pre[s + 1] != s_pre[s]) continue;
            for (int i = threadIdx.x; i < a.num_q_heads * D; i += kThreads)
                store_out(a.out, (int64_t)s * a.num_q_heads * D + i, 0.f, a.out_dtype);
            if (a.lse)
                for (int i = threadIdx.x; i < a.num_q_heads; i += kThreads) a.lse[(int64_t)s * a.num_q_heads + i] = -INFINITY;
        }
    }

    const int G = a.num_q_heads / Hkv;
    const int GC = HW * G;                // B-operand columns in use: the q heads of the wave's kv heads
    // MFMA operand roles (v_mfma_f32_16x16x32): A = 16 tokens x 32 d of K,
    // B = 32 d x 16 heads of q (heads >= G are zero), C = scores[token][head].
    // Lane l supplies A row l%16 and B column l%16, d-chunk 8*(l/16) of each
    // 32-wide k-step, and receives C[4*(l/16) + i][l%16], i = 0..3.
    const int mrow = lane & 15;           // K row (token in tile) / head of B and C
    const int kq = lane >> 4;             // d-chunk of the k-step / token quad of C
    // V layout: 16 lanes share a row; lane l owns the EPL values
    // [EPL (l%16), EPL (l%16 + 1)) of rows l/16 + 4i, i = 0..3.
    const float sl2 = a.scale * kLog2e;
    using KvElem = typename Pick<KV8, uint8_t, uint16_t>::type;
    const KvElem* kc = reinterpret_cast<const KvElem*>(a.k_cache);
    const KvElem* vc = reinterpret_cast<const KvElem*>(a.v_cache);
    // Lane's K element offset inside a tile (+ 32 * ks for 16-bit values).  With
    // 8-bit values a lane loads 16 codes, d in [16 cq, 16 cq + 16) with
    // cq = 4 u + kq, which feed k-steps 2u and 2u + 1; the q operand follows
    // the same d order, so the dot products are unchanged.
    const int krow = (mrow >> 2) + 4 * (mrow & 3);   // token of A-operand row mrow
    const int k_off = KV8 ? krow * D + kq * 16 : krow * D + kq * 8;
    const int v_off = kq * D + mrow * EPL;    // lane's V element offset inside a tile (+ i * 4 * D)

    // Softmax state of the current segment, per lane for head l%16 (equal in
    // the 4 lanes of a head): m_lane the reference (-inf before the first
    // tile, 0 for the padding heads >= G), l_lane the sum of this lane's
    // weights, acc[e] rows 4 (l/16) + i of PV MFMA e, i.e. output values
    // d = EPL (4 (l/16) + i) + e of head l%16.
    floatx4 acc[EPL];
    float m_lane = 0.f, l_lane = 0.f;
    int seg_s = 0, seg_g = 0, seg_ctx = 0, seg_nt = 0;
    int64_t seg_row = 0;                  // workspace row of the segment: chunk index + pair index
    bool seg_direct = false;

    auto tile_base = [&](int j, int g, int32_t blk) -> int64_t {
        return (((int64_t)blk * Hkv + g) * BS + (j * kTile) % BS) * D;
    };
    // QK on the matrix core, then the online-softmax update.  The tile's
    // weights come back in the B-operand layout of the PV MFMAs, split into
    // 16-bit hi and lo parts, times the tile's V scale (8-bit V) or kPScale
    // (the weight sum l keeps the unscaled weights).  8-bit K: codes widened
    // to bf16 in registers, the tile's K scale folded into the score scale.
    // With two kv heads per wave (HW == 2) both heads' K tiles go through the
    // same B operand (columns [0, G) are the first head's q heads, [G, 2G) the
    // second's) and each lane keeps the score of its own column's head.
    const bool second = HW == 2 && mrow >= G;   // this lane's column is a q head of the second kv head
    auto qk_softmax = [&](int j, const uint4 (&kb)[HW * KL], const MfmaIn (&qb)[KS], float ksc, float vsc,
                          float ksc1, float vsc1, uint2& phi, uint2& plo) {
        const int t0 = j * kTile;
        const bool full = t0 + kTile <= seg_ctx;
        floatx4 sch[HW];
#pragma unroll
        for (int h = 0; h < HW; ++h) {
            floatx4 sc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (KV8) {
#pragma unroll
                for (int u = 0; u < KL; ++u) {
                    const uint4 kw = kb[h * KL + u];
                    uint4 lo, hi;
                    fp8x4_to_bf16x4(kw.x, lo.x, lo.y);
                    fp8x4_to_bf16x4(kw.y, lo.z, lo.w);
                    fp8x4_to_bf16x4(kw.z, hi.x, hi.y);
                    fp8x4_to_bf16x4(kw.w, hi.z, hi.w);
                    sc = mfma_16x16x32<BF16>(__builtin_bit_cast(MfmaIn, lo), qb[2 * u], sc);
                    sc = mfma_16x16x32<BF16>(__builtin_bit_cast(MfmaIn, hi), qb[2 * u + 1], sc);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sc = mfma_16x16x32<BF16>(__builtin_bit_cast(MfmaIn, kb[h * KL + ks]), qb[ks], sc);
            }
            sch[h] = sc;
        }
        floatx4 sc = sch[0];
        if constexpr (HW == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = second ? sch[HW - 1][i] : sc[i];
        }
        const float sk = KV8 ? sl2 * (second ? ksc1 : ksc) : sl2;
        float x[4];
        bool need = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = sc[i] * sk;
            if (!full && t0 + kq + 4 * i >= seg_ctx) x[i] = -INFINITY;
            need |= x[i] > m_lane + kTau;
        }
        // Rare path: some score exceeds its head's reference by more than TAU.
        if (__builtin_amdgcn_ballot_w64(need)) {
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            mx = xmax16(mx);
            mx = xmax32(mx);                    // lane (j, n): tile max of head n
            if (mrow < GC && mx > m_lane + kTau) {
                const float alpha = __builtin_amdgcn_exp2f(m_lane - mx);   // 0 when m = -inf
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
                l_lane *= alpha;
                m_lane = mx;
            }
        }
        // Weights <= 2^TAU; a row past the context has x = -inf and weight 0.
        const float pm = KV8 ? (second ? vsc1 : vsc) : kPScale;
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = __builtin_amdgcn_exp2f(x[i] - m_lane);
            l_lane += e;
            pw[i] = e * pm;
        }
        split2<BF16>(pw[0], pw[1], phi.x, plo.x);
        split2<BF16>(pw[2], pw[3], phi.y, plo.y);
    };
    // PV on the matrix core.  For each of the lane's EPL values e the A
    // operand is (V[l/16][e], V[l/16 + 4][e], V[l/16 + 8][e], V[l/16 + 12][e])
    // of the tile in 16-bit form; the weights' hi parts, then lo parts, are
    // the B operand.
    auto pv = [&](int j, const VLoad (&vbh)[HW * NI], uint2 phi, uint2 plo) {
        const int t0 = j * kTile;
        const bool full = t0 + kTile <= seg_ctx;
#pragma unroll
        for (int h = 0; h < HW; ++h) {
        // B operand for head h: this lane's weights if its column is a q head of h, else 0.
        const bool mine = HW == 1 || (h == 1) == second;
        const uint2 ph = mine ? phi : make_uint2(0u, 0u), pl = mine ? plo : make_uint2(0u, 0u);
        uint32_t w[NI][NW];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int k = 0; k < NW; ++k) w[i][k] = vbh[h * NI + i].w[k];
        if (!full) {
            // Unused slots may hold anything (NaN included): never let them into a sum.
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (t0 + kq + 4 * i >= seg_ctx)
#pragma unroll
                    for (int k = 0; k < NW; ++k) w[i][k] = 0u;
        }
        uint2 av[EPL];
        if constexpr (KV8) {
            // Codes 4k .. 4k + 3 of the four rows: interleave rows (0, 1) and
            // (2, 3) byte by byte, then v_cvt_scalef32_pk_bf16_fp8 (scale 1,
            // exact) turns each pair of codes into the bf16 pair of one word.
#pragma unroll
            for (int k = 0; k < NW; ++k) {
                const uint32_t c01 = __builtin_amdgcn_perm(w[1][k], w[0][k], 0x05010400u);   // codes 0, 1
                const uint32_t c23 = __builtin_amdgcn_perm(w[1][k], w[0][k], 0x07030602u);   // codes 2, 3
                const uint32_t d01 = __builtin_amdgcn_perm(w[3][k], w[2][k], 0x05010400u);
                const uint32_t d23 = __builtin_amdgcn_perm(w[3][k], w[2][k], 0x07030602u);
                av[4 * k + 0] = make_uint2(fp8x2_to_bf16x2<false>(c01), fp8x2_to_bf16x2<false>(d01));
                av[4 * k + 1] = make_uint2(fp8x2_to_bf16x2<true>(c01), fp8x2_to_bf16x2<true>(d01));
                av[4 * k + 2] = make_uint2(fp8x2_to_bf16x2<false>(c23), fp8x2_to_bf16x2<false>(d23));
                av[4 * k + 3] = make_uint2(fp8x2_to_bf16x2<true>(c23), fp8x2_to_bf16x2<true>(d23));
            }
        } else {
            // Value e is half e & 1 of word e >> 1: pair it across rows (0, 1) and (2, 3).
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                av[e] = make_uint2(__builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel),
                                   __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel));
            }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = mfma_16x16x16<BF16>(av[e], ph, acc[e]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = mfma_16x16x16<BF16>(av[e], pl, acc[e]);
        }
    };
    // keep: plain loads (the lines stay cached) instead of non-temporal ones.
    // g is the list's head group: kv heads g * HW .. g * HW + HW - 1, whose
    // (block, kv head) pieces are adjacent in memory (BS * D values apart).
    // Fused append: a tile holding a sequence's new token (sub >= 0) reads that
    // row from the item's k_new / v_new instead of the cache (the cache row is
    // written by this same position, see new_row_k / new_row_v).
    const KvElem* knew = reinterpret_cast<const KvElem*>(a.k_new);
    const KvElem* vnew = reinterpret_cast<const KvElem*>(a.v_new);
    auto load_k = [&](int j, int g, int32_t blk, uint4 (&kb)[HW * KL], bool keep, int sub) {
        const int64_t base = tile_base(j, g * HW, blk);
#pragma unroll
        for (int h = 0; h < HW; ++h) {
            const KvElem* kp = kc + base + (int64_t)h * BS * D + k_off;
            if constexpr (FUSE) {
                if (sub >= 0) {                    // uniform: the tile of a new token
                    if (krow == (sub & 15)) kp = knew + ((int64_t)(sub >> 4) * Hkv + g) * D + kq * 8;
#pragma unroll
                    for (int u = 0; u < KL; ++u) kb[h * KL + u] = *reinterpret_cast<const uint4*>(kp + u * 32);
                    continue;
                }
            }
            if (keep) {
#pragma unroll
                for (int u = 0; u < KL; ++u) kb[h * KL + u] = *reinterpret_cast<const uint4*>(kp + u * (KV8 ? 64 : 32));
            } else {
#pragma unroll
                for (int u = 0; u < KL; ++u) kb[h * KL + u] = load_once16(kp + u * (KV8 ? 64 : 32));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_v = [&](int j, int g, int32_t blk, VLoad (&vb)[HW * NI], bool keep, int sub) {
        const int64_t base = tile_base(j, g * HW, blk);
#pragma unroll
        for (int h = 0; h < HW; ++h) {
            const int64_t hb = base + (int64_t)h * BS * D + v_off;
            if constexpr (FUSE) {
                if (sub >= 0) {                    // uniform: the tile of a new token
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const KvElem* vp = vc + hb + i * 4 * D;
                        if (kq + 4 * i == (sub & 15)) vp = vnew + ((int64_t)(sub >> 4) * Hkv + g) * D + mrow * EPL;
                        vb[h * NI + i] = load_piece<NW, false>(vp);
                    }
                    continue;
                }
            }
            if (keep) {
#pragma unroll
                for (int i = 0; i < NI; ++i) vb[h * NI + i] = load_piece<NW, false>(vc + hb + i * 4 * D);
            } else {
#pragma unroll
                for (int i = 0; i < NI; ++i) vb[h * NI + i] = load_piece<NW, true>(vc + hb + i * 4 * D);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Fused append: the lanes holding the new row write it to its cache slot
    // once it is in registers (K: the 4 lanes of A-operand row krow; V: the 16
    // lanes whose i-th load is that row) -- the rows kv_append would write.
    KvElem* kc_w = reinterpret_cast<KvElem*>(const_cast<void*>(a.k_cache));
    KvElem* vc_w = reinterpret_cast<KvElem*>(const_cast<void*>(a.v_cache));
    auto new_row_k = [&](int j, int g, int32_t blk, const uint4 (&kb)[HW * KL], int sub) {
        if constexpr (FUSE) {
            if (sub >= 0 && krow == (sub & 15)) {
                KvElem* kp = kc_w + tile_base(j, g, blk) + k_off;
#pragma unroll
                for (int u = 0; u < KL; ++u) *reinterpret_cast<uint4*>(kp + u * 32) = kb[u];
            }
        }
    };
    auto new_row_v = [&](int j, int g, int32_t blk, const VLoad (&vb)[HW * NI], int sub) {
        if constexpr (FUSE) {
            if (sub >= 0) {
                const int r = sub & 15;
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    if (kq + 4 * i == r) {
                        KvElem* vp = vc_w + tile_base(j, g, blk) + v_off + i * 4 * D;
                        if constexpr (NW == 4) {
                            *reinterpret_cast<uint4*>(vp) = make_uint4(vb[i].w[0], vb[i].w[1], vb[i].w[2], vb[i].w[3]);
                        } else if constexpr (NW == 2) {
                            *reinterpret_cast<uint2*>(vp) = make_uint2(vb[i].w[0], vb[i].w[1]);
                        } else {
                            *reinterpret_cast<uint32_t*>(vp) = vb[i].w[0];
                        }
                    }
            }
        }
    };
    // The q rows of kv group g of sequence s, as the QK B operand.
    auto load_q = [&](int s, int g, MfmaIn (&qb)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (mrow < GC) {
                const int d0 = KV8 ? 16 * (4 * (ks / 2) + kq) + 8 * (ks % 2) : ks * 32 + kq * 8;
                const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                                     ((int64_t)s * a.num_q_heads + g * GC + mrow) * D + d0;
                w = *reinterpret_cast<const uint4*>(qp);
            }
            qb[ks] = __builtin_bit_cast(MfmaIn, w);
        }
    };
    // End of a segment: l per head; lane l holds D/4 values of head l%16.
    auto finish_segment = [&]() {
        const float L = xsum32(xsum16(l_lane));   // lane (j, n): total of head n
        if (mrow < GC) {
            const float inv = 1.f / (L * kPScale);   // L >= 1: the tile that set the reference has weight 1
            const float lse2 = m_lane + __builtin_amdgcn_logf(L);
            const int64_t sh = (int64_t)seg_s * a.num_q_heads + seg_g * GC + mrow;
            const int d0 = 4 * EPL * kq;           // acc[e][i] is value d0 + EPL i + e
            if (seg_direct) {
                // Values d0 .. d0 + 4 EPL - 1 of the row, contiguous: acc[e][i] at EPL i + e.
                const int64_t o = sh * D + d0;
                if (a.out_dtype == kOutF32) {
                    float* op = reinterpret_cast<float*>(a.out) + o;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int e = 0; e < EPL; e += 4)
                            *reinterpret_cast<float4*>(op + EPL * i + e) =
                                make_float4(acc[e][i] * inv, acc[e + 1][i] * inv, acc[e + 2][i] * inv, acc[e + 3][i] * inv);
                } else {
                    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + o;
                    const bool bf = a.out_dtype == kOutBF16;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int e = 0; e < EPL; e += 2) {
                            const float v0 = acc[e][i] * inv, v1 = acc[e + 1][i] * inv;
                            const uint32_t w = bf ? (uint32_t)f32_to_bf16_rne(v0) | ((uint32_t)f32_to_bf16_rne(v1) << 16)
                                                  : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0) |
                                                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1) << 16);
                            *reinterpret_cast<uint32_t*>(op + EPL * i + e) = w;
                        }
                }
                if (kq == 0 && a.lse) a.lse[sh] = lse2 * kLn2;
            } else {
                float* o = a.ws_out + (seg_row * GC + mrow) * D + d0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < EPL; e += 4)
                        *reinterpret_cast<float4*>(o + EPL * i + e) =
                            make_float4(acc[e][i] * inv, acc[e + 1][i] * inv, acc[e + 2][i] * inv, acc[e + 3][i] * inv);
                if (kq == 0) a.ws_lse[seg_row * GC + mrow] = lse2;
            }
        }
    };

    // ---- the wave's chunks: w, w + NW, w + 2 NW, ... ----
    // A chunk's positions [lo, hi) of the flattened list run through one
    // pipeline, DEPTH tiles in flight, across the segments inside it: a
    // segment boundary only finishes one (s, g) and starts the next, the loads
    // keep going.  Position p's tile comes from per-lane windows of 128
    // positions (lane i: p = c0 + i and c0 + 64 + i): its sequence (~s when p
    // is not a tile to process: past the chunk, or padding of a fixed chunk),
    // kv head, tile index and block id (8-bit K/V: the block's scales come
    // with each tile, see issue_k).  A new window (every 128 positions of a
    // chunk) waits for its block ids once.  A position that is not processed still loads the
    // chunk's last real tile (see issue_k: a cache hit).
    // sub (fused append): (item << 4) | row when the position's tile holds the
    // sequence's new token at that row (the row comes from the item's k_new /
    // v_new, and this position writes it to the cache), else -1.
    struct Win { int sv, g, j, blk; int sub; };
    auto win_info = [&](int p, int hi) -> Win {
        const int pc = min(p, hi - 1);
        int sl = 0, sh = B;                        // invariant: pre[sl] <= pc < pre[sh]
        while (sh - sl > 1) {
            const int mid = (sl + sh) >> 1;
            if (s_pre[mid] <= pc) sl = mid; else sh = mid;
        }
        const int nt = len_tiles(s_len[sl]);       // >= 1: sequence sl owns position pc
        const int pt = padded_tiles(nt, a.fixed_chunk);
        const int rel = pc - s_pre[sl];
        Win w;
        w.g = rel / pt;
        const int j = rel - w.g * pt;
        w.j = min(j, nt - 1);
        w.sv = (p < hi && j < nt) ? sl : ~sl;
        w.blk = a.block_tables[(int64_t)sl * a.table_stride + (w.j * kTile) / BS];
        w.sub = -1;
        if constexpr (FUSE) {
            const int ii = s_item[sl];
            if (ii != kNoItem) {
                const FuseItem it = s_fit[ii];
                const int tn = it.new_len() - 1;   // position of the new token
                if (it.new_block >= 0 && (w.j * kTile) / BS == tn / BS) w.blk = it.new_block;
                if (w.j == tn / kTile) w.sub = (ii << 4) | (tn % kTile);
            }
        }
        return w;
    };
    // Positions [lo, hi) of chunk ch through the pipeline.  finish: each
    // segment ending in the range is written (else the caller combines the
    // range's softmax state with its partner's first).
    auto run_range = [&](int ch, int lo, int hi, bool finish) {
        int c0 = lo;
        Win wlo = win_info(c0 + lane, hi);
        Win whi = win_info(c0 + 64 + lane, hi);
        auto pick = [&](int vlo, int vhi, int x) -> int {
            const int i = x - c0;                  // in [0, 128)
            return i < 64 ? __builtin_amdgcn_readlane(vlo, i) : __builtin_amdgcn_readlane(vhi, i - 64);
        };
        // Per pipeline slot: the K, V and q operands of the position it holds,
        // and that position's (~)s, kv head, tile index and scales.
        uint4 kbuf[DEPTH][HW * KL];
        VLoad vbuf[DEPTH][HW * NI];
        MfmaIn qs[DEPTH][KS];
        int ps[DEPTH], pg[DEPTH], pj[DEPTH], pblk[DEPTH], psub[DEPTH];
        bool pkeep[DEPTH];
        float pks[DEPTH], pvs[DEPTH], pks1[DEPTH], pvs1[DEPTH];
        // Slot st takes position x: its K, and its q rows when the slot's
        // previous position (x - DEPTH) was another segment or before lo.
        auto issue_k = [&](int st, int x) {
            ps[st] = pick(wlo.sv, whi.sv, x);
            pg[st] = pick(wlo.g, whi.g, x);
            pj[st] = pick(wlo.j, whi.j, x);
            pblk[st] = pick(wlo.blk, whi.blk, x);
            psub[st] = FUSE ? pick(wlo.sub, whi.sub, x) : -1;
            pks[st] = pvs[st] = pks1[st] = pvs1[st] = 1.f;
            // The chunk's last real tile, and the positions past it that
            // re-read it, use plain loads: that tile stays in the cache and
            // the re-reads hit.
            pkeep[st] = ps[st] < 0 || x == hi - 1;
            load_k(pj[st], pg[st], pblk[st], kbuf[st], pkeep[st], psub[st]);
            if constexpr (KV8) {
                // The tile's K and V scales (one per (block, kv head)), wave-uniform:
                // scalar loads through the constant address space (the scales are not
                // written during the kernel), issued after the tile's K loads and first
                // used at its QK, and never waited on together with the vector loads.
                typedef const __attribute__((address_space(4))) float* ConstScale;
                const int64_t si = (int64_t)pblk[st] * Hkv + pg[st] * HW;   // the group's first kv head
                pks[st] = ((ConstScale)a.k_scale)[si];
                pvs[st] = ((ConstScale)a.v_scale)[si];
                if constexpr (HW == 2) {
                    pks1[st] = ((ConstScale)a.k_scale)[si + 1];
                    pvs1[st] = ((ConstScale)a.v_scale)[si + 1];
                }
            }
            if (ps[st] >= 0 && (x < lo + DEPTH || pj[st] < DEPTH)) load_q(ps[st], pg[st], qs[st]);
        };
        auto issue_v = [&](int st) { load_v(pj[st], pg[st], pblk[st], vbuf[st], pkeep[st], psub[st]); };
#pragma unroll
        for (int st = 0; st < DEPTH; ++st) {
            issue_k(st, lo + st);
            issue_v(st);
        }
        for (int p = lo; p < hi; p += DEPTH) {
            if (p + DEPTH - c0 == 128) {
                // The loads below run into the next window: read its block ids
                // (the positions in flight keep theirs in the slots).
                c0 += 128;
                wlo = win_info(c0 + lane, hi);
                whi = win_info(c0 + 64 + lane, hi);
            }
#pragma unroll
            for (int st = 0; st < DEPTH; ++st) {
                const int x = p + st;
                const int sv = ps[st], g = pg[st], j = pj[st];
                const bool live = sv >= 0;
                if (live && (x == lo || j == 0)) {
                    // A segment starts: (sv, g) from tile j on.
                    seg_s = sv;
                    seg_g = g;
                    seg_ctx = s_len[sv];
                    seg_nt = len_tiles(seg_ctx);
                    const int first = s_pre[sv] + g * padded_tiles(seg_nt, a.fixed_chunk);
                    // Segment k of pair p (sequence sv, head group g) is chunk first / C + k:
                    // rows chunk + p are distinct over all segments (a pair's chunks come after
                    // those of the pairs before it) and fewer than chunks + pairs.
                    seg_row = (int64_t)ch + (int64_t)sv * HG + g;
                    seg_direct = (first + seg_nt - 1) / C == first / C;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
                    m_lane = mrow < GC ? -INFINITY : 0.f;
                    l_lane = 0.f;
                }
                uint2 phi = make_uint2(0u, 0u), plo = make_uint2(0u, 0u);
                if (live) qk_softmax(j, kbuf[st], qs[st], pks[st], pvs[st], pks1[st], pvs1[st], phi, plo);
                const int32_t blk_x = pblk[st];    // issue_k below moves the slot on to x + DEPTH
                const int sub_x = psub[st];
                if constexpr (FUSE) {
                    if (live) new_row_k(j, g, blk_x, kbuf[st], sub_x);
                }
                issue_k(st, x + DEPTH);
                if (live) pv(j, vbuf[st], phi, plo);
                if constexpr (FUSE) {
                    if (live) new_row_v(j, g, blk_x, vbuf[st], sub_x);
                }
                issue_v(st);
                if (finish && live && (x == hi - 1 || j == seg_nt - 1)) finish_segment();
            }
        }
    };
    auto reset_state = [&]() {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
        m_lane = mrow < GC ? -INFINITY : 0.f;
        l_lane = 0.f;
    };
    if (!a.pair_halves) {
        const int w_global = lwg * kWaves + wave;
        for (int ch = w_global; ch < NC; ch += a.num_waves) run_range(ch, ch * C, min(ch * C + C, T), true);
        return;
    }
    // Fixed partitions, two waves per chunk: waves 2 q and 2 q + 1 of a
    // workgroup take the two halves of chunk 2 lwg + q + k NP (NP: wave pairs
    // in the grid), k = 0, 1, ...  The second half's softmax state goes
    // through LDS to the first, which merges it into its own and writes the
    // chunk's one segment (the same segment, row and output as one wave
    // taking the whole chunk).  Twice as many work units as chunks: a number
    // of partitions just above the grid's wave count no longer costs a second
    // full round.  Every wave passes one barrier per k; the exchange buffers
    // alternate with k, so a second-half wave never overwrites a state its
    // partner has not read.
    const int pq = wave >> 1, half = wave & 1;
    const int NP = a.num_waves >> 1;
    constexpr int XF = 4 * EPL + 2;                 // floats per lane: acc, m, l
    for (int k = 0; 2 * lwg + k * NP < NC; ++k) {
        const int ch = 2 * lwg + pq + k * NP;
        reset_state();
        const int mid = ch * C + C / 2;
        if (ch < NC) run_range(ch, half ? mid : ch * C, half ? min(ch * C + C, T) : min(mid, T), false);
        float* xb = xch + (size_t)(((k & 1) * 2 + pq) * XF) * 64;   // [field][lane]
        if (half == 1 && ch < NC) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) xb[(4 * e + i) * 64 + lane] = acc[e][i];
            xb[(4 * EPL) * 64 + lane] = m_lane;
            xb[(4 * EPL + 1) * 64 + lane] = l_lane;
        }
        __syncthreads();
        if (half == 0 && ch < NC) {
            const float m1 = xb[(4 * EPL) * 64 + lane], l1 = xb[(4 * EPL + 1) * 64 + lane];
            const float M = fmaxf(m_lane, m1);
            // Scale factors of the two halves (a half with no tile of this
            // chunk has m = -inf, l = 0, acc = 0: factor 0).  Padding heads
            // (rows >= GC) keep m = 0 in both halves.
            const float f0 = m_lane == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_lane - M);
            const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[e][i] = acc[e][i] * f0 + xb[(4 * e + i) * 64 + lane] * f1;
            l_lane = l_lane * f0 + l1 * f1;
            m_lane = M;
            finish_segment();
        }
    }
}

template <int D, int BS, int GP, bool BF16, bool KV8, int HW>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KV8 ? (HW == 2 ? 2 : 3) : 1)))
paged_decode_split_kernel(DecodeArgs a) {
    split_body<D, BS, GP, BF16, KV8, HW, false>(a, nullptr);
}

// The split with the step's append folded in: a.n_items new tokens (items in
// the kernel arguments, rows in a.k_new / a.v_new) are part of the contexts
// this launch decodes, and the launch stores what kv_append stores: each new
// K/V row (by the wave that reads it), each new length and each table entry
// of a block the step opened or copied into (by workgroup 0).  Readers in
// this launch take lengths and those table entries from the items, so the
// stores race with nothing they use.
template <int D, int BS, int GP, bool BF16>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
paged_decode_append_split_kernel(DecodeArgs a, FuseItems items) {
    split_body<D, BS, GP, BF16, false, 1, true>(a, items.it);
}

// Merge kernel: WPP waves per (sequence, q head) whose (s, g) spans more than
// one chunk -- one wave (four pairs per workgroup) or a whole workgroup.  With
// M = max_k lse_k and w_k = 2^(lse_k - M): out = sum_k w_k o_k / sum_k w_k and
// lse = M + log2(sum_k w_k) -- the online-softmax identity applied to the
// segments.  Segment k of the pair p (sequence s, head group g / HW) sits in
// workspace row first / C + k + p, column hq - (g / HW) GC of its GC q heads.
// A wave load covers RPL segment rows (lane l reads 4 consecutive d values of
// row l / (D/4)); the pair's waves take rows in turn and each lane keeps
// UNROLL rows in flight, so a pair's first WPP RPL UNROLL rows arrive in one
// round trip once the length and the header (chunk size, tile prefix) have
// given the first row.  Every wave computes M itself from the lse values;
// rows with the same d slice are summed by lane swaps, waves by LDS.
template <int D, int WPP>
__global__ void __launch_bounds__(kThreads)
paged_decode_merge_kernel(MergeArgs a) {
    constexpr int LPR = D / 4;                 // lanes per segment row (4 floats each)
    constexpr int RPL = 64 / LPR;              // rows per wave load
    constexpr int STEP = RPL * WPP;            // rows per load across the pair's waves
    constexpr int UNROLL = 4;
    constexpr int PAIRS = kWaves / WPP;        // pairs per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wp = wave % WPP;                 // this wave's index within its pair
    const int64_t sh = (int64_t)blockIdx.x * PAIRS + wave / WPP;
    if (sh >= (int64_t)a.num_seqs * a.num_q_heads) return;   // uniform over a pair's waves
    const int s = (int)(sh / a.num_q_heads);
    const int hq = (int)(sh % a.num_q_heads);
    const int G = a.num_q_heads / a.num_kv_heads;
    const int HW = a.heads_per_wave;
    const int GC = HW * G;                     // q heads per workspace row
    const int gp = hq / GC;                    // head group of the list
    const int d4 = (lane % LPR) * 4;
    const int r0 = wp * RPL + lane / LPR;      // this lane's first row

    const int len = a.context_lens[s];
    const int C = a.ws_hdr[1];
    const int pre = a.ws_hdr[2 + s];
    const int n = min(max(len, 0), a.max_context_len);
    const int nt = (n + kTile - 1) / kTile;
    const int pt = a.fixed_chunk > 0 ? (nt + a.fixed_chunk - 1) / a.fixed_chunk * a.fixed_chunk : nt;
    const int first = pre + gp * pt;
    // Empty pairs are written by the split kernel, one-segment pairs directly.
    const int nseg = nt == 0 ? 0 : (first + nt - 1) / C - first / C + 1;
    if (nseg <= 1) return;                     // uniform over a pair's waves
    const int64_t row0 = (int64_t)(first / C) + (int64_t)s * (a.num_kv_heads / HW) + gp;
    const int hcol = hq - gp * GC;
    const float* lse_p = a.ws_lse + row0 * GC + hcol;             // row k at lse_p[k GC]
    const float* out_p = a.ws_out + (row0 * GC + hcol) * D + d4;  // row k at out_p[k GC D]
    const int64_t rs = (int64_t)GC * D;

    float4 v0[UNROLL];
    float l0[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int k = r0 + u * STEP;
        v0[u] = k < nseg ? *reinterpret_cast<const float4*>(out_p + k * rs) : make_float4(0.f, 0.f, 0.f, 0.f);
        l0[u] = k < nseg ? lse_p[(int64_t)k * GC] : -INFINITY;
    }
    float M = -INFINITY;
    for (int k = lane; k < nseg; k += 64) M = fmaxf(M, lse_p[(int64_t)k * GC]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float W = 0.f;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        if (r0 + u * STEP < nseg) {
            const float w = __builtin_amdgcn_exp2f(l0[u] - M);
            acc.x = fmaf(w, v0[u].x, acc.x);
            acc.y = fmaf(w, v0[u].y, acc.y);
            acc.z = fmaf(w, v0[u].z, acc.z);
            acc.w = fmaf(w, v0[u].w, acc.w);
            W += w;
        }
    }
    for (int kb = r0 + UNROLL * STEP; kb < nseg; kb += UNROLL * STEP) {
        float4 v[UNROLL];
        float l[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int k = kb + u * STEP;
            v[u] = k < nseg ? *reinterpret_cast<const float4*>(out_p + k * rs) : make_float4(0.f, 0.f, 0.f, 0.f);
            l[u] = k < nseg ? lse_p[(int64_t)k * GC] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (kb + u * STEP < nseg) {
                const float w = __builtin_amdgcn_exp2f(l[u] - M);
                acc.x = fmaf(w, v[u].x, acc.x);
                acc.y = fmaf(w, v[u].y, acc.y);
                acc.z = fmaf(w, v[u].z, acc.z);
                acc.w = fmaf(w, v[u].w, acc.w);
                W += w;
            }
        }
    }
    // Rows of one wave load that share a d slice: lanes LPR apart.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off);
        acc.y += __shfl_xor(acc.y, off);
        acc.z += __shfl_xor(acc.z, off);
        acc.w += __shfl_xor(acc.w, off);
        W += __shfl_xor(W, off);
    }
    if constexpr (WPP > 1) {
        // PAIRS == 1 here: every wave of the workgroup reaches this barrier.
        __shared__ float4 s_acc[kWaves][LPR];
        __shared__ float s_w[kWaves];
        if (lane < LPR) s_acc[wave][lane] = acc;
        if (lane == 0) s_w[wave] = W;
        __syncthreads();
        if (wave != 0) return;
        if (lane < LPR) {
#pragma unroll
            for (int w2 = 1; w2 < kWaves; ++w2) {
                const float4 o = s_acc[w2][lane];
                acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
            }
        }
#pragma unroll
        for (int w2 = 1; w2 < kWaves; ++w2) W += s_w[w2];
    }
    if (lane >= LPR) return;
    const int64_t o = sh * D + d4;
    store_out(a.out, o + 0, acc.x / W, a.out_dtype);
    store_out(a.out, o + 1, acc.y / W, a.out_dtype);
    store_out(a.out, o + 2, acc.z / W, a.out_dtype);
    store_out(a.out, o + 3, acc.w / W, a.out_dtype);
    if (a.lse && lane == 0) a.lse[sh] = (M + __builtin_amdgcn_logf(W)) * kLn2;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------

// Timing events of a split launch: null, or start and stop events that the
// dispatch itself stamps (hipExtLaunchKernel).
struct LaunchEvents { hipEvent_t start, stop; };

template <int D, int BS, int GP, bool BF16, bool KV8, int HW>
static hipError_t split_dispatch(const DecodeArgs* a, int* waves_per_cu, hipStream_t stream, const LaunchEvents* ev) {
    auto kern = paged_decode_split_kernel<D, BS, GP, BF16, KV8, HW>;
    if (waves_per_cu) {
        int blocks = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kern, kThreads, 0);
        if (e != hipSuccess) return e;
        *waves_per_cu = blocks * kWaves;
        return hipSuccess;
    }
    const dim3 grid((unsigned)(a->num_waves / kWaves));
    const unsigned lds = a->pair_halves ? (unsigned)split_pair_lds_bytes(D) : 0u;
    if (ev && (ev->start || ev->stop))
        hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, ev->start, ev->stop, 0, *a);
    else
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, *a);
    return hipGetLastError();
}

template <int D, int BS, int GP, bool BF16>
static hipError_t split_append_dispatch(const DecodeArgs& a, const FuseItems& items, hipStream_t stream,
                                        const LaunchEvents& ev) {
    auto kern = paged_decode_append_split_kernel<D, BS, GP, BF16>;
    const dim3 grid((unsigned)(a.num_waves / kWaves));
    const unsigned lds = a.pair_halves ? (unsigned)split_pair_lds_bytes(D) : 0u;
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, ev.start, ev.stop, 0, a, items);
    else
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a, items);
    return hipGetLastError();
}

template <int D, int BS, bool BF16>
static hipError_t split_append_g(const DecodeArgs& a, const FuseItems& items, int gp, hipStream_t st,
                                 const LaunchEvents& ev) {
    switch (gp) {
        case 1: return split_append_dispatch<D, BS, 1, BF16>(a, items, st, ev);
        case 2: return split_append_dispatch<D, BS, 2, BF16>(a, items, st, ev);
        case 4: return split_append_dispatch<D, BS, 4, BF16>(a, items, st, ev);
        case 8: return split_append_dispatch<D, BS, 8, BF16>(a, items, st, ev);
    }
    return hipErrorInvalidValue;
}

template <int D, int BS, bool BF16, bool KV8, int HW>
static hipError_t split_g(const DecodeArgs* a, int gp, int* wpc, hipStream_t st, const LaunchEvents* ev) {
    if constexpr (HW == 1) {
        switch (gp) {
            case 1: return split_dispatch<D, BS, 1, BF16, KV8, 1>(a, wpc, st, ev);
            case 2: return split_dispatch<D, BS, 2, BF16, KV8, 1>(a, wpc, st, ev);
            case 4: return split_dispatch<D, BS, 4, BF16, KV8, 1>(a, wpc, st, ev);
            case 8: return split_dispatch<D, BS, 8, BF16, KV8, 1>(a, wpc, st, ev);
        }
    } else {
        switch (gp) {          // columns of two kv heads' q groups: 2 G
            case 2: return split_dispatch<D, BS, 2, BF16, KV8, 2>(a, wpc, st, ev);
            case 4: return split_dispatch<D, BS, 4, BF16, KV8, 2>(a, wpc, st, ev);
            case 8: return split_dispatch<D, BS, 8, BF16, KV8, 2>(a, wpc, st, ev);
            case 16: return split_dispatch<D, BS, 16, BF16, KV8, 2>(a, wpc, st, ev);
        }
    }
    return hipErrorInvalidValue;
}

template <int D, bool BF16, bool KV8, int HW>
static hipError_t split_b(const DecodeArgs* a, int bs, int gp, int* wpc, hipStream_t st, const LaunchEvents* ev) {
    if (bs == 16) return split_g<D, 16, BF16, KV8, HW>(a, gp, wpc, st, ev);
    if (bs == 32) return split_g<D, 32, BF16, KV8, HW>(a, gp, wpc, st, ev);
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t split_t(const DecodeArgs* a, int bs, int gp, KvKind kind, int* wpc, hipStream_t st,
                          const LaunchEvents* ev) {
    switch (kind) {
        case KvKind::F16: return split_b<D, false, false, 1>(a, bs, gp, wpc, st, ev);
        case KvKind::BF16: return split_b<D, true, false, 1>(a, bs, gp, wpc, st, ev);
        case KvKind::FP8_BF16Q: return split_b<D, true, true, 1>(a, bs, gp, wpc, st, ev);
        case KvKind::FP8_BF16Q_PAIR: return split_b<D, true, true, 2>(a, bs, gp, wpc, st, ev);
    }
    return hipErrorInvalidValue;
}

static hipError_t split_any(const DecodeArgs* a, int head_dim, int bs, int gp, KvKind kind, int* wpc, hipStream_t st,
                            const LaunchEvents* ev) {
    if (head_dim == 128) return split_t<128>(a, bs, gp, kind, wpc, st, ev);
    if (head_dim == 64) return split_t<64>(a, bs, gp, kind, wpc, st, ev);
    return hipErrorInvalidValue;
}

hipError_t split_waves_per_cu(int head_dim, int block_size, int group_pad, KvKind kind, int* waves_per_cu) {
    return split_any(nullptr, head_dim, block_size, group_pad, kind, waves_per_cu, nullptr, nullptr);
}

hipError_t launch_split(const DecodeArgs& a, int head_dim, int block_size, int group_pad, KvKind kind,
                        hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (a.num_waves < kWaves || a.num_waves % kWaves) return hipErrorInvalidValue;
    const bool pair = kind == KvKind::FP8_BF16Q_PAIR;
    if ((kind == KvKind::FP8_BF16Q || pair) && (!a.k_scale || !a.v_scale)) return hipErrorInvalidValue;
    if (a.heads_per_wave != (pair ? 2 : 1) || a.num_kv_heads % a.heads_per_wave) return hipErrorInvalidValue;
    const LaunchEvents ev{start, stop};
    return split_any(&a, head_dim, block_size, group_pad, kind, nullptr, stream, &ev);
}

hipError_t launch_split_append(const DecodeArgs& a, const FuseItems& items, int head_dim, int block_size, int group_pad,
                               KvKind kind, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (a.num_waves < kWaves || a.num_waves % kWaves || a.heads_per_wave != 1) return hipErrorInvalidValue;
    if (a.n_items < 0 || a.n_items > kFuseItems || (a.n_items > 0 && (!a.k_new || !a.v_new)) || !a.lens_out ||
        !a.tables_out || a.num_seqs > kMaxSeqs)
        return hipErrorInvalidValue;
    const LaunchEvents ev{start, stop};
    const bool bf = kind == KvKind::BF16;
    if (kind != KvKind::BF16 && kind != KvKind::F16) return hipErrorInvalidValue;
    if (head_dim == 128) {
        if (block_size == 16) return bf ? split_append_g<128, 16, true>(a, items, group_pad, stream, ev)
                                        : split_append_g<128, 16, false>(a, items, group_pad, stream, ev);
        if (block_size == 32) return bf ? split_append_g<128, 32, true>(a, items, group_pad, stream, ev)
                                        : split_append_g<128, 32, false>(a, items, group_pad, stream, ev);
    } else if (head_dim == 64) {
        if (block_size == 16) return bf ? split_append_g<64, 16, true>(a, items, group_pad, stream, ev)
                                        : split_append_g<64, 16, false>(a, items, group_pad, stream, ev);
        if (block_size == 32) return bf ? split_append_g<64, 32, true>(a, items, group_pad, stream, ev)
                                        : split_append_g<64, 32, false>(a, items, group_pad, stream, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
    const int64_t pairs = (int64_t)a.num_seqs * a.num_q_heads;
    if (pairs == 0) return hipSuccess;
    if (a.heads_per_wave < 1 || a.heads_per_wave > 2 || a.num_kv_heads % a.heads_per_wave) return hipErrorInvalidValue;
    // A workgroup per pair where segment lists may be long: the fixed split
    // of a long context, or few pairs (where one long context among short ones
    // spans many of the balanced split's chunks and the grid is small anyway).
    // Otherwise one wave per pair: many pairs of a few segments each, for which
    // a workgroup each would only add dispatch work.
    const bool wide = pairs <= kMergeWidePairs || (a.fixed_chunk > 0 && a.max_seg > kMergeWideSegments);
    const int per_block = wide ? 1 : kWaves;
    const unsigned n = (unsigned)((pairs + per_block - 1) / per_block);
    if (head_dim == 128) {
        if (wide) hipLaunchKernelGGL((paged_decode_merge_kernel<128, kWaves>), dim3(n), dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((paged_decode_merge_kernel<128, 1>), dim3(n), dim3(kThreads), 0, stream, a);
    } else if (head_dim == 64) {
        if (wide) hipLaunchKernelGGL((paged_decode_merge_kernel<64, kWaves>), dim3(n), dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((paged_decode_merge_kernel<64, 1>), dim3(n), dim3(kThreads), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
