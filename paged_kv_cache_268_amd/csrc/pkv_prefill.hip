// pkv_prefill.hip -- chunked prefill attention over the paged KV cache, gfx950.
//
// What is computed ("架构解构：推理引擎的四层抽象", FlashAttention section: tiled
// attention with an online softmax, scores never in HBM, K/V reached through
// the block table): sequence s holds context_lens[s] = n tokens in the cache,
// the last m of which are this chunk (rows cu_q[s] .. cu_q[s+1]-1 of q and
// out).  Chunk query i sits at position n - m + i and attends to the tokens at
// positions 0 .. n - m + i (causal); scores are q.k times the scale, softmax
// is the stable form, sums are fp32.  A query head h uses kv head h / (Hq/Hkv).
//
// Work decomposition.  The G q heads of one kv head share every K/V tile, so a
// workgroup takes one kv head g and kPrefillRows = 128 rows (chunk query,
// q head): Qt = 128 / G consecutive chunk queries times the G heads of the
// group, row r = (query r / G, head g G + r % G).  Four waves of 32 rows each
// (two 16-row column blocks per wave, so every K or V operand a wave reads
// from LDS feeds two (QK) or four (PV, hi and lo weights) matrix
// instructions); two workgroups per CU, so the two waves on a SIMD belong to
// different workgroups and do not wait at each other's barriers.  The
// workgroup walks 32-key tiles from position 0 to its last query's position;
// each tile is read once per workgroup from the pool (16-byte loads through
// the block table, block ids by scalar loads) into LDS, double buffered, with
// the loads issued two tiles ahead (two register stages).  Workgroup i covers
// kv head i / tiles, so consecutive workgroups (one XCD, one L2) read the
// same kv head's blocks, and within a kv head the query tiles go longest
// first (sequences by context length, each sequence's tiles last first), so
// that each XCD's last workgroups are short ones.
//
// LDS layout.  K rows are 2D bytes apart and stored in a key order that
// puts the 16 keys of each A operand in consecutive rows: LDS row 16 h + 4 a + i
// holds key 8 a + 4 h + i (a, i < 4, h < 2).  V is stored transposed, one row
// of 32 keys per d, written by units of 2 keys x 8 d (two 16-byte loads, each
// d's 2 keys stored as one 32-bit word).  No row padding: 16-byte chunks are
// swizzled (kswz, vrow_phys, vchunk) so that no access shape has a bank
// conflict.  Rows past the context end: K as loaded (those scores are masked
// before use), V zeroed.
//
// Both contractions run on v_mfma_f32_16x16x32 (bf16 or f16 inputs, fp32
// accumulation):
//   S^T = K Q^T: A = 16 keys x 32 d from LDS (half h: LDS rows 16 h ..
//   16 h + 15), B = 16 rows x 32 d of the queries, held in registers.  Lane l
//   receives, for row l % 16, the scores of keys 8 (l / 16) + 4 h + i
//   (i = 0..3): with both halves, 8 consecutive keys.
//   O^T += V^T P^T: those 8 weights are exactly lane l's B operand (8 keys of
//   row l % 16), and the A operand is one 16-byte LDS read: the same 8 keys
//   of one transposed V row.  D/16 output blocks of 16 d.
// Softmax per row: a reference max that moves only when a score exceeds it by
// more than 8 (log2 units), so the accumulator rescale is a rare event
// (skipped for the whole wave when no row needs it) and every weight stays
// <= 2^8.  The weights enter the second product as a bf16 (f16) pair hi + lo
// with hi = round(p) and lo = round(p - hi), two matrix instructions per
// block: one rounded 16-bit weight carries up to 2^-9 relative error, too
// coarse for outputs checked to 2e-3; the pair carries about 2^-17.  The
// running max, the rescale and the weight sum stay in fp32 per row (reduced
// over the 4 lanes of a row with permlane swaps).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"
#include "pkv_prefill.h"

namespace pkv {
namespace {

constexpr int kPWaves = kPrefillWaves;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPBlocks = kPrefillRows / kPWaves / 16;   // 16-row column blocks per wave
constexpr int kPKeys = 32;                      // keys per tile
constexpr float kPLog2e = 1.4426950408889634f;
constexpr float kPLn2 = 0.6931471805599453f;
constexpr float kPTau = 8.0f;                   // lazy-rescale threshold (log2 units)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes staged as a plain vector value
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

template <bool BF16> struct PType { using v8 = f16x8v; using e = _Float16; };
template <> struct PType<true> { using v8 = bf16x8v; using e = __bf16; };

template <bool BF16>
__device__ __forceinline__ f32x4 mma(typename PType<BF16>::v8 a, typename PType<BF16>::v8 b, f32x4 c) {
    if constexpr (BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Maximum that propagates NaN (v_maximum3_f32 on gfx950): unlike fmaxf it needs
// no quieting of its inputs, so a chain of them is one instruction per two values.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax8(const float (&v)[8]) {
    return vmax(vmax(vmax(vmax(vmax(vmax(vmax(v[0], v[1]), v[2]), v[3]), v[4]), v[5]), v[6]), v[7]);
}

// Reductions across lanes l ^ 16 and l ^ 32 (the 4 lanes of one score column).
__device__ __forceinline__ float pmax16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return vmax(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pmax32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return vmax(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float psum16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float psum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Two weights -> their 16-bit roundings (hi, one packed word) and the
// roundings of what is left (lo): p = hi + lo to about 2^-17 relative.
// bf16: each residual p - hi comes from one v_dot2_f32_bf16, hi . (-1, 0) + p0
// and hi . (0, -1) + p1, exact (every term is); sel0 / sel1 hold those two
// bf16 pairs in registers: encoded by the compiler as an inline constant, the
// pair (-1, 0) gave wrong residuals.  Checked bit-exact against p - RNE(p) on
// four million weights, denormals included.
template <bool BF16>
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t sel0, uint32_t sel1, uint32_t& hi, uint32_t& lo) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    if constexpr (BF16) {
        const b2 h = {(__bf16)p0, (__bf16)p1};
        const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(b2, sel0), p0, false);
        const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(b2, sel1), p1, false);
        const b2 l = {(__bf16)r0, (__bf16)r1};
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, l);
    } else {
        const h2 h = {(_Float16)p0, (_Float16)p1};
        const h2 l = {(_Float16)(p0 - (float)h.x), (_Float16)(p1 - (float)h.y)};
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, l);
    }
}

// LDS layouts without padding and without bank conflicts on gfx950, whose LDS
// serves a 16-byte read in four passes of 16 lanes (lanes 32 h + 4 j .. + 3
// for the j of one popcount parity) and a 4-byte write in two passes of 32
// lanes, over 64 banks of 4 bytes.  K: row R (D bf16 values, D / 8 chunks of
// 16 bytes) keeps chunk c at chunk c ^ kswz(R).  V transposed: rows of 32
// keys (64 bytes, four chunks of 8 keys); row d is stored at row
// vrow_phys(d) = d ^ ((d >> 3) & 3) and chunk q of it at chunk q ^ vchunk(row).
// Checked against the hardware's conflict counter for every access shape of
// this kernel: the operand reads (16 rows of one chunk column per wave), the
// K row stores (16 lanes per row) and the two-key V stores (four rows 8 apart
// per store).
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 7) << 1 : r & 6; }
__device__ __forceinline__ int vrow_phys(int d) { return d ^ ((d >> 3) & 3); }
__device__ __forceinline__ int vchunk(int p) { return (p & 4) >> 1; }

// Workgroup i runs on XCD i % 8; consecutive logical ids share an XCD (its L2).
__device__ __forceinline__ int prefill_xcd_remap(int i, int n) {
    const int per = n / kNumXcds;
    if (i < per * kNumXcds) return (i % kNumXcds) * per + i / kNumXcds;
    return i;
}

}  // namespace

template <int D, int BS, bool BF16>
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
paged_prefill_kernel(PrefillArgs a) {
    using V8 = typename PType<BF16>::v8;
    constexpr int KS = D / 32;                    // k-steps of S^T
    constexpr int DB = D / 16;                    // 16-row output blocks of O^T
    constexpr int NB = kPBlocks;                  // column blocks per wave
    constexpr int KROW = D * 2;                   // bytes per K row in LDS (unpadded: chunks swizzled, see kswz)
    constexpr int VROW = kPKeys * 2;              // bytes per transposed V row in LDS (see vrow_phys)
    constexpr int KBUF = kPKeys * KROW, VBUF = D * VROW;
    constexpr int CPR = D / 8;                    // 16-byte pieces per K/V row
    // Staging: every thread loads KPT 16-byte K pieces and one V unit (2 keys x
    // 8 d, two 16-byte loads) per tile; all threads run the same loads, so the
    // wait for a tile's loads is exact.  At D = 64 there are half as many V
    // units as threads and the upper half repeats the lower half's.
    constexpr int KPT = kPKeys * CPR / kPThreads; // K pieces per thread
    constexpr int VU = (kPKeys / 2) * CPR;        // V units per tile
    constexpr int SR = KPT + 2;                   // staging registers per thread
    static_assert(KPT >= 1 && KPT * kPThreads == kPKeys * CPR && kPThreads % VU == 0, "tile shape");
    // The tile buffers, or the tile prefix over sequences that precedes them (it
    // aliases their space), whichever is larger.
    constexpr int LDS = 2 * (KBUF + VBUF) > (kPrefillMaxSeqs + 1) * 4 ? 2 * (KBUF + VBUF) : ((kPrefillMaxSeqs + 1) * 4 + 15) / 16 * 16;
    static_assert((4 * kPrefillSortSeqs + 1) * 4 <= LDS, "the sorted work order fits");
    __shared__ __align__(16) uint8_t s_mem[LDS];
    __shared__ int s_wsum[kPWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int B = a.num_seqs, Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
    const int Qt = a.query_tile;

    // ---- work order (in LDS, aliasing the tile buffers) ----
    // Query tiles are handed out longest first, so that the last workgroups of
    // each XCD are short ones: sequences in order of context length, longest
    // first (ties by index; up to kPrefillSortSeqs sequences, else last to
    // first), and a sequence's tiles last to first.  Position i of the order
    // holds sequence ord(i); s_pre[i] counts the query tiles before it.
    auto tiles_of = [&](int s) {
        const int m = a.cu_q[s + 1] - a.cu_q[s];
        return m > 0 ? (m + Qt - 1) / Qt : 0;
    };
    int* s_pre = reinterpret_cast<int*>(s_mem);    // [B + 1]
    int* s_key = s_pre + B + 1;                    // [B], sorted order only: context lengths
    int* s_ord = s_key + B;                        // [B]: the sequence at position i
    int* s_cnt = s_ord + B;                        // [B]: its query tiles
    const bool by_len = B <= kPrefillSortSeqs;     // uniform
    if (by_len) {
        for (int s = tid; s < B; s += kPThreads) s_key[s] = min(max(a.context_lens[s], 0), a.max_context_len);
        __syncthreads();
        for (int s = tid; s < B; s += kPThreads) {
            const int k = s_key[s];
            int r = 0;                             // sequences ahead of s
            for (int t = 0; t < B; ++t) {
                const int kt = s_key[t];
                r += (kt > k || (kt == k && t < s)) ? 1 : 0;
            }
            s_ord[r] = s;
            s_cnt[r] = tiles_of(s);
        }
        __syncthreads();
    }
    int running = 0;
    for (int base = 0; base < B; base += kPThreads) {
        const int i = base + tid;
        const int v = i < B ? (by_len ? s_cnt[i] : tiles_of(B - 1 - i)) : 0;
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
        for (int w = 0; w < kPWaves; ++w) {
            woff += w < wave ? s_wsum[w] : 0;
            tot += s_wsum[w];
        }
        if (i < B) s_pre[i] = running + woff + x - v;
        running += tot;
        __syncthreads();
    }
    if (tid == 0) s_pre[B] = running;
    __syncthreads();
    const int T = s_pre[B];
    const int lwg = prefill_xcd_remap(blockIdx.x, gridDim.x);
    const int g = lwg / a.grid_tiles;              // kv head: consecutive workgroups share it
    const int tl = lwg - g * a.grid_tiles;         // rank of the query tile in the order
    if (g >= Hkv || tl >= T) return;               // uniform over the workgroup
    int sl = 0, sh = B;                            // pre[sl] <= tl < pre[sh]
    while (sh - sl > 1) {
        const int mid = (sl + sh) >> 1;
        if (s_pre[mid] <= tl) sl = mid; else sh = mid;
    }
    const int s = by_len ? s_ord[sl] : B - 1 - sl;
    const int qt = s_pre[sl + 1] - 1 - tl;         // the sequence's tiles, last first
    __syncthreads();                               // order dead: LDS now holds K/V tiles

    const int n = min(max(a.context_lens[s], 0), a.max_context_len);
    const int q0 = a.cu_q[s];
    const int m = max(a.cu_q[s + 1] - q0, 0);
    const int base_pos = n - m;                    // position of chunk row 0
    const int qa = qt * Qt;
    const int nq = min(Qt, m - qa);                // chunk queries of this tile
    const int rows = nq * G;                       // rows in use (<= 256)
    const int last_pos = base_pos + qa + nq - 1;
    const int NT = last_pos >= 0 ? (last_pos + kPKeys) / kPKeys : 0;

    const int col = lane & 15, quad = lane >> 4;
    // This lane's rows (one per column block): chunk query, q head, validity, position.
    int qrow[NB], qhead[NB], qpos[NB];
    bool qvalid[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        const int r = wave * (16 * NB) + c * 16 + col;
        const int qi = qa + r / G;
        qrow[c] = q0 + qi;
        qhead[c] = g * G + r % G;
        qvalid[c] = r < rows && q0 + qi < a.total_q;
        qpos[c] = base_pos + qi;
    }
    // Scores in log2 units: s * sl2 with sl2 > 0, so that the maximum of the
    // scaled scores is the scaled maximum (rounding is monotone).  A negative
    // scale is carried by the q operand instead (its sign bits flipped: exact);
    // a zero scale becomes the smallest normal float (weights 1 to within
    // 1e-37, and a masked score -inf still scales to -inf, not NaN).
    const bool qneg = a.scale < 0.f;
    const float sl2 = fmaxf(fabsf(a.scale) * kPLog2e, __FLT_MIN__);
    // The wave's rows [r0, r1): tiles [0, nomask_tiles) need no causal mask
    // (all 32 rows real and the tile's last key before the first row's
    // query), and tiles from wave_tiles on are masked out for every row.
    const int r0 = wave * (16 * NB), r1 = min(r0 + 16 * NB, rows);
    int wave_tiles = 0, nomask_tiles = 0;
    if (r1 > r0) {
        const int p0 = base_pos + qa + r0 / G, p1 = base_pos + qa + (r1 - 1) / G;
        wave_tiles = p1 >= 0 ? p1 / kPKeys + 1 : 0;
        const bool full = r1 == r0 + 16 * NB && q0 + qa + (r1 - 1) / G < a.total_q;
        nomask_tiles = (full && p0 >= 0) ? (p0 + 1) / kPKeys : 0;
    }
    wave_tiles = __builtin_amdgcn_readfirstlane(wave_tiles);
    nomask_tiles = __builtin_amdgcn_readfirstlane(nomask_tiles);

    V8 qb[NB][KS];
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (qvalid[c])
                w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                    ((int64_t)qrow[c] * Hq + qhead[c]) * D + 32 * ks + 8 * quad);
            if (qneg) w = make_uint4(w.x ^ 0x80008000u, w.y ^ 0x80008000u, w.z ^ 0x80008000u, w.w ^ 0x80008000u);
            qb[c][ks] = __builtin_bit_cast(V8, w);
        }

    // The block table is not written during the kernel: read it through the
    // constant address space, so the (wave-uniform) entries come in by scalar
    // loads, which the vector-load counter does not track (a wait for a table
    // entry is then not a wait for every K/V load issued before it).
    typedef const __attribute__((address_space(4))) int32_t* ConstTable;
    const ConstTable table = (ConstTable)(a.block_tables + (int64_t)s * a.table_stride);
    const u32x4* kg = reinterpret_cast<const u32x4*>(a.k_cache);
    const u32x4* vg = reinterpret_cast<const u32x4*>(a.v_cache);

    // Block ids of a tile (a 32-key tile spans one block of 32 or two of 16),
    // read one iteration before the tile's K/V loads need them.  Keys at or
    // past the context end are zeros, never loaded; only the last tile checks.
    const int last_blk = (n + BS - 1) / BS - 1;
    auto load_ids = [&](int kt) {
        const int f = (kt * kPKeys) / BS;
        return make_int2(table[min(f, last_blk)], BS == kPKeys ? 0 : table[min(f + 1, last_blk)]);
    };
    // K: piece tid + kPThreads c is key (tid + kPThreads c) / CPR, 16-byte
    // chunk (tid + kPThreads c) % CPR, stored at LDS row 16 h + 4 a + i for key
    // 8 a + 4 h + i.  V: unit u = tid % VU is keys 2 (u % 16), 2 (u % 16) + 1 of
    // d chunk u / 16.
    int kkey[KPT], ksrc[KPT], kdst[KPT];
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
        const int piece = tid + kPThreads * c, key = piece / CPR;
        kkey[c] = key;
        ksrc[c] = (key % BS) * CPR + piece % CPR;
        const int row = 16 * ((key >> 2) & 1) + 4 * (key >> 3) + (key & 3);
        kdst[c] = row * KROW + ((piece % CPR) ^ kswz<D>(row)) * 16;
    }
    const int vu = tid % VU, vkey = 2 * (vu % 16), vcd = vu / 16;
    // Byte offsets of this thread's 8 two-key words in a transposed V buffer
    // (row d = 8 vcd + r, keys vkey and vkey + 1; see vrow_phys and vchunk).
    int vst[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int pr = vrow_phys(vcd * 8 + r);
        vst[r] = pr * VROW + ((vkey >> 3) ^ vchunk(pr)) * 16 + (vkey & 7) * 2;
    }
    const int64_t blk_stride = (int64_t)Hkv * BS * CPR, head_off = (int64_t)g * BS * CPR;
    // The keys of K piece c (tid + kPThreads c) lie in one block of the tile
    // when a piece index spans at most a block (D = 128: 16 keys per c): that
    // block's base is then wave-uniform, and the piece's address a 32-bit
    // lane offset from it.
    constexpr int SETK = kPThreads / CPR;
    constexpr bool KUNI = SETK <= BS;
    // Loads are unconditional (a key past the context end reads its clamped
    // block's stale row); the store to LDS zeroes the V values of such keys,
    // once the loads have arrived.  gload returns the tile's first key.
    auto gload = [&](int kt, int2 ids, u32x4 (&r)[SR], int& t0) {
        const int64_t o0 = ids.x * blk_stride + head_off, o1 = ids.y * blk_stride + head_off;   // uniform
        t0 = kt * kPKeys;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            if constexpr (KUNI) {
                const uint8_t* kb = reinterpret_cast<const uint8_t*>(kg + ((c * SETK) / BS ? o1 : o0));
                r[c] = *reinterpret_cast<const u32x4*>(kb + (uint32_t)ksrc[c] * 16u);
            } else {
                r[c] = kg[(kkey[c] < BS ? o0 : o1) + ksrc[c]];
            }
        }
        const u32x4* p = vg + (vkey < BS ? o0 : o1) + (vkey % BS) * CPR + vcd;
        r[KPT] = p[0];
        r[KPT + 1] = p[CPR];
    };
    auto lstore = [&](int b, const u32x4 (&r)[SR], int t0) {
        uint8_t* kb = s_mem + b * KBUF;
        // K rows past the context end stay as loaded: their scores are masked
        // to -inf before use.  V rows there are zeroed (weight 0 times a stale
        // NaN would still be NaN), on the tile that holds the context end only.
#pragma unroll
        for (int c = 0; c < KPT; ++c) *reinterpret_cast<u32x4*>(kb + kdst[c]) = r[c];
        uint8_t* vb = s_mem + 2 * KBUF + b * VBUF;
        u32x4 v0 = r[KPT], v1 = r[KPT + 1];
        if (t0 + kPKeys > n) {                     // uniform
            const u32x4 z = {0u, 0u, 0u, 0u};
            v0 = t0 + vkey < n ? v0 : z;
            v1 = t0 + vkey + 1 < n ? v1 : z;
        }
        const uint32_t w0[4] = {v0[0], v0[1], v0[2], v0[3]};
        const uint32_t w1[4] = {v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // d = 8 cd + 2e from the low halves, 8 cd + 2e + 1 from the high halves: the two keys' values.
            *reinterpret_cast<uint32_t*>(vb + vst[2 * e]) = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
            *reinterpret_cast<uint32_t*>(vb + vst[2 * e + 1]) = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
        }
    };

    f32x4 acc[NB][DB];
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[c][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_l[NB], l_l[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        m_l[c] = -__FLT_MAX__;   // finite: the first tile's exponents are +huge, so it sets the reference
        l_l[c] = 0.f;
    }

    // This lane's LDS read offsets: its K row col at 16-byte chunk 4 ks + quad
    // (the rows 16 + col of the second half add 16 KROW), and its transposed V
    // row col of an even or an odd 16-row block (vrow_phys depends on the
    // block's parity, not its index).
    int krd[KS], vrd[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) krd[ks] = col * KROW + ((4 * ks + quad) ^ kswz<D>(col)) * 16;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int pr = vrow_phys(16 * par + col) - 16 * par;
        vrd[par] = pr * VROW + 16 * (quad ^ vchunk(pr));
    }

    // The bf16 pairs (-1, 0) and (0, -1) of split_pair, opaque to the compiler.
    uint32_t sel0 = 0x0000BF80u, sel1 = 0xBF800000u;
    asm("" : "+v"(sel0), "+v"(sel1));

    auto compute = [&](int b, int kt) {
        const uint8_t* kb = s_mem + b * KBUF;
        const uint8_t* vb = s_mem + 2 * KBUF + b * VBUF;
        f32x4 sc[NB][2];
#pragma unroll
        for (int c = 0; c < NB; ++c) sc[c][0] = sc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const V8 a0 = *reinterpret_cast<const V8*>(kb + krd[ks]);
            const V8 a1 = *reinterpret_cast<const V8*>(kb + 16 * KROW + krd[ks]);
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                sc[c][0] = mma<BF16>(a0, qb[c][ks], sc[c][0]);
                sc[c][1] = mma<BF16>(a1, qb[c][ks], sc[c][1]);
            }
        }
        // Lane (col, quad), half h, i: key kt * 32 + 8 quad + 4 h + i, weight j = 4 h + i.
        // Keys j < lim of the lane's 8 are at or before its row's query
        // (every key on the tiles before the diagonal).
        const int t0 = kt * kPKeys + 8 * quad;
        const bool nomask = kt < nomask_tiles;     // uniform
        // Exponents x = s sl2 - m of the lane's 8 keys per row (one fma each),
        // relative to the row's reference m.  The reference moves only when a
        // score exceeds it by more than kPTau: a lane that sees no such score
        // needs no row maximum, so the maximum and its reduction over the
        // row's 4 lanes run only when some lane of the wave sees one (the
        // first tile of every row, where m starts at -FLT_MAX, and rare later
        // tiles).  Masked keys are -inf and stay -inf (sl2 > 0 and finite).
        float sv[NB][8], x[NB][8];
        bool hot = false;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[c][j] = sc[c][j >> 2][j & 3];
            if (!nomask) {
                // Keys past the row's query (and every key of an unused row)
                // get -inf: weight exp2(-inf) = 0.  Stale K rows past the
                // context end only ever reach this branch.
                const int lim = qvalid[c] ? qpos[c] - t0 : -1;
#pragma unroll
                for (int j = 0; j < 8; ++j) sv[c][j] = j <= lim ? sv[c][j] : -INFINITY;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) x[c][j] = __builtin_fmaf(sv[c][j], sl2, -m_l[c]);
            hot |= vmax8(x[c]) > kPTau;
        }
        if (__builtin_amdgcn_ballot_w64(hot)) {
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                const float mt = pmax32(pmax16(vmax8(sv[c]))) * sl2;   // the row's scaled maximum
                const bool need = mt > m_l[c] + kPTau;                 // uniform over the row's 4 lanes
                if (need) {
                    const float alpha = __builtin_amdgcn_exp2f(m_l[c] - mt);   // 0 on the first tile
                    l_l[c] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[c][db] *= alpha;
                    m_l[c] = mt;
#pragma unroll
                    for (int j = 0; j < 8; ++j) x[c][j] = __builtin_fmaf(sv[c][j], sl2, -mt);
                }
            }
        }
        uint4 ph[NB], pl[NB];
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            float pw[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pw[j] = __builtin_amdgcn_exp2f(x[c][j]);   // <= 2^8 (about); 0 for a masked key
            l_l[c] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
            split_pair<BF16>(pw[0], pw[1], sel0, sel1, ph[c].x, pl[c].x);
            split_pair<BF16>(pw[2], pw[3], sel0, sel1, ph[c].y, pl[c].y);
            split_pair<BF16>(pw[4], pw[5], sel0, sel1, ph[c].z, pl[c].z);
            split_pair<BF16>(pw[6], pw[7], sel0, sel1, ph[c].w, pl[c].w);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            // Row 16 db + col, keys 8 quad .. 8 quad + 7: one 16-byte chunk.
            const V8 av = *reinterpret_cast<const V8*>(vb + db * 16 * VROW + vrd[db & 1]);
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                acc[c][db] = mma<BF16>(av, __builtin_bit_cast(V8, ph[c]), acc[c][db]);
                acc[c][db] = mma<BF16>(av, __builtin_bit_cast(V8, pl[c]), acc[c][db]);
            }
        }
    };

    // Two register stages: the global loads of tile kt + 2 are issued while
    // tile kt is consumed, and stored to LDS one iteration later, so each
    // tile's loads have a whole iteration to arrive.  Every iteration issues
    // the same loads and stores (past the last tile it reloads the last tile,
    // a cache hit, and stores it where nothing reads it): the wait before a
    // store to LDS is then for that tile's loads only, not for the ones just
    // issued (the vector-load counter is in order, and a path that skips a
    // load or its store would force a wait for all of them).
    // LDS stays double buffered: the barrier that ends an iteration separates
    // the reads of one buffer from the next store into it.  A wave whose rows
    // are all past a tile's keys only stages and waits.
    u32x4 st_a[SR], st_b[SR];
    int t_a = 0, t_b = 0;
    if (NT > 0) {                                  // uniform; rows with no key still get their output below
    gload(0, load_ids(0), st_a, t_a);
    lstore(0, st_a, t_a);
    gload(min(1, NT - 1), load_ids(min(1, NT - 1)), st_a, t_a);   // tile 1 in flight in st_a
    int2 ids_next = load_ids(min(2, NT - 1));      // block ids of the next tile to load
    __syncthreads();
    // cur holds tile kt + 1's loads in flight; nxt is free.
    auto step = [&](int kt, u32x4 (&cur)[SR], int& t_cur, u32x4 (&nxt)[SR], int& t_nxt) {
        gload(min(kt + 2, NT - 1), ids_next, nxt, t_nxt);
        ids_next = load_ids(min(kt + 3, NT - 1));
        if (kt < wave_tiles) compute(kt & 1, kt);
        lstore((kt + 1) & 1, cur, t_cur);       // past the last tile: a copy nobody reads
        __syncthreads();
    };
    // Steps in pairs, both unconditional (an odd NT ends with a step that only
    // stages a copy: no wave computes tile NT), so the staging registers carry
    // over the loop edge without copies, which would wait for their loads.
    for (int kt = 0; kt < NT; kt += 2) {
        step(kt, st_a, t_a, st_b, t_b);
        step(kt + 1, st_b, t_b, st_a, t_a);
    }
    }

    // ---- finalize: row totals, normalised output, lse ----
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        const float lt = psum32(psum16(l_l[c]));
        if (!qvalid[c]) continue;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int64_t row = (int64_t)qrow[c] * Hq + qhead[c];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 16 + 4 * quad;
            const float o0 = acc[c][db][0] * inv, o1 = acc[c][db][1] * inv, o2 = acc[c][db][2] * inv,
                        o3 = acc[c][db][3] * inv;
            if (a.out_dtype == kOutF32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + row * D + d0) = make_float4(o0, o1, o2, o3);
            } else if (a.out_dtype == kOutBF16) {
                typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
                const bf16x4v v = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
                *reinterpret_cast<bf16x4v*>(reinterpret_cast<__bf16*>(a.out) + row * D + d0) = v;
            } else {
                typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
                const f16x4v v = {(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3};
                *reinterpret_cast<f16x4v*>(reinterpret_cast<_Float16*>(a.out) + row * D + d0) = v;
            }
        }
        if (a.lse && quad == 0) a.lse[row] = lt > 0.f ? (m_l[c] + __builtin_amdgcn_logf(lt)) * kPLn2 : -INFINITY;
    }
}

template <int D, int BS, bool BF16>
static hipError_t prefill_t(const PrefillArgs& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.grid_tiles * a.num_kv_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((paged_prefill_kernel<D, BS, BF16>), dim3((unsigned)grid), dim3(kPThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, bool bf16, hipStream_t stream) {
    if (a.num_seqs > kPrefillMaxSeqs || a.num_kv_heads < 1 || a.num_q_heads % a.num_kv_heads ||
        a.query_tile != prefill_query_tile(a.num_q_heads / a.num_kv_heads))
        return hipErrorInvalidValue;
    if (head_dim == 128) {
        if (block_size == 16) return bf16 ? prefill_t<128, 16, true>(a, stream) : prefill_t<128, 16, false>(a, stream);
        if (block_size == 32) return bf16 ? prefill_t<128, 32, true>(a, stream) : prefill_t<128, 32, false>(a, stream);
    } else if (head_dim == 64) {
        if (block_size == 16) return bf16 ? prefill_t<64, 16, true>(a, stream) : prefill_t<64, 16, false>(a, stream);
        if (block_size == 32) return bf16 ? prefill_t<64, 32, true>(a, stream) : prefill_t<64, 32, false>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
