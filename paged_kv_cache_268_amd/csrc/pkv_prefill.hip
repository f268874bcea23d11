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
// Work decomposition.  One 256-thread workgroup (4 wave64) per (64-query tile
// of a chunk, q head); wave w owns 16 queries.  The workgroup walks 32-key
// tiles from position 0 to its last query's position.  Each K/V tile is read
// once per workgroup (16-byte loads through the block table) into LDS, double
// buffered, with the loads issued two tiles ahead (two register stages).
// K sits row-major (rows padded by 16 bytes), V transposed ([d][key], rows
// padded to 72 bytes).  Waves 2-3 load K (four 16-byte pieces per thread);
// waves 0-1 load V as units of 4 consecutive keys x 8 d values and store, for
// each d, the 4 keys as one 8-byte word: with 18-dword rows those stores hit
// every LDS bank once per half wave (2-byte stores of a transposed row would
// conflict 8- to 16-fold).  Keys at or past the context end are written as
// zeros, never loaded.
//
// Both contractions run on v_mfma_f32_16x16x32 (bf16 or f16 inputs, fp32
// accumulation):
//   S^T = K Q^T: A = 16 keys x 32 d from LDS, B = the wave's 16 queries x 32 d
//   held in registers; two 16-key halves per tile.  Lane l receives the scores
//   of keys 4(l/16) + r and 16 + 4(l/16) + r (r = 0..3) for query l % 16.
//   O^T += V^T P^T: those 8 weights are already lane l's B operand (query
//   l % 16, 8 keys), and the A operand is the same 8 keys of one d row of the
//   transposed V tile (two 8-byte LDS reads), D/16 output blocks.
// Softmax per query column: a reference max that moves only when a score
// exceeds it by more than 8 (log2 units), so the accumulator rescale is a rare
// event (skipped for the whole wave when no column needs it) and every weight
// stays <= 2^8.  The weights enter the second product as a bf16 (f16) pair hi + lo with
// hi = round(p) and lo = round(p - hi), two MFMAs per block: one rounded
// 16-bit weight carries up to 2^-9 relative error, which is too coarse for
// outputs checked to 2e-3; the pair carries about 2^-17.  The running max,
// the rescale and the weight sum stay in fp32 per query column (reduced over
// the 4 lanes of a column with permlane swaps).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"
#include "pkv_prefill.h"

namespace pkv {
namespace {

constexpr int kPThreads = 256;
constexpr int kPKeys = 32;                      // keys per tile
constexpr float kPLog2e = 1.4426950408889634f;
constexpr float kPLn2 = 0.6931471805599453f;
constexpr float kPTau = 8.0f;                   // lazy-rescale threshold (log2 units)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

template <bool BF16> struct PType { using v8 = f16x8v; using e = _Float16; };
template <> struct PType<true> { using v8 = bf16x8v; using e = __bf16; };

template <bool BF16>
__device__ __forceinline__ f32x4 mma(typename PType<BF16>::v8 a, typename PType<BF16>::v8 b, f32x4 c) {
    if constexpr (BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Reductions across lanes l ^ 16 and l ^ 32 (the 4 lanes of one score column).
__device__ __forceinline__ float pmax16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pmax32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float psum16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float psum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup i runs on XCD i % 8; consecutive logical ids share an XCD (its L2).
__device__ __forceinline__ int prefill_xcd_remap(int i, int n) {
    const int per = n / kNumXcds;
    if (i < per * kNumXcds) return (i % kNumXcds) * per + i / kNumXcds;
    return i;
}

}  // namespace

template <int D, int BS, bool BF16>
// Four waves per SIMD (at most 128 VGPRs; 128 used at D = 128, no spills):
// with the 35.8 KB of LDS per workgroup that is 4 workgroups per CU, each with
// two tiles' loads in flight.
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
paged_prefill_kernel(PrefillArgs a) {
    using V8 = typename PType<BF16>::v8;
    using E = typename PType<BF16>::e;
    constexpr int KS = D / 32;                    // k-steps of S^T
    constexpr int DB = D / 16;                    // 16-row output blocks of O^T
    constexpr int KROW = D * 2 + 16;              // bytes per K row in LDS
    constexpr int VROW = kPKeys * 2 + 8;          // bytes per transposed V row (8-byte aligned)
    constexpr int KBUF = kPKeys * KROW, VBUF = D * VROW;
    constexpr int CPR = D / 8;                    // 16-byte pieces per K/V row
    constexpr int HT = kPThreads / 2;             // threads of the K half and of the V half
    constexpr int KPT = kPKeys * CPR / HT;        // K pieces per K-half thread
    constexpr int VU = (kPKeys / 4) * CPR;        // V units (4 keys x 8 d) per tile
    constexpr int VPT = (VU + HT - 1) / HT;       // V units per V-half thread
    constexpr int SR = KPT > 4 * VPT ? KPT : 4 * VPT;   // staging registers per thread
    static_assert(KPT * HT == kPKeys * CPR && VU <= VPT * HT, "tile shape");
    constexpr int LDS = 2 * (KBUF + VBUF);
    static_assert(LDS >= (kPrefillMaxSeqs + 1) * 4, "tile prefix fits the tile buffers");
    __shared__ __align__(16) uint8_t s_mem[LDS];
    __shared__ int s_wsum[kPThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int B = a.num_seqs, Hq = a.num_q_heads;

    // ---- query tiles per sequence, prefix in LDS (aliases the tile buffers) ----
    int* s_pre = reinterpret_cast<int*>(s_mem);
    int running = 0;
    for (int base = 0; base < B; base += kPThreads) {
        const int s = base + tid;
        int v = 0;
        if (s < B) {
            const int m = a.cu_q[s + 1] - a.cu_q[s];
            v = m > 0 ? (m + kPrefillQ - 1) / kPrefillQ : 0;
        }
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
        for (int w = 0; w < kPThreads / 64; ++w) {
            woff += w < wave ? s_wsum[w] : 0;
            tot += s_wsum[w];
        }
        if (s < B) s_pre[s] = running + woff + x - v;
        running += tot;
        __syncthreads();
    }
    if (tid == 0) s_pre[B] = running;
    __syncthreads();
    const int T = s_pre[B];
    const int lwg = prefill_xcd_remap(blockIdx.x, gridDim.x);
    const int h = lwg % Hq;
    const int tl = lwg / Hq;
    if (tl >= T) return;                           // uniform over the workgroup
    const int tile = T - 1 - tl;                   // later (longer) tiles first
    int sl = 0, sh = B;                            // pre[sl] <= tile < pre[sh]
    while (sh - sl > 1) {
        const int mid = (sl + sh) >> 1;
        if (s_pre[mid] <= tile) sl = mid; else sh = mid;
    }
    const int s = sl;
    const int qt = tile - s_pre[s];
    __syncthreads();                               // prefix dead: LDS now holds K/V tiles

    const int Hkv = a.num_kv_heads, G = Hq / Hkv, g = h / G;
    const int n = min(max(a.context_lens[s], 0), a.max_context_len);
    const int q0 = a.cu_q[s];
    const int m = max(a.cu_q[s + 1] - q0, 0);
    const int base_pos = n - m;                    // position of chunk row 0
    const int qa = qt * kPrefillQ;
    const int nq = min(kPrefillQ, m - qa);
    const int last_pos = base_pos + qa + nq - 1;
    const int NT = last_pos >= 0 ? (last_pos + kPKeys) / kPKeys : 0;

    const int col = lane & 15, quad = lane >> 4;
    const int qi = qa + wave * 16 + col;           // this lane's chunk query (score column)
    const bool qvalid = qi < m && q0 + qi < a.total_q;
    const int qpos = base_pos + qi;
    const float sl2 = a.scale * kPLog2e;
    // Tiles [0, nomask_tiles) need no causal mask for this wave: all 16 of its
    // queries are real and the tile's last key precedes its first query.
    const int wq0 = qa + wave * 16;
    const bool wave_full = wq0 + 16 <= m && q0 + wq0 + 16 <= a.total_q;
    const int wave_pos0 = base_pos + wq0;
    const int nomask_tiles = (wave_full && wave_pos0 >= 0) ? (wave_pos0 + 1) / kPKeys : 0;

    V8 qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (qvalid)
            w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                ((int64_t)(q0 + qi) * Hq + h) * D + 32 * ks + 8 * quad);
        qb[ks] = __builtin_bit_cast(V8, w);
    }

    const int32_t* table = a.block_tables + (int64_t)s * a.table_stride;
    const uint4* kg = reinterpret_cast<const uint4*>(a.k_cache);
    const uint4* vg = reinterpret_cast<const uint4*>(a.v_cache);

    // Block ids of a tile (a 32-key tile spans one block of 32 or two of 16):
    // lane l loads entry (first + (l & 1)) as a vector load one iteration
    // before the tile's K/V loads need it, so the table read is off the
    // critical path; read back with v_readlane, so the two block bases are
    // wave-uniform (scalar registers) and a lane's offset inside a block is
    // the same for every tile (computed once below).  Keys at or past the
    // context end are zeros, never loaded; only the last tile checks.
    const int last_blk = (n + BS - 1) / BS - 1;
    auto load_ids = [&](int kt) {
        return table[min((kt * kPKeys) / BS + (lane & 1), last_blk)];
    };
    const bool k_half = wave >= 2;                 // uniform per wave
    const int ht = tid & (HT - 1);
    // K half: piece ht + HT c is key (ht + HT c) / CPR, chunk (ht + HT c) % CPR;
    // the keys of one c lie in one block (KEYS_PER_C divides the block size).
    // V half: unit ht + HT c is keys 4 ((ht + HT c) % 8) .. +3, chunk (ht + HT c) / 8.
    constexpr int KEYS_PER_C = HT / CPR;
    static_assert(HT % CPR == 0 && BS % KEYS_PER_C == 0, "a K piece group stays inside one block");
    int koff[KPT], vkey[VPT], voff[VPT];           // offsets in 16-byte units inside a block
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
        const int piece = ht + HT * c;
        koff[c] = ((piece / CPR) % BS) * CPR + piece % CPR;
    }
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
        const int u = ht + HT * c;
        vkey[c] = 4 * (u % 8);
        voff[c] = (vkey[c] % BS) * CPR + u / 8;
    }
    const int64_t blk_stride = (int64_t)Hkv * BS * CPR, head_off = (int64_t)g * BS * CPR;
    auto gload = [&](int kt, int32_t ids, uint4 (&r)[SR]) {
        const int32_t b0 = __builtin_amdgcn_readlane(ids, 0), b1 = __builtin_amdgcn_readlane(ids, 1);
        const int t0 = kt * kPKeys;
        const bool full = t0 + kPKeys <= n;        // uniform: every key of the tile is cached
        if (k_half) {
            const uint4* p0 = kg + b0 * blk_stride + head_off;
            const uint4* p1 = kg + b1 * blk_stride + head_off;
#pragma unroll
            for (int c = 0; c < KPT; ++c) {
                const uint4* p = (BS == kPKeys || (c + 1) * KEYS_PER_C <= BS) ? p0 : p1;
                const int key = (ht + HT * c) / CPR;
                r[c] = (full || t0 + key < n) ? p[koff[c]] : make_uint4(0, 0, 0, 0);
            }
        } else {
            const uint4* p0 = vg + b0 * blk_stride + head_off;
            const uint4* p1 = vg + b1 * blk_stride + head_off;
#pragma unroll
            for (int c = 0; c < VPT; ++c) {
                const int u = ht + HT * c;
                const uint4* p = ((BS == kPKeys || vkey[c] < BS) ? p0 : p1) + voff[c];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    r[4 * c + kk] = (u < VU && (full || t0 + vkey[c] + kk < n)) ? p[kk * CPR] : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto lstore = [&](int b, const uint4 (&r)[SR]) {
        if (k_half) {
            uint8_t* kb = s_mem + b * KBUF;
#pragma unroll
            for (int c = 0; c < KPT; ++c) {
                const int piece = ht + HT * c;
                *reinterpret_cast<uint4*>(kb + (piece / CPR) * KROW + (piece % CPR) * 16) = r[c];
            }
        } else {
            uint8_t* vb = s_mem + 2 * KBUF + b * VBUF;
#pragma unroll
            for (int c = 0; c < VPT; ++c) {
                const int u = ht + HT * c;
                if (u >= VU) continue;
                const int q4 = u % 8, cd = u / 8;
                const uint32_t w0[4] = {r[4 * c].x, r[4 * c].y, r[4 * c].z, r[4 * c].w};
                const uint32_t w1[4] = {r[4 * c + 1].x, r[4 * c + 1].y, r[4 * c + 1].z, r[4 * c + 1].w};
                const uint32_t w2[4] = {r[4 * c + 2].x, r[4 * c + 2].y, r[4 * c + 2].z, r[4 * c + 2].w};
                const uint32_t w3[4] = {r[4 * c + 3].x, r[4 * c + 3].y, r[4 * c + 3].z, r[4 * c + 3].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // d = 8 cd + 2e from the low halves, 8 cd + 2e + 1 from the high halves
                    const uint2 lo = make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u),
                                                __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u));
                    const uint2 hi = make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u),
                                                __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u));
                    *reinterpret_cast<uint2*>(vb + (cd * 8 + 2 * e) * VROW + q4 * 8) = lo;
                    *reinterpret_cast<uint2*>(vb + (cd * 8 + 2 * e + 1) * VROW + q4 * 8) = hi;
                }
            }
        }
    };

    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_l = -INFINITY, l_l = 0.f;

    auto compute = [&](int b, int kt) {
        const uint8_t* kb = s_mem + b * KBUF;
        const uint8_t* vb = s_mem + 2 * KBUF + b * VBUF;
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const V8 a0 = *reinterpret_cast<const V8*>(kb + col * KROW + (32 * ks + 8 * quad) * 2);
            const V8 a1 = *reinterpret_cast<const V8*>(kb + (16 + col) * KROW + (32 * ks + 8 * quad) * 2);
            c0 = mma<BF16>(a0, qb[ks], c0);
            c1 = mma<BF16>(a1, qb[ks], c1);
        }
        const int t0 = kt * kPKeys + 4 * quad;
        float x[8];
        float mx = -INFINITY;
        if (kt < nomask_tiles) {
            // Every key of the tile is at or before every query of the wave.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = c0[r] * sl2;
                x[4 + r] = c1[r] * sl2;
                mx = fmaxf(mx, fmaxf(x[r], x[4 + r]));
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = (qvalid && t0 + r <= qpos) ? c0[r] * sl2 : -INFINITY;
                x[4 + r] = (qvalid && t0 + 16 + r <= qpos) ? c1[r] * sl2 : -INFINITY;
                mx = fmaxf(mx, fmaxf(x[r], x[4 + r]));
            }
        }
        mx = pmax32(pmax16(mx));                       // column max of this tile
        const bool need = mx > m_l + kPTau;            // uniform over the column's 4 lanes
        const float m_new = need ? mx : m_l;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_l - m_new) : 1.f;   // 0 while nothing was seen
        const float ref = m_new == -INFINITY ? 0.f : m_new;
        V8 ph, pl;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[i] - ref);    // <= 2^8; 0 for a masked key
            ps += p;
            const E hi = (E)p;
            ph[i] = hi;
            pl[i] = (E)(p - (float)hi);
        }
        l_l = l_l * alpha + ps;
        m_l = m_new;
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint8_t* row = vb + (db * 16 + col) * VROW;
            const uint2 lo4 = *reinterpret_cast<const uint2*>(row + 8 * quad);        // keys 4 quad + 0..3
            const uint2 hi4 = *reinterpret_cast<const uint2*>(row + 32 + 8 * quad);   // keys 16 + 4 quad + 0..3
            const V8 av = __builtin_bit_cast(V8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
            acc[db] = mma<BF16>(av, ph, acc[db]);
            acc[db] = mma<BF16>(av, pl, acc[db]);
        }
    };

    // Two register stages: the global loads of tile kt + 2 are issued while
    // tile kt is consumed, and stored to LDS one iteration later, so each
    // tile's loads have a whole iteration to arrive.  LDS stays double
    // buffered: the barrier that ends an iteration separates the reads of one
    // buffer from the next store into it.
    uint4 st_a[SR], st_b[SR];
    int32_t ids_next = 0;                          // block ids of the next tile to load
    if (NT > 0) {
        gload(0, load_ids(0), st_a);
        lstore(0, st_a);
    }
    if (NT > 1) gload(1, load_ids(1), st_a);       // tile 1 in flight in st_a
    if (NT > 2) ids_next = load_ids(2);
    __syncthreads();
    // cur holds tile kt + 1's loads in flight; nxt is free.
    auto step = [&](int kt, uint4 (&cur)[SR], uint4 (&nxt)[SR]) {
        if (kt + 2 < NT) {
            gload(kt + 2, ids_next, nxt);
            if (kt + 3 < NT) ids_next = load_ids(kt + 3);
        }
        compute(kt & 1, kt);
        if (kt + 1 < NT) lstore((kt + 1) & 1, cur);
        __syncthreads();
    };
    for (int kt = 0; kt < NT; kt += 2) {
        step(kt, st_a, st_b);
        if (kt + 1 < NT) step(kt + 1, st_b, st_a);
    }

    // ---- finalize: column totals, normalised output, lse ----
    const float lt = psum32(psum16(l_l));
    if (qvalid) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int64_t row = (int64_t)(q0 + qi) * Hq + h;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 16 + 4 * quad;
            const float o0 = acc[db][0] * inv, o1 = acc[db][1] * inv, o2 = acc[db][2] * inv, o3 = acc[db][3] * inv;
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
        if (a.lse && quad == 0) a.lse[row] = lt > 0.f ? (m_l + __builtin_amdgcn_logf(lt)) * kPLn2 : -INFINITY;
    }
}

template <int D, int BS, bool BF16>
static hipError_t prefill_t(const PrefillArgs& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.grid_tiles * a.num_q_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((paged_prefill_kernel<D, BS, BF16>), dim3((unsigned)grid), dim3(kPThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, bool bf16, hipStream_t stream) {
    if (a.num_seqs > kPrefillMaxSeqs) return hipErrorInvalidValue;
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
