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
// Work decomposition.  One 256-thread workgroup (4 wave64) per work item
// (sequence s, kv head g, partition p).  A partition is P consecutive tokens
// [p*P, min((p+1)*P, len)); it is cut into 16-token tiles (a tile never
// crosses a block because block_size is 16 or 32 and P a multiple of it), and
// wave w takes tiles w, w+4, w+8, ...
//
// Lane layout inside a wave.  A K (or V) row of one token is D 16-bit values
// = D*2 bytes.  LPR = D/8 lanes share a row, each holding one 16-byte slice
// (8 values, d in [8c, 8c+8)); a wave load instruction therefore covers
// RPI = 64/LPR consecutive rows = 1 KiB of contiguous memory.  A 16-token tile
// of one (block, kv head) is 16*D*2 bytes contiguous and takes NI = 16/RPI
// load instructions for K and NI for V.  Each lane keeps the G q heads of the
// group for its own d-slice in registers, so a K/V row is read from HBM once
// per kv head, not once per q head.
//
// QK: per lane, 4 packed dot2 (fp32 accumulate) per head per row, then a
// butterfly over the LPR lanes of the row with DPP row operations.
// Softmax: each row-group (the LPR lanes sharing rows) runs its own online
// softmax in the log2 domain; the running max is only moved when a tile's max
// exceeds it by more than TAU, so a rescale of the accumulator is rare, and
// every weight stays <= 2^TAU.  Rows past the context are excluded (their
// weight is 0 by selection and their V is not used), so stale or NaN data in
// unused slots never reaches the sums.
// End of a work item: row-group states merge by shuffles, the 4 waves merge
// through LDS, and the result is either the final output (a one-partition
// sequence) or a normalised partial plus its log2-domain lse in the workspace
// for the merge kernel.
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DPP controls (row = 16 lanes).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // reverse within 8 lanes
constexpr int kDppMirror = 0x140;      // reverse within 16 lanes

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    // After the first two steps all lanes of a quad agree, so a mirror inside
    // 8 (then 16) lanes pairs each quad with the other quad (half) of the row.
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kDppXor1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kDppXor2, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kDppHalfMirror, 0xF, 0xF, false));
    if constexpr (LPR == 16)
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kDppMirror, 0xF, 0xF, false));
    return x;
}

template <bool BF16>
__device__ __forceinline__ float dot8(const uint4 k, const uint4 q, float acc) {
    if constexpr (BF16) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x), __builtin_bit_cast(bf16x2, q.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y), __builtin_bit_cast(bf16x2, q.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z), __builtin_bit_cast(bf16x2, q.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w), __builtin_bit_cast(bf16x2, q.w), acc, false);
    } else {
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, k.x), __builtin_bit_cast(f16x2, q.x), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, k.y), __builtin_bit_cast(f16x2, q.y), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, k.z), __builtin_bit_cast(f16x2, q.z), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, k.w), __builtin_bit_cast(f16x2, q.w), acc, false);
    }
    return acc;
}

// Two packed 16-bit values -> two floats (exact widening).
template <bool BF16>
__device__ __forceinline__ void widen2(uint32_t w, float& lo, float& hi) {
    if constexpr (BF16) {
        lo = __builtin_bit_cast(float, w << 16);
        hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
    } else {
        f16x2 h = __builtin_bit_cast(f16x2, w);
        lo = (float)h.x;
        hi = (float)h.y;
    }
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

// Work-group id -> logical work item id.  The hardware hands workgroup i to
// XCD i % 8; this makes consecutive logical ids land on one XCD (and so share
// its L2) -- sequences that share prefix blocks sit next to each other.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n) {
    const int64_t per = n / kNumXcds;
    if (i < per * kNumXcds) return (i % kNumXcds) * per + i / kNumXcds;
    return i;
}

template <int D, int BS, int GP, bool BF16>
__global__ void __launch_bounds__(kThreads)
paged_decode_partition_kernel(DecodeArgs a) {
    constexpr int LPR = D / 8;            // lanes per K/V row
    constexpr int RPI = 64 / LPR;         // rows per wave load instruction
    constexpr int NI = kTile / RPI;       // load instructions per tile (K or V)
    static_assert(NI * RPI == kTile, "tile shape");

    const int64_t n_items = (int64_t)a.num_seqs * a.num_kv_heads * a.max_parts;
    const int64_t item = xcd_remap(blockIdx.x, n_items);
    const int s = (int)(item % a.num_seqs);
    const int64_t rest = item / a.num_seqs;
    const int g = (int)(rest % a.num_kv_heads);
    const int p = (int)(rest / a.num_kv_heads);

    // A length outside [0, max_context_len] breaks the caller's contract; it
    // is clamped so that no access leaves the declared table and workspace.
    const int ctx = min(max(a.context_lens[s], 0), a.max_context_len);
    const int nparts = (ctx + a.part_size - 1) / a.part_size;
    // Partition 0 always runs, so an empty context still gets its output.
    if (p >= (nparts > 0 ? nparts : 1)) return;

    const int t_lo = p * a.part_size;
    const int t_hi = min(t_lo + a.part_size, ctx);
    const int n_tiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;

    const int lane = threadIdx.x & 63;
    // Wave index as a uniform (scalar) value, so loops over tiles stay scalar.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % LPR;              // 16-byte slice of the row
    const int r = lane / LPR;              // row inside a load instruction
    const int G = a.num_q_heads / a.num_kv_heads;
    const int h0 = g * G;

    // q slices of the group's heads (zero for padded heads h >= G).
    uint4 qv[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        if (h < G) {
            const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)s * a.num_q_heads + h0 + h) * D + c * 8;
            qv[h] = *reinterpret_cast<const uint4*>(qp);
        } else {
            qv[h] = make_uint4(0, 0, 0, 0);
        }
    }

    float m[GP], l[GP], acc[GP][8];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    const float sl2 = a.scale * kLog2e;
    const int32_t* table = a.block_tables + (int64_t)s * a.table_stride;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache);
    // Element offset of this lane's slice inside a tile (row r of instruction 0).
    const int lane_off = r * D + c * 8;

    // Tiles of this wave: j = wave + WAVES * it, it in [0, n_w).
    const int n_w = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;

    auto tile_base = [&](int it, int32_t blk) -> int64_t {
        const int t0 = t_lo + (wave + kWaves * it) * kTile;
        return (((int64_t)blk * a.num_kv_heads + g) * BS + (t0 % BS)) * D + lane_off;
    };

    auto compute_tile = [&](int it, const uint4 (&kb)[NI], const uint4 (&vb)[NI]) {
        const int t0 = t_lo + (wave + kWaves * it) * kTile;
        const bool full = t0 + kTile <= t_hi;
        float x[NI][GP];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int h = 0; h < GP; ++h) x[i][h] = row_sum<LPR>(dot8<BF16>(kb[i], qv[h], 0.f)) * sl2;
        }
        bool valid[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) valid[i] = full || (t0 + i * RPI + r < t_hi);
        if (!full) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int h = 0; h < GP; ++h) x[i][h] = valid[i] ? x[i][h] : -INFINITY;
        }
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            float mt = x[0][h];
#pragma unroll
            for (int i = 1; i < NI; ++i) mt = fmaxf(mt, x[i][h]);
            if (mt > m[h] + kTau) {
                const float alpha = __builtin_amdgcn_exp2f(m[h] - mt);   // 0 when m = -inf
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
                m[h] = mt;
            }
        }
        float pw[NI][GP];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                const float e = __builtin_amdgcn_exp2f(x[i][h] - m[h]);
                pw[i][h] = valid[i] ? e : 0.f;
                l[h] += pw[i][h];
            }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float vf[8];
            widen2<BF16>(vb[i].x, vf[0], vf[1]);
            widen2<BF16>(vb[i].y, vf[2], vf[3]);
            widen2<BF16>(vb[i].z, vf[4], vf[5]);
            widen2<BF16>(vb[i].w, vf[6], vf[7]);
            if (!full) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vf[e] = valid[i] ? vf[e] : 0.f;
            }
#pragma unroll
            for (int h = 0; h < GP; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw[i][h], vf[e], acc[h][e]);
        }
    };

    // Chunks of up to 64 tiles: lane i first loads the block id of the chunk's
    // tile i.  Two register buffers then alternate (no copies between them):
    // while one tile is computed the next tile's K/V loads are in flight.
    auto load_tile = [&](int it, int32_t blocks, uint4 (&kb)[NI], uint4 (&vb)[NI], int c0) {
        const int64_t base = tile_base(c0 + it, __builtin_amdgcn_readlane(blocks, it));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            kb[i] = *reinterpret_cast<const uint4*>(kc + base + i * RPI * D);
            vb[i] = *reinterpret_cast<const uint4*>(vc + base + i * RPI * D);
        }
        // Keep the scheduler from sinking these loads below the compute of the
        // previous tile: they must be issued before that compute waits.
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int c0 = 0; c0 < n_w; c0 += 64) {
        const int cn = min(64, n_w - c0);
        const int32_t blocks = lane < cn ? table[(t_lo + (wave + kWaves * (c0 + lane)) * kTile) / BS] : 0;
        uint4 ka[NI], va[NI], kb2[NI], vb2[NI];
        load_tile(0, blocks, ka, va, c0);
        int it = 0;
        for (; it + 2 < cn; it += 2) {
            load_tile(it + 1, blocks, kb2, vb2, c0);
            compute_tile(c0 + it, ka, va);
            load_tile(it + 2, blocks, ka, va, c0);
            compute_tile(c0 + it + 1, kb2, vb2);
        }
        if (it + 1 < cn) {
            load_tile(it + 1, blocks, kb2, vb2, c0);
            compute_tile(c0 + it, ka, va);
            compute_tile(c0 + it + 1, kb2, vb2);
        } else {
            compute_tile(c0 + it, ka, va);
        }
    }

    // ---- merge the row-groups of this wave (lanes sharing c, different r) ----
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        float mx = m[h];
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float f = (m[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[h] - mx);
        float lh = l[h] * f;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) lh += __shfl_xor(lh, off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[h][e] * f;
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) v += __shfl_xor(v, off);
            acc[h][e] = v;
        }
        m[h] = mx;
        l[h] = lh;
    }

    // ---- merge the 4 waves through LDS ----
    __shared__ float s_acc[kWaves][GP][D];
    __shared__ float s_m[kWaves][GP];
    __shared__ float s_l[kWaves][GP];
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[wave][h][c * 8 + e] = acc[h][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
    }
    __syncthreads();

    const bool direct = nparts <= 1;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int h = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (s_m[w][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
            L += s_l[w][h] * f;
            O += s_acc[w][h][d] * f;
        }
        O = L > 0.f ? O / L : 0.f;
        const float lse2 = L > 0.f ? M + __builtin_amdgcn_logf(L) : -INFINITY;   // log2 domain
        const int64_t sh = (int64_t)s * a.num_q_heads + h0 + h;
        if (direct) {
            store_out(a.out, sh * D + d, O, a.out_dtype);
            if (a.lse && d == 0) a.lse[sh] = lse2 * kLn2;
        } else {
            a.ws_out[(sh * a.max_parts + p) * D + d] = O;
            if (d == 0) a.ws_lse[sh * a.max_parts + p] = lse2;
        }
    }
}

// Merge kernel: one 256-thread workgroup per (sequence, q head) whose
// sequence spans more than one partition.  With M = max_p lse_p and
// w_p = 2^(lse_p - M): out = sum_p w_p o_p / sum_p w_p and
// lse = M + log2(sum_p w_p) -- the online-softmax identity applied to the
// partitions.  Threads own 4 consecutive d values of one partition slot; the
// slots stride over the partitions and meet in LDS.
template <int D>
__global__ void __launch_bounds__(kThreads)
paged_decode_merge_kernel(MergeArgs a) {
    constexpr int TPP = D / 4;                 // threads per partition row
    constexpr int SLOTS = kThreads / TPP;      // partitions handled at once
    const int64_t sh = blockIdx.x;
    const int s = (int)(sh / a.num_q_heads);
    const int ctx = min(max(a.context_lens[s], 0), a.max_context_len);
    const int nparts = (ctx + a.part_size - 1) / a.part_size;
    if (nparts <= 1) return;                  // written by the partition kernel

    const float* lse_p = a.ws_lse + sh * a.max_parts;
    const float* out_p = a.ws_out + sh * a.max_parts * D;
    __shared__ float s_red[kThreads / 64];
    __shared__ float s_acc[SLOTS][D];
    __shared__ float s_w[SLOTS];

    // M = max over partitions.
    float mx = -INFINITY;
    for (int pp = threadIdx.x; pp < nparts; pp += kThreads) mx = fmaxf(mx, lse_p[pp]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, s_red[w]);

    const int slot = threadIdx.x / TPP;
    const int d4 = (threadIdx.x % TPP) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    for (int pp = slot; pp < nparts; pp += SLOTS) {
        const float w = __builtin_amdgcn_exp2f(lse_p[pp] - M);
        const float4 o = *reinterpret_cast<const float4*>(out_p + (int64_t)pp * D + d4);
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
        wsum += w;
    }
    s_acc[slot][d4 + 0] = acc.x;
    s_acc[slot][d4 + 1] = acc.y;
    s_acc[slot][d4 + 2] = acc.z;
    s_acc[slot][d4 + 3] = acc.w;
    if (threadIdx.x % TPP == 0) s_w[slot] = wsum;
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += kThreads) {
        float o = 0.f, W = 0.f;
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) { o += s_acc[k][d]; W += s_w[k]; }
        store_out(a.out, sh * D + d, o / W, a.out_dtype);
        if (a.lse && d == 0) a.lse[sh] = (M + __builtin_amdgcn_logf(W)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------

template <int D, int BS, int GP, bool BF16>
static hipError_t launch_partition_t(const DecodeArgs& a, hipStream_t stream) {
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.max_parts;
    hipLaunchKernelGGL((paged_decode_partition_kernel<D, BS, GP, BF16>), dim3((unsigned)n), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int BS, bool BF16>
static hipError_t launch_partition_g(const DecodeArgs& a, int gp, hipStream_t stream) {
    switch (gp) {
        case 1: return launch_partition_t<D, BS, 1, BF16>(a, stream);
        case 2: return launch_partition_t<D, BS, 2, BF16>(a, stream);
        case 4: return launch_partition_t<D, BS, 4, BF16>(a, stream);
        case 8: return launch_partition_t<D, BS, 8, BF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int D, bool BF16>
static hipError_t launch_partition_b(const DecodeArgs& a, int bs, int gp, hipStream_t stream) {
    if (bs == 16) return launch_partition_g<D, 16, BF16>(a, gp, stream);
    if (bs == 32) return launch_partition_g<D, 32, BF16>(a, gp, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_partition(const DecodeArgs& a, int head_dim, int block_size, int group_pad, bool bf16,
                            hipStream_t stream) {
    if (head_dim == 128) {
        return bf16 ? launch_partition_b<128, true>(a, block_size, group_pad, stream)
                    : launch_partition_b<128, false>(a, block_size, group_pad, stream);
    }
    if (head_dim == 64) {
        return bf16 ? launch_partition_b<64, true>(a, block_size, group_pad, stream)
                    : launch_partition_b<64, false>(a, block_size, group_pad, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
    const unsigned n = (unsigned)((int64_t)a.num_seqs * a.num_q_heads);
    if (n == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL(paged_decode_merge_kernel<128>, dim3(n), dim3(kThreads), 0, stream, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL(paged_decode_merge_kernel<64>, dim3(n), dim3(kThreads), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pkv
