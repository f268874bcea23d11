"""Seeded synthetic decode workloads: shapes, context lengths, block tables, values.

This module is shared by the oracle's tests and by the GPU path's tests and
benchmark.  It holds no arithmetic of the attention method itself: it only
draws context lengths, lays out a block table over a shuffled physical pool,
and fills tensors with seeded normal samples.

The workloads follow the paged-KV setting of the pages:
  * fixed-size KV blocks reached through a per-sequence logical->physical
    block table ("架构解构：推理引擎的四层抽象", PagedAttention section);
  * a sequence of n tokens holds ceil(n / block_size) blocks ("LLM+Agent 全栈
    推理底座", 4.2 paged KV cache, BlockManager.allocate).

Metadata is drawn with NumPy's PCG64 (`default_rng(seed)`) in a fixed order
(context lengths, then the physical-block permutation), so tables and lengths
are bit-identical on every machine.  Values (q, K pool, V pool) are N(0, 1)
fp32 samples from a seeded torch generator on the target device, rounded to
fp16/bf16 by torch's round-to-nearest-even conversion.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np

DTYPES = ("f16", "bf16")


@dataclasses.dataclass
class DecodeWorkload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f16" | "bf16" for q, K and V
    scale: float                    # an fp32 value
    context_lens: np.ndarray        # int32 [B]
    block_tables: np.ndarray        # int32 [B][W], -1 in unused entries
    num_blocks: int                 # physical blocks in the pool
    alloc_order: np.ndarray         # int32 [num_blocks], the seeded permutation
    partition_size: int = 0         # 0 = library's choice
    seed: int = 0
    shared_groups: int = 0          # >0: sequences in groups of this size share a prefix

    @property
    def table_width(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elt_bytes(self) -> int:
        return 2

    def kv_bytes_logical(self) -> int:
        """K and V bytes one decode step reads: each token once per kv head."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * 2

    def kv_bytes_unique(self) -> int:
        """Same, counting each physical (block, slot) once even if shared."""
        used = used_slot_mask(self)
        return int(used.sum()) * self.num_kv_heads * self.head_dim * 2 * 2

    def metadata_sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.context_lens, self.block_tables, self.alloc_order):
            h.update(np.ascontiguousarray(a, dtype=np.int32).tobytes())
        return h.hexdigest()


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _fill_tables(ctx: np.ndarray, bs: int, alloc_order: np.ndarray, width: int) -> np.ndarray:
    """Give each sequence, in order, the next ceil(ctx/bs) ids of alloc_order."""
    B = len(ctx)
    tables = np.full((B, width), -1, dtype=np.int32)
    cur = 0
    for s in range(B):
        n = _ceil_div(int(ctx[s]), bs)
        tables[s, :n] = alloc_order[cur:cur + n]
        cur += n
    return tables


def make_workload(
    num_seqs: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    dtype: str,
    context_lens,
    seed: int,
    num_blocks: Optional[int] = None,
    pool_factor: float = 1.25,
    extra_table_entries: int = 0,
    partition_size: int = 0,
    name: str = "custom",
    rng: Optional[np.random.Generator] = None,
) -> DecodeWorkload:
    """A workload with given context lengths and a shuffled physical pool."""
    assert dtype in DTYPES
    rng = rng if rng is not None else np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32).reshape(-1)
    assert len(ctx) == num_seqs
    need = int(sum(_ceil_div(int(c), block_size) for c in ctx))
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * need))
    assert num_blocks >= need
    alloc_order = rng.permutation(num_blocks).astype(np.int32)
    width = max(1, max((_ceil_div(int(c), block_size) for c in ctx), default=0) + extra_table_entries)
    tables = _fill_tables(ctx, block_size, alloc_order, width)
    return DecodeWorkload(
        name=name, num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, dtype=dtype,
        scale=float(np.float32(1.0 / math.sqrt(head_dim))),
        context_lens=ctx, block_tables=tables, num_blocks=num_blocks,
        alloc_order=alloc_order, partition_size=partition_size, seed=seed)


def make_shared_prefix_workload(
    num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
    dtype: str, context_lens, group: int, prefix_tokens: int, seed: int,
    rng: Optional[np.random.Generator] = None, pool_factor: float = 1.25,
    extra_table_entries: int = 0, name: str = "shared-prefix",
) -> DecodeWorkload:
    """Sequences in consecutive groups of `group` share their leading blocks.

    Each group owns ceil(min(prefix_tokens, longest member)/block_size) shared
    blocks.  Member i maps its logical block j to the group's shared block j
    while j is below that count, and to a private block after it.  A member
    shorter than the prefix reads a leading part of it.  Physical ids are taken
    from the seeded permutation in turn: a group's shared blocks first, then
    each member's private blocks in member order.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32).reshape(-1)
    B, bs = num_seqs, block_size
    nblk = [_ceil_div(int(c), bs) for c in ctx]
    groups = [list(range(g0, min(g0 + group, B))) for g0 in range(0, B, group)]
    nshared = []
    need = 0
    for mem in groups:
        longest = max(int(ctx[i]) for i in mem)
        ns = _ceil_div(min(prefix_tokens, longest), bs)
        nshared.append(ns)
        need += ns + sum(max(0, nblk[i] - ns) for i in mem)
    num_blocks = max(1, math.ceil(pool_factor * need))
    alloc_order = rng.permutation(num_blocks).astype(np.int32)
    width = max(1, max(nblk) + extra_table_entries)
    tables = np.full((B, width), -1, dtype=np.int32)
    cur = 0
    for mem, ns in zip(groups, nshared):
        shared = alloc_order[cur:cur + ns]
        cur += ns
        for i in mem:
            k = min(nblk[i], ns)
            tables[i, :k] = shared[:k]
            npriv = nblk[i] - k
            tables[i, k:k + npriv] = alloc_order[cur:cur + npriv]
            cur += npriv
    wl = DecodeWorkload(
        name=name, num_seqs=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=bs, dtype=dtype,
        scale=float(np.float32(1.0 / math.sqrt(head_dim))), context_lens=ctx,
        block_tables=tables, num_blocks=num_blocks, alloc_order=alloc_order,
        seed=seed, shared_groups=group)
    return wl


# ---------------------------------------------------------------------------
# The five decode configurations.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-mha-d64",
    2: "llama2-7b-shape-mha",
    3: "llama3-8b-shape-gqa",
    4: "long-skewed-gqa-splitk",
    5: "cbatch-mix-shared-prefix",
}


def config(cid: int, seed: Optional[int] = None, extra_table_entries: int = 0) -> DecodeWorkload:
    """Configuration `cid` (1..5) drawn with seed 1000 + cid unless given."""
    seed = 1000 + cid if seed is None else seed
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[cid]
    if cid == 1:
        # 4 sequences, fixed lengths, MHA, D=64, bs=16, fp16, a 64-block pool.
        return make_workload(4, 4, 4, 64, 16, "f16", [1, 17, 100, 256], seed,
                             num_blocks=64, extra_table_entries=extra_table_entries,
                             name=name, rng=rng)
    if cid == 2:
        ctx = rng.integers(512, 2048 + 1, size=32)
        return make_workload(32, 32, 32, 128, 16, "f16", ctx, seed,
                             extra_table_entries=extra_table_entries, name=name, rng=rng)
    if cid == 3:
        ctx = rng.integers(1024, 8192 + 1, size=64)
        return make_workload(64, 32, 8, 128, 16, "bf16", ctx, seed,
                             extra_table_entries=extra_table_entries, name=name, rng=rng)
    if cid == 4:
        u = rng.uniform(math.log(4096), math.log(131072), size=8)
        ctx = np.clip(np.floor(np.exp(u)), 4096, 131072).astype(np.int64)
        return make_workload(8, 64, 8, 128, 16, "bf16", ctx, seed, partition_size=512,
                             extra_table_entries=extra_table_entries, name=name, rng=rng)
    if cid == 5:
        B = 256
        n_long = round(0.3 * B)
        is_long = np.zeros(B, dtype=bool)
        is_long[rng.permutation(B)[:n_long]] = True
        long_ctx = rng.integers(4096, 32768 + 1, size=B)
        short_ctx = rng.integers(128, 1024 + 1, size=B)
        ctx = np.where(is_long, long_ctx, short_ctx)
        return make_shared_prefix_workload(B, 32, 8, 128, 32, "bf16", ctx, group=8,
                                           prefix_tokens=2048, seed=seed, rng=rng,
                                           extra_table_entries=extra_table_entries, name=name)
    raise ValueError(f"unknown config {cid}")


def used_slot_mask(wl: DecodeWorkload) -> np.ndarray:
    """bool [num_blocks][block_size]: slots some sequence's context covers."""
    used = np.zeros((wl.num_blocks, wl.block_size), dtype=bool)
    bs = wl.block_size
    for s in range(wl.num_seqs):
        c = int(wl.context_lens[s])
        nfull, rem = divmod(c, bs)
        if nfull:
            used[wl.block_tables[s, :nfull], :] = True
        if rem:
            used[wl.block_tables[s, nfull], :rem] = True
    return used


# ---------------------------------------------------------------------------
# Values.
# ---------------------------------------------------------------------------

def _torch_dtype(dtype: str):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def fill_normal_(t, seed: int, chunk: int = 1 << 26):
    """Fill a 16-bit tensor with N(0,1) fp32 samples rounded to its dtype."""
    import torch
    gen = torch.Generator(device=t.device)
    gen.manual_seed(int(seed))
    flat = t.view(-1)
    n = flat.numel()
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        flat[i:i + m] = torch.randn(m, generator=gen, device=t.device, dtype=torch.float32).to(t.dtype)
    return t


def make_values(wl: DecodeWorkload, device="cpu", poison: bool = False, seed_offset: int = 0):
    """q [B][Hq][D], k_cache and v_cache [NB][Hkv][bs][D], all in wl.dtype.

    With poison=True every slot no sequence reads holds NaN, so a read of an
    unused slot or block shows up in the output.
    """
    import torch
    dt = _torch_dtype(wl.dtype)
    base = (wl.seed * 7919 + seed_offset) & 0x7FFFFFFF
    q = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=dt, device=device)
    k = torch.empty((wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim), dtype=dt, device=device)
    v = torch.empty_like(k)
    fill_normal_(q, base + 1)
    fill_normal_(k, base + 2)
    fill_normal_(v, base + 3)
    if poison:
        poison_unused_(wl, k, v)
    return q, k, v


def poison_unused_(wl: DecodeWorkload, k, v):
    import torch
    used = torch.from_numpy(used_slot_mask(wl)).to(k.device)          # [NB][bs]
    mask = (~used)[:, None, :, None].expand_as(k)
    k.masked_fill_(mask, float("nan"))
    v.masked_fill_(mask, float("nan"))


def bits16(t) -> np.ndarray:
    """Raw 16-bit storage of a fp16/bf16 tensor, as a contiguous uint16 array."""
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def make_fp8_cache(wl: DecodeWorkload, device="cpu", poison: bool = False, seed_offset: int = 0,
                   scale_log2=(-9.0, -6.0)):
    """An 8-bit K/V cache for the workload's pool: (k_codes, v_codes uint8 [NB][Hkv][bs][D],
    k_scale, v_scale float32 [NB][Hkv]).

    Codes are drawn uniformly over the 254 finite E4M3 codes (0x7F and 0xFF, the
    NaN codes, are skipped); each (block, kv head) scale is 2^u with u uniform in
    scale_log2.  With poison=True every unused slot holds the NaN code 0x7F.
    """
    import torch
    base = (wl.seed * 7919 + seed_offset + 101) & 0x7FFFFFFF
    gen = torch.Generator(device=device)
    shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    out = []
    for i in range(2):
        gen.manual_seed(base + i)
        c = torch.randint(0, 254, shape, generator=gen, device=device, dtype=torch.int16)
        c = c + (c >= 127).to(torch.int16)               # 0..126, 128..254
        out.append(c.to(torch.uint8))
    scales = []
    for i in range(2):
        gen.manual_seed(base + 10 + i)
        u = torch.rand((wl.num_blocks, wl.num_kv_heads), generator=gen, device=device, dtype=torch.float32)
        scales.append(torch.exp2(scale_log2[0] + (scale_log2[1] - scale_log2[0]) * u))
    kc, vc = out
    if poison:
        used = torch.from_numpy(used_slot_mask(wl)).to(device)
        mask = (~used)[:, None, :, None].expand_as(kc)
        kc.masked_fill_(mask, 0x7F)
        vc.masked_fill_(mask, 0x7F)
    return kc, vc, scales[0], scales[1]


def make_prefill_workload(num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int, dtype: str,
                          prefix_lens, chunk_lens, seed: int, name: str = "prefill"):
    """A chunked-prefill batch: sequence s has prefix_lens[s] cached tokens and a chunk of
    chunk_lens[s] new ones (already in the cache); its context is their sum.  Returns the
    workload and cu_q (int32 [B + 1], the chunk rows of each sequence)."""
    pre = np.asarray(prefix_lens, dtype=np.int64)
    chk = np.asarray(chunk_lens, dtype=np.int64)
    wl = make_workload(len(pre), num_q_heads, num_kv_heads, head_dim, block_size, dtype, pre + chk, seed, name=name)
    cu = np.concatenate([[0], np.cumsum(chk)]).astype(np.int32)
    return wl, cu


def llama3_8b_prefill(seed: int = 2003):
    """Chunked prefill on the Llama-3-8B GQA shape (32 q / 8 kv heads, head_dim 128, block 16,
    bf16): 16 sequences, each with a cached prefix drawn uniformly from [0, 3584] tokens and a
    512-token chunk."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, 3585, 16)
    return make_prefill_workload(32, 8, 128, 16, "bf16", prefix, [512] * 16, seed, name="llama3-8b-chunked-prefill")


def make_prefill_q(wl: DecodeWorkload, cu_q, device="cpu", seed_offset: int = 0):
    """q [total_q][Hq][D] of N(0,1) samples rounded to the workload's dtype."""
    import torch
    q = torch.empty((int(cu_q[-1]), wl.num_q_heads, wl.head_dim), dtype=_torch_dtype(wl.dtype), device=device)
    return fill_normal_(q, (wl.seed * 7919 + seed_offset + 211) & 0x7FFFFFFF)
