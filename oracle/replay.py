"""Integer replays of the paged-KV bookkeeping, in pure Python.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.  It shares nothing with the GPU library.

What is replayed, from the definitions:

  * blocks a sequence of n tokens holds: ceil(n / block_size), i.e.
    (n + block_size - 1) // block_size ("LLM+Agent 全栈推理底座" 4.2,
    BlockManager.allocate);
  * allocation pops the LAST element of a free list (the same section's
    BlockManager takes `free_blocks.pop()`).  The pool's free list starts as the
    seeded allocation order reversed, so the first block handed out is
    alloc_order[0], the second alloc_order[1], and so on.  A fixed device pool
    cannot grow, so where that section grows the pool this replay reports
    exhaustion instead, with no change to any state;
  * a token at logical position t of a sequence lives in slot
    table[t // bs] * bs + t % bs, the block table being the logical->physical map
    ("架构解构：推理引擎的四层抽象", PagedAttention section);
  * blocks shared by several sequences (a common prefix, "LLM+Agent 全栈推理底座"
    2.2 and 4.4 prefix reuse) carry a reference count.  Appending into a shared,
    partly filled tail block first copies its used slots into a fresh block
    (copy-on-write), so the other holders never see the write;
  * freeing a sequence drops one reference from each of its blocks in logical
    order; a block whose count reaches zero is pushed back onto the free list,
    so the next allocation reuses the last block released;
  * the host tier ("LLM+Agent 全栈推理底座" 4.2, TieredBlockManager): a sequence
    keeps its last gpu_window blocks on the GPU; the blocks before them (the
    listing's blocks[:-gpu_window], taken only when the sequence holds more than
    gpu_window blocks) are cold and move to a pool of pinned host blocks; when
    the sequence is needed again they are copied back ("DMA back").  Host blocks
    come from their own LIFO free list (first handed out: 0, 1, 2, ...).  Moving
    a block gives the moving sequence a private copy in the other tier; the old
    block loses one reference and is freed at zero, so a block still shared by
    another holder stays where it is.  In a block list a host block c is written
    -2 - c.  A sequence holding host blocks is parked: it cannot be appended to
    and it publishes length 0 (table row all -1) until it is restored;
  * the decode split: every (sequence s, head group q, 16-token tile j) in one
    sequence-major list, a group being the H kv heads one wave takes together
    (H = 2 for 8-bit K/V with an even kv head count, else 1) -- the tiles of
    kv head g start at first(s, g) = (Hkv / H) * sum_{s'<s} pt_s' + (g // H) * pt_s
    -- cut into chunks of C tiles.  With a
    fixed partition size P, C = P / 16 and pt_s = ceil(nt_s / C) * C (so a
    chunk is the partition [p*P, min((p+1)*P, n)) of one (s, g)); balanced,
    pt_s = nt_s and C = max(4, ceil(T / W)) for W waves and T tiles in all.
    A segment is the part of one chunk inside one (s, g); its slot is the
    chunk index minus first(s, g) // C.  Segments are listed in (s, g, slot)
    order.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


def ceil_div(a: int, b: int) -> int:
    return (a + b - 1) // b


def blocks_needed(num_tokens: int, block_size: int) -> int:
    return ceil_div(num_tokens, block_size)


class PoolError(Exception):
    def __init__(self, kind: str, msg: str = ""):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind          # "EINVAL" | "ENOMEM"


class AppendItem(tuple):
    """(seq, slot, table_pos, new_block, cow_src, cow_ntok, new_len)."""
    __slots__ = ()

    def __new__(cls, seq, slot, tpos, new_block, cow_src, cow_n, new_len):
        return tuple.__new__(cls, (seq, slot, tpos, new_block, cow_src, cow_n, new_len))


class PoolReplay:
    def __init__(self, num_blocks: int, block_size: int, max_seqs: int,
                 max_blocks_per_seq: int, alloc_order: Optional[Sequence[int]] = None):
        self.num_blocks = num_blocks
        self.bs = block_size
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        order = list(range(num_blocks)) if alloc_order is None else [int(b) for b in alloc_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError("EINVAL", "alloc_order is not a permutation")
        self.free: List[int] = list(reversed(order))       # pop() yields order[0] first
        self.ref = [0] * num_blocks
        self.seqs: Dict[int, Tuple[List[int], int]] = {}
        self.num_host_blocks = 0
        self.host_free: List[int] = []
        self.host_ref: List[int] = []

    # -- host tier ---------------------------------------------------------
    def attach_host_tier(self, num_host_blocks: int) -> None:
        if num_host_blocks < 1 or self.num_host_blocks:
            raise PoolError("EINVAL", "bad or repeated host tier")
        self.num_host_blocks = num_host_blocks
        self.host_free = list(reversed(range(num_host_blocks)))
        self.host_ref = [0] * num_host_blocks

    @staticmethod
    def is_host(entry: int) -> bool:
        return entry <= -2

    @staticmethod
    def host_id(entry: int) -> int:
        return -2 - entry

    def parked(self, sid: int) -> bool:
        return any(e <= -2 for e in self.seqs[sid][0])

    def _unref(self, entry: int) -> None:
        if entry <= -2:
            c = -2 - entry
            self.host_ref[c] -= 1
            if self.host_ref[c] == 0:
                self.host_free.append(c)
        else:
            self.ref[entry] -= 1
            if self.ref[entry] == 0:
                self.free.append(entry)

    def _check_ids(self, ids: Sequence[int]) -> List[int]:
        ids = [int(s) for s in ids]
        if len(set(ids)) != len(ids):
            raise PoolError("EINVAL", "duplicate sequence id")
        for s in ids:
            if s not in self.seqs:
                raise PoolError("EINVAL", "unknown sequence")
        return ids

    def offload(self, seq_ids: Sequence[int], gpu_window: int) -> List[Tuple[int, int]]:
        """Move each sequence's cold GPU blocks to the host tier; the (gpu, host) copies in order."""
        if not self.num_host_blocks:
            raise PoolError("EINVAL", "no host tier")
        if gpu_window < 1:
            raise PoolError("EINVAL", "gpu_window must be >= 1")
        ids = self._check_ids(seq_ids)
        cold = {s: self.seqs[s][0][:-gpu_window] if len(self.seqs[s][0]) > gpu_window else [] for s in ids}
        need = sum(1 for s in ids for e in cold[s] if e >= 0)
        if need > len(self.host_free):
            raise PoolError("ENOMEM", "host tier exhausted")
        copies = []
        for s in ids:
            blocks, _ = self.seqs[s]
            for i in range(len(cold[s])):
                b = blocks[i]
                if b < 0:
                    continue
                c = self.host_free.pop()
                self.host_ref[c] = 1
                copies.append((b, c))
                blocks[i] = -2 - c
                self._unref(b)
        return copies

    def restore(self, seq_ids: Sequence[int]) -> List[Tuple[int, int]]:
        """Copy each sequence's host blocks back into fresh GPU blocks; the (host, gpu) copies in order."""
        ids = self._check_ids(seq_ids)
        need = sum(1 for s in ids for e in self.seqs[s][0] if e <= -2)
        if need > len(self.free):
            raise PoolError("ENOMEM", "pool exhausted")
        copies = []
        for s in ids:
            blocks, _ = self.seqs[s]
            for i, e in enumerate(blocks):
                if e > -2:
                    continue
                b = self.free.pop()
                self.ref[b] = 1
                copies.append((-2 - e, b))
                blocks[i] = b
                self._unref(e)
        return copies

    # -- sequences -------------------------------------------------------
    def _new_id(self) -> int:
        for i in range(self.max_seqs):
            if i not in self.seqs:
                return i
        raise PoolError("ENOMEM", "no free sequence slot")

    def add_seq(self) -> int:
        sid = self._new_id()
        self.seqs[sid] = ([], 0)
        return sid

    def import_seq(self, blocks: Sequence[int], length: int) -> int:
        blocks = [int(b) for b in blocks]
        if length < 0 or len(blocks) != blocks_needed(length, self.bs):
            raise PoolError("EINVAL", "block count does not match length")
        if len(blocks) > self.max_blocks_per_seq or len(set(blocks)) != len(blocks):
            raise PoolError("EINVAL", "bad block list")
        for b in blocks:
            if not 0 <= b < self.num_blocks:
                raise PoolError("EINVAL", "block id out of range")
        sid = self._new_id()
        for b in blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        self.seqs[sid] = (blocks, length)
        return sid

    def fork(self, src: int) -> int:
        if src not in self.seqs:
            raise PoolError("EINVAL", "unknown sequence")
        sid = self._new_id()
        blocks, length = self.seqs[src]
        for b in blocks:
            if b <= -2:
                self.host_ref[-2 - b] += 1
            else:
                self.ref[b] += 1
        self.seqs[sid] = (list(blocks), length)
        return sid

    def free_seq(self, sid: int) -> None:
        if sid not in self.seqs:
            raise PoolError("EINVAL", "unknown sequence")
        blocks, _ = self.seqs.pop(sid)
        for b in blocks:
            self._unref(b)

    def _copies(self, tails: Sequence[int]) -> int:
        """Blocks copy-on-write takes for the listed shared tails (one entry per listed
        sequence that writes into its shared, partly filled tail block).  The sequences
        copy in list order while the tail has another holder and each copy drops one
        reference, so k listed holders of a tail held r times take min(k, r - 1) copies."""
        n = 0
        for b in set(tails):
            n += min(tails.count(b), self.ref[b] - 1)
        return n

    # -- append one token to each listed sequence (all-or-nothing) --------
    def append(self, seq_ids: Sequence[int]) -> List[AppendItem]:
        ids = [int(s) for s in seq_ids]
        if len(set(ids)) != len(ids):
            raise PoolError("EINVAL", "duplicate sequence id")
        need = 0
        tails = []
        for s in ids:
            if s not in self.seqs:
                raise PoolError("EINVAL", "unknown sequence")
            if self.parked(s):
                raise PoolError("EINVAL", "sequence has blocks in the host tier")
            blocks, t = self.seqs[s]
            if t % self.bs == 0:
                if t // self.bs >= self.max_blocks_per_seq:
                    raise PoolError("EINVAL", "sequence reached max_blocks_per_seq")
                need += 1
            elif self.ref[blocks[-1]] > 1:
                tails.append(blocks[-1])
        need += self._copies(tails)
        if need > len(self.free):
            raise PoolError("ENOMEM", "pool exhausted")
        items = []
        for s in ids:
            blocks, t = self.seqs[s]
            tpos, off = divmod(t, self.bs)
            new_block, cow_src, cow_n = -1, -1, 0
            if off == 0:
                new_block = self.free.pop()
                self.ref[new_block] = 1
                blocks.append(new_block)
            elif self.ref[blocks[-1]] > 1:
                new_block = self.free.pop()
                self.ref[new_block] = 1
                cow_src, cow_n = blocks[-1], off
                self.ref[cow_src] -= 1
                blocks[-1] = new_block
            slot = blocks[tpos] * self.bs + off
            self.seqs[s] = (blocks, t + 1)
            items.append(AppendItem(s, slot, tpos, new_block, cow_src, cow_n, t + 1))
        return items

    # -- append several tokens per sequence (all-or-nothing) ----------------
    def append_tokens(self, seq_ids: Sequence[int], counts: Sequence[int]) -> List[AppendItem]:
        """counts[i] tokens to seq_ids[i]: the same as appending them one at a time, each
        sequence's tokens in a row, sequences in list order; nothing changes on an error."""
        ids = [int(s) for s in seq_ids]
        cnt = [int(c) for c in counts]
        if len(ids) != len(cnt) or len(set(ids)) != len(ids) or any(c < 0 for c in cnt):
            raise PoolError("EINVAL", "bad sequence list or counts")
        need = 0
        tails = []
        for s, c in zip(ids, cnt):
            if s not in self.seqs:
                raise PoolError("EINVAL", "unknown sequence")
            if self.parked(s):
                raise PoolError("EINVAL", "sequence has blocks in the host tier")
            blocks, t = self.seqs[s]
            if c == 0:
                continue
            if blocks_needed(t + c, self.bs) > self.max_blocks_per_seq:
                raise PoolError("EINVAL", "sequence would exceed max_blocks_per_seq")
            need += blocks_needed(t + c, self.bs) - blocks_needed(t, self.bs)
            if t % self.bs and self.ref[blocks[-1]] > 1:
                tails.append(blocks[-1])
        need += self._copies(tails)
        if need > len(self.free):
            raise PoolError("ENOMEM", "pool exhausted")
        items = []
        for s, c in zip(ids, cnt):
            for _ in range(c):
                items += self.append([s])
        return items

    # -- views ------------------------------------------------------------
    def tables(self, width: Optional[int] = None):
        """(block_tables [max_seqs][width] with -1 fill, context_lens [max_seqs])."""
        w = self.max_blocks_per_seq if width is None else width
        tab = [[-1] * w for _ in range(self.max_seqs)]
        lens = [0] * self.max_seqs
        for s, (blocks, length) in self.seqs.items():
            if self.parked(s):
                continue
            tab[s][:len(blocks)] = blocks
            lens[s] = length
        return tab, lens

    def num_free(self) -> int:
        return len(self.free)

    def num_host_free(self) -> int:
        return len(self.host_free)


TILE = 16
MIN_CHUNK = 4


def plan(context_lens: Sequence[int], num_kv_heads: int, partition_size: int, num_waves: int = 1,
         heads_per_wave: int = 1):
    """Segments (seq, kv_head, slot, tok_lo, tok_hi) of the decode split, in order."""
    if partition_size < 0 or num_waves < 1 or heads_per_wave < 1 or num_kv_heads % heads_per_wave:
        raise ValueError("bad split parameters")
    lens = [max(0, int(n)) for n in context_lens]
    nt = [ceil_div(n, TILE) for n in lens]
    if partition_size > 0:
        C = partition_size // TILE
        pt = [ceil_div(x, C) * C for x in nt]
    else:
        pt = list(nt)
    firsts = []
    acc = 0
    for s in range(len(lens)):
        firsts.append(acc)
        acc += (num_kv_heads // heads_per_wave) * pt[s]
    total = acc
    if partition_size == 0:
        C = max(MIN_CHUNK, ceil_div(total, num_waves))
    items = []
    for s, n in enumerate(lens):
        for g in range(num_kv_heads):
            if nt[s] == 0:
                continue
            first = firsts[s] + (g // heads_per_wave) * pt[s]
            c0, c1 = first // C, (first + nt[s] - 1) // C
            for ch in range(c0, c1 + 1):
                j0 = max(ch * C - first, 0)
                j1 = min((ch + 1) * C - first, nt[s])
                items.append((s, g, ch - c0, j0 * TILE, min(j1 * TILE, n)))
    return items


def segment_rows(context_lens: Sequence[int], num_kv_heads: int, partition_size: int, num_waves: int = 1,
                 heads_per_wave: int = 1):
    """Workspace row of every segment of the split, {(seq, kv_head, slot): row}: segment slot k of
    the pair p = (sequence s, head group g // heads_per_wave), p = s * (num_kv_heads //
    heads_per_wave) + g // heads_per_wave, is chunk first // C + k of the flattened tile list and
    sits in row (that chunk) + p.  The kv heads of one group share their rows."""
    lens = [max(0, int(n)) for n in context_lens]
    nt = [ceil_div(n, TILE) for n in lens]
    hg = num_kv_heads // heads_per_wave
    if partition_size > 0:
        C = partition_size // TILE
        pt = [ceil_div(x, C) * C for x in nt]
    else:
        pt = list(nt)
    total = hg * sum(pt)
    if partition_size == 0:
        C = max(MIN_CHUNK, ceil_div(total, num_waves))
    rows = {}
    acc = 0
    for s in range(len(lens)):
        for g in range(num_kv_heads):
            if nt[s] == 0:
                continue
            first = acc + (g // heads_per_wave) * pt[s]
            c0, c1 = first // C, (first + nt[s] - 1) // C
            for k in range(c1 - c0 + 1):
                rows[(s, g, k)] = c0 + k + s * hg + g // heads_per_wave
        acc += hg * pt[s]
    return rows
