"""The oracle's integer replays against the page's allocation rule and invariants."""
import json
import os
import random

import pytest

from oracle import replay as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blockmanager_allocate.json")


def test_golden_blockmanager_allocate():
    g = json.load(open(GOLDEN))
    bs = g["block_size"]
    # The page's free list [0..9] popped from the end == alloc_order [9, 8, ..., 0].
    order = list(reversed(g["free_blocks"]))
    pool = R.PoolReplay(len(order), bs, max_seqs=8, max_blocks_per_seq=8, alloc_order=order)
    for call in g["calls"]:
        assert R.blocks_needed(call["num_tokens"], bs) == call["needed"]
        sid = pool.add_seq()
        assert sid == call["seq_id"]
        for _ in range(call["num_tokens"]):
            pool.append([sid])
        assert pool.seqs[sid][0] == call["blocks"]
    assert sorted(pool.free) == g["free_blocks_after"]
    assert list(reversed(pool.free)) == sorted(g["free_blocks_after"], reverse=True)


@pytest.mark.parametrize("n,bs,want", [(0, 16, 0), (1, 16, 1), (16, 16, 1), (17, 16, 2),
                                       (32, 32, 1), (33, 32, 2), (131072, 16, 8192)])
def test_blocks_needed(n, bs, want):
    assert R.blocks_needed(n, bs) == want


def test_append_slots_and_tables():
    pool = R.PoolReplay(8, 4, max_seqs=2, max_blocks_per_seq=4, alloc_order=[5, 2, 7, 0, 1, 3, 4, 6])
    a, b = pool.add_seq(), pool.add_seq()
    items = []
    for _ in range(5):
        items += pool.append([a, b])
    # a takes 5, b takes 2 (t = 0); a takes 7, b takes 0 (t = 4).
    assert pool.seqs[a] == ([5, 7], 5) and pool.seqs[b] == ([2, 0], 5)
    slots_a = [it[1] for it in items if it[0] == a]
    assert slots_a == [20, 21, 22, 23, 28]
    tab, lens = pool.tables(width=4)
    assert tab == [[5, 7, -1, -1], [2, 0, -1, -1]] and lens == [5, 5]


def test_append_all_or_nothing():
    pool = R.PoolReplay(3, 2, max_seqs=4, max_blocks_per_seq=4, alloc_order=[0, 1, 2])
    ids = [pool.add_seq() for _ in range(4)]
    pool.append(ids[:3])                         # three blocks taken, pool empty
    before = (list(pool.free), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()})
    with pytest.raises(R.PoolError) as e:
        pool.append(ids)                         # seq 3 needs a block
    assert e.value.kind == "ENOMEM"
    assert (list(pool.free), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()}) == before
    pool.append(ids[:3])                         # t = 1 fits in each tail block
    with pytest.raises(R.PoolError):
        pool.append([0, 0])


def test_fork_copy_on_write():
    pool = R.PoolReplay(6, 4, max_seqs=3, max_blocks_per_seq=3, alloc_order=[3, 1, 4, 0, 5, 2])
    a = pool.add_seq()
    for _ in range(6):
        pool.append([a])                         # blocks [3, 1], len 6
    b = pool.fork(a)
    assert pool.ref[3] == 2 and pool.ref[1] == 2
    (it,) = pool.append([b])                     # b's tail block 1 is shared and partly full
    seq, slot, tpos, new_block, cow_src, cow_n, new_len = it
    assert (tpos, new_block, cow_src, cow_n, new_len) == (1, 4, 1, 2, 7)
    assert slot == 4 * 4 + 2
    assert pool.seqs[b][0] == [3, 4] and pool.seqs[a][0] == [3, 1]
    assert pool.ref[1] == 1 and pool.ref[4] == 1 and pool.ref[3] == 2
    (it,) = pool.append([a])                     # a's tail is private again: no copy
    assert it[3] == -1 and it[4] == -1
    pool.free_seq(a)                             # 3 still held by b; 1 freed
    assert pool.free[-1] == 1 and pool.ref[3] == 1


def test_shared_tail_listed_holders_charge_min_k_r_minus_1():
    """Two forked sequences share a partly filled tail and are appended in one call with a
    single free block: the first copies (the tail then has one holder left), the second
    writes in place, so one block suffices (worked by hand)."""
    pool = R.PoolReplay(3, 4, max_seqs=3, max_blocks_per_seq=2, alloc_order=[0, 1, 2])
    a = pool.add_seq()
    pool.append([a])
    pool.append([a])                             # a: block 0, 2 tokens
    b = pool.fork(a)                             # block 0 held twice
    c = pool.add_seq()
    pool.append([c])                             # c: block 1; free list [2]
    assert pool.num_free() == 1 and pool.ref[0] == 2
    ia, ib = pool.append([a, b])
    assert tuple(ia) == (a, 2 * 4 + 2, 0, 2, 0, 2, 3)   # a copies block 0's 2 rows into block 2
    assert tuple(ib) == (b, 0 * 4 + 2, 0, -1, -1, 0, 3)  # b is the last holder: in place
    assert pool.num_free() == 0 and pool.ref[0] == 1 and pool.ref[2] == 1
    # the same through append_tokens (one token each)
    pool2 = R.PoolReplay(3, 4, max_seqs=3, max_blocks_per_seq=2, alloc_order=[0, 1, 2])
    a = pool2.add_seq()
    pool2.append_tokens([a], [2])
    b = pool2.fork(a)
    c = pool2.add_seq()
    pool2.append([c])
    items = pool2.append_tokens([a, b], [1, 1])
    assert [tuple(i) for i in items] == [(a, 10, 0, 2, 0, 2, 3), (b, 2, 0, -1, -1, 0, 3)]


def test_shared_tail_three_holders():
    """A tail held by three sequences: listing two of them takes two copies, listing all
    three also takes two (the last one writes in place); one block short is ENOMEM."""
    for listed, copies in ((2, 2), (3, 2)):
        pool = R.PoolReplay(4, 4, max_seqs=4, max_blocks_per_seq=2, alloc_order=[0, 1, 2, 3])
        a = pool.add_seq()
        pool.append([a])                         # block 0, 1 token
        b, c = pool.fork(a), pool.fork(a)        # held three times; free [3, 2, 1]
        ids = [a, b, c][:listed]
        d = pool.add_seq()
        pool.append([d])                         # block 1 to d; free [3, 2]
        assert pool.num_free() == copies
        items = pool.append(ids)
        assert sum(1 for it in items if it[4] >= 0) == copies
        assert pool.num_free() == 0
        pool3 = R.PoolReplay(4, 4, max_seqs=5, max_blocks_per_seq=2, alloc_order=[0, 1, 2, 3])
        a = pool3.add_seq()
        pool3.append([a])
        b, c = pool3.fork(a), pool3.fork(a)
        d, e = pool3.add_seq(), pool3.add_seq()
        pool3.append([d, e])                     # free [3]: one block short
        with pytest.raises(R.PoolError):
            pool3.append([a, b, c][:listed])


def test_free_returns_blocks_lifo():
    pool = R.PoolReplay(4, 2, max_seqs=2, max_blocks_per_seq=4, alloc_order=[0, 1, 2, 3])
    a = pool.add_seq()
    for _ in range(5):
        pool.append([a])                         # blocks [0, 1, 2]
    pool.free_seq(a)                             # pushed in logical order: 0, 1, 2
    b = pool.add_seq()
    pool.append([b])
    assert pool.seqs[b][0] == [2]                # last released is reused first


def test_random_ops_conserve_blocks():
    rnd = random.Random(0)
    pool = R.PoolReplay(64, 4, max_seqs=8, max_blocks_per_seq=16)
    live = []
    for _ in range(2000):
        op = rnd.random()
        try:
            if op < 0.1 and len(live) < 8:
                live.append(pool.add_seq())
            elif op < 0.15 and live and len(live) < 8:
                live.append(pool.fork(rnd.choice(live)))
            elif op < 0.2 and live:
                s = rnd.choice(live); live.remove(s); pool.free_seq(s)
            elif live:
                pool.append(rnd.sample(live, rnd.randint(1, len(live))))
        except R.PoolError:
            pass
        held = {}
        for blocks, n in pool.seqs.values():
            assert len(blocks) == R.blocks_needed(n, 4)
            for b in blocks:
                held[b] = held.get(b, 0) + 1
        assert all(pool.ref[b] == c for b, c in held.items())
        assert len(held) + len(pool.free) == 64
        assert not set(held) & set(pool.free)


def test_plan_fixed_partitions():
    items = R.plan([0, 5, 1024, 1025], num_kv_heads=2, partition_size=512)
    assert items[:2] == [(1, 0, 0, 0, 5), (1, 1, 0, 0, 5)]
    assert (2, 1, 1, 512, 1024) in items and (3, 0, 2, 1024, 1025) in items
    assert len(items) == 2 * (1 + 2 + 3)
    assert items == sorted(items)


def test_plan_balanced_worked_example():
    # Two sequences of 40 and 200 tokens, one kv head: 3 + 13 = 16 tiles.
    # 2 waves -> C = max(4, 8) = 8 tiles: chunk 0 = tiles 0..7, chunk 1 = 8..15.
    # Sequence 0 (tiles 0..2) is whole in chunk 0; sequence 1 starts at tile 3:
    # its tiles 0..4 are in chunk 0 (slot 0), tiles 5..12 in chunk 1 (slot 1).
    items = R.plan([40, 200], num_kv_heads=1, partition_size=0, num_waves=2)
    assert items == [(0, 0, 0, 0, 40), (1, 0, 0, 0, 80), (1, 0, 1, 80, 200)]
    # Many waves: the chunk never drops below 4 tiles (64 tokens).  Chunks 0..3 are list
    # positions 0-3, 4-7, 8-11, 12-15: sequence 1 (positions 3..15) gets its tile 0 in
    # chunk 0, tiles 1-4, 5-8 and 9-12 in chunks 1, 2, 3 (tokens 16, 80, 144 apart).
    items = R.plan([40, 200], num_kv_heads=1, partition_size=0, num_waves=1000)
    assert items == [(0, 0, 0, 0, 40), (1, 0, 0, 0, 16), (1, 0, 1, 16, 80), (1, 0, 2, 80, 144),
                     (1, 0, 3, 144, 200)]
    # One wave: C = max(4, 34) = 34 tiles, everything in one chunk, every (seq, head) whole.
    items = R.plan([40, 200, 0, 7], num_kv_heads=2, partition_size=0, num_waves=1)
    assert items == [(0, 0, 0, 0, 40), (0, 1, 0, 0, 40), (1, 0, 0, 0, 200), (1, 1, 0, 0, 200),
                     (3, 0, 0, 0, 7), (3, 1, 0, 0, 7)]


def test_plan_two_heads_per_wave_worked_example():
    # Two kv heads taken together: the list holds one entry per (sequence,
    # pair, tile), 3 + 13 = 16 tiles; 2 waves -> C = 8.  Sequence 1 starts at
    # tile 3: its tiles 0..4 fall in chunk 0, 5..12 in chunk 1, for both heads.
    items = R.plan([40, 200], num_kv_heads=2, partition_size=0, num_waves=2, heads_per_wave=2)
    assert items == [(0, 0, 0, 0, 40), (0, 1, 0, 0, 40), (1, 0, 0, 0, 80), (1, 0, 1, 80, 200),
                     (1, 1, 0, 0, 80), (1, 1, 1, 80, 200)]
    # One head per wave on the same input: 32 tiles, C = 16, and head 1 of
    # sequence 1 starts at tile 19, so the two heads are cut differently.
    items = R.plan([40, 200], num_kv_heads=2, partition_size=0, num_waves=2)
    assert items == [(0, 0, 0, 0, 40), (0, 1, 0, 0, 40), (1, 0, 0, 0, 160), (1, 0, 1, 160, 200),
                     (1, 1, 0, 0, 200)]


@pytest.mark.parametrize("P,nw", [(0, 1), (0, 7), (0, 64), (0, 5000), (256, 3), (512, 100)])
def test_plan_pairs_equal_half_the_heads(P, nw):
    # With two heads per wave the list over Hkv heads is the one-head list over
    # Hkv / 2 heads, and each of its segments belongs to both heads of a pair.
    rng = random.Random(nw + P)
    lens = [rng.randrange(3000) for _ in range(37)] + [0, 1, 16, 17, 128, 129]
    for hkv in (2, 4, 8):
        pair = R.plan(lens, hkv, P, nw, heads_per_wave=2)
        half = R.plan(lens, hkv // 2, P, nw)
        want = [(s, 2 * g + h, k, lo, hi) for (s, g, k, lo, hi) in half for h in (0, 1)]
        assert sorted(pair) == sorted(want)
    with pytest.raises(ValueError):
        R.plan(lens, 3, P, nw, heads_per_wave=2)


@pytest.mark.parametrize("seed", range(12))
def test_plan_covers_each_context_once(seed):
    """Invariants of the split, whatever the lengths, heads, partition size and grid: the segments
    of each (sequence, kv head) have slots 0, 1, ... in token order and tile [0, len) with no gap or
    overlap; a segment holds at least one token and at most one chunk of tiles; fixed partitions
    cut at multiples of P (ceil(len / P) segments per pair); and the tiles of all segments add up
    to the list's total."""
    rnd = random.Random(1000 + seed)
    B = rnd.randint(1, 30)
    lens = [rnd.choice([0, 1, 15, 16, 17, 128, 129, rnd.randint(0, 9000)]) for _ in range(B)]
    hw = rnd.choice([1, 2])
    hkv = hw * rnd.randint(1, 4)
    P = rnd.choice([0, 0, 16, 48, 512])
    nw = rnd.choice([1, 3, 4, 64, 2048])
    items = R.plan(lens, hkv, P, nw, heads_per_wave=hw)
    tiles = [-(-n // R.TILE) for n in lens]
    total = sum(tiles) * (hkv // hw) if P == 0 else None
    C = max(R.MIN_CHUNK, -(-total // nw)) if P == 0 else P // R.TILE
    by_pair = {}
    for s, g, k, lo, hi in items:
        by_pair.setdefault((s, g), []).append((k, lo, hi))
    for s in range(B):
        for g in range(hkv):
            segs = sorted(by_pair.get((s, g), []))
            if lens[s] == 0:
                assert segs == []
                continue
            assert [k for k, _, _ in segs] == list(range(len(segs)))
            assert segs[0][1] == 0 and segs[-1][2] == lens[s]
            for (_, lo, hi), (_, lo2, _) in zip(segs, segs[1:]):
                assert hi == lo2
            for _, lo, hi in segs:
                assert lo < hi and -(-hi // R.TILE) - lo // R.TILE <= C
            if P:
                assert len(segs) == -(-lens[s] // P)
                assert all(lo % P == 0 for _, lo, _ in segs)
    if P == 0:
        seg_tiles = sum(-(-hi // R.TILE) - lo // R.TILE for s, g, k, lo, hi in items if g % hw == 0)
        assert seg_tiles == total


# ---------------------------------------------------------------- host tier

GOLDEN_TIER = os.path.join(os.path.dirname(__file__), "golden", "tiered_evict_to_cpu.json")


def _seq_with_blocks(pool, blocks, bs):
    return pool.import_seq(blocks, len(blocks) * bs)


def test_golden_tiered_evict_to_cpu():
    g = json.load(open(GOLDEN_TIER))
    for case in g["cases"]:
        pool = R.PoolReplay(16, 4, max_seqs=2, max_blocks_per_seq=8)
        pool.attach_host_tier(8)
        sid = _seq_with_blocks(pool, g["blocks"], 4)
        copies = pool.offload([sid], case["gpu_window"])
        assert [b for b, _ in copies] == case["cold"]
        # host blocks come out 0, 1, 2, ... and replace the cold entries in place
        assert [c for _, c in copies] == list(range(len(case["cold"])))
        blocks = pool.seqs[sid][0]
        assert blocks[len(case["cold"]):] == case["kept"]
        assert [R.PoolReplay.host_id(e) for e in blocks[:len(case["cold"])]] == list(range(len(case["cold"])))
        # cold GPU blocks went back to the free list in logical order (last one on top)
        if case["cold"]:
            assert pool.free[-len(case["cold"]):] == case["cold"]
    # the listing's gpu_window = 0 slice moves nothing; the replay refuses the case instead
    assert g["blocks"][:-0] == g["listing_quirk"]["listing_cold"]
    pool = R.PoolReplay(16, 4, max_seqs=2, max_blocks_per_seq=8)
    pool.attach_host_tier(8)
    sid = _seq_with_blocks(pool, g["blocks"], 4)
    with pytest.raises(R.PoolError):
        pool.offload([sid], 0)


def test_offload_restore_round_trip_and_parking():
    pool = R.PoolReplay(12, 4, max_seqs=4, max_blocks_per_seq=8, alloc_order=list(range(11, -1, -1)))
    pool.attach_host_tier(6)
    a = pool.add_seq()
    for _ in range(18):                      # 5 blocks: 11, 10, 9, 8, 7
        pool.append([a])
    b = pool.add_seq()
    for _ in range(5):                       # 2 blocks: 6, 5
        pool.append([b])
    assert pool.seqs[a][0] == [11, 10, 9, 8, 7]
    copies = pool.offload([a, b], 2)
    assert copies == [(11, 0), (10, 1), (9, 2)]
    assert pool.seqs[a][0] == [-2, -3, -4, 8, 7] and pool.parked(a) and not pool.parked(b)
    tab, lens = pool.tables()
    assert lens[a] == 0 and tab[a] == [-1] * 8 and lens[b] == 5
    with pytest.raises(R.PoolError):
        pool.append([a])
    assert pool.num_host_free() == 3
    back = pool.restore([a, b])
    # free list top was 9 (freed last), then 10, 11
    assert back == [(0, 9), (1, 10), (2, 11)]
    assert pool.seqs[a][0] == [9, 10, 11, 8, 7] and not pool.parked(a)
    assert pool.num_host_free() == 6 and pool.host_free[-3:] == [0, 1, 2]
    assert pool.append([a])[0][1] == 7 * 4 + 2      # slot in the tail block, offset 2


def test_offload_all_or_nothing():
    pool = R.PoolReplay(16, 4, max_seqs=4, max_blocks_per_seq=8)
    pool.attach_host_tier(3)
    a = _seq_with_blocks(pool, [0, 1, 2, 3], 4)
    b = _seq_with_blocks(pool, [4, 5, 6], 4)
    snap = (list(pool.free), list(pool.host_free), [list(x[0]) for x in pool.seqs.values()])
    with pytest.raises(R.PoolError):
        pool.offload([a, b], 1)              # needs 3 + 2 host blocks, 3 free
    assert snap == (list(pool.free), list(pool.host_free), [list(x[0]) for x in pool.seqs.values()])
    with pytest.raises(R.PoolError):
        pool.offload([a, a], 1)
    pool.offload([a], 1)
    full = R.PoolReplay(4, 4, max_seqs=2, max_blocks_per_seq=4)
    full.attach_host_tier(4)
    s = _seq_with_blocks(full, [0, 1, 2], 4)
    full.offload([s], 1)
    t = _seq_with_blocks(full, [0, 1, 3], 4)
    with pytest.raises(R.PoolError):
        full.restore([s])                    # 2 host blocks back, 0 GPU blocks free
    assert full.seqs[s][0] == [-2, -3, 2]


def test_offload_shared_block_copies_for_the_mover_only():
    pool = R.PoolReplay(16, 4, max_seqs=4, max_blocks_per_seq=8)
    pool.attach_host_tier(8)
    a = _seq_with_blocks(pool, [3, 4, 5], 4)
    b = pool.fork(a)
    copies = pool.offload([a], 1)
    assert copies == [(3, 0), (4, 1)]
    assert pool.ref[3] == 1 and pool.ref[4] == 1 and pool.seqs[b][0] == [3, 4, 5]
    assert 3 not in pool.free
    c = pool.fork(a)                          # a parked sequence forks with its host blocks
    assert pool.host_ref[0] == 2
    pool.free_seq(a)
    assert pool.host_ref[0] == 1 and 0 not in pool.host_free
    pool.free_seq(c)
    assert pool.host_free[-2:] == [0, 1]


def test_random_tier_ops_conserve_blocks():
    rnd = random.Random(1)
    pool = R.PoolReplay(48, 4, max_seqs=8, max_blocks_per_seq=12)
    pool.attach_host_tier(24)
    live = []
    for _ in range(3000):
        op = rnd.random()
        try:
            if op < 0.08 and len(live) < 8:
                live.append(pool.add_seq())
            elif op < 0.12 and live and len(live) < 8:
                live.append(pool.fork(rnd.choice(live)))
            elif op < 0.17 and live:
                s = rnd.choice(live); live.remove(s); pool.free_seq(s)
            elif op < 0.27 and live:
                pool.offload(rnd.sample(live, rnd.randint(1, len(live))), rnd.randint(1, 4))
            elif op < 0.37 and live:
                pool.restore(rnd.sample(live, rnd.randint(1, len(live))))
            elif live:
                pool.append(rnd.sample(live, rnd.randint(1, len(live))))
        except R.PoolError:
            pass
        held, hheld = {}, {}
        for blocks, n in pool.seqs.values():
            assert len(blocks) == R.blocks_needed(n, 4)
            for e in blocks:
                d = hheld if e <= -2 else held
                k = -2 - e if e <= -2 else e
                d[k] = d.get(k, 0) + 1
        assert all(pool.ref[b] == c for b, c in held.items())
        assert all(pool.host_ref[b] == c for b, c in hheld.items())
        assert len(held) + len(pool.free) == 48 and not set(held) & set(pool.free)
        assert len(hheld) + len(pool.host_free) == 24 and not set(hheld) & set(pool.host_free)


def test_append_tokens_is_sequential_single_appends():
    rnd = random.Random(5)
    for trial in range(40):
        order = list(range(40))
        rnd.shuffle(order)
        setup = [rnd.randint(0, 9) for _ in range(3)]
        fork = rnd.random() < 0.5
        pools = []
        for _ in range(2):
            pool = R.PoolReplay(40, 4, max_seqs=6, max_blocks_per_seq=12, alloc_order=order)
            for c in setup:
                sid = pool.add_seq()
                for _ in range(c):
                    pool.append([sid])
            if fork:
                pool.fork(0)
            pools.append(pool)
        a, b = pools
        ids = sorted(a.seqs)
        rnd.shuffle(ids)
        counts = [rnd.randint(0, 9) for _ in ids]
        try:
            got = a.append_tokens(ids, counts)
        except R.PoolError:
            continue
        want = []
        for s_, c in zip(ids, counts):
            for _ in range(c):
                want += b.append([s_])
        assert got == want and a.seqs == b.seqs and a.free == b.free and a.ref == b.ref


def test_append_tokens_all_or_nothing():
    pool = R.PoolReplay(6, 4, max_seqs=3, max_blocks_per_seq=4)
    s, t = pool.add_seq(), pool.add_seq()
    snap = (list(pool.free), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()})
    with pytest.raises(R.PoolError):
        pool.append_tokens([s, t], [12, 13])      # 3 + 4 blocks > 6 free
    with pytest.raises(R.PoolError):
        pool.append_tokens([s], [17])             # 5 blocks > max_blocks_per_seq
    assert snap == (list(pool.free), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()})
    items = pool.append_tokens([s, t], [5, 3])
    assert [it[0] for it in items] == [s] * 5 + [t] * 3
    assert pool.seqs[s][1] == 5 and pool.seqs[t][1] == 3


def test_segment_rows_worked_examples():
    """Balanced: lengths 5, 700, 40, two kv heads, 4 waves: 1 + 44 + 3 tiles per kv head, T = 96,
    C = max(4, 24) = 24.  Pair (1, 1) starts at list position 46 and spans chunks 1, 2, 3; its
    pair index is 3, so its rows are 4, 5, 6.  Fixed P = 128 (C = 8 tiles): lengths 300, 40 pad to
    24 and 8 tiles; pair (0, 1) starts at 24 (chunks 3, 4, 5, pair 1: rows 4, 5, 6), pair (1, 1) at
    56 (chunk 7, pair 3: row 10)."""
    assert R.segment_rows([5, 700, 40], 2, 0, 4) == {
        (0, 0, 0): 0, (0, 1, 0): 1, (1, 0, 0): 2, (1, 0, 1): 3, (1, 1, 0): 4, (1, 1, 1): 5, (1, 1, 2): 6,
        (2, 0, 0): 7, (2, 1, 0): 8}
    assert R.segment_rows([300, 40], 2, 128, 4) == {
        (0, 0, 0): 0, (0, 0, 1): 1, (0, 0, 2): 2, (0, 1, 0): 4, (0, 1, 1): 5, (0, 1, 2): 6,
        (1, 0, 0): 8, (1, 1, 0): 10}


@pytest.mark.parametrize("seed", range(8))
def test_segment_rows_distinct_and_bounded(seed):
    """Every segment of the plan has a row; rows of distinct pairs or slots differ, the kv heads of
    one group share theirs, and all rows are below chunks + pairs (balanced: at most num_waves
    chunks; fixed: at most ceil(max_len / P) per pair)."""
    rnd = random.Random(seed)
    B = rnd.randint(1, 40)
    lens = [rnd.choice([0, 1, 15, 16, 17, rnd.randint(0, 5000)]) for _ in range(B)]
    hw = rnd.choice([1, 2])
    hkv = hw * rnd.randint(1, 4)
    P = rnd.choice([0, 0, 16, 64, 512])
    nw = rnd.choice([1, 4, 64, 2048])
    items = R.plan(lens, hkv, P, nw, heads_per_wave=hw)
    rows = R.segment_rows(lens, hkv, P, nw, heads_per_wave=hw)
    assert set(rows) == {(s, g, k) for s, g, k, _, _ in items}
    pairs = B * (hkv // hw)
    chunks = nw if P == 0 else pairs * max(1, -(-max(lens) // P)) if max(lens) else pairs
    by_row = {}
    for (s, g, k), r in rows.items():
        assert 0 <= r < chunks + pairs
        by_row.setdefault(r, set()).add((s, g // hw, k))
    assert all(len(v) == 1 for v in by_row.values())
