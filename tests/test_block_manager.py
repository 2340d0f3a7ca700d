"""The block manager (tv_bm_*) on the CPU: the pages' paging example,
copy-on-write after a fork, error handling that leaves the state unchanged,
and bookkeeping invariants under long random operation sequences.

The manager is host code inside libtv; these tests load the library but launch
nothing on a GPU."""

import json
import os

import numpy as np
import pytest

import paged_kv_cache_tv_amd as tv

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BS = 16


def _bm(num_blocks=64, max_seqs=16, width=64):
    return tv.BlockManager(num_blocks, BS, max_seqs, width)


def test_pages_paging_example():
    """'vLLM' page, section '가상 메모리 방식의 해결': 300 tokens take 19 blocks
    and leave 4 free slots in the last one; further blocks are added only as
    tokens arrive."""
    g = json.load(open(os.path.join(GOLDEN, "paging_examples.json")))["on_demand"]
    bm = _bm()
    bm.add_sequence(0, g["tokens"])
    table = bm.block_table(0)
    assert len(table) == g["blocks"]
    assert bm.num_free() == 64 - g["blocks"]
    assert len(set(table.tolist())) == g["blocks"]
    last = int(table[-1])
    for i in range(g["free_slots_in_last_block"]):          # the 4 free slots, no allocation
        slot, src, dst = bm.append_slot(0)
        assert slot == last * BS + (g["tokens"] % BS) + i and src == dst == -1
        assert bm.num_free() == 64 - g["blocks"]
    slot, src, dst = bm.append_slot(0)                       # the 305th token opens block 20
    assert bm.num_free() == 64 - g["blocks"] - 1
    assert slot % BS == 0 and slot // BS not in table.tolist() and src == dst == -1
    assert bm.length(0) == g["tokens"] + g["free_slots_in_last_block"] + 1
    assert (bm.slots(0, 0, 3) == table[0] * BS + np.arange(3)).all()


def test_fork_shares_and_copies_on_write():
    bm = _bm()
    bm.add_sequence(0, 40)                                   # blocks b0, b1, b2 (8 tokens in b2)
    t0 = bm.block_table(0).tolist()
    bm.fork(0, 1)
    bm.fork(0, 2)
    assert bm.block_table(1).tolist() == t0 and bm.block_table(2).tolist() == t0
    assert [bm.refcount(b) for b in t0] == [3, 3, 3]
    free = bm.num_free()
    # Sample 1 writes position 40 into the shared, partly filled last block: copy on write.
    slot, src, dst = bm.append_slot(1)
    assert src == t0[2] and dst not in t0 and slot == dst * BS + 8
    assert bm.block_table(1).tolist() == t0[:2] + [dst]
    assert bm.refcount(t0[2]) == 2 and bm.refcount(dst) == 1 and bm.num_free() == free - 1
    # Its next write stays in its own block.
    assert bm.append_slot(1) == (dst * BS + 9, -1, -1)
    # The last sharer of b2 writes in place once the others have their copies.
    s2 = bm.append_slot(2)
    assert s2[1] == t0[2] and bm.refcount(t0[2]) == 1
    assert bm.append_slot(0) == (t0[2] * BS + 8, -1, -1)
    # Freeing returns only blocks nobody refers to.
    before = bm.num_free()
    bm.free_sequence(1)
    assert bm.num_free() == before + 1                       # its private copy
    bm.free_sequence(2)
    bm.free_sequence(0)
    assert bm.num_free() == 64


def test_fork_at_block_boundary_needs_no_copy():
    bm = _bm()
    bm.add_sequence(0, 32)
    bm.fork(0, 1)
    slot, src, dst = bm.append_slot(1)                       # position 32 opens a fresh block
    assert src == dst == -1 and slot % BS == 0
    assert bm.refcount(bm.block_table(0)[-1]) == 2


def test_errors_leave_state_unchanged():
    bm = _bm(num_blocks=4, max_seqs=4, width=3)
    bm.add_sequence(0, 16)
    with pytest.raises(tv.TvError) as e:
        bm.add_sequence(0, 1)                                # sequence in use
    assert e.value.status == 2
    with pytest.raises(tv.TvError) as e:
        bm.add_sequence(1, 49)                               # 4 blocks > width 3
    assert e.value.status == 2
    bm.add_sequence(1, 33)                                   # 3 blocks: pool now empty
    assert bm.num_free() == 0
    with pytest.raises(tv.TvError) as e:
        bm.append_slot(0)                                    # needs a block, none free
    assert e.value.status == 6
    assert bm.length(0) == 16 and bm.num_free() == 0
    bm.fork(1, 2)
    with pytest.raises(tv.TvError) as e:
        bm.append_slot(2)                                    # copy on write, none free
    assert e.value.status == 6
    assert bm.length(2) == 33 and bm.refcount(bm.block_table(2)[-1]) == 2
    with pytest.raises(tv.TvError) as e:
        bm.append_slot(3)                                    # unused sequence
    assert e.value.status == 2
    with pytest.raises(tv.TvError) as e:
        bm.fork(3, 0)                                        # child in use / parent unused
    assert e.value.status == 2
    with pytest.raises(tv.TvError) as e:
        bm.slots(0, 10, 7)                                   # past the sequence's length
    assert e.value.status == 2
    bm.free_sequence(2)
    bm.free_sequence(1)
    assert bm.num_free() == 3
    with pytest.raises(tv.TvError):
        tv.BlockManager(0, BS, 1, 1)


def _check_invariants(bm, live, num_blocks):
    refs = np.zeros(num_blocks, np.int64)
    for seq, n in live.items():
        assert bm.length(seq) == n
        table = bm.block_table(seq)
        assert len(table) == -(-n // BS)
        assert len(set(table.tolist())) == len(table)
        np.add.at(refs, table, 1)
    for b in range(num_blocks):
        assert bm.refcount(b) == refs[b]
    assert bm.num_free() == int((refs == 0).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_operations_keep_the_books(seed):
    """Random add / fork / append / free: reference counts equal the number of
    tables holding each block, free blocks are exactly the unreferenced ones, a
    slot just handed out lies in a block its sequence owns alone, and no two
    live positions of different sequences share a slot unless their block is
    shared."""
    rng = np.random.default_rng(seed)
    NB, SEQS = 48, 12
    bm = tv.BlockManager(NB, BS, SEQS, NB)
    live = {}
    for step in range(400):
        op = rng.integers(4)
        free_ids = [s for s in range(SEQS) if s not in live]
        if op == 0 and free_ids:
            s, n = int(rng.choice(free_ids)), int(rng.integers(0, 60))
            try:
                bm.add_sequence(s, n)
                live[s] = n
            except tv.TvError as e:
                assert e.status == 6
        elif op == 1 and live and free_ids:
            p, c = int(rng.choice(list(live))), int(rng.choice(free_ids))
            bm.fork(p, c)
            live[c] = live[p]
        elif op == 2 and live:
            s = int(rng.choice(list(live)))
            try:
                slot, src, dst = bm.append_slot(s)
            except tv.TvError as e:
                assert e.status == 6
            else:
                table = bm.block_table(s)
                assert slot == table[live[s] // BS] * BS + live[s] % BS
                assert bm.refcount(int(slot // BS)) == 1, "a written block must not be shared"
                if src >= 0:
                    assert dst == slot // BS and src != dst and bm.refcount(src) >= 1
                live[s] += 1
        elif op == 3 and live:
            s = int(rng.choice(list(live)))
            bm.free_sequence(s)
            del live[s]
        _check_invariants(bm, live, NB)


def _state(bm, seqs, num_blocks):
    """Everything observable about a manager: lengths, tables, reference counts,
    and the order in which free blocks would be handed out."""
    live = {s: (bm.length(s), bm.block_table(s).tolist()) for s in seqs if bm.length(s) >= 0}
    refs = [bm.refcount(b) for b in range(num_blocks)]
    return live, refs, bm.num_free()


def _free_order(bm, num_blocks, probe_seq):
    """The free list from the top down, read by taking every free block with one
    add_sequence on an unused sequence number (then giving them back)."""
    n = bm.num_free()
    if n == 0:
        return []
    bm.add_sequence(probe_seq, n * BS)
    order = bm.block_table(probe_seq).tolist()
    bm.free_sequence(probe_seq)
    return order


def _scenario(seed, NB=96, SEQS=24, width=24):
    rng = np.random.default_rng(seed)
    bm = tv.BlockManager(NB, BS, SEQS + 1, width)
    live = []
    for i in range(6):
        bm.add_sequence(3 * i, int(rng.integers(1, 100)))
        live.append(3 * i)
        for j in (1, 2):
            if rng.random() < 0.7:
                bm.fork(3 * i, 3 * i + j)
                live.append(3 * i + j)
    return bm, live, rng


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_prepare_decode_equals_per_sequence_appends(seed):
    """A batch call gives the same slots, tables, lengths and copy pairs as
    append_slot / block_table / length called per sequence in the same order on
    an identical manager, over several steps with forks sharing blocks."""
    a, live, rng = _scenario(seed)
    b, _, _ = _scenario(seed)
    width = 24
    for step in range(20):
        order = [int(s) for s in rng.permutation(live)]
        tables, lens, slots, pairs = a.prepare_decode(order, width)
        exp_pairs = []
        for r, s in enumerate(order):
            slot, src, dst = b.append_slot(s)
            assert slots[r] == slot and lens[r] == b.length(s)
            t = b.block_table(s)
            assert (tables[r, :len(t)] == t).all() and (tables[r, len(t):] == 0).all()
            if src >= 0:
                exp_pairs.append((src, dst))
        assert pairs.tolist() == [list(p) for p in exp_pairs]
        # The outputs meet tv_copy_blocks' and the fused append's preconditions.
        dsts = pairs[:, 1].tolist()
        assert len(set(dsts)) == len(dsts) and not set(dsts) & set(pairs[:, 0].tolist())
        for r, s in enumerate(order):
            assert a.refcount(int(slots[r] // BS)) == 1
            assert slots[r] == tables[r, (lens[r] - 1) // BS] * BS + (lens[r] - 1) % BS
        assert _state(a, range(25), 96) == _state(b, range(25), 96)


def test_prepare_decode_rolls_back_when_blocks_run_out():
    bm = tv.BlockManager(10, BS, 8, 8)
    bm.add_sequence(0, 20)            # blocks 0, 1 (4 tokens in block 1)
    bm.fork(0, 1)
    bm.fork(0, 2)
    bm.add_sequence(3, 32)            # blocks 2, 3: position 32 opens a block
    bm.add_sequence(4, 80)            # blocks 4..8: one block left free
    before = _state(bm, range(8), 10)
    order_before = _free_order(bm, 10, 7)
    # Needs: seq 1 copy, seq 2 copy, seq 3 new block, seq 0 in place -> 3 blocks, 1 free.
    free = bm.num_free()
    assert free < 3
    for order in ([1, 2, 3, 0], [3, 1, 2]):      # undo a copy / a new block
        with pytest.raises(tv.TvError) as e:
            bm.prepare_decode(order, 8)
        assert e.value.status == 6
        assert _state(bm, range(8), 10) == before
        assert _free_order(bm, 10, 7) == order_before
    # The same step succeeds once blocks are returned.
    bm.free_sequence(4)
    tables, lens, slots, pairs = bm.prepare_decode([1, 2, 3, 0], 8)
    assert len(pairs) == 2 and lens.tolist() == [21, 21, 33, 21]


def test_prepare_decode_argument_errors_change_nothing():
    bm = tv.BlockManager(16, BS, 4, 3)
    bm.add_sequence(0, 16)
    bm.add_sequence(1, 48)            # 3 blocks: its next position needs a 4th
    before = _state(bm, range(4), 16)
    for seqs, width in (([0, 0], 3),      # repeated sequence
                        ([0, 2], 3),      # unused sequence
                        ([0, 9], 3),      # out of range
                        ([0], 1),         # 2 blocks after the append > width 1
                        ([1], 8)):        # 4 blocks > max_blocks_per_seq 3
        with pytest.raises(tv.TvError) as e:
            bm.prepare_decode(seqs, width)
        assert e.value.status == 2, (seqs, width)
        assert _state(bm, range(4), 16) == before
    tables, lens, slots, pairs = bm.prepare_decode([], 3)
    assert tables.shape == (0, 3) and len(pairs) == 0
