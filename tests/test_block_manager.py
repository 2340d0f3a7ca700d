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
