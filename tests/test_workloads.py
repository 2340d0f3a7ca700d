"""The seeded input generators: reproducible, well-formed, and shaped as the workloads say."""

import numpy as np
import pytest

from paged_kv_cache_tv_amd import workloads as W


def _check_batch(b):
    S = b.num_seqs
    assert b.block_tables.dtype == np.int32 and b.block_tables.shape[0] == S
    assert b.q.shape == (S, b.num_q_heads, b.head_dim) and b.q.dtype == np.uint16
    assert (b.block_tables >= 0).all() and (b.block_tables < b.num_blocks).all()
    # every slot written (fill + step) is unique and inside the pool
    slots = np.concatenate([b.fill_slots, b.new_slots[b.new_slots >= 0]])
    assert len(np.unique(slots)) == len(slots)
    assert (slots >= 0).all() and (slots < b.num_blocks * b.block_size).all()
    for s in range(S):
        n = int(b.context_lens[s])
        nb = W.blocks_needed(n, b.block_size)
        assert len(b.token_rows[s]) == n
        # unused table entries point at the never-allocated poison block
        assert (b.block_tables[s, nb:] == b.poison_block).all()
        assert b.poison_block not in set(b.block_tables[s, :nb].tolist())
        if n:
            last = b.block_tables[s, (n - 1) // b.block_size] * b.block_size + (n - 1) % b.block_size
            assert b.new_slots[s] == last
    return b


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], np.float32)
    bits = W.round_to_bf16_bits(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7: ties go to the even mantissa (1.0)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82
    assert bits[3] == 0xC020
    back = W.bf16_bits_to_float32(bits)
    assert back[0] == 1.0 and back[3] == -2.5


@pytest.mark.parametrize("i", [1, 2, 3])
def test_workloads_wellformed_and_reproducible(i):
    a = _check_batch(W.make_workload(i))
    b = W.make_workload(i)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.kv_k[:1000], b.kv_k[:1000]) and np.array_equal(a.q, b.q)


def test_workload_1_shape():
    b = W.make_workload(1)
    assert b.num_seqs == 1 and int(b.context_lens[0]) == 37 and b.num_blocks == 8
    t = b.block_tables[0]
    assert len(t) == 3 and len(set(t.tolist())) == 3
    assert not (t[1] == t[0] + 1 and t[2] == t[1] + 1)
    # the 37th token goes to offset 4 of the third block
    assert b.new_slots[0] == t[2] * 16 + 4


def test_workload_2_3_ranges():
    b2 = W.make_workload(2)
    assert b2.num_seqs == 8 and b2.num_blocks == 1024
    assert (b2.context_lens >= 128).all() and (b2.context_lens <= 1024).all()
    b3 = W.make_workload(3)
    assert b3.num_seqs == 64
    assert (b3.context_lens >= 512).all() and (b3.context_lens <= 4096).all()
    need = sum(W.blocks_needed(int(n)) for n in b3.context_lens)
    assert b3.num_blocks == need + int(np.ceil(0.1 * need))
    q = W.bf16_bits_to_float32(b3.q)
    assert 0.45 < q.std() < 0.55              # q ~ N(0, 0.5)


def test_shared_prefix_structure():
    b = W.make_shared_prefix_batch(3, 4, 64, [0, 5, 16, 40, 1, 2, 3, 4, 0, 0, 31, 32], seed=7)
    _check_batch(b)
    for i in range(3):
        rows = [b.block_tables[i * 4 + j, :4] for j in range(4)]
        assert all(np.array_equal(rows[0], r) for r in rows)           # 4 tables share the prefix blocks
        for j in range(4):
            assert np.array_equal(b.token_rows[i * 4 + j][:64], b.token_rows[i * 4][:64])
    # each prefix token is written once
    assert len(b.fill_slots) == len(np.unique(b.fill_slots))
    assert b.kv_k.shape[0] == 3 * 64 + sum(r + 1 for r in [0, 5, 16, 40, 1, 2, 3, 4, 0, 0, 31, 32])
    # the step's writes never land in a shared block
    shared = set(b.block_tables[:, :4].ravel().tolist())
    assert not (set((b.new_slots // 16).tolist()) & shared)


def test_outlier_rule():
    b = W.make_batch([200], 3, k_outlier_period=97, k_outlier_factor=8.0)
    b0 = W.make_batch([200], 3)
    k, k0 = W.bf16_bits_to_float32(b.kv_k), W.bf16_bits_to_float32(b0.kv_k)
    for t in range(200):
        if t % 97 == 96:
            assert np.array_equal(k[t], 8 * k0[t])
        else:
            assert np.array_equal(k[t], k0[t])
