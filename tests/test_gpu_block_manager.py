"""Copy-on-write on the GPU, and live parallel sampling driven by the block manager.

* tv_copy_blocks against the oracle's block copy: whole pools bit-exact.
* Prompts are prefilled, each forked into four samples that share the prompt's
  blocks, then several decode steps run. Each step asks the manager for slots
  (per sequence, or with one tv_bm_prepare_decode call), copies shared blocks
  on write (tv_copy_blocks), and runs the two-launch step.
  After every step:
  - each live sequence's K/V, gathered from the GPU pools through its own
    block table, equals that sequence's token history bit for bit;
  - the attention output matches the oracle on pools the oracle builds from
    those histories with the same tables.
  Samples are freed midway, so freed blocks are reused.
"""

import numpy as np
import pytest

import oracle as O
from paged_kv_cache_tv_amd import workloads as W

pytestmark = pytest.mark.gpu

HKV, HQ, D, BS = 8, 32, 64, 16
CONTRACT_MAX, CONTRACT_MEAN, INTERNAL_MAX = 1e-2, 1e-3, 1e-4


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_cache_tv_amd as tv
    tv.lib()
    return torch.device("cuda:0")


def _bf16(rng, shape):
    return W.round_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _to_dev(a, dev):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("count", [100, 700])
def test_copy_blocks_parity(dev, oracle_lib, count):
    """Whole pools bit-exact after the copy, in both launch shapes (up to 512
    pairs: 256-thread workgroups; more: 128-thread ones), with skipped pairs
    (source = destination, out of range)."""
    import torch
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(50 + count)
    NB = 3 * count
    kc_ref = _bf16(rng, (NB, HKV, D // 8, BS, 8))
    vc_ref = _bf16(rng, (NB, HKV, D, BS))
    src = rng.choice(NB // 2, size=count, replace=False)
    dst = NB // 2 + rng.choice(NB // 2, size=count, replace=False)
    pairs = np.stack([src, dst], 1).astype(np.int64)
    pairs = np.concatenate([pairs, [[7, 7], [NB, 3], [-1, 5], [4, NB + 9]]])   # skipped pairs
    kc, vc = _to_dev(kc_ref, dev), _to_dev(vc_ref, dev)
    assert oracle_lib.copy_blocks(kc_ref, vc_ref, pairs) == count
    tv.copy_blocks(kc, vc, _to_dev(pairs, dev))
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), kc_ref)
    assert np.array_equal(vc.cpu().numpy().view(np.uint16), vc_ref)


def _gather(kc, vc, slots):
    blk, off = slots // BS, slots % BS
    k = kc[blk, :, :, off, :].reshape(len(slots), HKV, D)
    v = vc[blk, :, :, off].reshape(len(slots), HKV, D)
    return k, v


@pytest.mark.parametrize("batch_call", [False, True], ids=["per-sequence", "prepare_decode"])
def test_parallel_sampling_live(dev, oracle_lib, batch_call):
    import torch
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(51)
    NB, SEQS, WIDTH = 640, 32, 128
    bm = tv.BlockManager(NB, BS, SEQS, WIDTH)
    kc, vc = tv.new_pools(NB, HKV, D, BS, dev, fill=W.BF16_NAN)
    hist = {}                                       # seq -> (K rows, V rows), uint16 [n, HKV, D]
    prompts = [37, 100, 255, 256, 511, 700]
    for i, n in enumerate(prompts):
        seq = 4 * i
        bm.add_sequence(seq, n)
        k, v = _bf16(rng, (n, HKV, D)), _bf16(rng, (n, HKV, D))
        tv.cache_write(_to_dev(k, dev), _to_dev(v, dev), kc, vc, _to_dev(bm.slots(seq, 0, n), dev))
        hist[seq] = (k, v)
        for j in (1, 2, 3):
            bm.fork(seq, seq + j)
            hist[seq + j] = (k, v)
    copies_seen = 0
    for step in range(4):
        if step == 2:                               # drop one sample per prompt
            for i in range(len(prompts)):
                bm.free_sequence(4 * i + 3)
                del hist[4 * i + 3]
        live = sorted(hist)
        S = len(live)
        k_new, v_new = _bf16(rng, (S, HKV, D)), _bf16(rng, (S, HKV, D))
        if batch_call:
            tables, lens, slots, pairs = bm.prepare_decode(live, WIDTH)
            pairs = [tuple(p) for p in pairs.tolist()]
        else:
            slots, pairs = [], []
            for seq in live:
                slot, src, dst = bm.append_slot(seq)
                slots.append(slot)
                if src >= 0:
                    pairs.append((src, dst))
            lens = np.array([bm.length(s) for s in live], np.int32)
            tables = np.zeros((S, WIDTH), np.int32)
            for r, seq in enumerate(live):
                t = bm.block_table(seq)
                tables[r, :len(t)] = t
        for r, seq in enumerate(live):
            k, v = hist[seq]
            hist[seq] = (np.concatenate([k, k_new[r:r + 1]]), np.concatenate([v, v_new[r:r + 1]]))
        copies_seen += len(pairs)
        if pairs:
            tv.copy_blocks(kc, vc, _to_dev(np.array(pairs, np.int64), dev))
        q = _bf16(rng, (S, HQ, D))
        max_ctx = int(lens.max())
        ws = tv.new_workspace(S, HQ, D, max_ctx, 512, dev)
        out = torch.empty((S, HQ, D), dtype=torch.float32, device=dev)
        q_d, bt_d, cl_d = _to_dev(q, dev), _to_dev(tables, dev), _to_dev(lens, dev)
        tv.paged_attention_decode_append(*ws, q_d, _to_dev(k_new, dev), _to_dev(v_new, dev),
                                         _to_dev(np.array(slots, np.int64), dev), kc, vc, bt_d,
                                         cl_d, max_ctx, 512, 0.125)
        tv.paged_attention_reduce(out, *ws, cl_d, max_ctx, 512)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        # Every live sequence reads exactly its own history through its table.
        kc_h, vc_h = kc.cpu().numpy().view(np.uint16), vc.cpu().numpy().view(np.uint16)
        for seq in live:
            gk, gv = _gather(kc_h, vc_h, bm.slots(seq, 0, bm.length(seq)))
            assert np.array_equal(gk, hist[seq][0]), f"step {step}: K of sequence {seq}"
            assert np.array_equal(gv, hist[seq][1]), f"step {step}: V of sequence {seq}"
        # Attention against the oracle on pools it writes itself from the histories.
        kr, vr = O.Oracle.new_pools(NB, HKV, D, BS)
        for seq in live:
            oracle_lib.cache_write(hist[seq][0], hist[seq][1], kr, vr,
                                   bm.slots(seq, 0, bm.length(seq)))
        ref = oracle_lib.paged_attention(q, kr, vr, tables, lens, 0.125)
        err = np.abs(got.astype(np.float64) - ref)
        print(f"step {step}: {S} sequences, {len(pairs)} block copies, max_abs={err.max():.3e}",
              flush=True)
        assert np.isfinite(got).all()
        assert err.max() <= min(CONTRACT_MAX, INTERNAL_MAX) and err.mean() <= CONTRACT_MEAN
    assert copies_seen > 0, "the scenario never exercised copy-on-write"
    for seq in list(hist):
        bm.free_sequence(seq)
    assert bm.num_free() == NB
