"""The whole hot path as an engine would drive it, on the GPU, against the oracle.

Prompts are admitted by the block manager and prefilled:
  * their K/V are written with the rotary embedding applied
    (tv_cache_write_rope);
  * q is rotated in place (tv_rope);
  * prefill attention runs (tv_paged_attention_prefill).
Each prompt is then forked into samples, and several decode steps follow
(while all samples live, the shared-prefix pass is run on the same pools too
and must reproduce the step's output bit for bit).
Each step:
  * reserves slots and copy-on-write pairs (tv_bm_prepare_decode);
  * copies the shared blocks (tv_copy_blocks);
  * rotates the new q and K (tv_rope);
  * runs the fused step (tv_paged_attention_decode_append, then
    tv_paged_attention_reduce).

The oracle side keeps the token histories, rotates them with its own RoPE,
writes its own pools through the same tables and computes prefill and decode
attention.  No value the oracle uses comes from the GPU.  Where a rotated
bf16 value on the GPU lands on the other neighbour of a near-tie (see
tests/test_gpu_rope.py), attention moves by far less than the bars used here.
"""

import numpy as np
import pytest

import oracle as O
from paged_kv_cache_tv_amd import workloads as W

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS, PART = 32, 8, 64, 16, 512
SCALE = 0.125


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_cache_tv_amd as tv
    tv.lib()
    return torch.device("cuda:0")


def _to_dev(a, dev):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _bf16(rng, shape):
    return W.round_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_engine_flow(dev, oracle_lib):
    import torch
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(130)
    NB, WIDTH, SAMPLES = 400, 64, 3
    prompts = [45, 300, 513]
    nseq = len(prompts) * SAMPLES
    bm = tv.BlockManager(NB, BS, nseq, WIDTH)
    f = W.rope_inv_freq(D, 500000.0)
    fd = _to_dev(f, dev)
    kc, vc = tv.new_pools(NB, HKV, D, BS, dev, fill=W.BF16_NAN)
    kr, vr = O.Oracle.new_pools(NB, HKV, D, BS)
    hist = {}                          # sequence -> (raw K rows, V rows), uint16 [n, HKV, D]

    # Prefill: every prompt in one call, rows of sequence i*SAMPLES.
    q_rows, qs, tables, lens = [], [0], [], []
    for i, n in enumerate(prompts):
        seq = i * SAMPLES
        bm.add_sequence(seq, n)
        k, v = _bf16(rng, (n, HKV, D)), _bf16(rng, (n, HKV, D))
        pos = np.arange(n, dtype=np.int32)
        slots = bm.slots(seq, 0, n)
        tv.cache_write_rope(_to_dev(k, dev), _to_dev(v, dev), kc, vc, _to_dev(slots, dev),
                            _to_dev(pos, dev), fd, 0)
        oracle_lib.cache_write(oracle_lib.rope(k, pos, f, 0)[1], v, kr, vr, slots)
        hist[seq] = (k, v)
        q_rows.append(_bf16(rng, (n, HQ, D)))
        qs.append(qs[-1] + n)
        row = np.zeros(WIDTH, np.int32)
        t = bm.block_table(seq)
        row[:len(t)] = t
        tables.append(row)
        lens.append(n)
    q = np.concatenate(q_rows)
    qs, tables, lens = np.array(qs, np.int32), np.stack(tables), np.array(lens, np.int32)
    pos_q = np.concatenate([np.arange(n, dtype=np.int32) for n in prompts])
    qd = _to_dev(q, dev)
    tv.rope(qd, _to_dev(pos_q, dev), fd, 0)
    out = torch.empty((len(q), HQ, D), dtype=torch.float32, device=dev)
    tv.paged_attention_prefill(out, qd, _to_dev(qs, dev), kc, vc, _to_dev(tables, dev),
                               _to_dev(lens, dev), int(max(prompts)), int(max(prompts)), SCALE)
    torch.cuda.synchronize()
    ref = oracle_lib.paged_prefill(oracle_lib.rope(q, pos_q, f, 0)[1], qs, kr, vr, tables, lens,
                                   SCALE)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    print(f"prefill: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all() and err.max() <= 1e-2 and err.mean() <= 1e-3

    # Samples share the prompt's blocks.
    for i in range(len(prompts)):
        for j in range(1, SAMPLES):
            bm.fork(i * SAMPLES, i * SAMPLES + j)
            hist[i * SAMPLES + j] = hist[i * SAMPLES]

    copies = 0
    for step in range(5):
        live = sorted(hist)
        S = len(live)
        tables, lens, slots, pairs = bm.prepare_decode(live, WIDTH)
        copies += len(pairs)
        if len(pairs):
            tv.copy_blocks(kc, vc, _to_dev(pairs, dev))
            oracle_lib.copy_blocks(kr, vr, pairs)
        k_new, v_new, qn = _bf16(rng, (S, HKV, D)), _bf16(rng, (S, HKV, D)), _bf16(rng, (S, HQ, D))
        pos = (lens - 1).astype(np.int32)
        kd, qd = _to_dev(k_new, dev), _to_dev(qn, dev)
        tv.rope(kd, _to_dev(pos, dev), fd, 0)
        tv.rope(qd, _to_dev(pos, dev), fd, 0)
        mc = int(lens.max())
        ws = tv.new_workspace(S, HQ, D, mc, PART, dev)
        outd = torch.empty((S, HQ, D), dtype=torch.float32, device=dev)
        bt, cl = _to_dev(tables, dev), _to_dev(lens, dev)
        tv.paged_attention_decode_append(*ws, qd, kd, _to_dev(v_new, dev), _to_dev(slots, dev),
                                         kc, vc, bt, cl, mc, PART, SCALE)
        tv.paged_attention_reduce(outd, *ws, cl, mc, PART)
        torch.cuda.synchronize()
        # Oracle: the same step from its own rotated values.
        oracle_lib.cache_write(oracle_lib.rope(k_new, pos, f, 0)[1], v_new, kr, vr, slots)
        ref = oracle_lib.paged_attention(oracle_lib.rope(qn, pos, f, 0)[1], kr, vr, tables, lens,
                                         SCALE)
        err = np.abs(outd.cpu().numpy().astype(np.float64) - ref)
        print(f"decode step {step}: {S} sequences, {len(pairs)} block copies, "
              f"max_abs={err.max():.3e}", flush=True)
        assert np.isfinite(err).all() and err.max() <= 1e-3 and err.mean() <= 1e-4
        if step < 3:
            # Before any sample ends, rows 3i .. 3i+2 are prompt i's samples:
            # the shared-prefix pass over the same pools must give the fused
            # step's output bit for bit (prompt blocks never written since the
            # fork stay shared; partial blocks were copied on write).
            shared = np.array([(n // BS) * BS for n in prompts], np.int32)
            ws2 = tv.new_workspace(S, HQ, D, mc, PART, dev)
            out2 = torch.empty_like(outd)
            tv.paged_attention_decode_shared(*ws2, qd, kc, vc, bt, cl, _to_dev(shared, dev),
                                             SAMPLES, mc, PART, SCALE)
            tv.paged_attention_reduce(out2, *ws2, cl, mc, PART)
            torch.cuda.synchronize()
            assert torch.equal(out2.view(torch.int32), outd.view(torch.int32)), step
        else:
            # After a sample has ended the prompts' samples are no longer in
            # consecutive rows: give the groups as a member order (prompt 0,
            # prompt 2, then prompt 1's two remaining samples as a partial
            # last group), with the new tokens appended again by the shared
            # pass (the same bits into the same slots).
            by_prompt = {i: [r for r, seq in enumerate(live) if seq // SAMPLES == i]
                         for i in range(len(prompts))}
            groups = [0, 2, 1]
            order = np.array(sum((by_prompt[i] for i in groups), []), np.int32)
            assert [len(by_prompt[i]) for i in groups] == [SAMPLES, SAMPLES, SAMPLES - 1]
            shared = np.array([(prompts[i] // BS) * BS for i in groups], np.int32)
            ws2 = tv.new_workspace(S, HQ, D, mc, PART, dev)
            out2 = torch.empty_like(outd)
            tv.paged_attention_decode_shared_append(
                *ws2, qd, kd, _to_dev(v_new, dev), _to_dev(slots, dev), kc, vc, bt, cl,
                _to_dev(shared, dev), SAMPLES, mc, PART, SCALE, group_order=_to_dev(order, dev))
            tv.paged_attention_reduce(out2, *ws2, cl, mc, PART)
            torch.cuda.synchronize()
            assert torch.equal(out2.view(torch.int32), outd.view(torch.int32)), step
        for r, seq in enumerate(live):
            k, v = hist[seq]
            hist[seq] = (np.concatenate([k, k_new[r:r + 1]]), np.concatenate([v, v_new[r:r + 1]]))
        if step == 2:                                   # one sample of the second prompt ends
            bm.free_sequence(SAMPLES + 1)
            del hist[SAMPLES + 1]
    assert copies > 0, "no copy on write happened"
    # V pools agree bit for bit (V is never rotated); K agrees off the RoPE near-ties.
    vc_h = vc.cpu().numpy().view(np.uint16)
    for seq in hist:
        sl = bm.slots(seq, 0, bm.length(seq))
        blk, off = sl // BS, sl % BS
        assert np.array_equal(vc_h[blk, :, :, off], vr[blk, :, :, off]), seq
