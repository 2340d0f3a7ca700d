"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` (the real build, or a build of a
deliberately broken copy in the mutation test) and raises AssertionError when
the oracle disagrees with:
  * brute-force contiguous, unpaged attention on tiny inputs;
  * ``torch.nn.functional.scaled_dot_product_attention`` (a library routine)
    in float64 with grouped K/V heads;
  * closed forms: one-token context, constant V, zero query (mean of V),
    two-token logistic weights, one dominant key;
  * invariances: physical block permutation, a constant shift of all scores,
    thread count;
  * the pages' worked paging example (300 tokens -> 19 blocks) and the GQA
    grouping figure, stored under tests/golden/ with their citations;
  * a hand-derived literal cache layout (tests/golden/cache_layout_tiny.json)
    and a hand-derived literal block copy (tests/golden/block_copy_tiny.json);
  * for prefill: torch SDPA with its own causal mask on full prompts and with
    a bottom-right mask on chunks, chunking invariance, single rows equal to
    the decode oracle, position 0 equal to V_0, rows before the context,
    block permutation.

Run as a script (``python tests/oracle_pins.py LIB``) it executes every pin
against the oracle library LIB and prints one line per pin: the mutation test
uses that so that a crashing broken oracle counts as detected.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import oracle as O  # noqa: E402
from paged_kv_cache_tv_amd import workloads as W  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f64(bits):
    return W.bf16_bits_to_float32(bits).astype(np.float64)


def _run(orc, batch, num_threads=2):
    return O.decode_step(orc, batch, num_threads)


def _kv_of_head():
    return np.asarray(_golden("attention_shape.json")["gqa_figure"]["kv_head_of_query_head"])


def _contiguous_reference(batch):
    """softmax(q K^T * scale) V on the unpaged sequences, plain numpy float64."""
    kv_of = _kv_of_head() if batch.num_q_heads == 32 and batch.num_kv_heads == 8 else \
        np.repeat(np.arange(batch.num_kv_heads), batch.num_q_heads // batch.num_kv_heads)
    out = np.zeros((batch.num_seqs, batch.num_q_heads, batch.head_dim))
    for s in range(batch.num_seqs):
        n = int(batch.context_lens[s])
        if n == 0:
            continue
        k, v = batch.logical_kv(s)
        k, v = _f64(k), _f64(v)
        q = _f64(batch.q[s])
        for h in range(batch.num_q_heads):
            g = kv_of[h]
            sc = (k[:, g, :] @ q[h]) * batch.scale
            w = np.exp(sc - sc.max())
            out[s, h] = (w @ v[:, g, :]) / w.sum()
    return out


def _sdpa_reference(batch):
    import torch
    import torch.nn.functional as F
    out = np.zeros((batch.num_seqs, batch.num_q_heads, batch.head_dim))
    for s in range(batch.num_seqs):
        n = int(batch.context_lens[s])
        if n == 0:
            continue
        k, v = batch.logical_kv(s)
        qt = torch.from_numpy(_f64(batch.q[s]))[None, :, None, :]            # [1, Hq, 1, D]
        kt = torch.from_numpy(_f64(k)).permute(1, 0, 2)[None].contiguous()    # [1, Hkv, n, D]
        vt = torch.from_numpy(_f64(v)).permute(1, 0, 2)[None].contiguous()
        o = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)     # scale = 1/sqrt(D)
        out[s] = o[0, :, 0, :].numpy()
    return out


# --------------------------------------------------------------------------- pins


def pin_contiguous_bruteforce(orc):
    """Paged oracle == unpaged brute force on tiny ragged batches."""
    for seed, lens in ((11, [1, 17, 45, 64]), (12, [2, 16, 31, 33, 48, 5])):
        b = W.make_batch(lens, seed)
        out, _, _ = _run(orc, b)
        ref = _contiguous_reference(b)
        err = np.abs(out - ref).max()
        assert err <= 1e-12, f"brute force mismatch {err}"


def pin_torch_sdpa(orc):
    """Paged oracle == torch SDPA (float64, grouped K/V heads) on the unpaged data."""
    b = W.make_batch([3, 16, 33, 100], 13)
    out, _, _ = _run(orc, b)
    ref = _sdpa_reference(b)
    err = np.abs(out - ref).max()
    assert err <= 1e-12, f"SDPA mismatch {err}"


def pin_block_permutation(orc):
    """Moving physical blocks (and rewriting the tables) leaves the output bit-identical."""
    b = W.make_batch([40, 77, 16, 129], 14)
    out, kc, vc = _run(orc, b)
    perm = np.random.default_rng(99).permutation(b.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = perm[b.block_tables].astype(np.int32)
    out2 = orc.paged_attention(b.q, kc2, vc2, bt2, b.context_lens, b.scale, 2)
    assert np.array_equal(out, out2), "output changed under block permutation"


def pin_single_token(orc):
    """A one-token context returns exactly that token's V (per the GQA figure's head map)."""
    b = W.make_batch([1, 1, 1], 15)
    out, _, _ = _run(orc, b)
    kv_of = _kv_of_head()
    for s in range(3):
        _, v = b.logical_kv(s)
        expect = _f64(v[0])[kv_of]                       # [Hq, D]
        assert np.array_equal(out[s], expect), "n=1 must return V exactly"


def _with_values(batch, k_fn=None, v_fn=None, q=None):
    if k_fn is not None:
        batch.kv_k = k_fn(batch.kv_k)
    if v_fn is not None:
        batch.kv_v = v_fn(batch.kv_v)
    if q is not None:
        batch.q = q
    return batch


def pin_constant_v(orc):
    """V identically c gives c, whatever the scores."""
    c = np.float32(0.75)
    bits = W.round_to_bf16_bits(np.array([c]))[0]
    b = _with_values(W.make_batch([5, 40, 300], 16), v_fn=lambda v: np.full_like(v, bits))
    out, _, _ = _run(orc, b)
    assert np.abs(out - 0.75).max() <= 1e-12, "constant V not reproduced"


def pin_zero_query_mean(orc):
    """q = 0 makes every score 0: the output is the plain mean of V over exactly n tokens.
    Unused slots hold NaN, so reading one position too many shows as NaN."""
    lens = [1, 15, 16, 17, 31, 33]
    b = _with_values(W.make_batch(lens, 17), q=None)
    b.q = np.zeros_like(b.q)
    out, _, _ = _run(orc, b)
    kv_of = _kv_of_head()
    for s, n in enumerate(lens):
        _, v = b.logical_kv(s)
        mean = _f64(v).mean(axis=0)[kv_of]
        assert np.isfinite(out[s]).all(), "stray read of a poisoned slot"
        assert np.abs(out[s] - mean).max() <= 1e-12, f"mean of V over {n} tokens wrong"


def pin_gqa_figure(orc):
    """K/V head g filled with the constant (g+1)/2: query head h must return the
    constant of the K/V head the GQA figure assigns to it; equal queries inside a
    group give bit-equal outputs."""
    b = W.make_batch([23, 50], 18)
    consts = ((np.arange(8) + 1) * 0.5).astype(np.float32)
    cbits = W.round_to_bf16_bits(consts)

    def v_fn(v):
        v = v.copy()
        v[:] = cbits[None, :, None]
        return v
    b = _with_values(b, v_fn=v_fn)
    q = b.q.copy()
    for g in range(8):
        q[:, 4 * g + 1:4 * g + 4] = q[:, 4 * g:4 * g + 1]
    b.q = q
    out, _, _ = _run(orc, b)
    kv_of = _kv_of_head()
    for h in range(32):
        assert np.abs(out[:, h] - consts[kv_of[h]]).max() <= 1e-12, f"head {h} reads the wrong K/V head"
    b2 = W.make_batch([23, 50], 18)
    b2.q = q
    out2, _, _ = _run(orc, b2)
    for g in range(8):
        for j in range(1, 4):
            assert np.array_equal(out2[:, 4 * g], out2[:, 4 * g + j]), "equal queries in a group differ"


def pin_one_dominant_key(orc):
    """One key far more aligned with the query than the rest takes all the weight.
    Its score (about 0.125 * 256 * |u|^2, i.e. ~2000) exceeds every other by far
    more than exp() can span in double precision, so the softmax must also be
    taken relative to the true maximum, not to an arbitrary score."""
    b = W.make_batch([50], 19)
    q = b.q.copy()
    q[0, :] = q[0, 0:1]                                   # every head asks the same question
    b.q = q
    u = W.bf16_bits_to_float32(q[0, 0])
    j = 29
    k = b.kv_k.copy()
    k[b.token_rows[0][j], :, :] = W.round_to_bf16_bits(256.0 * u)[None, :]  # exact: power-of-2 scale
    b.kv_k = k
    out, _, _ = _run(orc, b)
    _, v = b.logical_kv(0)
    expect = _f64(v[j])[_kv_of_head()]
    assert np.abs(out[0] - expect).max() <= 1e-14, "dominant key must win"


def pin_two_token_logistic(orc):
    """Two tokens with scores s0, s1: weights are logistic(s0-s1) and logistic(s1-s0).
    q = 2 e_0, K_0 = e_0, K_1 = -3 e_0 give s0 = 0.125*2*1 = 0.25 and s1 = -0.75."""
    from scipy.special import expit
    b = W.make_batch([2], 20)
    q = np.zeros_like(b.q)
    q[..., 0] = W.round_to_bf16_bits(np.array([2.0], np.float32))[0]
    k = np.zeros_like(b.kv_k)
    rows = b.token_rows[0]
    k[rows[0], :, 0] = W.round_to_bf16_bits(np.array([1.0], np.float32))[0]
    k[rows[1], :, 0] = W.round_to_bf16_bits(np.array([-3.0], np.float32))[0]
    b.q, b.kv_k = q, k
    out, _, _ = _run(orc, b)
    _, v = b.logical_kv(0)
    v = _f64(v)
    w0, w1 = expit(1.0), expit(-1.0)
    expect = (w0 * v[0] + w1 * v[1])[_kv_of_head()]
    assert np.abs(out[0] - expect).max() <= 1e-12, "two-token weights wrong (scale or sign)"


def pin_score_shift(orc):
    """Adding the same amount (here 1024) to every score changes nothing: the
    softmax must be computed relative to the largest score."""
    b = W.make_batch([9, 70], 21)
    one = W.round_to_bf16_bits(np.array([1.0], np.float32))[0]
    k = b.kv_k.copy()
    k[:, :, 0] = one
    b.kv_k = k
    q = b.q.copy()
    q[..., 0] = 0
    b.q = q
    base, _, _ = _run(orc, b)
    q2 = q.copy()
    q2[..., 0] = W.round_to_bf16_bits(np.array([8192.0], np.float32))[0]   # +0.125*8192 = +1024
    b.q = q2
    shifted, _, _ = _run(orc, b)
    assert np.isfinite(shifted).all(), "overflow: scores not taken relative to their maximum"
    assert np.abs(shifted - base).max() <= 1e-12, "shift of all scores changed the output"


def pin_paging_example(orc):
    """The pages' worked example: 300 tokens occupy 19 blocks of 16 with 4 slots
    free in the last one.  The oracle must read all 300 and nothing else."""
    g = _golden("paging_examples.json")
    bs, n = g["block_size"], g["on_demand"]["tokens"]
    assert W.blocks_needed(n, bs) == g["on_demand"]["blocks"]
    assert W.paged_waste(n, bs) == g["on_demand"]["free_slots_in_last_block"]
    assert W.contiguous_waste(g["contiguous"]["max_length"], n) == g["contiguous"]["wasted_slots"]
    b = W.make_batch([n], 22, table_width=g["on_demand"]["blocks"] + 5)
    out, kc, vc = _run(orc, b)
    assert np.isfinite(out).all(), "a poisoned slot or table entry was read"
    assert np.abs(out - _contiguous_reference(b)).max() <= 1e-12
    # The 300th token (offset 11 of the 19th block) is read ...
    last_blk = b.block_tables[0, g["on_demand"]["blocks"] - 1]
    kc2 = kc.copy()
    kc2[last_blk, :, :, (n - 1) % bs, :] = W.round_to_bf16_bits(np.array([4.0], np.float32))[0]
    out2 = orc.paged_attention(b.q, kc2, vc, b.block_tables, b.context_lens, b.scale, 2)
    assert not np.array_equal(out, out2), "the last token was not read"
    # ... and table entries past the 19th are not.
    bt = b.block_tables.copy()
    bt[0, g["on_demand"]["blocks"]:] = b.block_tables[0, 0]
    out3 = orc.paged_attention(b.q, kc, vc, bt, b.context_lens, b.scale, 2)
    assert np.array_equal(out, out3), "an unused table entry was read"


def pin_cache_layout_literal(orc):
    """Writes land exactly where the hand-derived literal pools say; padding and
    out-of-pool slots are skipped."""
    g = _golden("cache_layout_tiny.json")
    nb, hkv, bs, d = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    kc, vc = O.Oracle.new_pools(nb, hkv, d, bs, fill=0)
    k = np.array([t["k"] for t in g["tokens"]], np.uint16)
    v = np.array([t["v"] for t in g["tokens"]], np.uint16)
    slots = np.array([t["slot"] for t in g["tokens"]], np.int64)
    written = orc.cache_write(k, v, kc, vc, slots)
    assert written == g["written"]
    assert kc.tolist() == g["expected_k_pool"], "K pool layout"
    assert vc.tolist() == g["expected_v_pool"], "V pool layout"


def pin_cache_write_untouched(orc):
    """Only the named slots change; every other element keeps its (NaN) bits;
    a repeated slot is refused."""
    b = W.make_batch([20, 3, 47], 23)
    kc, vc = O.Oracle.new_pools(b.num_blocks, 8, 64, 16)
    k, v, slots = b.fill_inputs()
    slots = slots.copy()
    slots[0] = -1                                         # padding
    slots[1] = b.num_blocks * 16                          # past the pool
    written = orc.cache_write(k, v, kc, vc, slots)
    assert written == len(slots) - 2
    changed = (kc != W.BF16_NAN).sum() + (vc != W.BF16_NAN).sum()
    expect_changed = ((k[2:] != W.BF16_NAN).sum() + (v[2:] != W.BF16_NAN).sum())
    assert changed == expect_changed, "elements outside the written slots changed"
    dup = np.array([5, 9, 5], np.int64)
    kc2, vc2 = O.Oracle.new_pools(b.num_blocks, 8, 64, 16)
    try:
        orc.cache_write(k[:3], v[:3], kc2, vc2, dup)
    except ValueError:
        pass
    else:
        raise AssertionError("duplicate slot accepted")
    assert (kc2 == W.BF16_NAN).all(), "refused write touched the pool"


def pin_empty(orc):
    """A sequence with no context yields zeros; an empty batch yields nothing."""
    b = W.make_batch([0, 5, 0], 24)
    out, _, _ = _run(orc, b)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert np.abs(out[1] - _contiguous_reference(b)[1]).max() <= 1e-12
    kc, vc = O.Oracle.new_pools(4, 8, 64, 16)
    e = orc.paged_attention(np.zeros((0, 32, 64), np.uint16), kc, vc,
                            np.zeros((0, 1), np.int32), np.zeros(0, np.int32), 0.125, 1)
    assert e.shape == (0, 32, 64)


def pin_thread_invariance(orc):
    """Results do not depend on the number of threads."""
    b = W.make_batch([33, 250, 64, 17, 100], 25)
    kc, vc = O.build_pools(orc, b)
    a = orc.paged_attention(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, 1)
    c = orc.paged_attention(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, 4)
    assert np.array_equal(a, c)


def pin_block_copy_literal(orc):
    """Copy-on-write copies land exactly where the hand-derived literal pools say;
    pairs naming one block twice or a block past the pool are skipped; a pair
    list whose destination repeats is refused without touching the pools."""
    g = _golden("block_copy_tiny.json")
    nb, hkv, bs, d = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    kc = np.array(g["k_pool_before"], np.uint16).reshape(nb, hkv, d // 8, bs, 8)
    vc = np.array(g["v_pool_before"], np.uint16).reshape(nb, hkv, d, bs)
    copied = orc.copy_blocks(kc, vc, g["pairs"])
    assert copied == g["copied"]
    assert kc.reshape(nb, -1).tolist() == g["expected_k_pool"], "K pool after the copy"
    assert vc.reshape(nb, -1).tolist() == g["expected_v_pool"], "V pool after the copy"
    kc2, vc2 = kc.copy(), vc.copy()
    for bad in ([[0, 1], [2, 1]], [[0, 1], [1, 2]]):       # repeated destination; dst also a source
        try:
            orc.copy_blocks(kc2, vc2, bad)
        except ValueError:
            pass
        else:
            raise AssertionError(f"conflicting pairs {bad} accepted")
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc), "refused copy touched the pools"


# ------------------------------------------------------------------ prefill pins


def _prefill(orc, pb, num_threads=2):
    """Pools holding every position of the prefill batch (prior and chunk, written
    by the oracle's own cache write) and the oracle's prefill output."""
    kc, vc = O.Oracle.new_pools(pb.base.num_blocks, pb.base.num_kv_heads, pb.base.head_dim,
                                pb.base.block_size)
    for k, v, sl in (pb.prior_inputs(), pb.chunk_inputs()):
        orc.cache_write(k, v, kc, vc, sl)
    out = orc.paged_prefill(pb.q, pb.query_start, kc, vc, pb.base.block_tables,
                            pb.context_lens, pb.base.scale, num_threads)
    return out, kc, vc


def _sdpa_prefill_reference(pb):
    """torch SDPA (float64, grouped K/V heads) per sequence on the unpaged data,
    with a boolean mask: chunk row i (position n - m + i) may see key t iff
    t <= n - m + i."""
    import torch
    import torch.nn.functional as F
    b = pb.base
    out = np.zeros((pb.num_rows, b.num_q_heads, b.head_dim))
    for s in range(pb.num_seqs):
        n, m, r0 = int(b.context_lens[s]), int(pb.query_lens[s]), int(pb.query_start[s])
        if m == 0:
            continue
        k, v = b.logical_kv(s)
        qt = torch.from_numpy(_f64(pb.q[r0:r0 + m])).permute(1, 0, 2)[None].contiguous()
        kt = torch.from_numpy(_f64(k)).permute(1, 0, 2)[None].contiguous()
        vt = torch.from_numpy(_f64(v)).permute(1, 0, 2)[None].contiguous()
        mask = torch.arange(n)[None, :] <= (n - m + torch.arange(m))[:, None]
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, enable_gqa=True)
        out[r0:r0 + m] = o[0].permute(1, 0, 2).numpy()
    return out


def pin_prefill_sdpa_full_prompts(orc):
    """Full prefill (chunk = whole prompt) == torch SDPA with is_causal=True, the
    library's own causal mask, which is the right one when queries and keys
    cover the same positions."""
    import torch
    import torch.nn.functional as F
    pb = W.make_prefill_batch([0, 0, 0, 0], [1, 16, 37, 90], 31)
    out, _, _ = _prefill(orc, pb)
    b = pb.base
    for s in range(pb.num_seqs):
        m, r0 = int(pb.query_lens[s]), int(pb.query_start[s])
        k, v = b.logical_kv(s)
        qt = torch.from_numpy(_f64(pb.q[r0:r0 + m])).permute(1, 0, 2)[None].contiguous()
        kt = torch.from_numpy(_f64(k)).permute(1, 0, 2)[None].contiguous()
        vt = torch.from_numpy(_f64(v)).permute(1, 0, 2)[None].contiguous()
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
        err = np.abs(out[r0:r0 + m] - o[0].permute(1, 0, 2).numpy()).max()
        assert err <= 1e-12, f"sequence {s}: SDPA causal mismatch {err}"


def pin_prefill_sdpa_chunks(orc):
    """Chunks on top of cached positions == torch SDPA with the bottom-right mask."""
    pb = W.make_prefill_batch([0, 5, 40, 100, 17], [3, 20, 33, 1, 64], 32)
    out, _, _ = _prefill(orc, pb)
    err = np.abs(out - _sdpa_prefill_reference(pb)).max()
    assert err <= 1e-12, f"SDPA chunk mismatch {err}"


def pin_prefill_chunking_invariance(orc):
    """A prompt run as one chunk and as several consecutive chunks gives the same
    rows bit for bit (each chunk on the pools that hold the whole prompt)."""
    pb = W.make_prefill_batch([0, 0], [70, 129], 33)
    full, kc, vc = _prefill(orc, pb)
    b = pb.base
    for s, chunks in ((0, [30, 40]), (1, [16, 100, 13])):
        done = 0
        for m in chunks:
            r = int(pb.query_start[s]) + done
            out = orc.paged_prefill(pb.q[r:r + m], np.array([0, m], np.int32), kc, vc,
                                    b.block_tables[s:s + 1], np.array([done + m], np.int32),
                                    b.scale, 2)
            assert np.array_equal(out, full[r:r + m]), f"sequence {s}, chunk at {done}"
            done += m


def pin_prefill_single_rows_are_decode(orc):
    """One query row per sequence is a decode step: equal to the decode oracle,
    which has pins of its own."""
    pb = W.make_prefill_batch([0, 15, 64, 200], [1, 1, 1, 1], 34)
    out, kc, vc = _prefill(orc, pb)
    dec = orc.paged_attention(pb.q, kc, vc, pb.base.block_tables, pb.context_lens,
                              pb.base.scale, 2)
    assert np.array_equal(out, dec)


def pin_prefill_first_position(orc):
    """The row at position 0 sees one key, so its output is V_0 of its K/V head."""
    pb = W.make_prefill_batch([0, 0], [5, 21], 35)
    out, _, _ = _prefill(orc, pb)
    b = pb.base
    kv_of = _kv_of_head()
    for s in range(2):
        _, v = b.logical_kv(s)
        row = out[int(pb.query_start[s])]
        for h in range(b.num_q_heads):
            assert np.array_equal(row[h], _f64(v[0, kv_of[h]])), f"sequence {s} head {h}"


def pin_prefill_rows_before_context(orc):
    """A chunk longer than the context: rows at negative positions are zero and
    the rest equal the rows of the chunk that fits."""
    pb = W.make_prefill_batch([0], [10], 36)
    full, kc, vc = _prefill(orc, pb)
    b = pb.base
    q = np.concatenate([pb.q[:4], pb.q])                        # 14 rows, context 10
    out = orc.paged_prefill(q, np.array([0, 14], np.int32), kc, vc, b.block_tables,
                            np.array([10], np.int32), b.scale, 2)
    assert not out[:4].any(), "rows before the context are not zero"
    assert np.array_equal(out[4:], full)


def pin_prefill_block_permutation(orc):
    """Moving physical blocks (and rewriting the tables) leaves prefill bit-identical."""
    pb = W.make_prefill_batch([3, 40], [30, 50], 37)
    out, kc, vc = _prefill(orc, pb)
    b = pb.base
    perm = np.random.default_rng(98).permutation(b.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    out2 = orc.paged_prefill(pb.q, pb.query_start, kc2, vc2, perm[b.block_tables].astype(np.int32),
                             pb.context_lens, b.scale, 2)
    assert np.array_equal(out, out2)


# --------------------------------------------------------------------- RoPE pins


def _inv_freq(d, base=500000.0):
    return (base ** (-np.arange(0, d, 2, dtype=np.float64) / d)).astype(np.float32)


def _pair_dims(style, k, d):
    return (2 * k, 2 * k + 1) if style == 0 else (k, k + d // 2)


def pin_rope_pair_closed_form(orc):
    """A unit vector in the first (second) dim of pair k turns into
    (cos, sin) ((-sin, cos)) of position * inv_freq[k], numpy's cos and sin."""
    d = 16
    f = _inv_freq(d, 10000.0)
    pos = np.array([0, 1, 7, 1000, 131071, -5], np.int32)
    for style in (0, 1):
        for k in (0, 3, 7):
            ia, ib = _pair_dims(style, k, d)
            x = np.zeros((len(pos), 2, d), np.uint16)
            x[:, 0, ia] = 0x3F80                               # 1.0
            x[:, 1, ib] = 0x3F80
            out, _ = orc.rope(x, pos, f, style)
            ang = pos.astype(np.float64) * np.float64(f[k])
            c, s_ = np.cos(ang), np.sin(ang)
            for h, (ea, eb) in enumerate(((c, s_), (-s_, c))):
                assert np.abs(out[:, h, ia] - ea).max() <= 1e-15, (style, k, h)
                assert np.abs(out[:, h, ib] - eb).max() <= 1e-15, (style, k, h)
            rest = np.ones(d, bool)
            rest[[ia, ib]] = False
            assert not out[:, :, rest].any(), "other dims must stay zero"


def pin_rope_complex_form(orc):
    """Style 0 is multiplication of a + i b by e^{i p f_k} (numpy complex)."""
    rng = np.random.default_rng(41)
    d = 64
    x = W.round_to_bf16_bits(rng.standard_normal((9, 4, d)).astype(np.float32))
    pos = rng.integers(0, 140000, 9).astype(np.int32)
    f = _inv_freq(d)
    out, _ = orc.rope(x, pos, f, 0)
    xf = _f64(x)
    z = xf[..., 0::2] + 1j * xf[..., 1::2]
    zr = z * np.exp(1j * pos[:, None, None] * f.astype(np.float64)[None, None, :])
    assert np.abs(out[..., 0::2] - zr.real).max() <= 1e-12
    assert np.abs(out[..., 1::2] - zr.imag).max() <= 1e-12


def pin_rope_half_split_is_permuted_interleaved(orc):
    """Style 1 equals style 0 applied after moving dims (k, k + D/2) to (2k, 2k+1)."""
    rng = np.random.default_rng(42)
    d = 64
    x = W.round_to_bf16_bits(rng.standard_normal((5, 3, d)).astype(np.float32))
    pos = rng.integers(0, 5000, 5).astype(np.int32)
    f = _inv_freq(d)
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2                    # interleaved dim j <- half-split perm[j]
    o1, b1 = orc.rope(x, pos, f, 1)
    o0, b0 = orc.rope(x[..., perm], pos, f, 0)
    assert np.array_equal(o1[..., perm], o0) and np.array_equal(b1[..., perm], b0)


def pin_rope_position_zero(orc):
    """Position 0 is the identity, bit for bit."""
    rng = np.random.default_rng(43)
    x = W.round_to_bf16_bits(rng.standard_normal((4, 8, 64)).astype(np.float32))
    for style in (0, 1):
        out, bits = orc.rope(x, np.zeros(4, np.int32), _inv_freq(64), style)
        assert np.array_equal(bits, x) and np.array_equal(out, _f64(x))


def pin_rope_relative_identity(orc):
    """The pages' identity (R_i q)^T (R_j k) = q^T R_{j-i} k, per head and pair
    of positions, and the norm of every pair is kept."""
    rng = np.random.default_rng(44)
    d = 64
    f = _inv_freq(d, 10000.0)
    q = W.round_to_bf16_bits(rng.standard_normal((1, 2, d)).astype(np.float32))
    k = W.round_to_bf16_bits(rng.standard_normal((1, 2, d)).astype(np.float32))
    for style in (0, 1):
        for i, j in ((0, 5), (3, 3), (100, 37), (70000, 131000), (9, -4)):
            qi, _ = orc.rope(q, np.array([i], np.int32), f, style)
            kj, _ = orc.rope(k, np.array([j], np.int32), f, style)
            kd, _ = orc.rope(k, np.array([j - i], np.int32), f, style)
            lhs = (qi[0] * kj[0]).sum(-1)
            rhs = (_f64(q[0]) * kd[0]).sum(-1)
            assert np.abs(lhs - rhs).max() <= 1e-9 * (1 + np.abs(rhs).max()), (style, i, j)
        out, _ = orc.rope(k, np.array([12345], np.int32), f, style)
        a, b = (slice(0, None, 2), slice(1, None, 2)) if style == 0 else \
            (slice(0, d // 2), slice(d // 2, None))
        n0 = _f64(k)[..., a] ** 2 + _f64(k)[..., b] ** 2
        n1 = out[..., a] ** 2 + out[..., b] ** 2
        assert np.abs(n0 - n1).max() <= 1e-12


def pin_bf16_round(orc):
    """Rounding to bf16: the nearest of the two bf16 neighbours, ties to even,
    found by brute force on the float32 bit patterns."""
    rng = np.random.default_rng(45)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-3, 4, 4000),
                        [1.0, -2.5, 1.00390625, 1.01171875, -1.01171875, 3.0e-5]])
    # exact ties: midpoints of adjacent bf16 values
    lo = W.round_to_bf16_bits(rng.standard_normal(200).astype(np.float32))
    lof = W.bf16_bits_to_float32(lo).astype(np.float64)
    hif = W.bf16_bits_to_float32((lo.astype(np.uint32) + 1).astype(np.uint16)).astype(np.float64)
    v = np.concatenate([v, (lof + hif) / 2])
    got = orc.bf16_round(v)
    for x, g in zip(v, got):
        f32 = np.float32(x)
        b = int(np.array([f32]).view(np.uint32)[0]) >> 16
        cands = [(b + dlt) & 0xFFFF for dlt in (-1, 0, 1, 2)]
        vals = [float(W.bf16_bits_to_float32(np.array([c], np.uint16))[0]) for c in cands]
        errs = [abs(val - x) for val in vals]
        best = min(errs)
        ties = [c for c, e in zip(cands, errs) if e == best]
        want = ties[0] if len(ties) == 1 else [c for c in ties if c % 2 == 0][0]
        assert int(g) == want, (x, hex(int(g)), hex(want))


ALL_PINS = [
    pin_contiguous_bruteforce, pin_torch_sdpa, pin_block_permutation, pin_single_token,
    pin_constant_v, pin_zero_query_mean, pin_gqa_figure, pin_one_dominant_key,
    pin_two_token_logistic, pin_score_shift, pin_paging_example, pin_cache_layout_literal,
    pin_cache_write_untouched, pin_empty, pin_thread_invariance, pin_block_copy_literal,
    pin_prefill_sdpa_full_prompts, pin_prefill_sdpa_chunks, pin_prefill_chunking_invariance,
    pin_prefill_single_rows_are_decode, pin_prefill_first_position,
    pin_prefill_rows_before_context, pin_prefill_block_permutation,
    pin_rope_pair_closed_form, pin_rope_complex_form, pin_rope_half_split_is_permuted_interleaved,
    pin_rope_position_zero, pin_rope_relative_identity, pin_bf16_round,
]


def main(argv):
    orc = O.Oracle(argv[1])
    failed = 0
    for pin in ALL_PINS:
        try:
            pin(orc)
            print(f"PASS {pin.__name__}", flush=True)
        except (AssertionError, ValueError) as e:
            failed += 1
            print(f"FAIL {pin.__name__}: {e}", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
