"""GPU path (libtv through its C interface) against the CPU oracle.

Bars:
  * cache writes: the whole K and V pools bit-exact against the oracle's pools;
  * attention output (fp32 accumulation from bf16 inputs): max-abs <= 1e-2 and
    mean-abs <= 1e-3 (the contract), plus a tighter internal bar, max-abs <=
    1e-4, that a dropped or extra token would break (the GPU keeps P to ~16
    mantissa bits and accumulates in fp32; expected error ~1e-6).
"""

import numpy as np
import pytest

import oracle as O
from paged_kv_cache_tv_amd import workloads as W

pytestmark = pytest.mark.gpu

CONTRACT_MAX, CONTRACT_MEAN, INTERNAL_MAX = 1e-2, 1e-3, 1e-4


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_cache_tv_amd as tv
    tv.lib()                          # fails loudly if libtv.so is missing
    return torch.device("cuda:0")


def _gpu_step(batch, dev, partition_size=None, max_context_len=None, fused=False):
    """One step through the C interface: three launches, or with ``fused`` the
    write folded into the partition pass (tv_paged_attention_decode_append)."""
    import torch
    from paged_kv_cache_tv_amd.step import DeviceBatch
    db = DeviceBatch(batch, dev, partition_size=partition_size, max_context_len=max_context_len)
    db.fill()
    out = (db.fused_step() if fused else db.step()).clone()
    torch.cuda.synchronize()
    return out.cpu().numpy(), db


def _errors(got, ref):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def _assert_close(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = _errors(got, ref)
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= CONTRACT_MAX and mean <= CONTRACT_MEAN, f"{what}: contract broken"
    assert mx <= INTERNAL_MAX, f"{what}: internal bar broken ({mx:.3e})"


_oracle_cache = {}


def _oracle_step(orc, key, batch):
    if key not in _oracle_cache:
        _oracle_cache.clear()
        _oracle_cache[key] = O.decode_step(orc, batch)
    return _oracle_cache[key]


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_workload_parity(dev, oracle_lib, index):
    """Full-size workloads: bit-exact pools after the step's writes, output within the bars."""
    print(f"workload {index}: {W.WORKLOADS[index]}", flush=True)
    batch = W.make_workload(index)
    ref, kc_ref, vc_ref = _oracle_step(oracle_lib, ("workload", index), batch)
    got, db = _gpu_step(batch, dev)
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref), "K pool differs from the oracle's"
    assert np.array_equal(vc, vc_ref), "V pool differs from the oracle's"
    del kc, vc, kc_ref, vc_ref
    _assert_close(got, ref, f"workload {index}")


RAGGED = [1, 15, 16, 17, 200, 511, 512, 513, 1024, 1500, 3001, 4096]


@pytest.mark.parametrize("partition_size", [16, 64, 512, 4096, 8192])
def test_partition_invariance(dev, oracle_lib, partition_size):
    """Same answer for any partition size (one partition when >= the longest context)."""
    batch = W.make_batch(RAGGED, 31)
    ref, _, _ = _oracle_step(oracle_lib, ("ragged", 31), batch)
    got, _ = _gpu_step(batch, dev, partition_size=partition_size)
    _assert_close(got, ref, f"partition {partition_size}")
    base, _ = _gpu_step(batch, dev, partition_size=512)
    assert np.abs(got - base).max() <= 1e-5


# ---------------------------------------------------------------------------
# tv_paged_attention_decode_step: the whole step in one call.  With one
# partition the pass divides by the sum itself (one launch); the output must
# equal the two-launch step bit for bit either way.
# ---------------------------------------------------------------------------

def _call_step(db):
    import torch
    db.out.fill_(float("nan"))                    # every row must be written by the call
    got = db.call_step().clone()
    torch.cuda.synchronize()
    return got.cpu().numpy()


def _forms_bar(batch):
    """How far two correct orders of the same step may differ.  Each form
    folds P into V as bf16 hi + lo parts, at least 16 significant bits
    (relative error <= 2^-17 per weight), against an exact fp32 sum, so each
    output is within 2^-17 * max|V| of the exactly weighted mean, and two
    forms that weight against different maxima within twice that; 1e-6
    covers their different fp32 summation orders."""
    v = W.bf16_bits_to_float32(batch.kv_v)
    return 2.0 ** -16 * float(np.abs(v[np.isfinite(v)]).max()) + 1e-6


# The form tv_paged_attention_decode_step takes per workload on MI355X: the
# whole-sequence launch (2 to 8 partitions, every (sequence, K/V head)
# workgroup resident at once) for 8 x U[128, 1024] and 64 x U[512, 4096]; one
# partition for workload 1; two launches for workloads 4 (2048 (sequence, head)
# pairs) and 5 (256 partitions).
_STEP_FORM = {1: 1, 2: 2, 3: 2, 4: 3, 5: 3}


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_decode_step_call_workloads(dev, oracle_lib, index):
    """Full workloads through tv_paged_attention_decode_step: pools bit-exact
    against the oracle's cache write, output within the bars and run-to-run
    identical.  Where the call takes the one-partition launch or the two
    launches, the output is the two-launch step's bit for bit; in the
    whole-sequence form each context is split into 8 equal ranges instead of
    the workspace's 512-token partitions (none longer than a partition), so
    the two agree to rounding (_forms_bar)."""
    batch = W.make_workload(index)
    ref, kc_ref, vc_ref = _oracle_step(oracle_lib, ("workload", index), batch)
    two, db = _gpu_step(batch, dev, fused=True)
    import paged_kv_cache_tv_amd as tv
    form = tv.decode_step_form(batch.num_seqs, batch.num_q_heads, batch.num_kv_heads,
                               batch.head_dim, batch.block_size, db.max_context_len,
                               db.partition_size)
    assert form == _STEP_FORM[index], f"workload {index}: step form {form}"
    got = _call_step(db)
    assert np.array_equal(got, _call_step(db)), f"workload {index}: two calls differ"
    if form == 2:                                 # one launch: other ranges
        assert np.abs(got - two).max() <= _forms_bar(batch), \
            f"workload {index}: one call far from two launches"
    else:
        assert np.array_equal(got, two), f"workload {index}: one call differs from two launches"
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    _assert_close(got, ref, f"workload {index}, one call")


_WHOLE_SEQUENCE_CASES = [
    # (seed, lengths or (count, low, high), query heads, K/V heads, partition, host bound)
    (80, [0, 1, 2, 15, 16, 17, 511, 512, 513, 1023, 1024, 1025, 4095, 4096], 32, 8, 512, None),
    (81, (64, 513, 4096), 32, 8, 512, 4096),         # loose host bound: 8 partitions
    (82, (200, 1, 600), 16, 2, 128, 1000),           # 400 (sequence, head) pairs, 8 partitions
    (83, (256, 0, 300), 8, 1, 64, 500),              # 256 sequences, one K/V head
    (84, (9, 1, 2048), 16, 1, 512, None),            # the largest group (16 query heads)
    (85, (40, 1, 1000), 8, 8, 256, None),            # one query head per K/V head
    (86, (3, 3000, 4000), 32, 8, 1024, None),        # 4 partitions of 1024
    (87, (63, 0, 2000), 32, 8, 512, 2048),           # an odd count of sequences
    (88, [0] * 20 + [4096] * 20 + [1] * 20, 32, 8, 512, None),   # empty, full and 1-token
]


@pytest.mark.parametrize("case", _WHOLE_SEQUENCE_CASES, ids=[f"seed{c[0]}" for c in _WHOLE_SEQUENCE_CASES])
def test_decode_step_whole_sequence_form(dev, oracle_lib, case):
    """The one-launch whole-sequence form across its range: empty and
    one-token contexts, lengths at tile and partition edges, group sizes 1 to
    16, partition sizes 64 to 1024, up to 256 sequences and 512 (sequence,
    head) workgroups: pools bit-exact against the oracle's, output within the
    bars, run-to-run identical, and within rounding of the two-launch step."""
    seed, lens, hq, hkv, part, bound = case
    if isinstance(lens, tuple):
        n_seq, lo, hi = lens
        lens = np.random.default_rng(seed).integers(lo, hi, size=n_seq, endpoint=True)
    lens = np.asarray(lens)
    mc = int(lens.max()) if bound is None else bound
    assert 2 <= -(-mc // part) <= 8
    batch = W.make_batch(lens, seed, num_q_heads=hq, num_kv_heads=hkv, table_width=mc // 16 + 1)
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, batch)
    two, db = _gpu_step(batch, dev, partition_size=part, max_context_len=mc, fused=True)
    import paged_kv_cache_tv_amd as tv
    assert tv.decode_step_form(len(lens), hq, hkv, 64, 16, mc, part) == 2
    got = _call_step(db)
    assert np.array_equal(got, _call_step(db)), "two calls differ"
    assert np.abs(got - two).max() <= _forms_bar(batch), "one call far from the two-launch step"
    assert not got[lens == 0].any(), "empty contexts must give zero rows"
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    _assert_close(got, ref, f"whole-sequence form, {len(lens)} sequences, {hq}/{hkv} heads, "
                            f"partition {part}, host bound {mc}")


_ONE_PARTITION = [
    # (seed, sequences, longest context, partition, host bound, query heads, K/V heads)
    (70, 1, 37, 512, 37, 32, 8),
    (71, 7, 512, 512, 512, 32, 8),      # contexts up to the whole partition
    (72, 64, 300, 512, 512, 32, 8),     # host bound above every context
    (73, 300, 64, 64, 64, 32, 8),       # small partitions, a large grid
    (74, 40, 500, 512, 500, 16, 2),     # 8 query heads per K/V head
    (75, 33, 200, 256, 256, 8, 8),      # 1 query head per K/V head
    (76, 20, 400, 512, 400, 32, 2),     # 16 query heads per K/V head (the largest group)
]


@pytest.mark.parametrize("case", _ONE_PARTITION, ids=[f"seed{c[0]}" for c in _ONE_PARTITION])
def test_decode_step_one_partition(dev, oracle_lib, case):
    """Host bounds that fit one partition, so the call is one launch whose
    pass writes acc / l: output within the bars against the oracle and bitwise
    the two-launch step's, including empty contexts (zero rows), one-token
    contexts, 1 to 16 query heads per K/V head and both launch forms (4
    wavefronts or 1 per partition)."""
    seed, S, maxlen, part, mc, hq, hkv = case
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, maxlen + 1, size=S)
    lens[0] = maxlen
    if S > 2:
        lens[1], lens[2] = 0, 1
    batch = W.make_batch(lens, seed, num_q_heads=hq, num_kv_heads=hkv, table_width=-(-mc // 16))
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, batch)
    two, db = _gpu_step(batch, dev, partition_size=part, max_context_len=mc, fused=True)
    got = _call_step(db)
    assert np.array_equal(got, two), f"seed {seed}: one launch differs from two"
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    _assert_close(got, ref, f"seed {seed}: {S} x <= {maxlen} tokens, host bound {mc}, "
                            f"partition {part}, {hq}/{hkv} heads")
    if S > 2:
        assert not got[1].any(), "an empty context must give a zero row"


_MERGE_FORMS = [
    # (sequences, partition size, workspace partitions): 32 query heads each
    (8, 256, 9),      # 256 rows, 9 partitions: split form
    (8, 32, 100),     # split form
    (8, 16, 256),     # split form, its largest partition count
    (9, 16, 256),     # 288 rows: wide form
    (8, 16, 257),     # 257 partitions: wide form
]


@pytest.mark.parametrize("case", _MERGE_FORMS, ids=[f"s{c[0]}-p{c[2]}" for c in _MERGE_FORMS])
def test_merge_forms(dev, oracle_lib, case):
    """The merge past eight workspace partitions takes one of two forms --
    each row split over four workgroups (at most 256 rows, at most 256
    partitions) or one workgroup per row -- on both sides of each limit the
    output meets the bars against the oracle, with contexts that end in
    every partition position (the workspace's later partitions unused)."""
    S, part, parts = case
    mc = part * parts
    rng = np.random.default_rng(97 + 7 * S + parts)
    lens = rng.integers(1, mc + 1, size=S)
    lens[1] = mc
    lens[2] = 1
    batch = W.make_batch(lens, 97 + parts, table_width=-(-mc // 16))
    ref, _, _ = O.decode_step(oracle_lib, batch)
    got, _ = _gpu_step(batch, dev, partition_size=part, max_context_len=mc)
    _assert_close(got, ref, f"{S} sequences, {parts} partitions of {part}")


def test_block_permutation_and_determinism(dev, oracle_lib):
    """Moving physical blocks leaves the GPU result bit-identical; so does re-running."""
    batch = W.make_batch([70, 513, 1111, 16], 32)
    a, _ = _gpu_step(batch, dev)
    b, _ = _gpu_step(batch, dev)
    assert np.array_equal(a, b), "run-to-run difference"
    perm = np.random.default_rng(5).permutation(batch.num_blocks).astype(np.int32)
    batch.block_tables = perm[batch.block_tables]
    batch.fill_slots = perm[batch.fill_slots // 16].astype(np.int64) * 16 + batch.fill_slots % 16
    ok = batch.new_slots >= 0
    batch.new_slots[ok] = perm[batch.new_slots[ok] // 16].astype(np.int64) * 16 + batch.new_slots[ok] % 16
    batch.poison_block = int(perm[batch.poison_block])
    c, _ = _gpu_step(batch, dev)
    assert np.array_equal(a, c), "block permutation changed the GPU result"


def test_edge_lengths(dev, oracle_lib):
    """Empty, single-token, block-boundary and partition-boundary contexts."""
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1023, 1024, 1025, 0]
    batch = W.make_batch(lens, 33)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    got, _ = _gpu_step(batch, dev)
    assert (got[0] == 0).all() and (got[-1] == 0).all(), "empty context must give zeros"
    _assert_close(got, ref, "edge lengths")
    one = [i for i, n in enumerate(lens) if n == 1][0]
    _, v = batch.logical_kv(one)
    expect = W.bf16_bits_to_float32(v[0])[np.repeat(np.arange(8), 4)]
    assert np.array_equal(got[one], expect), "a one-token context must return that V exactly"


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (12, 4), (32, 4), (32, 2), (4, 1), (64, 4)])
def test_group_sizes(dev, oracle_lib, hq, hkv):
    """Query heads per K/V head from 1 to 16."""
    batch = W.make_batch([37, 300, 1000], 34, num_q_heads=hq, num_kv_heads=hkv)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    got, _ = _gpu_step(batch, dev)
    _assert_close(got, ref, f"Hq={hq} Hkv={hkv}")


def test_zero_query_is_mean_of_v(dev, oracle_lib):
    """q = 0: every weight equal, output = mean of exactly n V rows (NaN poison beyond)."""
    lens = [1, 15, 17, 530, 1029]
    batch = W.make_batch(lens, 35)
    batch.q = np.zeros_like(batch.q)
    got, _ = _gpu_step(batch, dev)
    for s, n in enumerate(lens):
        _, v = batch.logical_kv(s)
        mean = W.bf16_bits_to_float32(v).astype(np.float64).mean(axis=0)[np.repeat(np.arange(8), 4)]
        assert np.isfinite(got[s]).all()
        assert np.abs(got[s] - mean).max() <= 2e-6, f"mean over {n} tokens"


def test_gqa_equal_queries_equal_outputs(dev):
    batch = W.make_batch([45, 700], 36)
    q = batch.q.copy()
    for g in range(8):
        q[:, 4 * g + 1:4 * g + 4] = q[:, 4 * g:4 * g + 1]
    batch.q = q
    got, _ = _gpu_step(batch, dev)
    for g in range(8):
        for j in range(1, 4):
            assert np.array_equal(got[:, 4 * g], got[:, 4 * g + j])


def test_score_shift_stability(dev, oracle_lib):
    """All scores raised by 1024: the online maximum keeps the result finite and unchanged."""
    batch = W.make_batch([90, 1300], 37)
    one = W.round_to_bf16_bits(np.array([1.0], np.float32))[0]
    batch.kv_k[:, :, 0] = one
    batch.q[..., 0] = 0
    base, _ = _gpu_step(batch, dev)
    batch.q[..., 0] = W.round_to_bf16_bits(np.array([8192.0], np.float32))[0]
    shifted, _ = _gpu_step(batch, dev)
    assert np.isfinite(shifted).all()
    # fp32 scores near 1024 carry ~1e-4 relative rounding: stability, not precision, is tested
    assert np.abs(shifted - base).max() <= 5e-3


def test_context_len_clamp_and_bad_table_entries(dev, oracle_lib):
    """Device data the kernels define: n < 0 -> zeros; n > max_context_len is cut;
    a table entry outside the pool drops that block (memory-safe) without
    touching other sequences."""
    import torch
    from paged_kv_cache_tv_amd.step import DeviceBatch
    batch = W.make_batch([100, 64, 300], 38)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    db = DeviceBatch(batch, dev)
    db.fill()
    db.write_step()
    # sequence 1: negative length -> zero row
    cl = db.context_lens.clone()
    db.context_lens[1] = -7
    # sequence 2: an entry past the pool and one negative entry
    db.block_tables[2, 3] = batch.num_blocks + 11
    db.block_tables[2, 5] = -2
    db.decode()
    db.reduce()
    got = db.out.cpu().numpy()
    torch.cuda.synchronize()
    assert (got[1] == 0).all()
    assert np.isfinite(got[2]).all()
    _assert_close(got[0:1], ref[0:1], "untouched sequence")
    # n above max_context_len is cut to max_context_len (= 300 here): same as n = 300
    db.context_lens.copy_(cl)
    db.block_tables.copy_(torch.from_numpy(batch.block_tables).to(dev))
    db.context_lens[2] = 100000
    db.decode()
    db.reduce()
    got2 = db.out.cpu().numpy()
    _assert_close(got2, ref, "clamped length")


@pytest.mark.parametrize("num_seqs", [256, 300])
def test_odd_device_data_large_grids(dev, oracle_lib, num_seqs):
    """The same defined behaviour on grids past one resident round: 256
    sequences (4 wavefronts, balanced order, whose scan reads every length)
    and 300 (one wavefront, plain order)."""
    import torch
    from paged_kv_cache_tv_amd.step import DeviceBatch
    rng = np.random.default_rng(48 + num_seqs)
    lens = rng.integers(1, 1500, size=num_seqs)
    lens[0] = 1500                                   # the longest: the clamp target
    batch = W.make_batch(lens, 48 + num_seqs)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    db = DeviceBatch(batch, dev)
    db.fill()
    db.write_step()
    cl = db.context_lens.clone()
    db.context_lens[1] = -7                          # negative length -> zero row
    db.block_tables[2, 3] = batch.num_blocks + 11    # an entry past the pool
    db.block_tables[2, 5] = -2                       # and a negative one
    db.decode()
    db.reduce()
    got = db.out.cpu().numpy()
    torch.cuda.synchronize()
    assert (got[1] == 0).all()
    assert np.isfinite(got[2]).all()
    keep = np.ones(num_seqs, bool)
    keep[[1, 2]] = False
    _assert_close(got[keep], ref[keep], f"{num_seqs} sequences, untouched rows")
    db.context_lens.copy_(cl)
    db.block_tables.copy_(torch.from_numpy(batch.block_tables).to(dev))
    db.context_lens[0] = 100000                      # cut to max_context_len = 1500
    db.decode()
    db.reduce()
    _assert_close(db.out.cpu().numpy(), ref, f"{num_seqs} sequences, clamped length")


def test_cache_write_skips_padding_and_out_of_pool(dev, oracle_lib):
    import torch
    import paged_kv_cache_tv_amd as tv
    batch = W.make_batch([40, 3], 39)
    k, v, slots = batch.fill_inputs()
    slots = slots.copy()
    slots[0] = -1
    slots[5] = batch.num_blocks * 16
    slots[7] = batch.num_blocks * 16 + 12345
    kc_ref, vc_ref = O.Oracle.new_pools(batch.num_blocks, 8, 64, 16)
    oracle_lib.cache_write(k, v, kc_ref, vc_ref, slots)
    kc, vc = tv.new_pools(batch.num_blocks, 8, 64, 16, dev, fill=W.BF16_NAN)
    kt = torch.from_numpy(k.view(np.int16)).to(dev)
    vt = torch.from_numpy(v.view(np.int16)).to(dev)
    tv.cache_write(kt, vt, kc, vc, torch.from_numpy(slots).to(dev))
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), kc_ref)
    assert np.array_equal(vc.cpu().numpy().view(np.uint16), vc_ref)


def test_errors_are_raised_before_launch(dev):
    import torch
    import paged_kv_cache_tv_amd as tv
    q = torch.zeros((2, 32, 64), dtype=torch.int16, device=dev)
    kc, vc = tv.new_pools(4, 8, 64, 16, dev)
    bt = torch.zeros((2, 4), dtype=torch.int32, device=dev)
    cl = torch.ones(2, dtype=torch.int32, device=dev)
    ws = tv.new_workspace(2, 32, 64, 64, 32, dev)
    with pytest.raises(tv.TvError) as e:          # partition not a multiple of the block size
        tv.paged_attention_decode(*tv.new_workspace(2, 32, 64, 64, 24, dev), q, kc, vc, bt, cl,
                                  64, 24, 0.125)
    assert e.value.status == 2
    with pytest.raises(tv.TvError) as e:          # max_context_len beyond the table
        tv.paged_attention_decode(*tv.new_workspace(2, 32, 64, 65, 32, dev), q, kc, vc, bt, cl,
                                  65, 32, 0.125)
    assert e.value.status == 2
    with pytest.raises(tv.TvError) as e:          # scale must be > 0
        tv.paged_attention_decode(*ws, q, kc, vc, bt, cl, 64, 32, -1.0)
    assert e.value.status == 2
    q48 = torch.zeros((2, 32, 48), dtype=torch.int16, device=dev)
    kc48, vc48 = tv.new_pools(4, 8, 48, 16, dev)
    with pytest.raises(tv.TvError) as e:          # head_dim 48 is not implemented
        tv.paged_attention_decode(*tv.new_workspace(2, 32, 48, 64, 32, dev), q48, kc48, vc48,
                                  bt, cl, 64, 32, 0.125)
    assert e.value.status == 3
    torch.cuda.synchronize()


def test_many_sequences(dev, oracle_lib):
    """1100 sequences of 0..700 tokens: a grid far larger than the chip, with
    empty contexts and many empty partitions mixed in."""
    rng = np.random.default_rng(40)
    lens = rng.integers(0, 700, size=1100)
    batch = W.make_batch(lens, 40)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    got, _ = _gpu_step(batch, dev)
    _assert_close(got, ref, "1100 sequences")


def test_short_sequences(dev, oracle_lib):
    """300 sequences of 1..40 tokens: one to three blocks each, nearly every
    tile a partial one."""
    rng = np.random.default_rng(41)
    lens = rng.integers(1, 40, size=300)
    batch = W.make_batch(lens, 41)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    got, _ = _gpu_step(batch, dev)
    _assert_close(got, ref, "300 short sequences")


@pytest.mark.parametrize("num_seqs", [64, 256, 300])
def test_launch_policy_paths(dev, oracle_lib, num_seqs):
    """The same batch through each launch form of the partition pass: a tight
    host bound on the lengths gives a small grid (4 wavefronts per partition);
    a loose one (65536) gives a grid of mostly empty partitions, served in the
    balanced order for up to 256 sequences (256: all four 64-sequence chunks
    of the in-kernel order) and in the plain order beyond.
    Every form meets the bars, its two-launch step equals its three-launch step
    bit for bit, and the forms agree with each other to rounding."""
    rng = np.random.default_rng(43 + num_seqs)
    lens = rng.integers(0, 1500, size=num_seqs)
    lens[:3] = [0, 1, 1500]
    batch = W.make_batch(lens, 43 + num_seqs, table_width=65536 // 16)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    outs = []
    for mc in (int(lens.max()), 65536):
        got, _ = _gpu_step(batch, dev, max_context_len=mc)
        _assert_close(got, ref, f"{num_seqs} sequences, max_context_len {mc}")
        fused, _ = _gpu_step(batch, dev, max_context_len=mc, fused=True)
        assert np.array_equal(got, fused), "two-launch step differs from the three-launch step"
        outs.append(got)
    assert np.abs(outs[0] - outs[1]).max() <= 1e-5


@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 4), (32, 2)])
def test_launch_policy_head_counts(dev, oracle_lib, hq, hkv):
    """Loose host bounds (the balanced order) and tight ones (4 wavefronts) with
    1, 2 and 4 K/V heads: the order deals each head's workgroups over
    cus / gcd(heads, cus) compute units, which is 256, 128 or 64 here."""
    rng = np.random.default_rng(47 + hkv)
    lens = rng.integers(1, 1200, size=96)
    batch = W.make_batch(lens, 47 + hkv, num_q_heads=hq, num_kv_heads=hkv,
                         table_width=131072 // 16)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    for mc in (int(lens.max()), 131072):
        got, _ = _gpu_step(batch, dev, max_context_len=mc)
        _assert_close(got, ref, f"{hq}/{hkv} heads, max_context_len {mc}")


_RANDOM_CASES = [
    # (seed, sequences, max length, partition, query heads, K/V heads, loose host bound)
    (60, 1, 5000, 512, 32, 8, False),
    (61, 5, 3000, 64, 16, 2, True),
    (62, 33, 2500, 256, 32, 8, False),
    (63, 130, 1800, 512, 8, 8, False),
    (64, 17, 4100, 2048, 32, 4, True),
    (65, 300, 600, 128, 32, 8, False),
    (66, 64, 4096, 512, 32, 8, True),
    (67, 200, 900, 512, 64, 4, False),
]


@pytest.mark.parametrize("case", _RANDOM_CASES, ids=[f"seed{c[0]}" for c in _RANDOM_CASES])
def test_random_configurations(dev, oracle_lib, case):
    """Seeded batches across the launch forms (4 wavefronts or 1, balanced or
    plain order), partition sizes, group sizes and host bounds: the output
    meets the bars against the oracle, the pools match its cache write bit
    for bit, and the two-launch step equals the three-launch step bit for
    bit."""
    seed, S, maxlen, part, hq, hkv, loose = case
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, maxlen + 1, size=S)
    width = 8192 if loose else None
    batch = W.make_batch(lens, seed, num_q_heads=hq, num_kv_heads=hkv, table_width=width)
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, batch)
    mc = 8192 * 16 if loose else int(lens.max())
    got, db = _gpu_step(batch, dev, partition_size=part, max_context_len=mc)
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    _assert_close(got, ref, f"seed {seed}: {S} x <= {maxlen} tokens, partition {part}, "
                            f"{hq}/{hkv} heads, host bound {mc}")
    fused, _ = _gpu_step(batch, dev, partition_size=part, max_context_len=mc, fused=True)
    assert np.array_equal(got, fused)


# ---------------------------------------------------------------------------
# tv_paged_attention_decode_append: the cache write folded into the partition
# pass.  Under its precondition it must equal the three-call step bit for bit.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_append_workload_parity(dev, oracle_lib, index):
    """Full-size workloads through the two-launch step: pools bit-exact against
    the oracle, output within the bars and bitwise equal to the three-launch step."""
    batch = W.make_workload(index)
    ref, kc_ref, vc_ref = _oracle_step(oracle_lib, ("workload", index), batch)
    got, db = _gpu_step(batch, dev, fused=True)
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref), "K pool differs from the oracle's cache write"
    assert np.array_equal(vc, vc_ref), "V pool differs from the oracle's cache write"
    _assert_close(got, ref, f"append workload {index}")
    sep, _ = _gpu_step(batch, dev)
    assert np.array_equal(got, sep), "fused step differs from the three-launch step"


def test_append_edge_positions(dev, oracle_lib):
    """The new token at every kind of position: first of a block, last of a block,
    alone in a partition, the whole context (n = 1 returns V_new exactly)."""
    lens = [1, 2, 16, 17, 32, 33, 512, 513, 1024, 1025, 1, 0]
    batch = W.make_batch(lens, 42)
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, batch)
    got, db = _gpu_step(batch, dev, fused=True)
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    _assert_close(got, ref, "append edge positions")
    sep, _ = _gpu_step(batch, dev)
    assert np.array_equal(got, sep)
    k_new, v_new, _ = batch.step_inputs()
    vnew = W.bf16_bits_to_float32(v_new)[:, np.repeat(np.arange(8), 4)]
    for s, n in enumerate(lens):
        if n == 1:
            assert np.array_equal(got[s], vnew[s]), "a one-token context must return V_new exactly"
        if n == 0:
            assert (got[s] == 0).all()


def test_append_skips_and_slots_elsewhere(dev, oracle_lib):
    """slot -1 and slots past the pool append nothing; a slot in a block no
    sequence reads is written there while position n-1 is read from the pool."""
    import torch
    import paged_kv_cache_tv_amd as tv
    from paged_kv_cache_tv_amd.step import DeviceBatch
    batch = W.make_batch([40, 70, 300, 5], 43)
    k_new, v_new, step_slots = batch.step_inputs()
    rng = np.random.default_rng(43)
    k_old = W.round_to_bf16_bits(rng.standard_normal(k_new.shape).astype(np.float32))
    v_old = W.round_to_bf16_bits(rng.standard_normal(v_new.shape).astype(np.float32))
    used = set(batch.block_tables.ravel().tolist())
    spare = next(b for b in range(batch.num_blocks) if b not in used and b != batch.poison_block)
    slots = step_slots.copy()
    slots[0] = -1                                   # no new token for sequence 0
    slots[1] = batch.num_blocks * 16 + 3            # past the pool: skipped
    slots[2] = spare * 16 + 7                       # written elsewhere; not read by anyone
    # Reference: position n-1 first holds (k_old, v_old); then the oracle's cache
    # write of the new tokens at `slots`; then attention.
    kc_ref, vc_ref = O.build_pools(oracle_lib, batch, include_step=False)
    oracle_lib.cache_write(k_old, v_old, kc_ref, vc_ref, step_slots)
    oracle_lib.cache_write(k_new, v_new, kc_ref, vc_ref, slots)
    ref = oracle_lib.paged_attention(batch.q, kc_ref, vc_ref, batch.block_tables,
                                     batch.context_lens, batch.scale)
    db = DeviceBatch(batch, dev)
    db.fill()
    tv.cache_write(torch.from_numpy(k_old.view(np.int16)).to(dev),
                   torch.from_numpy(v_old.view(np.int16)).to(dev), db.k_cache, db.v_cache,
                   db.step_slots)
    db.step_slots = torch.from_numpy(slots).to(dev)
    out = db.fused_step().clone()
    torch.cuda.synchronize()
    kc, vc = db.pools_numpy()
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    _assert_close(out.cpu().numpy(), ref, "append skips")


def test_append_errors(dev):
    import torch
    import paged_kv_cache_tv_amd as tv
    q = torch.zeros((2, 32, 64), dtype=torch.int16, device=dev)
    kc, vc = tv.new_pools(4, 8, 64, 16, dev)
    kn = torch.zeros((2, 8, 64), dtype=torch.int16, device=dev)
    bt = torch.zeros((2, 4), dtype=torch.int32, device=dev)
    cl = torch.ones(2, dtype=torch.int32, device=dev)
    ws = tv.new_workspace(2, 32, 64, 64, 32, dev)
    sm = torch.zeros(2, dtype=torch.int64, device=dev)
    with pytest.raises(ValueError):                   # k_new of the wrong shape
        tv.paged_attention_decode_append(*ws, q, kn[:1], kn, sm, kc, vc, bt, cl, 64, 32, 0.125)
    lib = tv.lib()
    pa, pm, ps = ws
    st = lib.tv_paged_attention_decode_append(pa.data_ptr(), pm.data_ptr(), ps.data_ptr(),
                                              q.data_ptr(), None, kn.data_ptr(), sm.data_ptr(),
                                              kc.data_ptr(), vc.data_ptr(), bt.data_ptr(),
                                              cl.data_ptr(), 2, 32, 8, 64, 16, 4, 4, 64, 32,
                                              0.125, None)
    assert st == 1                                    # TV_ERR_NULL, nothing launched
    torch.cuda.synchronize()
