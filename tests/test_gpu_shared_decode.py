"""Shared-prefix decode (tv_paged_attention_decode_shared) on the GPU.

Each MFMA column is computed independently, so reading a shared prefix once
for the whole group must give the same partials, and after the merge the
same output, as the per-sequence pass, bit for bit.  The tests compare the
two paths on the shared-prefix workload and on ragged groups, and the output
against the oracle.  Pools are NaN-poisoned outside the written slots.
"""

import numpy as np
import pytest

import oracle as O
from paged_kv_cache_tv_amd import workloads as W

pytestmark = pytest.mark.gpu


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


def _run(b, dev, part, shared=None, group_size=1, lens=None):
    """Both pools written, then either pass and the merge: (out, partials)."""
    import torch
    import paged_kv_cache_tv_amd as tv
    lens = b.context_lens if lens is None else lens
    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev,
                          fill=W.BF16_NAN)
    for k, v, sl in (b.fill_inputs(), b.step_inputs()):
        live = sl >= 0
        tv.cache_write(_to_dev(k[live], dev), _to_dev(v[live], dev), kc, vc,
                       _to_dev(sl[live], dev))
    mc = int(lens.max())
    ws = tv.new_workspace(b.num_seqs, b.num_q_heads, b.head_dim, mc, part, dev)
    for t in ws:
        t.fill_(float("nan"))
    q, bt, cl = _to_dev(b.q, dev), _to_dev(b.block_tables, dev), _to_dev(lens, dev)
    if shared is None:
        tv.paged_attention_decode(*ws, q, kc, vc, bt, cl, mc, part, b.scale)
    else:
        tv.paged_attention_decode_shared(*ws, q, kc, vc, bt, cl, _to_dev(shared, dev), group_size,
                                         mc, part, b.scale)
    out = torch.empty((b.num_seqs, b.num_q_heads, b.head_dim), dtype=torch.float32, device=dev)
    tv.paged_attention_reduce(out, *ws, cl, mc, part)
    torch.cuda.synchronize()
    return out.cpu().numpy(), [t.cpu().numpy() for t in ws]


def _same_partials(pa, pb, lens, part):
    """Partials equal bit for bit wherever the call defines them."""
    for s, n in enumerate(lens):
        P = -(-int(n) // part)
        for x, y in zip(pa, pb):
            assert np.array_equal(x[s, :, :P].view(np.uint32), y[s, :, :P].view(np.uint32)), s


def test_shared_prefix_workload(dev, oracle_lib):
    """64 prompts x 4 samples sharing 1024 tokens, partitions of 512: two
    shared partitions per group."""
    b = W.make_workload(4)
    shared = np.full(64, 1024, np.int32)
    out_s, part_s = _run(b, dev, 512, shared, 4)
    out_p, part_p = _run(b, dev, 512)
    _same_partials(part_s, part_p, b.context_lens, 512)
    assert np.array_equal(out_s.view(np.uint32), out_p.view(np.uint32))
    ref, _, _ = O.decode_step(oracle_lib, b)
    err = np.abs(out_s.astype(np.float64) - ref)
    print(f"shared-prefix workload: max_abs={err.max():.3e}", flush=True)
    assert err.max() <= 1e-4 and err.mean() <= 1e-6


@pytest.mark.parametrize("samples,prefix,part", [(3, 704, 64), (2, 1536, 512), (4, 512, 512),
                                                 (4, 256, 64)])
def test_shared_prefix_ragged_groups(dev, samples, prefix, part):
    """Groups of 2-4, prefixes that are not a whole number of partitions, a
    partial last group, a member whose context is cut below the prefix, and a
    group that declares no sharing."""
    rng = np.random.default_rng(120 + samples + part)
    prompts = 5
    priv = rng.integers(0, 300, prompts * samples)
    b = W.make_shared_prefix_batch(prompts, samples, prefix, priv, 121 + prefix)
    S = b.num_seqs - 1                               # drop the last sequence: partial last group
    b.context_lens = b.context_lens[:S].copy()
    b.block_tables = b.block_tables[:S]
    b.q = b.q[:S]
    b.new_slots = b.new_slots[:S]
    b.new_rows = b.new_rows[:S]
    lens = b.context_lens.copy()
    lens[samples] = prefix // 2                      # member of group 1 cut below the prefix
    ngroups = -(-S // samples)
    shared = np.full(ngroups, prefix, np.int32)
    shared[2] = 0                                    # group 2: no sharing declared
    out_s, part_s = _run(b, dev, part, shared, samples, lens)
    out_p, part_p = _run(b, dev, part, lens=lens)
    _same_partials(part_s, part_p, lens, part)
    assert np.array_equal(out_s.view(np.uint32), out_p.view(np.uint32))


# ---------------------------------------------------------------------------
# tv_paged_attention_decode_shared_append: the new tokens' cache write folded
# into the shared-prefix pass.  Under its preconditions it must equal
# tv_cache_write of the new tokens followed by tv_paged_attention_decode_shared
# bit for bit: pools and partials.
# ---------------------------------------------------------------------------

def _run_append(b, dev, part, shared, group_size, lens=None, group_order=None):
    """Cached tokens written with tv_cache_write, then the shared pass with the
    new tokens appended: (out, partials, pools)."""
    import torch
    import paged_kv_cache_tv_amd as tv
    lens = b.context_lens if lens is None else lens
    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev,
                          fill=W.BF16_NAN)
    k, v, sl = b.fill_inputs()
    live = sl >= 0
    tv.cache_write(_to_dev(k[live], dev), _to_dev(v[live], dev), kc, vc, _to_dev(sl[live], dev))
    sk, sv, ss = b.step_inputs()
    mc = int(lens.max())
    ws = tv.new_workspace(b.num_seqs, b.num_q_heads, b.head_dim, mc, part, dev)
    for t in ws:
        t.fill_(float("nan"))
    q, bt, cl = _to_dev(b.q, dev), _to_dev(b.block_tables, dev), _to_dev(lens, dev)
    go = None if group_order is None else _to_dev(group_order, dev)
    tv.paged_attention_decode_shared_append(*ws, q, _to_dev(sk, dev), _to_dev(sv, dev),
                                            _to_dev(ss.astype(np.int64), dev), kc, vc, bt, cl,
                                            _to_dev(shared, dev), group_size, mc, part, b.scale,
                                            group_order=go)
    out = torch.empty((b.num_seqs, b.num_q_heads, b.head_dim), dtype=torch.float32, device=dev)
    tv.paged_attention_reduce(out, *ws, cl, mc, part)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), [t.cpu().numpy() for t in ws],
            (kc.cpu().numpy().view(np.uint16), vc.cpu().numpy().view(np.uint16)))


def test_shared_append_workload(dev, oracle_lib):
    """The parallel-sampling step of the shared-prefix workload in two
    launches: pools bit-exact against the oracle's cache write, partials and
    output bitwise equal to the write followed by the shared pass."""
    b = W.make_workload(4)
    shared = np.full(64, 1024, np.int32)
    out_a, part_a, (kc, vc) = _run_append(b, dev, 512, shared, 4)
    out_s, part_s = _run(b, dev, 512, shared, 4)
    _same_partials(part_a, part_s, b.context_lens, 512)
    assert np.array_equal(out_a.view(np.uint32), out_s.view(np.uint32))
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, b)
    assert np.array_equal(kc, kc_ref), "K pool differs from the oracle's cache write"
    assert np.array_equal(vc, vc_ref), "V pool differs from the oracle's cache write"
    err = np.abs(out_a.astype(np.float64) - ref)
    print(f"shared-prefix append step: max_abs={err.max():.3e}", flush=True)
    assert err.max() <= 1e-4 and err.mean() <= 1e-6


@pytest.mark.parametrize("samples,prefix,part", [(3, 704, 64), (4, 256, 64), (2, 1536, 512)])
def test_shared_append_ragged_groups(dev, samples, prefix, part):
    """Ragged groups as above.  The member cut below the prefix keeps the new
    token of its full length: with (4, 256, 64) its last position falls in a
    shared partition, the case where the token is only written."""
    rng = np.random.default_rng(130 + samples + part)
    prompts = 5
    priv = rng.integers(0, 300, prompts * samples)
    b = W.make_shared_prefix_batch(prompts, samples, prefix, priv, 131 + prefix)
    lens = b.context_lens.copy()
    lens[samples] = prefix // 2
    ngroups = -(-b.num_seqs // samples)
    shared = np.full(ngroups, prefix, np.int32)
    shared[2] = 0
    out_a, part_a, pools_a = _run_append(b, dev, part, shared, samples, lens)
    out_s, part_s = _run(b, dev, part, shared, samples, lens)
    _same_partials(part_a, part_s, lens, part)
    assert np.array_equal(out_a.view(np.uint32), out_s.view(np.uint32))
    # Pools: the same as writing every token with tv_cache_write.
    import paged_kv_cache_tv_amd as tv
    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev,
                          fill=W.BF16_NAN)
    for k, v, sl in (b.fill_inputs(), b.step_inputs()):
        live = sl >= 0
        tv.cache_write(_to_dev(k[live], dev), _to_dev(v[live], dev), kc, vc,
                       _to_dev(sl[live], dev))
    assert np.array_equal(pools_a[0], kc.cpu().numpy().view(np.uint16))
    assert np.array_equal(pools_a[1], vc.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("append", [False, True])
def test_shared_groups_in_any_order(dev, append):
    """Groups given by a member order instead of consecutive positions: the
    shared-prefix workload with its sequences shuffled must give, sequence
    for sequence, the partials and output of the consecutive layout bit for
    bit (and with appends, the same pools)."""
    import torch
    import paged_kv_cache_tv_amd as tv
    b = W.make_workload(4)
    S = b.num_seqs
    perm = np.random.default_rng(140).permutation(S)      # sequence i moves to index perm[i]
    order = perm.astype(np.int32)                         # position i (group i // 4) -> perm[i]
    part = 512
    shared = np.full(S // 4, 1024, np.int32)

    def run(shuffled):
        kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev,
                              fill=W.BF16_NAN)
        k, v, sl = b.fill_inputs()
        live = sl >= 0
        tv.cache_write(_to_dev(k[live], dev), _to_dev(v[live], dev), kc, vc,
                       _to_dev(sl[live], dev))
        sk, sv, ss = b.step_inputs()
        if not append:
            live = ss >= 0
            tv.cache_write(_to_dev(sk[live], dev), _to_dev(sv[live], dev), kc, vc,
                           _to_dev(ss[live], dev))

        def arr(x):                                       # row i of x -> row perm[i]
            if not shuffled:
                return x
            y = np.empty_like(x)
            y[perm] = x
            return y
        mc = int(b.context_lens.max())
        ws = tv.new_workspace(S, b.num_q_heads, b.head_dim, mc, part, dev)
        for t in ws:
            t.fill_(float("nan"))
        q, bt, cl = _to_dev(arr(b.q), dev), _to_dev(arr(b.block_tables), dev), \
            _to_dev(arr(b.context_lens), dev)
        go = _to_dev(order, dev) if shuffled else None
        if append:
            tv.paged_attention_decode_shared_append(
                *ws, q, _to_dev(arr(sk), dev), _to_dev(arr(sv), dev),
                _to_dev(arr(ss.astype(np.int64)), dev), kc, vc, bt, cl, _to_dev(shared, dev), 4,
                mc, part, b.scale, group_order=go)
        else:
            tv.paged_attention_decode_shared(*ws, q, kc, vc, bt, cl, _to_dev(shared, dev), 4, mc,
                                             part, b.scale, group_order=go)
        out = torch.empty((S, b.num_q_heads, b.head_dim), dtype=torch.float32, device=dev)
        tv.paged_attention_reduce(out, *ws, cl, mc, part)
        torch.cuda.synchronize()
        res = [out.cpu().numpy()] + [t.cpu().numpy() for t in ws]
        if shuffled:
            res = [r[perm] for r in res]                  # back to the original sequence order
        pools = (kc.cpu().numpy().view(np.uint16), vc.cpu().numpy().view(np.uint16))
        return res, pools

    (out_c, *part_c), pools_c = run(False)
    (out_s, *part_s), pools_s = run(True)
    _same_partials(part_s, part_c, b.context_lens, part)
    assert np.array_equal(out_s.view(np.uint32), out_c.view(np.uint32))
    assert np.array_equal(pools_s[0], pools_c[0]) and np.array_equal(pools_s[1], pools_c[1])


# ---------------------------------------------------------------------------
# tv_paged_attention_decode_shared_step: the parallel-sampling step in one
# call.  In its one-launch form (groups of up to 4, in their own order or
# through group_order, every (group, K/V head) workgroup resident) the shared
# tiles and each member's own
# tiles are cut into 8 equal parts per range instead of the workspace's
# partitions, so the output equals the two-call step (shared append + merge)
# to rounding; the pools equal it bit for bit.
# ---------------------------------------------------------------------------

def _forms_bar(b):
    """How far two correct orders of the same step may differ: each folds P
    into V as bf16 hi + lo parts (relative error <= 2^-17 per weight) against
    an exact fp32 sum, so each is within 2^-17 * max|V| of the exactly
    weighted mean; 1e-6 covers their fp32 summation orders."""
    v = W.bf16_bits_to_float32(b.kv_v)
    return 2.0 ** -16 * float(np.abs(v[np.isfinite(v)]).max()) + 1e-6


def _run_shared_step(b, dev, part, shared, group_size, lens=None, group_order=None):
    import torch
    import paged_kv_cache_tv_amd as tv
    lens = b.context_lens if lens is None else lens
    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim, b.block_size, dev,
                          fill=W.BF16_NAN)
    k, v, sl = b.fill_inputs()
    live = sl >= 0
    tv.cache_write(_to_dev(k[live], dev), _to_dev(v[live], dev), kc, vc, _to_dev(sl[live], dev))
    sk, sv, ss = b.step_inputs()
    mc = int(lens.max())
    ws = tv.new_workspace(b.num_seqs, b.num_q_heads, b.head_dim, mc, part, dev)
    for t in ws:
        t.fill_(float("nan"))
    out = torch.full((b.num_seqs, b.num_q_heads, b.head_dim), float("nan"), dtype=torch.float32,
                     device=dev)
    q, bt, cl = _to_dev(b.q, dev), _to_dev(b.block_tables, dev), _to_dev(lens, dev)
    go = None if group_order is None else _to_dev(group_order, dev)
    tv.paged_attention_decode_shared_step(out, ws, q, _to_dev(sk, dev), _to_dev(sv, dev),
                                          _to_dev(ss.astype(np.int64), dev), kc, vc, bt, cl,
                                          _to_dev(shared, dev), group_size, mc, part, b.scale,
                                          group_order=go)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (kc.cpu().numpy().view(np.uint16), vc.cpu().numpy().view(np.uint16))


def test_shared_step_workload(dev, oracle_lib):
    """The shared-prefix workload's step in one launch: pools bit-exact against
    the oracle's cache write, output within the oracle bars, run-to-run
    identical, and within rounding (_forms_bar) of the two-call step."""
    import paged_kv_cache_tv_amd as tv
    b = W.make_workload(4)
    shared = np.full(64, 1024, np.int32)
    mc = int(b.context_lens.max())
    assert tv.decode_shared_step_form(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                      b.block_size, mc, 512, 4) == 1
    out, (kc, vc) = _run_shared_step(b, dev, 512, shared, 4)
    out2, _ = _run_shared_step(b, dev, 512, shared, 4)
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "two calls differ"
    two, _, _ = _run_append(b, dev, 512, shared, 4)
    d = np.abs(out - two).max()
    print(f"shared step vs two calls: max_abs={d:.3e}", flush=True)
    assert d <= _forms_bar(b)
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, b)
    assert np.array_equal(kc, kc_ref), "K pool differs from the oracle's cache write"
    assert np.array_equal(vc, vc_ref), "V pool differs from the oracle's cache write"
    err = np.abs(out.astype(np.float64) - ref)
    print(f"shared step: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 1e-4 and err.mean() <= 1e-6


@pytest.mark.parametrize("samples,prefix,part,hq,hkv", [
    (3, 704, 64, 32, 8),       # prefix not a whole number of partitions
    (4, 256, 64, 32, 8),       # a member's last position in a shared partition
    (2, 1536, 512, 32, 8),
    (1, 512, 128, 32, 8),      # groups of one
    (4, 608, 128, 16, 16),     # one query head per K/V head: 4 columns
    (2, 304, 64, 16, 2),       # 8 query heads per K/V head: 16 columns
])
def test_shared_step_ragged_groups(dev, samples, prefix, part, hq, hkv):
    """Ragged groups in one launch: a partial last group, a member cut below the
    prefix, a group that declares no sharing, an empty context and a skipped
    slot; output within rounding of the two-call step (zero rows for the empty
    context; the sequence whose slot is skipped attends its NaN-poisoned last
    position in both), pools bit for bit the two-call step's."""
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(150 + samples + part + hkv)
    prompts = 5
    priv = rng.integers(0, 300, prompts * samples)
    b = W.make_shared_prefix_batch(prompts, samples, prefix, priv, 151 + prefix,
                                   num_q_heads=hq, num_kv_heads=hkv)
    S = b.num_seqs - 1 if samples > 1 else b.num_seqs
    b.context_lens = b.context_lens[:S].copy()
    b.block_tables = b.block_tables[:S]
    b.q = b.q[:S]
    b.new_slots = b.new_slots[:S].copy()
    b.new_rows = b.new_rows[:S]
    lens = b.context_lens.copy()
    if samples > 1:
        lens[samples] = prefix // 2                  # member of group 1 cut below the prefix
    lens[-1] = 0                                     # an empty context
    b.new_slots[1] = -1                              # a skipped slot
    ngroups = -(-S // samples)
    shared = np.full(ngroups, prefix, np.int32)
    shared[min(2, ngroups - 1)] = 0                  # no sharing declared
    mc = int(lens.max())
    assert tv.decode_shared_step_form(S, hq, hkv, 64, 16, mc, part, samples) == 1
    out, pools = _run_shared_step(b, dev, part, shared, samples, lens)
    two, _, pools2 = _run_append(b, dev, part, shared, samples, lens)
    nan = np.isnan(out)
    assert np.array_equal(nan, np.isnan(two)), "NaN rows differ from the two-call step"
    assert not np.delete(nan, 1, axis=0).any(), "NaN outside the skipped slot's sequence"
    assert not out[lens == 0].any(), "an empty context gives zero rows"
    d = np.abs(np.where(nan, 0.0, out - two)).max()
    print(f"ragged shared step ({samples}, {prefix}, {part}, {hq}/{hkv}): max_abs={d:.3e}",
          flush=True)
    assert d <= _forms_bar(b)
    assert np.array_equal(pools[0], pools2[0]) and np.array_equal(pools[1], pools2[1])


def test_shared_step_two_launch_form(dev):
    """Outside the one-launch form (groups of more than 4) the step is the
    shared append and the merge: bit for bit the two calls."""
    import paged_kv_cache_tv_amd as tv
    b = W.make_workload(4)
    S = b.num_seqs
    part = 512
    mc = int(b.context_lens.max())
    b.q = b.q[:, :16].copy()                         # 16 query heads: G = 2, groups of 8
    b.num_q_heads = 16
    gs = 8
    shared = np.full(S // 8, 1024, np.int32)
    assert tv.decode_shared_step_form(S, b.num_q_heads, b.num_kv_heads, 64, 16, mc, part, gs,
                                      False) == 2
    out, pools = _run_shared_step(b, dev, part, shared, gs)
    two, _, pools2 = _run_append(b, dev, part, shared, gs)
    assert np.array_equal(out.view(np.uint32), two.view(np.uint32))
    assert np.array_equal(pools[0], pools2[0]) and np.array_equal(pools[1], pools2[1])


@pytest.mark.parametrize("left_out", [False, True], ids=["permuted", "one-left-out"])
def test_shared_step_group_order(dev, oracle_lib, left_out):
    """Groups given by group_order in the one-launch form: the prompts' groups
    and their members in a shuffled order (each group still its prompt's 4
    samples, so the shared blocks are shared), and optionally one position
    whose entry lies outside the batch (its sequence is then not computed and
    its group shares nothing).  Output within rounding of the two-call step
    with the same order and within the oracle bars, pools bit-exact against
    the two-call step's (and the oracle's when nothing is left out)."""
    import paged_kv_cache_tv_amd as tv
    b = W.make_workload(4)
    S = b.num_seqs
    part = 512
    mc = int(b.context_lens.max())
    rng = np.random.default_rng(73)
    order = np.concatenate([4 * g + rng.permutation(4) for g in rng.permutation(S // 4)])
    order = order.astype(np.int32)
    skipped = None
    if left_out:
        skipped = int(order[5])
        order[5] = -1                                # position 5: outside the batch
    shared = np.full(S // 4, 1024, np.int32)
    assert tv.decode_shared_step_form(S, b.num_q_heads, b.num_kv_heads, 64, 16, mc, part, 4,
                                      True) == 1
    out, pools = _run_shared_step(b, dev, part, shared, 4, group_order=order)
    out2, _ = _run_shared_step(b, dev, part, shared, 4, group_order=order)
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "two calls differ"
    two, _, pools2 = _run_append(b, dev, part, shared, 4, group_order=order)
    keep = np.ones(S, bool)
    if skipped is not None:
        keep[skipped] = False
        assert np.isnan(out[skipped]).all(), "a sequence not listed keeps its row"
    d = np.abs(out[keep] - two[keep]).max()
    print(f"group_order shared step vs two calls: max_abs={d:.3e}", flush=True)
    assert d <= _forms_bar(b)
    assert np.array_equal(pools[0], pools2[0]) and np.array_equal(pools[1], pools2[1])
    ref, kc_ref, vc_ref = O.decode_step(oracle_lib, b)
    if skipped is None:
        assert np.array_equal(pools[0], kc_ref) and np.array_equal(pools[1], vc_ref)
    err = np.abs(out[keep].astype(np.float64) - ref[keep])
    print(f"group_order shared step: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 1e-4 and err.mean() <= 1e-6
