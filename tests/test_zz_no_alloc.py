"""tv_paged_attention_decode_step_noalloc (the decode step for callers that
cannot allocate) against tv_paged_attention_decode_step, through the C-ABI.

The two calls run the same kernels; the only difference is where the
partition workspace lives (caller buffers, or the library's fixed per-GPU
array).  Each case runs the existing call and then the allocation-free one on
the same inputs and requires the outputs to be bitwise equal, and within the
contract of the oracle comparison (max-abs <= 1e-2, mean-abs <= 1e-3).  The
cases run back to back in one process, the later ones smaller, so the array
holds the previous call's partials when the next call starts: a result that
depended on stale contents would differ from the existing call's.
"""

import numpy as np
import pytest

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


def _pair(db, dev):
    """(out of the existing call, out of the allocation-free call), each after
    its own run of the step on the same device batch.  The step writes each
    sequence's new token into its own slot, so running it twice leaves the
    pools as after one run."""
    import torch
    import paged_kv_cache_tv_amd as tv
    b = db.batch
    db.out.fill_(float("nan"))
    ref = db.call_step().clone()
    got = torch.full_like(ref, float("nan"))
    tv.paged_attention_decode_step_noalloc(got, db.q, db.step_k, db.step_v, db.step_slots,
                                           db.k_cache, db.v_cache, db.block_tables,
                                           db.context_lens, db.max_context_len,
                                           db.partition_size, b.scale)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def _check(ref, got, oracle_out, what):
    assert np.isfinite(got).all(), what
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), f"{what}: not bitwise equal"
    err = np.abs(got.astype(np.float64) - oracle_out)
    print(f"{what}: bitwise equal to tv_paged_attention_decode_step; vs oracle "
          f"max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, what


def test_noalloc_step_matches_existing_call_twice(dev, oracle_lib):
    """Calls in a row whose steps go through the workspace (partition pass,
    then the merge kernel): batch 64 x U[512, 4096] in 16 partitions of 256
    tokens (4.3 MB of the array), then the smaller batch 8 x U[128, 1024] in
    16 partitions of 64 (0.5 MB), then one 37-token sequence (one partition:
    no workspace).  The 512-token partitions of the first two workloads take
    the one-launch whole-sequence form, which needs no workspace at all: run
    last, it must match too."""
    import oracle as O
    from paged_kv_cache_tv_amd.step import DeviceBatch
    for idx, part in ((3, 256), (2, 64), (1, 512), (3, 512), (2, 512)):
        batch = W.make_workload(idx)
        print(f"workload {idx}: {batch.name}, partition {part}", flush=True)
        db = DeviceBatch(batch, dev, partition_size=part)
        db.fill()
        ref, got = _pair(db, dev)
        want, _, _ = O.decode_step(oracle_lib, batch)
        _check(ref, got, want, f"{batch.name} partition {part}")
        del db


def test_noalloc_partition_sizes(dev, oracle_lib):
    """The same batch under partition sizes that change the workspace's shape
    (and so where each row lands in the array): 16 and 64 tokens, and 512
    (the one-launch form, no workspace)."""
    import oracle as O
    from paged_kv_cache_tv_amd.step import DeviceBatch
    batch = W.make_workload(2)
    want, _, _ = O.decode_step(oracle_lib, batch)
    for part in (512, 64, 16):
        db = DeviceBatch(batch, dev, partition_size=part)
        db.fill()
        ref, got = _pair(db, dev)
        _check(ref, got, want, f"{batch.name} partition {part}")
        del db


def test_noalloc_rejects_oversized_workspace(dev):
    """A workspace above the fixed array is refused before anything runs, and
    the output is left untouched."""
    import torch
    import paged_kv_cache_tv_amd as tv
    from paged_kv_cache_tv_amd.step import DeviceBatch
    batch = W.make_workload(2)
    db = DeviceBatch(batch, dev)
    db.fill()
    out = torch.full_like(db.out, 7.0)
    # 8 sequences x 32 heads x P x 66 floats > 16 MiB needs P > 248: one
    # 16-token partition per block of a 4096-token bound.
    with pytest.raises(tv.TvError) as e:
        tv.paged_attention_decode_step_noalloc(out, db.q, db.step_k, db.step_v, db.step_slots,
                                               db.k_cache, db.v_cache, db.block_tables,
                                               db.context_lens, 4096 * 4, 16, batch.scale)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool((out == 7.0).all().item())
