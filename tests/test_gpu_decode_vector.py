"""tv_paged_attention_decode_vector -- the partition pass with its QK and PV
contractions on the vector ALUs -- against the CPU oracle and against the
matrix (MFMA) form tv_paged_attention_decode, through the C interface.

Bars: the oracle's (max-abs <= 1e-2, mean-abs <= 1e-3, internal max-abs <=
1e-4, as in test_gpu_parity).  Against the matrix form: within
2^-16 * max|V| + 1e-6.  The matrix form keeps each weight to at least 16
significant bits (bf16 hi + lo parts) and this form keeps it in fp32, so each
is within 2^-17 * max|V| of the exactly weighted mean; 1e-6 covers their
different fp32 summation orders.  Where the two forms' definitions are exact
(an empty context, a one-token context) the results are compared exactly.
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


def _assert_close(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got.astype(np.float64) - ref)
    mx, mean = float(d.max()), float(d.mean())
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= CONTRACT_MAX and mean <= CONTRACT_MEAN, f"{what}: contract broken"
    assert mx <= INTERNAL_MAX, f"{what}: internal bar broken ({mx:.3e})"


def _forms_bar(batch):
    v = W.bf16_bits_to_float32(batch.kv_v)
    return 2.0 ** -16 * float(np.abs(v[np.isfinite(v)]).max()) + 1e-6


def _vector_pass(db):
    import paged_kv_cache_tv_amd as tv
    pa, pm, ps = db.workspace
    tv.paged_attention_decode_vector(pa, pm, ps, db.q, db.k_cache, db.v_cache, db.block_tables,
                                     db.context_lens, db.max_context_len, db.partition_size,
                                     db.batch.scale)


def _both_forms(db):
    """(vector, matrix) outputs of pass + merge on the device batch as it stands."""
    import torch
    db.out.fill_(float("nan"))
    _vector_pass(db)
    db.reduce()
    vec = db.out.clone()
    db.out.fill_(float("nan"))
    db.decode()
    db.reduce()
    mat = db.out.clone()
    torch.cuda.synchronize()
    return vec.cpu().numpy(), mat.cpu().numpy()


def _device_batch(batch, dev, partition_size=None):
    from paged_kv_cache_tv_amd.step import DeviceBatch
    db = DeviceBatch(batch, dev, partition_size=partition_size)
    db.fill()
    db.write_step()
    return db


@pytest.mark.parametrize("index", [2, 3])
def test_vector_workloads(dev, oracle_lib, index):
    """8 x U[128, 1024] (plain order) and 64 x U[512, 4096] (balanced order):
    within the bars against the oracle, within the forms bar of the matrix
    form, and run-to-run identical."""
    print(f"workload {index}: {W.WORKLOADS[index]}", flush=True)
    batch = W.make_workload(index)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    db = _device_batch(batch, dev)
    vec, mat = _both_forms(db)
    _assert_close(vec, ref, f"workload {index}, vector form")
    assert np.abs(vec - mat).max() <= _forms_bar(batch), "vector form far from the matrix form"
    vec2, _ = _both_forms(db)
    assert np.array_equal(vec, vec2), "run-to-run difference"


RAGGED = [1, 15, 16, 17, 200, 511, 512, 513, 1024, 1500, 3001, 4096]


@pytest.mark.parametrize("partition_size", [16, 512, 4096])
def test_vector_ragged_partitions(dev, oracle_lib, partition_size):
    """Ragged contexts with one-block, standard and single partitions: several
    tiles per wavefront, partial last tiles and wavefronts with no tile."""
    batch = W.make_batch(RAGGED, 31)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    db = _device_batch(batch, dev, partition_size=partition_size)
    vec, mat = _both_forms(db)
    _assert_close(vec, ref, f"partition {partition_size}, vector form")
    assert np.abs(vec - mat).max() <= _forms_bar(batch)


def test_vector_edge_lengths(dev, oracle_lib):
    """Empty contexts give zero rows and a one-token context returns that
    token's V exactly (its weight is 2^0 = 1 and the sum is 1)."""
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1023, 1024, 1025, 0]
    batch = W.make_batch(lens, 33)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    db = _device_batch(batch, dev)
    vec, mat = _both_forms(db)
    assert (vec[0] == 0).all() and (vec[-1] == 0).all(), "empty context must give zeros"
    _assert_close(vec, ref, "edge lengths, vector form")
    one = lens.index(1)
    _, v = batch.logical_kv(one)
    expect = W.bf16_bits_to_float32(v[0])[np.repeat(np.arange(8), 4)]
    assert np.array_equal(vec[one], expect), "a one-token context must return that V exactly"
    assert np.array_equal(vec[one], mat[one])


def test_vector_odd_device_data(dev, oracle_lib):
    """The defined behaviour of the matrix form on odd device data: a negative
    length gives a zero row, table entries outside the pool drop their blocks
    (the same blocks in both forms), other sequences are untouched."""
    batch = W.make_batch([100, 64, 300, 700], 38)
    ref, _, _ = O.decode_step(oracle_lib, batch)
    db = _device_batch(batch, dev)
    db.context_lens[1] = -7
    db.block_tables[2, 3] = batch.num_blocks + 11
    db.block_tables[2, 5] = -2
    vec, mat = _both_forms(db)
    assert (vec[1] == 0).all()
    assert np.isfinite(vec[2]).all()
    assert np.abs(vec[2] - mat[2]).max() <= _forms_bar(batch), "dropped blocks differ between forms"
    keep = [0, 3]
    _assert_close(vec[keep], ref[keep], "untouched sequences")


def test_vector_leaves_unused_partitions(dev):
    """Partitions at or past a sequence's context end are not written (the
    workspace keeps what it held), as in the matrix form."""
    import torch
    lens = [600, 17, 0, 1536]
    batch = W.make_batch(lens, 39)
    db = _device_batch(batch, dev, partition_size=512)
    pa, pm, ps = db.workspace
    for t in (pa, pm, ps):
        t.fill_(12345.0)
    _vector_pass(db)
    torch.cuda.synchronize()
    pm_h = pm.cpu().numpy()
    for s, n in enumerate(lens):
        used = -(-n // 512)
        assert (pm_h[s, :, used:] == 12345.0).all(), f"sequence {s}: unused partition written"
        assert np.isfinite(pm_h[s, :, :used]).all() and (pm_h[s, :, :used] != 12345.0).all()


def test_vector_rejects_other_groupings(dev):
    """Only 4 query heads per K/V head: other groupings are refused before any
    launch with TV_ERR_UNSUPPORTED."""
    import paged_kv_cache_tv_amd as tv
    from paged_kv_cache_tv_amd.step import DeviceBatch
    batch = W.make_batch([37, 300], 40, num_q_heads=16, num_kv_heads=8)
    db = DeviceBatch(batch, dev)
    db.fill()
    with pytest.raises(tv.TvError, match="UNSUPPORTED|unsupported"):
        _vector_pass(db)
