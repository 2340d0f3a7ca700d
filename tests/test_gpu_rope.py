"""Rotary position embedding on the GPU (tv_rope, tv_cache_write_rope) against
the CPU oracle, through the C-ABI.

The kernel computes each rotated value in fp32 from an exactly reduced angle
and rounds it to bf16; the oracle computes it in fp64.  The kernel's fp32
value is within eps = (|a| + |b|) * 2^-20 of the exact one for the pair
(a, b) it comes from: a few ulp of the reduced angle (|angle error| <= 2^-21),
one ulp each for cos and sin, and two roundings in the multiply-adds.  So the
GPU's bf16 value must lie between the oracle's roundings of v - eps and of
v + eps.  Those are the same bits (bit-exact) unless v lies within eps of a
bf16 rounding boundary; the tests also report how often that happened.
"""

import numpy as np
import pytest

import oracle as O
from paged_kv_cache_tv_amd import workloads as W

pytestmark = pytest.mark.gpu

D = 64


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


def _pair_mag(x, style):
    """|a| + |b| of the pair each element of x [T, H, D] belongs to."""
    f = np.abs(W.bf16_bits_to_float32(x).astype(np.float64))
    m = np.empty_like(f)
    if style == 0:
        s = f[..., 0::2] + f[..., 1::2]
        m[..., 0::2] = s
        m[..., 1::2] = s
    else:
        h = f.shape[-1] // 2
        s = f[..., :h] + f[..., h:]
        m[..., :h] = s
        m[..., h:] = s
    return m


def _check_rotated(orc, got_bits, x, positions, inv_freq, style, what):
    exact, rne = orc.rope(x, positions, inv_freq, style)
    eps = _pair_mag(x, style) * 2.0 ** -20
    lo = orc.bf16_round(exact - eps)
    hi = orc.bf16_round(exact + eps)
    val = W.bf16_bits_to_float32(got_bits)
    ok = (W.bf16_bits_to_float32(lo) <= val) & (val <= W.bf16_bits_to_float32(hi))
    near = int((lo != hi).sum())
    differ = int((got_bits != rne).sum())
    print(f"{what}: {got_bits.size} values, {near} within eps of a rounding boundary, "
          f"{differ} differ from the oracle's rounding", flush=True)
    assert ok.all(), f"{what}: {int((~ok).sum())} values outside the fp32 error bound"
    assert differ <= near


@pytest.mark.parametrize("style", [0, 1])
def test_rope_in_place(dev, oracle_lib, style):
    import torch
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(80 + style)
    T, H = 300, 32
    x = W.round_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    pos = np.concatenate([[0, 1, 2, 15, 16, 4095, 65535, 131071, 131072, -7],
                          rng.integers(0, 140000, T - 10)]).astype(np.int32)
    f = W.rope_inv_freq(D, 500000.0)
    xd = _to_dev(x, dev)
    tv.rope(xd, _to_dev(pos, dev), _to_dev(f, dev), style)
    torch.cuda.synchronize()
    got = xd.cpu().numpy().view(np.uint16)
    _check_rotated(oracle_lib, got, x, pos, f, style, f"tv_rope style {style}")
    # Position 0 leaves the row untouched, bit for bit.
    assert np.array_equal(got[0], x[0])


@pytest.mark.parametrize("style,head_dim,heads", [(0, 64, 8), (1, 64, 8), (0, 128, 2),
                                                  (1, 16, 4), (1, 128, 1)])
def test_cache_write_rope(dev, oracle_lib, style, head_dim, heads):
    """K lands rotated (to the bound above), V bit-exact, skipped slots and
    every other element untouched."""
    import torch
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(90 + head_dim + style)
    NB, BS, T = 40, 16, 200
    k = W.round_to_bf16_bits(rng.standard_normal((T, heads, head_dim)).astype(np.float32))
    v = W.round_to_bf16_bits(rng.standard_normal((T, heads, head_dim)).astype(np.float32))
    slots = rng.choice(NB * BS, T, replace=False).astype(np.int64)
    slots[[3, 50, 199]] = [-1, NB * BS, -5]                 # skipped
    pos = rng.integers(0, 131072, T).astype(np.int32)
    f = W.rope_inv_freq(head_dim, 10000.0)
    kc, vc = tv.new_pools(NB, heads, head_dim, BS, dev, fill=W.BF16_NAN)
    tv.cache_write_rope(_to_dev(k, dev), _to_dev(v, dev), kc, vc, _to_dev(slots, dev),
                        _to_dev(pos, dev), _to_dev(f, dev), style)
    torch.cuda.synchronize()
    kc_h, vc_h = kc.cpu().numpy().view(np.uint16), vc.cpu().numpy().view(np.uint16)
    # V and the untouched elements: bit-exact against the oracle's plain write.
    kr, vr = O.Oracle.new_pools(NB, heads, head_dim, BS)
    _, krot = oracle_lib.rope(k, pos, f, style)
    oracle_lib.cache_write(krot, v, kr, vr, slots)
    assert np.array_equal(vc_h, vr), "V pool"
    live = (slots >= 0) & (slots < NB * BS)
    blk, off = slots[live] // BS, slots[live] % BS
    got_k = kc_h[blk, :, :, off, :].reshape(live.sum(), heads, head_dim)
    mask = np.ones(kc_h.shape, bool)
    mask[blk, :, :, off, :] = False
    assert np.array_equal(kc_h[mask], kr[mask]), "K elements outside the written slots"
    _check_rotated(oracle_lib, got_k, k[live], pos[live], f, style,
                   f"tv_cache_write_rope style {style} D {head_dim}")


def test_decode_with_rope_end_to_end(dev, oracle_lib):
    """A decode step with RoPE: q turned by tv_rope, every position's K written
    by tv_cache_write_rope, then the two-launch step; against the oracle's
    attention over its own rotated q and K."""
    import torch
    import paged_kv_cache_tv_amd as tv
    b = W.make_batch([1, 37, 300, 1025], 95)
    f = W.rope_inv_freq(D, 500000.0)
    fd = _to_dev(f, dev)
    kc, vc = tv.new_pools(b.num_blocks, b.num_kv_heads, D, b.block_size, dev, fill=W.BF16_NAN)
    kr, vr = O.Oracle.new_pools(b.num_blocks, b.num_kv_heads, D, b.block_size)
    for s in range(b.num_seqs):
        n = int(b.context_lens[s])
        k, v = b.logical_kv(s)
        pos = np.arange(n, dtype=np.int32)
        slots = b.block_tables[s][pos // b.block_size].astype(np.int64) * b.block_size + \
            pos % b.block_size
        tv.cache_write_rope(_to_dev(k, dev), _to_dev(v, dev), kc, vc, _to_dev(slots, dev),
                            _to_dev(pos, dev), fd, 0)
        _, krot = oracle_lib.rope(k, pos, f, 0)
        oracle_lib.cache_write(krot, v, kr, vr, slots)
    qpos = (b.context_lens - 1).astype(np.int32)
    qd = _to_dev(b.q, dev)
    tv.rope(qd, _to_dev(qpos, dev), fd, 0)
    _, qrot = oracle_lib.rope(b.q, qpos, f, 0)
    ws = tv.new_workspace(b.num_seqs, b.num_q_heads, D, b.max_context_len, 512, dev)
    out = torch.empty((b.num_seqs, b.num_q_heads, D), dtype=torch.float32, device=dev)
    bt, cl = _to_dev(b.block_tables, dev), _to_dev(b.context_lens, dev)
    tv.paged_attention_decode(*ws, qd, kc, vc, bt, cl, b.max_context_len, 512, b.scale)
    tv.paged_attention_reduce(out, *ws, cl, b.max_context_len, 512)
    torch.cuda.synchronize()
    ref = oracle_lib.paged_attention(qrot, kr, vr, b.block_tables, b.context_lens, b.scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    print(f"decode with RoPE: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    # A rotated value that rounds to the other bf16 neighbour moves a score by
    # at most 2^-8 |q||k| * scale; the decode bars hold with room to spare.
    assert err.max() <= 1e-3 and err.mean() <= 1e-4
