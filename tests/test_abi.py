"""The C interface on the CPU: libtv loads, exports every function include/tv.h
declares, and rejects bad arguments before launching anything.

Every call here fails host-side validation: arguments that would pass are
never given, so no kernel is launched (the pointers are not real device
memory)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tv.h")

TV_OK, TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED, TV_ERR_HIP, TV_ERR_ALIGNMENT = range(6)
BAD = 0x11          # a non-NULL, misaligned pointer: if a check were missed, the alignment check
                    # (last before launch) still refuses the call


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_tv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(tv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("tv_cache_write", "tv_paged_attention_decode", "tv_paged_attention_reduce",
              "tv_paged_attention_decode_append", "tv_paged_attention_decode_shared_append"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    for code in range(7):
        assert lib.tv_status_string(code)
    assert b"unknown" in lib.tv_status_string(99)


def test_num_partitions(lib):
    assert lib.tv_num_partitions(4096, 512) == 8
    assert lib.tv_num_partitions(4097, 512) == 9
    assert lib.tv_num_partitions(1, 512) == 1
    assert lib.tv_num_partitions(0, 512) == 0
    assert lib.tv_num_partitions(100, 0) == -1


def test_decode_step_form_host_cases(lib):
    """The forms decided without the device: rejected shapes, nothing to launch,
    one partition.  (Forms 2 and 3 read the device and are covered on the GPU.)"""
    f = lib.tv_paged_attention_decode_step_form
    assert f(64, 32, 8, 64, 16, 512, 512) == 1
    assert f(64, 32, 8, 64, 16, 37, 512) == 1
    assert f(0, 32, 8, 64, 16, 4096, 512) == 0
    assert f(64, 32, 8, 64, 16, 0, 512) == 0
    assert f(64, 32, 8, 128, 16, 4096, 512) == -1      # head_dim other than 64
    assert f(64, 32, 8, 64, 32, 4096, 512) == -1       # block size other than 16
    assert f(64, 30, 8, 64, 16, 4096, 512) == -1       # query heads not a multiple
    assert f(64, 32, 8, 64, 16, 4096, 500) == -1       # partition not whole blocks
    assert f(-1, 32, 8, 64, 16, 4096, 512) == -1
    assert f(64, 32, 8, 64, 16, -1, 512) == -1


def _cw(lib, T=4, hkv=8, d=64, bs=16, nb=8, ptrs=(BAD,) * 5):
    return lib.tv_cache_write(*ptrs, T, hkv, d, bs, nb, None)


def test_cache_write_validation(lib):
    assert _cw(lib, T=-1) == TV_ERR_SHAPE
    assert _cw(lib, hkv=0) == TV_ERR_SHAPE
    assert _cw(lib, bs=0) == TV_ERR_SHAPE
    assert _cw(lib, nb=0) == TV_ERR_SHAPE
    assert _cw(lib, T=0, ptrs=(None,) * 5) == TV_OK          # no-op, nothing launched
    assert _cw(lib, ptrs=(None, BAD, BAD, BAD, BAD)) == TV_ERR_NULL
    assert _cw(lib, ptrs=(BAD, BAD, BAD, BAD, None)) == TV_ERR_NULL
    assert _cw(lib, d=60) == TV_ERR_UNSUPPORTED
    assert _cw(lib, T=4 * 0xffffff + 1) == TV_ERR_UNSUPPORTED    # launch grid
    assert _cw(lib, T=4 * 0xffffff) == TV_ERR_ALIGNMENT
    assert _cw(lib) == TV_ERR_ALIGNMENT


def _dec(lib, S=2, hq=32, hkv=8, d=64, bs=16, mb=4, nb=8, mctx=64, part=32, scale=0.125,
         ptrs=(BAD,) * 8):
    return lib.tv_paged_attention_decode(*ptrs, S, hq, hkv, d, bs, mb, nb, mctx, part, scale, None)


def test_decode_validation(lib):
    assert _dec(lib, S=-1) == TV_ERR_SHAPE
    assert _dec(lib, hq=30) == TV_ERR_SHAPE                  # not a multiple of hkv
    assert _dec(lib, part=24) == TV_ERR_SHAPE                # not a multiple of the block size
    assert _dec(lib, part=0) == TV_ERR_SHAPE
    assert _dec(lib, mctx=65) == TV_ERR_SHAPE                # beyond max_blocks * block_size
    assert _dec(lib, mctx=-1) == TV_ERR_SHAPE
    assert _dec(lib, scale=0.0) == TV_ERR_SHAPE
    assert _dec(lib, scale=float("nan")) == TV_ERR_SHAPE
    assert _dec(lib, scale=float("inf")) == TV_ERR_SHAPE
    assert _dec(lib, d=128) == TV_ERR_UNSUPPORTED
    assert _dec(lib, bs=32, part=64, mctx=64) == TV_ERR_UNSUPPORTED
    assert _dec(lib, hq=8 * 17) == TV_ERR_UNSUPPORTED       # group of 17
    # launch grid of 8 heads x S x 2 partitions: 2^24 - 1 workgroups is the limit
    assert _dec(lib, S=(1 << 20)) == TV_ERR_UNSUPPORTED    # 2^24
    assert _dec(lib, S=(1 << 20) - 1) == TV_ERR_ALIGNMENT   # 2^24 - 16 passes the grid check
    assert _dec(lib, S=0) == TV_OK
    assert _dec(lib, mctx=0) == TV_OK
    assert _dec(lib, ptrs=(BAD,) * 7 + (None,)) == TV_ERR_NULL
    assert _dec(lib) == TV_ERR_ALIGNMENT


ALIGNED = 0x1000     # a non-NULL, aligned fake address: only ever paired with an argument
                     # that fails validation, so nothing is launched


def _app(lib, S=2, hq=32, hkv=8, d=64, bs=16, mb=4, nb=8, mctx=64, part=32, scale=0.125,
         ptrs=(BAD,) * 11):
    return lib.tv_paged_attention_decode_append(*ptrs, S, hq, hkv, d, bs, mb, nb, mctx, part,
                                                scale, None)


def test_decode_append_validation(lib):
    assert _app(lib, S=-1) == TV_ERR_SHAPE
    assert _app(lib, hq=30) == TV_ERR_SHAPE
    assert _app(lib, part=24) == TV_ERR_SHAPE
    assert _app(lib, mctx=65) == TV_ERR_SHAPE
    assert _app(lib, scale=-1.0) == TV_ERR_SHAPE
    assert _app(lib, d=128) == TV_ERR_UNSUPPORTED
    assert _app(lib, S=0) == TV_OK
    assert _app(lib, mctx=0) == TV_OK
    assert _app(lib) == TV_ERR_ALIGNMENT
    # The partition-pass arguments pass their checks; the append ones do not.
    for i in (4, 5, 6):                                   # k_new, v_new, slot_mapping
        ptrs = [ALIGNED] * 11
        ptrs[i] = None
        assert _app(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL
    ptrs = [ALIGNED] * 11
    ptrs[4] = BAD                                         # k_new misaligned
    assert _app(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT
    ptrs = [ALIGNED] * 11
    ptrs[6] = 0x1004                                      # slot_mapping not 8-byte aligned
    assert _app(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT
    for bad_v in (0x1002, 0x1004, 0x1008):                # v_new: loaded 4 bytes per lane,
        ptrs = [ALIGNED] * 11                             # required 16-byte aligned like k_new
        ptrs[5] = bad_v
        assert _app(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT


def _vec(lib, S=2, hq=32, hkv=8, d=64, bs=16, mb=4, nb=8, mctx=64, part=32, scale=0.125,
         ptrs=(BAD,) * 8):
    return lib.tv_paged_attention_decode_vector(*ptrs, S, hq, hkv, d, bs, mb, nb, mctx, part,
                                                scale, None)


def test_decode_vector_validation(lib):
    """The vector-ALU form checks its arguments as tv_paged_attention_decode
    does, then refuses every grouping other than 4 query heads per K/V head
    (empty batches included) before any launch."""
    assert _vec(lib, S=-1) == TV_ERR_SHAPE
    assert _vec(lib, hq=30) == TV_ERR_SHAPE
    assert _vec(lib, part=24) == TV_ERR_SHAPE
    assert _vec(lib, mctx=65) == TV_ERR_SHAPE
    assert _vec(lib, scale=0.0) == TV_ERR_SHAPE
    assert _vec(lib, d=128) == TV_ERR_UNSUPPORTED
    assert _vec(lib, S=0) == TV_OK
    assert _vec(lib, mctx=0) == TV_OK
    assert _vec(lib, ptrs=(BAD,) * 7 + (None,)) == TV_ERR_NULL
    assert _vec(lib) == TV_ERR_ALIGNMENT
    ptrs = [ALIGNED] * 8
    ptrs[0] = 0x1004                                      # part_acc: 16-byte stores
    assert _vec(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT
    for hq, hkv in ((16, 8), (8, 8), (64, 8), (12, 4)):
        assert _vec(lib, hq=hq, hkv=hkv, ptrs=(ALIGNED,) * 8) == TV_ERR_UNSUPPORTED
        assert _vec(lib, S=0, hq=hq, hkv=hkv) == TV_ERR_UNSUPPORTED


def test_partition_pass_part_acc_alignment(lib):
    """The partition pass writes part_acc with 16-byte stores: every call that
    takes the workspace refuses a part_acc that is only 4-byte aligned."""
    dec = [ALIGNED] * 8
    dec[0] = 0x1004
    assert _dec(lib, ptrs=tuple(dec)) == TV_ERR_ALIGNMENT
    app = [ALIGNED] * 11
    app[0] = 0x1004
    assert _app(lib, ptrs=tuple(app)) == TV_ERR_ALIGNMENT
    shd = [ALIGNED] * 10
    shd[0] = 0x1004
    assert _shd(lib, ptrs=tuple(shd)) == TV_ERR_ALIGNMENT
    sha = [ALIGNED] * 12 + [None]
    sha[0] = 0x1004
    assert _sha(lib, ptrs=tuple(sha)) == TV_ERR_ALIGNMENT


def _stp(lib, S=2, hq=32, hkv=8, d=64, mctx=64, part=32, ptrs=(BAD,) * 12):
    return lib.tv_paged_attention_decode_step(*ptrs, S, hq, hkv, d, 16, 4, 8, mctx, part,
                                              0.125, None)


def test_decode_step_validation(lib):
    """tv_paged_attention_decode_step: every argument error is found before a
    launch; the workspace is needed only with more than one partition.  Each
    case below keeps at least one argument that fails, so nothing launches."""
    assert _stp(lib, S=-1) == TV_ERR_SHAPE
    assert _stp(lib, part=24) == TV_ERR_SHAPE
    assert _stp(lib, d=128) == TV_ERR_UNSUPPORTED
    assert _stp(lib, S=0) == TV_OK
    assert _stp(lib) == TV_ERR_ALIGNMENT
    # max_context_len == 0: the merge alone zeroes out; out is still checked.
    assert _stp(lib, mctx=0) == TV_ERR_ALIGNMENT
    assert _stp(lib, mctx=0, ptrs=(None,) + (BAD,) * 11) == TV_ERR_NULL
    # One partition (64 <= 64): no workspace needed.
    one = [ALIGNED] * 12
    one[1:4] = [None] * 3
    one[0] = BAD                                          # out misaligned
    assert _stp(lib, part=64, ptrs=tuple(one)) == TV_ERR_ALIGNMENT
    one[0] = ALIGNED
    one[5] = None                                         # k_new
    assert _stp(lib, part=64, ptrs=tuple(one)) == TV_ERR_NULL
    one[5] = ALIGNED
    one[7] = 0x1004                                       # slot_mapping not 8-byte aligned
    assert _stp(lib, part=64, ptrs=tuple(one)) == TV_ERR_ALIGNMENT
    assert _stp(lib, part=64, S=1 << 19, ptrs=tuple(one)) == TV_ERR_UNSUPPORTED   # 2^24 rows
    # Two partitions: the workspace is required, part_acc 16-byte aligned.
    two = [ALIGNED] * 12
    two[1] = None
    assert _stp(lib, ptrs=tuple(two)) == TV_ERR_NULL
    two[1] = 0x1004
    assert _stp(lib, ptrs=tuple(two)) == TV_ERR_ALIGNMENT
    two[1] = ALIGNED
    two[0] = None                                         # out
    assert _stp(lib, ptrs=tuple(two)) == TV_ERR_NULL
    two[0] = ALIGNED
    two[6] = 0x1004                                       # v_new not 16-byte aligned
    assert _stp(lib, ptrs=tuple(two)) == TV_ERR_ALIGNMENT


def _shd(lib, S=2, hq=32, hkv=8, gs=4, mctx=64, part=32, ptrs=(BAD,) * 10):
    return lib.tv_paged_attention_decode_shared(*ptrs, gs, S, hq, hkv, 64, 16, 4, 8, mctx, part,
                                                0.125, None)


def test_decode_shared_validation(lib):
    assert _shd(lib, S=-1) == TV_ERR_SHAPE
    assert _shd(lib, gs=0) == TV_ERR_SHAPE
    assert _shd(lib, gs=5) == TV_ERR_UNSUPPORTED         # 5 sequences x 4 heads > 16 columns
    assert _shd(lib, hq=64, gs=3) == TV_ERR_UNSUPPORTED  # 3 x 8 heads
    assert _shd(lib, S=0) == TV_OK
    assert _shd(lib, mctx=0) == TV_OK
    assert _shd(lib) == TV_ERR_ALIGNMENT                  # the decode arguments are checked first
    ptrs = [ALIGNED] * 10
    ptrs[8] = None
    assert _shd(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL
    ptrs[8] = 0x1002
    assert _shd(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT
    ptrs = [ALIGNED] * 10
    ptrs[9] = 0x1002                                      # group_order misaligned (NULL is allowed)
    assert _shd(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT


def _sha(lib, S=2, hq=32, hkv=8, gs=4, mctx=64, part=32, ptrs=(BAD,) * 13):
    return lib.tv_paged_attention_decode_shared_append(*ptrs, gs, S, hq, hkv, 64, 16, 4, 8, mctx,
                                                       part, 0.125, None)


def test_decode_shared_append_validation(lib):
    assert _sha(lib, S=-1) == TV_ERR_SHAPE
    assert _sha(lib, gs=0) == TV_ERR_SHAPE
    assert _sha(lib, gs=5) == TV_ERR_UNSUPPORTED
    assert _sha(lib, part=24) == TV_ERR_SHAPE
    assert _sha(lib, S=0) == TV_OK
    assert _sha(lib, mctx=0) == TV_OK
    assert _sha(lib) == TV_ERR_ALIGNMENT                  # the decode arguments are checked first
    # The partition-pass arguments pass their checks; each of the shared and
    # append ones is then refused when NULL or misaligned (nothing launches).
    for i in (4, 5, 6, 11):                               # k_new, v_new, slot_mapping, shared_len
        ptrs = [ALIGNED] * 12 + [None]                    # group_order NULL: consecutive groups
        ptrs[i] = None
        assert _sha(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL
        ptrs[i] = BAD
        assert _sha(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT
    ptrs = [ALIGNED] * 12 + [BAD]                         # group_order misaligned
    assert _sha(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT


def _pre(lib, S=2, hq=32, hkv=8, d=64, bs=16, mb=4, nb=8, mq=40, mctx=64, scale=0.125,
         ptrs=(BAD,) * 7):
    return lib.tv_paged_attention_prefill(*ptrs, S, hq, hkv, d, bs, mb, nb, mq, mctx, scale, None)


def test_prefill_validation(lib):
    assert _pre(lib, S=-1) == TV_ERR_SHAPE
    assert _pre(lib, hq=30) == TV_ERR_SHAPE
    assert _pre(lib, mq=-1) == TV_ERR_SHAPE
    assert _pre(lib, mctx=65) == TV_ERR_SHAPE
    assert _pre(lib, scale=0.0) == TV_ERR_SHAPE
    assert _pre(lib, scale=float("inf")) == TV_ERR_SHAPE
    assert _pre(lib, d=128) == TV_ERR_UNSUPPORTED
    assert _pre(lib, bs=32, mb=2) == TV_ERR_UNSUPPORTED
    assert _pre(lib, hq=24) == TV_ERR_UNSUPPORTED          # group 3
    assert _pre(lib, hq=256) == TV_ERR_UNSUPPORTED         # group 32
    assert _pre(lib, S=1 << 20, mq=64) == TV_ERR_UNSUPPORTED   # 2^23 workgroups
    assert _pre(lib, S=(1 << 20) - 1, mq=64) == TV_ERR_ALIGNMENT
    assert _pre(lib, S=0) == TV_OK
    assert _pre(lib, mq=0) == TV_OK
    assert _pre(lib) == TV_ERR_ALIGNMENT
    for i in range(7):
        ptrs = [ALIGNED] * 7
        ptrs[i] = None
        assert _pre(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL, i
    for i, bad in ((0, 0x1004), (1, 0x1008), (2, 0x1002), (3, 0x1008)):   # out, q, query_start, k_cache
        ptrs = [ALIGNED] * 7
        ptrs[i] = bad
        assert _pre(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT, i


def _cwr(lib, T=4, hkv=8, d=64, bs=16, nb=8, style=0, ptrs=(BAD,) * 7):
    return lib.tv_cache_write_rope(*ptrs, T, hkv, d, bs, nb, style, None)


def _rope(lib, T=4, h=8, d=64, style=0, ptrs=(BAD,) * 3):
    return lib.tv_rope(*ptrs, T, h, d, style, None)


def test_rope_validation(lib):
    assert _cwr(lib, T=-1) == TV_ERR_SHAPE
    assert _cwr(lib, style=2) == TV_ERR_SHAPE
    assert _cwr(lib, nb=0) == TV_ERR_SHAPE
    assert _cwr(lib, T=0) == TV_OK
    assert _cwr(lib, d=12) == TV_ERR_UNSUPPORTED
    assert _cwr(lib, d=136) == TV_ERR_UNSUPPORTED
    assert _cwr(lib) == TV_ERR_ALIGNMENT
    for i in range(7):
        ptrs = [ALIGNED] * 7
        ptrs[i] = None
        assert _cwr(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL, i
    for i, bad in ((0, 0x1008), (4, 0x1004), (5, 0x1002), (6, 0x1001)):   # k, slots, positions, inv_freq
        ptrs = [ALIGNED] * 7
        ptrs[i] = bad
        assert _cwr(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT, i
    assert _rope(lib, T=-1) == TV_ERR_SHAPE
    assert _rope(lib, style=-1) == TV_ERR_SHAPE
    assert _rope(lib, T=0) == TV_OK
    assert _rope(lib, d=20) == TV_ERR_UNSUPPORTED
    assert _rope(lib, T=4 * 0xffffff + 1) == TV_ERR_UNSUPPORTED
    assert _rope(lib, T=4 * 0xffffff) == TV_ERR_ALIGNMENT
    assert _rope(lib) == TV_ERR_ALIGNMENT
    for i in range(3):
        ptrs = [ALIGNED] * 3
        ptrs[i] = None
        assert _rope(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL, i
    ptrs = [0x1008, ALIGNED, ALIGNED]
    assert _rope(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT


def _copy(lib, n=3, hkv=8, d=64, bs=16, nb=8, ptrs=(BAD,) * 3):
    return lib.tv_copy_blocks(*ptrs, n, hkv, d, bs, nb, None)


def test_copy_blocks_validation(lib):
    assert _copy(lib, n=-1) == TV_ERR_SHAPE
    assert _copy(lib, hkv=0) == TV_ERR_SHAPE
    assert _copy(lib, nb=0) == TV_ERR_SHAPE
    assert _copy(lib, hkv=1, d=3, bs=1) == TV_ERR_UNSUPPORTED    # 3 values per block
    assert _copy(lib, n=1 << 24) == TV_ERR_UNSUPPORTED           # launch grid
    assert _copy(lib, n=(1 << 24) - 1) == TV_ERR_ALIGNMENT
    assert _copy(lib, n=0, ptrs=(None,) * 3) == TV_OK           # no-op
    assert _copy(lib, ptrs=(BAD, BAD, None)) == TV_ERR_NULL
    assert _copy(lib) == TV_ERR_ALIGNMENT


def _red(lib, S=2, hq=32, d=64, mctx=64, part=32, ptrs=(BAD,) * 5):
    return lib.tv_paged_attention_reduce(*ptrs, S, hq, d, mctx, part, None)


def test_reduce_validation(lib):
    assert _red(lib, S=-1) == TV_ERR_SHAPE
    assert _red(lib, part=0) == TV_ERR_SHAPE
    assert _red(lib, mctx=-3) == TV_ERR_SHAPE
    assert _red(lib, d=32) == TV_ERR_UNSUPPORTED
    assert _red(lib, S=1 << 19, hq=32) == TV_ERR_UNSUPPORTED          # 2^24 rows
    assert _red(lib, S=(1 << 19) - 1, hq=32) == TV_ERR_ALIGNMENT     # just under the limit
    assert _red(lib, S=0) == TV_OK
    assert _red(lib, ptrs=(None,) + (BAD,) * 4) == TV_ERR_NULL
    assert _red(lib, ptrs=(BAD, None, BAD, BAD, BAD)) == TV_ERR_NULL
    assert _red(lib) == TV_ERR_ALIGNMENT


def test_stream_read_validation(lib):
    f = lib.tv_stream_read
    assert f(BAD, -16, BAD, None) == TV_ERR_SHAPE
    assert f(BAD, 24, BAD, None) == TV_ERR_UNSUPPORTED               # not a multiple of 16
    assert f(None, 0, None, None) == TV_OK                            # no-op
    assert f(None, 16, BAD, None) == TV_ERR_NULL
    assert f(BAD, 16, None, None) == TV_ERR_NULL
    assert f(BAD, 8192 * 0xffffff + 16, BAD, None) == TV_ERR_UNSUPPORTED   # 2^24 chunks
    assert f(BAD, 8192 * 0xffffff, BAD, None) == TV_ERR_ALIGNMENT
    assert f(ALIGNED, 16, ALIGNED + 2, None) == TV_ERR_ALIGNMENT
    assert f(ALIGNED + 8, 16, ALIGNED, None) == TV_ERR_ALIGNMENT


def test_binding_refuses_host_tensors():
    import torch
    import paged_kv_cache_tv_amd as tv
    x = torch.zeros((1, 8, 64), dtype=torch.int16)
    with pytest.raises(ValueError):
        tv.cache_write(x, x, torch.zeros((2, 8, 8, 16, 8), dtype=torch.int16),
                       torch.zeros((2, 8, 64, 16), dtype=torch.int16),
                       torch.zeros(1, dtype=torch.int64))


def test_decode_step_noalloc_refuses_oversized_workspace(lib):
    """tv_paged_attention_decode_step_noalloc: a workspace above the fixed
    scratch array (16 MiB) is refused before anything touches the GPU; the
    refusal needs no device, so it runs here.  Below the limit the call
    checks its arguments as tv_paged_attention_decode_step does."""
    TV_ERR_SCRATCH = 7
    fn = lib.tv_paged_attention_decode_step_noalloc

    def call(S, mctx, part, ptrs=(ALIGNED,) * 9, hq=32, d=64):
        return fn(*ptrs, S, hq, 8, d, 16, max(1, mctx // 16), 1 << 20, mctx, part, 0.125, None)

    # 64 x 32 x 248 x 66 x 4 B = 16.76 MB > 16 MiB; 64 x 32 x 8 x 66 x 4 B = 4.3 MB fits.
    assert call(64, 248 * 16, 16) == TV_ERR_SCRATCH
    assert call(1 << 20, 1 << 20, 512) == TV_ERR_SCRATCH       # no overflow in the size
    assert call((1 << 31) - 1, (1 << 31) - 1, 16, hq=(1 << 31) - 1) == TV_ERR_SCRATCH
    # One partition needs no workspace: no limit; the step's own checks then
    # report the misaligned pointers (nothing launches).
    assert call(1 << 20, 512, 512, ptrs=(BAD,) * 9) == TV_ERR_ALIGNMENT
    assert call(-1, 4096, 512) == TV_ERR_SHAPE
    assert call(0, 4096, 512) == TV_OK
    assert lib.tv_status_string(TV_ERR_SCRATCH).startswith(b"TV_ERR_SCRATCH")


def _shs(lib, S=2, hq=32, hkv=8, gs=4, mctx=64, part=32, ptrs=(BAD,) * 14):
    return lib.tv_paged_attention_decode_shared_step(*ptrs, gs, S, hq, hkv, 64, 16, 4, 8, mctx,
                                                     part, 0.125, None)


def test_decode_shared_step_validation(lib):
    """tv_paged_attention_decode_shared_step: argument errors before any launch
    (pointer order: out, part_acc, part_max, part_sum, q, k_new, v_new,
    slot_mapping, k_cache, v_cache, block_tables, context_lens, shared_len,
    group_order)."""
    assert _shs(lib, S=-1) == TV_ERR_SHAPE
    assert _shs(lib, gs=0) == TV_ERR_SHAPE
    assert _shs(lib, gs=5) == TV_ERR_UNSUPPORTED          # 5 x 4 columns > 16
    assert _shs(lib, part=24) == TV_ERR_SHAPE
    assert _shs(lib, S=0) == TV_OK
    assert _shs(lib) == TV_ERR_ALIGNMENT                  # the decode arguments first
    for i in (0, 5, 6, 7, 12):                            # out, k_new, v_new, slot_mapping, shared_len
        ptrs = [ALIGNED] * 13 + [None]
        ptrs[i] = None
        assert _shs(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL, i
        ptrs[i] = BAD
        assert _shs(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT, i
    ptrs = [ALIGNED] * 13 + [BAD]                         # group_order misaligned
    assert _shs(lib, ptrs=tuple(ptrs)) == TV_ERR_ALIGNMENT
    ptrs = [ALIGNED] * 13 + [None]
    ptrs[1] = None                                        # the workspace is always required
    assert _shs(lib, ptrs=tuple(ptrs)) == TV_ERR_NULL
    # max_context_len == 0: the merge alone zeroes out; out is still checked.
    assert _shs(lib, mctx=0, ptrs=(None,) + (BAD,) * 13) == TV_ERR_NULL


def test_decode_shared_step_form_host_cases(lib):
    f = lib.tv_paged_attention_decode_shared_step_form
    assert f(0, 32, 8, 64, 16, 4096, 512, 4, 0) == 0
    assert f(64, 32, 8, 64, 16, 0, 512, 4, 0) == 0
    assert f(64, 32, 8, 64, 16, 4096, 512, 5, 0) == -1   # 5 x 4 columns > 16
    assert f(64, 32, 8, 64, 16, 4096, 512, 0, 0) == -1
    assert f(64, 32, 8, 128, 16, 4096, 512, 4, 0) == -1
    assert f(64, 32, 8, 64, 16, 4096, 500, 4, 0) == -1
    assert f(-1, 32, 8, 64, 16, 4096, 512, 4, 0) == -1
