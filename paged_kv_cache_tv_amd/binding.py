"""Python binding of libtv (ctypes).  Argument marshalling only.

Every function takes torch tensors that live on the current HIP device,
checks dtype/shape/contiguity, and passes raw pointers and sizes to the C entry
point of the same name in ``include/tv.h``.  No step of the computation runs
here, and there is no fallback: if ``libtv.so`` is missing or a call fails, a
``TvError`` is raised.

bf16 tensors may be ``torch.bfloat16`` or any 2-byte integer dtype holding the
bit patterns.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtv.so")

TV_OK = 0
STATUS_NAMES = {0: "TV_OK", 1: "TV_ERR_NULL", 2: "TV_ERR_SHAPE", 3: "TV_ERR_UNSUPPORTED",
                4: "TV_ERR_HIP", 5: "TV_ERR_ALIGNMENT", 6: "TV_ERR_NO_BLOCKS",
                7: "TV_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024     # TV_NOALLOC_SCRATCH_BYTES


class TvError(RuntimeError):
    """A libtv call returned a status other than TV_OK (or the library is missing)."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {STATUS_NAMES.get(status, status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtv and declare its C signatures."""
    if not os.path.exists(path):
        raise TvError("load_library", -1) from FileNotFoundError(
            f"{path} is not built; run `python -m paged_kv_cache_tv_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.tv_status_string.restype = ctypes.c_char_p
    lib.tv_status_string.argtypes = [ctypes.c_int]
    lib.tv_num_partitions.restype = i32
    lib.tv_num_partitions.argtypes = [i32, i32]
    lib.tv_paged_attention_decode_step_form.restype = i32
    lib.tv_paged_attention_decode_step_form.argtypes = [i32] * 7
    lib.tv_paged_attention_decode_shared_step_form.restype = i32
    lib.tv_paged_attention_decode_shared_step_form.argtypes = [i32] * 9
    lib.tv_cache_write.restype = ctypes.c_int
    lib.tv_cache_write.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, vp]
    lib.tv_paged_attention_decode.restype = ctypes.c_int
    lib.tv_paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                              i32, i32, i64, i32, i32, f32, vp]
    lib.tv_paged_attention_decode_vector.restype = ctypes.c_int
    lib.tv_paged_attention_decode_vector.argtypes = lib.tv_paged_attention_decode.argtypes
    lib.tv_paged_attention_decode_append.restype = ctypes.c_int
    lib.tv_paged_attention_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                     i32, i32, i32, i32, i32, i32, i64, i32, i32,
                                                     f32, vp]
    lib.tv_paged_attention_decode_step.restype = ctypes.c_int
    lib.tv_paged_attention_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                   vp, i32, i32, i32, i32, i32, i32, i64, i32,
                                                   i32, f32, vp]
    lib.tv_paged_attention_decode_step_noalloc.restype = ctypes.c_int
    lib.tv_paged_attention_decode_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                           i32, i32, i32, i32, i32, i64, i32, i32,
                                                           f32, vp]
    lib.tv_paged_attention_decode_shared.restype = ctypes.c_int
    lib.tv_paged_attention_decode_shared.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                     i32, i32, i32, i32, i32, i32, i64, i32, i32,
                                                     ctypes.c_float, vp]
    lib.tv_paged_attention_decode_shared_append.restype = ctypes.c_int
    lib.tv_paged_attention_decode_shared_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                            vp, vp, vp, i32, i32, i32, i32, i32,
                                                            i32, i32, i64, i32, i32, ctypes.c_float,
                                                            vp]
    lib.tv_paged_attention_decode_shared_step.restype = ctypes.c_int
    lib.tv_paged_attention_decode_shared_step.argtypes = [vp] * 14 + [i32] * 7 + [i64, i32, i32,
                                                                                ctypes.c_float, vp]
    lib.tv_paged_attention_reduce.restype = ctypes.c_int
    lib.tv_paged_attention_reduce.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.tv_paged_attention_prefill.restype = ctypes.c_int
    lib.tv_paged_attention_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                               i32, i32, i64, i32, i32, ctypes.c_float, vp]
    lib.tv_cache_write_rope.restype = ctypes.c_int
    lib.tv_cache_write_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, i32,
                                        vp]
    lib.tv_rope.restype = ctypes.c_int
    lib.tv_rope.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp]
    lib.tv_copy_blocks.restype = ctypes.c_int
    lib.tv_copy_blocks.argtypes = [vp, vp, vp, i64, i32, i32, i32, i64, vp]
    lib.tv_stream_read.restype = ctypes.c_int
    lib.tv_stream_read.argtypes = [vp, i64, vp, vp]
    i32p, i64p = ctypes.POINTER(i32), ctypes.POINTER(i64)
    lib.tv_bm_create.restype = ctypes.c_int
    lib.tv_bm_create.argtypes = [i32, i32, i32, i32, ctypes.POINTER(vp)]
    lib.tv_bm_destroy.restype = None
    lib.tv_bm_destroy.argtypes = [vp]
    for name in ("tv_bm_num_free",):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [vp]
    for name in ("tv_bm_refcount", "tv_bm_length"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [vp, i32]
    lib.tv_bm_add_sequence.restype = ctypes.c_int
    lib.tv_bm_add_sequence.argtypes = [vp, i32, i32]
    lib.tv_bm_fork.restype = ctypes.c_int
    lib.tv_bm_fork.argtypes = [vp, i32, i32]
    lib.tv_bm_append_slot.restype = ctypes.c_int
    lib.tv_bm_append_slot.argtypes = [vp, i32, i64p, i64p, i64p]
    lib.tv_bm_free_sequence.restype = ctypes.c_int
    lib.tv_bm_free_sequence.argtypes = [vp, i32]
    lib.tv_bm_block_table.restype = ctypes.c_int
    lib.tv_bm_block_table.argtypes = [vp, i32, i32p, i32, i32p]
    lib.tv_bm_slots.restype = ctypes.c_int
    lib.tv_bm_slots.argtypes = [vp, i32, i32, i32, i64p]
    lib.tv_bm_prepare_decode.restype = ctypes.c_int
    lib.tv_bm_prepare_decode.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, i32p]
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _check(func: str, status: int) -> None:
    if status != TV_OK:
        raise TvError(func, status)


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, *, itemsize=None, dtype=None, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def num_partitions(max_context_len: int, partition_size: int) -> int:
    return int(lib().tv_num_partitions(int(max_context_len), int(partition_size)))


DECODE_STEP_FORMS = {0: "nothing launched", 1: "one launch, one partition",
                     2: "one launch, one workgroup per (sequence, K/V head)",
                     3: "two launches through the workspace"}


def decode_step_form(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     block_size: int, max_context_len: int, partition_size: int) -> int:
    """Form code of tv_paged_attention_decode_step for these shapes on the
    current device (0-3, or -1 for shapes the step rejects)."""
    return int(lib().tv_paged_attention_decode_step_form(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len), int(partition_size)))


def decode_shared_step_form(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            block_size: int, max_context_len: int, partition_size: int,
                            group_size: int, has_group_order: bool = False) -> int:
    """Form code of tv_paged_attention_decode_shared_step for these shapes on
    the current device (0 nothing, 1 one launch, 2 two launches, -1 rejected)."""
    return int(lib().tv_paged_attention_decode_shared_step_form(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len), int(partition_size), int(group_size), int(bool(has_group_order))))


def _pool_dims(k_cache, v_cache):
    """(NB, Hkv, BS, D) of a K pool [NB, Hkv, D/8, BS, 8] and V pool [NB, Hkv, D, BS]."""
    _need(k_cache, "k_cache", itemsize=2, ndim=5)
    _need(v_cache, "v_cache", itemsize=2, ndim=4)
    nb, hkv, dc, bs, x = k_cache.shape
    if x != 8:
        raise ValueError("k_cache must be [NB, Hkv, D/8, BS, 8]")
    d = dc * x
    if tuple(v_cache.shape) != (nb, hkv, d, bs):
        raise ValueError("v_cache must be [NB, Hkv, D, BS] matching k_cache [NB, Hkv, D/8, BS, 8]")
    return nb, hkv, bs, d


def new_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, device,
              fill: int = 0):
    """Allocate K and V pools (int16 bit patterns) in the library's layout."""
    import torch
    if head_dim % 8:
        raise ValueError("head_dim must be a multiple of 8")
    k = torch.full((num_blocks, num_kv_heads, head_dim // 8, block_size, 8), fill,
                   dtype=torch.int16, device=device)
    v = torch.full((num_blocks, num_kv_heads, head_dim, block_size), fill, dtype=torch.int16,
                   device=device)
    return k, v


def cache_write(k, v, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """tv_cache_write.  k, v: [T, Hkv, D]; k_cache: [NB, Hkv, D/8, BS, 8]; v_cache:
    [NB, Hkv, D, BS]; slot_mapping: int64 [T]."""
    import torch
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    T = slot_mapping.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d):
        raise ValueError("k and v must be [T, Hkv, D] with T = len(slot_mapping)")
    st = lib().tv_cache_write(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              slot_mapping.data_ptr(), T, hkv, d, bs, nb,
                              _stream_handle(stream, k_cache.device))
    _check("tv_cache_write", st)


def _decode_pass(name, part_acc, part_max, part_sum, q, k_cache, v_cache, block_tables,
                 context_lens, max_context_len, partition_size, scale, stream):
    import torch
    _need(q, "q", itemsize=2, ndim=3)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
        _need(t, n, dtype=torch.float32)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d:
        raise ValueError("cache shapes do not match q")
    P = num_partitions(max_context_len, partition_size)
    if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
            tuple(part_sum.shape) != (S, hq, P):
        raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    st = getattr(lib(), name)(
        part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr(), q.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        S, hq, hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), int(partition_size),
        float(scale), _stream_handle(stream, q.device))
    _check(name, st)


def paged_attention_decode(part_acc, part_max, part_sum, q, k_cache, v_cache, block_tables,
                           context_lens, max_context_len: int, partition_size: int,
                           scale: float, stream=None) -> None:
    """tv_paged_attention_decode.  q: [S, Hq, D]; block_tables: int32 [S, max_blocks];
    context_lens: int32 [S]; part_acc: float32 [S, Hq, P, D]; part_max/part_sum: [S, Hq, P]."""
    _decode_pass("tv_paged_attention_decode", part_acc, part_max, part_sum, q, k_cache, v_cache,
                 block_tables, context_lens, max_context_len, partition_size, scale, stream)


def paged_attention_decode_vector(part_acc, part_max, part_sum, q, k_cache, v_cache,
                                  block_tables, context_lens, max_context_len: int,
                                  partition_size: int, scale: float, stream=None) -> None:
    """tv_paged_attention_decode_vector: the same partition pass with the
    contractions on the vector ALUs (4 query heads per K/V head only).
    Arguments as for paged_attention_decode."""
    _decode_pass("tv_paged_attention_decode_vector", part_acc, part_max, part_sum, q, k_cache,
                 v_cache, block_tables, context_lens, max_context_len, partition_size, scale,
                 stream)


def cache_write_rope(k, v, k_cache, v_cache, slot_mapping, positions, inv_freq,
                     rope_style: int = 0, stream=None) -> None:
    """tv_cache_write_rope: tv_cache_write with K turned by the rotary embedding
    of positions (int32 [T]); inv_freq: float32 [D/2] on the device."""
    import torch
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(positions, "positions", dtype=torch.int32, ndim=1)
    _need(inv_freq, "inv_freq", dtype=torch.float32, ndim=1)
    T, hkv, d = k.shape
    nb, hkv2, bs, d2 = _pool_dims(k_cache, v_cache)
    if (hkv2, d2) != (hkv, d) or tuple(v.shape) != (T, hkv, d):
        raise ValueError("k, v and the cache must agree on [Hkv, D]")
    if slot_mapping.shape[0] != T or positions.shape[0] != T or inv_freq.shape[0] != d // 2:
        raise ValueError("slot_mapping, positions: [T]; inv_freq: [D/2]")
    st = lib().tv_cache_write_rope(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), slot_mapping.data_ptr(),
                                   positions.data_ptr(), inv_freq.data_ptr(), T, hkv, d, bs, nb,
                                   int(rope_style), _stream_handle(stream, k.device))
    _check("tv_cache_write_rope", st)


def rope(x, positions, inv_freq, rope_style: int = 0, stream=None) -> None:
    """tv_rope: turn x ([T, H, D] bf16) in place by the rotary embedding of positions."""
    import torch
    _need(x, "x", itemsize=2, ndim=3)
    _need(positions, "positions", dtype=torch.int32, ndim=1)
    _need(inv_freq, "inv_freq", dtype=torch.float32, ndim=1)
    T, h, d = x.shape
    if positions.shape[0] != T or inv_freq.shape[0] != d // 2:
        raise ValueError("positions: [T]; inv_freq: [D/2]")
    st = lib().tv_rope(x.data_ptr(), positions.data_ptr(), inv_freq.data_ptr(), T, h, d,
                       int(rope_style), _stream_handle(stream, x.device))
    _check("tv_rope", st)


def paged_attention_prefill(out, q, query_start, k_cache, v_cache, block_tables, context_lens,
                            max_query_len: int, max_context_len: int, scale: float,
                            stream=None) -> None:
    """tv_paged_attention_prefill.  q, out: [rows, Hq, D] (bf16 / float32);
    query_start: int32 [S + 1]; block_tables: int32 [S, max_blocks];
    context_lens: int32 [S]."""
    import torch
    _need(q, "q", itemsize=2, ndim=3)
    _need(out, "out", dtype=torch.float32, ndim=3)
    _need(query_start, "query_start", dtype=torch.int32, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    rows, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d or tuple(out.shape) != (rows, hq, d):
        raise ValueError("out, q and the cache must agree on [rows, Hq, D]")
    S = context_lens.shape[0]
    if query_start.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("query_start must have S + 1 entries and block_tables S rows")
    st = lib().tv_paged_attention_prefill(
        out.data_ptr(), q.data_ptr(), query_start.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), S, hq, hkv, d, bs,
        block_tables.shape[1], nb, int(max_query_len), int(max_context_len), float(scale),
        _stream_handle(stream, q.device))
    _check("tv_paged_attention_prefill", st)


def _group_order_ptr(group_order, S):
    import torch
    if group_order is None:
        return None
    _need(group_order, "group_order", dtype=torch.int32, ndim=1)
    if group_order.shape[0] != S:
        raise ValueError("group_order must have one entry per sequence")
    return group_order.data_ptr()


def paged_attention_decode_shared(part_acc, part_max, part_sum, q, k_cache, v_cache,
                                  block_tables, context_lens, shared_len, group_size: int,
                                  max_context_len: int, partition_size: int, scale: float,
                                  stream=None, group_order=None) -> None:
    """tv_paged_attention_decode_shared: the partition pass with the shared
    prefix of each group of ``group_size`` sequences read once; shared_len:
    int32 [ceil(S / group_size)]; group_order: int32 [S] (position p holds
    sequence group_order[p]) or None for consecutive groups."""
    import torch
    _need(q, "q", itemsize=2, ndim=3)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(shared_len, "shared_len", dtype=torch.int32, ndim=1)
    for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
        _need(t, n, dtype=torch.float32)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d:
        raise ValueError("cache shapes do not match q")
    P = num_partitions(max_context_len, partition_size)
    if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
            tuple(part_sum.shape) != (S, hq, P):
        raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    if group_size < 1 or shared_len.shape[0] != -(-S // group_size):
        raise ValueError("shared_len must have ceil(S / group_size) entries")
    order = _group_order_ptr(group_order, S)
    st = lib().tv_paged_attention_decode_shared(
        part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr(), q.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        shared_len.data_ptr(), order, int(group_size), S, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), int(partition_size), float(scale), _stream_handle(stream, q.device))
    _check("tv_paged_attention_decode_shared", st)


def paged_attention_decode_append(part_acc, part_max, part_sum, q, k_new, v_new, slot_mapping,
                                  k_cache, v_cache, block_tables, context_lens,
                                  max_context_len: int, partition_size: int, scale: float,
                                  stream=None) -> None:
    """tv_paged_attention_decode_append: the cache write of one new token per
    sequence (k_new, v_new: [S, Hkv, D]; slot_mapping: int64 [S]) and the
    partition pass, in one launch."""
    import torch
    _need(q, "q", itemsize=2, ndim=3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
        _need(t, n, dtype=torch.float32)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d:
        raise ValueError("cache shapes do not match q")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d) or \
            slot_mapping.shape[0] != S:
        raise ValueError("k_new, v_new must be [S, Hkv, D] and slot_mapping [S]")
    P = num_partitions(max_context_len, partition_size)
    if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
            tuple(part_sum.shape) != (S, hq, P):
        raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    st = lib().tv_paged_attention_decode_append(
        part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr(), q.data_ptr(),
        k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), S, hq, hkv, d, bs,
        block_tables.shape[1], nb, int(max_context_len), int(partition_size), float(scale),
        _stream_handle(stream, q.device))
    _check("tv_paged_attention_decode_append", st)


def paged_attention_decode_step(out, workspace, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                block_tables, context_lens, max_context_len: int,
                                partition_size: int, scale: float, stream=None) -> None:
    """tv_paged_attention_decode_step: cache write, partition pass and merge in
    one call -- one launch when max_context_len fits one partition (workspace
    unused, may be None), else the append pass and the merge through
    `workspace` = (part_acc, part_max, part_sum).  out: float32 [S, Hq, D]."""
    import torch
    _need(out, "out", dtype=torch.float32, ndim=3)
    _need(q, "q", itemsize=2, ndim=3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d or tuple(out.shape) != (S, hq, d):
        raise ValueError("out must be [S, Hq, D] and the caches must match q")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d) or \
            slot_mapping.shape[0] != S:
        raise ValueError("k_new, v_new must be [S, Hkv, D] and slot_mapping [S]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    P = num_partitions(max_context_len, partition_size)
    if P > 1:
        if workspace is None:
            raise ValueError(f"{P} partitions need the workspace")
        part_acc, part_max, part_sum = workspace
        for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
            _need(t, n, dtype=torch.float32)
        if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
                tuple(part_sum.shape) != (S, hq, P):
            raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
        ptrs = (part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr())
    else:
        ptrs = (None, None, None)
    st = lib().tv_paged_attention_decode_step(
        out.data_ptr(), *ptrs, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), S, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), int(partition_size), float(scale), _stream_handle(stream, q.device))
    _check("tv_paged_attention_decode_step", st)


def paged_attention_decode_step_noalloc(out, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                        block_tables, context_lens, max_context_len: int,
                                        partition_size: int, scale: float, stream=None) -> None:
    """tv_paged_attention_decode_step_noalloc: the whole decode step with the
    partition workspace in the library's fixed per-GPU array (nothing is
    allocated by the call; workspaces above NOALLOC_SCRATCH_BYTES raise
    TvError TV_ERR_SCRATCH)."""
    import torch
    _need(out, "out", dtype=torch.float32, ndim=3)
    _need(q, "q", itemsize=2, ndim=3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d or tuple(out.shape) != (S, hq, d):
        raise ValueError("out must be [S, Hq, D] and the caches must match q")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d) or \
            slot_mapping.shape[0] != S:
        raise ValueError("k_new, v_new must be [S, Hkv, D] and slot_mapping [S]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    st = lib().tv_paged_attention_decode_step_noalloc(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), S, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), int(partition_size), float(scale), _stream_handle(stream, q.device))
    _check("tv_paged_attention_decode_step_noalloc", st)


def paged_attention_decode_shared_step(out, workspace, q, k_new, v_new, slot_mapping, k_cache,
                                       v_cache, block_tables, context_lens, shared_len,
                                       group_size: int, max_context_len: int, partition_size: int,
                                       scale: float, stream=None, group_order=None) -> None:
    """tv_paged_attention_decode_shared_step: the parallel-sampling decode step
    (appends, shared-prefix attention, merge) in one call, into out [S, Hq, D];
    workspace = (part_acc, part_max, part_sum) as for paged_attention_decode."""
    import torch
    part_acc, part_max, part_sum = workspace
    _need(out, "out", dtype=torch.float32, ndim=3)
    _need(q, "q", itemsize=2, ndim=3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(shared_len, "shared_len", dtype=torch.int32, ndim=1)
    for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
        _need(t, n, dtype=torch.float32)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d:
        raise ValueError("cache shapes do not match q")
    if tuple(out.shape) != (S, hq, d):
        raise ValueError("out must be [S, Hq, D]")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d) or \
            slot_mapping.shape[0] != S:
        raise ValueError("k_new, v_new must be [S, Hkv, D] and slot_mapping [S]")
    P = num_partitions(max_context_len, partition_size)
    if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
            tuple(part_sum.shape) != (S, hq, P):
        raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    if group_size < 1 or shared_len.shape[0] != -(-S // group_size):
        raise ValueError("shared_len must have ceil(S / group_size) entries")
    order = _group_order_ptr(group_order, S)
    st = lib().tv_paged_attention_decode_shared_step(
        out.data_ptr(), part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr(),
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        shared_len.data_ptr(), order, int(group_size), S, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_context_len), int(partition_size), float(scale), _stream_handle(stream, q.device))
    _check("tv_paged_attention_decode_shared_step", st)


def paged_attention_decode_shared_append(part_acc, part_max, part_sum, q, k_new, v_new,
                                         slot_mapping, k_cache, v_cache, block_tables,
                                         context_lens, shared_len, group_size: int,
                                         max_context_len: int, partition_size: int, scale: float,
                                         stream=None, group_order=None) -> None:
    """tv_paged_attention_decode_shared_append: the cache write of one new
    token per sequence and the shared-prefix partition pass, in one launch;
    group_order as for paged_attention_decode_shared."""
    import torch
    _need(q, "q", itemsize=2, ndim=3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, itemsize=2, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(shared_len, "shared_len", dtype=torch.int32, ndim=1)
    for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
        _need(t, n, dtype=torch.float32)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = _pool_dims(k_cache, v_cache)
    if d2 != d:
        raise ValueError("cache shapes do not match q")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d) or \
            slot_mapping.shape[0] != S:
        raise ValueError("k_new, v_new must be [S, Hkv, D] and slot_mapping [S]")
    P = num_partitions(max_context_len, partition_size)
    if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
            tuple(part_sum.shape) != (S, hq, P):
        raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    if group_size < 1 or shared_len.shape[0] != -(-S // group_size):
        raise ValueError("shared_len must have ceil(S / group_size) entries")
    order = _group_order_ptr(group_order, S)
    st = lib().tv_paged_attention_decode_shared_append(
        part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr(), q.data_ptr(),
        k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        shared_len.data_ptr(), order, int(group_size), S, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), int(partition_size), float(scale), _stream_handle(stream, q.device))
    _check("tv_paged_attention_decode_shared_append", st)


def paged_attention_reduce(out, part_acc, part_max, part_sum, context_lens, max_context_len: int,
                           partition_size: int, stream=None) -> None:
    """tv_paged_attention_reduce.  out: float32 [S, Hq, D]."""
    import torch
    _need(out, "out", dtype=torch.float32, ndim=3)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, hq, d = out.shape
    P = num_partitions(max_context_len, partition_size)
    for t, n in ((part_acc, "part_acc"), (part_max, "part_max"), (part_sum, "part_sum")):
        _need(t, n, dtype=torch.float32)
    if tuple(part_acc.shape) != (S, hq, P, d) or tuple(part_max.shape) != (S, hq, P) or \
            tuple(part_sum.shape) != (S, hq, P):
        raise ValueError(f"workspace must be [S, Hq, P(={P}), D] and [S, Hq, P]")
    st = lib().tv_paged_attention_reduce(
        out.data_ptr(), part_acc.data_ptr(), part_max.data_ptr(), part_sum.data_ptr(),
        context_lens.data_ptr(), S, hq, d, int(max_context_len), int(partition_size),
        _stream_handle(stream, out.device))
    _check("tv_paged_attention_reduce", st)


def new_workspace(num_seqs: int, num_q_heads: int, head_dim: int, max_context_len: int,
                  partition_size: int, device) -> Tuple:
    """Allocate (part_acc, part_max, part_sum) for the decode/reduce pair."""
    import torch
    P = num_partitions(max_context_len, partition_size)
    return (torch.empty((num_seqs, num_q_heads, P, head_dim), dtype=torch.float32, device=device),
            torch.empty((num_seqs, num_q_heads, P), dtype=torch.float32, device=device),
            torch.empty((num_seqs, num_q_heads, P), dtype=torch.float32, device=device))


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                    partition_size: int = 512, scale: Optional[float] = None, out=None,
                    workspace=None, stream=None):
    """Decode pass + merge; returns out (float32 [S, Hq, D])."""
    import torch
    S, hq, d = q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if workspace is None:
        workspace = new_workspace(S, hq, d, max_context_len, partition_size, q.device)
    if out is None:
        out = torch.empty((S, hq, d), dtype=torch.float32, device=q.device)
    pa, pm, ps = workspace
    paged_attention_decode(pa, pm, ps, q, k_cache, v_cache, block_tables, context_lens,
                           max_context_len, partition_size, scale, stream)
    paged_attention_reduce(out, pa, pm, ps, context_lens, max_context_len, partition_size, stream)
    return out


def copy_blocks(k_cache, v_cache, block_pairs, stream=None) -> None:
    """tv_copy_blocks.  block_pairs: int64 [num_pairs, 2] (source, destination) on
    the device; pools as for cache_write."""
    import torch
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    _need(block_pairs, "block_pairs", dtype=torch.int64, ndim=2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    st = lib().tv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), block_pairs.data_ptr(),
                              block_pairs.shape[0], hkv, d, bs, nb,
                              _stream_handle(stream, k_cache.device))
    _check("tv_copy_blocks", st)


STREAM_CHUNK_BYTES = 8192


def stream_read(buf, chunk_xor, stream=None) -> None:
    """tv_stream_read: read every byte of the contiguous device tensor `buf`
    (its size a multiple of 16 bytes) once; chunk_xor (int32, one entry per
    8 KiB chunk, the last possibly partial) receives each chunk's XOR of
    32-bit words.  The plain-read yardstick for HBM-bound kernels."""
    import torch
    _need(buf, "buf")
    _need(chunk_xor, "chunk_xor", dtype=torch.int32, ndim=1)
    nbytes = buf.numel() * buf.element_size()
    chunks = -(-nbytes // STREAM_CHUNK_BYTES)
    if chunk_xor.numel() < chunks:
        raise ValueError(f"chunk_xor needs {chunks} entries, has {chunk_xor.numel()}")
    st = lib().tv_stream_read(buf.data_ptr(), nbytes, chunk_xor.data_ptr(),
                              _stream_handle(stream, buf.device))
    _check("tv_stream_read", st)


class BlockManager:
    """The library's block manager (tv_bm_*): free list, per-sequence block
    tables, reference counts and copy-on-write.  Host-only bookkeeping; the
    caller moves the K/V data (cache_write / decode_append for slots,
    copy_blocks for copy-on-write pairs)."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int):
        self._lib = lib()
        h = ctypes.c_void_p()
        _check("tv_bm_create", self._lib.tv_bm_create(num_blocks, block_size, max_seqs,
                                                      max_blocks_per_seq, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_seqs, self.max_blocks_per_seq = max_seqs, max_blocks_per_seq

    def close(self) -> None:
        if self._h:
            self._lib.tv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(self._lib.tv_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.tv_bm_refcount(self._h, block))

    def length(self, seq: int) -> int:
        return int(self._lib.tv_bm_length(self._h, seq))

    def add_sequence(self, seq: int, num_tokens: int) -> None:
        _check("tv_bm_add_sequence", self._lib.tv_bm_add_sequence(self._h, seq, num_tokens))

    def fork(self, parent: int, child: int) -> None:
        _check("tv_bm_fork", self._lib.tv_bm_fork(self._h, parent, child))

    def append_slot(self, seq: int):
        """(slot, copy_src, copy_dst) for the next position of ``seq``; copy_src /
        copy_dst are -1 unless a shared block had to be copied."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check("tv_bm_append_slot", self._lib.tv_bm_append_slot(
            self._h, seq, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def free_sequence(self, seq: int) -> None:
        _check("tv_bm_free_sequence", self._lib.tv_bm_free_sequence(self._h, seq))

    def block_table(self, seq: int):
        import numpy as np
        row = np.zeros(self.max_blocks_per_seq, np.int32)
        nb = ctypes.c_int32()
        _check("tv_bm_block_table", self._lib.tv_bm_block_table(
            self._h, seq, row.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), row.shape[0],
            ctypes.byref(nb)))
        return row[:nb.value].copy()

    def slots(self, seq: int, start: int, count: int):
        import numpy as np
        out = np.zeros(count, np.int64)
        _check("tv_bm_slots", self._lib.tv_bm_slots(
            self._h, seq, start, count, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return out

    def prepare_decode(self, seqs, width: int):
        """Reserve one position for each of ``seqs`` (in order) and return the
        host arrays of that decode step: (block_tables int32 [S][width],
        context_lens int32 [S], slot_mapping int64 [S], copy_pairs int64 [C][2]).
        All-or-nothing: on error nothing has changed."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        S = seqs.shape[0]
        tables = np.empty((S, width), np.int32)
        lens = np.empty(S, np.int32)
        slots = np.empty(S, np.int64)
        pairs = np.empty((S, 2), np.int64)
        nc = ctypes.c_int32()
        _check("tv_bm_prepare_decode", self._lib.tv_bm_prepare_decode(
            self._h, seqs.ctypes.data, S, width, tables.ctypes.data, lens.ctypes.data,
            slots.ctypes.data, pairs.ctypes.data, ctypes.byref(nc)))
        return tables, lens, slots, pairs[:nc.value].copy()
