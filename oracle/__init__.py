"""CPU oracle for paged GQA attention (decode, prefill, block copy) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  It wraps ``liboracle.so`` (built from
``oracle.c`` with plain gcc, no fast-math) through ctypes and never touches the
GPU library.

Cache layout indexed by the oracle: K pool ``[NB][Hkv][D/8][BS][8]``, V pool
``[NB][Hkv][D][BS]``, bf16 as raw uint16.  Results are float64.

Parity status of each function (pins live in ``tests/test_oracle.py`` and
``tests/oracle_pins.py``):
  * ``cache_write``     -- pinned (round trip through paging equals the
                           contiguous sequence; skip rules; untouched bits).
  * ``paged_attention`` -- pinned (contiguous brute force, torch SDPA,
                           closed forms, invariances, the 300-token paging
                           example).
  * ``copy_blocks``     -- pinned (hand-derived literal pools; skip rules;
                           refused conflicting pairs).
  * ``rope``            -- pinned (single-pair closed form with numpy's
                           cos/sin, numpy complex multiplication, half-split
                           = interleaved on permuted dims, position 0,
                           relative-position identity, R_a R_b = R_(a+b),
                           bf16 rounding against a brute-force neighbour
                           search).
  * ``paged_prefill``   -- pinned (torch SDPA with a causal mask on full
                           prompts, chunking invariance, one row per sequence
                           equals decode, first position equals V_0, block
                           permutation, rows past the context).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def cpu_count() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class Oracle:
    """ctypes front end of one build of ``oracle.c``."""

    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built (run __graft_entry__.build())")
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_cache_write.restype = ctypes.c_long
        lib.oracle_cache_write.argtypes = [_u16p, _u16p, _u16p, _u16p, _i64p, ctypes.c_long,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long]
        lib.oracle_paged_attention.restype = ctypes.c_int
        lib.oracle_paged_attention.argtypes = [_f64p, _u16p, _u16p, _u16p, _i32p, _i32p,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_long, ctypes.c_double, ctypes.c_int]
        lib.oracle_paged_prefill.restype = ctypes.c_int
        lib.oracle_paged_prefill.argtypes = [_f64p, _u16p, _i32p, _u16p, _u16p, _i32p, _i32p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_long, ctypes.c_double, ctypes.c_int]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_rope.argtypes = [_u16p, _i32p, ctypes.POINTER(ctypes.c_float), ctypes.c_long,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _u16p]
        lib.oracle_bf16_round.restype = None
        lib.oracle_bf16_round.argtypes = [_f64p, ctypes.c_long, _u16p]
        lib.oracle_copy_blocks.restype = ctypes.c_long
        lib.oracle_copy_blocks.argtypes = [_u16p, _u16p, _i64p, ctypes.c_long, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_long]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        self.lib = lib

    @staticmethod
    def new_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                  fill: int = 0x7FC0):
        """Fresh K and V pools in the oracle's layout, every element set to ``fill`` bits.
        K: [NB, Hkv, D/8, BS, 8]; V: [NB, Hkv, D, BS]."""
        assert head_dim % 8 == 0
        k = np.full((num_blocks, num_kv_heads, head_dim // 8, block_size, 8), fill, np.uint16)
        v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill, np.uint16)
        return k, v

    def cache_write(self, k: np.ndarray, v: np.ndarray, k_cache: np.ndarray,
                    v_cache: np.ndarray, slot_mapping: np.ndarray) -> int:
        """Write rows k[i], v[i] ([T, Hkv, D] uint16) into slot slot_mapping[i], in place."""
        k = np.ascontiguousarray(k, np.uint16)
        v = np.ascontiguousarray(v, np.uint16)
        sm = np.ascontiguousarray(slot_mapping, np.int64)
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
        nb, hkv, dc, bs, x = k_cache.shape
        d = dc * x
        assert x == 8 and v_cache.shape == (nb, hkv, d, bs)
        T = sm.shape[0]
        assert k.shape == (T, hkv, d) and v.shape == (T, hkv, d)
        r = self.lib.oracle_cache_write(_ptr(k, _u16p), _ptr(v, _u16p), _ptr(k_cache, _u16p),
                                        _ptr(v_cache, _u16p), _ptr(sm, _i64p), T, hkv, d, bs, nb)
        if r == -2:
            raise ValueError("duplicate slot in slot_mapping")
        if r < 0:
            raise ValueError("oracle_cache_write rejected its arguments")
        return int(r)

    def copy_blocks(self, k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> int:
        """Copy block src to block dst (both pools, all heads) for each (src, dst)
        in ``pairs``, in place.  Returns the number of blocks copied."""
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        nb, hkv, dc, bs, x = k_cache.shape
        d = dc * x
        assert x == 8 and v_cache.shape == (nb, hkv, d, bs)
        pr = np.ascontiguousarray(np.asarray(pairs, np.int64).reshape(-1, 2))
        r = self.lib.oracle_copy_blocks(_ptr(k_cache, _u16p), _ptr(v_cache, _u16p),
                                        _ptr(pr, _i64p), pr.shape[0], hkv, d, bs, nb)
        if r == -2:
            raise ValueError("a destination block repeats or is also a source")
        if r < 0:
            raise ValueError("oracle_copy_blocks rejected its arguments")
        return int(r)

    def paged_attention(self, q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                        block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                        num_threads: Optional[int] = None) -> np.ndarray:
        """Decode attention for every (sequence, query head); float64 [S, Hq, D]."""
        q = np.ascontiguousarray(q, np.uint16)
        bt = np.ascontiguousarray(block_tables, np.int32)
        cl = np.ascontiguousarray(context_lens, np.int32)
        S, hq, d = q.shape
        nb, hkv, dc, bs, x = k_cache.shape
        assert x == 8 and dc * x == d and v_cache.shape == (nb, hkv, d, bs)
        assert bt.ndim == 2 and bt.shape[0] == S and cl.shape == (S,)
        out = np.zeros((S, hq, d), np.float64)
        threads = cpu_count() if num_threads is None else int(num_threads)
        r = self.lib.oracle_paged_attention(_ptr(out, _f64p), _ptr(q, _u16p),
                                            _ptr(k_cache, _u16p), _ptr(v_cache, _u16p),
                                            _ptr(bt, _i32p), _ptr(cl, _i32p), S, hq, hkv, d, bs,
                                            bt.shape[1], nb, float(scale), threads)
        if r != 0:
            raise ValueError("oracle_paged_attention rejected its arguments")
        return out

    def paged_prefill(self, q: np.ndarray, query_start: np.ndarray, k_cache: np.ndarray,
                      v_cache: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
                      scale: float, num_threads: Optional[int] = None) -> np.ndarray:
        """Causal attention of the query rows of every sequence (rows
        query_start[s] .. query_start[s+1]-1, the last positions of its context)
        over its cached context; float64 [rows, Hq, D]."""
        q = np.ascontiguousarray(q, np.uint16)
        qs = np.ascontiguousarray(query_start, np.int32)
        bt = np.ascontiguousarray(block_tables, np.int32)
        cl = np.ascontiguousarray(context_lens, np.int32)
        T, hq, d = q.shape
        S = cl.shape[0]
        nb, hkv, dc, bs, x = k_cache.shape
        assert x == 8 and dc * x == d and v_cache.shape == (nb, hkv, d, bs)
        assert qs.shape == (S + 1,) and qs[S] <= T and bt.ndim == 2 and bt.shape[0] == S
        out = np.zeros((T, hq, d), np.float64)
        threads = cpu_count() if num_threads is None else int(num_threads)
        r = self.lib.oracle_paged_prefill(_ptr(out, _f64p), _ptr(q, _u16p), _ptr(qs, _i32p),
                                          _ptr(k_cache, _u16p), _ptr(v_cache, _u16p),
                                          _ptr(bt, _i32p), _ptr(cl, _i32p), S, hq, hkv, d, bs,
                                          max(bt.shape[1], 1), nb, float(scale), threads)
        if r != 0:
            raise ValueError("oracle_paged_prefill rejected its arguments")
        return out

    def rope(self, x: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray, style: int = 0):
        """Rotary embedding of x ([T, H, D] bf16 bits) at the given positions:
        (rotated values in float64, the same rounded to bf16 bits)."""
        x = np.ascontiguousarray(x, np.uint16)
        pos = np.ascontiguousarray(positions, np.int32)
        f = np.ascontiguousarray(inv_freq, np.float32)
        T, H, D = x.shape
        assert pos.shape == (T,) and f.shape == (D // 2,)
        out = np.zeros((T, H, D), np.float64)
        bits = np.zeros((T, H, D), np.uint16)
        r = self.lib.oracle_rope(_ptr(x, _u16p), _ptr(pos, _i32p),
                                 f.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), T, H, D,
                                 int(style), _ptr(out, _f64p), _ptr(bits, _u16p))
        if r != 0:
            raise ValueError("oracle_rope rejected its arguments")
        return out, bits

    def bf16_round(self, v: np.ndarray) -> np.ndarray:
        """Nearest bf16 (ties to even) of each double, as bits."""
        v = np.ascontiguousarray(v, np.float64)
        out = np.zeros(v.shape, np.uint16)
        self.lib.oracle_bf16_round(_ptr(v, _f64p), v.size, _ptr(out, _u16p))
        return out

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` next to this file."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def build_pools(oracle: Oracle, batch, include_step: bool = True):
    """Pools holding every cached token of ``batch`` (poison elsewhere), written
    through the oracle's own cache write; with ``include_step`` the step's new
    tokens are written too."""
    kc, vc = Oracle.new_pools(batch.num_blocks, batch.num_kv_heads, batch.head_dim,
                              batch.block_size)
    fk, fv, fs = batch.fill_inputs()
    oracle.cache_write(fk, fv, kc, vc, fs)
    if include_step:
        sk, sv, ss = batch.step_inputs()
        oracle.cache_write(sk, sv, kc, vc, ss)
    return kc, vc


def decode_step(oracle: Oracle, batch, num_threads: Optional[int] = None):
    """The whole step on the CPU: write the new tokens, then attend. Returns (out, kc, vc)."""
    kc, vc = build_pools(oracle, batch, include_step=True)
    out = oracle.paged_attention(batch.q, kc, vc, batch.block_tables, batch.context_lens,
                                 batch.scale, num_threads)
    return out, kc, vc
