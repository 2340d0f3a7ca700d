"""Seeded synthetic inputs for one paged GQA decode step.

This module only draws random numbers and lays out the bookkeeping an engine
would hand to the attention step (context lengths, block tables, slot
numbers).  It holds none of the attention arithmetic: the CPU oracle and the
GPU library each consume these inputs with code of their own.

Shapes follow the Llama-3.2-1B attention layer described on the page
"tiny-vllm 씹뜯맛즐 - (1)" (sections "2. Multi-Head Attention 대신 GQA" and the
dimension list after section 6): hidden size 2048 over 32 query heads gives
head_dim 64; consecutive groups of 4 query heads share one of 8 KV heads.
The cache is cut into 16-token blocks addressed through a per-sequence table
("vLLM" page, section "가상 메모리 방식의 해결").

Values are bf16, carried as raw ``uint16`` bit patterns (round-to-nearest-even
from float32 normals).  Unused cache slots and blocks are left for the caller
to fill with the bf16 NaN pattern ``BF16_NAN`` so that any stray read shows.

Draw order for every batch, from ``numpy.random.Generator(PCG64(seed))``:
  1. context lengths (when drawn);
  2. the physical placement permutation of the block pool;
  3. q for all sequences, shape [S, Hq, D];
  4. K then V for each sequence's positions 0..n-1, sequence by sequence
     (a shared prefix is drawn once, before the private tokens of the
     sequences that share it);
  5. per-workload extras (none draw further numbers at present).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 64
BLOCK_SIZE = 16
SCALE = 0.125           # 1/sqrt(64)
PARTITION_SIZE = 512    # split-context partition length used by the workloads
BF16_NAN = 0x7FC0       # quiet NaN bit pattern in bf16


def blocks_needed(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Number of fixed-size blocks that hold ``num_tokens`` tokens (ceiling division)."""
    if num_tokens < 0:
        raise ValueError("num_tokens must be >= 0")
    return -(-num_tokens // block_size)


def paged_waste(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Slots left empty in the last block when blocks are allocated on demand."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def contiguous_waste(max_length: int, num_tokens: int) -> int:
    """Slots reserved but unused when a whole max-length region is preallocated."""
    if num_tokens > max_length:
        raise ValueError("num_tokens exceeds max_length")
    return max_length - num_tokens


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """The caller-supplied rotary frequency table for plain RoPE, base^(-2k /
    head_dim) for k < head_dim / 2, as float32.  It is an input of the rotary
    calls (both the GPU library and the oracle take it as given), built here
    with the other inputs; a context-extension scheme would supply another
    table.  The Llama-3 family uses base 500000."""
    k = np.arange(0, head_dim, 2, dtype=np.float64)
    return (base ** (-k / head_dim)).astype(np.float32)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class DecodeBatch:
    """Everything one decode step consumes, before anything is written to a cache.

    Token rows: ``kv_k``/``kv_v`` hold one row ``[Hkv, D]`` per distinct cached
    token (a shared prefix appears once).  ``token_rows[s][t]`` names the row
    holding logical position ``t`` of sequence ``s``.  Position ``n-1`` of each
    non-empty sequence is the token produced by this step: it is written to the
    cache by the step itself (``new_*``); every other position is already in the
    cache when the step starts (``fill_*``).
    """

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    partition_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, max_blocks]
    q: np.ndarray                     # uint16 [S, Hq, D]
    kv_k: np.ndarray                  # uint16 [R, Hkv, D]
    kv_v: np.ndarray                  # uint16 [R, Hkv, D]
    token_rows: List[np.ndarray]      # per sequence, int64 [n]
    fill_rows: np.ndarray             # int64 [F]
    fill_slots: np.ndarray            # int64 [F]
    new_rows: np.ndarray              # int64 [S]  (-1 for an empty sequence)
    new_slots: np.ndarray             # int64 [S]  (-1 for an empty sequence)
    poison_block: int                 # a never-allocated block; unused table entries point here
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def step_inputs(self):
        """(k, v, slot_mapping) for the tokens this step writes: one row per sequence."""
        k = np.zeros((self.num_seqs, self.num_kv_heads, self.head_dim), np.uint16)
        v = np.zeros_like(k)
        live = self.new_rows >= 0
        k[live] = self.kv_k[self.new_rows[live]]
        v[live] = self.kv_v[self.new_rows[live]]
        return k, v, self.new_slots.copy()

    def fill_inputs(self):
        """(k, v, slot_mapping) for every token already cached before the step."""
        return (self.kv_k[self.fill_rows], self.kv_v[self.fill_rows], self.fill_slots.copy())

    def logical_kv(self, s: int):
        """Contiguous (unpaged) K and V of sequence ``s``: uint16 [n, Hkv, D] each."""
        rows = self.token_rows[s]
        return self.kv_k[rows], self.kv_v[rows]

    def kv_bytes_logical(self) -> int:
        """K+V bytes one decode step reads, counted once per reading sequence."""
        return self.total_tokens * 2 * self.num_kv_heads * self.head_dim * 2

    def kv_bytes_unique(self) -> int:
        """K+V bytes of distinct cached tokens the step reads (shared blocks once)."""
        return int(self.kv_k.shape[0]) * 2 * self.num_kv_heads * self.head_dim * 2


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _draw_bf16(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return round_to_bf16_bits(x)


def _slots_for(table_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    return table_row[positions // block_size].astype(np.int64) * block_size + positions % block_size


def _finish(name, seed, context_lens, tables, num_blocks, poison_block, q, kv_k, kv_v,
            token_rows, writer_rows, block_size, hq, hkv, d, notes) -> DecodeBatch:
    """Assemble fill/new token lists.  ``writer_rows[s]`` are the rows whose slot
    sequence ``s`` defines (a shared prefix is listed under one sequence only)."""
    S = len(context_lens)
    new_rows = np.full(S, -1, np.int64)
    new_slots = np.full(S, -1, np.int64)
    fill_rows, fill_slots = [], []
    for s in range(S):
        n = int(context_lens[s])
        rows = token_rows[s]
        if n == 0:
            continue
        new_rows[s] = rows[n - 1]
        new_slots[s] = _slots_for(tables[s], np.array([n - 1]), block_size)[0]
        own = writer_rows[s]
        pos = np.nonzero(np.isin(rows, own))[0]
        pos = pos[pos != n - 1]
        fill_rows.append(rows[pos])
        fill_slots.append(_slots_for(tables[s], pos, block_size))
    fill_rows = np.concatenate(fill_rows) if fill_rows else np.zeros(0, np.int64)
    fill_slots = np.concatenate(fill_slots) if fill_slots else np.zeros(0, np.int64)
    return DecodeBatch(
        name=name, seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=block_size, scale=1.0 / float(np.sqrt(d)), partition_size=PARTITION_SIZE,
        num_blocks=int(num_blocks), context_lens=np.asarray(context_lens, np.int32),
        block_tables=tables, q=q, kv_k=kv_k, kv_v=kv_v, token_rows=token_rows,
        fill_rows=fill_rows.astype(np.int64), fill_slots=fill_slots.astype(np.int64),
        new_rows=new_rows, new_slots=new_slots, poison_block=int(poison_block), notes=notes)


def make_batch(context_lens: Sequence[int], seed: int, **kw) -> DecodeBatch:
    """Independent sequences with seeded random physical placement.

    See ``_independent`` for the keyword arguments.
    """
    return _independent(_rng(seed), seed, context_lens, **kw)


def _independent(rng: np.random.Generator, seed: int, context_lens: Sequence[int], *,
                 name: str = "custom", num_q_heads: int = NUM_Q_HEADS,
                 num_kv_heads: int = NUM_KV_HEADS, head_dim: int = HEAD_DIM,
                 block_size: int = BLOCK_SIZE, q_sigma: float = 1.0,
                 spare_fraction: float = 0.1, num_blocks: Optional[int] = None,
                 k_outlier_period: int = 0, k_outlier_factor: float = 8.0,
                 table_width: Optional[int] = None) -> DecodeBatch:
    """Independent sequences drawn from ``rng`` (already past any length draw).

    The pool holds the blocks the batch needs plus ``spare_fraction`` (at least
    one spare block, used as the poison target of unused table entries) unless
    ``num_blocks`` is given.  The free list is a seeded permutation of the pool
    and sequences take their blocks from it in order.  With
    ``k_outlier_period = P > 0`` every token at a 0-based position t with
    ``t % P == P - 1`` has its K multiplied by ``k_outlier_factor`` before
    rounding (a power of two keeps this exact in bf16).
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    if lens.ndim != 1 or (lens < 0).any():
        raise ValueError("context_lens must be a 1-D list of non-negative lengths")
    S = lens.shape[0]
    need = [blocks_needed(int(n), block_size) for n in lens]
    total = int(sum(need))
    if num_blocks is None:
        num_blocks = total + max(1, int(np.ceil(spare_fraction * total)))
    if num_blocks < total + 1:
        raise ValueError("pool too small: need one spare block for poison")
    perm = rng.permutation(num_blocks).astype(np.int32)       # the free list, shuffled
    width = max(1, max(need) if need else 1) if table_width is None else table_width
    poison = int(perm[total])
    tables = np.full((S, width), poison, np.int32)
    cursor = 0
    for s in range(S):
        tables[s, :need[s]] = perm[cursor:cursor + need[s]]
        cursor += need[s]
    q = _draw_bf16(rng, (S, num_q_heads, head_dim), q_sigma)
    ks, vs, token_rows = [], [], []
    row = 0
    for s in range(S):
        n = int(lens[s])
        kf = rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32)
        if k_outlier_period > 0 and n:
            sel = np.arange(n) % k_outlier_period == k_outlier_period - 1
            kf[sel] *= np.float32(k_outlier_factor)
        ks.append(round_to_bf16_bits(kf))
        del kf
        vs.append(_draw_bf16(rng, (n, num_kv_heads, head_dim)))
        token_rows.append(np.arange(row, row + n, dtype=np.int64))
        row += n
    kv_k = np.concatenate(ks) if ks else np.zeros((0, num_kv_heads, head_dim), np.uint16)
    kv_v = np.concatenate(vs) if vs else np.zeros((0, num_kv_heads, head_dim), np.uint16)
    del ks, vs
    return _finish(name, seed, lens, tables, num_blocks, poison, q, kv_k, kv_v, token_rows,
                   token_rows, block_size, num_q_heads, num_kv_heads, head_dim,
                   {"q_sigma": q_sigma, "k_outlier_period": k_outlier_period})


def make_shared_prefix_batch(num_prompts: int, samples: int, prefix_len: int,
                             private_lens: Sequence[int], seed: int, *,
                             rng: Optional[np.random.Generator] = None,
                             name: str = "shared-prefix", spare_fraction: float = 0.1,
                             num_q_heads: int = NUM_Q_HEADS, num_kv_heads: int = NUM_KV_HEADS,
                             head_dim: int = HEAD_DIM, block_size: int = BLOCK_SIZE) -> DecodeBatch:
    """Parallel sampling: each prompt's first ``prefix_len`` tokens live once in
    blocks that all ``samples`` block tables reference; sample ``j`` of prompt
    ``i`` (sequence ``i*samples + j``) then holds ``private_lens[i*samples+j]``
    private cached tokens plus the token this step writes.  ``prefix_len`` must be
    a whole number of blocks so that no write lands in a shared block."""
    if prefix_len % block_size:
        raise ValueError("prefix_len must be a multiple of block_size")
    rng = _rng(seed) if rng is None else rng
    S = num_prompts * samples
    priv = np.asarray(private_lens, np.int64)
    if priv.shape != (S,):
        raise ValueError("private_lens must have num_prompts*samples entries")
    lens = prefix_len + priv + 1
    pblocks = prefix_len // block_size
    own_blocks = [blocks_needed(int(r) + 1, block_size) for r in priv]
    total = num_prompts * pblocks + int(sum(own_blocks))
    num_blocks = total + max(1, int(np.ceil(spare_fraction * total)))
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = int(max(blocks_needed(int(n), block_size) for n in lens))
    poison = int(perm[total])
    tables = np.full((S, width), poison, np.int32)
    cursor = 0
    for i in range(num_prompts):
        shared = perm[cursor:cursor + pblocks]
        cursor += pblocks
        for j in range(samples):
            s = i * samples + j
            tables[s, :pblocks] = shared
            tables[s, pblocks:pblocks + own_blocks[s]] = perm[cursor:cursor + own_blocks[s]]
            cursor += own_blocks[s]
    q = _draw_bf16(rng, (S, num_q_heads, head_dim))
    ks, vs, token_rows, writer_rows = [], [], [], []
    row = 0
    for i in range(num_prompts):
        ks.append(_draw_bf16(rng, (prefix_len, num_kv_heads, head_dim)))
        vs.append(_draw_bf16(rng, (prefix_len, num_kv_heads, head_dim)))
        prefix_rows = np.arange(row, row + prefix_len, dtype=np.int64)
        row += prefix_len
        for j in range(samples):
            s = i * samples + j
            m = int(priv[s]) + 1
            ks.append(_draw_bf16(rng, (m, num_kv_heads, head_dim)))
            vs.append(_draw_bf16(rng, (m, num_kv_heads, head_dim)))
            own = np.arange(row, row + m, dtype=np.int64)
            row += m
            token_rows.append(np.concatenate([prefix_rows, own]))
            writer_rows.append(np.concatenate([prefix_rows, own]) if j == 0 else own)
    kv_k = np.concatenate(ks)
    kv_v = np.concatenate(vs)
    del ks, vs
    return _finish(name, seed, lens, tables, num_blocks, poison, q, kv_k, kv_v, token_rows,
                   writer_rows, block_size, num_q_heads, num_kv_heads, head_dim,
                   {"prefix_len": prefix_len, "samples": samples})


# ----------------------------------------------------------------------------
# The five decode-step workloads.  Seed = 1000 + workload number.
# ----------------------------------------------------------------------------

WORKLOADS = {
    1: "single sequence, context 37, pool of 8 blocks, 3 scattered blocks",
    2: "batch 8, context U[128,1024], pool 1024 blocks",
    3: "batch 64 ragged, context U[512,4096], q ~ N(0,0.5), pool +10%",
    4: "batch 256 = 64 prompts x 4 samples, shared 1024-token prefix + U[0,1024] private",
    5: "batch 4 long context {32768,65536,98304,131072}, every 97th K x8",
}


def _workload_1() -> DecodeBatch:
    seed = 1001
    rng = _rng(seed)
    n, nb = 37, 8
    # Three distinct blocks from a permutation of the 8-block pool, redrawn while
    # they form an ascending run b, b+1, b+2 (the table must be non-contiguous).
    while True:
        perm = rng.permutation(nb).astype(np.int32)
        t = perm[:3]
        if not (t[1] == t[0] + 1 and t[2] == t[1] + 1):
            break
    tables = t.reshape(1, 3).copy()
    poison = int(perm[3])
    q = _draw_bf16(rng, (1, NUM_Q_HEADS, HEAD_DIM))
    kv_k = _draw_bf16(rng, (n, NUM_KV_HEADS, HEAD_DIM))
    kv_v = _draw_bf16(rng, (n, NUM_KV_HEADS, HEAD_DIM))
    rows = [np.arange(n, dtype=np.int64)]
    return _finish("decode-b1-ctx37", seed, np.array([n]), tables, nb, poison, q, kv_k, kv_v,
                   rows, rows, BLOCK_SIZE, NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM, {})


def make_workload(index: int) -> DecodeBatch:
    """Build one of the five seeded decode-step workloads (1-based index)."""
    if index == 1:
        return _workload_1()
    if index == 2:
        rng = _rng(1002)
        lens = rng.integers(128, 1024, size=8, endpoint=True)
        return _independent(rng, 1002, lens, name="decode-b8-ctx128-1024", num_blocks=1024)
    if index == 3:
        rng = _rng(1003)
        lens = rng.integers(512, 4096, size=64, endpoint=True)
        return _independent(rng, 1003, lens, name="decode-b64-ctx512-4096", q_sigma=0.5)
    if index == 4:
        rng = _rng(1004)
        priv = rng.integers(0, 1024, size=256, endpoint=True)
        return make_shared_prefix_batch(64, 4, 1024, priv, 1004, rng=rng,
                                        name="decode-b256-shared-prefix-1024")
    if index == 5:
        lens = np.array([32768, 65536, 98304, 131072])
        return _independent(_rng(1005), 1005, lens, name="decode-b4-ctx32k-128k",
                            k_outlier_period=97, k_outlier_factor=8.0)
    raise ValueError("workload index must be 1..5")


# --------------------------------------------------------------------------- prefill


@dataclass
class PrefillBatch:
    """One prefill (or chunked-prefill) step.

    Sequence ``s`` has ``prior_lens[s]`` positions already cached and a chunk of
    ``query_lens[s]`` new tokens at the positions after them, so its context
    holds ``context_lens[s] = prior + chunk`` positions once the step has
    written the chunk.  ``q`` holds one row ``[Hq, D]`` per chunk token,
    sequence by sequence (rows ``query_start[s] .. query_start[s+1]-1``).
    Pools, tables and the K/V rows of every position come from ``base``.
    """

    name: str
    base: DecodeBatch
    prior_lens: np.ndarray            # int32 [S]
    query_lens: np.ndarray            # int32 [S]
    query_start: np.ndarray           # int32 [S + 1]
    q: np.ndarray                     # uint16 [T, Hq, D]

    @property
    def num_seqs(self) -> int:
        return self.base.num_seqs

    @property
    def num_rows(self) -> int:
        return int(self.query_start[-1])

    @property
    def context_lens(self) -> np.ndarray:
        return self.base.context_lens

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    def _positions(self, chunk: bool):
        k, v, slots = [], [], []
        b = self.base
        for s in range(self.num_seqs):
            lo, hi = (int(self.prior_lens[s]), int(b.context_lens[s])) if chunk else \
                (0, int(self.prior_lens[s]))
            pos = np.arange(lo, hi)
            rows = b.token_rows[s][pos]
            k.append(b.kv_k[rows])
            v.append(b.kv_v[rows])
            slots.append(_slots_for(b.block_tables[s], pos, b.block_size))
        return (np.concatenate(k), np.concatenate(v), np.concatenate(slots).astype(np.int64))

    def prior_inputs(self):
        """(k, v, slot_mapping) of the positions cached before the step."""
        return self._positions(chunk=False)

    def chunk_inputs(self):
        """(k, v, slot_mapping) of the chunk's tokens, in q row order (the step writes these)."""
        return self._positions(chunk=True)

    def causal_flops(self) -> int:
        """Multiply-adds x 2 of QK^T and PV over the (query, key) pairs the causal
        mask keeps: row i of sequence s at position p = n - m + i sees p + 1 keys."""
        pairs = 0
        for s in range(self.num_seqs):
            n, m = int(self.context_lens[s]), int(self.query_lens[s])
            p = np.arange(n - m, n, dtype=np.int64)
            pairs += int(np.maximum(p + 1, 0).sum())
        b = self.base
        return pairs * b.num_q_heads * 4 * b.head_dim


def make_prefill_batch(prior_lens: Sequence[int], query_lens: Sequence[int], seed: int, *,
                       name: str = "prefill-custom", q_sigma: float = 1.0,
                       **kw) -> PrefillBatch:
    """Independent sequences of ``prior + chunk`` positions (K/V, tables and pool
    drawn as by ``make_batch``), then the chunk's query rows [T, Hq, D] from the
    same generator."""
    prior = np.asarray(prior_lens, np.int64)
    ql = np.asarray(query_lens, np.int64)
    if prior.shape != ql.shape or (prior < 0).any() or (ql < 0).any():
        raise ValueError("prior_lens and query_lens: same length, non-negative")
    rng = _rng(seed)
    base = _independent(rng, seed, prior + ql, **kw)
    qs = np.zeros(len(ql) + 1, np.int32)
    qs[1:] = np.cumsum(ql)
    q = _draw_bf16(rng, (int(qs[-1]), base.num_q_heads, base.head_dim), q_sigma)
    return PrefillBatch(name=name, base=base, prior_lens=prior.astype(np.int32),
                        query_lens=ql.astype(np.int32), query_start=qs, q=q)


PREFILL_WORKLOADS = {
    1: "3 prompts of 37, 100 and 300 tokens, full prefill",
    2: "8 sequences: chunk U[1,512] on top of U[0,2048] cached positions",
    3: "8 prompts of 2048 tokens, full prefill",
}


def make_prefill_workload(index: int) -> PrefillBatch:
    """Build one of the seeded prefill workloads (1-based index)."""
    if index == 1:
        return make_prefill_batch([0, 0, 0], [37, 100, 300], 2001, name="prefill-b3-37-100-300")
    if index == 2:
        rng = _rng(2002)
        prior = rng.integers(0, 2048, size=8, endpoint=True)
        chunk = rng.integers(1, 512, size=8, endpoint=True)
        return make_prefill_batch(prior, chunk, 2002, name="prefill-b8-chunk1-512-ctx0-2048")
    if index == 3:
        return make_prefill_batch([0] * 8, [2048] * 8, 2003, name="prefill-b8-prompt2048")
    raise ValueError("prefill workload index must be 1..3")
