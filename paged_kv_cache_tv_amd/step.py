"""One decode step on the GPU for a ``workloads.DecodeBatch``.

``DeviceBatch`` uploads a batch, builds the K/V pools on the device (poison
everywhere, then every already-cached token written through ``tv_cache_write``)
and runs the step: cache write of the new tokens, partition pass, merge.  Every
step of the path runs in libtv's kernels; torch only allocates memory and
provides the stream.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding as tv
from .workloads import BF16_NAN, DecodeBatch


def _dev(a: np.ndarray, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceBatch:
    def __init__(self, batch: DecodeBatch, device="cuda:0", partition_size: Optional[int] = None,
                 max_context_len: Optional[int] = None):
        import torch
        self.batch = batch
        self.device = torch.device(device)
        self.partition_size = int(partition_size or batch.partition_size)
        self.max_context_len = int(batch.max_context_len if max_context_len is None
                                   else max_context_len)
        b = batch
        self.q = _dev(b.q, self.device)
        self.block_tables = _dev(b.block_tables.astype(np.int32), self.device)
        self.context_lens = _dev(b.context_lens.astype(np.int32), self.device)
        sk, sv, ss = b.step_inputs()
        self.step_k, self.step_v = _dev(sk, self.device), _dev(sv, self.device)
        self.step_slots = _dev(ss.astype(np.int64), self.device)
        self.k_cache, self.v_cache = tv.new_pools(b.num_blocks, b.num_kv_heads, b.head_dim,
                                                  b.block_size, self.device, fill=BF16_NAN)
        self.out = torch.empty((b.num_seqs, b.num_q_heads, b.head_dim), dtype=torch.float32,
                               device=self.device)
        self.workspace = tv.new_workspace(b.num_seqs, b.num_q_heads, b.head_dim,
                                          self.max_context_len, self.partition_size, self.device)

    def fill(self, chunk_tokens: int = 1 << 18) -> None:
        """Write every token cached before the step into the pools (tv_cache_write)."""
        b = self.batch
        n = b.fill_rows.shape[0]
        for lo in range(0, n, chunk_tokens):
            hi = min(n, lo + chunk_tokens)
            rows = b.fill_rows[lo:hi]
            k = _dev(b.kv_k[rows], self.device)
            v = _dev(b.kv_v[rows], self.device)
            s = _dev(b.fill_slots[lo:hi].astype(np.int64), self.device)
            tv.cache_write(k, v, self.k_cache, self.v_cache, s)

    def write_step(self, stream=None) -> None:
        tv.cache_write(self.step_k, self.step_v, self.k_cache, self.v_cache, self.step_slots,
                       stream)

    def decode(self, stream=None) -> None:
        pa, pm, ps = self.workspace
        tv.paged_attention_decode(pa, pm, ps, self.q, self.k_cache, self.v_cache,
                                  self.block_tables, self.context_lens, self.max_context_len,
                                  self.partition_size, self.batch.scale, stream)

    def reduce(self, stream=None) -> None:
        pa, pm, ps = self.workspace
        tv.paged_attention_reduce(self.out, pa, pm, ps, self.context_lens, self.max_context_len,
                                  self.partition_size, stream)

    def decode_append(self, stream=None) -> None:
        """Cache write of the new tokens and partition pass in one launch."""
        pa, pm, ps = self.workspace
        tv.paged_attention_decode_append(pa, pm, ps, self.q, self.step_k, self.step_v,
                                         self.step_slots, self.k_cache, self.v_cache,
                                         self.block_tables, self.context_lens,
                                         self.max_context_len, self.partition_size,
                                         self.batch.scale, stream)

    def step(self, stream=None):
        """Cache write of the new tokens, partition pass, merge (three launches).
        Returns ``out``."""
        self.write_step(stream)
        self.decode(stream)
        self.reduce(stream)
        return self.out

    def fused_step(self, stream=None):
        """The same step in two launches: write + partition pass, then merge."""
        self.decode_append(stream)
        self.reduce(stream)
        return self.out

    def call_step(self, stream=None):
        """The same step through one library call (tv_paged_attention_decode_step):
        one launch when the host bound fits one partition, else two."""
        tv.paged_attention_decode_step(self.out, self.workspace, self.q, self.step_k, self.step_v,
                                       self.step_slots, self.k_cache, self.v_cache,
                                       self.block_tables, self.context_lens,
                                       self.max_context_len, self.partition_size,
                                       self.batch.scale, stream)
        return self.out

    def pools_numpy(self):
        return (self.k_cache.cpu().numpy().view(np.uint16),
                self.v_cache.cpu().numpy().view(np.uint16))
