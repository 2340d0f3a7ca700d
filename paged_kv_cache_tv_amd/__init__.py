"""MI355X-native paged GQA attention: libtv (HIP, gfx950) and its Python binding.

The three steps of one decode step -- cache write, partitioned paged attention,
log-sum-exp merge --, prefill / chunked-prefill attention, copy-on-write block
copies and the host block manager run in ``libtv.so``; this package only
marshals torch tensors into the C calls declared in ``include/tv.h``.
"""

from .binding import (LIB_PATH, STREAM_CHUNK_BYTES, DECODE_STEP_FORMS, BlockManager,
                      TvError, cache_write, cache_write_rope, copy_blocks,
                      decode_shared_step_form, decode_step_form, lib, load_library,
                      new_pools, new_workspace, num_partitions, paged_attention,
                      paged_attention_decode, paged_attention_decode_append,
                      paged_attention_decode_vector,
                      paged_attention_decode_shared, paged_attention_decode_shared_append,
                      paged_attention_decode_shared_step, paged_attention_decode_step,
                      paged_attention_decode_step_noalloc, paged_attention_prefill,
                      paged_attention_reduce, rope, stream_read)

__all__ = ["LIB_PATH", "STREAM_CHUNK_BYTES", "DECODE_STEP_FORMS", "BlockManager", "TvError",
           "cache_write", "cache_write_rope", "copy_blocks", "decode_shared_step_form",
           "decode_step_form", "lib", "load_library", "new_pools", "new_workspace",
           "num_partitions", "paged_attention", "paged_attention_decode",
           "paged_attention_decode_append", "paged_attention_decode_shared",
           "paged_attention_decode_shared_append", "paged_attention_decode_shared_step",
           "paged_attention_decode_step", "paged_attention_decode_step_noalloc",
           "paged_attention_decode_vector", "paged_attention_prefill", "paged_attention_reduce",
           "rope", "stream_read"]
